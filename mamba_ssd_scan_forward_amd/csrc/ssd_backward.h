// ssd_backward.h -- the small HBM-bound kernels of the SSD layer's backward pass.
//
// The pages give only the cost of training (page "Transformers are SSMs" paper
// summary, section 6: training FLOPs of order T N^2); the derivative itself follows
// from the recurrence of section 2.4.  With G the adjoint of the P x N state, walked
// backwards from the final state's gradient dF,
//     G_t = a_{t+1} G_{t+1} + dy_t C_t^T,   dx_t = G_t B_t,   dB_t = sum_h G_t^T x_t,
//     dC_t = sum_h S_t^T dy_t,              dlogA_t = a_t <G_t, S_{t-1}>,
//     dinit = a_0 G_0.
// Each of G's contractions is an SSD forward pass of its own, so the backward runs the
// forward kernels three times on re-arranged operands:
//   dX, dinit: time reversed within every sequence, X' = dY, B' = C, C' = B, the
//              decays shifted by one token (logA'_0 = 0, logA'_j = logA_{len-j}), the
//              initial state dF: Y' is dX reversed, the final state is G_0;
//   dB:        time reversed, X' = C (the heads of a group read its row), B' = dY,
//              C' = X, initial state dF^T: Y' reversed is dB per head;
//   dC:        forward time, X' = B (read per group), B' = X, C' = dY, initial state
//              init^T: Y' is dC per head;
// then per-group sums over heads.  Where the fused walker takes these shapes, its reversed
// form walks the time-reversed problems in place (no reversed copies); the kernels below that
// reverse rows serve the other shapes.  The decay gradient uses the identity
//     dL/dcs_k = dy_k . y_k - x_k . dx_k  (+ <dF, final> at a sequence's last token)
// for the inclusive cumsum cs of logA, and dlogA_t = sum_{k >= t} dL/dcs_k.
// The kernels below do the re-arranging, the sums and that reverse cumsum.
#pragma once

#include "ssd_kernels.h"

namespace ssd {

// Token rows of a [rows, ...] tensor: fixed-length sequences of T rows, or packed ones
// delimited by seq_offsets.  src(r) is r itself, or its mirror within its sequence.
struct RowMap {
    const int32_t* off;
    int64_t T;
    int nseq;
    int reverse;

    __device__ __forceinline__ void range(int64_t r, int64_t* r0, int64_t* r1) const {
        if (!off) {
            const int64_t s = r / T;
            *r0 = s * T;
            *r1 = *r0 + T;
            return;
        }
        // the last sequence that starts at or before r (empty ones are skipped over)
        int lo = 0, hi = nseq - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (off[mid] <= r) lo = mid;
            else hi = mid - 1;
        }
        *r0 = off[lo];
        *r1 = off[lo + 1];
    }
    __device__ __forceinline__ int64_t src(int64_t r) const {
        if (!reverse) return r;
        int64_t r0, r1;
        range(r, &r0, &r1);
        return r0 + r1 - 1 - r;
    }
};

__device__ __forceinline__ void seq_rows(int s, int64_t T, const int32_t* off, int64_t* r0, int64_t* r1) {
    if (off) {
        *r0 = off[s];
        *r1 = off[s + 1];
    } else {
        *r0 = (int64_t)s * T;
        *r1 = *r0 + T;
    }
}

// out[r][k][:] = in[src(r)][k / (K / Kin)][:], rows of K segments of `seg` 16-byte vectors
// (a reversed copy when K == Kin, a per-head expansion of per-group rows otherwise)
__global__ void __launch_bounds__(256) ssd_bwd_remap_kernel(const uint4* in, uint4* out, int64_t rows, int K,
                                                            int Kin, int seg, RowMap m) {
    const int64_t total = rows * K * seg;
    const int per = K / Kin;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int v = (int)(i % seg);
        const int64_t rk = i / seg;
        const int k = (int)(rk % K);
        const int64_t r = rk / K;
        out[i] = in[(m.src(r) * Kin + k / per) * seg + v];
    }
}

// the decays of the reversed sequences: out[r0 + j][h] = j == 0 ? 0 : logA[r1 - j][h]
__global__ void __launch_bounds__(256) ssd_bwd_logA_kernel(const float* logA, float* out, int64_t rows, int H,
                                                           RowMap m) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows * H; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / H;
        const int h = (int)(i % H);
        int64_t r0, r1;
        m.range(r, &r0, &r1);
        const int64_t j = r - r0;
        out[i] = j == 0 ? 0.f : logA[(r1 - j) * H + h];
    }
}

// [S][P][N] -> [S][N][P], float32, through 16 x 16 tiles in LDS (rows of 64 bytes read and
// written whole); P and N are multiples of 16.  A workgroup takes tiles tile, tile + grid, ...
__global__ void __launch_bounds__(256) ssd_bwd_transpose_kernel(const float* in, float* out, int64_t S, int P, int N) {
    __shared__ float t16[16][17];
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int tp = P / 16, tn = N / 16;
    const int64_t ntiles = S * tp * tn;
    const int64_t pn = (int64_t)P * N;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t sidx = tile / (tp * tn);
        const int rem = (int)(tile - sidx * tp * tn);
        const int p0 = 16 * (rem / tn), n0 = 16 * (rem % tn);
        t16[ty][tx] = in[sidx * pn + (int64_t)(p0 + ty) * N + n0 + tx];
        __syncthreads();
        out[sidx * pn + (int64_t)(n0 + ty) * P + p0 + tx] = t16[tx][ty];
        __syncthreads();
    }
}

// out[r][g][:] = sum over the heads h of group g of in[src(r)][h][:] (float32 sums,
// stored in the element type), 8 values per thread
template <typename T>
__global__ void __launch_bounds__(256) ssd_bwd_group_sum_kernel(const T* in, T* out, int64_t rows, int H, int G,
                                                                int N, RowMap m) {
    using E = Elem<T>;
    typedef typename E::frag frag;
    const int nv = N / 8, hpg = H / G;
    const int64_t total = rows * G * nv;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int v = (int)(i % nv);
        const int64_t rg = i / nv;
        const int g = (int)(rg % G);
        const int64_t r = rg / G;
        const int64_t src = m.src(r);
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        const T* base = in + (src * H + g * hpg) * (int64_t)N + 8 * v;
        int h = 0;
        // eight heads' loads in flight at a time
        for (; h + 8 <= hpg; h += 8) {
            frag x[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) x[k] = E::ldg8(base + (int64_t)(h + k) * N);
#pragma unroll
            for (int k = 0; k < 8; ++k)
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[q] += E::to_f(x[k][q]);
        }
        for (; h < hpg; ++h) {
            const frag x = E::ldg8(base + (int64_t)h * N);
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[q] += E::to_f(x[q]);
        }
        frag o;
#pragma unroll
        for (int q = 0; q < 8; ++q) o[q] = E::from_f(acc[q]);
        *reinterpret_cast<frag*>(out + (r * G + g) * (int64_t)N + 8 * v) = o;
    }
}

// rr[h][r] = dy . y - x . dx over the head's P values (stored head-major, so that the
// reverse cumsum below reads each head's tokens contiguously).  Each thread takes one 16-byte
// vector of the flat [rows * H * P] arrays (coalesced) per window of 256 vectors; the
// window's partial sums meet in LDS and each (row, head) that starts in the window adds
// its P / 8 partial sums in column order (those past the window's end recomputed from
// memory), so rr does not depend on the order in which threads finish.
template <typename T>
__global__ void __launch_bounds__(256) ssd_bwd_dot_kernel(const T* dY, const T* Y, const T* X, const T* dX,
                                                          float* rr, int64_t rows, int H, int P) {
    using E = Elem<T>;
    typedef typename E::frag frag;
    // each thread's partial sum of 8 columns, then each (row, head) item sums its vectors
    // in column order: a fixed order, so the result does not depend on thread timing
    __shared__ float part[256];
    const int vpi = P / 8;                             // vectors per (row, head)
    const int64_t nvec = rows * H * vpi;
    for (int64_t base = (int64_t)blockIdx.x * 256; base < nvec; base += (int64_t)gridDim.x * 256) {
        const int64_t v = base + threadIdx.x;
        float acc = 0.f;
        if (v < nvec) {
            const int64_t e = v * 8;
            const frag a = E::ldg8(dY + e), b = E::ldg8(Y + e), x = E::ldg8(X + e), d = E::ldg8(dX + e);
#pragma unroll
            for (int q = 0; q < 8; ++q) acc += E::to_f(a[q]) * E::to_f(b[q]) - E::to_f(x[q]) * E::to_f(d[q]);
        }
        part[threadIdx.x] = acc;
        __syncthreads();
        // the items that start in this 256-vector window (an item that starts in the
        // previous window was summed there: windows are whole items when vpi divides 256,
        // else an item's vectors past the window are read from the next window's loads)
        const int64_t first = (base + vpi - 1) / vpi, last = (min(nvec, base + 256) - 1) / vpi;
        for (int64_t it = first + threadIdx.x; it <= last; it += 256) {
            float sum = 0.f;
            for (int k = 0; k < vpi; ++k) {
                const int64_t w = it * vpi + k;
                if (w < base + 256) {
                    sum += part[w - base];
                } else {
                    // past the window: recompute from global memory, in the same order
                    const int64_t e = w * 8;
                    const frag a = E::ldg8(dY + e), b = E::ldg8(Y + e), x = E::ldg8(X + e), d = E::ldg8(dX + e);
                    float r = 0.f;
#pragma unroll
                    for (int q = 0; q < 8; ++q) r += E::to_f(a[q]) * E::to_f(b[q]) - E::to_f(x[q]) * E::to_f(d[q]);
                    sum += r;
                }
            }
            rr[(it % H) * rows + it / H] = sum;   // [H][rows]: each head's tokens contiguous
        }
        __syncthreads();
    }
}

// dlogA[t][h] = sum over the tokens k >= t of its sequence of rr[k][h], plus <dF, final>
// of (sequence, head) when dF is given: one wavefront per (sequence, head), 64 tokens
// per step from the end, a lane scan and a carry.
__global__ void __launch_bounds__(64) ssd_bwd_dlogA_kernel(const float* rr, const float* dF, const float* F,
                                                           float* dlogA, int64_t T, const int32_t* off, int H,
                                                           int PN, int64_t rows) {
    const int sh = blockIdx.x, lane = threadIdx.x;
    const int s = sh / H, h = sh % H;
    float carry = 0.f;
    if (dF) {
        float acc = 0.f;
        const f32x4* a4 = reinterpret_cast<const f32x4*>(dF + (int64_t)sh * PN);
        const f32x4* b4 = reinterpret_cast<const f32x4*>(F + (int64_t)sh * PN);
#pragma unroll 8
        for (int i = lane; i < PN / 4; i += 64) {
            const f32x4 x = a4[i], y = b4[i];
            acc += x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
        }
        carry = __shfl(wave_inclusive_sum(acc, lane), 63, 64);
    }
    int64_t r0, r1;
    seq_rows(s, T, off, &r0, &r1);
    // 16 steps of 64 tokens loaded at once, then scanned one after the other
    for (int64_t top = r1; top > r0; top -= 16 * 64) {
        float v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int64_t t = top - 1 - 64 * k - lane;
            v[k] = t >= r0 ? rr[h * rows + t] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int64_t t = top - 1 - 64 * k - lane;
            const float sum = wave_inclusive_sum(v[k], lane);
            if (t >= r0) dlogA[t * H + h] = carry + sum;
            carry += __shfl(sum, 63, 64);
        }
    }
}

// dinit = a_0 G_0 in place (G_0 as the reversed pass left it; an empty sequence keeps
// dF, which that pass passed through): a workgroup per (sequence, head) at a time, its
// scale formed once, then PN / 4 float4 of the state
__global__ void __launch_bounds__(256) ssd_bwd_dinit_kernel(float* dinit, const float* logA, int64_t T,
                                                            const int32_t* off, int nseq, int H, int PN) {
    for (int64_t sh = blockIdx.x; sh < (int64_t)nseq * H; sh += gridDim.x) {
        const int s = (int)(sh / H), h = (int)(sh % H);
        int64_t r0, r1;
        seq_rows(s, T, off, &r0, &r1);
        if (r1 <= r0) continue;
        const float a0 = fast_exp2(logA[r0 * H + h] * kLog2e);
        f32x4* d4 = reinterpret_cast<f32x4*>(dinit + sh * PN);
        for (int i = threadIdx.x; i < PN / 4; i += blockDim.x) {
            const f32x4 v = d4[i];
            d4[i] = f32x4{v[0] * a0, v[1] * a0, v[2] * a0, v[3] * a0};
        }
    }
}

}  // namespace ssd
