// ssd_kernels.h -- the HIP kernels of the SSD forward on gfx950.
//
// Page: "Transformers are SSMs" (paper summary).  The chunked algorithm of
// section 6 is computed by two launches:
//
//   ssd_prep_kernel  (a) chunk cumsum of logA per head (wavefront scans), kept in
//                        log2 units so that every decay is one exp2;
//                    (b) the Q x Q matrix C B^T of every chunk and group, lower
//                        32 x 32 tiles only, on MFMA (section 6.1; shared by the
//                        H/G heads of a group, section 7.2).
//   ssd_walk_kernel  one workgroup per (sequence, head, P tile) walks the chunks
//                    of its sequence in order and fuses the rest:
//                      output   Y_c = diag(exp(cs)) C_c h_c^T            (left factor, 6.2)
//                                   + (L o C B^T)_c X_c                  (diagonal block, 6.1)
//                      state    h_{c+1} = exp(cs_last) h_c + B_c^T (decay o X_c)
//                                                              (right and center factors, 6.2)
//                    The state stays in MFMA accumulators from chunk to chunk.
//
// Inside a chunk the decay mask is never formed for off-diagonal 32 x 32 tiles.
// With e_j the last row of 32-row block j and cs the inclusive cumsum of logA
// (log2 units), X~[s] = 2^(cs[e_j] - cs[s]) X[s] for s in block j.  For an output
// row l of block i the part of the output due to earlier blocks and to the entry
// state is accumulated as
//      acc = C h^T ;  for j < i:  acc = 2^(cs[e_j] - cs[e_{j-1}]) acc + (C B^T)_{ij} X~_j
//      acc[l] *= 2^(cs[l] - cs[e_{i-1}])                (cs[e_{-1}] = 0)
// which telescopes to sum_s 2^(cs[l]-cs[s]) (C_l.B_s) X[s] + 2^(cs[l]) C_l h^T.
// Every factor is <= 1, so nothing overflows for any logA <= 0.  Only the
// diagonal tile uses the exact mask 2^(cs[l]-cs[s]) (s <= l) on unscaled X.
// The chunk state uses the same telescoping over blocks with B^T X~.
#pragma once

#include "ssd_device.h"

namespace ssd {

struct PrepArgs {
    const float* logA;
    const void* B;
    const void* C;
    const int32_t* seq_offsets;
    float* cs;        // [nslots, H, Qp] float, log2 units
    void* cb;         // [nslots, G, ntile, 32, 32] elements of the input dtype
    int64_t T;
    int H, N, G, Q, Qp, ntile, nseq, cs_blocks, hblocks;
};

struct WalkArgs {
    const void* X;
    const void* B;
    const void* C;
    const float* init;
    const int32_t* seq_offsets;
    void* Y;
    float* final_state;
    const float* cs;
    const void* cb;
    int64_t T;
    int H, P, N, G, Q, Qp, ntile, nseq, ptiles, nitems, qb;
    int xs_off, xts_off, bs_off, hs_off, cs_off;   // LDS byte offsets
};

// Consecutive workgroup ids are dispatched round-robin over the 8 XCDs.  Give each
// XCD a contiguous range of work items, so the heads of one sequence (which share
// B, C and C B^T) meet in the same L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    const int nx = 8;
    const int xcd = bid % nx, slot = bid / nx;
    const int per = nblocks / nx, rem = nblocks % nx;
    const int base = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
    return base + slot;
}

// Chunk slot k -> first token row and length.  Without seq_offsets, slot
// k = s * ceil(T/Q) + c; with seq_offsets, slots are numbered sequence by sequence.
__device__ __forceinline__ bool locate_chunk(int k, const int32_t* off, int64_t T, int Q, int nseq,
                                             int64_t* rowc, int* len) {
    if (!off) {
        const int nc = (int)((T + Q - 1) / Q);
        if (k >= nseq * nc) return false;
        const int s = k / nc, c = k % nc;
        *rowc = (int64_t)s * T + (int64_t)c * Q;
        *len = (int)min((int64_t)Q, T - (int64_t)c * Q);
        return true;
    }
    int acc = 0;
    for (int s = 0; s < nseq; ++s) {
        const int l = off[s + 1] - off[s];
        const int nch = (l + Q - 1) / Q;
        if (k < acc + nch) {
            const int c = k - acc;
            *rowc = (int64_t)off[s] + (int64_t)c * Q;
            *len = min(Q, l - c * Q);
            return true;
        }
        acc += nch;
    }
    return false;
}

__device__ __forceinline__ float wave_inclusive_sum(float x, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    return x;
}

template <typename T>
__global__ void __launch_bounds__(256) ssd_prep_kernel(PrepArgs a) {
    using E = Elem<T>;
    typedef typename E::frag frag;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 31, lg = lane >> 5;
    int bid = blockIdx.x;
    const bool cs_role = bid < a.cs_blocks;
    int k, rest;
    if (cs_role) {
        k = bid / a.hblocks;
        rest = bid % a.hblocks;
    } else {
        bid -= a.cs_blocks;
        k = bid / a.G;
        rest = bid % a.G;
    }
    int64_t rowc;
    int len;
    if (!locate_chunk(k, a.seq_offsets, a.T, a.Q, a.nseq, &rowc, &len)) return;

    if (cs_role) {
        // (a) one wavefront per head: 4 consecutive tokens per lane, then a lane scan.
        const int h = rest * 4 + wave;
        if (h >= a.H) return;
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * lane + j;
            v[j] = (r < len) ? a.logA[(rowc + r) * a.H + h] : 0.f;
        }
        v[1] += v[0];
        v[2] += v[1];
        v[3] += v[2];
        const float excl = wave_inclusive_sum(v[3], lane) - v[3];
        if (4 * lane < a.Qp) {
            f32x4 o = {(excl + v[0]) * kLog2e, (excl + v[1]) * kLog2e, (excl + v[2]) * kLog2e,
                       (excl + v[3]) * kLog2e};
            *reinterpret_cast<f32x4*>(a.cs + ((int64_t)k * a.H + h) * a.Qp + 4 * lane) = o;
        }
        return;
    }

    // (b) C B^T tiles (i, j), j <= i, of this chunk and group.  The tile is computed
    // transposed, D[s][l] = sum_n B[s][n] C[l][n], so that each lane ends with one
    // row l of C B^T and writes it as runs of 4 consecutive s.
    const int g = rest;
    const T* Bp = static_cast<const T*>(a.B);
    const T* Cp = static_cast<const T*>(a.C);
    const int nlb = (len + 31) >> 5;
    const int ntl = nlb * (nlb + 1) / 2;
    for (int t = wave; t < ntl; t += 4) {
        int i = 0;
        while ((i + 1) * (i + 2) / 2 <= t) ++i;
        const int j = t - i * (i + 1) / 2;
        const bool svalid = 32 * j + lr < len, lvalid = 32 * i + lr < len;
        const T* brow = Bp + ((rowc + 32 * j + lr) * a.G + g) * (int64_t)a.N + 8 * lg;
        const T* crow = Cp + ((rowc + 32 * i + lr) * a.G + g) * (int64_t)a.N + 8 * lg;
        f32x16 acc = {};
        for (int ks = 0; ks < a.N / 16; ++ks) {
            const frag av = svalid ? E::ldg8(brow + 16 * ks) : E::zero();
            const frag bv = lvalid ? E::ldg8(crow + 16 * ks) : E::zero();
            acc = E::mma(acc, av, bv);
        }
        T* out = static_cast<T*>(a.cb) + ((int64_t)(k * a.G + g) * a.ntile + t) * 1024 + lr * 32 + 4 * lg;
#pragma unroll
        for (int q = 0; q < 4; ++q) E::st4(out + 8 * q, acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
    }
}

template <typename T, int PT, int NP>
__global__ void __launch_bounds__(512) ssd_walk_kernel(WalkArgs a) {
    using E = Elem<T>;
    typedef typename E::frag frag;
    constexpr int PAD = 16 / sizeof(T);
    constexpr int XS = PT + PAD, BS = NP + PAD, HS = NP + PAD;
    constexpr int PSUB = PT / 32, NT = NP / 32;
    constexpr int NTILE_S = PSUB * NT;
    constexpr int TPW = (NTILE_S + 7) / 8;
    extern __shared__ __align__(16) unsigned char smem[];
    T* Xs = reinterpret_cast<T*>(smem + a.xs_off);
    T* Xts = reinterpret_cast<T*>(smem + a.xts_off);
    T* Bs = reinterpret_cast<T*>(smem + a.bs_off);
    T* hs = reinterpret_cast<T*>(smem + a.hs_off);
    float* css = reinterpret_cast<float*>(smem + a.cs_off);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 31, lg = lane >> 5;
    const int item = xcd_remap(blockIdx.x, gridDim.x);
    if (item >= a.nitems) return;
    const int pt = item % a.ptiles;
    const int sh = item / a.ptiles;
    const int h = sh % a.H, s = sh / a.H;
    const int g = h / (a.H / a.G);
    const int p_base = pt * PT;
    const int H = a.H, P = a.P, N = a.N, G = a.G, Q = a.Q;

    int64_t row0;
    int len_seq, slot0;
    if (!a.seq_offsets) {
        row0 = (int64_t)s * a.T;
        len_seq = (int)a.T;
        slot0 = s * (int)((a.T + Q - 1) / Q);
    } else {
        row0 = a.seq_offsets[s];
        len_seq = a.seq_offsets[s + 1] - a.seq_offsets[s];
        slot0 = 0;
        for (int u = 0; u < s; ++u) slot0 += (a.seq_offsets[u + 1] - a.seq_offsets[u] + Q - 1) / Q;
    }
    const int nchunks = (len_seq + Q - 1) / Q;

    const T* X = static_cast<const T*>(a.X);
    const T* Bg = static_cast<const T*>(a.B);
    const T* Cg = static_cast<const T*>(a.C);
    T* Y = static_cast<T*>(a.Y);
    const int64_t state_base = ((int64_t)s * H + h) * P * (int64_t)N;

    // ---- state h (P tile x N) in accumulators: wave owns tiles wave, wave + 8, ...
    //      tile t -> (n tile t / PSUB, p sub-tile t % PSUB); element i is (n, p) =
    //      (32 nt + acc_row(i), 32 ps + lr).
    f32x16 hacc[TPW];
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
        hacc[k] = f32x16{};
        const int t = wave + 8 * k;
        if (t >= NTILE_S || !a.init) continue;
        const int n0 = 32 * (t / PSUB), p = p_base + 32 * (t % PSUB) + lr;
        if (p >= P) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int n = n0 + 8 * q + 4 * lg;
            if (n < N) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(a.init + state_base + (int64_t)p * N + n);
                hacc[k][4 * q] = v[0];
                hacc[k][4 * q + 1] = v[1];
                hacc[k][4 * q + 2] = v[2];
                hacc[k][4 * q + 3] = v[3];
            }
        }
    }
    auto write_state_lds = [&]() {
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
            const int t = wave + 8 * k;
            if (t >= NTILE_S) continue;
            const int n0 = 32 * (t / PSUB), p = 32 * (t % PSUB) + lr;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                E::st4(hs + p * HS + n0 + 8 * q + 4 * lg, hacc[k][4 * q], hacc[k][4 * q + 1],
                       hacc[k][4 * q + 2], hacc[k][4 * q + 3]);
        }
    };
    write_state_lds();

    const bool one_stage = a.qb >= a.Qp;

    for (int c = 0; c < nchunks; ++c) {
        const int64_t rowc = row0 + (int64_t)c * Q;
        const int len = min(Q, len_seq - c * Q);
        const int nlb = (len + 31) >> 5;
        const int rows = nlb * 32;
        const int slot = slot0 + c;
        const float* csg = a.cs + ((int64_t)slot * H + h) * a.Qp;

        // ---- phase 1: chunk cumsum, X and decay-scaled X~ into LDS (and B if it fits)
        for (int i = tid; i < rows; i += 512) css[i] = csg[i];
        for (int idx = tid; idx < rows * (PT / 8); idx += 512) {
            const int r = idx / (PT / 8), c8 = (idx % (PT / 8)) * 8;
            const int p = p_base + c8;
            frag v = E::zero();
            if (r < len && p < P) v = E::ldg8(X + ((rowc + r) * H + h) * (int64_t)P + p);
            const float f = fast_exp2(csg[r | 31] - csg[r]);
            frag vt;
#pragma unroll
            for (int q = 0; q < 8; ++q) vt[q] = E::from_f(E::to_f(v[q]) * f);
            *reinterpret_cast<frag*>(Xs + r * XS + c8) = v;
            *reinterpret_cast<frag*>(Xts + r * XS + c8) = vt;
        }
        auto load_b_rows = [&](int rb0, int rb1) {
            for (int idx = tid; idx < (rb1 - rb0) * (NP / 8); idx += 512) {
                const int r = rb0 + idx / (NP / 8), c8 = (idx % (NP / 8)) * 8;
                frag v = E::zero();
                if (r < len && c8 < N) v = E::ldg8(Bg + ((rowc + r) * G + g) * (int64_t)N + c8);
                *reinterpret_cast<frag*>(Bs + (r - rb0) * BS + c8) = v;
            }
        };
        if (one_stage) load_b_rows(0, rows);
        __syncthreads();

        // ---- phase 2: output tiles Y^T[p][l] for (32-row block i, 32-wide p sub-tile).
        //      Wave units pair block a with block nlb-1-a to balance the causal work.
        const T* cbase_g = static_cast<const T*>(a.cb) + (int64_t)(slot * G + g) * a.ntile * 1024;
        auto out_tile = [&](int i, int ps) {
            const int l0 = 32 * i, p0 = 32 * ps;
            const bool lvalid = l0 + lr < len;
            f32x16 acc = {};
            // left factor: C_l . h  (A = h rows from LDS, B = C rows from global)
            const T* crow = Cg + ((rowc + l0 + lr) * G + g) * (int64_t)N + 8 * lg;
            for (int ks = 0; ks < N / 16; ++ks) {
                const frag av = E::lds8(hs + (p0 + lr) * HS + 16 * ks + 8 * lg);
                const frag bv = lvalid ? E::ldg8(crow + 16 * ks) : E::zero();
                acc = E::mma(acc, av, bv);
            }
            // earlier blocks j < i through (C B^T)_{ij} and X~_j, decayed block to block
            const T* cbase = cbase_g + (int64_t)(i * (i + 1) / 2) * 1024 + lr * 32 + 8 * lg;
            float prev = 0.f;
            for (int j = 0; j < i; ++j) {
                const float e = css[32 * j + 31];
                acc *= fast_exp2(e - prev);
                prev = e;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const frag av = lds_col<T>(Xts, XS, 32 * j + 16 * ks, p0, lane);
                    const frag bv = E::ldg8(cbase + j * 1024 + 16 * ks);
                    acc = E::mma(acc, av, bv);
                }
            }
            const float csl = css[l0 + lr];
            acc *= fast_exp2(csl - prev);
            // diagonal tile: exact mask 2^(cs[l] - cs[s]), s <= l, on unscaled X
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const frag av = lds_col<T>(Xs, XS, l0 + 16 * ks, p0, lane);
                const frag raw = E::ldg8(cbase + i * 1024 + 16 * ks);
                frag m;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int sl = 16 * ks + 8 * lg + q;
                    const float w = (sl <= lr) ? E::to_f(raw[q]) * fast_exp2(csl - css[l0 + sl]) : 0.f;
                    m[q] = E::from_f(w);
                }
                acc = E::mma(acc, av, m);
            }
            if (lvalid) {
                T* yrow = Y + ((rowc + l0 + lr) * H + h) * (int64_t)P;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int p = p_base + p0 + 8 * q + 4 * lg;
                    if (p < P) E::st4(yrow + p, acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
                }
            }
        };
        const int npairs = (nlb + 1) >> 1;
        for (int u = wave; u < npairs * PSUB; u += 8) {
            const int ps = u % PSUB, pa = u / PSUB;
            if (p_base + 32 * ps >= P) continue;
            out_tile(pa, ps);
            if (nlb - 1 - pa != pa) out_tile(nlb - 1 - pa, ps);
        }

        // ---- phase 3: chunk state, h = 2^(cs_last) h + B^T (decay o X), telescoped
        //      block by block: h = 2^(cs[e_j] - cs[e_{j-1}]) h + B_j^T X~_j.
        float prev[TPW];
#pragma unroll
        for (int k = 0; k < TPW; ++k) prev[k] = 0.f;
        const int bpb = one_stage ? nlb : a.qb / 32;   // 32-row blocks per B stage
        for (int jb0 = 0; jb0 < nlb; jb0 += bpb) {
            const int jb1 = min(nlb, jb0 + bpb);
            if (!one_stage) {
                __syncthreads();
                load_b_rows(32 * jb0, 32 * jb1);
                __syncthreads();
            }
#pragma unroll
            for (int k = 0; k < TPW; ++k) {
                const int t = wave + 8 * k;
                if (t >= NTILE_S) continue;
                const int n0 = 32 * (t / PSUB), p0 = 32 * (t % PSUB);
                if (n0 >= N || p_base + p0 >= P) continue;
                for (int j = jb0; j < jb1; ++j) {
                    const float e = css[32 * j + 31];
                    hacc[k] *= fast_exp2(e - prev[k]);
                    prev[k] = e;
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        const frag av = lds_col<T>(Bs, BS, 32 * (j - jb0) + 16 * ks, n0, lane);
                        const frag bv = lds_col<T>(Xts, XS, 32 * j + 16 * ks, p0, lane);
                        hacc[k] = E::mma(hacc[k], av, bv);
                    }
                }
            }
        }
        __syncthreads();
        write_state_lds();
    }

    if (a.final_state) {
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
            const int t = wave + 8 * k;
            if (t >= NTILE_S) continue;
            const int n0 = 32 * (t / PSUB), p = p_base + 32 * (t % PSUB) + lr;
            if (p >= P) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + 8 * q + 4 * lg;
                if (n < N) {
                    const f32x4 v = {hacc[k][4 * q], hacc[k][4 * q + 1], hacc[k][4 * q + 2], hacc[k][4 * q + 3]};
                    *reinterpret_cast<f32x4*>(a.final_state + state_base + (int64_t)p * N + n) = v;
                }
            }
        }
    }
}

}  // namespace ssd
