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
    int H, N, G, Q, Qp, ntile, nseq;
    int cs_blocks;    // workgroups of the cumsum role: nslots * hblocks
    int hblocks;      // 64-head blocks per chunk
    int cb_blocks;    // workgroups of the C B^T role: nslots * G
    int ldn, n0;      // B, C rows hold ldn values; the fragment copies take columns [n0, n0 + N)
    int cb_n;         // C B^T contracts columns [0, cb_n) (ldn: all of them), or 0: no tiles
    void* bt2;        // optional: fragment copies of columns [n0 + N, n0 + 2 N) (the second
    void* ct2;        // column half of a d_state walked in two passes)
    void* bt;         // optional: B^T of every 256-row chunk in MFMA A-operand fragment
                      // order, [nslots, G, N/32, 8, 2, 64 lanes, 8], and
    void* ct;         // C in MFMA B-operand fragment order, [nslots, G, 8, N/16, 64 lanes,
                      // 8]; written by the C B^T role (bf16 only)
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
    const void* bt;   // B^T fragments (split-role walker only)
    const void* ct;   // C fragments (split-role walker only)
    float* seg_state;   // segmented walk: [nseq][nseg - 1][nsplit][H][P][N] float32
    float* seg_decay;   // states of the summed-up parts and their total log2 decays
    int nseg;           // segments per segmented sequence (1: none is segmented)
    int nsplit;         // summary parts per segment
    int nwhole, ntail;  // items walked whole, then items walked in nseg segments
    int lpt;            // packed sequences: (sequence, group) units dealt to XCDs longest first
    int xh;             // X rows per token: H (one per head), or fewer, shared by H / xh heads
    int ldn, ns0;       // init / final state rows hold ldn values; this call's are [ns0, ns0 + N)
    int64_t T;
    int H, P, N, G, Q, Qp, ntile, nseq, ptiles, nitems, qb;
    int cb_lds;                                    // stage off-diagonal C B^T tiles in LDS
    int xs_off, xts_off, bs_off, hs_off, cs_off;   // LDS byte offsets
};

struct DecodeArgs {
    const void* x;       // [b, H, P]   input dtype
    const float* logA;   // [b, H]
    const void* B;       // [b, G, N]   input dtype
    const void* C;       // [b, G, N]   input dtype
    float* state;        // [b, H, P, N] float32, updated in place
    void* y;             // [b, H, P]   input dtype
    int H, P, N, G;
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

constexpr int kPrepHeads = 16;   // heads per cumsum workgroup (small LDS tile: the C B^T role
                                 // shares the launch and its occupancy)
constexpr int kPrepThreads = 512;                 // 8 wavefronts per workgroup
constexpr int kPrepWaves = kPrepThreads / 64;

// The C B^T role stages the chunk's B and C rows in LDS in slabs of kCbSlab<T> columns,
// 128 bytes of each row (a whole cache line: a narrower slab would leave the rest of the
// line to be fetched again by the next one when rows are far apart, G > 1); rows padded
// by 16 bytes: 72 KB for either element type.
template <typename T> constexpr int kCbSlab = 128 / (int)sizeof(T);
template <typename T> constexpr int kCbStride = kCbSlab<T> + 16 / (int)sizeof(T);
template <typename T> constexpr int kPrepLds = 2 * 256 * kCbStride<T> * (int)sizeof(T);

template <typename T>
__global__ void __launch_bounds__(kPrepThreads, 2) ssd_prep_kernel(PrepArgs a) {
    using E = Elem<T>;
    typedef typename E::frag frag;
    static_assert(kPrepLds<T> >= 256 * (kPrepHeads + 1) * 4, "cumsum tile must fit");
    __shared__ __align__(16) unsigned char smem[kPrepLds<T>];
    float (*lt)[kPrepHeads + 1] = reinterpret_cast<float (*)[kPrepHeads + 1]>(smem);
    // (the wavefront index is uniform: in a scalar register, so are the tile coordinates)
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 31, lg = lane >> 5;
    // (the C B^T workgroups first: the longer role is dispatched to compute units of its
    // own before the cumsum workgroups double up)
    int bid = blockIdx.x;
    const bool cs_role = bid >= a.cb_blocks;
    int k, rest;
    if (cs_role) {
        bid -= a.cb_blocks;
        k = bid / a.hblocks;
        rest = bid % a.hblocks;
    } else {
        k = bid / a.G;
        rest = bid % a.G;
    }
    int64_t rowc;
    int len;
    if (!locate_chunk(k, a.seq_offsets, a.T, a.Q, a.nseq, &rowc, &len)) return;

    if (cs_role) {
        // (a) a Qp x 16 block of logA (tokens x heads) through LDS with coalesced loads,
        //     then one wavefront per head: 4 consecutive tokens per lane and a lane scan.
        const int h0 = rest * kPrepHeads;
        const int nh = min(kPrepHeads, a.H - h0);
        constexpr int per = 256 * kPrepHeads / kPrepThreads;   // values per thread for Qp = 256
        for (int base = 0; base < a.Qp * kPrepHeads; base += per * kPrepThreads) {
            float v[per];
#pragma unroll
            for (int q = 0; q < per; ++q) {
                const int idx = base + tid + kPrepThreads * q;
                const int r = idx / kPrepHeads, hh = idx % kPrepHeads;
                v[q] = (r < len && hh < nh) ? a.logA[(rowc + r) * a.H + h0 + hh] : 0.f;
            }
#pragma unroll
            for (int q = 0; q < per; ++q) {
                const int idx = base + tid + kPrepThreads * q;
                if (idx < a.Qp * kPrepHeads) lt[idx / kPrepHeads][idx % kPrepHeads] = v[q];
            }
        }
        __syncthreads();
        for (int hh = wave; hh < nh; hh += kPrepWaves) {
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = (4 * lane + j < a.Qp) ? lt[4 * lane + j][hh] : 0.f;
            v[1] += v[0];
            v[2] += v[1];
            v[3] += v[2];
            const float excl = wave_inclusive_sum(v[3], lane) - v[3];
            const f32x4 o = {(excl + v[0]) * kLog2e, (excl + v[1]) * kLog2e, (excl + v[2]) * kLog2e,
                             (excl + v[3]) * kLog2e};
            if (4 * lane < a.Qp) *reinterpret_cast<f32x4*>(a.cs + ((int64_t)k * a.H + h0 + hh) * a.Qp + 4 * lane) = o;
        }
        return;
    }

    // (b) C B^T of one (chunk slot, group): all ntile lower tiles (i, j), j <= i, of the
    // chunk.  B and C rows of the chunk go through LDS in slabs of columns (rows past the
    // chunk's end as zeros), and wavefront w accumulates tiles w, w + 4, ... over the
    // slabs, so every row is read from memory once per (chunk, group).  Each tile is
    // computed transposed, D[s][l] = sum_n B[s][n] C[l][n], so that each lane ends with
    // one row l of C B^T and writes it as runs of 4 consecutive s.  Tiles are stored in
    // the order of the walk kernels' B-operand fragments: element (l, s) of a tile sits
    // at ((s / 16) * 64 + ((s % 16) / 8) * 32 + l) * 8 + s % 8, so one fragment of one
    // wavefront is 1 KB of contiguous memory.
    constexpr int SW = kCbSlab<T>, SS = kCbStride<T>;
    constexpr int MAXT = (36 + kPrepWaves - 1) / kPrepWaves;   // tiles per wavefront, 256-row chunks
    const int g = rest;
    T* Bs = reinterpret_cast<T*>(smem);
    T* Cs = Bs + 256 * SS;
    const char* Bp = static_cast<const char*>(a.B);
    const char* Cp = static_cast<const char*>(a.C);
    // tile u of this wavefront: (ti, tj), stored as tile tt of the chunk (tt >= ntile: none)
    int ti[MAXT], tj[MAXT], tt[MAXT];
#pragma unroll
    for (int u = 0; u < MAXT; ++u) {
        const int t = wave + kPrepWaves * u;
        int i = 0;
        while ((i + 1) * (i + 2) / 2 <= t) ++i;
        ti[u] = i;
        tj[u] = t - i * (i + 1) / 2;
        tt[u] = t;
    }
    f32x16 acc[MAXT];
#pragma unroll
    for (int u = 0; u < MAXT; ++u) acc[u] = f32x16{};
    constexpr int pieces = SW * (int)sizeof(T) / 16;   // 16-byte pieces per slab row
    constexpr int PPT = 256 * pieces / kPrepThreads;   // pieces per thread for 256 rows
    // global columns walked: [0, cb_n) for the tiles, or only the fragment copies' range
    const int col_lo = a.cb_n > 0 ? 0 : a.n0, col_hi = a.cb_n > 0 ? a.cb_n : a.n0 + a.N;
    // One slab's pieces are loaded into registers at once (all of a thread's loads in
    // flight together), and the next slab's loads are issued before the current slab is
    // used, so their latency overlaps the MFMAs and the fragment stores.
    uint4 rb[PPT], rc[PPT];
    auto load_slab = [&](int cg) {
#pragma unroll
        for (int u = 0; u < PPT; ++u) {
            const int idx = tid + kPrepThreads * u;
            const int r = idx / pieces, c = (idx % pieces) * (16 / (int)sizeof(T));
            rb[u] = uint4{0u, 0u, 0u, 0u};
            rc[u] = uint4{0u, 0u, 0u, 0u};
            // (the widths are multiples of 16, so a 16-byte piece is wholly inside or past)
            if (r < len && cg + c < col_hi) {
                const int64_t off = (((rowc + r) * a.G + g) * (int64_t)a.ldn + cg + c) * (int64_t)sizeof(T);
                rb[u] = *reinterpret_cast<const uint4*>(Bp + off);
                rc[u] = *reinterpret_cast<const uint4*>(Cp + off);
            }
        }
    };
    load_slab(col_lo);
    for (int cg = col_lo; cg < col_hi; cg += SW) {
        const int n0 = cg - a.n0;   // column within the fragment copies' range
        __syncthreads();   // the previous slab has been read
#pragma unroll
        for (int u = 0; u < PPT; ++u) {
            const int idx = tid + kPrepThreads * u;
            const int r = idx / pieces, c = (idx % pieces) * (16 / (int)sizeof(T));
            if (r < a.Qp) {
                *reinterpret_cast<uint4*>(Bs + r * SS + c) = rb[u];
                *reinterpret_cast<uint4*>(Cs + r * SS + c) = rc[u];
            }
        }
        __syncthreads();
        if (cg + SW < col_hi) load_slab(cg + SW);
        if constexpr (sizeof(T) == 2) {
            // (c) for the split walker (256-row chunks; the slab holds n tiles n0 / 32 and
            //     n0 / 32 + 1): B^T as A-operand fragments, (nt, j, ks) lane (lr, lg)
            //     holding B[32 j + 16 ks + 8 lg + q][32 nt + lr], and C as B-operand
            //     fragments, (j, ks) lane (lr, lg) holding C[32 j + lr][16 ks + 8 lg + q]:
            //     one fragment is 1 KB of contiguous memory
            if (a.bt) {
                for (int o = tid; o < (SW / 32) * 16 * 64; o += kPrepThreads) {
                    const int sub = o >> 10, ln = o & 63, f = (o >> 6) & 15, j = f >> 1, ks = f & 1;
                    const int ns = n0 + 32 * sub;   // the n tile's first column within the copies' range
                    const bool second = a.bt2 && ns >= a.N && ns < 2 * a.N;
                    if (!((ns >= 0 && ns < a.N) || second)) continue;
                    const int nf = second ? ns - a.N : ns;   // column within its half
                    const int nt = nf / 32;
                    T* bto = static_cast<T*>(second ? a.bt2 : a.bt) + (int64_t)(k * a.G + g) * (a.N / 32) * 16 * 512;
                    T* cto = static_cast<T*>(second ? a.ct2 : a.ct) + (int64_t)(k * a.G + g) * 8 * (a.N / 16) * 512;
                    frag v;
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        v[q] = Bs[(32 * j + 16 * ks + 8 * (ln >> 5) + q) * SS + 32 * sub + (ln & 31)];
                    *reinterpret_cast<frag*>(bto + ((nt * 8 + j) * 2 + ks) * 512 + ln * 8) = v;
                    const frag w = E::lds8(Cs + (32 * j + (ln & 31)) * SS + 32 * sub + 16 * ks + 8 * (ln >> 5));
                    *reinterpret_cast<frag*>(cto + (j * (a.N / 16) + nf / 16 + ks) * 512 + ln * 8) = w;
                }
            }
        }
        if (a.cb_n == 0) continue;
#pragma unroll
        for (int u = 0; u < MAXT; ++u) {
            if (tt[u] >= a.ntile) break;
#pragma unroll
            for (int ks = 0; ks < SW / 16; ++ks) {
                const frag av = E::lds8(Bs + (32 * tj[u] + lr) * SS + 16 * ks + 8 * lg);
                const frag bv = E::lds8(Cs + (32 * ti[u] + lr) * SS + 16 * ks + 8 * lg);
                acc[u] = E::mma(acc[u], av, bv);
            }
        }
    }
    if (a.cb_n == 0) return;
#pragma unroll
    for (int u = 0; u < MAXT; ++u) {
        const int t = tt[u];
        if (t >= a.ntile) break;
        T* out = static_cast<T*>(a.cb) + ((int64_t)(k * a.G + g) * a.ntile + t) * 1024;
        if (ti[u] == tj[u]) {
            // diagonal tiles carry the causal mask: (C B^T)_{ls} = 0 for s > l
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (acc_row(e, lane) > lr) acc[u][e] = 0.f;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // rows s = 8q + 4lg + 0..3 of this lane's column l = lr
            T* o = out + (((q >> 1) * 64 + (q & 1) * 32 + lr) * 8 + 4 * lg);
            E::st4(o, acc[u][4 * q], acc[u][4 * q + 1], acc[u][4 * q + 2], acc[u][4 * q + 3]);
        }
    }
}

// y <- y + z elementwise (float32 sums, stored in the element type), 8 values per thread:
// the two column halves of a d_state that is walked as two passes
template <typename T>
__global__ void __launch_bounds__(256) ssd_add_kernel(T* y, const T* z, int64_t n8) {
    using E = Elem<T>;
    typedef typename E::frag frag;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
        const frag a = E::ldg8(y + 8 * i), b = E::ldg8(z + 8 * i);
        frag o;
#pragma unroll
        for (int q = 0; q < 8; ++q) o[q] = E::from_f(E::to_f(a[q]) + E::to_f(b[q]));
        *reinterpret_cast<frag*>(y + 8 * i) = o;
    }
}

// One recurrent step of every (sequence, head): h <- a h + x B^T, y = h C (page "Transformers
// are SSMs" paper summary, section 2.4 with A_t = a_t I; the recurrent mode of section 3,
// one token at a time from a state the forward pass returned).  One 256-thread workgroup
// per (sequence, head) streams the P x N state once: each of the first N/4 threads of a
// row owns 4 consecutive state entries of that row per pass, and a row's threads (N/4
// rounded up to a power of two, so that a row is a run of lanes inside one wavefront and
// the rows of a pass tile the workgroup exactly) reduce y[p] with lane shuffles.  The
// state goes from HBM to registers and back, nothing is staged.
template <typename T>
__global__ void __launch_bounds__(256) ssd_decode_kernel(DecodeArgs a) {
    using E = Elem<T>;
    const int bh = blockIdx.x;
    const int b = bh / a.H, h = bh % a.H, g = h / (a.H / a.G);
    const int tid = threadIdx.x;
    const int nq = a.N / 4;                  // threads of a row that hold state (4 .. 64)
    int tpr = 4;                             // threads per state row: nq rounded up to a
    while (tpr < nq) tpr <<= 1;              // power of two (4 .. 64)
    const int rpp = 256 / tpr;               // rows per pass
    const int j = tid % tpr, rsub = tid / tpr;
    const bool holds = j < nq;
    float b0 = 0.f, b1 = 0.f, b2 = 0.f, b3 = 0.f, c0 = 0.f, c1 = 0.f, c2 = 0.f, c3 = 0.f;
    if (holds) {
        const T* Bv = static_cast<const T*>(a.B) + ((int64_t)b * a.G + g) * a.N + 4 * j;
        const T* Cv = static_cast<const T*>(a.C) + ((int64_t)b * a.G + g) * a.N + 4 * j;
        b0 = E::to_f(Bv[0]), b1 = E::to_f(Bv[1]), b2 = E::to_f(Bv[2]), b3 = E::to_f(Bv[3]);
        c0 = E::to_f(Cv[0]), c1 = E::to_f(Cv[1]), c2 = E::to_f(Cv[2]), c3 = E::to_f(Cv[3]);
    }
    const float da = fast_exp2(a.logA[(int64_t)b * a.H + h] * kLog2e);
    const T* xv = static_cast<const T*>(a.x) + ((int64_t)b * a.H + h) * a.P;
    T* yv = static_cast<T*>(a.y) + ((int64_t)b * a.H + h) * a.P;
    float* st = a.state + ((int64_t)b * a.H + h) * a.P * (int64_t)a.N;
    for (int p0 = 0; p0 < a.P; p0 += rpp) {
        const int p = p0 + rsub;
        float part = 0.f;
        if (p < a.P && holds) {
            f32x4* s4 = reinterpret_cast<f32x4*>(st + (int64_t)p * a.N + 4 * j);
            const float xp = E::to_f(xv[p]);
            f32x4 v = *s4;
            v[0] = da * v[0] + xp * b0;
            v[1] = da * v[1] + xp * b1;
            v[2] = da * v[2] + xp * b2;
            v[3] = da * v[3] + xp * b3;
            *s4 = v;
            part = v[0] * c0 + v[1] * c1 + v[2] * c2 + v[3] * c3;
        }
        // sum over the tpr threads of the row (consecutive lanes of one wavefront)
        for (int d = tpr >> 1; d > 0; d >>= 1) part += __shfl_xor(part, d, 64);
        if (p < a.P && j == 0) yv[p] = E::from_f(part);
    }
}

template <typename T, int PT, int NP, bool CBL>
__global__ void __launch_bounds__(512) ssd_walk_kernel(WalkArgs a) {
    using E = Elem<T>;
    typedef typename E::frag frag;
    constexpr int PAD = 16 / sizeof(T);
    constexpr int XS = PT + PAD, BS = NP + PAD, HS = NP + PAD;
    constexpr int PSUB = PT / 32, NT = NP / 32;
    constexpr int NTILE_S = PSUB * NT;
    constexpr int TPW = (NTILE_S + 7) / 8;
    // register prefetch of the next chunk: X rows (PT/8 fragments of 8 per row) and,
    // when a whole chunk of B fits in LDS and in registers, B rows (NP/8 fragments)
    constexpr int XSEG = PT / 8, BSEG = NP / 8;
    constexpr int XPASS = (256 * XSEG + 511) / 512;
    constexpr int BPASS = (256 * BSEG + 511) / 512;
    // B of the next chunk is not held in registers across the output phase (registers
    // are the limit there); it is loaded straight into LDS when the chunk is committed
    constexpr bool BPRE = false;
    constexpr int BPASS_R = 1;
    constexpr int KC = NP / 16 < 4 ? NP / 16 : 4;   // C fragments issued per batch
    // off-diagonal C B^T tiles of one chunk (at most 28 for 8 blocks), 128 fragments each
    constexpr int CBPASS = (28 * 128 + 511) / 512;

    extern __shared__ __align__(16) unsigned char smem[];
    T* Xs = reinterpret_cast<T*>(smem + a.xs_off);
    T* Xts = reinterpret_cast<T*>(smem + a.xts_off);
    T* Bs = reinterpret_cast<T*>(smem + a.bs_off);
    T* CBs = Bs;   // the off-diagonal C B^T tiles reuse the B region after the state phase
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
    constexpr bool cb_lds = CBL;

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
    const bool one_stage = a.qb >= a.Qp;

    const T* X = static_cast<const T*>(a.X);
    const T* Bg = static_cast<const T*>(a.B);
    const T* Cg = static_cast<const T*>(a.C);
    T* Y = static_cast<T*>(a.Y);
    const int64_t state_base = ((int64_t)s * H + h) * P * (int64_t)N;
    const int XH = a.xh, xhi = h / (H / XH);   // X row of this head

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

    auto chunk_rows = [&](int c, int64_t* rowc, int* len) {
        *rowc = row0 + (int64_t)c * Q;
        *len = min(Q, len_seq - c * Q);
        return ((*len + 31) >> 5) * 32;
    };

    // ---- staging of X, X~, B and the cumsum: global -> registers -> LDS
    frag px[XPASS];
    float pcs_r[XPASS], pcs_e[XPASS];
    frag pb[BPASS_R];
    float pcs;
    constexpr uint32_t ES = sizeof(T);
    auto x_rsrc = [&](int64_t rowc, int len) {
        return make_rsrc(X + rowc * XH * (int64_t)P, (uint32_t)len * XH * P * ES);
    };
    auto bc_rsrc = [&](const T* base, int64_t rowc, int len) {
        return make_rsrc(base + rowc * G * (int64_t)N, (uint32_t)len * G * N * ES);
    };
    auto prefetch_in = [&](int c) {
        int64_t rowc;
        int len;
        const int rows = chunk_rows(c, &rowc, &len);
        const rsrc_t xr = x_rsrc(rowc, len);
        const rsrc_t csr = make_rsrc(a.cs + ((int64_t)(slot0 + c) * H + h) * a.Qp, rows * 4);
#pragma unroll
        for (int k = 0; k < XPASS; ++k) {
            const int idx = tid + 512 * k;
            const int r = idx / XSEG, c8 = (idx % XSEG) * 8;
            const int p = p_base + c8;
            px[k] = E::ldb8(xr, p < P ? (uint32_t)((r * XH + xhi) * P + p) * ES : kOutOfRange);
            pcs_r[k] = ldb_f32(csr, 4u * r);
            pcs_e[k] = ldb_f32(csr, 4u * (r | 31));
        }
        if (BPRE && one_stage) {
            const rsrc_t br = bc_rsrc(Bg, rowc, len);
#pragma unroll
            for (int k = 0; k < BPASS_R; ++k) {
                const int idx = tid + 512 * k;
                const int r = idx / BSEG, c8 = (idx % BSEG) * 8;
                pb[k] = E::ldb8(br, c8 < N ? (uint32_t)((r * G + g) * N + c8) * ES : kOutOfRange);
            }
        }
        pcs = ldb_f32(csr, 4u * tid);
    };
    // B rows [rb0, rb1) of chunk c straight into LDS, all loads of a batch issued first
    auto load_b_rows = [&](int c, int rb0, int rb1) {
        int64_t rowc;
        int len;
        chunk_rows(c, &rowc, &len);
        const rsrc_t br = bc_rsrc(Bg, rowc, len);
        constexpr int BB = 8;
        for (int base = 0; base < (rb1 - rb0) * BSEG; base += BB * 512) {
            frag v[BB];
#pragma unroll
            for (int k = 0; k < BB; ++k) {
                const int idx = base + tid + 512 * k;
                const int r = rb0 + idx / BSEG, c8 = (idx % BSEG) * 8;
                v[k] = E::ldb8(br, (c8 < N && r < rb1) ? (uint32_t)((r * G + g) * N + c8) * ES : kOutOfRange);
            }
#pragma unroll
            for (int k = 0; k < BB; ++k) {
                const int idx = base + tid + 512 * k;
                const int r = rb0 + idx / BSEG, c8 = (idx % BSEG) * 8;
                if (r < rb1) *reinterpret_cast<frag*>(Bs + (r - rb0) * BS + c8) = v[k];
            }
        }
    };
    auto commit_in = [&](int c) {
        int64_t rowc;
        int len;
        const int rows = chunk_rows(c, &rowc, &len);
#pragma unroll
        for (int k = 0; k < XPASS; ++k) {
            const int idx = tid + 512 * k;
            const int r = idx / XSEG, c8 = (idx % XSEG) * 8;
            if (r < rows) {
                const float f = fast_exp2(pcs_e[k] - pcs_r[k]);
                frag vt;
#pragma unroll
                for (int q = 0; q < 8; ++q) vt[q] = E::from_f(E::to_f(px[k][q]) * f);
                *reinterpret_cast<frag*>(Xs + r * XS + c8) = px[k];
                *reinterpret_cast<frag*>(Xts + r * XS + c8) = vt;
            }
        }
        if (BPRE && one_stage) {
#pragma unroll
            for (int k = 0; k < BPASS_R; ++k) {
                const int idx = tid + 512 * k;
                const int r = idx / BSEG, c8 = (idx % BSEG) * 8;
                if (r < rows) *reinterpret_cast<frag*>(Bs + r * BS + c8) = pb[k];
            }
        } else if (one_stage) {
            load_b_rows(c, 0, rows);
        }
        if (tid < rows) css[tid] = pcs;
    };

    // ---- operands of the output phase, prefetched during the state phase
    frag pcb[cb_lds ? CBPASS : 1];   // off-diagonal C B^T tiles of the chunk (staged to LDS)
    frag pdg[4];            // diagonal C B^T fragments of this wave's first unit
    frag pc1[KC];           // first C fragments of this wave's first tile
    auto row_of_offdiag = [](int o) {   // o = i (i - 1) / 2 + j, j < i  ->  i
        int i = 1;
        while ((i + 1) * i / 2 <= o) ++i;
        return i;
    };
    auto cb_rsrc = [&](int slot) {
        return make_rsrc(static_cast<const T*>(a.cb) + (int64_t)(slot * G + g) * a.ntile * 1024,
                         (uint32_t)a.ntile * 1024 * ES);
    };
    // byte offset of the C fragment (row l of the chunk, K-step ks) of this lane
    auto c_off = [&](int l, int ks) {
        return 16 * ks < N ? (uint32_t)((l * G + g) * N + 16 * ks + 8 * lg) * ES : kOutOfRange;
    };
    auto prefetch_out = [&](int c) {
        int64_t rowc;
        int len;
        const int rows = chunk_rows(c, &rowc, &len);
        const int nlb = rows >> 5;
        const rsrc_t cbr = cb_rsrc(slot0 + c);
        if constexpr (cb_lds) {
            const int nto = nlb * (nlb - 1) / 2;
#pragma unroll
            for (int k = 0; k < CBPASS; ++k) {
                const int e = tid + 512 * k;
                const int o = e >> 7, f = e & 127;
                pcb[k] = E::ldb8(cbr, o < nto ? (uint32_t)((o + row_of_offdiag(o)) * 1024 + f * 8) * ES : kOutOfRange);
            }
        }
        const int npairs = (nlb + 1) >> 1;
        if (wave < npairs * PSUB) {
            const int pa = wave / PSUB;
            const int i1 = pa, i2 = nlb - 1 - pa;
            const bool two = i2 != i1;
            const uint32_t d1 = (uint32_t)((i1 * (i1 + 1) / 2 + i1) * 1024 + lane * 8) * ES;
            const uint32_t d2 = two ? (uint32_t)((i2 * (i2 + 1) / 2 + i2) * 1024 + lane * 8) * ES : kOutOfRange;
            pdg[0] = E::ldb8(cbr, d1);
            pdg[1] = E::ldb8(cbr, d1 + 512 * ES);
            pdg[2] = E::ldb8(cbr, d2);
            pdg[3] = E::ldb8(cbr, two ? d2 + 512 * ES : kOutOfRange);
            const rsrc_t cr = bc_rsrc(Cg, rowc, len);
#pragma unroll
            for (int q = 0; q < KC; ++q) pc1[q] = E::ldb8(cr, c_off(32 * i1 + lr, q));
        }
    };

    auto cb_frag_diag = [&](rsrc_t cbr, int i, int ks) {
        return E::ldb8(cbr, (uint32_t)((i * (i + 1) / 2 + i) * 1024 + ks * 512 + lane * 8) * ES);
    };

    if (nchunks > 0) {
        prefetch_in(0);
        commit_in(0);
    }
    write_state_lds();
    __syncthreads();

    for (int c = 0; c < nchunks; ++c) {
        int64_t rowc;
        int len;
        const int rows = chunk_rows(c, &rowc, &len);
        const int nlb = rows >> 5;
        const int slot = slot0 + c;
        prefetch_out(c);

        // ---- state phase: h = 2^(cs_last) h + B^T (decay o X), telescoped block by
        //      block: h = 2^(cs[e_j] - cs[e_{j-1}]) h + B_j^T X~_j   (right and center factors)
        float prev[TPW];
#pragma unroll
        for (int k = 0; k < TPW; ++k) prev[k] = 0.f;
        const int bpb = one_stage ? nlb : a.qb / 32;   // 32-row blocks per B stage
        for (int jb0 = 0; jb0 < nlb; jb0 += bpb) {
            const int jb1 = min(nlb, jb0 + bpb);
            if (!one_stage) {
                __syncthreads();
                load_b_rows(c, 32 * jb0, 32 * jb1);
                __syncthreads();
            }
#pragma unroll
            for (int k = 0; k < TPW; ++k) {
                const int t = wave + 8 * k;
                if (t >= NTILE_S) continue;
                const int n0 = 32 * (t / PSUB), p0 = 32 * (t % PSUB);
                if (n0 >= N || p_base + p0 >= P) continue;
                for (int j = jb0; j < jb1; ++j) {
                    const frag a0 = lds_col<T>(Bs, BS, 32 * (j - jb0), n0, lane);
                    const frag b0 = lds_col<T>(Xts, XS, 32 * j, p0, lane);
                    const frag a1 = lds_col<T>(Bs, BS, 32 * (j - jb0) + 16, n0, lane);
                    const frag b1 = lds_col<T>(Xts, XS, 32 * j + 16, p0, lane);
                    const float e = css[32 * j + 31];
                    hacc[k] *= fast_exp2(e - prev[k]);
                    prev[k] = e;
                    hacc[k] = E::mma(hacc[k], a0, b0);
                    hacc[k] = E::mma(hacc[k], a1, b1);
                }
            }
        }
        __syncthreads();
        if constexpr (cb_lds) {
            const int nto = nlb * (nlb - 1) / 2;
#pragma unroll
            for (int k = 0; k < CBPASS; ++k) {
                const int e = tid + 512 * k;
                if ((e >> 7) < nto) *reinterpret_cast<frag*>(CBs + e * 8) = pcb[k];
            }
        }
        // the next chunk's inputs travel while the outputs of this one are computed
        if (c + 1 < nchunks) prefetch_in(c + 1);
        if constexpr (cb_lds) __syncthreads();

        // ---- output phase: tiles Y^T[p][l] for (32-row block i, 32-wide p sub-tile).
        //      A wave takes blocks i1 = pa and i2 = nlb-1-pa of one p sub-tile, so the
        //      causal work is balanced and the X~ fragments are shared by both tiles.
        const rsrc_t cbr = cb_rsrc(slot);
        const rsrc_t cr = bc_rsrc(Cg, rowc, len);
        auto cb_frag = [&](int i, int j, int ks) -> frag {
            if constexpr (cb_lds) return E::lds8(CBs + (i * (i - 1) / 2 + j) * 1024 + ks * 512 + lane * 8);
            return E::ldb8(cbr, (uint32_t)((i * (i + 1) / 2 + j) * 1024 + ks * 512 + lane * 8) * ES);
        };
        // one output tile: block i, p sub-tile p0; the first unit of a wave takes its
        // diagonal and first C fragments from the prefetch registers
        auto out_tile = [&](int i, int p0, bool pre, frag da, frag db) {
            const bool lvalid = 32 * i + lr < len;
            f32x16 acc = {};
            // left factor: acc = h C_l^T over n, C fragments issued KC at a time
#pragma unroll
            for (int kb = 0; kb < NP / 16; kb += KC) {
                frag cf[KC];
#pragma unroll
                for (int q = 0; q < KC; ++q) cf[q] = (pre && kb == 0) ? pc1[q] : E::ldb8(cr, c_off(32 * i + lr, kb + q));
#pragma unroll
                for (int q = 0; q < KC; ++q) {
                    if (16 * (kb + q) >= N) continue;
                    const frag av = E::lds8(hs + (p0 + lr) * HS + 16 * (kb + q) + 8 * lg);
                    acc = E::mma(acc, av, cf[q]);
                }
            }
            // earlier blocks j through (C B^T)_{ij} and X~_j, decayed block to block
            float prevf = 0.f;
            for (int j = 0; j < i; ++j) {
                const frag x0 = lds_col<T>(Xts, XS, 32 * j, p0, lane);
                const frag x1 = lds_col<T>(Xts, XS, 32 * j + 16, p0, lane);
                const frag u0 = cb_frag(i, j, 0), u1 = cb_frag(i, j, 1);
                const float e = css[32 * j + 31];
                acc *= fast_exp2(e - prevf);
                prevf = e;
                acc = E::mma(acc, x0, u0);
                acc = E::mma(acc, x1, u1);
            }
            // row scale and diagonal tile: exact mask 2^(cs[l] - cs[s]), s <= l, on unscaled X
            const int l0 = 32 * i;
            const float csl = css[l0 + lr];
            acc *= fast_exp2(csl - prevf);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const frag av = lds_col<T>(Xs, XS, l0 + 16 * ks, p0, lane);
                const frag raw = ks == 0 ? da : db;
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
            const bool first = u == wave;
            const int ps = u % PSUB, pa = u / PSUB;
            const int p0 = 32 * ps;
            if (p_base + p0 >= P) continue;
            const int i1 = pa, i2 = nlb - 1 - pa;
            if (first) out_tile(i1, p0, true, pdg[0], pdg[1]);
            else out_tile(i1, p0, false, cb_frag_diag(cbr, i1, 0), cb_frag_diag(cbr, i1, 1));
            if (i2 != i1) {
                if (first) out_tile(i2, p0, false, pdg[2], pdg[3]);
                else out_tile(i2, p0, false, cb_frag_diag(cbr, i2, 0), cb_frag_diag(cbr, i2, 1));
            }
        }
        __syncthreads();
        write_state_lds();
        if (c + 1 < nchunks) commit_in(c + 1);
        __syncthreads();
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
