// ssd_walk_split.h -- the chunk walker for the common Mamba-2 layer shapes on gfx950:
// bf16 operands, 256-row chunks, 64-wide tiles of the head dimension, d_state 64 or
// 128 (page "Transformers are SSMs" paper summary, sections 6 and 6.2; the
// head/state sizes of section 9 and the chunk length used there).
//
// It computes what ssd_walk_kernel computes (same decompositions, same factors), with
// another division of the work inside the workgroup:
//
//   eight wavefronts, two per SIMD.  Waves 0-3 ("state waves") carry the recurrence
//   h_{c+1} = 2^(cs_last) h_c + B_c^T (decay o X_c); waves 4-7 ("output waves")
//   compute Y_c from h_c, C_c, (C B^T)_c and X_c.  Both read the same staged chunk
//   and run at the same time, sharing each SIMD's matrix and vector pipes.
//
//   Operands shared by the heads of a group come from global memory (L2) straight
//   into registers, already in MFMA fragment order: B^T (written by the prep kernel)
//   for the state waves, C rows and C B^T tiles for the output waves.  Each set is
//   reloaded for the next chunk as soon as it has been consumed.  Only per-head data
//   is staged in LDS: X, X~ and the cumsum of the chunk, and h at its start.
//
//   The state waves also stage the next chunk (X~ and the cumsum) and h_{c+1}.  X~
//   and the cumsum are double-buffered, h is not, which gives two barriers per chunk:
//     state waves : state(c), X~ of c+1               | B_mid | store Y of block i2,
//                                                      |       | write h of c+1
//     output waves: block i2 whole, block i1 up to its | B_mid | block i1's diagonal
//                   chain                              |       |
//     then B_end, after which the state waves store Y of block i1.  (h of chunk c is
//   last read before B_mid; X~ and the cumsum of chunk c may be read after it: the
//   state waves write the other buffer.)  Output tiles go through LDS, where the
//   state waves, which have time to spare, pick them up and write whole 128-byte rows
//   of Y (a lane of an output wave holds 16 of a row's values in 4-value pieces).
//
//   An output wave owns the 32-row blocks k and 7 - k of the chunk for both 32-wide
//   p sub-tiles, so the causal work is the same for every output wave, and every C,
//   C B^T and decay-mask fragment it builds feeds two MFMAs.
//
//   All block loops are unrolled: a ragged last chunk is computed in full with zero
//   X, B and C rows past its end and a flat cumsum there (the prep kernel writes the
//   cumsum of all 256 rows), and its rows past the end are not stored.
#pragma once

#include <type_traits>

#include "ssd_kernels.h"

namespace ssd {

// LDS of the split walker: X~ [2][256][64] (swizzled), h [64][NP + 8], the cumsum
// [2][256], per output wave its two 32 x 64 Y tiles [2][32][72] on their way to global
// memory, and per state wave a private copy of the next chunk's cumsum [256].
template <int NP> struct SplitLds {
    static constexpr int xts = 0;                       // two buffers
    static constexpr int hs = xts + 2 * 256 * 64 * 2;
    static constexpr int hstride = NP + 8;
    static constexpr int cs = hs + 64 * hstride * 2;    // two buffers
    static constexpr int ystride = 72;                  // Y rows padded by 16 bytes
    static constexpr int ys = cs + 2 * 256 * 4;         // [2 blocks][4 output waves]
    static constexpr int csp = ys + 2 * 4 * 32 * ystride * 2;   // [4 state waves][256]
    static constexpr int bytes = csp + 4 * 256 * 4;
};

// LDS of the segment summaries (state waves only): X~ [2][256][64], the cumsum [2][256]
// and the private copies [4][256]; small enough for two workgroups per compute unit.
template <int NP> struct SummaryLds {
    static constexpr int xts = 0;
    static constexpr int cs = xts + 2 * 256 * 64 * 2;
    static constexpr int csp = cs + 2 * 256 * 4;
    static constexpr int bytes = csp + 4 * 256 * 4;
    static constexpr int hs = 0, hstride = NP + 8, ys = 0, ystride = 72;   // not used
};

// Bytes of B^T fragments per (chunk slot, group) in the workspace.
__host__ __device__ constexpr int split_bt_bytes(int N) { return N * 512; }

// A long sequence may be walked as nseg segments of consecutive chunks, one workgroup
// per (sequence, segment, head, P tile), so that few sequences still fill the chip.
// This is the chunk recurrence h_{c+1} = a_c h_c + S_c taken two levels deep, as in a
// scan over an associative operator on pairs (a, S):
// (Only some items may be segmented: those of the last, partial round of workgroups.)
//   SUMMARY = true : every segment but the last is cut into nsplit parts; for each part
//                    the state waves alone walk its chunks from a zero state and store
//                    that state and the part's total log2 decay (256 threads per
//                    workgroup, two workgroups per compute unit);
//   SUMMARY = false: segment k starts from E_k: the initial state (or zero) folded with
//                    the parts of segments 0 .. k-1 in order, E <- 2^(decay) E + state,
//                    in the prologue; it then walks its chunks in full.  Only the last
//                    segment writes the final state.
// LEFT = true: the output waves compute only the left factors 2^(cs[l]) C_l h of every
// block (no C B^T chains or diagonal blocks): the second pass of a d_state walked as two
// column halves, whose within-chunk part the first pass, which sees the full C B^T, holds.
template <int NP, bool SUMMARY, bool LEFT>
__device__ __forceinline__ void walk_split_body(const WalkArgs& a, const int bid, const int nblocks) {
    typedef Elem<__bf16> E;
    typedef bf16x8 frag;
    typedef std::conditional_t<SUMMARY, SummaryLds<NP>, SplitLds<NP>> L;
    typedef LdsMat<__bf16, 64> XL;
    typedef LdsCol<__bf16, 64> XC;
    constexpr int NT = NP / 32;        // 32-wide n tiles
    constexpr int NKS = NP / 16;       // K-steps over n
    constexpr int TPS = NT / 2;        // state tiles per state wave (2 p sub-tiles x NT / 4)
    constexpr int HS = L::hstride;

    extern __shared__ __align__(16) unsigned char smem[];
    __bf16* hs = reinterpret_cast<__bf16*>(smem + L::hs);

    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
    // the wavefront index is uniform: keep it (and every role offset) in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // The whole items and the segments of the tail are remapped to XCDs separately, so
    // that every XCD gets its share of both (dispatch follows the block index).
    const int item = (SUMMARY || a.nwhole == 0) ? xcd_remap(bid, nblocks)
                     : bid < a.nwhole ? xcd_remap(bid, a.nwhole)
                                      : a.nwhole + xcd_remap(bid - a.nwhole, nblocks - a.nwhole);
    if (item >= a.nitems) return;
    // Work items are the (sequence, head, P tile) triples, gi = (s * H + h) * ptiles + pt.
    // The first nwhole walk their whole sequence; each of the other ntail is walked as
    // nseg segments, so that the last round of workgroups still fills the chip.  The walk
    // launch has nwhole + ntail * nseg workgroups (the tail segment-major), the summary
    // launch ntail * (nseg - 1) * nsplit ((segment, part)-major): consecutive workgroups
    // of an XCD share one stretch of chunks and its B, C and C B^T in L2.
    int gi, seg = 0, part = 0, nseg = 1;
    if (SUMMARY) {
        gi = a.nwhole + item % a.ntail;
        const int sp = item / a.ntail;
        part = sp % a.nsplit;
        seg = sp / a.nsplit;
        nseg = a.nseg;
    } else if (item < a.nwhole) {
        gi = item;
    } else {
        const int u = item - a.nwhole;
        gi = a.nwhole + u % a.ntail;
        seg = u / a.ntail;
        nseg = a.nseg;
    }
    if (!SUMMARY && a.lpt) {
        // Packed sequences of different lengths: the units (sequence, group) are dealt to
        // the XCDs round-robin, longest sequence first, each XCD taking its units in that
        // order.  Every XCD gets an equal share of every length (the contiguous ranges
        // above would give one XCD all heads of a long sequence), and the heads of a
        // group, which share B, C and C B^T, stay on one XCD.
        const int ipu = a.H / a.G * a.ptiles;              // items per unit
        const int xcd = bid % 8, slot = bid / 8;
        const int u = (slot / ipu) * 8 + xcd, within = slot % ipu;
        const int r = u / a.G, gg = u % a.G;
        // the sequence of length rank r (longest first, ties by index): one lane per sequence
        const int* off = a.seq_offsets;
        bool mine = false;
        if (lane < a.nseq) {
            const int L = off[lane + 1] - off[lane];
            int rank = 0;
            for (int v = 0; v < a.nseq; ++v) {
                const int Lv = off[v + 1] - off[v];
                rank += (Lv > L) || (Lv == L && v < lane);
            }
            mine = rank == r;
        }
        const int sr = __builtin_ctzll(__ballot(mine));
        gi = (sr * a.H + gg * (a.H / a.G)) * a.ptiles + within;
    }
    const int pt = gi % a.ptiles;
    const int h = gi / a.ptiles % a.H;
    const int s = gi / a.ptiles / a.H;
    const int g = h / (a.H / a.G);
    const int p_base = pt * 64;
    const int H = a.H, P = a.P, N = a.N, G = a.G;

    int64_t row0;
    int len_seq, slot0;
    if (!a.seq_offsets) {
        row0 = (int64_t)s * a.T;
        len_seq = (int)a.T;
        slot0 = s * (int)((a.T + 255) / 256);
    } else {
        row0 = a.seq_offsets[s];
        len_seq = a.seq_offsets[s + 1] - a.seq_offsets[s];
        slot0 = 0;
        for (int u = 0; u < s; ++u) slot0 += (a.seq_offsets[u + 1] - a.seq_offsets[u] + 255) / 256;
    }
    if (nseg > 1) {
        // segments of a batch without seq_offsets: chunks [c0, c1) of sequence s; every
        // segment but the last holds whole chunks only
        const int nc = (len_seq + 255) / 256;
        int c0 = (int)((int64_t)seg * nc / nseg), c1 = (int)((int64_t)(seg + 1) * nc / nseg);
        if (SUMMARY) {
            const int l = c1 - c0;
            c1 = c0 + (part + 1) * l / a.nsplit;
            c0 = c0 + part * l / a.nsplit;
        }
        row0 += (int64_t)c0 * 256;
        slot0 += c0;
        len_seq = min(len_seq, c1 * 256) - c0 * 256;
    }
    const int nchunks = (len_seq + 255) / 256;

    const __bf16* X = static_cast<const __bf16*>(a.X);
    const __bf16* CBg = static_cast<const __bf16*>(a.cb);
    const __bf16* BTg = static_cast<const __bf16*>(a.bt);
    const __bf16* CTg = static_cast<const __bf16*>(a.ct);
    __bf16* Y = static_cast<__bf16*>(a.Y);
    // init / final state of this (sequence, head): rows of ldn values, this call's
    // columns from ns0 (a d_state walked in two passes of half the columns)
    const int64_t state_base = ((int64_t)s * H + h) * P * (int64_t)a.ldn + a.ns0;
    const int XH = a.xh, xhi = h / (H / XH);   // X row of this head

    auto xts_buf = [&](int c) { return reinterpret_cast<__bf16*>(smem + L::xts + (c & 1) * 256 * 64 * 2); };
    auto cs_buf = [&](int c) { return reinterpret_cast<float*>(smem + L::cs + (c & 1) * 256 * 4); };
    auto chunk_at = [&](int c, int64_t* rowc, int* len) {
        *rowc = row0 + (int64_t)c * 256;
        *len = min(256, len_seq - c * 256);
    };
    auto cb_rsrc = [&](int c) {
        return make_rsrc(CBg + (int64_t)((slot0 + c) * G + g) * a.ntile * 1024, (uint32_t)a.ntile * 1024 * 2);
    };

    if (wave < 4) {
        // ========================================================== state waves
        const int sw = wave, ts = tid;
        // state tile u: n tile (sw * TPS + u) / 2, p sub-tile (sw * TPS + u) % 2
        auto tile_n0 = [&](int u) { return 32 * ((sw * TPS + u) >> 1); };
        auto tile_p0 = [&](int u) { return 32 * ((sw * TPS + u) & 1); };
        const int my_nt = (sw * TPS) >> 1;   // the n tile of every state tile of this wave
        f32x16 hacc[TPS];
        frag pbt[16];                         // B^T fragments of the chunk: (block j, K-step)
        frag px[8];

        auto load_bt_to = [&](frag (&dst)[16], int c) {
            const rsrc_t r = make_rsrc(BTg + (int64_t)((slot0 + c) * G + g) * (split_bt_bytes(N) / 2),
                                       (uint32_t)split_bt_bytes(N));
            const uint32_t lb = opaque(16u * lane);
#pragma unroll
            for (int f = 0; f < 16; ++f) dst[f] = E::ldb8(r, lb, (uint32_t)((my_nt * 16 + f) * 1024));
        };
        auto load_bt = [&](int c) { load_bt_to(pbt, c); };
        auto prefetch_x = [&](int c) {
            int64_t rowc;
            int len;
            chunk_at(c, &rowc, &len);
            const rsrc_t xr = make_rsrc(X + rowc * XH * (int64_t)P, (uint32_t)len * XH * P * 2);
            const uint32_t xb = opaque((uint32_t)(((ts >> 3) * XH + xhi) * P + p_base + (ts & 7) * 8) * 2);
            const uint32_t xstep = (uint32_t)(32 * XH * P * 2);
#pragma unroll
            for (int k = 0; k < 8; ++k) px[k] = E::ldb8(xr, xb + k * xstep);
        };
        // The cumsum of a chunk (1 KB, four values per lane) is loaded into registers
        // together with X and written to LDS once the wave no longer reads the buffer:
        // wave 0 fills the shared buffer (c & 1) and reads it itself, waves 1-3 fill and
        // read private copies.  (The destination is a select, not a branch, so that
        // every wave issues the same memory operations and the compiler's wait counts
        // stay exact.)
        float* const csp = reinterpret_cast<float*>(smem + L::csp) + sw * 256;
        auto cs_own = [&](int c) { return sw == 0 ? cs_buf(c) : csp; };
        f32x4 csv;
        auto load_cs = [&](int src) {
            const rsrc_t csr = make_rsrc(a.cs + ((int64_t)(slot0 + src) * H + h) * 256, 256 * 4);
            csv = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(csr, (int)opaque(16u * lane), 0, 0));
        };
        auto put_cs = [&](int c) { *reinterpret_cast<f32x4*>(cs_own(c) + 4 * lane) = csv; };
        // X~ = X scaled by its decay to the end of its 32-row block, from the private copy
        // of the cumsum; done before B_mid, while the output waves still read this chunk
        frag pxt[8];
        auto scale_x = [&](int c) {
            const float* csx = cs_own(c);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int r = (ts >> 3) + 32 * k;
                const float f = fast_exp2(csx[32 * k + 31] - csx[r]);
#pragma unroll
                for (int q = 0; q < 8; ++q) pxt[k][q] = E::from_f(E::to_f(px[k][q]) * f);
            }
        };
        // X~ of chunk c into its LDS buffer (c & 1)
        auto commit_x = [&](int c) {
            __bf16* Xt = xts_buf(c);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int r = (ts >> 3) + 32 * k, c8 = (ts & 7) * 8;
                *reinterpret_cast<frag*>(Xt + XL::idx(r, c8)) = pxt[k];
            }
        };
        // Y tile (block slot u) of output wave sw for chunk c: 8 whole rows per store
        auto store_y = [&](int c, int u) {
            int64_t rowc;
            int len;
            chunk_at(c, &rowc, &len);
            const int i = u == 0 ? sw : 7 - sw;
            const __bf16* ys = reinterpret_cast<const __bf16*>(smem + L::ys) + (u * 4 + sw) * 32 * L::ystride;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r = 8 * t + (lane >> 3);
                const frag v = E::lds8(ys + r * L::ystride + 8 * (lane & 7));
                if (32 * i + r < len)
                    *reinterpret_cast<frag*>(Y + ((rowc + 32 * i + r) * H + h) * (int64_t)P + p_base + 8 * (lane & 7)) = v;
            }
        };
        // h as bf16, packed before B_mid and written after it
        u32x2 hpk[TPS][4];
        auto pack_h = [&]() {
#pragma unroll
            for (int u = 0; u < TPS; ++u)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const bf16x4 v = {(__bf16)hacc[u][4 * q], (__bf16)hacc[u][4 * q + 1],
                                      (__bf16)hacc[u][4 * q + 2], (__bf16)hacc[u][4 * q + 3]};
                    hpk[u][q] = __builtin_bit_cast(u32x2, v);
                }
        };
        auto write_h = [&]() {
#pragma unroll
            for (int u = 0; u < TPS; ++u) {
                const int n0 = tile_n0(u), p = tile_p0(u) + lr;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<u32x2*>(hs + p * HS + n0 + 8 * q + 4 * lg) = hpk[u][q];
            }
        };
        // h = 2^(cs_last) h + B^T (decay o X), telescoped over the 8 blocks.  With one
        // tile per wave the even and odd blocks run as two chains (one chain's rescale
        // overlaps the other's MFMAs), merged at the end; two tiles interleave by
        // themselves.
        constexpr bool DUAL = TPS == 1;
        auto state_chunk_with = [&](int c, const frag (&bt)[16]) {
            const float* css = cs_buf(c);
            const __bf16* Xts = xts_buf(c);
            f32x16 hodd = {};
            float ref0 = 0.f, ref1 = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float e = css[32 * j + 31];
                frag bv[TPS][2];
#pragma unroll
                for (int u = 0; u < TPS; ++u)
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) bv[u][ks] = XC::get(Xts, 32 * j + 16 * ks, tile_p0(u), lane);
                if (DUAL && (j & 1)) {
                    const float f = fast_exp2(e - ref1);
                    ref1 = e;
                    hodd *= f;
                    hodd = E::mma(hodd, bt[2 * j], bv[0][0]);
                    hodd = E::mma(hodd, bt[2 * j + 1], bv[0][1]);
                } else {
                    const float f = fast_exp2(e - ref0);
                    ref0 = e;
#pragma unroll
                    for (int u = 0; u < TPS; ++u) {
                        hacc[u] *= f;
                        hacc[u] = E::mma(hacc[u], bt[2 * j], bv[u][0]);
                        hacc[u] = E::mma(hacc[u], bt[2 * j + 1], bv[u][1]);
                    }
                }
            }
            if constexpr (DUAL) {
                // ref1 is the last block's end: the odd chain needs no factor
                hacc[0] = hacc[0] * fast_exp2(ref1 - ref0) + hodd;
            }
        };
        auto state_chunk = [&](int c) { state_chunk_with(c, pbt); };

        // the state tiles of this wave from / to a float32 state at `base`, rows of ld values
        auto add_state = [&](const float* base, int64_t ld, float f) {
#pragma unroll
            for (int u = 0; u < TPS; ++u) {
                const int n0 = tile_n0(u), p = p_base + tile_p0(u) + lr;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 v = *reinterpret_cast<const f32x4*>(base + (int64_t)p * ld + n0 + 8 * q + 4 * lg);
#pragma unroll
                    for (int e = 0; e < 4; ++e) hacc[u][4 * q + e] = hacc[u][4 * q + e] * f + v[e];
                }
            }
        };
        auto put_state = [&](float* base, int64_t ld) {
#pragma unroll
            for (int u = 0; u < TPS; ++u) {
                const int n0 = tile_n0(u), p = p_base + tile_p0(u) + lr;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 v = {hacc[u][4 * q], hacc[u][4 * q + 1], hacc[u][4 * q + 2], hacc[u][4 * q + 3]};
                    *reinterpret_cast<f32x4*>(base + (int64_t)p * ld + n0 + 8 * q + 4 * lg) = v;
                }
            }
        };
        const int64_t pn = (int64_t)P * N;
        auto summary_at = [&](int k, int j) { return (((int64_t)s * (a.nseg - 1) + k) * a.nsplit + j) * H + h; };
#pragma unroll
        for (int u = 0; u < TPS; ++u) hacc[u] = f32x16{};

        if constexpr (SUMMARY) {
            // ---------------------------------------------- segment summary (state only)
            // One barrier per chunk: X~ is double-buffered and written right after it
            // has been scaled, and nothing else is shared.  The next chunk's cumsum, X
            // and B^T (into the other buffer) are issued in that order before this
            // chunk's products; the wave then waits for all but the 16 B^T loads.
            // Every step issues the same loads (the last chunk's step reloads that chunk
            // into buffers nobody reads again; a step past the end only loads), so the
            // compiler's wait counts need not allow for skipped loads.
            float dsum = 0.f;
            frag pbt2[16];
            if (nchunks > 0) {
                load_cs(0);
                load_bt(0);
                prefetch_x(0);
                put_cs(0);
                scale_x(0);
                commit_x(0);
            }
            __syncthreads();
            auto summary_step = [&](int c, const frag (&cur)[16], frag (&nxt)[16]) {
                const int cn = min(c + 1, nchunks - 1);
                load_cs(cn);
                prefetch_x(cn);
                load_bt_to(nxt, cn);
                __builtin_amdgcn_sched_barrier(0);
                if (c < nchunks) {
                    state_chunk_with(c, cur);
                    dsum += cs_buf(c)[255];
                }
                put_cs(c + 1);
                scale_x(c + 1);
                commit_x(c + 1);
                __syncthreads();
            };
            for (int c = 0; c < nchunks; c += 2) {
                summary_step(c, pbt, pbt2);
                summary_step(c + 1, pbt2, pbt);
            }
            put_state(a.seg_state + summary_at(seg, part) * pn, N);
            if (sw == 0 && pt == 0 && lane == 0) a.seg_decay[summary_at(seg, part)] = dsum;
            return;
        }

        // the entry state of this segment
        if (a.init) add_state(a.init + state_base, a.ldn, 0.f);
        for (int k = 0; k < seg; ++k)
            for (int j = 0; j < a.nsplit; ++j)
                add_state(a.seg_state + summary_at(k, j) * pn, N, fast_exp2(a.seg_decay[summary_at(k, j)]));

        if (nchunks > 0) {
            load_cs(0);
            load_bt(0);
            prefetch_x(0);
            put_cs(0);
        }
        __syncthreads();   // the cumsum of chunk 0 is in LDS
        if (nchunks > 0) {
            scale_x(0);
            commit_x(0);
        }
        pack_h();
        write_h();
        __syncthreads();
        // The loop issues the same loads and stores in every iteration: the last one
        // reloads its own chunk into buffers that nobody reads again (a skipped load
        // would make the compiler wait for every newer one before the next use).
        for (int c = 0; c < nchunks; ++c) {
            const int cn = min(c + 1, nchunks - 1);
            load_cs(cn);
            prefetch_x(cn);
            // keep the prefetch ahead of the products (the scheduler would sink it to
            // shorten the live ranges, and then wait for it right after them)
            __builtin_amdgcn_sched_barrier(0);
            state_chunk(c);
            load_bt(cn);
            put_cs(c + 1);
            scale_x(c + 1);
            // X~ of chunk c + 1 goes to the other buffer, which nobody reads in chunk c:
            // written while the output waves are still before B_mid
            commit_x(c + 1);
            pack_h();
            __syncthreads();   // B_mid: h of chunk c is no longer read
            store_y(c, 1);
            write_h();
            __syncthreads();   // B_end
            store_y(c, 0);
        }
        if (a.final_state && seg == nseg - 1) put_state(a.final_state + state_base, a.ldn);
    } else if constexpr (!SUMMARY) {
        // ========================================================== output waves
        // The two blocks are done one after the other, the later one (longer chain)
        // first; only the second block's diagonal and store come after B_mid.  The code
        // is specialised per block pair, so every chain is straight-line code that the
        // compiler can schedule across steps.
        auto output_role = [&](auto kc) {
        constexpr int ok_ = decltype(kc)::value;
        constexpr int i1 = ok_, i2 = 7 - ok_;   // the wave's two blocks, i1 < i2
        frag pc[2][NKS];    // C fragments (block u: 0 = i1, 1 = i2; K-step), each set
                            // reloaded for the next chunk once its block has taken it
        frag pcb[14];       // off-diagonal C B^T: tile t < i2 is (i2, t), else (i1, 6 - t)
        frag pdg[2][2];     // diagonal C B^T (block, K-step)
        f32x16 acc[2];      // Y^T tiles of the current block (p sub-tile)

        // C rows of block u of chunk c, from the fragment-ordered copy (1 KB per fragment)
        auto load_c = [&](int c, int u) {
            const rsrc_t r = make_rsrc(CTg + (int64_t)((slot0 + c) * G + g) * (split_bt_bytes(N) / 2),
                                       (uint32_t)split_bt_bytes(N));
            const uint32_t lb = opaque(16u * lane);
            const int i = u == 0 ? i1 : i2;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) pc[u][ks] = E::ldb8(r, lb, (uint32_t)((i * NKS + ks) * 1024));
        };
        auto load_cb = [&](int c) {
            const rsrc_t cbr = cb_rsrc(c);
            const uint32_t lb = opaque(16u * lane);
#pragma unroll
            for (int t = 0; t < 7; ++t) {
                // tile (i, j), j <= i, is slot i (i + 1) / 2 + j of the chunk
                const int slot = t < i2 ? i2 * (i2 + 1) / 2 + t : i1 * (i1 + 1) / 2 + 6 - t;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    pcb[2 * t + ks] = E::ldb8(cbr, lb, (uint32_t)(slot * 2048 + ks * 1024));
            }
        };
        auto load_dg = [&](int c, int u) {
            const rsrc_t cbr = cb_rsrc(c);
            const uint32_t lb = opaque(16u * lane);
            const int i = u == 0 ? i1 : i2;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                pdg[u][ks] = E::ldb8(cbr, lb, (uint32_t)((i * (i + 3) / 2) * 2048 + ks * 1024));
        };
        // left factor h C_i^T, then the earlier blocks j < i: the telescoped chain; returns
        // cs[e_{i-1}] (0 for the first block)
        auto left_and_chain = [&](int c, int u) -> float {
            const float* css = cs_buf(c);
            const __bf16* Xts = xts_buf(c);
            const int i = u == 0 ? i1 : i2;
            acc[0] = f32x16{};
            acc[1] = f32x16{};
            // LDS operands are read one step ahead of the MFMAs that take them
            frag hv[2][2];
#pragma unroll
            for (int v = 0; v < 2; ++v) hv[0][v] = E::lds8(hs + (32 * v + lr) * HS + 8 * lg);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                if (ks + 1 < NKS) {
#pragma unroll
                    for (int v = 0; v < 2; ++v)
                        hv[(ks + 1) & 1][v] = E::lds8(hs + (32 * v + lr) * HS + 16 * (ks + 1) + 8 * lg);
                }
#pragma unroll
                for (int v = 0; v < 2; ++v) acc[v] = E::mma(acc[v], hv[ks & 1][v], pc[u][ks]);
            }
            load_c(min(c + 1, nchunks - 1), u);
            float prev = 0.f;
            frag xf[2][2][2];   // (buffer, p sub-tile, K-step)
            if (i > 0) {
#pragma unroll
                for (int v = 0; v < 2; ++v)
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) xf[0][v][ks] = XC::get(Xts, 16 * ks, 32 * v, lane);
            }
#pragma unroll
            for (int j = 0; j < 7; ++j) {
                if (j >= i) break;
                if (j + 1 < i) {
#pragma unroll
                    for (int v = 0; v < 2; ++v)
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks)
                            xf[(j + 1) & 1][v][ks] = XC::get(Xts, 32 * (j + 1) + 16 * ks, 32 * v, lane);
                }
                const float e = css[32 * j + 31];
                const float f = fast_exp2(e - prev);
                prev = e;
                const int t = u == 1 ? j : 6 - j;   // register slot of tile (i, j)
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    acc[v] *= f;
                    acc[v] = E::mma(acc[v], xf[j & 1][v][0], pcb[2 * t]);
                    acc[v] = E::mma(acc[v], xf[j & 1][v][1], pcb[2 * t + 1]);
                }
            }
            return prev;
        };
        // the exact decay mask of a diagonal tile, 2^(cs[l] - cs[s]) (C B^T)_{ls} for s <= l
        // (one fragment serves both p sub-tiles)
        // The diagonal block.  When the block's decay span R = cs[first row] - cs[e_i] is
        // at most 100 (log2 units; Mamba-2 parameters give at most about 74) it is one
        // more step of the chain, on X~ and the causally masked tile (masked once by the
        // prep kernel): acc = 2^(cs[e_i] - cs[e_{i-1}]) acc + (C B^T)_ii X~_i, then the row
        // scale 2^(cs[l] - cs[e_i]) <= 2^R.  Otherwise (very strong decay, where X~ would
        // lose rows to underflow) the exact mask 2^(cs[l] - cs[s]) (C B^T)_{ls} is applied
        // to unscaled X read from global memory.  The tile then goes to this wave's LDS
        // area (block slot u) for the state waves to store.
        auto diag = [&](int c, int u, float prev) {
            const float* css = cs_buf(c);
            const int l0 = 32 * (u == 0 ? i1 : i2);
            const float e = css[l0 + 31];
            const float csl = css[l0 + lr];
            const bool moderate = __builtin_amdgcn_readfirstlane((int)(css[l0] - e <= 100.f)) != 0;
            // acc = f2 (f1 acc + X_blk^T D): the branches only choose X_blk, D, f1 and f2
            const __bf16* xsrc;
            frag dg[2];
            float f1, f2;
            if (moderate) {
                xsrc = xts_buf(c) + l0 * 64;   // row l0 of X~ (the swizzle depends on row & 3 only)
                dg[0] = pdg[u][0];
                dg[1] = pdg[u][1];
                f1 = fast_exp2(e - prev);
                f2 = fast_exp2(csl - e);
            } else {
                // unscaled X of the block from global memory, staged in this wave's Y area
                // (the transposing reads need it in LDS), and the exact mask
                int64_t rowc;
                int len;
                chunk_at(c, &rowc, &len);
                __bf16* xb = reinterpret_cast<__bf16*>(smem + L::ys) + (u * 4 + ok_) * 32 * L::ystride;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    // (opaque: the row indexes of this cold path are not worth registers
                    // held across the loop)
                    const int r = 8 * k + (int)opaque((uint32_t)lane >> 3), c8 = (lane & 7) * 8;
                    const frag v = l0 + r < len ? E::ldg8(X + ((rowc + l0 + r) * XH + xhi) * (int64_t)P + p_base + c8) : E::zero();
                    *reinterpret_cast<frag*>(xb + XL::idx(r, c8)) = v;
                }
                xsrc = xb;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const int sl = 16 * ks + 8 * lg + q;
                        const float w = (sl <= lr) ? E::to_f(pdg[u][ks][q]) * fast_exp2(csl - css[l0 + sl]) : 0.f;
                        dg[ks][q] = E::from_f(w);
                    }
                f1 = fast_exp2(csl - prev);
                f2 = 1.f;
            }
            frag xv[2][2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int v = 0; v < 2; ++v) xv[ks][v] = XC::get(xsrc, 16 * ks, 32 * v, lane);
            acc[0] *= f1;
            acc[1] *= f1;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int v = 0; v < 2; ++v) acc[v] = E::mma(acc[v], xv[ks][v], dg[ks]);
            acc[0] *= f2;
            acc[1] *= f2;
            // the next chunk's diagonal tile of this block travels while this one is used
            load_dg(min(c + 1, nchunks - 1), u);
            __bf16* ys = reinterpret_cast<__bf16*>(smem + L::ys) + (u * 4 + ok_) * 32 * L::ystride;
#pragma unroll
            for (int v = 0; v < 2; ++v)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    E::st4(ys + lr * L::ystride + 32 * v + 8 * q + 4 * lg, acc[v][4 * q], acc[v][4 * q + 1],
                           acc[v][4 * q + 2], acc[v][4 * q + 3]);
        };

        if constexpr (LEFT) {
            // left factor of block u scaled by its rows' decay from the chunk start, then
            // to this wave's LDS area (block slot u) for the state waves to store
            auto left_only = [&](int c, int u) {
                const int i = u == 0 ? i1 : i2;
                acc[0] = f32x16{};
                acc[1] = f32x16{};
                frag hv[2][2];
#pragma unroll
                for (int v = 0; v < 2; ++v) hv[0][v] = E::lds8(hs + (32 * v + lr) * HS + 8 * lg);
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    if (ks + 1 < NKS) {
#pragma unroll
                        for (int v = 0; v < 2; ++v)
                            hv[(ks + 1) & 1][v] = E::lds8(hs + (32 * v + lr) * HS + 16 * (ks + 1) + 8 * lg);
                    }
#pragma unroll
                    for (int v = 0; v < 2; ++v) acc[v] = E::mma(acc[v], hv[ks & 1][v], pc[u][ks]);
                }
                load_c(min(c + 1, nchunks - 1), u);
                const float f = fast_exp2(cs_buf(c)[32 * i + lr]);
                acc[0] *= f;
                acc[1] *= f;
            };
            auto store_acc = [&](int u) {
                __bf16* ys = reinterpret_cast<__bf16*>(smem + L::ys) + (u * 4 + ok_) * 32 * L::ystride;
#pragma unroll
                for (int v = 0; v < 2; ++v)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        E::st4(ys + lr * L::ystride + 32 * v + 8 * q + 4 * lg, acc[v][4 * q], acc[v][4 * q + 1],
                               acc[v][4 * q + 2], acc[v][4 * q + 3]);
            };
            if (nchunks > 0) {
                load_c(0, 1);
                load_c(0, 0);
            }
            __syncthreads();
            __syncthreads();
            for (int c = 0; c < nchunks; ++c) {
                left_only(c, 1);
                store_acc(1);
                left_only(c, 0);
                __syncthreads();   // B_mid
                store_acc(0);
                __syncthreads();   // B_end
            }
            return;
        }
        if (nchunks > 0) {
            load_c(0, 1);
            load_c(0, 0);
            load_cb(0);
            load_dg(0, 1);
            load_dg(0, 0);
        }
        __syncthreads();
        __syncthreads();
        for (int c = 0; c < nchunks; ++c) {
            const float prev2 = left_and_chain(c, 1);
            diag(c, 1, prev2);
            const float prev1 = left_and_chain(c, 0);
            load_cb(min(c + 1, nchunks - 1));
            __syncthreads();   // B_mid: X~ and h of chunk c are no longer read
            diag(c, 0, prev1);
            __syncthreads();   // B_end
        }
        };
        switch (wave & 3) {
            case 0: output_role(std::integral_constant<int, 0>{}); break;
            case 1: output_role(std::integral_constant<int, 1>{}); break;
            case 2: output_role(std::integral_constant<int, 2>{}); break;
            default: output_role(std::integral_constant<int, 3>{}); break;
        }
    }
}

template <int NP, bool SUMMARY, bool LEFT = false>
__global__ void __launch_bounds__(512) ssd_walk_split_kernel(WalkArgs a) {
    walk_split_body<NP, SUMMARY, LEFT>(a, blockIdx.x, gridDim.x);
}

// Both passes of a d_state walked as two column halves in one launch (they are independent
// until their outputs are added): blocks [0, a0.nitems) walk the first half, the rest the
// second (left factors only).  Each range is remapped to the XCDs on its own.
template <int NP>
__global__ void __launch_bounds__(512) ssd_walk_split_pair_kernel(WalkArgs a0, WalkArgs a1) {
    const int bid = blockIdx.x;
    if (bid < a0.nitems) walk_split_body<NP, false, false>(a0, bid, a0.nitems);
    else walk_split_body<NP, false, true>(a1, bid - a0.nitems, a1.nitems);
}

}  // namespace ssd
