// ssd_walk_split.h -- the chunk walker for the common Mamba-2 layer shapes on gfx950:
// bf16 operands, 256-row chunks, 64-wide tiles of the head dimension, d_state 64 or
// 128 (page "Transformers are SSMs" paper summary, sections 6 and 6.2; the
// head/state sizes of section 9 and the chunk length used there).
//
// It computes what ssd_walk_kernel computes (same workspace, same decompositions,
// same factors), with another division of the work inside the workgroup:
//
//   eight wavefronts, two per SIMD.  Waves 0-3 ("state waves") carry the recurrence
//   h_{c+1} = 2^(cs_last) h_c + B_c^T (decay o X_c); waves 4-7 ("output waves")
//   compute Y_c from h_c, C_c, (C B^T)_c and X_c.  The two depend on the same staged
//   chunk only, so they run at the same time and share each SIMD's matrix and vector
//   pipes.
//
//   The state waves also stage the next chunk: its X, B and cumsum travel from HBM
//   into their registers while the current chunk is computed and are written to LDS
//   (with X~) between two barriers at the chunk boundary.  The output waves keep the
//   operands that come from global memory (C rows, C B^T tiles) in registers, each
//   set reloaded for the next chunk as soon as it has been consumed.
//
//   An output wave owns the 32-row blocks k and 7 - k of the chunk for both 32-wide
//   p sub-tiles, so the causal work is the same for every output wave, and every C,
//   C B^T and decay-mask fragment it builds feeds two MFMAs.
//
//   All block loops are unrolled: a ragged last chunk is computed in full with zero
//   X, B and C rows past its end and a flat cumsum there (the prep kernel writes the
//   cumsum of all 256 rows), and its rows past the end are not stored.
#pragma once

#include "ssd_kernels.h"

namespace ssd {

// LDS of the split walker: X and X~ [256][64] (swizzled), B [256][NP] (swizzled),
// h [64][NP + 8], the cumsum [256] and the 8 block-end values of the cumsum.
template <int NP> struct SplitLds {
    static constexpr int xs = 0;
    static constexpr int xts = xs + 256 * 64 * 2;
    static constexpr int bs = xts + 256 * 64 * 2;
    static constexpr int hs = bs + 256 * NP * 2;
    static constexpr int hstride = NP + 8;
    static constexpr int cs = hs + 64 * hstride * 2;
    static constexpr int ends = cs + 256 * 4;
    static constexpr int bytes = ends + 8 * 4;
};

template <int NP>
__global__ void __launch_bounds__(512) ssd_walk_split_kernel(WalkArgs a) {
    typedef Elem<__bf16> E;
    typedef bf16x8 frag;
    typedef SplitLds<NP> L;
    typedef LdsMat<__bf16, 64> XL;
    typedef LdsMat<__bf16, NP> BL;
    typedef LdsCol<__bf16, 64> XC;
    typedef LdsCol<__bf16, NP> BC;
    constexpr int NT = NP / 32;        // 32-wide n tiles
    constexpr int NKS = NP / 16;       // K-steps over n
    constexpr int TPS = NT / 2;        // state tiles per state wave (2 p sub-tiles x NT / 4)
    constexpr int BSEG = NP / 8;       // 16-byte units per B row
    constexpr int BPF = 256 * BSEG / 256;   // B units per state thread
    constexpr int HS = L::hstride;

    extern __shared__ __align__(16) unsigned char smem[];
    __bf16* Xs = reinterpret_cast<__bf16*>(smem + L::xs);
    __bf16* Xts = reinterpret_cast<__bf16*>(smem + L::xts);
    __bf16* Bs = reinterpret_cast<__bf16*>(smem + L::bs);
    __bf16* hs = reinterpret_cast<__bf16*>(smem + L::hs);
    float* css = reinterpret_cast<float*>(smem + L::cs);
    float* ends = reinterpret_cast<float*>(smem + L::ends);

    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
    // the wavefront index is uniform: keep it (and every role offset) in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int item = xcd_remap(blockIdx.x, gridDim.x);
    if (item >= a.nitems) return;
    const int pt = item % a.ptiles;
    const int sh = item / a.ptiles;
    const int h = sh % a.H, s = sh / a.H;
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
    const int nchunks = (len_seq + 255) / 256;

    const __bf16* X = static_cast<const __bf16*>(a.X);
    const __bf16* Bg = static_cast<const __bf16*>(a.B);
    const __bf16* Cg = static_cast<const __bf16*>(a.C);
    const __bf16* CBg = static_cast<const __bf16*>(a.cb);
    __bf16* Y = static_cast<__bf16*>(a.Y);
    const int64_t state_base = ((int64_t)s * H + h) * P * (int64_t)N;

    auto chunk_at = [&](int c, int64_t* rowc, int* len) {
        *rowc = row0 + (int64_t)c * 256;
        *len = min(256, len_seq - c * 256);
    };
    auto cb_rsrc = [&](int c) {
        return make_rsrc(CBg + (int64_t)((slot0 + c) * G + g) * a.ntile * 1024, (uint32_t)a.ntile * 1024 * 2);
    };

    const bool state_role = wave < 4;
    // -------------------------------------------------------------- state waves
    const int sw = wave & 3, ts = tid & 255;
    f32x16 hacc[TPS];
    frag px[8];
    float pcr[8], pce[8], pcs = 0.f;
    frag pb[BPF];
    // state tile u of this wave: n tile (sw * TPS + u) / 2, p sub-tile (sw * TPS + u) % 2
    auto tile_n0 = [&](int u) { return 32 * ((sw * TPS + u) >> 1); };
    auto tile_p0 = [&](int u) { return 32 * ((sw * TPS + u) & 1); };

    auto prefetch_in = [&](int c) {
        int64_t rowc;
        int len;
        chunk_at(c, &rowc, &len);
        const rsrc_t xr = make_rsrc(X + rowc * H * (int64_t)P, (uint32_t)len * H * P * 2);
        const rsrc_t csr = make_rsrc(a.cs + ((int64_t)(slot0 + c) * H + h) * 256, 256 * 4);
        const rsrc_t br = make_rsrc(Bg + rowc * G * (int64_t)N, (uint32_t)len * G * N * 2);
        // lane bases; row k of a family is a uniform step further
        const uint32_t xb = opaque((uint32_t)(((ts >> 3) * H + h) * P + p_base + (ts & 7) * 8) * 2);
        const uint32_t xstep = (uint32_t)(32 * H * P * 2);
        const uint32_t cb0 = opaque(4u * (ts >> 3));
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            px[k] = E::ldb8(xr, xb + k * xstep);
            pcr[k] = ldb_f32(csr, cb0 + 128u * k);
            pce[k] = ldb_f32(csr, 4u * (32 * k + 31));
        }
        pcs = ldb_f32(csr, opaque(4u * ts));
        const uint32_t bb = opaque((uint32_t)(((ts / BSEG) * G + g) * N + (ts % BSEG) * 8) * 2);
        const uint32_t bstep = (uint32_t)((256 / BSEG) * G * N * 2);
#pragma unroll
        for (int k = 0; k < BPF; ++k) pb[k] = E::ldb8(br, bb + k * bstep);
    };
    auto commit_in = [&]() {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int r = (ts >> 3) + 32 * k, c8 = (ts & 7) * 8;
            const float f = fast_exp2(pce[k] - pcr[k]);
            frag vt;
#pragma unroll
            for (int q = 0; q < 8; ++q) vt[q] = E::from_f(E::to_f(px[k][q]) * f);
            *reinterpret_cast<frag*>(Xs + XL::idx(r, c8)) = px[k];
            *reinterpret_cast<frag*>(Xts + XL::idx(r, c8)) = vt;
        }
#pragma unroll
        for (int k = 0; k < BPF; ++k) {
            const int idx = ts + 256 * k;
            const int r = idx / BSEG, c8 = (idx % BSEG) * 8;
            *reinterpret_cast<frag*>(Bs + BL::idx(r, c8)) = pb[k];
        }
        css[ts] = pcs;
        if (ts == 0) {
#pragma unroll
            for (int k = 0; k < 8; ++k) ends[k] = pce[k];
        }
    };
    auto write_h = [&]() {
#pragma unroll
        for (int u = 0; u < TPS; ++u) {
            const int n0 = tile_n0(u), p = tile_p0(u) + lr;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                E::st4(hs + p * HS + n0 + 8 * q + 4 * lg, hacc[u][4 * q], hacc[u][4 * q + 1],
                       hacc[u][4 * q + 2], hacc[u][4 * q + 3]);
        }
    };
    // h = 2^(cs_last) h + B^T (decay o X), telescoped over the 8 blocks.  With one
    // tile per wave the even and odd blocks run as two chains (one chain's rescale
    // overlaps the other's MFMAs), merged at the end; two tiles interleave by
    // themselves.
    constexpr bool DUAL = TPS == 1;
    auto state_chunk = [&]() {
        f32x16 hodd[DUAL ? TPS : 1];
        float ref0 = 0.f, ref1 = 0.f;
        if constexpr (DUAL) hodd[0] = f32x16{};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float e = ends[j];
            frag av[TPS][2], bv[TPS][2];
#pragma unroll
            for (int u = 0; u < TPS; ++u) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    if (u == 0 || tile_n0(u) != tile_n0(0)) av[u][ks] = BC::get(Bs, 32 * j + 16 * ks, tile_n0(u), lane);
                    else av[u][ks] = av[0][ks];
                    bv[u][ks] = XC::get(Xts, 32 * j + 16 * ks, tile_p0(u), lane);
                }
            }
            if (DUAL && (j & 1)) {
                const float f = fast_exp2(e - ref1);
                ref1 = e;
                hodd[0] *= f;
                hodd[0] = E::mma(hodd[0], av[0][0], bv[0][0]);
                hodd[0] = E::mma(hodd[0], av[0][1], bv[0][1]);
            } else {
                const float f = fast_exp2(e - ref0);
                ref0 = e;
#pragma unroll
                for (int u = 0; u < TPS; ++u) {
                    hacc[u] *= f;
                    hacc[u] = E::mma(hacc[u], av[u][0], bv[u][0]);
                    hacc[u] = E::mma(hacc[u], av[u][1], bv[u][1]);
                }
            }
        }
        if constexpr (DUAL) {
            // ref1 is the last block's end: the odd chain needs no factor
            hacc[0] = hacc[0] * fast_exp2(ref1 - ref0) + hodd[0];
        }
    };

    // -------------------------------------------------------------- output waves
    const int ok_ = wave & 3;
    const int i1 = ok_, i2 = 7 - ok_;   // the wave's two blocks, i1 < i2
    frag pc[2][NKS];    // C fragments (block, K-step)
    frag pcb[14];       // off-diagonal C B^T: tile t < i2 is (i2, t), else (i1, 6 - t)
    frag pdg[2][2];     // diagonal C B^T (block, K-step)
    f32x16 acc[2][2];   // Y^T tiles (block, p sub-tile)
    auto prefetch_c = [&](int c) {
        int64_t rowc;
        int len;
        chunk_at(c, &rowc, &len);
        const rsrc_t cr = make_rsrc(Cg + rowc * G * (int64_t)N, (uint32_t)len * G * N * 2);
        const uint32_t lb = opaque((uint32_t)((lr * G + g) * N + 8 * lg) * 2);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint32_t base = lb + (uint32_t)(32 * (u == 0 ? i1 : i2) * G * N * 2);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) pc[u][ks] = E::ldb8(cr, base + 32u * ks);
        }
    };
    auto prefetch_cb = [&](int c) {
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
    auto prefetch_dg = [&](int c) {
        const rsrc_t cbr = cb_rsrc(c);
        const uint32_t lb = opaque(16u * lane);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                pdg[u][ks] = E::ldb8(cbr, lb, (uint32_t)(((u == 0 ? i1 : i2) * ((u == 0 ? i1 : i2) + 3) / 2) * 2048 + ks * 1024));
    };
    auto output_chunk = [&](int c) {
        const bool more = c + 1 < nchunks;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int v = 0; v < 2; ++v) acc[u][v] = f32x16{};
        // left factor h C^T, the h fragments shared by both blocks
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const frag hv = E::lds8(hs + (32 * v + lr) * HS + 16 * ks + 8 * lg);
                acc[0][v] = E::mma(acc[0][v], hv, pc[0][ks]);
                acc[1][v] = E::mma(acc[1][v], hv, pc[1][ks]);
            }
        }
        // earlier blocks: j < i2 for the later block, j < i1 for both
        float prev1 = 0.f, prev2 = 0.f;
#pragma unroll
        for (int j = 0; j < 7; ++j) {
            if (j >= i2) break;
            const float e = ends[j];
            const float f = fast_exp2(e - prev2);
            prev2 = e;
            const bool both = j < i1;
            if (both) prev1 = e;
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const frag x0 = XC::get(Xts, 32 * j, 32 * v, lane);
                const frag x1 = XC::get(Xts, 32 * j + 16, 32 * v, lane);
                acc[1][v] *= f;
                acc[1][v] = E::mma(acc[1][v], x0, pcb[2 * j]);
                acc[1][v] = E::mma(acc[1][v], x1, pcb[2 * j + 1]);
                if (both) {
                    acc[0][v] *= f;
                    acc[0][v] = E::mma(acc[0][v], x0, pcb[2 * (6 - j)]);
                    acc[0][v] = E::mma(acc[0][v], x1, pcb[2 * (6 - j) + 1]);
                }
            }
        }
        if (more) {
            prefetch_c(c + 1);
            prefetch_cb(c + 1);
        }
        // row scale 2^(cs[l] - cs[e_{i-1}]), then the diagonal tile with the exact
        // decay mask on unscaled X; the mask fragments serve both p sub-tiles
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int i = u == 0 ? i1 : i2;
            const int l0 = 32 * i;
            const float csl = css[l0 + lr];
            const float fr = fast_exp2(csl - (u == 0 ? prev1 : prev2));
#pragma unroll
            for (int v = 0; v < 2; ++v) acc[u][v] *= fr;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const f32x4 c0 = *reinterpret_cast<const f32x4*>(css + l0 + 16 * ks + 8 * lg);
                const f32x4 c1 = *reinterpret_cast<const f32x4*>(css + l0 + 16 * ks + 8 * lg + 4);
                const float cv[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
                frag m;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int sl = 16 * ks + 8 * lg + q;
                    const float w = (sl <= lr) ? E::to_f(pdg[u][ks][q]) * fast_exp2(csl - cv[q]) : 0.f;
                    m[q] = E::from_f(w);
                }
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    const frag xv = XC::get(Xs, l0 + 16 * ks, 32 * v, lane);
                    acc[u][v] = E::mma(acc[u][v], xv, m);
                }
            }
        }
        if (more) prefetch_dg(c + 1);
    };
    auto store_y = [&](int c) {
        int64_t rowc;
        int len;
        chunk_at(c, &rowc, &len);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int l = 32 * (u == 0 ? i1 : i2) + lr;
            if (l >= len) continue;
            __bf16* yrow = Y + ((rowc + l) * H + h) * (int64_t)P + p_base;
#pragma unroll
            for (int v = 0; v < 2; ++v)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    E::st4(yrow + 32 * v + 8 * q + 4 * lg, acc[u][v][4 * q], acc[u][v][4 * q + 1],
                           acc[u][v][4 * q + 2], acc[u][v][4 * q + 3]);
        }
    };

    // -------------------------------------------------------------- walk
    // Each role runs its own loop (so that neither role's registers are held by the
    // other); both meet the same barriers: one after the prologue and two per chunk.
    if (state_role) {
#pragma unroll
        for (int u = 0; u < TPS; ++u) {
            hacc[u] = f32x16{};
            if (!a.init) continue;
            const int n0 = tile_n0(u), p = p_base + tile_p0(u) + lr;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(a.init + state_base + (int64_t)p * N + n0 + 8 * q + 4 * lg);
                hacc[u][4 * q] = v[0];
                hacc[u][4 * q + 1] = v[1];
                hacc[u][4 * q + 2] = v[2];
                hacc[u][4 * q + 3] = v[3];
            }
        }
        if (nchunks > 0) {
            prefetch_in(0);
            commit_in();
        }
        write_h();
        __syncthreads();
        for (int c = 0; c < nchunks; ++c) {
            if (c + 1 < nchunks) prefetch_in(c + 1);
            state_chunk();
            __syncthreads();
            write_h();
            if (c + 1 < nchunks) commit_in();
            __syncthreads();
        }
        if (a.final_state) {
#pragma unroll
            for (int u = 0; u < TPS; ++u) {
                const int n0 = tile_n0(u), p = p_base + tile_p0(u) + lr;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 v = {hacc[u][4 * q], hacc[u][4 * q + 1], hacc[u][4 * q + 2], hacc[u][4 * q + 3]};
                    *reinterpret_cast<f32x4*>(a.final_state + state_base + (int64_t)p * N + n0 + 8 * q + 4 * lg) = v;
                }
            }
        }
    } else {
        if (nchunks > 0) {
            prefetch_c(0);
            prefetch_cb(0);
            prefetch_dg(0);
        }
        __syncthreads();
        for (int c = 0; c < nchunks; ++c) {
            output_chunk(c);
            __syncthreads();
            store_y(c);
            __syncthreads();
        }
    }
}

}  // namespace ssd
