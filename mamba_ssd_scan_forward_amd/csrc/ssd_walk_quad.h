// ssd_walk_quad.h -- the chunk walker with HQ = 3 or 4 heads per workgroup (the "quad"
// walker), for bf16 operands, 256-row chunks, head dimension 64 and d_state 64 or 128
// (page "Transformers are SSMs" paper summary, sections 6 and 6.2; heads of a group share
// B and C, section 7.2).
//
// One workgroup per (sequence, group, HQ heads of the group); each head's 64 columns of
// P are split over 2 / PW wavefronts (PW = 32-wide p sub-tiles per wave), and a wave
// keeps its part of the head's state h^T (N x 32 PW, float32) in MFMA accumulators for
// the whole sequence.  (The waves of the last workgroup of a group whose heads are used
// up shadow the group's last head and store nothing.)
//
// The walk goes block by block (32 rows), and each block's output comes from the state
// at the end of the previous block instead of from the earlier blocks' C B^T tiles:
// with X~[s] = 2^(cs[e_j] - cs[s]) X[s] (e_j the last row of block j, cs the inclusive
// cumsum of logA within the chunk, log2 units) and h^(j) the state after block j,
//      Y_j^T = h^(j-1) C_j^T                          (left factor, section 6.2)
//      Y_j^T = 2^(cs[e_j] - cs[e_{j-1}]) Y_j^T + X~_j^T (C B^T)_jj^T    (diagonal block)
//      Y_j^T[:, l] *= 2^(cs[l] - cs[e_j])
//      h^(j) = 2^(cs[e_j] - cs[e_{j-1}]) h^(j-1) + B_j^T X~_j            (state, 6.2)
// (cs[e_{-1}] = 0 at a chunk's start, h^(-1) the chunk's entry state).  This is the block
// decomposition of section 6 with 32-row blocks for the state passing and the chunk's
// cumsum for the decays; only the diagonal C B^T tiles are used.  The row scale of the
// diagonal is at most 2^R, R = cs[first row] - cs[e_j]; when R > 100 (log2 units;
// Mamba-2's parameters give at most about 74) the block takes the exact mask
// 2^(cs[l] - cs[s]) (C B^T)_ls on unscaled X instead.  Every other factor is <= 1.
//
// The operands the heads of a group share (B^T and C of the block in MFMA fragment
// order, and the diagonal C B^T tile: one run of memory per block, written by the prep
// kernel) are loaded once per workgroup: the waves deal the 1 KB pieces among themselves
// and each loads its share of its own head's X, straight from global memory into a
// four-slot LDS ring three blocks ahead; one barrier per block hands a slot over.  The
// state accumulator converts to the A operand of the left factor without moving data
// between lanes: a lane holds rows 8 (e / 4) + 4 lg + e % 4 of a 32 x 32 accumulator,
// and the prep kernel writes C's fragments with the contraction index in that order.
#pragma once

#include "ssd_walk_split.h"

namespace ssd {

// LDS of the quad walker: a ring of four slots, each with the block's shared fragments
// (B^T [N/16], C [N/16], diagonal C B^T [2], 1 KB each, in the order of their run in
// memory), the HQ heads' X rows [HQ][32][64] (swizzled) and their rows' cumsums and
// decays to the block's end [HQ][2][32]; per wave its Y tile on the way to global memory
// [32][32 PW + 8].  The slots are separate
// arrays, so that the compiler can tell a slot being filled (by direct-to-LDS loads)
// from the slot being read.
template <int NP, int PW, int HQ> struct QuadLds {
    static constexpr int nsh = NP / 8 + 2;
    static constexpr int bt = 0;
    static constexpr int ct = NP / 16 * 1024;
    static constexpr int cb = NP / 8 * 1024;
    static constexpr int x = nsh * 1024;
    static constexpr int cs = x + HQ * 32 * 64 * 2;
    static constexpr int slot = cs + HQ * 64 * 4;
    static constexpr int nslot = 4;
    static constexpr int nwave = 2 * HQ / PW;
    static constexpr int ystride = 32 * PW + 8;
    static constexpr int ybytes = nwave * 32 * ystride * 2;
    static_assert(nslot * slot + ybytes <= 160 * 1024, "LDS");
};

__device__ __forceinline__ void store_b128(rsrc_t r, uint32_t off, bf16x8 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, 0);
}

// Global memory straight to LDS: lane i's 16 (4) bytes from voff land at dst + 16 i (4 i).
__device__ __forceinline__ void load_lds16(rsrc_t r, void* dst, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, (int)voff, 0, 0, 0);
}
__device__ __forceinline__ void load_lds4(rsrc_t r, void* dst, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 4, (int)voff, 0, 0, 0);
}
// the same with a scalar offset (uniform; it takes no part in the range check)
__device__ __forceinline__ void load_lds16(rsrc_t r, void* dst, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, (int)voff, (int)soff, 0, 0);
}
__device__ __forceinline__ void load_lds4(rsrc_t r, void* dst, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 4, (int)voff, (int)soff, 0, 0);
}

// The transposing LDS reads of one block's X operand fragments, per p sub-tile v: two
// K-steps x two 4-row halves from a[v] (rows + 4 are 512 bytes on, K-step 1 is 2048 bytes
// on: row + 16 keeps the swizzle), and the four 4-value pieces of the rows' decays
// (rows 8 lg + 16 ks + 0..7 from d0).  One asm block that waits for its own reads before it
// ends (its results are complete when the compiler sees them), and that the compiler's
// wait-count analysis does not take for a read of the slots being filled by
// direct-to-LDS loads (it would wait for all of them).
__device__ __forceinline__ void x_frags_tr(uint32_t a0, uint32_t d0, bf16x8 (&xf)[1][2], f32x4 (&dxr)[2][2]) {
    u32x2 r[4];
    asm volatile(
        "ds_read_b128 %4, %9\n"
        "ds_read_b128 %5, %9 offset:16\n"
        "ds_read_b128 %6, %9 offset:64\n"
        "ds_read_b128 %7, %9 offset:80\n"
        "ds_read_b64_tr_b16 %0, %8\n"
        "ds_read_b64_tr_b16 %1, %8 offset:512\n"
        "ds_read_b64_tr_b16 %2, %8 offset:2048\n"
        "ds_read_b64_tr_b16 %3, %8 offset:2560\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(dxr[0][0]), "=&v"(dxr[0][1]), "=&v"(dxr[1][0]),
          "=&v"(dxr[1][1])
        : "v"(a0), "v"(d0)
        : "memory");
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const bf16x4 lo = __builtin_bit_cast(bf16x4, r[2 * ks]), hi = __builtin_bit_cast(bf16x4, r[2 * ks + 1]);
        xf[0][ks] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
}
__device__ __forceinline__ void x_frags_tr(uint32_t a0, uint32_t a1, uint32_t d0, bf16x8 (&xf)[2][2],
                                           f32x4 (&dxr)[2][2]) {
    u32x2 r[8];
    asm volatile(
        "ds_read_b128 %8, %14\n"
        "ds_read_b128 %9, %14 offset:16\n"
        "ds_read_b128 %10, %14 offset:64\n"
        "ds_read_b128 %11, %14 offset:80\n"
        "ds_read_b64_tr_b16 %0, %12\n"
        "ds_read_b64_tr_b16 %1, %12 offset:512\n"
        "ds_read_b64_tr_b16 %2, %12 offset:2048\n"
        "ds_read_b64_tr_b16 %3, %12 offset:2560\n"
        "ds_read_b64_tr_b16 %4, %13\n"
        "ds_read_b64_tr_b16 %5, %13 offset:512\n"
        "ds_read_b64_tr_b16 %6, %13 offset:2048\n"
        "ds_read_b64_tr_b16 %7, %13 offset:2560\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
          "=&v"(dxr[0][0]), "=&v"(dxr[0][1]), "=&v"(dxr[1][0]), "=&v"(dxr[1][1])
        : "v"(a0), "v"(a1), "v"(d0)
        : "memory");
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bf16x4 lo = __builtin_bit_cast(bf16x4, r[4 * v + 2 * ks]);
            const bf16x4 hi = __builtin_bit_cast(bf16x4, r[4 * v + 2 * ks + 1]);
            xf[v][ks] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
}

// The Y tile's round trip through this wave's LDS area, in asm for the same reason.
// Write: 8-byte pieces (p sub-tile v, 4-row group q) at byte 64 v + 16 q from wa.
// Read: 16-byte pieces of whole rows, rows 8 (PW = 2) or 16 (PW = 1) apart per read.
__device__ __forceinline__ void y_stage_write(uint32_t wa, const u32x2 (&d)[4]) {
    asm volatile(
        "ds_write_b64 %0, %1\n"
        "ds_write_b64 %0, %2 offset:16\n"
        "ds_write_b64 %0, %3 offset:32\n"
        "ds_write_b64 %0, %4 offset:48"
        :
        : "v"(wa), "v"(d[0]), "v"(d[1]), "v"(d[2]), "v"(d[3])
        : "memory");
}
__device__ __forceinline__ void y_stage_write(uint32_t wa, const u32x2 (&d)[8]) {
    asm volatile(
        "ds_write_b64 %0, %1\n"
        "ds_write_b64 %0, %2 offset:16\n"
        "ds_write_b64 %0, %3 offset:32\n"
        "ds_write_b64 %0, %4 offset:48\n"
        "ds_write_b64 %0, %5 offset:64\n"
        "ds_write_b64 %0, %6 offset:80\n"
        "ds_write_b64 %0, %7 offset:96\n"
        "ds_write_b64 %0, %8 offset:112"
        :
        : "v"(wa), "v"(d[0]), "v"(d[1]), "v"(d[2]), "v"(d[3]), "v"(d[4]), "v"(d[5]), "v"(d[6]), "v"(d[7])
        : "memory");
}
// PW = 1: rows of 40 elements, 16 rows per read (1280 bytes)
__device__ __forceinline__ void y_stage_read(uint32_t ra, u32x4 (&r)[2]) {
    asm volatile(
        "ds_read_b128 %0, %2\n"
        "ds_read_b128 %1, %2 offset:1280\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1])
        : "v"(ra)
        : "memory");
}
// PW = 2: rows of 72 elements, 8 rows per read (1152 bytes)
__device__ __forceinline__ void y_stage_read(uint32_t ra, u32x4 (&r)[4]) {
    asm volatile(
        "ds_read_b128 %0, %4\n"
        "ds_read_b128 %1, %4 offset:1152\n"
        "ds_read_b128 %2, %4 offset:2304\n"
        "ds_read_b128 %3, %4 offset:3456\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(ra)
        : "memory");
}

// s_waitcnt vmcnt(n) alone (gfx9 encoding: expcnt and lgkmcnt at their maxima)
template <int n>
__device__ __forceinline__ void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// One block of the quad walker when its row span R = cs[first row] - e exceeds 100
// (log2 units; beyond Mamba-2's parameter ranges): X~ would lose rows to underflow and the
// state decays by more than 2^-100 within the block.  The state g (scale 2^lsig) is
// brought to h^(j-1) first; the left factor takes it with 2^(cs[l] - prev), and only then
// does each tile decay to the block's end before its update g = 2^dlt h + B^T X~:
//     Y^T = 2^(cs[l] - prev) C h^T + X^T D'^T,  D'_ls = 2^(cs[l] - cs[s]) (C B^T)_ls
// on unscaled X (every factor <= 1).
template <int NT, int PW>
__device__ __forceinline__ void quad_exact_block(f32x16 (&hacc)[NT][PW], f32x16 (&acc)[PW], const __bf16* cts,
                                                 const __bf16* bts, bf16x8 (&dg)[2], const bf16x8 (&xf)[PW][2],
                                                 const float* csb, float e, float prev, float lsig, float csl,
                                                 int lane) {
    typedef Elem<__bf16> E;
    const int lr = lane & 31, lg = lane >> 5;
    const float f0 = fast_exp2(lsig);
    const float fd = fast_exp2(e - prev);
    bf16x8 xt[PW][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const float fs = fast_exp2(e - csb[16 * ks + 8 * lg + q]);
#pragma unroll
            for (int v = 0; v < PW; ++v) xt[v][ks][q] = E::from_f(E::to_f(xf[v][ks][q]) * fs);
        }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        bf16x8 hb[2][PW];
#pragma unroll
        for (int v = 0; v < PW; ++v) hacc[nt][v] *= f0;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int v = 0; v < PW; ++v)
#pragma unroll
                for (int q = 0; q < 8; ++q) hb[kk][v][q] = E::from_f(hacc[nt][v][8 * kk + q]);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const bf16x8 cf = E::lds8(cts + (2 * nt + kk) * 512 + 8 * lane);
#pragma unroll
            for (int v = 0; v < PW; ++v) acc[v] = E::mma(acc[v], hb[kk][v], cf);
        }
        const bf16x8 b0 = E::lds8(bts + (2 * nt) * 512 + 8 * lane), b1 = E::lds8(bts + (2 * nt + 1) * 512 + 8 * lane);
#pragma unroll
        for (int v = 0; v < PW; ++v) {
            hacc[nt][v] *= fd;
            hacc[nt][v] = E::mma(hacc[nt][v], b0, xt[v][0]);
            hacc[nt][v] = E::mma(hacc[nt][v], b1, xt[v][1]);
        }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int sl = 16 * ks + 8 * lg + q;
            const float w = sl <= lr ? E::to_f(dg[ks][q]) * fast_exp2(csl - csb[sl]) : 0.f;
            dg[ks][q] = E::from_f(w);
        }
    const float f1 = fast_exp2(csl - prev);
#pragma unroll
    for (int v = 0; v < PW; ++v) {
        acc[v] *= f1;
        acc[v] = E::mma(acc[v], xf[v][0], dg[0]);
        acc[v] = E::mma(acc[v], xf[v][1], dg[1]);
    }
}

// The walk of one work item (sequence s, group g, quad qd) over the LDS ring r0..r3 and
// the Y staging area ystage.  EXACT: whether a block of very steep decay may come.
template <int NP, int PW, int HQ, bool EXACT>
__device__ __forceinline__ void quad_walk(const WalkArgs& a, unsigned char* ring0, unsigned char* ring1,
                                          unsigned char* ring2, unsigned char* ring3, __bf16* ystage, int s, int g,
                                          int qd) {
    typedef Elem<__bf16> E;
    typedef bf16x8 frag;
    typedef QuadLds<NP, PW, HQ> L;
    typedef LdsMat<__bf16, 64> XL;
    constexpr int NT = NP / 32;            // n tiles of the state
    constexpr int WPH = 2 / PW;            // waves per head
    constexpr int NW = HQ * WPH;           // waves per workgroup
    constexpr int XQ = 4 / WPH;            // 1 KB pieces of its head's X rows loaded by one wave
    constexpr int D = 3;                   // blocks in flight ahead of the one computed
    constexpr int LPS = (L::nsh + NW - 1) / NW + XQ + 1;   // vector memory loads per step (per wave)
    constexpr int SPS = 2 * PW;            // vector memory stores per step
    constexpr int YS = L::ystride;
    static_assert(L::nslot >= D + 1, "ring");

    auto ring = [&](auto kc) __attribute__((always_inline)) -> unsigned char* {
        constexpr int k = decltype(kc)::value;
        if constexpr (k == 0) return ring0;
        else if constexpr (k == 1) return ring1;
        else if constexpr (k == 2) return ring2;
        else return ring3;
    };
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hw = wave / WPH;             // head of the quad
    const int ps0 = (wave % WPH) * PW;     // first p sub-tile of this wave
    const int H = a.H, G = a.G, hpg = H / G;

    const int hl = HQ * qd + hw;
    const bool valid = hl < hpg;
    const int h = g * hpg + (valid ? hl : hpg - 1);

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
    const int nb = 8 * nchunks;   // 32-row blocks (a ragged chunk is walked in full)

    const __bf16* X = static_cast<const __bf16*>(a.X);
    const __bf16* CBg = static_cast<const __bf16*>(a.cb);
    __bf16* Y = static_cast<__bf16*>(a.Y);
    const int XH = a.xh, xhi = h / (H / XH);   // X row of this head
    const int64_t state_base = ((int64_t)s * H + h) * 64 * (int64_t)a.ldn + a.ns0;

    // ---- block min(b, nb - 1)'s share of this wave, global memory -> LDS slot b % 4
    //      (LPS loads; a block past the end loads the last one, into a slot nobody
    //      reads).  The block's shared operands -- N/16 B^T fragments (n tile f / 2,
    //      K-step f % 2), N/16 C fragments (K-step f) and the diagonal C B^T tile's two
    //      K-steps, 1 KB each -- are one run of memory, in the slot's order (prep kernel);
    //      wave w loads pieces w + NW i (a wave past the last piece loads the last one
    //      again, to the same place, with the same bytes: every wave issues the same
    //      loads).  The wave's part of each offset is in the vector offset, the block's in
    //      the scalar offset.
    const rsrc_t wsr = make_rsrc(CBg, 0xFFFFFFFFu);
    constexpr int NSH = L::nsh;                 // shared 1 KB pieces of a block
    constexpr int NI = (NSH + NW - 1) / NW;     // of them loaded by one wave
    int pk[NI];
    uint32_t pv[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        pk[i] = min(wave + NW * i, NSH - 1);
        pv[i] = opaque(16u * lane + (uint32_t)(pk[i] * 1024));
    }
    // X: lane i of each 1 KB piece fills 16-byte unit i % 8 of row 8 q + i / 8, which
    // holds column unit (i % 8) ^ swz(row); swz depends on row % 4 = (i / 8) % 4 only
    const uint32_t xlane = opaque((uint32_t)(((lane >> 3) * XH + xhi) * 64 + 8 * ((lane & 7) ^ XL::swz(lane >> 3))) * 2);
    // cumsum (lanes 0..31) and per-row decays to the block's end (lanes 32..63) of the
    // block's rows, in one load: the decays' array lies after the cumsum's in the workspace
    const rsrc_t csr = make_rsrc(a.cs, 0xFFFFFFFFu);
    const uint32_t cslane =
        opaque(4u * lr + (lg ? (uint32_t)(reinterpret_cast<const char*>(a.dx) - reinterpret_cast<const char*>(a.cs)) : 0u));
    auto issue = [&](int b, auto kc) __attribute__((always_inline)) {
        b = min(b, nb - 1);
        const int c = b >> 3, j = b & 7;
        const int sl = slot0 + c;
        unsigned char* sb = ring(kc);
        const uint32_t sq = ((uint32_t)(sl * G + g) * 8 + j) * (uint32_t)(NSH * 1024);
#pragma unroll
        for (int i = 0; i < NI; ++i) load_lds16(wsr, sb + pk[i] * 1024, pv[i], sq);
        // X rows 8 q .. 8 q + 7 of the block (this wave's share of q; rows past the
        // chunk's end read as zeros: buffer range)
        const int64_t rowc = row0 + (int64_t)c * 256;
        const int len = min(256, len_seq - c * 256);
        const rsrc_t xrs = make_rsrc(X + rowc * XH * 64, (uint32_t)len * XH * 64 * 2);
        unsigned char* xs = sb + L::x + hw * 32 * 64 * 2;
#pragma unroll
        for (int i = 0; i < XQ; ++i) {
            const int q = (wave % WPH) + WPH * i;
            load_lds16(xrs, xs + q * 1024, xlane + (uint32_t)((32 * j + 8 * q) * XH * 64 * 2));
        }
        // the cumsum and the decays of the block's rows (the waves of a head write the
        // same bytes)
        load_lds4(csr, sb + L::cs + hw * 256, cslane, (((uint32_t)sl * H + h) * 256 + 32 * j) * 4);
    };

    // ---- the state, kept as g = h / 2^lsig with a per-head scalar lsig (log2) so that
    //      the block decays need no pass over the accumulators: h^T tiles (n tile, p
    //      sub-tile ps0 + v), element e of a lane at (n = 32 nt + acc_row(e), p = 32 (ps0 + v) + lr)
    f32x16 hacc[NT][PW];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int v = 0; v < PW; ++v) hacc[nt][v] = f32x16{};
    if (a.init) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int v = 0; v < PW; ++v)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 iv = *reinterpret_cast<const f32x4*>(
                        a.init + state_base + (int64_t)(32 * (ps0 + v) + lr) * a.ldn + 32 * nt + 8 * q + 4 * lg);
#pragma unroll
                    for (int e = 0; e < 4; ++e) hacc[nt][v][4 * q + e] = iv[e];
                }
    }
    float lsig = 0.f;   // log2 of the state's scale
    float prev = 0.f;   // cs[e_{j-1}] of the next block (0 at a chunk's start)

    auto compute = [&](int t, auto kc, auto) __attribute__((always_inline)) {
        const int c = t >> 3, j = t & 7;
        const unsigned char* sb = ring(kc);
        const float* csb = reinterpret_cast<const float*>(sb + L::cs + hw * 256);
        const float e = csb[31];
        const float csl = csb[lr];
        const float dlt = e - prev;   // this block's log2 decay (<= 0)
        // every LDS operand of the block is read first: the C and B^T fragments and the
        // diagonal tile, then X through the asm reads, whose final wait covers them all
        // (the instance that may take the steep path reads them where they are used:
        // fewer registers)
        const __bf16* cts = reinterpret_cast<const __bf16*>(sb + L::ct);
        const __bf16* bts = reinterpret_cast<const __bf16*>(sb + L::bt);
        frag ctf[NT][2], btf[NT][2], dg[2];
        if constexpr (!EXACT) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    ctf[nt][kk] = E::lds8(cts + (2 * nt + kk) * 512 + 8 * lane);
                    btf[nt][kk] = E::lds8(bts + (2 * nt + kk) * 512 + 8 * lane);
                }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            dg[ks] = E::lds8(reinterpret_cast<const __bf16*>(sb + L::cb + ks * 1024) + 8 * lane);
        // the rows' decays to the block's end: 2^(e - cs[s]) for s = 16 ks + 8 lg + q (read
        // with X below)
        f32x4 dxr[2][2];
        const float cs0 = csb[0];
        const __bf16* xs = reinterpret_cast<const __bf16*>(sb + L::x + hw * 32 * 64 * 2);
        // X of the block as operand fragments: lane holds X[16 ks + 8 lg + q][32 (ps0 + v) + lr]
        // (the addressing of LdsCol: lane i of each 16 reads 4 elements of row i / 4)
        frag xf[PW][2];
        {
            const int row = 8 * lg + ((lane & 15) >> 2);
            const int col = 32 * ps0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
            const uint32_t base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) __bf16*)xs;
            const uint32_t d0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) float*)(csb + 32 + 8 * lg);
            if constexpr (PW == 1) x_frags_tr(base + 2u * (uint32_t)XL::idx(row, col), d0, xf, dxr);
            else
                x_frags_tr(base + 2u * (uint32_t)XL::idx(row, col), base + 2u * (uint32_t)XL::idx(row, col + 32), d0, xf,
                           dxr);
        }
        // X~' = X 2^(e - cs[s] - lsig): X~ divided by the state's scale (lsig after this
        // block), from the rows' decays to the block's end 2^(e - cs[s]) (prep kernel)
        auto scale_x = [&](frag (&xt)[PW][2]) __attribute__((always_inline)) {
            const float isig = fast_exp2(-lsig);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const f32x4 c0 = dxr[ks][0], c1 = dxr[ks][1];
                float fs[8];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    fs[q] = c0[q] * isig;
                    fs[4 + q] = c1[q] * isig;
                }
#pragma unroll
                for (int v = 0; v < PW; ++v)
#pragma unroll
                    for (int q = 0; q < 8; ++q) xt[v][ks][q] = E::from_f(E::to_f(xf[v][ks][q]) * fs[q]);
            }
        };
        f32x16 acc[PW];
#pragma unroll
        for (int v = 0; v < PW; ++v) acc[v] = f32x16{};
        frag xt[PW][2];
        // The block's row span R = cs[first row] - e decides the path (uniform).
        bool moderate = true;
        if constexpr (EXACT) moderate = __builtin_amdgcn_readfirstlane((int)(cs0 - e <= 100.f)) != 0;
        if (!EXACT || moderate) {
            // ---- moderate span (every block of Mamba-2's parameter ranges).  The state's
            // scale becomes lsig + dlt while that stays above 2^-64; otherwise g is first
            // brought to h^(j-1) 2^dlt, scale 1 at the block's end (one pass, rarely; the
            // decayed state is then within 2^-100 of h^(j-1)).  Then
            //   Y^T = 2^(cs[l] - e + lsig) (C g^T + X~'^T D^T),  g += B^T X~'
            // with D the masked diagonal tile, g taken by the left factor before the update.
            if (lsig + dlt < -64.f) {
                // (kept a branch: as a select it would cost the multiplies in every block)
                asm volatile("");
                const float f = fast_exp2(lsig + dlt);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int v = 0; v < PW; ++v) hacc[nt][v] *= f;
                lsig = 0.f;
            } else {
                lsig += dlt;
            }
            scale_x(xt);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                frag hb[2][PW];   // (K-step within the tile, p sub-tile)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int v = 0; v < PW; ++v)
#pragma unroll
                        for (int q = 0; q < 8; ++q) hb[kk][v][q] = E::from_f(hacc[nt][v][8 * kk + q]);
                frag cf[2], bf[2];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    if constexpr (EXACT) {
                        cf[kk] = E::lds8(cts + (2 * nt + kk) * 512 + 8 * lane);
                        bf[kk] = E::lds8(bts + (2 * nt + kk) * 512 + 8 * lane);
                    } else {
                        cf[kk] = ctf[nt][kk];
                        bf[kk] = btf[nt][kk];
                    }
                }
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int v = 0; v < PW; ++v) acc[v] = E::mma(acc[v], hb[kk][v], cf[kk]);
#pragma unroll
                for (int v = 0; v < PW; ++v) {
                    hacc[nt][v] = E::mma(hacc[nt][v], bf[0], xt[v][0]);
                    hacc[nt][v] = E::mma(hacc[nt][v], bf[1], xt[v][1]);
                }
            }
#pragma unroll
            for (int v = 0; v < PW; ++v) {
                acc[v] = E::mma(acc[v], xt[v][0], dg[0]);
                acc[v] = E::mma(acc[v], xt[v][1], dg[1]);
            }
            const float f2 = fast_exp2(csl - e + lsig);
#pragma unroll
            for (int v = 0; v < PW; ++v) acc[v] *= f2;
        } else {
            // ---- very strong decay (R > 100): outside this loop's registers
            quad_exact_block<NT, PW>(hacc, acc, cts, bts, dg, xf, csb, e, prev, lsig, csl, lane);
            lsig = 0.f;
        }
        prev = j == 7 ? 0.f : e;
        // Y^T tile -> this wave's LDS area -> 16-byte pieces of whole rows of Y (rows past
        // the sequence's end, and every row of a shadowing wave, fall outside the store's
        // range)
        const uint32_t ysb = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16*)(ystage + wave * 32 * YS);
        {
            u32x2 d[4 * PW];
#pragma unroll
            for (int v = 0; v < PW; ++v)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const bf16x4 w = {(__bf16)acc[v][4 * q], (__bf16)acc[v][4 * q + 1], (__bf16)acc[v][4 * q + 2],
                                      (__bf16)acc[v][4 * q + 3]};
                    d[4 * v + q] = __builtin_bit_cast(u32x2, w);
                }
            y_stage_write(ysb + 2u * (uint32_t)(lr * YS + 4 * lg), d);
        }
        const int64_t rowb = row0 + (int64_t)c * 256 + 32 * j;
        const int nrows = valid ? max(0, min(32, len_seq - c * 256 - 32 * j)) : 0;
        const rsrc_t yr = make_rsrc(Y + (rowb * H + h) * 64, nrows > 0 ? (uint32_t)(((nrows - 1) * H + 1) * 64 * 2) : 0u);
        constexpr int LPR = 4 * PW;   // lanes per row (16-byte pieces)
        constexpr int RPR = 64 / LPR; // rows per read
        u32x4 yv[SPS];
        y_stage_read(ysb + 2u * (uint32_t)((lane / LPR) * YS + 8 * (lane % LPR)), yv);
#pragma unroll
        for (int q = 0; q < SPS; ++q) {
            const int r = RPR * q + lane / LPR;
            store_b128(yr, opaque((uint32_t)(r * H * 64 + 32 * ps0 + 8 * (lane % LPR)) * 2),
                       __builtin_bit_cast(frag, yv[q]));
        }
    };

    // Blocks 0 .. D-1 are in flight before the first step; step t issues block t + D
    // (past the end: the last block again, so that every step issues LPS loads and SPS
    // stores), computes block t, waits for its own loads of block t + 1 and meets the
    // other waves at a barrier, after which block t + 1's slot is complete and block
    // t's slot (reused by block t + 4) has been read by everyone.  The waits count the
    // vector memory operations issued after those loads: the rest of their step's, and
    // every later step's (fewer for the first two steps).
    using K0 = std::integral_constant<int, 0>;
    using K1 = std::integral_constant<int, 1>;
    using K2 = std::integral_constant<int, 2>;
    using K3 = std::integral_constant<int, 3>;
    if (nb > 0) {
        issue(0, K0{});
        issue(1, K1{});
        issue(2, K2{});
        wait_vm<2 * LPS>();
    }
    __builtin_amdgcn_s_barrier();
    auto step = [&](int t, auto kc, auto exc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        issue(t + D, std::integral_constant<int, (k + D) % 4>{});
        compute(t, kc, exc);
        __builtin_amdgcn_sched_barrier(0);
        if (t == 0) wait_vm<2 * LPS + SPS>();
        else if (t == 1) wait_vm<2 * LPS + 2 * SPS>();
        else wait_vm<2 * LPS + 3 * SPS>();
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS reads are done
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    using Ex = std::integral_constant<bool, EXACT>;
    for (int t = 0; t < nb; t += 4) {
        step(t, K0{}, Ex{});
        step(t + 1, K1{}, Ex{});
        step(t + 2, K2{}, Ex{});
        step(t + 3, K3{}, Ex{});
    }
    if (a.final_state && valid) {
        const float f = fast_exp2(lsig);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int v = 0; v < PW; ++v)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 o = {hacc[nt][v][4 * q] * f, hacc[nt][v][4 * q + 1] * f, hacc[nt][v][4 * q + 2] * f,
                                     hacc[nt][v][4 * q + 3] * f};
                    *reinterpret_cast<f32x4*>(a.final_state + state_base + (int64_t)(32 * (ps0 + v) + lr) * a.ldn +
                                              32 * nt + 8 * q + 4 * lg) = o;
                }
    }
}

// The steep instance of the walk, not inlined: the common one keeps the kernel's registers
// (this one reaches the LDS ring through pointers, which costs it the overlap of its loads
// with the walk; it only runs where the decay is far beyond Mamba-2's parameter ranges).
template <int NP, int PW, int HQ>
__device__ __noinline__ void quad_walk_steep(WalkArgs a, unsigned char* r0, unsigned char* r1, unsigned char* r2,
                                             unsigned char* r3, __bf16* ys, int s, int g, int qd) {
    quad_walk<NP, PW, HQ, true>(a, r0, r1, r2, r3, ys, s, g, qd);
}

template <int NP, int PW, int HQ>
__global__ void __launch_bounds__(128 * HQ / PW, 2 / PW) ssd_walk_quad_kernel(WalkArgs a) {
    typedef QuadLds<NP, PW, HQ> L;
    constexpr int WPH = 2 / PW;            // waves per head
    constexpr int NW = HQ * WPH;           // waves per workgroup
    __shared__ __align__(16) unsigned char ring0[L::slot], ring1[L::slot], ring2[L::slot], ring3[L::slot];
    __shared__ __align__(16) __bf16 ystage[L::ybytes / 2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hw = wave / WPH;
    const int H = a.H, G = a.G, hpg = H / G, nq = a.quads;

    // ---- work item: (sequence, group, quad); consecutive items of an XCD share a
    //      (sequence, group) and so its B, C and C B^T in L2
    int s, g, qd;
    if (a.lpt) {
        // packed sequences: the (sequence, group) units are dealt to the XCDs
        // round-robin, longest sequence first (as in the split walker)
        const int bid = blockIdx.x;
        const int xcd = bid % 8, slot = bid / 8;
        const int u = (slot / nq) * 8 + xcd;
        qd = slot % nq;
        const int r = u / G;
        g = u % G;
        const int* off = a.seq_offsets;
        bool mine = false;
        if (lane < a.nseq) {
            const int Ln = off[lane + 1] - off[lane];
            int rank = 0;
            for (int v = 0; v < a.nseq; ++v) {
                const int Lv = off[v + 1] - off[v];
                rank += (Lv > Ln) || (Lv == Ln && v < lane);
            }
            mine = rank == r;
        }
        s = __builtin_ctzll(__ballot(mine));
    } else {
        const int item = xcd_remap(blockIdx.x, gridDim.x);
        if (item >= a.nitems) return;
        qd = item % nq;
        const int sg = item / nq;
        g = sg % G;
        s = sg / G;
    }
    // whether any chunk of this workgroup's heads has a block of very steep decay (flags
    // written by the prep kernel's cumsum role; each wave votes into the Y staging area,
    // unused until the walk starts)
    {
        const int hl = HQ * qd + hw;
        const int h = g * hpg + (hl < hpg ? hl : hpg - 1);
        int slot0, nchunks;
        if (!a.seq_offsets) {
            nchunks = (int)((a.T + 255) / 256);
            slot0 = s * nchunks;
        } else {
            nchunks = (a.seq_offsets[s + 1] - a.seq_offsets[s] + 255) / 256;
            slot0 = 0;
            for (int u = 0; u < s; ++u) slot0 += (a.seq_offsets[u + 1] - a.seq_offsets[u] + 255) / 256;
        }
        int steep = 0;
        for (int c = lane; c < nchunks; c += 64) steep |= a.xflag[(int64_t)(slot0 + c) * H + h];
        steep = __ballot(steep != 0) != 0;
        int* vote = reinterpret_cast<int*>(ystage);
        if (lane == 0) vote[wave] = steep;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < NW; ++w) steep |= vote[w];
        __syncthreads();
        if (steep) {
            quad_walk_steep<NP, PW, HQ>(a, ring0, ring1, ring2, ring3, ystage, s, g, qd);
            return;
        }
    }
    quad_walk<NP, PW, HQ, false>(a, ring0, ring1, ring2, ring3, ystage, s, g, qd);
}

}  // namespace ssd
