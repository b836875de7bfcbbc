// ssd_walk_fused.h -- the fused walker: the whole SSD forward of a (sequence, group, run of
// 32-column units of P) in one launch, with no workspace, for bf16 operands, head
// dimension a multiple of 32 and d_state 64, 128 or 256 (page "Transformers are SSMs"
// paper summary: the recurrence of sections 2.4 / 5.1, the block decomposition of
// section 6, heads of a group sharing B and C as in section 7.2, packed sequences as in
// section 8.3).
//
// Block decomposition with 32-row blocks and the state passed between blocks.  With
// cs[l] the inclusive cumsum of logA inside block j (log2 units), e = cs[31], and the
// state before the block h = 2^lsig g (g is what the accumulators hold):
//      Y_l   = 2^(cs_l) C_l h + sum_{s <= l} 2^(cs_l - cs_s) (C_l . B_s) X_s
//      h_end = 2^e h + sum_s 2^(e - cs_s) B_s^T X_s
// Taking lsig' = lsig + e (the state's new log scale) both become products with per-row
// factors and one shared, causally masked tile D = tril(C B^T) of the block:
//      X~_s  = 2^(e - cs_s - lsig') X_s                         (w_s)
//      Y_l   = 2^(cs_l - e + lsig') [C_l g + sum_s D_ls X~_s]    (r_l)
//      g'    = g + sum_s B_s^T X~_s
// so the decays touch 32 rows of X and of Y per block, never the state itself.  When
// lsig' would fall below -64 the state is first brought to h 2^e (one pass over the
// accumulators) and lsig' = 0.  A block whose span cs[0] - e exceeds 100 (beyond any
// Mamba-2 parameter range) would lose rows of X~ to underflow; it takes the exact form
// instead: the left factor with 2^(cs_l + lsig), the tile masked per head with
// 2^(cs_l - cs_s) on unscaled X, the state brought to 2^e h before its update with
// X~ = 2^(e - cs_s) X (every factor <= 1).
//
// Workgroup: NW compute waves, two loader waves and a storer.  Compute wave k holds unit
// u = q NW + k of its group (head u / (P/32), columns 32 (u % (P/32)) .. + 31): the state
// g^T of that slice (N x 32 float32, N/32 MFMA accumulators of 32 x 32) for the whole
// sequence.  The X-loader brings each unit's X rows and the heads' logA, the BC-loader
// the group's B and C rows (and its own copy of logA), all straight from global memory
// into a ring of LDS slots, two or three blocks ahead.  The loaders also turn each block
// into its products one step before it is used: the cumsums, w and r of every head, the
// renormalisation and steep flags (X-loader; with two compute waves it also writes
// X~ = w X into the slot), and the masked tile D in the layout of an MFMA operand
// (v_mfma_f32_32x32x16_bf16 on B and C rows; BC-loader).  Compute waves issue no global
// memory instruction at all: they read LDS and write their Y tile to a staging buffer in LDS,
// from which the storer writes the workgroup's block of Y one block later as whole
// contiguous row spans (NW units of 64 bytes per row: few, line-sized write requests
// instead of 32-byte pieces, and no compute wave ever waits behind the loaders' traffic
// in the vector memory path).  One barrier per block hands the ring slot, the products
// and the staging buffer over.
//
// Direction.  The walker also runs in reverse (template argument REV), for the backward
// pass's time-reversed problems: each sequence walked from its last row to its first, the
// decay of each walked row being that of the row after it, read and written in place.
//
// Contraction order.  A lane holds accumulator rows 8 (e / 4) + 4 lg + e % 4 of a 32 x 32
// tile (lg = lane / 32).  The state tile g^T (n x p) therefore enters the left factor
// Y^T = g C^T as an A operand whose K index k = 8 lg + q is the row
// sigma(k) = 8 (q / 4) + 4 lg + q % 4; C is read in that order (two 8-byte pieces per
// K-step).  The same order is used for the rows s of X~ and of the tile D, which is how
// the BC-loader's accumulator of D^T = B C^T becomes the B operand of Y^T += X~^T D^T
// without moving data between lanes, and why X is read with 4-row transposing reads.
#pragma once

#include <type_traits>

#include "ssd_kernels.h"

namespace ssd {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct FusedArgs {
    const __bf16* X;
    const float* logA;
    const __bf16* B;
    const __bf16* C;
    const float* init;
    const int32_t* seq_offsets;
    __bf16* Y;
    float* final_state;
    int64_t T;      // tokens per sequence (without seq_offsets)
    int H, P, N, G, nseq;
    int xh;         // X rows per token: H (one per head), or fewer, each shared by a run of H / xh heads
    int upg;        // 32-column units per group: (H / G) (P / 32)
    int wpg;        // workgroups per group: ceil(upg / NW)
    int nitems;     // nseq G wpg
    int lpt;        // packed sequences dealt to XCDs longest first
    int nseg;       // > 1: every sequence walked as nseg segments of seglen rows, each a
    int seglen;     // sequence of its own (nseq counts the segments); init then holds every
                    // segment's entry state but the first's, which is init0's (the
                    // sequences' initial states, or NULL), and only the last segment
                    // writes a final state
    const float* init0;
};

// LDS of the fused walker.  Ring slot: X [32][NW][32] (the block's rows of the units side by side), B and C
// [32][N] (16-byte units of a row XOR-swizzled by fused_swz), logA [NHL][32].  Products
// (two buffers): the masked tile D^T as MFMA B-operand fragments [2][64][8] bf16, per
// head w [32] (in the sigma order of the K index), r [32], the cumsum [32], the
// renormalisation factor and the path flag, and the per-head exact tiles of steep blocks
// [NHL][2][64][8] bf16.  The BC-loader keeps its own copy of each block's logA [NHL][32].
template <int NP, int NW> struct FusedLds {
    static constexpr int NHL = NW / 2 + 2;             // heads a workgroup can touch (P >= 64)
    static constexpr int xbytes = NW * 2048;
    static constexpr int bcbytes = 32 * NP * 2;
    static constexpr int labytes = ((NHL + 1) / 2) * 256;
    // blocks in flight: nslot - 1 (three slots where four would not fit next to the rest)
    static constexpr int nslot = (NP == 256 || (NP == 128 && NW == 6)) ? 3 : 4;
    static constexpr int dg = 0;
    static constexpr int w = 2048;
    static constexpr int r = w + NHL * 128;
    static constexpr int cs = r + NHL * 128;
    static constexpr int f = cs + NHL * 128;
    static constexpr int fl = f + NHL * 4;
    static constexpr int st = (fl + NHL * 4 + 15) / 16 * 16;
    static constexpr int prod = st + NHL * 2048;
    // the staging of Y for the storer: [32 rows][NW units x 64 bytes + 16], two buffers
    static constexpr int ystride = NW * 64 + 16;
    static constexpr int ybytes = 32 * ystride;
    static constexpr int total = nslot * (xbytes + 2 * bcbytes + 2 * labytes) + 2 * prod + 2 * ybytes;
    static_assert(total <= 160 * 1024, "LDS");
};

// Position of 16-byte unit u of B / C row r in LDS (units per row U = N / 8): the unit
// index XOR 4 (r % (U / 4)) + (r / (U / 4)) % 4, which spreads the rows read together by
// every access pattern of the walk (8-byte C pieces of 32 rows, transposing reads of 8
// rows of B, 16-byte rows of B and C for the tile) evenly over the banks.
template <int NP> __device__ __forceinline__ int fused_swz(int r) {
    constexpr int U4 = NP / 32;
    return 4 * (r % U4) + (r / U4) % 4;
}

// Global memory straight to LDS: lane i's 16 (4) bytes land at dst + 16 i (4 i).
// (LDS addresses are kept in address space 3 throughout: a generic pointer converted at
// each use would cost a null test per load)
typedef SSD_LDS unsigned char* lds_ptr;
// cache policy of the Y stores: nontemporal (gfx950 "nt"), the kernel never reads Y back
constexpr int kStreamAux = 2;
__device__ __forceinline__ void fused_lds16(rsrc_t r, lds_ptr dst, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (SSD_LDS void*)dst, 16, (int)voff, (int)soff, 0, 0);
}
__device__ __forceinline__ void fused_lds4(rsrc_t r, lds_ptr dst, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (SSD_LDS void*)dst, 4, (int)voff, (int)soff, 0, 0);
}
template <typename T> __device__ __forceinline__ T ldsv(lds_ptr p) { return *reinterpret_cast<SSD_LDS const T*>(p); }
template <typename T> __device__ __forceinline__ void ldsw(lds_ptr p, T v) { *reinterpret_cast<SSD_LDS T*>(p) = v; }
template <int n>
__device__ __forceinline__ void fused_wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}
__device__ __forceinline__ bf16x4 tr4(lds_ptr p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SSD_LDS bf16x4*)p);
}
__device__ __forceinline__ uint32_t lds_addr(lds_ptr p) { return (uint32_t)(uintptr_t)p; }
// Eight 16-byte LDS reads in one asm block that also waits for them.  The BC-loader reads
// its slot's B and C rows this way: with each ring one array, the compiler's bookkeeping of
// the wave's direct-to-LDS loads could not tell the slot being read from the slots still
// being filled and would wait for all of them (the loader has waited for this slot
// itself).  (A load written in asm completes inside its block: the compiler treats the
// outputs as written when the block ends.)
__device__ __forceinline__ void lds_read8x16(const uint32_t (&ad)[8], bf16x8 (&r)[8]) {
    asm volatile(
        "ds_read_b128 %0, %8\n"
        "ds_read_b128 %1, %9\n"
        "ds_read_b128 %2, %10\n"
        "ds_read_b128 %3, %11\n"
        "ds_read_b128 %4, %12\n"
        "ds_read_b128 %5, %13\n"
        "ds_read_b128 %6, %14\n"
        "ds_read_b128 %7, %15\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7])
        : "memory");
}
// Four 4-row transposing LDS reads (ds_read_b64_tr_b16) in an asm block that waits for
// them (the same reason as above).
__device__ __forceinline__ void lds_tr4x4(lds_ptr p0, lds_ptr p1, lds_ptr p2, lds_ptr p3, bf16x4 (&r)[4]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n"
        "ds_read_b64_tr_b16 %1, %5\n"
        "ds_read_b64_tr_b16 %2, %6\n"
        "ds_read_b64_tr_b16 %3, %7\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(lds_addr(p0)), "v"(lds_addr(p1)), "v"(lds_addr(p2)), "v"(lds_addr(p3))
        : "memory");
}
// One 4-byte LDS read in an asm block that waits for it (the same reason as above).
__device__ __forceinline__ float lds_read4(lds_ptr p) {
    float r;
    asm volatile("ds_read_b32 %0, %1\n"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r)
                 : "v"(lds_addr(p))
                 : "memory");
    return r;
}
__device__ __forceinline__ bf16x8 cat44(bf16x4 lo, bf16x4 hi) {
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// DPP row operations (gfx9): lanes whose source lies outside the row, or whose row is
// masked off, keep `old` (here 0)
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWMASK, 0xF, false));
}
// Inclusive sum over the 32 lanes of each half of the wave: shifts by 1, 2, 4, 8 inside
// each 16-lane row, then lane 15 (47) of the first row of a half added to its second row.
__device__ __forceinline__ float scan32(float x) {
    x += dpp_f<0x111>(x);
    x += dpp_f<0x112>(x);
    x += dpp_f<0x114>(x);
    x += dpp_f<0x118>(x);
    x += dpp_f<0x142, 0xA>(x);   // row_bcast:15 into rows 1 and 3
    return x;
}
__device__ __forceinline__ float lane_f(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// position of row s (0..31) in the sigma order of the K index (bits 2 and 3 swapped)
__device__ __forceinline__ int sigma_pos(int s) { return (s & 19) | ((s & 4) << 1) | ((s & 8) >> 1); }

// The walker's LDS: separate arrays (ring slots, product buffers, Y staging), so that the
// compiler can tell the slot a direct-to-LDS load is filling from the slot being read.
struct FusedSmem {
    lds_ptr cring, bring;   // one array per ring: [nslot][bcbytes]
    lds_ptr x[4], l[4], m[4], p[2], ys[2];
};
template <int NP, int NW>
__device__ __forceinline__ FusedSmem fused_smem() {
    typedef FusedLds<NP, NW> LL;
    constexpr int NSL = LL::nslot;
    __shared__ __align__(16) unsigned char cring[NSL][LL::bcbytes], bring[NSL][LL::bcbytes];
    __shared__ __align__(16) unsigned char x0[LL::xbytes], x1[LL::xbytes], x2[LL::xbytes], x3[NSL == 4 ? LL::xbytes : 16];
    __shared__ __align__(16) unsigned char l0[LL::labytes], l1[LL::labytes], l2[LL::labytes], l3[NSL == 4 ? LL::labytes : 16];
    __shared__ __align__(16) unsigned char m0[LL::labytes], m1[LL::labytes], m2[LL::labytes], m3[NSL == 4 ? LL::labytes : 16];
    __shared__ __align__(16) unsigned char p0[LL::prod], p1[LL::prod];
    __shared__ __align__(16) unsigned char ys0[LL::ybytes], ys1[LL::ybytes];
    return FusedSmem{(lds_ptr)cring[0], (lds_ptr)bring[0],
                     {(lds_ptr)x0, (lds_ptr)x1, (lds_ptr)x2, (lds_ptr)x3},
                     {(lds_ptr)l0, (lds_ptr)l1, (lds_ptr)l2, (lds_ptr)l3},
                     {(lds_ptr)m0, (lds_ptr)m1, (lds_ptr)m2, (lds_ptr)m3},
                     {(lds_ptr)p0, (lds_ptr)p1},
                     {(lds_ptr)ys0, (lds_ptr)ys1}};
}

// REV: the sequences walked from their last row to their first, each row's decay that of
// the row after it (the first walked row's decay 0): the reversed problem of the backward
// pass, read and written in place (rows outside the sequence fall outside the buffers'
// ranges, so their loads read 0 and their stores are dropped).
template <int NP, int NW, bool REV>
__device__ __forceinline__ void fused_walk(const FusedArgs& a, int s,
                                           int g, int q) {
    typedef FusedLds<NP, NW> LL;
    constexpr int NSL = LL::nslot;
    // ring slots and product buffers: separate arrays, so that the compiler can tell the
    // slot a direct-to-LDS load is filling from the slot being read; selected by constant
    // index (a constant table of LDS addresses cannot be emitted)
    // (B and C: one array per ring, so that a compute wave reads any slot at an immediate
    // offset from one per-lane address)
    // (declared in fused_smem, which does not depend on REV: both directions of a two-walk
    // launch use the one set of arrays)
    const FusedSmem sm = fused_smem<NP, NW>();
    auto pick = [](int k, lds_ptr a0, lds_ptr a1, lds_ptr a2, lds_ptr a3)
                    __attribute__((always_inline)) -> lds_ptr {
        return k == 0 ? a0 : k == 1 ? a1 : k == 2 ? a2 : a3;
    };
    auto XS = [&](int k) __attribute__((always_inline)) { return pick(k, sm.x[0], sm.x[1], sm.x[2], sm.x[3]); };
    auto BS = [&](int k) __attribute__((always_inline)) { return sm.bring + k * LL::bcbytes; };
    auto CS = [&](int k) __attribute__((always_inline)) { return sm.cring + k * LL::bcbytes; };
    auto LA = [&](int k) __attribute__((always_inline)) { return pick(k, sm.l[0], sm.l[1], sm.l[2], sm.l[3]); };
    auto LA2 = [&](int k) __attribute__((always_inline)) { return pick(k, sm.m[0], sm.m[1], sm.m[2], sm.m[3]); };

    typedef Elem<__bf16> E;
    typedef FusedLds<NP, NW> L;
    constexpr int NT = NP / 32;            // n tiles of the state
    constexpr int NS = L::nslot;
    constexpr int D = NS - 1;              // blocks in flight ahead of the one computed
    constexpr int UPR = NP / 8;            // 16-byte units of a B / C row
    constexpr int RPL = 64 / UPR;          // rows per 1 KB load
    constexpr int NBL = NP / 16;           // 1 KB loads of B (and of C) per block
    constexpr int NHL = L::NHL;
    constexpr int NPAIR = (NHL + 1) / 2;
    constexpr int LX = 2 * NW + NPAIR;     // X-loader loads per block
    constexpr int LB = 2 * NBL + NPAIR;    // BC-loader loads per block
    // (a wave's wait counts must fit the 6-bit counter; more loads in flight than that
    // stall at issue until the oldest complete)
    static_assert((D - 1) * LX < 64 && (D - 1) * LB < 64, "vmcnt range");
    // Units XS0 .. NW - 1 get X~ = w X from the X-loader, in place in the slot; the others
    // form it themselves.  With two compute waves the X-loader has a SIMD of its own and
    // scales both units; with more it shares a SIMD with a compute wave or the BC-loader,
    // and the compute waves scale their own.
    constexpr int XS0 = NW == 2 ? 0 : NW;
    constexpr int XSP = (NW - XS0) * 2;   // pieces per X-loader lane

    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool compute = (wave & 3) != 3 && wave - (wave >> 2) < NW;
    const int ci = wave - (wave >> 2);     // compute index (compute waves)
    const bool bcloader = wave == 3;
    const bool storer = wave == NW + 2;
    const bool xloader = !compute && !bcloader && !storer;
    const int H = a.H, P = a.P, G = a.G, hpg = H / G, uph = P / 32;

    int64_t row0;
    int len;
    int64_t sfin = s;   // slot of the final state (-1: none)
    const float* init = a.init;   // the entry state: [init_slot][H][P][N], or none
    int64_t init_slot = s;
    if (a.nseg > 1) {
        const int b = s / a.nseg, sg = s % a.nseg;
        row0 = (int64_t)b * a.T + (int64_t)sg * a.seglen;
        len = (int)min((int64_t)a.seglen, a.T - (int64_t)sg * a.seglen);
        sfin = sg == a.nseg - 1 ? b : -1;
        if (sg == 0) {
            init = a.init0;
            init_slot = b;
        }
    } else if (!a.seq_offsets) {
        row0 = (int64_t)s * a.T;
        len = (int)a.T;
    } else {
        row0 = a.seq_offsets[s];
        len = a.seq_offsets[s + 1] - a.seq_offsets[s];
    }
    const int nb = (len + 31) / 32;
    const int u0 = q * NW;                 // first unit of the workgroup
    const int hfirst = u0 / uph;           // first head (within the group) it touches
    const int64_t xrow = (int64_t)H * P;   // elements per token row of X / Y

    // ---- per-block product buffers and Y staging
    auto pbuf = [&](int t) __attribute__((always_inline)) -> lds_ptr { return (t & 1) ? sm.p[1] : sm.p[0]; };
    auto ybuf = [&](int t) __attribute__((always_inline)) -> lds_ptr { return (t & 1) ? sm.ys[1] : sm.ys[0]; };

    // ring and barrier discipline shared by both loaders: blocks 0 .. D-1 in flight before
    // the first step; step t issues block t + D (past the end: the last block again, so
    // that every step issues the same loads and the wait counts stay exact), waits for its
    // own loads of block t + 1, turns block t + 1 into its products and meets the other
    // waves at the barrier after which block t + 1 is complete and block t's slot is free.
    auto loader_loop = [&](auto issue, auto products, auto wait_rest) __attribute__((always_inline)) {
        if (nb > 0) {
            issue(0, std::integral_constant<int, 0>{});
            issue(1, std::integral_constant<int, 1>{});
            if constexpr (D == 3) issue(2, std::integral_constant<int, 2>{});
            wait_rest();
            products(0, std::integral_constant<int, 0>{});
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        auto step = [&](int t, auto kc) __attribute__((always_inline)) {
            constexpr int k = decltype(kc)::value;
            issue(t + D, std::integral_constant<int, (k + D) % NS>{});
            wait_rest();
            if (t + 1 < nb) products(t + 1, std::integral_constant<int, (k + 1) % NS>{});
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_s_barrier();
        };
        for (int t = 0; t < nb; t += NS) {
            step(t, std::integral_constant<int, 0>{});
            if (t + 1 < nb) step(t + 1, std::integral_constant<int, 1>{});
            if (t + 2 < nb) step(t + 2, std::integral_constant<int, 2>{});
            if constexpr (NS == 4)
                if (t + 3 < nb) step(t + 3, std::integral_constant<int, 3>{});
        }
        fused_wait_vm<0>();
        __builtin_amdgcn_s_barrier();
    };

    if (xloader) {
        // ------------------------------------------------------------ X loader: every unit's
        // X rows and the heads' logA; per head the block's cumsum, the row factors w and r,
        // the renormalisation factor and the path flag
        const int64_t xrx = (int64_t)a.xh * P;   // elements per token row of X
        const int hrep = H / a.xh;
        const rsrc_t xr = make_rsrc(a.X + row0 * xrx, (uint32_t)((int64_t)len * xrx * 2));
        // (REV: the decay of walked row j is that of the sequence's row len - j, rows 1 .. len - 1;
        // the buffer starts at row 1, so that walked row 0 and the rows past the sequence
        // read 0)
        const rsrc_t lar = REV ? make_rsrc(a.logA + (row0 + 1) * H, (uint32_t)(len > 0 ? (int64_t)(len - 1) * H * 4 : 0))
                               : make_rsrc(a.logA + row0 * H, (uint32_t)((int64_t)len * H * 4));
        // the slot holds the block's rows of the NW units side by side, [32][NW x 64 bytes],
        // filled in that order by 2 NW loads of 64 16-byte pieces: lane i of load j takes
        // piece 64 j + i, row (64 j + i) / 4 NW; with one X row per head the pieces of a
        // row are one contiguous run of memory (units past the group's last repeat it)
        uint32_t xl[2 * NW];
#pragma unroll
        for (int j = 0; j < 2 * NW; ++j) {
            const int pc = 64 * j + lane, row = pc / (4 * NW), piece = pc % (4 * NW);
            const int u = min(u0 + piece / 4, a.upg - 1);
            const int h = g * hpg + u / uph, c0 = 32 * (u % uph);
            const int64_t grow = REV ? (int64_t)len - 1 - row : row;
            xl[j] = (uint32_t)((grow * xrx + (int64_t)(h / hrep) * P + c0 + 8 * (piece % 4)) * 2);
        }
        // logA: lanes 0..31 head 2 p, lanes 32..63 head 2 p + 1 (clamped to the group)
        uint32_t ll[NPAIR];
#pragma unroll
        for (int p = 0; p < NPAIR; ++p) {
            const int hl = min(hfirst + 2 * p + lg, hpg - 1);
            ll[p] = (uint32_t)(((int64_t)(REV ? len - 1 - lr : lr) * H + g * hpg + hl) * 4);
        }
        const uint32_t rb32 = (uint32_t)(32 * xrx * 2), lab32 = (uint32_t)(32 * H * 4);
        // for the scaling in place: lane's piece j is 16-byte piece q % 4 of row (q % 128) / 4
        // of unit XS0 + q / 128, q = 64 j + lane; its head (local index), its byte offset in
        // the slot and the position of its row factor w in the products
        int xj[XSP > 0 ? XSP : 1];
        uint32_t xo[XSP > 0 ? XSP : 1], xw[XSP > 0 ? XSP : 1];
#pragma unroll
        for (int j = 0; j < XSP; ++j) {
            const int q = 64 * j + lane, unit = XS0 + q / 128, row = (q % 128) / 4;
            const int u = min(u0 + unit, a.upg - 1);
            xj[j] = u / uph - hfirst;
            xo[j] = (uint32_t)(row * NW * 64 + unit * 64 + 16 * (q % 4));
            xw[j] = (uint32_t)(L::w + 4 * (32 * xj[j] + sigma_pos(row)));
        }
        auto issue = [&](int b, auto kc) __attribute__((always_inline)) {
            constexpr int k = decltype(kc)::value;
            b = min(b, nb - 1);
#pragma unroll
            for (int j = 0; j < 2 * NW; ++j)
                fused_lds16(xr, XS(k) + 1024 * j, opaque(REV ? xl[j] - (uint32_t)b * rb32 : xl[j]), REV ? 0u : (uint32_t)b * rb32);
#pragma unroll
            for (int p = 0; p < NPAIR; ++p)
                fused_lds4(lar, LA(k) + 256 * p, opaque(REV ? ll[p] - (uint32_t)b * lab32 : ll[p]), REV ? 0u : (uint32_t)b * lab32);
        };
        float lsig[NPAIR];
#pragma unroll
        for (int p = 0; p < NPAIR; ++p) lsig[p] = 0.f;
        auto products = [&](int b, auto kc) __attribute__((always_inline)) {
            constexpr int k = decltype(kc)::value;
            lds_ptr pb = pbuf(b);
            const lds_ptr la = LA(k);
            uint32_t steep_heads = 0;   // bit jh: head jh takes the exact form
#pragma unroll
            for (int p = 0; p < NPAIR; ++p) {
                const int jh = 2 * p + lg;
                // inclusive cumsum over the 32 rows of each half (log2 units)
                const float c = scan32(ldsv<float>(la + 4 * (64 * p + lane)) * kLog2e);
                const float e = lg ? lane_f(c, 63) : lane_f(c, 31);
                const float c0 = lg ? lane_f(c, 32) : lane_f(c, 0);
                // path: 2 = exact form (span over 100), 1 = renormalise first, 0 = plain
                const bool steep = c0 - e > 100.f;
                const float ls = lsig[p];
                const bool renorm = steep || ls + e < -64.f;
                const float lnew = renorm ? 0.f : ls + e;
                const float w = fast_exp2(e - c - lnew);
                const float r = fast_exp2(steep ? c + ls : c - e + lnew);
                const float f = fast_exp2(ls + e);
                lsig[p] = lnew;
                const uint64_t sb = __ballot(steep);
                steep_heads |= (uint32_t)(sb & 1) << (2 * p) | (uint32_t)((sb >> 32) & 1) << (2 * p + 1);
                if (jh < NHL) {
                    ldsw<float>(pb + L::w + 4 * (32 * jh + sigma_pos(lr)), w);
                    ldsw<float>(pb + L::r + 4 * (32 * jh + lr), r);
                    ldsw<float>(pb + L::cs + 4 * (32 * jh + lr), c);
                    if (lr == 0) {
                        ldsw<float>(pb + L::f + 4 * jh, f);
                        ldsw<int>(pb + L::fl + 4 * jh, steep ? 2 : renorm ? 1 : 0);
                    }
                }
            }
            // X~ = w X in place, rounded to bf16 as the products read it; the rows of
            // heads that take the exact form stay unscaled (that form needs X itself)
            const lds_ptr xs = XS(k);
            u32x4 xv[XSP > 0 ? XSP : 1];
            float wv[XSP > 0 ? XSP : 1];
#pragma unroll
            for (int j = 0; j < XSP; ++j) {
                xv[j] = ldsv<u32x4>(xs + xo[j]);
                wv[j] = ldsv<float>(pb + xw[j]);
            }
#pragma unroll
            for (int j = 0; j < XSP; ++j) {
                const float wj = (steep_heads >> xj[j]) & 1 ? 1.f : wv[j];
                bf16x8 v = __builtin_bit_cast(bf16x8, xv[j]);
#pragma unroll
                for (int q = 0; q < 8; ++q) v[q] = (__bf16)((float)v[q] * wj);
                ldsw<u32x4>(xs + xo[j], __builtin_bit_cast(u32x4, v));
            }
        };
        loader_loop(issue, products, [&]() __attribute__((always_inline)) { fused_wait_vm<(D - 1) * LX>(); });
        // the heads' final log scales for the compute waves' final states
#pragma unroll
        for (int p = 0; p < NPAIR; ++p)
            if (2 * p + lg < NHL && lr == 0) ldsw<float>(pbuf(0) + L::f + 4 * (2 * p + lg), lsig[p]);
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        return;
    }

    if (storer) {
        // ------------------------------------------------------------ storer: once the
        // barrier after block t has passed, the workgroup's Y rows of block t from the
        // staging buffer: 32 rows of NW contiguous units (64 bytes each) as 16-byte
        // pieces, 4 NW per row, 64 pieces per store, streamed past the caches' reuse (the
        // kernel never reads Y)
        constexpr int NST = 2 * NW;
        const rsrc_t yr = make_rsrc(a.Y + row0 * xrow, (uint32_t)((int64_t)len * xrow * 2));
        uint32_t yo[NST], yl[NST];
        bool yv[NST];
#pragma unroll
        for (int i = 0; i < NST; ++i) {
            const int pc = 64 * i + lane, row = pc / (4 * NW), piece = pc % (4 * NW);
            const int64_t grow = REV ? (int64_t)len - 1 - row : row;
            yo[i] = (uint32_t)((grow * xrow + (int64_t)g * hpg * P + 32 * u0 + 8 * piece) * 2);
            yl[i] = (uint32_t)(row * L::ystride + 16 * piece);
            yv[i] = u0 + piece / 4 < a.upg;   // (units past the group's last are not ours)
        }
        const uint32_t yb32 = (uint32_t)(32 * xrow * 2);
        auto ystore = [&](int t) __attribute__((always_inline)) {
            const lds_ptr yb = ybuf(t);
            u32x4 v[NST];
#pragma unroll
            for (int i = 0; i < NST; ++i) v[i] = ldsv<u32x4>(yb + yl[i]);
#pragma unroll
            for (int i = 0; i < NST; ++i)
                if (yv[i])
                    __builtin_amdgcn_raw_buffer_store_b128(v[i], yr, (int)(REV ? yo[i] - (uint32_t)t * yb32 : yo[i]),
                                                           (int)(REV ? 0u : (uint32_t)t * yb32), kStreamAux);
        };
        // the same barriers as the other waves: the first, one per block, the last two
        __builtin_amdgcn_s_barrier();
        for (int t = 0; t < nb; ++t) {
            if (t > 0) ystore(t - 1);
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_s_barrier();
        }
        __builtin_amdgcn_s_barrier();
        if (nb > 0) ystore(nb - 1);
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        return;
    }

    if (bcloader) {
        // ------------------------------------------------------------ BC loader: the group's
        // B and C rows; per block the causally masked tile D^T = B C^T as MFMA fragments
        const rsrc_t br = make_rsrc(a.B + row0 * G * NP + g * NP, (uint32_t)((int64_t)len * G * NP * 2));
        const rsrc_t cr = make_rsrc(a.C + row0 * G * NP + g * NP, (uint32_t)((int64_t)len * G * NP * 2));
        // lane i of load k fills position i % UPR of row k RPL + i / UPR
        const int brow = lane / UPR, bpos = lane % UPR;
        uint32_t bl[NBL];
#pragma unroll
        for (int k = 0; k < NBL; ++k) {
            const int r = k * RPL + brow;
            const int64_t grow = REV ? (int64_t)len - 1 - r : r;
            bl[k] = (uint32_t)((grow * G * NP + 8 * (bpos ^ fused_swz<NP>(r))) * 2);
        }
        // its own copy of the heads' logA, for the exact tiles of steep blocks
        // (REV: the decay of walked row j is that of the sequence's row len - j, rows 1 .. len - 1;
        // the buffer starts at row 1, so that walked row 0 and the rows past the sequence
        // read 0)
        const rsrc_t lar = REV ? make_rsrc(a.logA + (row0 + 1) * H, (uint32_t)(len > 0 ? (int64_t)(len - 1) * H * 4 : 0))
                               : make_rsrc(a.logA + row0 * H, (uint32_t)((int64_t)len * H * 4));
        uint32_t ll[NPAIR];
#pragma unroll
        for (int p = 0; p < NPAIR; ++p) {
            const int hl = min(hfirst + 2 * p + lg, hpg - 1);
            ll[p] = (uint32_t)(((int64_t)(REV ? len - 1 - lr : lr) * H + g * hpg + hl) * 4);
        }
        const uint32_t bcb32 = (uint32_t)(32 * G * NP * 2), lab32 = (uint32_t)(32 * H * 4);
        auto issue = [&](int b, auto kc) __attribute__((always_inline)) {
            constexpr int k = decltype(kc)::value;
            b = min(b, nb - 1);
#pragma unroll
            for (int i = 0; i < NBL; ++i)
                fused_lds16(br, BS(k) + 1024 * i, opaque(REV ? bl[i] - (uint32_t)b * bcb32 : bl[i]), REV ? 0u : (uint32_t)b * bcb32);
#pragma unroll
            for (int i = 0; i < NBL; ++i)
                fused_lds16(cr, CS(k) + 1024 * i, opaque(REV ? bl[i] - (uint32_t)b * bcb32 : bl[i]), REV ? 0u : (uint32_t)b * bcb32);
#pragma unroll
            for (int p = 0; p < NPAIR; ++p)
                fused_lds4(lar, LA2(k) + 256 * p, opaque(REV ? ll[p] - (uint32_t)b * lab32 : ll[p]), REV ? 0u : (uint32_t)b * lab32);
        };
        auto products = [&](int b, auto kc) __attribute__((always_inline)) {
            constexpr int k = decltype(kc)::value;
            lds_ptr pb = pbuf(b);
            // D^T = B C^T (s x l) on MFMA, rows of both from the slot, two accumulator chains;
            // every fragment is read before the first product (one LDS round trip, not one per
            // K-step)
            const lds_ptr bsl = BS(k), csl = CS(k);
            // (in passes of at most four K-step pairs: eight reads of B and C each)
            constexpr int NK = NP / 16, KP = NK < 8 ? NK : 8;
            f32x16 acc0 = f32x16{}, acc1 = f32x16{};
#pragma unroll
            for (int k0 = 0; k0 < NK; k0 += KP) {
                bf16x8 r[2 * KP];
#pragma unroll
                for (int c = 0; c < 2 * KP; c += 8) {
                    uint32_t a8[8];
                    bf16x8 r8[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int kk = k0 + (c + i) % KP;
                        const int o = 2 * (lr * NP + 8 * ((2 * kk + lg) ^ fused_swz<NP>(lr)));
                        a8[i] = lds_addr(((c + i) < KP ? bsl : csl) + o);
                    }
                    lds_read8x16(a8, r8);
#pragma unroll
                    for (int i = 0; i < 8; ++i) r[c + i] = r8[i];
                }
#pragma unroll
                for (int kk = 0; kk < KP; kk += 2) {
                    acc0 = E::mma(acc0, r[kk], r[KP + kk]);
                    acc1 = E::mma(acc1, r[kk + 1], r[KP + kk + 1]);
                }
            }
            // causal mask (s <= l) and the fragments (K-step ks = elements 8 ks .. 8 ks + 7)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8 d;
#pragma unroll
                for (int q8 = 0; q8 < 8; ++q8) {
                    const int e8 = 8 * ks + q8;
                    const int srow = 8 * (e8 >> 2) + 4 * lg + (e8 & 3);
                    d[q8] = (__bf16)(srow <= lr ? acc0[e8] + acc1[e8] : 0.f);
                }
                ldsw<bf16x8>(pb + L::dg + 1024 * ks + 16 * lane, d);
            }
            // exact tiles of the heads whose block spans more than 100 (the X-loader's test
            // on the same cumsum): D'^T[s][l] = D^T[s][l] 2^(cs_l - cs_s)
            const lds_ptr la = LA2(k);
#pragma unroll
            for (int p = 0; p < NPAIR; ++p) {
                const float c = scan32(ldsv<float>(la + 4 * (64 * p + lane)) * kLog2e);
                const float e = lg ? lane_f(c, 63) : lane_f(c, 31);
                const float c0 = lg ? lane_f(c, 32) : lane_f(c, 0);
                const bool steep_lo = lane_f(c, 0) - lane_f(c, 31) > 100.f;
                const bool steep_hi = lane_f(c, 32) - lane_f(c, 63) > 100.f;
                if (steep_lo || steep_hi) {
                    (void)e;
                    (void)c0;
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int jh = 2 * p + hh;
                        if (jh >= NHL || !(hh ? steep_hi : steep_lo)) continue;
                        // lane (lg, lr) needs cs at l = lr and at its rows s of this head
                        const float cl = __shfl(c, 32 * hh + lr);
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks) {
                            bf16x8 t8;
#pragma unroll
                            for (int q8 = 0; q8 < 8; ++q8) {
                                const int e8 = 8 * ks + q8;
                                const int srow = 8 * (e8 >> 2) + 4 * lg + (e8 & 3);
                                const float csr = __shfl(c, 32 * hh + srow);
                                t8[q8] = (__bf16)(srow <= lr ? (acc0[e8] + acc1[e8]) * fast_exp2(cl - csr) : 0.f);
                            }
                            ldsw<bf16x8>(pb + L::st + 2048 * jh + 1024 * ks + 16 * lane, t8);
                        }
                    }
                }
            }
        };
        loader_loop(issue, products, [&]() __attribute__((always_inline)) { fused_wait_vm<(D - 1) * LB>(); });
        __builtin_amdgcn_s_barrier();
        return;
    }

    // ---------------------------------------------------------------- compute waves
    const int u = u0 + ci;
    const bool valid = u < a.upg;
    const int uc = valid ? u : a.upg - 1;
    const int hl = uc / uph;                      // head within the group
    const int h = g * hpg + hl;
    const int c0 = 32 * (uc % uph);               // first column of P
    const int jh = hl - hfirst;                   // local head index
    const int64_t state_base = (init_slot * H + h) * (int64_t)P * NP;

    f32x16 gs[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) gs[nt] = f32x16{};
    if (init) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 iv = *reinterpret_cast<const f32x4*>(init + state_base + (int64_t)(c0 + lr) * NP + 32 * nt +
                                                                  8 * q4 + 4 * lg);
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) gs[nt][4 * q4 + e4] = iv[e4];
            }
    }
    // LDS addresses (byte offsets inside a slot).  With the swizzle of B / C rows the unit
    // position of n tile nt is 4 (nt ^ a) + (m ^ b) for per-lane a, b: one base per n tile
    // and one per 16-byte unit inside it.
    constexpr int XR = NW * 64;   // bytes per row of the X slot
    const int xa0 = ci * 64 + XR * (4 * lg + ((lane & 15) >> 2)) + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
    // Per-lane LDS addresses of every operand read in slot 0: slot k is k bcbytes further
    // on, so each read is one register plus an immediate offset.  Kept in registers for up
    // to four n tiles (32 of them).  Beyond that each read's address is formed from one of
    // eight per-lane offsets of n tile 0: the tile part of the swizzle, 64 (nt ^ a), sits in
    // bits of its own (above the 16-byte unit, below the row), so n tile nt is that offset
    // XOR 64 nt, one instruction a read.
    const int sa = fused_swz<NP>(lr);
    const int rb = 4 * lg + ((lane & 15) >> 2);   // row of the transposing read, K-step 0, half 0
    const int vb = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    auto coff = [&](int m) __attribute__((always_inline)) -> uint32_t {
        return (uint32_t)(2 * lr * NP + 8 * lg + 16 * (sa & ~3) + 16 * (m ^ (sa & 3)));
    };
    auto boff = [&](int ks, int j) __attribute__((always_inline)) -> uint32_t {
        return (uint32_t)(2 * rb * NP + 8 * (lane & 1) + 16 * (fused_swz<NP>(rb) & ~3) +
                          16 * (vb ^ (fused_swz<NP>(16 * ks + 8 * j + rb) & 3)) + 32 * NP * ks + 16 * NP * j);
    };
    constexpr bool kept = NT <= 4;           // every n tile's addresses in registers
    constexpr int NTK = kept ? NT : 1;
    lds_ptr ca[NTK][4];      // C pieces of row lr: n tile nt, piece m = 2 kk + j
    lds_ptr ba[NTK][2][2];   // B^T transposing reads: n tile nt, K-step, 4-row half
    uint32_t co[4], bo[2][2];   // (beyond four n tiles) the offsets of n tile 0
#pragma unroll
    for (int m = 0; m < 4; ++m) co[m] = coff(m);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int j = 0; j < 2; ++j) bo[ks][j] = boff(ks, j);
#pragma unroll
    for (int nt = 0; nt < NTK; ++nt) {
#pragma unroll
        for (int m = 0; m < 4; ++m) ca[nt][m] = CS(0) + (co[m] ^ (64 * nt));
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int j = 0; j < 2; ++j) ba[nt][ks][j] = BS(0) + (bo[ks][j] ^ (64 * nt));
    }
    // (rows 16 ks + 8 j + rb have rb's part 4 (r % U4) of the swizzle, U4 dividing 8; only the
    // low two bits, (r / U4) % 4, change with ks and j)

    __builtin_amdgcn_s_barrier();
    auto step = [&](int t, auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        const lds_ptr pb = pbuf(t);
        const lds_ptr xsl = XS(k);
        constexpr int ko = k * LL::bcbytes;   // slot k of the B and C rings
        // X of the block (K-step ks: rows 16 ks + sigma(8 lg + q))
        bf16x8 xf[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            xf[ks] = cat44(tr4(xsl + xa0 + 16 * XR * ks), tr4(xsl + xa0 + 16 * XR * ks + 8 * XR));
        const int flag = __builtin_amdgcn_readfirstlane(ldsv<int>(pb + L::fl + 4 * jh));
        const float f = ldsv<float>(pb + L::f + 4 * jh);
        const float rl = ldsv<float>(pb + L::r + 4 * (32 * jh + lr));
        // the slot holds X~ = w X (units the X-loader scales, but for a block of this head
        // that takes the exact form) or X itself: then X~ is formed here
        bf16x8 xt[2] = {xf[0], xf[1]};
        if (ci < XS0 || flag == 2) {
            asm volatile("");
            const lds_ptr wp = pb + L::w + 128 * jh + 32 * lg;
            const f32x4 w00 = ldsv<f32x4>(wp), w01 = ldsv<f32x4>(wp + 16), w10 = ldsv<f32x4>(wp + 64),
                        w11 = ldsv<f32x4>(wp + 80);
            const float ws[2][8] = {{w00[0], w00[1], w00[2], w00[3], w01[0], w01[1], w01[2], w01[3]},
                                    {w10[0], w10[1], w10[2], w10[3], w11[0], w11[1], w11[2], w11[3]}};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int q8 = 0; q8 < 8; ++q8) xt[ks][q8] = (__bf16)((float)xf[ks][q8] * ws[ks][q8]);
        }
        // One code path for the three kinds of block; the flag only switches in-place
        // scalings and the diagonal tile's operands, so the state stays in the same
        // registers whatever the path (branches of their own around the scalings: as
        // selects every block would pay them).
        //   plain (0):        Y = r [C g + D X~],                 g' = g + B^T X~
        //   renormalise (1):  g <- f g first, then as plain
        //   exact (2):        Y = r C g + D_exact X,              g' = f g + B^T X~
        // The left factor C g over every n tile comes first, then the diagonal tile's two
        // products, then the state update: runs of straight-line code, so that the reads of
        // later n tiles can be issued ahead of the products of earlier ones (no branch
        // between them), and Y leaves the accumulator while the state update runs.
        const bool renorm = flag == 1, exact = flag == 2;
        // the diagonal tile's fragments (shared, or this head's exact tile)
        const lds_ptr dp = exact ? pb + L::st + 2048 * jh : pb + L::dg;
        const bf16x8 d0 = ldsv<bf16x8>(dp + 16 * lane);
        const bf16x8 d1 = ldsv<bf16x8>(dp + 1024 + 16 * lane);
        // (beyond four n tiles: this block's copies of the tile-0 offsets, through opaque()
        // so that the compiler cannot hoist every tile's addresses out of the walk and hold
        // them in registers after all)
        uint32_t cq[4], bq[2][2];
        if constexpr (!kept) {
#pragma unroll
            for (int m = 0; m < 4; ++m) cq[m] = opaque(co[m]);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int j = 0; j < 2; ++j) bq[ks][j] = opaque(bo[ks][j]);
        }
        auto cad = [&](int nt, int m) __attribute__((always_inline)) -> lds_ptr {
            if constexpr (kept) return ca[nt % NTK][m];
            else return CS(0) + (cq[m] ^ (64 * nt));
        };
        auto bad = [&](int nt, int ks, int j) __attribute__((always_inline)) -> lds_ptr {
            if constexpr (kept) return ba[nt % NTK][ks][j];
            else return BS(0) + (bq[ks][j] ^ (64 * nt));
        };
        // the left factor's two K-steps per n tile on the state before its update; the C
        // pieces of n tile nt + PF are read before the products of n tile nt (scheduling
        // barriers keep that order)
        constexpr int PF = 2;
        u32x2 cp[NT][4];
        auto cread = [&](int nt) __attribute__((always_inline)) {
#pragma unroll
            for (int m = 0; m < 4; ++m) cp[nt][m] = ldsv<u32x2>(cad(nt, m) + ko);
        };
        bf16x8 bt[NT][2];
        auto bread = [&](int nt) __attribute__((always_inline)) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) bt[nt][kk] = cat44(tr4(bad(nt, kk, 0) + ko), tr4(bad(nt, kk, 1) + ko));
        };
        if (renorm) {
            asm volatile("");
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) gs[nt] *= f;
        }
        f32x16 acc = f32x16{};
#pragma unroll
        for (int nt = 0; nt < PF && nt < NT; ++nt) cread(nt);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            if (nt + PF < NT) cread(nt + PF);
            else if (nt + PF - NT < PF) bread(nt + PF - NT);
            __builtin_amdgcn_sched_barrier(0);
            bf16x8 hb[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
                for (int q8 = 0; q8 < 8; ++q8) hb[kk][q8] = (__bf16)gs[nt][8 * kk + q8];
                const bf16x8 cf = __builtin_bit_cast(bf16x8, u32x4{cp[nt][2 * kk][0], cp[nt][2 * kk][1],
                                                                   cp[nt][2 * kk + 1][0], cp[nt][2 * kk + 1][1]});
                acc = E::mma(acc, hb[kk], cf);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // the diagonal tile: the shared masked tile on X~, or (exact) this head's tile with
        // the exact decays on unscaled X, added after the row factor.  It does not depend
        // on the state update, so it comes first and the row factor and the bf16 rows of Y
        // are issued between the state update's products (their latency hidden under them).
        if (exact) {
            asm volatile("");
            acc *= rl;
        }
        // (X~ for the shared tile, X itself for the exact one)
        bf16x8 xd[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) xd[ks] = exact ? xf[ks] : xt[ks];
        acc = E::mma(acc, xd[0], d0);
        acc = E::mma(acc, xd[1], d1);
        if (exact) {
            asm volatile("");
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) gs[nt] *= f;
        }
        // Y^T (p x l) to the staging buffer as bf16 rows: lane (l, lg) holds columns
        // 8 q + 4 lg .. + 3 of row l, q = 0 .. 3 (the storer writes the block out after the
        // barrier)
        auto ywrite = [&]() __attribute__((always_inline)) {
            if (!exact) {
                asm volatile("");
                acc *= rl;
            }
            const lds_ptr yb = ybuf(t) + lr * L::ystride + ci * 64 + 8 * lg;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const bf16x2 v0 = {(__bf16)acc[4 * q], (__bf16)acc[4 * q + 1]};
                const bf16x2 v1 = {(__bf16)acc[4 * q + 2], (__bf16)acc[4 * q + 3]};
                ldsw<u32x2>(yb + 16 * q, u32x2{__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1)});
            }
        };
        // the state update (B^T fragments of n tile nt + PF read before the products of nt);
        // Y's row factor and bf16 rows after the products of the second n tile (by then the
        // diagonal tile's result has arrived, and the rest of the update runs under them)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            if (nt + PF < NT) bread(nt + PF);
            __builtin_amdgcn_sched_barrier(0);
            gs[nt] = E::mma(gs[nt], bt[nt][0], xt[0]);
            gs[nt] = E::mma(gs[nt], bt[nt][1], xt[1]);
            __builtin_amdgcn_sched_barrier(0);
            if (nt == 1) ywrite();
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
    };
    for (int t = 0; t < nb; t += NS) {
        step(t, std::integral_constant<int, 0>{});
        if (t + 1 < nb) step(t + 1, std::integral_constant<int, 1>{});
        if (t + 2 < nb) step(t + 2, std::integral_constant<int, 2>{});
        if constexpr (NS == 4)
            if (t + 3 < nb) step(t + 3, std::integral_constant<int, 3>{});
    }
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_s_barrier();
    if (a.final_state && valid && sfin >= 0) {
        const int64_t fin_base = (sfin * H + h) * (int64_t)P * NP;
        const float fs = fast_exp2(ldsv<float>(pbuf(0) + L::f + 4 * jh));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 o = {gs[nt][4 * q4] * fs, gs[nt][4 * q4 + 1] * fs, gs[nt][4 * q4 + 2] * fs,
                                 gs[nt][4 * q4 + 3] * fs};
                *reinterpret_cast<f32x4*>(a.final_state + fin_base + (int64_t)(c0 + lr) * NP + 32 * nt + 8 * q4 +
                                          4 * lg) = o;
            }
    }
}

// Workgroup bid of nblocks (a multiple of 8 where sequences are dealt to XCDs) -> its
// (sequence, group, run of units), then the walk.
template <int NP, int NW, bool REV>
__device__ __forceinline__ void fused_item_walk(const FusedArgs& a, int bid, int nblocks) {
    const int lane = threadIdx.x & 63;
    const int G = a.G, wpg = a.wpg;
    int s, g, q;
    if (a.lpt) {
        // packed sequences: the (sequence, group) units are dealt to the XCDs
        // round-robin, longest sequence first
        const int xcd = bid % 8, slot = bid / 8;
        const int un = (slot / wpg) * 8 + xcd;
        q = slot % wpg;
        const int r = un / G;
        g = un % G;
        if (r >= a.nseq) return;
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
        const int item = xcd_remap(bid, nblocks);
        if (item >= a.nitems) return;
        q = item % wpg;
        const int sg = item / wpg;
        g = sg % G;
        s = sg / G;
    }
    fused_walk<NP, NW, REV>(a, s, g, q);
}

template <int NP, int NW, bool REV = false>
__global__ void __launch_bounds__(64 * (NW + 3), 1) ssd_walk_fused_kernel(FusedArgs a) {
    fused_item_walk<NP, NW, REV>(a, blockIdx.x, gridDim.x);
}

// Two independent walks of one shape in one launch (the backward pass's dB and dC passes):
// workgroups [0, n0) walk a0, the rest a1.  n0 is a multiple of 8, so that both ranges meet
// the XCDs alike; the two together leave fewer partial rounds of workgroups over the chip
// than two launches.
template <int NP, int NW, bool REV0, bool REV1>
__global__ void __launch_bounds__(64 * (NW + 3), 1) ssd_walk_fused_pair_kernel(FusedArgs a0, FusedArgs a1, int n0) {
    if constexpr (REV0 == REV1) {
        const bool second = (int)blockIdx.x >= n0;
        const FusedArgs a = second ? a1 : a0;
        fused_item_walk<NP, NW, REV0>(a, second ? (int)blockIdx.x - n0 : (int)blockIdx.x, second ? (int)gridDim.x - n0 : n0);
    } else {
        if ((int)blockIdx.x < n0) fused_item_walk<NP, NW, REV0>(a0, blockIdx.x, n0);
        else fused_item_walk<NP, NW, REV1>(a1, (int)blockIdx.x - n0, (int)gridDim.x - n0);
    }
}

}  // namespace ssd
