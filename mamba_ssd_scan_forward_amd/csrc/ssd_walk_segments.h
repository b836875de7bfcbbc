// ssd_walk_segments.h -- one long sequence walked as segments in parallel (page
// "Transformers are SSMs" paper summary, section 6.2 and Appendix B: the state passed
// between consecutive pieces of the sequence is a linear recurrence over the pieces, so
// each piece's contribution can be formed on its own and the pieces chained afterwards).
//
// A sequence too long for the chip to be filled by its (group, run of head columns)
// workgroups is cut into nseg segments of seglen rows.  Three launches:
//   summary  every segment but the last, from a zero state: its end state
//                loc_s = sum_t exp(L_{t+1..end}) x_t B_t^T     (L: the sum of logA)
//            and its total log decay D_s = sum_t logA_t; the first segment from the
//            sequence's initial state h_0 instead, which gives the second one's entry
//            state h_1 = exp(D_0) h_0 + loc_0 directly;
//   combine  (three segments or more) the entry states of the others,
//                h_{s+1} = exp(D_s) h_s + loc_s,
//            one segment after the other for short chains, as an associative scan of
//            the (decay, state) pairs for long ones;
//   walk     the fused walker with every segment a sequence of its own, entering with
//            h_s (the first with h_0 itself); the last segment's final state is the
//            sequence's.
// The summary is a plain contraction over the segment's rows: each row is weighted by its
// decay to the segment's end (a suffix sum of logA, at most 1 in size), so there is no
// running scale to keep, and it reads X and B once.
#pragma once

#include "ssd_walk_fused.h"

namespace ssd {

struct SegSumArgs {
    const __bf16* X;
    const float* logA;
    const __bf16* B;
    const float* init;   // the sequences' initial states [nseq][H][P][N] float32, or NULL (zero)
    float* loc;     // [nseq][nseg - 1][H][P][N] float32 (segment 0's entry unused)
    float* dsum;    // [nseq][nseg - 1][H] float32 (natural log; segment 0's entry unused)
    float* sinit;   // the segments' entry states [nseq][nseg][H][P][N] float32: h_1 written here
    int64_t T;      // rows per sequence
    int seglen, nseg, nseq;
    int H, P, G, xh;
    int upg;        // 32-column units per group: (H / G) (P / 32)
    int wpg;        // summary workgroups per group: ceil(upg / kSumUnits)
    int nitems;     // nseq (nseg - 1) G wpg
};

constexpr int kSumUnits = 5;                   // units per summary workgroup, one compute wave each
constexpr int kSumThreads = 64 * (kSumUnits + 3);   // and three loader waves

// One workgroup per (sequence, segment but the last, group, run of kSumUnits units): the
// segment's 32-row blocks from the last to the first, two blocks a step, per unit
//     g^T += B^T X~,   X~_t = exp(L_{t+1..end}) X_t
// on MFMA with the operand layouts of the fused walker (B rows swizzled by fused_swz,
// X read with 4-row transposing reads, rows of the contraction in the sigma order).
// Waves 0 .. kSumUnits - 1 compute one unit each and issue no memory instruction; the
// B-loader (wave kSumUnits), the X-loader (the next wave: the units' X rows) and the
// logA-loader (the last) bring each block straight from global memory into a ring of
// eight LDS slots, three steps (six blocks) ahead.  The step's fixed chain (the logA read, one scan over both
// blocks' 64 rows, the weights' round trip through LDS, the barrier) is paid once per 64
// rows.  Five units make a d_state-128 layer of 80 heads 32 workgroups a segment, so the
// seven segments but the last of a 16K-token sequence take one compute unit each.
template <int NP>
__global__ void __launch_bounds__(kSumThreads, 1) ssd_seg_summary_kernel(SegSumArgs a) {
    typedef Elem<__bf16> E;
    constexpr int NT = NP / 32;
    constexpr int UPR = NP / 8;             // 16-byte units of a B row
    constexpr int RPL = 64 / UPR;           // B rows per 1 KB load
    constexpr int NBL = NP / 16;            // 1 KB loads of B per block
    constexpr int XR = kSumUnits * 64;      // bytes per row of the X slot
    static_assert(32 * XR % 1024 == 0, "whole 1 KB loads of X");
    constexpr int NXL = 32 * XR / 1024;     // 1 KB loads of X per block
    constexpr int NLL = (kSumUnits + 1) / 2;   // logA loads per block (two units' heads each)
    constexpr int LSZ = 256 * NLL;          // bytes of a logA slot: [units][32] float
    constexpr int NSL = 8, DS = 3;          // ring slots (four steps of two blocks), steps in flight
    constexpr int LB = 2 * NBL, LX = 2 * NXL, LL = 2 * NLL;   // loads per step of each loader
    static_assert(DS * LB < 64 && DS * LX < 64 && DS * LL < 64, "vmcnt range");
    // (separate arrays per slot, so that the compiler can tell the slots being read from
    // the slots still being filled by direct-to-LDS loads; selected by constant index)
    __shared__ __align__(16) unsigned char b0[32 * NP * 2], b1[32 * NP * 2], b2[32 * NP * 2], b3[32 * NP * 2],
        b4[32 * NP * 2], b5[32 * NP * 2], b6[32 * NP * 2], b7[32 * NP * 2];
    __shared__ __align__(16) unsigned char x0[32 * XR], x1[32 * XR], x2[32 * XR], x3[32 * XR], x4[32 * XR],
        x5[32 * XR], x6[32 * XR], x7[32 * XR];
    __shared__ __align__(16) unsigned char l0[LSZ], l1[LSZ], l2[LSZ], l3[LSZ], l4[LSZ], l5[LSZ], l6[LSZ], l7[LSZ];
    __shared__ __align__(16) unsigned char wsm[kSumUnits * 256];   // row weights, [wave][64] float
    auto pick = [](int k, unsigned char* a0, unsigned char* a1, unsigned char* a2, unsigned char* a3,
                   unsigned char* a4, unsigned char* a5, unsigned char* a6,
                   unsigned char* a7) __attribute__((always_inline)) -> lds_ptr {
        return k == 0 ? (lds_ptr)a0 : k == 1 ? (lds_ptr)a1 : k == 2 ? (lds_ptr)a2 : k == 3 ? (lds_ptr)a3
             : k == 4 ? (lds_ptr)a4 : k == 5 ? (lds_ptr)a5 : k == 6 ? (lds_ptr)a6 : (lds_ptr)a7;
    };
    auto BS = [&](int k) __attribute__((always_inline)) { return pick(k, b0, b1, b2, b3, b4, b5, b6, b7); };
    auto XS = [&](int k) __attribute__((always_inline)) { return pick(k, x0, x1, x2, x3, x4, x5, x6, x7); };
    auto LS = [&](int k) __attribute__((always_inline)) { return pick(k, l0, l1, l2, l3, l4, l5, l6, l7); };

    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool bloader = wave == kSumUnits, xloader = wave == kSumUnits + 1, lloader = wave == kSumUnits + 2;
    // (consecutive items, the units of one segment and group, on one XCD: its L2 then
    // fetches the segment's B rows and logA once, not once per XCD)
    const int item = xcd_remap(blockIdx.x, gridDim.x);
    if (item >= a.nitems) return;
    const int H = a.H, P = a.P, G = a.G, hpg = H / G, uph = P / 32;
    const int q = item % a.wpg;
    int rest = item / a.wpg;
    const int g = rest % G;
    rest /= G;
    const int sg = rest % (a.nseg - 1), b = rest / (a.nseg - 1);
    const int64_t row0 = (int64_t)b * a.T + (int64_t)sg * a.seglen;
    const int nblk = a.seglen / 32;
    const int u0 = q * kSumUnits;
    const int64_t xrx = (int64_t)a.xh * P;
    const int hrep = H / a.xh;

    // ---- loads: lane i of B load k fills position i % UPR of row k RPL + i / UPR (global
    // unit position ^ swizzle); lane i of logA load p row i % 32 of the head of unit 2 p
    // (i < 32) or 2 p + 1; lane i of X load j piece 64 j + i of the [32][units] rows (units
    // clamped to the group's last)
    const rsrc_t br = make_rsrc(a.B + row0 * G * NP + g * NP, (uint32_t)((int64_t)a.seglen * G * NP * 2));
    const rsrc_t xr = make_rsrc(a.X + row0 * xrx, (uint32_t)((int64_t)a.seglen * xrx * 2));
    const rsrc_t lar = make_rsrc(a.logA + row0 * H, (uint32_t)((int64_t)a.seglen * H * 4));
    uint32_t off[NBL > NXL ? NBL : NXL];
    uint32_t loff[NLL] = {};
    if (bloader) {
        const int brow = lane / UPR, bpos = lane % UPR;
#pragma unroll
        for (int k = 0; k < NBL; ++k) {
            const int r = k * RPL + brow;
            off[k] = (uint32_t)((r * G * NP + 8 * (bpos ^ fused_swz<NP>(r))) * 2);
        }
    } else if (lloader) {
#pragma unroll
        for (int p = 0; p < NLL; ++p)
            loff[p] = (uint32_t)((lr * H + g * hpg + min(u0 + 2 * p + lg, a.upg - 1) / uph) * 4);
    } else if (xloader) {
#pragma unroll
        for (int j = 0; j < NXL; ++j) {
            const int pc = 64 * j + lane, r = pc / (4 * kSumUnits), piece = pc % (4 * kSumUnits);
            const int u = min(u0 + piece / 4, a.upg - 1);
            const int h = g * hpg + u / uph, c0 = 32 * (u % uph);
            off[j] = (uint32_t)((r * xrx + (int64_t)(h / hrep) * P + c0 + 8 * (piece % 4)) * 2);
        }
    }
    const uint32_t bb32 = (uint32_t)(32 * G * NP * 2), xb32 = (uint32_t)(32 * xrx * 2), lb32 = (uint32_t)(32 * H * 4);
    // walk position t (0, 1, ...) is block nblk - 1 - t of the segment, in slot t % NSL
    // (past the first block: the first again, so that every step issues the same loads and
    // the wait counts stay exact); step s holds positions 2 s and 2 s + 1
    auto issue = [&](int t, auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        const uint32_t blk = (uint32_t)max(nblk - 1 - t, 0);
        if (bloader) {
#pragma unroll
            for (int i = 0; i < NBL; ++i) fused_lds16(br, BS(k) + 1024 * i, opaque(off[i]), blk * bb32);
        } else if (lloader) {
#pragma unroll
            for (int p = 0; p < NLL; ++p) fused_lds4(lar, LS(k) + 256 * p, opaque(loff[p]), blk * lb32);
        } else if (xloader) {
#pragma unroll
            for (int j = 0; j < NXL; ++j) fused_lds16(xr, XS(k) + 1024 * j, opaque(off[j]), blk * xb32);
        }
    };

    // this wave's unit
    const int u = u0 + wave;
    const bool valid = wave < kSumUnits && u < a.upg;
    const int uc = min(u, a.upg - 1);
    const int h = g * hpg + uc / uph, c0 = 32 * (uc % uph);

    // operand addresses (as in the fused walker, one X slot row of kSumUnits units)
    const int xa0 = wave * 64 + XR * (4 * lg + ((lane & 15) >> 2)) + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
    int ba[NT][2][2];
    {
        const int rb4 = 4 * lg + ((lane & 15) >> 2);
        const int v = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int bnt = 2 * rb4 * NP + 8 * (lane & 1) + 16 * ((4 * nt) ^ (fused_swz<NP>(rb4) & ~3));
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    ba[nt][ks][j] = bnt + 16 * (v ^ (fused_swz<NP>(16 * ks + 8 * j + rb4) & 3)) + 32 * NP * ks + 16 * NP * j;
        }
    }

    f32x16 gs[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) gs[nt] = f32x16{};
    float carry = 0.f;   // sum of logA over the rows after this step, within the segment
    issue(0, std::integral_constant<int, 0>{});
    issue(1, std::integral_constant<int, 1>{});
    issue(2, std::integral_constant<int, 2>{});
    issue(3, std::integral_constant<int, 3>{});
    issue(4, std::integral_constant<int, 4>{});
    issue(5, std::integral_constant<int, 5>{});
    const lds_ptr wme = (lds_ptr)wsm + 256 * (wave < kSumUnits ? wave : 0);
    // one block's products: its B^T operands, its X rows and their weights (at wo in the
    // wave's weights), eight MFMAs
    auto block = [&](lds_ptr bsl, lds_ptr xsl, int wo) __attribute__((always_inline)) {
        bf16x8 bt[NT][2];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) bt[nt][ks] = cat44(tr4(bsl + ba[nt][ks][0]), tr4(bsl + ba[nt][ks][1]));
        bf16x8 xt[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            // rows 16 ks + sigma(8 lg + q) of the block
            const bf16x8 xf = cat44(tr4(xsl + xa0 + 16 * XR * ks), tr4(xsl + xa0 + 16 * XR * ks + 8 * XR));
            const f32x4 w0 = ldsv<f32x4>(wme + wo + 4 * (16 * ks + 4 * lg));
            const f32x4 w1 = ldsv<f32x4>(wme + wo + 4 * (16 * ks + 8 + 4 * lg));
            const float ws[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
#pragma unroll
            for (int q8 = 0; q8 < 8; ++q8) xt[ks][q8] = (__bf16)((float)xf[q8] * ws[q8]);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) gs[nt] = E::mma(gs[nt], bt[nt][ks], xt[ks]);
    };
    auto step = [&](int s, auto kc) __attribute__((always_inline)) {
        constexpr int j = decltype(kc)::value;
        constexpr int kL = 2 * j, kE = 2 * j + 1;   // slots of the later and the earlier block
        // the loaders' loads of step s are in (the steps after it still in flight), and after the
        // barrier every loader's are; every wave has also finished step s - 1, whose slots
        // the next issue reuses
        // (a bare barrier: __syncthreads would also wait for every load in flight)
        if (bloader) fused_wait_vm<(DS - 1) * LB>();
        else if (xloader) fused_wait_vm<(DS - 1) * LX>();
        else if (lloader) fused_wait_vm<(DS - 1) * LL>();
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        issue(2 * s + 2 * DS, std::integral_constant<int, (kL + 2 * DS) % NSL>{});
        issue(2 * s + 2 * DS + 1, std::integral_constant<int, (kE + 2 * DS) % NSL>{});
        if (wave >= kSumUnits) return;
        // whether the step has an earlier block (an odd block count leaves the last step one)
        const bool hasE = 2 * s + 1 < nblk;
        // row weights of this wave's head over both blocks: lanes 0..31 the earlier block's
        // rows, 32..63 the later block's; exp of the logA sum over the later rows (in asm with
        // its own wait: as a plain read the compiler would first wait for every
        // direct-to-LDS load in flight)
        const float la = lds_read4((lg ? LS(kL) : LS(kE)) + 4 * (32 * wave + lr));
        const float c = scan32(la);   // inclusive, within each half
        const float totE = hasE ? lane_f(c, 31) : 0.f, totL = lane_f(c, 63);
        const float w = (lg || hasE) ? fast_exp2((carry + (lg ? totL - c : totE - c + totL)) * kLog2e) : 0.f;
        ldsw<float>(wme + 4 * lane, w);
        carry += totE + totL;
        block(BS(kL), XS(kL), 128);
        if (hasE) block(BS(kE), XS(kE), 0);
    };
    const int nstep = (nblk + 1) / 2;
    for (int s = 0; s < nstep; s += 4) {
        step(s, std::integral_constant<int, 0>{});
        if (s + 1 < nstep) step(s + 1, std::integral_constant<int, 1>{});
        if (s + 2 < nstep) step(s + 2, std::integral_constant<int, 2>{});
        if (s + 3 < nstep) step(s + 3, std::integral_constant<int, 3>{});
    }
    // no load may still be landing in LDS when the workgroup ends
    fused_wait_vm<0>();
    if (!valid) return;
    if (sg == 0) {
        // h_1 = exp(D_0) h_0 + loc_0 (carry is D_0 now): the second segment's entry state
        const float d = fast_exp2(carry * kLog2e);
        const int64_t off = (int64_t)(c0 + lr) * NP + 4 * lg;
        const float* ip = a.init ? a.init + ((int64_t)b * H + h) * (int64_t)P * NP + off : nullptr;
        float* o = a.sinit + (((int64_t)b * a.nseg + 1) * H + h) * (int64_t)P * NP + off;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                f32x4 v = {gs[nt][4 * q4], gs[nt][4 * q4 + 1], gs[nt][4 * q4 + 2], gs[nt][4 * q4 + 3]};
                if (ip) {
                    const f32x4 iv = *reinterpret_cast<const f32x4*>(ip + 32 * nt + 8 * q4);
                    v = f32x4{d * iv[0] + v[0], d * iv[1] + v[1], d * iv[2] + v[2], d * iv[3] + v[3]};
                }
                *reinterpret_cast<f32x4*>(o + 32 * nt + 8 * q4) = v;
            }
        return;
    }
    const int64_t slot = ((int64_t)b * (a.nseg - 1) + sg) * H + h;
    float* o = a.loc + slot * (int64_t)P * NP;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 v = {gs[nt][4 * q4], gs[nt][4 * q4 + 1], gs[nt][4 * q4 + 2], gs[nt][4 * q4 + 3]};
            *reinterpret_cast<f32x4*>(o + (int64_t)(c0 + lr) * NP + 32 * nt + 8 * q4 + 4 * lg) = v;
        }
    if (c0 == 0 && lane == 0) a.dsum[slot] = carry;
}

// Entry states of the third segment on, by an associative scan over the segments (page
// "Transformers are SSMs" paper summary, Appendix B: the recurrence's step from one piece of
// the sequence to the next is the affine map h -> a h + b, and composing two of them,
// (a2, b2) after (a1, b1) = (a2 a1, a2 b1 + b2), is associative, so the entry states of all
// pieces are an inclusive scan of these pairs).  Segment s (1 <= s <= nseg - 2) contributes
// (exp(D_s), loc_s); with h_1 (which the first segment's summary wrote),
//     h_{s+1} = A_s h_1 + B_s,   (A_s, B_s) = (a_s, b_s) o ... o (a_1, b_1).
// A workgroup takes one (sequence, head, 256 consecutive state elements): 64 lanes of 4
// elements each by kScanSeg segment rows; the pairs of kScanSeg segments at a time are
// scanned in log2(kScanSeg) steps (each row combines its pair with the one 1, 2, 4, 8 rows
// earlier, through LDS), then applied to the entry state carried from the previous rows.
// Used for chains longer than kScanSeg segments (a sequence cut into many segments: 64 of
// 1024 rows, 8 heads, measured 89.3 -> 78.6 us for the whole forward against the chain
// below); shorter chains take ssd_seg_chain_kernel (8 segments: 5 us faster).
constexpr int kScanSeg = 16;
__global__ void __launch_bounds__(64 * kScanSeg) ssd_seg_scan_kernel(const float* loc, const float* dsum,
                                                                        float* seg_init, int nseq, int nseg, int H,
                                                                        int PN) {
    __shared__ float sa[kScanSeg][64];
    __shared__ f32x4 sb[kScanSeg][64];
    __shared__ f32x4 carry[64];
    const int x = threadIdx.x & 63, j = threadIdx.x >> 6;
    const int e = 256 * blockIdx.x + 4 * x;   // (PN is a multiple of 256)
    const int h = blockIdx.y, b = blockIdx.z;
    if (j == 0) carry[x] = *reinterpret_cast<const f32x4*>(seg_init + (((int64_t)b * nseg + 1) * H + h) * PN + e);
    for (int c0 = 1; c0 + 1 < nseg; c0 += kScanSeg) {
        const int s = c0 + j;
        const bool valid = s + 1 < nseg;
        float a = 1.f;
        f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
        if (valid) {
            const int64_t slot = ((int64_t)b * (nseg - 1) + s) * H + h;
            a = fast_exp2(dsum[slot] * kLog2e);
            v = *reinterpret_cast<const f32x4*>(loc + slot * PN + e);
        }
        // inclusive scan over the rows: after the step of distance k, row j holds the
        // composite of segments max(c0, s - 2k + 1) .. s
#pragma unroll
        for (int k = 1; k < kScanSeg; k *= 2) {
            sa[j][x] = a;
            sb[j][x] = v;
            __syncthreads();
            if (j >= k) {
                const float ap = sa[j - k][x];
                const f32x4 bp = sb[j - k][x];
                v = f32x4{a * bp[0] + v[0], a * bp[1] + v[1], a * bp[2] + v[2], a * bp[3] + v[3]};
                a *= ap;
            }
            __syncthreads();
        }
        // h_{s+1} from the entry state of segment c0 (h_1, or the previous rows' last)
        const f32x4 hin = carry[x];
        const f32x4 hout = f32x4{a * hin[0] + v[0], a * hin[1] + v[1], a * hin[2] + v[2], a * hin[3] + v[3]};
        if (valid) *reinterpret_cast<f32x4*>(seg_init + (((int64_t)b * nseg + s + 1) * H + h) * PN + e) = hout;
        __syncthreads();
        if (j == kScanSeg - 1) carry[x] = hout;   // (only read when another pass follows: then every row was valid)
        __syncthreads();
    }
}

// Entry states of the third segment on for chains of at most kScanSeg segments, one after
// the other: h_{s+1} = exp(D_s) h_s + loc_s from h_1 (which the summary of the first segment
// wrote), for every (sequence, head) and 4 consecutive state elements per thread (its loads
// of every segment independent of each other, so all of them are in flight at once).
__global__ void __launch_bounds__(256) ssd_seg_chain_kernel(const float* loc, const float* dsum, float* seg_init,
                                                              int nseq, int nseg, int H, int PN) {
    const int n4 = PN / 4;
    const int64_t total = (int64_t)nseq * H * n4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int e4 = (int)(i % n4);
        const int64_t bh = i / n4;
        const int h = (int)(bh % H), b = (int)(bh / H);
        f32x4 v = *reinterpret_cast<const f32x4*>(seg_init + (((int64_t)b * nseg + 1) * H + h) * PN + 4 * e4);
        for (int s = 1; s + 1 < nseg; ++s) {
            const int64_t slot = ((int64_t)b * (nseg - 1) + s) * H + h;
            const float d = fast_exp2(dsum[slot] * kLog2e);
            const f32x4 l = *reinterpret_cast<const f32x4*>(loc + slot * PN + 4 * e4);
            v = f32x4{d * v[0] + l[0], d * v[1] + l[1], d * v[2] + l[2], d * v[3] + l[3]};
            *reinterpret_cast<f32x4*>(seg_init + (((int64_t)b * nseg + s + 1) * H + h) * PN + 4 * e4) = v;
        }
    }
}


}  // namespace ssd
