// ssd_api.hip -- host side of libssd.so: argument checks, workspace plan and the
// two kernel launches of the SSD forward (declarations and contract in ssd.h).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <cstdio>
#include <mutex>

#include "ssd.h"
#include "ssd_kernels.h"
#include "ssd_walk_split.h"
#include "ssd_walk_fused.h"
#include "ssd_walk_segments.h"
#include "ssd_backward.h"

namespace {

constexpr int kLdsMax = 160 * 1024;   // LDS per workgroup on gfx950
constexpr int kWalkThreads = 512;
constexpr int kComputeUnits = 256;     // MI355X: 8 XCDs x 32 CUs

typedef void (*walk_fn_t)(ssd::WalkArgs);

struct Plan {
    int dtype;
    int Q, Qp, nlb, ntile;
    int PT, NP, ptiles, qb, cb_lds;
    int64_t nslots, nitems;
    size_t cs_off, cb_off, bt_off, ct_off, ws_bytes;
    int lds_bytes, xs_off, xts_off, bs_off, hs_off, cs_lds_off;
    int split;        // the split-role walker (bf16, 256-row chunks, d_state 64 / 128)
    int nseg;         // segments per segmented sequence of a batch without seq_offsets
    int nsplit;       // summary parts per segment
    int64_t ntail;    // items walked in segments: the last ones
    int summary_lds;
    size_t seg_off, segd_off;
    int npass;        // d_state walked as npass passes of N / npass columns (1 or 2)
    size_t pass_ws, y2_off;   // workspace of one pass; the second pass's output
    walk_fn_t walk;   // the walk kernel instance for this plan
    walk_fn_t walk_left;   // the second pass of a two-pass d_state (left factors only)
    void (*walk_pair)(ssd::WalkArgs, ssd::WalkArgs);   // both passes in one launch
    walk_fn_t summary;   // the segment-summary instance (nseg > 1)
    int fused;        // compute waves per workgroup of the fused walker (0: not used)
    int fused_wpg;    // its workgroups per group
    int64_t fused_items;
    void (*fused_fn)(ssd::FusedArgs);
    void (*fused_pair_fn)(ssd::FusedArgs, ssd::FusedArgs, int);   // two walks of the shape in one launch
    int fseg, fseglen;   // the fused walker's segments per sequence (1: none) and their rows
    size_t loc_off, dsum_off, sinit_off;   // segment end states, log decays, entry states
    int sum_wpg;
    int64_t sum_items;
    void (*sum_fn)(ssd::SegSumArgs);
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int check_problem(const ssd_problem* p) {
    if (!p) return SSD_ERR_INVALID_ARG;
    if (p->batch < 1 || p->seqlen < 1 || p->nheads < 1 || p->headdim < 1 || p->dstate < 1 ||
        p->ngroups < 1 || p->chunk_len < 1 || p->reserved != 0)
        return SSD_ERR_INVALID_ARG;
    if (p->nheads % p->ngroups != 0) return SSD_ERR_INVALID_ARG;
    if (p->nseq < 1) return SSD_ERR_INVALID_ARG;
    // int32 indexing limits of the kernels (token rows, element offsets use int64)
    // (each factor is bounded before the product, which then cannot overflow)
    if (p->batch > (int64_t)1 << 30 || p->seqlen > (int64_t)1 << 30 || p->batch * p->seqlen > (int64_t)1 << 30 ||
        p->nheads > (1 << 20) || p->nseq > (1 << 24))
        return SSD_ERR_UNSUPPORTED;
    if (p->dtype != SSD_DTYPE_F32 && p->dtype != SSD_DTYPE_BF16) return SSD_ERR_UNSUPPORTED;
    const int64_t Q = p->chunk_len;
    if (Q != 16 && Q != 32 && Q != 64 && Q != 128 && Q != 256) return SSD_ERR_UNSUPPORTED;
    if (p->headdim % 16 != 0 || p->headdim > 256) return SSD_ERR_UNSUPPORTED;
    if (p->dstate % 16 != 0 || p->dstate > 256) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

// LDS of the walk kernel: X, X~ [Qp][PT+pad]; a region holding B rows [qb][NP+pad]
// during the state phase and, when cb_lds, the off-diagonal C B^T tiles of the chunk
// during the output phase; h [PT][NP+pad]; the chunk cumsum [Qp] floats.
int lds_layout(Plan* pl, int es) {
    const int pad = 16 / es;
    const int XS = pl->PT + pad, BS = pl->NP + pad, HS = pl->NP + pad;
    const int nlb = pl->Qp / 32;
    int region = pl->qb * BS * es;
    const int cb_bytes = nlb * (nlb - 1) / 2 * 1024 * es;
    if (pl->cb_lds && cb_bytes > region) region = cb_bytes;
    pl->xs_off = 0;
    pl->xts_off = pl->xs_off + pl->Qp * XS * es;
    pl->bs_off = pl->xts_off + pl->Qp * XS * es;
    pl->hs_off = pl->bs_off + region;
    pl->cs_lds_off = pl->hs_off + pl->PT * HS * es;
    pl->lds_bytes = pl->cs_lds_off + pl->Qp * 4;
    return pl->lds_bytes;
}

typedef void (*walk_fn)(ssd::WalkArgs);
typedef void (*prep_fn)(ssd::PrepArgs);

template <typename T, int PT, int NP, bool CBL>
walk_fn walk_instance() { return ssd::ssd_walk_kernel<T, PT, NP, CBL>; }

// float32: 32-wide P tiles, C B^T tiles read from global memory
walk_fn pick_walk_f32(int NP) {
    switch (NP) {
        case 32: return walk_instance<float, 32, 32, false>();
        case 64: return walk_instance<float, 32, 64, false>();
        case 128: return walk_instance<float, 32, 128, false>();
        case 256: return walk_instance<float, 32, 256, false>();
    }
    return nullptr;
}

template <int PT, bool CBL>
walk_fn pick_walk_bf16_np(int NP) {
    switch (NP) {
        case 32: return walk_instance<__bf16, PT, 32, CBL>();
        case 64: return walk_instance<__bf16, PT, 64, CBL>();
        case 128: return walk_instance<__bf16, PT, 128, CBL>();
        case 256: return walk_instance<__bf16, PT, 256, CBL>();
    }
    return nullptr;
}

walk_fn pick_walk_bf16(int PT, int NP, bool cbl) {
    if (PT == 32) return cbl ? pick_walk_bf16_np<32, true>(NP) : pick_walk_bf16_np<32, false>(NP);
    if (PT == 64) return cbl ? pick_walk_bf16_np<64, true>(NP) : pick_walk_bf16_np<64, false>(NP);
    return nullptr;
}

// Workspace and launch plan.  `nseq_total` slots: batch mode has batch * ceil(T/Q)
// chunks; a packed batch has at most ceil(T/Q) + nseq (one ragged chunk per sequence).
// The fused walker (ssd_walk_fused.h): bf16, head dimension a multiple of 32 from 64,
// d_state 64, 128 or 256, any chunk length (its 32-row blocks pass the state between them,
// so the chunking does not change the result).  NW compute waves per workgroup, each
// holding 32 columns of one head; it takes the NW that needs the fewest rounds of
// workgroups over the compute units times rows walked (a packed batch: the fewest
// workgroups), then leaves the fewest compute waves idle, then the larger NW.  Sequences
// of one length too few to fill the chip are walked in segments (ssd_walk_segments.h).  It
// is used when its workgroups, segments counted, fill at least half the chip (d_state
// 256: without segments).
typedef void (*fused_fn_t)(ssd::FusedArgs);
typedef void (*fused_pair_fn_t)(ssd::FusedArgs, ssd::FusedArgs, int);
// the two-walk launch, for the shapes of the backward pass's dB and dC passes (head dimension
// the layer's d_state, d_state the layer's head dimension: 64 or 128)
template <int NP, bool REV0, bool REV1>
fused_pair_fn_t fused_pair_instance(int nw) {
    switch (nw) {
        case 4: return ssd::ssd_walk_fused_pair_kernel<NP, 4, REV0, REV1>;
        case 5: return ssd::ssd_walk_fused_pair_kernel<NP, 5, REV0, REV1>;
    }
    return nullptr;
}
// a pair of walks of d_state NP: both forward, or the first reversed (the backward pass's dB
// pass) and the second forward (its dC pass)
fused_pair_fn_t fused_pair_for(int np, int nw, bool rev0) {
    if (np == 64) return rev0 ? fused_pair_instance<64, true, false>(nw) : fused_pair_instance<64, false, false>(nw);
    if (np == 128) return rev0 ? fused_pair_instance<128, true, false>(nw) : fused_pair_instance<128, false, false>(nw);
    return nullptr;
}
// the walker over reversed sequences (the backward pass's dX and dB passes)
fused_fn_t fused_rev_for(int np, int nw) {
    if (np == 64) return nw == 4 ? ssd::ssd_walk_fused_kernel<64, 4, true> : nw == 5 ? ssd::ssd_walk_fused_kernel<64, 5, true> : nullptr;
    if (np == 128) return nw == 4 ? ssd::ssd_walk_fused_kernel<128, 4, true> : nw == 5 ? ssd::ssd_walk_fused_kernel<128, 5, true> : nullptr;
    return nullptr;
}
template <int NP>
fused_fn_t fused_instance(int nw) {
    if constexpr (NP == 256) {
        // (the state of a d_state 256 column takes 128 registers a lane and the B and C rows
        // of a block 32 KB: two or three compute waves)
        switch (nw) {
            case 2: return ssd::ssd_walk_fused_kernel<256, 2>;
            case 3: return ssd::ssd_walk_fused_kernel<256, 3>;
        }
        return nullptr;
    } else {
        switch (nw) {
            case 4: return ssd::ssd_walk_fused_kernel<NP, 4>;
            case 5: return ssd::ssd_walk_fused_kernel<NP, 5>;
        }
        // (six compute waves only at d_state 64: the planner never takes them at 128)
        if constexpr (NP == 64)
            if (nw == 6) return ssd::ssd_walk_fused_kernel<64, 6>;
        return nullptr;
    }
}

bool plan_fused(const ssd_problem* p, Plan* pl) {
    pl->fused = 0;
    pl->fseg = 1;
    const int64_t P = p->headdim, N = p->dstate, H = p->nheads, G = p->ngroups, T = p->seqlen;
    if (p->dtype != SSD_DTYPE_BF16 || P % 32 != 0 || P < 64 || (N != 64 && N != 128 && N != 256)) return false;
    // 32-bit byte offsets inside one sequence's rows of X / Y, B / C and logA
    if (p->batch * p->seqlen * H * P * 2 >= ((int64_t)1 << 31) ||
        p->batch * p->seqlen * G * N * 2 >= ((int64_t)1 << 31))
        return false;
    const int64_t upg = (H / G) * (P / 32);
    const bool packed = p->nseq != p->batch;
    // Sequences of one length (a batch, or one packed sequence) whose workgroups would not
    // fill the chip are walked as segments (ssd_walk_segments.h): as many as bring the
    // workgroups to one per compute unit, of at least 8 blocks (256 rows) each.
    auto segments = [&](int64_t items, int* nseg, int* seglen) {
        *nseg = 1;
        *seglen = (int)T;
        if (packed || items >= kComputeUnits) return;
        int64_t k = kComputeUnits / items;
        if (k > T / 256) k = T / 256;
        if (k < 2) return;
        const int64_t sl = ((T + k - 1) / k + 31) / 32 * 32;
        *nseg = (int)((T + sl - 1) / sl);
        *seglen = (int)sl;
    };
    int best = 0, best_seg = 1, best_sl = 0;
    int64_t best_cost = 0, best_waste = 0, best_items = 0, best_wpg = 0;
    // (d_state 128 with six compute waves keeps only two blocks in flight: too few to
    // cover the latency of memory when the inputs are not in the last-level cache)
    const int nw_hi = N == 256 ? 3 : N == 128 ? 5 : 6, nw_lo = N == 256 ? 2 : 4;
    for (int nw = nw_hi; nw >= nw_lo; --nw) {
        const int64_t wpg = (upg + nw - 1) / nw;
        const int64_t items = p->nseq * G * wpg;
        int nseg, sl;
        segments(items, &nseg, &sl);
        const int64_t eff = items * nseg;
        // rounds of workgroups over the compute units times the rows each walks (a packed
        // batch: the workgroups)
        const int64_t cost = packed ? items : (eff + kComputeUnits - 1) / kComputeUnits * sl;
        const int64_t waste = items * nw - p->nseq * G * upg;
        if (!best || cost < best_cost || (cost == best_cost && waste < best_waste)) {
            best = nw;
            best_cost = cost;
            best_waste = waste;
            best_items = eff;
            best_wpg = wpg;
            best_seg = nseg;
            best_sl = sl;
        }
    }
    if (best_items < kComputeUnits / 2 || best_items > INT32_MAX / 8) return false;
    // d_state 256 only where the workgroups fill the chip without segments: its summary
    // plus the walk of the segments takes longer than the two passes over the column
    // halves of the state (ssd_walk_split_pair_kernel and the add)
    if (N == 256 && best_seg > 1) return false;
    pl->fused = best;
    pl->fused_wpg = (int)best_wpg;
    pl->fused_items = best_items;
    pl->fused_fn = N == 64 ? fused_instance<64>(best) : N == 128 ? fused_instance<128>(best) : fused_instance<256>(best);
    pl->fused_pair_fn = fused_pair_for((int)N, best, false);
    pl->fseg = best_seg;
    pl->fseglen = best_sl;
    size_t ws = 256;
    if (best_seg > 1) {
        const size_t state = (size_t)(H * P * N) * sizeof(float);
        pl->loc_off = 0;
        pl->dsum_off = align_up((size_t)p->nseq * (best_seg - 1) * state, 256);
        pl->sinit_off = align_up(pl->dsum_off + (size_t)p->nseq * (best_seg - 1) * H * sizeof(float), 256);
        ws = align_up(pl->sinit_off + (size_t)p->nseq * best_seg * state, 256);
        pl->sum_wpg = (int)((upg + ssd::kSumUnits - 1) / ssd::kSumUnits);
        pl->sum_items = p->nseq * (best_seg - 1) * G * pl->sum_wpg;
        pl->sum_fn = N == 64 ? ssd::ssd_seg_summary_kernel<64> : ssd::ssd_seg_summary_kernel<128>;
        if (pl->sum_items > INT32_MAX) return false;
    }
    pl->ws_bytes = ws;
    return pl->fused_fn != nullptr;
}

int make_plan(const ssd_problem* p, Plan* pl, bool allow_fused = true) {
    const int rc = check_problem(p);
    if (rc != SSD_OK) return rc;
    pl->dtype = p->dtype;
    pl->fused = 0;
    if (allow_fused && plan_fused(p, pl)) {
        pl->npass = 1;
        pl->nseg = 1;
        return SSD_OK;
    }
    pl->summary = nullptr;
    pl->walk_left = nullptr;
    pl->walk_pair = nullptr;
    pl->npass = 1;
    // d_state 256 on the layer-shape walker: the layer is linear in C B^T and its state
    // splits by columns, so it is the sum of two d_state-128 problems on the column
    // halves of B, C and the state (init and final state each take their half).  Each
    // half gets its own workspace; the second writes its output to the workspace and a
    // last kernel adds it to Y.
    if (p->dtype == SSD_DTYPE_BF16 && p->chunk_len == 256 && p->dstate == 256 && p->headdim % 64 == 0) {
        ssd_problem q = *p;
        q.dstate = 128;
        const int qrc = make_plan(&q, pl, false);   // (the split walker's plan for each half)
        if (qrc != SSD_OK) return qrc;
        pl->npass = 2;
        pl->walk_left = ssd::ssd_walk_split_kernel<128, false, true>;
        pl->walk_pair = ssd::ssd_walk_split_pair_kernel<128>;
        // both passes side by side fill twice the compute units: segment only if even
        // that leaves a partial last round
        {
            const int64_t items2 = 2 * p->nseq * p->nheads * (p->headdim / 64);
            const int64_t tail2 = items2 % kComputeUnits;
            if (tail2 == 0 || items2 >= kComputeUnits) {
                pl->nseg = 1;
                pl->nsplit = 1;
                pl->ntail = 0;
            }
        }
        pl->pass_ws = pl->ws_bytes;
        pl->y2_off = 2 * pl->pass_ws;
        pl->ws_bytes = align_up(pl->y2_off + (size_t)(p->batch * p->seqlen * p->nheads * p->headdim) * 2, 256);
        return SSD_OK;
    }
    const int es = p->dtype == SSD_DTYPE_BF16 ? 2 : 4;
    pl->Q = (int)p->chunk_len;
    pl->Qp = (pl->Q + 31) / 32 * 32;
    pl->nlb = pl->Qp / 32;
    pl->ntile = pl->nlb * (pl->nlb + 1) / 2;
    const int N = (int)p->dstate, P = (int)p->headdim;
    pl->NP = N <= 32 ? 32 : N <= 64 ? 64 : N <= 128 ? 128 : 256;
    // 64-wide P tiles when there are enough (sequence, head) items to fill the chip
    pl->PT = (p->dtype == SSD_DTYPE_BF16 && P > 32 && p->nseq * p->nheads * ((P + 63) / 64) >= 512) ? 64 : 32;
    pl->ptiles = (P + pl->PT - 1) / pl->PT;
    const int64_t nc = (p->seqlen + pl->Q - 1) / pl->Q;
    // slots are sized for the larger of the two numberings, so one plan serves
    // a call with or without seq_offsets
    const int64_t slots_batch = p->batch * nc;
    const int64_t slots_packed = nc + p->nseq;
    pl->nslots = slots_batch > slots_packed ? slots_batch : slots_packed;
    pl->nitems = p->nseq * p->nheads * pl->ptiles;
    if (pl->nitems > ((int64_t)1 << 31) - 1) return SSD_ERR_UNSUPPORTED;
    pl->cs_off = 0;
    const size_t cs_bytes = (size_t)pl->nslots * p->nheads * pl->Qp * sizeof(float);
    pl->cb_off = align_up(pl->cs_off + cs_bytes, 256);
    const size_t cb_bytes = (size_t)pl->nslots * p->ngroups * pl->ntile * 1024 * es;
    pl->bt_off = align_up(pl->cb_off + cb_bytes, 256);
    // the common layer shapes take the split-role walker (64-wide P tiles, whole
    // chunks), which also needs B^T of every chunk in fragment order
    pl->split = p->dtype == SSD_DTYPE_BF16 && pl->Q == 256 && (N == 64 || N == 128) && P % 64 == 0;
    const size_t bt_bytes = pl->split ? (size_t)pl->nslots * p->ngroups * ssd::split_bt_bytes(N) : 0;
    pl->ct_off = align_up(pl->bt_off + bt_bytes, 256);
    pl->seg_off = align_up(pl->ct_off + bt_bytes, 256);   // C fragments: as many bytes as B^T
    // Segmented walk: the (sequence, head, P tile) items of a batch run one workgroup per
    // CU.  The items of the last round, when they are too few to fill the 256 compute
    // units of the part (all items, for a small batch), are walked as nseg segments of
    // at least 8 chunks each, after a pass that sums up every segment but the last in
    // parts of at least 2 chunks, about two summary workgroups per compute unit.  (A
    // summary part costs about half a walked chunk and its first loads are exposed, so
    // segments shorter than 8 chunks do not pay back.)
    pl->nseg = 1;
    pl->nsplit = 1;
    pl->ntail = 0;
    if (pl->split) {
        const int64_t items = p->nseq * p->nheads * (P / 64);
        const int64_t tail = items % kComputeUnits;
        int64_t k = tail > 0 ? kComputeUnits / tail : 1;
        if (k > nc / 8) k = nc / 8;
        if (k > 1) {
            pl->nseg = (int)k;
            pl->ntail = tail;
            int64_t m = 2 * kComputeUnits / (tail * (k - 1));
            if (m > nc / k / 2) m = nc / k / 2;
            pl->nsplit = m > 1 ? (int)m : 1;
        }
    }
    const size_t nparts = (size_t)p->nseq * (pl->nseg - 1) * pl->nsplit * p->nheads;
    pl->segd_off = align_up(pl->seg_off + nparts * P * N * sizeof(float), 256);
    pl->ws_bytes = align_up(pl->segd_off + nparts * sizeof(float), 256);
    // stage the off-diagonal C B^T tiles in LDS when they fit next to a whole chunk of B
    // (or the largest B stage that fits), else read them from global memory
    pl->cb_lds = p->dtype == SSD_DTYPE_BF16 ? 1 : 0;
    pl->qb = pl->Qp;
    while (lds_layout(pl, es) > kLdsMax && pl->qb > 32) pl->qb -= 32;
    if (pl->lds_bytes > kLdsMax) {
        pl->cb_lds = 0;
        pl->qb = pl->Qp;
        while (lds_layout(pl, es) > kLdsMax && pl->qb > 32) pl->qb -= 32;
    }
    if (pl->lds_bytes > kLdsMax) return SSD_ERR_UNSUPPORTED;
    pl->walk = p->dtype == SSD_DTYPE_BF16 ? pick_walk_bf16(pl->PT, pl->NP, pl->cb_lds != 0)
                                          : (pl->cb_lds ? nullptr : pick_walk_f32(pl->NP));
    if (!pl->walk) return SSD_ERR_UNSUPPORTED;
    if (pl->split) {
        pl->PT = 64;
        pl->ptiles = P / 64;
        pl->nitems = p->nseq * p->nheads * pl->ptiles;
        pl->qb = pl->Qp;
        pl->cb_lds = 0;
        if (N == 64) {
            pl->walk = ssd::ssd_walk_split_kernel<64, false>;
            pl->summary = ssd::ssd_walk_split_kernel<64, true>;
            pl->lds_bytes = ssd::SplitLds<64>::bytes;
            pl->summary_lds = ssd::SummaryLds<64>::bytes;
        } else {
            pl->walk = ssd::ssd_walk_split_kernel<128, false>;
            pl->summary = ssd::ssd_walk_split_kernel<128, true>;
            pl->lds_bytes = ssd::SplitLds<128>::bytes;
            pl->summary_lds = ssd::SummaryLds<128>::bytes;
        }
    }
    return SSD_OK;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

// Raise the dynamic-LDS limit of a walk kernel to the full 160 KiB, once per kernel
// per process (setting it twice is harmless, so a race only repeats the call).
int ensure_lds_limit(const void* fn) {
    static std::atomic<const void*> done[32] = {};
    for (auto& d : done)
        if (d.load(std::memory_order_acquire) == fn) return SSD_OK;
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax) != hipSuccess)
        return SSD_ERR_HIP;
    for (auto& d : done) {
        const void* expected = nullptr;
        if (d.compare_exchange_strong(expected, fn, std::memory_order_acq_rel)) break;
        if (expected == fn) break;
    }
    return SSD_OK;
}

}  // namespace

extern "C" {

int ssd_abi_version(void) { return SSD_ABI_VERSION; }

const char* ssd_status_string(int status) {
    switch (status) {
        case SSD_OK: return "ok";
        case SSD_ERR_INVALID_ARG: return "invalid argument";
        case SSD_ERR_UNSUPPORTED: return "unsupported problem (dtype, chunk_len, headdim or dstate)";
        case SSD_ERR_WORKSPACE: return "workspace too small";
        case SSD_ERR_HIP: return "HIP runtime error";
        case SSD_ERR_TOO_LARGE: return "problem needs more scratch than the no-allocation entry point holds";
        default: return "unknown status";
    }
}

int ssd_check_problem(const ssd_problem* p) {
    if (!p) return SSD_ERR_INVALID_ARG;
    Plan pl;
    return make_plan(p, &pl);
}

int ssd_plan_describe(const ssd_problem* p, char* buf, size_t len) {
    if (!buf || len == 0) return SSD_ERR_INVALID_ARG;
    buf[0] = 0;
    if (!p) return SSD_ERR_INVALID_ARG;
    Plan pl;
    const int rc = make_plan(p, &pl);
    if (rc != SSD_OK) return rc;
    char walk[96];
    const char* prep = p->dtype == SSD_DTYPE_BF16 ? "ssd_prep_kernel<bf16>" : "ssd_prep_kernel<float>";
    const char* summary = "none";
    if (pl.fused) {
        snprintf(walk, sizeof walk, "ssd_walk_fused_kernel<%d, %d>", (int)p->dstate, pl.fused);
        prep = "none";
        if (pl.fseg > 2 + ssd::kScanSeg)
            summary = p->dstate == 64 ? "ssd_seg_summary_kernel<64>+ssd_seg_scan_kernel"
                                      : "ssd_seg_summary_kernel<128>+ssd_seg_scan_kernel";
        else if (pl.fseg > 2)
            summary = p->dstate == 64 ? "ssd_seg_summary_kernel<64>+ssd_seg_chain_kernel"
                                      : "ssd_seg_summary_kernel<128>+ssd_seg_chain_kernel";
        else if (pl.fseg == 2)
            summary = p->dstate == 64 ? "ssd_seg_summary_kernel<64>" : "ssd_seg_summary_kernel<128>";
    } else if (pl.npass == 2) {
        snprintf(walk, sizeof walk, "ssd_walk_split_pair_kernel<128>+ssd_add_kernel<bf16>");
    } else if (pl.split) {
        snprintf(walk, sizeof walk, "ssd_walk_split_kernel<%d, false, false>", (int)p->dstate);
        if (pl.nseg > 1) summary = p->dstate == 64 ? "ssd_walk_split_kernel<64, true, false>"
                                                    : "ssd_walk_split_kernel<128, true, false>";
    } else {
        // the general walker: element type, P tile, padded d_state, C B^T tiles in LDS, and
        // the rows of B staged at once (fewer than the padded chunk: B goes in stages)
        snprintf(walk, sizeof walk, "ssd_walk_kernel<%s, %d, %d, %s> qb=%d/%d",
                 p->dtype == SSD_DTYPE_BF16 ? "bf16" : "float", pl.PT, pl.NP, pl.cb_lds ? "true" : "false", pl.qb,
                 pl.Qp);
    }
    snprintf(buf, len, "walk=%s;prep=%s;summary=%s", walk, prep, summary);
    return SSD_OK;
}

size_t ssd_workspace_bytes(const ssd_problem* p) {
    Plan pl;
    if (make_plan(p, &pl) != SSD_OK) return 0;
    return pl.ws_bytes;
}

}  // extern "C"

namespace {

// stages: bit 0 = prep launch, bit 1 = walk launch.  x_heads: X rows per token (the
// heads share them in contiguous runs of H / x_heads); 0 means one per head.
// A fused walk prepared but not launched, for the caller to launch with another (the
// backward pass's dB and dC passes); captured = false when the plan was launched as usual.
struct FusedCapture {
    bool captured;
    ssd::FusedArgs a;
    int64_t grid;
    int nw;
    int np;           // d_state
    bool rev;         // the walk over reversed sequences
    fused_fn_t fn;
};

int run_forward(int stages, const ssd_problem* p, const void* X, const float* logA, const void* B,
                const void* C, const float* init_state, const int32_t* seq_offsets, void* Y,
                float* final_state, void* workspace, size_t workspace_bytes, void* hip_stream,
                int64_t x_heads = 0, FusedCapture* cap = nullptr, bool reversed = false) {
    if (cap) cap->captured = false;
    Plan pl;
    int rc = make_plan(p, &pl);
    if (rc != SSD_OK) return rc;
    if (reversed && (!pl.fused || pl.fseg > 1 || !fused_rev_for((int)p->dstate, pl.fused))) return SSD_ERR_UNSUPPORTED;
    if (!X || !logA || !B || !C || !Y || !workspace) return SSD_ERR_INVALID_ARG;
    if (seq_offsets) {
        if (p->batch != 1) return SSD_ERR_INVALID_ARG;
    } else if (p->nseq != p->batch) {
        return SSD_ERR_INVALID_ARG;
    }
    const void* ptrs[] = {X, logA, B, C, init_state, seq_offsets, Y, final_state};
    for (const void* q : ptrs)
        if (q && !aligned16(q)) return SSD_ERR_INVALID_ARG;
    if (((uintptr_t)workspace & 255u) != 0) return SSD_ERR_INVALID_ARG;
    const size_t es = p->dtype == SSD_DTYPE_BF16 ? 2 : 4;
    const int64_t b = p->batch, T = p->seqlen, H = p->nheads, P = p->headdim, N = p->dstate,
                  G = p->ngroups;
    if (x_heads == 0) x_heads = H;
    if (x_heads < 1 || H % x_heads != 0) return SSD_ERR_INVALID_ARG;
    const size_t nx = (size_t)(b * T * H * P) * es, nxin = (size_t)(b * T * x_heads * P) * es;
    const size_t na = (size_t)(b * T * H) * sizeof(float);
    const size_t nbc = (size_t)(b * T * G * N) * es;
    const size_t ns = (size_t)(p->nseq * H * P * N) * sizeof(float);
    const size_t no = seq_offsets ? (size_t)(p->nseq + 1) * sizeof(int32_t) : 0;
    // outputs must not overlap inputs, each other or the workspace
    const void* ins[] = {X, logA, B, C, init_state, seq_offsets, workspace};
    const size_t nin[] = {nxin, na, nbc, nbc, init_state ? ns : 0, no, workspace_bytes};
    for (int i = 0; i < 7; ++i) {
        if (overlap(Y, nx, ins[i], nin[i])) return SSD_ERR_INVALID_ARG;
        if (final_state && overlap(final_state, ns, ins[i], nin[i])) return SSD_ERR_INVALID_ARG;
    }
    if (final_state && overlap(Y, nx, final_state, ns)) return SSD_ERR_INVALID_ARG;
    // the workspace is written too (by the prep, read back by the walk): it overlaps no input
    for (int i = 0; i < 6; ++i)
        if (overlap(workspace, workspace_bytes, ins[i], nin[i])) return SSD_ERR_INVALID_ARG;
    if (workspace_bytes < pl.ws_bytes) return SSD_ERR_WORKSPACE;

    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (pl.fused) {
        // one launch and no workspace; sequences walked as segments: stage 1 is the
        // segments' summary and their entry states, stage 2 the walk
        const bool seg = pl.fseg > 1;
        unsigned char* ws = static_cast<unsigned char*>(workspace);
        float* sinit = reinterpret_cast<float*>(ws + pl.sinit_off);
        if (seg && (stages & 1)) {
            ssd::SegSumArgs sa;
            sa.X = static_cast<const __bf16*>(X);
            sa.logA = logA;
            sa.B = static_cast<const __bf16*>(B);
            sa.init = init_state;
            sa.loc = reinterpret_cast<float*>(ws + pl.loc_off);
            sa.dsum = reinterpret_cast<float*>(ws + pl.dsum_off);
            sa.sinit = sinit;
            sa.T = T;
            sa.seglen = pl.fseglen;
            sa.nseg = pl.fseg;
            sa.nseq = (int)p->nseq;
            sa.H = (int)H;
            sa.P = (int)P;
            sa.G = (int)G;
            sa.xh = (int)x_heads;
            sa.upg = (int)((H / G) * (P / 32));
            sa.wpg = pl.sum_wpg;
            sa.nitems = (int)pl.sum_items;
            hipLaunchKernelGGL(pl.sum_fn, dim3((unsigned)pl.sum_items), dim3(ssd::kSumThreads), 0, stream, sa);
            if (pl.fseg > 2) {
                // one workgroup per (256 state elements, head, sequence); P N is a multiple of
                // 256 on this path (P a multiple of 32, N 64 or 128), and a segmented plan has
                // fewer workgroups than compute units, so fewer sequences and heads than the
                // grid's y and z limits
                if (pl.fseg - 2 > ssd::kScanSeg) {
                    hipLaunchKernelGGL(ssd::ssd_seg_scan_kernel, dim3((unsigned)(P * N / 256), (unsigned)H, (unsigned)p->nseq),
                                       dim3(64 * ssd::kScanSeg), 0, stream, static_cast<const float*>(sa.loc),
                                       static_cast<const float*>(sa.dsum), sinit, (int)p->nseq, pl.fseg, (int)H,
                                       (int)(P * N));
                } else {
                    const int64_t n4 = p->nseq * H * P * N / 4;
                    const int64_t cblocks = (n4 + 255) / 256 < 8192 ? (n4 + 255) / 256 : 8192;
                    hipLaunchKernelGGL(ssd::ssd_seg_chain_kernel, dim3((unsigned)cblocks), dim3(256), 0, stream,
                                       static_cast<const float*>(sa.loc), static_cast<const float*>(sa.dsum), sinit,
                                       (int)p->nseq, pl.fseg, (int)H, (int)(P * N));
                }
            }
        }
        if (!(stages & 2)) return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
        ssd::FusedArgs fa;
        fa.X = static_cast<const __bf16*>(X);
        fa.logA = logA;
        fa.B = static_cast<const __bf16*>(B);
        fa.C = static_cast<const __bf16*>(C);
        fa.init = seg ? sinit : init_state;
        fa.init0 = init_state;
        // (a segmented plan has sequences of one length: a batch, or one packed sequence
        // that spans the rows)
        fa.seq_offsets = seg ? nullptr : seq_offsets;
        fa.Y = static_cast<__bf16*>(Y);
        fa.final_state = final_state;
        fa.T = T;
        fa.H = (int)H;
        fa.P = (int)P;
        fa.N = (int)N;
        fa.G = (int)G;
        fa.xh = (int)x_heads;
        fa.nseq = (int)(p->nseq * pl.fseg);
        fa.upg = (int)((H / G) * (P / 32));
        fa.wpg = pl.fused_wpg;
        fa.nitems = (int)pl.fused_items;
        fa.nseg = pl.fseg;
        fa.seglen = pl.fseglen;
        // packed sequences: (sequence, group) units dealt to the XCDs longest first
        fa.lpt = (!seg && seq_offsets && p->nseq <= 64) ? 1 : 0;
        int64_t grid = pl.fused_items;
        if (fa.lpt) grid = ((p->nseq * G + 7) / 8) * 8 * pl.fused_wpg;
        // (reversed sequences: the backward pass's own form, only for plans without segments)
        const fused_fn_t fn = reversed ? fused_rev_for((int)N, pl.fused) : pl.fused_fn;
        if (!fn || (reversed && seg)) return SSD_ERR_UNSUPPORTED;
        if (cap && !seg && pl.fused_pair_fn) {
            cap->captured = true;
            cap->a = fa;
            cap->grid = grid;
            cap->nw = pl.fused;
            cap->np = (int)N;
            cap->rev = reversed;
            cap->fn = fn;
            return SSD_OK;
        }
        hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(64 * (pl.fused + 3)), 0, stream, fa);
        return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
    }
    walk_fn walk = pl.walk;
    prep_fn prep = p->dtype == SSD_DTYPE_BF16 ? ssd::ssd_prep_kernel<__bf16>
                                              : ssd::ssd_prep_kernel<float>;
    rc = ensure_lds_limit(reinterpret_cast<const void*>(walk));
    if (rc != SSD_OK) return rc;
    if (pl.npass == 2) {
        rc = ensure_lds_limit(reinterpret_cast<const void*>(pl.walk_left));
        if (rc == SSD_OK) rc = ensure_lds_limit(reinterpret_cast<const void*>(pl.walk_pair));
        if (rc != SSD_OK) return rc;
    }
    // packed sequences are walked whole
    const int nseg = seq_offsets ? 1 : pl.nseg;
    if (nseg > 1) {
        rc = ensure_lds_limit(reinterpret_cast<const void*>(pl.summary));
        if (rc != SSD_OK) return rc;
    }

    // slots actually addressed by this call
    const int64_t nc = (T + pl.Q - 1) / pl.Q;
    const int64_t nslots = seq_offsets ? nc + p->nseq : b * nc;
    const int64_t NPASS = N / pl.npass;   // state columns of one pass
    auto pass_args = [&](int k, ssd::PrepArgs* ppa, ssd::WalkArgs* pwa) {
        unsigned char* ws = static_cast<unsigned char*>(workspace) + k * pl.pass_ws;
        // the cumsum of logA is the same for both passes: the first pass's serves both
        float* cs = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + pl.cs_off);
        void* cb = ws + pl.cb_off;
        ssd::PrepArgs& pa = *ppa;
        pa.logA = logA;
        pa.B = B;
        pa.C = C;
        pa.seq_offsets = seq_offsets;
        pa.cs = cs;
        pa.cb = cb;
        pa.T = T;
        pa.H = (int)H;
        pa.N = (int)NPASS;
        pa.G = (int)G;
        pa.Q = pl.Q;
        pa.Qp = pl.Qp;
        pa.ntile = pl.ntile;
        pa.nseq = (int)p->nseq;
        pa.hblocks = (int)((H + ssd::kPrepHeads - 1) / ssd::kPrepHeads);
        pa.cs_blocks = (int)(nslots * pa.hblocks);
        pa.cb_blocks = (int)(nslots * G);
        pa.bt = pl.split ? ws + pl.bt_off : nullptr;
        pa.ct = pl.split ? ws + pl.ct_off : nullptr;
        pa.ldn = (int)N;
        pa.n0 = (int)(k * NPASS);
        // the first pass's tiles contract all columns (its walk adds the whole
        // within-chunk part); the second pass only needs its fragment copies
        pa.cb_n = k == 0 ? (int)N : 0;
        // one prep serves both passes: it walks every column for the tiles anyway
        pa.bt2 = (pl.npass == 2 && k == 0) ? static_cast<unsigned char*>(workspace) + pl.pass_ws + pl.bt_off : nullptr;
        pa.ct2 = (pl.npass == 2 && k == 0) ? static_cast<unsigned char*>(workspace) + pl.pass_ws + pl.ct_off : nullptr;

        ssd::WalkArgs& wa = *pwa;
        wa.X = X;
        wa.B = B;
        wa.C = C;
        wa.init = init_state;
        wa.seq_offsets = seq_offsets;
        wa.Y = k == 0 ? Y : static_cast<unsigned char*>(workspace) + pl.y2_off;
        wa.final_state = final_state;
        wa.cs = cs;
        wa.cb = cb;
        wa.bt = ws + pl.bt_off;
        wa.ct = ws + pl.ct_off;
        wa.T = T;
        wa.H = (int)H;
        wa.P = (int)P;
        wa.N = (int)NPASS;
        wa.G = (int)G;
        wa.Q = pl.Q;
        wa.Qp = pl.Qp;
        wa.ntile = pl.ntile;
        wa.nseq = (int)p->nseq;
        wa.ptiles = pl.ptiles;
        wa.nitems = (int)pl.nitems;
        wa.qb = pl.qb;
        wa.cb_lds = pl.cb_lds;
        wa.xs_off = pl.xs_off;
        wa.xts_off = pl.xts_off;
        wa.bs_off = pl.bs_off;
        wa.hs_off = pl.hs_off;
        wa.cs_off = pl.cs_lds_off;
        wa.xh = (int)x_heads;
        wa.ldn = (int)N;
        wa.ns0 = (int)(k * NPASS);
        wa.nseg = nseg;
        wa.nsplit = pl.nsplit;
        wa.ntail = nseg > 1 ? (int)pl.ntail : 0;
        wa.nwhole = (int)(pl.nitems - wa.ntail);
        wa.lpt = (pl.split && seq_offsets && p->nseq <= 64 && (p->nseq * G) % 8 == 0) ? 1 : 0;
        wa.seg_state = reinterpret_cast<float*>(ws + pl.seg_off);
        wa.seg_decay = reinterpret_cast<float*>(ws + pl.segd_off);
    };
    const int64_t prep_blocks = nslots * ((H + ssd::kPrepHeads - 1) / ssd::kPrepHeads) + nslots * G;
    if (prep_blocks > INT32_MAX) return SSD_ERR_UNSUPPORTED;
    ssd::PrepArgs pa;
    ssd::WalkArgs wa;
    if (stages & 1) {
        pass_args(0, &pa, &wa);
        hipLaunchKernelGGL(prep, dim3((unsigned)prep_blocks), dim3(ssd::kPrepThreads), 0, stream, pa);
    }
    if ((stages & 2) && pl.npass == 2 && nseg == 1) {
        // both column halves in one launch
        ssd::WalkArgs wb;
        pass_args(0, &pa, &wa);
        pass_args(1, &pa, &wb);
        wa.nitems = wa.nwhole;
        wb.nitems = wb.nwhole;
        hipLaunchKernelGGL(pl.walk_pair, dim3((unsigned)(wa.nitems + wb.nitems)), dim3(kWalkThreads), pl.lds_bytes,
                           stream, wa, wb);
    } else if (stages & 2) {
        for (int k = 0; k < pl.npass; ++k) {
            pass_args(k, &pa, &wa);
            if (nseg > 1) {
                wa.nitems = wa.ntail * (nseg - 1) * pl.nsplit;
                hipLaunchKernelGGL(pl.summary, dim3((unsigned)wa.nitems), dim3(kWalkThreads / 2), pl.summary_lds,
                                   stream, wa);
            }
            wa.nitems = wa.nwhole + wa.ntail * nseg;
            hipLaunchKernelGGL(k == 0 ? walk : pl.walk_left, dim3((unsigned)wa.nitems), dim3(kWalkThreads),
                               pl.lds_bytes, stream, wa);
        }
    }
    if ((stages & 2) && pl.npass == 2) {
        const int64_t n8 = b * T * H * P / 8;
        const int64_t blocks = (n8 + 255) / 256 < 16384 ? (n8 + 255) / 256 : 16384;
        hipLaunchKernelGGL(ssd::ssd_add_kernel<__bf16>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           static_cast<__bf16*>(Y),
                           reinterpret_cast<const __bf16*>(static_cast<unsigned char*>(workspace) + pl.y2_off), n8);
    }
    if (hipGetLastError() != hipSuccess) return SSD_ERR_HIP;
    return SSD_OK;
}

}  // namespace

extern "C" {

int ssd_forward(const ssd_problem* p, const void* X, const float* logA, const void* B,
                const void* C, const float* init_state, const int32_t* seq_offsets, void* Y,
                float* final_state, void* workspace, size_t workspace_bytes, void* hip_stream) {
    return run_forward(3, p, X, logA, B, C, init_state, seq_offsets, Y, final_state, workspace,
                       workspace_bytes, hip_stream);
}

}  // extern "C"

namespace {

// The scratch of ssd_forward_noalloc: one array per device, loaded with the code object.
// In host code its name is a host-side stand-in; only the address that
// hipGetSymbolAddress returns on a device is a device address.
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_addr[kMaxDevices] = {};

// the current device's scratch address, looked up on the first call on that device
int scratch_for_current_device(hipStream_t stream, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return SSD_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return SSD_ERR_UNSUPPORTED;
    if (stream) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return SSD_ERR_HIP;
        if (sdev != dev) return SSD_ERR_INVALID_ARG;
    }
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_addr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SSD_ERR_HIP;
        scratch_addr[dev] = ptr;
    }
    *out = scratch_addr[dev];
    return SSD_OK;
}

}  // namespace

extern "C" {

int ssd_forward_noalloc(const ssd_problem* p, const void* X, const float* logA, const void* B,
                        const void* C, const float* init_state, const int32_t* seq_offsets,
                        void* Y, float* final_state, void* hip_stream) {
    Plan pl;
    const int rc = make_plan(p, &pl);
    if (rc != SSD_OK) return rc;
    if (pl.ws_bytes > SSD_NOALLOC_SCRATCH_BYTES) return SSD_ERR_TOO_LARGE;
    void* ws = nullptr;
    const int src = scratch_for_current_device(static_cast<hipStream_t>(hip_stream), &ws);
    if (src != SSD_OK) return src;
    return run_forward(3, p, X, logA, B, C, init_state, seq_offsets, Y, final_state, ws,
                       SSD_NOALLOC_SCRATCH_BYTES, hip_stream);
}

int ssd_decode_step(const ssd_problem* p, const void* x, const float* logA, const void* B,
                    const void* C, float* state, void* y, void* hip_stream) {
    if (!p) return SSD_ERR_INVALID_ARG;
    if (p->batch < 1 || p->seqlen != 1 || p->nheads < 1 || p->headdim < 1 || p->dstate < 1 ||
        p->ngroups < 1 || p->nseq != p->batch || p->reserved != 0)
        return SSD_ERR_INVALID_ARG;
    if (p->nheads % p->ngroups != 0) return SSD_ERR_INVALID_ARG;
    if (p->dtype != SSD_DTYPE_F32 && p->dtype != SSD_DTYPE_BF16) return SSD_ERR_UNSUPPORTED;
    if (p->headdim % 16 != 0 || p->headdim > 256 || p->dstate % 16 != 0 || p->dstate > 256)
        return SSD_ERR_UNSUPPORTED;
    // (each factor is bounded before the product, which then cannot overflow)
    if (p->batch > INT32_MAX || p->nheads > INT32_MAX || p->batch * p->nheads > INT32_MAX) return SSD_ERR_UNSUPPORTED;
    if (!x || !logA || !B || !C || !state || !y) return SSD_ERR_INVALID_ARG;
    const void* ptrs[] = {x, logA, B, C, state, y};
    for (const void* q : ptrs)
        if (!aligned16(q)) return SSD_ERR_INVALID_ARG;
    const size_t es = p->dtype == SSD_DTYPE_BF16 ? 2 : 4;
    const int64_t b = p->batch, H = p->nheads, P = p->headdim, N = p->dstate, G = p->ngroups;
    const size_t nx = (size_t)(b * H * P) * es, na = (size_t)(b * H) * 4, nbc = (size_t)(b * G * N) * es;
    const size_t ns = (size_t)(b * H * P * N) * 4;
    // y and the state are written: neither may overlap an input or the other
    const void* ins[] = {x, logA, B, C};
    const size_t nin[] = {nx, na, nbc, nbc};
    for (int i = 0; i < 4; ++i)
        if (overlap(y, nx, ins[i], nin[i]) || overlap(state, ns, ins[i], nin[i])) return SSD_ERR_INVALID_ARG;
    if (overlap(y, nx, state, ns)) return SSD_ERR_INVALID_ARG;
    ssd::DecodeArgs da;
    da.x = x;
    da.logA = logA;
    da.B = B;
    da.C = C;
    da.state = state;
    da.y = y;
    da.H = (int)H;
    da.P = (int)P;
    da.N = (int)N;
    da.G = (int)G;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (p->dtype == SSD_DTYPE_BF16)
        hipLaunchKernelGGL(ssd::ssd_decode_kernel<__bf16>, dim3((unsigned)(b * H)), dim3(256), 0, stream, da);
    else
        hipLaunchKernelGGL(ssd::ssd_decode_kernel<float>, dim3((unsigned)(b * H)), dim3(256), 0, stream, da);
    if (hipGetLastError() != hipSuccess) return SSD_ERR_HIP;
    return SSD_OK;
}

int ssd_forward_stage(int stage, const ssd_problem* p, const void* X, const float* logA,
                      const void* B, const void* C, const float* init_state,
                      const int32_t* seq_offsets, void* Y, float* final_state, void* workspace,
                      size_t workspace_bytes, void* hip_stream) {
    if (stage != 1 && stage != 2) return SSD_ERR_INVALID_ARG;
    return run_forward(stage, p, X, logA, B, C, init_state, seq_offsets, Y, final_state, workspace,
                       workspace_bytes, hip_stream);
}

}  // extern "C"

// The backward pass: its plan and entry points (forward passes on re-arranged operands).
#include "ssd_backward_api.h"
