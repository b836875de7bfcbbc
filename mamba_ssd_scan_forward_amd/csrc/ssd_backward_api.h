// ssd_backward_api.h -- plan and C entry points of the backward pass.  Included once, at
// the end of ssd_api.hip: it drives the forward passes (run_forward, make_plan) of that
// translation unit and the kernels of ssd_backward.h.
#pragma once

namespace {

// Backward workspace: the forward workspace of the larger of the two forward problems,
// then the re-arranged operands and the per-head partial gradients.
struct BwdPlan {
    ssd_problem p1;   // dX pass: the layer's own shape
    ssd_problem p2;   // dB and dC passes: head dimension N, state P, one group per head
    size_t fws_bytes;
    size_t la, revdy, revc, revb, tmpp, rr, revx, tmpn, st, tmpn2, st2, bytes;
};

int make_bwd_plan(const ssd_problem* p, BwdPlan* bp) {
    int rc = check_problem(p);
    if (rc != SSD_OK) return rc;
    bp->p1 = *p;
    bp->p2 = *p;
    bp->p2.headdim = p->dstate;
    bp->p2.dstate = p->headdim;
    bp->p2.ngroups = p->nheads;
    rc = check_problem(&bp->p2);
    if (rc != SSD_OK) return rc;
    Plan a, b;
    if (make_plan(&bp->p1, &a) != SSD_OK || make_plan(&bp->p2, &b) != SSD_OK) return SSD_ERR_UNSUPPORTED;
    bp->fws_bytes = a.ws_bytes > b.ws_bytes ? a.ws_bytes : b.ws_bytes;
    const size_t es = p->dtype == SSD_DTYPE_BF16 ? 2 : 4;
    const size_t rows = (size_t)(p->batch * p->seqlen), H = (size_t)p->nheads, P = (size_t)p->headdim,
                 N = (size_t)p->dstate, G = (size_t)p->ngroups, ns = (size_t)p->nseq;
    size_t o = align_up(bp->fws_bytes, 256);
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align_up(o + bytes, 256);
        return at;
    };
    bp->la = take(rows * H * 4);
    bp->revdy = take(rows * H * P * es);
    bp->revc = take(rows * G * N * es);
    bp->revb = take(rows * G * N * es);
    bp->tmpp = take(rows * H * P * es);
    bp->rr = take(rows * H * 4);
    bp->revx = take(rows * H * P * es);
    bp->tmpn = take(rows * H * N * es);
    bp->st = take(ns * H * P * N * 4);
    // (the dC pass's own output and initial state: it may run in one launch with the dB pass)
    bp->tmpn2 = take(rows * H * N * es);
    bp->st2 = take(ns * H * P * N * 4);
    bp->bytes = o;
    return SSD_OK;
}

unsigned grid_for(int64_t n) {
    const int64_t b = (n + 255) / 256;
    return (unsigned)(b < 1 ? 1 : b > 16384 ? 16384 : b);
}

}  // namespace

extern "C" {

size_t ssd_backward_workspace_bytes(const ssd_problem* p) {
    BwdPlan bp;
    if (!p || make_bwd_plan(p, &bp) != SSD_OK) return 0;
    return bp.bytes;
}

int ssd_backward(const ssd_problem* p, const void* X, const float* logA, const void* B, const void* C,
                 const float* init_state, const int32_t* seq_offsets, const void* Y,
                 const float* final_state, const void* dY, const float* dfinal, void* dX, float* dlogA,
                 void* dB, void* dC, float* dinit, void* workspace, size_t workspace_bytes,
                 void* hip_stream) {
    if (!p) return SSD_ERR_INVALID_ARG;
    BwdPlan bp;
    int rc = make_bwd_plan(p, &bp);
    if (rc != SSD_OK) return rc;
    if (!X || !logA || !B || !C || !Y || !dY || !dX || !dlogA || !dB || !dC || !workspace)
        return SSD_ERR_INVALID_ARG;
    if (dfinal && !final_state) return SSD_ERR_INVALID_ARG;
    if (seq_offsets) {
        if (p->batch != 1) return SSD_ERR_INVALID_ARG;
    } else if (p->nseq != p->batch) {
        return SSD_ERR_INVALID_ARG;
    }
    const void* all[] = {X, logA, B, C, init_state, seq_offsets, Y, final_state, dY, dfinal, dX, dlogA, dB, dC, dinit};
    for (const void* q : all)
        if (q && !aligned16(q)) return SSD_ERR_INVALID_ARG;
    if (((uintptr_t)workspace & 255u) != 0) return SSD_ERR_INVALID_ARG;
    if (workspace_bytes < bp.bytes) return SSD_ERR_WORKSPACE;
    const size_t es = p->dtype == SSD_DTYPE_BF16 ? 2 : 4;
    const int64_t b = p->batch, T = p->seqlen, H = p->nheads, P = p->headdim, N = p->dstate,
                  G = p->ngroups, nseq = p->nseq;
    const int64_t rows = b * T;
    const size_t nx = (size_t)(rows * H * P) * es, na = (size_t)(rows * H) * 4,
                 nbc = (size_t)(rows * G * N) * es, ns = (size_t)(nseq * H * P * N) * 4,
                 no = seq_offsets ? (size_t)(nseq + 1) * 4 : 0;
    // the outputs overlap no input, no other output and not the workspace
    const void* ins[] = {X, logA, B, C, init_state, seq_offsets, Y, final_state, dY, dfinal, workspace};
    const size_t nin[] = {nx, na, nbc, nbc, ns, no, nx, ns, nx, ns, workspace_bytes};
    const void* outs[] = {dX, dlogA, dB, dC, dinit};
    const size_t nout[] = {nx, na, nbc, nbc, dinit ? ns : 0};
    for (int i = 0; i < 5; ++i) {
        for (int j = 0; j < 11; ++j)
            if (overlap(outs[i], nout[i], ins[j], nin[j])) return SSD_ERR_INVALID_ARG;
        for (int j = i + 1; j < 5; ++j)
            if (overlap(outs[i], nout[i], outs[j], nout[j])) return SSD_ERR_INVALID_ARG;
    }
    // the workspace is written too: it overlaps no input
    for (int j = 0; j < 10; ++j)
        if (overlap(workspace, workspace_bytes, ins[j], nin[j])) return SSD_ERR_INVALID_ARG;

    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    float* la = reinterpret_cast<float*>(ws + bp.la);
    void* revdy = ws + bp.revdy;
    void* revc = ws + bp.revc;
    void* revb = ws + bp.revb;
    void* tmpp = ws + bp.tmpp;
    float* rr = reinterpret_cast<float*>(ws + bp.rr);
    void* revx = ws + bp.revx;
    void* tmpn = ws + bp.tmpn;
    float* st = reinterpret_cast<float*>(ws + bp.st);
    void* tmpn2 = ws + bp.tmpn2;
    float* st2 = reinterpret_cast<float*>(ws + bp.st2);
    const ssd::RowMap fwd{seq_offsets, T, (int)nseq, 0}, rev{seq_offsets, T, (int)nseq, 1};
    const int segx = (int)(H * P * es / 16), segbc = (int)(G * N * es / 16);
    auto remap = [&](const void* in, void* out, int K, int Kin, int seg, const ssd::RowMap& m) {
        hipLaunchKernelGGL(ssd::ssd_bwd_remap_kernel, dim3(grid_for(rows * K * seg)), dim3(256), 0, stream,
                           static_cast<const uint4*>(in), static_cast<uint4*>(out), rows, K, Kin, seg, m);
    };
    auto group_sum = [&](const void* in, void* out, const ssd::RowMap& m) {
        if (p->dtype == SSD_DTYPE_BF16)
            hipLaunchKernelGGL(ssd::ssd_bwd_group_sum_kernel<__bf16>, dim3(grid_for(rows * G * N / 8)), dim3(256), 0,
                               stream, static_cast<const __bf16*>(in), static_cast<__bf16*>(out), rows, (int)H,
                               (int)G, (int)N, m);
        else
            hipLaunchKernelGGL(ssd::ssd_bwd_group_sum_kernel<float>, dim3(grid_for(rows * G * N / 8)), dim3(256), 0,
                               stream, static_cast<const float*>(in), static_cast<float*>(out), rows, (int)H,
                               (int)G, (int)N, m);
    };
    auto transpose = [&](const float* in, float* out) {
        hipLaunchKernelGGL(ssd::ssd_bwd_transpose_kernel, dim3(grid_for(nseq * H * (P / 16) * (N / 16) * 256)),
                           dim3(256), 0, stream, in, out, nseq * H, (int)P, (int)N);
    };

    // The reversed passes read and write the sequences in place, from their last row to
    // their first, where both plans are fused walks without segments (the walker's reversed
    // form); otherwise they run on reversed copies of the operands.
    bool in_place = false;
    {
        Plan a1, a2;
        in_place = make_plan(&bp.p1, &a1) == SSD_OK && make_plan(&bp.p2, &a2) == SSD_OK && a1.fused && a2.fused &&
                   a1.fseg == 1 && a2.fseg == 1 && fused_rev_for((int)bp.p1.dstate, a1.fused) &&
                   fused_rev_for((int)bp.p2.dstate, a2.fused);
    }
    auto dot_and_dlogA = [&]() {
        // dlogA
        if (p->dtype == SSD_DTYPE_BF16)
            hipLaunchKernelGGL(ssd::ssd_bwd_dot_kernel<__bf16>, dim3(grid_for(rows * H * P / 8)), dim3(256), 0, stream,
                               static_cast<const __bf16*>(dY), static_cast<const __bf16*>(Y),
                               static_cast<const __bf16*>(X), static_cast<const __bf16*>(dX), rr, rows, (int)H, (int)P);
        else
            hipLaunchKernelGGL(ssd::ssd_bwd_dot_kernel<float>, dim3(grid_for(rows * H * P / 8)), dim3(256), 0, stream,
                               static_cast<const float*>(dY), static_cast<const float*>(Y),
                               static_cast<const float*>(X), static_cast<const float*>(dX), rr, rows, (int)H, (int)P);
        hipLaunchKernelGGL(ssd::ssd_bwd_dlogA_kernel, dim3((unsigned)(nseq * H)), dim3(64), 0, stream, rr, dfinal,
                           final_state, dlogA, T, seq_offsets, (int)H, (int)(P * N), rows);
    };
    auto dinit_scale = [&]() {
        if (dinit)
            hipLaunchKernelGGL(ssd::ssd_bwd_dinit_kernel, dim3(grid_for(nseq * H * 256)), dim3(256), 0, stream,
                               dinit, logA, T, seq_offsets, (int)nseq, (int)H, (int)(P * N));
    };
    FusedCapture cb, cc;
    if (in_place) {
        // dX and dinit: X' = dY, B' = C, C' = B, initial state dF, walked in reverse
        rc = run_forward(3, &bp.p1, dY, logA, C, B, dfinal, seq_offsets, dX, dinit, ws, bp.fws_bytes, hip_stream, 0,
                         nullptr, true);
        if (rc != SSD_OK) return rc;
        dinit_scale();
        dot_and_dlogA();
        // dB: walked in reverse, X' = C (read per group), B' = dY, C' = X, initial state dF^T
        if (dfinal) transpose(dfinal, st);
        rc = run_forward(3, &bp.p2, C, logA, dY, X, dfinal ? st : nullptr, seq_offsets, tmpn, nullptr, ws,
                         bp.fws_bytes, hip_stream, G, &cb, true);
        if (rc != SSD_OK) return rc;
    } else {
        // dX and dinit: the reversed pass
        remap(dY, revdy, 1, 1, segx, rev);
        remap(C, revc, 1, 1, segbc, rev);
        remap(B, revb, 1, 1, segbc, rev);
        hipLaunchKernelGGL(ssd::ssd_bwd_logA_kernel, dim3(grid_for(rows * H)), dim3(256), 0, stream, logA, la, rows,
                           (int)H, rev);
        rc = run_forward(3, &bp.p1, revdy, la, revc, revb, dfinal, seq_offsets, tmpp, dinit, ws, bp.fws_bytes,
                         hip_stream);
        if (rc != SSD_OK) return rc;
        remap(tmpp, dX, 1, 1, segx, rev);
        dinit_scale();
        dot_and_dlogA();
        // dB: reversed, X' = C (the reversed copy of the dX pass, read per group), B' = dY,
        // C' = X, initial state dF^T
        remap(X, revx, 1, 1, segx, rev);
        if (dfinal) transpose(dfinal, st);
        rc = run_forward(3, &bp.p2, revc, la, revdy, revx, dfinal ? st : nullptr, seq_offsets, tmpn, nullptr, ws,
                         bp.fws_bytes, hip_stream, G, &cb);
        if (rc != SSD_OK) return rc;
    }
    // dC: forward time, X' = B (read per group), B' = X, C' = dY, initial state init^T
    if (init_state) transpose(init_state, st2);
    rc = run_forward(3, &bp.p2, B, logA, X, dY, init_state ? st2 : nullptr, seq_offsets, tmpn2, nullptr, ws,
                     bp.fws_bytes, hip_stream, G, &cc);
    if (rc != SSD_OK) return rc;
    // the dB and dC passes as one launch where both are fused walks of one shape (each a
    // walk of its own, with no workspace): fewer partial rounds of workgroups than two
    const fused_pair_fn_t pair =
        (cb.captured && cc.captured && !cc.rev && cb.np == cc.np && cb.nw == cc.nw) ? fused_pair_for(cb.np, cb.nw, cb.rev)
                                                                                   : nullptr;
    if (pair) {
        const int64_t n0 = (cb.grid + 7) / 8 * 8;
        if (n0 + cc.grid > INT32_MAX) return SSD_ERR_UNSUPPORTED;
        hipLaunchKernelGGL(pair, dim3((unsigned)(n0 + cc.grid)), dim3(64 * (cb.nw + 3)), 0, stream, cb.a, cc.a, (int)n0);
    } else {
        if (cb.captured)
            hipLaunchKernelGGL(cb.fn, dim3((unsigned)cb.grid), dim3(64 * (cb.nw + 3)), 0, stream, cb.a);
        if (cc.captured)
            hipLaunchKernelGGL(cc.fn, dim3((unsigned)cc.grid), dim3(64 * (cc.nw + 3)), 0, stream, cc.a);
    }
    // per-group sums over the heads (the copied dB pass wrote its rows reversed)
    group_sum(tmpn, dB, in_place ? fwd : rev);
    group_sum(tmpn2, dC, fwd);
    if (hipGetLastError() != hipSuccess) return SSD_ERR_HIP;
    return SSD_OK;
}

}  // extern "C"
