"""ssd_forward_noalloc, the forward entry point that allocates nothing, against ssd_forward
on the same inputs (needs an MI355X).

Both run the same kernels in the same order, so their outputs must agree bit for bit.  Two
calls in a row go through the no-allocation entry point, the second on a smaller problem,
so the second runs on scratch that the first left behind.
"""
import numpy as np
import pytest

from workloads import make_inputs

pytestmark = pytest.mark.gpu

# label, batch, seqlen, heads, headdim, d_state, groups, chunk_len, dtype, seed, init, lengths
FIRST = ("one long sequence walked in segments", 1, 16384, 80, 64, 128, 1, 256, "bf16", 71, False, None)
SECOND = ("packed ragged sequences with init state", 1, 3000, 8, 64, 64, 2, 256, "bf16", 72, True,
          [1000, 7, 0, 1993])


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _device_inputs(case):
    torch = _torch()
    _, b, T, H, P, N, G, Q, dtype, seed, init, lens = case
    inp = make_inputs(b, T, H, P, N, G, dtype, seed, init_state=init, seq_lengths=lens)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return dict(X=torch.from_numpy(inp.X).to(dt).cuda(), logA=torch.from_numpy(inp.logA).cuda(),
                B=torch.from_numpy(inp.B).to(dt).cuda(), C=torch.from_numpy(inp.C).to(dt).cuda(),
                init=None if inp.init is None else torch.from_numpy(inp.init).cuda(),
                off=None if inp.seq_offsets is None else torch.from_numpy(inp.seq_offsets).cuda(),
                Q=Q, nseq=len(lens) if lens else b)


def _noalloc(d):
    import mamba_ssd_scan_forward_amd as ssd
    torch = _torch()
    X = d["X"]
    b, T, H, P = X.shape
    G, N = d["B"].shape[2], d["B"].shape[3]
    dt = ssd.SSD_DTYPE_BF16 if X.dtype == torch.bfloat16 else ssd.SSD_DTYPE_F32
    prob = ssd.problem_for(b, T, H, P, N, G, d["Q"], d["nseq"], dt)
    Y = torch.empty_like(X)
    F = torch.empty((d["nseq"], H, P, N), dtype=torch.float32, device=X.device)
    ptr = lambda t: None if t is None else t.data_ptr()
    rc = ssd.ssd_forward_noalloc(prob, ptr(X), ptr(d["logA"]), ptr(d["B"]), ptr(d["C"]), ptr(d["init"]),
                                 ptr(d["off"]), ptr(Y), ptr(F), torch.cuda.current_stream().cuda_stream or None)
    assert rc == ssd.SSD_OK, ssd.ssd_status_string(rc)
    return prob, Y, F


def test_noalloc_matches_forward_on_two_calls_in_a_row():
    import mamba_ssd_scan_forward_amd as ssd
    torch = _torch()
    d1, d2 = _device_inputs(FIRST), _device_inputs(SECOND)
    print(f"[no-alloc] {FIRST[0]} then {SECOND[0]}", flush=True)
    p1, Y1, F1 = _noalloc(d1)
    p2, Y2, F2 = _noalloc(d2)
    torch.cuda.synchronize()
    # both problems take a plan whose kernels use scratch
    assert ssd.ssd_workspace_bytes(p1) > 1 << 20 and ssd.ssd_plan_describe(p1)["summary"] != "none"
    assert ssd.ssd_workspace_bytes(p2) > 1 << 10 and ssd.ssd_plan_describe(p2)["prep"] != "none"
    assert ssd.ssd_workspace_bytes(p2) <= ssd.ssd_workspace_bytes(p1) <= ssd.SSD_NOALLOC_SCRATCH_BYTES
    for d, Y, F in ((d1, Y1, F1), (d2, Y2, F2)):
        Yr, Fr = ssd.forward(d["X"], d["logA"], d["B"], d["C"], d["Q"], d["init"], d["off"])
        torch.cuda.synchronize()
        assert torch.isfinite(Y.float()).all() and torch.isfinite(F).all()
        assert torch.equal(Y, Yr), float((Y.float() - Yr.float()).abs().max())
        assert torch.equal(F, Fr), float((F - Fr).abs().max())


def test_noalloc_rejects_a_problem_beyond_its_scratch():
    import mamba_ssd_scan_forward_amd as ssd
    torch = _torch()
    # 32 float32 sequences of 4096 tokens, 32 heads, d_state 256 need more than the fixed scratch
    prob = ssd.problem_for(32, 4096, 32, 64, 256, 1, 256, 32, ssd.SSD_DTYPE_F32)
    assert ssd.ssd_workspace_bytes(prob) > ssd.SSD_NOALLOC_SCRATCH_BYTES
    t = torch.empty(16, dtype=torch.uint8, device="cuda")
    a = t.data_ptr()
    assert ssd.ssd_forward_noalloc(prob, a, a, a, a, None, None, a, None, None) == ssd.SSD_ERR_TOO_LARGE
