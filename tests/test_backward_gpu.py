"""GPU parity of ssd_backward against the float64 adjoint recurrence of the oracle.

For L = <dY, Y> + <dF, final>: dX, dlogA, dB, dC and dinit from the HIP path (three
forward passes on re-arranged operands plus small kernels) against ``oracle.backward``
on the same, already quantized, inputs.  Metric per gradient: max|out - ref| / max|ref|.
Bars: 2e-4 for float32 inputs (the three passes and the cumsum of the decay gradient
each add float32 rounding to the forward pass's 1e-4), 2e-2 for bfloat16 inputs (the
forward pass's bar; the per-head partial gradients are rounded to bfloat16 before their
sum over the heads of a group, as the outputs are).

dlogA is the reverse cumsum of dy . y - x . dx: a difference of two cumulative sums that
are several times larger than itself (pairs of tokens on the same side of t enter both
and cancel).  With bfloat16 operands y and dx carry relative errors of a few 1e-3, so
its error scales with those sums, not with dlogA: for bfloat16 its metric divides by
max(max|ref|, max_t |sum_{k >= t} dy_k . y_k|) (oracle values); the plain metric is printed
beside it.  float32 keeps the plain metric and bar, which pins the computation itself.
"""
import numpy as np
import pytest

import oracle
from workloads import bf16_round, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 2e-4, "bf16": 2e-2}


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def rel_err(out, ref):
    return float(np.max(np.abs(out - ref))) / max(float(np.max(np.abs(ref))), 1e-30)


def cumsum_scale(inp, dY):
    """max over sequences, heads and tokens t of |sum_{k >= t} dy_k . y_k| (oracle Y)."""
    Y, _ = oracle.recurrence(inp.X, inp.logA, inp.B, inp.C, inp.init, inp.seq_offsets)
    r = np.sum(dY.astype(np.float64) * Y, axis=-1).reshape(-1, Y.shape[2])   # [rows, H]
    b, T = Y.shape[0], Y.shape[1]
    bounds = ([(s * T, (s + 1) * T) for s in range(b)] if inp.seq_offsets is None
              else list(zip(inp.seq_offsets[:-1], inp.seq_offsets[1:])))
    m = 0.0
    for r0, r1 in bounds:
        if r1 > r0:
            m = max(m, float(np.max(np.abs(np.cumsum(r[r0:r1][::-1], axis=0)))))
    return m


def check_backward(inp, Q, label, with_dfinal=True, seed=0):
    import mamba_ssd_scan_forward_amd as ssd
    torch = _torch()
    dt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    q = bf16_round if inp.dtype == "bf16" else (lambda a: a.astype(np.float32))
    rng = np.random.default_rng(seed)
    nseq = inp.X.shape[0] if inp.seq_offsets is None else len(inp.seq_offsets) - 1
    H, P = inp.X.shape[2], inp.X.shape[3]
    N = inp.B.shape[3]
    dY = q(rng.standard_normal(inp.X.shape))
    dF = (rng.standard_normal((nseq, H, P, N)) * 0.5).astype(np.float32) if with_dfinal else None
    print(f"[backward] {label} X{tuple(inp.X.shape)} G={inp.B.shape[2]} N={N} Q={Q} {inp.dtype} "
          f"init={inp.init is not None} varlen={inp.seq_offsets is not None} dF={with_dfinal}", flush=True)
    dev = lambda a, t=dt: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(t).cuda()
    X, logA, B, C = dev(inp.X), dev(inp.logA, torch.float32), dev(inp.B), dev(inp.C)
    init = dev(inp.init, torch.float32)
    off = None if inp.seq_offsets is None else torch.from_numpy(inp.seq_offsets).cuda()
    Y, F = ssd.forward(X, logA, B, C, Q, init, off)
    grads = ssd.backward(X, logA, B, C, Q, Y, dev(dY), init, off, F, dev(dF, torch.float32))
    torch.cuda.synchronize()
    got = [None if g is None else g.float().cpu().numpy().astype(np.float64) for g in grads]
    ref = oracle.backward(inp.X, inp.logA, inp.B, inp.C, inp.init, inp.seq_offsets, dY, dF)
    names = ["dX", "dlogA", "dB", "dC", "dinit"]
    errs = {}
    for name, g, r in zip(names, got, ref):
        if r is None:
            continue
        assert np.all(np.isfinite(g)), name
        errs[name] = rel_err(g, r)
    if inp.dtype == "bf16":
        scale = cumsum_scale(inp, dY)
        errs["dlogA_plain"] = errs["dlogA"]
        errs["dlogA"] = float(np.max(np.abs(got[1] - ref[1]))) / max(float(np.max(np.abs(ref[1]))), scale)
    print("[backward]   " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    errs.pop("dlogA_plain", None)
    for k, v in errs.items():
        assert v <= TOL[inp.dtype], (k, v)
    return got, ref


@pytest.mark.parametrize("case", ["layer_shape", "varlen", "f32_general", "bf16_q64", "no_init_no_dfinal",
                                  "segmented", "headdim128", "f32_headdim48", "in_place_ragged",
                                  "in_place_varlen", "in_place_many_seqs"])
def test_backward_matches_oracle(case):
    if case in ("in_place_ragged", "in_place_varlen", "in_place_many_seqs"):
        # shapes whose dX, dB and dC passes are fused walks without segments: the reversed
        # passes read and write the sequences in place (ragged last blocks; packed
        # sequences with an empty one and a length-1 one)
        if case == "in_place_ragged":
            inp = make_inputs(16, 300, 16, 64, 128, 2, "bf16", seed=2008, init_state=True)
        elif case == "in_place_varlen":
            lens = [300, 1, 0, 257, 511, 33, 700, 64] * 4
            inp = make_inputs(1, sum(lens), 16, 64, 128, 2, "bf16", seed=2009, init_state=True, seq_lengths=lens)
        else:
            # more sequences than the longest-first dealing takes (64): the plain workgroup order
            lens = [37, 0, 129, 64, 1, 95, 200, 31, 160] * 8
            inp = make_inputs(1, sum(lens), 16, 64, 128, 2, "bf16", seed=2010, init_state=True, seq_lengths=lens)
        b, T, H, P = inp.X.shape
        N, G = inp.B.shape[3], inp.B.shape[2]
        nseq = b if inp.seq_offsets is None else len(inp.seq_offsets) - 1
        import mamba_ssd_scan_forward_amd as ssd
        bf = ssd.SSD_DTYPE_BF16
        for prob in (ssd.problem_for(b, T, H, P, N, G, 256, nseq, bf), ssd.problem_for(b, T, H, N, P, H, 256, nseq, bf)):
            d = ssd.ssd_plan_describe(prob)
            assert d["walk"].startswith("ssd_walk_fused_kernel") and d["summary"] == "none", d
        check_backward(inp, 256, case)
    elif case == "layer_shape":
        inp = make_inputs(2, 600, 4, 64, 128, 2, "bf16", seed=2000, init_state=True)
        check_backward(inp, 256, case)
    elif case == "varlen":
        lens = [5, 0, 300, 1, 256, 257, 33]
        inp = make_inputs(1, sum(lens), 4, 64, 128, 2, "bf16", seed=2001, init_state=True, seq_lengths=lens)
        got, ref = check_backward(inp, 256, case)
        # the empty sequence hands dF straight back as dinit
        np.testing.assert_allclose(got[4][1], ref[4][1], rtol=0, atol=0)
    elif case == "f32_general":
        inp = make_inputs(2, 200, 3, 32, 64, 1, "f32", seed=2002, init_state=True)
        check_backward(inp, 64, case)
    elif case == "bf16_q64":
        inp = make_inputs(1, 300, 2, 64, 64, 1, "bf16", seed=2003, init_state=True)
        check_backward(inp, 64, case)
    elif case == "no_init_no_dfinal":
        inp = make_inputs(2, 400, 2, 64, 128, 1, "bf16", seed=2004)
        check_backward(inp, 256, case, with_dfinal=False)
    elif case == "segmented":
        inp = make_inputs(1, 4200, 4, 64, 128, 1, "bf16", seed=2005, init_state=True)
        check_backward(inp, 256, case)
    elif case == "headdim128":
        inp = make_inputs(2, 520, 3, 128, 64, 1, "bf16", seed=2006, init_state=True)
        check_backward(inp, 256, case)
    else:
        # P = 48: a (row, head) item of 6 vectors can straddle two 256-vector windows of
        # the decay-gradient dot product
        inp = make_inputs(2, 300, 5, 48, 32, 1, "f32", seed=2007, init_state=True)
        check_backward(inp, 64, case)


def test_backward_is_bitwise_repeatable():
    """Two backward passes on the same inputs give the same bits in every gradient (no
    atomics and no order that depends on thread timing); the layer shape and a packed
    batch at P = 48 (items straddling reduction windows)."""
    import mamba_ssd_scan_forward_amd as ssd
    torch = _torch()
    cases = [(make_inputs(2, 600, 4, 64, 128, 2, "bf16", seed=2100, init_state=True), 256),
             (make_inputs(1, 700, 5, 48, 32, 1, "f32", seed=2101, init_state=True,
                          seq_lengths=[300, 0, 1, 399]), 64)]
    for inp, Q in cases:
        dt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
        dev = lambda a, t=dt: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(t).cuda()
        rng = np.random.default_rng(5)
        nseq = inp.X.shape[0] if inp.seq_offsets is None else len(inp.seq_offsets) - 1
        H, P, N = inp.X.shape[2], inp.X.shape[3], inp.B.shape[3]
        dY = rng.standard_normal(inp.X.shape)
        dF = (rng.standard_normal((nseq, H, P, N)) * 0.5).astype(np.float32)
        X, logA, B, C = dev(inp.X), dev(inp.logA, torch.float32), dev(inp.B), dev(inp.C)
        init = dev(inp.init, torch.float32)
        off = None if inp.seq_offsets is None else torch.from_numpy(inp.seq_offsets).cuda()
        print(f"[backward] repeatability X{tuple(inp.X.shape)} {inp.dtype}", flush=True)
        Y, F = ssd.forward(X, logA, B, C, Q, init, off)
        runs = [ssd.backward(X, logA, B, C, Q, Y, dev(dY), init, off, F, dev(dF, torch.float32)) for _ in range(3)]
        torch.cuda.synchronize()
        for name, a, b, c in zip(["dX", "dlogA", "dB", "dC", "dinit"], *runs):
            assert torch.equal(a, b) and torch.equal(a, c), name


@pytest.mark.parametrize("name,sample", [("cfg1_mamba2_2.7b_bf16", [0, 7]), ("cfg4_varlen32k_bf16", [6, 13])])
def test_backward_full_size_sampled_sequences(name, sample):
    """The backward pass of a whole workload configuration in the launch configuration the
    benchmark times; the oracle recomputes the gradients of two sampled sequences (the
    sequences are independent, so their slices of every gradient are exact references)."""
    import copy
    import mamba_ssd_scan_forward_amd as ssd
    from workloads import CONFIGS, workload_inputs
    torch = _torch()
    w = CONFIGS[name]
    inp = workload_inputs(w)
    rng = np.random.default_rng(77)
    nseq = w.batch if inp.seq_offsets is None else len(inp.seq_offsets) - 1
    dY = bf16_round(rng.standard_normal(inp.X.shape))
    dF = (rng.standard_normal((nseq, w.nheads, w.headdim, w.dstate)) * 0.5).astype(np.float32)
    print(f"[backward] full size {name}, sampled sequences {sample}", flush=True)
    dt = torch.bfloat16
    dev = lambda a, t=dt: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(t).cuda()
    X, logA, B, C = dev(inp.X), dev(inp.logA, torch.float32), dev(inp.B), dev(inp.C)
    init = dev(inp.init, torch.float32)
    off = None if inp.seq_offsets is None else torch.from_numpy(inp.seq_offsets).cuda()
    Y, F = ssd.forward(X, logA, B, C, w.chunk_len, init, off)
    grads = ssd.backward(X, logA, B, C, w.chunk_len, Y, dev(dY), init, off, F, dev(dF, torch.float32))
    torch.cuda.synchronize()
    got = [g.float().cpu().numpy().astype(np.float64) for g in grads]
    for s in sample:
        if inp.seq_offsets is None:
            rows = slice(None)
            sub = copy.deepcopy(inp)
            sub.X, sub.logA, sub.B, sub.C = (a[s:s + 1] for a in (inp.X, inp.logA, inp.B, inp.C))
            sub.init = None if inp.init is None else inp.init[s:s + 1]
            sl = lambda a: a[s:s + 1]
        else:
            r0, r1 = int(inp.seq_offsets[s]), int(inp.seq_offsets[s + 1])
            sub = copy.deepcopy(inp)
            sub.X, sub.logA, sub.B, sub.C = (a[:, r0:r1] for a in (inp.X, inp.logA, inp.B, inp.C))
            sub.init = None if inp.init is None else inp.init[s:s + 1]
            sub.seq_offsets = None
            sl = lambda a: a[:, r0:r1]
        ref = oracle.backward(sub.X, sub.logA, sub.B, sub.C, sub.init, None, sl(dY), dF[s:s + 1])
        mine = [sl(got[0]), sl(got[1]), sl(got[2]), sl(got[3]), got[4][s:s + 1]]
        errs = {n: rel_err(g, r) for n, g, r in zip(["dX", "dlogA", "dB", "dC", "dinit"], mine, ref)
                if r is not None}
        scale = cumsum_scale(sub, sl(dY))
        errs["dlogA_plain"] = errs["dlogA"]
        errs["dlogA"] = float(np.max(np.abs(mine[1] - ref[1]))) / max(float(np.max(np.abs(ref[1]))), scale)
        print(f"[backward]   seq {s}: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
        errs.pop("dlogA_plain", None)
        for k, v in errs.items():
            assert v <= TOL["bf16"], (s, k, v)
