"""GPU parity of ssd_decode_step (the recurrent step) against the float64 oracle.

Same metric and bars as the forward pass: max|out - ref| / max|ref| for y and for the
updated state, 1e-4 for float32 inputs and 2e-2 for bfloat16 inputs; the state itself is
float32 in both cases.
"""
import numpy as np
import pytest

import oracle
from workloads import bf16_round, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def rel_err(out, ref):
    return float(np.max(np.abs(out - ref))) / max(float(np.max(np.abs(ref))), 1e-30)


def step_inputs(b, H, P, N, G, dtype, seed):
    rng = np.random.default_rng(seed)
    q = (lambda a: bf16_round(a)) if dtype == "bf16" else (lambda a: a.astype(np.float32))
    x = q(rng.standard_normal((b, H, P)))
    B = q(rng.standard_normal((b, G, N)) / np.sqrt(N))
    C = q(rng.standard_normal((b, G, N)) / np.sqrt(N))
    logA = (-rng.uniform(0.001, 0.1, (b, H)) * rng.uniform(1, 16, (1, H))).astype(np.float32)
    S = (rng.standard_normal((b, H, P, N)) * 0.3).astype(np.float32)
    return x, logA, B, C, S


def run_step(x, logA, B, C, S, dtype):
    import mamba_ssd_scan_forward_amd as ssd
    torch = _torch()
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dS = torch.from_numpy(S).cuda()
    y = ssd.decode_step(torch.from_numpy(x).to(dt).cuda(), torch.from_numpy(logA).cuda(),
                        torch.from_numpy(B).to(dt).cuda(), torch.from_numpy(C).to(dt).cuda(), dS)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), dS.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("b,H,P,N,G,dtype", [
    (8, 80, 64, 128, 1, "bf16"),     # the 2.7B-shaped layer
    (3, 8, 32, 64, 4, "bf16"),
    (2, 4, 16, 16, 2, "f32"),
    (2, 6, 48, 256, 3, "f32"),
    (1, 2, 256, 32, 1, "bf16"),
    # d_state not a power of two: a row's threads are rounded up to one
    (3, 4, 64, 48, 2, "bf16"),
    (2, 4, 80, 80, 1, "f32"),
    (2, 3, 32, 144, 3, "bf16"),
    (1, 2, 48, 240, 1, "f32"),
])
def test_decode_step_matches_oracle(b, H, P, N, G, dtype):
    x, logA, B, C, S = step_inputs(b, H, P, N, G, dtype, seed=b * 1000 + H + P + N)
    print(f"[decode] b={b} H={H} P={P} N={N} G={G} {dtype}", flush=True)
    y, S1 = run_step(x, logA, B, C, S, dtype)
    yr, Sr = oracle.decode_step(S, x, logA, B, C)
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(S1))
    assert rel_err(y, yr) <= TOL[dtype], rel_err(y, yr)
    assert rel_err(S1, Sr) <= TOL[dtype], rel_err(S1, Sr)


def test_forward_then_decode_continues_the_sequence():
    """GPU forward over 300 tokens, then 5 GPU decode steps from its final state, against
    the oracle's recurrence over all 305 tokens."""
    import mamba_ssd_scan_forward_amd as ssd
    torch = _torch()
    inp = make_inputs(2, 305, 4, 64, 128, 2, "bf16", seed=1100, init_state=True)
    T0 = 300
    dt = torch.bfloat16
    dev = lambda a, t=dt: torch.from_numpy(np.ascontiguousarray(a)).to(t).cuda()
    print("[decode] forward 300 + 5 steps", flush=True)
    _, F = ssd.forward(dev(inp.X[:, :T0]), dev(inp.logA[:, :T0], torch.float32), dev(inp.B[:, :T0]),
                       dev(inp.C[:, :T0]), 256, dev(inp.init, torch.float32))
    ys = []
    for t in range(T0, 305):
        y = ssd.decode_step(dev(inp.X[:, t]), dev(inp.logA[:, t], torch.float32), dev(inp.B[:, t]),
                            dev(inp.C[:, t]), F)
        ys.append(y.float().cpu().numpy())
    torch.cuda.synchronize()
    Yr, Fr = oracle.recurrence(inp.X, inp.logA, inp.B, inp.C, inp.init)
    assert rel_err(np.stack(ys, axis=1).astype(np.float64), Yr[:, T0:]) <= 2e-2
    assert rel_err(F.cpu().numpy().astype(np.float64), Fr) <= 2e-2
