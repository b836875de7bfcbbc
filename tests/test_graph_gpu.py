"""The C entry points under HIP graph capture: ssd_forward and ssd_decode_step enqueue only
kernels on the caller's stream (no allocation, no memset, no synchronisation), so a captured
graph replays them.  Each replay, with eager work and synchronisation between replays, must
reproduce the eager result bit for bit (the kernels are deterministic)."""
import numpy as np
import pytest

from workloads import make_inputs

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.mark.parametrize("T,Q", [(600, 256), (4100, 256), (300, 64)])
def test_forward_replays_in_a_graph(T, Q):
    import mamba_ssd_scan_forward_amd as ssd
    torch = _torch()
    b, H, P, N, G = 2, 4, 64, 128, 2
    inp = make_inputs(b, T, H, P, N, G, "bf16", seed=3000 + T, init_state=True)
    dev = torch.device("cuda", 0)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).to(dev)
    X, B, C = bf(inp.X), bf(inp.B), bf(inp.C)
    logA = torch.from_numpy(inp.logA).to(dev)
    init = torch.from_numpy(inp.init).to(dev)
    prob = ssd.problem_for(b, T, H, P, N, G, Q, b, ssd.SSD_DTYPE_BF16)
    wsb = ssd.ssd_workspace_bytes(prob)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    Y = torch.empty_like(X)
    F = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
    args = lambda stream: (prob, X.data_ptr(), logA.data_ptr(), B.data_ptr(), C.data_ptr(), init.data_ptr(),
                           None, Y.data_ptr(), F.data_ptr(), ws.data_ptr(), wsb, stream)
    print(f"[graph] forward T={T} Q={Q}", flush=True)
    assert ssd.ssd_forward(*args(torch.cuda.current_stream().cuda_stream)) == 0
    torch.cuda.synchronize()
    Y0, F0 = Y.clone(), F.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        assert ssd.ssd_forward(*args(torch.cuda.current_stream().cuda_stream)) == 0
    for _ in range(3):
        Y.zero_()
        F.fill_(float("nan"))
        ws.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, Y0)
        assert torch.equal(F, F0)


def test_decode_step_replays_in_a_graph():
    import mamba_ssd_scan_forward_amd as ssd
    torch = _torch()
    b, H, P, N, G = 8, 80, 64, 128, 1
    dev = torch.device("cuda", 0)
    gen = torch.Generator(device="cpu").manual_seed(5)
    x = torch.randn(b, H, P, generator=gen).to(torch.bfloat16).to(dev)
    a = (-torch.rand(b, H, generator=gen)).to(dev)
    Bv = (torch.randn(b, G, N, generator=gen) / N ** 0.5).to(torch.bfloat16).to(dev)
    Cv = (torch.randn(b, G, N, generator=gen) / N ** 0.5).to(torch.bfloat16).to(dev)
    S0 = torch.randn(b, H, P, N, generator=gen).to(dev)
    S = S0.clone()
    y = torch.empty_like(x)
    prob = ssd.problem_for(b, 1, H, P, N, G, 16, b, ssd.SSD_DTYPE_BF16)
    ptrs = lambda stream: (prob, x.data_ptr(), a.data_ptr(), Bv.data_ptr(), Cv.data_ptr(), S.data_ptr(),
                           y.data_ptr(), stream)
    print("[graph] decode step", flush=True)
    assert ssd.ssd_decode_step(*ptrs(torch.cuda.current_stream().cuda_stream)) == 0
    torch.cuda.synchronize()
    y0, S1 = y.clone(), S.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    S.copy_(S0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        assert ssd.ssd_decode_step(*ptrs(torch.cuda.current_stream().cuda_stream)) == 0
    for _ in range(3):
        S.copy_(S0)
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y0)
        assert torch.equal(S, S1)
