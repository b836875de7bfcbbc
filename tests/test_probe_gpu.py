"""The machine measurements of include/ssd_probe.h on the GPU: the MFMA-rate and clock
kernels run, stamp every workgroup, and give a plausible shader clock."""
import numpy as np
import pytest

import mamba_ssd_scan_forward_amd as ssd

pytestmark = pytest.mark.gpu


def clocks(stamps):
    t = stamps.reshape(-1, 4).astype(np.float64)
    assert np.all(t[:, 2] > t[:, 0]) and np.all(t[:, 3] > t[:, 1])
    return (t[:, 2] - t[:, 0]) / (t[:, 3] - t[:, 1]) * 100.0


def test_probe_device_mfma_and_clock():
    import ctypes
    import torch
    probe = ssd.load_probe_library()
    cus, khz = ctypes.c_int(0), ctypes.c_int(0)
    assert probe.ssd_probe_device(ctypes.byref(cus), ctypes.byref(khz)) == 0
    print(f"[probe] {cus.value} CUs, {khz.value / 1000:.0f} MHz", flush=True)
    assert cus.value > 0 and khz.value > 0
    s = torch.cuda.current_stream().cuda_stream
    st = torch.zeros(4 * 8, dtype=torch.int64, device="cuda")
    assert probe.ssd_probe_mfma_bf16(2000, 8, st.data_ptr(), s) == 0
    torch.cuda.synchronize()
    c = clocks(st.cpu().numpy())
    print(f"[probe] MFMA clock {c.mean():.0f} MHz", flush=True)
    assert np.all((c > 300) & (c < 4000))
    sc = torch.zeros(4 * 4, dtype=torch.int64, device="cuda")
    assert probe.ssd_probe_clock(200, 4, sc.data_ptr(), s) == 0
    torch.cuda.synchronize()
    c = clocks(sc.cpu().numpy())
    print(f"[probe] sampler clock {c.mean():.0f} MHz", flush=True)
    assert np.all((c > 300) & (c < 4000))
