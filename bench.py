"""Benchmark of the SSD layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one whole SSD forward over one synthetic batch already resident in HBM: the
launches the library plans for the shape (one fused walk for bf16 layer shapes that fill
the chip; else a prep launch of chunk cumsums and C B^T tiles, then the chunk walk, and a
summary pass where sequences are split).  Prints ONE JSON line on stdout; progress goes to
stderr.  The kernels timed are the ones the library reports for the shape
(``ssd_plan_describe``).

Warm-up runs the requested steps, then more until it has run for at least MIN_WARM_S
seconds (the chip needs some tens of milliseconds to reach its steady clocks).  Besides
the warm figure the line carries a cold one: the median of per-step times with a 512 MiB
buffer read before each step, which evicts the inputs from the last-level cache.

Roofline: the dominant launch is the chunk walk.  Its algorithmic bytes are the
minimum traffic of the layer: read X, B, C and logA once, write Y and the final state
once (the per-token figure times the tokens of one launch, plus the states).  Its
duration is measured here with HIP events on the stream it runs on, one pair around a run
of walk launches back to back (as the timed steps run them); the mean of one event pair
around each walk launch is reported beside it (events recorded between launches slow the
launch after them down, which a kernel trace of the same run shows).  HBM traffic
measured by counters is read from the committed counter summary when it was taken on the
current kernel source, else null.

``--mode copy`` runs only a plain device copy of known size; it is the calibration
program for the FETCH_SIZE / WRITE_SIZE counters.

``--mode report`` prints one JSON line per workload configuration (all of them, or the
one ``--workload`` names): the median of per-step HIP-event times with the last-level
cache flushed before every step (a 512 MiB read) and without, the FLOP rates by the
pages' count and by its causal half, and the fractions of the MFMA peak and of the
roofline (the parity of each configuration is the full-size tests' business).
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSD fwd tokens/s + MFMA util, bf16 H=80 P=64 N=128 T=2K batch 8"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 matrix/vector, published
COUNTERS_JSON = os.path.join(ROOT, "profiles", "walk_cfg1_hbm_counters.json")
MIN_WARM_S = 0.5               # least wall time of warm-up before the timed steps


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# the sources of the forward kernels and of their launch plan (the backward pass's files
# are not among them)
FORWARD_SOURCES = ("ssd_device.h", "ssd_kernels.h", "ssd_walk_split.h", "ssd_walk_fused.h",
                   "ssd_walk_segments.h", "ssd_api.hip")


def kernel_source_hash():
    h = hashlib.sha256()
    for name in FORWARD_SOURCES:
        with open(os.path.join(ROOT, "mamba_ssd_scan_forward_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w, es):
    """Minimum HBM traffic of one forward: read X, B, C, logA (+ init), write Y, final."""
    tokens = w.batch * w.seqlen
    per_token = (2 * w.nheads * w.headdim * es          # X in, Y out
                 + 2 * w.ngroups * w.dstate * es         # B, C in
                 + w.nheads * 4)                         # logA in
    nseq = w.nseq if w.varlen else w.batch
    state = nseq * w.nheads * w.headdim * w.dstate * 4
    return tokens * per_token + state * (2 if w.init_state else 1)


def flops_pages(w, chunk_lens):
    """Block-decomposition FLOPs counted as the pages count them (section 6.3 BMMs):
    per chunk 2*[G*Q^2*N + H*(Q^2*P + 2*Q*N*P)], C B^T once per group."""
    f = 0
    for q in chunk_lens:
        f += 2 * (w.ngroups * q * q * w.dstate + w.nheads * (q * q * w.headdim + 2 * q * w.dstate * w.headdim))
    return f


def flops_causal(w, chunk_lens):
    """The same count with only the causal half of each chunk's Q x Q blocks: q(q+1)/2."""
    f = 0
    for q in chunk_lens:
        tri = q * (q + 1) // 2
        f += 2 * (w.ngroups * tri * w.dstate + w.nheads * (tri * w.headdim + 2 * q * w.dstate * w.headdim))
    return f


def chunk_lengths(w, lens):
    out = []
    for L in lens:
        full, rem = divmod(L, w.chunk_len)
        out += [w.chunk_len] * full + ([rem] if rem else [])
    return out


def flush_by_reading(buf):
    """Evict the last-level cache by reading a buffer twice its size: the cache is left
    holding clean lines, so the next kernel neither hits on its inputs nor pays for
    writing back a flush buffer's dirty lines."""
    buf.max()


def executed_mfma_flops(plan, w, lens):
    """FLOPs of the MFMA instructions the fused walker issues (v_mfma_f32_32x32x16_bf16,
    32768 each): per 32-row block and 32-column unit of a head, 8 for the left factor, 8
    for the state update and 2 for the diagonal block (N = 128; N/16 each of the first two
    in general); per block and workgroup N/16 for the tile C B^T.  None for other walks."""
    walk = plan.get("walk", "")
    if not walk.startswith("ssd_walk_fused_kernel<"):
        return None
    nw = int(walk.split("<")[1].split(",")[1].strip(" >"))
    ks = w.dstate // 16
    units = (w.nheads // w.ngroups) * (w.headdim // 32)
    wpg = -(-units // nw)
    blocks = sum(-(-int(L) // 32) for L in lens)
    per_unit = 2 * ks + 2
    mfmas = blocks * w.ngroups * (units * per_unit + wpg * ks)
    return mfmas * 32768


PAGES_CONTEXT = {
    "vs_mamba_selective_scan": "2-8x faster (paper summary page, section 9.3, Fig. 10 left; state size 64)",
    "vs_flashattention2": "on par at sequence length 2K (news page) / faster from 2K (paper summary page), "
                          "about 6x faster at 16K",
    "state_size_sweep": "SSD slows little as the state grows, the selective scan linearly (Fig. 10 right)",
    "hardware": "A100 80GB PCIe per the paper summary page's appendix; absolute times are not given",
}


def run_copy_mode(steps):
    import torch
    n = 512 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "copy", "bytes_read": n, "bytes_written": n, "launches": steps}))


def clocks_mhz(stamps):
    """Shader clock of each workgroup from its (s_memtime, s_memrealtime) stamps at start
    and end (the real-time counter runs at 100 MHz)."""
    import numpy as np
    t = stamps.reshape(-1, 4).astype(np.float64)
    return (t[:, 2] - t[:, 0]) / np.maximum(t[:, 3] - t[:, 1], 1.0) * 100.0


def measure_machine(walk, stream, dev):
    """The roofline constants as this chip reaches them (libssd_probe.so): the dense bf16
    MFMA rate and the clock under it, a 512 MiB device copy, and the clock while the walk
    kernel runs (a one-wave-per-workgroup sampler on a second stream beside five walk
    launches, bracketed on the walk's stream by two one-workgroup markers)."""
    out = measure_peaks(stream, dev)
    out.update(measure_walk_clock(walk, stream, dev))
    return out


def measure_peaks(stream, dev):
    """The dense bf16 MFMA rate (and the clock under it) and a 512 MiB device copy."""
    import ctypes
    import numpy as np
    import torch
    import mamba_ssd_scan_forward_amd as ssd
    probe = ssd.load_probe_library()
    cus, khz = ctypes.c_int(0), ctypes.c_int(0)
    if probe.ssd_probe_device(ctypes.byref(cus), ctypes.byref(khz)) != 0:
        raise RuntimeError("ssd_probe_device failed")
    sp = stream.cuda_stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # MFMA: two workgroups of four waves per CU
    blocks, iters = 2 * cus.value, 40000
    st = torch.zeros(4 * blocks, dtype=torch.int64, device=dev)
    for rep in range(3):   # (the first launch warms up)
        e0.record(stream)
        assert probe.ssd_probe_mfma_bf16(iters, blocks, st.data_ptr(), sp) == 0
        e1.record(stream)
        torch.cuda.synchronize()
    mfma_s = e0.elapsed_time(e1) * 1e-3
    mfma_tflops = blocks * 4 * 4 * iters * 32768 / mfma_s / 1e12
    mfma_clk = float(np.mean(clocks_mhz(st.cpu().numpy())))
    # copy
    n = 512 << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * n * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return {"compute_units": cus.value, "max_clock_mhz": khz.value / 1000.0,
            "mfma_bf16_tflops": round(mfma_tflops, 1), "mfma_clock_mhz": round(mfma_clk, 0),
            "hbm_copy_gbs": round(copy_gbs, 1)}


def measure_walk_clock(walk, stream, dev):
    """The shader clock while the walk runs: a one-wave-per-workgroup sampler on a second
    stream, started when the first of five walk launches has ended, its window checked
    against two one-workgroup markers on the walk's stream."""
    import numpy as np
    import torch
    import mamba_ssd_scan_forward_amd as ssd
    probe = ssd.load_probe_library()
    sp = stream.cuda_stream
    side = torch.cuda.Stream(device=dev)
    nsamp = 32
    samp = torch.zeros(4 * nsamp, dtype=torch.int64, device=dev)
    marks = torch.zeros(8, dtype=torch.int64, device=dev)
    assert probe.ssd_probe_clock(1, nsamp, samp.data_ptr(), side.cuda_stream) == 0   # (first use of the stream)
    torch.cuda.synchronize()
    first = torch.cuda.Event()
    assert probe.ssd_probe_clock(1, 1, marks.data_ptr(), sp) == 0
    walk()
    first.record(stream)
    for _ in range(4):
        walk()
    assert probe.ssd_probe_clock(1, 1, marks.data_ptr() + 32, sp) == 0
    # the sampler starts when the first walk launch has ended, during the second
    side.wait_event(first)
    assert probe.ssd_probe_clock(3000, nsamp, samp.data_ptr(), side.cuda_stream) == 0
    torch.cuda.synchronize()
    sv, mv = samp.cpu().numpy(), marks.cpu().numpy()
    t = sv.reshape(-1, 4)
    inside = bool(t[:, 1].min() >= mv[3] and t[:, 3].max() <= mv[5])
    log(f"[bench] clock sampler: starts {(t[:, 1].min() - mv[3]) / 100:.1f} us after the walks' first marker, "
        f"ends {(mv[5] - t[:, 3].max()) / 100:.1f} us before their last; walks span {(mv[5] - mv[3]) / 100:.1f} us")
    walk_clk = float(np.mean(clocks_mhz(sv))) if inside else None
    return {"walk_clock_mhz": None if walk_clk is None else round(walk_clk, 0),
            "walk_clock_window_inside_walks": inside}


def run_report_mode(args):
    """One JSON line per workload configuration (the measurement table of the layer)."""
    import numpy as np
    import torch

    import mamba_ssd_scan_forward_amd as ssd
    from workloads import CONFIGS, workload_inputs

    names = [args.workload] if args.workload else list(CONFIGS)
    dev = torch.device("cuda", 0)
    measured = measure_peaks(torch.cuda.current_stream(dev), dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    steps = max(args.steps, 1)
    for name in names:
        w = CONFIGS[name]
        inp = workload_inputs(w)
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        es = 2 if w.dtype == "bf16" else 4
        X = torch.from_numpy(inp.X).to(dt).to(dev)
        logA = torch.from_numpy(inp.logA).to(dev)
        B = torch.from_numpy(inp.B).to(dt).to(dev)
        C = torch.from_numpy(inp.C).to(dt).to(dev)
        init = None if inp.init is None else torch.from_numpy(inp.init).to(dev)
        off = None if inp.seq_offsets is None else torch.from_numpy(inp.seq_offsets).to(dev)
        nseq = w.nseq if w.varlen else w.batch
        prob = ssd.problem_for(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_len,
                               nseq, ssd.SSD_DTYPE_BF16 if w.dtype == "bf16" else ssd.SSD_DTYPE_F32)
        wsb = ssd.ssd_workspace_bytes(prob)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
        Y = torch.empty_like(X)
        final = torch.empty((nseq, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device=dev)
        stream = torch.cuda.current_stream(dev)
        ptrs = [X.data_ptr(), logA.data_ptr(), B.data_ptr(), C.data_ptr(),
                None if init is None else init.data_ptr(), None if off is None else off.data_ptr(),
                Y.data_ptr(), final.data_ptr(), ws.data_ptr(), wsb, stream.cuda_stream]

        def step():
            rc = ssd.ssd_forward(prob, *ptrs)
            if rc != 0:
                raise ssd.SsdError(rc)

        def timed(cold):
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(steps)]
            for i, (a, b) in enumerate(evs):
                if cold:
                    flush_by_reading(flush)
                a.record(stream)
                step()
                b.record(stream)
            torch.cuda.synchronize()
            return statistics.median(a.elapsed_time(b) * 1e3 for a, b in evs)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        warm_us = timed(False)
        cold_us = timed(True)

        lens = [w.seqlen] * w.batch if not w.varlen else [int(v) for v in np.diff(inp.seq_offsets)]
        cl = chunk_lengths(w, lens)
        fp, fc = flops_pages(w, cl), flops_causal(w, cl)
        abytes = algorithmic_bytes(w, es)
        peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
        t_roof = max(fp / (peak * 1e12), abytes / (HBM_PEAK_GBS * 1e9)) * 1e6
        tokens = w.batch * w.seqlen
        line = {
            "workload": name, "config": w.shape_dict(), "chunk_len": w.chunk_len,
            "time_us": round(cold_us, 2), "time_us_warm": round(warm_us, 2),
            "timing": f"median of {steps} HIP-event-timed steps; 'time_us' with a 512 MiB buffer read "
                      f"before each step (evicts the inputs from the 256 MB last-level cache and leaves "
                      f"it holding clean lines), 'time_us_warm' back to back",
            "tokens_per_s": round(tokens / (cold_us * 1e-6), 1),
            "tokens_per_s_warm": round(tokens / (warm_us * 1e-6), 1),
            "gflop_pages": round(fp / 1e9, 3), "gflop_causal": round(fc / 1e9, 3),
            "tflops_pages": round(fp / (cold_us * 1e-6) / 1e12, 2),
            "tflops_causal": round(fc / (cold_us * 1e-6) / 1e12, 2),
            "frac_mfma_peak": round(fp / (cold_us * 1e-6) / 1e12 / peak, 4),
            "mfma_peak_tflops": peak,
            "algorithmic_bytes": abytes,
            # a problem whose roofline time is below a couple of microseconds is bound by
            # launch and dependency latency, not by either unit
            "bound": ("latency" if t_roof < 2.0 else
                      "hbm" if abytes / (HBM_PEAK_GBS * 1e9) >= fp / (peak * 1e12) else "mfma"),
            "roofline_us": round(t_roof, 2),
            "frac_roofline": round(t_roof / cold_us, 4),
            "frac_roofline_warm": round(t_roof / warm_us, 4),
        }
        # the same against the rates this chip reaches (bf16 MFMA and a device copy)
        mm = measured["mfma_bf16_tflops"] if w.dtype == "bf16" else peak
        t_meas = max(fp / (mm * 1e12), abytes / (measured["hbm_copy_gbs"] * 1e9)) * 1e6
        line["measured_peaks"] = measured
        line["frac_mfma_measured"] = round(fp / (cold_us * 1e-6) / 1e12 / mm, 4)
        line["roofline_us_measured"] = round(t_meas, 2)
        line["frac_roofline_measured"] = round(t_meas / cold_us, 4)
        if w.varlen:
            line["seq_lengths"] = lens
        print(json.dumps(line), flush=True)
        del X, B, C, Y, final, ws, init, off
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # (the chip takes a few hundred steps, some tens of milliseconds, to reach its steady
    # clocks from idle: the first tens of steps run up to 20% slower)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-machine", action="store_true",
                    help="skip the machine measurements (MFMA rate, copy bandwidth, clocks)")
    ap.add_argument("--mode", default="bench", choices=["bench", "copy", "report"])
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the single-GPU hot path only; run it with --gpus 1 "
              "(multi-GPU sharding of the SSD layer is designed, not built).", file=sys.stderr)
        sys.exit(2)
    if args.mode == "copy":
        run_copy_mode(args.steps)
        return
    if args.mode == "report":
        run_report_mode(args)
        return

    import numpy as np
    import torch

    import mamba_ssd_scan_forward_amd as ssd
    from workloads import CONFIGS, HEADLINE, workload_inputs

    name = args.workload or HEADLINE
    w = CONFIGS[name]
    t0 = time.time()
    inp = workload_inputs(w)
    log(f"[bench] {name}: inputs drawn in {time.time() - t0:.1f}s")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    es = 2 if w.dtype == "bf16" else 4
    dev = torch.device("cuda", 0)
    X = torch.from_numpy(inp.X).to(dt).to(dev)
    logA = torch.from_numpy(inp.logA).to(dev)
    B = torch.from_numpy(inp.B).to(dt).to(dev)
    C = torch.from_numpy(inp.C).to(dt).to(dev)
    init = None if inp.init is None else torch.from_numpy(inp.init).to(dev)
    off = None if inp.seq_offsets is None else torch.from_numpy(inp.seq_offsets).to(dev)
    nseq = w.nseq if w.varlen else w.batch
    prob = ssd.problem_for(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_len,
                           nseq, ssd.SSD_DTYPE_BF16 if w.dtype == "bf16" else ssd.SSD_DTYPE_F32)
    wsb = ssd.ssd_workspace_bytes(prob)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    Y = torch.empty_like(X)
    final = torch.empty((nseq, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    ptrs = [X.data_ptr(), logA.data_ptr(), B.data_ptr(), C.data_ptr(),
            None if init is None else init.data_ptr(), None if off is None else off.data_ptr(),
            Y.data_ptr(), final.data_ptr(), ws.data_ptr(), wsb, sp]

    def step():
        rc = ssd.ssd_forward(prob, *ptrs)
        if rc != 0:
            raise ssd.SsdError(rc)

    def stage(k):
        rc = ssd.ssd_forward_stage(k, prob, *ptrs)
        if rc != 0:
            raise ssd.SsdError(rc, f"ssd_forward_stage({k})")

    plan = ssd.ssd_plan_describe(prob)
    log(f"[bench] plan {plan}")
    # warm-up: the requested steps, then more until the chip has run for MIN_WARM_S (it
    # takes a few hundred steps, some tens of milliseconds, to reach its steady clocks)
    t0 = time.perf_counter()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    warm_steps = args.warmup
    while time.perf_counter() - t0 < MIN_WARM_S:
        for _ in range(50):
            step()
        torch.cuda.synchronize()
        warm_steps += 50
    warm_s = time.perf_counter() - t0
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # cold: each step after a 512 MiB read that evicts the inputs from the last-level cache
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flush.fill_(1)
    n_cold = max(5, min(args.steps, 30))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_cold)]
    for a_, b_ in evs:
        flush_by_reading(flush)
        a_.record(stream)
        step()
        b_.record(stream)
    torch.cuda.synchronize()
    cold_ms = statistics.median(a_.elapsed_time(b_) for a_, b_ in evs)
    del flush

    # each launch alone, on the same stream, same events
    stage_ms = {}
    for k in (1, 2):
        for _ in range(max(2, args.warmup // 2)):
            stage(k)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            stage(k)
        e1.record(stream)
        torch.cuda.synchronize()
        stage_ms[k] = e0.elapsed_time(e1) / args.steps
    # the walk launch's own duration inside whole steps (prep, then walk): an event after
    # each stage, so the interval covers the walk from the prep's end to its own last
    # workgroup (what a kernel trace reports per launch; back to back, as above, the tail
    # of one walk launch overlaps the start of the next)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a_, b_ in ev:
        stage(1)
        a_.record(stream)
        stage(2)
        b_.record(stream)
    torch.cuda.synchronize()
    walk_in_step_ms = statistics.mean(a_.elapsed_time(b_) for a_, b_ in ev)
    log(f"[bench] step {ms_step * 1e3:.1f} us warm ({warm_steps} warm-up steps, {warm_s:.2f} s), "
        f"{cold_ms * 1e3:.1f} us cold; prep {stage_ms[1] * 1e3:.1f} us; "
        f"walk {stage_ms[2] * 1e3:.1f} us back to back, {walk_in_step_ms * 1e3:.1f} us per launch in steps")

    # the recurrent decode step (one token per sequence, state updated in place) at the
    # same sequences, heads and sizes; HBM-bound on the float32 state
    dec = None
    if not args.no_decode:
        g = torch.Generator(device="cpu").manual_seed(5)
        H_, P_, N_, G_ = w.nheads, w.headdim, w.dstate, w.ngroups
        xd = torch.randn(nseq, H_, P_, generator=g).to(dt).to(dev)
        ld = (-torch.rand(nseq, H_, generator=g) * 0.5).to(dev)
        Bd = (torch.randn(nseq, G_, N_, generator=g) / N_ ** 0.5).to(dt).to(dev)
        Cd = (torch.randn(nseq, G_, N_, generator=g) / N_ ** 0.5).to(dt).to(dev)
        Sd = torch.zeros(nseq, H_, P_, N_, dtype=torch.float32, device=dev)
        yd = torch.empty_like(xd)
        dprob = ssd.problem_for(nseq, 1, H_, P_, N_, G_, w.chunk_len, nseq, prob.dtype)
        dptr = [xd.data_ptr(), ld.data_ptr(), Bd.data_ptr(), Cd.data_ptr(), Sd.data_ptr(), yd.data_ptr(), sp]
        for _ in range(10):
            assert ssd.ssd_decode_step(dprob, *dptr) == 0
        torch.cuda.synchronize()
        nd = 200
        e0.record(stream)
        for _ in range(nd):
            ssd.ssd_decode_step(dprob, *dptr)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / nd
        dbytes = 2 * nseq * H_ * P_ * N_ * 4 + 2 * nseq * H_ * P_ * es + 2 * nseq * G_ * N_ * es + nseq * H_ * 4
        dec = {"kernel": "ssd_decode_kernel", "us_per_step": round(us, 2),
               "tokens_per_s": round(nseq / (us * 1e-6), 1),
               "bytes_per_step": dbytes, "achieved_gbs": round(dbytes / (us * 1e-6) / 1e9, 1),
               "frac_hbm": round(dbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"[bench] decode step {us:.2f} us, {dec['achieved_gbs']} GB/s")

    # the backward pass of the same workload (gradients of <dY, Y> + <dF, final>), all
    # buffers and the workspace allocated before the timed region
    bwd = None
    if not args.no_backward:
        g = torch.Generator(device="cpu").manual_seed(6)
        dYb = torch.randn(Y.shape, generator=g).to(dt).to(dev)
        dFb = torch.randn(final.shape, generator=g).to(dev)
        outs = [torch.empty_like(X), torch.empty_like(logA), torch.empty_like(B), torch.empty_like(C),
                torch.empty_like(final)]
        bwsb = ssd.ssd_backward_workspace_bytes(prob)
        bws = torch.empty(bwsb, dtype=torch.uint8, device=dev)
        bptr = [X.data_ptr(), logA.data_ptr(), B.data_ptr(), C.data_ptr(),
                None if init is None else init.data_ptr(), None if off is None else off.data_ptr(),
                Y.data_ptr(), final.data_ptr(), dYb.data_ptr(), dFb.data_ptr()] + [o.data_ptr() for o in outs] + \
               [bws.data_ptr(), bwsb, sp]
        for _ in range(2):
            assert ssd.ssd_backward(prob, *bptr) == 0
        torch.cuda.synchronize()
        nb = max(3, args.steps // 5)
        e0.record(stream)
        for _ in range(nb):
            ssd.ssd_backward(prob, *bptr)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / nb
        bwd = {"us_per_step": round(us, 1), "tokens_per_s": round(w.batch * w.seqlen / (us * 1e-6), 1),
               "vs_forward_step": round(us / (ms_step * 1e3), 2)}
        log(f"[bench] backward {us:.1f} us")
        del outs, bws

    machine = None
    if not args.no_machine:
        machine = measure_machine(lambda: stage(2), stream, dev)
        log(f"[bench] machine: {machine}")

    lens = [w.seqlen] * w.batch if not w.varlen else [int(v) for v in np.diff(inp.seq_offsets)]
    tokens = w.batch * w.seqlen
    cl = chunk_lengths(w, lens)
    fl, fc = flops_pages(w, cl), flops_causal(w, cl)
    fx = executed_mfma_flops(plan, w, lens)
    abytes = algorithmic_bytes(w, es)
    tok_s = tokens / (ms_step * 1e-3)
    peak_mm = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
    # the walk's launches back to back on its stream, HIP events around the whole run (as the
    # timed steps run it; an event recorded between launches slows the launch after it, by
    # up to a third in a kernel trace, so the per-launch figure is reported beside it only)
    achieved_gbs = abytes / (stage_ms[2] * 1e-3) / 1e9
    t_roof_ms = max(fl / (peak_mm * 1e12), abytes / (HBM_PEAK_GBS * 1e9)) * 1e3

    traffic = None
    if os.path.exists(COUNTERS_JSON):
        try:
            c = json.load(open(COUNTERS_JSON))
            if c.get("kernel_source_hash") == kernel_source_hash() and c.get("workload") == name:
                traffic = c.get("hbm_bytes_per_launch")
        except (OSError, ValueError):
            traffic = None

    result = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded: X~N(0,1), B,C~N(0,1/N), logA=-U[.001,.1]*U[1,16])",
        "config": dict(workload=name, **w.shape_dict()),
        "warmup_run": {"steps": warm_steps, "seconds": round(warm_s, 3), "min_seconds": MIN_WARM_S,
                       "note": "the requested warm-up steps, then more until the chip had run for min_seconds"},
        "cold": {"ms_per_step": round(cold_ms, 5), "tokens_per_s": round(tokens / (cold_ms * 1e-3), 1),
                 "steps": n_cold, "timing": "median of per-step HIP-event times, a 512 MiB buffer read "
                                            "before each step (inputs evicted from the 256 MB last-level cache)"},
        "tflops_pages": round(fl / (ms_step * 1e-3) / 1e12, 2),
        "tflops_causal": round(fc / (ms_step * 1e-3) / 1e12, 2),
        "mfma_util_pages": round(fl / (ms_step * 1e-3) / 1e12 / peak_mm, 4),
        "mfma_util_causal": round(fc / (ms_step * 1e-3) / 1e12 / peak_mm, 4),
        "mfma_util_executed": None if fx is None else round(fx / (ms_step * 1e-3) / 1e12 / peak_mm, 4),
        "mfma_util_note": "pages: the block decomposition's products as the pages count them (dense QxQ "
                          "diagonal blocks, the figure the 0.40 target is stated in); causal: their lower "
                          "halves; executed: the MFMA instructions the kernel issues",
        "plan": plan,
        "stage_us": {"prep": round(stage_ms[1] * 1e3, 2), "walk": round(stage_ms[2] * 1e3, 2),
                     "walk_per_launch_in_steps": round(walk_in_step_ms * 1e3, 2),
                     "note": "walk: the walk launches back to back (the roofline's figure); "
                             "walk_per_launch_in_steps: a stage-1 launch and an event pair around each "
                             "walk launch (events between launches slow the launches down)"},
        "roofline": {
            "kernel": plan["walk"],
            "bound": "hbm",
            "achieved": round(achieved_gbs, 1),
            "kernel_us": round(stage_ms[2] * 1e3, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes": abytes,
            "step_frac": round(t_roof_ms / ms_step, 4),
            "step_frac_cold": round(t_roof_ms / cold_ms, 4),
        },
        "pages_context": PAGES_CONTEXT,
    }

    if machine is not None:
        # the same rates against what the chip reaches: the walk's FLOPs per launch over
        # the measured dense bf16 rate, its clock against the clock under that rate
        machine["walk_tflops_pages"] = round(fl / (stage_ms[2] * 1e-3) / 1e12, 1)
        machine["walk_frac_of_measured_mfma"] = round(machine["walk_tflops_pages"] / machine["mfma_bf16_tflops"], 4)
        machine["walk_frac_of_measured_copy"] = round(achieved_gbs / machine["hbm_copy_gbs"], 4)
        result["measured_peaks"] = machine
    if dec is not None:
        result["decode"] = dec
    if bwd is not None:
        result["backward"] = bwd

    if not args.no_cpu_baseline:
        import oracle
        x64 = [np.asarray(a, dtype=np.float64) for a in (inp.X, inp.logA, inp.B, inp.C)]
        i64 = None if inp.init is None else inp.init.astype(np.float64)
        # every core this process may run on (sched_getaffinity), no more than the OpenMP
        # thread limit of the environment when one is set
        affinity = len(os.sched_getaffinity(0))
        nthr = min(affinity, oracle.threads()) if os.environ.get("OMP_NUM_THREADS") else affinity
        oracle.recurrence(*[a[:, :64] for a in x64], None if i64 is None else i64, None, nthreads=nthr)  # warm
        # whole passes over the workload until about 10 s of CPU work have run
        times = []
        while len(times) < 3 or (sum(times) < 10.0 and len(times) < 200):
            t0 = time.perf_counter()
            oracle.recurrence(*x64, i64, inp.seq_offsets, nthreads=nthr)
            times.append(time.perf_counter() - t0)
        t = statistics.median(times)
        result["cpu_baseline"] = {
            "value": round(tokens / t, 1),
            "unit": "tokens/s",
            "cores": nthr,
            "affinity_cores": affinity,
            "kind": "oracle",
            "sample": f"whole workload ({tokens} tokens, all {w.nheads} heads), float64 "
                      f"recurrence on {nthr} threads, median of {len(times)} passes ({t:.2f}s each, "
                      f"{sum(times):.1f}s in all)",
        }
        log(f"[bench] oracle {t:.2f}s on {nthr} threads ({affinity} cores in the affinity mask)")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
