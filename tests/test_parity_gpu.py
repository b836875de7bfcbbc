"""GPU parity of the HIP path against the float64 oracle (needs an MI355X).

Metric, for Y and for the final state: max|out - ref| / max|ref| with ref the oracle's
unrounded float64 result on the same (already quantized) inputs.  Bars:
  float32 inputs  <= 1e-4
  bfloat16 inputs <= 2e-2 (fp32 accumulation)
Small cases compare every element; the five workload configurations run at full size in
the launch configuration the benchmark times and are compared on every element too.
"""
import os
import sys

import numpy as np
import pytest

import oracle
from workloads import CONFIGS, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def dev(inp):
    torch = _torch()
    dt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    d = {
        "X": torch.from_numpy(inp.X).to(dt).cuda(),
        "logA": torch.from_numpy(inp.logA).cuda(),
        "B": torch.from_numpy(inp.B).to(dt).cuda(),
        "C": torch.from_numpy(inp.C).to(dt).cuda(),
        "init": None if inp.init is None else torch.from_numpy(inp.init).cuda(),
        "off": None if inp.seq_offsets is None else torch.from_numpy(inp.seq_offsets).cuda(),
    }
    return d


def run_gpu(inp, Q, d=None):
    import mamba_ssd_scan_forward_amd as ssd
    torch = _torch()
    d = d or dev(inp)
    Y, F = ssd.forward(d["X"], d["logA"], d["B"], d["C"], Q, d["init"], d["off"])
    torch.cuda.synchronize()
    return Y.float().cpu().numpy().astype(np.float64), F.cpu().numpy().astype(np.float64)


def rel_err(out, ref):
    den = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(out - ref))) / max(den, 1e-30)


def plan_of(inp, Q):
    """The kernels the library plans for this input (host logic, no device work)."""
    import mamba_ssd_scan_forward_amd as ssd
    b, T, H, P = inp.X.shape
    G, N = inp.B.shape[2], inp.B.shape[3]
    nseq = b if inp.seq_offsets is None else len(inp.seq_offsets) - 1
    dt = ssd.SSD_DTYPE_BF16 if inp.dtype == "bf16" else ssd.SSD_DTYPE_F32
    return ssd.ssd_plan_describe(ssd.problem_for(b, T, H, P, N, G, Q, nseq, dt))


def check(inp, Q, label=""):
    print(f"[parity] {label} X{tuple(inp.X.shape)} G={inp.B.shape[2]} N={inp.B.shape[3]} "
          f"Q={Q} {inp.dtype} init={inp.init is not None} varlen={inp.seq_offsets is not None} "
          f"walk={plan_of(inp, Q)['walk']}", flush=True)
    Y, F = run_gpu(inp, Q)
    Yr, Fr = oracle.recurrence(inp.X, inp.logA, inp.B, inp.C, inp.init, inp.seq_offsets)
    ey, ef = rel_err(Y, Yr), rel_err(F, Fr)
    print(f"[parity]   err Y {ey:.3e}  final {ef:.3e}", flush=True)
    assert np.all(np.isfinite(Y)) and np.all(np.isfinite(F))
    assert ey <= TOL[inp.dtype], ey
    assert ef <= TOL[inp.dtype], ef
    return Y, F


def test_cfg0_tiny_fp32_full():
    w = CONFIGS["cfg0_tiny_f32"]
    check(workload_inputs(w), w.chunk_len, w.name)


@pytest.mark.parametrize("Q", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("init", [False, True])
def test_bf16_chunk_sweep_ragged(Q, init):
    inp = make_inputs(2, 300, 4, 64, 128, 2, "bf16", seed=100 + Q, init_state=init)
    check(inp, Q, "bf16 ragged")


@pytest.mark.parametrize("Q", [32, 64, 256])
def test_fp32_ragged(Q):
    inp = make_inputs(2, 200, 3, 32, 64, 1, "f32", seed=200 + Q, init_state=True)
    check(inp, Q, "fp32 ragged")


@pytest.mark.parametrize("P,N", [(16, 16), (32, 32), (48, 80), (64, 64), (128, 128), (64, 256),
                                 (256, 32)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_head_and_state_sizes(P, N, dtype):
    inp = make_inputs(1, 130, 2, P, N, 1, dtype, seed=300 + P + N, init_state=True)
    check(inp, 64, "sizes")


def test_varlen_ragged_with_empty_and_short_sequences():
    lens = [5, 0, 300, 1, 64, 129, 33]
    inp = make_inputs(1, sum(lens), 4, 64, 128, 2, "bf16", seed=400, init_state=True,
                      seq_lengths=lens)
    Y, F = check(inp, 64, "varlen")
    # the empty sequence returns its initial state unchanged
    np.testing.assert_array_equal(F[1], inp.init[1].astype(np.float64))


def test_a_one_linear_attention():
    inp = make_inputs(1, 200, 2, 64, 64, 1, "f32", seed=500, init_state=True)
    inp.logA[:] = 0.0
    check(inp, 64, "a=1")


def test_a_zero_via_length_one_sequences():
    """Every token its own sequence, zero initial state: y_t = (C_t . B_t) x_t, the a = 0
    closed form, reached exactly through sequence boundaries."""
    T = 70
    inp = make_inputs(1, T, 2, 32, 32, 1, "f32", seed=600, seq_lengths=[1] * T)
    Y, F = check(inp, 32, "a=0")
    cb = np.einsum("tn,tn->t", inp.C[0, :, 0].astype(np.float64), inp.B[0, :, 0].astype(np.float64))
    np.testing.assert_allclose(Y[0], cb[:, None, None] * inp.X[0].astype(np.float64), rtol=1e-4, atol=1e-5)


def test_strong_decay_is_finite():
    """logA down to -1e4: every off-diagonal term underflows to zero, nothing overflows."""
    inp = make_inputs(1, 256, 2, 64, 128, 1, "bf16", seed=700)
    inp.logA[:] = -1e4
    check(inp, 128, "strong decay")


def test_split_resume_matches_full_run():
    inp = make_inputs(2, 512, 4, 64, 128, 1, "bf16", seed=800, init_state=True)
    Y, F = run_gpu(inp, 256)
    split = 200
    import copy
    a = copy.deepcopy(inp)
    a.X, a.logA, a.B, a.C = inp.X[:, :split], inp.logA[:, :split], inp.B[:, :split], inp.C[:, :split]
    Y1, F1 = run_gpu(a, 256)
    b = copy.deepcopy(inp)
    b.X, b.logA, b.B, b.C = inp.X[:, split:], inp.logA[:, split:], inp.B[:, split:], inp.C[:, split:]
    b.init = F1.astype(np.float32)
    Y2, F2 = run_gpu(b, 256)
    assert rel_err(np.concatenate([Y1, Y2], axis=1), Y) <= 2e-2
    assert rel_err(F2, F) <= 2e-2


def test_bitwise_repeatable():
    inp = make_inputs(2, 700, 4, 64, 128, 2, "bf16", seed=900, init_state=True)
    d = dev(inp)
    Y1, F1 = run_gpu(inp, 256, d)
    Y2, F2 = run_gpu(inp, 256, d)
    np.testing.assert_array_equal(Y1, Y2)
    np.testing.assert_array_equal(F1, F2)


# The common layer shapes (bf16, 256-row chunks, d_state 64 or 128, head dimension a
# multiple of 64) run on their own walker; these cases reach its edges.
@pytest.mark.parametrize("case", ["varlen", "varlen_ties", "strong_decay", "mixed_decay", "headdim128",
                                  "one_chunk_n64", "a_one", "state256", "state256_varlen",
                                  "state256_segmented"])
def test_layer_shape_walker_edges(case):
    if case.startswith("state256"):
        # d_state 256: two passes over the column halves of B, C and the state
        if case == "state256":
            inp = make_inputs(2, 600, 4, 64, 256, 2, "bf16", seed=1007, init_state=True)
        elif case == "state256_varlen":
            lens = [300, 0, 513, 7, 256, 90, 1, 44]
            inp = make_inputs(1, sum(lens), 2, 64, 256, 1, "bf16", seed=1008, init_state=True,
                              seq_lengths=lens)
        else:
            inp = make_inputs(1, 4200, 2, 128, 256, 2, "bf16", seed=1009, init_state=True)
        Y, F = check(inp, 256, case)
        if case == "state256_varlen":
            np.testing.assert_array_equal(F[1], inp.init[1].astype(np.float64))
    elif case == "varlen_ties":
        # packed sequences dealt to XCDs longest first: equal lengths, an empty one
        lens = [300, 300, 5, 0, 300, 77, 256, 1]
        inp = make_inputs(1, sum(lens), 3, 64, 128, 1, "bf16", seed=1006, init_state=True,
                          seq_lengths=lens)
        Y, F = check(inp, 256, case)
        np.testing.assert_array_equal(F[3], inp.init[3].astype(np.float64))
    elif case == "varlen":
        lens = [5, 0, 300, 1, 256, 257, 600, 33]
        inp = make_inputs(1, sum(lens), 4, 64, 128, 2, "bf16", seed=1000, init_state=True,
                          seq_lengths=lens)
        Y, F = check(inp, 256, case)
        np.testing.assert_array_equal(F[1], inp.init[1].astype(np.float64))
    elif case == "strong_decay":
        inp = make_inputs(1, 512, 2, 64, 128, 1, "bf16", seed=1001)
        inp.logA[:] = -1e4
        check(inp, 256, case)
    elif case == "mixed_decay":
        # ordinary decay with a few 32-row blocks whose decay span is huge (rows of
        # logA = -30 or -70), next to blocks where it is not, in every chunk
        inp = make_inputs(2, 700, 3, 64, 128, 1, "bf16", seed=1005, init_state=True)
        for t0 in (40, 300, 620):
            inp.logA[:, t0:t0 + 4, :] = -30.0
        inp.logA[:, 170, 1] = -70.0
        inp.logA[1, 455, :] = -70.0
        check(inp, 256, case)
    elif case == "headdim128":
        inp = make_inputs(2, 520, 3, 128, 64, 1, "bf16", seed=1002, init_state=True)
        check(inp, 256, case)
    elif case == "one_chunk_n64":
        inp = make_inputs(3, 256, 2, 64, 64, 2, "bf16", seed=1003)
        check(inp, 256, case)
    else:
        inp = make_inputs(1, 700, 2, 64, 128, 1, "bf16", seed=1004, init_state=True)
        inp.logA[:] = 0.0
        check(inp, 256, case)


# Few long sequences: each is walked as several segments of chunks (a first pass sums
# up every segment but the last; each segment then starts from the combined state).
# The plan picks the segment count from the number of (sequence, head, P tile) items and
# chunks (at least 8 chunks per segment): 2 here for 9 to 23 chunks, 3 for 24 or more.
@pytest.mark.parametrize("case", ["two_segments", "three_segments_mixed", "a_one", "strong_decay",
                                  "partial_tail"])
def test_segmented_walk(case):
    if case == "partial_tail":
        # 260 items (P = 128: two tiles per head): the first 256 walk whole, the last 4
        # in two segments each
        inp = make_inputs(2, 4096, 65, 128, 64, 1, "bf16", seed=1204, init_state=True)
    elif case == "two_segments":
        inp = make_inputs(2, 4100, 4, 64, 128, 2, "bf16", seed=1200, init_state=True)
    elif case == "three_segments_mixed":
        inp = make_inputs(1, 6200, 2, 128, 64, 1, "bf16", seed=1201, init_state=True)
        for t0 in (100, 2030, 4300):
            inp.logA[:, t0:t0 + 3, :] = -30.0
        inp.logA[0, 3800, 1] = -70.0
    elif case == "a_one":
        inp = make_inputs(1, 4096, 2, 64, 128, 1, "bf16", seed=1202, init_state=True)
        inp.logA[:] = 0.0
    else:
        inp = make_inputs(1, 4096, 2, 64, 64, 1, "bf16", seed=1203, init_state=True)
        inp.logA[:] = -1e4
    check(inp, 256, "segmented " + case)


def test_segmented_walk_matches_whole_walk():
    """The same sequence as a batch of one (segmented) and as one packed sequence
    (walked whole): both within the bar of each other."""
    import copy
    inp = make_inputs(1, 4200, 4, 64, 128, 1, "bf16", seed=1210, init_state=True)
    Y1, F1 = run_gpu(inp, 256)
    packed = copy.deepcopy(inp)
    packed.seq_offsets = np.array([0, 4200], dtype=np.int32)
    Y2, F2 = run_gpu(packed, 256)
    assert rel_err(Y1, Y2) <= 2e-2 and rel_err(F1, F2) <= 2e-2


FULL_SIZE = ["cfg1_mamba2_2.7b_bf16", "cfg2a_state64_bf16", "cfg2b_state256_bf16", "cfg3_long16k_bf16",
             "cfg4_varlen32k_bf16"]


@pytest.mark.parametrize("name", FULL_SIZE)
def test_full_size_config(name):
    """A whole workload configuration in the launch configuration the benchmark times,
    every token of every head against the oracle (C, float64, all host cores)."""
    w = CONFIGS[name]
    inp = workload_inputs(w)
    print(f"[parity] {name} full size", flush=True)
    Y, F = run_gpu(inp, w.chunk_len)
    assert np.all(np.isfinite(Y)) and np.all(np.isfinite(F))
    Yr, Fr = oracle.recurrence(inp.X, inp.logA, inp.B, inp.C, inp.init, inp.seq_offsets)
    ey, ef = rel_err(Y, Yr), rel_err(F, Fr)
    print(f"[parity]   {name}: max_rel_err_Y {ey:.3e} max_rel_err_final {ef:.3e}", flush=True)
    assert ey <= TOL[w.dtype] and ef <= TOL[w.dtype], (ey, ef)


# Shapes whose (sequence, group, NW units of 32 head columns) workgroups fill at least
# half of the chip, so the library walks them on the fused walker with the heads of a
# group sharing one load of B and C: ragged chunks with an initial state; d_state 64 with
# groups of five heads and of 14 heads (a group's last workgroup partly idle); a packed
# batch with empty and length-1 sequences (longest-first dealing); the same with groups of
# three heads; groups of two heads; strong decay, where most 32-row blocks take the
# exact-mask path, at two head counts.
@pytest.mark.parametrize("case", ["ragged_init", "state64_partial", "state64_four", "packed", "packed_three",
                                  "two_per_group", "strong_decay", "strong_decay_four"])
def test_group_shared_walker(case):
    if case == "ragged_init":
        inp = make_inputs(32, 300, 16, 64, 128, 1, "bf16", seed=1300, init_state=True)
    elif case == "state64_partial":
        inp = make_inputs(32, 520, 10, 64, 64, 2, "bf16", seed=1301, init_state=True)
    elif case == "state64_four":
        inp = make_inputs(64, 200, 14, 64, 64, 1, "bf16", seed=1304, init_state=True)
    elif case == "packed":
        lens = [1, 0, 300, 257, 5, 1200, 256, 31, 0, 700, 64, 129, 2, 500, 33, 522]
        inp = make_inputs(1, sum(lens), 80, 64, 128, 8, "bf16", seed=1302, init_state=True, seq_lengths=lens)
    elif case == "packed_three":
        lens = [1, 0, 300, 257, 5, 700, 256, 31, 0, 400, 64, 129, 2, 300, 33, 222]
        inp = make_inputs(1, sum(lens), 24, 64, 128, 8, "bf16", seed=1306, init_state=True, seq_lengths=lens)
    elif case == "two_per_group":
        inp = make_inputs(16, 260, 16, 64, 128, 8, "bf16", seed=1307, init_state=True)
    elif case == "strong_decay":
        inp = make_inputs(32, 300, 16, 64, 128, 1, "bf16", seed=1303, init_state=True)
        inp.logA = (inp.logA * 40.0).astype(np.float32)
    else:
        inp = make_inputs(64, 300, 14, 64, 128, 1, "bf16", seed=1305, init_state=True)
        inp.logA = (inp.logA * 40.0).astype(np.float32)
    assert plan_of(inp, 256)["walk"].startswith("ssd_walk_fused_kernel"), plan_of(inp, 256)
    check(inp, 256, case)


# The general walker with B staged in parts (fewer B rows than the padded chunk fit in
# LDS next to the rest): float32 with 256-row chunks at d_state 128, float32 with 128-row
# chunks at d_state 256, bfloat16 with 256-row chunks at head dimension 48 and d_state 256
# (C B^T tiles staged in LDS too); ragged last chunks, initial states, and one packed batch.
@pytest.mark.parametrize("case", ["f32_q256_n128", "f32_q128_n256", "bf16_q256_p48_n256", "f32_q256_n128_packed"])
def test_general_walker_staged_b(case):
    if case == "f32_q256_n128":
        inp, Q = make_inputs(2, 700, 4, 64, 128, 2, "f32", seed=1400, init_state=True), 256
    elif case == "f32_q128_n256":
        inp, Q = make_inputs(2, 300, 4, 64, 256, 2, "f32", seed=1401, init_state=True), 128
    elif case == "bf16_q256_p48_n256":
        inp, Q = make_inputs(2, 600, 4, 48, 256, 2, "bf16", seed=1402, init_state=True), 256
    else:
        lens = [300, 0, 1, 257, 142]
        inp, Q = make_inputs(1, sum(lens), 4, 64, 128, 2, "f32", seed=1403, init_state=True, seq_lengths=lens), 256
    walk = plan_of(inp, Q)["walk"]
    qb, qp = (int(v) for v in walk.split("qb=")[1].split("/"))
    assert walk.startswith("ssd_walk_kernel<") and qb < qp, walk
    check(inp, Q, case)


def test_library_loaded_before_the_first_gpu_use():
    """The library loaded before anything touches the GPU (here: before torch is imported)
    still runs: the binding makes it share PyTorch's HIP runtime instead of holding a
    second one that finds no device.  In a fresh process, since the order of loading is
    what is tested."""
    import subprocess
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import mamba_ssd_scan_forward_amd as ssd\n"
            "ssd.load_library()\n"
            "import torch\n"
            "from workloads import CONFIGS, workload_inputs\n"
            "inp = workload_inputs(CONFIGS['cfg0_tiny_f32'])\n"
            "d = [torch.from_numpy(a).cuda() for a in (inp.X, inp.logA, inp.B, inp.C)]\n"
            "Y, F = ssd.forward(*d, 64)\n"
            "torch.cuda.synchronize()\n"
            "print('ok', float(Y.abs().max()))\n") % os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=100)
    assert res.returncode == 0 and "ok" in res.stdout, res.stdout + res.stderr


# Sequences walked as segments by the fused walker (a summary of every segment but the
# last, their entry states chained, then every segment walked on its own): ragged lengths
# (a short last segment and a ragged last block) with initial states, one and several
# groups, d_state 64 and 128, head dimension 128, a batch of two, strong decay (blocks
# that renormalise or take the exact form inside segments), and one packed sequence given
# through seq_offsets.
@pytest.mark.parametrize("case", ["n128_init", "groups2", "n64_batch2", "groups3", "p128", "strong_decay",
                                  "a_one", "a_zero", "packed_one", "weak_decay", "many_segments"])
def test_segmented_fused_walk(case):
    if case == "n128_init":
        inp = make_inputs(1, 8292, 16, 64, 128, 1, "bf16", seed=1500, init_state=True)
    elif case == "groups2":
        inp = make_inputs(1, 8292, 16, 64, 128, 2, "bf16", seed=1501, init_state=True)
    elif case == "n64_batch2":
        inp = make_inputs(2, 4160, 16, 64, 64, 1, "bf16", seed=1502, init_state=True)
    elif case == "groups3":
        inp = make_inputs(1, 6000, 24, 64, 128, 3, "bf16", seed=1503, init_state=False)
    elif case == "p128":
        inp = make_inputs(1, 9000, 8, 128, 128, 1, "bf16", seed=1504, init_state=True)
    elif case == "strong_decay":
        inp = make_inputs(1, 8292, 16, 64, 128, 1, "bf16", seed=1505, init_state=True)
        inp.logA = (inp.logA * 40.0).astype(np.float32)
    elif case == "a_one":
        # no decay: every segment's summary weights are 1 and its total decay exp(0)
        inp = make_inputs(1, 8292, 16, 64, 128, 1, "bf16", seed=1507, init_state=True)
        inp.logA[:] = 0.0
    elif case == "a_zero":
        # total decay: every state is forgotten at once (weights and totals underflow to 0)
        inp = make_inputs(1, 8292, 16, 64, 64, 1, "bf16", seed=1508, init_state=True)
        inp.logA[:] = -1e4
    elif case == "weak_decay":
        # 29 segments (the entry states by the associative scan over segments) with decays
        # weak enough that each segment's entry state carries the earlier ones
        inp = make_inputs(1, 8292, 16, 64, 128, 1, "bf16", seed=1509, init_state=True)
        inp.logA = (inp.logA * 0.01).astype(np.float32)
    elif case == "many_segments":
        # 64 segments of 1024 rows: the scan in four passes of 16 segments, each carrying
        # the last entry state of the one before
        inp = make_inputs(1, 65536, 8, 64, 128, 1, "bf16", seed=1510, init_state=True)
        inp.logA = (inp.logA * 0.01).astype(np.float32)
    else:
        inp = make_inputs(1, 8292, 16, 64, 128, 1, "bf16", seed=1506, init_state=True, seq_lengths=[8292])
    plan = plan_of(inp, 256)
    assert plan["walk"].startswith("ssd_walk_fused_kernel") and plan["summary"].startswith("ssd_seg_summary"), plan
    if case in ("weak_decay", "many_segments", "a_one"):
        assert plan["summary"].endswith("ssd_seg_scan_kernel"), plan
    check(inp, 256, case)


# d_state 256 on the fused walker (two or three compute waves, three ring slots), where
# the workgroups fill the chip without segments: a batch of ragged sequences with initial
# states (two compute waves), one where three waves take fewer rounds, a packed batch with
# empty and length-1 sequences and two groups (three waves: the fewest workgroups), strong
# decay.  Long sequences that would need segments take the two passes over the column
# halves of the state instead (ordinary and strong decay).
@pytest.mark.parametrize("case", ["batch_init", "three_waves", "packed_groups2", "strong_decay", "long",
                                  "long_strong_decay"])
def test_fused_walker_state256(case):
    if case == "batch_init":
        inp, nw = make_inputs(32, 300, 8, 64, 256, 1, "bf16", seed=1600, init_state=True), 2
    elif case == "three_waves":
        inp, nw = make_inputs(48, 300, 6, 64, 256, 1, "bf16", seed=1601, init_state=True), 3
    elif case == "packed_groups2":
        lens = [1, 0, 300, 257, 5, 600, 256, 31, 0, 400, 64, 129, 2, 300, 33, 222]
        inp, nw = make_inputs(1, sum(lens), 32, 64, 256, 2, "bf16", seed=1602, init_state=True,
                              seq_lengths=lens), 3
    elif case == "strong_decay":
        inp, nw = make_inputs(32, 300, 8, 64, 256, 1, "bf16", seed=1603, init_state=True), 2
        inp.logA = (inp.logA * 40.0).astype(np.float32)
    elif case == "long":
        inp, nw = make_inputs(1, 8292, 16, 64, 256, 1, "bf16", seed=1604, init_state=True), 0
    else:
        inp, nw = make_inputs(1, 8292, 16, 64, 256, 1, "bf16", seed=1605, init_state=True), 0
        inp.logA = (inp.logA * 40.0).astype(np.float32)
    plan = plan_of(inp, 256)
    if nw:
        assert plan["walk"] == f"ssd_walk_fused_kernel<256, {nw}>" and plan["summary"] == "none", plan
    else:
        assert plan["walk"].startswith("ssd_walk_split_pair_kernel"), plan
    Y, F = check(inp, 256, case)
    if case == "packed_groups2":
        np.testing.assert_array_equal(F[1], inp.init[1].astype(np.float64))


def test_fused_walker_result_does_not_depend_on_chunk_len():
    """The block decomposition gives the same product for any chunking (paper summary page,
    section 6); the fused walker passes the state between 32-row blocks whatever chunk_len
    says, so every valid chunk length gives the same bits."""
    inp = make_inputs(32, 300, 16, 64, 128, 1, "bf16", seed=1700, init_state=True)
    for q in (16, 64, 256):
        assert plan_of(inp, q)["walk"] == "ssd_walk_fused_kernel<128, 4>", plan_of(inp, q)
    d = dev(inp)
    Y0, F0 = run_gpu(inp, 256, d)
    for q in (16, 64):
        Y, F = run_gpu(inp, q, d)
        np.testing.assert_array_equal(Y, Y0)
        np.testing.assert_array_equal(F, F0)
    check(inp, 64, "chunk_len 64")
