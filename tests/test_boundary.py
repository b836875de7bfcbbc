"""The C-ABI boundary without a GPU: the library loads, exports every symbol that
include/ssd.h declares, sizes workspaces, and rejects bad arguments on the host
before anything is enqueued (no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import mamba_ssd_scan_forward_amd as ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ssd.lib_path()),
                                reason="libssd.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(["ssd_abi_version", "ssd_backward", "ssd_backward_workspace_bytes",
                                           "ssd_check_problem", "ssd_decode_step", "ssd_forward", "ssd_forward_noalloc",
                                           "ssd_forward_stage", "ssd_plan_describe", "ssd_status_string",
                                           "ssd_workspace_bytes"])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(ssd.lib_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


PROBE_HEADER = os.path.join(ROOT, "include", "ssd_probe.h")


def test_probe_library_exports_every_declared_symbol():
    """The machine measurements (include/ssd_probe.h) in their own library."""
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(ssd_[a-z_0-9]+)\s*\(", text)))
    assert names == ["ssd_probe_clock", "ssd_probe_device", "ssd_probe_mfma_bf16"]
    lib = ssd.load_probe_library()
    for name in names:
        assert hasattr(lib, name), name


def test_probe_rejects_bad_arguments():
    lib = ssd.load_probe_library()
    assert lib.ssd_probe_mfma_bf16(0, 1, 16, None) == -1
    assert lib.ssd_probe_mfma_bf16(1, 0, 16, None) == -1
    assert lib.ssd_probe_mfma_bf16(1, 1, None, None) == -1
    assert lib.ssd_probe_clock(1 << 25, 1, 16, None) == -1
    assert lib.ssd_probe_clock(1, 1, None, None) == -1


def test_abi_and_status_strings():
    assert ssd.ssd_abi_version() == ssd.ABI_VERSION
    for code in (0, -1, -2, -3, -4, -5):
        assert ssd.ssd_status_string(code)
    assert ssd.ssd_status_string(12345) == "unknown status"


def prob(**kw):
    d = dict(batch=2, seqlen=300, nheads=4, headdim=64, dstate=128, ngroups=2, chunk_len=64,
             nseq=2, dtype=ssd.SSD_DTYPE_BF16)
    d.update(kw)
    return ssd.problem_for(**d)


@pytest.mark.parametrize("kw,code", [
    ({}, ssd.SSD_OK),
    (dict(batch=0), ssd.SSD_ERR_INVALID_ARG),
    (dict(seqlen=0), ssd.SSD_ERR_INVALID_ARG),
    (dict(nheads=3), ssd.SSD_ERR_INVALID_ARG),           # H % G != 0
    (dict(nseq=0), ssd.SSD_ERR_INVALID_ARG),
    (dict(dtype=7), ssd.SSD_ERR_UNSUPPORTED),
    (dict(chunk_len=48), ssd.SSD_ERR_UNSUPPORTED),
    (dict(chunk_len=512), ssd.SSD_ERR_UNSUPPORTED),
    (dict(headdim=40), ssd.SSD_ERR_UNSUPPORTED),
    (dict(dstate=24), ssd.SSD_ERR_UNSUPPORTED),
    (dict(dstate=272), ssd.SSD_ERR_UNSUPPORTED),
    (dict(chunk_len=16, headdim=16, dstate=16, dtype=ssd.SSD_DTYPE_F32), ssd.SSD_OK),
    (dict(headdim=256, dstate=256, dtype=ssd.SSD_DTYPE_F32), ssd.SSD_OK),
])
def test_check_problem(kw, code):
    p = prob(**kw)
    assert ssd.ssd_check_problem(p) == code
    assert (ssd.ssd_workspace_bytes(p) > 0) == (code == ssd.SSD_OK)


def test_workspace_grows_with_problem():
    small = ssd.ssd_workspace_bytes(prob(seqlen=128))
    large = ssd.ssd_workspace_bytes(prob(seqlen=4096))
    assert 0 < small < large
    assert ssd.ssd_workspace_bytes(prob()) % 256 == 0


# Fake, aligned, non-overlapping addresses: every call below must fail validation on
# the host, so nothing is dereferenced and no kernel is launched.
GB = 1 << 30
ADDR = dict(X=1 * GB, logA=2 * GB, B=3 * GB, C=4 * GB, init=5 * GB, off=6 * GB, Y=7 * GB,
            final=8 * GB, ws=9 * GB)


def call(p, ws_bytes=None, **over):
    a = dict(ADDR)
    a.update(over)
    wsb = ssd.ssd_workspace_bytes(p) if ws_bytes is None else ws_bytes
    return ssd.ssd_forward(p, a["X"], a["logA"], a["B"], a["C"], a["init"], a["off"], a["Y"],
                           a["final"], a["ws"], wsb, None)


def test_forward_rejects_invalid_problem():
    assert call(prob(nheads=3), ws_bytes=1 << 20, off=None) == ssd.SSD_ERR_INVALID_ARG
    assert call(prob(chunk_len=100), ws_bytes=1 << 20, off=None) == ssd.SSD_ERR_UNSUPPORTED


@pytest.mark.parametrize("name", ["X", "logA", "B", "C", "Y", "ws"])
def test_forward_rejects_null_required_pointer(name):
    assert call(prob(), off=None, **{name: None}) == ssd.SSD_ERR_INVALID_ARG


@pytest.mark.parametrize("name", ["X", "logA", "B", "C", "init", "Y", "final"])
def test_forward_rejects_misaligned_pointer(name):
    assert call(prob(), off=None, **{name: ADDR[name] + 4}) == ssd.SSD_ERR_INVALID_ARG


def test_forward_rejects_misaligned_workspace():
    assert call(prob(), off=None, ws=ADDR["ws"] + 16) == ssd.SSD_ERR_INVALID_ARG


def test_forward_rejects_seq_offsets_with_batch():
    assert call(prob(batch=2, nseq=3)) == ssd.SSD_ERR_INVALID_ARG


def test_forward_rejects_nseq_mismatch_without_offsets():
    assert call(prob(batch=2, nseq=3), off=None) == ssd.SSD_ERR_INVALID_ARG


@pytest.mark.parametrize("out,inp", [("Y", "X"), ("final", "init"), ("Y", "B"), ("final", "ws"),
                                     ("final", "Y")])
def test_forward_rejects_aliased_outputs(out, inp):
    assert call(prob(), off=None, **{out: ADDR[inp]}) == ssd.SSD_ERR_INVALID_ARG


@pytest.mark.parametrize("inp", ["X", "logA", "B", "C", "init", "off"])
def test_forward_rejects_workspace_overlapping_an_input(inp):
    # the workspace starts at the input's first byte, or 256 bytes into it (seq_offsets
    # holds only 8 bytes here: its first byte only)
    p = prob(batch=1, nseq=1) if inp == "off" else prob()
    for shift in ((0,) if inp == "off" else (0, 256)):
        over = {"ws": ADDR[inp] + shift}
        if inp != "off":
            over["off"] = None
        assert call(p, **over) == ssd.SSD_ERR_INVALID_ARG, (inp, shift)


def test_forward_rejects_small_workspace():
    p = prob()
    assert call(p, ws_bytes=ssd.ssd_workspace_bytes(p) - 256, off=None) == ssd.SSD_ERR_WORKSPACE


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    X = torch.zeros(1, 4, 1, 16)
    with pytest.raises(ValueError):
        ssd.forward(X, torch.zeros(1, 4, 1), torch.zeros(1, 4, 1, 16), torch.zeros(1, 4, 1, 16), 16)


@pytest.mark.parametrize("stage", [0, 3, -1])
def test_forward_stage_rejects_unknown_stage(stage):
    p = prob()
    a = ADDR
    assert ssd.ssd_forward_stage(stage, p, a["X"], a["logA"], a["B"], a["C"], a["init"], None,
                                 a["Y"], a["final"], a["ws"], ssd.ssd_workspace_bytes(p),
                                 None) == ssd.SSD_ERR_INVALID_ARG


@pytest.mark.parametrize("stage", [1, 2])
def test_forward_stage_validates_like_forward(stage):
    p = prob()
    a = ADDR
    assert ssd.ssd_forward_stage(stage, p, a["X"] + 4, a["logA"], a["B"], a["C"], a["init"], None,
                                 a["Y"], a["final"], a["ws"], ssd.ssd_workspace_bytes(p),
                                 None) == ssd.SSD_ERR_INVALID_ARG


# ssd_decode_step: the same fake-address discipline (validation fails before any launch).
DADDR = dict(x=1 * GB, logA=2 * GB, B=3 * GB, C=4 * GB, state=5 * GB, y=6 * GB)


def dprob(**kw):
    d = dict(batch=3, seqlen=1, nheads=4, headdim=64, dstate=128, ngroups=2, chunk_len=16,
             nseq=3, dtype=ssd.SSD_DTYPE_BF16)
    d.update(kw)
    return ssd.problem_for(**d)


def dcall(p, **over):
    a = dict(DADDR)
    a.update(over)
    return ssd.ssd_decode_step(p, a["x"], a["logA"], a["B"], a["C"], a["state"], a["y"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(seqlen=2), ssd.SSD_ERR_INVALID_ARG),
    (dict(nseq=2), ssd.SSD_ERR_INVALID_ARG),
    (dict(nheads=3), ssd.SSD_ERR_INVALID_ARG),
    (dict(batch=0, nseq=0), ssd.SSD_ERR_INVALID_ARG),
    (dict(dtype=5), ssd.SSD_ERR_UNSUPPORTED),
    (dict(headdim=40), ssd.SSD_ERR_UNSUPPORTED),
    (dict(dstate=512), ssd.SSD_ERR_UNSUPPORTED),
])
def test_decode_rejects_invalid_problem(kw, code):
    assert dcall(dprob(**kw)) == code


@pytest.mark.parametrize("name", list(DADDR))
def test_decode_rejects_null_and_misaligned_pointers(name):
    assert dcall(dprob(), **{name: None}) == ssd.SSD_ERR_INVALID_ARG
    assert dcall(dprob(), **{name: DADDR[name] + 8}) == ssd.SSD_ERR_INVALID_ARG


@pytest.mark.parametrize("out,inp", [("y", "x"), ("state", "B"), ("state", "y")])
def test_decode_rejects_aliased_outputs(out, inp):
    assert dcall(dprob(), **{out: DADDR[inp]}) == ssd.SSD_ERR_INVALID_ARG



# ssd_backward: validation on the host with fake addresses, as above.
BADDR = dict(ADDR, Yf=10 * GB, dY=11 * GB, dF=12 * GB, dX=13 * GB, dlogA=14 * GB, dB=15 * GB, dC=16 * GB,
             dinit=17 * GB, bws=18 * GB)


def bcall(p, ws_bytes=None, **over):
    a = dict(BADDR)
    a.update(over)
    wsb = ssd.ssd_backward_workspace_bytes(p) if ws_bytes is None else ws_bytes
    return ssd.ssd_backward(p, a["X"], a["logA"], a["B"], a["C"], a["init"], a["off"], a["Yf"], a["final"],
                            a["dY"], a["dF"], a["dX"], a["dlogA"], a["dB"], a["dC"], a["dinit"], a["bws"], wsb, None)


def test_backward_workspace_covers_the_forward_workspaces():
    p = prob()
    q = prob(headdim=128, dstate=64, ngroups=4)   # the transposed problem of p
    assert ssd.ssd_backward_workspace_bytes(p) > max(ssd.ssd_workspace_bytes(p), ssd.ssd_workspace_bytes(q))
    assert ssd.ssd_backward_workspace_bytes(prob(nheads=3)) == 0


@pytest.mark.parametrize("name", ["X", "logA", "B", "C", "Yf", "dY", "dX", "dlogA", "dB", "dC", "bws"])
def test_backward_rejects_null_required_pointer(name):
    assert bcall(prob(), off=None, **{name: None}) == ssd.SSD_ERR_INVALID_ARG


def test_backward_needs_final_state_with_dfinal():
    assert bcall(prob(), off=None, final=None) == ssd.SSD_ERR_INVALID_ARG


@pytest.mark.parametrize("out,inp", [("dX", "X"), ("dB", "dY"), ("dinit", "init"), ("dC", "bws"), ("dB", "dC")])
def test_backward_rejects_aliased_outputs(out, inp):
    assert bcall(prob(), off=None, **{out: BADDR[inp]}) == ssd.SSD_ERR_INVALID_ARG


@pytest.mark.parametrize("inp", ["X", "logA", "B", "C", "init", "Yf", "final", "dY", "dF"])
def test_backward_rejects_workspace_overlapping_an_input(inp):
    assert bcall(prob(), off=None, bws=BADDR[inp]) == ssd.SSD_ERR_INVALID_ARG


def test_backward_rejects_small_workspace_and_misalignment():
    p = prob()
    assert bcall(p, ws_bytes=ssd.ssd_backward_workspace_bytes(p) - 256, off=None) == ssd.SSD_ERR_WORKSPACE
    assert bcall(p, off=None, dlogA=BADDR["dlogA"] + 4) == ssd.SSD_ERR_INVALID_ARG


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    # no fallback: a missing libssd.so is an import error, not a silent CPU path
    monkeypatch.setattr(ssd, "_lib", None)
    monkeypatch.setattr(ssd, "lib_path", lambda: str(tmp_path / "libssd.so"))
    with pytest.raises(ImportError):
        ssd.load_library()


def test_plan_describe_names_the_kernels():
    # the planner is host logic: the kernels a shape gets are known without a device
    bf16, f32 = ssd.SSD_DTYPE_BF16, ssd.SSD_DTYPE_F32
    layer = ssd.problem_for(8, 2048, 80, 64, 128, 1, 256, 8, bf16)
    assert ssd.ssd_plan_describe(layer) == {"walk": "ssd_walk_fused_kernel<128, 5>", "prep": "none",
                                            "summary": "none"}
    small = ssd.problem_for(1, 256, 4, 64, 64, 1, 256, 1, f32)
    d = ssd.ssd_plan_describe(small)
    assert d["walk"] != "none" and "fused" not in d["walk"] and d["prep"] != "none"
    bad = ssd.problem_for(1, 256, 4, 64, 64, 3, 256, 1, bf16)     # heads not a multiple of groups
    with pytest.raises(ssd.SsdError):
        ssd.ssd_plan_describe(bad)


def test_plan_long_sequences_and_state_256():
    bf16 = ssd.SSD_DTYPE_BF16
    # one long sequence: segments of the fused walker, after their summary
    long = ssd.ssd_plan_describe(ssd.problem_for(1, 16384, 80, 64, 128, 1, 256, 1, bf16))
    assert long["walk"] == "ssd_walk_fused_kernel<128, 5>" and long["summary"].startswith("ssd_seg_summary_kernel<128>")
    # its eight segments' entry states chained one after the other; many segments (64 of
    # 1024 rows for eight heads) by the associative scan over the segments
    assert long["summary"].endswith("ssd_seg_chain_kernel")
    many = ssd.ssd_plan_describe(ssd.problem_for(1, 65536, 8, 64, 128, 1, 256, 1, bf16))
    assert many["summary"] == "ssd_seg_summary_kernel<128>+ssd_seg_scan_kernel", many
    # d_state 256 on the fused walker where no segments are needed ...
    wide = ssd.ssd_plan_describe(ssd.problem_for(32, 300, 8, 64, 256, 1, 256, 32, bf16))
    assert wide == {"walk": "ssd_walk_fused_kernel<256, 2>", "prep": "none", "summary": "none"}
    # ... and the two passes over the state's column halves where they would be
    few = ssd.ssd_plan_describe(ssd.problem_for(4, 4096, 32, 64, 256, 1, 256, 4, bf16))
    assert few["walk"].startswith("ssd_walk_split_pair_kernel") and few["prep"] != "none"
    # the fused walker's result does not depend on the chunk length: every valid one plans it
    for q in (16, 32, 64, 128, 256):
        d = ssd.ssd_plan_describe(ssd.problem_for(8, 2048, 80, 64, 128, 1, q, 8, bf16))
        assert d["walk"] == "ssd_walk_fused_kernel<128, 5>", (q, d)


def test_noalloc_rejects_a_problem_beyond_its_scratch_before_device_work():
    # the size check comes before any HIP call, so fake addresses are never touched
    prob = ssd.problem_for(32, 4096, 32, 64, 256, 1, 256, 32, ssd.SSD_DTYPE_F32)
    assert ssd.ssd_workspace_bytes(prob) > ssd.SSD_NOALLOC_SCRATCH_BYTES
    rc = ssd.ssd_forward_noalloc(prob, 1 * GB, 2 * GB, 3 * GB, 4 * GB, None, None, 6 * GB, None, None)
    assert rc == ssd.SSD_ERR_TOO_LARGE
    assert "scratch" in ssd.ssd_status_string(rc)
