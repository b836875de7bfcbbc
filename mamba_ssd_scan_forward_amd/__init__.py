"""MI355X-native SSD (structured state space duality) layer forward.

A thin ctypes binding over ``libssd.so`` (C ABI in ``include/ssd.h``).  This module only
marshals arguments: every step of the computation runs in the library's HIP kernels on
the caller's current HIP stream.  PyTorch supplies device memory and the stream.

    Y, final_state = forward(X, logA, B, C, chunk_len, init_state=None, seq_offsets=None)
    y = decode_step(x, logA, B, C, state)      # one recurrent step, state updated in place

Shapes (row-major): X [b, T, H, P] (float32 or bfloat16); logA [b, T, H] float32;
B, C [b, T, G, N] (same dtype as X); init_state [nseq, H, P, N] float32 or None;
seq_offsets [nseq + 1] int32 or None (packed variable-length batch, b == 1).
Y has X's dtype; final_state is float32 [nseq, H, P, N].

The library must be built first (``python -m mamba_ssd_scan_forward_amd.build``); a
missing library raises instead of falling back to any other implementation.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "SSD_OK", "SSD_ERR_INVALID_ARG", "SSD_ERR_UNSUPPORTED", "SSD_ERR_WORKSPACE", "SSD_ERR_HIP",
    "SSD_DTYPE_F32", "SSD_DTYPE_BF16", "SsdProblem", "SsdError", "lib_path", "load_library",
    "ssd_check_problem", "ssd_workspace_bytes", "ssd_forward", "ssd_forward_stage",
    "ssd_decode_step", "ssd_backward_workspace_bytes", "ssd_backward", "ssd_status_string",
    "ssd_abi_version", "ssd_plan_describe", "ssd_forward_noalloc", "SSD_NOALLOC_SCRATCH_BYTES",
    "SSD_ERR_TOO_LARGE", "forward", "decode_step", "backward", "problem_for",
]

SSD_OK = 0
SSD_ERR_INVALID_ARG = -1
SSD_ERR_UNSUPPORTED = -2
SSD_ERR_WORKSPACE = -3
SSD_ERR_HIP = -4
SSD_ERR_TOO_LARGE = -5
SSD_NOALLOC_SCRATCH_BYTES = 64 << 20
SSD_DTYPE_F32 = 0
SSD_DTYPE_BF16 = 1
ABI_VERSION = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


class SsdProblem(ctypes.Structure):
    """Mirror of ``ssd_problem`` in include/ssd.h."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
        ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
        ("chunk_len", ctypes.c_int64), ("nseq", ctypes.c_int64), ("dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class SsdError(RuntimeError):
    def __init__(self, status: int, what: str = "ssd_forward"):
        self.status = status
        super().__init__(f"{what} failed: {ssd_status_string(status)} ({status})")


def _share_hip_runtime():
    """One HIP runtime per process.  PyTorch for ROCm ships its own libamdhip64 and loads
    it by path: if a library of ours came first (binding the system runtime of the same
    soname), the process would hold two runtimes and the one ours uses would find no
    device.  Loaded after torch, our libraries bind to torch's runtime."""
    try:
        import torch  # noqa: F401
    except ImportError:
        pass


def lib_path() -> str:
    return os.path.join(_HERE, "libssd.so")


def load_library():
    """Load libssd.so from the package directory.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m mamba_ssd_scan_forward_amd.build`")
    _share_hip_runtime()
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    pp = ctypes.POINTER(SsdProblem)
    lib.ssd_check_problem.argtypes = [pp]
    lib.ssd_check_problem.restype = ctypes.c_int
    lib.ssd_workspace_bytes.argtypes = [pp]
    lib.ssd_workspace_bytes.restype = sz
    lib.ssd_forward.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ssd_forward.restype = ctypes.c_int
    lib.ssd_forward_stage.argtypes = [ctypes.c_int, pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ssd_forward_stage.restype = ctypes.c_int
    lib.ssd_decode_step.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp]
    lib.ssd_decode_step.restype = ctypes.c_int
    lib.ssd_backward_workspace_bytes.argtypes = [pp]
    lib.ssd_backward_workspace_bytes.restype = sz
    lib.ssd_backward.argtypes = [pp] + [vp] * 16 + [sz, vp]
    lib.ssd_backward.restype = ctypes.c_int
    lib.ssd_status_string.argtypes = [ctypes.c_int]
    lib.ssd_status_string.restype = ctypes.c_char_p
    lib.ssd_forward_noalloc.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ssd_forward_noalloc.restype = ctypes.c_int
    lib.ssd_plan_describe.argtypes = [pp, ctypes.c_char_p, sz]
    lib.ssd_plan_describe.restype = ctypes.c_int
    lib.ssd_abi_version.argtypes = []
    lib.ssd_abi_version.restype = ctypes.c_int
    if lib.ssd_abi_version() != ABI_VERSION:
        raise ImportError(f"libssd.so ABI {lib.ssd_abi_version()} != binding ABI {ABI_VERSION}")
    _lib = lib
    return lib


_probe = None


def probe_lib_path() -> str:
    return os.path.join(_HERE, "libssd_probe.so")


def load_probe_library():
    """Load libssd_probe.so (machine measurements, include/ssd_probe.h).  Raises if it has
    not been built."""
    global _probe
    if _probe is not None:
        return _probe
    path = probe_lib_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m mamba_ssd_scan_forward_amd.build`")
    _share_hip_runtime()
    lib = ctypes.CDLL(path)
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.ssd_probe_mfma_bf16.argtypes = [i64, ci, vp, vp]
    lib.ssd_probe_mfma_bf16.restype = ci
    lib.ssd_probe_clock.argtypes = [i64, ci, vp, vp]
    lib.ssd_probe_clock.restype = ci
    lib.ssd_probe_device.argtypes = [ctypes.POINTER(ci), ctypes.POINTER(ci)]
    lib.ssd_probe_device.restype = ci
    _probe = lib
    return lib


def ssd_status_string(status: int) -> str:
    return load_library().ssd_status_string(int(status)).decode()


def ssd_abi_version() -> int:
    return int(load_library().ssd_abi_version())


def ssd_plan_describe(problem: SsdProblem) -> dict:
    """The kernels ssd_forward launches for this problem: {"walk": ..., "prep": ...,
    "summary": ...} ("none" where a launch is not made)."""
    buf = ctypes.create_string_buffer(256)
    rc = load_library().ssd_plan_describe(ctypes.byref(problem), buf, len(buf))
    if rc != SSD_OK:
        raise SsdError(rc, "ssd_plan_describe")
    return dict(kv.split("=", 1) for kv in buf.value.decode().split(";"))


def ssd_check_problem(problem: SsdProblem) -> int:
    return int(load_library().ssd_check_problem(ctypes.byref(problem)))


def ssd_workspace_bytes(problem: SsdProblem) -> int:
    return int(load_library().ssd_workspace_bytes(ctypes.byref(problem)))


def ssd_forward(problem: SsdProblem, X, logA, B, C, init_state, seq_offsets, Y, final_state,
                workspace, workspace_bytes: int, hip_stream) -> int:
    """Direct call of the C entry point.  Pointer arguments are integers (device
    addresses) or None; returns the ssd_status code."""
    return int(load_library().ssd_forward(ctypes.byref(problem), X, logA, B, C, init_state,
                                          seq_offsets, Y, final_state, workspace,
                                          int(workspace_bytes), hip_stream))


def ssd_forward_noalloc(problem: SsdProblem, X, logA, B, C, init_state, seq_offsets, Y, final_state,
                        hip_stream) -> int:
    """Direct call of the no-allocation entry point (its scratch is the library's own
    per-device array of SSD_NOALLOC_SCRATCH_BYTES).  Pointer arguments are integers
    (device addresses) or None; returns the ssd_status code."""
    return int(load_library().ssd_forward_noalloc(ctypes.byref(problem), X, logA, B, C, init_state,
                                                  seq_offsets, Y, final_state, hip_stream))


def ssd_forward_stage(stage: int, problem: SsdProblem, X, logA, B, C, init_state, seq_offsets, Y,
                      final_state, workspace, workspace_bytes: int, hip_stream) -> int:
    """Direct call of ssd_forward_stage (stage 1: prep launch, stage 2: chunk walk)."""
    return int(load_library().ssd_forward_stage(int(stage), ctypes.byref(problem), X, logA, B, C,
                                                init_state, seq_offsets, Y, final_state,
                                                workspace, int(workspace_bytes), hip_stream))


def ssd_decode_step(problem: SsdProblem, x, logA, B, C, state, y, hip_stream) -> int:
    """Direct call of ssd_decode_step (device addresses as integers); returns the status."""
    return int(load_library().ssd_decode_step(ctypes.byref(problem), x, logA, B, C, state, y,
                                              hip_stream))


def ssd_backward_workspace_bytes(problem: SsdProblem) -> int:
    return int(load_library().ssd_backward_workspace_bytes(ctypes.byref(problem)))


def ssd_backward(problem: SsdProblem, X, logA, B, C, init_state, seq_offsets, Y, final_state, dY,
                 dfinal, dX, dlogA, dB, dC, dinit, workspace, workspace_bytes: int, hip_stream) -> int:
    """Direct call of ssd_backward (device addresses as integers or None); returns the status."""
    return int(load_library().ssd_backward(ctypes.byref(problem), X, logA, B, C, init_state, seq_offsets,
                                           Y, final_state, dY, dfinal, dX, dlogA, dB, dC, dinit,
                                           workspace, int(workspace_bytes), hip_stream))


def problem_for(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_len, nseq, dtype) -> SsdProblem:
    return SsdProblem(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_len, nseq, dtype, 0)


def _ptr(t):
    return None if t is None else t.data_ptr()


def forward(X, logA, B, C, chunk_len: int, init_state=None, seq_offsets=None,
            return_final_state: bool = True, workspace=None):
    """SSD forward on the current HIP stream.  Returns (Y, final_state or None)."""
    import torch

    if X.dtype == torch.bfloat16:
        dt = SSD_DTYPE_BF16
    elif X.dtype == torch.float32:
        dt = SSD_DTYPE_F32
    else:
        raise TypeError(f"unsupported dtype {X.dtype}")
    if not X.is_cuda:
        raise ValueError("forward() needs device tensors")
    if X.dim() != 4 or logA.dim() != 3 or B.dim() != 4 or C.dim() != 4:
        raise ValueError("expected X [b,T,H,P], logA [b,T,H], B/C [b,T,G,N]")
    b, T, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    if tuple(logA.shape) != (b, T, H) or tuple(B.shape) != (b, T, G, N) or tuple(C.shape) != (b, T, G, N):
        raise ValueError("shape mismatch between X, logA, B and C")
    if B.dtype != X.dtype or C.dtype != X.dtype or logA.dtype != torch.float32:
        raise TypeError("B and C must share X's dtype; logA must be float32")
    X, logA, B, C = X.contiguous(), logA.contiguous(), B.contiguous(), C.contiguous()
    nseq = b
    if seq_offsets is not None:
        if seq_offsets.dtype != torch.int32:
            raise TypeError("seq_offsets must be int32")
        seq_offsets = seq_offsets.contiguous()
        nseq = seq_offsets.numel() - 1
    if init_state is not None:
        if init_state.dtype != torch.float32 or tuple(init_state.shape) != (nseq, H, P, N):
            raise ValueError("init_state must be float32 [nseq, H, P, N]")
        init_state = init_state.contiguous()
    prob = problem_for(b, T, H, P, N, G, int(chunk_len), nseq, dt)
    rc = ssd_check_problem(prob)
    if rc != SSD_OK:
        raise SsdError(rc, "ssd_check_problem")
    wsb = ssd_workspace_bytes(prob)
    if workspace is None or workspace.numel() < wsb:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=X.device)
    Y = torch.empty_like(X)
    final = torch.empty((nseq, H, P, N), dtype=torch.float32, device=X.device) if return_final_state else None
    stream = torch.cuda.current_stream(X.device).cuda_stream
    rc = ssd_forward(prob, _ptr(X), _ptr(logA), _ptr(B), _ptr(C), _ptr(init_state),
                     _ptr(seq_offsets), _ptr(Y), _ptr(final), _ptr(workspace), wsb, stream)
    if rc != SSD_OK:
        raise SsdError(rc)
    return Y, final


def decode_step(x, logA, B, C, state, y=None):
    """One recurrent step on the current HIP stream: for every sequence s and head h,
    state[s, h] <- exp(logA[s, h]) state[s, h] + x[s, h] B[s, g]^T and
    y[s, h] = state[s, h] C[s, g].  x [b, H, P], logA [b, H] float32, B/C [b, G, N],
    state [b, H, P, N] float32 (updated in place).  Returns y [b, H, P] (x's dtype)."""
    import torch

    if x.dtype == torch.bfloat16:
        dt = SSD_DTYPE_BF16
    elif x.dtype == torch.float32:
        dt = SSD_DTYPE_F32
    else:
        raise TypeError(f"unsupported dtype {x.dtype}")
    if x.dim() != 3 or logA.dim() != 2 or B.dim() != 3 or C.dim() != 3 or state.dim() != 4:
        raise ValueError("expected x [b,H,P], logA [b,H], B/C [b,G,N], state [b,H,P,N]")
    b, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    if (tuple(logA.shape) != (b, H) or tuple(B.shape) != (b, G, N) or tuple(C.shape) != (b, G, N)
            or tuple(state.shape) != (b, H, P, N)):
        raise ValueError("shape mismatch between x, logA, B, C and state")
    if B.dtype != x.dtype or C.dtype != x.dtype or logA.dtype != torch.float32 or state.dtype != torch.float32:
        raise TypeError("B and C must share x's dtype; logA and state must be float32")
    if not state.is_contiguous():
        raise ValueError("state must be contiguous (it is updated in place)")
    x, logA, B, C = x.contiguous(), logA.contiguous(), B.contiguous(), C.contiguous()
    if y is None:
        y = torch.empty_like(x)
    prob = problem_for(b, 1, H, P, N, G, 16, b, dt)
    stream = torch.cuda.current_stream(x.device).cuda_stream
    rc = ssd_decode_step(prob, _ptr(x), _ptr(logA), _ptr(B), _ptr(C), _ptr(state), _ptr(y), stream)
    if rc != SSD_OK:
        raise SsdError(rc, "ssd_decode_step")
    return y


def backward(X, logA, B, C, chunk_len: int, Y, dY, init_state=None, seq_offsets=None,
             final_state=None, dfinal=None, need_dinit: bool = True, workspace=None):
    """Gradients of <dY, Y> + <dfinal, final_state> for the forward pass
    ``(Y, final_state) = forward(X, logA, B, C, chunk_len, init_state, seq_offsets)``, on the
    current HIP stream.  Returns (dX, dlogA, dB, dC, dinit or None)."""
    import torch

    if X.dtype == torch.bfloat16:
        dt = SSD_DTYPE_BF16
    elif X.dtype == torch.float32:
        dt = SSD_DTYPE_F32
    else:
        raise TypeError(f"unsupported dtype {X.dtype}")
    if not X.is_cuda:
        raise ValueError("backward() needs device tensors")
    b, T, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    if tuple(Y.shape) != tuple(X.shape) or tuple(dY.shape) != tuple(X.shape):
        raise ValueError("Y and dY must have X's shape")
    if Y.dtype != X.dtype or dY.dtype != X.dtype:
        raise TypeError("Y and dY must share X's dtype")
    nseq = b if seq_offsets is None else seq_offsets.numel() - 1
    if dfinal is not None and final_state is None:
        raise ValueError("dfinal needs the forward pass's final_state")
    for name, t in (("init_state", init_state), ("final_state", final_state), ("dfinal", dfinal)):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (nseq, H, P, N)):
            raise ValueError(f"{name} must be float32 [nseq, H, P, N]")
    X, logA, B, C, Y, dY = (t.contiguous() for t in (X, logA, B, C, Y, dY))
    init_state, final_state, dfinal, seq_offsets = (None if t is None else t.contiguous()
                                                    for t in (init_state, final_state, dfinal, seq_offsets))
    prob = problem_for(b, T, H, P, N, G, int(chunk_len), nseq, dt)
    wsb = ssd_backward_workspace_bytes(prob)
    if wsb == 0:
        raise SsdError(ssd_check_problem(prob) or SSD_ERR_UNSUPPORTED, "ssd_backward_workspace_bytes")
    if workspace is None or workspace.numel() < wsb:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=X.device)
    dX = torch.empty_like(X)
    dlogA = torch.empty_like(logA)
    dB = torch.empty_like(B)
    dC = torch.empty_like(C)
    dinit = torch.empty((nseq, H, P, N), dtype=torch.float32, device=X.device) if need_dinit else None
    stream = torch.cuda.current_stream(X.device).cuda_stream
    rc = ssd_backward(prob, _ptr(X), _ptr(logA), _ptr(B), _ptr(C), _ptr(init_state), _ptr(seq_offsets),
                      _ptr(Y), _ptr(final_state), _ptr(dY), _ptr(dfinal), _ptr(dX), _ptr(dlogA), _ptr(dB),
                      _ptr(dC), _ptr(dinit), _ptr(workspace), wsb, stream)
    if rc != SSD_OK:
        raise SsdError(rc, "ssd_backward")
    return dX, dlogA, dB, dC, dinit
