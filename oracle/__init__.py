"""Float64 CPU oracle for the SSD layer forward -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path:
no kernels, headers, helpers or constants; the product library never loads it.

What is computed (page: "Transformers are SSMs" paper summary):

* ``recurrence`` -- the plain definition, run by ``ssd_oracle.c``: per head a
  scalar-identity SSM (section 2.4; section 5.1 with A_t = a_t I) in linear
  mode (section 3.4.1): S = a_t S + x_t B_t^T, y_t = S C_t, a_t = exp(logA_t).
* ``recurrence_np`` -- the same definition as a pure NumPy loop, for tiny inputs.
* ``quadratic`` -- the dual (attention-like) form of section 5.1:
  Y = (L o C B^T) X with the 1-semiseparable mask L[i, j] = a_{j+1} ... a_i
  (i >= j), plus the decayed initial state.  Tiny T only.
* ``chunked`` -- the block decomposition of section 6 (6.1 diagonal blocks,
  6.2 right / center / left factors of the low-rank blocks), for any chunk
  length, ragged last chunk included.
* ``decode_step`` -- one step of the recurrence for a single token per sequence
  (the recurrent mode of section 3), continuing from a given state.
* ``backward`` -- the reverse-mode derivative of ``recurrence`` (the adjoint
  recurrence, walked backwards over the tokens; the pages state only its cost,
  section 6's training FLOPs), run by ``ssd_oracle.c``.  Pinned by central
  finite differences of ``recurrence``.

Readings of the pages that these functions take:
A is the log decay (logA <= 0, a_t = exp(logA_t), -inf allowed, giving a = 0);
the mask is L[i, j] = a_{j+1} ... a_i with L[i, i] = 1; the initial state is
the state before token 0 and is decayed by a_0; the state is stored P x N;
head h reads group h // (H // G); with ``seq_offsets`` every packed sequence
is an independent problem starting from its own initial state.

Shapes (float64, row-major): X [b, T, H, P]; logA [b, T, H]; B, C [b, T, G, N];
init and final [nseq, H, P, N]; seq_offsets [nseq + 1] with b == 1.

Parity: every function here is pinned by ``tests/test_oracle.py`` against
values fixed by the mathematics (duality, closed forms, worked examples,
split/packing/linearity/group invariants); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libssd_oracle.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        src = os.path.join(_HERE, "ssd_oracle.c")
        if (not os.path.exists(_LIB_PATH)
                or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src)):
            from . import build as _build
            _build.build()
        lib = ctypes.CDLL(_LIB_PATH)
        d = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.ssd_oracle_recurrence.argtypes = [i64, i64, i64, i64, i64, i64, d, d, d, d, d,
                                              ctypes.POINTER(ctypes.c_int64), i64, d, d,
                                              ctypes.c_int]
        lib.ssd_oracle_recurrence.restype = ctypes.c_int
        lib.ssd_oracle_backward.argtypes = [i64, i64, i64, i64, i64, i64, d, d, d, d, d,
                                            ctypes.POINTER(ctypes.c_int64), i64, d, d,
                                            d, d, d, d, d, ctypes.c_int]
        lib.ssd_oracle_backward.restype = ctypes.c_int
        lib.ssd_oracle_threads.argtypes = []
        lib.ssd_oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def threads() -> int:
    """OpenMP threads the C oracle uses by default."""
    return int(_load().ssd_oracle_threads())


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _shapes(X, logA, B, C):
    b, T, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    assert logA.shape == (b, T, H), logA.shape
    assert B.shape == (b, T, G, N) and C.shape == (b, T, G, N), (B.shape, C.shape)
    assert H % G == 0
    return b, T, H, P, N, G


def _sequences(b, T, seq_offsets):
    """Row ranges [r0, r1) into the flattened [b*T] token axis, one per sequence."""
    if seq_offsets is None:
        return [(s * T, (s + 1) * T) for s in range(b)]
    assert b == 1
    off = [int(v) for v in np.asarray(seq_offsets).reshape(-1)]
    assert off[0] == 0 and off[-1] == T and all(off[i] <= off[i + 1] for i in range(len(off) - 1))
    return [(off[i], off[i + 1]) for i in range(len(off) - 1)]


def recurrence(X, logA, B, C, init=None, seq_offsets=None, nthreads: int = 0):
    """Plain recurrence in C (float64).  Returns (Y [b,T,H,P], final [nseq,H,P,N])."""
    X, logA, B, C = _f64(X), _f64(logA), _f64(B), _f64(C)
    b, T, H, P, N, G = _shapes(X, logA, B, C)
    nseq = b if seq_offsets is None else int(np.asarray(seq_offsets).size - 1)
    Y = np.zeros((b, T, H, P), dtype=np.float64)
    final = np.zeros((nseq, H, P, N), dtype=np.float64)
    dp = ctypes.POINTER(ctypes.c_double)
    init_p = None
    if init is not None:
        init = _f64(init)
        assert init.shape == (nseq, H, P, N), init.shape
        init_p = init.ctypes.data_as(dp)
    off_p = None
    if seq_offsets is not None:
        off = np.ascontiguousarray(np.asarray(seq_offsets, dtype=np.int64).reshape(-1))
        off_p = off.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    rc = _load().ssd_oracle_recurrence(b, T, H, P, N, G, X.ctypes.data_as(dp),
                                       logA.ctypes.data_as(dp), B.ctypes.data_as(dp),
                                       C.ctypes.data_as(dp), init_p, off_p, nseq,
                                       Y.ctypes.data_as(dp), final.ctypes.data_as(dp),
                                       int(nthreads))
    if rc != 0:
        raise ValueError(f"ssd_oracle_recurrence failed with code {rc}")
    return Y, final


def recurrence_np(X, logA, B, C, init=None, seq_offsets=None):
    """The same definition as ``recurrence`` as a NumPy loop over tokens (tiny inputs)."""
    X, logA, B, C = _f64(X), _f64(logA), _f64(B), _f64(C)
    b, T, H, P, N, G = _shapes(X, logA, B, C)
    rows = _sequences(b, T, seq_offsets)
    Xf, Af = X.reshape(b * T, H, P), logA.reshape(b * T, H)
    Bf, Cf = B.reshape(b * T, G, N), C.reshape(b * T, G, N)
    Y = np.zeros((b * T, H, P))
    final = np.zeros((len(rows), H, P, N))
    for s, (r0, r1) in enumerate(rows):
        for h in range(H):
            g = h // (H // G)
            S = np.zeros((P, N)) if init is None else np.array(init[s, h], dtype=np.float64)
            for r in range(r0, r1):
                S = np.exp(Af[r, h]) * S + np.outer(Xf[r, h], Bf[r, g])
                Y[r, h] = S @ Cf[r, g]
            final[s, h] = S
    return Y.reshape(b, T, H, P), final


def mask_1ss(logA_seq):
    """1-semiseparable mask of one head: L[i, j] = a_{j+1} * ... * a_i for i >= j, L[i, i] = 1,
    zero above the diagonal; built column by column from explicit products of a = exp(logA)."""
    a = np.exp(np.asarray(logA_seq, dtype=np.float64))
    T = a.shape[0]
    L = np.zeros((T, T))
    for j in range(T):
        L[j, j] = 1.0
        for i in range(j + 1, T):
            L[i, j] = L[i - 1, j] * a[i]
    return L


def quadratic(X, logA, B, C, init=None, seq_offsets=None):
    """Dual quadratic form Y = (L o C B^T) X + diag(a_0...a_t) C init^T (tiny T only)."""
    X, logA, B, C = _f64(X), _f64(logA), _f64(B), _f64(C)
    b, T, H, P, N, G = _shapes(X, logA, B, C)
    rows = _sequences(b, T, seq_offsets)
    Xf, Af = X.reshape(b * T, H, P), logA.reshape(b * T, H)
    Bf, Cf = B.reshape(b * T, G, N), C.reshape(b * T, G, N)
    Y = np.zeros((b * T, H, P))
    final = np.zeros((len(rows), H, P, N))
    for s, (r0, r1) in enumerate(rows):
        if r1 == r0:
            if init is not None:
                final[s] = init[s]
            continue
        for h in range(H):
            g = h // (H // G)
            x, c, bb = Xf[r0:r1, h], Cf[r0:r1, g], Bf[r0:r1, g]
            L = mask_1ss(Af[r0:r1, h])
            M = L * (c @ bb.T)                       # M[t, u] = (C_t . B_u) a_{u+1} ... a_t
            y = M @ x
            fin = (L[-1][:, None] * x).T @ bb        # sum_u a_{u+1} ... a_{T-1} x_u B_u^T
            if init is not None:
                through = np.cumprod(np.exp(Af[r0:r1, h]))   # a_0 ... a_t
                y = y + through[:, None] * (c @ np.asarray(init[s, h]).T)
                fin = fin + through[-1] * np.asarray(init[s, h])
            Y[r0:r1, h] = y
            final[s, h] = fin
    return Y.reshape(b, T, H, P), final


def segsum(logA_chunk):
    """segsum[i, j] = logA_{j+1} + ... + logA_i for i >= j (0 on the diagonal), -inf above.

    Built as a cumulative sum down each column of the strictly-lower part, so that a
    logA of -inf gives -inf rather than (-inf) - (-inf)."""
    la = np.asarray(logA_chunk, dtype=np.float64)
    Q = la.shape[0]
    low = np.where(np.arange(Q)[:, None] > np.arange(Q)[None, :], la[:, None], 0.0)
    seg = np.cumsum(low, axis=0)
    return np.where(np.arange(Q)[:, None] >= np.arange(Q)[None, :], seg, -np.inf)


def chunked(X, logA, B, C, chunk_len: int, init=None, seq_offsets=None):
    """Block decomposition of M (section 6) with chunk length Q = chunk_len.

    Per sequence and head: (1) the diagonal blocks in quadratic form with a zero
    entry state; (2) right factor: each chunk's final state from a zero entry state;
    (3) center factor: a scalar recurrence over chunks giving each chunk's true entry
    state; (4) left factor: the entry state read out by C and decayed within the chunk.
    The last chunk of a sequence may be shorter than Q."""
    X, logA, B, C = _f64(X), _f64(logA), _f64(B), _f64(C)
    b, T, H, P, N, G = _shapes(X, logA, B, C)
    Q = int(chunk_len)
    assert Q >= 1
    rows = _sequences(b, T, seq_offsets)
    Xf, Af = X.reshape(b * T, H, P), logA.reshape(b * T, H)
    Bf, Cf = B.reshape(b * T, G, N), C.reshape(b * T, G, N)
    Y = np.zeros((b * T, H, P))
    final = np.zeros((len(rows), H, P, N))
    for s, (r0, r1) in enumerate(rows):
        starts = list(range(r0, r1, Q))
        for h in range(H):
            g = h // (H // G)
            y_diag, chunk_state, chunk_decay, decay_in = [], [], [], []
            for c0 in starts:
                c1 = min(c0 + Q, r1)
                la = Af[c0:c1, h]
                x, bb, cc = Xf[c0:c1, h], Bf[c0:c1, g], Cf[c0:c1, g]
                Lc = np.exp(segsum(la))
                # (1) diagonal block: intra-chunk output from a zero entry state
                y_diag.append((Lc * (cc @ bb.T)) @ x)
                # (2) right (B) factor: chunk's final state from a zero entry state
                chunk_state.append((x * Lc[-1][:, None]).T @ bb)
                chunk_decay.append(np.exp(np.sum(la)))
                decay_in.append(np.exp(np.cumsum(la)))
            # (3) center (A) factor: scalar SSM scan over chunks -> entry state of each chunk
            state = np.zeros((P, N)) if init is None else np.array(init[s, h], dtype=np.float64)
            entry = []
            for k in range(len(starts)):
                entry.append(state)
                state = chunk_decay[k] * state + chunk_state[k]
            final[s, h] = state
            # (4) left (C) factor: entry state -> output, decayed from the chunk start
            for k, c0 in enumerate(starts):
                c1 = min(c0 + Q, r1)
                cc = Cf[c0:c1, g]
                y_off = decay_in[k][:, None] * (cc @ entry[k].T)
                Y[c0:c1, h] = y_diag[k] + y_off
    return Y.reshape(b, T, H, P), final


def decode_step(state, x, logA, B, C):
    """One token of the recurrence for every sequence and head, from ``state``
    (section 2.4 with A_t = a_t I; the recurrent mode of section 3):
    S <- a S + x B^T, y = S C with a = exp(logA), S of head h using group h // (H // G).
    Shapes: state [b, H, P, N]; x [b, H, P]; logA [b, H]; B, C [b, G, N].
    Returns (y [b, H, P], new state [b, H, P, N]), float64; ``state`` is not modified."""
    S = _f64(state).copy()
    x, logA, B, C = _f64(x), _f64(logA), _f64(B), _f64(C)
    b, H, P, N = S.shape
    G = B.shape[1]
    hpg = H // G
    y = np.empty((b, H, P))
    for s in range(b):
        for h in range(H):
            g = h // hpg
            S[s, h] = np.exp(logA[s, h]) * S[s, h] + np.outer(x[s, h], B[s, g])
            y[s, h] = S[s, h] @ C[s, g]
    return y, S


def backward(X, logA, B, C, init=None, seq_offsets=None, dY=None, dfinal=None, nthreads: int = 0):
    """Gradients of L = <dY, Y> + <dfinal, final> with respect to X, logA, B, C and init,
    where (Y, final) = recurrence(X, logA, B, C, init, seq_offsets).  float64.
    Returns (dX [b,T,H,P], dlogA [b,T,H], dB, dC [b,T,G,N], dinit [nseq,H,P,N] or None)."""
    X, logA, B, C = _f64(X), _f64(logA), _f64(B), _f64(C)
    b, T, H, P, N, G = _shapes(X, logA, B, C)
    nseq = b if seq_offsets is None else int(np.asarray(seq_offsets).size - 1)
    dY = _f64(dY)
    assert dY.shape == X.shape, dY.shape
    dp = ctypes.POINTER(ctypes.c_double)
    init_p = dfinal_p = None
    if init is not None:
        init = _f64(init)
        assert init.shape == (nseq, H, P, N), init.shape
        init_p = init.ctypes.data_as(dp)
    if dfinal is not None:
        dfinal = _f64(dfinal)
        assert dfinal.shape == (nseq, H, P, N), dfinal.shape
        dfinal_p = dfinal.ctypes.data_as(dp)
    off_p = None
    if seq_offsets is not None:
        off = np.ascontiguousarray(np.asarray(seq_offsets, dtype=np.int64).reshape(-1))
        off_p = off.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    dX = np.zeros_like(X)
    dlogA = np.zeros_like(logA)
    dB = np.zeros_like(B)
    dC = np.zeros_like(C)
    dinit = np.zeros((nseq, H, P, N)) if init is not None else None
    rc = _load().ssd_oracle_backward(b, T, H, P, N, G, X.ctypes.data_as(dp), logA.ctypes.data_as(dp),
                                     B.ctypes.data_as(dp), C.ctypes.data_as(dp), init_p, off_p, nseq,
                                     dY.ctypes.data_as(dp), dfinal_p, dX.ctypes.data_as(dp),
                                     dlogA.ctypes.data_as(dp), dB.ctypes.data_as(dp),
                                     dC.ctypes.data_as(dp),
                                     None if dinit is None else dinit.ctypes.data_as(dp), int(nthreads))
    if rc != 0:
        raise ValueError(f"ssd_oracle_backward failed with code {rc}")
    return dX, dlogA, dB, dC, dinit
