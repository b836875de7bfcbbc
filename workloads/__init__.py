"""Seeded synthetic inputs for the SSD layer forward, shared by the tests, the smoke
check and the benchmark.

This module holds no arithmetic of the method itself: it only draws random tensors,
rounds them to the storage dtype, and describes the workload configurations.  The
draws are NumPy PCG64 streams from ``SeedSequence(seed)``, one spawned child per
tensor, so every tensor is reproducible on its own.

Value distributions (all configurations):
  X ~ N(0, 1); B, C ~ N(0, variance 1/N); Delta ~ U[0.001, 0.1] per (b, t, h);
  a_h ~ U[1, 16] per head (shared over batch and time); logA = -Delta * a_h, so the
  per-token decay a = exp(logA) lies in [0.20, 0.999]; the optional initial state
  is N(0, variance 0.1).  Values are drawn in float64, then rounded to float32, and
  for bf16 storage rounded once more to bf16 with round-to-nearest-even.  logA,
  the initial state and the final state are always float32.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

DTYPES = ("f32", "bf16")


def bf16_round(a) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returned as float32."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32).reshape(f.shape)


def bf16_bits(a) -> np.ndarray:
    """Upper 16 bits of float32 values already on the bf16 grid (for device upload)."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    return (f.view(np.uint32) >> 16).astype(np.uint16)


@dataclasses.dataclass
class Workload:
    name: str
    batch: int
    seqlen: int            # tokens per batch row (total packed tokens when varlen)
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk_len: int
    dtype: str             # "f32" or "bf16": storage / MFMA dtype of X, B, C, Y
    seed: int
    init_state: bool = False
    nseq: int = 0          # > 0: packed variable-length batch with this many sequences
    len_lo: int = 0
    len_hi: int = 0

    @property
    def varlen(self) -> bool:
        return self.nseq > 0

    def shape_dict(self):
        d = dict(batch=self.batch, seqlen=self.seqlen, nheads=self.nheads, headdim=self.headdim,
                 dstate=self.dstate, ngroups=self.ngroups, chunk_len=self.chunk_len,
                 dtype=self.dtype)
        if self.varlen:
            d["nseq"] = self.nseq
        return d


# The five workload configurations: index 0 is the tiny fp32 case, 1 the
# Mamba-2-2.7B-shaped layer the headline metric is quoted on, 2a/2b the state
# size sweep, 3 the long sequence, 4 the packed variable-length batch.
CONFIGS = {
    "cfg0_tiny_f32": Workload("cfg0_tiny_f32", 1, 256, 1, 16, 16, 1, 64, "f32", 1234 + 0),
    "cfg1_mamba2_2.7b_bf16": Workload("cfg1_mamba2_2.7b_bf16", 8, 2048, 80, 64, 128, 1, 256,
                                      "bf16", 1234 + 1),
    "cfg2a_state64_bf16": Workload("cfg2a_state64_bf16", 4, 4096, 32, 64, 64, 1, 256, "bf16",
                                   1234 + 2),
    "cfg2b_state256_bf16": Workload("cfg2b_state256_bf16", 4, 4096, 32, 64, 256, 1, 256, "bf16",
                                    1234 + 2),
    "cfg3_long16k_bf16": Workload("cfg3_long16k_bf16", 1, 16384, 80, 64, 128, 1, 256, "bf16",
                                  1234 + 3),
    "cfg4_varlen32k_bf16": Workload("cfg4_varlen32k_bf16", 1, 32768, 80, 64, 128, 8, 256, "bf16",
                                    1234 + 4, init_state=True, nseq=16, len_lo=256, len_hi=4096),
}
HEADLINE = "cfg1_mamba2_2.7b_bf16"


def packed_lengths(rng: np.random.Generator, nseq: int, total: int, lo: int, hi: int) -> List[int]:
    """Sequence lengths for a packed batch: draw nseq integers from U[lo, hi], scale them to
    sum to ``total``, clamp to [lo, hi], then hand out the remainder one token at a time in
    index order within the bounds."""
    assert nseq * lo <= total <= nseq * hi
    raw = rng.integers(lo, hi + 1, size=nseq).astype(np.float64)
    lens = np.clip(np.floor(raw * total / raw.sum()).astype(np.int64), lo, hi)
    rem = int(total - lens.sum())
    i = 0
    while rem != 0:
        step = 1 if rem > 0 else -1
        if lo <= lens[i] + step <= hi:
            lens[i] += step
            rem -= step
        i = (i + 1) % nseq
    return [int(v) for v in lens]


@dataclasses.dataclass
class Inputs:
    """Host tensors on the storage grid (float32 arrays; bf16 values are exactly representable)."""
    X: np.ndarray                 # [b, T, H, P]
    logA: np.ndarray              # [b, T, H] float32
    B: np.ndarray                 # [b, T, G, N]
    C: np.ndarray                 # [b, T, G, N]
    init: Optional[np.ndarray]    # [nseq, H, P, N] float32 or None
    seq_offsets: Optional[np.ndarray]   # [nseq + 1] int32 or None
    dtype: str


def make_inputs(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int, ngroups: int,
                dtype: str, seed: int, init_state: bool = False,
                seq_lengths: Optional[List[int]] = None, heads: Optional[List[int]] = None,
                ) -> Inputs:
    """Draw one problem.  ``seq_lengths`` makes it a packed batch (batch must be 1 and the
    lengths must sum to ``seqlen``).  ``heads`` restricts X, logA and init to those head
    indices (B and C keep every group); the draws are the same as for the full problem."""
    assert dtype in DTYPES
    b, T, H, P, N, G = batch, seqlen, nheads, headdim, dstate, ngroups
    ss = np.random.SeedSequence(seed)
    kx, kb, kc, kd, ka, ki = ss.spawn(6)
    X = np.random.Generator(np.random.PCG64(kx)).standard_normal((b, T, H, P))
    Bm = np.random.Generator(np.random.PCG64(kb)).standard_normal((b, T, G, N)) / np.sqrt(N)
    Cm = np.random.Generator(np.random.PCG64(kc)).standard_normal((b, T, G, N)) / np.sqrt(N)
    delta = np.random.Generator(np.random.PCG64(kd)).uniform(0.001, 0.1, size=(b, T, H))
    a_h = np.random.Generator(np.random.PCG64(ka)).uniform(1.0, 16.0, size=(H,))
    logA = (-delta * a_h[None, None, :]).astype(np.float32)
    offsets = None
    nseq = b
    if seq_lengths is not None:
        assert b == 1 and sum(seq_lengths) == T
        nseq = len(seq_lengths)
        offsets = np.zeros(nseq + 1, dtype=np.int32)
        offsets[1:] = np.cumsum(seq_lengths)
    init = None
    if init_state:
        init = (np.random.Generator(np.random.PCG64(ki)).standard_normal((nseq, H, P, N))
                * np.sqrt(0.1)).astype(np.float32)
    X = X.astype(np.float32)
    Bm = Bm.astype(np.float32)
    Cm = Cm.astype(np.float32)
    if dtype == "bf16":
        X, Bm, Cm = bf16_round(X), bf16_round(Bm), bf16_round(Cm)
    if heads is not None:
        X = np.ascontiguousarray(X[:, :, heads])
        logA = np.ascontiguousarray(logA[:, :, heads])
        if init is not None:
            init = np.ascontiguousarray(init[:, heads])
    return Inputs(X, logA, Bm, Cm, init, offsets, dtype)


def workload_inputs(w: Workload, heads: Optional[List[int]] = None) -> Inputs:
    lengths = None
    if w.varlen:
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(w.seed + 1000)))
        lengths = packed_lengths(rng, w.nseq, w.seqlen, w.len_lo, w.len_hi)
    return make_inputs(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.dtype,
                       w.seed, init_state=w.init_state, seq_lengths=lengths, heads=heads)
