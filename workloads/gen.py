"""Seeded synthetic sampler workloads.

The pages describe a DeepSeek-V4 LM head with a 129,280-token vocabulary,
decode batches up to 512 rows, the server defaults (top_k=-1, top_p=1,
min_p=0) and the bench settings T=0.7 / top_k=32 / top_p=0.95 (ArcInfer PR
#222, "ARC_SAMPLE_ON_DEVICE" premise and the CPU probe table; PR #194, the
H200 batch sweep).  Real LM-head logits are not available, so these inputs
stand in for them with the same shapes:

* ``normal``: logits ~ N(0, 3^2), 4 rows.
* ``zipf``: logit[v] = -1.1*ln(rank(v)) + N(0, 0.5^2), rank a seeded
  permutation of 1..V per row (an LM-head-like heavy head and long tail).
* ``flat``: logit[v] = -0.3*ln(rank(v)) + N(0, 1), fp32, a flat tail whose
  top-p=0.95 nucleus spans tens of thousands of tokens.

Every row is drawn from its own numpy PCG64 stream keyed by
(workload seed, row, purpose), so any subset of rows can be regenerated on
its own.  Values are computed in float64, rounded to float32 and then,
for bf16 workloads, rounded to bfloat16 with round-to-nearest-even.

Nothing here implements the sampler: the per-row parameter record is only a
data layout (32 bytes, see ``PARAMS_DTYPE``).
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

V_DEFAULT = 129_280

# Per-row parameter record, 32 bytes, little endian, field order fixed.
PARAMS_DTYPE = np.dtype(
    [
        ("temperature", "<f4"),
        ("top_k", "<i4"),
        ("top_p", "<f4"),
        ("min_p", "<f4"),
        ("presence", "<f4"),
        ("frequency", "<f4"),
        ("repetition", "<f4"),
        ("flags", "<i4"),
    ]
)
assert PARAMS_DTYPE.itemsize == 32

# Per-row DRY penalty record, 16 bytes (arcs_dry_params).
DRY_DTYPE = np.dtype([("multiplier", "<f4"), ("base", "<f4"), ("allowed_length", "<i4"), ("range", "<i4")])
assert DRY_DTYPE.itemsize == 16


def make_dry(n: int, multiplier=0.0, base=1.75, allowed_length=2, range=0) -> np.ndarray:
    """DRY records for ``n`` rows (scalars broadcast)."""
    d = np.zeros(n, dtype=DRY_DTYPE)
    d["multiplier"] = multiplier
    d["base"] = base
    d["allowed_length"] = allowed_length
    d["range"] = range
    return d

_PURPOSE_LOGITS = 0
_PURPOSE_PARAMS = 1
_PURPOSE_HISTORY = 2


def _row_rng(seed: int, row: int, purpose: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, row, purpose])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Inputs must be finite; returns the raw 16-bit patterns as uint16.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of raw bfloat16 patterns to float32 (bit shift)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_params(n: int, temperature=1.0, top_k=-1, top_p=1.0, min_p=0.0,
                presence=0.0, frequency=0.0, repetition=1.0, flags=0) -> np.ndarray:
    """Uniform parameter records for ``n`` rows (scalars broadcast)."""
    p = np.zeros(n, dtype=PARAMS_DTYPE)
    p["temperature"] = temperature
    p["top_k"] = top_k
    p["top_p"] = top_p
    p["min_p"] = min_p
    p["presence"] = presence
    p["frequency"] = frequency
    p["repetition"] = repetition
    p["flags"] = flags
    return p


@dataclasses.dataclass
class Workload:
    name: str
    B: int                      # rows in the full batch
    V: int                      # vocabulary size
    dtype: str                  # "bf16" (uint16 bit patterns) or "f32"
    logits: np.ndarray          # [len(rows), V] uint16 or float32
    params: np.ndarray          # [len(rows)] PARAMS_DTYPE
    hist_ids: Optional[np.ndarray]      # int32 CSR values, or None
    hist_offsets: Optional[np.ndarray]  # int64 [len(rows)+1], or None
    seed: int                   # sampling seed
    step: int                   # sampling step
    rows: np.ndarray            # original row indices of the rows held here
    greedy_only: bool           # the workload is an argmax-only batch
    top_n: int = 0              # > 0: a top-n logprobs batch (temperature from params)

    @property
    def nbytes_logits(self) -> int:
        return int(self.logits.nbytes)


def _logits_row(kind: str, seed: int, row: int, V: int) -> np.ndarray:
    rng = _row_rng(seed, row, _PURPOSE_LOGITS)
    if kind == "normal":
        x = rng.normal(0.0, 3.0, V)
    elif kind == "zipf":
        rank = rng.permutation(V).astype(np.float64) + 1.0
        x = -1.1 * np.log(rank) + rng.normal(0.0, 0.5, V)
    elif kind == "flat":
        rank = rng.permutation(V).astype(np.float64) + 1.0
        x = -0.3 * np.log(rank) + rng.normal(0.0, 1.0, V)
    else:
        raise ValueError(kind)
    return x.astype(np.float32)


# name -> (logit kind, dtype, default B, logits seed, argmax-only)
_SPECS = {
    "normal_b4_bf16": ("normal", "bf16", 4, 0, False),
    "zipf_b256_bf16_greedy": ("zipf", "bf16", 256, 1, True),
    "zipf_b256_bf16_t0.7_k50_p0.9_minp0.05": ("zipf", "bf16", 256, 1, False),
    "zipf_b512_bf16_mixed_penalties": ("zipf", "bf16", 512, 2, False),
    "flat_b1024_f32_t1_p0.95": ("flat", "f32", 1024, 3, False),
    "zipf_b256_bf16_top_logprobs20": ("zipf", "bf16", 256, 1, False),
}
WORKLOAD_NAMES = tuple(_SPECS)


def _params_row(name: str, seed: int, row: int, B: int) -> tuple:
    """(temperature, top_k, top_p, min_p, presence, frequency, repetition)."""
    if name == "normal_b4_bf16":
        return (1.0, -1, 1.0, 0.0, 0.0, 0.0, 1.0)
    if name == "zipf_b256_bf16_greedy":
        return (0.0, -1, 1.0, 0.0, 0.0, 0.0, 1.0)
    if name == "zipf_b256_bf16_t0.7_k50_p0.9_minp0.05":
        return (0.7, 50, 0.9, 0.05, 0.0, 0.0, 1.0)
    if name == "zipf_b256_bf16_top_logprobs20":
        return (0.7, -1, 1.0, 0.0, 0.0, 0.0, 1.0)
    if name == "flat_b1024_f32_t1_p0.95":
        return (1.0, -1, 0.95, 0.0, 0.0, 0.0, 1.0)
    if name == "zipf_b512_bf16_mixed_penalties":
        rng = _row_rng(seed, row, _PURPOSE_PARAMS)
        group = min(3, (4 * row) // max(B, 1))
        t = float(rng.uniform(0.3, 1.5))
        pen = (0.5, 0.3, 1.1)
        if group == 0:      # greedy (top_k = 1)
            return (t, 1, 1.0, 0.0) + pen
        if group == 1:      # server defaults: no filter
            return (t, -1, 1.0, 0.0) + pen
        if group == 2:      # top-k only
            return (t, int(rng.integers(20, 1001)), 1.0, 0.0) + pen
        return (t, -1, float(rng.uniform(0.5, 0.95)), 0.02) + pen
    raise ValueError(name)


def make_workload(name: str, B: Optional[int] = None, V: int = V_DEFAULT,
                  rows: Optional[Sequence[int]] = None, seed: int = 0, step: int = 0,
                  hist_len: int = 1024) -> Workload:
    """Build a named workload.

    ``B`` overrides the batch size, ``V`` the vocabulary, ``rows`` selects a
    subset of rows (their logits/params/history are identical to those rows
    of the full batch).  ``seed``/``step`` are the sampling seed and step.
    """
    kind, dtype, B0, lseed, greedy = _SPECS[name]
    B = B0 if B is None else int(B)
    rows = np.arange(B, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    n = len(rows)
    f32 = np.empty((n, V), dtype=np.float32)
    for i, r in enumerate(rows):
        f32[i] = _logits_row(kind, lseed, int(r), V)
    logits = f32_to_bf16_bits(f32) if dtype == "bf16" else f32
    params = np.zeros(n, dtype=PARAMS_DTYPE)
    for i, r in enumerate(rows):
        t, k, p, mp, pres, freq, rep = _params_row(name, lseed, int(r), B)
        params[i] = (t, k, p, mp, pres, freq, rep, 0)
    hist_ids = hist_offsets = None
    if name == "zipf_b512_bf16_mixed_penalties":
        hs = []
        for r in rows:
            rng = _row_rng(lseed, int(r), _PURPOSE_HISTORY)
            hs.append(rng.integers(0, V, hist_len, dtype=np.int64).astype(np.int32))
        hist_ids = np.concatenate(hs) if hs else np.zeros(0, np.int32)
        hist_offsets = np.arange(n + 1, dtype=np.int64) * hist_len
    return Workload(name=name, B=B, V=V, dtype=dtype, logits=logits, params=params,
                    hist_ids=hist_ids, hist_offsets=hist_offsets, seed=seed, step=step,
                    rows=rows, greedy_only=greedy,
                    top_n=20 if name == "zipf_b256_bf16_top_logprobs20" else 0)
