"""ctypes binding of libarcs.so (argument marshalling only).

Every computation runs in the library's HIP kernels; this module checks
tensor shapes, dtypes and devices, takes raw device pointers and the current
HIP stream from PyTorch, and calls the C ABI of include/arcs.h with the same
names.  It never falls back to any other implementation: if the library is
missing or a call fails, it raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libarcs.so")

DTYPE_BF16 = 0
DTYPE_F32 = 1

# C enum values of include/arcs.h
OK = 0
ERR_NULL_POINTER = -1
ERR_BAD_BATCH = -2
ERR_BAD_VOCAB = -3
ERR_BAD_STRIDE = -4
ERR_BAD_DTYPE = -5
ERR_WORKSPACE_TOO_SMALL = -6
ERR_LAUNCH = -7
ERR_MISALIGNED = -8
ERR_BAD_HISTORY = -9
ERR_BAD_TOP_N = -10
ERR_BAD_CAPACITY = -11
ERR_SCRATCH_TOO_SMALL = -12
ERR_BAD_BUDGET = -13
ERR_BAD_DRY = -14
DRY_MAX_WINDOW = 2048
DRY_MAX_BREAKERS = 64
NOALLOC_SCRATCH_BYTES = 16384
ROW_OK = 0
ROW_BAD_TEMPERATURE = 1
ROW_BAD_TOP_P = 2
ROW_BAD_MIN_P = 3
ROW_BAD_PENALTY = 4
ROW_BAD_FLAGS = 5
ROW_TIES_WIDE = 1  # arcs_row_params.flags bit
ROW_HISTORY_TOO_LONG = 6
ROW_VOCAB_TOO_LARGE = 7
MAX_HISTORY = 4096
MAX_PENALTY_VOCAB = 262144
TOP_LOGPROBS_MAX_VOCAB = 262144  # ARCS_TOP_LOGPROBS_MAX_VOCAB

PATH_GREEDY = 1
PATH_SORT_SKIP = 2
PATH_CUTOFF = 4
PATH_MINP_FLOOR = 8
PATH_TIE_SPLIT = 16
PATH_PENALTY = 32
PATH_SPECIAL = 64
PATH_RESIDENT = 128
PATH_REREAD = 256

# struct arcs_row_params (32 bytes)
ROW_PARAMS_DTYPE = np.dtype(
    [("temperature", "<f4"), ("top_k", "<i4"), ("top_p", "<f4"), ("min_p", "<f4"),
     ("presence", "<f4"), ("frequency", "<f4"), ("repetition", "<f4"), ("flags", "<i4")]
)
# struct arcs_row_stats (64 bytes)
ROW_STATS_DTYPE = np.dtype(
    [("id", "<i4"), ("argmax", "<i4"), ("kept", "<i4"), ("cut_index", "<i4"),
     ("cut_value", "<f4"), ("max_logit", "<f4"), ("status", "<i4"), ("path", "<u4"),
     ("mass_total", "<f8"), ("mass_kept", "<f8"), ("uniform", "<f8"), ("reserved", "<u8")]
)
assert ROW_PARAMS_DTYPE.itemsize == 32 and ROW_STATS_DTYPE.itemsize == 64


class ArcsError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: arcs status {code} ({status_string(code)})")


_lib = None


def library() -> ctypes.CDLL:
    """Load libarcs.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
        lib = ctypes.CDLL(LIB_PATH)
        c_i64, c_u64, c_p, c_i = ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int
        lib.arcs_argmax.argtypes = [c_p, c_i, c_i64, c_i64, c_i64, c_p, c_p]
        lib.arcs_argmax.restype = c_i
        lib.arcs_sample.argtypes = [c_p, c_i, c_i64, c_i64, c_i64, c_p, c_p, c_p, c_u64, c_u64,
                                    c_p, c_p, c_p, ctypes.c_size_t, c_p]
        lib.arcs_sample.restype = c_i
        lib.arcs_sample_debug.argtypes = [c_p, c_i, c_i64, c_i64, c_i64, c_p, c_p, c_p, c_u64, c_u64,
                                          c_p, c_p, c_p, ctypes.c_size_t, c_p, c_p, c_p, c_p]
        lib.arcs_sample_debug.restype = c_i
        lib.arcs_sample_dry.argtypes = [c_p, c_i, c_i64, c_i64, c_i64, c_p, c_p, c_p, c_p, c_p, c_i, c_u64,
                                         c_u64, c_p, c_p, c_p, c_u64, c_p]
        lib.arcs_sample_dry.restype = c_i
        lib.arcs_sample_hybrid_nucleus.argtypes = [c_p, c_i, c_i64, c_i64, c_i64, c_p, c_p, c_i, c_u64, c_u64,
                                                    c_p, c_p, c_p, c_p]
        lib.arcs_sample_hybrid_nucleus.restype = c_i
        lib.arcs_sample_noalloc.argtypes = [c_p, c_i, c_i64, c_i64, c_i64, c_p, c_p, c_p, c_u64, c_u64,
                                             c_p, c_p, c_p]
        lib.arcs_sample_noalloc.restype = c_i
        lib.arcs_sample_keyed.argtypes = [c_p, c_i, c_i64, c_i64, c_i64, c_p, c_p, c_p, c_p, c_i,
                                          c_p, c_p, c_p, ctypes.c_size_t, c_p]
        lib.arcs_sample_keyed.restype = c_i
        lib.arcs_top_logprobs.argtypes = [c_p, c_i, c_i64, c_i64, c_i64, c_p, c_i, c_p, c_p, c_p, c_p]
        lib.arcs_top_logprobs.restype = c_i
        lib.arcs_commit_tokens.argtypes = [c_p, c_i64, c_i64, c_p, c_p, c_p, c_u64, c_p, c_p, c_p, c_p]
        lib.arcs_commit_tokens.restype = c_i
        lib.arcs_sample_workspace_bytes.argtypes = [c_i64, c_i64, c_i]
        lib.arcs_sample_workspace_bytes.restype = ctypes.c_size_t
        lib.arcs_long_history_workspace_bytes.argtypes = [c_i64, c_i64]
        lib.arcs_long_history_workspace_bytes.restype = ctypes.c_size_t
        lib.arcs_status_string.argtypes = [c_i]
        lib.arcs_status_string.restype = ctypes.c_char_p
        lib.arcs_version.argtypes = []
        lib.arcs_version.restype = c_i
        _lib = lib
    return _lib


def status_string(code: int) -> str:
    return library().arcs_status_string(int(code)).decode()


def version() -> int:
    return int(library().arcs_version())


def workspace_bytes(B: int, V: int, dtype: int) -> int:
    return int(library().arcs_sample_workspace_bytes(int(B), int(V), int(dtype)))


def long_history_workspace_bytes(B: int, V: int) -> int:
    return int(library().arcs_long_history_workspace_bytes(int(B), int(V)))


# --------------------------------------------------------------------------
# torch-facing helpers
# --------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream_ptr(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _check_logits(logits):
    if not logits.is_cuda:
        raise ValueError("logits must be a device tensor")
    if logits.dim() != 2:
        raise ValueError("logits must be [B, V]")
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous (stride(1) == 1)")
    return logits.shape[0], logits.shape[1], logits.stride(0)


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def params_to_device(params: np.ndarray, device="cuda"):
    """Copy a structured array of arcs_row_params records to the device (uint8 [B, 32])."""
    torch = _torch()
    arr = np.ascontiguousarray(params).view(np.uint8).reshape(len(params), 32)
    return torch.from_numpy(arr.copy()).to(device)


def _check_out(t, dtype, n: int, name: str):
    """A caller-provided device buffer: dtype, element count and a dense layout
    (the kernels write from the base pointer in row order)."""
    torch = _torch()
    if t.dtype != dtype or t.numel() != n or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device {dtype} tensor of {n} elements")


def argmax(logits, out=None, stream=None):
    """out[b] = lowest index of the row maximum of logits[b] (int32, on device)."""
    torch = _torch()
    B, V, stride = _check_logits(logits)
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=logits.device)
    _check_out(out, torch.int32, B, "out")
    st = library().arcs_argmax(_ptr(logits), _dtype_code(logits), B, V, stride, _ptr(out), _stream_ptr(stream))
    if st != OK:
        raise ArcsError(st, "arcs_argmax")
    return out


def top_logprobs(logits, n: int, temperature=None, out_ids=None, out_logprobs=None, out_status=None,
                 stream=None):
    """arcs_top_logprobs: (ids int32 [B, n], logprobs float32 [B, n]) on device.

    ``temperature`` is a device float32 tensor of B values or None (T = 1);
    ``out_status`` an optional device int32 tensor of B values.
    """
    torch = _torch()
    B, V, stride = _check_logits(logits)
    dev = logits.device
    if temperature is not None and (temperature.dtype != torch.float32 or not temperature.is_cuda
                                    or temperature.numel() != B or not temperature.is_contiguous()):
        raise ValueError("temperature must be a contiguous device float32 tensor of B elements")
    if out_ids is None:
        out_ids = torch.empty((B, n), dtype=torch.int32, device=dev)
    if out_logprobs is None:
        out_logprobs = torch.empty((B, n), dtype=torch.float32, device=dev)
    if out_ids.dtype != torch.int32 or out_ids.numel() != B * n or not out_ids.is_cuda or not out_ids.is_contiguous():
        raise ValueError("out_ids must be a device int32 tensor of B * n elements")
    if (out_logprobs.dtype != torch.float32 or out_logprobs.numel() != B * n or not out_logprobs.is_cuda
            or not out_logprobs.is_contiguous()):
        raise ValueError("out_logprobs must be a device float32 tensor of B * n elements")
    if out_status is not None:
        _check_out(out_status, torch.int32, B, "out_status")
    st = library().arcs_top_logprobs(_ptr(logits), _dtype_code(logits), B, V, stride, _ptr(temperature),
                                     int(n), _ptr(out_ids), _ptr(out_logprobs), _ptr(out_status),
                                     _stream_ptr(stream))
    if st != OK:
        raise ArcsError(st, "arcs_top_logprobs")
    return out_ids, out_logprobs


def commit_tokens(ids, V: int, position, ring, published, drained, fault, next_input=None, stream=None):
    """arcs_commit_tokens: publish one step's tokens into a pinned host ring.

    ``ids`` device int32 [B]; ``position`` device int64 [1]; ``ring`` pinned
    CPU int32 [capacity, B]; ``published`` and ``drained`` pinned CPU int64
    [1]; ``fault`` pinned CPU int32 [1]; ``next_input`` device int32 [B] or None.
    """
    torch = _torch()
    B = ids.numel()
    if not ids.is_cuda or ids.dtype != torch.int32 or not ids.is_contiguous():
        raise ValueError("ids must be a contiguous device int32 tensor")
    _check_out(position, torch.int64, 1, "position")
    for name, t, dt in (("ring", ring, torch.int32), ("published", published, torch.int64),
                        ("drained", drained, torch.int64), ("fault", fault, torch.int32)):
        if t.is_cuda or not t.is_pinned() or t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous pinned CPU tensor of {dt}")
    if ring.numel() % B != 0:
        raise ValueError("ring must hold capacity * B elements")
    if next_input is not None:
        _check_out(next_input, torch.int32, B, "next_input")
    st = library().arcs_commit_tokens(_ptr(ids), B, int(V), _ptr(next_input), _ptr(position), _ptr(ring),
                                      ring.numel() // B, _ptr(published), _ptr(drained), _ptr(fault),
                                      _stream_ptr(stream))
    if st != OK:
        raise ArcsError(st, "arcs_commit_tokens")


def _check_params(params, B):
    torch = _torch()
    if not params.is_cuda or params.dtype != torch.uint8 or params.numel() != 32 * B or not params.is_contiguous():
        raise ValueError("params must be a contiguous device uint8 tensor of B * 32 bytes")


def _check_hist(hist_ids, hist_offsets, B):
    torch = _torch()
    if (hist_ids is None) != (hist_offsets is None):
        raise ValueError("hist_ids and hist_offsets go together")
    if hist_ids is not None:
        if hist_ids.dtype != torch.int32 or not hist_ids.is_cuda or not hist_ids.is_contiguous():
            raise ValueError("hist_ids must be a contiguous device int32 tensor")
        _check_out(hist_offsets, torch.int64, B + 1, "hist_offsets")


def sample(logits, params, hist_ids=None, hist_offsets=None, seed: int = 0, step: int = 0,
           out=None, out_status=None, workspace=None, stream=None):
    """One token per row (int32, on device); see arcs_sample in include/arcs.h."""
    torch = _torch()
    B, V, stride = _check_logits(logits)
    _check_params(params, B)
    _check_hist(hist_ids, hist_offsets, B)
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=logits.device)
    _check_out(out, torch.int32, B, "out")
    if out_status is not None:
        _check_out(out_status, torch.int32, B, "out_status")
    ws_need = workspace_bytes(B, V, _dtype_code(logits))
    if workspace is not None and (not workspace.is_cuda or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous device tensor")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if ws_need and workspace is None:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=logits.device)
        ws_bytes = ws_need
    st = library().arcs_sample(_ptr(logits), _dtype_code(logits), B, V, stride, _ptr(params),
                               _ptr(hist_ids), _ptr(hist_offsets), int(seed) & (2**64 - 1),
                               int(step) & (2**64 - 1), _ptr(out), _ptr(out_status), _ptr(workspace),
                               ws_bytes, _stream_ptr(stream))
    if st != OK:
        raise ArcsError(st, "arcs_sample")
    return out


def sample_noalloc(logits, params, hist_ids=None, hist_offsets=None, seed: int = 0, step: int = 0,
                   out=None, out_status=None, stream=None):
    """arcs_sample_noalloc: as sample, with the library's own device scratch
    instead of a workspace (the C call allocates nothing; pass `out` to keep
    this wrapper from allocating it)."""
    torch = _torch()
    B, V, stride = _check_logits(logits)
    _check_params(params, B)
    _check_hist(hist_ids, hist_offsets, B)
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=logits.device)
    _check_out(out, torch.int32, B, "out")
    if out_status is not None:
        _check_out(out_status, torch.int32, B, "out_status")
    st = library().arcs_sample_noalloc(_ptr(logits), _dtype_code(logits), B, V, stride, _ptr(params),
                                       _ptr(hist_ids), _ptr(hist_offsets), int(seed) & (2**64 - 1),
                                       int(step) & (2**64 - 1), _ptr(out), _ptr(out_status), _stream_ptr(stream))
    if st != OK:
        raise ArcsError(st, "arcs_sample_noalloc")
    return out


def dry_to_device(dry, device="cuda"):
    """A DRY_DTYPE structured numpy array (workloads.make_dry) as device bytes."""
    torch = _torch()
    arr = np.ascontiguousarray(dry).view(np.uint8).reshape(len(dry), 16)
    return torch.from_numpy(arr.copy()).to(device)


def sample_dry(logits, params, hist_ids, hist_offsets, dry, breakers=None, seed: int = 0, step: int = 0,
               out=None, out_status=None, workspace=None, stream=None):
    """arcs_sample_dry: arcs_sample with per-row DRY records (device bytes from
    dry_to_device) and optional device int32 sequence breakers."""
    torch = _torch()
    B, V, stride = _check_logits(logits)
    _check_params(params, B)
    _check_hist(hist_ids, hist_offsets, B)
    if dry is not None and (not dry.is_cuda or dry.dtype != torch.uint8 or dry.numel() != 16 * B
                            or not dry.is_contiguous()):
        raise ValueError("dry must be contiguous device bytes of B DRY records (dry_to_device)")
    nb = 0
    if breakers is not None:
        nb = breakers.numel()
        _check_out(breakers, torch.int32, nb, "breakers")
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=logits.device)
    _check_out(out, torch.int32, B, "out")
    if out_status is not None:
        _check_out(out_status, torch.int32, B, "out_status")
    ws_need = workspace_bytes(B, V, _dtype_code(logits))
    if ws_need and workspace is None:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=logits.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = library().arcs_sample_dry(_ptr(logits), _dtype_code(logits), B, V, stride, _ptr(params), _ptr(hist_ids),
                                   _ptr(hist_offsets), _ptr(dry), _ptr(breakers), nb, int(seed) & (2**64 - 1),
                                   int(step) & (2**64 - 1), _ptr(out), _ptr(out_status), _ptr(workspace),
                                   ws_bytes, _stream_ptr(stream))
    if st != OK:
        raise ArcsError(st, "arcs_sample_dry")
    return out


def sample_hybrid_nucleus(logits, temperature, top_p, budget: int = 32, seed: int = 0, step: int = 0,
                          out=None, out_kept=None, out_status=None, stream=None):
    """arcs_sample_hybrid_nucleus: the baseline enumeration / bisection nucleus
    sampler (per-row float32 temperature and top_p on the device)."""
    torch = _torch()
    B, V, stride = _check_logits(logits)
    for name, t in (("temperature", temperature), ("top_p", top_p)):
        _check_out(t, torch.float32, B, name)
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=logits.device)
    _check_out(out, torch.int32, B, "out")
    for name, t in (("out_kept", out_kept), ("out_status", out_status)):
        if t is not None:
            _check_out(t, torch.int32, B, name)
    st = library().arcs_sample_hybrid_nucleus(_ptr(logits), _dtype_code(logits), B, V, stride, _ptr(temperature),
                                              _ptr(top_p), int(budget), int(seed) & (2**64 - 1),
                                              int(step) & (2**64 - 1), _ptr(out), _ptr(out_kept),
                                              _ptr(out_status), _stream_ptr(stream))
    if st != OK:
        raise ArcsError(st, "arcs_sample_hybrid_nucleus")
    return out


def make_key(seed: int = 0, step: int = 0, device="cuda"):
    """A device RNG key {seed, step} for sample_keyed (int64 storage of the
    two uint64 words)."""
    torch = _torch()
    words = [int(seed) & (2**64 - 1), int(step) & (2**64 - 1)]
    words = [w - 2**64 if w >= 2**63 else w for w in words]
    return torch.tensor(words, dtype=torch.int64, device=device)


def sample_keyed(logits, params, key, hist_ids=None, hist_offsets=None, advance: bool = True,
                 out=None, out_status=None, workspace=None, stream=None):
    """arcs_sample_keyed: seed and step read from the device key (see make_key);
    with `advance` the key's step moves on by one after the draw."""
    torch = _torch()
    B, V, stride = _check_logits(logits)
    _check_params(params, B)
    _check_hist(hist_ids, hist_offsets, B)
    if not key.is_cuda or key.dtype != torch.int64 or key.numel() != 2 or not key.is_contiguous():
        raise ValueError("key must be a contiguous device int64 tensor of 2 elements (seed, step)")
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=logits.device)
    _check_out(out, torch.int32, B, "out")
    if out_status is not None:
        _check_out(out_status, torch.int32, B, "out_status")
    ws_need = workspace_bytes(B, V, _dtype_code(logits))
    if workspace is not None and (not workspace.is_cuda or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous device tensor")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if ws_need and workspace is None:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=logits.device)
        ws_bytes = ws_need
    st = library().arcs_sample_keyed(_ptr(logits), _dtype_code(logits), B, V, stride, _ptr(params),
                                     _ptr(hist_ids), _ptr(hist_offsets), _ptr(key), 1 if advance else 0,
                                     _ptr(out), _ptr(out_status), _ptr(workspace), ws_bytes,
                                     _stream_ptr(stream))
    if st != OK:
        raise ArcsError(st, "arcs_sample_keyed")
    return out


def sample_debug(logits, params, hist_ids=None, hist_offsets=None, seed: int = 0, step: int = 0,
                 uniforms=None, want_probs: bool = False, workspace=None, stream=None):
    """arcs_sample_debug: returns (ids, status, stats[B] numpy structured, probs or None)."""
    torch = _torch()
    B, V, stride = _check_logits(logits)
    _check_params(params, B)
    _check_hist(hist_ids, hist_offsets, B)
    dev = logits.device
    out = torch.empty(B, dtype=torch.int32, device=dev)
    status = torch.empty(B, dtype=torch.int32, device=dev)
    stats = torch.zeros(B * ROW_STATS_DTYPE.itemsize, dtype=torch.uint8, device=dev)
    probs = torch.empty((B, V), dtype=torch.float32, device=dev) if want_probs else None
    if uniforms is not None:
        _check_out(uniforms, torch.float64, B, "uniforms")
    ws_need = workspace_bytes(B, V, _dtype_code(logits))
    if workspace is not None and (not workspace.is_cuda or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous device tensor")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if ws_need and workspace is None:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
        ws_bytes = ws_need
    st = library().arcs_sample_debug(_ptr(logits), _dtype_code(logits), B, V, stride, _ptr(params),
                                     _ptr(hist_ids), _ptr(hist_offsets), int(seed) & (2**64 - 1),
                                     int(step) & (2**64 - 1), _ptr(out), _ptr(status), _ptr(workspace),
                                     ws_bytes, _ptr(uniforms), _ptr(probs), _ptr(stats), _stream_ptr(stream))
    if st != OK:
        raise ArcsError(st, "arcs_sample_debug")
    torch.cuda.synchronize(dev)
    st_np = stats.cpu().numpy().view(ROW_STATS_DTYPE)
    return out, status, st_np, probs
