"""Shared helpers for the tests (no sampler arithmetic here)."""

import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "arcs.h")


def ensure_built():
    import decode_step_token_row_amd as arcs
    if not os.path.exists(arcs.LIB_PATH):
        from decode_step_token_row_amd import build
        build.build()
    return arcs


def header_functions():
    """Names of the functions include/arcs.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*(arcs_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def to_device_logits(logits_np, dtype, device="cuda", stride=None):
    """numpy bf16 bit patterns (uint16) or float32 -> device tensor [B, V].

    With ``stride`` > V the rows are laid out in a wider buffer (a view).
    """
    import torch
    B, V = logits_np.shape
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(logits_np).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(logits_np, dtype=np.float32))
    if stride is None or stride == V:
        return t.to(device)
    big = torch.zeros((B, stride), dtype=t.dtype)
    big[:, :V] = t
    return big.to(device)[:, :V]


def hist_to_device(w, device="cuda"):
    import torch
    if w.hist_ids is None:
        return None, None
    return (torch.from_numpy(w.hist_ids).to(device), torch.from_numpy(w.hist_offsets).to(device))
