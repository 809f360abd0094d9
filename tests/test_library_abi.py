"""The C-ABI library loads, exports every symbol include/arcs.h declares, and
rejects bad host arguments before launching anything (no GPU needed)."""

import ctypes
import os
import subprocess

import numpy as np
import pytest

from _util import ensure_built, header_functions


@pytest.fixture(scope="module")
def arcs():
    return ensure_built()


def test_header_declares_the_boundary():
    fns = header_functions()
    for name in ("arcs_argmax", "arcs_sample", "arcs_sample_keyed", "arcs_sample_workspace_bytes",
                 "arcs_status_string", "arcs_sample_debug", "arcs_version", "arcs_top_logprobs",
                 "arcs_commit_tokens", "arcs_sample_noalloc", "arcs_sample_hybrid_nucleus",
                 "arcs_sample_dry", "arcs_long_history_workspace_bytes"):
        assert name in fns


def test_library_exports_every_declared_symbol(arcs):
    lib = arcs.library()
    out = subprocess.run(["nm", "-D", "--defined-only", arcs.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for name in header_functions():
        assert hasattr(lib, name), name
        assert name in exported, name


def test_status_strings_and_version(arcs):
    for code in [0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10, -11, -12, -13, -14, 1, 2, 3, 4, 5, 6, 7]:
        assert arcs.status_string(code) != "unknown status", code
    assert arcs.status_string(12345) == "unknown status"
    assert arcs.version() >= 100
    assert arcs.workspace_bytes(256, 129280, arcs.DTYPE_BF16) >= 0


def test_struct_layouts_match_the_header(arcs):
    from workloads import PARAMS_DTYPE
    assert arcs.ROW_PARAMS_DTYPE == PARAMS_DTYPE
    assert arcs.ROW_PARAMS_DTYPE.itemsize == 32 and arcs.ROW_STATS_DTYPE.itemsize == 64


def test_host_validation_rejects_before_launch(arcs):
    lib = arcs.library()
    buf = (ctypes.c_uint8 * 4096)()
    base = (ctypes.addressof(buf) + 63) // 64 * 64  # aligned dummy address, never dereferenced
    p = ctypes.c_void_p(base)
    # argmax
    assert lib.arcs_argmax(None, 0, 4, 10, 10, p, None) == -1
    assert lib.arcs_argmax(p, 0, 4, 10, 10, None, None) == -1
    assert lib.arcs_argmax(p, 7, 4, 10, 10, p, None) == -5
    assert lib.arcs_argmax(p, 0, 0, 10, 10, p, None) == -2
    assert lib.arcs_argmax(p, 0, -3, 10, 10, p, None) == -2
    assert lib.arcs_argmax(p, 0, 4, 0, 10, p, None) == -3
    assert lib.arcs_argmax(p, 0, 4, 2**31, 2**31, p, None) == -3
    assert lib.arcs_argmax(p, 0, 4, 10, 9, p, None) == -4
    assert lib.arcs_argmax(ctypes.c_void_p(base + 1), 0, 4, 10, 10, p, None) == -8
    assert lib.arcs_argmax(ctypes.c_void_p(base + 2), 1, 4, 10, 10, p, None) == -8
    # sample
    S = lib.arcs_sample
    assert S(p, 0, 4, 10, 10, None, None, None, 0, 0, p, None, None, 0, None) == -1
    assert S(p, 0, 4, 10, 10, p, p, None, 0, 0, p, None, None, 0, None) == -9
    assert S(p, 0, 4, 10, 10, p, None, p, 0, 0, p, None, None, 0, None) == -9
    assert S(p, 0, 4, 10, 5, p, None, None, 0, 0, p, None, None, 0, None) == -4
    assert S(p, 3, 4, 10, 10, p, None, None, 0, 0, p, None, None, 0, None) == -5
    # small bf16 batches need the split workspace: B * clamp(512 / B, 8, 128) * 16 bytes
    W = lib.arcs_sample_workspace_bytes
    for B in (1, 3, 4, 17, 64):
        assert W(B, 129_280, 0) == B * min(128, max(8, -(-512 // B))) * 16
    assert W(65, 129_280, 0) == 0 and W(4, 129_280, 1) == 0 and W(4, 8184, 0) == 0
    assert W(4, 131_080, 0) == 0 and W(4, 20_004, 0) == 0 and W(4, 8192, 0) == 4 * 128 * 16
    # the long-history workspace: one binary32 copy of a row per row, saturating
    L = lib.arcs_long_history_workspace_bytes
    assert L(4, 129_280) == 4 * 129_280 * 4 and L(1, 1) == 4 and L(0, 10) == 0 and L(3, 0) == 0
    assert L(2**31 - 1, 2**31 - 1) == (2**31 - 1) ** 2 * 4 and L(2**62, 2**31 - 1) == 2**64 - 1
    need = W(4, 129_280, 0)
    V = 129_280
    assert S(p, 0, 4, V, V, p, None, None, 0, 0, p, None, None, 0, None) == -6
    assert S(p, 0, 4, V, V, p, None, None, 0, 0, p, None, p, need - 1, None) == -6
    assert S(p, 0, 4, V, V, p, None, None, 0, 0, p, None, None, need, None) == -1
    assert S(p, 0, 4, V, V, p, None, None, 0, 0, p, None, ctypes.c_void_p(base + 8), need, None) == -8
    # the no-allocation variant checks its arguments first too
    N = lib.arcs_sample_noalloc
    assert N(None, 0, 4, 10, 10, p, None, None, 0, 0, p, None, None) == -1
    assert N(p, 0, 4, 10, 10, p, None, None, 0, 0, None, None, None) == -1
    assert N(p, 5, 4, 10, 10, p, None, None, 0, 0, p, None, None) == -5
    assert N(p, 0, 0, 10, 10, p, None, None, 0, 0, p, None, None) == -2
    assert N(p, 0, 4, 10, 9, p, None, None, 0, 0, p, None, None) == -4
    assert N(p, 0, 4, 10, 10, None, None, None, 0, 0, p, None, None) == -1
    assert N(p, 0, 4, 10, 10, p, p, None, 0, 0, p, None, None) == -9
    # DRY: breakers bounded and present when counted, records aligned
    D = lib.arcs_sample_dry
    assert D(p, 0, 4, 10, 10, p, None, None, p, None, 1, 0, 0, p, None, None, 0, None) == -14
    assert D(p, 0, 4, 10, 10, p, None, None, p, p, 65, 0, 0, p, None, None, 0, None) == -14
    assert D(p, 0, 4, 10, 10, p, None, None, p, p, -1, 0, 0, p, None, None, 0, None) == -14
    assert D(p, 0, 4, 10, 10, p, None, None, ctypes.c_void_p(base + 2), None, 0, 0, 0, p, None, None, 0, None) == -8
    assert D(None, 0, 4, 10, 10, p, None, None, p, None, 0, 0, 0, p, None, None, 0, None) == -1
    # the baseline hybrid nucleus sampler: bf16 only, V % 8 == 0 and <= 131072,
    # aligned rows, both parameter arrays, a budget in [0, 4096]
    H = lib.arcs_sample_hybrid_nucleus
    assert H(p, 0, 4, 64, 64, None, p, 32, 0, 0, p, None, None, None) == -1
    assert H(p, 1, 4, 64, 64, p, p, 32, 0, 0, p, None, None, None) == -5
    assert H(p, 0, 4, 60, 60, p, p, 32, 0, 0, p, None, None, None) == -3
    assert H(p, 0, 4, 131080, 131080, p, p, 32, 0, 0, p, None, None, None) == -3
    assert H(ctypes.c_void_p(base + 2), 0, 4, 64, 64, p, p, 32, 0, 0, p, None, None, None) == -8
    assert H(p, 0, 4, 64, 64, p, p, -1, 0, 0, p, None, None, None) == -13
    assert H(p, 0, 4, 64, 64, p, p, 4097, 0, 0, p, None, None, None) == -13
    # sample with a device key: the key is checked before anything else runs
    K = lib.arcs_sample_keyed
    assert K(p, 0, 4, 10, 10, p, None, None, None, 1, p, None, None, 0, None) == -1
    assert K(p, 0, 4, 10, 10, p, None, None, ctypes.c_void_p(base + 4), 1, p, None, None, 0, None) == -8
    assert K(p, 0, 4, 10, 10, None, None, None, p, 1, p, None, None, 0, None) == -1
    assert K(p, 0, 4, 10, 9, p, None, None, p, 0, p, None, None, 0, None) == -4
    # top logprobs: n in [1, 64], V <= 262144, both outputs required
    L = lib.arcs_top_logprobs
    assert L(p, 0, 4, 10, 10, None, 5, p, None, None, None) == -1
    assert L(p, 0, 4, 10, 10, None, 5, None, p, None, None) == -1
    assert L(p, 0, 4, 10, 10, None, 0, p, p, None, None) == -10
    assert L(p, 0, 4, 10, 10, None, 65, p, p, None, None) == -10
    assert L(p, 0, 4, 262145, 262145, None, 5, p, p, None, None) == -3
    assert L(p, 0, 4, 10, 10, ctypes.c_void_p(base + 2), 5, p, p, None, None) == -8
    assert L(p, 0, 4, 10, 9, None, 5, p, p, None, None) == -4
    assert L(p, 2, 4, 10, 10, None, 5, p, p, None, None) == -5
    # token commit: every word but next_input required, capacity >= 1, alignment
    C = lib.arcs_commit_tokens
    assert C(None, 4, 10, None, p, p, 2, p, p, p, None) == -1
    assert C(p, 4, 10, None, p, p, 2, p, None, p, None) == -1
    assert C(p, 4, 10, None, p, p, 2, p, p, None, None) == -1
    assert C(p, 0, 10, None, p, p, 2, p, p, p, None) == -2
    assert C(p, 4, 0, None, p, p, 2, p, p, p, None) == -3
    assert C(p, 4, 10, None, p, p, 0, p, p, p, None) == -11
    assert C(p, 4, 10, None, ctypes.c_void_p(base + 4), p, 2, p, p, p, None) == -8
    assert C(ctypes.c_void_p(base + 2), 4, 10, None, p, p, 2, p, p, p, None) == -8


def test_binding_constants_match_the_header():
    """The limits the Python binding exports are the header's #defines."""
    import re
    import decode_step_token_row_amd as arcs
    src = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "arcs.h")).read()
    defs = {k: int(v) for k, v in re.findall(r"#define (ARCS_[A-Z_]+) (\d+)", src)}
    assert defs["ARCS_MAX_HISTORY"] == arcs.MAX_HISTORY
    assert defs["ARCS_MAX_PENALTY_VOCAB"] == arcs.MAX_PENALTY_VOCAB
    assert defs["ARCS_TOP_LOGPROBS_MAX_VOCAB"] == arcs.TOP_LOGPROBS_MAX_VOCAB
