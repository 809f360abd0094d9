"""GPU parity of the split-row path: batches of at most 64 bf16 rows with
8192 <= V <= 131072 (V % 8 == 0), whose greedy rows and rows without filters
are read by many workgroups per row (slice partials in the workspace, then
the row's own workgroup draws).  The debug entry point never splits, so
these tests go through arcs_sample / arcs_sample_keyed and compare ids."""

import math

import numpy as np
import pytest

from _util import ensure_built, to_device_logits
from oracle import sampler as oracle
from workloads import f32_to_bf16_bits, make_params, make_workload

pytestmark = pytest.mark.gpu

MARGIN_ID = 1e-5
MARGIN_P = 1e-7
MARGIN_M = 1e-6


@pytest.fixture(scope="module")
def arcs():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return ensure_built()


def _check_ids(got, refs, where):
    excused = 0
    for b, r in enumerate(refs):
        if got[b] != r.id:
            assert r.status == 0 and not r.greedy, (where, b, int(got[b]), r.id)
            assert r.margin_id < MARGIN_ID or r.margin_p < MARGIN_P or r.margin_m < MARGIN_M, (where, b)
            excused += 1
    assert excused <= max(1, len(refs) // 10000), (where, excused)


def _mixed_rows(B, V, seed):
    """Rows of every kind the split path sees: greedy, temperature only
    (several temperatures), filtered rows (left to the whole-row path), and
    special rows: NaN, +inf, all -inf, -inf mixed in, a maximum tied across
    slices, values large enough to leave the double weights' range."""
    rng = np.random.default_rng(seed)
    z = rng.normal(0.0, 2.5, (B, V)).astype(np.float32)
    p = make_params(B, temperature=1.0)
    for b in range(B):
        kind = b % 12
        if kind == 0:
            p[b]["temperature"] = 0.0
        elif kind == 1:
            p[b]["temperature"] = float(rng.uniform(0.2, 2.0))
        elif kind == 2:
            p[b]["top_k"] = 1
        elif kind == 3:
            p[b]["top_p"] = 0.9
        elif kind == 4:
            p[b]["min_p"] = 0.05
            p[b]["top_k"] = 40
        elif kind == 5:
            z[b, rng.integers(0, V, 5)] = np.nan
            p[b]["temperature"] = 0.0 if b % 24 == 5 else 0.8
        elif kind == 6:
            z[b, rng.integers(0, V)] = np.inf
        elif kind == 7:
            z[b] = -np.inf
            p[b]["temperature"] = 0.0 if b % 24 == 7 else 1.0
        elif kind == 8:
            z[b, rng.random(V) < 0.5] = -np.inf
            p[b]["temperature"] = 0.7
        elif kind == 9:
            # the maximum tied in several slices: the lowest index wins
            mx = float(z[b].max()) + 1.0
            z[b, [V - 9, V // 2 + 3, 17, V // 3]] = mx
            p[b]["temperature"] = 0.0
        elif kind == 10:
            # z c far beyond the double range at a tiny temperature: the row
            # leaves the split path
            p[b]["temperature"] = 1e-3
        else:
            z[b] = z[b] * 40.0  # wide logits, T = 1
    return z, p


@pytest.mark.parametrize("B,V", [(1, 129_280), (3, 8192), (12, 131_072), (24, 20_000), (64, 129_280),
                                 (17, 50_008)])
def test_split_batches_against_the_oracle(arcs, B, V):
    import torch
    z, p = _mixed_rows(B, V, B * 1000 + V)
    bits = f32_to_bf16_bits(z)
    logits = to_device_logits(bits, "bf16")
    params = arcs.params_to_device(p)
    ws = torch.empty(arcs.workspace_bytes(B, V, arcs.DTYPE_BF16), dtype=torch.uint8, device="cuda")
    assert ws.numel() > 0
    for step in (0, 7):
        status = torch.empty(B, dtype=torch.int32, device="cuda")
        got = arcs.sample(logits, params, seed=11, step=step, out_status=status, workspace=ws).cpu().numpy()
        refs = oracle.sample(bits, "bf16", p, None, None, 11, step, band_p=MARGIN_P, band_m=MARGIN_M)
        _check_ids(got, refs, f"B={B} V={V} step={step}")
        assert status.cpu().tolist() == [r.status for r in refs]
        # the whole-row path (the debug entry point never splits) agrees
        dbg = arcs.sample_debug(logits, params, seed=11, step=step)[0].cpu().numpy()
        assert np.array_equal(got, dbg), (np.nonzero(got != dbg)[0], got[got != dbg], dbg[got != dbg])


def test_split_normal_b4_mismatch_rate(arcs):
    """The 4-row workload (temperature only): 25,600 steps of 4 rows, each
    row filtered once by the oracle and redrawn per step."""
    import torch
    w = make_workload("normal_b4_bf16")
    logits = to_device_logits(w.logits, "bf16")
    params = arcs.params_to_device(w.params)
    ws = torch.empty(arcs.workspace_bytes(w.B, w.V, arcs.DTYPE_BF16), dtype=torch.uint8, device="cuda")
    steps = 25_600
    got = torch.empty((steps, w.B), dtype=torch.int32, device="cuda")
    for s in range(steps):
        arcs.sample(logits, params, seed=w.seed, step=s, out=got[s], workspace=ws)
    got = got.cpu().numpy()
    mismatches = near = 0
    for b in range(w.B):
        r = oracle.sample_row(w.logits[b], "bf16", w.params[b], None, w.seed, b, 0, want_probs=True)
        us = np.array([oracle.uniform(w.seed, b, s) for s in range(steps)])
        want, margins = oracle.draw(r.kept, r.weights[r.kept], us)
        bad = got[:, b] != want
        near += int(np.count_nonzero(margins < MARGIN_ID))
        assert np.all(margins[bad] < MARGIN_ID), (b, np.nonzero(bad)[0][:5])
        mismatches += int(bad.sum())
    total = steps * w.B
    print(f"normal_b4 split: draws={total} mismatches={mismatches} near-boundary={near}")
    assert mismatches <= max(1, int(1e-4 * total)), (mismatches, total)


def test_split_keyed_graph_replays(arcs):
    """The split launch (slice kernel, row kernel, key advance) captured once:
    each replay samples the next step, with eager work between replays."""
    import torch
    B, V, s0, seed = 4, 129_280, 3, 99
    w = make_workload("normal_b4_bf16")
    logits = to_device_logits(w.logits, "bf16")
    params = arcs.params_to_device(w.params)
    ws = torch.empty(arcs.workspace_bytes(B, V, arcs.DTYPE_BF16), dtype=torch.uint8, device="cuda")
    want = [arcs.sample(logits, params, seed=seed, step=s0 + i, workspace=ws).cpu().numpy() for i in range(6)]
    key = arcs.make_key(seed, s0)
    out = torch.empty(B, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        arcs.sample_keyed(logits, params, key, advance=False, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        arcs.sample_keyed(logits, params, key, out=out, workspace=ws)
    for i in range(6):
        out.fill_(-5)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), want[i]), i
        refs = oracle.sample(w.logits, "bf16", w.params, None, None, seed, s0 + i)
        _check_ids(out.cpu().numpy(), refs, f"replay {i}")
        arcs.sample(logits, params, seed=5, step=i, workspace=ws)  # eager work in between
        torch.cuda.synchronize()


def test_split_with_a_caller_workspace(arcs):
    import ctypes
    import torch
    B, V = 4, 129_280
    logits = torch.zeros((B, V), dtype=torch.bfloat16, device="cuda")
    params = arcs.params_to_device(make_params(B, temperature=1.0))
    out = torch.empty(B, dtype=torch.int32, device="cuda")
    lib = arcs.library()
    need = arcs.workspace_bytes(B, V, arcs.DTYPE_BF16)
    ws = torch.empty(need + 16, dtype=torch.uint8, device="cuda")
    call = lambda ptr, nbytes: lib.arcs_sample(ctypes.c_void_p(logits.data_ptr()), arcs.DTYPE_BF16, B, V, V,
                                               ctypes.c_void_p(params.data_ptr()), None, None, 1, 0,
                                               ctypes.c_void_p(out.data_ptr()), None, ptr, nbytes, None)
    assert call(None, 0) == arcs.ERR_WORKSPACE_TOO_SMALL
    assert call(ctypes.c_void_p(ws.data_ptr() + 8), need) == arcs.ERR_MISALIGNED
    assert call(ctypes.c_void_p(ws.data_ptr()), need) == arcs.OK
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    # equal logits, no filter: the id is floor(u * V)
    want = [math.floor(oracle.uniform(1, b, 0) * V) for b in range(B)]
    assert got.tolist() == want
