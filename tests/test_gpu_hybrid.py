"""GPU parity of arcs_sample_hybrid_nucleus, the baseline enumeration /
bisection nucleus sampler, against the oracle's hybrid_nucleus_row: the kept
set size (exact unless the top-p crossing lies within its margin) and the ids
(exact unless the uniform lies within its margin of a boundary)."""

import numpy as np
import pytest

from _util import ensure_built, to_device_logits
from oracle import sampler as oracle
from workloads import f32_to_bf16_bits, make_workload

pytestmark = pytest.mark.gpu

MARGIN_ID = 1e-5
MARGIN_P = 1e-6  # fp32 weights in the baseline: relative errors of a few 1e-7


@pytest.fixture(scope="module")
def arcs():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return ensure_built()


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _support_rows(B, V, widths, rng):
    """Rows whose mass sits on `width` tokens (zipf-like values at random ids,
    coarsely rounded so that ties occur), the rest far below."""
    z = np.full((B, V), -60.0, dtype=np.float32)
    for b in range(B):
        w = int(widths[b % len(widths)])
        ids = rng.choice(V, size=w, replace=False)
        z[b, ids] = np.round(-0.6 * np.log1p(np.arange(w)) * 4.0) / 4.0 + rng.normal(0, 0.01, w) * (b % 2)
    return z


def _run(arcs, bits, T, P, budget, seed, step):
    import torch
    B = bits.shape[0]
    logits = to_device_logits(bits, "bf16")
    kept = torch.empty(B, dtype=torch.int32, device="cuda")
    status = torch.empty(B, dtype=torch.int32, device="cuda")
    ids = arcs.sample_hybrid_nucleus(logits, _dev(T.astype(np.float32)), _dev(P.astype(np.float32)), budget,
                                     seed=seed, step=step, out_kept=kept, out_status=status)
    return ids.cpu().numpy(), kept.cpu().numpy(), status.cpu().numpy()


def _compare(bits, T, P, budget, seed, step, ids, kept, status, where):
    excused = 0
    for b in range(bits.shape[0]):
        r = oracle.hybrid_nucleus_row(bits[b], "bf16", T[b], P[b], budget, seed, b, step, band_p=MARGIN_P)
        assert status[b] == r.status, (where, b)
        if r.status != 0:
            assert ids[b] == -1
            continue
        near = r.margin_p < MARGIN_P
        assert kept[b] == r.L or near, (where, b, int(kept[b]), r.L, r.margin_p)
        if ids[b] != r.id:
            assert near or r.margin_id < MARGIN_ID, (where, b, int(ids[b]), r.id, r.margin_id)
            excused += 1
    assert excused <= 1, (where, excused)


@pytest.mark.parametrize("budget", [0, 8, 32, 4096])
def test_hybrid_support_widths(arcs, budget):
    rng = np.random.default_rng(budget + 1)
    B, V = 48, 20_000
    z = _support_rows(B, V, [1, 2, 8, 30, 64, 200, 512, 4096], rng)
    bits = f32_to_bf16_bits(z)
    T = rng.uniform(0.6, 1.4, B)
    P = rng.uniform(0.3, 0.97, B)
    P[::7] = 1.0  # every id kept
    for step in (0, 5):
        ids, kept, status = _run(arcs, bits, T, P, budget, 21, step)
        _compare(bits, T, P, budget, 21, step, ids, kept, status, f"budget={budget} step={step}")


def test_hybrid_full_size_zipf_rows(arcs):
    """The filtered zipf rows at V = 129,280 (bf16: many tied values), top_p
    0.9 and 0.5 at T 0.7: a budget of 32 forces the bisection (and the wide
    rule) on the rows whose nucleus is longer."""
    w = make_workload("zipf_b256_bf16_t0.7_k50_p0.9_minp0.05", B=32)
    T = np.full(32, 0.7)
    P = np.where(np.arange(32) % 2 == 0, 0.9, 0.5)
    ids, kept, status = _run(arcs, w.logits, T, P, 32, 4, 9)
    _compare(w.logits, T, P, 32, 4, 9, ids, kept, status, "zipf 129280")
    assert (kept > 32).any() and (kept <= 32).any()


def test_hybrid_bad_rows(arcs):
    B, V = 6, 1024
    bits = f32_to_bf16_bits(np.zeros((B, V), dtype=np.float32))
    T = np.array([1.0, 0.0, -1.0, np.inf, 1.0, 1.0])
    P = np.array([0.5, 0.5, 0.5, 0.5, 0.0, np.nan])
    ids, kept, status = _run(arcs, bits, T, P, 8, 0, 0)
    assert status.tolist() == [0, 1, 1, 1, 2, 2]
    assert (ids[1:] == -1).all() and 0 <= ids[0] < V
    _compare(bits, T, P, 8, 0, 0, ids, kept, status, "bad rows")
