"""GPU parity of arcs_top_logprobs against the fp64 oracle.

Ids: exact (the order value desc, id asc is total).  Logprobs: within
5e-6 + 2^-23 |lp|.  The kernel takes each weight as exp2 of a float32
argument (relative error about (1 + |arg|) 2^-23, on weights that carry the
mass well under 1e-6), sums groups of at most 8 weights in float32 and the
rest in binary64, and rescales a thread's sum by a float32 factor each time
its maximum grows; ln S is then within about 2e-6 of the oracle's, the
difference (z - m) / T is taken in binary64, and the result is rounded to
binary32 (2^-24 |lp|).
"""

import math

import numpy as np
import pytest

from _util import ensure_built, to_device_logits
from oracle import sampler as oracle
from workloads import f32_to_bf16_bits, make_workload

pytestmark = pytest.mark.gpu

ATOL = 5e-6
RTOL = 2.0 ** -23


@pytest.fixture(scope="module")
def arcs():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return ensure_built()


def _run(arcs, raw, dtype, temps, n, stride=None):
    import torch
    x = to_device_logits(raw, dtype, stride=stride)
    t = None if temps is None else torch.from_numpy(np.asarray(temps, np.float32)).cuda()
    st = torch.full((raw.shape[0],), -99, dtype=torch.int32, device="cuda")
    ids, lps = arcs.top_logprobs(x, n, temperature=t, out_status=st)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), lps.cpu().numpy(), st.cpu().numpy()


def _check(ids, lps, st, raw, dtype, temps, n, rows=None, where=""):
    rows = range(raw.shape[0]) if rows is None else rows
    for b in rows:
        T = 1.0 if temps is None else float(np.float32(temps[b]))
        r = oracle.top_logprobs_row(raw[b], dtype, T, n)
        assert st[b] == r.status, (where, b, st[b], r.status)
        assert ids[b].tolist() == r.ids.tolist(), (where, b, ids[b][:8], r.ids[:8])
        if r.status != 0:
            assert np.isnan(lps[b]).all(), (where, b)
            continue
        fin = np.isfinite(r.logprobs)
        assert (np.isneginf(lps[b]) == np.isneginf(r.logprobs)).all(), (where, b)
        err = np.abs(lps[b][fin].astype(np.float64) - r.logprobs[fin])
        tol = ATOL + RTOL * np.abs(r.logprobs[fin])
        assert (err <= tol).all(), (where, b, float(err.max()), r.logprobs[fin][np.argmax(err - tol)])


def _rows(V, B, seed):
    """Zipf-shaped rows plus normal, tied, peaked and flat ones."""
    w = make_workload("zipf_b256_bf16_greedy", B=B, V=V)
    rng = np.random.default_rng(seed)
    z = np.empty((B, V), np.float32)
    for b in range(B):
        kind = b % 5
        if kind == 0:
            z[b] = (w.logits[b].astype(np.uint32) << 16).view(np.float32)
        elif kind == 1:
            z[b] = rng.normal(0, 3, V)
        elif kind == 2:
            z[b] = np.round(rng.normal(0, 2, V) * 2) / 2
        elif kind == 3:
            z[b] = rng.normal(0, 1, V)
            z[b, rng.integers(0, V)] += 25.0
        else:
            z[b] = rng.uniform(-0.01, 0.01, V)
    return z


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [1000, 1003, 4096, 50_000, 129_280])
def test_top_logprobs_parity(arcs, dtype, V):
    B = 10
    z = _rows(V, B, seed=V)
    raw = f32_to_bf16_bits(z) if dtype == "bf16" else z
    temps = np.random.default_rng(V + 1).uniform(0.2, 2.0, B)
    for n in (1, 7, 64):
        ids, lps, st = _run(arcs, raw, dtype, temps, n)
        _check(ids, lps, st, raw, dtype, temps, n, where=(dtype, V, n))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_top_logprobs_unaligned_rows(arcs, dtype):
    # a row stride that breaks 16-byte alignment takes the element path
    B, V, n = 6, 5000, 20
    z = _rows(V, B, seed=7)
    raw = f32_to_bf16_bits(z) if dtype == "bf16" else z
    ids, lps, st = _run(arcs, raw, dtype, None, n, stride=V + 3)
    _check(ids, lps, st, raw, dtype, None, n, where=(dtype, "stride"))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_top_logprobs_special_rows(arcs, dtype):
    V, n = 2048, 16
    rng = np.random.default_rng(2)
    z = rng.normal(0, 2, (7, V)).astype(np.float32)
    z[0, [5, 900, 1700]] = np.nan                 # NaN counts as -inf
    z[1, [3, 1000]] = np.inf                      # +inf ids share the mass
    z[2, :] = -np.inf                             # uniform over the row
    z[3, ::2] = -0.0                              # -0 == +0, ties by id
    z[3, 1::2] = 0.0
    z[4, :] = 1.5                                 # all equal
    z[5, 100:] = -np.inf                          # fewer finite values than n
    z[5, :100] = np.nan
    z[6, 7] = np.inf
    z[6, 9] = -np.inf
    raw = f32_to_bf16_bits(z) if dtype == "bf16" else z
    temps = np.array([1.0, 0.5, 1.0, 2.0, 0.7, 1.0, 1.0])
    ids, lps, st = _run(arcs, raw, dtype, temps, n)
    _check(ids, lps, st, raw, dtype, temps, n, where=(dtype, "special"))


def test_top_logprobs_short_rows_and_bad_temperatures(arcs):
    # V < n: trailing ids -1 / -inf; a bad temperature gives -1 / NaN and a status
    z = np.random.default_rng(4).normal(0, 1, (5, 10)).astype(np.float32)
    temps = np.array([1.0, 0.0, -2.0, np.nan, np.inf], np.float32)
    ids, lps, st = _run(arcs, z, "f32", temps, 20)
    _check(ids, lps, st, z, "f32", temps, 20, where="short")
    assert st.tolist() == [0, 1, 1, 1, 1]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("aligned", [True, False])
@pytest.mark.parametrize("V", [131_072, 262_144])
def test_top_logprobs_many_candidates(arcs, dtype, aligned, V):
    # 64 threads own nothing but large values, one of them only its smallest:
    # every element of the other 63 is at or above the 64th thread maximum,
    # so about 63 * V / 1024 elements are gathered (the rank-count path; at
    # the largest V that is almost the whole candidate area)
    n = 64
    E = (8 if dtype == "bf16" else 4) if aligned else 1
    rng = np.random.default_rng(9)
    z = rng.normal(0, 1, (2, V)).astype(np.float32)
    owner = (np.arange(V) // E) % 1024
    heavy = owner < 64
    z[:, heavy] = 10.5 + rng.uniform(0, 0.4, (2, int(heavy.sum())))
    z[:, owner == 63] = 10.0
    raw = f32_to_bf16_bits(z) if dtype == "bf16" else z
    ids, lps, st = _run(arcs, raw, dtype, [1.0, 0.3], n, stride=None if aligned else V + 1)
    _check(ids, lps, st, raw, dtype, [1.0, 0.3], n, where=(dtype, aligned))


@pytest.mark.parametrize("dtype,V,aligned", [("bf16", 262_144, True), ("bf16", 200_003, False),
                                              ("f32", 262_140, True), ("f32", 151_936, False)])
def test_top_logprobs_vocabularies_beyond_131072(arcs, dtype, V, aligned):
    # up to ARCS_TOP_LOGPROBS_MAX_VOCAB: each thread then owns up to 256
    # elements; the row kinds of _rows, every id checked against the oracle
    B, n = 5, 33
    z = _rows(V, B, seed=V % 1000)
    raw = f32_to_bf16_bits(z) if dtype == "bf16" else z
    temps = [0.7, 1.0, 1.3, 0.25, 2.0]
    ids, lps, st = _run(arcs, raw, dtype, temps, n, stride=None if aligned else V + 3)
    _check(ids, lps, st, raw, dtype, temps, n, where=(dtype, V))


def test_top_logprobs_vocabulary_bound(arcs):
    import torch
    x = torch.zeros((1, arcs.TOP_LOGPROBS_MAX_VOCAB + 8), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(Exception):
        arcs.top_logprobs(x, 4)


def test_top_logprobs_full_size_sampled_rows(arcs):
    # the measured configuration: B = 256, V = 129,280 bf16 Zipf rows, T = 0.7, n = 20
    w = make_workload("zipf_b256_bf16_top_logprobs20")
    temps = w.params["temperature"]
    ids, lps, st = _run(arcs, w.logits, "bf16", temps, w.top_n)
    assert (st == 0).all()
    # properties at every row: valid distinct ids, non-increasing logprobs, mass <= 1
    assert ((ids >= 0) & (ids < w.V)).all()
    assert all(len(set(r.tolist())) == w.top_n for r in ids)
    assert (np.diff(lps, axis=1) <= 0).all()
    assert (np.exp(lps.astype(np.float64)).sum(axis=1) <= 1.0 + 1e-5).all()
    rows = sorted(set(np.random.default_rng(0).choice(w.B, 12, replace=False).tolist()) | {0, w.B - 1})
    _check(ids, lps, st, w.logits, "bf16", temps, w.top_n, rows=rows, where="full")


def test_top_logprobs_graph_replays_match_eager(arcs):
    # captured once, replayed over logits rewritten in place between replays
    import torch
    B, V, n = 16, 20_000, 12
    rows = [_rows(V, B, seed=s) for s in (21, 22, 23)]
    x = to_device_logits(f32_to_bf16_bits(rows[0]), "bf16")
    temps = torch.from_numpy(np.linspace(0.3, 1.7, B).astype(np.float32)).cuda()
    ids = torch.empty((B, n), dtype=torch.int32, device="cuda")
    lps = torch.empty((B, n), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        arcs.top_logprobs(x, n, temperature=temps, out_ids=ids, out_logprobs=lps)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        arcs.top_logprobs(x, n, temperature=temps, out_ids=ids, out_logprobs=lps)
    for r in range(6):
        z = rows[r % 3]
        x.copy_(to_device_logits(f32_to_bf16_bits(z), "bf16"))
        g.replay()
        torch.cuda.synchronize()
        want_ids, want_lps = arcs.top_logprobs(x, n, temperature=temps)
        torch.cuda.synchronize()
        assert torch.equal(ids, want_ids), r
        assert torch.equal(lps, want_lps), r
        if r == 0:
            raw = f32_to_bf16_bits(z)
            _check(ids.cpu().numpy(), lps.cpu().numpy(), np.zeros(B, np.int32), raw, "bf16",
                   temps.cpu().numpy(), n, rows=[0, 7, 15], where="graph")
