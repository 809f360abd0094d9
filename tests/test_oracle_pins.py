"""Pins for the fp64 CPU oracle: it is checked against facts that do not come
from itself -- published generator outputs, a library's float32 arithmetic,
a library's bf16 widening and softmax, brute-force enumeration on tiny
vocabularies, closed forms and the invariants the method must satisfy.

Each mistake a plausible oracle bug would make (a dropped penalty term, a
wrong tie-break, >= instead of > in the draw, renormalising between filters,
measuring top-p against the kept mass instead of the full mass) fails at
least one test here; ``test_planted_mistakes_are_caught`` plants some of
them in the oracle and checks that a pin goes red.
"""

import itertools
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

from oracle import sampler as o
from workloads import bf16_bits_to_f32, f32_to_bf16_bits, make_params

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _p(**kw):
    return make_params(1, **kw)[0]


def _f32_row(vals):
    return np.asarray(vals, dtype=np.float32)


# --------------------------------------------------------------------------
# SplitMix64
# --------------------------------------------------------------------------
def test_splitmix64_published_outputs():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "splitmix64_seed0.txt")) if l.strip() and not l.startswith("#")]
    assert len(rows) == 10
    for k, hexval in rows:
        assert o.splitmix64_output(0, int(k)) == int(hexval, 16)


def test_counter_keying_and_uniform():
    # (seed, row, step) -> output number n + 1, n = step * 2**32 + row
    assert o.uniform_bits(0, 0, 0) == o.splitmix64_output(0, 1)
    assert o.uniform_bits(0, 1, 0) == o.splitmix64_output(0, 2)
    assert o.uniform_bits(0, 5, 1) == o.splitmix64_output(0, (1 << 32) + 6)
    # seed shifts the whole stream: state seed + k*gamma
    assert o.uniform_bits(o.SPLITMIX_GAMMA, 0, 0) == o.splitmix64_output(0, 2)
    u = o.uniform(0, 0, 0)
    assert u == (0xE220A8397B1DCDAF >> 11) / 2.0 ** 53
    assert 0.0 <= u < 1.0
    # the 53-bit uniform is exact: scaling back gives the integer
    for r in range(50):
        x = o.uniform_bits(7, r, 3)
        assert o.uniform(7, r, 3) * 2.0 ** 53 == float(x >> 11)


def test_uniform_distribution_is_uniform():
    us = np.array([o.uniform(123, r, s) for r in range(100) for s in range(200)])
    assert scipy.stats.kstest(us, "uniform").pvalue > 1e-3


# --------------------------------------------------------------------------
# widening (exhaustive over all bf16 patterns)
# --------------------------------------------------------------------------
def test_widen_bf16_exhaustive_against_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = o.widen(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    visited = 0
    for i in range(65536):
        r = ref[i]
        if np.isnan(r):
            assert ours[i] == -np.inf
        elif r == 0:
            assert ours[i] == 0 and not np.signbit(ours[i])
        else:
            assert ours[i] == r
        visited += 1
    assert visited == 65536
    # ordering of the widened values matches float ordering of torch's values
    finite = ~np.isnan(ref)
    assert np.array_equal(np.argsort(ours[finite], kind="stable"), np.argsort(np.where(ref[finite] == 0, 0, ref[finite]), kind="stable"))


def test_widen_f32_rules():
    z = o.widen(_f32_row([np.nan, -0.0, 0.0, -np.inf, np.inf, 1.5]), "f32")
    assert z[0] == -np.inf and z[3] == -np.inf and z[4] == np.inf and z[5] == np.float32(1.5)
    assert not np.signbit(z[1]) and not np.signbit(z[2])


def test_bf16_rounding_generator_roundtrip():
    x = np.random.default_rng(0).normal(0, 5, 10000).astype(np.float32)
    b = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(bf16_bits_to_f32(b), ref)


# --------------------------------------------------------------------------
# penalties: binary32 emulation against numpy's float32 arithmetic
# --------------------------------------------------------------------------
def _np_penalty(z, c, pres, freq, rep):
    z = np.float32(z)
    if not (rep == 1.0 or rep == 0.0):
        z = z / np.float32(rep) if z > 0 else z * np.float32(rep)
    if freq != 0.0:
        z = z - np.float32(freq) * np.float32(c)
    if pres != 0.0:
        z = z - np.float32(pres)
    return np.float32(z)


def test_penalty_matches_numpy_float32():
    rng = np.random.default_rng(1)
    for _ in range(20000):
        z = float(np.float32(rng.normal(0, 8)))
        c = int(rng.integers(1, 3000))
        pres = float(np.float32(rng.choice([0.0, rng.uniform(-2, 2)])))
        freq = float(np.float32(rng.choice([0.0, rng.uniform(-2, 2)])))
        rep = float(np.float32(rng.choice([1.0, 0.0, rng.uniform(0.1, 3)])))
        ours = np.float32(o.penalize_one(z, c, pres, freq, rep))
        ref = _np_penalty(z, c, pres, freq, rep)
        assert ours.view(np.uint32) == ref.view(np.uint32) or (ours == 0 and ref == 0), (z, c, pres, freq, rep)


def test_penalty_hand_cases():
    # repetition divides positive logits and multiplies the rest
    assert o.penalize_one(2.2, 1, 0.0, 0.0, 1.1) == float(np.float32(2.2) / np.float32(1.1))
    assert o.penalize_one(-2.0, 1, 0.0, 0.0, 2.0) == -4.0
    assert o.penalize_one(0.0, 1, 0.0, 0.0, 2.0) == 0.0
    # frequency scales with the count, presence does not
    assert o.penalize_one(1.0, 3, 0.0, 0.5, 1.0) == -0.5
    assert o.penalize_one(1.0, 3, 0.25, 0.0, 1.0) == 0.75
    # order: repetition, then frequency, then presence
    assert o.penalize_one(3.0, 2, 1.0, 0.5, 2.0) == 3.0 / 2.0 - 1.0 - 1.0


def test_penalty_off_values_leave_logits_bit_identical():
    rng = np.random.default_rng(2)
    z = rng.normal(0, 4, 512).astype(np.float32)
    hist = rng.integers(-5, 600, 300).astype(np.int32)
    for pres, freq, rep in [(0.0, 0.0, 1.0), (0.0, 0.0, 0.0)]:
        out = o.penalize(z, hist, pres, freq, rep)
        assert np.array_equal(out.view(np.uint32), z.view(np.uint32))
    # a multiplier-0 penalty is a no-op; a non-zero one is not
    assert not np.array_equal(o.penalize(z, hist, 0.5, 0.0, 1.0), z)


def test_penalty_counts_duplicates_and_skips_out_of_range():
    z = np.zeros(8, dtype=np.float32) + 1.0
    hist = np.array([3, 3, 3, 5, -1, 8, 100], dtype=np.int32)
    out = o.penalize(z, hist, 0.0, 0.25, 1.0)
    assert out[3] == 1.0 - 0.75 and out[5] == 0.75
    assert np.all(out[[0, 1, 2, 4, 6, 7]] == 1.0)


# --------------------------------------------------------------------------
# argmax
# --------------------------------------------------------------------------
def _bf_argmax(z):
    best = 0
    for i in range(len(z)):
        if z[i] > z[best]:
            best = i
    return best


def test_argmax_bruteforce_with_ties():
    rng = np.random.default_rng(3)
    for _ in range(500):
        V = int(rng.integers(1, 40))
        raw = rng.integers(-3, 4, V).astype(np.float32)
        z = o.widen(raw, "f32")
        assert o.argmax_first(z) == _bf_argmax(z)


def test_argmax_special_rows():
    assert o.argmax_first(o.widen(_f32_row([1, 1, 1, 1]), "f32")) == 0
    assert o.argmax_first(o.widen(_f32_row([0, 1, 2, 3]), "f32")) == 3
    assert o.argmax_first(o.widen(_f32_row([-1, -0.0, 0.0, -2]), "f32")) == 1   # -0 == +0
    assert o.argmax_first(o.widen(_f32_row([np.nan, -np.inf, np.nan]), "f32")) == 0
    assert o.argmax_first(o.widen(_f32_row([np.nan, 5, np.inf, np.inf]), "f32")) == 2
    r = o.sample_row(_f32_row([-np.inf] * 5), "f32", _p(temperature=1.0), None, 0, 0, 0)
    assert r.id == 0


# --------------------------------------------------------------------------
# kept sets: brute force on tiny vocabularies
# --------------------------------------------------------------------------
def _prec(z, a, b):
    return z[a] > z[b] or (z[a] == z[b] and a < b)


def _prefix_closed(z, S):
    V = len(z)
    return all(_prec(z, a, b) for a in S for b in range(V) if b not in S)


def _bf_topk(z, k):
    sols = [set(C) for C in itertools.combinations(range(len(z)), k) if _prefix_closed(z, set(C))]
    assert len(sols) == 1
    return sols[0]


def _softmax_w(z, T):
    zz = z.astype(np.float64)
    return np.exp((zz - zz.max()) / T)


def _bf_topp(z, w, p):
    V = len(z)
    target = p * math.fsum(w)
    for n in range(1, V + 1):
        ok = [set(C) for C in itertools.combinations(range(V), n) if math.fsum(w[list(C)]) >= target]
        if ok:
            closed = [C for C in ok if _prefix_closed(z, C)]
            assert len(closed) == 1
            return closed[0]
    return set(range(V))


def test_topk_set_bruteforce():
    rng = np.random.default_rng(4)
    for _ in range(200):
        V = int(rng.integers(2, 10))
        z = o.widen(rng.integers(-2, 3, V).astype(np.float32), "f32")
        k = int(rng.integers(2, V + 1))
        r = o.sample_row(z, "f32", _p(temperature=1.0, top_k=k), None, 1, 0, 0)
        want = _bf_topk(z, min(k, V))
        assert set(r.kept.tolist()) == want


def test_topp_set_bruteforce():
    rng = np.random.default_rng(5)
    checked = 0
    for _ in range(300):
        V = int(rng.integers(2, 10))
        z = o.widen((rng.integers(-3, 3, V) + rng.choice([0, 0.5], V)).astype(np.float32), "f32")
        T = float(np.float32(rng.uniform(0.3, 2.0)))
        p = float(np.float32(rng.uniform(0.05, 0.99)))
        r = o.sample_row(z, "f32", _p(temperature=T, top_p=p), None, 1, 0, 0)
        if r.margin_p < 1e-12:
            continue
        want = _bf_topp(z, _softmax_w(z, T), p)
        assert set(r.kept.tolist()) == want
        checked += 1
    assert checked > 250


def _bf_wide(z, strict):
    """The wide rule by its definition: the strict set plus every id whose
    value equals the smallest value in it."""
    vb = min(z[i] for i in strict)
    return set(strict) | {i for i in range(len(z)) if z[i] == vb}


def test_wide_ties_bruteforce():
    rng = np.random.default_rng(14)
    grew = 0
    for _ in range(300):
        V = int(rng.integers(2, 10))
        z = o.widen(rng.integers(-2, 3, V).astype(np.float32), "f32")
        if rng.random() < 0.5:
            k = int(rng.integers(2, V + 1))
            kw = dict(temperature=1.0, top_k=k)
            strict = _bf_topk(z, min(k, V))
        else:
            T = float(np.float32(rng.uniform(0.3, 2.0)))
            pp = float(np.float32(rng.uniform(0.05, 0.99)))
            kw = dict(temperature=T, top_p=pp)
            r0 = o.sample_row(z, "f32", _p(**kw), None, 1, 0, 0)
            if r0.margin_p < 1e-12:
                continue
            strict = _bf_topp(z, _softmax_w(z, T), pp)
        r = o.sample_row(z, "f32", _p(flags=o.ROW_TIES_WIDE, **kw), None, 1, 0, 0)
        want = _bf_wide(z, strict)
        assert r.status == 0 and set(r.kept.tolist()) == want, (z, kw, strict, want)
        grew += len(want) > len(strict)
    assert grew > 50


def test_wide_ties_on_a_tied_diffuse_support():
    """105 tokens of distinct values, then 11 tied at a lower value; top_p set
    so that the crossing falls on the 6th tied token: the strict prefix keeps
    111 tokens, the wide rule 116 (the sizes the pages report for their
    fallback selector on a tied diffuse support)."""
    z = np.full(300, -50.0, dtype=np.float32)
    z[:105] = np.linspace(2.0, 1.0, 105, dtype=np.float32)
    z[105:116] = 0.5
    zz = o.widen(z, "f32")
    _, w = o.weights(zz, 1.0)
    order = o.total_order(zz)
    cum = np.cumsum(w[order])
    p = float(np.float32((cum[109] + 0.5 * w[105]) / cum[-1]))
    strict = o.sample_row(z, "f32", _p(temperature=1.0, top_p=p), None, 1, 0, 0)
    wide = o.sample_row(z, "f32", _p(temperature=1.0, top_p=p, flags=o.ROW_TIES_WIDE), None, 1, 0, 0)
    assert strict.L == 111 and wide.L == 116
    assert set(wide.kept.tolist()) == set(range(116))
    # top-k at the same place: k = 111 keeps 111 strictly, 116 wide
    assert o.sample_row(z, "f32", _p(temperature=1.0, top_k=111, flags=o.ROW_TIES_WIDE), None, 1, 0, 0).L == 116
    assert o.sample_row(z, "f32", _p(temperature=1.0, top_k=111), None, 1, 0, 0).L == 111
    # min-p sets are defined by value: the flag changes nothing
    a = o.sample_row(z, "f32", _p(temperature=1.0, min_p=0.5), None, 1, 0, 0)
    b = o.sample_row(z, "f32", _p(temperature=1.0, min_p=0.5, flags=o.ROW_TIES_WIDE), None, 1, 0, 0)
    assert a.L == b.L


def test_hybrid_nucleus_is_the_strict_prefix_within_budget_else_the_wide_one():
    rng = np.random.default_rng(15)
    for _ in range(100):
        V = int(rng.integers(2, 12))
        z = o.widen(rng.integers(-2, 3, V).astype(np.float32), "f32")
        T = float(np.float32(rng.uniform(0.3, 2.0)))
        pp = float(np.float32(rng.uniform(0.05, 0.99)))
        strict = o.sample_row(z, "f32", _p(temperature=T, top_p=pp), None, 3, 1, 2)
        wide = o.sample_row(z, "f32", _p(temperature=T, top_p=pp, flags=o.ROW_TIES_WIDE), None, 3, 1, 2)
        assert o.hybrid_nucleus_row(z, "f32", T, pp, V, 3, 1, 2).L == strict.L
        assert o.hybrid_nucleus_row(z, "f32", T, pp, strict.L, 3, 1, 2).L == strict.L
        h0 = o.hybrid_nucleus_row(z, "f32", T, pp, strict.L - 1, 3, 1, 2)
        assert h0.L == wide.L and set(h0.kept.tolist()) == set(wide.kept.tolist())
        assert h0.id == wide.id
    # the tied diffuse support: 111 within a budget of 200, 116 past a budget of 32
    z = np.full(300, -50.0, dtype=np.float32)
    z[:105] = np.linspace(2.0, 1.0, 105, dtype=np.float32)
    z[105:116] = 0.5
    zz = o.widen(z, "f32")
    _, w = o.weights(zz, 1.0)
    cum = np.cumsum(w[o.total_order(zz)])
    pp = float(np.float32((cum[109] + 0.5 * w[105]) / cum[-1]))
    assert o.hybrid_nucleus_row(z, "f32", 1.0, pp, 200, 0, 0, 0).L == 111
    assert o.hybrid_nucleus_row(z, "f32", 1.0, pp, 32, 0, 0, 0).L == 116
    assert o.hybrid_nucleus_row(z, "f32", 1.0, 1.0, 0, 0, 0, 0).L == 300
    assert o.hybrid_nucleus_row(z, "f32", 0.0, 0.5, 8, 0, 0, 0).status == o.ROW_BAD_TEMPERATURE
    assert o.hybrid_nucleus_row(z, "f32", 1.0, 0.0, 8, 0, 0, 0).status == o.ROW_BAD_TOP_P


def test_minp_set_against_softmax_definition():
    rng = np.random.default_rng(6)
    for _ in range(200):
        V = int(rng.integers(2, 30))
        z = o.widen(rng.normal(0, 2, V).astype(np.float32), "f32")
        T = float(np.float32(rng.uniform(0.3, 2.0)))
        mp = float(np.float32(rng.uniform(0.01, 0.9)))
        r = o.sample_row(z, "f32", _p(temperature=T, min_p=mp), None, 1, 0, 0)
        q = scipy.special.softmax(z.astype(np.float64) / T)
        want = set(np.nonzero(q >= mp * q.max() * (1 - 1e-15))[0].tolist())
        if r.margin_m < 1e-9:
            continue
        assert set(r.kept.tolist()) == want


def test_combined_filters_take_the_shortest_prefix_without_renormalising():
    # weights 0.4 0.3 0.2 0.1 (as logits).  top_p = 0.75 measured on the FULL
    # mass needs 3 tokens (0.4+0.3 < 0.75); renormalising after the top_k=3
    # cut would compare against 0.75*0.9 = 0.675 and keep only 2.
    w = np.array([0.4, 0.3, 0.2, 0.1])
    z = np.log(w).astype(np.float32)
    r = o.sample_row(z, "f32", _p(temperature=1.0, top_k=3, top_p=0.65), None, 0, 0, 0)
    assert set(r.kept.tolist()) == {0, 1}
    r = o.sample_row(z, "f32", _p(temperature=1.0, top_k=3, top_p=0.75), None, 0, 0, 0)
    assert set(r.kept.tolist()) == {0, 1, 2}
    # min-p relative to the max: 0.2/0.4 = 0.5 kept at min_p 0.45, 0.1/0.4 dropped
    r = o.sample_row(z, "f32", _p(temperature=1.0, min_p=0.45), None, 0, 0, 0)
    assert set(r.kept.tolist()) == {0, 1, 2}


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
def test_all_equal_logits_closed_forms():
    V = 37
    z = np.zeros(V, dtype=np.float32) + 0.5
    for k in (1, 2, 5, 36):
        r = o.sample_row(z, "f32", _p(temperature=1.0, top_k=k + (k == 1)), None, 0, 0, 0)
        kk = k + (k == 1)
        assert r.kept.tolist() == list(range(kk))
    for p in (0.1, 0.33, 0.5, 0.77, 0.99):
        assert (p * V) % 1 != 0
        r = o.sample_row(z, "f32", _p(temperature=0.8, top_p=p), None, 0, 0, 0)
        assert r.L == math.ceil(np.float32(p) * V)
        assert r.kept.tolist() == list(range(r.L))


def test_two_level_row_probabilities():
    # a logits, b logits, delta = a - b: each top token has q = 1 / (na + nb * e^(-delta/T))
    na, nb, delta, T = 3, 5, 1.25, 0.7
    z = np.array([0.0] * nb + [delta] * na, dtype=np.float32)
    r = o.sample_row(z, "f32", _p(temperature=T), None, 0, 0, 0, want_probs=True)
    qa = 1.0 / (na + nb * math.exp(-delta / T))
    qb = math.exp(-delta / T) * qa
    assert np.allclose(r.probs[nb:], qa, rtol=1e-14) and np.allclose(r.probs[:nb], qb, rtol=1e-14)


def test_no_filter_probs_equal_library_softmax():
    rng = np.random.default_rng(7)
    for _ in range(20):
        V = int(rng.integers(2, 3000))
        z = o.widen(rng.normal(0, 3, V).astype(np.float32), "f32")
        T = float(np.float32(rng.uniform(0.2, 2.0)))
        r = o.sample_row(z, "f32", _p(temperature=T, top_k=-1, top_p=1.0, min_p=0.0), None, 0, 0, 0,
                         want_probs=True)
        assert r.L == V
        ref = scipy.special.softmax(z.astype(np.float64) / T)
        assert np.allclose(r.probs, ref, rtol=1e-12, atol=0)
        assert abs(math.fsum(r.probs.tolist()) - 1.0) < 1e-14


# --------------------------------------------------------------------------
# the draw
# --------------------------------------------------------------------------
def test_draw_crafted_uniforms():
    z = np.zeros(4, dtype=np.float32)
    p = _p(temperature=1.0)
    assert o.sample_row(z, "f32", p, None, 0, 0, 0, u_override=0.25).id == 1    # t = 1.0, strict >
    assert o.sample_row(z, "f32", p, None, 0, 0, 0, u_override=0.0).id == 0
    assert o.sample_row(z, "f32", p, None, 0, 0, 0, u_override=1 - 2 ** -53).id == 3
    assert o.sample_row(z, "f32", p, None, 0, 0, 0, u_override=0.2499999).id == 0
    # the draw walks kept ids in id order, not in value order
    z = np.array([0.0, 5.0, 0.0, 5.0], dtype=np.float32)
    p = _p(temperature=1.0, top_k=2)
    assert o.sample_row(z, "f32", p, None, 0, 0, 0, u_override=0.1).id == 1
    assert o.sample_row(z, "f32", p, None, 0, 0, 0, u_override=0.9).id == 3


def _chisq(counts, expected):
    keep = expected >= 5
    obs = np.append(counts[keep], counts[~keep].sum())
    exp = np.append(expected[keep], expected[~keep].sum())
    if exp[-1] == 0:
        obs, exp = obs[:-1], exp[:-1]
    return scipy.stats.chisquare(obs, exp * obs.sum() / exp.sum()).pvalue


def test_chi_square_one_million_seeded_draws():
    rng = np.random.default_rng(8)
    V = 48
    z = o.widen(rng.normal(0, 1.5, V).astype(np.float32), "f32")
    p = _p(temperature=0.9, top_k=30, top_p=0.93, min_p=0.01)
    base = o.sample_row(z, "f32", p, None, 11, 0, 0, want_probs=True)
    N = 1_000_000
    us = np.fromiter(((o.uniform_bits(11, 0, s) >> 11) * 2.0 ** -53 for s in range(N)), dtype=np.float64, count=N)
    ids, _ = o.draw(base.kept, base.probs[base.kept], us)
    counts = np.bincount(ids, minlength=V).astype(np.float64)
    assert counts[np.setdiff1d(np.arange(V), base.kept)].sum() == 0
    pval = _chisq(counts[base.kept], base.probs[base.kept] * N)
    assert pval > 1e-3, pval
    # spot-check that the vectorised draw is the per-row draw
    for s in (0, 1, 2, 999_999):
        assert o.sample_row(z, "f32", p, None, 11, 0, s).id == ids[s]


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
def test_argmax_equals_topk1_equals_temperature_to_zero():
    rng = np.random.default_rng(9)
    for i in range(100):
        V = int(rng.integers(2, 500))
        z = o.widen(rng.normal(0, 2, V).astype(np.float32), "f32")
        am = o.argmax_first(z)
        for u in (0.0, 0.3, 0.999):
            assert o.sample_row(z, "f32", _p(temperature=1.3, top_k=1), None, 0, i, 0, u_override=u).id == am
        assert o.sample_row(z, "f32", _p(temperature=0.0), None, 0, i, 0).id == am
        if np.count_nonzero(z == z[am]) == 1:
            assert o.sample_row(z, "f32", _p(temperature=1e-6), None, 0, i, 0).id == am


def test_temperature_to_zero_with_tied_maximum_is_uniform_over_ties():
    z = np.array([1.0, 3.0, 0.5, 3.0, 3.0, 2.9], dtype=np.float32)
    p = _p(temperature=1e-4)
    ids = [o.sample_row(z, "f32", p, None, 5, 0, s).id for s in range(30000)]
    counts = np.bincount(ids, minlength=6)
    assert counts[[0, 2, 5]].sum() == 0
    assert scipy.stats.chisquare(counts[[1, 3, 4]]).pvalue > 1e-3


def test_sort_skip_does_not_move_the_token():
    # top_k=-1, top_p=1, min_p=0 is inert: a filter that is active but keeps
    # every token (top_k >= V, min_p below every weight) draws the same token.
    rng = np.random.default_rng(10)
    for i in range(50):
        V = int(rng.integers(2, 2000))
        z = o.widen(rng.normal(0, 2, V).astype(np.float32), "f32")
        a = o.sample_row(z, "f32", _p(temperature=0.8), None, 3, i, 0)
        b = o.sample_row(z, "f32", _p(temperature=0.8, top_k=V + 3), None, 3, i, 0)
        c = o.sample_row(z, "f32", _p(temperature=0.8, top_p=1.0, min_p=1e-38), None, 3, i, 0)
        assert a.L == V and a.id == b.id
        if c.L == V:
            assert c.id == a.id


def test_invalid_params_give_status_and_minus_one():
    z = np.zeros(4, dtype=np.float32)
    cases = [(dict(temperature=-1.0), o.ROW_BAD_TEMPERATURE), (dict(temperature=np.nan), o.ROW_BAD_TEMPERATURE),
             (dict(top_p=0.0), o.ROW_BAD_TOP_P), (dict(top_p=np.nan), o.ROW_BAD_TOP_P),
             (dict(min_p=-0.1), o.ROW_BAD_MIN_P), (dict(min_p=1.5), o.ROW_BAD_MIN_P),
             (dict(repetition=-1.0), o.ROW_BAD_PENALTY), (dict(presence=np.inf), o.ROW_BAD_PENALTY),
             (dict(flags=2), o.ROW_BAD_FLAGS), (dict(flags=-1), o.ROW_BAD_FLAGS)]
    for kw, code in cases:
        r = o.sample_row(z, "f32", _p(**kw), None, 0, 0, 0)
        assert r.status == code and r.id == -1


# --------------------------------------------------------------------------
# DRY
# --------------------------------------------------------------------------
def _bf_dry(seq, breakers):
    """Brute force by substring search: for every tail length n (no breaker in
    it), every earlier occurrence of the tail that is followed by a token t
    (not a breaker) gives t a repeat of at least n."""
    brk = set(breakers)
    N = len(seq)
    best = {}
    for n in range(1, N):
        tail = list(seq[N - n:])
        if brk & set(tail):
            break
        for i in range(0, N - n):
            if list(seq[i:i + n]) == tail and seq[i + n] not in brk:
                best[seq[i + n]] = max(best.get(seq[i + n], 0), n)
    return best


def _dry(**kw):
    from workloads import make_dry
    return make_dry(1, **kw)[0]


def test_dry_match_lengths_hand_cases():
    assert o.dry_match_lengths([5, 6, 7, 5, 6]) == {7: 2}
    assert o.dry_match_lengths([1, 2, 3, 4, 1, 2, 3]) == {4: 3}
    assert o.dry_match_lengths([9, 9, 9, 9]) == {9: 3}
    assert o.dry_match_lengths([1, 2, 3]) == {}
    # a breaker inside the repeat stops it; a breaker as the next token is never penalised
    assert o.dry_match_lengths([1, 0, 2, 3, 1, 0, 2], breakers=[0]) == {3: 1}
    assert o.dry_match_lengths([4, 0, 5, 4], breakers=[0]) == {}


def test_dry_match_lengths_bruteforce():
    rng = np.random.default_rng(31)
    for _ in range(400):
        N = int(rng.integers(1, 24))
        seq = [int(x) for x in rng.integers(0, 4, N)]
        brk = [int(x) for x in rng.choice(4, size=int(rng.integers(0, 2)), replace=False)]
        assert o.dry_match_lengths(seq, brk) == _bf_dry(seq, brk), (seq, brk)


def test_dry_penalty_values_and_window():
    z = np.zeros(10, dtype=np.float32)
    hist = np.array([1, 2, 3, 4, 1, 2, 3])  # 4 repeats a tail of 3
    out = o.dry_penalize(o.widen(z, "f32"), hist, _dry(multiplier=0.5, base=2.0, allowed_length=2))
    want = np.zeros(10)
    want[4] = -0.5 * 2.0 ** (3 - 2)
    assert np.array_equal(out, want)
    # allowed_length above the repeat: nothing
    out = o.dry_penalize(o.widen(z, "f32"), hist, _dry(multiplier=0.5, base=2.0, allowed_length=4))
    assert np.array_equal(out, np.zeros(10))
    # range 3 keeps the last three tokens [1, 2, 3]: no repeat
    out = o.dry_penalize(o.widen(z, "f32"), hist, _dry(multiplier=0.5, base=2.0, allowed_length=1, range=3))
    assert np.array_equal(out, np.zeros(10))
    # binary32 arithmetic: 1.75^3 by repeated multiplication, then the product
    hist = np.array([7, 1, 2, 3, 4, 5, 7, 1, 2, 3, 4])  # 5 repeats a tail of 4 ([7,1,2,3,4])
    out = o.dry_penalize(o.widen(np.full(10, 0.3, dtype=np.float32), "f32"), hist,
                         _dry(multiplier=0.8, base=1.75, allowed_length=1))
    v = np.float32(1.0)
    for _ in range(5 - 1):
        v = np.float32(v * np.float32(1.75))
    assert out[5] == np.float32(np.float32(0.3) - np.float32(np.float32(0.8) * v))
    assert np.count_nonzero(out != np.float32(0.3)) == 1
    # ids outside [0, V) break repeats: [1, 2, -5, 1, 2] -> no repeat of 2 through -5
    hist = np.array([1, 2, -5, 1, 2])
    out = o.dry_penalize(o.widen(np.zeros(10, dtype=np.float32), "f32"), hist,
                         _dry(multiplier=0.5, base=2.0, allowed_length=1))
    assert np.array_equal(out, np.zeros(10))
    hist = np.array([1, 2, 6, 1, 2])
    out = o.dry_penalize(o.widen(np.zeros(10, dtype=np.float32), "f32"), hist,
                         _dry(multiplier=0.5, base=2.0, allowed_length=1))
    assert out[6] == -1.0 and np.count_nonzero(out) == 1


def test_disabled_dry_is_a_no_op_and_enabled_dry_is_not():
    """The pages' invariant: DRY at multiplier 0.0 leaves every logit (and so
    the token) unchanged; at 0.8 it moves them."""
    rng = np.random.default_rng(32)
    V = 64
    z = rng.normal(0, 1, V).astype(np.float32)
    hist = np.array([3, 9, 11, 3, 9, 11, 3, 9])  # 11 repeats a tail of 5
    z[11] = z.max() + 0.5  # 11 is the argmax without DRY
    p = _p(temperature=0.0)
    plain = o.sample_row(z, "f32", p, hist, 1, 0, 0)
    off = o.sample_row(z, "f32", p, hist, 1, 0, 0, dry=_dry(multiplier=0.0))
    on = o.sample_row(z, "f32", p, hist, 1, 0, 0, dry=_dry(multiplier=0.8))
    assert np.array_equal(o.dry_penalize(o.widen(z, "f32"), hist, _dry(multiplier=0.0)), o.widen(z, "f32"))
    assert off.id == plain.id == 11 and off.max_logit == plain.max_logit
    assert on.id != 11


def test_dry_parameter_errors():
    z = np.zeros(4, dtype=np.float32)
    for field, bad in (("multiplier", -0.1), ("multiplier", np.inf), ("base", 0.0), ("base", np.nan),
                       ("allowed_length", 0), ("range", -1)):
        d = _dry(multiplier=0.5)
        d[field] = bad
        r = o.sample_row(z, "f32", _p(), np.array([1, 2]), 0, 0, 0, dry=d)
        assert r.status == o.ROW_BAD_PENALTY and r.id == -1, (field, bad)


# --------------------------------------------------------------------------
# anti-vacuity: planted mistakes must turn a pin red
# --------------------------------------------------------------------------
def _red(test_fn):
    try:
        test_fn()
    except AssertionError:
        return True
    return False


def test_planted_mistakes_are_caught(monkeypatch):
    # highest-index tie-break in argmax
    with monkeypatch.context() as m:
        m.setattr(o, "argmax_first", lambda z: int(len(z) - 1 - np.argmax(z[::-1])))
        assert _red(test_argmax_bruteforce_with_ties)
    # >= instead of > in the draw
    with monkeypatch.context() as m:
        real = o.draw

        def draw_ge(kept, wk, u):
            u = np.atleast_1d(np.asarray(u, dtype=np.float64))
            C = np.cumsum(wk.astype(np.longdouble))
            t = u * math.fsum(wk.tolist())
            pos = np.minimum(np.searchsorted(C, t, side="left"), len(C) - 1)
            return kept[pos], np.ones_like(u)
        m.setattr(o, "draw", draw_ge)
        assert _red(test_draw_crafted_uniforms)
        m.setattr(o, "draw", real)
    # dropped frequency term
    with monkeypatch.context() as m:
        real_pen = o.penalize_one
        m.setattr(o, "penalize_one", lambda z, c, pr, fr, rp: real_pen(z, c, pr, 0.0, rp))
        assert _red(test_penalty_hand_cases)
    # top-p measured against the mass kept by top-k (renormalisation)
    with monkeypatch.context() as m:
        real_cut = o.cutoff

        def renorm(z, w, k, p, mp, *bands):
            c = real_cut(z, w, k, 1.0, mp, *bands)
            kept = c.order[: c.L]
            c2 = real_cut(z[kept], w[kept], -1, p, 0.0)
            c.L = min(c.L, c2.L)
            return c
        m.setattr(o, "cutoff", renorm)
        assert _red(test_combined_filters_take_the_shortest_prefix_without_renormalising)
    # the wide rule not applied, or applied without the ties themselves
    with monkeypatch.context() as m:
        m.setattr(o, "widen_ties", lambda z, order, L: L)
        assert _red(test_wide_ties_bruteforce)
        assert _red(test_wide_ties_on_a_tied_diffuse_support)
    with monkeypatch.context() as m:
        m.setattr(o, "widen_ties", lambda z, order, L: max(L, int(np.count_nonzero(z > z[order[L - 1]]))))
        assert _red(test_wide_ties_bruteforce)
    # DRY: a repeat counted one token too long, or breakers ignored
    with monkeypatch.context() as m:
        real_ml = o.dry_match_lengths
        m.setattr(o, "dry_match_lengths", lambda seq, breakers=(): {t: n + 1 for t, n in real_ml(seq, breakers).items()})
        assert _red(test_dry_match_lengths_hand_cases)
        assert _red(test_dry_penalty_values_and_window)
    with monkeypatch.context() as m:
        real_ml = o.dry_match_lengths
        m.setattr(o, "dry_match_lengths", lambda seq, breakers=(): real_ml(seq, ()))
        assert _red(test_dry_match_lengths_bruteforce)
    # a draw margin of zero (every mismatch would be excused)
    with monkeypatch.context() as m:
        real = o.draw
        m.setattr(o, "draw", lambda kept, wk, u: (real(kept, wk, u)[0], np.zeros(np.atleast_1d(u).shape)))
        assert _red(test_margin_id_closed_form)
        assert _red(test_margin_id_is_the_distance_to_a_flip)
    # top-p and min-p margins of zero, or measured against the wrong quantity
    for field, bad in (("margin_p", lambda c: 0.0), ("margin_m", lambda c: 0.0),
                       ("margin_p", lambda c: c.margin_p * c.S), ("margin_m", lambda c: c.margin_m * 10.0)):
        with monkeypatch.context() as m:
            real_cut = o.cutoff

            def planted(*args, _f=field, _b=bad, _r=real_cut):
                c = _r(*args)
                if math.isfinite(getattr(c, _f)):
                    setattr(c, _f, _b(c))
                return c
            m.setattr(o, "cutoff", planted)
            pin = test_margin_p_is_the_distance_to_a_flip if field == "margin_p" else test_margin_m_is_the_distance_to_a_flip
            closed = test_margin_p_closed_form if field == "margin_p" else test_margin_m_closed_form
            assert _red(pin) or _red(closed), field


# --------------------------------------------------------------------------
# the margins the parity tests use to excuse a decision near its threshold
# --------------------------------------------------------------------------
def test_margin_id_closed_form():
    # four equal weights (S_K = 4, CDF boundaries at 1, 2, 3): u = 0.25 + d puts
    # t = 1 + 4d inside id 1's interval [1, 2), at 4d from its lower edge
    z = np.zeros(4, dtype=np.float32)
    p = _p(temperature=1.0)
    for d in (0.125, 2.0 ** -10, 2.0 ** -20, 2.0 ** -30):
        r = o.sample_row(z, "f32", p, None, 0, 0, 0, u_override=0.25 + d)
        assert r.id == 1 and math.isclose(r.margin_id, d, rel_tol=1e-9), (d, r.margin_id)
        r = o.sample_row(z, "f32", p, None, 0, 0, 0, u_override=0.75 - d)
        assert r.id == 2 and math.isclose(r.margin_id, d, rel_tol=1e-9), (d, r.margin_id)
    # exactly on a boundary the margin is zero
    assert o.sample_row(z, "f32", p, None, 0, 0, 0, u_override=0.5).margin_id == 0.0


def test_margin_id_is_the_distance_to_a_flip():
    # moving u by less than the margin keeps the id; by a little more, one way
    # or the other, changes it
    rng = np.random.default_rng(31)
    checked = 0
    for _ in range(300):
        V = int(rng.integers(2, 12))
        z = o.widen(rng.normal(0, 1.5, V).astype(np.float32), "f32")
        p = _p(temperature=float(rng.uniform(0.5, 2.0)))
        u = float(rng.uniform(0.0, 1.0))
        r = o.sample_row(z, "f32", p, None, 0, 0, 0, u_override=u)
        mg = r.margin_id
        if not (1e-9 < mg < 0.2) or u - 1.1 * mg < 0 or u + 1.1 * mg >= 1:
            continue
        same = [o.sample_row(z, "f32", p, None, 0, 0, 0, u_override=u + s * 0.9 * mg).id for s in (-1, 1)]
        moved = [o.sample_row(z, "f32", p, None, 0, 0, 0, u_override=u + s * 1.1 * mg).id for s in (-1, 1)]
        assert same == [r.id, r.id], (u, mg)
        assert moved[0] != r.id or moved[1] != r.id, (u, mg)
        checked += 1
    assert checked > 200


def test_margin_p_closed_form():
    # eight equal weights, cumulative sums 1..8 (S = 8); top_p = 3/8 - d puts the
    # target 8d below the cumulative sum 3: L_p = 3 and margin_p = d
    z = np.zeros(8, dtype=np.float32)
    for d in (2.0 ** -6, 2.0 ** -10, 2.0 ** -16):
        tp = 0.375 - d
        assert float(np.float32(tp)) == tp
        r = o.sample_row(z, "f32", _p(temperature=1.0, top_p=tp), None, 0, 0, 0)
        assert r.L_p == 3 and math.isclose(r.margin_p, d, rel_tol=1e-12), (d, r.margin_p)
        tp = 0.375 + d  # now just past the sum 3: L_p = 4, margin d again
        r = o.sample_row(z, "f32", _p(temperature=1.0, top_p=tp), None, 0, 0, 0)
        assert r.L_p == 4 and math.isclose(r.margin_p, d, rel_tol=1e-12), (d, r.margin_p)


def test_margin_p_is_the_distance_to_a_flip():
    rng = np.random.default_rng(32)
    checked = 0
    for _ in range(300):
        V = int(rng.integers(3, 40))
        z = o.widen(rng.normal(0, 1.5, V).astype(np.float32), "f32")
        T = float(rng.uniform(0.5, 2.0))
        tp = float(rng.uniform(0.1, 0.95))
        _, w = o.weights(z, T)
        c = o.cutoff(z, w, -1, tp, 0.0)
        mg = c.margin_p
        if not (1e-9 < mg < 0.05):
            continue
        near = [o.cutoff(z, w, -1, tp + s * 0.9 * mg, 0.0).L_p for s in (-1, 1)]
        far = [o.cutoff(z, w, -1, tp + s * 1.1 * mg, 0.0).L_p for s in (-1, 1)]
        assert near == [c.L_p, c.L_p], (tp, mg)
        assert far[0] != c.L_p or far[1] != c.L_p, (tp, mg)
        checked += 1
    assert checked > 150


def test_margin_m_closed_form():
    # at T = 1/ln 2 (rounded to binary32) the weights are powers of two to
    # within 1e-7, so a min_p of 2^-4 (1 + d) sits d above the weight of the
    # value 4 below the maximum: margin_m = d / (1 + d)
    T = float(np.float32(1.0 / math.log(2.0)))
    z = np.array([0.0, -4.0, -9.0, -20.0], dtype=np.float32)
    for d in (2.0 ** -6, 2.0 ** -10, 2.0 ** -14):
        mp = 2.0 ** -4 * (1.0 + d)
        assert float(np.float32(mp)) == mp
        r = o.sample_row(z, "f32", _p(temperature=T, min_p=mp), None, 0, 0, 0)
        assert r.L_m == 1 and abs(r.margin_m - d / (1 + d)) < 1e-6, (d, r.margin_m)
        mp = 2.0 ** -4 * (1.0 - d)  # now just below that weight: it is kept
        r = o.sample_row(z, "f32", _p(temperature=T, min_p=mp), None, 0, 0, 0)
        assert r.L_m == 2 and abs(r.margin_m - d / (1 - d)) < 1e-6, (d, r.margin_m)


def test_margin_m_is_the_distance_to_a_flip():
    rng = np.random.default_rng(33)
    checked = 0
    for _ in range(300):
        V = int(rng.integers(3, 40))
        z = o.widen(rng.normal(0, 1.5, V).astype(np.float32), "f32")
        T = float(rng.uniform(0.5, 2.0))
        mp = float(rng.uniform(0.01, 0.9))
        _, w = o.weights(z, T)
        c = o.cutoff(z, w, -1, 1.0, mp)
        mg = c.margin_m
        if not (1e-9 < mg < 0.2):
            continue
        near = [o.cutoff(z, w, -1, 1.0, mp * (1 + s * 0.9 * mg)).L_m for s in (-1, 1)]
        far = [o.cutoff(z, w, -1, 1.0, mp * (1 + s * 1.1 * mg)).L_m for s in (-1, 1)]
        assert near == [c.L_m, c.L_m], (mp, mg)
        assert far[0] != c.L_m or far[1] != c.L_m, (mp, mg)
        checked += 1
    assert checked > 150


def test_near_counts():
    # equal weights: every cut position is its own cumulative sum k; with
    # top_p * S on one of them only that position is within a small band, and
    # with min_p = 1 every id sits on the threshold
    z = np.zeros(10, dtype=np.float32)
    r = o.sample_row(z, "f32", _p(temperature=1.0, top_p=0.5), None, 0, 0, 0, band_p=1e-7, band_m=1e-6)
    assert r.L_p == 5 and r.near_p == 1 and r.margin_p == 0.0
    r = o.sample_row(z, "f32", _p(temperature=1.0, min_p=1.0), None, 0, 0, 0, band_p=1e-7, band_m=1e-6)
    assert r.L_m == 10 and r.near_m == 10
    # a band wider than the spacing of the sums takes in the neighbours
    r = o.sample_row(z, "f32", _p(temperature=1.0, top_p=0.5), None, 0, 0, 0, band_p=0.15)
    assert r.near_p == 3


# --------------------------------------------------------------------------
# top-n log-probabilities (Arc PR #222, section 3(c); reading in the oracle)
# --------------------------------------------------------------------------
def test_top_logprobs_uniform_row_closed_form():
    # equal logits: every id has probability 1/V, the order is by id
    V, n = 37, 10
    row = np.full(V, 1.25, np.float32)
    r = o.top_logprobs_row(row, "f32", 0.6, n)
    assert r.status == o.ROW_OK
    assert r.ids.tolist() == list(range(n))
    assert np.allclose(r.logprobs, -math.log(V), rtol=0, atol=1e-15)


def test_top_logprobs_two_levels_closed_form():
    # k ids at value a, the rest at b < a: S = k + (V - k) exp((b - a) / T)
    V, k, T, n = 50, 7, 0.8, 12
    rng = np.random.default_rng(3)
    hi = np.sort(rng.choice(V, k, replace=False))
    row = np.full(V, -0.5, np.float32)
    row[hi] = 2.0
    S = k + (V - k) * math.exp((-0.5 - 2.0) / T)
    r = o.top_logprobs_row(row, "f32", T, n)
    lo_ids = [v for v in range(V) if v not in set(hi.tolist())][: n - k]
    assert r.ids.tolist() == hi.tolist() + lo_ids
    assert np.allclose(r.logprobs[:k], -math.log(S), rtol=0, atol=1e-14)
    assert np.allclose(r.logprobs[k:], (-0.5 - 2.0) / T - math.log(S), rtol=0, atol=1e-14)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_top_logprobs_against_scipy_log_softmax(dtype):
    # scipy's log_softmax of z / T and a stable sort of -z (first ids first)
    rng = np.random.default_rng(11)
    for trial in range(20):
        V = int(rng.integers(1, 400))
        T = float(rng.uniform(0.05, 3.0))
        n = int(rng.integers(1, 65))
        z = (rng.normal(0, 2, V) * (4 if trial % 3 == 0 else 1)).astype(np.float32)
        if trial % 4 == 1:
            z = np.round(z * 2) / 2  # many ties
        raw = f32_to_bf16_bits(z) if dtype == "bf16" else z.astype(np.float32)
        zw = o.widen(raw, dtype).astype(np.float64)
        ref_lp = scipy.special.log_softmax(zw / T)
        ref_ids = np.argsort(-zw, kind="stable")[:n]
        r = o.top_logprobs_row(raw, dtype, T, n)
        k = min(n, V)
        assert r.ids[:k].tolist() == ref_ids.tolist()
        assert np.allclose(r.logprobs[:k], ref_lp[ref_ids], rtol=1e-12, atol=1e-12)
        assert (r.ids[k:] == -1).all() and np.isneginf(r.logprobs[k:]).all()


def test_top_logprobs_full_row_sums_to_one():
    rng = np.random.default_rng(5)
    V = 300
    z = rng.normal(0, 3, V).astype(np.float32)
    r = o.top_logprobs_row(z, "f32", 0.7, V)
    assert sorted(r.ids.tolist()) == list(range(V))
    assert abs(math.fsum(np.exp(r.logprobs).tolist()) - 1.0) < 1e-13
    assert np.all(np.diff(r.logprobs) <= 0)


def test_top_logprobs_special_values():
    # +inf logits share all the mass; NaN counts as -inf; a row of -inf is uniform
    row = np.array([1.0, np.inf, np.nan, 3.0, np.inf, -np.inf], np.float32)
    r = o.top_logprobs_row(row, "f32", 1.0, 6)
    assert r.ids.tolist() == [1, 4, 3, 0, 2, 5]
    assert np.allclose(r.logprobs[:2], -math.log(2), atol=1e-15)
    assert np.isneginf(r.logprobs[2:]).all()
    allneg = np.array([-np.inf, np.nan, -np.inf, -np.inf], np.float32)
    r = o.top_logprobs_row(allneg, "f32", 2.0, 3)
    assert r.ids.tolist() == [0, 1, 2]
    assert np.allclose(r.logprobs, -math.log(4), atol=1e-15)
    # -0 and +0 are one value: ties broken by id
    r = o.top_logprobs_row(np.array([-0.0, 0.0, -1.0], np.float32), "f32", 1.0, 2)
    assert r.ids.tolist() == [0, 1]


def test_top_logprobs_bad_temperature():
    for T in (0.0, -1.0, float("nan"), float("inf")):
        r = o.top_logprobs_row(np.zeros(4, np.float32), "f32", T, 3)
        assert r.status == o.ROW_BAD_TEMPERATURE
        assert (r.ids == -1).all() and np.isnan(r.logprobs).all()
