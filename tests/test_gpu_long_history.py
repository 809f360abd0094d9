"""GPU parity of penalised rows beyond the LDS penalty tables (more than
ARCS_MAX_HISTORY distinct history ids, or V above ARCS_MAX_PENALTY_VOCAB)
when the call brings a long-history workspace: such a row's penalised
logits go to its slice of the workspace in binary32 and the general pipeline
samples that copy.  Ids are compared with the oracle (greedy rows exactly,
sampled rows up to the id margin); rows within the tables in the same batch
keep their own path; without the workspace the rows keep their status codes."""

import numpy as np
import pytest

from _util import ensure_built, to_device_logits
from oracle import sampler as oracle
from workloads import make_dry, make_params, make_workload

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


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _history(rng, V, distinct, length, phrase=None):
    """`distinct` distinct ids in [0, V) spread over `length` entries (the rest
    repeats of them, so counts vary), three entries outside [0, V), and, when
    given, a phrase repeated at the end (DRY repeats)."""
    base = rng.choice(V, size=distinct, replace=False)
    h = np.concatenate([base, rng.choice(base, size=length - distinct), [-1, V + 5, V]])
    rng.shuffle(h)
    if phrase is not None:
        h = np.concatenate([h, np.tile(phrase, 4)])
    return h.astype(np.int32)


def _batch(rng, V, distincts, length_of, phrases=None):
    hs = [_history(rng, V, d, length_of(d), None if phrases is None else phrases[b]) for b, d in enumerate(distincts)]
    offs = np.concatenate([[0], np.cumsum([len(h) for h in hs])]).astype(np.int64)
    return np.concatenate(hs), offs


def _params(B, rng):
    """Greedy, top-k, top-p + min-p and unfiltered rows, all penalised."""
    p = make_params(B, temperature=0.8, presence=0.5, frequency=0.3, repetition=1.1)
    for b in range(B):
        kind = b % 4
        if kind == 0:
            p[b]["temperature"] = 0.0
        elif kind == 1:
            p[b]["top_k"] = int(rng.integers(5, 300))
        elif kind == 2:
            p[b]["top_p"] = float(rng.uniform(0.5, 0.95))
            p[b]["min_p"] = 0.02
        else:
            p[b]["temperature"] = float(rng.uniform(0.5, 1.5))
    p[5]["presence"], p[5]["repetition"] = 0.0, 1.0  # frequency alone
    return p


def _compare(ids, status, refs, where):
    excused = 0
    for b, r in enumerate(refs):
        assert status[b] == r.status == 0, (where, b, status[b], r.status)
        if ids[b] != r.id:
            assert not r.greedy, (where, b, int(ids[b]), r.id)
            assert r.margin_id < MARGIN_ID or r.margin_p < MARGIN_P or r.margin_m < MARGIN_M, (where, b)
            excused += 1
    assert excused <= 1, (where, excused)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_long_histories_match_the_oracle(arcs, dtype):
    import torch
    B, V = 12, 129_280
    rng = np.random.default_rng(17 if dtype == "bf16" else 18)
    w = make_workload("zipf_b512_bf16_mixed_penalties", B=B, V=V)
    logits_np = w.logits if dtype == "bf16" else oracle.widen(w.logits, "bf16").astype(np.float32)
    distincts = [300, 8_000, 32_000, 4_097, 6_000, 12_000, 200, 20_000, 4_096, 9_000, 50, 16_000]
    hist, offs = _batch(rng, V, distincts, lambda d: d + d // 4 + 10)
    p = _params(B, rng)
    logits = to_device_logits(logits_np, dtype)
    params = arcs.params_to_device(p)
    hi, ho = _dev(hist), _dev(offs)
    long_rows = [b for b, d in enumerate(distincts) if d > arcs.MAX_HISTORY]  # 4,097 and up; 4,096 fits
    # without the workspace: the long rows fail with their status, the others are sampled
    status = torch.empty(B, dtype=torch.int32, device="cuda")
    got = arcs.sample(logits, params, hi, ho, seed=5, step=2, out_status=status).cpu().numpy()
    st = status.cpu().numpy()
    assert [b for b in range(B) if st[b] != 0] == long_rows
    assert all(st[b] == arcs.ROW_HISTORY_TOO_LONG and got[b] == -1 for b in long_rows)
    # with it: every row
    ws = torch.empty(arcs.long_history_workspace_bytes(B, V), dtype=torch.uint8, device="cuda")
    for step in (2, 9):
        got = arcs.sample(logits, params, hi, ho, seed=5, step=step, out_status=status, workspace=ws).cpu().numpy()
        refs = oracle.sample(logits_np, dtype, p, hist, offs, 5, step, band_p=MARGIN_P, band_m=MARGIN_M)
        _compare(got, status.cpu().numpy(), refs, f"{dtype} step {step}")
    # the debug entry point: the same ids, and the long rows' maxima are the penalised ones
    ids, status_d, stats, _ = arcs.sample_debug(logits, params, hi, ho, seed=5, step=9, workspace=ws)
    assert np.array_equal(ids.cpu().numpy(), got) and (status_d.cpu().numpy() == 0).all()
    for b in long_rows:
        assert stats[b]["max_logit"] == np.float32(refs[b].max_logit), (b, stats[b]["max_logit"], refs[b].max_logit)
        if not refs[b].greedy:
            assert stats[b]["kept"] == refs[b].L or refs[b].margin_p < MARGIN_P or refs[b].margin_m < MARGIN_M, b


def test_long_histories_with_dry(arcs):
    """DRY on rows beyond the tables: the repeat lengths of the window's ids
    (a phrase repeated at the end of each history) lower the ids that would
    continue a repeat, on top of the other penalties."""
    import torch
    B, V = 8, 129_280
    rng = np.random.default_rng(23)
    w = make_workload("zipf_b256_bf16_greedy", B=B, V=V)
    phrases = []
    for b in range(B):
        z = oracle.widen(w.logits[b], "bf16")
        top = np.argsort(-z, kind="stable")[:10]
        phrases.append(rng.choice(top, size=int(rng.integers(3, 7))).astype(np.int32))
    distincts = [6_000, 300, 10_000, 5_000, 7_000, 9_000, 4_500, 8_000]
    hist, offs = _batch(rng, V, distincts, lambda d: d + 100, phrases)
    p = make_params(B, temperature=0.0, presence=0.2, frequency=0.1)
    p["temperature"][1::2] = 0.9
    p["min_p"][1::2] = 0.05
    dry = make_dry(B, multiplier=rng.uniform(0.5, 3.0, B), base=1.75, allowed_length=2,
                   range=np.where(np.arange(B) % 3 == 0, 64, 0))
    breakers = [int(phrases[2][0])]
    logits = to_device_logits(w.logits, "bf16")
    ws = torch.empty(arcs.long_history_workspace_bytes(B, V), dtype=torch.uint8, device="cuda")
    status = torch.empty(B, dtype=torch.int32, device="cuda")
    bd = torch.tensor(breakers, dtype=torch.int32, device="cuda")
    got = arcs.sample_dry(logits, arcs.params_to_device(p), _dev(hist), _dev(offs), arcs.dry_to_device(dry), bd,
                          seed=3, step=1, out_status=status, workspace=ws).cpu().numpy()
    refs = oracle.sample(w.logits, "bf16", p, hist, offs, 3, 1, band_p=MARGIN_P, band_m=MARGIN_M, dry=dry,
                         breakers=breakers)
    _compare(got, status.cpu().numpy(), refs, "dry")
    # the penalty moved some greedy rows' argmax
    plain = oracle.sample(w.logits, "bf16", p, hist, offs, 3, 1)
    assert any(r.id != q.id for r, q in zip(refs[::2], plain[::2]))


def test_vocabulary_beyond_the_tables(arcs):
    """V above ARCS_MAX_PENALTY_VOCAB with active penalties: with the
    workspace the rows are sampled (general pipeline on the binary32 copy),
    without it they keep ARCS_ROW_VOCAB_TOO_LARGE."""
    import torch
    B, V = 3, arcs.MAX_PENALTY_VOCAB + 8
    rng = np.random.default_rng(29)
    z = rng.normal(0.0, 2.0, (B, V)).astype(np.float32)
    hist = np.concatenate([np.argsort(-z[b])[:40] for b in range(B)]).astype(np.int32)
    offs = np.array([0, 40, 80, 120], dtype=np.int64)
    p = make_params(B, temperature=0.0, presence=3.0)
    p[1]["temperature"], p[1]["top_k"] = 1.0, 20
    p[2]["temperature"] = 0.7
    logits = to_device_logits(z, "f32")
    params = arcs.params_to_device(p)
    status = torch.empty(B, dtype=torch.int32, device="cuda")
    got = arcs.sample(logits, params, _dev(hist), _dev(offs), seed=1, step=0, out_status=status).cpu().numpy()
    assert (status.cpu().numpy() == arcs.ROW_VOCAB_TOO_LARGE).all() and (got == -1).all()
    ws = torch.empty(arcs.long_history_workspace_bytes(B, V), dtype=torch.uint8, device="cuda")
    got = arcs.sample(logits, params, _dev(hist), _dev(offs), seed=1, step=0, out_status=status,
                      workspace=ws).cpu().numpy()
    refs = oracle.sample(z, "f32", p, hist, offs, 1, 0, band_p=MARGIN_P, band_m=MARGIN_M)
    _compare(got, status.cpu().numpy(), refs, "vocab")
    assert got[0] not in set(hist[:40].tolist())  # the penalty moved the greedy row off its top ids
