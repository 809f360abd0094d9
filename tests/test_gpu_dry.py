"""GPU parity of arcs_sample_dry (the DRY penalty) against the oracle: greedy
rows exactly (the penalised argmax), sampled rows up to the id margin, with
and without the other penalties, sequence breakers and windows; the
disabled default (multiplier 0) gives arcs_sample's ids; invalid records
give the row error."""

import numpy as np
import pytest

from _util import ensure_built, hist_to_device, to_device_logits
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


def _repeat_histories(w, rng, hist_len):
    """Histories built from the row's own top tokens so that repeats of the
    tail are continued by tokens that matter: a random phrase over a small
    alphabet of high-logit ids, repeated with variations."""
    from oracle.sampler import widen
    hs = []
    for i in range(w.logits.shape[0]):
        z = widen(w.logits[i], w.dtype)
        top = np.argsort(-z, kind="stable")[:12]
        phrase = rng.choice(top, size=int(rng.integers(3, 9)))
        seq = []
        while len(seq) < hist_len:
            seq.extend(phrase.tolist())
            if rng.random() < 0.3:
                seq.append(int(rng.choice(top)))
        seq = seq[:hist_len]
        # a few ids outside [0, V) and plain random ids
        for _ in range(3):
            seq[int(rng.integers(0, hist_len))] = int(rng.choice([-1, w.V + 3, int(rng.integers(0, w.V))]))
        hs.append(np.asarray(seq, dtype=np.int32))
    w.hist_ids = np.concatenate(hs)
    w.hist_offsets = np.concatenate([[0], np.cumsum([len(h) for h in hs])]).astype(np.int64)


def _run(arcs, w, dry, breakers=None, seed=3, step=1):
    import torch
    logits = to_device_logits(w.logits, w.dtype)
    hi, ho = hist_to_device(w)
    status = torch.empty(w.B, dtype=torch.int32, device="cuda")
    bd = None if breakers is None else torch.tensor(breakers, dtype=torch.int32, device="cuda")
    ids = arcs.sample_dry(logits, arcs.params_to_device(w.params), hi, ho, arcs.dry_to_device(dry), bd,
                          seed=seed, step=step, out_status=status)
    return ids.cpu().numpy(), status.cpu().numpy()


def _refs(w, dry, breakers=None, seed=3, step=1):
    return oracle.sample(w.logits, w.dtype, w.params, w.hist_ids, w.hist_offsets, seed, step,
                         band_p=MARGIN_P, band_m=MARGIN_M, dry=dry, breakers=breakers or ())


def _compare(ids, status, refs, where):
    excused = 0
    for b, r in enumerate(refs):
        assert status[b] == r.status, (where, b, status[b], r.status)
        if ids[b] != r.id:
            assert r.status == 0 and not r.greedy, (where, b, int(ids[b]), r.id)
            assert r.margin_id < MARGIN_ID or r.margin_p < MARGIN_P or r.margin_m < MARGIN_M, (where, b)
            excused += 1
    assert excused <= 1, (where, excused)


@pytest.mark.parametrize("V", [129_280, 20_005])
def test_dry_greedy_rows_are_exact(arcs, V):
    """Greedy rows: the argmax of the penalised logits, bit for bit, so every
    DRY penalty the kernel folds in must equal the oracle's."""
    rng = np.random.default_rng(V)
    B = 48
    w = make_workload("zipf_b256_bf16_greedy", B=B, V=V)
    _repeat_histories(w, rng, 300)
    w.params = make_params(B, temperature=0.0)
    w.params["presence"][::3] = 0.4
    w.params["repetition"][1::3] = 1.2
    dry = make_dry(B, multiplier=rng.uniform(0.2, 3.0, B), base=rng.uniform(1.1, 2.0, B),
                   allowed_length=rng.integers(1, 4, B), range=np.where(np.arange(B) % 4 == 0, 64, 0))
    ids, status = _run(arcs, w, dry)
    refs = _refs(w, dry)
    _compare(ids, status, refs, f"greedy V={V}")
    # the penalty moved the argmax on many rows
    plain = oracle.sample(w.logits, w.dtype, w.params, w.hist_ids, w.hist_offsets, 3, 1)
    assert sum(r.id != q.id for r, q in zip(refs, plain)) >= B // 4


@pytest.mark.parametrize("V", [129_280, 20_005])
def test_dry_sampled_rows(arcs, V):
    rng = np.random.default_rng(V + 1)
    B = 40
    w = make_workload("zipf_b256_bf16_greedy", B=B, V=V)
    _repeat_histories(w, rng, 200)
    p = make_params(B, temperature=0.8)
    for b in range(B):
        mode = b % 4
        if mode == 0:
            p[b]["top_k"] = int(rng.integers(2, 200))
        elif mode == 1:
            p[b]["top_p"] = float(rng.uniform(0.5, 0.95))
        elif mode == 2:
            p[b]["min_p"] = 0.05
            p[b]["frequency"] = 0.3
    w.params = p
    dry = make_dry(B, multiplier=0.8, base=1.75, allowed_length=2)
    breakers = [int(x) for x in w.hist_ids[:2]]
    for step in (0, 4):
        ids, status = _run(arcs, w, dry, breakers, step=step)
        _compare(ids, status, _refs(w, dry, breakers, step=step), f"sampled V={V} step={step}")


def test_disabled_dry_gives_the_plain_ids(arcs):
    """The pages' invariant: at multiplier 0 the record changes nothing (the
    rows keep arcs_sample's path and ids)."""
    import torch
    B, V = 32, 129_280
    rng = np.random.default_rng(5)
    w = make_workload("zipf_b256_bf16_t0.7_k50_p0.9_minp0.05", B=B, V=V)
    _repeat_histories(w, rng, 100)
    dry = make_dry(B, multiplier=0.0)
    ids, status = _run(arcs, w, dry)
    hi, ho = hist_to_device(w)
    plain = arcs.sample(to_device_logits(w.logits, "bf16"), arcs.params_to_device(w.params), hi, ho,
                        seed=3, step=1).cpu().numpy()
    assert np.array_equal(ids, plain) and (status == 0).all()
    on = _run(arcs, w, make_dry(B, multiplier=5.0, allowed_length=1))[0]
    assert not np.array_equal(on, plain)
    torch.cuda.synchronize()


def test_dry_record_errors(arcs):
    B, V = 6, 4096
    w = make_workload("normal_b4_bf16", B=B, V=V)
    w.hist_ids = np.array([1, 2, 3] * B, dtype=np.int32)
    w.hist_offsets = np.arange(B + 1, dtype=np.int64) * 3
    dry = make_dry(B, multiplier=0.5)
    dry[0]["multiplier"] = -1.0
    dry[1]["base"] = 0.0
    dry[2]["allowed_length"] = 0
    dry[3]["range"] = -2
    dry[4]["multiplier"] = np.nan
    ids, status = _run(arcs, w, dry)
    assert status.tolist() == [4, 4, 4, 4, 4, 0]
    assert (ids[:5] == -1).all() and ids[5] >= 0
    _compare(ids, status, _refs(w, dry), "errors")
