"""CPU oracle for batched on-device token sampling (fp64, plain, slow).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
path never calls it, and it shares no code with the HIP kernels.

What it computes follows the Arc engine's pull-request pages:

* Arc PR #222 ("ARC_SAMPLE_ON_DEVICE"), section 3(b): the host sampler sorts the
  probabilities of the whole vocabulary, then three consumers read the sorted
  list in turn -- zero-the-rest (top-k), the top-p walk, the min-p scan --
  before a multinomial draw over the (unsorted) probability vector.  Under
  top_k=-1, top_p=1, min_p=0 all three are inert, the sort can be skipped,
  and the drawn token does not move.
* Arc PR #222, section 3(a): a penalty whose multiplier is 0 changes no logit.
* Arc PR #217 ("device decode loop"), "What this does" and "Default OFF": device argmax is compared bit for bit with
  the host argmax; the device sampler draws from a SplitMix64 stream.

Where the pages are silent this module takes these readings:

1. Widen the logit to float32 exactly; NaN becomes -inf, -0 becomes +0.
2. Penalties (only for token ids that occur in the row's history, ids outside
   [0, V) skipped, c = occurrence count): repetition r first
   (z/r if z > 0 else z*r), then frequency f (z - f*c), then presence p
   (z - p).  Every operation is one IEEE binary32 round-to-nearest-even
   operation, no fused multiply-add; it is computed here in binary64 and
   rounded once to binary32, which is exact for a single +, -, * or /
   because 53 >= 2*24 + 2.  Off values: p = 0, f = 0, r = 1 (r = 0 is also
   treated as off, the "multiplier 0 is a no-op" convention).
3. Greedy when T == 0 or top_k == 1: argmax of the penalised logits, lowest
   index among equals.
4. Total order: u before v iff z'_u > z'_v, or z'_u == z'_v and u < v.
5. m = max z'; w_v = exp((z'_v - m) / T) in binary64 (w = 1 where z'_v == m,
   which also covers +inf logits); S = sum of w (math.fsum).
6. Kept set K = the first L ids in the total order, L = min(L_k, L_p, L_m):
   L_k = k for 1 <= k < V else V; L_p = the smallest n >= 1 whose cumulative
   mass reaches top_p * S (V when top_p >= 1); L_m = #{v : w_v >= min_p}
   (V when min_p == 0).  No renormalisation between filters.
7. q_v = w_v / S_K on K.
8. u = SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): x is output number
   n + 1 of the generator seeded with ``seed``, n = step * 2**32 + row, and
   u = (x >> 11) * 2**-53.
9. t = u * S_K; walking K in token-id order, the token is the first id whose
   running sum exceeds t (strictly); if rounding leaves none, the last kept id.
10. A row whose logits are all -inf (or NaN) returns id 0.

Error bound: S is correctly rounded (fsum); cumulative sums are taken in
x87 extended precision (64-bit significand), so every cumulative value is
within ~V * 2**-64 * S of the exact one, far below the 1e-7 relative margins
the parity tests excuse.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

MASK64 = (1 << 64) - 1
SPLITMIX_GAMMA = 0x9E3779B97F4A7C15

# Per-row status codes (the library's ABI uses the same numbers).
ROW_OK = 0
ROW_BAD_TEMPERATURE = 1
ROW_BAD_TOP_P = 2
ROW_BAD_MIN_P = 3
ROW_BAD_PENALTY = 4
ROW_BAD_FLAGS = 5

# Row flags (arcs_row_params.flags).
ROW_TIES_WIDE = 1   # keep every id sharing the value of the kept prefix's last id


# --------------------------------------------------------------------------
# step 8: SplitMix64 uniform
# --------------------------------------------------------------------------
def splitmix64_mix(z: int) -> int:
    """The SplitMix64 output function (Stafford's "Mix13" constants)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def splitmix64_output(seed: int, k: int) -> int:
    """Output number k (k >= 1) of SplitMix64 started from state ``seed``.

    The generator adds the golden gamma to its state before every output, so
    output k mixes seed + k * gamma.
    """
    return splitmix64_mix((seed + k * SPLITMIX_GAMMA) & MASK64)


def counter(row: int, step: int) -> int:
    return ((step << 32) + row) & MASK64


def uniform_bits(seed: int, row: int, step: int) -> int:
    return splitmix64_output(seed, counter(row, step) + 1)


def uniform(seed: int, row: int, step: int) -> float:
    x = uniform_bits(seed, row, step)
    return float(x >> 11) * 2.0 ** -53


# --------------------------------------------------------------------------
# step 1: widening
# --------------------------------------------------------------------------
def widen(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Raw logits (bf16 bit patterns as uint16, or float32) -> float32."""
    if dtype == "bf16":
        z = (np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    elif dtype == "f32":
        z = np.array(raw, dtype=np.float32)
    else:
        raise ValueError(dtype)
    z = np.array(z, dtype=np.float32, copy=True)
    z[np.isnan(z)] = -np.inf
    z[z == 0] = np.float32(0.0)  # canonical +0
    return z


# --------------------------------------------------------------------------
# step 2: penalties
# --------------------------------------------------------------------------
def fl32(x: float) -> float:
    """Round a binary64 value to the nearest binary32 (ties to even)."""
    return float(np.float32(x))


def repetition_active(r: float) -> bool:
    return not (r == 1.0 or r == 0.0)


def penalties_active(presence: float, frequency: float, repetition: float) -> bool:
    return presence != 0.0 or frequency != 0.0 or repetition_active(repetition)


def penalize_one(z: float, count: int, presence: float, frequency: float, repetition: float) -> float:
    if repetition_active(repetition):
        z = fl32(z / repetition) if z > 0 else fl32(z * repetition)
    if frequency != 0.0:
        z = fl32(z - fl32(frequency * float(count)))
    if presence != 0.0:
        z = fl32(z - presence)
    if z == 0.0:
        z = 0.0
    return z


def penalize(z: np.ndarray, hist: Optional[np.ndarray], presence: float, frequency: float,
             repetition: float) -> np.ndarray:
    z = z.copy()
    if hist is None or len(hist) == 0 or not penalties_active(presence, frequency, repetition):
        return z
    V = len(z)
    h = np.asarray(hist, dtype=np.int64)
    h = h[(h >= 0) & (h < V)]
    if len(h) == 0:
        return z
    counts = np.bincount(h, minlength=V)
    for v in np.nonzero(counts)[0]:
        z[v] = np.float32(penalize_one(float(z[v]), int(counts[v]), presence, frequency, repetition))
    return z


# --------------------------------------------------------------------------
# step 2b: the DRY penalty
# --------------------------------------------------------------------------
# The pages name it (DrySamplingParams, apply_dry_penalty, a multiplier whose
# disabled default 0.0 leaves every logit untouched: Arc PR #222, section
# 3(a)) but do not define it; this is the published "Don't Repeat Yourself"
# sampler: a token that would extend a repeat of the context's tail by one
# more token is penalised, growing exponentially with the repeat's length.
DRY_MAX_WINDOW = 2048   # history tokens matched at most (the last ones)


def dry_validate(d) -> int:
    mult, base = float(d["multiplier"]), float(d["base"])
    if not (math.isfinite(mult) and mult >= 0.0 and math.isfinite(base) and base > 0.0) \
            or int(d["allowed_length"]) < 1 or int(d["range"]) < 0:
        return ROW_BAD_PENALTY
    return ROW_OK


def dry_match_lengths(seq, breakers=()) -> dict:
    """For every token t of seq (but its first): the length n of the longest
    tail of seq that also ends right before an occurrence of t, i.e.
    seq[j-n:j] == seq[N-n:N] with seq[j] == t; no matched token and no t may be
    a sequence breaker.  Returns {t: largest n} over the t with n >= 1."""
    brk = set(int(b) for b in breakers)
    N = len(seq)
    best = {}
    for j in range(1, N):
        t = int(seq[j])
        if t in brk:
            continue
        n = 0
        while n < j and int(seq[j - 1 - n]) == int(seq[N - 1 - n]) and int(seq[j - 1 - n]) not in brk:
            n += 1
        if n > 0:
            best[t] = max(best.get(t, 0), n)
    return best


def dry_penalize(z: np.ndarray, hist: Optional[np.ndarray], d, breakers=()) -> np.ndarray:
    """z[t] -= multiplier * base^(n - allowed_length) for every token t in [0, V)
    with a repeat length n >= allowed_length over the last min(range, 2048)
    history tokens (range 0: all of them, up to 2048).  History ids outside
    [0, V) are not tokens of the vocabulary and break repeats like the
    sequence breakers.  binary32 arithmetic: the power by repeated
    multiplication, then the product, then the subtraction, each rounded."""
    z = z.copy()
    if hist is None or d is None or float(d["multiplier"]) == 0.0:
        return z
    h = np.asarray(hist, dtype=np.int64)
    win = int(d["range"]) if int(d["range"]) > 0 else len(h)
    win = min(win, DRY_MAX_WINDOW, len(h))
    seq = h[len(h) - win:]
    al = int(d["allowed_length"])
    base = np.float32(d["base"])
    mult = np.float32(d["multiplier"])
    V = len(z)
    brk = set(int(b) for b in breakers) | {int(t) for t in seq if not (0 <= int(t) < len(z))}
    for t, n in dry_match_lengths(seq, brk).items():
        if n < al or not (0 <= t < V):
            continue
        v = np.float32(1.0)
        for _ in range(n - al):
            v = np.float32(v * base)
            if not np.isfinite(v):
                break
        pen = np.float32(mult * v)
        z[t] = np.float64(np.float32(np.float32(z[t]) - pen))
    return z


# --------------------------------------------------------------------------
# step 3: argmax
# --------------------------------------------------------------------------
def argmax_first(z: np.ndarray) -> int:
    """Index of the maximum, lowest index among equals (numpy's documented rule)."""
    return int(np.argmax(z))


# --------------------------------------------------------------------------
# steps 4-7: weights, order, cutoffs
# --------------------------------------------------------------------------
def weights(z: np.ndarray, T: float):
    m = float(z.max())
    with np.errstate(invalid="ignore", over="ignore"):
        w = np.exp((z.astype(np.float64) - m) / float(T))
    w[z == m] = 1.0
    w[np.isnan(w)] = 0.0
    return m, w


def total_order(z: np.ndarray) -> np.ndarray:
    """All ids sorted by value descending, then id ascending."""
    return np.lexsort((np.arange(len(z)), -z.astype(np.float64)))


@dataclasses.dataclass
class Cutoff:
    order: np.ndarray
    L: int
    L_k: int
    L_p: int
    L_m: int
    S: float
    margin_p: float   # |top_p*S - nearest bracketing cumulative| / S (inf if off)
    margin_m: float   # min |w - min_p| / min_p (inf if off)
    near_p: int = 0   # cut positions whose cumulative lies within band_p * S of top_p*S
    near_m: int = 0   # ids whose weight lies within band_m * min_p of min_p


def cutoff(z: np.ndarray, w: np.ndarray, top_k: int, top_p: float, min_p: float,
           band_p: float = 0.0, band_m: float = 0.0) -> Cutoff:
    """Step 6.  The margins say how far the two threshold decisions are from
    flipping: margin_p is the distance of top_p*S from the nearer of the two
    cumulative sums around the crossing, over S; margin_m the distance of the
    nearest weight from min_p, over min_p.  near_p / near_m count the cut
    positions (ids) that lie within band_p * S (band_m * min_p) of the
    threshold: the number of places where a computation with that much error
    could put the cut instead."""
    V = len(z)
    S = math.fsum(w.tolist())
    order = total_order(z)
    L_k = top_k if 1 <= top_k < V else V
    L_p, margin_p, near_p = V, math.inf, 0
    if top_p < 1.0:
        cum = np.cumsum(w[order].astype(np.longdouble))
        target = np.longdouble(top_p) * np.longdouble(S)
        n = int(np.searchsorted(cum, target, side="left")) + 1
        L_p = min(n, V)
        hi = float(cum[L_p - 1] - target)
        lo = float(target - cum[L_p - 2]) if L_p >= 2 else float(target)
        margin_p = min(abs(hi), abs(lo)) / S
        if band_p > 0.0:
            near_p = int(np.count_nonzero(np.abs(cum - target) <= np.longdouble(band_p * S)))
    L_m, margin_m, near_m = V, math.inf, 0
    if min_p > 0.0:
        L_m = int(np.count_nonzero(w >= float(min_p)))
        margin_m = float(np.min(np.abs(w - float(min_p)))) / float(min_p)
        if band_m > 0.0:
            near_m = int(np.count_nonzero(np.abs(w - float(min_p)) <= band_m * float(min_p)))
    L = max(1, min(L_k, L_p, L_m))
    return Cutoff(order, L, L_k, L_p, L_m, S, margin_p, margin_m, near_p, near_m)


def widen_ties(z: np.ndarray, order: np.ndarray, L: int) -> int:
    """The wide tie rule, the alternative the pages report for their device
    fallback selector (Arc PR #194, squashed commit #130, "hybrid nucleus
    selector": on tied supports it keeps every token sharing the boundary bit
    pattern, erring wider): the kept prefix of length L grows to every id whose
    value equals that of its last element, i.e. to all ids with z >= that value."""
    vb = z[order[L - 1]]
    return int(np.count_nonzero(z >= vb))


# --------------------------------------------------------------------------
# steps 9-10: inverse-CDF draw in token-id order
# --------------------------------------------------------------------------
def draw(kept_ids_sorted: np.ndarray, w_kept: np.ndarray, u) -> tuple:
    """Draw for one or many uniforms over a fixed kept set.

    ``kept_ids_sorted`` are the kept ids in increasing order, ``w_kept``
    their weights.  Returns (ids, margins) where margin = distance of t from
    the nearest edge of the chosen CDF interval, over S_K.
    """
    u = np.atleast_1d(np.asarray(u, dtype=np.float64))
    S_K = math.fsum(w_kept.tolist())
    C = np.cumsum(w_kept.astype(np.longdouble))
    t = u.astype(np.longdouble) * np.longdouble(S_K)
    pos = np.searchsorted(C, t, side="right")
    pos = np.minimum(pos, len(C) - 1)
    prev = np.where(pos > 0, C[np.maximum(pos - 1, 0)], np.longdouble(0))
    margin = np.minimum(t - prev, C[pos] - t).astype(np.float64) / S_K
    return kept_ids_sorted[pos], np.abs(margin)


# --------------------------------------------------------------------------
# the whole row
# --------------------------------------------------------------------------
@dataclasses.dataclass
class RowResult:
    status: int
    id: int
    greedy: bool = False
    argmax: int = -1
    max_logit: float = math.nan   # the penalised logit at argmax
    L: int = 0
    cut_value: float = math.nan
    cut_index: int = -1
    S: float = math.nan
    S_K: float = math.nan
    u: float = math.nan
    margin_id: float = math.inf
    margin_p: float = math.inf
    margin_m: float = math.inf
    near_p: int = 0
    near_m: int = 0
    L_k: int = 0
    L_p: int = 0
    L_m: int = 0
    kept: Optional[np.ndarray] = None     # kept ids, increasing
    probs: Optional[np.ndarray] = None    # q over the full vocabulary (float64)
    order: Optional[np.ndarray] = None    # the cutoff order (with probs), for kept sets of another size
    weights: Optional[np.ndarray] = None  # unnormalised weights w over the vocabulary (with probs)


def validate(p) -> int:
    T = float(p["temperature"])
    if math.isnan(T) or T < 0:
        return ROW_BAD_TEMPERATURE
    tp = float(p["top_p"])
    if math.isnan(tp) or tp <= 0:
        return ROW_BAD_TOP_P
    mp = float(p["min_p"])
    if math.isnan(mp) or mp < 0 or mp > 1:
        return ROW_BAD_MIN_P
    pres, freq, rep = float(p["presence"]), float(p["frequency"]), float(p["repetition"])
    if not (math.isfinite(pres) and math.isfinite(freq) and math.isfinite(rep)) or rep < 0:
        return ROW_BAD_PENALTY
    if int(p["flags"]) & ~ROW_TIES_WIDE:
        return ROW_BAD_FLAGS
    return ROW_OK


def sample_row(raw_row: np.ndarray, dtype: str, p, hist: Optional[np.ndarray], seed: int,
               row: int, step: int, u_override: Optional[float] = None,
               want_probs: bool = False, band_p: float = 0.0, band_m: float = 0.0,
               dry=None, breakers=()) -> RowResult:
    st = validate(p)
    if st == ROW_OK and dry is not None and hist is not None:
        st = dry_validate(dry)
    if st != ROW_OK:
        return RowResult(status=st, id=-1)
    z = widen(raw_row, dtype)
    z = penalize(z, hist, float(p["presence"]), float(p["frequency"]), float(p["repetition"]))
    z = dry_penalize(z, hist, dry, breakers)
    am = argmax_first(z)
    T = float(p["temperature"])
    top_k = int(p["top_k"])
    if T == 0.0 or top_k == 1 or z[am] == -np.inf:
        return RowResult(status=ROW_OK, id=am, greedy=True, argmax=am, max_logit=float(z[am]))
    _, w = weights(z, T)
    c = cutoff(z, w, top_k, float(p["top_p"]), float(p["min_p"]), band_p, band_m)
    if int(p["flags"]) & ROW_TIES_WIDE:
        c.L = widen_ties(z, c.order, c.L)
    kept = np.sort(c.order[: c.L])
    wk = w[kept]
    S_K = math.fsum(wk.tolist())
    u = uniform(seed, row, step) if u_override is None else float(u_override)
    ids, margins = draw(kept, wk, u)
    last = int(c.order[c.L - 1])
    res = RowResult(status=ROW_OK, id=int(ids[0]), argmax=am, max_logit=float(z[am]), L=c.L,
                    cut_value=float(z[last]),
                    cut_index=last, S=c.S, S_K=S_K, u=u, margin_id=float(margins[0]),
                    margin_p=c.margin_p, margin_m=c.margin_m, L_k=c.L_k, L_p=c.L_p, L_m=c.L_m,
                    kept=kept, near_p=c.near_p, near_m=c.near_m)
    if want_probs:
        q = np.zeros(len(z), dtype=np.float64)
        q[kept] = wk / S_K
        res.probs = q
        res.order = c.order
        res.weights = w
    return res


def sample(logits: np.ndarray, dtype: str, params: np.ndarray, hist_ids: Optional[np.ndarray],
           hist_offsets: Optional[np.ndarray], seed: int, step: int,
           rows: Optional[Sequence[int]] = None, uniforms: Optional[Sequence[float]] = None,
           want_probs: bool = False, band_p: float = 0.0, band_m: float = 0.0,
           dry: Optional[np.ndarray] = None, breakers=()) -> List[RowResult]:
    """Oracle over a batch.  ``rows`` are the batch indices that key the RNG."""
    n = logits.shape[0]
    rows = list(range(n)) if rows is None else [int(r) for r in rows]
    out = []
    for i in range(n):
        hist = None
        if hist_ids is not None and hist_offsets is not None:
            hist = hist_ids[int(hist_offsets[i]): int(hist_offsets[i + 1])]
        u = None if uniforms is None else float(uniforms[i])
        out.append(sample_row(logits[i], dtype, params[i], hist, seed, rows[i], step, u, want_probs,
                              band_p, band_m, None if dry is None else dry[i], breakers))
    return out


def hybrid_nucleus_row(raw_row: np.ndarray, dtype: str, T: float, top_p: float, budget: int, seed: int,
                       row: int, step: int, band_p: float = 0.0) -> RowResult:
    """The pages' baseline nucleus selector (Arc PR #194, squashed commit #130,
    "hybrid nucleus selector"): enumerating the order until the mass reaches
    top_p keeps the strict prefix, and does so when that prefix has at most
    `budget` ids; past the budget, threshold bisection over the values keeps
    every id at or above the crossing value, i.e. the prefix widened to its
    ties.  No penalties, top-k or min-p; T must be finite and > 0, top_p > 0."""
    T = float(T)
    top_p = float(top_p)
    if not (T > 0.0 and math.isfinite(T)):
        return RowResult(status=ROW_BAD_TEMPERATURE, id=-1)
    if not (top_p > 0.0):
        return RowResult(status=ROW_BAD_TOP_P, id=-1)
    z = widen(raw_row, dtype)
    _, w = weights(z, T)
    c = cutoff(z, w, -1, top_p, 0.0, band_p)
    L = c.L
    if top_p < 1.0 and L > budget:
        L = widen_ties(z, c.order, L)
    kept = np.sort(c.order[:L])
    wk = w[kept]
    u = uniform(seed, row, step)
    ids, margins = draw(kept, wk, u)
    return RowResult(status=ROW_OK, id=int(ids[0]), L=L, S=c.S, S_K=math.fsum(wk.tolist()), u=u,
                     margin_id=float(margins[0]), margin_p=c.margin_p, near_p=c.near_p, kept=kept)


def argmax(logits: np.ndarray, dtype: str) -> np.ndarray:
    """Row-wise argmax of the widened raw logits (no penalties)."""
    return np.array([argmax_first(widen(r, dtype)) for r in logits], dtype=np.int32)


# --------------------------------------------------------------------------
# top-n log-probabilities (the response feature next to the draw)
# --------------------------------------------------------------------------
@dataclasses.dataclass
class TopLogprobs:
    status: int
    ids: np.ndarray        # int64 [n]
    logprobs: np.ndarray   # float64 [n]


def top_logprobs_row(raw_row: np.ndarray, dtype: str, T: float, n: int) -> TopLogprobs:
    """The n most probable ids of a row and their log-probabilities.

    Arc PR #222, section 3(c): next to the draw, the host sampler reports the
    most probable tokens with their log-probabilities, found by a partial sort
    of the probabilities.  Reading taken here: the distribution is that of the
    widened logits at temperature T (no penalties, no filters), so with
    m = max z and S = sum of w (step 5 above, math.fsum),
    logprob_v = (z_v - m) / T - ln S, and 0 - ln S where z_v == m (which covers
    +inf logits and a row of -inf, then uniform).  The ids are the first n of
    the total order (step 4); a row shorter than n ends with id -1 and -inf.
    T must be finite and > 0, else the row's status is ROW_BAD_TEMPERATURE
    (ids -1, logprobs NaN).
    """
    if not (T > 0.0 and math.isfinite(T)):
        return TopLogprobs(ROW_BAD_TEMPERATURE, np.full(n, -1, np.int64), np.full(n, np.nan))
    z = widen(raw_row, dtype)
    m, w = weights(z, T)
    lnS = math.log(math.fsum(w.tolist()))
    order = total_order(z)[:n]
    ids = np.full(n, -1, np.int64)
    lps = np.full(n, -np.inf)
    for r, v in enumerate(order):
        zv = float(z[v])
        lw = 0.0 if zv == m else (zv - m) / T
        ids[r] = int(v)
        lps[r] = lw - lnS
    return TopLogprobs(ROW_OK, ids, lps)


def top_logprobs(logits: np.ndarray, dtype: str, temperature: Optional[Sequence[float]], n: int):
    """Oracle over a batch: (ids [B, n] int64, logprobs [B, n] float64, status [B])."""
    B = logits.shape[0]
    ids = np.empty((B, n), np.int64)
    lps = np.empty((B, n), np.float64)
    st = np.empty(B, np.int32)
    for b in range(B):
        T = 1.0 if temperature is None else float(temperature[b])
        r = top_logprobs_row(logits[b], dtype, T, n)
        ids[b], lps[b], st[b] = r.ids, r.logprobs, r.status
    return ids, lps, st
