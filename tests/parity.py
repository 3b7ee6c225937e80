"""Comparison rules between the HIP path and the oracle (test helpers).

Masks: a GPU kept set is accepted when it is a valid answer of the same rule
up to a score gap of 1e-4, measured on the oracle's float64 values:
  * top-k: forced blocks kept, k blocks in total, and every dropped non-forced
    score at most 1e-4 above the lowest kept non-forced score (pooled logits);
  * CDF: the set is a top-n set in that sense, with n a valid count for some
    prefix whose cumulative pooled mass lies within 1e-4 of tau;
  * drift: the initial set is a top-k set by drift score up to a relative gap
    of 1e-4, and every logged swap is optimal, and every stop justified, up to
    a relative 1e-4 in J (2e-4 in J^2) when replayed on the oracle's
    contributions, under the objective the selection used (for the renormalised
    one with an absolute allowance for float32 rounding, see drift_valid);
  * drift by re-rank rounds: the initial set and every logged round's set are
    top-k sets of their scores up to a gap of 1e-4 of the largest |score|, and
    the returned set is the last one or, with track-best, one of least J up to
    a relative 2e-4 (see rerank_valid).
Outputs: fp32 max |O - O_ref| <= 1e-3; bf16 max_d |O - O_ref| <= 2e-2 * RMS_d(O_ref)
for every real query row (see output_check).
"""
from __future__ import annotations

from typing import List, Sequence

import numpy as np

import oracle

GAP = 1e-4
TOL_F32 = 1e-3
TOL_BF16_REL_RMS = 2e-2


def csr_rows(row_ptr: np.ndarray, col_idx: np.ndarray) -> List[List[int]]:
    rp = np.asarray(row_ptr, dtype=np.int64)
    ci = np.asarray(col_idx, dtype=np.int64)
    return [ci[rp[r]:rp[r + 1]].tolist() for r in range(len(rp) - 1)]


def check_csr_wellformed(row_ptr: np.ndarray, col_idx: np.ndarray, nb: int):
    rp = np.asarray(row_ptr, dtype=np.int64)
    assert rp[0] == 0 and np.all(np.diff(rp) >= 0), "row_ptr not monotone from 0"
    for r in range(len(rp) - 1):
        row = np.asarray(col_idx[rp[r]:rp[r + 1]], dtype=np.int64)
        assert np.all((row >= 0) & (row < nb)), f"row {r}: index out of range"
        assert np.all(np.diff(row) > 0), f"row {r}: not strictly ascending"


def topk_valid(kept: Sequence[int], score_row: np.ndarray, k: int, forced: Sequence[int],
               gap: float = GAP) -> bool:
    ks = set(kept)
    if len(ks) != k or len(kept) != k or not set(forced) <= ks:
        return False
    nonforced_kept = [score_row[j] for j in ks if j not in set(forced)]
    dropped = [score_row[j] for j in range(len(score_row)) if j not in ks]
    if not nonforced_kept or not dropped:
        return True
    return max(dropped) <= min(nonforced_kept) + gap


def cdf_valid(kept: Sequence[int], score_row: np.ndarray, p_row: np.ndarray, tau: float,
              cap: int, forced: Sequence[int], gap: float = GAP) -> bool:
    n = len(kept)
    if not topk_valid(kept, score_row, n, forced, gap):
        return False
    order = oracle.priority_order(score_row, forced)
    cum = np.concatenate([[0.0], np.cumsum(p_row[order])])
    nb = len(score_row)
    allowed = set()
    for n_prime in range(1, nb + 1):
        ok_reach = cum[n_prime] >= tau - gap or n_prime == nb
        ok_first = cum[n_prime - 1] < tau + gap
        if ok_reach and ok_first:
            allowed.add(max(len(forced), min(n_prime, cap), 1))
    return n in allowed


def drift_valid(kept_final: Sequence[int], swaps: np.ndarray, chat: np.ndarray, k: int,
                forced: Sequence[int], gap: float = GAP, zhat=None, floor: float = 0.0) -> tuple:
    """Replays the GPU's swap log on the oracle's contributions.

    zhat None: the dropped-sum objective J(S) = ||sum_{j not in S} chat_j||.
    zhat given: the renormalised objective J(S) = ||sum_S chat_j / sum_S zhat_j -
    sum_j chat_j||. Comparisons of J^2 allow a relative 2*gap plus `floor` (an
    absolute allowance in J^2 for the float32 rounding of the kernel's update
    rule, which works with differences of squared norms).
    Returns (ok, reason, replayed final J).
    """
    nb = chat.shape[0]
    fset = set(forced)
    d = np.sqrt((chat * chat).sum(axis=1))
    obar = chat.sum(axis=0)
    # the initial set: final set with the logged swaps undone, newest first
    init = set(kept_final)
    for a, b in reversed([tuple(s) for s in swaps if s[0] >= 0]):
        if a not in init or b in init:
            return False, "swap log inconsistent with the final set", None
        init.remove(a)
        init.add(b)
    nf_kept = [d[j] for j in init if j not in fset]
    dropped = [d[j] for j in range(nb) if j not in init]
    if len(init) != k or not fset <= init:
        return False, "initial set has the wrong size or misses a forced block", None
    if nf_kept and dropped and max(dropped) > min(nf_kept) * (1 + gap):
        return False, "initial set is not the top-k by drift score", None

    def j2_of(cur):
        """J^2 of the kept set cur."""
        if zhat is None:
            r = chat[sorted(set(range(nb)) - cur)].sum(axis=0)
            return float(r @ r)
        return oracle.drift_j_renorm(chat, zhat, sorted(cur)) ** 2

    def j2_swaps(cur, drop, cand_b):
        """J^2 after each swap, [len(drop), len(cand_b)]."""
        if zhat is None:
            r = chat[drop].sum(axis=0)
            trial = r[None, None, :] - chat[drop][:, None, :] + chat[cand_b][None, :, :]
            return (trial * trial).sum(axis=-1)
        S = sorted(cur)
        cs, zs = chat[S].sum(axis=0), float(zhat[S].sum())
        c2 = cs[None, None, :] + chat[drop][:, None, :] - chat[cand_b][None, :, :]
        z2 = zs + zhat[drop][:, None] - zhat[cand_b][None, :]
        with np.errstate(divide="ignore", invalid="ignore"):
            u = c2 / z2[:, :, None] - obar[None, None, :]
            return np.where(z2 > 0, (u * u).sum(axis=-1), np.inf)

    cur = set(init)
    for s in swaps:
        a, b = int(s[0]), int(s[1])
        drop = sorted(set(range(nb)) - cur)
        cand_b = sorted(cur - fset)
        rr = j2_of(cur)
        trial = j2_swaps(cur, drop, cand_b) if drop and cand_b else None
        best = float(trial.min()) if trial is not None else np.inf
        if a < 0:
            if best < rr * (1 - 2 * gap) - floor:
                return False, "stopped although a swap lowers J", None
            break
        if trial is None:
            return False, "swap logged with nothing to swap", None
        if a in cur or b not in cur or b in fset:
            return False, "swap does not move a dropped block in and a kept block out", None
        j2 = float(trial[drop.index(a), cand_b.index(b)])
        if j2 > best * (1 + 2 * gap) + floor + 1e-30:
            return False, f"swap not optimal: {j2} vs best {best}", None
        if j2 > rr * (1 + 2 * gap) + floor:
            return False, "swap raises J", None
        cur.remove(b)
        cur.add(a)
    if cur != set(kept_final):
        return False, "replay does not reach the final set", None
    if zhat is None:
        return True, "", oracle.drift_j(chat, sorted(cur))
    return True, "", oracle.drift_j_renorm(chat, zhat, sorted(cur))


def output_error(o_gpu: np.ndarray, o_ref: np.ndarray, valid: np.ndarray):
    """(max abs error, RMS of the reference) over real query rows."""
    g = np.asarray(o_gpu, dtype=np.float64)[..., valid, :]
    r = np.asarray(o_ref, dtype=np.float64)[..., valid, :]
    return float(np.abs(g - r).max()), float(np.sqrt((r * r).mean()))


def output_check(o_gpu: np.ndarray, o_ref: np.ndarray, valid: np.ndarray, dtype: str):
    """Applies the output tolerance; returns (ok, worst error / allowance, max abs error).

    fp32: max |O - O_ref| <= 1e-3 over real query rows.
    bf16: for every real query row t, max_d |O[t,d] - O_ref[t,d]| <= 2e-2 * RMS_d(O_ref[t,:]).
    The relative bound is taken per output row: storing a bf16 output alone moves an
    element by up to 2^-9 of its magnitude, i.e. up to 2^-9 * 8 = 1.6 % of its row RMS
    at head_dim 64, while one global RMS over rows of very different magnitude would be
    exceeded by that rounding alone wherever max|O| > 10 * RMS.
    """
    g = np.asarray(o_gpu, dtype=np.float64)[..., valid, :]
    r = np.asarray(o_ref, dtype=np.float64)[..., valid, :]
    err = np.abs(g - r)
    if dtype == "f32":
        worst = float(err.max()) / TOL_F32
    else:
        allow = TOL_BF16_REL_RMS * np.sqrt((r * r).mean(axis=-1))
        worst = float((err.max(axis=-1) / np.maximum(allow, 1e-300)).max())
        worst = 0.0 if not np.isfinite(worst) and float(err.max()) == 0 else worst
    return worst <= 1.0, worst, float(err.max())


def mask_words_to_set(words, nb: int):
    """Kept blocks of a bitmask row (bit j % 32 of word j // 32)."""
    w = np.asarray(words, dtype=np.int64) & 0xFFFFFFFF
    return [j for j in range(nb) if (w[j >> 5] >> (j & 31)) & 1]


def rerank_valid(sets, final, chat: np.ndarray, k: int, forced: Sequence[int], track_best: bool,
                 gap: float = GAP) -> tuple:
    """Checks a GPU re-rank run, given the kept set it logged for the initial
    selection and every round, and the set it returned, on the oracle's
    contributions: the initial set is a top-k by drift score and each round's
    set a top-k by the round's scores against the previous logged set, both up
    to a relative gap; the returned set is the last one, or with track-best one
    of least J up to a relative 2 * gap. Returns (ok, reason)."""
    nb = chat.shape[0]
    fset = set(forced)
    d2 = (chat * chat).sum(axis=1)

    def topk_ok(s, score):
        s = set(s)
        if len(s) != k or not fset <= s:
            return False
        kept_nf = [score[j] for j in s if j not in fset]
        dropped = [score[j] for j in range(nb) if j not in s]
        if not kept_nf or not dropped:
            return True
        return max(dropped) <= min(kept_nf) + gap * float(np.abs(score).max())

    if not topk_ok(sets[0], d2):
        return False, "initial set is not the top-k by drift score"
    for x in range(1, len(sets)):
        prev = set(sets[x - 1])
        drop = [j for j in range(nb) if j not in prev]
        r = chat[drop].sum(axis=0) if drop else np.zeros(chat.shape[1])
        g = np.array([2.0 * float(r @ chat[j]) + (d2[j] if j in prev else -d2[j])
                      for j in range(nb)])
        if not topk_ok(sets[x], g):
            return False, f"round {x} is not the top-k of its scores"
    js = [oracle.drift_j(chat, s) for s in sets]
    if not track_best:
        return (list(final) == list(sets[-1])), "returned set is not the last round's"
    if list(final) not in [list(s) for s in sets]:
        return False, "returned set is not one of the logged sets"
    if oracle.drift_j(chat, final) > min(js) * (1 + 2 * gap) + 1e-30:
        return False, "returned set is not of least J"
    return True, ""
