"""Pins of the oracle's drift contributions and residual restoration (no GPU)."""
import itertools
import math
import types

import numpy as np
import pytest
import torch

import oracle


def layout(frames=2, frame_len=8, frame_valid=6, block=4, D=4, heads=1, scale=0.5):
    return types.SimpleNamespace(batch=1, heads=heads, head_dim=D, frames=frames,
                                 frame_len=frame_len, frame_valid=frame_valid,
                                 block=block, scale=scale)


def rand_kv(lay, seed):
    rng = np.random.default_rng(seed)
    N = lay.frames * lay.frame_len
    k = rng.standard_normal((N, lay.head_dim))
    v = rng.standard_normal((N, lay.head_dim))
    pad = (np.arange(N) % lay.frame_len) >= lay.frame_valid
    k[pad] = 0
    v[pad] = 0
    return k, v


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_contributions_sum_to_dense_attention_of_pooled_query(seed):
    lay = layout(frames=3, frame_len=8, frame_valid=6, block=4, D=5, scale=0.8)
    k, v = rand_kv(lay, seed)
    qbar = np.random.default_rng(10 + seed).standard_normal(5)
    chat, z, Z = oracle.drift_row(qbar, k, v, lay)
    valid = oracle.valid_mask(lay)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qbar)[None, None, None], torch.from_numpy(k[valid])[None, None],
        torch.from_numpy(v[valid])[None, None], scale=0.8)[0, 0, 0].numpy()
    np.testing.assert_allclose(chat.sum(axis=0), ref, atol=1e-13)
    assert z.sum() / Z == pytest.approx(1.0, abs=1e-14)
    # each block's share, token by token with math.exp (shift-free form)
    for j in range(oracle.num_blocks(lay)):
        toks = [u for u in range(4 * j, 4 * j + 4) if valid[u]]
        allv = [u for u in range(len(valid)) if valid[u]]
        w = {u: math.exp(0.8 * float(qbar @ k[u])) for u in allv}
        tot = sum(w.values())
        for d in range(5):
            assert chat[j, d] == pytest.approx(sum(w[u] * v[u, d] for u in toks) / tot, abs=1e-13)


def test_single_block_contribution_is_attention_output():
    lay = layout(frames=1, frame_len=8, frame_valid=8, block=8, D=4)
    k, v = rand_kv(lay, 3)
    qbar = np.ones(4) * 0.3
    chat, z, Z = oracle.drift_row(qbar, k, v, lay)
    o, _ = oracle.attention_rows(qbar[None], k, v, lay.scale)
    np.testing.assert_allclose(chat[0], o[0], atol=1e-14)


def _exhaustive_best_j(chat, k, forced=()):
    nb = chat.shape[0]
    best = math.inf
    for cand in itertools.combinations(range(nb), k):
        if not set(forced) <= set(cand):
            continue
        best = min(best, oracle.drift_j(chat, cand))
    return best


@pytest.mark.parametrize("seed", range(8))
def test_restoration_invariants(seed):
    rng = np.random.default_rng(seed)
    nb = int(rng.integers(4, 11))
    D = int(rng.integers(2, 6))
    chat = rng.standard_normal((nb, D))
    k = int(rng.integers(1, nb))
    forced = sorted(rng.choice(nb, size=int(rng.integers(0, k)), replace=False).tolist())
    # rounds = 0: initial set = forced + largest norms
    kept0, j0, sw0 = oracle.restore_row(chat, k, 0, forced)
    norms = np.linalg.norm(chat, axis=1)
    rest = sorted((j for j in range(nb) if j not in forced), key=lambda j: (-norms[j], j))
    assert kept0 == sorted(forced + rest[:k - len(forced)]) and sw0 == []
    prev_j, prev_kept = j0, kept0
    for rounds in range(1, 30):
        kept, j, swaps = oracle.restore_row(chat, k, rounds, forced)
        assert len(kept) == k and set(forced) <= set(kept)
        assert j <= prev_j + 1e-15                       # drift never grows
        assert j == pytest.approx(oracle.drift_j(chat, kept), abs=1e-14)
        assert len(swaps) <= rounds
        for a, b in swaps:
            assert b not in forced
        prev_j, prev_kept = j, kept
    # converged: no single swap lowers J
    drop = [x for x in range(nb) if x not in prev_kept]
    for a in drop:
        for b in prev_kept:
            if b in forced:
                continue
            trial = sorted(set(prev_kept) - {b} | {a})
            assert oracle.drift_j(chat, trial) >= prev_j - 1e-12
    assert prev_j >= _exhaustive_best_j(chat, k, forced) - 1e-12


def test_restoration_is_a_local_single_swap_search():
    """Closed form: kept {0,1,2}, drop {3,4}, r = (0.5,1.5), J^2 = 2.5. Round 1:
    restoring 4 and dropping 2 gives r = (1,1), J^2 = 2 (the other five swaps give
    30.5, 20.61, 2.5, 26, 26.21). Round 2 from r = (1,1): the swaps give 26, 26.21,
    2.5, 36, 16.01, 2.5, none below 2, so the search stops at J = sqrt 2 although
    dropping the opposite pair {0,1} would give J = 0.1: one swap per round cannot
    move both."""
    chat = np.array([[5.0, 0.0], [-5.0, 0.1], [1.0, 0.0], [0.0, 1.0], [0.5, 0.5]])
    kept0, j0, _ = oracle.restore_row(chat, 3, 0)
    assert kept0 == [0, 1, 2] and j0 == pytest.approx(math.sqrt(2.5), abs=1e-15)
    kept, j, swaps = oracle.restore_row(chat, 3, 3)
    assert swaps == [(4, 2)] and kept == [0, 1, 4]
    assert j == pytest.approx(math.sqrt(2.0), abs=1e-15)
    assert _exhaustive_best_j(chat, 3) == pytest.approx(0.1, abs=1e-15)


def test_swap_ties_prefer_lower_indices():
    chat = np.array([[2.0, 0.0], [2.0, 0.0], [-1.0, 0.0], [-1.0, 0.0]])
    # kept {0,1}; drop {2,3}, r = (-2,0). Restore 2 or 3 (same vector), drop 0 or 1
    # (same vector): every swap gives r = (-2+1+2, 0) = (1,0), J^2 = 1 < 4.
    kept, j, swaps = oracle.restore_row(chat, 2, 1)
    assert swaps == [(2, 0)] and kept == [1, 2]


def test_drift_selection_planted_block():
    """A key block that carries nearly all of the pooled query's attention has
    the largest contribution and is kept."""
    lay = layout(frames=2, frame_len=8, frame_valid=8, block=4, D=8, scale=1.0)
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, 16, 8)) * 0.1
    k = rng.standard_normal((1, 1, 16, 8)) * 0.1
    v = rng.standard_normal((1, 1, 16, 8))
    q[0, 0, 0:4, 2] += 3.0
    k[0, 0, 8:12, 2] += 3.0
    sets, stat = oracle.select(q, k, v, lay, oracle.DRIFT, [1], rounds=3)
    assert sets[0][0][0] == [2]


def _output_shift_by_attention(qbar, k, v, lay, kept):
    """The renormalised drift written as two attention computations: the pooled
    query attending to the real keys of the kept blocks only, minus the same
    query attending densely (oracle.attention_rows, a separate code path)."""
    valid = oracle.valid_mask(lay)
    keys = np.concatenate([oracle.block_tokens(lay, j) for j in sorted(kept)])
    o_s, _ = oracle.attention_rows(qbar[None], k[keys], v[keys], lay.scale)
    o_d, _ = oracle.attention_rows(qbar[None], k[valid], v[valid], lay.scale)
    return float(np.sqrt(((o_s[0] - o_d[0]) ** 2).sum()))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_renormalised_drift_is_the_output_shift(seed):
    lay = layout(frames=3, frame_len=8, frame_valid=6, block=4, D=5, scale=0.8)
    k, v = rand_kv(lay, 20 + seed)
    qbar = np.random.default_rng(30 + seed).standard_normal(5)
    chat, z, Z = oracle.drift_row(qbar, k, v, lay)
    nb = oracle.num_blocks(lay)
    rng = np.random.default_rng(40 + seed)
    for _ in range(5):
        kept = sorted(rng.choice(nb, size=int(rng.integers(1, nb + 1)), replace=False).tolist())
        assert oracle.drift_j_renorm(chat, z / Z, kept) == pytest.approx(
            _output_shift_by_attention(qbar, k, v, lay, kept), rel=1e-10, abs=1e-13)
    assert oracle.drift_j_renorm(chat, z / Z, list(range(nb))) == pytest.approx(0.0, abs=1e-14)


@pytest.mark.parametrize("seed,force,swapped", [(1, False, True), (3, True, True), (6, False, True),
                                               (0, False, False)])
def test_renormalised_restoration_takes_the_best_swap(seed, force, swapped):
    """Every round's swap is the best single swap by the output shift computed
    with attention_rows, every stop is justified, and J never rises."""
    lay = layout(frames=3, frame_len=8, frame_valid=6, block=2, D=4, scale=0.9)
    k, v = rand_kv(lay, 50 + seed)
    qbar = np.random.default_rng(60 + seed).standard_normal(4) * 1.5
    chat, z, Z = oracle.drift_row(qbar, k, v, lay)
    nb = oracle.num_blocks(lay)
    forced = oracle.forced_blocks(lay, force)
    kbudget = 5
    kept, j_final, swaps = oracle.restore_row_renorm(chat, z / Z, kbudget, 6, forced)
    d = np.sqrt((chat * chat).sum(axis=1))
    # replay: each logged swap is the best one and lowers J; the stop is justified
    cur = set(oracle.priority_order(d, forced)[:kbudget])
    j_cur = _output_shift_by_attention(qbar, k, v, lay, cur)
    for a, b in swaps:
        cands = [(aa, bb) for aa in sorted(set(range(nb)) - cur) for bb in sorted(cur - set(forced))]
        scored = sorted((_output_shift_by_attention(qbar, k, v, lay, (cur - {bb}) | {aa}), aa, bb)
                        for aa, bb in cands)
        assert (scored[0][1], scored[0][2]) == (a, b) or scored[0][0] == pytest.approx(
            _output_shift_by_attention(qbar, k, v, lay, (cur - {b}) | {a}), rel=1e-12)
        j_new = _output_shift_by_attention(qbar, k, v, lay, (cur - {b}) | {a})
        assert j_new < j_cur
        cur = (cur - {b}) | {a}
        j_cur = j_new
    if len(swaps) < 6:
        cands = [(aa, bb) for aa in sorted(set(range(nb)) - cur) for bb in sorted(cur - set(forced))]
        assert all(_output_shift_by_attention(qbar, k, v, lay, (cur - {bb}) | {aa}) >= j_cur * (1 - 1e-12)
                   for aa, bb in cands)
    assert sorted(cur) == kept
    assert j_final == pytest.approx(j_cur, rel=1e-10)
    assert (len(swaps) >= 1) == swapped


# --------------------------------------------------------------------------
# re-rank rounds with and without track-best (ReSS abstract and Fig. 3(c):
# the drop set is refined as a whole; Table S3: keeping the best set seen)
# --------------------------------------------------------------------------
PLANTED_RERANK = np.array([[-2.0, 0.0], [-2.0, -2.0], [2.0, -3.0], [-3.0, 3.0]])


def test_rerank_planted_row_rises_and_track_best_keeps_the_best_set():
    """Four 2-d contributions, keep 2. Squared norms 4, 8, 13, 18, so the
    initial set is {2, 3}, D = {0, 1}, r = (-4, -2), J^2 = 20.
    Round 1, g_j = ||r_j + c_j||^2 - ||r_j||^2: g0 = 20 - |(-2,-2)|^2 = 12,
    g1 = 20 - |(-2,0)|^2 = 16, g2 = |(-2,-5)|^2 - 20 = 9, g3 = |(-7,1)|^2 - 20 =
    30 -> keep {1, 3}, r = (0, -3), J^2 = 9.
    Round 2: g0 = 9 - |(2,-3)|^2 = -4, g2 = 9 - |(-2,0)|^2 = 5,
    g1 = |(-2,-5)|^2 - 9 = 20, g3 = |(-3,0)|^2 - 9 = 0 -> keep {1, 2},
    r = (-5, 3), J^2 = 34: J rises.
    Round 3: g0 = 34 - |(-3,3)|^2 = 16, g3 = 34 - |(-2,0)|^2 = 30,
    g1 = |(-7,1)|^2 - 34 = 16, g2 = |(-3,0)|^2 - 34 = -25 -> 3, then the tie
    g0 = g1 = 16 goes to block 0: keep {0, 3}, r = (0, -5), J^2 = 25."""
    kept, j, sets, js = oracle.rerank_row(PLANTED_RERANK, 2, 3, track_best=False)
    assert sets == [[2, 3], [1, 3], [1, 2], [0, 3]]
    np.testing.assert_allclose(np.square(js), [20.0, 9.0, 34.0, 25.0], rtol=0, atol=1e-12)
    assert kept == [0, 3] and j == pytest.approx(5.0, abs=1e-12)
    kept_b, j_b, sets_b, _ = oracle.rerank_row(PLANTED_RERANK, 2, 3, track_best=True)
    assert sets_b == sets and kept_b == [1, 3] and j_b == pytest.approx(3.0, abs=1e-12)
    # the exhaustive optimum (keep {0, 1}: r = (-1, 0)) is below both
    best = min(oracle.drift_j(PLANTED_RERANK, list(c)) for c in itertools.combinations(range(4), 2))
    assert best == pytest.approx(1.0, abs=1e-12)
    # and the single best-swap restoration of the same row reaches it in two rounds:
    # (1, 2) to J^2 = 9, then (0, 3) to J^2 = 1
    kept_s, j_s, swaps = oracle.restore_row(PLANTED_RERANK, 2, 3)
    assert swaps == [(1, 2), (0, 3)] and kept_s == [0, 1] and j_s == pytest.approx(1.0, abs=1e-12)


def rerank_scores_by_set_sums(chat, kept):
    """Each block's score as two drift values computed from whole sets: J^2 of the
    drop set with the block added, minus J^2 of the drop set without it."""
    nb = chat.shape[0]
    g = []
    for j in range(nb):
        drop_without = [x for x in range(nb) if x not in kept and x != j]
        with_j = drop_without + [j]
        jw = oracle.drift_j(chat, [x for x in range(nb) if x not in with_j]) ** 2
        jo = oracle.drift_j(chat, [x for x in range(nb) if x not in drop_without]) ** 2
        g.append(jw - jo)
    return np.array(g)


@pytest.mark.parametrize("seed,nb,k,forced", [(0, 7, 3, ()), (1, 9, 4, (2,)), (2, 10, 5, (0, 5)),
                                                (3, 8, 2, ())])
def test_rerank_rounds_exhaustive(seed, nb, k, forced):
    """Small rows: every round's set is the forced blocks plus the top scores
    computed from whole-set drift values; the track-best J is the least J of the
    trace, never above the initial J and never below the exhaustive optimum
    over all k-sets that hold the forced blocks."""
    rng = np.random.default_rng(300 + seed)
    chat = rng.standard_normal((nb, 3)) * rng.uniform(0.2, 2.0, (nb, 1))
    rounds = 6
    kept, j, sets, js = oracle.rerank_row(chat, k, rounds, forced, track_best=True)
    for x in range(1, len(sets)):
        g = rerank_scores_by_set_sums(chat, set(sets[x - 1]))
        rest = sorted((j2 for j2 in range(nb) if j2 not in forced), key=lambda j2: (-g[j2], j2))
        assert sets[x] == sorted(list(forced) + rest[:k - len(forced)]), x
    for x, sx in enumerate(sets):
        assert len(sx) == k and set(forced) <= set(sx)
        assert js[x] == pytest.approx(oracle.drift_j(chat, sx), abs=1e-12)
    assert j == pytest.approx(min(js), abs=1e-15) and j <= js[0] + 1e-15
    opt = min(oracle.drift_j(chat, list(c)) for c in itertools.combinations(range(nb), k)
              if set(forced) <= set(c))
    assert j >= opt - 1e-12
    kept_n, j_n, _, js_n = oracle.rerank_row(chat, k, rounds, forced, track_best=False)
    assert js_n == js and kept_n == sets[-1]


def test_rerank_zero_rounds_is_the_initial_drift_set():
    rng = np.random.default_rng(7)
    chat = rng.standard_normal((12, 4))
    for forced in ((), (3, 8)):
        kept, j, sets, js = oracle.rerank_row(chat, 5, 0, forced)
        k0, j0, _ = oracle.restore_row(chat, 5, 0, forced)
        assert kept == k0 and sets == [k0] and j == pytest.approx(j0, abs=1e-15)


def test_rerank_fixed_point_stays():
    """A set that a round leaves unchanged stays for every later round."""
    chat = np.array([[5.0, 0.0], [0.0, 4.0], [0.1, 0.0], [0.0, -0.1]])
    kept, j, sets, js = oracle.rerank_row(chat, 2, 4)
    assert all(sx == [0, 1] for sx in sets) and len(set(js)) == 1


def test_expanded_round_score_needs_no_contributions():
    """The identity the expanded re-rank rests on: for any residual r,
    <r, c_ij> = sum_{u in block j} w_iu <v_u, r> with w_iu the pooled query's
    softmax weights over the real keys, so a round's scores can be formed from
    Q, K and V without the contributions."""
    lay = layout(frames=3, frame_len=32, frame_valid=27, block=8, D=16, scale=0.25)
    rng = np.random.default_rng(5)
    ntok = lay.frames * lay.frame_len
    q, k, v = (rng.standard_normal((1, 1, ntok, 16)) for _ in range(3))
    pad = (np.arange(ntok) % lay.frame_len) >= lay.frame_valid
    for a in (q, k, v):
        a[:, :, pad] = 0
    qbar = oracle.pool(q, lay)[0, 0]
    nb = ntok // lay.block
    real = np.flatnonzero(~pad)
    for i in (0, 5, nb - 1):
        chat, _, _ = oracle.drift_row(qbar[i], k[0, 0], v[0, 0], lay)
        logits = lay.scale * (k[0, 0, real] @ qbar[i])
        w = np.exp(logits - logits.max())
        w /= w.sum()
        r = rng.standard_normal(16)
        vr = v[0, 0, real] @ r
        blk = real // lay.block
        for j in range(nb):
            lhs = float(r @ chat[j])
            rhs = float(np.sum(w[blk == j] * vr[blk == j]))
            assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs)), (i, j, lhs, rhs)
