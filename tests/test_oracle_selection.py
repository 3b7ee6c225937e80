"""Pins of the oracle's pooling, pooled scores and budgeted selection (no GPU)."""
import itertools
import math
import types

import numpy as np
import pytest

import oracle


def layout(frames=2, frame_len=8, frame_valid=6, block=4, D=4, heads=1, scale=0.5):
    return types.SimpleNamespace(batch=1, heads=heads, head_dim=D, frames=frames,
                                 frame_len=frame_len, frame_valid=frame_valid,
                                 block=block, scale=scale)


def test_pool_is_mean_over_real_tokens_loop():
    lay = layout(frames=2, frame_len=8, frame_valid=5, block=4, D=3)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((1, 1, 16, 3))
    x[0, 0, np.arange(16) % 8 >= 5] = 7.0        # padding must not enter the mean
    got = oracle.pool(x, lay)[0, 0]
    for j in range(4):
        toks = [t for t in range(4 * j, 4 * j + 4) if t % 8 < 5]
        for d in range(3):
            assert got[j, d] == pytest.approx(sum(x[0, 0, t, d] for t in toks) / len(toks), abs=1e-15)


def test_pooled_scores_orientation_loop():
    rng = np.random.default_rng(1)
    qb, kb = rng.standard_normal((1, 1, 3, 5)), rng.standard_normal((1, 1, 4, 5))
    s = oracle.pooled_scores(qb, kb, 0.25)[0, 0]
    assert s.shape == (3, 4)
    for i in range(3):
        for j in range(4):
            assert s[i, j] == pytest.approx(0.25 * sum(qb[0, 0, i, d] * kb[0, 0, j, d] for d in range(5)), abs=1e-14)


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force(seed):
    rng = np.random.default_rng(seed)
    nb = int(rng.integers(4, 12))
    row = rng.standard_normal(nb)
    k = int(rng.integers(1, nb + 1))
    forced = sorted(rng.choice(nb, size=int(rng.integers(0, k + 1)), replace=False).tolist())
    kept = oracle.select_topk_row(row, k, forced)
    best = None
    for cand in itertools.combinations(range(nb), k):
        if not set(forced) <= set(cand):
            continue
        total = sum(row[j] for j in cand)
        if best is None or total > best[0] + 1e-12:
            best = (total, list(cand))
    assert kept == best[1]


def test_topk_ties_go_to_lower_index():
    row = np.array([1.0, 2.0, 2.0, 0.5, 2.0, 2.0])
    assert oracle.select_topk_row(row, 2) == [1, 2]
    assert oracle.select_topk_row(row, 3, forced=[3]) == [1, 2, 3]
    assert oracle.select_topk_row(np.zeros(5), 2) == [0, 1]


def test_forced_more_than_budget_raises():
    with pytest.raises(ValueError):
        oracle.select_topk_row(np.zeros(4), 1, forced=[0, 2])


def test_forced_blocks_are_frame_first_blocks():
    lay = layout(frames=3, frame_len=8, frame_valid=6, block=4)
    assert oracle.forced_blocks(lay, True) == [0, 2, 4]
    assert oracle.forced_blocks(lay, False) == []


def test_block_of_one_token_is_token_level_topk_attention():
    """With block = 1 the method is per-token top-k attention; written here
    token by token with plain loops."""
    lay = layout(frames=1, frame_len=12, frame_valid=12, block=1, D=4, scale=0.7)
    rng = np.random.default_rng(2)
    q, k, v = (rng.standard_normal((1, 1, 12, 4)) for _ in range(3))
    kk = 5
    sets, _ = oracle.select(q, k, v, lay, oracle.TOPK, [kk])
    o, _ = oracle.sparse_attention(q, k, v, lay, *oracle.csr(sets))
    for t in range(12):
        s = [0.7 * sum(q[0, 0, t, d] * k[0, 0, u, d] for d in range(4)) for u in range(12)]
        top = sorted(range(12), key=lambda u: (-s[u], u))[:kk]
        assert sorted(top) == sets[0][0][t]
        m = max(s[u] for u in top)
        w = {u: math.exp(s[u] - m) for u in top}
        tot = sum(w.values())
        for d in range(4):
            assert o[0, 0, t, d] == pytest.approx(sum(w[u] * v[0, 0, u, d] for u in top) / tot, abs=1e-13)


def test_cdf_planted_rows():
    """A peaked row: the CDF stops before the cap with mass >= tau, and the
    prefix without its last block stays below tau; with a tight cap the rule
    is top-cap."""
    s = np.log(np.array([0.05, 0.5, 0.02, 0.3, 0.08, 0.05]))    # masses sum to 1
    p = oracle.row_softmax(s)
    np.testing.assert_allclose(p, np.exp(s), atol=1e-15)
    kept = oracle.select_cdf_row(s, p, 0.75, cap=6)
    assert kept == [1, 3]                       # 0.5 + 0.3 = 0.8 >= 0.75; 0.5 < 0.75
    assert p[kept].sum() >= 0.75 and p[kept].sum() - p[3] < 0.75
    kept = oracle.select_cdf_row(s, p, 0.9, cap=6)
    assert kept == [0, 1, 3, 4]                 # tie 0.05 at blocks 0 and 5 -> lower index
    assert oracle.select_cdf_row(s, p, 0.9, cap=2) == [1, 3]
    assert oracle.select_cdf_row(s, p, 1.5, cap=6) == [0, 1, 2, 3, 4, 5]
    assert oracle.select_cdf_row(s, p, 0.01, cap=6) == [1]
    assert oracle.select_cdf_row(s, p, 0.01, cap=6, forced=[2, 4]) == [2, 4]
    assert oracle.select_cdf_row(s, p, 0.6, cap=6, forced=[2]) == [1, 2, 3]


def test_cdf_random_rows_properties():
    rng = np.random.default_rng(3)
    for _ in range(50):
        nb = int(rng.integers(2, 30))
        s = rng.standard_normal(nb) * 2
        p = oracle.row_softmax(s)
        tau = float(rng.uniform(0.1, 0.99))
        cap = int(rng.integers(1, nb + 1))
        kept = oracle.select_cdf_row(s, p, tau, cap)
        order = sorted(range(nb), key=lambda j: (-s[j], j))
        n = len(kept)
        assert kept == sorted(order[:n])
        if n < cap:
            assert p[kept].sum() >= tau - 1e-12
        if n >= 2:
            assert sum(p[j] for j in order[:n - 1]) < tau


def test_planted_cluster_block_is_selected():
    """A key block whose tokens repeat the query block's direction wins top-k."""
    lay = layout(frames=2, frame_len=8, frame_valid=8, block=4, D=8, scale=1.0)
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 1, 16, 8)) * 0.1
    k = rng.standard_normal((1, 1, 16, 8)) * 0.1
    v = rng.standard_normal((1, 1, 16, 8))
    direction = np.zeros(8)
    direction[3] = 3.0
    q[0, 0, 4:8] += direction            # query block 1
    k[0, 0, 12:16] += direction          # key block 3
    sets, _ = oracle.select(q, k, v, lay, oracle.TOPK, [1])
    assert sets[0][0][1] == [3]


def test_csr_layout():
    sets = [[[[0, 2], [1]], [[3], [0, 1, 2]]]]
    rp, ci = oracle.csr(sets)
    assert rp.tolist() == [0, 2, 3, 4, 7]
    assert ci.tolist() == [0, 2, 1, 3, 0, 1, 2]
