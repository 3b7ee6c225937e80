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
