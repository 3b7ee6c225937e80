"""Pins of the oracle's value-aware selection and pair memory (no GPU).

Closed forms of each reading (pairing, RMS contrast, proportional clipping,
ranking copy, memory update), the special case that reduces to pooled top-k,
and the conservation of the memory balance.
"""
import types

import numpy as np
import pytest

import oracle


def layout(frames=2, frame_len=64, frame_valid=64, block=8, D=4, heads=1, scale=0.5):
    return types.SimpleNamespace(batch=1, heads=heads, head_dim=D, frames=frames,
                                 frame_len=frame_len, frame_valid=frame_valid,
                                 block=block, scale=scale)


def test_pairs_with_singleton_tail():
    assert oracle.pair_children(4) == [[0, 1], [2, 3]]
    assert oracle.pair_children(5) == [[0, 1], [2, 3], [4]]
    assert oracle.pair_children(1) == [[0]]


def test_contrast_closed_form():
    v = np.array([[1.0, 2.0, 3.0, 4.0], [1.0, 0.0, 3.0, 0.0], [7.0, 7.0, 7.0, 7.0]])
    c = oracle.pair_contrast(v)
    # diff (0, 2, 0, 4): mean square (4 + 16) / 4 = 5; the singleton has none
    assert c == pytest.approx([np.sqrt(5.0), 0.0], abs=1e-15)


def test_proportional_clipping_closed_forms():
    p = np.array([0.5, 0.3, 0.2, 0.0])
    a, d = oracle.demand_row(p, np.zeros(2), 2)
    assert a == pytest.approx(p)
    assert d == pytest.approx([1.0, 0.6, 0.4, 0.0])
    # pair 0 has contrast 1, pair 1 none: mean 0.5, factors (3, 3, 1, 1)
    a, d = oracle.demand_row(p, np.array([1.0, 0.0]), 2)
    assert a == pytest.approx([1.5, 0.9, 0.2, 0.0])
    assert d == pytest.approx([1.0, 2 * 0.9 / 2.6, 2 * 0.2 / 2.6, 0.0])
    # no element reaches one: the demand is the capacity, spread in proportion
    a, d = oracle.demand_row(np.full(8, 1 / 8), np.zeros(4), 3)
    assert d.sum() == pytest.approx(3.0) and np.all(d < 1)


@pytest.mark.parametrize("seed", range(5))
def test_demand_bounds(seed):
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.full(11, 0.3))
    c = rng.random(6)
    k = int(rng.integers(1, 11))
    _, d = oracle.demand_row(p, c, k)
    assert np.all(d <= 1.0 + 1e-15) and np.all(d >= 0)
    assert d.sum() <= k + 1e-12
    if np.all(d < 1.0):
        assert d.sum() == pytest.approx(k)


def test_rank_copy_closed_form():
    assert oracle.memory_rank_copy(np.array([-1.0, 0.5, 2.0, 0.0])) == pytest.approx(
        [0.0, 0.25, 1.0, 0.0])
    assert np.all(oracle.memory_rank_copy(np.array([-1.0, -0.5])) == 0)


def test_memory_update_closed_form():
    d = np.array([[1.0, 0.5, 0.25], [0.0, 0.5, 0.75]])
    x = np.array([[1.0, 1.0, 0.0], [0.0, 1.0, 1.0]])
    # pair (0, 1): demand 2 / 4, service 3 / 4; singleton 2: demand 1 / 2, service 1 / 2
    out = oracle.memory_update(np.array([0.1, -0.2]), d, x)
    assert out == pytest.approx([0.1 - 0.25, -0.2])


def _inputs(lay, seed, qk_scale=1.0, pair_equal_v=False):
    rng = np.random.default_rng(seed)
    N, D = lay.frames * lay.frame_len, lay.head_dim
    q = rng.standard_normal((1, lay.heads, N, D)) * qk_scale
    k = rng.standard_normal((1, lay.heads, N, D)) * qk_scale
    v = rng.standard_normal((1, lay.heads, N, D))
    if pair_equal_v:
        blk = lay.block
        for j in range(1, N // blk, 2):
            v[:, :, j * blk:(j + 1) * blk] = v[:, :, (j - 1) * blk:j * blk]
    pad = (np.arange(N) % lay.frame_len) >= lay.frame_valid
    for a in (q, k, v):
        a[:, :, pad] = 0
    return q, k, v


@pytest.mark.parametrize("seed", range(4))
def test_reduces_to_pooled_topk(seed):
    """Equal pooled values within every pair (no contrast), no memory and no
    clipped demand: the ranking is the pooled relevance, i.e. pooled top-k."""
    lay = layout(heads=2)
    nb = oracle.num_blocks(lay)
    q, k, v = _inputs(lay, seed, qk_scale=0.3, pair_equal_v=True)
    keep = [4, 3]
    sets, stat, d, x, raw = oracle.vasc_select(q, k, v, lay, keep, False,
                                               np.zeros((1, 2, nb // 2)))
    assert np.all(d < 1)     # nothing clipped at this capacity
    ref, ref_stat = oracle.select(q, k, v, lay, oracle.TOPK, keep)
    assert sets == ref
    assert stat == pytest.approx(ref_stat)


@pytest.mark.parametrize("seed,force", [(0, False), (1, True), (2, False)])
def test_selection_invariants_and_memory_balance(seed, force):
    lay = layout(frames=3, frame_len=48, frame_valid=43, block=8, heads=2)
    nb = oracle.num_blocks(lay)            # 18 blocks, 9 pairs
    q, k, v = _inputs(lay, 10 + seed)
    keep = [5, 7]
    raw0 = np.random.default_rng(seed).standard_normal((1, 2, (nb + 1) // 2)) * 0.1
    sets, stat, d, x, raw1 = oracle.vasc_select(q, k, v, lay, keep, force, raw0)
    forced = oracle.forced_blocks(lay, force)
    for h in range(2):
        for i in range(nb):
            assert len(sets[0][h][i]) == keep[h] and set(forced) <= set(sets[0][h][i])
            assert np.array_equal(np.nonzero(x[0, h, i])[0], sets[0][h][i])
        # the balance moves by total demand minus total execution, which the
        # clipping keeps at or below zero
        w = np.array([len(ch) for ch in oracle.pair_children(nb)]) * nb
        moved = float((w * (raw1[0, h] - raw0[0, h])).sum())
        assert moved == pytest.approx(d[0, h].sum() - nb * keep[h], abs=1e-9)
        assert moved <= 1e-9


def test_memory_deficit_wins_a_slot():
    """A pair with the largest deficit ranks above every unclipped demand:
    its children are kept in every row once the memory holds that deficit."""
    lay = layout(heads=1)
    nb = oracle.num_blocks(lay)            # 16 blocks, 8 pairs
    q, k, v = _inputs(lay, 3, qk_scale=0.3)
    keep = [3]
    raw = np.zeros((1, 1, nb // 2))
    sets0, *_ = oracle.vasc_select(q, k, v, lay, keep, False, raw)
    # a pair that no row keeps without memory
    unused = [p for p in range(nb // 2)
              if all(2 * p not in s and 2 * p + 1 not in s for s in sets0[0][0])]
    assert unused
    p = unused[0]
    raw[0, 0, p] = 0.5
    sets1, *_ = oracle.vasc_select(q, k, v, lay, keep, False, raw)
    for s in sets1[0][0]:
        assert {2 * p, 2 * p + 1} <= set(s)


def test_memory_carried_over_layers_and_reset():
    """Two layers in a row: the second ranks with the first's balance; a fresh
    inference (zero balance) reproduces the first layer."""
    lay = layout(heads=1)
    nb = oracle.num_blocks(lay)
    q, k, v = _inputs(lay, 5)
    keep = [4]
    z = np.zeros((1, 1, nb // 2))
    s1, _, d1, x1, r1 = oracle.vasc_select(q, k, v, lay, keep, False, z)
    assert r1[0, 0] == pytest.approx(oracle.memory_update(z[0, 0], d1[0, 0], x1[0, 0]))
    s2, _, _, _, r2 = oracle.vasc_select(q, k, v, lay, keep, False, r1)
    assert np.any(r1 > 0)          # some pair is under-served after one layer
    s1b, *_ = oracle.vasc_select(q, k, v, lay, keep, False, z)
    assert s1b == s1
