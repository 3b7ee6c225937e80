"""Oracle against the hand-derived closed-form fixtures in tests/golden/."""
import json
import math
import os
import types

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


@pytest.fixture(scope="module")
def hand():
    g = _load("hand_example.json")
    lay = types.SimpleNamespace(**g["layout"])
    arr = lambda key: np.array(g[key], dtype=np.float64)[None, None]
    return g, lay, arr("q"), arr("k"), arr("v")


def _lse(vals):
    return np.array([-np.inf if x is None else x for x in vals])


def test_dense_attention_closed_form(hand):
    g, lay, q, k, v = hand
    o, lse = oracle.dense_attention(q, k, v, lay)
    np.testing.assert_allclose(o[0, 0], np.array(g["dense_o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], _lse(g["dense_lse"]), rtol=0, atol=1e-14)


@pytest.mark.parametrize("kept,key", [([0], "keep0"), ([1], "keep1"), ([0, 1], "dense")])
def test_sparse_attention_closed_form(hand, kept, key):
    g, lay, q, k, v = hand
    o = np.zeros((4, 2))
    lse = np.zeros(4)
    for i in range(2):
        ob, lb = oracle.sparse_attention_row(q[0, 0], k[0, 0], v[0, 0], lay, i, kept)
        o[2 * i:2 * i + 2] = ob
        lse[2 * i:2 * i + 2] = lb
    np.testing.assert_allclose(o, np.array(g[key + "_o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, _lse(g[key + "_lse"]), rtol=0, atol=1e-14)


def test_pooling_scores_and_topk_closed_form(hand):
    g, lay, q, k, v = hand
    qbar = oracle.pool(q, lay)[0, 0]
    kbar = oracle.pool(k, lay)[0, 0]
    np.testing.assert_allclose(qbar, np.array(g["qbar"]), atol=1e-15)
    np.testing.assert_allclose(kbar, np.array(g["kbar"]), atol=1e-15)
    s = oracle.pooled_scores(qbar[None, None], kbar[None, None], lay.scale)[0, 0]
    np.testing.assert_allclose(s, np.array(g["scores"]), atol=1e-15)
    sets, _ = oracle.select(q, k, v, lay, oracle.TOPK, [1])
    assert sets[0][0] == g["top1"]


def test_drift_closed_form(hand):
    g, lay, q, k, v = hand
    qbar = oracle.pool(q, lay)[0, 0]
    chat, z, Z = oracle.drift_row(qbar[0], k[0, 0], v[0, 0], lay)
    np.testing.assert_allclose(chat, np.array(g["drift_q0_chat"]), atol=1e-15)
    np.testing.assert_allclose(z / Z, np.array(g["drift_q0_z_over_Z"]), atol=1e-15)


def test_restoration_closed_form():
    g = _load("restoration_example.json")
    chat = np.array(g["chat"], dtype=np.float64)
    kept0, j0, sw0 = oracle.restore_row(chat, g["keep"], 0)
    assert kept0 == g["initial_kept"] and sw0 == []
    assert j0 == pytest.approx(g["initial_J"], abs=1e-15)
    kept, j, swaps = oracle.restore_row(chat, g["keep"], 3)
    assert kept == g["final_kept_3_rounds"]
    assert [list(s) for s in swaps] == g["swaps"]
    assert j == pytest.approx(g["final_J"], abs=1e-15)
    assert j == pytest.approx(g["exhaustive_best_J"], abs=1e-15)
