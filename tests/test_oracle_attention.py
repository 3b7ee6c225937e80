"""Pins of the oracle's block-sparse attention (no GPU).

Each test checks the oracle against something other than itself: pure-Python
brute force, torch's scaled_dot_product_attention in float64 on the CPU (a
textbook routine), closed forms, or an identity between two computations.
"""
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


def rand_qkv(lay, seed, pad_zero=True):
    rng = np.random.default_rng(seed)
    N = lay.frames * lay.frame_len
    shape = (lay.batch, lay.heads, N, lay.head_dim)
    q, k, v = (rng.standard_normal(shape) for _ in range(3))
    if pad_zero:
        valid = (np.arange(N) % lay.frame_len) < lay.frame_valid
        for x in (q, k, v):
            x[:, :, ~valid] = 0.0
    return q, k, v


def brute_force(q, k, v, lay, kept_sets):
    """Token-by-token softmax written out with math.exp (no numpy reductions)."""
    N, D = q.shape[2], q.shape[3]
    out = [[0.0] * D for _ in range(N)]
    for t in range(N):
        if t % lay.frame_len >= lay.frame_valid:
            continue
        i = t // lay.block
        keys = [u for j in kept_sets[i] for u in range(j * lay.block, (j + 1) * lay.block)
                if u % lay.frame_len < lay.frame_valid]
        s = [lay.scale * sum(q[0, 0, t, d] * k[0, 0, u, d] for d in range(D)) for u in keys]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        tot = sum(w)
        for d in range(D):
            out[t][d] = sum(w[n] * v[0, 0, u, d] for n, u in enumerate(keys)) / tot
    return np.array(out)


def kept_to_csr(kept_sets):
    row_ptr = np.concatenate([[0], np.cumsum([len(s) for s in kept_sets])])
    col_idx = np.array([j for s in kept_sets for j in sorted(s)])
    return row_ptr, col_idx


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_sparse_attention_matches_brute_force(seed):
    lay = layout()
    q, k, v = rand_qkv(lay, seed)
    nb = oracle.num_blocks(lay)
    rng = np.random.default_rng(100 + seed)
    kept = [sorted(rng.choice(nb, size=rng.integers(1, nb + 1), replace=False).tolist())
            for _ in range(nb)]
    rp, ci = kept_to_csr(kept)
    o, _ = oracle.sparse_attention(q, k, v, lay, rp, ci)
    np.testing.assert_allclose(o[0, 0], brute_force(q, k, v, lay, kept), rtol=0, atol=1e-13)


@pytest.mark.parametrize("seed", [0, 1])
def test_all_blocks_kept_equals_dense_and_sdpa(seed):
    lay = layout(frames=3, frame_len=16, frame_valid=13, block=8, D=8, heads=2, scale=1 / math.sqrt(8))
    q, k, v = rand_qkv(lay, seed)
    nb = oracle.num_blocks(lay)
    kept = [[list(range(nb))] * nb for _ in range(lay.heads)]
    rp, ci = oracle.csr([kept])
    o, lse = oracle.sparse_attention(q, k, v, lay, rp, ci)
    od, lsed = oracle.dense_attention(q, k, v, lay)
    np.testing.assert_allclose(o, od, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lsed, rtol=0, atol=1e-12)
    valid = oracle.valid_mask(lay)
    tq, tk, tv = (torch.from_numpy(x[:, :, valid]) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=lay.scale).numpy()
    np.testing.assert_allclose(o[:, :, valid], ref, rtol=0, atol=1e-12)
    assert np.all(o[:, :, ~valid] == 0) and np.all(np.isneginf(lse[:, :, ~valid]))


def test_constant_values_give_constant_output():
    """Rows of the renormalised masked softmax sum to one: V = 1 gives O = 1."""
    lay = layout(frames=2, frame_len=8, frame_valid=5, block=4)
    q, k, _ = rand_qkv(lay, 3)
    v = np.ones_like(q)
    nb = oracle.num_blocks(lay)
    kept = [[0], [1, 3], [2], [0, 1, 2, 3]]
    rp, ci = kept_to_csr(kept)
    o, _ = oracle.sparse_attention(q, k, v, lay, rp, ci)
    valid = oracle.valid_mask(lay)
    np.testing.assert_allclose(o[0, 0, valid], 1.0, atol=1e-14)


def test_lse_merge_of_complementary_masks():
    lay = layout(frames=2, frame_len=8, frame_valid=7, block=4)
    q, k, v = rand_qkv(lay, 4)
    nb = oracle.num_blocks(lay)
    kept_s = [[0, 2], [1], [3], [0, 1, 3]]
    kept_d = [sorted(set(range(nb)) - set(s)) for s in kept_s]
    o_s, l_s = oracle.sparse_attention(q, k, v, lay, *kept_to_csr(kept_s))
    o_d, l_d = oracle.sparse_attention(q, k, v, lay, *kept_to_csr(kept_d))
    o_a, l_a = oracle.dense_attention(q, k, v, lay)
    valid = oracle.valid_mask(lay)
    ws, wd = np.exp(l_s[0, 0, valid])[:, None], np.exp(l_d[0, 0, valid])[:, None]
    merged = (ws * o_s[0, 0, valid] + wd * o_d[0, 0, valid]) / (ws + wd)
    np.testing.assert_allclose(merged, o_a[0, 0, valid], atol=1e-13)
    np.testing.assert_allclose(np.logaddexp(l_s, l_d)[0, 0, valid], l_a[0, 0, valid], atol=1e-13)


def test_dropped_block_identity():
    """Sparse output = (C - sum_dropped C_j) / (Z - sum_dropped z_j) from dense
    per-block partials computed token by token, with one shared shift."""
    lay = layout(frames=2, frame_len=8, frame_valid=6, block=4, D=3)
    q, k, v = rand_qkv(lay, 5)
    nb = oracle.num_blocks(lay)
    kept = [[1, 2], [0], [0, 1, 2, 3], [3]]
    o, _ = oracle.sparse_attention(q, k, v, lay, *kept_to_csr(kept))
    valid = oracle.valid_mask(lay)
    for t in np.nonzero(valid)[0]:
        i = t // lay.block
        s_all = {u: lay.scale * float(q[0, 0, t] @ k[0, 0, u]) for u in np.nonzero(valid)[0]}
        shift = max(s_all.values())
        Cj = np.zeros((nb, lay.head_dim))
        zj = np.zeros(nb)
        for u, s in s_all.items():
            Cj[u // lay.block] += math.exp(s - shift) * v[0, 0, u]
            zj[u // lay.block] += math.exp(s - shift)
        dropped = [j for j in range(nb) if j not in kept[i]]
        expect = (Cj.sum(0) - Cj[dropped].sum(0)) / (zj.sum() - zj[dropped].sum())
        np.testing.assert_allclose(o[0, 0, t], expect, atol=1e-12)


def test_identical_keys_give_mean_of_kept_values():
    lay = layout(frames=2, frame_len=8, frame_valid=6, block=4)
    q, _, v = rand_qkv(lay, 6)
    valid = oracle.valid_mask(lay)
    k = np.zeros_like(q)
    k[:, :, valid] = np.array([0.3, -1.0, 2.0, 0.5])
    kept = [[0, 3], [2], [1], [0, 1, 2, 3]]
    o, _ = oracle.sparse_attention(q, k, v, lay, *kept_to_csr(kept))
    for i, ks in enumerate(kept):
        toks = [u for j in ks for u in range(4 * j, 4 * j + 4) if valid[u]]
        mean_v = v[0, 0, toks].mean(axis=0)
        for t in range(4 * i, 4 * i + 4):
            if valid[t]:
                np.testing.assert_allclose(o[0, 0, t], mean_v, atol=1e-14)


def test_frame_permutation_equivariance():
    """Permuting whole frames of K and V, with the kept block lists relabelled,
    leaves the output unchanged."""
    lay = layout(frames=3, frame_len=8, frame_valid=6, block=4)
    q, k, v = rand_qkv(lay, 7)
    nb = oracle.num_blocks(lay)
    perm = [2, 0, 1]                     # new frame f holds old frame perm[f]
    tok = np.concatenate([np.arange(p * 8, p * 8 + 8) for p in perm])
    k2, v2 = k[:, :, tok], v[:, :, tok]
    old_to_new_block = {}
    for f, p in enumerate(perm):
        for b in range(2):
            old_to_new_block[2 * p + b] = 2 * f + b
    rng = np.random.default_rng(8)
    kept = [sorted(rng.choice(nb, size=3, replace=False).tolist()) for _ in range(nb)]
    kept2 = [sorted(old_to_new_block[j] for j in s) for s in kept]
    o1, l1 = oracle.sparse_attention(q, k, v, lay, *kept_to_csr(kept))
    o2, l2 = oracle.sparse_attention(q, k2, v2, lay, *kept_to_csr(kept2))
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_empty_block_list_gives_zero_output():
    """A query block with no listed key block attends to nothing: o = 0 and
    lse = -inf, as for padding rows."""
    lay = layout()
    q, k, v = rand_qkv(lay, 9)
    o, lse = oracle.sparse_attention_row(q[0, 0], k[0, 0], v[0, 0], lay, 1, [])
    assert np.all(o == 0) and np.all(np.isneginf(lse))


@pytest.mark.parametrize("n_special", [1, 2])
def test_special_rows_dense_brute_force(n_special):
    """Camera/register rows (the first n_special tokens of every frame) attend
    over every real key; all other rows keep the sparse output unchanged."""
    lay = layout(frames=3)
    q, k, v = rand_qkv(lay, 12)
    nb = oracle.num_blocks(lay)
    rng = np.random.default_rng(13)
    kept = [sorted(rng.choice(nb, size=2, replace=False).tolist()) for _ in range(nb)]
    rp, ci = kept_to_csr(kept)
    o, lse = oracle.sparse_attention(q, k, v, lay, rp, ci)
    o2, l2 = oracle.special_rows_dense(q, k, v, lay, o, lse, n_special)
    dense_ref = brute_force(q, k, v, lay, [list(range(nb))] * nb)
    N = lay.frames * lay.frame_len
    special = np.array([(t % lay.frame_len) < n_special for t in range(N)])
    np.testing.assert_allclose(o2[0, 0, special], dense_ref[special], rtol=0, atol=1e-13)
    assert np.array_equal(o2[0, 0, ~special], o[0, 0, ~special])
    assert np.array_equal(l2[0, 0, ~special], lse[0, 0, ~special])
    # lse of a special row: log of the sum of exp over all real keys, written out
    t = lay.frame_len + n_special - 1
    keys = [u for u in range(N) if u % lay.frame_len < lay.frame_valid]
    s = [lay.scale * sum(q[0, 0, t, d] * k[0, 0, u, d] for d in range(lay.head_dim)) for u in keys]
    m = max(s)
    assert abs(l2[0, 0, t] - (m + math.log(sum(math.exp(x - m) for x in s)))) <= 1e-12


def test_special_rows_dense_limits():
    """n_special = 0 changes nothing; n_special = frame_valid makes every real
    row dense, which is the oracle's dense attention (itself pinned to SDPA)."""
    lay = layout(frames=2)
    q, k, v = rand_qkv(lay, 14)
    nb = oracle.num_blocks(lay)
    kept = [[i] for i in range(nb)]
    o, lse = oracle.sparse_attention(q, k, v, lay, *kept_to_csr(kept))
    o0, l0 = oracle.special_rows_dense(q, k, v, lay, o, lse, 0)
    assert np.array_equal(o0, o) and np.array_equal(l0, lse)
    oa, la = oracle.special_rows_dense(q, k, v, lay, o, lse, lay.frame_valid)
    od, ld = oracle.dense_attention(q, k, v, lay)
    np.testing.assert_allclose(oa, od, atol=1e-13)
    np.testing.assert_allclose(la, ld, atol=1e-13)
