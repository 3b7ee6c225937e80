"""Plain float64 reference of the block-sparse global attention path.

TEST INFRASTRUCTURE ONLY (see the package docstring). Layout convention: a
``layout`` is any object with attributes batch, heads, head_dim, frames,
frame_len, frame_valid, block, scale. Tensors are [B, H, N, D] with
N = frames * frame_len; token f*frame_len + p is real iff p < frame_valid.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

TOPK, CDF, DRIFT = 0, 1, 2


# --------------------------------------------------------------------------
# Token layout (ReSS abstract: global attention over all concatenated view
# tokens; VASC section 4.2 / A.5: camera and register tokens in every frame).
# --------------------------------------------------------------------------
def valid_mask(layout) -> np.ndarray:
    """Boolean [N]: token f*L + p is a real token iff p < frame_valid."""
    p = np.arange(layout.frames * layout.frame_len) % layout.frame_len
    return p < layout.frame_valid


def num_blocks(layout) -> int:
    return (layout.frames * layout.frame_len) // layout.block


def block_tokens(layout, j: int) -> np.ndarray:
    """Indices of the real tokens of block j (block j covers [j*Bk, (j+1)*Bk))."""
    idx = np.arange(j * layout.block, (j + 1) * layout.block)
    return idx[valid_mask(layout)[idx]]


def forced_blocks(layout, force: bool) -> List[int]:
    """Blocks that hold the first token of a frame (the camera/register block).

    The VASC summary (section 4.2) keeps key blocks that hold only special
    tokens at all times; with specials first in each frame that is the block
    containing token f*frame_len.
    """
    if not force:
        return []
    return sorted({(f * layout.frame_len) // layout.block for f in range(layout.frames)})


# --------------------------------------------------------------------------
# Pooling and pooled scores (ReSS Table S5, SpargeAttn row: cumulative
# threshold on pooled query/key inner products; VASC A.1: pooled query blocks
# index physical key/value child blocks).
# --------------------------------------------------------------------------
def pool(x: np.ndarray, layout, dtype=np.float64) -> np.ndarray:
    """Mean of x over the real tokens of every block: [B,H,N,D] -> [B,H,Nb,D].
    Computed in ``dtype`` (float64 for every parity check; float32 only for
    timing the oracle at the GPU's accumulation precision)."""
    B, H, N, D = x.shape
    nb = num_blocks(layout)
    out = np.zeros((B, H, nb, D), dtype=dtype)
    for j in range(nb):
        t = block_tokens(layout, j)
        out[:, :, j, :] = x[:, :, t, :].astype(dtype).mean(axis=2)
    return out


def pooled_scores(qbar: np.ndarray, kbar: np.ndarray, scale: float) -> np.ndarray:
    """S[b,h,i,j] = scale * <qbar_i, kbar_j>."""
    return scale * np.einsum("bhid,bhjd->bhij", qbar, kbar)


def row_softmax(s: np.ndarray) -> np.ndarray:
    """Softmax over the last axis."""
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


# --------------------------------------------------------------------------
# Budgeted selection (VASC A.2: exact binary capacity per query; ReSS Fig. 3b:
# per-head budget c_h; ReSS Table 2: the CDF-threshold rule of SparseVGGT).
# --------------------------------------------------------------------------
def priority_order(score_row: np.ndarray, forced: Sequence[int]) -> List[int]:
    """Forced blocks (ascending) first, then the rest by score desc, index asc."""
    fset = set(forced)
    rest = [j for j in range(len(score_row)) if j not in fset]
    rest.sort(key=lambda j: (-float(score_row[j]), j))
    return sorted(fset) + rest


def select_topk_row(score_row: np.ndarray, k: int, forced: Sequence[int] = ()) -> List[int]:
    """Kept blocks of one query block: the forced ones plus the best-scoring rest,
    k in total. Returned ascending."""
    if len(forced) > k:
        raise ValueError("more forced blocks than the budget")
    return sorted(priority_order(score_row, forced)[:k])


def cdf_count(p_row: np.ndarray, order: Sequence[int], tau: float) -> int:
    """Smallest n >= 1 whose first n blocks (in ``order``) hold mass >= tau;
    the row length if rounding never reaches tau."""
    total = 0.0
    for n, j in enumerate(order, start=1):
        total += float(p_row[j])
        if total >= tau:
            return n
    return len(order)


def select_cdf_row(score_row: np.ndarray, p_row: np.ndarray, tau: float, cap: int,
                   forced: Sequence[int] = ()) -> List[int]:
    """Cumulative-mass rule under a per-head cap: keep the shortest prefix of the
    priority order whose pooled mass reaches tau, at most ``cap`` blocks, never
    fewer than the forced blocks (and at least one)."""
    if len(forced) > cap:
        raise ValueError("more forced blocks than the cap")
    order = priority_order(score_row, forced)
    n = cdf_count(p_row, order, tau)
    n = max(len(forced), min(n, cap), 1)
    return sorted(order[:n])


# --------------------------------------------------------------------------
# Drift score and residual restoration (ReSS abstract, Figs. 1-3: masking a
# block shifts what attention writes into the residual stream; the drop set's
# drift is the norm of its summed contribution vectors; restoration swaps
# blocks at a fixed budget to reduce it).
# --------------------------------------------------------------------------
def drift_row(qbar_i: np.ndarray, k_bh: np.ndarray, v_bh: np.ndarray, layout
              ) -> Tuple[np.ndarray, np.ndarray, float]:
    """Contribution of every key block to the attention output of pooled query i.

    Over the real key tokens u: l_u = scale*<qbar_i, k_u>, e_u = exp(l_u - max l).
    c_j = sum_{u in j} e_u v_u,  z_j = sum_{u in j} e_u,  Z = sum_j z_j.
    Returns (c_j / Z for every j [Nb, D], z_j [Nb], Z).
    """
    nb = num_blocks(layout)
    valid = valid_mask(layout)
    logits = layout.scale * (k_bh.astype(np.float64) @ qbar_i.astype(np.float64))
    m = logits[valid].max()
    e = np.where(valid, np.exp(np.where(valid, logits - m, -np.inf)), 0.0)
    D = v_bh.shape[-1]
    c = np.zeros((nb, D))
    z = np.zeros(nb)
    for j in range(nb):
        t = block_tokens(layout, j)
        z[j] = e[t].sum()
        c[j] = e[t] @ v_bh[t].astype(np.float64)
    Z = z.sum()
    return c / Z, z, Z


def restore_row(chat: np.ndarray, k: int, rounds: int, forced: Sequence[int] = ()
                ) -> Tuple[List[int], float, List[Tuple[int, int]]]:
    """Drift selection of one query block at budget k.

    Initial kept set: the forced blocks plus the highest drift scores
    d_j = ||chat_j||, so the initial drop set holds the lowest-norm blocks.
    Each round finds the single swap (restore a dropped block a, drop a kept
    non-forced block b) that minimises J^2 = ||r - chat_a + chat_b||^2, with
    r = sum of chat over the drop set; ties go to the lower a, then the lower b.
    The swap is made only if it lowers J; otherwise the procedure stops.
    Returns (kept ascending, final J = ||r||, swaps made as (a, b)).
    """
    nb = chat.shape[0]
    d = np.sqrt((chat * chat).sum(axis=1))
    kept = set(priority_order(d, forced)[:k])
    fset = set(forced)
    swaps: List[Tuple[int, int]] = []
    for _ in range(rounds):
        drop = sorted(set(range(nb)) - kept)
        cand_b = sorted(kept - fset)
        r = chat[drop].sum(axis=0)
        if not drop or not cand_b:
            break
        trial = r[None, None, :] - chat[drop][:, None, :] + chat[cand_b][None, :, :]
        j2 = (trial * trial).sum(axis=-1)            # [len(drop), len(cand_b)]
        flat = int(np.argmin(j2))                    # first minimum: lowest a, then b
        ia, ib = divmod(flat, len(cand_b))
        if not j2[ia, ib] < float(r @ r):
            break
        a, b = drop[ia], cand_b[ib]
        kept.remove(b)
        kept.add(a)
        swaps.append((a, b))
    drop = sorted(set(range(nb)) - kept)
    r = chat[drop].sum(axis=0) if drop else np.zeros(chat.shape[1])
    return sorted(kept), float(math.sqrt(float(r @ r))), swaps


def rerank_row(chat: np.ndarray, k: int, rounds: int, forced: Sequence[int] = (),
               track_best: bool = True) -> Tuple[List[int], float, List[List[int]], List[float]]:
    """Drift selection of one query block at budget k by re-rank rounds.

    ReSS scores each block by the shift that dropping it leaves (Fig. 3(b):
    the blocks of highest drift score form the initial selected set) and then
    refines the drop set as a whole (abstract; Fig. 3(c)). Reading of a round
    here: every block is scored again against the residual of the current drop
    set D, r = sum_{j in D} chat_j. With r_j = r minus chat_j when j is in D
    (else r), block j's score is the growth of J^2 that dropping it causes,
        g_j = ||r_j + chat_j||^2 - ||r_j||^2,
    and the new kept set is the forced blocks plus the highest g (ties: lower
    index), k in all, all blocks moving at once. With D empty, g_j = ||chat_j||^2:
    the initial set is the round-0 case of the same rule. Since many blocks move
    together a round can raise J (ReSS Table S3 compares keeping the best set
    seen, "track-best", with keeping the last); with track_best the returned set
    is the one of least J among the initial set and every round's set (ties: the
    earlier), else the last one.
    Returns (kept ascending, J of that set, the kept set of every round with the
    initial set first, J of each of those sets).
    """
    nb = chat.shape[0]
    d2 = (chat * chat).sum(axis=1)
    fset = set(forced)
    kept = set(priority_order(d2, forced)[:k])

    def jdrift(kset):
        drop = [j for j in range(nb) if j not in kset]
        r = chat[drop].sum(axis=0) if drop else np.zeros(chat.shape[1])
        return r, float(math.sqrt(float(r @ r)))

    r, j0 = jdrift(kept)
    sets, js = [sorted(kept)], [j0]
    for _ in range(rounds):
        g = np.empty(nb)
        for j in range(nb):
            rj = r - chat[j] if j not in kept else r
            g[j] = float((rj + chat[j]) @ (rj + chat[j])) - float(rj @ rj)
        kept = set(priority_order(g, forced)[:k])
        r, jn = jdrift(kept)
        sets.append(sorted(kept))
        js.append(jn)
    if track_best:
        best = min(range(len(js)), key=lambda x: (js[x], x))
    else:
        best = len(js) - 1
    return sets[best], js[best], sets, js


def drift_j(chat: np.ndarray, kept: Sequence[int]) -> float:
    """Realised drift of a kept set: the norm of the summed dropped contributions."""
    drop = sorted(set(range(chat.shape[0])) - set(kept))
    if not drop:
        return 0.0
    r = chat[drop].sum(axis=0)
    return float(math.sqrt(float(r @ r)))


# Drift objectives: RAW is the norm of the summed dropped contributions (the
# objective the restoration above minimises); RENORM is the shift of the pooled
# query's attention output once the dropped blocks are removed and the kept
# weights renormalised, (C - C_D)/(Z - Z_D) - C/Z (ReSS Fig. 3(a): masking a
# block shifts what attention writes into the residual stream).
RAW, RENORM = 0, 1


def drift_j_renorm(chat: np.ndarray, zhat: np.ndarray, kept: Sequence[int]) -> float:
    """|| sum_{j in S} chat_j / sum_{j in S} zhat_j - sum_j chat_j || for the kept set S,
    with chat_j = c_j / Z and zhat_j = z_j / Z (so sum_j zhat_j = 1)."""
    S = sorted(set(kept))
    obar = chat.sum(axis=0)
    zs = float(zhat[S].sum()) if S else 0.0
    if zs <= 0.0:
        return math.inf
    u = chat[S].sum(axis=0) / zs - obar
    return float(math.sqrt(float(u @ u)))


def restore_row_renorm(chat: np.ndarray, zhat: np.ndarray, k: int, rounds: int,
                       forced: Sequence[int] = ()) -> Tuple[List[int], float, List[Tuple[int, int]]]:
    """Drift selection at budget k under the RENORM objective.

    The initial kept set is that of restore_row (forced blocks, then the highest
    ||chat_j||). Each round evaluates every swap (restore a dropped block a, drop
    a kept non-forced block b) by the renormalised drift of the resulting set,
    J^2 = || (C_S + chat_a - chat_b) / (Z_S + zhat_a - zhat_b) - sum_j chat_j ||^2,
    takes the least (ties: lower a, then lower b) and makes it only if it lowers
    J; otherwise the procedure stops. Returns (kept ascending, final J, swaps).
    """
    nb = chat.shape[0]
    d = np.sqrt((chat * chat).sum(axis=1))
    kept = set(priority_order(d, forced)[:k])
    fset = set(forced)
    obar = chat.sum(axis=0)
    swaps: List[Tuple[int, int]] = []
    for _ in range(rounds):
        drop = sorted(set(range(nb)) - kept)
        cand_b = sorted(kept - fset)
        if not drop or not cand_b:
            break
        S = sorted(kept)
        cs, zs = chat[S].sum(axis=0), float(zhat[S].sum())
        cur = drift_j_renorm(chat, zhat, S) ** 2
        c2 = cs[None, None, :] + chat[drop][:, None, :] - chat[cand_b][None, :, :]
        z2 = zs + zhat[drop][:, None] - zhat[cand_b][None, :]
        with np.errstate(divide="ignore", invalid="ignore"):
            u = c2 / z2[:, :, None] - obar[None, None, :]
            j2 = np.where(z2 > 0, (u * u).sum(axis=-1), np.inf)
        flat = int(np.argmin(j2))
        ia, ib = divmod(flat, len(cand_b))
        if not j2[ia, ib] < cur:
            break
        a, b = drop[ia], cand_b[ib]
        kept.remove(b)
        kept.add(a)
        swaps.append((a, b))
    return sorted(kept), drift_j_renorm(chat, zhat, sorted(kept)), swaps


# --------------------------------------------------------------------------
# Whole-layer selection and CSR emission.
# --------------------------------------------------------------------------
def select(q: np.ndarray, k: np.ndarray, v: np.ndarray, layout, mode: int,
           keep: Sequence[int], tau: float = 0.9, force: bool = False,
           rounds: int = 0, objective: int = RAW):
    """Kept key blocks for every (b, h, query block).

    Returns (sets, row_stat) where sets[b][h][i] is an ascending list and
    row_stat[b,h,i] is the kept pooled mass (TOPK, CDF) or the final drift J
    (DRIFT, under the given objective).
    """
    B, H = q.shape[0], q.shape[1]
    nb = num_blocks(layout)
    forced = forced_blocks(layout, force)
    qbar = pool(q, layout)
    stat = np.zeros((B, H, nb))
    sets = [[[None] * nb for _ in range(H)] for _ in range(B)]
    if mode in (TOPK, CDF):
        kbar = pool(k, layout)
        s = pooled_scores(qbar, kbar, layout.scale)
        p = row_softmax(s)
        for b in range(B):
            for h in range(H):
                for i in range(nb):
                    if mode == TOPK:
                        kept = select_topk_row(s[b, h, i], int(keep[h]), forced)
                    else:
                        kept = select_cdf_row(s[b, h, i], p[b, h, i], tau, int(keep[h]), forced)
                    sets[b][h][i] = kept
                    stat[b, h, i] = p[b, h, i, kept].sum()
    elif mode == DRIFT:
        for b in range(B):
            for h in range(H):
                for i in range(nb):
                    chat, z, Z = drift_row(qbar[b, h, i], k[b, h], v[b, h], layout)
                    if objective == RENORM:
                        kept, j, _ = restore_row_renorm(chat, z / Z, int(keep[h]), rounds, forced)
                    else:
                        kept, j, _ = restore_row(chat, int(keep[h]), rounds, forced)
                    sets[b][h][i] = kept
                    stat[b, h, i] = j
    else:
        raise ValueError("unknown mode")
    return sets, stat


def csr(sets) -> Tuple[np.ndarray, np.ndarray]:
    """Row pointer and ascending column indices, rows ordered (b, h, i)."""
    rows = [kept for per_b in sets for per_h in per_b for kept in per_h]
    row_ptr = np.zeros(len(rows) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    col_idx = np.array([j for r in rows for j in sorted(r)], dtype=np.int64)
    return row_ptr, col_idx


# --------------------------------------------------------------------------
# Block-sparse attention (VASC section 3: retained weights are renormalised
# after dropping connections; ReSS Table S6: every selection rule feeds the
# same block grid and the same sparse kernel).
# --------------------------------------------------------------------------
def attention_rows(q_rows: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float,
                   dtype=np.float64) -> Tuple[np.ndarray, np.ndarray]:
    """Exact softmax attention of the given query rows over the given keys, in
    ``dtype`` (float64 for parity; float32 only for timing)."""
    s = dtype(scale) * (q_rows.astype(dtype) @ keys.astype(dtype).T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    o = (e @ vals.astype(dtype)) / l
    return o, (m + np.log(l))[:, 0]


def sparse_attention_row(q_bh, k_bh, v_bh, layout, i: int, kept: Sequence[int],
                         dtype=np.float64) -> Tuple[np.ndarray, np.ndarray]:
    """Output rows of query block i attending to the real keys of the kept blocks.

    Returns (o [Bk, D], lse [Bk]); padding query rows give o = 0, lse = -inf.
    """
    Bk, D = layout.block, q_bh.shape[-1]
    o = np.zeros((Bk, D), dtype=dtype)
    lse = np.full(Bk, -np.inf, dtype=dtype)
    rows = block_tokens(layout, i)
    if not len(kept):
        return o, lse          # no listed block: nothing to attend to
    keys = np.concatenate([block_tokens(layout, j) for j in sorted(kept)])
    if len(rows) and len(keys):
        orow, lrow = attention_rows(q_bh[rows], k_bh[keys], v_bh[keys], layout.scale, dtype)
        o[rows - i * Bk] = orow
        lse[rows - i * Bk] = lrow
    return o, lse


def sparse_attention(q, k, v, layout, row_ptr, col_idx) -> Tuple[np.ndarray, np.ndarray]:
    """Block-sparse attention of the whole layer from a CSR block list."""
    B, H, N, D = q.shape
    nb = num_blocks(layout)
    o = np.zeros((B, H, N, D))
    lse = np.full((B, H, N), -np.inf)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                r = (b * H + h) * nb + i
                kept = [int(x) for x in col_idx[row_ptr[r]:row_ptr[r + 1]]]
                ob, lb = sparse_attention_row(q[b, h], k[b, h], v[b, h], layout, i, kept)
                o[b, h, i * layout.block:(i + 1) * layout.block] = ob
                lse[b, h, i * layout.block:(i + 1) * layout.block] = lb
    return o, lse


def dense_attention(q, k, v, layout) -> Tuple[np.ndarray, np.ndarray]:
    """Dense attention over all real keys (padding queries give 0, -inf)."""
    B, H, N, D = q.shape
    valid = valid_mask(layout)
    keys = np.nonzero(valid)[0]
    o = np.zeros((B, H, N, D))
    lse = np.full((B, H, N), -np.inf)
    for b in range(B):
        for h in range(H):
            ob, lb = attention_rows(q[b, h, keys], k[b, h, keys], v[b, h, keys], layout.scale)
            o[b, h, keys] = ob
            lse[b, h, keys] = lb
    return o, lse


def special_rows_dense(q, k, v, layout, o, lse, n_special: int) -> Tuple[np.ndarray, np.ndarray]:
    """Camera and register query rows keep dense attention (VASC section 4.2 and
    A.5): in every frame the first n_special tokens (the special tokens, at the
    start of the frame) attend over all real keys of their (b, h); every other
    row keeps the given output. Returns new (o, lse) arrays.
    """
    B, H, N, D = q.shape
    o2 = np.array(o, dtype=np.float64, copy=True)
    l2 = np.array(lse, dtype=np.float64, copy=True)
    keys = np.nonzero(valid_mask(layout))[0]
    rows = np.array([f * layout.frame_len + p for f in range(layout.frames) for p in range(n_special)],
                    dtype=np.int64)
    if not len(rows):
        return o2, l2
    for b in range(B):
        for h in range(H):
            ob, lb = attention_rows(q[b, h, rows], k[b, h, keys], v[b, h, keys], layout.scale)
            o2[b, h, rows] = ob
            l2[b, h, rows] = lb
    return o2, l2


def executed_block_pairs(row_ptr) -> int:
    return int(row_ptr[-1])
