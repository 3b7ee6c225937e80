"""Value-aware block selection with cross-layer memory, float64 reference.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows "VASC: Value-Aware Sparse Attention with Cross-Layer Memory for
Efficient 3D Reconstruction" (paperlayer.ai summary): sections 4.1 (relevance
modulated by the RMS contrast of adjacent pooled value blocks, demand rescaled
and clipped to the query's capacity), 4.2 (memory augments demand; binary
selection within capacity; special-only key blocks always kept), 4.3 (pair
memory adds averaged demand and subtracts averaged execution), and appendix
A.1-A.5 (fixed pairs of adjacent child blocks with a singleton tail,
proportional clipping, zero contrast for the singleton, per-(batch, head)
normalisation of the ranking copy only, state reset per inference).

The summary prints no formulas. The readings taken here, each the plainest
one the text supports:
  pairs       children 2p and 2p+1 of the native block order form pair p; an
              odd last child is a singleton pair.
  contrast    c_p = sqrt(mean_d (vbar_{2p,d} - vbar_{2p+1,d})^2); 0 for the
              singleton.
  demand      a_ij = P_ij * (1 + c_{p(j)} / cbar), P the row softmax of the
              pooled scores and cbar the mean contrast over the pairs of the
              (batch, head) (factor 1 when cbar = 0);
              d_ij = min(1, k * a_ij / sum_j a_ij).
  ranking     rho_ij = d_ij + mhat_{p(j)}; forced blocks first, then rho
              descending, ties to the lower block; exactly k kept.
  memory      raw R_p += D_p - S_p, with D_p and S_p the means of d_ij and of
              the executed flags x_ij over all query blocks i and the children
              j of pair p; the ranking copy is
              mhat_p = max(0, R_p) / max_p' max(0, R_p') per (batch, head)
              (0 when no pair has a deficit). R starts at 0 for an inference.
Parity with the published VASC code is unpinned: neither that code nor
step-level numbers from it are on the pages.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

from .reference import forced_blocks, num_blocks, pool, pooled_scores, priority_order, row_softmax

__all__ = ["pair_children", "pair_contrast", "demand_row", "memory_rank_copy", "memory_update",
           "vasc_select"]


def pair_children(nb: int) -> List[List[int]]:
    """Children of every pair: [0, 1], [2, 3], ..., and [nb-1] when nb is odd
    (VASC A.1)."""
    return [list(range(2 * p, min(2 * p + 2, nb))) for p in range((nb + 1) // 2)]


def pair_contrast(vbar_bh: np.ndarray) -> np.ndarray:
    """RMS difference of the two pooled value vectors of every pair; 0 for a
    singleton (VASC A.3). vbar_bh: [Nb, D] -> [Npairs]."""
    nb = vbar_bh.shape[0]
    out = np.zeros((nb + 1) // 2)
    for p, ch in enumerate(pair_children(nb)):
        if len(ch) == 2:
            diff = vbar_bh[ch[0]] - vbar_bh[ch[1]]
            out[p] = float(np.sqrt(np.mean(diff * diff)))
    return out


def demand_row(p_row: np.ndarray, contrast: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Relevance modulated by the pair contrast, then proportional clipping to
    the capacity k (VASC 4.1, A.2). Returns (a, d) over the row's key blocks."""
    nb = len(p_row)
    cbar = float(contrast.mean()) if len(contrast) else 0.0
    factor = np.ones(nb)
    if cbar > 0.0:
        factor = 1.0 + contrast[np.arange(nb) // 2] / cbar
    a = p_row * factor
    d = np.minimum(1.0, k * a / a.sum())
    return a, d


def memory_rank_copy(raw_bh: np.ndarray) -> np.ndarray:
    """Ranking copy of one (batch, head)'s pair memory: deficits clipped at zero,
    scaled so the largest is 1 (VASC 4.3, A.4)."""
    pos = np.maximum(raw_bh, 0.0)
    top = float(pos.max()) if len(pos) else 0.0
    return pos / top if top > 0.0 else np.zeros_like(pos)


def memory_update(raw_bh: np.ndarray, d_bh: np.ndarray, x_bh: np.ndarray) -> np.ndarray:
    """raw += mean demand - mean execution per pair, the means over all query
    blocks and the pair's children (VASC 4.3, A.3, A.5). d_bh, x_bh: [Nq, Nb]."""
    nq, nb = d_bh.shape
    out = np.array(raw_bh, dtype=np.float64, copy=True)
    for p, ch in enumerate(pair_children(nb)):
        dem = d_bh[:, ch].sum() / (nq * len(ch))
        srv = x_bh[:, ch].sum() / (nq * len(ch))
        out[p] += dem - srv
    return out


def vasc_select(q: np.ndarray, k: np.ndarray, v: np.ndarray, layout, keep: Sequence[int],
                force: bool, raw: np.ndarray):
    """One layer: selection from the current memory, then the memory update.

    raw: [B, H, Npairs] pair memory before the layer. Returns (sets, stat, d, x,
    raw_after) with sets[b][h][i] the kept blocks (ascending), stat the kept
    pooled mass sum_kept P, d the clipped demand [B,H,Nb,Nb] and x the executed
    flags [B,H,Nb,Nb].
    """
    B, H = q.shape[0], q.shape[1]
    nb = num_blocks(layout)
    qbar, kbar, vbar = pool(q, layout), pool(k, layout), pool(v, layout)
    s = pooled_scores(qbar, kbar, layout.scale)
    p = row_softmax(s)
    forced = forced_blocks(layout, force)
    sets = [[[None] * nb for _ in range(H)] for _ in range(B)]
    stat = np.zeros((B, H, nb))
    d = np.zeros((B, H, nb, nb))
    x = np.zeros((B, H, nb, nb))
    raw_after = np.array(raw, dtype=np.float64, copy=True)
    for b in range(B):
        for h in range(H):
            c = pair_contrast(vbar[b, h])
            mhat = memory_rank_copy(raw[b, h])
            kh = int(keep[h])
            if len(forced) > kh:
                raise ValueError("more forced blocks than the budget")
            for i in range(nb):
                _, drow = demand_row(p[b, h, i], c, kh)
                rho = drow + mhat[np.arange(nb) // 2]
                kept = sorted(priority_order(rho, forced)[:kh])
                sets[b][h][i] = kept
                stat[b, h, i] = p[b, h, i, kept].sum()
                d[b, h, i] = drow
                x[b, h, i, kept] = 1.0
            raw_after[b, h] = memory_update(raw[b, h], d[b, h], x[b, h])
    return sets, stat, d, x, raw_after
