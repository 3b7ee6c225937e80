"""Workload presets and seeded generators.

The five presets mirror the multi-view global-attention layers that the pages
time and ablate:

* the ReSS page (thelatestinai.com 2609.35593), Table 1 and Table S7: VGGT at
  100 views, bf16, sparsity about 0.745, with a shared sparse kernel whose key
  blocks are 64 wide (Table S5, FlexPrefill granularity row);
* the VASC summary (paperlayer.ai 2610.01013v1), section 4.2 and appendix A.5:
  camera and register tokens per frame, special-only key blocks always kept.

Real images and trained backbones are not available, so token features are
synthetic: 64 Gaussian cluster centres plus noise, projected per head by random
64x64 matrices (queries and keys share the token features), values i.i.d.
normal. Each frame holds 1374 valid tokens (5 special + 1369 patch tokens,
specials first) padded with zeros to 1408 = 11 blocks of 128.

Every random number is drawn here, in a fixed order, from
``numpy.random.default_rng(seed)``; bf16 tensors are rounded once, to nearest
even, and both sides read exactly those bits.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"

MODE_TOPK = 0
MODE_CDF = 1
MODE_DRIFT = 2


@dataclasses.dataclass(frozen=True)
class Layout:
    """Token layout of one global-attention layer.

    Tensors are [batch, heads, frames * frame_len, head_dim], row-major with
    head_dim contiguous. Token ``f * frame_len + p`` is a real token iff
    ``p < frame_valid``; the rest are zero padding.
    """

    batch: int
    heads: int
    head_dim: int
    frames: int
    frame_len: int
    frame_valid: int
    block: int
    dtype: str
    scale: float

    @property
    def tokens(self) -> int:
        return self.frames * self.frame_len

    @property
    def nblocks(self) -> int:
        return self.tokens // self.block


@dataclasses.dataclass(frozen=True)
class Workload:
    """One preset: layout, selection rule and its parameters, seed."""

    name: str
    layout: Layout
    mode: int
    sparsity: Optional[float]          # requested block sparsity (TOPK / DRIFT)
    cdf_tau: float
    force_frame_first_block: bool
    swap_rounds: int
    seed: int
    description: str


def keep_from_sparsity(nblocks: int, sparsity: float) -> int:
    """Kept key blocks per query block for a requested block sparsity.

    Sparsity counts dropped blocks, rounded half up, and at least one block is
    kept: keep = nblocks - floor(sparsity * nblocks + 1/2), clamped to >= 1.
    """
    dropped = int(np.floor(sparsity * nblocks + 0.5))
    return max(1, nblocks - dropped)


def _layer(frames: int, block: int = 128) -> Layout:
    return Layout(batch=1, heads=16, head_dim=64, frames=frames, frame_len=1408,
                  frame_valid=1374, block=block, dtype=BF16, scale=0.125)


CONFIGS: List[Workload] = [
    Workload("tiny_f32_1024tok", Layout(1, 1, 64, 4, 256, 256, 64, F32, 0.125),
             MODE_TOPK, 0.75, 0.9, False, 0, 0,
             "1 head, 4 frames x 256 tokens, block 64, keep top-4 of 16 key blocks, fp32"),
    Workload("vggt_layer_8f_s50", _layer(8), MODE_TOPK, 0.50, 0.9, False, 0, 1,
             "8 frames x 1408 (1374 valid), 16 heads, block 128, 50% block sparsity, top-k"),
    Workload("vggt_layer_32f_s75", _layer(32), MODE_TOPK, 0.75, 0.9, True, 0, 2,
             "32 frames x 1408, 16 heads, block 128, 75% sparsity, top-k, "
             "per-frame special-token block always kept"),
    Workload("vggt_layer_100f_cdf", _layer(100), MODE_CDF, None, 0.9, False, 0, 3,
             "100 frames x 1408, 16 heads, block 128, per-head caps for 70-97% sparsity, "
             "cumulative pooled-mass threshold 0.9"),
    Workload("vggt_layer_16f_drift", _layer(16), MODE_DRIFT, 0.80, 0.9, False, 3, 4,
             "16 frames x 1408, 16 heads, block 128, 80% sparsity, drift score + "
             "3 rounds of swap restoration"),
]


def config(index_or_name) -> Workload:
    if isinstance(index_or_name, int):
        return CONFIGS[index_or_name]
    for w in CONFIGS:
        if w.name == index_or_name:
            return w
    raise KeyError(index_or_name)


def bf16_bits_from_float(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even, returning uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def float_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits to float32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _scatter_frames(x: np.ndarray, lay: Layout) -> np.ndarray:
    """[B,H,F,Lv,D] -> [B,H,F*L,D] with zero padding at the end of each frame."""
    B, H, F, Lv, D = x.shape
    out = np.zeros((B, H, F, lay.frame_len, D), dtype=x.dtype)
    out[:, :, :, :Lv, :] = x
    return out.reshape(B, H, F * lay.frame_len, D)


def generate(w: Workload, heads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw the inputs of preset ``w``.

    Returns a dict with
      ``q, k, v``: float32 arrays [B,H,N,D] holding exactly the values both
                   sides compute on (bf16-representable for bf16 presets);
      ``q_bits, k_bits, v_bits``: uint16 bf16 bits (bf16 presets only);
      ``keep``: int32 [H] kept blocks per query block (TOPK / DRIFT) or the
                per-head cap (CDF);
      ``sparsity_h``: float64 [H] per-head requested sparsity.

    ``heads`` limits the output to the first ``heads`` heads (all draws are
    still made in full so the values equal those of the full preset).
    """
    lay = w.layout
    rng = np.random.default_rng(w.seed)
    B, H, D = lay.batch, lay.heads, lay.head_dim
    out: Dict[str, np.ndarray] = {}
    if lay.dtype == F32:
        shape = (B, H, lay.tokens, D)
        q = rng.standard_normal(shape, dtype=np.float32)
        k = rng.standard_normal(shape, dtype=np.float32)
        v = rng.standard_normal(shape, dtype=np.float32)
        sparsity_h = np.full(H, w.sparsity, dtype=np.float64)
    else:
        F, Lv = lay.frames, lay.frame_valid
        centres = rng.standard_normal((64, D), dtype=np.float32)
        ids = rng.integers(0, 64, size=(B, F, Lv))
        noise = rng.standard_normal((B, F, Lv, D), dtype=np.float32) * np.float32(0.3)
        wq = rng.standard_normal((H, D, D), dtype=np.float32) * np.float32(1.0 / 8.0)
        wk = rng.standard_normal((H, D, D), dtype=np.float32) * np.float32(1.0 / 8.0)
        vraw = rng.standard_normal((B, H, F, Lv, D), dtype=np.float32)
        if w.mode == MODE_CDF:
            sparsity_h = rng.uniform(0.70, 0.97, H)
        else:
            sparsity_h = np.full(H, w.sparsity, dtype=np.float64)
        x = centres[ids] + noise                                   # [B,F,Lv,D]
        q = np.einsum("bfld,hde->bhfle", x, wq, optimize=True).astype(np.float32)
        k = np.einsum("bfld,hde->bhfle", x, wk, optimize=True).astype(np.float32)
        qb = bf16_bits_from_float(_scatter_frames(q, lay))
        kb = bf16_bits_from_float(_scatter_frames(k, lay))
        vb = bf16_bits_from_float(_scatter_frames(vraw, lay))
        del q, k, vraw, x, noise
        out["q_bits"], out["k_bits"], out["v_bits"] = qb, kb, vb
        q, k, v = float_from_bf16_bits(qb), float_from_bf16_bits(kb), float_from_bf16_bits(vb)
    nb = lay.nblocks
    keep = np.array([keep_from_sparsity(nb, s) for s in sparsity_h], dtype=np.int32)
    out.update(q=q, k=k, v=v, keep=keep, sparsity_h=sparsity_h)
    if heads is not None:
        for name in ("q", "k", "v", "q_bits", "k_bits", "v_bits"):
            if name in out:
                out[name] = np.ascontiguousarray(out[name][:, :heads])
        out["keep"] = out["keep"][:heads].copy()
        out["sparsity_h"] = out["sparsity_h"][:heads].copy()
    return out


def restrict(w: Workload, heads: int) -> Workload:
    """The preset with its layout limited to the first ``heads`` heads."""
    return dataclasses.replace(w, layout=dataclasses.replace(w.layout, heads=heads))
