"""ctypes binding of the bsgm C ABI (include/bsgm.h).

Argument marshalling only: every step of the method runs in the HIP kernels of
libbsgm.so. PyTorch supplies device memory and the current stream. If the
library is missing, every entry point raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbsgm.so")

F32, BF16 = 0, 1
TOPK, CDF, DRIFT, VASC = 0, 1, 2, 3
# Drift objectives: the norm of the dropped blocks' summed contribution, or the
# output shift after the kept blocks are renormalised.
DROPPED_SUM, RENORMALISED = 0, 1
BEST_SWAP, RERANK, RERANK_TRACK_BEST = 0, 1, 2

STATUS = {0: "BSGM_OK", -1: "BSGM_E_ARG", -2: "BSGM_E_UNSUPPORTED", -3: "BSGM_E_CAPACITY",
          -4: "BSGM_E_WORKSPACE", -5: "BSGM_E_HIP"}

# Every symbol include/bsgm.h declares.
EXPORTS = ("bsgm_version", "bsgm_last_error", "bsgm_workspace_bytes", "bsgm_col_capacity",
           "bsgm_pool_blocks", "bsgm_pool_blocks2", "bsgm_drift_scores", "bsgm_select_blocks", "bsgm_sparse_attn_fwd",
           "bsgm_special_rows_workspace_bytes", "bsgm_special_rows_dense_fwd",
           "bsgm_vasc_select_blocks", "bsgm_attn_workspace_bytes", "bsgm_attn_prepare",
           "bsgm_sparse_attn_fwd_prepared", "bsgm_select_blocks_fused", "bsgm_fused_workspace_bytes",
           "bsgm_select_blocks_pooled", "bsgm_select_blocks_noalloc", "bsgm_select_drift_streamed",
           "bsgm_drift_streamed_workspace_bytes")


class BsgmError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS.get(code, code)}: {message}")
        self.code = code


class CLayout(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("frames", ctypes.c_int32), ("frame_len", ctypes.c_int32),
                ("frame_valid", ctypes.c_int32), ("block", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float)]


class CSelectParams(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("keep_per_head", ctypes.POINTER(ctypes.c_int32)),
                ("cdf_tau", ctypes.c_float), ("force_frame_first_block", ctypes.c_int32),
                ("swap_rounds", ctypes.c_int32), ("drift_objective", ctypes.c_int32),
                ("restoration", ctypes.c_int32)]


_lib = None


def library() -> ctypes.CDLL:
    """Loads libbsgm.so (built in-tree); raises if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_global_mean_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        lp, pp = ctypes.POINTER(CLayout), ctypes.POINTER(CSelectParams)
        lib.bsgm_version.restype = ctypes.c_int32
        lib.bsgm_last_error.restype = ctypes.c_char_p
        lib.bsgm_workspace_bytes.argtypes = [lp, ctypes.c_int32]
        lib.bsgm_workspace_bytes.restype = sz
        lib.bsgm_col_capacity.argtypes = [lp, pp]
        lib.bsgm_col_capacity.restype = ctypes.c_int64
        lib.bsgm_pool_blocks.argtypes = [lp, vp, vp, vp]
        lib.bsgm_pool_blocks2.argtypes = [lp, vp, vp, vp, vp, vp]
        lib.bsgm_drift_scores.argtypes = [lp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.bsgm_select_blocks.argtypes = [lp, pp, vp, vp, vp, vp, vp, vp, ctypes.c_int64, vp, vp, vp,
                                           vp, sz, vp]
        lib.bsgm_sparse_attn_fwd.argtypes = [lp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.bsgm_attn_prepare.argtypes = [lp, vp, vp, sz, vp]
        lib.bsgm_sparse_attn_fwd_prepared.argtypes = [lp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.bsgm_select_blocks_fused.argtypes = [lp, pp, vp, vp, vp, vp, ctypes.c_int64, vp, vp, vp,
                                                 sz, vp]
        lib.bsgm_select_blocks_pooled.argtypes = [lp, pp, vp, vp, vp, vp, ctypes.c_int64, vp, vp,
                                                  vp, sz, vp]
        lib.bsgm_select_blocks_noalloc.argtypes = [lp, pp, vp, vp, vp, vp, ctypes.c_int64, vp, vp,
                                                   vp]
        lib.bsgm_fused_workspace_bytes.argtypes = [lp]
        lib.bsgm_fused_workspace_bytes.restype = sz
        lib.bsgm_attn_workspace_bytes.argtypes = [lp]
        lib.bsgm_attn_workspace_bytes.restype = sz
        lib.bsgm_special_rows_workspace_bytes.argtypes = [lp, ctypes.c_int32]
        lib.bsgm_special_rows_workspace_bytes.restype = sz
        lib.bsgm_special_rows_dense_fwd.argtypes = [lp, vp, vp, vp, ctypes.c_int32, vp, vp, vp, sz, vp]
        lib.bsgm_vasc_select_blocks.argtypes = [lp, pp, vp, vp, vp, vp, vp, vp, ctypes.c_int64, vp,
                                                vp, vp, sz, vp]
        lib.bsgm_select_drift_streamed.argtypes = [lp, pp, vp, vp, vp, vp, vp, ctypes.c_int64, vp,
                                                   vp, vp, sz, vp]
        lib.bsgm_drift_streamed_workspace_bytes.argtypes = [lp]
        lib.bsgm_drift_streamed_workspace_bytes.restype = sz
        for name in ("bsgm_pool_blocks", "bsgm_pool_blocks2", "bsgm_drift_scores", "bsgm_select_blocks",
                     "bsgm_sparse_attn_fwd", "bsgm_special_rows_dense_fwd",
                     "bsgm_vasc_select_blocks", "bsgm_select_blocks_fused", "bsgm_select_blocks_pooled",
                     "bsgm_select_blocks_noalloc", "bsgm_select_drift_streamed",
                     "bsgm_attn_prepare",
                     "bsgm_sparse_attn_fwd_prepared"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


def c_layout(layout) -> CLayout:
    """Any object with batch, heads, head_dim, frames, frame_len, frame_valid,
    block, dtype ('f32' / 'bf16' or 0 / 1) and scale."""
    dt = layout.dtype
    if isinstance(dt, str):
        dt = {"f32": F32, "bf16": BF16}[dt]
    return CLayout(layout.batch, layout.heads, layout.head_dim, layout.frames, layout.frame_len,
                   layout.frame_valid, layout.block, dt, layout.scale)


def c_params(mode: int, keep: Sequence[int], cdf_tau: float = 0.9, force: bool = False,
             swap_rounds: int = 0, objective: int = 0,
             restoration: int = 0) -> Tuple[CSelectParams, ctypes.Array]:
    arr = (ctypes.c_int32 * len(keep))(*[int(x) for x in keep])
    return CSelectParams(mode, arr, cdf_tau, 1 if force else 0, swap_rounds, objective,
                         restoration), arr


def _check(code: int):
    if code != 0:
        raise BsgmError(code, library().bsgm_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ws(t: Optional[torch.Tensor], name: str = "workspace"):
    """(pointer, size in bytes) of a caller's workspace tensor, or (None, 0)."""
    if t is None:
        return None, 0
    if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    return ctypes.c_void_p(t.data_ptr()), t.numel() * t.element_size()


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _expect(t: torch.Tensor, name: str, dtype: torch.dtype, shape: Tuple[int, ...]):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)}, got "
                         f"{t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()}")


def _opt(t: Optional[torch.Tensor], name: str, dtype: torch.dtype, shape: Tuple[int, ...]):
    """_expect for an optional tensor."""
    if t is not None:
        _expect(t, name, dtype, shape)


def _expect_1d(t: torch.Tensor, name: str, dtype: torch.dtype):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype or t.dim() != 1 or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous 1-D {dtype} tensor, got {t.dtype} "
                         f"{tuple(t.shape)} contiguous={t.is_contiguous()}")


def _dims(layout):
    n = layout.frames * layout.frame_len
    nb = n // layout.block
    return n, nb, layout.batch * layout.heads * nb


def _tdtype(layout) -> torch.dtype:
    return torch.bfloat16 if c_layout(layout).dtype == BF16 else torch.float32


def version() -> int:
    return library().bsgm_version()


def workspace_bytes(layout, mode: int) -> int:
    L = c_layout(layout)
    n = library().bsgm_workspace_bytes(ctypes.byref(L), mode)
    if n == 0:
        raise BsgmError(-1, library().bsgm_last_error().decode())
    return n


def col_capacity(layout, mode: int, keep: Sequence[int], force: bool = False) -> int:
    L = c_layout(layout)
    P, _keep = c_params(mode, keep, force=force)
    n = library().bsgm_col_capacity(ctypes.byref(L), ctypes.byref(P))
    if n < 0:
        raise BsgmError(-1, library().bsgm_last_error().decode())
    return n


def pool_blocks(layout, x: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None):
    """Block means of x over real tokens -> float32 [B,H,Nb,64]."""
    n, nb, _ = _dims(layout)
    _expect(x, "x", _tdtype(layout), (layout.batch, layout.heads, n, layout.head_dim))
    _opt(out, "out", torch.float32, (layout.batch, layout.heads, nb, layout.head_dim))
    if out is None:
        out = torch.empty((layout.batch, layout.heads, nb, layout.head_dim), dtype=torch.float32,
                          device=x.device)
    L = c_layout(layout)
    _check(library().bsgm_pool_blocks(ctypes.byref(L), _ptr(x), _ptr(out), _stream(stream)))
    return out


def pool_blocks2(layout, x0: torch.Tensor, x1: torch.Tensor, out0: Optional[torch.Tensor] = None,
                 out1: Optional[torch.Tensor] = None, stream=None):
    """Block means of two tensors (e.g. Q and K) in one launch -> (out0, out1),
    each float32 [B,H,Nb,64]; the same values as two pool_blocks calls."""
    n, nb, _ = _dims(layout)
    mshape = (layout.batch, layout.heads, nb, layout.head_dim)
    outs = []
    for x, name, out, oname in ((x0, "x0", out0, "out0"), (x1, "x1", out1, "out1")):
        _expect(x, name, _tdtype(layout), (layout.batch, layout.heads, n, layout.head_dim))
        _opt(out, oname, torch.float32, mshape)
        outs.append(out if out is not None else
                    torch.empty(mshape, dtype=torch.float32, device=x.device))
    if outs[0].data_ptr() == outs[1].data_ptr():
        raise ValueError("out0 and out1 must be different buffers")
    L = c_layout(layout)
    _check(library().bsgm_pool_blocks2(ctypes.byref(L), _ptr(x0), _ptr(outs[0]), _ptr(x1),
                                       _ptr(outs[1]), _stream(stream)))
    return outs[0], outs[1]


def drift_scores(layout, q, k, v, contrib=None, score=None, workspace=None, stream=None,
                 zmass=None):
    """Drift contributions [B,H,Nb,Nb,64] and their norms [B,H,Nb,Nb] (float32).

    If `zmass` (float32 [B,H,Nb,Nb]) is given it receives each block's normalised
    softmax mass, which the renormalised drift objective needs."""
    n, nb, _ = _dims(layout)
    shape = (layout.batch, layout.heads, n, layout.head_dim)
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _expect(t, name, _tdtype(layout), shape)
    dev = q.device
    _opt(contrib, "contrib", torch.float32, (layout.batch, layout.heads, nb, nb, layout.head_dim))
    _opt(score, "score", torch.float32, (layout.batch, layout.heads, nb, nb))
    if contrib is None:
        contrib = torch.empty((layout.batch, layout.heads, nb, nb, layout.head_dim),
                              dtype=torch.float32, device=dev)
    if score is None:
        score = torch.empty((layout.batch, layout.heads, nb, nb), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(workspace_bytes(layout, DRIFT), dtype=torch.uint8, device=dev)
    L = c_layout(layout)
    if zmass is not None:
        _expect(zmass, "zmass", torch.float32, (layout.batch, layout.heads, nb, nb))
    _check(library().bsgm_drift_scores(ctypes.byref(L), _ptr(q), _ptr(k), _ptr(v), _ptr(contrib),
                                       _ptr(score), _ptr(zmass), *_ws(workspace),
                                       _stream(stream)))
    return contrib, score


def select_blocks(layout, mode: int, keep: Sequence[int], q=None, k=None, contrib=None,
                  cdf_tau: float = 0.9, force: bool = False, swap_rounds: int = 0,
                  objective: int = 0, zmass=None,
                  row_ptr=None, col_idx=None, row_stat=None, scores_out=None, swap_log=None,
                  workspace=None, want_stat: bool = True, stream=None, restoration: int = 0):
    """Selected key blocks as CSR (row_ptr, col_idx) plus the per-row statistic.

    restoration (DRIFT): BEST_SWAP, RERANK or RERANK_TRACK_BEST. swap_log holds
    [rows, swap_rounds, 2] swaps for BEST_SWAP, [rows, swap_rounds + 1,
    ceil(nb / 32)] kept bitmasks for the re-rank rules."""
    n, nb, rows = _dims(layout)
    dev = (q if q is not None else contrib).device
    if mode in (TOPK, CDF):
        shape = (layout.batch, layout.heads, n, layout.head_dim)
        _expect(q, "q", _tdtype(layout), shape)
        _expect(k, "k", _tdtype(layout), shape)
    else:
        _expect(contrib, "contrib", torch.float32,
                (layout.batch, layout.heads, nb, nb, layout.head_dim))
        if zmass is not None:
            _expect(zmass, "zmass", torch.float32, (layout.batch, layout.heads, nb, nb))
    _opt(row_ptr, "row_ptr", torch.int32, (rows + 1,))
    if col_idx is not None:
        _expect_1d(col_idx, "col_idx", torch.int32)
    _opt(row_stat, "row_stat", torch.float32, (rows,))
    _opt(scores_out, "scores_out", torch.float32, (layout.batch, layout.heads, nb, nb))
    if swap_log is not None:
        per_row = swap_rounds * 2 if restoration == BEST_SWAP else \
            (swap_rounds + 1) * ((nb + 31) // 32)
        if not isinstance(swap_log, torch.Tensor) or not swap_log.is_cuda or \
                swap_log.dtype != torch.int32 or not swap_log.is_contiguous() or \
                swap_log.numel() < rows * per_row:
            raise ValueError(f"swap_log must be a contiguous int32 device tensor of at least "
                             f"{rows} x {per_row} elements")
    cap = col_capacity(layout, mode, keep, force)
    if row_ptr is None:
        row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    if row_stat is None and want_stat:
        row_stat = torch.empty(rows, dtype=torch.float32, device=dev)
    if workspace is None and mode != DRIFT:
        workspace = torch.empty(workspace_bytes(layout, mode), dtype=torch.uint8, device=dev)
    L = c_layout(layout)
    P, _keep = c_params(mode, keep, cdf_tau, force, swap_rounds, objective, restoration)
    _check(library().bsgm_select_blocks(
        ctypes.byref(L), ctypes.byref(P), _ptr(q), _ptr(k), _ptr(contrib), _ptr(zmass), _ptr(row_ptr),
        _ptr(col_idx), col_idx.numel(), _ptr(row_stat), _ptr(scores_out), _ptr(swap_log),
        *_ws(workspace), _stream(stream)))
    return row_ptr, col_idx, row_stat


def drift_streamed_workspace_bytes(layout) -> int:
    L = c_layout(layout)
    n = library().bsgm_drift_streamed_workspace_bytes(ctypes.byref(L))
    if n == 0:
        raise BsgmError(1, library().bsgm_last_error().decode())
    return n


def select_drift_streamed(layout, keep: Sequence[int], q, k, v, swap_rounds: int = 5,
                          track_best: bool = True, force: bool = False, row_ptr=None,
                          col_idx=None, row_stat=None, set_log=None, workspace=None,
                          want_stat: bool = True, stream=None):
    """Drift selection by re-rank rounds straight from Q, K and V, without the
    [B,H,Nb,Nb,D] contributions (dropped-sum objective). set_log, when given,
    receives [rows, swap_rounds + 1, ceil(nb / 32)] kept bitmasks."""
    n, nb, rows = _dims(layout)
    shape = (layout.batch, layout.heads, n, layout.head_dim)
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _expect(t, name, _tdtype(layout), shape)
    dev = q.device
    _opt(row_ptr, "row_ptr", torch.int32, (rows + 1,))
    if col_idx is not None:
        _expect_1d(col_idx, "col_idx", torch.int32)
    _opt(row_stat, "row_stat", torch.float32, (rows,))
    if set_log is not None:
        per_row = (swap_rounds + 1) * ((nb + 31) // 32)
        if not isinstance(set_log, torch.Tensor) or not set_log.is_cuda or \
                set_log.dtype != torch.int32 or not set_log.is_contiguous() or \
                set_log.numel() < rows * per_row:
            raise ValueError(f"set_log must be a contiguous int32 device tensor of at least "
                             f"{rows} x {per_row} elements")
    cap = col_capacity(layout, DRIFT, keep, force)
    if row_ptr is None:
        row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    if row_stat is None and want_stat:
        row_stat = torch.empty(rows, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(drift_streamed_workspace_bytes(layout), dtype=torch.uint8,
                                device=dev)
    L = c_layout(layout)
    P, _keep = c_params(DRIFT, keep, 0.9, force, swap_rounds, DROPPED_SUM,
                        RERANK_TRACK_BEST if track_best else RERANK)
    _check(library().bsgm_select_drift_streamed(
        ctypes.byref(L), ctypes.byref(P), _ptr(q), _ptr(k), _ptr(v), _ptr(row_ptr), _ptr(col_idx),
        col_idx.numel(), _ptr(row_stat), _ptr(set_log), *_ws(workspace), _stream(stream)))
    return row_ptr, col_idx, row_stat


def select_blocks_pooled(layout, mode: int, keep: Sequence[int], qbar, kbar, cdf_tau: float = 0.9,
                         force: bool = False, row_ptr=None, col_idx=None, row_stat=None,
                         scores_out=None, workspace=None, want_stat: bool = True, stream=None):
    """TOPK or CDF selection from block means already computed (pool_blocks or pool_blocks2
    of Q and K)."""
    n, nb, rows = _dims(layout)
    pshape = (layout.batch, layout.heads, nb, layout.head_dim)
    _expect(qbar, "qbar", torch.float32, pshape)
    _expect(kbar, "kbar", torch.float32, pshape)
    _opt(row_ptr, "row_ptr", torch.int32, (rows + 1,))
    if col_idx is not None:
        _expect_1d(col_idx, "col_idx", torch.int32)
    _opt(row_stat, "row_stat", torch.float32, (rows,))
    _opt(scores_out, "scores_out", torch.float32, (layout.batch, layout.heads, nb, nb))
    dev = qbar.device
    cap = col_capacity(layout, mode, keep, force)
    if row_ptr is None:
        row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    if row_stat is None and want_stat:
        row_stat = torch.empty(rows, dtype=torch.float32, device=dev)
    if workspace is None and mode == CDF:
        workspace = torch.empty(workspace_bytes(layout, CDF), dtype=torch.uint8, device=dev)
    L = c_layout(layout)
    P, _keep = c_params(mode, keep, cdf_tau, force)
    _check(library().bsgm_select_blocks_pooled(
        ctypes.byref(L), ctypes.byref(P), _ptr(qbar), _ptr(kbar), _ptr(row_ptr), _ptr(col_idx),
        col_idx.numel(), _ptr(row_stat), _ptr(scores_out), *_ws(workspace), _stream(stream)))
    return row_ptr, col_idx, row_stat


NOALLOC_SCRATCH_BYTES = 16 << 20   # BSGM_NOALLOC_SCRATCH_BYTES of the header


def select_blocks_noalloc(layout, mode: int, keep: Sequence[int], q, k, cdf_tau: float = 0.9,
                          force: bool = False, row_ptr=None, col_idx=None, row_stat=None,
                          scores_out=None, want_stat: bool = True, stream=None):
    """TOPK or CDF selection like select_blocks, with the library's own scratch
    array instead of a workspace (the C call allocates nothing; tensors not
    given here are still allocated by this wrapper)."""
    n, nb, rows = _dims(layout)
    shape = (layout.batch, layout.heads, n, layout.head_dim)
    _expect(q, "q", _tdtype(layout), shape)
    _expect(k, "k", _tdtype(layout), shape)
    _opt(row_ptr, "row_ptr", torch.int32, (rows + 1,))
    if col_idx is not None:
        _expect_1d(col_idx, "col_idx", torch.int32)
    _opt(row_stat, "row_stat", torch.float32, (rows,))
    _opt(scores_out, "scores_out", torch.float32, (layout.batch, layout.heads, nb, nb))
    dev = q.device
    cap = col_capacity(layout, mode, keep, force)
    if row_ptr is None:
        row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    if row_stat is None and want_stat:
        row_stat = torch.empty(rows, dtype=torch.float32, device=dev)
    L = c_layout(layout)
    P, _keep = c_params(mode, keep, cdf_tau, force)
    _check(library().bsgm_select_blocks_noalloc(
        ctypes.byref(L), ctypes.byref(P), _ptr(q), _ptr(k), _ptr(row_ptr), _ptr(col_idx),
        col_idx.numel(), _ptr(row_stat), _ptr(scores_out), _stream(stream)))
    return row_ptr, col_idx, row_stat


def fused_workspace_bytes(layout) -> int:
    L = c_layout(layout)
    n = library().bsgm_fused_workspace_bytes(ctypes.byref(L))
    if n == 0:
        raise BsgmError(-1, library().bsgm_last_error().decode())
    return n


def select_blocks_fused(layout, keep: Sequence[int], q, k, force: bool = False,
                        row_ptr=None, col_idx=None, row_stat=None, scores_out=None,
                        workspace=None, want_stat: bool = True, stream=None):
    """TOPK selection with pooling and selection in one launch; same CSR as select_blocks.

    A caller's `workspace` (uint8, >= fused_workspace_bytes) must be zero before its
    first use; every call leaves it ready for the next. None allocates a zeroed one."""
    n, nb, rows = _dims(layout)
    shape = (layout.batch, layout.heads, n, layout.head_dim)
    _expect(q, "q", _tdtype(layout), shape)
    _expect(k, "k", _tdtype(layout), shape)
    _opt(row_ptr, "row_ptr", torch.int32, (rows + 1,))
    if col_idx is not None:
        _expect_1d(col_idx, "col_idx", torch.int32)
    _opt(row_stat, "row_stat", torch.float32, (rows,))
    _opt(scores_out, "scores_out", torch.float32, (layout.batch, layout.heads, nb, nb))
    dev = q.device
    cap = col_capacity(layout, TOPK, keep, force)
    if row_ptr is None:
        row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    if row_stat is None and want_stat:
        row_stat = torch.empty(rows, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.zeros(fused_workspace_bytes(layout), dtype=torch.uint8, device=dev)
    L = c_layout(layout)
    P, _keep = c_params(TOPK, keep, force=force)
    _check(library().bsgm_select_blocks_fused(
        ctypes.byref(L), ctypes.byref(P), _ptr(q), _ptr(k), _ptr(row_ptr), _ptr(col_idx),
        col_idx.numel(), _ptr(row_stat), _ptr(scores_out), *_ws(workspace), _stream(stream)))
    return row_ptr, col_idx, row_stat


def vasc_pairs(layout) -> int:
    """Pairs of adjacent key blocks per (b, h): ceil(Nb / 2)."""
    return (_dims(layout)[1] + 1) // 2


def vasc_select_blocks(layout, keep: Sequence[int], q, k, v, memory, force: bool = False,
                       row_ptr=None, col_idx=None, row_stat=None, demand_out=None,
                       workspace=None, want_stat: bool = True, stream=None):
    """One layer of value-aware selection; updates `memory` (float32
    [B, H, ceil(Nb/2)], zero for a new inference) in place. Returns (row_ptr,
    col_idx, row_stat)."""
    n, nb, rows = _dims(layout)
    shape = (layout.batch, layout.heads, n, layout.head_dim)
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _expect(t, name, _tdtype(layout), shape)
    _expect(memory, "memory", torch.float32, (layout.batch, layout.heads, vasc_pairs(layout)))
    if demand_out is not None:
        _expect(demand_out, "demand_out", torch.float32, (layout.batch, layout.heads, nb, nb))
    dev = q.device
    _opt(row_ptr, "row_ptr", torch.int32, (rows + 1,))
    if col_idx is not None:
        _expect_1d(col_idx, "col_idx", torch.int32)
    _opt(row_stat, "row_stat", torch.float32, (rows,))
    cap = col_capacity(layout, VASC, keep, force)
    if row_ptr is None:
        row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    if row_stat is None and want_stat:
        row_stat = torch.empty(rows, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(workspace_bytes(layout, VASC), dtype=torch.uint8, device=dev)
    L = c_layout(layout)
    P, _keep = c_params(VASC, keep, force=force)
    _check(library().bsgm_vasc_select_blocks(
        ctypes.byref(L), ctypes.byref(P), _ptr(q), _ptr(k), _ptr(v), _ptr(memory), _ptr(row_ptr),
        _ptr(col_idx), col_idx.numel(), _ptr(row_stat), _ptr(demand_out), *_ws(workspace),
        _stream(stream)))
    return row_ptr, col_idx, row_stat


def attn_workspace_bytes(layout) -> int:
    """Scratch of the attention forward's fp16 logits (the fp16 copy of K and two
    int32 flags per (b, h, block)); 0 for fp32 layouts."""
    L = c_layout(layout)
    return int(library().bsgm_attn_workspace_bytes(ctypes.byref(L)))


def attn_prepare(layout, k, workspace, stream=None):
    """The fp16 copy of K into `workspace` (a uint8 tensor of attn_workspace_bytes),
    for a later sparse_attn_fwd(..., workspace=workspace, prepared=True)."""
    n, _, _ = _dims(layout)
    _expect(k, "k", _tdtype(layout), (layout.batch, layout.heads, n, layout.head_dim))
    L = c_layout(layout)
    _check(library().bsgm_attn_prepare(ctypes.byref(L), _ptr(k), *_ws(workspace),
                                       _stream(stream)))


def sparse_attn_fwd(layout, q, k, v, row_ptr, col_idx, o=None, lse=None, want_lse=False,
                    workspace="auto", stream=None, prepared: bool = False):
    """Block-sparse attention forward; returns (o, lse or None).

    workspace: a uint8 tensor of attn_workspace_bytes(layout), "auto" (allocated
    here), or None (bf16 products for the logits, no fp16 copy of K). With a
    workspace, rows whose scaled queries or listed key blocks leave the fp16
    range still take bf16 products. prepared: the workspace already holds the
    fp16 copy of this k (attn_prepare), so the call skips it."""
    if isinstance(workspace, str) and workspace != "auto":
        raise ValueError('workspace must be a tensor, "auto" or None')
    n, nb, rows = _dims(layout)
    shape = (layout.batch, layout.heads, n, layout.head_dim)
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _expect(t, name, _tdtype(layout), shape)
    _expect(row_ptr, "row_ptr", torch.int32, (rows + 1,))
    _expect_1d(col_idx, "col_idx", torch.int32)
    _opt(o, "o", _tdtype(layout), shape)
    _opt(lse, "lse", torch.float32, (layout.batch, layout.heads, n))
    if o is None:
        o = torch.empty(shape, dtype=_tdtype(layout), device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((layout.batch, layout.heads, n), dtype=torch.float32, device=q.device)
    if isinstance(workspace, str):
        nbytes = attn_workspace_bytes(layout)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None
    L = c_layout(layout)
    fn = library().bsgm_sparse_attn_fwd_prepared if prepared else library().bsgm_sparse_attn_fwd
    _check(fn(ctypes.byref(L), _ptr(q), _ptr(k), _ptr(v), _ptr(row_ptr), _ptr(col_idx), _ptr(o),
              _ptr(lse), *_ws(workspace), _stream(stream)))
    return o, lse


def special_rows_workspace_bytes(layout, n_special: int) -> int:
    L = c_layout(layout)
    nbytes = library().bsgm_special_rows_workspace_bytes(ctypes.byref(L), int(n_special))
    if nbytes == 0:
        raise BsgmError(-1, library().bsgm_last_error().decode())
    return nbytes


def special_rows_dense_fwd(layout, q, k, v, n_special: int, o, lse=None, workspace=None,
                           stream=None):
    """Dense attention of the first n_special tokens of every frame, written into
    the matching rows of o (and lse); returns (o, lse)."""
    n, nb, rows = _dims(layout)
    shape = (layout.batch, layout.heads, n, layout.head_dim)
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _expect(t, name, _tdtype(layout), shape)
    _opt(lse, "lse", torch.float32, (layout.batch, layout.heads, n))
    if workspace is None:
        workspace = torch.empty(special_rows_workspace_bytes(layout, n_special), dtype=torch.uint8,
                                device=q.device)
    L = c_layout(layout)
    _check(library().bsgm_special_rows_dense_fwd(
        ctypes.byref(L), _ptr(q), _ptr(k), _ptr(v), int(n_special), _ptr(o), _ptr(lse),
        *_ws(workspace), _stream(stream)))
    return o, lse
