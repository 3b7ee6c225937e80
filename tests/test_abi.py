"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host with the documented codes (no device work involved)."""
import ctypes
import os
import re

import pytest
import torch

import block_sparse_global_mean_amd as bsgm
from block_sparse_global_mean_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "bsgm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsgm_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_symbols() == sorted(bsgm.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = bsgm.library()
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert bsgm.version() == 10600


class L:
    def __init__(self, **kw):
        base = dict(batch=1, heads=2, head_dim=64, frames=4, frame_len=256, frame_valid=250,
                    block=128, dtype="bf16", scale=0.125)
        base.update(kw)
        self.__dict__.update(base)


def ws(layout, mode):
    lib = bsgm.library()
    c = _lib.c_layout(layout)
    return lib.bsgm_workspace_bytes(ctypes.byref(c), mode)


def test_workspace_sizes():
    lay = L()
    rows = 2 * 8
    assert ws(lay, bsgm.TOPK) == 2 * rows * 64 * 4
    nb = 8
    al = lambda x: (x + 255) // 256 * 256
    # pooled q; per (row, block): max and mass; per row: M and 1/Z; per row: the
    # three bf16 terms of the pooled query
    assert ws(lay, bsgm.DRIFT) == (rows * 64 * 4 + al(rows * nb * 8) + al(rows * 8)
                                   + al(rows * 3 * 64 * 2))
    assert ws(lay, bsgm.CDF) == 2 * rows * 64 * 4 + 256 + 256
    # pooled q, k, v; per (b, h) and pair: factor and memory copy; per row and
    # pair: demand and execution (4 pairs of 8 blocks)
    assert ws(lay, bsgm.VASC) == 3 * rows * 64 * 4 + 2 * al(2 * 4 * 4) + 2 * al(rows * 4 * 4)
    assert ws(lay, 7) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=128), -2), (dict(block=32), -2), (dict(frame_len=200, frame_valid=200), -2),
    (dict(frame_valid=100), -2), (dict(frame_valid=0), -1), (dict(frame_valid=300), -1),
    (dict(dtype=5), -1), (dict(scale=0.0), -1), (dict(scale=float("nan")), -1),
    (dict(heads=0), -1), (dict(heads=129), -2),
])
def test_bad_layouts_rejected(kw, code):
    lib = bsgm.library()
    c = _lib.c_layout(L(**kw))
    fake = ctypes.c_void_p(16)
    rc = lib.bsgm_sparse_attn_fwd(ctypes.byref(c), fake, fake, fake, fake, fake, fake, None, None,
                                  0, None)
    assert rc == code, lib.bsgm_last_error()
    assert lib.bsgm_last_error().decode() != ""


def _select(lay, mode=0, keep=(2, 2), force=False, rounds=0, tau=0.9, cap=None, wsb=None,
            q=16, k=16, contrib=None, rp=16, ci=16, objective=0, zmass=None, restoration=0):
    lib = bsgm.library()
    c = _lib.c_layout(lay)
    P, arr = _lib.c_params(mode, keep, tau, force, rounds, objective, restoration)
    need = lib.bsgm_col_capacity(ctypes.byref(c), ctypes.byref(P))
    cap = need if cap is None else cap
    wsb = ws(lay, mode) if wsb is None else wsb
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    rc = lib.bsgm_select_blocks(ctypes.byref(c), ctypes.byref(P), v(q), v(k), v(contrib),
                                v(zmass), v(rp), v(ci), cap, None, None, None, ctypes.c_void_p(16), wsb, None)
    return rc, lib.bsgm_last_error().decode(), need


def test_select_argument_errors():
    lay = L()
    assert _select(lay, keep=(0, 2))[0] == -1
    assert _select(lay, keep=(2, 9))[0] == -1                  # Nb = 8
    assert _select(lay, keep=(2, 2), force=True)[0] == -1      # 4 forced blocks > 2
    rc, msg, need = _select(lay, keep=(3, 5))
    assert need == 8 * 3 + 8 * 5
    assert _select(lay, keep=(3, 5), cap=need - 1)[0] == -3
    assert _select(lay, keep=(3, 5), wsb=100)[0] == -4
    assert _select(lay, mode=1, tau=0.0)[0] == -1
    assert _select(lay, mode=1, tau=1.5)[0] == -1
    assert _select(lay, mode=9)[0] == -1
    assert _select(lay, mode=2, contrib=None)[0] == -1
    assert _select(lay, mode=2, contrib=16, rounds=-1)[0] == -1
    assert _select(lay, mode=2, contrib=16, objective=2, zmass=16)[0] == -1
    assert _select(lay, mode=2, contrib=16, objective=1)[0] == -1       # renormalised needs zmass
    assert _select(lay, q=None)[0] == -1
    assert _select(lay, rp=None)[0] == -1
    big = L(frames=2, frame_len=128 * 2100, frame_valid=128 * 2100)
    assert _select(big, mode=2, keep=(5, 5), contrib=16)[0] == -2      # 4200 blocks > 4096
    wide = L(frames=2, frame_len=128 * 9930, frame_valid=128 * 9930)  # 19860 blocks
    assert _select(wide, mode=2, keep=(5, 5), contrib=16, restoration=bsgm.RERANK)[0] == -2


def _streamed(lay, mode=2, keep=(3, 5), force=False, rounds=2, objective=0,
              restoration=bsgm.RERANK_TRACK_BEST, cap=None, wsb=None, q=16, k=16, v=16, rp=16,
              ci=16, wsp=256):
    lib = bsgm.library()
    c = _lib.c_layout(lay)
    P, arr = _lib.c_params(mode, keep, 0.9, force, rounds, objective, restoration)
    need = lib.bsgm_col_capacity(ctypes.byref(c), ctypes.byref(P))
    cap = need if cap is None else cap
    wsb = lib.bsgm_drift_streamed_workspace_bytes(ctypes.byref(c)) if wsb is None else wsb
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.bsgm_select_drift_streamed(ctypes.byref(c), ctypes.byref(P), p(q), p(k), p(v),
                                          p(rp), p(ci), cap, None, None, p(wsp), wsb, None)


def test_streamed_drift_workspace_and_errors():
    lay = L()                             # 2 heads x 8 blocks: 16 rows
    rows, nb, words = 16, 8, 1
    al = lambda x: (x + 255) // 256 * 256
    groups = 8                            # min(16, nb): the most groups the residual pass uses
    # pooled q and its bf16 terms; per (row, block) two floats (statistics, then
    # the squared scores and the round's dot products); M and 1/Z; the total
    # o = sum_j c_j; the group partials of the residual and its bf16 terms; J^2 and the best J^2; three
    # kept-set bitmasks
    expect = (al(rows * 64 * 4) + al(rows * 192 * 2) + al(rows * nb * 8) + al(rows * 8)
              + al(rows * 64 * 4) + al(rows * groups * 64 * 4) + al(rows * 192 * 2) + 2 * al(rows * 4)
              + 3 * al(rows * words * 4))
    c = _lib.c_layout(lay)
    assert bsgm.library().bsgm_drift_streamed_workspace_bytes(ctypes.byref(c)) == expect
    assert bsgm.drift_streamed_workspace_bytes(lay) == expect
    assert _streamed(lay, keep=(0, 2)) == -1
    assert _streamed(lay, mode=0) == -1
    assert _streamed(lay, restoration=bsgm.BEST_SWAP) == -2
    assert _streamed(lay, objective=1) == -2
    assert _streamed(lay, rounds=-1) == -1
    for name in ("q", "k", "v", "rp", "ci", "wsp"):
        assert _streamed(lay, **{name: None}) == -1, name
    assert _streamed(lay, cap=8 * 3 + 8 * 5 - 1) == -3
    assert _streamed(L(frames=2, frame_len=128 * 19860, frame_valid=128 * 19860)) == -2
    assert _streamed(lay, wsb=expect - 1) == -4


def _fused(lay, mode=0, keep=(2, 2), force=False, cap=None, wsb=None, wsp=256, q=16, k=16,
           rp=16, ci=16):
    lib = bsgm.library()
    c = _lib.c_layout(lay)
    P, arr = _lib.c_params(mode, keep, 0.9, force)
    need = lib.bsgm_col_capacity(ctypes.byref(c), ctypes.byref(P))
    cap = need if cap is None else cap
    wsb = lib.bsgm_fused_workspace_bytes(ctypes.byref(c)) if wsb is None else wsb
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.bsgm_select_blocks_fused(ctypes.byref(c), ctypes.byref(P), v(q), v(k), v(rp), v(ci),
                                        cap, None, None, v(wsp), wsb, None)


def test_fused_select_workspace_and_errors():
    lay = L(batch=3)                      # 3 x 2 (b, h), 8 blocks each, 48 rows
    al = lambda x: (x + 255) // 256 * 256
    assert bsgm.fused_workspace_bytes(lay) == al(128 * (3 + 6 + 16)) + 2 * al(48 * 64 * 4)
    with pytest.raises(bsgm.BsgmError):
        bsgm.fused_workspace_bytes(L(head_dim=32))
    assert _fused(lay, mode=bsgm.CDF) == -2
    assert _fused(lay, mode=bsgm.DRIFT) == -2
    assert _fused(lay, keep=(0, 2)) == -1
    assert _fused(lay, keep=(2, 2), force=True) == -1       # 4 forced blocks > 2
    assert _fused(lay, q=None) == -1
    assert _fused(lay, k=None) == -1
    assert _fused(lay, rp=None) == -1
    assert _fused(lay, ci=None) == -1
    assert _fused(lay, wsp=None) == -1
    assert _fused(lay, wsp=272) == -1                       # not 256-byte aligned
    assert "aligned" in bsgm.library().bsgm_last_error().decode()
    assert _fused(lay, wsb=1000) == -4
    assert _fused(lay, cap=3 * 2 * 8 * 2 - 1) == -3
    big = L(frames=2, frame_len=128 * 2100, frame_valid=128 * 2100)
    assert _fused(big) == -2                                # 4200 blocks > 4096


def test_select_from_pooled_means_errors():
    lay = L(batch=3)
    lib = bsgm.library()
    c = _lib.c_layout(lay)

    def call(mode=0, keep=(2, 2), tau=0.9, qb=16, kb=16, rp=16, ci=16, cap=None, ws=256, wsb=None):
        P, arr = _lib.c_params(mode, keep, tau, False)
        need = lib.bsgm_col_capacity(ctypes.byref(c), ctypes.byref(P))
        cap = need if cap is None else cap
        wsb = ws_(lay, mode) if wsb is None else wsb
        v = lambda x: None if x is None else ctypes.c_void_p(x)
        return lib.bsgm_select_blocks_pooled(ctypes.byref(c), ctypes.byref(P), v(qb), v(kb), v(rp),
                                             v(ci), cap, None, None, v(ws), wsb, None)

    ws_ = lambda lay, mode: ws(lay, mode if mode in (0, 1) else 0)
    assert call(mode=bsgm.DRIFT) == -2
    assert call(mode=bsgm.VASC) == -2
    assert call(qb=None) == -1
    assert call(kb=None) == -1
    assert call(rp=None) == -1
    assert call(ci=None) == -1
    assert call(keep=(0, 2)) == -1
    assert call(cap=3 * 8 * 4 - 1) == -3
    assert call(mode=bsgm.CDF, tau=0.0) == -1
    assert call(mode=bsgm.CDF, ws=None) == -1
    assert call(mode=bsgm.CDF, wsb=10) == -4


def test_noalloc_select_errors():
    """The scratch-array selection checks everything on the host, the scratch
    size first among the workspace checks, before any device call."""
    lib = bsgm.library()

    def call(lay, mode=0, keep=None, tau=0.9, q=16, k=16, rp=16, ci=16, cap=None):
        c = _lib.c_layout(lay)
        keep = [2] * lay.heads if keep is None else keep
        P, arr = _lib.c_params(mode, keep, tau, False)
        need = lib.bsgm_col_capacity(ctypes.byref(c), ctypes.byref(P))
        cap = need if cap is None else cap
        v = lambda x: None if x is None else ctypes.c_void_p(x)
        return lib.bsgm_select_blocks_noalloc(ctypes.byref(c), ctypes.byref(P), v(q), v(k), v(rp),
                                              v(ci), cap, None, None, None)

    lay = L(batch=3)
    assert call(lay, mode=bsgm.DRIFT) == -2
    assert call(lay, mode=bsgm.VASC) == -2
    assert call(lay, q=None) == -1
    assert call(lay, k=None) == -1
    assert call(lay, rp=None) == -1
    assert call(lay, ci=None) == -1
    assert call(lay, keep=(0, 2)) == -1
    assert call(lay, cap=3 * 8 * 4 - 1) == -3
    assert call(lay, mode=bsgm.CDF, tau=1.5) == -1
    # 4 x 16 heads of a 100-frame layer: 4 * 16 * 1100 rows of two 256-byte means
    big = L(batch=4, heads=16, frames=100, frame_len=1408, frame_valid=1374, block=128)
    assert ws(big, bsgm.TOPK) > bsgm.NOALLOC_SCRATCH_BYTES
    assert call(big) == -4
    assert "scratch" in lib.bsgm_last_error().decode()
    one = L(batch=1, heads=16, frames=100, frame_len=1408, frame_valid=1374, block=128)
    assert ws(one, bsgm.CDF) <= bsgm.NOALLOC_SCRATCH_BYTES


def test_noalloc_scratch_size_matches_header():
    text = open(os.path.join(ROOT, "include", "bsgm.h")).read()
    m = re.search(r"#define BSGM_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == bsgm.NOALLOC_SCRATCH_BYTES


def test_col_capacity_and_errors():
    lay = L(batch=3)
    assert bsgm.col_capacity(lay, bsgm.TOPK, [2, 5]) == 3 * 8 * 7
    with pytest.raises(bsgm.BsgmError):
        bsgm.col_capacity(lay, bsgm.TOPK, [0, 5])


def test_pool_and_drift_null_arguments():
    lib = bsgm.library()
    c = _lib.c_layout(L())
    assert lib.bsgm_pool_blocks(ctypes.byref(c), None, ctypes.c_void_p(16), None) == -1
    one = ctypes.c_void_p(16)
    assert lib.bsgm_drift_scores(ctypes.byref(c), one, one, one, None, one, None, one, 1 << 20,
                                 None) == -1
    assert lib.bsgm_drift_scores(ctypes.byref(c), one, one, one, one, one, None, one, 10, None) == -4
    assert lib.bsgm_pool_blocks(None, one, one, None) == -1
    two = ctypes.c_void_p(32)
    assert lib.bsgm_pool_blocks2(ctypes.byref(c), one, two, None, two, None) == -1
    assert lib.bsgm_pool_blocks2(ctypes.byref(c), one, None, one, two, None) == -1
    assert lib.bsgm_pool_blocks2(None, one, two, one, two, None) == -1


def test_attention_workspace():
    lib = bsgm.library()
    lay = L()                                  # 2 heads, 4 x 256 tokens
    c = _lib.c_layout(lay)
    need = lib.bsgm_attn_workspace_bytes(ctypes.byref(c))
    # the fp16 copy of K, then a flag per (b, h, key block) and one per row (16 rows)
    assert need == 2 * 1024 * 64 * 2 + 256 + 256
    assert bsgm.attn_workspace_bytes(L(dtype="f32")) == 0
    one = ctypes.c_void_p(16)
    assert lib.bsgm_sparse_attn_fwd(ctypes.byref(c), one, one, one, one, one, one, None, one,
                                    need - 1, None) == -4
    assert lib.bsgm_sparse_attn_fwd(ctypes.byref(c), one, one, one, one, one, one, None, one,
                                    need, None) == -1          # not 256-byte aligned
    assert "aligned" in lib.bsgm_last_error().decode()
    # the prepared form needs its workspace; the prepare call too
    assert lib.bsgm_sparse_attn_fwd_prepared(ctypes.byref(c), one, one, one, one, one, one, None,
                                             None, 0, None) == -1
    assert lib.bsgm_attn_prepare(ctypes.byref(c), one, None, 0, None) == -1
    assert lib.bsgm_attn_prepare(ctypes.byref(c), one, one, need - 1, None) == -4
    assert lib.bsgm_attn_prepare(ctypes.byref(c), None, one, need, None) == -1
    f32 = _lib.c_layout(L(dtype="f32"))
    assert lib.bsgm_attn_prepare(ctypes.byref(f32), one, None, 0, None) == 0   # nothing to do


def test_vasc_argument_errors():
    lib = bsgm.library()
    lay = L()
    c = _lib.c_layout(lay)
    one = ctypes.c_void_p(16)
    nbytes = ws(lay, bsgm.VASC)

    def call(mode=bsgm.VASC, keep=(3, 3), force=False, q=one, v=one, mem=one, cap=48,
             wsb=nbytes):
        P, arr = _lib.c_params(mode, keep, force=force)
        return lib.bsgm_vasc_select_blocks(ctypes.byref(c), ctypes.byref(P), q, one, v, mem, one,
                                           one, cap, None, None, one, wsb, None)
    assert call(mode=bsgm.TOPK) == -1
    assert call(q=None) == -1 and call(v=None) == -1 and call(mem=None) == -1
    assert call(keep=(0, 3)) == -1
    assert call(keep=(3, 3), force=True) == -1             # 4 forced blocks > 3
    assert call(cap=47) == -3
    assert call(wsb=nbytes - 1) == -4
    P, arr = _lib.c_params(bsgm.VASC, (3, 3))
    assert lib.bsgm_select_blocks(ctypes.byref(c), ctypes.byref(P), one, one, None, None, one, one,
                                  48, None, None, None, one, nbytes, None) == -1
    assert lib.bsgm_last_error().decode() != ""


def test_special_rows_workspace_and_errors():
    lib = bsgm.library()
    lay = L()                                  # 2 heads, 4 frames x 256 (250 real), block 128
    c = _lib.c_layout(lay)
    nbytes = lib.bsgm_special_rows_workspace_bytes(ctypes.byref(c), 5)
    # 4 frames x 5 rows = 20 rows -> one group of 128; chunks of >= 4 of the 8 key blocks
    assert nbytes == 2 * 128 * 64 * 4 * 2 + 2 * 128 * 2 * 4 * 2
    assert lib.bsgm_special_rows_workspace_bytes(ctypes.byref(c), 0) == 0
    assert lib.bsgm_special_rows_workspace_bytes(ctypes.byref(c), 251) == 0
    one = ctypes.c_void_p(16)
    f = lib.bsgm_special_rows_dense_fwd
    assert f(ctypes.byref(c), one, one, one, 5, one, None, one, nbytes - 1, None) == -4
    assert f(ctypes.byref(c), one, one, one, 0, one, None, one, nbytes, None) == -1
    assert f(ctypes.byref(c), None, one, one, 5, one, None, one, nbytes, None) == -1
    assert f(ctypes.byref(c), one, one, one, 5, None, None, one, nbytes, None) == -1
    c32 = _lib.c_layout(L(dtype="f32"))
    assert f(ctypes.byref(c32), one, one, one, 5, one, None, one, nbytes, None) == -2
    assert lib.bsgm_last_error().decode() != ""


def test_workspace_arguments_validated_in_the_binding():
    """A workspace must be a contiguous device tensor; its size is taken in bytes."""
    assert _lib._ws(None) == (None, 0)
    with pytest.raises(ValueError, match="device tensor"):
        _lib._ws(torch.empty(16, dtype=torch.uint8))            # host memory
    q = torch.empty(1)
    with pytest.raises(ValueError, match="auto"):
        bsgm.sparse_attn_fwd(L(), q, q, q, q, q, workspace="yes")
