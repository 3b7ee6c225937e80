"""The allocation-free selection entry point (bsgm_select_blocks_noalloc)
against bsgm_select_blocks, through the C ABI (needs an MI355X).

Two calls in a row share the library's scratch array, the second on a smaller
layout in the other mode, so the second also shows that the first call's
leftovers in the array do not leak into its results. Index work must match bit
for bit; the per-row statistic and the pooled logits too (same kernels).
"""
import sys

import numpy as np
import pytest
import torch

import block_sparse_global_mean_amd as bsgm
import workloads
from workloads import synthetic

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bsgm.library()
    return torch.device("cuda:0")


def to_dev(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def compare(dev, lay, mode, keep, q, k, force, tau, label):
    nb = lay.nblocks
    sc0 = torch.empty((lay.batch, lay.heads, nb, nb), dtype=torch.float32, device=dev)
    sc1 = torch.full_like(sc0, float("nan"))
    rp0, ci0, st0 = bsgm.select_blocks(lay, mode, keep, q=q, k=k, cdf_tau=tau, force=force,
                                       scores_out=sc0)
    rp1 = torch.full_like(rp0, -5)
    ci1 = torch.full_like(ci0, -5)
    st1 = torch.full_like(st0, float("nan"))
    bsgm.select_blocks_noalloc(lay, mode, keep, q, k, cdf_tau=tau, force=force, row_ptr=rp1,
                               col_idx=ci1, row_stat=st1, scores_out=sc1)
    torch.cuda.synchronize()
    nnz = int(rp0[-1].item())
    say(f"{label}: {lay.batch * lay.heads * nb} rows, {nnz} kept blocks")
    assert torch.equal(rp0, rp1), label
    assert torch.equal(ci0[:nnz], ci1[:nnz]), label
    assert torch.equal(st0.view(torch.int32), st1.view(torch.int32)), label
    assert torch.equal(sc0.view(torch.int32), sc1.view(torch.int32)), label


def test_noalloc_selection_two_calls(dev):
    """First the 32-frame layer (16 heads, top-88 with forced special blocks),
    then a smaller ragged layout (2 heads, 8 frames) with the CDF rule."""
    w = workloads.config("vggt_layer_32f_s75")
    data = workloads.generate(w)
    q, k = (to_dev(data[n + "_bits"], dev) for n in ("q", "k"))
    compare(dev, w.layout, bsgm.TOPK, data["keep"], q, k, True, 0.9, "32 frames top-k")
    del q, k
    w2 = synthetic.restrict(workloads.config(1), 2)
    data2 = workloads.generate(workloads.config(1), heads=2)
    q2, k2 = (to_dev(data2[n + "_bits"], dev) for n in ("q", "k"))
    compare(dev, w2.layout, bsgm.CDF, [30, 12], q2, k2, False, 0.5, "8 frames, 2 heads, CDF")


def test_noalloc_rejects_oversized_layout(dev):
    """A layout whose pooled means exceed the array is refused before any work."""
    lay = synthetic.Layout(4, 16, 64, 100, 1408, 1374, 128, "bf16", 0.125)
    assert bsgm.workspace_bytes(lay, bsgm.TOPK) > bsgm.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((4, 16, 140800, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(bsgm.BsgmError, match="scratch"):
        bsgm.select_blocks_noalloc(lay, bsgm.TOPK, [4] * 16, q, q)
    del q
    torch.cuda.synchronize()
