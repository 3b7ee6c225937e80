"""HIP path against the oracle, through the C ABI (needs an MI355X).

Small cases compare every element; the full-size presets run in the launch
configuration that bench.py times and compare sampled rows the oracle computes
one by one. Rules and tolerances are in tests/parity.py.
"""
import dataclasses
import math
import sys
import types

import numpy as np
import pytest
import torch

import block_sparse_global_mean_amd as bsgm
import oracle
import workloads
from workloads import synthetic
import parity

pytestmark = pytest.mark.gpu

_CACHE = {}


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bsgm.library()
    return torch.device("cuda:0")


def to_dev(arr_bits_or_f32, dev):
    a = np.ascontiguousarray(arr_bits_or_f32)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a.astype(np.float32)).to(dev)


def preset(idx, heads=None):
    key = (idx, heads)
    if key not in _CACHE:
        w = workloads.config(idx)
        if heads is not None:
            w = synthetic.restrict(w, heads)
        data = workloads.generate(workloads.config(idx), heads=heads)
        _CACHE[key] = (w, data)
    return _CACHE[key]


def inputs(w, data, dev):
    if w.layout.dtype == "bf16":
        return tuple(to_dev(data[n + "_bits"], dev) for n in ("q", "k", "v"))
    return tuple(to_dev(data[n], dev) for n in ("q", "k", "v"))


def custom_layout(frames, frame_len, frame_valid, block, heads=1, dtype="bf16", batch=1):
    return synthetic.Layout(batch, heads, 64, frames, frame_len, frame_valid, block, dtype, 0.125)


def random_inputs(lay, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    shape = (lay.batch, lay.heads, lay.tokens, lay.head_dim)
    arrs = [rng.standard_normal(shape, dtype=np.float32) * np.float32(scale) for _ in range(3)]
    pad = (np.arange(lay.tokens) % lay.frame_len) >= lay.frame_valid
    for a in arrs:
        a[:, :, pad] = 0
    if lay.dtype == "bf16":
        bits = [workloads.bf16_bits_from_float(a) for a in arrs]
        return bits, [workloads.float_from_bf16_bits(b) for b in bits]
    return arrs, arrs


def oracle_csr_rows(sets):
    return [kept for per_b in sets for per_h in per_b for kept in per_h]


def upload_csr(rows, dev):
    rp = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    ci = np.array([j for r in rows for j in r], dtype=np.int32)
    if ci.size == 0:
        ci = np.zeros(1, dtype=np.int32)
    return torch.from_numpy(rp).to(dev), torch.from_numpy(ci).to(dev)


def assert_outputs(lay, o, o_ref, valid, label):
    ok, worst, err = parity.output_check(o, o_ref, valid, lay.dtype)
    say(f"{label}: max abs err {err:.3e}, worst error / allowance {worst:.3f}")
    assert ok, (label, worst, err)


# --------------------------------------------------------------------------
# pooling
# --------------------------------------------------------------------------
@pytest.mark.parametrize("case", ["tiny_f32", "layer8_2heads", "ragged_bf16_b64", "ragged_f32_b128"])
def test_pool_matches_oracle(dev, case):
    say(f"pool {case}")
    if case == "tiny_f32":
        w, data = preset(0)
        lay, host_in, vals = w.layout, [data["q"]], [data["q"]]
    elif case == "layer8_2heads":
        w, data = preset(1, heads=2)
        lay, host_in, vals = w.layout, [data["q_bits"]], [data["q"]]
    elif case == "ragged_bf16_b64":
        lay = custom_layout(3, 192, 150, 64, heads=2)
        host_in, vals = random_inputs(lay, 1)
    else:
        lay = custom_layout(2, 384, 300, 128, heads=1, dtype="f32")
        host_in, vals = random_inputs(lay, 2)
    x = to_dev(host_in[0], dev)
    got = bsgm.pool_blocks(lay, x).cpu().numpy()
    torch.cuda.synchronize()
    ref = oracle.pool(vals[0], lay)
    np.testing.assert_allclose(got, ref, rtol=0, atol=2e-6 * max(1.0, np.abs(ref).max()))


@pytest.mark.parametrize("case", ["tiny_f32", "ragged_bf16_b64", "ragged_bf16_b128_2batch"])
def test_pool_two_tensors_one_launch(dev, case):
    """pool_blocks2 pools two tensors in one launch: both means equal, bit for
    bit, what two pool_blocks calls write, and match the oracle's means."""
    say(f"pool two tensors {case}")
    if case == "tiny_f32":
        w, data = preset(0)
        lay, host_in, vals = w.layout, [data["q"], data["k"]], [data["q"], data["k"]]
    elif case == "ragged_bf16_b64":
        lay = custom_layout(3, 192, 150, 64, heads=2)
        host_in, vals = random_inputs(lay, 3)
    else:
        lay = custom_layout(2, 384, 300, 128, heads=3, batch=2)
        host_in, vals = random_inputs(lay, 4)
    x0, x1 = to_dev(host_in[0], dev), to_dev(host_in[1], dev)
    m0, m1 = bsgm.pool_blocks2(lay, x0, x1)
    s0, s1 = bsgm.pool_blocks(lay, x0), bsgm.pool_blocks(lay, x1)
    torch.cuda.synchronize()
    assert torch.equal(m0, s0) and torch.equal(m1, s1)
    for got, v in ((m0, vals[0]), (m1, vals[1])):
        ref = oracle.pool(v, lay)
        np.testing.assert_allclose(got.cpu().numpy(), ref, rtol=0,
                                   atol=2e-6 * max(1.0, np.abs(ref).max()))


# --------------------------------------------------------------------------
# pooled top-k selection
# --------------------------------------------------------------------------
def check_topk(lay, vals, keep, force, row_ptr, col_idx, scores_gpu, stat_gpu):
    q, k, v = vals
    nb = lay.nblocks
    parity.check_csr_wellformed(row_ptr, col_idx, nb)
    qbar, kbar = oracle.pool(q, lay), oracle.pool(k, lay)
    s = oracle.pooled_scores(qbar, kbar, lay.scale)
    p = oracle.row_softmax(s)
    np.testing.assert_allclose(scores_gpu, s, rtol=0, atol=2e-5 * max(1.0, np.abs(s).max()))
    forced = oracle.forced_blocks(lay, force)
    rows = parity.csr_rows(row_ptr, col_idx)
    mism = 0
    for b in range(lay.batch):
        for h in range(lay.heads):
            for i in range(nb):
                r = (b * lay.heads + h) * nb + i
                exact = oracle.select_topk_row(s[b, h, i], int(keep[h]), forced)
                if rows[r] != exact:
                    mism += 1
                    assert parity.topk_valid(rows[r], s[b, h, i], int(keep[h]), forced), \
                        f"row {r}: {rows[r]} vs oracle {exact}"
                else:
                    assert abs(stat_gpu[r] - p[b, h, i, exact].sum()) < 1e-4
    return mism


@pytest.mark.parametrize("case", ["tiny_f32", "layer8_2heads", "layer32_forced_1head", "ragged_b64_2batch"])
def test_topk_selection_matches_oracle(dev, case):
    say(f"topk select {case}")
    force = False
    if case == "tiny_f32":
        w, data = preset(0)
        lay, dev_in, vals, keep = w.layout, inputs(w, data, dev), (data["q"], data["k"], data["v"]), data["keep"]
    elif case == "layer8_2heads":
        w, data = preset(1, heads=2)
        lay, dev_in, vals, keep = w.layout, inputs(w, data, dev), (data["q"], data["k"], data["v"]), data["keep"]
    elif case == "layer32_forced_1head":
        w, data = preset(2, heads=1)
        lay, dev_in, vals, keep = w.layout, inputs(w, data, dev), (data["q"], data["k"], data["v"]), data["keep"]
        force = True
    else:
        lay = custom_layout(5, 192, 170, 64, heads=3, batch=2)
        host_in, vals = random_inputs(lay, 3)
        dev_in = tuple(to_dev(x, dev) for x in host_in)
        keep = np.array([1, 7, 15], dtype=np.int32)
        force = False
    nb = lay.nblocks
    scores = torch.empty((lay.batch, lay.heads, nb, nb), dtype=torch.float32, device=dev)
    rp, ci, st = bsgm.select_blocks(lay, bsgm.TOPK, keep, q=dev_in[0], k=dev_in[1], force=force,
                                    scores_out=scores)
    torch.cuda.synchronize()
    mism = check_topk(lay, vals, keep, force, rp.cpu().numpy(), ci.cpu().numpy(),
                      scores.cpu().numpy(), st.cpu().numpy())
    say(f"topk {case}: rows differing from the oracle by near-ties: {mism}")


@pytest.mark.parametrize("nb,keep", [(4095, 700), (2100, 300), (1600, 1), (999, 64), (702, 9)])
def test_topk_selection_wide_rows(dev, nb, keep):
    """Rows of 702 to 4095 key blocks: 11 to 64 blocks per lane of the selection
    wave (every register layout above 8), with 2 heads in one launch."""
    per = nb // 3
    lay = custom_layout(3, 64 * per, 64 * per - 30, 64, heads=2)
    host, vals = random_inputs(lay, 5 + nb)
    dev_in = tuple(to_dev(x, dev) for x in host)
    keeps = np.array([keep, max(1, keep // 2)], dtype=np.int32)
    say(f"topk wide rows: nb {lay.nblocks}, keep {keeps.tolist()}")
    scores = torch.empty((1, lay.heads, lay.nblocks, lay.nblocks), dtype=torch.float32,
                         device=dev)
    rp, ci, st = bsgm.select_blocks(lay, bsgm.TOPK, keeps, q=dev_in[0], k=dev_in[1],
                                    force=True if keep > 3 else False, scores_out=scores)
    torch.cuda.synchronize()
    mism = check_topk(lay, vals, keeps, keep > 3, rp.cpu().numpy(), ci.cpu().numpy(),
                      scores.cpu().numpy(), st.cpu().numpy())
    say(f"topk wide rows: near-tie rows {mism}")


def test_cdf_selection_wide_rows(dev):
    lay = custom_layout(3, 64 * 700, 64 * 700 - 30, 64, heads=1)
    host, vals = planted_peaked(lay, 43)
    keep = np.array([500], dtype=np.int32)
    say(f"cdf wide rows: nb {lay.nblocks}")
    q, k = to_dev(host[0], dev), to_dev(host[1], dev)
    rp, ci, st = bsgm.select_blocks(lay, bsgm.CDF, keep, q=q, k=k, cdf_tau=0.9)
    torch.cuda.synchronize()
    bound, mism = check_cdf(lay, vals, keep, 0.9, False, rp.cpu().numpy(), ci.cpu().numpy(),
                            st.cpu().numpy())
    say(f"cdf wide rows: rows stopped by the threshold {bound}, near-tie rows {mism}")


def test_topk_deterministic(dev):
    w, data = preset(1, heads=2)
    q, k, _ = inputs(w, data, dev)
    a = bsgm.select_blocks(w.layout, bsgm.TOPK, data["keep"], q=q, k=k)
    b = bsgm.select_blocks(w.layout, bsgm.TOPK, data["keep"], q=q, k=k)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("mode", [bsgm.TOPK, bsgm.CDF])
@pytest.mark.parametrize("case", ["layer8_2heads", "ragged_b64_2batch", "layer32_forced"])
def test_select_from_pooled_means(dev, mode, case):
    """Selection from means pooled by separate pool_blocks calls equals the
    pool-and-select call bit for bit (CSR, statistic and scores)."""
    say(f"select from pooled means {case} mode {mode}")
    force = False
    if case == "layer8_2heads":
        w, data = preset(1, heads=2)
        lay, (q, k, _), keep = w.layout, inputs(w, data, dev), data["keep"]
    elif case == "layer32_forced":
        w, data = preset(2)
        lay, (q, k, _), keep = w.layout, inputs(w, data, dev), data["keep"]
        force = True
    else:
        lay = custom_layout(5, 192, 170, 64, heads=3, batch=2)
        host_in, _ = random_inputs(lay, 3)
        q, k = to_dev(host_in[0], dev), to_dev(host_in[1], dev)
        keep = np.array([1, 7, 15], dtype=np.int32)
    nb = lay.nblocks
    sc1 = torch.empty((lay.batch, lay.heads, nb, nb), dtype=torch.float32, device=dev)
    sc2 = torch.full_like(sc1, float("nan"))
    ref = bsgm.select_blocks(lay, mode, keep, q=q, k=k, force=force, cdf_tau=0.9, scores_out=sc1)
    qbar, kbar = bsgm.pool_blocks(lay, q), bsgm.pool_blocks(lay, k)
    got = bsgm.select_blocks_pooled(lay, mode, keep, qbar, kbar, cdf_tau=0.9, force=force,
                                    scores_out=sc2)
    torch.cuda.synchronize()
    nnz = int(ref[0][-1].item())
    assert torch.equal(got[0], ref[0])
    assert torch.equal(got[1][:nnz], ref[1][:nnz])
    assert torch.equal(got[2], ref[2]) and torch.equal(sc2, sc1)


# --------------------------------------------------------------------------
# pooled top-k selection in one launch
# --------------------------------------------------------------------------
def sync_words(lay, ws):
    """The fused workspace's synchronisation area: an unused line, the exit count,
    the error flag, one count per (b, h) and 16 queue tickets, each on a 128-byte
    line (the rest of every line unused)."""
    n = 32 * (3 + lay.batch * lay.heads + 16)
    return ws[:4 * n].view(torch.int32).cpu().numpy()


def fused_vs_two_launch(lay, q, k, keep, force, ws=None, calls=2):
    """Runs the one-launch selection `calls` times on one workspace and the
    two-launch selection once; every output must agree bit for bit, and the
    workspace's synchronisation words must be back at zero after each call."""
    nb = lay.nblocks
    ws = torch.zeros(bsgm.fused_workspace_bytes(lay), dtype=torch.uint8, device=q.device) \
        if ws is None else ws
    sc2 = torch.empty((lay.batch, lay.heads, nb, nb), dtype=torch.float32, device=q.device)
    ref = bsgm.select_blocks(lay, bsgm.TOPK, keep, q=q, k=k, force=force, scores_out=sc2)
    outs = []
    for c in range(calls):
        sc1 = torch.full_like(sc2, float("nan"))
        got = bsgm.select_blocks_fused(lay, keep, q, k, force=force, scores_out=sc1, workspace=ws)
        torch.cuda.synchronize()
        assert not sync_words(lay, ws).any(), f"call {c}: synchronisation words not reset"
        for x, y, name in zip(got + (sc1,), ref + (sc2,), ("row_ptr", "col_idx", "row_stat", "scores")):
            assert torch.equal(x, y), (c, name)
        outs.append(got + (sc1,))
    return outs[-1]


@pytest.mark.parametrize("case", ["tiny_f32", "layer8_2heads", "layer32_forced_1head", "ragged_b64_2batch"])
def test_fused_topk_matches_oracle(dev, case):
    say(f"fused topk select {case}")
    force = False
    if case in ("tiny_f32", "layer8_2heads", "layer32_forced_1head"):
        idx, heads = {"tiny_f32": (0, None), "layer8_2heads": (1, 2), "layer32_forced_1head": (2, 1)}[case]
        w, data = preset(idx, heads=heads)
        lay, dev_in, vals, keep = w.layout, inputs(w, data, dev), (data["q"], data["k"], data["v"]), data["keep"]
        force = case == "layer32_forced_1head"
    else:
        lay = custom_layout(5, 192, 170, 64, heads=3, batch=2)
        host_in, vals = random_inputs(lay, 3)
        dev_in = tuple(to_dev(x, dev) for x in host_in)
        keep = np.array([1, 7, 15], dtype=np.int32)
    rp, ci, st, sc = fused_vs_two_launch(lay, dev_in[0], dev_in[1], keep, force)
    mism = check_topk(lay, vals, keep, force, rp.cpu().numpy(), ci.cpu().numpy(),
                      sc.cpu().numpy(), st.cpu().numpy())
    say(f"fused topk {case}: rows differing from the oracle by near-ties: {mism}")


@pytest.mark.parametrize("nb,keep", [(4095, 700), (999, 64), (702, 9)])
def test_fused_topk_wide_rows(dev, nb, keep):
    per = nb // 3
    lay = custom_layout(3, 64 * per, 64 * per - 30, 64, heads=2)
    host, vals = random_inputs(lay, 5 + nb)
    q, k = to_dev(host[0], dev), to_dev(host[1], dev)
    keeps = np.array([keep, max(1, keep // 2)], dtype=np.int32)
    say(f"fused topk wide rows: nb {lay.nblocks}, keep {keeps.tolist()}")
    rp, ci, st, sc = fused_vs_two_launch(lay, q, k, keeps, keep > 3)
    if nb == 999:
        check_topk(lay, vals, keeps, True, rp.cpu().numpy(), ci.cpu().numpy(), sc.cpu().numpy(),
                   st.cpu().numpy())


def test_fused_topk_layer32_full_size(dev):
    """32 frames, 16 heads, forced special blocks, in the bench's launch
    configuration: one workspace reused over three calls, equal to the
    two-launch selection; sampled rows are valid top-k sets of the oracle's scores."""
    say("fused topk 32 frames full size")
    w, data = preset(2)
    lay = w.layout
    q, k, _ = inputs(w, data, dev)
    rp, ci, st, sc = fused_vs_two_launch(lay, q, k, data["keep"], True, calls=3)
    rpn, cin = rp.cpu().numpy(), ci.cpu().numpy()
    parity.check_csr_wellformed(rpn, cin, lay.nblocks)
    rows = parity.csr_rows(rpn, cin)
    forced = oracle.forced_blocks(lay, True)
    nb = lay.nblocks
    for h in (0, 9, 15):
        qbar = oracle.pool(data["q"][:, h:h + 1], lay)[0, 0]
        kbar = oracle.pool(data["k"][:, h:h + 1], lay)[0, 0]
        for i in (0, 10, 177, 351):
            s = lay.scale * (kbar @ qbar[i])
            assert parity.topk_valid(rows[h * nb + i], s, 88, forced), (h, i)


def test_fused_topk_graph_replay(dev):
    """The one-launch selection captured in a HIP graph and replayed: its
    synchronisation words reset inside every replay, so each replay reproduces
    the eager result and leaves them zero."""
    w, data = preset(1, heads=2)
    lay = w.layout
    q, k, _ = inputs(w, data, dev)
    keep = data["keep"]
    rows = lay.heads * lay.nblocks
    cap = bsgm.col_capacity(lay, bsgm.TOPK, keep, force=True)
    rp = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    ci = torch.empty(cap, dtype=torch.int32, device=dev)
    ws = torch.zeros(bsgm.fused_workspace_bytes(lay), dtype=torch.uint8, device=dev)

    def step():
        bsgm.select_blocks_fused(lay, keep, q, k, force=True, row_ptr=rp, col_idx=ci,
                                 workspace=ws, want_stat=False)

    ref = bsgm.select_blocks(lay, bsgm.TOPK, keep, q=q, k=k, force=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        rp.zero_()
        ci.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(rp, ref[0]) and torch.equal(ci, ref[1]), rep
        assert not sync_words(lay, ws).any(), rep
    say("fused graph replay: 3 replays equal to the two-launch selection")


# --------------------------------------------------------------------------
# attention on the oracle's CSR
# --------------------------------------------------------------------------
def run_attention_case(dev, lay, host_in, vals, rows, label, workspace="auto"):
    """workspace "auto": the scaled-f16 logits (with a workspace), None: bf16."""
    say(f"attention {label} ({'bf16' if workspace is None else 'f16'} logits)")
    q, k, v = (to_dev(x, dev) for x in host_in)
    rp, ci = upload_csr(rows, dev)
    o, lse = bsgm.sparse_attn_fwd(lay, q, k, v, rp, ci, want_lse=True, workspace=workspace)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    row_ptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])])
    col_idx = np.array([j for r in rows for j in r], dtype=np.int64)
    o_ref, lse_ref = oracle.sparse_attention(vals[0], vals[1], vals[2], lay, row_ptr, col_idx)
    valid = oracle.valid_mask(lay)
    assert_outputs(lay, o, o_ref, valid, f"attention {label}")
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin)
    lse_tol = 1e-4 if lay.dtype == "f32" else 2e-3
    assert np.abs(lse[fin] - lse_ref[fin]).max() <= lse_tol * max(1.0, np.abs(lse_ref[fin]).max())
    assert np.all(o[..., ~valid, :] == 0)
    return o, lse


def sweep_case(seed):
    """Seeded random layout for the end-to-end sweep: frames, frame length (whole
    blocks), ragged valid length (padding under one block, as the library
    requires), block 64 or 128, fp32 or bf16, batch, heads, per-head budgets
    (at least the forced blocks, as the library requires), forced blocks, TOPK
    or CDF."""
    rng = np.random.default_rng(1000 + seed)
    block = (64, 128)[seed % 2]
    dtype = "f32" if seed % 3 == 0 else "bf16"
    mode = bsgm.CDF if seed % 4 == 3 else bsgm.TOPK
    frames = int(rng.integers(2, 11))
    frame_len = block * int(rng.integers(1, 7))
    frame_valid = frame_len - int(rng.integers(0, block))   # padding under a block (no empty blocks)
    heads = int(rng.integers(1, 4))
    batch = 1 if mode == bsgm.CDF else int(rng.integers(1, 3))
    lay = custom_layout(frames, frame_len, frame_valid, block, heads=heads, dtype=dtype, batch=batch)
    force = bool(rng.integers(0, 2))
    lo = max(1, len(oracle.forced_blocks(lay, force)))   # the budget covers the forced blocks
    keep = np.array([int(rng.integers(lo, lay.nblocks + 1)) for _ in range(heads)], dtype=np.int32)
    tau = float(rng.uniform(0.5, 0.97))
    return lay, mode, force, keep, tau


@pytest.mark.parametrize("seed", range(16))
def test_end_to_end_random_layouts(dev, seed):
    """Selection then attention on seeded random layouts (see sweep_case): every
    row's list is a valid answer of its rule against the oracle's pooled scores,
    and every output row equals the oracle's attention over the GPU's own list."""
    lay, mode, force, keep, tau = sweep_case(seed)
    say(f"sweep seed {seed}: frames {lay.frames}x{lay.frame_len} ({lay.frame_valid} real), block "
        f"{lay.block}, {lay.dtype}, batch {lay.batch}, heads {lay.heads}, "
        f"{'CDF' if mode == bsgm.CDF else 'TOPK'}, keep {keep.tolist()}, force {force}")
    host_in, vals = random_inputs(lay, 2000 + seed)
    q, k, v = (to_dev(x, dev) for x in host_in)
    nb = lay.nblocks
    if mode == bsgm.TOPK:
        scores = torch.empty((lay.batch, lay.heads, nb, nb), dtype=torch.float32, device=dev)
        rp, ci, st = bsgm.select_blocks(lay, bsgm.TOPK, keep, q=q, k=k, force=force,
                                        scores_out=scores)
        torch.cuda.synchronize()
        check_topk(lay, vals, keep, force, rp.cpu().numpy(), ci.cpu().numpy(),
                   scores.cpu().numpy(), st.cpu().numpy())
    else:
        rp, ci, st = bsgm.select_blocks(lay, bsgm.CDF, keep, q=q, k=k, cdf_tau=tau, force=force)
        torch.cuda.synchronize()
        check_cdf(lay, vals, keep, tau, force, rp.cpu().numpy(), ci.cpu().numpy(),
                  st.cpu().numpy())
    rows = parity.csr_rows(rp.cpu().numpy(), ci.cpu().numpy())
    run_attention_case(dev, lay, host_in, vals, rows, f"sweep seed {seed}",
                       workspace="auto" if seed % 2 == 0 else None)


def test_binding_rejects_bad_buffers(dev):
    """Host, mistyped or misshaped buffers are refused before anything is enqueued."""
    w, data = preset(0)
    lay = w.layout
    q, k, v = (torch.from_numpy(data[n]).to(dev) for n in ("q", "k", "v"))
    nb, rows = lay.nblocks, lay.heads * lay.nblocks
    rp = torch.zeros(rows + 1, dtype=torch.int32, device=dev)
    ci = torch.zeros(1, dtype=torch.int32, device=dev)
    with pytest.raises(ValueError, match="row_ptr"):
        bsgm.sparse_attn_fwd(lay, q, k, v, rp.cpu(), ci)
    with pytest.raises(ValueError, match="col_idx"):
        bsgm.sparse_attn_fwd(lay, q, k, v, rp, ci.to(torch.int64))
    with pytest.raises(ValueError, match="lse"):
        bsgm.sparse_attn_fwd(lay, q, k, v, rp, ci, lse=torch.empty(3, device=dev))
    with pytest.raises(ValueError, match="workspace"):
        bsgm.sparse_attn_fwd(lay, q, k, v, rp, ci, workspace=torch.empty(8, dtype=torch.uint8))
    with pytest.raises(ValueError, match="scores_out"):
        bsgm.select_blocks(lay, bsgm.TOPK, data["keep"], q=q, k=k,
                           scores_out=torch.empty((1, lay.heads, nb, nb), dtype=torch.float64,
                                                  device=dev))
    with pytest.raises(ValueError, match="swap_log"):
        bsgm.select_blocks(lay, bsgm.TOPK, data["keep"], q=q, k=k, swap_rounds=2,
                           swap_log=torch.empty((rows, 1, 2), dtype=torch.int32, device=dev))
    torch.cuda.synchronize()


def test_attention_tiny_f32(dev):
    w, data = preset(0)
    vals = (data["q"], data["k"], data["v"])
    sets, _ = oracle.select(*vals, w.layout, oracle.TOPK, data["keep"])
    run_attention_case(dev, w.layout, vals, vals, oracle_csr_rows(sets), "tiny f32 top-4")


@pytest.mark.parametrize("workspace", ["auto", None])
def test_attention_layer8_2heads(dev, workspace):
    w, data = preset(1, heads=2)
    vals = (data["q"], data["k"], data["v"])
    sets, _ = oracle.select(*vals, w.layout, oracle.TOPK, data["keep"])
    host = (data["q_bits"], data["k_bits"], data["v_bits"])
    run_attention_case(dev, w.layout, host, vals, oracle_csr_rows(sets), "8 frames, 2 heads, 50%",
                       workspace)


@pytest.mark.parametrize("dtype,block,workspace", [("bf16", 64, "auto"), ("bf16", 128, "auto"),
                                                   ("bf16", 128, None), ("f32", 64, "auto"),
                                                   ("f32", 128, "auto")])
def test_attention_ragged_random_lists(dev, dtype, block, workspace):
    """Random kept lists (including empty rows and the partial last block of
    each frame) on a ragged layout with two batch entries."""
    lay = custom_layout(3, 2 * block, 2 * block - 37, block, heads=2, dtype=dtype, batch=2)
    host, vals = random_inputs(lay, 11 + block)
    nb = lay.nblocks
    rng = np.random.default_rng(5)
    rows = []
    for r in range(lay.batch * lay.heads * nb):
        n = int(rng.integers(0, nb + 1)) if r % 7 else 0
        rows.append(sorted(rng.choice(nb, size=n, replace=False).tolist()))
    run_attention_case(dev, lay, host, vals, rows, f"ragged {dtype} block {block}", workspace)


@pytest.mark.parametrize("dtype,block", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_attention_long_rows(dev, dtype, block):
    """Kept lists longer than 512, 1024 and 1536 blocks (the kernels buffer a
    row's column list in pieces), checked row by row against the oracle."""
    lay = custom_layout(85 * block // 64, 20 * 64, 20 * 64 - 30, block, heads=1, dtype=dtype)
    host, vals = random_inputs(lay, 41 + block)
    nb = lay.nblocks
    rng = np.random.default_rng(8)
    lengths = {3: min(nb, 1100), 7: min(nb, 1600), nb // 2: nb, nb - 1: 513, 11: 1025}
    rows = []
    for i in range(nb):
        n = lengths.get(i, 2)
        rows.append(sorted(rng.choice(nb, size=n, replace=False).tolist()))
    say(f"attention long rows {dtype} block {block}: nb {nb}, lengths {sorted(lengths.values())}")
    q, k, v = (to_dev(x, dev) for x in host)
    rp, ci = upload_csr(rows, dev)
    o, lse = bsgm.sparse_attn_fwd(lay, q, k, v, rp, ci, want_lse=True)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()[0, 0]
    lse = lse.cpu().numpy()[0, 0]
    for i in sorted(set(lengths) | {0, 1}):
        ob, lb = oracle.sparse_attention_row(vals[0][0, 0], vals[1][0, 0], vals[2][0, 0], lay, i,
                                             rows[i])
        sl = slice(i * block, (i + 1) * block)
        valid = np.isfinite(lb)
        assert valid.any()
        full_valid = oracle.valid_mask(lay)[sl]
        assert np.array_equal(valid, full_valid)
        ok, worst, err = parity.output_check(o[sl], ob, valid, lay.dtype)
        say(f"  row {i} ({len(rows[i])} blocks): max abs err {err:.3e}, worst/allowance {worst:.3f}")
        assert ok, (i, worst, err)
        lse_tol = 1e-4 if dtype == "f32" else 2e-3
        assert np.abs(lse[sl][valid] - lb[valid]).max() <= lse_tol * max(1.0, np.abs(lb[valid]).max())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attention_all_kept_is_dense(dev, dtype):
    lay = custom_layout(2, 256, 200, 128, heads=2, dtype=dtype)
    host, vals = random_inputs(lay, 21)
    nb = lay.nblocks
    rows = [list(range(nb))] * (lay.heads * nb)
    o, lse = run_attention_case(dev, lay, host, vals, rows, f"all kept {dtype}")
    od, lsed = oracle.dense_attention(*vals, lay)
    valid = oracle.valid_mask(lay)
    assert_outputs(lay, o, od, valid, f"all kept vs dense {dtype}")


def test_attention_constant_values_and_lse_merge(dev):
    lay = custom_layout(2, 256, 230, 128, heads=1)
    host, vals = random_inputs(lay, 31)
    nb = lay.nblocks
    q, k, _ = (to_dev(x, dev) for x in host)
    ones = torch.ones_like(q)
    rng = np.random.default_rng(6)
    rows_s = [sorted(rng.choice(nb, size=2, replace=False).tolist()) for _ in range(nb)]
    rows_d = [sorted(set(range(nb)) - set(s)) for s in rows_s]
    rp, ci = upload_csr(rows_s, dev)
    o1, _ = bsgm.sparse_attn_fwd(lay, q, k, ones, rp, ci)
    valid = torch.from_numpy(oracle.valid_mask(lay)).to(dev)
    assert torch.all((o1.float()[0, 0, valid] - 1).abs() <= 2 ** -7)
    v = to_dev(host[2], dev)
    os_, ls_ = bsgm.sparse_attn_fwd(lay, q, k, v, rp, ci, want_lse=True)
    rp2, ci2 = upload_csr(rows_d, dev)
    od_, ld_ = bsgm.sparse_attn_fwd(lay, q, k, v, rp2, ci2, want_lse=True)
    rp3, ci3 = upload_csr([list(range(nb))] * nb, dev)
    oa_, la_ = bsgm.sparse_attn_fwd(lay, q, k, v, rp3, ci3, want_lse=True)
    torch.cuda.synchronize()
    ws, wd = ls_[0, 0, valid].exp()[:, None], ld_[0, 0, valid].exp()[:, None]
    merged = (ws * os_.float()[0, 0, valid] + wd * od_.float()[0, 0, valid]) / (ws + wd)
    ref = oa_.float()[0, 0, valid]
    allow = 2 * 2e-2 * ref.pow(2).mean(dim=-1).sqrt()
    assert bool(((merged - ref).abs().max(dim=-1).values <= allow).all())
    assert float((torch.logaddexp(ls_, ld_)[0, 0, valid] - la_[0, 0, valid]).abs().max()) <= 2e-3


@pytest.mark.parametrize("dtype,block,workspace", [("bf16", 128, "auto"), ("bf16", 64, "auto"),
                                                   ("bf16", 128, None)])
def test_attention_growing_logits(dev, dtype, block, workspace):
    """Key blocks whose logits grow along the list by up to ~60 (moderate) and
    ~330 (past the rescale bound of a 2^64 softmax weight) in log2 units over
    the first kept block: every row must still match the float64 softmax."""
    lay = custom_layout(2, 4 * block, 4 * block - 20, block, heads=2, dtype=dtype)
    nb, N, D = lay.nblocks, lay.tokens, lay.head_dim
    rng = np.random.default_rng(91 + block)
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    q = np.zeros((1, 2, N, D), np.float32)
    k = np.zeros_like(q)
    blk_of = np.arange(N) // block
    for h, top in enumerate((40.0, 220.0)):      # logit of the last block: scale * 8 * top
        q[0, h] = 8.0 * u[None, :] + 0.05 * rng.standard_normal((N, D))
        growth = np.linspace(0.2, top, nb)[blk_of]
        k[0, h] = growth[:, None] * u[None, :] + 0.05 * rng.standard_normal((N, D))
    v = rng.standard_normal(q.shape).astype(np.float32)
    pad = (np.arange(N) % lay.frame_len) >= lay.frame_valid
    for a_ in (q, k, v):
        a_[:, :, pad] = 0
    if dtype == "bf16":
        host = [workloads.bf16_bits_from_float(a_) for a_ in (q, k, v)]
        vals = [workloads.float_from_bf16_bits(b) for b in host]
    else:
        host = vals = [q, k, v]
    rows = [list(range(nb)) for _ in range(lay.heads * nb)]
    o, lse = run_attention_case(dev, lay, host, vals, rows, f"growing logits {dtype} block {block}",
                                workspace)
    assert np.all(np.isfinite(o))


@pytest.mark.parametrize("block", [128, 64])
def test_attention_outside_fp16_range(dev, block):
    """Key block 0 of head 1 holds a key beyond the fp16 range and query block 1
    of head 0 a scaled query beyond it. Rows whose scaled Q or one of whose
    listed key blocks leaves the range take bf16 products, the rest fp16 ones:
    the flags in the workspace must route exactly those rows, and every row
    must match the float64 softmax."""
    lay = custom_layout(2, 3 * block, 3 * block - 20, block, heads=2, dtype="bf16")
    rng = np.random.default_rng(7 + block)
    shape = (1, 2, lay.tokens, 64)
    q = (rng.standard_normal(shape) * 0.5).astype(np.float32)
    k = (rng.standard_normal(shape) * 0.5).astype(np.float32)
    v = rng.standard_normal(shape).astype(np.float32)
    k[0, 1, 5, 3] = 9.0e4                 # |k| > 65504 in key block 0 of head 1
    q[0, 0, block + 3, 7] = 4.0e5         # |q * scale * log2 e| > 65504 in query block 1
    pad = (np.arange(lay.tokens) % lay.frame_len) >= lay.frame_valid
    for a_ in (q, k, v):
        a_[:, :, pad] = 0
    host = [workloads.bf16_bits_from_float(a_) for a_ in (q, k, v)]
    vals = [workloads.float_from_bf16_bits(b) for b in host]
    nb = lay.nblocks
    rows = [list(range(nb)) for _ in range(nb)]                       # head 0: everything
    rows += [list(range(nb)) if i % 2 == 0 else list(range(1, nb)) for i in range(nb)]
    want_redo = [int(i == 1) for i in range(nb)] + [int(i % 2 == 0) for i in range(nb)]
    nbytes = bsgm.attn_workspace_bytes(lay)
    ws = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device=dev)   # stale contents
    run_attention_case(dev, lay, host, vals, rows, f"outside the fp16 range block {block}", ws)
    al = lambda x: (x + 255) // 256 * 256
    off = al(lay.tokens * lay.heads * 64 * 2)
    flags = ws.cpu().numpy()[off:].view(np.int32)
    kbad, redo = flags[:2 * nb], flags[al(2 * nb * 4) // 4:][:2 * nb]
    assert kbad.tolist() == [0] * nb + [1] + [0] * (nb - 1)
    assert redo.tolist() == want_redo


@pytest.mark.parametrize("block", [128, 64])
def test_attention_fp16_form_small_keys(dev, block):
    """The fp16-logit form where fp16 loses bits: every key of head 0 is near
    2^-20 (below 2^-17 a bf16 value is not exact in fp16), query block 1 of
    head 0 scales to |q * scale * log2 e| = 6e4 (near the top of the fp16
    range) and query block 3 to 100; key block 4 of head 1 holds a key of 200.
    The form's error bound holds only below 128 in both, so query block 1 and
    the head-1 rows that list key block 4 must be routed to the bf16 form, query
    block 3 must stay on the fp16 form, and every row must match the float64
    softmax."""
    lay = custom_layout(2, 3 * block, 3 * block - 20, block, heads=2, dtype="bf16")
    rng = np.random.default_rng(29 + block)
    shape = (1, 2, lay.tokens, 64)
    c = lay.scale * 1.4426950408889634
    q = (rng.standard_normal(shape) * 0.5).astype(np.float32)
    k = (rng.standard_normal(shape) * 0.5).astype(np.float32)
    v = rng.standard_normal(shape).astype(np.float32)
    k[0, 0] = (rng.uniform(0.5, 1.5, (lay.tokens, 64)) * 2.0 ** -20 *
               rng.choice([-1.0, 1.0], (lay.tokens, 64))).astype(np.float32)
    sign = rng.choice([-1.0, 1.0], (block, 64))
    q[0, 0, block:2 * block] = (6.0e4 / c * sign).astype(np.float32)
    q[0, 0, 3 * block:4 * block] = (100.0 / c * sign).astype(np.float32)
    k[0, 1, 4 * block + 7, 11] = 200.0
    pad = (np.arange(lay.tokens) % lay.frame_len) >= lay.frame_valid
    for a_ in (q, k, v):
        a_[:, :, pad] = 0
    host = [workloads.bf16_bits_from_float(a_) for a_ in (q, k, v)]
    vals = [workloads.float_from_bf16_bits(b) for b in host]
    kv = vals[1][0, 0][~pad]
    tiny = np.abs(kv) < 2.0 ** -17
    assert tiny.mean() > 0.9 and np.any(kv[tiny] != kv[tiny].astype(np.float16))
    nb = lay.nblocks
    rows = [list(range(nb)) for _ in range(nb)]                       # head 0: everything
    rows += [list(range(nb)) if i % 2 == 0 else [j for j in range(nb) if j != 4]
             for i in range(nb)]
    want_redo = [int(i == 1) for i in range(nb)] + [int(i % 2 == 0) for i in range(nb)]
    nbytes = bsgm.attn_workspace_bytes(lay)
    ws = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device=dev)   # stale contents
    run_attention_case(dev, lay, host, vals, rows, f"fp16 form with small keys block {block}", ws)
    al = lambda x: (x + 255) // 256 * 256
    off = al(lay.tokens * lay.heads * 64 * 2)
    flags = ws.cpu().numpy()[off:].view(np.int32)
    kbad, redo = flags[:2 * nb], flags[al(2 * nb * 4) // 4:][:2 * nb]
    assert nb == 6 and kbad.tolist() == [0] * nb + [0, 0, 0, 0, 1, 0]
    assert redo.tolist() == want_redo


# --------------------------------------------------------------------------
# CDF selection
# --------------------------------------------------------------------------
def check_cdf(lay, vals, keep, tau, force, row_ptr, col_idx, stat_gpu, rows_to_check=None):
    """Every row (or, with rows_to_check = {head: rows}, the given rows of the
    given heads) is a valid CDF-under-cap answer with the oracle's kept mass."""
    q, k, _ = vals
    nb = lay.nblocks
    parity.check_csr_wellformed(row_ptr, col_idx, nb)
    rows = parity.csr_rows(row_ptr, col_idx)
    forced = oracle.forced_blocks(lay, force)
    bound_by_cdf = 0
    mism = 0
    heads = range(lay.heads) if rows_to_check is None else sorted(rows_to_check)
    for h in heads:
        qbar = oracle.pool(q[:, h:h + 1], lay)[0, 0]
        kbar = oracle.pool(k[:, h:h + 1], lay)[0, 0]
        for i in (range(nb) if rows_to_check is None else rows_to_check[h]):
            r = h * nb + i
            s = lay.scale * (kbar @ qbar[i])
            p = oracle.row_softmax(s)
            exact = oracle.select_cdf_row(s, p, tau, int(keep[h]), forced)
            if len(exact) < keep[h]:
                bound_by_cdf += 1
            if rows[r] != exact:
                mism += 1
                assert parity.cdf_valid(rows[r], s, p, tau, int(keep[h]), forced), \
                    f"row {r}: {rows[r]} vs oracle {exact}"
            else:
                assert abs(stat_gpu[r] - p[exact].sum()) < 1e-4
    return bound_by_cdf, mism


def planted_peaked(lay, seed):
    """Pooled scores with a few dominant key blocks per row, so that the
    cumulative-mass rule stops before the cap."""
    rng = np.random.default_rng(seed)
    N, D = lay.tokens, lay.head_dim
    u = rng.standard_normal(D).astype(np.float32)
    u /= np.linalg.norm(u)
    nb = lay.nblocks
    qs = (rng.standard_normal((lay.heads, nb)) * 2).astype(np.float32)
    ks = (rng.standard_normal((lay.heads, nb)) * 4).astype(np.float32)
    q = np.zeros((1, lay.heads, N, D), np.float32)
    k = np.zeros_like(q)
    for h in range(lay.heads):
        q[0, h] = np.repeat(qs[h], lay.block)[:, None] * u[None, :] * 4
        k[0, h] = np.repeat(ks[h], lay.block)[:, None] * u[None, :] * 4
    q += rng.standard_normal(q.shape).astype(np.float32) * 0.3
    k += rng.standard_normal(k.shape).astype(np.float32) * 0.3
    v = rng.standard_normal(q.shape).astype(np.float32)
    pad = (np.arange(N) % lay.frame_len) >= lay.frame_valid
    for a in (q, k, v):
        a[:, :, pad] = 0
    bits = [workloads.bf16_bits_from_float(a) for a in (q, k, v)]
    return bits, [workloads.float_from_bf16_bits(b) for b in bits]


@pytest.mark.parametrize("force", [False, True])
def test_cdf_selection_planted(dev, force):
    say(f"cdf planted force={force}")
    lay = synthetic.restrict(workloads.config(1), 3).layout
    host, vals = planted_peaked(lay, 41)
    keep = np.array([44, 30, 12], dtype=np.int32)
    q, k = to_dev(host[0], dev), to_dev(host[1], dev)
    rp, ci, st = bsgm.select_blocks(lay, bsgm.CDF, keep, q=q, k=k, cdf_tau=0.9, force=force)
    torch.cuda.synchronize()
    bound, mism = check_cdf(lay, vals, keep, 0.9, force, rp.cpu().numpy(), ci.cpu().numpy(),
                            st.cpu().numpy())
    say(f"cdf planted: rows stopped by the threshold {bound}, near-tie rows {mism}")
    assert bound > 0


def xcd_boundary_rows(nb):
    """Query blocks at the edges of the eighths that the attention grid hands to
    the eight XCDs (i = x * ceil(nb / 8)) and their neighbours."""
    c = (nb + 7) // 8
    rows = set()
    for x in range(8):
        for i in (x * c - 1, x * c, x * c + 1):
            if 0 <= i < nb:
                rows.add(i)
    rows.update((nb - 2, nb - 1))
    return sorted(rows)


def spread_rows(nb, count):
    """The XCD boundary rows plus evenly spaced rows, ``count`` or more in all."""
    rows = set(xcd_boundary_rows(nb))
    extra = max(0, count - len(rows))
    rows.update(int(x) for x in np.linspace(0, nb - 1, extra + 2).round())
    return sorted(rows)


def test_cdf_selection_layer100_sampled(dev):
    """100 frames, 16 heads, per-head caps: the bench launch. On the heads with
    the smallest, a middle and the largest cap, 64 or more rows each (XCD
    boundary rows included): the list is a valid CDF-under-cap answer, and the
    output equals the oracle's attention over that same list."""
    say("cdf 100 frames full size")
    w, data = preset(3)
    lay = w.layout
    q, k, v = inputs(w, data, dev)
    rp, ci, st = bsgm.select_blocks(lay, bsgm.CDF, data["keep"], q=q, k=k, cdf_tau=w.cdf_tau)
    o, _ = bsgm.sparse_attn_fwd(lay, q, k, v, rp, ci)
    torch.cuda.synchronize()
    rpn, cin = rp.cpu().numpy(), ci.cpu().numpy()
    keep = np.asarray(data["keep"])
    order = np.argsort(keep, kind="stable")
    heads = sorted({int(order[0]), int(order[len(order) // 2]), int(order[-1])})
    rows = spread_rows(lay.nblocks, 64)
    say(f"cdf 100 frames: heads {heads} (caps {[int(keep[h]) for h in heads]}), "
        f"{len(rows)} rows each")
    check_cdf(lay, (data["q"], data["k"], None), keep, w.cdf_tau, False, rpn, cin,
              st.cpu().numpy(), rows_to_check={h: rows for h in heads})
    check_sampled_attention(lay, data, o, rpn, cin, [(h, i) for h in heads for i in rows])


def check_sampled_attention(lay, data, o_gpu, rpn, cin, samples):
    """The output of every sampled row (h, i) against the oracle's attention
    over the GPU's own list of that row, which the caller has already accepted
    under the selection rule. No row is skipped."""
    rows = parity.csr_rows(rpn, cin)
    nb, bk = lay.nblocks, lay.block
    valid_all = oracle.valid_mask(lay)
    worst = 0.0
    for h, i in samples:
        kept = rows[h * nb + i]
        o_ref, _ = oracle.sparse_attention_row(data["q"][0, h], data["k"][0, h], data["v"][0, h],
                                               lay, i, kept)
        og = o_gpu[0, h, i * bk:(i + 1) * bk].float().cpu().numpy()
        ok, w_, err = parity.output_check(og, o_ref, valid_all[i * bk:(i + 1) * bk], lay.dtype)
        worst = max(worst, w_)
        assert ok, (f"sampled row (h={h}, i={i})", w_, err)
    say(f"sampled outputs: {len(samples)} rows, worst error / allowance {worst:.3f}")


@pytest.mark.parametrize("workspace", ["auto", None])
def test_topk_layer32_full_size_sampled(dev, workspace):
    """32 frames, 16 heads, 75 % sparse with forced special blocks: the bench
    launch (select + attention, fp16 logits with a workspace, else bf16).
    Heads 0 and 15 are checked on every query block (so every XCD boundary of
    the attention grid), head 5 on sampled rows: each list is a valid top-k
    answer, and each output equals the oracle's attention over that list."""
    say(f"topk 32 frames full size, attention workspace {workspace}")
    w, data = preset(2)
    lay = w.layout
    q, k, v = inputs(w, data, dev)
    rp, ci, st = bsgm.select_blocks(lay, bsgm.TOPK, data["keep"], q=q, k=k, force=True)
    o, _ = bsgm.sparse_attn_fwd(lay, q, k, v, rp, ci, workspace=workspace)
    torch.cuda.synchronize()
    rpn, cin = rp.cpu().numpy(), ci.cpu().numpy()
    parity.check_csr_wellformed(rpn, cin, lay.nblocks)
    assert rpn[-1] == lay.heads * lay.nblocks * 88
    rows = parity.csr_rows(rpn, cin)
    forced = oracle.forced_blocks(lay, True)
    nb = lay.nblocks
    samples = [(0, i) for i in range(nb)] + [(15, i) for i in range(nb)] + \
        [(5, i) for i in spread_rows(nb, 24)]
    same = 0
    for h in (0, 5, 15):
        qbar = oracle.pool(data["q"][:, h:h + 1], lay)[0, 0]
        kbar = oracle.pool(data["k"][:, h:h + 1], lay)[0, 0]
        s_all = lay.scale * (qbar @ kbar.T)
        for hh, i in samples:
            if hh != h:
                continue
            kept = rows[h * nb + i]
            assert parity.topk_valid(kept, s_all[i], 88, forced), (h, i)
            same += kept == oracle.select_topk_row(s_all[i], 88, forced)
    say(f"topk 32 frames: {same} of {len(samples)} sampled lists equal the oracle's")
    check_sampled_attention(lay, data, o, rpn, cin, samples)


def test_hot_path_graph_replay(dev):
    """Selection and attention captured once in a HIP graph (the library enqueues
    no memset, allocation or synchronisation) and replayed several times, with
    eager work that clobbers the outputs between replays: every replay must
    reproduce the eager results bit for bit."""
    w, data = preset(1, heads=2)
    lay = w.layout
    q, k, v = inputs(w, data, dev)
    keep = data["keep"]
    rows = lay.heads * lay.nblocks
    cap = bsgm.col_capacity(lay, bsgm.TOPK, keep, force=True)
    rp = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    ci = torch.empty(cap, dtype=torch.int32, device=dev)
    sws = torch.empty(bsgm.workspace_bytes(lay, bsgm.TOPK), dtype=torch.uint8, device=dev)
    aws = torch.empty(bsgm.attn_workspace_bytes(lay), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((1, lay.heads, lay.tokens), dtype=torch.float32, device=dev)

    def step():
        bsgm.select_blocks(lay, bsgm.TOPK, keep, q=q, k=k, force=True, row_ptr=rp, col_idx=ci,
                           workspace=sws, want_stat=False)
        bsgm.sparse_attn_fwd(lay, q, k, v, rp, ci, o=o, lse=lse, workspace=aws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (rp, ci, o, lse)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (rp, ci, o, lse):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want, name in zip((rp, ci, o, lse), ref, ("row_ptr", "col_idx", "o", "lse")):
            assert torch.equal(got, want), (rep, name)
    say("graph replay: 3 replays equal to the eager step")


@pytest.mark.parametrize("block", [128, 64])
def test_attention_prepared_on_a_side_stream(dev, block):
    """The fp16 copy of K made by attn_prepare on another stream, overlapping the
    selection, then the prepared attention call: bit-identical to the one-call
    form."""
    lay = custom_layout(3, 2 * block, 2 * block - 37, block, heads=2, dtype="bf16", batch=2)
    host, vals = random_inputs(lay, 77 + block)
    q, k, v = (to_dev(x, dev) for x in host)
    keep = [max(1, lay.nblocks // 2)] * lay.heads
    ws1 = torch.empty(bsgm.attn_workspace_bytes(lay), dtype=torch.uint8, device=dev)
    ws2 = torch.empty_like(ws1)
    rp, ci, _ = bsgm.select_blocks(lay, bsgm.TOPK, keep, q=q, k=k, force=True)
    o1, l1 = bsgm.sparse_attn_fwd(lay, q, k, v, rp, ci, want_lse=True, workspace=ws1)
    torch.cuda.synchronize()
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    side.wait_stream(main)
    with torch.cuda.stream(side):
        bsgm.attn_prepare(lay, k, ws2)
    rp2, ci2, _ = bsgm.select_blocks(lay, bsgm.TOPK, keep, q=q, k=k, force=True)
    main.wait_stream(side)
    o2, l2 = bsgm.sparse_attn_fwd(lay, q, k, v, rp2, ci2, want_lse=True, workspace=ws2,
                                  prepared=True)
    torch.cuda.synchronize()
    assert torch.equal(rp, rp2) and torch.equal(ci, ci2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_padding_contents_are_ignored(dev):
    """Finite garbage in the padding tokens of Q, K and V (including values past
    the fp16 range, which route blocks to the bf16 form) changes neither the
    selection nor any real output, in both attention forms."""
    lay = custom_layout(3, 256, 200, 128, heads=2, dtype="bf16")
    host, vals = random_inputs(lay, 91)
    pad = (np.arange(lay.tokens) % lay.frame_len) >= lay.frame_valid
    rng = np.random.default_rng(5)
    dirty = []
    for x in vals:
        y = x.copy()
        y[:, :, pad] = rng.uniform(-9e4, 9e4, size=y[:, :, pad].shape).astype(np.float32)
        dirty.append(workloads.bf16_bits_from_float(y))
    keep = [4] * lay.heads          # the 3 forced blocks and one more
    outs = []
    aws = torch.empty(bsgm.attn_workspace_bytes(lay), dtype=torch.uint8, device=dev)
    for h in (host, dirty):
        q, k, v = (to_dev(x, dev) for x in h)
        rp, ci, _ = bsgm.select_blocks(lay, bsgm.TOPK, keep, q=q, k=k, force=True)
        for ws in (aws, None):
            o, l = bsgm.sparse_attn_fwd(lay, q, k, v, rp, ci, want_lse=True, workspace=ws)
            outs.append((rp.clone(), ci.clone(), o.float(), l))
    torch.cuda.synchronize()
    # the dirty padding left some rows to the bf16 form (the fallback flags per row)
    al = lambda x: (x + 255) // 256 * 256
    rows = lay.heads * lay.nblocks
    off = al(lay.tokens * lay.heads * 64 * 2) + al(rows * 4)
    redo = aws.cpu().numpy()[off:off + 4 * rows].view(np.int32)
    assert redo.sum() > 0
    rp0, ci0 = outs[0][0].cpu().numpy(), outs[0][1].cpu().numpy()
    o_ref, lse_ref = oracle.sparse_attention(vals[0], vals[1], vals[2], lay, rp0, ci0)
    valid = oracle.valid_mask(lay)
    fin = np.isfinite(lse_ref)
    for n, (rp, ci, o, l) in enumerate(outs):
        assert np.array_equal(rp.cpu().numpy(), rp0) and np.array_equal(ci.cpu().numpy(), ci0)
        o, l = o.cpu().numpy(), l.cpu().numpy()
        assert np.all(np.isfinite(o)) and np.all(o[..., ~valid, :] == 0)
        assert_outputs(lay, o, o_ref, valid, f"padding run {n}")
        assert np.array_equal(np.isfinite(l), fin)
        assert np.abs(l[fin] - lse_ref[fin]).max() <= 2e-3 * max(1.0, np.abs(lse_ref[fin]).max())


def test_topk_layer8_full_size(dev):
    say("topk 8 frames full size")
    w, data = preset(1)
    lay = w.layout
    q, k, v = inputs(w, data, dev)
    scores = torch.empty((1, lay.heads, lay.nblocks, lay.nblocks), dtype=torch.float32, device=dev)
    rp, ci, st = bsgm.select_blocks(lay, bsgm.TOPK, data["keep"], q=q, k=k, scores_out=scores)
    torch.cuda.synchronize()
    mism = check_topk(lay, (data["q"], data["k"], data["v"]), data["keep"], False, rp.cpu().numpy(),
                      ci.cpu().numpy(), scores.cpu().numpy(), st.cpu().numpy())
    say(f"topk 8 frames: near-tie rows {mism}")


# --------------------------------------------------------------------------
# drift
# --------------------------------------------------------------------------
# Unit roundoffs of float32 that the renormalised-drift check allows per element
# of the swap rows x_j = zhat_j * obar - chat_j (see renorm_floor).
RENORM_KAPPA = 16


def renorm_floor(chat, zhat, kept):
    """Absolute allowance in J^2 for the renormalised objective on the GPU,
    written from float32's unit roundoff u = 2^-24 and the oracle's own values
    only (nothing the GPU returned enters it).

    The kernel scores swaps on float32 contributions and masses, with rows
    x_j = zhat_j * obar - chat_j (obar = sum_j chat_j), as (||u||^2 + delta) / Z^2,
    u = sum_{dropped} x_j + (1 - sum_j zhat_j) obar. Two allowances:
      * its inputs: each element of x_j off by up to RENORM_KAPPA * u of the row's
        size, so J may move by dJ_in = RENORM_KAPPA * u * sum_j ||x_j|| / Z, Z taken
        as half the final kept mass (a lower bound for the sets a few swaps away
        in these tests). A float32 evaluation of the same sums on the CPU moves
        x_j by 2.2 u or less in that measure, so the allowance has an 8x margin.
        (The rigorous worst-case bound, n * u per sum of n terms, comes out near
        0.6 J on these rows and would accept any swap.)
      * the update rule's own rounding: 16 * 2u * (||u|| + 2 max_j ||x_j||)^2 / Z^2
        in J^2, from differences of squared norms.
    Returns (allowance in J^2, dJ_in)."""
    u = 2.0 ** -24
    obar = chat.sum(axis=0)
    x_ref = zhat[:, None] * obar[None, :] - chat
    xnorm = np.sqrt((x_ref * x_ref).sum(axis=1))
    zmin = 0.5 * float(zhat[sorted(kept)].sum())
    dj = RENORM_KAPPA * u * float(xnorm.sum()) / zmin
    xmax = float(xnorm.max())
    drop = sorted(set(range(chat.shape[0])) - set(kept))
    unorm = float(np.sqrt((x_ref[drop].sum(axis=0) ** 2).sum()))
    jmax = (unorm + 2 * xmax) / zmin
    return 2 * jmax * dj + dj * dj + 16 * 2 * u * (unorm + 2 * xmax) ** 2 / zmin ** 2, dj


def check_drift(lay, vals, keep, rounds, force, contrib_g, score_g, rpn, cin, stat_g, log_g,
                rows_to_check, objective=oracle.RAW, zmass_g=None):
    q, k, v = vals
    nb = lay.nblocks
    forced = oracle.forced_blocks(lay, force)
    rows = parity.csr_rows(rpn, cin)
    differ = 0
    needs_floor = 0
    for (h, i) in rows_to_check:
        qbar = oracle.pool(q[:, h:h + 1], lay)[0, 0]
        chat, z, Z = oracle.drift_row(qbar[i], k[0, h], v[0, h], lay)
        zhat = z / Z
        cg = contrib_g[0, h, i]
        scale = np.sqrt((chat * chat).sum(axis=1)).max()
        assert np.abs(cg - chat).max() <= 1e-4 * scale, (h, i)
        dref = np.sqrt((chat * chat).sum(axis=1))
        assert np.abs(score_g[0, h, i] - dref).max() <= 1e-4 * dref.max()
        if zmass_g is not None:
            # normalised masses lie in [0, 1] and sum to one; a float32 logit
            # error of ~1e-6 moves each by that relative amount
            assert np.abs(zmass_g[0, h, i] - zhat).max() <= 1e-5, (h, i)
        r = h * nb + i
        swaps = log_g[r] if rounds > 0 else np.zeros((0, 2), np.int64)
        if objective == oracle.RENORM:
            floor, dj = renorm_floor(chat, zhat, rows[r])
            ok, why, jrep = parity.drift_valid(rows[r], swaps, chat, int(keep[h]), forced,
                                               zhat=zhat, floor=floor)
            assert ok, f"row {(h, i)}: {why}"
            plain, _, _ = parity.drift_valid(rows[r], swaps, chat, int(keep[h]), forced,
                                             zhat=zhat, floor=0.0)
            needs_floor += not plain
            assert abs(stat_g[r] - jrep) <= 1e-4 * jrep + dj + 1e-30, (h, i, stat_g[r], jrep, dj)
            kept_ref, j_ref, _ = oracle.restore_row_renorm(chat, zhat, int(keep[h]), rounds,
                                                           forced)
            if kept_ref != rows[r]:
                differ += 1
                assert jrep <= j_ref * (1 + 1e-3) + dj
            continue
        ok, why, jrep = parity.drift_valid(rows[r], swaps, chat, int(keep[h]), forced)
        assert ok, f"row {(h, i)}: {why}"
        assert abs(stat_g[r] - jrep) <= 1e-4 * max(jrep, 1e-30), (h, i, stat_g[r], jrep)
        kept_ref, j_ref, _ = oracle.restore_row(chat, int(keep[h]), rounds, forced)
        if kept_ref != rows[r]:
            differ += 1
            assert jrep <= j_ref * (1 + 1e-3)
    if objective == oracle.RENORM:
        say(f"renormalised drift: {needs_floor} of {len(rows_to_check)} rows pass only "
            f"with the float32 allowance (the others pass the plain 1e-4 rule)")
    return differ


@pytest.mark.parametrize("rounds,force", [(3, False), (0, False), (5, True)])
def test_drift_layer16_two_heads(dev, rounds, force):
    say(f"drift 16 frames, 2 heads, rounds {rounds}, force {force}")
    w, data = preset(4, heads=2)
    lay = w.layout
    q, k, v = inputs(w, data, dev)
    contrib, score = bsgm.drift_scores(lay, q, k, v)
    nb = lay.nblocks
    log = torch.full((lay.heads * nb, max(rounds, 1), 2), -7, dtype=torch.int32, device=dev)
    rp, ci, st = bsgm.select_blocks(lay, bsgm.DRIFT, data["keep"], contrib=contrib,
                                    swap_rounds=rounds, force=force, swap_log=log)
    torch.cuda.synchronize()
    rpn, cin = rp.cpu().numpy(), ci.cpu().numpy()
    parity.check_csr_wellformed(rpn, cin, nb)
    assert rpn[-1] == lay.heads * nb * int(data["keep"][0])
    logn = log.cpu().numpy()
    if rounds > 0:
        assert np.all(logn >= -1)
    sample = [(h, i) for h in range(2) for i in range(0, nb, 5)]
    differ = check_drift(lay, (data["q"], data["k"], data["v"]), data["keep"], rounds, force,
                         contrib.cpu().numpy(), score.cpu().numpy(), rpn, cin, st.cpu().numpy(),
                         logn, sample)
    say(f"drift: sampled rows whose final set differs from the oracle's own run: {differ}")


@pytest.mark.parametrize("dtype,block,force", [("bf16", 64, False), ("bf16", 128, True),
                                               ("f32", 64, True), ("f32", 128, False)])
def test_drift_small_layouts(dev, dtype, block, force):
    """Every row of ragged layouts with 40 (block 64) or 33 (block 128) key
    blocks per head: two 32-row query tiles, the second partial, and for 33 an
    odd block count (the kernels pair key blocks)."""
    frames, per = (10, 4) if block == 64 else (11, 3)
    lay = custom_layout(frames, per * block, per * block - 37, block, heads=2, dtype=dtype)
    host, vals = random_inputs(lay, 51 + block)
    nb = lay.nblocks
    nf = frames if force else 0
    keep = np.array([max(10, nf + 3), max(7, nf + 1)], dtype=np.int32)
    rounds = 3
    say(f"drift small {dtype} block {block} force {force}: nb {nb}")
    q, k, v = (to_dev(x, dev) for x in host)
    contrib, score = bsgm.drift_scores(lay, q, k, v)
    log = torch.full((lay.heads * nb, rounds, 2), -7, dtype=torch.int32, device=dev)
    rp, ci, st = bsgm.select_blocks(lay, bsgm.DRIFT, keep, contrib=contrib, swap_rounds=rounds,
                                    force=force, swap_log=log)
    torch.cuda.synchronize()
    rpn, cin = rp.cpu().numpy(), ci.cpu().numpy()
    parity.check_csr_wellformed(rpn, cin, nb)
    rows = [(h, i) for h in range(lay.heads) for i in range(nb)]
    differ = check_drift(lay, vals, keep, rounds, force, contrib.cpu().numpy(), score.cpu().numpy(),
                         rpn, cin, st.cpu().numpy(), log.cpu().numpy(), rows)
    say(f"drift small: rows whose final set differs from the oracle's own run: {differ}")


def test_drift_512_blocks_uncached_search(dev):
    """512 key blocks (the largest drift row) with half of them kept: the pair
    inner products D x S no longer fit in LDS, so every round recomputes them."""
    lay = custom_layout(32, 1024, 1000, 64, heads=1, dtype="bf16")
    host, vals = random_inputs(lay, 61)
    nb = lay.nblocks
    assert nb == 512
    keep = np.array([256], dtype=np.int32)
    rounds = 2
    say("drift 512 blocks, keep 256, 2 rounds")
    q, k, v = (to_dev(x, dev) for x in host)
    contrib, score = bsgm.drift_scores(lay, q, k, v)
    log = torch.full((nb, rounds, 2), -7, dtype=torch.int32, device=dev)
    rp, ci, st = bsgm.select_blocks(lay, bsgm.DRIFT, keep, contrib=contrib, swap_rounds=rounds,
                                    swap_log=log)
    torch.cuda.synchronize()
    rpn, cin = rp.cpu().numpy(), ci.cpu().numpy()
    parity.check_csr_wellformed(rpn, cin, nb)
    rows = [(0, i) for i in (0, 1, 255, 511)]
    differ = check_drift(lay, vals, keep, rounds, False, contrib.cpu().numpy(),
                         score.cpu().numpy(), rpn, cin, st.cpu().numpy(), log.cpu().numpy(), rows)
    say(f"drift 512: sampled rows whose final set differs from the oracle's own run: {differ}")


@pytest.mark.parametrize("objective", [oracle.RAW, oracle.RENORM])
def test_drift_wide_rows_cached_search(dev, objective):
    """Rows of 333 key blocks (more than 256, an odd count), 60 kept of which
    37 forced (one per frame), two heads: every block is ranked by one thread
    against every key, and the D x S products (273 x 23, 25 KB) still fit in
    LDS beside the rows, so they are computed once per row on the matrix cores
    and refreshed after each swap."""
    lay = custom_layout(37, 576, 550, 64, heads=2, dtype="bf16")
    host, vals = random_inputs(lay, 67)
    nb = lay.nblocks
    assert nb == 333
    keep = np.array([60, 60], dtype=np.int32)
    rounds = 4
    say(f"drift wide rows: nb {nb}, keep {keep.tolist()}, objective {objective}")
    q, k, v = (to_dev(x, dev) for x in host)
    zmass = None
    if objective == oracle.RENORM:
        zmass = torch.empty((1, lay.heads, nb, nb), dtype=torch.float32, device=dev)
    contrib, score = bsgm.drift_scores(lay, q, k, v, zmass=zmass)
    log = torch.full((lay.heads * nb, rounds, 2), -7, dtype=torch.int32, device=dev)
    rp, ci, st = bsgm.select_blocks(lay, bsgm.DRIFT, keep, contrib=contrib, swap_rounds=rounds,
                                    force=True, objective=objective, zmass=zmass, swap_log=log)
    torch.cuda.synchronize()
    rpn, cin = rp.cpu().numpy(), ci.cpu().numpy()
    parity.check_csr_wellformed(rpn, cin, nb)
    rows = [(h, i) for h in range(lay.heads) for i in (0, 1, 100, 255, 256, 257, 332)]
    differ = check_drift(lay, vals, keep, rounds, True, contrib.cpu().numpy(),
                         score.cpu().numpy(), rpn, cin, st.cpu().numpy(), log.cpu().numpy(), rows,
                         objective=objective,
                         zmass_g=None if zmass is None else zmass.cpu().numpy())
    say(f"drift wide rows: sampled rows whose final set differs from the oracle's own run: {differ}")


@pytest.mark.parametrize("keep,objective", [(20, oracle.RAW), (264, oracle.RAW),
                                            (20, oracle.RENORM)])
def test_drift_best_swap_rows_beyond_512(dev, keep, objective):
    """Best-swap selection on rows of 528 key blocks, wider than the LDS row
    cache: the row stays in global memory. Keep 20 caches the D x S products in
    LDS (508 x 20); keep 264 recomputes them every round (264 x 264)."""
    lay = custom_layout(48, 1408, 1374, 128, heads=1)
    assert lay.nblocks == 528
    host, vals = random_inputs(lay, 73 + keep)
    nb = lay.nblocks
    keep_a = np.array([keep], dtype=np.int32)
    rounds = 3
    say(f"drift best-swap 528 blocks, keep {keep}, objective {objective}")
    q, k, v = (to_dev(x, dev) for x in host)
    zmass = None
    if objective == oracle.RENORM:
        zmass = torch.empty((1, 1, nb, nb), dtype=torch.float32, device=dev)
    contrib, score = bsgm.drift_scores(lay, q, k, v, zmass=zmass)
    log = torch.full((nb, rounds, 2), -7, dtype=torch.int32, device=dev)
    rp, ci, st = bsgm.select_blocks(lay, bsgm.DRIFT, keep_a, contrib=contrib, swap_rounds=rounds,
                                    objective=objective, zmass=zmass, swap_log=log)
    torch.cuda.synchronize()
    rpn, cin = rp.cpu().numpy(), ci.cpu().numpy()
    parity.check_csr_wellformed(rpn, cin, nb)
    assert rpn[-1] == nb * keep
    rows = [(0, i) for i in (0, 1, 255, 256, 300, 511, 512, 527)]
    differ = check_drift(lay, vals, keep_a, rounds, False, contrib.cpu().numpy(),
                         score.cpu().numpy(), rpn, cin, st.cpu().numpy(), log.cpu().numpy(), rows,
                         objective=objective,
                         zmass_g=None if zmass is None else zmass.cpu().numpy())
    say(f"drift 528: sampled rows whose final set differs from the oracle's own run: {differ}")


def test_drift_best_swap_100_frame_rows(dev):
    """Best-swap selection on one head of the 100-frame layer (1 100 key blocks
    per row, keep 220, 3 rounds): pair products recomputed every round."""
    lay = custom_layout(100, 1408, 1374, 128, heads=1)
    assert lay.nblocks == 1100
    host, vals = random_inputs(lay, 79)
    nb = lay.nblocks
    keep = np.array([220], dtype=np.int32)
    rounds = 3
    q, k, v = (to_dev(x, dev) for x in host)
    contrib, score = bsgm.drift_scores(lay, q, k, v)
    log = torch.full((nb, rounds, 2), -7, dtype=torch.int32, device=dev)
    rp, ci, st = bsgm.select_blocks(lay, bsgm.DRIFT, keep, contrib=contrib, swap_rounds=rounds,
                                    swap_log=log)
    torch.cuda.synchronize()
    rpn, cin = rp.cpu().numpy(), ci.cpu().numpy()
    parity.check_csr_wellformed(rpn, cin, nb)
    rows = [(0, i) for i in (0, 549, 1099)]
    differ = check_drift(lay, vals, keep, rounds, False, contrib.cpu().numpy(),
                         score.cpu().numpy(), rpn, cin, st.cpu().numpy(), log.cpu().numpy(), rows)
    say(f"drift 1100: sampled rows whose final set differs from the oracle's own run: {differ}")


# renormalised objective: the output shift once dropped blocks are removed
@pytest.mark.parametrize("dtype,block,force", [("bf16", 64, False), ("bf16", 128, True),
                                               ("f32", 64, True), ("f32", 128, False)])
def test_drift_renorm_small_layouts(dev, dtype, block, force):
    frames, per = (10, 4) if block == 64 else (11, 3)
    lay = custom_layout(frames, per * block, per * block - 37, block, heads=2, dtype=dtype)
    host, vals = random_inputs(lay, 71 + block)
    nb = lay.nblocks
    nf = frames if force else 0
    keep = np.array([max(10, nf + 3), max(7, nf + 1)], dtype=np.int32)
    rounds = 4
    say(f"drift renorm small {dtype} block {block} force {force}: nb {nb}")
    q, k, v = (to_dev(x, dev) for x in host)
    zmass = torch.full((1, lay.heads, nb, nb), -1.0, dtype=torch.float32, device=dev)
    contrib, score = bsgm.drift_scores(lay, q, k, v, zmass=zmass)
    log = torch.full((lay.heads * nb, rounds, 2), -7, dtype=torch.int32, device=dev)
    rp, ci, st = bsgm.select_blocks(lay, bsgm.DRIFT, keep, contrib=contrib, swap_rounds=rounds,
                                    force=force, swap_log=log, objective=bsgm.RENORMALISED,
                                    zmass=zmass)
    torch.cuda.synchronize()
    rpn, cin = rp.cpu().numpy(), ci.cpu().numpy()
    parity.check_csr_wellformed(rpn, cin, nb)
    logn = log.cpu().numpy()
    assert np.all(logn >= -1)
    rows = [(h, i) for h in range(lay.heads) for i in range(nb)]
    differ = check_drift(lay, vals, keep, rounds, force, contrib.cpu().numpy(),
                         score.cpu().numpy(), rpn, cin, st.cpu().numpy(), logn, rows,
                         objective=oracle.RENORM, zmass_g=zmass.cpu().numpy())
    nswaps = int((logn[..., 0] >= 0).sum())
    say(f"drift renorm small: {nswaps} swaps; rows differing from the oracle's run: {differ}")


@pytest.mark.parametrize("rounds,force,heads", [(3, False, 2), (6, True, 1)])
def test_drift_renorm_layer16(dev, rounds, force, heads):
    say(f"drift renorm 16 frames, {heads} heads, rounds {rounds}, force {force}")
    w, data = preset(4, heads=heads)
    lay = w.layout
    q, k, v = inputs(w, data, dev)
    nb = lay.nblocks
    zmass = torch.empty((1, lay.heads, nb, nb), dtype=torch.float32, device=dev)
    contrib, score = bsgm.drift_scores(lay, q, k, v, zmass=zmass)
    log = torch.full((lay.heads * nb, rounds, 2), -7, dtype=torch.int32, device=dev)
    rp, ci, st = bsgm.select_blocks(lay, bsgm.DRIFT, data["keep"], contrib=contrib,
                                    swap_rounds=rounds, force=force, swap_log=log,
                                    objective=bsgm.RENORMALISED, zmass=zmass)
    torch.cuda.synchronize()
    rpn, cin = rp.cpu().numpy(), ci.cpu().numpy()
    parity.check_csr_wellformed(rpn, cin, nb)
    logn = log.cpu().numpy()
    assert np.all(logn >= -1)
    sample = [(h, i) for h in range(heads) for i in range(0, nb, 7)]
    differ = check_drift(lay, (data["q"], data["k"], data["v"]), data["keep"], rounds, force,
                         contrib.cpu().numpy(), score.cpu().numpy(), rpn, cin, st.cpu().numpy(),
                         logn, sample, objective=oracle.RENORM, zmass_g=zmass.cpu().numpy())
    nswaps = int((logn[..., 0] >= 0).sum())
    say(f"drift renorm 16: {nswaps} swaps over all rows; sampled rows differing: {differ}")


def test_drift_renorm_512_blocks_uncached_search(dev):
    lay = custom_layout(32, 1024, 1000, 64, heads=1, dtype="bf16")
    host, vals = random_inputs(lay, 67)
    nb = lay.nblocks
    keep = np.array([256], dtype=np.int32)
    rounds = 2
    say("drift renorm 512 blocks, keep 256, 2 rounds")
    q, k, v = (to_dev(x, dev) for x in host)
    zmass = torch.empty((1, 1, nb, nb), dtype=torch.float32, device=dev)
    contrib, score = bsgm.drift_scores(lay, q, k, v, zmass=zmass)
    log = torch.full((nb, rounds, 2), -7, dtype=torch.int32, device=dev)
    rp, ci, st = bsgm.select_blocks(lay, bsgm.DRIFT, keep, contrib=contrib, swap_rounds=rounds,
                                    swap_log=log, objective=bsgm.RENORMALISED, zmass=zmass)
    torch.cuda.synchronize()
    rpn, cin = rp.cpu().numpy(), ci.cpu().numpy()
    parity.check_csr_wellformed(rpn, cin, nb)
    rows = [(0, i) for i in (0, 3, 256, 511)]
    check_drift(lay, vals, keep, rounds, False, contrib.cpu().numpy(), score.cpu().numpy(), rpn,
                cin, st.cpu().numpy(), log.cpu().numpy(), rows, objective=oracle.RENORM,
                zmass_g=zmass.cpu().numpy())


def test_drift_layer16_full_size_sampled(dev):
    """16 frames, 16 heads, drift + 3 rounds: the bench launch. On heads 0, 7
    and 15, the XCD boundary rows and more (24 or more per head): the swap log
    replays as optimal on the oracle's contributions, and every output equals
    the oracle's attention over the GPU's own list."""
    say("drift 16 frames full size")
    w, data = preset(4)
    lay = w.layout
    q, k, v = inputs(w, data, dev)
    contrib, score = bsgm.drift_scores(lay, q, k, v)
    nb = lay.nblocks
    log = torch.empty((lay.heads * nb, 3, 2), dtype=torch.int32, device=dev)
    rp, ci, st = bsgm.select_blocks(lay, bsgm.DRIFT, data["keep"], contrib=contrib, swap_rounds=3,
                                    swap_log=log)
    o, _ = bsgm.sparse_attn_fwd(lay, q, k, v, rp, ci)
    torch.cuda.synchronize()
    rpn, cin = rp.cpu().numpy(), ci.cpu().numpy()
    parity.check_csr_wellformed(rpn, cin, nb)
    sample = [(h, i) for h in (0, 7, 15) for i in spread_rows(nb, 24)]
    differ = check_drift(lay, (data["q"], data["k"], data["v"]), data["keep"], 3, False,
                         contrib.cpu().numpy(), score.cpu().numpy(), rpn, cin, st.cpu().numpy(),
                         log.cpu().numpy(), sample)
    say(f"drift full size: {len(sample)} sampled rows, {differ} with lists other than the oracle's")
    check_sampled_attention(lay, data, o, rpn, cin, sample)


def check_rerank(lay, vals, keep, rounds, track_best, force, contrib_g, rpn, cin, stat_g, log_g,
                 rows_to_check):
    """Every checked row: the logged sets replay as top-k choices on the
    oracle's contributions, the returned set is the last one (or of least J),
    and the reported J is the oracle's J of the returned set."""
    q, k, v = vals
    nb = lay.nblocks
    forced = oracle.forced_blocks(lay, force)
    rows = parity.csr_rows(rpn, cin)
    words = (nb + 31) // 32
    qbar_cache = {}
    differ = 0
    for row in rows_to_check:
        b, h, i = row if len(row) == 3 else (0,) + tuple(row)
        if (b, h) not in qbar_cache:
            qbar_cache[(b, h)] = oracle.pool(q[b:b + 1, h:h + 1], lay)[0, 0]
        chat, _, _ = oracle.drift_row(qbar_cache[(b, h)][i], k[b, h], v[b, h], lay)
        r = (b * lay.heads + h) * nb + i
        lg = log_g[r].reshape(rounds + 1, words)
        sets = [parity.mask_words_to_set(lg[x], nb) for x in range(rounds + 1)]
        ok, why = parity.rerank_valid(sets, rows[r], chat, int(keep[h]), forced, track_best)
        assert ok, f"row {(b, h, i)}: {why}"
        jref = oracle.drift_j(chat, rows[r])
        assert abs(stat_g[r] - jref) <= 1e-4 * max(jref, 1e-30), (b, h, i, stat_g[r], jref)
        kept_ref, _, _, _ = oracle.rerank_row(chat, int(keep[h]), rounds, forced, track_best)
        differ += kept_ref != rows[r]
    return differ


def run_rerank(dev, lay, host, vals, keep, rounds, track_best, force, rows_to_check, label):
    q, k, v = (to_dev(x, dev) for x in host)
    contrib, score = bsgm.drift_scores(lay, q, k, v)
    nb = lay.nblocks
    rows = lay.batch * lay.heads * nb
    log = torch.full((rows, rounds + 1, (nb + 31) // 32), -7, dtype=torch.int32, device=dev)
    rule = bsgm.RERANK_TRACK_BEST if track_best else bsgm.RERANK
    rp, ci, st = bsgm.select_blocks(lay, bsgm.DRIFT, keep, contrib=contrib, swap_rounds=rounds,
                                    force=force, swap_log=log, restoration=rule)
    torch.cuda.synchronize()
    rpn, cin = rp.cpu().numpy(), ci.cpu().numpy()
    parity.check_csr_wellformed(rpn, cin, nb)
    assert rpn[-1] == lay.batch * nb * int(np.sum(keep))
    differ = check_rerank(lay, vals, keep, rounds, track_best, force, contrib.cpu().numpy(), rpn,
                          cin, st.cpu().numpy(), log.cpu().numpy(), rows_to_check)
    say(f"{label}: {len(rows_to_check)} rows checked, {differ} with sets other than the oracle's")
    return rp, ci


@pytest.mark.parametrize("rounds,track_best,force", [(5, True, False), (5, False, False),
                                                     (10, True, True), (10, False, False)])
def test_drift_rerank_layer16(dev, rounds, track_best, force):
    """16 frames, 2 heads (176 key blocks, keep 35): re-rank rounds at 5 and 10
    rounds with and without track-best (ReSS Table S3's arms); every row of
    head 0 and the XCD boundary rows of head 1."""
    w, data = preset(4, heads=2)
    lay = w.layout
    host = [data[n + "_bits"] for n in ("q", "k", "v")]
    vals = (data["q"], data["k"], data["v"])
    keep = data["keep"]
    if force:
        keep = np.maximum(keep, lay.frames + 3).astype(np.int32)
    rows = [(0, i) for i in range(lay.nblocks)] + [(1, i) for i in xcd_boundary_rows(lay.nblocks)]
    run_rerank(dev, lay, host, vals, keep, rounds, track_best, force, rows,
               f"re-rank 16 frames, {rounds} rounds, track-best {track_best}, force {force}")


@pytest.mark.parametrize("force", [False, True])
def test_drift_rerank_wide_rows_exact_ties(dev, force):
    """Rows of 528 key blocks (wider than 512, so the top-k comes from the
    MSB-first priority search) in which the value rows of frames 24 to 47 are
    zero: 264 blocks contribute exactly nothing and tie at score 0 in every
    round. Keep is set so that the initial cut falls inside those ties, so the
    lowest-block rule decides it; the initial set must equal the oracle's
    exactly, and every round must replay as a valid top-k. With force, keep
    equals the 48 forced blocks, which all tie at the top priority."""
    lay = custom_layout(48, 1408, 1374, 128, heads=1)
    assert lay.nblocks == 528
    host, vals = random_inputs(lay, 71)
    tok = np.arange(lay.tokens)
    zero = (tok // lay.frame_len) >= 24
    q, k, v = vals
    v = v.copy()
    v[:, :, zero] = 0
    vals = (q, k, v)
    host = list(host)
    host[2] = workloads.bf16_bits_from_float(v)
    nb = lay.nblocks
    keep = np.array([lay.frames if force else 264 + 40], dtype=np.int32)
    rounds = 3
    rows = [(0, i) for i in (0, 5, 263, 264, 300, 527)]
    label = f"re-rank exact ties, force {force}"
    rp, ci = run_rerank(dev, lay, host, vals, keep, rounds, True, force, rows, label)
    # the initial set, taken from the oracle's own run, must match exactly
    qd, kd, vd = (to_dev(x, dev) for x in host)
    contrib, _ = bsgm.drift_scores(lay, qd, kd, vd)
    log = torch.full((nb, rounds + 1, (nb + 31) // 32), -7, dtype=torch.int32, device=dev)
    bsgm.select_blocks(lay, bsgm.DRIFT, keep, contrib=contrib, swap_rounds=rounds, force=force,
                       swap_log=log, restoration=bsgm.RERANK_TRACK_BEST)
    torch.cuda.synchronize()
    lg = log.cpu().numpy()
    forced = oracle.forced_blocks(lay, force)
    qbar = oracle.pool(q[:, 0:1], lay)[0, 0]
    for (_, i) in rows:
        chat, _, _ = oracle.drift_row(qbar[i], k[0, 0], v[0, 0], lay)
        _, _, sets, _ = oracle.rerank_row(chat, int(keep[0]), rounds, forced, True)
        got = parity.mask_words_to_set(lg[i].reshape(rounds + 1, -1)[0], nb)
        assert got == sorted(sets[0]), (i, len(got))


@pytest.mark.parametrize("nb,frames", [(1100, 100), (61, 1)])
def test_drift_rerank_wide_and_small_rows(dev, nb, frames):
    """Rows of 1100 key blocks (a 100-frame layer's width, beyond what the
    best-swap search holds) and a single ragged frame of 61 blocks of 64."""
    if nb == 1100:
        lay = custom_layout(frames, 1408, 1374, 128, heads=1)
    else:
        lay = custom_layout(1, 61 * 64, 61 * 64 - 40, 64, heads=1, dtype="f32")
    assert lay.nblocks == nb
    host, vals = random_inputs(lay, 55 + nb)
    keep = np.array([max(4, nb // 5)], dtype=np.int32)
    rows = [(0, i) for i in spread_rows(nb, 24)]
    run_rerank(dev, lay, host, vals, keep, 5, True, False, rows, f"re-rank rows of {nb} blocks")


# --------------------------------------------------------------------------
# re-rank rounds in the expanded form (no contributions kept)
def run_streamed(dev, lay, host, vals, keep, rounds, track_best, force, rows_to_check, label,
                 min_same=0.9):
    """The streamed selection on every checked row against the oracle (the same
    rule as the materialised re-rank: logged sets replay as top-k choices, the
    returned set, its J), then the logged sets of every row against the
    materialised form's: the two round the same sums differently, so only
    near-ties may differ, and at least min_same of the rows must match."""
    q, k, v = (to_dev(x, dev) for x in host)
    nb = lay.nblocks
    rows = lay.batch * lay.heads * nb
    words = (nb + 31) // 32
    log = torch.full((rows, rounds + 1, words), -7, dtype=torch.int32, device=dev)
    say(f"{label}: streamed selection")
    rp, ci, st = bsgm.select_drift_streamed(lay, keep, q, k, v, swap_rounds=rounds,
                                            track_best=track_best, force=force, set_log=log)
    torch.cuda.synchronize()
    rpn, cin = rp.cpu().numpy(), ci.cpu().numpy()
    parity.check_csr_wellformed(rpn, cin, nb)
    assert rpn[-1] == lay.batch * nb * int(np.sum(keep))
    differ = check_rerank(lay, vals, keep, rounds, track_best, force, None, rpn, cin,
                          st.cpu().numpy(), log.cpu().numpy(), rows_to_check)
    say(f"{label}: {len(rows_to_check)} rows checked, {differ} with sets other than the oracle's")
    contrib, _ = bsgm.drift_scores(lay, q, k, v)
    log_m = torch.full_like(log, -7)
    rule = bsgm.RERANK_TRACK_BEST if track_best else bsgm.RERANK
    rp_m, ci_m, _ = bsgm.select_blocks(lay, bsgm.DRIFT, keep, contrib=contrib, swap_rounds=rounds,
                                       force=force, swap_log=log_m, restoration=rule)
    torch.cuda.synchronize()
    del contrib
    same = int((log == log_m).all(dim=2).all(dim=1).sum().item())
    say(f"{label}: {rows - same} of {rows} rows log other sets than the materialised form")
    assert same >= min_same * rows, (same, rows)
    return rp, ci, st, log


@pytest.mark.parametrize("rounds,track_best,force", [(5, True, False), (10, False, True),
                                                     (0, True, False)])
def test_drift_streamed_layer16(dev, rounds, track_best, force):
    """16 frames, 2 heads (176 key blocks, keep 35): the expanded-form re-rank
    at 0, 5 and 10 rounds; every row of head 0 and the XCD boundary rows of
    head 1 against the oracle; a second call gives bitwise the same result."""
    w, data = preset(4, heads=2)
    lay = w.layout
    host = [data[n + "_bits"] for n in ("q", "k", "v")]
    vals = (data["q"], data["k"], data["v"])
    keep = data["keep"]
    if force:
        keep = np.maximum(keep, lay.frames + 3).astype(np.int32)
    rows = [(0, i) for i in range(lay.nblocks)] + [(1, i) for i in xcd_boundary_rows(lay.nblocks)]
    label = f"streamed re-rank 16 frames, {rounds} rounds, track-best {track_best}, force {force}"
    rp, ci, st, log = run_streamed(dev, lay, host, vals, keep, rounds, track_best, force, rows,
                                   label)
    q, k, v = (to_dev(x, dev) for x in host)
    log2 = torch.full_like(log, -7)
    rp2, ci2, st2 = bsgm.select_drift_streamed(lay, keep, q, k, v, swap_rounds=rounds,
                                               track_best=track_best, force=force, set_log=log2)
    torch.cuda.synchronize()
    assert torch.equal(rp, rp2) and torch.equal(ci, ci2) and torch.equal(log, log2)
    assert torch.equal(st.view(torch.int32), st2.view(torch.int32))


DRIFT_SWEEP_RULES = ("best-swap dropped sum", "best-swap renormalised", "re-rank", "streamed re-rank")


def drift_sweep_case(seed):
    """Seeded random layout and rule for the drift sweep: frames, frame length
    (whole blocks), padding under one block, block 64 or 128, fp32 or bf16,
    heads, batch (the re-rank rules), budgets covering the forced blocks,
    rounds, track-best."""
    rng = np.random.default_rng(3000 + seed)
    rule = seed % 4
    block = (64, 128)[(seed // 4) % 2]
    dtype = "f32" if seed % 3 == 0 else "bf16"
    frames = int(rng.integers(2, 9))
    frame_len = block * int(rng.integers(1, 6))
    frame_valid = frame_len - int(rng.integers(0, block))
    heads = int(rng.integers(1, 3))
    batch = 1 if rule < 2 else int(rng.integers(1, 3))
    lay = custom_layout(frames, frame_len, frame_valid, block, heads=heads, dtype=dtype, batch=batch)
    force = bool(rng.integers(0, 2))
    nb = lay.nblocks
    lo = max(1, len(oracle.forced_blocks(lay, force)))
    keep = np.array([int(rng.integers(lo, max(lo, nb - 1) + 1)) for _ in range(heads)],
                    dtype=np.int32)
    rounds = int(rng.integers(0, 5)) if rule < 2 else int(rng.integers(0, 7))
    track_best = bool(rng.integers(0, 2))
    return lay, rule, force, keep, rounds, track_best


@pytest.mark.parametrize("seed", range(12))
def test_drift_random_layouts(dev, seed):
    """Drift selection on seeded random layouts (see drift_sweep_case), each
    rule in turn: every row's contributions against the oracle's, and its list
    replayed under the rule on the oracle's contributions; then attention over
    the selected lists against the oracle on every row."""
    lay, rule, force, keep, rounds, track_best = drift_sweep_case(seed)
    nb = lay.nblocks
    label = (f"drift sweep seed {seed}: {DRIFT_SWEEP_RULES[rule]}, frames {lay.frames}x"
             f"{lay.frame_len} ({lay.frame_valid} real), block {lay.block}, {lay.dtype}, batch "
             f"{lay.batch}, heads {lay.heads}, keep {keep.tolist()}, rounds {rounds}, "
             f"track-best {track_best}, force {force}")
    say(label)
    host, vals = random_inputs(lay, 4000 + seed)
    q, k, v = (to_dev(x, dev) for x in host)
    if rule < 2:
        renorm = rule == 1
        zmass = (torch.full((1, lay.heads, nb, nb), -1.0, dtype=torch.float32, device=dev)
                 if renorm else None)
        contrib, score = bsgm.drift_scores(lay, q, k, v, zmass=zmass)
        log = torch.full((lay.heads * nb, max(rounds, 1), 2), -7, dtype=torch.int32, device=dev)
        rp, ci, st = bsgm.select_blocks(
            lay, bsgm.DRIFT, keep, contrib=contrib, swap_rounds=rounds, force=force, swap_log=log,
            objective=bsgm.RENORMALISED if renorm else bsgm.DROPPED_SUM, zmass=zmass)
        torch.cuda.synchronize()
        rpn, cin = rp.cpu().numpy(), ci.cpu().numpy()
        parity.check_csr_wellformed(rpn, cin, nb)
        rows = [(h, i) for h in range(lay.heads) for i in range(nb)]
        check_drift(lay, vals, keep, rounds, force, contrib.cpu().numpy(), score.cpu().numpy(),
                    rpn, cin, st.cpu().numpy(), log.cpu().numpy(), rows,
                    objective=oracle.RENORM if renorm else oracle.RAW,
                    zmass_g=zmass.cpu().numpy() if renorm else None)
    else:
        rows = [(b, h, i) for b in range(lay.batch) for h in range(lay.heads) for i in range(nb)]
        if rule == 2:
            rp, ci = run_rerank(dev, lay, host, vals, keep, rounds, track_best, force, rows, label)
        else:
            rp, ci, _, _ = run_streamed(dev, lay, host, vals, keep, rounds, track_best, force,
                                        rows, label, min_same=0.5)
        rpn, cin = rp.cpu().numpy(), ci.cpu().numpy()
    run_attention_case(dev, lay, host, vals, parity.csr_rows(rpn, cin), f"drift sweep seed {seed}",
                       workspace="auto" if seed % 2 == 0 else None)


def test_drift_streamed_more_kept_than_dropped(dev):
    """Keep 120 of 176 blocks (more kept than dropped, so the rounds sum the
    dropped blocks directly rather than the total minus the kept ones), with a
    second head at keep 40 (mixed budgets take the dropped sums as well)."""
    w, data = preset(4, heads=2)
    lay = w.layout
    host = [data[n + "_bits"] for n in ("q", "k", "v")]
    vals = (data["q"], data["k"], data["v"])
    keep = np.array([120, 40], dtype=np.int32)
    rows = [(h, i) for h in (0, 1) for i in spread_rows(lay.nblocks, 24)]
    run_streamed(dev, lay, host, vals, keep, 4, True, False, rows,
                 "streamed re-rank, more kept than dropped")


@pytest.mark.parametrize("force", [False, True])
def test_drift_streamed_exact_ties(dev, force):
    """Rows of 528 key blocks whose value rows of frames 24 to 47 are zero: 264
    blocks score exactly 0 in every round (their weighted value dot products
    are exact zeros too), and keep cuts inside those ties, so the lowest-block
    rule decides; the initial set must equal the oracle's exactly."""
    lay = custom_layout(48, 1408, 1374, 128, heads=1)
    host, vals = random_inputs(lay, 71)
    tok = np.arange(lay.tokens)
    zero = (tok // lay.frame_len) >= 24
    q, k, v = vals
    v = v.copy()
    v[:, :, zero] = 0
    vals = (q, k, v)
    host = list(host)
    host[2] = workloads.bf16_bits_from_float(v)
    nb = lay.nblocks
    keep = np.array([lay.frames if force else 264 + 40], dtype=np.int32)
    rounds = 3
    rows = [(0, i) for i in (0, 5, 263, 264, 300, 527)]
    _, _, _, log = run_streamed(dev, lay, host, vals, keep, rounds, True, force, rows,
                                f"streamed re-rank exact ties, force {force}")
    lg = log.cpu().numpy()
    forced = oracle.forced_blocks(lay, force)
    qbar = oracle.pool(q[:, 0:1], lay)[0, 0]
    for (_, i) in rows:
        chat, _, _ = oracle.drift_row(qbar[i], k[0, 0], v[0, 0], lay)
        _, _, sets, _ = oracle.rerank_row(chat, int(keep[0]), rounds, forced, True)
        got = parity.mask_words_to_set(lg[i].reshape(rounds + 1, -1)[0], nb)
        assert got == sorted(sets[0]), (i, len(got))


@pytest.mark.parametrize("nb,frames,block,dtype", [(1100, 100, 128, "bf16"), (2200, 25, 64, "bf16"),
                                                   (61, 1, 64, "bf16"), (61, 1, 64, "f32"),
                                                   (24, 3, 128, "f32")])
def test_drift_streamed_wide_and_small_rows(dev, nb, frames, block, dtype):
    """Rows of 1100 key blocks (a 100-frame layer's width; one wave per row in
    the selection step), of 2200 blocks of 64 (one workgroup per row there), a
    single ragged frame of 61 blocks of 64 in bf16 and fp32 (the vector-ALU
    passes), and three fp32 frames of 8 blocks of 128."""
    if nb == 1100:
        lay = custom_layout(frames, 1408, 1374, block, heads=1)
    elif nb == 2200:
        lay = custom_layout(frames, 88 * 64, 88 * 64 - 30, block, heads=1)
    elif nb == 61:
        lay = custom_layout(1, 61 * 64, 61 * 64 - 40, block, heads=1, dtype=dtype)
    else:
        lay = custom_layout(frames, 8 * 128, 8 * 128 - 100, block, heads=2, dtype=dtype)
    assert lay.nblocks == nb
    host, vals = random_inputs(lay, 55 + nb)
    keep = np.full(lay.heads, max(4, nb // 5), dtype=np.int32)
    rows = [(0, i) for i in spread_rows(nb, 24)]
    run_streamed(dev, lay, host, vals, keep, 5, True, False, rows,
                 f"streamed re-rank rows of {nb} blocks")


def test_drift_streamed_block64_wide_forced(dev):
    """Blocks of 64, 600 per row (wider than 512, so every round's top k comes
    from the MSB-first priority search), ragged frames, forced frame blocks,
    3 rounds with track-best."""
    lay = custom_layout(25, 24 * 64, 24 * 64 - 36, 64, heads=1)
    assert lay.nblocks == 600
    host, vals = random_inputs(lay, 97)
    keep = np.array([120], dtype=np.int32)
    rows = [(0, i) for i in spread_rows(lay.nblocks, 24)]
    run_streamed(dev, lay, host, vals, keep, 3, True, True, rows,
                 "streamed re-rank 600 blocks of 64, forced")


def test_drift_streamed_batch2_ragged(dev):
    """Two batch entries, two heads with different budgets, ragged frames of
    blocks of 64: every row of both batch entries of head 1."""
    lay = custom_layout(3, 1408, 1374, 64, heads=2, batch=2)
    host, vals = random_inputs(lay, 91)
    keep = np.array([9, 23], dtype=np.int32)
    nb = lay.nblocks
    rows = [(b, 1, i) for b in range(2) for i in range(nb)] + [(1, 0, i) for i in spread_rows(nb, 8)]
    run_streamed(dev, lay, host, vals, keep, 4, True, True, rows, "streamed re-rank batch 2")


def test_drift_streamed_layer16_full_size(dev):
    """The 16-frame drift layer at full size (16 heads, 5 rounds, track-best):
    the XCD boundary rows and evenly spaced rows of heads 0, 7 and 15 against
    the oracle; every row against the materialised form."""
    w, data = preset(4)
    lay = w.layout
    host = [data[n + "_bits"] for n in ("q", "k", "v")]
    vals = (data["q"], data["k"], data["v"])
    rows = [(h, i) for h in (0, 7, 15) for i in spread_rows(lay.nblocks, 24)]
    run_streamed(dev, lay, host, vals, data["keep"], 5, True, False, rows,
                 "streamed re-rank 16 frames full size")


# --------------------------------------------------------------------------
# dense camera/register query rows
# --------------------------------------------------------------------------
@pytest.mark.parametrize("block,ns", [(128, 5), (64, 5), (128, 50)])
def test_special_rows_dense_on_sparse_output(dev, block, ns):
    """Sparse attention on random kept lists, then the first ns tokens of every
    frame recomputed densely; the whole output against the oracle's composite."""
    lay = custom_layout(6, 4 * block, 4 * block - 37, block, heads=2, batch=2)
    host, vals = random_inputs(lay, 71 + block + ns)
    nb = lay.nblocks
    rng = np.random.default_rng(9)
    rows = [sorted(rng.choice(nb, size=int(rng.integers(1, nb + 1)), replace=False).tolist())
            for _ in range(lay.batch * lay.heads * nb)]
    say(f"special rows {ns} per frame, block {block}")
    q, k, v = (to_dev(x, dev) for x in host)
    rp, ci = upload_csr(rows, dev)
    o, lse = bsgm.sparse_attn_fwd(lay, q, k, v, rp, ci, want_lse=True)
    bsgm.special_rows_dense_fwd(lay, q, k, v, ns, o, lse)
    torch.cuda.synchronize()
    row_ptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])])
    col_idx = np.array([j for r in rows for j in r], dtype=np.int64)
    o_s, l_s = oracle.sparse_attention(vals[0], vals[1], vals[2], lay, row_ptr, col_idx)
    o_ref, l_ref = oracle.special_rows_dense(vals[0], vals[1], vals[2], lay, o_s, l_s, ns)
    valid = oracle.valid_mask(lay)
    assert_outputs(lay, o.float().cpu().numpy(), o_ref, valid, f"special rows ns={ns} block {block}")
    lse_g = lse.cpu().numpy()
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(lse_g), fin)
    assert np.abs(lse_g[fin] - l_ref[fin]).max() <= 2e-3 * max(1.0, np.abs(l_ref[fin]).max())


def test_special_rows_all_rows_is_dense(dev):
    """n_special = frame_valid: every real row dense, i.e. dense attention."""
    lay = custom_layout(3, 256, 230, 128, heads=2)
    host, vals = random_inputs(lay, 81)
    q, k, v = (to_dev(x, dev) for x in host)
    o = torch.zeros_like(q)
    lse = torch.full((lay.batch, lay.heads, lay.tokens), -float("inf"), device=dev)
    bsgm.special_rows_dense_fwd(lay, q, k, v, lay.frame_valid, o, lse)
    torch.cuda.synchronize()
    od, ld = oracle.dense_attention(*vals, lay)
    valid = oracle.valid_mask(lay)
    assert_outputs(lay, o.float().cpu().numpy(), od, valid, "all rows special vs dense")
    assert np.abs(lse.cpu().numpy()[..., valid] - ld[..., valid]).max() <= 2e-3 * np.abs(ld[..., valid]).max()
    assert torch.all(o[..., torch.from_numpy(~valid).to(dev), :] == 0)


def test_special_rows_full_size_sampled(dev):
    """32-frame layer at full size: special rows of two heads, sampled, against
    the oracle's softmax over all real keys."""
    w, data = preset(2)
    lay = w.layout
    q, k, v = inputs(w, data, dev)
    o = torch.zeros_like(q)
    lse = torch.zeros((lay.batch, lay.heads, lay.tokens), dtype=torch.float32, device=dev)
    say("special rows 32 frames full size")
    bsgm.special_rows_dense_fwd(lay, q, k, v, 5, o, lse)
    torch.cuda.synchronize()
    og, lg = o.float().cpu().numpy(), lse.cpu().numpy()
    keys = np.nonzero(oracle.valid_mask(lay))[0]
    for h in (0, 15):
        toks = np.array([f * lay.frame_len + p for f in (0, 13, 31) for p in (0, 4)])
        orf, lrf = oracle.attention_rows(data["q"][0, h, toks], data["k"][0, h, keys],
                                         data["v"][0, h, keys], lay.scale)
        for n, t in enumerate(toks):
            err = np.abs(og[0, h, t] - orf[n]).max()
            allow = 2e-2 * np.sqrt((orf[n] ** 2).mean())
            assert err <= allow, (h, t, err, allow)
            assert abs(lg[0, h, t] - lrf[n]) <= 2e-3 * max(1.0, abs(lrf[n]))
        # rows that are not special are left alone
        assert float(np.abs(og[0, h, 5:lay.frame_len]).max()) == 0.0


# --------------------------------------------------------------------------
# value-aware selection with pair memory
# --------------------------------------------------------------------------
def check_vasc(lay, vals, keep, force, mem_before, rpn, cin, stat_g, dem_g, mem_after_g,
               rows_to_check=None):
    """Selection of one layer against the oracle's demand and ranking (rows a
    valid top-k by rho up to the 1e-4 gap), and the memory update against the
    oracle's demand and the GPU's own executed flags."""
    q, k, v = vals
    nb = lay.nblocks
    parity.check_csr_wellformed(rpn, cin, nb)
    rows = parity.csr_rows(rpn, cin)
    forced = oracle.forced_blocks(lay, force)
    mism = 0
    for b in range(lay.batch):
        for h in range(lay.heads):
            sl = (slice(b, b + 1), slice(h, h + 1))
            qbar = oracle.pool(q[sl], lay)[0, 0]
            kbar = oracle.pool(k[sl], lay)[0, 0]
            vbar = oracle.pool(v[sl], lay)[0, 0]
            p = oracle.row_softmax(lay.scale * (qbar @ kbar.T))
            c = oracle.pair_contrast(vbar)
            mhat = oracle.memory_rank_copy(mem_before[b, h])
            kh = int(keep[h])
            d = np.zeros((nb, nb))
            x = np.zeros((nb, nb))
            for i in range(nb):
                r = (b * lay.heads + h) * nb + i
                _, d[i] = oracle.demand_row(p[i], c, kh)
                x[i, rows[r]] = 1.0
                if rows_to_check is not None and i not in rows_to_check:
                    continue
                rho = d[i] + mhat[np.arange(nb) // 2]
                exact = oracle.select_topk_row(rho, kh, forced)
                if rows[r] != exact:
                    mism += 1
                    assert parity.topk_valid(rows[r], rho, kh, forced), \
                        f"row {(b, h, i)}: {rows[r]} vs oracle {exact}"
                assert abs(stat_g[r] - p[i, rows[r]].sum()) < 1e-4
                if dem_g is not None:
                    assert np.abs(dem_g[b, h, i] - d[i]).max() <= 1e-5, (b, h, i)
            want = oracle.memory_update(mem_before[b, h], d, x)
            assert np.abs(mem_after_g[b, h] - want).max() <= 1e-5, (b, h)
    return mism


def run_vasc_layers(dev, lay, host, vals, keep, force, layers, rows_to_check=None, label=""):
    q, k, v = (to_dev(x_, dev) for x_ in host)
    nb = lay.nblocks
    mem = torch.zeros((lay.batch, lay.heads, bsgm.vasc_pairs(lay)), dtype=torch.float32,
                      device=dev)
    dem = torch.empty((lay.batch, lay.heads, nb, nb), dtype=torch.float32, device=dev)
    total = 0
    for layer in range(layers):
        before = mem.cpu().numpy().astype(np.float64)
        rp, ci, st = bsgm.vasc_select_blocks(lay, keep, q, k, v, mem, force=force, demand_out=dem)
        torch.cuda.synchronize()
        mism = check_vasc(lay, vals, keep, force, before, rp.cpu().numpy(), ci.cpu().numpy(),
                          st.cpu().numpy(), dem.cpu().numpy(), mem.cpu().numpy().astype(np.float64),
                          rows_to_check)
        total += mism
        say(f"vasc {label} layer {layer}: near-tie rows {mism}, "
            f"max deficit {float(mem.max()):.4f}")
    return total


@pytest.mark.parametrize("dtype,block,force", [("bf16", 64, False), ("bf16", 128, True),
                                               ("f32", 64, True), ("f32", 128, False)])
def test_vasc_small_layouts_three_layers(dev, dtype, block, force):
    """Ragged layouts with 40 (block 64) or 33 (block 128: odd, a singleton
    pair) key blocks, two heads and batch 2, three layers carrying the memory."""
    frames, per = (10, 4) if block == 64 else (11, 3)
    lay = custom_layout(frames, per * block, per * block - 37, block, heads=2, dtype=dtype, batch=2)
    host, vals = random_inputs(lay, 81 + block)
    nf = frames if force else 0
    keep = np.array([max(8, nf + 2), max(5, nf + 1)], dtype=np.int32)
    say(f"vasc small {dtype} block {block} force {force}: nb {lay.nblocks}")
    run_vasc_layers(dev, lay, host, vals, keep, force, 3, label="small")


@pytest.mark.parametrize("seed", range(8))
def test_vasc_random_layouts(dev, seed):
    """Value-aware selection with pair memory on seeded random layouts (frames,
    frame length in whole blocks, padding under one block, block 64 or 128,
    fp32 or bf16, batch, heads, budgets covering the forced blocks, odd and
    even block counts), two to four layers carrying the memory: every row and
    every pair against the oracle."""
    rng = np.random.default_rng(5000 + seed)
    block = (64, 128)[seed % 2]
    dtype = "f32" if seed % 3 == 0 else "bf16"
    frames = int(rng.integers(2, 9))
    frame_len = block * int(rng.integers(1, 6))
    lay = custom_layout(frames, frame_len, frame_len - int(rng.integers(0, block)), block,
                        heads=int(rng.integers(1, 3)), dtype=dtype, batch=int(rng.integers(1, 3)))
    force = bool(rng.integers(0, 2))
    lo = max(1, len(oracle.forced_blocks(lay, force)))
    keep = np.array([int(rng.integers(lo, max(lo, lay.nblocks - 1) + 1))
                     for _ in range(lay.heads)], dtype=np.int32)
    layers = int(rng.integers(2, 5))
    say(f"vasc sweep seed {seed}: frames {lay.frames}x{lay.frame_len} ({lay.frame_valid} real), "
        f"block {block}, {dtype}, batch {lay.batch}, heads {lay.heads}, nb {lay.nblocks}, "
        f"keep {keep.tolist()}, force {force}, layers {layers}")
    host, vals = random_inputs(lay, 6000 + seed)
    run_vasc_layers(dev, lay, host, vals, keep, force, layers, label=f"sweep seed {seed}")


def test_vasc_layer32_full_size_sampled(dev):
    """The 32-frame layer (16 heads, 352 blocks, 88 kept with the 32 forced
    special blocks): two layers, sampled rows, every pair's memory."""
    w, data = preset(2)
    lay = w.layout
    host = [data[n + "_bits"] for n in ("q", "k", "v")]
    vals = (data["q"], data["k"], data["v"])
    say("vasc 32 frames full size")
    run_vasc_layers(dev, lay, host, vals, data["keep"], True, 2,
                    rows_to_check={0, 1, 10, 11, 175, 351}, label="32 frames")


@pytest.mark.parametrize("nb", [1099, 301])
def test_vasc_wide_rows(dev, nb):
    """Rows of 1099 and 301 key blocks (odd: a singleton pair), so the
    value-aware mode runs in the 24- and 8-block-per-lane register layouts."""
    lay = custom_layout(7, 64 * (nb // 7), 64 * (nb // 7) - 30, 64, heads=1)
    assert lay.nblocks == nb
    host, vals = random_inputs(lay, 13 + nb)
    keep = np.array([max(9, nb // 5)], dtype=np.int32)
    say(f"vasc wide rows: nb {nb}, keep {int(keep[0])}")
    run_vasc_layers(dev, lay, host, vals, keep, True, 2,
                    rows_to_check={0, 1, nb // 2, nb - 2, nb - 1}, label=f"wide {nb}")
