#!/usr/bin/env python3
"""Benchmark of one block-sparse global-attention layer on one MI355X.

A step is the whole hot path on one batch of resident synthetic input:
pooled top-k block selection (mean-pool Q and K per block, pooled scores,
per-frame special-token blocks forced, CSR emission) followed by the
block-sparse flash-attention forward over the selected blocks. The workload is
the 32-frame layer: 32 x 1408 padded tokens (1374 real), 16 heads, head_dim 64,
bf16, blocks of 128, 75 % block sparsity.

Prints one JSON line (see the keys below). `value` is the layer-effective
throughput: algorithmic FLOP of the executed blocks (4 * 128^2 * 64 per
executed block pair) divided by the measured time of the whole step. The
step pools Q and K in one launch (`pool_blocks2`), then selects from the pooled means
(`select_blocks_pooled`) while a second stream makes the fp16 copy of K
(`attn_prepare`), so the copy's HBM stream overlaps the selection kernel
rather than the pooling. The prepared attention call then runs the
fp16-logit attention kernel and the bf16 launch for rows left over (none
here); `roofline.achieved` divides the FLOP by the duration of that call.
`detail.other_layers` gives the per-layer times of the other presets (8 frames
at 50 %, 100 frames with the cumulative-mass rule and per-head caps, 16 frames
with drift selection and three restoration rounds), each phase timed over
back-to-back launches; `detail.special_rows_dense` and `detail.vasc_selection`
time the dense camera/register rows and the value-aware selection with pair
memory on the bench layer, `detail.graph_replay` the same step (both
streams) captured once in a HIP graph and replayed, and `detail.cold` one step after a 512 MiB write
has evicted the caches (median of 3). All are side measurements, not part of
`value`.

Per preset (`detail.other_layers`, the bench layer included, and the tiny
fp32 layer), `selection_phases` times pooling, selection from the means and
the whole selection call (or drift scores and drift selection) both back to
back ("cache_warm_gbs": the inputs may still sit in the L2 and Infinity
caches) and after a 512 MiB write ("cold_hbm_gbs", the figure that speaks for
HBM), each against its algorithmic bytes (real-token inputs read once, outputs
written once); `workspace_mib` gives the device scratch of each call.
`detail.drift_100_frames` runs drift selection on the 100-frame layer (1 100
key blocks per row): contributions materialised, five re-rank rounds with
track-best (and, timed beside it, 3 best-swap rounds), attention; the
16-frame drift layer also times re-rank rounds at 5 and 10 rounds. `detail.attn_prepare_ms` is the fp16 copy of K alone (it runs beside the
selection in the step), `attn_with_prepare_frac` the attention's roofline
fraction with that time charged too, and `attn_rows_bf16_form` the rows the
fp16-logit form handed to the bf16 form. `cpu_baseline` times the oracle on
the host in float64 (`value`) and float32, BLAS threads pinned to the cores in
this process's affinity mask.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_vggt_layer_32f_s75_traffic.json")
CSRC = os.path.join(ROOT, "block_sparse_global_mean_amd", "csrc")
# the translation unit of the attention kernel
ATTN_SRCS = [os.path.join(CSRC, f) for f in ("attn_bf16.hip", "device_util.h", "internal.h")]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for path in ATTN_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_per_launch():
    """HBM bytes per attention launch from the committed counter summary, or
    None if there is none or the kernel source changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def to_dev(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def cpu_info():
    """(model name, number of cores this process may run on) of the host."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    cores = len(os.sched_getaffinity(0))
    return model, cores


def oracle_sample(w, data, budget_s: float, dtype):
    """The oracle, as it stands, on a bounded sample of the bench layer in the
    given float type: head by head, pooled scores and top-k selection, then
    block-sparse attention per query block, until about `budget_s` seconds."""
    import oracle
    lay = w.layout
    keep = data["keep"]
    forced = oracle.forced_blocks(lay, w.force_frame_first_block)
    t0 = time.perf_counter()
    pairs = rows = heads = 0
    for h in range(lay.heads):
        q, k, v = data["q"][:, h:h + 1], data["k"][:, h:h + 1], data["v"][:, h:h + 1]
        qbar, kbar = oracle.pool(q, lay, dtype), oracle.pool(k, lay, dtype)
        s = oracle.pooled_scores(qbar, kbar, lay.scale)[0, 0]
        heads += 1
        for i in range(lay.nblocks):
            kept = oracle.select_topk_row(s[i], int(keep[h]), forced)
            oracle.sparse_attention_row(q[0, 0], k[0, 0], v[0, 0], lay, i, kept, dtype)
            pairs += len(kept)
            rows += 1
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    flops = pairs * 4.0 * lay.block ** 2 * lay.head_dim
    return {"value": flops / dt / 1e12, "seconds": round(dt, 3),
            "sample": f"the 32-frame layer, head by head until the time budget: pooling and "
                      f"pooled scores of {heads} head(s), then top-k selection + "
                      f"{np.dtype(dtype).name} block-sparse attention for {rows} of "
                      f"{lay.heads * lay.nblocks} query blocks ({pairs} executed block "
                      f"pairs, {flops / 1e9:.1f} GFLOP)"}


def cpu_baseline(w, data, budget_s: float):
    """The oracle on the host cores: float64 (the parity oracle, `value`) and
    float32 (the GPU's accumulation precision), each on a bounded sample, with
    BLAS threads pinned to the cores this process may run on."""
    model, cores = cpu_info()
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:
        limiter = None
    try:
        r64 = oracle_sample(w, data, budget_s, np.float64)
        r32 = oracle_sample(w, data, budget_s * 0.5, np.float32)
    finally:
        if limiter is not None:
            limiter.restore_original_limits()
    return {"value": r64["value"], "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "cpu_model": model, "seconds": r64["seconds"], "sample": r64["sample"],
            "fp32": {"value": r32["value"], "seconds": r32["seconds"], "sample": r32["sample"]}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=20)   # the card's clock settles over ~10 steps
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, copy this many MiB once (counter calibration)")
    ap.add_argument("--no-side", "--no-drift", dest="no_side", action="store_true",
                    help="skip the side measurements (other presets, value-aware selection)")
    ap.add_argument("--layer", default=None,
                    help="time only this other preset (e.g. vggt_layer_16f_drift) and print "
                         "its per-layer JSON; for profiling its kernels")
    ap.add_argument("--drift-wide", action="store_true",
                    help="time only the drift selection on the 100-frame layer (stored and "
                         "streamed forms) and print its JSON; for profiling its kernels")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import torch
    import block_sparse_global_mean_amd as bsgm
    import workloads

    dev = torch.device("cuda:0")
    bsgm.library()
    if args.layer:
        res = side_config(bsgm, workloads, torch, dev, args.layer, args.steps)
        calibration_copy(torch, dev, args.calib_copy_mib)
        print(json.dumps({"layer": args.layer, **res}), flush=True)
        return
    if args.drift_wide:
        res = drift_wide_layer(bsgm, workloads, torch, dev)
        print(json.dumps({"drift_100_frames": res}), flush=True)
        return
    w = workloads.config("vggt_layer_32f_s75")
    lay = w.layout
    log(f"generating {w.name}")
    data = workloads.generate(w)
    q, k, v = (to_dev(data[n + "_bits"], dev) for n in ("q", "k", "v"))
    keep = data["keep"]
    nb, rows = lay.nblocks, lay.batch * lay.heads * lay.nblocks
    cap = bsgm.col_capacity(lay, bsgm.TOPK, keep, force=True)
    row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(cap, dtype=torch.int32, device=dev)
    ws = torch.empty(bsgm.workspace_bytes(lay, bsgm.TOPK), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    aws = torch.empty(bsgm.attn_workspace_bytes(lay), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def select():
        bsgm.select_blocks(lay, bsgm.TOPK, keep, q=q, k=k, force=True, row_ptr=row_ptr,
                           col_idx=col_idx, workspace=ws, want_stat=False)

    def attend():
        bsgm.sparse_attn_fwd(lay, q, k, v, row_ptr, col_idx, o=o, workspace=aws)

    # The timed step: Q and K are pooled, then the fp16 copy of K (which
    # depends on K only) runs on a second stream while the selection kernel
    # works from the pooled means; the attention call then skips the copy.
    # The side stream waits for the pooling (and so for the previous step's
    # attention, which reads the same workspace): the copy's HBM stream then
    # overlaps the latency-bound selection instead of the HBM-bound pooling.
    side = torch.cuda.Stream()
    qbar = torch.empty((lay.batch, lay.heads, nb, lay.head_dim), dtype=torch.float32, device=dev)
    kbar = torch.empty_like(qbar)

    def pool():
        bsgm.pool_blocks2(lay, q, k, out0=qbar, out1=kbar)

    def prepare_side():
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            bsgm.attn_prepare(lay, k, aws)

    def select_pooled():
        bsgm.select_blocks_pooled(lay, bsgm.TOPK, keep, qbar, kbar, force=True, row_ptr=row_ptr,
                                  col_idx=col_idx, want_stat=False)

    def attend_prepared():
        torch.cuda.current_stream().wait_stream(side)
        bsgm.sparse_attn_fwd(lay, q, k, v, row_ptr, col_idx, o=o, workspace=aws, prepared=True)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        pool()
        prepare_side()
        select_pooled()
        attend_prepared()
    torch.cuda.synchronize()
    executed = int(row_ptr[-1].item())
    flops = executed * 4.0 * lay.block ** 2 * lay.head_dim

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    ev_all = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    log(f"timing {K} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_all[0].record(stream)
    for s in range(K):
        ev[s][0].record(stream)
        pool()
        prepare_side()
        select_pooled()
        ev[s][1].record(stream)
        attend_prepared()
        ev[s][2].record(stream)
    ev_all[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = ev_all[0].elapsed_time(ev_all[1])
    sel_ms = [ev[s][0].elapsed_time(ev[s][1]) for s in range(K)]
    att_ms = [ev[s][1].elapsed_time(ev[s][2]) for s in range(K)]
    ms_per_step = max(total_ms, wall * 1e3) / K
    attn_avg = float(np.mean(att_ms))
    achieved = flops / (attn_avg * 1e-3) / 1e12
    log(f"step {ms_per_step:.3f} ms (select {np.mean(sel_ms):.3f}, attention {attn_avg:.3f})")

    def step():
        pool()
        prepare_side()
        select_pooled()
        attend_prepared()

    graph = None if args.no_side else graph_step(torch, step, K)
    calibration_copy(torch, dev, args.calib_copy_mib)

    traffic = traffic_per_launch()
    detail = {
        "select_ms": round(float(np.mean(sel_ms)), 4),
        "attn_ms": round(attn_avg, 4),
        "attn_ms_min": round(float(np.min(att_ms)), 4),
        "attn_ms_median": round(float(np.median(att_ms)), 4),
        "select_ms_median": round(float(np.median(sel_ms)), 4),
        "executed_block_pairs": executed,
        "measured_block_sparsity": round(1.0 - executed / (rows * nb), 6),
        "executed_gflop": round(flops / 1e9, 3),
        "attn_effective_tflops": round(achieved, 2),
        "device": device_info(torch),
        "graph_replay": graph,
    }
    # the fp16 copy of K (on the side stream in the step, beside the selection)
    # timed alone, and the attention fraction with its time charged as well
    prep_ms = gpu_ms(torch, lambda: bsgm.attn_prepare(lay, k, aws), 20)
    detail["attn_prepare_ms"] = round(prep_ms, 4)
    detail["attn_with_prepare_frac"] = round(
        flops / ((attn_avg + prep_ms) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
    # rows the fp16-logit form handed to the bf16 form (its range flags)
    al = lambda x: (x + 255) // 256 * 256
    redo = aws[al(lay.batch * lay.heads * lay.tokens * 64 * 2) + al(rows * 4):].view(torch.int32)
    detail["attn_rows_bf16_form"] = int(redo[:rows].sum().item())
    flush = None
    if not args.no_side:
        flush = torch.empty(512 * (1 << 20) // 4, dtype=torch.float32, device=dev)
        detail["cold"] = cold_step(torch, dev, select, attend, flush)

    # the same selection with pooling and selection in one launch, timed alone
    # beside the two-launch form over back-to-back launches
    fws = torch.zeros(bsgm.fused_workspace_bytes(lay), dtype=torch.uint8, device=dev)
    rp1, ci1 = torch.empty_like(row_ptr), torch.empty_like(col_idx)

    def select_fused():
        bsgm.select_blocks_fused(lay, keep, q, k, force=True, row_ptr=rp1, col_idx=ci1,
                                 workspace=fws, want_stat=False)

    two_ms = gpu_ms(torch, select, 20)
    one_ms = gpu_ms(torch, select_fused, 20)
    select()
    torch.cuda.synchronize()
    detail["select_one_launch"] = {
        "ms": round(one_ms, 4), "two_launch_ms": round(two_ms, 4),
        "same_csr": bool(torch.equal(rp1, row_ptr) and torch.equal(ci1, col_idx))}

    # dense camera/register rows (5 per frame) on the same layer, after the sparse pass
    ns = 5
    sws = torch.empty(bsgm.special_rows_workspace_bytes(lay, ns), dtype=torch.uint8, device=dev)
    sp_ms = gpu_ms(torch, lambda: bsgm.special_rows_dense_fwd(lay, q, k, v, ns, o, workspace=sws),
                   10)
    real_keys = lay.frames * lay.frame_valid
    sp_flops = 4.0 * lay.batch * lay.heads * lay.frames * ns * real_keys * lay.head_dim
    detail["special_rows_dense"] = {
        "rows_per_frame": ns, "ms": round(sp_ms, 4),
        "gflop": round(sp_flops / 1e9, 3),
        "tflops": round(sp_flops / (sp_ms * 1e-3) / 1e12, 2)}

    if not args.no_side:
        # value-aware selection with pair memory on the same layer and budget; each
        # call is one layer (the memory carries over), timed over back-to-back calls
        vmem = torch.zeros((lay.batch, lay.heads, bsgm.vasc_pairs(lay)), dtype=torch.float32,
                           device=dev)
        vws = torch.empty(bsgm.workspace_bytes(lay, bsgm.VASC), dtype=torch.uint8, device=dev)

        def vasc_select():
            bsgm.vasc_select_blocks(lay, keep, q, k, v, vmem, force=True, row_ptr=row_ptr,
                                    col_idx=col_idx, workspace=vws, want_stat=False)
        vasc_warm, vasc_reps = 10, 10
        vasc_ms = gpu_ms(torch, vasc_select, vasc_reps, warm=vasc_warm)
        vasc_attn_ms = gpu_ms(torch, attend, 5)
        detail["vasc_selection"] = {
            "select_ms": round(vasc_ms, 4), "attn_ms": round(vasc_attn_ms, 4),
            "layers_carried": vasc_warm + vasc_reps, "max_pair_deficit": round(float(vmem.max()), 4),
            "executed_block_pairs": int(row_ptr[-1].item())}
        detail["other_layers"] = {
            name: side_config(bsgm, workloads, torch, dev, name, flush=flush)
            for name in ("tiny_f32_1024tok", "vggt_layer_8f_s50", "vggt_layer_32f_s75",
                         "vggt_layer_100f_cdf", "vggt_layer_16f_drift")}
        detail["drift_100_frames"] = drift_wide_layer(bsgm, workloads, torch, dev)

    out = {
        "metric": "block-sparse global attn effective TFLOP/s + ms/layer, 32 frames, 75% sparse",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "vggt_layer_32f_s75: 32 frames x 1408 tokens (1374 real), "
                               "16 heads, head_dim 64, block 128, top-88 of 352 key blocks "
                               "per query block with 32 forced special-token blocks",
                   "batch": lay.batch, "heads": lay.heads, "tokens": lay.tokens,
                   "block": lay.block, "keep_per_query_block": int(keep[0]),
                   "attention_arithmetic": "QK^T on fp16 MFMA (K copied to fp16, "
                                           "q*scale*log2e rounded to fp16) for query blocks "
                                           "whose |q*scale*log2e| and listed |k| stay below "
                                           "128, else bf16 MFMA; PV on bf16 MFMA; fp32 "
                                           "accumulation and softmax; bf16 output"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "detail": detail,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(w, data, args.cpu_budget)
    print(json.dumps(out), flush=True)


def device_info(torch):
    """Name, compute units and architecture of cuda:0 as the runtime reports them."""
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "compute_units": p.multi_processor_count,
            "arch": getattr(p, "gcnArchName", "")}


def cold_step(torch, dev, select, attend, flush, reps: int = 3):
    """One step after writing the 512 MiB `flush` buffer, which evicts the L2
    caches and the 256 MB Infinity Cache; the median of `reps` such steps
    (side measurement)."""
    stream = torch.cuda.current_stream()
    sel, att = [], []
    for r in range(reps):
        flush.fill_(float(r))
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        select()
        e[1].record(stream)
        attend()
        e[2].record(stream)
        torch.cuda.synchronize()
        sel.append(e[0].elapsed_time(e[1]))
        att.append(e[1].elapsed_time(e[2]))
    return {"select_ms": round(float(np.median(sel)), 4), "attn_ms": round(float(np.median(att)), 4),
            "flush_mib": 512, "reps": reps}


def graph_step(torch, step, reps: int):
    """The same step, both streams included, captured once in a HIP graph and
    replayed `reps` times (side measurement: launch overhead is all it can
    remove)."""
    try:
        warm = torch.cuda.Stream()
        warm.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(warm):
            step()
        torch.cuda.current_stream().wait_stream(warm)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        g.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return {"step_ms": round(e0.elapsed_time(e1) / reps, 4), "replays": reps}
    except Exception as exc:   # a side measurement must not cost the bench line
        return {"error": str(exc)[:200]}


def calibration_copy(torch, dev, mib: int):
    """One device copy of `mib` MiB: a transfer of known size for scaling the
    HBM byte counters."""
    if mib <= 0:
        return
    src = torch.ones(mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"calibration copy of {mib} MiB done")


def gpu_ms(torch, fn, reps: int, warm: int = 10) -> float:
    """Average GPU time of fn over `reps` back-to-back launches on the current
    stream (HIP events), after `warm` untimed calls (the card's clock settles
    over about ten calls of the larger kernels)."""
    stream = torch.cuda.current_stream()
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def cold_ms(torch, fn, flush, reps: int = 3) -> float:
    """Median GPU time of fn, each call right after a write of the 512 MiB `flush`
    buffer, which evicts the L2 caches and the 256 MB Infinity Cache: the
    inputs then come from HBM."""
    stream = torch.cuda.current_stream()
    times = []
    for r in range(reps):
        flush.fill_(float(r))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return float(np.median(times))


def rate(nbytes: float, ms: float) -> float:
    return round(nbytes / (ms * 1e-3) / 1e9, 1)


def mib(nbytes: float) -> float:
    return round(nbytes / (1 << 20), 2)


def drift_wide_layer(bsgm, workloads, torch, dev, reps: int = 3):
    """Drift selection on the 100-frame layer (1 100 key blocks per row, 16 heads,
    keep 220 = 80 % sparsity): contributions materialised in HBM, then five
    re-rank rounds with track-best, then the attention over the kept blocks;
    the best-swap rule at 3 rounds is timed beside it."""
    w = workloads.config("vggt_layer_100f_cdf")
    lay = w.layout
    log("generating the 100-frame layer for drift selection")
    data = workloads.generate(w)
    q, k, v = (to_dev(data[n + "_bits"], dev) for n in ("q", "k", "v"))
    del data
    nb, rows = lay.nblocks, lay.batch * lay.heads * lay.nblocks
    keep = [nb - int(round(0.8 * nb))] * lay.heads
    contrib = torch.empty((lay.batch, lay.heads, nb, nb, 64), dtype=torch.float32, device=dev)
    score = torch.empty((lay.batch, lay.heads, nb, nb), dtype=torch.float32, device=dev)
    ws = torch.empty(bsgm.workspace_bytes(lay, bsgm.DRIFT), dtype=torch.uint8, device=dev)
    row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(bsgm.col_capacity(lay, bsgm.DRIFT, keep), dtype=torch.int32, device=dev)
    aws = torch.empty(bsgm.attn_workspace_bytes(lay), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)

    def scores():
        bsgm.drift_scores(lay, q, k, v, contrib=contrib, score=score, workspace=ws)

    def select():
        bsgm.select_blocks(lay, bsgm.DRIFT, keep, contrib=contrib, swap_rounds=5,
                           row_ptr=row_ptr, col_idx=col_idx, want_stat=False,
                           restoration=bsgm.RERANK_TRACK_BEST)

    def attend():
        bsgm.sparse_attn_fwd(lay, q, k, v, row_ptr, col_idx, o=o, workspace=aws)
    def select_best_swap():
        bsgm.select_blocks(lay, bsgm.DRIFT, keep, contrib=contrib, swap_rounds=3,
                           row_ptr=row_ptr, col_idx=col_idx, want_stat=False)
    sc_ms = gpu_ms(torch, scores, reps)
    bs_ms = gpu_ms(torch, select_best_swap, reps)
    sel_ms = gpu_ms(torch, select, reps)
    at_ms = gpu_ms(torch, attend, reps)
    executed = int(row_ptr[-1].item())
    scoring_mib = mib(contrib.numel() * 4 + score.numel() * 4 + ws.numel())
    del contrib, score, ws
    torch.cuda.empty_cache()
    # the same selection in the expanded form, with no contributions allocated
    sws = torch.empty(bsgm.drift_streamed_workspace_bytes(lay), dtype=torch.uint8, device=dev)

    def select_streamed():
        bsgm.select_drift_streamed(lay, keep, q, k, v, swap_rounds=5, track_best=True,
                                   row_ptr=row_ptr, col_idx=col_idx, workspace=sws,
                                   want_stat=False)
    st_ms = gpu_ms(torch, select_streamed, reps)
    out = {"keep_per_query_block": keep[0], "rounds": 5, "restoration": "re-rank, track-best",
           "drift_scores_ms": round(sc_ms, 4), "drift_select_ms": round(sel_ms, 4),
           "best_swap_3_rounds_select_ms": round(bs_ms, 4),
           "attn_ms": round(at_ms, 4), "ms_per_layer": round(sc_ms + sel_ms + at_ms, 4),
           "executed_block_pairs": executed,
           "scoring_memory_mib": scoring_mib,
           "streamed_scores_and_select_ms": round(st_ms, 4),
           "streamed_scoring_memory_mib": mib(sws.numel()),
           "attn_effective_tflops": round(executed * 4.0 * 128 * 128 * 64 / (at_ms * 1e-3) / 1e12,
                                          2)}
    del sws, q, k, v, o
    torch.cuda.empty_cache()
    return out


def side_config(bsgm, workloads, torch, dev, name: str, reps: int = 5, flush=None):
    """Per-layer times of a preset: selection (drift scores + restoration for the
    drift preset) and attention, each timed over back-to-back launches. The
    selection's phases are also timed alone, warm (back to back, inputs still in
    the caches) and cold (after `flush` has evicted them), with their
    algorithmic bytes (real-token inputs read once, outputs written once) over
    the time; only the cold rate speaks for HBM. Also the device memory each
    phase needs besides inputs and outputs (workspace)."""
    w = workloads.config(name)
    lay = w.layout
    log(f"generating {w.name}")
    data = workloads.generate(w)
    if lay.dtype == "bf16":
        q, k, v = (to_dev(data[n + "_bits"], dev) for n in ("q", "k", "v"))
    else:
        q, k, v = (torch.from_numpy(np.ascontiguousarray(data[n])).to(dev) for n in ("q", "k", "v"))
    esize = 2 if lay.dtype == "bf16" else 4
    keep = data["keep"]
    nb, rows = lay.nblocks, lay.batch * lay.heads * lay.nblocks
    real = lay.batch * lay.heads * lay.frames * lay.frame_valid
    tensor_real = real * lay.head_dim * esize          # real-token bytes of Q, K or V
    pooled = rows * lay.head_dim * 4
    row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    cap = max(bsgm.col_capacity(lay, w.mode, keep, w.force_frame_first_block), 1)
    col_idx = torch.empty(cap, dtype=torch.int32, device=dev)
    ws_bytes = bsgm.workspace_bytes(lay, w.mode)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    out = {}
    phases = {}

    def phase(label, fn, nbytes):
        warm = gpu_ms(torch, fn, reps)
        ent = {"ms": round(warm, 4), "bytes": int(nbytes), "cache_warm_gbs": rate(nbytes, warm)}
        if flush is not None:
            cold = cold_ms(torch, fn, flush)
            ent.update({"cold_ms": round(cold, 4), "cold_hbm_gbs": rate(nbytes, cold)})
        phases[label] = ent
        return warm

    if w.mode == bsgm.DRIFT:
        contrib = torch.empty((lay.batch, lay.heads, nb, nb, 64), dtype=torch.float32, device=dev)
        score = torch.empty((lay.batch, lay.heads, nb, nb), dtype=torch.float32, device=dev)
        zmass = torch.empty((lay.batch, lay.heads, nb, nb), dtype=torch.float32, device=dev)

        def scores():
            bsgm.drift_scores(lay, q, k, v, contrib=contrib, score=score, workspace=ws)

        def select():
            bsgm.select_blocks(lay, bsgm.DRIFT, keep, contrib=contrib, swap_rounds=w.swap_rounds,
                               force=w.force_frame_first_block, row_ptr=row_ptr,
                               col_idx=col_idx, want_stat=False)

        def scores_z():
            bsgm.drift_scores(lay, q, k, v, contrib=contrib, score=score, workspace=ws,
                              zmass=zmass)

        def select_z():
            bsgm.select_blocks(lay, bsgm.DRIFT, keep, contrib=contrib, swap_rounds=w.swap_rounds,
                               force=w.force_frame_first_block, row_ptr=row_ptr,
                               col_idx=col_idx, want_stat=False,
                               objective=bsgm.RENORMALISED, zmass=zmass)
        chat_bytes = rows * nb * 64 * 4
        csr_bytes = 4 * (rows + 1) + 4 * lay.batch * nb * int(np.sum(keep))
        # the renormalised objective on the same layer (scores with block masses)
        out["renorm_drift_scores_ms"] = round(gpu_ms(torch, scores_z, reps), 4)
        out["renorm_drift_select_ms"] = round(gpu_ms(torch, select_z, reps), 4)
        out["drift_scores_ms"] = round(phase(
            "drift_scores", scores, 3 * tensor_real + chat_bytes + rows * nb * 4), 4)
        out["drift_select_ms"] = round(phase("drift_select", select, chat_bytes + csr_bytes), 4)
        # the re-rank restoration rule at the round counts of ReSS Table S3
        for rr_rounds in (5, 10):
            def select_rr(rounds=rr_rounds):
                bsgm.select_blocks(lay, bsgm.DRIFT, keep, contrib=contrib, swap_rounds=rounds,
                                   force=w.force_frame_first_block, row_ptr=row_ptr,
                                   col_idx=col_idx, want_stat=False,
                                   restoration=bsgm.RERANK_TRACK_BEST)
            out[f"rerank_track_best_{rr_rounds}_rounds_select_ms"] = round(
                gpu_ms(torch, select_rr, reps), 4)
        # the 5-round re-rank in the expanded form (scores and selection from
        # Q, K and V, no contributions)
        sws = torch.empty(bsgm.drift_streamed_workspace_bytes(lay), dtype=torch.uint8, device=dev)

        def select_streamed():
            bsgm.select_drift_streamed(lay, keep, q, k, v, swap_rounds=5, track_best=True,
                                       force=w.force_frame_first_block, row_ptr=row_ptr,
                                       col_idx=col_idx, workspace=sws, want_stat=False)
        out["streamed_rerank_track_best_5_rounds_ms"] = round(gpu_ms(torch, select_streamed, reps),
                                                              4)
        out["streamed_workspace_mib"] = mib(sws.numel())
        del sws
        sel = out["drift_scores_ms"] + out["drift_select_ms"]
        out["workspace_mib"] = {"drift_scores": mib(ws_bytes),
                                "contributions_and_scores": mib(chat_bytes + 2 * rows * nb * 4)}
    else:
        def select():
            bsgm.select_blocks(lay, w.mode, keep, q=q, k=k, cdf_tau=w.cdf_tau,
                               force=w.force_frame_first_block, row_ptr=row_ptr,
                               col_idx=col_idx, workspace=ws, want_stat=False)
        qbar = torch.empty((lay.batch, lay.heads, nb, lay.head_dim), dtype=torch.float32,
                           device=dev)
        kbar = torch.empty_like(qbar)

        def pool():
            bsgm.pool_blocks(lay, q, out=qbar)
            bsgm.pool_blocks(lay, k, out=kbar)

        def select_pooled():
            bsgm.select_blocks_pooled(lay, w.mode, keep, qbar, kbar, cdf_tau=w.cdf_tau,
                                      force=w.force_frame_first_block, row_ptr=row_ptr,
                                      col_idx=col_idx, workspace=ws, want_stat=False)
        pool()
        select()
        torch.cuda.synchronize()
        csr_bytes = 4 * (rows + 1) + 4 * int(row_ptr[-1].item())
        phase("pool_q_k", pool, 2 * tensor_real + 2 * pooled)
        phase("select_from_means", select_pooled, 2 * pooled + csr_bytes)
        out["select_ms"] = round(phase("select", select, 2 * tensor_real + csr_bytes), 4)
        sel = out["select_ms"]
        out["workspace_mib"] = {"select": mib(ws_bytes)}

    aws_bytes = bsgm.attn_workspace_bytes(lay)
    aws = torch.empty(aws_bytes, dtype=torch.uint8, device=dev) if aws_bytes else None
    out["workspace_mib"]["attention"] = mib(aws_bytes)

    def attend():
        bsgm.sparse_attn_fwd(lay, q, k, v, row_ptr, col_idx, o=o, workspace=aws)
    select()
    attn = gpu_ms(torch, attend, reps)
    executed = int(row_ptr[-1].item())
    flops = executed * 4.0 * lay.block ** 2 * lay.head_dim
    out.update({
        "attn_ms": round(attn, 4),
        "ms_per_layer": round(sel + attn, 4),
        "executed_block_pairs": executed,
        "measured_block_sparsity": round(1.0 - executed / (rows * nb), 6),
        "attn_effective_tflops": round(flops / (attn * 1e-3) / 1e12, 2),
        "layer_effective_tflops": round(flops / ((sel + attn) * 1e-3) / 1e12, 2),
        "selection_phases": phases,
    })
    del q, k, v, o, data
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
