#!/usr/bin/env python3
"""Benchmark of absorbed MLA decode on one MI355X.

One step = one mla_decode call (one MLA layer for the whole batch, including
the merge of split requests) on inputs already resident in HBM.  The step is
enqueued as its two halves (mla_decode_attend, then mla_decode_merge) with an
event between them, so the decode kernel's own duration is measured live on
the launch stream; that duration prices the roofline.  The default
workload is the per-GPU share the pages time their B200 kernels on: 16
requests x 100000 tokens, q_len 5 (causal among the drafts), 96 heads, FP8
e4m3fn latent KV with a per-token scale, BF16 queries.

Prints ONE JSON line (metric: us/layer, lower is better) with a `roofline`
object for the decode kernel and a `cpu_baseline` object (the float64 oracle
timed on a bounded sample of the same workload, scaled to the whole layer).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode us/layer + achieved KV HBM TB/s (% of peak) at 100k ctx, q_len 5"
HBM_PEAK_TBPS = 8.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure
MFMA_FP8_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 (e4m3) MFMA, vendor figure


def mfma_peak_tflops(kv_dtype: str) -> float:
    """MFMA peak that prices the decode kernel's algorithmic FLOPs.

    BF16 KV: the bf16 dense peak (2.5 PFLOP/s).  FP8, FP4 and MXFP8 KV: the
    e4m3 dense peak (5.0 PFLOP/s), the rate of the scaled f8f6f4 MFMA that
    takes these stored codes as operands (an FP4 key against a query that is
    not FP4 runs at the FP8 rate).  Whatever the kernel does to keep the
    products exact (two e4m3 terms per query and probability, or widening to
    BF16) is charged to the kernel, not to the peak.
    """
    return MFMA_BF16_PEAK_TFLOPS if kv_dtype == "bf16" else MFMA_FP8_PEAK_TFLOPS


def measured_hbm_peak():
    """The HBM read rate measured on an MI355X by bench.py --hbm-peak, from
    profiles/hbm_peak.txt (TB/s), or None when that summary is missing."""
    path = os.path.join(ROOT, "profiles", "hbm_peak.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("read_tb_per_s:"):
            try:
                return float(line.split(":", 1)[1])
            except ValueError:
                return None
    return None


B200_CONTEXT_US = {"mtp": 1240.0, "dcp8": 826.0}  # the pages' numbers (other hardware)

WORKLOADS = {
    "mtp": 3,       # 16 x 100k, q5, h96, fp8  (default)
    "standard": 2,  # 32 x 4096, q1, h128, bf16
    "tiny": 1,      # 2 x {1024, 1536}, q1, h16, bf16
    "dcp8": 4,      # one shard of 128 x 100k over 8 shards, q5, h96, fp8
    "mtp-fp4": 6,   # the mtp shape over an FP4 pool
    "standard-fp4": 7,  # the standard shape over an FP4 pool
    "mtp-mxfp8": 8,  # the mtp shape over an MXFP8 pool
    "mtp-q1": 9,    # the mtp shape at q_len 1 (one query row per head): HBM bound
}


KERNEL_SOURCES = ("mla_kernels.hip", "tile_asm.inc", "kernels.h", "plan_layout.h", "mla_api.cpp")


def source_code_hash(texts) -> str:
    """sha256 of source texts with their comments and blank lines left out."""
    import hashlib
    import re
    h = hashlib.sha256()
    for text in texts:
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(l.rstrip() for l in text.splitlines() if l.strip()).encode())
        h.update(b"\0")
    return h.hexdigest()


def kernel_source_hash() -> str:
    """sha256 of the decode kernel's code, to tell stale counter summaries:
    the kernel, its generated statements, its headers and the planner that
    cuts its work, without comments, so that rewording a comment does not
    orphan a summary taken on the same code."""
    texts = []
    for fn in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "mla_latent_kv_absorbed_amd", "csrc", fn)) as f:
            texts.append(f.read())
    return source_code_hash(texts)


def committed_traffic(workload: str):
    """HBM bytes per decode-kernel launch from the committed counter summary.

    profiles/decode_kernel_<workload>_traffic.txt holds FETCH_SIZE and
    WRITE_SIZE per dispatch from two rocprofv3 --pmc runs of this script,
    scaled by what the same counters read for a plain copy of known size.
    Returns None when the summary is missing or was taken on other kernel
    sources.
    """
    path = os.path.join(ROOT, "profiles", f"decode_kernel_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_counts(x):
    """FLOPs and bytes the method needs, independent of the implementation.

    FLOPs: 2 x (576 + 512) per (query row, visible token); visible tokens of
    draft row i are the positions p <= L - q + i held by this shard.
    Bytes: every stored token's latent row (+ its fp32 scale for FP8) read
    once, the queries read once, O and LSE written once.
    """
    from workload import kv_bytes_per_token
    W, r, q, H = x.dcp_size, x.dcp_rank, x.q_len, x.num_heads
    vis = 0
    for L in x.seq_lens:
        for i in range(q):
            last = int(L) - q + i
            if last >= r:
                vis += (last - r) // W + 1
    flops = 2.0 * (576 + 512) * H * vis
    kv_bytes = float(x.local_lens.sum()) * kv_bytes_per_token(x.kv_dtype)
    rows = x.batch * q * H
    other = rows * (576 * 2) + rows * (512 * 4 + 4) + float(x.local_lens.sum()) * 4
    return flops, kv_bytes, kv_bytes + other


def prepare_bytes(x) -> float:
    """Algorithmic HBM bytes of one mla_prepare call: w_kc read once, the
    queries read and written once, the new rows and their positions' cos /
    sin read once, and the pool rows (and FP8 scales) written once (FP4: 336
    bytes a row, MXFP8: 608)."""
    T, H = x["T"], x["H"]
    row = {"bf16": 576 * 2, "fp8": 576 + 4, "fp4": 336, "mxfp8": 608}[x["kv_dtype"]]
    return float(H * 512 * 128 * 2 + T * H * 128 * 2 + 2 * T * H * 64 * 2 + T * H * 512 * 2
                 + T * 576 * 2 + T * 64 * 4 + T * row + T * 8)


def run_prepare(args, dev):
    """mla_prepare (Q absorption, RoPE, KV append) on the prepare workloads.

    Per workload: mean event-timed us per call (both kernels), algorithmic
    HBM bytes / time against 8 TB/s, and the CPU oracle on the same inputs.
    """
    import torch
    import mla_latent_kv_absorbed_amd as mla
    from oracle import mla_prepare_ref
    from workload import PREPARE_CONFIGS, prepare_inputs
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    rows = []
    stream = torch.cuda.current_stream(dev)
    for key in PREPARE_CONFIGS:
        x = prepare_inputs(key, device=dev)
        qa = torch.empty((x["T"], x["H"], 512), dtype=torch.bfloat16, device=dev)
        qr = torch.empty((x["T"], x["H"], 64), dtype=torch.bfloat16, device=dev)

        def step():
            mla.prepare(x["q_nope"], x["q_rope_in"], x["w_kc_t"], x["c_kv_new"], x["k_rope_new"],
                        x["positions"], x["cos_sin"], x["slots"], x["kv_pool"], x["kv_scale"],
                        q_nope_absorbed=qa, q_rope_out=qr, stream=stream)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        queue_ahead(step, args.steps, args.warmup)
        for a, b in ev:
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        us = float(np.mean([a.elapsed_time(b) for a, b in ev]) * 1e3)
        nbytes = prepare_bytes(x)
        # The oracle on the same inputs (host copies), timed once.
        bits = {k: x[k].cpu().view(torch.int16).numpy().view(np.uint16)
                for k in ("q_nope", "q_rope_in", "w_kc_t", "c_kv_new", "k_rope_new")}
        pool = x["kv_pool"].cpu()
        pool = pool.view(torch.int16).numpy().view(np.uint16) if x["kv_dtype"] == "bf16" \
            else pool.numpy()
        sc = None if x["kv_scale"] is None else x["kv_scale"].cpu().numpy()
        t0 = time.perf_counter()
        mla_prepare_ref(bits["q_nope"], bits["q_rope_in"], bits["w_kc_t"], bits["c_kv_new"],
                        bits["k_rope_new"], x["cos_sin"].cpu().numpy(),
                        x["positions"].cpu().numpy(), x["slots"].cpu().numpy(), pool, sc,
                        x["kv_dtype"])
        cpu_us = (time.perf_counter() - t0) * 1e6
        rows.append({"workload": x["name"], "tokens": x["T"], "heads": x["H"],
                     "kv": x["kv_dtype"], "us_per_call": round(us, 2),
                     "roofline": {"bound": "hbm", "achieved": round(nbytes / (us * 1e-6) / 1e9, 1),
                                  "peak": HBM_PEAK_TBPS * 1e3, "unit": "GB/s",
                                  "frac": round(nbytes / (us * 1e-6) / 1e12 / HBM_PEAK_TBPS, 4),
                                  "algorithmic_bytes": nbytes},
                     "cpu_baseline": {"value": round(cpu_us, 1), "unit": "us/call",
                                      "cores": int(cores), "kind": "oracle",
                                      "sample": "one call on the same inputs (float64 absorption, "
                                                "float32 RoPE and quantisation in numpy)"}})
        log(f"  prepare {x['name']}: {us:.2f} us")
        del x
        torch.cuda.empty_cache()
    print(json.dumps({"prepare": rows, "steps": args.steps, "warmup": args.warmup,
                      "context_b200": "mla_prepare: 0.44 ms per step in total over the 24 MLA "
                                      "layers (about 18 us per layer) for 640 rows (DP16-vs-DP2 "
                                      "page, section MLA)"}), flush=True)


def cpu_baseline(x, max_requests: int, budget_s: float):
    """Time the float64 oracle on a bounded sample of requests, scale to the layer.

    The pool, its scales and the table are copied to host memory once,
    untimed; each sampled request is then one oracle call on the whole pool
    and its own table row, so the timed region holds the oracle's page-table
    gather, its exact dequantization, the score matmul, the softmax and the
    value sum.
    """
    import torch
    from oracle import mla_decode_ref
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    nb = x.numpy_bits()
    done, t_total = 0, 0.0
    for b in range(min(max_requests, x.batch)):
        t0 = time.perf_counter()
        mla_decode_ref(nb["q_nope"][b:b + 1], nb["q_rope"][b:b + 1], nb["pool"], nb["kv_scale"],
                       nb["req_to_token"][b:b + 1], nb["seq_lens"][b:b + 1], x.q_len,
                       x.softmax_scale, x.kv_dtype, x.dcp_size, x.dcp_rank)
        t_total += time.perf_counter() - t0
        done += 1
        log(f"  oracle request {b}: {t_total:.1f}s so far")
        if t_total > budget_s:
            break
    per_layer_us = t_total / done * x.batch * 1e6
    return {"value": per_layer_us, "unit": "us/layer", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} of {x.batch} requests of the same workload (float64 numpy "
                      f"oracle on the host copy of the whole pool: table gather + exact "
                      f"dequant + matmul + softmax + value sum, all timed), scaled by "
                      f"{x.batch}/{done}"}


_SPIN_CYCLES_PER_MS = None


def queue_ahead(run_step, steps: int, warmup: int):
    """Run the warmup steps; if the host enqueues a step more slowly than the
    GPU runs it, hold the stream so that the timed steps queue up first.

    The warmup gives h, the host time to enqueue one step (the binding
    checks its tensors and marshals the call in Python), and g, the GPU
    time of one step.  When h > g / 2, events around the timed steps would
    also count the GPU idling between launches.  A spin kernel of about
    steps * h * 1.5 ms then goes first on the stream, so that every timed
    step is queued before the GPU reaches it and the steps run back to
    back.  GPU-bound workloads get no spin kernel and so no idle gap.
    """
    global _SPIN_CYCLES_PER_MS
    import torch
    stream = torch.cuda.current_stream()
    run_step()  # first launches load code objects: not part of h
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(max(warmup, 1)):
        run_step()
    b.record(stream)
    host_ms = (time.perf_counter() - t0) * 1e3 / max(warmup, 1)
    torch.cuda.synchronize()
    gpu_ms = a.elapsed_time(b) / max(warmup, 1)
    if host_ms <= 0.5 * gpu_ms:
        return
    if _SPIN_CYCLES_PER_MS is None:
        # torch's spin kernel counts the GPU's own clock; calibrate it once.
        torch.cuda._sleep(1000)
        torch.cuda.synchronize()
        a.record(stream)
        torch.cuda._sleep(1_000_000)
        b.record(stream)
        torch.cuda.synchronize()
        _SPIN_CYCLES_PER_MS = 1e6 / max(a.elapsed_time(b), 1e-3)
    hold_ms = steps * host_ms * 1.5 + 1.0
    log(f"  host {host_ms:.3f} ms/step > GPU {gpu_ms:.3f} ms/step / 2: "
        f"queueing the timed steps behind a {hold_ms:.1f} ms spin")
    torch.cuda._sleep(int(hold_ms * _SPIN_CYCLES_PER_MS))


def time_decode(x, dev, steps: int, warmup: int) -> float:
    """Mean us of mla_decode (attend + merge) on resident inputs, HIP events on the stream."""
    import torch
    import mla_latent_kv_absorbed_amd as mla
    seq_dev = torch.from_numpy(np.asarray(x.seq_lens, np.int32)).to(dev)
    desc = mla.make_desc(x.batch, x.q_len, x.num_heads, x.kv_dtype, page_size=x.page_size,
                         dcp_size=x.dcp_size, dcp_rank=x.dcp_rank)
    plan = mla.make_plan(desc, x.seq_lens, device=dev)
    ws = torch.zeros(max(plan.header["workspace_bytes"], 256), dtype=torch.uint8, device=dev)
    out = torch.empty((x.batch, x.q_len, x.num_heads, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((x.batch, x.q_len, x.num_heads), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        mla.decode(plan, x.q_nope, x.q_rope, x.pool, x.kv_scale, x.req_to_token, seq_dev,
                   x.softmax_scale, workspace=ws, out=out, lse=lse, stream=stream)

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    queue_ahead(step, steps, warmup)
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]) * 1e3)


def run_sweep(args, dev):
    """Batch sweep at 200k tokens, q_len 5, 96 heads, FP8: e(B) = t_floor(B) / t(B).

    t_floor is the MFMA time of the algorithmic FLOPs at the vendor peaks;
    no cliff means e(B) varies little over B = 1..24 and t(B) never drops as
    B grows.
    """
    import torch
    from workload import SWEEP_BATCHES, config_inputs
    rows = []
    for B in list(SWEEP_BATCHES) + ["ragged64"]:
        x = (config_inputs(5, device=dev, ragged=True) if B == "ragged64"
             else config_inputs(5, device=dev, batch=B))
        torch.cuda.synchronize()
        t_us = time_decode(x, dev, args.steps, args.warmup)
        flops, kv_bytes, _ = algorithmic_counts(x)
        t_floor = flops / (mfma_peak_tflops(x.kv_dtype) * 1e12) * 1e6
        rows.append({"batch": B, "tokens": int(np.sum(x.seq_lens)), "us_per_layer": round(t_us, 1),
                     "kv_tb_per_s": round(kv_bytes / (t_us * 1e-6) / 1e12, 3),
                     "e": round(t_floor / t_us, 4)})
        log(f"  sweep {B}: {t_us:.1f} us  e={t_floor / t_us:.3f}")
        del x
        torch.cuda.empty_cache()
    fixed = [r for r in rows if r["batch"] != "ragged64"]
    es = [r["e"] for r in fixed]
    ts = [r["us_per_layer"] for r in fixed]
    print(json.dumps({"sweep": "200k-q5-h96-fp8", "rows": rows,
                      "e_spread": round(max(es) - min(es), 4),
                      "t_non_decreasing": all(b >= a for a, b in zip(ts, ts[1:])),
                      "steps": args.steps, "warmup": args.warmup}), flush=True)


def run_dcp_full(args, dev):
    """All 8 DCP shards of 128 x 100k (q_len 5, 96 heads, FP8) on this GPU, then
    mla_lse_combine of their (O, LSE) into the full-context result.

    Each shard call writes its (O, LSE) into slot r of a stacked [8, rows, 512]
    buffer, which is exactly the combine's input layout.
    """
    import torch
    import mla_latent_kv_absorbed_amd as mla
    from workload import config_inputs
    W = 8
    shards, plans = [], []
    for r in range(W):
        x = config_inputs(4, device=dev, dcp_rank=r)
        desc = mla.make_desc(x.batch, x.q_len, x.num_heads, x.kv_dtype, page_size=x.page_size,
                             dcp_size=x.dcp_size, dcp_rank=x.dcp_rank)
        plans.append(mla.make_plan(desc, x.seq_lens, device=dev))
        shards.append(x)
        log(f"  shard {r} ready")
    x0 = shards[0]
    rows = x0.batch * x0.q_len * x0.num_heads
    part_o = torch.empty((W, rows, 512), dtype=torch.float32, device=dev)
    part_lse = torch.empty((W, rows), dtype=torch.float32, device=dev)
    out = torch.empty((rows, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((rows,), dtype=torch.float32, device=dev)
    seq_dev = torch.from_numpy(np.asarray(x0.seq_lens, np.int32)).to(dev)
    wss = [torch.zeros(max(p.header["workspace_bytes"], 256), dtype=torch.uint8, device=dev)
           for p in plans]
    stream = torch.cuda.current_stream(dev)

    def shard(r):
        x = shards[r]
        mla.decode(plans[r], x.q_nope, x.q_rope, x.pool, x.kv_scale, x.req_to_token, seq_dev,
                   x.softmax_scale, workspace=wss[r], out=part_o[r].view(x.batch, x.q_len,
                                                                         x.num_heads, 512),
                   lse=part_lse[r].view(x.batch, x.q_len, x.num_heads), stream=stream)

    def combine():
        mla.lse_combine(part_o, part_lse, out=out, lse=lse, stream=stream)

    # The same merge fused with the w_vc up-projection (512 -> 128 per head,
    # random bf16 weights of that shape): the merged latent O is not stored.
    T_tok, H = x0.batch * x0.q_len, x0.num_heads
    gen = torch.Generator(device=dev).manual_seed(4)
    w_vc_t = (torch.randn((H, 128, 512), generator=gen, device=dev) * 0.05).to(torch.bfloat16)
    out_v = torch.empty((T_tok, H, 128), dtype=torch.bfloat16, device=dev)
    po4 = part_o.view(W, T_tok, H, 512)
    pl3 = part_lse.view(W, T_tok, H)

    def combine_project():
        mla.lse_combine_project(po4, pl3, w_vc_t, out_v=out_v, lse=lse, stream=stream)

    # Unfused, for comparison: the projection of the combine's stored O (the
    # same kernel with one part of LSE 0).
    o1 = out.view(1, T_tok, H, 512)
    l1 = torch.zeros((1, T_tok, H), dtype=torch.float32, device=dev)
    lse_1 = torch.empty((T_tok, H), dtype=torch.float32, device=dev)

    def project_only():
        mla.lse_combine_project(o1, l1, w_vc_t, out_v=out_v, lse=lse_1, stream=stream)

    def full():
        for r in range(W):
            shard(r)
        combine()
        combine_project()
        project_only()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(W + 4)] for _ in range(args.steps)]
    queue_ahead(full, args.steps, args.warmup)
    for k in range(args.steps):
        ev[k][0].record(stream)
        for r in range(W):
            shard(r)
            ev[k][r + 1].record(stream)
        combine()
        ev[k][W + 1].record(stream)
        combine_project()
        ev[k][W + 2].record(stream)
        project_only()
        ev[k][W + 3].record(stream)
    torch.cuda.synchronize()
    per_shard = np.array([[ev[k][r].elapsed_time(ev[k][r + 1]) for r in range(W)]
                          for k in range(args.steps)]) * 1e3
    comb = np.array([ev[k][W].elapsed_time(ev[k][W + 1]) for k in range(args.steps)]) * 1e3
    total = np.array([ev[k][0].elapsed_time(ev[k][W + 1]) for k in range(args.steps)]) * 1e3
    comb_bytes = (W + 1) * rows * (512 * 4 + 4)
    cp = np.array([ev[k][W + 1].elapsed_time(ev[k][W + 2]) for k in range(args.steps)]) * 1e3
    cp_bytes = W * rows * (512 * 4 + 4) + rows * (128 * 2 + 4) + H * 128 * 512 * 2
    po_us = np.array([ev[k][W + 2].elapsed_time(ev[k][W + 3]) for k in range(args.steps)]) * 1e3
    print(json.dumps({
        "dcp": "128x100k-q5-h96-fp8 over 8 shards (p % 8 == r), all on one GPU",
        "per_shard_us_median": round(float(np.median(per_shard)), 1),
        "per_shard_us_by_rank": [round(float(v), 1) for v in np.median(per_shard, axis=0)],
        "sum_8_shards_plus_combine_us": round(float(np.median(total)), 1),
        "combine_us": round(float(np.median(comb)), 1),
        "combine_hbm_tb_per_s": round(comb_bytes / (float(np.median(comb)) * 1e-6) / 1e12, 3),
        "combine_project_us": round(float(np.median(cp)), 1),
        "combine_project_hbm_tb_per_s": round(cp_bytes / (float(np.median(cp)) * 1e-6) / 1e12, 3),
        "combine_project_note": "the same 8-part merge fused with the w_vc up-projection "
                                "(512 -> 128 per head, bf16 out); the merged fp32 O is not stored",
        "unfused_combine_then_project_us": round(float(np.median(comb)) + float(np.median(po_us)), 1),
        "project_only_us": round(float(np.median(po_us)), 1),
        "context_b200_us": {"per_shard_attn_mqa": 826.0, "dcp_pack_plus_lse_combine": 30.0},
        "steps": args.steps, "warmup": args.warmup}), flush=True)


def run_hbm_peak(args, dev):
    """HBM ceiling measured on this GPU with plain streaming kernels.

    Buffers of 4 GiB (16x the 256 MB MALL, so no cache holds them).  read:
    libmla_probe's streaming read (each lane keeps eight 16-byte loads in
    flight; 4 GiB read).  copy: its streaming copy (4 GiB read + 4 GiB
    written).  write: torch's fill (4 GiB written).  Each is timed with HIP
    events on the launch stream, median of `steps` runs after `warmup`.  The
    read rate is the ceiling of the decode kernel, whose HBM traffic is
    almost all reads.
    """
    import ctypes
    import torch
    probe = ctypes.CDLL(os.path.join(ROOT, "mla_latent_kv_absorbed_amd", "libmla_probe.so"))
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    probe.mla_probe_read.argtypes = [vp, i64, vp, i32, vp]
    probe.mla_probe_copy.argtypes = [vp, vp, i64, i32, vp]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    nbytes = 4 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    sink = torch.zeros(2048 * cus, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = int(stream.cuda_stream)

    def read():
        if probe.mla_probe_read(src.data_ptr(), nbytes, sink.data_ptr(), cus, sp) != 0:
            raise RuntimeError("mla_probe_read failed")

    def copy():
        if probe.mla_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, cus, sp) != 0:
            raise RuntimeError("mla_probe_copy failed")

    kinds = {"read": (read, nbytes), "write": (lambda: dst.fill_(2.0), nbytes),
             "copy": (copy, 2 * nbytes)}
    rows = {}
    for name, (fn, moved) in kinds.items():
        for _ in range(max(args.warmup, 1)):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) for a, b in ev]) * 1e3
        med = float(np.median(us))
        rows[name] = {"bytes": moved, "us_median": round(med, 1),
                      "tb_per_s": round(moved / (med * 1e-6) / 1e12, 3),
                      "tb_per_s_best": round(moved / (float(us.min()) * 1e-6) / 1e12, 3)}
        log(f"  {name}: {rows[name]['tb_per_s']} TB/s")
    if not torch.equal(dst, src):
        raise RuntimeError("probe copy mismatch")
    print(json.dumps({"hbm_peak": rows, "vendor_tb_per_s": HBM_PEAK_TBPS,
                      "read_frac_of_vendor": round(rows["read"]["tb_per_s"] / HBM_PEAK_TBPS, 4),
                      "buffers_gib": 4, "compute_units": cus, "steps": args.steps,
                      "warmup": args.warmup}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first: the first few dozen launches run slower while "
                         "the GPU clocks settle")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="mtp")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-requests", type=int, default=4)
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--flush-mb", type=int, default=0,
                    help="read this many MB between steps (outside the events) to evict L2/MALL; "
                         "a read leaves the caches holding clean lines, so the timed kernel pays "
                         "no write-back for the eviction")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the one-line step benchmark: time the batch sweep at "
                         "200k tokens (B in 1..24, and the ragged 64-request batch) and "
                         "print its efficiency spread as one JSON object")
    ap.add_argument("--dcp-full", action="store_true",
                    help="instead of the one-line step benchmark: run all 8 shards of the DCP "
                         "workload plus mla_lse_combine, and print per-shard, sum and "
                         "combine times as one JSON object")
    ap.add_argument("--prepare", action="store_true",
                    help="instead of the one-line step benchmark: time mla_prepare (Q "
                         "absorption, RoPE, KV append) on the prepare workloads and print one "
                         "JSON object")
    ap.add_argument("--hbm-peak", action="store_true",
                    help="instead of the one-line step benchmark: measure this GPU's HBM read, "
                         "write and copy rates with plain streaming kernels over 4 GiB buffers")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="before the warmup, run one plain device copy of this many MB (for "
                         "scaling HBM counters); not timed")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode path has no multi-GPU part "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import mla_latent_kv_absorbed_amd as mla
    from workload import CONFIGS, config_inputs

    dev = torch.device("cuda:0")
    if args.sweep:
        run_sweep(args, dev)
        return
    if args.dcp_full:
        run_dcp_full(args, dev)
        return
    if args.prepare:
        run_prepare(args, dev)
        return
    if args.hbm_peak:
        run_hbm_peak(args, dev)
        return
    cfg = WORKLOADS[args.workload]
    log(f"generating inputs for {CONFIGS[cfg]['name']} on {dev}")
    x = config_inputs(cfg, device=dev, dcp_rank=3 if cfg == 4 else 0)
    torch.cuda.synchronize()
    seq_dev = torch.from_numpy(np.asarray(x.seq_lens, np.int32)).to(dev)
    desc = mla.make_desc(x.batch, x.q_len, x.num_heads, x.kv_dtype, page_size=x.page_size,
                         dcp_size=x.dcp_size, dcp_rank=x.dcp_rank)
    plan = mla.make_plan(desc, x.seq_lens, device=dev)
    h = plan.header
    out = torch.empty((x.batch, x.q_len, x.num_heads, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((x.batch, x.q_len, x.num_heads), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(h["workspace_bytes"], 256), dtype=torch.uint8, device=dev)
    flush = (torch.ones(args.flush_mb << 18, dtype=torch.int32, device=dev)
             if args.flush_mb else None)
    stream = torch.cuda.current_stream(dev)

    def step(mid=None):
        mla.decode(plan, x.q_nope, x.q_rope, x.pool, x.kv_scale, x.req_to_token, seq_dev,
                   x.softmax_scale, workspace=ws, out=out, lse=lse, stream=stream,
                   phase="attend")
        if mid is not None:
            mid.record(stream)
        mla.decode(plan, x.q_nope, x.q_rope, x.pool, x.kv_scale, x.req_to_token, seq_dev,
                   x.softmax_scale, workspace=ws, out=out, lse=lse, stream=stream,
                   phase="merge")

    if args.copy_calibration_mb:
        # Plain kernels of known size for scaling HBM counters: a fill that
        # writes n bytes, then a uint8 -> int16 copy that reads n and writes
        # 2n (a 256 MB fill between them evicts the source from L2).
        n = args.copy_calibration_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        evict = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty(n, dtype=torch.int16, device=dev)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: fill of {n} bytes; copy reading {n} and writing {2 * n} bytes")
        del src, dst, evict

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    mids = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]

    def flushed_step():
        if flush is not None:
            flush.sum()
        step()

    queue_ahead(flushed_step, args.steps, args.warmup)
    t0 = time.perf_counter()
    for k in range(args.steps):
        if flush is not None:
            flush.sum()
        starts[k].record(stream)
        step(mids[k])
        ends[k].record(stream)
    host_enqueue = time.perf_counter() - t0
    torch.cuda.synchronize()
    times_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    kern_ms = np.array([s.elapsed_time(m) for s, m in zip(starts, mids)])
    t_us = float(np.mean(times_ms) * 1e3)
    k_us = float(np.mean(kern_ms) * 1e3)

    flops, kv_bytes, all_bytes = algorithmic_counts(x)
    tflops = flops / (t_us * 1e-6) / 1e12
    kv_tbps = kv_bytes / (t_us * 1e-6) / 1e12
    # Roofline of the dominant kernel (mla::decode_kernel), priced by its own
    # average duration; the merge of split requests is not in it.
    k_tflops = flops / (k_us * 1e-6) / 1e12
    traffic = committed_traffic(args.workload)
    peak = mfma_peak_tflops(x.kv_dtype)
    roofline = {
        "bound": "mfma", "achieved": round(k_tflops, 2), "peak": round(peak, 1),
        "unit": "TFLOP/s", "frac": round(k_tflops / peak, 4),
        "traffic": traffic, "kernel": "mla::decode_kernel", "kernel_us": round(k_us, 2),
        "flops_per_launch": flops, "algorithmic_bytes_per_launch": all_bytes,
    }
    # The bound is whichever floor is longer at the vendor peaks: MFMA time
    # of the algorithmic FLOPs, or HBM time of the algorithmic bytes.
    t_mfma_floor = flops / (peak * 1e12)
    t_hbm_floor = all_bytes / (HBM_PEAK_TBPS * 1e12)
    if t_hbm_floor > t_mfma_floor:
        bw = all_bytes / (k_us * 1e-6) / 1e12
        roofline.update({"bound": "hbm", "achieved": round(bw * 1e3, 1),
                         "peak": HBM_PEAK_TBPS * 1e3, "unit": "GB/s",
                         "frac": round(bw / HBM_PEAK_TBPS, 4)})
    hbm_meas = measured_hbm_peak()

    result = {
        "metric": METRIC,
        "value": round(t_us, 2),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_us / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8_e4m3+bf16", "fp4": "fp4_e2m1+bf16",
                  "mxfp8": "mxfp8_e4m3+bf16"}[x.kv_dtype],
        "data": "synthetic",
        "config": {"workload": CONFIGS[cfg]["name"], "requests": x.batch,
                   "context": int(max(x.seq_lens)), "q_len": x.q_len, "heads": x.num_heads,
                   "kv": x.kv_dtype, "page_size": x.page_size, "dcp": [x.dcp_size, x.dcp_rank]},
        "kv_tb_per_s": round(kv_tbps, 3),
        "kv_hbm_peak_frac": round(kv_tbps / HBM_PEAK_TBPS, 4),
        "kv_hbm_measured_peak_frac": (round(kv_tbps / hbm_meas, 4) if hbm_meas else None),
        "hbm_measured_read_peak_tb_per_s": hbm_meas,
        "floors_us": {"mfma": round(t_mfma_floor * 1e6, 1), "hbm": round(t_hbm_floor * 1e6, 1)},
        "mfma_frac": round(tflops / peak, 4),
        "step_us_p10_p50_p90": [round(float(np.percentile(times_ms, p)) * 1e3, 2)
                                for p in (10, 50, 90)],
        "merge_us": round(t_us - k_us, 2),
        "host_enqueue_ms_per_step": round(host_enqueue / args.steps * 1e3, 4),
        "plan": {k: h[k] for k in ("num_wgs", "num_units", "num_parts", "num_split_reqs")},
        "context_b200_us_per_layer": B200_CONTEXT_US.get(args.workload),
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(x, args.cpu_requests, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
