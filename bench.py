#!/usr/bin/env python3
"""Benchmark of the MSA training hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
proxy block scores -> block selection (+ inverted index) -> sparse GQA
forward (+ proxy LSE) -> fused main + proxy backward, all through the C ABI.
Inputs are drawn on the device before timing (resident in HBM).

Default workload: ``varlen-1m-packed`` (1,048,576 tokens packed from seeded
log-uniform document lengths, 32 query / 8 KV heads, d 128, dp 64, query
block 128, top-k 64), bf16 inputs with fp32 accumulation.

Prints one JSON line.  ``value`` is the attention rate over the selected
(query, key) pairs: the counted forward and backward FLOPs (FlashAttention
convention: 4 d per pair and head forward, 10 d backward; proxy 2 dp forward,
6 dp backward, per pair and proxy head) divided by the forward and backward
kernel time (``attn_fwd_bwd_ms``).  ``ms_per_step`` is the whole step
(scoring, selection, forward, backward) between two events, and
``step_tflops`` adds the quadratic scoring FLOPs over that whole step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X published dense bf16/fp16
HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E
METRIC = "MSA fwd+bwd ms/step and TFLOP/s (selected FLOPs) at 128k–1M tok; % MFMA peak"
PREFILL_METRIC = "MSA forward-only (prefill) ms and TFLOP/s (scoring + selected forward FLOPs)"
ROOFLINE_KERNELS = ("proxy_scores", "fwd", "bwd_dq", "bwd_dkdv")


def selected_pairs(seqlens, q_block, topk, window, dilation=1):
    """Exactly-valid (query, key) pairs attended per KV group (every group has
    the same count: the number of selected blocks depends only on the
    diagonal).  Non-diagonal selected blocks lie wholly before the query
    block; the diagonal block contributes the causal triangle.  Selected
    blocks: min(k - 1, blocks below the window's span) + the forced ones."""
    total = 0
    for L in seqlens:
        nq = -(-L // q_block)
        for I in range(nq):
            lo = I * q_block
            rows = min(q_block, L - lo)
            diag = lo // 128
            cnt = min(topk - 1, max(0, diag - window * dilation)) + min(window, diag // dilation) + 1
            first = lo - diag * 128 + 1           # keys of the diagonal block for query lo
            total += rows * 128 * (cnt - 1) + rows * first + rows * (rows - 1) // 2
    return total


def flop_model(w, seqlens, scored_pairs):
    """Counted FLOPs use the proxy-head count Hp (Hkv, or 1 for the shared
    head); the per-kernel figures use what the kernels run (the attention
    kernels work per KV group either way; scoring runs once per proxy head)."""
    d, dp, Hq, Hkv = w.head_dim, w.proxy_dim, w.heads_q, w.heads_kv
    Hp = 1 if getattr(w, "proxy_heads", 0) == 1 else Hkv
    n = selected_pairs(seqlens, w.q_block, w.topk, w.local_window, w.dilation)
    f = {
        "pairs_per_group": n,
        "scoring": 2 * dp * Hp * scored_pairs,
        "fwd_counted": 4 * d * Hq * n + 2 * dp * Hp * n,
        "bwd_counted": 10 * d * Hq * n + 6 * dp * Hp * n,
        # what the split backward executes: S and dP are recomputed in both
        # passes (14 d per head), the query-major pass also forms P kp per
        # head for the group-mean term, and each pass recomputes Y and applies
        # one proxy product per group
        "bwd_executed": 14 * d * Hq * n + 2 * dp * Hq * n + 8 * dp * Hkv * n,
        # per-kernel algorithmic work
        "k:proxy_scores": 2 * dp * Hp * scored_pairs,
        "k:fwd": 4 * d * Hq * n,
        "k:proxy_lse": 2 * dp * Hkv * n,
        "k:bwd_dq": 6 * d * Hq * n + 4 * dp * Hkv * n,
        "k:bwd_dkdv": 8 * d * Hq * n + 4 * dp * Hkv * n,
    }
    return f


def _code_only(text):
    """The source without // and /* */ comments and without blank or
    indentation-only differences (no string literal here holds either)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).strip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def source_hash(files):
    """Hash of the code of a kernel's sources: edits to comments keep it."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


_HDR = ["block_sparse_attention_proxy_amd/csrc/msa_device.h", "block_sparse_attention_proxy_amd/csrc/msa_internal.h"]
KERNEL_SOURCES = {
    "proxy_scores": ["block_sparse_attention_proxy_amd/csrc/select.hip"] + _HDR,
    "select": ["block_sparse_attention_proxy_amd/csrc/select.hip"] + _HDR,
    "fwd": ["block_sparse_attention_proxy_amd/csrc/attn_fwd.hip"] + _HDR,
    "proxy_lse": ["block_sparse_attention_proxy_amd/csrc/attn_fwd.hip"] + _HDR,
    "bwd_dq": ["block_sparse_attention_proxy_amd/csrc/attn_bwd.hip",
               "block_sparse_attention_proxy_amd/csrc/attn_bwd_q.hip"] + _HDR,
    "bwd_dkdv": ["block_sparse_attention_proxy_amd/csrc/attn_bwd.hip",
                 "block_sparse_attention_proxy_amd/csrc/attn_bwd_kv.hip"] + _HDR,
}


def traffic_for(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tab = json.load(f)
    ent = tab.get(workload, {}).get(kernel)
    if not ent or ent.get("source_hash") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(w, seqlens, x, budget_s, seed):
    """The oracle, untuned, on a bounded sample of the same workload: scoring,
    selection, forward and backward of sampled query blocks of the longest
    document, in the oracle's fp64 numpy.  Returns TFLOP/s under the same
    FLOP convention."""
    import numpy as np
    import torch
    from oracle import msa_oracle as om
    # the host cores this process may run on; BLAS gets that many threads,
    # unless the environment caps the thread count lower
    affinity = len(os.sched_getaffinity(0))
    cap = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    want = min(affinity, cap) if cap > 0 else affinity
    vendor, threads, limiter = "unknown", want, None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=want, user_api="blas")
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if blas:
            vendor = ",".join(sorted({f"{p.get('internal_api')} {p.get('version')}" for p in blas}))
            threads = max(p.get("num_threads", want) for p in blas)
    except Exception:
        pass
    ocfg = om.Config(w.heads_q, w.heads_kv, w.head_dim, w.proxy_dim, w.q_block, w.topk, w.local_window)
    b = max(range(len(seqlens)), key=lambda i: seqlens[i])
    s0 = int(sum(seqlens[:b]))
    L = seqlens[b]
    doc = om.Doc(0, L, -(-L // w.q_block), -(-L // 128), 0, 0, 0)
    g = 0
    sl = slice(s0, s0 + L)

    def host(name, heads):
        return x[name][sl, heads].float().cpu().numpy().astype(np.float64)

    G = w.group
    arrs = dict(q=host("q", slice(g * G, (g + 1) * G)), k=host("k", slice(g, g + 1)),
                v=host("v", slice(g, g + 1)), qp=host("qp", slice(g, g + 1)),
                kp=host("kp", slice(g, g + 1)), dO=host("dO", slice(g * G, (g + 1) * G)))
    c1 = om.Config(G, 1, w.head_dim, w.proxy_dim, w.q_block, w.topk, w.local_window)
    rng = np.random.default_rng(seed)
    order = rng.permutation(doc.nq)
    flops, done, t0 = 0, 0, time.perf_counter()
    for I in order:
        I = int(I)
        S = om.proxy_row_scores(arrs["qp"], arrs["kp"], doc, 0, I, c1)
        sel = om.select_row(S, I, c1)
        fw = om.qblock_forward(arrs["q"], arrs["k"], arrs["v"], arrs["qp"], arrs["kp"], doc, 0, I, sel, c1)
        om.qblock_backward(fw, arrs["q"], arrs["k"], arrs["v"], arrs["qp"], arrs["kp"], arrs["dO"], 0, c1)
        rows = len(fw["rows"])
        n = int(fw["mask"].sum())
        flops += 2 * w.proxy_dim * rows * len(S) * 128
        flops += (4 + 10) * w.head_dim * G * n + (2 + 6) * w.proxy_dim * n
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.restore_original_limits()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "affinity_cores": affinity, "blas": vendor,
            "sample": f"{done} query blocks (group 0, all {G} heads) of the longest document "
                      f"({L} tokens): scoring, selection, forward and backward in fp64 numpy, "
                      f"{dt:.1f} s wall", "seconds": dt}


def dense_compare(a, w, seqlens, x, msa, torch):
    """The workload through the autograd API twice: with its top-k, and with
    every causal block selected (dense).  Each is run once untimed, then
    timed once: forward (scores, selection, forward) and backward separately.
    Memory: bytes allocated between the end of the forward and the start of
    the backward beyond the inputs (O, the LSEs, the block lists), and the
    peak over the step."""
    host = [int(c) for c in x["cu_seqlens"].cpu().tolist()]
    names = ("q", "k", "v", "qp", "kp")
    res = {}
    for label, dense in (("sparse", False), ("dense", True)):
        leaves = {n: x[n].detach().clone().requires_grad_(True) for n in names}

        def forward():
            return msa.msa_attention(*(leaves[n] for n in names), x["cu_seqlens"], topk=w.topk,
                                     q_block=w.q_block, local_window=w.local_window,
                                     proxy_loss_weight=w.proxy_loss_weight, cu_seqlens_host=host,
                                     dense=dense, dilation=w.dilation, proxy_heads=w.proxy_heads)

        for _ in range(max(a.warmup, 1)):
            o = forward()
            o.backward(x["dO"])
            del o
            for t in leaves.values():
                t.grad = None
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        o = forward()
        e[1].record()
        torch.cuda.synchronize()
        kept = torch.cuda.memory_allocated() - base
        o.backward(x["dO"])
        e[2].record()
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        fwd_ms, bwd_ms = e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2])
        topk = max(-(-L // 128) for L in seqlens) if dense else w.topk
        n = (selected_pairs(seqlens, w.q_block, topk, 0, 1) if dense
             else selected_pairs(seqlens, w.q_block, topk, w.local_window, w.dilation))
        d, dp, Hq, Hp = w.head_dim, w.proxy_dim, w.heads_q, w.heads_kv
        fwd_fl = 4 * d * Hq * n + 2 * dp * Hp * n
        bwd_fl = 10 * d * Hq * n + 6 * dp * Hp * n
        res[label] = {"topk": topk, "pairs_per_group": n, "fwd_ms": round(fwd_ms, 3), "bwd_ms": round(bwd_ms, 3),
                      "fwd_tflops": round(fwd_fl / (fwd_ms * 1e-3) / 1e12, 2),
                      "bwd_tflops": round(bwd_fl / (bwd_ms * 1e-3) / 1e12, 2),
                      "kept_bytes_fwd_to_bwd": int(kept), "peak_bytes_over_inputs": int(peak)}
        del o, leaves
        torch.cuda.synchronize()
    T, Hq, d = sum(seqlens), w.heads_q, w.head_dim
    esz = 2 if w.dtype == "bf16" else 4
    fused = T * Hq * d * esz + T * Hq * 4          # a fused dense kernel keeps O and LSE only
    sp, de = res["sparse"], res["dense"]
    out = {"mode": "dense-compare", "workload": w.name, "total_tokens": T, "docs": len(seqlens),
           "sparse": sp, "dense": de,
           "speedup": {"fwd": round(de["fwd_ms"] / sp["fwd_ms"], 3), "bwd": round(de["bwd_ms"] / sp["bwd_ms"], 3),
                       "step": round((de["fwd_ms"] + de["bwd_ms"]) / (sp["fwd_ms"] + sp["bwd_ms"]), 3)},
           "kept_ratio_dense_over_sparse": round(de["kept_bytes_fwd_to_bwd"] / sp["kept_bytes_fwd_to_bwd"], 3),
           "fused_dense_kept_bytes": fused,
           "note": "dense = the same kernels with every causal block selected; fused_dense_kept_bytes "
                   "is what a fused dense attention keeps (O and LSE)"}
    line = json.dumps(out)
    print(line, flush=True)
    if a.report:
        with open(a.report, "w") as fh:
            fh.write(line + "\n")
    return 0


def calibrate_copy(mib):
    """A plain copy kernel of known size: reads and writes mib MiB per launch."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": n, "copy_bytes_written_per_launch": n, "launches": 4}))
    return 0


# rocprofv3 kernel names (mangled or demangled) -> the library's kernel names
_TRACE_KERNELS = (("proxy_scores", "proxy_scores"), ("select_kernel", "select"),
                  ("proxy_lse", "proxy_lse"), ("fwd_kernel", "fwd"), ("dq_kernel", "bwd_dq"),
                  ("dq128_kernel", "bwd_dq"), ("dkdv", "bwd_dkdv"))


def _counter_per_dispatch(csv_dir, counter):
    """Mean value of one counter per dispatch of each library kernel (and of
    the plain copy) in a rocprofv3 counter-collection CSV directory."""
    import csv
    import glob
    sums = {}
    for path in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"]
                key = "copy" if "copyBuffer" in name else next(
                    (k for pat, k in _TRACE_KERNELS if pat in name), None)
                if key is None:
                    continue
                d = sums.setdefault(key, {})
                d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in sums.items()}


def write_traffic(workload, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_mib):
    """HBM bytes per launch of each kernel from two counter runs (FETCH_SIZE,
    WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads
    for a plain copy of copy_mib MiB; written to profiles/traffic.json with
    the hash of the kernel sources they were taken on."""
    fetch = _counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _counter_per_dispatch(write_dir, "WRITE_SIZE")
    cf = _counter_per_dispatch(copy_fetch_dir, "FETCH_SIZE")["copy"]
    cw = _counter_per_dispatch(copy_write_dir, "WRITE_SIZE")["copy"]
    fetch_factor = copy_mib * 1024.0 / cf
    write_factor = copy_mib * 1024.0 / cw
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    ent = {}
    print(f"copy: FETCH_SIZE {cf:.1f} KiB, WRITE_SIZE {cw:.1f} KiB per dispatch "
          f"-> factors {fetch_factor:.5f}, {write_factor:.5f}")
    print("| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per launch (scaled) |")
    print("|---|---:|---:|---:|")
    for k in KERNEL_SOURCES:
        if k not in fetch or k not in write:
            continue
        b = fetch[k] * 1024 * fetch_factor + write[k] * 1024 * write_factor
        ent[k] = {"bytes_per_launch": int(round(b)), "fetch_kib": round(fetch[k], 1),
                  "write_kib": round(write[k], 1), "fetch_factor": round(fetch_factor, 5),
                  "write_factor": round(write_factor, 5),
                  "source_hash": source_hash(KERNEL_SOURCES[k])}
        print(f"| {k} | {fetch[k]:.1f} | {write[k]:.1f} | {b:.4e} |")
    data[workload] = ent
    with open(path, "w") as fh:
        json.dump(data, fh, indent=1)
        fh.write("\n")
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="varlen-1m-packed")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work (0 = skip)")
    ap.add_argument("--report", default=None, help="also write the JSON (plus details) here")
    ap.add_argument("--mode", choices=("train", "prefill", "dense-compare"), default="train",
                    help="train: the training step (default); prefill: forward only (scores, "
                         "selection, forward); dense-compare: the same workload once sparse and once "
                         "with every causal block selected, through the autograd API, with the "
                         "memory kept between forward and backward")
    ap.add_argument("--proxy-heads", type=int, default=None, choices=(0, 1),
                    help="override the workload's proxy heads (0: one per KV group, 1: one shared head)")
    ap.add_argument("--dilation", type=int, default=None, help="override the window dilation")
    ap.add_argument("--local-window", type=int, default=None, help="override the local window")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of this many MiB, 4 times (the "
                         "known-size reference for scaling HBM byte counters), then exit")
    ap.add_argument("--write-traffic", nargs=4, default=None,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="no GPU work: turn four rocprofv3 counter runs (this workload's step with "
                         "FETCH_SIZE, then WRITE_SIZE; the copy with each) into profiles/traffic.json")
    ap.add_argument("--copy-mib", type=int, default=1024, help="size of the copy in --write-traffic")
    a = ap.parse_args(argv)
    if a.calibrate_copy:
        return calibrate_copy(a.calibrate_copy)
    if a.write_traffic:
        return write_traffic(a.workload, *a.write_traffic, a.copy_mib)
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {a.gpus} is not supported (this path has no "
              "multi-GPU mode: each GPU would run the same op on its own documents).", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        return 1
    import block_sparse_attention_proxy_amd as msa
    from msa_inputs import WORKLOADS, make_case_torch, seqlens_of

    w = WORKLOADS[a.workload]
    over = {k: v for k, v in (("proxy_heads", a.proxy_heads), ("dilation", a.dilation),
                              ("local_window", a.local_window)) if v is not None}
    if over:
        from dataclasses import replace
        w = replace(w, **over)
    seqlens = seqlens_of(w, a.seed)
    t_gen = time.perf_counter()
    x = make_case_torch(w, a.seed, device="cuda", seqlens=seqlens)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    cfg = msa.Config(w.heads_q, w.heads_kv, w.head_dim, w.proxy_dim, w.q_block, w.topk, w.local_window,
                     128, 0.0, 0.0, w.proxy_loss_weight, w.dtype, w.dilation, w.proxy_heads)
    vl = msa.Varlen(x["cu_seqlens"], x["cu_seqlens"].cpu().numpy())
    buf = msa.Buffers(cfg, vl, device="cuda", need_bwd=True)
    lay = buf.layout

    if a.mode == "dense-compare":
        return dense_compare(a, w, seqlens, x, msa, torch)

    def step():
        msa.run_forward(cfg, vl, x["q"], x["k"], x["v"], x["qp"], x["kp"], buf)
        if a.mode == "train":
            msa.run_backward(cfg, vl, x["q"], x["k"], x["v"], x["qp"], x["kp"], x["dO"], buf)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    msa.profile_enable(True)
    msa.profile_collect()                       # drop anything recorded before the timed region
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record()
    for _ in range(a.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = ev0.elapsed_time(ev1) / a.steps
    kern = msa.profile_collect()
    msa.profile_enable(False)

    f = flop_model(w, seqlens, lay["scored_pairs"])
    per_kernel = {k: {"avg_ms": ms / n, "launches_per_step": n / a.steps} for k, (ms, n) in kern.items()}
    stage_of = {"proxy_scores": "scores", "select": "select", "k2q_count": "select", "k2q_scan": "select",
                "k2q_emit": "select",
                "fwd": "fwd", "proxy_lse": "fwd", "bwd_dq": "bwd",
                "bwd_dqp_reduce": "bwd", "bwd_dkdv": "bwd", "meta": "meta"}
    stages = {}
    for k, (ms, n) in kern.items():
        stages[stage_of.get(k, k)] = stages.get(stage_of.get(k, k), 0.0) + ms / a.steps
    for k, v in per_kernel.items():
        if "k:" + k in f:
            v["tflops"] = f["k:" + k] / (v["avg_ms"] * 1e-3) / 1e12
    if a.mode == "prefill":
        total_flops = f["scoring"] + f["fwd_counted"]
    else:
        total_flops = f["scoring"] + f["fwd_counted"] + f["bwd_counted"]
    step_tflops = total_flops / (step_ms * 1e-3) / 1e12
    attn_ms = stages.get("fwd", 0.0) + stages.get("bwd", 0.0)
    attn_flops = f["fwd_counted"] + (f["bwd_counted"] if a.mode == "train" else 0)
    attn_tflops = attn_flops / (attn_ms * 1e-3) / 1e12 if attn_ms else None
    # the headline: counted (forward + backward) FLOPs over the selected pairs
    # per forward + backward time; prefill keeps its own metric (scoring and
    # forward over the forward pass)
    value = attn_tflops if a.mode == "train" else step_tflops
    bwd_ms = stages.get("bwd", 0.0)
    bwd_rates = None
    if bwd_ms:
        bwd_rates = {"counted_tflops": round(f["bwd_counted"] / (bwd_ms * 1e-3) / 1e12, 2),
                     "executed_tflops": round(f["bwd_executed"] / (bwd_ms * 1e-3) / 1e12, 2),
                     "executed_mfma_frac": round(f["bwd_executed"] / (bwd_ms * 1e-3) / 1e12
                                                / MFMA_BF16_PEAK_TFLOPS, 4)}

    dom = max([k for k in ROOFLINE_KERNELS if k in per_kernel], key=lambda k: per_kernel.get(k, {}).get("avg_ms", 0.0) *
              per_kernel.get(k, {}).get("launches_per_step", 0.0))
    achieved = per_kernel[dom]["tflops"]
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": traffic_for(dom, a.workload), "kernel": dom,
                "avg_launch_ms": round(per_kernel[dom]["avg_ms"], 4),
                "flops_per_launch": f["k:" + dom]}
    # selection kernel against HBM: candidate scores read + block lists written
    n_cand_entries = 0
    for L in seqlens:
        nq = -(-L // w.q_block)
        for I in range(nq):
            pool = I * w.q_block // 128 - w.local_window * w.dilation
            if pool > w.topk - 1:
                n_cand_entries += pool
    sel_bytes = lay["proxy_heads"] * (4 * n_cand_entries + 4 * lay["total_qblocks"] * (lay["sel_stride"] + 1))
    selection = None
    if "select" in per_kernel:
        gbps = sel_bytes / (per_kernel["select"]["avg_ms"] * 1e-3) / 1e9
        selection = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "bytes_per_launch": sel_bytes}

    cpu = None
    if a.cpu_budget > 0 and a.mode == "train":
        cpu = cpu_baseline(w, seqlens, x, a.cpu_budget, a.seed)

    out = {
        "metric": METRIC if a.mode == "train" else PREFILL_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(step_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "total_tokens": int(sum(seqlens)), "docs": len(seqlens),
                   "heads_q": w.heads_q, "heads_kv": w.heads_kv, "head_dim": w.head_dim,
                   "proxy_dim": w.proxy_dim, "kv_block": 128, "q_block": w.q_block, "topk": w.topk,
                   "local_window": w.local_window, "dilation": w.dilation,
                   "proxy_heads": lay["proxy_heads"], "seed": a.seed,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": None if cpu is None else {k: v for k, v in cpu.items() if k != "seconds"},
        "stages_ms": {k: round(v, 3) for k, v in sorted(stages.items())},
        "step_tflops": round(step_tflops, 2),
        "attn_fwd_bwd_ms": round(attn_ms, 3),
        "attn_fwd_bwd_tflops": None if attn_tflops is None else round(attn_tflops, 2),
        "attn_mfma_frac": None if attn_tflops is None else round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "selection_roofline": selection,
        "bwd_rates": bwd_rates,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in sorted(per_kernel.items())},
        "flops": {k: v for k, v in f.items() if not k.startswith("k:")},
        "tokens_per_s": round(sum(seqlens) / (step_ms * 1e-3), 1),
        "wall_s_timed": round(wall, 3),
        "input_gen_s": round(t_gen, 2),
    }
    line = json.dumps(out)
    print(line, flush=True)
    if a.report:
        with open(a.report, "w") as fh:
            fh.write(line + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
