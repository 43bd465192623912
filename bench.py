"""Benchmark of the RecSA hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
build the tree over the L cached tokens, decode a batch at length L (per
query head, then again with one selection per KV group), the backward of that
decode batch (selection fixed; a synthetic output gradient), append the
prefill chunk (growing the tree) and run the causal prefill of that chunk.
Each call is timed with HIP events on the stream it is launched on; times are
the median (with p10 and p90) over the timed steps.  The roofline line follows
the dominant forward call.

The headline workload is the 524K-token Qwen3-4B-shaped layer.  The other
workloads of the path (131K; 1M with block drift; 2M) are measured after it in
the same run, each with its own build, decode batches and (1M) append + prefill,
and reported under "configs".  Before any GPU work, the oracle is timed on the
host's cores (the CPU baseline).

Prints one JSON line: value = decode queries/s at 524K; prefill tokens/s,
tree-build bandwidth and the roofline fractions of every call ride along.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
CSRC = os.path.join(ROOT, "long_context_recsa_amd", "csrc")
COUNTERS = os.path.join(ROOT, "profiles", "hbm_counters_{workload}.md")


# Sources each library call's kernels are built from (with the shared headers and the
# host-side launch code); HBM counters taken with other versions of them do not apply.
OP_SOURCES = {
    "tree_build": ["tree_kernels.hip"],
    "append": ["tree_kernels.hip"],
    "decode": ["descend_impl.hpp", "descend_kernels.hip", "select_topk.hpp"],
    "decode_grouped": ["descend_impl.hpp", "descend_grouped_bf16.hip", "descend_grouped_f32.hip",
                       "select_topk.hpp"],
    "prefill": ["prefill_tiled.hip", "select_topk.hpp"],
    "backward": ["backward_kernels.hip", "prefill_tiled.hip", "select_topk.hpp"],
    "backward_bf16": ["backward_kernels.hip", "prefill_tiled.hip", "select_topk.hpp"],
}
COMMON_SOURCES = ["recsa_internal.hpp", "recsa_api.hip"]


def sources_digest(op):
    """sha256 over the kernel sources of one library call."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(OP_SOURCES[op] + COMMON_SOURCES):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` (read + write) from the committed counter summary
    for this workload: lines 'traffic <kernel> fetch_bytes=F write_bytes=W sources=<sha256>'
    (decode per batch as decode_B<batch>).  None when there is no summary or the kernels
    changed since it was taken."""
    path = COUNTERS.format(workload=workload)
    if not os.path.exists(path):
        return None
    op = "decode" if kernel.startswith("decode_B") else kernel
    digest = sources_digest(op) if op in OP_SOURCES else None
    with open(path) as fh:
        for line in fh:
            parts = line.strip().strip("`").split()
            if len(parts) == 5 and parts[0] == "traffic" and parts[1] == kernel:
                kv = dict(p.split("=", 1) for p in parts[2:])
                if kv.get("sources") != digest:
                    return None
                return {"fetch": int(kv["fetch_bytes"]), "write": int(kv["write_bytes"])}
    return None


def level_sizes(n, b):
    out = [n]
    while out[-1] // b >= 1:
        out.append(out[-1] // b)
    return out


def row_entries(n_ctx, b, k):
    """(keys scored, values read) of one row: candidate counts per level."""
    N = level_sizes(n_ctx, b)
    H = len(N) - 1
    keys = vals = 0
    c = N[H]
    for l in range(H, -1, -1):
        keys += c
        if l == 0:
            vals += c
            break
        m = min(k, c)
        vals += c - m
        c = b * m + (N[l - 1] - b * N[l])
    return keys, vals


def algorithmic(w, B):
    """Bytes (and FLOPs) each call must move, from the tree geometry."""
    esz = 2 if w.dtype == "bf16" else 4
    row_b = w.d * esz
    N = level_sizes(w.L, w.b)
    build_bytes = 2 * w.n_kv * w.L * row_b + 2 * w.n_kv * sum(N[1:]) * row_b
    kd, vd = row_entries(w.L, w.b, w.k)
    decode_bytes = B * w.n_q * (kd + vd) * row_b
    decode_flops = B * w.n_q * (kd + vd) * 2 * w.d
    # one selection per (query, KV group): each group row reads its keys and values once
    # for its G heads
    grouped_bytes = B * w.n_kv * (kd + vd) * row_b
    pk = pv = 0
    for j in range(w.prefill_n):
        a, c = row_entries(w.L + j + 1, w.b, w.k)
        pk += a
        pv += c
    prefill_bytes = w.n_q * (pk + pv) * row_b
    Lt_ = w.L + w.prefill_n
    # read-once bound: all K/V rows and tree nodes a chunk row can reach, the queries, the output
    prefill_read_once = (2 * w.n_kv * (Lt_ * row_b + sum(level_sizes(Lt_, w.b)[1:]) * row_b)
                         + w.prefill_n * w.n_q * (row_b + 4 * w.d))
    prefill_flops = w.n_q * (pk + pv) * 2 * w.d
    Lt = w.L + w.prefill_n
    Nt = level_sizes(Lt, w.b)
    new_nodes = sum(Nt[l] - (N[l] if l < len(N) else 0) for l in range(1, len(Nt)))
    append_bytes = 2 * 2 * w.n_kv * w.prefill_n * row_b + 2 * w.n_kv * new_nodes * row_b
    return dict(build=build_bytes, decode=decode_bytes, decode_flops=decode_flops,
                decode_grouped=grouped_bytes,
                prefill=prefill_bytes, prefill_flops=prefill_flops, append=append_bytes,
                prefill_read_once=prefill_read_once,
                decode_entries_per_row=kd + vd)


def cpu_cores():
    """Host threads the oracle may use: the process's CPU affinity, capped by the
    thread budget the environment sets (OMP_NUM_THREADS)."""
    aff = len(os.sched_getaffinity(0))
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "") or aff)
    except ValueError:
        cap = aff
    return max(1, min(aff, cap))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


# state the forked oracle workers inherit (set before the fork, read-only after)
_CPU = {}


def _oracle_rows(args):
    """Run oracle descents for `seconds`: kind 'decode' (rows of the decode batch at
    length L) or 'prefill' (rows of the causal chunk), starting at row `start` and
    striding by `stride`.  Returns the number of rows done and the time taken."""
    from oracle import recsa as O
    kind, start, stride, seconds = args
    st = _CPU
    w = st["w"]
    G = w.n_q // w.n_kv
    done = 0
    r = start
    t0 = time.perf_counter()
    while True:
        if kind == "decode":
            i, h = divmod(r % (st["B"] * G), G)
            O.descend(st["tree"], st["Qd"][i, h], 0, w.L, w.k, w.rope_base, w.softmax_scale)
        else:
            j, h = divmod(r % (w.prefill_n * G), G)
            O.descend(st["tree_p"], st["Qp"][j, h], 0, w.L + j + 1, w.k, w.rope_base,
                      w.softmax_scale)
        done += 1
        r += stride
        if time.perf_counter() - t0 > seconds:
            break
    return done, time.perf_counter() - t0


def cpu_baseline(w, B, seconds=20.0, queries=None):
    """The oracle (never tuned) on the host: the tree of KV head 0, then decode rows
    (and causal-prefill rows when the workload has a chunk) of that head's query
    heads, on one thread and on every core (independent rows over forked worker
    processes).  Runs before the process touches the GPU, so the workers fork a
    process without GPU state.  A query (token) counts n_q rows."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits

    import synth
    from oracle import recsa as O
    cores = cpu_cores()
    kinds = ["decode"] + (["prefill"] if w.prefill_n else [])
    per = seconds / (2 * len(kinds))
    with threadpool_limits(1):
        Lt = w.L + w.prefill_n
        K, V = synth.gen_kv(w, 0, Lt, heads=[0])
        W = synth.pool_w(w)[:1]
        t0 = time.perf_counter()
        tree = O.build_tree(K, V, W, w.b, w.dtype, w.pool_scale, w.L)
        t_build = time.perf_counter() - t0
        Qd = synth.decode_queries(w, B) if queries is None else queries
        _CPU.update(w=w, B=B, tree=tree, Qd=np.asarray(Qd, np.float64))
        if w.prefill_n:
            _CPU.update(tree_p=O.build_tree(K, V, W, w.b, w.dtype, w.pool_scale, Lt),
                        Qp=synth.prefill_queries(w).astype(np.float64))
        del K, V
        res = {}
        for kind in kinds:
            n1, t1 = _oracle_rows((kind, 0, 1, per))
            with mp.get_context("fork").Pool(cores) as pool:
                t0 = time.perf_counter()
                outs = pool.map(_oracle_rows, [(kind, c, cores, per) for c in range(cores)])
                tall = time.perf_counter() - t0
            nall = sum(o[0] for o in outs)
            res[kind] = {"one_thread": n1 / t1 / w.n_q, "all_cores": nall / tall / w.n_q,
                         "rows_one_thread": n1, "rows_all_cores": nall}
    _CPU.clear()
    out = {
        "value": res["decode"]["all_cores"], "unit": "decode queries/s", "cores": cores, "kind": "oracle",
        "cpu_model": cpu_model(),
        "decode_queries_per_s": {"one_thread": res["decode"]["one_thread"],
                                 "all_cores": res["decode"]["all_cores"]},
        "build_tokens_per_s_one_thread": w.L / t_build,
        "sample": (f"KV head 0 of the workload at L={w.L}: its tree built once ({t_build:.2f} s, one "
                   f"thread), then decode rows (query x head of that KV head) for {per:.0f} s on one "
                   f"thread ({res['decode']['rows_one_thread']} rows) and {per:.0f} s on {cores} forked "
                   f"workers ({res['decode']['rows_all_cores']} rows); rows/s / {w.n_q} = queries/s"),
    }
    if w.prefill_n:
        out["prefill_tokens_per_s"] = {"one_thread": res["prefill"]["one_thread"],
                                       "all_cores": res["prefill"]["all_cores"]}
        out["sample"] += (f"; causal-prefill rows of the {w.prefill_n}-query chunk over the tree at "
                          f"L+{w.prefill_n} for {per:.0f} s each way ({res['prefill']['rows_one_thread']} / "
                          f"{res['prefill']['rows_all_cores']} rows); rows/s / {w.n_q} = tokens/s")
    return out


def timing(samples):
    """Median, p10, p90 and mean of per-launch times (ms)."""
    a = np.asarray(samples, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "mean": float(a.mean())}


def run_serve(args, name):
    """A serving batch: independent sequences (own caches and trees) at ragged lengths,
    one decode query each, in one call.  Step = that call."""
    import torch

    import long_context_recsa_amd as R
    import synth
    from long_context_recsa_amd.layer import decode_multi

    seqs, Q = synth.serve_batch(name)
    w0 = seqs[0]
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(seqs[0], 1, args.cpu_seconds, queries=Q[:1])
        cpu["sample"] += " (sequence 0 of the batch)"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cap = max(w.L for w in seqs)
    p = R.make_params(w0.n_kv, w0.n_q, w0.d, w0.b, w0.k, cap, store=w0.dtype, out="f32",
                      rope_base=w0.rope_base, softmax_scale=w0.softmax_scale,
                      pool_scale=w0.pool_scale)

    def dev_store(x):
        bits = synth.storage_bits(x, w0.dtype)
        if w0.dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(bits)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    t_setup = time.perf_counter()
    layers = []
    for w in seqs:
        K, V = synth.gen_kv(w, 0, w.L)
        layer = R.RecsaLayer(p, dev)
        for g in range(w.n_kv):
            layer.k_cache[g, :w.L].copy_(dev_store(K[g]))
            layer.v_cache[g, :w.L].copy_(dev_store(V[g]))
        layer.pool_w.copy_(torch.from_numpy(synth.pool_w(w)))
        layer.build(w.L)
        layers.append(layer)
        del K, V
    q = dev_store(Q)
    out = torch.empty((len(seqs), w0.n_q, w0.d), dtype=torch.float32, device=dev)
    nws = R.recsa_multi_workspace_bytes(len(seqs))
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t_setup

    for _ in range(args.warmup):
        decode_multi(layers, q, out=out, ws=ws)
    torch.cuda.synchronize()
    evs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        decode_multi(layers, q, out=out, ws=ws)
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = timing([a.elapsed_time(b) for a, b in evs])["median"]
    row_b = w0.d * (2 if w0.dtype == "bf16" else 4)
    nbytes = sum(w.n_q * sum(row_entries(w.L, w.b, w.k)) * row_b for w in seqs)
    ach = nbytes / ms / 1e6
    tr = measured_traffic(name, "decode")
    res = {
        "metric": f"decode queries/s, {len(seqs)} independent sequences at ragged lengths "
                  f"{min(w.L for w in seqs)}..{cap}, one query each",
        "value": len(seqs) / (ms / 1e3), "unit": "decode queries/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": name, "storage": w0.dtype, "n_seq": len(seqs),
                   "lengths": [w.L for w in seqs], "n_kv_heads": w0.n_kv, "n_q_heads": w0.n_q,
                   "head_dim": w0.d, "b": w0.b, "k": w0.k},
        "ms": {"decode": ms},
        "roofline": {"kernel": "decode", "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                     "traffic": None if tr is None else tr["fetch"] + tr["write"]},
        "setup_s": t_setup,
    }
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


def run_distill(args, name):
    """Pooler distillation from dense attention on a workload's cache: B training
    queries at the cache's length, their dense outputs once (the teacher), then
    distillation steps (student decode, loss, dloss/dw with the selection fixed,
    SGD with momentum, tree rebuild).  Step = one recsa_distill_step."""
    import torch

    import long_context_recsa_amd as R
    import synth

    w = synth.WORKLOADS[name]
    B = args.batch or w.max_batch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    K, V = synth.gen_kv(w, 0, w.L)
    W = synth.pool_w(w)
    Q = synth.decode_queries(w, B)

    def dev_store(x):
        bits = synth.storage_bits(x, w.dtype)
        if w.dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(bits)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    p = R.make_params(w.n_kv, w.n_q, w.d, w.b, w.k, w.L, store=w.dtype, out="f32",
                      rope_base=w.rope_base, softmax_scale=w.softmax_scale, pool_scale=w.pool_scale)
    layer = R.RecsaLayer(p, dev)
    for g in range(w.n_kv):
        layer.k_cache[g].copy_(dev_store(K[g]))
        layer.v_cache[g].copy_(dev_store(V[g]))
    layer.pool_w.copy_(torch.from_numpy(W))
    layer.build(w.L)
    del K, V
    q = dev_store(Q)
    teacher = torch.empty((B, w.n_q, w.d), dtype=torch.float32, device=dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    layer.dense_decode(q, out=teacher)
    a.record()
    layer.dense_decode(q, out=teacher)
    b.record()
    torch.cuda.synchronize()
    t_teacher = a.elapsed_time(b)
    vel = torch.zeros_like(layer.pool_w)
    n = args.warmup + args.steps
    losses = torch.zeros(n, dtype=torch.float32, device=dev)
    ws = torch.empty(R.recsa_distill_workspace_bytes(p, B), dtype=torch.uint8, device=dev)
    lr, mu = args.lr, 0.9
    for i in range(args.warmup):
        layer.distill_step(q, teacher, lr, mu, vel, losses[i:i + 1], ws)
    torch.cuda.synchronize()
    evs = []
    t0 = time.perf_counter()
    for i in range(args.warmup, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        layer.distill_step(q, teacher, lr, mu, vel, losses[i:i + 1], ws)
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = timing([a.elapsed_time(b) for a, b in evs])["median"]
    lv = losses.cpu().numpy().tolist()
    res = {
        "metric": "pooler distillation steps/s (decode + loss + dw + update + tree rebuild per step)",
        "value": 1e3 / ms, "unit": "steps/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": name, "storage": w.dtype, "L": w.L, "n_kv_heads": w.n_kv,
                   "n_q_heads": w.n_q, "head_dim": w.d, "b": w.b, "k": w.k, "train_queries": B,
                   "lr": lr, "momentum": mu},
        "ms": {"distill_step": ms, "teacher_dense_decode": t_teacher},
        "loss_first": lv[0], "loss_last": lv[-1], "losses": lv,
    }
    print(json.dumps(res), flush=True)


def run_backward_chunk(args, name, n):
    """Backward of a causal chunk at the end of a workload's cache (training-shaped):
    the last n tokens' queries attend causally over the tree built on the L cached
    tokens; a synthetic output gradient; the selection of the forward held fixed.
    Step = one recsa_backward (dq, dk, dv, dw written), or recsa_backward_bf16 with
    --grad-dtype bf16."""
    import torch

    import long_context_recsa_amd as R
    import synth

    w = synth.WORKLOADS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    K, V = synth.gen_kv(w, 0, w.L)
    W = synth.pool_w(w)

    def dev_store(x):
        bits = synth.storage_bits(x, w.dtype)
        if w.dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(bits)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    p = R.make_params(w.n_kv, w.n_q, w.d, w.b, w.k, w.L, store=w.dtype, out="f32",
                      rope_base=w.rope_base, softmax_scale=w.softmax_scale, pool_scale=w.pool_scale)
    layer = R.RecsaLayer(p, dev)
    for g in range(w.n_kv):
        layer.k_cache[g].copy_(dev_store(K[g]))
        layer.v_cache[g].copy_(dev_store(V[g]))
    layer.pool_w.copy_(torch.from_numpy(W))
    layer.build(w.L)
    del K, V
    rng = np.random.default_rng(2024)
    q = dev_store(rng.standard_normal((n, w.n_q, w.d)).astype(np.float32))
    dO = torch.from_numpy(rng.standard_normal((n, w.n_q, w.d)).astype(np.float32)).to(dev)
    gd = args.grad_dtype
    grads = layer.backward(q, dO, causal=True, grad_dtype=gd)
    for _ in range(max(args.warmup - 1, 0)):
        layer.backward(q, dO, causal=True, grads=grads, grad_dtype=gd)
    torch.cuda.synchronize()
    evs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        layer.backward(q, dO, causal=True, grads=grads, grad_dtype=gd)
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = timing([a.elapsed_time(b) for a, b in evs])["median"]
    res = {
        "metric": "causal-chunk backward query tokens/s (dq, dk, dv, dw; selection fixed)",
        "value": n / (ms * 1e-3), "unit": "query tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": name, "storage": w.dtype, "L": w.L, "n_kv_heads": w.n_kv,
                   "n_q_heads": w.n_q, "head_dim": w.d, "b": w.b, "k": w.k, "chunk": n,
                   "rows": n * w.n_q, "path": "auto", "token_grad_dtype": gd},
        "ms": {"backward": ms},
    }
    print(json.dumps(res), flush=True)


# Workloads measured after the headline in a default run (each with its own
# build, decode batches and, where it has a chunk, append + prefill).
OTHER_WORKLOADS = ["qwen3_4b_131k", "qwen3_4b_1m_drift", "qwen3_4b_2m"]
PRECISION = ("fp32 arithmetic on bf16 storage; the parent-major prefill's q.k and P.V "
             "products are split-bf16 MFMA (hi + lo halves, about 16 significant bits) "
             "with fp32 accumulation")


def dev_store(x, dtype, dev):
    import synth
    import torch
    bits = synth.storage_bits(x, dtype)
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(bits)).to(dev)
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def measure_workload(w, batches, steps, warmup, backward=True):
    """Time every call of the path on one workload: build, decode at each batch,
    grouped decode (largest batch), the decode batch's backward (optional), append
    + prefill (when the workload has a chunk).  Returns per-op timings (ms) and the
    algorithmic-roofline figures."""
    import torch

    import long_context_recsa_amd as R
    import synth

    dev = torch.device("cuda:0")
    t_setup = time.perf_counter()
    Lt = w.L + w.prefill_n
    K, V = synth.gen_kv(w, 0, Lt)
    W = synth.pool_w(w)
    Bmax = max(batches)
    Qd = synth.decode_queries(w, Bmax)
    p = R.make_params(w.n_kv, w.n_q, w.d, w.b, w.k, Lt, store=w.dtype, out="f32",
                      rope_base=w.rope_base, softmax_scale=w.softmax_scale, pool_scale=w.pool_scale)
    layer = R.RecsaLayer(p, dev)
    for g in range(w.n_kv):
        layer.k_cache[g, :w.L].copy_(dev_store(K[g, :w.L], w.dtype, dev))
        layer.v_cache[g, :w.L].copy_(dev_store(V[g, :w.L], w.dtype, dev))
    layer.pool_w.copy_(torch.from_numpy(W))
    q_dec = {B: dev_store(Qd[:B], w.dtype, dev) for B in batches}
    out_dec = {B: torch.empty((B, w.n_q, w.d), dtype=torch.float32, device=dev) for B in batches}
    out_grp = torch.empty_like(out_dec[Bmax])
    if w.prefill_n:
        k_new = dev_store(np.ascontiguousarray(K[:, w.L:].transpose(1, 0, 2)), w.dtype, dev)
        v_new = dev_store(np.ascontiguousarray(V[:, w.L:].transpose(1, 0, 2)), w.dtype, dev)
        q_pre = dev_store(synth.prefill_queries(w), w.dtype, dev)
        out_pre = torch.empty((w.prefill_n, w.n_q, w.d), dtype=torch.float32, device=dev)
    # the same backward with bf16 token gradients (recsa_backward_bf16), where it runs
    bwd16 = backward and w.dtype == "bf16" and w.b <= 32
    if backward:
        # the output gradient is synthetic; every step writes the same gradient buffers
        d_out = torch.from_numpy(np.random.default_rng(5).standard_normal((Bmax, w.n_q, w.d))
                                 .astype(np.float32)).to(dev)
        grads = {"dk": torch.zeros((w.n_kv, Lt, w.d), dtype=torch.float32, device=dev),
                 "dv": torch.zeros((w.n_kv, Lt, w.d), dtype=torch.float32, device=dev),
                 "dw": torch.zeros((w.n_kv, w.d), dtype=torch.float32, device=dev)}
    if bwd16:
        grads16 = {"dk": torch.zeros((w.n_kv, Lt, w.d), dtype=torch.bfloat16, device=dev),
                   "dv": torch.zeros((w.n_kv, Lt, w.d), dtype=torch.bfloat16, device=dev),
                   "dw": torch.zeros((w.n_kv, w.d), dtype=torch.float32, device=dev)}
    del K, V
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t_setup
    dense = dense_context(layer, w, q_dec[Bmax])

    ops = (["build"] + [f"decode_B{B}" for B in batches] + ["decode_grouped"]
           + (["backward"] if backward else []) + (["backward_bf16"] if bwd16 else [])
           + (["append", "prefill"] if w.prefill_n else []))
    ev = {o: [] for o in ops}

    def step(record):
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)]
        marks[0].record()
        i = 1
        layer.build(w.L)
        marks[i].record(); i += 1
        for B in batches:
            layer.decode(q_dec[B], out=out_dec[B])
            marks[i].record(); i += 1
        layer.decode_grouped(q_dec[Bmax], out=out_grp)
        marks[i].record(); i += 1
        if backward:
            layer.backward(q_dec[Bmax], d_out, grads=grads)
            marks[i].record(); i += 1
        if bwd16:
            layer.backward(q_dec[Bmax], d_out, grads=grads16, grad_dtype="bf16")
            marks[i].record(); i += 1
        if w.prefill_n:
            layer.append(k_new, v_new)
            marks[i].record(); i += 1
            layer.prefill(q_pre, out=out_pre)
            marks[i].record(); i += 1
        if record:
            for j, o in enumerate(ops):
                ev[o].append((marks[j], marks[j + 1]))

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {o: timing([a.elapsed_time(b) for a, b in ev[o]]) for o in ops}
    del layer
    torch.cuda.empty_cache()

    kern = {}
    alg = {B: algorithmic(w, B) for B in batches}
    a0 = alg[Bmax]
    med = {o: ms[o]["median"] for o in ops}
    kern["tree_build"] = {"bound": "hbm", "bytes": a0["build"], "ms": med["build"],
                          "achieved": a0["build"] / med["build"] / 1e6, "unit": "GB/s"}
    for B in batches:
        kern[f"decode_B{B}"] = {"bound": "hbm", "bytes": alg[B]["decode"], "ms": med[f"decode_B{B}"],
                                "achieved": alg[B]["decode"] / med[f"decode_B{B}"] / 1e6, "unit": "GB/s"}
    kern["decode_grouped"] = {"bound": "hbm", "bytes": a0["decode_grouped"], "ms": med["decode_grouped"],
                              "achieved": a0["decode_grouped"] / med["decode_grouped"] / 1e6, "unit": "GB/s"}
    if backward:
        # the backward's bytes depend on which nodes the rows read (its tree pass writes the
        # fp32 gradients of every token), so its floor is the rows' gathers plus the token
        # gradients written once: see backward_bytes
        bb = backward_bytes(w, Bmax)
        kern["backward"] = {"bound": "hbm", "bytes": bb, "ms": med["backward"],
                            "achieved": bb / med["backward"] / 1e6, "unit": "GB/s"}
    if bwd16:
        bb = backward_bytes(w, Bmax, token_bytes=2)
        kern["backward_bf16"] = {"bound": "hbm", "bytes": bb, "ms": med["backward_bf16"],
                                 "achieved": bb / med["backward_bf16"] / 1e6, "unit": "GB/s"}
    if w.prefill_n:
        # the chunk's rows share parents, so the HBM floor is reading every reachable K/V row,
        # tree node and query once and writing the output; the bytes the rows would gather
        # one by one ride along for context
        kern["prefill"] = {"bound": "hbm", "bytes": a0["prefill_read_once"], "flops": a0["prefill_flops"],
                           "ms": med["prefill"],
                           "achieved": a0["prefill_read_once"] / med["prefill"] / 1e6, "unit": "GB/s",
                           "per_row_gather_bytes": a0["prefill"],
                           "mfma_frac": a0["prefill_flops"] / med["prefill"] / 1e9 / BF16_PEAK_TFLOPS}
        kern["append"] = {"bound": "hbm", "bytes": a0["append"], "ms": med["append"],
                          "achieved": a0["append"] / med["append"] / 1e6, "unit": "GB/s"}
    for name_, v in kern.items():
        t_ = measured_traffic(w.name, name_)
        v["traffic"] = None if t_ is None else t_["fetch"] + t_["write"]
        v["frac"] = v["achieved"] / HBM_PEAK_GBS
    res = {
        "L": w.L, "storage": w.dtype, "b": w.b, "k": w.k, "decode_batches": list(batches),
        "prefill_chunk": w.prefill_n, "ms": ms, "kernels": kern,
        "decode_queries_per_s": {f"B={B}": B / (med[f"decode_B{B}"] / 1e3) for B in batches},
        "grouped_decode_queries_per_s": Bmax / (med["decode_grouped"] / 1e3),
        "prefill_tokens_per_s": (w.prefill_n / ((med["append"] + med["prefill"]) / 1e3)
                                 if w.prefill_n else None),
        "setup_s": t_setup, "timed_wall_s": wall,
    }
    if dense is not None:
        # context only: the same batch through dense causal attention (recsa_dense_decode,
        # every cached token) on the same cache; the pages quote RecSA against dense
        # attention on their own hardware
        res["dense_context"] = {"dense_decode_ms": dense, "batch": Bmax,
                                "recsa_decode_speedup": dense / med[f"decode_B{Bmax}"]}
    return res, wall


def dense_context(layer, w, q, reps=5):
    """Median time (ms) of dense decode of the batch q over the first w.L tokens: one
    untimed call, then `reps` timed ones, outside the timed steps."""
    import torch
    layer.build(w.L)
    out = torch.empty((q.shape[0], w.n_q, w.d), dtype=torch.float32, device=q.device)
    layer.dense_decode(q, out=out)
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        layer.dense_decode(q, out=out)
        b.record()
        ts.append((a, b))
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ts]))


def backward_bytes(w, B, token_bytes=4):
    """Read-once floor of the decode batch's backward: the forward's gathers of every
    row (keys and values read again), the token gradients dk, dv of every cached token
    written once (the tree pass writes them all; fp32, or bf16 with token_bytes=2), and
    the summaries' fp32 gradients written and read once."""
    esz = 2 if w.dtype == "bf16" else 4
    kd, vd = row_entries(w.L, w.b, w.k)
    N = level_sizes(w.L, w.b)
    gathers = B * w.n_q * (kd + vd) * w.d * esz
    tokens = 2 * w.n_kv * w.L * w.d * token_bytes
    summaries = 2 * 2 * w.n_kv * sum(N[1:]) * w.d * 4
    return gathers + tokens + summaries


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_4b_524k")
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-configs", action="store_true",
                    help="measure the headline workload only (not the 131K, 1M and 2M workloads)")
    ap.add_argument("--distill", action="store_true",
                    help="time pooler distillation steps on the workload instead of the hot path")
    ap.add_argument("--lr", type=float, default=1000.0, help="distillation learning rate")
    ap.add_argument("--backward-chunk", type=int, default=0, metavar="N",
                    help="time the backward of a causal chunk of N queries at the workload's length")
    ap.add_argument("--grad-dtype", choices=["f32", "bf16"], default="f32",
                    help="token gradients of --backward-chunk: fp32 (recsa_backward) or bf16 "
                         "(recsa_backward_bf16)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (to scale HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the path shards by KV head "
              f"without communication, so the one-GPU figure is the per-GPU rate", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        src = torch.empty(args.calibrate_copy // 4, dtype=torch.float32, device="cuda:0")
        src.fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": src.numel() * 4, "launches": 5}), flush=True)
        return

    import long_context_recsa_amd as R
    import synth

    if args.workload in synth.SERVE_BATCHES:
        return run_serve(args, args.workload)
    if args.distill:
        return run_distill(args, args.workload)
    if args.backward_chunk:
        return run_backward_chunk(args, args.workload, args.backward_chunk)
    w = synth.WORKLOADS[args.workload]
    batches = [args.batch] if args.batch else list(w.decode_batches)
    B = max(batches)
    # the oracle's leg first: its worker processes fork a process that has not touched the GPU
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, B, args.cpu_seconds)
    R.load_library()
    torch.cuda.set_device(0)
    head, wall = measure_workload(w, batches, args.steps, args.warmup, backward=True)
    configs = {}
    if not args.no_configs and args.workload == "qwen3_4b_524k":
        for name in OTHER_WORKLOADS:
            wo = synth.WORKLOADS[name]
            configs[name], _ = measure_workload(wo, list(wo.decode_batches), args.steps, args.warmup,
                                                backward=False)
            print(f"measured {name}", file=sys.stderr, flush=True)

    kern = head["kernels"]
    ms = {o: v["median"] for o, v in head["ms"].items()}
    ms["decode"] = ms[f"decode_B{B}"]
    # the roofline line follows the forward path's dominant call; the backward rides along
    dom = max((n for n in kern if not n.startswith("backward")), key=lambda n: kern[n]["ms"])
    roof = {"kernel": dom, "bound": kern[dom]["bound"], "achieved": kern[dom]["achieved"],
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": kern[dom]["frac"],
            "traffic": kern[dom]["traffic"]}
    tr = measured_traffic(w.name, dom)
    if tr is not None:
        roof["traffic_split"] = tr
    if dom == "prefill":
        roof["mfma_frac"] = kern["prefill"]["mfma_frac"]
        roof["per_row_gather_bytes"] = kern["prefill"]["per_row_gather_bytes"]

    res = {
        "metric": "decode queries/s & prefill tokens/s at L=524K; % of HBM / bf16-MFMA roofline",
        "value": B / (ms[f"decode_B{B}"] / 1e3),
        "unit": "decode queries/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "precision": PRECISION,
        "data": "synthetic",
        "config": {"workload": w.name, "storage": w.dtype, "L": w.L, "n_kv_heads": w.n_kv,
                   "n_q_heads": w.n_q,
                   "head_dim": w.d, "b": w.b, "k": w.k, "decode_batch": B,
                   "prefill_chunk": w.prefill_n},
        "grouped_decode_queries_per_s": head["grouped_decode_queries_per_s"],
        "prefill_tokens_per_s": head["prefill_tokens_per_s"],
        "ms": ms,
        "timing": head["ms"],
        "kernels": kern,
        "roofline": roof,
        "configs": configs,
        "setup_s": head["setup_s"],
    }
    if "dense_context" in head:
        res["dense_context"] = head["dense_context"]
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
