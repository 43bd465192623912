"""Benchmark of the RecSA hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
build the tree over the L cached tokens, decode a batch at length L (per
query head, then again with one selection per KV group), the backward of that
decode batch (selection fixed; a synthetic output gradient), append the
prefill chunk (growing the tree) and run the causal prefill of that chunk.
Each call is timed with HIP events on the stream it is launched on.  The
roofline line follows the forward calls.

Prints one JSON line: value = decode queries/s; prefill tokens/s, tree-build
bandwidth and the roofline fractions of every kernel ride along.
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
    for this workload: lines 'traffic <kernel> fetch_bytes=F write_bytes=W sources=<sha256>'.
    None when there is no summary or the kernels changed since it was taken."""
    path = COUNTERS.format(workload=workload)
    if not os.path.exists(path):
        return None
    digest = sources_digest(kernel) if kernel in OP_SOURCES else None
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


def cpu_baseline(w, B, seconds=15.0, queries=None):
    """The oracle (never tuned) on the host: tree over one KV head, then decode
    rows of that head until about `seconds` have passed."""
    from threadpoolctl import threadpool_limits

    import synth
    from oracle import recsa as O
    with threadpool_limits(1):
        K, V = synth.gen_kv(w, 0, w.L, heads=[0])
        W = synth.pool_w(w)[:1]
        Q = synth.decode_queries(w, B) if queries is None else queries
        t0 = time.perf_counter()
        tree = O.build_tree(K, V, W, w.b, w.dtype, w.pool_scale, w.L)
        t_build = time.perf_counter() - t0
        rows = 0
        t0 = time.perf_counter()
        G = w.n_q // w.n_kv
        while True:
            i, h = divmod(rows, G)
            O.descend(tree, Q[i % B, h].astype(np.float64), 0, w.L, w.k, w.rope_base,
                      w.softmax_scale)
            rows += 1
            if time.perf_counter() - t0 > seconds:
                break
        t_dec = time.perf_counter() - t0
    return {
        "value": rows / t_dec / w.n_q, "unit": "decode queries/s", "cores": 1, "kind": "oracle",
        "sample": f"{rows} decode rows (query x head) of KV head 0 at L={w.L}, single thread, "
                  f"after building that head's tree in {t_build:.1f} s; queries/s = rows/s / {w.n_q}",
    }


def run_serve(args, name):
    """A serving batch: independent sequences (own caches and trees) at ragged lengths,
    one decode query each, in one call.  Step = that call."""
    import torch

    import long_context_recsa_amd as R
    import synth
    from long_context_recsa_amd.layer import decode_multi

    seqs, Q = synth.serve_batch(name)
    w0 = seqs[0]
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
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
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
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(seqs[0], 1, args.cpu_seconds, queries=Q[:1])
        res["cpu_baseline"]["sample"] += " (sequence 0 of the batch)"
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
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
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
    Step = one recsa_backward (dq, dk, dv, dw written)."""
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
    grads = layer.backward(q, dO, causal=True)
    for _ in range(max(args.warmup - 1, 0)):
        layer.backward(q, dO, causal=True, grads=grads)
    torch.cuda.synchronize()
    evs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        layer.backward(q, dO, causal=True, grads=grads)
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    res = {
        "metric": "causal-chunk backward query tokens/s (dq, dk, dv, dw; selection fixed)",
        "value": n / (ms * 1e-3), "unit": "query tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": name, "storage": w.dtype, "L": w.L, "n_kv_heads": w.n_kv,
                   "n_q_heads": w.n_q, "head_dim": w.d, "b": w.b, "k": w.k, "chunk": n,
                   "rows": n * w.n_q, "path": "auto"},
        "ms": {"backward": ms},
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="qwen3_4b_524k")
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--distill", action="store_true",
                    help="time pooler distillation steps on the workload instead of the hot path")
    ap.add_argument("--lr", type=float, default=1000.0, help="distillation learning rate")
    ap.add_argument("--backward-chunk", type=int, default=0, metavar="N",
                    help="time the backward of a causal chunk of N queries at the workload's length")
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
    B = args.batch or w.max_batch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_setup = time.perf_counter()
    Lt = w.L + w.prefill_n
    K, V = synth.gen_kv(w, 0, Lt)
    W = synth.pool_w(w)
    Qd = synth.decode_queries(w, B)
    Qp = synth.prefill_queries(w) if w.prefill_n else None

    def dev_store(x):
        bits = synth.storage_bits(x, w.dtype)
        if w.dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(bits)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    p = R.make_params(w.n_kv, w.n_q, w.d, w.b, w.k, Lt, store=w.dtype, out="f32",
                      rope_base=w.rope_base, softmax_scale=w.softmax_scale, pool_scale=w.pool_scale)
    layer = R.RecsaLayer(p, dev)
    for g in range(w.n_kv):
        layer.k_cache[g, :w.L].copy_(dev_store(K[g, :w.L]))
        layer.v_cache[g, :w.L].copy_(dev_store(V[g, :w.L]))
    layer.pool_w.copy_(torch.from_numpy(W))
    q_dec = dev_store(Qd)
    if w.prefill_n:
        k_new = dev_store(np.ascontiguousarray(K[:, w.L:].transpose(1, 0, 2)))
        v_new = dev_store(np.ascontiguousarray(V[:, w.L:].transpose(1, 0, 2)))
        q_pre = dev_store(Qp)
        out_pre = torch.empty((w.prefill_n, w.n_q, w.d), dtype=torch.float32, device=dev)
    out_dec = torch.empty((B, w.n_q, w.d), dtype=torch.float32, device=dev)
    out_grp = torch.empty_like(out_dec)
    # backward of the decode batch: the output gradient is synthetic; every step writes
    # the same token and pooler gradient buffers
    d_out = torch.from_numpy(np.random.default_rng(5).standard_normal((B, w.n_q, w.d)).astype(np.float32)).to(dev)
    grads = {"dk": torch.zeros((w.n_kv, Lt, w.d), dtype=torch.float32, device=dev),
             "dv": torch.zeros((w.n_kv, Lt, w.d), dtype=torch.float32, device=dev),
             "dw": torch.zeros((w.n_kv, w.d), dtype=torch.float32, device=dev)}
    del K, V
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t_setup

    ops = ["build", "decode", "decode_grouped", "backward"] + (["append", "prefill"] if w.prefill_n else [])
    ev = {o: [] for o in ops}

    def step(record):
        marks = {}
        def mark(name):
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            marks[name] = e
        mark("t0")
        layer.build(w.L)
        mark("build")
        layer.decode(q_dec, out=out_dec)
        mark("decode")
        layer.decode_grouped(q_dec, out=out_grp)
        mark("decode_grouped")
        layer.backward(q_dec, d_out, grads=grads)
        mark("backward")
        if w.prefill_n:
            layer.append(k_new, v_new)
            mark("append")
            layer.prefill(q_pre, out=out_pre)
            mark("prefill")
        if record:
            order = ["t0"] + ops
            ev_pairs = [(order[i], order[i + 1]) for i in range(len(ops))]
            for a_, b_ in ev_pairs:
                ev[b_].append((marks[a_], marks[b_]))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {o: float(np.mean([a.elapsed_time(b) for a, b in ev[o]])) for o in ops}

    alg = algorithmic(w, B)
    kern = {}
    kern["tree_build"] = {"bound": "hbm", "bytes": alg["build"], "ms": ms["build"],
                          "achieved": alg["build"] / ms["build"] / 1e6, "unit": "GB/s"}
    kern["decode"] = {"bound": "hbm", "bytes": alg["decode"], "ms": ms["decode"],
                      "achieved": alg["decode"] / ms["decode"] / 1e6, "unit": "GB/s"}
    # the backward's bytes depend on which nodes the rows read (its tree pass rewrites the
    # fp32 gradients of every token under a touched node), so it is reported by its measured
    # HBM traffic alone
    kern["backward"] = {"bound": "hbm", "bytes": None, "ms": ms["backward"], "achieved": None,
                        "unit": "GB/s"}
    kern["decode_grouped"] = {"bound": "hbm", "bytes": alg["decode_grouped"], "ms": ms["decode_grouped"],
                              "achieved": alg["decode_grouped"] / ms["decode_grouped"] / 1e6,
                              "unit": "GB/s"}
    if w.prefill_n:
        # the chunk's rows share parents, so the HBM floor is reading every reachable K/V row,
        # tree node and query once and writing the output; the bytes the rows would gather
        # one by one ride along for context
        kern["prefill"] = {"bound": "hbm", "bytes": alg["prefill_read_once"], "flops": alg["prefill_flops"],
                           "ms": ms["prefill"],
                           "achieved": alg["prefill_read_once"] / ms["prefill"] / 1e6, "unit": "GB/s",
                           "per_row_gather_bytes": alg["prefill"],
                           "mfma_frac": alg["prefill_flops"] / ms["prefill"] / 1e9 / BF16_PEAK_TFLOPS}
        kern["append"] = {"bound": "hbm", "bytes": alg["append"], "ms": ms["append"],
                          "achieved": alg["append"] / ms["append"] / 1e6, "unit": "GB/s"}
    for name_, v in kern.items():
        t_ = measured_traffic(w.name, name_)
        v["traffic"] = None if t_ is None else t_["fetch"] + t_["write"]
        if v["achieved"] is None and v["traffic"] is not None:
            v["traffic_GBs"] = v["traffic"] / v["ms"] / 1e6
            v["frac"] = v["traffic_GBs"] / HBM_PEAK_GBS
        else:
            v["frac"] = None if v["achieved"] is None else v["achieved"] / HBM_PEAK_GBS
    # the roofline line follows the forward path; the backward rides along in `kernels`
    dom = max((n for n in kern if n != "backward"), key=lambda n: kern[n]["ms"])
    tr = measured_traffic(w.name, dom)
    roof = {"kernel": dom, "bound": kern[dom]["bound"], "achieved": kern[dom]["achieved"],
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": kern[dom]["frac"],
            "traffic": None if tr is None else tr["fetch"] + tr["write"]}
    if tr is not None:
        roof["traffic_split"] = tr
    if dom == "prefill":
        roof["mfma_frac"] = kern["prefill"]["mfma_frac"]
        roof["per_row_gather_bytes"] = alg["prefill"]

    step_ms = wall / args.steps * 1e3
    res = {
        "metric": "decode queries/s & prefill tokens/s at L=524K; % of HBM / bf16-MFMA roofline",
        "value": B / (ms["decode"] / 1e3),
        "unit": "decode queries/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": step_ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "storage": w.dtype, "L": w.L, "n_kv_heads": w.n_kv,
                   "n_q_heads": w.n_q,
                   "head_dim": w.d, "b": w.b, "k": w.k, "decode_batch": B,
                   "prefill_chunk": w.prefill_n},
        "grouped_decode_queries_per_s": B / (ms["decode_grouped"] / 1e3),
        "prefill_tokens_per_s": (w.prefill_n / ((ms["append"] + ms["prefill"]) / 1e3)
                                 if w.prefill_n else None),
        "ms": ms,
        "kernels": kern,
        "roofline": roof,
        "setup_s": t_setup,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, B, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
