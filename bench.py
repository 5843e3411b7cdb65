"""Benchmark: tree-attention forward + backward on the navigation-episode spine
tree (one GPU), plus per-kernel roofline, decode bandwidth and an oracle CPU
baseline.  Prints ONE JSON line.

Workload (the headline one): spine tree with a 512-token root, 44 history
nodes of 96 tokens chained under it and a 264-token leaf (256 observation +
8 action-query tokens) under every history node -- 16,352 unique tokens,
K = 44 paths; 32 query / 8 KV heads, head dim 128, bf16, N(0,1) inputs,
depth RoPE with base 10000.  A step is one tree_attn_fwd + tree_attn_bwd.
FLOPs count visible (i, j) pairs only: P = sum_t (pos(t) + 1) per query head,
4 d P Hq forward and 10 d P Hq backward.

Also reported (fields beside the headline): the random agentic tree and the
varlen forest (same heads and dtype), split-KV decode at 32K/64K/128K/256K
(B = 8) in GB/s of KV read, the host planner time, and the per-kernel times
from HIP events recorded between the library's launches.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "tree-attn fwd+bwd TFLOP/s on visible pairs (% bf16 MFMA peak); decode GB/s"
# the sources of the attention kernels (their traffic counts are keyed by this hash)
KERNEL_SOURCES = ["attn_fwd.hip", "attn_bwd.hip", "common.h", "plan.cpp", "plan_internal.h"]


def source_hash() -> str:
    h = hashlib.sha256()
    for s in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "prefix_shared_masked_amd", "csrc", s), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def make_inputs(n, Hq, Hkv, d, seed, dev):
    import torch
    g = torch.Generator(device=dev).manual_seed(seed)
    mk = lambda h: torch.randn(n, h, d, generator=g, device=dev, dtype=torch.float32).bfloat16()
    return mk(Hq), mk(Hkv), mk(Hkv), mk(Hq)


def time_tree(pkg, tree, steps, warmup, dev, seed=0, Hq=32, Hkv=8, d=128, rope=10000.0):
    """fwd+bwd timing with stage events.  Returns a dict of averages (ms)."""
    import torch
    t0 = time.perf_counter()
    plan = pkg.tree_plan(tree.parent, tree.seg_len)
    plan_ms = (time.perf_counter() - t0) * 1e3
    t0 = time.perf_counter()
    plan.device(dev)
    upload_ms = (time.perf_counter() - t0) * 1e3
    q, k, v, do = make_inputs(plan.n_tokens, Hq, Hkv, d, seed, dev)
    o = torch.empty_like(q)
    lse = torch.empty(Hq, plan.n_tokens, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    wf = torch.empty(max(1, pkg.attn_ws_bytes(plan, 0, 1, Hq, Hkv, d, rope)), dtype=torch.uint8, device=dev)
    # the backward workspace the binding picks by default: the full dS workspace when it fits the
    # default budget (8 GiB), else the dS blocks of as many KV heads as fit, run in rounds
    wb_bytes, kv_per_round = pkg.bwd_ws_budget(plan, 1, Hq, Hkv, d, rope)
    wb = torch.empty(max(1, wb_bytes), dtype=torch.uint8, device=dev)
    ev = pkg.HipEvents(7 * steps)

    def step(i=None):
        ef = ev.slice(7 * i, 3) if i is not None else None
        eb = ev.slice(7 * i + 3, 4) if i is not None else None
        pkg.tree_attn_fwd(plan, q, k, v, rope_base=rope, o=o, lse=lse, ws=wf, events=ef)
        pkg.tree_attn_bwd(plan, q, k, v, o, lse, do, rope_base=rope, dq=dq, dk=dk, dv=dv, ws=wb, events=eb)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - wall0) * 1e3 / steps
    span = lambda a, b: [ev.elapsed_ms(7 * i + a, 7 * i + b) for i in range(steps)]
    avg = lambda a, b: sum(span(a, b)) / steps
    med = lambda a, b: float(statistics.median(span(a, b)))
    P, flop_pair = plan.visible_pairs, d * Hq
    res = dict(
        n_tokens=plan.n_tokens, n_leaves=plan.n_leaves, n_flat=plan.n_flat, visible_pairs=P,
        por=round(1.0 - plan.n_tokens / plan.n_flat, 4) if plan.n_flat else 0.0,
        fwd_tile_efficiency=round(P / plan.computed_pairs_fwd, 4),
        bwd_tile_efficiency=round(P / plan.computed_pairs_bwd, 4),
        plan_ms=round(plan_ms, 3), upload_ms=round(upload_ms, 3),
        bwd_ws_bytes=wb_bytes, bwd_kv_heads_per_round=kv_per_round,
        # the timed region: K steps between two device synchronisations (host wall clock)
        ms_per_step=wall, event_ms_per_step=avg(0, 6), event_median_ms_per_step=med(0, 6),
        fwd_ms=avg(0, 2), bwd_ms=avg(3, 6),
        # backward events: [0] start, [1] after the preparation passes, [2] after dK/dV (and its
        # partial sum), [3] after dQ, which reads the dS blocks dK/dV stored (one product)
        k_fwd_prep_ms=avg(0, 1), k_fwd_ms=avg(1, 2), k_bwd_prep_ms=avg(3, 4), k_dkv_ms=avg(4, 5), k_dq_ms=avg(5, 6),
        k_median_ms=dict(fwd=med(1, 2), dkv=med(4, 5), dq=med(5, 6)),
        flops_fwd=4 * flop_pair * P, flops_bwd=10 * flop_pair * P,
        flops_alg=dict(fwd=4 * flop_pair * P, dq=2 * flop_pair * P, dkv=8 * flop_pair * P))
    if kv_per_round < Hkv:
        # the backward ran in rounds of KV heads; its events mark the end of the
        # first round's dK/dV, so the two spans are that and everything after it
        res["k_dkv_first_round_ms"] = res.pop("k_dkv_ms")
        res["k_dq_and_later_rounds_ms"] = res.pop("k_dq_ms")
        res["k_median_ms"] = dict(fwd=res["k_median_ms"]["fwd"])
    res["tflops"] = (res["flops_fwd"] + res["flops_bwd"]) / (res["ms_per_step"] * 1e-3) / 1e12
    del q, k, v, do, o, dq, dk, dv, wf, wb
    torch.cuda.empty_cache()
    return res


def time_partitioned(pkg, tree, capacity, steps, warmup, dev, seed=0, Hq=32, Hkv=8, d=128, rope=10000.0):
    """fwd+bwd through tree_partition_fwd/bwd (partition at a time, gateway
    gathers and the fp32 relay of chain dK/dV).  Returns averages (ms)."""
    import torch
    part = pkg.tree_partition(tree.parent, tree.seg_len, capacity)
    part.device(dev)
    whole = pkg.tree_plan(tree.parent, tree.seg_len)
    q, k, v, do = make_inputs(part.n_tokens, Hq, Hkv, d, seed, dev)
    o = torch.empty_like(q)
    lse = torch.empty(Hq, part.n_tokens, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    wf = torch.empty(max(1, pkg.partition_ws_bytes(part, 0, 1, Hq, Hkv, d, rope)), dtype=torch.uint8, device=dev)
    wb = torch.empty(max(1, pkg.partition_ws_bytes(part, 1, 1, Hq, Hkv, d, rope)), dtype=torch.uint8, device=dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
            torch.cuda.Event(enable_timing=True)) for _ in range(steps)]

    def step(i=None):
        if i is not None:
            evs[i][0].record()
        pkg.tree_partition_fwd(part, q, k, v, rope_base=rope, o=o, lse=lse, ws=wf)
        if i is not None:
            evs[i][1].record()
        pkg.tree_partition_bwd(part, q, k, v, o, lse, do, rope_base=rope, dq=dq, dk=dk, dv=dv, ws=wb)
        if i is not None:
            evs[i][2].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    fwd = sum(a.elapsed_time(b) for a, b, _ in evs) / steps
    bwd = sum(b.elapsed_time(c) for _, b, c in evs) / steps
    P = whole.visible_pairs
    local_pairs = sum(pl.visible_pairs for pl in part.plans if pl is not None)
    assert local_pairs == P  # every visible (query, key) pair is computed exactly once
    ms = fwd + bwd
    res = dict(capacity=capacity, n_parts=part.n_parts, n_tokens=part.n_tokens, naive_tokens=part.naive_tokens,
               max_local_tokens=part.max_local_tokens, ms_per_step=ms, fwd_ms=fwd, bwd_ms=bwd,
               tflops=14 * d * Hq * P / (ms * 1e-3) / 1e12)
    del q, k, v, do, o, dq, dk, dv, wf, wb
    torch.cuda.empty_cache()
    return res


def time_lmhead(pkg, tree, steps, warmup, dev, V=151936, Dm=1024, seed=9):
    """Output layer (Qwen3-0.6B shape: V = 151,936, Dm = 1,024) fused with the
    g/K weighted NLL over the tree's tokens: forward alone and forward+backward."""
    import torch
    plan = pkg.tree_plan(tree.parent, tree.seg_len)
    N = plan.n_tokens
    g = torch.Generator(device=dev).manual_seed(seed)
    h = torch.randn(N, Dm, generator=g, device=dev).bfloat16()
    W = (torch.randn(V, Dm, generator=g, device=dev) / Dm ** 0.5).bfloat16()
    labels = torch.randint(0, V, (N,), generator=g, device=dev, dtype=torch.int32)
    w = torch.from_numpy((plan.view()["g"] / plan.n_leaves).astype("float32")).to(dev)
    loss = torch.zeros(1, device=dev)
    lse = torch.empty(N, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    dh, dW = torch.empty_like(h), torch.empty_like(W)
    ws = torch.empty(pkg.lmhead_ws_bytes(N, V, Dm, True), dtype=torch.uint8, device=dev)

    def timed(grad):
        for _ in range(warmup):
            pkg.tree_lmhead_nll(h, W, labels, w, need_grad=grad, loss=loss, lse=lse, dh=dh, dW=dW,
                                err_flag=err, ws=ws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            pkg.tree_lmhead_nll(h, W, labels, w, need_grad=grad, loss=loss, lse=lse, dh=dh, dW=dW,
                                err_flag=err, ws=ws)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    fwd = timed(False)
    total = timed(True)
    gemm = 2.0 * N * V * Dm
    res = dict(n_tokens=N, vocab=V, hidden=Dm, fwd_ms=fwd, fwd_bwd_ms=total, bwd_ms=total - fwd,
               fwd_tflops=gemm / (fwd * 1e-3) / 1e12,
               # forward, the backward's recompute, dh and dW: four products of 2 N V Dm
               fwd_bwd_tflops=4 * gemm / (total * 1e-3) / 1e12,
               logits_gb_never_held=N * V * 4 / 1e9)
    del h, W, dh, dW, ws
    torch.cuda.empty_cache()
    return res


def time_nll(pkg, tree, steps, warmup, dev, V=151936, seed=10):
    """g/K weighted NLL over materialised fp32 logits [N, V] (the spine tree's
    tokens, the Qwen3-0.6B vocabulary; logits ~ N(0, 1), uniform labels with
    10% ignored): loss alone and loss + dlogits.  GB/s on the bytes each must
    move: V * 4 per row for the loss (read once), 3 V * 4 with the gradient
    (read twice: the row's max/sum, then softmax; dlogits written once)."""
    import torch
    plan = pkg.tree_plan(tree.parent, tree.seg_len)
    N = plan.n_tokens
    g = torch.Generator(device=dev).manual_seed(seed)
    x = torch.randn(N, V, generator=g, device=dev)
    labels = torch.randint(0, V, (N,), generator=g, device=dev, dtype=torch.int32)
    labels[torch.rand(N, generator=g, device=dev) < 0.1] = -100
    w = torch.from_numpy((plan.view()["g"] / plan.n_leaves).astype("float32")).to(dev)
    loss = torch.zeros(1, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    dx = torch.empty_like(x)

    def timed(grad):
        for _ in range(warmup):
            pkg.tree_weighted_nll(x, labels, w, need_grad=grad, loss=loss, dlogits=dx if grad else None,
                                  err_flag=err)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            pkg.tree_weighted_nll(x, labels, w, need_grad=grad, loss=loss, dlogits=dx if grad else None,
                                  err_flag=err)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    fwd = timed(False)
    both = timed(True)
    row = V * 4
    res = dict(n_tokens=N, vocab=V, logits_gb=N * row / 1e9, loss_ms=fwd, loss_GBps=N * row / (fwd * 1e-3) / 1e9,
               loss_grad_ms=both, loss_grad_GBps=3 * N * row / (both * 1e-3) / 1e9)
    del x, dx
    torch.cuda.empty_cache()
    return res


def time_ssm(pkg, tree, steps, warmup, dev, C=4096, K=4, seed=11):
    """Tree-routed scan and causal conv (fp32, [N, C]) over the tree's tokens:
    forward and backward of each, GB/s on the bytes each must move."""
    import torch
    plan = pkg.tree_plan(tree.parent, tree.seg_len)
    route = pkg.tree_route(plan, K)
    route.device(dev)
    N = plan.n_tokens
    g = torch.Generator(device=dev).manual_seed(seed)
    a = torch.rand(N, C, generator=g, device=dev) * 0.4 + 0.6
    b, x, dy = (torch.randn(N, C, generator=g, device=dev) for _ in range(3))
    w = torch.randn(C, K, generator=g, device=dev)
    h, da, db, y, dx = (torch.empty(N, C, device=dev) for _ in range(5))
    dw = torch.empty(C, K, device=dev)
    ws = torch.empty(max(pkg._route_ws("tree_scan_ws_bytes", route, C), pkg._route_ws("tree_conv_ws_bytes", route, C)),
                     dtype=torch.uint8, device=dev)
    calls = {
        "scan_fwd": (lambda: pkg.tree_scan_fwd(route, a, b, h=h, ws=ws), 3 * 4),          # a, b in; h out
        "scan_bwd": (lambda: pkg.tree_scan_bwd(route, a, h, dy, da=da, db=db, ws=ws), 5 * 4),  # a, h, dh in; da, db out
        "conv_fwd": (lambda: pkg.tree_conv_fwd(route, x, w, y=y), 2 * 4),                 # x in; y out
        "conv_bwd": (lambda: pkg.tree_conv_bwd(route, x, w, dy, dx=dx, dw=dw, ws=ws), 3 * 4),  # x, dy in; dx out
    }
    res = dict(n_tokens=N, channels=C, conv_k=K, n_chunks=route.n_chunks)
    for name, (fn, bpe) in calls.items():
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        res[name + "_us"] = ms * 1e3
        res[name + "_GBps"] = N * C * bpe / (ms * 1e-3) / 1e9
    del a, b, x, dy, h, da, db, y, dx, ws
    torch.cuda.empty_cache()
    return res


def time_decode(pkg, L, steps, warmup, dev, B=8, Hq=32, Hkv=8, d=128, seed=5):
    import torch
    g = torch.Generator(device=dev).manual_seed(seed)
    q = torch.randn(B, Hq, d, generator=g, device=dev).bfloat16()
    k = torch.randn(B * L, Hkv, d, generator=g, device=dev).bfloat16()
    v = torch.randn(B * L, Hkv, d, generator=g, device=dev).bfloat16()
    span_ptr = torch.arange(B + 1, dtype=torch.int32, device=dev)
    spans = torch.stack([torch.arange(B, dtype=torch.int32) * L, torch.full((B,), L, dtype=torch.int32)], 1)
    spans = spans.to(torch.int32).contiguous().to(dev)
    nbytes, n_splits = pkg.decode_ws_bytes(B, Hq, d, L)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    call = lambda evs=None: pkg.tree_decode_splitkv(q, k, v, span_ptr, spans, L, o=o, lse=lse, ws=ws, events=evs,
                                                    check_spans=False)
    pkg.tree_decode_splitkv(q, k, v, span_ptr, spans, L, o=o, lse=lse, ws=ws)  # spans checked once
    for _ in range(warmup):
        call()
    # each rep: overwrite a 512 MiB buffer (flushes the 4 MiB L2s and the 256 MiB MALL), then one
    # whole call between two events; the median over the reps
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    reps = max(steps, 20)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in evs:
        flush.fill_(1)
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    times = [e0.elapsed_time(e1) for e0, e1 in evs]
    call_ms = float(statistics.median(times))
    # the partial kernel alone, from the library's stage events (also after a flush)
    ev = pkg.HipEvents(3 * reps)
    for i in range(reps):
        flush.fill_(1)
        call(ev.slice(3 * i, 3))
    torch.cuda.synchronize()
    part = float(statistics.median(ev.elapsed_ms(3 * i, 3 * i + 1) for i in range(reps)))
    kv_bytes = 2 * B * L * Hkv * d * 2
    del k, v, flush
    torch.cuda.empty_cache()
    return dict(L=L, n_splits=n_splits, kv_bytes=kv_bytes, reps=reps, call_us=call_ms * 1e3,
                call_us_mean=sum(times) / reps * 1e3, partial_us=part * 1e3,
                GBps=kv_bytes / (call_ms * 1e-3) / 1e9, partial_GBps=kv_bytes / (part * 1e-3) / 1e9)


def cpu_baseline(tree, budget_s=20.0, seed=0):
    """The float64 oracle (per-path attention, forward + backward) on a bounded
    sample of the same workload: one KV head group (query heads 0-3), paths
    taken in order until about budget_s seconds of work.  Reported in the
    metric's unit (visible-pair FLOPs of the sampled paths per second)."""
    import numpy as np
    import oracle
    import workloads as W
    from oracle.plan import OraclePlan
    t0 = time.perf_counter()
    op = oracle.oracle_plan(tree.parent, tree.seg_len)
    plan_s = time.perf_counter() - t0
    q, k, v, do = W.attention_inputs(seed, op.n_tokens, 32, 8, 128)
    heads = [0, 1, 2, 3]
    path_pairs, t_total, n_paths = 0, 0.0, 0
    covered = np.zeros(op.n_tokens, bool)
    for idx in op.paths:
        sub = OraclePlan(**{**op.__dict__, "paths": [idx]})
        t0 = time.perf_counter()
        oracle.per_path_attention(sub, q, k, v, rope_base=10000.0, dO=do, heads=heads, check_consistency=False)
        t_total += time.perf_counter() - t0
        L = len(idx)
        path_pairs += L * (L + 1) // 2 * len(heads)
        covered[np.asarray(idx)] = True
        n_paths += 1
        if t_total >= budget_s:
            break
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=os.cpu_count())
    except Exception:
        cores = os.cpu_count()
    # the metric counts the tree's visible pairs: the sampled paths cover a subtree, whose tokens
    # see pos(t) + 1 keys each (every key of a token's path is in the subtree); the per-path run
    # computes each shared prefix once per path, the causal pairs counted separately below
    visible = int((op.pos[covered].astype(np.int64) + 1).sum()) * len(heads)
    return dict(value=14 * 128 * visible / t_total / 1e12, unit="TFLOP/s", cores=int(cores), kind="oracle",
                sample=f"per-path float64 oracle, fwd+bwd, query heads 0-3 (one KV group), first {n_paths} of "
                       f"{len(op.paths)} root-to-leaf paths of the spine tree: {visible} visible pairs of the "
                       f"subtree they cover ({path_pairs} per-path causal pairs), {t_total:.1f} s",
                seconds=round(t_total, 2), visible_pairs=visible, per_path_causal_pairs=path_pairs,
                per_path_tflops=14 * 128 * path_pairs / t_total / 1e12, oracle_plan_s=round(plan_s, 3))


# kernels launched between the same two events as the named one (their HBM
# bytes count toward its launch): dK/dV and the sum of its cut tiles' partials
SPAN = {"dkv_bf16_kernel": ("dkv_bf16_kernel", "dkv_sum_kernel")}


def load_traffic(kernel):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    total = 0
    for i, k in enumerate(SPAN.get(kernel, (kernel,))):
        e = t.get(k)
        if e is None and i > 0:
            continue
        if not e or e.get("source_hash") != source_hash():
            return None
        total += e.get("bytes_per_launch")
    return total


def load_mfma(kernel):
    """MFMA counters of a kernel (profiles/mfma.json, rocprofv3 --pmc on the spine-tree
    headline), when recorded for the current kernel sources: the MFMA-busy share of SIMD
    cycles and the FLOPs the matrix units executed per launch (SQ_INSTS_VALU_MFMA_MOPS_*
    x 512)."""
    path = os.path.join(ROOT, "profiles", "mfma.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        e = json.load(f).get(kernel)
    if not e or e.get("source_hash") != source_hash():
        return None
    return e


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--secondary", default="random_agentic_tree,varlen_forest,spine_partitioned_4096,lmhead,nll,ssm,decode",
                    help="comma-separated secondary workloads to run after the headline")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: tree attention here runs on a single device "
              "(no collectives between GPUs); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import prefix_shared_masked_amd as pkg
    import workloads as W
    pkg.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    spine = W.spine_tree()
    print("[bench] spine tree fwd+bwd", flush=True)
    head = time_tree(pkg, spine, args.steps, args.warmup, dev)
    extra = {}
    chosen = set() if args.headline_only else {x for x in args.secondary.split(",") if x}
    if chosen:
        for name, mk in (("random_agentic_tree", lambda: W.random_agentic_tree(0)),
                         ("varlen_forest", lambda: W.varlen_forest(0))):
            if name not in chosen:
                continue
            tree = mk()
            print(f"[bench] {name} fwd+bwd", flush=True)
            r = time_tree(pkg, tree, max(3, args.steps // 2), args.warmup, dev)
            extra[name] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items() if k != "flops_alg"}
        for cap in (4096,):
            if f"spine_partitioned_{cap}" not in chosen:
                continue
            print(f"[bench] spine tree partitioned at {cap} tokens, fwd+bwd", flush=True)
            r = time_partitioned(pkg, spine, cap, max(3, args.steps // 2), args.warmup, dev)
            r["vs_whole_tree"] = round(head["ms_per_step"] / r["ms_per_step"], 4)
            extra[f"spine_partitioned_{cap}"] = {k: (round(v, 4) if isinstance(v, float) else v)
                                                 for k, v in r.items()}
        if "lmhead" in chosen:
            print("[bench] output layer + weighted NLL over the spine tree's tokens", flush=True)
            r = time_lmhead(pkg, spine, max(3, args.steps // 2), args.warmup, dev)
            extra["lmhead"] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
        if "nll" in chosen:
            print("[bench] weighted NLL over materialised logits of the spine tree's tokens", flush=True)
            r = time_nll(pkg, spine, args.steps, args.warmup, dev)
            extra["nll"] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
        if "ssm" in chosen:
            print("[bench] tree-routed scan and causal conv over the spine tree's tokens", flush=True)
            r = time_ssm(pkg, spine, args.steps, args.warmup, dev)
            extra["ssm"] = {k: (round(v, 3) if isinstance(v, float) else v) for k, v in r.items()}
        for L in (32768, 65536, 131072, 262144) if "decode" in chosen else ():
            extra.setdefault("decode", [])
            print(f"[bench] decode L={L}", flush=True)
            r = time_decode(pkg, L, args.steps, args.warmup, dev)
            extra["decode"].append({k: (round(v, 3) if isinstance(v, float) else v) for k, v in r.items()})

    kernels = {"fwd": head["k_fwd_ms"], "dq": head["k_dq_ms"], "dkv": head["k_dkv_ms"]}
    dom = max(kernels, key=kernels.get)
    names = {"fwd": "fwd_bf16_kernel", "dq": "dq_ds_kernel", "dkv": "dkv_bf16_kernel"}
    achieved = head["flops_alg"][dom] / (kernels[dom] * 1e-3) / 1e12
    roofline = dict(bound="mfma", kernel=names[dom], achieved=round(achieved, 2), peak=PEAK_BF16_TFLOPS,
                    unit="TFLOP/s", frac=round(achieved / PEAK_BF16_TFLOPS, 4), traffic=load_traffic(names[dom]),
                    avg_launch_ms=round(kernels[dom], 4))
    mdom = load_mfma(names[dom])
    roofline["mfma_busy"] = mdom["mfma_busy"] if mdom else None
    per_kernel = {}
    for k2, v in kernels.items():
        e = dict(ms=round(v, 4), median_ms=round(head["k_median_ms"][k2], 4),
                 tflops=round(head["flops_alg"][k2] / (v * 1e-3) / 1e12, 2))
        m = load_mfma(names[k2])
        if m:
            e["mfma_busy"] = m["mfma_busy"]
            e["mfma_flops_over_algorithmic"] = round(m["mfma_flops_per_launch"] / head["flops_alg"][k2], 4)
            e["valu_mfma_coexec"] = m.get("coexec_over_busy")
            e["clock_ghz_under_counters"] = m.get("clock_ghz")
        per_kernel[names[k2]] = e
    per_kernel["k_prep_fwd"] = dict(ms=round(head["k_fwd_prep_ms"], 4))
    per_kernel["k_prep_bwd"] = dict(ms=round(head["k_bwd_prep_ms"], 4))

    out = {
        "metric": METRIC,
        "value": round(head["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "navigation-episode spine tree (512-token root, 44 x 96-token history nodes, "
                               "44 x 264-token leaves), fwd+bwd, depth RoPE base 10000",
                   "n_tokens": head["n_tokens"], "paths": head["n_leaves"], "n_flat": head["n_flat"],
                   "heads_q": 32, "heads_kv": 8, "head_dim": 128, "visible_pairs_per_head": head["visible_pairs"]},
        "frac_bf16_peak": round(head["tflops"] / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline,
        "per_kernel": per_kernel,
        "fwd_ms": round(head["fwd_ms"], 4), "bwd_ms": round(head["bwd_ms"], 4),
        "event_ms_per_step": round(head["event_ms_per_step"], 4),
        "event_median_ms_per_step": round(head["event_median_ms_per_step"], 4),
        "plan_ms": head["plan_ms"], "plan_upload_ms": head["upload_ms"],
        "por": head["por"], "fwd_tile_efficiency": head["fwd_tile_efficiency"],
        "bwd_tile_efficiency": head["bwd_tile_efficiency"],
        "kernel_source_hash": source_hash(),  # attention kernels and planner
    }
    if extra:
        out["secondary"] = extra
    dec = extra.get("decode")
    if dec:
        out["decode_GBps"] = {str(r["L"]): r["GBps"] for r in dec}
        out["decode_frac_hbm_peak"] = {str(r["L"]): round(r["GBps"] / PEAK_HBM_GBS, 4) for r in dec}
    if not args.no_cpu_baseline:
        print("[bench] oracle cpu baseline", flush=True)
        out["cpu_baseline"] = cpu_baseline(spine, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
