"""Throughput of one draft-tree verification step on one MI355X.

A step is the whole verification path for one attention layer over one batch:
tv_tree_attention_from_parents (the tree mask and depths built inside the
attention kernel, which also writes them for the accept) -> tv_accept_commit
(greedy accept and the in-place KV commit in one launch); the paged step is
tv_tree_attention_paged_from_parents -> tv_accept_commit_paged (--separate-tree:
tv_build_tree -> tv_tree_attention(_paged) -> tv_accept -> tv_commit(_paged)).
All through the C ABI. The headline workload is the Llama-3-8B-shaped GQA batch (32 q / 8 kv
heads, head dim 128, batch 8, prefix 4096, 60-node EAGLE-2-style trees, bf16).

Inputs are generated once on the host, copied to HBM, and replicated into
enough independent copies that consecutive steps never find their prefix KV in
the 256 MB Infinity Cache; step k uses copy k mod R. Each step re-appends the
tree KV into its copy and commits from the same starting prefix length, so all
steps do identical work.

Prints one JSON line. `value` = tree nodes verified per second over the timed
steps (wall clock between two device synchronisations; the timed loop calls
the C ABI with arguments built once, as a native caller would). `roofline`
reports the attention call (with the tree set-up in the dense step):
algorithmic HBM bytes per call divided by the call's average duration, from
HIP events on its launch stream around K calls back to back after the timed
steps (the rocprofv3 average of its kernels agrees with this figure); the
line also carries the call timed inside K further steps, an event pair around
each (which adds a few microseconds, so the timed steps carry none); `traffic` is the measured HBM bytes per call from
profiles/ when it matches the source.

`--workload typical` measures typical acceptance instead (tv_accept_typical on
the same trees, bf16 target logits over a 32000-token vocabulary by default):
its roofline counts the live rows of logits, read once.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "tree-verify nodes/sec and achieved HBM GB/s (% of peak), 8B-shaped GQA batch 8"
HBM_PEAK_GBS = 8000.0
INFINITY_CACHE_BYTES = 256 << 20
KERNEL_SOURCES = ["tv_attn_bf16.hip", "tv_attn_waits.h", "tv_attn_f32.hip", "tv_device.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "tree_attention_verification_tv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w) -> dict:
    """HBM bytes the attention must move at least once (live nodes only)."""
    import numpy as np
    es = 4 if w.dtype == "f32" else 2
    D = w.D
    n = w.n_nodes.astype(np.int64)
    P = w.prefix_len.astype(np.int64)
    prefix_kv = int((P * w.Hkv * D * 2 * es).sum())
    q_in = int((n * w.Hq * D * es).sum())
    tree_kv_in = int((n * w.Hkv * D * 2 * es).sum())
    tree_kv_append = tree_kv_in
    out = q_in
    total = prefix_kv + q_in + tree_kv_in + tree_kv_append + out
    return dict(prefix_kv=prefix_kv, q=q_in, tree_kv_read=tree_kv_in,
                tree_kv_append=tree_kv_append, out=out, total=total)


MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak of one MI355X
# one vector-ALU operation per lane per cycle: 256 CUs x 4 SIMDs x 32 lanes'
# worth of fp32 FMAs at 2.4 GHz is 157.3 TFLOP/s counted as two flops each,
# so 78.6 T single operations (a compare) per second
ALU_OPS_PEAK_T = 157.3 / 2


def algorithmic_flops(w) -> int:
    """Multiply-add flops of the attention (live nodes only): per query row,
    2 D for each score and 2 D for each value row it weighs, over the prefix
    and the node's ancestors-or-self (depth + 1 keys)."""
    import numpy as np
    total = 0
    for b in range(w.B):
        n = int(w.n_nodes[b])
        depth = np.zeros(n, dtype=np.int64)
        for i in range(1, n):
            depth[i] = depth[w.parents[b, i]] + 1
        keys = int(w.prefix_len[b]) * n + int((depth + 1).sum())
        total += 4 * w.D * w.Hq * keys
    return total


def roofline_bound(w, bytes_: int, flops: int) -> str:
    """The bound of a bf16 call is the matrix cores when its arithmetic
    intensity exceeds the chip's ridge (peak flops / peak bytes), else HBM;
    fp32 calls run on the vector ALU at about one flop per byte (HBM)."""
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    return "mfma" if w.dtype == "bf16" and flops > ridge * bytes_ else "hbm"


def load_traffic(workload: str):
    """Measured HBM bytes per tv_tree_attention call (rocprofv3 FETCH_SIZE +
    WRITE_SIZE of its kernels, scaled by a plain copy), valid only for the
    kernel source they were taken on."""
    path = os.path.join(ROOT, "profiles", f"traffic_attention_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def device_warmup(step, seconds: float) -> float:
    """Runs step(k) until `seconds` of wall clock have passed (synchronising
    every 64 calls) and returns the time spent. The device's clocks take tens
    of milliseconds of load to settle: the first ~50 ms of attention calls
    measured 7% slower than the rest. This precedes the W warmup steps."""
    import torch
    t0 = time.perf_counter()
    k = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(64):
            step(k)
            k += 1
        torch.cuda.synchronize()
    return time.perf_counter() - t0


def cpu_baseline(w, budget_s: float = 12.0, paged: bool = False) -> dict:
    """The oracle, as it is, on whole sequences of the same workload until
    about budget_s seconds of CPU work; one BLAS thread. paged: each
    sequence's cache first goes to shuffled pages and back through the block
    table (oracle.scatter_pages / gather_pages), inside the timed region."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    nodes = 0
    done = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        rng = np.random.default_rng(0)
        for b in range(w.B):
            inp = w.oracle_inputs(b)
            if paged:
                mp = w.cap // oracle.PAGE
                bt = rng.permutation(mp)[None, :].astype(np.int32)
                shape = (mp, w.Hkv, oracle.PAGE, w.D)
                kp, vp = oracle.scatter_pages(inp["k_cache"], inp["v_cache"], bt, np.zeros(shape), np.zeros(shape))
                inp["k_cache"], inp["v_cache"] = oracle.gather_pages(kp, vp, bt)
            oracle.verify_step(inp)
            nodes += int(w.n_nodes[b])
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
    dt = time.perf_counter() - t0
    cpu = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu = next(l.split(":", 1)[1].strip() for l in fh if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": nodes / dt, "unit": "tree-nodes/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} of {w.B} sequences ({nodes} nodes), full verification step "
                      f"(tree set-up, attention over prefix {int(np.mean(w.prefix_len[:done]))} "
                      f"+ ancestors, accept, commit{', through a shuffled block table' if paged else ''}), "
                      f"numpy float64, 1 BLAS thread of "
                      f"{len(os.sched_getaffinity(0))} available ({cpu}), {dt:.1f} s"}


TYPICAL_EPS, TYPICAL_DELTA = 0.09, 0.3
TYPICAL_SOURCES = ["tv_typical.hip", "tv_tree.hip", "tv_device.h"]


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "tree_attention_verification_tv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def typical_source_hash() -> str:
    h = hashlib.sha256()
    for f in TYPICAL_SOURCES:
        with open(os.path.join(ROOT, "tree_attention_verification_tv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_typical_traffic(workload: str):
    """Measured HBM bytes per tv_accept_typical call (as load_traffic)."""
    path = os.path.join(ROOT, "profiles", f"traffic_typical_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_hash") != typical_source_hash():
        return None
    return rec.get("bytes_per_launch")


def typical_cpu_baseline(w, x64, budget_s: float = 8.0) -> dict:
    """The oracle's typical acceptance, as it is, on the whole batch, repeated
    for about budget_s seconds; one thread."""
    from threadpoolctl import threadpool_limits

    import oracle
    runs = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while True:
            oracle.typical_accept(x64, w.tok, w.parents, w.n_nodes, TYPICAL_EPS, TYPICAL_DELTA)
            runs += 1
            if time.perf_counter() - t0 >= budget_s:
                break
    dt = time.perf_counter() - t0
    return {"value": runs * w.total_nodes / dt, "unit": "tree-nodes/s", "cores": 1, "kind": "oracle",
            "sample": f"{runs} passes over the whole batch ({w.total_nodes} nodes, vocabulary "
                      f"{x64.shape[2]}), numpy float64 softmax / entropy / tree scan, 1 thread, "
                      f"{dt:.1f} s"}


def bench_typical(args) -> None:
    """Typical acceptance from the target's logits on the headline trees:
    one tv_accept_typical call (statistics kernel + tree scan) per step."""
    import numpy as np
    import torch

    import tree_attention_verification_tv_amd as tv
    from workloads import bf16_bits_to_f32, generate, target_logits

    dev = torch.device("cuda:0")
    w = generate(args.config, seed=args.seed)
    L = target_logits(w, vocab=args.vocab, dtype="bf16")
    x = torch.from_numpy(L).view(torch.int16).view(torch.bfloat16).to(dev)
    row_bytes = args.vocab * 2
    logits_bytes = w.total_nodes * row_bytes            # live rows, read once
    copies = args.copies or max(2, -(-4 * INFINITY_CACHE_BYTES // x.numel() // 2))
    sets = [x] + [x.clone() for _ in range(copies - 1)]

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    parents, n_nodes, tok = up(w.parents), up(w.n_nodes), up(w.tok)
    anc, depth, err = tv.build_tree(parents, n_nodes)
    stream = torch.cuda.current_stream()
    # one checked call through the binding, then the C ABI with fixed arguments
    r = tv.accept_typical(sets[0], tok, parents, anc, depth, n_nodes, err, epsilon=TYPICAL_EPS,
                          delta=TYPICAL_DELTA)
    acc_len, path, bonus, toks, ent, p_tok, am = r
    lib = tv._lib.load()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def P(t):
        return ctypes.c_void_p(t.data_ptr())

    tail = (P(tok), P(parents), P(anc), P(depth), P(n_nodes), P(err), w.B, w.n_max,
            ctypes.c_float(TYPICAL_EPS), ctypes.c_float(TYPICAL_DELTA), P(ent), P(p_tok), P(am),
            P(acc_len), P(path), P(bonus), P(toks), sp)
    heads = [(P(x_k), tv._lib.TV_BF16, args.vocab) for x_k in sets]

    def step(k):
        if lib.tv_accept_typical(*heads[k % copies], *tail):
            raise RuntimeError("tv_accept_typical failed")

    warm_s = device_warmup(step, args.device_warmup)
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(args.warmup + k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # the call alone, K calls back to back between one pair of HIP events
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for k in range(args.steps):
        step(k)
    e1.record(stream)
    torch.cuda.synchronize()
    call_s = e0.elapsed_time(e1) * 1e-3 / args.steps
    achieved = logits_bytes / call_s / 1e9
    rec = {
        "metric": "typical acceptance: tree nodes/s and logits GB/s (% of HBM peak), "
                  "8B-shaped batch 8 trees",
        "value": w.total_nodes / ((t1 - t0) / args.steps),
        "unit": "tree-nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "device_warmup_s": round(warm_s, 3),
        "ms_per_step": (t1 - t0) * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"typical-accept-{w.name}-v{args.vocab}", "batch": w.B,
                   "tree_nodes": int(w.n_nodes.max()), "vocab": args.vocab,
                   "epsilon": TYPICAL_EPS, "delta": TYPICAL_DELTA, "input_copies_rotated": copies,
                   "seed": args.config if args.seed is None else args.seed},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": load_typical_traffic(f"{w.name}-v{args.vocab}"),
                     "kernel": "tv_accept_typical call: typical_stats_kernel + accept_kernel<true>; "
                               "HIP events on its stream around K calls back to back",
                     "algorithmic_bytes_per_launch": logits_bytes,
                     "call_us_mean": call_s * 1e6},
        "mean_accept_len": float(acc_len.float().mean().item()),
        "kernel_source_hash": typical_source_hash(),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = typical_cpu_baseline(w, bf16_bits_to_f32(L).astype(np.float64))
    print(json.dumps(rec), flush=True)


DRAFT_SHAPES = {3: (8, 6, 8, 8, 60), 5: (64, 7, 4, 3, 32)}   # B, S, K, M, n per workload


def bench_draft_tree(args) -> None:
    """EAGLE-2 tree construction (tv_eagle2_tree) for the batch of the
    headline workload (8 trees: 6 steps, top-8 of each layer grown by 8
    children, 60 nodes kept) or, with --config 5, the ragged serving batch
    (64 trees: 7 steps, top-4 by 3, 32 nodes)."""
    import numpy as np
    import torch

    import tree_attention_verification_tv_amd as tv
    from workloads import draft_proposals

    dev = torch.device("cuda:0")
    B, S, K, M, n = DRAFT_SHAPES[args.config]
    conf, cand, root = draft_proposals(B, S, K, M, seed=args.config if args.seed is None else args.seed)
    c_d, k_d, r_d = (torch.from_numpy(x).to(dev) for x in (conf, cand, root))
    parents, tokens, values, n_nodes = tv.eagle2_tree(c_d, k_d, r_d, n)
    lib = tv._lib.load()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())   # noqa: E731
    call = (P(c_d), P(k_d), P(r_d), B, S, K, M, n, P(parents), P(tokens), P(values), P(n_nodes), sp)

    def step():
        if lib.tv_eagle2_tree(*call):
            raise RuntimeError("tv_eagle2_tree failed")

    warm_s = device_warmup(lambda k: step(), args.device_warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    call_s = e0.elapsed_time(e1) * 1e-3 / args.steps
    # work: the rank comparisons (each layer node against its layer, each
    # created node against all created nodes, each against those before it)
    created, layer, comps = 1, 1, 0
    for _ in range(S):
        comps += layer * layer
        layer = min(K, layer) * M
        created += layer
    comps += 2 * created * created
    comps *= B
    achieved = comps / call_s / 1e12
    rec = {
        "metric": "EAGLE-2 draft trees built per second (tree construction before verification)",
        "value": B / ((t1 - t0) / args.steps),
        "unit": "trees/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "device_warmup_s": round(warm_s, 3),
        "ms_per_step": (t1 - t0) * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"eagle2-draft-tree-b{B}-s{S}-k{K}-m{M}-n{n}", "batch": B, "steps": S,
                   "grown_per_layer": K, "children": M, "nodes_kept": n},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": ALU_OPS_PEAK_T, "unit": "Tcompare/s",
                     "frac": achieved / ALU_OPS_PEAK_T, "traffic": None,
                     "kernel": "eagle2_tree_kernel (one workgroup per tree); HIP events around K calls "
                               "back to back; work = rank comparisons, peak = one vector-ALU operation "
                               "per lane per cycle (the fp32 FMA rate 157.3 TFLOP/s counts two flops "
                               "per FMA)",
                     "comparisons_per_launch": comps, "call_us_mean": call_s * 1e6},
        "kernel_source_hash": source_hash(["tv_draft.hip"]),
    }
    if not args.no_cpu_baseline:
        import oracle
        runs, t2 = 0, time.perf_counter()
        while time.perf_counter() - t2 < 5.0:
            for b in range(B):
                oracle.eagle2_tree(conf[b], cand[b], root[b], n)
            runs += 1
        dt = time.perf_counter() - t2
        rec["cpu_baseline"] = {"value": runs * B / dt, "unit": "trees/s", "cores": 1, "kind": "oracle",
                               "sample": f"{runs} passes over the {B} trees, Python/NumPy, 1 thread, {dt:.1f} s"}
    print(json.dumps(rec), flush=True)


def bench_spec_sample(args) -> None:
    """Chain speculative sampling (tv_speculative_sample): batch 8, 5 drafted
    tokens per sequence, bf16 target and draft logits over a 32000-entry
    vocabulary (the headline batch and vocabulary)."""
    import numpy as np
    import torch

    import tree_attention_verification_tv_amd as tv
    from workloads import bf16_bits_to_f32, speculative_inputs

    dev = torch.device("cuda:0")
    B, L, V = 8, 5, args.vocab
    p, q, draft, u_acc, u_res = speculative_inputs(B, L, V=V, seed=args.config if args.seed is None else args.seed)
    bf = lambda a: torch.from_numpy(a).view(torch.int16).view(torch.bfloat16)   # noqa: E731
    row_bytes = V * 2
    copies = args.copies or max(2, -(-4 * INFINITY_CACHE_BYTES // ((p.size + q.size) * 2)))
    sets = [(bf(p).to(dev), bf(q).to(dev)) for _ in range(copies)]
    d_draft, d_ua, d_ur = (torch.from_numpy(x).to(dev) for x in (draft, u_acc, u_res))
    acc, toks, pt, qt = tv.speculative_sample(sets[0][0], sets[0][1], d_draft, d_ua, d_ur)
    lib = tv._lib.load()
    ws_n = int(lib.tv_speculative_sample_workspace_size(B, L))
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())   # noqa: E731
    tail = (P(d_draft), P(d_ua), P(d_ur), B, L, P(pt), P(qt), P(acc), P(toks), P(ws), ws_n, sp)

    def step(k):
        pp, qq = sets[k % copies]
        if lib.tv_speculative_sample(P(pp), P(qq), tv._lib.TV_BF16, V, *tail):
            raise RuntimeError("tv_speculative_sample failed")

    warm_s = device_warmup(step, args.device_warmup)
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for k in range(args.steps):
        step(k)
    e1.record(stream)
    torch.cuda.synchronize()
    call_s = e0.elapsed_time(e1) * 1e-3 / args.steps
    # every target and draft row is read once; the row drawn from is read again
    algo = (B * (L + 1) + B * L) * row_bytes + 2 * B * row_bytes
    achieved = algo / call_s / 1e9
    rec = {
        "metric": "chain speculative sampling: drafted tokens verified per second, 8 sequences x 5 tokens",
        "value": B * L / ((t1 - t0) / args.steps),
        "unit": "drafted-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "device_warmup_s": round(warm_s, 3),
        "ms_per_step": (t1 - t0) * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"spec-sample-b{B}-l{L}-v{V}", "batch": B, "drafted": L, "vocab": V,
                   "input_copies_rotated": copies},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "tv_speculative_sample call: spec_stats_kernel + spec_sample_kernel; HIP events "
                               "around K calls back to back",
                     "algorithmic_bytes_per_launch": algo, "call_us_mean": call_s * 1e6},
        "mean_accept_len": float(acc.float().mean().item()),
        "kernel_source_hash": source_hash(["tv_typical.hip"]),
    }
    if not args.no_cpu_baseline:
        import oracle
        pf, qf = bf16_bits_to_f32(p).astype(np.float64), bf16_bits_to_f32(q).astype(np.float64)
        runs, t2 = 0, time.perf_counter()
        while time.perf_counter() - t2 < 5.0:
            for b in range(B):
                oracle.speculative_sample(pf[b], qf[b], draft[b], u_acc[b].astype(np.float64), float(u_res[b]))
            runs += 1
        dt = time.perf_counter() - t2
        rec["cpu_baseline"] = {"value": runs * B * L / dt, "unit": "drafted-tokens/s", "cores": 1,
                               "kind": "oracle", "sample": f"{runs} passes over the {B} sequences, NumPy float64, "
                                                           f"1 thread, {dt:.1f} s"}
    print(json.dumps(rec), flush=True)


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3, help="workload 1..5 (3 = headline)")
    ap.add_argument("--copies", type=int, default=0, help="input copies rotated per step (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--device-warmup", type=float, default=0.3,
                    help="seconds of untimed steps before the W warmup steps (the clocks settle)")
    ap.add_argument("--separate-tree", action="store_true",
                    help="dense step with tv_build_tree + tv_tree_attention instead of the combined call")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--workload", choices=("step", "typical", "paged", "draft-tree", "spec-sample"), default="step",
                    help="step: the verification step (default); typical: typical acceptance "
                         "from target logits on the same trees; paged: the step over a paged "
                         "KV cache (shuffled 64-slot pages); draft-tree: EAGLE-2 tree "
                         "construction from draft proposals; spec-sample: chain speculative "
                         "sampling of 5 drafted tokens per sequence")
    ap.add_argument("--vocab", type=int, default=32000, help="vocabulary of --workload typical")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the verification "
              "path has no multi-GPU form in this library; see DESIGN.md for how it would shard)",
              file=sys.stderr)
        sys.exit(2)

    if args.workload == "typical":
        bench_typical(args)
        return
    if args.workload == "draft-tree":
        bench_draft_tree(args)
        return
    if args.workload == "spec-sample":
        bench_spec_sample(args)
        return

    import numpy as np
    import torch

    import tree_attention_verification_tv_amd as tv
    from workloads import generate

    dev = torch.device("cuda:0")
    w = generate(args.config, seed=args.seed)
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16

    def up(a):
        x = torch.from_numpy(np.ascontiguousarray(a))
        if w.dtype == "bf16" and a.dtype == np.uint16:
            x = x.view(torch.int16).view(torch.bfloat16)
        return x.to(dev)

    parents, n_nodes, plen = up(w.parents), up(w.n_nodes), up(w.prefix_len)
    tok, tgt = up(w.tok), up(w.tgt)
    base = {k: up(getattr(w, k)) for k in ("q", "k_new", "v_new", "k_cache", "v_cache")}
    base["v_cache"] = tv.v_cache_blocked(base["v_cache"])
    per_copy = sum(t.numel() * t.element_size() for t in base.values())
    copies = args.copies or max(2, -(-4 * INFINITY_CACHE_BYTES // per_copy))
    sets = [base] + [{k: t.clone() for k, t in base.items()} for _ in range(copies - 1)]
    paged = args.workload == "paged"
    if paged:
        # each copy's cache moves to page pools under its own random table
        # (every 64-slot block of every sequence on a page drawn without
        # replacement); the dense copy is dropped
        mp = w.cap // tv.PAGE
        n_pages = B_pages = w.B * mp
        rng = np.random.default_rng(7)
        for s in sets:
            s["bt"] = torch.from_numpy(rng.permutation(B_pages).reshape(w.B, mp).astype(np.int32)).to(dev)
            s["k_cache"], s["v_cache"] = tv.pages_from_dense(s["k_cache"], s["v_cache"], s["bt"], n_pages)
            s["pk"] = tv._lib.TvPagedKv()
            s["pk"].block_table, s["pk"].max_pages, s["pk"].num_pages = s["bt"].data_ptr(), mp, n_pages
        torch.cuda.synchronize()

    B, n_max = w.B, w.n_max
    anc = torch.empty((B, n_max), dtype=torch.int64, device=dev)
    depth = torch.empty((B, n_max), dtype=torch.int32, device=dev)
    err = torch.empty(B, dtype=torch.int32, device=dev)
    out = torch.empty_like(base["q"])
    acc_len = torch.empty(B, dtype=torch.int32, device=dev)
    path = torch.empty((B, n_max), dtype=torch.int32, device=dev)
    bonus = torch.empty(B, dtype=torch.int32, device=dev)
    toks = torch.empty((B, n_max), dtype=torch.int32, device=dev)
    plen_out = torch.empty_like(plen)
    a0 = tv.attn_args(base["q"], base["k_new"], base["v_new"], base["k_cache"], base["v_cache"],
                      plen, n_nodes, anc, depth, err, out, w.rope_theta,
                      block_table=base["bt"] if paged else None)
    ws_bytes = tv.tree_attention_workspace_size(a0)
    workspace = tv.new_workspace(ws_bytes, dev)

    stream = torch.cuda.current_stream()
    # The timed loop calls the C ABI with arguments built once per input
    # copy (as a native caller would); the binding's checks run here, once.
    lib = tv._lib.load()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def P(t):
        return ctypes.c_void_p(t.data_ptr())

    calls = []
    for s in sets:
        a = tv.attn_args(s["q"], s["k_new"], s["v_new"], s["k_cache"], s["v_cache"], plen, n_nodes,
                         anc, depth, err, out, w.rope_theta, workspace=workspace,
                         block_table=s["bt"] if paged else None)
        if paged:
            cm = (P(s["k_cache"]), P(s["v_cache"]), ctypes.byref(s["pk"]), B, w.Hkv, w.D, a.dtype, P(plen),
                  P(acc_len), P(path), n_max, P(plen_out), sp)
        else:
            cm = (P(s["k_cache"]), P(s["v_cache"]), B, w.Hkv, w.cap, w.D, a.dtype, P(plen), P(acc_len),
                  P(path), n_max, P(plen_out), sp)
        if paged:
            acm = (P(tok), P(tgt), P(parents), P(anc), P(depth), P(n_nodes), P(err), B, n_max, P(acc_len), P(path),
                   P(bonus), P(toks), P(s["k_cache"]), P(s["v_cache"]), ctypes.byref(s["pk"]), w.Hkv, w.D, a.dtype,
                   P(plen), P(plen_out), sp)
        else:
            acm = (P(tok), P(tgt), P(parents), P(anc), P(depth), P(n_nodes), P(err), B, n_max, P(acc_len), P(path),
                   P(bonus), P(toks), P(s["k_cache"]), P(s["v_cache"]), w.Hkv, w.cap, w.D, a.dtype, P(plen),
                   P(plen_out), sp)
        calls.append((a, cm, acm))
    commit_fn = lib.tv_commit_paged if paged else lib.tv_commit
    bt = (P(parents), P(n_nodes), B, n_max, P(anc), P(depth), P(err), sp)
    ac = (P(tok), P(tgt), P(parents), P(anc), P(depth), P(n_nodes), P(err), B, n_max, P(acc_len),
          P(path), P(bonus), P(toks), sp)

    # The step builds the tree inside the attention kernel
    # (tv_tree_attention_from_parents, or its paged form, writes anc, depth
    # and err for the accept), then accepts and commits in one launch;
    # --separate-tree makes it tv_build_tree + tv_tree_attention(_paged) +
    # tv_accept + tv_commit(_paged) for comparison.
    separate = args.separate_tree

    def attention(k: int) -> int:
        if paged:
            if separate:
                return lib.tv_tree_attention_paged(ctypes.byref(calls[k % copies][0]),
                                                   ctypes.byref(sets[k % copies]["pk"]), sp)
            return lib.tv_tree_attention_paged_from_parents(ctypes.byref(calls[k % copies][0]),
                                                            ctypes.byref(sets[k % copies]["pk"]), P(parents),
                                                            P(anc), P(depth), sp)
        if separate:
            return lib.tv_tree_attention(ctypes.byref(calls[k % copies][0]), sp)
        return lib.tv_tree_attention_from_parents(ctypes.byref(calls[k % copies][0]), P(parents), P(anc), P(depth),
                                                  sp)

    def accept_commit(k: int) -> int:
        if separate:
            return lib.tv_accept(*ac) | commit_fn(*calls[k % copies][1])
        if paged:
            return lib.tv_accept_commit_paged(*calls[k % copies][2])
        return lib.tv_accept_commit(*calls[k % copies][2])

    def step(k: int) -> None:
        st = lib.tv_build_tree(*bt) if separate else 0
        st |= attention(k)
        st |= accept_commit(k)
        if st:
            raise RuntimeError(f"library call failed with status {st}")

    warm_s = device_warmup(step, args.device_warmup)
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(args.warmup + k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    nodes = w.total_nodes
    value = nodes / ((t1 - t0) / args.steps)
    mean_accept = float(acc_len.float().mean().item())

    # The attention call in its step: K more steps, each with a pair of HIP
    # events on the launch stream around the call (outside the timed loop,
    # since each event pair adds a few microseconds to its step). Then the
    # call alone, K calls back to back between one pair of events (each call
    # re-appends the tree KV into its copy, so all do the same work).
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        st = lib.tv_build_tree(*bt) if separate else 0
        events[k][0].record(stream)
        st |= attention(k)
        events[k][1].record(stream)
        st |= accept_commit(k)
        if st:
            raise RuntimeError(f"library call failed with status {st}")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for k in range(args.steps):
        if attention(k):
            raise RuntimeError("tv_tree_attention failed")
    e1.record(stream)
    # the rest of the step alone, K calls back to back (the same moves each
    # time: the prefix lengths are not advanced)
    e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e2.record(stream)
    for k in range(args.steps):
        if accept_commit(k):
            raise RuntimeError("accept and commit failed")
    e3.record(stream)
    torch.cuda.synchronize()
    rest_b2b_s = e2.elapsed_time(e3) * 1e-3 / args.steps
    attn_ms = [a.elapsed_time(b) for a, b in events]
    attn_mean_s = float(np.mean(attn_ms)) * 1e-3
    attn_b2b_s = e0.elapsed_time(e1) * 1e-3 / args.steps
    ab = algorithmic_bytes(w)
    flops = algorithmic_flops(w)
    bound = roofline_bound(w, ab["total"], flops)
    if bound == "mfma":
        achieved, peak, unit = flops / attn_b2b_s / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = ab["total"] / attn_b2b_s / 1e9, HBM_PEAK_GBS, "GB/s"
    wname = f"{w.name}-paged" if paged else w.name
    traffic = load_traffic(wname)

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "tree-nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "device_warmup_s": round(warm_s, 3),
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wname, "batch": B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "tree_set_up": "tv_build_tree" if separate else "inside the attention kernel",
                   "head_dim": w.D, "prefix_len_mean": float(np.mean(w.prefix_len)),
                   "tree_nodes": int(w.n_nodes.max()), "input_copies_rotated": copies,
                   "seed": args.config if args.seed is None else args.seed},
        "roofline": {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak, "traffic": traffic,
                     "kernel": (("tv_tree_attention_paged" if paged else "tv_tree_attention") + " call" if separate
                                else ("tv_tree_attention_paged_from_parents" if paged else
                                      "tv_tree_attention_from_parents") + " call (the tree built in the kernel)") +
                               ": attn_bf16_kernel (key splits merged and tree appended inside the kernel on the "
                               "automatic plan; merge_bf16_kernel otherwise); its average duration from HIP "
                               "events on its stream around K calls back to back (attention_us_mean: an event pair "
                               "around the call inside each of K further steps, event overheads included)",
                     "algorithmic_bytes_per_launch": ab["total"],
                     "algorithmic_flops_per_launch": flops,
                     "hbm_frac": ab["total"] / attn_b2b_s / 1e9 / HBM_PEAK_GBS,
                     "mfma_frac": flops / attn_b2b_s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                     "hbm_frac_in_step": ab["total"] / attn_mean_s / 1e9 / HBM_PEAK_GBS,
                     "attention_us_mean": attn_mean_s * 1e6,
                     "attention_us_p10": float(np.percentile(attn_ms, 10)) * 1e3,
                     "attention_us_p90": float(np.percentile(attn_ms, 90)) * 1e3,
                     "attention_us_back_to_back": attn_b2b_s * 1e6},
        "attention_only_nodes_per_s": nodes / attn_mean_s,
        "accept_commit_us_back_to_back": rest_b2b_s * 1e6,
        "mean_accept_len": mean_accept,
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, paged=paged)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
