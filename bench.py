"""Throughput of one draft-tree verification step on one MI355X.

A step is the whole verification path for one attention layer over one batch:
tv_build_tree -> tv_tree_attention -> tv_accept -> tv_commit, all through the
C ABI. The headline workload is the Llama-3-8B-shaped GQA batch (32 q / 8 kv
heads, head dim 128, batch 8, prefix 4096, 60-node EAGLE-2-style trees, bf16).

Inputs are generated once on the host, copied to HBM, and replicated into
enough independent copies that consecutive steps never find their prefix KV in
the 256 MB Infinity Cache; step k uses copy k mod R. Each step re-appends the
tree KV into its copy and commits from the same starting prefix length, so all
steps do identical work.

Prints one JSON line. `value` = tree nodes verified per second over the timed
steps (wall clock between two device synchronisations). `roofline` reports the
attention call (its three kernels): algorithmic HBM bytes per call divided by
its mean duration, measured with HIP events on the launch stream; `traffic` is
the measured HBM bytes per call from profiles/ when it matches the source.
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

METRIC = "tree-verify nodes/sec and achieved HBM GB/s (% of peak), 8B-shaped GQA batch 8"
HBM_PEAK_GBS = 8000.0
INFINITY_CACHE_BYTES = 256 << 20
KERNEL_SOURCES = ["tv_attn_bf16.hip", "tv_attn_f32.hip", "tv_device.h"]


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


def cpu_baseline(w, budget_s: float = 12.0) -> dict:
    """The oracle, as it is, on whole sequences of the same workload until
    about budget_s seconds of CPU work; one BLAS thread."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    nodes = 0
    done = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        for b in range(w.B):
            oracle.verify_step(w.oracle_inputs(b))
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
                      f"+ ancestors, accept, commit), numpy float64, 1 BLAS thread of "
                      f"{len(os.sched_getaffinity(0))} available ({cpu}), {dt:.1f} s"}


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3, help="workload 1..5 (3 = headline)")
    ap.add_argument("--copies", type=int, default=0, help="input copies rotated per step (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=None)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the verification "
              "path has no multi-GPU form in this library; see DESIGN.md for how it would shard)",
              file=sys.stderr)
        sys.exit(2)

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
                      plen, n_nodes, anc, depth, err, out, w.rope_theta)
    ws_bytes = tv.tree_attention_workspace_size(a0)
    workspace = tv.new_workspace(ws_bytes, dev)

    stream = torch.cuda.current_stream()

    def step(k: int, ev=None):
        s = sets[k % copies]
        tv.build_tree(parents, n_nodes, anc, depth, err)
        if ev is not None:
            ev[0].record(stream)
        tv.tree_attention(s["q"], s["k_new"], s["v_new"], s["k_cache"], s["v_cache"], plen, n_nodes,
                          anc, depth, err, rope_theta=w.rope_theta, out=out, workspace=workspace)
        if ev is not None:
            ev[1].record(stream)
        tv.accept(tok, tgt, parents, anc, depth, n_nodes, err, acc_len, path, bonus, toks)
        tv.commit(s["k_cache"], s["v_cache"], plen, acc_len, path, plen_out)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(args.warmup + k, events[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    nodes = w.total_nodes
    value = nodes / ((t1 - t0) / args.steps)
    attn_ms = [e0.elapsed_time(e1) for e0, e1 in events]
    attn_mean_s = float(np.mean(attn_ms)) * 1e-3
    ab = algorithmic_bytes(w)
    achieved = ab["total"] / attn_mean_s / 1e9
    traffic = load_traffic(w.name)
    mean_accept = float(acc_len.float().mean().item())

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "tree-nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.D, "prefix_len_mean": float(np.mean(w.prefix_len)),
                   "tree_nodes": int(w.n_nodes.max()), "input_copies_rotated": copies,
                   "seed": args.config if args.seed is None else args.seed},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "tv_tree_attention call: attn_bf16_kernel + merge_bf16_kernel (split merge "
                               "and tree append), HIP events around the call on its stream",
                     "algorithmic_bytes_per_launch": ab["total"],
                     "attention_us_mean": attn_mean_s * 1e6,
                     "attention_us_p10": float(np.percentile(attn_ms, 10)) * 1e3,
                     "attention_us_p90": float(np.percentile(attn_ms, 90)) * 1e3},
        "attention_only_nodes_per_s": nodes / attn_mean_s,
        "mean_accept_len": mean_accept,
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
