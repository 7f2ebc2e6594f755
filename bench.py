"""Benchmark of the Split-KV block-sparse draft attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c3]

One step = one pass of the whole hot path over one synthetic batch: realized
cost model + LPT plan (host, uploaded asynchronously), the partial forward of
every (sequence, KV head, chunk, draft-block range) item, the log-sum-exp merge
of each sequence, and the backward (Delta, key-owning main kernel, dQ
finalize).  Inputs are resident in HBM before the timed region.

Prints ONE JSON line.  ``value`` is unmasked fwd+bwd TFLOP/s: 4*d (forward) +
10*d (backward, including the QK^T recompute that reusing the LSE needs) FLOPs
per token-exact visible (query head, query row, key) triple, divided by the
wall time of the K timed steps.  Per-kernel times come from HIP events recorded
on the stream the kernels run on.  ``cpu_baseline`` times the float64 CPU oracle
on a bounded sample of the same workload on this host.
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

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

WORKLOAD_TEXT = {
    "c1": "tiny fp32: 1 seq, N=1024, 4 anchors U[64,N) x 16 tokens, 2/2 heads, d64, chunk 256, forward",
    "c2": "bf16 forward: 1 seq, N=16384, 32 anchors U[256,N) x 16, 32/8 heads, d128, chunk 1024",
    "c3": "bf16 fwd+bwd: 4 seqs, N_s U[16384,65536], 64 anchors U[256,N_s) x 16, 32/8 heads, d128, chunk 2048, LPT",
    "c4": "bf16 fwd+bwd: 1 seq, N=524288 as 64 chunks of 8192, 64 anchors U[0,N) x 16, 16/4 heads, d128",
    "c5": "bf16 fwd+bwd: 1 seq, N=262144, 128 anchors N*Beta(5,1) x 32, 16/16 heads, d128, chunk 4096",
}


def merge_bytes(path, d: int) -> int:
    """Algorithmic merge traffic: (m, lse) of every partial row, d fp32 of every
    visible partial row, and d output elements + one LSE per merged row."""
    import torch
    lse = path.lse_part[: int(path.part_base[-1])]
    visible = int(torch.isfinite(lse).sum().item())
    rows = int(path.part_base[-1])
    out_rows = path.problem.total_q * path.problem.hq
    out_el = 2 if path.skv_dtype == 1 else 4
    return rows * 8 + visible * d * 4 + out_rows * (d * out_el + 4)


def cpu_baseline(w, budget_s: float = 12.0):
    """Time the float64 oracle (forward + backward) on (sequence, KV head) slices
    of the workload until ~budget_s of CPU work; report unmasked TFLOP/s on the
    same 14*d-per-triple convention."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    c = w.cfg
    G = c.hq // c.hkv
    done, flops, t = [], 0.0, 0.0
    for s in range(c.n_seq):
        for g in range(c.hkv):
            t0 = time.perf_counter()
            if c.bwd and w.do is not None:
                oracle.bwd_workload(w, kv_heads=[g], seqs=[s])
                per_pair = 14 * c.d
            else:
                q = w.as_f64("q", rows=slice(int(w.q_off[s]), int(w.q_off[s + 1])))
                k = w.as_f64("k", rows=slice(int(w.kv_off[s]), int(w.kv_off[s + 1])))
                v = w.as_f64("v", rows=slice(int(w.kv_off[s]), int(w.kv_off[s + 1])))
                oracle.attention(q, k, v, w.seq_anchors(s), c.block, w.sm_scale, heads=range(g * G, (g + 1) * G))
                per_pair = 4 * c.d
            t += time.perf_counter() - t0
            e = np.minimum(w.seq_anchors(s).astype(np.int64) + c.block, int(w.n_ctx[s]))
            flops += float(e.sum()) * c.block * G * per_pair
            done.append((s, g))
            if t >= budget_s:
                break
        if t >= budget_s:
            break
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"float64 numpy oracle, {'fwd+bwd' if c.bwd else 'fwd'} of {len(done)} (sequence, KV head) "
                      f"slice(s) {done} of {c.name}, {t:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c3")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--policy", default="lpt", choices=["lpt", "static"])
    ap.add_argument("--bwd-granule", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-replan", action="store_true", help="plan once outside the timed region")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the multi-GPU Split-KV exchange is not "
              "part of this build.", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_sparse_draft_amd import SplitKVAttention, unmasked_pairs
    from synthetic import make

    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    w = make(args.config, seed=args.seed)
    c = w.cfg
    t_gen = time.perf_counter() - t_gen
    dt = torch.bfloat16 if w.is_bf16 else torch.float32

    def up(name):
        x = getattr(w, name)
        if w.is_bf16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    q, k, v = up("q"), up("k"), up("v")
    with_bwd = c.bwd and w.is_bf16
    do = up("do") if with_bwd else None
    path = SplitKVAttention(w.q_off, w.kv_off, w.anchors, c.block, c.hq, c.hkv, c.d, c.chunk, w.sm_scale, dt, dev,
                            policy=args.policy, bwd_granule=args.bwd_granule, with_bwd=with_bwd)
    if with_bwd:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    plan_s = []

    def step(i=None):
        if not args.no_replan:
            t0 = time.perf_counter()
            path.replan()
            plan_s.append(time.perf_counter() - t0)
        e = ev[i] if i is not None else None
        if e: e[0].record()
        path.partial_fwd(q, k, v)
        if e: e[1].record()
        path.merge()
        if e: e[2].record()
        if with_bwd:
            path.backward(q, k, v, do, dq, dk, dv)
        if e: e[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    plan_s.clear()
    t0 = time.perf_counter()
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    mrg_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    bwd_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    pairs = unmasked_pairs(w.q_off, w.kv_off, w.anchors, c.block, c.hq)
    fwd_flops = 4.0 * c.d * pairs
    bwd_flops = 10.0 * c.d * pairs if with_bwd else 0.0
    ms_per_step = wall / K * 1e3
    value = (fwd_flops + bwd_flops) / (wall / K) / 1e12
    mbytes = merge_bytes(path, c.d)
    n_merge = c.n_seq
    fwd_tf = fwd_flops / (fwd_ms * 1e-3) / 1e12
    bwd_tf = bwd_flops / (bwd_ms * 1e-3) / 1e12 if with_bwd else 0.0
    merge_gbs = mbytes / (mrg_ms * 1e-3) / 1e9
    if with_bwd:
        roof = {"bound": "mfma", "kernel": "sparse_attn_bwd (bwd_main_kernel; with its Delta and dQ-finalize launches)",
                "achieved": round(bwd_tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(bwd_tf / PEAK_BF16_TFLOPS, 4), "traffic": None}
    else:
        roof = {"bound": "mfma", "kernel": "sparse_attn_partial_fwd (fwd_bf16_kernel)", "achieved": round(fwd_tf, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
                "traffic": None}
    out = {
        "metric": "unmasked-FLOP TFLOP/s fwd+bwd, % of bf16 MFMA peak; merge GB/s",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.is_bf16 else "f32", "data": "synthetic",
        "config": {"workload": f"{c.name}: {WORKLOAD_TEXT.get(c.name, c.note)}", "seed": args.seed,
                   "n_ctx": [int(x) for x in w.n_ctx], "unmasked_pairs": int(pairs), "policy": args.policy,
                   "n_workers": path.n_workers, "fwd_granule_blocks": path.fwd_granule,
                   "bwd_granule_keys": path.bwd_granule if with_bwd else None},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd": {"ms": round(fwd_ms, 4), "tflops": round(fwd_tf, 2), "frac": round(fwd_tf / PEAK_BF16_TFLOPS, 4)},
        "merge": {"ms": round(mrg_ms, 4), "launches": n_merge, "bytes": mbytes, "gbs": round(merge_gbs, 1),
                  "frac": round(merge_gbs / PEAK_HBM_GBS, 4)},
        "bwd": {"ms": round(bwd_ms, 4), "tflops": round(bwd_tf, 2), "frac": round(bwd_tf / PEAK_BF16_TFLOPS, 4)}
        if with_bwd else None,
        "plan": {"ms_per_step": round(1e3 * float(np.mean(plan_s)), 3) if plan_s else None,
                 "fwd_items": path.fwd_plan.n_items, "fwd_imbalance": round(path.fwd_plan.imbalance, 5),
                 "bwd_items": path.bwd_plan.n_items if with_bwd else None,
                 "bwd_imbalance": round(path.bwd_plan.imbalance, 5) if with_bwd else None},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
