"""Benchmark of the Split-KV block-sparse draft attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c3]

One step = one pass of the whole hot path over one synthetic batch: realized
cost model + LPT plan (host; copied asynchronously on the stream ahead of the
forward), the partial forward of every chunk-run item (sequence, KV head, run
of chunks, draft-block range), the log-sum-exp merge of every sequence in one
launch, and the backward (Delta, key-owning dK/dV kernel, query-owning dQ
kernel, dQ finalize).  Inputs are resident in HBM before the timed region.

Prints ONE JSON line.  ``value`` is unmasked fwd+bwd TFLOP/s: 4*d (forward) +
10*d (backward, including the QK^T recompute that reusing the LSE needs) FLOPs
per token-exact visible (query head, query row, key) triple, divided by the
wall time of the K timed steps, which record no events.  A second pass of K
steps is instrumented: HIP events on the stream time the phases, and the
library brackets each of its own launches with events on the stream it runs on
(skv_timing_*), which gives the per-kernel durations behind ``roofline``; each
workgroup's busy time (s_memrealtime) gives the measured balance in ``plan``.
``cpu_baseline`` times the float64 CPU oracle on a bounded sample of the same
workload on this host, with BLAS on every core the process may use, and the
oracle's LPT on the step's item sets.

    --plan-compare     also run the workload under static and LPT plans, with
                       and without tail stealing, and report cost-model and
                       measured per-workgroup imbalance and step times
    --copy-calibration MB   run one device copy of MB MiB before the steps
                       (reference dispatch for HBM byte counters)
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


def cpu_baseline(w, budget_s: float = 12.0, mask: str = "prefix", lpt_costs=None, n_workers: int = 256):
    """Time the float64 oracle (forward + backward) on (sequence, KV head) slices
    of the workload until ~budget_s of CPU work; report unmasked TFLOP/s on the
    same 14*d-per-triple convention.  BLAS runs on every core this process may
    use (``cores``).  ``lpt_costs``: item costs (name -> int64 array) on which
    the oracle's LPT is timed as well, for comparison with the library's."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limits = threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover
        limits = None
    c = w.cfg
    G = c.hq // c.hkv
    done, flops, t = [], 0.0, 0.0
    for s in range(c.n_seq):
        for g in range(c.hkv):
            t0 = time.perf_counter()
            if mask == "own_block":
                qs = slice(int(w.q_off[s]), int(w.q_off[s + 1]))
                ks = slice(int(w.kv_off[s]), int(w.kv_off[s + 1]))
                args = [w.as_f64(n, rows=qs if n in ("q", "k_own", "v_own") else ks)
                        for n in ("q", "k", "v", "k_own", "v_own")]
                if c.bwd and w.do is not None:
                    oracle.attention_own_bwd(*args, w.seq_anchors(s), c.block, w.sm_scale,
                                             w.as_f64("do", rows=qs), kv_heads=[g])
                    per_pair = 14 * c.d
                else:
                    oracle.attention_own(*args, w.seq_anchors(s), c.block, w.sm_scale,
                                         heads=range(g * G, (g + 1) * G))
                    per_pair = 4 * c.d
            elif c.bwd and w.do is not None:
                oracle.bwd_workload(w, kv_heads=[g], seqs=[s])
                per_pair = 14 * c.d
            else:
                q = w.as_f64("q", rows=slice(int(w.q_off[s]), int(w.q_off[s + 1])))
                k = w.as_f64("k", rows=slice(int(w.kv_off[s]), int(w.kv_off[s + 1])))
                v = w.as_f64("v", rows=slice(int(w.kv_off[s]), int(w.kv_off[s + 1])))
                oracle.attention(q, k, v, w.seq_anchors(s), c.block, w.sm_scale, heads=range(g * G, (g + 1) * G))
                per_pair = 4 * c.d
            t += time.perf_counter() - t0
            if mask == "own_block":
                e = np.minimum(w.seq_anchors(s).astype(np.int64), int(w.n_ctx[s])) + c.block
            else:
                e = np.minimum(w.seq_anchors(s).astype(np.int64) + c.block, int(w.n_ctx[s]))
            flops += float(e.sum()) * c.block * G * per_pair
            done.append((s, g))
            if t >= budget_s:
                break
        if t >= budget_s:
            break
    out = {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
           "sample": f"float64 numpy oracle, {'fwd+bwd' if c.bwd else 'fwd'} of {len(done)} (sequence, KV head) "
                     f"slice(s) {done} of {c.name}, {t:.1f} s, BLAS limited to {cores} threads"}
    if lpt_costs:
        out["lpt_ms"] = {}
        for name, cost in lpt_costs.items():
            t0 = time.perf_counter()
            oracle.lpt(cost, n_workers)
            out["lpt_ms"][name] = round(1e3 * (time.perf_counter() - t0), 3)
    if limits is not None:
        limits.restore_original_limits()
    return out


# Algorithmic FLOPs per token-exact visible (q head, row, key) triple, in units
# of head_dim, that each kernel contributes to the 4d + 10d count: the forward
# does QK^T and PV; the key-owner backward recomputes QK^T and forms dP, dV and
# dK; the query-owner backward forms dQ (it also recomputes QK^T and dP, 4d
# more per triple, which the count leaves out).
KERNEL_FLOPS_D = {"partial_fwd_bf16": 4, "partial_fwd_f32": 4, "bwd_kv": 8, "bwd_dq": 2}
KERNEL_EXEC_FLOPS_D = {"partial_fwd_bf16": 4, "partial_fwd_f32": 4, "bwd_kv": 8, "bwd_dq": 6}
# Sources whose text defines each kernel's device code (the kernel file and
# the device-side helpers it includes).
# Files a kernel's machine code depends on: its source, the shared device
# headers and the build script (compile flags), relative to the package.
KERNEL_SOURCES = {
    "bwd_kv": ["csrc/bwd_bf16.hip", "csrc/device.h", "csrc/fastdiv.h", "build.py"],
    "bwd_dq": ["csrc/bwd_bf16.hip", "csrc/device.h", "csrc/fastdiv.h", "build.py"],
    "partial_fwd_bf16": ["csrc/fwd_bf16.hip", "csrc/device.h", "csrc/fastdiv.h", "build.py"],
}


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(ROOT, "block_sparse_draft_amd", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def hbm_traffic(kernel: str, config: str):
    """HBM bytes per launch of `kernel` on `config` from the committed counter
    summary (rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by a copy kernel of
    known size), or None when there is none or the kernel's sources or build
    flags have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{config}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith((" ", "#")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != kernel_source_hash(kernel):
        return None
    try:
        return int(float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def kernel_alg_bytes(w, path, merge_b: int) -> dict:
    """Algorithmic HBM bytes per launch: what a kernel must move at least, with
    every input read once and every output written once.
      partial_fwd_bf16: K and V rows some draft block sees (keys below the
        sequence's largest prefix end), per KV head; every Q row; d + 2 fp32
        per partial row written.
      bwd_kv: those K and V rows read, every dK and dV row written; the packed
        bf16 Q and dO copies and 12 bytes (LSE, Delta, prefix end) per (row,
        query head) read.
      bwd_dq: K and V rows seen read; packed Q and dO and 12 bytes per (row,
        query head) read; d + 1 words per dQ partial row written.
      lse_merge: see merge_bytes."""
    c = w.cfg
    if not w.is_bf16:
        return {"lse_merge": merge_b}
    el = 2
    seen = 0
    for s in range(c.n_seq):
        e = np.minimum(w.seq_anchors(s).astype(np.int64) + (c.block if path.mask == "prefix" else 0), int(w.n_ctx[s]))
        seen += int(e.max()) if len(e) else 0
    kv_row = c.hkv * c.d * el
    q_rows = int(w.q_off[-1]) * c.hq
    out = {"lse_merge": merge_b}
    import torch
    part_rows = int(torch.isfinite(path.lse_part).sum().item())
    out["partial_fwd_bf16"] = 2 * seen * kv_row + q_rows * c.d * el + part_rows * (c.d + 2) * 4
    if path.bwd_plan is not None:
        total_kv = int(w.kv_off[-1])
        q_side = q_rows * (2 * c.d * el + 12)
        out["bwd_kv"] = 2 * seen * kv_row + 2 * total_kv * kv_row + q_side
        out["bwd_dq"] = 2 * seen * kv_row + q_side + part_rows * (c.d + 1) * 4
    return out


def run_steps(path, q, k, v, do, grads, K: int, warmup: int, replan: bool, with_bwd: bool, own=None,
              instrument: bool = True):
    """Warm up, then time K steps.  Returns wall seconds, the host planning
    seconds of each timed step, and (``instrument``) per-phase event ms (lists)
    and the library's per-kernel event times.  Without ``instrument`` the timed
    steps record no events at all (the headline number); with it, the library's
    event pool is filled during the warm-up, so the timed steps create none."""
    import torch
    from block_sparse_draft_amd import binding as Bd
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)] if instrument else None
    plan_s = []

    def step(e=None):
        if replan:
            path.replan()
            plan_s.append(path.plan_s)
        if e: e[0].record()
        if own is None:
            path.partial_fwd(q, k, v)
        else:
            path.partial_fwd(q, k, v, k_own=own[0], v_own=own[1])
        if e: e[1].record()
        path.merge()
        if e: e[2].record()
        if with_bwd:
            path.backward(q, k, v, do, *grads, own=own)
        if e: e[3].record()

    if instrument:
        Bd.timing_enable(True)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    Bd.timing_collect()   # the warm-up's launches (the events return to the pool)
    plan_s.clear()
    t0 = time.perf_counter()
    for i in range(K):
        step(ev[i] if instrument else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if not instrument:
        return wall, plan_s, None, None
    Bd.timing_enable(False)
    kt = Bd.timing_collect()
    ph = {"fwd": [e[0].elapsed_time(e[1]) for e in ev], "merge": [e[1].elapsed_time(e[2]) for e in ev],
          "bwd": [e[2].elapsed_time(e[3]) for e in ev]}
    return wall, plan_s, ph, kt


def imbalance(x) -> float:
    x = np.asarray(x, dtype=np.float64)
    m = x.mean()
    return float(x.max() / m - 1.0) if m > 0 else 0.0


def plan_compare(w, q, k, v, do, grads, dt, dev, K: int, warmup: int, bwd_granule: int, with_bwd: bool):
    """Static token-count vs cost-aware LPT plans, each with and without tail
    stealing: cost-model imbalance of the plan, measured imbalance of the
    per-workgroup busy times (s_memrealtime) and the step times."""
    import torch
    from block_sparse_draft_amd import SplitKVAttention
    c = w.cfg
    out = []
    # one chunk per forward item in the four static/LPT rows; the last row adds chunk runs
    for policy, steal, runs in (("static", False, None), ("static", True, None), ("lpt", False, None),
                                ("lpt", True, None), ("lpt", True, 4.0)):
        path = SplitKVAttention(w.q_off, w.kv_off, w.anchors, c.block, c.hq, c.hkv, c.d, c.chunk, w.sm_scale,
                                dt, dev, policy=policy, bwd_granule=bwd_granule, with_bwd=with_bwd,
                                steal=steal, ticks=True, fwd_runs_per_worker=runs)
        wall, _, ph, kt = run_steps(path, q, k, v, do, grads, K, warmup, False, with_bwd)
        rec = {"policy": policy, "steal": steal, "fwd_runs_per_worker": runs,
               "ms_per_step": round(wall / K * 1e3, 4),
               "fwd_ms": round(float(np.mean(ph["fwd"])), 4),
               "bwd_ms": round(float(np.mean(ph["bwd"])), 4) if with_bwd else None,
               "fwd_cost_imbalance": round(path.fwd_plan.imbalance, 5),
               "fwd_measured_imbalance": round(imbalance(path.fwd_plan.ticks.cpu().numpy()), 5)}
        if with_bwd:
            rec.update({"bwd_kv_cost_imbalance": round(path.bwd_plan.imbalance, 5),
                        "bwd_kv_measured_imbalance": round(imbalance(path.bwd_plan.ticks.cpu().numpy()), 5),
                        "bwd_dq_measured_imbalance": round(imbalance(path.dq_plan.ticks.cpu().numpy()), 5)})
        out.append(rec)
        del path
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c3")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--policy", default="lpt", choices=["lpt", "static"])
    ap.add_argument("--bwd-granule", type=int, default=256)
    ap.add_argument("--fwd-granule", type=int, default=0,
                    help="draft blocks per forward item (0: the library's default, 256 packed rows)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-replan", action="store_true", help="plan once outside the timed region")
    ap.add_argument("--no-steal", action="store_true", help="workgroups run only their own plan lists")
    ap.add_argument("--plan-compare", action="store_true")
    ap.add_argument("--mask", default="prefix", choices=["prefix", "own_block"],
                    help="own_block: context prefix [0, a_b) plus each block's own keys (seeded k_own, v_own)")
    ap.add_argument("--runs-per-worker", type=float, default=4.0,
                    help="forward items cover runs of consecutive chunks of the same rows (one partial per run), "
                         "about this many runs per workgroup; 0 = one chunk per item (LPT only)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the multi-GPU Split-KV exchange is not "
              "part of this build.", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_sparse_draft_amd import SplitKVAttention, unmasked_pairs
    from synthetic import add_own_block, make

    dev = torch.device("cuda:0")
    w = make(args.config, seed=args.seed)
    if args.mask == "own_block":
        add_own_block(w)
    c = w.cfg
    dt = torch.bfloat16 if w.is_bf16 else torch.float32

    def up(name):
        x = getattr(w, name)
        if w.is_bf16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    q, k, v = up("q"), up("k"), up("v")
    with_bwd = c.bwd and w.is_bf16
    do = up("do") if with_bwd else None
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)) if with_bwd else None
    own = None
    if args.mask == "own_block":
        ko, vo = up("k_own"), up("v_own")
        own = (ko, vo, torch.empty_like(ko), torch.empty_like(vo)) if with_bwd else (ko, vo, None, None)

    if args.copy_calibration > 0:
        # one plain device-to-device copy of known size, for scaling HBM byte counters
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    path = SplitKVAttention(w.q_off, w.kv_off, w.anchors, c.block, c.hq, c.hkv, c.d, c.chunk, w.sm_scale, dt, dev,
                            policy=args.policy, bwd_granule=args.bwd_granule, with_bwd=with_bwd,
                            fwd_granule=args.fwd_granule or None,
                            steal=not args.no_steal, fwd_runs_per_worker=args.runs_per_worker or None,
                            mask=args.mask, ticks=True)
    K = args.steps
    # headline: no events of any kind inside the timed steps
    wall, plan_s, _, _ = run_steps(path, q, k, v, do, grads, K, args.warmup, not args.no_replan, with_bwd, own,
                                   instrument=False)
    # per-phase and per-kernel event times, in a second pass of the same steps
    wall_i, _, ph, kt = run_steps(path, q, k, v, do, grads, K, max(1, min(args.warmup, 3)), not args.no_replan,
                                  with_bwd, own, instrument=True)

    fwd_ms = float(np.mean(ph["fwd"]))
    mrg_ms = float(np.mean(ph["merge"]))
    bwd_ms = float(np.mean(ph["bwd"]))
    pairs = unmasked_pairs(w.q_off, w.kv_off, w.anchors, c.block, c.hq, mask=args.mask)
    # triples the context kernels handle (the own-block keys go to own_fwd / own_bwd)
    ctx_pairs = pairs - (int(w.q_off[-1]) * c.hq * c.block if args.mask == "own_block" else 0)
    fwd_flops = 4.0 * c.d * pairs
    bwd_flops = 10.0 * c.d * pairs if with_bwd else 0.0
    ms_per_step = wall / K * 1e3
    value = (fwd_flops + bwd_flops) / (wall / K) / 1e12
    mbytes = merge_bytes(path, c.d)
    fwd_tf = fwd_flops / (fwd_ms * 1e-3) / 1e12
    bwd_tf = bwd_flops / (bwd_ms * 1e-3) / 1e12 if with_bwd else 0.0
    merge_gbs = mbytes / (mrg_ms * 1e-3) / 1e9
    alg_bytes = kernel_alg_bytes(w, path, mbytes)

    kernels = {}
    for name, (n_launch, tot) in kt.items():
        avg = tot / max(n_launch, 1)
        rec = {"launches_per_step": n_launch / K, "avg_ms": round(avg, 4)}
        if name in KERNEL_FLOPS_D:
            alg = KERNEL_FLOPS_D[name] * c.d * ctx_pairs
            rec["alg_tflops"] = round(alg / (avg * 1e-3) / 1e12, 2)
            rec["exec_tflops"] = round(KERNEL_EXEC_FLOPS_D[name] * c.d * ctx_pairs / (avg * 1e-3) / 1e12, 2)
        if name in alg_bytes:
            rec["alg_bytes"] = alg_bytes[name]
            rec["alg_gbs"] = round(alg_bytes[name] / (avg * 1e-3) / 1e9, 1)
        kernels[name] = rec
    compute = {n: kt[n][1] for n in KERNEL_FLOPS_D if n in kt}
    dom = max(compute, key=compute.get)
    dom_avg = kt[dom][1] / kt[dom][0]
    dom_flops = KERNEL_FLOPS_D[dom] * c.d * ctx_pairs
    achieved = dom_flops / (dom_avg * 1e-3) / 1e12
    traffic = hbm_traffic(dom, c.name) if args.mask == "prefix" else None
    roof = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS
            if w.is_bf16 else 157.3, "unit": "TFLOP/s",
            "frac": round(achieved / (PEAK_BF16_TFLOPS if w.is_bf16 else 157.3), 4),
            "traffic": traffic, "alg_bytes": alg_bytes.get(dom),
            "traffic_over_alg_bytes": round(traffic / alg_bytes[dom], 3) if traffic and alg_bytes.get(dom) else None,
            "alg_flops_per_launch": dom_flops, "avg_launch_ms": round(dom_avg, 4)}

    # measured balance of the last instrumented step: per-workgroup busy time
    # (s_memrealtime, 100 MHz) against the kernel's event-timed duration
    measured = {}
    for name, plan in (("partial_fwd_bf16", path.fwd_plan), ("bwd_kv", path.bwd_plan), ("bwd_dq", path.dq_plan)):
        if plan is None or plan.ticks is None or name not in kt:
            continue
        us = plan.ticks.cpu().numpy().astype(np.float64) / 100.0
        measured[name] = {"imbalance": round(imbalance(us), 5), "mean_busy_us": round(float(us.mean()), 1),
                          "max_busy_us": round(float(us.max()), 1),
                          "kernel_us": round(1e3 * kt[name][1] / kt[name][0], 1)}
    # planner alone: lpt_plan on the step's item sets (the oracle's LPT on the
    # same costs is timed in cpu_baseline)
    lpt_sets = {"fwd_runs": path.fwd_plan.table[1]}
    if with_bwd:
        lpt_sets["bwd_items"] = path.bwd_plan.table[1]
    lpt_us = {}
    from block_sparse_draft_amd import binding as Bd
    for name, cost in lpt_sets.items():
        reps = 20
        t0 = time.perf_counter()
        for _ in range(reps):
            Bd.lpt_plan(cost, path.n_workers)
        lpt_us[name] = {"items": int(len(cost)), "us": round(1e6 * (time.perf_counter() - t0) / reps, 1)}

    out = {
        "metric": "unmasked-FLOP TFLOP/s fwd+bwd, % of bf16 MFMA peak; merge GB/s",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.is_bf16 else "f32", "data": "synthetic",
        "config": {"workload": f"{c.name}: {WORKLOAD_TEXT.get(c.name, c.note)}", "seed": args.seed,
                   "n_ctx": [int(x) for x in w.n_ctx], "unmasked_pairs": int(pairs), "policy": args.policy,
                   "steal": not args.no_steal, "n_workers": path.n_workers, "fwd_granule_blocks": path.fwd_granule,
                   "bwd_granule_keys": path.bwd_granule if with_bwd else None,
                   "fwd_runs_per_worker": path.fwd_runs_per_worker, "mask": args.mask},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        # the same steps counted at 12*d per triple (backward without the QK^T recompute)
        "value_12d": round(12.0 * c.d * pairs / (wall / K) / 1e12, 3) if with_bwd else None,
        "instrumented_ms_per_step": round(wall_i / K * 1e3, 4),
        "fwd": {"ms": round(fwd_ms, 4), "tflops": round(fwd_tf, 2), "frac": round(fwd_tf / PEAK_BF16_TFLOPS, 4)},
        "merge": {"ms": round(mrg_ms, 4), "launches": 1, "bytes": mbytes, "gbs": round(merge_gbs, 1),
                  "frac": round(merge_gbs / PEAK_HBM_GBS, 4)},
        "bwd": {"ms": round(bwd_ms, 4), "tflops": round(bwd_tf, 2), "frac": round(bwd_tf / PEAK_BF16_TFLOPS, 4)}
        if with_bwd else None,
        "kernels": kernels,
        "plan": {"host_ms_per_step": round(1e3 * float(np.mean(plan_s)), 3) if plan_s else None,
                 "lpt_plan": lpt_us,
                 "fwd_items": path.fwd_plan.n_items, "fwd_items_planned": path.fwd_plan.n_planned,
                 "fwd_partial_rows_written": int(torch.isfinite(path.lse_part).sum().item()),
                 "fwd_runs_per_worker_used": path.fwd_plan.runs_used,
                 "fwd_imbalance": round(path.fwd_plan.imbalance, 5),
                 "bwd_items": path.bwd_plan.n_items if with_bwd else None,
                 "bwd_imbalance": round(path.bwd_plan.imbalance, 5) if with_bwd else None,
                 "measured": measured},
        "roofline": roof,
    }
    del path
    torch.cuda.empty_cache()
    if args.plan_compare:
        out["plan_compare"] = plan_compare(w, q, k, v, do, grads, dt, dev, max(3, K // 2), 2, args.bwd_granule,
                                           with_bwd)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, mask=args.mask, lpt_costs=lpt_sets, n_workers=out["config"]["n_workers"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
