#!/usr/bin/env python3
"""Benchmark of the batched, rank-specialized LoRA-delta apply on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

A step is one pass of the whole hot path over one batch: token grouping,
shrink and expand, i.e. one lora_apply_batched call with adapter ids (one
fused kernel for decode-sized calls, else two: the shrink, which also groups
the tokens, and the expand), on inputs already resident in HBM.  Steps rotate through independent copies of
(store, x, y) whose total size exceeds the 256 MB last-level cache, so every
step reads its factors and activations from HBM (cold-HBM timing).

Prints ONE JSON line: tokens/s of the rank-specialized apply, achieved
algorithmic HBM GB/s and fraction of the 8 TB/s peak, the roofline of the
dominant kernel (HIP events on the launch stream), the same kernels on
rank-padded stores, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LoRA-delta tokens/s and achieved HBM GB/s (% of ~8 TB/s peak), 1 MI355X"
PEAK_GBPS = 8000.0
COLD_BYTES = 2.0e9  # rotation set size: well past the 256 MB Infinity Cache
# Sources each measured kernel family is built from: a counter record is used
# only while the sources of its family are unchanged.
# Sources of each kernel family: a traffic record holds only while its own
# family's sources are unchanged.
APPLY_SOURCES = ["shrink.hip", "expand.hip", "tile_ops.h", "device_common.h", "plan.h"]
DECODE_SOURCES = ["decode.hip", "device_common.h", "plan.h"]
KERNEL_SOURCES = APPLY_SOURCES + ["decode.hip"]
JD_SOURCES = APPLY_SOURCES + ["jd.hip"]
RSVD_SOURCES = ["rsvd.hip", "device_common.h", "plan.h"]


def sources_of(kernel: str):
    if kernel == "decode_apply":
        return DECODE_SOURCES
    if kernel.startswith("rsvd_"):
        return RSVD_SOURCES
    if kernel.startswith("jd_"):
        return JD_SOURCES
    return APPLY_SOURCES
PEAK_FP64_TFLOPS = 78.6  # 256 CUs x 4 SIMDs x 16 lanes x 2 (FMA) x 2.4 GHz

WORKLOAD_NAMES = {
    "1": "tiny-fp32: d_in=d_out=256 f32, 4 adapters ranks {1,2,3,4}, T=16",
    "2": "decode-uniform: d_in=d_out=4096 bf16, 64 adapters rank 4 (orig 16), T=256 uniform ids",
    "3": "decode-spectral: d_in=d_out=3584 bf16, 512 adapters ranks max(6,ceil(64e)) e~Beta(2,5), "
         "T=2048 Zipf(1.1) ids",
    "4": "prefill: 4096->14336 bf16, 32 adapters ranks in {8,12,16,24,32}, T=8192 in 32x256 segments",
    "jd-full": "shared-basis decode (JD-Full): d_in=d_out=4096 bf16, 1024 adapters in 32 clusters of rank 16, "
               "full 16x16 Sigma per adapter, T=2048 Zipf(1.1) ids",
    "jd-diag": "shared-basis decode (JD-Diag): d_in=d_out=4096 bf16, 1024 adapters in 32 clusters of rank 16, "
               "diagonal Sigma per adapter, T=2048 Zipf(1.1) ids",
    "rsvd-q": "retained-factor construction (r-SVD through tall-skinny QR): 1024 adapters of rank 64 of one "
              "3584->3584 projection, bf16, spectral-budget ranks (floor 4, budget 6 per adapter)",
    "ranks-fleet": "retained-rank allocation on the host: 1024 adapters x 196 modules (200704 units) of "
                   "original rank 64, uniform (ratio 1/12, floor 4) and spectral at the same budget",
    "5U": "fleet decode step: 28 layers x 7 projections (3584/512/18944 dims) bf16, 1024 adapters rank 6 "
          "(orig 64), T=4096 Zipf(1.1) ids, one grouping reused by 196 applies (q/k/v and gate/up concurrent)",
    "5S": "fleet decode step: 28 layers x 7 projections (3584/512/18944 dims) bf16, 1024 adapters ranks "
          "4..16 per module, T=4096 Zipf(1.1) ids, one grouping reused by 196 applies (q/k/v and gate/up concurrent)",
}


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default="2", choices=sorted(WORKLOAD_NAMES))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-padded", action="store_true")
    p.add_argument("--no-multi", action="store_true", help="fleet: skip the multi-slice (q/k/v, gate/up) step")
    p.add_argument("--streams", type=int, default=3,
                   help="fleet: run the modules of one stage (q/k/v; gate/up) on up to this many streams")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--warm", action="store_true", help="no rotation (cache-resident timing)")
    p.add_argument("--no-graph", action="store_true", help="time eager launches only (counter runs)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="first run one elementwise copy of 256 MiB (reads and writes 256 MiB), the "
                        "reference that scales the HBM byte counters")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="no GPU work: read two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of "
                        "this script with --calibrate-copy and record HBM bytes per launch of each "
                        "kernel in profiles/traffic.json")
    return p.parse_args()


def kernel_source_digest(sources=None) -> str:
    h = hashlib.sha256()
    for name in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, "rank_specialized_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------ bytes
def algorithmic_bytes(ids: np.ndarray, ranks: np.ndarray, n: int, d_in: int, d_out: int, e: int):
    """Bytes the method itself must move per call (nothing for untouched
    adapters or padding): the ids, each used adapter's factors once, each
    token's x row once, each token's y row read and written once, and the
    float32 intermediate h (sum of the tokens' ranks) written once and read
    once.  The shrink kernel owns the ids, A, x and the h write; the expand
    the h read, B and y."""
    valid = (ids >= 0) & (ids < n)
    tok_r = np.where(valid, ranks[np.clip(ids, 0, n - 1)], 0)
    active = valid & (tok_r > 0)
    touched = np.unique(ids[active])
    R_touched = int(ranks[touched].sum())
    Tv = int(active.sum())
    sum_r = int(tok_r.sum())
    T = len(ids)
    shrink = 4 * T + R_touched * d_in * e + Tv * d_in * e + 4 * sum_r
    expand = R_touched * d_out * e + 2 * Tv * d_out * e + 4 * sum_r
    return {"shrink": shrink, "expand": expand, "total": shrink + expand,
            "flops": 2 * sum_r * (d_in + d_out), "touched": int(len(touched)), "R_touched": R_touched}


# ------------------------------------------------------------------ workload
def build_workload(key: str):
    from workloads import make_config
    return make_config(key, with_y0=True)


class Copy:
    def __init__(self, store, x, y):
        self.store, self.x, self.y = store, x, y


def make_copies(rs, torch, wl, dev, pad_to: int, cold: bool):
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    A = [torch.from_numpy(a).to(dev).to(dt) for a in wl.module.A]
    B = [torch.from_numpy(b).to(dev).to(dt) for b in wl.module.B]
    store = rs.lora_pack_retained(A, B, wl.module.scales, pad_to=pad_to)
    del A, B
    x = torch.from_numpy(wl.x).to(dev).to(dt)
    y = torch.from_numpy(wl.y0).to(dev).to(dt)
    per_copy = store.A_pack.numel() + store.B_pack.numel() + x.numel() * x.element_size() \
        + y.numel() * y.element_size()
    n_copies = 1 if not cold else int(min(512, max(1, math.ceil(COLD_BYTES / per_copy))))
    copies = [Copy(store, x, y)]
    for _ in range(n_copies - 1):
        copies.append(Copy(store.clone(), x.clone(), y.clone()))
    return copies, per_copy


def _lora_step(rs, ids, ws):
    return lambda c: rs.lora_apply_batched(c.store, c.x, c.y, ids=ids, ws=ws)


def time_apply(rs, torch, copies, ids, ws, steps, warmup, step=None):
    """Events bracket exactly `steps` eager calls; returns ms per call."""
    step = step or _lora_step(rs, ids, ws)
    for k in range(warmup):
        step(copies[k % len(copies)])
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for k in range(steps):
        step(copies[(warmup + k) % len(copies)])
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def time_apply_graph(rs, torch, copies, ids, ws, steps, warmup, step=None):
    """The same `steps` calls captured once in a HIP graph (a decode loop's
    launches replayed without host work per kernel); events bracket one
    replay of all of them.  Returns ms per call."""
    step = step or _lora_step(rs, ids, ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for k in range(max(1, warmup)):
            step(copies[k % len(copies)])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(steps):
            step(copies[(warmup + k) % len(copies)])
    g.replay()  # untimed warm replay
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del g
    return e0.elapsed_time(e1) / steps, wall


def time_kernels(rs, torch, copies, ids, ws, steps, warmup, graph=True):
    """Average duration of each of the apply's two kernels, measured alone:
    the same rotation of calls with only that kernel (lora_apply_batched_phases),
    captured in a HIP graph; HIP events on the launch stream bracket one
    replay of `steps` launches.  The expand replays read the plan and partial
    sums the last shrink left in the workspace."""
    out = {}
    for name, phase in (("shrink", 1), ("expand", 2)):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for k in range(max(1, warmup)):
                c = copies[k % len(copies)]
                rs.lora_apply_batched(c.store, c.x, c.y, ids=ids, ws=ws)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        def run():
            for k in range(steps):
                c = copies[k % len(copies)]
                rs.lora_apply_batched_phases(c.store, c.x, c.y, phase, ids=ids, ws=ws)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        if graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run()
            g.replay()
            torch.cuda.synchronize()
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            del g
        else:
            e0.record()
            run()
            e1.record()
            torch.cuda.synchronize()
        out[name] = {"avg_us": 1e3 * e0.elapsed_time(e1) / steps, "launches": steps,
                     "timed_as": "one HIP-graph replay" if graph else "eager launches"}
    return out


def traffic_for(workload: str, kernel: str, sources=None):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current sources of that kernel family."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get(workload, {}).get(kernel)
    if not ent or ent.get("kernel_sources_sha") != kernel_source_digest(sources or sources_of(kernel)):
        return None
    return ent.get("hbm_bytes_per_launch")


CALIBRATE_BYTES = 256 << 20


def read_pmc(run_dir: str, counter: str):
    """{kernel name: [values per dispatch]} from a rocprofv3 counter run."""
    import csv
    import glob
    out = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return out


def summarize_pmc(key: str, fetch_dir: str, write_dir: str):
    """HBM bytes per launch of the shrink and expand kernels: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) averaged over the dispatches, each scaled by
    what the same counter reads for an elementwise copy of 256 MiB."""
    fetch, write = read_pmc(fetch_dir, "FETCH_SIZE"), read_pmc(write_dir, "WRITE_SIZE")

    def calib(d):
        vals = [v for k, vs in d.items() if "neg" in k for v in vs]
        if not vals:
            raise SystemExit("no calibration copy kernel in the counter run (use --calibrate-copy)")
        return max(vals) * 1024.0 / CALIBRATE_BYTES

    cf, cw = calib(fetch), calib(write)
    if key.startswith("rsvd-"):
        import rank_specialized_amd as rs
        from workloads import RSVD_CONFIGS
        c = RSVD_CONFIGS[key]
        keep = sum(rs.lora_ranks_uniform([c["r"]] * c["n"], 1.0 / 12.0, 4))  # the spectral budget, met exactly
        alg = rsvd_algorithmic(c["n"], c["r"], c["d_in"], c["d_out"], keep, 2)
        kernels = (("rsvd_gram", alg["gram_bytes"]), ("rsvd_write", alg["write_bytes"]))
    else:
        wl = build_workload(key)
        m = wl.module
        nb = algorithmic_bytes(wl.ids, m.ranks, m.n, m.d_in, m.d_out, 2 if wl.dtype == "bf16" else 4)
        kernels = (("shrink", nb["shrink"]), ("expand", nb["expand"]), ("decode_apply", nb["total"]))
    path = os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(path)) if os.path.exists(path) else {}
    ent = {}
    for kern, alg in kernels:
        fk = [v for k, vs in fetch.items() if f"{kern}_kernel" in k for v in vs]
        wk = [v for k, vs in write.items() if f"{kern}_kernel" in k for v in vs]
        if not fk or not wk:
            continue
        fb = float(np.mean(fk)) * 1024.0 / cf
        wb = float(np.mean(wk)) * 1024.0 / cw
        ent[kern] = {"hbm_bytes_per_launch": round(fb + wb), "fetch_bytes": round(fb), "write_bytes": round(wb),
                     "algorithmic_bytes": alg, "traffic_over_algorithmic": round((fb + wb) / alg, 3),
                     "dispatches": len(fk), "kernel_sources_sha": kernel_source_digest(sources_of(kern))}
    if not ent:
        raise SystemExit("no library kernel dispatches in the counter runs")
    ent["calibration"] = {"copy_bytes": CALIBRATE_BYTES, "fetch_factor": round(cf, 4), "write_factor": round(cw, 4)}
    rec[f"config{key}"] = ent
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print(json.dumps({f"config{key}": ent}))


def jd_algorithmic_bytes(w, e: int):
    """What the shared-basis apply must move: ids, x rows and y read + write of the tokens with an adapter in a cluster,
    U_j and V_j of every touched cluster once, Sigma_i, scale and cluster of
    every touched adapter once, and the two float32 buffers of [tokens, r]
    (V^T x, then Sigma applied) written and read once."""
    ids = w.ids.astype(np.int64)
    ok = (ids >= 0) & (ids < w.n)
    c = np.where(ok, w.cluster_of[np.clip(ids, 0, w.n - 1)], -1)
    ok &= (c >= 0) & (c < w.k)
    tv = int(ok.sum())
    adapters = np.unique(ids[ok])
    clusters = np.unique(c[ok])
    sig = w.r * w.r if w.mode == "full" else w.r
    parts = {"ids": 4 * w.T, "x": tv * w.d_in * e, "y": 2 * tv * w.d_out * e,
             "basis": len(clusters) * w.r * (w.d_in + w.d_out) * e, "sigma": len(adapters) * (4 * sig + 8),
             "h": 16 * tv * w.r}
    parts["total"] = sum(parts.values())
    return parts


def run_jd(args, rs, torch, dev, key):
    from workloads import make_jd_config
    w = make_jd_config(key)
    e = 2
    dt = torch.bfloat16
    gen = torch.Generator(device=dev).manual_seed(7)
    st = rs.lora_jd_pack([torch.from_numpy(u).to(dev).to(dt) for u in w.U],
                         [torch.from_numpy(v).to(dev).to(dt) for v in w.V], w.cluster_of, w.sigma, w.scales)
    x = torch.from_numpy(w.x).to(dev).to(dt)
    y = torch.randn(w.T, w.d_out, generator=gen, device=dev).to(dt)
    ids = torch.from_numpy(w.ids).to(dev)
    per_copy = (st.basis.A_pack.numel() + st.basis.B_pack.numel() + st.sigma.numel() * 4
                + x.numel() * 2 + y.numel() * 2)
    n_copies = 1 if args.warm else int(min(512, max(1, math.ceil(COLD_BYTES / per_copy))))
    copies = [Copy(st, x, y)] + [Copy(st.clone(), x.clone(), y.clone()) for _ in range(n_copies - 1)]
    ws = torch.empty(rs.lora_jd_workspace_bytes(st, w.T), dtype=torch.uint8, device=dev)
    step = lambda c: rs.lora_jd_apply(c.store, c.x, c.y, ids, ws=ws)
    eager_ms, _ = time_apply(rs, torch, copies, ids, ws, args.steps, args.warmup, step=step)
    ms, wall = (eager_ms, 0.0) if args.no_graph else \
        time_apply_graph(rs, torch, copies, ids, ws, args.steps, args.warmup, step=step)
    nb = jd_algorithmic_bytes(w, e)
    gbps = nb["total"] / (ms * 1e-3) / 1e9
    del copies
    torch.cuda.empty_cache()
    # The same adapters served as ordinary rank-r LoRA: B_i = U_j Sigma_i, A_i = V_j^T.
    as_lora = None
    if not args.no_padded:
        A_l, B_l = [], []
        for a in range(w.n):
            cj = int(w.cluster_of[a])
            S = torch.from_numpy(w.sigma[a]).to(dev)
            S = S if S.dim() == 2 else torch.diag(S)
            U = torch.from_numpy(w.U[cj]).to(dev)
            B_l.append((U @ S).to(dt).contiguous())
            A_l.append(torch.from_numpy(w.V[cj]).to(dev).t().contiguous().to(dt))
        ls = rs.lora_pack_retained(A_l, B_l, w.scales)
        del A_l, B_l
        lper = ls.A_pack.numel() + ls.B_pack.numel() + x.numel() * 2 + y.numel() * 2
        lcopies = [Copy(ls, x, y)] + [Copy(ls.clone(), x.clone(), y.clone())
                                      for _ in range((1 if args.warm else max(1, math.ceil(COLD_BYTES / lper))) - 1)]
        lws = torch.empty(rs.lora_workspace_bytes(ls, w.T), dtype=torch.uint8, device=dev)
        lms, _ = (time_apply if args.no_graph else time_apply_graph)(rs, torch, lcopies, ids, lws,
                                                                   max(20, args.steps // 2), args.warmup)
        as_lora = {"ms_per_step": round(lms, 5), "tokens_per_s": round(w.T / (lms * 1e-3), 1),
                   "store_bytes": ls.A_pack.numel() + ls.B_pack.numel(),
                   "jd_store_bytes": st.basis.A_pack.numel() + st.basis.B_pack.numel() + st.sigma.numel() * 4,
                   "jd_speedup": round(lms / ms, 3)}
        del lcopies, lws, ls
        torch.cuda.empty_cache()
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import jd_apply_ref
        try:
            from threadpoolctl import threadpool_limits
            limiter = threadpool_limits(1)
        except Exception:  # pragma: no cover
            limiter = None
        Ts = min(w.T, 256)
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds:
            jd_apply_ref(w.x[:Ts], w.ids[:Ts], w.cluster_of, w.U, w.V, w.sigma, w.scales)
            reps += 1
        el = time.perf_counter() - t0
        if limiter is not None:
            limiter.unregister()
        cpu = {"value": round(reps * Ts / el, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"first {Ts} tokens, float64 per-token loop, {reps} repetitions over {el:.1f} s, "
                         "BLAS pinned to 1 thread"}
    roofline = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps / PEAK_GBPS, 4), "traffic": None,
                "kernel": "the step's three launches together (shrink grouped by cluster, Sigma, expand)",
                "algorithmic_bytes_per_launch": nb["total"], "avg_launch_us": round(ms * 1e3, 2)}
    out = {
        "metric": METRIC, "value": round(w.T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded orthonormal (full) or N(0,1/sqrt(d)) (diag) bases, N(0,.) Sigma, N(0,1) x, bf16",
        "config": {"workload": WORKLOAD_NAMES[key], "T": w.T, "n_adapters": w.n, "clusters": w.k, "r": w.r,
                   "d_in": w.d_in, "d_out": w.d_out, "timing": "warm" if args.warm else
                   f"cold-HBM rotation over {n_copies} copies"},
        "gbps": round(gbps, 1), "hbm_frac": round(gbps / PEAK_GBPS, 4), "bytes_per_step": nb["total"],
        "bytes_breakdown": nb, "roofline": roofline, "cpu_baseline": cpu, "launches_per_step": 3,
        "as_lora": as_lora, "eager_ms_per_step": round(eager_ms, 5),
        "timed_as": "eager launches" if args.no_graph else "one HIP-graph replay of the K captured steps",
        "kernel_sources_sha": kernel_source_digest(JD_SOURCES),
    }
    print(json.dumps(out), flush=True)


def rsvd_algorithmic(n: int, r: int, d_in: int, d_out: int, keep_total: int, e: int):
    """Algorithmic work of retained-factor construction: the Grams B^T B and
    A A^T (symmetric: r (r + 1) / 2 entries of d multiply-adds, r (r + 1) d
    flops each), reading every factor once; the write reads them once more
    (the retained factors depend on all rows) and forms k_a columns of B' and
    rows of A' (2 r k_a d flops)."""
    d = d_in + d_out
    return {"gram_flops": n * r * (r + 1) * d, "gram_bytes": n * r * d * e,
            "write_flops": 2 * r * keep_total * d, "write_bytes": n * r * d * e + keep_total * d * e}


def run_rsvd(args, rs, torch, dev, key):
    from workloads import make_rsvd_config
    t0 = time.perf_counter()
    w = make_rsvd_config(key)
    print(f"[rsvd] inputs drawn in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    dt = torch.bfloat16
    A = torch.from_numpy(w.A).to(dev).to(dt)
    B = torch.from_numpy(w.B).to(dev).to(dt)
    f = rs.lora_rsvd_factor(A, B)
    torch.cuda.synchronize()
    sig = f.sigma.cpu().numpy()
    bad = int(f.status.cpu().numpy().sum())
    r_orig = [w.r] * w.n
    budget = sum(rs.lora_ranks_uniform(r_orig, 1.0 / 12.0, 4))
    t0 = time.perf_counter()
    ranks = rs.lora_ranks_spectral(r_orig, list(sig), 4, budget)
    policy_ms = 1e3 * (time.perf_counter() - t0)
    store = rs.lora_rsvd_write(f, ranks, w.scales)
    torch.cuda.synchronize()

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def step():
        rs.lora_rsvd_factor(A, B, out=f)
        rs.lora_rsvd_write(f, None, None, store=store)

    steps, warmup = args.steps, args.warmup
    ms = timed(step, steps, warmup)
    kern = {name: timed(lambda ph=ph: rs.lora_rsvd_factor(A, B, phases=ph, out=f), steps, warmup)
            for name, ph in (("rsvd_gram", 1), ("rsvd_prep", 2), ("rsvd_jacobi", 4), ("rsvd_post", 8))}
    kern["rsvd_write"] = timed(lambda: rs.lora_rsvd_write(f, None, None, store=store), steps, warmup)
    keep = int(sum(ranks))
    alg = rsvd_algorithmic(w.n, w.r, w.d_in, w.d_out, keep, 2)
    g_tf = alg["gram_flops"] / (kern["rsvd_gram"] * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import retained_factors_ref
        try:
            from threadpoolctl import threadpool_limits
            limiter = threadpool_limits(1)
        except Exception:  # pragma: no cover
            limiter = None
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds:
            a = reps % w.n
            retained_factors_ref(w.A[a].astype(np.float64), w.B[a].astype(np.float64), ranks[a])
            reps += 1
        el = time.perf_counter() - t0
        if limiter is not None:
            limiter.unregister()
        cpu = {"value": round(reps / el, 2), "unit": "adapters/s", "cores": 1, "kind": "oracle",
               "sample": f"{reps} adapters in {el:.1f} s (numpy QR + SVD in float64 per adapter), BLAS pinned "
                         "to 1 thread"}
    roofline = {"bound": "alu", "achieved": round(g_tf, 2), "peak": PEAK_FP64_TFLOPS, "unit": "TFLOP/s",
                "frac": round(g_tf / PEAK_FP64_TFLOPS, 4),
                "traffic": traffic_for(f"config{key}", "rsvd_gram", RSVD_SOURCES), "kernel": "rsvd_gram",
                "algorithmic_flops_per_launch": alg["gram_flops"],
                "avg_launch_us": round(kern["rsvd_gram"] * 1e3, 2)}
    out = {
        "metric": "retained-factor construction adapters/s (r-SVD through tall-skinny QR), 1 MI355X",
        "value": round(w.n / (ms * 1e-3), 1), "unit": "adapters/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64",
        "data": "synthetic: seeded N(0,1/sqrt(d)) factors, B columns scaled by (j+1)^-alpha, alpha~U(0,1.5), bf16",
        "config": {"workload": WORKLOAD_NAMES[key], "n_adapters": w.n, "r": w.r, "d_in": w.d_in,
                   "d_out": w.d_out, "retained_total": keep, "rank_range": [int(min(ranks)), int(max(ranks))]},
        "kernels_avg_ms": {k: round(v, 4) for k, v in kern.items()},
        "gram_tflops": round(g_tf, 2),
        "algorithmic": alg, "roofline": roofline, "cpu_baseline": cpu, "status_flagged": bad,
        "host_policy_ms": round(policy_ms, 3),
        "write_gbps": round(alg["write_bytes"] / (kern["rsvd_write"] * 1e-3) / 1e9, 1),
        "timed_as": "eager launches (a step: factor, i.e. Gram + core, then write), HIP events on the stream",
        "kernel_sources_sha": kernel_source_digest(RSVD_SOURCES),
    }
    print(json.dumps(out), flush=True)


def run_ranks(args):
    """Host timing of the rank policies at fleet scale (no GPU work): the
    library's C calls on arrays marshalled once (the Python binding's list
    conversions are not the policy's cost)."""
    import ctypes as C

    from rank_specialized_amd import _lib as L
    from oracle import spectral_ranks_ref
    rng = np.random.default_rng(5)
    m, r = 1024 * 196, 64
    # singular values of a rank-64 adapter product: a decaying spectrum, per unit
    sig = np.sort(rng.gamma(2.0, 1.0, size=(m, r)).astype(np.float32) *
                  np.exp(-np.arange(r) / 16.0).astype(np.float32), axis=1)[:, ::-1].copy()
    ro = np.full(m, r, np.int32)
    off = np.arange(m + 1, dtype=np.int64) * r
    u = np.zeros(m, np.int32)
    s = np.zeros(m, np.int32)
    lib = L.lib()

    def timed(fn):
        reps, t0 = 0, time.perf_counter()
        while True:
            L.check("rank policy", fn())
            reps += 1
            if time.perf_counter() - t0 > 1.0:
                return (time.perf_counter() - t0) / reps

    t_u = timed(lambda: lib.lora_ranks_uniform(m, ro.ctypes.data, C.c_double(1 / 12), 4, u.ctypes.data))
    budget = int(u.sum())
    t_s = timed(lambda: lib.lora_ranks_spectral(m, ro.ctypes.data, sig.ctypes.data, off.ctypes.data, 4, budget,
                                                s.ctypes.data))
    e_u = float(sum((sig[i, : u[i]].astype(np.float64) ** 2).sum() for i in range(0, m, 97)))
    e_s = float(sum((sig[i, : s[i]].astype(np.float64) ** 2).sum() for i in range(0, m, 97)))
    ms_o = 64
    t0 = time.perf_counter()
    spectral_ranks_ref([r] * ms_o, [x.astype(np.float64) for x in sig[:ms_o]], 4, budget=int(u[:ms_o].sum()))
    t_o = time.perf_counter() - t0
    print(json.dumps({
        "metric": "retained-rank allocation units per second (host, one thread)", "value": round(m / t_s, 1),
        "unit": "units/s", "n_gpus": 0, "ms_per_step": round(t_s * 1e3, 3), "higher_is_better": True,
        "config": {"workload": WORKLOAD_NAMES["ranks-fleet"], "units": m, "r_orig": r, "budget": budget},
        "uniform_ms": round(t_u * 1e3, 3), "spectral_ms": round(t_s * 1e3, 3),
        "spectral_rank_range": [int(s.min()), int(s.max())], "budget_met": int(s.sum()) == budget,
        "energy_kept_sampled": {"uniform": round(e_u, 1), "spectral": round(e_s, 1)},
        "cpu_baseline": {"value": round(ms_o / t_o, 1), "unit": "units/s", "cores": 1, "kind": "oracle",
                         "sample": f"first {ms_o} units, the oracle's repeated greedy selection"},
    }), flush=True)


def cpu_baseline(wl, seconds: float):
    """The CPU oracle as it stands, on a bounded sample of the same workload,
    with BLAS pinned to one thread."""
    from oracle import apply_ref
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(1)
    except Exception:  # pragma: no cover
        limiter = None
    m = wl.module
    T = wl.T
    sample = min(T, 256)
    x, ids, y0 = wl.x[:sample], wl.ids[:sample], wl.y0[:sample]
    tokens, t0 = 0, time.perf_counter()
    while True:
        apply_ref(x, ids, m.A, m.B, m.scales, y0)
        tokens += sample
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    if limiter is not None:
        limiter.unregister()
    return {"value": tokens / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {sample} tokens of the same workload, float64 per-token loop, repeated "
                      f"{tokens // sample}x over {el:.1f} s on {platform.processor() or platform.machine()}"
                      f" (host has {os.cpu_count()} logical CPUs; BLAS pinned to 1 thread)"}


# ------------------------------------------------------------------ fleet
def build_fleet(rs, torch, key: str, dev, pad_to_rmax: bool):
    """The 196 module stores of one decode step.  Factor values are drawn on
    the GPU (N(0, 1/sqrt(d)), bf16): the apply's time depends only on shapes,
    ranks and ids, and parity of fleet modules is tested on the oracle's
    inputs separately."""
    from workloads import fleet_module_shapes, fleet_ranks
    ranks = fleet_ranks(key)
    gen = torch.Generator(device=dev)
    gen.manual_seed(2611)
    stores, meta = [], []
    for (layer, proj, name, d_in, d_out, kind) in fleet_module_shapes():
        r = ranks[layer, proj]
        off = np.concatenate([[0], np.cumsum(r)])
        R = int(off[-1])
        A_src = (torch.randn(R, d_in, generator=gen, device=dev) * d_in ** -0.5).to(torch.bfloat16)
        B_src = (torch.randn(R * d_out, generator=gen, device=dev) * d_out ** -0.5).to(torch.bfloat16)
        A = [A_src[off[a]:off[a + 1]] for a in range(len(r))]
        B = [B_src[off[a] * d_out:off[a + 1] * d_out].view(d_out, int(r[a])) for a in range(len(r))]
        pad = int(r.max()) if pad_to_rmax else 0
        stores.append(rs.lora_pack_retained(A, B, np.full(len(r), 0.5, np.float32), pad_to=pad))
        del A, B, A_src, B_src
        meta.append((layer, proj, name, d_in, d_out, kind, r))
    return stores, meta


def run_fleet(args, rs, torch, dev):
    from workloads import FLEET_INPUT_DIMS, fleet_ids
    key = args.config
    T, n = 4096, 1024
    ids_np = fleet_ids(T, n)
    ids = torch.from_numpy(ids_np).to(dev)
    stores, meta = build_fleet(rs, torch, key, dev, False)
    gen = torch.Generator(device=dev)
    gen.manual_seed(2612)
    layers = max(m[0] for m in meta) + 1
    xs = {(l, k): torch.randn(T, d, generator=gen, device=dev).to(torch.bfloat16)
          for l in range(layers) for k, d in enumerate(FLEET_INPUT_DIMS)}
    ys = [torch.randn(T, m[4], generator=gen, device=dev).to(torch.bfloat16) for m in meta]
    ws = torch.empty(max(rs.lora_workspace_bytes(st, T) for st in stores), dtype=torch.uint8, device=dev)
    seg = rs.lora_segment(ids, n)
    per_mod = [algorithmic_bytes(ids_np, m[6], n, m[3], m[4], 2) for m in meta]
    seg_bytes = 4 * (2 * T + n + 2)
    step_bytes = seg_bytes + sum(b["total"] for b in per_mod)

    # The shrink-only and expand-only passes need one workspace per module:
    # a module's expand reads the plan and partial sums of its own shrink.
    mod_ws = [torch.empty(rs.lora_workspace_bytes(st, T), dtype=torch.uint8, device=dev) for st in stores]

    nstr = max(1, args.streams)
    stages = []  # module indices per (layer, input kind), in forward order
    for i, m in enumerate(meta):
        if stages and meta[stages[-1][0]][0] == m[0] and meta[stages[-1][0]][5] == m[5]:
            stages[-1].append(i)
        else:
            stages.append([i])
    side_streams = [torch.cuda.Stream() for _ in range(nstr - 1)]  # default priority
    str_ws = [ws] + [torch.empty_like(ws) for _ in range(nstr - 1)]

    def step(phases=3):
        if phases == 3:
            rs.lora_segment(ids, n, seg=seg)
        if phases == 3 and nstr > 1:
            # The modules of one stage (those reading the same input: q/k/v,
            # then o, then gate/up, then down, layer after layer) go to
            # different streams, each with its own workspace; a stage starts
            # when the previous one has finished, as in a forward pass, where
            # each stage's input comes from the one before.
            main = torch.cuda.current_stream()
            for stage in stages:
                for sst in side_streams:
                    sst.wait_stream(main)
                for k, i in enumerate(stage):
                    m = meta[i]
                    with torch.cuda.stream(main if k % nstr == 0 else side_streams[k % nstr - 1]):
                        rs.lora_apply_batched(stores[i], xs[(m[0], m[5])], ys[i], seg=seg, ws=str_ws[k % nstr])
                for sst in side_streams:
                    main.wait_stream(sst)
            return
        for st, m, y, w in zip(stores, meta, ys, mod_ws):
            x = xs[(m[0], m[5])]
            if phases == 3:
                rs.lora_apply_batched(st, x, y, seg=seg, ws=ws)
            else:
                rs.lora_apply_batched_phases(st, x, y, phases, seg=seg, ws=w)

    def timed(phases, reps):
        for _ in range(max(1, args.warmup)):
            step(phases)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        if args.no_graph:
            e0.record()
            for _ in range(reps):
                step(phases)
            e1.record()
            torch.cuda.synchronize()
        else:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step(phases)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(phases)
            g.replay()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            del g
        return e0.elapsed_time(e1) / reps

    steps = args.steps
    t0 = time.perf_counter()
    ms = timed(3, steps)
    wall = time.perf_counter() - t0
    k_ms = {"shrink": timed(1, steps), "expand": timed(2, steps)}  # expand after shrink: plans in place
    mod_ws[:] = [None] * len(mod_ws)  # only the full step (one shared workspace) runs from here
    kern = {}
    for name, kms in k_ms.items():
        nb = sum(b[name] for b in per_mod)
        kern[name] = {"avg_us": round(1e3 * kms / len(stores), 2), "launches_per_step": len(stores),
                      "algorithmic_bytes_per_step": nb, "gbps": round(nb / (kms * 1e-3) / 1e9, 1)}
    dom = max(kern, key=lambda k: kern[k]["avg_us"])
    achieved = kern[dom]["algorithmic_bytes_per_step"] / (k_ms[dom] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_GBPS, 4), "traffic": traffic_for(f"config{key}", dom),
                "kernel": f"{dom}_kernel<BF16> over the 196 modules of a step",
                "algorithmic_bytes_per_launch": round(kern[dom]["algorithmic_bytes_per_step"] / len(stores)),
                "avg_launch_us": kern[dom]["avg_us"]}
    multi = {}
    if not args.no_multi:
        # The same step with the projections that share an input applied
        # together (q/k/v, gate/up): one x read per group.
        groups = {}
        for i, m in enumerate(meta):
            groups.setdefault((m[0], m[5]), []).append(i)
        mstores = {g: rs.lora_pack_multi([stores[i] for i in idx]) for g, idx in groups.items() if len(idx) > 1}
        mbytes = max([rs.lora_multi_workspace_bytes(mst, T) for mst in mstores.values()] + [ws.numel()])
        mws = [torch.empty(mbytes, dtype=torch.uint8, device=dev)]

        def step_multi(phases=3):
            # One call per stage: nothing is left to overlap in a forward pass.
            rs.lora_segment(ids, n, seg=seg)
            for g, idx in groups.items():
                if len(idx) > 1:
                    rs.lora_apply_multi(mstores[g], xs[g], [ys[j] for j in idx], seg=seg, ws=mws[0])
                else:
                    rs.lora_apply_batched(stores[idx[0]], xs[g], ys[idx[0]], seg=seg, ws=mws[0])

        saved = sum(T * meta[idx[0]][3] * 2 * (len(idx) - 1) for idx in groups.values())
        step_fn = step
        step = step_multi
        mms = timed(3, steps)
        step = step_fn
        multi = {"groups": "per layer: q+k+v, o, gate+up, down", "calls_per_step": len(groups),
                 "ms_per_step": round(mms, 4), "tokens_per_s": round(T / (mms * 1e-3), 1),
                 "x_bytes_saved_per_step": saved, "algorithmic_bytes_per_step": step_bytes - saved,
                 "gbps": round((step_bytes - saved) / (mms * 1e-3) / 1e9, 1), "speedup": round(ms / mms, 3)}
        del mstores, mws
        torch.cuda.empty_cache()
    padded = {}
    if not args.no_padded and key == "5S":
        del stores
        torch.cuda.empty_cache()
        stores, _ = build_fleet(rs, torch, key, dev, True)
        ws = torch.empty(max(rs.lora_workspace_bytes(st, T) for st in stores), dtype=torch.uint8, device=dev)
        pms = timed(3, max(2, steps // 2))
        padded["pad_r_max"] = {"pad_to": "r_max of each module (16)", "ms_per_step": round(pms, 4),
                               "tokens_per_s": round(T / (pms * 1e-3), 1),
                               "effective_gbps": round(step_bytes / (pms * 1e-3) / 1e9, 1),
                               "specialized_speedup": round(pms / ms, 3)}
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import apply_ref
        from workloads import make_fleet_module
        try:
            from threadpoolctl import threadpool_limits
            limiter = threadpool_limits(1)
        except Exception:  # pragma: no cover
            limiter = None
        wl = make_fleet_module(key, 0, 0)
        sample = 64
        done, c0 = 0, time.perf_counter()
        while True:
            apply_ref(wl.x[:sample], wl.ids[:sample], wl.module.A, wl.module.B, wl.module.scales)
            done += sample
            el = time.perf_counter() - c0
            if el >= args.cpu_seconds:
                break
        if limiter is not None:
            limiter.unregister()
        cpu = {"value": round(done / el / len(meta), 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"first {sample} tokens through module L0.q (3584->3584), float64 per-token loop, "
                         f"{done // sample} repetitions over {el:.1f} s, BLAS pinned to 1 thread; token-module "
                         f"rate divided by the {len(meta)} modules of a step"}
    out = {
        "metric": METRIC, "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded Zipf(1.1) ids; factors, activations and y0 drawn on the GPU, bf16",
        "config": {"workload": WORKLOAD_NAMES[key], "T": T, "n_adapters": n, "modules": len(meta),
                   "ranks_sum_per_module_mean": float(np.mean([int(m[6].sum()) for m in meta])),
                   "timing": "HBM-resident working set of ~50 GB (no rotation needed)"},
        "gbps": round(step_bytes / (ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / PEAK_GBPS, 4),
        "bytes_per_step": step_bytes, "roofline": roofline, "cpu_baseline": cpu, "kernels": kern,
        "padded": padded, "multi_slice": multi, "streams": nstr, "wall_s_timed": round(wall, 6),
        "timed_as": "eager launches" if args.no_graph else "HIP-graph replays of one captured step",
        "kernel_sources_sha": kernel_source_digest(),
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.config, *args.summarize_pmc)
        return
    if args.config == "ranks-fleet":
        run_ranks(args)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; the apply's sharding across GPUs "
                                   "is described in DESIGN.md but not built", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import rank_specialized_amd as rs

    rs.load_library()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda", 0)
    if args.calibrate_copy:
        src = torch.ones(CALIBRATE_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    key = args.config
    if key in ("5U", "5S"):
        run_fleet(args, rs, torch, dev)
        return
    if key.startswith("jd-"):
        run_jd(args, rs, torch, dev, key)
        return
    if key.startswith("rsvd-"):
        run_rsvd(args, rs, torch, dev, key)
        return
    wl = build_workload(key)
    m = wl.module
    e = 2 if wl.dtype == "bf16" else 4
    ids = torch.from_numpy(wl.ids).to(dev)
    nbytes = algorithmic_bytes(wl.ids, m.ranks, m.n, m.d_in, m.d_out, e)

    copies, per_copy = make_copies(rs, torch, wl, dev, 0, not args.warm)
    ws = torch.empty(rs.lora_workspace_bytes(copies[0].store, wl.T), dtype=torch.uint8, device=dev)
    eager_ms, eager_wall = time_apply(rs, torch, copies, ids, ws, args.steps, args.warmup)
    if args.no_graph:
        ms, wall = eager_ms, eager_wall
    else:
        ms, wall = time_apply_graph(rs, torch, copies, ids, ws, args.steps, args.warmup)
    launches = rs.lora_apply_launches(copies[0].store, wl.T, True)
    # The two-launch form's kernels, each alone (for a fused call: a comparison).
    split = time_kernels(rs, torch, copies, ids, ws, args.steps, args.warmup, graph=not args.no_graph)
    gbps = nbytes["total"] / (ms * 1e-3) / 1e9
    for k in ("shrink", "expand"):
        split[k]["algorithmic_bytes"] = nbytes[k]
        split[k]["gbps"] = round(nbytes[k] / (split[k]["avg_us"] * 1e-6) / 1e9, 1)
        split[k] = {a: (round(b, 2) if isinstance(b, float) else b) for a, b in split[k].items()}
    if launches == 1:
        # One fused kernel per step: the step's timed replay is K launches of it.
        kern = {"decode_apply": {"avg_us": round(ms * 1e3, 2), "launches": args.steps,
                                 "timed_as": "the step's timing (one launch per step)",
                                 "algorithmic_bytes": nbytes["total"], "gbps": round(gbps, 1)}}
        dom, dom_bytes = "decode_apply", nbytes["total"]
    else:
        kern = split
        dom = max(("shrink", "expand"), key=lambda k: kern[k]["avg_us"])
        dom_bytes = nbytes[dom]
    achieved = dom_bytes / (kern[dom]["avg_us"] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_GBPS, 4),
                "traffic": traffic_for(f"config{key}", dom),
                "kernel": f"{dom}_kernel<{'BF16' if e == 2 else 'F32'}>",
                "algorithmic_bytes_per_launch": dom_bytes,
                "avg_launch_us": round(kern[dom]["avg_us"], 2)}
    del copies
    torch.cuda.empty_cache()

    padded = {}
    if not args.no_padded:
        r_max = int(m.ranks.max())
        variants = {"pad_r_max": r_max}
        if m.orig_rank and m.orig_rank > r_max:
            variants["pad_orig"] = int(m.orig_rank)
        p8 = int(-(-r_max // 8) * 8)
        if p8 != r_max:
            variants["pad8"] = p8
        for name, pad in variants.items():
            pc, _ = make_copies(rs, torch, wl, dev, pad, not args.warm)
            pws = torch.empty(rs.lora_workspace_bytes(pc[0].store, wl.T), dtype=torch.uint8, device=dev)
            pms, _ = (time_apply if args.no_graph else time_apply_graph)(rs, torch, pc, ids, pws,
                                                                       max(20, args.steps // 2), args.warmup)
            own = algorithmic_bytes(wl.ids, np.full(m.n, pad), m.n, m.d_in, m.d_out, e)["total"]
            padded[name] = {"pad_to": pad, "ms_per_step": round(pms, 5),
                            "tokens_per_s": round(wl.T / (pms * 1e-3), 1),
                            "effective_gbps": round(nbytes["total"] / (pms * 1e-3) / 1e9, 1),
                            "own_bytes": own, "own_gbps": round(own / (pms * 1e-3) / 1e9, 1),
                            "specialized_speedup": round(pms / ms, 3)}
            del pc, pws
            torch.cuda.empty_cache()

    cpu = None if args.no_cpu_baseline else cpu_baseline(wl, args.cpu_seconds)
    out = {
        "metric": METRIC,
        "value": round(wl.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic: seeded N(0,1) activations and y0, N(0,1/sqrt(d)) factors, rounded to bf16",
        "config": {"workload": WORKLOAD_NAMES[key], "T": wl.T, "n_adapters": m.n, "d_in": m.d_in,
                   "d_out": m.d_out, "ranks_sum": int(m.ranks.sum()), "r_max": int(m.ranks.max()),
                   "touched_adapters": nbytes["touched"], "timing": "warm" if args.warm else
                   f"cold-HBM rotation over {max(1, min(512, math.ceil(COLD_BYTES / per_copy)))} copies"},
        "gbps": round(gbps, 1),
        "hbm_frac": round(gbps / PEAK_GBPS, 4),
        "bytes_per_step": nbytes["total"],
        "roofline": roofline,
        "cpu_baseline": cpu,
        "launches_per_step": launches,
        "kernels": kern,
        "two_launch_kernels": split if launches == 1 else None,
        "padded": padded,
        "wall_s_timed": round(wall, 6),
        "timed_as": "eager launches" if args.no_graph else
                    "one HIP-graph replay of the K captured steps (eager launches: see eager_ms_per_step)",
        "eager_ms_per_step": round(eager_ms, 5),
        "kernel_sources_sha": kernel_source_digest(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
