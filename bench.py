#!/usr/bin/env python3
"""Benchmark of the batched, rank-specialized LoRA-delta apply on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 5S]

Default workload: the fleet decode step (5S): 28 layers x 7 projections of a
Qwen2-7B-like model (hidden 3584, k/v 512, MLP 18944), bf16, 1024 adapters
whose retained ranks vary 4..16 per module, T = 4096 decode tokens with
Zipf(1.1) adapter popularity.  A step is one pass of the whole hot path over
that batch: one token grouping with its plan of sub-tiles (lora_group) and
the 196 module applies on that plan (lora_apply_planned: shrink, then
expand), inputs resident in HBM.  A step streams ~50 GB, 200 times the 256 MB last-level cache, so it
reads its factors and activations from HBM by construction.

`--config 1|2|3|4` times one lora_apply_batched call with ids of the smaller
workloads instead; there the timed steps rotate through distinct copies of
(store, x, y) and every timed segment of steps starts after a 2 GiB cache
flush (outside the timed events), so each step reads from HBM too.

Timing: W untimed warm-up steps, then exactly K timed steps, bracketed by a
device synchronization on both sides.  The K steps are replays of HIP
graphs in at least 5 segments (one step per replay for the fleet), each
bracketed by HIP events on the launch stream: ms_per_step is their total
over K, and the line also carries the median, p10 and p90 per step.

Prints ONE JSON line: tokens/s of the rank-specialized apply, achieved
algorithmic HBM GB/s and fraction of the 8 TB/s peak, the roofline of the
dominant kernel (HIP events on its launch stream), the same kernels on
rank-padded stores, and the CPU oracle timed on a bounded sample (one core
and all host cores), run before the GPU is touched.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import multiprocessing
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LoRA-delta tokens/s and achieved HBM GB/s (% of ~8 TB/s peak), 1 MI355X"
PEAK_GBPS = 8000.0
FLUSH_BYTES = 2 << 30  # cache flush between timed segments: 8x the 256 MB Infinity Cache
MIN_SEGMENTS = 5       # the K timed steps are split into at least this many timed replays
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
PEAK_BF16_TFLOPS = 2500.0  # dense bf16 matrix-core peak of the MI355X

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
    "fused": "base layer with the branch fused: the fleet step's L0.q (3584->3584) and L0.gate (3584->18944) "
             "modules with a bf16 W0, y = x W0^T + s B A x for T=4096 Zipf(1.1) ids, against hipBLASLt's GEMM "
             "followed by the apply",
    "5U": "fleet decode step: 28 layers x 7 projections (3584/512/18944 dims) bf16, 1024 adapters rank 6 "
          "(orig 64), T=4096 Zipf(1.1) ids, one grouping and plan reused by 196 applies (q/k/v and gate/up "
          "concurrent)",
    "5S": "fleet decode step: 28 layers x 7 projections (3584/512/18944 dims) bf16, 1024 adapters ranks "
          "4..16 per module, T=4096 Zipf(1.1) ids, one grouping and plan reused by 196 applies (q/k/v and gate/up "
          "concurrent)",
}


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="5S", choices=sorted(WORKLOAD_NAMES))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-padded", action="store_true")
    p.add_argument("--no-multi", action="store_true", help="fleet: skip the multi-slice (q/k/v, gate/up) step")
    p.add_argument("--no-5u", action="store_true", help="fleet 5S: skip the uniform-rank (5U) step")
    p.add_argument("--no-fused", action="store_true", help="fleet: skip the base-fused comparison")
    p.add_argument("--legs", default="fused,unfused,gemm,gemm_hipblaslt",
                   help="base-fused comparison: which legs to time (comma list; counter runs take fewer)")
    p.add_argument("--no-kernels", action="store_true", help="skip the per-kernel timing passes")
    p.add_argument("--streams", type=int, default=3,
                   help="fleet: run the modules of one stage (q/k/v; gate/up) on up to this many streams")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="seconds per CPU-oracle leg")
    p.add_argument("--warm", action="store_true", help="no rotation and no flush (cache-resident timing)")
    p.add_argument("--no-graph", action="store_true", help="time eager launches only (counter runs)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="first run one elementwise copy of 256 MiB (reads and writes 256 MiB), the "
                        "reference that scales the HBM byte counters")
    p.add_argument("--summarize-trace", metavar="TRACE_DIR",
                   help="no GPU work: per-kernel durations of a rocprofv3 --kernel-trace run of this script, over "
                        "all dispatches and over the isolated ones (no other library kernel running: the "
                        "one-stream per-kernel passes), as a markdown table")
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


def fleet_algorithmic(key: str, T: int = 4096, n: int = 1024):
    """Per-module algorithmic bytes of the fleet step (module order), and the
    segmentation's own bytes (ids read, perm written, seg_off written)."""
    from workloads import fleet_ids, fleet_module_shapes, fleet_ranks
    ids = fleet_ids(T, n)
    ranks = fleet_ranks(key, n)
    per_mod = [algorithmic_bytes(ids, ranks[l, p], n, d_in, d_out, 2)
               for (l, p, _nm, d_in, d_out, _k) in fleet_module_shapes()]
    return ids, per_mod, 4 * (2 * T + n + 2)


# ------------------------------------------------------------------ CPU oracle
# The oracle as it stands, timed on the host on a bounded sample of the same
# workload: one core (BLAS pinned to one thread), then every core the process
# may use (capped at 16, the host share of one GPU), one forked worker per
# core on its own slice of tokens.  It runs before anything touches the GPU,
# so the forked workers inherit no GPU state.
_CPU_JOB = {}


def _blas_one_thread():
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(1)
    except Exception:  # pragma: no cover
        return None


def _cpu_leg(i: int):
    """Worker i of a leg: apply_ref over its slice of the sample until the
    leg's time is up; returns (tokens, seconds)."""
    from oracle import apply_ref
    job = _CPU_JOB
    lim = _blas_one_thread()
    lo = (i * job["per"]) % max(1, job["T"] - job["per"] + 1)
    x, ids = job["x"][lo:lo + job["per"]], job["ids"][lo:lo + job["per"]]
    done, t0 = 0, time.perf_counter()
    while True:
        apply_ref(x, ids, job["A"], job["B"], job["scales"])
        done += len(ids)
        el = time.perf_counter() - t0
        if el >= job["seconds"]:
            break
    if lim is not None:
        lim.unregister()
    return done, el


def host_cores() -> int:
    try:
        c = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        c = os.cpu_count() or 1
    return max(1, min(16, c))


def cpu_oracle(x, ids, A, B, scales, seconds: float, per: int, scale_to_step: int, what: str):
    """tokens/s of the oracle on a bounded sample (per tokens per worker),
    divided by scale_to_step (the modules of a fleet step; 1 otherwise)."""
    _CPU_JOB.update(x=x, ids=ids, A=A, B=B, scales=scales, seconds=seconds, per=per, T=len(ids))
    d1, e1 = _cpu_leg(0)
    one = d1 / e1 / scale_to_step
    cores = host_cores()
    with multiprocessing.get_context("fork").Pool(cores) as pool:
        res = pool.map(_cpu_leg, range(cores))
    all_rate = sum(d for d, _ in res) / max(e for _, e in res) / scale_to_step
    cpu = platform.processor() or platform.machine()
    unit_note = (f"; token-module rate divided by the {scale_to_step} modules of a step"
                 if scale_to_step > 1 else "")
    return {"value": round(all_rate, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{what}: float64 per-token loop (oracle apply_ref), {cores} forked workers of "
                      f"{per} tokens each (distinct slices), {seconds:.0f} s per leg, BLAS pinned to 1 thread "
                      f"per worker, on {cpu} ({os.cpu_count()} logical CPUs visible){unit_note}",
            "one_core": {"value": round(one, 3), "unit": "tokens/s", "cores": 1,
                         "sample": f"worker 0 alone, {d1} tokens in {e1:.1f} s"}}


# ------------------------------------------------------------------ timing
def split_steps(K: int):
    """K timed steps as R = min(K, MIN_SEGMENTS) segments of consecutive
    steps (the last takes the remainder)."""
    R = max(1, min(K, MIN_SEGMENTS))
    g = K // R
    return [g] * (R - 1) + [K - g * (R - 1)]


def percentiles(per_step_ms):
    v = np.asarray(per_step_ms, dtype=np.float64)
    return {"median_ms": round(float(np.median(v)), 6), "p10_ms": round(float(np.percentile(v, 10)), 6),
            "p90_ms": round(float(np.percentile(v, 90)), 6), "samples": int(len(v))}


class Flush:
    """A 2 GiB buffer read between timed segments (outside the timed
    events): afterwards neither the L2s nor the 256 MB last-level cache hold
    anything a step reads.  Read only, so that no dirty lines of the flush
    itself are still being written back when the timed segment starts (with
    a read-and-write flush, decode-spectral measured 73.5 against 65.0 us
    per step, prefill 181.0 against 167.9)."""

    def __init__(self, torch, dev, enabled: bool):
        self.torch = torch
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev) if enabled else None
        self.out = torch.zeros((), dtype=torch.float32, device=dev) if enabled else None

    def __call__(self):
        if self.buf is not None:
            self.torch.sum(self.buf, dim=0, out=self.out)


def time_steps(torch, step, copies, K, W, flush, graph=True):
    """Exactly K timed steps, as segments (split_steps) of consecutive steps
    on distinct copies (step i of a segment uses copies[i]), each segment one
    HIP-graph replay (or eager launches) bracketed by events on the launch
    stream and preceded by a cache flush.  W untimed eager warm-up steps come
    first.  Returns ms per step (total over K) and the per-segment
    distribution of ms per step."""
    lengths = split_steps(K)
    assert len(copies) >= max(lengths)
    for k in range(W):
        step(copies[k % len(copies)])
    torch.cuda.synchronize()
    graphs = {}
    if graph:
        for L in sorted(set(lengths)):
            side = torch.cuda.Stream()  # default priority
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for i in range(L):
                    step(copies[i])
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(L):
                    step(copies[i])
            g.replay()  # untimed first replay
            graphs[L] = g
    torch.cuda.synchronize()
    ev = []
    t0 = time.perf_counter()
    for L in lengths:
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        if graph:
            graphs[L].replay()
        else:
            for i in range(L):
                step(copies[i])
        e1.record()
        ev.append((L, e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    seg_ms = [e0.elapsed_time(e1) for _, e0, e1 in ev]
    per_step = [t / L for (L, _, _), t in zip(ev, seg_ms)]
    graphs.clear()
    return {"ms_per_step": sum(seg_ms) / K, "dist": percentiles(per_step), "wall_s": wall,
            "segments": lengths}


def time_replays(torch, step, K, W, graph=True):
    """Exactly K timed steps of a self-contained step (the fleet: each step
    streams ~50 GB, so no flush is needed): W eager warm-up steps, then one
    step captured in a HIP graph and replayed K times, each replay bracketed
    by events on the launch stream."""
    for _ in range(max(1, W)):
        step()
    torch.cuda.synchronize()
    g = None
    if graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        g.replay()
        torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    t0 = time.perf_counter()
    evs[0].record()
    for k in range(K):
        if g is not None:
            g.replay()
        else:
            step()
        evs[k + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [evs[k].elapsed_time(evs[k + 1]) for k in range(K)]
    del g
    return {"ms_per_step": evs[0].elapsed_time(evs[K]) / K, "dist": percentiles(per), "wall_s": wall}


# ------------------------------------------------------------------ counters
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


def summarize_trace(trace_dir: str):
    """Markdown table of the library's kernels in a rocprofv3 kernel trace:
    calls and average duration over all dispatches, and over the isolated
    ones (no other library kernel overlapping in time: the one-stream
    per-kernel passes, which bench.py's per-kernel figures time)."""
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            rows += [r for r in csv.DictReader(f) if "lora::" in r["Kernel_Name"]]
    ev = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]),
                 r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", ""))
                for r in rows)
    stats = {}
    for i, (s0, e0, k) in enumerate(ev):
        prev_end = ev[i - 1][1] if i else -1
        next_start = ev[i + 1][0] if i + 1 < len(ev) else 1 << 62
        d = (e0 - s0) / 1000.0
        a = stats.setdefault(k, ([], []))
        a[0].append(d)
        if prev_end <= s0 and e0 <= next_start:
            a[1].append(d)
    print("| kernel | calls | average (us) | isolated calls | isolated average (us) | isolated median (us) |")
    print("|---|---|---|---|---|---|")
    for k, (al, iso) in sorted(stats.items(), key=lambda kv: -sum(kv[1][0])):
        print(f"| `{k}` | {len(al)} | {np.mean(al):.2f} | {len(iso)} | "
              f"{(np.mean(iso) if iso else float('nan')):.2f} | {(np.median(iso) if iso else float('nan')):.2f} |")


def summarize_pmc(key: str, fetch_dir: str, write_dir: str):
    """HBM bytes per launch of the library's kernels: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) averaged over the dispatches, each scaled
    by what the same counter reads for an elementwise copy of 256 MiB.  For
    the fleet the algorithmic bytes are the mean over its 196 modules (every
    pass of a run covers each module once)."""
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
    elif key in ("5U", "5S"):
        _, per_mod, _ = fleet_algorithmic(key)
        kernels = tuple((k, float(np.mean([b[k] for b in per_mod]))) for k in ("shrink", "expand"))
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
                     "algorithmic_bytes": round(alg), "traffic_over_algorithmic": round((fb + wb) / alg, 3),
                     "dispatches": len(fk), "kernel_sources_sha": kernel_source_digest(sources_of(kern))}
    if not ent:
        raise SystemExit("no library kernel dispatches in the counter runs")
    ent["calibration"] = {"copy_bytes": CALIBRATE_BYTES, "fetch_factor": round(cf, 4), "write_factor": round(cw, 4)}
    rec[f"config{key}"] = ent
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print(json.dumps({f"config{key}": ent}))


# ------------------------------------------------------------------ workloads 1-4
def build_workload(key: str):
    from workloads import make_config
    return make_config(key, with_y0=True)


class Copy:
    def __init__(self, store, x, y):
        self.store, self.x, self.y = store, x, y


def make_copies(rs, torch, wl, dev, pad_to: int, n_copies: int):
    """n_copies independent (store, x, y) triples of the workload."""
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    A = [torch.from_numpy(a).to(dev).to(dt) for a in wl.module.A]
    B = [torch.from_numpy(b).to(dev).to(dt) for b in wl.module.B]
    store = rs.lora_pack_retained(A, B, wl.module.scales, pad_to=pad_to)
    del A, B
    x = torch.from_numpy(wl.x).to(dev).to(dt)
    y = torch.from_numpy(wl.y0).to(dev).to(dt)
    copies = [Copy(store, x, y)]
    for _ in range(n_copies - 1):
        copies.append(Copy(store.clone(), x.clone(), y.clone()))
    return copies


def run_config(args, rs, torch, dev, key, cpu):
    wl = build_workload(key)
    m = wl.module
    e = 2 if wl.dtype == "bf16" else 4
    ids = torch.from_numpy(wl.ids).to(dev)
    nbytes = algorithmic_bytes(wl.ids, m.ranks, m.n, m.d_in, m.d_out, e)
    K, W = args.steps, args.warmup
    n_copies = 1 if args.warm else max(split_steps(K))
    flush = Flush(torch, dev, not args.warm)
    copies = make_copies(rs, torch, wl, dev, 0, n_copies)
    ws = torch.empty(rs.lora_workspace_bytes(copies[0].store, wl.T), dtype=torch.uint8, device=dev)
    graph = not args.no_graph

    def step(c):
        rs.lora_apply_batched(c.store, c.x, c.y, ids=ids, ws=ws)

    t = time_steps(torch, step, copies, K, W, flush, graph=graph)
    eager = time_steps(torch, step, copies, K, 0, flush, graph=False) if graph else t
    ms = t["ms_per_step"]
    launches = rs.lora_apply_launches(copies[0].store, wl.T, True)
    # The two-launch form's kernels, each alone (for a fused call: a comparison).
    split = {}
    if not args.no_kernels:
        # Each kernel alone on a plan formed once (lora_group): the shrink,
        # then the expand on what the shrink left in ws; the grouping alone.
        seg = rs.lora_group(ids, m.n)
        for name, phase in (("shrink", 1), ("expand", 2)):
            kt = time_steps(torch, lambda c, ph=phase: rs.lora_apply_planned(c.store, c.x, c.y, seg, ws=ws, phases=ph),
                            copies, K, 1, flush, graph=graph)
            us = kt["ms_per_step"] * 1e3
            split[name] = {"avg_us": round(us, 2), "launches": K, "algorithmic_bytes": nbytes[name],
                           "gbps": round(nbytes[name] / (us * 1e-6) / 1e9, 1),
                           "timed_as": "graph replays of that kernel alone on a plan formed once, each segment "
                                       "after a cache flush (an expand alone then reads a cold plan and partial "
                                       "sums)"}
        gt = time_steps(torch, lambda c: rs.lora_group(ids, m.n, seg=seg), copies, K, 1, flush, graph=graph)
        split["grouping"] = {"avg_us": round(gt["ms_per_step"] * 1e3, 2), "launches": K,
                             "timed_as": "lora_group alone (seg_off, perm and the plan in one kernel)"}
    gbps = nbytes["total"] / (ms * 1e-3) / 1e9
    if launches == 1:
        kern = {"decode_apply": {"avg_us": round(ms * 1e3, 2), "launches": K,
                                 "timed_as": "the step's timing (one launch per step)",
                                 "algorithmic_bytes": nbytes["total"], "gbps": round(gbps, 1)}}
        dom, dom_bytes = "decode_apply", nbytes["total"]
    else:
        kern = split
        dom = max(("shrink", "expand"), key=lambda k: kern[k]["avg_us"]) if split else "shrink"  # not the grouping
        dom_bytes = nbytes[dom]
    dom_us = kern[dom]["avg_us"] if dom in kern else ms * 1e3
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_GBPS, 4), "traffic": traffic_for(f"config{key}", dom),
                "kernel": f"{dom}_kernel<{'BF16' if e == 2 else 'F32'}>",
                "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_us, 2)}
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
            pc = make_copies(rs, torch, wl, dev, pad, n_copies)
            pws = torch.empty(rs.lora_workspace_bytes(pc[0].store, wl.T), dtype=torch.uint8, device=dev)
            pt = time_steps(torch, lambda c: rs.lora_apply_batched(c.store, c.x, c.y, ids=ids, ws=pws),
                            pc, K, W, flush, graph=graph)
            pms = pt["ms_per_step"]
            own = algorithmic_bytes(wl.ids, np.full(m.n, pad), m.n, m.d_in, m.d_out, e)["total"]
            padded[name] = {"pad_to": pad, "ms_per_step": round(pms, 5), "median_ms": pt["dist"]["median_ms"],
                            "tokens_per_s": round(wl.T / (pms * 1e-3), 1),
                            "effective_gbps": round(nbytes["total"] / (pms * 1e-3) / 1e9, 1),
                            "own_bytes": own, "own_gbps": round(own / (pms * 1e-3) / 1e9, 1),
                            "specialized_speedup": round(pms / ms, 3)}
            del pc, pws
            torch.cuda.empty_cache()

    out = {
        "metric": METRIC, "value": round(wl.T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic: seeded N(0,1) activations and y0, N(0,1/sqrt(d)) factors, rounded to bf16",
        "config": {"workload": WORKLOAD_NAMES[key], "T": wl.T, "n_adapters": m.n, "d_in": m.d_in,
                   "d_out": m.d_out, "ranks_sum": int(m.ranks.sum()), "r_max": int(m.ranks.max()),
                   "touched_adapters": nbytes["touched"],
                   "timing": "warm (cache-resident)" if args.warm else
                   f"cold: {len(split_steps(K))} timed segments, each after a 2 GiB cache flush, steps of a "
                   f"segment on {n_copies} distinct copies of (store, x, y)"},
        "timing": dict(t["dist"], segments=t["segments"]),
        "gbps": round(gbps, 1), "hbm_frac": round(gbps / PEAK_GBPS, 4), "bytes_per_step": nbytes["total"],
        "roofline": roofline, "cpu_baseline": cpu, "launches_per_step": launches, "kernels": kern,
        "two_launch_kernels": split if launches == 1 else None, "padded": padded,
        "wall_s_timed": round(t["wall_s"], 6),
        "timed_as": "eager launches" if args.no_graph else "HIP-graph replays (see timing.segments)",
        "eager_ms_per_step": round(eager["ms_per_step"], 6),
        "kernel_sources_sha": kernel_source_digest(),
    }
    print(json.dumps(out), flush=True)


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
    K, W = args.steps, args.warmup
    n_copies = 1 if args.warm else max(split_steps(K))
    flush = Flush(torch, dev, not args.warm)
    copies = [Copy(st, x, y)] + [Copy(st.clone(), x.clone(), y.clone()) for _ in range(n_copies - 1)]
    ws = torch.empty(rs.lora_jd_workspace_bytes(st, w.T), dtype=torch.uint8, device=dev)
    step = lambda c: rs.lora_jd_apply(c.store, c.x, c.y, ids, ws=ws)
    graph = not args.no_graph
    t = time_steps(torch, step, copies, K, W, flush, graph=graph)
    eager_ms = time_steps(torch, step, copies, K, 0, flush, graph=False)["ms_per_step"] if graph else t["ms_per_step"]
    ms, wall = t["ms_per_step"], t["wall_s"]
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
        lcopies = [Copy(ls, x, y)] + [Copy(ls.clone(), x.clone(), y.clone()) for _ in range(n_copies - 1)]
        lws = torch.empty(rs.lora_workspace_bytes(ls, w.T), dtype=torch.uint8, device=dev)
        lms = time_steps(torch, lambda c: rs.lora_apply_batched(c.store, c.x, c.y, ids=ids, ws=lws), lcopies, K, W,
                         flush, graph=graph)["ms_per_step"]
        as_lora = {"ms_per_step": round(lms, 5), "tokens_per_s": round(w.T / (lms * 1e-3), 1),
                   "store_bytes": ls.A_pack.numel() + ls.B_pack.numel(),
                   "jd_store_bytes": st.basis.A_pack.numel() + st.basis.B_pack.numel() + st.sigma.numel() * 4,
                   "jd_speedup": round(lms / ms, 3)}
        del lcopies, lws, ls
        torch.cuda.empty_cache()
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import jd_apply_ref
        limiter = _blas_one_thread()
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
                   f"cold: timed segments each after a 2 GiB cache flush, on {n_copies} distinct copies"},
        "timing": t["dist"],
        "gbps": round(gbps, 1), "hbm_frac": round(gbps / PEAK_GBPS, 4), "bytes_per_step": nb["total"],
        "bytes_breakdown": nb, "roofline": roofline, "cpu_baseline": cpu, "launches_per_step": 3,
        "as_lora": as_lora, "eager_ms_per_step": round(eager_ms, 5),
        "timed_as": "eager launches" if args.no_graph else "HIP-graph replays in timed segments",
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


# ------------------------------------------------------------------ fleet
def build_fleet(rs, torch, key: str, dev, pad_to_rmax: bool, layers=None):
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
        if layers is not None and layer >= layers:
            break
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


def fleet_stages(meta):
    """Module indices per (layer, input kind), in forward order: the modules
    of a stage read the same input (q/k/v; o; gate/up; down)."""
    stages = []
    for i, m in enumerate(meta):
        if stages and meta[stages[-1][0]][0] == m[0] and meta[stages[-1][0]][5] == m[5]:
            stages[-1].append(i)
        else:
            stages.append([i])
    return stages


def fleet_step(rs, torch, stores, meta, xs, ys, ids, seg, n, nstr, str_ws):
    """One decode step: the grouping and its plan (lora_group), then every
    module's apply on that plan (lora_apply_planned).  The
    modules of a stage go to up to nstr streams (default priority, one
    workspace each); a stage starts when the previous one has finished, as in
    a forward pass, where each stage's input comes from the one before."""
    stages = fleet_stages(meta)
    side = [torch.cuda.Stream() for _ in range(nstr - 1)]

    def step():
        rs.lora_group(ids, n, seg=seg)  # the grouping and its plan, once per step
        if nstr == 1:
            for st, m, y in zip(stores, meta, ys):
                rs.lora_apply_planned(st, xs[(m[0], m[5])], y, seg, ws=str_ws[0])
            return
        main = torch.cuda.current_stream()
        for stage in stages:
            for s in side:
                s.wait_stream(main)
            for k, i in enumerate(stage):
                m = meta[i]
                with torch.cuda.stream(main if k % nstr == 0 else side[k % nstr - 1]):
                    rs.lora_apply_planned(stores[i], xs[(m[0], m[5])], ys[i], seg, ws=str_ws[k % nstr])
            for s in side:
                main.wait_stream(s)
    return step


def run_fleet_key(args, rs, torch, dev, key, xs, ys, ids, full: bool):
    """Time the fleet step of `key` (5U or 5S); with `full`, also each kernel
    alone, the multi-slice step and the rank-padded stores."""
    T, n = 4096, 1024
    _, per_mod, seg_bytes = fleet_algorithmic(key, T, n)
    step_bytes = seg_bytes + sum(b["total"] for b in per_mod)
    stores, meta = build_fleet(rs, torch, key, dev, False)
    seg = rs.lora_group(ids, n)
    nstr = max(1, args.streams)
    wsb = max(rs.lora_workspace_bytes(st, T) for st in stores)
    str_ws = [torch.empty(wsb, dtype=torch.uint8, device=dev) for _ in range(nstr)]
    graph = not args.no_graph
    K, W = args.steps, args.warmup
    t = time_replays(torch, fleet_step(rs, torch, stores, meta, xs, ys, ids, seg, n, nstr, str_ws), K, W, graph)
    ms = t["ms_per_step"]
    res = {"ms_per_step": ms, "timing": t["dist"], "wall_s": t["wall_s"], "bytes_per_step": step_bytes,
           "gbps": step_bytes / (ms * 1e-3) / 1e9, "tokens_per_s": T / (ms * 1e-3),
           "ranks_sum_per_module_mean": float(np.mean([int(m[6].sum()) for m in meta]))}
    if not full:
        del stores, str_ws
        torch.cuda.empty_cache()
        return res

    kern = {}
    if not args.no_kernels:
        # Each kernel alone over the 196 modules (one stream, a workspace per
        # module: a module's expand reads the plan and partial sums its own
        # shrink left).
        mod_ws = [torch.empty(rs.lora_workspace_bytes(st, T), dtype=torch.uint8, device=dev) for st in stores]

        def phase_step(ph):
            def f():
                for st, m, y, w in zip(stores, meta, ys, mod_ws):
                    rs.lora_apply_planned(st, xs[(m[0], m[5])], y, seg, ws=w, phases=ph)
            return f

        reps = max(MIN_SEGMENTS, min(K, 10))
        for name, ph in (("shrink", 1), ("expand", 2)):  # expand after shrink: plans in place
            kt = time_replays(torch, phase_step(ph), reps, 1, graph)
            nb = sum(b[name] for b in per_mod)
            us = kt["ms_per_step"] * 1e3 / len(stores)
            kern[name] = {"avg_us": round(us, 2), "launches_per_step": len(stores), "replays": reps,
                          "algorithmic_bytes_per_step": nb, "gbps": round(nb / (kt["ms_per_step"] * 1e-3) / 1e9, 1),
                          "timed_as": "graph replays of the 196 launches of that kernel alone, one stream"}
        del mod_ws
        torch.cuda.empty_cache()
    res["kernels"] = kern
    if kern:
        dom = max(kern, key=lambda k: kern[k]["avg_us"])
        dom_bytes = kern[dom]["algorithmic_bytes_per_step"] / len(stores)
        achieved = dom_bytes / (kern[dom]["avg_us"] * 1e-6) / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                           "frac": round(achieved / PEAK_GBPS, 4), "traffic": traffic_for(f"config{key}", dom),
                           "kernel": f"{dom}_kernel<BF16>, mean over the 196 modules of a step",
                           "algorithmic_bytes_per_launch": round(dom_bytes), "avg_launch_us": kern[dom]["avg_us"]}

    if not args.no_fused:
        res["base_fused"] = run_base_fused(args, rs, torch, dev, stores, meta, xs, ids, T)

    if not args.no_multi:
        # The projections that share an input applied together (q/k/v,
        # gate/up): one x read per group, one call per stage.
        groups = {}
        for i, m in enumerate(meta):
            groups.setdefault((m[0], m[5]), []).append(i)
        mstores = {g: rs.lora_pack_multi([stores[i] for i in idx]) for g, idx in groups.items() if len(idx) > 1}
        mbytes = max([rs.lora_multi_workspace_bytes(mst, T) for mst in mstores.values()] + [wsb])
        mws = torch.empty(mbytes, dtype=torch.uint8, device=dev)

        def step_multi():
            rs.lora_group(ids, n, seg=seg)
            for g, idx in groups.items():
                if len(idx) > 1:
                    rs.lora_apply_multi(mstores[g], xs[g], [ys[j] for j in idx], seg=seg, ws=mws)
                else:
                    rs.lora_apply_planned(stores[idx[0]], xs[g], ys[idx[0]], seg, ws=mws)

        saved = sum(T * meta[idx[0]][3] * 2 * (len(idx) - 1) for idx in groups.values())
        mt = time_replays(torch, step_multi, K, 1, graph)
        mms = mt["ms_per_step"]
        res["multi_slice"] = {"groups": "per layer: q+k+v, o, gate+up, down", "calls_per_step": len(groups),
                              "ms_per_step": round(mms, 5), "median_ms": mt["dist"]["median_ms"],
                              "tokens_per_s": round(T / (mms * 1e-3), 1), "x_bytes_saved_per_step": saved,
                              "algorithmic_bytes_per_step": step_bytes - saved,
                              "gbps": round((step_bytes - saved) / (mms * 1e-3) / 1e9, 1),
                              "speedup": round(ms / mms, 3)}
        del mstores, mws
    del stores, str_ws
    torch.cuda.empty_cache()

    if not args.no_padded and key == "5S":
        pstores, pmeta = build_fleet(rs, torch, key, dev, True)
        pwsb = max(rs.lora_workspace_bytes(st, T) for st in pstores)
        pws = [torch.empty(pwsb, dtype=torch.uint8, device=dev) for _ in range(nstr)]
        pt = time_replays(torch, fleet_step(rs, torch, pstores, pmeta, xs, ys, ids, seg, n, nstr, pws),
                          max(MIN_SEGMENTS, K // 2), 1, graph)
        pms = pt["ms_per_step"]
        res["padded"] = {"pad_r_max": {"pad_to": "r_max of each module (16)", "ms_per_step": round(pms, 5),
                                       "median_ms": pt["dist"]["median_ms"],
                                       "tokens_per_s": round(T / (pms * 1e-3), 1),
                                       "effective_gbps": round(step_bytes / (pms * 1e-3) / 1e9, 1),
                                       "specialized_speedup": round(pms / ms, 3)}}
        del pstores, pws
        torch.cuda.empty_cache()
    return res


def run_base_fused(args, rs, torch, dev, stores, meta, xs, ids, T=4096):
    """The base layer with the branch in its epilogue (lora_apply_base_fused)
    against the unfused pair (hipBLASLt's GEMM through torch.matmul, then
    lora_apply_batched), and the two GEMMs alone, for the L0.q and L0.gate
    modules of the fleet step.  W0 is drawn on the GPU (N(0, 1/d_in), bf16).
    Each figure: consecutive eager calls, events around each (hipBLASLt is
    kept out of graph capture; every call runs 100 us or more, so launches
    stay ahead of the GPU), caches warm (the GEMMs are bound by the matrix
    cores, not by HBM)."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(2613)
    out = {}
    reps = max(MIN_SEGMENTS, min(args.steps, 20))
    for name, idx in (("q", 0), ("gate", 4)):
        st, m = stores[idx], meta[idx]
        d_in, d_out = m[3], m[4]
        x = xs[(m[0], m[5])]
        W0 = (torch.randn(d_out, d_in, generator=gen, device=dev) * d_in ** -0.5).to(torch.bfloat16)
        y = torch.empty(T, d_out, dtype=torch.bfloat16, device=dev)
        ws = torch.empty(rs.lora_workspace_bytes(st, T), dtype=torch.uint8, device=dev)
        Wt = W0.t()
        legs = {
            "fused": lambda: rs.lora_apply_base_fused(st, W0, x, y, ids=ids, ws=ws),
            "unfused": lambda: (torch.matmul(x, Wt, out=y), rs.lora_apply_batched(st, x, y, ids=ids, ws=ws)),
            "gemm": lambda: rs.lora_apply_base_fused(st, W0, x, y),
            "gemm_hipblaslt": lambda: torch.matmul(x, Wt, out=y),
        }
        flops = 2.0 * T * d_in * d_out
        r = {"shape": f"{T} x {d_in} -> {d_out}", "gemm_flops": flops}
        wanted = args.legs.split(",")
        for leg, f in legs.items():
            if leg not in wanted:
                continue
            t = time_replays(torch, f, reps, 2, False)
            us = t["ms_per_step"] * 1e3
            r[leg] = {"us": round(us, 2), "median_us": round(t["dist"]["median_ms"] * 1e3, 2),
                      "tflops": round(flops / (us * 1e-6) / 1e12, 1)}
        if "fused" in r and "unfused" in r:
            r["fused_speedup"] = round(r["unfused"]["us"] / r["fused"]["us"], 3)
        r["y_bytes_not_moved"] = 2 * T * d_out * 2  # the unfused expand reads y and writes it again
        if "fused" in r:
            r["roofline"] = {"bound": "mfma", "achieved": r["fused"]["tflops"], "peak": PEAK_BF16_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(r["fused"]["tflops"] / PEAK_BF16_TFLOPS, 4)}
        out[name] = r
        del W0, y, ws
        torch.cuda.empty_cache()
    return out


def run_fused_only(args, rs, torch, dev):
    """--config fused: the base-fused comparison alone (for counter runs)."""
    from workloads import fleet_ids, fleet_module_shapes
    T, n = 4096, 1024
    ids = torch.from_numpy(fleet_ids(T, n)).to(dev)
    shapes = fleet_module_shapes()[:7]
    xs, _ = fleet_inputs(torch, dev, shapes, T, with_y=False)
    stores, meta = build_fleet(rs, torch, "5S", dev, False, layers=1)
    res = run_base_fused(args, rs, torch, dev, stores, meta, xs, ids, T)
    print(json.dumps({"metric": "base-fused apply us per call", "config": {"workload": WORKLOAD_NAMES["fused"]},
                      "base_fused": res}), flush=True)


def fleet_inputs(torch, dev, meta_shapes, T=4096, with_y=True):
    """The step's activations (drawn on the GPU, N(0, 1), bf16): per layer
    one input per kind (q/k/v, o, gate/up, down), and one y per module."""
    from workloads import FLEET_INPUT_DIMS
    gen = torch.Generator(device=dev)
    gen.manual_seed(2612)
    layers = max(m[0] for m in meta_shapes) + 1
    xs = {(l, k): torch.randn(T, d, generator=gen, device=dev).to(torch.bfloat16)
          for l in range(layers) for k, d in enumerate(FLEET_INPUT_DIMS)}
    ys = [torch.randn(T, m[4], generator=gen, device=dev).to(torch.bfloat16) for m in meta_shapes] if with_y else None
    return xs, ys


def _stream_ref_lib():
    """The benchmark's bandwidth references (libstream_ref.so, built beside the
    LoRA library): a plain copy and a plain read, 16 bytes per thread with
    streaming loads and stores.  None when it has not been built."""
    import ctypes
    path = os.path.join(ROOT, "rank_specialized_amd", "libstream_ref.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    for name, args in (("stream_ref_copy", [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
                       ("stream_ref_read", [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p])):
        getattr(lib, name).argtypes = args
        getattr(lib, name).restype = ctypes.c_int
    return lib


def copy_reference(torch, dev, nbytes=1 << 30, reps=5):
    """What plain streams reach here, beside the 8 TB/s peak: torch's copy of
    nbytes (read nbytes, write nbytes), the reference copy kernel on the same
    buffers, and the reference read of nbytes (buffers well beyond the
    last-level cache; events around each of `reps` runs, median).  The expand
    reads and writes its y rows (a read-write stream); the shrink only reads."""
    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev)
    b = torch.empty_like(a)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    a.fill_(1.0)
    b.copy_(a)
    torch.cuda.synchronize()
    lib = _stream_ref_lib()
    stream = torch.cuda.current_stream().cuda_stream

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    def check(rc):
        if rc != 0:
            raise RuntimeError(f"stream reference failed ({rc})")

    ms = timed(lambda: b.copy_(a))
    out = {"bytes_moved": 2 * nbytes, "ms": round(ms, 4), "gbps": round(2 * nbytes / (ms * 1e-3) / 1e9, 1),
           "what": "torch copy of 1 GiB (read + write), median of 5"}
    if lib is not None:
        ms_c = timed(lambda: check(lib.stream_ref_copy(a.data_ptr(), b.data_ptr(), nbytes, stream)))
        ms_r = timed(lambda: check(lib.stream_ref_read(a.data_ptr(), nbytes, sink.data_ptr(), stream)))
        out["stream_copy_gbps"] = round(2 * nbytes / (ms_c * 1e-3) / 1e9, 1)
        out["stream_read_gbps"] = round(nbytes / (ms_r * 1e-3) / 1e9, 1)
        out["stream_what"] = ("reference kernels (libstream_ref.so): copy of 1 GiB (read + write) and read of "
                              "1 GiB, 16 bytes per thread, streaming loads and stores, median of 5")
    del a, b
    torch.cuda.empty_cache()
    return out


def run_fleet(args, rs, torch, dev, cpu):
    from workloads import fleet_ids, fleet_module_shapes
    key = args.config
    T, n = 4096, 1024
    ids_np = fleet_ids(T, n)
    ids = torch.from_numpy(ids_np).to(dev)
    shapes = fleet_module_shapes()
    xs, ys = fleet_inputs(torch, dev, shapes, T)
    res = run_fleet_key(args, rs, torch, dev, key, xs, ys, ids, full=True)
    other = None
    if key == "5S" and not args.no_5u:
        u = run_fleet_key(args, rs, torch, dev, "5U", xs, ys, ids, full=False)
        other = {"workload": WORKLOAD_NAMES["5U"], "ms_per_step": round(u["ms_per_step"], 5),
                 "median_ms": u["timing"]["median_ms"], "p10_ms": u["timing"]["p10_ms"],
                 "p90_ms": u["timing"]["p90_ms"], "tokens_per_s": round(u["tokens_per_s"], 1),
                 "bytes_per_step": u["bytes_per_step"], "gbps": round(u["gbps"], 1),
                 "hbm_frac": round(u["gbps"] / PEAK_GBPS, 4)}
    ms = res["ms_per_step"]
    out = {
        "metric": METRIC, "value": round(res["tokens_per_s"], 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded Zipf(1.1) ids; factors, activations and y0 drawn on the GPU, bf16",
        "config": {"workload": WORKLOAD_NAMES[key], "T": T, "n_adapters": n, "modules": len(shapes),
                   "ranks_sum_per_module_mean": res["ranks_sum_per_module_mean"],
                   "timing": "each step streams ~50 GB from HBM (200x the last-level cache); one HIP-graph "
                             "replay per step, events around each"},
        "timing": res["timing"],
        "gbps": round(res["gbps"], 1), "hbm_frac": round(res["gbps"] / PEAK_GBPS, 4),
        "bytes_per_step": res["bytes_per_step"], "roofline": res.get("roofline"), "cpu_baseline": cpu,
        "kernels": res.get("kernels"), "padded": res.get("padded", {}), "multi_slice": res.get("multi_slice", {}),
        "fleet_5U": other, "base_fused": res.get("base_fused"), "copy_reference": copy_reference(torch, dev),
        "streams": max(1, args.streams),
        "wall_s_timed": round(res["wall_s"], 6),
        "timed_as": "eager launches" if args.no_graph else "HIP-graph replays of one captured step",
        "kernel_sources_sha": kernel_source_digest(),
    }
    print(json.dumps(out), flush=True)


def cpu_for(args, key):
    """The CPU-oracle leg of the bench line (before the GPU is touched)."""
    if args.no_cpu_baseline:
        return None
    if key in ("5U", "5S"):
        from workloads import make_fleet_module
        wl = make_fleet_module(key, 0, 0)
        return cpu_oracle(wl.x, wl.ids, wl.module.A, wl.module.B, wl.module.scales, args.cpu_seconds, 32, 196,
                          "tokens of the step's module L0.q (3584->3584)")
    wl = build_workload(key)
    per = min(wl.T, 64)
    return cpu_oracle(wl.x, wl.ids, wl.module.A, wl.module.B, wl.module.scales, args.cpu_seconds, per, 1,
                      "tokens of the same workload")


def main():
    args = parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
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
    key = args.config
    cpu = cpu_for(args, key) if key in ("1", "2", "3", "4", "5U", "5S") else None
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
    if key in ("5U", "5S"):
        run_fleet(args, rs, torch, dev, cpu)
    elif key == "fused":
        run_fused_only(args, rs, torch, dev)
    elif key.startswith("jd-"):
        run_jd(args, rs, torch, dev, key)
    elif key.startswith("rsvd-"):
        run_rsvd(args, rs, torch, dev, key)
    else:
        run_config(args, rs, torch, dev, key, cpu)


if __name__ == "__main__":
    main()
