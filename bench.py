#!/usr/bin/env python3
"""Throughput of the BitLinear forward path on one MI355X, on all five
synthetic workloads (Qwen3-0.6B and Gemma3-270M shapes).

Headline (the line's "value"): decode, M = 1, through the seven BitLinears of
a Qwen3-0.6B-shaped layer (q 1024->2048, k/v 1024->1024, o 2048->1024,
gate/up 1024->3072, down 3072->1024), in weight GB/s (packed I2_S bytes
streamed per second).  One layer is 3.93 MB, far below a kernel launch and
below the 256 MB MALL, so the step runs R distinct seeded copies of the layer
(R * 3.93 MB >= 1 GiB) as one group: the weights come from HBM, not from a
cache, and launch latency is amortised.  A step is the whole path for every
copy: RMSNorm + int8 quantization, the ternary product and the scale
epilogue, which at M = 1 run as one fused launch.

Also measured, each with its roofline and the oracle timed on the host:
  * "single_m8": one BitLinear 1024->3072 at M = 8 (per-call latency);
  * "gemma3_layer_m512": the seven Gemma3-270M projections at M = 512;
  * "prefill": the 28-layer Qwen3-0.6B projection stack at M = 16384 (196
    BitLinears), int8-equivalent TOPS, plus each shape's product alone;
  * "long_context_m32768": gate/up/down at M = 32768 with heavy-tailed
    activations, with the code-flip rate against the oracle;
  * the FFN glue and device-side packing.
Warm-up: the W steps asked for, then more until the GPU has run for at least
--min-warmup-ms (its clock settles), before every timed region.  Per-launch
durations come from HIP events on the stream the kernels run on and are
reported as mean, median, p10 and p90.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--skip-prefill] [--skip-cpu]
                    [--library-reference]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from ternary_weight_amd import inputs  # noqa: E402

METRIC = "ternary GEMM int8-eq TOPS (prefill) + GEMV weight GB/s (M=1), Qwen3-0.6B shapes"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA
DECODE_BYTES_TARGET = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # 500 decode steps (about 0.1 s): with 100 the fixed cost of starting and
    # draining the timed region moved the wall-clock step by up to 3%.
    ap.add_argument("--steps", type=int, default=500)
    # A short warmup leaves the first timed steps slow (the decode step then
    # measured 0.229 ms against 0.204 ms later in the same process).
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--replicas", type=int, default=0, help="decode layer copies (0 = enough for 1 GiB)")
    ap.add_argument("--skip-prefill", action="store_true")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--skip-variants", action="store_true",
                    help="skip the no-norm and float16-norm repeats (profiling runs)")
    ap.add_argument("--cpu-seconds", type=float, default=4.0,
                    help="single-core oracle time per workload (the all-core leg takes about as long)")
    # The GPU clock needs tens of milliseconds of load to settle: with 5
    # warmup steps (1 ms) the decode launch measured 203 us against 196 us.
    ap.add_argument("--min-warmup-ms", type=float, default=300.0)
    ap.add_argument("--library-reference", action="store_true",
                    help="also time the platform's int8 GEMM (torch._int_mm, hipBLASLt) on the stack's "
                         "shapes, as context for the prefill GEMM's rate (not part of the path)")
    return ap.parse_args()


# ------------------------------------------------------------ input prep ---

def _affinity() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def _threads() -> int:
    """Host threads for the oracle: every core this process may run on,
    capped by OMP_NUM_THREADS when the environment sets it (the host's CPU
    share per GPU)."""
    n = _affinity()
    cap = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(n, int(cap))) if cap.isdigit() and int(cap) > 0 else n


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def stats(values) -> dict:
    """mean, median, p10 and p90 of a list of durations (same unit)."""
    a = np.asarray(values, np.float64)
    return {"mean": float(a.mean()), "median": float(np.median(a)),
            "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90)), "n": int(a.size)}


def make_projections(workload: int, layers: int, projs, pack) -> list:
    """Seeded weights and norm weights of every (layer, proj), packed; in parallel."""
    def one(job):
        layer, pi, K, N = job
        packed, scale = pack(inputs.weight(workload, layer, pi, N, K))
        return dict(layer=layer, proj=pi, K=K, N=N, packed=packed, scale=scale,
                    norm_w=inputs.norm_weight(workload, layer, pi, K))
    jobs = [(layer, pi, K, N) for layer in range(layers) for pi, (_, K, N) in enumerate(projs)]
    with cf.ThreadPoolExecutor(_threads()) as ex:
        return list(ex.map(one, jobs))


class Arena:
    """Sub-allocates 256-byte-aligned views from one device buffer."""

    def __init__(self, torch, nbytes: int, device):
        self.torch = torch
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.off = 0

    @staticmethod
    def size(nbytes: int) -> int:
        return (nbytes + 255) // 256 * 256

    def take(self, nbytes: int, dtype, shape):
        view = self.buf[self.off:self.off + nbytes].view(dtype).view(shape)
        self.off += self.size(nbytes)
        return view


# -------------------------------------------------------------- timing ---

def warm_up(torch, step, warmup: int, min_ms: float) -> int:
    """The `warmup` steps asked for, then more (in tens) until the GPU has
    been busy for at least `min_ms` of wall time.  Returns the steps run."""
    t0 = time.perf_counter()
    n = 0
    for _ in range(warmup):
        step()
        n += 1
    torch.cuda.synchronize()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(10):
            step()
            n += 1
        torch.cuda.synchronize()
    return n


def time_steps(torch, step, steps: int, warmup: int, min_warm_ms: float):
    """Warm up, then time exactly `steps` steps.

    The timed region is bracketed by synchronisations and holds nothing but
    the steps: a timing event recorded between two steps makes the second
    kernel wait for the first one's completion signal and costs several
    microseconds per step.  A second pass records one pair of HIP events
    around the same number of steps (on the current stream, where the steps
    start and end) as a device-side cross-check.  Returns the wall-clock ms
    per step, the events' ms per step and the warm-up steps run.
    """
    stream = torch.cuda.current_stream()
    warm = warm_up(torch, step, warmup, min_warm_ms)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    return wall * 1e3 / steps, a.elapsed_time(b) / steps, warm


def time_launches(torch, group, steps: int):
    """The forward as individual launches in order on the current stream,
    HIP events around each (recorded on the stream the kernels run on), over
    `steps` repetitions: the launch list and, per launch, the list of its
    durations in ms (one per repetition)."""
    stream = torch.cuda.current_stream()
    info = group.forward_launches()
    nl = len(info)
    for i in range(nl):
        group.forward_launch(i)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nl + 1)] for _ in range(steps)]
    for e in ev:
        e[0].record(stream)
        for i in range(nl):
            group.forward_launch(i)
            e[i + 1].record(stream)
    torch.cuda.synchronize()
    launch_ms = [[e[i].elapsed_time(e[i + 1]) for e in ev] for i in range(nl)]
    return info, launch_ms


def time_calls(torch, call, reps: int, warmup: int, min_warm_ms: float):
    """A single call repeated: warm up, then `reps` back-to-back calls
    between one pair of events (mean ms), then `reps` calls each between its
    own pair (the distribution)."""
    stream = torch.cuda.current_stream()
    warm_up(torch, call, warmup, min_warm_ms)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        call()
        e1.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps, [e0.elapsed_time(e1) for e0, e1 in ev]


def us_stats(ms_list) -> dict:
    return {k: (round(v * 1e3, 2) if k != "n" else v) for k, v in stats(ms_list).items()}


def launch_bytes(kind: str, M: int, K: int, N: int, norm=True) -> int:
    """Algorithmic HBM bytes of one BitLinear in a launch of the given kind
    (norm False: a projection without a norm weight, which is not read;
    "f16": a float16 norm weight)."""
    nw = {True: 4 * K, "f16": 2 * K, False: 0}[norm]
    if kind in ("decode", "prefill"):  # packed weights, int8 codes, factor + row sum, fp32 y
        return N * K // 4 + M * K + 8 * M + 4 * M * N
    if kind == "decode_fused":   # packed weights, fp32 x and norm weight, fp32 y
        return N * K // 4 + 4 * M * K + nw + 4 * M * N
    if kind == "quant":          # fp32 x and norm weight in, int8 codes, factor + row sum out
        return 4 * M * K + nw + M * K + 8 * M
    raise ValueError(kind)


def profile_value(name: str, field: str, source: str):
    """A number recorded in a committed rocprofv3 summary (profiles/<name>.md),
    or None when the summary is missing or the kernel source changed since it
    was taken (the summary names the source's sha256)."""
    path = os.path.join(ROOT, "profiles", f"{name}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_v = re.search(field + r":\s*([0-9.eE+-]+)", text)
    if not (m_sha and m_v):
        return None
    src = open(os.path.join(ROOT, "ternary_weight_amd", "csrc", source), "rb").read()
    if hashlib.sha256(src).hexdigest() != m_sha.group(1):
        return None
    return float(m_v.group(1))


def traffic_from_profiles(kernel_tag: str, source: str):
    """HBM bytes per launch from a committed rocprofv3 PMC summary, or None.

    The summary names the kernel source's sha256; a changed kernel makes the
    counters stale and the figure is dropped.
    """
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_sha and m_b):
        return None
    src = open(os.path.join(ROOT, "ternary_weight_amd", "csrc", source), "rb").read()
    if hashlib.sha256(src).hexdigest() != m_sha.group(1):
        return None
    return float(m_b.group(1))


# ------------------------------------------------------------- workloads ---

def bench_decode(torch, bl, args):
    w = inputs.WORKLOADS[2]
    layer_bytes = sum(N * K // 4 for _, K, N in w.projs)
    R = args.replicas or math.ceil(DECODE_BYTES_TARGET / layer_bytes)
    t0 = time.time()
    projs = make_projections(2, R, w.projs, bl.i2s_pack)
    log(f"decode: {len(projs)} BitLinears prepared in {time.time() - t0:.1f}s")
    dev = torch.device("cuda")
    sz = Arena.size
    # Each BitLinear's packed weights, norm weight and x sit together in one
    # buffer; the outputs y in another.  Outputs interleaved with the weights
    # put the step's writes into the DRAM rows the weight streams read, and
    # the decode launch then ran 3.5% slower (203.8 against 196.9 us).
    total = sum(sz(len(p["packed"])) + sz(4 * p["K"]) * 2 for p in projs)
    arena = Arena(torch, total, dev)
    yarena = Arena(torch, sum(sz(4 * p["N"]) for p in projs), dev)
    items = []
    for p in projs:
        K, N = p["K"], p["N"]
        pw = arena.take(len(p["packed"]), torch.uint8, (len(p["packed"]),))
        pw.copy_(torch.from_numpy(p["packed"]))
        nw = arena.take(4 * K, torch.float32, (K,))
        nw.copy_(torch.from_numpy(p["norm_w"]))
        x = arena.take(4 * K, torch.float32, (1, K))
        x.copy_(torch.from_numpy(inputs.activations(2, p["layer"], p["proj"], 1, K)))
        y = yarena.take(4 * N, torch.float32, (1, N))
        items.append(dict(x=x, norm_w=nw, packed_w=pw, w_scale=p["scale"], eps=inputs.EPS, N=N, y=y))
    weight_bytes = sum(p["N"] * p["K"] // 4 for p in projs)

    def run(items, norm):
        group = bl.Group(items)
        ms, ms_events, warm = time_steps(torch, group.forward, args.steps, args.warmup,
                                         args.min_warmup_ms)
        info, launch_ms = time_launches(torch, group, args.steps)
        group.close()
        # Algorithmic bytes per launch (launch_bytes, M = 1): the quantization
        # launch when there is one, then one decode launch per superblock
        # count ceil(K/256) (bucket 0: every K in one merged launch).
        per_launch = []
        for d, t in zip(info, launch_ms):
            members = [p for p in projs if (p["K"] + 255) // 256 == d["bucket"]] if d["bucket"] else projs
            nbytes = sum(launch_bytes(d["kind"], 1, p["K"], p["N"], norm) for p in members)
            mean = float(np.mean(t))
            per_launch.append(dict(kind=d["kind"], bucket=d["bucket"], bitlinears=len(members),
                                   K="/".join(str(k) for k in sorted({p["K"] for p in members})),
                                   bytes=nbytes, us=mean * 1e3, us_stats=us_stats(t),
                                   GBps=nbytes / (mean * 1e-3) / 1e9))
        dom = max(per_launch, key=lambda d: d["bytes"])
        step_ms = np.sum(np.asarray(launch_ms), axis=0)
        return dict(ms=ms, ms_events=ms_events, warm=warm, per_launch=per_launch, dominant=dom,
                    step_us_stats=us_stats(step_ms), value=weight_bytes / (ms * 1e-3) / 1e9)

    out = run(items, True)
    # the same step with projections that have no norm weight of their own
    if not args.skip_variants:
        out["no_norm"] = run([dict(it, norm_w=None) for it in items], False)
        # and with float16 norm weights (the pages' stored dtype for norms)
        out["f16_norm"] = run([dict(it, norm_w=it["norm_w"].half()) for it in items], "f16")
    out.update(R=R, projs=projs, weight_bytes=weight_bytes)
    return out


def quant_bytes_by_launch(M: int, projs) -> dict:
    """Algorithmic bytes of each quantization launch, keyed (kind, chunk
    count): a share set (projections reading one x) reads x once and writes
    each member's codes, factor and row sum; a set of P members at K reads
    4MK + 4PK (norm weights) and writes P(MK + 8M).  Sets go to launches by
    chunk count ceil(K/256) and by sharing."""
    sets = {}
    for p in projs:
        sets.setdefault(p["xkey"], []).append(p)
    out = {}
    for members in sets.values():
        K = members[0]["K"]
        key = ("quant_shared" if len(members) > 1 else "quant", (K + 255) // 256)
        P = len(members)
        out[key] = out.get(key, 0) + 4 * M * K + 4 * P * K + P * (M * K + 8 * M)
    return out


def run_prefill_group(torch, bl, items, projs, M, args, steps):
    """A group whose forward is quantization launches then one prefill
    launch: step timing, per-launch duration statistics, the quantization
    launches' bandwidth and the prefill launch's int8-equivalent rate."""
    group = bl.Group(items)
    ms, ms_events, warm = time_steps(torch, group.forward, steps, max(1, args.warmup // 2),
                                     args.min_warmup_ms)
    info, launch_ms = time_launches(torch, group, steps)
    group.close()
    assert [d["kind"] for d in info][-1] == "prefill" and all(
        d["kind"].startswith("quant") for d in info[:-1]), info
    qbytes = quant_bytes_by_launch(M, projs)
    quant_launches = []
    for d, t in zip(info[:-1], launch_ms[:-1]):
        # a merged launch (small groups) does every set's work
        nb = sum(qbytes.values()) if d["kind"] == "quant_merged" else qbytes.get((d["kind"], d["bucket"]))
        mean = float(np.mean(t))
        quant_launches.append(dict(kind=d["kind"], chunks=d["bucket"], bitlinears=d["count"],
                                   us=round(mean * 1e3, 1), us_stats=us_stats(t), bytes=nb,
                                   GBps=round(nb / (mean * 1e-3) / 1e9, 1) if nb else None))
    quant_ms = float(np.sum(np.mean(np.asarray(launch_ms[:-1]), axis=1))) if len(info) > 1 else 0.0
    mm = launch_ms[-1]
    mm_ms = float(np.mean(mm))
    ops = sum(2 * M * p["N"] * p["K"] for p in projs)
    gemm_bytes = sum(M * p["K"] + p["N"] * p["K"] // 4 + 8 * M + 4 * M * p["N"] for p in projs)
    return dict(ms=ms, ms_events=ms_events, warm=warm, quant_ms=quant_ms, mm_ms=mm_ms,
                mm_us_stats=us_stats(mm), ops=ops, gemm_bytes=gemm_bytes,
                quant_launches=quant_launches, tops=ops / (ms * 1e-3) / 1e12,
                mm_tops=ops / (mm_ms * 1e-3) / 1e12,
                step_us_stats=us_stats(np.sum(np.asarray(launch_ms), axis=0)))


def prefill_items(torch, projs, xs, M, dev):
    return [dict(x=xs[p["xkey"]], norm_w=torch.from_numpy(p["norm_w"]).to(dev),
                 packed_w=torch.from_numpy(p["packed"]).to(dev), w_scale=p["scale"],
                 eps=inputs.EPS, N=p["N"], y=torch.empty((M, p["N"]), dtype=torch.float32, device=dev))
            for p in projs]


def mfma_roofline(r: dict, peaks: dict, kernel: str, counters=None) -> dict:
    out = {"bound": "mfma", "kernel": kernel,
           "achieved": round(r["mm_tops"], 1), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
           "frac": round(r["mm_tops"] / INT8_PEAK_TOPS, 4), "traffic": None,
           "algorithmic_ops_per_launch": r["ops"], "avg_launch_us": round(r["mm_ms"] * 1e3, 1),
           "launch_us_stats": r["mm_us_stats"],
           "frac_of_measured": round(r["mm_tops"] / peaks["mfma_i8_TOPS"], 4)}
    if counters:
        out.update(counters)
    return out


def bench_prefill(torch, bl, args):
    """The 28-layer Qwen3-0.6B stack at M = 16384 (196 BitLinears) as one
    group, then each projection shape of the stack as its own group of 28
    (one prefill launch per shape: per-shape rates)."""
    w = inputs.WORKLOADS[4]
    t0 = time.time()
    projs = make_projections(4, w.layers, w.projs, bl.i2s_pack)
    log(f"prefill: {len(projs)} BitLinears prepared in {time.time() - t0:.1f}s")
    dev = torch.device("cuda")
    # Each layer has its own inputs (drawn on the device); within a layer q, k
    # and v read one input and gate and up another, as in the model.
    xs = {}
    names = [name for name, _, _ in w.projs]
    for p in projs:
        key = (p["layer"], inputs.SHARED_INPUT[names[p["proj"]]])
        if key not in xs:
            xs[key] = inputs.activations_device(torch, 4, key[0], key[1], w.M, p["K"], dev)
        p["xkey"] = key
    torch.cuda.synchronize()
    items = prefill_items(torch, projs, xs, w.M, dev)
    steps = prefill_steps(args)
    r = run_prefill_group(torch, bl, items, projs, w.M, args, steps)
    nn_quant_ms = f16_quant_ms = None
    if not args.skip_variants:
        # the quantization stage for projections without a norm weight
        group = bl.Group([dict(it, norm_w=None) for it in items])
        _, nn_ms = time_launches(torch, group, steps)
        group.close()
        nn_quant_ms = float(np.sum(np.mean(np.asarray(nn_ms[:-1]), axis=1)))
        group = bl.Group([dict(it, norm_w=it["norm_w"].half()) for it in items])
        _, h_ms = time_launches(torch, group, steps)
        group.close()
        f16_quant_ms = float(np.sum(np.mean(np.asarray(h_ms[:-1]), axis=1)))
    # Each shape alone: the 28 layers' projections of one name, one launch
    # each for quantization and product (q/k/v and gate/up then do not share
    # their input's pass).
    per_shape = []
    for pi, (name, K, N) in enumerate(w.projs):
        sel = [i for i, p in enumerate(projs) if p["proj"] == pi]
        rs = run_prefill_group(torch, bl, [items[i] for i in sel],
                               [dict(projs[i], xkey=(i,)) for i in sel], w.M, args,
                               max(3, steps // 2))
        per_shape.append({"proj": name, "K": K, "N": N, "bitlinears": len(sel),
                          "gemm_us": round(rs["mm_ms"] * 1e3, 1), "gemm_us_stats": rs["mm_us_stats"],
                          "gemm_TOPS": round(rs["mm_tops"], 1),
                          "frac_of_peak": round(rs["mm_tops"] / INT8_PEAK_TOPS, 4),
                          "gemm_bytes_GBps": round(rs["gemm_bytes"] / (rs["mm_ms"] * 1e-3) / 1e9, 1),
                          "quant_GBps": rs["quant_launches"][0]["GBps"]})
        log(f"prefill shape {name} {K}->{N} x28: GEMM {rs['mm_ms'] * 1e3:.1f} us "
            f"({rs['mm_tops']:.0f} TOPS)")
    r.update(projs=projs, xs=xs, M=w.M, no_norm_quant_ms=nn_quant_ms, f16_quant_ms=f16_quant_ms,
             per_shape=per_shape, steps=steps)
    return r


def bench_gemma_layer(torch, bl, args):
    """The seven Gemma3-270M projections at M = 512 (q, k, v read one input,
    gate and up another, as in the model) as one group forward."""
    w = inputs.WORKLOADS[3]
    projs = make_projections(3, w.layers, w.projs, bl.i2s_pack)
    dev = torch.device("cuda")
    names = [name for name, _, _ in w.projs]
    xs, xs_host = {}, {}
    for p in projs:
        key = (0, inputs.SHARED_INPUT[names[p["proj"]]])
        if key not in xs:
            xs_host[key] = inputs.activations(3, 0, key[1], w.M, p["K"])
            xs[key] = torch.from_numpy(xs_host[key]).to(dev)
        p["xkey"] = key
    items = prefill_items(torch, projs, xs, w.M, dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    splits = bl.prefill_splits(items, cus)
    r = run_prefill_group(torch, bl, items, projs, w.M, args, args.steps)
    r.update(projs=projs, xs_host=xs_host, M=w.M, cus=cus,
             splits={names[p["proj"]]: s for p, s in zip(projs, splits)})
    return r


def bench_long_context(torch, bl, args):
    """Gate, up and down at M = 32768 with heavy-tailed activations (Student-t,
    3 degrees of freedom, 0.1% of the channels x20): gate and up read one
    input, down its own.  One group forward; the GPU codes of the long rows
    are kept for the code-flip rate against the oracle."""
    w = inputs.WORKLOADS[5]
    projs = make_projections(5, w.layers, w.projs, bl.i2s_pack)
    dev = torch.device("cuda")
    names = [name for name, _, _ in w.projs]
    xs, xs_host = {}, {}
    for p in projs:
        key = (0, inputs.SHARED_INPUT[names[p["proj"]]])
        if key not in xs:
            xs_host[key] = inputs.activations(5, 0, key[1], w.M, p["K"], heavy_tail=True)
            xs[key] = torch.from_numpy(xs_host[key]).to(dev)
        p["xkey"] = key
    items = prefill_items(torch, projs, xs, w.M, dev)
    r = run_prefill_group(torch, bl, items, projs, w.M, args, prefill_steps(args))
    rows = inputs.sample_rows(w.M, 64, seed=5)
    idx = torch.as_tensor(rows, device=dev)
    codes = []
    for p, it in zip(projs, items):
        xq, _ = bl.bitlinear_quant(it["x"], it["norm_w"], inputs.EPS)
        codes.append(xq[idx].cpu().numpy())
    r.update(projs=projs, xs_host=xs_host, M=w.M, rows=rows, gpu_codes=codes)
    return r


def bench_single_m8(torch, bl, args, floor_us: float):
    """One BitLinear 1024 -> 3072 at M = 8: the per-call latency of
    bitlinear_forward (quantization launch + decode launch)."""
    w = inputs.WORKLOADS[1]
    (name, K, N), M = w.projs[0], w.M
    dev = torch.device("cuda")
    packed, scale = bl.i2s_pack(inputs.weight(1, 0, 0, N, K))
    x_host = inputs.activations(1, 0, 0, M, K)
    nw_host = inputs.norm_weight(1, 0, 0, K)
    x, nw = torch.from_numpy(x_host).to(dev), torch.from_numpy(nw_host).to(dev)
    pw = torch.from_numpy(packed).to(dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    call = lambda: bl.bitlinear_forward(x, nw, pw, scale, N, inputs.EPS, y=y)
    mean_ms, per_call = time_calls(torch, call, max(50, args.steps), args.warmup, args.min_warmup_ms)
    st = us_stats(per_call)
    nbytes = N * K // 4 + 4 * M * K + 4 * K + 4 * M * N
    return dict(M=M, K=K, N=N, packed=packed, x_host=x_host, nw_host=nw_host,
                back_to_back_us=mean_ms * 1e3, per_call_us=st, bytes=nbytes,
                weight_GBps=(N * K // 4) / (st["median"] * 1e-6) / 1e9,
                GBps=nbytes / (st["median"] * 1e-6) / 1e9, floor_us=floor_us)


def prefill_steps(args) -> int:
    """Steps of the prefill-sized measurements (13 ms each): half the decode
    steps, between 3 and 50."""
    return max(3, min(50, args.steps // 2))


def bench_prefill_fused(torch, bl, args):
    """One BitLinear per call at M = 16384 for each Qwen3-0.6B shape: the
    forward as quantization launch + tiled product (bitlinear_forward) against
    the forward whose product quantizes in its producer (statistics launch +
    tiled product reading fp32 rows; bitlinear_forward_prefill_fused).  Same
    outputs bit for bit (checked here on every shape)."""
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(23)
    M = 16384
    res = {}
    for name, K, N in (("q", 1024, 2048), ("k", 1024, 1024), ("o", 2048, 1024),
                       ("gate", 1024, 3072), ("down", 3072, 1024)):
        w = torch.randn((N, K), generator=g, device=dev) * 0.02
        pw, scale = bl.i2s_pack_device(w)
        del w
        x = torch.randn((M, K), generator=g, device=dev)
        nw = 1.0 + 0.1 * torch.randn((K,), generator=g, device=dev)
        y1 = torch.empty((M, N), device=dev)
        y2 = torch.empty((M, N), device=dev)
        t1, _ = time_calls(torch, lambda: bl.bitlinear_forward(x, nw, pw, scale, N, inputs.EPS, y=y1),
                           20, 5, 100.0)
        t2, _ = time_calls(torch, lambda: bl.bitlinear_forward_prefill_fused(x, nw, pw, scale, N, inputs.EPS, y=y2),
                           20, 5, 100.0)
        torch.cuda.synchronize()
        same = bool(torch.equal(y1, y2))
        ops = 2 * M * N * K
        res[name] = {"K": K, "N": N, "forward_us": round(t1 * 1e3, 1), "fused_producer_us": round(t2 * 1e3, 1),
                     "forward_TOPS": round(ops / t1 / 1e9, 1), "fused_producer_TOPS": round(ops / t2 / 1e9, 1),
                     "forward_frac": round(ops / t1 / 1e9 / INT8_PEAK_TOPS, 4),
                     "fused_producer_frac": round(ops / t2 / 1e9 / INT8_PEAK_TOPS, 4),
                     "fused_over_forward": round(t2 / t1, 3), "bit_identical": same}
        del x, nw, pw, y1, y2
    return {"workload": "one BitLinear per call at M=16384, Qwen3-0.6B shapes: bitlinear_forward "
                        "(quantization launch + product) against bitlinear_forward_prefill_fused "
                        "(statistics launch + product whose producer quantizes fp32 rows)",
            "per_shape": res,
            "roofline": {"bound": "mfma", "kernel": "quant_stats_kernel + gemm_kernel<PQ> (one call per shape)",
                         "achieved": round(max(v["fused_producer_TOPS"] for v in res.values()), 1),
                         "peak": INT8_PEAK_TOPS, "unit": "TOPS",
                         "frac": round(max(v["fused_producer_frac"] for v in res.values()), 4),
                         "note": "best shape; whole calls (statistics launch + product), per shape in per_shape"}}


def bench_ffn_glue(torch, bl, args):
    """The Qwen3 FFN down projection fed by the glue act(gate) * up at the
    prefill size (M = 16384, K = 3072 -> N = 1024, SiLU): the fused glue +
    quantization kernel (act(gate) * up formed in registers, never stored)
    against its HBM roofline, and the whole glue-fed forward."""
    M, K, N = 16384, 3072, 1024
    dev = torch.device("cuda")
    gate = inputs.activations_device(torch, 4, 0, 100, M, K, dev)
    up = inputs.activations_device(torch, 4, 0, 101, M, K, dev)
    nw = torch.from_numpy(inputs.norm_weight(4, 0, 6, K)).to(dev)
    packed, scale = bl.i2s_pack(inputs.weight(4, 0, 6, N, K))
    pw = torch.from_numpy(packed).to(dev)
    xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    f = torch.empty((M,), dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)

    def timed(fn, reps):
        warm_up(torch, fn, max(1, args.warmup // 2), args.min_warmup_ms / 2)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps
    reps = prefill_steps(args)
    q_ms = timed(lambda: bl.bitlinear_glu_quant(gate, up, bl.ACT_SILU, nw, inputs.EPS, xq=xq, x_factor=f), reps)
    fwd_ms = timed(lambda: bl.bitlinear_glu_forward(gate, up, bl.ACT_SILU, nw, pw, scale, N, inputs.EPS, y=y), reps)
    q_bytes = 8 * M * K + M * K + 8 * M + 4 * K     # gate + up in, codes + factor + row sum out
    unfused = q_bytes + 8 * M * K                     # the product written and read back in fp32
    # Decode size (M = 1): glue, RMSNorm, quantization and the product in the
    # one fused decode launch, no workspace.
    g1, u1, y1 = gate[:1].contiguous(), up[:1].contiguous(), y[:1].contiguous()
    dec_us = 1e3 * timed(lambda: bl.bitlinear_glu_forward(g1, u1, bl.ACT_SILU, nw, pw, scale, N, inputs.EPS,
                                                          y=y1), reps)
    dec_bytes = N * K // 4 + 8 * K + 4 * K + 4 * N
    return {
        "workload": f"Qwen3 FFN down projection fed by SiLU(gate)*up, M={M}, K={K} -> N={N}",
        "glue_quant_us": round(q_ms * 1e3, 1),
        "roofline": {"bound": "hbm", "kernel": "quant_reg_kernel<12, SiLU> (glue + RMSNorm + int8)",
                     "achieved": round(q_bytes / (q_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(q_bytes / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes_per_launch": q_bytes},
        "bytes_saved_vs_storing_the_product": round(1 - q_bytes / unfused, 3),
        "forward_ms": round(fwd_ms, 4),
        "forward_TOPS": round(2 * M * N * K / (fwd_ms * 1e-3) / 1e12, 1),
        "decode_M1_forward_us": round(dec_us, 2),
        "decode_M1_GBs": round(dec_bytes / (dec_us * 1e-6) / 1e9, 1),
    }


def bench_device_pack(torch, bl, args):
    """i2s_pack_device on a [16384, 4096] float32 weight (268 MB, beyond the
    MALL): absmean reduction + packing against the HBM roofline.  Algorithmic
    bytes: the weights read twice (reduction, packing) and the codes written
    once, 8.25 bytes per weight."""
    N, K = 16384, 4096
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(20)
    w = torch.randn((N, K), generator=g, device=dev) * 0.02
    packed = torch.empty((bl.i2s_packed_bytes(K, N),), dtype=torch.uint8, device=dev)
    reps = max(3, args.steps // 5)
    warm_up(torch, lambda: bl.i2s_pack_device(w, packed, read_scale=False), max(1, args.warmup // 10),
            args.min_warmup_ms / 2)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        bl.i2s_pack_device(w, packed, read_scale=False)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    nbytes = 8 * N * K + N * K // 4 + 4
    return {"workload": f"device-side absmean + I2_S packing of a [{N}, {K}] float32 weight",
            "us": round(ms * 1e3, 1),
            "roofline": {"bound": "hbm", "kernels": "absmean_partial_kernel + absmean_final_kernel + "
                         "i2s_pack_kernel", "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes_per_call": nbytes}}


def library_reference(torch) -> dict:
    """The platform library's int8 GEMM on the Qwen3-0.6B stack shapes at
    M = 16384, as context for the prefill GEMM: torch._int_mm (int8 x int8 ->
    int32, hipBLASLt) with plain int8 weights (four times the packed bytes, no
    unpacking, no scale epilogue), one product per call, B column-major (the
    faster of its two layouts here).  Not part of the path."""
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    M = 16384
    res = {}
    for name, K, N in (("q", 1024, 2048), ("k", 1024, 1024), ("o", 2048, 1024),
                       ("gate", 1024, 3072), ("down", 3072, 1024)):
        a = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev, generator=g)
        b = torch.randint(-1, 2, (N, K), dtype=torch.int8, device=dev, generator=g).t()
        call = lambda: torch._int_mm(a, b)
        mean_ms, _ = time_calls(torch, call, 30, 5, 200.0)
        us = mean_ms * 1e3
        ops = 2 * M * N * K
        res[name] = {"K": K, "N": N, "us": round(us, 1), "TOPS": round(ops / us / 1e6, 1),
                     "frac": round(ops / us / 1e6 / INT8_PEAK_TOPS, 4)}
        del a, b
    return {"what": "torch._int_mm (hipBLASLt) int8 x int8 -> int32 on plain int8 weights, M=16384, "
                    "one GEMM per call; context only", "per_shape": res}


def measure_peaks(torch, bl):
    """Sustained HBM read / copy bandwidth and int8 MFMA rate of this GPU (probes)."""
    dev = torch.device("cuda")
    sink = torch.zeros(4, dtype=torch.int32, device=dev)

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    read = {}
    for blocks in (2048, 4096, 8192, 16384):
        read[blocks] = nbytes / timed(lambda: bl.probe_read(buf, sink, blocks)) / 1e9
    half = nbytes // 2
    src, dst = buf[:half], buf[half:]
    copy = max(2 * half / timed(lambda: bl.probe_copy(src, dst, b)) / 1e9 for b in (4096, 16384))
    write = {}
    for nt in (False, True):
        write[nt] = max(nbytes / timed(lambda: bl.probe_write(buf, b, nt)) / 1e9 for b in (4096, 16384))
    # reads with one 16-byte write per 64 (or 16) 16-byte reads: HBM under a
    # decode launch's kind of traffic (its outputs are about 1.2% of its bytes)
    mixed = {}
    msrc, mdst = buf[: nbytes // 2], buf[nbytes // 2: nbytes // 2 + (128 << 20)]
    for rd in (64, 16):
        moved = msrc.numel() * (1 + 1 / rd)
        mixed[rd] = max(moved / timed(lambda: bl.probe_mixed(msrc, mdst, rd, sink, b)) / 1e9 for b in (1024, 2048))
    # one write per 4, 2 or 1 reads (20%, 33%, 50% of the bytes written): the
    # quantization launches' mixes (fp32 rows in, int8 codes out: 20-43%)
    msrc, mdst = buf[: nbytes // 4], buf[nbytes // 2: 3 * nbytes // 4]
    for rd in (4, 2, 1):
        moved = msrc.numel() * (1 + 1 / rd)
        mixed[rd] = max(moved / timed(lambda: bl.probe_mixed(msrc, mdst, rd, sink, b)) / 1e9 for b in (1024, 2048))
    del buf, src, dst, msrc, mdst
    # Launch floor: back-to-back launches of a one-workgroup kernel that
    # writes 16 bytes (what any launch costs on this stream).
    tiny = torch.empty(256, dtype=torch.uint8, device=dev)
    for _ in range(20):
        bl.probe_write(tiny, 1)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(500):
        bl.probe_write(tiny, 1)
    e1.record()
    torch.cuda.synchronize()
    floor_us = e0.elapsed_time(e1) / 500 * 1e3
    iters, blocks = 4000, 256 * 8
    mfma = {}
    for shape in (16, 32):
        t = timed(lambda: bl.probe_mfma_i8(iters, blocks, sink, shape=shape), reps=3)
        mfma[shape] = blocks * 4 * iters * 131072 / t / 1e12
    return {"hbm_read_GBps": round(max(read.values()), 1),
            "hbm_read_by_blocks": {str(k): round(v, 1) for k, v in read.items()},
            "copy_GBps_read_plus_write": round(copy, 1),
            "hbm_write_GBps": round(max(write.values()), 1),
            "hbm_write_by_kind": {"plain": round(write[False], 1), "nontemporal": round(write[True], 1)},
            "hbm_mixed_GBps": {f"1_write_per_{rd}_reads": round(mixed[rd], 1) for rd in (64, 16, 4, 2, 1)},
            "launch_floor_us": round(floor_us, 2),
            "mfma_i8_TOPS": round(max(mfma.values()), 1),
            "mfma_i8_TOPS_by_shape": {f"{k}x{k}": round(v, 1) for k, v in mfma.items()}}


def _oracle_parallel(fn, jobs, threads: int):
    """Run fn on every job with `threads` host threads (the C oracle runs
    outside the GIL); returns the wall time."""
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(fn, jobs))
    return time.perf_counter() - t0


def host_info() -> dict:
    return {"cpu_model": cpu_model(), "cores_available": _affinity(),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def cpu_baseline_decode(projs, seconds: float):
    """The oracle, unchanged, on the BitLinears of the decode step: one host
    core on the first BitLinears (about `seconds`), then the host's cores,
    each thread running the single-threaded oracle on its own BitLinears."""
    import oracle
    jobs = []
    done_bytes, t_used, n = 0, 0.0, 0
    for p in projs:
        x = inputs.activations(2, p["layer"], p["proj"], 1, p["K"])
        jobs.append((x, p["norm_w"], p["packed"], p["N"]))
        t0 = time.perf_counter()
        oracle.bitlinear(x, p["norm_w"], p["packed"], p["N"], inputs.EPS)
        t_used += time.perf_counter() - t0
        done_bytes += p["N"] * p["K"] // 4
        n += 1
        if t_used >= seconds:
            break
    single = dict(value=done_bytes / t_used / 1e9, unit="GB/s", cores=1,
                  sample=f"first {n} of {len(projs)} BitLinears ({t_used:.1f} s)")
    P = _threads()
    m = min(len(projs), max(n, int(n * P * 0.9)))
    for p in projs[len(jobs):m]:
        jobs.append((inputs.activations(2, p["layer"], p["proj"], 1, p["K"]), p["norm_w"], p["packed"], p["N"]))
    wall = _oracle_parallel(lambda j: oracle.bitlinear(j[0], j[1], j[2], j[3], inputs.EPS), jobs[:m], P)
    nbytes = sum(p["N"] * p["K"] // 4 for p in projs[:m])
    return dict(value=nbytes / wall / 1e9, unit="GB/s", cores=P, kind="oracle",
                sample=f"first {m} of {len(projs)} M=1 BitLinears of the decode step "
                       f"({nbytes / 1e6:.0f} MB of packed weights), {P} threads each running the "
                       f"single-threaded oracle on its own BitLinears, {wall:.1f} s wall",
                single_core=single, host=host_info())


def cpu_baseline_rows(projs, x_rows, nrows: int, seconds: float, what: str):
    """The oracle, unchanged, on `nrows` token rows through the BitLinears
    (rows are independent, so the rate on sampled rows is the workload's):
    one core on the first BitLinears until about `seconds` have passed, then
    the host's cores, each thread running the single-threaded oracle on its
    own BitLinears.  x_rows(p): the host rows of p's input.  TOPS."""
    import oracle
    ops, t_used, n = 0, 0.0, 0
    for p in projs:
        t0 = time.perf_counter()
        oracle.bitlinear(x_rows(p), p["norm_w"], p["packed"], p["N"], inputs.EPS)
        t_used += time.perf_counter() - t0
        ops += 2 * nrows * p["N"] * p["K"]
        n += 1
        if t_used >= seconds:
            break
    single = dict(value=ops / t_used / 1e12, unit="TOPS", cores=1,
                  sample=f"{nrows} rows through the first {n} BitLinears ({t_used:.1f} s)")
    P = _threads()
    reps = max(1, -(-int(n * P * 0.9) // len(projs)))  # cycle over the BitLinears when few
    sel = (list(projs) * reps)[:max(n, min(len(projs) * reps, int(n * P * 0.9)))]
    wall = _oracle_parallel(lambda p: oracle.bitlinear(x_rows(p), p["norm_w"], p["packed"], p["N"],
                                                       inputs.EPS), sel, P)
    ops = sum(2 * nrows * p["N"] * p["K"] for p in sel)
    return dict(value=ops / wall / 1e12, unit="TOPS", cores=P, kind="oracle",
                sample=f"{nrows} {what} through {len(sel)} BitLinear calls ({len(projs)} distinct), "
                       f"{P} threads each running the single-threaded oracle on its own "
                       f"BitLinears, {wall:.1f} s wall",
                single_core=single, host=host_info())


def cpu_baseline_m8(w1, seconds: float):
    """The oracle on the whole M = 8 call, repeated: one core for about
    `seconds`, then the host's cores each repeating it."""
    import oracle
    call = lambda _: oracle.bitlinear(w1["x_host"], w1["nw_host"], w1["packed"], w1["N"], inputs.EPS)
    wbytes = w1["N"] * w1["K"] // 4
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        call(None)
        n += 1
    t1 = time.perf_counter() - t0
    single = dict(value=n * wbytes / t1 / 1e9, unit="GB/s", cores=1, sample=f"{n} calls ({t1:.1f} s)")
    P = _threads()
    m = max(n, int(n * P * 0.9))
    wall = _oracle_parallel(call, range(m), P)
    return dict(value=m * wbytes / wall / 1e9, unit="GB/s", cores=P, kind="oracle",
                sample=f"the whole M=8 call repeated {m} times on {P} threads (weight bytes "
                       f"per second), {wall:.1f} s wall",
                single_core=single, host=host_info())


def torch_rows(x, rows):
    import torch
    return torch.as_tensor(rows, device=x.device)


def code_flips(lc) -> dict:
    """Codes of the long-context rows: the GPU's (quantization kernel) against
    the oracle's, on the sampled rows; part of the oracle leg."""
    import oracle
    flips = total = worst = 0
    for p, q_gpu in zip(lc["projs"], lc["gpu_codes"]):
        q_ref, _ = oracle.quant(lc["xs_host"][p["xkey"]][lc["rows"]], p["norm_w"], inputs.EPS)
        d = np.abs(q_gpu.astype(np.int32) - q_ref.astype(np.int32))
        flips += int(np.count_nonzero(d))
        total += d.size
        worst = max(worst, int(d.max(initial=0)))
    return {"flips": flips, "codes": total, "rate": flips / total, "max_abs_diff": worst,
            "rows": len(lc["rows"])}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the path shards over token rows with no exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from ternary_weight_amd import bitlinear as bl
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    peaks = measure_peaks(torch, bl)
    log(f"measured peaks: {peaks}")
    dec = bench_decode(torch, bl, args)
    dom = dec["dominant"]
    log(f"decode: {dec['ms']:.3f} ms/step ({dec['ms_events']:.3f} by events), "
        f"{dec['value']:.0f} GB/s weights; launches: "
        + ", ".join(f"{d['kind']} K={d['K']} {d['us']:.1f} us {d['GBps']:.0f} GB/s"
                    for d in dec["per_launch"]))
    traffic = traffic_from_profiles("gemv_decode_merged", "gemv.hip")
    out = {
        "metric": METRIC,
        "value": round(dec["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": dec["warm"],
        "ms_per_step": round(dec["ms"], 5),
        "ms_per_step_events": round(dec["ms_events"], 5),
        "step_us_stats": dec["step_us_stats"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {
            "workload": f"decode M=1 through a Qwen3-0.6B-shaped layer (7 BitLinears), "
                        f"{dec['R']} distinct seeded layer copies per step (>= 1 GiB of I2_S weights)",
            "M": 1, "bitlinears": len(dec["projs"]), "layer_copies": dec["R"],
            "weight_bytes": dec["weight_bytes"], "parallelism": "single GPU",
            "step": "one group forward: one fused RMSNorm+quant+decode launch over every K "
                    "(longest units first)",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": (f"gemv_fused_merged_kernel (fused decode, K={dom['K']}, "
                       f"{dom['bitlinears']} BitLinears per launch)" if dom["kind"] == "decode_fused" and dom["bucket"] == 0
                       else f"gemv_kernel ({dom['kind'].replace('_', ' ')}, K={dom['K']}, "
                            f"{dom['bitlinears']} BitLinears per launch)"),
            "achieved": round(dom["GBps"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(dom["GBps"] / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": dom["bytes"],
            "avg_launch_us": round(dom["us"], 2),
            "launch_us_stats": dom["us_stats"],
        },
        "launches_us": [{"kind": d["kind"], "K": d["K"], "bitlinears": d["bitlinears"],
                         "us": round(d["us"], 2), "GBps": round(d["GBps"], 1)} for d in dec["per_launch"]],
        "measured_peaks": peaks,
    }
    out["roofline"]["frac_of_measured"] = round(dom["GBps"] / peaks["hbm_read_GBps"], 4)
    # against this box's reads with 1.5% of the bytes written (the decode
    # launch writes 1.2%): writes mixed into a read stream cost more than their bytes
    out["roofline"]["frac_of_measured_mixed"] = round(
        dom["GBps"] / peaks["hbm_mixed_GBps"]["1_write_per_64_reads"], 4)
    if not args.skip_variants:
        for key, what in (("no_norm", "the decode step with norm_w NULL on every projection "
                                      "(no per-projection norm)"),
                          ("f16_norm", "the decode step with float16 norm weights on every projection")):
            v = dec[key]
            out[key] = {"workload": what, "ms_per_step": round(v["ms"], 5), "value": round(v["value"], 2),
                        "unit": "GB/s",
                        "launches_us": [{"kind": d["kind"], "K": d["K"], "us": round(d["us"], 2),
                                         "GBps": round(d["GBps"], 1)} for d in v["per_launch"]]}
            log(f"decode ({key}): {v['ms']:.3f} ms/step, {v['value']:.0f} GB/s weights")
    if not args.skip_cpu:
        out["cpu_baseline"] = cpu_baseline_decode(dec["projs"], args.cpu_seconds)
    del dec

    if not args.skip_prefill:
        # one BitLinear 1024 -> 3072 at M = 8: per-call latency
        w1 = bench_single_m8(torch, bl, args, peaks["launch_floor_us"])
        st = w1["per_call_us"]
        out["single_m8"] = {
            "workload": "one BitLinear 1024->3072 at M=8 (x ~ N(0,1), norm_w ~ N(1,0.1)): "
                        "bitlinear_forward per call (quantization launch + decode launch)",
            "per_call_us": st, "back_to_back_us": round(w1["back_to_back_us"], 2),
            "weight_GBps": round(w1["weight_GBps"], 1),
            "roofline": {"bound": "hbm", "kernel": "quant_reg_kernel + gemv_kernel (one call, two launches)",
                         "achieved": round(w1["GBps"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(w1["GBps"] / HBM_PEAK_GBS, 4),
                         # HBM bytes of the call's decode launch (the dominant one)
                         "traffic": profile_value("gemv_single_m8", "traffic_bytes_per_launch", "gemv.hip"),
                         "algorithmic_bytes_per_call": w1["bytes"],
                         "launch_floor_us": round(w1["floor_us"], 2),
                         "call_over_two_launch_floors": round(st["median"] / (2 * w1["floor_us"]), 2),
                         "note": "latency-bound: 0.79 MB of weights is 0.1 us at the HBM peak"},
        }
        log(f"single M=8: {st['median']:.2f} us per call (p10 {st['p10']:.2f}, p90 {st['p90']:.2f}), "
            f"{w1['back_to_back_us']:.2f} us back to back; launch floor {w1['floor_us']:.2f} us")
        if not args.skip_cpu:
            out["single_m8"]["cpu_baseline"] = cpu_baseline_m8(w1, args.cpu_seconds / 2)
        del w1

        # the Gemma3-270M layer at M = 512
        g3 = bench_gemma_layer(torch, bl, args)
        out["gemma3_layer_m512"] = {
            "workload": "the seven Gemma3-270M projections at M=512 (q/k/v share x, gate/up share x), "
                        "one group forward",
            "value": round(g3["tops"], 2), "unit": "TOPS (int8-equivalent)",
            "ms_per_step": round(g3["ms"], 5), "ms_per_step_events": round(g3["ms_events"], 5),
            "step_us_stats": g3["step_us_stats"],
            "roofline": mfma_roofline(g3, peaks, "gemm_kernel (7 problems, one launch)",
                                      {"launch_floor_us": peaks["launch_floor_us"],
                                       # HBM bytes of the GEMM launch, K-split partials included
                                       "traffic": profile_value("gemm_gemma3_layer_m512",
                                                                "traffic_bytes_per_launch", "gemm.hip"),
                                       "note": "launch/latency-bound: 5.7 G ops is 1.1 us at the MFMA peak"}),
            "stages_us": {"quant": round(g3["quant_ms"] * 1e3, 2), "matmul": round(g3["mm_ms"] * 1e3, 2)},
            "quant_launches": g3["quant_launches"],
            # K split of each projection in the prefill launch (bl_prefill_splits)
            "k_splits": g3["splits"], "cus": g3["cus"],
        }
        log(f"gemma3 layer M=512: {g3['ms'] * 1e3:.1f} us/step, GEMM {g3['mm_ms'] * 1e3:.1f} us "
            f"({g3['mm_tops']:.0f} TOPS), quant {g3['quant_ms'] * 1e3:.1f} us")
        if not args.skip_cpu:
            out["gemma3_layer_m512"]["cpu_baseline"] = cpu_baseline_rows(
                g3["projs"], lambda p: g3["xs_host"][p["xkey"]], g3["M"], args.cpu_seconds,
                "token rows (all)")
        del g3

        pre = bench_prefill(torch, bl, args)
        log(f"prefill: {pre['ms']:.3f} ms/step, {pre['tops']:.1f} TOPS; MFMA kernel "
            f"{pre['mm_ms']:.3f} ms ({pre['mm_tops']:.1f} TOPS), quant {pre['quant_ms']:.3f} ms")
        log("prefill quant launches: " + "; ".join(
            f"{q['kind']} chunks={q['chunks']} x{q['bitlinears']}: {q['us']:.0f} us {q['GBps']} GB/s"
            for q in pre["quant_launches"]))
        counters = {
            "traffic": traffic_from_profiles("gemm_prefill_qwen3_stack", "gemm.hip"),
            # rocprofv3 counters of the same launch: SQ_VALU_MFMA_BUSY_CYCLES over
            # GRBM_GUI_ACTIVE x SIMDs, and the shader clock GRBM_GUI_ACTIVE implies
            "mfma_busy_from_counters": profile_value("gemm_prefill_qwen3_stack_mfma",
                                                     "mfma_busy_fraction", "gemm.hip"),
            "clock_GHz_from_counters": profile_value("gemm_prefill_qwen3_stack_mfma",
                                                     "effective_clock_GHz", "gemm.hip"),
        }
        pf = {
            "workload": "prefill M=16384 through the 28-layer Qwen3-0.6B projection stack (196 BitLinears)",
            "value": round(pre["tops"], 2), "unit": "TOPS (int8-equivalent)",
            "ms_per_step": round(pre["ms"], 4), "ms_per_step_events": round(pre["ms_events"], 4),
            "step_us_stats": pre["step_us_stats"],
            "steps": pre["steps"],
            "roofline": mfma_roofline(pre, peaks, "gemm_kernel (prefill, M>16; 196 problems, one launch)",
                                      counters),
            "stages_us": {"quant": round(pre["quant_ms"] * 1e3, 1), "matmul": round(pre["mm_ms"] * 1e3, 1)},
            "quant_launches": pre["quant_launches"],
            "per_shape": pre["per_shape"],
        }
        if not args.skip_variants:
            out["no_norm"]["prefill_quant_us"] = round(pre["no_norm_quant_ms"] * 1e3, 1)
            out["f16_norm"]["prefill_quant_us"] = round(pre["f16_quant_ms"] * 1e3, 1)
            log(f"prefill quant with float16 norm weights: {pre['f16_quant_ms']:.3f} ms")
            log(f"prefill quant without norm weights: {pre['no_norm_quant_ms']:.3f} ms")
        if not args.skip_cpu:
            rows = inputs.sample_rows(pre["M"], 64, seed=4)
            idx = torch_rows(next(iter(pre["xs"].values())), rows)
            xr = {key: x[idx].cpu().numpy() for key, x in pre["xs"].items()}
            pf["cpu_baseline"] = cpu_baseline_rows(pre["projs"], lambda p: xr[p["xkey"]], len(rows),
                                                   args.cpu_seconds, "sampled token rows")
        out["prefill"] = pf
        del pre

        lc = bench_long_context(torch, bl, args)
        out["long_context_m32768"] = {
            "workload": "gate/up/down at M=32768, heavy-tailed x (Student-t df=3, 0.1% channels x20); "
                        "gate/up share x; one group forward",
            "value": round(lc["tops"], 2), "unit": "TOPS (int8-equivalent)",
            "ms_per_step": round(lc["ms"], 4), "ms_per_step_events": round(lc["ms_events"], 4),
            "step_us_stats": lc["step_us_stats"],
            "roofline": mfma_roofline(lc, peaks, "gemm_kernel (3 problems, one launch)", {
                "traffic": profile_value("gemm_long_context_m32768", "traffic_bytes_per_launch", "gemm.hip"),
                "mfma_busy_from_counters": profile_value("gemm_long_context_m32768",
                                                         "mfma_busy_fraction", "gemm.hip"),
                "clock_GHz_from_counters": profile_value("gemm_long_context_m32768",
                                                         "effective_clock_GHz", "gemm.hip")}),
            "stages_us": {"quant": round(lc["quant_ms"] * 1e3, 1), "matmul": round(lc["mm_ms"] * 1e3, 1)},
            "quant_launches": lc["quant_launches"],
        }
        log(f"long context M=32768: {lc['ms']:.3f} ms/step, GEMM {lc['mm_ms'] * 1e3:.1f} us "
            f"({lc['mm_tops']:.0f} TOPS), quant {lc['quant_ms'] * 1e3:.1f} us")
        if not args.skip_cpu:
            out["long_context_m32768"]["code_flips_vs_oracle"] = code_flips(lc)
            out["long_context_m32768"]["cpu_baseline"] = cpu_baseline_rows(
                lc["projs"], lambda p: lc["xs_host"][p["xkey"]][lc["rows"]], len(lc["rows"]),
                args.cpu_seconds, "sampled token rows")
        del lc

        pq = bench_prefill_fused(torch, bl, args)
        log("prefill, quantization in the product's producer (one call, M=16384): " + ", ".join(
            f"{k} {v['fused_producer_us']:.0f} us vs {v['forward_us']:.0f} us"
            + ("" if v["bit_identical"] else " (OUTPUTS DIFFER)") for k, v in pq["per_shape"].items()))
        out["prefill_fused_producer"] = pq

        glue = bench_ffn_glue(torch, bl, args)
        log(f"ffn glue: glue+quant {glue['glue_quant_us']:.1f} us ({glue['roofline']['achieved']:.0f} GB/s), "
            f"glue-fed down forward {glue['forward_ms']:.3f} ms ({glue['forward_TOPS']:.0f} TOPS); "
            f"M=1 one-launch glue forward {glue['decode_M1_forward_us']:.1f} us")
        out["ffn_glue"] = glue
    if args.library_reference:
        ref = library_reference(torch)
        log("library int8 GEMM reference: " + ", ".join(
            f"{k} {v['TOPS']:.0f} TOPS" for k, v in ref["per_shape"].items()))
        out["library_reference"] = ref
    dp = bench_device_pack(torch, bl, args)
    log(f"device pack: {dp['us']:.1f} us ({dp['roofline']['achieved']:.0f} GB/s)")
    out["device_pack"] = dp
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
