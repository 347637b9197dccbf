"""Benchmark of split-KV decode attention on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one fd_decode_attn call (split kernel + log-sum-exp combine) over
one synthetic decode batch whose K/V already sit in HBM. The default workload
is batch 1, 16 query / 2 kv heads, head_dim 128, 65536 cached tokens, bf16.
K/V are replicated into R copies (>= 512 MiB in total) and successive steps
rotate through them, so the 256 MB Infinity Cache cannot serve a step from
the previous one. The K timed steps are captured once into a HIP graph and
replayed between two events, so host-side launch cost is not timed.

Prints one JSON line (rank 0). Besides the metric it carries
  roofline      the split kernel's algorithmic bytes per launch over its
                average launch time, measured here with events around a
                graph of split-only launches, against 8 TB/s HBM peak;
  cpu_baseline  the float64 CPU oracle timed on the same call (all host
                cores, and one core);
  stream_loop_us_per_call  the same calls enqueued in a plain loop, no graph;
  warm_one_copy_us_per_call  every call on the same K/V copy, which the
                Infinity Cache may serve: context only, not an HBM figure.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 * 2 ** 20
COUNTERS_FILE = os.path.join(ROOT, "profiles",
                             "split_mfma_long_gqa_64k_counters.md")
KERNEL_SOURCES = [os.path.join(ROOT, "split_kv_long_amd", "csrc", f)
                  for f in ("fd_kernels.hip", "fd_device.h", "fd_internal.h",
                            "fd_host.cpp")]


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="long_gqa_64k")
    p.add_argument("--splits", type=int, default=0,
                   help="force the split count (0: planner)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time for the oracle baseline")
    p.add_argument("--no-read-probe", action="store_true",
                   help="skip the bare HBM read probe (fd_read_probe)")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run a plain device copy of known size (for "
                        "scaling HBM byte counters)")
    p.add_argument("--set", action="append", default=[], metavar="KEY=VALUE",
                   help="override a workload recipe field, e.g. "
                        "--set batch=8 --set max_seq_len=131072")
    p.add_argument("--all", action="store_true",
                   help="also time every workload (extra JSON lines, "
                        "stderr)")
    p.add_argument("--sparse-delta", type=float, default=None,
                   help="time the block-sparse path (fd_decode_attn_sparse, "
                        "top-delta with this delta) on the chosen workload "
                        "instead of the dense one")
    p.add_argument("--frontier-kv", default="bf16",
                   choices=["bf16", "fp8_e4m3", "int8"],
                   help="cache encoding of the --frontier sweep")
    p.add_argument("--frontier", action="store_true",
                   help="instead of the metric: sweep batch x history x "
                        "splits (uniform lengths, 16q/2kv d128 bf16) and "
                        "print one JSON line per point")
    return p.parse_args()


def kernel_source_digest() -> str:
    """Digest of the sources that decide what the split kernel does and how
    it is launched; counters taken on other sources are not reported."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per split-kernel launch from the committed counter summary,
    or None if absent or taken on a different kernel source."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    text = open(COUNTERS_FILE).read()
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_source_digest():
        return None
    return float(t.group(1))


def parse_overrides(items):
    out = {}
    for it in items:
        k, v = it.split("=", 1)
        if v.lower() in ("true", "false"):
            out[k] = v.lower() == "true"
        else:
            try:
                out[k] = int(v)
            except ValueError:
                out[k] = float(v) if v.replace(".", "", 1).isdigit() else v
    return out


class Bench:
    def __init__(self, name, splits, steps, overrides=None,
                 step_fraction=None):
        import torch
        import workloads
        from split_kv_long_amd import binding as fb
        self.torch, self.fb = torch, fb
        self.w = w = workloads.make(name, **(overrides or {}))
        self.shape = fb.make_shape(**w.shape_dict())
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        self.cus = cus
        self.S = splits or fb.fd_plan_splits(self.shape, cus, w.sum_seq_len())
        self.P = -(-(-(-max(w.max_seq_len, 1) // self.S)) // 16) * 16
        dev = torch.device("cuda")
        # Enough copies that one step's reads cannot be served from the
        # Infinity Cache left over from earlier steps (step_fraction: the
        # share of the K/V bytes one step reads, when it reads less; the
        # caller then runs at least R steps per replay).
        kv = int(w.kv_bytes() * (step_fraction or 1))
        self.R = max(1, math.ceil(2 * MALL_BYTES / max(kv, 1)))
        if not step_fraction:
            self.R = min(self.R, max(1, steps))
        self.q = w.q.to(dev)
        self.lens = w.seq_lens.to(dev)
        self.bt = None if w.block_table is None else w.block_table.to(dev)
        self.ks = [w.k.to(dev) for _ in range(self.R)]
        self.vs = [w.v.to(dev) for _ in range(self.R)]
        # 8-bit caches: their calls and scales (one per kv head for E4M3,
        # rotated with the codes when there is one per position, int8).
        self.q8 = {"fp8_e4m3": (fb.fd_decode_attn_fp8,
                                fb.fd_decode_partials_fp8),
                   "int8": (fb.fd_decode_attn_int8,
                            fb.fd_decode_partials_int8)}.get(w.cache_dtype)
        nsc = self.R if w.k_scale is not None and w.k_scale.dim() > 1 else 1
        self.kscales = ([None] if w.k_scale is None else
                        [w.k_scale.to(dev) for _ in range(nsc)])
        self.vscales = ([None] if w.v_scale is None else
                        [w.v_scale.to(dev) for _ in range(nsc)])
        B, Hq, D = w.batch, w.num_q_heads, w.head_dim
        self.out = torch.empty(B, Hq, D, device=dev)
        self.lse = torch.empty(B, Hq, device=dev)
        nb = fb.fd_workspace_size(self.shape, self.S)
        self.ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        self.op = torch.empty(B, Hq, max(self.S, 1), D, device=dev)
        self.lp = torch.empty(B, Hq, max(self.S, 1), device=dev)
        esz = 4 if w.dtype == "f32" else 2
        self.bytes_alg = (kv + B * Hq * D * esz + B * Hq * D * 4 + B * Hq * 4
                          + (0 if self.bt is None else
                             4 * w.batch * -(-w.max_seq_len // w.block_size)))
        self.bytes_split = kv + B * Hq * D * esz   # K/V + q, per split launch

    def scales(self, r):
        return (self.kscales[r % len(self.kscales)],
                self.vscales[r % len(self.vscales)])

    def step(self, i):
        r = i % self.R
        if self.q8:
            self.q8[0](self.shape, self.q, self.ks[r], self.vs[r],
                       *self.scales(r), self.bt, self.lens, self.S, self.ws,
                       self.out, self.lse)
        else:
            self.fb.fd_decode_attn(self.shape, self.q, self.ks[r], self.vs[r],
                                   self.bt, self.lens, self.S, self.ws,
                                   self.out, self.lse)

    def split_only(self, i):
        r = i % self.R
        if self.q8:
            self.q8[1](self.shape, self.q, self.ks[r], self.vs[r],
                       *self.scales(r), self.bt, self.lens, self.S, self.op,
                       self.lp)
        else:
            self.fb.fd_decode_partials(self.shape, self.q, self.ks[r],
                                       self.vs[r], self.bt, self.lens, self.S,
                                       self.op, self.lp)

    def combine_only(self, i):
        w = self.w
        self.fb.fd_combine_partials(w.batch, w.num_q_heads, w.head_dim,
                                    self.S, self.op, self.lp, self.out,
                                    self.lse)

    def time_graph(self, fn, steps, warmup):
        return time_graph(self.torch, fn, steps, warmup)


def time_stream(torch, fn, steps, warmup):
    """The same calls enqueued eagerly on the current stream, timed with
    events around the loop (host enqueue cost included)."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def time_graph(torch, fn, steps, warmup, replays=1, spread=None):
    """Eager warmup, capture `steps` calls in a graph, replay once untimed,
    then time `replays` replays. Returns (median ms per replay, wall ms of
    the timed region); `spread`, if a dict, receives min/median/max."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                fn(i)
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    times = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(replays):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    wall = (time.perf_counter() - t0) * 1e3
    if spread is not None:
        spread.update(min=min(times), median=statistics.median(times),
                      max=max(times))
    return statistics.median(times), wall


def copy_probe(torch):
    """A plain device-to-device copy of a known size (counter scaling and
    achievable-bandwidth context)."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return dict(bytes_read=n, bytes_written=n, ms=ms,
                GBps_read_plus_write=2 * n / (ms * 1e6))


# Shapes the read probe is timed at: the split kernel's launch shape at
# the headline workload (256 workgroups of 4 waves, 16 KB per wave in
# flight: a 32-token subtile of K and of V), the same grid with half of
# that in flight, and the others a sweep found fastest on MI355X.
PROBE_SHAPES = [(256, 4, 16), (256, 4, 8), (256, 16, 2), (256, 16, 4),
                (512, 4, 8), (2048, 8, 2)]


def read_probe(torch, nbytes, steps, warmup):
    """Bare streaming reads of nbytes (rounded down to what every probe
    shape divides) from buffers rotated over >= 512 MiB, each shape timed
    like the call: a graph of back-to-back launches, median of 5 replays."""
    from split_kv_long_amd import binding as fb
    unit = max(w * nw * 64 * 16 * u for w, nw, u in PROBE_SHAPES)
    n = nbytes // unit * unit
    if n == 0:
        return None
    R = max(1, math.ceil(2 * MALL_BYTES / n))
    bufs = [torch.empty(n, dtype=torch.uint8, device="cuda") for _ in range(R)]
    for b in bufs:
        b.fill_(1)
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    shapes = {}
    for wg, nw, u in PROBE_SHAPES:
        def fn(i, wg=wg, nw=nw, u=u):
            fb.fd_read_probe(bufs[i % R], wg, nw, u, sink, nbytes=n)
        ms, _ = time_graph(torch, fn, steps, warmup, replays=5)
        us = ms * 1e3 / steps
        shapes[f"{wg}x{nw}w_{u * 16}B"] = {"us": round(us, 3),
                                           "GBps": round(n / (us * 1e3), 1)}
    del bufs
    best = max(shapes, key=lambda k: shapes[k]["GBps"])
    return {"bytes": n, "copies_rotated": R, "shapes": shapes,
            "split_grid_shape": "256x4w_256B", "best_shape": best,
            "best_GBps": shapes[best]["GBps"]}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, target_s):
    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:
        threadpool_limits = None
        threads = os.cpu_count() or 1
    a = w.numpy_view()

    def timed(budget_s, max_calls):
        times = []
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            oracle.decode_attention(a["q"], a["k"], a["v"], a["seq_lens"],
                                    dtype=a["dtype"], scale=a["scale"],
                                    block_table=a["block_table"],
                                    block_size=a["block_size"],
                                    kv_dtype=a["kv_dtype"],
                                    k_scale=a["k_scale"], v_scale=a["v_scale"])
            times.append(time.perf_counter() - t0)
            if (time.perf_counter() - t_start >= budget_s
                    or len(times) >= max_calls):
                return times
    times = timed(target_s, 1000)      # the time budget ends the sample
    rec = dict(value=statistics.median(times) * 1e6, unit="us/call",
               cores=threads, kind="oracle",
               sample=(f"{len(times)} full calls of the {w.name} workload "
                       f"(float64 NumPy oracle, median)"),
               host_cpu_count=os.cpu_count(), cpu_model=cpu_model())
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            t1 = timed(target_s / 2, 1000)
        rec["value_one_core"] = statistics.median(t1) * 1e6
        rec["sample_one_core"] = f"{len(t1)} calls, BLAS limited to 1 thread"
    return rec


def workloads_compare_splits(name):
    import workloads
    return workloads.SPECS.get(name, {}).get("compare_splits")


def run_one(args, name, steps, warmup, with_cpu):
    import torch
    b = Bench(name, args.splits if name == args.workload else 0, steps,
              parse_overrides(args.set) if name == args.workload else None)
    spread = {}
    ms, wall = time_graph(torch, b.step, steps, warmup, replays=5,
                          spread=spread)
    us_call = ms * 1e3 / steps
    ms_loop = time_stream(torch, b.step, steps, warmup)
    warm_steps = min(steps, 50)
    ms_warm, _ = b.time_graph(lambda i: b.step(0), warm_steps, warmup)
    # The kernels alone, each the median of five replays like the call.
    split_spread = {}
    ms_split, _ = time_graph(torch, b.split_only, steps, warmup, replays=5,
                             spread=split_spread)
    us_split = ms_split * 1e3 / steps
    us_comb = None
    if b.S > 1:
        ms_c, _ = time_graph(torch, b.combine_only, steps, 2, replays=5)
        us_comb = ms_c * 1e3 / steps
    w = b.w
    # Batched calls (2..64 sequences) cut sequences into length-aware pieces
    # inside fd_decode_attn; the split-only entry point keeps uniform splits,
    # so the kernel the call runs is timed as the call minus the combine.
    split_timing = "split-only launches (fd_decode_partials)"
    if 1 < w.batch <= 64 and b.S > 1 and w.dtype != "f32":
        us_split = us_call - us_comb
        split_timing = ("call minus combine (length-aware pieces; "
                        f"uniform-split launches: {round(ms_split * 1e3 / steps, 3)} us)")
    gbps = b.bytes_alg / (us_call * 1e3)
    split_gbps = b.bytes_split / (us_split * 1e3)
    # The counters were taken on the default 64K launch (planned splits).
    custom = name == args.workload and (args.splits or args.set)
    traffic = (read_traffic() if name == "long_gqa_64k" and not custom
               else None)
    rec = {
        "metric": ("decode-attn us/call + achieved HBM GB/s (% of peak), "
                   "B=1 L=64K GQA 16/2 d128"),
        "value": round(us_call, 3),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms / steps, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1), see workloads/)",
        "config": {
            "workload": name, "batch": w.batch, "num_q_heads": w.num_q_heads,
            "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
            "max_seq_len": w.max_seq_len, "sum_seq_len": w.sum_seq_len(),
            "paged": w.paged, "kv_dtype": w.cache_dtype,
            "num_splits": b.S, "tokens_per_split": b.P,
            "kv_copies_rotated": b.R, "timing": "hip graph replay of all "
            "timed steps between two events, median of 5 replays",
            "overrides": parse_overrides(args.set) if name == args.workload
            else {},
        },
        "achieved_GBps": round(gbps, 1),
        "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "algorithmic_bytes_per_call": b.bytes_alg,
        "wall_ms_timed_region": round(wall, 3),
        "replays": {"count": 5, "us_per_call_min": round(spread["min"] * 1e3 / steps, 3),
                    "us_per_call_max": round(spread["max"] * 1e3 / steps, 3),
                    "value_is": "median"},
        "stream_loop_us_per_call": round(ms_loop * 1e3 / steps, 3),
        "warm_one_copy_us_per_call": round(ms_warm * 1e3 / warm_steps, 3),
        "split_kernel_us": round(us_split, 3),
        "combine_kernel_us": None if us_comb is None else round(us_comb, 3),
        "roofline": {
            "kernel": "split_mfma" if w.dtype == "bf16" else "split_f32",
            "bound": "hbm",
            "achieved": round(split_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(split_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "bytes_per_launch": b.bytes_split,
            "launch_us": round(us_split, 3),
            "timing": split_timing,
            "split_only_replays_us": {
                "min": round(split_spread["min"] * 1e3 / steps, 3),
                "max": round(split_spread["max"] * 1e3 / steps, 3),
                "value_is": "median of 5"},
        },
    }
    # The workload recipes that name split counts to compare (the tiny MHA
    # case, the short-history batch) get the call time at each of them.
    cmp = workloads_compare_splits(name)
    if cmp:
        res = {}
        for S in sorted(set(cmp) | {b.S}):
            b2 = Bench(name, S, steps, None)
            ms2, _ = b2.time_graph(b2.step, steps, warmup)
            res[str(S)] = round(ms2 * 1e3 / steps, 3)
            del b2
        rec["split_comparison_us_per_call"] = res
        rec["split_comparison_planned"] = b.S
    if name == args.workload and not args.no_read_probe:
        probe = read_probe(torch, b.bytes_split - (b.bytes_split % 16), steps,
                           warmup)
        if probe:
            rec["roofline"]["probe_GBps"] = probe["best_GBps"]
            rec["roofline"]["frac_of_probe"] = round(
                split_gbps / probe["best_GBps"], 4)
            same = probe["shapes"].get(probe["split_grid_shape"])
            if same:
                # against a bare read with the split kernel's grid and
                # bytes in flight per wave
                rec["roofline"]["frac_of_probe_same_shape"] = round(
                    split_gbps / same["GBps"], 4)
            rec["read_probe"] = probe
    if args.copy_probe and name == args.workload:
        rec["copy_probe"] = copy_probe(torch)
    if with_cpu:
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    rec["platform"] = platform_info(torch)
    del b
    torch.cuda.empty_cache()
    return rec


def platform_info(torch):
    """GPU, ROCm / HIP and torch versions the numbers were taken on."""
    props = torch.cuda.get_device_properties(0)
    rocm = None
    try:
        root = os.environ.get("ROCM_PATH", "/opt/rocm")
        with open(os.path.join(root, ".info", "version")) as f:
            rocm = f.read().strip()
    except OSError:
        pass
    return {"gpu": props.name, "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count,
            "rocm": rocm, "hip": torch.version.hip, "torch": torch.__version__}


FRONTIER_B = (1, 4, 16, 64, 256)
FRONTIER_L = (512, 2048, 8192, 32768, 131072, 262144)
FRONTIER_S = (1, 2, 4, 8, 16, 32, 64, 128, 256)
FRONTIER_MAX_TOKENS = 1 << 24          # B * L cap: 17 GB of bf16 K/V


def frontier(args):
    """Where splitting pays: every (batch, history) point of the grid at
    every split count, plus the planner's choice. Inputs are drawn on the
    device from a seeded generator (timing only; parity is the tests')."""
    import torch
    from split_kv_long_amd import binding as fb
    Hq, Hkv, D = 16, 2, 128
    kvd = args.frontier_kv
    esz = 2 if kvd == "bf16" else 1
    dev = torch.device("cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    gen = torch.Generator(device=dev)
    for B in FRONTIER_B:
        for L in FRONTIER_L:
            if B * L > FRONTIER_MAX_TOKENS:
                continue
            gen.manual_seed(1000 * B + L // 512)
            kv = B * Hkv * L * D * esz
            R = max(1, min(args.steps, math.ceil(2 * MALL_BYTES / kv)))
            q = torch.randn(B, Hq, D, generator=gen, device=dev).to(
                torch.bfloat16)

            def cache():
                # Timing inputs: random finite codes (E4M3 codes below 0x7E
                # with either sign; int8 in [-127, 127]) and unit scales.
                if kvd == "bf16":
                    return torch.randn(B, Hkv, L, D, generator=gen,
                                       device=dev).to(torch.bfloat16)
                if kvd == "int8":
                    return torch.randint(-127, 128, (B, Hkv, L, D),
                                         generator=gen, device=dev,
                                         dtype=torch.int8)
                c = torch.randint(0, 0x7E, (B, Hkv, L, D), generator=gen,
                                  device=dev, dtype=torch.int32)
                c |= torch.randint(0, 2, c.shape, generator=gen, device=dev,
                                   dtype=torch.int32) << 7
                return c.to(torch.uint8).view(torch.float8_e4m3fn)
            ks = [cache() for _ in range(R)]
            vs = [cache() for _ in range(R)]
            sc_shape = (Hkv,) if kvd == "fp8_e4m3" else (B, Hkv, -(-L // 16) * 16)
            ksc = torch.ones(sc_shape, device=dev)
            vsc = torch.ones(sc_shape, device=dev)
            lens = torch.full((B,), L, dtype=torch.int32, device=dev)
            out = torch.empty(B, Hq, D, device=dev)
            shape = fb.make_shape(B, Hq, Hkv, D, L, kvd)
            planned = fb.fd_plan_splits(shape, cus, B * L)
            res = {}
            for S in sorted(set(FRONTIER_S) | {planned}):
                if S > 1 and -(-L // S) < 16:
                    continue
                nb = fb.fd_workspace_size(shape, S)
                ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)

                def step(i, S=S, ws=ws):
                    r = i % R
                    if kvd == "bf16":
                        fb.fd_decode_attn(shape, q, ks[r], vs[r], None, lens,
                                          S, ws, out)
                    else:
                        call = (fb.fd_decode_attn_int8 if kvd == "int8"
                                else fb.fd_decode_attn_fp8)
                        call(shape, q, ks[r], vs[r], ksc, vsc, None, lens, S,
                             ws, out)
                ms, _ = time_graph(torch, step, args.steps, 3)
                res[S] = ms * 1e3 / args.steps
            best = min(res, key=res.get)
            rec = dict(batch=B, max_seq_len=L, num_q_heads=Hq,
                       num_kv_heads=Hkv, head_dim=D, dtype=kvd,
                       kv_bytes=kv, us_per_call={str(k): round(v, 3)
                                                 for k, v in res.items()},
                       best_splits=best, planned_splits=planned,
                       planned_over_best=round(res[planned] / res[best], 4),
                       split_gain=round(res[1] / res[best], 4))
            print(json.dumps(rec), flush=True)
            del q, ks, vs, out
            torch.cuda.empty_cache()


def sparse_run(args):
    """Block-sparse decode on one workload: the key summary is built once
    per K copy outside the timed region (a serving loop would update it
    incrementally), then K timed fd_decode_attn_sparse calls."""
    import torch
    import numpy as np
    from split_kv_long_amd import binding as fb
    # A call reads the 4-bit summary (1/8 of the K/V bytes) and the kept
    # blocks; copies are rotated on that basis, and every replay runs
    # through all of them, so the summary, which would fit the Infinity
    # Cache, is read cold like the dense path's K/V.
    b = Bench(args.workload, args.splits, args.steps,
              parse_overrides(args.set), step_fraction=1 / 8)
    w, dev = b.w, torch.device("cuda")
    q8 = {"fp8_e4m3": "fp8", "int8": "int8"}.get(w.cache_dtype)
    if q8 is None and w.cache_dtype != "bf16":
        raise SystemExit("the block-sparse path takes bf16, E4M3 or int8 "
                         "caches")
    f8 = q8 is not None
    steps = max(args.steps, b.R)
    D, Hkv = w.head_dim, w.num_kv_heads
    nblk = -(-w.max_seq_len // 16)

    def build_into(r, c, sc):
        if f8:
            getattr(fb, "fd_build_key_summary_" + q8)(
                b.shape, b.ks[r], b.scales(r)[0], b.bt, b.lens, c, sc)
        else:
            fb.fd_build_key_summary(b.shape, b.ks[r], b.bt, b.lens, c, sc)
    codes, scales = [], []
    for r in range(b.R):
        nrec = ((w.k.shape[0], Hkv, w.block_size // 16) if w.paged
                else (w.batch, Hkv, nblk))
        c = torch.empty(nrec + (8 * D,), dtype=torch.uint8, device=dev)
        sc = torch.empty(nrec, device=dev)
        build_into(r, c, sc)
        codes.append(c)
        scales.append(sc)

    def build(i):
        r = i % b.R
        build_into(r, codes[r], scales[r])
    kept = torch.zeros(w.batch, Hkv, nblk, dtype=torch.uint8, device=dev)

    def step(i):
        r = i % b.R
        if f8:
            getattr(fb, "fd_decode_attn_sparse_" + q8)(
                b.shape, b.q, b.ks[r], b.vs[r], *b.scales(r), codes[r],
                scales[r], b.bt, b.lens, args.sparse_delta, b.S, b.ws, b.out,
                b.lse, kept)
        else:
            fb.fd_decode_attn_sparse(b.shape, b.q, b.ks[r], b.vs[r], codes[r],
                                     scales[r], b.bt, b.lens,
                                     args.sparse_delta, b.S, b.ws, b.out,
                                     b.lse, kept)
    ms, _ = time_graph(torch, step, steps, args.warmup)
    us = ms * 1e3 / steps
    ms_b, _ = time_graph(torch, build, max(1, args.steps // 4), 2)
    lens = w.seq_lens.numpy().astype(np.int64)
    k = kept.cpu().numpy()
    attended = kept_tok = 0
    for bb in range(w.batch):
        n = int(lens[bb])
        nb = -(-n // 16)
        for h in range(Hkv):
            m = k[bb, h, :nb].astype(bool)
            attended += n
            kept_tok += int(m[:-1].sum()) * 16 + (
                (n - 16 * (nb - 1)) if nb and m[-1] else 0)
    row = D * (1 if f8 else 2)                        # cache bytes per row
    if q8 == "int8":
        row += 4                                      # its per-position scale
    scan = attended * D // 2 + attended // 16 * 4     # codes + scales
    bytes_read = scan + 2 * kept_tok * row + w.batch * w.num_q_heads * D * 2
    dense = 2 * attended * row
    return {
        "metric": "block-sparse decode us/call (top-delta over a 4-bit key "
                  "summary)",
        "value": round(us, 3), "unit": "us/call", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup,
        "higher_is_better": False, "dtype": "bf16",
        "data": "synthetic (seeded, see workloads/)",
        "config": {"workload": args.workload, "kv_dtype": w.cache_dtype,
                   "delta": args.sparse_delta,
                   "copies_rotated": b.R,
                   "num_splits": b.S, "tokens_per_split": b.P,
                   "overrides": parse_overrides(args.set)},
        "kept_token_fraction": round(kept_tok / max(attended, 1), 4),
        "bytes_read_per_call": bytes_read,
        "dense_kv_bytes": dense,
        "achieved_GBps": round(bytes_read / (us * 1e3), 1),
        "summary_build_us": round(ms_b * 1e3 / max(1, args.steps // 4), 3),
    }


def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only; --gpus must be 1 "
              "(sequence- or head-sharded multi-GPU decode is not built)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    from split_kv_long_amd import binding
    binding.load()     # fails loudly if the HIP library is missing
    if args.frontier:
        frontier(args)
        return
    if args.sparse_delta is not None:
        print(json.dumps(sparse_run(args)), flush=True)
        return
    rec = run_one(args, args.workload, args.steps, args.warmup,
                  not args.no_cpu_baseline)
    if args.all:
        import workloads
        for name in workloads.ORDER + workloads.EXTRA:
            if name == args.workload:
                continue
            r = run_one(args, name, args.steps, args.warmup, False)
            print(json.dumps(r), file=sys.stderr, flush=True)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
