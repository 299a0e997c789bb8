"""Benchmark of the embedding weight-gradient accumulation on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--configs all|none|A,B]

One step = one whole call (one kernel: sort, chunk sums, single-chunk runs,
ordered combine of long runs) over the headline workload: 8192 Zipf(1.1)
token ids into a 129280 x 7168 fp32 main_grad with a bf16 grad. Inputs are
resident in HBM before timing. Before every step, outside its timed interval,
a 1 GiB buffer is read (summed) so that neither L2 nor the 256 MB Infinity
Cache holds the inputs; reading rather than writing leaves no dirty lines for
the timed call to write back. Each step is timed with two HIP events that the
library records on its launch stream right before and after the call (value,
us_per_call). A second pass of the same steps dispatches the kernel with two
more events of its own (roofline.achieved and us_per_launch: the kernel's
execution alone, the figure a kernel trace shows); that pass is kept apart
because such a dispatch adds time around the kernel.

Prints one JSON line: value = algorithmic bytes / mean call time (GB/s), the
roofline of the kernel (the whole call is one kernel), and the CPU oracle
timed on the host as cpu_baseline (one thread, and every host thread over
column blocks). Also, each in its own object: the same two passes on each of
the five generated workloads (configs), the copy and read ceilings of a
plain device copy and reduction timed in the same run (copy_ceiling), the
dense PyTorch path on the same inputs (dense_baseline), the many-token entry
point on a batch of more than 8192 tokens (many_tokens, with its own dense
baseline), and with --vocab-shards S the vocabulary-shard entry point.
"""
import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
FLUSH_BYTES = 1 << 30
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["accumulate.hip", "chunk_sums.h", "sort_lds.h", "ewg_device.h", "ewg_internal.h"]


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=None,
                   help="the headline workload (value and roofline); default the 8192-token "
                        "Zipf(1.1) one")
    p.add_argument("--configs", default="all",
                   help="workloads timed under configs: all (default), none, or a comma list")
    p.add_argument("--cpu-threads", type=int, default=0,
                   help="threads of the all-core CPU oracle timing (default: OMP_NUM_THREADS, "
                        "else the CPUs this process may run on)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="rough budget for the CPU oracle timing")
    p.add_argument("--flush", choices=["read", "write", "none"], default="read",
                   help="how the caches are emptied before each step: read (default) or write a "
                        "1 GiB buffer, or not at all")
    p.add_argument("--vocab-shards", type=int, default=0,
                   help="also time the vocabulary-shard entry point: the table split into this "
                        "many equal row ranges, one call per shard (reported under vocab_shards)")
    p.add_argument("--no-dense-baseline", action="store_true",
                   help="skip timing PyTorch's dense embedding backward + main_grad.add_")
    p.add_argument("--many-workload", default=None,
                   help="workload of the many-token entry point timed under many_tokens "
                        "(default: the 32768-token one)")
    p.add_argument("--no-many-tokens", action="store_true",
                   help="skip timing the many-token entry point")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a 256 MiB device fill (reference for counter scaling)")
    return p.parse_args()


class HipEvents:
    """Raw hipEvent_t handles (the library records them on its launch stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[i] = h.value
        return arr

    def ms(self, a, b):
        out = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def destroy(self, arr):
        for h in arr:
            self.hip.hipEventDestroy(h)


def strip_c_comments(text):
    """C/C++ source without its comments and with runs of whitespace made one space, so
    that an edit of comments or layout alone leaves the kernel hash unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash():
    """Hash of the fused kernel's sources, comments and layout aside."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "sparse_embedding_weight_amd", "csrc", name)) as f:
            h.update(strip_c_comments(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload_name):
    """HBM bytes per launch of the fused accumulate kernel from the committed counter
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"accumulate_{workload_name}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    src = re.search(r"kernel_source_sha256:\s*(\w+)", text)
    val = re.search(r"traffic_bytes_per_launch:\s*(\d+)", text)
    if not src or not val or src.group(1) != kernel_source_hash():
        return None
    return int(val.group(1))


def host_threads(requested):
    """Threads of the all-core CPU timing: --cpu-threads, else OMP_NUM_THREADS, else the
    CPUs this process may run on."""
    if requested > 0:
        return requested
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return min(int(env), len(os.sched_getaffinity(0)))
    return len(os.sched_getaffinity(0))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, ids_np, grad_np, budget_s, threads):
    """The oracle as it stands, on the whole workload with main_grad restricted to its
    touched rows (ids relabelled in order): median seconds per call of the serial C
    routine, and of the same routine run at once on `threads` column blocks (each
    column's arithmetic is independent, so the bits are the serial call's)."""
    import oracle
    import workloads as wl

    rows = np.unique(ids_np)
    compact = np.searchsorted(rows, ids_np).astype(np.int32)
    rng = np.random.default_rng(0)
    mg = wl.to_numpy_bits(wl.normal_tensor(rng, (rows.size, w.hidden), w.main_grad_sigma,
                                           w.main_grad_dtype))

    def median_time(call):
        times = []
        start = time.perf_counter()
        while not times or (time.perf_counter() - start < budget_s / 2 and len(times) < 20):
            m = mg.copy()
            t0 = time.perf_counter()
            call(m)
            times.append(time.perf_counter() - t0)
        return float(np.median(times)), len(times)

    serial = median_time(lambda m: oracle.accumulate_embedding_wgrad(
        compact, grad_np, m, w.grad_dtype, w.main_grad_dtype))
    blocks = []
    threaded = median_time(lambda m: blocks.append(oracle.accumulate_embedding_wgrad_column_blocks(
        compact, grad_np, m, w.grad_dtype, w.main_grad_dtype, threads)))
    return serial, threaded, blocks[-1]


def copy_ceiling(torch, dev, reps=10):
    """Device bandwidth ceilings measured in this run (context for the roofline, never
    its peak): a 1 GiB device-to-device tensor copy (bytes read + written per second)
    and a 1 GiB fp32 sum (bytes read per second), each the best of `reps`, timed with
    events on the current stream."""
    src = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    sink = torch.zeros((), dtype=torch.float32, device=dev)
    out = {}
    for kind, fn, nbytes in (("copy", lambda: dst.copy_(src), 2 << 30),
                             ("read", lambda: sink.copy_(src.sum()), 1 << 30)):
        best = None
        for _ in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        out[kind] = round(nbytes / (best * 1e-3) / 1e9, 1)
    del src, dst
    return {"copy_ceiling_GBps": out["copy"], "read_ceiling_GBps": out["read"],
            "kind": "torch copy_ of 1 GiB (read + write bytes) and torch sum of 1 GiB fp32 "
                    "(read bytes), best of %d, HIP events" % reps}


def time_vocab_shards(torch, ewg, wl, w, ids, ids_np, grad, mg, flush, flush_sink, flush_mode,
                      shards, steps, warmup):
    """Each of `shards` equal row ranges of the table through the vocabulary-shard entry
    point, as one device of a row-sharded table would call it (the whole batch of ids,
    its own rows). Per shard: mean µs per call (events on the current stream, caches
    emptied before each call) and GB/s of that shard's algorithmic bytes."""
    bounds = [w.vocab * k // shards for k in range(shards + 1)]
    ws = ewg.new_workspace(w.num_tokens, w.hidden, mg.device)
    out = []
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        in_shard = (ids_np >= lo) & (ids_np < hi)
        uniq = int(np.unique(ids_np[in_shard]).size)
        alg = wl.algorithmic_bytes(int(in_shard.sum()), w.hidden, uniq, w.grad_dtype,
                                   w.main_grad_dtype, 0) + ids_np.size * ids_np.itemsize
        view = mg[lo:hi]
        times = []
        for k in range(warmup + steps):
            if flush_mode == "read":
                flush_sink.copy_(flush.sum())
            elif flush_mode == "write":
                flush.fill_(float(k))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            ewg.accumulate_embedding_wgrad_vocab_shard(ids, grad, view, lo, workspace=ws)
            e1.record()
            if k >= warmup:
                times.append((e0, e1))
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in times]))
        out.append({"rows": [lo, hi], "tokens_in_shard": int(in_shard.sum()), "distinct_ids": uniq,
                    "algorithmic_bytes": alg, "us_per_call": round(ms * 1e3, 2),
                    "GB_per_s": round(alg / (ms * 1e-3) / 1e9, 1)})
    if ewg.wait_timeouts(ws):
        raise RuntimeError("bounded waits gave up inside the kernel (vocabulary shards)")
    return {"shards": shards, "per_shard": out}


def dense_baseline(torch, w, ids, grad, mg, flush, flush_sink, flush_mode, our_ms, calls=5):
    """The path the fused call replaces, on the same GPU and inputs: PyTorch-ROCm's
    aten::embedding_dense_backward (a zero-filled [vocab, hidden] gradient in grad's
    dtype) followed by main_grad.add_ over the whole table. Timed with events on the
    current stream, caches emptied before each call as for the fused call."""
    times = []
    for k in range(calls + 1):
        if flush_mode == "read":
            flush_sink.copy_(flush.sum())
        elif flush_mode == "write":
            flush.fill_(float(k))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        gw = torch.ops.aten.embedding_dense_backward(grad, ids.long(), w.vocab, -1, False)
        mg.add_(gw)
        e1.record()
        torch.cuda.synchronize()
        del gw
        if k:   # the first call warms up
            times.append(e0.elapsed_time(e1))
    ms = float(np.mean(times))
    return {"us_per_call": round(ms * 1e3, 1), "calls": calls,
            "kind": "aten::embedding_dense_backward + main_grad.add_ (PyTorch-ROCm)",
            "speedup_of_fused_call": round(ms / our_ms, 2)}


def time_many_tokens(torch, ewg, B, wl, name, hip, flush, flush_sink, flush_mode, steps, warmup,
                     dense):
    """The many-token entry point (more tokens than one LDS sort holds) on its own
    workload: mean µs per call between two HIP events the library records on its
    stream around its five kernels, caches emptied before each call; GB/s of the
    same algorithmic bytes as the headline."""
    w = wl.MANY_WORKLOADS[name]
    dev = torch.device("cuda:0")
    ids_np = wl.make_ids(w).reshape(-1)
    ids = torch.from_numpy(ids_np).to(dev)
    grad = wl.make_grad(w).reshape(w.num_tokens, w.hidden).to(dev)
    mg = wl.make_main_grad(w, dev)
    counts = np.bincount(ids_np, minlength=w.vocab)
    uniq = int((counts > 0).sum())
    alg = wl.algorithmic_bytes(w.num_tokens, w.hidden, uniq, w.grad_dtype, w.main_grad_dtype,
                               ids_np.itemsize)
    ws = ewg.new_many_tokens_workspace(w.num_tokens, w.hidden, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    call_args = (ids.data_ptr(), grad.data_ptr(), mg.data_ptr(), w.num_tokens, w.hidden, w.vocab,
                 grad.stride(0), mg.stride(0), B.DTYPE_CODE[ids.dtype], B.DTYPE_CODE[grad.dtype],
                 B.DTYPE_CODE[mg.dtype], ws.data_ptr(), ws.numel(), stream)
    events = [hip.create(2) for _ in range(warmup + steps)]
    for k in range(warmup + steps):
        if flush_mode == "read":
            flush_sink.copy_(flush.sum())
        elif flush_mode == "write":
            flush.fill_(float(k))
        st = B.lib.accumulate_embedding_wgrad_many_tokens_timed(*call_args, events[k])
        if st != 0:
            raise B.EmbeddingWgradError(st, "accumulate_embedding_wgrad_many_tokens_timed")
    torch.cuda.synchronize()
    t = np.array([hip.ms(e[0], e[1]) for e in events[warmup:]])
    for e in events:
        hip.destroy(e)
    ms = float(t.mean())
    gbs = alg / (ms * 1e-3) / 1e9
    out = {"workload": name, "num_tokens": w.num_tokens, "vocab": w.vocab, "hidden": w.hidden,
           "grad_dtype": w.grad_dtype, "main_grad_dtype": w.main_grad_dtype,
           "distinct_ids": uniq, "runs_longer_than_10": int((counts > ewg.NROWS).sum()),
           "algorithmic_bytes": alg, "us_per_call": round(ms * 1e3, 2),
           "us_per_call_p10_p50_p90": [round(float(np.percentile(t, q)) * 1e3, 2) for q in (10, 50, 90)],
           "GB_per_s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
           "kernels": "tile sort, ranks, chunk lists, chunk sums, ordered combine (one stream)"}
    if dense:
        out["dense_baseline"] = dense_baseline(torch, w, ids, grad, mg, flush, flush_sink,
                                               flush_mode, ms)
    return out


class Workload:
    """One generated workload resident on the device, with its call arguments."""

    def __init__(self, torch, ewg, B, wl, name, dev):
        w = self.w = wl.WORKLOADS[name]
        self.name = name
        self.ids_np = wl.make_ids(w).reshape(-1)
        self.ids = torch.from_numpy(self.ids_np).to(dev)
        self.grad_cpu = wl.make_grad(w).reshape(w.num_tokens, w.hidden)
        self.grad = self.grad_cpu.to(dev)
        self.mg = wl.make_main_grad(w, dev)
        counts = np.bincount(self.ids_np, minlength=w.vocab)
        self.uniq = int((counts > 0).sum())
        self.u_long = int((counts > ewg.NROWS).sum())
        self.alg_bytes = wl.algorithmic_bytes(w.num_tokens, w.hidden, self.uniq, w.grad_dtype,
                                              w.main_grad_dtype, self.ids_np.itemsize)
        self.ws = ewg.new_workspace(w.num_tokens, w.hidden, dev)
        stream = torch.cuda.current_stream(dev).cuda_stream
        self.call_args = (self.ids.data_ptr(), self.grad.data_ptr(), self.mg.data_ptr(),
                          w.num_tokens, w.hidden, w.vocab, self.grad.stride(0), self.mg.stride(0),
                          B.DTYPE_CODE[self.ids.dtype], B.DTYPE_CODE[self.grad.dtype],
                          B.DTYPE_CODE[self.mg.dtype], self.ws.data_ptr(), self.ws.numel(), stream)

    def describe(self):
        w = self.w
        return {"workload": self.name, "num_tokens": w.num_tokens, "vocab": w.vocab,
                "hidden": w.hidden,
                "ids": f"{w.ids_kind}" + (f"(s={w.zipf_s})" if w.ids_kind == "zipf" else ""),
                "grad_dtype": w.grad_dtype, "main_grad_dtype": w.main_grad_dtype,
                "distinct_ids": self.uniq, "runs_longer_than_10": self.u_long,
                "algorithmic_bytes": self.alg_bytes}


def timed_pass(torch, B, hip, work, args, flush, flush_sink, kernel_events):
    """warmup + steps calls of one workload; per timed call the (call, kernel)
    durations in ms and the wall time of the timed steps. Without kernel_events the
    kernel is dispatched plainly (slots 2, 3 NULL): a dispatch that takes its own
    events costs extra time around it."""
    nsteps = args.warmup + args.steps
    events = [hip.create(4 if kernel_events else 2) for _ in range(nsteps)]
    slots = [(ctypes.c_void_p * 4)(*(list(e) + [None, None])[:4]) for e in events]
    torch.cuda.synchronize()
    t0 = None
    for step in range(nsteps):
        if step == args.warmup:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
        if args.flush == "read":
            flush_sink.copy_(flush.sum())
        elif args.flush == "write":
            flush.fill_(float(step))
        st = B.lib.accumulate_embedding_wgrad_timed(*work.call_args, slots[step])
        if st != 0:
            raise B.EmbeddingWgradError(st, "accumulate_embedding_wgrad_timed")
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    timed = events[args.warmup:]
    calls = np.array([hip.ms(e[0], e[1]) for e in timed])
    kernels = np.array([hip.ms(e[2], e[3]) for e in timed]) if kernel_events else None
    for e in events:
        hip.destroy(e)
    return calls, kernels, elapsed


def pct(t):
    return [round(float(np.percentile(t, q)) * 1e3, 2) for q in (10, 50, 90)]


def measure(torch, ewg, B, hip, work, args, flush, flush_sink):
    """The two passes on one workload: plain dispatches between the call's own events
    (us_per_call, GB_per_s), then dispatches with the kernel's own events
    (us_per_launch and the roofline fraction). Raises if a bounded wait gave up."""
    t_call, _, wall = timed_pass(torch, B, hip, work, args, flush, flush_sink, False)
    _, t_kernel, _ = timed_pass(torch, B, hip, work, args, flush, flush_sink, True)
    timeouts = ewg.wait_timeouts(work.ws)
    if timeouts:
        raise RuntimeError(f"{timeouts} bounded waits gave up inside the kernel ({work.name})")
    call_ms, kernel_ms = float(t_call.mean()), float(t_kernel.mean())
    kernel_gbs = work.alg_bytes / (kernel_ms * 1e-3) / 1e9
    rec = work.describe()
    rec.update({
        "us_per_call": round(call_ms * 1e3, 2), "us_per_call_p10_p50_p90": pct(t_call),
        "GB_per_s": round(work.alg_bytes / (call_ms * 1e-3) / 1e9, 1),
        "us_per_launch": round(kernel_ms * 1e3, 2), "us_per_launch_p10_p50_p90": pct(t_kernel),
        "kernel_GB_per_s": round(kernel_gbs, 1), "frac": round(kernel_gbs / PEAK_HBM_GBS, 4),
        # the same at the median launch: a memory-system stall of one launch in
        # tens (~20-120 us longer) moves the mean of 50 but not the median
        "frac_at_median_launch": round(
            work.alg_bytes / (float(np.median(t_kernel)) * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "traffic": measured_traffic(work.name),
    })
    return rec, call_ms, kernel_ms, wall


def main():
    args = parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus must be 1 "
                          "(the path needs no collective and is not sharded here)"}))
        sys.exit(2)

    import torch

    import sparse_embedding_weight_amd as ewg
    from sparse_embedding_weight_amd import _binding as B
    import workloads as wl

    name = args.workload or wl.HEADLINE
    if name not in wl.WORKLOADS:
        raise SystemExit(f"unknown workload {name!r}; known: {', '.join(wl.WORKLOADS)}")
    if args.configs == "all":
        config_names = list(wl.WORKLOADS)
    elif args.configs == "none":
        config_names = []
    else:
        config_names = args.configs.split(",")
        for c in config_names:
            if c not in wl.WORKLOADS:
                raise SystemExit(f"unknown workload {c!r} in --configs")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    flush_sink = torch.zeros((), dtype=torch.float32, device=dev)
    hip = HipEvents()

    # the headline workload: value and roofline
    work = Workload(torch, ewg, B, wl, name, dev)
    w = work.w
    head, mean_call_ms, mean_kernel_ms, wall = measure(torch, ewg, B, hip, work, args, flush,
                                                       flush_sink)
    value = work.alg_bytes / (mean_call_ms * 1e-3) / 1e9
    achieved = work.alg_bytes / (mean_kernel_ms * 1e-3) / 1e9

    if args.copy_calibration:
        buf = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        for _ in range(3):
            buf.fill_(1)
        torch.cuda.synchronize()
        del buf

    cfg = work.describe()
    cfg["cache_flush_between_calls"] = args.flush
    result = {
        "metric": "us/call + achieved HBM GB/s, 8192 tokens into 129280x7168 main_grad",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mean_call_ms, 5),
        "us_per_call": head["us_per_call"],
        "us_per_call_p10_p50_p90": head["us_per_call_p10_p50_p90"],
        "wall_ms_per_step_incl_cache_flush": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{w.grad_dtype}->{w.main_grad_dtype}",
        "data": "synthetic",
        "config": cfg,
        "roofline": {"bound": "hbm", "kernel": "accumulate_kernel", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "algorithmic_bytes_per_launch": work.alg_bytes,
                     "us_per_launch": head["us_per_launch"],
                     "traffic": head["traffic"]},
    }

    if args.vocab_shards > 1:
        result["vocab_shards"] = time_vocab_shards(torch, ewg, wl, w, work.ids, work.ids_np,
                                                   work.grad, work.mg, flush, flush_sink,
                                                   args.flush, args.vocab_shards, args.steps,
                                                   args.warmup)

    if not args.no_dense_baseline:
        result["dense_baseline"] = dense_baseline(torch, w, work.ids, work.grad, work.mg, flush,
                                                  flush_sink, args.flush, mean_call_ms)
    ids_np, grad_cpu = work.ids_np, work.grad_cpu
    del work
    torch.cuda.empty_cache()

    # every generated workload (the headline's record is the one measured above)
    if config_names:
        configs = []
        for c in config_names:
            if c == name:
                configs.append(head)
                continue
            cw = Workload(torch, ewg, B, wl, c, dev)
            configs.append(measure(torch, ewg, B, hip, cw, args, flush, flush_sink)[0])
            del cw
            torch.cuda.empty_cache()
        result["configs"] = configs

    result["copy_ceiling"] = copy_ceiling(torch, dev)

    if not args.no_many_tokens:
        result["many_tokens"] = time_many_tokens(
            torch, ewg, B, wl, args.many_workload or wl.MANY_HEADLINE, hip, flush, flush_sink,
            args.flush, args.steps, args.warmup, not args.no_dense_baseline)

    if not args.no_cpu_baseline:
        threads = host_threads(args.cpu_threads)
        (t1, r1), (tn, rn), blocks = cpu_baseline(w, ids_np, wl.to_numpy_bits(grad_cpu),
                                                  args.cpu_seconds, threads)
        result["cpu_baseline"] = {
            "value": round(alg_bytes_of(result) / tn / 1e9, 3), "unit": "GB/s", "cores": blocks,
            "kind": "oracle", "seconds_per_call": round(tn, 4),
            "one_core": {"value": round(alg_bytes_of(result) / t1 / 1e9, 3), "unit": "GB/s",
                         "seconds_per_call": round(t1, 4), "calls": r1},
            "cpu_model": cpu_model(),
            "sample": f"the whole workload ({w.num_tokens} tokens, hidden {w.hidden}); main_grad "
                      f"restricted to its {result['config']['distinct_ids']} touched rows (ids "
                      f"relabelled in order); median of {rn} calls of the C oracle run at once "
                      f"on {blocks} column blocks, one thread each (one_core: median of {r1} "
                      f"serial calls)"}
    print(json.dumps(result), flush=True)


def alg_bytes_of(result):
    return result["config"]["algorithmic_bytes"]


if __name__ == "__main__":
    main()
