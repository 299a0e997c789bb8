"""Benchmark of the embedding weight-gradient accumulation on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

One step = one whole call (one kernel: sort, chunk sums, single-chunk runs,
ordered combine of long runs) over the headline workload: 8192 Zipf(1.1) token ids into a 129280 x 7168 fp32
main_grad with a bf16 grad. Inputs are resident in HBM before timing. Before
every step, outside its timed interval, a 1 GiB buffer is read (summed) so
that neither L2 nor the 256 MB Infinity Cache holds the inputs; reading
rather than writing leaves no dirty lines for the timed call to write back.
Each step is timed with two HIP events that the library records on its
launch stream right before and after the call (value, us_per_call). A second
pass of the same steps dispatches the kernel with two more events of its own
(roofline.achieved and us_per_launch: the kernel's execution alone, the figure
a kernel trace shows); that pass is kept apart because such a dispatch adds
time around the kernel.

Prints one JSON line: value = algorithmic bytes / mean call time (GB/s), the
roofline of the kernel (the whole call is one kernel), and the CPU oracle
timed on the host as cpu_baseline. Also timed, each in its own object: the
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
    p.add_argument("--workload", default=None)
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
                   help="also run a 256 MiB device copy (reference for counter scaling)")
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


def kernel_source_hash():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "sparse_embedding_weight_amd", "csrc", name), "rb") as f:
            h.update(f.read())
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


def cpu_baseline(w, ids_np, grad_np, budget_s):
    """The oracle as it stands (single-threaded C), on the whole workload with
    main_grad restricted to its touched rows (ids relabelled in order)."""
    import oracle
    import workloads as wl

    rows = np.unique(ids_np)
    compact = np.searchsorted(rows, ids_np).astype(np.int32)
    rng = np.random.default_rng(0)
    mg = wl.to_numpy_bits(wl.normal_tensor(rng, (rows.size, w.hidden), w.main_grad_sigma,
                                           w.main_grad_dtype))
    times = []
    start = time.perf_counter()
    while not times or (time.perf_counter() - start < budget_s and len(times) < 20):
        m = mg.copy()
        t0 = time.perf_counter()
        oracle.accumulate_embedding_wgrad(compact, grad_np, m, w.grad_dtype, w.main_grad_dtype)
        times.append(time.perf_counter() - t0)
    return float(np.median(times)), len(times)


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
    w = wl.WORKLOADS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    ids_np = wl.make_ids(w).reshape(-1)
    ids = torch.from_numpy(ids_np).to(dev)
    grad_cpu = wl.make_grad(w).reshape(w.num_tokens, w.hidden)
    grad = grad_cpu.to(dev)
    mg = wl.make_main_grad(w, dev)
    counts = np.bincount(ids_np, minlength=w.vocab)
    uniq = int((counts > 0).sum())
    u_long = int((counts > ewg.NROWS).sum())
    alg_bytes = wl.algorithmic_bytes(w.num_tokens, w.hidden, uniq, w.grad_dtype,
                                     w.main_grad_dtype, ids_np.itemsize)

    ws = ewg.new_workspace(w.num_tokens, w.hidden, dev)
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    flush_sink = torch.zeros((), dtype=torch.float32, device=dev)
    hip = HipEvents()
    nsteps = args.warmup + args.steps
    stream = torch.cuda.current_stream(dev).cuda_stream
    call_args = (ids.data_ptr(), grad.data_ptr(), mg.data_ptr(), w.num_tokens, w.hidden, w.vocab,
                 grad.stride(0), mg.stride(0), B.DTYPE_CODE[ids.dtype], B.DTYPE_CODE[grad.dtype],
                 B.DTYPE_CODE[mg.dtype], ws.data_ptr(), ws.numel(), stream)

    def timed_pass(kernel_events):
        """warmup + steps calls; per timed call the (call, kernel) durations in ms.
        Without kernel_events the kernel is dispatched plainly (slots 2, 3 NULL):
        a dispatch that takes its own events costs extra time around it."""
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
            st = B.lib.accumulate_embedding_wgrad_timed(*call_args, slots[step])
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

    # value and us_per_call: plain dispatches between the call's own events
    t_call, _, wall = timed_pass(False)
    # roofline: the kernel's execution alone, from events its dispatch takes
    _, t_kernel, _ = timed_pass(True)
    timeouts = ewg.wait_timeouts(ws)
    if timeouts:
        raise RuntimeError(f"{timeouts} bounded waits gave up inside the kernel")

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    mean_call_ms = float(t_call.mean())
    value = alg_bytes / (mean_call_ms * 1e-3) / 1e9
    mean_kernel_ms = float(t_kernel.mean())
    achieved = alg_bytes / (mean_kernel_ms * 1e-3) / 1e9

    result = {
        "metric": "us/call + achieved HBM GB/s, 8192 tokens into 129280x7168 main_grad",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mean_call_ms, 5),
        "us_per_call": round(mean_call_ms * 1e3, 2),
        "us_per_call_p10_p50_p90": [round(float(np.percentile(t_call, q)) * 1e3, 2) for q in (10, 50, 90)],
        "wall_ms_per_step_incl_cache_flush": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": name, "num_tokens": w.num_tokens, "vocab": w.vocab,
                   "hidden": w.hidden, "ids": f"{w.ids_kind}" + (f"(s={w.zipf_s})" if w.ids_kind == "zipf" else ""),
                   "grad_dtype": w.grad_dtype, "main_grad_dtype": w.main_grad_dtype,
                   "distinct_ids": uniq, "runs_longer_than_10": u_long,
                   "algorithmic_bytes": alg_bytes, "cache_flush_between_calls": args.flush},
        "roofline": {"bound": "hbm", "kernel": "accumulate_kernel", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "us_per_launch": round(mean_kernel_ms * 1e3, 2),
                     "traffic": measured_traffic(name)},
    }

    if args.vocab_shards > 1:
        result["vocab_shards"] = time_vocab_shards(torch, ewg, wl, w, ids, ids_np, grad, mg, flush,
                                                   flush_sink, args.flush, args.vocab_shards,
                                                   args.steps, args.warmup)

    if not args.no_dense_baseline:
        result["dense_baseline"] = dense_baseline(torch, w, ids, grad, mg, flush, flush_sink,
                                                  args.flush, mean_call_ms)

    if not args.no_many_tokens:
        result["many_tokens"] = time_many_tokens(
            torch, ewg, B, wl, args.many_workload or wl.MANY_HEADLINE, hip, flush, flush_sink,
            args.flush, args.steps, args.warmup, not args.no_dense_baseline)

    if not args.no_cpu_baseline:
        t_cpu, reps = cpu_baseline(w, ids_np, wl.to_numpy_bits(grad_cpu), args.cpu_seconds)
        result["cpu_baseline"] = {
            "value": round(alg_bytes / t_cpu / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "seconds_per_call": round(t_cpu, 4),
            "sample": f"the whole workload ({w.num_tokens} tokens, hidden {w.hidden}); main_grad "
                      f"restricted to its {uniq} touched rows (ids relabelled in order); median of "
                      f"{reps} calls of the single-threaded C oracle"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
