"""Benchmark of the two-stage RVQ KV-cache codec on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload llama_layer] [--gpus 1]

One step is one pass of the whole path over one synthetic layer: encode+pack of a
[1, 32, 8192, 128] fp16 key tensor at b = 2 bits per stage (4 outlier channels, random
signs), then an unpack+decode of a tensor of the same size. Inputs are resident in HBM before
timing starts and rotate through a pool of distinct tensors (and distinct output buffers)
larger than twice the 256 MB last-level cache, so every encode streams its input from HBM;
the decodes read their own pool of packed caches (also more than twice that cache), written
before the timed region.

Timing: the K steps' encodes run first, then their decodes, on one stream, in blocks of
min(10, K / 4) back-to-back launches. HIP events recorded on that stream bracket every
block, and the timed region is bracketed by device synchronisation on both sides; a short
spin kernel ahead of the first event keeps the stream busy while the host queues the first
launches (see prime). The average encode launch duration is the sum of the
encode blocks' spans over K (it includes the gaps between back-to-back launches); the
per-block averages give p10, p50, p90 and an A/A noise floor (even against odd blocks).
`value` is encode+pack throughput: algorithmic bytes per launch (fp16 bytes in + packed
bytes out; the 4-byte norms are reported separately, not counted) over that average,
checked against the 8 TB/s HBM peak in `roofline`. Before timing, the line records whether
any other process holds the GPU and how busy it is (`gpu_idle_check`), and which GPU, ROCm
and host it ran on (`host`). `cpu_baseline` is the CPU oracle timed on a bounded sample of
the same tensor, with its BLAS threads and with one thread.

`roofline.traffic` (measured HBM bytes per encode launch) comes from
profiles/traffic_<workload>.json, which `--traffic-from FETCH.csv WRITE.csv COPY_BYTES`
writes from two rocprofv3 counter runs of this script (FETCH_SIZE, then WRITE_SIZE, with
--copy-calibration, which adds plain device copies of a known size whose counter readings
give the scale factors). It is reported only while the kernel sources are unchanged since.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
LLC_BYTES = 256 << 20  # MI355X last-level (Infinity) cache
COPY_BYTES = 1 << 30  # --copy-calibration: one plain device copy reads and writes this many bytes
WORKLOADS = {
    # name: (tensor preset in synth.WORKLOADS, bits, pool size, stages)
    "llama_layer": ("llama_layer", 2, 8, 2),
    "gqa_long_b1": ("gqa_long", 1, 8, 2),
    "gqa_long_b4": ("gqa_long", 4, 8, 2),
    "prefill_kv_b4": ("prefill_kv", 4, 2, 2),
    # the single-stage codec (stage 1 only, one code stream) on the Llama layer
    "llama_layer_mse": ("llama_layer", 2, 8, 1),
    # 3 bits per stage: 10 codes per word, words straddle the lanes of a vector
    "llama_layer_b3": ("llama_layer", 3, 8, 2),
    # other head dimensions, same bytes as the Llama layer
    "head_dim_64": ("head_dim_64", 2, 8, 2),
    "head_dim_256": ("head_dim_256", 2, 8, 2),
    "head_dim_512": ("head_dim_512", 2, 8, 2),
    "head_dim_1024": ("head_dim_1024", 2, 8, 2),
}
# 1-bit sign codes of the Llama layer's keys: the RaBitQ-style code of the rotated vector
# (D bits + fp32 norm per vector) and the QJL sketch with m = 128 rows (128 bits + fp16 norm)
SIGN_WORKLOADS = {"rabitq_llama_layer": ("llama_layer", "rabitq", 0, 8),
                  "qjl_llama_layer_m128": ("llama_layer", "qjl", 128, 8)}
# attention over packed caches: one decode step of a GQA layer (32 query heads over 8
# key/value heads of the gqa_long cache shape [1, 8, 32768, 128], b = 2, keys and values)
ATTEND_WORKLOADS = {"attend_decode": {"B": 1, "Hq": 32, "Hkv": 8, "Sq": 1, "S_kv": 32768, "D": 128, "bits": 2,
                                      "pool": 16}}


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence: recording it
    does not write back and invalidate the caches with a system-scope fence, which a default
    event does, and which stalls the kernels queued behind it (about 2.8 us per event between
    back-to-back encodes of the Llama layer). The timed regions read these events only after a
    device synchronisation, so they need no fence. Same interface as torch.cuda.Event."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def hip(cls):
        if cls._hip is None:
            import ctypes
            # the HIP runtime this process already runs (torch's), found by its mapped path
            path = "libamdhip64.so"
            with open("/proc/self/maps") as f:
                for line in f:
                    if "libamdhip64.so" in line:
                        path = line.split()[-1]
                        break
            lib = ctypes.CDLL(path)
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = lib
        return cls._hip

    def __init__(self):
        import ctypes
        self._ev = ctypes.c_void_p()
        if self.hip().hipEventCreateWithFlags(ctypes.byref(self._ev), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream=None) -> None:
        import ctypes
        import torch
        if stream is None:
            stream = torch.cuda.current_stream()
        if self.hip().hipEventRecord(self._ev, ctypes.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end: "TimingEvent") -> float:
        """Milliseconds from this event to `end` (both recorded and complete)."""
        import ctypes
        ms = ctypes.c_float()
        if self.hip().hipEventElapsedTime(ctypes.byref(ms), self._ev, end._ev) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        if self._hip is not None and self._ev:
            self._hip.hipEventDestroy(self._ev)


PRIME_CYCLES = 1_000_000  # GPU clock cycles of the spin kernel that opens a timed region


def prime(stream) -> None:
    """Occupies the stream with a short spin kernel, enqueued after the pre-timing
    synchronisation and before the first timing event, so that the host's latency to its
    first launches (a few us each through ctypes) is hidden behind it: the first timed block
    then starts with launches already queued, as every later block does, and measures the
    kernels back to back rather than the host's catch-up. The spin itself is outside the
    events."""
    import torch
    if not hasattr(torch.cuda, "_sleep"):  # a torch without the spin kernel: no priming
        return
    with torch.cuda.stream(stream):
        torch.cuda._sleep(PRIME_CYCLES)


def output_sets(pool: int, set_bytes: int) -> int:
    """Number of output buffer sets an encode rotates through: the smallest multiple of the
    input pool whose bytes exceed twice the last-level cache (at most 128 sets), so a
    launch's writes never land in lines an earlier launch left in that cache, and encode k
    always pairs input k mod pool with output set k."""
    need = -(-(2 * LLC_BYTES + 1) // set_bytes)
    return pool * max(1, min(max(1, 128 // pool), -(-need // pool)))


def block_size(steps: int) -> int:
    """Launches per timed block: 10, or fewer so that even a short run has 4 blocks (the A/A
    noise floor compares even and odd blocks)."""
    return max(1, min(10, steps // 4))


def spread(per_block, block):
    """p10 / p50 / p90 of per-launch block averages (us), and the A/A noise floor: the
    relative gap between the medians of the even and the odd blocks (the same kernel on the
    same pool, interleaved in time)."""
    import numpy as np
    v = np.asarray(per_block, dtype=np.float64)
    out = {"blocks": int(v.size), "launches_per_block": block}
    for q in (10, 50, 90):
        out[f"p{q}"] = round(float(np.percentile(v, q)), 3)
    if v.size >= 4:
        a, b = float(np.median(v[0::2])), float(np.median(v[1::2]))
        out["aa_noise"] = round(abs(a - b) / float(np.median(v)), 4)
    return out


def encode_kernel_name(D: int, bits: int, contig: bool, stages: int) -> str:
    """The encode kernel libkvq launches for this shape (the matrix-core kernel covers
    D = 128 and, except at 3 bits, D = 256; the butterfly kernel everything else)."""
    c = "true" if contig else "false"
    if D == 128 or (D == 256 and bits != 3):
        return f"kvq::encode_mx_kernel<{D}, {bits}, {c}, {stages}>"
    return f"kvq::encode_kernel<{D}, {bits}, {c}, {stages}>"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("codec.h", "kernels.hip", "device.h", "params.h"):
        h.update(open(os.path.join(ROOT, "residual_vq_encode_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def host_info() -> dict:
    """The GPU, the ROCm stack and the host the numbers come from."""
    import torch
    info = {"host_cores": os.cpu_count()}
    try:
        info["affinity_cores"] = len(os.sched_getaffinity(0))
    except Exception:
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
                break
    except Exception:
        pass
    try:
        pr = torch.cuda.get_device_properties(0)
        info["gpu"] = pr.name
        info["gpu_arch"] = getattr(pr, "gcnArchName", "")
        info["gpu_cus"] = pr.multi_processor_count
    except Exception:
        pass
    info["torch_hip"] = torch.version.hip
    try:
        info["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except Exception:
        pass
    return info


def gpu_idle_check() -> dict:
    """Is anything else using the GPU? Other processes holding the device (their entries under
    /sys/class/kfd/kfd/proc) and the device's busy percentage, sampled a few times before the
    timed region. A busy GPU makes every timing below it wrong, so the line says so."""
    out = {}
    try:
        pids = [int(p) for p in os.listdir("/sys/class/kfd/kfd/proc") if p.isdigit()]
        out["other_gpu_processes"] = sorted(p for p in pids if p != os.getpid())
        out["source"] = "/sys/class/kfd/kfd/proc"
    except Exception:
        try:
            import re
            import subprocess
            if any(k.startswith("ROCPROF") for k in os.environ) or "rocprof" in os.environ.get("LD_PRELOAD", ""):
                # under a profiler every child process starts with its library preloaded (and the
                # GPU initialised), and rocm-smi's launcher hop would then replace such a process
                raise RuntimeError("skipped under a profiler")
            r = subprocess.run(["rocm-smi", "--showpids"], capture_output=True, text=True, timeout=20)
            pids = [int(m) for m in re.findall(r"^\s*(\d+)\s+\S+", r.stdout, re.M)]
            out["other_gpu_processes"] = sorted(p for p in pids if p != os.getpid()) if r.returncode == 0 else None
            out["source"] = "rocm-smi --showpids"
        except Exception as e:
            out["other_gpu_processes"] = None
            out["source"] = f"unavailable ({type(e).__name__})"
    busy = []
    try:
        import glob
        files = sorted(glob.glob("/sys/class/drm/card*/device/gpu_busy_percent"))
        for _ in range(5):
            busy.append(max(int(open(f).read()) for f in files))
            time.sleep(0.02)
    except Exception:
        busy = []
    out["gpu_busy_percent_samples"] = busy or None
    others = out["other_gpu_processes"]
    out["idle"] = (others is not None and len(others) == 0) and (not busy or max(busy) <= 10)
    return out


def stream_reference(in_bytes: int, out_bytes: int, reps: int = 50) -> dict:
    """A plain device-to-device copy (hipMemcpyAsync) moving the encode's total byte count:
    (in + out) / 2 bytes read and as many written, over a pool of distinct buffers larger than
    twice the last-level cache, back to back under events. A reference for what the machine
    streams without any arithmetic, next to the encode's own rate."""
    import torch
    dev = torch.device("cuda:0")
    half = ((in_bytes + out_bytes) // 2) // 16 * 16
    pool = max(2, -(-(2 * LLC_BYTES + 1) // (2 * half)))
    src = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(pool)]
    dst = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(pool)]
    for i in range(10):
        dst[i % pool].copy_(src[i % pool])
    torch.cuda.synchronize()
    e0, e1 = TimingEvent(), TimingEvent()
    e0.record()
    for i in range(reps):
        dst[i % pool].copy_(src[i % pool])
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return {"copy_us": round(us, 3), "copy_GBps": round(2 * half / us / 1e3, 1), "bytes_moved": 2 * half,
            "pool": pool, "kernel": "device-to-device copy (hipMemcpyAsync) of the same total bytes"}


def blas_threads() -> int:
    try:
        import threadpoolctl
        return max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas")
    except Exception:
        return 1


def one_thread(fn):
    """Run fn with the BLAS thread pools held to one thread (the oracle's other steps are
    single-threaded numpy already)."""
    try:
        import threadpoolctl
        with threadpoolctl.threadpool_limits(1):
            return fn()
    except ImportError:
        return fn()


def cpu_baseline(spec, signs, bits, stages: int = 2, target_s: float = 15.0) -> dict:
    """The oracle, as it stands, on a contiguous sample of the workload's first tensor: with
    numpy's BLAS thread pool as the process has it (only the Hadamard products use it; the
    nearest-centroid search and the packing are single-threaded numpy), and again held to
    one thread on a smaller sample."""
    import numpy as np
    import synth
    from oracle import codebooks as ocb
    from oracle import rvq
    t = ocb.build_tables(spec.D, bits)
    s = np.asarray(signs, np.int8)
    run = rvq.encode if stages == 2 else rvq.encode_mse
    probe = synth.rows(spec, 0, 8192).numpy()
    t0 = time.perf_counter()
    run(probe, s, t)
    dt_probe = time.perf_counter() - t0
    n = int(min(spec.rows, max(8192, 8192 * target_s / max(dt_probe, 1e-3))))
    n = (n // 8192) * 8192
    x = synth.rows(spec, 0, n).numpy()
    t0 = time.perf_counter()
    run(x, s, t)
    dt = time.perf_counter() - t0
    nw = -(-spec.D // (32 // bits))
    per_vec = spec.D * 2 + stages * nw * 4
    threads = blas_threads()
    n1 = min(n, 65536)
    x1 = x[:n1]
    t0 = time.perf_counter()
    one_thread(lambda: run(x1, s, t))
    dt1 = time.perf_counter() - t0
    info = host_info()
    return {"value": round(n * per_vec / dt / 1e9, 6), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {spec.rows} vectors of the workload tensor, encode+pack, {dt:.1f} s wall; "
                      f"numpy float64 oracle (not an optimised CPU codec), its Hadamard products on "
                      f"{threads} BLAS threads, the rest on one",
            "one_thread": {"value": round(n1 * per_vec / dt1 / 1e9, 6), "unit": "GB/s",
                           "sample": f"first {n1} vectors, {dt1:.1f} s wall, BLAS held to one thread"},
            "host_cores": info.get("host_cores"), "affinity_cores": info.get("affinity_cores"),
            "cpu_model": info.get("cpu_model")}


def traffic_for(workload: str):
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None, None
    rec = json.load(open(path))
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None, rec
    return rec.get("bytes_per_launch"), rec


def _counter_rows(path: str, counter: str):
    """(kernel name, value in bytes) per dispatch from a rocprofv3 counter_collection.csv.
    FETCH_SIZE and WRITE_SIZE are reported in KiB."""
    out = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") == counter:
                out.append((r["Kernel_Name"], float(r["Counter_Value"]) * 1024.0))
    return out


def traffic_from(fetch_csv: str, write_csv: str, workload: str, copy_bytes: int) -> dict:
    """Per-launch HBM bytes of the encode kernel from two counter runs. Each counter is
    scaled by (bytes a plain copy moves) / (what the counter reads for that copy)."""
    import statistics as st
    rec = {"workload": workload, "kernel_source_hash": kernel_source_hash(), "copy_bytes": copy_bytes}
    for name, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        rows = _counter_rows(path, counter)
        enc = [v for k, v in rows if "encode_kernel" in k or "encode_mx_kernel" in k]
        copy = [v for k, v in rows if "copy" in k.lower()]
        copy = [v for v in copy if v > copy_bytes / 4]  # the 1 GiB copies, not small helper kernels
        if not enc or not copy:
            raise SystemExit(f"{path}: no encode or copy dispatches with {counter}")
        factor = copy_bytes / st.median(copy)
        rec[name] = {"counter": counter, "encode_median_bytes": st.median(enc), "copy_median_bytes": st.median(copy),
                     "factor": factor, "encode_scaled_bytes": st.median(enc) * factor, "dispatches": len(enc)}
    rec["bytes_per_launch"] = round(rec["fetch"]["encode_scaled_bytes"] + rec["write"]["encode_scaled_bytes"])
    return rec


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 200; decode_append: its 2000 steps)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama_layer",
                    choices=sorted(WORKLOADS) + sorted(ATTEND_WORKLOADS) + sorted(SIGN_WORKLOADS)
                    + ["decode_append"])
    ap.add_argument("--pool", type=int, default=None, help="distinct input tensors to rotate through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help=f"also run plain {COPY_BYTES >> 30} GiB device copies (the counter-scaling reference)")
    ap.add_argument("--stream-reference", action="store_true",
                    help="also time a plain device copy moving the encode's total byte count")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<workload>.json from two rocprofv3 counter runs and exit")
    args = ap.parse_args()

    if args.traffic_from:
        rec = traffic_from(args.traffic_from[0], args.traffic_from[1], args.workload, COPY_BYTES)
        os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
        path = os.path.join(ROOT, "profiles", f"traffic_{args.workload}.json")
        json.dump(rec, open(path, "w"), indent=1)
        print(json.dumps(rec))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this codec runs on one GPU only (every vector is independent; a multi-GPU "
              "deployment shards the heads with no communication); run it with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import residual_vq_encode_amd as kvq
    import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    idle = gpu_idle_check()  # before this process puts any work on the GPU
    if args.workload == "decode_append":
        return bench_append(args, idle)
    if args.steps is None:
        args.steps = 200
    if args.workload in ATTEND_WORKLOADS:
        return bench_attend(args, idle)
    if args.workload in SIGN_WORKLOADS:
        return bench_signcodes(args, idle)
    wname, bits, pool_default, stages = WORKLOADS[args.workload]
    w = synth.WORKLOADS[wname]
    spec = w.tensors[0]
    P = args.pool or pool_default
    dev = torch.device("cuda:0")
    B, H, S, D = spec.B, spec.H, spec.S, spec.D
    signs = synth.signs(w.sign_seed, D).numpy()
    cb = kvq.build_codebooks(D, bits, signs)
    nw = cb.n_words

    # pool: the workload tensor itself plus P-1 more of the same recipe with other seeds
    xs = [synth.tensor(spec, device=dev)]
    for i in range(1, P):
        xs.append(synth.tensor(synth.TensorSpec(B, H, S, D, spec.kind, spec.seed + 1000 * i), device=dev))
    # The encodes write their own pool of packed outputs, more than twice the 256 MB
    # last-level cache, so their writes go to HBM rather than to lines still held there.
    packed_bytes = B * H * S * (stages * nw * 4 + 4)
    PO = output_sets(P, packed_bytes)
    p1s = [torch.empty((B, H, S, nw), dtype=torch.int32, device=dev) for _ in range(PO)]
    p2s = [torch.empty_like(p1s[0]) for _ in range(PO)]
    ns = [torch.empty((B, H, S), dtype=torch.float32, device=dev) for _ in range(PO)]
    outs = [torch.empty((B, H, S, D), dtype=torch.float16, device=dev) for _ in range(P)]
    stream = torch.cuda.current_stream()
    # The decodes read their own pool of packed caches, more than twice the 256 MB last-level
    # cache, each written by an encode before the timed region: a decode's input then comes
    # from HBM, not from the caches the encode blocks have just written.
    PD = min(64, max(P, -(-(2 * LLC_BYTES + 1) // packed_bytes)))
    dq1 = [torch.empty_like(p1s[0]) for _ in range(PD)]
    dq2 = [torch.empty_like(p1s[0]) for _ in range(PD)] if stages == 2 else None
    dqn = [torch.empty_like(ns[0]) for _ in range(PD)]

    if args.copy_calibration:
        a = torch.empty(COPY_BYTES // 2, dtype=torch.int16, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # Launches are prepared once (arguments checked and marshalled by the binding), so the
    # timed loop issues them as fast as the host can call the C ABI and the events measure
    # the GPU rather than per-call Python checks.
    encs = [kvq.prepare_encode(cb, xs[k % P], p1s[k], p2s[k] if stages == 2 else None, ns[k], 0, stream, stages)
            for k in range(PO)]
    decs = [kvq.prepare_decode(cb, dq1[k], dq2[k] if stages == 2 else None, dqn[k], outs[k % P], 0, stream, stages)
            for k in range(PD)]
    for k in range(PD):
        kvq.prepare_encode(cb, xs[k % P], dq1[k], dq2[k] if stages == 2 else None, dqn[k], 0, stream, stages)()

    def enc(j):
        encs[j % PO]()

    def dec(j):
        decs[j % PD]()

    # warm-up: the decodes first, then the encodes, so the timed encodes follow encodes
    for i in range(args.warmup):
        dec(i)
    for i in range(args.warmup):
        enc(i)
    torch.cuda.synchronize()

    # The K steps' encodes run first, then their decodes, all back to back, with one event
    # before the encodes, one between the two phases and one after the decodes: an event
    # between launches leaves a gap in the stream (about 0.4 us per launch with one every 5
    # launches), so the timed region holds none. Grouping the kernels keeps each in its own
    # steady state: a decode writes a 67 MB output, and encodes interleaved with the decodes
    # would share the HBM with the write-back of those bytes.
    K = args.steps
    ev = [TimingEvent() for _ in range(3)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    prime(stream)
    ev[0].record(stream)
    for i in range(K):
        enc(args.warmup + i)
    ev[1].record(stream)
    for i in range(K):
        dec(args.warmup + i)
    ev[2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    enc_us = ev[0].elapsed_time(ev[1]) * 1e3 / K
    dec_us = ev[1].elapsed_time(ev[2]) * 1e3 / K
    total_ms = ev[0].elapsed_time(ev[2])

    # Spread pass, after the timed region and not part of its figures: K more encodes, then K
    # more decodes, in blocks with an event after each block. The per-block averages give
    # p10 / p50 / p90 and the A/A noise floor (alternate blocks).
    BLOCK = block_size(K)
    blocks = [(a, min(a + BLOCK, K)) for a in range(0, K, BLOCK)]
    nb = len(blocks)
    evs = [TimingEvent() for _ in range(2 * nb + 1)]
    torch.cuda.synchronize()
    prime(stream)
    evs[0].record(stream)
    for bi, (a, b) in enumerate(blocks):
        for i in range(a, b):
            enc(args.warmup + K + i)
        evs[bi + 1].record(stream)
    for bi, (a, b) in enumerate(blocks):
        for i in range(a, b):
            dec(args.warmup + K + i)
        evs[nb + bi + 1].record(stream)
    torch.cuda.synchronize()
    enc_blk = [evs[bi].elapsed_time(evs[bi + 1]) * 1e3 / (b - a) for bi, (a, b) in enumerate(blocks)]
    dec_blk = [evs[nb + bi].elapsed_time(evs[nb + bi + 1]) * 1e3 / (b - a) for bi, (a, b) in enumerate(blocks)]

    n_vec = B * H * S
    enc_bytes = n_vec * (D * 2 + stages * nw * 4)
    dec_bytes = n_vec * (stages * nw * 4 + 4 + D * 2)
    enc_gbps = enc_bytes / (enc_us * 1e-6) / 1e9
    dec_gbps = dec_bytes / (dec_us * 1e-6) / 1e9

    # parity re-check of one timed output against the oracle on a sample of its vectors
    from oracle import codebooks as ocb
    from oracle import flips, rvq
    k = (args.warmup + K - 1) % PO
    j = k % P
    # a strided sample (the whole tensor when smaller): the flip cap is a rate. At b <= 2
    # flips are rare and 65536 vectors suffice; at b >= 3 the float32 transform leaves about
    # 5e-7 of the codes flipped next to a boundary, so the sample takes 2^18 vectors (67M
    # codes, a count of ~35 against a cap of 67) for its count to resolve the rate
    n_check = 65536 if bits <= 2 else 262144
    idx = torch.arange(0, n_vec, max(1, n_vec // n_check))[:n_check]
    rows = xs[j].reshape(-1, D)[idx.to(dev)].cpu().numpy()
    t = ocb.build_tables(D, bits)
    dev_p1 = p1s[k].reshape(-1, nw)[idx.to(dev)].cpu().numpy().view(np.uint32)
    dev_n = ns[k].reshape(-1)[idx.to(dev)].cpu().numpy()
    if stages == 2:
        ref = rvq.encode(rows, signs, t)
        rep = flips.compare_encode(dev_p1, p2s[k].reshape(-1, nw)[idx.to(dev)].cpu().numpy().view(np.uint32),
                                   dev_n, ref, t, 1e-5)
    else:
        rep = flips.compare_encode_single(dev_p1, dev_n, rvq.encode_mse(rows, signs, t), t, 1e-5)
    parity_ok = rep.ok(max(1e-6, 1.0 / max(1, rep.n_codes)), 1e-6)

    traffic, _ = traffic_for(args.workload)
    result = {
        "metric": "encode+pack GB/s (fp16 in + packed out) and % of HBM peak; tokens/sec",
        "value": round(enc_gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded counter-based generator; no dataset)",
        "config": {"workload": f"{args.workload}: {w.note.split('; b')[0]}; b={bits}"
                               + ("" if stages == 2 else "; single-stage codec"),
                   "shape": [B, H, S, D], "bits": bits, "stages": stages,
                   "pool_tensors": P, "encode_output_sets": PO, "step": "encode+pack then unpack+decode of one tensor"},
        "pct_of_hbm_peak": round(100.0 * enc_gbps / HBM_PEAK_GBPS, 2),
        "tokens_per_s": round(B * S / (enc_us * 1e-6), 1),
        "head_vectors_per_s": round(n_vec / (enc_us * 1e-6), 1),
        "encode_us_per_launch": round(enc_us, 3),
        "encode_us_blocks": spread(enc_blk, BLOCK),
        "spread_pass": "the blocks' figures come from K more launches after the timed region, "
                       "with an event after each block; value and the per-launch times do not use them",
        "decode_us_per_launch": round(dec_us, 3),
        "decode_us_blocks": spread(dec_blk, BLOCK),
        "decode_GBps": round(dec_gbps, 1),
        "decode_input_pool": {"caches": PD, "bytes": PD * packed_bytes,
                              "note": "decodes read packed caches written before the timed region, "
                                      "more than twice the last-level cache"},
        "norm_bytes_per_launch_not_counted": n_vec * 4,
        "wall_s_timed_region": round(wall, 4),
        "parity_recheck": {"vectors": int(len(idx)), "flip_fraction": rep.flip_fraction, "ok": bool(parity_ok)},
        "roofline": {"bound": "hbm", "achieved": round(enc_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(enc_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": enc_bytes, "kernel": encode_kernel_name(D, bits, True, stages)},
        "gpu_idle_check": idle,
        "host": host_info(),
    }
    if args.stream_reference:
        result["stream_reference"] = stream_reference(n_vec * D * 2, n_vec * stages * nw * 4)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(spec, signs, bits, stages)
    print(json.dumps(result), flush=True)
    return 0 if parity_ok else 1


def bench_signcodes(args, idle: dict) -> int:
    """One 1-bit sign-code encoder over the workload tensor: K launches back to back over a
    pool of distinct inputs and outputs, events around the group, then a parity re-check of
    the last output on a sample of its vectors."""
    import numpy as np
    import torch

    import residual_vq_encode_amd as kvq
    import synth
    from oracle import packing, signcodes

    wname, kind, m, pool_default = SIGN_WORKLOADS[args.workload]
    w = synth.WORKLOADS[wname]
    spec = w.tensors[0]
    P = args.pool or pool_default
    dev = torch.device("cuda:0")
    B, H, S, D = spec.B, spec.H, spec.S, spec.D
    n_vec = B * H * S
    xs = [synth.tensor(spec, device=dev)]
    for i in range(1, P):
        xs.append(synth.tensor(synth.TensorSpec(B, H, S, D, spec.kind, spec.seed + 1000 * i), device=dev))
    stream = torch.cuda.current_stream()
    if kind == "rabitq":
        signs = synth.signs(w.sign_seed, D).numpy()
        cb = kvq.build_codebooks(D, 1, signs)
        nw = cb.n_words
        PO = output_sets(P, n_vec * (nw * 4 + 4))
        ps = [torch.empty((B, H, S, nw), dtype=torch.int32, device=dev) for _ in range(PO)]
        ns = [torch.empty((B, H, S), dtype=torch.float32, device=dev) for _ in range(PO)]

        def enc(j):
            kvq.kvq_rabitq_encode_pack(cb, xs[j % P], ps[j % PO], ns[j % PO], 0, stream)
        out_bytes, norm_bytes, kname = nw * 4, 4, encode_kernel_name(D, 1, True, 0)
    else:
        sk = synth.tensor(synth.TensorSpec(1, 1, m, D, "gauss", 707), device=dev).reshape(m, D).contiguous()
        nw = m // 32
        PO = output_sets(P, n_vec * (nw * 4 + 2))
        ps = [torch.empty((B, H, S, nw), dtype=torch.int32, device=dev) for _ in range(PO)]
        ns = [torch.empty((B, H, S), dtype=torch.float16, device=dev) for _ in range(PO)]

        def enc(j):
            kvq.kvq_qjl_encode_pack(sk, xs[j % P], ps[j % PO], ns[j % PO], 0, stream)
        out_bytes, norm_bytes, kname = nw * 4, 2, f"kvq::qjl_encode_kernel<{D}, {m // 32}, true>"

    for i in range(args.warmup):
        enc(i)
    torch.cuda.synchronize()
    K = args.steps
    e0, e1 = TimingEvent(), TimingEvent()
    wall0 = time.perf_counter()
    prime(stream)
    e0.record(stream)
    for i in range(K):
        enc(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    us = e0.elapsed_time(e1) * 1e3 / K
    alg = n_vec * (D * 2 + out_bytes)
    gbps = alg / (us * 1e-6) / 1e9

    # parity re-check on a strided sample of the last timed output, and the oracle's time
    k = (args.warmup + K - 1) % PO
    idx = torch.arange(0, n_vec, max(1, n_vec // 65536))
    rows = xs[k % P].reshape(-1, D)[idx.to(dev)].cpu().numpy()
    dev_p = ps[k].reshape(-1, nw)[idx.to(dev)].cpu().numpy().view(np.uint32)
    dev_n = ns[k].reshape(-1)[idx.to(dev)].cpu().numpy()
    t0 = time.perf_counter()
    if kind == "rabitq":
        ref = signcodes.rabitq_encode(rows, signs)
        diff = packing.unpack(dev_p, 1, D) != ref["bits"]
        in_window = bool(np.all(np.abs(ref["y"][diff]) <= 1e-5 / math.sqrt(D)))
        norm_ok = bool(np.all(np.abs(dev_n - ref["norm64"]) <= 1e-6 * ref["norm64"]))
    else:
        ref = signcodes.qjl_encode(rows, sk.cpu().numpy())
        diff = packing.unpack(dev_p, 1, m) != ref["bits"]
        in_window = bool(np.all(np.abs(ref["dots"][diff]) <= D * 2.0 ** -24 * ref["absdots"][diff]))
        lo = (ref["norm64"] * (1 - 1e-6)).astype(np.float16)
        hi = (ref["norm64"] * (1 + 1e-6)).astype(np.float16)
        norm_ok = bool(np.all((dev_n == lo) | (dev_n == hi)))
    dt_oracle = time.perf_counter() - t0
    frac = float(diff.mean())
    ok = in_window and norm_ok and frac <= max(1e-6, 1.0 / diff.size)
    cores = blas_threads()
    result = {
        "metric": "encode+pack GB/s (fp16 in + packed out) and % of HBM peak; tokens/sec",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "gpu_idle_check": idle, "host": host_info(),
        "ms_per_step": round(us / 1e3, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic (seeded counter-based generator; no dataset)",
        "config": {"workload": f"{args.workload}: {w.note.split('; b=')[0]}; " + (
            "1-bit sign code of the rotated vector + fp32 norm" if kind == "rabitq"
            else f"1-bit sign sketch, m = {m} Gaussian rows (fp16) + fp16 norm"),
            "shape": [B, H, S, D], "pool_tensors": P, "encode_output_sets": PO},
        "pct_of_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "tokens_per_s": round(B * S / (us * 1e-6), 1), "encode_us_per_launch": round(us, 3),
        "norm_bytes_per_launch_not_counted": n_vec * norm_bytes, "wall_s_timed_region": round(wall, 4),
        "parity_recheck": {"vectors": int(len(idx)), "differing_bit_fraction": frac, "ok": bool(ok)},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None, "algorithmic_bytes_per_launch": alg,
                     "kernel": kname},
        "cpu_baseline": {"value": round(len(idx) * (D * 2 + out_bytes) / dt_oracle / 1e9, 6), "unit": "GB/s",
                         "cores": cores, "kind": "oracle",
                         "sample": f"{len(idx)} of {n_vec} vectors (strided), {dt_oracle:.1f} s wall, numpy oracle"},
    }
    if kind == "qjl":
        result["mfma"] = {"flops_per_launch": 2 * n_vec * m * D,
                          "tflops": round(2 * n_vec * m * D / (us * 1e-6) / 1e12, 1), "peak_fp16_tflops": 2500.0}
    print(json.dumps(result), flush=True)
    return 0 if ok else 1


def bench_attend(args, idle: dict) -> int:
    """kvq_rvq_attend on one decode step: K launches back to back over a pool of distinct
    packed caches (device-encoded; pool larger than the last-level cache), events around
    the group. The parity re-check runs on a cache the oracle encoded itself."""
    import numpy as np
    import torch

    import residual_vq_encode_amd as kvq
    import synth
    from oracle import attend as oatt
    from oracle import codebooks as ocb
    from oracle import rvq

    cfg = ATTEND_WORKLOADS[args.workload]
    B, Hq, Hkv, Sq, S, D, bits = (cfg[k] for k in ("B", "Hq", "Hkv", "Sq", "S_kv", "D", "bits"))
    P = args.pool or cfg["pool"]
    dev = torch.device("cuda:0")
    sk, sv = synth.signs(103, D).numpy(), synth.signs(203, D).numpy()
    cbk, cbv = kvq.build_codebooks(D, bits, sk), kvq.build_codebooks(D, bits, sv)
    nw = cbk.n_words
    stream = torch.cuda.current_stream()

    def dev_cache(seed, cb):
        x = synth.tensor(synth.TensorSpec(B, Hkv, S, D, "gauss_laplace_heads", seed), device=dev)
        p1, p2, n = kvq.encode(x, cb)
        return p1, p2, n

    kcs = [dev_cache(3 + 1000 * i, cbk) for i in range(P)]
    vcs = [dev_cache(5 + 1000 * i, cbv) for i in range(P)]
    qs = [synth.tensor(synth.TensorSpec(B, Hq, Sq, D, "gauss", 77 + i), device=dev) for i in range(P)]
    outs = [torch.empty_like(qs[0]) for _ in range(P)]
    ws = torch.empty(kvq.kvq_rvq_attend_workspace_size(D, bits, B, Hq, Sq, Hkv, S) // 4 + 4, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(D)

    def run(j):
        kvq.kvq_rvq_attend(cbk, cbv, qs[j], kcs[j], vcs[j], S, scale, ws, outs[j], stream)

    for i in range(args.warmup):
        run(i % P)
    torch.cuda.synchronize()
    K = args.steps
    e0, e1 = TimingEvent(), TimingEvent()
    wall0 = time.perf_counter()
    prime(stream)
    e0.record(stream)
    for i in range(K):
        run((args.warmup + i) % P)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    us = e0.elapsed_time(e1) * 1e3 / K
    gq = (Hq // Hkv) * Sq  # query vectors per key/value head; a wave serves nqw of them
    if D in (64, 128) and bits != 3 and D * bits >= 128:
        nqw = 16  # the matrix-core pass
    else:
        nqw = 4 if gq % 4 == 0 and D <= 512 else 2 if gq % 2 == 0 and D <= 512 else 1
    cache_bytes = B * Hkv * S * 2 * (2 * nw * 4 + 4)
    alg = cache_bytes + 2 * B * Hq * Sq * D * 2
    gbps = alg / (us * 1e-6) / 1e9

    # parity re-check on caches the oracle encoded (uploaded), against the oracle's attention
    tk = ocb.build_tables(D, bits)
    hosts, devs = [], []
    for seed, signs in ((3, sk), (5, sv)):
        x = synth.rows(synth.TensorSpec(B, Hkv, S, D, "gauss_laplace_heads", seed)).numpy()
        e = rvq.encode(x, signs, tk)
        h = (e["packed1"].reshape(B, Hkv, S, nw), e["packed2"].reshape(B, Hkv, S, nw), e["norms"].reshape(B, Hkv, S))
        hosts.append(h)
        devs.append(tuple(torch.from_numpy(a.view(np.int32) if a.dtype == np.uint32 else a).to(dev) for a in h))
    out = kvq.attend(qs[0], devs[0], devs[1], cbk, cbv, S, scale)
    torch.cuda.synchronize()
    qh = qs[0].cpu().numpy()
    t0 = time.perf_counter()
    want = oatt.attend(qh, hosts[0], hosts[1], sk, sv, tk, tk, S, scale).astype(np.float64)
    dt_oracle = time.perf_counter() - t0
    got = out.cpu().numpy().astype(np.float64)
    rowmax = np.max(np.abs(want), axis=-1, keepdims=True)
    ok = bool(np.all(np.abs(got - want) <= 2.0 ** -10 * np.abs(want) + 1e-3 * rowmax))
    cores = blas_threads()
    result = {
        "metric": "attention over the packed cache: packed key+value bytes read per second (GB/s); decode steps/s",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic (seeded counter-based generator; no dataset)",
        "config": {"workload": f"{args.workload}: one decode step, q [{B},{Hq},{Sq},{D}] over packed K and V "
                               f"[{B},{Hkv},{S},{D}] b={bits}", "bits": bits, "pool": P},
        "us_per_step": round(us, 3), "steps_per_s": round(1e6 / us, 1), "gpu_idle_check": idle, "host": host_info(),
        "parity_recheck": {"query_vectors": B * Hq * Sq, "ok": ok,
                           "max_rel_err": float(np.max(np.abs(got - want) / np.maximum(rowmax, 1e-30)))},
        "wall_s_timed_region": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None, "algorithmic_bytes_per_launch": alg,
                     "kernel": (f"kvq::attend_mfma<{D}, {bits}>" if nqw == 16 else f"kvq::attend_partial<{D}, {bits}, {nqw}>")
                               + f" + attend_combine<{D}>"},
        "cpu_baseline": {"value": round(alg / dt_oracle / 1e9, 6), "unit": "GB/s", "cores": cores, "kind": "oracle",
                         "sample": f"the whole step ({B * Hq * Sq} query vectors over {S} positions), "
                                   f"{dt_oracle:.1f} s wall, numpy float64 oracle"},
    }
    print(json.dumps(result), flush=True)
    return 0 if ok else 1


def bench_append(args, idle: dict) -> int:
    """Decode-step appends: step t encodes one token for every (batch, head) of
    [256, 8, 1, 128] into caches [256, 8, 32768, n_words] at s_offset = t. K steps with
    distinct inputs run back to back twice: launched one by one from the host (eager), and
    replayed from one captured graph of the same K launches. The graph's span is the device
    time per step; the eager span also counts the host's launch cost."""
    import numpy as np
    import torch

    import residual_vq_encode_amd as kvq
    import synth
    from oracle import codebooks as ocb
    from oracle import flips, rvq

    w = synth.WORKLOADS["decode_append"]
    spec = w.tensors[0]
    B, H, D, S_cap = spec.B, spec.H, spec.D, synth.DECODE_APPEND_S_CAP
    bits = w.bits[0]
    K = min(args.steps if args.steps is not None else spec.S, spec.S)
    dev = torch.device("cuda:0")
    signs = synth.signs(w.sign_seed, D).numpy()
    cb = kvq.build_codebooks(D, bits, signs)
    nw = cb.n_words
    p1 = torch.empty((B, H, S_cap, nw), dtype=torch.int32, device=dev)
    p2 = torch.empty_like(p1)
    nrm = torch.empty((B, H, S_cap), dtype=torch.float32, device=dev)
    steps = [synth.step_rows(spec, t, device=dev).contiguous() for t in range(K)]
    stream = torch.cuda.current_stream()

    # one prepared launch per step and stream (arguments checked and marshalled once)
    launches = {}

    def run_all():
        st = torch.cuda.current_stream()
        key = st.cuda_stream
        if key not in launches:
            launches[key] = [kvq.prepare_encode(cb, steps[t], p1, p2, nrm, t, st) for t in range(K)]
        for launch in launches[key]:
            launch()

    for t in range(min(args.warmup, K)):
        kvq.kvq_rvq_encode_pack(cb, steps[t], p1, p2, nrm, t, stream)
    torch.cuda.synchronize()

    e0, e1 = TimingEvent(), TimingEvent()
    run_all()  # prepares this stream's launches (and runs the steps once, untimed)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record(stream)
    run_all()
    e1.record(stream)
    torch.cuda.synchronize()
    wall_eager = time.perf_counter() - wall0
    eager_us = e0.elapsed_time(e1) * 1e3 / K

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            run_all()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g.replay()  # untimed first replay
    torch.cuda.synchronize()
    g0, g1 = TimingEvent(), TimingEvent()
    wall0 = time.perf_counter()
    g0.record(stream)
    g.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    graph_us = g0.elapsed_time(g1) * 1e3 / K

    # parity of sampled steps of the replayed caches against the oracle
    t_tab = ocb.build_tables(D, bits)
    ok = True
    n_flip = n_codes = 0
    for t in sorted({0, K // 2, K - 1}):
        rows = steps[t].reshape(-1, D).cpu().numpy()
        ref = rvq.encode(rows, signs, t_tab)
        rep = flips.compare_encode(p1[:, :, t].reshape(-1, nw).cpu().numpy().view(np.uint32),
                                   p2[:, :, t].reshape(-1, nw).cpu().numpy().view(np.uint32),
                                   nrm[:, :, t].reshape(-1).cpu().numpy(), ref, t_tab, 1e-5)
        ok = ok and rep.ok(max(1e-6, 1.0 / max(1, rep.n_codes)), 1e-6)
        n_flip += rep.flip_fraction * rep.n_codes
        n_codes += rep.n_codes

    step_bytes = B * H * (D * 2 + 2 * nw * 4)
    result = {
        "metric": "decode-step append: tokens/s (one token of every sequence per step) and us/step",
        "value": round(B / (graph_us * 1e-6), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(graph_us / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded counter-based generator; no dataset)",
        "config": {"workload": f"decode_append: {K} steps of [{B},{H},1,{D}] appended into S_cap={S_cap} caches; b={bits}",
                   "bits": bits, "timing": "one captured graph of the K launches, replayed"},
        "gpu_idle_check": idle, "host": host_info(),
        "us_per_step_graph": round(graph_us, 3),
        "us_per_step_eager": round(eager_us, 3),
        "wall_s_timed_region": round(wall, 4),
        "wall_s_eager": round(wall_eager, 4),
        "parity_recheck": {"steps": sorted({0, K // 2, K - 1}), "flip_fraction": n_flip / max(1, n_codes), "ok": bool(ok)},
        "roofline": {"bound": "launch", "achieved": round(step_bytes / (graph_us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(step_bytes / (graph_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 5),
                     "traffic": None, "algorithmic_bytes_per_launch": step_bytes,
                     "kernel": encode_kernel_name(D, bits, False, 2)},
    }
    if not args.no_cpu_baseline:
        n_s = min(K, 20)
        x = np.concatenate([steps[t].reshape(-1, D).cpu().numpy() for t in range(n_s)])
        t0 = time.perf_counter()
        rvq.encode(x, signs, t_tab)
        dt = time.perf_counter() - t0
        cores = blas_threads()
        result["cpu_baseline"] = {"value": round(n_s * B / dt, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
                                  "sample": f"the first {n_s} steps ({n_s * B * H} vectors), encode+pack, {dt:.2f} s wall, "
                                            f"numpy float64 oracle"}
    print(json.dumps(result), flush=True)
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
