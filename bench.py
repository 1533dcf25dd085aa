"""Benchmark of the two-stage RVQ KV-cache codec on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload llama_layer] [--gpus 1]

One step is one pass of the whole path over one synthetic layer: encode+pack of a
[1, 32, 8192, 128] fp16 key tensor at b = 2 bits per stage (4 outlier channels, random
signs), then the unpack+decode round trip of the packed result. Inputs are resident in HBM
before timing starts and rotate through a pool of distinct tensors (and distinct output
buffers) larger than twice the 256 MB last-level cache, so every launch streams from HBM.

Timing: HIP events recorded on the stream the kernels run on bracket every encode and
every decode launch; the whole timed region is bracketed by device synchronisation. The
printed JSON line reports encode+pack throughput (fp16 bytes in + packed bytes out, per
launch, over the mean encode-launch duration) as `value`, against the 8 TB/s HBM peak in
`roofline`, and the CPU oracle timed on a bounded sample as `cpu_baseline`.

`traffic` (measured HBM bytes per launch) is read from profiles/traffic_<workload>.json,
written from two rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE) scaled by a plain copy of
known size; it is reported only if the encode kernel source is unchanged since then.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
WORKLOADS = {
    # name: (tensor spec index in synth.WORKLOADS, bits, pool size)
    "llama_layer": ("llama_layer", 2, 8),
    "gqa_long_b1": ("gqa_long", 1, 8),
    "gqa_long_b4": ("gqa_long", 4, 8),
}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("kernels.hip", "params.h"):
        h.update(open(os.path.join(ROOT, "residual_vq_encode_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def cpu_baseline(spec, signs, bits, target_s: float = 15.0) -> dict:
    """The oracle, as it stands, on a contiguous sample of the workload's first tensor."""
    import numpy as np
    import synth
    from oracle import codebooks as ocb
    from oracle import rvq
    t = ocb.build_tables(spec.D, bits)
    s = np.asarray(signs, np.int8)
    probe = synth.rows(spec, 0, 8192).numpy()
    t0 = time.perf_counter()
    rvq.encode(probe, s, t)
    dt_probe = time.perf_counter() - t0
    n = int(min(spec.rows, max(8192, 8192 * target_s / max(dt_probe, 1e-3))))
    n = (n // 8192) * 8192
    x = synth.rows(spec, 0, n).numpy()
    t0 = time.perf_counter()
    rvq.encode(x, s, t)
    dt = time.perf_counter() - t0
    nw = -(-spec.D // (32 // bits))
    nbytes = n * (spec.D * 2 + 2 * nw * 4)
    try:
        import threadpoolctl
        cores = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas")
    except Exception:
        cores = os.cpu_count()
    return {"value": round(nbytes / dt / 1e9, 6), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"first {n} of {spec.rows} vectors of the workload tensor, encode+pack, "
                      f"{dt:.1f} s wall, numpy float64 oracle on {cores} BLAS threads"}


def traffic_for(workload: str):
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None, None
    rec = json.load(open(path))
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None, rec
    return rec.get("bytes_per_launch"), rec


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama_layer", choices=sorted(WORKLOADS))
    ap.add_argument("--pool", type=int, default=None, help="distinct input tensors to rotate through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run plain 1 GiB device copies (the counter-scaling reference)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this codec runs on one GPU only (every vector is independent; see the "
              "sharding note in DESIGN.md); run it with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import residual_vq_encode_amd as kvq
    import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    wname, bits, pool_default = WORKLOADS[args.workload]
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
    p1s = [torch.empty((B, H, S, nw), dtype=torch.int32, device=dev) for _ in range(P)]
    p2s = [torch.empty_like(p1s[0]) for _ in range(P)]
    ns = [torch.empty((B, H, S), dtype=torch.float32, device=dev) for _ in range(P)]
    outs = [torch.empty((B, H, S, D), dtype=torch.float16, device=dev) for _ in range(P)]
    stream = torch.cuda.current_stream()

    def step(i):
        j = i % P
        kvq.kvq_rvq_encode_pack(cb, xs[j], p1s[j], p2s[j], ns[j], 0, stream)
        kvq.kvq_rvq_unpack_decode(cb, p1s[j], p2s[j], ns[j], outs[j], 0, stream)

    if args.copy_calibration:
        a = torch.empty(1 << 29, dtype=torch.int16, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(K):
        j = (args.warmup + i) % P
        ev[i][0].record(stream)
        kvq.kvq_rvq_encode_pack(cb, xs[j], p1s[j], p2s[j], ns[j], 0, stream)
        ev[i][1].record(stream)
        kvq.kvq_rvq_unpack_decode(cb, p1s[j], p2s[j], ns[j], outs[j], 0, stream)
        ev[i][2].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0

    enc_ms = np.array([a.elapsed_time(b) for a, b, _ in ev])
    dec_ms = np.array([b.elapsed_time(c) for _, b, c in ev])
    total_ms = t_start.elapsed_time(t_end)
    n_vec = B * H * S
    enc_bytes = n_vec * (D * 2 + 2 * nw * 4)
    dec_bytes = n_vec * (2 * nw * 4 + 4 + D * 2)
    enc_mean_s = float(enc_ms.mean()) / 1e3
    enc_gbps = enc_bytes / enc_mean_s / 1e9
    dec_gbps = dec_bytes / (float(dec_ms.mean()) / 1e3) / 1e9

    # parity re-check of one timed output against the oracle on a sample of its vectors
    from oracle import codebooks as ocb
    from oracle import flips, rvq
    j = (args.warmup + K - 1) % P
    torch.cuda.synchronize()
    idx = torch.arange(0, n_vec, max(1, n_vec // 4096))
    rows = xs[j].reshape(-1, D)[idx.to(dev)].cpu().numpy()
    t = ocb.build_tables(D, bits)
    ref = rvq.encode(rows, signs, t)
    rep = flips.compare_encode(p1s[j].reshape(-1, nw)[idx.to(dev)].cpu().numpy().view(np.uint32),
                               p2s[j].reshape(-1, nw)[idx.to(dev)].cpu().numpy().view(np.uint32),
                               ns[j].reshape(-1)[idx.to(dev)].cpu().numpy(), ref, t, 1e-5)
    parity_ok = rep.ok(1e-6, 1e-6)

    traffic, trec = traffic_for(args.workload)
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
        "dtype": "fp16 in, fp32 compute, u32 packed out",
        "data": "synthetic (seeded counter-based generator; no dataset)",
        "config": {"workload": f"{wname}: {w.note}", "shape": [B, H, S, D], "bits": bits,
                   "pool_tensors": P, "step": "encode+pack then unpack+decode of one tensor"},
        "pct_of_hbm_peak": round(100.0 * enc_gbps / HBM_PEAK_GBPS, 2),
        "tokens_per_s": round(B * S / enc_mean_s, 1),
        "head_vectors_per_s": round(n_vec / enc_mean_s, 1),
        "encode_us": {"mean": round(float(enc_ms.mean()) * 1e3, 3), "p10": round(float(np.percentile(enc_ms, 10)) * 1e3, 3),
                      "p50": round(float(np.median(enc_ms)) * 1e3, 3), "p90": round(float(np.percentile(enc_ms, 90)) * 1e3, 3)},
        "decode_us": {"mean": round(float(dec_ms.mean()) * 1e3, 3), "p50": round(float(np.median(dec_ms)) * 1e3, 3)},
        "decode_GBps": round(dec_gbps, 1),
        "norm_bytes_per_launch_not_counted": n_vec * 4,
        "wall_s_timed_region": round(wall, 4),
        "parity_recheck": {"vectors": int(len(idx)), "flip_fraction": rep.flip_fraction, "ok": bool(parity_ok)},
        "roofline": {"bound": "hbm", "achieved": round(enc_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(enc_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": enc_bytes, "kernel": f"kvq::encode_l1<{D},{bits}>"},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(spec, signs, bits)
    print(json.dumps(result), flush=True)
    return 0 if parity_ok else 1


if __name__ == "__main__":
    sys.exit(main())
