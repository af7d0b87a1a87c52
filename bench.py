"""Benchmark of the HCA hot path on one MI355X.

One step = the whole prefill path over one 128K-token sequence with 64 query
heads: block compression of K and V (1024 entries each), then HCA prefill
attention (entries + 128-token window, 512-wide heads, sigmoid gate), bf16 in
and out.  Inputs are seeded synthetic N(0,1) bf16 tensors already resident in
HBM.  The reported value is algorithmic TFLOP/s of the step:
    FLOPs = 4 * 512 * H * sum_t (floor((t+1)/128) + min(t+1, 128))
(visible keys only; masked work, exp and the gate are not counted).

Also reported:
  roofline      the prefill kernel's own rate (HIP events on its stream) against
                the 2.5 PFLOP/s dense bf16 MFMA peak, plus HBM bytes from
                rocprofv3 counters when they were taken on the current source;
  decode        batched decode (64 sequences, 256 entries + 128 window rows, 64
                heads) in GB/s of compulsory HBM traffic, against 8 TB/s;
  decode_multi  the same with 3 new tokens per sequence (the verify step of
                two-token drafts);
  prefill_vha   the prefill launch with the VHA head mix fused into its
                epilogue, beside the plain launch;
  cpu_baseline  the fp64 oracle timed on a bounded sample of the same workload.

python bench.py [--gpus 1] [--steps K] [--warmup W]
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

D, BLOCK, WINDOW = 512, 128, 128
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense bf16
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
METRIC = "HCA attn TFLOP/s (128K prefill, % bf16 MFMA peak); decode HBM GB/s"
COUNTERS = os.path.join(ROOT, "profiles", "prefill_128k_counters.json")
PREFILL_SRC = os.path.join(ROOT, "long_context_compressed_hca_amd", "csrc", "prefill.hip")
COPY_BYTES = 1 << 30           # calibration copy for the HBM byte counters


def visible_keys(t0: int, t1: int, Nc_cap: int | None = None) -> int:
    """sum over query positions t0..t1-1 of floor((t+1)/128) + min(t+1, 128)."""
    t = np.arange(t0, t1, dtype=np.int64)
    nc = (t + 1) // BLOCK
    if Nc_cap is not None:
        nc = np.minimum(nc, Nc_cap)
    return int(nc.sum() + np.minimum(t + 1, WINDOW).sum())


def prefill_flops(T: int, H: int, q_start: int = 0) -> float:
    return 4.0 * D * H * visible_keys(q_start, q_start + T)


def sha256(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def load_traffic():
    """HBM bytes per prefill launch from committed rocprofv3 counter runs, or None
    if the counters were taken on a different prefill source."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha256") != sha256(PREFILL_SRC):
        return None
    return c.get("hbm_bytes_per_launch")


def counters_workload(args, torch, hca, synth):
    """One 128K compress + prefill launch and one plain copy of COPY_BYTES, for
    rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE)."""
    dev = torch.device("cuda:0")
    T, H = args.T, 64
    gen = lambda tid, shape: synth.normal_bf16_device(3, tid, shape, dev)
    q, g = gen(synth.Q, (T, H, D)), gen(synth.G, (T, H, D))
    k, v = gen(synth.K, (T, D)), gen(synth.V, (T, D))
    ck = torch.empty((T // BLOCK, D), dtype=torch.bfloat16, device=dev)
    cv = torch.empty_like(ck)
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    hca.hca_compress(k, v, ck, cv)
    hca.hca_attn_prefill(q, g, k, v, ck, cv, out)
    dst.copy_(src)
    torch.cuda.synchronize()
    print("counters workload done", flush=True)


def _pmc_per_kernel(csv_dir, counter):
    """Per-dispatch values of one counter from a rocprofv3 --pmc csv output dir,
    grouped by kernel name."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r.get("Counter_Name") == counter:
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return vals


def write_counters(fetch_dir, write_dir):
    """Scale the prefill kernel's FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by
    what the same counters read for the plain copy of COPY_BYTES, and write
    the per-launch HBM bytes next to the source hash they belong to."""
    fetch = _pmc_per_kernel(fetch_dir, "FETCH_SIZE")
    write = _pmc_per_kernel(write_dir, "WRITE_SIZE")
    pick = lambda d, key: [v for n, vs in d.items() if key in n for v in vs]
    pf_f, pf_w = pick(fetch, "prefill_kernel"), pick(write, "prefill_kernel")
    cp_f = pick(fetch, "copy") or pick(fetch, "elementwise")
    cp_w = pick(write, "copy") or pick(write, "elementwise")
    if not (pf_f and pf_w and cp_f and cp_w):
        raise SystemExit(f"missing counters: {sorted(fetch)} {sorted(write)}")
    f_scale = COPY_BYTES / (max(cp_f) * 1024.0)
    w_scale = COPY_BYTES / (max(cp_w) * 1024.0)
    rd = float(np.median(pf_f)) * 1024.0 * f_scale
    wr = float(np.median(pf_w)) * 1024.0 * w_scale
    T, H = 131072, 64
    algo = 3 * T * H * D * 2 + 2 * T * D * 2 + 2 * (T // BLOCK) * D * 2
    rec = {"kernel": "hca prefill_kernel (bf16 out), 128K tokens, 64 heads",
           "kernel_source_sha256": sha256(PREFILL_SRC),
           "fetch_kib_per_dispatch": float(np.median(pf_f)),
           "write_kib_per_dispatch": float(np.median(pf_w)),
           "copy_bytes": COPY_BYTES, "copy_fetch_kib": max(cp_f), "copy_write_kib": max(cp_w),
           "fetch_scale": f_scale, "write_scale": w_scale,
           "hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr,
           "hbm_bytes_per_launch": rd + wr, "algorithmic_bytes_per_launch": algo,
           "traffic_over_algorithmic": (rd + wr) / algo}
    with open(COUNTERS, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def bench_prefill(args, torch, hca, synth):
    dev = torch.device("cuda:0")
    T, H = args.T, 64
    gen = lambda tid, shape: synth.normal_bf16_device(3, tid, shape, dev)
    q, g = gen(synth.Q, (T, H, D)), gen(synth.G, (T, H, D))
    k, v = gen(synth.K, (T, D)), gen(synth.V, (T, D))
    Nc = T // BLOCK
    ck = torch.empty((Nc, D), dtype=torch.bfloat16, device=dev)
    cv = torch.empty_like(ck)
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]

    def step(i=None):
        hca.hca_compress(k, v, ck, cv)
        if i is not None:
            ev[i][0].record(stream)
        hca.hca_attn_prefill(q, g, k, v, ck, cv, out)
        if i is not None:
            ev[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kernel_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    flops = prefill_flops(T, H)
    return dict(T=T, H=H, flops=flops, ms_per_step=elapsed * 1e3 / args.steps,
                prefill_ms=kernel_ms, tensors=(q, g, k, v, ck, cv, out))


def bench_prefill_vha(args, torch, hca, synth, tensors, rank=16):
    """The prefill launch of the step with the VHA head mix fused (rank 16, factors
    N(0,1)/8), timed like the plain launch; reported beside it, not part of the step."""
    dev = torch.device("cuda:0")
    q, g, k, v, ck, cv, out = tensors
    H = q.shape[1]
    up = (synth.normal_bf16_device(9, synth.CK, (H, rank), dev) * 0.125).contiguous()
    down = (synth.normal_bf16_device(9, synth.CV, (rank, H), dev) * 0.125).contiguous()
    stream = torch.cuda.current_stream(dev)
    n = max(3, args.steps)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    hca.hca_attn_prefill_vha(q, g, k, v, ck, cv, up, down, out)
    torch.cuda.synchronize()
    for i in range(n):
        ev[i][0].record(stream)
        hca.hca_attn_prefill_vha(q, g, k, v, ck, cv, up, down, out)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    T = q.shape[0]
    mix_flops = 2 * 2 * T * H * rank * D  # down and up products, every dim
    return {"launch_ms": round(ms, 4), "rank": rank,
            "tflops_attention": round(prefill_flops(T, H) / (ms * 1e-3) / 1e12, 2),
            "mix_gflop": round(mix_flops / 1e9, 1),
            "workload": f"the 128K prefill launch with the VHA head mix fused (rank {rank})"}


def bench_decode(args, torch, hca, synth, M=1):
    """64 sequences, new token at position 32768: 256 entries + 128 window rows each.
    M > 1: M new tokens at 32768 .. 32768+M-1 (the verify step of (M-1)-token drafts);
    each still sees 256 entries and 128 raw rows."""
    dev = torch.device("cuda:0")
    B, H, nc_cap, pos = 64, 64, 256, 32768
    reps = 6
    sets = []
    qs = (B, H, D) if M == 1 else (B, M, H, D)
    for r in range(reps):
        gen = lambda tid, shape: synth.normal_bf16_device(40 + r, tid, shape, dev)
        sets.append(dict(q=gen(synth.Q, qs), g=gen(synth.G, qs),
                         ck=gen(synth.CK, (B, nc_cap, D)), cv=gen(synth.CV, (B, nc_cap, D)),
                         wk=gen(synth.WK, (B, WINDOW, D)), wv=gen(synth.WV, (B, WINDOW, D)),
                         nk=gen(synth.NK, (B, M, D)), nv=gen(synth.NV, (B, M, D)),
                         out=torch.empty(qs, dtype=torch.bfloat16, device=dev)))
    posd = torch.full((B,), pos, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)
    n = 240
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]

    def call(s):
        if M == 1:
            hca.hca_attn_decode(s["q"], s["g"], s["ck"], s["cv"], s["wk"], s["wv"], posd,
                                s["out"])
        else:
            hca.hca_attn_decode_multi(s["q"], s["g"], s["ck"], s["cv"], s["wk"], s["wv"],
                                      s["nk"], s["nv"], posd, s["out"])

    for i in range(24):
        call(sets[i % reps])
    torch.cuda.synchronize()
    # Back to back (the throughput a serving loop sees): n calls between two events.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        call(sets[i % reps])
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    # Each call alone between its own events (adds the launch gap): reported too.
    for i in range(n):
        ev[i][0].record(stream)
        call(sets[i % reps])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    us_alone = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3
    # Compulsory bytes: every distinct key row (the entries of the last token, the
    # ring rows and the new rows) once, q, g and out once.
    n_rows = (pos + M) // BLOCK + (pos + M - max(0, pos - WINDOW + 1))
    kv_bytes = B * n_rows * D * 2 * 2
    qgo_bytes = 3 * B * M * H * D * 2
    total = kv_bytes + qgo_bytes
    gbs = total / (us * 1e-6) / 1e9
    flops = 4 * D * H * B * sum((pos + j + 1) // BLOCK + min(pos + j + 1, WINDOW)
                                for j in range(M))
    what = ("HCA batched decode: 64 sequences x (256 entries + 128 window rows), 64 heads, "
            "dim 512, bf16") if M == 1 else (
            f"HCA multi-token decode: 64 sequences x {M} new tokens (causal among "
            "themselves), each seeing 256 entries + 128 raw rows, 64 heads, dim 512, bf16")
    return dict(metric="decode HBM GB/s", value=round(gbs, 1), unit="GB/s",
                us_per_call=round(us, 2), us_per_call_alone=round(us_alone, 2),
                bytes_per_call=total, tflops=round(flops / (us * 1e-6) / 1e12, 2),
                config={"workload": what, "input_replicas": reps},
                roofline={"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                          "traffic": None})


def cpu_baseline(args, torch, synth, tensors):
    """The oracle, as it stands, on a bounded sample of query positions of the same
    128K workload (every head), timed on this host's cores."""
    import oracle
    q, g, k, v = tensors[:4]
    T, H = q.shape[0], q.shape[1]
    rng = np.random.default_rng(2024)
    pos = np.sort(rng.choice(T, size=args.cpu_positions, replace=False)).astype(np.int64)
    host = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    idx = torch.as_tensor(pos, device=q.device)
    qh, gh = host(q.index_select(0, idx)), host(g.index_select(0, idx))
    kh, vh = host(k), host(v)
    threads = oracle.threads()
    t0 = time.perf_counter()
    ck, cv = oracle.compress(kh), oracle.compress(vh)
    oracle.attn(qh, gh, pos, kh, vh, 0, ck, cv, nthreads=threads)
    dt = time.perf_counter() - t0
    t = pos
    keys = int(((t + 1) // BLOCK).sum() + np.minimum(t + 1, WINDOW).sum())
    flops = 4.0 * D * H * keys
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{len(pos)} seeded query positions (all {H} heads) of the 128K-token "
                      f"workload, plus compressing its full K and V; fp64 C oracle"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--T", type=int, default=131072, help=argparse.SUPPRESS)
    ap.add_argument("--cpu-positions", type=int, default=8192)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--counters-workload", action="store_true",
                    help="one prefill launch + one calibration copy, for rocprofv3 --pmc")
    ap.add_argument("--write-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc csv dirs into " + COUNTERS)
    args = ap.parse_args()
    if args.write_counters:
        write_counters(*args.write_counters)
        return
    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU only (asked for --gpus {args.gpus}); "
              "sharding across GPUs is not built.", file=sys.stderr)
        sys.exit(2)

    import torch
    import long_context_compressed_hca_amd as hca
    import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    hca.lib()  # fail loudly if the HIP library is missing
    if args.counters_workload:
        counters_workload(args, torch, hca, synth)
        return

    pf = bench_prefill(args, torch, hca, synth)
    value = pf["flops"] / (pf["ms_per_step"] * 1e-3) / 1e12
    achieved = pf["flops"] / (pf["prefill_ms"] * 1e-3) / 1e12
    traffic = load_traffic()
    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(pf["ms_per_step"], 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "HCA prefill at 128K context: batch 1, T=131072, 64 query "
                   "heads, 1 KV head, dim 512, block 128, window 128; compress + prefill "
                   "per step; bf16 in/out", "seq_len": pf["T"], "heads": pf["H"],
                   "global_batch": 1, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_PEAK_TFLOPS, 4), "traffic": traffic,
                     "kernel": "hca prefill_kernel", "flops_per_launch": pf["flops"],
                     "launch_ms": round(pf["prefill_ms"], 4)},
    }
    rec["prefill_vha"] = bench_prefill_vha(args, torch, hca, synth, pf["tensors"])
    rec["prefill_vha"]["overhead_vs_plain"] = round(
        rec["prefill_vha"]["launch_ms"] / pf["prefill_ms"] - 1, 4)
    if not args.no_decode:
        rec["decode"] = bench_decode(args, torch, hca, synth)
        rec["decode_multi"] = bench_decode(args, torch, hca, synth, M=3)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(args, torch, synth, pf["tensors"])
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
