"""Benchmark of the HCA hot path on one MI355X.

One step = the whole prefill path over one 128K-token sequence with 64 query
heads: block compression of K and V (1024 entries each), then HCA prefill
attention (entries + 128-token window, 512-wide heads, sigmoid gate), bf16 in
and out.  Inputs are seeded synthetic N(0,1) bf16 tensors already resident in
HBM.  The reported value is algorithmic TFLOP/s of the step:
    FLOPs = 4 * 512 * H * sum_t (floor((t+1)/128) + min(t+1, 128))
(visible keys only; masked work, exp and the gate are not counted).

Also reported (each launch timed with HIP events on the stream it runs on):
  roofline      the 128K prefill kernel's rate against the 2.5 PFLOP/s dense bf16
                MFMA peak, with HBM bytes and counter-derived MFMA FLOPs from
                rocprofv3 counters taken on the current kernel source;
  workloads     every other measured configuration: block compression at 128K,
                prefill at 2K tokens x 8 heads (fp32 out), at 8K x 64, the last 64K queries of a 1M-token
                sequence, prefill with the VHA head mix, batched and multi-token
                decode, the low-rank gate GEMM and the backward pass; each with
                its bound (MFMA or HBM: whichever roofline time is longer), the
                achieved rate and its fraction of that peak;
  cpu_baseline  the fp64 oracle timed on a bounded sample of the 128K workload.
  parity        the GPU output of the bench step on that sample's rows against the
                oracle's (rel-L2, max-abs, worst row) and the compressed entries
                compared bit for bit.

python bench.py [--gpus 1] [--steps K] [--warmup W]

Profiling modes (their outputs are summarised under profiles/):
  --copy-rate OUT_MD      per-CU rate of the copy path (LDS DMA and VGPR loads of
                          1 KiB rows) at 1, 32 and 256 workgroups, table to OUT_MD;
  --counters-workload [--reps N]
                          N launches of every workload plus a 1 GiB copy, for a
                          rocprofv3 kernel trace and --pmc passes;
  --write-profiles KT FETCH WRITE MFMA OUT KT_ORDER PMC_ORDER BENCH_JSON
                          turn those runs into OUT/*.md and OUT/counters.json (the
                          commands are in the header of each summary).
"""
from __future__ import annotations

import argparse
import csv
import glob
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
XCC = 8                        # accelerator complexes (GRBM_GUI_ACTIVE is per XCC)
METRIC = "HCA attn TFLOP/s (128K prefill, % bf16 MFMA peak); decode HBM GB/s"
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
CSRC = os.path.join(ROOT, "long_context_compressed_hca_amd", "csrc")
COPY_BYTES = 1 << 30           # calibration copy for the HBM byte counters


# ----------------------------------------------------------------- work counts
def visible_keys(t0: int, t1: int) -> int:
    """sum over query positions t0..t1-1 of floor((t+1)/128) + min(t+1, 128)."""
    t = np.arange(t0, t1, dtype=np.int64)
    return int(((t + 1) // BLOCK).sum() + np.minimum(t + 1, WINDOW).sum())


def prefill_flops(T: int, H: int, q_start: int = 0) -> float:
    return 4.0 * D * H * visible_keys(q_start, q_start + T)


def prefill_bytes(T: int, H: int, q_start: int, out_bytes: int) -> int:
    """Compulsory HBM bytes of one prefill launch: q, g in, out, the raw K/V rows
    the queries see, the entries they see."""
    kv_start = max(0, q_start - (WINDOW - 1))
    n_raw = q_start + T - kv_start
    nc = (q_start + T) // BLOCK
    return T * H * D * (2 + 2 + out_bytes) + 2 * n_raw * D * 2 + 2 * nc * D * 2


def sha256_files(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def roofline(flops: float, nbytes: float, ms: float) -> dict:
    """Bound = the roofline whose time is longer; achieved rate in its unit."""
    t_mfma = flops / (MFMA_PEAK_TFLOPS * 1e12)
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    if t_mfma >= t_hbm:
        ach = flops / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_PEAK_TFLOPS, 4)}
    ach = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4)}


# ----------------------------------------------------------------- workloads
# Each workload builds its seeded inputs on the GPU and returns a dict with
#   call()    one launch of the library entry point(s) measured
#   kernels   [(kernel-name substring, dispatches per call)] in launch order
#   src       the kernel sources whose hash keys the counters
#   flops, bytes, what
# Sizes are the ones the pages' workloads describe (see each docstring).

def log(msg: str):
    """Progress on stderr (stdout carries the one JSON line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def _gen(synth, torch, seed):
    dev = torch.device("cuda:0")
    return lambda tid, shape: synth.normal_bf16_device(seed, tid, shape, dev)


def w_prefill(torch, hca, synth, T, H, q_start=0, out_f32=False, seed=3):
    """Prefill of T queries at q_start .. q_start+T-1 with 64 (or H) heads; K/V rows
    exist for every position (entries compressed before timing)."""
    dev = torch.device("cuda:0")
    gen = _gen(synth, torch, seed)
    end = q_start + T
    kv_start = max(0, q_start - (WINDOW - 1))
    Nc = end // BLOCK
    k_all, v_all = gen(synth.K, (end, D)), gen(synth.V, (end, D))
    q, g = gen(synth.Q, (T, H, D)), gen(synth.G, (T, H, D))
    ck = torch.empty((Nc, D), dtype=torch.bfloat16, device=dev)
    cv = torch.empty_like(ck)
    hca.hca_compress(k_all[:Nc * BLOCK], v_all[:Nc * BLOCK], ck, cv)
    k, v = k_all[kv_start:], v_all[kv_start:]
    out = torch.empty((T, H, D), dtype=torch.float32 if out_f32 else torch.bfloat16, device=dev)

    def call():
        hca.hca_attn_prefill(q, g, k, v, ck if Nc else None, cv if Nc else None, out,
                             q_start=q_start, kv_start=kv_start)

    def step():  # compress + prefill (the bench step)
        hca.hca_compress(k_all[:Nc * BLOCK], v_all[:Nc * BLOCK], ck, cv)
        call()

    return dict(call=call, step=step, kernels=[("prefill_kernel", 1)],
                src=["prefill.hip"], flops=prefill_flops(T, H, q_start),
                bytes=prefill_bytes(T, H, q_start, 4 if out_f32 else 2),
                tensors=(q, g, k_all, v_all, ck, cv, out), q_start=q_start)


def parity_sample(torch, w, n_pos, seed):
    """Host copies of what the oracle needs for n_pos seeded query positions of a
    prefill workload (all heads), with the GPU's output of those rows from its last
    timed launch.  No arithmetic: the cpu_baseline leg runs the oracle on them."""
    q, g, k_all, v_all, ck, cv, out = w["tensors"]
    T, q_start = q.shape[0], w["q_start"]
    rng = np.random.default_rng(seed)
    i = np.sort(rng.choice(T, size=min(n_pos, T), replace=False)).astype(np.int64)
    t = q_start + i
    lo = int(max(0, t.min() - (WINDOW - 1)))
    host = lambda x: x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    idx = torch.as_tensor(i, device=q.device)
    return {"t": t, "q": host(q.index_select(0, idx)), "g": host(g.index_select(0, idx)),
            "k": host(k_all[lo:int(t.max()) + 1]), "v": host(v_all[lo:int(t.max()) + 1]),
            "kv_start": lo, "ck": host(ck), "cv": host(cv),
            "got": out.index_select(0, idx).float().cpu().numpy().astype(np.float64)}


def parity_figures(got, ref, tol=(1e-2, 3e-2)):
    """rel-L2, max-abs and the worst row's rel-L2 of got against ref ([..., D])."""
    diff = got - ref
    row_err = (np.linalg.norm(diff.reshape(-1, diff.shape[-1]), axis=1)
               / np.maximum(np.linalg.norm(ref.reshape(-1, ref.shape[-1]), axis=1), 1e-300))
    rel = float(np.linalg.norm(diff) / np.linalg.norm(ref))
    mx = float(np.abs(diff).max())
    return {"rows": int(row_err.size), "rel_l2": rel, "max_abs": mx,
            "worst_row_rel_l2": float(row_err.max()),
            "pass": bool(rel <= tol[0] and mx <= tol[1])}


def w_compress(torch, hca, synth, T=131072, seed=5):
    """Block compression of T rows of K and V into T/128 entries each (the first
    kernel of the prefill step)."""
    dev = torch.device("cuda:0")
    gen = _gen(synth, torch, seed)
    k, v = gen(synth.K, (T, D)), gen(synth.V, (T, D))
    ck = torch.empty((T // BLOCK, D), dtype=torch.bfloat16, device=dev)
    cv = torch.empty_like(ck)

    def call():
        hca.hca_compress(k, v, ck, cv)

    nbytes = 2 * T * D * 2 + 2 * (T // BLOCK) * D * 2
    return dict(call=call, kernels=[("compress_kernel", 1)], src=["compress.hip"],
                flops=0.0, bytes=nbytes)


def w_prefill_vha(torch, hca, synth, base, rank=16):
    """The 128K prefill launch with the VHA head mix fused (rank 16, factors N(0,1)/8)."""
    dev = torch.device("cuda:0")
    q, g, k, v, ck, cv, out = base["tensors"]
    H = q.shape[1]
    up = (synth.normal_bf16_device(9, synth.CK, (H, rank), dev) * 0.125).contiguous()
    down = (synth.normal_bf16_device(9, synth.CV, (rank, H), dev) * 0.125).contiguous()

    def call():
        hca.hca_attn_prefill_vha(q, g, k, v, ck, cv, up, down, out)

    T = q.shape[0]
    mix = 2 * 2 * T * H * rank * D
    return dict(call=call, kernels=[("prefill_kernel", 1)], src=["prefill.hip"],
                flops=base["flops"] + mix, bytes=base["bytes"], rank=rank)


def w_decode(torch, hca, synth, M=1, reps=6):
    """64 sequences with 32768 tokens of history: 256 entries + 128 ring rows each,
    64 heads; M new tokens per sequence at 32768 .. 32768+M-1.  `reps` input
    replicas are cycled so that consecutive calls do not hit in L2."""
    dev = torch.device("cuda:0")
    B, H, nc_cap, pos = 64, 64, 256, 32768
    qs = (B, H, D) if M == 1 else (B, M, H, D)
    sets = []
    for r in range(reps):
        gen = _gen(synth, torch, 40 + r)
        sets.append(dict(q=gen(synth.Q, qs), g=gen(synth.G, qs),
                         ck=gen(synth.CK, (B, nc_cap, D)), cv=gen(synth.CV, (B, nc_cap, D)),
                         wk=gen(synth.WK, (B, WINDOW, D)), wv=gen(synth.WV, (B, WINDOW, D)),
                         nk=gen(synth.NK, (B, M, D)), nv=gen(synth.NV, (B, M, D)),
                         out=torch.empty(qs, dtype=torch.bfloat16, device=dev)))
    posd = torch.full((B,), pos, dtype=torch.int64, device=dev)
    ctr = [0]

    def call():
        s = sets[ctr[0] % reps]
        ctr[0] += 1
        if M == 1:
            hca.hca_attn_decode(s["q"], s["g"], s["ck"], s["cv"], s["wk"], s["wv"], posd,
                                s["out"])
        else:
            hca.hca_attn_decode_multi(s["q"], s["g"], s["ck"], s["cv"], s["wk"], s["wv"],
                                      s["nk"], s["nv"], posd, s["out"])

    # compulsory bytes: every distinct key row (entries of the last token, ring rows,
    # new rows) once, q, g and out once
    n_rows = (pos + M) // BLOCK + (pos + M - max(0, pos - WINDOW + 1))
    nbytes = B * n_rows * D * 2 * 2 + 3 * B * M * H * D * 2
    flops = 4 * D * H * B * sum((pos + j + 1) // BLOCK + min(pos + j + 1, WINDOW)
                                for j in range(M))
    return dict(call=call, kernels=[("decode", 1)], src=["decode.hip", "decode_sk.hip"],
                flops=float(flops), bytes=nbytes, sets=sets, pos=posd, M=M)


def decode_parity_sample(torch, w):
    """Host copies of the first input set of a one-token decode workload and the
    GPU's output for it from the timed calls (no arithmetic)."""
    s = w["sets"][0]
    host = lambda x: x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return {k: host(s[k]) for k in ("q", "g", "ck", "cv", "wk", "wv")} | {
        "pos": w["pos"].cpu().numpy(), "got": s["out"].float().cpu().numpy().astype(np.float64)}


def w_gate(torch, hca, synth, T=131072, R=1024, H=64):
    """Gate logits of the low-rank gate for a 128K sequence: latent [T, 1024]
    (the 4096-wide hidden state / 4) times W_g [64 * 512, 1024]^T."""
    dev = torch.device("cuda:0")
    gen = _gen(synth, torch, 11)
    lat = gen(10, (T, R))
    w = (gen(11, (H * D, R)) * (1.0 / 32)).contiguous()
    g = torch.empty((T, H * D), dtype=torch.bfloat16, device=dev)

    def call():
        hca.hca_gate_logits(lat, w, g)

    return dict(call=call, kernels=[("gate_kernel", 1)], src=["gate.hip"],
                flops=2.0 * T * R * H * D, bytes=(T * R + H * D * R + T * H * D) * 2)


def backward_pairs(T: int, H: int) -> int:
    return H * visible_keys(0, T)


def w_backward(torch, hca, synth, T, H=64, saved=False):
    """Backward pass of a whole-sequence prefill (T tokens, 64 heads): fp32 dq, dk,
    dv, dg.  Algorithmic FLOPs: 5 products of 2 * 512 per (query row, visible key)
    pair (scores, dP, dV, dK, dQ), 2.5 times the forward's.  saved: from the
    forward's output and row log-sum-exp (hca_attn_prefill_lse, run once before)."""
    dev = torch.device("cuda:0")
    gen = _gen(synth, torch, 7)
    q, g, do = gen(synth.Q, (T, H, D)), gen(synth.G, (T, H, D)), gen(12, (T, H, D))
    k, v = gen(synth.K, (T, D)), gen(synth.V, (T, D))
    Nc = T // BLOCK
    ck = torch.empty((Nc, D), dtype=torch.bfloat16, device=dev)
    cv = torch.empty_like(ck)
    hca.hca_compress(k[:Nc * BLOCK], v[:Nc * BLOCK], ck, cv)
    f32 = dict(dtype=torch.float32, device=dev)
    dq, dg = torch.empty((T, H, D), **f32), torch.empty((T, H, D), **f32)
    dk, dv = torch.empty((T, D), **f32), torch.empty((T, D), **f32)
    ws = torch.empty(hca.backward_workspace_size(T, H), dtype=torch.uint8, device=dev)
    if saved:
        out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((T, H), **f32)
        hca.hca_attn_prefill_lse(q, g, k, v, ck, cv, out, lse)

        def call():
            hca.hca_attn_backward_saved(q, g, k, v, ck, cv, out, lse, do, dq, dk, dv, dg,
                                        workspace=ws)
    else:
        def call():
            hca.hca_attn_backward(q, g, k, v, ck, cv, do, dq, dk, dv, dg, workspace=ws)

    nbytes = 3 * T * H * D * 2 + 2 * T * H * D * 4 + 2 * T * D * (2 + 4) + 2 * Nc * D * 2
    if saved:
        nbytes += T * H * (D * 2 + 4)
    return dict(call=call, kernels=[("zero_kernel", 2), ("rows_kernel", 1), ("keys_kernel", 1),
                                    ("pool_kernel", 1)],
                src=["backward.hip"], flops=10.0 * D * backward_pairs(T, H), bytes=nbytes)


# Prefill workloads whose sampled rows the cpu_baseline leg checks against the
# oracle: name -> (query positions, seed).
PARITY_SAMPLES = {"prefill_2k_h8_f32": (2048, 11), "prefill_8k": (256, 12),
                  "prefill_1m_chunk": (32, 13)}


# name -> (builder, description); the step's own workload is "prefill_128k"
def workload_table(torch, hca, synth):
    return [
        ("compress_128k", "block compression of K and V at T=131072 (1024 entries each), "
         "bf16", lambda: w_compress(torch, hca, synth)),
        ("prefill_2k_h8_f32", "HCA prefill, batch 1, T=2048, 8 query heads, 1 KV head, dim "
         "512, block 128, window 128; fp32 output",
         lambda: w_prefill(torch, hca, synth, 2048, 8, out_f32=True)),
        ("prefill_8k", "HCA prefill, one layer at full shape: T=8192, 64 query heads, dim "
         "512; bf16 output", lambda: w_prefill(torch, hca, synth, 8192, 64)),
        ("prefill_1m_chunk", "HCA chunked prefill: the last 65536 queries of a 1,048,576-"
         "token sequence (8192 entries), 64 heads, dim 512; bf16 output",
         lambda: w_prefill(torch, hca, synth, 65536, 64, q_start=(1 << 20) - 65536)),
        ("decode", "HCA batched decode: 64 sequences x (256 entries + 128 window rows), "
         "1 new token each, 64 heads, dim 512, bf16", lambda: w_decode(torch, hca, synth)),
        ("decode_multi", "HCA multi-token decode: 64 sequences x 3 new tokens (causal among "
         "themselves), each seeing 256 entries + 128 raw rows, 64 heads, bf16",
         lambda: w_decode(torch, hca, synth, M=3)),
        ("gate_128k", "low-rank gate logits: latent [131072, 1024] x W_g [32768, 1024]^T, "
         "bf16 out", lambda: w_gate(torch, hca, synth)),
        ("backward_8k", "HCA backward (dq, dk, dv, dg in fp32): T=8192, 64 heads, dim 512",
         lambda: w_backward(torch, hca, synth, 8192)),
        ("backward_128k", "HCA backward (dq, dk, dv, dg in fp32): T=131072, 64 heads, dim 512",
         lambda: w_backward(torch, hca, synth, 131072)),
        ("backward_saved_8k", "HCA backward from the forward's saved output and row "
         "log-sum-exp: T=8192, 64 heads, dim 512",
         lambda: w_backward(torch, hca, synth, 8192, saved=True)),
        ("backward_saved_128k", "HCA backward from the forward's saved output and row "
         "log-sum-exp: T=131072, 64 heads, dim 512",
         lambda: w_backward(torch, hca, synth, 131072, saved=True)),
    ]


def time_launches(torch, call, n: int, warmup: int = 2) -> float:
    """Mean ms per launch, each launch between its own HIP events on the current
    stream (where the library enqueues its kernels)."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


def time_back_to_back(torch, call, n: int) -> float:
    """Mean ms per launch of n launches between two events (no gaps measured)."""
    stream = torch.cuda.current_stream()
    for _ in range(8):
        call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(n):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def load_counters():
    try:
        with open(COUNTERS) as f:
            return json.load(f)
    except (OSError, ValueError):
        return {}


def counter_fields(counters, name, src):
    """HBM traffic and counter-derived MFMA FLOPs of a workload, if its counters were
    taken on the current kernel sources."""
    c = counters.get("workloads", {}).get(name)
    if not c or c.get("source_sha256") != sha256_files(src):
        return {"traffic": None}
    out = {"traffic": c.get("hbm_bytes")}
    if c.get("mfma_flops") is not None:
        out["mfma_flops_counted"] = c["mfma_flops"]
    return out


def run_workload(torch, name, what, w, n, counters, back_to_back=False):
    ms = time_back_to_back(torch, w["call"], n) if back_to_back else \
        time_launches(torch, w["call"], n)
    rec = {"workload": what, "ms": round(ms, 5),
           "tflops": round(w["flops"] / (ms * 1e-3) / 1e12, 2),
           "gbs": round(w["bytes"] / (ms * 1e-3) / 1e9, 1),
           "flops": w["flops"], "algorithmic_bytes": w["bytes"]}
    rec["roofline"] = roofline(w["flops"], w["bytes"], ms)
    rec["roofline"].update(counter_fields(counters, name, w["src"]))
    return rec


# ----------------------------------------------------------------- cpu baseline
def cpu_baseline(args, torch, tensors, hca):
    """The oracle, as it stands, on a bounded sample of query positions of the same
    128K workload (every head), timed on this host's cores.  The rows it computes
    are then compared with the GPU's output of the bench step (re-run once, since
    the VHA workload writes the same output tensor), and the entries it compresses
    with the GPU's: the parity of the measured configuration."""
    import oracle
    q, g, k, v, ck_d, cv_d, out = tensors
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
    ref = oracle.attn(qh, gh, pos, kh, vh, 0, ck, cv, nthreads=threads)
    dt = time.perf_counter() - t0
    t = pos
    keys = int(((t + 1) // BLOCK).sum() + np.minimum(t + 1, WINDOW).sum())
    flops = 4.0 * D * H * keys
    rec = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
           "kind": "oracle", "seconds": round(dt, 2),
           "sample": f"{len(pos)} seeded query positions (all {H} heads) of the 128K-token "
                     f"workload, plus compressing its full K and V; fp64 C oracle"}
    # parity of the same rows: the GPU's bf16 output of the bench step
    hca.hca_compress(k, v, ck_d, cv_d)
    hca.hca_attn_prefill(q, g, k, v, ck_d, cv_d, out)
    torch.cuda.synchronize()
    got = out.index_select(0, idx).float().cpu().numpy().astype(np.float64)
    diff = got - ref
    row_err = np.linalg.norm(diff, axis=2) / np.maximum(np.linalg.norm(ref, axis=2), 1e-300)
    parity = {"reference": "fp64 C oracle, the rows of the cpu_baseline sample",
              "rows": int(ref.shape[0] * ref.shape[1]),
              "rel_l2": float(np.linalg.norm(diff) / np.linalg.norm(ref)),
              "max_abs": float(np.abs(diff).max()),
              "worst_row_rel_l2": float(row_err.max()),
              "tolerance": {"rel_l2": 1e-2, "max_abs": 3e-2},
              "compress_bit_exact": bool(np.array_equal(host(ck_d), ck)
                                         and np.array_equal(host(cv_d), cv))}
    parity["pass"] = bool(parity["rel_l2"] <= 1e-2 and parity["max_abs"] <= 3e-2
                          and parity["compress_bit_exact"])
    return rec, parity


def cpu_parity(samples):
    """The oracle on the sampled rows of the other prefill workloads (configs of 2K x
    8 heads, 8K x 64 and the 1M-token chunk) and on every output of the batched
    decode's first input set, compared with the GPU's."""
    import oracle
    out = {}
    for name, sm in samples.items():
        if name == "decode":
            ref = oracle.decode(sm["q"], sm["g"], sm["ck"], sm["cv"], sm["wk"], sm["wv"],
                                sm["pos"], nthreads=oracle.threads())
            out[name] = parity_figures(sm["got"], ref)
            out[name]["sequences"] = int(len(sm["pos"]))
            continue
        ref = oracle.attn(sm["q"], sm["g"], sm["t"], sm["k"], sm["v"], sm["kv_start"],
                          sm["ck"], sm["cv"], nthreads=oracle.threads())
        out[name] = parity_figures(sm["got"], ref)
        out[name]["positions"] = int(len(sm["t"]))
    return out


# ----------------------------------------------------------------- profiling
def counters_workload(torch, hca, synth, reps: int):
    """Each workload in table order (the 128K prefill and its VHA variant right
    after prefill_8k): its inputs are built, it is launched `reps` times, and it
    is freed before the next is built (so the 128K backward fits); then a plain
    copy of COPY_BYTES.  For rocprofv3 runs (--pmc passes with reps = 1, the
    kernel trace with more); --write-profiles finds each workload's launches by
    their kernel names, in this order."""
    dev = torch.device("cuda:0")
    order = []

    warm = 1 if reps > 1 else 0  # the trace's launches follow one untimed launch

    def run(name, w):
        torch.cuda.synchronize()
        print(f"counters: {name}", flush=True)
        for _ in range(warm + reps):
            w["call"]()
            torch.cuda.synchronize()
        order.append({"name": name, "kernels": w["kernels"], "src": w["src"], "reps": reps,
                      "warm": warm})

    for name, what, build in workload_table(torch, hca, synth):
        w = build()
        run(name, w)
        del w
        if name == "prefill_8k":
            pf = w_prefill(torch, hca, synth, 131072, 64)
            run("prefill_128k", pf)
            vha = w_prefill_vha(torch, hca, synth, pf)
            run("prefill_vha_128k", vha)
            del pf, vha
        torch.cuda.empty_cache()
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"order": order}), flush=True)


def _csv_rows(d, suffix):
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        rows.extend(csv.DictReader(open(f)))
    return rows


def _dispatches(pmc_dir):
    """Per dispatch (in dispatch order): kernel name and counter values (summed over
    dimensions), from a rocprofv3 --pmc csv directory."""
    per = {}
    rows = _csv_rows(pmc_dir, "counter_collection.csv")
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {pmc_dir}")
    for r in rows:
        key = int(r["Dispatch_Id"])
        e = per.setdefault(key, {"name": r["Kernel_Name"], "c": {}})
        e["c"][r["Counter_Name"]] = e["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [per[k] for k in sorted(per)]


def _traced(run_dir):
    """Per dispatch (in dispatch order): kernel name and duration (ns), from the
    kernel trace of a rocprofv3 csv directory."""
    rows = _csv_rows(run_dir, "kernel_trace.csv")
    if not rows:
        raise SystemExit(f"no kernel_trace.csv under {run_dir}")
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return [{"name": r["Kernel_Name"],
             "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])} for r in rows]


def _match(dispatches, order):
    """Assign dispatches to workloads: in the run's order, each workload's
    launches are the first run of its kernels, `warm` + `reps` times over, after
    the previous workload's (the dispatches of building its inputs come before
    it), of which the first `warm` are left out;
    the run's last dispatch is the copy.  Returns {name: [[dispatches of launch
    1], ...]}."""
    names = [d["name"] for d in dispatches]
    out, i = {}, 0
    for w in order:
        n_l = w.get("warm", 0) + w["reps"]  # warm-up launches first, then the counted ones
        seq = [pat for _ in range(n_l) for pat, n in w["kernels"] for _ in range(n)]
        while i + len(seq) <= len(names) and not all(p in names[i + k] for k, p in enumerate(seq)):
            i += 1
        if i + len(seq) > len(names):
            raise SystemExit(f"the launches of {w['name']} are not in the trace")
        per = len(seq) // n_l
        out[w["name"]] = [dispatches[i + r * per:i + (r + 1) * per]
                          for r in range(w.get("warm", 0), n_l)]
        i += len(seq)
    out["copy"] = [[dispatches[-1]]]
    return out


def _short(kernel: str) -> str:
    k = kernel.replace("void ", "").replace("hca::(anonymous namespace)::", "")
    return k.split("(")[0]


PROFILE_HEADER = """# {what}

Commands, in one job on one box (from /tmp with TMPDIR=/tmp; R = the repository):

    python3 $R/bench.py > $R/gpurun_out/bench.json
    rocprofv3 --kernel-trace --stats --output-format csv -d $R/gpurun_out/kt -o kt -- \\
        python3 $R/bench.py --counters-workload --reps 5 > $R/gpurun_out/kt_order.log
    rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d $R/gpurun_out/pf -o f -- \\
        python3 $R/bench.py --counters-workload > $R/gpurun_out/order.log
    rocprofv3 --pmc WRITE_SIZE --kernel-trace --output-format csv -d $R/gpurun_out/pw -o w -- \\
        python3 $R/bench.py --counters-workload
    rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES \\
        GRBM_GUI_ACTIVE --kernel-trace --output-format csv -d $R/gpurun_out/pm -o m -- \\
        python3 $R/bench.py --counters-workload
    python3 $R/bench.py --write-profiles $R/gpurun_out/kt $R/gpurun_out/pf $R/gpurun_out/pw \\
        $R/gpurun_out/pm $R/gpurun_out/profiles $R/gpurun_out/kt_order.log \\
        $R/gpurun_out/order.log $R/gpurun_out/bench.json

"""


def _read_order(path):
    with open(path) as f:
        return [json.loads(l)["order"] for l in f if l.startswith('{"order"')][-1]


def write_profiles(kt_dir, fetch_dir, write_dir, mfma_dir, out_dir, kt_order, pmc_order,
                   bench_json):
    kt = _match(_traced(kt_dir), _read_order(kt_order))
    order = _read_order(pmc_order)
    fetch = _match(_dispatches(fetch_dir), order)
    write = _match(_dispatches(write_dir), order)
    mfma = _match(_dispatches(mfma_dir), order)
    mdur = _match(_traced(mfma_dir), order)
    with open(bench_json) as f:
        bench = [json.loads(l) for l in f if l.startswith("{")][-1]
    bench_ms = {k: v["ms"] for k, v in bench.get("workloads", {}).items()}
    bench_ms["prefill_128k"] = bench["roofline"]["launch_ms"]
    cp_f = fetch["copy"][0][0]["c"]["FETCH_SIZE"]
    cp_w = write["copy"][0][0]["c"]["WRITE_SIZE"]
    f_scale = COPY_BYTES / (cp_f * 1024.0)
    w_scale = COPY_BYTES / (cp_w * 1024.0)
    rec = {"copy_bytes": COPY_BYTES, "copy_fetch_kib": cp_f, "copy_write_kib": cp_w,
           "fetch_scale": f_scale, "write_scale": w_scale, "workloads": {}}
    for w in order:
        name = w["name"]
        fd, wd, md, dd = fetch[name][0], write[name][0], mfma[name][0], mdur[name][0]
        fk = sum(d["c"]["FETCH_SIZE"] for d in fd)
        wk = sum(d["c"]["WRITE_SIZE"] for d in wd)
        ns = [d["ns"] for d in dd]
        main = int(np.argmax(ns))  # the workload's longest dispatch, for the clock
        gui = md[main]["c"].get("GRBM_GUI_ACTIVE", 0.0)
        launch_ns = [sum(d["ns"] for d in launch) for launch in kt[name]]
        e = {"source_sha256": sha256_files(w["src"]),
             "kernels": sorted({_short(d["name"]) for d in fd}),
             "trace_launches": len(launch_ns), "trace_avg_us": float(np.mean(launch_ns)) / 1e3,
             "trace_min_us": min(launch_ns) / 1e3, "trace_max_us": max(launch_ns) / 1e3,
             "bench_ms": bench_ms.get(name),
             "fetch_kib": fk, "write_kib": wk, "hbm_read_bytes": fk * 1024 * f_scale,
             "hbm_write_bytes": wk * 1024 * w_scale,
             "mfma_flops": 512.0 * sum(d["c"].get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) for d in md),
             "mfma_busy_cycles": sum(d["c"].get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for d in md),
             "pmc_duration_ns": int(sum(ns)),
             # the counter window exceeds a short dispatch: the clock only from >= 1 ms
             "sclk_mhz": round(gui / XCC / ns[main] * 1e3, 1) if ns[main] >= 1e6 else None}
        e["hbm_bytes"] = e["hbm_read_bytes"] + e["hbm_write_bytes"]
        rec["workloads"][name] = e
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, "counters.json"), "w") as f:
        json.dump(rec, f, indent=1)

    lines = ["| workload | kernels | launches | avg us | min us | max us | bench.py us (HIP "
             "events, same job) |", "|---|---|---:|---:|---:|---:|---:|"]
    for name, e in rec["workloads"].items():
        b = f"{e['bench_ms'] * 1e3:,.2f}" if e["bench_ms"] is not None else "-"
        lines.append(f"| {name} | {', '.join(e['kernels'])} | {e['trace_launches']} | "
                     f"{e['trace_avg_us']:,.2f} | {e['trace_min_us']:,.2f} | "
                     f"{e['trace_max_us']:,.2f} | {b} |")
    with open(os.path.join(out_dir, "kernel_trace_workloads.md"), "w") as f:
        f.write(PROFILE_HEADER.format(what="rocprofv3 kernel trace per workload launch (all "
                                      "kernels of one library call summed)")
                + "\n".join(lines) + "\n")
    lines = ["| workload | pmc-run us | HBM read GB | HBM write GB | MFMA TFLOP (counted) | "
             "MFMA busy / SIMD cycle | sclk MHz |", "|---|---:|---:|---:|---:|---:|---:|"]
    for name, e in rec["workloads"].items():
        clk = (e["sclk_mhz"] or 2400.0) * 1e6
        busy = e["mfma_busy_cycles"] / 1024 / (e["pmc_duration_ns"] * 1e-9 * clk)
        lines.append(f"| {name} | {e['pmc_duration_ns'] / 1e3:,.1f} | "
                     f"{e['hbm_read_bytes'] / 1e9:.3f} | {e['hbm_write_bytes'] / 1e9:.3f} | "
                     f"{e['mfma_flops'] / 1e12:.4f} | {busy:.3f} | {e['sclk_mhz'] or '-'} |")
    with open(os.path.join(out_dir, "counters.md"), "w") as f:
        f.write(PROFILE_HEADER.format(what="rocprofv3 counters per workload launch: HBM bytes "
                                      "(FETCH_SIZE, WRITE_SIZE scaled by a 1 GiB copy: "
                                      f"x{f_scale:.5f}, x{w_scale:.5f}), MFMA FLOPs "
                                      "(SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512), MFMA busy "
                                      "cycles per SIMD cycle (SQ_VALU_MFMA_BUSY_CYCLES / 1024 "
                                      "SIMDs), clock (GRBM_GUI_ACTIVE / 8 XCC / duration)")
                + "\n".join(lines) + "\n")
    print(json.dumps(rec, indent=1))


# ----------------------------------------------------------------- copy path
def copy_rate(out_md):
    """Per-CU rate of the copy path: one workgroup per CU moves 512 KiB (or 64
    KiB) of 1 KiB rows by LDS DMA or by 16-byte loads into VGPRs, 16 rows in
    flight per wave, with 4 or 8 waves, for 1, 32 and 256 workgroups, from HBM
    (the MALL flushed by a 1 GiB write first) or warm (a second pass over the
    same data: from L2 where the workgroups' data fit in it, 4 MiB per XCD,
    else from the MALL).  Bytes per shader clock (s_memtime) per workgroup,
    the median over workgroups; the clock from s_memtime against
    s_memrealtime (100 MHz)."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "long_context_compressed_hca_amd", "libhca_probe.so"))
    lib.hca_probe_copy_rate.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p]
    dev = torch.device("cuda:0")
    src = torch.ones(256 * (512 << 10) // 4, dtype=torch.float32, device=dev)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    rows = []
    for warm in (False, True):
        for grid, per_wg in ((1, 512 << 10), (32, 512 << 10), (256, 512 << 10),
                             (256, 64 << 10)):
            for waves in (4, 8):
                for dma in (1, 0):
                    clk = torch.zeros(3 * grid, dtype=torch.int64, device=dev)
                    flush.zero_()
                    torch.cuda.synchronize()
                    rc = lib.hca_probe_copy_rate(src.data_ptr(), grid, waves, per_wg,
                                                 2 if warm else 1, dma, clk.data_ptr(), stream)
                    if rc != 0:
                        raise SystemExit(f"copy probe launch failed: {rc}")
                    torch.cuda.synchronize()
                    c = clk.view(grid, 3).cpu().numpy()
                    bpc = per_wg / c[:, 0].astype(np.float64)
                    mhz = c[:, 0].astype(np.float64) / (c[:, 1].astype(np.float64) / 100.0)
                    rows.append({"source": "warm" if warm else "HBM", "workgroups": grid,
                                 "kib_per_wg": per_wg >> 10, "waves": waves, "path": "LDS DMA" if dma else "VGPR loads",
                                 "bytes_per_clk_per_cu": round(float(np.median(bpc)), 2),
                                 "min": round(float(bpc.min()), 2),
                                 "sclk_mhz": round(float(np.median(mhz)), 1)})
                    print(json.dumps(rows[-1]), flush=True)
    lib.hca_probe_mfma_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p]
    mfma = []
    for chains in (1, 4):
        clk = torch.zeros(8, dtype=torch.int64, device=dev)
        n = 4096
        if lib.hca_probe_mfma_rate(n, chains, clk.data_ptr(), stream) != 0:
            raise SystemExit("mfma probe launch failed")
        torch.cuda.synchronize()
        cyc = clk.view(4, 2)[:, 0].cpu().numpy().astype(np.float64) / n
        mfma.append({"chains": chains, "cycles_per_mfma_32x32x16_bf16": round(float(cyc.mean()), 2)})
        print(json.dumps(mfma[-1]), flush=True)
    lines = ["| source | workgroups | KiB each | waves | path | B/clk per CU (median) | min | "
             "sclk MHz |", "|---|---:|---:|---:|---|---:|---:|---:|"]
    for r in rows:
        lines.append(f"| {r['source']} | {r['workgroups']} | {r['kib_per_wg']} | {r['waves']} | "
                     f"{r['path']} | "
                     f"{r['bytes_per_clk_per_cu']} | {r['min']} | {r['sclk_mhz']} |")
    with open(out_md, "w") as f:
        f.write("# Per-CU copy path: 1 KiB rows, one workgroup per CU, 16 rows in flight "
                "per wave\n\nCommand (R = the repository):\n\n    python3 $R/bench.py "
                "--copy-rate $R/gpurun_out/copy_rate.md\n\n" + "\n".join(lines) + "\n\n"
                "MFMA issue (one wave per SIMD, 4096 v_mfma_f32_32x32x16_bf16 each, "
                "s_memtime cycles per MFMA): "
                + ", ".join(f"{m['chains']} accumulator chain(s): {m['cycles_per_mfma_32x32x16_bf16']}"
                            for m in mfma) + "\n")


# ----------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--cpu-positions", type=int, default=8192)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-step", action="store_true", help="skip the other workloads")
    ap.add_argument("--counters-workload", action="store_true")
    ap.add_argument("--reps", type=int, default=1, help="launches per workload (profiling)")
    ap.add_argument("--copy-rate", metavar="OUT_MD", help="per-CU copy-path probe, table to OUT_MD")
    ap.add_argument("--write-profiles", nargs=8,
                    metavar=("KT", "FETCH", "WRITE", "MFMA", "OUT", "KT_ORDER", "PMC_ORDER",
                             "BENCH_JSON"))
    args = ap.parse_args()
    if args.write_profiles:
        write_profiles(*args.write_profiles)
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
    if args.copy_rate:
        copy_rate(args.copy_rate)
        return
    if args.counters_workload:
        counters_workload(torch, hca, synth, args.reps)
        return
    counters = load_counters()

    # ---- the step: compress + prefill at 128K
    T, H = 131072, 64
    pf = w_prefill(torch, hca, synth, T, H)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for _ in range(args.warmup):
        pf["step"]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        hca.hca_compress(pf["tensors"][2], pf["tensors"][3], pf["tensors"][4], pf["tensors"][5])
        ev[i][0].record(stream)
        pf["call"]()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    launch_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    ms_step = elapsed * 1e3 / args.steps
    value = pf["flops"] / (ms_step * 1e-3) / 1e12
    achieved = pf["flops"] / (launch_ms * 1e-3) / 1e12
    cf = counter_fields(counters, "prefill_128k", pf["src"])
    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "HCA prefill at 128K context: batch 1, T=131072, 64 query "
                   "heads, 1 KV head, dim 512, block 128, window 128; compress + prefill "
                   "per step; bf16 in/out", "seq_len": T, "heads": H, "global_batch": 1,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_PEAK_TFLOPS, 4),
                     "traffic": cf["traffic"], "kernel": "hca prefill_kernel",
                     "flops_per_launch": pf["flops"], "algorithmic_bytes": pf["bytes"],
                     "launch_ms": round(launch_ms, 4)},
    }
    if "mfma_flops_counted" in cf:
        rec["roofline"]["mfma_flops_counted"] = cf["mfma_flops_counted"]
    c128 = counters.get("workloads", {}).get("prefill_128k", {})
    if cf["traffic"] is not None and c128.get("sclk_mhz"):
        rec["sclk_mhz"] = c128["sclk_mhz"]
        rec["sclk_source"] = "GRBM_GUI_ACTIVE / 8 XCC / prefill_kernel duration (rocprofv3 --pmc)"

    if not args.only_step:
        wl = {}
        vha = w_prefill_vha(torch, hca, synth, pf)
        r = run_workload(torch, "prefill_vha_128k", "the 128K prefill launch with the VHA head "
                         "mix fused (rank 16)", vha, max(3, args.steps), counters)
        r["overhead_vs_plain"] = round(r["ms"] / launch_ms - 1, 4)
        wl["prefill_vha_128k"] = r
        tensors = pf["tensors"]
        del pf, vha
        log(f"step: {ms_step:.3f} ms, prefill launch {launch_ms:.3f} ms")
        samples = {}
        for name, what, build in workload_table(torch, hca, synth):
            w = build()
            log(f"{name}")
            n = {"decode": 240, "decode_multi": 240, "compress_128k": 50}.get(name, max(3, args.steps))
            wl[name] = run_workload(torch, name, what, w, n, counters,
                                    back_to_back=name.startswith("decode"))
            if name in PARITY_SAMPLES and not args.no_cpu_baseline:
                samples[name] = parity_sample(torch, w, *PARITY_SAMPLES[name])
            if name == "decode" and not args.no_cpu_baseline:
                samples[name] = decode_parity_sample(torch, w)
            if name.startswith("decode"):
                wl[name]["us_per_call"] = round(wl[name]["ms"] * 1e3, 2)
                wl[name]["us_per_call_alone"] = round(
                    time_launches(torch, w["call"], n) * 1e3, 2)
            del w
            torch.cuda.empty_cache()
        rec["workloads"] = wl
        # decode in its own keys too (the metric's second half)
        rec["decode"] = {"metric": "decode HBM GB/s", "value": wl["decode"]["gbs"],
                         "unit": "GB/s", "us_per_call": wl["decode"]["us_per_call"],
                         "roofline": wl["decode"]["roofline"]}
    else:
        tensors = pf["tensors"]
    if not args.no_cpu_baseline:
        log("cpu baseline")
        rec["cpu_baseline"], rec["parity"] = cpu_baseline(args, torch, tensors, hca)
        if not args.only_step:
            rec["parity"].update(cpu_parity(samples))
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
