#!/usr/bin/env python3
"""Benchmark of the StateKV frame step on one MI355X (gfx950).

A step is one StateKV frame step of one layer (virtual-position RoPE, append
to D, attention over [compressed state; frame], scores, Top-B, gather) on one
frame of the synthetic stream.  Default workload: the InternVL3-1B-like layer
(bf16, 14 query / 2 KV heads, d = 64, T = 256, B = 4096); the stream generator
is the seeded one of the tests, extended past its 64 frames when more steps
are asked for.  All frames are resident in HBM before timing starts.  Setup
runs the B/T = 16 frames that fill the state (a step is an evicting frame
step, so the fill is part of building its state, like loading weights); then
W untimed warm-up steps and K timed steps follow, every one of them evicting
T tokens (constant work per frame).

--layers L steps a stack of L independent layers of the workload's shape
(each with its own seeded stream) through one launch per kernel; value is
then layer-frames/s, L times the stack's steps/s.

Printed: one JSON line with frames/s (value, wall clock over the K timed
steps), per-step latency statistics from events between steps in a second
pass of K steps (flatness), per-kernel execution times from start / stop
events recorded by each dispatch in a third pass, the roofline of the
dominant kernel (attention pass 1), and the CPU oracle timed on the host
cores on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "frames/s per layer StateKV step at B=4096,T=256; MFMA % of bf16 peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "kv_cache_compression_statekv_amd", "csrc", "statekv_kernels.hip")


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=512, help="timed frame steps (K)")
    p.add_argument("--warmup", type=int, default=16,
                   help="untimed evicting steps before timing (W), after the B/T frames that "
                        "fill the state")
    p.add_argument("--workload", default="ivl3_1b")
    p.add_argument("--distinct-frames", type=int, default=0,
                   help="frames drawn from the generator; later steps reuse them cyclically "
                        "(default: 128 for one layer, 4 for a stack)")
    p.add_argument("--layers", type=int, default=1,
                   help="run a stack of L independent layers of the workload's shape, every "
                        "kernel of the step covering all L layers in one launch; value is then "
                        "layer-frames/s (L x stack steps/s)")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="bounded CPU work for the oracle baseline (0 disables it)")
    p.add_argument("--no-kernel-timing", action="store_true")
    p.add_argument("--recent-window", action="store_true",
                   help="keep the B most recent tokens (the compute-matched ReKV-style window) "
                        "instead of the B best-scoring candidates")
    p.add_argument("--b-sweep", default="",
                   help="comma-separated budgets: run the workload's shape over --sweep-frames "
                        "frames at each B and compare with one-shot full causal attention over "
                        "the same tokens")
    p.add_argument("--sweep-frames", type=int, default=512)
    p.add_argument("--quadratic", action="store_true",
                   help="also run the quadratic comparison over the workload's full stream: "
                        "one-shot full causal attention over all N*T tokens, full attention "
                        "streamed frame by frame (no eviction), and StateKV streamed")
    p.add_argument("--decode-tokens", type=int, default=0,
                   help="also time the text phase: after --decode-frames frames of the workload "
                        "(default: its full stream), a --decode-prompt-token chunk and then this "
                        "many single-token steps, each attending over the whole detailed cache")
    p.add_argument("--decode-frames", type=int, default=0)
    p.add_argument("--decode-prompt", type=int, default=64)
    p.add_argument("--decode-only", action="store_true",
                   help="skip the frame-step measurement (only with --decode-tokens)")
    p.add_argument("--copy-calibration-mb", type=int, default=0,
                   help="first run one device-to-device copy of this many MiB (a kernel of known "
                        "traffic that rocprofv3 counters are scaled by)")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="no GPU work: turn two rocprofv3 --pmc counter_collection.csv files "
                        "(FETCH_SIZE, WRITE_SIZE) of a run with --copy-calibration-mb into "
                        "profiles/attn_fwd_<workload>_traffic.json")
    p.add_argument("--reference-rates", action="store_true",
                   help="only measure the libraries' own reference rates on this GPU: torch's bf16 "
                        "GEMM (hipBLASLt) and a read-only bf16 sum, as context for the roofline "
                        "fractions")
    return p.parse_args()


def pair_count(T: int, kept: int) -> int:
    """Query-key pairs of one head in a frame step: T*kept state pairs + causal frame pairs."""
    return T * kept + T * (T + 1) // 2


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch measured by rocprofv3 counters, if taken on the current source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def summarize_pmc(fetch_csv: str, write_csv: str, workload: str, copy_mb: int) -> dict:
    """HBM bytes per attn_fwd launch, scaled by the counters of a known copy."""
    import csv
    import statistics

    def per_kernel(path, counter):
        """Median over attn_fwd dispatches; the largest copy dispatch (the calibration copy)."""
        attn, copies = [], []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"]) * 1024.0  # KiB -> bytes
            if "attn_fwd_kernel" in r["Kernel_Name"]:
                attn.append(v)
            elif "copyBuffer" in r["Kernel_Name"]:
                copies.append((int(r["Grid_Size"]), v))
        return {"attn_fwd": statistics.median(attn), "copy": max(copies)[1]}

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    copy_bytes = copy_mb * (1 << 20)
    f_scale = copy_bytes / f["copy"]
    w_scale = copy_bytes / w["copy"]
    rec = {
        "kernel": "attn_fwd", "workload": workload,
        "source_sha256": kernel_source_hash(),
        "fetch_bytes_raw": f["attn_fwd"], "write_bytes_raw": w["attn_fwd"],
        "copy_calibration_bytes": copy_bytes,
        "copy_fetch_raw": f["copy"], "copy_write_raw": w["copy"],
        "fetch_scale": f_scale, "write_scale": w_scale,
        "bytes_per_launch": f["attn_fwd"] * f_scale + w["attn_fwd"] * w_scale,
    }
    path = os.path.join(ROOT, "profiles", f"attn_fwd_{workload}_traffic.json")
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
    return rec


def reference_rates(torch) -> dict:
    """torch's bf16 GEMM and read-only bf16 sum on this GPU (HIP events, 20
    repetitions after 3 warm-ups): the libraries' practical matrix-core and
    streaming rates, context for the fractions of the published peaks."""
    torch.cuda.set_device(0)

    def timed(fn, reps=20):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps * 1e3   # us

    gemm = []
    for m, n, k in ((4096, 4096, 4096), (8192, 8192, 8192), (16384, 16384, 8192)):
        a = torch.randn(m, k, dtype=torch.bfloat16, device="cuda")
        b = torch.randn(k, n, dtype=torch.bfloat16, device="cuda")
        us = timed(lambda: a @ b)
        tf = 2.0 * m * n * k / us / 1e6
        gemm.append({"m": m, "n": n, "k": k, "us": round(us, 1), "tflops": round(tf, 1),
                     "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
        del a, b
    reads = []
    for nbytes in (134_479_872, 500_000_000, 1_070_000_000, 4_000_000_000):
        x = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
        us = timed(lambda: x.sum(dtype=torch.float32))
        reads.append({"bytes": nbytes, "us": round(us, 1), "gbs": round(nbytes / us / 1e3, 1)})
        del x
    return {"bf16_gemm": gemm, "bf16_sum_read": reads}


def quadratic_comparison(skv, torch, np, wl):
    """Full causal attention vs StateKV over the same N*T tokens (one layer)."""
    from kv_cache_compression_statekv_amd.workload import stream_tokens

    N, T = wl.n_frames, wl.tokens_per_frame
    Hq, Hkv, d = wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    L = N * T
    tdtype = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    Q, K, V = (torch.from_numpy(x).to(tdtype).cuda() for x in stream_tokens(wl, N))
    common = dict(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, alpha=wl.alpha, dtype=wl.dtype,
                  rope_base=wl.rope_base, rope_orig_ctx=wl.rope_orig_ctx)
    stream = torch.cuda.current_stream()

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    # (i) one-shot: one frame of all L tokens in a state that never evicts.
    one_ms = []
    out = torch.empty((L, Hq, d), dtype=tdtype, device="cuda")
    for rep_i in range(3):
        st = skv.StateKV(tokens_per_frame=L, max_frames=1, budget=L, **common)
        ms = timed(lambda: st.prefill_frame(Q, K, V, 0, out=out))
        st.close()
        if rep_i:
            one_ms.append(ms)
    causal_pairs = L * (L + 1) / 2
    one_flops = 4.0 * Hq * d * causal_pairs

    def streamed(budget):
        st = skv.StateKV(tokens_per_frame=T, max_frames=N, budget=budget, **common)
        o = torch.empty((T, Hq, d), dtype=tdtype, device="cuda")
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(N + 1)]
        evs[0].record(stream)
        for n in range(N):
            sl = slice(n * T, (n + 1) * T)
            st.prefill_frame(Q[sl], K[sl], V[sl], n, out=o)
            evs[n + 1].record(stream)
        torch.cuda.synchronize()
        lat = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(N)]) * 1e3
        st.close()
        idx = np.arange(N)
        return {"total_ms": round(float(lat.sum()) / 1e3, 3),
                "frame_us_first": round(float(lat[0]), 2),
                "frame_us_median": round(float(np.median(lat)), 2),
                "frame_us_last": round(float(lat[-1]), 2),
                "slope_us_per_frame": round(float(np.polyfit(idx, lat, 1)[0]), 4)}

    full_stream = streamed(L)
    statekv = streamed(wl.budget)
    one = float(np.median(one_ms))
    return {
        "tokens": L, "frames": N, "budget": wl.budget,
        "full_causal_one_shot_ms": round(one, 3),
        "full_causal_algorithmic_tflop": round(one_flops / 1e12, 2),
        "full_causal_tflops": round(one_flops / (one * 1e-3) / 1e12, 1),
        "full_causal_mfma_frac": round(one_flops / (one * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "full_attention_streamed": full_stream,
        "statekv_streamed": statekv,
        "statekv_over_one_shot_time": round(statekv["total_ms"] / one, 4),
        "statekv_over_full_streamed_time": round(statekv["total_ms"] / full_stream["total_ms"], 4),
    }


def budget_sweep(skv, torch, np, wl, budgets, n_frames):
    """Per-budget cost of a stream of n_frames frames (one layer), and one-shot
    full causal attention over the same n_frames*T tokens."""
    from kv_cache_compression_statekv_amd.workload import FrameStream

    T, Hq, Hkv, d = wl.tokens_per_frame, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    tdtype = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    fs = FrameStream(wl, 0)
    distinct = 16   # frames reused cyclically (positions still advance)
    frames = [tuple(torch.from_numpy(x).to(tdtype).cuda() for x in fs.frame(n)) for n in range(distinct)]
    common = dict(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, alpha=wl.alpha, dtype=wl.dtype,
                  rope_base=wl.rope_base, rope_orig_ctx=wl.rope_orig_ctx)
    stream = torch.cuda.current_stream()
    L = n_frames * T
    out = []
    for B in budgets:
        st = skv.StateKV(tokens_per_frame=T, max_frames=n_frames, budget=B, **common)
        o = torch.empty((T, Hq, d), dtype=tdtype, device="cuda")
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_frames + 1)]
        evs[0].record(stream)
        for n in range(n_frames):
            st.prefill_frame(*frames[n % distinct], n, out=o)
            evs[n + 1].record(stream)
        torch.cuda.synchronize()
        lat = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(n_frames)]) * 1e3
        st.close()
        flops = 0.0
        for n in range(n_frames):
            k = min(B, n * T)
            pairs = T * k + T * (T + 1) // 2
            evicts = k + T > B
            flops += (6.0 if evicts else 4.0) * Hq * d * pairs
        steady = lat[min(n_frames - 1, -(-B // T)):]
        out.append({"budget": B, "total_ms": round(float(lat.sum()) / 1e3, 3),
                    "steady_frame_us_median": round(float(np.median(steady)), 2),
                    "executed_tflop": round(flops / 1e12, 3)})
    # One-shot full causal attention over the same L tokens (a state that never evicts).
    Q = torch.cat([frames[n % distinct][0] for n in range(n_frames)])
    K = torch.cat([frames[n % distinct][1] for n in range(n_frames)])
    V = torch.cat([frames[n % distinct][2] for n in range(n_frames)])
    o = torch.empty((L, Hq, d), dtype=tdtype, device="cuda")
    ms = []
    for i in range(3):
        st = skv.StateKV(tokens_per_frame=L, max_frames=1, budget=L, **common)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        st.prefill_frame(Q, K, V, 0, out=o)
        e1.record(stream)
        torch.cuda.synchronize()
        st.close()
        if i:
            ms.append(e0.elapsed_time(e1))
    full_ms = float(np.median(ms))
    full_flops = 4.0 * Hq * d * L * (L + 1) / 2
    for r in out:
        r["time_vs_full_one_shot"] = round(r["total_ms"] / full_ms, 4)
        r["flops_vs_full"] = round(r["executed_tflop"] * 1e12 / full_flops, 4)
    return {"frames": n_frames, "tokens": L, "full_causal_one_shot_ms": round(full_ms, 3),
            "full_causal_tflop": round(full_flops / 1e12, 3), "budgets": out}


def decode_bench(skv, torch, np, wl, n_frames, n_tokens, prompt, distinct=8):
    """Text phase after a stream of n_frames frames (one layer): a prompt chunk
    of `prompt` tokens, then n_tokens single-token steps, each attending over
    every row of D.  Frames cycle through `distinct` seeded frames (positions,
    so rotated keys, still advance)."""
    from kv_cache_compression_statekv_amd.workload import FrameStream, text_tokens

    T, Hq, Hkv, d, B = wl.tokens_per_frame, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.budget
    tdtype = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    esize = 2 if wl.dtype == "bf16" else 4
    prompt = max(1, min(prompt, T))
    fs = FrameStream(wl, 0)
    frames = [tuple(torch.from_numpy(x).to(tdtype).cuda() for x in fs.frame(n))
              for n in range(min(distinct, n_frames))]
    P0 = n_frames * T
    n_text = prompt + 2 * n_tokens
    text = [torch.from_numpy(x).to(tdtype).cuda() for x in text_tokens(wl, P0, n_text)]
    st = skv.StateKV(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, tokens_per_frame=T,
                     max_frames=n_frames, budget=B, alpha=wl.alpha, dtype=wl.dtype,
                     rope_base=wl.rope_base, rope_orig_ctx=wl.rope_orig_ctx, max_text=n_text)
    o = torch.empty((T, Hq, d), dtype=tdtype, device="cuda")
    for n in range(n_frames):
        st.prefill_frame(*frames[n % len(frames)], n, out=o)
    stream = torch.cuda.current_stream()
    lib, h = st._lib, st._h
    row = [(x.data_ptr(), x[0].numel() * x.element_size()) for x in text]
    optr = o.data_ptr()

    def dec(i, t):
        ptr = [p + i * rb for p, rb in row]
        rc = lib.statekv_decode(h, ptr[0], ptr[1], ptr[2], t, optr)
        if rc:
            raise skv.StateKVError(rc, "statekv_decode")

    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    dec(0, prompt)
    e1.record(stream)
    torch.cuda.synchronize()
    prompt_us = e0.elapsed_time(e1) * 1e3

    def token_pass(first):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_tokens + 1)]
        evs[0].record(stream)
        for i in range(n_tokens):
            dec(first + i, 1)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        return np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(n_tokens)]) * 1e3

    lat = token_pass(prompt)
    st.set_flags(skv.FLAG_KERNEL_TIMING)
    st.kernel_times(reset=True)
    token_pass(prompt + n_tokens)
    kernels = {}
    for name, (ms, cnt) in st.kernel_times().items():
        if name.startswith("decode") and cnt:
            kernels[name] = {"avg_us": round(1e3 * ms / cnt, 2), "launches": cnt}
    st.close()
    # Bytes the attention kernel must read per token: K and V of every visible
    # key (the context, the prompt and the earlier generated tokens).
    keys = P0 + prompt + n_tokens + (n_tokens - 1) / 2.0
    kv_bytes = keys * Hkv * d * esize * 2
    res = {"frames": n_frames, "frame_tokens": P0, "prompt_tokens": prompt,
           "prompt_us": round(prompt_us, 2), "token_steps": n_tokens,
           "token_us_median": round(float(np.median(lat)), 2),
           "token_us_p99": round(float(np.quantile(lat, 0.99)), 2),
           "tokens_per_s": round(1e6 / float(np.median(lat)), 1),
           "kv_bytes_per_token": int(kv_bytes), "kernels": kernels}
    t_attn = kernels.get("decode_attn", {}).get("avg_us")
    if t_attn:
        gbs = kv_bytes / (t_attn * 1e-6) / 1e9
        res["roofline_decode_attn"] = {"bound": "hbm", "achieved": round(gbs, 1),
                                       "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                       "frac": round(gbs / PEAK_HBM_GBS, 4)}
        res["step_hbm_frac"] = round(kv_bytes / (float(np.median(lat)) * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
    return res


def main():
    args = parse_args()
    if args.summarize_pmc:
        print(json.dumps(summarize_pmc(*args.summarize_pmc, args.workload,
                                       args.copy_calibration_mb or 256)))
        return
    if args.reference_rates:
        import torch
        print(json.dumps({"reference_rates": reference_rates(torch)}))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the StateKV frame step on one GPU only; "
              f"--gpus {args.gpus} (WORLD_SIZE={world}) is not supported: the library has no "
              "multi-GPU path (one state runs on one device).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import kv_cache_compression_statekv_amd as skv
    from kv_cache_compression_statekv_amd.workload import CONFIGS, FrameStream

    wl = CONFIGS[args.workload]
    if args.decode_only:
        if args.decode_tokens <= 0:
            print("--decode-only needs --decode-tokens", file=sys.stderr)
            sys.exit(2)
        torch.cuda.set_device(0)
        rec = {"workload": wl.name, "decode": decode_bench(
            skv, torch, np, wl, args.decode_frames or wl.n_frames, args.decode_tokens,
            args.decode_prompt)}
        print(json.dumps(rec))
        return
    T, Hq, Hkv, d, B = wl.tokens_per_frame, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.budget
    L = args.layers
    fill = math.ceil(B / T)     # frames that fill the state (setup, not steps)
    W = args.warmup
    K = args.steps
    timing_pass = 0 if args.no_kernel_timing else K
    latency_pass = K            # per-step events, no kernel timing: flatness
    total = fill + W + K + latency_pass + timing_pass
    tdtype = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.copy_calibration_mb:
        n = args.copy_calibration_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Inputs resident in HBM before timing (layer l of a stack: the seeded
    # stream of layer l).
    streams = [FrameStream(wl, l) for l in range(L)]
    fs = streams[0]
    distinct = min(total, args.distinct_frames or (128 if L == 1 else 4))
    frames = []
    for n in range(distinct):
        per_layer = [f.frame(n) for f in streams]
        frames.append(tuple(
            torch.from_numpy(per_layer[0][i] if L == 1 else np.stack([x[i] for x in per_layer]))
            .to(tdtype).to(dev).contiguous() for i in range(3)))
        if L > 1:
            print(f"bench: frame {n + 1}/{distinct} of {L} layers uploaded", file=sys.stderr, flush=True)
    out = torch.empty((T, Hq, d) if L == 1 else (L, T, Hq, d), dtype=tdtype, device=dev)
    torch.cuda.synchronize()

    st = skv.StateKV(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, tokens_per_frame=T,
                     max_frames=total, budget=B, alpha=wl.alpha, dtype=wl.dtype,
                     rope_base=wl.rope_base, rope_orig_ctx=wl.rope_orig_ctx, n_layers=L)
    if args.recent_window:
        st.set_flags(skv.FLAG_RECENT_WINDOW)
    lib, h = st._lib, st._h
    ptrs = [tuple(t.data_ptr() for t in f) for f in frames]
    optr = out.data_ptr()

    def step(n):
        q, k, v = ptrs[n % distinct]
        rc = lib.statekv_prefill_frame(h, q, k, v, n, optr)
        if rc:
            raise skv.StateKVError(rc, f"statekv_prefill_frame({n})")

    for n in range(fill + W):
        step(n)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for n in range(fill + W, fill + W + K):
        step(n)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    fps = L * K / elapsed      # layer-frames per second

    # Second pass: per-step events on the stream (GPU time of each step, for
    # flatness).  Third pass: per-kernel execution times from start / stop
    # events that each dispatch records.
    stream = torch.cuda.current_stream()
    n0 = fill + W + K
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(latency_pass + 1)]
    evs[0].record(stream)
    for i in range(latency_pass):
        step(n0 + i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    lat = [evs[i].elapsed_time(evs[i + 1]) for i in range(latency_pass)]
    n0 += latency_pass
    kernels = {}
    if timing_pass:
        st.set_flags(skv.FLAG_KERNEL_TIMING | (skv.FLAG_RECENT_WINDOW if args.recent_window else 0))
        st.kernel_times(reset=True)
        for n in range(n0, n0 + timing_pass):
            step(n)
        torch.cuda.synchronize()
        for name, (ms, cnt) in st.kernel_times().items():
            if cnt:
                kernels[name] = {"avg_us": 1e3 * ms / cnt, "launches": cnt}
        st.set_flags(skv.FLAG_RECENT_WINDOW if args.recent_window else 0)

    merge_kernel = "score_merge"     # the launch that merges pass 1's key splits
    pairs = pair_count(T, B)
    attn_flops = 4.0 * Hq * d * pairs * L             # QK^T + PV, causal-counted, all layers
    # + QK^T recomputed by the score pass (skipped by the recency window)
    executed_flops = (4.0 if args.recent_window else 6.0) * Hq * d * pairs * L
    roofline = None
    extra = {}
    if kernels.get("attn_fwd", {}).get("avg_us"):
        t_attn = kernels["attn_fwd"]["avg_us"] * 1e-6
        achieved = attn_flops / t_attn / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                    "traffic": load_traffic("attn_fwd", args.workload) if L == 1 else None}
        # Attention passes: pass 1, the score pass and the merge of pass 1's key
        # splits.  The merge runs in the launch named by merge_kernel, whose whole
        # time is counted (conservative when it shares the launch with other work).
        passes = ["attn_fwd", merge_kernel]
        t_passes = sum(kernels[k]["avg_us"] for k in passes if k in kernels) * 1e-6
        extra["attention_passes_mfma_frac"] = round(executed_flops / t_passes / 1e12 / PEAK_BF16_TFLOPS, 4)
        extra["attention_passes_kernels"] = [k for k in passes if k in kernels]
        # The bar the path is held to: half the bf16 peak in the attention
        # passes at B = 4096.
        extra["attention_passes_target_frac"] = 0.5
        extra["attention_passes_target_met"] = extra["attention_passes_mfma_frac"] >= 0.5
        t_step_kernels = sum(v["avg_us"] for v in kernels.values()) * 1e-6
        extra["kernel_sum_us_per_step"] = round(t_step_kernels * 1e6, 2)
    if kernels.get("rope_select", {}).get("avg_us"):
        # RoPE + append (copy-like, HBM roofline): reads Q, K, V of the frame and
        # its rows of the cos/sin table; writes the rotated queries, the frame's
        # pool rows and its D rows (K and V).  The previous frame's moves (at
        # most T rows per KV head, K and V, read and written) are not counted.
        esz = 2 if wl.dtype == "bf16" else 4
        rope_bytes = L * ((Hq + 2 * Hkv) * T * d * esz + T * d * 4 + (Hq + 4 * Hkv) * T * d * esz)
        gbs = rope_bytes / (kernels["rope_select"]["avg_us"] * 1e-6) / 1e9
        extra["hbm_rope_append"] = {"bytes": rope_bytes, "achieved_gbs": round(gbs, 1),
                                    "peak_gbs": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4),
                                    "note": "algorithmic bytes of the frame's RoPE and appends over "
                                            "the frame launch, which also makes the previous frame's "
                                            "Top-B decision and moves; latency-bound at these sizes"}
    if lat:
        lat_a = np.array(lat)
        idx = np.arange(lat_a.size)
        slope = float(np.polyfit(idx, lat_a, 1)[0]) if lat_a.size > 1 else 0.0
        q = max(1, lat_a.size // 8)
        extra["step_latency_us"] = {
            "median": round(float(np.median(lat_a)) * 1e3, 2),
            "p99": round(float(np.quantile(lat_a, 0.99)) * 1e3, 2),
            "slope_us_per_frame": round(slope * 1e3, 5),
            "last_over_first_median": round(float(np.median(lat_a[-q:]) / np.median(lat_a[:q])), 4),
        }

    quadratic = quadratic_comparison(skv, torch, np, wl) if args.quadratic else None
    decode = None
    if args.decode_tokens > 0:
        decode = decode_bench(skv, torch, np, wl, args.decode_frames or wl.n_frames,
                              args.decode_tokens, args.decode_prompt)
    b_sweep = None
    if args.b_sweep:
        b_sweep = budget_sweep(skv, torch, np, wl, [int(b) for b in args.b_sweep.split(",")],
                               args.sweep_frames)

    # CPU baseline: the oracle, started from the GPU's state, on the next frames.
    cpu = None
    if args.cpu_seconds > 0:
        from oracle import CompressedState, LayerConfig, frame_step
        try:
            from threadpoolctl import threadpool_info
            blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()
                                if i.get("user_api") == "blas"] or [1])
        except Exception:
            blas_threads = 1
        cfg = LayerConfig(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, tokens_per_frame=T,
                          budget=B, dtype=wl.dtype, rope_base=wl.rope_base, alpha=wl.alpha,
                          rope_orig_ctx=wl.rope_orig_ctx)
        kk, vv, pp = st.compressed_view(0)
        ostate = CompressedState(kk.float().cpu().numpy().astype(np.float64),
                                 vv.float().cpu().numpy().astype(np.float64),
                                 pp.cpu().numpy().astype(np.int64))
        n0 = total
        done, tc = 0, 0.0
        while tc < args.cpu_seconds and done < 512:
            q, k, v = fs.frame(n0 + done)
            c0 = time.perf_counter()
            ostate = frame_step(cfg, ostate, q, k, v, n0 + done).state
            tc += time.perf_counter() - c0
            done += 1
        # The same oracle on one thread (its matrix products' BLAS limited to
        # one thread), on a third of the time budget.
        one = None
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1, user_api="blas"):
                d1, t1 = 0, 0.0
                while t1 < args.cpu_seconds / 3 and d1 < 512:
                    q, k, v = fs.frame(n0 + done + d1)
                    c0 = time.perf_counter()
                    ostate = frame_step(cfg, ostate, q, k, v, n0 + done + d1).state
                    t1 += time.perf_counter() - c0
                    d1 += 1
            one = round(d1 / t1, 4)
        except ImportError:
            pass
        cpu = {"value": round(done / tc, 4), "unit": "frames/s", "cores": blas_threads,
               "value_1_thread": one,
               "kind": "oracle",
               "sample": f"{done} steady-state frames of the same stream (n={n0}..{n0 + done - 1}), "
                         f"float64 numpy oracle, {tc:.1f} s; cores = BLAS threads of its matrix "
                         "products (element-wise steps run on one thread); value_1_thread: the "
                         "following frames with BLAS limited to one thread, a third of the time"}

    st.close()
    rec = {
        "metric": METRIC,
        "value": round(fps, 2),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "fill_frames": fill,
        "ms_per_step": round(1e3 * elapsed / K, 5),
        "stack_steps_per_s": round(K / elapsed, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {L} layer{'s' if L > 1 else ''}"
                               f"{' stepped together (one launch per kernel)' if L > 1 else ''}, "
                               f"Hq={Hq}, Hkv={Hkv}, d={d}, T={T}, B={B}, "
                               f"alpha={wl.alpha:g}, seeded Gaussian frames with {wl.n_sinks} "
                               f"drifting sink keys per frame",
                   "tokens_per_frame": T, "budget": B, "layers": L,
                   "policy": "recent window (ReKV-style)" if args.recent_window else "StateKV Top-B"},
        "tokens_per_s": round(fps * T, 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        **extra,
        **({"quadratic": quadratic} if quadratic else {}),
        **({"b_sweep": b_sweep} if b_sweep else {}),
        **({"decode": decode} if decode else {}),
        "attn_fwd_algorithmic_gflop": round(attn_flops / 1e9, 4),
        "executed_gflop_attention_passes": round(executed_flops / 1e9, 4),
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
