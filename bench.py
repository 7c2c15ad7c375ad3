#!/usr/bin/env python3
"""Benchmark of the batch-1 codebook-TTS decode path on one MI355X.

Workload (one "step" = one utterance through the whole hot path): the
36-layer Qwen3-4B-shaped backbone with the fused 8 x 1026 head in FP8 e4m3
W8A8 (per-row weight scales, static activation scales calibrated on a seeded
16-token prompt plus 16 BF16 frames), a P = 13 prompt prefilled in one batched
pass, then 1017 greedy delay-pattern decode frames (KV 14 -> 1030), each frame
one replay of the position-agnostic frame graph.  Weights and prompts are
seeded synthetic draws (no trained checkpoint exists here).

The JSON line reports decode ms/frame (FP8) as the metric, plus BF16 decode
ms/frame, prefill ms/token, the roofline of the dominant kernel (the
persistent frame kernel) measured with HIP events on the library's stream,
and the CPU oracle timed on a bounded sample on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
KV_BYTES_PER_POS = 147456  # 36 layers x 2 (K, V) x 8 kv heads x 128 x 2 bytes


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def frame_bytes(shape, precision: str, kv_len: float) -> float:
    """Algorithmic HBM bytes of one decode frame: every projection and the head read once,
    FP8 row scales, norm gains, the 8 embedding rows, and the K/V of kv_len positions."""
    d, hd, F, L = shape.hidden, shape.head_dim, shape.ffn, shape.n_layers
    qd, kvd = shape.q_dim, shape.kv_dim
    per_layer = (qd + 2 * kvd) * d + d * qd + 2 * F * d + d * F
    head = shape.n_codebooks * shape.codebook_size * d
    wb = 1 if precision == "fp8" else 2
    scales = 4 * (L * (qd + 2 * kvd + d + 2 * F + d) + shape.n_codebooks * shape.codebook_size) if precision == "fp8" else 0
    gains = 4 * (L * (2 * d + 2 * hd) + d)
    emb = shape.n_codebooks * d * 2
    kv = kv_len * L * 2 * shape.n_kv_heads * hd * 2
    return (per_layer * L + head) * wb + scales + gains + emb + kv


def cpu_oracle_baseline(shape, weights, scales, prompt, n_frames=2):
    """The CPU oracle (FP8 storage-faithful mode, float32 weight storage) on the whole
    36-layer model: the prompt prefilled, then n_frames decode frames with the BLAS on every
    host thread, then one more frame on one thread.  Building the oracle (the float32 copies
    and the e4m3 weight quantisation) is not timed."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle.model import OracleModel

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    t0 = time.perf_counter()
    m = OracleModel(shape, weights, "fp8", "S", act_scales=scales, storage=np.float32,
                    max_seq=len(prompt) + n_frames + 2)
    t_build = time.perf_counter() - t0
    m.prefill(prompt)
    t1 = time.perf_counter()
    for _ in range(n_frames):
        m.decode_frame()
    t2 = time.perf_counter()
    with threadpool_limits(1):
        t3 = time.perf_counter()
        m.decode_frame()
        t4 = time.perf_counter()
    ms = (t2 - t1) / n_frames * 1e3
    return {"value": round(ms, 1), "unit": "ms/frame", "cores": int(threads), "kind": "oracle",
            "cpu_count": os.cpu_count(), "one_thread_ms_per_frame": round((t4 - t3) * 1e3, 1),
            "sample": f"whole {shape.n_layers}-layer FP8 decode frames (KV {len(prompt) + 1}..{len(prompt) + n_frames}) "
                      f"after a P={len(prompt)} prefill: {n_frames} frames on {threads} BLAS threads, then one frame "
                      f"on 1 thread; building the oracle ({t_build:.0f} s) not timed"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--frames", type=int, default=1017, help="decode frames per FP8 utterance")
    ap.add_argument("--bf16-frames", type=int, default=256)
    ap.add_argument("--prompt", type=int, default=13)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bf16", action="store_true")
    ap.add_argument("--layers", type=int, default=36, help="backbone depth (36 = the benchmark model)")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the prefix-reuse and KV-4096 decode measurements")
    ap.add_argument("--no-kv-slope", action="store_true",
                    help="skip the chunked utterance that measures frame time against KV length")
    ap.add_argument("--no-batched", action="store_true",
                    help="skip batched multi-stream decode (M = 2 .. 128 utterances per step)")
    ap.add_argument("--no-one-layer", action="store_true",
                    help="skip the one-layer decode step with one and rotated weight copies")
    ap.add_argument("--no-kernel-classes", action="store_true",
                    help="skip the per-kernel-class event timing that follows the timed region")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="also time the vendor GEMM library (torch.matmul in bf16, torch._scaled_mm in e4m3: "
                         "hipBLASLt) on the prefill's GEMM shapes, as context for the tiled GEMM's MFMA fraction")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain elementwise copy of this many MiB before the timed region (a known-size "
                         "kernel that calibrates the HBM byte counters of a rocprofv3 --pmc run)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this path runs on one GPU; multi-GPU runs are not part of this build "
              "(each GPU would run its own independent utterances)", file=sys.stderr)
        return 2

    import torch

    import synthetic as S
    from autoregressive_codebook_tts_amd import hta

    shape = S.QWEN3_4B.with_layers(args.layers)
    max_seq = args.prompt + args.frames + 8
    log(f"drawing weights ({shape.n_layers} layers, bf16, seed {S.SEEDS['full_weights']})")
    w = S.make_weights(shape, S.SEEDS["full_weights"], "bf16")
    log("uploading weights")
    tensors, src = hta.weights_to_device(w, shape.n_layers)
    prompt = S.token_ids(S.SEEDS["full_prompt"], args.prompt, shape.text_vocab)
    calib = S.token_ids(S.SEEDS["calib_prompt"], 16, shape.text_vocab)
    extra = {}

    # ---------------------------------------------------------------- BF16 context: calibration + BF16 numbers
    log("BF16 context: load + FP8 calibration")
    b_seq = max(max_seq, args.prompt + args.bf16_frames + 8, 520)  # room for the P = 512 prefill
    bctx = hta.Hta(shape, "bf16", max_seq=b_seq, max_prefill=min(512, b_seq))
    bctx.load_weights(tensors, src)
    scales = bctx.calibrate(calib, 16)
    if not args.no_bf16:
        log("BF16 decode timing")
        ms_b = []
        for i in range(args.warmup + args.steps):
            bctx.reset(0)
            bctx.prefill(prompt)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(bctx.stream)
            bctx.decode_frames(args.bf16_frames)
            e1.record(bctx.stream)
            e1.synchronize()
            if i >= args.warmup:
                ms_b.append(e0.elapsed_time(e1) / args.bf16_frames)
        extra["decode_ms_per_frame_bf16"] = round(statistics.mean(ms_b), 4)
        kv_mean = args.prompt + (args.bf16_frames + 1) / 2
        extra["frame_hbm_frac_bf16"] = round(frame_bytes(shape, "bf16", kv_mean) / (extra["decode_ms_per_frame_bf16"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        extra["prefill_ms_per_token_bf16_p13"] = round(_prefill_ms(bctx, prompt) / len(prompt), 4)
        if shape.n_layers == 36:
            extra.update(_prefill_sizes(bctx, shape, "bf16"))
    if not args.no_bf16 and not args.no_kernel_classes:
        bctx.reset(0)
        bctx.prefill(prompt)
        extra["kernel_us_bf16"] = {k: round(v, 2) for k, v in bctx.time_kernels(16).items() if v > 0}
    bctx.close()
    del bctx

    # ---------------------------------------------------------------- FP8 context: the timed workload
    log("FP8 context: load")
    # room for the long-context measurement (4095 prompt keys + the timed frames); the KV
    # length a frame attends, not the cache's capacity, sets the frame's work
    long_kv = shape.n_layers == 36 and not args.no_long
    f_seq = max(max_seq, LONG_PROMPT + LONG_FRAMES + 8) if long_kv else max(max_seq, 520)
    ctx = hta.Hta(shape, "fp8", max_seq=f_seq, max_prefill=min(512, f_seq))
    ctx.load_weights(tensors, src, act_scales=scales)
    del tensors
    if args.copy_probe_mib:
        n = args.copy_probe_mib * 1024 * 1024 // 4
        src_t = torch.ones(n, dtype=torch.float32, device="cuda")
        dst_t = torch.empty_like(src_t)
        with torch.cuda.stream(ctx.stream):
            torch.neg(src_t, out=dst_t)
        torch.cuda.synchronize()
        del src_t, dst_t
    log(f"FP8 timed region: {args.warmup} warmup + {args.steps} steps of prefill {args.prompt} + {args.frames} frames")
    dec_ms = []
    for i in range(args.warmup):
        ctx.reset(0)
        ctx.prefill(prompt)
        ctx.decode_frames(args.frames)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    clock = {}
    for i in range(args.steps):
        ctx.reset(0)
        ctx.prefill(prompt)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # the last utterance: read the clocks on a host thread while its frames run
        sampler = _clock_sampler(clock) if i == args.steps - 1 else None
        e0.record(ctx.stream)
        codes, done = ctx.decode_frames(args.frames)
        e1.record(ctx.stream)
        e1.synchronize()
        if sampler is not None:
            sampler.join(timeout=30)
        dec_ms.append(e0.elapsed_time(e1) / args.frames)
    torch.cuda.synchronize()
    # device memory the process has held so far (weights, both contexts' workspaces: all through torch)
    extra["peak_device_memory_gb"] = round(torch.cuda.max_memory_reserved() / 1e9, 2)
    extra["gpu_clocks_during_decode"] = clock.get("value")
    wall = time.perf_counter() - t0
    ms_frame = statistics.mean(dec_ms)
    kv_mean = args.prompt + (args.frames + 1) / 2
    extra["frame_hbm_frac_fp8"] = round(frame_bytes(shape, "fp8", kv_mean) / (ms_frame * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    extra["frame_bytes_fp8_mean"] = int(frame_bytes(shape, "fp8", kv_mean))
    extra["prefill_ms_per_token_fp8_p13"] = round(_prefill_ms(ctx, prompt) / len(prompt), 4)
    if shape.n_layers == 36:
        extra.update(_prefill_sizes(ctx, shape, "fp8"))
        extra["prefill_e4m3_mfma"] = _prefill_e4m3_mfma(ctx, shape, prompt)
    # roofline of the dominant kernel: the persistent frame kernel is the whole decode step (every
    # weight, scale, gain and the KV once per launch); its average launch duration is the event-timed
    # decode region divided by the frame count (back-to-back launches on the library's stream, so the
    # few-microsecond launch gaps are included)
    workload = (f"FP8 W8A8 decode, P={args.prompt} prompt then {args.frames} greedy delay-pattern frames "
                f"(KV {args.prompt + 1}->{args.prompt + args.frames}), seeded random weights")
    k_bytes = frame_bytes(shape, "fp8", kv_mean)
    k_us = ms_frame * 1e3
    achieved = k_bytes / (k_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": "k_frame<1, 128> (persistent decode frame: 36 layers + head)",
                "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": _traffic(workload, shape),
                "bytes_per_launch": int(k_bytes), "avg_launch_us": round(k_us, 3)}
    if shape.n_layers == 36 and not args.no_kv_slope:
        log("per-frame time against KV length (FP8)")
        extra.update(_frame_vs_kv(ctx, prompt, args.frames))
    if long_kv:
        log("prefix reuse and long-context decode (FP8)")
        extra.update(_prefix_reuse(ctx, shape))
        extra.update(_long_decode(ctx, shape))
    if not args.no_kernel_classes:
        log("per-kernel timing (FP8)")
        ctx.reset(0)
        ctx.prefill(prompt)
        extra["kernel_us_fp8"] = {k: round(v, 2) for k, v in ctx.time_kernels(32).items() if v > 0}
    ctx.close()

    if shape.n_layers == 36 and not args.no_batched:
        log("batched multi-stream decode (FP8), M = 2 .. 128")
        extra["batched_decode_fp8"] = _batched(shape, w, scales, prompt, ms_frame)
    if shape.n_layers == 36 and args.vendor_gemm:
        log("vendor GEMM library on the prefill shapes")
        extra["vendor_gemm_us"] = _vendor_gemm(shape)
    if shape.n_layers == 36 and not args.no_one_layer:
        log("one-layer decode step at KV 512 / 2048, one weight copy and rotated copies")
        extra["one_layer"] = _one_layer(shape, w, scales)
    cpu = None
    if not args.no_cpu_baseline:
        log("CPU oracle baseline (bounded sample)")
        cpu = cpu_oracle_baseline(shape, w, scales, prompt)

    line = {
        "metric": "decode ms/frame @bs1 (FP8 e4m3 W8A8), 36-layer Qwen3-4B-shaped TTS backbone + 8x1026 head",
        "value": round(ms_frame, 4), "unit": "ms/frame", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 2), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": workload,
                   "layers": shape.n_layers, "hidden": shape.hidden, "heads": f"{shape.n_q_heads}q/{shape.n_kv_heads}kv",
                   "ffn": shape.ffn, "codebooks": f"{shape.n_codebooks}x{shape.codebook_size}",
                   "prompt_tokens": args.prompt, "frames": args.frames},
        "roofline": roofline, "cpu_baseline": cpu,
    }
    line.update(extra)
    print(json.dumps(line), flush=True)
    hta.close_all()
    return 0


def _clock_sampler(out: dict):
    """Start a host thread that reads the GPU's current clock levels once (the driver's
    pp_dpm_sclk / pp_dpm_mclk / pp_dpm_fclk files in sysfs, read-only; no child process)
    while the caller's decode runs; out["value"] gets the current level of each, per card,
    or the reason none were read.  Context for the timings, not part of them."""
    import glob
    import threading

    def run():
        try:
            time.sleep(0.3)  # well inside the 1017-frame decode (about 1.3 s)
            cards = {}
            for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
                levels = {}
                for name in ("pp_dpm_sclk", "pp_dpm_mclk", "pp_dpm_fclk"):
                    try:
                        with open(os.path.join(dev, name)) as f:
                            cur = [ln.strip() for ln in f if ln.strip().endswith("*")]
                    except OSError:
                        continue
                    if cur:
                        levels[name[7:]] = cur[0].split(":", 1)[-1].rstrip("*").strip()
                if levels:
                    cards[os.path.basename(os.path.dirname(dev))] = levels
            out["value"] = cards or "unavailable: no readable clock levels in sysfs"
        except Exception as ex:  # another sysfs layout
            out["value"] = f"unavailable: {type(ex).__name__}"

    t = threading.Thread(target=run, daemon=True)
    t.start()
    return t


def _vendor_gemm(shape, reps: int = 20) -> dict:
    """Device us per call of the vendor library on the prefill GEMMs (M = P rows against
    the [N][K] weights): torch.matmul in bf16 and torch._scaled_mm in e4m3 (unit scales),
    random operands, after 3 warm-up calls; the e4m3 library GEMM uses the fp8 MFMA."""
    import torch

    d, F, W = shape.hidden, shape.ffn, shape.q_dim + 2 * shape.kv_dim
    out = {}
    for P in (128, 512):
        for name, N, K in (("qkv", W, d), ("o", d, shape.q_dim), ("gate_up", 2 * F, d), ("down", d, F)):
            a = torch.randn(P, K, device="cuda", dtype=torch.bfloat16)
            b = torch.randn(N, K, device="cuda", dtype=torch.bfloat16)
            a8, b8 = a.to(torch.float8_e4m3fn), b.to(torch.float8_e4m3fn)
            one = torch.ones((), device="cuda")
            res = {}
            for kind, fn in (("bf16", lambda: a @ b.t()),
                             ("e4m3", lambda: torch._scaled_mm(a8, b8.t(), scale_a=one, scale_b=one,
                                                               out_dtype=torch.bfloat16))):
                try:
                    for _ in range(3):
                        fn()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(reps):
                        fn()
                    e1.record()
                    e1.synchronize()
                    us = e0.elapsed_time(e1) / reps * 1e3
                    res[kind] = {"us": round(us, 2), "mfma_frac_of_bf16_peak": round(
                        2.0 * P * N * K / (us * 1e-6) / 1e12 / PEAK_MFMA_BF16_TFLOPS, 4)}
                except Exception as ex:  # a library build without the e4m3 path
                    res[kind] = f"unavailable: {type(ex).__name__}"
            out[f"{name}_p{P}"] = res
    return out


def _traffic(workload: str, shape):
    """HBM bytes per frame-kernel launch from the rocprofv3 counter runs recorded in traffic.json,
    or None when they were taken on another workload or before the kernel's sources last changed."""
    from autoregressive_codebook_tts_amd import pmc_traffic

    path = pmc_traffic.TRAFFIC_JSON
    if shape.n_layers != 36 or not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("workload") != workload or t.get("source_sha256") != pmc_traffic.source_digest():
        return None
    return t["traffic_bytes_per_launch"]


PEAK_MFMA_BF16_TFLOPS = 2500.0  # dense bf16; the FP8 prefill widens e4m3 weights to bf16 for the MFMA
PEAK_MFMA_FP8_TFLOPS = 5000.0   # dense e4m3 (the opt-in e4m3 MFMA form of the prefill GEMMs)


def prefill_flops(shape, P: int) -> float:
    """GEMM flops (2 per weight per token) plus causal attention (QK^T and PV over the P(P+1)/2
    visible pairs per head) of one cold P-token prefill."""
    d, hd, F = shape.hidden, shape.head_dim, shape.ffn
    qd, kvd = shape.q_dim, shape.kv_dim
    per_layer = (qd + 2 * kvd) * d + d * qd + 2 * F * d + d * F
    attn = 2 * 2 * shape.n_q_heads * hd * P * (P + 1) / 2
    return shape.n_layers * (2 * per_layer * P + attn)


def _prefill_sizes(ctx, shape, prec: str) -> dict:
    """ms/token at P = 128 and 512 (seeded prompts) and the MFMA fraction at P = 512."""
    import synthetic as S

    out = {}
    for P in (128, 512):
        ids = S.token_ids(S.SEEDS[f"prefill_{P}"], P, shape.text_vocab)
        ms = _prefill_ms(ctx, ids, reps=5)
        out[f"prefill_ms_per_token_{prec}_p{P}"] = round(ms / P, 4)
        if P == 512:
            out[f"prefill_mfma_frac_{prec}_p512"] = round(prefill_flops(shape, P) / (ms * 1e-3) / 1e12 / PEAK_MFMA_BF16_TFLOPS, 4)
    return out


def _prefill_e4m3_mfma(ctx, shape, prompt) -> dict:
    """The FP8 prefills again with the opt-in e4m3 MFMA form of the GEMMs (hta option
    FP8_MFMA): faster contractions whose sums carry fewer bits than fp32, so not the FP8
    path the parity tests hold to; reported beside it, MFMA fraction against the e4m3 peak."""
    import synthetic as S
    from autoregressive_codebook_tts_amd import hta

    ctx.set_option(hta.OPT_FP8_MFMA, 1)
    try:
        out = {"prefill_ms_per_token_p13": round(_prefill_ms(ctx, prompt) / len(prompt), 4)}
        for P in (128, 512):
            ids = S.token_ids(S.SEEDS[f"prefill_{P}"], P, shape.text_vocab)
            ms = _prefill_ms(ctx, ids, reps=5)
            out[f"prefill_ms_per_token_p{P}"] = round(ms / P, 4)
            if P == 512:
                out["prefill_mfma_frac_of_e4m3_peak_p512"] = round(
                    prefill_flops(shape, P) / (ms * 1e-3) / 1e12 / PEAK_MFMA_FP8_TFLOPS, 4)
    finally:
        ctx.set_option(hta.OPT_FP8_MFMA, 0)
    return out


LONG_PROMPT, LONG_FRAMES = 4095, 64


def _batched(shape, w, scales, prompt, ms_single, Ms=(2, 4, 8, 16, 32, 64, 128), warm: int = 8, frames: int = 64) -> dict:
    """Batched decode: M utterances (the P=13 prompt's seed plus m) prefilled into one
    FP8 context, then `warm` steps and `frames` timed steps of all M together (one
    captured step graph each); aggregate frames/s against the single-stream frame kernel."""
    import torch
    import synthetic as S
    from autoregressive_codebook_tts_amd import hta

    tensors, src = hta.weights_to_device(w, shape.n_layers)
    out = {"single_stream_frames_per_s": round(1e3 / ms_single, 1)}
    for M in Ms:
        rows = max(16, len(prompt), M)  # the row buffers hold one row per stream (max_prefill <= max_seq)
        ctx = hta.Hta(shape, "fp8", max_seq=max(len(prompt) + warm + frames + 8, rows), max_prefill=rows, n_streams=M)
        ctx.load_weights(tensors, src, act_scales=scales)
        for m in range(M):
            ctx.select_stream(m)
            ctx.prefill(S.token_ids(S.SEEDS["full_prompt"] + m, len(prompt), shape.text_vocab))
        ctx.decode_frames(warm)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(ctx.stream)
        ctx.decode_frames(frames)
        e1.record(ctx.stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1) / frames
        out[f"M{M}"] = {"ms_per_step": round(ms, 4), "frames_per_s": round(M * 1e3 / ms, 1)}
        ctx.close()
    del tensors
    return out


def _frame_vs_kv(ctx, prompt, n_frames: int, chunk: int = 64) -> dict:
    """One utterance decoded in chunks of `chunk` frames, each chunk event-timed: device us
    per frame against the mean number of keys attended, and the least-squares slope."""
    import torch

    ctx.reset(0)
    ctx.prefill(prompt)
    kv, us = [], []
    done = 0
    while done + chunk <= n_frames:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(ctx.stream)
        ctx.decode_frames(chunk)
        e1.record(ctx.stream)
        e1.synchronize()
        kv.append(len(prompt) + done + (chunk + 1) / 2)
        us.append(e0.elapsed_time(e1) * 1e3 / chunk)
        done += chunk
    slope, icpt = np.polyfit(np.array(kv), np.array(us), 1)
    return {"frame_us_vs_kv_fp8": {"kv": [round(k, 1) for k in kv], "us": [round(u, 2) for u in us],
                                   "slope_ns_per_key": round(slope * 1e3, 3), "intercept_us": round(icpt, 2)}}


def _one_layer(shape, w, scales, kvs=(512, 2048), rounds: int = 8) -> dict:
    """The one-layer decode step (one 4B layer plus the head, on the decode frame kernel) at
    KV length L: the mean kernel time over `rounds` frames of one context (its weights stay
    in the 256 MB memory-side cache between frames) and over rounds of frames rotated
    across enough contexts that their weight copies exceed 800 MB (each frame then reads
    its weights from HBM).  Each context holds its own copy; all share one stream."""
    import dataclasses

    import torch
    import synthetic as S
    from autoregressive_codebook_tts_amd import hta

    sh1 = dataclasses.replace(shape.with_layers(1), text_vocab=1024)
    w1 = {k: v for k, v in w.items() if not k.startswith("layers.") or k.startswith("layers.0.")}
    w1["e_text"] = w["e_text"][:1024]
    tensors, src = hta.weights_to_device(w1, 1)
    sc1 = np.concatenate([scales[:4], scales[-1:]]).astype(np.float32)
    stream = torch.cuda.Stream()
    out = {}
    for prec in ("bf16", "fp8"):
        copy_bytes = frame_bytes(sh1, prec, 0)
        n_copies = max(4, int(np.ceil(800e6 / copy_bytes)))
        for L in kvs:
            ids = S.token_ids(S.SEEDS["full_prompt"], L - 1, sh1.text_vocab)
            ctxs = []
            for _ in range(n_copies):
                c = hta.Hta(sh1, prec, max_seq=L + 2 * rounds * n_copies + 4, max_prefill=512, stream=stream)
                c.load_weights(tensors, src, act_scales=sc1 if prec == "fp8" else None)
                for i in range(0, L - 1, 512):
                    c.prefill(ids[i:i + 512])
                c.time_kernels(1)  # warm
                ctxs.append(c)
            one = [ctxs[0].time_kernels(1)["frame"] for _ in range(rounds)]
            rot = [c.time_kernels(1)["frame"] for _ in range(rounds) for c in ctxs]
            b = frame_bytes(sh1, prec, L)
            out[f"{prec}_kv{L}"] = {
                "one_copy_us": round(statistics.mean(one), 2), "rotated_us": round(statistics.mean(rot), 2),
                "copies": n_copies, "bytes_per_frame": int(b),
                "rotated_frac_of_8TBs": round(b / (statistics.mean(rot) * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
            for c in ctxs:
                c.close()
    del tensors
    return out


def _prefix_reuse(ctx, shape, reps: int = 5) -> dict:
    """A 64-token preamble prefilled once and kept (hta_reset(64)), then 8 different
    16-token suffixes, against cold 80-token prefills of the same ids: device ms per
    suffix (median over suffixes of the median over reps)."""
    import torch
    import synthetic as S

    pre = S.token_ids(S.SEEDS["preamble"], 64, shape.text_vocab)
    sufs = [S.token_ids(S.SEEDS["suffix_base"] + i, 16, shape.text_vocab) for i in range(8)]

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(ctx.stream)
        fn()
        e1.record(ctx.stream)
        e1.synchronize()
        return e0.elapsed_time(e1)

    ctx.reset(0)
    ctx.prefill(pre)
    reuse, cold = [], []
    for suf in sufs:
        r = [timed(lambda: (ctx.reset(64), ctx.prefill(suf))) for _ in range(reps + 1)][1:]
        reuse.append(statistics.median(r))
    for suf in sufs:
        full = np.concatenate([pre, suf]).astype(np.int32)
        c = [timed(lambda: (ctx.reset(0), ctx.prefill(full))) for _ in range(reps + 1)][1:]
        cold.append(statistics.median(c))
    r_ms, c_ms = statistics.median(reuse), statistics.median(cold)
    return {"prefix_reuse_fp8": {"preamble": 64, "suffix": 16, "suffixes": 8, "reuse_ms": round(r_ms, 4),
                                 "cold_80_ms": round(c_ms, 4), "saved_frac": round(1.0 - r_ms / c_ms, 4)}}


def _long_decode(ctx, shape) -> dict:
    """FP8 decode with 4096 keys: a 4095-token prompt prefilled in chunks of 512, then
    LONG_FRAMES frames timed (KV 4096 -> 4096 + LONG_FRAMES - 1)."""
    import torch
    import synthetic as S

    ids = S.token_ids(S.SEEDS["long_prompt"], LONG_PROMPT, shape.text_vocab)
    ctx.reset(0)
    for i in range(0, LONG_PROMPT, 512):
        ctx.prefill(ids[i:i + 512])
    ctx.decode_frames(1)  # warm: the first frame attends 4096 keys
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(ctx.stream)
    _, done = ctx.decode_frames(LONG_FRAMES)
    e1.record(ctx.stream)
    e1.synchronize()
    # every requested frame runs the whole step; `done` only says an end-of-audio code
    # appeared among them (random weights)
    ms = e0.elapsed_time(e1) / LONG_FRAMES
    kv_mean = LONG_PROMPT + 1 + (LONG_FRAMES + 1) / 2
    frac = frame_bytes(shape, "fp8", kv_mean) / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS
    return {"decode_ms_per_frame_fp8_kv4096": round(ms, 4), "frame_hbm_frac_fp8_kv4096": round(frac, 4),
            "kv4096_end_of_audio_seen": bool(done)}


def _prefill_ms(ctx, prompt, reps: int = 20) -> float:
    """Median of reps (reset + prefill) device times, after one warm-up."""
    import torch

    ts = []
    for i in range(reps + 1):
        ctx.reset(0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(ctx.stream)
        ctx.prefill(prompt)
        e1.record(ctx.stream)
        e1.synchronize()
        if i:
            ts.append(e0.elapsed_time(e1))
    return statistics.median(ts)


if __name__ == "__main__":
    try:
        rc = main()
    finally:
        # contexts are destroyed while the HIP runtime is up, also after an error
        _hta = sys.modules.get("autoregressive_codebook_tts_amd.hta")
        if _hta is not None:
            _hta.close_all()
    if rc:  # a clean run returns from the script instead of raising SystemExit
        sys.exit(rc)
