#!/usr/bin/env python3
"""Benchmark of the KV-cached GQA decoder hot path on one MI355X.

One step is one frame step of the Qwen2.5-1.5B-shaped decoder (28 layers,
hidden 1536, 12 query heads, 2 KV heads, head dim 128, SwiGLU 8960, vocab
151936, bf16) with a 1024-token context already cached in 16-token blocks:

  1. roll the cache back to the 1024-token context (host bookkeeping only);
  2. prefill a 256-token visual chunk (N(0,1) embeddings, resident in HBM);
  3. 16 greedy decode steps (each returns its next token to the host);
  4. score the resident frames on layer 0 (fp64 mean keys, all-pairs cosine).

Printed: one JSON line. ``value`` is the prefill throughput in tokens/s
(HIP events around the prefill calls of the timed steps); ``ms_per_step`` is
the wall time of a whole frame step. ``phases`` holds the decode-step latency,
the frame-step time, the eviction leg (semantic eviction workload: 128 cached
frames of 64 tokens, 32 score-and-evict cycles each followed by a 64-token
prefill), the long-context leg (Llama-3-8B-shaped decoder with INT4 group-128
weights: a 120,000-token cached prefix, a 512-token chunk, 32 decodes), the
pi0-style policy leg (Gemma-2B-shaped prefix model over 512 image tokens, then
10 Euler steps of the 300M action expert on a 63-token chunk) and roofline
fractions. ``roofline`` covers the dominant kernel of the frame step
(the decode gate/up projection); ``cpu_baseline`` times the CPU oracle on a
bounded sample of the same prefill.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                       [--no-eviction] [--no-longctx] [--no-pi0]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill tok/s + decode ms/step at Qwen2.5-1.5B shape; % MFMA/HBM peak"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published

# Qwen2.5-1.5B-shaped decoder
L, H, HQ, HKV, D, F, V = 28, 1536, 12, 2, 128, 8960, 151936
CONTEXT, CHUNK, DECODES = 1024, 256, 16


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic work (weights-only GEMM traffic plus KV reads; FLOPs of the GEMMs
# and the attention products)
# ---------------------------------------------------------------------------
def layer_weight_params():
    return (HQ + 2 * HKV) * D * H + H * HQ * D + 2 * F * H + H * F


def prefill_flops(n=CHUNK, ctx=CONTEXT):
    lin = 2 * n * layer_weight_params() * L + 2 * V * H          # last row through W_Y
    # q.k and p.v over the visible keys: ctx + causal part of the chunk
    keys = n * ctx + n * (n + 1) // 2
    attn = L * HQ * 2 * 2 * D * keys
    return lin + attn


def decode_bytes(ctx_tokens):
    w = 2 * (layer_weight_params() * L + V * H)
    kv = L * 2 * HKV * D * 2 * ctx_tokens
    return w + kv


def gateup_bytes():
    # the decode gate/up projection: both weight matrices, the input row, the gated output
    return 2 * F * H * 2 + H * 2 + F * 2


# the sources the decode gate/up GEMV is built from (its own file, the one-shot body,
# the shared device helpers, the epilogues, the argument structs)
GEMV_SOURCES = ("gemv.hip", "gemv_body.hpp", "common.hpp", "epilogue.hpp", "kernels.hpp")


def file_sha(paths):
    """First 16 hex digits of the SHA-256 of the files' bytes, concatenated in order."""
    h = hashlib.sha256()
    for path in ([paths] if isinstance(paths, str) else paths):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel_src):
    """HBM traffic per launch of the gate/up GEMV from the committed counter summary,
    or None when the summary is missing or any of its kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", "gemv_gateup_qwen1p5b_decode_traffic.txt")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_sha = re.search(r"^kernel_source_sha256_16:\s*(\S+)", txt, re.M)
    m_b = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt, re.M)
    if not m_sha or not m_b or m_sha.group(1) != file_sha(kernel_src):
        return None
    return float(m_b.group(1))


# ---------------------------------------------------------------------------
def gpu_leg(args):
    import numpy as np
    import torch

    import kv_cached_gqa_decoder_amd as vla
    import synth

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    p = vla.PRESETS["c2_qwen1p5b_bf16"]
    log(f"[bench] creating the Qwen2.5-1.5B-shaped model (seed {p['seed']})")
    m = vla.Model(vla.make_config(**p))
    # context: 1024 uniform ids, prefilled untimed in 4 chunks of 256
    ctx_fid = -1
    for c in range(CONTEXT // CHUNK):
        ids = synth.token_ids(p["seed"], c, CHUNK, V)
        ctx_fid = m.prefill_chunk(tokens=ids, stream=sh)
    _, xs = synth.embeddings(p["seed"], 0, CHUNK, H, "bf16")
    chunk = torch.from_numpy(np.ascontiguousarray(xs).view(np.int16)).view(torch.bfloat16).cuda()
    torch.cuda.synchronize()

    def step(ev=None):
        m.kv_rollback(ctx_fid)
        if ev:
            ev[0].record(stream)
        m.prefill_chunk(embeds=chunk, n=CHUNK, stream=sh)
        if ev:
            ev[1].record(stream)
        tok = m.decode_step(1, stream=sh)
        for _ in range(DECODES - 1):
            tok = m.decode_step(tok, stream=sh)
        if ev:
            ev[2].record(stream)
        m.kv_score(0, stream=sh)
        if ev:
            ev[3].record(stream)

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the roofline kernel (decode gate/up GEMV): replayed over the 28 layers' weights
    # back to back between two stream events, on the decode state of the last step
    # (events in each dispatch would lengthen a 12 us kernel by about 1.3 us)
    gu_reps = 8
    gu_avg = m.profile_replay("gemv_gateup", reps=gu_reps, stream=sh)
    gu_n = gu_reps * L
    # the same kernel inside decode steps, with a start/stop event pair carried in each of
    # its dispatches (the events lengthen a 12 us kernel by about 1.3 us)
    m.kv_rollback(ctx_fid)
    m.prefill_chunk(embeds=chunk, n=CHUNK, stream=sh)
    m.profile_enable("gemv_gateup")
    tok = 1
    for _ in range(DECODES):
        tok = m.decode_step(tok, stream=sh)
    gi_ms, gi_n = m.profile_read()
    m.profile_enable(0)
    gu_in_step = gi_ms / max(gi_n, 1)

    pre = [e[0].elapsed_time(e[1]) for e in evs]
    dec = [e[1].elapsed_time(e[2]) / DECODES for e in evs]
    sco = [e[2].elapsed_time(e[3]) for e in evs]
    pre_ms = statistics.mean(pre)
    dec_ms = statistics.mean(dec)

    # per-decode-step latency distribution (separate short pass, events per step)
    m.kv_rollback(ctx_fid)
    m.prefill_chunk(embeds=chunk, n=CHUNK, stream=sh)
    de = [torch.cuda.Event(enable_timing=True) for _ in range(DECODES + 1)]
    tok = 1
    de[0].record(stream)
    for i in range(DECODES):
        tok = m.decode_step(tok, stream=sh)
        de[i + 1].record(stream)
    torch.cuda.synchronize()
    per_dec = [de[i].elapsed_time(de[i + 1]) for i in range(DECODES)]
    # greedy decodes chained on the device (the token never visits the host)
    chained = []
    for _ in range(3):
        m.kv_rollback(ctx_fid)
        m.prefill_chunk(embeds=chunk, n=CHUNK, stream=sh)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(DECODES):
            m.decode_step(vla.VLA_TOKEN_DEVICE, stream=sh, want_token=False)
        e1.record(stream)
        torch.cuda.synchronize()
        chained.append(e0.elapsed_time(e1) / DECODES)
    # the same greedy decodes as one persistent launch per step (phases separated by
    # device-scope barriers), and the latency of such a barrier alone
    m.set_option(vla.VLA_OPT_PERSISTENT_DECODE, 1)
    pers = []
    for _ in range(3):
        m.kv_rollback(ctx_fid)
        m.prefill_chunk(embeds=chunk, n=CHUNK, stream=sh)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(DECODES):
            m.decode_step(vla.VLA_TOKEN_DEVICE, stream=sh, want_token=False)
        e1.record(stream)
        torch.cuda.synchronize()
        pers.append(e0.elapsed_time(e1) / DECODES)
    used_persistent = m.get_option(vla.VLA_INFO_LAST_DECODE_PERSISTENT)
    m.set_option(vla.VLA_OPT_PERSISTENT_DECODE, 0)
    bar_us = {g: round(vla.vla_probe_barrier(g, 200, sh), 2) for g in (64, 256)}
    m.close()
    del chunk
    torch.cuda.synchronize()

    c1 = c1_leg(args)
    peaks = measured_peaks()
    ev_leg = eviction_leg(args) if not args.no_eviction else None
    lc_leg = longctx_leg(args) if not args.no_longctx else None
    p0_leg = pi0_leg(args) if not args.no_pi0 else None
    as_leg = asr_leg(args)

    fl = prefill_flops()
    dbytes = decode_bytes(CONTEXT + CHUNK + DECODES // 2)
    gu_gbs = gateup_bytes() / (gu_avg * 1e-3) / 1e9
    kernel_src = [os.path.join(ROOT, "kv_cached_gqa_decoder_amd", "csrc", f) for f in GEMV_SOURCES]
    traffic = read_traffic(kernel_src)
    res = {
        "metric": METRIC,
        "value": round(CHUNK / (pre_ms * 1e-3), 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init weights N(0,0.02); uniform context ids; "
                "N(0,1) visual-token embeddings)",
        "config": {
            "workload": "Qwen2.5-1.5B-shaped GQA decoder frame step: 1024-token cached context, "
                        "256-token visual-chunk prefill, 16 greedy decode steps, layer-0 frame "
                        "scoring; batch 1, 16-token KV blocks",
            "layers": L, "hidden": H, "q_heads": HQ, "kv_heads": HKV, "head_dim": D,
            "ffn": F, "vocab": V, "context": CONTEXT, "chunk": CHUNK, "decode_steps": DECODES,
            "batch": 1, "parallelism": "single GPU",
        },
        "phases": {
            "prefill_ms": round(pre_ms, 4),
            "prefill_tok_s": round(CHUNK / (pre_ms * 1e-3), 1),
            "prefill_mfma_frac": round(fl / (pre_ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4),
            "prefill_flop": fl,
            "decode_ms_per_step": round(dec_ms, 4),
            "decode_ms_per_step_median": round(statistics.median(per_dec), 4),
            "decode_ms_per_step_max": round(max(per_dec), 4),
            "decode_ms_per_step_device_tokens": round(statistics.median(chained), 4),
            "decode_hbm_frac": round(dbytes / (dec_ms * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
            "decode_bytes_per_step": dbytes,
            "frame_step_ms": round(pre_ms + DECODES * dec_ms, 4),
            "frame_budget_ms": 33.0,
            "score_ms": round(statistics.mean(sco), 4),
        },
        "roofline": {
            "kernel": "gemv gate/up + SwiGLU (decode)",
            "bound": "hbm",
            "achieved": round(gu_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gu_gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": gateup_bytes(),
            "avg_launch_us": round(gu_avg * 1e3, 3),
            "launches": gu_n,
            "timing": "replayed back to back over the 28 layers' weights between two stream "
                      "events",
            "in_step_avg_launch_us_with_events": round(gu_in_step * 1e3, 3),
            "in_step_frac_with_events": round(gateup_bytes() / (gu_in_step * 1e-3)
                                              / (PEAK_HBM_GBS * 1e9), 4),
            "measured_peak_copy_gbs": peaks["copy_gbs"],
            "measured_peak_read_gbs": peaks["read_gbs"],
            "frac_of_measured_read_peak": round(gu_gbs / peaks["read_gbs"], 4),
        },
    }
    res["phases"].update(c1)
    res["phases"]["decode_ms_per_step_persistent_kernel"] = (round(statistics.median(pers), 4)
                                                             if used_persistent else None)
    res["phases"]["device_barrier_us_64_workgroups"] = bar_us[64]
    res["phases"]["device_barrier_us_256_workgroups"] = bar_us[256]
    res["phases"]["measured_peak_copy_gbs"] = peaks["copy_gbs"]
    res["phases"]["measured_peak_read_gbs"] = peaks["read_gbs"]
    res["phases"]["measured_peak_mfma_bf16_tflops"] = peaks["mfma_bf16_tflops"]
    res["phases"]["prefill_frac_of_measured_mfma_peak"] = round(
        fl / (pre_ms * 1e-3) / (peaks["mfma_bf16_tflops"] * 1e12), 4)
    res["phases"]["decode_frac_of_measured_read_peak"] = round(
        dbytes / (dec_ms * 1e-3) / (peaks["read_gbs"] * 1e9), 4)
    if ev_leg:
        res["phases"].update(ev_leg)
    if lc_leg:
        res["phases"].update(lc_leg)
    if p0_leg:
        res["phases"].update(p0_leg)
    res["phases"].update(as_leg)
    return res


def frame_leg(args):
    """The Qwen2.5-1.5B-shaped frame step alone (for kernel traces and counter passes):
    the 1024-token context, then per step a 256-token chunk prefill, 16 greedy decodes
    and the layer-0 frame scoring; prints the median phase times."""
    import numpy as np
    import torch

    import kv_cached_gqa_decoder_amd as vla
    import synth

    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    p = vla.PRESETS["c2_qwen1p5b_bf16"]
    m = vla.Model(vla.make_config(**p))
    ctx_fid = -1
    for c in range(CONTEXT // CHUNK):
        ctx_fid = m.prefill_chunk(tokens=synth.token_ids(p["seed"], c, CHUNK, V), stream=sh)
    _, xs = synth.embeddings(p["seed"], 0, CHUNK, H, "bf16")
    chunk = torch.from_numpy(np.ascontiguousarray(xs).view(np.int16)).view(torch.bfloat16).cuda()
    evs = []
    for i in range(args.warmup + args.steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        m.kv_rollback(ctx_fid)
        ev[0].record(stream)
        m.prefill_chunk(embeds=chunk, n=CHUNK, stream=sh)
        ev[1].record(stream)
        tok = m.decode_step(1, stream=sh)
        for _ in range(DECODES - 1):
            tok = m.decode_step(tok, stream=sh)
        ev[2].record(stream)
        m.kv_score(0, stream=sh)
        ev[3].record(stream)
        if i >= args.warmup:
            evs.append(ev)
    torch.cuda.synchronize()
    m.close()
    med = lambda a, b: round(statistics.median(e[a].elapsed_time(e[b]) for e in evs), 4)
    return {"prefill_ms": med(0, 1), "decode_ms_per_step": round(med(1, 2) / DECODES, 4),
            "score_ms": med(2, 3)}


def asr_leg(args):
    """Reconciliation on a second state at the Qwen2.5-1.5B shape: 5 frames of 256 ids
    through the reconciler, one all-pairs eviction, then the spare re-prefills the 4 kept
    frames (1,024 tokens) on its own stream while the serving model prefills a new
    256-token frame; times: the reconciliation (begin to swap), and the serving prefill
    alone and during the reconciliation (events on the caller's stream)."""
    import torch

    import kv_cached_gqa_decoder_amd as vla
    import synth

    stream = torch.cuda.current_stream()
    p = vla.PRESETS["c2_qwen1p5b_bf16"]
    m = vla.Model(vla.make_config(**p))
    ids = [synth.token_ids(p["seed"], 100 + i, CHUNK, V) for i in range(8)]
    rows = {"alone": [], "during": [], "reconcile": []}
    for rep in range(3):
        rec = vla.Reconciler(m)
        for i in range(5):
            rec.prefill(tokens=ids[i], stream=stream)
        rec.evict("semantic", 0, stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rec.prefill(tokens=ids[5], stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        rows["alone"].append(e0.elapsed_time(e1))
        rec.evict("fifo", 0, stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        rec.begin(stream)
        e0.record(stream)
        rec.prefill(tokens=ids[6], stream=stream)
        e1.record(stream)
        while not rec.try_swap(stream):
            time.sleep(0.0002)
        torch.cuda.synchronize()
        rows["reconcile"].append((time.perf_counter() - t0) * 1e3)
        rows["during"].append(e0.elapsed_time(e1))
        rec.close()
        m.kv_rollback(-1)
    m.close()
    med = lambda k: round(statistics.median(rows[k]), 3)
    return {"asr_reconcile_ms_5_frames_1280_tokens": med("reconcile"),
            "asr_serving_prefill_ms_alone": med("alone"),
            "asr_serving_prefill_ms_during_reconcile": med("during")}


def eviction_leg(args):
    """Semantic eviction workload: 128 raw frames of 64 tokens (layer-0 keys clustered
    around 16 centres, sigma 0.1), 512-block budget, 32 cycles of score-and-evict followed
    by a 64-token prefill of N(0,1) embeddings; plus a full mean-key refresh."""
    import numpy as np
    import torch

    import kv_cached_gqa_decoder_amd as vla
    import synth

    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    p = vla.PRESETS["c3_semantic_eviction"]
    log("[bench] eviction leg: creating the model and 128 raw frames")
    m = vla.Model(vla.make_config(**p))
    raw = []
    for f in range(128):
        _, (ks, vs) = synth.clustered_frame(p["seed"], f, L, 64, HKV, D)
        kt = torch.from_numpy(ks.view(np.int16)).view(torch.bfloat16).cuda()
        vt = torch.from_numpy(vs.view(np.int16)).view(torch.bfloat16).cuda()
        raw.append((kt, vt))
        m.kv_append_raw(kt, vt, 64, stream=sh)
    embeds = []
    for c in range(32):
        _, xs = synth.embeddings(p["seed"], c, 64, H, "bf16")
        embeds.append(torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16).cuda())
    torch.cuda.synchronize()
    sc_us, pf_ms = [], []
    for c in range(32):
        t0 = time.perf_counter()
        m.kv_score_and_evict(0, stream=sh)          # synchronises (returns the frame id)
        sc_us.append((time.perf_counter() - t0) * 1e6)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        m.prefill_chunk(embeds=embeds[c], n=64, stream=sh)
        e1.record(stream)
        torch.cuda.synchronize()
        pf_ms.append(e0.elapsed_time(e1))
    # device time of the scoring kernels alone
    m.profile_enable("score")
    for _ in range(10):
        m.kv_score(0, stream=sh)
    s_ms, s_n = m.profile_read()
    # full refresh of every frame's mean keys on all 28 layers (reads the whole key cache)
    m.profile_enable("meankeys")
    for _ in range(5):
        m.kv_refresh_mean_keys(stream=sh)
    r_ms, r_n = m.profile_read()
    m.profile_enable(0)
    # the same 32 insert cycles under each eviction policy (evict-until-room, then the
    # 64-token prefill): time per call, and how the 16 clusters' 8 frames each fare
    ab = {}
    for policy in ("semantic", "adjacent", "fifo"):
        m.kv_rollback(-1)
        for kt, vt in raw:
            m.kv_append_raw(kt, vt, 64, stream=sh)
        torch.cuda.synchronize()
        t_us = []
        for c in range(32):
            torch.cuda.synchronize()       # the previous cycle's prefill is not timed here
            t0 = time.perf_counter()
            m.kv_make_room(policy, 64, stream=sh)
            t_us.append((time.perf_counter() - t0) * 1e6)
            m.prefill_chunk(embeds=embeds[c], n=64, stream=sh)
        torch.cuda.synchronize()
        kept = [int(f) for f in m.frames() if f < 128]
        per = [sum(1 for f in kept if f % 16 == k) for k in range(16)]
        ab[policy] = {"make_room_us_median": round(statistics.median(t_us), 2),
                      "raw_frames_kept_per_cluster_min": min(per),
                      "raw_frames_kept_per_cluster_max": max(per),
                      "max_similarity_left": round(m.kv_score(0, stream=sh)[1], 9)}
    m.close()
    torch.cuda.synchronize()
    refresh_bytes = L * 128 * 64 * HKV * D * 2
    r_avg = r_ms / max(r_n, 1)
    return {
        "eviction_policy_ab": ab,
        "evict_score_us_median": round(statistics.median(sc_us), 2),
        "evict_score_kernel_us": round(s_ms / max(s_n, 1) * 1e3, 2),
        "evict_cycle_prefill64_ms_median": round(statistics.median(pf_ms), 4),
        "meankey_refresh_us": round(r_avg * 1e3, 2),
        "meankey_refresh_gbs": round(refresh_bytes / (r_avg * 1e-3) / 1e9, 1),
        "meankey_refresh_hbm_frac": round(refresh_bytes / (r_avg * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
    }


# ---------------------------------------------------------------------------
def c1_leg(args):
    """The fp32 tiny decoder (2 layers, hidden 256, 4/2 heads, head dim 64, FFN 688, vocab
    1024): a 64-token prompt of uniform ids prefilled, then 16 greedy decodes; median over
    repeats (rolled back between them)."""
    import torch

    import kv_cached_gqa_decoder_amd as vla
    import synth

    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    p = vla.PRESETS["c1_tiny_f32"]
    m = vla.Model(vla.make_config(**p))
    ids = synth.token_ids(p["seed"], 0, 64, p["vocab"])

    def run(ev=None):
        m.kv_rollback(-1)
        if ev:
            ev[0].record(stream)
        m.prefill_chunk(tokens=ids, stream=sh)
        if ev:
            ev[1].record(stream)
        tok = m.decode_step(1, stream=sh)
        for _ in range(15):
            tok = m.decode_step(tok, stream=sh)
        if ev:
            ev[2].record(stream)

    for _ in range(3):
        run()
    reps = max(10, args.steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for i in range(reps):
        run(evs[i])
    torch.cuda.synchronize()
    m.close()
    return {
        "c1_prefill_ms": round(statistics.median(e[0].elapsed_time(e[1]) for e in evs), 4),
        "c1_decode_ms_per_step": round(statistics.median(e[1].elapsed_time(e[2]) / 16
                                                         for e in evs), 4),
    }


def measured_peaks():
    """This box's measured ceilings beside the published ones: a 1 GiB device-to-device
    copy (read + write bytes) and a register-only bf16 MFMA loop."""
    import torch

    import kv_cached_gqa_decoder_amd as vla

    stream = torch.cuda.current_stream()
    a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1.0)
    b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        b.copy_(a)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * a.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    # a streaming read of 1 GiB (16-byte loads, 8 in flight per thread)
    read_gbs = vla.vla_probe_read_bandwidth(1 << 30, 5, stream.cuda_stream)
    out = torch.empty(4096, dtype=torch.float32, device="cuda")
    tf = vla.vla_probe_mfma_peak(out, 4096, 2000, stream.cuda_stream)
    return {"copy_gbs": round(copy_gbs, 1), "read_gbs": round(read_gbs, 1),
            "mfma_bf16_tflops": round(tf, 1)}


# ---------------------------------------------------------------------------
# Llama-3-8B-shaped long-context workload: INT4 group-128 weights, bf16 activations
C5_L, C5_H, C5_HQ, C5_HKV, C5_D, C5_F, C5_V = 32, 4096, 32, 8, 128, 14336, 128256
C5_PREFIX, C5_CHUNK, C5_DECODES, C5_FRAME = 120000, 512, 32, 512


def c5_layer_params():
    return (C5_HQ + 2 * C5_HKV) * C5_D * C5_H + C5_H * C5_HQ * C5_D + 3 * C5_F * C5_H


def c5_prefill_flops():
    lin = 2 * C5_CHUNK * c5_layer_params() * C5_L + 2 * C5_V * C5_H
    keys = C5_CHUNK * C5_PREFIX + C5_CHUNK * (C5_CHUNK + 1) // 2
    return lin, C5_L * C5_HQ * 2 * 2 * C5_D * keys


def c5_kv_bytes_per_token():
    return C5_L * 2 * C5_HKV * C5_D * 2


def c5_decode_bytes(ctx_tokens):
    int4 = lambda n: n // 2 + n // 128 * 2      # codes + one fp16 scale per 128
    w = int4(c5_layer_params()) * C5_L + int4(C5_V * C5_H) + C5_H * 2
    return w + c5_kv_bytes_per_token() * ctx_tokens


def longctx_leg(args):
    """120,000-token cached prefix (raw bf16 K/V ~ N(0,1) per layer, appended as frames of
    512 tokens), a 512-token chunk of uniform ids, then 32 greedy decodes."""
    import torch

    import kv_cached_gqa_decoder_amd as vla
    import synth

    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    p = vla.PRESETS["c5_llama3_8b_int4"]
    log("[bench] long-context leg: creating the Llama-3-8B-shaped INT4 model")
    m = vla.Model(vla.make_config(**p))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(p["seed"])
    done, fid = 0, -1
    while done < C5_PREFIX:
        n = min(C5_FRAME, C5_PREFIX - done)
        shape = (C5_L, n, C5_HKV, C5_D)
        k = torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16)
        v = torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16)
        fid = m.kv_append_raw(k, v, n, stream=sh)
        done += n
    del k, v
    ids = synth.token_ids(p["seed"], 0, C5_CHUNK, C5_V)
    torch.cuda.synchronize()
    log(f"[bench] long-context leg: {done}-token prefix resident in {fid + 1} frames")

    def run(ev=None):
        m.kv_rollback(fid)
        if ev:
            ev[0].record(stream)
        m.prefill_chunk(tokens=ids, stream=sh)
        if ev:
            ev[1].record(stream)
        tok = m.decode_step(1, stream=sh)
        for _ in range(C5_DECODES - 1):
            tok = m.decode_step(tok, stream=sh)
        if ev:
            ev[2].record(stream)

    run()
    torch.cuda.synchronize()
    reps = max(2, min(args.steps, 4))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for i in range(reps):
        run(evs[i])
    torch.cuda.synchronize()
    pre_ms = statistics.median(e[0].elapsed_time(e[1]) for e in evs)
    dec_ms = statistics.median(e[1].elapsed_time(e[2]) / C5_DECODES for e in evs)
    # kernel time of the attention alone (split pass + merge), prefill then decode
    m.kv_rollback(fid)
    m.profile_enable("attn_prefill")
    m.prefill_chunk(tokens=ids, stream=sh)
    ap_ms, ap_n = m.profile_read()
    m.profile_enable("attn_decode")
    tok = m.decode_step(1, stream=sh)
    for _ in range(C5_DECODES - 1):
        tok = m.decode_step(tok, stream=sh)
    ad_ms, ad_n = m.profile_read()
    m.profile_enable(0)
    m.close()
    torch.cuda.synchronize()

    lin, attn = c5_prefill_flops()
    ctx_mid = C5_PREFIX + C5_CHUNK + C5_DECODES // 2
    dbytes = c5_decode_bytes(ctx_mid)
    attn_layer_bytes = 2 * C5_HKV * C5_D * 2 * ctx_mid        # K and V of one layer
    ad_avg = ad_ms / max(ad_n, 1)
    return {
        "longctx_prefill_ms": round(pre_ms, 3),
        "longctx_prefill_tok_s": round(C5_CHUNK / (pre_ms * 1e-3), 1),
        "longctx_prefill_flop": lin + attn,
        "longctx_prefill_mfma_frac": round((lin + attn) / (pre_ms * 1e-3)
                                           / (PEAK_BF16_TFLOPS * 1e12), 4),
        "longctx_prefill_attention_ms": round(ap_ms, 3),
        "longctx_prefill_attention_mfma_frac": round(attn / (ap_ms * 1e-3)
                                                     / (PEAK_BF16_TFLOPS * 1e12), 4),
        "longctx_decode_ms_per_step": round(dec_ms, 4),
        "longctx_decode_bytes_per_step": dbytes,
        "longctx_decode_hbm_frac": round(dbytes / (dec_ms * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
        "longctx_decode_attention_us_per_layer": round(ad_avg * 1e3, 2),
        "longctx_decode_attention_hbm_frac": round(attn_layer_bytes / (ad_avg * 1e-3)
                                                   / (PEAK_HBM_GBS * 1e9), 4),
    }


# ---------------------------------------------------------------------------
# pi0-style policy step: Gemma-2B-shaped prefix model + 300M action expert, bf16
P0_L, P0_H, P0_HQ, P0_D, P0_F = 18, 2048, 8, 256, 16384       # prefix (17 + K/V-only 18th)
AE_H, AE_F, AE_N, AE_STEPS = 1024, 4096, 63, 10
P0_PREFIX = 512                                                  # 2 views x 256 image tokens


def pi0_prefix_flops():
    qkv = (P0_HQ + 2) * P0_D * P0_H
    full = qkv + P0_H * P0_HQ * P0_D + 3 * P0_F * P0_H
    lin = 2 * P0_PREFIX * (full * (P0_L - 1) + 2 * P0_D * P0_H)     # 18th layer: K/V only
    attn = (P0_L - 1) * P0_HQ * 2 * 2 * P0_D * (P0_PREFIX * (P0_PREFIX + 1) // 2)
    return lin + attn


def pi0_expert_bytes():
    per = (P0_HQ + 2) * P0_D * AE_H + AE_H * P0_HQ * P0_D + 3 * AE_F * AE_H
    return 2 * per * P0_L


def pi0_leg(args):
    """Prefill 2 x 256 image-token embeddings (N(0,1)) into the prefix model, then
    10 Euler steps of the action expert on a 63-token N(0,1) chunk."""
    import numpy as np
    import torch

    import kv_cached_gqa_decoder_amd as vla
    import synth

    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    vp = vla.PRESETS["c4_pi0_vlm"]
    ap = vla.PRESETS["c4_pi0_action_expert"]
    log("[bench] pi0 leg: creating the prefix model and the action expert")
    m = vla.Model(vla.make_config(**vp))
    e = vla.Expert(m, vla.make_config(**ap), AE_N)
    _, xs = synth.embeddings(vp["seed"], 0, P0_PREFIX, P0_H, "bf16")
    img = torch.from_numpy(np.ascontiguousarray(xs).view(np.int16)).view(torch.bfloat16).cuda()
    noise = torch.from_numpy(synth.action_noise(vp["seed"], 0, AE_N, AE_H)).cuda()
    x = torch.empty_like(noise)

    def step(ev=None):
        m.kv_rollback(-1)
        x.copy_(noise)
        if ev:
            ev[0].record(stream)
        m.prefill_chunk(embeds=img, n=P0_PREFIX, stream=sh)
        if ev:
            ev[1].record(stream)
        e.denoise(x, n_steps=AE_STEPS, stream=sh)
        if ev:
            ev[2].record(stream)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    reps = max(5, args.steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for i in range(reps):
        step(evs[i])
    torch.cuda.synchronize()
    # the same frames through the overlapped prefix / expert streams: frame t's prefill
    # beside the expert's run on the newest finished prefix; wall time per frame with
    # 1 and 2 expert runs per frame, and sequentially on one stream for comparison
    pl = None

    def frames(n, acts, piped):
        t0 = time.perf_counter()
        for _ in range(n):
            if piped:
                pl.prefill(img, P0_PREFIX, stream)
            else:
                m.kv_rollback(-1)
                m.prefill_chunk(embeds=img, n=P0_PREFIX, stream=sh)
            for _ in range(acts):
                x.copy_(noise)
                if piped:
                    pl.act(x, n_steps=AE_STEPS, stream=stream)
                else:
                    e.denoise(x, n_steps=AE_STEPS, stream=sh)
        if piped:
            pl.sync()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / n

    overlap = {}
    for acts in (() if getattr(args, "no_overlap", False) else (1, 2)):
        overlap[f"{acts}_runs_per_frame"] = {
            "one_stream_ms_per_frame": round(statistics.median(frames(8, acts, False)
                                                               for _ in range(3)), 3)}
    pl = vla.Pipeline(m, e)  # (the pair is used only through the pipeline from here)
    for acts in (() if getattr(args, "no_overlap", False) else (1, 2)):
        frames(2, acts, True)
        overlap[f"{acts}_runs_per_frame"]["overlapped_ms_per_frame"] = round(
            statistics.median(frames(8, acts, True) for _ in range(3)), 3)
    overlap["runs_on_older_prefix"] = pl.stats()["acts_on_older"]
    overlap["runs"] = pl.stats()["acts"]
    pl.close()
    e.close()
    m.close()
    pre = statistics.median(ev[0].elapsed_time(ev[1]) for ev in evs)
    ae = statistics.median(ev[1].elapsed_time(ev[2]) for ev in evs)
    fl = pi0_prefix_flops()
    ab = pi0_expert_bytes()
    it = ae / AE_STEPS
    return {
        "pi0_overlapped_streams": overlap,
        "pi0_step_ms": round(pre + ae, 3),
        "pi0_prefix_prefill_ms": round(pre, 3),
        "pi0_prefix_prefill_mfma_frac": round(fl / (pre * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4),
        "pi0_prefix_prefill_flop": fl,
        "pi0_expert_iteration_ms": round(it, 4),
        "pi0_expert_iteration_hbm_frac": round(ab / (it * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
        "pi0_expert_weight_bytes": ab,
    }


# ---------------------------------------------------------------------------
def _vm_hwm_kib():
    try:
        for ln in open("/proc/self/status"):
            if ln.startswith("VmHWM:"):
                return int(ln.split()[1])
    except OSError:
        pass
    return None


def cpu_baseline(layers_sample: int):
    """The oracle (fp64 numpy) on the host cores, per phase, on bounded samples of the
    same workloads: the Qwen2.5-1.5B-shaped 256-token chunk prefill over the 1024-token
    context through the first `layers_sample` of the 28 layers plus the output head (the
    reported value, scaled per layer to 28 layers), two decode steps after it, one
    scoring cycle over 128 clustered frames, and the fp32 tiny decoder's prompt and
    decode steps; the scoring cycle and the tiny decoder also on one thread. The BLAS
    thread count is set to the cores this process may run on; peak host memory is
    VmHWM."""
    import numpy as np

    import synth
    from oracle import decoder as D_
    from oracle import rng

    if not rng.have_c():
        from oracle import build as ob
        ob.build()
    cores = len(os.sched_getaffinity(0))
    try:
        import threadpoolctl
        limit = threadpoolctl.threadpool_limits
    except Exception:            # no control over the BLAS threads: report the default
        limit = None
    ctx = limit(cores) if limit else None
    log(f"[bench] cpu baseline: oracle, {layers_sample} of {L} layers, {cores} cores")
    cfg = D_.C2.with_(n_layers=layers_sample)
    sess = D_.Session(cfg)
    for c in range(CONTEXT // CHUNK):
        sess.prefill_chunk(tokens=synth.token_ids(cfg.seed, c, CHUNK, V))
    x32, _ = synth.embeddings(cfg.seed, 0, CHUNK, H, "bf16")
    ctx_fid = sess.frames()[-1].frame_id
    runs = []
    for _ in range(3):
        sess.rollback(ctx_fid)
        t0 = time.perf_counter()
        _, ref = sess.prefill_chunk(embeds=x32)
        runs.append(time.perf_counter() - t0)
    t_all = statistics.median(runs)
    h = np.asarray(x32[-1], dtype=np.float64)
    t0 = time.perf_counter()
    sess._logits(h)
    t_head = time.perf_counter() - t0
    per_layer = (t_all - t_head) / layers_sample
    est = per_layer * L + t_head
    dec = []
    tok = int(np.argmax(ref))
    for _ in range(2):
        t0 = time.perf_counter()
        tok, _ = sess.decode_step(tok)
        dec.append(time.perf_counter() - t0)
    # per-layer part scaled to 28 layers, the output head once
    dec_ms = ((statistics.median(dec) - t_head) / layers_sample * L + t_head) * 1e3
    del sess

    def scoring_cycle():
        c3 = D_.C3.with_(n_layers=1)
        s3 = D_.Session(c3)
        for f in range(128):
            (k32, v32), _ = synth.clustered_frame(c3.seed, f, 1, 64, HKV, D)
            s3.append_raw(k32, v32)
        t = []
        for _ in range(3):
            t0 = time.perf_counter()
            s3.score(0)
            t.append(time.perf_counter() - t0)
        return statistics.median(t) * 1e3

    w1 = D_.Weights(D_.C1)
    ids1 = synth.token_ids(D_.C1.seed, 0, 64, D_.C1.vocab)
    D_.Session(D_.C1, w1).prefill_chunk(tokens=ids1)     # generates the weights (untimed)

    def tiny():
        s1 = D_.Session(D_.C1, w1)
        ids = ids1
        t0 = time.perf_counter()
        _, r = s1.prefill_chunk(tokens=ids)
        tp = time.perf_counter() - t0
        tok1 = int(np.argmax(r))
        t0 = time.perf_counter()
        for _ in range(16):
            tok1, _ = s1.decode_step(tok1)
        return tp * 1e3, (time.perf_counter() - t0) / 16 * 1e3

    score_ms = scoring_cycle()
    c1_pre, c1_dec = tiny()
    if ctx is not None:
        ctx.restore_original_limits()
    one = limit(1) if limit else None
    score_ms_1t = scoring_cycle()
    c1_pre_1t, c1_dec_1t = tiny()
    if one is not None:
        one.restore_original_limits()
    return {
        "value": round(CHUNK / est, 3),
        "unit": "tok/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"256-token chunk prefill over a 1024-token cached context through "
                  f"{layers_sample} of {L} layers plus the output head (median of 3: "
                  f"{t_all:.2f} s); scaled per layer to {L} layers: est. {est:.2f} s",
        "phases_ms": {
            "qwen_prefill_256": round(est * 1e3, 1),
            "qwen_decode_step": round(dec_ms, 1),
            "scoring_cycle_128_frames": round(score_ms, 2),
            "scoring_cycle_128_frames_1_thread": round(score_ms_1t, 2),
            "tiny_f32_prefill_64": round(c1_pre, 2),
            "tiny_f32_decode_step": round(c1_dec, 2),
            "tiny_f32_prefill_64_1_thread": round(c1_pre_1t, 2),
            "tiny_f32_decode_step_1_thread": round(c1_dec_1t, 2),
        },
        "host_peak_rss_mib": round(_vm_hwm_kib() / 1024, 1) if _vm_hwm_kib() else None,
        "blas_threads": cores if limit else "default",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-eviction", action="store_true")
    ap.add_argument("--no-longctx", action="store_true")
    ap.add_argument("--no-pi0", action="store_true")
    ap.add_argument("--no-overlap", action="store_true",
                    help="pi0 leg: skip the overlapped-stream comparison (short profiling runs)")
    ap.add_argument("--cpu-layers", type=int, default=28)
    ap.add_argument("--only", choices=["frame", "eviction", "longctx", "pi0", "asr"],
                    help="run one leg alone and print its numbers (for kernel traces)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first copy 256 MiB on the device three times (a plain copy of known "
                         "size, the reference for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decoder's hot path here runs on a single "
              "MI355X (no multi-GPU path is built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        import torch
        a = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    if args.only:
        leg = {"frame": frame_leg, "eviction": eviction_leg, "longctx": longctx_leg,
               "pi0": pi0_leg, "asr": asr_leg}[args.only]
        print(json.dumps(leg(args)), flush=True)
        return
    res = gpu_leg(args)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args.cpu_layers)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
