"""Throughput of the LFM3-1.7B forward pass on one MI355X, through the C ABI.

Headline (one JSON line on stdout): decode tokens/s at batch 1 on the 24-layer geometry with 4-bit
g64 weights -- a step is one whole job: a 2048-token prompt prefilled in one 2048-row pass, then
256 greedy decode steps; value = decode tokens / decode time over the timed steps. The same line
carries the 2048-token prefill rate, the 8-stream decode, the 8192-token prefill (warm, and the
first pass of a fresh context) and the other weight schemes (extras), the roofline figure of the
dominant kernel (the dequant-GEMV: algorithmic bytes per launch over its event-timed launch
duration, with the HBM bytes of the committed counter record), the prefill's MfmaUtil from the
committed counter record, the NVFP4 layout's decode and prefill, and the float64 oracle timed on
the host cores (cpu_baseline). --profile-only, --profile-8stream and --profile-prefill run one short
job each for profiler runs.

Inputs are seeded and synthetic (random-init weights quantized from N(0, 0.02), token ids uniform
in [0, 128000)); they are resident in HBM before the timed region starts.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--prompt", type=int, default=2048)
    ap.add_argument("--decode", type=int, default=256)
    ap.add_argument("--no-extras", action="store_true", help="skip the 8-stream decode and 8k prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-steps", type=int, default=16, help="oracle decode steps timed for cpu_baseline")
    ap.add_argument("--profile-only", action="store_true", help="one short step for rocprofv3 runs")
    ap.add_argument("--profile-prefill", action="store_true",
                    help="one 8192-token prefill in 2048-row passes, for rocprofv3 runs")
    ap.add_argument("--profile-8stream", action="store_true",
                    help="the 8-stream job (prompts U[300, 2960], then 16 greedy steps at B = 8), for rocprofv3 runs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="with --profile-only: also run three 256 MiB device copies (the reference kernel that "
                         "scales rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; multi-GPU sharding is described in DESIGN.md, not built",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    from attention_decoder_amd import synth
    from attention_decoder_amd.lfm3 import Engine

    cfg = synth.full_config(bits=4, group=64, max_slots=8, max_ctx=8704, max_chunk=2048)
    t0 = time.time()
    blob = synth.cached_blob(cfg, seed=0)
    log(f"blob {len(blob) / 1e9:.3f} GB in {time.time() - t0:.1f}s")
    eng = Engine(cfg, blob)
    dev = torch.device("cuda:0")
    prompt = torch.from_numpy(synth.prompt_tokens(2, args.prompt)).to(dev)
    # device-side greedy loop: the id of step t feeds step t + 1 without a host sync
    ids = torch.empty((args.decode + 1,), dtype=torch.int32, device=dev)
    stream = eng.stream

    def job(timing=None):
        eng.reset(0)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e2 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        out = eng.prefill(0, tokens=prompt, logits=False, argmax=True)
        ids[0:1].copy_(out["argmax"])
        e1.record(stream)
        for t in range(args.decode):
            eng.decode([0], tokens=ids[t:t + 1], logits=False, argmax=True,
                       out={"argmax": ids[t + 1:t + 2]})
        e2.record(stream)
        if timing is not None:
            timing.append((e0, e1, e2))

    if args.profile_prefill:
        toks = torch.from_numpy(synth.prompt_tokens(5, 8192)).to(dev)
        eng.reset(0)
        eng.prefill(0, tokens=toks, logits=True, argmax=True)
        torch.cuda.synchronize()
        log("profile-prefill step done")
        return

    if args.profile_8stream:
        lens = synth.stream_prompt_lengths(4, 8)
        prompts = synth.stream_prompts(4, lens)
        for i in range(8):
            eng.reset(i)
            eng.prefill(i, tokens=torch.from_numpy(prompts[i]).to(dev), logits=False, argmax=False)
        sid = torch.empty((17, 8), dtype=torch.int32, device=dev)
        sid[0] = torch.from_numpy(np.array([p[-1] for p in prompts], dtype=np.int32)).to(dev)
        for t in range(16):
            eng.decode(list(range(8)), tokens=sid[t], logits=False, argmax=True, out={"argmax": sid[t + 1]})
        torch.cuda.synchronize()
        log("profile-8stream job done")
        return

    if args.profile_only:
        args.decode = min(args.decode, 32)
        job()
        torch.cuda.synchronize()
        if args.copy_calibration:
            src = torch.empty((64 << 20,), dtype=torch.float32, device=dev).fill_(1.0)
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
        log("profile-only step done")
        return

    for _ in range(args.warmup):
        job()
    torch.cuda.synchronize()
    log("warmup done")
    timing = []
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for _ in range(args.steps):
        job(timing)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    pre_ms = [a.elapsed_time(b) for a, b, _ in timing]
    dec_ms = [b.elapsed_time(c) for _, b, c in timing]
    decode_tok_s = args.decode * args.steps / (sum(dec_ms) / 1e3)
    prefill_tok_s = args.prompt * args.steps / (sum(pre_ms) / 1e3)
    log(f"decode {decode_tok_s:.1f} tok/s ({np.mean(dec_ms) / args.decode * 1e3:.1f} us/token), "
        f"prefill {args.prompt} {prefill_tok_s:.0f} tok/s ({np.mean(pre_ms):.2f} ms)")

    # roofline of the dominant decode kernel: one more job with event-bracketed launches
    eng.profile(True)
    eng.reset(0)
    out = eng.prefill(0, tokens=prompt, logits=False, argmax=True)
    eng.profile(False)
    eng.profile(True)
    ids[0:1].copy_(out["argmax"])
    for t in range(args.decode):
        eng.decode([0], tokens=ids[t:t + 1], logits=False, argmax=True, out={"argmax": ids[t + 1:t + 2]})
    prof = eng.profile_read()
    eng.profile(False)
    g = prof["gemv"]
    per_launch_bytes = g["bytes"] / g["launches"]
    per_launch_us = g["ms"] * 1e3 / g["launches"]
    achieved = per_launch_bytes / (per_launch_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": "k_gemv (decode dequant-GEMV, all linears + tied head)",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": gemv_traffic(),
                "bytes_per_launch": round(per_launch_bytes), "us_per_launch": round(per_launch_us, 3),
                "launches_per_token": g["launches"] // args.decode}
    breakdown = {k: {"ms_per_token": round(v["ms"] / args.decode, 4), "launches_per_token": v["launches"] / args.decode}
                 for k, v in prof.items() if v["launches"]}
    log(f"decode breakdown per token: {breakdown}")

    extras = {"prefill_2048_tok_s": round(prefill_tok_s, 1)}
    if not args.no_extras:
        extras.update(run_extras(eng, synth, torch, dev))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, blob, args.cpu_steps, args.prompt)

    tokens_per_step = args.decode
    line = {
        "metric": "decode tok/s (1 & 8 streams), prefill tok/s @8k, LFM3-1.7B q4 g64",
        "value": round(decode_tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic (seeded random-init weights, uniform token ids)",
        "config": {"workload": "LFM3-1.7B geometry (24 layers: 13 conv, 6 full, 5 sliding), affine 4-bit g64; "
                               "2048-token prompt in one pass, then 256 greedy decode steps at batch 1",
                   "prompt": args.prompt, "decode_steps": args.decode, "batch": 1, "bits": 4, "group": 64,
                   "tokens_per_step": tokens_per_step},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extras": extras,
        "decode_breakdown": breakdown,
    }
    print(json.dumps(line))
    eng.close()


def committed_record(name):
    """A committed profiles/ record, or None when the kernel sources it was measured on have
    changed since (its source_sha256 over its source_files)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name)
    try:
        with open(path) as f:
            rec = json.load(f)
        h = hashlib.sha256()
        for p in rec["source_files"]:
            with open(os.path.join(ROOT, p), "rb") as f:
                h.update(f.read())
    except (OSError, KeyError, ValueError):
        return None
    return rec if h.hexdigest() == rec.get("source_sha256") else None


def gemv_traffic():
    """HBM bytes per decode GEMV launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE record
    (each counter scaled by a 256 MiB device copy of known size), or None when the kernel sources
    have changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemv_decode_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        h = hashlib.sha256()
        for p in rec["source_files"]:
            with open(os.path.join(ROOT, p), "rb") as f:
                h.update(f.read())
    except (OSError, KeyError, ValueError):
        return None
    if h.hexdigest() != rec.get("source_sha256"):
        return None
    return rec["traffic_bytes_per_launch"]


def decode_8stream(eng, synth, torch, dev):
    """8 concurrent streams: prompts U[300, 2960] (untimed prefill), then 128 greedy steps at B = 8."""
    lens = synth.stream_prompt_lengths(4, 8)
    prompts = synth.stream_prompts(4, lens)
    for i in range(8):
        eng.reset(i)
        eng.prefill(i, tokens=torch.from_numpy(prompts[i]).to(dev), logits=False, argmax=False)
    n_steps = 128
    ids = torch.empty((n_steps + 1, 8), dtype=torch.int32, device=dev)
    ids[0] = torch.from_numpy(np.array([p[-1] for p in prompts], dtype=np.int32)).to(dev)
    slots = list(range(8))
    eng.decode(slots, tokens=ids[0], logits=False, argmax=True, out={"argmax": ids[1]})  # warm
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(eng.stream)
    for t in range(1, n_steps):
        eng.decode(slots, tokens=ids[t], logits=False, argmax=True, out={"argmax": ids[t + 1]})
    e1.record(eng.stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    return round(8 * (n_steps - 1) / (ms / 1e3), 1), [int(x) for x in lens], step_breakdown(eng, slots, ids[n_steps])


def step_breakdown(eng, slots, tokens):
    """Kernel-family milliseconds of one more decode step (library event timing, untimed above)."""
    eng.profile(True)
    eng.decode(slots, tokens=tokens, logits=False, argmax=True)
    prof = eng.profile_read()
    eng.profile(False)
    return {k: round(v["ms"], 4) for k, v in prof.items() if v["launches"]}


def prefill_8k(eng, synth, torch, dev):
    """8192-token prefill in four 2048-row passes (weights resident; median of 3): (tok/s, ms)."""
    toks = torch.from_numpy(synth.prompt_tokens(5, 8192)).to(dev)
    times = []
    for r in range(4):
        eng.reset(0)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(eng.stream)
        eng.prefill(0, tokens=toks, logits=True, argmax=True)
        b.record(eng.stream)
        torch.cuda.synchronize()
        if r > 0:
            times.append(a.elapsed_time(b))
    ms = float(np.median(times))
    return round(8192 / (ms / 1e3), 1), ms, toks


def cold_prefill_8k(synth, torch, dev):
    """The first 8192-token prefill of a freshly created q4 g64 context, to the last row's logits and
    id (weights already copied to HBM and re-tiled at create; caches, TLBs and the new context's
    KV pages cold): the cold time to first token, in ms."""
    from attention_decoder_amd.lfm3 import Engine
    cfg = synth.full_config(bits=4, group=64, max_slots=8, max_ctx=8704, max_chunk=2048)
    e = Engine(cfg, synth.cached_blob(cfg, seed=0))
    toks = torch.from_numpy(synth.prompt_tokens(5, 8192)).to(dev)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(e.stream)
    e.prefill(0, tokens=toks, logits=True, argmax=True)
    b.record(e.stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    e.close()
    return ms


def run_extras(eng, synth, torch, dev, schemes=True):
    from attention_decoder_amd.lfm3 import Engine
    out = {}
    out["decode_8stream_tok_s"], out["decode_8stream_prompt_lengths"], out["decode_8stream_step_breakdown_ms"] = \
        decode_8stream(eng, synth, torch, dev)
    log(f"8-stream decode {out['decode_8stream_tok_s']} tok/s")
    out["prefill_8k_tok_s"], ms, toks = prefill_8k(eng, synth, torch, dev)
    out["prefill_8k_ms"] = round(ms, 3)
    # MFMA fraction of the prefill GEMM on the same workload
    eng.reset(0)
    eng.profile(True)
    eng.prefill(0, tokens=toks, logits=True, argmax=True)
    prof = eng.profile_read()
    eng.profile(False)
    g = prof["gemm"]
    a = prof["attn_prefill"]
    # algorithmic flops only (the library records 2 M N K per linear once, even where the input
    # runs as an fp16 pair in two K passes, and 4 * 128 * heads per visible key for attention)
    tf = g["flops"] / (g["ms"] * 1e-3) / 1e12
    out["prefill_8k_gemm_tflops"] = round(tf, 1)
    out["prefill_8k_gemm_frac_of_f16_peak"] = round(tf / MFMA_F16_PEAK_TFLOPS, 4)
    out["prefill_8k_attn_tflops"] = round(a["flops"] / (a["ms"] * 1e-3) / 1e12, 1) if a["ms"] else None
    out["prefill_8k_breakdown_ms"] = {k: round(v["ms"], 3) for k, v in prof.items() if v["launches"]}
    total_flops = g["flops"] + a["flops"] + 2.0 * 128000 * 2048     # + the last row's tied head
    out["prefill_8k_flops_algorithmic"] = total_flops
    out["prefill_8k_frac_of_f16_peak"] = round(total_flops / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)
    mf = committed_record("prefill_8k_q4g64_mfma.json")
    out["prefill_8k_mfma_util_pct_profile"] = (
        {"gemm": mf["gemm_time_weighted_pct"], "attn_prefill": mf["attn_prefill_time_weighted_pct"]} if mf else None)
    log(f"8k prefill {out['prefill_8k_tok_s']} tok/s ({ms:.2f} ms); {out['prefill_8k_breakdown_ms']}")
    out["prefill_8k_cold_ttft_ms"] = round(cold_prefill_8k(synth, torch, dev), 3)
    log(f"8k prefill, first pass of a fresh context: {out['prefill_8k_cold_ttft_ms']} ms")
    if schemes:
        # the same two workloads at the 8-bit (8 streams) and 6-bit (8k prefill) schemes
        for bits, key in [(8, "q8"), (6, "q6")]:
            cfg = synth.full_config(bits=bits, group=64, max_slots=8, max_ctx=8704, max_chunk=2048)
            e2 = Engine(cfg, synth.cached_blob(cfg, seed=0))
            if bits == 8:
                out["q8_decode_8stream_tok_s"], _, out["q8_decode_8stream_step_breakdown_ms"] = decode_8stream(e2, synth, torch, dev)
                log(f"q8 8-stream decode {out['q8_decode_8stream_tok_s']} tok/s")
            else:
                out["q6_prefill_8k_tok_s"], ms6, _ = prefill_8k(e2, synth, torch, dev)
                log(f"q6 8k prefill {out['q6_prefill_8k_tok_s']} tok/s ({ms6:.2f} ms)")
            e2.close()
        out.update(cfg5_extras(synth, torch, dev))
        out.update(nvfp4_extras(synth, torch, dev))
    return out


def nvfp4_extras(synth, torch, dev):
    """The NVFP4 export's layout (FFN NVFP4, mixers / embedding / head bf16): B = 1 decode on the
    headline job's shape (2048-token prompt, 128 greedy steps), the 8-stream decode and the 8k
    prefill."""
    from attention_decoder_amd.lfm3 import Engine
    out = {}
    cfg = synth.nvfp4_config(max_slots=8, max_ctx=8704, max_chunk=2048)
    eng = Engine(cfg, synth.cached_blob(cfg, seed=0))
    prompt = torch.from_numpy(synth.prompt_tokens(2, 2048)).to(dev)
    ids = torch.empty((129,), dtype=torch.int32, device=dev)
    best = 0.0
    for _ in range(2):
        eng.reset(0)
        o = eng.prefill(0, tokens=prompt, logits=False, argmax=True)
        ids[0:1].copy_(o["argmax"])
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(eng.stream)
        for t in range(128):
            eng.decode([0], tokens=ids[t:t + 1], logits=False, argmax=True, out={"argmax": ids[t + 1:t + 2]})
        b.record(eng.stream)
        torch.cuda.synchronize()
        best = max(best, 128 / (a.elapsed_time(b) / 1e3))
    out["nvfp4_decode_b1_tok_s"] = round(best, 1)
    out["nvfp4_decode_8stream_tok_s"], _, _ = decode_8stream(eng, synth, torch, dev)
    out["nvfp4_prefill_8k_tok_s"], _, _ = prefill_8k(eng, synth, torch, dev)
    log(f"NVFP4 layout: decode {out['nvfp4_decode_b1_tok_s']} tok/s at B = 1, {out['nvfp4_decode_8stream_tok_s']} at 8 "
        f"streams, 8k prefill {out['nvfp4_prefill_8k_tok_s']} tok/s")
    eng.close()
    return out


def cfg5_extras(synth, torch, dev):
    """4-bit g32 linears with an 8-bit g64 embedding / head: a 32768-token prefill (one stream, 2048-row
    chunks), then 32 streams at contexts uniform in [1024, 32768] decoding 64 greedy tokens each at
    batch 32 (the first step untimed)."""
    from attention_decoder_amd.lfm3 import Engine
    out = {}
    cfg = synth.full_config(bits=4, group=32, embed_bits=8, embed_group=64, max_slots=32, max_ctx=32768 + 128,
                            max_chunk=2048)
    eng = Engine(cfg, synth.cached_blob(cfg, seed=0))
    toks = torch.from_numpy(synth.prompt_tokens(10, 32768)).to(dev)
    times = []
    for r in range(2):
        eng.reset(0)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(eng.stream)
        eng.prefill(0, tokens=toks, logits=True, argmax=True)
        b.record(eng.stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    out["cfg5_prefill_32k_ms"] = round(times[-1], 2)
    out["cfg5_prefill_32k_tok_s"] = round(32768 / (times[-1] / 1e3), 1)
    lens = synth.stream_prompt_lengths(11, 32, lo=1024, hi=32768)
    for i in range(32):
        eng.reset(i)
        eng.prefill(i, tokens=torch.from_numpy(synth.prompt_tokens(1000 + i, int(lens[i]))).to(dev), logits=False,
                    argmax=False)
    n_steps = 64
    ids = torch.empty((n_steps + 1, 32), dtype=torch.int32, device=dev)
    ids[0] = torch.from_numpy(synth.prompt_tokens(12, 32)).to(dev)
    slots = list(range(32))
    # one untimed step first, as in the 8-stream decode: the batch-32 kernels' first launches (code
    # loading) stay out of the timed steps
    eng.decode(slots, tokens=ids[0], logits=False, argmax=True, out={"argmax": ids[1]})
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(eng.stream)
    for t in range(1, n_steps):
        eng.decode(slots, tokens=ids[t], logits=False, argmax=True, out={"argmax": ids[t + 1]})
    e1.record(eng.stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    out["cfg5_decode_32stream_tok_s"] = round(32 * (n_steps - 1) / (ms / 1e3), 1)
    out["cfg5_decode_32stream_mean_context"] = int(np.mean(lens))
    out["cfg5_decode_step_breakdown_ms"] = step_breakdown(eng, slots, ids[n_steps])
    log(f"g32 + 8-bit head: 32k prefill {out['cfg5_prefill_32k_tok_s']} tok/s, 32-stream decode "
        f"{out['cfg5_decode_32stream_tok_s']} tok/s")
    eng.close()
    return out


def host_facts():
    """Host CPU model, logical CPUs and the BLAS library numpy runs on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = None, None
    try:
        from threadpoolctl import threadpool_info
        for p in threadpool_info():
            if p.get("user_api") == "blas":
                blas = f"{p.get('internal_api')} {p.get('version')}"
                threads = p.get("num_threads")
                break
    except Exception:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "blas": blas, "blas_threads": threads}


def cpu_baseline(cfg, blob, steps, prompt_len):
    """The float64 oracle on the host cores, on the GPU line's own workload: the same weights and
    the same 2048-token prompt prefilled in one call (timed), then `steps` greedy decode steps at
    T = 2049.. (timed). Decode tok/s is the value (the metric's unit); weight dequantisation is
    untimed setup."""
    from oracle import Oracle
    from attention_decoder_amd import synth
    facts = host_facts()
    orc = Oracle(cfg, blob)
    t0 = time.time()
    orc.preload(min(16, os.cpu_count() or 1))
    log(f"oracle preload {time.time() - t0:.1f}s")
    st = orc.new_slot()
    toks = synth.prompt_tokens(2, prompt_len)
    t0 = time.perf_counter()
    out = orc.forward(st, tokens=toks, logits="last")
    t_pre = time.perf_counter() - t0
    tok = int(np.argmax(out["logits"][0]))
    log(f"oracle prefill {prompt_len} in {t_pre:.1f}s")
    t0 = time.perf_counter()
    for _ in range(steps):
        out = orc.forward(st, tokens=[tok], logits="last")
        tok = int(np.argmax(out["logits"][0]))
    dt = time.perf_counter() - t0
    orc.drop_cache()
    val = steps / dt
    log(f"oracle decode {val:.3f} tok/s ({dt:.1f}s), prefill {prompt_len / t_pre:.1f} tok/s; {facts}")
    return {"value": round(val, 4), "unit": "tok/s", "cores": facts["blas_threads"] or facts["os_cpu_count"],
            "kind": "oracle",
            "sample": f"float64 oracle, full 24-layer q4 g64 geometry and the GPU line's weights: the same "
                      f"{prompt_len}-token prompt prefilled in one call ({t_pre:.1f} s, "
                      f"{prompt_len / t_pre:.1f} tok/s), then {steps} greedy decode steps at T = {prompt_len + 1}.. "
                      f"({dt:.1f} s timed; per-token rate taken as the decode rate of all 256 steps); "
                      f"weight dequantisation untimed",
            "prefill_tok_s": round(prompt_len / t_pre, 2), **facts}


if __name__ == "__main__":
    main()
