"""Benchmark of the decoder hot path on one MI355X.

Workload (default): 8B-shape LLaMA-style decoder with Q4_0 weights drawn
from N(0, 0.02) and an f16 KV cache; a 4096-token random prompt prefilled
in 8 ubatches of 512, then greedy decode at batch 1 (one token per step,
each step = decode call + on-device argmax + 4-byte readback, the
generation loop of the article's step 8).  A "step" is one decode token.

Prints ONE JSON line: decode tokens/s (value), prefill tokens/s, the
roofline of the dominant decode kernel (the fused gate/up mat-vec, timed
live with HIP events captured into the decode graph on the library's
stream) and of the dominant prefill kernel (gate/up MFMA GEMM), and the
CPU oracle timed on a bounded sample on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense f16 MFMA, TFLOP/s
METRIC = "decode tokens/s + % HBM roofline (8B-shape Q4_0, bs=1); prefill tokens/s"


def block_bytes(wtype: int) -> float:
    """Bytes per weight of the file form: Q8_0 34 / 32, Q4_0 18 / 32, Q4_K 144 / 256, F32 4."""
    return {2: 34.0 / 32, 3: 18.0 / 32, 4: 144.0 / 256}.get(wtype, 4.0)


def algorithmic(hp, n_prompt, steps):
    """Bytes per decode token (weights once, the embedding as one row, and the
    K/V rows of every layer at the mean context) and FLOPs of the prefill
    (2 per MAC; causal attention counts unmasked pairs only)."""
    d, L, F, V = hp["n_embd"], hp["n_layer"], hp["n_ff"], hp["n_vocab"]
    qd, kd = hp["n_head"] * hp["head_dim"], hp["n_head_kv"] * hp["head_dim"]
    per_layer = d * (qd + 2 * kd) + qd * d + 3 * F * d
    params = L * per_layer + V * d                       # output matrix; embedding: one row
    wbytes = params * block_bytes(hp["wtype"]) + d * block_bytes(hp["wtype"])
    kv_row = L * 2 * kd * (2 if hp["kvtype"] == 1 else 4)   # bytes per cached position
    mean_ctx = n_prompt + (steps + 1) / 2.0
    tok_bytes = wbytes + kv_row * mean_ctx
    lin_flops = 2.0 * L * per_layer * n_prompt
    attn_flops = 4.0 * hp["head_dim"] * hp["n_head"] * L * n_prompt * (n_prompt + 1) / 2.0
    out_flops = 2.0 * V * d
    return dict(weight_bytes=wbytes, kv_row_bytes=kv_row, mean_ctx=mean_ctx, token_bytes=tok_bytes,
                prefill_flops=lin_flops + attn_flops + out_flops)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_matvec_gate_up__8b_q4_decode_bs1__hbm_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "decode_amd", "csrc", f)
                  for f in ("matvec.hip", "mvcore.h", "common.h", "epilogue.h", "kernels.h")]


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the gate/up mat-vec from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel factor), or
    None when the summary is missing or was taken on different kernel source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            kv = dict(l.split(":", 1) for l in fh.read().splitlines() if l.startswith("- ") and ":" in l)
    except OSError:
        return None
    kv = {k[2:].strip(): v.strip() for k, v in kv.items()}
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _omp_set_threads(n: int) -> None:
    """Thread count of the oracle's later parallel regions (libgomp of this process)."""
    import ctypes
    ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))


def cpu_baseline(hp, weights_dev, prompt, n_prompt_tokens, n_decode_tokens, n_decode_1t, gpu_ctx):
    """The oracle (its fp32 build, as it stands) on a bounded sample of the
    same workload: n_prompt_tokens prompt tokens, then greedy decode steps,
    timed with all host threads and then with one thread."""
    import numpy as np

    import oracle
    host = {}
    for k, v in weights_dev.items():
        host[k] = [t.cpu().numpy() for t in v] if isinstance(v, list) else v.cpu().numpy()
    om = oracle.Model(hp, host, "f32")
    del host
    ctx = oracle.Context(om, 1, n_prompt_tokens + n_decode_tokens + n_decode_1t + 2)
    for t in prompt[:n_prompt_tokens - 1]:
        ctx.eval(0, int(t), want_logits=False)
    lg = ctx.eval(0, int(prompt[n_prompt_tokens - 1]))
    tok = oracle.argmax(lg, "f32")
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    _omp_set_threads(threads)

    def run(n):
        nonlocal tok
        t0 = time.perf_counter()
        for _ in range(n):
            lg = ctx.eval(0, tok)
            tok = oracle.argmax(lg, "f32")
        return time.perf_counter() - t0
    dt = run(n_decode_tokens)
    _omp_set_threads(1)
    dt1 = run(n_decode_1t)
    _omp_set_threads(threads)
    c_end = n_prompt_tokens + n_decode_tokens + n_decode_1t
    return {"value": n_decode_tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "value_1_thread": n_decode_1t / dt1, "nproc": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": f"fp32 oracle build, same weights: {n_prompt_tokens}-token prompt, then "
                      f"{n_decode_tokens} greedy decode steps on {threads} threads ({dt:.1f} s) and "
                      f"{n_decode_1t} on 1 thread ({dt1:.1f} s), at contexts {n_prompt_tokens + 1}.."
                      f"{c_end}; the GPU line decodes at context ~{gpu_ctx:.0f} (attention is about "
                      f"{100 * attention_share(hp, gpu_ctx):.0f}% of a step's multiply-adds there)"}


def attention_share(hp, ctx_len):
    """Fraction of a decode step's multiply-adds spent in attention at ctx_len."""
    d, L, F, V = hp["n_embd"], hp["n_layer"], hp["n_ff"], hp["n_vocab"]
    qd, kd = hp["n_head"] * hp["head_dim"], hp["n_head_kv"] * hp["head_dim"]
    lin = L * (d * (qd + 2 * kd) + qd * d + 3 * F * d) + V * d
    att = L * 2 * qd * ctx_len
    return att / (lin + att)


def kv_bytes_per_elem(kvtype: int) -> float:
    return {0: 4.0, 1: 2.0, 2: 34.0 / 32.0}[kvtype]


def attention_roofline(hp, kvtype, probe, ctx_len):
    """Achieved bandwidth of one layer's decode attention (partials + merge)
    from its probe: the K and V rows of ctx_len cached positions are the
    algorithmic bytes (codes and scales for Q8_0)."""
    if not probe or not probe[1]:
        return None
    kd = hp["n_head_kv"] * hp["head_dim"]
    nbytes = ctx_len * 2 * kd * kv_bytes_per_elem(kvtype)
    avg = probe[0] / 1e3 / probe[1]
    ach = nbytes / avg / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "bytes_per_launch": int(nbytes),
            "mean_context": ctx_len, "avg_us": round(avg * 1e6, 2), "launches_timed": probe[1]}


def kv_q8_leg(dec, torch, model, hp, prompt, n_ctx, n_ubatch, sp, warm, steps, probe_layer, log):
    """The generation loop again with a Q8_0 KV cache: timed prefill, then
    `steps` timed greedy decode steps; attention of the probed layer timed
    live over the same steps."""
    ctx = dec.Context(model, n_ctx=n_ctx, n_batch=len(prompt), n_ubatch=n_ubatch, stream=sp)
    ctx.set_probe(dec.K_ATTN, probe_layer)
    assert ctx.prefill(prompt, 0) == 0
    tok = ctx.argmax(-1)
    for _ in range(warm):
        assert ctx.decode([tok], [0]) == 0
        tok = ctx.argmax(0)
    ctx.clear(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    assert ctx.prefill(prompt, 0) == 0
    tok = ctx.argmax(-1)
    prefill_s = time.perf_counter() - t0
    ctx.set_probe(dec.K_ATTN, probe_layer)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        if ctx.decode([tok], [0]) != 0:
            raise RuntimeError("Q8_0-cache decode step failed")
        tok = ctx.argmax(0)
    torch.cuda.synchronize()
    decode_s = time.perf_counter() - t0
    probe = ctx.probe()
    mean_ctx = len(prompt) + (steps + 1) / 2.0
    ctx.close()
    log(f"Q8_0 KV cache: prefill {len(prompt) / prefill_s:.0f} tok/s, decode {steps / decode_s:.1f} tok/s")
    return {"decode_tokens_per_s": round(steps / decode_s, 2), "steps": steps,
            "prefill_tokens_per_s": round(len(prompt) / prefill_s, 1),
            "kv_bytes_per_position": int(hp["n_layer"] * 2 * hp["n_head_kv"] * hp["head_dim"] * 34 / 32),
            "attention": attention_roofline(hp, 2, probe, mean_ctx),
            "note": "same weights and prompt, K/V cached as Q8_0 blocks; attention = split-K partials "
                    "+ merge of one layer, timed live; prefill attention takes the flash kernel on the codes"}


def q4k_leg(dec, torch, model, hp, prompt, n_ctx, n_ubatch, sp, warm, steps, probe_layer, log):
    """The generation loop with the same fp32 weights quantized to Q4_K
    super-blocks: timed prefill (median of 3) and `steps` timed greedy decode
    steps, then the gate/up mat-vec of the probed layer timed live over 16
    decode steps and the gate/up GEMM of one prefill."""
    ctx = dec.Context(model, n_ctx=n_ctx, n_batch=len(prompt), n_ubatch=n_ubatch, stream=sp)
    assert ctx.prefill(prompt, 0) == 0
    tok = ctx.argmax(-1)
    for _ in range(warm):
        assert ctx.decode([tok], [0]) == 0
        tok = ctx.argmax(0)
    pf = []
    for _ in range(3):
        ctx.clear(0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        assert ctx.prefill(prompt, 0) == 0
        tok = ctx.argmax(-1)
        pf.append(time.perf_counter() - t0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        if ctx.decode([tok], [0]) != 0:
            raise RuntimeError("Q4_K decode step failed")
        tok = ctx.argmax(0)
    torch.cuda.synchronize()
    decode_s = time.perf_counter() - t0
    ctx.set_probe(dec.K_FFN_GU, probe_layer)
    for _ in range(16):
        assert ctx.decode([tok], [0]) == 0
        tok = ctx.argmax(0)
    mv = ctx.probe()
    ctx.set_probe(-1, 0)
    ctx.clear(0)
    ctx.set_probe(dec.K_FFN_GU, probe_layer)
    assert ctx.prefill(prompt, 0) == 0
    gm = ctx.probe()
    ctx.close()
    F, d = hp["n_ff"], hp["n_embd"]
    prefill_s = sorted(pf)[1]
    alg = algorithmic(hp, len(prompt), steps)
    step_gbs = alg["token_bytes"] / (decode_s / steps) / 1e9
    out = {"decode_tokens_per_s": round(steps / decode_s, 2), "steps": steps,
           "prefill_tokens_per_s": round(len(prompt) / prefill_s, 1),
           "decode_step_hbm": {"bytes_per_token": int(alg["token_bytes"]), "achieved_GBs": round(step_gbs, 1),
                               "frac": round(step_gbs / HBM_PEAK_GBS, 4)}}
    if mv and mv[1]:
        avg = mv[0] / 1e3 / mv[1]
        nb = 2 * F * d * block_bytes(4)
        out["gate_up_matvec"] = {"bound": "hbm", "avg_us": round(avg * 1e6, 2), "bytes": int(nb),
                                 "achieved": round(nb / avg / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": round(nb / avg / 1e9 / HBM_PEAK_GBS, 4), "launches": mv[1]}
    if gm and gm[1]:
        avg = gm[0] / 1e3 / gm[1]
        fl = 2.0 * n_ubatch * 2 * F * d
        out["gate_up_gemm"] = {"bound": "mfma", "avg_us": round(avg * 1e6, 1),
                               "achieved": round(fl / avg / 1e12, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                               "unit": "TFLOP/s", "frac": round(fl / avg / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                               "launches": gm[1]}
    out["note"] = ("same fp32 weights quantized to Q4_K super-blocks (144 bytes per 256 weights; the "
                   "library stores 148: codes, a 2-byte scale/min word per 32 and d/dmin per 256); "
                   "algorithmic bytes count 144 per 256")
    log(f"Q4_K weights: prefill {out['prefill_tokens_per_s']:.0f} tok/s, decode {out['decode_tokens_per_s']} tok/s")
    return out


def prefill_flops(hp, n_prompt, n_out=1):
    """FLOPs of a prefill of n_prompt tokens: the layers' projections for
    every token, causal attention over the unmasked pairs, and the output
    projection for the n_out rows whose logits are asked for."""
    d, L, F, V = hp["n_embd"], hp["n_layer"], hp["n_ff"], hp["n_vocab"]
    qd, kd = hp["n_head"] * hp["head_dim"], hp["n_head_kv"] * hp["head_dim"]
    per_layer = d * (qd + 2 * kd) + qd * d + 3 * F * d
    lin = 2.0 * L * per_layer * n_prompt
    attn = 4.0 * hp["head_dim"] * hp["n_head"] * L * n_prompt * (n_prompt + 1) / 2.0
    return lin + attn + 2.0 * V * d * n_out


def prefill_workload(args, dec, torch, W, hp, log):
    """A prefill-only workload (the 8B Q8_0 8192-token prompt in ubatches of
    512, logits for the last token): prefill tokens/s against the f16 MFMA
    peak, with the gate/up GEMM of the middle layer timed live."""
    import synth
    stream = torch.cuda.Stream()
    sp = stream.cuda_stream
    with torch.cuda.stream(stream):
        weights = synth.weights_torch(hp, W["seed"], "cuda")
    torch.cuda.synchronize()
    model = dec.Model(hp, weights, stream=sp)
    torch.cuda.synchronize()
    del weights
    torch.cuda.empty_cache()
    n = W["n_prompt"]
    prompt = synth.prompt(hp["n_vocab"], n, 2000 + W["seed"] % 1000)
    ctx = dec.Context(model, n_ctx=n + 64, n_batch=n, n_ubatch=W["n_ubatch"], stream=sp)
    layer = hp["n_layer"] // 2
    assert ctx.prefill(prompt, 0) == 0                       # warm-up
    times = []
    probe = None
    for rep in range(max(1, args.prefill_reps)):
        ctx.clear(0)
        ctx.set_probe(dec.K_FFN_GU, layer)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        assert ctx.prefill(prompt, 0) == 0
        tok = ctx.argmax(-1)
        times.append(time.perf_counter() - t0)
        probe = ctx.probe()
        log(f"prefill {n} tokens: {n / times[-1]:.0f} tok/s (token {tok})")
    ctx.close()
    model.close()
    t = sorted(times)[len(times) // 2]
    flops = prefill_flops(hp, n)
    gu = None
    if probe and probe[1]:
        avg = probe[0] / 1e3 / probe[1]
        gflop = 2.0 * W["n_ubatch"] * 2 * hp["n_ff"] * hp["n_embd"]
        gu = {"bound": "mfma", "achieved": round(gflop / avg / 1e12, 1), "peak": MFMA_F16_PEAK_TFLOPS,
              "unit": "TFLOP/s", "frac": round(gflop / avg / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
              "kernel": "gate/up GEMM of a 512-token ubatch (k_gemm_dw, the wide direct-to-LDS form)", "avg_us": round(avg * 1e6, 1),
              "launches_timed": probe[1]}
    out = {"metric": "prefill tokens/s (8B-shape Q8_0, 8192-token prompt, ubatches of 512)",
           "value": round(n / t, 1), "unit": "tokens/s", "n_gpus": 1, "steps": len(times), "warmup": 1,
           "ms_per_step": round(t * 1e3, 2), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f16", "data": "synthetic",
           "config": {"workload": f"8B-shape decoder, {'Q8_0' if hp['wtype'] == 2 else 'Q4_0'} weights "
                                  f"N(0,0.02), f16 KV cache: {n}-token random prompt in ubatches of "
                                  f"{W['n_ubatch']}, logits for the last token", "n_layer": hp["n_layer"],
                      "d_model": hp["n_embd"], "heads": hp["n_head"], "kv_heads": hp["n_head_kv"],
                      "head_dim": hp["head_dim"], "ffn": hp["n_ff"], "vocab": hp["n_vocab"]},
           "prefill_mfma": {"flops": flops, "achieved_TFLOPs": round(flops / t / 1e12, 1),
                            "frac": round(flops / t / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)},
           "roofline": gu, "cpu_baseline": None}
    print(json.dumps(out), flush=True)


def batched_workload(args, dec, torch, W, hp, log):
    """Batched decode of independent sequences (the 7B MHA Q4_0 workload: 32
    sequences of 2048 prompt tokens, then decode calls of one token per
    sequence): aggregate tokens/s and the decode step's HBM fraction, with
    the attention of the middle layer timed live, on an f16 and then on a
    Q8_0 cache."""
    import numpy as np

    import synth
    stream = torch.cuda.Stream()
    sp = stream.cuda_stream
    with torch.cuda.stream(stream):
        weights = synth.weights_torch(hp, W["seed"], "cuda")
    torch.cuda.synchronize()
    S, n = W["n_seq"], W["n_prompt"]
    steps, warm = min(args.steps, W["n_decode"]), args.warmup
    prompts = [synth.prompt(hp["n_vocab"], n, 3000 + s) for s in range(S)]
    layer = hp["n_layer"] // 2
    legs = {}
    for kvt, name in ((synth.F16, "f16"), (synth.Q8_0, "q8_0")):
        hpk = dict(hp, kvtype=kvt)
        model = dec.Model(hpk, weights, stream=sp)
        ctx = dec.Context(model, n_ctx=n + steps + warm + 8, n_batch=n, n_ubatch=W["n_ubatch"],
                          n_seq_max=S, stream=sp)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(S):
            assert ctx.prefill(prompts[s], s) == 0
        torch.cuda.synchronize()
        prefill_s = time.perf_counter() - t0
        seqs = np.arange(S, dtype=np.int32)
        toks = np.asarray(synth.prompt(hp["n_vocab"], S, 4000), np.int32)
        for _ in range(warm):
            assert ctx.decode(toks, seqs) == 0
            toks = ctx.argmax_all().astype(np.int32)
        ctx.set_probe(dec.K_ATTN, layer)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            if ctx.decode(toks, seqs) != 0:
                raise RuntimeError("batched decode step failed")
            toks = ctx.argmax_all().astype(np.int32)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        probe = ctx.probe()
        mean_ctx = n + warm + (steps + 1) / 2.0
        wbytes = algorithmic(hpk, 0, 0)["weight_bytes"]
        kv_row = hp["n_layer"] * 2 * hp["n_head_kv"] * hp["head_dim"] * kv_bytes_per_elem(kvt)
        step_bytes = wbytes + S * kv_row * mean_ctx
        gbs = step_bytes / (dt / steps) / 1e9
        attn = None
        if probe and probe[1]:
            avg = probe[0] / 1e3 / probe[1]
            ab = S * mean_ctx * 2 * hp["n_head_kv"] * hp["head_dim"] * kv_bytes_per_elem(kvt)
            attn = {"bound": "hbm", "achieved": round(ab / avg / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ab / avg / 1e9 / HBM_PEAK_GBS, 4), "avg_us": round(avg * 1e6, 2),
                    "bytes_per_launch": int(ab), "launches_timed": probe[1]}
        legs[name] = {"decode_tokens_per_s": round(S * steps / dt, 1), "ms_per_step": round(dt / steps * 1e3, 3),
                      "prefill_tokens_per_s": round(S * n / prefill_s, 1),
                      "step_hbm": {"bytes_per_step": int(step_bytes), "achieved_GBs": round(gbs, 1),
                                   "frac": round(gbs / HBM_PEAK_GBS, 4)},
                      "attention": attn}
        log(f"{name} cache: decode {S * steps / dt:.0f} tok/s, prefill {S * n / prefill_s:.0f} tok/s")
        ctx.close()
        model.close()
    f = legs["f16"]
    out = {"metric": "aggregate decode tokens/s (7B-shape Q4_0 MHA, 32 sequences)",
           "value": f["decode_tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warm,
           "ms_per_step": f["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f16", "data": "synthetic",
           "config": {"workload": f"7B-shape decoder, Q4_0 weights N(0,0.02), MHA: {S} sequences with their "
                                  f"own caches, {n}-token random prompts, decode calls of one token per "
                                  f"sequence", "n_layer": hp["n_layer"], "d_model": hp["n_embd"],
                      "heads": hp["n_head"], "kv_heads": hp["n_head_kv"], "head_dim": hp["head_dim"],
                      "ffn": hp["n_ff"], "vocab": hp["n_vocab"], "sequences": S},
           "decode_step_hbm": f["step_hbm"], "roofline": f["attention"], "legs": legs, "cpu_baseline": None}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256, help="timed decode steps")
    ap.add_argument("--warmup", type=int, default=8, help="untimed decode steps (graph capture)")
    ap.add_argument("--workload", default="8b_q4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-prompt", type=int, default=3)
    ap.add_argument("--cpu-decode", type=int, default=24, help="oracle decode steps on all host threads")
    ap.add_argument("--cpu-decode-1t", type=int, default=2, help="oracle decode steps on one thread")
    ap.add_argument("--reps", type=int, default=5, help="timed repetitions (prefill + steps decode steps)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the attainable stream-read / MFMA measurements")
    ap.add_argument("--no-kv-q8", action="store_true",
                    help="skip the leg that reruns the decode loop with a Q8_0 KV cache")
    ap.add_argument("--kv-q8-steps", type=int, default=128)
    ap.add_argument("--no-q4k", action="store_true",
                    help="skip the leg that reruns the generation loop with Q4_K weights")
    ap.add_argument("--q4k-steps", type=int, default=128)
    ap.add_argument("--prefill-reps", type=int, default=3, help="timed prefills of a prefill-only workload")
    ap.add_argument("--no-step-kernel", action="store_true",
                    help="skip the leg that runs decode steps through the one-launch step kernel")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (4 times), the reference kernel for "
                         "scaling the HBM fetch/write counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the library runs on exactly one GPU (the decode step of one sequence "
              "batch on one MI355X); --gpus N>1 is not supported.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import decode_amd as dec
    import synth

    W = synth.WORKLOADS[args.workload]
    hp = synth.hparams(W)
    n_prompt = W["n_prompt"]
    if W["n_decode"] == 0 or W["n_seq"] > 1:
        torch.cuda.set_device(0)
        dec.lib()

        def log(msg):
            print(f"[bench] {msg}", file=sys.stderr, flush=True)
        if W["n_decode"] == 0:
            prefill_workload(args, dec, torch, W, hp, log)
        else:
            batched_workload(args, dec, torch, W, hp, log)
        return
    steps, warm, reps = args.steps, args.warmup, max(1, args.reps)
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    sp = stream.cuda_stream
    dec.lib()

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        weights = synth.weights_torch(hp, W["seed"], "cuda")
    torch.cuda.synchronize()
    log(f"weights generated in {time.perf_counter() - t0:.1f} s")
    t0 = time.perf_counter()
    model = dec.Model(hp, weights, stream=sp)
    torch.cuda.synchronize()
    log(f"model loaded (quantized on device) in {time.perf_counter() - t0:.1f} s")
    model_q8 = None
    if not args.no_kv_q8:
        # same weights, Q8_0 KV cache (the KV-cache appendix's quantized cache types)
        model_q8 = dec.Model(dict(hp, kvtype=synth.Q8_0), weights, stream=sp)
        torch.cuda.synchronize()
    model_k4 = None
    if not args.no_q4k and hp["wtype"] != synth.Q4_K:
        # same weights as Q4_K super-blocks (the k-quant type of the GGUF type list)
        model_k4 = dec.Model(dict(hp, wtype=synth.Q4_K), weights, stream=sp)
        torch.cuda.synchronize()
    if args.no_cpu_baseline:
        del weights
        torch.cuda.empty_cache()

    prompt = synth.prompt(hp["n_vocab"], n_prompt, 2000 + W["seed"] % 1000)
    n_probe = 16                        # decode steps per probed kernel role, after the timed loops
    roles = [("qkv", dec.K_QKV), ("attention", dec.K_ATTN), ("o", dec.K_WO), ("gate_up", dec.K_FFN_GU),
             ("down", dec.K_FFN_DOWN), ("output", dec.K_OUTPUT)]
    n_sampled = 64                      # decode steps run with the sampler chain
    n_step_leg = 64                     # decode steps through the one-launch step kernel
    n_ctx = n_prompt + max(steps, warm) + n_probe * len(roles) + n_sampled + n_step_leg + 32
    ctx = dec.Context(model, n_ctx=n_ctx, n_batch=n_prompt, n_ubatch=W["n_ubatch"], stream=sp)
    probe_layer = hp["n_layer"] // 2

    # warm-up: prefill + decode steps (captures the decode graph)
    assert ctx.prefill(prompt, 0) == 0
    tok = ctx.argmax(-1)
    for _ in range(warm):
        assert ctx.decode([tok], [0]) == 0
        tok = ctx.argmax(0)
    torch.cuda.synchronize()
    log("warm-up done")

    # timed repetitions, no probe set: each clears the cache, prefills the
    # prompt (timed to its greedy token on the host), then times exactly
    # `steps` decode steps, each a decode call + greedy token readback
    pf_s, dc_s = [], []
    for r in range(reps):
        ctx.clear(0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        assert ctx.prefill(prompt, 0) == 0
        tok = ctx.argmax(-1)
        pf_s.append(time.perf_counter() - t0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            rc = ctx.decode([tok], [0])
            if rc != 0:
                raise RuntimeError(f"dec_decode returned {rc}")
            tok = ctx.argmax(0)
        torch.cuda.synchronize()
        dc_s.append(time.perf_counter() - t0)
        log(f"rep {r}: prefill {n_prompt / pf_s[-1]:.0f} tok/s, decode {steps / dc_s[-1]:.1f} tok/s")
    st = ctx.stats()
    decode_s = sorted(dc_s)[len(dc_s) // 2]
    prefill_s = sorted(pf_s)[len(pf_s) // 2]

    # probe pass (outside the timed repetitions): each kernel role of the middle
    # layer timed live over n_probe further decode steps, then one more prefill
    # with its gate/up GEMM and its attention probed
    per_kernel = {}
    alg0 = algorithmic(hp, 0, 0)
    F, d, V = hp["n_ff"], hp["n_embd"], hp["n_vocab"]
    qd, kd = hp["n_head"] * hp["head_dim"], hp["n_head_kv"] * hp["head_dim"]
    bb = block_bytes(hp["wtype"])
    role_bytes = {"qkv": (qd + 2 * kd) * d * bb, "o": d * qd * bb, "gate_up": 2 * F * d * bb,
                  "down": d * F * bb, "output": V * d * bb}
    dc_probe = None
    for name, role in roles:
        ctx.set_probe(role, probe_layer)
        c0 = ctx.pos_max(0) + 1
        for _ in range(n_probe):
            assert ctx.decode([tok], [0]) == 0
            tok = ctx.argmax(0)
        pr = ctx.probe()
        if not pr or not pr[1]:
            continue
        avg = pr[0] / 1e3 / pr[1]
        nb = role_bytes.get(name)
        if name == "attention":
            nb = (c0 + (n_probe - 1) / 2.0) * 2 * kd * kv_bytes_per_elem(hp["kvtype"])
        ach = nb / avg / 1e9
        per_kernel[name] = {"avg_us": round(avg * 1e6, 2), "bytes": int(nb), "achieved_GBs": round(ach, 1),
                            "frac": round(ach / HBM_PEAK_GBS, 4), "launches": pr[1]}
        if name == "gate_up":
            dc_probe = pr
    ctx.set_probe(-1, 0)
    pf_probe = pf_attn = None
    ctx2 = dec.Context(model, n_ctx=n_prompt + 8, n_batch=n_prompt, n_ubatch=W["n_ubatch"], stream=sp)
    for role in (dec.K_FFN_GU, dec.K_ATTN):
        ctx2.clear(0)
        ctx2.set_probe(role, probe_layer)
        assert ctx2.prefill(prompt, 0) == 0
        if role == dec.K_FFN_GU:
            pf_probe = ctx2.probe()
        else:
            pf_attn = ctx2.probe()
    ctx2.close()
    log("probe pass done")

    # the sampler chain in the generation loop (outside the timed region):
    # penalty over the last 64 tokens, top-k 40, top-p 0.95, min-p 0.05, temperature 0.8
    sprm = dict(top_k=40, top_p=0.95, min_p=0.05, temp=0.8, repeat_penalty=1.1, penalty_last_n=64, seed=1234)
    smp = dec.Sampler(**sprm)
    smp.accept(prompt[-64:])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_sampled):
        tok = smp.sample(ctx, 0)
        if tok < 0 or ctx.decode([tok], [0]) != 0:
            raise RuntimeError("sampled decode step failed")
    torch.cuda.synchronize()
    sampled_s = time.perf_counter() - t0
    n_calls = 256
    t0 = time.perf_counter()
    for _ in range(n_calls):
        if smp.sample(ctx, 0) < 0:
            raise RuntimeError("dec_sampler_sample failed")
    call_s = (time.perf_counter() - t0) / n_calls
    smp.close()
    sampler = {"chain": sprm, "n_vocab": hp["n_vocab"],
               "decode_tokens_per_s_sampled": round(n_sampled / sampled_s, 2),
               "us_per_call": round(call_s * 1e6, 2),
               "note": "us_per_call = one dec_sampler_sample on a resident logits row: history upload, "
                       "the k_sample kernel, token download and stream synchronisation"}
    log(f"sampled decode {n_sampled / sampled_s:.1f} tok/s, sampler call {call_s * 1e6:.1f} us")
    tok = ctx.argmax(0)

    # the same generation loop through the persistent one-launch step kernel
    # (opt-in; reported beside the default per-layer graph)
    step_leg = None
    if not args.no_step_kernel and ctx.step_kernel(1) >= 0:
        ctx.set_probe(dec.K_STEP, 0)
        for _ in range(4):
            assert ctx.decode([tok], [0]) == 0
            tok = ctx.argmax(0)
        ctx.set_probe(dec.K_STEP, 0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n_step_leg - 4):
            if ctx.decode([tok], [0]) != 0:
                raise RuntimeError("step-kernel decode step failed")
            tok = ctx.argmax(0)
            if tok < 0:
                raise RuntimeError("step kernel: a grid barrier timed out")
        torch.cuda.synchronize()
        sk_s = time.perf_counter() - t0
        sk_probe = ctx.probe()
        ctx.set_probe(-1, 0)
        ctx.step_kernel(0)
        sk_ctx = ctx.pos_max(0) + 1 - (n_step_leg - 4 - 1) / 2.0
        sk_bytes = alg0["weight_bytes"] + alg0["kv_row_bytes"] * sk_ctx
        sk_us = sk_probe[0] * 1e3 / sk_probe[1] if sk_probe and sk_probe[1] else None
        step_leg = {"decode_tokens_per_s": round((n_step_leg - 4) / sk_s, 2), "steps": n_step_leg - 4,
                    "kernel_us": round(sk_us, 1) if sk_us else None,
                    "achieved_GBs": round(sk_bytes / (sk_us * 1e-6) / 1e9, 1) if sk_us else None,
                    "frac": round(sk_bytes / (sk_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4) if sk_us else None,
                    "bytes_per_token": int(sk_bytes), "mean_context": sk_ctx,
                    "note": "whole decode step as one cooperative launch with grid barriers between the "
                            "layer stages (dec_set_step_kernel); kernel_us from events around the launch"}
        log(f"step kernel: {step_leg['decode_tokens_per_s']} tok/s, {step_leg['kernel_us']} us per launch")
    ctx.close()

    kv_q8 = None
    if model_q8 is not None:
        kv_q8 = kv_q8_leg(dec, torch, model_q8, hp, prompt, n_ctx, W["n_ubatch"], sp, warm,
                          args.kv_q8_steps, probe_layer, log)
        if "attention" in per_kernel:
            kv_q8["f16_attention"] = per_kernel["attention"]
        model_q8.close()
    q4k = None
    if model_k4 is not None:
        q4k = q4k_leg(dec, torch, model_k4, dict(hp, wtype=synth.Q4_K), prompt, n_ctx, W["n_ubatch"], sp, warm,
                      args.q4k_steps, probe_layer, log)
        model_k4.close()
    model.close()

    alg = algorithmic(hp, n_prompt, steps)
    gu_bytes = role_bytes["gate_up"]
    gu_avg_s = dc_probe[0] / 1e3 / max(dc_probe[1], 1) if dc_probe and dc_probe[1] else None
    roofline = None
    if gu_avg_s:
        ach = gu_bytes / gu_avg_s / 1e9
        traffic = measured_traffic()
        roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBS, 4),
                    "traffic": None if traffic is None else int(traffic),
                    "kernel": "k_matvec (gate/up block-quantized mat-vec + RMSNorm prologue + SwiGLU epilogue)",
                    "bytes_per_launch": gu_bytes, "avg_us": round(gu_avg_s * 1e6, 2),
                    "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                    "kernel_source_sha256_16": kernel_source_hash(),
                    "launches_timed": dc_probe[1]}
    pf_roof = None
    if pf_probe and pf_probe[1]:
        T = W["n_ubatch"]
        flops = 2.0 * T * 2 * F * d
        avg = pf_probe[0] / 1e3 / pf_probe[1]
        ach = flops / avg / 1e12
        pf_roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                   "unit": "TFLOP/s", "frac": round(ach / MFMA_F16_PEAK_TFLOPS, 4),
                   "kernel": "gate/up GEMM of a 512-token ubatch (k_gemm_dw, the wide direct-to-LDS form)", "avg_us": round(avg * 1e6, 1),
                   "launches_timed": pf_probe[1]}
        if pf_attn and pf_attn[1]:
            pf_roof["attention_avg_us_per_ubatch"] = round(pf_attn[0] * 1e3 / pf_attn[1], 1)
    step_gbs = alg["token_bytes"] / (decode_s / steps) / 1e9

    if args.copy_calibration:
        with torch.cuda.stream(stream):
            src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
            dst = torch.empty_like(src)
            for _ in range(4):
                dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ceilings = None
    if not args.no_ceilings:
        rd = dec.measure_stream_read(2 << 30, 10, sp)
        mf = dec.measure_mfma_f16(20000, 5, sp)
        ceilings = {"hbm_stream_read_GBs": round(rd, 1), "mfma_f16_TFLOPs": round(mf, 1),
                    "decode_step_frac_of_attainable": round(step_gbs / rd, 4),
                    "note": "dec_measure_stream_read (2 GiB read with 16-byte loads) and "
                            "dec_measure_mfma_f16 (independent 32x32x16 f16 MFMAs, 8 wavefronts per CU), "
                            "measured in this run"}
        if roofline:
            roofline["frac_of_attainable"] = round(roofline["achieved"] / rd, 4)
        if pf_roof:
            pf_roof["frac_of_attainable"] = round(pf_roof["achieved"] / mf, 4)
        log(f"ceilings: stream read {rd:.0f} GB/s, f16 MFMA {mf:.0f} TFLOP/s")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host cores")
        cpu = cpu_baseline(hp, weights, prompt, args.cpu_prompt, args.cpu_decode, args.cpu_decode_1t,
                           alg["mean_ctx"])
        del weights

    wname = {synth.Q8_0: "Q8_0", synth.Q4_0: "Q4_0", synth.Q4_K: "Q4_K"}.get(hp["wtype"], "F32")
    kvname = {0: "f32", 1: "f16", 2: "Q8_0"}[hp["kvtype"]]
    out = {
        "metric": METRIC,
        "value": round(steps / decode_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(decode_s / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "repetitions": {"n": reps, "decode_tokens_per_s": [round(steps / t, 2) for t in dc_s],
                        "decode_min_tokens_per_s": round(steps / max(dc_s), 2),
                        "decode_max_tokens_per_s": round(steps / min(dc_s), 2),
                        "prefill_tokens_per_s": [round(n_prompt / t, 1) for t in pf_s],
                        "note": "value and prefill_tokens_per_s are the medians; no probe is set during "
                                "these repetitions"},
        "config": {"workload": f"{args.workload}: {hp['n_layer']}-layer decoder (d {d}, {hp['n_head']} heads / "
                               f"{hp['n_head_kv']} KV heads of {hp['head_dim']}, FFN {F}, vocab {V}), {wname} "
                               f"weights N(0,0.02), {kvname} KV cache, batch 1: {n_prompt}-token random prompt "
                               f"in ubatches of {W['n_ubatch']}, then {steps} greedy decode steps",
                   "n_layer": hp["n_layer"], "d_model": d, "heads": hp["n_head"],
                   "kv_heads": hp["n_head_kv"], "head_dim": hp["head_dim"], "ffn": F,
                   "vocab": V, "prefill_tokens": n_prompt, "n_ubatch": W["n_ubatch"],
                   "mean_decode_context": alg["mean_ctx"]},
        "precision": {"weights": wname.lower(), "activations": "f16 value + f16 remainder", "accumulate": "f32",
                      "kv": kvname},
        "prefill_tokens_per_s": round(n_prompt / prefill_s, 1),
        "prefill_ms": round(prefill_s * 1e3, 2),
        "decode_step_hbm": {"bytes_per_token": int(alg["token_bytes"]), "achieved_GBs": round(step_gbs, 1),
                            "frac": round(step_gbs / HBM_PEAK_GBS, 4)},
        "prefill_mfma": {"flops": alg["prefill_flops"],
                         "achieved_TFLOPs": round(alg["prefill_flops"] / prefill_s / 1e12, 1),
                         "frac": round(alg["prefill_flops"] / prefill_s / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)},
        "roofline": roofline,
        "prefill_roofline": pf_roof,
        "decode_kernels": {"layer": probe_layer, "steps_each": n_probe, "kernels": per_kernel,
                           "note": "per kernel role of one layer (output: the final projection), timed live "
                                   "in a probe pass after the timed repetitions; bytes are algorithmic"},
        "ceilings": ceilings,
        "graph_replays": st["n_graph_replays"],
        "sampler": sampler,
        "kv_q8_0": kv_q8,
        "q4_k": q4k,
        "step_kernel": step_leg,
        "cpu_baseline": cpu,
    }
    torch.cuda.synchronize()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
