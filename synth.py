"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the decoder: it only draws random numbers.
Both the HIP library and the oracle receive the same fp32 bytes from here and
each quantizes them with its own codec.

Recipe (the decoder shapes come from the workloads below):
  * every 2-D matrix ~ N(0, 0.02) in fp32, one independent stream per tensor,
    tensors in the order tok_embd; per layer wq, wk, wv, wo, ffn_gate, ffn_up,
    ffn_down; output;
  * the 1-D norm gains are 1.0 (the standard LLaMA initialisation);
  * prompt ids are uniform integers in [0, n_vocab).
Two generators exist: ``numpy`` (PCG64 streams seeded by (seed, tensor index);
used on the CPU and for the small workloads) and ``torch`` (torch.Generator
on the target device seeded with seed*1_000_003 + tensor index; used where
numpy would take minutes, e.g. the 8B shapes).  They give different values
for the same seed; a run always hands the same bytes to both sides.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

# element types (same numbering as the library's public header)
F32, F16, Q8_0, Q4_0, Q4_K = 0, 1, 2, 3, 4

WORKLOADS = {
    # 2 layers, d 256, 4 heads (hd 64, no GQA), FFN 688, vocab 1024, fp32
    # weights and KV; 16-token prompt in one ubatch, 16 greedy decode steps.
    "tiny": dict(n_layer=2, n_embd=256, n_head=4, n_head_kv=4, head_dim=64, n_ff=688,
                 n_vocab=1024, wtype=F32, kvtype=F32, n_prompt=16, n_ubatch=16,
                 n_decode=16, n_seq=1, seed=1001),
    # 1B shape, Q8_0 weights, f16 KV; 512 prompt (one ubatch), 128 decode steps.
    "1b_q8": dict(n_layer=16, n_embd=2048, n_head=32, n_head_kv=8, head_dim=64, n_ff=8192,
                  n_vocab=32000, wtype=Q8_0, kvtype=F16, n_prompt=512, n_ubatch=512,
                  n_decode=128, n_seq=1, seed=1002),
    # 8B shape, Q4_0 weights, f16 KV; 4096 prompt in ubatches of 512, 256 decode steps.
    "8b_q4": dict(n_layer=32, n_embd=4096, n_head=32, n_head_kv=8, head_dim=128, n_ff=14336,
                  n_vocab=32000, wtype=Q4_0, kvtype=F16, n_prompt=4096, n_ubatch=512,
                  n_decode=256, n_seq=1, seed=1003),
    # 8B shape, Q8_0 weights; 8192 prompt in 16 ubatches of 512, last-token logits.
    "8b_q8_long": dict(n_layer=32, n_embd=4096, n_head=32, n_head_kv=8, head_dim=128,
                       n_ff=14336, n_vocab=32000, wtype=Q8_0, kvtype=F16, n_prompt=8192,
                       n_ubatch=512, n_decode=0, n_seq=1, seed=1004),
    # 8B shape with Q4_K super-block weights, f16 KV; 4096 prompt, 256 decode steps.
    "8b_q4k": dict(n_layer=32, n_embd=4096, n_head=32, n_head_kv=8, head_dim=128, n_ff=14336,
                   n_vocab=32000, wtype=Q4_K, kvtype=F16, n_prompt=4096, n_ubatch=512,
                   n_decode=256, n_seq=1, seed=1006),
    # 7B shape (MHA), Q4_0; 32 sequences x 2048 prompt, 128 steps of 32 tokens.
    "7b_q4_b32": dict(n_layer=32, n_embd=4096, n_head=32, n_head_kv=32, head_dim=128,
                      n_ff=11008, n_vocab=32000, wtype=Q4_0, kvtype=F16, n_prompt=2048,
                      n_ubatch=512, n_decode=128, n_seq=32, seed=1005),
}

HP_KEYS = ("n_layer", "n_embd", "n_head", "n_head_kv", "head_dim", "n_ff", "n_vocab",
           "wtype", "kvtype")
MATS = ("wq", "wk", "wv", "wo", "ffn_gate", "ffn_up", "ffn_down")


def hparams(w: dict, **over) -> dict:
    hp = {k: w[k] for k in HP_KEYS}
    hp.update(rms_eps=1e-5, rope_base=10000.0)
    hp.update(over)
    return hp


def shapes(hp: dict) -> dict:
    d, qd, kd, F, V = (hp["n_embd"], hp["n_head"] * hp["head_dim"],
                       hp["n_head_kv"] * hp["head_dim"], hp["n_ff"], hp["n_vocab"])
    return {"tok_embd": (V, d), "output": (V, d), "wq": (qd, d), "wk": (kd, d), "wv": (kd, d),
            "wo": (d, qd), "ffn_gate": (F, d), "ffn_up": (F, d), "ffn_down": (d, F)}


def tensor_order(hp: dict):
    """(name, layer) in stream order; layer is None for the global tensors."""
    order = [("tok_embd", None)]
    for l in range(hp["n_layer"]):
        order += [(m, l) for m in MATS]
    order.append(("output", None))
    return order


def _np_normal(seed: int, idx: int, shape) -> np.ndarray:
    a = np.random.default_rng([seed, idx]).standard_normal(shape, dtype=np.float32)
    a *= np.float32(0.02)
    return a


def weights_numpy(hp: dict, seed: int, threads: int = 8) -> dict:
    """All weights as fp32 numpy arrays (dict of arrays / per-layer lists)."""
    sh = shapes(hp)
    order = tensor_order(hp)
    with ThreadPoolExecutor(threads) as ex:
        arrs = list(ex.map(lambda it: _np_normal(seed, it[0], sh[it[1][0]]), enumerate(order)))
    return _assemble(hp, order, arrs, lambda n: np.ones(n, np.float32))


def weights_torch(hp: dict, seed: int, device) -> dict:
    """All weights as fp32 torch tensors on ``device`` (same layout as numpy)."""
    import torch
    sh = shapes(hp)
    order = tensor_order(hp)
    arrs = []
    for idx, (name, _) in enumerate(order):
        g = torch.Generator(device=device)
        g.manual_seed(seed * 1_000_003 + idx)
        t = torch.randn(sh[name], generator=g, device=device, dtype=torch.float32)
        t.mul_(0.02)
        arrs.append(t)
    return _assemble(hp, order, arrs,
                     lambda n: torch.ones(n, device=device, dtype=torch.float32))


def _assemble(hp, order, arrs, ones):
    L = hp["n_layer"]
    w = {m: [None] * L for m in MATS}
    for (name, layer), a in zip(order, arrs):
        if layer is None:
            w[name] = a
        else:
            w[name][layer] = a
    w["output_norm"] = ones(hp["n_embd"])
    w["attn_norm"] = [ones(hp["n_embd"]) for _ in range(L)]
    w["ffn_norm"] = [ones(hp["n_embd"]) for _ in range(L)]
    return w


def prompt(n_vocab: int, n: int, seed: int) -> np.ndarray:
    return np.random.default_rng(seed).integers(0, n_vocab, n, dtype=np.int64).astype(np.int32)


def normal(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    a = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return a
