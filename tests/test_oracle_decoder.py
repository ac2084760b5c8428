"""Pins for the oracle's decoder as a whole.

The oracle runs tokens one at a time against its KV cache.  Here an
independent dense formulation recomputes the whole sequence at once in numpy
(matrix products, complex-number RoPE, an explicit [T, T] causal mask): the
KV-cache path must equal full-sequence recompute, which pins positions,
cache rows, the append-then-attend order, head grouping and the residual
wiring.  Further pins: GQA equals MHA with repeated K/V heads, sequences in
one context do not interact, the f32 build stays within 1e-4 of the f64
build, and degenerate weights reduce the model to closed forms.
"""
import numpy as np
import pytest

import synth

TINY = dict(n_layer=2, n_embd=64, n_head=4, n_head_kv=2, head_dim=16, n_ff=96, n_vocab=50,
            rms_eps=1e-5, rope_base=10000.0)


def _hp(**over):
    hp = dict(TINY, wtype=synth.F32, kvtype=synth.F32)
    hp.update(over)
    return hp


def _weights(hp, seed, gain_noise=True):
    w = synth.weights_numpy(hp, seed, threads=2)
    if gain_noise:      # non-unit gains so that a dropped gain would show
        rng = np.random.default_rng(seed + 99)
        w["output_norm"] = rng.uniform(0.5, 1.5, hp["n_embd"]).astype(np.float32)
        w["attn_norm"] = [rng.uniform(0.5, 1.5, hp["n_embd"]).astype(np.float32)
                          for _ in range(hp["n_layer"])]
        w["ffn_norm"] = [rng.uniform(0.5, 1.5, hp["n_embd"]).astype(np.float32)
                         for _ in range(hp["n_layer"])]
        # larger weights give logits well away from zero
        for k in ("wq", "wk", "wv", "wo", "ffn_gate", "ffn_up", "ffn_down"):
            w[k] = [a * np.float32(10) for a in w[k]]
        w["tok_embd"] = w["tok_embd"] * np.float32(50)
        w["output"] = w["output"] * np.float32(10)
    return w


def _deq(orc, a, wtype):
    if wtype == synth.F32:
        return a.astype(np.float64)
    return orc.dequantize(orc.quantize(a, wtype), a.size, wtype).reshape(a.shape).astype(np.float64)


def dense_forward(orc, hp, w, tokens):
    """Whole-sequence causal forward pass in numpy float64."""
    T = len(tokens)
    d, H, Hkv, hd = hp["n_embd"], hp["n_head"], hp["n_head_kv"], hp["head_dim"]
    wt = hp["wtype"]
    X = _deq(orc, w["tok_embd"], wt)[np.asarray(tokens)]
    pos = np.arange(T)
    inv = hp["rope_base"] ** (-np.arange(0, hd, 2) / hd)
    rot = np.exp(1j * pos[:, None] * inv[None, :])          # [T, hd/2]

    def rms(Z, g):
        return Z / np.sqrt(np.mean(Z * Z, axis=1, keepdims=True) + hp["rms_eps"]) * g

    def rope(Z, nh):
        Zc = Z.reshape(T, nh, hd // 2, 2)
        c = (Zc[..., 0] + 1j * Zc[..., 1]) * rot[:, None, :]
        return np.stack([c.real, c.imag], -1).reshape(T, nh * hd)

    mask = np.tril(np.ones((T, T), bool))
    for l in range(hp["n_layer"]):
        Xn = rms(X, w["attn_norm"][l].astype(np.float64))
        Q = rope(Xn @ _deq(orc, w["wq"][l], wt).T, H)
        K = rope(Xn @ _deq(orc, w["wk"][l], wt).T, Hkv)
        Vv = Xn @ _deq(orc, w["wv"][l], wt).T
        # the cache stores K and V in its element type (f32, f16, or Q8_0 blocks
        # of 32 consecutive elements of a position's row, coded from fp32)
        if hp["kvtype"] == synth.Q8_0:
            K = _deq(orc, K.astype(np.float32), synth.Q8_0)
            Vv = _deq(orc, Vv.astype(np.float32), synth.Q8_0)
        else:
            ct = np.float16 if hp["kvtype"] == synth.F16 else np.float32
            K = K.astype(ct).astype(np.float64)
            Vv = Vv.astype(ct).astype(np.float64)
        O = np.zeros((T, H * hd))
        for h in range(H):
            g = h // (H // Hkv)
            q = Q[:, h * hd:(h + 1) * hd]
            k = K[:, g * hd:(g + 1) * hd]
            v = Vv[:, g * hd:(g + 1) * hd]
            S = np.where(mask, q @ k.T / np.sqrt(hd), -np.inf)
            P = np.exp(S - S.max(1, keepdims=True))
            P /= P.sum(1, keepdims=True)
            O[:, h * hd:(h + 1) * hd] = P @ v
        X = X + O @ _deq(orc, w["wo"][l], wt).T
        Xn = rms(X, w["ffn_norm"][l].astype(np.float64))
        U = Xn @ _deq(orc, w["ffn_gate"][l], wt).T
        G = Xn @ _deq(orc, w["ffn_up"][l], wt).T
        Hh = U / (1 + np.exp(-U)) * G
        X = X + Hh @ _deq(orc, w["ffn_down"][l], wt).T
    Xn = rms(X, w["output_norm"].astype(np.float64))
    return Xn @ _deq(orc, w["output"], wt).T


def _oracle_all_logits(orc, hp, w, tokens, kind="f64", n_ctx=64):
    m = orc.Model(hp, w, kind)
    c = orc.Context(m, 1, n_ctx)
    return np.stack([c.eval(0, int(t)) for t in tokens]).astype(np.float64)


@pytest.mark.parametrize("wtype,kvtype", [(synth.F32, synth.F32), (synth.F32, synth.F16),
                                          (synth.Q8_0, synth.F16), (synth.Q4_0, synth.F16),
                                          (synth.F32, synth.Q8_0), (synth.Q4_0, synth.Q8_0)])
def test_cache_equals_full_recompute(orc, wtype, kvtype):
    # a Q8_0 cache needs whole 32-element blocks per head
    hp = _hp(wtype=wtype, kvtype=kvtype, head_dim=32 if kvtype == synth.Q8_0 else 16)
    w = _weights(hp, 5)
    toks = synth.prompt(hp["n_vocab"], 21, 6)
    got = _oracle_all_logits(orc, hp, w, toks)
    ref = dense_forward(orc, hp, w, toks)
    assert np.abs(ref).max() > 1.0
    # the f16 cache rounds K/V; the dense model rounds the same values
    # (identical up to double-rounding ties), so both agree to ~1e-9
    tol = 1e-9 if kvtype == synth.F32 else 1e-6
    assert np.abs(got - ref).max() <= tol * np.abs(ref).max()


def test_q4_k_weights_equal_full_recompute(orc):
    # Q4_K rows are whole 256-element super-blocks: d, H*hd and F multiples of 256
    hp = _hp(wtype=synth.Q4_K, kvtype=synth.F16, n_embd=256, head_dim=64, n_ff=512)
    w = _weights(hp, 6)
    toks = synth.prompt(hp["n_vocab"], 9, 7)
    got = _oracle_all_logits(orc, hp, w, toks)
    ref = dense_forward(orc, hp, w, toks)
    assert np.abs(ref).max() > 1.0
    assert np.abs(got - ref).max() <= 1e-6 * np.abs(ref).max()
    # and the Q4_K model is not the F32 one: the codes moved the logits
    f32 = _oracle_all_logits(orc, dict(hp, wtype=synth.F32), w, toks)
    assert np.abs(f32 - got).max() > 1e-3 * np.abs(ref).max()


def test_gqa_equals_mha_with_repeated_heads(orc):
    hp = _hp()
    w = _weights(hp, 7)
    hp_m = _hp(n_head_kv=hp["n_head"])
    rep = hp["n_head"] // hp["n_head_kv"]
    hd = hp["head_dim"]
    wm = dict(w)
    for name in ("wk", "wv"):
        wm[name] = [np.concatenate([a[g * hd:(g + 1) * hd] for g in range(hp["n_head_kv"])
                                    for _ in range(rep)]) for a in w[name]]
    toks = synth.prompt(hp["n_vocab"], 12, 8)
    a = _oracle_all_logits(orc, hp, w, toks)
    b = _oracle_all_logits(orc, hp_m, wm, toks)
    assert np.array_equal(a, b)


def test_sequences_are_independent(orc):
    hp = _hp(kvtype=synth.F16)
    w = _weights(hp, 9)
    m = orc.Model(hp, w)
    t0 = synth.prompt(hp["n_vocab"], 10, 10)
    t1 = synth.prompt(hp["n_vocab"], 10, 11)
    c = orc.Context(m, 2, 32)
    inter0, inter1 = [], []
    for a, b in zip(t0, t1):
        inter0.append(c.eval(0, int(a)))
        inter1.append(c.eval(1, int(b)))
    s0 = orc.Context(m, 1, 32)
    s1 = orc.Context(m, 1, 32)
    assert np.array_equal(np.stack(inter0), np.stack([s0.eval(0, int(a)) for a in t0]))
    assert np.array_equal(np.stack(inter1), np.stack([s1.eval(0, int(b)) for b in t1]))
    assert c.pos_max(0) == 9 and c.pos_max(1) == 9
    # clearing a sequence restarts it at position 0
    c.clear(1)
    assert c.pos_max(1) == -1
    assert np.array_equal(c.eval(1, int(t1[0])), inter1[0])


def test_f32_build_within_1e4_of_f64(orc):
    hp = _hp(wtype=synth.Q8_0, kvtype=synth.F16, n_layer=3)
    w = _weights(hp, 12, gain_noise=False)
    toks = synth.prompt(hp["n_vocab"], 30, 13)
    a = _oracle_all_logits(orc, hp, w, toks, "f64")
    b = _oracle_all_logits(orc, hp, w, toks, "f32")
    assert np.abs(a - b).max() <= 1e-4


def test_zero_sublayers_reduce_to_embedding_readout(orc):
    hp = _hp()
    w = _weights(hp, 14)
    w["wo"] = [np.zeros_like(a) for a in w["wo"]]
    w["ffn_down"] = [np.zeros_like(a) for a in w["ffn_down"]]
    toks = [3, 17, 3]
    got = _oracle_all_logits(orc, hp, w, toks)
    E = w["tok_embd"].astype(np.float64)[toks]
    g = w["output_norm"].astype(np.float64)
    Xn = E / np.sqrt(np.mean(E * E, 1, keepdims=True) + 1e-5) * g
    ref = Xn @ w["output"].astype(np.float64).T
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(got[0], got[2])       # same token, no mixing -> same logits


def test_return_codes(orc):
    hp = _hp()
    m = orc.Model(hp, _weights(hp, 15))
    c = orc.Context(m, 1, 4)
    L = orc.load()
    assert L.orc_eval(c.ptr, 0, hp["n_vocab"], None) == -1      # token out of range
    assert L.orc_eval(c.ptr, 1, 0, None) == -1                  # seq out of range
    for _ in range(4):
        assert L.orc_eval(c.ptr, 0, 1, None) == 0
    assert L.orc_eval(c.ptr, 0, 1, None) == 1                   # context full
    assert c.pos_max(0) == 3
    # Q4_K needs rows of whole 256-element super-blocks
    with pytest.raises(ValueError):
        orc.Model(_hp(wtype=synth.Q4_K), _weights(_hp(), 15))


def test_kv_rows_hold_rotated_keys(orc):
    hp = _hp()
    w = _weights(hp, 16)
    m = orc.Model(hp, w)
    c = orc.Context(m, 1, 8)
    toks = [5, 9, 2]
    for t in toks:
        c.eval(0, t)
    # layer 0 K row of position 2 = RoPE(Wk . rmsnorm(emb), 2)
    e = w["tok_embd"][toks[2]].astype(np.float64)
    xn = e / np.sqrt(np.mean(e * e) + 1e-5) * w["attn_norm"][0]
    k = w["wk"][0].astype(np.float64) @ xn
    hd = hp["head_dim"]
    kc = k[hd:2 * hd].reshape(-1, 2)
    th = 2 * 10000.0 ** (-np.arange(0, hd, 2) / hd)
    z = (kc[:, 0] + 1j * kc[:, 1]) * np.exp(1j * th)
    ref = np.stack([z.real, z.imag], -1).ravel()
    assert np.allclose(c.kv_row(0, 0, 0, 2, 1), ref, rtol=1e-6, atol=1e-6)
    assert np.allclose(c.kv_row(1, 0, 0, 2, 1),
                       (w["wv"][0].astype(np.float64) @ xn)[hd:2 * hd], rtol=1e-6, atol=1e-6)


def test_q8_0_cache_rows_within_half_step(orc):
    """Layer-0 K/V rows depend on the token only, so a Q8_0 cache and an f32
    cache of the same run hold the same rows up to the codec's error: at most
    half a step of the block's fp32 scale amax/127, plus the f16 rounding of
    the stored scale times the largest code."""
    hp32 = _hp(head_dim=32)
    w = _weights(hp32, 17)
    toks = [3, 41, 7, 7, 19]
    ctx = {}
    for kvt in (synth.F32, synth.Q8_0):
        m = orc.Model(dict(hp32, kvtype=kvt), w)
        c = orc.Context(m, 1, 8)
        for t in toks:
            c.eval(0, t)
        ctx[kvt] = (m, c)
    hd = hp32["head_dim"]
    worst = 0.0
    for which in (0, 1):
        for p in range(len(toks)):
            for g in range(hp32["n_head_kv"]):
                x = ctx[synth.F32][1].kv_row(which, 0, 0, p, g).astype(np.float64)
                y = ctx[synth.Q8_0][1].kv_row(which, 0, 0, p, g).astype(np.float64)
                for b in range(hd // 32):
                    xb, yb = x[32 * b:32 * b + 32], y[32 * b:32 * b + 32]
                    d = np.abs(xb).max() / 127
                    bound = d * (0.5 + 127 * 2.0 ** -11) * (1 + 1e-6)
                    err = np.abs(xb - yb).max()
                    assert err <= bound, (which, p, g, b, err, bound)
                    worst = max(worst, err / d)
    assert worst > 0.3          # the cache really is quantized
    # the codes themselves: the stored row re-coded from its fp32 source
    x = ctx[synth.F32][1].kv_row(0, 0, 0, 2, 1)
    blocks = orc.quantize(x, synth.Q8_0)
    assert np.array_equal(orc.dequantize(blocks, hd, synth.Q8_0), ctx[synth.Q8_0][1].kv_row(0, 0, 0, 2, 1))


def test_q8_0_cache_rejects_partial_blocks(orc):
    with pytest.raises(ValueError):
        orc.Model(_hp(kvtype=synth.Q8_0, head_dim=16), _weights(_hp(head_dim=16), 1))
