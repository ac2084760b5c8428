"""Pins for the oracle's RMSNorm, mat-vec, RoPE, attention, SwiGLU and argmax.

Checked against closed forms, invariants and brute force, never against a
retyped copy of the oracle's own formula.
"""
import math

import numpy as np
import pytest


@pytest.mark.parametrize("kind", ["f64", "f32"])
def test_rmsnorm_closed_forms(orc, kind):
    # [3, 4] with eps 0: mean square 12.5 -> y = x / sqrt(12.5)
    y = orc.rmsnorm([3.0, 4.0], np.ones(2, np.float32), 0.0, kind)
    assert np.allclose(y, [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=1e-6)
    rng = np.random.default_rng(1)
    x = rng.standard_normal(4096) * 0.7
    g1 = np.ones(4096, np.float32)
    y = orc.rmsnorm(x, g1, 1e-5, kind).astype(np.float64)
    ms = np.mean(x * x)
    assert abs(np.mean(y * y) - ms / (ms + 1e-5)) < (1e-12 if kind == "f64" else 2e-6)
    # scale invariance when mean square >> eps
    y2 = orc.rmsnorm(x * 1000.0, g1, 1e-5, kind).astype(np.float64)
    assert np.allclose(y, y2, rtol=1e-4, atol=1e-6)
    # gains multiply elementwise
    g = rng.uniform(0.5, 2, 4096).astype(np.float32)
    yg = orc.rmsnorm(x, g, 1e-5, kind).astype(np.float64)
    assert np.allclose(yg, y * g, rtol=1e-5 if kind == "f32" else 1e-12)
    # eps sits inside the root: zero input gives zero, tiny input is damped
    assert np.all(orc.rmsnorm(np.zeros(8), np.ones(8, np.float32), 1e-5, kind) == 0)


def test_matvec_identity_and_library(orc):
    rng = np.random.default_rng(2)
    x = rng.standard_normal(96)
    eye = np.eye(96, dtype=np.float32)
    assert np.array_equal(orc.matvec(orc.T_F32, eye, 96, 96, x), x)
    # quantized: equals a dense product with the dequantized matrix
    for wt in (orc.T_Q8_0, orc.T_Q4_0):
        W = rng.standard_normal((40, 256)).astype(np.float32) * 0.02
        blocks = orc.quantize(W, wt)
        Wd = orc.dequantize(blocks, W.size, wt).reshape(W.shape).astype(np.float64)
        y = orc.matvec(wt, blocks, 40, 256, x[:96].repeat(3)[:256])
        assert np.allclose(y, Wd @ x[:96].repeat(3)[:256], rtol=1e-12, atol=1e-14)


def test_matvec_f32_vs_f64_accumulation(orc):
    rng = np.random.default_rng(3)
    K = 14336
    W = (rng.standard_normal((64, K)) * 0.02).astype(np.float32)
    b = orc.quantize(W, orc.T_Q4_0)
    x = rng.standard_normal(K)
    y64 = orc.matvec(orc.T_Q4_0, b, 64, K, x, "f64")
    y32 = orc.matvec(orc.T_Q4_0, b, 64, K, x.astype(np.float32), "f32").astype(np.float64)
    scale = np.abs(y64).max()
    assert np.abs(y64 - y32).max() <= 1e-5 * scale


@pytest.mark.parametrize("kind", ["f64", "f32"])
def test_rope_pins(orc, kind):
    rng = np.random.default_rng(4)
    hd, H = 128, 3
    v = rng.standard_normal(H * hd)
    # p = 0 is the identity
    assert np.array_equal(orc.rope(v, H, hd, 0, 10000.0, kind), v.astype(orc.real_dtype(kind)))
    # per-pair norm preserved
    r = orc.rope(v, H, hd, 777, 10000.0, kind).astype(np.float64)
    n0 = np.hypot(v[0::2], v[1::2])
    n1 = np.hypot(r[0::2], r[1::2])
    assert np.allclose(n0, n1, rtol=1e-14 if kind == "f64" else 1e-6)
    # pair 0 turns by exactly pos radians; pair i by pos * base^(-2i/hd)
    e = np.zeros(hd)
    e[0] = 1.0
    e[2 * 5] = 1.0
    r = orc.rope(e, 1, hd, 3, 10000.0, kind).astype(np.float64)
    assert np.allclose(r[0:2], [math.cos(3), math.sin(3)], atol=1e-6 if kind == "f32" else 1e-15)
    th = 3 * 10000.0 ** (-10 / hd)
    assert np.allclose(r[10:12], [math.cos(th), math.sin(th)], atol=1e-6 if kind == "f32" else 1e-15)
    # relative position: <R(m)q, R(n)k> depends only on m - n
    q = rng.standard_normal(hd)
    k = rng.standard_normal(hd)
    a = np.dot(orc.rope(q, 1, hd, 100, 1e4, kind), orc.rope(k, 1, hd, 37, 1e4, kind))
    b = np.dot(orc.rope(q, 1, hd, 8000, 1e4, kind), orc.rope(k, 1, hd, 7937, 1e4, kind))
    assert abs(a - b) <= (1e-9 if kind == "f64" else 2e-4) * np.linalg.norm(q) * np.linalg.norm(k)


def _dense_attention(q, K, V, row_pos, pos):
    """Brute force: one [n] score row in double with an explicit -inf mask."""
    s = (K.astype(np.float64) @ q) / math.sqrt(q.size)
    s = np.where(row_pos <= pos, s, -np.inf)
    e = np.exp(s - s.max())
    w = e / e.sum()
    return w @ V.astype(np.float64), w


def _q8_blocks_to_f64(b):
    """Q8_0 block bytes -> values, read straight from the block format (f16
    little-endian scale, then 32 int8 codes)."""
    blk = np.frombuffer(np.ascontiguousarray(b, np.uint8).tobytes(), np.uint8).reshape(-1, 34)
    d = blk[:, :2].copy().view("<f2").astype(np.float64)
    codes = blk[:, 2:].view(np.int8).astype(np.float64)
    return (codes * d).ravel()


@pytest.mark.parametrize("kvtype", ["f32", "f16", "q8_0"])
def test_attention_brute_force(orc, kvtype):
    rng = np.random.default_rng(5)
    n, hd = 37, 64
    q = rng.standard_normal(hd)
    K = rng.standard_normal((n, hd)).astype(np.float32)
    V = rng.standard_normal((n, hd)).astype(np.float32)
    rp = rng.permutation(n).astype(np.int32)          # cells in any order
    pos = 20
    ld = None
    if kvtype == "f16":
        Kb, Vb, t = orc.f16_from_f32(K), orc.f16_from_f32(V), orc.T_F16
        K, V = orc.f16_to_f32(Kb), orc.f16_to_f32(Vb)
    elif kvtype == "q8_0":
        Kb, Vb, t, ld = orc.quantize(K, orc.T_Q8_0), orc.quantize(V, orc.T_Q8_0), orc.T_Q8_0, hd
        K, V = _q8_blocks_to_f64(Kb).reshape(n, hd), _q8_blocks_to_f64(Vb).reshape(n, hd)
    else:
        Kb, Vb, t = K, V, orc.T_F32
    o, w = orc.attend(q, Kb, Vb, t, pos, row_pos=rp, ld=ld, n=n)
    o_ref, w_ref = _dense_attention(q, K, V, rp, pos)
    assert np.allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    assert np.allclose(w, w_ref, rtol=1e-12, atol=0)
    assert abs(w.sum() - 1) < 1e-12
    assert np.all(w[rp > pos] == 0)                   # masked cells get exactly 0


def test_attention_single_row_and_stride(orc):
    rng = np.random.default_rng(6)
    hd = 128
    q = rng.standard_normal(hd)
    V = rng.standard_normal((1, hd)).astype(np.float32)
    K = rng.standard_normal((1, hd)).astype(np.float32)
    o, w = orc.attend(q, K, V, orc.T_F32, 0)
    assert np.array_equal(o, V[0].astype(np.float64)) and w[0] == 1.0
    # a row stride larger than hd (several heads per cached row) reads the right slice
    n = 9
    KK = rng.standard_normal((n, 3 * hd)).astype(np.float32)
    VV = rng.standard_normal((n, 3 * hd)).astype(np.float32)
    o_s, _ = orc.attend(q, KK.ravel()[hd:], VV.ravel()[hd:], orc.T_F32, n, ld=3 * hd, n=n)
    o_ref, _ = _dense_attention(q, KK[:, hd:2 * hd], VV[:, hd:2 * hd], np.arange(n), n)
    assert np.allclose(o_s, o_ref, rtol=1e-12)
    # the same with a Q8_0 cache: the middle head starts hd/32 blocks into each row
    Kq, Vq = orc.quantize(KK, orc.T_Q8_0), orc.quantize(VV, orc.T_Q8_0)
    skip = hd // 32 * 34
    o_q, _ = orc.attend(q, Kq[skip:], Vq[skip:], orc.T_Q8_0, n, ld=3 * hd, n=n)
    Kd = _q8_blocks_to_f64(Kq).reshape(n, 3 * hd)
    Vd = _q8_blocks_to_f64(Vq).reshape(n, 3 * hd)
    o_ref, _ = _dense_attention(q, Kd[:, hd:2 * hd], Vd[:, hd:2 * hd], np.arange(n), n)
    assert np.allclose(o_q, o_ref, rtol=1e-12)


def test_attention_f32_build_sums_to_one(orc):
    rng = np.random.default_rng(8)
    q = rng.standard_normal(128) * 4
    K = rng.standard_normal((500, 128)).astype(np.float32)
    o, w = orc.attend(q, K, K, orc.T_F32, 499, kind="f32")
    assert abs(float(w.astype(np.float64).sum()) - 1) < 1e-5


def test_swiglu_pins(orc):
    u = np.array([0.0, 1.0, 40.0, -40.0, 0.0])
    v = np.array([3.0, 2.0, 1.5, 7.0, 0.0])
    h = orc.swiglu(u, v)
    assert h[0] == 0.0
    assert abs(h[1] - 2.0 / (1 + math.exp(-1))) < 1e-15
    assert abs(h[2] - 40 * 1.5) < 1e-12                # large gate -> gate * up
    assert abs(h[3]) < 1e-12                           # large negative gate -> 0
    # silu(u) = u * sigmoid(u); torch's silu agrees
    import torch
    uu = np.random.default_rng(9).standard_normal(1000) * 5
    ref = torch.nn.functional.silu(torch.from_numpy(uu)).numpy()
    assert np.allclose(orc.swiglu(uu, np.ones(1000)), ref, rtol=1e-12, atol=1e-15)


def test_argmax_ties(orc):
    assert orc.argmax([1.0, 3.0, 3.0, 2.0]) == 1
    assert orc.argmax([-5.0]) == 0
    x = np.random.default_rng(10).standard_normal(32000)
    assert orc.argmax(x) == int(np.argmax(x))
