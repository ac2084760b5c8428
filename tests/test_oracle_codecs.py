"""Pins for the oracle's f16 conversion and Q8_0 / Q4_0 / Q4_K block codecs.

Each pin checks the oracle against something other than itself: numpy's own
IEEE half conversion, exhaustive enumeration, hand-worked blocks under
tests/golden/, brute-force nearest-code search, and error bounds that follow
from the block definitions.
"""
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _fixture(name):
    blocks, cur = [], {}
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, v = line.split(":", 1)
        cur[k.strip()] = v.split()
        if k.strip() in ("scale_f16", "y"):
            blocks.append(cur)
            cur = {}
    return blocks


# ------------------------------------------------------------------ f16
def test_f16_exhaustive_roundtrip(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = orc.f16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(f[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.isnan(f[nan]).all()
    back = orc.f16_from_f32(f)
    assert np.array_equal(back[~nan], h[~nan])


@pytest.mark.filterwarnings("ignore:overflow encountered")
def test_f16_random_vs_numpy(orc):
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    assert np.array_equal(orc.f16_from_f32(x), x.astype(np.float16).view(np.uint16))
    y = (rng.standard_normal(500_000) * 10.0 ** rng.integers(-9, 6, 500_000)).astype(np.float32)
    assert np.array_equal(orc.f16_from_f32(y), y.astype(np.float16).view(np.uint16))


@pytest.mark.filterwarnings("ignore:overflow encountered")
def test_f16_ties_and_edges(orc):
    # every midpoint between consecutive finite halves (ties to even), the
    # subnormal range, the overflow threshold and signed zeros
    h = np.arange(0, 0x7bff, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)          # exact in f32
    xs = np.concatenate([mid, -mid, np.float32([0.0, -0.0, 65504, 65519.99, 65520, 1e-8,
                                               2.0 ** -25, 2.0 ** -24, 3 * 2.0 ** -26, np.inf,
                                               -np.inf])]).astype(np.float32)
    assert np.array_equal(orc.f16_from_f32(xs), xs.astype(np.float16).view(np.uint16))


def test_f16_from_f64_single_rounding(orc):
    L = orc.load("f64")
    rng = np.random.default_rng(3)
    xs = rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 5, 20000)
    # values a hair above a half-way point: rounding through f32 first would tie-break wrongly
    h = np.arange(0x0400, 0x7000, 97, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    xs = np.concatenate([xs, (lo + hi) / 2 + (hi - lo) * 2.0 ** -40])
    got = np.array([L.orc_f16_from_f64(float(v)) for v in xs], np.uint16)
    assert np.array_equal(got, xs.astype(np.float16).view(np.uint16))


# ------------------------------------------------------------------ Q8_0
def test_q8_0_golden(orc):
    for blk in _fixture("q8_0_halfway.txt"):
        x = np.array(blk["x"], np.float32)
        b = orc.quantize(x, orc.T_Q8_0)
        assert b.size == 34
        assert int(b[0]) | int(b[1]) << 8 == int(blk["scale_f16"][0], 16)
        assert np.array_equal(b[2:].view(np.int8), np.array(blk["codes"], np.int8))


def test_q8_0_properties(orc):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((4000, 32)) * rng.uniform(1e-3, 10, (4000, 1))).astype(np.float32)
    x[5] = 0.0
    b = orc.quantize(x, orc.T_Q8_0).reshape(-1, 34)
    q = b[:, 2:].view(np.int8).astype(np.int32)
    d16 = b[:, :2].copy().view(np.uint16)[:, 0]
    dh = d16.view(np.float16).astype(np.float64)
    # (iii) zero block
    assert d16[5] == 0 and (q[5] == 0).all()
    nz = np.abs(x).max(1) > 0
    # (i) the largest element maps to +-127
    am = np.abs(x).argmax(1)
    assert (np.abs(q[nz, am[nz]]) == 127).all()
    assert (np.abs(q).max(1)[nz] == 127).all()
    # (iv) brute force: each code is the integer nearest to x/d with the fp32
    # d = amax/127, ties away from zero
    d = (np.abs(x).max(1) / np.float32(127)).astype(np.float32)
    idv = np.where(d != 0, np.float32(1) / np.where(d != 0, d, 1), 0).astype(np.float32)
    t = (x * idv[:, None]).astype(np.float32).astype(np.float64)
    cand = np.arange(-127, 128)
    dist = np.abs(t[..., None] - cand)
    best = cand[dist.argmin(-1)]
    tie = np.isclose(dist.min(-1), 0.5, atol=0) & (np.sort(dist, -1)[..., 1] == 0.5)
    best = np.where(tie, np.sign(t) * np.ceil(np.abs(t)), best)
    assert np.array_equal(q, best.astype(np.int32))
    # (ii) reconstruction bound |x - xhat| <= d/2 + 127*|d - fp16(d)| (+ ulp slack)
    y = orc.dequantize(b.ravel(), x.size, orc.T_Q8_0).reshape(x.shape).astype(np.float64)
    bound = d / 2 + 127 * np.abs(d.astype(np.float64) - dh) + 1e-6 * np.abs(x).max(1)
    assert (np.abs(x - y) <= bound[:, None]).all()
    # decode rule: y = q * f32(f16(d))
    assert np.array_equal(y, q * dh[:, None])


# ------------------------------------------------------------------ Q4_0
def test_q4_0_golden(orc):
    (blk,) = _fixture("q4_0_ramp.txt")
    x = np.array(blk["x"], np.float32)
    b = orc.quantize(x, orc.T_Q4_0)
    assert b.tolist() == [int(v, 16) for v in blk["bytes"]]
    y = orc.dequantize(b, 32, orc.T_Q4_0)
    assert y.tolist() == [float(v) for v in blk["y"]]


def test_q4_0_properties(orc):
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((4000, 32)) * rng.uniform(1e-3, 10, (4000, 1))).astype(np.float32)
    x[7] = 0.0
    b = orc.quantize(x, orc.T_Q4_0).reshape(-1, 18)
    d16 = b[:, :2].copy().view(np.uint16)[:, 0]
    dh = d16.view(np.float16).astype(np.float64)
    lo = (b[:, 2:] & 0x0F).astype(np.int32)
    hi = (b[:, 2:] >> 4).astype(np.int32)
    code = np.concatenate([lo, hi], 1)
    # (iii) zero block -> all codes 8 (bytes 0x88), scale +-0 (m/-8 of m = 0 is -0)
    assert (d16[7] & 0x7FFF) == 0 and (b[7, 2:] == 0x88).all()
    nz = np.abs(x).max(1) > 0
    # (i) the signed-max element encodes to 0 and decodes to m up to f16(d)
    am = np.abs(x).argmax(1)
    assert (code[nz, am[nz]] == 0).all()
    m = x[np.arange(len(x)), am].astype(np.float64)
    y = orc.dequantize(b.ravel(), x.size, orc.T_Q4_0).reshape(x.shape).astype(np.float64)
    assert np.allclose(y[nz, am[nz]], m[nz], rtol=2e-3, atol=0)
    # (ii) error bound; the clamped top code (x within |m|/16 of -m) gets |d|
    d = (m / -8.0).astype(np.float32).astype(np.float64)
    err = np.abs(x - y)
    fp16_term = 8 * np.abs(d - dh)
    clamp = (code == 15) & ((x.astype(np.float64) / np.where(d != 0, d, 1)[:, None]) > 7.0)
    bound = np.where(clamp, np.abs(d)[:, None], np.abs(d)[:, None] / 2) + fp16_term[:, None] \
        + 1e-6 * np.abs(x).max(1)[:, None]
    assert (err <= bound).all()
    # brute force: each code is the nearest level (code-8)*d to x with ties
    # going up, clamped to 15
    t = x.astype(np.float64) / np.where(d != 0, d, 1)[:, None]
    cand = np.arange(0, 16)
    dist = np.abs(t[..., None] + 8 - cand)
    best = cand[dist.argmin(-1)]
    near_tie = np.abs(np.abs(t + 8 - np.floor(t + 8)) - 0.5) < 1e-4
    ok = (best == code) | near_tie | ~nz[:, None]
    assert ok.all()


# ------------------------------------------------------------------ Q4_K
def test_q4_k_golden(orc):
    (blk,) = _fixture("q4_k_block.txt")
    x = np.array(blk["x"], np.float32)
    b = orc.quantize(x, orc.T_Q4_K)
    assert b.size == 144
    assert b[:16].tolist() == [int(v, 16) for v in blk["header"]]
    assert b[16:].tolist() == [int(v, 16) for v in blk["codes"]]
    sc, m = orc.q4_k_scales(b)
    assert sc.tolist() == [10, 63, 1, 30, 16, 47, 2, 55]
    assert m.tolist() == [63, 0, 5, 17, 33, 48, 1, 20]
    y = orc.dequantize(b, 256, orc.T_Q4_K)
    assert y.tolist() == [float(v) for v in blk["y"]]


def _q4_k_fields(orc, b):
    """Per super-block d, dmin (as fp64), sub-block sc, m and the 256 codes."""
    b = b.reshape(-1, 144)
    d = b[:, 0:2].copy().view(np.float16)[:, 0].astype(np.float64)
    dmin = b[:, 2:4].copy().view(np.float16)[:, 0].astype(np.float64)
    sc = np.empty((len(b), 8), np.int64)
    m = np.empty((len(b), 8), np.int64)
    for i in range(len(b)):
        s_, m_ = orc.q4_k_scales(b[i])
        sc[i], m[i] = s_, m_
    qs = b[:, 16:].reshape(-1, 4, 32)
    code = np.empty((len(b), 4, 2, 32), np.int64)
    code[:, :, 0, :] = qs & 15
    code[:, :, 1, :] = qs >> 4
    return d, dmin, sc, m, code.reshape(-1, 8, 32)


def test_q4_k_properties(orc):
    rng = np.random.default_rng(21)
    nb = 1500
    x = rng.standard_normal((nb, 8, 32)) * rng.uniform(1e-3, 10, (nb, 1, 1))
    x *= rng.uniform(0.05, 1.0, (nb, 8, 1))                # uneven sub-block ranges
    x += rng.uniform(-1, 1, (nb, 8, 1)) * np.abs(x).max((1, 2), keepdims=True) * 0.5
    x[3] = 0.0                                             # zero super-block
    x[4] = np.abs(x[4])                                    # no negative element
    x[5] = -np.abs(x[5])                                   # no positive element
    x[6, :, :] = 0.25                                      # constant
    x = x.astype(np.float32)
    b = orc.quantize(x, orc.T_Q4_K)
    y = orc.dequantize(b, x.size, orc.T_Q4_K).reshape(x.shape).astype(np.float64)
    d, dmin, sc, m, code = _q4_k_fields(orc, b)
    xd = x.astype(np.float64)
    # (i) an all-zero super-block encodes to 144 zero bytes and decodes to zeros
    assert (b.reshape(-1, 144)[3] == 0).all() and (y[3] == 0).all()
    # (ii) a super-block without negative elements needs no min
    assert (m[4] == 0).all() and dmin[4] == 0
    # (iii) the decode rule, element by element, from the unpacked fields
    step = d[:, None] * sc
    mf = dmin[:, None] * m
    assert np.allclose(y, code * step[..., None] - mf[..., None], rtol=0, atol=1e-6 * np.abs(xd).max())
    # (iv) the largest sub-block scale and min use the six-bit range (62 or 63;
    # 62 when the f16 rounding of d or dmin went up)
    nzr = np.abs(x).max((1, 2)) > 0
    assert (sc.max(1)[nzr] >= 62).all()
    neg = x.min((1, 2)) < 0
    assert (m.max(1)[neg] >= 62).all()
    # (v) every element within half a step of its decoded value, apart from the
    # slack that a clamped six-bit scale or min leaves (s_j > step_j, mn_j > mf_j)
    lo, hi = xd.min(2), xd.max(2)
    s_need = np.maximum(0, (hi + mf) / 15)
    mn_need = np.maximum(0, -lo)
    slack = 15 * np.maximum(0, s_need - step) + np.maximum(0, mn_need - mf)
    bound = step / 2 + slack + 1e-6 * np.maximum(np.abs(xd).max(2), 1e-30)
    assert (np.abs(xd - y) <= bound[..., None]).all()
    # (vi) brute force: each code is the nearest of the 16 levels c*step - mf
    # (away from exact ties)
    lev = np.arange(16)[None, None, None, :] * step[..., None, None] - mf[..., None, None]
    dist = np.abs(xd[..., None] - lev)
    best = dist.argmin(-1)
    srt = np.sort(dist, -1)
    tie = (srt[..., 1] - srt[..., 0]) <= 1e-5 * np.maximum(step[..., None], 1e-30)
    zero_step = (step == 0)[..., None]
    assert ((best == code) | tie | zero_step).all()


def test_q4_k_sub_block_addressing(orc):
    # each sub-block's scale/min must land on its own 32 elements: a block whose
    # sub-block j is the constant j+1 (all others untouched) decodes sub-block
    # j to within half a step of j+1 and the rest to zero
    for j in range(8):
        x = np.zeros(256, np.float32)
        x[32 * j:32 * j + 32] = j + 1
        b = orc.quantize(x, orc.T_Q4_K)
        y = orc.dequantize(b, 256, orc.T_Q4_K)
        sc, m = orc.q4_k_scales(b)
        assert sc[j] == 63 and (np.delete(sc, j) == 0).all() and (m == 0).all()
        assert np.abs(y[32 * j:32 * j + 32] - (j + 1)).max() <= (j + 1) / 15 / 2 * 1.01
        assert (np.delete(y, np.s_[32 * j:32 * j + 32]) == 0).all()


def test_codecs_reject_ragged(orc):
    L = orc.load()
    x = np.zeros(33, np.float32)
    assert L.orc_q8_0_quantize(x.ctypes.data, 33, None) == -1
    assert L.orc_q4_0_quantize(x.ctypes.data, 33, None) == -1
    x = np.zeros(288, np.float32)
    assert L.orc_q4_k_quantize(x.ctypes.data, 288, None) == -1
