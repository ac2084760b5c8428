"""Operand modes of the ubatch GEMM (prefill and batched decode) against the oracle.

By default every ubatch takes exact operands (integer codes, activations as
f16 value + remainder, per-block scale applied in fp32).  With
DECODE_GEMM_F16=1 (read when a context is created) ubatches of more than 64
tokens take f16 operands instead: each weight enters the matrix cores as its
dequantized value d * code rounded to f16 and each activation as its f16
value, with fp32 accumulation; from 256 tokens on a block covers 256 tokens.
At this small shape both modes meet the oracle bar on every output row of a
300-token ubatch (a full 256-token tile and a ragged 44-token tile), and they
differ, which shows that the switch took effect.  (At the 8B shape the f16
mode does not meet the bar, which is why it is opt-in.)
"""
import numpy as np
import pytest

import synth
from gpu_util import assert_logits_close, logit_err, small_hp

pytestmark = pytest.mark.gpu

ROWS = (0, 1, 63, 64, 255, 256, 257, 299)


@pytest.fixture(scope="module")
def dec():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_amd
    decode_amd.lib()
    return decode_amd


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.load("f64")
    return oracle


def _rows(dec, gm, prompt, n_ubatch):
    ctx = dec.Context(gm, n_ctx=512, n_batch=len(prompt), n_ubatch=n_ubatch)
    assert ctx.prefill(prompt, 0, output_all=True) == 0
    rows = {i: np.array(ctx.logits(i)) for i in ROWS}
    am = {i: ctx.argmax(i) for i in ROWS}
    ctx.close()
    return rows, am


@pytest.mark.parametrize("wtype", [synth.Q4_0, synth.Q8_0])
def test_both_operand_modes_match_oracle(dec, orc, wtype, monkeypatch):
    hp = small_hp(wtype, synth.F16)
    w = synth.weights_numpy(hp, 900 + wtype, threads=4)
    prompt = synth.prompt(hp["n_vocab"], 300, 901)
    oc = orc.Context(orc.Model(hp, w), 1, 512)
    o_rows = {}
    for i, t in enumerate(prompt):
        r = oc.eval(0, int(t))
        if i in ROWS:
            o_rows[i] = r
    gm = dec.Model(hp, w)
    got = {}
    for exact in (False, True):
        monkeypatch.setenv("DECODE_GEMM_F16", "0" if exact else "1")
        rows, am = _rows(dec, gm, prompt, 300)
        for i in ROWS:
            assert_logits_close(rows[i], o_rows[i], f"exact={exact} row {i}")
            assert am[i] == int(np.argmax(rows[i]))
        got[exact] = rows
    monkeypatch.delenv("DECODE_GEMM_F16")
    diff = max(logit_err(got[False][i], got[True][i])[0] for i in ROWS)
    assert 0.0 < diff < 1e-2, f"modes differ by {diff:.3e}"


def test_small_ubatch_exact_in_both_modes(dec, monkeypatch):
    """Ubatches of at most 64 tokens take exact operands whatever the switch says."""
    hp = small_hp(synth.Q4_0, synth.F16)
    w = synth.weights_numpy(hp, 910, threads=4)
    prompt = synth.prompt(hp["n_vocab"], 300, 911)
    gm = dec.Model(hp, w)
    got = []
    for exact in (False, True):
        monkeypatch.setenv("DECODE_GEMM_F16", "0" if exact else "1")
        got.append(_rows(dec, gm, prompt, 64)[0])
    monkeypatch.delenv("DECODE_GEMM_F16")
    for i in ROWS:
        assert np.array_equal(got[0][i], got[1][i]), f"row {i}"


@pytest.mark.parametrize("wtype", [synth.Q4_0, synth.Q8_0])
def test_skinny_form_matches_tiles_and_oracle(dec, orc, wtype, monkeypatch):
    """With DECODE_GEMM_SMALL=tiles, ubatches of at most 32 tokens take the
    skinny form (wavefronts stream their own weight rows, K ranges over
    blocks); DECODE_GEMM_SKINNY=0 sends them through the tiled kernel instead.
    Same exact operands, different summation order: rows within 1e-3 of each
    other and within the oracle bar, on a 45-token prompt in ubatches of 32 (a
    full and a ragged 13-token one)."""
    hp = small_hp(wtype, synth.F16, n_embd=512, n_head=8, n_ff=1024)
    w = synth.weights_numpy(hp, 920 + wtype, threads=4)
    prompt = synth.prompt(hp["n_vocab"], 45, 921)
    oc = orc.Context(orc.Model(hp, w), 1, 256)
    o_rows = [oc.eval(0, int(t)) for t in prompt]
    gm = dec.Model(hp, w)
    got = {}
    monkeypatch.setenv("DECODE_GEMM_SMALL", "tiles")
    for skinny in (True, False):
        monkeypatch.setenv("DECODE_GEMM_SKINNY", "1" if skinny else "0")
        ctx = dec.Context(gm, n_ctx=256, n_batch=45, n_ubatch=32)
        assert ctx.prefill(prompt, 0, output_all=True) == 0
        got[skinny] = [np.array(ctx.logits(i)) for i in range(45)]
        ctx.close()
    monkeypatch.delenv("DECODE_GEMM_SKINNY")
    monkeypatch.delenv("DECODE_GEMM_SMALL")
    for i in (0, 1, 31, 32, 44):
        assert_logits_close(got[True][i], o_rows[i], f"skinny row {i}")
        ma, _ = logit_err(got[True][i], got[False][i])
        assert ma <= 1e-3, f"row {i}: skinny vs tiles {ma:.3e}"


@pytest.mark.parametrize("wtype", [synth.Q4_0, synth.Q8_0])
def test_direct_load_form_bitwise_equals_staged_tiles(dec, orc, wtype, monkeypatch):
    """Ubatches of more than 64 tokens on matrices of whole 256-feature tiles
    take the direct-to-LDS form (DECODE_GEMM_DL = 3 or 4 stages on 32x32
    tiles, 23 with 64-feature wavefront tiles, 13 on 16x16 tiles; 0 keeps the
    register-staged tiles); Q4_0 and Q8_0 matrices of whole 512-feature tiles
    take the wide form unless DECODE_GEMM_DW=0 (here the gate/up and QKV
    matrices, whose K of 8 blocks is two periods of code super-stages).  On
    32x32 tiles all these forms feed the matrix cores the same operands in the same
    order and, at this shape, split K the same way (not at all), so every
    logits row of a 300-token ubatch (token tiles of 128, 128 and a ragged 44)
    is bitwise equal across them; the 16x16x32 MFMA sums a quant block in one
    instruction, so there the rows agree to rounding.  All meet the oracle bar."""
    hp = small_hp(wtype, synth.F16)
    w = synth.weights_numpy(hp, 930 + wtype, threads=4)
    prompt = synth.prompt(hp["n_vocab"], 300, 931)
    oc = orc.Context(orc.Model(hp, w), 1, 512)
    o_rows = {}
    for i, t in enumerate(prompt):
        r = oc.eval(0, int(t))
        if i in ROWS:
            o_rows[i] = r
    gm = dec.Model(hp, w)
    got = {}
    monkeypatch.setenv("DECODE_GEMM_DW", "0")
    for ns in ("0", "3", "4", "23", "13"):
        monkeypatch.setenv("DECODE_GEMM_DL", ns)
        got[ns] = _rows(dec, gm, prompt, 300)[0]
    monkeypatch.delenv("DECODE_GEMM_DL")
    monkeypatch.delenv("DECODE_GEMM_DW")
    wide = ("dw",)
    got["dw"] = _rows(dec, gm, prompt, 300)[0]
    for i in ROWS:
        for ns in ("3", "13") + wide:
            assert_logits_close(got[ns][i], o_rows[i], f"direct-load {ns} row {i}")
        for ns in ("3", "4", "23") + wide:
            assert np.array_equal(got[ns][i], got["0"][i]), f"variant {ns}, row {i}"
        for ns in ("13",):
            assert logit_err(got[ns][i], got["0"][i])[0] <= 1e-4, f"16x16 tiles ({ns}), row {i}"


@pytest.mark.parametrize("wtype", [synth.Q4_0, synth.Q8_0])
def test_small_direct_load_form_matches_tiles_and_oracle(dec, orc, wtype, monkeypatch):
    """Ubatches of at most 32 tokens on matrices of whole 256-feature tiles
    take the direct-to-LDS form with 32-token block tiles (4, 6 or 8 stages,
    DECODE_GEMM_DLS_NS; K split into possibly uneven ranges: the down matrix
    here has 41 K blocks).  Against the skinny / tiled kernels
    (DECODE_GEMM_SMALL=tiles): the same exact operands in another summation
    order, so rows agree to 1e-3; every form meets the oracle bar on a
    45-token prompt in ubatches of 32 (a full and a ragged 13-token one)."""
    hp = small_hp(wtype, synth.F16, n_embd=512, n_head=8, n_ff=1312, n_vocab=1024)
    w = synth.weights_numpy(hp, 940 + wtype, threads=4)
    prompt = synth.prompt(hp["n_vocab"], 45, 941)
    oc = orc.Context(orc.Model(hp, w), 1, 256)
    o_rows = [oc.eval(0, int(t)) for t in prompt]
    gm = dec.Model(hp, w)
    got = {}
    monkeypatch.setenv("DECODE_GEMM_WS", "0")
    for form in ("tiles", "4", "6", "8"):
        if form == "tiles":
            monkeypatch.setenv("DECODE_GEMM_SMALL", "tiles")
        else:
            monkeypatch.delenv("DECODE_GEMM_SMALL", raising=False)
            monkeypatch.setenv("DECODE_GEMM_DLS_NS", form)
        ctx = dec.Context(gm, n_ctx=256, n_batch=45, n_ubatch=32)
        assert ctx.prefill(prompt, 0, output_all=True) == 0
        got[form] = [np.array(ctx.logits(i)) for i in range(45)]
        ctx.close()
    monkeypatch.delenv("DECODE_GEMM_SMALL", raising=False)
    monkeypatch.delenv("DECODE_GEMM_DLS_NS", raising=False)
    monkeypatch.delenv("DECODE_GEMM_WS", raising=False)
    for i in (0, 1, 12, 31, 32, 44):
        for form in ("tiles", "4", "6", "8"):
            assert_logits_close(got[form][i], o_rows[i], f"{form} row {i}")
        for form in ("4", "6", "8"):
            ma, _ = logit_err(got[form][i], got["tiles"][i])
            assert ma <= 1e-3, f"row {i}: 32-token direct-load ({form} stages) vs tiles {ma:.3e}"
        # the stage count changes only the pipelining, not the arithmetic
        assert np.array_equal(got["4"][i], got["6"][i]) and np.array_equal(got["4"][i], got["8"][i])


def test_weight_streaming_form_matches_oracle(dec, orc, monkeypatch):
    """Q4_0 ubatches of at most 32 tokens on matrices of whole 256-feature
    tiles with K a multiple of 256 take the weight-streaming form (2 K blocks
    per stage by default, DECODE_GEMM_WS=4 for 4; the split's scales loaded
    once; K split in whole octets of K blocks, unevenly where K = 768 is three
    octets).  Against the 32-token direct-to-LDS form (DECODE_GEMM_WS=0): the
    same operands and per-block scaling in another K split, so rows agree to
    1e-3; every form meets the oracle bar on a 45-token prompt in ubatches of
    32, and on five sequences decoded in one call."""
    hp = small_hp(synth.Q4_0, synth.F16, n_embd=768, n_head=12, n_head_kv=4, n_ff=1024, n_vocab=1024)
    w = synth.weights_numpy(hp, 950, threads=4)
    prompt = synth.prompt(hp["n_vocab"], 45, 951)
    om = orc.Model(hp, w)
    oc = orc.Context(om, 1, 256)
    o_rows = [oc.eval(0, int(t)) for t in prompt]
    gm = dec.Model(hp, w)
    got = {}
    for form in ("0", "2", "4"):
        monkeypatch.setenv("DECODE_GEMM_WS", form)
        ctx = dec.Context(gm, n_ctx=256, n_batch=45, n_ubatch=32)
        assert ctx.prefill(prompt, 0, output_all=True) == 0
        got[form] = [np.array(ctx.logits(i)) for i in range(45)]
        ctx.close()
    for i in (0, 1, 12, 31, 32, 44):
        for form in ("0", "2", "4"):
            assert_logits_close(got[form][i], o_rows[i], f"form {form} row {i}")
        for form in ("2", "4"):
            ma, _ = logit_err(got[form][i], got["0"][i])
            assert ma <= 1e-3, f"row {i}: streaming ({form} K blocks per stage) vs 32-token direct-load {ma:.3e}"
    # five sequences, one decode call of five tokens (M = 5)
    monkeypatch.setenv("DECODE_GEMM_WS", "2")
    S = 5
    prompts = [synth.prompt(hp["n_vocab"], 10 + 2 * s, 960 + s) for s in range(S)]
    feeds = synth.prompt(hp["n_vocab"], S, 970)
    ctx = dec.Context(gm, n_ctx=128, n_batch=32, n_ubatch=32, n_seq_max=S)
    for s in range(S):
        assert ctx.prefill(prompts[s], s) == 0
    assert ctx.decode([int(t) for t in feeds], list(range(S))) == 0
    for s in range(S):
        oc = orc.Context(om, 1, 128)
        for t in prompts[s]:
            oc.eval(0, int(t))
        assert_logits_close(ctx.logits(s), oc.eval(0, int(feeds[s])), f"sequence {s}")
    ctx.close()
    monkeypatch.delenv("DECODE_GEMM_WS")
