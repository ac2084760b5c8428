"""Q4_K super-block weights on the device, against the oracle.

* The device quantizer writes the oracle's super-blocks bit for bit (every
  tensor, with zero, constant, one-signed and tie-prone sub-blocks planted).
* Prefill in several ubatches (a ragged last one) and decode steps match the
  oracle's logits within the acceptance bound, teacher-forced, and give the
  oracle's greedy tokens free-running; MHA and GQA, head_dim 64 and 128.
* A vocabulary that is not a whole number of 256-row GEMM tiles takes the
  plain kernel for the output projection and still matches.
* The wide and 256-feature direct-to-LDS GEMM forms agree bitwise, and the
  plain kernel closely (the same arithmetic in another order).
* Several sequences decoded in one call (a GEMM of a few tokens) equal the
  same sequences decoded one at a time.
"""
import os

import numpy as np
import pytest

import synth
from gpu_util import assert_logits_close, compare_runs, gpu_greedy, small_hp

pytestmark = pytest.mark.gpu


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


def test_q4k_blocks_bit_exact(dec, orc):
    hp = small_hp(synth.Q4_K, synth.F16)
    w = synth.weights_numpy(hp, 131, threads=4)
    wq = w["wq"][0]
    wq[0, :256] = 0.0                                       # a zero super-block
    wq[1, :256] = 0.125                                     # constant
    wq[2, :256] = np.abs(wq[2, :256])                       # no negative element
    wq[3, :256] = -np.abs(wq[3, :256])                      # no positive element
    wq[4, :32] = np.arange(32, dtype=np.float32) / 15.0     # codes at exact halves of a step
    wq[5, 32:64] = 1e-8                                     # tiny sub-block beside normal ones
    w["ffn_down"][1][7, :256] *= 1e4                        # large range
    gm = dec.Model(hp, w)
    om = orc.Model(hp, w)
    for name in ("tok_embd", "output"):
        assert np.array_equal(gm.tensor_blocks(name), om.tensor_bytes(name)), name
    for l in range(hp["n_layer"]):
        for name in ("wq", "wk", "wv", "wo", "ffn_gate", "ffn_up", "ffn_down"):
            assert np.array_equal(gm.tensor_blocks(name, l), om.tensor_bytes(name, l)), (name, l)


@pytest.mark.parametrize("hd,H,Hkv", [(64, 8, 2), (128, 4, 4), (128, 8, 1)])
def test_q4k_multi_ubatch_matches_oracle(dec, orc, hd, H, Hkv):
    hp = small_hp(synth.Q4_K, synth.F16, n_embd=512, n_head=H, n_head_kv=Hkv, head_dim=hd, n_ff=1024,
                  n_vocab=2048)
    w = synth.weights_numpy(hp, 140 + hd + H, threads=4)
    prompt = synth.prompt(hp["n_vocab"], 150, 141)
    n_dec = 10
    om = orc.Model(hp, w)
    o_toks, o_rows = orc.run_greedy(om, prompt, n_dec, 512)
    gm = dec.Model(hp, w)
    ctx = dec.Context(gm, n_ctx=512, n_ubatch=64)      # 3 ubatches, ragged tail of 22
    g_toks, g_rows = gpu_greedy(ctx, prompt, n_dec, teacher=o_toks)
    compare_runs(g_toks, g_rows, o_toks, o_rows, f"Q4_K hd {hd} H {H}/{Hkv}")
    ctx.clear(0)
    f_toks, _ = gpu_greedy(ctx, prompt, n_dec)
    assert f_toks == o_toks


def test_q4k_odd_vocab_plain_output_kernel(dec, orc):
    # 1000 output rows: not whole 256-row tiles, so the output projection of
    # the prompt takes the plain kernel
    hp = small_hp(synth.Q4_K, synth.F16, n_vocab=1000)
    w = synth.weights_numpy(hp, 150, threads=4)
    prompt = synth.prompt(hp["n_vocab"], 40, 151)
    om = orc.Model(hp, w)
    oc = orc.Context(om, 1, 128)
    o_rows = [oc.eval(0, int(t)) for t in prompt]
    gm = dec.Model(hp, w)
    ctx = dec.Context(gm, n_ctx=128, n_ubatch=32)
    assert ctx.prefill(prompt, 0, output_all=True) == 0
    for i in (0, 1, 31, 32, 39):
        assert_logits_close(ctx.logits(i), o_rows[i], f"row {i}")


def test_q4k_gemm_forms_agree(dec):
    # wide direct-to-LDS form (512-feature tiles: the gate/up and down
    # matrices here), the 256-feature form (DECODE_GEMM_DW=0), the plain
    # kernel (DECODE_GEMM_DL=0)
    hp = small_hp(synth.Q4_K, synth.F16, n_embd=512, n_ff=1024, n_vocab=2048)
    w = synth.weights_numpy(hp, 160, threads=4)
    prompt = synth.prompt(hp["n_vocab"], 200, 161)
    gm = dec.Model(hp, w)
    rows = {}
    saved = {k: os.environ.get(k) for k in ("DECODE_GEMM_DL", "DECODE_GEMM_DW")}
    try:
        for form, dl, dw in (("wide", "23", "1"), ("256", "23", "0"), ("plain", "0", "1")):
            os.environ["DECODE_GEMM_DL"] = dl
            os.environ["DECODE_GEMM_DW"] = dw
            ctx = dec.Context(gm, n_ctx=256, n_ubatch=128)
            assert ctx.prefill(prompt, 0, output_all=True) == 0
            rows[form] = np.stack([ctx.logits(i) for i in range(len(prompt))]).astype(np.float64)
            del ctx
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    # the two direct-to-LDS forms: the same operands, order and K split
    assert np.array_equal(rows["wide"], rows["256"])
    a, b = rows["wide"], rows["plain"]
    assert np.abs(a).max() > 1e-2
    assert np.abs(a - b).max() <= 1e-4 * np.abs(b).max(), np.abs(a - b).max()


def test_q4k_batched_decode_equals_single_sequences(dec):
    hp = small_hp(synth.Q4_K, synth.F16)
    w = synth.weights_numpy(hp, 170, threads=4)
    gm = dec.Model(hp, w)
    n_seq = 5
    prompts = [synth.prompt(hp["n_vocab"], 20 + 3 * s, 171 + s) for s in range(n_seq)]
    feeds = [synth.prompt(hp["n_vocab"], 4, 181 + s) for s in range(n_seq)]
    single = []
    for s in range(n_seq):
        ctx = dec.Context(gm, n_ctx=128, n_ubatch=32)
        assert ctx.prefill(prompts[s], 0) == 0
        rows = []
        for k in range(4):
            assert ctx.decode([int(feeds[s][k])], [0]) == 0
            rows.append(ctx.logits(0))
        single.append(rows)
    ctx = dec.Context(gm, n_ctx=128, n_ubatch=32, n_seq_max=n_seq)
    for s in range(n_seq):
        assert ctx.prefill(prompts[s], s) == 0
    for k in range(4):
        assert ctx.decode([int(feeds[s][k]) for s in range(n_seq)], list(range(n_seq))) == 0
        for s in range(n_seq):
            assert_logits_close(ctx.logits(s), single[s][k], f"seq {s} step {k}")
