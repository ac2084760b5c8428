"""The one-token decode step as one persistent kernel (dec_set_step_kernel).

The step kernel runs every layer of a decode step inside one launch, with
grid barriers between the layer's stages.  It is checked
  * against the oracle: greedy runs over several weight types, head sizes
    and GQA ratios (identical tokens, logits within 2e-2, teacher-forced);
  * against the per-layer kernels on the same GPU (which have their own
    oracle parity): logits within 1e-3 at every step, including contexts
    long enough that the attention's blocks take several rounds of 32-key
    pieces, and a first decode step right after a one-token prompt;
  * for its switch: supported shapes report 1, others -1, and the probe
    role DEC_K_STEP times one launch per step.
"""
import numpy as np
import pytest

import synth
from gpu_util import ABS_TOL, assert_logits_close, gpu_greedy, logit_err, small_hp

pytestmark = pytest.mark.gpu

STEP_TOL = 1e-3   # step kernel vs per-layer kernels: same arithmetic but the attention's merge order


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


def _run(dec, gm, prompt, n, step, n_ctx=256, n_ubatch=32, teacher=None):
    ctx = dec.Context(gm, n_ctx=n_ctx, n_batch=max(len(prompt), 1), n_ubatch=n_ubatch)
    prev = ctx.step_kernel(1 if step else 0)
    assert prev in (0, 1), "the step kernel should cover this shape"
    toks, rows = gpu_greedy(ctx, prompt, n, teacher=teacher)
    ctx.close()
    return toks, rows


@pytest.mark.parametrize("wtype,hd,H,Hkv", [(synth.Q4_0, 64, 4, 2), (synth.Q8_0, 64, 8, 1),
                                            (synth.Q4_0, 128, 4, 4), (synth.Q8_0, 128, 8, 2)])
def test_step_kernel_matches_oracle(dec, orc, wtype, hd, H, Hkv):
    hp = small_hp(wtype, synth.F16, head_dim=hd, n_head=H, n_head_kv=Hkv, n_embd=H * hd)
    w = synth.weights_numpy(hp, 400 + hd + H, threads=4)
    prompt = synth.prompt(hp["n_vocab"], 45, 401)
    om = orc.Model(hp, w)
    o_toks, o_rows = orc.run_greedy(om, prompt, 12, 256)
    g_toks, g_rows = _run(dec, dec.Model(hp, w), prompt, 12, True, teacher=o_toks[:-1])
    for k, (g, o) in enumerate(zip(g_rows, o_rows)):
        assert_logits_close(g, o, f"step {k}")
    f_toks, _ = _run(dec, dec.Model(hp, w), prompt, 12, True)
    assert f_toks == o_toks


@pytest.mark.parametrize("wtype,hd,Hkv,n_prompt", [(synth.Q4_0, 64, 2, 1), (synth.Q8_0, 128, 1, 700),
                                                   (synth.Q4_0, 128, 2, 2500)])
def test_step_kernel_equals_layer_kernels(dec, wtype, hd, Hkv, n_prompt):
    """Same weights, same prompt: the step kernel's logits stay within 1e-3 of
    the per-layer kernels' at every step (teacher-forced on the per-layer
    tokens).  2500 cached positions with one KV head give 79 pieces of 32 keys
    over the blocks of the head: most blocks take two pieces; one KV head at
    hd 128 with 700 positions takes several rounds in one block when the
    device has few compute units."""
    hp = small_hp(wtype, synth.F16, head_dim=hd, n_head=4, n_head_kv=Hkv, n_embd=4 * hd)
    w = synth.weights_numpy(hp, 500 + n_prompt, threads=4)
    gm = dec.Model(hp, w)
    prompt = synth.prompt(hp["n_vocab"], n_prompt, 501)
    n_ctx = n_prompt + 64
    l_toks, l_rows = _run(dec, gm, prompt, 10, False, n_ctx=n_ctx, n_ubatch=256)
    s_toks, s_rows = _run(dec, gm, prompt, 10, True, n_ctx=n_ctx, n_ubatch=256, teacher=l_toks[:-1])
    assert s_toks[0] == l_toks[0]
    for k, (a, b) in enumerate(zip(s_rows, l_rows)):
        ma, _ = logit_err(a, b)
        assert ma <= STEP_TOL, f"step {k}: {ma:.3e}"


def test_long_context_pieces(dec):
    """A context of 12000 positions with one KV head: 375 pieces of 32 keys
    per head spread over the head's blocks (several per block), compared with
    the per-layer kernels."""
    hp = small_hp(synth.Q4_0, synth.F16, head_dim=128, n_head=4, n_head_kv=1, n_embd=512, n_layer=2)
    w = synth.weights_numpy(hp, 600, threads=4)
    gm = dec.Model(hp, w)
    prompt = synth.prompt(hp["n_vocab"], 12000, 601)
    l_toks, l_rows = _run(dec, gm, prompt, 4, False, n_ctx=12288, n_ubatch=512)
    s_toks, s_rows = _run(dec, gm, prompt, 4, True, n_ctx=12288, n_ubatch=512, teacher=l_toks[:-1])
    for k, (a, b) in enumerate(zip(s_rows, l_rows)):
        ma, _ = logit_err(a, b)
        assert ma <= STEP_TOL, f"step {k}: {ma:.3e}"


def test_switch_and_probe(dec):
    hp = small_hp(synth.Q4_0, synth.F16)
    w = synth.weights_numpy(hp, 700, threads=4)
    gm = dec.Model(hp, w)
    ctx = dec.Context(gm, n_ctx=256, n_ubatch=32)
    assert ctx.step_kernel() == 0                      # off by default
    assert ctx.step_kernel(1) == 0 and ctx.step_kernel() == 1
    assert ctx.set_probe(dec.K_STEP, 0) == 0
    prompt = synth.prompt(hp["n_vocab"], 20, 701)
    toks, _ = gpu_greedy(ctx, prompt, 5)
    ms, n = ctx.probe()
    assert n == 5 and ms > 0                           # one timed launch per decode step
    assert ctx.stats()["n_graph_captures"] == 0        # no per-layer graph was needed
    assert ctx.step_kernel(0) == 1 and ctx.step_kernel() == 0
    ctx.close()
    # shapes the kernel does not cover: f32 weights, a Q8_0 cache
    for wt, kt in ((synth.F32, synth.F32), (synth.Q4_0, synth.Q8_0)):
        hp2 = small_hp(wt, kt, n_ff=544 if wt == synth.F32 else 512)
        m2 = dec.Model(hp2, synth.weights_numpy(hp2, 702, threads=4))
        c2 = dec.Context(m2, n_ctx=256, n_ubatch=32)
        assert c2.step_kernel() == -1
        c2.close()
