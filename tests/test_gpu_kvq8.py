"""Q8_0 KV cache through the C ABI against the oracle's Q8_0 cache.

Each cached head row is coded in 32-element Q8_0 blocks as it is appended
(both sides code the fp32 K / V values with the weights' Q8_0 definition),
and attention reads code * scale.  The two sides compute K / V in different
precisions (fp32 on the device, fp64 in the oracle), so an occasional code
differs by one step; the comparison is the usual logit tolerance, and greedy
tokens must agree.
"""
import numpy as np
import pytest

import synth
from gpu_util import assert_logits_close, compare_runs, gpu_greedy, logit_err, small_hp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dec():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_amd
    decode_amd.lib()
    return decode_amd


@pytest.mark.parametrize("wtype,hd,H,Hkv", [(synth.Q4_0, 128, 8, 2), (synth.Q8_0, 64, 8, 8),
                                           (synth.Q8_0, 64, 8, 1), (synth.F32, 64, 4, 2)])
def test_q8_cache_multi_ubatch_matches_oracle(dec, orc, wtype, hd, H, Hkv):
    """Prefill in 3 ubatches (the last one ragged), then decode steps (the
    second and later replayed from a captured graph)."""
    hp = small_hp(wtype, synth.Q8_0, n_embd=512, n_head=H, n_head_kv=Hkv, head_dim=hd,
                  n_ff=1024 if wtype != synth.F32 else 1000, n_vocab=2048)
    w = synth.weights_numpy(hp, 140 + wtype, threads=4)
    prompt = synth.prompt(hp["n_vocab"], 150, 141)
    n_dec = 12
    om = orc.Model(hp, w)
    o_toks, o_rows = orc.run_greedy(om, prompt, n_dec, 512)
    gm = dec.Model(hp, w)
    ctx = dec.Context(gm, n_ctx=512, n_ubatch=64)
    g_toks, g_rows = gpu_greedy(ctx, prompt, n_dec, teacher=o_toks)
    compare_runs(g_toks, g_rows, o_toks, o_rows, f"q8 cache, wtype {wtype}")
    ctx.clear(0)
    f_toks, _ = gpu_greedy(ctx, prompt, n_dec)
    assert f_toks == o_toks
    assert ctx.stats()["n_graph_replays"] > 0


def test_q8_cache_differs_from_f16_cache(dec, orc):
    """The cache type reaches the arithmetic: Q8_0 and f16 caches give logits
    that differ by far more than the f16 run's own error, on both sides, and
    by about the same amount."""
    base = small_hp(synth.Q8_0, synth.F16)
    w = synth.weights_numpy(base, 150, threads=4)
    prompt = synth.prompt(base["n_vocab"], 60, 151)
    rows = {}
    for kvt in (synth.F16, synth.Q8_0):
        hp = dict(base, kvtype=kvt)
        om = orc.Model(hp, w)
        o_toks, o_rows = orc.run_greedy(om, prompt, 3, 256)
        ctx = dec.Context(dec.Model(hp, w), n_ctx=256, n_ubatch=32)
        g_toks, g_rows = gpu_greedy(ctx, prompt, 3, teacher=o_toks)
        for g, o in zip(g_rows, o_rows):
            assert_logits_close(g, o, f"kvtype {kvt}")
        rows[kvt] = (np.asarray(g_rows[-1], np.float64), np.asarray(o_rows[-1], np.float64))
    g_gap = np.abs(rows[synth.Q8_0][0] - rows[synth.F16][0]).max()
    o_gap = np.abs(rows[synth.Q8_0][1] - rows[synth.F16][1]).max()
    own = logit_err(rows[synth.F16][0], rows[synth.F16][1])[0]
    assert o_gap > 5 * own and g_gap > 5 * own
    assert abs(g_gap - o_gap) <= 0.25 * o_gap


def test_q8_cache_batched_decode(dec, orc):
    """Five sequences decoded together in one call, each against its own
    oracle sequence."""
    hp = small_hp(synth.Q4_0, synth.Q8_0)
    w = synth.weights_numpy(hp, 160, threads=4)
    gm = dec.Model(hp, w)
    om = orc.Model(hp, w)
    S = 5
    prompts = [synth.prompt(hp["n_vocab"], 20 + 7 * s, 400 + s) for s in range(S)]
    ctx = dec.Context(gm, n_ctx=256, n_ubatch=32, n_seq_max=S)
    for s in range(S):
        assert ctx.prefill(prompts[s], s) == 0
    oc = orc.Context(om, S, 256)
    for s in range(S):
        for t in prompts[s]:
            oc.eval(s, int(t), want_logits=False)
    feeds = synth.prompt(hp["n_vocab"], 5 * S, 161).reshape(5, S)
    for k in range(5):
        assert ctx.decode(feeds[k], np.arange(S)) == 0
        for s in range(S):
            assert_logits_close(ctx.logits(s), oc.eval(s, int(feeds[k][s])), f"step {k} seq {s}")


def test_q8_cache_gguf_load(dec, orc, tmp_path):
    """A model loaded from a GGUF file with a Q8_0 cache runs like the same
    model built from fp32 weights."""
    hp = small_hp(synth.Q4_0, synth.Q8_0)
    w = synth.weights_numpy(hp, 170, threads=4)
    gm = dec.Model(hp, w)
    path = tmp_path / "m.gguf"
    gm.save_gguf(path)
    lm = dec.Model.from_gguf(path, kvtype=synth.Q8_0)
    prompt = synth.prompt(hp["n_vocab"], 40, 171)
    res = []
    for m in (gm, lm):
        ctx = dec.Context(m, n_ctx=128, n_ubatch=16)
        res.append(gpu_greedy(ctx, prompt, 4))
        ctx.close()
    assert res[0][0] == res[1][0]
    for a, b in zip(res[0][1], res[1][1]):
        assert np.array_equal(np.asarray(a), np.asarray(b))


@pytest.mark.parametrize("hd,H,Hkv", [(128, 8, 2), (64, 8, 8)])
def test_q8_cache_flash_prefill_matches_splitk_and_oracle(dec, orc, hd, H, Hkv):
    """Prefill ubatches over a Q8_0 cache take the flash kernel, whose K and V
    tiles hold code * scale as f16 value + remainder (exact); the split-K
    decode kernels (DECODE_PREFILL_ATTN=splitk) read the codes directly.
    Every logits row of a 600-token prompt (ubatches of 128: key ranges split
    over blocks, a ragged last ubatch) agrees between the two to rounding,
    and rows at each ubatch's end meet the oracle."""
    import os
    hp = small_hp(synth.Q4_0, synth.Q8_0, n_layer=2, n_embd=H * hd, n_head=H, n_head_kv=Hkv, head_dim=hd,
                  n_ff=1024, n_vocab=1024)
    w = synth.weights_numpy(hp, 160 + hd, threads=4)
    prompt = synth.prompt(hp["n_vocab"], 600, 161)
    gm = dec.Model(hp, w)
    rows = {}
    saved = os.environ.get("DECODE_PREFILL_ATTN")
    try:
        for form in ("flash", "splitk"):
            if form == "splitk":
                os.environ["DECODE_PREFILL_ATTN"] = "splitk"
            else:
                os.environ.pop("DECODE_PREFILL_ATTN", None)
            ctx = dec.Context(gm, n_ctx=1024, n_batch=600, n_ubatch=128)
            assert ctx.prefill(prompt, 0, output_all=True) == 0
            rows[form] = np.stack([ctx.logits(i) for i in range(len(prompt))]).astype(np.float64)
            del ctx
    finally:
        if saved is None:
            os.environ.pop("DECODE_PREFILL_ATTN", None)
        else:
            os.environ["DECODE_PREFILL_ATTN"] = saved
    a, b = rows["flash"], rows["splitk"]
    assert np.abs(a).max() > 1e-2
    assert np.abs(a - b).max() <= 1e-4 * np.abs(b).max(), np.abs(a - b).max()
    oc = orc.Context(orc.Model(hp, w), 1, 1024)
    for i, t in enumerate(prompt):
        r = oc.eval(0, int(t))
        if i in (127, 255, 383, 511, 599):
            assert_logits_close(a[i], r, f"flash q8 row {i}")
