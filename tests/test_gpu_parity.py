"""GPU-vs-oracle parity of the whole decoder step through the C ABI.

Every case runs the same seeded fp32 weights through libdecode (HIP, gfx950)
and through the oracle, then compares: quantized block bytes bit for bit,
greedy tokens exactly, logits within max-abs 2e-2 and 1e-2 relative to the
row's largest |logit|.  Teacher-forced runs feed both sides the oracle's
tokens so that logits are compared on identical histories.
"""
import numpy as np
import pytest

import synth
from gpu_util import (ABS_TOL, assert_logits_close, compare_runs, gpu_greedy, logit_err,
                      small_hp, top2_margin)

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


@pytest.mark.parametrize("wtype", [synth.Q8_0, synth.Q4_0, synth.F32])
def test_stored_blocks_bit_exact(dec, orc, wtype):
    hp = small_hp(wtype, synth.F16, n_ff=544 if wtype == synth.F32 else 512)
    w = synth.weights_numpy(hp, 31, threads=4)
    # blocks with ties, zeros and extreme values exercise the rounding rules
    w["wq"][0][:4] = 0.0
    w["wq"][0][4, :32] = np.arange(32, dtype=np.float32) - 16
    w["wk"][1][3, :32] = 1e-8
    gm = dec.Model(hp, w)
    om = orc.Model(hp, w)
    for name in ("tok_embd", "output"):
        assert np.array_equal(gm.tensor_blocks(name), om.tensor_bytes(name)), name
    for l in range(hp["n_layer"]):
        for name in ("wq", "wk", "wv", "wo", "ffn_gate", "ffn_up", "ffn_down"):
            assert np.array_equal(gm.tensor_blocks(name, l), om.tensor_bytes(name, l)), (name, l)


def test_tiny_workload_matches_oracle(dec, orc):
    """2 layers, d 256, fp32 weights and KV: 16-token prompt, 16 greedy steps."""
    W = synth.WORKLOADS["tiny"]
    hp = synth.hparams(W)
    w = synth.weights_numpy(hp, W["seed"], threads=4)
    prompt = synth.prompt(hp["n_vocab"], W["n_prompt"], 2001)
    om = orc.Model(hp, w)
    o_toks, o_rows = orc.run_greedy(om, prompt, W["n_decode"], 256)
    gm = dec.Model(hp, w)
    ctx = dec.Context(gm, n_ctx=256, n_ubatch=W["n_ubatch"])
    g_toks, g_rows = gpu_greedy(ctx, prompt, W["n_decode"], teacher=o_toks)
    compare_runs(g_toks, g_rows, o_toks, o_rows, "tiny teacher-forced")
    ctx.clear(0)
    f_toks, f_rows = gpu_greedy(ctx, prompt, W["n_decode"])
    assert f_toks == o_toks
    st = ctx.stats()
    # first step of the shape eager, second captured, the rest replayed
    assert st["n_graph_captures"] == 1 and st["n_graph_replays"] == 2 * W["n_decode"] - 2


@pytest.mark.parametrize("wtype,hd,H,Hkv", [(synth.Q8_0, 64, 8, 2), (synth.Q4_0, 64, 8, 2),
                                           (synth.Q4_0, 128, 4, 4), (synth.Q8_0, 128, 8, 1)])
def test_quantized_multi_ubatch_matches_oracle(dec, orc, wtype, hd, H, Hkv):
    """Prefill in 3 ubatches (the last one ragged) then decode steps; covers MHA
    and GQA groups of 4 and 8, head_dim 64 and 128."""
    hp = small_hp(wtype, synth.F16, n_embd=512, n_head=H, n_head_kv=Hkv, head_dim=hd, n_ff=1024,
                  n_vocab=2048)
    w = synth.weights_numpy(hp, 40 + wtype, threads=4)
    prompt = synth.prompt(hp["n_vocab"], 150, 41)
    n_dec = 12
    om = orc.Model(hp, w)
    o_toks, o_rows = orc.run_greedy(om, prompt, n_dec, 512)
    gm = dec.Model(hp, w)
    ctx = dec.Context(gm, n_ctx=512, n_ubatch=64)      # 3 ubatches, ragged tail of 22
    g_toks, g_rows = gpu_greedy(ctx, prompt, n_dec, teacher=o_toks)
    compare_runs(g_toks, g_rows, o_toks, o_rows, f"wtype {wtype}")
    ctx.clear(0)
    f_toks, _ = gpu_greedy(ctx, prompt, n_dec)
    assert f_toks == o_toks


def test_output_all_rows_and_indices(dec, orc):
    hp = small_hp(synth.Q8_0, synth.F16)
    w = synth.weights_numpy(hp, 50, threads=4)
    prompt = synth.prompt(hp["n_vocab"], 70, 51)
    om = orc.Model(hp, w)
    oc = orc.Context(om, 1, 256)
    o_rows = [oc.eval(0, int(t)) for t in prompt]
    gm = dec.Model(hp, w)
    ctx = dec.Context(gm, n_ctx=256, n_ubatch=32)
    assert ctx.prefill(prompt, 0, output_all=True) == 0
    for i in (0, 1, 31, 32, 33, 63, 64, 69):
        assert_logits_close(ctx.logits(i), o_rows[i], f"row {i}")
        assert ctx.argmax(i) == int(np.argmax(ctx.logits(i)))
    assert np.array_equal(ctx.logits(-1), ctx.logits(69))
    assert ctx.logits(70) is None and ctx.argmax(70) == -1
    am = ctx.argmax_all()
    assert am.size == 70 and am[5] == ctx.argmax(5)


def test_decode_equals_recompute_on_gpu(dec):
    hp = small_hp(synth.Q4_0, synth.F16)
    w = synth.weights_numpy(hp, 60, threads=4)
    prompt = synth.prompt(hp["n_vocab"], 40, 61)
    gm = dec.Model(hp, w)
    ctx = dec.Context(gm, n_ctx=256, n_ubatch=64)
    toks, rows = gpu_greedy(ctx, prompt, 10)
    full = np.concatenate([prompt, np.array(toks[:-1], np.int32)])
    ctx2 = dec.Context(gm, n_ctx=256, n_ubatch=64)
    assert ctx2.prefill(full, 0) == 0
    ma, _ = logit_err(ctx2.logits(-1), rows[-1])
    assert ma <= ABS_TOL
    assert ctx2.argmax(-1) == toks[-1]


def test_batched_decode_equals_single_sequences(dec, orc):
    hp = small_hp(synth.Q8_0, synth.F16)
    w = synth.weights_numpy(hp, 70, threads=4)
    gm = dec.Model(hp, w)
    om = orc.Model(hp, w)
    S = 5
    prompts = [synth.prompt(hp["n_vocab"], 20 + 3 * s, 300 + s) for s in range(S)]
    ctx = dec.Context(gm, n_ctx=256, n_ubatch=32, n_seq_max=S)
    for s in range(S):
        assert ctx.prefill(prompts[s], s) == 0
    oc = orc.Context(om, S, 256)
    for s in range(S):
        for t in prompts[s]:
            oc.eval(s, int(t), want_logits=False)
    # feed every sequence the same fixed tokens for 4 steps, all sequences in one call
    feeds = synth.prompt(hp["n_vocab"], 4 * S, 77).reshape(4, S)
    for k in range(4):
        assert ctx.decode(feeds[k], np.arange(S)) == 0
        for s in range(S):
            ol = oc.eval(s, int(feeds[k][s]))
            assert_logits_close(ctx.logits(s), ol, f"step {k} seq {s}")
    assert [ctx.pos_max(s) for s in range(S)] == [len(prompts[s]) + 3 for s in range(S)]


def test_return_codes_and_rollback(dec):
    hp = small_hp(synth.Q8_0, synth.F16)
    w = synth.weights_numpy(hp, 80, threads=4)
    gm = dec.Model(hp, w)
    ctx = dec.Context(gm, n_ctx=256, n_batch=256, n_ubatch=32)
    p = synth.prompt(hp["n_vocab"], 200, 81)
    assert ctx.prefill(p, 0) == 0 and ctx.pos_max(0) == 199
    assert ctx.prefill(p[:100], 0) == 1 and ctx.pos_max(0) == 199     # no room: nothing changes
    assert ctx.prefill([hp["n_vocab"]], 0) == -1                        # token out of range
    assert ctx.prefill(p[:5], 1) == -1                                  # seq out of range
    assert ctx.decode([1, 2], [0, 0]) == -1                             # duplicate sequence
    calls = []

    def abort(ud):
        calls.append(1)
        return 1 if len(calls) >= 2 else 0

    ctx2 = dec.Context(gm, n_ctx=256, n_ubatch=32, abort=abort)
    assert ctx2.prefill(p[:100], 0) == 2
    assert ctx2.pos_max(0) == 63            # two ubatches of 32 finished and kept
    ctx2.clear(0)
    assert ctx2.pos_max(0) == -1


def test_eager_decode_equals_graph_decode_and_probe_counts(dec):
    hp = small_hp(synth.Q4_0, synth.F16)
    w = synth.weights_numpy(hp, 90, threads=4)
    gm = dec.Model(hp, w)
    prompt = synth.prompt(hp["n_vocab"], 33, 91)
    a = dec.Context(gm, n_ctx=256, n_ubatch=16)
    b = dec.Context(gm, n_ctx=256, n_ubatch=16)
    assert b.use_graphs(False) is True
    assert a.set_probe(dec.K_FFN_GU, 1) == 0 and b.set_probe(dec.K_ATTN, 0) == 0
    ta, ra = gpu_greedy(a, prompt, 6)
    tb, rb = gpu_greedy(b, prompt, 6)
    assert ta == tb
    for x, y in zip(ra, rb):
        assert np.array_equal(x, y)        # same kernels, same order: bitwise equal
    ms, n = a.probe()
    assert n == 3 + 6 and ms > 0           # 3 prefill ubatches + 6 decode steps
    ms, n = b.probe()
    assert n == 3 + 6 and ms > 0
    assert a.stats()["n_graph_captures"] == 1 and b.stats()["n_graph_captures"] == 0


@pytest.mark.parametrize("kvtype", [synth.F16, synth.Q8_0])
def test_decode_merge_over_chunk_rounds_matches_prefill_rows(dec, kvtype):
    # decode attention splits the keys into 64-key chunks and merges their
    # partials; the merge loads the first 128 chunks at once and takes
    # further rounds of 64 past them.  Decode steps at positions whose chunk
    # counts sit at each edge (1, 64, 65, 128, 129, 130, 193) must give the
    # rows that prefilling the same tokens gives (flash attention, no merge
    # of decode partials).
    hp = small_hp(synth.Q8_0, kvtype, n_layer=2, n_embd=256, n_head=4, n_head_kv=2, n_vocab=512)
    w = synth.weights_numpy(hp, 1450 + kvtype, threads=4)
    targets = [63, 4095, 4096, 8191, 8192, 8255, 8256, 12345]
    n = targets[-1] + 1
    prompt = synth.prompt(hp["n_vocab"], n, 1451)
    gm = dec.Model(hp, w)
    piece = 4096
    a = dec.Context(gm, n_ctx=12544, n_batch=piece, n_ubatch=512)
    steps, done = {}, 0
    for t in targets:
        for s in range(done, t, piece):
            assert a.prefill(prompt[s:min(t, s + piece)], 0) == 0
        assert a.decode([int(prompt[t])]) == 0
        steps[t] = a.logits(0)
        done = t + 1
    assert a.pos_max(0) == targets[-1]
    a.close()
    b = dec.Context(gm, n_ctx=12544, n_batch=piece, n_ubatch=512)
    rows = {}
    for s in range(0, n, piece):
        assert b.prefill(prompt[s:min(n, s + piece)], 0, output_all=True) == 0
        for t in targets:
            if s <= t < s + piece:
                rows[t] = b.logits(t - s)
    b.close()
    for t in targets:
        ma, rel = logit_err(steps[t], rows[t])
        print(f"position {t} ({t // 64 + 1} chunks): max-abs {ma:.3e} rel {rel:.3e}")
        assert rel <= 1e-4, (t, ma, rel)


def test_largest_context_and_row(dec, orc):
    # the limits the header states: a context of DEC_MAX_CTX positions
    # (decode merges 1024 chunks there) and an FFN row of DEC_MAX_ROW
    # elements (the down mat-vec's whole LDS image, K 16384 in the GEMMs)
    max_ctx, max_row = 65536, 16384
    hp = small_hp(synth.Q4_0, synth.F16, n_layer=1, n_embd=256, n_head=4, n_head_kv=2, n_ff=max_row,
                  n_vocab=512)
    w = synth.weights_numpy(hp, 1460, threads=4)
    prompt = synth.prompt(hp["n_vocab"], max_ctx, 1461)
    gm = dec.Model(hp, w)
    piece = 8192
    # b: the whole context as prefill; its first rows against the oracle
    b = dec.Context(gm, n_ctx=max_ctx, n_batch=piece, n_ubatch=512)
    assert b.prefill(prompt[:5], 0, output_all=True) == 0
    oc = orc.Context(orc.Model(hp, w), 1, 16)
    for i in range(5):
        assert_logits_close(b.logits(i), oc.eval(0, int(prompt[i])), f"row {i}")
    for s in range(5, max_ctx, piece):
        assert b.prefill(prompt[s:min(max_ctx, s + piece)], 0) == 0
    assert b.pos_max(0) == max_ctx - 1
    want = b.logits(-1)
    assert b.prefill(prompt[:1], 0) == 1          # full: nothing changes
    assert b.pos_max(0) == max_ctx - 1
    b.close()
    # a: all but the last position as prefill, the last one as a decode step
    a = dec.Context(gm, n_ctx=max_ctx, n_batch=piece, n_ubatch=512)
    for s in range(0, max_ctx - 1, piece):
        assert a.prefill(prompt[s:min(max_ctx - 1, s + piece)], 0) == 0
    assert a.decode([int(prompt[-1])]) == 0
    got = a.logits(0)
    assert a.pos_max(0) == max_ctx - 1
    assert a.decode([int(prompt[0])]) == 1        # no room for another position
    a.close()
    ma, rel = logit_err(got, want)
    print(f"position {max_ctx - 1}: decode vs prefill max-abs {ma:.3e} rel {rel:.3e}")
    # the two paths add 65536 keys' fp32 terms in different orders (1024
    # chunk partials and a merge, against 64-key tiles in at most 8 key
    # ranges); measured 4.3e-5
    assert rel <= 2e-4, (ma, rel)
