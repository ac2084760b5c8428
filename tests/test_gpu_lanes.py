"""Prefill lanes: the ubatches of one prefill call go round several sets of
activation buffers and streams (DECODE_PREFILL_LANES, default 2), ubatch
u+1's attention at each layer waiting for ubatch u's K/V of that layer.
Each ubatch's arithmetic is the same for any number of lanes, except that
with two or more the wide GEMM form splits K at most 4 ways (8 alone): where
that split is the same, every logits row is bitwise equal across lane
counts, and where it differs the rows agree to rounding.  Rows also meet the
oracle, and the decode steps that follow (on the context's own stream) see
every ubatch's cache rows.
"""
import os

import numpy as np
import pytest

import synth
from gpu_util import assert_logits_close, small_hp

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


def _run(dec, gm, prompt, feed, n_ubatch, lanes, split_at=None):
    key = "DECODE_PREFILL_LANES"
    saved = os.environ.get(key)
    try:
        os.environ[key] = str(lanes)
        ctx = dec.Context(gm, n_ctx=1024, n_batch=len(prompt), n_ubatch=n_ubatch)
    finally:
        if saved is None:
            os.environ.pop(key, None)
        else:
            os.environ[key] = saved
    rows = []
    parts = [prompt] if split_at is None else [prompt[:split_at], prompt[split_at:]]
    for part in parts:
        assert ctx.prefill(part, 0, output_all=True) == 0
        rows += [ctx.logits(i) for i in range(len(part))]
    steps = []
    for t in feed:
        assert ctx.decode([int(t)]) == 0
        steps.append(ctx.logits(0))
    del ctx
    return np.stack(rows), np.stack(steps)


@pytest.mark.parametrize("wtype,kvtype", [(synth.Q4_0, synth.F16), (synth.Q8_0, synth.F16),
                                          (synth.Q4_0, synth.Q8_0)])
def test_lanes_bitwise_equal_one_lane_and_match_oracle(dec, orc, wtype, kvtype):
    # (a Q8_0 cache: each lane codes its ubatch's new K / V from staging rows of its own)
    hp = small_hp(wtype, kvtype, n_layer=3, n_embd=512, n_head=8, n_head_kv=2, n_ff=1024, n_vocab=1024)
    w = synth.weights_numpy(hp, 1410 + wtype + 7 * kvtype, threads=4)
    prompt = synth.prompt(hp["n_vocab"], 600, 1411)           # ubatches 128 x 4 and a ragged 88
    feed = synth.prompt(hp["n_vocab"], 3, 1412)
    gm = dec.Model(hp, w)
    one = _run(dec, gm, prompt, feed, 128, lanes=1)
    two = _run(dec, gm, prompt, feed, 128, lanes=2)
    for k in (3, 4):
        more = _run(dec, gm, prompt, feed, 128, lanes=k)
        assert np.array_equal(one[0], more[0]) and np.array_equal(one[1], more[1]), f"{k} lanes"
    assert np.array_equal(one[0], two[0])
    assert np.array_equal(one[1], two[1])
    # the oracle at the last row of each ubatch and at the decode steps
    oc = orc.Context(orc.Model(hp, w), 1, 1024)
    want = {127, 255, 383, 511, 599}
    for i, t in enumerate(prompt):
        r = oc.eval(0, int(t))
        if i in want:
            assert_logits_close(two[0][i], r, f"prefill row {i}")
    for k, t in enumerate(feed):
        assert_logits_close(two[1][k], oc.eval(0, int(t)), f"decode step {k}")


def test_lanes_over_two_prefill_calls(dec):
    # a second prefill call continues the sequence: its first ubatch attends
    # to the first call's rows written from both lanes
    hp = small_hp(synth.Q4_0, synth.F16, n_layer=2, n_embd=256, n_head=4, n_head_kv=2, n_vocab=640)
    w = synth.weights_numpy(hp, 1420, threads=4)
    prompt = synth.prompt(hp["n_vocab"], 400, 1421)
    feed = synth.prompt(hp["n_vocab"], 2, 1422)
    gm = dec.Model(hp, w)
    one = _run(dec, gm, prompt, feed, 64, lanes=1, split_at=230)
    two = _run(dec, gm, prompt, feed, 64, lanes=2, split_at=230)
    whole = _run(dec, gm, prompt, feed, 64, lanes=2)
    assert np.array_equal(one[0], two[0])
    assert np.array_equal(one[1], two[1])
    # splitting the call moves the ubatch boundaries, so rows agree to rounding
    assert np.abs(two[0] - whole[0]).max() <= 1e-3 * np.abs(whole[0]).max()


def test_lanes_split_cap_rows_agree(dec, orc):
    # the down matrix (K 4096, 512 rows) splits 8 ways with one lane and 4
    # ways with lanes: rows agree to rounding, lanes 2 and 3 bitwise
    hp = small_hp(synth.Q4_0, synth.F16, n_layer=2, n_embd=512, n_head=8, n_head_kv=2, n_ff=4096, n_vocab=1024)
    w = synth.weights_numpy(hp, 1430, threads=4)
    prompt = synth.prompt(hp["n_vocab"], 300, 1431)          # ubatches 128, 128, 44
    feed = synth.prompt(hp["n_vocab"], 2, 1432)
    gm = dec.Model(hp, w)
    one = _run(dec, gm, prompt, feed, 128, lanes=1)
    two = _run(dec, gm, prompt, feed, 128, lanes=2)
    three = _run(dec, gm, prompt, feed, 128, lanes=3)
    assert np.array_equal(two[0], three[0]) and np.array_equal(two[1], three[1])
    scale = np.abs(one[0]).max()
    assert scale > 1e-2
    assert np.abs(one[0] - two[0]).max() <= 1e-4 * scale
    assert np.abs(one[1] - two[1]).max() <= 1e-4 * scale
    oc = orc.Context(orc.Model(hp, w), 1, 1024)
    want = {127, 255, 299}
    for i, t in enumerate(prompt):
        r = oc.eval(0, int(t))
        if i in want:
            assert_logits_close(two[0][i], r, f"prefill row {i}")


def test_lanes_abort_then_continue(dec):
    # an abort between ubatches returns after the lanes are joined: the rows
    # written so far stay, and a later call continues from them
    hp = small_hp(synth.Q4_0, synth.F16)
    w = synth.weights_numpy(hp, 1440, threads=4)
    gm = dec.Model(hp, w)
    p = synth.prompt(hp["n_vocab"], 100, 1441)
    key = "DECODE_PREFILL_LANES"
    saved = os.environ.get(key)
    last = {}
    try:
        for lanes in (1, 2):
            os.environ[key] = str(lanes)
            state = {"calls": 0, "armed": True}

            def abort(ud):
                state["calls"] += 1
                return 1 if state["armed"] and state["calls"] >= 2 else 0

            ctx = dec.Context(gm, n_ctx=256, n_batch=128, n_ubatch=32, abort=abort)
            assert ctx.prefill(p, 0) == 2
            assert ctx.pos_max(0) == 63
            state["armed"] = False                      # no abort during the second call
            assert ctx.prefill(p[64:], 0) == 0
            assert ctx.pos_max(0) == 99
            last[lanes] = ctx.logits(0)
            assert ctx.decode([int(p[0])]) == 0
            last[(lanes, "step")] = ctx.logits(0)
            del ctx
    finally:
        if saved is None:
            os.environ.pop(key, None)
        else:
            os.environ[key] = saved
    assert np.array_equal(last[1], last[2])
    assert np.array_equal(last[(1, "step")], last[(2, "step")])
    whole = dec.Context(gm, n_ctx=256, n_batch=128, n_ubatch=32)
    assert whole.prefill(p, 0) == 0
    ref = whole.logits(0)
    assert np.abs(last[2] - ref).max() <= 1e-4 * np.abs(ref).max()
