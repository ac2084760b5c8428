"""GPU-vs-oracle parity of the sampler chain (penalty, top-k, top-p, min-p,
temperature, draw) through the C ABI.

Both sides draw u from the same counter-based generator (SplitMix64 of the
seed and the draw index), so every draw is compared token for token.  The
candidate set and its order are decided by integer keys (exact on both
sides); the weights are fp32 sums of expf on both sides, whose last bits can
differ between the device and the host C library.  A differing token is
therefore accepted only when u falls within 1e-5 of the total weight of a
cumulative boundary of the oracle's candidate list, where such a one-ulp
difference can move the draw to a neighbour -- and at most once per case.
Greedy selection (temperature 0 or top-k 1) must match exactly.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

BOUNDARY_REL = 1e-5


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


def near_boundary(orc, row, hist, prm, draw, g_tok):
    """True when the oracle's draw lies within BOUNDARY_REL of a cumulative
    boundary next to its pick and the device token is that neighbour (or the
    candidate one past a top-p / min-p cut)."""
    o_tok, ids, cum, t = orc.sample(row, hist, draw=draw, detail=True, **prm)
    if len(ids) == 0:
        return False
    tot = float(cum[-1])
    ids = list(ids)
    if g_tok in ids:
        a, b = sorted((ids.index(o_tok), ids.index(g_tok)))
        if b - a != 1:
            return False
        return abs(float(cum[a]) - t) <= BOUNDARY_REL * tot
    # the device kept one candidate more than the oracle at a top-p / min-p cut
    full = dict(prm, top_p=1.0, min_p=0.0)
    _, fids, _, _ = orc.sample(row, hist, draw=draw, detail=True, **full)
    fids = list(fids)
    return g_tok in fids and fids.index(g_tok) == len(ids)


def run_case(dec, orc, rows, prm, hist0=(), on_device=False, max_boundary=1):
    """Samples every row in turn with one Sampler (history and draw counter
    carried along) and compares each token with the oracle's."""
    import torch
    s = dec.Sampler(**prm)
    hist = [int(t) for t in hist0]
    s.accept(hist)
    n_boundary = 0
    try:
        for d, row in enumerate(rows):
            row = np.ascontiguousarray(row, np.float32)
            if on_device:
                g = s.sample_row(torch.from_numpy(row).cuda(), torch.cuda.current_stream().cuda_stream)
            else:
                g = s.sample_row(row)
            assert g >= 0, f"dec_sampler_sample_row returned {g}"
            o = orc.sample(row, hist, draw=d, **prm)
            if g != o:
                assert prm["temp"] > 0 and prm["top_k"] > 1, f"draw {d}: greedy mismatch {g} vs {o}"
                assert near_boundary(orc, row, hist, prm, d, g), f"draw {d}: {g} vs oracle {o}, not a boundary case"
                n_boundary += 1
            hist.append(g)
        assert s.draws() == len(rows)
    finally:
        s.close()
    assert n_boundary <= max_boundary, f"{n_boundary} boundary mismatches"
    return n_boundary


def tie_rows(n, seed):
    """Vocabulary 16 with logits drawn from 4 values: many exact ties."""
    r = np.random.default_rng(seed)
    vals = np.array([-1.0, 0.0, 0.5, 1.0], np.float32)
    return [vals[r.integers(0, 4, 16)] for _ in range(n)]


def vocab_rows(n, V, seed, scale=3.0):
    r = np.random.default_rng(seed)
    return [(r.standard_normal(V) * scale).astype(np.float32) for _ in range(n)]


P_DEFAULT = dict(top_k=40, top_p=0.95, min_p=0.05, temp=0.8, repeat_penalty=1.0, penalty_last_n=64, seed=7)


@pytest.mark.parametrize("prm", [
    dict(top_k=16, top_p=1.0, min_p=0.0, temp=1.0, repeat_penalty=1.0, penalty_last_n=64, seed=1),
    dict(top_k=5, top_p=0.7, min_p=0.0, temp=0.5, repeat_penalty=1.0, penalty_last_n=64, seed=2),
    dict(top_k=12, top_p=1.0, min_p=0.5, temp=2.0, repeat_penalty=1.0, penalty_last_n=64, seed=3),
    dict(top_k=16, top_p=0.9, min_p=0.1, temp=1.0, repeat_penalty=1.5, penalty_last_n=8, seed=4),
])
def test_vocab16_ties(dec, orc, prm):
    """Tied logits: the lower id must win every tie in the cut and the order."""
    run_case(dec, orc, tie_rows(300, 11), prm, hist0=[3, 3, 15, 0])


def test_vocab16_draw_frequencies(dec, orc):
    """Many draws on one row: the empirical frequencies follow the softmax of
    the kept candidates (a check that does not go through the oracle)."""
    row = np.array([2.0, 1.0, 1.0, 0.0, -1.0] + [-30.0] * 11, np.float32)
    prm = dict(top_k=16, top_p=1.0, min_p=0.0, temp=1.0, repeat_penalty=1.0, penalty_last_n=64, seed=99)
    s = dec.Sampler(**prm)
    n = 4000
    try:
        toks = [s.sample_row(row) for _ in range(n)]
    finally:
        s.close()
    p = np.exp(row.astype(np.float64) - row.max())
    p /= p.sum()
    f = np.bincount(toks, minlength=16) / n
    assert np.all(np.abs(f - p) <= 4 * np.sqrt(p * (1 - p) / n) + 1e-3), (f, p)


@pytest.mark.parametrize("prm", [
    P_DEFAULT,
    dict(top_k=1024, top_p=1.0, min_p=0.0, temp=1.5, repeat_penalty=1.0, penalty_last_n=64, seed=8),
    dict(top_k=1024, top_p=0.5, min_p=0.0, temp=1.0, repeat_penalty=1.0, penalty_last_n=64, seed=9),
    dict(top_k=200, top_p=1.0, min_p=0.3, temp=0.7, repeat_penalty=1.0, penalty_last_n=64, seed=10),
    dict(top_k=40, top_p=0.95, min_p=0.05, temp=0.8, repeat_penalty=1.3, penalty_last_n=64, seed=11),
])
def test_vocab32000(dec, orc, prm):
    """LLaMA's vocabulary size, logits ~ N(0, 3^2), host and device rows."""
    rows = vocab_rows(40, 32000, 21)
    run_case(dec, orc, rows[:20], prm, hist0=np.arange(0, 32000, 977))
    run_case(dec, orc, rows[20:], prm, hist0=[5, 5, 31999], on_device=True)


def test_penalty_hits_the_leader(dec, orc):
    """History holding the row's top tokens (positive and negative logits)
    changes the ranking: the penalty must be applied once per distinct token."""
    prm = dict(top_k=8, top_p=1.0, min_p=0.0, temp=0.0, repeat_penalty=1.8, penalty_last_n=64, seed=0)
    r = np.random.default_rng(5)
    rows = []
    for _ in range(30):
        x = (r.standard_normal(32000) * 2).astype(np.float32)
        x[:4] = [9.0, 8.5, -0.5, 8.0]
        rows.append(x)
    run_case(dec, orc, rows, prm, hist0=[0, 0, 0, 1, 2, 2])


def test_dense_ties_and_minus_inf(dec, orc):
    """Rows whose nearest logits are too many to compact (all equal, a few
    integer values over 32000 tokens) take the exact radix-select path; -inf
    entries must never be drawn unless nothing else is left."""
    r = np.random.default_rng(9)
    rows = [np.zeros(32000, np.float32),
            r.integers(-3, 4, 32000).astype(np.float32),
            r.integers(0, 2, 32000).astype(np.float32)]
    x = (r.standard_normal(32000) * 3).astype(np.float32)
    x[r.integers(0, 32000, 20000)] = -np.inf
    rows.append(x)
    for prm in (dict(top_k=40, top_p=0.9, min_p=0.0, temp=1.0, repeat_penalty=1.0, penalty_last_n=64, seed=13),
                dict(top_k=1024, top_p=1.0, min_p=0.0, temp=1.0, repeat_penalty=1.3, penalty_last_n=64, seed=14),
                dict(top_k=7, top_p=1.0, min_p=0.2, temp=0.0, repeat_penalty=1.0, penalty_last_n=64, seed=15)):
        run_case(dec, orc, rows * 3, prm, hist0=[0, 1, 2, 31999])


@pytest.mark.parametrize("V", [1, 2, 1023, 32768])
def test_vocab_edges(dec, orc, V):
    k = min(V, 1024)
    prm = dict(top_k=k, top_p=0.9, min_p=0.0, temp=1.0, repeat_penalty=1.1, penalty_last_n=16, seed=12)
    run_case(dec, orc, vocab_rows(10, V, 31 + V), prm, hist0=[0])


def test_greedy_is_argmax(dec, orc):
    """temp 0: the leader of the penalised row, exactly; top-k 1 likewise."""
    rows = vocab_rows(20, 32000, 41, scale=1.0)
    for r in rows[::4]:
        r[100:110] = r.max() + 1.0          # a 10-way tie at the top: lowest id wins
    for prm in (dict(top_k=40, top_p=0.9, min_p=0.1, temp=0.0, repeat_penalty=1.0, penalty_last_n=64, seed=0),
                dict(top_k=1, top_p=1.0, min_p=0.0, temp=1.0, repeat_penalty=1.0, penalty_last_n=64, seed=5)):
        s = dec.Sampler(**prm)
        try:
            for r in rows:
                assert s.sample_row(r) == int(np.argmax(r))
        finally:
            s.close()


def test_bad_arguments(dec):
    s = dec.Sampler(top_k=40)
    try:
        assert s.sample_row(np.zeros(32769, np.float32)) == -1      # above the LDS row bound
        assert s.sample_row(np.zeros(20, np.float32)) == -1         # top_k > n_vocab
        assert s.draws() == 0
    finally:
        s.close()
    with pytest.raises(Exception):
        dec.Sampler(top_k=0)
    with pytest.raises(Exception):
        dec.Sampler(top_k=2000)
    with pytest.raises(Exception):
        dec.Sampler(top_p=0.0)
    with pytest.raises(Exception):
        dec.Sampler(penalty_last_n=65)


def test_sampling_from_the_decoder(dec, orc):
    """The chain on the context's own logits: prefill, then sampled decode
    steps, each token drawn on the device from the output row and fed back."""
    W = synth.WORKLOADS["tiny"]
    hp = synth.hparams(W)
    w = synth.weights_numpy(hp, W["seed"], threads=4)
    prompt = synth.prompt(hp["n_vocab"], W["n_prompt"], 2002)
    gm = dec.Model(hp, w)
    ctx = dec.Context(gm, n_ctx=256, n_ubatch=W["n_ubatch"])
    prm = dict(top_k=40, top_p=0.95, min_p=0.05, temp=0.9, repeat_penalty=1.2, penalty_last_n=32, seed=77)
    s = dec.Sampler(**prm)
    hist = list(prompt)
    s.accept(hist)
    n_boundary = 0
    try:
        assert ctx.prefill(prompt, 0) == 0
        for d in range(24):
            row = ctx.logits(-1 if d == 0 else 0)
            g = s.sample(ctx, -1 if d == 0 else 0)
            o = orc.sample(row, hist, draw=d, **prm)
            if g != o:
                assert near_boundary(orc, row, hist, prm, d, g), f"step {d}: {g} vs {o}"
                n_boundary += 1
            hist.append(g)
            assert ctx.decode([g], [0]) == 0
    finally:
        s.close()
        ctx.close()
        gm.close()
    assert n_boundary <= 1
