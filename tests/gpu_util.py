"""Helpers for the GPU parity tests: run the same seeded workload through the
HIP library (decode_amd) and the oracle, and compare them."""
from __future__ import annotations

import numpy as np

# acceptance: max-abs logit error <= 2e-2 and <= 1e-2 of the row's largest |logit|
ABS_TOL = 2e-2
REL_TOL = 1e-2


def small_hp(wtype, kvtype, **over):
    hp = dict(n_layer=2, n_embd=256, n_head=4, n_head_kv=2, head_dim=64, n_ff=512,
              n_vocab=640, wtype=wtype, kvtype=kvtype, rms_eps=1e-5, rope_base=10000.0)
    hp.update(over)
    return hp


def logit_err(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    ma = float(np.abs(g - o).max())
    return ma, ma / float(np.abs(o).max())


def assert_logits_close(g, o, what=""):
    ma, rel = logit_err(g, o)
    assert ma <= ABS_TOL and rel <= REL_TOL, f"{what}: max-abs {ma:.3e}, rel {rel:.3e}"
    return ma


def top2_margin(row):
    r = np.sort(np.asarray(row, np.float64))
    return float(r[-1] - r[-2])


def oracle_greedy(om, prompt, n_decode, n_ctx, teacher=None):
    import oracle
    return oracle.run_greedy(om, prompt, n_decode, n_ctx, teacher=teacher)


def gpu_greedy(ctx, prompt, n_decode, seq=0, teacher=None):
    """Prefill + n_decode greedy steps through the C ABI; returns (tokens, logits rows)."""
    rc = ctx.prefill(prompt, seq)
    assert rc == 0, f"dec_prefill returned {rc}"
    toks = [ctx.argmax(-1)]
    rows = [ctx.logits(-1)]
    for k in range(n_decode):
        feed = toks[-1] if teacher is None else int(teacher[k])
        rc = ctx.decode([feed], [seq])
        assert rc == 0, f"dec_decode returned {rc}"
        toks.append(ctx.argmax(0))
        rows.append(ctx.logits(0))
    return toks, rows


def compare_runs(g_toks, g_rows, o_toks, o_rows, what):
    """Teacher-forced rows must agree within tolerance at every step; free-running
    tokens must be identical unless the oracle's top-2 margin at the first
    divergence is below the measured logit error (reported as a near-tie)."""
    worst = 0.0
    for k, (g, o) in enumerate(zip(g_rows, o_rows)):
        worst = max(worst, assert_logits_close(g, o, f"{what} step {k}"))
        assert int(np.argmax(g)) == int(g_toks[k])  # device argmax agrees with its own logits
    return worst
