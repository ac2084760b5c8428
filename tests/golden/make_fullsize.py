"""Writes the stored oracle results for the full-size parity tests.

For each case of ``fullsize_cases.py``: weights from ``synth.weights_numpy``,
the f64 oracle (``oracle/``) prefills the prompt token by token (logits kept
for the listed rows), then runs the greedy decode steps, feeding back its own
argmax.  Output: ``fullsize_<case>.npz`` beside this file with
  rows, prompt_logits [len(rows)][V]      (float32)
  tokens [n_decode + 1]                   greedy tokens (first = after the prompt)
  decode_logits [n_decode][V]             (float32) logits of each decode step
  margins [n_decode + 1]                  top-1 minus top-2 logit of each greedy row
Only ``oracle`` and ``synth`` are called: no value comes from the HIP library.

  python tests/golden/make_fullsize.py 8b_q4_520 [more cases]
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path[:0] = [ROOT, HERE]

import fullsize_cases as fc  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402


def margin(row):
    r = np.sort(np.asarray(row, np.float64))
    return float(r[-1] - r[-2])


def make(name):
    c = fc.CASES[name]
    hp, seed = fc.case_hparams(name)
    t0 = time.time()
    w = synth.weights_numpy(hp, seed, threads=min(8, os.cpu_count() or 1))
    om = oracle.Model(hp, w, "f64")
    del w
    print(f"[{name}] weights + oracle model in {time.time() - t0:.1f} s", flush=True)
    prompt = fc.case_prompt(name)
    ctx = oracle.Context(om, 1, fc.n_ctx_for(name))
    keep = set(c["rows"])
    plog = []
    t0 = time.time()
    for i, t in enumerate(prompt):
        lg = ctx.eval(0, int(t), want_logits=i in keep)
        if i in keep:
            plog.append(np.asarray(lg, np.float32))
        if i % 32 == 31:
            print(f"[{name}] prompt token {i + 1}/{len(prompt)}  {time.time() - t0:.0f} s", flush=True)
    last = np.asarray(lg, np.float64)
    toks = [oracle.argmax(last)]
    margins = [margin(last)]
    dlog = []
    for k in range(c["n_decode"]):
        lg = ctx.eval(0, toks[-1], want_logits=True)
        dlog.append(np.asarray(lg, np.float32))
        toks.append(oracle.argmax(lg))
        margins.append(margin(lg))
    out = os.path.join(HERE, f"fullsize_{name}.npz")
    np.savez(out, rows=np.asarray(c["rows"], np.int32), prompt_logits=np.stack(plog),
             tokens=np.asarray(toks, np.int32),
             decode_logits=np.stack(dlog) if dlog else np.zeros((0, hp["n_vocab"]), np.float32),
             margins=np.asarray(margins, np.float64))
    print(f"[{name}] wrote {out} ({time.time() - t0:.0f} s of oracle time); tokens {toks}", flush=True)


if __name__ == "__main__":
    for n in sys.argv[1:] or list(fc.CASES):
        make(n)
