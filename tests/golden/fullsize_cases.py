"""Workloads of the stored full-size oracle results (inputs only, no arithmetic).

Each case names a decoder shape from ``synth.WORKLOADS`` (or its own small
shape), the numpy weight seed, a prompt (length and seed), the prompt rows
whose logits are kept, and the number of greedy decode steps that follow the
prompt.  ``make_fullsize.py`` runs the oracle on these inputs and writes
``fullsize_<case>.npz``; ``tests/test_gpu_fullsize_oracle.py`` runs the HIP
library on the same inputs and compares.  Weights always come from
``synth.weights_numpy`` (PCG64 streams), so both sides see the same fp32
bytes on any machine.
"""
import synth

CASES = {
    # 8B shape, Q4_0 (the headline shape): one full ubatch of 512 and a
    # ragged second one of 8 tokens, then 4 decode steps
    "8b_q4_520": dict(workload="8b_q4", n_prompt=520, prompt_seed=4003, n_ubatch=512,
                      rows=(0, 127, 128, 255, 256, 511, 512, 519), n_decode=4),
    # the same with Q8_0 weights (the long-prefill shape)
    "8b_q8_520": dict(workload="8b_q8_long", n_prompt=520, prompt_seed=4004, n_ubatch=512,
                      rows=(0, 127, 128, 255, 256, 511, 512, 519), n_decode=4),
    # 1B shape, Q8_0: the workload's own 512-token ubatch, then 8 decode steps
    "1b_q8_512": dict(workload="1b_q8", n_prompt=512, prompt_seed=4002, n_ubatch=512,
                      rows=(0, 63, 64, 255, 256, 511), n_decode=8),
    # 8B shape, Q4_K super-block weights: a full ubatch of 256 and a ragged
    # one of 8 tokens, then 3 decode steps
    "8b_q4k_264": dict(workload="8b_q4k", n_prompt=264, prompt_seed=4006, n_ubatch=256,
                       rows=(0, 127, 128, 255, 256, 263), n_decode=3),
    # narrow and long: d 512, 2 layers, head_dim 128, 8 query / 2 KV heads
    # (GQA 4), Q4_0; a 4200-token prompt in ubatches of 512 (attention over
    # up to 4200 cached positions: many split-K chunks and flash key ranges)
    "narrow_q4_4200": dict(workload=None, n_prompt=4200, prompt_seed=4005, n_ubatch=512,
                           hp=dict(n_layer=2, n_embd=512, n_head=8, n_head_kv=2, head_dim=128,
                                   n_ff=1024, n_vocab=2048, wtype=synth.Q4_0, kvtype=synth.F16),
                           seed=1105,
                           rows=(0, 511, 512, 1023, 2047, 2048, 3583, 3584, 4095, 4096, 4199),
                           n_decode=8),
}


def case_hparams(name):
    c = CASES[name]
    if c["workload"] is not None:
        W = synth.WORKLOADS[c["workload"]]
        return synth.hparams(W), W["seed"]
    return synth.hparams(dict(c["hp"])), c["seed"]


def case_prompt(name):
    c = CASES[name]
    hp, _ = case_hparams(name)
    return synth.prompt(hp["n_vocab"], c["n_prompt"], c["prompt_seed"])


def n_ctx_for(name):
    c = CASES[name]
    n = c["n_prompt"] + c["n_decode"] + 1
    return (n + 255) // 256 * 256
