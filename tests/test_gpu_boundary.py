"""Boundary checks through the C ABI that need a GPU: the greedy tie rule of
the device argmax (ties to the lowest token id) and the caller-supplied
device allocator (every allocation of a model and a context goes through
it and is returned when they are freed)."""
import numpy as np
import pytest

import synth
from gpu_util import assert_logits_close, gpu_greedy, small_hp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dec():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_amd
    decode_amd.lib()
    return decode_amd


TIE = (37, 38, 500, 601)


def _tied_output(hp, w, seed):
    """Output rows: the rows in TIE are one vector v, all others -v, so every
    logits row has two exactly tied groups (identical rows give identical
    logits in any reduction order the kernels use)."""
    v = synth.normal(hp["n_embd"], seed, 0.05)
    out = np.repeat(-v[None, :], hp["n_vocab"], axis=0).astype(np.float32)
    out[list(TIE)] = v
    w["output"] = np.ascontiguousarray(out)


@pytest.mark.parametrize("wtype", [synth.F32, synth.Q8_0, synth.Q4_0])
def test_argmax_ties_go_to_lowest_id(dec, wtype):
    import oracle
    hp = small_hp(wtype, synth.F16, n_vocab=640, n_ff=544 if wtype == synth.F32 else 512)
    w = synth.weights_numpy(hp, 61, threads=4)
    _tied_output(hp, w, 62)
    gm = dec.Model(hp, w)
    ctx = dec.Context(gm, n_ctx=256, n_ubatch=16)
    prompt = synth.prompt(hp["n_vocab"], 20, 63)
    toks, rows = gpu_greedy(ctx, prompt, 12)
    om = oracle.Model(hp, w)
    o_toks, _ = oracle.run_greedy(om, prompt, 12, 256, teacher=toks)
    seen = set()
    for k, (t, r) in enumerate(zip(toks, rows)):
        top = np.flatnonzero(r == r.max())
        assert top.size >= 2, f"step {k}: no tie in the logits row"
        assert t == int(top[0]), f"step {k}: argmax {t}, lowest tied id {top[0]}"
        assert t == o_toks[k], f"step {k}: oracle {o_toks[k]}"
        seen.add(t)
    assert seen <= {TIE[0], 0}      # the tied group that wins, by its lowest id
    # every output row at once (prefill with output_all, then dec_argmax_all)
    ctx.clear(0)
    assert ctx.prefill(prompt, 0, output_all=True) == 0
    allt = ctx.argmax_all()
    assert allt.size == len(prompt)
    for i in range(len(prompt)):
        r = ctx.logits(i)
        assert allt[i] == int(np.flatnonzero(r == r.max())[0])


class CountingAllocator:
    """dec_allocator over torch's caching allocator that counts every call."""

    def __init__(self, dec):
        self.inner = dec.TorchAllocator()
        self.n_alloc = self.n_free = 0
        self.bytes = 0
        a, f = self.inner._alloc, self.inner._free

        def alloc(nbytes, ud):
            self.n_alloc += 1
            self.bytes += int(nbytes)
            return a(nbytes, ud)

        def free(p, ud):
            self.n_free += 1
            return f(p, ud)

        self.inner._alloc, self.inner._free = alloc, free
        self.inner.c_alloc = dec.ALLOC_FN(alloc)
        self.inner.c_free = dec.FREE_FN(free)
        self.inner.struct = dec.Allocator(self.inner.c_alloc, self.inner.c_free, None)

    @property
    def live(self):
        return len(self.inner._live)


@pytest.mark.parametrize("wtype,kvtype", [(synth.Q4_0, synth.F16), (synth.Q8_0, synth.Q8_0)])
def test_torch_allocator_routes_every_allocation(dec, wtype, kvtype):
    import torch

    import oracle
    hp = small_hp(wtype, kvtype)
    w = synth.weights_numpy(hp, 71, threads=4)
    prompt = synth.prompt(hp["n_vocab"], 40, 72)
    al = CountingAllocator(dec)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    gm = dec.Model(hp, w, allocator=al.inner)
    # the weights stay; the host weights' staging buffer is returned after the load
    n_model = al.live
    assert n_model > 0 and al.n_alloc == n_model + 1 and al.n_free == 1
    n_before = al.n_alloc
    ctx = dec.Context(gm, n_ctx=256, n_ubatch=16)
    n_ctx_allocs = al.n_alloc - n_before
    assert n_ctx_allocs > 0                      # the context takes the model's allocator
    live_bytes = sum(t.numel() for t in al.inner._live.values())
    assert torch.cuda.memory_allocated() - base >= live_bytes > 0
    om = oracle.Model(hp, w)
    o_toks, o_rows = oracle.run_greedy(om, prompt, 6, 256)
    g_toks, g_rows = gpu_greedy(ctx, prompt, 6, teacher=o_toks)
    for k, (g, o) in enumerate(zip(g_rows, o_rows)):
        assert_logits_close(g, o, f"allocator run step {k}")
    assert g_toks == o_toks
    assert al.n_alloc == n_before + n_ctx_allocs   # nothing allocated after creation
    ctx.close()
    assert al.n_free == 1 + n_ctx_allocs and al.live == n_model
    gm.close()
    assert al.n_free == al.n_alloc and al.live == 0
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == base
