"""dec_sample_row_noalloc (the sampler chain as one call that allocates
nothing: its window and host-row staging live in the library's fixed device
buffer) against dec_sampler_sample_row, the entry point it is a variant of:
the same chain, window and draw index give the same token, on two calls in a
row, the second on a smaller row (and from device memory), so the buffer's
leftover contents from the first call must not matter."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dec():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_amd
    decode_amd.lib()
    return decode_amd


CHAINS = [
    dict(top_k=40, top_p=0.95, min_p=0.05, temp=0.8, repeat_penalty=1.1, penalty_last_n=64, seed=1234),
    dict(top_k=1, top_p=1.0, min_p=0.0, temp=1.0, repeat_penalty=1.0, penalty_last_n=0, seed=7),
    dict(top_k=200, top_p=0.5, min_p=0.0, temp=1.3, repeat_penalty=1.3, penalty_last_n=8, seed=99),
    dict(top_k=1024, top_p=1.0, min_p=0.01, temp=2.0, repeat_penalty=1.0, penalty_last_n=64, seed=5),
]


@pytest.mark.parametrize("ci", range(len(CHAINS)))
def test_noalloc_matches_sampler_two_calls(dec, ci):
    import torch
    ch = CHAINS[ci]
    # the second call's row is smaller; both carry ties and the penalised tokens
    rows = [synth.normal(32000, 500 + ci, 2.0), synth.normal(1100, 600 + ci, 2.0)]
    rows[0][[5, 6, 31999]] = rows[0].max()
    hist0 = [int(t) for t in synth.prompt(1100, 70, 700 + ci)]
    ref = dec.Sampler(**ch)
    ref.accept(hist0)
    hist = list(hist0)
    out = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    for k, row in enumerate(rows):
        src = row if k == 0 else torch.from_numpy(row).cuda()   # host row, then device row
        torch.cuda.synchronize()
        rc = dec.sample_row_noalloc(src, out[k:k + 1], hist=hist[-64:], draw=k, **ch)
        assert rc == 0, rc
        torch.cuda.synchronize()
        got = int(out[k].item())
        want = ref.sample_row(row)
        assert got == want, f"chain {ci} call {k}: no-alloc {got}, sampler {want}"
        hist.append(want)
    assert ref.draws() == 2


def test_noalloc_rejects_what_it_cannot_hold(dec):
    import torch
    out = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    big = np.zeros(dec.NOALLOC_MAX_VOCAB + 1, np.float32)
    assert dec.sample_row_noalloc(big, out) == -4
    host_out = torch.zeros(1, dtype=torch.int32)      # pageable host memory: not writable by the device
    assert dec.sample_row_noalloc(np.zeros(100, np.float32), host_out) == -1
    torch.cuda.synchronize()
    assert int(out.item()) == -7                      # nothing was enqueued
