"""GGUF v3 save / load through the C ABI on the device.

* A saved file is read back by the independent test parser (tests/gguf_py.py):
  header, keys, tensor names / dims / types, and every tensor's bytes equal
  the library's block export and the oracle's own quantization of the same
  fp32 weights (bit for bit).
* A model loaded from that file holds the same blocks, and its logits equal
  the original model's bit for bit (same blocks, same kernels).
* A file written by the test writer from the oracle's blocks, with the
  tensors shuffled, extra keys and tensors, and the output matrix tied to the
  embedding, loads and runs within the usual tolerance of the oracle.
"""
import numpy as np
import pytest

import gguf_py as G
import synth
from gpu_util import assert_logits_close, gpu_greedy, small_hp

pytestmark = pytest.mark.gpu

MATS = {"tok_embd": "token_embd.weight", "output": "output.weight"}
LAYER_MATS = {"wq": "attn_q", "wk": "attn_k", "wv": "attn_v", "wo": "attn_output", "ffn_gate": "ffn_gate",
              "ffn_up": "ffn_up", "ffn_down": "ffn_down"}
FILE_TYPE = {synth.Q4_0: G.T_Q4_0, synth.Q8_0: G.T_Q8_0, synth.F32: G.T_F32, synth.Q4_K: G.T_Q4_K}


@pytest.fixture(scope="module")
def dec():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_amd
    decode_amd.lib()
    return decode_amd


def model_hp(wtype):
    return small_hp(wtype, synth.F16, n_ff=544 if wtype == synth.F32 else 512)


def weights(hp, seed):
    """Seeded weights with non-trivial norm gains, so that the 1-D tensors
    carry information through the file too."""
    w = synth.weights_numpy(hp, seed, threads=4)
    r = np.random.default_rng(seed)
    w["output_norm"] = r.uniform(0.5, 1.5, hp["n_embd"]).astype(np.float32)
    for key in ("attn_norm", "ffn_norm"):
        w[key] = [r.uniform(0.5, 1.5, hp["n_embd"]).astype(np.float32) for _ in range(hp["n_layer"])]
    return w


@pytest.mark.parametrize("wtype", [synth.Q4_0, synth.Q8_0, synth.F32, synth.Q4_K])
def test_saved_file_layout_and_bytes(dec, orc, tmp_path, wtype):
    hp = model_hp(wtype)
    w = weights(hp, 51 + wtype)
    gm = dec.Model(hp, w)
    om = orc.Model(hp, w)
    path = tmp_path / "m.gguf"
    gm.save_gguf(path)
    p = G.parse(path.read_bytes())
    assert p["version"] == 3
    kv = p["kv"]
    assert kv["general.architecture"] == "llama" and kv["general.alignment"] == 32
    assert kv["llama.block_count"] == hp["n_layer"] and kv["llama.embedding_length"] == hp["n_embd"]
    assert kv["llama.feed_forward_length"] == hp["n_ff"] and kv["llama.attention.head_count"] == hp["n_head"]
    assert kv["llama.attention.head_count_kv"] == hp["n_head_kv"]
    assert kv["llama.attention.key_length"] == hp["head_dim"]
    table = G.tensor_table(hp)
    assert sorted(p["tensors"]) == sorted(n for n, _, _, _ in table)
    ft = FILE_TYPE[wtype]
    for name, key, layer, dims in table:
        t, got_dims, data = p["tensors"][name]
        assert got_dims == dims, name
        if len(dims) == 1:
            src = w[key] if layer is None else w[key][layer]
            assert t == G.T_F32 and data == np.asarray(src, np.float32).tobytes(), name
            continue
        assert t == ft, name
        blocks = gm.tensor_blocks(key, layer or 0)
        assert np.array_equal(np.frombuffer(data, np.uint8), blocks), name
        assert np.array_equal(blocks, om.tensor_bytes(key, layer or 0)), name


@pytest.mark.parametrize("wtype,n_ff", [(synth.Q4_0, 512), (synth.Q8_0, 512), (synth.F32, 688), (synth.Q4_K, 512)])
def test_load_round_trip_is_bitwise(dec, tmp_path, wtype, n_ff):
    """n_ff 688 with fp32 weights leaves the stored FFN rows / columns padded
    to 704: the loader must place the file's 688 and leave the rest zero."""
    hp = small_hp(wtype, synth.F16, n_ff=n_ff)
    w = weights(hp, 61 + wtype)
    gm = dec.Model(hp, w)
    path = tmp_path / "m.gguf"
    gm.save_gguf(path)
    lm = dec.Model.from_gguf(path, kvtype=synth.F16)
    for key in MATS:
        assert np.array_equal(lm.tensor_blocks(key), gm.tensor_blocks(key)), key
    for l in range(hp["n_layer"]):
        for key in LAYER_MATS:
            assert np.array_equal(lm.tensor_blocks(key, l), gm.tensor_blocks(key, l)), (key, l)
    prompt = synth.prompt(hp["n_vocab"], 20, 77)
    runs = []
    for m in (gm, lm):
        ctx = dec.Context(m, n_ctx=256, n_ubatch=8)
        runs.append(gpu_greedy(ctx, prompt, 6))
        ctx.close()
    (t0, r0), (t1, r1) = runs
    assert t0 == t1
    for a, b in zip(r0, r1):
        assert np.array_equal(np.asarray(a), np.asarray(b))
    lm.close()
    gm.close()


@pytest.mark.parametrize("wtype", [synth.Q8_0, synth.Q4_K])
def test_foreign_file_tied_output_matches_oracle(dec, orc, tmp_path, wtype):
    """Blocks quantized by the oracle, written by the test writer in shuffled
    order with extra keys and tensors, no output.weight (tied): the loaded
    model runs within tolerance of the oracle, and bit for bit like a model
    loaded from the same fp32 weights."""
    hp = model_hp(wtype)
    w = weights(hp, 71)
    w["output"] = w["tok_embd"].copy()               # tied output
    om = orc.Model(hp, w)
    ts = []
    for name, key, layer, dims in G.tensor_table(hp):
        if name == "output.weight":
            continue
        if len(dims) == 1:
            src = w[key] if layer is None else w[key][layer]
            ts.append((name, G.T_F32, dims, np.asarray(src, np.float32).tobytes()))
        else:
            ts.append((name, FILE_TYPE[wtype], dims, om.tensor_bytes(key, layer or 0).tobytes()))
    order = np.random.default_rng(3).permutation(len(ts))
    ts = [ts[i] for i in order] + [("rope_freqs.weight", G.T_F32, [32], bytes(128))]
    kv = [("general.name", G.STR, "synthetic")] + G.llama_kv(hp)[::-1] + [
        ("tokenizer.ggml.tokens", G.ARR, (G.STR, [f"t{i}" for i in range(hp["n_vocab"])]))]
    path = tmp_path / "foreign.gguf"
    path.write_bytes(G.build(kv, ts))
    lm = dec.Model.from_gguf(path, kvtype=synth.F16)
    gm = dec.Model(hp, w)
    prompt = synth.prompt(hp["n_vocab"], 16, 78)
    o_toks, o_rows = orc.run_greedy(om, prompt, 4, 256)
    res = []
    for m in (lm, gm):
        ctx = dec.Context(m, n_ctx=256, n_ubatch=8)
        res.append(gpu_greedy(ctx, prompt, 4, teacher=o_toks))
        ctx.close()
    (lt, lr), (gt, gr) = res
    for a, b in zip(lr, gr):
        assert np.array_equal(np.asarray(a), np.asarray(b))
    for k, (a, o) in enumerate(zip(lr, o_rows)):
        assert_logits_close(a, o, f"step {k}")
    lm.close()
    gm.close()


def test_rejected_file_raises(dec, tmp_path):
    path = tmp_path / "bad.gguf"
    path.write_bytes(b"GGUF" + bytes(4) + bytes(16))   # version 0
    with pytest.raises(dec.DecodeError):
        dec.Model.from_gguf(path)
