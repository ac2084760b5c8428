"""GGUF v3 container checks on the CPU: dec_gguf_inspect against files
written by the independent test writer (tests/gguf_py.py), valid and
corrupted.  dec_gguf_inspect touches no device."""
import struct

import numpy as np
import pytest

import gguf_py as G

HP = dict(n_layer=2, n_embd=256, n_head=4, n_head_kv=2, head_dim=64, n_ff=512, n_vocab=640,
          rms_eps=1e-5, rope_base=10000.0)


@pytest.fixture(scope="module")
def dec():
    import decode_amd
    decode_amd.lib()
    return decode_amd


def tensors(hp=HP, ttype=G.T_Q4_0, seed=0, skip=(), tied=False):
    r = np.random.default_rng(seed)
    out = []
    for name, _, _, dims in G.tensor_table(hp):
        if name in skip or (tied and name == "output.weight"):
            continue
        t = G.T_F32 if len(dims) == 1 else ttype
        out.append((name, t, dims, r.integers(0, 256, G.tensor_nbytes(t, dims), dtype=np.uint8).tobytes()))
    return out


def write(tmp_path, data: bytes, name="m.gguf"):
    p = tmp_path / name
    p.write_bytes(data)
    return p


def inspect(dec, path):
    return dec.gguf_inspect(path)


def test_helper_round_trip():
    ts = tensors()
    b = G.build(G.llama_kv(HP), ts)
    p = G.parse(b)
    assert p["version"] == 3 and p["order"] == [t[0] for t in ts]
    for name, t, dims, data in ts:
        assert p["tensors"][name] == (t, dims, data)
    assert p["kv"]["llama.block_count"] == HP["n_layer"]


@pytest.mark.parametrize("ttype,wt", [(G.T_Q4_0, 3), (G.T_Q8_0, 2), (G.T_F32, 0), (G.T_Q4_K, 4)])
def test_valid_file(dec, tmp_path, ttype, wt):
    ts = tensors(ttype=ttype)
    n, hp = inspect(dec, write(tmp_path, G.build(G.llama_kv(HP), ts)))
    assert n == len(ts)
    for k in ("n_layer", "n_embd", "n_head", "n_head_kv", "head_dim", "n_ff", "n_vocab"):
        assert hp[k] == HP[k], k
    assert hp["wtype"] == wt and hp["kvtype"] == 1
    assert abs(hp["rms_eps"] - 1e-5) < 1e-12 and hp["rope_base"] == 10000.0


def test_optional_keys_defaults_and_extras(dec, tmp_path):
    """head_count_kv, key_length, eps and base default as documented; unknown
    keys (arrays of strings, nested arrays) and extra tensors are ignored;
    output.weight may be absent (tied)."""
    kv = [x for x in G.llama_kv(HP) if x[0] not in ("llama.attention.head_count_kv", "llama.attention.key_length",
                                                      "llama.rope.freq_base", "llama.attention.layer_norm_rms_epsilon")]
    kv += [("tokenizer.ggml.tokens", G.ARR, (G.STR, ["<s>", "</s>", "a"])),
           ("x.nested", G.ARR, (G.ARR, [(G.U32, [1, 2]), (G.U32, [3])])),
           ("x.flag", G.BOOL, True), ("x.big", G.U64, 1 << 40)]
    hp = dict(HP, n_head_kv=HP["n_head"], head_dim=HP["n_embd"] // HP["n_head"])
    ts = tensors(hp, tied=True) + [("extra.weight", G.T_F32, [8], bytes(32))]
    n, got = inspect(dec, write(tmp_path, G.build(kv, ts)))
    assert n == len(ts)
    assert got["n_head_kv"] == HP["n_head"] and got["head_dim"] == 64
    assert abs(got["rms_eps"] - 1e-5) < 1e-12 and got["rope_base"] == 10000.0


def test_alignment_key(dec, tmp_path):
    ts = tensors()
    kv = G.llama_kv(HP) + [("general.alignment", G.U32, 64)]
    n, _ = inspect(dec, write(tmp_path, G.build(kv, ts, alignment=64)))
    assert n == len(ts)
    # offsets laid out for 32 but 64 declared: a 32-byte tensor first leaves
    # every later offset at an odd multiple of 32
    ts = [("extra.a", G.T_F32, [8], bytes(32))] + ts
    b = G.build(kv, ts, alignment=32)
    assert inspect(dec, write(tmp_path, b, "a.gguf"))[0] == -6


@pytest.mark.parametrize("case,code", [
    ("magic", -4), ("version2", -5), ("version4", -5), ("truncated_header", -6), ("truncated_data", -8),
    ("duplicate", -7), ("unknown_type", -10), ("missing_key", -9), ("missing_tensor", -9), ("wrong_dims", -9),
    ("mixed_types", -9), ("arch", -9), ("bad_string", -6), ("empty", -6), ("q4_k_partial_superblock", -6)])
def test_rejected(dec, tmp_path, case, code):
    kv, ts = G.llama_kv(HP), tensors()
    if case == "magic":
        b = G.build(kv, ts, magic=b"GGML")
    elif case == "version2":
        b = G.build(kv, ts, version=2)
    elif case == "version4":
        b = G.build(kv, ts, version=4)
    elif case == "truncated_header":
        b = G.build(kv, ts)[:200]
    elif case == "truncated_data":
        b = G.build(kv, ts)[:-100]
    elif case == "duplicate":
        b = G.build(kv, ts + [ts[3]])
    elif case == "unknown_type":
        b = G.build(kv, ts + [("extra.weight", 14, [256, 4], bytes(210 * 4))])
    elif case == "missing_key":
        b = G.build([x for x in kv if x[0] != "llama.block_count"], ts)
    elif case == "missing_tensor":
        b = G.build(kv, [t for t in ts if t[0] != "blk.1.ffn_up.weight"])
    elif case == "wrong_dims":
        # blk.0.attn_k.weight stored as [kd, d] instead of [d, kd] (same byte count)
        b = G.build(kv, [(n, t, (d[::-1] if n == "blk.0.attn_k.weight" else d), x) for n, t, d, x in ts])
    elif case == "mixed_types":
        b = G.build(kv, [(n, G.T_Q8_0 if n == "blk.1.ffn_gate.weight" else t, d,
                          bytes(G.tensor_nbytes(G.T_Q8_0, d)) if n == "blk.1.ffn_gate.weight" else x)
                         for n, t, d, x in ts])
    elif case == "arch":
        b = G.build([("general.architecture", G.STR, "gptx")] + kv[1:], ts)
    elif case == "q4_k_partial_superblock":
        # Q4_K rows are whole 256-weight super-blocks: ffn_down rows of 288 are not
        hp = dict(HP, n_ff=288)
        b = G.build(G.llama_kv(hp), tensors(hp, ttype=G.T_Q4_K))
    elif case == "bad_string":
        good = G.build(kv, ts)
        # the first key's length field claims more bytes than the file holds
        b = good[:24] + struct.pack("<Q", 1 << 40) + good[32:]
    else:
        b = b""
    assert inspect(dec, write(tmp_path, b))[0] == code


def test_missing_file(dec, tmp_path):
    assert inspect(dec, tmp_path / "absent.gguf")[0] == -1
