"""A small GGUF v3 writer and parser for the tests, written from the format's
published layout independently of the library's C++ reader/writer.

File: magic b"GGUF", u32 version, u64 tensor count, u64 key/value count;
key/value pairs (string key, u32 value type, value; an array is u32
element type, u64 count, elements); per tensor: string name, u32 n_dims,
u64 dims (row length first), u32 element type, u64 offset from the data
section; the data section at the next multiple of general.alignment (32 by
default).  Strings are u64 length + bytes, everything little-endian.
"""
from __future__ import annotations

import struct

U8, I8, U16, I16, U32, I32, F32, BOOL, STR, ARR, U64, I64, F64 = range(13)
T_F32, T_F16, T_Q4_0, T_Q8_0, T_Q4_K = 0, 1, 2, 8, 12
_SCALAR = {U8: "<B", I8: "<b", U16: "<H", I16: "<h", U32: "<I", I32: "<i", F32: "<f", BOOL: "<?",
           U64: "<Q", I64: "<q", F64: "<d"}


def _str(s: str) -> bytes:
    b = s.encode()
    return struct.pack("<Q", len(b)) + b


def _value(t: int, v) -> bytes:
    if t == STR:
        return _str(v)
    if t == ARR:
        et, items = v
        out = struct.pack("<IQ", et, len(items))
        return out + b"".join(_value(et, x) for x in items)
    return struct.pack(_SCALAR[t], v)


def tensor_nbytes(ttype: int, dims) -> int:
    n = 1
    for d in dims:
        n *= d
    if ttype == T_F32:
        return 4 * n
    if ttype == T_F16:
        return 2 * n
    if ttype == T_Q4_0:
        return n // 32 * 18
    if ttype == T_Q8_0:
        return n // 32 * 34
    if ttype == T_Q4_K:
        return n // 256 * 144
    raise ValueError(ttype)


def build(kv, tensors, alignment: int = 32, version: int = 3, magic: bytes = b"GGUF") -> bytes:
    """kv: [(key, type, value)]; tensors: [(name, type, dims, data bytes)].
    Returns the file bytes."""
    head = bytearray(magic + struct.pack("<IQQ", version, len(tensors), len(kv)))
    for key, t, v in kv:
        head += _str(key) + struct.pack("<I", t) + _value(t, v)
    offs, off = [], 0
    for _, _, _, data in tensors:
        offs.append(off)
        off = (off + len(data) + alignment - 1) // alignment * alignment
    for (name, t, dims, _), o in zip(tensors, offs):
        head += _str(name) + struct.pack("<I", len(dims)) + b"".join(struct.pack("<Q", d) for d in dims)
        head += struct.pack("<IQ", t, o)
    head += b"\0" * ((-len(head)) % alignment)
    body = bytearray()
    for (_, _, _, data), o in zip(tensors, offs):
        body += b"\0" * (o - len(body))
        body += data
    return bytes(head + body)


class _Reader:
    def __init__(self, b: bytes):
        self.b, self.p = b, 0

    def take(self, n):
        if self.p + n > len(self.b):
            raise ValueError("truncated")
        out = self.b[self.p:self.p + n]
        self.p += n
        return out

    def fmt(self, f):
        return struct.unpack(f, self.take(struct.calcsize(f)))[0]

    def s(self):
        return self.take(self.fmt("<Q")).decode()

    def value(self, t):
        if t == STR:
            return self.s()
        if t == ARR:
            et, n = self.fmt("<I"), self.fmt("<Q")
            return [self.value(et) for _ in range(n)]
        return self.fmt(_SCALAR[t])


def parse(b: bytes) -> dict:
    """Returns {"version", "kv": {key: value}, "tensors": {name: (type, dims, data)}, "order": [names]}."""
    r = _Reader(b)
    if r.take(4) != b"GGUF":
        raise ValueError("magic")
    version = r.fmt("<I")
    n_t, n_kv = r.fmt("<Q"), r.fmt("<Q")
    kv = {}
    for _ in range(n_kv):
        k = r.s()
        kv[k] = r.value(r.fmt("<I"))
    infos = []
    for _ in range(n_t):
        name = r.s()
        nd = r.fmt("<I")
        dims = [r.fmt("<Q") for _ in range(nd)]
        infos.append((name, r.fmt("<I"), dims, r.fmt("<Q")))
    al = kv.get("general.alignment", 32)
    start = (r.p + al - 1) // al * al
    tensors = {}
    for name, t, dims, off in infos:
        n = tensor_nbytes(t, dims)
        if start + off + n > len(b):
            raise ValueError("tensor outside the file")
        tensors[name] = (t, dims, b[start + off:start + off + n])
    return {"version": version, "kv": kv, "tensors": tensors, "order": [i[0] for i in infos]}


def llama_kv(hp: dict) -> list:
    return [("general.architecture", STR, "llama"),
            ("llama.embedding_length", U32, hp["n_embd"]),
            ("llama.block_count", U32, hp["n_layer"]),
            ("llama.feed_forward_length", U32, hp["n_ff"]),
            ("llama.attention.head_count", U32, hp["n_head"]),
            ("llama.attention.head_count_kv", U32, hp["n_head_kv"]),
            ("llama.attention.key_length", U32, hp["head_dim"]),
            ("llama.rope.freq_base", F32, hp.get("rope_base", 10000.0)),
            ("llama.attention.layer_norm_rms_epsilon", F32, hp.get("rms_eps", 1e-5))]


# (GGUF name, tensor key of the test weight dicts, per layer, dims(hp))
def tensor_table(hp: dict) -> list:
    d, F, V = hp["n_embd"], hp["n_ff"], hp["n_vocab"]
    qd, kd = hp["n_head"] * hp["head_dim"], hp["n_head_kv"] * hp["head_dim"]
    out = [("token_embd.weight", "tok_embd", None, [d, V]),
           ("output_norm.weight", "output_norm", None, [d]),
           ("output.weight", "output", None, [d, V])]
    for l in range(hp["n_layer"]):
        for g, k, dims in (("attn_norm", "attn_norm", [d]), ("attn_q", "wq", [d, qd]), ("attn_k", "wk", [d, kd]),
                           ("attn_v", "wv", [d, kd]), ("attn_output", "wo", [qd, d]), ("ffn_norm", "ffn_norm", [d]),
                           ("ffn_gate", "ffn_gate", [d, F]), ("ffn_up", "ffn_up", [d, F]),
                           ("ffn_down", "ffn_down", [F, d])):
            out.append((f"blk.{l}.{g}.weight", k, l, dims))
    return out
