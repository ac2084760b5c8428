"""CPU oracle of the LLaMA-style decoder step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library (``decode_amd``)
never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, sequential reductions); this
module only builds it and marshals arguments through ctypes.  Two builds of
the same source exist: ``f64`` (the oracle of record: every activation,
accumulator and softmax in double) and ``f32`` (the fp32 decoder, used to
bound the oracle's own rounding error).  Block quantizers and the f16
conversion run in fp32 in both builds.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")

T_F32, T_F16, T_Q8_0, T_Q4_0, T_Q4_K = 0, 1, 2, 3, 4
TENSOR_IDS = {"tok_embd": 0, "output": 1, "wq": 2, "wk": 3, "wv": 4, "wo": 5,
              "ffn_gate": 6, "ffn_up": 7, "ffn_down": 8}


def lib_path(kind: str) -> str:
    return os.path.join(HERE, f"liboracle_{kind}.so")


def build(force: bool = True) -> None:
    """Compile both oracle builds with gcc (no GPU involved)."""
    for kind, real in (("f64", "double"), ("f32", "float")):
        out = lib_path(kind)
        if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(SRC):
            continue
        tmp = out + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
               "-Wall", "-Wextra", "-Wno-unused-parameter", "-shared", "-fPIC",
               f"-DORC_REAL={real}", SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)


class _Hparams(C.Structure):
    _fields_ = [("n_layer", C.c_int32), ("n_embd", C.c_int32), ("n_head", C.c_int32),
                ("n_head_kv", C.c_int32), ("head_dim", C.c_int32), ("n_ff", C.c_int32),
                ("n_vocab", C.c_int32), ("rms_eps", C.c_float), ("rope_base", C.c_float),
                ("wtype", C.c_int32), ("kvtype", C.c_int32)]


_PP = C.POINTER(C.c_void_p)


class _Weights(C.Structure):
    _fields_ = [("tok_embd", C.c_void_p), ("output_norm", C.c_void_p), ("output", C.c_void_p),
                ("attn_norm", _PP), ("wq", _PP), ("wk", _PP), ("wv", _PP), ("wo", _PP),
                ("ffn_norm", _PP), ("ffn_gate", _PP), ("ffn_up", _PP), ("ffn_down", _PP)]


_LIBS: dict = {}


def load(kind: str = "f64") -> C.CDLL:
    if kind in _LIBS:
        return _LIBS[kind]
    path = lib_path(kind)
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(SRC):
        build(force=True)
    L = C.CDLL(path)
    vp, i32, i64, f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_float
    sig = {
        "orc_real_size": (i32, []),
        "orc_f16_from_f32": (C.c_uint16, [f32]),
        "orc_f16_from_f64": (C.c_uint16, [C.c_double]),
        "orc_f16_to_f32": (f32, [C.c_uint16]),
        "orc_f16_from_f32_n": (None, [vp, i64, vp]),
        "orc_f16_to_f32_n": (None, [vp, i64, vp]),
        "orc_q8_0_quantize": (i64, [vp, i64, vp]),
        "orc_q4_0_quantize": (i64, [vp, i64, vp]),
        "orc_q8_0_dequantize": (None, [vp, i64, vp]),
        "orc_q4_0_dequantize": (None, [vp, i64, vp]),
        "orc_q4_k_quantize": (i64, [vp, i64, vp]),
        "orc_q4_k_dequantize": (None, [vp, i64, vp]),
        "orc_q4_k_scales": (None, [vp, vp, vp]),
        "orc_rmsnorm": (None, [vp, vp, i32, f32, vp]),
        "orc_matvec": (None, [i32, vp, i32, i32, vp, vp]),
        "orc_rope": (None, [vp, i32, i32, i32, f32]),
        "orc_attend": (None, [vp, vp, vp, i32, i64, vp, i32, i32, i32, vp, vp]),
        "orc_swiglu": (None, [vp, vp, i32, vp]),
        "orc_argmax": (i32, [vp, i32]),
        "orc_model_new": (vp, [vp, vp]),
        "orc_model_free": (None, [vp]),
        "orc_model_tensor_bytes": (i64, [vp, i32, i32, vp, i64]),
        "orc_ctx_new": (vp, [vp, i32, i32]),
        "orc_ctx_free": (None, [vp]),
        "orc_seq_pos_max": (i32, [vp, i32]),
        "orc_seq_clear": (None, [vp, i32]),
        "orc_eval": (i32, [vp, i32, i32, vp]),
        "orc_eval_tap": (i32, [vp, i32, i32, vp, i32, vp]),
        "orc_kv_row": (i32, [vp, i32, i32, i32, i32, i32, vp]),
        "orc_splitmix64": (C.c_uint64, [C.c_uint64, C.c_uint64]),
        "orc_uniform24": (f32, [C.c_uint64, C.c_uint64]),
        "orc_sample": (i32, [vp, i32, vp, i32, vp, C.c_uint64, vp, vp, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _LIBS[kind] = L
    return L


def real_dtype(kind: str = "f64"):
    return np.float64 if load(kind).orc_real_size() == 8 else np.float32


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


# ---------------------------------------------------------------- primitives
def f16_from_f32(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    h = np.empty(x.shape, np.uint16)
    load().orc_f16_from_f32_n(_p(x), x.size, _p(h))
    return h


def f16_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    x = np.empty(h.shape, np.float32)
    load().orc_f16_to_f32_n(_p(h), h.size, _p(x))
    return x


# block elements and bytes per block of each quantized type
BLOCK = {T_Q8_0: (32, 34), T_Q4_0: (32, 18), T_Q4_K: (256, 144)}


def quantize(x: np.ndarray, wtype: int) -> np.ndarray:
    """fp32 array (size a multiple of the block) -> GGUF-style block bytes."""
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    be, bsz = BLOCK[wtype]
    out = np.empty(x.size // be * bsz, np.uint8)
    L = load()
    fn = {T_Q8_0: L.orc_q8_0_quantize, T_Q4_0: L.orc_q4_0_quantize, T_Q4_K: L.orc_q4_k_quantize}[wtype]
    n = fn(_p(x), x.size, _p(out))
    if n < 0:
        raise ValueError(f"size must be a multiple of {be}")
    return out


def dequantize(blocks: np.ndarray, n: int, wtype: int) -> np.ndarray:
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    y = np.empty(n, np.float32)
    L = load()
    fn = {T_Q8_0: L.orc_q8_0_dequantize, T_Q4_0: L.orc_q4_0_dequantize, T_Q4_K: L.orc_q4_k_dequantize}[wtype]
    fn(_p(blocks), n, _p(y))
    return y


def q4_k_scales(block: np.ndarray):
    """The eight six-bit (scale, min) pairs of one 144-byte Q4_K block."""
    b = np.ascontiguousarray(block, dtype=np.uint8)
    sc = np.empty(8, np.int32)
    m = np.empty(8, np.int32)
    load().orc_q4_k_scales(_p(b), _p(sc), _p(m))
    return sc, m


def rmsnorm(x, g, eps, kind="f64"):
    rt = real_dtype(kind)
    x = np.ascontiguousarray(x, rt)
    g = np.ascontiguousarray(g, np.float32)
    y = np.empty_like(x)
    load(kind).orc_rmsnorm(_p(x), _p(g), x.size, eps, _p(y))
    return y


def matvec(wtype, w, rows, cols, x, kind="f64"):
    rt = real_dtype(kind)
    w = np.ascontiguousarray(w)
    x = np.ascontiguousarray(x, rt)
    y = np.empty(rows, rt)
    load(kind).orc_matvec(wtype, _p(w), rows, cols, _p(x), _p(y))
    return y


def rope(v, n_heads, hd, pos, base, kind="f64"):
    rt = real_dtype(kind)
    v = np.array(v, dtype=rt, copy=True, order="C")
    load(kind).orc_rope(_p(v), n_heads, hd, pos, base)
    return v


def attend(q, K, V, kvtype, pos, row_pos=None, ld=None, n=None, kind="f64"):
    """q [hd]; K,V [n][ld] (float32 or uint16 f16 bits), or flat arrays with
    explicit ``n`` and ``ld`` -> (o[hd], w[n])."""
    rt = real_dtype(kind)
    q = np.ascontiguousarray(q, rt)
    K = np.ascontiguousarray(K)
    V = np.ascontiguousarray(V)
    n = K.shape[0] if n is None else n
    hd = q.size
    ld = K.shape[1] if ld is None else ld
    rp = None if row_pos is None else np.ascontiguousarray(row_pos, np.int32)
    o = np.empty(hd, rt)
    w = np.empty(max(n, 1), rt)
    load(kind).orc_attend(_p(q), _p(K), _p(V), kvtype, ld, None if rp is None else _p(rp),
                          n, hd, pos, _p(o), _p(w))
    return o, w[:n]


def swiglu(u, v, kind="f64"):
    rt = real_dtype(kind)
    u = np.ascontiguousarray(u, rt)
    v = np.ascontiguousarray(v, rt)
    h = np.empty_like(u)
    load(kind).orc_swiglu(_p(u), _p(v), u.size, _p(h))
    return h


def argmax(x, kind="f64"):
    x = np.ascontiguousarray(x, real_dtype(kind))
    return int(load(kind).orc_argmax(_p(x), x.size))


# ------------------------------------------------------------------- sampler
class SamplerParams(C.Structure):
    """Mirror of orc_sampler_params (article, step 15: the sampler list)."""
    _fields_ = [("top_k", C.c_int32), ("top_p", C.c_float), ("min_p", C.c_float), ("temp", C.c_float),
                ("repeat_penalty", C.c_float), ("penalty_last_n", C.c_int32), ("seed", C.c_uint64)]


def splitmix64(seed: int, index: int) -> int:
    return int(load().orc_splitmix64(seed, index))


def uniform24(seed: int, index: int) -> float:
    return float(load().orc_uniform24(seed, index))


def sample(logits, hist=(), top_k=40, top_p=1.0, min_p=0.0, temp=1.0, repeat_penalty=1.0,
           penalty_last_n=64, seed=0, draw=0, detail=False):
    """The sampler chain on one fp32 logits row.  Returns the token, or with
    detail=True (token, candidate ids, inclusive cumulative weights, target)."""
    x = np.ascontiguousarray(logits, np.float32)
    h = np.ascontiguousarray(np.asarray(hist, np.int32))
    prm = SamplerParams(top_k, top_p, min_p, temp, repeat_penalty, penalty_last_n, seed)
    ids = np.zeros(x.size, np.int32)
    cum = np.zeros(x.size, np.float32)
    nk = C.c_int32(0)
    tg = C.c_float(0.0)
    tok = load().orc_sample(_p(x), x.size, _p(h) if h.size else None, h.size, C.byref(prm), draw,
                            _p(ids), _p(cum), C.byref(nk), C.byref(tg))
    if not detail:
        return int(tok)
    return int(tok), ids[:nk.value].copy(), cum[:nk.value].copy(), float(tg.value)


# ------------------------------------------------------------------- decoder
class Model:
    """The oracle decoder.  ``weights`` is a dict of fp32 numpy arrays named as
    in the article's LLaMA tensor set (tok_embd, output_norm, output, and per
    layer lists attn_norm, wq, wk, wv, wo, ffn_norm, ffn_gate, ffn_up, ffn_down)."""

    def __init__(self, hp: dict, weights: dict, kind: str = "f64"):
        self.kind = kind
        self.L = load(kind)
        self.rt = real_dtype(kind)
        self.hp = dict(hp)
        h = _Hparams(hp["n_layer"], hp["n_embd"], hp["n_head"], hp["n_head_kv"], hp["head_dim"],
                     hp["n_ff"], hp["n_vocab"], hp.get("rms_eps", 1e-5), hp.get("rope_base", 10000.0),
                     hp["wtype"], hp["kvtype"])
        keep = []

        def arr(a):
            a = np.ascontiguousarray(a, np.float32)
            keep.append(a)
            return _p(a)

        def lst(name):
            ptrs = (C.c_void_p * hp["n_layer"])(*[arr(a).value for a in weights[name]])
            keep.append(ptrs)
            return C.cast(ptrs, _PP)

        w = _Weights(arr(weights["tok_embd"]), arr(weights["output_norm"]), arr(weights["output"]),
                     lst("attn_norm"), lst("wq"), lst("wk"), lst("wv"), lst("wo"),
                     lst("ffn_norm"), lst("ffn_gate"), lst("ffn_up"), lst("ffn_down"))
        self.ptr = self.L.orc_model_new(C.byref(h), C.byref(w))
        if not self.ptr:
            raise ValueError("oracle rejected the hyper-parameters")

    def tensor_bytes(self, name: str, layer: int = 0) -> np.ndarray:
        tid = TENSOR_IDS[name]
        need = -self.L.orc_model_tensor_bytes(self.ptr, tid, layer, None, 0)
        out = np.empty(need, np.uint8)
        n = self.L.orc_model_tensor_bytes(self.ptr, tid, layer, _p(out), need)
        assert n == need
        return out

    def __del__(self):
        if getattr(self, "ptr", None):
            self.L.orc_model_free(self.ptr)
            self.ptr = None


class Context:
    def __init__(self, model: Model, n_seq: int, n_ctx: int):
        self.model = model
        self.L = model.L
        self.ptr = self.L.orc_ctx_new(model.ptr, n_seq, n_ctx)
        if not self.ptr:
            raise MemoryError("oracle context allocation failed")

    def eval(self, seq: int, token: int, want_logits: bool = True, tap: int = -1):
        V = self.model.hp["n_vocab"]
        logits = np.empty(V, self.model.rt) if want_logits else None
        xt = np.empty(self.model.hp["n_embd"], self.model.rt) if tap >= 0 else None
        rc = self.L.orc_eval_tap(self.ptr, seq, int(token), None if logits is None else _p(logits),
                                 tap, None if xt is None else _p(xt))
        if rc != 0:
            raise RuntimeError(f"orc_eval returned {rc}")
        return (logits, xt) if tap >= 0 else logits

    def pos_max(self, seq: int) -> int:
        return int(self.L.orc_seq_pos_max(self.ptr, seq))

    def clear(self, seq: int) -> None:
        self.L.orc_seq_clear(self.ptr, seq)

    def kv_row(self, which: int, layer: int, seq: int, pos: int, kv_head: int) -> np.ndarray:
        out = np.empty(self.model.hp["head_dim"], np.float32)
        rc = self.L.orc_kv_row(self.ptr, which, layer, seq, pos, kv_head, _p(out))
        if rc != 0:
            raise IndexError("kv row out of range")
        return out

    def __del__(self):
        if getattr(self, "ptr", None):
            self.L.orc_ctx_free(self.ptr)
            self.ptr = None


def run_greedy(model: Model, prompt, n_decode: int, n_ctx: int, seq_count: int = 1,
               teacher=None, keep_logits: bool = True):
    """Prefill ``prompt`` (logits for its last token only), then ``n_decode``
    greedy steps; returns (tokens, list of logit rows).  With ``teacher`` the
    fed-back tokens come from that list instead of the oracle's own argmax."""
    ctx = Context(model, seq_count, n_ctx)
    toks, rows = [], []
    for i, t in enumerate(prompt):
        last = i == len(prompt) - 1
        lg = ctx.eval(0, int(t), want_logits=last)
    nxt = argmax(lg, model.kind)
    toks.append(nxt)
    if keep_logits:
        rows.append(lg)
    for k in range(n_decode):
        feed = nxt if teacher is None else int(teacher[k])
        lg = ctx.eval(0, feed, want_logits=True)
        nxt = argmax(lg, model.kind)
        toks.append(nxt)
        if keep_logits:
            rows.append(lg)
    return toks, rows
