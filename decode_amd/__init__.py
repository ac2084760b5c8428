"""Python binding of libdecode.so (argument marshalling only).

Every step of the decoder runs in the library's HIP kernels; this module
converts Python / numpy / torch arguments into the C ABI of
``include/decode.h`` and back.  PyTorch is used for device memory (optional
allocator callbacks) and streams only.  The library must have been built
(``python decode_amd/build.py``); importing fails loudly when it is missing.
"""
from __future__ import annotations

import ctypes as C
import os
import re

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdecode.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "decode.h")

F32, F16, Q8_0, Q4_0, Q4_K = 0, 1, 2, 3, 4
K_QKV, K_ATTN, K_WO, K_FFN_GU, K_FFN_DOWN, K_OUTPUT, K_STEP = 0, 1, 2, 3, 4, 5, 6
TENSOR_IDS = {"tok_embd": 0, "output": 1, "wq": 2, "wk": 3, "wv": 4, "wo": 5,
              "ffn_gate": 6, "ffn_up": 7, "ffn_down": 8}


class DecodeError(RuntimeError):
    pass


class Hparams(C.Structure):
    _fields_ = [("n_layer", C.c_int32), ("n_embd", C.c_int32), ("n_head", C.c_int32),
                ("n_head_kv", C.c_int32), ("head_dim", C.c_int32), ("n_ff", C.c_int32),
                ("n_vocab", C.c_int32), ("rms_eps", C.c_float), ("rope_base", C.c_float),
                ("wtype", C.c_int32), ("kvtype", C.c_int32)]


_PP = C.POINTER(C.c_void_p)


class Weights(C.Structure):
    _fields_ = [("tok_embd", C.c_void_p), ("output_norm", C.c_void_p), ("output", C.c_void_p),
                ("attn_norm", _PP), ("wq", _PP), ("wk", _PP), ("wv", _PP), ("wo", _PP),
                ("ffn_norm", _PP), ("ffn_gate", _PP), ("ffn_up", _PP), ("ffn_down", _PP)]


ALLOC_FN = C.CFUNCTYPE(C.c_void_p, C.c_size_t, C.c_void_p)
FREE_FN = C.CFUNCTYPE(None, C.c_void_p, C.c_void_p)


class Allocator(C.Structure):
    _fields_ = [("alloc", ALLOC_FN), ("free", FREE_FN), ("ud", C.c_void_p)]


ABORT_FN = C.CFUNCTYPE(C.c_int, C.c_void_p)


class CtxParams(C.Structure):
    _fields_ = [("n_ctx", C.c_uint32), ("n_batch", C.c_uint32), ("n_ubatch", C.c_uint32),
                ("n_seq_max", C.c_uint32), ("kv_unified", C.c_int32), ("hip_stream", C.c_void_p),
                ("abort_cb", ABORT_FN), ("abort_ud", C.c_void_p)]


class Stats(C.Structure):
    _fields_ = [("n_prefill_calls", C.c_int64), ("n_ubatches", C.c_int64),
                ("n_decode_calls", C.c_int64), ("n_graph_captures", C.c_int64),
                ("n_graph_replays", C.c_int64)]


LOG_FN = C.CFUNCTYPE(None, C.c_int, C.c_char_p, C.c_void_p)

_lib = None


def header_functions() -> list:
    """Names of the functions include/decode.h declares."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dec_[a-z_0-9]+)\s*\(", src)))


def lib() -> C.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise DecodeError(f"{LIB_PATH} is missing: build it with `python decode_amd/build.py`")
    L = C.CDLL(LIB_PATH)
    vp, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
    sig = {
        "dec_model_load": (vp, [vp, vp, vp, vp]),
        "dec_model_tensor_blocks": (i64, [vp, i32, i32, vp, C.c_size_t]),
        "dec_model_free": (None, [vp]),
        "dec_gguf_inspect": (i32, [C.c_char_p, vp]),
        "dec_model_load_gguf": (vp, [C.c_char_p, i32, vp, vp]),
        "dec_model_save_gguf": (i32, [vp, C.c_char_p]),
        "dec_ctx_new": (vp, [vp, vp]),
        "dec_prefill": (i32, [vp, vp, i32, i32, i32]),
        "dec_decode": (i32, [vp, vp, vp, i32]),
        "dec_get_logits": (C.POINTER(C.c_float), [vp, i32]),
        "dec_argmax": (i32, [vp, i32]),
        "dec_argmax_all": (i32, [vp, vp, i32]),
        "dec_seq_pos_max": (i32, [vp, i32]),
        "dec_seq_clear": (i32, [vp, i32]),
        "dec_get_stats": (None, [vp, vp]),
        "dec_ctx_free": (None, [vp]),
        "dec_set_log_callback": (None, [LOG_FN, vp]),
        "dec_set_probe": (i32, [vp, i32, i32]),
        "dec_get_probe": (i32, [vp, C.POINTER(C.c_double), C.POINTER(C.c_int64)]),
        "dec_set_use_graphs": (i32, [vp, i32]),
        "dec_set_step_kernel": (i32, [vp, i32]),
        "dec_version": (C.c_char_p, []),
        "dec_sampler_new": (vp, [vp]),
        "dec_sampler_accept": (i32, [vp, i32]),
        "dec_sampler_sample": (i32, [vp, vp, i32]),
        "dec_sampler_sample_row": (i32, [vp, vp, i32, vp]),
        "dec_sampler_reset": (None, [vp]),
        "dec_sampler_draws": (i64, [vp]),
        "dec_sampler_free": (None, [vp]),
        "dec_sample_row_noalloc": (i32, [vp, vp, i32, C.c_uint64, vp, i32, vp, vp]),
        "dec_measure_stream_read": (i32, [C.c_size_t, i32, vp, C.POINTER(C.c_double)]),
        "dec_measure_mfma_f16": (i32, [i32, i32, vp, C.POINTER(C.c_double)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _ptr(a):
    """Address of a numpy array or torch tensor (host or device)."""
    if isinstance(a, np.ndarray):
        if not a.flags.c_contiguous or a.dtype != np.float32:
            raise ValueError("weights must be C-contiguous float32")
        return a.ctypes.data
    if hasattr(a, "data_ptr"):
        if not a.is_contiguous() or str(a.dtype) != "torch.float32":
            raise ValueError("weights must be contiguous float32")
        return a.data_ptr()
    raise TypeError(type(a))


class TorchAllocator:
    """dec_allocator backed by PyTorch's caching allocator on the current device."""

    def __init__(self):
        import torch
        self._torch = torch
        self._live = {}
        self.c_alloc = ALLOC_FN(self._alloc)
        self.c_free = FREE_FN(self._free)
        self.struct = Allocator(self.c_alloc, self.c_free, None)

    def _alloc(self, nbytes, ud):
        try:
            t = self._torch.empty(int(nbytes), dtype=self._torch.uint8, device="cuda")
        except Exception:
            return None
        p = t.data_ptr()
        self._live[p] = t
        return p

    def _free(self, p, ud):
        self._live.pop(p, None)


def gguf_inspect(path) -> tuple[int, dict | None]:
    """dec_gguf_inspect: (tensor count or negative status, hyper-parameters)."""
    h = Hparams()
    n = int(lib().dec_gguf_inspect(str(path).encode(), C.byref(h)))
    if n < 0:
        return n, None
    return n, {f: getattr(h, f) for f, _ in Hparams._fields_}


class Model:
    @classmethod
    def from_gguf(cls, path, kvtype: int = 1, stream=None, allocator: "TorchAllocator | None" = None) -> "Model":
        """dec_model_load_gguf."""
        self = cls.__new__(cls)
        self.L = lib()
        self.allocator = allocator
        al = C.byref(allocator.struct) if allocator else None
        self.ptr = self.L.dec_model_load_gguf(str(path).encode(), kvtype, al, stream)
        if not self.ptr:
            raise DecodeError(f"dec_model_load_gguf rejected {path}")
        n, hp = gguf_inspect(path)
        hp["kvtype"] = kvtype
        self.hp = hp
        return self

    def save_gguf(self, path) -> None:
        rc = self.L.dec_model_save_gguf(self.ptr, str(path).encode())
        if rc != 0:
            raise DecodeError(f"dec_model_save_gguf returned {rc}")

    def __init__(self, hp: dict, weights: dict, stream=None, allocator: TorchAllocator | None = None):
        L = lib()
        self.L = L
        self.hp = dict(hp)
        self.allocator = allocator
        h = Hparams(hp["n_layer"], hp["n_embd"], hp["n_head"], hp["n_head_kv"], hp["head_dim"],
                    hp["n_ff"], hp["n_vocab"], hp.get("rms_eps", 1e-5), hp.get("rope_base", 10000.0),
                    hp["wtype"], hp["kvtype"])
        keep = []

        def lst(name):
            arr = (C.c_void_p * hp["n_layer"])(*[_ptr(a) for a in weights[name]])
            keep.append(arr)
            return C.cast(arr, _PP)

        w = Weights(_ptr(weights["tok_embd"]), _ptr(weights["output_norm"]), _ptr(weights["output"]),
                    lst("attn_norm"), lst("wq"), lst("wk"), lst("wv"), lst("wo"),
                    lst("ffn_norm"), lst("ffn_gate"), lst("ffn_up"), lst("ffn_down"))
        al = C.byref(allocator.struct) if allocator else None
        self.ptr = L.dec_model_load(C.byref(h), C.byref(w), al, stream)
        if not self.ptr:
            raise DecodeError("dec_model_load failed")

    def tensor_blocks(self, name: str, layer: int = 0) -> np.ndarray:
        tid = TENSOR_IDS[name]
        need = -self.L.dec_model_tensor_blocks(self.ptr, tid, layer, None, 0)
        if need <= 0:
            raise DecodeError("bad tensor id / layer")
        out = np.empty(need, np.uint8)
        n = self.L.dec_model_tensor_blocks(self.ptr, tid, layer, out.ctypes.data, need)
        if n != need:
            raise DecodeError(f"tensor export failed ({n})")
        return out

    def close(self):
        if getattr(self, "ptr", None):
            self.L.dec_model_free(self.ptr)
            self.ptr = None

    def __del__(self):
        self.close()


class SamplerParams(C.Structure):
    """Mirror of dec_sampler_params."""
    _fields_ = [("top_k", C.c_int32), ("top_p", C.c_float), ("min_p", C.c_float), ("temp", C.c_float),
                ("repeat_penalty", C.c_float), ("penalty_last_n", C.c_int32), ("seed", C.c_uint64)]


class Sampler:
    """The device sampler chain (dec_sampler_*)."""

    def __init__(self, top_k=40, top_p=1.0, min_p=0.0, temp=1.0, repeat_penalty=1.0, penalty_last_n=64,
                 seed=0):
        self.L = lib()
        p = SamplerParams(top_k, top_p, min_p, temp, repeat_penalty, penalty_last_n, seed)
        self.ptr = self.L.dec_sampler_new(C.byref(p))
        if not self.ptr:
            raise DecodeError("dec_sampler_new rejected the parameters")

    def accept(self, tokens) -> None:
        for t in np.atleast_1d(np.asarray(tokens, np.int64)):
            if self.L.dec_sampler_accept(self.ptr, int(t)) != 0:
                raise DecodeError("dec_sampler_accept failed")

    def sample(self, ctx, i: int = -1) -> int:
        return int(self.L.dec_sampler_sample(self.ptr, ctx.ptr, i))

    def sample_row(self, logits, stream=None) -> int:
        """logits: float32 numpy array (host) or contiguous torch float32 tensor."""
        if isinstance(logits, np.ndarray):
            a = np.ascontiguousarray(logits, np.float32)
            return int(self.L.dec_sampler_sample_row(self.ptr, a.ctypes.data, a.size, stream))
        return int(self.L.dec_sampler_sample_row(self.ptr, _ptr(logits), logits.numel(), stream))

    def reset(self) -> None:
        self.L.dec_sampler_reset(self.ptr)

    def draws(self) -> int:
        return int(self.L.dec_sampler_draws(self.ptr))

    def close(self):
        if getattr(self, "ptr", None):
            self.L.dec_sampler_free(self.ptr)
            self.ptr = None

    def __del__(self):
        self.close()


def measure_stream_read(nbytes: int = 2 << 30, reps: int = 10, stream=None) -> float:
    """dec_measure_stream_read: attainable HBM read GB/s on the current device."""
    v = C.c_double()
    rc = lib().dec_measure_stream_read(nbytes, reps, stream, C.byref(v))
    if rc != 0:
        raise DecodeError(f"dec_measure_stream_read returned {rc}")
    return float(v.value)


def measure_mfma_f16(iters: int = 20000, reps: int = 5, stream=None) -> float:
    """dec_measure_mfma_f16: attainable f16 MFMA TFLOP/s on the current device."""
    v = C.c_double()
    rc = lib().dec_measure_mfma_f16(iters, reps, stream, C.byref(v))
    if rc != 0:
        raise DecodeError(f"dec_measure_mfma_f16 returned {rc}")
    return float(v.value)


NOALLOC_MAX_VOCAB = 32768


def sample_row_noalloc(logits, token_out, hist=(), draw=0, stream=None, top_k=40, top_p=1.0, min_p=0.0,
                       temp=1.0, repeat_penalty=1.0, penalty_last_n=64, seed=0) -> int:
    """dec_sample_row_noalloc: enqueue one draw of the chain on ``logits``
    (float32 numpy array or contiguous torch tensor, host or device); the token
    is written to ``token_out`` (an int32 torch tensor on the device).  Returns
    the call's status (0 enqueued)."""
    p = SamplerParams(top_k, top_p, min_p, temp, repeat_penalty, penalty_last_n, seed)
    h = np.ascontiguousarray(np.asarray(hist, np.int32))
    if isinstance(logits, np.ndarray):
        row = np.ascontiguousarray(logits, np.float32)
        rp, n = row.ctypes.data, row.size
    else:
        rp, n = _ptr(logits), logits.numel()
    if str(token_out.dtype) != "torch.int32" or not token_out.is_contiguous():
        raise ValueError("token_out must be a contiguous int32 tensor")
    return int(lib().dec_sample_row_noalloc(C.byref(p), h.ctypes.data if h.size else None, h.size, int(draw),
                                            rp, n, token_out.data_ptr(), stream))


class Context:
    def __init__(self, model: Model, n_ctx=0, n_batch=0, n_ubatch=0, n_seq_max=1, stream=None,
                 abort=None):
        self.model = model
        self.L = model.L
        self._abort = ABORT_FN(abort) if abort else ABORT_FN()
        p = CtxParams(n_ctx, n_batch, n_ubatch, n_seq_max, 0, stream, self._abort, None)
        self.ptr = self.L.dec_ctx_new(model.ptr, C.byref(p))
        if not self.ptr:
            raise DecodeError("dec_ctx_new failed")
        self.n_vocab = model.hp["n_vocab"]

    def prefill(self, tokens, seq: int = 0, output_all: bool = False) -> int:
        t = np.ascontiguousarray(tokens, np.int32)
        return int(self.L.dec_prefill(self.ptr, t.ctypes.data, t.size, seq, int(output_all)))

    def decode(self, tokens, seqs=None) -> int:
        t = np.ascontiguousarray(tokens, np.int32).ravel()
        s = np.arange(t.size, dtype=np.int32) if seqs is None else np.ascontiguousarray(seqs, np.int32)
        return int(self.L.dec_decode(self.ptr, t.ctypes.data, s.ctypes.data, t.size))

    def logits(self, i: int = -1):
        p = self.L.dec_get_logits(self.ptr, i)
        if not p:
            return None
        return np.ctypeslib.as_array(p, shape=(self.n_vocab,)).copy()

    def argmax(self, i: int = -1) -> int:
        return int(self.L.dec_argmax(self.ptr, i))

    def argmax_all(self) -> np.ndarray:
        out = np.empty(1 << 16, np.int32)
        n = self.L.dec_argmax_all(self.ptr, out.ctypes.data, out.size)
        if n < 0:
            raise DecodeError("dec_argmax_all failed")
        return out[:n].copy()

    def pos_max(self, seq: int = 0) -> int:
        return int(self.L.dec_seq_pos_max(self.ptr, seq))

    def clear(self, seq: int = 0) -> int:
        return int(self.L.dec_seq_clear(self.ptr, seq))

    def stats(self) -> dict:
        s = Stats()
        self.L.dec_get_stats(self.ptr, C.byref(s))
        return {k: int(getattr(s, k)) for k, _ in Stats._fields_}

    def set_probe(self, role: int, layer: int = 0) -> int:
        return int(self.L.dec_set_probe(self.ptr, role, layer))

    def probe(self):
        ms, n = C.c_double(), C.c_int64()
        if self.L.dec_get_probe(self.ptr, C.byref(ms), C.byref(n)) != 0:
            return None
        return float(ms.value), int(n.value)

    def use_graphs(self, on: bool) -> bool:
        return bool(self.L.dec_set_use_graphs(self.ptr, int(on)))

    def step_kernel(self, on: int = -1) -> int:
        """One-token decode steps as one persistent kernel: 1 on, 0 off, -1
        query.  Returns the setting before the call, or -1 when the context
        cannot use it."""
        return int(self.L.dec_set_step_kernel(self.ptr, int(on)))

    def close(self):
        if getattr(self, "ptr", None):
            self.L.dec_ctx_free(self.ptr)
            self.ptr = None

    def __del__(self):
        self.close()
