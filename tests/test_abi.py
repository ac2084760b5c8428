"""The C-ABI library loads on the CPU, exports every function its header
declares, and rejects invalid arguments before touching the device."""
import ctypes as C

import pytest


@pytest.fixture(scope="module")
def dec():
    import decode_amd
    return decode_amd


def test_exports_every_declared_function(dec):
    names = dec.header_functions()
    assert len(names) >= 15
    L = dec.lib()
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    assert b"gfx950" in L.dec_version()


def test_null_and_invalid_arguments(dec):
    L = dec.lib()
    assert not L.dec_model_load(None, None, None, None)
    bad = dec.Hparams(2, 256, 4, 3, 64, 688, 1024, 1e-5, 1e4, dec.F32, dec.F32)   # 4 % 3 != 0
    w = dec.Weights()
    assert not L.dec_model_load(C.byref(bad), C.byref(w), None, None)
    bad_hd = dec.Hparams(2, 256, 4, 4, 48, 688, 1024, 1e-5, 1e4, dec.F32, dec.F32)
    assert not L.dec_model_load(C.byref(bad_hd), C.byref(w), None, None)
    bad_q = dec.Hparams(2, 256, 4, 4, 64, 688, 1024, 1e-5, 1e4, dec.Q4_0, dec.F16)  # 688 % 32
    assert not L.dec_model_load(C.byref(bad_q), C.byref(w), None, None)
    assert not L.dec_ctx_new(None, None)
    assert L.dec_prefill(None, None, 0, 0, 0) == -1
    assert L.dec_decode(None, None, None, 0) == -1
    assert not L.dec_get_logits(None, -1)
    assert L.dec_argmax(None, -1) == -1
    assert L.dec_seq_pos_max(None, 0) == -1
    assert L.dec_seq_clear(None, 0) == -1
    assert L.dec_model_tensor_blocks(None, 0, 0, None, 0) == 0
    L.dec_model_free(None)
    L.dec_ctx_free(None)


def test_log_callback_receives_errors(dec):
    L = dec.lib()
    got = []
    cb = dec.LOG_FN(lambda level, msg, ud: got.append((level, msg)))
    L.dec_set_log_callback(cb, None)
    try:
        assert not L.dec_model_load(None, None, None, None)
    finally:
        L.dec_set_log_callback(dec.LOG_FN(), None)
    assert got and got[0][0] == 3 and b"invalid" in got[0][1]


def test_product_path_does_not_import_the_oracle():
    import os
    import re
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    pkg = os.path.join(root, "decode_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                src = open(os.path.join(dirpath, f), errors="ignore").read()
                assert not re.search(r"\boracle\b|liboracle|orc_", src), f


def test_shape_limits_rejected_before_the_device(dec):
    L = dec.lib()
    w = dec.Weights()
    wide = dec.Hparams(2, 16384 + 32, 4, 4, 64, 512, 1024, 1e-5, 1e4, dec.Q4_0, dec.F16)
    assert not L.dec_model_load(C.byref(wide), C.byref(w), None, None)
    wide_ff = dec.Hparams(2, 256, 4, 4, 64, 16384 + 32, 1024, 1e-5, 1e4, dec.Q8_0, dec.F16)
    assert not L.dec_model_load(C.byref(wide_ff), C.byref(w), None, None)
    gqa16 = dec.Hparams(2, 256, 16, 1, 64, 512, 1024, 1e-5, 1e4, dec.Q8_0, dec.F16)
    assert not L.dec_model_load(C.byref(gqa16), C.byref(w), None, None)
    # Q4_K rows are whole 256-weight super-blocks (d, n_head * head_dim, n_ff)
    for d, nh, ff in ((288, 4, 512), (256, 2, 512), (256, 4, 544)):
        k4 = dec.Hparams(2, d, nh, nh, 64, ff, 1024, 1e-5, 1e4, dec.Q4_K, dec.F16)
        assert not L.dec_model_load(C.byref(k4), C.byref(w), None, None)


def test_noalloc_sampler_rejects_arguments_before_the_device(dec):
    L = dec.lib()
    p = dec.SamplerParams(40, 1.0, 0.0, 1.0, 1.0, 64, 0)
    buf = (C.c_float * 8)()
    tok = (C.c_int32 * 1)()
    addr, taddr = C.addressof(buf), C.addressof(tok)
    assert L.dec_sample_row_noalloc(None, None, 0, 0, addr, 100, taddr, None) == -1
    assert L.dec_sample_row_noalloc(C.byref(p), None, 0, 0, None, 100, taddr, None) == -1
    assert L.dec_sample_row_noalloc(C.byref(p), None, 0, 0, addr, 100, None, None) == -1
    assert L.dec_sample_row_noalloc(C.byref(p), None, 0, 0, addr, 39, taddr, None) == -1      # below top_k
    assert L.dec_sample_row_noalloc(C.byref(p), None, 3, 0, addr, 100, taddr, None) == -1     # hist missing
    assert L.dec_sample_row_noalloc(C.byref(p), None, 65, 0, addr, 100, taddr, None) == -1
    big = dec.NOALLOC_MAX_VOCAB + 1
    assert L.dec_sample_row_noalloc(C.byref(p), None, 0, 0, addr, big, taddr, None) == -4
