"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol the header declares, validates configs and arguments before it
touches a device, and reports a missing device as DUALAR_ERR_NO_DEVICE."""
import ctypes as C
import os
import re

import pytest

import synth
from dual_autoregressive_tts_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return bd.load_library()


@pytest.mark.parametrize("path", [bd.LIB_PATH, bd.CHECKED_LIB_PATH], ids=["normal", "checked"])
def test_exports_every_declared_symbol(path):
    # both builds of the library (the checked one has the device index checks)
    lib = bd.load_library(path)
    hdr = open(os.path.join(ROOT, "include", "dualar.h")).read()
    declared = set(re.findall(r"\b(dualar_[a-z_]+)\s*\(", hdr))
    assert declared == set(bd.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.dualar_status_string(-9) == b"device index check failed"


def test_status_strings(lib):
    for code in bd.STATUS:
        assert lib.dualar_status_string(code)
    assert lib.dualar_status_string(0) == b"ok"


@pytest.mark.parametrize("name,batch,seq", [("tiny", 1, 64), ("s2", 1, 1344), ("s2", 32, 4352)])
def test_workspace_bytes_valid(lib, name, batch, seq):
    m = synth.model(name)
    n = bd.workspace_bytes(bd.make_config(m, batch, seq))
    esz = 2 if m["weight_dtype"] == "bf16" else 4
    kv = 2 * m["n_layer"] * batch * m["n_kv_head"] * seq * m["head_dim"] * esz
    assert kv < n < kv + 2 * 1024 ** 3


def test_inherit_fast_fields_give_same_layout(lib):
    m = synth.model("s2")
    a = bd.workspace_bytes(bd.make_config(m, 2, 2048))
    b = bd.workspace_bytes(bd.make_config(m, 2, 2048, inherit_fast=True))
    assert a == b > 0


@pytest.mark.parametrize("field,value", [
    ("dim", 2500), ("head_dim", 96), ("n_kv_head", 3), ("semantic_end_id", 155000),
    ("end_id", 151700), ("num_codebooks", 1), ("codebook_size", 8192), ("weight_dtype", 7),
    ("fast_dim", 1024), ("max_batch", 0), ("max_batch", 1000), ("max_seq_len", 1), ("rope_base", 0.5),
])
def test_invalid_config_rejected(lib, field, value):
    cfg = bd.make_config(synth.model("s2"), 1, 2048)
    setattr(cfg, field, value)
    assert lib.dualar_workspace_bytes(C.byref(cfg)) == 0
    h = C.c_void_p()
    st = lib.dualar_create(C.byref(cfg), None, C.c_void_p(256), 1 << 40, None, C.byref(h))
    assert st == -1 and not h.value
    assert lib.dualar_last_error(None)


def _fake_weights(m):
    # non-NULL pointers that are never dereferenced: create() fails before use
    def layers(n, qk):
        arr = (bd.LayerWeights * n)()
        for i in range(n):
            for f in bd._LAYER_FIELDS:
                setattr(arr[i], f, 4096 if (qk or f not in ("q_norm", "k_norm")) else None)
        return arr
    w = bd.Weights()
    for f in ("tok_embedding", "codebook_embedding", "norm", "fast_embeddings", "fast_norm", "fast_output"):
        setattr(w, f, 4096)
    w.layers = layers(m["n_layer"], m["slow_qk_norm"])
    w.fast_layers = layers(m["n_fast_layer"], m["fast_qk_norm"])
    return w


def test_create_checks_before_device(lib):
    m = synth.model("tiny")
    cfg = bd.make_config(m, 1, 64)
    need = lib.dualar_workspace_bytes(C.byref(cfg))
    w = _fake_weights(m)
    h = C.c_void_p()
    assert lib.dualar_create(C.byref(cfg), None, C.c_void_p(256), need, None, C.byref(h)) == -1
    assert lib.dualar_create(C.byref(cfg), C.byref(w), None, need, None, C.byref(h)) == -1
    assert lib.dualar_create(C.byref(cfg), C.byref(w), C.c_void_p(257), need, None, C.byref(h)) == -1
    assert lib.dualar_create(C.byref(cfg), C.byref(w), C.c_void_p(256), need - 1, None, C.byref(h)) == -3
    w.layers[1].w2 = None
    assert lib.dualar_create(C.byref(cfg), C.byref(w), C.c_void_p(256), need, None, C.byref(h)) == -1
    w.layers[1].w2 = 4096 + 8          # not 16-byte aligned
    assert lib.dualar_create(C.byref(cfg), C.byref(w), C.c_void_p(256), need, None, C.byref(h)) == -1
    assert b"aligned" in lib.dualar_last_error(None)
    assert not h.value


def test_create_checks_w4_forms(lib):
    # 4-bit matrices (W4A16): batches of at most 8, prefill steps of one
    # position or of at least 256 (the 2-D tile form);
    # a 4-bit form may stand in for a missing bf16 matrix, not a missing one of
    # both; q/k/v share a form; pointers 16-byte aligned
    import torch
    m = synth.model("tiny", weight_dtype="bf16", dim=512, ffn_dim=1024, fast_dim=512, fast_ffn_dim=1024,
                    n_head=4, n_kv_head=1, head_dim=128, fast_n_head=4, fast_n_kv_head=1, fast_head_dim=128)
    w = _fake_weights(m)
    l4 = (bd.LayerW4 * m["n_layer"])()
    for j in range(7):
        l4[0].q4[j] = 8192
        l4[0].s4[j] = 8192
    w.layers_w4 = l4
    w.layers[0].wq = None                                   # given in 4-bit form only
    h = C.c_void_p()

    def create(batch, pc):
        cfg = bd.make_config(m, batch, 64, prefill_chunk=pc)
        need = lib.dualar_workspace_bytes(C.byref(cfg))
        return lib.dualar_create(C.byref(cfg), C.byref(w), C.c_void_p(256), need, None, C.byref(h))

    assert create(9, 1) == -1 and b"max_batch at most 8" in lib.dualar_last_error(None)
    for pc in (2, 255):
        assert create(1, pc) == -1 and b"prefill_chunk 1 or at least 256" in lib.dualar_last_error(None)
    if not torch.cuda.is_available():
        for batch, pc in ((1, 1), (1, 256), (1, 0), (4, 1), (3, 0), (8, 1)):   # 0: the default chunk
            assert create(batch, pc) == -2                  # valid: fails only for want of a device
    l4[0].q4[1] = None                                      # wk bf16 while wq, wv are 4-bit
    assert create(1, 1) == -1 and b"all 4-bit or all bf16" in lib.dualar_last_error(None)
    l4[0].q4[1] = 8192
    l4[0].s4[6] = 8192 + 2                                  # unaligned scales
    assert create(1, 1) == -1 and b"aligned" in lib.dualar_last_error(None)
    l4[0].s4[6] = 8192
    l4[0].q4[0] = l4[0].q4[1] = l4[0].q4[2] = None          # wq now missing in both forms
    assert create(1, 1) == -1
    assert not h.value


def test_create_without_gpu_reports_no_device(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    m = synth.model("tiny")
    cfg = bd.make_config(m, 1, 64)
    need = lib.dualar_workspace_bytes(C.byref(cfg))
    h = C.c_void_p()
    st = lib.dualar_create(C.byref(cfg), C.byref(_fake_weights(m)), C.c_void_p(256), need, None, C.byref(h))
    assert st == -2 and not h.value


def test_null_context_calls(lib):
    s = bd.Sampling(1.0, 1.0, 1, 0)
    assert lib.dualar_prefill(None, 1, None, 1, None, C.byref(s), None, None, None) == -1
    assert lib.dualar_decode_frames(None, 1, C.byref(s), None, None, None, None) == -1
    assert lib.dualar_fast_frames(None, 1, 1, None, None, C.byref(s), None, None, None) == -1
    assert lib.dualar_fast_teacher_forced(None, 1, None, None, None) == -1
    assert lib.dualar_sync(None, None) == -1
    ids = (C.c_int32 * 1)(0)
    assert lib.dualar_reset(None, ids, 1) == -1
    assert lib.dualar_reset(None, None, 0) == -1
    lib.dualar_destroy(None)


def test_create_static_validation_without_gpu(lib):
    # dualar_create_static: NULL out / bad config -> INVALID_ARG; a config
    # whose workspace exceeds the static array -> WORKSPACE before any device
    # call; a config that fits reaches the device lookup (NO_DEVICE here)
    import torch
    m = synth.model("tiny")
    h = C.c_void_p()
    small = bd.make_config(m, 1, 64, prefill_chunk=16)
    assert lib.dualar_create_static(C.byref(small), C.byref(_fake_weights(m)), None, None) == -1
    bad = bd.make_config(m, 1, 64, prefill_chunk=16)
    bad.n_layer = 0
    assert lib.dualar_create_static(C.byref(bad), C.byref(_fake_weights(m)), None, C.byref(h)) == -1
    big = bd.make_config(m, 8, 4096)
    assert lib.dualar_workspace_bytes(C.byref(big)) > 32 << 20
    assert lib.dualar_create_static(C.byref(big), C.byref(_fake_weights(m)), None, C.byref(h)) == -3
    assert b"static workspace" in lib.dualar_last_error(None) and not h.value
    assert lib.dualar_workspace_bytes(C.byref(small)) <= 32 << 20
    if not torch.cuda.is_available():
        assert lib.dualar_create_static(C.byref(small), C.byref(_fake_weights(m)), None, C.byref(h)) == -2
        assert not h.value
