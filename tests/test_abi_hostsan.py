"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU needed).

tests/hostsan/build_hostsan.py compiles the library with its host code
instrumented (sanitizer flags on the host pass only) and links it with
tests/hostsan/abi_hostsan_driver.cpp.  The driver feeds every config below
through dualar_workspace_bytes, dualar_create (NULL weights, then placeholder
weights in layer arrays of exactly the configured lengths), and
dualar_create_static, then calls every entry point with a NULL context and
prints every status string.  The run must end cleanly with no sanitizer
report (any report aborts it), and print what the same calls print through
ctypes on the normal library.

The configs are valid S2-shaped and small ones plus every single-field
mutation the validation rejects and extreme values chosen to overflow naive
size arithmetic (2^31 - 1 positions or sequences, 2^30 dims, negative
counts).
"""
import ctypes as C
import math
import os
import subprocess
import sys

import pytest

import synth
from dual_autoregressive_tts_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "tests", "hostsan"))

I32_MAX = 2 ** 31 - 1


def _configs():
    out = []
    for name, batch, seq, kw in (("tiny", 1, 64, {}), ("tiny", 4, 300, {"prefill_chunk": 16}),
                                 ("s2", 1, 1344, {}), ("s2", 32, 4352, {}), ("s2", 2, 2048, {"inherit_fast": True}),
                                 ("s2", 1, 16448, {"prefill_chunk": 1})):
        out.append(bd.make_config(synth.model(name), batch, seq, **kw))
    mutations = [
        ("dim", 2500), ("dim", 0), ("dim", -512), ("dim", 1 << 30), ("head_dim", 96), ("head_dim", 0),
        ("n_kv_head", 3), ("n_kv_head", 0), ("n_head", -32), ("n_layer", 0), ("n_layer", -1), ("n_layer", 1 << 20),
        ("n_fast_layer", 0), ("n_fast_layer", -4), ("ffn_dim", I32_MAX), ("vocab_size", I32_MAX), ("vocab_size", 0),
        ("semantic_end_id", 155000), ("semantic_begin_id", -1), ("end_id", 151700), ("end_id", -7),
        ("num_codebooks", 1), ("num_codebooks", 1 << 30), ("codebook_size", 8192), ("codebook_size", 0),
        ("weight_dtype", 7), ("kv_dtype", 9), ("fast_dim", 1024), ("fast_head_dim", 96), ("fast_n_head", 7),
        ("fast_qk_norm", 5), ("fast_qk_norm", -2), ("slow_qk_norm", 2), ("scale_codebook_embeddings", -1),
        ("fast_ffn_dim", -512), ("fast_n_kv_head", -8), ("max_batch", 0), ("max_batch", 1000), ("max_batch", I32_MAX),
        ("max_seq_len", 1), ("max_seq_len", I32_MAX), ("max_seq_len", -5), ("prefill_chunk", -5),
        ("prefill_chunk", 1 << 30), ("rope_base", 0.5), ("rope_base", math.nan), ("rope_base", math.inf),
        ("norm_eps", -1.0), ("norm_eps", math.nan), ("semantic_head", 3),
    ]
    for field, value in mutations:
        c = bd.make_config(synth.model("s2"), 2, 2048)
        setattr(c, field, value)
        out.append(c)
    return out


N_VALID = 6      # the first six configs are valid; every mutation is rejected


def _fake(k):
    return 4096 + 16 * k


def _line_via_ctypes(lib, cfg):
    """What the driver prints for one config, by the same calls through ctypes."""
    ws = lib.dualar_workspace_bytes(C.byref(cfg))
    h = C.c_void_p()
    size = ws if ws else 1 << 40
    st_null = lib.dualar_create(C.byref(cfg), None, C.c_void_p(256), size, None, C.byref(h))

    def layers(n):
        arr = (bd.LayerWeights * max(n, 1))()
        k = 0
        for i in range(n):
            for f in bd._LAYER_FIELDS:
                setattr(arr[i], f, _fake(k))
                k += 1
        return arr if n else None
    n = cfg.n_layer if 0 <= cfg.n_layer <= 4096 else 0
    fn = cfg.n_fast_layer if 0 <= cfg.n_fast_layer <= 4096 else 0
    w = bd.Weights()
    w.tok_embedding, w.codebook_embedding, w.norm = _fake(100000), _fake(100001), _fake(100002)
    sl, fl = layers(n), layers(fn)
    w.layers = C.cast(sl, C.POINTER(bd.LayerWeights)) if sl is not None else None
    w.fast_layers = C.cast(fl, C.POINTER(bd.LayerWeights)) if fl is not None else None
    w.fast_embeddings, w.fast_norm, w.fast_output = _fake(100003), _fake(100004), _fake(100005)
    st_fake = lib.dualar_create(C.byref(cfg), C.byref(w), C.c_void_p(256), size, None, C.byref(h))
    e1 = lib.dualar_last_error(None).decode()
    st_static = lib.dualar_create_static(C.byref(cfg), C.byref(w), None, C.byref(h))
    e2 = lib.dualar_last_error(None).decode()
    return f"ws={ws} null={st_null} fake={st_fake} static={st_static} handle={int(bool(h.value))} err={e1} | {e2}"


@pytest.fixture(scope="module")
def hostsan_bin():
    if not os.path.exists(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    import torch
    if torch.cuda.is_available():
        pytest.skip("the driver's placeholder weights are for a host without a GPU")
    import build_hostsan
    return build_hostsan.build()


def test_abi_host_code_is_sanitizer_clean(hostsan_bin, tmp_path):
    cfgs = _configs()
    blob = tmp_path / "configs.bin"
    blob.write_bytes(b"".join(bytes(c) for c in cfgs))
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([hostsan_bin, str(blob)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    lines = r.stdout.splitlines()
    assert lines[-1] == f"records {len(cfgs)}"
    lib = bd.load_library()
    want = [_line_via_ctypes(lib, c) for c in cfgs]
    assert lines[:len(cfgs)] == want
    # the valid configs get as far as the device lookup, the mutated ones not
    assert all(" fake=-2 " in ln for ln in lines[:N_VALID]), lines[:N_VALID]
    assert all(" null=-1 fake=-1 static=-1 " in ln for ln in lines[N_VALID:len(cfgs)]), lines[N_VALID:len(cfgs)]
    assert lines[len(cfgs)].startswith("null-ctx ") and set(lines[len(cfgs)].split()[1:]) == {
        f"{k}=-1" for k in ("prefill", "decode", "fast", "fast_tf", "sync", "reset", "reset0", "prof_begin",
                            "prof_end")}
    status = dict(ln.split(" ", 2)[1:] for ln in lines[len(cfgs) + 1:-1])
    for code in range(-10, 2):
        assert status[str(code)] == lib.dualar_status_string(code).decode()
