"""ctypes binding of libdualar.so (include/dualar.h).

Argument marshalling only: every step of the decode path runs in the HIP
library.  PyTorch supplies device memory (weights, workspace, inputs,
outputs) and the stream.  If the library is missing this module raises on
import of the library; there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# DUALAR_LIBRARY selects another build of the library (e.g. the checked one)
LIB_PATH = os.environ.get("DUALAR_LIBRARY") or os.path.join(HERE, "libdualar.so")
CHECKED_LIB_PATH = os.path.join(HERE, "libdualar_checked.so")

OK = 0
STATUS = {0: "OK", -1: "INVALID_ARG", -2: "NO_DEVICE", -3: "WORKSPACE", -4: "CONTEXT_FULL",
          -5: "BAD_TOKEN", -6: "STATE", -7: "HIP", -8: "DEVICE_FAULT", -9: "DEVICE_INDEX"}
F32, BF16 = 0, 1


class DualARError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class Config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "n_layer", "dim", "n_head", "n_kv_head", "head_dim", "ffn_dim", "vocab_size",
        "n_fast_layer", "fast_dim", "fast_n_head", "fast_n_kv_head", "fast_head_dim", "fast_ffn_dim",
        "slow_qk_norm", "fast_qk_norm", "num_codebooks", "codebook_size",
        "semantic_begin_id", "semantic_end_id", "end_id", "scale_codebook_embeddings")] + [
        ("rope_base", C.c_float), ("norm_eps", C.c_float),
        ("weight_dtype", C.c_int32), ("max_batch", C.c_int32), ("max_seq_len", C.c_int32),
        ("kv_dtype", C.c_int32), ("prefill_chunk", C.c_int32), ("semantic_head", C.c_int32)]


_LAYER_FIELDS = ("attention_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "ffn_norm", "w1", "w3", "w2")


class LayerWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in _LAYER_FIELDS]


W4_MATS = ("wq", "wk", "wv", "wo", "w1", "w3", "w2")


class LayerW4(C.Structure):
    _fields_ = [("q4", C.c_void_p * 7), ("s4", C.c_void_p * 7)]


class Weights(C.Structure):
    _fields_ = [("tok_embedding", C.c_void_p), ("codebook_embedding", C.c_void_p), ("norm", C.c_void_p),
                ("layers", C.POINTER(LayerWeights)), ("fast_layers", C.POINTER(LayerWeights)),
                ("fast_embeddings", C.c_void_p), ("fast_norm", C.c_void_p), ("fast_output", C.c_void_p),
                ("layers_w4", C.POINTER(LayerW4)), ("fast_layers_w4", C.POINTER(LayerW4))]


class Sampling(C.Structure):
    _fields_ = [("temperature", C.c_float), ("top_p", C.c_float), ("greedy", C.c_int32),
                ("min_frames", C.c_int32), ("ras_window", C.c_int32), ("ras_temperature", C.c_float),
                ("ras_top_p", C.c_float)]


class Taps(C.Structure):
    _fields_ = [("fused_x", C.c_void_p), ("slow_hidden", C.c_void_p), ("slow_logits", C.c_void_p),
                ("fast_logits", C.c_void_p)]


# Every symbol the header declares.
EXPORTS = ("dualar_workspace_bytes", "dualar_create", "dualar_create_static", "dualar_prefill", "dualar_decode_frames",
           "dualar_fast_frames", "dualar_fast_teacher_forced", "dualar_sync", "dualar_reset",
           "dualar_profile_begin", "dualar_profile_end",
           "dualar_destroy", "dualar_status_string", "dualar_last_error")
K_GEMV, K_ATTN, K_SAMPLE, K_EMBED, K_GEMV_SWIGLU = 0, 1, 2, 3, 4

_libs = {}


def load_library(path: str = LIB_PATH):
    """Load a build of the library (default libdualar.so) and declare its
    signatures; fails loudly if it is absent.  Each path is loaded once."""
    path = os.path.abspath(path)
    if path in _libs:
        return _libs[path]
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} is not built; run `python -m dual_autoregressive_tts_amd.build --all`")
    lib = C.CDLL(path)
    P, I32, VP = C.POINTER, C.c_int32, C.c_void_p
    lib.dualar_workspace_bytes.argtypes = [P(Config)]
    lib.dualar_workspace_bytes.restype = C.c_size_t
    lib.dualar_create.argtypes = [P(Config), P(Weights), VP, C.c_size_t, VP, P(VP)]
    lib.dualar_create.restype = I32
    lib.dualar_create_static.argtypes = [P(Config), P(Weights), VP, P(VP)]
    lib.dualar_create_static.restype = I32
    lib.dualar_prefill.argtypes = [VP, I32, VP, I32, P(I32), P(Sampling), VP, VP, P(Taps)]
    lib.dualar_prefill.restype = I32
    lib.dualar_decode_frames.argtypes = [VP, I32, P(Sampling), VP, VP, VP, P(Taps)]
    lib.dualar_decode_frames.restype = I32
    lib.dualar_fast_frames.argtypes = [VP, I32, I32, VP, VP, P(Sampling), VP, VP, P(Taps)]
    lib.dualar_fast_frames.restype = I32
    lib.dualar_fast_teacher_forced.argtypes = [VP, I32, VP, VP, VP]
    lib.dualar_fast_teacher_forced.restype = I32
    lib.dualar_sync.argtypes = [VP, P(I32)]
    lib.dualar_sync.restype = I32
    lib.dualar_reset.argtypes = [VP, P(I32), I32]
    lib.dualar_reset.restype = I32
    lib.dualar_profile_begin.argtypes = [VP, I32]
    lib.dualar_profile_begin.restype = I32
    lib.dualar_profile_end.argtypes = [VP, P(C.c_int64), P(C.c_double), P(C.c_double)]
    lib.dualar_profile_end.restype = I32
    lib.dualar_destroy.argtypes = [VP]
    lib.dualar_destroy.restype = None
    lib.dualar_status_string.argtypes = [I32]
    lib.dualar_status_string.restype = C.c_char_p
    lib.dualar_last_error.argtypes = [VP]
    lib.dualar_last_error.restype = C.c_char_p
    _libs[path] = lib
    return lib


def make_config(m: dict, max_batch: int, max_seq_len: int, inherit_fast: bool = False,
                prefill_chunk: int = 0) -> Config:
    """Model dict (synth.MODELS layout) -> dualar_config.  With inherit_fast,
    fast_* sizes are passed as 0 (inherit) where they equal the slow ones.
    prefill_chunk: prompt positions per sequence per prefill step (0 = the
    library's choice, 8192 rows per step)."""
    c = Config()
    for f in ("n_layer", "dim", "n_head", "n_kv_head", "head_dim", "ffn_dim", "vocab_size",
              "n_fast_layer", "fast_dim", "fast_n_head", "fast_n_kv_head", "fast_head_dim",
              "fast_ffn_dim", "slow_qk_norm", "fast_qk_norm", "num_codebooks", "codebook_size",
              "semantic_begin_id", "semantic_end_id", "end_id", "scale_codebook_embeddings"):
        setattr(c, f, int(m[f]))
    if inherit_fast:
        for f, s in (("fast_dim", "dim"), ("fast_n_head", "n_head"), ("fast_n_kv_head", "n_kv_head"),
                     ("fast_head_dim", "head_dim"), ("fast_ffn_dim", "ffn_dim")):
            if m[f] == m[s]:
                setattr(c, f, 0)
        if m["fast_qk_norm"] == m["slow_qk_norm"]:
            c.fast_qk_norm = -1
    c.rope_base = float(m["rope_base"])
    c.norm_eps = float(m["norm_eps"])
    c.weight_dtype = BF16 if m["weight_dtype"] == "bf16" else F32
    c.max_batch = int(max_batch)
    c.max_seq_len = int(max_seq_len)
    kv = m.get("kv_dtype")
    c.kv_dtype = -1 if kv is None else (BF16 if kv == "bf16" else F32)
    c.prefill_chunk = prefill_chunk
    c.semantic_head = int(m.get("semantic_head", 0))
    return c


def workspace_bytes(cfg: Config, lib=None) -> int:
    return int((lib or load_library()).dualar_workspace_bytes(C.byref(cfg)))


def upload_weights(m: dict, w: dict, device="cuda"):
    """numpy weights from synth.make_weights -> device tensors (bf16 or fp32)."""
    import torch
    out = {}
    for k, v in w.items():
        t = torch.from_numpy(np.ascontiguousarray(v))
        if k.endswith(".q4"):
            pass                                     # packed 4-bit values stay bytes
        elif m["weight_dtype"] == "bf16":
            t = t.view(torch.int16).view(torch.bfloat16)
        out[k] = t.to(device)
    return out


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


class DualAR:
    """One decode context (dualar_create) over device weights."""

    def __init__(self, m: dict, dev_weights: dict, max_batch: int, max_seq_len: int, stream=None,
                 inherit_fast: bool = False, prefill_chunk: int = 0, static_workspace: bool = False,
                 library: str | None = None):
        """static_workspace: dualar_create_static (the library's static device
        workspace, nothing allocated here; one such context per GPU at a time).
        library: path of another build of the library (e.g. CHECKED_LIB_PATH)."""
        import torch
        self.torch = torch
        self.lib = load_library() if library is None else load_library(library)
        self.m = m
        self.N = m["num_codebooks"]
        self.cfg = make_config(m, max_batch, max_seq_len, inherit_fast, prefill_chunk)
        self.ws_bytes = workspace_bytes(self.cfg, self.lib)
        if self.ws_bytes == 0:
            raise DualARError(-1, "invalid config")
        self.dev_weights = dev_weights
        self.workspace = None if static_workspace else torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        self._keep = []
        self.wstruct = self._weights_struct(dev_weights)
        h = C.c_void_p()
        if static_workspace:
            st = self.lib.dualar_create_static(C.byref(self.cfg), C.byref(self.wstruct),
                                               C.c_void_p(self.stream.cuda_stream), C.byref(h))
        else:
            st = self.lib.dualar_create(C.byref(self.cfg), C.byref(self.wstruct), _ptr(self.workspace),
                                        self.ws_bytes, C.c_void_p(self.stream.cuda_stream), C.byref(h))
        if st != OK:
            raise DualARError(st, self.lib.dualar_last_error(None).decode())
        self.h = h
        self.batch = 0

    def _weights_struct(self, w):
        m = self.m

        def layers(prefix, n):
            arr = (LayerWeights * n)()
            for i in range(n):
                for f in _LAYER_FIELDS:
                    t = w.get(f"{prefix}.{i}.{f}")
                    setattr(arr[i], f, None if t is None else t.data_ptr())
            self._keep.append(arr)
            return arr
        def layers_w4(prefix, n):
            # None (NULL) unless some matrix of these layers is given as 4-bit groups
            if not any(k.startswith(prefix + ".") and k.endswith(".q4") for k in w):
                return None
            arr = (LayerW4 * n)()
            for i in range(n):
                for j, f in enumerate(W4_MATS):
                    q, sc = w.get(f"{prefix}.{i}.{f}.q4"), w.get(f"{prefix}.{i}.{f}.s4")
                    arr[i].q4[j] = None if q is None else q.data_ptr()
                    arr[i].s4[j] = None if sc is None else sc.data_ptr()
            self._keep.append(arr)
            return arr
        s = Weights()
        s.tok_embedding = w["tok_embedding"].data_ptr()
        s.codebook_embedding = w["codebook_embedding"].data_ptr()
        s.norm = w["norm"].data_ptr()
        s.layers = layers("layers", m["n_layer"])
        s.fast_layers = layers("fast_layers", m["n_fast_layer"])
        s.fast_embeddings = w["fast_embeddings"].data_ptr()
        s.fast_norm = w["fast_norm"].data_ptr()
        s.fast_output = w["fast_output"].data_ptr()
        s.layers_w4 = layers_w4("layers", m["n_layer"])
        s.fast_layers_w4 = layers_w4("fast_layers", m["n_fast_layer"])
        return s

    def _check(self, st):
        if st != OK:
            raise DualARError(st, self.lib.dualar_last_error(self.h).decode())

    @staticmethod
    def sampling(greedy=True, temperature=1.0, top_p=1.0, min_frames=0, ras_window=0, ras_temperature=1.0,
                 ras_top_p=0.9) -> Sampling:
        """ras_window > 0 turns on the slow loop breaker (the pages' window is
        10); its draws then take slot N of N + 1 uniforms per sequence."""
        return Sampling(float(temperature), float(top_p), int(bool(greedy)), int(min_frames), int(ras_window),
                        float(ras_temperature), float(ras_top_p))

    def _need(self, t, shape, dtype, what):
        torch = self.torch
        if t is None:
            return
        if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
            raise DualARError(-1, f"{what}: expected contiguous cuda {dtype} {tuple(shape)}, got "
                                  f"{t.dtype} {tuple(t.shape)} on {t.device}")

    def _taps(self, B, with_fused=True, which=True):
        """Tap buffers: which = True for all, or a collection of tap names."""
        torch, m, N = self.torch, self.m, self.N
        td = {"slow_hidden": torch.empty((B, m["dim"]), device="cuda"),
              "slow_logits": torch.empty((B, m["vocab_size"]), device="cuda"),
              "fast_logits": torch.empty((B, N - 1, m["codebook_size"]), device="cuda")}
        if with_fused:
            td["fused_x"] = torch.empty((B, m["dim"]), device="cuda")
        if which is not True:
            td = {k: v for k, v in td.items() if k in which}
        tp = Taps(*[td[k].data_ptr() if k in td else None
                    for k in ("fused_x", "slow_hidden", "slow_logits", "fast_logits")])
        return tp, td

    def prefill(self, tokens, prompt_len, sampling: Sampling, uniforms=None, taps=False):
        """tokens: cuda int32 [B][N+1][T]; prompt_len: host ints [B].  Returns
        frame 0 [B][N+1], or (frame 0, taps) when taps is set (True, or the
        names of the taps wanted)."""
        torch = self.torch
        B, _, T = tokens.shape
        self._need(tokens, (B, self.N + 1, T), torch.int32, "tokens")
        self._need(uniforms, (B, self.N + (sampling.ras_window > 0)), torch.float32, "uniforms")
        if len(prompt_len) != B:
            raise DualARError(-1, "prompt_len must have one entry per sequence")
        plen = (C.c_int32 * B)(*[int(x) for x in prompt_len])
        frame0 = torch.empty((B, self.N + 1), dtype=torch.int32, device="cuda")
        tp, td = self._taps(B, with_fused=False, which=taps) if taps else (None, None)
        self._check(self.lib.dualar_prefill(self.h, B, _ptr(tokens), T, plen, C.byref(sampling),
                                            _ptr(uniforms), _ptr(frame0), C.byref(tp) if tp is not None else None))
        self.batch = B
        return (frame0, td) if taps else frame0

    def decode_frames(self, n: int, sampling: Sampling, uniforms=None, taps: bool = False, out=None):
        torch = self.torch
        B, N, m = self.batch, self.N, self.m
        codes = out if out is not None else torch.empty((B, n, N + 1), dtype=torch.int32, device="cuda")
        self._need(uniforms, (n, B, N + (sampling.ras_window > 0)), torch.float32, "uniforms")
        self._need(codes, (B, n, N + 1), torch.int32, "codes")
        emitted = torch.empty(B, dtype=torch.int32, device="cuda")
        tp, td = self._taps(B, which=taps) if taps else (None, None)
        self._check(self.lib.dualar_decode_frames(self.h, n, C.byref(sampling), _ptr(uniforms), _ptr(codes),
                                                  _ptr(emitted), C.byref(tp) if tp is not None else None))
        return codes, emitted, td

    def fast_teacher_forced(self, hidden, codes, out=None):
        """hidden: cuda fp32 [n][fast_dim]; codes: cuda int32 [n][N].  Returns
        the fast head's logits [n][N][C] (slot k >= 1 predicts q^(k))."""
        torch, m, N = self.torch, self.m, self.N
        n = hidden.shape[0]
        self._need(hidden, (n, m["dim"]), torch.float32, "hidden")
        self._need(codes, (n, N), torch.int32, "codes")
        logits = out if out is not None else torch.empty((n, N, m["codebook_size"]), device="cuda")
        self._need(logits, (n, N, m["codebook_size"]), torch.float32, "logits")
        self._check(self.lib.dualar_fast_teacher_forced(self.h, n, _ptr(hidden), _ptr(codes), _ptr(logits)))
        return logits

    def fast_frames(self, hidden, q0, sampling: Sampling, uniforms=None, taps: bool = False, out=None):
        """hidden: cuda fp32 [F][B][dim]; q0: cuda int32 [F][B] -> codes [B][F][N]."""
        torch = self.torch
        F, B = q0.shape
        codes = out if out is not None else torch.empty((B, F, self.N), dtype=torch.int32, device="cuda")
        self._need(hidden, (F, B, self.m["fast_dim"]), torch.float32, "hidden")
        self._need(q0, (F, B), torch.int32, "q0")
        self._need(uniforms, (F, B, self.N), torch.float32, "uniforms")
        self._need(codes, (B, F, self.N), torch.int32, "codes")
        tp, td = None, None
        if taps:
            td = {"fast_logits": torch.empty((B, self.N - 1, self.m["codebook_size"]), device="cuda")}
            tp = Taps(None, None, None, td["fast_logits"].data_ptr())
        self._check(self.lib.dualar_fast_frames(self.h, B, F, _ptr(hidden), _ptr(q0), C.byref(sampling),
                                                _ptr(uniforms), _ptr(codes), C.byref(tp) if tp is not None else None))
        return codes, td

    def profile_begin(self, kernel_class: int):
        self._check(self.lib.dualar_profile_begin(self.h, kernel_class))

    def profile_end(self):
        n, ms, by = C.c_int64(), C.c_double(), C.c_double()
        self._check(self.lib.dualar_profile_end(self.h, C.byref(n), C.byref(ms), C.byref(by)))
        return {"launches": n.value, "total_ms": ms.value, "bytes": by.value}

    def reset(self, seq_ids):
        """Retire sequences of the current batch (host ints): later frames
        emit -1 rows for them; the other sequences are unaffected."""
        ids = [int(i) for i in seq_ids]
        arr = (C.c_int32 * max(len(ids), 1))(*ids)
        self._check(self.lib.dualar_reset(self.h, arr if ids else None, len(ids)))

    def sync(self) -> int:
        st = C.c_int32(0)
        self._check(self.lib.dualar_sync(self.h, C.byref(st)))
        return st.value

    def close(self):
        if getattr(self, "h", None):
            self.lib.dualar_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
