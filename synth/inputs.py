"""Seeded synthetic inputs: hyper-parameters, weights, prompts, uniforms.

Sources for the shapes (Fish Audio S2 pages):
  * "Fish Audio S2: a Qwen3-4B on the time axis ..." (ai.thesatyajit.com),
    summary table and section "The slow AR is Qwen3-4B. The fast AR is not
    small": slow AR 36 layers, width 2560, 32 query / 8 KV heads, head_dim 128,
    FFN 9728, vocabulary 155,776, tied head; fast AR 4 layers of the same
    width with its own 4,096-row embedding and head; a 40,960 x 2560
    codebook-fusion table.
  * Same page, "The slow AR is Qwen3-4B": semantic ids 151,678 .. 155,773;
    Qwen's 151,643 BPE ids below a block of added tokens.
  * Same page, "The codec": one 4,096-entry semantic codebook and nine
    1,024-entry acoustic codebooks (acoustic prompt ids are drawn from 0..1023).
  * Same page, "Tags are text": the voice-clone prompt layout (text, then the
    reference frames, then text), used here as the three-segment prompt.

Randomness: numpy PCG64 seeded by SeedSequence([base, stream, ...]).  Weight
tensors are generated in chunks of 2**22 values, chunk j of tensor `name`
from SeedSequence([base, crc32(name), j]), so generation can run on a thread
pool and still be bit-reproducible.  Matrices are N(0, 0.02); norm gains are
1 + N(0, 0.02).  For bf16 workloads the fp32 draw is rounded to bf16 with
round-to-nearest-even and handed out as uint16 bit patterns.
"""
from __future__ import annotations

import os
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# ----------------------------------------------------------------------------
# Model hyper-parameters (data, not code: both sides read these dicts)
# ----------------------------------------------------------------------------

_S2 = dict(
    n_layer=36, dim=2560, n_head=32, n_kv_head=8, head_dim=128, ffn_dim=9728,
    vocab_size=155776,
    n_fast_layer=4, fast_dim=2560, fast_n_head=32, fast_n_kv_head=8,
    fast_head_dim=128, fast_ffn_dim=9728,
    slow_qk_norm=1, fast_qk_norm=1,
    num_codebooks=10, codebook_size=4096,
    semantic_begin_id=151678, semantic_end_id=155773,
    # <|im_end|>: not printed on the pages; Qwen's id inside the added-token
    # block 151,643..151,677.
    end_id=151645,
    scale_codebook_embeddings=1,
    rope_base=1.0e6, norm_eps=1.0e-6,
    weight_dtype="bf16",
    text_vocab=151643,       # ordinary BPE ids are drawn from [0, text_vocab)
    acoustic_size=1024,      # acoustic prompt codes are drawn from [0, 1024)
)

_TINY = dict(
    n_layer=2, dim=256, n_head=4, n_kv_head=2, head_dim=64, ffn_dim=768,
    vocab_size=5120,
    n_fast_layer=2, fast_dim=256, fast_n_head=4, fast_n_kv_head=2,
    fast_head_dim=64, fast_ffn_dim=768,
    slow_qk_norm=1, fast_qk_norm=1,
    num_codebooks=4, codebook_size=256,
    semantic_begin_id=1024, semantic_end_id=1279, end_id=1000,
    scale_codebook_embeddings=1,
    rope_base=1.0e6, norm_eps=1.0e-6,
    weight_dtype="f32",
    text_vocab=1000,
    acoustic_size=256,
)

MODELS = {"tiny": _TINY, "s2": _S2}


def model(name: str, **overrides) -> dict:
    m = dict(MODELS[name])
    m.update(overrides)
    return m


# The five measured / parity workloads.  "prompt" describes the prompt layout:
#   ("segments", P)       text P/8, frames P/2, text for the rest
#   ("ragged", lo, hi)    per-sequence P_b ~ U{lo..hi}, same segment layout
#   ("frames", P)         every position is a frame
WORKLOADS = {
    "tiny_b1": dict(model="tiny", batch=1, prompt=("fixed", 4, 16, 12), frames=16,
                    sampling=dict(greedy=1, temperature=1.0, top_p=1.0)),
    "fast_s2": dict(model="s2", batch=1, fast_only=True, frames=512,
                    sampling=dict(greedy=1, temperature=1.0, top_p=1.0)),
    "s2_b1": dict(model="s2", batch=1, prompt=("fixed", 128, 512, 384), frames=256,
                  sampling=dict(greedy=1, temperature=1.0, top_p=1.0)),
    "s2_b32": dict(model="s2", batch=32, prompt=("ragged", 512, 4096), frames=128,
                   sampling=dict(greedy=0, temperature=1.0, top_p=0.9)),
    "s2_prefill": dict(model="s2", batch=4, prompt=("frames", 16384), frames=64,
                       sampling=dict(greedy=1, temperature=1.0, top_p=1.0)),
}

# ----------------------------------------------------------------------------
# bf16 bit helpers (pure data conversion)
# ----------------------------------------------------------------------------


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 -> bf16 with round-to-nearest-even; returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# Weights
# ----------------------------------------------------------------------------


def tensor_specs(m: dict):
    """(name, shape, kind) for every parameter; kind is 'mat' or 'gain'.

    Matrices use the [out, in] row-major layout of nn.Linear."""
    specs = []
    D, V = m["dim"], m["vocab_size"]
    N, C = m["num_codebooks"], m["codebook_size"]
    specs.append(("tok_embedding", (V, D), "mat"))
    specs.append(("codebook_embedding", (N * C, D), "mat"))

    def layer(prefix, dim, nh, nkv, hd, ffn, qk):
        out = [
            (f"{prefix}.attention_norm", (dim,), "gain"),
            (f"{prefix}.wq", (nh * hd, dim), "mat"),
            (f"{prefix}.wk", (nkv * hd, dim), "mat"),
            (f"{prefix}.wv", (nkv * hd, dim), "mat"),
        ]
        if qk:
            out += [(f"{prefix}.q_norm", (hd,), "gain"), (f"{prefix}.k_norm", (hd,), "gain")]
        out += [
            (f"{prefix}.wo", (dim, nh * hd), "mat"),
            (f"{prefix}.ffn_norm", (dim,), "gain"),
            (f"{prefix}.w1", (ffn, dim), "mat"),
            (f"{prefix}.w3", (ffn, dim), "mat"),
            (f"{prefix}.w2", (dim, ffn), "mat"),
        ]
        return out

    for i in range(m["n_layer"]):
        specs += layer(f"layers.{i}", D, m["n_head"], m["n_kv_head"], m["head_dim"],
                       m["ffn_dim"], m["slow_qk_norm"])
    specs.append(("norm", (D,), "gain"))
    FD = m["fast_dim"]
    for i in range(m["n_fast_layer"]):
        specs += layer(f"fast_layers.{i}", FD, m["fast_n_head"], m["fast_n_kv_head"],
                       m["fast_head_dim"], m["fast_ffn_dim"], m["fast_qk_norm"])
    specs.append(("fast_embeddings", (C, FD), "mat"))
    specs.append(("fast_norm", (FD,), "gain"))
    specs.append(("fast_output", (C, FD), "mat"))
    return specs


_CHUNK = 1 << 22


def _threads(n):
    if n:
        return n
    return max(1, min(16, os.cpu_count() or 1))


def make_weights(m: dict, seed: int = 0, threads: int | None = None, only=None) -> dict:
    """Random-init weights.  bf16 models -> uint16 bit arrays, f32 -> float32.

    `only` optionally restricts generation to a set of tensor names (the
    values of each tensor do not depend on which others are generated)."""
    bf16 = m["weight_dtype"] == "bf16"
    specs = [s for s in tensor_specs(m) if only is None or s[0] in only]
    out = {}
    jobs = []
    for name, shape, kind in specs:
        n = int(np.prod(shape))
        arr = np.empty(n, dtype=np.uint16 if bf16 else np.float32)
        out[name] = (arr, shape)
        key = zlib.crc32(name.encode())
        for j, s in enumerate(range(0, n, _CHUNK)):
            jobs.append((arr, key, j, s, min(n, s + _CHUNK), kind))

    def run(job):
        arr, key, j, s, e, kind = job
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, key, j])))
        v = g.standard_normal(e - s, dtype=np.float32)
        v *= np.float32(0.02)
        if kind == "gain":
            v += np.float32(1.0)
        arr[s:e] = f32_to_bf16_bits(v) if bf16 else v

    with ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(run, jobs))
    return {k: a.reshape(shape) for k, (a, shape) in out.items()}


def weights_as_f32(m: dict, w: dict) -> dict:
    """float32 view of the weights (bf16 values are exact in fp32).  Packed
    4-bit matrices (".q4") are passed through as they are."""
    if m["weight_dtype"] == "bf16":
        return {k: (v if k.endswith(".q4") else bf16_bits_to_f32(v).reshape(v.shape)) for k, v in w.items()}
    return dict(w)


# ----------------------------------------------------------------------------
# W4A16 synthetic models (4-bit weights in groups, bf16 scales)
# ----------------------------------------------------------------------------
# The pages name a W4A16 variant of S2 that keeps the attention of its last 12
# layers in bf16, and give no recipe.  The synthetic W4A16 model here uses
# symmetric 4-bit groups of W4_GROUP consecutive input elements with a bf16
# scale per (row, group): scale = bf16(max |w| / 7), q = clamp(rne(w / scale),
# -8, 7), stored two per byte (element 2j in the low nibble of byte j, 2j+1
# in the high nibble, two's complement).  The model's weight is q * scale.

W4_GROUP = 128
W4_MATS = ("wq", "wk", "wv", "wo", "w1", "w3", "w2")


def w4_names(m: dict) -> list:
    """Matrices stored as 4-bit groups when m["w4a16"] is set: every linear
    matrix of the slow and fast layers except the attention projections of
    the last m["w4_bf16_attn_layers"] (default 12) slow layers."""
    if not m.get("w4a16"):
        return []
    keep = m.get("w4_bf16_attn_layers", 12)
    out = []
    for i in range(m["n_layer"]):
        late = i >= m["n_layer"] - keep
        out += [f"layers.{i}.{k}" for k in W4_MATS if not (late and k in ("wq", "wk", "wv", "wo"))]
    for i in range(m["n_fast_layer"]):
        out += [f"fast_layers.{i}.{k}" for k in W4_MATS]
    return out


def quantize_w4(bits: np.ndarray):
    """bf16 bits [rows, K] -> (packed uint8 [rows, K/2], scales bf16 bits [rows, K/W4_GROUP])."""
    w = bf16_bits_to_f32(bits).reshape(bits.shape).astype(np.float64)
    rows, K = w.shape
    if K % W4_GROUP:
        raise ValueError(f"row length {K} is not a multiple of {W4_GROUP}")
    g = w.reshape(rows, K // W4_GROUP, W4_GROUP)
    amax = np.abs(g).max(axis=2)
    sbits = f32_to_bf16_bits((amax / 7.0).astype(np.float32))
    s = bf16_bits_to_f32(sbits).reshape(amax.shape).astype(np.float64)
    s_safe = np.where(s > 0, s, 1.0)
    q = np.clip(np.round(g / s_safe[:, :, None]), -8, 7).astype(np.int64).reshape(rows, K)   # round half to even
    u = (q & 0xF).astype(np.uint8)
    packed = (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)
    return packed, sbits.reshape(rows, K // W4_GROUP)


def make_w4_model(m: dict, w: dict) -> dict:
    """The W4A16 form of a bf16 weight set: each matrix of w4_names(m) is
    replaced by name.q4 (packed) and name.s4 (scales); the rest is kept."""
    if m["weight_dtype"] != "bf16":
        raise ValueError("W4A16 models start from bf16 weights")
    out = dict(w)
    for name in w4_names(m):
        q, s = quantize_w4(out.pop(name))
        out[name + ".q4"], out[name + ".s4"] = q, s
    return out


# ----------------------------------------------------------------------------
# Prompts, uniforms, context lengths, fast-AR-only inputs
# ----------------------------------------------------------------------------


def _gen(seed, *stream):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *stream])))


def make_ctx_lengths(batch: int, lo: int, hi: int, seed: int = 0) -> np.ndarray:
    """Per-sequence prompt lengths ~ U{lo..hi} (stream 3)."""
    return _gen(seed, 3).integers(lo, hi + 1, size=batch).astype(np.int32)


def _segments(P, layout):
    if layout[0] == "fixed":
        a, b, c = layout[1:]
        assert a + b + c == P
        return a, b, c
    if layout[0] == "frames":
        return 0, P, 0
    a = P // 8
    b = P // 2
    return a, b, P - a - b


def prompt_lengths(w: dict, seed: int = 0) -> np.ndarray:
    p = w["prompt"]
    if p[0] == "fixed":
        return np.full(w["batch"], sum(p[1:]), dtype=np.int32)
    if p[0] == "frames":
        return np.full(w["batch"], p[1], dtype=np.int32)
    return make_ctx_lengths(w["batch"], p[1], p[2], seed)


def make_prompts(m: dict, layout, lengths, seed: int = 0) -> np.ndarray:
    """Prompt token columns, int32 [B][N+1][T_max] (stream 1).

    Row 0 holds the LM ids; rows 1..N hold codebook ids q^(0..N-1).  Text
    positions have LM id ~ U[0, text_vocab) and zero codes.  Frame positions
    have q^(0) ~ U{0..C-1}, LM id = semantic_begin_id + q^(0), and acoustic
    codes q^(1..N-1) ~ U{0..acoustic_size-1}.  Positions past a sequence's
    length are zero."""
    N, C = m["num_codebooks"], m["codebook_size"]
    lengths = np.asarray(lengths, dtype=np.int64)
    B, T = len(lengths), int(lengths.max())
    out = np.zeros((B, N + 1, T), dtype=np.int32)
    for b in range(B):
        g = _gen(seed, 1, b)
        P = int(lengths[b])
        a, f, c = _segments(P, layout)
        kinds = np.concatenate([np.zeros(a), np.ones(f), np.zeros(c)]).astype(bool)
        text = g.integers(0, m["text_vocab"], size=P)
        q0 = g.integers(0, C, size=P)
        qa = g.integers(0, m["acoustic_size"], size=(N - 1, P))
        out[b, 0, :P] = np.where(kinds, m["semantic_begin_id"] + q0, text)
        out[b, 1, :P] = np.where(kinds, q0, 0)
        out[b, 2:, :P] = np.where(kinds[None, :], qa, 0)
    return out


def make_uniforms(shape, seed: int = 0) -> np.ndarray:
    """fp32 uniforms in [0, 1) for top-p draws (stream 2)."""
    return _gen(seed, 2).random(size=shape, dtype=np.float32)


def make_fast_inputs(m: dict, n_frames: int, batch: int, seed: int = 0):
    """Fast-AR-only workload (stream 4): slow hidden states h ~ N(0,1) fp32
    [n_frames][B][fast_dim] and first codes q^(0) ~ U{0..C-1} [n_frames][B]."""
    g = _gen(seed, 4)
    h = g.standard_normal((n_frames, batch, m["fast_dim"]), dtype=np.float32)
    q0 = g.integers(0, m["codebook_size"], size=(n_frames, batch)).astype(np.int32)
    return h, q0
