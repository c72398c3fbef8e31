"""Rates and byte counts used to report throughput (no model arithmetic).

Codec rates ([P2] "The codec: 44.1 kHz in, 21.53 frames out"): 44,100 Hz
audio, hop 2,048 -> 21.53 frames of audio per second, N codec tokens per
frame.  RTF = seconds of compute per second of audio = frame_rate / fps.
[P2] = "Fish Audio S2: a Qwen3-4B on the time axis, four layers on the
codebook axis, and tags that are only text".

Bytes per decode step ([P2] "The slow AR is Qwen3-4B. The fast AR is not
small": batch-1 decode is bound by reading weights; one slow step reads the
36 layers plus the whole tied 155,776-row head, one fast pass the four fast
layers plus the 4,096-row head).
"""
from __future__ import annotations

SAMPLE_RATE = 44100
HOP = 2048
FRAME_RATE = SAMPLE_RATE / HOP


def codec_tokens_per_s(fps: float, num_codebooks: int = 10) -> float:
    return fps * num_codebooks


def rtf(fps_per_sequence: float) -> float:
    return FRAME_RATE / fps_per_sequence


def _layer_elems(dim, nh, nkv, hd, ffn, qk):
    return dim * (nh * hd + 2 * nkv * hd) + nh * hd * dim + 3 * dim * ffn + 2 * dim + (2 * hd if qk else 0)


def slow_step_weight_elems(m: dict) -> int:
    """Slow layers + tied head + final norm."""
    per = _layer_elems(m["dim"], m["n_head"], m["n_kv_head"], m["head_dim"], m["ffn_dim"], m["slow_qk_norm"])
    return m["n_layer"] * per + m["vocab_size"] * m["dim"] + m["dim"]


def fast_pass_weight_elems(m: dict) -> int:
    """Fast layers + fast head + fast norm (one pass)."""
    per = _layer_elems(m["fast_dim"], m["fast_n_head"], m["fast_n_kv_head"], m["fast_head_dim"],
                       m["fast_ffn_dim"], m["fast_qk_norm"])
    return m["n_fast_layer"] * per + m["codebook_size"] * m["fast_dim"] + m["fast_dim"]


def fast_pass0_weight_elems(m: dict) -> int:
    """What fast pass 0 reads here: its logits are never used, so it runs the
    first n_fast_layer - 1 layers and, of the last one, only the attention
    norm, the K/V projections and the k QK-norm gain (the cache entries of
    slot 0); no Q, O, FFN or fast head."""
    per = _layer_elems(m["fast_dim"], m["fast_n_head"], m["fast_n_kv_head"], m["fast_head_dim"],
                       m["fast_ffn_dim"], m["fast_qk_norm"])
    last = m["fast_dim"] + 2 * m["fast_n_kv_head"] * m["fast_head_dim"] * m["fast_dim"] + \
        (m["fast_head_dim"] if m["fast_qk_norm"] else 0)
    return (m["n_fast_layer"] - 1) * per + last


def _mat_shape(m: dict, name: str):
    """(rows, inputs) of a layer matrix `layers.i.wq`-style name."""
    fast = name.startswith("fast_layers.")
    pre = "fast_" if fast else ""
    dim = m["fast_dim"] if fast else m["dim"]
    H, KV, hd = m[pre + "n_head"], m[pre + "n_kv_head"], m[pre + "head_dim"]
    ffn = m["fast_ffn_dim"] if fast else m["ffn_dim"]
    return {"wq": (H * hd, dim), "wk": (KV * hd, dim), "wv": (KV * hd, dim), "wo": (dim, H * hd),
            "w1": (ffn, dim), "w3": (ffn, dim), "w2": (dim, ffn)}[name.rsplit(".", 1)[1]]


def w4_read_delta(m: dict, w4_names, fast_only: bool = False) -> int:
    """Change of a frame-step's weight bytes when the named matrices are 4-bit
    groups of 128 with bf16 scales (rows * (K/2 + K/64) bytes per read instead
    of rows * K * 2): slow matrices are read once per frame, fast ones by
    passes 1..N-1, and by pass 0 for all layers but the last, of which pass 0
    reads the K and V rows only."""
    N, nf = m["num_codebooks"], m["n_fast_layer"]
    d = 0
    for name in w4_names:
        rows, K = _mat_shape(m, name)
        per = rows * (K // 2 + K // 64) - rows * K * 2
        if name.startswith("fast_layers."):
            layer, mat = int(name.split(".")[1]), name.rsplit(".", 1)[1]
            reads = N - 1 + (1 if layer < nf - 1 or mat in ("wk", "wv") else 0)
            d += reads * per
        elif not fast_only:
            d += per
    return d


def frame_bytes(m: dict, ctx_lengths, fast_only: bool = False, semantic_head: bool = False,
                w4_names=()) -> dict:
    """Algorithmic HBM bytes of one decode frame-step over a batch whose
    sequences attend over `ctx_lengths` slow positions (new one included).

    Weights are read once per step whatever the batch; K/V and gathers scale
    with the batch.  Fast weights: passes 1..N-1 read the whole fast stack
    and head, pass 0 what `fast_pass0_weight_elems` counts.  With
    semantic_head the slow head reads only the C semantic rows and the end
    row."""
    esz = 2 if m["weight_dtype"] == "bf16" else 4
    kvesz = 2 if m.get("kv_dtype", m["weight_dtype"]) == "bf16" else 4
    N, D = m["num_codebooks"], m["dim"]
    B = len(ctx_lengths)
    fast_w = ((N - 1) * fast_pass_weight_elems(m) + fast_pass0_weight_elems(m)) * esz
    # fast K/V: pass k reads slots 0..k-1 and writes slot k, every layer
    fkv = m["n_fast_layer"] * 2 * m["fast_n_kv_head"] * m["fast_head_dim"] * kvesz
    fast_kv = B * fkv * sum(k + 1 for k in range(N))
    fast_gather = B * (N - 1) * D * esz        # E_fast rows for passes 1..N-1
    out = {"fast_weights": fast_w, "fast_kv": fast_kv, "gathers": fast_gather}
    if not fast_only:
        skv = m["n_layer"] * 2 * m["n_kv_head"] * m["head_dim"] * kvesz
        sw = slow_step_weight_elems(m)
        if semantic_head:
            sw -= (m["vocab_size"] - m["codebook_size"] - 1) * m["dim"]
        out["slow_weights"] = sw * esz
        # a sequence attending over L positions reads L-1 cached entries and appends one
        out["slow_kv"] = sum(int(L) for L in ctx_lengths) * skv
        out["gathers"] += B * (N + 1) * D * esz   # fusion rows
    if w4_names:
        out["w4_delta"] = w4_read_delta(m, w4_names, fast_only)
    out["total"] = sum(out.values())
    return out


def prefill_flops(m: dict, prompt_lengths) -> dict:
    """Arithmetic of a prefill (counted as multiply-add = 2 flops, bf16 MFMA
    work as the pages' model would do it): the slow layers' products over
    every prompt position, and causal attention, where position t of a
    sequence attends to positions 0..t (q.k and p.v: 4*hd flops per pair and
    query head).  The head, the sampler and the fast AR run once, for frame
    0, and are not counted."""
    per_layer = m["dim"] * (m["n_head"] * m["head_dim"] + 2 * m["n_kv_head"] * m["head_dim"]) + \
        m["n_head"] * m["head_dim"] * m["dim"] + 3 * m["dim"] * m["ffn_dim"]
    tokens = int(sum(int(t) for t in prompt_lengths))
    linear = 2 * tokens * m["n_layer"] * per_layer
    pairs = sum(int(t) * (int(t) + 1) // 2 for t in prompt_lengths)
    attention = 4 * m["head_dim"] * m["n_head"] * m["n_layer"] * pairs
    return {"linear": linear, "attention": attention, "total": linear + attention, "tokens": tokens}


def fast_tf_flops(m: dict, n: int) -> dict:
    """Arithmetic of one teacher-forced fast-AR call over n (hidden state,
    codes) pairs: the fast layers and the fast head over n*N rows (2 flops
    per weight per row: the 414.2 M weights of one fast pass on the S2
    shapes), and causal attention along depth, where depth position k attends
    to positions 0..k (4*hd flops per attended position and query head)."""
    N, d = m["num_codebooks"], m["fast_dim"]
    H, KV, hd, f = m["fast_n_head"], m["fast_n_kv_head"], m["fast_head_dim"], m["fast_ffn_dim"]
    per_layer = d * (H + 2 * KV) * hd + H * hd * d + 3 * d * f
    rows = n * N
    linear = 2 * rows * (m["n_fast_layer"] * per_layer + m["codebook_size"] * d)
    attention = 4 * hd * H * m["n_fast_layer"] * n * (N * (N + 1) // 2)
    return {"linear": linear, "attention": attention, "total": linear + attention, "rows": rows}
