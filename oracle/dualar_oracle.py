"""Plain CPU oracle of the Dual-AR decode step (float64, numpy).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the HIP library.

Pages cited (titles as published):
  [P1] "How the Dual-Autoregressive Architecture Works in Fish Speech S2:
       A Deep Dive" (instagit.com explainer of fish-speech).
  [P2] "Fish Audio S2: a Qwen3-4B on the time axis, four layers on the
       codebook axis, and tags that are only text" (ai.thesatyajit.com).

What is computed, in the pages' order:
  * Slow AR: a Qwen3-4B layer stack (RMSNorm, GQA with per-head QK-norm,
    RoPE, SwiGLU) with a tied head over the whole vocabulary
    ([P2] "The slow AR is Qwen3-4B. The fast AR is not small").
  * Semantic logit bias: -inf everywhere except the semantic ids and
    <|im_end|>, then a sample ([P2] "Two autoregressions ...", the
    `decode_one_token_ar` excerpt).
  * Fast AR: pass 0 writes the slow hidden state into the depth cache at
    position 0; passes 1..N-1 embed the previous code and sample the next,
    unmasked; the depth cache has N slots and is rewritten every frame
    ([P2] same section; [P1] "Fast Transformer: The Codebook Decoder").
  * Multi-codebook fusion, Eq. 1 of the S2 report with the sqrt(N+1) divide
    applied by `forward_generate` when `scale_codebook_embeddings` is on
    ([P2] "Two autoregressions ...", Eq. 1 and the paragraph after it).
  * Optional repetition-aware loop breaker (RAS) of the slow sample: a second
    draw at temperature 1.0 and top-p 0.9 replaces the normal one when the
    normal one repeats a semantic token of the last 10 frames ([P2] "Two
    autoregressions ...", the loop-breaker paragraph after Eq. 1).

Precision: every activation, norm, softmax and accumulation is float64.  The
rounding points that belong to the method are kept: the weights are the
given (bf16-exact) values, the RoPE table is rounded to bf16 ([P2]
"Streaming: whose numbers", last paragraph: the bf16 table is the correct
one), and for bf16 models the K/V cache entries are rounded to bf16.  Logits
are rounded to fp32 before a sampling decision, so the integer decision is
taken in the kernel's precision.

Readings where the pages are silent (each repeated in the design notes):
  hidden state handed to the fast AR is taken before the final norm; RMSNorm
  eps from the config; QK-norm (one gain of head_dim values shared by all
  heads) before RoPE; RoPE rotates interleaved pairs (2i, 2i+1) with
  theta_i = base^(-2i/hd) and angles in float64; GQA groups are contiguous;
  scores are scaled by 1/sqrt(head_dim); greedy ties go to the lowest id;
  top-p keeps the shortest (prob desc, id asc) prefix whose cumulative sum
  reaches top_p and picks the first kept token whose renormalised
  cumulative sum exceeds the supplied uniform u.  RAS: the window holds the
  slow ids the sequence emitted in its previous ras_window frames (frame 0
  of the prefill included, the prompt's own columns not); the second draw
  uses the same biased logits with its own uniform (slot N of the frame's
  draws), also after a greedy normal draw; <|im_end|> is never replaced;
  the id finally emitted enters the window; fast draws are unaffected.

Parity unpinned (no real S2 weights exist here): agreement with the released
checkpoint's outputs, and the readings above measured against it.
"""
from __future__ import annotations

import math
import os
from dataclasses import dataclass, field

import numpy as np

F64 = np.float64

# ----------------------------------------------------------------------------
# Parameters
# ----------------------------------------------------------------------------


def param_shapes(cfg: dict) -> dict:
    """Every parameter of the model as the pages describe it: no biases, a tied
    head, one [head_dim] QK-norm gain pair per layer where QK-norm is on, no
    fast `project_in` (fast width equals slow width), its own fast embedding
    and head, and a stacked N*C-row codebook-fusion table ([P2] summary table;
    [P1] "Fast Transformer: The Codebook Decoder")."""
    D, V = cfg["dim"], cfg["vocab_size"]
    N, C = cfg["num_codebooks"], cfg["codebook_size"]
    shapes = {"tok_embedding": (V, D), "codebook_embedding": (N * C, D), "norm": (D,)}

    def block(prefix, dim, nh, nkv, hd, ffn, qk):
        shapes[f"{prefix}.attention_norm"] = (dim,)
        shapes[f"{prefix}.wq"] = (nh * hd, dim)
        shapes[f"{prefix}.wk"] = (nkv * hd, dim)
        shapes[f"{prefix}.wv"] = (nkv * hd, dim)
        if qk:
            shapes[f"{prefix}.q_norm"] = (hd,)
            shapes[f"{prefix}.k_norm"] = (hd,)
        shapes[f"{prefix}.wo"] = (dim, nh * hd)
        shapes[f"{prefix}.ffn_norm"] = (dim,)
        shapes[f"{prefix}.w1"] = (ffn, dim)
        shapes[f"{prefix}.w3"] = (ffn, dim)
        shapes[f"{prefix}.w2"] = (dim, ffn)

    for i in range(cfg["n_layer"]):
        block(f"layers.{i}", D, cfg["n_head"], cfg["n_kv_head"], cfg["head_dim"],
              cfg["ffn_dim"], cfg["slow_qk_norm"])
    for i in range(cfg["n_fast_layer"]):
        block(f"fast_layers.{i}", cfg["fast_dim"], cfg["fast_n_head"], cfg["fast_n_kv_head"],
              cfg["fast_head_dim"], cfg["fast_ffn_dim"], cfg["fast_qk_norm"])
    shapes["fast_embeddings"] = (C, cfg["fast_dim"])
    shapes["fast_norm"] = (cfg["fast_dim"],)
    shapes["fast_output"] = (C, cfg["fast_dim"])
    return shapes


def count_params(cfg: dict, part: str = "all") -> int:
    """Parameter count of 'slow' (text_model: layers, tied embedding, final
    norm), 'fast', 'fusion' or 'all'."""
    total = 0
    for name, shp in param_shapes(cfg).items():
        if name.startswith("fast_"):
            grp = "fast"
        elif name == "codebook_embedding":
            grp = "fusion"
        else:
            grp = "slow"
        if part in ("all", grp):
            total += int(np.prod(shp))
    return total


# ----------------------------------------------------------------------------
# Elementary pieces
# ----------------------------------------------------------------------------


def bf16_round(x) -> np.ndarray:
    """Round to the nearest bf16 value (8 significant bits), ties to even."""
    x = np.asarray(x, dtype=F64)
    m, e = np.frexp(x)                 # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.round(m * 256.0), e - 8)   # np.round: half to even


def dequant_w4(weights: dict, group: int = 128) -> dict:
    """The weights of a W4A16 model as the method uses them: every
    `name.q4` (packed 4-bit values, [rows, K/2] bytes) with its `name.s4`
    (one scale per row and group of `group` consecutive inputs) becomes the
    matrix `name` = q * scale in float64.

    [P3] (the W4A16 "late12attn" S2 model card) names the variant but prints
    no format; the format read here (the same one the synthetic W4A16 model
    is written in) is: byte j of a row holds input 2j in its low nibble and
    2j+1 in its high nibble, each a two's-complement integer in [-8, 7].
    Parity unpinned against any real quantised checkpoint."""
    out = {}
    for k, v in weights.items():
        if k.endswith(".s4"):
            continue
        if not k.endswith(".q4"):
            out[k] = v
            continue
        name = k[:-3]
        b = np.asarray(v, dtype=np.uint8)
        nib = np.empty((b.shape[0], 2 * b.shape[1]), dtype=np.int64)
        nib[:, 0::2] = b & 0xF
        nib[:, 1::2] = b >> 4
        q = np.where(nib >= 8, nib - 16, nib).astype(F64)
        sc = np.asarray(weights[name + ".s4"])
        if not np.issubdtype(sc.dtype, np.floating):
            raise ValueError(f"{name}: scales must be given as values, not bit patterns")
        sc = sc.astype(F64)
        if sc.shape[1] * group != q.shape[1]:
            raise ValueError(f"{name}: scales {sc.shape} do not cover {q.shape[1]} inputs in groups of {group}")
        out[name] = q * np.repeat(sc, group, axis=1)
    return out


_POOL = None


def _pool():
    """Threads for independent attention heads (plumbing, no arithmetic)."""
    global _POOL
    if _POOL is None:
        from concurrent.futures import ThreadPoolExecutor
        _POOL = ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1)))
    return _POOL


def rms_norm(x, g, eps):
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def silu(x):
    return x / (1.0 + np.exp(-x))


def rope_table(n_pos: int, head_dim: int, base: float):
    """cos/sin table, [n_pos, head_dim/2], angles p * base^(-2i/hd) in float64,
    values rounded to bf16 ([P2] "Streaming: whose numbers", last paragraph)."""
    i = np.arange(head_dim // 2, dtype=F64)
    theta = 1.0 / (float(base) ** (2.0 * i / head_dim))
    ang = np.arange(n_pos, dtype=F64)[:, None] * theta[None, :]
    return bf16_round(np.cos(ang)), bf16_round(np.sin(ang))


def apply_rope(x, cos, sin):
    """Rotate interleaved pairs (x[2i], x[2i+1]) by the angle whose cos/sin are
    given; x [..., hd], cos/sin broadcastable to [..., hd/2]."""
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * cos - b * sin
    out[..., 1::2] = a * sin + b * cos
    return out


def embed_column(col, tok_emb, cb_emb, sb: int, se: int, N: int, C: int, scale: bool) -> np.ndarray:
    """Slow-AR input for one token column (id, q^(0..N-1)).

    Semantic position (sb <= id <= se): (E_tok[id] + sum_k E_F[k*C + q^(k)])
    / sqrt(N+1), the sum taken in the order E_tok first, then k = 0..N-1
    ([P2] "Two autoregressions ...", Eq. 1 and the sqrt(N+1) paragraph).
    Text position: E_tok[id] alone.  Every operation is done in the tables'
    own precision: float64 tables give the oracle's value; float32 tables
    give the float32 evaluation of the same formula (IEEE adds in that order
    and an IEEE divide by the float32 value of sqrt(N+1)), which a float32
    kernel that follows the formula reproduces bit for bit."""
    ident = int(col[0])
    x = np.array(tok_emb[ident], copy=True)
    if sb <= ident <= se:
        for k in range(N):
            x = x + cb_emb[k * C + int(col[1 + k])]
        if scale:
            x = x / x.dtype.type(math.sqrt(N + 1.0))
    return x


@dataclass
class Sampling:
    greedy: bool = True
    temperature: float = 1.0
    top_p: float = 1.0
    min_frames: int = 0
    ras_window: int = 0            # 0: off; [P2] sets 10
    ras_temperature: float = 1.0   # [P2]: the second draw at temperature 1.0 ...
    ras_top_p: float = 0.9         # ... and top-p 0.9


def sample_token(logits, s: Sampling, u=None) -> int:
    """Greedy or temperature + top-p draw from a logit vector (-inf = masked).

    The logits are first rounded to fp32 (the kernel's precision) so both sides
    take the integer decision from the same values.  Greedy: argmax, lowest id
    on ties.  Top-p: p = softmax(z / T) (float64); order by (p desc, id asc);
    keep the shortest prefix with cumulative sum >= top_p (at least one
    token; only tokens with p > 0); renormalise; return the first kept token
    whose cumulative sum is > u."""
    z = np.asarray(logits, dtype=np.float32).astype(F64)
    if s.greedy or u is None:
        return int(np.argmax(z))
    ok = np.isfinite(z)
    zz = np.where(ok, z / s.temperature, -np.inf)
    p = np.exp(zz - zz[ok].max())
    p /= p.sum()
    ids = np.arange(len(z))
    cand = ids[p > 0]
    order = cand[np.lexsort((cand, -p[cand]))]
    cum = np.cumsum(p[order])
    hit = np.nonzero(cum >= s.top_p)[0]
    n_keep = int(hit[0]) + 1 if len(hit) else len(order)
    kept = order[:n_keep]
    pk = p[kept] / p[kept].sum()
    ck = np.cumsum(pk)
    j = np.nonzero(ck > float(u))[0]
    return int(kept[j[0]] if len(j) else kept[-1])


# ----------------------------------------------------------------------------
# The model
# ----------------------------------------------------------------------------


@dataclass
class _Part:
    """One transformer stack (slow or fast)."""
    n_layer: int
    dim: int
    n_head: int
    n_kv_head: int
    head_dim: int
    qk_norm: bool
    layers: list


@dataclass
class SeqState:
    """Per-sequence decode state: slow K/V cache, next position, next input."""
    k: np.ndarray
    v: np.ndarray
    pos: int = 0
    next_col: np.ndarray | None = None
    frames: int = 0
    done: bool = False
    ras_hist: list = field(default_factory=list)   # slow ids emitted (all frames), oldest first


@dataclass
class Counters:
    slow_passes: int = 0
    fast_passes: int = 0
    fast_samples: int = 0
    slot_writes: list = field(default_factory=list)


class DualAROracle:
    """Dual-AR decoder over given weights (numpy arrays by name).

    `dtype` is the compute precision: float64 by default.  float32 exists only
    to measure how far an fp32 evaluation of the same steps drifts from the
    float64 one (a floor for comparing fp32 kernels).  The K/V caches are
    rounded to bf16 when cfg["kv_dtype"] (default: the weight dtype) is bf16."""

    def __init__(self, cfg: dict, weights: dict, max_seq: int = 4096, dtype=F64):
        self.cfg = cfg
        self.dt = dtype
        shapes = param_shapes(cfg)
        for name, shp in shapes.items():
            if tuple(weights[name].shape) != tuple(shp):
                raise ValueError(f"{name}: shape {weights[name].shape} != {shp}")
        self.w = {k: np.asarray(weights[k], dtype=dtype) for k in shapes}
        self.kv_bf16 = cfg.get("kv_dtype", cfg["weight_dtype"]) == "bf16"
        self.eps = float(cfg["norm_eps"])
        self.N = cfg["num_codebooks"]
        self.C = cfg["codebook_size"]
        self.sb, self.se, self.end = cfg["semantic_begin_id"], cfg["semantic_end_id"], cfg["end_id"]
        self.max_seq = max_seq

        def part(prefix, n, dim, nh, nkv, hd, qk):
            layers = []
            for i in range(n):
                p = f"{prefix}.{i}."
                layers.append({k[len(p):]: v for k, v in self.w.items() if k.startswith(p)})
            return _Part(n, dim, nh, nkv, hd, bool(qk), layers)

        c = cfg
        self.slow = part("layers", c["n_layer"], c["dim"], c["n_head"], c["n_kv_head"],
                         c["head_dim"], c["slow_qk_norm"])
        self.fast = part("fast_layers", c["n_fast_layer"], c["fast_dim"], c["fast_n_head"],
                         c["fast_n_kv_head"], c["fast_head_dim"], c["fast_qk_norm"])
        self.slow_cos, self.slow_sin = (t.astype(dtype) for t in rope_table(max_seq, c["head_dim"], c["rope_base"]))
        # The fast AR inherits the slow rope base; its positions are 0..N-1.
        self.fast_cos, self.fast_sin = (t.astype(dtype) for t in rope_table(self.N, c["fast_head_dim"], c["rope_base"]))
        # semantic_logit_bias: 0 on the semantic ids and <|im_end|>, -inf elsewhere.
        bias = np.full(c["vocab_size"], -np.inf)
        bias[self.sb:self.se + 1] = 0.0
        bias[self.end] = 0.0
        self.bias = bias
        self.count = Counters()
        self.taps = {}
        self.ras_used = False    # the last slow draw came from the loop breaker

    # --- cache helpers -----------------------------------------------------
    def _kv(self, t):
        return bf16_round(t).astype(self.dt) if self.kv_bf16 else t

    def new_sequence(self) -> SeqState:
        s = self.slow
        shp = (s.n_layer, self.max_seq, s.n_kv_head, s.head_dim)
        return SeqState(k=np.zeros(shp, dtype=self.dt), v=np.zeros(shp, dtype=self.dt))

    # --- a0: embedding + multi-codebook fusion -----------------------------
    def embed(self, col) -> np.ndarray:
        """Slow-AR input for one token column (id, q^(0..N-1)), in the
        oracle's precision (see `embed_column`)."""
        return embed_column(col, self.w["tok_embedding"], self.w["codebook_embedding"], self.sb, self.se,
                            self.N, self.C, bool(self.cfg["scale_codebook_embeddings"]))

    # --- one transformer layer, one new position ---------------------------
    def _layer_step(self, P: _Part, lw, x, pos, K, V, cos, sin):
        """x [dim]; K/V [max_pos, n_kv, hd] cache of this layer (written at pos)."""
        h = rms_norm(x, lw["attention_norm"], self.eps)
        q = (lw["wq"] @ h).reshape(P.n_head, P.head_dim)
        k = (lw["wk"] @ h).reshape(P.n_kv_head, P.head_dim)
        v = (lw["wv"] @ h).reshape(P.n_kv_head, P.head_dim)
        if P.qk_norm:
            q = rms_norm(q, lw["q_norm"], self.eps)
            k = rms_norm(k, lw["k_norm"], self.eps)
        q = apply_rope(q, cos[pos], sin[pos])
        k = apply_rope(k, cos[pos], sin[pos])
        K[pos] = self._kv(k)
        V[pos] = self._kv(v)
        rep = P.n_head // P.n_kv_head
        o = np.empty((P.n_head, P.head_dim), dtype=self.dt)
        for hh in range(P.n_head):
            g = hh // rep
            s = K[:pos + 1, g, :] @ q[hh] / math.sqrt(P.head_dim)
            p = np.exp(s - s.max())
            p /= p.sum()
            o[hh] = p @ V[:pos + 1, g, :]
        x = x + lw["wo"] @ o.reshape(-1)
        h2 = rms_norm(x, lw["ffn_norm"], self.eps)
        return x + lw["w2"] @ (silu(lw["w1"] @ h2) * (lw["w3"] @ h2))

    # --- the same layer over a whole causal sequence (prefill form) --------
    def _layer_seq(self, P: _Part, lw, X, pos0, K, V, cos, sin):
        """X [T, dim] for positions pos0..pos0+T-1, attending causally to the
        cache (positions < pos0 already filled) and to themselves."""
        T = X.shape[0]
        pos = np.arange(pos0, pos0 + T)
        H = rms_norm(X, lw["attention_norm"], self.eps)
        Q = (H @ lw["wq"].T).reshape(T, P.n_head, P.head_dim)
        Kn = (H @ lw["wk"].T).reshape(T, P.n_kv_head, P.head_dim)
        Vn = (H @ lw["wv"].T).reshape(T, P.n_kv_head, P.head_dim)
        if P.qk_norm:
            Q = rms_norm(Q, lw["q_norm"], self.eps)
            Kn = rms_norm(Kn, lw["k_norm"], self.eps)
        Q = apply_rope(Q, cos[pos][:, None, :], sin[pos][:, None, :])
        Kn = apply_rope(Kn, cos[pos][:, None, :], sin[pos][:, None, :])
        K[pos] = self._kv(Kn)
        V[pos] = self._kv(Vn)
        rep = P.n_head // P.n_kv_head
        O = np.empty((T, P.n_head, P.head_dim), dtype=self.dt)
        # Causal attention, QB query rows at a time: the rows of a block
        # attend to the keys up to the block's last position, and the keys
        # past a row's own position get a -inf score (exp gives exactly 0).
        # The blocks only skip scores that the mask would set to -inf.  The
        # heads are independent and run on a thread pool (numpy releases the
        # GIL), each with the same arithmetic as a serial loop.
        QB = 256

        def head(hh, r0, r1, Lb, future):
            g = hh // rep
            S = Q[r0:r1, hh, :] @ K[:Lb, g, :].T
            S /= math.sqrt(P.head_dim)
            S += future
            S -= S.max(axis=1, keepdims=True)
            np.exp(S, out=S)                                  # softmax numerator
            S /= S.sum(axis=1, keepdims=True)
            O[r0:r1, hh, :] = S @ V[:Lb, g, :]

        from threadpoolctl import threadpool_limits
        with threadpool_limits(1, user_api="blas"):       # one BLAS thread per head thread
            for r0 in range(0, T, QB):
                r1 = min(T, r0 + QB)
                Lb = pos0 + r1
                future = np.where(np.arange(Lb)[None, :] > pos[r0:r1, None], -np.inf, 0.0).astype(self.dt)
                list(_pool().map(lambda hh: head(hh, r0, r1, Lb, future), range(P.n_head)))
        X = X + O.reshape(T, -1) @ lw["wo"].T
        H2 = rms_norm(X, lw["ffn_norm"], self.eps)
        return X + (silu(H2 @ lw["w1"].T) * (H2 @ lw["w3"].T)) @ lw["w2"].T

    # --- slow AR -------------------------------------------------------------
    def slow_step(self, seq: SeqState, x, pos: int):
        """One slow-AR position; returns h_slow (the residual stream before the
        final norm, handed to the fast AR)."""
        for i, lw in enumerate(self.slow.layers):
            x = self._layer_step(self.slow, lw, x, pos, seq.k[i], seq.v[i],
                                 self.slow_cos, self.slow_sin)
        self.count.slow_passes += 1
        return x

    def slow_seq(self, seq: SeqState, X, pos0: int):
        for i, lw in enumerate(self.slow.layers):
            X = self._layer_seq(self.slow, lw, X, pos0, seq.k[i], seq.v[i],
                                self.slow_cos, self.slow_sin)
        return X

    def slow_logits(self, h):
        """Tied head over the whole vocabulary: E_tok . RMSNorm(h, g_final)."""
        return self.w["tok_embedding"] @ rms_norm(h, self.w["norm"], self.eps)

    def slow_sample(self, logits, s: Sampling, u, frames_emitted: int) -> int:
        """logits + semantic_logit_bias, then sample ([P2] `decode_one_token_ar`
        excerpt).  While fewer than `min_frames` frames are out, <|im_end|> is
        masked too."""
        bias = self.bias
        if frames_emitted < s.min_frames:
            bias = bias.copy()
            bias[self.end] = -np.inf
        return sample_token(logits + bias, s, u)

    def slow_sample_ras(self, seq: SeqState, logits, s: Sampling, u):
        """The slow draw with the loop breaker ([P2] "Two autoregressions ...",
        loop-breaker paragraph): draw normally; if that id is a semantic token
        among the ids emitted in the last `ras_window` frames, take a second
        draw at (ras_temperature, ras_top_p) with the frame's extra uniform
        u[N] instead.  Returns (id, whether the second draw was used)."""
        ident = self.slow_sample(logits, s, None if u is None else u[0], seq.frames)
        if s.ras_window <= 0 or ident == self.end or ident not in seq.ras_hist[-s.ras_window:]:
            return ident, False
        if u is None or len(u) <= self.N:
            raise ValueError("the loop breaker's draw needs a uniform in slot N of the frame's draws")
        s2 = Sampling(greedy=False, temperature=s.ras_temperature, top_p=s.ras_top_p, min_frames=s.min_frames)
        return self.slow_sample(logits, s2, u[self.N], seq.frames), True

    # --- fast AR ---------------------------------------------------------------
    def _fast_pass(self, x, k: int, Kf, Vf):
        for i, lw in enumerate(self.fast.layers):
            x = self._layer_step(self.fast, lw, x, k, Kf[i], Vf[i], self.fast_cos, self.fast_sin)
        self.count.fast_passes += 1
        self.count.slot_writes.append(k)
        return x

    def fast_logits(self, x):
        return self.w["fast_output"] @ rms_norm(x, self.w["fast_norm"], self.eps)

    def fast_frame(self, h_slow, q0: int, s: Sampling, u=None, force=None):
        """Ten (N) fast passes for one frame: pass 0 writes h_slow into slot 0
        (its output is not used); pass k = 1..N-1 embeds q^(k-1) at position k
        and samples q^(k) from the unmasked fast head.  Returns q^(0..N-1).
        force: codes q^(0..N-1) to take instead of sampling (the logits are
        still computed), so that another evaluation can follow this path."""
        F = self.fast
        Kf = np.zeros((F.n_layer, self.N, F.n_kv_head, F.head_dim), dtype=self.dt)
        Vf = np.zeros_like(Kf)
        self._fast_pass(np.asarray(h_slow, dtype=self.dt), 0, Kf, Vf)
        codes = [int(q0)]
        flog = []
        for k in range(1, self.N):
            x = self.w["fast_embeddings"][codes[-1]]
            x = self._fast_pass(x, k, Kf, Vf)
            lg = self.fast_logits(x)
            flog.append(lg)
            codes.append(int(force[k]) if force is not None else sample_token(lg, s, None if u is None else u[k]))
            self.count.fast_samples += 1
        self.taps["fast_logits"] = np.array(flog)
        return codes

    def fast_teacher_forced(self, h_slow, codes):
        """The training form of [P1] "Step 3": one causal pass over
        [h, E_fast(q^(0)), ..., E_fast(q^(N-2))]; returns the fast head's logits
        at positions 1..N-1 (the predictions of q^(1..N-1))."""
        F = self.fast
        X = np.concatenate([np.asarray(h_slow, dtype=self.dt)[None, :],
                            self.w["fast_embeddings"][np.asarray(codes[:self.N - 1])]], axis=0)
        Kf = np.zeros((F.n_layer, self.N, F.n_kv_head, F.head_dim), dtype=self.dt)
        Vf = np.zeros_like(Kf)
        for i, lw in enumerate(F.layers):
            X = self._layer_seq(F, lw, X, 0, Kf[i], Vf[i], self.fast_cos, self.fast_sin)
        return np.array([self.fast_logits(X[k]) for k in range(1, self.N)])

    # --- one frame: slow pass -> biased sample -> fast loop ----------------
    def _finish_frame(self, seq: SeqState, h, s: Sampling, u, force=None):
        logits = self.slow_logits(h)
        self.taps["slow_hidden"] = h
        self.taps["slow_logits"] = logits
        if force is not None:
            ident, self.ras_used = int(force[0]), False
        else:
            ident, self.ras_used = self.slow_sample_ras(seq, logits, s, u)
        if ident != self.end:
            # the loop breaker's window is the last frames' semantic ids,
            # whatever sampling produced them
            seq.ras_hist.append(ident)
        if ident == self.end:
            seq.done = True
            return [ident] + [-1] * self.N
        codes = self.fast_frame(h, ident - self.sb, s, u, None if force is None else force[1:])
        frame = [ident] + codes
        seq.next_col = np.array(frame)
        seq.frames += 1
        return frame

    def prefill(self, seq: SeqState, prompt, s: Sampling, u=None, force=None):
        """Run the slow AR over a prompt [N+1][P] (causal, all positions at
        once) and emit frame 0 from the last position (force: take that frame
        instead of sampling it)."""
        prompt = np.asarray(prompt)
        P = prompt.shape[1]
        X = np.stack([self.embed(prompt[:, t]) for t in range(P)])
        H = self.slow_seq(seq, X, 0)
        self.count.slow_passes += 1
        seq.pos = P
        return self._finish_frame(seq, H[-1], s, u, force)

    def prefill_stepwise(self, seq: SeqState, prompt, s: Sampling, u=None):
        """Same as `prefill`, one position at a time through the cache."""
        prompt = np.asarray(prompt)
        P = prompt.shape[1]
        for t in range(P):
            h = self.slow_step(seq, self.embed(prompt[:, t]), t)
        seq.pos = P
        return self._finish_frame(seq, h, s, u)

    def decode_frame(self, seq: SeqState, s: Sampling, u=None, force=None):
        """One frame: fuse the previous frame, one slow pass at the next
        position, biased sample, fast loop (force: take this frame instead of
        sampling it)."""
        if seq.done:
            return [-1] * (self.N + 1)
        x = self.embed(seq.next_col)
        self.taps["fused_x"] = x
        h = self.slow_step(seq, x, seq.pos)
        seq.pos += 1
        return self._finish_frame(seq, h, s, u, force)
