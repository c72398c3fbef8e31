"""HIP path vs the CPU oracle, through the C ABI, on seeded synthetic inputs.

Per frame: fused slow input, slow hidden state, slow logits and the fast
logits must agree to relative L2 <= 2e-3 (bf16 weights, fp32 accumulation;
the fp32 tiny model is held to 1e-4); sampled ids must match exactly where
the decision is clear (tests/parity.py).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import DualAROracle, Sampling as OSampling, embed_column, sample_token
from tests.parity import REL_L2, decision_margin, margin_ok, rel_l2, say

pytestmark = pytest.mark.gpu


def _dev():
    from dual_autoregressive_tts_amd import DualAR, load_library
    from dual_autoregressive_tts_amd.binding import upload_weights
    load_library()
    return DualAR, upload_weights


def run_and_compare(m, w_np, prompts, plen, n_frames, samp, uniforms=None, tol=REL_L2, min_frames=0,
                    tag="", weights_f32=None, floor=False, prefill_chunk=0, slow_logits_tap=True, ras=0,
                    stats=None, rows=None, weights_f64=None, seq_slack=2):
    """Prefill + n_frames single-frame decode calls on the GPU; the oracle
    replays every sequence (or the sequences in `rows`).  Returns per-row
    counts of frames compared (whole frames whose ids all matched) and the
    worst relative L2 distance per tap.  A frame's taps are compared before
    its ids, so a row whose first sampled ids differ within reach still has
    frame 0's slow hidden state and logits (and fast logits up to the first
    differing code) compared.  weights_f64 / weights_f32: the oracle's
    weights already converted, to skip the conversion on large models.

    The fused slow input of every decode frame must equal, bit for bit, the
    float32 evaluation of Eq. 1 on the oracle's previous frame (and lie
    within 1e-5 of the float64 value).

    With floor=True the oracle is also run in fp32, and each tap's bound is
    max(tol, min(1.5 fl, fl + tol)), fl = the fp32 oracle's distance to the
    fp64 oracle on the same frames: with bf16 K/V caches, rounding to bf16
    turns last-bit differences of fp32 arithmetic into occasional one-ulp
    (2^-8) cache differences, so an exact fp32 evaluation of the same steps
    already sits at that distance."""
    DualAR, upload = _dev()
    B, N = len(plen), m["num_codebooks"]
    greedy = samp["greedy"]
    # ras: the loop-breaker window of every call (an int), or one per frame
    # (frame 0 = the prefill's), so that calls can change it
    ras_f = list(ras) if isinstance(ras, (list, tuple)) else [ras] * (n_frames + 1)
    ras = max(ras_f)
    say(f"[{tag}] GPU: B={B} prompt_len={list(plen)[:8]} frames={n_frames} greedy={greedy}")
    dw = upload(m, w_np)
    # seq_slack: cache positions left over after the last frame (0 fills it)
    ctx = DualAR(m, dw, max_batch=B, max_seq_len=int(max(plen)) + n_frames + seq_slack, prefill_chunk=prefill_chunk)
    S_f = [DualAR.sampling(min_frames=min_frames, ras_window=r, **samp) for r in ras_f]
    tok = torch.from_numpy(np.ascontiguousarray(prompts)).cuda()
    U = None if uniforms is None else torch.from_numpy(np.ascontiguousarray(uniforms)).cuda()

    def u_at(f):   # frame f's draws, with slot N only when the breaker is on for that call
        if U is None:
            return None
        u = U[f:f + 1] if f > 0 else U[0]
        return u if ras_f[f] > 0 else u[..., :N].contiguous()
    # without the slow_logits tap a semantic-head context runs its restricted head
    which = True if slow_logits_tap else ("fused_x", "slow_hidden", "fast_logits")
    f0, t0 = ctx.prefill(tok, plen, S_f[0], u_at(0), taps=which)
    g_frames = [f0.cpu().numpy()]
    g_taps = [{k: v.cpu().numpy() for k, v in t0.items()}]
    for f in range(n_frames):
        codes, emitted, taps = ctx.decode_frames(1, S_f[1 + f], u_at(1 + f), taps=which)
        g_frames.append(codes[:, 0].cpu().numpy())
        g_taps.append({k: v.cpu().numpy() for k, v in taps.items()})
    g_emitted = emitted.cpu().numpy()
    assert ctx.sync() == 0
    ctx.close()
    del dw
    torch.cuda.empty_cache()

    say(f"[{tag}] oracle")
    wf = weights_f32 if weights_f32 is not None else synth.weights_as_f32(m, w_np)
    tok32 = np.asarray(wf["tok_embedding"], dtype=np.float32)
    cb32 = np.asarray(wf["codebook_embedding"], dtype=np.float32)
    fx_exact = 0
    osamp_f = [OSampling(greedy=bool(greedy), temperature=samp.get("temperature", 1.0),
                         top_p=samp.get("top_p", 1.0), min_frames=min_frames, ras_window=r) for r in ras_f]
    osamp = osamp_f[0]
    ras_used = 0
    compared = []
    worst = {"fused_x": 0.0, "slow_hidden": 0.0, "slow_logits": 0.0, "fast_logits": 0.0}
    floors = []
    taps_seen = []
    for b in (range(B) if rows is None else rows):
        o = DualAROracle(m, wf if weights_f64 is None else weights_f64, max_seq=int(plen[b]) + n_frames + 2)
        seq = o.new_sequence()
        n_taps = 0
        if floor:
            o32 = DualAROracle(m, wf, max_seq=int(plen[b]) + n_frames + 2, dtype=np.float32)
            seq32 = o32.new_sequence()
            fl = {"fused_x": 0.0, "slow_hidden": 0.0, "slow_logits": 0.0, "fast_logits": 0.0}
            in_step = True
        u = None if uniforms is None else uniforms[:, b, :].astype(np.float64)
        n_ok = 0
        for f in range(n_frames + 1):
            osamp = osamp_f[f]
            col = None if f == 0 or seq.done else seq.next_col.copy()
            ofr = o.prefill(seq, prompts[b][:, :plen[b]], osamp, None if u is None else u[0]) if f == 0 \
                else o.decode_frame(seq, osamp, None if u is None else u[f])
            gfr = g_frames[f][b].tolist()
            ras_used += int(osamp.ras_window > 0 and o.ras_used and ofr[0] != -1)
            bound = dict.fromkeys(worst, tol)
            bound["fused_x"] = 1e-5
            if floor and in_step:
                # the fp32 oracle takes the fp64 oracle's ids (its own draws may
                # flip on near-ties), so both evaluate the same path
                o32fr = o32.prefill(seq32, prompts[b][:, :plen[b]], osamp, None if u is None else u[0], force=ofr) \
                    if f == 0 else o32.decode_frame(seq32, osamp, None if u is None else u[f], force=ofr)
                if ofr[0] != -1:
                    for k in ("fused_x", "slow_hidden", "slow_logits"):
                        if k in o.taps and k in o32.taps and (f > 0 or k != "fused_x"):
                            fl[k] = max(fl[k], rel_l2(o32.taps[k], o.taps[k]))
                    if ofr[0] != m["end_id"]:
                        fl["fast_logits"] = max(fl["fast_logits"], rel_l2(o32.taps["fast_logits"], o.taps["fast_logits"]))
                in_step = o32fr == ofr
            if floor:
                for k in ("slow_hidden", "slow_logits", "fast_logits"):
                    bound[k] = max(tol, min(1.5 * fl[k], fl[k] + tol))
            t = g_taps[f]
            if col is not None and "fused_x" in t:
                # Eq. 1 in float32, bit for bit (the previous frames matched)
                fx = embed_column(col, tok32, cb32, m["semantic_begin_id"], m["semantic_end_id"], N,
                                  m["codebook_size"], bool(m["scale_codebook_embeddings"]))
                assert np.array_equal(t["fused_x"][b], fx), (tag, b, f, "fused_x not bit-exact",
                                                             int(np.sum(t["fused_x"][b] != fx)))
                fx_exact += 1
            if ofr[0] != -1:
                for k in ("fused_x", "slow_hidden", "slow_logits"):
                    if k not in t:
                        continue
                    e = rel_l2(t[k][b], o.taps[k])
                    worst[k] = max(worst[k], e)
                    assert e <= bound[k], (tag, b, f, k, e, bound[k])
                n_taps += 1
            if ofr[0] not in (-1, m["end_id"]) and gfr[0] == ofr[0]:
                # fast logits of pass k depend on q^(0..k-1): compare up to the first differing code
                kd = next((i for i in range(1, N) if gfr[1 + i] != ofr[1 + i]), N)
                e = rel_l2(g_taps[f]["fast_logits"][b][:kd], o.taps["fast_logits"][:kd])
                worst["fast_logits"] = max(worst["fast_logits"], e)
                assert e <= bound["fast_logits"], (tag, b, f, "fast_logits", e, bound["fast_logits"])
            if gfr == ofr:
                n_ok += 1
                if seq.done:
                    assert all(g_frames[ff][b].tolist() == [-1] * (N + 1) for ff in range(f + 1, n_frames + 1))
                    break
                continue
            # first differing id
            bias = o.bias.copy()
            if f < osamp.min_frames:          # frames emitted before this one = f
                bias[m["end_id"]] = -np.inf
            if gfr[0] != ofr[0] and "slow_logits" not in t:
                # restricted head, no GPU slow logits: greedy only, and the
                # oracle's own top-1 gap must be within the 1e-2 reach
                assert osamp.greedy, (tag, b, f, "slow id without slow logits")
                mg = decision_margin(o.taps["slow_logits"] + bias, True)
                assert mg <= 1e-2, (tag, b, f, "slow id", gfr[0], ofr[0], "oracle margin", mg)
            elif gfr[0] != ofr[0] and osamp.ras_window > 0:
                # loop breaker: the normal draws are compared first; where they
                # agree both sides hold the same window, so the breaker fired on
                # both or on neither
                zg, zo = t["slow_logits"][b] + bias, o.taps["slow_logits"] + bias
                ng, no = sample_token(zg, osamp, u[f][0]), sample_token(zo, osamp, u[f][0])
                if ng != no:
                    mg = check_decision(zg, zo, ng, no, osamp, u[f][0], (tag, b, f, "slow id (normal draw)"))
                else:
                    assert o.ras_used, (tag, b, f, "slow id differs with no loop-breaker draw", gfr[0], ofr[0])
                    s2 = OSampling(greedy=False, temperature=osamp.ras_temperature, top_p=osamp.ras_top_p,
                                   min_frames=min_frames)
                    mg = check_decision(zg, zo, gfr[0], ofr[0], s2, u[f][N], (tag, b, f, "slow id (loop breaker)"))
            elif gfr[0] != ofr[0]:
                mg = check_decision(t["slow_logits"][b] + bias, o.taps["slow_logits"] + bias, gfr[0], ofr[0],
                                    osamp, None if u is None else u[f][0], (tag, b, f, "slow id"))
            else:
                k = next(i for i in range(1, N) if gfr[1 + i] != ofr[1 + i])
                mg = check_decision(t["fast_logits"][b][k - 1], o.taps["fast_logits"][k - 1], gfr[1 + k],
                                    ofr[1 + k], osamp, None if u is None else u[f][k], (tag, b, f, "fast id", k))
            say(f"[{tag}] row {b} frame {f}: decision within the logits' reach (margin {mg:.2e}); "
                f"stop comparing this row")
            break
        compared.append(n_ok)
        taps_seen.append(n_taps)
        if floor:
            floors.append(fl)
        if n_ok == n_frames + 1 and not seq.done:
            assert g_emitted[b] == seq.frames, (tag, b, g_emitted[b], seq.frames)
    say(f"[{tag}] frames compared per row {compared} (frames with taps compared {taps_seen}); "
        f"worst rel L2 {worst}; fused inputs bit-exact: {fx_exact}")
    if stats is not None:
        stats["taps_compared"] = taps_seen
    if ras:
        say(f"[{tag}] loop-breaker draws taken by the oracle: {ras_used}")
    if stats is not None:
        stats["ras_used"] = ras_used
    if floor:
        say(f"[{tag}] fp32-oracle distance to the fp64 oracle per row: {floors}")
    return compared, worst


def check_decision(zg, zo, gid, oid, osamp, u, ctx):
    """A sampled id differs from the oracle's.  (1) The GPU sampler must draw
    exactly what the oracle's sampler draws from the GPU's own logits (up to a
    float32-vs-float64 cumulative-sum knife edge for top-p).  (2) The oracle's
    own decision must be within reach of the logit differences: greedy top-1
    margin <= 1e-2, top-p u-margin <= max(1e-4, 2 max|dz| / T)."""
    greedy = osamp.greedy or u is None
    sg = sample_token(zg, osamp, u)
    if sg != gid:
        mg_g = decision_margin(zg, greedy, osamp.temperature, osamp.top_p, u)
        assert not greedy and mg_g <= 1e-5, ctx + ("sampler", gid, sg, mg_g)
    fin = np.isfinite(zo)
    dz = float(np.max(np.abs(np.asarray(zg, np.float64)[fin] - np.asarray(zo, np.float64)[fin])))
    thr = 1e-2 if greedy else max(1e-4, 2.0 * dz / osamp.temperature)
    mg = decision_margin(zo, greedy, osamp.temperature, osamp.top_p, u)
    assert mg <= thr, ctx + ("ids", gid, oid, "oracle margin", mg, "reach", thr)
    return mg


# ----------------------------------------------------------------------------
# tiny model (the fp32 workload and variants)
# ----------------------------------------------------------------------------

@pytest.fixture(scope="module")
def tiny():
    m = synth.model("tiny")
    return m, synth.make_weights(m, seed=0)


def test_tiny_greedy_16_frames(tiny):
    m, w = tiny
    P = synth.make_prompts(m, ("fixed", 4, 16, 12), [32])
    c, worst = run_and_compare(m, w, P, [32], 16, dict(greedy=1), tol=1e-4, tag="tiny-b1")
    assert c[0] >= 12
    assert worst["slow_logits"] < 1e-4


def test_tiny_ragged_batch_top_p(tiny):
    m, w = tiny
    plen = np.array([32, 7, 1, 45, 20], dtype=np.int32)
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=3)
    U = synth.make_uniforms((9, 5, m["num_codebooks"]), seed=3)
    c, _ = run_and_compare(m, w, P, plen, 8, dict(greedy=0, temperature=1.0, top_p=0.9), U, tol=1e-4,
                           tag="tiny-topp")
    assert sum(c) >= 30


def test_tiny_semantic_head(tiny):
    # the slow head over the C semantic rows and the end row only: the same
    # draws (the other logits are masked to -inf anyway)
    m, w = tiny
    m = dict(m, semantic_head=1)
    plen = np.array([32, 7, 1, 45, 20], dtype=np.int32)
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=4)
    c, worst = run_and_compare(m, w, P, plen, 6, dict(greedy=1), tol=1e-4, tag="tiny-semhead",
                               slow_logits_tap=False)
    assert sum(c) >= 20
    assert "slow_logits" not in worst or worst["slow_logits"] == 0.0


@pytest.mark.parametrize("greedy", [1, 0])
def test_tiny_loop_breaker(tiny, greedy):
    # The slow loop breaker with the pages' window of 10 frames: a draw that
    # repeats a semantic id of the last 10 emitted frames is replaced by a
    # second draw at T = 1.0, top-p 0.9 from slot N of the frame's uniforms.
    # The greedy tiny model repeats itself, so the breaker fires.
    m, w = tiny
    plen = np.array([32, 7, 45], dtype=np.int32)
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=6)
    U = synth.make_uniforms((17, 3, m["num_codebooks"] + 1), seed=6)
    samp = dict(greedy=1) if greedy else dict(greedy=0, temperature=0.7, top_p=0.8)
    stats = {}
    c, _ = run_and_compare(m, w, P, plen, 16, samp, U, tol=1e-4, tag=f"tiny-ras-g{greedy}", ras=10, stats=stats)
    assert sum(c) >= 24
    if greedy:
        assert stats["ras_used"] > 0


def test_tiny_loop_breaker_window_changes(tiny):
    # calls that turn the loop breaker off and on and change its window: the
    # window is always the ids of the last `ras_window` emitted frames, those
    # emitted with the breaker off included ([P2] loop-breaker paragraph)
    m, w = tiny
    plen = np.array([32, 7, 45], dtype=np.int32)
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=6)
    U = synth.make_uniforms((17, 3, m["num_codebooks"] + 1), seed=16)
    windows = [0] * 6 + [3] * 6 + [10] * 5
    stats = {}
    c, _ = run_and_compare(m, w, P, plen, 16, dict(greedy=1), U, tol=1e-4, tag="tiny-ras-windows", ras=windows,
                           stats=stats)
    assert sum(c) >= 24, c
    assert stats["ras_used"] > 0


def test_tiny_loop_breaker_widest_window(tiny):
    # the widest window (DUALAR_RAS_MAX_WINDOW = 16, the whole per-sequence
    # ring of emitted ids) over 30 frames, so that the ring wraps and the
    # window reaches its oldest slot
    m, w = tiny
    plen = np.array([32, 7, 45], dtype=np.int32)
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=22)
    U = synth.make_uniforms((31, 3, m["num_codebooks"] + 1), seed=22)
    stats = {}
    c, _ = run_and_compare(m, w, P, plen, 30, dict(greedy=1), U, tol=1e-4, tag="tiny-ras-16", ras=16, stats=stats)
    assert sum(c) >= 45, c
    assert stats["ras_used"] > 0


@pytest.mark.timeout(600)
@pytest.mark.parametrize("pc", [4096, 1000])
def test_bf16_prefill_many_row_tiles(pc):
    # 8 sequences of 700..4,096 positions with 4,096 or 1,000 positions per
    # sequence per prefill step: 32,768 and 8,000 activation rows per step.
    # Past 128 tiles of 128 rows the host passes no live-tile mask and the
    # 2-D tile products run every tile, padding rows included; 1,000 leaves
    # a ragged 64-row last tile and five steps with the padding in front
    m = synth.model("tiny", weight_dtype="bf16", dim=512, ffn_dim=1024, fast_dim=512, fast_ffn_dim=1024,
                    n_head=4, n_kv_head=1, head_dim=128, fast_n_head=4, fast_n_kv_head=1, fast_head_dim=128)
    w = synth.make_weights(m, seed=18)
    plen = synth.make_ctx_lengths(8, 700, 4096, seed=18)
    plen[0] = 4096
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=18)
    c, worst = run_and_compare(m, w, P, plen, 2, dict(greedy=1), tag=f"bf16-prefill-pc{pc}", floor=True,
                               prefill_chunk=pc, rows=[0, 1, 4, 7])
    assert sum(c) >= 6


@pytest.mark.parametrize("pc", [1, 3, 16, 64])
def test_tiny_prefill_chunking(tiny, pc):
    # Prefill walks the right-aligned prompts pc positions at a time (pc = 1
    # is the one-position-per-step form; 64 covers the longest prompt in one
    # step); a chunk's rows attend to earlier rows of the same chunk.
    m, w = tiny
    plen = np.array([32, 7, 1, 45, 20], dtype=np.int32)
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=9)
    c, worst = run_and_compare(m, w, P, plen, 3, dict(greedy=1), tol=1e-4, tag=f"tiny-pc{pc}", prefill_chunk=pc)
    assert sum(c) >= 10
    assert worst["slow_logits"] < 1e-4


def test_tiny_temperature_top_p_half(tiny):
    m, w = tiny
    plen = np.array([12, 30], dtype=np.int32)
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=5)
    U = synth.make_uniforms((6, 2, m["num_codebooks"]), seed=5)
    c, _ = run_and_compare(m, w, P, plen, 5, dict(greedy=0, temperature=0.7, top_p=0.5), U, tol=1e-4,
                           tag="tiny-T0.7")
    assert sum(c) >= 8


@pytest.mark.parametrize("top_p,temp", [(1.0, 2.0), (0.02, 0.5), (0.999, 1.0), (0.9, 0.05), (0.9, 20.0)])
def test_tiny_top_p_extremes(tiny, top_p, temp):
    # the sampler's nucleus at its ends: every candidate kept (top_p 1 at a
    # high temperature: the draw walks the whole order), a nucleus of one or
    # two tokens, and a boundary near the tail of the order; temperatures
    # of 0.05 (most masses underflow: the fixed-point masses of all but the
    # top few candidates are 0) and 20 (nearly flat)
    m, w = tiny
    plen = np.array([7, 21, 3, 30, 16], dtype=np.int32)
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=9)
    U = synth.make_uniforms((5, 5, m["num_codebooks"]), seed=9)
    c, _ = run_and_compare(m, w, P, plen, 4, dict(greedy=0, temperature=temp, top_p=top_p), U, tol=1e-4,
                           tag=f"tiny-topp{top_p}-T{temp}")
    assert sum(c) >= 10


@pytest.mark.parametrize("greedy", [1, 0])
def test_tiny_degenerate_shapes(greedy):
    # the smallest model the config accepts: 2 codebooks of 2 codes (one fast
    # draw per frame, a draw between two candidates), one slow and one fast
    # layer (fast pass 0 is only the K/V rows of that layer)
    m = synth.model("tiny", num_codebooks=2, codebook_size=2, semantic_begin_id=1024, semantic_end_id=1025,
                    acoustic_size=2, n_layer=1, n_fast_layer=1)
    w = synth.make_weights(m, seed=4)
    plen = np.array([1, 9, 4], dtype=np.int32)
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=4)
    U = synth.make_uniforms((7, 3, m["num_codebooks"]), seed=4)
    samp = dict(greedy=1) if greedy else dict(greedy=0, temperature=1.0, top_p=0.9)
    c, _ = run_and_compare(m, w, P, plen, 6, samp, None if greedy else U, tol=1e-4, min_frames=1 << 20,
                           tag=f"tiny-degenerate-g{greedy}")
    assert sum(c) >= 9


@pytest.mark.parametrize("N,C,heads,B", [(32, 1000, "small", 3), (32, 1000, "s2", 1), (32, 1000, "s2", 6),
                                          (3, 4096, "small", 4)])
def test_codebook_counts_and_sizes(N, C, heads, B):
    # 32 codebooks, the most the config accepts (31 fast passes; the fast
    # layers' depth cache then holds more than the 16 positions of the fused
    # batch-1 attention + O kernel and of the one-wave depth attention, so
    # the general attention forms run there), a codebook of 1,000 codes;
    # 3 codebooks of 4,096.  "small": the fp32 model with 4 query heads of
    # 64 (top-p, strict bound); "s2": bf16 weights and cache with the S2
    # head shape at dim 512 (greedy, rounding-floor bound)
    kw = dict(num_codebooks=N, codebook_size=C, semantic_begin_id=1024, semantic_end_id=1024 + C - 1,
              acoustic_size=min(C, 256))
    if heads == "s2":
        kw.update(weight_dtype="bf16", dim=512, ffn_dim=1024, fast_dim=512, fast_ffn_dim=1024, n_head=32, n_kv_head=8,
                  head_dim=128, fast_n_head=32, fast_n_kv_head=8, fast_head_dim=128)
    m = synth.model("tiny", **kw)
    w = synth.make_weights(m, seed=16)
    plen = synth.make_ctx_lengths(B, 1, 40, seed=16)
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=16)
    if heads == "small":
        samp, U, tol = dict(greedy=0, temperature=1.0, top_p=0.9), synth.make_uniforms((4, B, N), seed=16), 1e-4
    else:
        samp, U, tol = dict(greedy=1), None, REL_L2
    c, worst = run_and_compare(m, w, P, plen, 3, samp, U, tol=tol, min_frames=1 << 20,
                               tag=f"codebooks-{N}x{C}-{heads}-B{B}", floor=heads == "s2")
    assert sum(c) >= 2 * B


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wdtype,B", [("f32", 1), ("f32", 3), ("bf16", 1), ("bf16", 3)])
def test_widest_model_dim(wdtype, B):
    # dim 12,288, the widest the config accepts: rows of 24 units (bf16) or 48
    # (fp32) take the general loop GEMV with the whole activation row staged
    # in 48 KB of LDS; at batch 3 the fp32 products stage one row at a time
    # (two or four would pass the LDS limit) and the bf16 ones run on the
    # matrix cores
    heads = {} if wdtype == "f32" else dict(n_head=8, n_kv_head=2, fast_n_head=8, fast_n_kv_head=2)   # 512-wide rows
    m = synth.model("tiny", weight_dtype=wdtype, dim=12288, fast_dim=12288, ffn_dim=512, fast_ffn_dim=512,
                    n_layer=1, n_fast_layer=1, **heads)
    w = synth.make_weights(m, seed=21)
    plen = synth.make_ctx_lengths(B, 5, 30, seed=21)
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=21)
    c, worst = run_and_compare(m, w, P, plen, 2, dict(greedy=1), tol=1e-4 if wdtype == "f32" else REL_L2,
                               tag=f"dim12288-{wdtype}-B{B}", floor=False)
    assert sum(c) >= 2 * B


@pytest.mark.parametrize("fast_qk", [1, 0])
def test_tiny_bf16_kv(fast_qk):
    m = synth.model("tiny", weight_dtype="bf16", dim=512, ffn_dim=1024, fast_dim=512, fast_ffn_dim=1024,
                    n_head=8, n_kv_head=2, fast_n_head=8, fast_n_kv_head=2, fast_qk_norm=fast_qk)
    w = synth.make_weights(m, seed=1)
    plen = np.array([40, 9, 64], dtype=np.int32)
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=1)
    c, worst = run_and_compare(m, w, P, plen, 6, dict(greedy=1), tag=f"tiny-bf16-fqk{fast_qk}", floor=True)
    assert sum(c) >= 12


@pytest.mark.parametrize("B", [11, 33, 70])
def test_tiny_bf16_batched_matrix_cores(B):
    # 2+ activation rows take the matrix-core products: one or two 32-row
    # activation tiles the stream-K form (11, 33), three the split-K form
    # with its finish (70); ragged batch tiles; top-p draws from supplied
    # uniforms.
    m = synth.model("tiny", weight_dtype="bf16", dim=512, ffn_dim=1024, fast_dim=512, fast_ffn_dim=1024,
                    n_head=8, n_kv_head=2, fast_n_head=8, fast_n_kv_head=2)
    w = synth.make_weights(m, seed=2)
    plen = synth.make_ctx_lengths(B, 1, 40, seed=B)
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=B)
    U = synth.make_uniforms((4, B, m["num_codebooks"]), seed=B)
    c, worst = run_and_compare(m, w, P, plen, 3, dict(greedy=0, temperature=1.0, top_p=0.9), U,
                               tag=f"tiny-bf16-B{B}", floor=True)
    assert sum(c) >= 2 * B


@pytest.mark.timeout(600)
def test_bf16_batched_long_context(tiny):
    # bf16 cache, head_dim 128, 4 query heads per KV head, 9 sequences with
    # contexts of 300..1400: decode attention walks several 128-position
    # tiles per workgroup and several workgroups per head (merged), with the
    # new position in the last, ragged tile.
    m = synth.model("tiny", weight_dtype="bf16", dim=512, ffn_dim=1024, fast_dim=512, fast_ffn_dim=1024,
                    n_head=4, n_kv_head=1, head_dim=128, fast_n_head=4, fast_n_kv_head=1, fast_head_dim=128)
    w = synth.make_weights(m, seed=6)
    plen = np.array([1400, 300, 777, 1024, 513, 640, 1151, 385, 900], dtype=np.int32)
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=6)
    c, worst = run_and_compare(m, w, P, plen, 3, dict(greedy=1), tag="bf16-long", floor=True)
    assert sum(c) >= 18


def test_bf16_small_batch_long_context():
    # batch 3 with contexts past 2,048 positions takes the balanced
    # flash-decoding form (tiles over all (sequence, KV head) pairs, heads
    # split over workgroups and merged); batch 1 past 2,048 too, with the
    # separate query preparation (no batched QKV finish at batch 1)
    m = synth.model("tiny", weight_dtype="bf16", dim=512, ffn_dim=1024, fast_dim=512, fast_ffn_dim=1024,
                    n_head=4, n_kv_head=1, head_dim=128, fast_n_head=4, fast_n_kv_head=1, fast_head_dim=128)
    w = synth.make_weights(m, seed=7)
    for plen in (np.array([2300, 2100, 2600], dtype=np.int32), np.array([2200], dtype=np.int32)):
        P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=7)
        c, worst = run_and_compare(m, w, P, plen, 3, dict(greedy=1), tag=f"bf16-long-b{len(plen)}", floor=True)
        assert sum(c) >= 3 * len(plen)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("plen,B", [(2046, 1), (2558, 1), (2046, 3), (16, 1), (126, 6)])
def test_attention_form_boundaries(plen, B):
    # decode frames whose context crosses the host's switches between the
    # attention forms from one frame to the next: 2,048 positions (4-load to 8-load
    # splits: batch 1 stays in the split form merged inside the O product,
    # batch 3 moves from the split form to the flash form), 2,560 (batch 1:
    # past 10 splits of 256 positions the O product no longer merges and the
    # flash form takes over), 16 positions at batch 1 and 128 at batch 6
    # (one attention chunk / flash tile to two); S2 head shape at dim 512,
    # bf16 cache, five frames
    m = synth.model("tiny", weight_dtype="bf16", dim=512, ffn_dim=1024, fast_dim=512, fast_ffn_dim=1024, n_head=32,
                    n_kv_head=8, head_dim=128, fast_n_head=32, fast_n_kv_head=8, fast_head_dim=128)
    w = synth.make_weights(m, seed=17)
    lens = np.full(B, plen, dtype=np.int32)
    lens[1:] -= np.arange(1, B, dtype=np.int32)          # ragged by one position per row
    P = synth.make_prompts(m, ("ragged", 1, 1), lens, seed=17)
    c, worst = run_and_compare(m, w, P, lens, 5, dict(greedy=1), min_frames=1 << 20,
                               tag=f"form-boundary-{plen}-B{B}", floor=True)
    assert sum(c) >= 3 * B


@pytest.mark.parametrize("plen,B", [(509, 1), (636, 6), (2555, 1)])
def test_cache_filled_to_the_last_position(plen, B):
    # max_seq_len = the longest prompt + the frames: the last frame writes
    # and attends to the cache's (and the RoPE table's) last position, with
    # the 128-position attention chunks / flash tiles ending exactly there
    # (512 and 640 positions; 2,560 at batch 1 past 10 splits of 256)
    m = synth.model("tiny", weight_dtype="bf16", dim=512, ffn_dim=1024, fast_dim=512, fast_ffn_dim=1024, n_head=32,
                    n_kv_head=8, head_dim=128, fast_n_head=32, fast_n_kv_head=8, fast_head_dim=128)
    w = synth.make_weights(m, seed=20)
    lens = np.full(B, plen, dtype=np.int32)
    lens[1:] -= 5 * np.arange(1, B, dtype=np.int32)
    P = synth.make_prompts(m, ("ragged", 1, 1), lens, seed=20)
    c, worst = run_and_compare(m, w, P, lens, 3, dict(greedy=1), min_frames=1 << 20, tag=f"cache-full-{plen}-B{B}",
                               floor=True, seq_slack=0)
    assert sum(c) >= 2 * B


@pytest.mark.timeout(900)
def test_bf16_long_context_past_32k():
    # positions past 32,767 (45,000 and 20,000 prompt positions at batch 2):
    # RoPE rows of the bf16 table that far out, the chunked prefill over 11
    # steps of 4,096 positions, then the flash-decoding form with ~350 tiles
    # per head split over the grid and merged
    m = synth.model("tiny", weight_dtype="bf16", dim=512, ffn_dim=1024, fast_dim=512, fast_ffn_dim=1024,
                    n_head=4, n_kv_head=1, head_dim=128, fast_n_head=4, fast_n_kv_head=1, fast_head_dim=128)
    w = synth.make_weights(m, seed=13)
    plen = np.array([45000, 20000], dtype=np.int32)
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=13)
    c, worst = run_and_compare(m, w, P, plen, 2, dict(greedy=1), tag="bf16-past-32k", floor=True)
    assert sum(c) >= 3


@pytest.mark.timeout(600)
@pytest.mark.parametrize("n_head,n_kv,hd,kv", [(4, 4, 128, "bf16"), (8, 1, 128, "bf16"), (8, 1, 64, "bf16"),
                                               (8, 1, 128, "f32"), (8, 4, 128, "bf16")])
@pytest.mark.parametrize("B", [1, 6])
def test_head_shapes(n_head, n_kv, hd, kv, B):
    # query heads per KV head 1, 2 and 8 (the S2 shape, 4, runs everywhere
    # else), head_dim 64 and 128, bf16 and fp32 caches, in the slow and the
    # fast layers alike; contexts up to 2,400 positions so that both the
    # 4-load and the 8-load attention splits run: 1 query head per KV head
    # takes the balanced flash-decoding form, 8 the split form with its
    # merge (matrix-core scores for head_dim 128 with a bf16 cache)
    m = synth.model("tiny", weight_dtype="bf16", kv_dtype=kv, dim=512, ffn_dim=1024, fast_dim=512,
                    fast_ffn_dim=1024, n_head=n_head, n_kv_head=n_kv, head_dim=hd, fast_n_head=n_head,
                    fast_n_kv_head=n_kv, fast_head_dim=hd)
    w = synth.make_weights(m, seed=14)
    plen = np.array([2400], dtype=np.int32) if B == 1 else synth.make_ctx_lengths(B, 100, 2400, seed=14)
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=14)
    c, worst = run_and_compare(m, w, P, plen, 2, dict(greedy=1), tag=f"heads-{n_head}-{n_kv}-{hd}-{kv}-B{B}",
                               floor=kv == "bf16")
    assert sum(c) >= (3 * B + 1) // 2
    if kv == "f32":
        assert max(worst.values()) < REL_L2


@pytest.mark.timeout(600)
@pytest.mark.parametrize("plen,kv", [(600, "bf16"), (1100, "bf16"), (1500, "bf16"), (300, "f32")])
def test_batch1_s2_heads_merged_in_o_product(plen, kv):
    # batch 1 with the S2 head shape (32 query / 8 KV heads of 128): the slow
    # attention runs in chunks (128 positions at 600 and 1,100: 5 and 9
    # splits; 256 at 1,500 so that at most 10 splits remain; 64 with an fp32
    # cache) and the O product merges each head's partials itself; the fast
    # layers attend inside the O product.  Dim 512 keeps the oracle's replay
    # short.
    m = synth.model("tiny", weight_dtype="bf16", kv_dtype=kv, dim=512, ffn_dim=1024, fast_dim=512,
                    fast_ffn_dim=1024, n_head=32, n_kv_head=8, head_dim=128, fast_n_head=32,
                    fast_n_kv_head=8, fast_head_dim=128)
    w = synth.make_weights(m, seed=8)
    P = synth.make_prompts(m, ("ragged", 1, 1), np.array([plen], dtype=np.int32), seed=8)
    c, worst = run_and_compare(m, w, P, np.array([plen], dtype=np.int32), 3, dict(greedy=1),
                               tag=f"b1-merge-o-{plen}-{kv}", floor=(kv == "bf16"))
    assert sum(c) >= 3


# ----------------------------------------------------------------------------
# W4A16 (the survey's NEXT 4): 4-bit weight groups, batch 1
# ----------------------------------------------------------------------------

def _w4_case(m, seed, plen, frames, tag, prefill_chunk=1):
    from oracle import dequant_w4
    w4 = synth.make_w4_model(m, synth.make_weights(m, seed=seed))
    wf = dequant_w4(synth.weights_as_f32(m, w4))          # the oracle's own q * scale
    P = synth.make_prompts(m, ("ragged", 1, 1), np.array([plen], dtype=np.int32), seed=seed)
    return run_and_compare(m, w4, P, np.array([plen], dtype=np.int32), frames, dict(greedy=1), tag=tag,
                           weights_f32=wf, floor=m.get("kv_dtype", "bf16") == "bf16", prefill_chunk=prefill_chunk)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("kv", ["bf16", "f32"])
def test_w4a16_batch1_small(kv):
    # rows of 512 and 1,024 inputs (one and two units of 512 per wave); slow
    # layer 0 fully 4-bit, layer 1 keeps its attention in bf16; fast layers
    # 4-bit (a head shape the split attention kernels do not take)
    m = synth.model("tiny", weight_dtype="bf16", kv_dtype=kv, dim=512, ffn_dim=1024, fast_dim=512,
                    fast_ffn_dim=1024, n_head=4, n_kv_head=1, head_dim=128, fast_n_head=4, fast_n_kv_head=1,
                    fast_head_dim=128, w4a16=1, w4_bf16_attn_layers=1)
    c, worst = _w4_case(m, 9, 40, 4, f"w4-small-{kv}")
    assert sum(c) >= 4


@pytest.mark.timeout(900)
def test_w4a16_batch1_s2_shapes():
    # the S2 shapes (rows of 2,560 / 4,096 / 9,728 inputs: 5 units of 512 in
    # one wave, 8 over two waves, 19 over four with one dead unit) with 3 slow
    # layers: layers 0-1 fully 4-bit, layer 2 keeps its attention in bf16 (so
    # its O product takes the fused bf16 kernels), the fast layers 4-bit.  A
    # 300-token prompt: the 4-bit-O slow layers attend in 3 splits of 128
    # positions joined by the plain merge; the fast layers in one split.
    m = synth.model("s2", n_layer=3, w4a16=1, w4_bf16_attn_layers=1)
    c, worst = _w4_case(m, 10, 300, 2, "w4-s2")
    assert sum(c) >= 2


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dim,ffn,n_head", [(10240, 5632, 8), (1536, 3072, 12)])
def test_w4a16_row_lengths(dim, ffn, n_head):
    # 4-bit rows of other lengths than the S2 ones: 10,240 inputs (the
    # largest accepted: 20 units over four waves, 80 chunks on the matrix
    # cores), 5,632 (11 units over four waves with one dead unit), 1,024,
    # 1,536 (3 units in one wave), 3,072 (6 units over two waves); slow layer
    # 1 keeps its attention in bf16
    m = synth.model("tiny", weight_dtype="bf16", dim=dim, ffn_dim=ffn, fast_dim=dim, fast_ffn_dim=ffn,
                    n_head=n_head, n_kv_head=n_head // 4, head_dim=128, fast_n_head=n_head,
                    fast_n_kv_head=n_head // 4, fast_head_dim=128, w4a16=1, w4_bf16_attn_layers=1)
    c, worst = _w4_case(m, 15, 30, 3, f"w4-rows-{dim}-{ffn}")
    assert sum(c) >= 2


@pytest.mark.timeout(900)
@pytest.mark.parametrize("plen", [300, 40])
def test_w4a16_chunked_prefill_s2_shapes(plen):
    # prefill steps of 256 positions: the 4-bit products on the matrix-core
    # 2-D tiles (each group of 128 inputs summed on the matrix cores, then
    # scaled in fp32).  A 300-token prompt takes two steps (the first one's
    # rows 0..211 are left padding, so only its last activation tile is
    # live), a 40-token prompt one padded step; the decode frames then run
    # the 4-bit GEMVs.  Layers 0-1 fully 4-bit, layer 2 with bf16 attention.
    m = synth.model("s2", n_layer=3, w4a16=1, w4_bf16_attn_layers=1)
    c, worst = _w4_case(m, 10, plen, 2, f"w4-s2-pc256-{plen}", prefill_chunk=256)
    assert sum(c) >= 2


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dim,ffn,n_head,kv", [(10240, 5632, 8, "bf16"), (1536, 3072, 12, "f32"),
                                               (512, 1024, 4, "f32")])
def test_w4a16_chunked_prefill_row_lengths(dim, ffn, n_head, kv):
    # the 4-bit 2-D tiles at other row lengths: 10,240 inputs (80 scale groups,
    # the LDS limit), 5,632, 3,072, 1,536, 1,024 and 512; a 600-token prompt in
    # two steps of 512 positions (the first one ragged)
    m = synth.model("tiny", weight_dtype="bf16", kv_dtype=kv, dim=dim, ffn_dim=ffn, fast_dim=dim, fast_ffn_dim=ffn,
                    n_head=n_head, n_kv_head=n_head // 4, head_dim=128, fast_n_head=n_head,
                    fast_n_kv_head=n_head // 4, fast_head_dim=128, w4a16=1, w4_bf16_attn_layers=1)
    c, worst = _w4_case(m, 16, 600, 3, f"w4-pc512-{dim}-{ffn}", prefill_chunk=512)
    assert sum(c) >= 2


def _w4_small(kv):
    return synth.model("tiny", weight_dtype="bf16", kv_dtype=kv, dim=512, ffn_dim=1024, fast_dim=512,
                       fast_ffn_dim=1024, n_head=4, n_kv_head=1, head_dim=128, fast_n_head=4, fast_n_kv_head=1,
                       fast_head_dim=128, w4a16=1, w4_bf16_attn_layers=1)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B,kv,pc", [(2, "bf16", 1), (3, "f32", 1), (4, "bf16", 1), (4, "f32", 0), (6, "f32", 1),
                                    (8, "bf16", 1), (8, "f32", 0)])
def test_w4a16_small_batch(B, kv, pc):
    # 4-bit products over 2-8 activation rows on the matrix cores (the batch's
    # rows as product rows 4b + t, t the activation term, in one or two
    # groups of four; up to 4 rows the kernel normalises and splits its input
    # itself, above that it reads the input planes); ragged prompts, greedy,
    # 5 frames; one position per prefill step, or (pc 0) one step of 256
    # padded positions per sequence on the 4-bit 2-D tiles
    m = _w4_small(kv)
    from oracle import dequant_w4
    w4 = synth.make_w4_model(m, synth.make_weights(m, seed=18))
    wf = dequant_w4(synth.weights_as_f32(m, w4))
    plen = np.array([40, 17, 33, 25, 9, 31, 22, 38][:B], dtype=np.int32)
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=18)
    c, worst = run_and_compare(m, w4, P, plen, 5, dict(greedy=1), tag=f"w4-b{B}-{kv}-pc{pc}", weights_f32=wf,
                               floor=kv == "bf16", prefill_chunk=pc)
    assert sum(c) >= 2 * B


@pytest.mark.timeout(900)
def test_w4a16_batch4_s2_shapes_top_p():
    # the S2 shapes with 3 slow layers (layers 0-1 fully 4-bit, layer 2 with
    # bf16 attention, 4-bit fast layers), batch 4, ragged prompts of 300, 120,
    # 77 and 210 tokens (one prefill step on the 4-bit 2-D tiles), top-p 0.9
    # on an fp32 cache, 3 frames
    from oracle import dequant_w4
    m = synth.model("s2", n_layer=3, w4a16=1, w4_bf16_attn_layers=1, kv_dtype="f32")
    w4 = synth.make_w4_model(m, synth.make_weights(m, seed=19))
    wf = dequant_w4(synth.weights_as_f32(m, w4))
    plen = np.array([300, 120, 77, 210], dtype=np.int32)
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=19)
    U = synth.make_uniforms((4, 4, m["num_codebooks"]), seed=19)
    c, worst = run_and_compare(m, w4, P, plen, 3, dict(greedy=0, temperature=1.0, top_p=0.9), U,
                               tag="w4-s2-b4-topp", weights_f32=wf)
    assert sum(c) >= 8


def test_end_token_stops_and_pads(tiny):
    m, w = tiny
    w = {k: v.copy() for k, v in w.items()}
    P = synth.make_prompts(m, ("fixed", 4, 16, 12), [32])
    # Make <|im_end|> win once the semantic logit it copies is large: its row
    # becomes a scaled copy of the row of the oracle's greedy frame-3 id.
    o = DualAROracle(m, synth.weights_as_f32(m, w), max_seq=64)
    seq = o.new_sequence()
    fr = [o.prefill(seq, P[0], OSampling())] + [o.decode_frame(seq, OSampling()) for _ in range(3)]
    w["tok_embedding"][m["end_id"]] = 3.0 * w["tok_embedding"][fr[3][0]]
    for mf in (0, 3):
        c, _ = run_and_compare(m, w, P, [32], 8, dict(greedy=1), tol=1e-4, min_frames=mf, tag=f"end-mf{mf}")
        assert c[0] >= 1


def test_bad_prompt_id_is_reported(tiny):
    DualAR, upload = _dev()
    from dual_autoregressive_tts_amd import DualARError
    m, w = tiny
    P = synth.make_prompts(m, ("fixed", 4, 16, 12), [32])
    P[0, 0, 3] = m["vocab_size"] + 7
    ctx = DualAR(m, upload(m, w), max_batch=1, max_seq_len=40)
    say("[bad-id] GPU prefill with an out-of-range id")
    ctx.prefill(torch.from_numpy(P).cuda(), [32], DualAR.sampling())
    with pytest.raises(DualARError) as e:
        ctx.sync()
    assert e.value.name == "BAD_TOKEN"
    assert ctx.sync() == 0


def test_context_full_and_state_errors(tiny):
    DualAR, upload = _dev()
    from dual_autoregressive_tts_amd import DualARError
    m, w = tiny
    ctx = DualAR(m, upload(m, w), max_batch=2, max_seq_len=36)
    S = DualAR.sampling()
    with pytest.raises(DualARError) as e:
        ctx.decode_frames(1, S)
    assert e.value.name == "STATE"
    P = synth.make_prompts(m, ("fixed", 4, 16, 12), [32])
    ctx.prefill(torch.from_numpy(P).cuda(), [32], S)
    ctx.decode_frames(4, S)
    with pytest.raises(DualARError) as e:
        ctx.decode_frames(1, S)
    assert e.value.name == "CONTEXT_FULL"
    with pytest.raises(DualARError) as e:
        ctx.decode_frames(1, DualAR.sampling(greedy=False))   # top-p without uniforms
    assert e.value.name == "INVALID_ARG"
    assert ctx.sync() == 0


def test_decode_is_deterministic(tiny):
    DualAR, upload = _dev()
    m, w = tiny
    plen = np.array([20, 33], dtype=np.int32)
    P = torch.from_numpy(synth.make_prompts(m, ("ragged", 1, 1), plen, seed=9)).cuda()
    U = torch.from_numpy(synth.make_uniforms((10, 2, m["num_codebooks"]), seed=9)).cuda()
    dw = upload(m, w)
    outs = []
    for _ in range(2):
        ctx = DualAR(m, dw, max_batch=2, max_seq_len=64)
        S = DualAR.sampling(greedy=False, top_p=0.9)
        f0 = ctx.prefill(P, plen, S, U[0])
        codes, _, taps = ctx.decode_frames(9, S, U[1:], taps=True)
        outs.append((f0.cpu(), codes.cpu(), {k: v.cpu() for k, v in taps.items()}))
        ctx.close()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    for k in outs[0][2]:
        assert torch.equal(outs[0][2][k], outs[1][2][k]), k


def test_multi_frame_call_equals_single_frame_calls(tiny):
    DualAR, upload = _dev()
    m, w = tiny
    plen = np.array([25, 31, 8], dtype=np.int32)
    P = torch.from_numpy(synth.make_prompts(m, ("ragged", 1, 1), plen, seed=4)).cuda()
    dw = upload(m, w)
    S = DualAR.sampling()
    a = DualAR(m, dw, max_batch=3, max_seq_len=64)
    a.prefill(P, plen, S)
    ca, ea, _ = a.decode_frames(7, S)
    b = DualAR(m, dw, max_batch=3, max_seq_len=64)
    b.prefill(P, plen, S)
    cb = torch.cat([b.decode_frames(1, S)[0] for _ in range(7)], dim=1)
    assert torch.equal(ca.cpu(), cb.cpu())


@pytest.mark.parametrize("wdtype", ["f32", "bf16"])
def test_two_contexts_on_two_streams(wdtype):
    # two contexts over the same device weights, each bound to its own stream
    # (default priority), their calls interleaved with no synchronisation in
    # between: each emits exactly what it emits alone.  The library keeps no
    # state shared between contexts.  bf16: batch 3 and 9, so the matrix-core
    # products, the flash-decoding attention and the sampler run on both
    # streams at once.
    DualAR, upload = _dev()
    kw = {} if wdtype == "f32" else dict(weight_dtype="bf16", dim=512, ffn_dim=1024, fast_dim=512, fast_ffn_dim=1024,
                                         n_head=4, n_kv_head=1, head_dim=128, fast_n_head=4, fast_n_kv_head=1,
                                         fast_head_dim=128)
    m = synth.model("tiny", **kw)
    dw = upload(m, synth.make_weights(m, seed=19))
    N = m["num_codebooks"]
    plens = [np.array([30, 12, 41], dtype=np.int32), synth.make_ctx_lengths(9, 1, 300, seed=19)]
    Ps = [torch.from_numpy(synth.make_prompts(m, ("ragged", 1, 1), pl, seed=19 + i)).cuda() for i, pl in enumerate(plens)]
    Us = [torch.from_numpy(synth.make_uniforms((7, len(pl), N), seed=19 + i)).cuda() for i, pl in enumerate(plens)]
    S = DualAR.sampling(greedy=False, top_p=0.9)

    def calls(ctx, i):
        # prefill, then decode calls of 2, 3 and 1 frames
        yield lambda: ctx.prefill(Ps[i], plens[i], S, Us[i][0].contiguous())
        yield lambda: ctx.decode_frames(2, S, Us[i][1:3].contiguous())[0]
        yield lambda: ctx.decode_frames(3, S, Us[i][3:6].contiguous())[0]
        yield lambda: ctx.decode_frames(1, S, Us[i][6:7].contiguous())[0]

    alone = []
    for i in range(2):
        ctx = DualAR(m, dw, max_batch=len(plens[i]), max_seq_len=400)
        alone.append([f().cpu() for f in calls(ctx, i)])
        ctx.close()
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    ctxs = [DualAR(m, dw, max_batch=len(plens[i]), max_seq_len=400, stream=streams[i]) for i in range(2)]
    gens = [calls(ctxs[i], i) for i in range(2)]
    outs = [[], []]
    for _ in range(4):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                outs[i].append(next(gens[i])())
    for i in range(2):
        assert ctxs[i].sync() == 0
    torch.cuda.synchronize()
    for i in range(2):
        for a, b in zip(alone[i], outs[i]):
            assert torch.equal(a, b.cpu()), i
        ctxs[i].close()


# ----------------------------------------------------------------------------
# S2-shaped fast AR alone (batch 1 and 16)
# ----------------------------------------------------------------------------

@pytest.fixture(scope="module")
def s2_fast():
    m = synth.model("s2")
    names = {n for n, _, _ in synth.tensor_specs(m) if n.startswith("fast_")}
    say("[s2-fast] generating fast-AR weights")
    return m, synth.make_weights(m, seed=0, only=names)


@pytest.mark.parametrize("B", [1, 16])
def test_s2_fast_only(s2_fast, B):
    DualAR, upload = _dev()
    m, w = s2_fast
    F = 3
    h, q0 = synth.make_fast_inputs(m, F, B, seed=0)
    # only the fast tensors are real; the slow ones are small placeholders
    full = dict(w)
    dev = upload(m, full)
    dummy = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    for n, _, _ in synth.tensor_specs(m):
        dev.setdefault(n, dummy)
    say(f"[s2-fast] GPU B={B} frames={F}")
    ctx = DualAR(m, dev, max_batch=B, max_seq_len=16)
    codes, taps = ctx.fast_frames(torch.from_numpy(h).cuda(), torch.from_numpy(q0).cuda(), DualAR.sampling(),
                                  taps=True)
    codes = codes.cpu().numpy()
    fl = taps["fast_logits"].cpu().numpy()
    assert ctx.sync() == 0
    ctx.close()
    say("[s2-fast] oracle")
    wf = synth.weights_as_f32(m, w)
    fo = _FastOracle(m, wf)
    agree = 0
    for b in range(B):
        for f in range(F):
            ref = fo.frame(h[f, b], int(q0[f, b]))
            got = codes[b, f].tolist()
            if f == F - 1:
                # pass k's logits depend on q^(0..k-1): compare up to the first differing code
                kd = next((i for i in range(1, m["num_codebooks"]) if got[i] != ref[i]), m["num_codebooks"])
                e = rel_l2(fl[b][:kd], fo.logits[:kd])
                assert e <= REL_L2, (b, e, kd)
            if got != ref:
                k = next(i for i in range(m["num_codebooks"]) if got[i] != ref[i])
                assert k >= 1, (b, f, got, ref)       # q^(0) is an input
                mg = decision_margin(fo.logits[k - 1], True)
                assert not margin_ok(mg, True), (b, f, k, got, ref, mg)
            else:
                agree += 1
    assert agree >= 0.8 * B * F


class _FastOracle:
    """The oracle's fast loop with only the fast weights present."""

    def __init__(self, m, wf):
        # a full oracle whose (unused) slow stack is one tiny layer of zeros
        shell = synth.model("s2", n_layer=1, dim=64, n_head=1, n_kv_head=1, head_dim=64, ffn_dim=64,
                            vocab_size=4160, semantic_begin_id=0, semantic_end_id=4095, end_id=4100)
        spec = {n: s for n, s, _ in synth.tensor_specs(shell)}
        w = {n: (wf[n] if n.startswith("fast_") else np.zeros(s, dtype=np.float32)) for n, s in spec.items()}
        self.o = DualAROracle(shell, w, max_seq=4)
        self.logits = None

    def frame(self, h, q0):
        codes = self.o.fast_frame(h.astype(np.float64), q0, OSampling())
        self.logits = self.o.taps["fast_logits"]
        return codes


# ----------------------------------------------------------------------------
# Full S2-shaped model, short prompt (oracle in seconds), batch 1
# ----------------------------------------------------------------------------

@pytest.fixture(scope="module")
def s2_full():
    m = synth.model("s2")
    say("[s2-full] generating 4.56 B weights")
    w = synth.make_weights(m, seed=0)
    w32 = synth.weights_as_f32(m, w)
    w64 = {k: np.asarray(v, dtype=np.float64) for k, v in w32.items()}   # converted once for every replay
    return m, w, w32, w64


@pytest.mark.timeout(400)
def test_s2_full_fp32_kv_strict(s2_full):
    # fp32 K/V caches: no rounding point between the two sides, so the bar is
    # the plain 2e-3 relative L2 on every tap.
    m, w, w32, w64 = s2_full
    m = dict(m, kv_dtype="f32")
    P = synth.make_prompts(m, ("fixed", 5, 20, 15), [40], seed=0)
    c, worst = run_and_compare(m, w, P, [40], 2, dict(greedy=1), tag="s2-full-kvf32", weights_f32=w32,
                               weights_f64=w64)
    assert c[0] >= 2
    assert max(worst.values()) < 2e-4


@pytest.mark.timeout(900)
@pytest.mark.parametrize("kv", ["f32", "bf16", "f32-semhead"])
def test_s2_full_batch8_matrix_cores(s2_full, kv):
    # Batch 8 of the full S2 shapes: every product on the matrix cores (the
    # tied head as 4-wave x 2-tile blocks, split-K with fused finish + norm
    # across the 36 slow layers), chunked prefill of ragged prompts, top-p on
    # the 4,097 slow candidates.  fp32 K/V keeps the plain 2e-3 bar.  bf16 K/V
    # also takes the matrix-core attention scores and the fp32-oracle floor;
    # it samples greedily, because its ~1e-3 logit drift (the fp32 oracle's
    # own) puts top-p draws over these near-uniform random-weight
    # distributions on near-ties at once, leaving nothing to compare.
    # f32-semhead runs the slow head over the 4,096 semantic rows and the end
    # row only (greedy; the GPU then has no full-vocabulary slow logits).
    m, w, w32, w64 = s2_full
    semhead = kv.endswith("semhead")
    kv = kv.split("-")[0]
    m = dict(m, kv_dtype=kv, semantic_head=int(semhead))
    plen = np.array([24, 9, 17, 3, 24, 12, 20, 6], dtype=np.int32)
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=8)
    if kv == "f32" and not semhead:
        samp, U = dict(greedy=0, temperature=1.0, top_p=0.9), synth.make_uniforms((3, 8, m["num_codebooks"]), seed=8)
    else:
        samp, U = dict(greedy=1), None
    c, worst = run_and_compare(m, w, P, plen, 2, samp, U, tag=f"s2-full-b8-kv{kv}{'-semhead' if semhead else ''}",
                               floor=kv == "bf16", slow_logits_tap=not semhead, weights_f32=w32, weights_f64=w64)
    assert sum(c) >= 8
    if kv == "f32":
        assert max(worst.values()) < 2e-3


# ----------------------------------------------------------------------------
# S2 layer shapes past the stream-K range, up to the largest batch
# ----------------------------------------------------------------------------

def _s2_layers_model(**kw):
    # S2 layer shapes with two slow layers and one fast layer; a 12,288-id
    # vocabulary (4,096 semantic ids) keeps the tied head and the oracle small
    return synth.model("s2", n_layer=2, n_fast_layer=1, vocab_size=12288, text_vocab=8000, end_id=8000,
                       semantic_begin_id=8192, semantic_end_id=8192 + 4095, **kw)


@pytest.fixture(scope="module")
def s2_layers():
    m = _s2_layers_model()
    say("[s2-layers] generating weights")
    w = synth.make_weights(m, seed=12)
    return m, w, synth.weights_as_f32(m, w)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("B,kv", [(96, "f32"), (96, "bf16"), (256, "f32")])
def test_s2_layers_large_batch(s2_layers, B, kv):
    # 96 rows: three activation tiles, so the split-K products with their
    # finish kernels, and the split attention with matrix-core scores (the
    # balanced flash form takes at most 64 rows); the fast layers' depth
    # attention.  256 rows, the largest batch a context holds: the 2-D tile
    # products in decode too, with the attention preparing its own q, k, v.
    # fp32 cache: top-p 0.9, ids compared strictly; bf16 cache: greedy under
    # the rounding-floor bound.  The oracle replays six rows: the first, the
    # last, the shortest and longest prompts and two in between.
    m, w, w32 = s2_layers
    m = dict(m, kv_dtype=kv)
    plen = synth.make_ctx_lengths(B, 1, 60, seed=B)
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=B)
    rows = sorted({0, B - 1, int(np.argmin(plen)), int(np.argmax(plen)), B // 3, (2 * B) // 3})
    F = 3
    if kv == "f32":
        samp, U = dict(greedy=0, temperature=1.0, top_p=0.9), synth.make_uniforms((F + 1, B, m["num_codebooks"]), seed=B)
    else:
        samp, U = dict(greedy=1), None
    c, worst = run_and_compare(m, w, P, plen, F, samp, U, tag=f"s2-layers-B{B}-kv{kv}", floor=kv == "bf16",
                               weights_f32=w32, rows=rows)
    say(f"[s2-layers B={B} kv {kv}] rows {rows}: frames compared {c}")
    assert sum(c) >= len(rows) * (F + 1) // 2
    if kv == "f32":
        assert max(worst.values()) < REL_L2


# ----------------------------------------------------------------------------
# teacher-forced fast AR (the scoring / training form, all pairs at once)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("n", [5, 100])
def test_tiny_fast_teacher_forced(tiny, n):
    # n (hidden state, codes) pairs -> n*N rows through the fast layers with
    # causal attention along depth; slot k >= 1 of each pair must equal the
    # oracle's teacher-forced logits of q^(k) (fp32 weights: 1e-4)
    DualAR, upload = _dev()
    m, w = tiny
    N, C = m["num_codebooks"], m["codebook_size"]
    rng = np.random.default_rng(11)
    h = rng.standard_normal((n, m["dim"])).astype(np.float32)
    codes = rng.integers(0, C, size=(n, N)).astype(np.int32)
    say(f"[tiny-tf] GPU n={n}")
    ctx = DualAR(m, upload(m, w), max_batch=1, max_seq_len=16)
    got = ctx.fast_teacher_forced(torch.from_numpy(h).cuda(), torch.from_numpy(codes).cuda()).cpu().numpy()
    assert ctx.sync() == 0
    ctx.close()
    o = DualAROracle(m, synth.weights_as_f32(m, w), max_seq=8)
    worst = 0.0
    for i in range(n):
        ref = o.fast_teacher_forced(h[i].astype(np.float64), codes[i].tolist())
        e = rel_l2(got[i, 1:], ref)
        worst = max(worst, e)
        assert e <= 1e-4, (i, e)
    say(f"[tiny-tf] worst rel L2 {worst:.2e}")


@pytest.mark.timeout(600)
def test_w4a16_fast_teacher_forced():
    # 4-bit fast layers in the teacher-forced form: 100 pairs x 4 codebooks =
    # 400 rows on the 4-bit 2-D tiles, and 2 pairs (8 rows) on the batched
    # 4-bit GEMV, against the oracle on its own q * scale weights; 5 pairs
    # (20 rows: more than the GEMV takes, fewer than the tiles) are rejected
    # before anything is enqueued
    from oracle import dequant_w4
    from dual_autoregressive_tts_amd import DualARError
    DualAR, upload = _dev()
    m = synth.model("tiny", weight_dtype="bf16", dim=512, ffn_dim=1024, fast_dim=512, fast_ffn_dim=1024, n_head=4,
                    n_kv_head=1, head_dim=128, fast_n_head=4, fast_n_kv_head=1, fast_head_dim=128, w4a16=1,
                    w4_bf16_attn_layers=1)
    w4 = synth.make_w4_model(m, synth.make_weights(m, seed=17))
    wf = dequant_w4(synth.weights_as_f32(m, w4))
    N, C, n = m["num_codebooks"], m["codebook_size"], 100
    rng = np.random.default_rng(13)
    h = torch.from_numpy(rng.standard_normal((n, m["fast_dim"])).astype(np.float32)).cuda()
    codes = torch.from_numpy(rng.integers(0, C, size=(n, N)).astype(np.int32)).cuda()
    say(f"[w4-tf] GPU n={n}")
    ctx = DualAR(m, upload(m, w4), max_batch=1, max_seq_len=16)
    with pytest.raises(DualARError) as e:
        ctx.fast_teacher_forced(h[:5].contiguous(), codes[:5].contiguous())
    assert e.value.name == "INVALID_ARG"
    got = ctx.fast_teacher_forced(h, codes).cpu().numpy()
    got2 = ctx.fast_teacher_forced(h[:2].contiguous(), codes[:2].contiguous()).cpu().numpy()
    assert ctx.sync() == 0
    ctx.close()
    o = DualAROracle(m, wf, max_seq=8)
    worst = 0.0
    for i in range(n):
        ref = o.fast_teacher_forced(h[i].cpu().numpy().astype(np.float64), codes[i].cpu().tolist())
        e2 = rel_l2(got[i, 1:], ref)
        worst = max(worst, e2)
        assert e2 <= REL_L2, (i, e2)
        if i < 2:
            e3 = rel_l2(got2[i, 1:], ref)
            worst = max(worst, e3)
            assert e3 <= REL_L2, (i, e3)
    say(f"[w4-tf] worst rel L2 {worst:.2e}")


@pytest.mark.timeout(600)
def test_s2_fast_teacher_forced(s2_fast):
    # S2 fast shapes in bf16: 32 pairs = 320 rows, so every product runs on
    # the 2-D matrix-core tiles
    DualAR, upload = _dev()
    m, w = s2_fast
    N, C, n = m["num_codebooks"], m["codebook_size"], 32
    rng = np.random.default_rng(12)
    h = rng.standard_normal((n, m["fast_dim"])).astype(np.float32)
    codes = rng.integers(0, C, size=(n, N)).astype(np.int32)
    dev = upload(m, dict(w))
    dummy = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    for name, _, _ in synth.tensor_specs(m):
        dev.setdefault(name, dummy)
    say(f"[s2-tf] GPU n={n}")
    ctx = DualAR(m, dev, max_batch=1, max_seq_len=16)
    got = ctx.fast_teacher_forced(torch.from_numpy(h).cuda(), torch.from_numpy(codes).cuda()).cpu().numpy()
    assert ctx.sync() == 0
    ctx.close()
    say("[s2-tf] oracle")
    fo = _FastOracle(m, synth.weights_as_f32(m, w))
    worst = 0.0
    for i in range(n):
        ref = fo.o.fast_teacher_forced(h[i].astype(np.float64), codes[i].tolist())
        e = rel_l2(got[i, 1:], ref)
        worst = max(worst, e)
        assert e <= REL_L2, (i, e)
    say(f"[s2-tf] worst rel L2 {worst:.2e}")
