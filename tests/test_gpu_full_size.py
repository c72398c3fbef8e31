"""The benchmark configurations at their full sizes, through the C ABI.

Against the oracle (the float64 CPU decoder replays whole sequences):
  * s2_b1: the full S2-shaped model, bf16 K/V cache, the bench's 1,024-token
    three-segment prompt, 8 greedy frames after frame 0, every tap and id;
  * s2_b32: the bench's batch of 32 ragged prompts (741..4,025 positions),
    top-p 0.9 with the bench's uniforms; the oracle replays the shortest and
    the longest sequence -- on the bf16 cache (frame 0's taps, then frames up
    to the first draw that differs within the logits' reach) and on an fp32
    cache (the strict bound, ids for at least half of the frames);
  * s2_prefill: the bench's launch configuration (4 sequences, 2,048
    positions per sequence per step, 8,192 rows on the 2-D matrix-core
    tiles) on 4,096-position all-frame prompts; the oracle replays one
    sequence: frame 0 and one decode frame.
Sampled outputs the oracle computes one by one: the teacher-forced fast AR
over 819 pairs.  Properties that hold exactly at any size: every product,
norm, split, attention and sampling step works on one sequence (one row) at
a time with a reduction order that does not depend on the others, so a
sequence's results are bit-identical whatever the other sequences hold,
whatever the prefill step size, and from one run to the next (checked at
the full 32-sequence batch and the 4 x 16,384-position prefill).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import DualAROracle
from tests.parity import REL_L2, rel_l2, say
from tests.test_gpu_parity import run_and_compare

pytestmark = pytest.mark.gpu


def _dev():
    from dual_autoregressive_tts_amd import DualAR, load_library
    from dual_autoregressive_tts_amd.binding import upload_weights
    load_library()
    return DualAR, upload_weights


@pytest.fixture(scope="module")
def s2_weights():
    m = synth.model("s2")
    say("[full] generating 4.56 B weights")
    return m, synth.make_weights(m, seed=0)


@pytest.fixture(scope="module")
def s2_oracle_weights(s2_weights):
    """The oracle's weights converted once: (float64, float32) dicts."""
    m, w = s2_weights
    say("[full] oracle weights (float32, float64)")
    w32 = synth.weights_as_f32(m, w)
    w64 = {k: np.asarray(v, dtype=np.float64) for k, v in w32.items()}
    return w64, w32


def _half(n_frames):
    return (n_frames + 2) // 2       # at least half of frame 0 + n_frames


@pytest.mark.timeout(900)
@pytest.mark.parametrize("kv", ["bf16", "f32"])
def test_s2_b1_bench_config_vs_oracle(s2_weights, s2_oracle_weights, kv):
    # the s2_b1 bench line: full S2 shapes, the 1,024-token three-segment
    # prompt, greedy, <|im_end|> held back as in the bench; bf16 K/V (the
    # bench's cache: bound relative to the fp32 rounding floor) and fp32 K/V
    # (the plain 2e-3 bound)
    m, w = s2_weights
    w64, w32 = s2_oracle_weights
    m = dict(m, kv_dtype=kv)
    wl = synth.WORKLOADS["s2_b1"]
    plen = synth.prompt_lengths(wl, seed=0)
    P = synth.make_prompts(m, wl["prompt"], plen, seed=0)
    F = 8
    c, worst = run_and_compare(m, w, P, plen, F, dict(greedy=1), min_frames=1 << 30, tag=f"s2-b1-bench-kv{kv}",
                               floor=kv == "bf16", weights_f32=w32, weights_f64=w64)
    assert c[0] >= _half(F), f"s2_b1 kv {kv}: {c[0]} of {F + 1} frames compared (need {_half(F)})"
    if kv == "f32":
        assert max(worst.values()) < REL_L2


@pytest.mark.timeout(900)
@pytest.mark.parametrize("kv", ["bf16", "f32"])
def test_s2_b32_bench_config_rows_vs_oracle(s2_weights, s2_oracle_weights, kv):
    # the s2_b32 bench line: 32 ragged prompts, top-p 0.9 from the bench's
    # seeded uniforms; the oracle replays the shortest and the longest row.
    # bf16 cache: the fp32 rounding floor moves logits by ~1e-3, which swaps
    # neighbours in the top-p order (the near-uniform candidates of random
    # weights sit ~1e-3 apart), so the draws differ within reach after a
    # frame or two; frame 0's taps (the batched ragged prefill up to 4,025
    # positions) are always compared.  fp32 cache: the strict bound, and the
    # ids must match for at least half of the frames.
    m, w = s2_weights
    w64, w32 = s2_oracle_weights
    m = dict(m, kv_dtype=kv)
    wl = synth.WORKLOADS["s2_b32"]
    plen = synth.prompt_lengths(wl, seed=0)
    P = synth.make_prompts(m, wl["prompt"], plen, seed=0)
    F = 4
    U = synth.make_uniforms((1 + F, len(plen), m["num_codebooks"]), seed=0)
    rows = [int(np.argmin(plen)), int(np.argmax(plen))]
    stats = {}
    c, worst = run_and_compare(m, w, P, plen, F, dict(wl["sampling"]), U, min_frames=1 << 30,
                               tag=f"s2-b32-bench-kv{kv}", floor=kv == "bf16", weights_f32=w32, weights_f64=w64,
                               rows=rows, stats=stats)
    say(f"[s2-b32-kv{kv}] rows {rows} (prompts {[int(plen[r]) for r in rows]}): frames compared {c}")
    assert all(t >= 1 for t in stats["taps_compared"]), stats
    if kv == "f32":
        assert min(c) >= _half(F), f"s2_b32 fp32 cache: rows {rows} compared {c} of {F + 1} frames"
        assert max(worst.values()) < REL_L2


@pytest.mark.timeout(900)
def test_s2_prefill_bench_launch_vs_oracle(s2_weights, s2_oracle_weights):
    # the s2_prefill bench line's launch configuration (4 sequences x 2,048
    # positions per step = 8,192 rows on the 2-D tiles, matrix-core causal
    # attention over the growing cache) on 4,096-position all-frame prompts
    m, w = s2_weights
    w64, w32 = s2_oracle_weights
    wl = synth.WORKLOADS["s2_prefill"]
    plen = np.full(4, 4096, dtype=np.int32)
    P = synth.make_prompts(m, ("frames", 4096), plen, seed=0)
    F = 1
    c, worst = run_and_compare(m, w, P, plen, F, dict(wl["sampling"]), min_frames=1 << 30, prefill_chunk=2048,
                               tag="s2-prefill-4096", floor=True, weights_f32=w32, weights_f64=w64, rows=[0])
    assert c[0] >= _half(F), f"s2_prefill: {c[0]} of {F + 1} frames compared"


@pytest.mark.timeout(600)
def test_teacher_forced_819_pairs_sampled(s2_weights):
    # the s2_fast_tf bench configuration: 819 pairs = 8,190 rows; six pairs
    # spread over the row range against the oracle
    DualAR, upload = _dev()
    m, w = s2_weights
    N, C, n = m["num_codebooks"], m["codebook_size"], 819
    rng = np.random.default_rng(0)
    h = rng.standard_normal((n, m["fast_dim"])).astype(np.float32)
    codes = rng.integers(0, C, size=(n, N)).astype(np.int32)
    ctx = DualAR(m, upload(m, w), max_batch=2, max_seq_len=16)
    got = ctx.fast_teacher_forced(torch.from_numpy(h).cuda(), torch.from_numpy(codes).cuda()).cpu().numpy()
    assert ctx.sync() == 0
    ctx.close()
    torch.cuda.empty_cache()
    shell = synth.model("s2", n_layer=1, dim=64, n_head=1, n_kv_head=1, head_dim=64, ffn_dim=64,
                        vocab_size=4160, semantic_begin_id=0, semantic_end_id=4095, end_id=4100)
    spec = {nm: sh for nm, sh, _ in synth.tensor_specs(shell)}
    fast = {nm: synth.weights_as_f32(m, {nm: w[nm]})[nm] for nm in spec if nm.startswith("fast_")}
    wf = {nm: (fast[nm] if nm in fast else np.zeros(sh, dtype=np.float32)) for nm, sh in spec.items()}
    o = DualAROracle(shell, wf, max_seq=4)
    for i in (0, 1, 255, 409, 700, 818):
        ref = o.fast_teacher_forced(h[i].astype(np.float64), codes[i].tolist())
        e = rel_l2(got[i, 1:], ref)
        say(f"[full-tf] pair {i}: rel L2 {e:.2e}")
        assert e <= REL_L2, (i, e)


def _decode(ctx, DualAR, tok, plen, U, frames):
    S = DualAR.sampling(greedy=False, temperature=1.0, top_p=0.9, min_frames=1 << 30)
    f0, t0 = ctx.prefill(tok, plen, S, U[0], taps=("slow_hidden",))
    out = [f0.cpu().numpy()]
    taps = t0["slow_hidden"].cpu().numpy()
    for f in range(frames):
        codes, _, t = ctx.decode_frames(1, S, U[1 + f:2 + f], taps=("slow_hidden",))
        out.append(codes[:, 0].cpu().numpy())
        taps = t["slow_hidden"].cpu().numpy()
    assert ctx.sync() == 0
    return np.stack(out, 1), taps


@pytest.mark.timeout(900)
def test_batch32_isolation_and_determinism(s2_weights):
    # the s2_b32 bench configuration (ragged prompts 512..4,096, top-p 0.9):
    # two identical runs agree bit for bit, and changing one sequence's
    # prompt leaves every other sequence's codes and hidden state unchanged
    DualAR, upload = _dev()
    m, w = s2_weights
    wl = synth.WORKLOADS["s2_b32"]
    B, frames = 32, 3
    plen = synth.prompt_lengths(wl, seed=0)
    P = synth.make_prompts(m, wl["prompt"], plen, seed=0)
    U = torch.from_numpy(synth.make_uniforms((1 + frames, B, m["num_codebooks"]), seed=0)).cuda()
    dev = upload(m, w)
    ctx = DualAR(m, dev, max_batch=B, max_seq_len=int(plen.max()) + frames + 2)
    say(f"[full-b32] prompts {int(plen.min())}..{int(plen.max())}")
    c1, h1 = _decode(ctx, DualAR, torch.from_numpy(P).cuda(), plen, U, frames)
    c2, h2 = _decode(ctx, DualAR, torch.from_numpy(P).cuda(), plen, U, frames)
    assert np.array_equal(c1, c2) and np.array_equal(h1, h2), "two runs differ"
    P3 = P.copy()
    j = 5
    t = int(plen[j]) - 10                     # a late (text) position of sequence j's prompt
    P3[j, 0, t] = (int(P3[j, 0, t]) + 1) % m["text_vocab"]
    c3, h3 = _decode(ctx, DualAR, torch.from_numpy(P3).cuda(), plen, U, frames)
    ctx.close()
    others = [b for b in range(B) if b != j]
    assert np.array_equal(c3[others], c1[others]), "another sequence's codes changed"
    assert np.array_equal(h3[others], h1[others]), "another sequence's hidden state changed"
    assert not np.array_equal(h3[j], h1[j])   # the changed prompt does reach its own sequence
    say(f"[full-b32] identical over {frames + 1} frames; sequence {j} alone changed")


@pytest.mark.timeout(900)
def test_prefill_16384_chunking_invariance(s2_weights):
    # the s2_prefill configuration (4 x 16,384 frame positions): walking the
    # prompts 4,096 or 2,048 positions per step gives frame 0 and its hidden
    # state, slow logits and fast logits bit for bit (a row's arithmetic does
    # not depend on which other rows share its step)
    DualAR, upload = _dev()
    m, w = s2_weights
    wl = synth.WORKLOADS["s2_prefill"]
    plen = synth.prompt_lengths(wl, seed=0)
    P = torch.from_numpy(synth.make_prompts(m, wl["prompt"], plen, seed=0)).cuda()
    dev = upload(m, w)
    res = []
    for pc in (4096, 2048):
        ctx = DualAR(m, dev, max_batch=4, max_seq_len=int(plen.max()) + 4, prefill_chunk=pc)
        f0, t = ctx.prefill(P, plen, DualAR.sampling(), taps=True)
        assert ctx.sync() == 0
        res.append((f0.cpu().numpy(), {k: v.cpu().numpy() for k, v in t.items()}))
        ctx.close()
        torch.cuda.empty_cache()
    (fa, ta), (fb, tb) = res
    assert np.array_equal(fa, fb)
    for k in ta:
        assert np.array_equal(ta[k], tb[k]), k
    say(f"[full-prefill] frame 0 {fa[:, :3].tolist()} identical for 4,096- and 2,048-position steps")
