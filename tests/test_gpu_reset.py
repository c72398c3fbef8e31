"""dualar_reset through the C ABI: retiring sequences of a batch.

A retired slot ends as a sequence that sampled <|im_end|> does ([P1]
"Inference Pipeline", "generate: Full Sequence Generation"): its later code
rows are -1 and its emitted-frame count is 0, while every other sequence's
codes and taps stay bit-identical to a run without the reset (each kernel
works on one row with a reduction order that does not depend on the others).
"""
import numpy as np
import pytest
import torch

import synth
from tests.parity import say

pytestmark = pytest.mark.gpu


def _dev():
    from dual_autoregressive_tts_amd import DualAR, load_library
    from dual_autoregressive_tts_amd.binding import upload_weights
    load_library()
    return DualAR, upload_weights


def _run(m, dev, P, plen, U, S, before, after, reset=None, bad_resets=()):
    """Prefill, `before` frames, optional reset, `after` frames; returns the
    code rows [B][1 + before + after][N+1], n_emitted and the last taps."""
    from dual_autoregressive_tts_amd import DualARError
    DualAR, _ = _dev()
    B = len(plen)
    ctx = DualAR(m, dev, max_batch=B, max_seq_len=int(max(plen)) + before + after + 2)
    f0 = ctx.prefill(P, plen, S, None if U is None else U[0])
    c1, _, _ = ctx.decode_frames(before, S, None if U is None else U[1:1 + before])
    for ids in bad_resets:   # rejected on the host: nothing changes
        with pytest.raises(DualARError) as e:
            ctx.reset(ids)
        assert e.value.name == "INVALID_ARG", ids
    if reset is not None:
        ctx.reset(reset)
    c2, emitted, taps = ctx.decode_frames(after, S, None if U is None else U[1 + before:1 + before + after],
                                          taps=True)
    assert ctx.sync() == 0
    codes = torch.cat([f0[:, None, :], c1, c2], dim=1).cpu().numpy()
    out = codes, emitted.cpu().numpy(), {k: v.cpu().numpy() for k, v in taps.items()}
    ctx.close()
    return out


def _check(m, w, plen, samp, U=None, retire=(1,), before=3, after=5, tag=""):
    DualAR, upload = _dev()
    B, N = len(plen), m["num_codebooks"]
    P = torch.from_numpy(synth.make_prompts(m, ("ragged", 1, 1), plen, seed=21)).cuda()
    Ud = None if U is None else torch.from_numpy(U).cuda()
    dev = upload(m, w)
    S = DualAR.sampling(min_frames=1 << 30, **samp)
    say(f"[reset-{tag}] B={B} retire {list(retire)} after {before} frames")
    ref = _run(m, dev, P, plen, Ud, S, before, after)
    got = _run(m, dev, P, plen, Ud, S, before, after, reset=list(retire),
               bad_resets=([B], [-1], [0] * (B + 1)))
    keep = [b for b in range(B) if b not in retire]
    assert np.array_equal(got[0][keep], ref[0][keep]), "another sequence's codes changed"
    for k in ref[2]:
        assert np.array_equal(got[2][k][keep], ref[2][k][keep]), ("another sequence's tap changed", k)
    assert np.array_equal(got[0][list(retire), :1 + before], ref[0][list(retire), :1 + before])
    assert (got[0][list(retire), 1 + before:] == -1).all(), "a retired slot emitted a frame"
    assert np.array_equal(got[1][keep], ref[1][keep])
    assert (got[1][list(retire)] == 0).all(), got[1]
    assert (ref[0][:, 1 + before:] != -1).all()   # without the reset every slot kept decoding
    say(f"[reset-{tag}] other sequences bit-identical; retired slots emit -1")
    return N


def test_reset_tiny_fp32_vector_path():
    m = synth.model("tiny")
    _check(m, synth.make_weights(m, seed=0), np.array([20, 33, 9], dtype=np.int32), dict(greedy=1),
           retire=(1,), tag="tiny")


def test_reset_bf16_matrix_core_path_top_p():
    # 11 sequences: stream-K products, batched attention, top-p draws
    m = synth.model("tiny", weight_dtype="bf16", dim=512, ffn_dim=1024, fast_dim=512, fast_ffn_dim=1024,
                    n_head=8, n_kv_head=2, fast_n_head=8, fast_n_kv_head=2)
    plen = synth.make_ctx_lengths(11, 1, 40, seed=11)
    U = synth.make_uniforms((9, 11, m["num_codebooks"]), seed=11)
    _check(m, synth.make_weights(m, seed=2), plen, dict(greedy=0, temperature=1.0, top_p=0.9), U,
           retire=(0, 7, 10), tag="bf16-b11")


def test_reset_batch1_s2_heads():
    # batch 1 with the S2 head shape (split attention merged in the O product):
    # retiring the only sequence leaves nothing to emit and no device fault
    DualAR, upload = _dev()
    m = synth.model("tiny", weight_dtype="bf16", dim=512, ffn_dim=1024, fast_dim=512, fast_ffn_dim=1024,
                    n_head=32, n_kv_head=8, head_dim=128, fast_n_head=32, fast_n_kv_head=8, fast_head_dim=128)
    w = synth.make_weights(m, seed=8)
    plen = np.array([300], dtype=np.int32)
    P = torch.from_numpy(synth.make_prompts(m, ("ragged", 1, 1), plen, seed=8)).cuda()
    dev = upload(m, w)
    S = DualAR.sampling()
    codes, emitted, _ = _run(m, dev, P, plen, None, S, 2, 3, reset=[0])
    assert (codes[0, :3] != -1).all() and (codes[0, 3:] == -1).all()
    assert emitted[0] == 0


def test_reset_state_errors():
    from dual_autoregressive_tts_amd import DualARError
    DualAR, upload = _dev()
    m = synth.model("tiny")
    ctx = DualAR(m, upload(m, synth.make_weights(m, seed=0)), max_batch=2, max_seq_len=40)
    with pytest.raises(DualARError) as e:
        ctx.reset([0])
    assert e.value.name == "STATE"
    ctx.close()
