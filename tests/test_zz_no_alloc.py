"""dualar_create_static through the C ABI: a context whose workspace is the
library's static device array must give the same codes and taps, bit for
bit, as a context over a caller-allocated workspace, on two calls in a row
(the second with a smaller batch, prompt and context, so the array still
holds the first call's contents)."""
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


def _decode(DualAR, m, dev, plen, frames, max_seq, pc, samp, U, static):
    P = torch.from_numpy(synth.make_prompts(m, ("ragged", 1, 1), plen, seed=31)).cuda()
    ctx = DualAR(m, dev, max_batch=len(plen), max_seq_len=max_seq, prefill_chunk=pc, static_workspace=static)
    assert (ctx.workspace is None) == static
    S = DualAR.sampling(min_frames=1 << 30, **samp)
    f0, t0 = ctx.prefill(P, plen, S, None if U is None else U[0], taps=True)
    codes, emitted, taps = ctx.decode_frames(frames, S, None if U is None else U[1:1 + frames], taps=True)
    assert ctx.sync() == 0
    out = (f0.cpu().numpy(), codes.cpu().numpy(), emitted.cpu().numpy(),
           {k: v.cpu().numpy() for k, v in t0.items()}, {k: v.cpu().numpy() for k, v in taps.items()})
    ctx.close()
    return out


def _same(a, b):
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])
    for i in (3, 4):
        for k in a[i]:
            assert np.array_equal(a[i][k], b[i][k]), k


@pytest.mark.parametrize("model", ["tiny", "bf16"])
def test_static_workspace_matches_allocated_workspace(model):
    DualAR, upload = _dev()
    if model == "tiny":
        m = synth.model("tiny")
        samp, U1, U2 = dict(greedy=1), None, None
    else:   # batched matrix-core path, top-p
        m = synth.model("tiny", weight_dtype="bf16", dim=512, ffn_dim=1024, fast_dim=512, fast_ffn_dim=1024,
                        n_head=8, n_kv_head=2, fast_n_head=8, fast_n_kv_head=2)
        samp = dict(greedy=0, temperature=1.0, top_p=0.9)
        U1 = torch.from_numpy(synth.make_uniforms((7, 5, m["num_codebooks"]), seed=31)).cuda()
        U2 = torch.from_numpy(synth.make_uniforms((5, 2, m["num_codebooks"]), seed=32)).cuda()
    dev = upload(m, synth.make_weights(m, seed=3))
    # first call: 5 sequences, prompts up to 60, 6 frames; second call: 2
    # sequences, prompts up to 20, 4 frames, a smaller context and chunk
    cases = [(np.array([60, 7, 33, 1, 45], dtype=np.int32), 6, 72, 32, U1),
             (np.array([20, 9], dtype=np.int32), 4, 28, 16, U2)]
    for i, (plen, frames, max_seq, pc, U) in enumerate(cases):
        say(f"[no-alloc-{model}] call {i}: B={len(plen)} prompts {plen.tolist()} frames {frames}")
        ref = _decode(DualAR, m, dev, plen, frames, max_seq, pc, samp, U, static=False)
        got = _decode(DualAR, m, dev, plen, frames, max_seq, pc, samp, U, static=True)
        _same(got, ref)
        assert (ref[1] != -1).all()
    say(f"[no-alloc-{model}] static workspace: codes and taps bit-identical on both calls")


def test_static_workspace_rejects_large_configs():
    from dual_autoregressive_tts_amd import DualARError
    DualAR, upload = _dev()
    m = synth.model("tiny")
    dev = upload(m, synth.make_weights(m, seed=3))
    with pytest.raises(DualARError) as e:
        DualAR(m, dev, max_batch=8, max_seq_len=4096, static_workspace=True)
    assert e.value.name == "WORKSPACE"
