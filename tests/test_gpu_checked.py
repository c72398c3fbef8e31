"""The checked build (libdualar_checked.so, kernels compiled with
DUALAR_DEVICE_CHECKS) against the normal build, through the C ABI.

The checked kernels hold every cache position they append at or read up to
below max_seq_len and every partial-sum slot below its buffer's slot count,
latching a status bit instead of touching memory outside the buffer.  Each
case runs a prefill and a few decode frames on both builds with the same
device weights, inputs and draws; the checked build's dualar_sync must
report no failed check, and both builds must emit the same ids and the same
taps (the checks change no arithmetic).

Cases, chosen to reach every kernel that carries a check:
  * the small fp32 model, batch 3, ragged prompts in prefill steps of 4
    positions, top-p: the vector split attention and its merge, the vector
    prefill attention and the cache append;
  * S2 layer shapes (two slow layers, one fast layer, a reduced vocabulary),
    bf16 weights and cache:
      - batch 1, a 300-position prompt, greedy: the 8-wave split attention,
        the merge inside the O product, the fast attention inside the O
        product, the 2-D tile products and the matrix-core prefill attention;
      - batch 6, ragged prompts, top-p 0.9: the stream-K products with the
        attention preparation in their finish, the flash-decoding attention
        and its merge, the depth attention of the fast layers;
      - batch 3 with an fp32 cache: the split form with matrix-core scores
        off and its merge.
"""
import numpy as np
import pytest
import torch

import synth
from tests.parity import rel_l2, say

pytestmark = pytest.mark.gpu


def _run(lib, m, dw, P, plen, frames, samp, U, prefill_chunk=0):
    from dual_autoregressive_tts_amd import DualAR
    B = len(plen)
    ctx = DualAR(m, dw, max_batch=B, max_seq_len=int(max(plen)) + frames + 2, prefill_chunk=prefill_chunk,
                 library=lib)
    S = DualAR.sampling(**samp)
    tok = torch.from_numpy(np.ascontiguousarray(P)).cuda()
    Ug = None if U is None else torch.from_numpy(np.ascontiguousarray(U)).cuda()
    f0 = ctx.prefill(tok, plen, S, None if Ug is None else Ug[0].contiguous())
    codes, _, taps = ctx.decode_frames(frames, S, None if Ug is None else Ug[1:].contiguous(), taps=True)
    out = (f0.cpu().numpy(), codes.cpu().numpy(), {k: v.cpu().numpy() for k, v in taps.items()})
    status = ctx.sync()            # raises DualARError(DEVICE_INDEX) on a failed check
    ctx.close()
    return out, status


def _compare(m, w, P, plen, frames, samp, U=None, prefill_chunk=0, tag=""):
    from dual_autoregressive_tts_amd.binding import CHECKED_LIB_PATH, LIB_PATH, upload_weights
    dw = upload_weights(m, w)
    say(f"[checked {tag}] normal build")
    (f0a, ca, ta), sa = _run(LIB_PATH, m, dw, P, plen, frames, samp, U, prefill_chunk)
    say(f"[checked {tag}] checked build")
    (f0b, cb, tb), sb = _run(CHECKED_LIB_PATH, m, dw, P, plen, frames, samp, U, prefill_chunk)
    del dw
    torch.cuda.empty_cache()
    assert sa == 0 and sb == 0
    np.testing.assert_array_equal(f0a, f0b)
    np.testing.assert_array_equal(ca, cb)
    for k in ta:
        e = rel_l2(tb[k], ta[k])
        say(f"[checked {tag}] tap {k}: rel L2 {e:.1e}")
        assert e <= 1e-6, (k, e)


def _s2_layers(**kw):
    # S2 layer shapes; a 12,288-id vocabulary keeps the tied head small
    return synth.model("s2", n_layer=2, n_fast_layer=1, vocab_size=12288, text_vocab=8000, end_id=8000,
                       semantic_begin_id=8192, semantic_end_id=8192 + 4095, **kw)


@pytest.fixture(scope="module")
def s2_layer_weights():
    m = _s2_layers()
    say("[checked] generating S2-layer weights")
    return synth.make_weights(m, seed=3)


def test_checked_build_tiny():
    m = synth.model("tiny")
    w = synth.make_weights(m, seed=1)
    plen = np.array([20, 9, 14], dtype=np.int32)
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=1)
    U = synth.make_uniforms((6, 3, m["num_codebooks"]), seed=1)
    _compare(m, w, P, plen, 5, dict(greedy=0, temperature=1.0, top_p=0.9), U, prefill_chunk=4, tag="tiny")


@pytest.mark.timeout(300)
def test_checked_build_s2_batch1(s2_layer_weights):
    m = _s2_layers(kv_dtype="bf16")
    plen = np.array([300], dtype=np.int32)
    P = synth.make_prompts(m, ("fixed", 40, 150, 110), plen, seed=2)
    _compare(m, s2_layer_weights, P, plen, 4, dict(greedy=1, min_frames=1 << 20), tag="s2-b1")


@pytest.mark.timeout(300)
def test_checked_build_s2_batch6(s2_layer_weights):
    m = _s2_layers(kv_dtype="bf16")
    plen = np.array([300, 128, 77, 260, 33, 190], dtype=np.int32)
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=4)
    U = synth.make_uniforms((4, 6, m["num_codebooks"]), seed=4)
    _compare(m, s2_layer_weights, P, plen, 3, dict(greedy=0, temperature=1.0, top_p=0.9), U, tag="s2-b6")


@pytest.mark.timeout(300)
def test_checked_build_s2_fp32_cache(s2_layer_weights):
    m = _s2_layers(kv_dtype="f32")
    plen = np.array([150, 61, 222], dtype=np.int32)
    P = synth.make_prompts(m, ("ragged", 1, 1), plen, seed=5)
    _compare(m, s2_layer_weights, P, plen, 3, dict(greedy=1), tag="s2-b3-f32kv")
