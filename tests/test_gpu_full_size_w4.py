"""The W4A16 bench configuration at its full size against the oracle.

`bench.py --workload s2_b1_w4`: the full S2-shaped model with every linear
matrix as 4-bit groups of 128 inputs with bf16 scales, except the attention
of the last 12 slow layers (kept bf16, as the W4A16 model card describes),
batch 1, the bench's 1,024-token three-segment prompt prefilled in one step
of 1,024 positions (the 4-bit products on the matrix-core 2-D tiles), greedy,
bf16 K/V cache; and, with an fp32 cache, also one position per step (the
4-bit GEMVs).  The oracle runs the same steps in float64
on its own dequantised weights (q * scale).  With the bench's bf16 cache the
taps are bound relative to the fp32 rounding floor, as for the bf16 bench
line; that floor (~1e-3 on the logits) reaches the near-ties of these
random-weight logits within a few frames, so frame 0 and at least one
decode frame must match whole.  With an fp32 cache the plain 2e-3 bound
holds and at least half of the frames must match whole.
Kept in a module of its own, so that the other full-size modules' weight
copies are released before this one builds its own.
"""
import numpy as np
import pytest

import synth
from tests.parity import REL_L2, say
from tests.test_gpu_parity import run_and_compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4_model():
    from oracle import dequant_w4
    m = dict(synth.model("s2"), w4a16=1)
    say("[full-w4] generating 4.56 B weights, quantising to 4-bit groups")
    w4 = synth.make_w4_model(m, synth.make_weights(m, seed=0))
    say(f"[full-w4] {len(synth.w4_names(m))} matrices as 4-bit groups; oracle weights")
    wf = dequant_w4(synth.weights_as_f32(m, w4))            # the oracle's own q * scale
    w64 = {k: np.asarray(v, dtype=np.float64) for k, v in wf.items()}
    return m, w4, wf, w64


@pytest.mark.timeout(900)
@pytest.mark.parametrize("kv,pc", [("bf16", 0), ("f32", 0), ("f32", 1)])
def test_s2_b1_w4_bench_config_vs_oracle(w4_model, kv, pc):
    m, w4, wf, w64 = w4_model
    m = dict(m, kv_dtype=kv)
    wl = synth.WORKLOADS["s2_b1"]
    plen = synth.prompt_lengths(wl, seed=0)
    P = synth.make_prompts(m, wl["prompt"], plen, seed=0)
    F = 4
    c, worst = run_and_compare(m, w4, P, plen, F, dict(greedy=1), min_frames=1 << 30,
                               tag=f"s2-b1-w4-bench-kv{kv}-pc{pc}", floor=kv == "bf16", weights_f32=wf,
                               weights_f64=w64, prefill_chunk=pc)
    say(f"[full-w4 kv {kv} pc {pc}] frames compared {c}; worst {worst}")
    if kv == "bf16":
        assert c[0] >= 2, f"s2_b1_w4 bf16 cache: {c[0]} of {F + 1} frames compared"
    else:
        assert c[0] >= (F + 2) // 2, f"s2_b1_w4 fp32 cache: {c[0]} of {F + 1} frames compared"
        assert max(worst.values()) < REL_L2
