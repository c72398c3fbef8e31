"""Reporting helpers against the numbers printed on the page (tests/golden)."""
import json
import os

import pytest

import synth
from dual_autoregressive_tts_amd import reporting as rp

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "s2_page_numbers.json")))


def g(k):
    return GOLD[k]["value"]


def test_codec_rates():
    assert g("sample_rate_hz") / g("hop") == rp.FRAME_RATE
    assert round(rp.FRAME_RATE, 2) == g("frames_per_s")
    assert round(1000.0 / rp.FRAME_RATE, 1) == g("frame_ms")
    assert round(rp.codec_tokens_per_s(rp.FRAME_RATE)) == g("codec_tokens_per_s")
    assert round(rp.rtf(g("fps_batch1")), 2) == g("rtf_batch1")
    assert round(rp.FRAME_RATE / g("rtf_fish")) == g("fps_implied_by_0195")
    assert round(1000.0 / g("fps_batch1"), 1) == g("ms_per_frame_at_63_3")
    assert round(g("context_tokens") / rp.FRAME_RATE / 60, 1) == g("frame_axis_minutes")
    assert round(g("context_tokens") / rp.codec_tokens_per_s(rp.FRAME_RATE)) == g("flattened_audio_s")
    assert round(g("max_new_tokens") / rp.FRAME_RATE, 1) == g("max_new_tokens_audio_s")
    bits = 12 + 9 * 10
    assert bits == g("bits_per_frame")
    assert round(bits * rp.FRAME_RATE / 1000, 2) == g("kbit_per_s")


def test_weights_per_frame_model():
    m = synth.model("s2", fast_qk_norm=0)
    assert round(rp.slow_step_weight_elems(m) / 1e9, 2) == g("slow_step_weights_B")
    assert round(rp.fast_pass_weight_elems(m) / 1e6, 1) == g("fast_pass_weights_M")
    assert round(10 * rp.fast_pass_weight_elems(m) / 1e9, 2) == g("ten_fast_passes_B")
    assert rp.slow_step_weight_elems(m) == g("text_model_params")


def test_frame_bytes_s2():
    m = synth.model("s2")
    fb = rp.frame_bytes(m, [1025])
    # The pages' model, fast QK-norm on: 16,348,828,672 B per frame.  This path
    # skips what fast pass 0 never uses: the fast head (4,096 x 2,560) and its
    # norm (2,560) and, of the last fast layer, Q (4,096 x 2,560), O
    # (2,560 x 4,096), W1/W3/W2 (3 x 9,728 x 2,560), the FFN norm and the q
    # QK-norm gain.
    skipped = 4096 * 2560 + 2560 + 4096 * 2560 + 2560 * 4096 + 3 * 9728 * 2560 + 2560 + 128
    assert fb["slow_weights"] + fb["fast_weights"] == 16348828672 - 2 * skipped
    assert fb["slow_kv"] == 147456 * 1025
    fo = rp.frame_bytes(m, [1, 1], fast_only=True)
    assert fo["fast_weights"] == 10 * 2 * rp.fast_pass_weight_elems(m) - 2 * skipped
    # semantic head: 4,097 of the 155,776 rows
    fs = rp.frame_bytes(m, [1025], semantic_head=True)
    assert fb["slow_weights"] - fs["slow_weights"] == 2 * (155776 - 4097) * 2560


def test_prefill_flops_config5():
    # 16,384 frame positions at batch 4 on the S2 shapes: 4.76e14 linear
    # (2 x 65,536 tokens x 36 x 100.9M weights) + 3.17e14 causal attention
    from dual_autoregressive_tts_amd import reporting
    m = synth.model("s2")
    f = reporting.prefill_flops(m, [16384] * 4)
    per_layer = 2560 * 6144 + 4096 * 2560 + 3 * 2560 * 9728
    assert f["linear"] == 2 * 65536 * 36 * per_layer
    assert f["attention"] == 4 * 128 * 32 * 36 * 4 * (16384 * 16385 // 2)
    assert 4.75e14 < f["linear"] < 4.77e14 and 3.16e14 < f["attention"] < 3.18e14


def test_fast_tf_flops_s2():
    # one teacher-forced row reads the weights of one fast pass: four layers
    # plus the 4,096-row head, 414.2 M on the S2 shapes ([P2], golden file)
    import json
    import os
    from dual_autoregressive_tts_amd import reporting
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "s2_page_numbers.json")))
    m = synth.model("s2")
    f = reporting.fast_tf_flops(m, 819)
    assert f["rows"] == 8190
    per_row = f["linear"] / (2 * f["rows"])
    assert abs(per_row / 1e6 - gold["fast_pass_weights_M"]["value"]) < 0.05
    assert f["attention"] == 4 * 128 * 32 * 4 * 819 * 55


def test_roofline_traffic_follows_the_measured_kernel(monkeypatch):
    # bench.py reports the HBM counters' bytes per launch of the roofline
    # kernel only while gemv_rx_kernel's source is the text they were taken on
    import bench
    t = bench.roofline_traffic()
    assert t is not None
    algo = 2 * 9728 * 2560 * 2 + 4 * 2560 + 4 * 9728          # weights + x + out of one launch
    assert algo <= t <= 1.01 * algo                           # read once: within 1 % of the algorithmic bytes
    src = open(os.path.join(bench.ROOT, "dual_autoregressive_tts_amd", "csrc", "gemv.hip")).read()
    changed = src.replace("// 4. dot products", "// 4. dot products (edited)", 1)
    assert changed != src
    real_open = open

    def fake_open(path, *a, **k):
        if str(path).endswith(os.path.join("csrc", "gemv.hip")):
            import io
            return io.StringIO(changed)
        return real_open(path, *a, **k)

    monkeypatch.setattr("builtins.open", fake_open)
    assert bench.roofline_traffic() is None


def test_w4_roofline_traffic_reads_weights_once():
    # the 4-bit W1|W3 kernel's counters: 4-bit weights, bf16 scales, x, out
    import bench
    t = bench.roofline_traffic("gemv_w4_kernel")
    assert t is not None
    algo = 2 * 9728 * 2560 // 2 + 2 * 9728 * 20 * 2 + 4 * 2560 + 4 * 9728
    assert algo == 25731072
    assert algo <= t <= 1.02 * algo
    assert bench.roofline_traffic("no_such_kernel") is None


def test_batch32_roofline_traffic_counts_the_stream_k_partials():
    # batch 32: the stream-K W1|W3 product and its finish, timed together.
    # Weights are read once (HBM bytes of the product >= the weights); the
    # partial tiles the product writes are what its finish reads; the finish
    # writes the SwiGLU output as three bf16 planes [3][32][9728]
    import bench
    p, f = bench.roofline_traffic("mfma_skw_kernel"), bench.roofline_traffic("sk_finish_kernel")
    assert p is not None and f is not None and bench.b32_traffic() == p + f
    weights = 2 * 9728 * 2560 * 2
    c = bench.ROOFLINE_COUNTERS
    wrote = c["mfma_skw_kernel"]["write_kib"] * 1024 * bench._WRITE_SCALE
    read_back = c["sk_finish_kernel"]["fetch_kib"] * 1024 * bench._FETCH_SCALE
    assert weights <= p - wrote <= 1.1 * weights
    assert abs(read_back - wrote) <= 0.02 * wrote
    assert abs(c["sk_finish_kernel"]["write_kib"] * 1024 - 3 * 32 * 9728 * 2) <= 4096


def test_w4_frame_bytes_by_enumeration():
    # the 4-bit byte change of a frame-step against a direct count over the
    # model's tensors: every 4-bit matrix costs rows * (K/2 + K/128 * 2) bytes
    # per read instead of rows * K * 2; slow matrices are read once, fast
    # matrices N-1 times plus pass 0 (the last layer's K and V rows only)
    m = synth.model("tiny", weight_dtype="bf16", dim=512, ffn_dim=1024, fast_dim=512, fast_ffn_dim=1024,
                    n_head=4, n_kv_head=1, head_dim=128, fast_n_head=4, fast_n_kv_head=1, fast_head_dim=128,
                    w4a16=1, w4_bf16_attn_layers=1)
    names = set(synth.w4_names(m))
    shapes = {n: s for n, s, _ in synth.tensor_specs(m)}
    N, nf = m["num_codebooks"], m["n_fast_layer"]
    want = 0
    for n in names:
        rows, K = shapes[n]
        per = rows * (K // 2 + K // 128 * 2) - rows * K * 2
        if n.startswith("fast_layers."):
            last = int(n.split(".")[1]) == nf - 1
            want += per * ((N - 1) + (0 if last and n.rsplit(".", 1)[1] not in ("wk", "wv") else 1))
        else:
            want += per
    b0 = rp.frame_bytes(m, [40])["total"]
    b4 = rp.frame_bytes(m, [40], w4_names=sorted(names))
    assert b4["w4_delta"] == want and b4["total"] == b0 + want


def test_bench_host_info_names_the_cpu_and_blas():
    # cpu_baseline records the host it ran on: logical CPUs, CPU model, numpy
    # and its BLAS thread pool
    import bench
    h = bench.host_info()
    assert h["nproc"] == os.cpu_count() and h["numpy"]
    assert h["cpu_model"] is None or isinstance(h["cpu_model"], str)
    assert h["blas"] is None or h["blas"]["threads"] >= 1


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr
