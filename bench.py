"""Benchmark: Dual-AR frames/s on one MI355X, with the HBM roofline of the
dominant kernel and the CPU oracle timed beside it.

    python bench.py [--steps K] [--warmup W] [--reps R] [--workload s2_b1|s2_b32|s2_prefill|s2_fast_tf|fast_s2|
                    fast_s2_b16|tiny_b1|s2_b1_w4|s2_b4_w4|s2_b8_w4] [--semantic-head] [--ras] [--no-batch32]

A step is one decode frame of the whole hot path (fusion, slow pass, biased
sample, ten fast passes with their samples) over one batch.  Inputs are
seeded synthetic data of the workload's shape, resident in HBM before the
timed region.  W untimed warm-up steps, then R repetitions of exactly K
timed steps (events on the context's stream, synchronised on both sides);
the median repetition is reported.  The default workload (s2_b1) also times
the batch-32 workload in the same process and nests its line under
"batch32" (the metric is quoted at batch 1 and 32).  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "Dual-AR frames/sec (codec tokens/s) at batch 1 & 32; % of HBM roofline"

WORKLOADS = {
    # name: (synth workload, batch override, description)
    "s2_b1": ("s2_b1", None, "full S2-shaped Dual-AR decode, batch 1, 1,024-token prompt, greedy"),
    "s2_b32": ("s2_b32", None, "full S2-shaped Dual-AR decode, batch 32, ragged prompts 512..4,096, top-p 0.9"),
    "fast_s2": ("fast_s2", 1, "S2-shaped fast AR alone, batch 1, greedy"),
    "fast_s2_b16": ("fast_s2", 16, "S2-shaped fast AR alone, batch 16, greedy"),
    "tiny_b1": ("tiny_b1", None, "tiny fp32 Dual-AR, batch 1, 32-token prompt, greedy"),
    "s2_prefill": ("s2_prefill", None, "full S2-shaped prefill of 16,384 frame positions at batch 4 "
                                       "(time to frame 0), then 64 greedy decode frames"),
    "s2_fast_tf": ("fast_s2", None, "S2-shaped teacher-forced fast AR: 819 (hidden state, codes) pairs, "
                                    "8,190 rows through the fast layers and head per step"),
    "s2_b1_w4": ("s2_b1", None, "full S2-shaped Dual-AR decode, batch 1, W4A16 weights (4-bit groups of 128 "
                                "with bf16 scales; the last 12 slow layers' attention, the embeddings and "
                                "heads in bf16), 1,024-token prompt, greedy"),
    "s2_b4_w4": ("s2_b1", 4, "full S2-shaped Dual-AR decode, batch 4, W4A16 weights (as s2_b1_w4), "
                             "1,024-token prompts, greedy"),
    "s2_b8_w4": ("s2_b1", 8, "full S2-shaped Dual-AR decode, batch 8, W4A16 weights (as s2_b1_w4), "
                             "1,024-token prompts, greedy"),
}
MFMA_BF16_PEAK_TFLOPS = 2500.0


# HBM bytes per dispatch of the roofline kernels (the batch-1 SwiGLU W1|W3
# GEMV: bf16 `gemv_rx_kernel`, 4-bit `gemv_w4_kernel`; at batch 32 the
# stream-K W1|W3 product `mfma_skw_kernel<2, ...>` and its finish
# `sk_finish_kernel<2, ...>`), from rocprofv3 --pmc runs restricted to that
# kernel (bf16: `bench.py --steps 4 --warmup 2 --profile-frames 0
# --no-cpu-baseline`; 4-bit: the same with `--workload s2_b1_w4 --prompt-len
# 16`; batch 32: `--workload s2_b32 --steps 4 --warmup 2 --reps 1
# --profile-frames 0 --no-cpu-baseline`): FETCH_SIZE and WRITE_SIZE (KiB per
# dispatch) times the factor the same counter reads for a plain 1 GiB device
# copy (bench.py --copy-calibration).  The figures hold for the kernel text
# they were taken on: if a kernel's source changes, `traffic` is reported as
# null until they are measured again.
_FETCH_SCALE = 1073741824 / 1024 / 524300.3125
_WRITE_SCALE = 1073741824 / 1024 / 1048576.0
ROOFLINE_COUNTERS = {
    "gemv_rx_kernel": {"fetch_kib": 48746.695, "write_kib": 38.05,
                       "sha256": "896f099c92dd1480f9cae59c9e461a974a00feaeec347ad0b0be964cd656bd96"},
    "gemv_w4_kernel": {"fetch_kib": 12721.425, "write_kib": 38.0,
                       "sha256": "56e7cfaa8dc156927292197036e869ffd7b4068527330939f40693f0a8368b6e"},
    "mfma_skw_kernel": {"fetch_kib": 52015.6, "write_kib": 9888.1, "file": "gemm.hip",
                        "sha256": "ab55fea37c92de250f2acc732bf687a8860b0d5ea2339bcc3dd5ed56bfce4415"},
    "sk_finish_kernel": {"fetch_kib": 4987.0, "write_kib": 1824.0, "file": "gemm.hip",
                         "sha256": "6246a8116a74dce359ca6730f2ec28dff62bde13e0765a06fe9c3d9b100547fc"},
}


def kernel_source_sha256(name, file="gemv.hip"):
    """SHA-256 of a kernel's text in a csrc file: its template line to its closing brace."""
    import hashlib
    src = open(os.path.join(ROOT, "dual_autoregressive_tts_amd", "csrc", file)).read()
    i = src.index(f" {name}(GemvParams p) {{")
    i = src.rindex("template", 0, i)
    j = src.index("\n}\n", i) + 3
    return hashlib.sha256(src[i:j].encode()).hexdigest()


def roofline_traffic(name="gemv_rx_kernel"):
    """Measured HBM bytes per launch of a roofline kernel, or None when they
    are missing or were taken on other kernel text."""
    c = ROOFLINE_COUNTERS.get(name)
    if not c or c["write_kib"] is None or kernel_source_sha256(name, c.get("file", "gemv.hip")) != c["sha256"]:
        return None
    return round(c["fetch_kib"] * 1024 * _FETCH_SCALE + c["write_kib"] * 1024 * _WRITE_SCALE)


def b32_traffic():
    """The batch-32 roofline pair (the stream-K W1|W3 product and its finish,
    timed together): the sum of both kernels' measured bytes, or None."""
    a, f = roofline_traffic("mfma_skw_kernel"), roofline_traffic("sk_finish_kernel")
    return None if a is None or f is None else a + f


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class _LazyF32(dict):
    """bf16 bit arrays -> float32 on access (the oracle copies each to float64)."""

    def __init__(self, m, w):
        super().__init__()
        self.m, self.w = m, w

    def __getitem__(self, k):
        import synth
        v = self.w[k]
        return synth.bf16_bits_to_f32(v).reshape(v.shape) if self.m["weight_dtype"] == "bf16" else v


def host_info():
    """The host the oracle is timed on: logical CPUs, CPU model, numpy and
    its BLAS (library, version, thread-pool size)."""
    info = {"nproc": os.cpu_count(), "cpu_model": None, "numpy": np.__version__, "blas": None}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if blas:
            b = blas[0]
            info["blas"] = {"library": b.get("internal_api"), "version": b.get("version"),
                            "threads": b.get("num_threads")}
    except Exception:
        pass
    return info


def cpu_baseline(m, w, fast_only, seed, prompt=None, plen=None, budget_s=20.0):
    """The oracle, untuned, on the host cores: frames/s on a bounded sample.
    With `prompt` the oracle first prefills that prompt (untimed), so the
    timed frames attend over the workload's own context."""
    import synth
    from oracle import DualAROracle, Sampling
    host = host_info()
    cores = (host["blas"] or {}).get("threads") or host["nproc"]
    t0 = time.time()
    if fast_only:
        shell = dict(m, n_layer=1, dim=m["fast_dim"], vocab_size=m["codebook_size"] + 64, semantic_begin_id=0,
                     semantic_end_id=m["codebook_size"] - 1, end_id=m["codebook_size"] + 8)
        spec = {n: s for n, s, _ in synth.tensor_specs(shell)}
        lw = _LazyF32(m, w)
        wf = {n: (lw[n] if n.startswith("fast_") else np.zeros(s, dtype=np.float32)) for n, s in spec.items()}
        o = DualAROracle(shell, wf, max_seq=8)
        h, q0 = synth.make_fast_inputs(m, 64, 1, seed=seed)
        log(f"[cpu] oracle built in {time.time() - t0:.1f}s")
        n, t1 = 0, time.time()
        while n < 64 and (n == 0 or time.time() - t1 < budget_s):
            o.fast_frame(h[n, 0].astype(np.float64), int(q0[n, 0]), Sampling())
            n += 1
        dt = time.time() - t1
        return {"value": n / dt, "unit": "frames/s", "cores": int(cores), "kind": "oracle",
                "sample": f"{n} fast-AR frames (10 passes each) at batch 1, float64 oracle", "host": host}
    if prompt is None:
        P = synth.make_prompts(m, ("fixed", 2, 8, 6), [16], seed=seed)[0]
        desc = "a 16-token prompt"
    else:
        P = np.asarray(prompt)[:, :int(plen)]
        desc = f"the workload's {int(plen):,}-token prompt (sequence 0)"
    o = DualAROracle(m, _LazyF32(m, w), max_seq=P.shape[1] + 40)
    seq = o.new_sequence()
    o.prefill(seq, P, Sampling())
    log(f"[cpu] oracle built + prefill of {P.shape[1]} positions in {time.time() - t0:.1f}s")
    n, t1 = 0, time.time()
    while n < 32 and (n == 0 or time.time() - t1 < budget_s):
        o.decode_frame(seq, Sampling())
        n += 1
    dt = time.time() - t1
    return {"value": n / dt, "unit": "frames/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n} greedy decode frames at batch 1 after {desc}, float64 oracle; the prefill is "
                      f"not timed", "host": host}


def bench_fast_tf(args, torch, synth, DualAR, upload_weights, reporting):
    """The teacher-forced fast AR (scoring form): K timed steps, each one call
    over n pairs; frames/s counts pairs (one frame's fast AR each)."""
    wl = synth.WORKLOADS["fast_s2"]
    m = synth.model(wl["model"])
    N, n = m["num_codebooks"], 819
    K = args.steps if args.steps is not None else 20
    W = args.warmup
    t0 = time.time()
    w = synth.make_weights(m, seed=args.seed)
    log(f"[bench] s2_fast_tf: weights generated in {time.time() - t0:.1f}s")
    dev_w = upload_weights(m, w)
    ctx = DualAR(m, dev_w, max_batch=2, max_seq_len=16)       # 2 x 4,096 prefill rows >= n*N
    rng = np.random.default_rng(args.seed)
    h = torch.from_numpy(rng.standard_normal((n, m["fast_dim"])).astype(np.float32)).cuda()
    codes = torch.from_numpy(rng.integers(0, m["codebook_size"], size=(n, N)).astype(np.int32)).cuda()
    out = torch.empty((n, N, m["codebook_size"]), device="cuda")
    for _ in range(W):
        ctx.fast_teacher_forced(h, codes, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        ctx.fast_teacher_forced(h, codes, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    assert ctx.sync() == 0
    fl = reporting.fast_tf_flops(m, n)
    tf = fl["total"] / (ms * 1e-3) / 1e12
    log(f"[bench] {K} steps of {n} pairs: {ms:.3f} ms/step, {n / ms * 1e3:.0f} frames/s, {tf:.1f} TFLOP/s")
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import DualAROracle
        try:
            from threadpoolctl import threadpool_info
            cores = max((p.get("num_threads", 1) for p in threadpool_info()), default=os.cpu_count())
        except Exception:
            cores = os.cpu_count()
        shell = dict(m, n_layer=1, dim=m["fast_dim"], vocab_size=m["codebook_size"] + 64, semantic_begin_id=0,
                     semantic_end_id=m["codebook_size"] - 1, end_id=m["codebook_size"] + 8)
        spec = {nm: sh for nm, sh, _ in synth.tensor_specs(shell)}
        lw = _LazyF32(m, w)
        wf = {nm: (lw[nm] if nm.startswith("fast_") else np.zeros(sh, dtype=np.float32)) for nm, sh in spec.items()}
        o = DualAROracle(shell, wf, max_seq=8)
        hh, cc = h.cpu().numpy(), codes.cpu().numpy()
        cnt, t1 = 0, time.time()
        while cnt < 64 and (cnt == 0 or time.time() - t1 < 20.0):
            o.fast_teacher_forced(hh[cnt].astype(np.float64), cc[cnt].tolist())
            cnt += 1
        cpu = {"value": cnt / (time.time() - t1), "unit": "frames/s", "cores": int(cores), "kind": "oracle",
               "sample": f"{cnt} teacher-forced pairs one at a time, float64 oracle"}
    ctx.close()
    print(json.dumps({
        "metric": METRIC, "value": round(n / ms * 1e3, 3), "unit": "frames/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded random-init weights of the S2 shapes, random hidden states "
                                 "and codes)",
        "config": {"workload": f"s2_fast_tf: {WORKLOADS['s2_fast_tf'][2]}", "pairs": n, "rows": fl["rows"],
                   "accumulate": "f32", "kv_cache": m["weight_dtype"]},
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 5), "traffic": None,
                     "flops_per_step": fl["total"]},
        "cpu_baseline": cpu,
    }))


def decode_workload(args, name, torch, synth, DualAR, reporting, kit, m, w, dev_w, K, W, reps,
                    semantic_head=False, ras_on=False, profile_frames=16):
    """Time K decode steps of workload `name`, `reps` times after W warm-up
    steps (each repetition: exactly K steps between two events on the
    context's stream, synchronised on both sides); the median repetition is
    reported.  Returns the JSON fields of the workload's line."""
    K_ATTN, K_GEMV, K_GEMV_SWIGLU = kit
    wl_name, b_over, desc = WORKLOADS[name]
    wl = synth.WORKLOADS[wl_name]
    w4 = name.endswith("_w4")
    B = b_over or wl["batch"]
    fast_only = wl.get("fast_only", False)
    N = m["num_codebooks"]
    samp = wl["sampling"]
    ras = 10 if ras_on and not fast_only else 0
    S = DualAR.sampling(greedy=samp["greedy"], temperature=samp["temperature"], top_p=samp["top_p"],
                        min_frames=1 << 30,   # fixed-length runs: <|im_end|> stays masked
                        ras_window=ras, ras_temperature=1.0, ras_top_p=0.9)
    Pf = profile_frames
    P_frames = W + reps * K + Pf + 1
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    plen, prompts = None, None
    if fast_only:
        h, q0 = synth.make_fast_inputs(m, P_frames, B, seed=args.seed)
        ctx = DualAR(m, dev_w, max_batch=B, max_seq_len=16)
        H = torch.from_numpy(h).cuda()
        Q = torch.from_numpy(q0).cuda()
        U = None
        if not samp["greedy"]:
            U = torch.from_numpy(synth.make_uniforms((P_frames, B, N), seed=args.seed)).cuda()
        run = lambda a, b: ctx.fast_frames(H[a:b], Q[a:b], S, None if U is None else U[a:b])  # noqa
        ttff_ms = None
    else:
        plen = synth.prompt_lengths(dict(wl, batch=B), seed=args.seed)
        layout = wl["prompt"]
        if args.prompt_len:
            P = args.prompt_len
            plen = np.full(B, P, dtype=np.int32)
            layout = ("fixed", P // 8, P // 2, P - P // 8 - P // 2)
        prompts = synth.make_prompts(m, layout, plen, seed=args.seed)
        # the default prefill chunk (4-bit weights too: their prefill steps run
        # on the matrix-core 2-D tiles)
        ctx = DualAR(m, dev_w, max_batch=B, max_seq_len=int(plen.max()) + P_frames + 2)
        U = None
        if not samp["greedy"] or ras:
            U = torch.from_numpy(synth.make_uniforms((1 + P_frames, B, N + (ras > 0)), seed=args.seed)).cuda()
        T = torch.from_numpy(prompts).cuda()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        ctx.prefill(T, plen, S, None if U is None else U[0])
        e1.record()
        torch.cuda.synchronize()
        ttff_ms = e0.elapsed_time(e1)
        log(f"[bench] {name}: prefill + frame 0: {ttff_ms:.1f} ms")
        run = lambda a, b: ctx.decode_frames(b - a, S, None if U is None else U[1 + a:1 + b])  # noqa

    # ---- warm-up, then `reps` repetitions of exactly K timed steps ----
    run(0, W)
    torch.cuda.synchronize()
    rep_ms = []
    for r in range(reps):
        a = W + r * K
        e0, e1 = ev(), ev()
        torch.cuda.synchronize()
        e0.record()
        run(a, a + K)
        e1.record()
        torch.cuda.synchronize()
        rep_ms.append(e0.elapsed_time(e1))
    ctx.sync()
    med = sorted(range(reps), key=lambda r: rep_ms[r])[reps // 2]
    ms = rep_ms[med]
    ms_per_step = ms / K
    fps = B * K / (ms / 1e3)
    log(f"[bench] {name}: {reps} x {K} steps, ms {[round(x, 2) for x in rep_ms]}; median {ms_per_step:.3f} "
        f"ms/step, {fps:.1f} frames/s")

    # ---- algorithmic bytes of the median repetition's steps ----
    if fast_only:
        step_bytes = reporting.frame_bytes(m, [1] * B, fast_only=True)["total"] * K
    else:
        step_bytes = 0
        a = W + med * K
        for f in range(K):
            L = [int(p) + a + f + 1 for p in plen]
            step_bytes += reporting.frame_bytes(m, L, semantic_head=semantic_head,
                                                w4_names=synth.w4_names(m))["total"]
    step_gbps = step_bytes / (ms / 1e3) / 1e9

    # ---- live per-launch timing (HIP events on the context's stream) ----
    roofline, extra = None, {}
    if Pf >= 2:   # (0 for profiler runs that only want the timed frames)
        a0 = W + reps * K
        ctx.profile_begin(K_GEMV)
        run(a0, a0 + Pf // 2)
        g = ctx.profile_end()
        ctx.profile_begin(K_GEMV_SWIGLU)
        run(a0 + Pf // 2, a0 + Pf)
        f = ctx.profile_end()
        gemv_avg_us = g["total_ms"] * 1e3 / max(g["launches"], 1)
        gemv_gbps = g["bytes"] / max(g["total_ms"] * 1e-3, 1e-12) / 1e9
        gemv_share = g["total_ms"] / ((Pf // 2) * ms_per_step)
        sw_avg_us = f["total_ms"] * 1e3 / max(f["launches"], 1)
        sw_bytes = f["bytes"] / max(f["launches"], 1)
        sw_gbps = sw_bytes / max(sw_avg_us * 1e-6, 1e-12) / 1e9
        log(f"[bench] {name}: GEMV family: {g['launches']} launches, avg {gemv_avg_us:.2f} us, {gemv_gbps:.0f} GB/s, "
            f"{100 * gemv_share:.1f}% of step time")
        log(f"[bench] {name}: SwiGLU gate|up product: {f['launches']} launches, avg {sw_avg_us:.2f} us, "
            f"{sw_bytes / 1e6:.2f} MB/launch, {sw_gbps:.0f} GB/s")
        if w4 and B == 1:
            kname = ("gemv_w4_kernel<2, 2, 5, 1, false> (SwiGLU W1|W3 GEMV, 2 x 9728 x 2560 as 4-bit groups of 128 with "
                     "bf16 scales)")
        elif w4:
            kname = ("gemv_w4b_kernel<2, 3, 8> (SwiGLU W1|W3 matrix-core GEMV over %d activation rows, 2 x 9728 x "
                     "2560 as 4-bit groups of 128 with bf16 scales)" % B)
        elif m["weight_dtype"] == "f32":
            kname = "SwiGLU W1|W3 GEMV"
        elif B == 1:
            kname = ("gemv_rx_kernel<bf16, 2 rows/wave, gate+up, 5 units> (SwiGLU W1|W3 GEMV, "
                     "2 x 9728 x 2560 bf16)")
        else:
            kname = ("mfma_skw_kernel<2, 4, 1, 3, 3> + sk_finish_kernel<2, 4, 1> (SwiGLU W1|W3 stream-K "
                     "matrix-core product and its finish, 2 x 9728 x 2560 bf16, %d activation rows; "
                     "timed together)" % B)
        roofline = {"bound": "hbm",
                    "kernel": kname,
                    "achieved": round(sw_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(sw_gbps / HBM_PEAK_GBPS, 4),
                    "traffic": ((roofline_traffic("gemv_w4_kernel") if w4 else roofline_traffic("gemv_rx_kernel"))
                                if (B == 1 and m["weight_dtype"] == "bf16") else
                                b32_traffic() if (B == 32 and not w4 and m["weight_dtype"] == "bf16") else None),
                    "avg_launch_us": round(sw_avg_us, 3), "bytes_per_launch": round(sw_bytes),
                    "launches_profiled": f["launches"],
                    "gemv_family": {"achieved_GBps": round(gemv_gbps, 1), "avg_launch_us": round(gemv_avg_us, 3),
                                    "launches": g["launches"], "share_of_step_time": round(gemv_share, 4)}}
        if not fast_only:
            ctx.profile_begin(K_ATTN)
            run(a0 + Pf, a0 + Pf + 1)
            at = ctx.profile_end()
            extra["attention"] = {"avg_launch_us": round(at["total_ms"] * 1e3 / max(at["launches"], 1), 3),
                                  "launches": at["launches"]}
        ctx.sync()
    ctx.close()

    prefill = {}
    if wl_name == "s2_prefill" and ttff_ms:
        # the prefill is the matrix-core roofline case: its flops over the time to frame 0
        fl = reporting.prefill_flops(m, plen)
        tf = fl["total"] / (ttff_ms * 1e-3) / 1e12
        prefill["prefill"] = {"tokens": fl["tokens"], "flops": fl["total"], "linear_flops": fl["linear"],
                              "attention_flops": fl["attention"], "ms": round(ttff_ms, 2),
                              "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                                           "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 5),
                                           "traffic": None}}
        log(f"[bench] prefill: {fl['total'] / 1e12:.0f} TFLOP in {ttff_ms:.0f} ms = {tf:.1f} TFLOP/s")

    fields = {
        "value": round(fps, 3), "unit": "frames/s", "steps": K, "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "repetitions_ms_per_step": [round(x / K, 4) for x in rep_ms],
        "config": {"workload": f"{name}: {desc}" + ("" if fast_only else (
                       ", semantic-candidate slow head" if semantic_head else ", full-vocabulary slow head"))
                   + (", loop breaker on (window 10)" if ras else ""), "batch": B,
                   "prompt_len": None if fast_only else [int(x) for x in plen][:4] + (["..."] if B > 4 else []),
                   "accumulate": "f32", "kv_cache": m.get("kv_dtype", m["weight_dtype"])},
        "codec_tokens_per_s": round(reporting.codec_tokens_per_s(fps, N), 1),
        "rtf_per_sequence": round(reporting.rtf(fps / B), 5),
        "step_hbm": {"bytes_per_step": round(step_bytes / K), "achieved_GBps": round(step_gbps, 1),
                     "frac": round(step_gbps / HBM_PEAK_GBPS, 4)},
        "ttff_ms": None if ttff_ms is None else round(ttff_ms, 2),
        **prefill,
        "roofline": roofline,
        **extra,
    }
    return fields, plen, prompts, fast_only


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--reps", type=int, default=5, help="timed repetitions of K steps; the median is reported")
    ap.add_argument("--workload", default="s2_b1", choices=sorted(WORKLOADS))
    ap.add_argument("--profile-frames", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-batch32", action="store_true",
                    help="s2_b1 only: skip the batch-32 line nested in the output")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--prompt-len", type=int, default=None,
                    help="override the prompt length (same three-segment layout); for counter runs")
    ap.add_argument("--ras", action="store_true",
                    help="turn on the slow loop breaker (window 10, second draw at T=1.0, top-p 0.9)")
    ap.add_argument("--semantic-head", action="store_true",
                    help="slow head over the semantic rows and the end row only (identical draws)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 10 times (scale for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(sequences are independent, so batch sharding would replicate the weights per GPU).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "copies": 10}))
        return

    import synth
    from dual_autoregressive_tts_amd import DualAR, reporting
    from dual_autoregressive_tts_amd.binding import K_ATTN, K_GEMV, K_GEMV_SWIGLU, upload_weights

    if args.workload == "s2_fast_tf":
        return bench_fast_tf(args, torch, synth, DualAR, upload_weights, reporting)
    wl_name, _, _ = WORKLOADS[args.workload]
    wl = synth.WORKLOADS[wl_name]
    m = synth.model(wl["model"])
    w4 = args.workload.endswith("_w4")
    if w4:
        m = dict(m, w4a16=1)
    if args.semantic_head:
        m = dict(m, semantic_head=1)
    # 20 steps per repetition unless given: five repetitions then span ~100
    # frames, so the context (and the attention's share) grows by under 10 %
    K = args.steps if args.steps is not None else 20
    W = args.warmup
    reps = max(1, args.reps)

    t0 = time.time()
    w = synth.make_weights(m, seed=args.seed)
    log(f"[bench] {args.workload}: weights generated in {time.time() - t0:.1f}s")
    if w4:
        t0 = time.time()
        w = synth.make_w4_model(m, w)
        log(f"[bench] {len(synth.w4_names(m))} matrices as 4-bit groups in {time.time() - t0:.1f}s")
    dev_w = upload_weights(m, w)
    torch.cuda.synchronize()
    log(f"[bench] weights on device ({sum(t.numel() * t.element_size() for t in dev_w.values()) / 1e9:.2f} GB)")

    kit = (K_ATTN, K_GEMV, K_GEMV_SWIGLU)
    fields, plen, prompts, fast_only = decode_workload(
        args, args.workload, torch, synth, DualAR, reporting, kit, m, w, dev_w, K, W, reps,
        semantic_head=args.semantic_head, ras_on=args.ras, profile_frames=args.profile_frames)

    nested = {}
    if args.workload == "s2_b1" and not args.no_batch32 and not args.semantic_head and not args.prompt_len:
        # the metric is quoted at batch 1 and 32: the batch-32 workload (same
        # weights, 32 ragged prompts, top-p 0.9) is timed in the same process
        K32 = args.steps if args.steps is not None else 20
        b32, _, _, _ = decode_workload(args, "s2_b32", torch, synth, DualAR, reporting, kit, m, w, dev_w, K32, W,
                                       reps, ras_on=args.ras, profile_frames=args.profile_frames)
        nested["batch32"] = b32

    cpu = None
    if not args.no_cpu_baseline and not w4:   # the oracle baseline is timed on the bf16 model
        del dev_w
        torch.cuda.empty_cache()
        if fast_only:
            cpu = cpu_baseline(m, w, True, args.seed)
        else:
            cpu = cpu_baseline(m, w, False, args.seed, prompt=prompts[0], plen=plen[0])
        log(f"[cpu] oracle {cpu['value']:.4f} frames/s on {cpu['cores']} threads")

    out = {
        "metric": METRIC, "value": fields.pop("value"), "unit": fields.pop("unit"), "n_gpus": 1,
        "steps": fields.pop("steps"), "warmup": fields.pop("warmup"), "ms_per_step": fields.pop("ms_per_step"),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if m["weight_dtype"] == "bf16" else "f32",
        "data": "synthetic (seeded random-init weights of the S2 shapes, synthetic prompts)",
        "config": fields.pop("config"),
        **fields,
        **nested,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
