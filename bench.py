#!/usr/bin/env python3
"""Throughput of the block-scaled FP8 linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--skip-cpu] [--skip-extra] [--copy-calibration]
    python bench.py --read-sweep     # what single reads of 8 to 419 MB reach (no projection timed)

One step is the large prefill on M = 8192 synthetic tokens: quantize X
[8192, 7168] per token in 1x128 groups, then the W8A8 GEMM against the block-FP8
weight [18432, 7168] (heavy-tailed per-block scales) with its F32 epilogue and
BF16 output.  ``value`` is the step's algorithmic FLOP rate, 2*M*N*K over the
step time (quantization included).  The step runs as one HIP graph of its two
calls, replayed back to back; the timed region is bracketed by HIP events on
the replay stream, inputs resident in HBM.

``roofline`` is the GEMM kernel alone: FLOPs per launch over its mean device
time from a graph of back-to-back launches, against the dense FP8 MFMA peak,
with the HBM traffic the profiled counters measured (profiles/traffic.json,
reported only while the kernel source matches the hash it was measured on).
``cpu_baseline`` is the oracle (NumPy) on the host cores, on the whole step
(all 8192 tokens; median of three repetitions of about five seconds each).

The same JSON line also carries:
* ``dense_ffn_prefill``: the dense-FFN prefill pass at M = 1024 (quantize ->
  W8A8 gate/up [2x17408, 5120] -> quantize -> W8A8 down [5120, 17408]) as a
  graph of four calls, with each GEMM's roofline, the step over two weight
  copies (``rotated``), and the chained form whose down input comes from the
  gate/up output through ``quant_glu`` (``ffn_chain``);
* ``decode_gemv`` (and ``decode_gemv_5000x4000``, ``qkv_decode``): the W8A16/F32
  arm at M in {1, 4, 8} on W [5120, 5120] (W [5000, 4000]; grouped Q/K/V at
  M = 1), rotating through >= 512 MiB of weight copies so the 256 MB Infinity
  Cache cannot serve them, per-launch median / p10 / p90 over 100 replays,
  with an HBM roofline on algorithmic bytes and a plain read of the same bytes
  (``bsf8_read_stream``) as context;
* ``qkv_w8a8_decode``: grouped Q/K/V through the W8A8 arm at M = 1, rotated;
* ``qkv_w8a8_dynamic_decode``: the same at M = 1 on F32 activations with the
  quantization inside the step: the dynamic call (quantized inside the
  one-token kernel) against quant_act followed by linear_w8a8, rotated;
* ``ffn_down_decode`` and ``ffn_down_w8a8_decode``: the FFN down projection
  [5120, 17408] at one token through both arms, rotated, and
  ``ffn_down_w8a8_dynamic_decode`` with the quantization inside the step;
* ``qkv_prefill`` and ``qkv_w8a16_m512``: grouped Q/K/V at M = 512 through the
  W8A8 and the W8A16/F32 arm;
* ``rotated``: the headline GEMM over three weight copies used in turn;
* ``dense_arm``: the resident=False arm on the grouped Q/K/V weight: the
  upcast to a dense BF16 copy (rotated over three weight copies, HBM roofline
  on its algorithmic bytes) and the dense BF16 product at M = 128 and 512
  (BF16 MFMA roofline).

Inputs are seeded synthetic data (``synth``) already resident in HBM before
timing starts.
"""
from __future__ import annotations

import argparse
import statistics
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0     # MI355X dense FP8 MFMA
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense BF16 MFMA
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
ROTATE_BYTES = 640 << 20     # > 512 MiB of distinct weight copies for the GEMV


def code_digest(path):
    """sha256[:16] of a C++/HIP source with its comments and whitespace removed: a change to the code
    changes it, a change to a comment does not."""
    import hashlib, re
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()[:16]


def profiled_traffic(key):
    """Bytes per launch moved between L2 and memory for ``key``, from the committed counter runs in
    profiles/traffic.json, or None when the kernel's source code has changed since those counters were
    taken."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            entry = json.load(f)[key]
        digest = code_digest(os.path.join(ROOT, "block_scaled_fp8_linear_amd", "csrc", entry["source"]))
    except (OSError, KeyError, ValueError):
        return None
    return entry["traffic_bytes"] if digest == entry["code_sha256_16"] else None


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--skip-cpu", action="store_true", help="leave out the oracle's CPU baseline")
    ap.add_argument("--skip-extra", action="store_true", help="leave out every line but the headline step")
    ap.add_argument("--no-clock-sample", action="store_true",
                    help="do not run rocm-smi for the clock under load (profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (for HBM counter scaling)")
    ap.add_argument("--read-sweep", action="store_true",
                    help="only time two plain read kernels over buffer sizes from 8 MB to 416 MB and print that line")
    return ap.parse_args()


def graph_of(torch, fn, reps=1):
    """A HIP graph of ``reps`` back-to-back calls of ``fn``.

    Every buffer, workspaces included, is allocated before capture; the call is
    made once eagerly first.  Replaying a graph launches its kernels back to
    back, so the time of a replay is device time, without the host's launch
    latency (which exceeds the shorter kernels here).
    """
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    torch.cuda.synchronize()
    return g


def replay_ms(torch, g, n):
    """Mean time of one replay of ``g`` over ``n`` back-to-back replays, from HIP events on the replay stream."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def under_profiler():
    """True when this process runs under rocprofv3 (its variables are in the environment)."""
    return any(k.startswith("ROCPROF") for k in os.environ)


def replay_stats(torch, g, n, per):
    """Per-launch device time from ``n`` replays of ``g`` (``per`` launches each),
    each replay between its own pair of HIP events; replays are queued back to
    back, so the device never waits for the host.  Milliseconds.  Under a
    profiler (counter runs) only a few replays are queued: its per-dispatch
    bookkeeping is not meant for thousands of queued graph launches."""
    if under_profiler():
        n = min(n, 5)
    pairs = []
    for _ in range(n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) / per for a, b in pairs])
    return dict(median=float(np.median(t)), p10=float(np.percentile(t, 10)), p90=float(np.percentile(t, 90)),
                mean=float(t.mean()), launches=int(n * per))


def sample_sclk(torch, g, replays):
    """The shader clock as rocm-smi reports it while ``replays`` replays of ``g`` run
    (best effort: the tool's own text, or None when it is not available).  Not
    under a profiler: the tool would be a second process on the profiled GPU."""
    if under_profiler() or os.environ.get("BSF8_BENCH_NO_CLOCK_SAMPLE"):
        return None
    import subprocess
    for _ in range(replays):
        g.replay()
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20)
        lines = [l.strip() for l in r.stdout.splitlines() if "sclk" in l.lower()]
    except Exception:
        lines = None
    torch.cuda.synchronize()
    return lines or None


def settle(torch, fn, seconds=1.0):
    """Run ``fn`` back to back for about ``seconds`` before anything is timed.

    The GPU raises its clock only under sustained load: the first milliseconds
    after an idle period run measurably slower (more than 20 % on the large
    GEMM), which would make the timed steps depend on what ran before them.
    """
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def to_device_member(torch, m, dev):
    w = torch.from_numpy(np.ascontiguousarray(m.codes)).to(dev)
    s = torch.from_numpy(np.ascontiguousarray(m.scale_bits).view(np.int16)).to(dev).view(torch.bfloat16)
    return w, s


def bench_prefill(torch, B, synth, steps, warmup, dev):
    log("prefill: generating dense-FFN inputs (M=1024)")
    gu = synth.config3_gate_up()
    dn = synth.config3_down()
    w_gu = B.BlockFP8Weight([to_device_member(torch, m, dev) for m in gu.members])
    w_dn = B.BlockFP8Weight([to_device_member(torch, m, dev) for m in dn.members])
    x_gu = torch.from_numpy(gu.x).to(dev)
    x_dn = torch.from_numpy(dn.x).to(dev)
    M = gu.x.shape[0]
    y_gu = torch.empty((M, w_gu.n_total), dtype=torch.bfloat16, device=dev)
    y_dn = torch.empty((M, w_dn.n_total), dtype=torch.bfloat16, device=dev)
    xq_gu = torch.empty((M, w_gu.K), dtype=torch.uint8, device=dev)
    xs_gu = B.scales_kmajor(M, -(-w_gu.K // 128), dev)   # [M, Kb] views, token index contiguous
    xq_dn = torch.empty((M, w_dn.K), dtype=torch.uint8, device=dev)
    xs_dn = B.scales_kmajor(M, -(-w_dn.K // 128), dev)
    ws_gu = w_gu.workspace(B.ARM_W8A8, M)
    ws_dn = w_dn.workspace(B.ARM_W8A8, M)
    calls = {
        "quant_gate_up": lambda: B.quant_act(x_gu, xq_gu, xs_gu),
        "gemm_gate_up": lambda: B.linear_w8a8(w_gu, xq_gu, xs_gu, out=y_gu, workspace=ws_gu),
        "quant_down": lambda: B.quant_act(x_dn, xq_dn, xs_dn),
        "gemm_down": lambda: B.linear_w8a8(w_dn, xq_dn, xs_dn, out=y_dn, workspace=ws_dn),
    }

    def step():
        for f in calls.values():
            f()

    # One step = one replay of a graph of the four calls.
    g_step = graph_of(torch, step)
    settle(torch, g_step.replay)
    for _ in range(warmup):
        g_step.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_step = replay_ms(torch, g_step, steps)
    wall = time.perf_counter() - t0
    sclk = sample_sclk(torch, g_step, 2000)
    # Device time of each call: a graph of 20 back-to-back launches, replayed
    # 50 times (1000 launches), each replay timed on its own.
    kms, kstats = {}, {}
    for name, f in calls.items():
        g = graph_of(torch, f, 20)
        g.replay()
        st = replay_stats(torch, g, 50, 20)
        kms[name] = st["mean"]
        kstats[name] = {k: (round(v * 1e3, 2) if k != "launches" else v) for k, v in st.items()}
        del g
    flop_gu = 2.0 * M * w_gu.n_total * w_gu.K
    flop_dn = 2.0 * M * w_dn.n_total * w_dn.K
    # Rotated: a second copy of both weights, and graphs that alternate the
    # copies, so each call's weights (178 + 89 MB per copy) were last touched a
    # copy ago and the 256 MB Infinity Cache cannot hold them between uses.
    w_gu2 = B.BlockFP8Weight([(t.clone(), sc.clone()) for t, sc in w_gu.members])
    w_dn2 = B.BlockFP8Weight([(t.clone(), sc.clone()) for t, sc in w_dn.members])
    ws_gu2 = w_gu2.workspace(B.ARM_W8A8, M)
    ws_dn2 = w_dn2.workspace(B.ARM_W8A8, M)

    def step2():
        step()
        B.quant_act(x_gu, xq_gu, xs_gu)
        B.linear_w8a8(w_gu2, xq_gu, xs_gu, out=y_gu, workspace=ws_gu2)
        B.quant_act(x_dn, xq_dn, xs_dn)
        B.linear_w8a8(w_dn2, xq_dn, xs_dn, out=y_dn, workspace=ws_dn2)

    g_rot = graph_of(torch, step2)
    settle(torch, g_rot.replay, 0.5)
    ms_step_rot = replay_ms(torch, g_rot, max(5, steps // 2)) / 2
    del g_rot
    rot_stats = {}
    for name, wa, wsa, wb, wsb, xq_, xs_, y_ in (("gemm_gate_up", w_gu, ws_gu, w_gu2, ws_gu2, xq_gu, xs_gu, y_gu),
                                                 ("gemm_down", w_dn, ws_dn, w_dn2, ws_dn2, xq_dn, xs_dn, y_dn)):
        def alt(wa=wa, wsa=wsa, wb=wb, wsb=wsb, xq_=xq_, xs_=xs_, y_=y_):
            B.linear_w8a8(wa, xq_, xs_, out=y_, workspace=wsa)
            B.linear_w8a8(wb, xq_, xs_, out=y_, workspace=wsb)
        g = graph_of(torch, alt, 10)
        g.replay()
        st = replay_stats(torch, g, 20, 20)
        rot_stats[name] = {k: (round(v * 1e3, 2) if k != "launches" else v) for k, v in st.items()}
        del g
    rotated = dict(ms_per_step=ms_step_rot, tflops=(flop_gu + flop_dn) / (ms_step_rot * 1e-3) / 1e12,
                   kernels_us_stats=rot_stats,
                   gemm_gate_up_tflops=flop_gu / (rot_stats["gemm_gate_up"]["mean"] * 1e-6) / 1e12,
                   gemm_down_tflops=flop_dn / (rot_stats["gemm_down"]["mean"] * 1e-6) / 1e12)
    del w_gu2, w_dn2
    res = dict(rotated=rotated,
        ms_per_step=ms_step, wall_s=wall, flop_per_step=flop_gu + flop_dn,
        tflops=(flop_gu + flop_dn) / (ms_step * 1e-3) / 1e12,
        kernels_ms=kms, kernels_us_stats=kstats, sclk=sclk,
        gemm_gate_up_tflops=flop_gu / (kms["gemm_gate_up"] * 1e-3) / 1e12,
        gemm_down_tflops=flop_dn / (kms["gemm_down"] * 1e-3) / 1e12,
        quant_gate_up_gbs=(M * w_gu.K * 5 + M * (-(-w_gu.K // 128)) * 4) / (kms["quant_gate_up"] * 1e-3) / 1e9,
        quant_down_gbs=(M * w_dn.K * 5 + M * (-(-w_dn.K // 128)) * 4) / (kms["quant_down"] * 1e-3) / 1e9,
        flop_gate_up=flop_gu, M=M,
        describe_gate_up=w_gu.describe(B.ARM_W8A8, M), describe_down=w_dn.describe(B.ARM_W8A8, M),
        fixture_sha256=synth.sha256_of(*(m.codes for m in gu.members), gu.x),
    )
    # Chained FFN: the down projection's input is the gate/up output taken
    # through the gated activation and the quantizer in one pass (quant_glu),
    # instead of a separate activation tensor.
    def chain():
        B.quant_act(x_gu, xq_gu, xs_gu)
        B.linear_w8a8(w_gu, xq_gu, xs_gu, out=y_gu, workspace=ws_gu)
        B.quant_glu(y_gu, xq_dn, xs_dn)
        B.linear_w8a8(w_dn, xq_dn, xs_dn, out=y_dn, workspace=ws_dn)
    g_chain = graph_of(torch, chain)
    settle(torch, g_chain.replay, 0.3)
    ms_chain = replay_ms(torch, g_chain, steps)
    del g_chain
    g_glu = graph_of(torch, lambda: B.quant_glu(y_gu, xq_dn, xs_dn), 20)
    g_glu.replay()
    sg = replay_stats(torch, g_glu, 50, 20)
    del g_glu
    F = w_dn.K
    glu_bytes = M * 2 * F * 2 + M * F + M * (-(-F // 128)) * 4
    res["ffn_chain"] = dict(ms_per_step=ms_chain, tflops=(flop_gu + flop_dn) / (ms_chain * 1e-3) / 1e12,
                            glu_us=sg["median"] * 1e3, glu_us_p10=sg["p10"] * 1e3, glu_us_p90=sg["p90"] * 1e3,
                            glu_launches=sg["launches"], glu_gbs=glu_bytes / (sg["median"] * 1e-3) / 1e9,
                            glu_bytes=glu_bytes)
    del g_step, w_gu, w_dn
    return res


def bench_w8a16_rotating(torch, B, members, x_np, Ms, dev, label):
    """W8A16/F32 at small M on ``members``, rotating through >= ROTATE_BYTES of
    weight copies (beyond the Infinity Cache): one HIP graph holds one launch per
    copy; 100 replays give the per-launch median / p10 / p90.  Also times a plain
    read of the same weight bytes (a torch int32 sum over each copy) as the
    achievable-bandwidth context."""
    per_copy = sum(m.codes.nbytes + m.scale_bits.nbytes for m in members)
    copies = max(2, -(-ROTATE_BYTES // per_copy))
    log(f"{label}: {copies} weight copies of {per_copy / 2**20:.1f} MiB")
    base = [to_device_member(torch, m, dev) for m in members]
    copies_t = [[(w.clone(), sc.clone()) for w, sc in base] for _ in range(copies)]
    handles = [B.BlockFP8Weight(c) for c in copies_t]
    N = sum(m.codes.shape[0] for m in members)
    K = members[0].codes.shape[1]
    Kb = -(-K // 128)
    grid_elems = sum(-(-m.codes.shape[0] // 128) for m in members) * Kb
    out = {"workload": f"{label}: W [{N},{K}] ({len(members)} member(s)) + bf16 grid, f32 x/y, "
                       f"rotating {copies} copies ({copies * per_copy >> 20} MiB)", "by_M": {}}
    for M in Ms:
        x = torch.from_numpy(np.ascontiguousarray(x_np[:M])).to(dev)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        ws = [h.workspace(B.ARM_W8A16, M) for h in handles]

        def run():
            for i in range(copies):
                B.linear_w8a16(handles[i], x, out=y, workspace=ws[i])

        g = graph_of(torch, run)
        settle(torch, g.replay, 0.3)
        st = replay_stats(torch, g, 100, copies)
        alg = N * K + 2 * grid_elems + 4 * M * K + 4 * M * N
        out["by_M"][f"M{M}"] = dict(us=st["median"] * 1e3, us_p10=st["p10"] * 1e3, us_p90=st["p90"] * 1e3,
                                    launches=st["launches"], gbs=alg / (st["median"] * 1e-3) / 1e9,
                                    algorithmic_bytes=alg, describe=handles[0].describe(B.ARM_W8A16, M))
        del g
    # read-stream context: a plain read of each copy's weight bytes, same rotation
    sink = torch.zeros(B.READ_STREAM_SINK_WORDS, dtype=torch.int32, device=dev)

    def read_all():
        for c in copies_t:
            for w, _ in c:
                B.read_stream(w, sink)

    g = graph_of(torch, read_all)
    settle(torch, g.replay, 0.2)
    st = replay_stats(torch, g, 50, copies)
    wbytes = sum(m.codes.nbytes for m in members)
    out["read_stream_context"] = dict(us=st["median"] * 1e3, gbs=wbytes / (st["median"] * 1e-3) / 1e9,
                                      launches_per_copy=len(members),
                                      kernel="bsf8_read_stream over the same weight bytes, same rotation "
                                             "(one launch per member buffer)")
    del g, handles, copies_t
    torch.cuda.empty_cache()
    return out


def bench_qkv_prefill(torch, B, synth, dev):
    """Grouped Q/K/V (members of 6144, 1000 and 1000 rows, K = 5120) at M = 512,
    W8A8 with its quantization; graphs of 20 back-to-back calls, warm."""
    wl = synth.config4(512)
    w = B.BlockFP8Weight([to_device_member(torch, m, dev) for m in wl.members])
    x = torch.from_numpy(wl.x).to(dev)
    M = wl.x.shape[0]
    xq, xs = B.quant_act(x)
    y = torch.empty((M, w.n_total), dtype=torch.bfloat16, device=dev)
    ws = w.workspace(B.ARM_W8A8, M)
    g = graph_of(torch, lambda: B.linear_w8a8(w, xq, xs, out=y, workspace=ws), 20)
    gq = graph_of(torch, lambda: B.quant_act(x, xq, xs), 20)
    settle(torch, g.replay, 0.3)
    st = replay_stats(torch, g, 20, 20)
    sq = replay_stats(torch, gq, 20, 20)
    flop = 2.0 * M * w.n_total * w.K
    del g, gq
    return dict(workload="grouped QKV W8A8, members [6144|1000|1000, 5120], M=512, bf16 out",
                gemm_us=st["median"] * 1e3, gemm_us_p10=st["p10"] * 1e3, gemm_us_p90=st["p90"] * 1e3,
                tflops=flop / (st["median"] * 1e-3) / 1e12, quant_us=sq["median"] * 1e3,
                describe=w.describe(B.ARM_W8A8, M))


def bench_large_step(torch, B, synth, steps, warmup, dev):
    """The headline: one step = quantize X [8192, 7168] -> W8A8 GEMM on W [18432, 7168] (BF16 out),
    as one HIP graph replayed back to back; per-kernel device times from graphs of
    back-to-back launches; the GEMM also over three weight copies used in turn."""
    log("large prefill: generating M=8192, K=7168, N=18432")
    wl = synth.config5()
    w = B.BlockFP8Weight([to_device_member(torch, m, dev) for m in wl.members])
    x = torch.from_numpy(wl.x).to(dev)
    M = wl.x.shape[0]
    Kb = -(-w.K // 128)
    xq = torch.empty((M, w.K), dtype=torch.uint8, device=dev)
    xs = B.scales_kmajor(M, Kb, dev)
    y = torch.empty((M, w.n_total), dtype=torch.bfloat16, device=dev)
    ws = w.workspace(B.ARM_W8A8, M)
    calls = {"quant": lambda: B.quant_act(x, xq, xs),
             "gemm": lambda: B.linear_w8a8(w, xq, xs, out=y, workspace=ws)}

    def step():
        for f in calls.values():
            f()
    g_step = graph_of(torch, step)
    settle(torch, g_step.replay)
    for _ in range(warmup):
        g_step.replay()
    torch.cuda.synchronize()
    ms_step = replay_ms(torch, g_step, steps)
    sclk = sample_sclk(torch, g_step, 400)
    del g_step
    stats = {}
    for name, f, reps, n in (("gemm", calls["gemm"], 4, 10), ("quant", calls["quant"], 20, 20)):
        g = graph_of(torch, f, reps)
        settle(torch, g.replay, 0.3)
        stats[name] = replay_stats(torch, g, n, reps)
        del g
    flop = 2.0 * M * w.n_total * w.K
    # rotated: three copies of the 132 MB weight used in turn (396 MB > the 256 MB Infinity Cache)
    copies = [w] + [B.BlockFP8Weight([(t.clone(), sc.clone()) for t, sc in w.members]) for _ in range(2)]
    wss = [c.workspace(B.ARM_W8A8, M) for c in copies]

    def rot():
        for c, wsc in zip(copies, wss):
            B.linear_w8a8(c, xq, xs, out=y, workspace=wsc)
    g_rot = graph_of(torch, rot)
    settle(torch, g_rot.replay, 0.5)
    st_rot = replay_stats(torch, g_rot, 5, len(copies))
    del g_rot, copies
    us = lambda st: {k: (round(v * 1e3, 2) if k != "launches" else v) for k, v in st.items()}
    quant_bytes = M * w.K * 4 + M * w.K + M * Kb * 4
    return dict(M=M, N=w.n_total, K=w.K, flop=flop, ms_per_step=ms_step, sclk=sclk,
                gemm_ms=stats["gemm"]["mean"], gemm_us_stats=us(stats["gemm"]), quant_us_stats=us(stats["quant"]),
                quant_gbs=quant_bytes / (stats["quant"]["mean"] * 1e-3) / 1e9, quant_bytes=quant_bytes,
                rotated_gemm_us_stats=us(st_rot),
                describe=w.describe(B.ARM_W8A8, M),
                fixture_sha256=synth.sha256_of(*(m.codes for m in wl.members), *(m.scale_bits for m in wl.members),
                                               wl.x))


def bench_qkv_w8a16_m512(torch, B, synth, dev):
    """Grouped Q/K/V through the W8A16/F32 arm at M = 512 (config 4's second token count):
    graphs of 20 back-to-back calls, F32 activations and output."""
    wl = synth.config4(512)
    w = B.BlockFP8Weight([to_device_member(torch, m, dev) for m in wl.members])
    x = torch.from_numpy(wl.x).to(dev)
    M = wl.x.shape[0]
    y = torch.empty((M, w.n_total), dtype=torch.float32, device=dev)
    g = graph_of(torch, lambda: B.linear_w8a16(w, x, out=y), 20)
    settle(torch, g.replay, 0.3)
    st = replay_stats(torch, g, 20, 20)
    del g
    flop = 2.0 * M * w.n_total * w.K
    return dict(workload="grouped QKV W8A16/F32, members [6144|1000|1000, 5120], M=512, f32 x and y",
                us=st["median"] * 1e3, us_p10=st["p10"] * 1e3, us_p90=st["p90"] * 1e3, us_mean=st["mean"] * 1e3,
                launches=st["launches"], tflops=flop / (st["mean"] * 1e-3) / 1e12, flop=flop,
                describe=w.describe(B.ARM_W8A16, M))


def bench_w8a8_rotating(torch, B, members, x_np, dev, label):
    """W8A8 at M = 1 (quantized once; the GEMM and its split-K reduction timed per call),
    rotating through >= ROTATE_BYTES of weight copies so HBM serves the weights."""
    per_copy = sum(m.codes.nbytes + m.scale_bits.nbytes for m in members)
    copies = max(2, -(-ROTATE_BYTES // per_copy))
    log(f"{label}: {copies} weight copies of {per_copy / 2**20:.1f} MiB")
    base = [to_device_member(torch, m, dev) for m in members]
    handles = [B.BlockFP8Weight([(w.clone(), sc.clone()) for w, sc in base]) for _ in range(copies)]
    N = handles[0].n_total
    K = handles[0].K
    Kb = -(-K // 128)
    M = x_np.shape[0]
    x = torch.from_numpy(np.ascontiguousarray(x_np)).to(dev)
    xq, xs = B.quant_act(x)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    wss = [h.workspace(B.ARM_W8A8, M) for h in handles]

    def run():
        for h, wsh in zip(handles, wss):
            B.linear_w8a8(h, xq, xs, out=y, workspace=wsh)
    g = graph_of(torch, run)
    settle(torch, g.replay, 0.3)
    st = replay_stats(torch, g, 100, copies)
    del g
    grid = sum(-(-m.codes.shape[0] // 128) for m in members) * Kb
    alg = N * K + 2 * grid + M * K + 4 * M * Kb + 2 * M * N
    out = dict(workload=f"{label}: W [{N},{K}] ({len(members)} member(s)) + bf16 grid, quantized x, bf16 y, "
                        f"rotating {copies} copies ({copies * per_copy >> 20} MiB)",
               us=st["median"] * 1e3, us_p10=st["p10"] * 1e3, us_p90=st["p90"] * 1e3, us_mean=st["mean"] * 1e3,
               launches=st["launches"], algorithmic_bytes=alg, gbs=alg / (st["mean"] * 1e-3) / 1e9,
               describe=handles[0].describe(B.ARM_W8A8, M))
    del handles
    torch.cuda.empty_cache()
    return out


def bench_w8a8_dynamic_rotating(torch, B, members, x_np, Ms, dev, label):
    """The W8A8 arm on F32 activations at a few tokens, rotating through >= ROTATE_BYTES
    of weight copies: one step is the projection including the activation quantization,
    timed two ways, each as one HIP graph of one step per copy: the dynamic call (the
    streaming kernels quantize in registers) and the two calls it replaces
    (quant_act, then linear_w8a8)."""
    per_copy = sum(m.codes.nbytes + m.scale_bits.nbytes for m in members)
    copies = max(2, -(-ROTATE_BYTES // per_copy))
    log(f"{label}: {copies} weight copies of {per_copy / 2**20:.1f} MiB")
    base = [to_device_member(torch, m, dev) for m in members]
    handles = [B.BlockFP8Weight([(w.clone(), sc.clone()) for w, sc in base]) for _ in range(copies)]
    N, K = handles[0].n_total, handles[0].K
    Kb = -(-K // 128)
    grid = sum(-(-m.codes.shape[0] // 128) for m in members) * Kb
    out = {"workload": f"{label}: W [{N},{K}] ({len(members)} member(s)) + bf16 grid, f32 x quantized in the step, "
                       f"bf16 y, rotating {copies} copies ({copies * per_copy >> 20} MiB)", "by_M": {}}
    for M in Ms:
        x = torch.from_numpy(np.ascontiguousarray(x_np[:M])).to(dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        xq, xs = B.quant_act(x)
        wsd = [h.workspace(B.ARM_W8A8_DYNAMIC, M) for h in handles]
        ws8 = [h.workspace(B.ARM_W8A8, M) for h in handles]

        def run_dynamic():
            for h, wsh in zip(handles, wsd):
                B.linear_w8a8_dynamic(h, x, out=y, workspace=wsh)

        def run_two():
            for h, wsh in zip(handles, ws8):
                B.quant_act(x, xq=xq, xs=xs)
                B.linear_w8a8(h, xq, xs, out=y, workspace=wsh)

        res = {}
        for key, fn in (("dynamic", run_dynamic), ("two_calls", run_two)):
            g = graph_of(torch, fn)
            settle(torch, g.replay, 0.3)
            st = replay_stats(torch, g, 100, copies)
            res[key] = st
            del g
        alg = N * K + 2 * grid + 4 * M * K + 2 * M * N
        out["by_M"][f"M{M}"] = dict(
            dynamic_us=res["dynamic"]["median"] * 1e3, dynamic_p10=res["dynamic"]["p10"] * 1e3,
            dynamic_p90=res["dynamic"]["p90"] * 1e3, two_calls_us=res["two_calls"]["median"] * 1e3,
            launches=res["dynamic"]["launches"], algorithmic_bytes=alg,
            gbs=alg / (res["dynamic"]["mean"] * 1e-3) / 1e9, describe=handles[0].describe(B.ARM_W8A8_DYNAMIC, M))
    del handles
    torch.cuda.empty_cache()
    return out


def cpu_baseline_large(synth, tokens=8192, reps=3):
    """The oracle on the host cores on the headline step: the first ``tokens`` of the
    8192 tokens (all of them by default) quantized (NumPy float32, as defined) and
    multiplied against all 18432 rows of the weight (float64, the oracle's row-chunked
    form), ``reps`` times; the median time gives the rate."""
    import oracle as O
    wl = synth.config5()
    om = [(m.codes, m.scale_f32()) for m in wl.members]
    x = wl.x[:tokens]
    N = sum(m.codes.shape[0] for m in wl.members)
    K = x.shape[1]
    times, parts = [], {"quant": [], "gemm": []}
    for _ in range(reps):
        ta = time.perf_counter()
        xq, xs = O.quant_act(x)
        tb = time.perf_counter()
        for r0 in range(0, N, 1024):
            O.linear_w8a8_rows(xq, xs, om, list(range(r0, min(N, r0 + 1024))))
        tc = time.perf_counter()
        times.append(tc - ta)
        parts["quant"].append(tb - ta)
        parts["gemm"].append(tc - tb)
    t = statistics.median(times)
    flop = 2.0 * tokens * N * K
    threads, blas = _blas_info()
    return {"value": flop / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{tokens} of the {wl.x.shape[0]} tokens of the headline step (quantize + W8A8 GEMM over all {N} rows, "
                      f"K={K}), float32 quantizer and float64 GEMM in NumPy, median of {reps} repetitions "
                      f"({t:.2f} s each)",
            "parts_s_median": {k: round(statistics.median(v), 3) for k, v in parts.items()},
            "blas": blas, "host_cpus": os.cpu_count()}


def _blas_info():
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([d.get("num_threads", 1) for d in info if d.get("user_api") == "blas"] or [1])
        blas = ",".join(sorted({d.get("internal_api", "?") for d in info if d.get("user_api") == "blas"})) or "none"
    except Exception:
        threads, blas = os.cpu_count() or 1, "unknown"
    return int(threads), blas


def bench_dense_arm(torch, B, synth, dev):
    """The resident=False arm on grouped Q/K/V [6144|1000|1000, 5120]: the upcast
    (BF16 copy; three weight copies and three outputs used in turn, 375 MB, so
    HBM rather than the Infinity Cache serves them) and the dense product over
    the copy with BF16 activations at M = 128 and 512 (graphs of 20 calls)."""
    wl = synth.config4(512)
    w = B.BlockFP8Weight([to_device_member(torch, m, dev) for m in wl.members])
    N, K = w.n_total, w.K
    copies = [w] + [B.BlockFP8Weight([(t.clone(), sc.clone()) for t, sc in w.members]) for _ in range(2)]
    outs = [torch.empty((N, K), dtype=torch.bfloat16, device=dev) for _ in copies]

    def up():
        for c, o in zip(copies, outs):
            B.upcast(c, out=o)
    g_up = graph_of(torch, up, 7)
    settle(torch, g_up.replay, 0.3)
    su = replay_stats(torch, g_up, 20, 7 * len(copies))
    grid = sum(-(-m.codes.shape[0] // 128) * -(-K // 128) for m in wl.members)
    up_bytes = N * K * 3 + 2 * grid
    del g_up
    wd = outs[0]
    x = torch.from_numpy(wl.x).to(dev).to(torch.bfloat16)
    gemm = {}
    for M in (128, 512):
        xm = x[:M]
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        need = B.dense_workspace_size(N, K, M)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        g = graph_of(torch, lambda: B.linear_dense(wd, xm, out_dtype=torch.bfloat16, out=y, workspace=ws), 20)
        settle(torch, g.replay, 0.3)
        st = replay_stats(torch, g, 20, 20)
        flop = 2.0 * M * N * K
        gemm[f"M{M}"] = dict(us=st["median"] * 1e3, us_p10=st["p10"] * 1e3, us_p90=st["p90"] * 1e3,
                             launches=st["launches"], tflops=flop / (st["median"] * 1e-3) / 1e12,
                             describe=w.describe(B.ARM_DENSE, M))
        del g
    del copies, outs
    return dict(upcast_us=su["median"] * 1e3, upcast_us_p10=su["p10"] * 1e3, upcast_us_p90=su["p90"] * 1e3,
                upcast_launches=su["launches"], upcast_gbs=up_bytes / (su["median"] * 1e-3) / 1e9,
                upcast_bytes=up_bytes, gemm=gemm)


def read_sweep(torch, B, dev):
    """What a single launch that moves N bytes achieves, for N from 8 MB to 416 MB read:
    bsf8_read_stream (all loads of a block issued at once), PyTorch's float32 sum (its
    reduction kernel) and a device copy (N read + N written, counted as 2N), each over
    enough distinct copies (>= 640 MiB in rotation) that
    the Infinity Cache cannot serve them; per-launch device time from graphs of
    back-to-back launches.  A fit t = t0 + N / R separates the fixed cost of a launch
    from the streaming rate."""
    sizes_mb = (8, 16, 26.2144, 52.4288, 104.8576, 209.7152, 419.4304)
    sink = torch.zeros(B.READ_STREAM_SINK_WORDS, dtype=torch.int32, device=dev)
    res = {}
    for kname in ("bsf8_read_stream", "torch_float32_sum", "torch_copy_read_plus_write"):
        pts = []
        for mb in sizes_mb:
            n = int(mb * 1e6) // 16 * 16
            copies = max(2, -(-ROTATE_BYTES // n))
            bufs = [torch.empty(n // 4, dtype=torch.float32, device=dev).fill_(i * 1e-3) for i in range(copies)]
            outs = torch.empty(copies, dtype=torch.float32, device=dev)
            if kname == "bsf8_read_stream":
                def run():
                    for b in bufs:
                        B.read_stream(b, sink)
            elif kname == "torch_float32_sum":
                def run():
                    for i, b in enumerate(bufs):
                        torch.sum(b, dim=0, out=outs[i])
            else:
                # a device copy reads n and writes n bytes: timed per n read (the rate counts both)
                dst = torch.empty_like(bufs[0])

                def run():
                    for b in bufs:
                        dst.copy_(b)
            g = graph_of(torch, run)
            settle(torch, g.replay, 0.2)
            st = replay_stats(torch, g, 30, copies)
            pts.append((n * (2 if kname == "torch_copy_read_plus_write" else 1), st["median"] * 1e-3))
            del g, bufs
            torch.cuda.empty_cache()
        # least-squares fit of t = t0 + n / R
        xs = np.array([p[0] for p in pts], np.float64)
        ts = np.array([p[1] for p in pts], np.float64)
        A = np.vstack([np.ones_like(xs), xs]).T
        (t0, inv_r), *_ = np.linalg.lstsq(A, ts, rcond=None)
        res[kname] = {"points": [{"mb": round(n / 1e6, 2), "us": round(t * 1e6, 2), "gbs": round(n / t / 1e9, 1),
                                  "frac_hbm": round(n / t / 1e9 / HBM_PEAK_GBS, 4)} for n, t in pts],
                      "fit_t0_us": round(t0 * 1e6, 2), "fit_rate_gbs": round(1.0 / inv_r / 1e9, 1)}
        log(f"read sweep {kname}: {res[kname]}")
    return res


def copy_calibration(torch, dev):
    """A plain streaming kernel of known traffic, run three times, so an HBM counter run can scale
    FETCH_SIZE / WRITE_SIZE: y = 2 * x over 2^28 float32 (reads 1 GiB, writes 1 GiB per launch)."""
    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        torch.mul(a, 2.0, out=b)
    torch.cuda.synchronize()
    return dict(kernel="elementwise mul, 2^28 float32", bytes_read_per_launch=4 * n, bytes_written_per_launch=4 * n,
                launches=3)


def main():
    a = parse()
    if a.no_clock_sample:
        os.environ["BSF8_BENCH_NO_CLOCK_SAMPLE"] = "1"
    if a.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus above 1 is not supported (how the path would shard is described with the design)"}))
        sys.exit(2)
    import torch
    import block_scaled_fp8_linear_amd as B
    import synth
    B.lib()  # fail loudly when the HIP library is missing: there is no CPU path
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} {props.gcnArchName} CUs={props.multi_processor_count}")
    if a.read_sweep:
        print(json.dumps({"read_sweep": read_sweep(torch, B, dev), "device": props.gcnArchName}), flush=True)
        return

    big = bench_large_step(torch, B, synth, a.steps, a.warmup, dev)
    log(f"large prefill step {big['ms_per_step']:.4f} ms, gemm {big['gemm_us_stats']}")
    torch.cuda.empty_cache()
    extra = {}
    if not a.skip_extra:
        extra["ffn"] = bench_prefill(torch, B, synth, a.steps, a.warmup, dev)
        log(f"dense FFN step {extra['ffn']['ms_per_step']:.4f} ms, kernels {extra['ffn']['kernels_ms']}")
        torch.cuda.empty_cache()
        c2 = synth.config2(8)
        extra["decode_gemv"] = bench_w8a16_rotating(torch, B, c2.members, c2.x, (1, 4, 8), dev, "decode 5120x5120")
        log(f"decode {extra['decode_gemv']['by_M']}")
        c2b = synth.config2(8, shape=(5000, 4000))
        extra["decode_gemv_5000x4000"] = bench_w8a16_rotating(torch, B, c2b.members, c2b.x, (1, 4, 8), dev,
                                                              "decode 5000x4000")
        c4 = synth.config4(1)
        extra["qkv_decode"] = bench_w8a16_rotating(torch, B, c4.members, c4.x, (1,), dev, "grouped QKV decode")
        extra["qkv_w8a8_decode"] = bench_w8a8_rotating(torch, B, c4.members, c4.x, dev, "grouped QKV W8A8 M=1")
        extra["qkv_w8a8_dynamic"] = bench_w8a8_dynamic_rotating(torch, B, c4.members, c4.x, (1,), dev,
                                                                "grouped QKV W8A8 dynamic")
        dn = synth.config3_down(1)
        extra["down_decode"] = bench_w8a16_rotating(torch, B, dn.members, dn.x, (1,), dev, "FFN down decode")
        extra["down_w8a8_decode"] = bench_w8a8_rotating(torch, B, dn.members, dn.x, dev, "FFN down W8A8 M=1")
        extra["down_w8a8_dynamic"] = bench_w8a8_dynamic_rotating(torch, B, dn.members, dn.x, (1,), dev,
                                                                 "FFN down W8A8 dynamic")
        del dn
        extra["qkv_prefill"] = bench_qkv_prefill(torch, B, synth, dev)
        extra["qkv_w8a16_m512"] = bench_qkv_w8a16_m512(torch, B, synth, dev)
        torch.cuda.empty_cache()
        extra["dense_arm"] = bench_dense_arm(torch, B, synth, dev)
        log(f"dense arm {extra['dense_arm']}")
    if a.copy_calibration:
        extra["copy_calibration"] = copy_calibration(torch, dev)
    cpu = None if a.skip_cpu else cpu_baseline_large(synth)

    achieved = big["flop"] / (big["gemm_ms"] * 1e-3) / 1e12
    line = {
        "metric": "W8A8 block-FP8 prefill GEMM TFLOP/s (% FP8 MFMA peak); decode GEMV HBM GB/s",
        "value": round(big["flop"] / (big["ms_per_step"] * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(big["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": "large_prefill: quantize X [8192,7168] per token 1x128 + W8A8 GEMM "
                               "M=8192 K=7168 N=18432 (heavy-tailed block scales), bf16 out",
                   "M": big["M"], "N": big["N"], "K": big["K"], "global_batch": big["M"],
                   "parallelism": "single_gpu", "act_scale_layout": "K-major (token index contiguous)"},
        "roofline": {"bound": "mfma", "kernel": "w8a8_gemm_fast (large prefill)", "achieved": round(achieved, 2),
                     "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
                     "traffic": profiled_traffic("w8a8_gemm_large_prefill_m8192"),
                     "algorithmic": "2*M*N*K FLOP per launch over the launch's mean device time"},
        "cpu_baseline": cpu,
        "kernels_us_stats": {"gemm": big["gemm_us_stats"], "quant": big["quant_us_stats"]},
        "quant_gbs": round(big["quant_gbs"], 1),
        "rotated": {"note": "three weight copies used in turn (396 MB > the 256 MB Infinity Cache)",
                    "gemm_us_stats": big["rotated_gemm_us_stats"],
                    "tflops": round(big["flop"] / (big["rotated_gemm_us_stats"]["mean"] * 1e-6) / 1e12, 2)},
        "device": {"name": props.name, "arch": props.gcnArchName, "compute_units": props.multi_processor_count,
                   "sclk_under_load": big["sclk"]},
        "path": big["describe"],
        "timing": "HIP graph replays bracketed by HIP events on the replay stream: one replay per step; "
                  "kernel times from graphs of back-to-back launches",
        "fixture_sha256": big["fixture_sha256"],
    }

    if "ffn" in extra:
        pre = extra["ffn"]
        gu_ms = pre["kernels_ms"]["gemm_gate_up"]
        dn_ms = pre["kernels_ms"]["gemm_down"]
        line["dense_ffn_prefill"] = {
            "workload": "quant + W8A8 gate/up [2x17408,5120] + quant + W8A8 down [5120,17408], M=1024, bf16 out",
            "ms_per_step": round(pre["ms_per_step"], 4), "tflops": round(pre["tflops"], 2),
            "kernels_us_stats": pre["kernels_us_stats"],
            "gemm_gate_up": {"tflops": round(pre["gemm_gate_up_tflops"], 2),
                             "frac": round(pre["gemm_gate_up_tflops"] / FP8_PEAK_TFLOPS, 4),
                             "traffic": profiled_traffic("w8a8_gemm_gate_up_m1024")},
            "gemm_down": {"tflops": round(pre["gemm_down_tflops"], 2),
                          "frac": round(pre["gemm_down_tflops"] / FP8_PEAK_TFLOPS, 4),
                          "traffic": profiled_traffic("w8a8_gemm_down_m1024")},
            "roofline": {"bound": "mfma", "kernel": "w8a8_gemm (gate/up, with its split-K reduction)",
                         "achieved": round(pre["flop_gate_up"] / (gu_ms * 1e-3) / 1e12, 2), "peak": FP8_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(pre["flop_gate_up"] / (gu_ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
                         "traffic": profiled_traffic("w8a8_gemm_gate_up_m1024")},
            "quant_gbs": {"gate_up": round(pre["quant_gate_up_gbs"], 1), "down": round(pre["quant_down_gbs"], 1)},
            "path": {"gate_up": pre["describe_gate_up"], "down": pre["describe_down"]},
            "rotated": {"note": "two copies of both weights, used in turn (534 MB > the 256 MB Infinity Cache)",
                        "ms_per_step": round(pre["rotated"]["ms_per_step"], 4),
                        "tflops": round(pre["rotated"]["tflops"], 2),
                        "gemm_gate_up_tflops": round(pre["rotated"]["gemm_gate_up_tflops"], 2),
                        "gemm_down_tflops": round(pre["rotated"]["gemm_down_tflops"], 2),
                        "kernels_us_stats": pre["rotated"]["kernels_us_stats"]},
            "ffn_chain": {"note": "quant -> W8A8 gate/up -> quant_glu (silu(gate)*up quantized in one pass) -> "
                                  "W8A8 down: the down input is the gate/up output",
                          "ms_per_step": round(pre["ffn_chain"]["ms_per_step"], 4),
                          "tflops": round(pre["ffn_chain"]["tflops"], 2),
                          "quant_glu": {"us": round(pre["ffn_chain"]["glu_us"], 2),
                                        "p10": round(pre["ffn_chain"]["glu_us_p10"], 2),
                                        "p90": round(pre["ffn_chain"]["glu_us_p90"], 2),
                                        "launches": pre["ffn_chain"]["glu_launches"],
                                        "gbs": round(pre["ffn_chain"]["glu_gbs"], 1),
                                        "bytes": pre["ffn_chain"]["glu_bytes"],
                                        "frac_hbm": round(pre["ffn_chain"]["glu_gbs"] / HBM_PEAK_GBS, 4),
                                        "traffic": profiled_traffic("quant_glu_ffn_m1024")}},
            "fixture_sha256": pre["fixture_sha256"],
        }
        del gu_ms, dn_ms

    def decode_line(d, roofline_traffic=None):
        bm = d["by_M"]
        last = sorted(bm)[-1]
        r = {"workload": d["workload"], "unit": "GB/s", "by_M": {k: round(v["gbs"], 1) for k, v in bm.items()},
             "us_by_M": {k: {"median": round(v["us"], 2), "p10": round(v["us_p10"], 2), "p90": round(v["us_p90"], 2),
                             "launches": v["launches"]} for k, v in bm.items()},
             "read_stream_context": {k: round(v, 1) for k, v in d["read_stream_context"].items() if k != "kernel"},
             "path": bm[last]["describe"],
             "frac_hbm_by_M": {k: round(v["gbs"] / HBM_PEAK_GBS, 4) for k, v in bm.items()},
             "path_by_M": {k: v["describe"].split("|")[1].strip() for k, v in bm.items()}}
        r["roofline"] = {"bound": "hbm", "kernel": f"w8a16 ({last})", "achieved": round(bm[last]["gbs"], 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(bm[last]["gbs"] / HBM_PEAK_GBS, 4),
                         "traffic": roofline_traffic}
        return r

    if "decode_gemv" in extra:
        line["decode_gemv"] = decode_line(extra["decode_gemv"], profiled_traffic("w8a16_decode_5120x5120"))
        line["decode_gemv_5000x4000"] = decode_line(extra["decode_gemv_5000x4000"],
                                                    profiled_traffic("w8a16_decode_5000x4000"))
        line["qkv_decode"] = decode_line(extra["qkv_decode"], profiled_traffic("w8a16_decode_qkv_m1"))
        d = extra["qkv_w8a8_decode"]
        line["qkv_w8a8_decode"] = {
            "workload": d["workload"], "us": round(d["us"], 2), "p10": round(d["us_p10"], 2),
            "p90": round(d["us_p90"], 2), "launches": d["launches"], "path": d["describe"],
            "roofline": {"bound": "hbm", "kernel": d["describe"].split("|")[1].split()[0] + " (M=1)",
                         "achieved": round(d["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(d["gbs"] / HBM_PEAK_GBS, 4), "traffic": profiled_traffic("w8a8_qkv_m1"),
                         "algorithmic_bytes": d["algorithmic_bytes"]}}
        d = extra["qkv_w8a8_dynamic"]
        d1 = d["by_M"]["M1"]
        line["qkv_w8a8_dynamic_decode"] = {
            "workload": d["workload"],
            "by_M": {k: {"dynamic_us": round(v["dynamic_us"], 2), "p10": round(v["dynamic_p10"], 2),
                         "p90": round(v["dynamic_p90"], 2), "two_calls_us": round(v["two_calls_us"], 2),
                         "launches": v["launches"], "path": v["describe"]} for k, v in d["by_M"].items()},
            "roofline": {"bound": "hbm", "kernel": "w8a16_m1<quantizing> (M=1, quantization inside)",
                         "achieved": round(d1["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(d1["gbs"] / HBM_PEAK_GBS, 4), "traffic": profiled_traffic("w8a8_dyn_qkv_m1"),
                         "algorithmic_bytes": d1["algorithmic_bytes"]}}
        line["ffn_down_decode"] = decode_line(extra["down_decode"], profiled_traffic("w8a16_decode_down_m1"))
        d = extra["down_w8a8_dynamic"]["by_M"]["M1"]
        line["ffn_down_w8a8_dynamic_decode"] = {
            "workload": extra["down_w8a8_dynamic"]["workload"], "dynamic_us": round(d["dynamic_us"], 2),
            "p10": round(d["dynamic_p10"], 2), "p90": round(d["dynamic_p90"], 2),
            "two_calls_us": round(d["two_calls_us"], 2), "launches": d["launches"], "path": d["describe"],
            "roofline": {"bound": "hbm", "kernel": "w8a16_m1_ring<quantizing> (M=1, quantization inside)",
                         "achieved": round(d["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(d["gbs"] / HBM_PEAK_GBS, 4), "traffic": profiled_traffic("w8a8_dyn_down_m1"),
                         "algorithmic_bytes": d["algorithmic_bytes"]}}
        d = extra["down_w8a8_decode"]
        line["ffn_down_w8a8_decode"] = {
            "workload": d["workload"], "us": round(d["us"], 2), "p10": round(d["us_p10"], 2),
            "p90": round(d["us_p90"], 2), "launches": d["launches"], "path": d["describe"],
            "roofline": {"bound": "hbm", "kernel": "w8a8 streaming (M=1)", "achieved": round(d["gbs"], 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(d["gbs"] / HBM_PEAK_GBS, 4),
                         "traffic": profiled_traffic("w8a8_decode_down_m1"), "algorithmic_bytes": d["algorithmic_bytes"]}}
        q = extra["qkv_prefill"]
        line["qkv_prefill"] = {k: (round(v, 2) if isinstance(v, float) else v) for k, v in q.items()}
        line["qkv_prefill"]["roofline"] = {"bound": "mfma", "kernel": "w8a8_gemm (QKV, M=512)",
                                           "achieved": round(q["tflops"], 2), "peak": FP8_PEAK_TFLOPS,
                                           "unit": "TFLOP/s", "frac": round(q["tflops"] / FP8_PEAK_TFLOPS, 4),
                                           "traffic": profiled_traffic("w8a8_gemm_qkv_m512")}
        q16 = extra["qkv_w8a16_m512"]
        line["qkv_w8a16_m512"] = {
            "workload": q16["workload"], "us": round(q16["us"], 2), "p10": round(q16["us_p10"], 2),
            "p90": round(q16["us_p90"], 2), "launches": q16["launches"], "path": q16["describe"],
            "roofline": {"bound": "mfma", "kernel": "w8a16_gemm (LDS-staged 256x64 tiles, M=512)",
                         "achieved": round(q16["tflops"], 2), "peak": round(BF16_PEAK_TFLOPS / 3, 1), "unit": "TFLOP/s",
                         "frac": round(q16["tflops"] / (BF16_PEAK_TFLOPS / 3), 4),
                         "traffic": profiled_traffic("w8a16_gemm_qkv_m512"),
                         "peak_note": "exact F32 activations as three BF16 terms: a third of the published BF16 MFMA "
                                      "peak; v_mfma_f32_16x16x32_bf16 itself issues once per 28-32 cycles per SIMD "
                                      "(1.1-1.27 PFLOP/s measured), half the published rate"}}
    if "dense_arm" in extra:
        d = extra["dense_arm"]
        g512 = d["gemm"]["M512"]
        line["dense_arm"] = {
            "workload": "resident=False arm, grouped QKV [6144|1000|1000, 5120]: upcast to BF16, then BF16 x BF16 "
                        "product with BF16 activations, bf16 out",
            "upcast": {"us": round(d["upcast_us"], 2), "p10": round(d["upcast_us_p10"], 2),
                       "p90": round(d["upcast_us_p90"], 2), "launches": d["upcast_launches"],
                       "gbs": round(d["upcast_gbs"], 1), "bytes": d["upcast_bytes"],
                       "frac_hbm": round(d["upcast_gbs"] / HBM_PEAK_GBS, 4),
                       "note": "1 B read + 2 B written per element (+ grid); three weight copies used in turn"},
            "gemm": {k: {"us": round(v["us"], 2), "p10": round(v["us_p10"], 2), "p90": round(v["us_p90"], 2),
                         "launches": v["launches"], "tflops": round(v["tflops"], 2), "path": v["describe"]}
                     for k, v in d["gemm"].items()},
            "roofline": {"bound": "mfma", "kernel": "dense_gemm (M512; traffic of the GEMM kernel, its split-K "
                                                    "reduction not included)", "achieved": round(g512["tflops"], 2),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(g512["tflops"] / BF16_PEAK_TFLOPS, 4),
                         "traffic": profiled_traffic("dense_gemm_qkv_m512")}}
    if "copy_calibration" in extra:
        line["copy_calibration"] = extra["copy_calibration"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
