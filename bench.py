#!/usr/bin/env python3
"""Throughput of the SVDQuant W4A4 + low-rank hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  (a) svdq_quantize_act  on the MLP up projection, M=4608 tokens, K=3072, r=32
  (b) svdq_linear_w4a4   M=4608, K=3072, N=12288, r=32 (int8 MFMA + fused bf16 low-rank epilogue)
  (c) awq_linear_w4a16   adaLN modulation projection, M=16, K=3072, N=18432
Inputs are resident in HBM before timing starts. Buffer sets rotate so that every step reads
its activations / W4A16 weights from HBM rather than the 256 MB Infinity Cache.

Prints one JSON line. ``value`` = algorithmic operations of the step / step time, in TOPS
(int8-MFMA ops 2MNK of (b) + bf16 low-rank flops 2Mr(K+N) + W4A16 flops 2MNK of (c)).
``roofline`` covers the dominant kernel (b): 2MNK / its median launch time, against the MI355X
dense int8 MFMA peak. The timed region holds no event; after it, ``--gemm-samples`` more steps
(default 200) each bracket their GEMM with HIP events on the launch stream, so the GEMM is sampled
in the same context as in the timed steps. The per-kernel rates of (a) and (c), and the GEMM
alone, are measured before the warmup steps (after one pass of the step over every buffer set),
each kernel back to back over the rotating buffers; that work also brings the GPU to its working
clock, so a short timed region after a few warmup steps measures the steady state.

``--all-configs`` reports every configuration (attn, up, down, QKV at r = 32/128/256, W4A16) and
the unit microbenchmarks (pure matrix-core and vector rates at the observed clock);
``--unit-peaks`` only the microbenchmarks; ``--only gemm|quant|awq`` launches one kernel of the
default workload ``--steps`` times (for hardware-counter runs).

``--naive-vs-fused`` instead measures the engine-design figure's panel (a) claim on this GPU (a
rank-32 low-rank branch run naively, with a separate down projection that reads the 16-bit input
again and a separate up projection that writes the 16-bit output again, costs 57% extra latency on
the pages' hardware): the 4-bit branch alone (r = 0 kernels), the naive branch (r = 0 kernels plus
torch/hipBLASLt bf16 GEMMs for X L1 and Y + T L2) and the fused kernels, and prints one JSON line
with the three step times.

``--mlp-pair`` times the FLUX MLP pair chained on real intermediates: the up projection (M4608,
3072 -> 12288, r32) with the tanh-form GELU fused into its epilogue, then the down projection
(12288 -> 3072, r32) quantizing that output; the pair fused across its boundary (the up
projection's epilogue also runs the down layer's activation step, then the partial-sum reduction
and the down GEMM); and the same chain with the GELU run as a separate bf16 pass (torch) between
the two layers. It prints one JSON line.

``--rank-sweep`` times the quantizer and the GEMM of the fused QKV projection (M4608, K3072,
N9216) at r = 0, 32, 128 and 256, beside the unfused down projection in torch.

``--mxfp4`` times the MXFP4 variant of the layer (quantizer, GEMM on the scaled FP4 matrix
instruction, layer) beside the INT4 layer on ``--config``.

``--qkv-epilogue`` times the fused QKV projection of FLUX attention (M4608, 3072 -> 3 x 24 heads x
128, r32) with the per-head RMS norm of Q and K and the rotary embedding in the GEMM epilogue,
against the plain projection followed by the same norm + rotation in torch (bf16 in and out).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5033.2     # 256 CU x 2.4 GHz x 8192 int8 ops / clk / CU (published 5.0 POP/s dense)
HBM_PEAK_GBS = 8000.0
METRIC = "W4A4+low-rank linear TOPS (M4608 K3072 N12288 r32) & % int8 MFMA peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--rotate", type=int, default=10, help="buffer sets cycled through (>256 MB total)")
    ap.add_argument("--config", default="up", help="W4A4 workload from synth.CONFIGS")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4608, help="token rows in the CPU-oracle sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="repeat the oracle sample for this long")
    ap.add_argument("--naive-vs-fused", action="store_true",
                    help="time the 4-bit branch alone, the naive unfused low-rank branch and the fused kernels")
    ap.add_argument("--mlp-pair", action="store_true",
                    help="time the up (+GELU) -> down MLP pair, GELU fused vs a separate GELU pass")
    ap.add_argument("--qkv-epilogue", action="store_true",
                    help="time the fused QKV projection with the Q/K norm + rotary epilogue vs torch after it")
    ap.add_argument("--rank-sweep", action="store_true",
                    help="time the quantizer and the GEMM of the QKV projection at ranks 0, 32, 128 and 256")
    ap.add_argument("--all-configs", action="store_true",
                    help="per-configuration throughput: quantizer, GEMM and layer of attn, up, down and the QKV "
                         "rank sweep (r32/128/256), the W4A16 projection, and the unit peaks at the observed clock")
    ap.add_argument("--unit-peaks", action="store_true",
                    help="only the execution-unit microbenchmarks (int8/bf16/f32 matrix core, f32 vector FMA)")
    ap.add_argument("--mxfp4", action="store_true",
                    help="the MXFP4 variant of the layer (quantizer, GEMM, layer) beside the INT4 layer, on --config")
    ap.add_argument("--only", choices=["gemm", "quant", "awq"], default=None,
                    help="launch one kernel of the default workload --steps times back to back (for counter runs)")
    ap.add_argument("--gemm-samples", type=int, default=200,
                    help="steps after the timed region whose GEMM is bracketed by HIP events (roofline samples)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before timing, run one plain device-to-device copy of this size (a known-traffic "
                         "kernel that scales the HBM byte counters)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# sources whose kernels a launch of the named unit runs (the W4A4 kernel body lives in a header)
KERNEL_SOURCES = {"w4a4_gemm.hip": ["w4a4_gemm_kernel.h", "w4a4_gemm.hip"]}


def kernel_source_hash(name: str) -> str:
    h = hashlib.sha256()
    for part in KERNEL_SOURCES.get(name, [name]):
        with open(os.path.join(ROOT, "quantized_gemm_amd", "csrc", part), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_file: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, when it was taken on the
    current kernel source (same hash); otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    h = kernel_source_hash(kernel_file)
    for line in open(path):
        parts = line.split()
        if len(parts) >= 4 and parts[0] == kernel_file and parts[1] == workload and parts[2] == h:
            return float(parts[3])
    return None


def cpu_baseline(cfg, awq_cfg, rows: int, seconds: float):
    """The oracle, as it stands, on a bounded sample of the same step (first ``rows`` tokens),
    repeated until ``seconds`` of CPU work have been timed; the mean pass is reported."""
    import oracle
    import synth
    from threadpoolctl import threadpool_info

    inp = synth.make_layer_inputs(cfg, M=rows)
    x = synth.f32_from_bf16_bits(inp["x"])
    w = synth.f32_from_bf16_bits(inp["w"])
    b = synth.f32_from_bf16_bits(inp["bias"])
    d = oracle.svdq_decompose(x, w, cfg.rank)          # offline preparation: not timed
    qw, sw = oracle.quantize_weights_w4a4(d["resid"])
    ainp = synth.make_layer_inputs(awq_cfg)
    ax = synth.f32_from_bf16_bits(ainp["x"])
    acodes, ascales = oracle.quantize_weights_w4a16(synth.f32_from_bf16_bits(ainp["w"]))
    passes, total = 0, 0.0
    while passes == 0 or (total < seconds and passes < 100):
        t0 = time.perf_counter()
        qa, sa, t = oracle.quantize_activations(x, d["inv"], d["l1_bf16"])
        oracle.svdq_linear(qa, sa, qw, sw, t, d["l2_bf16"], b)
        oracle.awq_linear(ax, acodes, ascales, None)
        total += time.perf_counter() - t0
        passes += 1
    dt = total / passes
    ops = 2.0 * rows * cfg.N * cfg.K + 2.0 * rows * cfg.rank * (cfg.K + cfg.N) + \
        2.0 * awq_cfg.M * awq_cfg.N * awq_cfg.K
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": int(threads), "kind": "oracle",
            "seconds_per_pass": round(dt, 4), "passes": passes,
            "sample": f"{rows} of {cfg.M} tokens of the {cfg.name} layer (activation quantization, float64 "
                      f"dequantized product, low-rank, bias) + the full W4A16 projection M={awq_cfg.M}, "
                      f"{passes} passes, mean"}


def batch_timing(fn, stream, launches=200, batches=10, warm=20):
    """Per-launch time (us) of ``fn(s)`` run back to back: ``warm`` untimed launches, then
    ``launches`` launches in ``batches`` equal batches, each between two HIP events on ``stream``;
    the statistics are over the batch means."""
    import torch
    for s in range(warm):
        fn(s)
    per = max(1, launches // batches)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(batches)]
    torch.cuda.synchronize()
    k = 0
    for a, b in evs:
        a.record(stream)
        for _ in range(per):
            fn(k)
            k += 1
        b.record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) / per * 1e3 for a, b in evs])
    return {"median": round(float(np.median(t)), 2), "min": round(float(t.min()), 2),
            "max": round(float(t.max()), 2), "mean": round(float(t.mean()), 2), "launches": per * batches}


def unit_peaks(dev, stream, blocks_per_cu=4):
    """Matrix-core and vector rates of this GPU from the microbenchmarks of include/svdq_bench.h:
    achieved rate, the shader clock it ran at (s_memtime / s_memrealtime), and the rate per CU and
    clock, for the int8 and bf16 matrix shapes, the float32 outer-product shape and the float32
    vector FMA; and the SIMD-cycles of int8 MFMAs and independent FMAs issued together in the
    W4A4 rescale's proportion, against the two parts added and overlapped. Cycles are SIMD-cycles
    per wave instruction over the whole launch (event time x clock / instructions per SIMD)."""
    import torch
    import quantized_gemm_amd as q
    props = torch.cuda.get_device_properties(dev)
    cus = props.multi_processor_count
    blocks = blocks_per_cu * cus
    clocks = torch.zeros((blocks, 2), dtype=torch.int64, device=dev)
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    out = {"compute_units": cus, "waves_per_simd": blocks_per_cu}
    for kind, (_, ops_per_inst) in q.SVDQ_BENCH_KINDS.items():
        iters = 4000 if kind == "mfma_i8_32x32x32" else 2000
        insts_per_iter = 64 if kind == "valu_fma_f32" else 16
        q.svdq_bench_unit_peak(kind, blocks, 10, clocks, sink, stream=stream)  # warm
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        q.svdq_bench_unit_peak(kind, blocks, iters, clocks, sink, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        t = a.elapsed_time(b) * 1e-3
        ops = float(blocks) * 4 * iters * insts_per_iter * ops_per_inst
        ck = clocks.cpu().numpy().astype(np.float64)
        ghz = float(np.median(ck[:, 0] / np.maximum(ck[:, 1], 1) * 0.1))
        rate = ops / t / 1e12
        out[kind] = {"T_per_s": round(rate, 2), "clock_GHz": round(ghz, 3),
                     "ops_per_clk_per_CU": round(rate * 1e12 / (ghz * 1e9) / cus, 1),
                     "cycles_per_wave_instruction": round(ghz * 1e9 * t / (iters * insts_per_iter * blocks * 4 /
                                                                          (4 * cus)), 2)}
    # (a block is 4 waves, one per SIMD: blocks_per_cu waves share each SIMD)
    # The mixed kind in the W4A4 rescale's proportion, 8 int8 MFMAs to 128 FMAs per wave: its
    # SIMD-cycles against the two parts run alone, added and overlapped.
    m8 = 8 * out["mfma_i8_32x32x32"]["cycles_per_wave_instruction"]
    f128 = 128 * out["valu_fma_f32"]["cycles_per_wave_instruction"]
    out["mix_i8_fma"] = {"cycles_per_8_mfma_and_128_fma": round(8 * out["mix_i8_fma"]["cycles_per_wave_instruction"], 1),
                         "parts_added": round(m8 + f128, 1), "parts_overlapped": round(max(m8, f128), 1),
                         "clock_GHz": out["mix_i8_fma"]["clock_GHz"]}
    return out


def naive_low_rank_layer(q, x, inv, l1s, l2, qw, sw, bias, qact, asc, y, stream=None):
    """The unfused form of the layer (engine-design figure, panel (a)): the 4-bit branch with the
    r = 0 kernels, a separate 16-bit down projection T = X (diag(inv) L1) that reads X again, and a
    separate up projection Y += T L2 in place, which reads and writes the 16-bit output again
    (torch bf16 GEMMs, float32 accumulation). l1s = bf16(diag(inv) L1) [K, r], l2 = bf16 L2 [r, N]."""
    import torch
    sh = None if stream is None else stream.cuda_stream
    t = torch.matmul(x, l1s)
    q.svdq_quantize_act(x, inv, None, qact, asc, None, stream=sh)
    q.svdq_linear_w4a4(qact, asc, qw, sw, None, None, bias, y, stream=sh)
    y.addmm_(t, l2)
    return y


def naive_vs_fused(args):
    import torch
    import synth
    import quantized_gemm_amd as q
    from quantized_gemm_amd import prep

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    q.load_library()
    q.svdq_check_device()
    cfg = synth.CONFIGS[args.config]
    M, K, N, r = cfg.M, cfg.K, cfg.N, cfg.rank
    assert r > 0, "the ablation needs a low-rank branch"
    log(f"[ablation] generating {cfg.name} M={M} K={K} N={N} r={r}")
    inp = synth.make_layer_inputs(cfg)
    d = prep.decompose(synth.f32_from_bf16_bits(inp["x"]), synth.f32_from_bf16_bits(inp["w"]), r)
    qw, sw = q.svdq_pack_weights(q.SVDQ_FMT_W4A4_F32SCALE, d["resid"])
    l1t, l2t = q.svdq_pack_lowrank(d["l1"], d["l2"])

    def bf16_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    R = max(1, args.rotate)
    xs = [bf16_dev(inp["x"]) for _ in range(R)]
    inv = torch.from_numpy(d["inv_smooth"]).to(dev)
    qw_d, sw_d = torch.from_numpy(qw).to(dev), torch.from_numpy(sw).to(dev)
    l1t_d, l2t_d = bf16_dev(l1t), bf16_dev(l2t)
    l1s = torch.from_numpy(d["inv_smooth"][:, None].astype(np.float64) * d["l1"]).to(dev).to(torch.bfloat16)
    l2 = torch.from_numpy(np.ascontiguousarray(d["l2"])).to(dev).to(torch.bfloat16)
    bias_d = bf16_dev(inp["bias"])
    qact = [torch.empty((K // 64, M, 32), dtype=torch.uint8, device=dev) for _ in range(R)]
    asc = [torch.empty((K // 64, M), dtype=torch.float32, device=dev) for _ in range(R)]
    tl = [torch.empty((M, r), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    y0 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def four_bit(s):
        k = s % R
        q.svdq_quantize_act(xs[k], inv, None, qact[k], asc[k], None, stream=sh)
        q.svdq_linear_w4a4(qact[k], asc[k], qw_d, sw_d, None, None, bias_d, y0, stream=sh)

    def naive(s):
        k = s % R
        naive_low_rank_layer(q, xs[k], inv, l1s, l2, qw_d, sw_d, bias_d, qact[k], asc[k], y, stream)

    def fused(s):
        k = s % R
        q.svdq_quantize_act(xs[k], inv, l1t_d, qact[k], asc[k], tl[k], stream=sh)
        q.svdq_linear_w4a4(qact[k], asc[k], qw_d, sw_d, tl[k], l2t_d, bias_d, y, stream=sh)

    def down_only(s):
        torch.matmul(xs[s % R], l1s)

    def up_only(s):
        y.addmm_(tl[s % R], l2)

    def timed(fn, n):
        for s in range(min(n, 20)):
            fn(s)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for s in range(n):
            fn(s)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e3

    n = max(1, args.steps)
    res = {}
    for name, fn in (("four_bit_only_us", four_bit), ("naive_us", naive), ("fused_us", fused),
                     ("down_projection_torch_us", down_only), ("up_projection_torch_us", up_only)):
        log(f"[ablation] {name}")
        res[name] = round(timed(fn, n), 2)
    out = {
        "metric": f"latency of the rank-{r} low-rank branch, naive (separate 16-bit down and up projections) "
                  f"vs fused ({cfg.name} M{M} K{K} N{N})",
        "unit": "us",
        "steps": n,
        "config": {"workload": f"svdq_w4a4 {cfg.name} M{M} K{K} N{N} r{r}", "rotating_buffer_sets": R},
        **res,
        "naive_overhead": round(res["naive_us"] / res["four_bit_only_us"] - 1.0, 4),
        "fused_overhead": round(res["fused_us"] / res["four_bit_only_us"] - 1.0, 4),
        "pages_naive_overhead": 0.57,
        "pages_context": "engine-design figure (a) of the Nunchaku README, NVIDIA GPU, rank 32",
    }
    print(json.dumps(out), flush=True)


def mlp_pair(args):
    import torch
    import synth
    import quantized_gemm_amd as q
    from quantized_gemm_amd import prep

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    q.load_library()
    q.svdq_check_device()
    cu, cd = synth.CONFIGS["up"], synth.CONFIGS["down"]
    M, D, F = cu.M, cu.K, cu.N
    assert cd.K == F and cd.N == D and cd.M == M

    def bf16_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    def layer(cfg):
        inp = synth.make_layer_inputs(cfg)
        d = prep.decompose(synth.f32_from_bf16_bits(inp["x"]), synth.f32_from_bf16_bits(inp["w"]), cfg.rank)
        qw, sw = q.svdq_pack_weights(q.SVDQ_FMT_W4A4_F32SCALE, d["resid"])
        l1t, l2t = q.svdq_pack_lowrank(d["l1"], d["l2"])
        return inp, {"inv": torch.from_numpy(d["inv_smooth"]).to(dev), "qw": torch.from_numpy(qw).to(dev),
                     "sw": torch.from_numpy(sw).to(dev), "l1t": bf16_dev(l1t), "l2t": bf16_dev(l2t),
                     "bias": bf16_dev(inp["bias"]), "r": cfg.rank, "K": cfg.K}

    log("[mlp pair] preparing the up and down layers")
    inp_u, up = layer(cu)
    _, dn = layer(cd)
    R = max(1, args.rotate)
    xs = [bf16_dev(inp_u["x"]) for _ in range(R)]

    def bufs(L, rows):
        return (torch.empty((L["K"] // 64, rows, 32), dtype=torch.uint8, device=dev),
                torch.empty((L["K"] // 64, rows), dtype=torch.float32, device=dev),
                torch.empty((rows, L["r"]), dtype=torch.bfloat16, device=dev))
    bu, bd = bufs(up, M), bufs(dn, M)
    h = torch.empty((M, F), dtype=torch.bfloat16, device=dev)
    y = torch.empty((M, D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def run(L, b, xin, out, act=None):
        q.svdq_quantize_act(xin, L["inv"], L["l1t"], *b, stream=sh)
        q.svdq_linear_w4a4(b[0], b[1], L["qw"], L["sw"], b[2], L["l2t"], L["bias"], out, stream=sh, activation=act)

    def fused(s):
        run(up, bu, xs[s % R], h, "gelu_tanh")
        run(dn, bd, h, y)

    ws = torch.empty(q.load_library().svdq_gelu_quant_workspace_bytes(M, F, dn["r"]), dtype=torch.uint8, device=dev)

    def fused_quant(s):
        # the up projection's epilogue runs the down layer's activation step: H is never stored
        q.svdq_quantize_act(xs[s % R], up["inv"], up["l1t"], *bu, stream=sh)
        q.svdq_linear_w4a4_gelu_quant(bu[0], bu[1], up["qw"], up["sw"], bu[2], up["l2t"], up["bias"], dn["inv"],
                                      dn["l1t"], *bd, workspace=ws, stream=sh)
        q.svdq_linear_w4a4(bd[0], bd[1], dn["qw"], dn["sw"], bd[2], dn["l2t"], dn["bias"], y, stream=sh)

    def up_gelu_quant(s):
        q.svdq_quantize_act(xs[s % R], up["inv"], up["l1t"], *bu, stream=sh)
        q.svdq_linear_w4a4_gelu_quant(bu[0], bu[1], up["qw"], up["sw"], bu[2], up["l2t"], up["bias"], dn["inv"],
                                      dn["l1t"], *bd, workspace=ws, stream=sh)

    def separate(s):
        run(up, bu, xs[s % R], h)
        run(dn, bd, torch.nn.functional.gelu(h, approximate="tanh"), y)

    def up_plain(s):
        run(up, bu, xs[s % R], h)

    def up_gelu(s):
        run(up, bu, xs[s % R], h, "gelu_tanh")

    def gelu_pass(s):
        torch.nn.functional.gelu(h, approximate="tanh")

    def timed(fn, n):
        for s in range(min(n, 10)):
            fn(s)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for s in range(n):
            fn(s)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e3

    n = max(1, args.steps)
    res = {}
    for name, fn in (("pair_gelu_quant_fused_us", fused_quant), ("pair_gelu_fused_us", fused),
                     ("pair_gelu_separate_us", separate), ("up_plain_us", up_plain), ("up_gelu_fused_us", up_gelu),
                     ("up_gelu_quant_fused_us", up_gelu_quant), ("gelu_pass_torch_us", gelu_pass)):
        log(f"[mlp pair] {name}")
        res[name] = round(timed(fn, n), 2)
    ops = 2.0 * M * F * D * 2 + 2.0 * M * cu.rank * (D + F) + 2.0 * M * cd.rank * (F + D)
    out = {
        "metric": f"FLUX MLP pair (up {D}->{F} + GELU, down {F}->{D}, M{M}, r{cu.rank}) step time",
        "unit": "us",
        "steps": n,
        "config": {"workload": f"svdq_w4a4 up M{M} K{D} N{F} r{cu.rank} + gelu_tanh + down M{M} K{F} N{D} r{cd.rank}",
                   "rotating_buffer_sets": R},
        **res,
        "pair_TOPS_fused": round(ops / (res["pair_gelu_fused_us"] * 1e-6) / 1e12, 1),
        "pair_TOPS_gelu_quant_fused": round(ops / (res["pair_gelu_quant_fused_us"] * 1e-6) / 1e12, 1),
        "saved_by_quant_fusion_us": round(res["pair_gelu_fused_us"] - res["pair_gelu_quant_fused_us"], 2),
        "gelu_epilogue_cost_us": round(res["up_gelu_fused_us"] - res["up_plain_us"], 2),
        "saved_by_fusion_us": round(res["pair_gelu_separate_us"] - res["pair_gelu_fused_us"], 2),
    }
    print(json.dumps(out), flush=True)


def qkv_epilogue(args):
    import torch
    import synth
    import quantized_gemm_amd as q
    from quantized_gemm_amd import prep

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    q.load_library()
    q.svdq_check_device()
    cfg = synth.CONFIGS["qkv_r32"]
    M, K, N, r = cfg.M, cfg.K, cfg.N, cfg.rank
    heads, D = N // (3 * 128), 128
    log(f"[qkv] preparing M={M} K={K} N={N} ({heads} heads) r={r}")
    inp = synth.make_layer_inputs(cfg)
    d = prep.decompose(synth.f32_from_bf16_bits(inp["x"]), synth.f32_from_bf16_bits(inp["w"]), r)
    qw, sw = q.svdq_pack_weights(q.SVDQ_FMT_W4A4_F32SCALE, d["resid"])
    l1t, l2t = q.svdq_pack_lowrank(d["l1"], d["l2"])

    def bf16_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    x = bf16_dev(inp["x"])
    inv = torch.from_numpy(d["inv_smooth"]).to(dev)
    qw_d, sw_d, l1t_d, l2t_d = torch.from_numpy(qw).to(dev), torch.from_numpy(sw).to(dev), bf16_dev(l1t), bf16_dev(l2t)
    bias = bf16_dev(inp["bias"])
    rng = np.random.default_rng(5)
    q_w = torch.from_numpy(rng.uniform(0.5, 1.5, D).astype(np.float32)).to(dev)
    k_w = torch.from_numpy(rng.uniform(0.5, 1.5, D).astype(np.float32)).to(dev)
    ang = np.arange(M)[:, None] * 10000.0 ** (-np.arange(64) / 64.0)[None, :]
    cs = torch.from_numpy(np.cos(ang).astype(np.float32)).to(dev)
    sn = torch.from_numpy(np.sin(ang).astype(np.float32)).to(dev)
    qact, asc, t = q.svdq_quantize_act(x, inv, l1t_d)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def plain(s):
        q.svdq_linear_w4a4(qact, asc, qw_d, sw_d, t, l2t_d, bias, y, stream=sh)

    def fused(s):
        q.svdq_linear_w4a4_qkv(qact, asc, qw_d, sw_d, t, l2t_d, bias, heads, q_w, k_w, cs, sn, y, stream=sh)

    def torch_norm_rope(s):
        # what the unfused FLUX attention runs after the projection (float32 math, bf16 out)
        qk = y[:, :2 * heads * D].view(M, 2, heads, D).float()
        w = torch.stack([q_w, k_w])[None, :, None, :]
        u = qk * torch.rsqrt(qk.pow(2).mean(-1, keepdim=True) + 1e-6) * w
        a, b = u[..., 0::2], u[..., 1::2]
        c, s_ = cs[:, None, None, :], sn[:, None, None, :]
        out = torch.stack([a * c - b * s_, a * s_ + b * c], dim=-1).flatten(-2)
        return out.to(torch.bfloat16)

    def separate(s):
        plain(s)
        torch_norm_rope(s)

    def timed(fn, n):
        for s in range(min(n, 10)):
            fn(s)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for s in range(n):
            fn(s)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e3

    def paired(fa, fb, n):
        """A/B: the two launches alternate in one loop, each between its own pair of events, so
        both see the same clock and cache state (every event adds the same small cost to both)."""
        for s in range(10):
            fa(s)
            fb(s)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
        torch.cuda.synchronize()
        for s in range(n):
            evs[s][0].record(stream)
            fa(s)
            evs[s][1].record(stream)
            fb(s)
            evs[s][2].record(stream)
        torch.cuda.synchronize()
        ta = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e3
        tb = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) * 1e3
        return ta, tb

    n = max(1, args.steps)
    res = {}
    log("[qkv] plain / fused, interleaved")
    tp, tf = paired(plain, fused, n)
    res["plain_us"], res["fused_norm_rope_us"] = round(tp, 2), round(tf, 2)
    for name, fn in (("plain_then_torch_us", separate), ("torch_norm_rope_us", torch_norm_rope)):
        log(f"[qkv] {name}")
        res[name] = round(timed(fn, n), 2)
    out = {
        "metric": f"fused QKV projection with the Q/K RMS norm + rotary epilogue (M{M} K{K} N{N}, {heads} heads, r{r})",
        "unit": "us",
        "steps": n,
        "config": {"workload": f"svdq_w4a4 qkv_r32 M{M} K{K} N{N} r{r} + qk norm + rope"},
        **res,
        "epilogue_cost_us": round(res["fused_norm_rope_us"] - res["plain_us"], 2),
        "saved_by_fusion_us": round(res["plain_then_torch_us"] - res["fused_norm_rope_us"], 2),
    }
    print(json.dumps(out), flush=True)


def rank_sweep(args):
    """How the low-rank branch's cost grows with r on the fused QKV shape (M4608 K3072 N9216): the
    quantizer (down projection fused) and the GEMM (T·L2 epilogue fused), each timed back to back
    over rotating buffer sets, at r = 0 (the 4-bit product alone), 32, 128 and 256. The SVD of the
    smoothed weight is computed once and truncated per rank."""
    import torch
    import synth
    import quantized_gemm_amd as q
    from quantized_gemm_amd import prep

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    q.load_library()
    q.svdq_check_device()
    cfg = synth.CONFIGS["qkv_r32"]
    M, K, N = cfg.M, cfg.K, cfg.N
    ranks = (0, 32, 128, 256)
    log(f"[rank sweep] generating M={M} K={K} N={N}")
    inp = synth.make_layer_inputs(cfg)
    xf, wf = synth.f32_from_bf16_bits(inp["x"]), synth.f32_from_bf16_bits(inp["w"])

    def bf16_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    R = max(1, args.rotate)
    xs = [bf16_dev(inp["x"]) for _ in range(R)]
    bias_d = bf16_dev(inp["bias"])
    qact = [torch.empty((K // 64, M, 32), dtype=torch.uint8, device=dev) for _ in range(R)]
    asc = [torch.empty((K // 64, M), dtype=torch.float32, device=dev) for _ in range(R)]
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def timed(fn, n):
        for s in range(min(n, 20)):
            fn(s)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for s in range(n):
            fn(s)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e3

    n = max(1, args.steps)
    svd, rows = None, []
    for r in ranks:
        log(f"[rank sweep] r={r}: decomposing and packing")
        d = prep.decompose(xf, wf, r, svd=svd)
        svd = d["svd"] if d["svd"] is not None else svd
        qw, sw = q.svdq_pack_weights(q.SVDQ_FMT_W4A4_F32SCALE, d["resid"])
        inv = torch.from_numpy(d["inv_smooth"]).to(dev)
        qw_d, sw_d = torch.from_numpy(qw).to(dev), torch.from_numpy(sw).to(dev)
        if r:
            l1t, l2t = q.svdq_pack_lowrank(d["l1"], d["l2"])
            l1t_d, l2t_d = bf16_dev(l1t), bf16_dev(l2t)
            tl = [torch.empty((M, r), dtype=torch.bfloat16, device=dev) for _ in range(R)]
        else:
            l1t_d = l2t_d = None
            tl = [None] * R

        def quant(s, inv=inv, l1t_d=l1t_d, tl=tl):
            k = s % R
            q.svdq_quantize_act(xs[k], inv, l1t_d, qact[k], asc[k], tl[k], stream=sh)

        def gemm(s, qw_d=qw_d, sw_d=sw_d, l2t_d=l2t_d, tl=tl):
            k = s % R
            q.svdq_linear_w4a4(qact[k], asc[k], qw_d, sw_d, tl[k], l2t_d, bias_d, ys[k], stream=sh)

        quant(0)
        torch.cuda.synchronize()
        log(f"[rank sweep] r={r}: timing")
        tq, tg = timed(quant, n), timed(gemm, n)
        ops = 2.0 * M * N * K + 2.0 * M * r * (K + N)
        row = {"rank": r, "quantize_act_us": round(tq, 2), "linear_w4a4_us": round(tg, 2),
               "layer_us": round(tq + tg, 2), "gemm_tops": round(ops / (tg * 1e-6) / 1e12, 1)}
        if r:
            # context for the fused down projection: the same product unfused, X (bf16) @ (inv * L1)
            # in torch (rocBLAS/hipBLASLt), which the unfused layer would add to the r = 0 quantizer
            l1s = torch.from_numpy(d["inv_smooth"][:, None].astype(np.float64) * d["l1"]).to(dev).to(torch.bfloat16)
            row["down_projection_torch_us"] = round(timed(lambda s: torch.matmul(xs[s % R], l1s), n), 2)
            del l1s
        rows.append(row)
        del quant, gemm, tl, qw_d, sw_d, l1t_d, l2t_d
    base = rows[0]
    for row in rows:
        row["low_rank_cost"] = round(row["layer_us"] / base["layer_us"] - 1.0, 4)
    out = {
        "metric": f"cost of the fused low-rank branch against its rank (QKV projection M{M} K{K} N{N})",
        "unit": "us",
        "steps": n,
        "config": {"workload": f"svdq_w4a4 qkv M{M} K{K} N{N} r0/32/128/256", "rotating_buffer_sets": R},
        "ranks": rows,
    }
    print(json.dumps(out), flush=True)


def quant_bytes(M, K, r):
    """Algorithmic bytes of kernel (a): X, codes, scales, T, the L1 operand and the smoothing vector."""
    return M * K * 2 + M * K // 2 + (K // 64) * M * 4 + M * r * 2 + r * K * 2 + K * 4


def gemm_bytes(M, K, N, r):
    """Algorithmic bytes of kernel (b): both code matrices, both scale arrays, T, L2, bias and Y."""
    return M * K // 2 + N * K // 2 + (K // 64) * (M + N) * 4 + M * r * 2 + N * r * 2 + N * 2 + M * N * 2


def awq_bytes(M, K, N):
    return N * K // 2 + (K // 64) * N * 2 + M * K * 2 + M * N * 2


def all_configs(args):
    """Throughput of every W4A4 configuration (attn, up, down, the QKV projection at r = 32, 128,
    256) and of the W4A16 projection, each kernel timed alone back to back over rotating buffer
    sets (10 batches of launches between HIP events; median, min and max of the batch means), and
    the layer (quantizer + GEMM alternating). Also the unit microbenchmarks, so that the GEMM is
    reported against both the published int8 peak and the matrix-core rate measured at the clock
    this GPU ran at."""
    import torch
    import synth
    import quantized_gemm_amd as q
    from quantized_gemm_amd import prep

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    q.load_library()
    q.svdq_check_device()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    n = max(20, args.steps)

    def bf16_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    log("[all] unit microbenchmarks")
    peaks = unit_peaks(dev, stream)
    i8 = peaks["mfma_i8_32x32x32"]
    rows = []
    svd_cache = {}
    for name, r in (("attn", 32), ("up", 32), ("down", 32), ("qkv_r32", 32), ("qkv_r32", 128), ("qkv_r32", 256)):
        cfg = synth.CONFIGS[name].with_rank(r) if name.startswith("qkv") else synth.CONFIGS[name]
        M, K, N = cfg.M, cfg.K, cfg.N
        log(f"[all] {cfg.name}: M={M} K={K} N={N} r={r}: preparing")
        base = name
        if base not in svd_cache:
            svd_cache.clear()
            inp = synth.make_layer_inputs(cfg)
            svd_cache[base] = (inp, synth.f32_from_bf16_bits(inp["x"]), synth.f32_from_bf16_bits(inp["w"]), None)
        inp, xf, wf, svd = svd_cache[base]
        d = prep.decompose(xf, wf, r, svd=svd)
        svd_cache[base] = (inp, xf, wf, d["svd"])
        qw, sw = q.svdq_pack_weights(q.SVDQ_FMT_W4A4_F32SCALE, d["resid"])
        l1t, l2t = q.svdq_pack_lowrank(d["l1"], d["l2"])
        ba, bb = quant_bytes(M, K, r), gemm_bytes(M, K, N, r)
        R = int(min(16, max(4, -(-600_000_000 // ba))))
        xs = [bf16_dev(inp["x"]) for _ in range(R)]
        inv = torch.from_numpy(d["inv_smooth"]).to(dev)
        qw_d, sw_d, l1t_d, l2t_d = (torch.from_numpy(qw).to(dev), torch.from_numpy(sw).to(dev), bf16_dev(l1t),
                                    bf16_dev(l2t))
        bias_d = bf16_dev(inp["bias"])
        qact = [torch.empty((K // 64, M, 32), dtype=torch.uint8, device=dev) for _ in range(R)]
        asc = [torch.empty((K // 64, M), dtype=torch.float32, device=dev) for _ in range(R)]
        tl = [torch.empty((M, r), dtype=torch.bfloat16, device=dev) for _ in range(R)]
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

        def quant(s):
            k = s % R
            q.svdq_quantize_act(xs[k], inv, l1t_d, qact[k], asc[k], tl[k], stream=sh)

        def gemm(s):
            k = s % R
            q.svdq_linear_w4a4(qact[k], asc[k], qw_d, sw_d, tl[k], l2t_d, bias_d, y, stream=sh)

        def layer(s):
            quant(s)
            gemm(s)

        for s in range(R):
            quant(s)
        torch.cuda.synchronize()
        log(f"[all] {cfg.name}: timing")
        tq = batch_timing(quant, stream, n)
        tg = batch_timing(gemm, stream, n)
        tlr = batch_timing(layer, stream, n)
        ops = 2.0 * M * N * K
        lr = 2.0 * M * r * (K + N)
        rows.append({
            "config": cfg.name, "M": M, "K": K, "N": N, "rank": r, "rotating_buffer_sets": R,
            "quantize_act_us": tq, "quantize_act_GBs": round(ba / (tq["median"] * 1e-6) / 1e9, 1),
            "quantize_act_hbm_frac": round(ba / (tq["median"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "linear_w4a4_us": tg, "linear_w4a4_TOPS": round(ops / (tg["median"] * 1e-6) / 1e12, 1),
            "linear_w4a4_frac_int8_peak": round(ops / (tg["median"] * 1e-6) / 1e12 / INT8_PEAK_TOPS, 4),
            "linear_w4a4_frac_measured_mfma": round(ops / (tg["median"] * 1e-6) / 1e12 / i8["T_per_s"], 4),
            "linear_w4a4_lowrank_GFLOP": round(lr / 1e9, 3),
            "linear_w4a4_alg_bytes": bb,
            "layer_us": tlr, "layer_TOPS": round((ops + lr) / (tlr["median"] * 1e-6) / 1e12, 1),
        })
        log(f"[all] {json.dumps(rows[-1])}")
        del xs, qact, asc, tl, y, qw_d, sw_d, l1t_d, l2t_d
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    acfg = synth.CONFIGS["awq"]
    ainp = synth.make_layer_inputs(acfg)
    aqw, ascl = q.svdq_pack_weights(q.SVDQ_FMT_W4A16_BF16SCALE, synth.f32_from_bf16_bits(ainp["w"]))
    bc = awq_bytes(acfg.M, acfg.K, acfg.N)
    R = int(min(32, max(4, -(-600_000_000 // bc))))
    ax = bf16_dev(ainp["x"])
    aqws = [torch.from_numpy(aqw).to(dev) for _ in range(R)]
    ascls = [bf16_dev(ascl) for _ in range(R)]
    ay = torch.empty((acfg.M, acfg.N), dtype=torch.bfloat16, device=dev)
    log("[all] awq: timing")
    tc = batch_timing(lambda s: q.awq_linear_w4a16(ax, aqws[s % R], ascls[s % R], None, ay, stream=sh), stream,
                      max(n, 500))
    awq = {"config": "awq", "M": acfg.M, "K": acfg.K, "N": acfg.N, "rotating_buffer_sets": R,
           "awq_linear_w4a16_us": tc, "GBs": round(bc / (tc["median"] * 1e-6) / 1e9, 1),
           "hbm_frac": round(bc / (tc["median"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "alg_bytes": bc}
    out = {"metric": "per-configuration throughput of the SVDQuant W4A4 + low-rank layer and the W4A16 projection",
           "unit_peaks": peaks, "int8_peak_published_TOPS": INT8_PEAK_TOPS, "hbm_peak_GBs": HBM_PEAK_GBS,
           "w4a4": rows, "w4a16": awq,
           "timing": "each kernel alone, back to back over rotating buffer sets; 10 batches between HIP events, "
                     "median / min / max / mean of the batch means (us per launch)"}
    print(json.dumps(out), flush=True)


FP4_PEAK_TOPS = 10066.3    # 256 CU x 2.4 GHz x 16384 FP4 ops / clk / CU (published 10.1 PFLOP/s dense)


def mxfp4_bench(args):
    """The 4-bit float (MXFP4) variant of the layer on one configuration (default: the MLP up
    projection): the quantizer, the GEMM (block scales applied inside the scaled FP4 matrix
    instruction) and the layer, each back to back over rotating buffer sets, beside the INT4 layer
    on the same problem. The GEMM is reported against the FP4 and the int8 dense peaks."""
    import torch
    import synth
    import quantized_gemm_amd as q
    from quantized_gemm_amd import prep

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    q.load_library()
    q.svdq_check_device()
    cfg = synth.CONFIGS[args.config]
    M, K, N, r = cfg.M, cfg.K, cfg.N, cfg.rank
    log(f"[mxfp4] {cfg.name} M={M} K={K} N={N} r={r}: preparing")
    inp = synth.make_layer_inputs(cfg)
    d = prep.decompose(synth.f32_from_bf16_bits(inp["x"]), synth.f32_from_bf16_bits(inp["w"]), r)
    qwm, swm = q.svdq_pack_weights(q.SVDQ_FMT_MXFP4_E8M0SCALE, d["resid"])
    qwi, swi = q.svdq_pack_weights(q.SVDQ_FMT_W4A4_F32SCALE, d["resid"])
    l1t, l2t = q.svdq_pack_lowrank(d["l1"], d["l2"])

    def bf16_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    R = int(min(16, max(4, -(-600_000_000 // quant_bytes(M, K, r)))))
    xs = [bf16_dev(inp["x"]) for _ in range(R)]
    inv = torch.from_numpy(d["inv_smooth"]).to(dev)
    qwm_d, swm_d = torch.from_numpy(qwm).to(dev), torch.from_numpy(swm).to(dev)
    qwi_d, swi_d = torch.from_numpy(qwi).to(dev), torch.from_numpy(swi).to(dev)
    l1t_d, l2t_d, bias_d = bf16_dev(l1t), bf16_dev(l2t), bf16_dev(inp["bias"])
    qa = [torch.empty((K // 64, M, 32), dtype=torch.uint8, device=dev) for _ in range(R)]
    sam = [torch.empty((K // 64, M, 2), dtype=torch.uint8, device=dev) for _ in range(R)]
    sai = [torch.empty((K // 64, M), dtype=torch.float32, device=dev) for _ in range(R)]
    tl = [torch.empty((M, r), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def quant_mx(s):
        k = s % R
        q.svdq_quantize_act_mxfp4(xs[k], inv, l1t_d, qa[k], sam[k], tl[k], stream=sh)

    def gemm_mx(s):
        k = s % R
        q.svdq_linear_mxfp4(qa[k], sam[k], qwm_d, swm_d, tl[k], l2t_d, bias_d, y, stream=sh)

    def quant_i4(s):
        k = s % R
        q.svdq_quantize_act(xs[k], inv, l1t_d, qa[k], sai[k], tl[k], stream=sh)

    def gemm_i4(s):
        k = s % R
        q.svdq_linear_w4a4(qa[k], sai[k], qwi_d, swi_d, tl[k], l2t_d, bias_d, y, stream=sh)

    n = max(20, args.steps)
    for s in range(R):
        quant_mx(s)
    torch.cuda.synchronize()
    log("[mxfp4] timing")
    tq, tg = batch_timing(quant_mx, stream, n), batch_timing(gemm_mx, stream, n)
    tl_mx = batch_timing(lambda s: (quant_mx(s), gemm_mx(s)), stream, n)
    for s in range(R):
        quant_i4(s)
    torch.cuda.synchronize()
    tqi, tgi = batch_timing(quant_i4, stream, n), batch_timing(gemm_i4, stream, n)
    tli = batch_timing(lambda s: (quant_i4(s), gemm_i4(s)), stream, n)
    ops = 2.0 * M * N * K
    lr = 2.0 * M * r * (K + N)
    mx_tops = ops / (tg["median"] * 1e-6) / 1e12
    out = {
        "metric": f"MXFP4 variant of the layer ({cfg.name} M{M} K{K} N{N} r{r})",
        "unit": "us", "steps": n, "rotating_buffer_sets": R,
        "mxfp4": {"quantize_act_us": tq, "linear_us": tg, "layer_us": tl_mx,
                  "linear_TOPS": round(mx_tops, 1), "frac_fp4_peak": round(mx_tops / FP4_PEAK_TOPS, 4),
                  "frac_int8_peak": round(mx_tops / INT8_PEAK_TOPS, 4),
                  "layer_TOPS": round((ops + lr) / (tl_mx["median"] * 1e-6) / 1e12, 1)},
        "int4": {"quantize_act_us": tqi, "linear_us": tgi, "layer_us": tli,
                 "linear_TOPS": round(ops / (tgi["median"] * 1e-6) / 1e12, 1),
                 "layer_TOPS": round((ops + lr) / (tli["median"] * 1e-6) / 1e12, 1)},
        "peaks_TOPS": {"fp4_dense": FP4_PEAK_TOPS, "int8_dense": INT8_PEAK_TOPS},
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer shards by tokens or output columns with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)

    if args.naive_vs_fused:
        naive_vs_fused(args)
        return
    if args.mlp_pair:
        mlp_pair(args)
        return
    if args.qkv_epilogue:
        qkv_epilogue(args)
        return
    if args.rank_sweep:
        rank_sweep(args)
        return
    if args.all_configs:
        all_configs(args)
        return
    if args.mxfp4:
        mxfp4_bench(args)
        return
    if args.unit_peaks:
        import torch
        import quantized_gemm_amd as q
        assert torch.cuda.is_available(), "bench.py needs a HIP device"
        q.load_library()
        q.svdq_check_device()
        dev, st = torch.device("cuda:0"), torch.cuda.current_stream()
        print(json.dumps({"unit_peaks": unit_peaks(dev, st),
                          "by_waves_per_simd": {w: unit_peaks(dev, st, w) for w in (1, 2)}}), flush=True)
        return

    import torch
    import synth
    import quantized_gemm_amd as q
    from quantized_gemm_amd import prep

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    q.load_library()
    q.svdq_check_device()

    cfg = synth.CONFIGS[args.config]
    awq_cfg = synth.CONFIGS["awq"]
    M, K, N, r = cfg.M, cfg.K, cfg.N, cfg.rank
    log(f"[bench] generating {cfg.name} M={M} K={K} N={N} r={r}")
    inp = synth.make_layer_inputs(cfg)
    x = synth.f32_from_bf16_bits(inp["x"])
    w = synth.f32_from_bf16_bits(inp["w"])
    t0 = time.time()
    d = prep.decompose(x, w, r)
    log(f"[bench] offline decomposition {time.time() - t0:.1f}s; packing")
    qw, sw = q.svdq_pack_weights(q.SVDQ_FMT_W4A4_F32SCALE, d["resid"])
    l1t, l2t = q.svdq_pack_lowrank(d["l1"], d["l2"]) if r else (None, None)
    ainp = synth.make_layer_inputs(awq_cfg)
    aqw, ascl = q.svdq_pack_weights(q.SVDQ_FMT_W4A16_BF16SCALE, synth.f32_from_bf16_bits(ainp["w"]))

    def bf16_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    R = max(1, args.rotate)
    xs = [bf16_dev(inp["x"]) for _ in range(R)]
    inv = torch.from_numpy(d["inv_smooth"]).to(dev)
    qw_d, sw_d = torch.from_numpy(qw).to(dev), torch.from_numpy(sw).to(dev)
    l1t_d = bf16_dev(l1t) if r else None
    l2t_d = bf16_dev(l2t) if r else None
    bias_d = bf16_dev(inp["bias"])
    qact = [torch.empty((K // 64, M, 32), dtype=torch.uint8, device=dev) for _ in range(R)]
    asc = [torch.empty((K // 64, M), dtype=torch.float32, device=dev) for _ in range(R)]
    tl = [torch.empty((M, r), dtype=torch.bfloat16, device=dev) if r else None for _ in range(R)]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ax = bf16_dev(ainp["x"])
    aqws = [torch.from_numpy(aqw).to(dev) for _ in range(R)]
    ascl_d = bf16_dev(ascl)
    ay = torch.empty((awq_cfg.M, awq_cfg.N), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def step(s, ev=None):
        k = s % R
        q.svdq_quantize_act(xs[k], inv, l1t_d, qact[k], asc[k], tl[k], stream=sh)
        if ev is not None:
            ev[0].record(stream)
        q.svdq_linear_w4a4(qact[k], asc[k], qw_d, sw_d, tl[k], l2t_d, bias_d, y, stream=sh)
        if ev is not None:
            ev[1].record(stream)
        q.awq_linear_w4a16(ax, aqws[k], ascl_d, None, ay, stream=sh)

    if args.only is not None:
        # one kernel of the step, --steps launches back to back (inputs from one pass of the step)
        step(0)
        torch.cuda.synchronize()
        fn = {"gemm": lambda s: q.svdq_linear_w4a4(qact[s % R], asc[s % R], qw_d, sw_d, tl[s % R], l2t_d, bias_d, y,
                                                   stream=sh),
              "quant": lambda s: q.svdq_quantize_act(xs[s % R], inv, l1t_d, qact[s % R], asc[s % R], tl[s % R],
                                                     stream=sh),
              "awq": lambda s: q.awq_linear_w4a16(ax, aqws[s % R], ascl_d, None, ay, stream=sh)}[args.only]
        for s in range(R):
            step(s)
        t = batch_timing(fn, stream, args.steps, batches=max(1, min(10, args.steps)), warm=args.warmup)
        print(json.dumps({"only": args.only, "us": t}), flush=True)
        return

    # Per-kernel rates, each kernel alone, back to back over the rotating buffers (after one pass of
    # the step over every buffer set). They run before the warmup steps, so the timed steps start on a
    # GPU at its working clock: after the idle set-up, 20 steps behind only 5 warmup steps measured
    # ~360 us per step against ~297 us behind 100 warmup steps (and ~288 us over 1000 steps).
    for s in range(R):
        step(s)
    t_a = batch_timing(lambda s: q.svdq_quantize_act(xs[s % R], inv, l1t_d, qact[s % R], asc[s % R], tl[s % R],
                                                     stream=sh), stream)
    t_c = batch_timing(lambda s: q.awq_linear_w4a16(ax, aqws[s % R], ascl_d, None, ay, stream=sh), stream, 500)
    t_b_alone = batch_timing(lambda s: q.svdq_linear_w4a4(qact[s % R], asc[s % R], qw_d, sw_d, tl[s % R], l2t_d,
                                                          bias_d, y, stream=sh), stream)

    log(f"[bench] warmup {args.warmup}")
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {n} bytes read, {n} bytes written")
        del src, dst

    # Timed region: exactly K steps, synchronised on both sides, with no event inside it.
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    start.record(stream)
    for s in range(args.steps):
        step(s)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / args.steps

    # Roofline samples of the dominant kernel (after the timed region): more steps of the same
    # workload, each with its GEMM between two HIP events on the launch stream, so the GEMM runs
    # in the same context (alternating with the memory-bound kernels) as in the timed steps.
    ns = max(20, args.gemm_samples)
    log(f"[bench] {ns} GEMM samples")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(ns)]
    torch.cuda.synchronize()
    for s in range(ns):
        step(args.steps + s, evs[s])
    torch.cuda.synchronize()
    tb_samples = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    t_b = float(np.median(tb_samples)) * 1e-3  # ms


    gemm_ops = 2.0 * M * N * K
    lr_flops = 2.0 * M * r * (K + N)
    awq_flops = 2.0 * awq_cfg.M * awq_cfg.N * awq_cfg.K
    step_ops = gemm_ops + lr_flops + awq_flops
    value = step_ops / (ms_step * 1e-3) / 1e12
    achieved_b = gemm_ops / (t_b * 1e-3) / 1e12
    bytes_a = quant_bytes(M, K, r)
    bytes_c = awq_bytes(awq_cfg.M, awq_cfg.K, awq_cfg.N)
    traffic = load_traffic("w4a4_gemm.hip", cfg.name)

    def rate(nbytes, us):
        return round(nbytes / (us * 1e-6) / 1e9, 1)

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"svdq_w4a4 {cfg.name} M{M} K{K} N{N} r{r} + awq_w4a16 M{awq_cfg.M} "
                               f"K{awq_cfg.K} N{awq_cfg.N}", "M": M, "K": K, "N": N, "rank": r, "group": 64,
                   "awq": [awq_cfg.M, awq_cfg.K, awq_cfg.N], "rotating_buffer_sets": R},
        "roofline": {"bound": "mfma", "achieved": round(achieved_b, 2), "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s",
                     "frac": round(achieved_b / INT8_PEAK_TOPS, 4), "traffic": traffic,
                     "kernel": "w4a4_gemm_kernel (svdq_linear_w4a4)", "ops_per_launch": gemm_ops,
                     "samples": int(len(tb_samples)), "us_median": round(float(np.median(tb_samples)), 2),
                     "us_min": round(float(tb_samples.min()), 2), "us_max": round(float(tb_samples.max()), 2)},
        "kernels": {
            "svdq_quantize_act_us": t_a["median"],
            "svdq_quantize_act_GBs": rate(bytes_a, t_a["median"]),
            "svdq_quantize_act_hbm_frac": round(rate(bytes_a, t_a["median"]) / HBM_PEAK_GBS, 4),
            "svdq_linear_w4a4_us": round(t_b * 1e3, 2),
            "svdq_linear_w4a4_TOPS": round(achieved_b, 2),
            "svdq_linear_w4a4_alone_us": t_b_alone["median"],
            "awq_linear_w4a16_us": t_c["median"],
            "awq_linear_w4a16_GBs": rate(bytes_c, t_c["median"]),
            "awq_linear_w4a16_hbm_frac": round(rate(bytes_c, t_c["median"]) / HBM_PEAK_GBS, 4),
            "layer_TOPS_a_plus_b": round(gemm_ops / ((t_a["median"] * 1e-3 + t_b) * 1e-3) / 1e12, 2),
            "timing": f"GEMM: HIP events around the GEMM of {len(tb_samples)} steps after the timed region "
                      f"(median); '_alone': the GEMM back to back; quantizer and W4A16: each alone, back to back "
                      f"over the rotating buffers, 10 batches (median of the batch means), before the warmup steps",
            "batches": {"quantize_act": t_a, "linear_w4a4_alone": t_b_alone, "awq_linear_w4a16": t_c},
        },
    }
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (oracle) on {args.cpu_rows} rows")
        out["cpu_baseline"] = cpu_baseline(cfg, awq_cfg, args.cpu_rows, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
