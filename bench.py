"""Benchmark of the low-precision MoE expert forward on one MI355X.

One step = one moe_expert_forward (route, permute, activation preparation,
chunked dequant + GEMM1 + SwiGLU, dequant + GEMM2, combine) over one batch of
synthetic input already resident in HBM.  Default workload: the
Qwen3-30B-A3B-shaped FP8 layer (4096 tokens, hidden 2048, 128 experts, top-8,
inter 768, [128,128] block-scaled E4M3 weights, chunks of 16 experts).

Prints one JSON line: tokens/s (value), TFLOP/s and % of the format's MFMA
peak, algorithmic HBM GB/s, the roofline of the dominant kernel (per-launch
durations from HIP events recorded on the launch stream by the library's
timed entry point), and the CPU oracle timed on a bounded token sample.
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

METRIC = "MoE expert-layer tokens/s + TFLOP/s (% MFMA peak) / HBM GB/s per weight format"
HBM_PEAK = 8.0e12
# fp16 MFMA (INT4 path), fp8, fp8 x fp4 (issued at the fp8 rate), fp8 with E8M0 block scales,
# fp16 MFMA (NVFP4 path)
MFMA_PEAK = {1: 2.5e15, 2: 5.0e15, 3: 5.0e15, 4: 5.0e15, 5: 2.5e15}
DTYPE = {1: "int4_w_fp16_mfma", 2: "fp8_e4m3", 3: "mxfp4_w_mxfp8_a", 4: "fp8_e4m3_pow2", 5: "nvfp4_w_fp16_mfma"}


def weight_bytes_per_expert(fmt: int, N: int, K: int) -> float:
    if fmt == 1:
        return N * K / 2 + N * (K // 32) * 2
    if fmt == 5:
        return N * K / 2 + N * (K // 16) + 4
    if fmt in (2, 4):
        return N * K + (N // 128) * (K // 128) * 4
    return N * K / 2 + N * (K // 32)


def act_bytes(fmt: int, rows: int, K: int) -> float:
    """Bytes of one activation matrix in the GEMM input format."""
    if fmt in (1, 5):
        return rows * K * 2
    if fmt in (2, 4):
        return rows * K + rows * (K // 128) * 4
    return rows * K + rows * (K // 32)


def accounting(cfg, counts: np.ndarray) -> dict:
    """Algorithmic FLOPs and compulsory HBM bytes of the step and of each GEMM stage."""
    T, H, I, E, k, fmt = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.fmt
    R = T * k
    na = int((counts > 0).sum())
    w13 = weight_bytes_per_expert(fmt, 2 * I, H)
    w2 = weight_bytes_per_expert(fmt, H, I)
    oft = 64 * H if cfg.oft else 0  # R_e: (H/32) blocks of 32x32 bf16
    flops1 = 4.0 * R * H * I + (2.0 * R * H * 32 if cfg.oft else 0.0)
    flops2 = 2.0 * R * H * I
    a_rows = R if cfg.oft else T
    g1_bytes = na * w13 + act_bytes(fmt, a_rows, H) + act_bytes(fmt, R, I)
    g2_bytes = na * w2 + act_bytes(fmt, R, I) + R * H * 2
    step_bytes = na * (w13 + w2 + oft) + 2 * T * H * 2 + 4 * T * E + 8 * T * k
    return dict(active=na, flops=flops1 + flops2, bytes=step_bytes, gemm1=(flops1, g1_bytes), gemm2=(flops2, g2_bytes))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c2", help="c1..c5, c2p, c4n (default c2: the Qwen3-30B-A3B-shaped FP8 layer)")
    ap.add_argument("--chunk", type=int, default=None, help="chunk_experts (default: the workload's)")
    ap.add_argument("--tile-rows", type=int, default=0, help="grouped-GEMM tile rows (0: automatic)")
    ap.add_argument("--cpu-tokens", type=int, default=None, help="oracle token sample (default: sized per workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--weight-layout", choices=("auto", "rows", "kblocked"), default="auto",
                    help="weight code order for the fused forward: rows [N][K] or 16 x 128 tiles "
                         "(auto: tiles, except for the materialized mode)")
    ap.add_argument("--materialized", action="store_true",
                    help="time the materialized-chunk scheme (per-chunk BF16 weight copy + BF16 GEMMs) instead")
    ap.add_argument("--backward", action="store_true",
                    help="time the frozen-base backward (d_x, d_logits, d_adapter; INT4 layers) instead")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the library runs one "
              "GPU's share of the layer; the expert-parallel split across GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch

    from precision_moe_expert_amd import binding, synth

    cfg = synth.CONFIGS[args.config]
    if args.chunk:
        cfg = cfg.replace(chunk=args.chunk)
    li = synth.make_inputs(cfg, with_lm=False)

    def dev(a, bf16=False):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()
        return t.view(torch.bfloat16) if bf16 else t

    x, logits = dev(li.x, True), dev(li.logits)
    w13, w2, s13, s2 = dev(li.w13), dev(li.w2), dev(li.s13), dev(li.s2)
    g13 = dev(li.g13) if li.g13 is not None else None   # NVFP4 second-level scales
    g2 = dev(li.g2) if li.g2 is not None else None
    oft = dev(li.oft, True) if li.oft is not None else None
    mat, bwd = args.materialized, args.backward
    tiled_ok = not mat
    if args.weight_layout == "kblocked" and not tiled_ok:
        sys.exit("--weight-layout kblocked: not with --materialized")
    wl = binding.WL_KBLOCKED if tiled_ok and args.weight_layout != "rows" else binding.WL_ROWS
    layer = binding.make_layer(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.fmt, oft=oft is not None,
                               tile_rows=args.tile_rows, weight_layout=wl)
    if wl == binding.WL_KBLOCKED:
        # the frozen codes re-laid once, outside the timed region, as a server stores them
        w13, w2 = binding.pack_weights_kblocked(layer, w13, w2)
        torch.cuda.synchronize()
    if bwd:
        ws_bytes = binding.backward_workspace_bytes(layer, cfg.chunk)
        bw = binding.prepare_backward_weights(layer, w13, w2, s13, s2)
        rng = np.random.default_rng(12345)
        d_out_bits = synth._to_bf16_bits(rng.standard_normal((cfg.T, cfg.H)).astype(np.float32))
        d_out = dev(d_out_bits, True)
        d_x = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
        d_lg = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device="cuda")
        d_ad = torch.empty(oft.shape, dtype=torch.float32, device="cuda") if oft is not None else None
    else:
        ws_bytes = (binding.materialized_workspace_bytes if mat else binding.workspace_bytes)(layer, cfg.chunk)
    ws = binding.alloc_workspace(ws_bytes)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")

    def step():
        if bwd:
            binding.expert_backward(layer, x, logits, w13, w2, s13, s2, bw, d_out, adapter=oft,
                                    chunk_experts=cfg.chunk, ws=ws, d_x=d_x, d_logits=d_lg, d_adapter=d_ad,
                                    g13=g13, g2=g2)
        elif mat:
            binding.expert_forward_materialized(layer, x, logits, w13, w2, s13, s2, adapter=oft,
                                                chunk_experts=cfg.chunk, out=out, ws=ws, g13=g13, g2=g2)
        else:
            binding.expert_forward(layer, x, logits, w13, w2, s13, s2, adapter=oft, chunk_experts=cfg.chunk,
                                   out=out, ws=ws, g13=g13, g2=g2)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = max(wall * 1e3, ev0.elapsed_time(ev1)) / args.steps

    # per-stage HIP-event durations over the same number of steps
    stage_ms = {s: 0.0 for s in binding.STAGES}
    stage_n = {s: 0 for s in binding.STAGES}
    for _ in range(args.steps):
        if bwd:
            st = binding.expert_backward(layer, x, logits, w13, w2, s13, s2, bw, d_out, adapter=oft,
                                         chunk_experts=cfg.chunk, ws=ws, d_x=d_x, d_logits=d_lg, d_adapter=d_ad,
                                         timed=True, g13=g13, g2=g2)[3]
        elif mat:
            _, st = binding.expert_forward_materialized(layer, x, logits, w13, w2, s13, s2, adapter=oft,
                                                        chunk_experts=cfg.chunk, out=out, ws=ws, timed=True,
                                                        g13=g13, g2=g2)
        else:
            _, st = binding.expert_forward_timed(layer, x, logits, w13, w2, s13, s2, adapter=oft,
                                                 chunk_experts=cfg.chunk, out=out, ws=ws, g13=g13, g2=g2)
        for s, (ms, n) in st.items():
            stage_ms[s] += ms
            stage_n[s] += n

    # expert row counts from the library's own routing (accounting only)
    r = binding.route_permute(logits, layer)
    torch.cuda.synchronize()
    counts = np.diff(r["expert_offsets"].cpu().numpy())
    acc = accounting(cfg, counts)

    sec = ms_per_step / 1e3
    peak = MFMA_PEAK[cfg.fmt]
    fmt_name = {1: "int4", 2: "fp8", 3: "mxfp4", 4: "fp8", 5: "nvfp4"}[cfg.fmt]
    bm = binding.tile_rows(layer)
    if bwd:
        # recompute (forward INT4 GEMM1) and the backward GEMM pair: 4 + 6 R H I FLOPs;
        # the dominant one by event time is reported
        R = cfg.T * cfg.k
        w13b = weight_bytes_per_expert(cfg.fmt, 2 * cfg.I, cfg.H)
        w2b = weight_bytes_per_expert(cfg.fmt, cfg.H, cfg.I)
        fam = {1: 1, 2: 2, 3: 3, 4: 2, 5: 5}[cfg.fmt]
        if stage_ms["gemm1"] > stage_ms["gemm2"]:
            # the forward GEMM1 kernel of the format (pre-activation recompute)
            peak = MFMA_PEAK[cfg.fmt]
            dom, launches = "gemm1", stage_n["gemm1"]
            f_dom = 4.0 * R * cfg.H * cfg.I
            b_dom = (acc["active"] * w13b + act_bytes(cfg.fmt, R if cfg.oft else cfg.T, cfg.H) + R * 2 * cfg.I * 4
                     + (act_bytes(cfg.fmt, R, cfg.I) if cfg.fmt not in (1, 5) else 0))
            if cfg.fmt in (2, 4):
                kname = f"k_gemm_fp8<{bm}, {'true' if cfg.fmt == 4 else 'false'}>"
            else:
                kname = f"k_gemm_{fmt_name}<{bm}>"
        else:
            # the backward GEMMs run on fp16 MFMA for every weight format
            peak = MFMA_PEAK[1]
            dom, launches = "gemm2", stage_n["gemm2"]
            f_dom = 6.0 * R * cfg.H * cfg.I
            # transposed weights, d_out rows, [da|db] written and read, pre-activations read, dx' written
            b_dom = (acc["active"] * (w13b + w2b) + cfg.T * cfg.H * 2 + 2 * R * 2 * cfg.I * 2 + R * 2 * cfg.I * 4
                     + R * cfg.H * 4)
            kname = f"k_gemm_bwd<{fam}, {min(bm, 64)}>"
        launch_ms = stage_ms[dom] / max(launches, 1)
        acc["flops"] = 10.0 * R * cfg.H * cfg.I + (4.0 * R * cfg.H * 32 if cfg.oft else 0.0)
    elif mat:
        # the BF16 copy: packed weights read and 2 bytes per weight written by the
        # dequant kernel, then read back by the BF16 GEMMs with bf16 activations
        nw = acc["active"] * 3 * cfg.H * cfg.I
        R = cfg.T * cfg.k
        deq_b = nw * 2 + acc["active"] * (weight_bytes_per_expert(cfg.fmt, 2 * cfg.I, cfg.H) +
                                          weight_bytes_per_expert(cfg.fmt, cfg.H, cfg.I))
        gemm_b = nw * 2 + (R if cfg.oft else cfg.T) * cfg.H * 2 + 2 * R * cfg.I * 2 + R * cfg.H * 2
        peak = MFMA_PEAK[1]  # bf16 MFMA, same peak as fp16
        g_ms = stage_ms["gemm1"] + stage_ms["gemm2"]
        if stage_ms["dequant"] > g_ms:
            dom, launches, f_dom, b_dom = "dequant", stage_n["dequant"], 0.0, deq_b
            launch_ms = stage_ms["dequant"] / max(launches, 1)
            kname = f"k_dequant_chunk<{ {1: 1, 2: 2, 3: 3, 4: 2, 5: 5}[cfg.fmt] }>"
        else:
            dom, launches = "gemm", stage_n["gemm1"] + stage_n["gemm2"]
            launch_ms = g_ms / max(launches, 1)
            f_dom, b_dom = acc["gemm1"][0] + acc["gemm2"][0], gemm_b
            kname = "k_gemm_bf16"
    else:
        # every launch is one kernel running chunk c's GEMM1 with chunk c-1's GEMM2
        dom = "gemm"
        launches = stage_n["gemm1"] + stage_n["gemm2"]
        launch_ms = (stage_ms["gemm1"] + stage_ms["gemm2"]) / max(launches, 1)
        f_dom, b_dom = acc["gemm1"][0] + acc["gemm2"][0], acc["gemm1"][1] + acc["gemm2"][1]
        if cfg.fmt in (2, 4):
            kname = f"k_gemm_fp8<{bm}, {'true' if cfg.fmt == 4 else 'false'}>"
        else:
            kname = f"k_gemm_{fmt_name}<{bm}>"
    launches_per_step = launches / args.steps
    f_launch, b_launch = f_dom / launches_per_step, b_dom / launches_per_step
    if f_launch == 0 or b_launch / HBM_PEAK >= f_launch / peak:
        roof = dict(bound="hbm", achieved=b_launch / (launch_ms / 1e3) / 1e9, peak=HBM_PEAK / 1e9, unit="GB/s")
    else:
        roof = dict(bound="mfma", achieved=f_launch / (launch_ms / 1e3) / 1e12, peak=peak / 1e12, unit="TFLOP/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = kname
    # HBM bytes per launch measured by rocprofv3 counters (copy-calibrated),
    # valid only while the kernel source is unchanged
    from precision_moe_expert_amd import profiling
    kfam = kname.split("<")[0].replace("k_gemm_", "")
    tr = profiling.read_traffic(os.path.join(ROOT, "profiles", f"gemm_{kfam}_{cfg.name}_traffic.txt"))
    roof["traffic"] = tr["hbm_bytes_per_dispatch"] if tr and tr["kernel"] == kname and not mat else None
    roof["launch_ms"] = launch_ms
    roof["algorithmic_bytes_per_launch"] = b_launch
    roof["algorithmic_flops_per_launch"] = f_launch

    result = {
        "metric": METRIC,
        "value": cfg.T / sec,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16_from_" + DTYPE[cfg.fmt] if mat else ("fp16_backward_" + DTYPE[cfg.fmt] if bwd
                                                             else DTYPE[cfg.fmt]),
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} MoE expert layer", "tokens": cfg.T, "hidden": cfg.H,
                   "experts": cfg.E, "top_k": cfg.k, "inter": cfg.I, "weight_format": synth.FMT_NAMES[cfg.fmt],
                   "chunk_experts": cfg.chunk, "tile_rows": args.tile_rows or "auto", "oft_adapter": cfg.oft,
                   "weight_layout": "kblocked_16x128" if wl == binding.WL_KBLOCKED else "rows",
                   "active_experts": acc["active"],
                   "mode": "materialized_bf16_copy" if mat else ("frozen_base_backward" if bwd else "fused")},
        "tflops": acc["flops"] / sec / 1e12,
        "pct_mfma_peak": 100.0 * acc["flops"] / sec / peak,
        "hbm_gbps_algorithmic": acc["bytes"] / sec / 1e9,
        "pct_hbm_peak": 100.0 * acc["bytes"] / sec / HBM_PEAK,
        "stages_ms_per_step": {s: stage_ms[s] / args.steps for s in binding.STAGES},
        "temp_dequant_bytes": {"materialized_chunk_scheme": min(cfg.chunk, cfg.E) * 3 * cfg.H * cfg.I * 2,
                               "this_run": min(cfg.chunk, cfg.E) * 3 * cfg.H * cfg.I * 2 if mat else 0},
        "workspace_bytes": ws_bytes,
        "roofline": roof,
    }

    if not args.no_cpu_baseline:
        import oracle
        n = args.cpu_tokens or {1: 64, 2: 4096, 3: 64, 4: 64, 5: 64, 6: 4096, 7: 64}[cfg.cfg_id]
        n = min(n, cfg.T)
        toks = np.arange(n, dtype=np.int32)
        # repeat short samples until about 10 s of oracle work has been timed
        passes, c0 = 0, time.perf_counter()
        if bwd:
            d_out_f32 = (d_out_bits[toks].astype(np.uint32) << 16).view(np.float32)
        while passes == 0 or (time.perf_counter() - c0 < 10.0 and passes < 8):
            if bwd:
                oracle.backward_inputs(li, d_out_f32, tokens=toks)
            else:
                oracle.forward_inputs(li, tokens=toks, materialized=mat)
            passes += 1
        csec = time.perf_counter() - c0
        result["cpu_baseline"] = {"value": n * passes / csec, "unit": "tokens/s", "cores": oracle.num_threads(),
                                  "kind": "oracle", "sample": f"first {n} of {cfg.T} tokens (full routing, "
                                  f"chunked dequant of the experts they touch), {passes} pass(es), {csec:.1f} s"}
    print(json.dumps(result))


if __name__ == "__main__":
    main()
