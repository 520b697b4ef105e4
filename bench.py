"""Benchmark of the low-precision MoE expert forward on one MI355X.

One step = one moe_expert_forward (route, permute, activation preparation,
chunked dequant + GEMM1 + SwiGLU, dequant + GEMM2, combine) over one batch of
synthetic input already resident in HBM.  Default workload (the headline): the
DeepSeek-V3-shaped MXFP4 layer -- 16384 tokens, hidden 7168, 256 experts,
top-8, inter 2048, Zipf-skewed routing, chunks of 32 experts.  Before every
timed step a 512 MiB buffer is written so that the 256 MB last-level cache
(MALL) holds none of the step's inputs; the step time is the median of the
per-step HIP-event times.

Prints one JSON line: tokens/s (value), TFLOP/s and % of the format's MFMA
peak, algorithmic HBM GB/s, the roofline of the dominant kernel (per-launch
durations from HIP events recorded on the launch stream by the library's
timed entry point), the CPU oracle timed on a bounded token sample (with the
GPU-vs-oracle errors on those tokens), and under "extras" the chunk-size
sweep and the other layer shapes (Qwen3-30B-A3B-shaped FP8, Kimi-K2-shaped
INT4 + OFT, the decode layer and its LM head).
"""
from __future__ import annotations

import argparse
import json
import os
import platform
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
FLUSH_BYTES = 512 << 20


class CacheFlush:
    """Between timed steps: write FLUSH_BYTES (more than the 256 MB MALL, so
    no weight byte of the last step is left in any cache), then read another
    FLUSH_BYTES buffer.  The write alone leaves the caches full of dirty
    lines, and writing those back to HBM takes ~60 us of the next kernel's
    bandwidth (a 459 MB stream measured 138 us after the write, 78 us after
    write + read); the read replaces them with clean lines, so the timed
    step starts cold and pays only for its own traffic.  Both are untimed."""

    def __init__(self):
        import torch
        self.w = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        self.r = torch.ones(FLUSH_BYTES // 8, dtype=torch.int64, device="cuda")
        self.sink = torch.empty((), dtype=torch.int64, device="cuda")

    def __call__(self, i: int):
        import torch
        self.w.fill_(i & 0x7F)
        torch.sum(self.r, dim=0, out=self.sink)


def weight_bytes_per_expert(fmt: int, N: int, K: int) -> float:
    """Packed codes + scales of one expert matrix [N][K]."""
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
    """Algorithmic FLOPs and compulsory HBM bytes of one step.

    FLOPs = 6 T k H I (+ 2 T k H 32 with the OFT rotation).  Compulsory bytes
    = the active experts' packed weights and scales (+ their OFT blocks) + x +
    out + logits + routing ids/weights.  The grouped GEMM's own compulsory
    bytes are the weights and scales alone; the activation rows it gathers,
    h and y_perm are intermediates of this implementation and are reported
    separately (intermediate_bytes)."""
    T, H, I, E, k, fmt = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.fmt
    R = T * k
    na = int((counts > 0).sum())
    w13 = weight_bytes_per_expert(fmt, 2 * I, H)
    w2 = weight_bytes_per_expert(fmt, H, I)
    oft = 64 * H if cfg.oft else 0  # R_e: (H/32) blocks of 32x32 bf16
    flops_gemm = 6.0 * R * H * I
    flops = flops_gemm + (2.0 * R * H * 32 if cfg.oft else 0.0)
    weights = na * (w13 + w2)
    step_bytes = weights + na * oft + 2 * T * H * 2 + 4 * T * E + 8 * T * k
    a_rows = R if cfg.oft else T
    inter = act_bytes(fmt, a_rows, H) + 2 * act_bytes(fmt, R, I) + 2 * R * H * 2
    return dict(active=na, flops=flops, flops_gemm=flops_gemm, bytes=step_bytes, gemm_bytes=weights,
                intermediate_bytes=inter)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


class Workload:
    """Device copies of one layer's synthetic inputs and the library calls on them."""

    def __init__(self, cfg, li, tile_rows=0, layout="auto", mode="fused"):
        import torch

        from precision_moe_expert_amd import binding
        self.cfg, self.li, self.mode, self.binding = cfg, li, mode, binding

        def dev(a, bf16=False):
            a = np.ascontiguousarray(a)
            t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()
            return t.view(torch.bfloat16) if bf16 else t

        self.x, self.logits = dev(li.x, True), dev(li.logits)
        w13, w2 = dev(li.w13), dev(li.w2)
        self.s13, self.s2 = dev(li.s13), dev(li.s2)
        self.g13 = dev(li.g13) if li.g13 is not None else None   # NVFP4 second-level scales
        self.g2 = dev(li.g2) if li.g2 is not None else None
        self.oft = dev(li.oft, True) if li.oft is not None else None
        tiled_ok = mode != "materialized"
        if layout == "kblocked" and not tiled_ok:
            sys.exit("--weight-layout kblocked: not with --materialized")
        self.wl = binding.WL_KBLOCKED if tiled_ok and layout != "rows" else binding.WL_ROWS
        self.layer = binding.make_layer(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.fmt, oft=self.oft is not None,
                                        tile_rows=tile_rows, weight_layout=self.wl)
        if self.wl == binding.WL_KBLOCKED:
            # the frozen codes re-laid once, outside the timed region, as a server stores them
            self.w13, self.w2 = binding.pack_weights_kblocked(self.layer, w13, w2)
            torch.cuda.synchronize()
            del w13, w2
        else:
            self.w13, self.w2 = w13, w2
        self.bw = None
        if mode == "backward":
            self.bw = binding.prepare_backward_weights(self.layer, self.w13, self.w2, self.s13, self.s2)
            rng = np.random.default_rng(12345)
            from precision_moe_expert_amd import synth
            self.d_out_bits = synth._to_bf16_bits(rng.standard_normal((cfg.T, cfg.H)).astype(np.float32))
            self.d_out = dev(self.d_out_bits, True)
            self.d_x = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
            self.d_lg = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device="cuda")
            self.d_ad = torch.empty(self.oft.shape, dtype=torch.float32, device="cuda") if self.oft is not None else None
        self.out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
        self.ws = None
        self.ws_chunk = None

    def workspace(self, chunk):
        b = self.binding
        if self.mode == "backward":
            n = b.backward_workspace_bytes(self.layer, chunk)
        elif self.mode == "materialized":
            n = b.materialized_workspace_bytes(self.layer, chunk)
        else:
            n = b.workspace_bytes(self.layer, chunk)
        if self.ws is None or self.ws.numel() < n:
            self.ws = None
            self.ws = b.alloc_workspace(n)
        self.ws_bytes = n
        return self.ws

    def step(self, chunk, timed=False):
        """One call; with timed=True returns {stage: (ms, launches)} (the call synchronises)."""
        b, ws = self.binding, self.workspace(chunk)
        common = dict(adapter=self.oft, chunk_experts=chunk, ws=ws, g13=self.g13, g2=self.g2)
        if self.mode == "backward":
            r = b.expert_backward(self.layer, self.x, self.logits, self.w13, self.w2, self.s13, self.s2, self.bw,
                                  self.d_out, d_x=self.d_x, d_logits=self.d_lg, d_adapter=self.d_ad, timed=timed,
                                  **common)
            return r[3] if timed else None
        if self.mode == "materialized":
            r = b.expert_forward_materialized(self.layer, self.x, self.logits, self.w13, self.w2, self.s13, self.s2,
                                              out=self.out, timed=timed, **common)
            return r[1] if timed else None
        if timed:
            return b.expert_forward_timed(self.layer, self.x, self.logits, self.w13, self.w2, self.s13, self.s2,
                                          out=self.out, **common)[1]
        b.expert_forward(self.layer, self.x, self.logits, self.w13, self.w2, self.s13, self.s2, out=self.out,
                         **common)
        return None


def time_steps(fn, steps, warmup, flush):
    """Median / mean per-step HIP-event time (ms) of fn() on the current stream,
    with the cache flush (CacheFlush) before every step (outside the events)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        flush(i)
        evs[i][0].record(stream)
        fn()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    return float(np.median(ms)), float(ms.mean()), ms


def stage_times(w: Workload, chunk, reps, flush):
    """Per-stage HIP-event times from the library's timed entry point (each
    rep after a flush), summed over reps."""
    import torch
    from precision_moe_expert_amd import binding
    stage_ms = {s: 0.0 for s in binding.STAGES}
    stage_n = {s: 0 for s in binding.STAGES}
    for i in range(reps):
        flush(i)
        torch.cuda.synchronize()
        st = w.step(chunk, timed=True)
        for s, (ms, n) in st.items():
            stage_ms[s] += ms
            stage_n[s] += n
    return stage_ms, stage_n


def kernel_name(cfg, bm, mode):
    fam = {1: 1, 2: 2, 3: 3, 4: 2, 5: 5}[cfg.fmt]
    fmt_name = {1: "int4", 2: "fp8", 3: "mxfp4", 4: "fp8", 5: "nvfp4"}[cfg.fmt]
    if mode == "materialized":
        return "k_gemm_bf16", f"k_dequant_chunk<{fam}>"
    if mode == "backward":
        return f"k_gemm_bwd<{fam}, {min(bm, 64)}>", None
    if cfg.fmt in (2, 4):
        return f"k_gemm_fp8<{bm}, {'true' if cfg.fmt == 4 else 'false'}>", None
    if cfg.fmt == 1:  # 16-row tiles take two 16-column subtiles per wave, taller ones four; 96-row tiles 64-K steps
        return f"k_gemm_int4<{bm}, {2 if bm == 16 else 4}, {64 if bm == 96 else 128}>", None
    if cfg.fmt == 5:  # 96-row tiles take 64-K steps
        return f"k_gemm_nvfp4<{bm}, {64 if bm == 96 else 128}>", None
    return f"k_gemm_{fmt_name}<{bm}>", None


def roofline(cfg, acc, stage_ms, stage_n, reps, bm, mode):
    """Roofline of the dominant kernel from the per-launch event times.

    Fused forward: every GEMM launch runs one chunk's GEMM1 with the previous
    chunk's GEMM2, so per launch = (6 R H I FLOPs, the active experts' weight
    and scale bytes) / GEMM launches per step.  Bound = the larger of
    FLOPs / MFMA peak and bytes / HBM peak."""
    from precision_moe_expert_amd import profiling
    R = cfg.T * cfg.k
    peak = MFMA_PEAK[cfg.fmt]
    kname, kname2 = kernel_name(cfg, bm, mode)
    if mode == "backward":
        w13b = weight_bytes_per_expert(cfg.fmt, 2 * cfg.I, cfg.H)
        w2b = weight_bytes_per_expert(cfg.fmt, cfg.H, cfg.I)
        if stage_ms["gemm1"] > stage_ms["gemm2"]:
            dom, launches = "gemm1", stage_n["gemm1"]
            f_dom, b_dom = 4.0 * R * cfg.H * cfg.I, acc["active"] * w13b
            kname = kernel_name(cfg, bm, "fused")[0]
        else:
            peak = MFMA_PEAK[1]  # the backward GEMMs run on fp16 MFMA for every weight format
            dom, launches = "gemm2", stage_n["gemm2"]
            f_dom, b_dom = 6.0 * R * cfg.H * cfg.I, acc["active"] * (w13b + w2b)
        launch_ms = stage_ms[dom] / max(launches, 1)
    elif mode == "materialized":
        nw = acc["active"] * 3 * cfg.H * cfg.I
        deq_b = nw * 2 + acc["gemm_bytes"]
        peak = MFMA_PEAK[1]  # bf16 MFMA
        g_ms = stage_ms["gemm1"] + stage_ms["gemm2"]
        if stage_ms["dequant"] > g_ms:
            launches, f_dom, b_dom, kname = stage_n["dequant"], 0.0, deq_b, kname2
            launch_ms = stage_ms["dequant"] / max(launches, 1)
        else:
            launches = stage_n["gemm1"] + stage_n["gemm2"]
            launch_ms = g_ms / max(launches, 1)
            f_dom, b_dom = acc["flops_gemm"], nw * 2
    else:
        launches = stage_n["gemm1"] + stage_n["gemm2"]
        launch_ms = (stage_ms["gemm1"] + stage_ms["gemm2"]) / max(launches, 1)
        f_dom, b_dom = acc["flops_gemm"], acc["gemm_bytes"]
    lps = launches / reps
    f_launch, b_launch = f_dom / lps, b_dom / lps
    if f_launch == 0 or b_launch / HBM_PEAK >= f_launch / peak:
        roof = dict(bound="hbm", achieved=b_launch / (launch_ms / 1e3) / 1e9, peak=HBM_PEAK / 1e9, unit="GB/s")
    else:
        roof = dict(bound="mfma", achieved=f_launch / (launch_ms / 1e3) / 1e12, peak=peak / 1e12, unit="TFLOP/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    # HBM bytes per launch measured by rocprofv3 counters (copy-calibrated),
    # valid only while the kernel and scheduler sources are unchanged
    kfam = kname.split("<")[0].replace("k_gemm_", "").replace("k_", "")
    tr = profiling.read_traffic(os.path.join(ROOT, "profiles", f"gemm_{kfam}_{cfg.name}_traffic.txt"))
    roof["traffic"] = tr["hbm_bytes_per_dispatch"] if tr and tr["kernel"] == kname and mode == "fused" else None
    roof.update(kernel=kname, launch_ms=launch_ms, launches_per_step=lps, algorithmic_bytes_per_launch=b_launch,
                algorithmic_flops_per_launch=f_launch)
    return roof


def lds_bytes(cfg, bm):
    """Static LDS of one grouped-GEMM workgroup (the register/LDS-resident
    dequantized operands that stand in for the pages' BF16 chunk copy)."""
    # stage buffers + activation-scale ring (MXFP4), as laid out by the kernels
    if cfg.fmt == 3:
        na = (bm * 8 + 255) // 256
        stage = na * 32 * 128 + 4 * 4 * 1024 + 4 * 256
        wpc = 2 if bm <= 128 else 1
        s = min(5, (152 * 1024 // wpc) // stage)
        return s * stage + 2 * ((bm + 63) // 64) * 64 * 16, wpc
    return None, None


def measure_layer(name, args, flush, chunk=None, mode="fused", with_roofline=True):
    """Times one layer shape; returns (result dict, Workload)."""
    import torch

    from precision_moe_expert_amd import binding, synth
    cfg = synth.CONFIGS[name]
    if chunk:
        cfg = cfg.replace(chunk=chunk)
    li = synth.make_inputs(cfg, with_lm=False)
    w = Workload(cfg, li, tile_rows=args.tile_rows, layout=args.weight_layout, mode=mode)
    med, mean, _ = time_steps(lambda: w.step(cfg.chunk), args.steps, args.warmup, flush)
    r = binding.route_permute(w.logits, w.layer)
    torch.cuda.synchronize()
    counts = np.diff(r["expert_offsets"].cpu().numpy())
    acc = accounting(cfg, counts)
    if mode == "backward":
        acc["flops"] = 10.0 * cfg.T * cfg.k * cfg.H * cfg.I + (4.0 * cfg.T * cfg.k * cfg.H * 32 if cfg.oft else 0.0)
    sec = med / 1e3
    peak = MFMA_PEAK[cfg.fmt] if mode == "fused" else MFMA_PEAK[1]
    bm = binding.tile_rows(w.layer)
    res = {
        "workload": f"{cfg.name} MoE expert layer", "tokens": cfg.T, "hidden": cfg.H, "experts": cfg.E,
        "top_k": cfg.k, "inter": cfg.I, "weight_format": synth.FMT_NAMES[cfg.fmt], "chunk_experts": cfg.chunk,
        "tile_rows": bm, "oft_adapter": cfg.oft,
        "weight_layout": "kblocked_16x128" if w.wl == binding.WL_KBLOCKED else "rows",
        "active_experts": acc["active"], "max_rows_per_expert": int(counts.max()), "mode": mode,
        "ms_per_step": med, "ms_per_step_mean": mean, "tokens_per_s": cfg.T / sec,
        "tflops": acc["flops"] / sec / 1e12, "pct_mfma_peak": 100.0 * acc["flops"] / sec / peak,
        "hbm_gbps_algorithmic": acc["bytes"] / sec / 1e9, "pct_hbm_peak": 100.0 * acc["bytes"] / sec / HBM_PEAK,
        "intermediate_gbps": acc["intermediate_bytes"] / sec / 1e9,
        "dtype": ("bf16_from_" + DTYPE[cfg.fmt]) if mode == "materialized" else
                 (("fp16_backward_" + DTYPE[cfg.fmt]) if mode == "backward" else DTYPE[cfg.fmt]),
        "workspace_bytes": w.ws_bytes,
        "temp_dequant_bytes": {"materialized_chunk_scheme": min(cfg.chunk, cfg.E) * 3 * cfg.H * cfg.I * 2,
                               "this_run_global": (min(cfg.chunk, cfg.E) * 3 * cfg.H * cfg.I * 2
                                                   if mode == "materialized" else 0)},
    }
    lb, wpc = lds_bytes(cfg, bm)
    if lb is not None and mode == "fused":
        res["temp_dequant_bytes"]["this_run_lds_per_workgroup"] = lb
        res["temp_dequant_bytes"]["this_run_lds_all_cus"] = lb * wpc * 256
    if cfg.lm_vocab > 0 and mode == "fused":
        res["lm_head"] = lm_head_measure(w, args, flush)
    if with_roofline:
        reps = max(3, min(args.steps, 10))
        sm, sn = stage_times(w, cfg.chunk, reps, flush)
        res["stages_ms_per_step"] = {s: sm[s] / reps for s in binding.STAGES}
        res["roofline"] = roofline(cfg, acc, sm, sn, reps, bm, mode)
    return res, w


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c4",
                    help="c1..c5, c2p, c4n (default c4: the DeepSeek-V3-shaped MXFP4 layer, Zipf routing)")
    ap.add_argument("--chunk", type=int, default=None, help="chunk_experts (default: the workload's)")
    ap.add_argument("--tile-rows", type=int, default=0, help="grouped-GEMM tile rows (0: automatic)")
    ap.add_argument("--cpu-tokens", type=int, default=None, help="oracle token sample (default: sized per workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the chunk sweep and the other layer shapes")
    ap.add_argument("--weight-layout", choices=("auto", "rows", "kblocked"), default="auto",
                    help="weight code order for the fused forward: rows [N][K] or 16 x 128 tiles "
                         "(auto: tiles, except for the materialized mode)")
    ap.add_argument("--materialized", action="store_true",
                    help="time the materialized-chunk scheme (per-chunk BF16 weight copy + BF16 GEMMs) instead")
    ap.add_argument("--backward", action="store_true",
                    help="time the frozen-base backward (d_x, d_logits, d_adapter) instead")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the library runs one "
              "GPU's share of the layer; the expert-parallel split across GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch

    from precision_moe_expert_amd import binding
    mode = "materialized" if args.materialized else ("backward" if args.backward else "fused")
    flush = CacheFlush()
    head, w = measure_layer(args.config, args, flush, chunk=args.chunk, mode=mode)
    cfg = w.cfg
    result = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": {k: head[k] for k in ("workload", "tokens", "hidden", "experts", "top_k", "inter",
                                        "weight_format", "chunk_experts", "tile_rows", "oft_adapter",
                                        "weight_layout", "active_experts", "max_rows_per_expert", "mode")},
        "timing": "median of per-step HIP-event times; 512 MiB written to the GPU before every step",
        "ms_per_step_mean": head["ms_per_step_mean"],
        "tflops": head["tflops"],
        "pct_mfma_peak": head["pct_mfma_peak"],
        "hbm_gbps_algorithmic": head["hbm_gbps_algorithmic"],
        "pct_hbm_peak": head["pct_hbm_peak"],
        "intermediate_gbps": head["intermediate_gbps"],
        "stages_ms_per_step": head.get("stages_ms_per_step"),
        "temp_dequant_bytes": head["temp_dequant_bytes"],
        "workspace_bytes": head["workspace_bytes"],
        "roofline": head.get("roofline"),
    }
    if "lm_head" in head:
        result["lm_head"] = head["lm_head"]

    if not args.no_cpu_baseline:
        import oracle
        n = args.cpu_tokens or {1: 64, 2: 4096, 3: 256, 4: 1024, 5: 64, 6: 4096, 7: 512}[cfg.cfg_id]
        n = min(n, cfg.T)
        toks = np.arange(n, dtype=np.int32)
        c0 = time.perf_counter()
        if mode == "backward":
            d_out_f32 = (w.d_out_bits[toks].astype(np.uint32) << 16).view(np.float32)
            oracle.backward_inputs(w.li, d_out_f32, tokens=toks)
            ref = None
        else:
            ref = oracle.forward_inputs(w.li, tokens=toks, materialized=(mode == "materialized"))
        csec = time.perf_counter() - c0
        cb = {"value": n / csec, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
              "cpu_model": cpu_model(), "seconds": csec,
              "sample": f"first {n} of {cfg.T} tokens (full routing; every expert those tokens select is "
                        f"dequantized, chunk by chunk, then their rows run), one pass"}
        if ref is not None:
            got = w.out.float().cpu().numpy()[toks].astype(np.float64)
            ref = ref.astype(np.float64)
            dn = np.linalg.norm(got - ref, axis=1)
            rn = np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
            rms = np.maximum(np.sqrt(np.mean(ref * ref, axis=1)), 1e-30)
            cb["max_row_rel_err"] = float((dn / rn).max())
            cb["max_elem_abs_err_over_row_rms"] = float((np.abs(got - ref).max(axis=1) / rms).max())
        result["cpu_baseline"] = cb

    if not args.no_extras and mode == "fused":
        extras = {}
        # chunk-size sweep of the headline layer (same inputs)
        sweep = {}
        for c in sorted({8, 32, 64, cfg.chunk}):
            med, mean, _ = time_steps(lambda: w.step(c), args.steps, args.warmup, flush)
            sweep[str(c)] = {"ms_per_step": med, "tokens_per_s": cfg.T / (med / 1e3),
                             "workspace_bytes": binding.workspace_bytes(w.layer, c),
                             "pages_materialized_copy_bytes": min(c, cfg.E) * 3 * cfg.H * cfg.I * 2}
        extras["chunk_sweep"] = sweep
        del w
        torch.cuda.empty_cache()
        for name in ("c2", "c3", "c5"):
            if name == args.config:
                continue
            r, wx = measure_layer(name, args, flush)
            extras[name] = r
            del wx
            torch.cuda.empty_cache()
        result["extras"] = extras
    print(json.dumps(result))


def lm_head_measure(w: Workload, args, flush) -> dict:
    """Times moe_lm_head_logprob on the decode layer's output (64 x 7168 into
    a 32000 x 7168 bf16 head): HBM-bound on the head's 459 MB."""
    import torch

    from precision_moe_expert_amd import binding, synth
    cfg = w.cfg
    wlm, tgt = synth.gen_lm_head(cfg)
    wlm_d = torch.from_numpy(wlm.view(np.int16)).cuda().view(torch.bfloat16)
    tgt_d = torch.from_numpy(tgt).cuda()
    ws = binding.alloc_workspace(binding.lib().moe_lm_head_workspace_bytes(cfg.T, cfg.lm_vocab))
    med, mean, _ = time_steps(lambda: binding.lm_head_logprob(w.out, wlm_d, tgt_d, ws=ws), args.steps,
                              args.warmup, flush)
    nbytes = cfg.lm_vocab * cfg.H * 2 + cfg.T * cfg.H * 2 + cfg.T * 8
    gbps = nbytes / (med / 1e3) / 1e9
    return {"ms": med, "ms_mean": mean, "vocab": cfg.lm_vocab, "algorithmic_bytes": nbytes,
            "flops": 2.0 * cfg.T * cfg.H * cfg.lm_vocab,
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                         "frac": gbps / (HBM_PEAK / 1e9)}}


if __name__ == "__main__":
    main()
