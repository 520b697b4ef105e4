"""Pins of the oracle's materialized (BF16 temporary) numerics, CPU only.

The announcement's paragraph on active-expert-chunked dequantization (Orbit
announcement, 技术细节) read literally: each chunk's experts are dequantized
into a temporary high-precision copy and a grouped GEMM runs on it.  The
oracle's reading: the copy is BF16 (weights rounded once, nearest-even), GEMM
inputs are bf16, h is rounded to bf16, no activation quantizer.

Pins: the bf16 rounding against exact rational arithmetic on bit-built
neighbours and against torch's fp32 -> bf16 cast; the BF16 weight copy
against a round-to-odd re-derivation; the forward against the dense
brute force; chunk-size invariance; exact formats stay exact."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from precision_moe_expert_amd import synth
from tests import refimpl


def _neighbours(v: float):
    """The two bf16 values around v (toward zero, away from zero), built by
    clearing the 45 low mantissa bits of the float64 pattern."""
    b = np.array([v], np.float64).view(np.uint64)[0]
    lo = int(b) & ~((1 << 45) - 1)
    hi = lo + (1 << 45)
    return (np.array([lo], np.uint64).view(np.float64)[0], np.array([hi], np.uint64).view(np.float64)[0],
            (lo >> 45) & 1)


def test_round_bf16_is_nearest_ties_even():
    r = np.random.default_rng(11)
    v = r.standard_normal(4000) * np.exp2(r.integers(-60, 60, 4000))
    # exact midpoints between neighbours, both parities, both signs
    mids = []
    for base in (1.0, 1.0 + 2 ** -7, 3.5, 1e-20, 7e15):
        lo, hi, _ = _neighbours(base)
        mids += [lo + (hi - lo) / 2, -(lo + (hi - lo) / 2)]
    v = np.concatenate([v, mids, [0.0, 1.0, -2.0, 2 ** -126, 2 ** 127 * 1.5]])
    got = oracle.round_bf16(v)
    for x, g in zip(v, got):
        if x == 0:
            assert g == 0
            continue
        lo, hi, lo_odd = _neighbours(abs(x))
        fx, flo, fhi = Fraction(abs(x)), Fraction(lo), Fraction(hi)
        dlo, dhi = fx - flo, fhi - fx
        want = lo if dlo < dhi else hi if dhi < dlo else (hi if lo_odd else lo)
        assert g == np.copysign(want, x), (x, g, want)


def test_round_bf16_matches_torch_for_fp32_inputs():
    r = np.random.default_rng(12)
    v32 = (r.standard_normal(100000) * np.exp2(r.integers(-30, 30, 100000))).astype(np.float32)
    # every fp32 pattern that sits exactly half-way between two bf16 values
    ties = (r.integers(0, 1 << 15, 2000).astype(np.uint32) << 16 | 0x8000).astype(np.uint32)
    ties = ties.view(np.float32)
    ties = ties[np.isfinite(ties) & (np.abs(ties) > 1e-30)]
    v32 = np.concatenate([v32, ties])
    want = torch.from_numpy(v32).to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(oracle.round_bf16(v32.astype(np.float64)), want)


@pytest.mark.parametrize("fmt", [1, 2, 3, 4])
def test_dequant_bf16_copy(fmt):
    cfg = synth.LayerConfig("mat_pin", 70 + fmt, T=8, H=256, E=2, k=1, I=128, fmt=fmt, chunk=1)
    li = synth.make_inputs(cfg)
    for e in range(cfg.E):
        got = oracle.dequant_bf16(fmt, 2 * cfg.I, cfg.H, li.w13[e], li.s13[e]).astype(np.float64)
        exact = refimpl.dequant(fmt, li.w13[e], li.s13[e], 2 * cfg.I, cfg.H)
        assert np.array_equal(got, refimpl.bf16_round_rto(exact))
        if fmt == 3:
            # E2M1 times a power of two has at most 2 significant bits: the copy is exact
            assert np.array_equal(got, exact)


def test_int4_with_pow2_scales_copy_is_exact():
    r = np.random.default_rng(3)
    N, K = 64, 128
    q = r.integers(0, 256, (N, K // 2)).astype(np.uint8)
    s = synth._to_bf16_bits(np.exp2(r.integers(-9, -3, (K // 32, N))).astype(np.float32))
    got = oracle.dequant_bf16(1, N, K, q, s)
    assert np.array_equal(got, oracle.dequant(1, N, K, q, s))


def tiny(fmt, oft=False, E=6, k=2, chunk=2, zipf=0.0):
    return synth.LayerConfig("tiny_mat", 80 + fmt, T=24, H=128, E=E, k=k, I=128, fmt=fmt, chunk=chunk,
                             oft=oft, zipf_alpha=zipf)


@pytest.mark.parametrize("fmt,oft", [(1, False), (1, True), (2, False), (3, False), (4, False)])
def test_materialized_forward_vs_dense_bruteforce(fmt, oft):
    cfg = tiny(fmt, oft=oft)
    li = synth.make_inputs(cfg)
    out = oracle.forward_inputs(li, materialized=True)
    ref, _, _ = refimpl.dense_moe(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, fmt, li.x, li.logits,
                                   li.w13, li.w2, li.s13, li.s2, oft=li.oft, materialized=True)
    rel = np.linalg.norm(out - ref, axis=1) / np.linalg.norm(ref, axis=1)
    # h is rounded to bf16 after fp64 sums taken in different orders: a rare
    # element may land on the other side of a rounding boundary
    assert rel.max() <= 1e-3, rel.max()
    assert np.mean(rel <= 1e-6) >= 0.9
    # and the two numerics really differ (bf16 copies vs the format's own path)
    fused = oracle.forward_inputs(li)
    assert np.max(np.abs(fused - out)) > 0


def test_materialized_chunk_invariance():
    cfg = tiny(2, E=7, k=3, zipf=1.2)
    li = synth.make_inputs(cfg)
    outs = [oracle.forward_inputs(li, chunk_experts=c, materialized=True) for c in (1, 3, 7)]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
