"""GPU parity of the materialized-chunk scheme (moe_expert_forward_materialized:
each chunk's experts dequantized to a BF16 copy, then BF16 grouped GEMMs)
against the oracle's materialized numerics, through the C ABI; and the
mismatch harness: the token-mult-prob-error (NeMo RL FP8 post) between the
fused low-precision numerics and the BF16-copy numerics on the decode layer's
LM-head log-probs, on the GPU and in the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
from precision_moe_expert_amd import binding, synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def small(fmt, T=77, H=256, I=384, E=12, k=3, oft=False, zipf=0.0, chunk=4, cfg_id=None):
    return synth.LayerConfig(f"mat_f{fmt}", cfg_id or (140 + fmt + (5 if oft else 0)), T=T, H=H, E=E, k=k, I=I,
                             fmt=fmt, chunk=chunk, oft=oft, zipf_alpha=zipf)


def check(li, chunk=None, tile_rows=0):
    d = gu.DevInputs(li)
    d.layer.tile_rows = tile_rows
    out = gu.bf16_to_np(d.forward_materialized(chunk=chunk))
    ref = oracle.forward_inputs(li, materialized=True)
    err = gu.row_rel_err(out, ref)
    print(f"{li.cfg.name} tile {tile_rows}: max row rel err {err.max():.3e}, mean {err.mean():.3e}")
    assert err.max() <= gu.ROW_TOL
    return d


@pytest.mark.parametrize("fmt", [1, 2, 3, 4, 5])
def test_materialized_small_vs_oracle(fmt):
    check(synth.make_inputs(small(fmt)))


def test_materialized_int4_oft_vs_oracle():
    check(synth.make_inputs(small(1, T=53, H=512, I=256, E=9, k=4, oft=True, chunk=2)))


@pytest.mark.parametrize("fmt", [1, 2, 3, 5])
@pytest.mark.parametrize("tile_rows", [16, 32, 64, 128])
def test_materialized_every_tile_height(fmt, tile_rows):
    """~250 rows per expert: tall tiles run full and ragged; I = 768 gives six
    128-wide h blocks and H = 512 two 256-wide output blocks."""
    check(synth.make_inputs(small(fmt, T=300, H=512, I=768, E=5, k=4, chunk=2, cfg_id=160 + fmt)),
          tile_rows=tile_rows)


@pytest.mark.parametrize("fmt", [1, 2])
def test_materialized_chunk_size_bitwise_invariance(fmt):
    cfg = small(fmt, E=9, k=3, zipf=1.2)
    d = gu.DevInputs(synth.make_inputs(cfg))
    outs = [d.forward_materialized(chunk=c).clone() for c in (1, 2, 4, 9, 64)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


@pytest.mark.parametrize("fmt,oft", [(1, False), (1, True), (2, False), (3, False), (4, False), (5, False)])
def test_materialized_tiled_codes_bitwise(fmt, oft):
    """Codes in 16 x 128 tiles give the same BF16 copy, so the same bits as rows."""
    cfg = small(fmt, H=512, I=384, oft=oft, cfg_id=170 + fmt + (10 if oft else 0))
    li = synth.make_inputs(cfg)
    d = gu.DevInputs(li)
    a = d.forward_materialized().clone()
    w13, w2 = binding.pack_weights_kblocked(d.layer, d.w13, d.w2)
    lk = binding.make_layer(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.fmt, oft=cfg.oft,
                            weight_layout=binding.WL_KBLOCKED)
    b = binding.expert_forward_materialized(lk, d.x, d.logits, w13, w2, d.s13, d.s2, adapter=d.oft,
                                            chunk_experts=cfg.chunk, g13=d.g13, g2=d.g2)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_materialized_timed_matches_untimed():
    li = synth.make_inputs(small(2))
    d = gu.DevInputs(li)
    a = d.forward_materialized().clone()
    b, st = binding.expert_forward_materialized(d.layer, d.x, d.logits, d.w13, d.w2, d.s13, d.s2,
                                                chunk_experts=li.cfg.chunk, timed=True)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    nchunks = -(-li.cfg.E // li.cfg.chunk)
    assert st["dequant"][1] == nchunks and st["gemm1"][1] == nchunks and st["gemm2"][1] == nchunks


def test_materialized_fullsize_fp8_sampled():
    cfg = synth.CONFIGS["c2"]
    li = synth.make_inputs(cfg, with_lm=False)
    d = gu.DevInputs(li)
    out = d.forward_materialized()
    torch.cuda.synchronize()
    toks = np.sort(np.random.default_rng(7).choice(cfg.T, size=32, replace=False)).astype(np.int32)
    ref = oracle.forward_inputs(li, tokens=toks, materialized=True)
    err = gu.row_rel_err(gu.bf16_to_np(out)[toks], ref)
    print(f"c2 materialized: max row rel err {err.max():.3e}")
    assert err.max() <= gu.ROW_TOL


def tmpe(a, b):
    """token-mult-prob-error: mean over tokens of exp(|logp_a - logp_b|)."""
    return float(np.mean(np.exp(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))))


def test_mismatch_harness_decode_lm_head():
    cfg = synth.CONFIGS["c5"]
    li = synth.make_inputs(cfg, with_lm=True)
    d = gu.DevInputs(li)
    wlm, tg = gu.dev(li.w_lm, "bf16"), gu.dev(li.targets)
    out_f = d.forward().clone()
    out_m = d.forward_materialized().clone()
    lp_f = binding.lm_head_logprob(out_f, wlm, tg).cpu().numpy()
    lp_m = binding.lm_head_logprob(out_m, wlm, tg).cpu().numpy()
    ref_f = oracle.forward_inputs(li)
    ref_m = oracle.forward_inputs(li, materialized=True)
    assert gu.row_rel_err(gu.bf16_to_np(out_m), ref_m).max() <= gu.ROW_TOL
    lpr_f = oracle.lm_head_logprob(ref_f, li.w_lm, li.targets)
    lpr_m = oracle.lm_head_logprob(ref_m, li.w_lm, li.targets)
    # each GPU path against the oracle of its own numerics
    assert tmpe(lp_f, lpr_f) <= math.exp(1e-2)
    assert tmpe(lp_m, lpr_m) <= math.exp(1e-2)
    # the mismatch between the two numerics, GPU and oracle
    gpu_mm, ref_mm = tmpe(lp_f, lp_m), tmpe(lpr_f, lpr_m)
    print(f"decode token-mult-prob-error fused vs BF16 copy: GPU {gpu_mm:.6f}, oracle {ref_mm:.6f}")
    assert gpu_mm >= 1.0 and ref_mm > 1.0
    assert abs(math.log(gpu_mm) - math.log(ref_mm)) <= 1e-2
