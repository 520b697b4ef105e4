"""Full-size parity: each layer configuration at its real shape, run on the GPU
exactly as bench.py runs it (same chunk size, automatic tile height), checked
against the oracle on a seeded sample of tokens (the oracle computes only the
sampled tokens' rows; routing and chunking are still global).

Decode shape: every token is checked, then the LM-head log-probs of seeded
targets are compared with the oracle's (|delta| <= 1e-2, i.e. a
token-mult-prob-error at most e^0.01; NeMo RL FP8 post, token-mult-prob-error)."""
import math

import numpy as np
import pytest
import torch

import oracle
from precision_moe_expert_amd import binding, synth
from tests import gpu_util as gu

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def sample_tokens(T, n, seed):
    r = np.random.default_rng(seed)
    return np.sort(r.choice(T, size=min(n, T), replace=False)).astype(np.int32)


def run_full(name, n_sample, chunk=None):
    cfg = synth.CONFIGS[name]
    li = synth.make_inputs(cfg, with_lm=False)
    d = gu.DevInputs(li)
    out = d.forward(chunk=chunk)
    torch.cuda.synchronize()
    toks = sample_tokens(cfg.T, n_sample, 7)
    got = gu.bf16_to_np(out)[toks]
    ref = oracle.forward_inputs(li, tokens=toks, chunk_experts=chunk)
    err = gu.row_rel_err(got, ref)
    print(f"{name}: {len(toks)} sampled tokens, max row rel err {err.max():.3e}, mean {err.mean():.3e}")
    assert err.max() <= gu.ROW_TOL
    return d, out


def test_qwen3_30b_a3b_fp8_full():
    run_full("c2", 64)


def test_qwen3_30b_a3b_fp8_pow2_full():
    run_full("c2p", 64)


def test_kimi_k2_int4_oft_full():
    run_full("c3", 16)


def test_deepseek_v3_nvfp4_zipf_full():
    run_full("c4n", 16)


def test_deepseek_v3_mxfp4_zipf_full_and_chunk_sweep():
    d, out = run_full("c4", 16, chunk=32)
    ref = out.clone()
    for c in (8, 64):
        o = d.forward(chunk=c)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), f"chunk {c} differs"


def test_decode_int4_oft_lm_head_logprob():
    cfg = synth.CONFIGS["c5"]
    li = synth.make_inputs(cfg, with_lm=True)
    d = gu.DevInputs(li)
    out = d.forward()
    lp = binding.lm_head_logprob(out, gu.dev(li.w_lm, "bf16"), gu.dev(li.targets)).cpu().numpy()
    ref_out = oracle.forward_inputs(li)
    err = gu.row_rel_err(gu.bf16_to_np(out), ref_out)
    assert err.max() <= gu.ROW_TOL
    lp_ref = oracle.lm_head_logprob(ref_out, li.w_lm, li.targets)
    delta = np.abs(lp.astype(np.float64) - lp_ref.astype(np.float64))
    tmpe = float(np.mean(np.exp(delta)))
    print(f"decode: max row rel err {err.max():.3e}; log-prob max |delta| {delta.max():.3e}, "
          f"token-mult-prob-error {tmpe:.6f}")
    assert delta.max() <= 1e-2
    assert tmpe <= math.exp(1e-2)
