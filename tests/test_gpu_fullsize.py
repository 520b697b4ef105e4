"""Full-size parity: each layer configuration at its real shape, run on the GPU
exactly as bench.py runs it (same chunk size, automatic tile height), checked
against the oracle.

- Qwen3-30B-A3B shape (FP8, both scale variants): every token.
- Kimi-K2, DeepSeek-V3 (MXFP4, NVFP4) shapes: the tokens that own the first
  and the last permuted row of every active expert (so every expert's first
  tile and ragged last tile is compared), the rows on either side of the
  expert's last full-tile boundary, and a seeded sample of other tokens.  The
  oracle computes only those tokens' rows; routing and chunking stay global.
- Decode shape: every token, then the LM-head log-probs of seeded targets
  against the oracle's (|delta| <= 1e-2, i.e. a token-mult-prob-error at most
  e^0.01; NeMo RL FP8 post, token-mult-prob-error).

Per row: relative L2 error within the per-format bound and max element error
over the row RMS within ELEM_TOL (tests/gpu_util.py)."""
import math

import numpy as np
import pytest
import torch

import oracle
from precision_moe_expert_amd import binding, synth
from tests import gpu_util as gu

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def covering_tokens(li, bm, n_extra, seed):
    """Tokens owning each active expert's first and last row, the rows around
    its last full-tile boundary, plus n_extra seeded random tokens."""
    c = li.cfg
    ids, _ = oracle.route(li.logits, c.k)
    P = oracle.permute(ids, c.E)
    off, sr = P["offsets"], P["sorted_rows"]
    rows = set()
    for e in P["active"]:
        a, b = int(off[e]), int(off[e + 1])
        rows.update((a, b - 1))
        n = b - a
        if n > bm:
            last_full = a + (n // bm) * bm
            rows.update(r for r in (last_full - 1, last_full) if a <= r < b)
    toks = {int(sr[r]) // c.k for r in rows}
    r = np.random.default_rng(seed)
    toks.update(int(t) for t in r.choice(c.T, size=min(n_extra, c.T), replace=False))
    return np.array(sorted(toks), np.int32), len(P["active"])


def run_full(name, chunk=None, all_tokens=False, n_extra=16):
    cfg = synth.CONFIGS[name]
    li = synth.make_inputs(cfg, with_lm=False)
    d = gu.DevInputs(li)
    out = d.forward(chunk=chunk)
    torch.cuda.synchronize()
    if all_tokens:
        toks, what = np.arange(cfg.T, dtype=np.int32), "all"
    else:
        toks, na = covering_tokens(li, binding.tile_rows(d.layer), n_extra, 7)
        what = f"{na} active experts covered by"
    got = gu.bf16_to_np(out)[toks]
    ref = oracle.forward_inputs(li, tokens=toks, chunk_experts=chunk)
    gu.check_rows(got, ref, cfg.fmt, f"{name} ({what} {len(toks)} tokens)")
    return d, out


def test_qwen3_30b_a3b_fp8_full():
    run_full("c2", all_tokens=True)


def test_qwen3_30b_a3b_fp8_pow2_full():
    run_full("c2p", all_tokens=True)


def test_kimi_k2_int4_oft_full():
    run_full("c3")


def test_deepseek_v3_nvfp4_zipf_full():
    run_full("c4n")


def test_deepseek_v3_mxfp4_zipf_full_and_chunk_sweep():
    d, out = run_full("c4", chunk=32)
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
    gu.check_rows(gu.bf16_to_np(out), ref_out, cfg.fmt, "decode (all 64 tokens)")
    lp_ref = oracle.lm_head_logprob(ref_out, li.w_lm, li.targets)
    delta = np.abs(lp.astype(np.float64) - lp_ref.astype(np.float64))
    tmpe = float(np.mean(np.exp(delta)))
    print(f"decode: log-prob max |delta| {delta.max():.3e}, token-mult-prob-error {tmpe:.6f}")
    assert delta.max() <= 1e-2
    assert tmpe <= math.exp(1e-2)
