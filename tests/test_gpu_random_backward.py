"""Seeded random layer shapes for the frozen-base backward (d_x, d_logits and,
with the OFT adapter, d_adapter) against the oracle's fp64 backward, through
the C ABI.  Each case draws a weight format, hidden and inter sizes, expert
count, top-k, token count, chunk size, tile height, weight layout, routing
skew and whether the adapter is present from a fixed seed; the checks and
bounds are those of tests/test_gpu_backward.py."""
import numpy as np
import pytest
import torch

from precision_moe_expert_amd import binding, synth
from tests import gpu_util as gu
from tests.test_gpu_backward import check, d_out_of

pytestmark = pytest.mark.gpu

N_CASES = 20
TILES = [0, 16, 32, 48, 64, 96, 128, 192]


def draw(i: int):
    r = np.random.default_rng([20261204, i])
    fmt = 1 + i % 5
    H = 256 * int(r.integers(1, 4))
    I = 256 * int(r.integers(1, 3))  # the backward needs I % 256 == 0
    E = int(r.integers(1, 25))
    k = int(r.integers(1, min(E, 6) + 1))
    T = int(r.integers(1, 121))
    chunk = int(r.integers(1, E + 2))
    tile = TILES[int(r.integers(0, len(TILES)))]
    oft = bool(r.integers(0, 2))
    zipf = float(r.choice([0.0, 0.8, 1.2]))
    layout = int(r.integers(0, 2))
    cfg = synth.LayerConfig(f"random_bwd_{i}", 500 + i, T=T, H=H, E=E, k=k, I=I, fmt=fmt, chunk=chunk, oft=oft,
                            zipf_alpha=zipf)
    return cfg, tile, layout


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_backward_vs_oracle(i):
    cfg, tile, layout = draw(i)
    li = synth.make_inputs(cfg)
    d = gu.DevInputs(li)
    layer = binding.make_layer(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.fmt, oft=cfg.oft, tile_rows=tile,
                               weight_layout=layout)
    w13, w2 = (d.w13, d.w2) if layout == binding.WL_ROWS else binding.pack_weights_kblocked(layer, d.w13, d.w2)
    bw = binding.prepare_backward_weights(layer, w13, w2, d.s13, d.s2)
    dout_bits = d_out_of(cfg, 11 + i)
    print(f"case {i}: fmt {cfg.fmt} T {cfg.T} H {cfg.H} I {cfg.I} E {cfg.E} k {cfg.k} chunk {cfg.chunk} "
          f"tile {tile} oft {cfg.oft} zipf {cfg.zipf_alpha} layout {layout}", flush=True)
    got = binding.expert_backward(layer, d.x, d.logits, w13, w2, d.s13, d.s2, bw, gu.dev(dout_bits, "bf16"),
                                  adapter=d.oft, chunk_experts=cfg.chunk, g13=d.g13, g2=d.g2)
    torch.cuda.synchronize()
    check(li, dout_bits, got)
