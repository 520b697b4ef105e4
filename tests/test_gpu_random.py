"""Seeded random layer shapes against the oracle, through the C ABI.

Each case draws a weight format, hidden and inter sizes, expert count, top-k,
token count, chunk size, tile height, weight layout, uniform or Zipf-skewed
routing, and with or without the OFT adapter (per-expert or one shared R),
from a fixed seed; the GPU output is checked row by row against the oracle
(tests/gpu_util.check_rows), and a second chunk size must give the same
bits.  Sizes stay small enough for the oracle to finish in about a second
per case."""
import numpy as np
import pytest
import torch

import oracle
from precision_moe_expert_amd import binding, synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

N_CASES = 30
TILES = [0, 16, 32, 48, 64, 96, 128, 192]


def draw(i: int):
    r = np.random.default_rng([20261203, i])
    fmt = 1 + i % 5
    H = 256 * int(r.integers(1, 5))
    I = 128 * int(r.integers(1, 7))
    E = int(r.integers(1, 41))
    k = int(r.integers(1, min(E, 8) + 1))
    T = int(r.integers(1, 201))
    chunk = int(r.integers(1, E + 2))
    chunk2 = int(r.integers(1, E + 2))
    tile = TILES[int(r.integers(0, len(TILES)))]
    oft = bool(r.integers(0, 2))
    shared = oft and bool(r.integers(0, 2))
    zipf = float(r.choice([0.0, 0.8, 1.2]))
    layout = int(r.integers(0, 2))
    cfg = synth.LayerConfig(f"random_{i}", 400 + i, T=T, H=H, E=E, k=k, I=I, fmt=fmt, chunk=chunk, oft=oft,
                            zipf_alpha=zipf)
    return cfg, chunk2, tile, shared, layout


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_vs_oracle(i):
    cfg, chunk2, tile, shared, layout = draw(i)
    li = synth.make_inputs(cfg)
    d = gu.DevInputs(li)
    oft_ref = None
    if cfg.oft:
        if shared:
            oft_ref = np.ascontiguousarray(li.oft[0])
            d.oft = gu.dev(oft_ref, "bf16")
        else:
            oft_ref = li.oft
    layer = binding.make_layer(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.fmt, oft=cfg.oft,
                               adapter_expert_stride=0 if shared else None, tile_rows=tile,
                               weight_layout=layout)
    w13, w2 = d.w13, d.w2
    if layout == binding.WL_KBLOCKED:
        w13, w2 = binding.pack_weights_kblocked(d.layer, d.w13, d.w2)

    def fwd(c):
        return binding.expert_forward(layer, d.x, d.logits, w13, w2, d.s13, d.s2, adapter=d.oft, chunk_experts=c,
                                      g13=d.g13, g2=d.g2)

    out = fwd(cfg.chunk)
    out2 = fwd(chunk2)
    torch.cuda.synchronize()
    label = (f"case {i}: fmt {cfg.fmt} T {cfg.T} H {cfg.H} I {cfg.I} E {cfg.E} k {cfg.k} chunk {cfg.chunk}/{chunk2} "
             f"tile {tile} oft {cfg.oft}{' shared' if shared else ''} zipf {cfg.zipf_alpha} layout {layout}")
    print(label, flush=True)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), f"{label}: chunk sizes differ"
    ref = oracle.forward(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.fmt, li.x, li.logits, li.w13, li.w2, li.s13,
                         li.s2, oft=oft_ref, chunk_experts=cfg.chunk,
                         adapter_expert_stride=0 if shared else None, g13=li.g13, g2=li.g2)
    gu.check_rows(gu.bf16_to_np(out), ref, cfg.fmt, label)
