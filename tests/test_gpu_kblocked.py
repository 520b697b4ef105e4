"""GPU tests of the 16-row x 128-K tiled code layout (MOE_WL_KBLOCKED) of
the weights of every format, through the C ABI.

The tiled copy (moe_pack_weights_kblocked) is checked byte for byte against
a numpy re-layout of the row-major codes.  Only the addresses the GEMMs read
change, so the fused forward on the tiled copy must equal the forward on the
row-major codes bit for bit; it is also checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from precision_moe_expert_amd import binding, synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def tiled_np(codes, N, K, kb):
    """[N][K*kb/128] bytes -> [N/16][K/128][16][kb] bytes."""
    return np.ascontiguousarray(codes.reshape(N // 16, 16, K // 128, kb).transpose(0, 2, 1, 3)).reshape(-1)


def run(d, layout, w13, w2, tile_rows=0, chunk=None):
    c = d.li.cfg
    layer = binding.make_layer(c.T, c.H, c.I, c.E, c.k, c.fmt, oft=d.oft is not None, tile_rows=tile_rows,
                               weight_layout=layout)
    return binding.expert_forward(layer, d.x, d.logits, w13, w2, d.s13, d.s2, adapter=d.oft,
                                  chunk_experts=c.chunk if chunk is None else chunk, g13=d.g13, g2=d.g2)


@pytest.mark.parametrize("fmt", [1, 2, 3, 5])
def test_pack_bitexact(fmt):
    cfg = synth.LayerConfig("kblk_pack", 290 + fmt, T=8, H=512, E=3, k=1, I=384, fmt=fmt, chunk=1)
    li = synth.make_inputs(cfg)
    d = gu.DevInputs(li)
    o13, o2 = binding.pack_weights_kblocked(d.layer, d.w13, d.w2)
    torch.cuda.synchronize()
    g13, g2 = o13.cpu().numpy().reshape(cfg.E, -1), o2.cpu().numpy().reshape(cfg.E, -1)
    kb = 128 if fmt == 2 else 64
    for e in range(cfg.E):
        w13 = np.asarray(li.w13[e]).reshape(2 * cfg.I, -1)
        w2 = np.asarray(li.w2[e]).reshape(cfg.H, -1)
        assert np.array_equal(g13[e], tiled_np(w13, 2 * cfg.I, cfg.H, kb))
        assert np.array_equal(g2[e], tiled_np(w2, cfg.H, cfg.I, kb))


@pytest.mark.parametrize("fmt,oft", [(1, False), (1, True), (2, False), (3, False), (4, False), (5, False)])
@pytest.mark.parametrize("tile_rows", [16, 32, 64, 128, 160, 192])
def test_forward_kblocked_equals_rows(fmt, oft, tile_rows):
    cfg = synth.LayerConfig("kblk_fwd", 300 + fmt + (5 if oft else 0), T=150, H=512, E=7, k=3, I=384, fmt=fmt,
                            chunk=3, oft=oft, zipf_alpha=0.8)
    li = synth.make_inputs(cfg)
    d = gu.DevInputs(li)
    o13, o2 = binding.pack_weights_kblocked(d.layer, d.w13, d.w2)
    ref = run(d, binding.WL_ROWS, d.w13, d.w2, tile_rows).clone()
    got = run(d, binding.WL_KBLOCKED, o13, o2, tile_rows)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    err = gu.row_rel_err(gu.bf16_to_np(got), oracle.forward_inputs(li))
    print(f"fmt {fmt} oft {oft} tile {tile_rows}: max row rel err {err.max():.3e}")
    assert err.max() <= gu.ROW_TOL


@pytest.mark.slow
@pytest.mark.parametrize("name", ["c5", "c3", "c2", "c2p", "c4"])
def test_fullsize_kblocked_equals_rows(name):
    """Decode and Kimi-K2 shapes (INT4 + OFT), Qwen3 shape (FP8, both scale
    kinds), DeepSeek-V3 shape (MXFP4): bit-identical outputs."""
    li = synth.make_inputs(synth.CONFIGS[name], with_lm=False)
    d = gu.DevInputs(li)
    o13, o2 = binding.pack_weights_kblocked(d.layer, d.w13, d.w2)
    ref = run(d, binding.WL_ROWS, d.w13, d.w2).clone()
    got = run(d, binding.WL_KBLOCKED, o13, o2)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("fmt,oft", [(1, True), (2, False), (3, False), (4, False), (5, False)])
def test_backward_kblocked_equals_rows(fmt, oft):
    """The backward on tiled codes: the transposed copy made from the tiles
    equals the one made from rows byte for byte, and d_x, d_logits and
    d_adapter are bit-identical."""
    cfg = synth.LayerConfig("kblk_bwd", 310 + fmt + (5 if oft else 0), T=90, H=512, E=6, k=3, I=512, fmt=fmt,
                            chunk=2, oft=oft, zipf_alpha=0.5)
    li = synth.make_inputs(cfg)
    d = gu.DevInputs(li)
    r = np.random.default_rng(3)
    dout = gu.dev(synth._to_bf16_bits(r.standard_normal((cfg.T, cfg.H)).astype(np.float32)), "bf16")
    outs, copies = [], []
    for wl in (binding.WL_ROWS, binding.WL_KBLOCKED):
        layer = binding.make_layer(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.fmt, oft=oft, weight_layout=wl)
        w13, w2 = (d.w13, d.w2) if wl == binding.WL_ROWS else binding.pack_weights_kblocked(layer, d.w13, d.w2)
        # zero-filled so that the alignment padding between sections compares equal
        bw = torch.zeros(binding.backward_weights_bytes(layer), dtype=torch.uint8, device="cuda")
        binding.prepare_backward_weights(layer, w13, w2, d.s13, d.s2, out=bw)
        got = binding.expert_backward(layer, d.x, d.logits, w13, w2, d.s13, d.s2, bw, dout, adapter=d.oft,
                                      chunk_experts=cfg.chunk, g13=d.g13, g2=d.g2)
        torch.cuda.synchronize()
        copies.append(bw.clone())
        outs.append([None if t is None else t.clone() for t in got])
    assert torch.equal(copies[0], copies[1])
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1])
    if oft:
        assert torch.equal(outs[0][2], outs[1][2])
