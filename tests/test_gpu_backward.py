"""GPU parity of the frozen-base backward (moe_expert_backward, INT4 weights)
against the oracle's fp64 backward, through the C ABI.

Transposed weight copy: bit-exact against numpy.  Gradients: d_x per token
row within the forward's relative L2 bound (ROW_TOL); d_logits per token
within ROW_TOL of the token's gradient norm (floor: 1e-3 of the layer's RMS
row norm, for tokens whose selected experts give nearly equal <d_out, y>);
d_adapter per expert within ROW_TOL (Frobenius).  The GPU rounds d_out and
the SwiGLU gradients to fp16 (2^-11 relative) and recomputes the
pre-activations from fp16 x R_e, so its errors are ~1e-3 of these norms."""
import numpy as np
import pytest
import torch

import oracle
from precision_moe_expert_amd import binding, synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def small(T=77, H=256, I=256, E=12, k=3, oft=False, zipf=0.0, chunk=4, cfg_id=None):
    return synth.LayerConfig("bwd_small", cfg_id or (240 + (5 if oft else 0)), T=T, H=H, E=E, k=k, I=I, fmt=1,
                             chunk=chunk, oft=oft, zipf_alpha=zipf)


def d_out_of(cfg, seed=5):
    r = np.random.default_rng(seed)
    return synth._to_bf16_bits(r.standard_normal((cfg.T, cfg.H)).astype(np.float32))


class Bwd:
    def __init__(self, li, tile_rows=0):
        self.d = gu.DevInputs(li)
        self.d.layer.tile_rows = tile_rows
        d = self.d
        self.bw = binding.prepare_backward_weights(d.layer, d.w13, d.w2, d.s13, d.s2)

    def run(self, dout_bits, chunk=None):
        d = self.d
        c = d.li.cfg
        return binding.expert_backward(d.layer, d.x, d.logits, d.w13, d.w2, d.s13, d.s2, self.bw,
                                       gu.dev(dout_bits, "bf16"), adapter=d.oft,
                                       chunk_experts=c.chunk if chunk is None else chunk)


def check(li, dout_bits, got, tokens=None, check_adapter=True):
    from tests import refimpl
    dout = refimpl.bf16_to_f32(dout_bits).reshape(li.cfg.T, li.cfg.H)
    toks = np.arange(li.cfg.T) if tokens is None else tokens
    rdx, rdl, rdR = oracle.backward_inputs(li, dout[toks], tokens=None if tokens is None else toks)
    dx = gu.bf16_to_np(got[0])[toks]
    dl = got[1].cpu().numpy()[toks].astype(np.float64)
    ex = gu.row_rel_err(dx, rdx)
    scale = np.linalg.norm(rdl, axis=1)
    floor = 1e-3 * np.sqrt(np.mean(scale ** 2))
    el = np.linalg.norm(dl - rdl, axis=1) / np.maximum(scale, floor)
    msg = f"{li.cfg.name}: d_x max row rel err {ex.max():.3e}; d_logits max rel err {el.max():.3e}"
    if li.oft is not None and check_adapter:
        dR = got[2].cpu().numpy().astype(np.float64)
        act = np.unique(oracle.route(li.logits, li.cfg.k)[0])
        eR = np.array([np.linalg.norm(dR[e] - rdR[e]) / np.linalg.norm(rdR[e]) for e in act])
        msg += f"; d_adapter max expert rel err {eR.max():.3e}"
        inact = np.setdiff1d(np.arange(li.cfg.E), act)
        assert np.all(dR[inact] == 0)
        assert eR.max() <= gu.ROW_TOL
    print(msg)
    assert ex.max() <= gu.ROW_TOL
    assert el.max() <= gu.ROW_TOL


def test_backward_weight_copy_bitexact():
    cfg = small(T=8, H=256, I=512, E=3, k=1)
    li = synth.make_inputs(cfg)
    b = Bwd(li)
    raw = b.bw.cpu().numpy()
    H, I, E = cfg.H, cfg.I, cfg.E

    def al(v):
        return (v + 255) // 256 * 256

    o13 = 0
    o2 = al(E * H * 2 * I // 2)
    os13 = o2 + al(E * I * H // 2)
    os2 = os13 + al(E * (H // 32) * 2 * I * 2)

    def nib_t(packed, N, K):
        from tests import refimpl
        v = refimpl.unpack_nibbles(packed).reshape(N, K).T.copy()          # [K][N] nibbles
        return (v[:, 0::2] | (v[:, 1::2] << 4)).astype(np.uint8)

    def f16_pairs(s_bits, G, L):
        from tests import refimpl
        f = refimpl.bf16_to_f32(s_bits).reshape(G, L // 8, 8)
        out = np.empty((G, L // 8, 8), np.float16)
        for w, (a, b_, d) in enumerate(((0, 4, 1.0), (1, 5, 1 / 16), (2, 6, 1.0), (3, 7, 1 / 16))):
            out[:, :, 2 * w] = (f[:, :, a] * d).astype(np.float16)
            out[:, :, 2 * w + 1] = (f[:, :, b_] * d).astype(np.float16)
        return out.view(np.uint8).reshape(-1)

    for e in range(E):
        w13t = raw[o13 + e * H * I: o13 + (e + 1) * H * I]
        assert np.array_equal(w13t, nib_t(li.w13[e], 2 * I, H).reshape(-1))
        w2t = raw[o2 + e * H * I // 2: o2 + (e + 1) * H * I // 2]
        assert np.array_equal(w2t, nib_t(li.w2[e], H, I).reshape(-1))
        n13 = (H // 32) * 2 * I * 2
        assert np.array_equal(raw[os13 + e * n13: os13 + (e + 1) * n13], f16_pairs(li.s13[e], H // 32, 2 * I))
        n2 = (I // 32) * H * 2
        assert np.array_equal(raw[os2 + e * n2: os2 + (e + 1) * n2], f16_pairs(li.s2[e], I // 32, H))


@pytest.mark.parametrize("oft", [False, True])
def test_backward_small_vs_oracle(oft):
    li = synth.make_inputs(small(oft=oft))
    dout = d_out_of(li.cfg)
    check(li, dout, Bwd(li).run(dout))


@pytest.mark.parametrize("tile_rows", [16, 32, 48, 64, 96, 128, 192])
def test_backward_every_tile_height(tile_rows):
    li = synth.make_inputs(small(T=300, H=512, I=512, E=5, k=4, chunk=2, oft=True, cfg_id=250))
    dout = d_out_of(li.cfg, 6)
    check(li, dout, Bwd(li, tile_rows).run(dout))


def test_backward_chunk_size_bitwise_invariance():
    li = synth.make_inputs(small(E=9, k=3, zipf=1.2, oft=True))
    dout = d_out_of(li.cfg, 7)
    b = Bwd(li)
    ref = [t.clone() for t in b.run(dout, chunk=1)]
    torch.cuda.synchronize()
    for c in (2, 4, 9, 64):
        got = b.run(dout, chunk=c)
        torch.cuda.synchronize()
        assert torch.equal(got[0].view(torch.int16), ref[0].view(torch.int16))
        assert torch.equal(got[1], ref[1]) and torch.equal(got[2], ref[2])


@pytest.mark.slow
def test_backward_decode_fullsize():
    """Decode shape (64 tokens, 384 experts, H 7168, I 2048, OFT): every token,
    every expert's adapter gradient."""
    li = synth.make_inputs(synth.CONFIGS["c5"], with_lm=False)
    dout = d_out_of(li.cfg, 8)
    check(li, dout, Bwd(li).run(dout))


@pytest.mark.slow
def test_backward_kimi_fullsize_sampled():
    """Kimi-K2 shape (8192 tokens, OFT): d_x and d_logits on sampled tokens."""
    li = synth.make_inputs(synth.CONFIGS["c3"], with_lm=False)
    dout = d_out_of(li.cfg, 9)
    got = Bwd(li).run(dout)
    torch.cuda.synchronize()
    toks = np.sort(np.random.default_rng(3).choice(li.cfg.T, size=12, replace=False)).astype(np.int32)
    check(li, dout, got, tokens=toks, check_adapter=False)
