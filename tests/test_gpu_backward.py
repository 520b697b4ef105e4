"""GPU parity of the frozen-base backward (moe_expert_backward; INT4, FP8
(fp32 and power-of-two block scales), MXFP4 and NVFP4 weights) against the oracle's
fp64 backward, through the C ABI.

Transposed weight copy: bit-exact against numpy.  Gradients: d_x per token
row within the forward's relative L2 bound (ROW_TOL); d_adapter per expert
within ROW_TOL (Frobenius); d_logits per token within ROW_TOL of
sum_j w_j |g_j| (g_j = <d_out, y_j>, from the oracle): d_logits_j =
w_j (g_j - sum_i w_i g_i) subtracts nearly equal terms, so its error is
bounded relative to the terms, not to the difference.  The GPU rounds d_out
and the SwiGLU gradients to fp16 (2^-11 relative), recomputes the
pre-activations from fp16 x R_e (INT4), and its FP8 / MXFP8 h codes may
differ from the oracle's by one step where h sits on a rounding boundary, so
its errors are ~1e-3 of these scales."""
import numpy as np
import pytest
import torch

import oracle
from precision_moe_expert_amd import binding, synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def small(T=77, H=256, I=256, E=12, k=3, oft=False, zipf=0.0, chunk=4, cfg_id=None, fmt=1):
    return synth.LayerConfig("bwd_small", cfg_id or (240 + (5 if oft else 0) + 10 * fmt), T=T, H=H, E=E, k=k, I=I,
                             fmt=fmt, chunk=chunk, oft=oft, zipf_alpha=zipf)


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
                                       chunk_experts=c.chunk if chunk is None else chunk, g13=d.g13, g2=d.g2)


def tiles(a, tb):
    """Row-major transposed copy [R][C] bytes -> the library's 16-row tiles
    [R/16][C/tb][16][tb] (tb = 64 bytes of nibbles or 128 of E4M3)."""
    R, C = a.shape
    return np.ascontiguousarray(a.reshape(R // 16, 16, C // tb, tb).transpose(0, 2, 1, 3)).reshape(-1)


def check(li, dout_bits, got, tokens=None, check_adapter=True):
    from tests import refimpl
    dout = refimpl.bf16_to_f32(dout_bits).reshape(li.cfg.T, li.cfg.H)
    toks = np.arange(li.cfg.T) if tokens is None else tokens
    rdx, rdl, rdR, rg = oracle.backward_inputs(li, dout[toks], tokens=None if tokens is None else toks,
                                               return_g=True)
    dx = gu.bf16_to_np(got[0])[toks]
    dl = got[1].cpu().numpy()[toks].astype(np.float64)
    ex = gu.row_rel_err(dx, rdx)
    _, w = oracle.route(li.logits, li.cfg.k)
    scale = np.sum(w[toks].astype(np.float64) * np.abs(rg), axis=1)
    el = np.linalg.norm(dl - rdl, axis=1) / np.maximum(scale, 1e-30)
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
        for w, (a, b_) in enumerate(((0, 4), (1, 5), (2, 6), (3, 7))):
            out[:, :, 2 * w] = f[:, :, a].astype(np.float16)
            out[:, :, 2 * w + 1] = f[:, :, b_].astype(np.float16)
        return out.view(np.uint8).reshape(-1)

    for e in range(E):
        w13t = raw[o13 + e * H * I: o13 + (e + 1) * H * I]
        assert np.array_equal(w13t, tiles(nib_t(li.w13[e], 2 * I, H), 64))
        w2t = raw[o2 + e * H * I // 2: o2 + (e + 1) * H * I // 2]
        assert np.array_equal(w2t, tiles(nib_t(li.w2[e], H, I), 64))
        n13 = (H // 32) * 2 * I * 2
        assert np.array_equal(raw[os13 + e * n13: os13 + (e + 1) * n13], f16_pairs(li.s13[e], H // 32, 2 * I))
        n2 = (I // 32) * H * 2
        assert np.array_equal(raw[os2 + e * n2: os2 + (e + 1) * n2], f16_pairs(li.s2[e], I // 32, H))


@pytest.mark.parametrize("fmt,oft", [(1, False), (1, True), (2, False), (2, True), (3, False), (3, True),
                                     (4, False), (4, True), (5, False), (5, True)])
def test_backward_small_vs_oracle(fmt, oft):
    li = synth.make_inputs(small(oft=oft, fmt=fmt))
    dout = d_out_of(li.cfg)
    check(li, dout, Bwd(li).run(dout))


@pytest.mark.parametrize("fmt,oft", [(1, True), (2, False), (3, False), (5, False)])
def test_backward_max_experts_and_top_k(fmt, oft):
    """E = 1024 with top-16 routing (most experts one or two rows, a few hot)."""
    li = synth.make_inputs(small(T=64, H=256, I=256, E=1024, k=16, zipf=0.4, chunk=64, oft=oft,
                                 cfg_id=280 + fmt, fmt=fmt))
    dout = d_out_of(li.cfg, 12)
    check(li, dout, Bwd(li).run(dout))


@pytest.mark.parametrize("fmt", [1, 2, 3, 5])
@pytest.mark.parametrize("tile_rows", [16, 32, 48, 64, 96, 128, 160, 192])
def test_backward_every_tile_height(fmt, tile_rows):
    li = synth.make_inputs(small(T=300, H=512, I=512, E=5, k=4, chunk=2, oft=fmt == 1, cfg_id=250 + fmt, fmt=fmt))
    dout = d_out_of(li.cfg, 6)
    check(li, dout, Bwd(li, tile_rows).run(dout))


@pytest.mark.parametrize("fmt", [1, 2, 3, 5])
def test_backward_chunk_size_bitwise_invariance(fmt):
    li = synth.make_inputs(small(E=9, k=3, zipf=1.2, oft=fmt == 1, fmt=fmt))
    dout = d_out_of(li.cfg, 7)
    b = Bwd(li)
    ref = [None if t is None else t.clone() for t in b.run(dout, chunk=1)]
    torch.cuda.synchronize()
    for c in (2, 4, 9, 64):
        got = b.run(dout, chunk=c)
        torch.cuda.synchronize()
        assert torch.equal(got[0].view(torch.int16), ref[0].view(torch.int16))
        assert torch.equal(got[1], ref[1])
        if ref[2] is not None:
            assert torch.equal(got[2], ref[2])


def test_backward_weight_copy_bitexact_fp8_mxfp4():
    """FP8: bytes transposed, block scales [N/128][K/128] -> [K/128][N/128];
    MXFP4: nibbles transposed, E8M0 scales as fp16 2^(e-127) pairs."""
    from tests import refimpl
    H, I, E = 256, 512, 3

    def al(v):
        return (v + 255) // 256 * 256

    for fmt in (2, 3):
        cfg = small(T=8, H=H, I=I, E=E, k=1, fmt=fmt, cfg_id=270 + fmt)
        li = synth.make_inputs(cfg)
        raw = Bwd(li).bw.cpu().numpy()
        per = 1 if fmt == 2 else 2
        o2 = al(E * H * 2 * I // per)
        os13 = o2 + al(E * I * H // per)
        for e in range(E):
            if fmt == 2:
                w13t = raw[e * H * 2 * I:(e + 1) * H * 2 * I]
                assert np.array_equal(w13t, tiles(li.w13[e].reshape(2 * I, H).T, 128))
                w2t = raw[o2 + e * H * I:o2 + (e + 1) * H * I]
                assert np.array_equal(w2t, tiles(li.w2[e].reshape(H, I).T, 128))
                n13 = (2 * I // 128) * (H // 128)
                s13t = raw[os13:].view(np.float32)[e * n13:(e + 1) * n13].reshape(H // 128, 2 * I // 128)
                assert np.array_equal(s13t, li.s13[e].reshape(2 * I // 128, H // 128).T)
            else:
                w2t = raw[o2 + e * H * I // 2:o2 + (e + 1) * H * I // 2]
                v = refimpl.unpack_nibbles(li.w2[e]).reshape(H, I).T.copy()
                assert np.array_equal(w2t, tiles((v[:, 0::2] | (v[:, 1::2] << 4)).astype(np.uint8), 64))
                n13 = (H // 32) * 2 * I
                got = raw[os13 + e * n13 * 2:os13 + (e + 1) * n13 * 2].view(np.float16).reshape(H // 32, 2 * I // 8, 8)
                ref = np.ldexp(1.0, li.s13[e].reshape(H // 32, 2 * I // 8, 8).astype(np.int64) - 127)
                order = [0, 4, 1, 5, 2, 6, 3, 7]
                assert np.array_equal(got.astype(np.float64), ref[:, :, order])


def test_backward_weight_copy_bitexact_nvfp4():
    """NVFP4: nibbles transposed, E4M3 scales [K/16][N] as their fp16 values
    in pairs; the second-level scales are not part of the copy."""
    from tests import refimpl
    H, I, E = 256, 512, 3
    al = lambda v: (v + 255) // 256 * 256  # noqa: E731
    cfg = small(T=8, H=H, I=I, E=E, k=1, fmt=5, cfg_id=275)
    li = synth.make_inputs(cfg)
    raw = Bwd(li).bw.cpu().numpy()
    o2 = al(E * H * 2 * I // 2)
    os13 = o2 + al(E * I * H // 2)
    os2 = os13 + al(E * (H // 16) * 2 * I * 2)
    order = [0, 4, 1, 5, 2, 6, 3, 7]
    for e in range(E):
        w13t = raw[e * H * I:(e + 1) * H * I]
        v = refimpl.unpack_nibbles(li.w13[e]).reshape(2 * I, H).T.copy()
        assert np.array_equal(w13t, tiles((v[:, 0::2] | (v[:, 1::2] << 4)).astype(np.uint8), 64))
        for off, s, G, L in ((os13, li.s13[e], H // 16, 2 * I), (os2, li.s2[e], I // 16, H)):
            n = G * L
            got = raw[off + e * n * 2:off + (e + 1) * n * 2].view(np.float16).reshape(G, L // 8, 8)
            val = torch.from_numpy(np.ascontiguousarray(s).reshape(-1)).view(torch.float8_e4m3fn).double().numpy()
            assert np.array_equal(got.astype(np.float64), val.reshape(G, L // 8, 8)[:, :, order])


@pytest.mark.slow
def test_backward_qwen3_fp8_fullsize_sampled():
    li = synth.make_inputs(synth.CONFIGS["c2"], with_lm=False)
    dout = d_out_of(li.cfg, 10)
    got = Bwd(li).run(dout)
    torch.cuda.synchronize()
    toks = np.sort(np.random.default_rng(4).choice(li.cfg.T, size=32, replace=False)).astype(np.int32)
    check(li, dout, got, tokens=toks)


@pytest.mark.slow
def test_backward_deepseek_mxfp4_fullsize_sampled():
    li = synth.make_inputs(synth.CONFIGS["c4"], with_lm=False)
    dout = d_out_of(li.cfg, 11)
    got = Bwd(li).run(dout)
    torch.cuda.synchronize()
    toks = np.sort(np.random.default_rng(5).choice(li.cfg.T, size=8, replace=False)).astype(np.int32)
    check(li, dout, got, tokens=toks)


@pytest.mark.slow
def test_backward_deepseek_nvfp4_fullsize_sampled():
    li = synth.make_inputs(synth.CONFIGS["c4n"], with_lm=False)
    dout = d_out_of(li.cfg, 13)
    got = Bwd(li).run(dout)
    torch.cuda.synchronize()
    toks = np.sort(np.random.default_rng(6).choice(li.cfg.T, size=8, replace=False)).astype(np.int32)
    check(li, dout, got, tokens=toks)


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


@pytest.mark.parametrize("fmt", [1, 3, 5])
def test_backward_shared_adapter(fmt):
    """One R shared by all experts: dL/dR sums every expert's x^T dx' blocks
    (per-expert partials added in ascending active order on the GPU)."""
    from tests import refimpl
    cfg = small(T=53, H=256, I=256, E=7, k=3, oft=True, fmt=fmt, cfg_id=300 + fmt)
    li = synth.make_inputs(cfg)
    shared = np.ascontiguousarray(li.oft[1])
    d = gu.DevInputs(li)
    d.layer = binding.make_layer(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, fmt, oft=True, adapter_expert_stride=0)
    d.oft = gu.dev(shared, "bf16")
    bw = binding.prepare_backward_weights(d.layer, d.w13, d.w2, d.s13, d.s2)
    dout_bits = d_out_of(cfg, 9)
    got = binding.expert_backward(d.layer, d.x, d.logits, d.w13, d.w2, d.s13, d.s2, bw, gu.dev(dout_bits, "bf16"),
                                  adapter=d.oft, chunk_experts=cfg.chunk, g13=d.g13, g2=d.g2)
    dout = refimpl.bf16_to_f32(dout_bits).reshape(cfg.T, cfg.H)
    rdx, rdl, rdR = oracle.backward(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, fmt, li.x, li.logits, li.w13, li.w2, li.s13,
                                    li.s2, dout, oft=shared, chunk_experts=cfg.chunk, adapter_expert_stride=0,
                                    g13=li.g13, g2=li.g2)
    ex = gu.row_rel_err(gu.bf16_to_np(got[0]), rdx)
    dR = got[2].cpu().numpy().astype(np.float64).reshape(rdR.shape)
    eR = np.linalg.norm(dR - rdR) / np.linalg.norm(rdR)
    print(f"shared adapter fmt {fmt}: d_x max row rel err {ex.max():.3e}; d_adapter rel err {eR:.3e}")
    assert ex.max() <= gu.ROW_TOL
    assert eR <= gu.ROW_TOL
