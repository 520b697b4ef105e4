"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Routing, permutation and index outputs are compared bit for bit; expert
outputs per row against the per-format relative L2 bound and the element
bound of tests/gpu_util.check_rows (bf16 output).  Shapes
span several tiles with ragged tails; the method's degenerate cases (ties,
k = E, one hot expert, chunk sizes 1..E) are included."""
import numpy as np
import pytest
import torch

import oracle
from precision_moe_expert_amd import binding, synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def small(fmt, T=77, H=256, I=384, E=12, k=3, oft=False, zipf=0.0, chunk=4, cfg_id=None):
    return synth.LayerConfig(f"small_f{fmt}", cfg_id or (40 + fmt + (5 if oft else 0)), T=T, H=H, E=E, k=k, I=I,
                             fmt=fmt, chunk=chunk, oft=oft, zipf_alpha=zipf)


def check_route(logits: np.ndarray, k: int, E: int):
    T = logits.shape[0]
    layer = binding.make_layer(T, 256, 256, E, k, 1)
    got = binding.route_permute(gu.dev(np.ascontiguousarray(logits, np.float32)), layer)
    torch.cuda.synchronize()
    ids, w = oracle.route(logits, k)
    P = oracle.permute(ids, E)
    assert np.array_equal(got["topk_ids"].cpu().numpy(), ids)
    assert np.max(np.abs(got["topk_w"].cpu().numpy() - w)) <= 1e-5
    assert np.array_equal(got["expert_offsets"].cpu().numpy(), P["offsets"])
    assert np.array_equal(got["sorted_rows"].cpu().numpy(), P["sorted_rows"])
    assert np.array_equal(got["row_of"].cpu().numpy(), P["row_of"])
    na = int(got["num_active"][0].item())
    assert na == len(P["active"])
    assert np.array_equal(got["active_experts"].cpu().numpy()[:na], P["active"])


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_route_bitexact_configs(name):
    cfg = synth.CONFIGS[name]
    check_route(synth.gen_logits(cfg), cfg.k, cfg.E)


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (5, 4, 4), (300, 130, 16), (2049, 1024, 8), (4099, 64, 1),
                                   (20000, 8, 2), (9000, 384, 8),
                                   # up to 1024 tokens and more than 64 experts take one token per wave
                                   (700, 1024, 16), (64, 512, 8), (1024, 257, 8), (1025, 257, 8), (3, 65, 16),
                                   # up to 512 pairs the permutation runs in one workgroup (one launch)
                                   (64, 384, 8), (65, 384, 8), (32, 384, 16), (1, 1024, 16)])
def test_route_bitexact_edge(T, E, k):
    r = np.random.default_rng(T * 7 + E)
    lg = r.standard_normal((T, E)).astype(np.float32)
    lg[0, :] = 0.25                          # all tied -> ids 0..k-1
    if T > 2:
        lg[1, ::2] = 1.0                     # many ties
        lg[2, :] = -0.0
        lg[2, 1::3] = 0.0                    # -0 == +0
    if T > 10:
        lg[3:10, 0] += 50.0                  # a hot expert
    check_route(lg, k, E)


@pytest.mark.parametrize("fmt", [1, 2, 3, 4, 5])
def test_forward_small_vs_oracle(fmt):
    cfg = small(fmt)
    li = synth.make_inputs(cfg)
    d = gu.DevInputs(li)
    out = gu.bf16_to_np(d.forward())
    ref = oracle.forward_inputs(li)
    gu.check_rows(out, ref, li.cfg.fmt, f"fmt {fmt}")


@pytest.mark.parametrize("oft", [False, True])
def test_forward_int4_oft_small(oft):
    cfg = small(1, T=53, H=512, I=256, E=9, k=4, oft=oft, chunk=2)
    li = synth.make_inputs(cfg)
    d = gu.DevInputs(li)
    out = gu.bf16_to_np(d.forward())
    ref = oracle.forward_inputs(li)
    gu.check_rows(out, ref, li.cfg.fmt, f"oft {oft}")


@pytest.mark.parametrize("T,fmt", [(64, 1), (65, 1), (64, 4), (65, 4)])
def test_forward_across_one_block_permutation(T, fmt):
    """64 tokens x top-8 = 512 pairs take the one-workgroup permutation, 65
    tokens (520 pairs) the histogram / scan / scatter launches; the whole
    layer (OFT on the INT4 base) must match the oracle on both sides."""
    cfg = small(fmt, T=T, H=256, I=256, E=40, k=8, oft=fmt == 1, chunk=8, cfg_id=90 + T + fmt)
    li = synth.make_inputs(cfg)
    d = gu.DevInputs(li)
    out = gu.bf16_to_np(d.forward())
    gu.check_rows(out, oracle.forward_inputs(li), li.cfg.fmt, f"T {T} fmt {fmt}")


def test_forward_int4_oft_partial_block_chunk():
    """H = 1280: 40 diagonal blocks, so the rotation's second 32-block item
    has blocks for one wave only (8), and 16-row groups are ragged."""
    cfg = small(1, T=45, H=1280, I=256, E=6, k=2, oft=True, chunk=3, cfg_id=68)
    li = synth.make_inputs(cfg)
    d = gu.DevInputs(li)
    out = gu.bf16_to_np(d.forward())
    gu.check_rows(out, oracle.forward_inputs(li), li.cfg.fmt, f"oft H=1280")


def test_forward_c1_vs_oracle():
    li = synth.make_inputs(synth.CONFIGS["c1"])
    d = gu.DevInputs(li)
    out = gu.bf16_to_np(d.forward())
    gu.check_rows(out, oracle.forward_inputs(li), li.cfg.fmt, f"c1")


@pytest.mark.parametrize("fmt", [1, 2, 3, 4, 5])
def test_forward_max_experts_and_top_k(fmt):
    """E = 1024 (the library's maximum) with top-16 routing: about 500 active
    experts, most with one or two rows, a few (Zipf bias) with up to ~50;
    16 chunks of 64."""
    cfg = small(fmt, T=96, H=256, I=128, E=1024, k=16, zipf=0.4, chunk=64, cfg_id=90 + fmt)
    li = synth.make_inputs(cfg)
    d = gu.DevInputs(li)
    out = gu.bf16_to_np(d.forward())
    gu.check_rows(out, oracle.forward_inputs(li), li.cfg.fmt, f"fmt {fmt} E=1024 k=16")


@pytest.mark.parametrize("fmt", [1, 2, 3, 4, 5])
def test_chunk_size_bitwise_invariance(fmt):
    cfg = small(fmt, E=9, k=3, zipf=1.2)
    d = gu.DevInputs(synth.make_inputs(cfg))
    outs = [d.forward(chunk=c).clone() for c in (1, 2, 4, 9, 64)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


@pytest.mark.parametrize("fmt", [1, 2, 3, 4, 5])
def test_run_twice_bitwise(fmt):
    d = gu.DevInputs(synth.make_inputs(small(fmt)))
    a = d.forward().clone()
    b = d.forward().clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_oft_identity_equals_no_adapter():
    cfg = small(1, oft=True)
    li = synth.make_inputs(cfg)
    li.oft[:] = 0
    li.oft[:, :, np.arange(32), np.arange(32)] = 0x3F80
    d = gu.DevInputs(li)
    a = d.forward().clone()
    li.oft = None
    d2 = gu.DevInputs(li)
    b = d2.forward().clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_combine_vs_oracle():
    r = np.random.default_rng(5)
    T, k, H, E = 97, 4, 512, 16
    lg = r.standard_normal((T, E)).astype(np.float32)
    ids, w = oracle.route(lg, k)
    P = oracle.permute(ids, E)
    y = synth._to_bf16_bits((r.standard_normal((T * k, H)) * 3).astype(np.float32))
    layer = binding.make_layer(T, H, 256, E, k, 1)
    out = binding.combine(layer, gu.dev(y, "bf16"), gu.dev(w), gu.dev(P["row_of"]))
    got = gu.bf16_to_np(out)
    ref = oracle.combine(y, w, P["row_of"])
    # fp32 fused sum in ascending j vs fp64: at most one bf16 rounding step apart
    ulp = np.abs(ref) * 2.0 ** -8 + 1e-30
    assert np.all(np.abs(got - ref) <= ulp)


def test_lm_head_logprob_vs_oracle():
    r = np.random.default_rng(6)
    T, H, V = 37, 512, 5000
    h = synth._to_bf16_bits((r.standard_normal((T, H)) * 20).astype(np.float32))
    w = synth._to_bf16_bits((r.standard_normal((V, H)) / np.sqrt(H)).astype(np.float32))
    tg = r.integers(0, V, T).astype(np.int32)
    lp = binding.lm_head_logprob(gu.dev(h, "bf16"), gu.dev(w, "bf16"), gu.dev(tg)).cpu().numpy()
    from tests import refimpl
    ref = oracle.lm_head_logprob(refimpl.bf16_to_f32(h), w, tg)
    assert np.max(np.abs(lp - ref)) <= 1e-3


@pytest.mark.parametrize("T,H,V", [(130, 256, 700), (1, 128, 100), (64, 384, 256), (65, 256, 513), (3, 128, 40000),
                                   (2, 256, 70001)])
def test_lm_head_blocks_and_edges(T, H, V):
    # several 64-token blocks, a last vocabulary block of 1..255 rows, targets on
    # block edges, vocabularies whose log-softmax parts take more than one pass
    # of 8192 entries; a second call on the same workspace gives the same bits
    r = np.random.default_rng(T * 1000 + V)
    h = synth._to_bf16_bits((r.standard_normal((T, H)) * 3).astype(np.float32))
    w = synth._to_bf16_bits((r.standard_normal((V, H)) * (4 / np.sqrt(H))).astype(np.float32))
    edges = [v for v in (0, V - 1, 255, 256, 511, 512) if v < V]
    tg = r.integers(0, V, T).astype(np.int32)
    tg[:len(edges)] = edges[:T]
    ws = binding.alloc_workspace(binding.lib().moe_lm_head_workspace_bytes(T, V))
    ws.fill_(0x7F)  # the call must not rely on a cleared workspace
    hd, wd, td = gu.dev(h, "bf16"), gu.dev(w, "bf16"), gu.dev(tg)
    lp = binding.lm_head_logprob(hd, wd, td, ws=ws)
    lp2 = binding.lm_head_logprob(hd, wd, td, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(lp, lp2)
    from tests import refimpl
    ref = oracle.lm_head_logprob(refimpl.bf16_to_f32(h), w, tg)
    assert np.max(np.abs(lp.cpu().numpy() - ref)) <= 1e-3


def test_t0_is_noop():
    layer = binding.make_layer(0, 256, 256, 8, 2, 1)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    lg = torch.empty((0, 8), dtype=torch.float32, device="cuda")
    z = torch.zeros(16, dtype=torch.uint8, device="cuda")
    out = binding.expert_forward(layer, x, lg, z, z, z, z, chunk_experts=1,
                                 out=torch.empty((0, 256), dtype=torch.bfloat16, device="cuda"))
    assert out.shape == (0, 256)


@pytest.mark.parametrize("fmt", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("tile_rows", [16, 32, 48, 64, 96, 128, 160, 192])
def test_forward_every_tile_height(fmt, tile_rows):
    """Each grouped-GEMM tile height against the oracle: ~250 rows per expert,
    so tall tiles run full and ragged; I = 768 gives three 256-wide N blocks."""
    cfg = small(fmt, T=300, H=512, I=768, E=5, k=4, chunk=2, cfg_id=60 + fmt)
    li = synth.make_inputs(cfg)
    d = gu.DevInputs(li)
    d.layer.tile_rows = tile_rows
    out = gu.bf16_to_np(d.forward())
    gu.check_rows(out, oracle.forward_inputs(li), li.cfg.fmt, f"fmt {fmt} tile {tile_rows}")


@pytest.mark.parametrize("oft,zipf,chunk", [(False, 0.0, 2), (True, 0.0, 3), (False, 1.2, 1)])
def test_mxfp4_128_row_tiles(oft, zipf, chunk):
    """MXFP4 at 128-row tiles, the headline tile height, on a shape whose H
    and I are multiples of 512 like the DeepSeek-V3 one: ~240 rows per
    expert, so the tiles run full and ragged; GEMM1 has four 128-wide h
    blocks and 8 K steps, GEMM2 four 256-wide output blocks and 4 K steps.
    Also bitwise independent of the chunk size."""
    cfg = small(3, T=300, H=1024, I=512, E=5, k=4, oft=oft, zipf=zipf, chunk=chunk,
                cfg_id=200 + 2 * int(oft) + int(zipf > 0))
    li = synth.make_inputs(cfg)
    d = gu.DevInputs(li)
    d.layer.tile_rows = 128
    out = d.forward()
    torch.cuda.synchronize()
    gu.check_rows(gu.bf16_to_np(out), oracle.forward_inputs(li), 3, f"mxfp4 128-row tiles oft={oft} zipf={zipf}")
    for c in (1, 5):
        o = d.forward(chunk=c)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), out.view(torch.int16)), f"chunk {c} differs"


def _scaled_int4_case(cfg_id, s_lo, s_hi, x_scale, x_max=None):
    cfg = small(1, T=64, H=512, I=256, E=6, k=2, chunk=3, cfg_id=cfg_id)
    li = synth.make_inputs(cfg)
    r = np.random.default_rng(cfg_id)
    for name in ("s13", "s2"):
        s = getattr(li, name)
        v = np.exp2(r.uniform(np.log2(s_lo), np.log2(s_hi), s.shape)).astype(np.float32)
        setattr(li, name, synth._to_bf16_bits(v))
    xf = (li.x.astype(np.uint32) << 16).view(np.float32) * np.float32(x_scale)
    if x_max is not None:
        xf = xf / np.abs(xf).max(axis=1, keepdims=True) * np.float32(x_max)
    li.x = synth._to_bf16_bits(xf)
    return li


@pytest.mark.parametrize("s_lo,s_hi,x_scale,x_max", [
    (2.0 ** -17, 2.0 ** -12, 64.0, None),   # tiny scales (an fp16 s/16 would lose bits below ~1.2e-4)
    (2.0 ** 8, 2.0 ** 12, 2.0 ** -12, None),  # large scales, small activations
    (2.0 ** -16, 2.0 ** -15, 1.0, 3.0e4),   # activations up to 3e4 (below fp16's 65504)
])
def test_int4_fp16_range_edges(s_lo, s_hi, x_scale, x_max):
    """INT4 group scales and activations at the ends of the fp16 range the
    header documents (bf16 scales in [2^-17, 8188], |x|, |h| < 65504): every
    q s is exact in fp16 and x converts exactly, so the error stays at the
    16-bit formats' usual level.  Inputs are scaled so that h stays in range."""
    li = _scaled_int4_case(84, s_lo, s_hi, x_scale, x_max)
    d = gu.DevInputs(li)
    out = gu.bf16_to_np(d.forward())
    ref = oracle.forward_inputs(li)
    assert np.isfinite(ref).all()
    gu.check_rows(out, ref, 1, f"int4 scales [{s_lo:.1e}, {s_hi:.1e}], x scale {x_scale}, x max {x_max}")


def test_nvfp4_full_e4m3_scale_range():
    """NVFP4 block scales drawn from every positive finite E4M3 code
    (subnormal 2^-9 up to 448), not only the [16, 448] band of the synthetic
    recipe; e2m1 x e4m3 stays exact in fp16 over that whole range."""
    cfg = small(5, T=64, H=512, I=256, E=6, k=2, chunk=3, cfg_id=83)
    li = synth.make_inputs(cfg)
    r = np.random.default_rng(83)
    for name in ("s13", "s2"):
        s = getattr(li, name)
        setattr(li, name, r.integers(1, 0x7F, s.shape, dtype=np.uint8))
    d = gu.DevInputs(li)
    out = gu.bf16_to_np(d.forward())
    ref = oracle.forward_inputs(li)
    gu.check_rows(out, ref, 5, "nvfp4 all E4M3 scale codes")


@pytest.mark.parametrize("fmt", [1, 2, 3, 4, 5])
def test_forward_oft_every_format(fmt):
    """The BF16 OFT adapter (per-expert R) on every frozen base: the rotated
    rows x R_e go through each format's GEMM1 input quantizer (Orbit analysis
    page, 核心判断: the base frozen at INT4, FP4 or FP8, the trainable
    freedom in a BF16 adapter)."""
    cfg = small(fmt, T=61, H=512, I=256, E=9, k=3, oft=True, chunk=2, cfg_id=150 + fmt)
    li = synth.make_inputs(cfg)
    d = gu.DevInputs(li)
    out = gu.bf16_to_np(d.forward())
    gu.check_rows(out, oracle.forward_inputs(li), fmt, f"fmt {fmt} oft")


@pytest.mark.parametrize("fmt", [1, 2, 3, 4, 5])
def test_forward_oft_shared_every_format(fmt):
    """One R shared by all experts (adapter_expert_stride = 0)."""
    cfg = small(fmt, T=61, H=512, I=256, E=9, k=3, oft=True, chunk=4, cfg_id=160 + fmt)
    li = synth.make_inputs(cfg)
    shared = np.ascontiguousarray(li.oft[3])
    d = gu.DevInputs(li)
    d.layer = binding.make_layer(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, fmt, oft=True, adapter_expert_stride=0)
    d.oft = gu.dev(shared, "bf16")
    out = gu.bf16_to_np(d.forward())
    ref = oracle.forward(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, fmt, li.x, li.logits, li.w13, li.w2, li.s13, li.s2,
                         oft=shared, chunk_experts=cfg.chunk, adapter_expert_stride=0, g13=li.g13, g2=li.g2)
    gu.check_rows(out, ref, fmt, f"fmt {fmt} shared oft")


def test_binding_rejects_mis_sized_tensors():
    """The binding checks every tensor against the sizes the layer implies
    before the library is called (a short or strided tensor would be read or
    written out of bounds on the GPU)."""
    cfg = small(3, T=40, H=256, I=256, E=6, k=2, cfg_id=190)
    d = gu.DevInputs(synth.make_inputs(cfg))
    c = d.li.cfg
    args = dict(adapter=None, chunk_experts=2, g13=None, g2=None)
    with pytest.raises(ValueError):
        binding.expert_forward(d.layer, d.x[:-1], d.logits, d.w13, d.w2, d.s13, d.s2, **args)   # short x
    with pytest.raises(ValueError):
        binding.expert_forward(d.layer, d.x, d.logits, d.w13.reshape(-1)[: d.w13.numel() // 2], d.w2, d.s13, d.s2, **args)
    with pytest.raises(ValueError):
        binding.expert_forward(d.layer, d.x, d.logits.t(), d.w13, d.w2, d.s13, d.s2, **args)  # strided
    with pytest.raises(ValueError):
        binding.expert_forward(d.layer, d.x.view(torch.int16).to(torch.int32), d.logits, d.w13, d.w2, d.s13, d.s2,
                               **args)                                                        # 4-byte elements
    out = binding.expert_forward(d.layer, d.x, d.logits, d.w13, d.w2, d.s13, d.s2, **args)
    assert out.shape == (c.T, c.H)
