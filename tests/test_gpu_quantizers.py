"""GPU activation quantizers (the GEMM1 input formats) against the oracle's,
code for code and scale for scale, through moe_quantize_activations.

Rows are built to sit on the quantizers' edges: all-zero blocks (with -0),
block maxima at exact powers of two and just below them, values that land
exactly on E4M3 rounding midpoints after scaling (ties to the even code),
also under scales whose reciprocal is inexact, and one bf16 step off them,
blocks whose scaled maximum reaches the saturation range [448, 512) of the
MX shared exponent, tiny values next to large ones (E4M3 subnormals and
underflow to zero), bf16 subnormals and very large magnitudes.  Both sides
take every rounding decision in fp32 on the same bf16 inputs, so the codes
and scales must agree bit for bit (NeMo RL FP8 post, Table 1: E4M3 input
activations with an fp32 scale per [1,128] block; the MXFP8 reading for the
MXFP4 weights: E4M3 elements with an E8M0 scale per 32)."""
import numpy as np
import pytest
import torch

import oracle
from precision_moe_expert_amd import binding, synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def bf16_bits(v: np.ndarray) -> np.ndarray:
    return synth._to_bf16_bits(np.asarray(v, np.float32))


def bf16_neighbour(v: np.ndarray, step: int) -> np.ndarray:
    """The bf16 value `step` codes from each (bf16-exact, nonzero) value."""
    b = bf16_bits(v).astype(np.int32) + step
    return (b.astype(np.uint32) << 16).view(np.float32)


def adversarial_rows(H: int, seed: int) -> np.ndarray:
    """[T][H] float32 values, every one exactly representable in bf16."""
    r = np.random.default_rng(seed)
    rows = []
    base = r.standard_normal((24, H)).astype(np.float32)
    rows.extend(base)
    z = np.zeros(H, np.float32)
    z[1::2] = -0.0
    rows.append(z)                                        # all-zero blocks, signed zeros
    for p in (-20, -3, 0, 1, 7, 40):                      # block maxima exactly 2^p
        v = r.standard_normal(H).astype(np.float32) * np.float32(2.0 ** (p - 3))
        v[::32] = np.float32(2.0 ** p) * np.where(r.random(H // 32) < 0.5, -1, 1)
        rows.append(v)
    for p in (0, 5):                                      # maxima just below a power of two
        v = r.standard_normal(H).astype(np.float32) * np.float32(2.0 ** (p - 4))
        v[5::32] = np.float32(2.0 ** p * (1 - 2.0 ** -8))
        rows.append(v)
    # E4M3 midpoints: with amax = 448 the FP8 scale is 1; the MX exponent of
    # 448 (2^8 * 1.75) is 0 as well, so values map to themselves
    mids = np.array([1.0625, 1.1875, 2.125, 3.375, 0.0107421875, 13.5, 208.0, 240.0, 2.0 ** -10, 3 * 2.0 ** -11],
                    np.float32)
    v = np.resize(np.concatenate([mids, -mids]), H).astype(np.float32)
    v[::32] = 448.0
    rows.append(v)
    v = v.copy()
    v[::32] = -448.0
    rows.append(v)
    # the same midpoints under FP8 scales 1.5 and 1.25 (block maxima 672 and
    # 560), whose reciprocals are inexact, and one bf16 step to either side
    for sc in (1.5, 1.25):
        m = (np.concatenate([mids, -mids]) * np.float32(sc)).astype(np.float32)
        near = np.concatenate([m, bf16_neighbour(m, +1), bf16_neighbour(m, -1)]).astype(np.float32)
        v = np.resize(near, H).astype(np.float32)
        v[::32] = np.float32(448.0 * sc)
        assert np.array_equal(bf16_bits(v).astype(np.uint32) << 16, v.view(np.uint32)), "rows must be bf16 values"
        rows.append(v)
    # saturation range of the MX exponent: amax mantissa >= 1.75 scales to [448, 512)
    v = r.uniform(-1, 1, H).astype(np.float32)
    v[::32] = 1.9375 * 4
    v[1::32] = -1.875 * 4
    v[2::32] = 1.75 * 4
    rows.append(v)
    # tiny next to large: E4M3 subnormals and underflow after scaling
    v = (r.standard_normal(H) * 1e-3).astype(np.float32)
    v[::32] = 300.0
    v[7::32] = 2.0 ** -20
    rows.append(v)
    # bf16 subnormals and huge magnitudes
    v = np.full(H, np.float32(2.0 ** -130))
    v[1::3] = -np.float32(2.0 ** -133)
    rows.append(v)
    v = (r.standard_normal(H) * 1e30).astype(np.float32)
    rows.append(v)
    a = np.stack(rows).astype(np.float32)
    bits = bf16_bits(a)
    return bits


@pytest.mark.parametrize("fmt", [binding.FMT_FP8, binding.FMT_FP8_POW2, binding.FMT_MXFP4])
@pytest.mark.parametrize("H", [256, 2304])
def test_activation_quantizer_bitexact(fmt, H):
    bits = adversarial_rows(H, seed=H + fmt)
    T = bits.shape[0]
    xf = (bits.astype(np.uint32) << 16).view(np.float32)
    layer = binding.make_layer(T, H, 256, 8, 2, fmt)
    codes, scales = binding.quantize_activations(layer, gu.dev(bits, "bf16"))
    torch.cuda.synchronize()
    got_q, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    if fmt == binding.FMT_FP8:
        ref_q, ref_s = oracle.quant_fp8(xf)
    elif fmt == binding.FMT_FP8_POW2:
        ref_q, ref_s = oracle.quant_fp8_pow2(xf)
    else:
        ref_q, ref_s = oracle.quant_mxfp8(xf)
    bad = np.argwhere(got_q != ref_q)
    assert bad.size == 0, (f"{len(bad)} code mismatches, first at {bad[:4].tolist()}: gpu "
                           f"{got_q[tuple(bad[0])]:#04x} oracle {ref_q[tuple(bad[0])]:#04x} "
                           f"(x = {xf[tuple(bad[0])]!r})")
    assert np.array_equal(got_s.view(np.uint8), np.ascontiguousarray(ref_s).view(np.uint8))


def test_quantizer_refuses_16bit_formats():
    layer = binding.make_layer(4, 256, 256, 8, 2, binding.FMT_INT4)
    x = torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(binding.MoeError) as e:
        binding.quantize_activations(layer, x)
    assert e.value.status == binding.MOE_ERR_UNSUPPORTED
