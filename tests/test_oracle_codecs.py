"""Pins of the oracle's codecs and activation quantizers (CPU only).

Each check compares the oracle's C code against something it does not share:
torch's float8/bfloat16 casts, numpy integer shifts, frexp/ldexp, or the OCP
value tables.  Formats: INT4 (Orbit announcement, 技术细节 / Kimi INT4 base),
FP8 E4M3 with [128,128] / [1,128] fp32 scales (NeMo RL FP8 post, Table 1),
MXFP4 / MXFP8 (the mixed-precision sampler post names MXFP4 as a serving
format; element and scale codes follow OCP MX v1.0)."""
import numpy as np
import pytest

import oracle
from tests import refimpl


def test_bf16_decode_all_patterns():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode("bf16", codes)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns widen to quiet NaNs
        ref = refimpl.bf16_to_f32(codes).astype(np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_int4_decode_matches_int8_shift():
    nib = np.arange(16, dtype=np.uint8)
    got = oracle.decode("int4", nib)
    assert np.array_equal(got, refimpl.int4_values(nib))
    assert got.min() == -8 and got.max() == 7


def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode("e4m3", codes)
    ref = refimpl.e4m3_to_f64(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    # OCP E4M3FN: only S.1111.111 is NaN, largest finite is 448, smallest subnormal 2^-9
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and np.isnan(got).sum() == 2
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_e2m1_decode_matches_ocp_table():
    nib = np.arange(16, dtype=np.uint8)
    got = oracle.decode("e2m1", nib)
    assert np.array_equal(got, refimpl.E2M1_TABLE)
    assert np.array_equal(np.signbit(got), np.signbit(refimpl.E2M1_TABLE))


def test_e8m0_decode():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode("e8m0", codes)
    assert np.isnan(got[255])
    assert np.array_equal(got[:255], np.ldexp(1.0, np.arange(255) - 127))
    assert got[127] == 1.0


def test_e4m3_encode_round_trip_every_code():
    """Representable values round-trip exactly (every non-NaN code, incl. -0)."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = refimpl.e4m3_to_f64(codes).astype(np.float32)
    vals[codes == 0x80] = -0.0
    assert np.array_equal(oracle.encode_e4m3(vals), codes)


def test_e4m3_encode_rne_vs_torch_all_bf16_values():
    v = refimpl.bf16_to_f32(np.arange(65536, dtype=np.uint32).astype(np.uint16))
    fin = np.isfinite(v) & (np.abs(v) <= 464.0)
    got = oracle.encode_e4m3(v[fin])
    ref = refimpl.f32_to_e4m3_sat(v[fin])
    assert np.array_equal(got, ref)


def test_e4m3_encode_midpoints_and_saturation():
    # exact midpoints between neighbouring codes go to the even code
    codes = np.arange(0, 0x7E, dtype=np.uint8)
    lo = refimpl.e4m3_to_f64(codes)
    hi = refimpl.e4m3_to_f64(codes + 1)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)  # exact in fp32
    got = oracle.encode_e4m3(mid)
    expect = np.where(codes % 2 == 0, codes, codes + 1).astype(np.uint8)
    assert np.array_equal(got, expect)
    big = np.array([448.0, 449.0, 500.0, 1e30, np.inf, -1e30, -np.inf], np.float32)
    assert list(oracle.encode_e4m3(big)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert oracle.encode_e4m3(np.array([np.nan], np.float32))[0] == 0x7F


@pytest.mark.parametrize("seed", [0, 1])
def test_fp8_act_quant_bitexact_vs_numpy(seed):
    r = np.random.default_rng(seed)
    v = (r.standard_normal((37, 512)) * np.exp(r.uniform(-8, 8, (37, 1)))).astype(np.float32)
    v[3, 128:256] = 0.0  # an all-zero block -> scale 1, codes 0
    q, s = oracle.quant_fp8(v)
    q2, s2 = refimpl.quant_fp8_rows(v)
    assert np.array_equal(s, s2)
    assert np.array_equal(q, q2)
    assert s[3, 1] == 1.0 and not q[3, 128:256].any()
    # every non-zero block holds a +-448 code (s = amax/448)
    blk = q.reshape(37, 4, 128)
    nz = np.abs(v.reshape(37, 4, 128)).max(axis=2) > 0
    has448 = ((blk & 0x7F) == 0x7E).any(axis=2)
    assert np.array_equal(has448, nz)
    # dequantization error within half an E4M3 step of the block scale
    deq = refimpl.e4m3_to_f64(q) * np.repeat(s.astype(np.float64), 128, axis=1)
    sc = np.repeat(s.astype(np.float64), 128, axis=1)
    a = np.abs(v) / sc  # magnitude in code space
    step = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(a, 1e-300))) - 3), 2.0 ** -9) * sc
    ulp = step
    assert np.all(np.abs(deq - v) <= ulp * 0.5 * (1 + 1e-6))


@pytest.mark.parametrize("seed", [0, 1])
def test_fp8_pow2_act_quant_properties(seed):
    """Power-of-two [1,128] scales (NeMo RL FP8 post, pow2 scaling-factor switches):
    s is an exact power of two with s/2 < fl32(amax/448) <= s (the smallest
    power of two that keeps every |v|/s <= 448), codes are E4M3 of the exact
    quotient, an all-zero block has scale 1."""
    r = np.random.default_rng(seed + 10)
    v = (r.standard_normal((41, 512)) * np.exp(r.uniform(-12, 12, (41, 1)))).astype(np.float32)
    v[2, 256:384] = 0.0
    v[4, :128] = 0.0
    v[4, 7] = 448.0 * 2.0 ** -3   # amax/448 exactly a power of two: s = 2^-3
    q, s = oracle.quant_fp8_pow2(v)
    blk = np.abs(v.reshape(41, 4, 128)).max(axis=2)
    x = (blk / np.float32(448.0)).astype(np.float32)          # fl32(amax/448)
    nz = blk > 0
    m, _ = np.frexp(s.astype(np.float64))
    assert np.all(m == 0.5)                                    # powers of two
    assert np.all(s[nz] >= x[nz]) and np.all(s[nz] / 2 < x[nz])
    assert s[2, 2] == 1.0 and not q[2, 256:384].any()
    assert s[4, 0] == np.float32(2.0 ** -3)
    sc = np.repeat(s.astype(np.float64), 128, axis=1)
    quot = (v.astype(np.float64) / sc).astype(np.float32)      # exact: power-of-two divisor
    assert np.all(np.abs(quot) <= 448.0)
    assert np.array_equal(q, refimpl.f32_to_e4m3_sat(quot))
    # the same blocks quantized with amax/448 scales: s_pow2 is the power of two at or above
    _, s1 = oracle.quant_fp8(v)
    assert np.all(s[nz] >= s1[nz]) and np.all(s[nz] < 2 * s1[nz])


@pytest.mark.parametrize("seed", [0, 1])
def test_mxfp8_act_quant_bitexact_vs_numpy(seed):
    r = np.random.default_rng(seed)
    v = (r.standard_normal((29, 256)) * np.exp(r.uniform(-20, 20, (29, 1)))).astype(np.float32)
    v[5, 32:64] = 0.0
    q, e = oracle.quant_mxfp8(v)
    q2, e2 = refimpl.quant_mxfp8_rows(v)
    assert np.array_equal(e, e2) and np.array_equal(q, q2)
    assert e[5, 1] == 127 and not q[5, 32:64].any()
    # the largest code of a non-zero block has exponent field 15 (values 256..448)
    mags = (q & 0x7F).reshape(29, 8, 32).max(axis=2)
    nz = np.abs(v.reshape(29, 8, 32)).max(axis=2) > 0
    assert np.all((mags[nz] >> 3) == 15)


@pytest.mark.parametrize("fmt", [1, 2, 3, 4, 5])
def test_dequant_matches_reference(fmt):
    r = np.random.default_rng(fmt)
    N, K = 256, 384
    if fmt == 1:
        q = r.integers(0, 256, (N, K // 2), dtype=np.uint8)
        s = refimpl.torch.from_numpy(r.uniform(0.005, 0.02, (N, K // 32)).astype(np.float32)).to(refimpl.torch.bfloat16).view(refimpl.torch.int16).numpy().view(np.uint16)
    elif fmt in (2, 4):
        q = refimpl.f32_to_e4m3_sat(r.standard_normal((N, K)).astype(np.float32) * 100)
        s = r.uniform(1e-4, 1e-3, (N // 128, K // 128)).astype(np.float32)
        if fmt == 4:
            s = np.ldexp(np.float32(1.0), np.floor(np.log2(s)).astype(np.int32)).astype(np.float32)
    elif fmt == 5:
        q = r.integers(0, 256, (N, K // 2), dtype=np.uint8)
        s = r.integers(0x01, 0x7F, (K // 16, N), dtype=np.uint8)   # every positive E4M3 code
    else:
        q = r.integers(0, 256, (N, K // 2), dtype=np.uint8)
        s = r.integers(110, 130, (N, K // 32), dtype=np.uint8)
    g = 3.0517578125e-05 * 1.375 if fmt == 5 else 1.0
    got = oracle.dequant(fmt, N, K, q, s, g)
    ref = refimpl.dequant(fmt, q, s, N, K, g)
    assert np.array_equal(got.astype(np.float64), ref.astype(np.float32).astype(np.float64))


def test_nvfp4_layout_one_hot():
    """Element 2i sits in the low nibble of byte i; scale byte [g][n] covers
    row n, k in [16g, 16g+16); the second-level scale multiplies everything."""
    N, K = 2, 64
    q = np.zeros((N, K // 2), np.uint8)
    q[0, 0] = 0x2 | (0xF << 4)    # k=0 -> +1.0, k=1 -> -6.0
    q[1, 12] = 0x07               # k=24 -> +6.0
    q[1, 8] = 0x10                # k=17 -> +0.5
    s = np.full((K // 16, N), 0x38, np.uint8)  # E4M3 1.0
    s[1, 1] = 0x40                # 2.0 for row 1, k in [16, 32)
    w = oracle.dequant(5, N, K, q, s, 0.25)
    expect = np.zeros((N, K), np.float32)
    expect[0, 0], expect[0, 1], expect[1, 24], expect[1, 17] = 0.25, -1.5, 3.0, 0.25
    assert np.array_equal(w, expect)


def test_nvfp4_power_of_two_scales_reduce_to_mxfp4():
    """With E4M3 block scales that are powers of two 2^e (the same for both
    16-halves of a 32-group) and g = 1, NVFP4 decodes to exactly the MXFP4
    value of the same codes with E8M0 scale 127 + e."""
    r = np.random.default_rng(11)
    N, K = 64, 256
    q = r.integers(0, 256, (N, K // 2), dtype=np.uint8)
    e = r.integers(-6, 9, (K // 32, N))
    e8m0 = (127 + e).astype(np.uint8)                       # [K/32][N]
    e4m3 = ((e + 7) << 3).astype(np.uint8)                   # 2^e, mantissa 0 (e >= -6 is normal)
    s16 = np.repeat(e4m3, 2, axis=0)                         # [K/16][N]
    assert np.array_equal(oracle.dequant(5, N, K, q, s16, 1.0), oracle.dequant(3, N, K, q, e8m0))


def _flat_swap_would_differ(G, N, g, n):
    """True when scale [g][n] of a [G][N] group-major array lands on another
    (row, group) under the transposed [N][G] reading."""
    flat = g * N + n
    return (flat // G, flat % G) != (n, g)


def test_int4_layout_one_hot():
    """Element 2i sits in the low nibble of byte i; the bf16 scale stored at
    [g][n] of the group-major [K/32][N] array covers row n, k in [32g, 32g+32).
    N = 3 rows and K/32 = 4 groups make the scale array non-square, and the
    scale changed is off the diagonal, so a row-major [N][K/32] reading or a
    swapped (n, g) index moves the 2.0 onto another (row, group)."""
    N, K = 3, 128
    G = K // 32
    q = np.zeros((N, K // 2), np.uint8)
    q[0, 0] = 0x0F | (0x3 << 4)   # row 0: k=0 -> -1, k=1 -> 3
    q[1, 40] = 0x08               # row 1: k=80 (group 2) -> -8
    q[1, 50] = 0x50               # row 1: k=101 (group 3) -> 5
    q[2, 10] = 0x07               # row 2: k=20 (group 0) -> 7
    s = np.full((G, N), 0x3F80, np.uint16)  # 1.0
    s[2, 1] = 0x4000              # 2.0: row 1, k in [64, 96)
    s[0, 2] = 0x3F00              # 0.5: row 2, k in [0, 32)
    assert _flat_swap_would_differ(G, N, 2, 1) and _flat_swap_would_differ(G, N, 0, 2)
    w = oracle.dequant(1, N, K, q, s)
    expect = np.zeros((N, K), np.float32)
    expect[0, 0], expect[0, 1] = -1.0, 3.0
    expect[1, 80], expect[1, 101] = -16.0, 5.0
    expect[2, 20] = 3.5
    assert np.array_equal(w, expect)


def test_mxfp4_layout_one_hot():
    """E2M1 element 2i in the low nibble of byte i; the E8M0 byte at [g][n] of
    the group-major [K/32][N] array scales row n, k in [32g, 32g+32).  Non-square
    (N = 3, K/32 = 4) with off-diagonal scales, so a transposed reading fails."""
    N, K = 3, 128
    G = K // 32
    q = np.zeros((N, K // 2), np.uint8)
    q[0, 17] = 0x2 << 4           # row 0: k=35 (group 1) -> +1.0
    q[1, 48] = 0xF                # row 1: k=96 (group 3) -> -6.0
    q[1, 0] = 0x3                 # row 1: k=0 (group 0) -> +1.5
    q[2, 33] = 0x1                # row 2: k=66 (group 2) -> +0.5
    s = np.full((G, N), 127, np.uint8)   # 2^0
    s[1, 0] = 130                 # row 0, group 1: 2^3
    s[3, 1] = 125                 # row 1, group 3: 2^-2
    s[2, 2] = 121                 # row 2, group 2: 2^-6
    for g, n in ((1, 0), (3, 1), (2, 2)):
        if g != n:
            assert _flat_swap_would_differ(G, N, g, n)
    w = oracle.dequant(3, N, K, q, s)
    expect = np.zeros((N, K), np.float32)
    expect[0, 35] = 8.0
    expect[1, 96], expect[1, 0] = -1.5, 1.5
    expect[2, 66] = 0.5 / 64
    assert np.array_equal(w, expect)


def test_nvfp4_layout_one_hot_nonsquare():
    """NVFP4 scales [K/16][N] group-major: the E4M3 byte at [g][n] scales row n,
    k in [16g, 16g+16).  N = 3, K/16 = 8, off-diagonal scales."""
    N, K = 3, 128
    G = K // 16
    q = np.zeros((N, K // 2), np.uint8)
    q[0, 56] = 0x4                # row 0: k=112 (group 7) -> 2.0
    q[1, 8] = 0x6 << 4            # row 1: k=17 (group 1) -> 4.0
    q[2, 20] = 0xA                # row 2: k=40 (group 2) -> -1.0
    s = np.full((G, N), 0x38, np.uint8)  # E4M3 1.0
    s[7, 0] = 0x30                # 0.5
    s[1, 1] = 0x48                # 4.0 (diagonal on purpose: a swapped index reads s[?] = 1.0 elsewhere)
    s[2, 2] = 0x44                # 3.0
    assert _flat_swap_would_differ(G, N, 7, 0) and _flat_swap_would_differ(G, N, 1, 1)
    w = oracle.dequant(5, N, K, q, s, 0.5)
    expect = np.zeros((N, K), np.float32)
    expect[0, 112] = 0.5
    expect[1, 17] = 8.0
    expect[2, 40] = -1.5
    assert np.array_equal(w, expect)


def test_fp8_pow2_scale_floor_is_e8m0_min():
    """Power-of-two activation scales stay within E8M0's range: a block whose
    amax/448 lies below 2^-127 (bf16 subnormal inputs) takes s = 2^-127, one
    just above 2^-127 takes 2^-126, and the codes are E4M3 of v / s."""
    v = np.zeros((3, 128), np.float32)
    v[0, 0] = np.float32(2.0 ** -130)                  # amax/448 ~ 2^-138.8
    v[0, 1] = -np.float32(2.0 ** -133)
    v[1, 5] = np.float32(448.0 * 1.5 * 2.0 ** -127)    # amax/448 = 1.5 * 2^-127
    v[2, 9] = np.float32(448.0 * 2.0 ** -127)          # amax/448 = 2^-127 exactly
    q, s = oracle.quant_fp8_pow2(v)
    assert s[0, 0] == np.float32(2.0 ** -127) and s[1, 0] == np.float32(2.0 ** -126)
    assert s[2, 0] == np.float32(2.0 ** -127)
    assert q[0, 0] == 0x20                              # 2^-3: exponent field 4, mantissa 0
    assert q[0, 1] == 0x88                              # -2^-6: sign, exponent field 1
    assert q[1, 5] == 0x7A                              # 336, midway between 320 and 352: even code 320
    assert q[2, 9] == 0x7E                              # 448
