"""Independent numpy/torch re-derivations used to pin the oracle.

Nothing here is shared with the oracle's C code or with the HIP library: the
codecs come from library casts (torch float8 / bfloat16, numpy int8 shifts,
frexp/ldexp) or from the value tables of the OCP formats, and the dense MoE is
written as "every expert on every token, masked by the routing weights"
instead of the oracle's permute / chunk / combine structure.
"""
import numpy as np
import torch

# OCP MX v1.0 E2M1 values for codes 0..15 (sign bit 3).
E2M1_TABLE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                       -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def bf16_to_f32(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16).float().numpy()


def e4m3_to_f64(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def f32_to_e4m3_sat(v):
    """RNE to E4M3FN by torch's cast after clamping to +-448 (saturation)."""
    v = np.clip(np.asarray(v, np.float32), -448.0, 448.0)
    return torch.from_numpy(np.ascontiguousarray(v)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def unpack_nibbles(packed):
    """[..., K/2] bytes -> [..., K] nibbles (element 2i = low nibble of byte i)."""
    p = np.asarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def int4_values(nibbles):
    return ((np.asarray(nibbles, np.uint8) << 4).astype(np.int8) >> 4).astype(np.float64)


def dequant(fmt, q, s, N, K, g=1.0):
    if fmt == 5:
        # NVFP4: E2M1 values times the E4M3 scale of (n, 16 along K), group-major, times g
        v = E2M1_TABLE[unpack_nibbles(q)].reshape(N, K)
        sc = np.repeat(e4m3_to_f64(s).reshape(K // 16, N).T, 16, axis=1)
        return v * sc * np.float64(g)
    if fmt == 1:
        v = int4_values(unpack_nibbles(q)).reshape(N, K)
        sc = np.repeat(bf16_to_f32(s).astype(np.float64).reshape(K // 32, N).T, 32, axis=1)  # group-major
        return v * sc
    if fmt in (2, 4):
        v = e4m3_to_f64(q).reshape(N, K)
        sc = np.kron(np.asarray(s, np.float64).reshape(N // 128, K // 128), np.ones((128, 128)))
        return v * sc
    v = E2M1_TABLE[unpack_nibbles(q)].reshape(N, K)
    sc = np.repeat(np.ldexp(1.0, np.asarray(s, np.int64).reshape(K // 32, N).T - 127), 32, axis=1)
    return v * sc


def bf16_round_rto(v):
    """float64 -> nearest bf16 value (ties to even), by round-to-odd to fp32
    followed by torch's fp32 -> bf16 cast.  Rounding to odd at 24 bits then
    to nearest at 8 bits equals one rounding to nearest (Boldo & Melquiond,
    "When double rounding is odd", 2005: at least two extra bits suffice)."""
    v = np.asarray(v, np.float64)
    t = v.astype(np.float32)
    over = np.abs(t.astype(np.float64)) > np.abs(v)
    t = np.where(over, np.nextafter(t, np.float32(0.0)), t)      # truncate toward zero
    inexact = t.astype(np.float64) != v
    bits = t.view(np.uint32) | inexact.astype(np.uint32)         # sticky bit -> odd
    t = bits.view(np.float32)
    b = torch.from_numpy(np.ascontiguousarray(t)).to(torch.bfloat16).float().numpy()
    return b.astype(np.float64)


def quant_fp8_rows(v):
    """[R][K] fp32 -> codes, scales (s = amax/448 in fp32; amax = 0 -> 1)."""
    v = np.asarray(v, np.float32)
    R, K = v.shape
    blk = v.reshape(R, K // 128, 128)
    amax = np.abs(blk).max(axis=2)
    s = np.where(amax == 0, np.float32(1.0), amax / np.float32(448.0)).astype(np.float32)
    q = f32_to_e4m3_sat((blk / s[:, :, None]).astype(np.float32)).reshape(R, K)
    return q, s


def quant_fp8_pow2_rows(v):
    """[R][K] fp32 -> codes, power-of-two scales (the power of two at or above
    fl32(amax/448); amax = 0 -> 1)."""
    v = np.asarray(v, np.float32)
    R, K = v.shape
    blk = v.reshape(R, K // 128, 128)
    amax = np.abs(blk).max(axis=2)
    x = (amax / np.float32(448.0)).astype(np.float32)
    m, e = np.frexp(x.astype(np.float64))
    p2 = np.where(m == 0.5, x.astype(np.float64), np.ldexp(1.0, e))
    s = np.where(amax == 0, 1.0, p2).astype(np.float32)
    q = f32_to_e4m3_sat((blk.astype(np.float64) / s[:, :, None].astype(np.float64)).astype(np.float32)).reshape(R, K)
    return q, s


def quant_mxfp8_rows(v):
    v = np.asarray(v, np.float32)
    R, K = v.shape
    blk = v.reshape(R, K // 32, 32)
    amax = np.abs(blk).max(axis=2).astype(np.float64)
    _, p = np.frexp(amax)
    X = np.where(amax > 0, np.clip(p - 1 - 8, -127, 127), 0)
    scaled = np.ldexp(blk.astype(np.float64), -X[:, :, None]).astype(np.float32)
    q = f32_to_e4m3_sat(scaled).reshape(R, K)
    return q, (X + 127).astype(np.uint8)


def act_values(fmt, v32):
    """Activation format applied to fp32 rows -> float64 values."""
    if fmt in (1, 5):
        return np.asarray(v32, np.float64)
    if fmt == 2:
        q, s = quant_fp8_rows(v32)
        return e4m3_to_f64(q) * np.repeat(s.astype(np.float64), 128, axis=1)
    if fmt == 4:
        q, s = quant_fp8_pow2_rows(v32)
        return e4m3_to_f64(q) * np.repeat(s.astype(np.float64), 128, axis=1)
    q, e = quant_mxfp8_rows(v32)
    return e4m3_to_f64(q) * np.repeat(np.ldexp(1.0, e.astype(np.int64) - 127), 32, axis=1)


def route_bruteforce(logits, k):
    logits = np.asarray(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
        ids[t] = order
        top = np.array([float(logits[t, e]) for e in order])
        ex = np.exp(top - top[0])
        w[t] = ex / ex.sum()
    return ids, w


def dense_moe(T, H, I, E, k, fmt, x, logits, w13, w2, s13, s2, oft=None, adapter_stride_zero=False,
              materialized=False, g13=None, g2=None):
    """Dense MoE in float64: every expert runs on every token; the routing mask
    (softmax over the top-k, zero elsewhere) weights the sum.  materialized:
    weights rounded to bf16, bf16 GEMM inputs, h rounded to bf16, no
    activation quantizer."""
    xf = bf16_to_f32(x).reshape(T, H).astype(np.float32)
    ids, w = route_bruteforce(logits, k)
    mask = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            mask[t, ids[t, j]] = np.float32(w[t, j])
    out = np.zeros((T, H))
    for e in range(E):
        ga = 1.0 if g13 is None else g13[e]
        gb = 1.0 if g2 is None else g2[e]
        if materialized:
            W13 = bf16_round_rto(dequant(fmt, w13[e], s13[e], 2 * I, H, ga))
            W2 = bf16_round_rto(dequant(fmt, w2[e], s2[e], H, I, gb))
        else:
            W13 = dequant(fmt, w13[e], s13[e], 2 * I, H, ga).astype(np.float32).astype(np.float64)
            W2 = dequant(fmt, w2[e], s2[e], H, I, gb).astype(np.float32).astype(np.float64)
        xin = xf.astype(np.float64)
        if oft is not None:
            R = bf16_to_f32(oft if adapter_stride_zero else oft[e]).astype(np.float64).reshape(H // 32, 32, 32)
            xr = np.einsum("tbi,bij->tbj", xin.reshape(T, H // 32, 32), R).reshape(T, H)
            xin = bf16_round_rto(xr) if materialized else xr.astype(np.float32).astype(np.float64)
        xq = xin if materialized else act_values(fmt, xin.astype(np.float32))
        g = (xq @ W13[:I].T).astype(np.float32).astype(np.float64)
        u = (xq @ W13[I:].T).astype(np.float32).astype(np.float64)
        if materialized:
            hq = bf16_round_rto(g / (1.0 + np.exp(-g)) * u)
        else:
            h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
            hq = act_values(fmt, h)
        y = (hq @ W2.T).astype(np.float32).astype(np.float64)
        out += mask[:, e:e + 1] * y
    return out, ids, w
