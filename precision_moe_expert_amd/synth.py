"""Seeded synthetic inputs for the low-precision MoE expert layer.

This module only draws random numbers and casts them to storage dtypes with
library routines (numpy / torch casts).  It holds none of the layer's
arithmetic: no routing, no quantizer, no dequantizer, no GEMM.  Both the
CPU oracle and the HIP path are fed the same arrays from here.

Workload shapes follow the five layer shapes the MoE expert path is
measured on (tiny, Qwen3-30B-A3B-shaped FP8, Kimi-K2-shaped INT4 + OFT,
DeepSeek-V3-shaped MXFP4 with skewed routing, and a decode-sized
Kimi-K2-shaped INT4 + OFT layer followed by an LM head).

Weight storage (all K-contiguous, Y = X @ W^T):
  W13[E][2I][H]  gate rows 0..I-1 then up rows I..2I-1;  W2[E][H][I]
  int4   : two's-complement nibbles, element 2i in the low nibble of byte i;
           bf16 scales, group-major [E][K/32][N]
  fp8    : OCP E4M3FN codes, one byte each; fp32 scales [E][N/128][K/128]
  mxfp4  : E2M1 nibbles (low nibble first); E8M0 scale bytes, group-major [E][K/32][N]
  nvfp4  : E2M1 nibbles (low nibble first); E4M3 scale bytes per 16 along K,
           group-major [E][K/16][N]; fp32 second-level scales g13[E], g2[E]
OFT adapter: R[E][H/32][32][32] bf16, x' = x @ blockdiag(R_e).
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import hashlib
import os

import numpy as np
import torch

SEED_ROOT = 20261202
FMT_INT4, FMT_FP8, FMT_MXFP4, FMT_FP8_POW2, FMT_NVFP4 = 1, 2, 3, 4, 5
FMT_NAMES = {FMT_INT4: "int4_g32_bf16", FMT_FP8: "fp8_e4m3_b128", FMT_MXFP4: "mxfp4",
             FMT_FP8_POW2: "fp8_e4m3_b128_pow2", FMT_NVFP4: "nvfp4"}

# tensor ids inside one seed sequence
_T_X, _T_LOGITS, _T_ZIPF, _T_W13, _T_W2, _T_S13, _T_S2, _T_OFT, _T_WLM, _T_TGT, _T_G = range(11)


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    cfg_id: int
    T: int
    H: int
    E: int
    k: int
    I: int
    fmt: int
    chunk: int
    oft: bool = False
    zipf_alpha: float = 0.0
    lm_vocab: int = 0
    oft_sigma: float = 0.1

    @property
    def R(self) -> int:
        return self.T * self.k

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "c1": LayerConfig("tiny", 1, T=64, H=256, E=8, k=2, I=512, fmt=FMT_INT4, chunk=4),
    "c2": LayerConfig("qwen3_30b_a3b_fp8", 2, T=4096, H=2048, E=128, k=8, I=768,
                      fmt=FMT_FP8, chunk=16),
    "c3": LayerConfig("kimi_k2_int4_oft", 3, T=8192, H=7168, E=384, k=8, I=2048,
                      fmt=FMT_INT4, chunk=32, oft=True),
    "c4": LayerConfig("deepseek_v3_mxfp4_zipf", 4, T=16384, H=7168, E=256, k=8, I=2048,
                      fmt=FMT_MXFP4, chunk=32, zipf_alpha=1.2),
    "c5": LayerConfig("kimi_k2_decode_int4_oft_lmhead", 5, T=64, H=7168, E=384, k=8, I=2048,
                      fmt=FMT_INT4, chunk=32, oft=True, lm_vocab=32000),
    # the Qwen3-30B-A3B shape with the power-of-two scale variant of the FP8 recipe
    "c2p": LayerConfig("qwen3_30b_a3b_fp8_pow2", 6, T=4096, H=2048, E=128, k=8, I=768,
                       fmt=FMT_FP8_POW2, chunk=16),
    # the DeepSeek-V3 shape and routing with NVFP4 weights (the format the
    # B200/B300 samplers serve) and 16-bit activations
    "c4n": LayerConfig("deepseek_v3_nvfp4_zipf", 7, T=16384, H=7168, E=256, k=8, I=2048,
                       fmt=FMT_NVFP4, chunk=32, zipf_alpha=1.2),
}


def _rng(cfg_id: int, tensor: int, extra: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([SEED_ROOT, cfg_id, tensor, extra]))


def _per_expert(fn, E: int) -> None:
    """Runs fn(e) for every expert on a thread pool.  Each expert draws from its
    own seed and writes its own slice, so the result does not depend on the
    thread count (numpy's generators and torch's casts release the GIL)."""
    workers = max(1, min(16, os.cpu_count() or 1, E))
    if workers == 1:
        for e in range(E):
            fn(e)
        return
    with cf.ThreadPoolExecutor(workers) as ex:
        for _ in ex.map(fn, range(E)):
            pass


def _to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16) via torch's RNE cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _to_e4m3_codes(a: np.ndarray) -> np.ndarray:
    """float32 array (already within +-448) -> E4M3FN codes via torch's cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


# E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 drawn with fixed frequencies (a
# bell-shaped code histogram, like a quantized Gaussian block); out of 256.
_E2M1_MAG_WEIGHTS = [34, 62, 52, 36, 28, 24, 14, 6]


def _e2m1_nibble_lut() -> np.ndarray:
    lut = np.empty(256, np.uint8)
    pos = 0
    for mag, w in enumerate(_E2M1_MAG_WEIGHTS):
        lut[pos:pos + w] = mag
        pos += w
    assert pos == 256
    return lut


def gen_x(cfg: LayerConfig) -> np.ndarray:
    """Activations x[T][H] ~ N(0,1), stored as bf16 bits (uint16)."""
    r = _rng(cfg.cfg_id, _T_X)
    return _to_bf16_bits(r.standard_normal((cfg.T, cfg.H), dtype=np.float32))


def gen_logits(cfg: LayerConfig) -> np.ndarray:
    """Router logits[T][E] fp32 ~ N(0,1); with zipf_alpha > 0 each expert gets the
    bias -alpha*ln(rank), rank a seeded permutation of 1..E (Zipf-like popularity)."""
    r = _rng(cfg.cfg_id, _T_LOGITS)
    lg = r.standard_normal((cfg.T, cfg.E), dtype=np.float32)
    if cfg.zipf_alpha > 0:
        rank = _rng(cfg.cfg_id, _T_ZIPF).permutation(cfg.E) + 1
        bias = (-cfg.zipf_alpha * np.log(rank.astype(np.float64))).astype(np.float32)
        lg = lg + bias[None, :]
    return np.ascontiguousarray(lg, dtype=np.float32)


def _gen_int4(cfg, N, K, tensor, stensor):
    E = cfg.E
    q = np.empty((E, N, K // 2), np.uint8)
    s = np.empty((E, K // 32, N), np.uint16)  # group-major: s[e][g][n] scales row n, k in [32g, 32g+32)
    def one(e):
        # uniform bytes = two independent uniform nibbles over all 16 codes
        q[e] = _rng(cfg.cfg_id, tensor, e).integers(0, 256, (N, K // 2), dtype=np.uint8)
        s[e] = _to_bf16_bits(_rng(cfg.cfg_id, stensor, e).uniform(0.005, 0.02, (N, K // 32)).astype(np.float32)).T
    _per_expert(one, E)
    return q, s


def _gen_fp8(cfg, N, K, tensor, stensor):
    E = cfg.E
    q = np.empty((E, N, K), np.uint8)
    s = np.empty((E, N // 128, K // 128), np.float32)
    sig = 448.0 / 4.5  # code-space spread: block maxima land near the top codes
    def one(e):
        v = _rng(cfg.cfg_id, tensor, e).standard_normal((N, K), dtype=np.float32) * sig
        q[e] = _to_e4m3_codes(np.clip(v, -448.0, 448.0))
        # block scales so that weights are ~N(0, 0.02^2)
        s[e] = (_rng(cfg.cfg_id, stensor, e).uniform(0.5, 1.5, (N // 128, K // 128)) * (0.02 / sig)).astype(np.float32)
    _per_expert(one, E)
    return q, s


def _gen_fp8_pow2(cfg, N, K, tensor, stensor):
    """FP8 weights whose [128,128] block scales are powers of two (the
    block scales of _gen_fp8 rounded down to a power of two)."""
    q, s = _gen_fp8(cfg, N, K, tensor, stensor)
    return q, np.ldexp(np.float32(1.0), np.floor(np.log2(s)).astype(np.int32)).astype(np.float32)


def _gen_mxfp4(cfg, N, K, tensor, stensor):
    E = cfg.E
    mag = _e2m1_nibble_lut()
    # byte value -> nibble code: low 8 bits choose magnitude, bit 8 chooses sign
    lut16 = np.empty(512, np.uint8)
    lut16[:256] = mag
    lut16[256:] = mag | 8
    q = np.empty((E, N, K // 2), np.uint8)
    s = np.empty((E, K // 32, N), np.uint8)  # group-major, as for INT4
    def one(e):
        r = _rng(cfg.cfg_id, tensor, e)
        lo = lut16[r.integers(0, 512, (N, K // 2), dtype=np.uint16)]
        hi = lut16[r.integers(0, 512, (N, K // 2), dtype=np.uint16)]
        q[e] = lo | (hi << 4)
        # E8M0 scale bytes 2^-8 .. 2^-6 -> weights of magnitude ~0.02
        s[e] = _rng(cfg.cfg_id, stensor, e).integers(119, 122, (N, K // 32), dtype=np.uint8).T
    _per_expert(one, E)
    return q, s


def _gen_nvfp4(cfg, N, K, tensor, stensor):
    """E2M1 codes as for MXFP4; E4M3 block scales log-uniform in [16, 448]
    (the range a per-16 amax / 6 maps to under a second-level scale)."""
    E = cfg.E
    q, _ = _gen_mxfp4(cfg, N, K, tensor, stensor)
    s = np.empty((E, K // 16, N), np.uint8)  # group-major: s[e][g][n] scales row n, k in [16g, 16g+16)
    def one(e):
        v = np.exp2(_rng(cfg.cfg_id, stensor, 1000 + e).uniform(4.0, np.log2(448.0), (K // 16, N)))
        s[e] = _to_e4m3_codes(v.astype(np.float32))
    _per_expert(one, E)
    return q, s


def gen_gscales(cfg: LayerConfig):
    """NVFP4 second-level scales (fp32, one per expert and matrix) such that
    weights are ~0.02 in magnitude; (None, None) for the other formats."""
    if cfg.fmt != FMT_NVFP4:
        return None, None
    r = _rng(cfg.cfg_id, _T_G)
    g13 = (r.uniform(0.8, 1.2, cfg.E) * 2.0e-4).astype(np.float32)
    g2 = (r.uniform(0.8, 1.2, cfg.E) * 2.0e-4).astype(np.float32)
    return g13, g2


def gen_weights(cfg: LayerConfig):
    """Returns (w13, w2, s13, s2) as numpy arrays in the storage layouts above."""
    H, I = cfg.H, cfg.I
    gen = {FMT_INT4: _gen_int4, FMT_FP8: _gen_fp8, FMT_MXFP4: _gen_mxfp4, FMT_FP8_POW2: _gen_fp8_pow2,
           FMT_NVFP4: _gen_nvfp4}[cfg.fmt]
    w13, s13 = gen(cfg, 2 * I, H, _T_W13, _T_S13)
    w2, s2 = gen(cfg, H, I, _T_W2, _T_S2)
    return w13, w2, s13, s2


def gen_oft(cfg: LayerConfig, sigma: float | None = None) -> np.ndarray:
    """OFT adapter R[E][H/32][32][32] bf16 bits: per 32x32 block the Cayley
    transform R = (I - S)(I + S)^-1 of a skew-symmetric S (upper-triangle
    entries ~N(0, sigma^2)), computed in float64 and cast to bf16."""
    sig = cfg.oft_sigma if sigma is None else sigma
    nb = cfg.H // 32
    out = np.empty((cfg.E, nb, 32, 32), np.uint16)
    eye = np.eye(32)
    iu = np.triu_indices(32, 1)
    def one(e):
        u = np.zeros((nb, 32, 32))
        u[:, iu[0], iu[1]] = _rng(cfg.cfg_id, _T_OFT, e).standard_normal((nb, len(iu[0]))) * sig
        s = u - np.transpose(u, (0, 2, 1))
        # (I - S)(I + S)^-1 == solve((I + S)^T, (I - S)^T)^T; both factors commute
        r = np.linalg.solve(eye + s, eye - s)
        out[e] = _to_bf16_bits(r.astype(np.float32))
    _per_expert(one, cfg.E)
    return out


def gen_lm_head(cfg: LayerConfig):
    """LM head W_lm[V][H] ~ N(0, 1/H) bf16 bits, targets[T] uniform int32 in [0, V)."""
    V = cfg.lm_vocab
    w = np.empty((V, cfg.H), np.uint16)
    step = 4096

    def one(b):
        i = b * step
        r = _rng(cfg.cfg_id, _T_WLM, i)
        n = min(step, V - i)
        w[i:i + n] = _to_bf16_bits(r.standard_normal((n, cfg.H), dtype=np.float32) / np.float32(np.sqrt(cfg.H)))
    _per_expert(one, (V + step - 1) // step)
    tgt = _rng(cfg.cfg_id, _T_TGT).integers(0, V, cfg.T, dtype=np.int64).astype(np.int32)
    return w, tgt


@dataclasses.dataclass
class LayerInputs:
    cfg: LayerConfig
    x: np.ndarray
    logits: np.ndarray
    w13: np.ndarray
    w2: np.ndarray
    s13: np.ndarray
    s2: np.ndarray
    oft: np.ndarray | None
    w_lm: np.ndarray | None = None
    targets: np.ndarray | None = None
    g13: np.ndarray | None = None  # NVFP4 second-level scales
    g2: np.ndarray | None = None

    def digest(self) -> dict:
        out = {}
        for name in ("x", "logits", "w13", "w2", "s13", "s2", "oft", "w_lm", "targets", "g13", "g2"):
            a = getattr(self, name)
            if a is not None:
                out[name] = hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]
        return out


def make_inputs(cfg: LayerConfig, with_lm: bool | None = None) -> LayerInputs:
    oft = gen_oft(cfg) if cfg.oft else None
    w13, w2, s13, s2 = gen_weights(cfg)
    li = LayerInputs(cfg, gen_x(cfg), gen_logits(cfg), w13, w2, s13, s2, oft)
    li.g13, li.g2 = gen_gscales(cfg)
    if (cfg.lm_vocab > 0) if with_lm is None else with_lm:
        li.w_lm, li.targets = gen_lm_head(cfg)
    return li
