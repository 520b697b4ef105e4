// Activation preparation: the expert GEMMs' A operand, once per token (no
// adapter) or once per permuted row (OFT adapter, which depends on the expert).
#include "common.h"
#include "kernels.h"

namespace moe {

// x bf16 [T][H] -> fp16, in the INT4-path layout (I4ORDER: groups of 8 stored
// in the order 0,4,1,5,2,6,3,7) or in natural order (the NVFP4 path).
// bf16 -> fp16 is exact for |x| in [2^-14, 65504].
template <bool I4ORDER>
__global__ __launch_bounds__(256) void k_act_f16(const uint16_t* __restrict__ x, int64_t n8,
                                                 uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const uint4 v = reinterpret_cast<const uint4*>(x)[i];
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float f[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = bf16_bits_to_f32(w[j] & 0xFFFFu);
    f[2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
  }
  uint4 o;
  if (I4ORDER) {
    o.x = pack_f16x2(f[0], f[4]);
    o.y = pack_f16x2(f[1], f[5]);
    o.z = pack_f16x2(f[2], f[6]);
    o.w = pack_f16x2(f[3], f[7]);
  } else {
    o.x = pack_f16x2(f[0], f[1]);
    o.y = pack_f16x2(f[2], f[3]);
    o.z = pack_f16x2(f[4], f[5]);
    o.w = pack_f16x2(f[6], f[7]);
  }
  reinterpret_cast<uint4*>(out)[i] = o;
}

// FP8 [1,128] activation quantization (NeMo RL FP8 post, Table 1, input
// activations): per 128-block s = amax/448 (IEEE fp32 division; 1 if amax =
// 0), codes = E4M3(v / s).  One wave per token; a lane owns 32 elements, four
// lanes a block.
template <bool POW2>
__global__ __launch_bounds__(256) void k_act_fp8(const uint16_t* __restrict__ x, int T, int H,
                                                 uint8_t* __restrict__ q, float* __restrict__ sc, int sc_stride) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (t >= T) return;
  for (int base = 0; base < H; base += 2048) {
    const int c0 = base + lane * 32;
    const bool valid = c0 < H;
    float v[32];
    float amax = 0.0f;
    if (valid) {
      const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)t * H + c0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 u = src[j];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          v[8 * j + 2 * h] = bf16_bits_to_f32(w[h] & 0xFFFFu);
          v[8 * j + 2 * h + 1] = bf16_bits_to_f32(w[h] >> 16);
        }
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
    amax = fmaxf(amax, shfl_xor(amax, 1));
    amax = fmaxf(amax, shfl_xor(amax, 2));
    if (!valid) continue;
    uint32_t packed[8];
    float s;
    if (POW2) {
      // the power of two at or above amax/448; codes v * 2^-e, exact scaling
      s = (amax == 0.0f) ? 1.0f : pow2_at_least(amax / 448.0f);
      const float inv = pow2_reciprocal(s);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        packed[j] = cvt_e4m3x4(v[4 * j] * inv, v[4 * j + 1] * inv, v[4 * j + 2] * inv, v[4 * j + 3] * inv);
    } else {
      s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        packed[j] = cvt_e4m3x4(v[4 * j] / s, v[4 * j + 1] / s, v[4 * j + 2] / s, v[4 * j + 3] / s);
    }
    uint4* dst = reinterpret_cast<uint4*>(q + (int64_t)t * H + c0);
    dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    if ((lane & 3) == 0) sc[(int64_t)t * (sc_stride / 4) + c0 / 128] = s;
  }
}

// floor(log2(a)) of a positive finite float, from its bit pattern.
MOE_DEV int floor_log2_pos(float a) {
  const uint32_t b = __float_as_uint(a);
  const int ef = (int)(b >> 23);
  if (ef > 0) return ef - 127;
  return (31 - __builtin_clz(b & 0x7FFFFFu)) - 149;
}

// 2^n as a float for n in [-127, 127].
MOE_DEV float exp2_int(int n) {
  return n >= -126 ? __uint_as_float((uint32_t)(n + 127) << 23) : __uint_as_float(0x00400000u);
}

// MXFP8 quantization of 32 values: shared exponent X = floor(log2 amax) - 8
// (clamped to [-127, 127]; 0 when amax = 0), codes = E4M3(v * 2^-X) with
// saturation.  Writes 32 code bytes as 8 dwords and returns the E8M0 byte.
MOE_DEV uint32_t mx_quant32(const float* v, float amax, uint32_t* packed) {
  int X = 0;
  if (amax > 0.0f) {
    X = floor_log2_pos(amax) - 8;
    X = X < -127 ? -127 : (X > 127 ? 127 : X);
  }
  const float m = exp2_int(-X);
#pragma unroll
  for (int j = 0; j < 8; ++j) packed[j] = cvt_e4m3x4(v[4 * j] * m, v[4 * j + 1] * m, v[4 * j + 2] * m, v[4 * j + 3] * m);
  return (uint32_t)(X + 127);
}

// MXFP8 activation quantization per token: a lane owns one 32-block.
__global__ __launch_bounds__(256) void k_act_mxfp8(const uint16_t* __restrict__ x, int T, int H,
                                                   uint8_t* __restrict__ q, uint8_t* __restrict__ e8, int e8_stride) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (t >= T) return;
  for (int c0 = lane * 32; c0 < H; c0 += 2048) {
    float v[32];
    float amax = 0.0f;
    const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)t * H + c0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 u = src[j];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        v[8 * j + 2 * h] = bf16_bits_to_f32(w[h] & 0xFFFFu);
        v[8 * j + 2 * h + 1] = bf16_bits_to_f32(w[h] >> 16);
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    uint32_t packed[8];
    const uint32_t eb = mx_quant32(v, amax, packed);
    uint4* dst = reinterpret_cast<uint4*>(q + (int64_t)t * H + c0);
    dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    e8[(int64_t)t * e8_stride + c0 / 32] = (uint8_t)eb;
  }
}

// LDS written by some lanes of a wave is visible to the wave's other lanes.
__device__ __forceinline__ void oft_wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Output formats of the OFT rotation: the GEMM1 input of each weight format.
enum { OFT_F16_I4 = 0,  // fp16 in the INT4-path layout (groups of 8 as 0,4,1,5,2,6,3,7)
       OFT_BF16 = 1,    // bf16, natural order (the BF16 GEMMs of the materialized scheme)
       OFT_F16 = 2,     // fp16, natural order (NVFP4 weights)
       OFT_FP8 = 3,     // E4M3 codes + fp32 scale per [1,128]: s = amax/448, RNE(v/s)
       OFT_FP8_POW2 = 4,// E4M3 codes + power-of-two fp32 scale per [1,128]
       OFT_MXFP8 = 5 }; // E4M3 codes + E8M0 scale per 32 (MXFP4 weights)

// OFT rotation x' = x R_e (R_e block-diagonal, 32x32 bf16 blocks; row i of a
// block indexes the input dim) for every permuted row, on bf16 MFMA with fp32
// accumulation, written in the GEMM1 input format OUT of the weight format.
// Work item = 16 rows of one expert (the 16-row tile list) times 16
// consecutive diagonal blocks, 4 per wave: a wave loads its 4 blocks of R_e
// (8 KB) and x values at once, stages the blocks in its own LDS slice and
// runs 8 MFMAs, so each item costs one memory round trip.  A wave's 4 blocks
// are 128 columns, i.e. exactly one FP8 [1,128] block per row (H is a
// multiple of 256), and each diagonal block is one MXFP8 32-block, so the
// quantized formats take their block maxima from the wave's own registers
// (16-lane row reductions), stage the codes in the wave's LDS slice and
// write 16-byte pieces.  The active experts' tile starts are kept in LDS for
// the item -> expert search.
template <int OUT>
__global__ __launch_bounds__(256) void k_oft(const uint16_t* __restrict__ x, const uint16_t* __restrict__ R,
                                             int64_t r_stride, int H, int k, const int32_t* __restrict__ offsets,
                                             const int32_t* __restrict__ sorted_rows,
                                             const int32_t* __restrict__ active,
                                             const int32_t* __restrict__ num_active,
                                             const int32_t* __restrict__ tile16,
                                             const int32_t* __restrict__ desc16, void* __restrict__ out,
                                             void* __restrict__ out_scale, int scale_stride) {
  constexpr int BPW = 4;  // diagonal blocks per wave and item
  constexpr bool QUANT = OUT == OFT_FP8 || OUT == OFT_FP8_POW2 || OUT == OFT_MXFP8;
  __shared__ __align__(16) uint16_t rs[4][BPW][32 * 32];
  __shared__ __align__(16) uint8_t qs[QUANT ? 4 : 1][16 * 128];  // a wave's 16 rows x 128 codes
  __shared__ int32_t s_t16[MAX_EXPERTS + 1];
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int ln = lane & 15, lg = lane >> 4;
  const int na = *num_active;
  for (int i = threadIdx.x; i <= na; i += 256) s_t16[i] = tile16[i];
  __syncthreads();
  const int ngroups = s_t16[na];
  const int nb = H / 32;
  const int nbc = (nb + 4 * BPW - 1) / (4 * BPW);
  const int64_t nitems = (int64_t)ngroups * nbc;
  for (int64_t it = blockIdx.x; it < nitems; it += gridDim.x) {
    const int gi = (int)(it / nbc), bc = (int)(it - (int64_t)gi * nbc);
    const int b0 = (bc * 4 + wave) * BPW;
    const int nbw = min(BPW, nb - b0);  // <= 0: no blocks for this wave
    if (nbw <= 0) continue;
    int e, r0, nrows;
    if (desc16 != nullptr) {
      // the group's descriptor {expert, first row, rows, active index}: one
      // load instead of the search and the expert / offset loads after it
      const i32x4 dd = *reinterpret_cast<const i32x4*>(desc16 + 4 * (int64_t)gi);
      e = dd[0];
      r0 = dd[1];
      nrows = dd[2];
    } else {
      int lo = 0, hi = na - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_t16[mid] <= gi) lo = mid; else hi = mid - 1;
      }
      e = active[lo];
      r0 = offsets[e] + (gi - s_t16[lo]) * 16;
      nrows = min(16, offsets[e + 1] - r0);
    }
    const int tok = sorted_rows[r0 + min(ln, nrows - 1)] / k;
    const uint16_t* xrow = x + (int64_t)tok * H;
    const uint4* src = reinterpret_cast<const uint4*>(R + (int64_t)e * r_stride + (int64_t)b0 * 1024);
    // (a wave with fewer than BPW blocks loads its last block again)
    uint4 rv[BPW][2], xv[BPW];
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const int jj = min(j, nbw - 1);
      rv[j][0] = src[jj * 128 + lane * 2];
      rv[j][1] = src[jj * 128 + lane * 2 + 1];
      xv[j] = *reinterpret_cast<const uint4*>(xrow + (b0 + jj) * 32 + lg * 8);
    }
    // a wave's LDS accesses run in order, so the previous item's reads of
    // this slice are done before these writes
#pragma unroll
    for (int j = 0; j < BPW; ++j)
      if (j < nbw) {
        uint4* dst = reinterpret_cast<uint4*>(rs[wave][j]);
        dst[lane * 2] = rv[j][0];
        dst[lane * 2 + 1] = rv[j][1];
      }
    oft_wave_lds_sync();
    // acc[j][half][i]: row lg*4 + i, column (b0 + j)*32 + half*16 + ln
    f32x4 acc[BPW][2];
#pragma unroll
    for (int j = 0; j < BPW; ++j)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        acc[j][half] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
        if (j < nbw) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, xv[j]);
          const uint16_t* rc = rs[wave][j] + lg * 8 * 32 + half * 16 + ln;
          u32x4 bw;
          bw.x = (uint32_t)rc[0] | ((uint32_t)rc[32] << 16);
          bw.y = (uint32_t)rc[64] | ((uint32_t)rc[96] << 16);
          bw.z = (uint32_t)rc[128] | ((uint32_t)rc[160] << 16);
          bw.w = (uint32_t)rc[192] | ((uint32_t)rc[224] << 16);
          acc[j][half] = mfma_bf16_16x16x32(a, __builtin_bit_cast(bf16x8, bw), acc[j][half]);
        }
      }
    if constexpr (!QUANT) {
      // The wave's 16 rows x 128 columns go through its own R slice (free
      // once the MFMAs above hold their operands; a wave's LDS accesses run
      // in order) and leave as 16-byte row pieces instead of 2-byte stores.
      // The INT4 activation order permutes within aligned groups of 8, so
      // it can be applied to the column within the wave's 128.
      uint8_t* stg = reinterpret_cast<uint8_t*>(rs[wave]);
      constexpr int SR = 272;  // staged row stride (bytes), 4 banks apart
#pragma unroll
      for (int j = 0; j < BPW; ++j)
        if (j < nbw)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int c = j * 32 + half * 16 + ln;
            const int col = OUT == OFT_F16_I4 ? i4act_pos(c) : c;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const _Float16 hv = (_Float16)acc[j][half][i];
              *reinterpret_cast<uint16_t*>(stg + (lg * 4 + i) * SR + col * 2) =
                  OUT == OFT_BF16 ? (uint16_t)f32_to_bf16_bits(acc[j][half][i]) : __builtin_bit_cast(uint16_t, hv);
            }
          }
      oft_wave_lds_sync();
      uint16_t* o = static_cast<uint16_t*>(out);
      const int nparts = nbw * 4;  // 16-byte pieces of a row that this wave holds
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int q = lane + h * 64, row = q >> 4, part = q & 15;
        if (row < nrows && part < nparts)
          *reinterpret_cast<uint4*>(o + (int64_t)(r0 + row) * H + b0 * 32 + part * 8) =
              *reinterpret_cast<const uint4*>(stg + row * SR + part * 16);
      }
    } else {
      // block maxima per row (the row's 16 lanes share lg), codes into the
      // wave's staging slice qs[wave][row][col - 128 * (b0 / 4)]
      uint8_t* q = qs[wave];
      if constexpr (OUT == OFT_MXFP8) {
#pragma unroll
        for (int j = 0; j < BPW; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float am = row16_max_nonneg(fmaxf(fabsf(acc[j][0][i]), fabsf(acc[j][1][i])));
            int X = 0;
            if (am > 0.0f) {
              X = floor_log2_pos(am) - 8;
              X = X < -127 ? -127 : (X > 127 ? 127 : X);
            }
            const float mul = exp2_int(-X);
            const uint32_t c2 = cvt_e4m3x2(acc[j][0][i] * mul, acc[j][1][i] * mul);
            const int m = lg * 4 + i;
            q[m * 128 + j * 32 + ln] = (uint8_t)(c2 & 0xFF);
            q[m * 128 + j * 32 + 16 + ln] = (uint8_t)(c2 >> 8);
            if (ln == 0 && m < nrows)
              static_cast<uint8_t*>(out_scale)[(int64_t)(r0 + m) * scale_stride + b0 + j] = (uint8_t)(X + 127);
          }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float am = 0.0f;
#pragma unroll
          for (int j = 0; j < BPW; ++j) am = fmaxf(am, fmaxf(fabsf(acc[j][0][i]), fabsf(acc[j][1][i])));
          am = row16_max_nonneg(am);
          const int m = lg * 4 + i;
          float sc;
          if constexpr (OUT == OFT_FP8_POW2) {
            sc = am == 0.0f ? 1.0f : pow2_at_least(am / 448.0f);
            const float inv = pow2_reciprocal(sc);
#pragma unroll
            for (int j = 0; j < BPW; ++j) {
              const uint32_t c2 = cvt_e4m3x2(acc[j][0][i] * inv, acc[j][1][i] * inv);
              q[m * 128 + j * 32 + ln] = (uint8_t)(c2 & 0xFF);
              q[m * 128 + j * 32 + 16 + ln] = (uint8_t)(c2 >> 8);
            }
          } else {
            sc = am == 0.0f ? 1.0f : am / 448.0f;
#pragma unroll
            for (int j = 0; j < BPW; ++j) {
              const uint32_t c2 = cvt_e4m3x2(acc[j][0][i] / sc, acc[j][1][i] / sc);
              q[m * 128 + j * 32 + ln] = (uint8_t)(c2 & 0xFF);
              q[m * 128 + j * 32 + 16 + ln] = (uint8_t)(c2 >> 8);
            }
          }
          if (ln == 0 && m < nrows)
            static_cast<float*>(out_scale)[(int64_t)(r0 + m) * (scale_stride / 4) + b0 / 4] = sc;
        }
      }
      oft_wave_lds_sync();
      // 16 rows x 128 codes: lane l writes 32 bytes of row l/4
      const int m = lane >> 2, part = lane & 3;
      if (m < nrows) {
        const u32x4* sp = reinterpret_cast<const u32x4*>(q + m * 128 + part * 32);
        u32x4* dp = reinterpret_cast<u32x4*>(static_cast<uint8_t*>(out) + (int64_t)(r0 + m) * H + b0 * 32 + part * 32);
        dp[0] = sp[0];
        dp[1] = sp[1];
      }
    }
    oft_wave_lds_sync();  // this item's LDS reads are issued before the next item's writes
  }
}

void launch_act_f16(const uint16_t* x, int T, int H, uint16_t* out, hipStream_t s) {
  const int64_t n8 = (int64_t)T * H / 8;
  if (n8 == 0) return;
  hipLaunchKernelGGL(k_act_f16<true>, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, x, n8, out);
}
void launch_act_f16_natural(const uint16_t* x, int T, int H, uint16_t* out, hipStream_t s) {
  const int64_t n8 = (int64_t)T * H / 8;
  if (n8 == 0) return;
  hipLaunchKernelGGL(k_act_f16<false>, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, x, n8, out);
}
void launch_act_fp8(const uint16_t* x, int T, int H, uint8_t* q, float* sc, int sc_stride, bool pow2,
                    hipStream_t s) {
  if (pow2) hipLaunchKernelGGL(k_act_fp8<true>, dim3((T + 3) / 4), dim3(256), 0, s, x, T, H, q, sc, sc_stride);
  else hipLaunchKernelGGL(k_act_fp8<false>, dim3((T + 3) / 4), dim3(256), 0, s, x, T, H, q, sc, sc_stride);
}
void launch_act_mxfp8(const uint16_t* x, int T, int H, uint8_t* q, uint8_t* e8, int e8_stride, hipStream_t s) {
  hipLaunchKernelGGL(k_act_mxfp8, dim3((T + 3) / 4), dim3(256), 0, s, x, T, H, q, e8, e8_stride);
}
void launch_oft(int out_fmt, const uint16_t* x, const uint16_t* R, int64_t r_expert_stride, int H, int k,
                const int32_t* offsets, const int32_t* sorted_rows, const int32_t* active, const int32_t* num_active,
                const int32_t* tile16, const int32_t* desc16, void* out, void* out_scale, int scale_stride,
                hipStream_t s) {
  switch (out_fmt) {
#define MOE_OFT_CASE(F)                                                                                              \
    case F:                                                                                                          \
      hipLaunchKernelGGL(k_oft<F>, dim3(1024), dim3(256), 0, s, x, R, r_expert_stride, H, k, offsets, sorted_rows, \
                         active, num_active, tile16, desc16, out, out_scale, scale_stride);                          \
      break;
    MOE_OFT_CASE(OFT_F16_I4)
    MOE_OFT_CASE(OFT_BF16)
    MOE_OFT_CASE(OFT_F16)
    MOE_OFT_CASE(OFT_FP8)
    MOE_OFT_CASE(OFT_FP8_POW2)
    MOE_OFT_CASE(OFT_MXFP8)
#undef MOE_OFT_CASE
    default: break;
  }
}

void launch_oft_f16(const uint16_t* x, const uint16_t* R, int64_t r_expert_stride, int H, int k,
                    const int32_t* offsets, const int32_t* sorted_rows, const int32_t* active,
                    const int32_t* num_active, const int32_t* tile16, int E, uint16_t* out, hipStream_t s) {
  (void)E;
  launch_oft(OFT_F16_I4, x, R, r_expert_stride, H, k, offsets, sorted_rows, active, num_active, tile16, nullptr, out, nullptr,
             0, s);
}

void launch_oft_bf16(const uint16_t* x, const uint16_t* R, int64_t r_expert_stride, int H, int k,
                     const int32_t* offsets, const int32_t* sorted_rows, const int32_t* active,
                     const int32_t* num_active, const int32_t* tile16, uint16_t* out, hipStream_t s) {
  launch_oft(OFT_BF16, x, R, r_expert_stride, H, k, offsets, sorted_rows, active, num_active, tile16, nullptr, out, nullptr, 0,
             s);
}

}  // namespace moe
