// Grouped expert GEMMs for MXFP4 weights (E2M1 + E8M0 per 32 along K) with
// MXFP8 activations (E4M3 + E8M0 per 32), on gfx950's block-scaled
// 16x16x128 MFMA: the hardware applies both E8M0 scales, so the
// dequantization costs no vector instructions at all.
//
// Operand layout of the scaled MFMA (lane l, row/column l%16, group g = l/16):
//   A (E4M3): bytes 0..15 = k in [16g, 16g+16), bytes 16..31 = k in [64+16g, 64+16g+16)
//   B (E2M1): 32 nibbles  = k in [32g, 32g+32)
//   scales  : lane l carries row (column) l%16's scale of K block g.
// GEMM1's epilogue quantizes h = silu(gate) * up to MXFP8; a wave's 32 h
// columns are exactly one scale block, so the block maximum is a wave-local
// shuffle reduction.
#include "common.h"
#include "kernels.h"
#include "moe_sched.h"

namespace moe {

MOE_DEV float floor_log2_pos_mx(float a) {
  const uint32_t b = __float_as_uint(a);
  const int ef = (int)(b >> 23);
  return ef > 0 ? (float)(ef - 127) : (float)((31 - __builtin_clz(b & 0x7FFFFFu)) - 149);
}

template <int BM, bool G1>
__global__ __launch_bounds__(256) void k_gemm_mxfp4(GemmArgs p) {
  constexpr int MT = BM / 16;
  constexpr int LDA = 128 + 16;
  constexpr int NCHUNK = BM * 8;
  constexpr int ALOADS = (NCHUNK + 255) / 256;
  __shared__ __align__(16) uint8_t As[2][BM * LDA];
  __shared__ __align__(16) uint32_t Ss[2][BM];
  const int nblk = G1 ? p.inter / 128 : p.N / 256;
  ChunkWork cw;
  if (!chunk_work(p, nblk, cw)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ln = lane & 15, lg = lane >> 4;
  const int K = p.K, KT = K / 128;
  const uint8_t* A = static_cast<const uint8_t*>(p.a);
  const uint8_t* AS = static_cast<const uint8_t*>(p.a_scale);
  const uint8_t* WS = static_cast<const uint8_t*>(p.w_scale);

  for (int wk = xcd_virtual_id(); wk < cw.nwork; wk += gridDim.x) {
    const Tile tl = tile_of(p, cw, wk, BM);
    int col[4];
    if (G1) {
      const int g0 = tl.nb * 128 + wave * 32;
      col[0] = g0; col[1] = g0 + 16; col[2] = p.inter + g0; col[3] = p.inter + g0 + 16;
    } else {
      const int c0 = tl.nb * 256 + wave * 64;
#pragma unroll
      for (int i = 0; i < 4; ++i) col[i] = c0 + 16 * i;
    }
    const uint8_t* wrow[4];
    const uint8_t* wsrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wrow[i] = p.w + tl.e * p.w_expert_bytes + (int64_t)(col[i] + ln) * (K / 2) + lg * 16;
      wsrow[i] = WS + tl.e * p.ws_expert_elems + (int64_t)(col[i] + ln) * (K / 32) + lg;
    }
    const uint8_t* arow[ALOADS];
    int lrow[ALOADS], lpart[ALOADS];
#pragma unroll
    for (int j = 0; j < ALOADS; ++j) {
      const int c = threadIdx.x + 256 * j;
      lrow[j] = c / 8;
      lpart[j] = c % 8;
      const int rr = tl.rbase + min(min(lrow[j], BM - 1), tl.nrows - 1);
      const int src = p.a_per_token ? p.sorted_rows[rr] / p.top_k : rr;
      arow[j] = A + (int64_t)src * K + lpart[j] * 16;
    }
    const uint32_t* srow = nullptr;
    if (threadIdx.x < BM) {
      const int rr = tl.rbase + min((int)threadIdx.x, tl.nrows - 1);
      const int src = p.a_per_token ? p.sorted_rows[rr] / p.top_k : rr;
      srow = reinterpret_cast<const uint32_t*>(AS + (int64_t)src * (K / 32));
    }
    f32x4 acc[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[m][i] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

    uint4 areg[ALOADS];
    uint32_t sreg = 0;
    uint4 bcur[4], bnext[4];
    int wscur[4], wsnext[4];
#pragma unroll
    for (int j = 0; j < ALOADS; ++j)
      if (lrow[j] < BM) areg[j] = *reinterpret_cast<const uint4*>(arow[j]);
    if (srow) sreg = srow[0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bcur[i] = *reinterpret_cast<const uint4*>(wrow[i]);
      wscur[i] = wsrow[i][0];
    }
#pragma unroll
    for (int j = 0; j < ALOADS; ++j)
      if (lrow[j] < BM) *reinterpret_cast<uint4*>(&As[0][lrow[j] * LDA + lpart[j] * 16]) = areg[j];
    if (srow) Ss[0][threadIdx.x] = sreg;
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < KT) {
#pragma unroll
        for (int j = 0; j < ALOADS; ++j)
          if (lrow[j] < BM) areg[j] = *reinterpret_cast<const uint4*>(arow[j] + (kt + 1) * 128);
        if (srow) sreg = srow[kt + 1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bnext[i] = *reinterpret_cast<const uint4*>(wrow[i] + (kt + 1) * 64);
          wsnext[i] = wsrow[i][(kt + 1) * 4];
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint8_t* ar = &As[buf][(m * 16 + ln) * LDA];
        const uint4 lo = *reinterpret_cast<const uint4*>(ar + lg * 16);
        const uint4 hi = *reinterpret_cast<const uint4*>(ar + 64 + lg * 16);
        const i32x8 af = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        const int sa = (int)((Ss[buf][m * 16 + ln] >> (8 * lg)) & 0xFFu);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const i32x4 bv = {(int)bcur[i].x, (int)bcur[i].y, (int)bcur[i].z, (int)bcur[i].w};
          acc[m][i] = mfma_fp8_fp4_scaled_16x16x128(af, bv, sa, wscur[i], acc[m][i]);
        }
      }
      if (kt + 1 < KT) {
#pragma unroll
        for (int j = 0; j < ALOADS; ++j)
          if (lrow[j] < BM) *reinterpret_cast<uint4*>(&As[buf ^ 1][lrow[j] * LDA + lpart[j] * 16]) = areg[j];
        if (srow) Ss[buf ^ 1][threadIdx.x] = sreg;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bcur[i] = bnext[i];
          wscur[i] = wsnext[i];
        }
      }
      __syncthreads();
    }

    if (G1) {
      uint8_t* Hq = static_cast<uint8_t*>(p.out);
      uint8_t* He = static_cast<uint8_t*>(p.out_scale);
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float h0 = silu_f32(acc[m][0][i]) * acc[m][2][i];
          const float h1 = silu_f32(acc[m][1][i]) * acc[m][3][i];
          float am = fmaxf(fabsf(h0), fabsf(h1));
          am = fmaxf(am, shfl_xor(am, 1));
          am = fmaxf(am, shfl_xor(am, 2));
          am = fmaxf(am, shfl_xor(am, 4));
          am = fmaxf(am, shfl_xor(am, 8));
          int X = 0;
          if (am > 0.0f) {
            X = (int)floor_log2_pos_mx(am) - 8;
            X = X < -127 ? -127 : (X > 127 ? 127 : X);
          }
          const float mul = (-X >= -126) ? __uint_as_float((uint32_t)(-X + 127) << 23) : __uint_as_float(0x00400000u);
          const int row = m * 16 + lg * 4 + i;
          if (row < tl.nrows) {
            const uint32_t c2 = cvt_e4m3x2(h0 * mul, h1 * mul);
            uint8_t* dst = Hq + (int64_t)(tl.rbase + row) * p.inter;
            dst[col[0] + ln] = (uint8_t)(c2 & 0xFF);
            dst[col[1] + ln] = (uint8_t)(c2 >> 8);
            if (ln == 0) He[(int64_t)(tl.rbase + row) * (p.inter / 32) + col[0] / 32] = (uint8_t)(X + 127);
          }
        }
    } else {
      uint16_t* Y = static_cast<uint16_t*>(p.out);
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = m * 16 + lg * 4 + i;
          if (row < tl.nrows) {
#pragma unroll
            for (int n = 0; n < 4; ++n)
              Y[(int64_t)(tl.rbase + row) * p.N + col[n] + ln] = (uint16_t)f32_to_bf16_bits(acc[m][n][i]);
          }
        }
    }
  }
}

template <bool G1>
static void launch_bm(const GemmArgs& a, int bm, int grid, hipStream_t s) {
  switch (bm) {
    case 16: hipLaunchKernelGGL((k_gemm_mxfp4<16, G1>), dim3(grid), dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((k_gemm_mxfp4<32, G1>), dim3(grid), dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((k_gemm_mxfp4<64, G1>), dim3(grid), dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((k_gemm_mxfp4<128, G1>), dim3(grid), dim3(256), 0, s, a); break;
  }
}

void launch_gemm_mxfp4(const GemmArgs& a, bool gemm1, int bm, int grid, hipStream_t s) {
  if (gemm1) launch_bm<true>(a, bm, grid, s);
  else launch_bm<false>(a, bm, grid, s);
}

}  // namespace moe
