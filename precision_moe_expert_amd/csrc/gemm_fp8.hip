// Grouped expert GEMMs for FP8 E4M3 weights with [128,128] fp32 block scales
// and FP8 [1,128] activations (NeMo RL FP8 post, Table 1).
//
// One 16x16x128 E4M3 MFMA covers exactly one 128-wide K block, so each MFMA
// result is an unscaled partial for (row, column, K block); it is rescaled by
// a_scale[row][kb] * w_scale[n/128][kb] and added to the fp32 accumulator.
// GEMM1's epilogue forms h = silu(gate) * up and quantizes it to FP8 with a
// [1,128] scale: the workgroup's 128 h columns are one scale block, so the
// row maximum is reduced across the 4 waves through LDS.
#include "common.h"
#include "kernels.h"
#include "moe_sched.h"

namespace moe {

template <int BM, bool G1>
__global__ __launch_bounds__(256) void k_gemm_fp8(GemmArgs p) {
  constexpr int MT = BM / 16;
  constexpr int LDA = 128 + 16;  // bytes per LDS row
  constexpr int NCHUNK = BM * 8;  // 16-byte pieces per A tile
  constexpr int ALOADS = (NCHUNK + 255) / 256;
  __shared__ __align__(16) uint8_t As[2][BM * LDA];
  __shared__ __align__(16) float Ss[2][BM];
  __shared__ float red[4][BM];
  const int nblk = G1 ? p.inter / 128 : p.N / 256;
  ChunkWork cw;
  if (!chunk_work(p, nblk, cw)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ln = lane & 15, lg = lane >> 4;
  const int K = p.K, KT = K / 128;
  const uint8_t* A = static_cast<const uint8_t*>(p.a);
  const float* AS = static_cast<const float*>(p.a_scale);
  const float* WS = static_cast<const float*>(p.w_scale);

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
    const float* wsrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wrow[i] = p.w + tl.e * p.w_expert_bytes + (int64_t)(col[i] + ln) * K + lg * 32;
      wsrow[i] = WS + tl.e * p.ws_expert_elems + (int64_t)(col[i] / 128) * KT;
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
    const float* srow = nullptr;
    if (threadIdx.x < BM) {
      const int rr = tl.rbase + min((int)threadIdx.x, tl.nrows - 1);
      const int src = p.a_per_token ? p.sorted_rows[rr] / p.top_k : rr;
      srow = AS + (int64_t)src * KT;
    }
    f32x4 acc[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[m][i] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

    uint4 areg[ALOADS];
    float sreg = 0.0f;
    uint4 bcur[4][2], bnext[4][2];
    float wscur[4], wsnext[4];
#pragma unroll
    for (int j = 0; j < ALOADS; ++j)
      if (lrow[j] < BM) areg[j] = *reinterpret_cast<const uint4*>(arow[j]);
    if (srow) sreg = srow[0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bcur[i][0] = *reinterpret_cast<const uint4*>(wrow[i]);
      bcur[i][1] = *reinterpret_cast<const uint4*>(wrow[i] + 16);
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
          bnext[i][0] = *reinterpret_cast<const uint4*>(wrow[i] + (kt + 1) * 128);
          bnext[i][1] = *reinterpret_cast<const uint4*>(wrow[i] + (kt + 1) * 128 + 16);
          wsnext[i] = wsrow[i][kt + 1];
        }
      }
      i32x8 bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        bf[i] = (i32x8){(int)bcur[i][0].x, (int)bcur[i][0].y, (int)bcur[i][0].z, (int)bcur[i][0].w,
                        (int)bcur[i][1].x, (int)bcur[i][1].y, (int)bcur[i][1].z, (int)bcur[i][1].w};
      const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const i32x8 af = *reinterpret_cast<const i32x8*>(&As[buf][(m * 16 + ln) * LDA + lg * 32]);
        const f32x4 sa = *reinterpret_cast<const f32x4*>(&Ss[buf][m * 16 + lg * 4]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 part = mfma_fp8_16x16x128(af, bf[i], zero);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[m][i][q] = fmaf(part[q], sa[q] * wscur[i], acc[m][i][q]);
        }
      }
      if (kt + 1 < KT) {
#pragma unroll
        for (int j = 0; j < ALOADS; ++j)
          if (lrow[j] < BM) *reinterpret_cast<uint4*>(&As[buf ^ 1][lrow[j] * LDA + lpart[j] * 16]) = areg[j];
        if (srow) Ss[buf ^ 1][threadIdx.x] = sreg;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bcur[i][0] = bnext[i][0];
          bcur[i][1] = bnext[i][1];
          wscur[i] = wsnext[i];
        }
      }
      __syncthreads();
    }

    if (G1) {
      float hv[MT][4][2];
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float am = 0.0f;
#pragma unroll
          for (int n = 0; n < 2; ++n) {
            hv[m][i][n] = silu_f32(acc[m][n][i]) * acc[m][n + 2][i];
            am = fmaxf(am, fabsf(hv[m][i][n]));
          }
          am = fmaxf(am, shfl_xor(am, 1));
          am = fmaxf(am, shfl_xor(am, 2));
          am = fmaxf(am, shfl_xor(am, 4));
          am = fmaxf(am, shfl_xor(am, 8));
          if (ln == 0) red[wave][m * 16 + lg * 4 + i] = am;
        }
      __syncthreads();
      uint8_t* Hq = static_cast<uint8_t*>(p.out);
      float* Hs = static_cast<float*>(p.out_scale);
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = m * 16 + lg * 4 + i;
          const float amax = fmaxf(fmaxf(red[0][row], red[1][row]), fmaxf(red[2][row], red[3][row]));
          const float s = amax == 0.0f ? 1.0f : amax / 448.0f;
          if (row < tl.nrows) {
            const uint32_t c2 = cvt_e4m3x2(hv[m][i][0] / s, hv[m][i][1] / s);
            uint8_t* dst = Hq + (int64_t)(tl.rbase + row) * p.inter;
            dst[col[0] + ln] = (uint8_t)(c2 & 0xFF);
            dst[col[1] + ln] = (uint8_t)(c2 >> 8);
            if (wave == 0 && ln == 0) Hs[(int64_t)(tl.rbase + row) * (p.inter / 128) + tl.nb] = s;
          }
        }
      __syncthreads();
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
    case 16: hipLaunchKernelGGL((k_gemm_fp8<16, G1>), dim3(grid), dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((k_gemm_fp8<32, G1>), dim3(grid), dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((k_gemm_fp8<64, G1>), dim3(grid), dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((k_gemm_fp8<128, G1>), dim3(grid), dim3(256), 0, s, a); break;
  }
}

void launch_gemm_fp8(const GemmArgs& a, bool gemm1, int bm, int grid, hipStream_t s) {
  if (gemm1) launch_bm<true>(a, bm, grid, s);
  else launch_bm<false>(a, bm, grid, s);
}

}  // namespace moe
