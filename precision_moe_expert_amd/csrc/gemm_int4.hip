// Grouped expert GEMMs for INT4 group-32 weights on gfx950.
//
// Dequantization (Orbit announcement, 技术细节: the active experts' weights
// are dequantized temporarily for the grouped GEMM) happens in registers:
// each lane unpacks its own 32 nibbles per 128-K step and multiplies by the
// group's scale in fp16.  Every INT4 code times a bf16 group scale is exact
// in fp16 (at most 3 + 8 significant bits), so the MFMA sees w = q*s exactly;
// nothing is written back to memory and no dequantized copy exists.
//
// Tile: BM rows x 256 output columns per workgroup (4 waves x 4 subtiles of
// 16 columns); K step 128.  A (fp16 activations) is staged through a
// double-buffered LDS tile shared by the 4 waves; B is read by each wave
// straight from HBM (every weight is used by exactly one wave).
// GEMM1 pairs gate column n with up column I + n inside the same wave and
// writes h = silu(gate) * up (fp16); GEMM2 writes y (bf16).
#include "common.h"
#include "kernels.h"
#include "moe_sched.h"

namespace moe {

// 8 INT4 codes (one dword, element i in bits 4i..4i+3) times scale s ->
// 8 fp16 values ordered (0,4),(1,5),(2,6),(3,7): (1024 + (q ^ 8)) as fp16
// bits 0x6400 | u, minus 1032, times s.
MOE_DEV f16x8 int4x8_to_f16(uint32_t w, f16x2 s2) {
  const uint32_t u = w ^ 0x88888888u;
  const f16x2 bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  f16x2 h[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t d = ((u >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
    h[j] = (__builtin_bit_cast(f16x2, d) + bias) * s2;
  }
  f16x8 r = {h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
  return r;
}

template <int BM, bool G1>
__global__ __launch_bounds__(256) void k_gemm_int4(GemmArgs p) {
  constexpr int MT = BM / 16;
  constexpr int LDA = 128 + 8;  // fp16 elements per LDS row (16-byte pad)
  constexpr int ALOADS = (BM * 16 + 255) / 256;
  __shared__ __align__(16) uint16_t As[2][BM * LDA];
  const int nblk = G1 ? p.inter / 128 : p.N / 256;
  ChunkWork cw;
  if (!chunk_work(p, nblk, cw)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ln = lane & 15, lg = lane >> 4;
  const int K = p.K, KT = K / 128;
  const uint16_t* A = static_cast<const uint16_t*>(p.a);

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
    const uint16_t* srow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wrow[i] = p.w + tl.e * p.w_expert_bytes + (int64_t)(col[i] + ln) * (K / 2) + lg * 16;
      srow[i] = static_cast<const uint16_t*>(p.w_scale) + tl.e * p.ws_expert_elems + (int64_t)(col[i] + ln) * (K / 32) + lg;
    }
    // loader: thread -> (row, 16-byte part) for each of its ALOADS rows
    const int lpart = threadIdx.x & 15;
    const uint16_t* arow[ALOADS];
    int lrow[ALOADS];
#pragma unroll
    for (int j = 0; j < ALOADS; ++j) {
      lrow[j] = (threadIdx.x >> 4) + 16 * j;
      const int rr = tl.rbase + min(lrow[j], tl.nrows - 1);
      const int src = p.a_per_token ? p.sorted_rows[rr] / p.top_k : rr;
      arow[j] = A + (int64_t)src * K + lpart * 8;
    }
    f32x4 acc[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[m][i] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

    uint4 areg[ALOADS];
    uint4 bcur[4], bnext[4];
    uint16_t scur[4], snext[4];
#pragma unroll
    for (int j = 0; j < ALOADS; ++j)
      if (lrow[j] < BM) areg[j] = *reinterpret_cast<const uint4*>(arow[j]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bcur[i] = *reinterpret_cast<const uint4*>(wrow[i]);
      scur[i] = srow[i][0];
    }
#pragma unroll
    for (int j = 0; j < ALOADS; ++j)
      if (lrow[j] < BM) *reinterpret_cast<uint4*>(&As[0][lrow[j] * LDA + lpart * 8]) = areg[j];
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < KT) {
#pragma unroll
        for (int j = 0; j < ALOADS; ++j)
          if (lrow[j] < BM) areg[j] = *reinterpret_cast<const uint4*>(arow[j] + (kt + 1) * 128);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bnext[i] = *reinterpret_cast<const uint4*>(wrow[i] + (kt + 1) * 64);
          snext[i] = srow[i][(kt + 1) * 4];
        }
      }
      f16x2 s2[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const _Float16 sh = (_Float16)bf16_bits_to_f32(scur[i]);
        s2[i] = (f16x2){sh, sh};
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        f16x8 bf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t wv = s == 0 ? bcur[i].x : s == 1 ? bcur[i].y : s == 2 ? bcur[i].z : bcur[i].w;
          bf[i] = int4x8_to_f16(wv, s2[i]);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const f16x8 af = *reinterpret_cast<const f16x8*>(&As[buf][(m * 16 + ln) * LDA + lg * 32 + s * 8]);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[m][i] = mfma_f16_16x16x32(af, bf[i], acc[m][i]);
        }
      }
      if (kt + 1 < KT) {
#pragma unroll
        for (int j = 0; j < ALOADS; ++j)
          if (lrow[j] < BM) *reinterpret_cast<uint4*>(&As[buf ^ 1][lrow[j] * LDA + lpart * 8]) = areg[j];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bcur[i] = bnext[i];
          scur[i] = snext[i];
        }
      }
      __syncthreads();
    }

    if (G1) {
      uint16_t* H = static_cast<uint16_t*>(p.out);
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = m * 16 + lg * 4 + i;
          if (row < tl.nrows) {
#pragma unroll
            for (int n = 0; n < 2; ++n) {
              const float hv = silu_f32(acc[m][n][i]) * acc[m][n + 2][i];
              const _Float16 hh = (_Float16)hv;
              H[(int64_t)(tl.rbase + row) * p.inter + i4act_pos(col[n] + ln)] = __builtin_bit_cast(uint16_t, hh);
            }
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
    case 16: hipLaunchKernelGGL((k_gemm_int4<16, G1>), dim3(grid), dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((k_gemm_int4<32, G1>), dim3(grid), dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((k_gemm_int4<64, G1>), dim3(grid), dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((k_gemm_int4<128, G1>), dim3(grid), dim3(256), 0, s, a); break;
  }
}

void launch_gemm_int4(const GemmArgs& a, bool gemm1, int bm, int grid, hipStream_t s) {
  if (gemm1) launch_bm<true>(a, bm, grid, s);
  else launch_bm<false>(a, bm, grid, s);
}

}  // namespace moe
