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
__global__ __launch_bounds__(256, (BM <= 96 ? 2 : 1)) void k_gemm_fp8(GemmArgs p) {
  constexpr int MT = BM / 16;
  // register prefetch ring: weights and activation rows of step kt + RING - 1
  // are issued while step kt computes (deep for short tiles, whose per-step
  // compute is too short to cover a memory round trip, shallow where
  // registers are scarce)
  constexpr int RING = (BM <= 16 ? 4 : BM <= 32 ? 3 : 2);  // deepest ring that fits without spills
  constexpr int LDA = 128 + 16;  // bytes per LDS row
  constexpr int NCHUNK = BM * 8;  // 16-byte pieces per A tile
  constexpr int ALOADS = (NCHUNK + 255) / 256;
  constexpr bool AFULL = NCHUNK % 256 == 0;  // every thread loads ALOADS pieces
  __shared__ __align__(16) uint8_t As[2][BM * LDA];
  __shared__ __align__(16) float Ss[2][BM];
  __shared__ float red[4][BM];
  const int nblk = G1 ? p.inter / 128 : p.N / 256;
  ChunkWork cw;
  if (!chunk_work(p, nblk, cw)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ln = lane & 15, lg = lane >> 4;
  const int K = p.K, KT = K / 128;
  const char* Abase = static_cast<const char*>(p.a);
  const float* AS = static_cast<const float*>(p.a_scale);

  for (int base = 0; base < cw.nwork; base += gridDim.x) {
    const int wk = xcd_item(base, cw.nwork);
    if (wk < 0) continue;
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
    const uint8_t* wexp = p.w + tl.e * p.w_expert_bytes;
    const float* wsexp = static_cast<const float*>(p.w_scale) + tl.e * p.ws_expert_elems;
    uint32_t woff[4], wsoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      woff[i] = (uint32_t)(col[i] + ln) * (uint32_t)K + lg * 32;
      wsoff[i] = (uint32_t)(col[i] / 128) * (uint32_t)KT;
    }
    uint32_t aoff[ALOADS];
    int lrow[ALOADS], lpart[ALOADS];
#pragma unroll
    for (int j = 0; j < ALOADS; ++j) {
      const int c = threadIdx.x + 256 * j;
      lrow[j] = c / 8;
      lpart[j] = c % 8;
      const int rr = tl.rbase + min(min(lrow[j], BM - 1), tl.nrows - 1);
      const int src = p.a_per_token ? p.sorted_rows[rr] / p.top_k : rr;
      aoff[j] = (uint32_t)src * (uint32_t)K + lpart[j] * 16;
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

    auto loadB = [&](int kt, u32x4 (&b)[4][2], float (&ws)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        b[i][0] = *reinterpret_cast<const u32x4*>(wexp + woff[i] + kt * 128);
        b[i][1] = *reinterpret_cast<const u32x4*>(wexp + woff[i] + kt * 128 + 16);
        ws[i] = wsexp[wsoff[i] + kt];
      }
    };
    auto loadA = [&](int kt, u32x4 (&areg)[ALOADS], float& sreg) {
#pragma unroll
      for (int j = 0; j < ALOADS; ++j)
        if (AFULL || lrow[j] < BM) areg[j] = *reinterpret_cast<const u32x4*>(Abase + aoff[j] + kt * 128);
      if (srow) sreg = srow[kt];
    };
    auto storeA = [&](int buf, const u32x4 (&areg)[ALOADS], float sreg) {
#pragma unroll
      for (int j = 0; j < ALOADS; ++j)
        if (AFULL || lrow[j] < BM) *reinterpret_cast<u32x4*>(&As[buf][lrow[j] * LDA + lpart[j] * 16]) = areg[j];
      if (srow) Ss[buf][threadIdx.x] = sreg;
    };
    auto step = [&](int kt, const u32x4 (&bc)[4][2], const float (&wc)[4], u32x4 (&bl)[4][2], float (&wl)[4], const u32x4 (&acur)[ALOADS], const float& scur, u32x4 (&al)[ALOADS], float& sl_a) {
      // prefetch target, clamped so that every step issues the same loads: the
      // compiler can then wait for exactly the loads a step needs instead of
      // draining all of them
      const int kpre = min(kt + RING - 1, KT - 1);
      loadA(kpre, al, sl_a);
      // A must be issued before B: the vector-memory counter
      // completes in order, so waiting for A would otherwise also wait for B
      __builtin_amdgcn_sched_barrier(0);
      loadB(kpre, bl, wl);
      // keep the prefetches here: the scheduler would otherwise sink them
      // next to their first use and expose the full memory latency
      __builtin_amdgcn_sched_barrier(0);
      const int buf = kt & 1;
      i32x8 bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        bf[i] = (i32x8){(int)bc[i][0].x, (int)bc[i][0].y, (int)bc[i][0].z, (int)bc[i][0].w,
                        (int)bc[i][1].x, (int)bc[i][1].y, (int)bc[i][1].z, (int)bc[i][1].w};
      const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const i32x8 af = *reinterpret_cast<const i32x8*>(&As[buf][(m * 16 + ln) * LDA + lg * 32]);
        const f32x4 sa = *reinterpret_cast<const f32x4*>(&Ss[buf][m * 16 + lg * 4]);
        // subtiles 0,1 share one weight-scale block and 2,3 another (GEMM1: gate, up)
        f32x4 sc01, sc23;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          sc01[q] = sa[q] * wc[0];
          sc23[q] = sa[q] * wc[2];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 part = mfma_fp8_16x16x128(af, bf[i], zero);
          const f32x4& sc = i < 2 ? sc01 : sc23;
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[m][i][q] = fmaf(part[q], sc[q], acc[m][i][q]);
        }
      }
      if (kt + 1 < KT) storeA(buf ^ 1, acur, scur);
      lds_barrier();
    };

    u32x4 bq[RING][4][2];
    float wq[RING][4];
    u32x4 aq[RING][ALOADS];
    float sq[RING];
#pragma unroll
    for (int r = 0; r < RING; ++r) sq[r] = 0;
    // prologue: steps 0 .. RING-2 in flight, step 0's activation tile in LDS
#pragma unroll
    for (int r = 0; r + 1 < RING; ++r) {
      loadA(min(r, KT - 1), aq[r], sq[r]);
      loadB(min(r, KT - 1), bq[r], wq[r]);
    }
    storeA(0, aq[0], sq[0]);
    lds_barrier();
    for (int kt = 0; kt < KT; kt += RING) {
#pragma unroll
      for (int r = 0; r < RING; ++r) {
        if (kt + r < KT)
          step(kt + r, bq[r], wq[r], bq[(r + RING - 1) % RING], wq[(r + RING - 1) % RING], aq[(r + 1) % RING],
               sq[(r + 1) % RING], aq[(r + RING - 1) % RING], sq[(r + RING - 1) % RING]);
      }
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
    case 48: hipLaunchKernelGGL((k_gemm_fp8<48, G1>), dim3(grid), dim3(256), 0, s, a); break;
    case 96: hipLaunchKernelGGL((k_gemm_fp8<96, G1>), dim3(grid), dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL((k_gemm_fp8<128, G1>), dim3(grid), dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((k_gemm_fp8<192, G1>), dim3(grid), dim3(256), 0, s, a); break;
  }
}

void launch_gemm_fp8(const GemmArgs& a, bool gemm1, int bm, int grid, hipStream_t s) {
  if (gemm1) launch_bm<true>(a, bm, grid, s);
  else launch_bm<false>(a, bm, grid, s);
}

}  // namespace moe
