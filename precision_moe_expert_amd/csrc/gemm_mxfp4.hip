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
__global__ __launch_bounds__(256, (BM <= 96 ? 2 : 1)) void k_gemm_mxfp4(GemmArgs p) {
  constexpr int MT = BM / 16;
  // register prefetch ring: weights and activation rows of step kt + RING - 1
  // are issued while step kt computes (deep for short tiles, whose per-step
  // compute is too short to cover a memory round trip, shallow where
  // registers are scarce)
  constexpr int RING = (BM <= 32 ? 6 : BM <= 64 ? 3 : BM <= 96 ? 2 : 3);  // deepest ring that fits without spills
  constexpr int LDA = 128 + 16;
  constexpr int NCHUNK = BM * 8;
  constexpr int ALOADS = (NCHUNK + 255) / 256;
  constexpr bool AFULL = NCHUNK % 256 == 0;  // every thread loads ALOADS pieces
  __shared__ __align__(16) uint8_t As[2][BM * LDA];
  __shared__ __align__(16) uint32_t Ss[2][BM];
  const int nblk = G1 ? p.inter / 128 : p.N / 256;
  ChunkWork cw;
  if (!chunk_work(p, nblk, cw)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ln = lane & 15, lg = lane >> 4;
  const int K = p.K, KT = K / 128;
  const char* Abase = static_cast<const char*>(p.a);
  const uint8_t* AS = static_cast<const uint8_t*>(p.a_scale);

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
    const uint8_t* wsexp = static_cast<const uint8_t*>(p.w_scale) + tl.e * p.ws_expert_elems;
    uint32_t woff[4], wsoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      woff[i] = (uint32_t)(col[i] + ln) * (uint32_t)(K / 2) + lg * 16;
      wsoff[i] = (uint32_t)(col[i] + ln) * (uint32_t)(K / 32) + lg;
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

    auto loadB = [&](int kt, u32x4 (&b)[4], int (&ws)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        b[i] = *reinterpret_cast<const u32x4*>(wexp + woff[i] + kt * 64);
        ws[i] = wsexp[wsoff[i] + kt * 4];
      }
    };
    auto loadA = [&](int kt, u32x4 (&areg)[ALOADS], uint32_t& sreg) {
#pragma unroll
      for (int j = 0; j < ALOADS; ++j)
        if (AFULL || lrow[j] < BM) areg[j] = *reinterpret_cast<const u32x4*>(Abase + aoff[j] + kt * 128);
      if (srow) sreg = srow[kt];
    };
    auto storeA = [&](int buf, const u32x4 (&areg)[ALOADS], uint32_t sreg) {
#pragma unroll
      for (int j = 0; j < ALOADS; ++j)
        if (AFULL || lrow[j] < BM) *reinterpret_cast<u32x4*>(&As[buf][lrow[j] * LDA + lpart[j] * 16]) = areg[j];
      if (srow) Ss[buf][threadIdx.x] = sreg;
    };
    auto step = [&](int kt, const u32x4 (&bc)[4], const int (&wc)[4], u32x4 (&bl)[4], int (&wl)[4], const u32x4 (&acur)[ALOADS], const uint32_t& scur, u32x4 (&al)[ALOADS], uint32_t& sl_a) {
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
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint8_t* ar = &As[buf][(m * 16 + ln) * LDA];
        const u32x4 lo = *reinterpret_cast<const u32x4*>(ar + lg * 16);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(ar + 64 + lg * 16);
        const i32x8 af = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        const int sa = (int)((Ss[buf][m * 16 + ln] >> (8 * lg)) & 0xFFu);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const i32x4 bv = {(int)bc[i].x, (int)bc[i].y, (int)bc[i].z, (int)bc[i].w};
          acc[m][i] = mfma_fp8_fp4_scaled_16x16x128(af, bv, sa, wc[i], acc[m][i]);
        }
      }
      if (kt + 1 < KT) storeA(buf ^ 1, acur, scur);
      lds_barrier();
    };

    u32x4 bq[RING][4];
    int wq[RING][4];
    u32x4 aq[RING][ALOADS];
    uint32_t sq[RING];
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
      uint8_t* Hq = static_cast<uint8_t*>(p.out);
      uint8_t* He = static_cast<uint8_t*>(p.out_scale);
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float h0 = silu_f32(acc[m][0][i]) * acc[m][2][i];
          const float h1 = silu_f32(acc[m][1][i]) * acc[m][3][i];
          float am = fmaxf(fabsf(h0), fabsf(h1));
          am = row16_max_nonneg(am);
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
    case 16: launch_persistent<k_gemm_mxfp4<16, G1>>(a, grid, s); break;
    case 32: launch_persistent<k_gemm_mxfp4<32, G1>>(a, grid, s); break;
    case 64: launch_persistent<k_gemm_mxfp4<64, G1>>(a, grid, s); break;
    case 48: launch_persistent<k_gemm_mxfp4<48, G1>>(a, grid, s); break;
    case 96: launch_persistent<k_gemm_mxfp4<96, G1>>(a, grid, s); break;
    case 128: launch_persistent<k_gemm_mxfp4<128, G1>>(a, grid, s); break;
    default: launch_persistent<k_gemm_mxfp4<192, G1>>(a, grid, s); break;
  }
}

void launch_gemm_mxfp4(const GemmArgs& a, bool gemm1, int bm, int grid, hipStream_t s) {
  if (gemm1) launch_bm<true>(a, bm, grid, s);
  else launch_bm<false>(a, bm, grid, s);
}

}  // namespace moe
