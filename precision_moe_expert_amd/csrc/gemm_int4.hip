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
// straight from HBM (every weight is used by exactly one wave) through a
// three-slot register ring, two K steps ahead of its use.  The unpack costs
// about 2.5 vector ops per weight, so the tile is as tall as the rows per
// expert allow (up to 192) to keep it under the MFMA time.
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

MOE_DEV uint32_t dword_of(const u32x4& v, int s) { return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w; }

template <int BM, bool G1>
__global__ __launch_bounds__(256, (BM <= 96 ? 2 : 1)) void k_gemm_int4(GemmArgs p) {
  constexpr int MT = BM / 16;
  // register prefetch ring: weights and activation rows of step kt + RING - 1
  // are issued while step kt computes (deep for short tiles, whose per-step
  // compute is too short to cover a memory round trip, shallow where
  // registers are scarce)
  constexpr int RING = (BM <= 16 ? 6 : BM <= 32 ? 4 : BM <= 48 ? 3 : BM <= 96 ? 2 : 3);  // deepest ring that fits without spills
  constexpr int LDA = 128 + 8;  // fp16 elements per LDS row (16-byte pad)
  __shared__ __align__(16) uint16_t As[2][BM * LDA];
  const int nblk = G1 ? p.inter / 128 : p.N / 256;
  ChunkWork cw;
  if (!chunk_work(p, nblk, cw)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ln = lane & 15, lg = lane >> 4;
  const int K = p.K, KT = K / 128;
  const char* Abase = static_cast<const char*>(p.a);
  const int lpart = threadIdx.x & 15;

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
    // B: per-expert base (uniform) + 32-bit per-lane offsets
    const uint8_t* wexp = p.w + tl.e * p.w_expert_bytes;
    const uint16_t* sexp = static_cast<const uint16_t*>(p.w_scale) + tl.e * p.ws_expert_elems;
    uint32_t woff[4], soff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      woff[i] = (uint32_t)(col[i] + ln) * (uint32_t)(K / 2) + lg * 16;
      soff[i] = (uint32_t)(col[i] + ln) * (uint32_t)(K / 32) + lg;
    }
    // A: thread copies 16-byte part `lpart` of rows (tid/16) + 16j
    uint32_t aoff[MT];
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int rr = tl.rbase + min((int)(threadIdx.x >> 4) + 16 * j, tl.nrows - 1);
      const int src = p.a_per_token ? p.sorted_rows[rr] / p.top_k : rr;
      aoff[j] = (uint32_t)src * (uint32_t)(K * 2) + lpart * 16;
    }
    f32x4 acc[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[m][i] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

    auto loadB = [&](int kt, u32x4 (&b)[4], uint16_t (&s)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        b[i] = *reinterpret_cast<const u32x4*>(wexp + woff[i] + kt * 64);
        s[i] = sexp[soff[i] + kt * 4];
      }
    };
    auto loadA = [&](int kt, u32x4 (&areg)[MT]) {
#pragma unroll
      for (int j = 0; j < MT; ++j) areg[j] = *reinterpret_cast<const u32x4*>(Abase + aoff[j] + kt * 256);
    };
    auto storeA = [&](int buf, const u32x4 (&areg)[MT]) {
#pragma unroll
      for (int j = 0; j < MT; ++j)
        *reinterpret_cast<u32x4*>(&As[buf][((threadIdx.x >> 4) + 16 * j) * LDA + lpart * 8]) = areg[j];
    };
    // one K step: prefetch B(kt+2) into bl and A(kt+1) into registers,
    // compute with B(kt) in bc and A(kt) in LDS, then publish A(kt+1)
    auto step = [&](int kt, const u32x4 (&bc)[4], const uint16_t (&sc)[4], u32x4 (&bl)[4], uint16_t (&sl)[4], const u32x4 (&acur)[MT], u32x4 (&al)[MT]) {
      // prefetch target, clamped so that every step issues the same loads: the
      // compiler can then wait for exactly the loads a step needs instead of
      // draining all of them
      const int kpre = min(kt + RING - 1, KT - 1);
      loadA(kpre, al);
      // A must be issued before B: the vector-memory counter
      // completes in order, so waiting for A would otherwise also wait for B
      __builtin_amdgcn_sched_barrier(0);
      loadB(kpre, bl, sl);
      // keep the prefetches here: the scheduler would otherwise sink them
      // next to their first use and expose the full memory latency
      __builtin_amdgcn_sched_barrier(0);
      const int buf = kt & 1;
      f16x2 s2[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const _Float16 sh = (_Float16)bf16_bits_to_f32(sc[i]);
        s2[i] = (f16x2){sh, sh};
      }
      const uint16_t* arow = &As[buf][ln * LDA + lg * 32];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        f16x8 bf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) bf[i] = int4x8_to_f16(dword_of(bc[i], s), s2[i]);
        // A fragments are read two m-subtiles ahead of their MFMAs
        f16x8 af[3];
        af[0] = *reinterpret_cast<const f16x8*>(arow + s * 8);
        if (MT > 1) af[1] = *reinterpret_cast<const f16x8*>(arow + 16 * LDA + s * 8);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m + 2 < MT) af[(m + 2) % 3] = *reinterpret_cast<const f16x8*>(arow + (m + 2) * 16 * LDA + s * 8);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[m][i] = mfma_f16_16x16x32(af[m % 3], bf[i], acc[m][i]);
        }
      }
      if (kt + 1 < KT) storeA(buf ^ 1, acur);
      lds_barrier();
    };

    u32x4 bq[RING][4];
    uint16_t wq[RING][4];
    u32x4 aq[RING][MT];
    // prologue: steps 0 .. RING-2 in flight, step 0's activation tile in LDS
#pragma unroll
    for (int r = 0; r + 1 < RING; ++r) {
      loadA(min(r, KT - 1), aq[r]);
      loadB(min(r, KT - 1), bq[r], wq[r]);
    }
    storeA(0, aq[0]);
    lds_barrier();
    for (int kt = 0; kt < KT; kt += RING) {
#pragma unroll
      for (int r = 0; r < RING; ++r)
        if (kt + r < KT)
          step(kt + r, bq[r], wq[r], bq[(r + RING - 1) % RING], wq[(r + RING - 1) % RING], aq[(r + 1) % RING],
               aq[(r + RING - 1) % RING]);
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
    case 16: launch_persistent<k_gemm_int4<16, G1>>(a, grid, s); break;
    case 32: launch_persistent<k_gemm_int4<32, G1>>(a, grid, s); break;
    case 64: launch_persistent<k_gemm_int4<64, G1>>(a, grid, s); break;
    case 48: launch_persistent<k_gemm_int4<48, G1>>(a, grid, s); break;
    case 96: launch_persistent<k_gemm_int4<96, G1>>(a, grid, s); break;
    case 128: launch_persistent<k_gemm_int4<128, G1>>(a, grid, s); break;
    default: launch_persistent<k_gemm_int4<192, G1>>(a, grid, s); break;
  }
}

void launch_gemm_int4(const GemmArgs& a, bool gemm1, int bm, int grid, hipStream_t s) {
  if (gemm1) launch_bm<true>(a, bm, grid, s);
  else launch_bm<false>(a, bm, grid, s);
}

}  // namespace moe
