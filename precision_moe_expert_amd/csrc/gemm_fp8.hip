// Grouped expert GEMMs for FP8 E4M3 weights with [128,128] fp32 block scales
// and FP8 [1,128] activations (NeMo RL FP8 post, Table 1).
//
// One 16x16x128 E4M3 MFMA covers exactly one 128-wide K block, so each MFMA
// result is an unscaled partial for (row, column, K block); it is rescaled by
// a_scale[row][kb] * w_scale[n/128][kb] and added to the fp32 accumulator.
// GEMM1's epilogue forms h = silu(gate) * up and quantizes it to FP8 with a
// [1,128] scale: the workgroup's 128 h columns are one scale block, so the
// row maximum is reduced across the column waves through LDS.
//
// Power-of-two scales (the recipe's pow2 switches) instead go into the
// block-scaled MFMA as E8M0 exponents: no VALU rescale at all.
//
// Workgroup: 8 waves, two per SIMD.  Wave (wr, wc) computes the 64 output
// columns of column group wc for half wr of the tile's row blocks; the two
// waves of a SIMD share their weight fragments in LDS, and while one waits
// on LDS or a barrier the other keeps the matrix core and the VALU busy
// (the per-block rescale costs 6 VALU instructions per MFMA).
#include "common.h"
#include "kernels.h"
#include "moe_sched.h"

namespace moe {

constexpr int FP8_THREADS = 512;

// LDS bytes of one pipeline stage: activation rows (128 B each, whole DMA
// groups of 8 rows per wave) and the weight rows (4 column groups x 64 rows
// x 128 B, each group loaded half by each of its two waves).
template <int BM>
struct Fp8Stage {
  static constexpr int NA = (BM * 8 + 511) / 512;  // activation DMA groups per wave
  static constexpr int A_BYTES = NA * 8 * 1024;
  static constexpr int B_OFF = A_BYTES;
  static constexpr int BYTES = B_OFF + 4 * 8 * 1024;
  static constexpr int S = (152 * 1024) / BYTES > 4 ? 4 : (152 * 1024) / BYTES;  // stages
  static constexpr int NPER = NA + 4;               // DMA instructions per wave per stage
  static constexpr int MT = BM / 16;                // row blocks of the tile
  static constexpr int MTW = (MT + 1) / 2;          // row blocks per wave (row group 0 takes the extra one)
  // Activation scales travel in blocks of 4 K steps (16 B per row, one
  // aligned piece of the padded scale row), double-buffered outside the
  // ring: waves 0..NASW-1 load 64 rows each with every 4th stage.
  static constexpr int NASW = (BM + 63) / 64;
  static constexpr int AS_BLOCK = NASW * 64 * 16;
};

// One work item: a BM-row tile times one N block (GEMM1: 128 h columns, i.e.
// 128 gate + 128 up weight rows; GEMM2: 256 output columns).
template <int BM, bool G1, bool P2>
__device__ __forceinline__ void fp8_item(const GemmArgs& p, const Tile& tl, uint8_t* smem, uint8_t* asb,
                                         float (*red)[BM]) {
  using ST = Fp8Stage<BM>;
  constexpr int S = ST::S, MT = ST::MT, MTW = ST::MTW;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wc = wave & 3, wr = wave >> 2;
  const int ln = lane & 15, lg = lane >> 4;
  const int mb0 = wr * MTW;                       // first row block of this wave
  // row blocks of this wave (wave-uniform); compile-time whenever the tile
  // splits evenly, so the row-block loop unrolls without branches
  const int nmb = (MT % 2 == 0) ? MTW : min(MTW, MT - mb0);
  const int K = p.K, KT = K / 128;
  const char* Abase = static_cast<const char*>(p.a);
  const char* ASbase = static_cast<const char*>(p.a_scale);
  const float* WS = static_cast<const float*>(p.w_scale);
  const uint32_t smem0 = lds_u32(smem), asb0 = lds_u32(asb);
  lds_barrier();  // every wave is done with the previous item's stages
  int col[4];
  if (G1) {
    const int g0 = tl.nb * 128 + wc * 32;
    col[0] = g0; col[1] = g0 + 16; col[2] = p.inter + g0; col[3] = p.inter + g0 + 16;
  } else {
    const int c0 = tl.nb * 256 + wc * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) col[i] = c0 + 16 * i;
  }
  // per-lane global sources of this item's DMA pieces (K offset added per step)
  const char* wexp = reinterpret_cast<const char*>(p.w) + tl.e * p.w_expert_bytes;
  const float* wsexp = WS + tl.e * p.ws_expert_elems;
  // Weight rows go to LDS as whole 128-byte lines (8 lanes per row, so every
  // request is a full line), 16-byte parts XOR-swizzled by row as for the
  // activations: column group wc's 64 rows take 8 DMAs, 4 from each of its
  // two waves.  Local row r < 32 is gate/first-half row col[0] + r, r >= 32
  // is col[2] + r - 32 (GEMM2: col[0] + r).
  const char* bsrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = (wr * 4 + j) * 64 + lane;
    const int r = c >> 3, part = (c & 7) ^ (r & 7);
    const int n = G1 ? (r < 32 ? col[0] + r : col[2] + r - 32) : col[0] + r;
    bsrc[j] = p.w_kblocked ? wexp + (int64_t)(n / 16) * (K / 128) * 2048 + (n % 16) * 128 + part * 16
                           : wexp + (int64_t)n * K + part * 16;
  }
  const int bstep = p.w_kblocked ? 2048 : 128;  // bytes between K steps of one lane's piece
  const char* asrc[ST::NA];
#pragma unroll
  for (int j = 0; j < ST::NA; ++j) {
    const int c = (wave * ST::NA + j) * 64 + lane;   // activation piece: row c/8, slot c%8
    const int row = c >> 3, slot = c & 7;
    const int part = slot ^ (row & 7);               // XOR swizzle of 16-byte parts
    const int rr = tl.rbase + min(min(row, BM - 1), tl.nrows - 1);
    const int sr = p.sorted_rows[rr];
    const int src = p.a_per_token ? sr / p.top_k : rr;
    asrc[j] = Abase + (int64_t)src * K + part * 16;
  }
  const char* ssrc;
  {
    const int row = wave * 64 + lane;
    const int rr = tl.rbase + min(min(row, BM - 1), tl.nrows - 1);
    const int sr = p.sorted_rows[rr];
    const int src = p.a_per_token ? sr / p.top_k : rr;
    ssrc = ASbase + (int64_t)src * p.a_scale_stride;
  }
  auto issue = [&](int kt, int slot) {
    const uint32_t sb = smem0 + slot * ST::BYTES;
#pragma unroll
    for (int j = 0; j < ST::NA; ++j) dma_b128(asrc[j] + kt * 128, sb + (wave * ST::NA + j) * 1024);
    if (wave < ST::NASW && (kt & 3) == 0)
      dma_b128(ssrc + (kt >> 2) * 16, asb0 + ((kt >> 2) & 1) * ST::AS_BLOCK + wave * 1024);
#pragma unroll
    for (int j = 0; j < 4; ++j) dma_b128(bsrc[j] + kt * bstep, sb + ST::B_OFF + (wc * 8 + wr * 4 + j) * 1024);
  };
  f32x4 acc[MTW][4];
#pragma unroll
  for (int m = 0; m < MTW; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[m][i] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
  for (int s = 0; s + 1 < S; ++s)
    if (s < KT) issue(s, s);
  const float* ws0 = wsexp + (col[0] / 128) * KT;
  const float* ws2 = wsexp + (col[2] / 128) * KT;
  float wnext[2] = {ld_uniform_f32(ws0), ld_uniform_f32(ws2)};
  for (int kt = 0; kt < KT; ++kt) {
    {
      // this wave's pieces of stage kt have landed (later stages in flight
      // hold one more load if a scale block starts among them)
      const int n = min(S - 2, KT - 1 - kt);
      wait_stages_x<ST::NPER>(n, (wave < ST::NASW && ((kt + n) >> 2) > (kt >> 2)) ? 1 : 0);
    }
    lds_barrier();                                    // ... and every other wave's
    if (kt + S - 1 < KT) issue(kt + S - 1, (kt + S - 1) % S);
    const float wc0 = wnext[0], wc2 = wnext[1];
    if (kt + 1 < KT) {
      wnext[0] = ld_uniform_f32(ws0 + kt + 1);
      wnext[1] = ld_uniform_f32(ws2 + kt + 1);
    }
    if (nmb == 0) continue;  // a 16-row tile leaves row group 1 without work
    __builtin_amdgcn_s_setprio(1);  // the MFMA phase at raised wave priority
    const uint8_t* st = smem + (kt % S) * ST::BYTES;
    const float* As = reinterpret_cast<const float*>(asb + ((kt >> 2) & 1) * ST::AS_BLOCK) + (kt & 3);
    i32x8 bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = i * 16 + ln;
      const uint8_t* brow = st + ST::B_OFF + wc * 8192 + r * 128;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(brow + ((lg ^ (r & 7)) << 4));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(brow + (((lg + 4) ^ (r & 7)) << 4));
      bf[i] = (i32x8){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    if constexpr (P2) {
      // power-of-two scales: the block-scaled MFMA applies 2^ea (the row's
      // activation scale) and 2^ew (the weight block's) exactly, so the
      // partials accumulate directly
      const int ew0 = e8m0_of_pow2(wc0), ew2 = e8m0_of_pow2(wc2);
      auto read_a2 = [&](int m, i32x8& af, int& ea) {
        const int r = (mb0 + m) * 16 + ln;
        const uint8_t* arow = st + r * 128;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(arow + ((lg ^ (r & 7)) << 4));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(arow + (((lg + 4) ^ (r & 7)) << 4));
        af = (i32x8){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        ea = e8m0_of_pow2(As[r * 4]);
      };
      // row block m + 1's operands are read while block m's MFMAs issue, one
      // LDS read between two MFMAs (as in the MXFP4 kernel)
      i32x8 af[2];
      int ea[2];
      read_a2(0, af[0], ea[0]);
#pragma unroll
      for (int m = 0; m < MTW; ++m)
        if (m < nmb) {
          __builtin_amdgcn_sched_barrier(0);
          if (m + 1 < nmb) read_a2(m + 1, af[(m + 1) & 1], ea[(m + 1) & 1]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[m][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[m & 1], bf[i], acc[m][i], 0, 0, 0,
                                                                          ea[m & 1], 0, i < 2 ? ew0 : ew2);
          if (m + 1 < nmb) {
#pragma unroll
            for (int j = 0; j < 3; ++j) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
    } else {
      const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
      auto read_a = [&](int m, i32x8& af, f32x4& sa) {
        const int r = (mb0 + m) * 16 + ln;
        const uint8_t* arow = st + r * 128;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(arow + ((lg ^ (r & 7)) << 4));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(arow + (((lg + 4) ^ (r & 7)) << 4));
        af = (i32x8){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        const int r0 = (mb0 + m) * 16 + lg * 4;
        sa = (f32x4){As[r0 * 4], As[(r0 + 1) * 4], As[(r0 + 2) * 4], As[(r0 + 3) * 4]};
      };
      // Software pipeline over row blocks: the MFMAs of block m run while the
      // VALU folds block m-1's partial products into the accumulators with
      // their (activation x weight) block scales.
      i32x8 afc;
      f32x4 sac;
      read_a(0, afc, sac);
      f32x4 prev[4], psc01, psc23;
#pragma unroll
      for (int m = 0; m < MTW; ++m) {
        if (m < nmb) {
          i32x8 afn;
          f32x4 san;
          if (m + 1 < nmb) read_a(m + 1, afn, san);
          // one MFMA of block m per group, with the VALU work of block m-1
          // (sched_barrier keeps the compiler from bunching the MFMAs, which
          // would leave the VALU work waiting behind them)
          f32x4 part[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            part[i] = mfma_fp8_16x16x128(afc, bf[i], zero);
            if (m > 0) {
#pragma unroll
              for (int q = 0; q < 4; ++q)
                acc[m - 1][i][q] = fmaf(prev[i][q], i < 2 ? psc01[q] : psc23[q], acc[m - 1][i][q]);
            }
            // subtiles 0,1 share one weight-scale block and 2,3 another (GEMM1: gate, up)
            if (i == 1) {
#pragma unroll
              for (int q = 0; q < 4; ++q) psc01[q] = sac[q] * wc0;
            }
            if (i == 3) {
#pragma unroll
              for (int q = 0; q < 4; ++q) psc23[q] = sac[q] * wc2;
            }
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) prev[i] = part[i];
          if (m + 1 < nmb) {
            afc = afn;
            sac = san;
          }
        }
      }
#pragma unroll
      for (int m = 0; m < MTW; ++m)
        if (m + 1 == nmb) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[m][i][q] = fmaf(prev[i][q], i < 2 ? psc01[q] : psc23[q], acc[m][i][q]);
        }
    }
    __builtin_amdgcn_s_setprio(0);
  }

  // Epilogue: results go through LDS (the stage buffers are free once every
  // wave has passed the barrier below) so that global stores are 16 B per lane.
  if (G1) {
    if (p.ab_out != nullptr) {
      // backward recompute: the gate and up pre-activations in fp32 as well
#pragma unroll
      for (int m = 0; m < MTW; ++m)
        if (m < nmb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = (mb0 + m) * 16 + lg * 4 + i;
            if (row < tl.nrows)
#pragma unroll
              for (int n = 0; n < 4; ++n) p.ab_out[(int64_t)(tl.rbase + row) * p.N + col[n] + ln] = acc[m][n][i];
          }
    }
    constexpr int HS = 144;  // staged row stride (bytes) of the 128 h codes
    float hv[MTW][4][2];
#pragma unroll
    for (int m = 0; m < MTW; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float am = 0.0f;
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          hv[m][i][n] = silu_f32(acc[m][n][i]) * acc[m][n + 2][i];
          am = fmaxf(am, fabsf(hv[m][i][n]));
        }
        am = row16_max_nonneg(am);
        if (m < nmb && ln == 0) red[wc][(mb0 + m) * 16 + lg * 4 + i] = am;
      }
    lds_barrier();
    // the four column waves' maxima of this lane's 4 rows per row block, all
    // read before the first is used (one 16-byte read per wave and block)
    f32x4 rmax[MTW][4];
#pragma unroll
    for (int m = 0; m < MTW; ++m)
      if (m < nmb)
#pragma unroll
        for (int c = 0; c < 4; ++c) rmax[m][c] = *reinterpret_cast<const f32x4*>(&red[c][(mb0 + m) * 16 + lg * 4]);
    float* Hs = static_cast<float*>(p.out_scale);
#pragma unroll
    for (int m = 0; m < MTW; ++m)
      if (m < nmb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = (mb0 + m) * 16 + lg * 4 + i;
          const float amax = fmaxf(fmaxf(rmax[m][0][i], rmax[m][1][i]), fmaxf(rmax[m][2][i], rmax[m][3][i]));
          // the row's [1,128] block scale: s = amax/448 with codes RNE(h/s), both
          // quotients correctly rounded (the activation quantizer's definition),
          // or the power of two at or above amax/448 (exact scaling)
          float sc;
          uint32_t c2;
          if constexpr (P2) {
            sc = amax == 0.0f ? 1.0f : pow2_at_least(amax / 448.0f);
            const float inv = pow2_reciprocal(sc);
            c2 = cvt_e4m3x2(hv[m][i][0] * inv, hv[m][i][1] * inv);
          } else {
            sc = amax == 0.0f ? 1.0f : amax / 448.0f;
            c2 = cvt_e4m3x2(hv[m][i][0] / sc, hv[m][i][1] / sc);
          }
          smem[row * HS + wc * 32 + ln] = (uint8_t)(c2 & 0xFF);
          smem[row * HS + wc * 32 + 16 + ln] = (uint8_t)(c2 >> 8);
          if (wc == 0 && ln == 0 && row < tl.nrows)
            Hs[(int64_t)(tl.rbase + row) * (p.out_scale_stride / 4) + tl.nb] = sc;
        }
      }
    lds_barrier();
    copy_out_rows<BM, 128, HS, FP8_THREADS>(smem, static_cast<char*>(p.out) + tl.nb * 128 + (int64_t)tl.rbase * p.inter,
                                            (int64_t)p.inter, tl.nrows);
  } else {
    constexpr int YS = 528;  // staged row stride (bytes) of the 256 bf16 outputs
    lds_barrier();
#pragma unroll
    for (int m = 0; m < MTW; ++m)
      if (m < nmb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = (mb0 + m) * 16 + lg * 4 + i;
#pragma unroll
          for (int n = 0; n < 4; ++n)
            *reinterpret_cast<uint16_t*>(smem + row * YS + (wc * 64 + n * 16 + ln) * 2) =
                (uint16_t)f32_to_bf16_bits(acc[m][n][i]);
        }
      }
    lds_barrier();
    copy_out_rows<BM, 512, YS, FP8_THREADS>(smem, static_cast<char*>(p.out) + (int64_t)tl.nb * 512 + (int64_t)tl.rbase * p.N * 2,
                                            (int64_t)p.N * 2, tl.nrows);
  }
}

// Persistent pair launch: the GEMM1 items of chunk p1.chunk and the GEMM2
// items of chunk p2.chunk (either may be empty: chunk < 0 or past the last
// active expert).  The two have no dependence on each other (GEMM2 of a chunk
// reads the h that the previous launch wrote), so one launch keeps every CU
// busy where two launches would each leave a partial last round.  Items are
// split into contiguous per-XCD ranges (neighbouring items share weights in
// that XCD's L2), GEMM1 items first; the workgroups of an XCD take items from
// its range through an atomic counter, so every workgroup exits once the
// range is used up.
template <int BM, bool P2>
__global__ __launch_bounds__(FP8_THREADS, 1) void k_gemm_fp8(GemmArgs p1, GemmArgs p2, int32_t* queue) {
  using ST = Fp8Stage<BM>;
  constexpr int S = ST::S;
  static_assert(S >= 2 && S <= 5, "LDS stages");
  __shared__ __align__(16) uint8_t smem[S * ST::BYTES];
  static_assert(S * ST::BYTES >= BM * 528, "epilogue staging fits in the stage buffers");
  __shared__ __align__(16) uint8_t asb[2 * ST::AS_BLOCK];
  __shared__ __align__(16) float red[4][BM];
  __shared__ int s_item;
  ChunkWork c1, c2;
  const int n1 = chunk_work(p1, p1.inter / 128, c1) ? c1.nwork : 0;
  const int n2 = chunk_work(p2, p2.N / 256, c2) ? c2.nwork : 0;
  const int x = blockIdx.x & 7;
  const int per1 = (n1 + 7) >> 3, per2 = (n2 + 7) >> 3;
  const int b1 = x * per1, b2 = x * per2;
  const int len1 = max(0, min(n1, b1 + per1) - b1), len2 = max(0, min(n2, b2 + per2) - b2);
  int32_t* q = queue + x;
  // the first item of each workgroup is its slot in the XCD; later ones come
  // from the counter (offset by the workgroups per XCD), so the launch does
  // not start with every workgroup contending for the same counter
  const int wpx = gridDim.x >> 3;
  int cur = blockIdx.x >> 3;
  while (cur < len1 + len2) {
    int nxt = 0;
    if (threadIdx.x == 0) nxt = atomicAdd(q, 1) + wpx;  // claimed now, read after the item
    if (cur < len1) fp8_item<BM, true, P2>(p1, tile_of(p1, c1, b1 + cur, BM), smem, asb, red);
    else fp8_item<BM, false, P2>(p2, tile_of(p2, c2, b2 + cur - len1, BM), smem, asb, red);
    if (threadIdx.x == 0) s_item = nxt;
    lds_barrier();
    cur = s_item;
  }
}

template <bool P2>
static void launch_fp8(const GemmArgs& g1, const GemmArgs& g2, int32_t* queue, int bm, int grid, hipStream_t s) {
  switch (bm) {
    case 16: launch_persistent2<k_gemm_fp8<16, P2>, FP8_THREADS>(g1, g2, queue, grid, s); break;
    case 32: launch_persistent2<k_gemm_fp8<32, P2>, FP8_THREADS>(g1, g2, queue, grid, s); break;
    case 64: launch_persistent2<k_gemm_fp8<64, P2>, FP8_THREADS>(g1, g2, queue, grid, s); break;
    case 48: launch_persistent2<k_gemm_fp8<48, P2>, FP8_THREADS>(g1, g2, queue, grid, s); break;
    case 96: launch_persistent2<k_gemm_fp8<96, P2>, FP8_THREADS>(g1, g2, queue, grid, s); break;
    case 128: launch_persistent2<k_gemm_fp8<128, P2>, FP8_THREADS>(g1, g2, queue, grid, s); break;
    case 160: launch_persistent2<k_gemm_fp8<160, P2>, FP8_THREADS>(g1, g2, queue, grid, s); break;
    default: launch_persistent2<k_gemm_fp8<192, P2>, FP8_THREADS>(g1, g2, queue, grid, s); break;
  }
}

void launch_gemm_fp8_pair(const GemmArgs& g1, const GemmArgs& g2, int32_t* queue, int bm, int grid,
                          hipStream_t s) {
  launch_fp8<false>(g1, g2, queue, bm, grid, s);
}

void launch_gemm_fp8_pow2_pair(const GemmArgs& g1, const GemmArgs& g2, int32_t* queue, int bm, int grid,
                               hipStream_t s) {
  launch_fp8<true>(g1, g2, queue, bm, grid, s);
}

}  // namespace moe
