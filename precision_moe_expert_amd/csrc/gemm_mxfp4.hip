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
// columns are exactly one scale block, so the block maximum is a row-local
// DPP reduction.  Operands stream through an LDS ring filled by
// global_load_lds DMA (see the FP8 kernel for the scheme).
#include "common.h"
#include "kernels.h"
#include "moe_sched.h"

namespace moe {

// MXFP8 shared exponent of a block with maximum magnitude am:
// X = floor(log2(am)) - 8 clamped to [-127, 127], 0 when am = 0 (or NaN).
// For a normal am, floor(log2(am)) is its biased exponent minus 127; a
// subnormal am (exponent field 0) gives X <= -135 and clamps to -127, which
// the exponent field gives too; the largest exponent field (255: inf) gives
// X = 120, so the upper clamp never applies.
MOE_DEV int mx_shared_exp(float am) {
  return am > 0.0f ? max((int)(__float_as_uint(am) >> 23) - 135, -127) : 0;
}

// LDS bytes of one pipeline stage: activation rows (128 B of E4M3 codes each,
// whole DMA groups of 8 rows per wave), each wave's weight fragments (4
// subtiles x 1 KB of E2M1) and the E8M0 scales of its 64 weight rows for the
// step's 4 groups (group-major storage: 16 contiguous runs of 16 bytes).
template <int BM>
struct MxStage {
  static constexpr int NA = (BM * 8 + 255) / 256;  // activation DMA groups per wave
  static constexpr int A_BYTES = NA * 32 * 128;
  static constexpr int B_OFF = A_BYTES;
  static constexpr int BS_OFF = B_OFF + 4 * 4 * 1024;
  static constexpr int BYTES = BS_OFF + 4 * 256;
  // Two workgroups per CU (up to 128-row tiles): with no per-block rescale
  // the MFMA loop fits in 256 registers, and a second resident workgroup
  // covers one's barrier and LDS waits with the other's MFMAs (measured on
  // MI355X: 19% faster than one workgroup with a deeper ring).
  static constexpr int WPC = BM <= 128 ? 2 : 1;
  static constexpr int S = (152 * 1024 / WPC) / BYTES > 5 ? 5 : (152 * 1024 / WPC) / BYTES;  // stages
  static constexpr int NPER = NA + 4 + 1;            // DMA instructions per wave per stage
  // Activation scales travel in blocks of 4 K steps (16 B per row), double-
  // buffered outside the ring: waves 0..NASW-1 load 64 rows each with
  // every 4th stage.
  static constexpr int NASW = (BM + 63) / 64;
  static constexpr int AS_BLOCK = NASW * 64 * 16;
};

// One work item: a BM-row tile times one N block (GEMM1: 128 h columns, i.e.
// 128 gate + 128 up weight rows; GEMM2: 256 output columns).
template <int BM, bool G1>
__device__ __forceinline__ void mx_item(const GemmArgs& p, const Tile& tl, uint8_t* smem, uint8_t* asb) {
  constexpr int MT = BM / 16;
  using ST = MxStage<BM>;
  constexpr int S = ST::S;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int ln = lane & 15, lg = lane >> 4;
  const int K = p.K, KT = K / 128;
  const char* Abase = static_cast<const char*>(p.a);
  const char* ASbase = static_cast<const char*>(p.a_scale);
  const uint32_t smem0 = lds_u32(smem), asb0 = lds_u32(asb);
  lds_barrier();  // every wave is done with the previous item's stages
  int col[4];
  if (G1) {
    const int g0 = tl.nb * 128 + wave * 32;
    col[0] = g0; col[1] = g0 + 16; col[2] = p.inter + g0; col[3] = p.inter + g0 + 16;
  } else {
    const int c0 = tl.nb * 256 + wave * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) col[i] = c0 + 16 * i;
  }
  // per-lane global sources of this item's DMA pieces (K offset added per step)
  const char* wexp = reinterpret_cast<const char*>(p.w) + tl.e * p.w_expert_bytes;
  const char* wsexp = static_cast<const char*>(p.w_scale) + tl.e * p.ws_expert_elems;
  // the four subtiles' weight rows are col[i] + ln: one per-lane pointer plus
  // wave-uniform row offsets (fewer live registers than four pointers)
  const char* bsrc0 = p.w_kblocked ? wexp + (int64_t)(col[0] / 16) * (K / 128) * 1024 + ln * 64 + lg * 16
                                   : wexp + (int64_t)(col[0] + ln) * (K / 2) + lg * 16;
  const int bstep = p.w_kblocked ? 1024 : 64;  // bytes between K steps of one lane's piece
  int64_t boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    boff[i] = p.w_kblocked ? (int64_t)((col[i] - col[0]) / 16) * (K / 128) * 1024 : (int64_t)(col[i] - col[0]) * (K / 2);
  // E8M0 weight scales (group-major): lane l < 16 takes 16 consecutive
  // weight rows of group l/4, i.e. one subtile
  uint32_t bsoff;  // from wsexp
  {
    const int g = (lane >> 2) & 3, pc = lane & 3;
    const int c = G1 ? (pc < 2 ? col[0] + pc * 16 : col[2] + (pc - 2) * 16) : col[0] + pc * 16;
    bsoff = (uint32_t)(g * p.N + c);
  }
  // activation pieces as 16-byte unit offsets from Abase (32 bits each)
  uint32_t aoff[ST::NA];
#pragma unroll
  for (int j = 0; j < ST::NA; ++j) {
    const int c = (wave * ST::NA + j) * 64 + lane;   // activation piece: row c/8, slot c%8
    const int row = c >> 3, slot = c & 7;
    const int part = slot ^ (row & 7);               // XOR swizzle of 16-byte parts
    const int rr = tl.rbase + min(min(row, BM - 1), tl.nrows - 1);
    const int sr = p.sorted_rows[rr];
    const int src = p.a_per_token ? sr / p.top_k : rr;
    aoff[j] = (uint32_t)src * (uint32_t)(K / 16) + (uint32_t)part;
  }
  uint32_t soff;  // from ASbase
  {
    const int row = wave * 64 + lane;
    const int rr = tl.rbase + min(min(row, BM - 1), tl.nrows - 1);
    const int sr = p.sorted_rows[rr];
    const int src = p.a_per_token ? sr / p.top_k : rr;
    soff = (uint32_t)src * (uint32_t)p.a_scale_stride;
  }
  auto issue = [&](int kt, int slot) {
    const uint32_t sb = smem0 + slot * ST::BYTES;
#pragma unroll
    for (int j = 0; j < ST::NA; ++j)
      dma_b128(Abase + (uint64_t)aoff[j] * 16 + kt * 128, sb + (wave * ST::NA + j) * 1024);
    if (wave < ST::NASW && (kt & 3) == 0)
      dma_b128(ASbase + (uint64_t)soff + (kt >> 2) * 16, asb0 + ((kt >> 2) & 1) * ST::AS_BLOCK + wave * 1024);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_b128(bsrc0 + boff[i] + kt * bstep, sb + ST::B_OFF + (wave * 4 + i) * 1024);
    if (lane < 16) dma_b128(wsexp + (uint64_t)bsoff + (int64_t)kt * 4 * p.N, sb + ST::BS_OFF + wave * 256);
  };
  f32x4 acc[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[m][i] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
  for (int s = 0; s + 1 < S; ++s)
    if (s < KT) issue(s, s);
  for (int kt = 0; kt < KT; ++kt) {
    {
      // this wave's pieces of stage kt have landed (later stages in flight
      // hold one more load if a scale block starts among them)
      const int n = min(S - 2, KT - 1 - kt);
      wait_stages_x<ST::NPER>(n, (wave < ST::NASW && ((kt + n) >> 2) > (kt >> 2)) ? 1 : 0);
    }
    // this wave's weight fragments and their scales come from its own DMAs
    // only, so they are read before the barrier, which then covers their
    // latency (headline GEMM 1.1% faster)
    const uint8_t* st = smem + (kt % S) * ST::BYTES;
    i32x4 bf[4];
    int sb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf[i] = *reinterpret_cast<const i32x4*>(st + ST::B_OFF + (wave * 4 + i) * 1024 + lane * 16);
      sb[i] = (int)st[ST::BS_OFF + wave * 256 + lg * 64 + i * 16 + ln];
    }
    lds_barrier();                                    // ... and every other wave's
    if (kt + S - 1 < KT) issue(kt + S - 1, (kt + S - 1) % S);
    auto read_a = [&](int m, i32x8& af, int& sa) {
      const int r = m * 16 + ln;
      const uint8_t* arow = st + r * 128;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(arow + ((lg ^ (r & 7)) << 4));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(arow + (((lg + 4) ^ (r & 7)) << 4));
      af = (i32x8){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      sa = (int)asb[((kt >> 2) & 1) * ST::AS_BLOCK + r * 16 + (kt & 3) * 4 + lg];
    };
    // Row block m + 1's operands are read while block m's MFMAs issue, one
    // LDS read between two MFMAs (the scheduling groups; without them the
    // compiler sinks the reads to their first use): headline GEMM 1.8%
    // faster than issuing the three reads ahead of the four MFMAs.
    i32x8 af[2];
    int sa[2];
    read_a(0, af[0], sa[0]);
    // the MFMA phase at raised wave priority: when this SIMD's other wave
    // (the other workgroup) is ready too, the matrix core's feeder issues
    // first (headline GEMM 1.2% faster)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      __builtin_amdgcn_sched_barrier(0);
      if (m + 1 < MT) read_a(m + 1, af[(m + 1) & 1], sa[(m + 1) & 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[m][i] = mfma_fp8_fp4_scaled_16x16x128(af[m & 1], bf[i], sa[m & 1], sb[i], acc[m][i]);
      if (m + 1 < MT) {
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  }

  // Epilogue: results go through LDS (the stage buffers are free once every
  // wave has passed the barrier below) so that global stores are 16 B per lane.
  if (G1) {
    if (p.ab_out != nullptr) {
      // backward recompute: the gate and up pre-activations in fp32 as well
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = m * 16 + lg * 4 + i;
          if (row < tl.nrows)
#pragma unroll
            for (int n = 0; n < 4; ++n) p.ab_out[(int64_t)(tl.rbase + row) * p.N + col[n] + ln] = acc[m][n][i];
        }
    }
    constexpr int HS = 144;  // staged row stride (bytes) of the 128 h codes
    uint8_t* He = static_cast<uint8_t*>(p.out_scale);
    lds_barrier();
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float h0[4], h1[4], am[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h0[i] = silu_f32(acc[m][0][i]) * acc[m][2][i];
        h1[i] = silu_f32(acc[m][1][i]) * acc[m][3][i];
        am[i] = fmaxf(fabsf(h0[i]), fabsf(h1[i]));
      }
      // this wave's 32 h columns of a row are one MXFP8 block
      row16_max_nonneg4(am);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int X = mx_shared_exp(am[i]);
        const float mul = __uint_as_float((uint32_t)(127 - X) << 23);  // 2^-X, X in [-127, 120]
        const int row = m * 16 + lg * 4 + i;
        const uint32_t c2 = cvt_e4m3x2(h0[i] * mul, h1[i] * mul);
        smem[row * HS + wave * 32 + ln] = (uint8_t)(c2 & 0xFF);
        smem[row * HS + wave * 32 + 16 + ln] = (uint8_t)(c2 >> 8);
        // the row's four block scales (one per wave) are staged as one dword
        if (ln == 0) smem[BM * HS + row * 4 + wave] = (uint8_t)(X + 127);
      }
    }
    lds_barrier();
    copy_out_rows<BM, 128, HS, 256, 1>(smem, static_cast<char*>(p.out) + tl.nb * 128 + (int64_t)tl.rbase * p.inter,
                                    (int64_t)p.inter, tl.nrows);
    for (int row = threadIdx.x; row < tl.nrows; row += 256)
      *reinterpret_cast<uint32_t*>(He + (int64_t)(tl.rbase + row) * p.out_scale_stride + tl.nb * 4) =
          *reinterpret_cast<const uint32_t*>(smem + BM * HS + row * 4);
  } else {
    constexpr int YS = 528;  // staged row stride (bytes) of the 256 bf16 outputs
    lds_barrier();
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m * 16 + lg * 4 + i;
#pragma unroll
        for (int n = 0; n < 4; ++n)
          *reinterpret_cast<uint16_t*>(smem + row * YS + (wave * 64 + n * 16 + ln) * 2) =
              (uint16_t)f32_to_bf16_bits(acc[m][n][i]);
      }
    lds_barrier();
    copy_out_rows<BM, 512, YS, 256, (BM <= 128 ? 4 : 1)>(smem, static_cast<char*>(p.out) + (int64_t)tl.nb * 512 + (int64_t)tl.rbase * p.N * 2,
                                    (int64_t)p.N * 2, tl.nrows);
  }
}

// Persistent pair launch: the GEMM1 items of chunk p1.chunk and the GEMM2
// items of chunk p2.chunk (either may be empty), dealt through per-XCD
// atomic work counters exactly as for the FP8 weights.
template <int BM>
__global__ __launch_bounds__(256, MxStage<BM>::WPC) void k_gemm_mxfp4(GemmArgs p1, GemmArgs p2, int32_t* queue) {
  using ST = MxStage<BM>;
  constexpr int S = ST::S;
  static_assert(S >= 2 && S <= 5, "LDS stages");
  __shared__ __align__(16) uint8_t smem[S * ST::BYTES];
  static_assert(S * ST::BYTES >= BM * 528, "epilogue staging fits in the stage buffers");
  __shared__ __align__(16) uint8_t asb[2 * ST::AS_BLOCK];
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
    if (cur < len1) mx_item<BM, true>(p1, tile_of(p1, c1, b1 + cur, BM), smem, asb);
    else mx_item<BM, false>(p2, tile_of(p2, c2, b2 + cur - len1, BM), smem, asb);
    if (threadIdx.x == 0) s_item = nxt;
    lds_barrier();
    cur = s_item;
  }
}

void launch_gemm_mxfp4_pair(const GemmArgs& g1, const GemmArgs& g2, int32_t* queue, int bm, int grid,
                            hipStream_t s) {
  switch (bm) {
    case 16: launch_persistent2<k_gemm_mxfp4<16>>(g1, g2, queue, grid, s); break;
    case 32: launch_persistent2<k_gemm_mxfp4<32>>(g1, g2, queue, grid, s); break;
    case 64: launch_persistent2<k_gemm_mxfp4<64>>(g1, g2, queue, grid, s); break;
    case 48: launch_persistent2<k_gemm_mxfp4<48>>(g1, g2, queue, grid, s); break;
    case 96: launch_persistent2<k_gemm_mxfp4<96>>(g1, g2, queue, grid, s); break;
    case 128: launch_persistent2<k_gemm_mxfp4<128>>(g1, g2, queue, grid, s); break;
    default: launch_persistent2<k_gemm_mxfp4<192>>(g1, g2, queue, grid, s); break;
  }
}

}  // namespace moe
