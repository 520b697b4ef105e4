// The materialized-chunk scheme, as the Orbit announcement (技术细节,
// active-expert-chunked dequantization) describes it literally: the experts of
// one chunk are dequantized into a temporary BF16 copy in device memory, an
// ordinary BF16 grouped GEMM runs on that copy, and the copy is overwritten by
// the next chunk.  It exists to measure what the fused kernels save (the copy
// costs 2 bytes written and read back per weight, and its size grows with the
// chunk) and to compare the two numerics.
//
// k_dequant_chunk: one pass over the chunk's packed experts, 8 weights per
// thread per iteration, bf16 written with round-to-nearest-even.
// k_gemm_bf16<BM>: BM rows x 256 weight rows per item (GEMM1: 128 gate + 128
// up rows, h = silu(gate) * up rounded to bf16; GEMM2: 256 output columns),
// K step 64, operands streamed into an LDS stage ring by global_load_lds DMA
// and consumed by bf16 16x16x32 MFMA.
#include "common.h"
#include "kernels.h"
#include "moe_sched.h"

namespace moe {

// ------------------------------------------------------------------ dequant

// E2M1 nibble -> fp32 (exact): 0, 0.5, 1, 1.5, 2, 3, 4, 6 with sign bit 3.
MOE_DEV float e2m1_to_f32(uint32_t nib) {
  const uint32_t s = (nib & 8u) << 28, e = (nib >> 1) & 3u, m = nib & 1u;
  const uint32_t mag = e == 0 ? (m ? 0x3F000000u : 0u) : (((e + 126u) << 23) | (m << 22));
  return __uint_as_float(s | mag);
}

// bf16 bits of the exact product a * s, rounded to nearest even.  The fp32
// product is turned into its round-to-odd form (truncate, then set the last
// bit if anything was lost; the FMA gives the exact remainder), and rounding
// that to nearest at 8 bits equals one rounding of the exact product, since
// fp32 keeps more than two extra bits.
MOE_DEV uint32_t bf16_of_product(float a, float s) {
  const float p = a * s;
  const float err = __builtin_fmaf(a, s, -p);
  uint32_t pb = __float_as_uint(p);
  if (err != 0.0f) {
    if ((__float_as_uint(err) ^ pb) >> 31) pb -= 1;  // |p| above the exact value: step toward zero
    pb |= 1u;
  }
  return f32_to_bf16_bits(__uint_as_float(pb));
}

// One unit: 8 consecutive weights of one row (16 bytes of bf16), so that a
// wave's loads and stores are contiguous.  Each thread loads four units
// before converting any, to keep four loads in flight per wave.
struct Raw8 {
  uint2 q;       // FP8: 8 codes; INT4 / MXFP4 / NVFP4: 8 nibbles in q.x
  uint32_t s;    // scale bits (fp32, bf16, E8M0 or E4M3)
};

// Byte offset of code (n, k0) in one expert's matrix of N x K codes: rows
// (each row's K codes contiguous) or 16 x 128 tiles (tile (n/16, k0/128)
// K-fastest, a row's 128 codes contiguous inside it); RB = bytes of 128 codes.
template <int RB>
MOE_DEV int64_t code_offset(bool kblocked, int K, int n, int k0) {
  if (!kblocked) return ((int64_t)n * K + k0) * RB / 128;
  return ((int64_t)(n >> 4) * (K / 128) + (k0 >> 7)) * (16 * RB) + (n & 15) * RB + (k0 & 127) * RB / 128;
}

template <int FMT>
MOE_DEV Raw8 load8(const uint8_t* __restrict__ w, const void* __restrict__ sc, int N, int K, int n, int k0,
                   bool kblocked) {
  Raw8 r;
  if (FMT == FMT_FP8) {
    r.q = *reinterpret_cast<const uint2*>(w + code_offset<128>(kblocked, K, n, k0));
    r.s = static_cast<const uint32_t*>(sc)[(n / 128) * (K / 128) + k0 / 128];
  } else {
    r.q.x = *reinterpret_cast<const uint32_t*>(w + code_offset<64>(kblocked, K, n, k0));
    r.q.y = 0;
    const int si = (k0 / (FMT == FMT_NVFP4 ? 16 : 32)) * N + n;  // group-major [K/32][N] ([K/16][N])
    r.s = FMT == FMT_INT4 ? (uint32_t) static_cast<const uint16_t*>(sc)[si]
                          : (uint32_t) static_cast<const uint8_t*>(sc)[si];
  }
  return r;
}

// g: the matrix's NVFP4 second-level scale (unused by the other formats).
template <int FMT>
MOE_DEV uint4 cvt8(const Raw8& r, float g) {
  uint32_t o[4];
  if (FMT == FMT_NVFP4) {
    const float s = e4m3_to_f32(r.s);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t b = r.q.x >> (i * 8);
      // E2M1 times an E4M3 scale is exact in fp32; the product with g is
      // rounded once to bf16
      o[i] = bf16_of_product(e2m1_to_f32(b & 15u) * s, g) | (bf16_of_product(e2m1_to_f32((b >> 4) & 15u) * s, g) << 16);
    }
  } else if (FMT == FMT_FP8) {
    const float s = __uint_as_float(r.s);
    const uint32_t qs[2] = {r.q.x, r.q.y};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t d = qs[i >> 1] >> ((i & 1) * 16);
      o[i] = bf16_of_product(e4m3_to_f32(d & 0xFFu), s) | (bf16_of_product(e4m3_to_f32((d >> 8) & 0xFFu), s) << 16);
    }
  } else if (FMT == FMT_INT4) {
    const float s = bf16_bits_to_f32(r.s);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t b = r.q.x >> (i * 8);
      const float lo = (float)((int32_t)(b << 28) >> 28), hi = (float)((int32_t)(b << 24) >> 28);
      // a 4-bit integer times a bf16 scale is exact in fp32
      o[i] = bf16x2_bits(lo * s, hi * s);
    }
  } else {
    const float s = __uint_as_float(r.s ? r.s << 23 : 0x00400000u);  // 2^(s - 127)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t b = r.q.x >> (i * 8);
      // E2M1 times a power of two is exact in bf16
      o[i] = bf16x2_bits(e2m1_to_f32(b & 15u) * s, e2m1_to_f32((b >> 4) & 15u) * s);
    }
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// grid.y = chunk slot (slots past the chunk's last active expert exit).
// Units u < u13 are W13's, the rest W2's, both in row-major order of the
// copy; the codes are read from rows or from 16 x 128 tiles (kblocked).
template <int FMT>
__global__ __launch_bounds__(256) void k_dequant_chunk(const uint8_t* __restrict__ w13, const void* __restrict__ s13,
                                                       const uint8_t* __restrict__ w2, const void* __restrict__ s2,
                                                       const int32_t* __restrict__ active,
                                                       const int32_t* __restrict__ num_active, int chunk, int C,
                                                       int H, int I, const float* __restrict__ g13,
                                                       const float* __restrict__ g2, bool kblocked,
                                                       uint16_t* __restrict__ scratch) {
  const int na = *num_active;
  const int slot = blockIdx.y;
  const int a = chunk * C + slot;
  if (slot >= C || a >= na) return;
  const int e = active[a];
  const int64_t n13 = (int64_t)2 * I * H, n2 = (int64_t)H * I;
  constexpr int64_t WB = FMT == FMT_FP8 ? 1 : 2;                 // weights per byte
  constexpr int64_t SB = FMT == FMT_FP8 ? 128 * 128 : FMT == FMT_NVFP4 ? 16 : 32;  // weights per scale
  constexpr int64_t SZ = FMT == FMT_FP8 ? 4 : FMT == FMT_INT4 ? 2 : 1;  // scale bytes
  const int u13 = (int)(n13 / 8), total = (int)((n13 + n2) / 8);
  const int KU1 = H / 8, KU2 = I / 8;
  const uint8_t* w13e = w13 + (int64_t)e * (n13 / WB);
  const uint8_t* w2e = w2 + (int64_t)e * (n2 / WB);
  const char* s13e = static_cast<const char*>(s13) + (int64_t)e * (n13 / SB) * SZ;
  const char* s2e = static_cast<const char*>(s2) + (int64_t)e * (n2 / SB) * SZ;
  uint16_t* dst = scratch + (int64_t)slot * (n13 + n2);
  const float ga = FMT == FMT_NVFP4 ? g13[e] : 1.0f, gb = FMT == FMT_NVFP4 ? g2[e] : 1.0f;
  const int stride = gridDim.x * 256;
  constexpr int U = 4;
  for (int u0 = blockIdx.x * 256 + threadIdx.x; u0 < total; u0 += U * stride) {
    Raw8 r[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int u = u0 + j * stride;
      if (u < u13) {
        const int n = u / KU1;
        r[j] = load8<FMT>(w13e, s13e, 2 * I, H, n, (u - n * KU1) * 8, kblocked);
      } else if (u < total) {
        const int v = u - u13, n = v / KU2;
        r[j] = load8<FMT>(w2e, s2e, H, I, n, (v - n * KU2) * 8, kblocked);
      }
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int u = u0 + j * stride;
      if (u < total) *reinterpret_cast<uint4*>(dst + (int64_t)u * 8) = cvt8<FMT>(r[j], u < u13 ? ga : gb);
    }
  }
}

void launch_dequant_chunk(int fmt, const uint8_t* w13, const void* s13, const uint8_t* w2, const void* s2,
                          const int32_t* active, const int32_t* num_active, int chunk, int C, int H, int I,
                          const float* g13, const float* g2, bool kblocked, uint16_t* scratch, hipStream_t s) {
  // about 4096 workgroups over the chunk's slots, at least 16 per slot
  const int gx = C >= 256 ? 16 : 4096 / C;
  const dim3 grid(gx, C), block(256);
  if (fmt == FMT_INT4)
    hipLaunchKernelGGL(k_dequant_chunk<FMT_INT4>, grid, block, 0, s, w13, s13, w2, s2, active, num_active, chunk, C,
                       H, I, g13, g2, kblocked, scratch);
  else if (fmt == FMT_FP8)
    hipLaunchKernelGGL(k_dequant_chunk<FMT_FP8>, grid, block, 0, s, w13, s13, w2, s2, active, num_active, chunk, C,
                       H, I, g13, g2, kblocked, scratch);
  else if (fmt == FMT_NVFP4)
    hipLaunchKernelGGL(k_dequant_chunk<FMT_NVFP4>, grid, block, 0, s, w13, s13, w2, s2, active, num_active, chunk,
                       C, H, I, g13, g2, kblocked, scratch);
  else
    hipLaunchKernelGGL(k_dequant_chunk<FMT_MXFP4>, grid, block, 0, s, w13, s13, w2, s2, active, num_active, chunk,
                       C, H, I, g13, g2, kblocked, scratch);
}

// ------------------------------------------------------------- BF16 GEMM

// LDS of one stage: BM activation rows and the 4 waves' 4 x 16 weight rows,
// 64 bf16 (128 bytes) each, 16-byte parts XOR-swizzled by (row & 7).
template <int BM>
struct BfStage {
  static constexpr int A_BYTES = BM * 128;
  static constexpr int B_OFF = A_BYTES;
  static constexpr int BYTES = B_OFF + 256 * 128;
  static constexpr int APW = BM * 2;              // activation 16-byte pieces per wave
  static constexpr int NA = (APW + 63) / 64;      // activation DMA instructions per wave
  static constexpr int SR = (152 * 1024) / BYTES;
  static constexpr int S = SR > 5 ? 5 : SR;       // stages
  static constexpr int NPER = NA + 8;             // DMA instructions per wave per stage
};

template <int BM, bool G1>
__device__ __forceinline__ void bf_item(const GemmArgs& p, const Tile& tl, uint8_t* smem) {
  constexpr int MT = BM / 16;
  using ST = BfStage<BM>;
  constexpr int S = ST::S;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int ln = lane & 15, lg = lane >> 4;
  const int K = p.K, KT = K / 64;
  const uint32_t smem0 = lds_u32(smem);
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
  // the chunk's BF16 copy holds its experts in active order
  const int slot = tl.a - p.chunk * p.chunk_experts;
  const char* wexp = reinterpret_cast<const char*>(p.w) + (int64_t)slot * p.w_expert_bytes;
  const char* bsrc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = h * 64 + lane, rr = c >> 3, part = c & 7;
      bsrc[i][h] = wexp + (int64_t)(col[i] + rr) * K * 2 + ((part ^ (rr & 7)) << 4);
    }
  const char* asrc[ST::NA];
#pragma unroll
  for (int j = 0; j < ST::NA; ++j) {
    const int c = min(wave * ST::APW + j * 64 + lane, BM * 8 - 1);
    const int row = c >> 3, part = c & 7;
    const int rr = tl.rbase + min(row, tl.nrows - 1);
    const int src = p.a_per_token ? p.sorted_rows[rr] / p.top_k : rr;
    asrc[j] = static_cast<const char*>(p.a) + (int64_t)src * K * 2 + ((part ^ (row & 7)) << 4);
  }
  auto issue = [&](int kt, int s) {
    const uint32_t sb = smem0 + s * ST::BYTES;
#pragma unroll
    for (int j = 0; j < ST::NA; ++j)
      if (ST::APW >= 64 || lane < ST::APW) dma_b128(asrc[j] + kt * 128, sb + (wave * ST::APW + j * 64) * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) dma_b128(bsrc[i][h] + kt * 128, sb + ST::B_OFF + (wave * 4 + i) * 2048 + h * 1024);
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
    wait_stages<ST::NPER>(min(S - 2, KT - 1 - kt));  // this wave's pieces of stage kt have landed
    lds_barrier();                                    // ... and every other wave's
    if (kt + S - 1 < KT) issue(kt + S - 1, (kt + S - 1) % S);
    const uint8_t* st = smem + (kt % S) * ST::BYTES;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int lp = 4 * s + lg;  // logical 16-byte part of this lane's 8 K values
      bf16x8 bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        bfr[i] = *reinterpret_cast<const bf16x8*>(st + ST::B_OFF + (wave * 4 + i) * 2048 + ln * 128 +
                                                  ((lp ^ (ln & 7)) << 4));
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int r = m * 16 + ln;
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(st + r * 128 + ((lp ^ (r & 7)) << 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[m][i] = mfma_bf16_16x16x32(af, bfr[i], acc[m][i]);
      }
    }
  }

  // Epilogue through LDS (stage buffers are free after the barrier) so that
  // global stores are 16 bytes per lane.
  lds_barrier();
  if (G1) {
    constexpr int HS = 272;  // staged row stride (bytes) of the 128 bf16 h values
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m * 16 + lg * 4 + i;
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const float hv = silu_f32(acc[m][n][i]) * acc[m][n + 2][i];
          *reinterpret_cast<uint16_t*>(smem + row * HS + (wave * 32 + n * 16 + ln) * 2) =
              (uint16_t)f32_to_bf16_bits(hv);
        }
      }
    lds_barrier();
    copy_out_rows<BM, 256, HS, 256>(smem, static_cast<char*>(p.out) + (int64_t)tl.nb * 256 + (int64_t)tl.rbase * p.inter * 2,
                                    (int64_t)p.inter * 2, tl.nrows);
  } else {
    constexpr int YS = 528;  // staged row stride (bytes) of the 256 bf16 outputs
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
    copy_out_rows<BM, 512, YS, 256>(smem, static_cast<char*>(p.out) + (int64_t)tl.nb * 512 + (int64_t)tl.rbase * p.N * 2,
                                    (int64_t)p.N * 2, tl.nrows);
  }
}

// Persistent launch over chunk p1.chunk's GEMM1 items and chunk p2.chunk's
// GEMM2 items (either may be empty), dealt through per-XCD atomic counters as
// in the fused kernels.
template <int BM>
__global__ __launch_bounds__(256, 1) void k_gemm_bf16(GemmArgs p1, GemmArgs p2, int32_t* queue) {
  using ST = BfStage<BM>;
  constexpr int S = ST::S;
  static_assert(S >= 2 && S <= 5, "LDS stages");
  static_assert(ST::NA * 64 >= ST::APW, "activation pieces");
  __shared__ __align__(16) uint8_t smem[S * ST::BYTES];
  static_assert(S * ST::BYTES >= BM * 528, "epilogue staging fits in the stage buffers");
  __shared__ int s_item;
  ChunkWork c1, c2;
  const int n1 = chunk_work(p1, p1.inter / 128, c1) ? c1.nwork : 0;
  const int n2 = chunk_work(p2, p2.N / 256, c2) ? c2.nwork : 0;
  const int x = blockIdx.x & 7;
  const int per1 = (n1 + 7) >> 3, per2 = (n2 + 7) >> 3;
  const int b1 = x * per1, b2 = x * per2;
  const int len1 = max(0, min(n1, b1 + per1) - b1), len2 = max(0, min(n2, b2 + per2) - b2);
  int32_t* q = queue + x;
  const int wpx = gridDim.x >> 3;
  int cur = blockIdx.x >> 3;
  while (cur < len1 + len2) {
    int nxt = 0;
    if (threadIdx.x == 0) nxt = atomicAdd(q, 1) + wpx;
    if (cur < len1) bf_item<BM, true>(p1, tile_of(p1, c1, b1 + cur, BM), smem);
    else bf_item<BM, false>(p2, tile_of(p2, c2, b2 + cur - len1, BM), smem);
    if (threadIdx.x == 0) s_item = nxt;
    lds_barrier();
    cur = s_item;
  }
}

void launch_gemm_bf16_pair(const GemmArgs& g1, const GemmArgs& g2, int32_t* queue, int bm, int grid,
                           hipStream_t s) {
  switch (bm) {
    case 16: launch_persistent2<k_gemm_bf16<16>>(g1, g2, queue, grid, s); break;
    case 32: launch_persistent2<k_gemm_bf16<32>>(g1, g2, queue, grid, s); break;
    case 64: launch_persistent2<k_gemm_bf16<64>>(g1, g2, queue, grid, s); break;
    default: launch_persistent2<k_gemm_bf16<128>>(g1, g2, queue, grid, s); break;
  }
}

}  // namespace moe
