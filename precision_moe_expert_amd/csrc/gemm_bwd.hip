// Frozen-base backward GEMMs (Orbit announcement, 技术细节: the GEMM backward
// that bypasses the base weight gradient).  The input gradients are
//   u  = dout W2            (per permuted row; contraction over H)
//   dx' = [da | db] W13     (contraction over 2I)
// so both GEMMs contract over the weights' output dimension.  They read a
// transposed copy of the frozen weights, made once by launch_repack_bwd:
// K-contiguous rows for the backward GEMMs.  A group scale of INT4 or MXFP4
// belongs to (weight row group, K) in the forward orientation, so in the
// transposed copy it varies along K: every element gets its own scale, kept
// as fp16 in the pair order the unpack multiplies.  NVFP4 groups 16 forward
// K values per E4M3 scale (16-row groups of the transposed copy) and applies
// its per-matrix fp32 scale to the accumulators, as the forward does.  FP8
// block scales cover 128 x 128 squares and stay per (row block, K block).
//
// k_gemm_bwd<FMT, BM>: the forward INT4 kernel's DMA ring, LDS layout and
// fp16 16x16x32 MFMA (weights become fp16: INT4 codes and E2M1 values times
// their scale exactly, E4M3 codes times the block scale rounded once);
// 256-column N blocks; two epilogues:
//   DH: SwiGLU backward from the recomputed pre-activations (a, b) and the
//       routing weight w: dh = w u, da = dh b silu'(a), db = dh silu(a) ->
//       fp16 [R][2I] in the INT4 activation order, and per-row partial sums
//       <u, h> for the router gradient (h as the forward fed it to GEMM2:
//       silu(a) b for INT4, the quantized h of the FP8 / MXFP8 formats).
//   DX: dx' rows in fp32 [R][H].
#include "common.h"
#include "int4.h"
#include "kernels.h"
#include "moe_sched.h"

namespace moe {

// ------------------------------------------------------------- repacking

// W [E][N][K] nibbles (element 2m in the low nibble of byte m) -> W^T with
// K rows of N nibbles in the same convention, stored in 16-row x 128-column
// tiles of 1 KB, columns fastest: [E][K/16][N/128][16][64 B], so that a
// backward GEMM step reads one contiguous run per 16 rows.  One 64 x 64
// nibble tile per iteration, transposed through LDS (one byte per nibble).
// (tiled = 1: the source codes are in the forward's 16-row x 128-K tiles.)
__global__ __launch_bounds__(256) void k_repack_int4_t(const uint8_t* __restrict__ w, int E, int N, int K,
                                                       int tiled, uint8_t* __restrict__ wt) {
  __shared__ uint8_t tile[64][65];
  const int tn = N / 64, tk = K / 64;
  const int64_t ntiles = (int64_t)E * tn * tk;
  const int t = threadIdx.x, row = t >> 2, part = t & 3;
  for (int64_t ti = blockIdx.x; ti < ntiles; ti += gridDim.x) {
    const int e = (int)(ti / ((int64_t)tn * tk));
    const int rem = (int)(ti - (int64_t)e * tn * tk);
    const int n0 = (rem / tk) * 64, k0 = (rem % tk) * 64;
    const uint8_t* src = w + (int64_t)e * N * K / 2;
    const int sn = n0 + row, sk = k0 + part * 16;  // source row and first K value
    const uint2 v = *reinterpret_cast<const uint2*>(
        src + (tiled ? ((int64_t)(sn / 16) * (K / 128) + sk / 128) * 1024 + (sn % 16) * 64 + (sk % 128) / 2
                     : ((int64_t)sn * K + sk) / 2));
    const uint32_t vs[2] = {v.x, v.y};
#pragma unroll
    for (int q = 0; q < 16; ++q) tile[row][part * 16 + q] = (uint8_t)((vs[q >> 3] >> ((q & 7) * 4)) & 15u);
    __syncthreads();
    // output row k0 + row, nibbles n0 + part*16 .. +15
    uint32_t o[2] = {0u, 0u};
#pragma unroll
    for (int q = 0; q < 16; ++q) o[q >> 3] |= (uint32_t)tile[part * 16 + q][row] << ((q & 7) * 4);
    uint8_t* dst = wt + (int64_t)e * N * K / 2;
    const int r = k0 + row, n = n0 + part * 16;
    *reinterpret_cast<uint2*>(dst + ((int64_t)(r / 16) * (N / 128) + n / 128) * 1024 + (r % 16) * 64 + (n % 128) / 2) =
        make_uint2(o[0], o[1]);
    __syncthreads();
  }
}

// W [E][N][K] bytes -> W^T with K rows of N bytes in 16-row x 128-column
// tiles of 2 KB, columns fastest ([E][K/16][N/128][16][128 B]); 64 x 64
// byte tiles through LDS.
__global__ __launch_bounds__(256) void k_repack_u8_t(const uint8_t* __restrict__ w, int E, int N, int K, int tiled,
                                                     uint8_t* __restrict__ wt) {
  __shared__ uint8_t tile[64][68];
  const int tn = N / 64, tk = K / 64;
  const int64_t ntiles = (int64_t)E * tn * tk;
  const int t = threadIdx.x, row = t >> 2, part = t & 3;
  for (int64_t ti = blockIdx.x; ti < ntiles; ti += gridDim.x) {
    const int e = (int)(ti / ((int64_t)tn * tk));
    const int rem = (int)(ti - (int64_t)e * tn * tk);
    const int n0 = (rem / tk) * 64, k0 = (rem % tk) * 64;
    const int sn = n0 + row, sk = k0 + part * 16;  // source row and first K value
    const u32x4 v = *reinterpret_cast<const u32x4*>(
        w + (int64_t)e * N * K +
        (tiled ? ((int64_t)(sn / 16) * (K / 128) + sk / 128) * 2048 + (sn % 16) * 128 + sk % 128
               : (int64_t)sn * K + sk));
    const uint32_t vs[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 16; ++q) tile[row][part * 16 + q] = (uint8_t)(vs[q >> 2] >> ((q & 3) * 8));
    __syncthreads();
    uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 16; ++q) o[q >> 2] |= (uint32_t)tile[part * 16 + q][row] << ((q & 3) * 8);
    const int r = k0 + row, n = n0 + part * 16;
    *reinterpret_cast<u32x4*>(wt + (int64_t)e * N * K + ((int64_t)(r / 16) * (N / 128) + n / 128) * 2048 +
                              (r % 16) * 128 + n % 128) = (u32x4){o[0], o[1], o[2], o[3]};
    __syncthreads();
  }
}

// Group scales [E][G][L] (G groups of the transposed copy's rows, L along its
// K) -> per 8 consecutive K values four fp16 pairs {s0, s4}, {s1, s5},
// {s2, s6}, {s3, s7}; INT4 bf16 scales are converted as they are, MXFP4
// turns E8M0 bytes into 2^(e-127), NVFP4 E4M3 bytes into their
// values (exact in fp16: at most 448, at least 2^-9).
template <int FMT>
__global__ __launch_bounds__(256) void k_repack_scales_f16(const void* __restrict__ s, int64_t n8,
                                                           u32x4* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    float f[8];
    if (FMT == FMT_INT4) {
      const u32x4 v = reinterpret_cast<const u32x4*>(s)[i];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = bf16_bits_to_f32((w[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu);
    } else {
      const uint2 v = reinterpret_cast<const uint2*>(s)[i];
      const uint32_t w[2] = {v.x, v.y};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t e = (w[j >> 2] >> ((j & 3) * 8)) & 0xFFu;
        f[j] = FMT == FMT_NVFP4 ? e4m3_to_f32(e) : __uint_as_float(e ? e << 23 : 0x00400000u);
      }
    }
    u32x4 o;
    o.x = pack_f16x2(f[0], f[4]);
    o.y = pack_f16x2(f[1], f[5]);
    o.z = pack_f16x2(f[2], f[6]);
    o.w = pack_f16x2(f[3], f[7]);
    out[i] = o;
  }
}

// FP8 block scales [E][NB][KB] -> [E][KB][NB].
__global__ __launch_bounds__(256) void k_repack_scales_t(const float* __restrict__ s, int E, int NB, int KB,
                                                         float* __restrict__ st) {
  const int64_t n = (int64_t)E * NB * KB;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t e = i / ((int64_t)NB * KB);
    const int r = (int)(i - e * NB * KB), nb = r / KB, kb = r % KB;
    st[e * NB * KB + (int64_t)kb * NB + nb] = s[i];
  }
}

static unsigned grid_of(int64_t n, int64_t cap) { return (unsigned)((n + 255) / 256 < cap ? (n + 255) / 256 : cap); }

void launch_repack_bwd(int fmt, const uint8_t* w, const void* s, int E, int N, int K, bool tiled, uint8_t* wt,
                       void* st, hipStream_t stream) {
  const int64_t tiles = (int64_t)E * (N / 64) * (K / 64);
  const unsigned tg = (unsigned)(tiles < 8192 ? tiles : 8192);
  if (fmt == FMT_FP8) {
    hipLaunchKernelGGL(k_repack_u8_t, dim3(tg), dim3(256), 0, stream, w, E, N, K, tiled ? 1 : 0, wt);
    const int64_t n = (int64_t)E * (N / 128) * (K / 128);
    hipLaunchKernelGGL(k_repack_scales_t, dim3(grid_of(n, 4096)), dim3(256), 0, stream, static_cast<const float*>(s),
                       E, N / 128, K / 128, static_cast<float*>(st));
    return;
  }
  hipLaunchKernelGGL(k_repack_int4_t, dim3(tg), dim3(256), 0, stream, w, E, N, K, tiled ? 1 : 0, wt);
  const int64_t n8 = (int64_t)E * N * K / (fmt == FMT_NVFP4 ? 16 : 32) / 8;
  if (fmt == FMT_NVFP4)
    hipLaunchKernelGGL(k_repack_scales_f16<FMT_NVFP4>, dim3(grid_of(n8, 4096)), dim3(256), 0, stream, s, n8,
                       reinterpret_cast<u32x4*>(st));
  else if (fmt == FMT_INT4)
    hipLaunchKernelGGL(k_repack_scales_f16<FMT_INT4>, dim3(grid_of(n8, 4096)), dim3(256), 0, stream, s, n8,
                       reinterpret_cast<u32x4*>(st));
  else
    hipLaunchKernelGGL(k_repack_scales_f16<FMT_MXFP4>, dim3(grid_of(n8, 4096)), dim3(256), 0, stream, s, n8,
                       reinterpret_cast<u32x4*>(st));
}

// ------------------------------------------------------------ unpacking

// 8 E2M1 codes (nibble i = element i, sign bit 3) times per-element fp16
// scales (pairs {s0, s4}, {s1, s5}, {s2, s6}, {s3, s7}) -> fp16 in the order
// 0,4,1,5,2,6,3,7.  The magnitude's fp16 high byte comes from an 8-entry byte
// table with one byte permute per pair (its low byte is always zero); the
// sign bit moves to bit 15 / 31.  E2M1 times a power of two is exact.
MOE_DEV uint32_t e2m1_pair(uint32_t w, int sh) {
  // elements at nibbles (sh/4) and (sh/4 + 4): magnitude indices into bytes 1 and 3
  const uint32_t sel = 0x000C000Cu | (((w >> sh) << 8) & 0x07000700u);
  const uint32_t mag = __builtin_amdgcn_perm(0x46444240u, 0x3E3C3800u, sel);
  return mag | (((w >> sh) << 12) & 0x80008000u);
}
MOE_DEV f16x8 e2m1x8_to_f16_se(uint32_t w, const u32x4& sc) {
  const uint32_t s0 = sc.x, s1 = sc.y, s2 = sc.z, s3 = sc.w;  // scalar copies (see int4.h)
  const f16x2 h0 = __builtin_bit_cast(f16x2, e2m1_pair(w, 0)) * __builtin_bit_cast(f16x2, s0);
  const f16x2 h1 = __builtin_bit_cast(f16x2, e2m1_pair(w, 4)) * __builtin_bit_cast(f16x2, s1);
  const f16x2 h2 = __builtin_bit_cast(f16x2, e2m1_pair(w, 8)) * __builtin_bit_cast(f16x2, s2);
  const f16x2 h3 = __builtin_bit_cast(f16x2, e2m1_pair(w, 12)) * __builtin_bit_cast(f16x2, s3);
  f16x8 r = {h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
  return r;
}

// 8 E4M3 codes (bytes 0..7 of lo, hi) times the block scale s = p2 * m
// (p2 a power of two, applied exactly by the conversion; m in [1, 2) as
// fp16) -> fp16 in the order 0,4,1,5,2,6,3,7.
MOE_DEV f16x8 e4m3x8_to_f16(uint32_t lo, uint32_t hi, float p2, f16x2 m2) {
  const uint32_t q04_15 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // bytes e0 e4 e1 e5
  const uint32_t q26_37 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // bytes e2 e6 e3 e7
  const f16x2 h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(q04_15, p2, false) * m2;
  const f16x2 h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(q04_15, p2, true) * m2;
  const f16x2 h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(q26_37, p2, false) * m2;
  const f16x2 h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(q26_37, p2, true) * m2;
  f16x8 r = {h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
  return r;
}

// ------------------------------------------------------------ backward GEMM

// LDS of one stage: activation rows (fp16, 256 B each, 16-byte parts
// XOR-swizzled by row), each wave's weight fragments (4 subtiles x 16 rows x
// 64 B of nibbles or 128 B of E4M3 codes) and, for INT4 / MXFP4, the fp16
// scales of the wave's 64 weight rows for the step (2 row groups x 128 K;
// NVFP4 4 row groups of 16).
template <int FMT, int BM>
struct BwStage {
  static constexpr int NA = BM / 16;                      // activation DMAs per wave
  static constexpr int A_BYTES = BM * 256;
  static constexpr int B_OFF = A_BYTES;
  static constexpr int NB = FMT == FMT_FP8 ? 8 : 4;       // weight DMAs per wave
  static constexpr int BS_OFF = B_OFF + 4 * NB * 1024;
  static constexpr int BS = FMT == FMT_FP8 ? 0 : FMT == FMT_NVFP4 ? 4 * 1024 : 4 * 512;
  static constexpr int BYTES = BS_OFF + BS;
  static constexpr int WPC = (FMT != FMT_FP8 && (BM == 16 || BM == 48 || BM == 64)) ? 2 : 1;
  static constexpr int SMAX = BM <= 32 ? 7 : 5;
  static constexpr int S = (152 * 1024 / WPC) / BYTES > SMAX ? SMAX : (152 * 1024 / WPC) / BYTES;
  static constexpr int NPER = NA + NB + (FMT == FMT_FP8 ? 0 : 1);
};

// The row's h value at column col as the forward fed it to GEMM2.
template <int FMT>
MOE_DEV float fwd_h(const GemmArgs& p, int r, int col, float a, float b, float sg) {
  if (FMT == FMT_INT4 || FMT == FMT_NVFP4) return a * sg * b;
  const float q = e4m3_to_f32(p.hq[(int64_t)r * p.inter + col]);
  const char* sr = static_cast<const char*>(p.hsc) + (int64_t)r * p.hsc_stride;
  if (FMT == FMT_FP8) return q * reinterpret_cast<const float*>(sr)[col / 128];
  const uint32_t e = reinterpret_cast<const uint8_t*>(sr)[col / 32];
  return q * __uint_as_float(e ? e << 23 : 0x00400000u);
}

template <int FMT, int BM, bool DH>
__device__ __forceinline__ void bwd_item(const GemmArgs& p, const Tile& tl, uint8_t* smem, float* red,
                                         float* wsc) {
  constexpr int MT = BM / 16;
  using ST = BwStage<FMT, BM>;
  constexpr int S = ST::S;
  constexpr int BROW = FMT == FMT_FP8 ? 128 : 64;  // weight bytes per row and K step
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int ln = lane & 15, lg = lane >> 4;
  const int K = p.K, KT = K / 128;
  const char* Abase = static_cast<const char*>(p.a);
  const uint32_t smem0 = lds_u32(smem);
  lds_barrier();  // every wave is done with the previous item's stages
  const int c0 = tl.nb * 256 + wave * 64;
  const char* wexp = reinterpret_cast<const char*>(p.w) + tl.e * p.w_expert_bytes;
  // weight fragments: lane holds 32 consecutive K values of row c0 + 16 i + ln
  // (the copy is tiled 16 rows x 128 K, BROW bytes per row and tile)
  const char* bsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    bsrc[i] = wexp + (int64_t)((c0 + 16 * i) / 16) * KT * (16 * BROW) + ln * BROW + lg * (BROW / 4);
  const char* bssrc = nullptr;
  if (FMT == FMT_NVFP4) {
    // fp16 scales of the wave's four 16-row groups: 4 runs of 128 K values per step
    const char* sexp = static_cast<const char*>(p.w_scale) + tl.e * p.ws_expert_elems * 2;
    bssrc = sexp + ((int64_t)(c0 / 16 + (lane >> 4)) * K + (lane & 15) * 8) * 2;
  } else if (FMT != FMT_FP8) {
    // fp16 scales of the wave's two row groups: 2 runs of 128 K values per step
    const char* sexp = static_cast<const char*>(p.w_scale) + tl.e * p.ws_expert_elems * 2;
    bssrc = sexp + ((int64_t)(c0 / 32 + ((lane >> 4) & 1)) * K + (lane & 15) * 8) * 2;
  } else if (wave < 2 && lane < KT) {
    // block scales of the item's two 128-row blocks, one per K step, for the whole item
    // (transposed block scales are [N/128][K/128] per expert: a row block's K run is contiguous)
    const float* sexp = static_cast<const float*>(p.w_scale) + tl.e * p.ws_expert_elems;
    dma_b32(sexp + (int64_t)(tl.nb * 2 + wave) * KT + lane, lds_u32(wsc) + wave * 256);
  }
  const char* asrc[ST::NA];
#pragma unroll
  for (int j = 0; j < ST::NA; ++j) {
    const int c = (wave * ST::NA + j) * 64 + lane;   // activation piece: row c/16, slot c%16
    const int row = c >> 4, slot = c & 15;
    const int part = slot ^ (row & 15);              // XOR swizzle of 16-byte parts
    const int rr = tl.rbase + min(row, tl.nrows - 1);
    const int src = p.a_per_token ? p.sorted_rows[rr] / p.top_k : rr;
    asrc[j] = Abase + (int64_t)src * K * 2 + part * 16;
  }
  auto issue = [&](int kt, int slot) {
    const uint32_t sb = smem0 + slot * ST::BYTES;
#pragma unroll
    for (int j = 0; j < ST::NA; ++j) dma_b128(asrc[j] + kt * 256, sb + (wave * ST::NA + j) * 1024);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < ST::NB / 4; ++h)
        dma_b128(bsrc[i] + kt * (16 * BROW) + h * 16, sb + ST::B_OFF + ((wave * 4 + i) * (ST::NB / 4) + h) * 1024);
    if (FMT == FMT_NVFP4) dma_b128(bssrc + (int64_t)kt * 256, sb + ST::BS_OFF + wave * 1024);
    else if (FMT != FMT_FP8)
      if (lane < 32) dma_b128(bssrc + (int64_t)kt * 256, sb + ST::BS_OFF + wave * 512);
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
    wait_stages<ST::NPER>(min(S - 2, KT - 1 - kt));
    lds_barrier();
    if (kt + S - 1 < KT) issue(kt + S - 1, (kt + S - 1) % S);
    const uint8_t* st = smem + (kt % S) * ST::BYTES;
    u32x4 bq[4][ST::NB / 4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < ST::NB / 4; ++h)
        bq[i][h] = *reinterpret_cast<const u32x4*>(st + ST::B_OFF + ((wave * 4 + i) * (ST::NB / 4) + h) * 1024 +
                                                    lane * 16);
    float p2 = 1.0f;
    f16x2 m2 = {(_Float16)1.0f, (_Float16)1.0f};
    if (FMT == FMT_FP8) {
      // the wave's 64 rows lie in one 128-row block: s = 2^e * m, m in [1, 2)
      const float s = wsc[(wave >> 1) * 64 + kt];
      p2 = __uint_as_float(__float_as_uint(s) & 0x7F800000u);
      const _Float16 mh = (_Float16)(s / p2);
      m2 = (f16x2){mh, mh};
    }
    auto read_a = [&](int m, int s) {
      const int r = m * 16 + ln;
      return *reinterpret_cast<const f16x8*>(st + r * 256 + (((4 * lg + s) ^ (r & 15)) << 4));
    };
    // Sub-step s (32 K) runs its MFMAs while the VALU unpacks the weights of
    // sub-step s + 1 and the activation fragments of sub-step s + 1 are
    // read: the scheduling groups alternate one MFMA with a few VALU
    // instructions, so the unpack hides behind the matrix core.
    auto unpack = [&](int s, f16x8 (&bf)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (FMT == FMT_FP8) {
          // K values 32 lg + 8 s .. +7: bytes 8 s .. 8 s + 7 of the lane's 32
          const u32x4& q = bq[i][s >> 1];
          const uint32_t lo = (s & 1) ? q.z : q.x, hi = (s & 1) ? q.w : q.y;
          bf[i] = e4m3x8_to_f16(lo, hi, p2, m2);
        } else {
          // K values 32 lg + 8 s .. +7 of weight row c0 + 16 i + ln: row group i / 2 (NVFP4: i), octet 4 lg + s
          const int soff = FMT == FMT_NVFP4 ? wave * 1024 + i * 256 : wave * 512 + (i >> 1) * 256;
          const u32x4 sc = *reinterpret_cast<const u32x4*>(st + ST::BS_OFF + soff + (4 * lg + s) * 16);
          bf[i] = FMT == FMT_INT4 ? int4x8_to_f16_se(dword_of(bq[i][0], s), sc)
                                  : e2m1x8_to_f16_se(dword_of(bq[i][0], s), sc);
        }
      }
    };
    f16x8 af[2][MT];
    f16x8 bf[2][4];
#pragma unroll
    for (int m = 0; m < MT; ++m) af[0][m] = read_a(m, 0);
    unpack(0, bf[0]);
    __builtin_amdgcn_s_setprio(1);  // the MFMA phase at raised wave priority
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      if (s + 1 < 4) {
#pragma unroll
        for (int m = 0; m < MT; ++m) af[(s + 1) & 1][m] = read_a(m, s + 1);
        unpack(s + 1, bf[(s + 1) & 1]);
      }
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[m][i] = mfma_f16_16x16x32(af[s & 1][m], bf[s & 1][i], acc[m][i]);
      if (s + 1 < 4) {
        // one MFMA, then the next sub-step's LDS reads and VALU work between MFMAs
#pragma unroll
        for (int j = 0; j < MT * 4; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (j < MT + 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  }
  if constexpr (FMT == FMT_NVFP4) {
    const float gs = ld_uniform_f32(p.gscale + tl.e);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[m][i] *= gs;
  }

  if (DH) {
    // SwiGLU backward per (row, column); columns are h indices i < I
    const int I = p.inter;
    _Float16* dAB = static_cast<_Float16*>(p.out);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = m * 16 + lg * 4 + v;
        float gp = 0.0f;
        if (row < tl.nrows) {
          const int r = tl.rbase + row;
          const float w = p.topk_w[p.sorted_rows[r]];
          const float* abr = p.ab + (int64_t)r * 2 * I;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int col = c0 + 16 * i + ln;
            const float u = acc[m][i][v];
            const float a = abr[col], b = abr[I + col];
            const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-a));
            gp += u * fwd_h<FMT>(p, r, col, a, b, sg);
            const float dh = w * u;
            dAB[(int64_t)r * 2 * I + i4act_pos(col)] = (_Float16)(dh * b * sg * (1.0f + a * (1.0f - sg)));
            dAB[(int64_t)r * 2 * I + I + i4act_pos(col)] = (_Float16)(dh * a * sg);
          }
        }
        // sum over the 16 lanes of this row (its 64 columns in this wave)
        gp += shfl_xor(gp, 1);
        gp += shfl_xor(gp, 2);
        gp += shfl_xor(gp, 4);
        gp += shfl_xor(gp, 8);
        if (ln == 0) red[wave * BM + row] = gp;
      }
    lds_barrier();
    for (int row = threadIdx.x; row < tl.nrows; row += 256)
      p.gpart[(int64_t)(tl.rbase + row) * (I / 256) + tl.nb] =
          red[row] + red[BM + row] + red[2 * BM + row] + red[3 * BM + row];
  } else {
    float* dX = static_cast<float*>(p.out);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = m * 16 + lg * 4 + v;
        if (row < tl.nrows) {
#pragma unroll
          for (int i = 0; i < 4; ++i) dX[(int64_t)(tl.rbase + row) * p.N + c0 + 16 * i + ln] = acc[m][i][v];
        }
      }
  }
}

// One launch: chunk p1.chunk's dh items and chunk p2.chunk's dx' items
// (either may be empty), dealt through per-XCD atomic counters.
template <int FMT, int BM>
__global__ __launch_bounds__(256, (BwStage<FMT, BM>::WPC)) void k_gemm_bwd(GemmArgs p1, GemmArgs p2,
                                                                           int32_t* queue) {
  using ST = BwStage<FMT, BM>;
  constexpr int S = ST::S;
  static_assert(S >= 2 && S <= 7, "LDS stages");
  static_assert(FMT != FMT_FP8 || S * ST::BYTES + 4 * BM * 4 + 512 <= 160 * 1024, "LDS budget");
  __shared__ __align__(16) uint8_t smem[S * ST::BYTES];
  __shared__ float red[4 * BM];
  __shared__ float wsc[FMT == FMT_FP8 ? 128 : 1];  // FP8: the item's block scales, 2 x 64
  __shared__ int s_item;
  ChunkWork c1, c2;
  const int n1 = chunk_work(p1, p1.N / 256, c1) ? c1.nwork : 0;
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
    if (cur < len1) bwd_item<FMT, BM, true>(p1, tile_of(p1, c1, b1 + cur, BM), smem, red, wsc);
    else bwd_item<FMT, BM, false>(p2, tile_of(p2, c2, b2 + cur - len1, BM), smem, red, wsc);
    if (threadIdx.x == 0) s_item = nxt;
    lds_barrier();
    cur = s_item;
  }
}

template <int FMT, int BM>
static void launch_bwd_bm(const GemmArgs& g1, const GemmArgs& g2, int32_t* queue, int grid, hipStream_t s) {
  if constexpr (BwStage<FMT, BM>::S >= 2) launch_persistent2<k_gemm_bwd<FMT, BM>>(g1, g2, queue, grid, s);
}

// Tile heights whose stage ring does not fit (FP8 at 192 rows) are never
// requested: the host caps the backward's tile height for FP8 at 128.
template <int FMT>
static void launch_bwd(const GemmArgs& g1, const GemmArgs& g2, int32_t* queue, int bm, int grid, hipStream_t s) {
  switch (bm) {
    case 16: launch_bwd_bm<FMT, 16>(g1, g2, queue, grid, s); break;
    case 32: launch_bwd_bm<FMT, 32>(g1, g2, queue, grid, s); break;
    case 48: launch_bwd_bm<FMT, 48>(g1, g2, queue, grid, s); break;
    case 64: launch_bwd_bm<FMT, 64>(g1, g2, queue, grid, s); break;
    case 96: launch_bwd_bm<FMT, 96>(g1, g2, queue, grid, s); break;
    case 128: launch_bwd_bm<FMT, 128>(g1, g2, queue, grid, s); break;
    default: launch_bwd_bm<FMT, 192>(g1, g2, queue, grid, s); break;
  }
}

void launch_gemm_bwd_pair(int fmt, const GemmArgs& g1, const GemmArgs& g2, int32_t* queue, int bm, int grid,
                          hipStream_t s) {
  if (fmt == FMT_INT4) launch_bwd<FMT_INT4>(g1, g2, queue, bm, grid, s);
  else if (fmt == FMT_FP8) launch_bwd<FMT_FP8>(g1, g2, queue, bm, grid, s);
  else if (fmt == FMT_NVFP4) launch_bwd<FMT_NVFP4>(g1, g2, queue, bm, grid, s);
  else launch_bwd<FMT_MXFP4>(g1, g2, queue, bm, grid, s);
}

}  // namespace moe
