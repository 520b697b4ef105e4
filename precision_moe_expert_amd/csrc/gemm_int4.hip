// Grouped expert GEMMs for 4-bit weights with 16-bit activations on gfx950:
// INT4 group-32 (bf16 scales) and NVFP4 (E2M1 values, an E4M3 scale per 16
// along K, an fp32 second-level scale per expert matrix).
//
// Dequantization (Orbit announcement, 技术细节: the active experts' weights
// are dequantized temporarily for the grouped GEMM) happens in registers:
// each lane unpacks its own 32 nibbles per 128-K step and multiplies by the
// group's scale in fp16.  Every INT4 code times a bf16 group scale in
// [2^-17, 8188] is exact in fp16 (at most 3 + 8 significant bits), so the
// MFMA sees w = q*s exactly;
// nothing is written back to memory and no dequantized copy exists.
//
// Tile: BM rows x 256 output columns per workgroup (4 waves x 4 subtiles of
// 16 columns); K step 128.  Activation rows, weight nibbles and group scales
// stream into an LDS stage ring by global_load_lds DMA (see the FP8 kernel
// for the scheme); each wave unpacks its own weight fragments from LDS.
// GEMM1 pairs gate column n with up column I + n inside the same wave and
// writes h = silu(gate) * up (fp16); GEMM2 writes y (bf16).
#include "common.h"
#include "kernels.h"
#include "moe_sched.h"
#include "int4.h"

namespace moe {

// NVFP4: 8 E2M1 codes (element i in bits 4i..4i+3) times the block scale s
// -> 8 fp16 in natural order.  The hardware conversion decodes each byte's
// two codes exactly (its scale operand takes only a power of two, so 1.0);
// q * s is exact in fp16 (at most 2 + 4 significant bits).
MOE_DEV f16x8 e2m1x8_to_f16(uint32_t w, f16x2 s2) {
  const f16x2 h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  const f16x2 h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  const f16x2 h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  const f16x2 h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  f16x8 r = {h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
  return r;
}

// One work item: a BM-row tile times one N block.  Each wave owns NS
// subtiles of 16 columns: GEMM1 items cover NS*32 h columns (NS*32 gate +
// NS*32 up weight rows), GEMM2 items NS*64 output columns.  NS = 4, except
// for the 16-row tiles of decode-sized batches, whose items take NS = 2:
// there an item streams a weight slice that no other item of its tile
// shares, and halving it halves the idle time at the end of each launch
// (a workgroup's last item then ends at most half as late as the others).
// NV: NVFP4 weights (activations and h in natural order, results times the
// expert's second-level scale); else INT4 (activations and h in the unpack
// order).
// KS: K per pipeline stage, 128 or (INT4) 64; a stage runs KS/32 MFMA
// sub-steps of 32 K.
template <int BM, bool G1, bool NV, int NS, int KS>
__device__ __forceinline__ void i4_item(const GemmArgs& p, const Tile& tl, uint8_t* smem) {
  static_assert(NS == 4 || (NS == 2 && !NV), "subtiles per wave");
  constexpr int MT = BM / 16;
  using ST = I4Stage<BM, NS, KS>;
  constexpr bool K64 = ST::K64;
  constexpr int NSUB = KS / 32;
  constexpr int S = ST::S;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int ln = lane & 15, lg = lane >> 4;
  const int K = p.K, KT = K / KS;
  const char* Abase = static_cast<const char*>(p.a);
  const uint32_t smem0 = lds_u32(smem);
  lds_barrier();  // every wave is done with the previous item's stages
  // subtile i's 16 weight rows start at col[i]; GEMM1: the first NS/2 are
  // gate rows, the rest the matching up rows (I + the same h columns)
  int col[NS];
  if (G1) {
    const int g0 = tl.nb * (NS * 32) + wave * (NS * 8);
#pragma unroll
    for (int i = 0; i < NS / 2; ++i) {
      col[i] = g0 + 16 * i;
      col[NS / 2 + i] = p.inter + g0 + 16 * i;
    }
  } else {
    const int c0 = tl.nb * (NS * 64) + wave * (NS * 16);
#pragma unroll
    for (int i = 0; i < NS; ++i) col[i] = c0 + 16 * i;
  }
  // per-lane global sources of this item's DMA pieces (K offset added per step)
  const char* wexp = reinterpret_cast<const char*>(p.w) + tl.e * p.w_expert_bytes;
  const char* sexp = static_cast<const char*>(p.w_scale) + tl.e * p.ws_expert_elems * (NV ? 1 : 2);
  // 128-K steps: DMA i moves subtile i, lane (ln, lg) the 16 bytes (32 K)
  // that it feeds to the MFMA.  64-K steps: DMA j moves subtiles 2j and
  // 2j+1, lane L the 16 bytes of row (L/2)%16 holding K [32 q, 32 q + 32),
  // q = L%2, of subtile 2j + L/32: the fragments of lanes (row, 2q) and
  // (row, 2q + 1), 8 bytes each.
  constexpr int NB = K64 ? NS / 2 : NS;
  const char* bsrc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    int c, r, part;  // first weight row of the subtile, row in it, 16-byte part of its 64-byte K block
    if constexpr (K64) {
      c = (lane >> 5) ? col[2 * i + 1] : col[2 * i];
      r = (lane >> 1) & 15;
      part = lane & 1;
    } else {
      c = col[i];
      r = ln;
      part = lg;
    }
    bsrc[i] = p.w_kblocked ? wexp + (int64_t)(c / 16) * (K / 128) * 1024 + r * 64 + part * 16
                           : wexp + (int64_t)(c + r) * (K / 2) + part * 16;
  }
  // bytes from step 0 to step kt of one lane's piece
  auto boff = [&](int kt) -> int64_t {
    if (K64) return p.w_kblocked ? (int64_t)(kt >> 1) * 1024 + (kt & 1) * 32 : (int64_t)kt * 32;
    return (int64_t)kt * (p.w_kblocked ? 1024 : 64);
  };
  // group scales: INT4 lane l < (KS/32)*2*NS takes 8 consecutive weight rows
  // (bf16) of 32-group l/(2*NS); NVFP4 lane l < KS/4 takes 16 consecutive
  // rows (E4M3 bytes) of 16-group l/4.  Either way 16 bytes, NS*KS per wave
  // and step.
  constexpr int PCN = 2 * NS;  // INT4: 16-byte scale pieces per group and wave
  const char* bssrc;
  if constexpr (NV) {
    const int g = (lane >> 2) & (K64 ? 3 : 7), pc = lane & 3;
    const int c = G1 ? (pc < 2 ? col[0] + pc * 16 : col[2] + (pc - 2) * 16) : col[0] + pc * 16;
    bssrc = sexp + (int64_t)g * p.N + c;
  } else {
    const int g = (lane / PCN) & (K64 ? 1 : 3), pc = lane % PCN;
    const int c = G1 ? (pc < NS ? col[0] + pc * 8 : col[NS / 2] + (pc - NS) * 8) : col[0] + pc * 8;
    bssrc = sexp + ((int64_t)g * p.N + c) * 2;
  }
  const char* asrc[ST::NA];
#pragma unroll
  for (int j = 0; j < ST::NA; ++j) {
    // activation piece: row c/PPR, slot c%PPR (PPR 16-byte parts per row and step)
    constexpr int PPR = KS / 8;
    const int c = (wave * ST::NA + j) * 64 + lane;
    const int row = c / PPR, slot = c % PPR;
    const int part = slot ^ (row % PPR);             // XOR swizzle of 16-byte parts
    const int rr = tl.rbase + min(row, tl.nrows - 1);
    const int sr = p.sorted_rows[rr];
    const int src = p.a_per_token ? sr / p.top_k : rr;
    asrc[j] = Abase + (int64_t)src * K * 2 + part * 16;
  }
  auto issue = [&](int kt, int slot) {
    const uint32_t sb = smem0 + slot * ST::BYTES;
#pragma unroll
    for (int j = 0; j < ST::NA; ++j) dma_b128(asrc[j] + kt * (KS * 2), sb + (wave * ST::NA + j) * 1024);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      // a 16-row tile's weight slice is read by no other item: non-temporal
      if constexpr (BM == 16) dma_b128_nt(bsrc[i] + boff(kt), sb + ST::B_OFF + (wave * NB + i) * 1024);
      else dma_b128(bsrc[i] + boff(kt), sb + ST::B_OFF + (wave * NB + i) * 1024);
    }
    // KS/16 * N scale bytes per step: 8 N for 128 K either way, 4 N for 64 K
    if (lane < (NV ? KS / 4 : (KS / 32) * PCN))
      dma_b128(bssrc + (int64_t)kt * (KS / 16) * p.N, sb + ST::BS_OFF + wave * (NS * KS));
  };
  f32x4 acc[MT][NS];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < NS; ++i) acc[m][i] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
  for (int s = 0; s + 1 < S; ++s)
    if (s < KT) issue(s, s);
  for (int kt = 0; kt < KT; ++kt) {
    wait_stages<ST::NPER>(min(S - 2, KT - 1 - kt));  // this wave's pieces of stage kt have landed
    lds_barrier();                                    // ... and every other wave's
    if (kt + S - 1 < KT) issue(kt + S - 1, (kt + S - 1) % S);
    const uint8_t* st = smem + (kt % S) * ST::BYTES;
    u32x4 bq[NS];
    f16x2 s2[NS], s2_16[NS];  // NVFP4: the scales of 16-groups 2 lg and 2 lg + 1
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if constexpr (K64) {
        const u32x2 b2 = *reinterpret_cast<const u32x2*>(st + ST::B_OFF + (wave * NB + (i >> 1)) * 1024 +
                                                         ((i & 1) * 32 + ln * 2 + (lg >> 1)) * 16 + (lg & 1) * 8);
        bq[i] = (u32x4){b2.x, b2.y, 0u, 0u};
      } else {
        bq[i] = *reinterpret_cast<const u32x4*>(st + ST::B_OFF + (wave * NS + i) * 1024 + lane * 16);
      }
      if constexpr (NV) {
        // E4M3 scales of the lane's 16-groups: 2 lg and 2 lg + 1 of a 128-K
        // step (sub-steps 0-1 and 2-3), lg of a 64-K step (both sub-steps)
        const uint8_t* sr = st + ST::BS_OFF + wave * (NS * KS) + i * 16 + ln;
        const uint32_t codes = K64 ? (uint32_t)sr[lg * 64]
                                   : (uint32_t)sr[(2 * lg) * 64] | ((uint32_t)sr[(2 * lg + 1) * 64] << 8);
        const f16x2 sv = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes, 1.0f, false);
        s2[i] = (f16x2){sv[0], sv[0]};
        s2_16[i] = (f16x2){sv[1], sv[1]};
      } else {
        // the lane's 32-group: lg of four (128-K steps), lg/2 of two (64-K steps)
        const uint16_t sw = *reinterpret_cast<const uint16_t*>(st + ST::BS_OFF + wave * (NS * KS) +
                                                               (K64 ? lg >> 1 : lg) * (PCN * 16) +
                                                               (2 * i + (ln >> 3)) * 16 + (ln & 7) * 2);
        const _Float16 sh = (_Float16)bf16_bits_to_f32(sw);
        s2[i] = (f16x2){sh, sh};
      }
    }
    // activation fragment of row block m, 32-K sub-step s: logical part
    // NSUB*lg + s (the lane's weight fragment covers K [32 lg, 32 lg + 32) of
    // a 128-K step, [16 lg, 16 lg + 16) of a 64-K step)
    auto read_a = [&](int m, int s) {
      constexpr int PPR = KS / 8;
      const int r = m * 16 + ln;
      return *reinterpret_cast<const f16x8*>(st + r * (KS * 2) + (((NSUB * lg + s) ^ (r % PPR)) << 4));
    };
    // Sub-step s (32 K) runs its MFMAs while the VALU unpacks the weights of
    // sub-step s + 1 and the activation fragments of sub-step s + 1 are
    // read: the scheduling groups below alternate one MFMA with a few VALU
    // instructions, so the unpack hides behind the matrix core instead of
    // preceding it (Kimi-K2 shape: 7.52 -> 7.39 ms of GEMM).
    auto unpack = [&](int s, f16x8 (&bf)[NS]) {
#pragma unroll
      for (int i = 0; i < NS; ++i)
        bf[i] = NV ? e2m1x8_to_f16(dword_of(bq[i], s), s < 2 ? s2[i] : s2_16[i])
                   : int4x8_to_f16(dword_of(bq[i], s), s2[i]);
    };
    f16x8 af[2][MT];
    f16x8 bf[2][NS];
#pragma unroll
    for (int m = 0; m < MT; ++m) af[0][m] = read_a(m, 0);
    unpack(0, bf[0]);
    // the MFMA phase at raised wave priority (Kimi-K2 shape 4% faster: the
    // SIMD's other wave, of the other workgroup, issues behind it)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      if (s + 1 < NSUB) {
#pragma unroll
        for (int m = 0; m < MT; ++m) af[(s + 1) & 1][m] = read_a(m, s + 1);
        unpack(s + 1, bf[(s + 1) & 1]);
      }
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < NS; ++i) acc[m][i] = mfma_f16_16x16x32(af[s & 1][m], bf[s & 1][i], acc[m][i]);
      if (s + 1 < NSUB) {
        // one MFMA, then the next sub-step's LDS reads and VALU work between MFMAs
#pragma unroll
        for (int j = 0; j < MT * NS; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (j < MT) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  }

  // Epilogue: results go through LDS (the stage buffers are free once every
  // wave has passed the barrier below) so that global stores are 16 B per lane.
  // NVFP4 results take the expert matrix's second-level scale here.
  if constexpr (NV) {
    const float gs = ld_uniform_f32(p.gscale + tl.e);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < NS; ++i) acc[m][i] *= gs;
  }
  lds_barrier();
  if (G1 && p.save_ab) {
    // backward recompute: the gate and up pre-activations in fp32, each at its W13 row index
    float* AB = static_cast<float*>(p.out);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m * 16 + lg * 4 + i;
        if (row < tl.nrows) {
#pragma unroll
          for (int n = 0; n < NS; ++n) AB[(int64_t)(tl.rbase + row) * p.N + col[n] + ln] = acc[m][n][i];
        }
      }
  } else if (G1) {
    constexpr int HS = NS * 64 + 16;  // staged row stride (bytes) of the NS*32 fp16 h values
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m * 16 + lg * 4 + i;
#pragma unroll
        for (int n = 0; n < NS / 2; ++n) {
          const float hv = silu_f32(acc[m][n][i]) * acc[m][n + NS / 2][i];
          const _Float16 hh = (_Float16)hv;
          // h is stored in the activation order that GEMM2's unpack expects
          const int c = wave * (NS * 8) + n * 16 + ln;
          *reinterpret_cast<uint16_t*>(smem + row * HS + (NV ? c : i4act_pos(c)) * 2) =
              __builtin_bit_cast(uint16_t, hh);
        }
      }
    lds_barrier();
    copy_out_rows<BM, NS * 64, HS, 256, 1>(smem, static_cast<char*>(p.out) + (int64_t)tl.nb * (NS * 64) +
                                                       (int64_t)tl.rbase * p.inter * 2,
                                           (int64_t)p.inter * 2, tl.nrows);
  } else {
    constexpr int YS = NS * 128 + 16;  // staged row stride (bytes) of the NS*64 bf16 outputs
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m * 16 + lg * 4 + i;
#pragma unroll
        for (int n = 0; n < NS; ++n)
          *reinterpret_cast<uint16_t*>(smem + row * YS + (wave * (NS * 16) + n * 16 + ln) * 2) =
              (uint16_t)f32_to_bf16_bits(acc[m][n][i]);
      }
    lds_barrier();
    copy_out_rows<BM, NS * 128, YS, 256, (BM <= 128 ? 4 : 1)>(smem, static_cast<char*>(p.out) +
                                                                      (int64_t)tl.nb * (NS * 128) +
                                                                      (int64_t)tl.rbase * p.N * 2,
                                                              (int64_t)p.N * 2, tl.nrows);
  }
}

// Persistent pair launch: the GEMM1 items of chunk p1.chunk and the GEMM2
// items of chunk p2.chunk (either may be empty), dealt through per-XCD
// atomic work counters exactly as for the FP8 weights.
template <int BM, bool NV, int NS, int KS>
__device__ __forceinline__ void w4_pair(const GemmArgs& p1, const GemmArgs& p2, int32_t* queue) {
  using ST = I4Stage<BM, NS, KS>;
  constexpr int S = ST::S;
  static_assert(S >= 2 && S <= 7, "LDS stages");
  __shared__ __align__(16) uint8_t smem[S * ST::BYTES];
  static_assert(S * ST::BYTES >= BM * (NS * 128 + 16), "epilogue staging fits in the stage buffers");
  __shared__ int s_item;
  ChunkWork c1, c2;
  const int n1 = chunk_work(p1, p1.inter / (NS * 32), c1) ? c1.nwork : 0;
  const int n2 = chunk_work(p2, p2.N / (NS * 64), c2) ? c2.nwork : 0;
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
    if (cur < len1) i4_item<BM, true, NV, NS, KS>(p1, tile_of(p1, c1, b1 + cur, BM), smem);
    else i4_item<BM, false, NV, NS, KS>(p2, tile_of(p2, c2, b2 + cur - len1, BM), smem);
    if (threadIdx.x == 0) s_item = nxt;
    lds_barrier();
    cur = s_item;
  }
}

template <int BM, int NS, int KS>
__global__ __launch_bounds__(256, (I4Stage<BM, NS, KS>::WPC)) void k_gemm_int4(GemmArgs p1, GemmArgs p2,
                                                                            int32_t* queue) {
  w4_pair<BM, false, NS, KS>(p1, p2, queue);
}

template <int BM, int KS>
__global__ __launch_bounds__(256, (I4Stage<BM, 4, KS>::WPC)) void k_gemm_nvfp4(GemmArgs p1, GemmArgs p2,
                                                                               int32_t* queue) {
  w4_pair<BM, true, 4, KS>(p1, p2, queue);
}

// One thread per 16-byte piece of the tiled copy: piece (e, n/16, k/128, row,
// part) takes bytes part*16 .. +15 of row n's KB bytes for K block k/128
// (KB = 64 for 4-bit codes, 128 for bytes; PP = KB / 16 pieces per row).
template <int PP>
__global__ __launch_bounds__(256) void k_pack_kblocked(const u32x4* __restrict__ w, int64_t npieces, int K,
                                                       u32x4* __restrict__ out) {
  const int kb = K / 128;
  const int64_t row_pieces = (int64_t)kb * PP;      // 16-byte pieces per row
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < npieces; i += (int64_t)gridDim.x * 256) {
    const int part = (int)(i % PP), row = (int)((i / PP) & 15);
    const int64_t tile = i / (16 * PP);                // (e, n/16, k/128)
    const int k128 = (int)(tile % kb);
    const int64_t g = tile / kb;                        // e * N/16 + n/16
    const int64_t n = g * 16 + row;                     // row index across experts ([E*N] rows)
    out[i] = w[n * row_pieces + (int64_t)k128 * PP + part];
  }
}

void launch_pack_kblocked(const uint8_t* w, int E, int N, int K, bool bytes, uint8_t* out, hipStream_t s) {
  const int64_t npieces = (int64_t)E * N * (bytes ? K : K / 2) / 16;
  if (npieces == 0) return;
  const int64_t b = (npieces + 255) / 256;
  const dim3 grid((unsigned)(b < 8192 ? b : 8192));
  if (bytes)
    hipLaunchKernelGGL(k_pack_kblocked<8>, grid, dim3(256), 0, s, reinterpret_cast<const u32x4*>(w), npieces, K,
                       reinterpret_cast<u32x4*>(out));
  else
    hipLaunchKernelGGL(k_pack_kblocked<4>, grid, dim3(256), 0, s, reinterpret_cast<const u32x4*>(w), npieces, K,
                       reinterpret_cast<u32x4*>(out));
}

void launch_gemm_nvfp4_pair(const GemmArgs& g1, const GemmArgs& g2, int32_t* queue, int bm, int grid,
                            hipStream_t s) {
  switch (bm) {
    case 16: launch_persistent2<k_gemm_nvfp4<16, 128>>(g1, g2, queue, grid, s); break;
    case 32: launch_persistent2<k_gemm_nvfp4<32, 128>>(g1, g2, queue, grid, s); break;
    case 64: launch_persistent2<k_gemm_nvfp4<64, 128>>(g1, g2, queue, grid, s); break;
    case 48: launch_persistent2<k_gemm_nvfp4<48, 128>>(g1, g2, queue, grid, s); break;
    case 96: launch_persistent2<k_gemm_nvfp4<96, 64>>(g1, g2, queue, grid, s); break;
    case 128: launch_persistent2<k_gemm_nvfp4<128, 128>>(g1, g2, queue, grid, s); break;
    default: launch_persistent2<k_gemm_nvfp4<192, 128>>(g1, g2, queue, grid, s); break;
  }
}

void launch_gemm_int4_pair(const GemmArgs& g1, const GemmArgs& g2, int32_t* queue, int bm, int grid,
                           hipStream_t s) {
  switch (bm) {
    case 16: launch_persistent2<k_gemm_int4<16, 2, 128>>(g1, g2, queue, grid, s); break;
    case 32: launch_persistent2<k_gemm_int4<32, 4, 128>>(g1, g2, queue, grid, s); break;
    case 64: launch_persistent2<k_gemm_int4<64, 4, 128>>(g1, g2, queue, grid, s); break;
    case 48: launch_persistent2<k_gemm_int4<48, 4, 128>>(g1, g2, queue, grid, s); break;
    case 96: launch_persistent2<k_gemm_int4<96, 4, 64>>(g1, g2, queue, grid, s); break;
    case 128: launch_persistent2<k_gemm_int4<128, 4, 128>>(g1, g2, queue, grid, s); break;
    default: launch_persistent2<k_gemm_int4<192, 4, 128>>(g1, g2, queue, grid, s); break;
  }
}

}  // namespace moe
