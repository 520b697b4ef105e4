// Frozen-base backward for INT4 group-32 weights (Orbit announcement, 技术细节:
// the GEMM backward that bypasses the base weight gradient).  The input
// gradients are
//   u  = dout W2            (per permuted row; contraction over H)
//   dx' = [da | db] W13     (contraction over 2I)
// so both GEMMs contract over the weights' output dimension.  The backward
// therefore reads a transposed copy of the frozen weights, made once by
// k_repack_int4: nibbles of W^T (K-contiguous for the backward GEMMs) and the
// group scales converted to fp16 and arranged per 8 consecutive K values in
// the pair order the unpack consumes.  A group scale belongs to (weight row
// group, K) in the forward orientation, so in the transposed copy it varies
// along K and every element gets its own scale.
//
// k_gemm_int4_bwd: the forward INT4 kernel's DMA ring, LDS layout and fp16
// MFMA with per-element scales; 256-column N blocks; two epilogues:
//   DH: SwiGLU backward from the saved pre-activations (a, b), routing weight
//       w: dh = w u, da = dh b silu'(a), db = dh silu(a) -> fp16 [R][2I] in the
//       INT4 activation order, and partial sums <u, h> for the router gradient.
//   DX: dx' rows in fp32 [R][H].
#include "common.h"
#include "int4.h"
#include "kernels.h"
#include "moe_sched.h"

namespace moe {

// ------------------------------------------------------------- repacking

// W [E][N][K] nibbles (element 2m in the low nibble of byte m) -> W^T
// [E][K][N] in the same convention.  One 64 x 64 nibble tile per iteration,
// transposed through LDS (one byte per nibble).
__global__ __launch_bounds__(256) void k_repack_int4_t(const uint8_t* __restrict__ w, int E, int N, int K,
                                                       uint8_t* __restrict__ wt) {
  __shared__ uint8_t tile[64][65];
  const int tn = N / 64, tk = K / 64;
  const int64_t ntiles = (int64_t)E * tn * tk;
  const int t = threadIdx.x, row = t >> 2, part = t & 3;
  for (int64_t ti = blockIdx.x; ti < ntiles; ti += gridDim.x) {
    const int e = (int)(ti / ((int64_t)tn * tk));
    const int rem = (int)(ti - (int64_t)e * tn * tk);
    const int n0 = (rem / tk) * 64, k0 = (rem % tk) * 64;
    const uint8_t* src = w + (int64_t)e * N * K / 2;
    const uint2 v = *reinterpret_cast<const uint2*>(src + ((int64_t)(n0 + row) * K + k0) / 2 + part * 8);
    const uint32_t vs[2] = {v.x, v.y};
#pragma unroll
    for (int q = 0; q < 16; ++q) tile[row][part * 16 + q] = (uint8_t)((vs[q >> 3] >> ((q & 7) * 4)) & 15u);
    __syncthreads();
    // output row k0 + row, nibbles n0 + part*16 .. +15
    uint32_t o[2] = {0u, 0u};
#pragma unroll
    for (int q = 0; q < 16; ++q) o[q >> 3] |= (uint32_t)tile[part * 16 + q][row] << ((q & 7) * 4);
    uint8_t* dst = wt + (int64_t)e * N * K / 2;
    *reinterpret_cast<uint2*>(dst + ((int64_t)(k0 + row) * N + n0) / 2 + part * 8) = make_uint2(o[0], o[1]);
    __syncthreads();
  }
}

// Group scales s [E][G][L] bf16 (G groups of the transposed copy's rows, L
// along its K) -> per 8 consecutive K values four fp16 pairs
// {s0, s4}, {s1/16, s5/16}, {s2, s6}, {s3/16, s7/16}.
__global__ __launch_bounds__(256) void k_repack_scales_f16(const uint16_t* __restrict__ s, int64_t n8,
                                                           u32x4* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const u32x4 v = reinterpret_cast<const u32x4*>(s)[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float f[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = bf16_bits_to_f32((w[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu);
    u32x4 o;
    o.x = pack_f16x2(f[0], f[4]);
    o.y = pack_f16x2(f[1] * 0.0625f, f[5] * 0.0625f);
    o.z = pack_f16x2(f[2], f[6]);
    o.w = pack_f16x2(f[3] * 0.0625f, f[7] * 0.0625f);
    out[i] = o;
  }
}

void launch_repack_int4(const uint8_t* w, const uint16_t* s, int E, int N, int K, uint8_t* wt, uint16_t* st,
                        hipStream_t stream) {
  const int64_t tiles = (int64_t)E * (N / 64) * (K / 64);
  hipLaunchKernelGGL(k_repack_int4_t, dim3((unsigned)(tiles < 8192 ? tiles : 8192)), dim3(256), 0, stream, w, E, N, K,
                     wt);
  const int64_t n8 = (int64_t)E * N * K / 32 / 8;
  hipLaunchKernelGGL(k_repack_scales_f16, dim3((unsigned)((n8 + 255) / 256 < 4096 ? (n8 + 255) / 256 : 4096)),
                     dim3(256), 0, stream, s, n8, reinterpret_cast<u32x4*>(st));
}

// ------------------------------------------------------------ backward GEMM

template <int BM, bool DH>
__device__ __forceinline__ void i4t_item(const GemmArgs& p, const Tile& tl, uint8_t* smem, float* red) {
  constexpr int MT = BM / 16;
  using ST = I4Stage<BM>;
  constexpr int S = ST::S;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int ln = lane & 15, lg = lane >> 4;
  const int K = p.K, KT = K / 128;
  const char* Abase = static_cast<const char*>(p.a);
  const uint32_t smem0 = lds_u32(smem);
  lds_barrier();  // every wave is done with the previous item's stages
  const int c0 = tl.nb * 256 + wave * 64;
  const char* wexp = reinterpret_cast<const char*>(p.w) + tl.e * p.w_expert_bytes;
  const char* sexp = static_cast<const char*>(p.w_scale) + tl.e * p.ws_expert_elems * 2;
  const char* bsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) bsrc[i] = wexp + (int64_t)(c0 + 16 * i + ln) * (K / 2) + lg * 16;
  // scales of the wave's two row groups: 2 runs of 128 K values (256 B) per step
  const char* bssrc = sexp + ((int64_t)(c0 / 32 + ((lane >> 4) & 1)) * K + (lane & 15) * 8) * 2;
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
    for (int i = 0; i < 4; ++i) dma_b128(bsrc[i] + kt * 64, sb + ST::B_OFF + (wave * 4 + i) * 1024);
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
    u32x4 bq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      bq[i] = *reinterpret_cast<const u32x4*>(st + ST::B_OFF + (wave * 4 + i) * 1024 + lane * 16);
    auto read_a = [&](int m, int s) {
      const int r = m * 16 + ln;
      return *reinterpret_cast<const f16x8*>(st + r * 256 + (((4 * lg + s) ^ (r & 15)) << 4));
    };
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      f16x8 bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // K values 32 lg + 8 s .. +7 of weight row c0 + 16 i + ln: run i / 2, octet 4 lg + s
        const u32x4 sc = *reinterpret_cast<const u32x4*>(st + ST::BS_OFF + wave * 512 + (i >> 1) * 256 +
                                                         (4 * lg + s) * 16);
        bf[i] = int4x8_to_f16_se(dword_of(bq[i], s), sc);
      }
      f16x8 afc = read_a(0, s);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        f16x8 afn = afc;
        if (m + 1 < MT) afn = read_a(m + 1, s);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[m][i] = mfma_f16_16x16x32(afc, bf[i], acc[m][i]);
        afc = afn;
      }
    }
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
            const float sl = a * sg;
            gp += u * (sl * b);
            const float dh = w * u;
            dAB[(int64_t)r * 2 * I + i4act_pos(col)] = (_Float16)(dh * b * sg * (1.0f + a * (1.0f - sg)));
            dAB[(int64_t)r * 2 * I + I + i4act_pos(col)] = (_Float16)(dh * sl);
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
template <int BM>
__global__ __launch_bounds__(256, I4Stage<BM>::WPC) void k_gemm_int4_bwd(GemmArgs p1, GemmArgs p2,
                                                                         int32_t* queue) {
  using ST = I4Stage<BM>;
  constexpr int S = ST::S;
  static_assert(S >= 2 && S <= 7, "LDS stages");
  __shared__ __align__(16) uint8_t smem[S * ST::BYTES];
  __shared__ float red[4 * BM];
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
    if (cur < len1) i4t_item<BM, true>(p1, tile_of(p1, c1, b1 + cur, BM), smem, red);
    else i4t_item<BM, false>(p2, tile_of(p2, c2, b2 + cur - len1, BM), smem, red);
    if (threadIdx.x == 0) s_item = nxt;
    lds_barrier();
    cur = s_item;
  }
}

void launch_gemm_int4_bwd_pair(const GemmArgs& g1, const GemmArgs& g2, int32_t* queue, int bm, int grid,
                               hipStream_t s) {
  switch (bm) {
    case 16: launch_persistent2<k_gemm_int4_bwd<16>>(g1, g2, queue, grid, s); break;
    case 32: launch_persistent2<k_gemm_int4_bwd<32>>(g1, g2, queue, grid, s); break;
    case 48: launch_persistent2<k_gemm_int4_bwd<48>>(g1, g2, queue, grid, s); break;
    case 64: launch_persistent2<k_gemm_int4_bwd<64>>(g1, g2, queue, grid, s); break;
    case 96: launch_persistent2<k_gemm_int4_bwd<96>>(g1, g2, queue, grid, s); break;
    case 128: launch_persistent2<k_gemm_int4_bwd<128>>(g1, g2, queue, grid, s); break;
    default: launch_persistent2<k_gemm_int4_bwd<192>>(g1, g2, queue, grid, s); break;
  }
}

}  // namespace moe
