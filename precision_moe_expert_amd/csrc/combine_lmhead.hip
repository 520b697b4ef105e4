// Weighted combine of the expert outputs and the LM-head log-prob.
#include "common.h"
#include "kernels.h"

namespace moe {

// out[t] = sum_{j<k} w[t][j] * y[row_of[t*k+j]]: a gather (no atomics), fp32
// fused multiply-adds in ascending j, RNE to bf16.  One workgroup per token;
// a thread owns 8 consecutive columns.
__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ y, const float* __restrict__ w,
                                                 const int32_t* __restrict__ row_of, int k, int H,
                                                 uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  __shared__ int rows[MAX_TOPK];
  __shared__ float wts[MAX_TOPK];
  if (threadIdx.x < k) {
    rows[threadIdx.x] = row_of[(int64_t)t * k + threadIdx.x];
    wts[threadIdx.x] = w[(int64_t)t * k + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < H / 8; c += 256) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j0 = 0; j0 < k; j0 += 8) {
      // up to 8 rows' loads in flight, then the FMAs in ascending j; the
      // expert outputs are read once, as non-temporal loads (combine 0.43 ->
      // 0.37 ms on the DeepSeek-V3 shape)
      uint4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (j0 + i < k) {
          const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(y + (int64_t)rows[j0 + i] * H + c * 8));
          v[i] = make_uint4(q.x, q.y, q.z, q.w);
        }
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (j0 + i < k) {
          const uint32_t u[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
          const float wj = wts[j0 + i];
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            acc[2 * h] = fmaf(wj, bf16_bits_to_f32(u[h] & 0xFFFFu), acc[2 * h]);
            acc[2 * h + 1] = fmaf(wj, bf16_bits_to_f32(u[h] >> 16), acc[2 * h + 1]);
          }
        }
    }
    uint4 o;
    o.x = bf16x2_bits(acc[0], acc[1]);
    o.y = bf16x2_bits(acc[2], acc[3]);
    o.z = bf16x2_bits(acc[4], acc[5]);
    o.w = bf16x2_bits(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(out + (int64_t)t * H + c * 8) = o;
  }
}

// LM head log-prob in two kernels.  k_lm_block: a workgroup of 8 waves owns
// 128 vocabulary rows and 64 tokens over the whole K.  The head is a skinny
// GEMM (<= 64 tokens against V x H weights) bound by streaming W once from
// HBM (250 workgroups for a 32000-row head, one per CU): 64-K steps of its W
// rows (128 B of each row, 16 KB) and of the token rows (8 KB, shared by all
// waves) go into an LDS ring of LM_S = 6 stages by global_load_lds DMA (80
// KB of W in flight).  Inside a stage each 128-byte row is kept as 8 parts
// of 16 B with part p at slot p ^ ((row >> 1) & 7): the 16 lanes reading one
// MFMA fragment then cover 16 distinct 16-byte bank groups.  While the
// tokens stream through, every thread also sums the squares of one 8-value
// part of one token row, for the final parameter-free RMSNorm
// inv_rms = 1 / sqrt(mean(h^2) + 1e-6), applied to the logits instead of
// the input.  The epilogue scales the workgroup's logits, reduces each
// token's maximum m and sum s of exp(logit - m) over its 128 vocabulary
// rows (16 lanes, then the 8 waves in order), writes (m, s) per (token,
// vocabulary block), and the target's logit where the target falls in the
// block: no logits leave the workgroup.  k_lm_final merges a token's blocks.
constexpr int LM_S = 6;            // stages in the ring
constexpr int LM_VB = 128;         // vocabulary rows per workgroup (16 per wave)
constexpr int LM_WAVES = 8;
constexpr int LM_KS = 64;          // K per stage
constexpr int LM_RB = LM_KS * 2;   // bytes of a row per stage
constexpr int LM_STAGE = (LM_VB + 64) * LM_RB;
constexpr int LM_NPER = 2 + 1;     // DMA instructions per wave per stage (W: 16 rows, h: 8 rows)
MOE_DEV int lm_slot(int row, int part) { return part ^ ((row >> 1) & 7); }
// Maximum and sum over the 16 lanes of a row (fixed butterfly: every lane
// ends with the same value).
template <int CTRL>
MOE_DEV float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
MOE_DEV float row16_max_f32(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x124>(v));
  return fmaxf(v, dpp_f32<0x128>(v));
}
MOE_DEV float row16_sum_f32(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x124>(v);
  return v + dpp_f32<0x128>(v);
}
MOE_DEV void lse_merge(float& m, float& s, float m2, float s2) {
  if (m2 == -INFINITY) return;  // an empty pair changes nothing
  if (m == -INFINITY) {
    m = m2;
    s = s2;
    return;
  }
  const float M = fmaxf(m, m2);
  s = s * expf(m - M) + s2 * expf(m2 - M);
  m = M;
}
__global__ __launch_bounds__(LM_WAVES * 64, 1) void k_lm_block(const uint16_t* __restrict__ h,
                                                              const uint16_t* __restrict__ W,
                                                              const int32_t* __restrict__ tgt, int T, int H, int V,
                                                              float* __restrict__ stats, float* __restrict__ tz) {
  __shared__ __align__(16) uint8_t smem[LM_S * LM_STAGE];
  __shared__ float s_ir[64];
  __shared__ float red_m[LM_WAVES][64], red_s[LM_WAVES][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int ln = lane & 15, lg = lane >> 4;
  const int vb = blockIdx.x, t0 = blockIdx.y * 64, nvb = gridDim.x;
  const int KT = H / LM_KS;
  const uint32_t smem0 = lds_u32(smem);
  // DMA sources: lane l of instruction j writes LDS slot l%8 of row 8j + l/8
  // of the wave's rows; that slot holds the part whose slot is l%8.
  const int rj = lane >> 3, sl = lane & 7;
  const char* wsrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = wave * 16 + j * 8 + rj;                      // row within the W block
    const int v = min(vb * LM_VB + r, V - 1);
    wsrc[j] = reinterpret_cast<const char*>(W) + ((int64_t)v * H + lm_slot(r, sl) * 8) * 2;
  }
  const char* hsrc;
  {
    const int r = wave * 8 + rj;                               // token row within the block
    const int t = min(t0 + r, T - 1);
    hsrc = reinterpret_cast<const char*>(h) + ((int64_t)t * H + lm_slot(r, sl) * 8) * 2;
  }
  // W is streamed once per call: non-temporal loads
  auto issue = [&](int kt, int slot) {
    const uint32_t sb = smem0 + slot * LM_STAGE;
#pragma unroll
    for (int j = 0; j < 2; ++j) dma_b128_nt(wsrc[j] + kt * LM_RB, sb + (wave * 16 + j * 8) * LM_RB);
    dma_b128(hsrc + kt * LM_RB, sb + (LM_VB + wave * 8) * LM_RB);
  };
  f32x4 acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) acc[m] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  float ss = 0.0f;                       // sum of squares of part (tid % 8) of token row tid / 8
  const int sq_r = threadIdx.x >> 3, sq_p = threadIdx.x & 7;
#pragma unroll
  for (int s = 0; s + 1 < LM_S; ++s)
    if (s < KT) issue(s, s);
  for (int kt = 0; kt < KT; ++kt) {
    wait_stages<LM_NPER>(min(LM_S - 2, KT - 1 - kt));  // this wave's pieces of stage kt have landed
    lds_barrier();                                      // ... and every other wave's
    if (kt + LM_S - 1 < KT) issue(kt + LM_S - 1, (kt + LM_S - 1) % LM_S);
    const uint8_t* st = smem + (kt % LM_S) * LM_STAGE;
    {
      const u32x4 q = *reinterpret_cast<const u32x4*>(st + (LM_VB + sq_r) * LM_RB + (lm_slot(sq_r, sq_p) << 4));
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float a = bf16_bits_to_f32(q[c] & 0xFFFFu), b = bf16_bits_to_f32(q[c] >> 16);
        ss = fmaf(a, a, ss);
        ss = fmaf(b, b, ss);
      }
    }
#pragma unroll
    for (int s = 0; s < LM_KS / 32; ++s) {
      const int part_ = s * 4 + lg;
      const int rw = wave * 16 + ln;
      const bf16x8 bw = *reinterpret_cast<const bf16x8*>(st + rw * LM_RB + (lm_slot(rw, part_) << 4));
      bf16x8 ah[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int r = m * 16 + ln;
        ah[m] = *reinterpret_cast<const bf16x8*>(st + (LM_VB + r) * LM_RB + (lm_slot(r, part_) << 4));
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[m] = mfma_bf16_16x16x32(ah[m], bw, acc[m]);
    }
  }
  // inv_rms per token: the 8 parts' sums of a token row sit in 8 consecutive lanes
  ss += shfl_xor(ss, 1);
  ss += shfl_xor(ss, 2);
  ss += shfl_xor(ss, 4);
  if (sq_p == 0) s_ir[sq_r] = 1.0f / sqrtf(ss / (float)H + 1e-6f);
  __syncthreads();
  // logits of this wave's 16 vocabulary rows (lane ln) for token rows
  // m*16 + lg*4 + i; per token the 16 lanes' maximum and sum of exponentials
  const int v = vb * LM_VB + wave * 16 + ln;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = m * 16 + lg * 4 + i, t = t0 + r;
      const float z = v < V ? acc[m][i] * s_ir[r] : -INFINITY;
      if (t < T && v == tgt[t]) tz[t] = z;
      const float mx = row16_max_f32(z);
      const float e = (z == -INFINITY) ? 0.0f : expf(z - mx);
      const float sm = row16_sum_f32(e);
      if (ln == 0) {
        red_m[wave][r] = mx;
        red_s[wave][r] = sm;
      }
    }
  __syncthreads();
  if (threadIdx.x < 64 && t0 + (int)threadIdx.x < T) {
    const int r = threadIdx.x;
    float M = red_m[0][r], S = red_s[0][r];
    for (int w = 1; w < LM_WAVES; ++w) lse_merge(M, S, red_m[w][r], red_s[w][r]);
    float* o = stats + ((int64_t)(t0 + r) * nvb + vb) * 2;
    o[0] = M;
    o[1] = S;
  }
}
// logprob[t] = logit[t][y_t] - (M + log S), one wave per token: lane l merges
// blocks l, l + 64, ... in order, then the lanes in a fixed butterfly (the
// merge is symmetric, so every lane ends with the same result).
__global__ __launch_bounds__(256) void k_lm_final(const float* __restrict__ stats, const float* __restrict__ tz,
                                                  const int32_t* __restrict__ tgt, int T, int V, int nvb,
                                                  float* __restrict__ lp) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (t >= T) return;
  float M = -INFINITY, S = 0.0f;
  for (int b = lane; b < nvb; b += 64) {
    const float* o = stats + ((int64_t)t * nvb + b) * 2;
    lse_merge(M, S, o[0], o[1]);
  }
#pragma unroll
  for (int x = 1; x < 64; x <<= 1) {
    const float m2 = shfl_xor(M, x), s2 = shfl_xor(S, x);
    lse_merge(M, S, m2, s2);
  }
  if (lane == 0) {
    const int y = tgt[t];  // out-of-range targets give NaN instead of a stray read
    lp[t] = (y >= 0 && y < V) ? tz[t] - (M + logf(S)) : __builtin_nanf("");
  }
}

void launch_combine(const uint16_t* y, const float* w, const int32_t* row_of, int T, int k, int H, uint16_t* out,
                    hipStream_t s) {
  if (T == 0) return;
  hipLaunchKernelGGL(k_combine, dim3(T), dim3(256), 0, s, y, w, row_of, k, H, out);
}

int lm_head_blocks(int V) { return (V + LM_VB - 1) / LM_VB; }
void launch_lm_head(const uint16_t* h, const uint16_t* wlm, const int32_t* targets, int T, int H, int V,
                    float* stats_ws, float* tz_ws, float* logprob, hipStream_t s) {
  if (T == 0) return;
  const int nvb = lm_head_blocks(V);
  hipLaunchKernelGGL(k_lm_block, dim3(nvb, (T + 63) / 64), dim3(LM_WAVES * 64), 0, s, h, wlm, targets, T, H, V,
                     stats_ws, tz_ws);
  hipLaunchKernelGGL(k_lm_final, dim3((T + 3) / 4), dim3(256), 0, s, stats_ws, tz_ws, targets, T, V, nvb, logprob);
}

}  // namespace moe
