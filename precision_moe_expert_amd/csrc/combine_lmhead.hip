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

// Partial logits part[ks][t][v] = sum over the ks-th K slice of h[t][k] W[v][k]
// (bf16 MFMA, fp32 accumulation).  The head is a skinny GEMM (<= 64 tokens
// against V x H weights) bound by streaming W once from HBM, so the kernel
// is built around keeping as much of that stream in flight as the LDS holds:
// a workgroup of 8 waves owns 256 vocabulary rows (32 per wave) and one K
// slice (KS = 2 slices: 250 workgroups for a 32000-row head, one per CU), and
// moves 64-K steps of its W rows (128 B of each row, 32 KB) and of the token
// rows (8 KB, shared by all waves) into an LDS ring of LM_S = 4 stages by
// global_load_lds DMA (all 160 KB of the CU's LDS, 96 KB of W in flight).
// Inside a stage each 128-byte row is kept as 8 parts of 16 B with part p at
// slot p ^ ((row >> 1) & 7): the 16 lanes reading one MFMA fragment then
// cover 16 distinct 16-byte bank groups.
constexpr int LM_S = 4;            // stages in flight
constexpr int LM_VB = 256;         // vocabulary rows per workgroup
constexpr int LM_WAVES = 8;
constexpr int LM_KS = 64;          // K per stage
constexpr int LM_RB = LM_KS * 2;   // bytes of a row per stage
constexpr int LM_STAGE = (LM_VB + 64) * LM_RB;
constexpr int LM_NPER = 4 + 1;     // DMA instructions per wave per stage (W: 32 rows, h: 8 rows)

MOE_DEV int lm_slot(int row, int part) { return part ^ ((row >> 1) & 7); }

__global__ __launch_bounds__(LM_WAVES * 64, 1) void k_lm_gemm(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W,
                                                    int T, int H, int V, int ks_len, float* __restrict__ part) {
  __shared__ __align__(16) uint8_t smem[LM_S * LM_STAGE];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int ln = lane & 15, lg = lane >> 4;
  const int vb = blockIdx.x, ks = blockIdx.y, t0 = blockIdx.z * 64;
  const int k0 = ks * ks_len, KT = ks_len / LM_KS;
  const uint32_t smem0 = lds_u32(smem);
  // DMA sources: lane l of instruction j writes LDS slot l%8 of row 8j + l/8
  // of the wave's rows; that slot holds the part whose slot is l%8.
  const int rj = lane >> 3, sl = lane & 7;
  const char* wsrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = wave * 32 + j * 8 + rj;                      // row within the W block
    const int v = min(vb * LM_VB + r, V - 1);
    wsrc[j] = reinterpret_cast<const char*>(W) + ((int64_t)v * H + k0 + lm_slot(r, sl) * 8) * 2;
  }
  const char* hsrc;
  {
    const int r = wave * 8 + rj;                               // token row within the block
    const int t = min(t0 + r, T - 1);
    hsrc = reinterpret_cast<const char*>(h) + ((int64_t)t * H + k0 + lm_slot(r, sl) * 8) * 2;
  }
  auto issue = [&](int kt, int slot) {
    const uint32_t sb = smem0 + slot * LM_STAGE;
#pragma unroll
    // W is streamed once per call: non-temporal (whole call 95 -> 87 us on the
    // 64 x 7168 x 32000 head)
    for (int j = 0; j < 4; ++j) dma_b128_nt(wsrc[j] + kt * LM_RB, sb + (wave * 32 + j * 8) * LM_RB);
    dma_b128(hsrc + kt * LM_RB, sb + (LM_VB + wave * 8) * LM_RB);
  };
  f32x4 acc[4][2];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int c = 0; c < 2; ++c) acc[m][c] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s + 1 < LM_S; ++s)
    if (s < KT) issue(s, s);
  for (int kt = 0; kt < KT; ++kt) {
    wait_stages<LM_NPER>(min(LM_S - 2, KT - 1 - kt));  // this wave's pieces of stage kt have landed
    lds_barrier();                                      // ... and every other wave's
    if (kt + LM_S - 1 < KT) issue(kt + LM_S - 1, (kt + LM_S - 1) % LM_S);
    const uint8_t* st = smem + (kt % LM_S) * LM_STAGE;
#pragma unroll
    for (int s = 0; s < LM_KS / 32; ++s) {
      const int part_ = s * 4 + lg;
      bf16x8 bw[2], ah[4];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int r = wave * 32 + c * 16 + ln;
        bw[c] = *reinterpret_cast<const bf16x8*>(st + r * LM_RB + (lm_slot(r, part_) << 4));
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int r = m * 16 + ln;
        ah[m] = *reinterpret_cast<const bf16x8*>(st + (LM_VB + r) * LM_RB + (lm_slot(r, part_) << 4));
      }
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int c = 0; c < 2; ++c) acc[m][c] = mfma_bf16_16x16x32(ah[m], bw[c], acc[m][c]);
    }
  }
  float* out = part + (int64_t)ks * T * V;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int v = vb * LM_VB + wave * 32 + c * 16 + ln;
    if (v < V)
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + m * 16 + lg * 4 + i;
          if (t < T) out[(int64_t)t * V + v] = acc[m][c][i];
        }
  }
}

// Per token and quarter of the vocabulary, one workgroup of 1024 threads:
// inv_rms = 1 / sqrt(mean(h^2) + 1e-6) (the final parameter-free RMSNorm,
// applied to the logits instead of the input), logits = inv_rms * (part[0] +
// part[1]) (slices summed in order), and the quarter's maximum logit m, its
// sum s of exp(logit - m) and the target's logit if it falls in the quarter.
// The token's h row and all of the quarter's partial logits of both slices
// are requested before the first reduction; thread i owns entries v0 + i +
// 1024 j.  Each thread keeps (max, sum) over its entries; the 64 lanes of a
// wave merge in a fixed butterfly and the 16 waves in order, so the result
// does not depend on timing.
constexpr int LMS_T = 1024;   // threads per workgroup
constexpr int LMS_Q = 4;      // vocabulary parts per token
constexpr int LMS_J = 8;      // entries per thread per pass

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

__global__ __launch_bounds__(LMS_T) void k_lm_softmax_part(const float* __restrict__ part, const uint16_t* __restrict__ h,
                                                           int H, const int32_t* __restrict__ tgt, int T, int V,
                                                           float* __restrict__ stats) {
  const int t = blockIdx.x, q = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (V + LMS_Q - 1) / LMS_Q, v0 = q * per, v1 = min(V, v0 + per);
  __shared__ float red_a[LMS_T / 64], red_b[LMS_T / 64];
  __shared__ float s_ir;
  const float* p0 = part + (int64_t)t * V;
  const float* p1 = part + ((int64_t)T + t) * V;
  // sum of squares of the h row: 8 values per thread per 8 K columns
  float ss = 0.0f;
  for (int c = tid * 8; c < H; c += LMS_T * 8) {
    const uint4 u = *reinterpret_cast<const uint4*>(h + (int64_t)t * H + c);
    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float a = bf16_bits_to_f32(w4[k] & 0xFFFFu), b = bf16_bits_to_f32(w4[k] >> 16);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
  }
  float a0[LMS_J], a1[LMS_J];
#pragma unroll
  for (int j = 0; j < LMS_J; ++j) {
    const int v = v0 + tid + j * LMS_T;
    a0[j] = v < v1 ? p0[v] : 0.0f;
    a1[j] = v < v1 ? p1[v] : 0.0f;
  }
#pragma unroll
  for (int x = 1; x < 64; x <<= 1) ss += shfl_xor(ss, x);
  if (lane == 0) red_a[wave] = ss;
  __syncthreads();
  if (tid == 0) {
    float sum = red_a[0];
    for (int w = 1; w < LMS_T / 64; ++w) sum += red_a[w];
    s_ir = 1.0f / sqrtf(sum / (float)H + 1e-6f);
  }
  __syncthreads();
  const float ir = s_ir;
  const int y = tgt[t];
  float* st = stats + ((int64_t)t * LMS_Q + q) * 3;
  float m = -INFINITY, s = 0.0f;
  for (int base = v0;; base += LMS_T * LMS_J) {
    float z[LMS_J];
    float cm = -INFINITY;
#pragma unroll
    for (int j = 0; j < LMS_J; ++j) {
      const int v = base + tid + j * LMS_T;
      z[j] = v < v1 ? (a0[j] + a1[j]) * ir : -INFINITY;
      if (v == y) st[2] = z[j];
      cm = fmaxf(cm, z[j]);
    }
    if (cm != -INFINITY) {
      float cs = 0.0f;
#pragma unroll
      for (int j = 0; j < LMS_J; ++j) cs += expf(z[j] - cm);
      lse_merge(m, s, cm, cs);
    }
    if (base + LMS_T * LMS_J >= v1) break;
    // the next pass (quarters wider than 8 K entries)
#pragma unroll
    for (int j = 0; j < LMS_J; ++j) {
      const int v = base + LMS_T * LMS_J + tid + j * LMS_T;
      a0[j] = v < v1 ? p0[v] : 0.0f;
      a1[j] = v < v1 ? p1[v] : 0.0f;
    }
  }
#pragma unroll
  for (int x = 1; x < 64; x <<= 1) {
    const float m2 = shfl_xor(m, x), s2 = shfl_xor(s, x);
    lse_merge(m, s, m2, s2);
  }
  if (lane == 0) {
    red_a[wave] = m;
    red_b[wave] = s;
  }
  __syncthreads();
  if (tid == 0) {
    float M = red_a[0], S = red_b[0];
    for (int w = 1; w < LMS_T / 64; ++w) lse_merge(M, S, red_a[w], red_b[w]);
    st[0] = M;
    st[1] = S;
  }
}

// logprob[t] = logit[t][y_t] - (M + log S), the parts merged in order.
__global__ __launch_bounds__(64) void k_lm_softmax_final(const float* __restrict__ stats,
                                                         const int32_t* __restrict__ tgt, int T, int V,
                                                         float* __restrict__ lp) {
  const int t = blockIdx.x * 64 + threadIdx.x;
  if (t >= T) return;
  const float* st = stats + (int64_t)t * LMS_Q * 3;
  float M = st[0], S = st[1];
  for (int q = 1; q < LMS_Q; ++q) lse_merge(M, S, st[q * 3], st[q * 3 + 1]);
  const int y = tgt[t];  // out-of-range targets give NaN instead of a stray read
  const int per = (V + LMS_Q - 1) / LMS_Q;
  lp[t] = (y >= 0 && y < V) ? st[(y / per) * 3 + 2] - (M + logf(S)) : __builtin_nanf("");
}

void launch_combine(const uint16_t* y, const float* w, const int32_t* row_of, int T, int k, int H, uint16_t* out,
                    hipStream_t s) {
  if (T == 0) return;
  hipLaunchKernelGGL(k_combine, dim3(T), dim3(256), 0, s, y, w, row_of, k, H, out);
}

int lm_head_slices(int H) { (void)H; return 2; }
int lm_head_parts() { return LMS_Q; }

void launch_lm_head(const uint16_t* h, const uint16_t* wlm, const int32_t* targets, int T, int H, int V,
                    float* part_ws, float* stats_ws, float* logprob, hipStream_t s) {
  if (T == 0) return;
  const int ks = lm_head_slices(H);
  hipLaunchKernelGGL(k_lm_gemm, dim3((V + LM_VB - 1) / LM_VB, ks, (T + 63) / 64), dim3(LM_WAVES * 64), 0, s, h, wlm, T, H, V,
                     H / ks, part_ws);
  hipLaunchKernelGGL(k_lm_softmax_part, dim3(T, LMS_Q), dim3(LMS_T), 0, s, part_ws, h, H, targets, T, V, stats_ws);
  hipLaunchKernelGGL(k_lm_softmax_final, dim3((T + 63) / 64), dim3(64), 0, s, stats_ws, targets, T, V, logprob);
}

}  // namespace moe
