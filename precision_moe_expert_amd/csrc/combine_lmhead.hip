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
      // up to 8 rows' loads in flight, then the FMAs in ascending j
      uint4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (j0 + i < k) v[i] = *reinterpret_cast<const uint4*>(y + (int64_t)rows[j0 + i] * H + c * 8);
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
    o.x = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
    o.y = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
    o.z = f32_to_bf16_bits(acc[4]) | (f32_to_bf16_bits(acc[5]) << 16);
    o.w = f32_to_bf16_bits(acc[6]) | (f32_to_bf16_bits(acc[7]) << 16);
    *reinterpret_cast<uint4*>(out + (int64_t)t * H + c * 8) = o;
  }
}

// inv_rms[t] = 1 / sqrt(mean(h[t]^2) + 1e-6): the final parameter-free RMSNorm,
// applied to the logits instead of the input (logits = inv_rms * (h W^T)).
__global__ __launch_bounds__(64) void k_inv_rms(const uint16_t* __restrict__ h, int H, float* __restrict__ inv_rms) {
  const int t = blockIdx.x, lane = lane_id();
  float ss = 0.0f;
  for (int c = lane * 8; c < H; c += 512) {
    const uint4 v = *reinterpret_cast<const uint4*>(h + (int64_t)t * H + c);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float a = bf16_bits_to_f32(u[q] & 0xFFFFu), b = bf16_bits_to_f32(u[q] >> 16);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += shfl_xor(ss, m);
  if (lane == 0) inv_rms[t] = 1.0f / sqrtf(ss / (float)H + 1e-6f);
}

// logits[t][v] = inv_rms[t] * sum_k h[t][k] W[v][k], bf16 MFMA with fp32
// accumulation.  A wave owns 16 vocabulary rows and 64 tokens; the weight
// rows stream from HBM once, the token rows are re-read from L2.
__global__ __launch_bounds__(256) void k_lm_gemm(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W,
                                                 const float* __restrict__ inv_rms, int T, int H, int V,
                                                 float* __restrict__ logits) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ln = lane & 15, lg = lane >> 4;
  const int v0 = (blockIdx.x * 4 + wave) * 16;
  const int t0 = blockIdx.y * 64;
  if (v0 >= V) return;
  const int vr = min(v0 + ln, V - 1);
  const uint16_t* wrow = W + (int64_t)vr * H + lg * 8;
  const uint16_t* hrow[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) hrow[m] = h + (int64_t)min(t0 + m * 16 + ln, T - 1) * H + lg * 8;
  f32x4 acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) acc[m] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  for (int kk = 0; kk < H; kk += 128) {
    uint4 bw[4], ah[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s) bw[s] = *reinterpret_cast<const uint4*>(wrow + kk + s * 32);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int s = 0; s < 4; ++s) ah[m][s] = *reinterpret_cast<const uint4*>(hrow[m] + kk + s * 32);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        acc[m] = mfma_bf16_16x16x32(__builtin_bit_cast(bf16x8, ah[m][s]), __builtin_bit_cast(bf16x8, bw[s]), acc[m]);
  }
  const int v = v0 + ln;
  if (v < V)
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + m * 16 + lg * 4 + i;
        if (t < T) logits[(int64_t)t * V + v] = acc[m][i] * inv_rms[t];
      }
}

// logprob[t] = logits[t][y_t] - (max + log(sum exp(logits - max))).
__global__ __launch_bounds__(256) void k_logsoftmax_gather(const float* __restrict__ logits, const int32_t* __restrict__ tgt,
                                                           int V, float* __restrict__ lp) {
  const int t = blockIdx.x;
  const float* row = logits + (int64_t)t * V;
  __shared__ float red[4];
  float mx = -INFINITY;
  for (int v = threadIdx.x; v < V; v += 256) mx = fmaxf(mx, row[v]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, shfl_xor(mx, m));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float se = 0.0f;
  for (int v = threadIdx.x; v < V; v += 256) se += expf(row[v] - mx);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) se += shfl_xor(se, m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = se;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int y = tgt[t];  // out-of-range targets give NaN instead of a stray read
    lp[t] = (y >= 0 && y < V) ? row[y] - (mx + logf((red[0] + red[1]) + (red[2] + red[3]))) : __builtin_nanf("");
  }
}

void launch_combine(const uint16_t* y, const float* w, const int32_t* row_of, int T, int k, int H, uint16_t* out,
                    hipStream_t s) {
  if (T == 0) return;
  hipLaunchKernelGGL(k_combine, dim3(T), dim3(256), 0, s, y, w, row_of, k, H, out);
}

void launch_lm_head(const uint16_t* h, const uint16_t* wlm, const int32_t* targets, int T, int H, int V,
                    float* logits_ws, float* inv_rms_ws, float* logprob, hipStream_t s) {
  if (T == 0) return;
  hipLaunchKernelGGL(k_inv_rms, dim3(T), dim3(64), 0, s, h, H, inv_rms_ws);
  hipLaunchKernelGGL(k_lm_gemm, dim3((V + 63) / 64, (T + 63) / 64), dim3(256), 0, s, h, wlm, inv_rms_ws, T, H, V,
                     logits_ws);
  hipLaunchKernelGGL(k_logsoftmax_gather, dim3(T), dim3(256), 0, s, logits_ws, targets, V, logprob);
}

}  // namespace moe
