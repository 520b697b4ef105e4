// The small kernels of the frozen-base backward (Orbit announcement, 技术细节:
// the GEMM backward that skips the base weight gradient; only the adapter and
// the layer inputs get gradients):
//   k_oft_bwd         dR_e = sum over the expert's rows of x^T dx' on each
//                     32x32 diagonal block, and dx = dx' R_e^T per row (fp32 MFMA)
//   k_unpermute_sum   dx_t = sum_j dx_(t, j) (fp32, ascending j) -> bf16
//   k_router_grad     dlogits[t][ids_tj] = w_tj (g_tj - sum_i w_ti g_ti)
#include "common.h"
#include "kernels.h"

namespace moe {

// Orders one wave's LDS accesses across its lanes (a slice only this wave
// touches): the fences keep the compiler from moving LDS loads and stores
// across the point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// One wave per (diagonal block b, active expert): the expert's rows are taken
// 16 at a time on fp32 16x16x4 MFMA.
//   dx[r][i] = sum_j dx'[r][j] R[i][j]: M = rows, N = i, K = j.  Lane
//     (l%16, l/16) supplies row l%16 and columns j = 8 (l/16) + s at step s
//     (the K order is free), i.e. 8 consecutive values of its row of dx' and
//     of row i of R_e's block.
//   dR[i][j] += sum_r x[r][i] dx'[r][j]: M = i, N = j, K = rows; the 16 x 32
//     tiles of x and dx' go through a wave-private LDS slice to put the row
//     index on l/16.
// Rows past the expert's end enter as zeros and are not stored.  Each wave
// owns its dx rows and its dR block, so there are no workgroup barriers and
// the sums run in a fixed order.
__global__ __launch_bounds__(256) void k_oft_bwd(const uint16_t* __restrict__ x, const uint16_t* __restrict__ R,
                                                 int64_t r_stride, const float* __restrict__ dxt, int H, int k,
                                                 const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ sorted_rows,
                                                 const int32_t* __restrict__ active,
                                                 const int32_t* __restrict__ num_active, float* __restrict__ dx,
                                                 float* __restrict__ dR, int64_t dr_stride, int dr_by_active) {
  __shared__ float sd[4][16][33], sx[4][16][33];
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int ln = lane & 15, lg = lane >> 4;
  const int a = blockIdx.y;
  if (a >= *num_active) return;
  const int b = blockIdx.x * 4 + wave;
  if (b >= H / 32) return;  // wave-uniform
  const int e = active[a];
  const int r0 = offsets[e], r1 = offsets[e + 1];
  const uint16_t* Rb = R + (int64_t)e * r_stride + (int64_t)b * 1024;
  float rv[2][8];  // R[i = ln + 16 h][j = 8 lg + s]
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint4 u = *reinterpret_cast<const uint4*>(Rb + (ln + 16 * h) * 32 + lg * 8);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      rv[h][2 * q] = bf16_bits_to_f32(w[q] & 0xFFFFu);
      rv[h][2 * q + 1] = bf16_bits_to_f32(w[q] >> 16);
    }
  }
  const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
  f32x4 acc[2][2] = {{zero, zero}, {zero, zero}};  // dR block (i half, j half)
  float* sdw = &sd[wave][0][0];
  float* sxw = &sx[wave][0][0];
  for (int c = r0; c < r1; c += 16) {
    const int nr = min(16, r1 - c);
    const bool ok = ln < nr;
    const int row = c + min(ln, nr - 1);
    const int tok = sorted_rows[row] / k;
    const float4* dp = reinterpret_cast<const float4*>(dxt + (int64_t)row * H + b * 32 + lg * 8);
    const float4 d0 = dp[0], d1 = dp[1];
    const uint4 xu = *reinterpret_cast<const uint4*>(x + (int64_t)tok * H + b * 32 + lg * 8);
    float dv[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
    float xv[8];
    {
      const uint32_t w[4] = {xu.x, xu.y, xu.z, xu.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xv[2 * q] = bf16_bits_to_f32(w[q] & 0xFFFFu);
        xv[2 * q + 1] = bf16_bits_to_f32(w[q] >> 16);
      }
    }
    if (!ok) {
#pragma unroll
      for (int s = 0; s < 8; ++s) dv[s] = 0.0f;
    }
    // dx for the 16 rows, 16 columns i per half
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 o = zero;
#pragma unroll
      for (int s = 0; s < 8; ++s) o = __builtin_amdgcn_mfma_f32_16x16x4f32(dv[s], rv[h][s], o, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = lg * 4 + i;
        if (rr < nr) dx[(int64_t)(c + rr) * H + b * 32 + 16 * h + ln] = o[i];
      }
    }
    // dR: rows onto the K lanes through LDS
    wave_lds_sync();  // the previous group's reads are done
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      sdw[ln * 33 + lg * 8 + s] = dv[s];
      sxw[ln * 33 + lg * 8 + s] = xv[s];
    }
    wave_lds_sync();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int q = s * 4 + lg;  // row of the group fed at step s
      const float a0 = sxw[q * 33 + ln], a1 = sxw[q * 33 + 16 + ln];
      const float b0 = sdw[q * 33 + ln], b1 = sdw[q * 33 + 16 + ln];
      acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b1, acc[1][1], 0, 0, 0);
    }
  }
  // per expert (its own R_e), or per active index into partials that
  // k_sum_active adds up when all experts share one R
  float* dRb = dR + (int64_t)(dr_by_active ? a : e) * dr_stride + (int64_t)b * 1024;
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int hj = 0; hj < 2; ++hj)
#pragma unroll
      for (int i = 0; i < 4; ++i) dRb[(16 * hi + 4 * lg + i) * 32 + 16 * hj + ln] = acc[hi][hj][i];
}

// One workgroup per token; 4 columns per thread and pass.
__global__ __launch_bounds__(256) void k_unpermute_sum(const float* __restrict__ src, const int32_t* __restrict__ row_of,
                                                       int k, int H, uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x * 4; c < H; c += 1024) {
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j0 = 0; j0 < k; j0 += 8) {
      // up to 8 rows' loads in flight, then the sums in ascending j
      float4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (j0 + i < k) v[i] = *reinterpret_cast<const float4*>(src + (int64_t)row_of[(int64_t)t * k + j0 + i] * H + c);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (j0 + i < k) {
          s[0] += v[i].x;
          s[1] += v[i].y;
          s[2] += v[i].z;
          s[3] += v[i].w;
        }
    }
    *reinterpret_cast<uint2*>(out + (int64_t)t * H + c) =
        make_uint2(bf16x2_bits(s[0], s[1]),
                   bf16x2_bits(s[2], s[3]));
  }
}

// One workgroup per token: g_tj = sum of the row's partial <u, h> over the
// nparts N blocks; unselected experts get 0.
__global__ __launch_bounds__(64) void k_router_grad(const int32_t* __restrict__ ids, const float* __restrict__ w,
                                                    const int32_t* __restrict__ row_of, const float* __restrict__ gpart,
                                                    int nparts, int k, int E, float* __restrict__ dlogits) {
  __shared__ float g[MAX_TOPK];
  const int t = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 64) dlogits[(int64_t)t * E + e] = 0.0f;
  if (threadIdx.x < k) {
    const int r = row_of[(int64_t)t * k + threadIdx.x];
    float s = 0.0f;
    for (int i = 0; i < nparts; ++i) s += gpart[(int64_t)r * nparts + i];
    g[threadIdx.x] = s;
  }
  __syncthreads();
  if (threadIdx.x < k) {
    float mean = 0.0f;
    for (int j = 0; j < k; ++j) mean += w[(int64_t)t * k + j] * g[j];
    const int j = threadIdx.x;
    dlogits[(int64_t)t * E + ids[(int64_t)t * k + j]] = w[(int64_t)t * k + j] * (g[j] - mean);
  }
}

__global__ __launch_bounds__(256) void k_zero_f32(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.0f;
}

void launch_zero_f32(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s, p, n);
}

// out[i] = sum over a = 0 .. num_active-1 of part[a][i], in ascending a
// (the shared adapter's gradient from the per-expert partials).
__global__ __launch_bounds__(256) void k_sum_active(const float* __restrict__ part, const int32_t* __restrict__ num_active,
                                                    int64_t n, float* __restrict__ out) {
  const int na = *num_active;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    float acc = 0.0f;
    for (int a = 0; a < na; ++a) acc += part[(int64_t)a * n + i];
    out[i] = acc;
  }
}

void launch_oft_bwd(const uint16_t* x, const uint16_t* R, int64_t r_stride, const float* dxt, int H, int k,
                    const int32_t* offsets, const int32_t* sorted_rows, const int32_t* active, const int32_t* num_active,
                    int E, float* dx, float* dR, float* dR_part, hipStream_t s) {
  const bool shared = r_stride == 0;
  hipLaunchKernelGGL(k_oft_bwd, dim3((H / 32 + 3) / 4, E), dim3(256), 0, s, x, R, r_stride, dxt, H, k, offsets,
                     sorted_rows, active, num_active, dx, shared ? dR_part : dR,
                     shared ? (int64_t)H * 32 : r_stride, shared ? 1 : 0);
  if (shared) {
    const int64_t n = (int64_t)H * 32;
    hipLaunchKernelGGL(k_sum_active, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dR_part, num_active, n, dR);
  }
}

void launch_unpermute_sum(const float* src, const int32_t* row_of, int T, int k, int H, uint16_t* out,
                          hipStream_t s) {
  hipLaunchKernelGGL(k_unpermute_sum, dim3(T), dim3(256), 0, s, src, row_of, k, H, out);
}

void launch_router_grad(const int32_t* ids, const float* w, const int32_t* row_of, const float* gpart, int nparts,
                        int T, int k, int E, float* dlogits, hipStream_t s) {
  hipLaunchKernelGGL(k_router_grad, dim3(T), dim3(64), 0, s, ids, w, row_of, gpart, nparts, k, E, dlogits);
}

}  // namespace moe
