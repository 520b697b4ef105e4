// The small kernels of the frozen-base backward (Orbit announcement, 技术细节:
// the GEMM backward that skips the base weight gradient; only the adapter and
// the layer inputs get gradients):
//   k_oft_bwd         dR_e = sum over the expert's rows of x^T dx' on each
//                     32x32 diagonal block, and dx = dx' R_e^T per row
//   k_unpermute_sum   dx_t = sum_j dx_(t, j) (fp32, ascending j) -> bf16
//   k_router_grad     dlogits[t][ids_tj] = w_tj (g_tj - sum_i w_ti g_ti)
#include "common.h"
#include "kernels.h"

namespace moe {

// Workgroup (block b, active expert index a).  The expert's rows are taken 32
// at a time: their x and dx' slices of block b go to LDS, every thread adds
// four entries of dR_e[b] and computes four entries of dx.
__global__ __launch_bounds__(256) void k_oft_bwd(const uint16_t* __restrict__ x, const uint16_t* __restrict__ R,
                                                 int64_t r_stride, const float* __restrict__ dxt, int H, int k,
                                                 const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ sorted_rows,
                                                 const int32_t* __restrict__ active,
                                                 const int32_t* __restrict__ num_active, float* __restrict__ dx,
                                                 float* __restrict__ dR) {
  __shared__ float Rb[32][33], xs[32][33], ds[32][33];
  const int b = blockIdx.x, a = blockIdx.y;
  if (a >= *num_active) return;
  const int e = active[a];
  const int r0 = offsets[e], r1 = offsets[e + 1];
  const int t = threadIdx.x, hi = t >> 3, lo = t & 7;
  const uint16_t* Rg = R + (int64_t)e * r_stride + (int64_t)b * 1024;
#pragma unroll
  for (int q = 0; q < 4; ++q) Rb[hi][4 * lo + q] = bf16_bits_to_f32(Rg[hi * 32 + 4 * lo + q]);
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int c = r0; c < r1; c += 32) {
    const int nr = min(32, r1 - c);
    __syncthreads();  // the previous rows are consumed (and Rb is in place)
    if (hi < nr) {
      const int r = c + hi;
      const int tok = sorted_rows[r] / k;
      const uint2 xv = *reinterpret_cast<const uint2*>(x + (int64_t)tok * H + b * 32 + 4 * lo);
      const float4 dv = *reinterpret_cast<const float4*>(dxt + (int64_t)r * H + b * 32 + 4 * lo);
      xs[hi][4 * lo + 0] = bf16_bits_to_f32(xv.x & 0xFFFFu);
      xs[hi][4 * lo + 1] = bf16_bits_to_f32(xv.x >> 16);
      xs[hi][4 * lo + 2] = bf16_bits_to_f32(xv.y & 0xFFFFu);
      xs[hi][4 * lo + 3] = bf16_bits_to_f32(xv.y >> 16);
      ds[hi][4 * lo + 0] = dv.x;
      ds[hi][4 * lo + 1] = dv.y;
      ds[hi][4 * lo + 2] = dv.z;
      ds[hi][4 * lo + 3] = dv.w;
    }
    __syncthreads();
    // dR[i = hi][j = 4 lo + q] += sum_rows x[i] dx'[j]
    for (int rr = 0; rr < nr; ++rr) {
      const float xi = xs[rr][hi];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] += xi * ds[rr][4 * lo + q];
    }
    // dx[row hi][i = 4 lo + q] = sum_j dx'[j] R[i][j]
    if (hi < nr) {
      float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int j = 0; j < 32; ++j) {
        const float d = ds[hi][j];
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] += d * Rb[4 * lo + q][j];
      }
      *reinterpret_cast<float4*>(dx + (int64_t)(c + hi) * H + b * 32 + 4 * lo) = make_float4(o[0], o[1], o[2], o[3]);
    }
  }
  *reinterpret_cast<float4*>(dR + (int64_t)e * r_stride + (int64_t)b * 1024 + hi * 32 + 4 * lo) =
      make_float4(acc[0], acc[1], acc[2], acc[3]);
}

// One workgroup per token; 4 columns per thread and pass.
__global__ __launch_bounds__(256) void k_unpermute_sum(const float* __restrict__ src, const int32_t* __restrict__ row_of,
                                                       int k, int H, uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x * 4; c < H; c += 1024) {
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = 0; j < k; ++j) {
      const float4 v = *reinterpret_cast<const float4*>(src + (int64_t)row_of[(int64_t)t * k + j] * H + c);
      s[0] += v.x;
      s[1] += v.y;
      s[2] += v.z;
      s[3] += v.w;
    }
    *reinterpret_cast<uint2*>(out + (int64_t)t * H + c) =
        make_uint2(f32_to_bf16_bits(s[0]) | (f32_to_bf16_bits(s[1]) << 16),
                   f32_to_bf16_bits(s[2]) | (f32_to_bf16_bits(s[3]) << 16));
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

void launch_oft_bwd(const uint16_t* x, const uint16_t* R, int64_t r_stride, const float* dxt, int H, int k,
                    const int32_t* offsets, const int32_t* sorted_rows, const int32_t* active, const int32_t* num_active,
                    int E, float* dx, float* dR, hipStream_t s) {
  hipLaunchKernelGGL(k_oft_bwd, dim3(H / 32, E), dim3(256), 0, s, x, R, r_stride, dxt, H, k, offsets, sorted_rows,
                     active, num_active, dx, dR);
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
