// Internal launcher interface between the C-ABI host code and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int MAX_EXPERTS = 1024;
constexpr int MAX_TOPK = 16;
constexpr int PAIRS_PER_BLOCK = 512;  // flat (token, slot) pairs per histogram / scatter block

// Everything a grouped-GEMM launch over one chunk of active experts needs.
struct GemmArgs {
  // A operand: activation rows.  a_per_token: row r reads token sorted_rows[r]/k.
  const void* a;            // codes / fp16 values, [rows][K]
  const void* a_scale;      // FP8: fp32 [rows][K/128]; MXFP4 path: E8M0 [rows][K/32]
  int a_scale_stride;       // bytes between rows of a_scale (scale_row_bytes(K))
  int a_per_token;
  // B operand: packed expert weights [E][N][K] and their scales.
  const uint8_t* w;
  const void* w_scale;
  int64_t w_expert_bytes;      // bytes between experts' packed weights
  int64_t ws_expert_elems;     // elements between experts' scales
  int N, K;                    // GEMM1: N = 2I, K = H.  GEMM2: N = H, K = I.
  int inter;                   // I (GEMM1 pairs column n with n + I)
  // output
  void* out;                   // GEMM1: activation-format h [R][I]; GEMM2: bf16 y [R][N]
  void* out_scale;             // GEMM1 FP8: fp32 [R][I/128]; MXFP4: E8M0 [R][I/32]
  int out_scale_stride;        // bytes between rows of out_scale (scale_row_bytes(I))
  // routing / schedule (device)
  const int32_t* offsets;
  const int32_t* sorted_rows;
  const int32_t* active;
  const int32_t* num_active;
  const int32_t* tile_start;   // per active expert prefix of ceil(count/BM) (+ total)
  const int32_t* tiles;        // per tile {expert, first row, valid rows, active index}
  int top_k;
  int chunk;                   // chunk index c
  int chunk_experts;           // C
  int nb_fastest;              // 1: item order (tile, N block) with N blocks fastest
  // backward (INT4): GEMM1 with save_ab writes the gate/up pre-activations
  // a, b as fp32 [R][2I] to out instead of h; the dh GEMM reads them (ab),
  // the routing weights (topk_w, per flat pair) and writes per-row partial
  // sums <u, h> over its 256 columns to gpart [R][I/256].
  int save_ab;
  // weights in 16-row x 128-K tiles, K-fastest ([N/16][K/128][16][KB] per
  // expert, KB = 64 bytes of 4-bit codes or 128 of E4M3) instead of rows
  int w_kblocked;
  const float* ab;
  const float* topk_w;
  float* gpart;
  // backward (FP8, MXFP4): GEMM1 also writes the fp32 pre-activations to
  // ab_out next to its usual h; the dh GEMM reads that quantized h (hq codes,
  // hsc scales with hsc_stride bytes per row) for the router term <u, Q(h)>.
  float* ab_out;
  const uint8_t* hq;
  const void* hsc;
  int hsc_stride;
  // NVFP4: per-expert fp32 second-level scale of this GEMM's weight matrix
  const float* gscale;
};

void launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s);
void launch_permute(const int32_t* ids, int R, int E, int bm_a, int32_t* hist, int32_t* offsets,
                    int32_t* sorted_rows, int32_t* row_of, int32_t* active, int32_t* num_active, int32_t* tile_a,
                    int32_t* tile_16, int32_t* tile_desc, int32_t* queue, int nqueue, hipStream_t s);
// Upper bound on the number of row tiles of any height >= 16 (descriptor table entries).
inline int64_t max_row_tiles(int64_t R, int E) { return R / 16 + E; }

// Activation preparation (per token rows, no adapter).
void launch_act_f16(const uint16_t* x, int T, int H, uint16_t* out, hipStream_t s);
// bf16 -> fp16 in natural element order (the NVFP4 GEMMs' input)
void launch_act_f16_natural(const uint16_t* x, int T, int H, uint16_t* out, hipStream_t s);
// Activation scale rows (FP8: fp32 per 128, MXFP8: E8M0 per 32, i.e. 4 bytes
// per 128-wide K step either way) are padded to a multiple of 16 bytes, so a
// GEMM can fetch the scales of 4 consecutive K steps of a row as one
// aligned 16-byte piece.
inline int scale_row_bytes(int K) { return ((K / 128) * 4 + 15) / 16 * 16; }
// pow2: scales are the power of two at or above amax/448 (else amax/448).
void launch_act_fp8(const uint16_t* x, int T, int H, uint8_t* q, float* sc, int sc_stride, bool pow2,
                    hipStream_t s);
void launch_act_mxfp8(const uint16_t* x, int T, int H, uint8_t* q, uint8_t* e8, int e8_stride, hipStream_t s);
// OFT rotation of every permuted row into a GEMM1 input format: out_fmt 0 fp16
// in the INT4-path layout, 1 bf16, 2 fp16 (NVFP4), 3 FP8 [1,128] (fp32 scales),
// 4 FP8 [1,128] with power-of-two scales, 5 MXFP8 (E8M0 bytes); out [R][H],
// out_scale rows of scale_stride bytes (quantized formats).
void launch_oft(int out_fmt, const uint16_t* x, const uint16_t* R, int64_t r_expert_stride, int H, int k,
                const int32_t* offsets, const int32_t* sorted_rows, const int32_t* active, const int32_t* num_active,
                const int32_t* tile16, const int32_t* desc16, void* out, void* out_scale, int scale_stride,
                hipStream_t s);
// OFT rotation of every permuted row into the INT4-path activation layout.
void launch_oft_f16(const uint16_t* x, const uint16_t* R, int64_t r_expert_stride, int H, int k,
                    const int32_t* offsets, const int32_t* sorted_rows, const int32_t* active,
                    const int32_t* num_active, const int32_t* tile16, int E, uint16_t* out, hipStream_t s);

// The same rotation written as bf16 rows in natural order (BF16 GEMM input).
void launch_oft_bf16(const uint16_t* x, const uint16_t* R, int64_t r_expert_stride, int H, int k,
                     const int32_t* offsets, const int32_t* sorted_rows, const int32_t* active,
                     const int32_t* num_active, const int32_t* tile16, uint16_t* out, hipStream_t s);

// Materialized-chunk scheme: dequantize chunk `chunk`'s experts (active order)
// into scratch [C][2I*H + H*I] bf16 (W13 rows then W2 rows per expert), then
// BF16 grouped GEMMs that read the copy (GemmArgs.w = the copy, w_expert_bytes
// = 2 * (2I*H + H*I), the W2 copy at an offset of 2I*H elements); bm in
// {16, 32, 64, 128}.
void launch_dequant_chunk(int fmt, const uint8_t* w13, const void* s13, const uint8_t* w2, const void* s2,
                          const int32_t* active, const int32_t* num_active, int chunk, int C, int H, int I,
                          const float* g13, const float* g2, bool kblocked, uint16_t* scratch, hipStream_t s);
void launch_gemm_bf16_pair(const GemmArgs& g1, const GemmArgs& g2, int32_t* queue, int bm, int grid,
                           hipStream_t s);

// Frozen-base backward.  Transposed weight copy of W [E][N][K]:
//   INT4 / MXFP4: nibbles W^T [E][K][N]; group scales [E][K/32][N] (forward
//     orientation) -> fp16 values regrouped per 8 consecutive entries of the
//     last dimension (INT4: bf16 scales, odd pairs pre-divided by 16; MXFP4:
//     E8M0 -> 2^(e-127));
//   FP8: bytes W^T [E][K][N]; block scales [E][N/128][K/128] -> [E][K/128][N/128].
void launch_repack_bwd(int fmt, const uint8_t* w, const void* s, int E, int N, int K, bool tiled, uint8_t* wt,
                       void* st, hipStream_t stream);
// One launch: chunk g1.chunk's dh items (SwiGLU backward epilogue) and chunk
// g2.chunk's dx' items, both reading the transposed copy; fmt = kernel family.
void launch_gemm_bwd_pair(int fmt, const GemmArgs& g1, const GemmArgs& g2, int32_t* queue, int bm, int grid,
                          hipStream_t s);
// r_stride = 0 (one R shared by all experts): per-active-expert partials go to
// dR_part [E][H/32][32][32] and are summed into dR in ascending active order.
void launch_oft_bwd(const uint16_t* x, const uint16_t* R, int64_t r_stride, const float* dxt, int H, int k,
                    const int32_t* offsets, const int32_t* sorted_rows, const int32_t* active, const int32_t* num_active,
                    int E, float* dx, float* dR, float* dR_part, hipStream_t s);
void launch_unpermute_sum(const float* src, const int32_t* row_of, int T, int k, int H, uint16_t* out, hipStream_t s);
void launch_router_grad(const int32_t* ids, const float* w, const int32_t* row_of, const float* gpart, int nparts,
                        int T, int k, int E, float* dlogits, hipStream_t s);
void launch_zero_f32(float* p, int64_t n, hipStream_t s);

// Grouped GEMMs; bm = rows per tile (16, 32, 48, 64, 96, 128 or 192).  One
// launch runs chunk g1.chunk's GEMM1 and chunk g2.chunk's GEMM2 (either may
// be empty); queue: 8 zeroed per-XCD item counters for this launch.
void launch_gemm_nvfp4_pair(const GemmArgs& g1, const GemmArgs& g2, int32_t* queue, int bm, int grid,
                            hipStream_t s);
// [E][N][K] code rows -> [E][N/16][K/128][16][KB] tiles (N % 16 == 0, K % 128 == 0;
// KB = 128 bytes for byte codes, else 64 for 4-bit codes)
void launch_pack_kblocked(const uint8_t* w, int E, int N, int K, bool bytes, uint8_t* out, hipStream_t s);
void launch_gemm_int4_pair(const GemmArgs& g1, const GemmArgs& g2, int32_t* queue, int bm, int grid,
                           hipStream_t s);
void launch_gemm_fp8_pair(const GemmArgs& g1, const GemmArgs& g2, int32_t* queue, int bm, int grid,
                          hipStream_t s);
// FP8 with power-of-two scales: both scales applied inside the block-scaled MFMA.
void launch_gemm_fp8_pow2_pair(const GemmArgs& g1, const GemmArgs& g2, int32_t* queue, int bm, int grid,
                               hipStream_t s);
void launch_gemm_mxfp4_pair(const GemmArgs& g1, const GemmArgs& g2, int32_t* queue, int bm, int grid,
                            hipStream_t s);

// Launch a persistent grouped-GEMM kernel on at most as many workgroups as
// can be resident at once (CUs x occupancy, rounded down to a multiple of 8),
// so that every workgroup that is dealt items starts immediately instead of
// waiting behind empty ones.  Occupancy is looked up once per kernel and the
// CU count once per device.
inline int device_cus(int dev) {
  static int cache[64] = {0};
  if (dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}
template <typename F>
inline int resident_grid(F kernel, int grid, int threads) {
  int o = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, kernel, threads, 0) != hipSuccess || o <= 0) o = 1;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  int cap = o * device_cus(dev) / 8 * 8;
  if (cap < 8) cap = 8;
  return grid > cap ? cap : grid;
}
template <void (*K)(GemmArgs, GemmArgs, int32_t*), int THREADS = 256>
inline void launch_persistent2(const GemmArgs& a, const GemmArgs& b, int32_t* q, int grid, hipStream_t s) {
  static int cap = 0;
  if (cap == 0) cap = resident_grid(K, 1 << 30, THREADS);
  hipLaunchKernelGGL(K, dim3(grid < cap ? grid : cap), dim3(THREADS), 0, s, a, b, q);
}

void launch_combine(const uint16_t* y, const float* w, const int32_t* row_of, int T, int k, int H, uint16_t* out,
                    hipStream_t s);
// LM head: per (token, block of 128 vocabulary rows) log-softmax statistics
// (maximum, sum of exponentials: T x blocks x 2 fp32) and the target logits
// (T fp32), then the per-token merge.
int lm_head_blocks(int V);
void launch_lm_head(const uint16_t* h, const uint16_t* wlm, const int32_t* targets, int T, int H, int V,
                    float* stats_ws, float* tz_ws, float* logprob, hipStream_t s);

}  // namespace moe
