// Router top-k + softmax and the expert permutation (histogram, scan,
// stable scatter) for gfx950.  Orbit announcement, 技术细节: each token
// activates only its router-selected experts, which are then grouped.
#include "common.h"
#include "kernels.h"

namespace moe {

// Monotone unsigned key of a float (larger float -> larger key); -0 and +0
// map to the same key.
MOE_DEV uint32_t float_key(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) == 0) b = 0;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
MOE_DEV float key_float(uint32_t k) { return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k); }

template <int CTRL>
MOE_DEV uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)dpp_i32<CTRL>((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)dpp_i32<CTRL>((int)(uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Maximum over each row of 16 lanes, returned in every lane of the row:
// quad swaps, then row rotations by 4 and 8 (DPP, register to register).
MOE_DEV uint64_t row16_max_u64(uint64_t v) {
  uint64_t o;
  o = dpp_u64<0xB1>(v);  v = o > v ? o : v;   // quad_perm [1,0,3,2]
  o = dpp_u64<0x4E>(v);  v = o > v ? o : v;   // quad_perm [2,3,0,1]
  o = dpp_u64<0x124>(v); v = o > v ? o : v;   // row_ror:4
  o = dpp_u64<0x128>(v); v = o > v ? o : v;   // row_ror:8
  return v;
}

// One token per row of 16 lanes (4 tokens per wave).  Lane r keeps the
// logits of experts r, r + 16, ... (SLOTS of them, E <= 16 SLOTS) as 64-bit
// keys (value key << 32 | (0xFFFF - id)), so the row maximum is the largest
// logit and, among equal logits, the smallest expert id.  Each of the k
// rounds takes the row maximum and clears it.  Rows past the last token
// still run the rounds (on zero keys) so that every DPP source lane is live.
template <int SLOTS>
__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits, int T, int E, int k,
                                                    int32_t* __restrict__ ids, float* __restrict__ w) {
  const int r = threadIdx.x & 15;
  const int t = blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool live = t < T;
  const float* row = logits + (int64_t)(live ? t : 0) * E;
  uint64_t key[SLOTS];
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int e = r + 16 * i;
    key[i] = (live && e < E) ? (((uint64_t)float_key(row[e]) << 32) | (uint64_t)(0xFFFFu - e)) : 0ull;
  }
  float sel_val[MAX_TOPK];
  int sel_id[MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MAX_TOPK; ++j) {
    if (j < k) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) best = key[i] > best ? key[i] : best;
      best = row16_max_u64(best);
      sel_id[j] = 0xFFFF - (int)(best & 0xFFFFu);
      sel_val[j] = key_float((uint32_t)(best >> 32));
#pragma unroll
      for (int i = 0; i < SLOTS; ++i)
        if (key[i] == best) key[i] = 0;  // keys are unique (distinct ids), so only the winner clears
    }
  }
  if (!live) return;
  // softmax over the selected logits, relative to the largest (slot 0)
  float z = 0.0f;
#pragma unroll
  for (int j = 0; j < MAX_TOPK; ++j)
    if (j < k) z += expf(sel_val[j] - sel_val[0]);
#pragma unroll
  for (int j = 0; j < MAX_TOPK; ++j)
    if (j < k && r == j) {
      ids[(int64_t)t * k + j] = sel_id[j];
      w[(int64_t)t * k + j] = expf(sel_val[j] - sel_val[0]) / z;
    }
}

// Per-block expert histogram of PAIRS_PER_BLOCK consecutive flat pairs.
__global__ __launch_bounds__(256) void k_hist(const int32_t* __restrict__ ids, int R, int E,
                                              int32_t* __restrict__ hist) {
  __shared__ int32_t cnt[MAX_EXPERTS];
  for (int e = threadIdx.x; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * PAIRS_PER_BLOCK;
  for (int i = threadIdx.x; i < PAIRS_PER_BLOCK; i += 256) {
    int p = p0 + i;
    if (p < R) atomicAdd(&cnt[ids[p]], 1);  // counting only: order-independent
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) hist[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// Orders one wave's LDS accesses before and after it (no other wave waits).
MOE_DEV void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Exclusive scan, over the 1024 threads of the block, of four independent
// ints per thread: a shuffle scan inside each wave, then each thread adds the
// totals of the waves before it (two barriers instead of twenty per scan).
MOE_DEV i32x4 block_excl_scan4_1024(i32x4 v, i32x4* sh, i32x4* total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  i32x4 incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    i32x4 o;
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = __shfl_up(incl[c], off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  i32x4 before = {0, 0, 0, 0}, all = {0, 0, 0, 0};
  for (int w = 0; w < 16; ++w) {
    const i32x4 t = sh[w];
    if (w < wave) before += t;
    all += t;
  }
  *total = all;
  __syncthreads();
  return before + incl - v;
}

// One workgroup of 1024 threads.  Turns the per-block histograms into
// per-(block, expert) scatter bases, writes the expert offsets, the ascending
// active-expert list, and the per-active-expert tile prefixes for tiles of
// bm_a rows and of 16 rows.  The blocks are split into G = 1024 / E
// contiguous ranges: thread (g, e) sums range g of expert e's column (all
// loads of a range in flight together), the experts' totals are scanned with
// thread = expert, and each thread then writes the bases of its range.
//
// ONE: all pairs form a single block (few tokens: decode).  The same
// workgroup then also counts them (LDS histogram, in place of k_hist) and
// scatters them (wave 0, the ranking of k_scatter with the expert offsets
// as its counters), so the permutation takes one launch instead of three.
template <bool ONE>
__global__ __launch_bounds__(1024) void k_scan(int32_t* __restrict__ hist, int nblk, int E, int bm_a,
                                               int32_t* __restrict__ offsets, int32_t* __restrict__ active,
                                               int32_t* __restrict__ num_active, int32_t* __restrict__ tile_a,
                                               int32_t* __restrict__ tile_16, int32_t* __restrict__ tile_desc,
                                               int32_t* __restrict__ queue, int nqueue,
                                               const int32_t* __restrict__ ids, int R,
                                               int32_t* __restrict__ sorted_rows, int32_t* __restrict__ row_of) {
  __shared__ i32x4 sh4[16];
  __shared__ int s_tstart[MAX_EXPERTS + 1], s_exp[MAX_EXPERTS], s_off[MAX_EXPERTS], s_cnt[MAX_EXPERTS];
  __shared__ int s_part[1024], s_base[MAX_EXPERTS];
  __shared__ int s_hist[ONE ? MAX_EXPERTS : 1];
  const int G = 1024 / E;
  const int tid = threadIdx.x;
  const int g = tid / E, ce = tid - g * E;  // this thread's range and column (g < G)
  const int b0 = (int)((int64_t)nblk * g / G), b1 = (int)((int64_t)nblk * (g + 1) / G);
  if constexpr (ONE) {
    for (int e = tid; e < E; e += 1024) s_hist[e] = 0;
    __syncthreads();
    for (int q = tid; q < R; q += 1024) atomicAdd(&s_hist[ids[q]], 1);  // counting only: order-independent
    __syncthreads();
    // the one block sits in exactly one range
    if (g < G) s_part[tid] = b0 < b1 ? s_hist[ce] : 0;
  } else if (g < G) {
    int sum = 0;
    for (int b = b0; b < b1; b += 16) {
      int h[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) h[i] = (b + i < b1) ? hist[(int64_t)(b + i) * E + ce] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) sum += h[i];
    }
    s_part[tid] = sum;
  }
  __syncthreads();
  const int e = tid;
  int cnt = 0;
  if (e < E)
    for (int q = 0; q < G; ++q) cnt += s_part[q * E + e];
  // one scan for: row offsets, active positions, bm_a-row tiles, 16-row tiles
  const int act = (e < E && cnt > 0) ? 1 : 0;
  const i32x4 v = {e < E ? cnt : 0, act, act ? (cnt + bm_a - 1) / bm_a : 0, act ? (cnt + 15) / 16 : 0};
  i32x4 tot;
  const i32x4 ex = block_excl_scan4_1024(v, sh4, &tot);
  const int off = ex[0], pos = ex[1], ta = ex[2], t16 = ex[3];
  const int na = tot[1], nta = tot[2], nt16 = tot[3];
  if (e < E) {
    offsets[e] = off;
    s_base[e] = off;
  }
  if (e == 0) offsets[E] = tot[0];
  if (act) {
    active[pos] = e;
    tile_a[pos] = ta;
    tile_16[pos] = t16;
    s_tstart[pos] = ta;
    s_exp[pos] = e;
    s_off[pos] = off;
    s_cnt[pos] = cnt;
  }
  if (e == 0) {
    *num_active = na;
    tile_a[na] = nta;
    tile_16[na] = nt16;
    s_tstart[na] = nta;
  }
  for (int i = threadIdx.x; i < nqueue; i += blockDim.x) queue[i] = 0;  // GEMM work-queue counters
  __syncthreads();
  if constexpr (ONE) {
    // stable scatter of the block's pairs by wave 0 (k_scatter's ranking);
    // the other waves go on to the tile descriptors
    if (tid < 64) {
      const int lane = tid;
      constexpr int NC = PAIRS_PER_BLOCK / 64;
      int eid[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) eid[c] = c * 64 + lane < R ? ids[c * 64 + lane] : 0;
      int nbits = 0;
      while ((1 << nbits) < E) ++nbits;
      const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int q = c * 64 + lane;
        const bool valid = q < R;
        const int e = eid[c];
        uint64_t m = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
          const uint64_t bb = __ballot(valid && ((e >> b) & 1));
          m &= ((e >> b) & 1) ? bb : ~bb;
        }
        const int pos = valid ? s_base[e] + __popcll(m & lt_mask) : 0;
        wave_lds_sync();  // every lane has read its counter before any is advanced
        if (valid) {
          sorted_rows[pos] = q;
          row_of[q] = pos;
          if ((m >> lane) == 1ull) s_base[e] = pos + 1;  // highest lane of the group advances the counter
        }
        wave_lds_sync();
      }
    }
  } else if (g < G) {
    // scatter bases of this thread's range: the expert's offset, the ranges
    // before it, then the blocks before it within the range
    int base = s_base[ce];
    for (int q = 0; q < g; ++q) base += s_part[q * E + ce];
    for (int b = b0; b < b1; b += 16) {
      int h[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) h[i] = (b + i < b1) ? hist[(int64_t)(b + i) * E + ce] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (b + i < b1) {
          hist[(int64_t)(b + i) * E + ce] = base;
          base += h[i];
        }
    }
  }
  // One descriptor per bm_a-row tile, in (active expert, tile) order:
  // {expert, first permuted row, valid rows, active index}.
  for (int t = threadIdx.x; t < nta; t += blockDim.x) {
    int lo = 0, hi = na - 1;  // last active expert whose first tile is <= t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_tstart[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int r0 = (t - s_tstart[lo]) * bm_a;
    const i32x4 d = {s_exp[lo], s_off[lo] + r0, min(bm_a, s_cnt[lo] - r0), lo};
    *reinterpret_cast<i32x4*>(tile_desc + 4 * (int64_t)t) = d;
  }
}

// Stable scatter: one wave walks its block's pairs in (t, j) order, 64 at a
// time.  Lanes holding the same expert are found with ballots over the bits
// of the id; a pair's rank is the number of lower lanes with its expert.
// Positions come from per-expert LDS counters seeded with the block's scatter
// bases, so no global atomics decide any position.
__global__ __launch_bounds__(64) void k_scatter(const int32_t* __restrict__ ids, int R, int E,
                                                const int32_t* __restrict__ base, int32_t* __restrict__ sorted_rows,
                                                int32_t* __restrict__ row_of) {
  __shared__ int32_t cnt[MAX_EXPERTS];
  const int lane = lane_id();
  const int p0 = blockIdx.x * PAIRS_PER_BLOCK;
  // every id of the block is requested, together with the block's scatter
  // bases, before the first ranking step (one memory round trip per block
  // instead of one per 64 pairs)
  constexpr int NC = PAIRS_PER_BLOCK / 64;
  int eid[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int p = p0 + c * 64 + lane;
    eid[c] = p < R ? ids[p] : 0;
  }
  for (int e = lane; e < E; e += 64) cnt[e] = base[(int64_t)blockIdx.x * E + e];
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int p = p0 + c * 64 + lane;
    const bool valid = p < R;
    const int e = eid[c];
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      uint64_t bb = __ballot(valid && ((e >> b) & 1));
      m &= ((e >> b) & 1) ? bb : ~bb;
    }
    const int rank = __popcll(m & lt_mask);
    int pos = 0;
    if (valid) pos = cnt[e] + rank;
    __syncthreads();
    if (valid) {
      sorted_rows[pos] = p;
      row_of[p] = pos;
      if ((m >> lane) == 1ull) cnt[e] = pos + 1;  // highest lane of the group advances the counter
    }
    __syncthreads();
  }
}

// The same selection with one token per wave (few tokens: decode): lane l
// keeps experts l, l + 64, ... (SLOTS of them, E <= 64 SLOTS), and each
// round's maximum is the 16-lane row maximum followed by two cross-row
// exchanges.  The keys and their order are those above, so both kernels
// select the same experts in the same order.
template <int SLOTS>
__global__ __launch_bounds__(256) void k_route_topk_wave(const float* __restrict__ logits, int T, int E, int k,
                                                         int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole waves only
  const float* row = logits + (int64_t)t * E;
  uint64_t key[SLOTS];
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? (((uint64_t)float_key(row[e]) << 32) | (uint64_t)(0xFFFFu - e)) : 0ull;
  }
  float sel_val[MAX_TOPK];
  int sel_id[MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MAX_TOPK; ++j) {
    if (j < k) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) best = key[i] > best ? key[i] : best;
      best = row16_max_u64(best);
#pragma unroll
      for (int x = 16; x < 64; x <<= 1) {
        const uint32_t lo = (uint32_t)shfl_xor((int)(uint32_t)best, x);
        const uint32_t hi = (uint32_t)shfl_xor((int)(uint32_t)(best >> 32), x);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        best = o > best ? o : best;
      }
      sel_id[j] = 0xFFFF - (int)(best & 0xFFFFu);
      sel_val[j] = key_float((uint32_t)(best >> 32));
#pragma unroll
      for (int i = 0; i < SLOTS; ++i)
        if (key[i] == best) key[i] = 0;
    }
  }
  float z = 0.0f;
#pragma unroll
  for (int j = 0; j < MAX_TOPK; ++j)
    if (j < k) z += expf(sel_val[j] - sel_val[0]);
#pragma unroll
  for (int j = 0; j < MAX_TOPK; ++j)
    if (j < k && lane == j) {
      ids[(int64_t)t * k + j] = sel_id[j];
      w[(int64_t)t * k + j] = expf(sel_val[j] - sel_val[0]) / z;
    }
}

void launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s) {
  if (T == 0) return;
  if (T <= 1024 && E > 64) {  // few tokens: one per wave, fewer slots per lane
    const dim3 g((T + 3) / 4), b(256);
    if (E <= 128) hipLaunchKernelGGL(k_route_topk_wave<2>, g, b, 0, s, logits, T, E, k, ids, w);
    else if (E <= 256) hipLaunchKernelGGL(k_route_topk_wave<4>, g, b, 0, s, logits, T, E, k, ids, w);
    else if (E <= 384) hipLaunchKernelGGL(k_route_topk_wave<6>, g, b, 0, s, logits, T, E, k, ids, w);
    else if (E <= 512) hipLaunchKernelGGL(k_route_topk_wave<8>, g, b, 0, s, logits, T, E, k, ids, w);
    else hipLaunchKernelGGL(k_route_topk_wave<16>, g, b, 0, s, logits, T, E, k, ids, w);
    return;
  }
  const dim3 g((T + 15) / 16), b(256);
  if (E <= 64) hipLaunchKernelGGL(k_route_topk<4>, g, b, 0, s, logits, T, E, k, ids, w);
  else if (E <= 128) hipLaunchKernelGGL(k_route_topk<8>, g, b, 0, s, logits, T, E, k, ids, w);
  else if (E <= 256) hipLaunchKernelGGL(k_route_topk<16>, g, b, 0, s, logits, T, E, k, ids, w);
  else if (E <= 384) hipLaunchKernelGGL(k_route_topk<24>, g, b, 0, s, logits, T, E, k, ids, w);
  else if (E <= 512) hipLaunchKernelGGL(k_route_topk<32>, g, b, 0, s, logits, T, E, k, ids, w);
  else hipLaunchKernelGGL(k_route_topk<64>, g, b, 0, s, logits, T, E, k, ids, w);
}

void launch_permute(const int32_t* ids, int R, int E, int bm_a, int32_t* hist, int32_t* offsets,
                    int32_t* sorted_rows, int32_t* row_of, int32_t* active, int32_t* num_active, int32_t* tile_a,
                    int32_t* tile_16, int32_t* tile_desc, int32_t* queue, int nqueue, hipStream_t s) {
  const int nblk = (R + PAIRS_PER_BLOCK - 1) / PAIRS_PER_BLOCK;
  if (nblk == 1) {  // one launch: histogram, scan and scatter in one workgroup
    hipLaunchKernelGGL(k_scan<true>, dim3(1), dim3(1024), 0, s, hist, nblk, E, bm_a, offsets, active, num_active,
                       tile_a, tile_16, tile_desc, queue, nqueue, ids, R, sorted_rows, row_of);
    return;
  }
  if (nblk > 0) hipLaunchKernelGGL(k_hist, dim3(nblk), dim3(256), 0, s, ids, R, E, hist);
  hipLaunchKernelGGL(k_scan<false>, dim3(1), dim3(1024), 0, s, hist, nblk, E, bm_a, offsets, active, num_active,
                     tile_a, tile_16, tile_desc, queue, nqueue, ids, R, sorted_rows, row_of);
  if (nblk > 0) hipLaunchKernelGGL(k_scatter, dim3(nblk), dim3(64), 0, s, ids, R, E, hist, sorted_rows, row_of);
}

}  // namespace moe
