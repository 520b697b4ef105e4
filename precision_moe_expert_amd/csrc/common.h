// Device-side helpers shared by the gfx950 kernels of the MoE expert library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
// Native 16-byte vector (HIP's uint4 is a union struct whose copies become
// memcpys through the stack; this one stays in registers).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

#define MOE_DEV __device__ __forceinline__

// Format ids (same values as moe_wformat).
enum { FMT_INT4 = 1, FMT_FP8 = 2, FMT_MXFP4 = 3, FMT_NVFP4 = 5 };

MOE_DEV float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even: gfx950's v_cvt_pk_bf16_f32 (one
// instruction; bit-identical to rounding the fp32 bits by hand for every
// finite input, checked on the GPU over 2^28 patterns with ties,
// subnormals and values next to the largest finite number).
MOE_DEV uint32_t f32_to_bf16_bits(float f) { return __builtin_bit_cast(unsigned short, (__bf16)f); }
// Two values in one conversion: a in the low half, b in the high half.
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
MOE_DEV uint32_t bf16x2_bits(float a, float b) {
  const bf16x2_hw v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// E4M3FN byte -> fp32 (exact; the NaN code is not expected in weights).
MOE_DEV float e4m3_to_f32(uint32_t b) {
  const uint32_t s = (b & 0x80u) << 24, e = (b >> 3) & 15u, m = b & 7u;
  if (e == 0) {  // subnormal: m * 2^-9
    const float v = (float)m * 0x1p-9f;
    return s ? -v : v;
  }
  return __uint_as_float(s | ((e + 120u) << 23) | (m << 20));
}

MOE_DEV uint32_t pack_f16x2(float a, float b) {
  _Float16 ha = (_Float16)a, hb = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// E4M3FN codes of two fp32 values (RNE, saturating to +-448) packed in the
// low 16 bits (a in byte 0, b in byte 1).  The hardware conversion rounds to
// nearest even but maps magnitudes above 464 to NaN, hence the clamp.
MOE_DEV uint32_t cvt_e4m3x2(float a, float b) {
  a = __builtin_fminf(__builtin_fmaxf(a, -448.0f), 448.0f);
  b = __builtin_fminf(__builtin_fmaxf(b, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Four E4M3FN codes in one dword (byte i = code of v[i]).
MOE_DEV uint32_t cvt_e4m3x4(float a, float b, float c, float d) {
  a = __builtin_fminf(__builtin_fmaxf(a, -448.0f), 448.0f);
  b = __builtin_fminf(__builtin_fmaxf(b, -448.0f), 448.0f);
  c = __builtin_fminf(__builtin_fmaxf(c, -448.0f), 448.0f);
  d = __builtin_fminf(__builtin_fmaxf(d, -448.0f), 448.0f);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return (uint32_t)r;
}

// Smallest power of two >= x for a positive float x (x itself when it is
// one), at least 2^-127, and the exact reciprocal of such a power of two.
MOE_DEV float pow2_at_least(float x) {
  const uint32_t b = __float_as_uint(x);
  // fp32 subnormals: 2^-126 above 2^-127, else 2^-127, the smallest power of
  // two an E8M0 scale holds (so every scale this returns is an E8M0 value)
  if ((b >> 23) == 0) return __uint_as_float(b > 0x00400000u ? 0x00800000u : 0x00400000u);
  return (b & 0x7FFFFFu) ? __uint_as_float(((b >> 23) + 1) << 23) : x;
}
MOE_DEV float pow2_reciprocal(float p) { return __uint_as_float((254u - (__float_as_uint(p) >> 23)) << 23); }
// E8M0 byte (biased exponent) of a power-of-two float.
MOE_DEV int e8m0_of_pow2(float p) { return (int)((__float_as_uint(p) >> 23) & 0xFFu); }

// silu(g) = g * sigmoid(g); the reciprocal is the hardware one (1 ulp).
MOE_DEV float silu_f32(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// 16x16x32 fp16 MFMA: lane l supplies A[l%16][8*(l/16)+i], B[8*(l/16)+i][l%16];
// accumulator element i of lane l is C[4*(l/16)+i][l%16].
MOE_DEV f32x4 mfma_f16_16x16x32(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
MOE_DEV f32x4 mfma_bf16_16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 16x16x128 E4M3 x E4M3 MFMA, no scaling.  Lane l supplies 32 bytes of row
// (A) / column (B) l%16; any K assignment shared by A and B gives the dot
// product.
MOE_DEV f32x4 mfma_fp8_16x16x128(const i32x8& a, const i32x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// 16x16x128 E4M3 (A) x E2M1 (B) MFMA with E8M0 block scales.  Layout on gfx950:
//   A lane l: bytes 0..15 = A[l%16][16*(l/16) + i], bytes 16..31 = A[l%16][64 + 16*(l/16) + i]
//   B lane l: 32 nibbles (low first) = B[32*(l/16) + i][l%16]
//   scale byte 0 of lane l: A row l%16 (resp. B column l%16), K block l/16 (k in [32j, 32j+32))
MOE_DEV f32x4 mfma_fp8_fp4_scaled_16x16x128(const i32x8& a, const i32x4& b, int sa, int sb, const f32x4& c) {
  i32x8 bb = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bb, c, 0, 4, 0, sa, 0, sb);
}

MOE_DEV int lane_id() { return (int)(threadIdx.x & 63); }

// Workgroup barrier that orders LDS only.  __syncthreads() also fences global
// memory, which makes every wave wait for all of its outstanding global loads
// (s_waitcnt vmcnt(0)) and so cancels any prefetch that runs across the
// barrier; the GEMM main loops keep weight loads in flight across K steps.
MOE_DEV void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <typename T>
MOE_DEV T shfl_xor(T v, int mask) { return __shfl_xor(v, mask, 64); }

// Writes a tile of ROWS rows staged in LDS (row stride LS bytes, RB bytes per
// row in 16-byte pieces) to global memory: row r goes to g + r * gs, rows at
// or beyond nrows are skipped.  NT threads share the pieces; each thread
// reads its pieces in groups of up to GMAX (at most four) before storing
// them, so the LDS latency is paid once per group rather than once per piece
// (the outer loop stays rolled to keep the calling kernel's registers down).
template <int ROWS, int RB, int LS, int NT, int GMAX = 4>
MOE_DEV void copy_out_rows(const uint8_t* lds, char* g, int64_t gs, int nrows) {
  constexpr int PPR = RB / 16;
  constexpr int NP = ROWS * PPR;
  constexpr int NI = (NP + NT - 1) / NT;
  constexpr int G = (NI % 4 == 0 && GMAX >= 4) ? 4 : ((NI % 2 == 0 && GMAX >= 2) ? 2 : 1);
#pragma unroll 1
  for (int j0 = 0; j0 < NI; j0 += G) {
    u32x4 v[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int c = min((int)threadIdx.x + (j0 + j) * NT, NP - 1);
      v[j] = *reinterpret_cast<const u32x4*>(lds + (c / PPR) * LS + (c % PPR) * 16);
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int c = (int)threadIdx.x + (j0 + j) * NT, row = c / PPR;
      if (c < NP && row < nrows) *reinterpret_cast<u32x4*>(g + row * gs + (c % PPR) * 16) = v[j];
    }
  }
}

// Maximum of non-negative floats (e.g. |x|) over the 16 lanes of a DPP row
// (lanes 16r .. 16r+15), returned in every lane of the row: quad swaps
// (xor 1, xor 2), then row rotations by 4 and 8, register to register.  For
// non-negative IEEE values the integer order of the bit patterns is the
// numeric order (a NaN, all exponent bits set, wins).
template <int CTRL>
MOE_DEV int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
MOE_DEV float row16_max_nonneg(float v) {
  int x = __float_as_int(v);
  x = max(x, dpp_i32<0xB1>(x));   // quad_perm [1,0,3,2]
  x = max(x, dpp_i32<0x4E>(x));   // quad_perm [2,3,0,1]
  x = max(x, dpp_i32<0x124>(x));  // row_ror:4
  x = max(x, dpp_i32<0x128>(x));  // row_ror:8
  return __int_as_float(x);
}
// The same for four values, the four reductions interleaved so that no DPP
// read directly follows the write of its operand (no wait states between).
MOE_DEV void row16_max_nonneg4(float (&v)[4]) {
  int x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = __float_as_int(v[i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = max(x[i], dpp_i32<0xB1>(x[i]));
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = max(x[i], dpp_i32<0x4E>(x[i]));
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = max(x[i], dpp_i32<0x124>(x[i]));
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = max(x[i], dpp_i32<0x128>(x[i]));
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __int_as_float(x[i]);
}

// Position of element n inside the INT4-path activation layout: every aligned
// group of 8 fp16 values is stored in the order [0,4,1,5,2,6,3,7], matching
// the order in which the in-register INT4 unpack produces weight pairs.
MOE_DEV int i4act_pos(int n) { return (n & ~7) | ((n & 3) << 1) | ((n >> 2) & 1); }

// ---- direct global -> LDS loads (gfx950 global_load_lds_*) ----------------
// Each lane moves its bytes to LDS at  base + lane * size  (base in M0; the
// base must be wave-uniform).  These loads count on the vector-memory counter
// like any other load; the GEMM main loops issue only these in their K loops
// and wait for exactly the stage they need with wait_vmcnt<N>().  Loads the
// compiler issues elsewhere are younger or older than the awaited ones, so
// they can only make such a wait longer, never too short.
MOE_DEV uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
MOE_DEV void dma_b128(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(g) : "memory");
}
// The same for data read once (non-temporal: streamed past the caches'
// normal allocation), e.g. weight slices that no other work item reads.
MOE_DEV void dma_b128_nt(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(g) : "memory");
}
MOE_DEV void dma_b32(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(g) : "memory");
}
MOE_DEV void dma_b16(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_ushort %1, off" ::"s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(g) : "memory");
}
MOE_DEV void dma_b8(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_ubyte %1, off" ::"s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(g) : "memory");
}
// Wave-uniform read through the scalar unit (constant address space), so that
// it is counted by lgkmcnt and never by the vmcnt that the LDS-DMA rings wait on.
MOE_DEV float ld_uniform_f32(const float* p) { return *(const __attribute__((address_space(4))) float*)p; }
template <int N>
MOE_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Wait until at most n (wave-uniform) stages of NPER loads each are in
// flight.  Counts above the counter's range (63) are clamped, which only
// waits longer.
template <int N>
MOE_DEV void wait_vmcnt_clamped() { wait_vmcnt<(N > 63 ? 63 : N)>(); }
// As wait_stages, when the stages in flight also hold `extra` (0 or 1) more
// loads of this wave.
template <int NPER>
MOE_DEV void wait_stages_x(int n, int extra) {
  if (extra == 0) {
    if (n >= 3) wait_vmcnt_clamped<3 * NPER>();
    else if (n == 2) wait_vmcnt_clamped<2 * NPER>();
    else if (n == 1) wait_vmcnt_clamped<NPER>();
    else wait_vmcnt<0>();
  } else {
    if (n >= 3) wait_vmcnt_clamped<3 * NPER + 1>();
    else if (n == 2) wait_vmcnt_clamped<2 * NPER + 1>();
    else if (n == 1) wait_vmcnt_clamped<NPER + 1>();
    else wait_vmcnt<0>();
  }
}
template <int NPER>
MOE_DEV void wait_stages(int n) {
  if (n >= 5) wait_vmcnt_clamped<5 * NPER>();
  else if (n == 4) wait_vmcnt_clamped<4 * NPER>();
  else if (n == 3) wait_vmcnt_clamped<3 * NPER>();
  else if (n == 2) wait_vmcnt_clamped<2 * NPER>();
  else if (n == 1) wait_vmcnt_clamped<NPER>();
  else wait_vmcnt<0>();
}
