// INT4 unpack and the LDS stage layout shared by the forward and backward
// INT4 grouped GEMMs.
#pragma once
#include "common.h"

namespace moe {

// 8 INT4 codes (one dword, element i in bits 4i..4i+3, two's complement) times
// scale s -> 8 fp16 values ordered (0,4),(1,5),(2,6),(3,7).  This is the
// "magic number" conversion of Kim et al., "Who Says Elephants Can't Run"
// (2022): each pair comes from one bitop3 that keeps the two code fields,
// flips their sign bit (q + 8) and sets the exponent of 1024, i.e. fp16
// 1024 + (q + 8) for codes in bits 0-3 / 16-19, or 1024 + 16 (q + 8) for
// codes in bits 4-7 / 20-23 (still inside the 10-bit mantissa, so no shift is
// needed).  Subtracting 1032 gives q; for the second form one fused
// multiply-add v/16 - 72 gives q (every intermediate is an integer below
// 2048, exact in fp16).  Multiplying by s then gives q s, exact in fp16
// whenever it is representable: s in [2^-17, 8188] for bf16 scales (at most
// 3 + 8 significant bits, lowest bit at or above fp16's 2^-24, |q s| < 65504).
// bitop3 truth table 0x6A: b ? (c ? ~a : a) : c.
MOE_DEV f16x2 int4_pair_hi(uint32_t d) {
  const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const f16x2 bias = {(_Float16)-72.0f, (_Float16)-72.0f};
  return __builtin_elementwise_fma(__builtin_bit_cast(f16x2, d), sixteenth, bias);
}
MOE_DEV f16x8 int4x8_to_f16(uint32_t w, f16x2 s2) {
  const f16x2 bias0 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const uint32_t v = w >> 8;
  const uint32_t d0 = __builtin_amdgcn_bitop3_b32(w, 0x000F000Fu, 0x64086408u, 0x6A);
  const uint32_t d1 = __builtin_amdgcn_bitop3_b32(w, 0x00F000F0u, 0x64806480u, 0x6A);
  const uint32_t d2 = __builtin_amdgcn_bitop3_b32(v, 0x000F000Fu, 0x64086408u, 0x6A);
  const uint32_t d3 = __builtin_amdgcn_bitop3_b32(v, 0x00F000F0u, 0x64806480u, 0x6A);
  const f16x2 h0 = (__builtin_bit_cast(f16x2, d0) + bias0) * s2;
  const f16x2 h1 = int4_pair_hi(d1) * s2;
  const f16x2 h2 = (__builtin_bit_cast(f16x2, d2) + bias0) * s2;
  const f16x2 h3 = int4_pair_hi(d3) * s2;
  f16x8 r = {h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
  return r;
}

MOE_DEV uint32_t dword_of(const u32x4& v, int s) { return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w; }

// LDS bytes of one pipeline stage: activation rows (256 B = 128 fp16 each,
// 16-byte parts XOR-swizzled by row), each wave's weight fragments (NS
// subtiles x 1 KB of nibbles) and the bf16 group scales of the wave's NS*16
// weight rows for the step's 4 groups (NS*128 B).  Scales are stored
// group-major, so those are 4 (GEMM2) or 8 (GEMM1: gate and up) contiguous
// runs of 16-byte pieces, one per lane.  (Per-row scale requests, 64 per
// wave per step, were measured to cost more time than the weight nibbles
// themselves.)
//
// KS = 64 (INT4 only): a stage holds 64 K, i.e. activation rows of 128 B,
// NS subtiles x 512 B of nibbles and the scales of the step's two groups
// (NS*64 B) per wave: about half the LDS of a 128-K stage, so that taller
// tiles keep two workgroups per CU.
template <int BM, int NS = 4, int KS = 128>
struct I4Stage {
  static_assert(KS == 128 || KS == 64, "K step");
  static constexpr bool K64 = KS == 64;
  // activation DMA groups per wave (4 rows of 256 B, or 8 rows of 128 B, each)
  static constexpr int NA = K64 ? (BM + 31) / 32 : BM / 16;
  static constexpr int A_BYTES = NA * 4 * 1024;
  static constexpr int B_OFF = A_BYTES;
  static constexpr int BS_OFF = B_OFF + 4 * NS * (KS * 8);
  static constexpr int BYTES = BS_OFF + 4 * NS * KS;
  // Workgroups per CU (measured on MI355X): two at 16 (four subtiles), 48
  // and 64 rows and with 64-K stages, where a second resident workgroup
  // covers one's item start-up and waits; three at 16 rows with two
  // subtiles (INT4 decode: more items start and end at different times, 2%
  // faster than two with deeper rings); one at 32 rows (a deeper ring wins
  // there) and above 64 rows with 128-K stages, where the activation tile
  // fills the LDS.
  static constexpr int WPC = (BM == 16 && NS == 2) ? 3 : ((K64 || BM == 16 || BM == 48 || BM == 64) ? 2 : 1);
  static constexpr int SMAX = BM <= 32 ? 7 : 5;
  // LDS for the rings: 152 KB of the CU's 160, or all but 256 B per
  // workgroup with three of them (four 13-KB decode stages each: 2% faster
  // than three)
  static constexpr int LDS = WPC == 3 ? 160 * 1024 - 3 * 256 : 152 * 1024;
  static constexpr int S = (LDS / WPC) / BYTES > SMAX ? SMAX : (LDS / WPC) / BYTES;  // stages
  // DMA instructions per wave per stage (64-K steps: one per two subtiles)
  static constexpr int NPER = NA + (K64 ? NS / 2 : NS) + 1;
};

// The same 8 codes with one scale per element: sc holds the fp16 pairs
// {s0, s4}, {s1, s5}, {s2, s6}, {s3, s7} for elements 0..7 (the layout the
// backward weight copy stores), output order as above.
MOE_DEV f16x8 int4x8_to_f16_se(uint32_t w, const u32x4& sc) {
  const f16x2 bias0 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const uint32_t v = w >> 8;
  const uint32_t d0 = __builtin_amdgcn_bitop3_b32(w, 0x000F000Fu, 0x64086408u, 0x6A);
  const uint32_t d1 = __builtin_amdgcn_bitop3_b32(w, 0x00F000F0u, 0x64806480u, 0x6A);
  const uint32_t d2 = __builtin_amdgcn_bitop3_b32(v, 0x000F000Fu, 0x64086408u, 0x6A);
  const uint32_t d3 = __builtin_amdgcn_bitop3_b32(v, 0x00F000F0u, 0x64806480u, 0x6A);
  // scalar copies first: a bit cast of a vector element expression (sc.y)
  // reads from the start of the vector, i.e. sc.x
  const uint32_t s0 = sc.x, s1 = sc.y, s2 = sc.z, s3 = sc.w;
  const f16x2 h0 = (__builtin_bit_cast(f16x2, d0) + bias0) * __builtin_bit_cast(f16x2, s0);
  const f16x2 h1 = int4_pair_hi(d1) * __builtin_bit_cast(f16x2, s1);
  const f16x2 h2 = (__builtin_bit_cast(f16x2, d2) + bias0) * __builtin_bit_cast(f16x2, s2);
  const f16x2 h3 = int4_pair_hi(d3) * __builtin_bit_cast(f16x2, s3);
  f16x8 r = {h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
  return r;
}

}  // namespace moe
