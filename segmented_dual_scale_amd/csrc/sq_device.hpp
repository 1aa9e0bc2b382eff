// sq_device.hpp -- device helpers shared by the gfx950 kernels of libsegquant.
//
// [P1] "SegQuant: A Semantics-Aware and Generalizable Quantization Framework
//      for Diffusion Models" (papernotes.org notes), "DualScale" section.
// [P2] "SegQuant" (hliangzhao.me), section 3, polarity-aware quantisation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

// 1.5 * 2^23: adding it to a float v with |v| < 2^22 rounds v to the nearest
// integer, ties to even (the sum lands where the fp32 spacing is exactly 1
// and 1.5*2^23 is even), and leaves that integer in the low mantissa bits:
// bits(v + kMagic) = 0x4B400000 + rne(v).  For a code q in [-128, 127] the low
// byte is q's two's-complement byte and byte 1 is 0xFF when q < 0, else 0x00.
constexpr float kMagic = 12582912.0f;
constexpr uint32_t kMagicBits = 0x4B400000u;

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// DualScale code of one activation [P2 s.3 Q_dual; P1 DualScale]: the sign of
// x picks the half (x < 0 -> the - half), then one fp32 multiply by that
// half's inverse scale, clamp to [-128, 127] (the two halves' ranges [0,127]
// and [-128,0] joined: the product keeps the sign of x), round half to even.
// Returns the magic word described above (code in byte 0, sign in byte 1).
// A zero inverse gives +-0 -> code 0 (that half is all zeros).
__device__ __forceinline__ uint32_t quant_magic(float x, float inv_pos, float inv_neg) {
  float inv = x < 0.0f ? inv_neg : inv_pos;
  float v = x * inv;
  v = __builtin_amdgcn_fmed3f(v, -128.0f, 127.0f);
  return __float_as_uint(v + kMagic);
}

// Byte permute with the 8 source bytes numbered 0..3 = lo4, 4..7 = hi4.
__device__ __forceinline__ uint32_t pick(uint32_t lo4, uint32_t hi4, uint32_t sel) {
  return __builtin_amdgcn_perm(hi4, lo4, sel);
}

// Four magic words (elements k..k+3) -> the packed signed codes q (byte i =
// code of element k+i) and the packed sign masks m (0xFF where negative).
__device__ __forceinline__ void pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                      uint32_t &q, uint32_t &m) {
  uint32_t t1 = pick(a, b, 0x05010400u);  // [a0 b0 a1 b1]
  uint32_t t2 = pick(c, d, 0x05010400u);  // [c0 d0 c1 d1]
  q = pick(t1, t2, 0x05040100u);          // [a0 b0 c0 d0]
  m = pick(t1, t2, 0x07060302u);          // [a1 b1 c1 d1]
}

// Eight bf16 (one 16-byte load, element order) -> two dwords of the + plane
// and two of the - plane.  The halves have disjoint support, so each plane is
// the signed code masked by the sign.
__device__ __forceinline__ void quant8_planes(v4u x, float inv_pos, float inv_neg, v2u &pos,
                                              v2u &neg) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t u0 = x[2 * h], u1 = x[2 * h + 1];
    uint32_t a = quant_magic(bf16_lo(u0), inv_pos, inv_neg);
    uint32_t b = quant_magic(bf16_hi(u0), inv_pos, inv_neg);
    uint32_t c = quant_magic(bf16_lo(u1), inv_pos, inv_neg);
    uint32_t d = quant_magic(bf16_hi(u1), inv_pos, inv_neg);
    uint32_t q, m;
    pack4(a, b, c, d, q, m);
    neg[h] = q & m;
    pos[h] = q ^ neg[h];
  }
}

// Eight bf16 -> two dwords of signed codes (q+ + q-).
__device__ __forceinline__ v2u quant8_signed(v4u x, float inv_pos, float inv_neg) {
  v2u out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t u0 = x[2 * h], u1 = x[2 * h + 1];
    uint32_t a = quant_magic(bf16_lo(u0), inv_pos, inv_neg);
    uint32_t b = quant_magic(bf16_hi(u0), inv_pos, inv_neg);
    uint32_t c = quant_magic(bf16_lo(u1), inv_pos, inv_neg);
    uint32_t d = quant_magic(bf16_hi(u1), inv_pos, inv_neg);
    uint32_t t1 = pick(a, b, 0x05010400u);
    uint32_t t2 = pick(c, d, 0x05010400u);
    out[h] = pick(t1, t2, 0x05040100u);
  }
  return out;
}

// Signed codes (4 per dword) -> the - plane (bytes with the sign bit set) and
// the + plane (the rest).  The byte mask m is 0xff where the sign bit is set:
// t holds the sign bits, t - (t >> 7) is 0x7f in those bytes (no borrow
// crosses a byte), and OR-ing t back gives 0xff.  (Full-rate integer ops; a
// multiply by 0xff would be a quarter-rate instruction.)
__device__ __forceinline__ void split_signed(uint32_t q, uint32_t &pos, uint32_t &neg) {
  const uint32_t t = q & 0x80808080u;
  const uint32_t m = (t - (t >> 7)) | t;
  neg = q & m;
  pos = q ^ neg;
}

// A 4-bit weight lane-row (8 bytes of codes biased by +8, so 1..15) -> the
// 16 signed int8 bytes of its matrix-core operand.  In each dword the low
// nibbles are operand bytes 0-3 and the high nibbles bytes 4-7 of that
// half; (v + 0x78) ^ 0x80 maps a biased nibble v to the byte v - 8 with no
// carry between bytes (v + 0x78 <= 0x87).
__device__ __forceinline__ v4u unpack_w4(v2u u) {
  v4u o;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    o[2 * h] = ((u[h] & 0x0f0f0f0fu) + 0x78787878u) ^ 0x80808080u;
    o[2 * h + 1] = (((u[h] >> 4) & 0x0f0f0f0fu) + 0x78787878u) ^ 0x80808080u;
  }
  return o;
}

// fp32 -> bf16 bits, round to nearest even (finite values; NaN stays NaN).
// A select, not a branch: in a store epilogue the branch cost more than the
// arithmetic.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet = (u >> 16) | 0x40u;
  return (u & 0x7fffffffu) > 0x7f800000u ? quiet : rounded;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Non-negative floats order like their bit patterns: the reductions below
// take atomic max over uint32 bits.
__device__ __forceinline__ float pos_part(float x) { return x > 0.0f ? x : 0.0f; }
__device__ __forceinline__ float neg_mag(float x) { return x < 0.0f ? -x : 0.0f; }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Scale and inverse of a non-negative range a over q levels [P2 s.3]:
// fp64 quotients rounded once to fp32.  A zero range, or one so small that
// its inverse overflows fp32, is treated as zero: scale 0 and inverse 0.
__device__ __forceinline__ void scale_pair(float a, double q, float &s, float &inv) {
  float iv = a > 0.0f ? (float)(q / (double)a) : 0.0f;
  if (iv > 3.40282346638528859812e38f) iv = 0.0f;  // +inf
  s = iv == 0.0f ? 0.0f : (float)((double)a / q);
  inv = iv;
}

}  // namespace sq
