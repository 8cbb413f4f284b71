// Device-side building blocks of the AWQ W4A16 kernels (gfx950 only).
//
// Layout facts used throughout (tensref.org "AWQ" format page, Reader; GPTQModel
// wiki "AWQ", section "Saved formats and packing"):
//   word (k, c) of qweight holds, in bits 4i..4i+3, the code of column 8c + ORDER[i]
//   with ORDER = {0,2,4,6,1,3,5,7}.  Byte t of the word therefore holds two columns:
//   its low nibble (nibble 2t) is column ORDER[2t] and its high nibble (nibble 2t+1)
//   is column ORDER[2t+1]:
//       byte 0 -> columns 0 (low), 2 (high)     byte 1 -> columns 4, 6
//       byte 2 -> columns 1, 3                  byte 3 -> columns 5, 7
//   qzeros words use the same packing; dequant is (q - z) * s with the stored zero.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "awq_kernels.h"

namespace awq {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// bfloat16 <-> float.  A bfloat16 is the top half of a binary32, so widening is a
// shift; narrowing rounds to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two floats -> packed bfloat16 pair (low half = a), rounded to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const float __attribute__((ext_vector_type(2))) f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// Activations as raw 16-bit patterns: fp16 or (BF16) bfloat16.
template <bool BF16>
__device__ __forceinline__ float act_to_float(uint16_t b) {
  if constexpr (BF16) return bf16_bits_to_float(b);
  else return (float)__builtin_bit_cast(_Float16, b);
}
template <bool BF16>
__device__ __forceinline__ uint16_t float_to_act(float f) {
  if constexpr (BF16) return float_to_bf16_bits(f);
  else return __builtin_bit_cast(uint16_t, (_Float16)f);
}
// Two rounded activations packed in one word (low half = a).
template <bool BF16>
__device__ __forceinline__ uint32_t pack_act2(float a, float b) {
  if constexpr (BF16) return pack_bf16x2(a, b);
  else return __builtin_bit_cast(uint32_t, half2v{(_Float16)a, (_Float16)b});
}

// Column held by the low / high nibble of byte t (see the table above).
__host__ __device__ constexpr int lo_col(int t) { return ((t & 1) << 2) | (t >> 1); }
__host__ __device__ constexpr int hi_col(int t) { return lo_col(t) + 2; }
// Nibble index (0..7) that holds column j of a word: the inverse of ORDER.
__host__ __device__ constexpr int nibble_of_col(int j) {
  return (j & 1) ? (4 + (j >> 1)) : (j >> 1);
}

static_assert(lo_col(0) == 0 && hi_col(0) == 2 && lo_col(1) == 4 && hi_col(1) == 6, "byte->column table");
static_assert(lo_col(2) == 1 && hi_col(2) == 3 && lo_col(3) == 5 && hi_col(3) == 7, "byte->column table");
static_assert(nibble_of_col(0) == 0 && nibble_of_col(1) == 4 && nibble_of_col(2) == 1 && nibble_of_col(3) == 5 &&
              nibble_of_col(4) == 2 && nibble_of_col(5) == 6 && nibble_of_col(6) == 3 && nibble_of_col(7) == 7,
              "column->nibble table");

__device__ __forceinline__ uint32_t as_u32(half2v h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ half2v as_h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }

// Interleave byte t of two words a (row r) and b (row r+1): result bytes are
// [a.t, 0, b.t, 0], so the low nibbles of byte t sit in bits 0-3 / 16-19 and the
// high nibbles in bits 4-7 / 20-23 of the two 16-bit halves.
template <int t>
__device__ __forceinline__ uint32_t pair_byte(uint32_t a, uint32_t b) {
  constexpr uint32_t sel = (uint32_t)t | (0x0Cu << 8) | ((uint32_t)(4 + t) << 16) | (0x0Cu << 24);
  return __builtin_amdgcn_perm(b, a, sel);
}

// Bit masks of the unpack, held in VGPRs.  gfx9 VOP3 encodings take no literal
// constants, so with literals the compiler splits (p & mask) | magic into two
// instructions; opaque register copies let it emit one v_and_or_b32.
struct UnpackConsts {
  uint32_t magic, mlo, mhi, bmagic;
};
__device__ __forceinline__ UnpackConsts unpack_consts() {
  UnpackConsts k{0x64006400u, 0x000F000Fu, 0x00F000F0u, 0x43004300u};
  asm volatile("" : "+v"(k.magic), "+v"(k.mlo), "+v"(k.mhi), "+v"(k.bmagic));
  return k;
}

// bfloat16 pair (128 + lo_a, 128 + lo_b): 0x4300 is 128.0 and 128..255 are exact in
// bfloat16 (7 fraction bits), so the nibble ORed into the fraction is exact.  A
// high nibble (bits 4-7 would reach the exponent) is shifted down first.
__device__ __forceinline__ uint32_t lo_magic_bf16(uint32_t p, const UnpackConsts& k) { return (p & k.mlo) | k.bmagic; }
__device__ __forceinline__ uint32_t hi_magic_bf16(uint32_t p, const UnpackConsts& k) {
  return ((p >> 4) & k.mlo) | k.bmagic;
}

// fp16 pair (1024 + lo_a, 1024 + lo_b): the nibble ORed into the mantissa of 1024.0
// (0x6400) gives the integer exactly, since 1024..2047 are exact in fp16.
__device__ __forceinline__ half2v lo_magic(uint32_t p, const UnpackConsts& k) { return as_h2((p & k.mlo) | k.magic); }
// fp16 pair (1024 + 16*hi_a, 1024 + 16*hi_b), also exact.
__device__ __forceinline__ half2v hi_magic(uint32_t p, const UnpackConsts& k) { return as_h2((p & k.mhi) | k.magic); }

// (code - zero) as exact small fp16 integers from the magic forms.
//   lo: (1024 + q) - (1024 + z)                      one packed add
//   hi: (1024 + 16 q) / 16 - (64 + z) = q - z         one packed fma, exact
__device__ __forceinline__ half2v lo_minus_zero(uint32_t p, half2v neg_1024_plus_z, const UnpackConsts& k) {
  return lo_magic(p, k) + neg_1024_plus_z;
}
__device__ __forceinline__ half2v hi_minus_zero(uint32_t p, half2v neg_64_plus_z, const UnpackConsts& k) {
  const half2v sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  return __builtin_elementwise_fma(hi_magic(p, k), sixteenth, neg_64_plus_z);
}

// Zero code of column j of a packed zero word.
__device__ __forceinline__ uint32_t zero_code(uint32_t zw, int j) {
  return (zw >> (4 * nibble_of_col(j))) & 0xFu;
}

__device__ __forceinline__ half2v splat(_Float16 v) { return half2v{v, v}; }

// ---- Split-K sums in 64-bit fixed point, one word per output element.
// Each of the `splits` workgroups that share an output element adds its fp32 partial p
// with one returning atomic; the word is zero between calls (the workgroup that
// completes it writes the output and clears it).  Layout of the word:
//   bits 63..57  arrivals: workgroups that have added their partial (<= 127)
//   bits 56..50  exceptional arrivals: partials that are NaN, +-inf or |p| >= 2^18
//   bits 49..0   signed sum of rint(p * 2^24) over the other partials
// Integer addition does not depend on order, so the sum is reproducible bit for bit;
// every fp16 value is a multiple of 2^-24, so a sum of exact products stays exact.
// An exceptional partial cannot be held in fixed point: it is added in fp32 to a float
// side word of the same element (zero between calls) before its arrival is counted,
// and the workgroup that completes the element adds that side word back.  The side
// add is released before the arrival (agent-scope fence) and the completing workgroup
// acquires before it reads, so it sees every side add: NaN, infinities and huge
// partials reach the output as an fp32 sum would produce them.  Normal partials are
// below 2^18 in magnitude, 2^42 in fixed point, so kFxMaxSplits = 127 of them stay
// below 2^49.
constexpr float kFxScale = 16777216.0f;  // 2^24
constexpr float kFxLimit = 262144.0f;    // 2^18

// False for NaN, +-inf and partials of magnitude >= 2^18.
__device__ __forceinline__ bool fx_normal(float p) { return __builtin_fabsf(p) < kFxLimit; }

// The word a workgroup adds for its partial p.
__device__ __forceinline__ uint64_t fx_word(float p) {
  const uint64_t arrival = 1ull << 57;
  if (fx_normal(p)) return arrival + (uint64_t)(int64_t)__builtin_rintf(p * kFxScale);
  return arrival + (1ull << 50);
}

struct FxSum {
  int64_t value;  // sum of the normal partials, in units of 2^-24
  uint32_t marks;  // exceptional partials (their fp32 sum is in the side word)
  uint32_t arrivals;
};
// Splits the word returned by an add (old value + the word added).
__device__ __forceinline__ FxSum fx_decode(uint64_t w) {
  const int64_t value = (int64_t)(w << 14) >> 14;  // low 50 bits, sign-extended
  const uint64_t rest = (w - (uint64_t)value) >> 50;  // arrivals * 128 + marks, exact
  return FxSum{value, (uint32_t)(rest & 127u), (uint32_t)(rest >> 7)};
}

// Side add of an exceptional partial (before its word is added).  After all side adds
// of the calling wave, fx_release() must precede the word adds.
__device__ __forceinline__ void fx_side_add(float* side, float p) {
  __hip_atomic_fetch_add(side, p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fx_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ uint64_t fx_add(uint64_t* word, uint64_t add) {
  return __hip_atomic_fetch_add(word, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + add;
}
// The completed element's fp32 sum (for the workgroup whose add brought the arrivals to
// `splits`); clears the side word.  The caller clears the 64-bit word.
__device__ __forceinline__ float fx_total(const FxSum& s, float* side) {
  float v = (float)s.value * (1.0f / kFxScale);
  if (s.marks != 0) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    v += __hip_atomic_exchange(side, 0.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return v;
}
__device__ __forceinline__ void fx_clear(uint64_t* word) {
  __hip_atomic_store(word, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sum over s < splits of the 4 floats at p + s * stride, added in split order (the
// same order, so the same bits, for every call).  The loads of the first B splits go
// out together (with B >= splits, one round trip to memory), the rest 8 at a time; a
// load past the last split re-reads the last one (in bounds) and is not added.
template <int B>
__device__ __forceinline__ floatx4 sum_splits(const float* __restrict__ p, int64_t stride, int splits) {
  floatx4 v[B];
#pragma unroll
  for (int j = 0; j < B; ++j) v[j] = *reinterpret_cast<const floatx4*>(p + (int64_t)min(j, splits - 1) * stride);
  floatx4 a = v[0];
#pragma unroll
  for (int j = 1; j < B; ++j)
    if (j < splits) a += v[j];
  for (int s = B; s < splits; s += 8) {
    floatx4 w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = *reinterpret_cast<const floatx4*>(p + (int64_t)min(s + j, splits - 1) * stride);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s + j < splits) a += w[j];
  }
  return a;
}

// Loads in the first batch of sum_splits for a given split count.
constexpr int split_batch(int splits) { return splits <= 4 ? 4 : (splits <= 8 ? 8 : 16); }

// Cache policy (sc1) of loads and stores that every XCD must see alike: each XCD has its
// own L2, so partial sums exchanged between workgroups inside one kernel are written
// through to, and read back from, the device-wide point of coherence, which is what
// agent-scope atomic stores and loads compile to.
constexpr int kCpolDevice = 16;

}  // namespace awq
