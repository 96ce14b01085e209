// Device helpers shared by the gfx950 kernels: bf16/fp16 bit helpers, wave
// reductions, and the decode of the packed group-RTN unit.
//
// Packed unit (format version 1): 32 codes of b bits in b little-endian u32
// words.  Each 16-bit half of a word holds F = 16/b fields from bit 0 up; the
// bits above the fields hold the codes that do not fit (b = 3, 5, 6).  Field
// j of the low half and field j of the high half of one word form a code
// pair; a pair becomes one bf16x2 operand with a single shift and a masked
// OR into 0x4300 (bf16 128.0, whose 7 mantissa bits weigh 1, 2, ..., 64).
// A b-bit code placed at mantissa bit p reads as 128 + q*2^p, so the
// matching activation is pre-scaled by 2^-p (exact in bf16) and the bias
// 128*x*2^-p is removed once per unit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr uint32_t kBias2 = 0x43004300u;  // two bf16 128.0

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16x2 with the hardware round-to-nearest-even
// conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes of a wave, returned as a wave-uniform value.
// DPP butterflies inside each 16-lane row (quad swaps, half-row and row
// mirrors), then the four row sums are read out with v_readlane.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v);  // row_half_mirror
  v += dpp_f32<0x140>(v);  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// ------------------------------------------------------------- buffer loads
// Weight streams are read through buffer resources: 32-bit byte offsets, the
// wave-uniform row offset in an SGPR, hardware range checking (a load past
// num_records returns 0, so no lane ever needs a branch or a clamp to stay
// in bounds).  aux = 2 sets the nontemporal bit: the packed weights are read
// once per call (measured on MI355X: ~7.1 TB/s streaming with nontemporal
// 16-byte loads vs ~6.3 TB/s without).
constexpr int kNT = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

template <int B, int AUX = kNT>
__device__ __forceinline__ void buf_load_unit(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                              uint32_t (&w)[B]) {
  if constexpr (B == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, AUX);
    w[0] = v[0]; w[1] = v[1];
  } else if constexpr (B == 3) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, AUX);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2];
  } else {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
    if constexpr (B == 5) {
      w[4] = __builtin_amdgcn_raw_buffer_load_b32(r, voff + 16, soff, AUX);
    } else if constexpr (B == 6) {
      const auto t = __builtin_amdgcn_raw_buffer_load_b64(r, voff + 16, soff, AUX);
      w[4] = t[0]; w[5] = t[1];
    }
  }
}
__device__ __forceinline__ uint32_t buf_load_u32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kNT);
}

// ---------------------------------------------------------------- unit layout
// Pair k of a unit (k = 0..15): low-half code ca, high-half code cb and the
// mantissa bit p the fields land on after decode.
struct PairInfo { int ca, cb, p; };

template <int B> struct Unit {
  // landing-bit classes: codes decoded at mantissa bit p = 0, 2, 4 (b = 2),
  // p = 0, 3 (b = 3), p = 0 (b >= 4)
  static constexpr int NCLS = B == 2 ? 3 : (B == 3 ? 2 : 1);
  static constexpr int cls_of_p(int p) { return B == 2 ? p / 2 : (B == 3 ? p / 3 : 0); }
  static constexpr int F = 16 / B;                 // fields per half-word
  static constexpr int kRegularPairs = F * B;      // F pairs per word, B words
  // shift that brings field j near bit 0, and its landing bit p
  static constexpr int shift_of(int j) {
    return B == 2 ? 6 * (j / 3) : B == 3 ? 6 * (j / 2) : B * j;
  }
  static constexpr int p_of(int j) {
    return B == 2 ? 2 * (j % 3) : B == 3 ? 3 * (j % 2) : 0;
  }
  static constexpr PairInfo pair(int k) {
    if (k < kRegularPairs) {
      const int w = k / F, j = k % F;
      return PairInfo{2 * F * w + j, 2 * F * w + F + j, p_of(j)};
    }
    if (B == 3 || B == 5) return PairInfo{30, 31, 0};
    const int pp = k - kRegularPairs;               // B == 6: spare pairs
    return PairInfo{24 + pp, 28 + pp, 0};
  }
};

// The bias is kept in an opaque register so (x & mask) | bias compiles to a
// single v_and_or_b32 (gfx9 VOP3 takes no literal operands; with both
// constants visible the compiler would emit v_and_b32 + v_or_b32 instead).
__device__ __forceinline__ uint32_t opaque_bias() {
  uint32_t b = kBias2;
  asm volatile("" : "+v"(b));
  return b;
}

// Decode one unit (B words) into 16 bf16x2 operands (128 + q*2^p per lane).
template <int B>
__device__ __forceinline__ void decode_unit(const uint32_t (&w)[B], uint32_t (&pr)[16], uint32_t bias) {
  using U = Unit<B>;
#pragma unroll
  for (int k = 0; k < U::kRegularPairs; ++k) {
    const int wi = k / U::F, j = k % U::F;
    const uint32_t m = ((1u << B) - 1u) << U::p_of(j);
    const uint32_t mask = m | (m << 16);
    pr[k] = ((w[wi] >> U::shift_of(j)) & mask) | bias;
  }
  if constexpr (B == 3 || B == 5) {
    uint32_t t = bias;
#pragma unroll
    for (int i = 0; i < B; ++i) t = ((w[i] >> (15 - i)) & (0x00010001u << i)) | t;
    pr[15] = t;
  } else if constexpr (B == 6) {
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const uint32_t lo = ((w[pp] >> 12) & 0x000F000Fu) | bias;
      pr[12 + pp] = ((w[4 + pp / 2] >> (8 + 2 * (pp % 2))) & 0x00300030u) | lo;
    }
  }
}
template <int B>
__device__ __forceinline__ void decode_unit(const uint32_t (&w)[B], uint32_t (&pr)[16]) {
  decode_unit<B>(w, pr, kBias2);
}

// Second decode of the same unit, for kernels that dequantize with
// v_fma_mix_f32: a field is masked into the mantissa of an fp16 with zero
// exponent, i.e. the subnormal q*2^(p-24), with no bias to remove.  Fields
// land at bit p <= 10 - b; a shift by S = b*floor(10/b) brings the upper
// fields down.  Then fma(v, s*2^(24-p), o) = fl32(q*s + o) exactly, since
// q*s has at most 17 significant bits.
template <int B> struct UnitH {
  static constexpr int F = 16 / B;
  static constexpr int S = B * (10 / B);
  static constexpr int kRegularPairs = F * B;
  static constexpr int NCLS = (S - 1) / B + 1;     // landing bits 0, B, ..., < S
  static constexpr int shift_of(int j) { return (B * j / S) * S; }
  static constexpr int p_of(int j) { return B * j - shift_of(j); }
  static constexpr PairInfo pair(int k) { return Unit<B>::pair(k); }
  static constexpr int p_of_pair(int k) { return k < kRegularPairs ? p_of(k % F) : 0; }
};

template <int B>
__device__ __forceinline__ void decode_unit_h(const uint32_t (&w)[B], uint32_t (&pr)[16]) {
  using U = UnitH<B>;
#pragma unroll
  for (int k = 0; k < U::kRegularPairs; ++k) {
    const int wi = k / U::F, j = k % U::F;
    const uint32_t m = ((1u << B) - 1u) << U::p_of(j);
    pr[k] = (w[wi] >> U::shift_of(j)) & (m | (m << 16));
  }
  if constexpr (B == 3 || B == 5) {
    uint32_t t = 0;
#pragma unroll
    for (int i = 0; i < B; ++i) t |= (w[i] >> (15 - i)) & (0x00010001u << i);
    pr[15] = t;
  } else if constexpr (B == 6) {
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const uint32_t lo = (w[pp] >> 12) & 0x000F000Fu;
      pr[12 + pp] = ((w[4 + pp / 2] >> (8 + 2 * (pp % 2))) & 0x00300030u) | lo;
    }
  }
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w)[0]; }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w)[1]; }

// Codes of one unit as fp32 values q (exact), natural code order.
template <int B>
__device__ __forceinline__ void unit_codes_f32(const uint32_t (&w)[B], float (&q)[32]) {
  uint32_t pr[16];
  decode_unit<B>(w, pr);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const PairInfo pi = Unit<B>::pair(k);
    const float inv = 1.0f / (float)(1 << pi.p);
    q[pi.ca] = (bf16_lo_to_f32(pr[k]) - 128.0f) * inv;
    q[pi.cb] = (bf16_hi_to_f32(pr[k]) - 128.0f) * inv;
  }
}

}  // namespace qg
