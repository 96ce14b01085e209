// Decode of group codes read through per-group books of a shared dictionary
// (shared by the decode GEMV and the prefill GEMM kernels).
#pragma once
#include "common.hpp"

namespace qg {

// ----------------------------------------------------- per-group codebooks
// Codebook format ("TurboQuant: cuantizar modelos grandes...", introduction
// and "Compresión por bloques": block compression with a shared dictionary,
// a compressed codebook per group): a dictionary of up to 16 books of 2^b
// byte entries e <= 127 is shared by a matrix; each group names one book in
// a byte, and code q of the group stands for the level e[q] / 2^(7-b) in
// code units, w_hat = s * e[q] / 2^(7-b) + o.
struct Books { const uint8_t* ids; const uint8_t* dict; int n; };   // n = 0: plain codes

// Decode one unit through its book T (the book's entries as bytes, little
// endian) into the 16 bf16x2 operands of decode_unit, 128 + e[q] per lane in
// the pair order of Unit<B> (every pair lands at mantissa bit 0).  The
// lookups are byte permutes: each code becomes a selector byte of
// v_perm_b32 over the table words.  2-bit codes: four codes per permute,
// one table word.  3-bit codes: one pair per permute over two table words.
// 4-bit codes: four codes per two permutes (entries 0..7 and 8..15) plus a
// third that keeps, byte by byte, the half that code bit 3 names.  A final
// permute or masked OR writes the 0x43 high bytes (bf16 128 + e, exact for
// e <= 127), or, with F16, zero high bytes: the fp16 subnormal e * 2^-24,
// which v_fma_mix_f32 scales and offsets in one instruction.
// Constants of the lookups, held in opaque registers (made once per kernel)
// so the masked ORs compile to single v_and_or_b32 (gfx9 VOP3 takes no
// literal operands).
struct CbConst { uint32_t m4, blend, lo16, bias; };
__device__ __forceinline__ CbConst cb_consts() {
  CbConst k{0x04040404u, 0x03020100u, 0x00FF00FFu, 0x43004300u};
  asm volatile("" : "+v"(k.m4), "+v"(k.blend), "+v"(k.lo16), "+v"(k.bias));
  return k;
}

template <int B, bool F16 = false>
__device__ __forceinline__ void decode_unit_cb(const uint32_t (&w)[B], const uint32_t (&T)[4],
                                               uint32_t (&pr)[16], const CbConst& kc) {
  constexpr uint32_t k43 = F16 ? 0u : 0x43434343u;
  if constexpr (B == 2) {
#pragma unroll
    for (int wi = 0; wi < 2; ++wi)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // bytes: low-half fields j, j+4, high-half fields j, j+4
        const uint32_t r = __builtin_amdgcn_perm(0u, T[0], (w[wi] >> (2 * j)) & 0x03030303u);
        pr[8 * wi + j] = __builtin_amdgcn_perm(k43, r, 0x04020400u);
        pr[8 * wi + j + 4] = __builtin_amdgcn_perm(k43, r, 0x04030401u);
      }
  } else if constexpr (B == 3) {
    auto look = [&](uint32_t t) {
      const uint32_t v = __builtin_amdgcn_perm(T[1], T[0], t) & kc.lo16;
      return F16 ? v : (v | kc.bias);
    };
#pragma unroll
    for (int k = 0; k < 15; ++k) pr[k] = look((w[k / 5] >> (3 * (k % 5))) & 0x00070007u);
    uint32_t t = 0;
#pragma unroll
    for (int i = 0; i < 3; ++i) t |= (w[i] >> (15 - i)) & (0x00010001u << i);
    pr[15] = look(t);
  } else {
    static_assert(B == 4, "codebooks hold 4, 8 or 16 entries");
    // a: the codes' low 3 bits (selectors into entries 0..7 and 8..15);
    // sh: the word shifted so each code's bit 3 sits at bit 2 of its byte,
    // giving the byte-wise choice between the two halves.
    auto look = [&](uint32_t a, uint32_t sh) {
      const uint32_t lo = __builtin_amdgcn_perm(T[1], T[0], a);
      const uint32_t hi = __builtin_amdgcn_perm(T[3], T[2], a);
      return __builtin_amdgcn_perm(hi, lo, (sh & kc.m4) | kc.blend);
    };
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
      // bytes: low-half fields 0, 2, high-half fields 0, 2 (then 1, 3)
      const uint32_t x = w[wi];
      const uint32_t r0 = look(x & 0x07070707u, x >> 1);
      const uint32_t r1 = look((x >> 4) & 0x07070707u, x >> 5);
      pr[4 * wi + 0] = __builtin_amdgcn_perm(k43, r0, 0x04020400u);
      pr[4 * wi + 2] = __builtin_amdgcn_perm(k43, r0, 0x04030401u);
      pr[4 * wi + 1] = __builtin_amdgcn_perm(k43, r1, 0x04020400u);
      pr[4 * wi + 3] = __builtin_amdgcn_perm(k43, r1, 0x04030401u);
    }
  }
}

}  // namespace qg
