// Prefill GEMM, Y[M][N] = X[M][K] W_hat^T, for both weight formats.
//
// Prefill multiplies many token rows by the same weights, so unlike decode it
// is a dense contraction (arithmetic intensity of thousands of flops per
// weight byte) and belongs on the matrix cores.  Each workgroup owns a
// 128 x 128 output tile and walks K in steps of 64:
//   * the X tile (bf16, optionally scaled by s2 and re-rounded) and the
//     decoded weight tile (bf16) are staged in LDS with a padded row pitch of
//     144 bytes so the 16-byte fragment reads of 8 consecutive rows hit
//     distinct banks;
//   * weight decode happens once per workgroup: group RTN unit -> fp32
//     s*q + o -> bf16 (round to nearest even); binary word -> +-1 (exact);
//   * 4 waves in a 2 x 2 layout each run 4 x 4 v_mfma_f32_16x16x32_bf16
//     tiles per 32-wide k slice, fp32 accumulation.
// The binary format runs two passes ("70B en 4GB de VRAM...", section 1):
// T = bf16((X (.) s2) V) into the workspace, then Y = (T U^T) (.) s1.
#include "common.hpp"
#include "launch.hpp"

namespace qg {

constexpr int BM = 128, BN = 128, BK = 64, PITCH = BK + 8;  // bf16 elements

// weight decoders: fill 32 consecutive k of weight row n starting at unit u
template <int BITS, int G>
struct DecRTN {
  const uint32_t* codes; const uint32_t* meta; int N; int U;
  __device__ __forceinline__ void operator()(int n, int u, uint32_t (&outp)[16]) const {
    if (n >= N || u >= U) {
#pragma unroll
      for (int i = 0; i < 16; ++i) outp[i] = 0u;
      return;
    }
    uint32_t w[BITS];
    const uint32_t* p = codes + ((size_t)n * U + u) * BITS;
#pragma unroll
    for (int i = 0; i < BITS; ++i) w[i] = p[i];
    const uint32_t m = meta[(size_t)n * (U * 32 / G) + (u * 32) / G];
    const float s = f16_bits_to_f32(m & 0xFFFFu), o = f16_bits_to_f32(m >> 16);
    float q[32];
    unit_codes_f32<BITS>(w, q);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      outp[i] = pack_bf16x2(__builtin_fmaf(s, q[2 * i], o), __builtin_fmaf(s, q[2 * i + 1], o));
  }
};

struct DecBIN {
  const uint32_t* bits; int N; int Wn;   // rows, words per stored row
  __device__ __forceinline__ void operator()(int n, int u, uint32_t (&outp)[16]) const {
    uint32_t w = 0u;
    const bool ok = n < N && u < Wn;
    if (ok) w = bits[(size_t)n * Wn + u];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // bit -> sign: 1 -> +1.0 (0x3F80), 0 -> -1.0 (0xBF80)
      const uint32_t lo = ((~w >> (2 * i)) & 1u) << 15;
      const uint32_t hi = ((~w >> (2 * i + 1)) & 1u) << 31;
      outp[i] = ok ? (0x3F803F80u | lo | hi) : 0u;
    }
  }
};

// AMODE 0: A = X (bf16).  AMODE 1: A = bf16(X * s2[k]).
// EPI_BF16: output bf16 instead of fp32.  oscale: per-column fp16 scale or null.
template <typename Dec, int AMODE>
__global__ __launch_bounds__(256) void gemm_kernel(const uint16_t* __restrict__ A, int64_t lda,
                                                   int M, int Kact, Dec dec, int N,
                                                   const uint16_t* __restrict__ kscale,
                                                   const uint16_t* __restrict__ oscale,
                                                   void* __restrict__ Y, int64_t ldy, int y_bf16) {
  __shared__ __align__(16) uint16_t As[BM * PITCH];
  __shared__ __align__(16) uint16_t Bs[BN * PITCH];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int ld_row = tid >> 1, ld_half = tid & 1;   // 128 rows x 2 halves of 32
  for (int k0 = 0; k0 < Kact; k0 += BK) {
    // ---- A tile
    {
      const int m = m0 + ld_row;
      const int kb = k0 + ld_half * 32;
      uint32_t v[16];
      if (m < M && kb + 32 <= Kact) {
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(A + (size_t)m * lda + kb);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4_t t = src[i];
          v[4 * i] = t[0]; v[4 * i + 1] = t[1]; v[4 * i + 2] = t[2]; v[4 * i + 3] = t[3];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          uint32_t lo = 0u, hi = 0u;
          if (m < M && kb + 2 * i < Kact) lo = A[(size_t)m * lda + kb + 2 * i];
          if (m < M && kb + 2 * i + 1 < Kact) hi = A[(size_t)m * lda + kb + 2 * i + 1];
          v[i] = lo | (hi << 16);
        }
      }
      if constexpr (AMODE == 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int k = kb + 2 * i;
          const float s0 = k < Kact ? f16_bits_to_f32(kscale[k]) : 0.f;
          const float s1v = k + 1 < Kact ? f16_bits_to_f32(kscale[k + 1]) : 0.f;
          v[i] = pack_bf16x2(bf16_lo_to_f32(v[i]) * s0, bf16_hi_to_f32(v[i]) * s1v);
        }
      }
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(As + ld_row * PITCH + ld_half * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = u32x4_t{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
    }
    // ---- weight tile, decoded once per workgroup
    {
      uint32_t v[16];
      dec(n0 + ld_row, k0 / 32 + ld_half, v);
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(Bs + ld_row * PITCH + ld_half * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = u32x4_t{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
    }
    __syncthreads();
    const int fr = lane & 15, fk = (lane >> 4) * 8;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(As + (wm * 64 + i * 16 + fr) * PITCH + kk + fk);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(Bs + (wn * 64 + j * 16 + fr) * PITCH + kk + fk);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  // ---- epilogue: lane holds D[4*(lane/16) + e][lane % 16] of each 16x16 tile
  const int col_l = lane & 15, row_l = (lane >> 4) * 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn * 64 + j * 16 + col_l;
    if (n >= N) continue;
    const float sc = oscale ? f16_bits_to_f32(oscale[n]) : 1.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm * 64 + i * 16 + row_l + e;
        if (m < M) {
          const float vout = acc[i][j][e] * sc;
          if (y_bf16) static_cast<uint16_t*>(Y)[(size_t)m * ldy + n] = (uint16_t)f32_to_bf16_rne(vout);
          else static_cast<float*>(Y)[(size_t)m * ldy + n] = vout;
        }
      }
    }
  }
}

template <int BITS, int G>
static hipError_t gemm_group_t(const uint32_t* codes, const uint32_t* meta, int64_t N, int64_t K,
                               const uint16_t* X, int64_t M, void* Y, int y_bf16, hipStream_t s) {
  DecRTN<BITS, G> dec{codes, meta, (int)N, (int)(K / 32)};
  dim3 grid((unsigned)((M + BM - 1) / BM), (unsigned)((N + BN - 1) / BN));
  hipLaunchKernelGGL((gemm_kernel<DecRTN<BITS, G>, 0>), grid, dim3(256), 0, s, X, K, (int)M,
                     (int)K, dec, (int)N, (const uint16_t*)nullptr, (const uint16_t*)nullptr, Y,
                     N, y_bf16);
  return hipGetLastError();
}

hipError_t launch_gemm_group(const uint32_t* codes, const uint32_t* meta, int64_t N,
                             int64_t K, int bits, int group, const uint16_t* X, int64_t M,
                             void* Y, int y_dtype, hipStream_t s) {
  const int yb = y_dtype == 1;
#define CALL(b, g) gemm_group_t<b, g>(codes, meta, N, K, X, M, Y, yb, s)
  switch (bits * 100 + group) {
    case 232: return CALL(2, 32); case 264: return CALL(2, 64);
    case 332: return CALL(3, 32); case 364: return CALL(3, 64);
    case 432: return CALL(4, 32); case 464: return CALL(4, 64);
    case 532: return CALL(5, 32); case 564: return CALL(5, 64);
    case 632: return CALL(6, 32); case 664: return CALL(6, 64);
    default: return hipErrorInvalidValue;
  }
#undef CALL
}

static int64_t pwords(int64_t n) { return ((n + 31) / 32 + 3) / 4 * 4; }

hipError_t launch_gemm_binlr(const uint32_t* ubits, const uint32_t* vtbits,
                             const uint16_t* s1, const uint16_t* s2, int64_t N, int64_t K,
                             int64_t r, const uint16_t* X, int64_t M, void* Y, int y_dtype,
                             uint16_t* T_ws, hipStream_t s) {
  const int64_t rp = pwords(r) * 32;
  // pass 1: T[M][rp] = bf16((X * s2) V), weight rows = VT rows (r of them)
  {
    DecBIN dec{vtbits, (int)r, (int)pwords(K)};
    dim3 grid((unsigned)((M + BM - 1) / BM), (unsigned)((r + BN - 1) / BN));
    hipLaunchKernelGGL((gemm_kernel<DecBIN, 1>), grid, dim3(256), 0, s, X, K, (int)M, (int)K,
                       dec, (int)r, s2, (const uint16_t*)nullptr, (void*)T_ws, rp, 1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // pass 2: Y = (T U^T) * s1
  {
    DecBIN dec{ubits, (int)N, (int)pwords(r)};
    dim3 grid((unsigned)((M + BM - 1) / BM), (unsigned)((N + BN - 1) / BN));
    hipLaunchKernelGGL((gemm_kernel<DecBIN, 0>), grid, dim3(256), 0, s, (const uint16_t*)T_ws,
                       rp, (int)M, (int)r, dec, (int)N, (const uint16_t*)nullptr, s1, Y, N,
                       y_dtype == 1);
    return hipGetLastError();
  }
}

}  // namespace qg
