// Group-RTN GEMV for decode, y[b][n] = sum_k (s*q[n][k] + o) x[b][k].
//
// A decode step reads every weight byte once and does two flops per weight,
// so it is bound by HBM bytes ("AirLLM corre un modelo 70B...", "Por qué es
// lento": time ~ bytes moved / bandwidth).  The kernels therefore stream the
// packed codes with coalesced vector loads, never write dequantized weights
// anywhere, and keep the per-weight ALU work small:
//
//  * B = 1 (VALU): a lane owns one 32-code unit per row.  Its activations
//    are turned once into bf16 pairs pre-scaled for the landing bit of each
//    code (see common.hpp) and held in registers for every row the wave
//    visits.  Per row a code pair costs one shift + one masked OR + one
//    v_dot2_f32_bf16; the 128*x bias and the group constants are applied once
//    per unit: y += s*(sum (128+q)x - 128 sum x) + o*sum x.  The weights are
//    exact in bf16, so the only roundings are fp32 accumulations.  Long rows
//    are split into up to 4 K-slices, one per wave of a workgroup, combined in
//    LDS.  fp32 activations are split into bf16 hi + lo halves (two dot2).
//  * 2 <= B <= 16 (MFMA): a wave owns a 16-row tile; each lane decodes one
//    unit per K-step to fp32 w_hat = s*q + o, rounds to bf16 and feeds
//    v_mfma_f32_16x16x32_bf16 with the activations (bf16) as the 16-column
//    operand, fp32 accumulation.
#include "common.hpp"
#include "launch.hpp"

namespace qg {

template <int B>
__device__ __forceinline__ void load_unit(const uint32_t* __restrict__ p, uint32_t (&w)[B]) {
  if constexpr (B == 4) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else if constexpr (B == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else if constexpr (B == 6) {
    const uint2* q = reinterpret_cast<const uint2*>(p);
#pragma unroll
    for (int i = 0; i < 3; ++i) { const uint2 v = q[i]; w[2 * i] = v.x; w[2 * i + 1] = v.y; }
  } else {
#pragma unroll
    for (int i = 0; i < B; ++i) w[i] = p[i];
  }
}

// ------------------------------------------------------------------ B = 1
template <int BITS, int G, bool XF32, int UI, int RPW>
__global__ __launch_bounds__(256) void gemv_b1_kernel(
    const uint32_t* __restrict__ codes, const uint32_t* __restrict__ meta, int N, int K,
    const void* __restrict__ xin, void* __restrict__ yout, int y_bf16, int S, int RS, int USL,
    int TMAX) {
  extern __shared__ float part[];
  constexpr int XS = XF32 ? 2 : 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sl = wave % S, rs = wave / S;
  const int U = K >> 5;
  const int GN = K / G;

  uint32_t xp[UI][16 * XS];
  float negC[UI], xsum[UI];
  int uidx[UI];
#pragma unroll
  for (int it = 0; it < UI; ++it) {
    const int lu = it * 64 + lane;
    const int u = sl * USL + lu;
    const bool v = (lu < USL) && (u < U);
    uidx[it] = v ? u : -1;
    float xv[32];
    if (v) {
      if constexpr (XF32) {
        const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(xin) + (size_t)u * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float4 t = src[i];
          xv[4 * i] = t.x; xv[4 * i + 1] = t.y; xv[4 * i + 2] = t.z; xv[4 * i + 3] = t.w;
        }
      } else {
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(xin) + (size_t)u * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4_t t = src[i];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            xv[8 * i + 2 * j] = bf16_lo_to_f32(t[j]);
            xv[8 * i + 2 * j + 1] = bf16_hi_to_f32(t[j]);
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) xv[i] = 0.f;
    }
    float c = 0.f, xs = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const PairInfo pi = Unit<BITS>::pair(k);
      const float sc = 1.0f / (float)(1 << pi.p);
      const float a = xv[pi.ca] * sc, b = xv[pi.cb] * sc;
      if constexpr (XF32) {
        const uint32_t ah = f32_to_bf16_rne(a), bh = f32_to_bf16_rne(b);
        const float al = a - bf16_bits_to_f32(ah), bl = b - bf16_bits_to_f32(bh);
        const uint32_t alb = f32_to_bf16_rne(al), blb = f32_to_bf16_rne(bl);
        xp[it][2 * k] = ah | (bh << 16);
        xp[it][2 * k + 1] = alb | (blb << 16);
        c += (bf16_bits_to_f32(ah) + bf16_bits_to_f32(alb)) + (bf16_bits_to_f32(bh) + bf16_bits_to_f32(blb));
      } else {
        xp[it][k] = (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
        c += a + b;
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) xs += xv[i];
    negC[it] = -128.0f * c;
    xsum[it] = xs;
  }

  const int nstreams = gridDim.x * RS;
  const int stream = blockIdx.x * RS + rs;
  for (int m0 = 0;; m0 += RPW) {
    const int row0 = stream + m0 * nstreams;
    if (row0 >= N) break;
    uint32_t wv[RPW][UI][BITS];
    uint32_t mv[RPW][UI];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int row = row0 + r * nstreams;
#pragma unroll
      for (int it = 0; it < UI; ++it) {
        if (row < N && uidx[it] >= 0) {
          load_unit<BITS>(codes + ((size_t)row * U + uidx[it]) * BITS, wv[r][it]);
          mv[r][it] = meta[(size_t)row * GN + (uidx[it] * 32) / G];
        } else {
#pragma unroll
          for (int i = 0; i < BITS; ++i) wv[r][it][i] = 0u;
          mv[r][it] = 0u;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      float acc_row = 0.f;
#pragma unroll
      for (int it = 0; it < UI; ++it) {
        uint32_t pr[16];
        decode_unit<BITS>(wv[r][it], pr);
        float a = negC[it];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          a = dot2_bf16(pr[k], xp[it][k * XS], a);
          if constexpr (XF32) a = dot2_bf16(pr[k], xp[it][k * XS + 1], a);
        }
        const float s = f16_bits_to_f32(mv[r][it] & 0xFFFFu);
        const float o = f16_bits_to_f32(mv[r][it] >> 16);
        acc_row = __builtin_fmaf(s, a, __builtin_fmaf(o, xsum[it], acc_row));
      }
      const float total = wave_sum(acc_row);
      const int row = row0 + r * nstreams;
      if (row < N && lane == 0) {
        if (S == 1) {
          if (y_bf16) static_cast<uint16_t*>(yout)[row] = (uint16_t)f32_to_bf16_rne(total);
          else static_cast<float*>(yout)[row] = total;
        } else {
          part[((size_t)rs * TMAX + (m0 + r)) * S + sl] = total;
        }
      }
    }
  }
  if (S > 1) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < RS * TMAX; idx += blockDim.x) {
      const int rs_ = idx / TMAX, m = idx % TMAX;
      const int row = blockIdx.x * RS + rs_ + m * nstreams;
      if (row < N) {
        float t = 0.f;
        for (int j = 0; j < S; ++j) t += part[(size_t)idx * S + j];
        if (y_bf16) static_cast<uint16_t*>(yout)[row] = (uint16_t)f32_to_bf16_rne(t);
        else static_cast<float*>(yout)[row] = t;
      }
    }
  }
}

// --------------------------------------------------------------- B = 2..16
template <int BITS, int G>
__global__ __launch_bounds__(256) void gemv_mfma_kernel(
    const uint32_t* __restrict__ codes, const uint32_t* __restrict__ meta, int N, int K,
    const uint16_t* __restrict__ x, int B, void* __restrict__ yout, int y_bf16) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * 4 + wave) * 16;
  if (row0 >= N) return;
  const int r = lane & 15, kg = lane >> 4;
  const int row = row0 + r;
  const bool rvalid = row < N;
  const int U = K >> 5, GN = K / G;
  const int bcol = lane & 15;
  const bool bvalid = bcol < B;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const int nq = (U + 3) >> 2;
  for (int qi = 0; qi < nq; ++qi) {
    const int u = 4 * qi + kg;
    const bool uvalid = u < U;
    uint32_t w[BITS];
    uint32_t m = 0u;
    if (rvalid && uvalid) {
      load_unit<BITS>(codes + ((size_t)row * U + u) * BITS, w);
      m = meta[(size_t)row * GN + (u * 32) / G];
    } else {
#pragma unroll
      for (int i = 0; i < BITS; ++i) w[i] = 0u;
    }
    u32x4_t xb[4];
    if (bvalid && uvalid) {
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + (size_t)bcol * K + (size_t)u * 32);
#pragma unroll
      for (int t = 0; t < 4; ++t) xb[t] = src[t];
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) xb[t] = u32x4_t{0u, 0u, 0u, 0u};
    }
    float qf[32];
    unit_codes_f32<BITS>(w, qf);
    const float s = f16_bits_to_f32(m & 0xFFFFu), o = f16_bits_to_f32(m >> 16);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4_t a;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        a[j] = pack_bf16x2(__builtin_fmaf(s, qf[8 * t + 2 * j], o),
                           __builtin_fmaf(s, qf[8 * t + 2 * j + 1], o));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                    __builtin_bit_cast(bf16x8_t, xb[t]), acc,
                                                    0, 0, 0);
    }
  }
  if (bvalid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ro = row0 + 4 * kg + i;
      if (ro < N) {
        if (y_bf16) static_cast<uint16_t*>(yout)[(size_t)bcol * N + ro] = (uint16_t)f32_to_bf16_rne(acc[i]);
        else static_cast<float*>(yout)[(size_t)bcol * N + ro] = acc[i];
      }
    }
  }
}

// --------------------------------------------------------------- launchers
template <int BITS, int G, bool XF32, int UI, int RPW>
static hipError_t gemv_b1_t(const uint32_t* codes, const uint32_t* meta, int64_t N, int64_t K,
                            const void* x, void* y, int y_bf16, hipStream_t s) {
  const int U = (int)(K / 32);
  const int S = (U + 64 * UI - 1) / (64 * UI);
  if (S > 4) return hipErrorInvalidValue;
  const int RS = 4 / S;
  const int USL = (U + S - 1) / S;
  const int threads = 64 * S * RS;
  const int64_t streams_wanted = (N + 15) / 16;  // about 16 rows per wave
  int64_t blocks = (streams_wanted + RS - 1) / RS;
  if (blocks < 1) blocks = 1;
  if (blocks > 2048) blocks = 2048;
  const int64_t nstreams = blocks * RS;
  const int TMAX = (int)((N + nstreams - 1) / nstreams);
  const size_t lds = S > 1 ? (size_t)RS * TMAX * S * sizeof(float) : 0;
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemv_b1_kernel<BITS, G, XF32, UI, RPW>), dim3((unsigned)blocks),
                     dim3(threads), lds, s, codes, meta, (int)N, (int)K, x, y, y_bf16, S, RS, USL,
                     TMAX);
  return hipGetLastError();
}

template <int BITS, int G>
static hipError_t gemv_mfma_t(const uint32_t* codes, const uint32_t* meta, int64_t N, int64_t K,
                              const uint16_t* x, int64_t B, void* y, int y_bf16, hipStream_t s) {
  const int64_t tiles = (N + 15) / 16;
  const int64_t blocks = (tiles + 3) / 4;
  hipLaunchKernelGGL((gemv_mfma_kernel<BITS, G>), dim3((unsigned)blocks), dim3(256), 0, s, codes,
                     meta, (int)N, (int)K, x, (int)B, y, y_bf16);
  return hipGetLastError();
}

template <int BITS, int G>
static hipError_t gemv_dispatch(const uint32_t* codes, const uint32_t* meta, int64_t N,
                                int64_t K, const void* x, int x_dtype, int64_t B, void* y,
                                int y_bf16, hipStream_t s) {
  if (B == 1) {
    if (x_dtype == 0) return gemv_b1_t<BITS, G, true, 2, 2>(codes, meta, N, K, x, y, y_bf16, s);
    return gemv_b1_t<BITS, G, false, 4, 2>(codes, meta, N, K, x, y, y_bf16, s);
  }
  if (x_dtype != 1) return hipErrorInvalidValue;
  return gemv_mfma_t<BITS, G>(codes, meta, N, K, static_cast<const uint16_t*>(x), B, y, y_bf16, s);
}

hipError_t launch_gemv_group(const uint32_t* codes, const uint32_t* meta, int64_t N,
                             int64_t K, int bits, int group, const void* x, int x_dtype,
                             int64_t B, void* y, int y_dtype, hipStream_t s) {
  const int yb = y_dtype == 1;
#define CALL(b, g) gemv_dispatch<b, g>(codes, meta, N, K, x, x_dtype, B, y, yb, s)
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

}  // namespace qg
