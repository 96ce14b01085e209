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

// Tile parameters of the B = 1 kernel (compile-time).
#ifndef QG_B1_UI
#define QG_B1_UI 2        // units per lane held in registers (K-slice = 2048*UI inputs)
#endif
#ifndef QG_B1_RPW
#define QG_B1_RPW 2       // rows decoded per pipeline stage
#endif
#ifndef QG_B1_WAVES
#define QG_B1_WAVES 0     // target waves per launch; 0 = by shape (8 or 16 per CU)
#endif

namespace qg {

// Packed weights are read exactly once per call: nontemporal loads keep them
// from displacing the activations in the caches (measured on MI355X: ~7.1
// TB/s streaming with nontemporal 16-byte loads vs ~6.3 TB/s without).
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
template <int B>
__device__ __forceinline__ void load_unit(const uint32_t* __restrict__ p, uint32_t (&w)[B]) {
  if constexpr (B == 4) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else if constexpr (B == 2) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    w[0] = v[0]; w[1] = v[1];
  } else if constexpr (B == 6) {
    const u32x2_t* q = reinterpret_cast<const u32x2_t*>(p);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const u32x2_t v = __builtin_nontemporal_load(q + i);
      w[2 * i] = v[0]; w[2 * i + 1] = v[1];
    }
  } else {
#pragma unroll
    for (int i = 0; i < B; ++i) w[i] = __builtin_nontemporal_load(p + i);
  }
}
__device__ __forceinline__ uint32_t load_meta(const uint32_t* __restrict__ p) {
  return __builtin_nontemporal_load(p);
}

// ------------------------------------------------------------------ B = 1
template <int BITS, int G, bool XF32, int UI, int RPW>
__global__ __launch_bounds__(512) void gemv_b1_kernel(
    const uint32_t* __restrict__ codes, const uint32_t* __restrict__ meta, int N, int K,
    const void* __restrict__ xin, void* __restrict__ yout, int y_bf16, int S, int RS, int USL,
    int TMAX) {
  extern __shared__ float part[];
  constexpr int XS = XF32 ? 2 : 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sl = wave % S, rs = wave / S;
  const int U = K >> 5;
  const int GN = K / G;

  int uidx[UI];
#pragma unroll
  for (int it = 0; it < UI; ++it) {
    const int lu = it * 64 + lane;
    const int u = sl * USL + lu;
    uidx[it] = ((lu < USL) && (u < U)) ? u : -1;
  }
  const int nstreams = gridDim.x * RS;
  const int stream = blockIdx.x * RS + rs;

  // Rows are visited in chunks of RPW; the loads of the next chunk are issued
  // before the current chunk is decoded (two register buffers, ping-pong).
  // The first chunk is requested before the activations are prepared.
  uint32_t wa[RPW][UI][BITS], ma[RPW][UI];
  uint32_t wb[RPW][UI][BITS], mb[RPW][UI];
  auto load = [&](uint32_t (&w)[RPW][UI][BITS], uint32_t (&m)[RPW][UI], int row0) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int row = row0 + r * nstreams;
#pragma unroll
      for (int it = 0; it < UI; ++it) {
        if (row < N && uidx[it] >= 0) {
          load_unit<BITS>(codes + ((size_t)row * U + uidx[it]) * BITS, w[r][it]);
          m[r][it] = load_meta(meta + (size_t)row * GN + (uidx[it] * 32) / G);
        } else {
#pragma unroll
          for (int i = 0; i < BITS; ++i) w[r][it][i] = 0u;
          m[r][it] = 0u;
        }
      }
    }
  };
  if (stream < N) load(wa, ma, stream);

  uint32_t xp[UI][16 * XS];
  float negC[UI], xsum[UI];
#pragma unroll
  for (int it = 0; it < UI; ++it) {
    const bool v = uidx[it] >= 0;
    const int u = uidx[it];
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

  auto compute = [&](const uint32_t (&w)[RPW][UI][BITS], const uint32_t (&m)[RPW][UI], int row0, int m0) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      float acc_row = 0.f;
#pragma unroll
      for (int it = 0; it < UI; ++it) {
        uint32_t pr[16];
        decode_unit<BITS>(w[r][it], pr);
        float a = negC[it];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          a = dot2_bf16(pr[k], xp[it][k * XS], a);
          if constexpr (XF32) a = dot2_bf16(pr[k], xp[it][k * XS + 1], a);
        }
        const float s = f16_bits_to_f32(m[r][it] & 0xFFFFu);
        const float o = f16_bits_to_f32(m[r][it] >> 16);
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
  };

  int row0 = stream, m0 = 0;
  const int step = RPW * nstreams;
  while (row0 < N) {
    const int row1 = row0 + step;
    if (row1 < N) load(wb, mb, row1);
    compute(wa, ma, row0, m0);
    if (row1 >= N) break;
    const int row2 = row1 + step;
    if (row2 < N) load(wa, ma, row2);
    compute(wb, mb, row1, m0 + RPW);
    row0 = row2;
    m0 += 2 * RPW;
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
// A workgroup owns RT 16-row tiles; its 4 waves split K (wave w takes unit
// quads w, w+4, ...), so the activation fragments a wave loads are reused by
// RT tiles.  Lane (r, kg) = (lane % 16, lane / 16) decodes unit 4*q + kg of
// row r of every tile; the 4 lane groups therefore cover 4 consecutive units
// (128 inputs) per MFMA quad, and the activation lane (b, kg) loads the
// matching 8-wide slices of x[b].  Partial sums of the 4 waves meet in LDS.
template <int BITS, int G, int RT>
__global__ __launch_bounds__(256) void gemv_mfma_kernel(
    const uint32_t* __restrict__ codes, const uint32_t* __restrict__ meta, int N, int K,
    const uint16_t* __restrict__ x, int B, void* __restrict__ yout, int y_bf16) {
  __shared__ float red[4][RT * 4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row_base = blockIdx.x * (16 * RT);
  const int r = lane & 15, kg = lane >> 4;
  const int U = K >> 5, GN = K / G;
  const int bcol = lane & 15;
  const bool bvalid = bcol < B;
  f32x4_t acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  struct Buf { u32x4_t xb[4]; uint32_t w[RT][BITS]; uint32_t m[RT]; };
  auto load = [&](Buf& b, int qi) {
    const int u = 4 * qi + kg;
    const bool uvalid = u < U;
    if (bvalid && uvalid) {
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + (size_t)bcol * K + (size_t)u * 32);
#pragma unroll
      for (int t = 0; t < 4; ++t) b.xb[t] = src[t];
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) b.xb[t] = u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int row = row_base + 16 * t + r;
      if (row < N && uvalid) {
        load_unit<BITS>(codes + ((size_t)row * U + u) * BITS, b.w[t]);
        b.m[t] = load_meta(meta + (size_t)row * GN + (u * 32) / G);
      } else {
#pragma unroll
        for (int i = 0; i < BITS; ++i) b.w[t][i] = 0u;
        b.m[t] = 0u;
      }
    }
  };
  auto compute = [&](const Buf& b) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      float qf[32];
      unit_codes_f32<BITS>(b.w[t], qf);
      const float s = f16_bits_to_f32(b.m[t] & 0xFFFFu), o = f16_bits_to_f32(b.m[t] >> 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4_t a;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          a[e] = cvt_pk_bf16(__builtin_fmaf(s, qf[8 * j + 2 * e], o), __builtin_fmaf(s, qf[8 * j + 2 * e + 1], o));
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                         __builtin_bit_cast(bf16x8_t, b.xb[j]), acc[t], 0, 0, 0);
      }
    }
  };

  const int nq = (U + 3) >> 2;
  Buf b0, b1;
  int qi = wave;
  if (qi < nq) load(b0, qi);
  while (qi < nq) {
    const int q1 = qi + 4;
    if (q1 < nq) load(b1, q1);
    compute(b0);
    if (q1 >= nq) break;
    const int q2 = q1 + 4;
    if (q2 < nq) load(b0, q2);
    compute(b1);
    qi = q2;
  }
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][t * 4 + i][lane] = acc[t][i];
  __syncthreads();
  // lane holds D[4*kg + i][bcol] of each tile: row 16t + 4kg + i, batch bcol
  for (int v = threadIdx.x; v < RT * 4 * 64; v += 256) {
    const int ti = v / 64, ln = v % 64;
    const float sum = (red[0][ti][ln] + red[1][ti][ln]) + (red[2][ti][ln] + red[3][ti][ln]);
    const int t = ti / 4, i = ti % 4;
    const int b = ln & 15, row = row_base + 16 * t + 4 * (ln >> 4) + i;
    if (b < B && row < N) {
      if (y_bf16) static_cast<uint16_t*>(yout)[(size_t)b * N + row] = (uint16_t)f32_to_bf16_rne(sum);
      else static_cast<float*>(yout)[(size_t)b * N + row] = sum;
    }
  }
}

// --------------------------------------------------------------- launchers
template <int BITS, int G, bool XF32, int UI, int RPW>
static hipError_t gemv_b1_t(const uint32_t* codes, const uint32_t* meta, int64_t N, int64_t K,
                            const void* x, void* y, int y_bf16, hipStream_t s) {
  const int64_t kTargetWaves = QG_B1_WAVES ? QG_B1_WAVES : (N >= 16384 ? 4096 : 2048);
  const int U = (int)(K / 32);
  int S = (U + 64 * UI - 1) / (64 * UI);
  if (S > 8) return hipErrorInvalidValue;
  // short matrices: split K further so the grid still has ~8 waves per CU
  while (S < 4 && N * S < kTargetWaves && (U + 2 * S - 1) / (2 * S) >= 64) S *= 2;
  const int RS = S <= 4 ? 4 / S : 1;   // 256 threads, or 64*S (<= 512) for long rows
  const int USL = (U + S - 1) / S;
  const int threads = 64 * S * RS;
  int64_t nstreams_wanted = kTargetWaves / S;
  if (nstreams_wanted > N) nstreams_wanted = N;
  int64_t blocks = (nstreams_wanted + RS - 1) / RS;
  if (blocks < 1) blocks = 1;
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
  // largest row-tile count that still gives >= 256 workgroups
  if ((N + 63) / 64 >= 256) {
    hipLaunchKernelGGL((gemv_mfma_kernel<BITS, G, 4>), dim3((unsigned)((N + 63) / 64)), dim3(256), 0, s,
                       codes, meta, (int)N, (int)K, x, (int)B, y, y_bf16);
  } else if ((N + 31) / 32 >= 256) {
    hipLaunchKernelGGL((gemv_mfma_kernel<BITS, G, 2>), dim3((unsigned)((N + 31) / 32)), dim3(256), 0, s,
                       codes, meta, (int)N, (int)K, x, (int)B, y, y_bf16);
  } else {
    hipLaunchKernelGGL((gemv_mfma_kernel<BITS, G, 1>), dim3((unsigned)((N + 15) / 16)), dim3(256), 0, s,
                       codes, meta, (int)N, (int)K, x, (int)B, y, y_bf16);
  }
  return hipGetLastError();
}

template <int BITS, int G>
static hipError_t gemv_dispatch(const uint32_t* codes, const uint32_t* meta, int64_t N,
                                int64_t K, const void* x, int x_dtype, int64_t B, void* y,
                                int y_bf16, hipStream_t s) {
  if (B == 1) {
    if (x_dtype == 0) return gemv_b1_t<BITS, G, true, 2, 2>(codes, meta, N, K, x, y, y_bf16, s);
    return gemv_b1_t<BITS, G, false, QG_B1_UI, QG_B1_RPW>(codes, meta, N, K, x, y, y_bf16, s);
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
