// Binary low-rank GEMV, W ~ s1 (.) (U+-1 V+-1^T) (.) s2^T ("70B en 4GB de
// VRAM...", section 1, NanoQuant formulation), read right to left:
//   stage 1  t = V^T (s2 (.) x)       rows of VTbits, reduction over K
//   stage 2  y = s1 (.) (U t)         rows of Ubits,  reduction over r
// Both stages are one kernel: a +-1 row dotted with a vector v,
//   sum_k (2 b_k - 1) v_k = 2 * sum_{b_k = 1} v_k - sum_k v_k.
// A lane owns one 32-bit word (32 signs) per row.  Bit j of the low half and
// bit j of the high half form a pair; one shift and one masked OR turn a
// pair into a bf16x2 operand 128 + b*2^p (p = landing mantissa bit), so the
// matching v is pre-scaled by 2^-p and the bias 128*v*2^-p is removed once
// per word.  v (s2*x in stage 1, t in stage 2) is fp32 and is carried as
// bf16 hi + lo halves (two v_dot2 per pair, 2^-16 relative residual).
#include "common.hpp"
#include "launch.hpp"

#ifndef QG_BIN_RPW
#define QG_BIN_RPW 8   // rows per pipeline stage (each row is one 4-byte word per lane)
#endif

namespace qg {

// word layout of a 32-sign word: pair j (0..15) = bits (j, 16+j)
__device__ __forceinline__ constexpr int bin_shift(int j) { return j < 7 ? 0 : (j < 14 ? 7 : 14); }
__device__ __forceinline__ constexpr int bin_p(int j) { return j - bin_shift(j); }

// MODE 0: v = s2 * x (x bf16), output t (fp32)
// MODE 1: v = s2 * x (x fp32), output t (fp32)
// MODE 2: v = t (fp32), output y = s1 * dot (fp32 or bf16)
template <int MODE, int UI, int RPW>
__global__ __launch_bounds__(512) void bin_gemv_kernel(
    const uint32_t* __restrict__ bits, int R, int Wn, int Lk, const void* __restrict__ vin,
    const uint16_t* __restrict__ vscale, const uint16_t* __restrict__ oscale,
    void* __restrict__ out, int y_bf16, int S, int RS, int WSL, int TMAX, int64_t in_bstride,
    int64_t out_bstride, int vec_ok) {
  extern __shared__ float part[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int sl = wave % S, rs = wave / S;
  const int b = blockIdx.y;
  const int Wv = (Lk + 31) >> 5;   // words holding real entries

  int widx[UI];
#pragma unroll
  for (int it = 0; it < UI; ++it) {
    const int lw = it * 64 + lane;
    const int wi = sl * WSL + lw;
    widx[it] = ((lw < WSL) && (wi < Wv)) ? wi : -1;
  }
  const int nstreams = gridDim.x * RS;
  const int stream = blockIdx.x * RS + rs;
  uint32_t wa[RPW][UI], wb[RPW][UI];
  // Sign words through a buffer resource: rows past R read 0 (never stored),
  // lanes without a word have zero activations.
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(bits, (uint32_t)((size_t)R * Wn * 4));
  uint32_t wvoff[UI];
#pragma unroll
  for (int it = 0; it < UI; ++it) wvoff[it] = (uint32_t)(sl * WSL + it * 64 + lane) * 4;
  const uint32_t wrow = (uint32_t)Wn * 4;
  auto load = [&](uint32_t (&w)[RPW][UI], int row0) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const uint32_t row = (uint32_t)(row0 + r * nstreams);
#pragma unroll
      for (int it = 0; it < UI; ++it) w[r][it] = buf_load_u32(brs, wvoff[it], row * wrow);
    }
  };
  const int step = RPW * nstreams;
  const int nst = stream < R ? (R - stream + step - 1) / step : 0;

  // vector: clamped unconditional loads before the first weight stage
  constexpr int XW = MODE == 0 ? 4 : 8;
  u32x4_t vraw[UI][XW], sraw[UI][4];
  const bool vec_tile = vec_ok && (Lk % 32 == 0);
  if (vec_tile) {
#pragma unroll
    for (int it = 0; it < UI; ++it) {
      const int k0 = (widx[it] >= 0 ? widx[it] : 0) * 32;
      const u32x4_t* src = MODE == 0
          ? reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(vin) + in_bstride * b + k0)
          : reinterpret_cast<const u32x4_t*>(static_cast<const float*>(vin) + in_bstride * b + k0);
#pragma unroll
      for (int i = 0; i < XW; ++i) vraw[it][i] = src[i];
      if constexpr (MODE != 2) {
        const u32x4_t* sp = reinterpret_cast<const u32x4_t*>(vscale + k0);
#pragma unroll
        for (int i = 0; i < 4; ++i) sraw[it][i] = sp[i];
      }
    }
  }
  if (nst > 0) load(wa, stream);

  uint32_t xp[UI][32];
  float negC[UI], vsum[UI];
#pragma unroll
  for (int it = 0; it < UI; ++it) {
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = 0.f;
    const int wi = widx[it];
    if (vec_tile) {
      const bool ok = wi >= 0;
#pragma unroll
      for (int i = 0; i < XW; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (MODE == 0) {
            v[8 * i + 2 * j] = ok ? bf16_lo_to_f32(vraw[it][i][j]) : 0.f;
            v[8 * i + 2 * j + 1] = ok ? bf16_hi_to_f32(vraw[it][i][j]) : 0.f;
          } else {
            v[4 * i + j] = ok ? __uint_as_float(vraw[it][i][j]) : 0.f;
          }
        }
      if constexpr (MODE != 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[8 * i + 2 * j] *= f16_bits_to_f32(sraw[it][i][j] & 0xFFFFu);
            v[8 * i + 2 * j + 1] *= f16_bits_to_f32(sraw[it][i][j] >> 16);
          }
      }
    } else if (wi >= 0) {
      const int k0 = wi * 32;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int k = k0 + i;
        if (k < Lk) {
          float xv;
          if constexpr (MODE == 0) xv = bf16_bits_to_f32(static_cast<const uint16_t*>(vin)[in_bstride * b + k]);
          else xv = static_cast<const float*>(vin)[in_bstride * b + k];
          if constexpr (MODE != 2) xv *= f16_bits_to_f32(vscale[k]);
          v[i] = xv;
        }
      }
    }
    // pairs (v_j, v_16+j) pre-scaled by 2^-p (exact), split into bf16
    // hi + lo with the hardware round-to-nearest conversion; the sums come
    // out of v_dot2 against (1, 1) on the very operands the rows will use.
    constexpr uint32_t kOnes = 0x3F803F80u;
    float c = 0.f, vs = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float sc = 1.0f / (float)(1 << bin_p(j));
      const float a = v[j] * sc, bb = v[16 + j] * sc;
      const uint32_t hi = cvt_pk_bf16(a, bb);
      const uint32_t lo = cvt_pk_bf16(a - bf16_lo_to_f32(hi), bb - bf16_hi_to_f32(hi));
      xp[it][2 * j] = hi;
      xp[it][2 * j + 1] = lo;
      c = dot2_bf16(hi, kOnes, c);
      c = dot2_bf16(lo, kOnes, c);
      vs += v[j] + v[16 + j];
    }
    negC[it] = -128.0f * c;
    vsum[it] = vs;
  }

  auto emit = [&](int row, float total) {
    if constexpr (MODE == 2) {
      const float yv = total * f16_bits_to_f32(oscale[row]);
      if (y_bf16) static_cast<uint16_t*>(out)[out_bstride * b + row] = (uint16_t)f32_to_bf16_rne(yv);
      else static_cast<float*>(out)[out_bstride * b + row] = yv;
    } else {
      static_cast<float*>(out)[out_bstride * b + row] = total;
    }
  };
  const uint32_t bias = opaque_bias();
  auto compute = [&](const uint32_t (&w)[RPW][UI], int row0, int m0) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int it = 0; it < UI; ++it) {
        float a = negC[it];
        const uint32_t ww = w[r][it];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const uint32_t m = 0x00010001u << bin_p(j);
          const uint32_t pr = ((ww >> bin_shift(j)) & m) | bias;
          a = dot2_bf16(pr, xp[it][2 * j], a);
          a = dot2_bf16(pr, xp[it][2 * j + 1], a);
        }
        acc += 2.0f * a - vsum[it];
      }
      const float total = wave_sum(acc);
      const int row = row0 + r * nstreams;
      if (row < R && lane == 0) {
        if (S == 1) emit(row, total);
        else part[((size_t)rs * TMAX + (m0 + r)) * S + sl] = total;
      }
    }
  };

  int st = 0;
  while (st + 2 < nst) {
    load(wb, stream + (st + 1) * step);
    __builtin_amdgcn_sched_barrier(0);  // keep the stage's loads issued here
    compute(wa, stream + st * step, st * RPW);
    load(wa, stream + (st + 2) * step);
    __builtin_amdgcn_sched_barrier(0);  // keep the stage's loads issued here
    compute(wb, stream + (st + 1) * step, (st + 1) * RPW);
    st += 2;
  }
  if (st + 1 < nst) {
    load(wb, stream + (st + 1) * step);
    __builtin_amdgcn_sched_barrier(0);  // keep the stage's loads issued here
    compute(wa, stream + st * step, st * RPW);
    compute(wb, stream + (st + 1) * step, (st + 1) * RPW);
  } else if (st < nst) {
    compute(wa, stream + st * step, st * RPW);
  }
  if (S > 1) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < RS * TMAX; idx += blockDim.x) {
      const int rs_ = idx / TMAX, m = idx % TMAX;
      const int row = blockIdx.x * RS + rs_ + m * nstreams;
      if (row < R) {
        float t = 0.f;
        for (int j = 0; j < S; ++j) t += part[(size_t)idx * S + j];
        emit(row, t);
      }
    }
  }
}

template <int MODE>
static hipError_t bin_gemv_t(const uint32_t* bits, int64_t R, int64_t Wn, int64_t Lk,
                             const void* vin, const uint16_t* vscale, const uint16_t* oscale,
                             void* out, int y_bf16, int64_t B, int64_t in_bstride,
                             int64_t out_bstride, hipStream_t s) {
  constexpr int UI = 2, RPW = QG_BIN_RPW;
  constexpr int64_t kTargetWaves = 2048;
  const int Wv = (int)((Lk + 31) / 32);
  int S = (Wv + 64 * UI - 1) / (64 * UI);
  if (S > 8) return hipErrorInvalidValue;
  while (S < 4 && R * S < kTargetWaves && (Wv + 2 * S - 1) / (2 * S) >= 64) S *= 2;
  const int RS = S <= 4 ? 4 / S : 1;
  const int WSL = (Wv + S - 1) / S;
  const int threads = 64 * S * RS;
  // rows per stream: a whole number of RPW-row stages, no decoded-but-idle rows
  const int64_t streams_target = kTargetWaves / S;
  const int64_t stages = (R + RPW * streams_target - 1) / (RPW * streams_target);
  const int64_t rows_per_stream = RPW * stages;
  int64_t blocks = ((R + rows_per_stream - 1) / rows_per_stream + RS - 1) / RS;
  if (blocks < 1) blocks = 1;
  const int64_t nstreams = blocks * RS;
  const int TMAX = (int)((R + nstreams - 1) / nstreams);
  const size_t lds = S > 1 ? (size_t)RS * TMAX * S * sizeof(float) : 0;
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  const size_t esz = MODE == 0 ? 2 : 4;
  const int vec_ok = ((reinterpret_cast<uintptr_t>(vin) % 16) == 0 && ((in_bstride * esz) % 16) == 0 &&
                      (MODE == 2 || (reinterpret_cast<uintptr_t>(vscale) % 16) == 0)) ? 1 : 0;
  hipLaunchKernelGGL((bin_gemv_kernel<MODE, UI, RPW>), dim3((unsigned)blocks, (unsigned)B),
                     dim3(threads), lds, s, bits, (int)R, (int)Wn, (int)Lk, vin, vscale, oscale,
                     out, y_bf16, S, RS, WSL, TMAX, in_bstride, out_bstride, vec_ok);
  return hipGetLastError();
}

static int64_t pw(int64_t n) { return ((n + 31) / 32 + 3) / 4 * 4; }

hipError_t launch_gemv_binlr(const uint32_t* ubits, const uint32_t* vtbits,
                             const uint16_t* s1, const uint16_t* s2, int64_t N, int64_t K,
                             int64_t r, const void* x, int x_dtype, int64_t B, void* y,
                             int y_dtype, float* t_ws, hipStream_t s) {
  const int64_t rp = pw(r) * 32;   // workspace row stride of t
  hipError_t e;
  if (x_dtype == 1)
    e = bin_gemv_t<0>(vtbits, r, pw(K), K, x, s2, nullptr, t_ws, 0, B, K, rp, s);
  else
    e = bin_gemv_t<1>(vtbits, r, pw(K), K, x, s2, nullptr, t_ws, 0, B, K, rp, s);
  if (e != hipSuccess) return e;
  return bin_gemv_t<2>(ubits, N, pw(r), r, t_ws, nullptr, s1, y, y_dtype == 1, B, rp, N, s);
}

}  // namespace qg
