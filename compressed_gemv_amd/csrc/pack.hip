// Packers and unpackers for both weight formats (offline, not on the timed
// path).
//
// Group RTN ("Métodos de cuantización de LLM...", RTN paragraph; "TurboQuant:
// cuantizar modelos grandes...", "Compresión por bloques"): one thread owns
// one group of G consecutive inputs of one row.  The constants are rounded
// outward to fp16 (offset down, scale up) so every weight lies inside the
// grid; the code decision q = rint((w - o)/s) is taken in IEEE fp64 with ties
// to even.  No fast-math and no contraction here: the codes must come out
// bit-identical to any other IEEE implementation of the same steps.
#pragma clang fp contract(off)

#include "common.hpp"
#include "launch.hpp"

#include <mutex>

namespace qg {

// ------------------------------------------------------------ status word
__device__ __align__(16) int qg_pack_status[4];

int* pack_status_ptr(hipError_t* err) {
  static std::mutex mu;
  static int* ptrs[64] = {nullptr};
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= 64) { *err = hipErrorInvalidDevice; return nullptr; }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(qg_pack_status));
    if (*err != hipSuccess) return nullptr;
    ptrs[dev] = static_cast<int*>(p);
  }
  *err = hipSuccess;
  return ptrs[dev];
}

__global__ void zero_status_kernel(int* status) { if (threadIdx.x == 0) status[0] = 0; }

hipError_t launch_zero_status(int* status, hipStream_t s) {
  hipLaunchKernelGGL(zero_status_kernel, dim3(1), dim3(64), 0, s, status);
  return hipGetLastError();
}

// ------------------------------------------------- fp16 directed rounding
// Magnitude a >= 0 truncated toward zero onto the fp16 grid; returns the
// fp16 bit pattern (0x7BFF for a >= 65536) and whether it was inexact.
__device__ uint32_t f16_trunc_bits(double a, bool* inexact) {
  if (a == 0.0) { *inexact = false; return 0u; }
  int e = 0;
  (void)frexp(a, &e);          // a = m * 2^e, m in [0.5, 1)
  const int E = e - 1;         // a in [2^E, 2^(E+1))
  if (E > 15) { *inexact = true; return 0x7BFFu; }
  const int qexp = (E >= -14) ? (E - 10) : -24;      // weight of the last fp16 bit
  const double k = floor(ldexp(a, -qexp));            // exact: power-of-two scaling
  *inexact = (ldexp(k, qexp) != a);
  const uint32_t ki = (uint32_t)k;
  return (E >= -14) ? ((uint32_t)(E + 15) << 10) + (ki - 1024u) : ki;
}

// Largest fp16 <= v (bits); canonical +0.  Overflow to -inf is flagged.
__device__ uint32_t f16_round_down_bits(double v, bool* bad) {
  bool inexact;
  if (v >= 0.0) return f16_trunc_bits(v, &inexact);
  uint32_t m = f16_trunc_bits(-v, &inexact);
  if (inexact) m += 1u;
  if (m >= 0x7C00u) *bad = true;
  return m == 0u ? 0u : (m | 0x8000u);
}

// Smallest fp16 >= v (bits); canonical +0.  Overflow to +inf is flagged.
__device__ uint32_t f16_round_up_bits(double v, bool* bad) {
  bool inexact;
  if (v <= 0.0) {
    uint32_t m = f16_trunc_bits(-v, &inexact);
    return m == 0u ? 0u : (m | 0x8000u);
  }
  uint32_t m = f16_trunc_bits(v, &inexact);
  if (inexact) m += 1u;
  if (m >= 0x7C00u) *bad = true;
  return m;
}

__device__ double f16_bits_to_f64(uint32_t h) {
  return (double)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Place code q (b bits) of unit code index c into the unit's words.
template <int B>
__device__ __forceinline__ void place_code(uint32_t (&w)[B], int c, uint32_t q) {
  constexpr int F = 16 / B;
  constexpr int nreg = 2 * F * B;
  if (c < nreg) {
    const int wi = c / (2 * F), h = (c % (2 * F)) / F, j = c % F;
    w[wi] |= q << (16 * h + B * j);
  } else if constexpr (B == 3 || B == 5) {
    const int h = c - 30;
#pragma unroll
    for (int i = 0; i < B; ++i) w[i] |= ((q >> i) & 1u) << (16 * h + 15);
  } else if constexpr (B == 6) {
    const int h = (c - 24) / 4, p = (c - 24) % 4;
    w[p] |= (q & 0xFu) << (16 * h + 12);
    w[4 + p / 2] |= ((q >> 4) & 3u) << (16 * h + 12 + 2 * (p % 2));
  }
}

template <int B, int G>
__global__ __launch_bounds__(256) void pack_group_kernel(const float* __restrict__ W, int64_t N,
                                                        int64_t K, uint32_t* __restrict__ codes,
                                                        uint32_t* __restrict__ meta, int* status) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t Gn = K / G;
  if (gid >= N * Gn) return;
  const int64_t n = gid / Gn, j = gid % Gn;
  const float* src = W + n * K + j * G;
  constexpr uint32_t L = (1u << B) - 1u;

  float v[G];
#pragma unroll
  for (int i = 0; i < G / 4; ++i) {
    const float4 t = reinterpret_cast<const float4*>(src)[i];
    v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
  }
  bool bad = false;
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const uint32_t bits = __float_as_uint(v[i]);
    if ((bits & 0x7F800000u) == 0x7F800000u) bad = true;
    mn = v[i] < mn ? v[i] : mn;
    mx = v[i] > mx ? v[i] : mx;
  }
  uint32_t obits = 0, sbits = 0;
  if (!bad) {
    obits = f16_round_down_bits((double)mn, &bad);
    const double o = f16_bits_to_f64(obits);
    const double vs = ((double)mx - o) / (double)L;
    sbits = f16_round_up_bits(vs, &bad);
  }
  if (bad) { atomicOr(status, 1); obits = 0; sbits = 0; }
  meta[gid] = sbits | (obits << 16);
  const double o = f16_bits_to_f64(obits);
  const double s = f16_bits_to_f64(sbits);

#pragma unroll
  for (int uu = 0; uu < G / 32; ++uu) {
    uint32_t w[B];
#pragma unroll
    for (int i = 0; i < B; ++i) w[i] = 0u;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      uint32_t q = 0u;
      if (s != 0.0) {
        const double d = (double)v[uu * 32 + c] - o;
        double t = rint(d / s);
        t = t < 0.0 ? 0.0 : (t > (double)L ? (double)L : t);
        q = (uint32_t)t;
      }
      place_code<B>(w, c, q);
    }
    uint32_t* dst = codes + ((n * (K / 32)) + j * (G / 32) + uu) * B;
#pragma unroll
    for (int i = 0; i < B; ++i) dst[i] = w[i];
  }
}

template <int B, int G>
__global__ __launch_bounds__(256) void unpack_group_kernel(const uint32_t* __restrict__ codes,
                                                          const uint32_t* __restrict__ meta,
                                                          int64_t N, int64_t K,
                                                          uint8_t* __restrict__ qout,
                                                          float* __restrict__ wout) {
  const int64_t uid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t U = K / 32;
  if (uid >= N * U) return;
  const int64_t n = uid / U, u = uid % U;
  uint32_t w[B];
#pragma unroll
  for (int i = 0; i < B; ++i) w[i] = codes[uid * B + i];
  float q[32];
  unit_codes_f32<B>(w, q);
  uint32_t packed[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    packed[i] = (uint32_t)q[4 * i] | ((uint32_t)q[4 * i + 1] << 8) |
                ((uint32_t)q[4 * i + 2] << 16) | ((uint32_t)q[4 * i + 3] << 24);
  }
  uint32_t* qdst = reinterpret_cast<uint32_t*>(qout + n * K + u * 32);
#pragma unroll
  for (int i = 0; i < 8; ++i) qdst[i] = packed[i];
  if (wout) {
    const uint32_t m = meta[n * (K / G) + (u * 32) / G];
    const float s = f16_bits_to_f32(m & 0xFFFFu), o = f16_bits_to_f32(m >> 16);
    float* wdst = wout + n * K + u * 32;
#pragma unroll
    for (int i = 0; i < 32; ++i) wdst[i] = __builtin_fmaf(s, q[i], o);
  }
}

template <int B, int G>
static hipError_t pack_group_t(const float* W, int64_t N, int64_t K, uint32_t* codes,
                               uint32_t* meta, int* status, hipStream_t s) {
  const int64_t groups = N * (K / G);
  const int64_t blocks = (groups + 255) / 256;
  hipLaunchKernelGGL((pack_group_kernel<B, G>), dim3((unsigned)blocks), dim3(256), 0, s, W, N,
                     K, codes, meta, status);
  return hipGetLastError();
}

template <int B, int G>
static hipError_t unpack_group_t(const uint32_t* codes, const uint32_t* meta, int64_t N,
                                 int64_t K, uint8_t* q, float* w, hipStream_t s) {
  const int64_t units = N * (K / 32);
  const int64_t blocks = (units + 255) / 256;
  hipLaunchKernelGGL((unpack_group_kernel<B, G>), dim3((unsigned)blocks), dim3(256), 0, s,
                     codes, meta, N, K, q, w);
  return hipGetLastError();
}

#define QG_DISPATCH_BG(bits, group, CALL)                                  \
  switch ((bits) * 100 + (group)) {                                        \
    case 232: return CALL(2, 32); case 264: return CALL(2, 64);            \
    case 332: return CALL(3, 32); case 364: return CALL(3, 64);            \
    case 432: return CALL(4, 32); case 464: return CALL(4, 64);            \
    case 532: return CALL(5, 32); case 564: return CALL(5, 64);            \
    case 632: return CALL(6, 32); case 664: return CALL(6, 64);            \
    default: return hipErrorInvalidValue;                                  \
  }

hipError_t launch_pack_group(const float* W, int64_t N, int64_t K, int bits, int group,
                             uint32_t* codes, uint32_t* meta, int* status, hipStream_t s) {
#define CALL(b, g) pack_group_t<b, g>(W, N, K, codes, meta, status, s)
  QG_DISPATCH_BG(bits, group, CALL)
#undef CALL
}

hipError_t launch_unpack_group(const uint32_t* codes, const uint32_t* meta, int64_t N,
                               int64_t K, int bits, int group, uint8_t* q, float* w,
                               hipStream_t s) {
#define CALL(b, g) unpack_group_t<b, g>(codes, meta, N, K, q, w, s)
  QG_DISPATCH_BG(bits, group, CALL)
#undef CALL
}

// ------------------------------------------------------------- binary LR
// +1 -> bit 1, -1 -> bit 0, LSB first; rows padded to 4-word multiples with
// zero bits ("70B en 4GB de VRAM...", section 1, binary factors U, V).
__host__ __device__ __forceinline__ int64_t padded_words(int64_t n) { return ((n + 31) / 32 + 3) / 4 * 4; }

// Ubits[n][w]: bits of U[n][32w .. 32w+31].  One thread per output word.
__global__ __launch_bounds__(256) void pack_rows_kernel(const int8_t* __restrict__ M, int64_t R,
                                                       int64_t C, uint32_t* __restrict__ out,
                                                       int* status) {
  const int64_t Wn = padded_words(C);
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= R * Wn) return;
  const int64_t row = gid / Wn, wi = gid % Wn;
  uint32_t bits = 0u;
  bool bad = false;
  for (int i = 0; i < 32; ++i) {
    const int64_t c = wi * 32 + i;
    if (c < C) {
      const int8_t v = M[row * C + c];
      if (v == 1) bits |= 1u << i;
      else if (v != -1) bad = true;
    }
  }
  if (bad) atomicOr(status, 1);
  out[gid] = bits;
}

// VTbits[l][w]: bits of V[32w .. 32w+31][l].  Consecutive threads take
// consecutive l so the column reads of V coalesce.
__global__ __launch_bounds__(256) void pack_cols_kernel(const int8_t* __restrict__ V, int64_t K,
                                                       int64_t r, uint32_t* __restrict__ out,
                                                       int* status) {
  const int64_t Kw = padded_words(K);
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= r * Kw) return;
  const int64_t wi = gid / r, l = gid % r;
  uint32_t bits = 0u;
  bool bad = false;
  for (int i = 0; i < 32; ++i) {
    const int64_t k = wi * 32 + i;
    if (k < K) {
      const int8_t v = V[k * r + l];
      if (v == 1) bits |= 1u << i;
      else if (v != -1) bad = true;
    }
  }
  if (bad) atomicOr(status, 1);
  out[l * Kw + wi] = bits;
}

__global__ __launch_bounds__(256) void unpack_rows_kernel(const uint32_t* __restrict__ in,
                                                         int64_t R, int64_t C,
                                                         int8_t* __restrict__ M) {
  const int64_t Wn = padded_words(C);
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= R * C) return;
  const int64_t row = gid / C, c = gid % C;
  M[gid] = ((in[row * Wn + c / 32] >> (c % 32)) & 1u) ? (int8_t)1 : (int8_t)-1;
}

__global__ __launch_bounds__(256) void unpack_cols_kernel(const uint32_t* __restrict__ in,
                                                         int64_t K, int64_t r,
                                                         int8_t* __restrict__ V) {
  const int64_t Kw = padded_words(K);
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= K * r) return;
  const int64_t k = gid / r, l = gid % r;
  V[gid] = ((in[l * Kw + k / 32] >> (k % 32)) & 1u) ? (int8_t)1 : (int8_t)-1;
}

static unsigned nblocks(int64_t n) { return (unsigned)((n + 255) / 256); }

hipError_t launch_pack_binlr(const int8_t* U, const int8_t* V, int64_t N, int64_t K,
                             int64_t r, uint32_t* ubits, uint32_t* vtbits, int* status,
                             hipStream_t s) {
  hipLaunchKernelGGL(pack_rows_kernel, dim3(nblocks(N * padded_words(r))), dim3(256), 0, s,
                     U, N, r, ubits, status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pack_cols_kernel, dim3(nblocks(r * padded_words(K))), dim3(256), 0, s,
                     V, K, r, vtbits, status);
  return hipGetLastError();
}

hipError_t launch_unpack_binlr(const uint32_t* ubits, const uint32_t* vtbits, int64_t N,
                               int64_t K, int64_t r, int8_t* U, int8_t* V, hipStream_t s) {
  if (U) {
    hipLaunchKernelGGL(unpack_rows_kernel, dim3(nblocks(N * r)), dim3(256), 0, s, ubits, N, r, U);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (V) {
    hipLaunchKernelGGL(unpack_cols_kernel, dim3(nblocks(K * r)), dim3(256), 0, s, vtbits, K, r, V);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace qg
