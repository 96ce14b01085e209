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

// Group constants of the RTN grid with L = 2^b - 1 steps: o = largest fp16
// <= min, s = smallest fp16 >= (max - o)/L in fp64 (fp16 bits).  A
// non-finite weight or a constant outside the fp16 range sets *bad and
// returns zero constants.
template <int G>
__device__ __forceinline__ void group_constants(const float (&v)[G], uint32_t L, uint32_t* obits,
                                                uint32_t* sbits, bool* bad) {
  bool b = false;
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const uint32_t bits = __float_as_uint(v[i]);
    if ((bits & 0x7F800000u) == 0x7F800000u) b = true;
    mn = v[i] < mn ? v[i] : mn;
    mx = v[i] > mx ? v[i] : mx;
  }
  uint32_t ob = 0, sb = 0;
  if (!b) {
    ob = f16_round_down_bits((double)mn, &b);
    const double o = f16_bits_to_f64(ob);
    sb = f16_round_up_bits(((double)mx - o) / (double)L, &b);
  }
  if (b) { ob = 0; sb = 0; }
  *obits = ob; *sbits = sb; *bad = b;
}

// zmask (optional): bit k set -> input channel k is encoded as 0 (the
// outlier channels of the mixed decomposition).
template <int B, int G>
__global__ __launch_bounds__(256) void pack_group_kernel(const float* __restrict__ W, int64_t N,
                                                        int64_t K, uint32_t* __restrict__ codes,
                                                        uint32_t* __restrict__ meta, int* status,
                                                        const uint32_t* __restrict__ zmask) {
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
  if (zmask) {
#pragma unroll
    for (int uu = 0; uu < G / 32; ++uu) {
      const uint32_t zw = zmask[(j * G) / 32 + uu];
#pragma unroll
      for (int c = 0; c < 32; ++c)
        if ((zw >> c) & 1u) v[uu * 32 + c] = 0.f;
    }
  }
  bool bad = false;
  uint32_t obits = 0, sbits = 0;
  group_constants<G>(v, L, &obits, &sbits, &bad);
  if (bad) atomicOr(status, 1);
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
                               uint32_t* meta, int* status, const uint32_t* zmask, hipStream_t s) {
  const int64_t groups = N * (K / G);
  const int64_t blocks = (groups + 255) / 256;
  hipLaunchKernelGGL((pack_group_kernel<B, G>), dim3((unsigned)blocks), dim3(256), 0, s, W, N,
                     K, codes, meta, status, zmask);
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
#define CALL(b, g) pack_group_t<b, g>(W, N, K, codes, meta, status, nullptr, s)
  QG_DISPATCH_BG(bits, group, CALL)
#undef CALL
}

// -------------------------------------------------- per-group codebooks
// Codes read through per-group books ("TurboQuant: cuantizar modelos
// grandes...", introduction and "Compresión por bloques": block compression
// with a shared dictionary, a compressed codebook per group).  One thread per
// group: the RTN constants s, o; u = (w - o)/s in fp64; for every book of
// the dictionary (levels c = e/2^(7-b), staged in LDS as fp64) each weight's
// nearest level (ties to the even index, then the lower) and the book's
// squared error summed in increasing k; the least-error book (ties to the
// lower index) and its codes.  s == 0: book 0, codes 0.
template <int B, int G>
__global__ __launch_bounds__(256) void pack_group_cb_kernel(const float* __restrict__ W, int64_t N, int64_t K,
                                                           const uint8_t* __restrict__ books, int nb,
                                                           uint32_t* __restrict__ codes, uint32_t* __restrict__ meta,
                                                           uint8_t* __restrict__ book_ids, int* status) {
  constexpr int NL = 1 << B;
  __shared__ double lv[16 * NL];
  for (int t = threadIdx.x; t < nb * NL; t += blockDim.x) {
    if (books[t] > 127) atomicOr(status, 2);   // level above the 7-bit grid
    lv[t] = ldexp((double)books[t], B - 7);
  }
  __syncthreads();
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t Gn = K / G;
  if (gid >= N * Gn) return;
  const int64_t n = gid / Gn, j = gid % Gn;
  const float* src = W + n * K + j * G;
  float v[G];
#pragma unroll
  for (int i = 0; i < G / 4; ++i) {
    const float4 t = reinterpret_cast<const float4*>(src)[i];
    v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
  }
  bool bad = false;
  uint32_t obits = 0, sbits = 0;
  group_constants<G>(v, (uint32_t)(NL - 1), &obits, &sbits, &bad);
  if (bad) atomicOr(status, 1);
  meta[gid] = sbits | (obits << 16);
  const double o = f16_bits_to_f64(obits);
  const double s = f16_bits_to_f64(sbits);
  double u[G];
#pragma unroll
  for (int i = 0; i < G; ++i) u[i] = s != 0.0 ? ((double)v[i] - o) / s : 0.0;
  // nearest level of book d for u; distance in *dist
  auto nearest = [&](int d, double x, double* dist) {
    int bj = 0;
    double bd = fabs(x - lv[d * NL]);
    for (int jj = 1; jj < NL; ++jj) {
      const double a = fabs(x - lv[d * NL + jj]);
      if (a < bd || (a == bd && (bj & 1) && !(jj & 1))) { bd = a; bj = jj; }
    }
    *dist = bd;
    return bj;
  };
  int best = 0;
  if (s != 0.0) {
    double best_err = 0.0;
    for (int d = 0; d < nb; ++d) {
      double err = 0.0;
#pragma unroll
      for (int i = 0; i < G; ++i) {
        double a;
        (void)nearest(d, u[i], &a);
        err = err + a * a;
      }
      if (d == 0 || err < best_err) { best_err = err; best = d; }
    }
  }
  book_ids[gid] = (uint8_t)best;
#pragma unroll
  for (int uu = 0; uu < G / 32; ++uu) {
    uint32_t w[B];
#pragma unroll
    for (int i = 0; i < B; ++i) w[i] = 0u;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      double a;
      const uint32_t q = s != 0.0 ? (uint32_t)nearest(best, u[uu * 32 + c], &a) : 0u;
      place_code<B>(w, c, q);
    }
    uint32_t* dst = codes + ((n * (K / 32)) + j * (G / 32) + uu) * B;
#pragma unroll
    for (int i = 0; i < B; ++i) dst[i] = w[i];
  }
}

template <int B, int G>
static hipError_t pack_group_cb_t(const float* W, int64_t N, int64_t K, const uint8_t* books, int nb,
                                  uint32_t* codes, uint32_t* meta, uint8_t* book_ids, int* status, hipStream_t s) {
  const int64_t blocks = (N * (K / G) + 255) / 256;
  hipLaunchKernelGGL((pack_group_cb_kernel<B, G>), dim3((unsigned)blocks), dim3(256), 0, s, W, N, K, books, nb,
                     codes, meta, book_ids, status);
  return hipGetLastError();
}

hipError_t launch_pack_group_cb(const float* W, int64_t N, int64_t K, int bits, int group, const uint8_t* books,
                                int n_books, uint32_t* codes, uint32_t* meta, uint8_t* book_ids, int* status,
                                hipStream_t s) {
#define CALL(b, g) pack_group_cb_t<b, g>(W, N, K, books, n_books, codes, meta, book_ids, status, s)
  switch (bits * 100 + group) {
    case 232: return CALL(2, 32); case 264: return CALL(2, 64);
    case 332: return CALL(3, 32); case 364: return CALL(3, 64);
    case 432: return CALL(4, 32); case 464: return CALL(4, 64);
    default: return hipErrorInvalidValue;
  }
#undef CALL
}

// ------------------------------------------------------ outlier channels
// Mixed decomposition ("Métodos de cuantización de LLM...", opening and
// LLM.int8() paragraph): the n_out input channels with the largest
// max_n |W[n][k]| (ties to the lower k) are encoded as 0 by the group RTN and
// kept as fp16 columns side[n][j] = fp16(W[n][idx_j] - w_rest[n][idx_j]).

// fp64 -> fp16 bits, rounded to nearest even, one rounding; +-0 keep their
// sign.  Non-finite input or a result beyond the fp16 range is flagged.
__device__ uint32_t f16_rne_bits(double v, bool* bad) {
  const uint32_t sign = signbit(v) ? 0x8000u : 0u;
  const double a = fabs(v);
  if (!(a <= 1.7976931348623157e308)) { *bad = true; return sign | 0x7C00u; }   // NaN, inf
  if (a == 0.0) return sign;
  int e = 0;
  (void)frexp(a, &e);
  const int E = e - 1;                                  // a in [2^E, 2^(E+1))
  if (E > 15) { *bad = true; return sign | 0x7C00u; }
  const int qexp = (E >= -14) ? (E - 10) : -24;         // weight of the last fp16 bit
  const double t = ldexp(a, -qexp);                     // exact
  double k = floor(t);
  const double frac = t - k;                            // exact
  if (frac > 0.5 || (frac == 0.5 && fmod(k, 2.0) == 1.0)) k += 1.0;
  const uint32_t ki = (uint32_t)k;
  const uint32_t m = (E >= -14) ? ((uint32_t)(E + 15) << 10) + (ki - 1024u) : ki;   // carries into the exponent
  if (m >= 0x7C00u) { *bad = true; return sign | 0x7C00u; }
  return sign | m;
}

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// score[k] = max over rows of |W[n][k]| as fp32 bits (monotonic for |w|; a
// NaN sorts above +inf).  Block (x, y): 256 columns x `rows` rows.
__global__ __launch_bounds__(256) void colmax_kernel(const float* __restrict__ W, int64_t N, int64_t K,
                                                     int rows, uint32_t* __restrict__ score) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  const int64_t n0 = (int64_t)blockIdx.y * rows;
  const int64_t n1 = n0 + rows < N ? n0 + rows : N;
  uint32_t m = 0u;
  for (int64_t n = n0; n < n1; ++n) {
    const uint32_t b = __float_as_uint(W[n * K + k]) & 0x7FFFFFFFu;
    m = b > m ? b : m;
  }
  atomicMax(&score[k], m);
}

// One workgroup: n_out rounds of a block-wide argmax over (score, -k); a
// taken channel is marked 0xFFFFFFFF.  idx[] is written in increasing k and
// zmask (K bits) marks the chosen channels.  A non-finite chosen score flags
// the status word.
__global__ __launch_bounds__(1024) void select_outliers_kernel(uint32_t* __restrict__ score, int64_t K,
                                                               int n_out, int32_t* __restrict__ idx,
                                                               uint32_t* __restrict__ zmask,
                                                               int* status) {
  __shared__ unsigned long long best[1024];
  __shared__ int32_t sel[64];
  const int tid = threadIdx.x;
  for (int r = 0; r < n_out; ++r) {
    unsigned long long b = 0ull;
    for (int64_t k = tid; k < K; k += 1024) {
      const uint32_t sc = score[k];
      if (sc != 0xFFFFFFFFu) {
        const unsigned long long key = ((unsigned long long)sc << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)k);
        b = key > b ? key : b;
      }
    }
    best[tid] = b;
    __syncthreads();
    for (int w = 512; w > 0; w >>= 1) {
      if (tid < w && best[tid + w] > best[tid]) best[tid] = best[tid + w];
      __syncthreads();
    }
    if (tid == 0) {
      const unsigned long long key = best[0];
      const uint32_t k = 0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull);
      if ((uint32_t)(key >> 32) >= 0x7F800000u) atomicOr(status, 1);
      sel[r] = (int32_t)k;
      score[k] = 0xFFFFFFFFu;
    }
    __syncthreads();
  }
  for (int64_t i = tid; i < (K + 31) / 32; i += 1024) zmask[i] = 0u;
  if (tid == 0) {
    for (int a = 1; a < n_out; ++a) {          // insertion sort, n_out <= 64
      const int32_t v = sel[a];
      int b2 = a - 1;
      while (b2 >= 0 && sel[b2] > v) { sel[b2 + 1] = sel[b2]; --b2; }
      sel[b2 + 1] = v;
    }
  }
  __syncthreads();
  if (tid < n_out) {
    idx[tid] = sel[tid];
    atomicOr(&zmask[sel[tid] >> 5], 1u << (sel[tid] & 31));
  }
}

// Code c of a unit (b words at w) in format v1.
template <int B>
__device__ __forceinline__ uint32_t unit_code_at(const uint32_t* w, int c) {
  constexpr int F = 16 / B;
  constexpr uint32_t L = (1u << B) - 1u;
  if (c < 2 * F * B) {
    const int wi = c / (2 * F), h = (c % (2 * F)) / F, j = c % F;
    return (w[wi] >> (16 * h + B * j)) & L;
  }
  if constexpr (B == 3 || B == 5) {
    const int h = c - 30;
    uint32_t q = 0u;
#pragma unroll
    for (int i = 0; i < B; ++i) q |= ((w[i] >> (16 * h + 15)) & 1u) << i;
    return q;
  } else if constexpr (B == 6) {
    const int h = (c - 24) / 4, p = (c - 24) % 4;
    return ((w[p] >> (16 * h + 12)) & 0xFu) | (((w[4 + p / 2] >> (16 * h + 12 + 2 * (p % 2))) & 3u) << 4);
  }
  return 0u;
}

// side[n][j] = fp16(W[n][k] - (s*q + o)) at k = idx[j], fp64 arithmetic.
template <int B, int G>
__global__ __launch_bounds__(256) void outlier_side_kernel(const float* __restrict__ W, int64_t N, int64_t K,
                                                           const uint32_t* __restrict__ codes,
                                                           const uint32_t* __restrict__ meta,
                                                           const int32_t* __restrict__ idx, int n_out,
                                                           uint16_t* __restrict__ side, int* status) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= N * n_out) return;
  const int64_t n = t / n_out;
  const int k = idx[t % n_out];
  const uint32_t q = unit_code_at<B>(codes + (n * (K / 32) + k / 32) * B, k % 32);
  const uint32_t m = meta[n * (K / G) + k / G];
  const double wr = f16_bits_to_f64(m & 0xFFFFu) * (double)q + f16_bits_to_f64(m >> 16);   // exact
  bool bad = false;
  const uint32_t h = f16_rne_bits((double)W[n * K + k] - wr, &bad);
  if (bad) atomicOr(status, 1);
  side[t] = (uint16_t)h;
}

template <int B, int G>
static hipError_t pack_outlier_t(const float* W, int64_t N, int64_t K, int n_out, uint32_t* codes,
                                 uint32_t* meta, uint16_t* side, int32_t* idx, uint32_t* score,
                                 uint32_t* zmask, int* status, hipStream_t s) {
  const unsigned kb = (unsigned)((K + 255) / 256);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(kb), dim3(256), 0, s, score, K, 0u);
  const int rows = 256;
  hipLaunchKernelGGL(colmax_kernel, dim3(kb, (unsigned)((N + rows - 1) / rows)), dim3(256), 0, s, W, N, K,
                     rows, score);
  hipLaunchKernelGGL(select_outliers_kernel, dim3(1), dim3(1024), 0, s, score, K, n_out, idx, zmask, status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = pack_group_t<B, G>(W, N, K, codes, meta, status, zmask, s);
  if (e != hipSuccess) return e;
  const int64_t t = N * n_out;
  if (t > 0)
    hipLaunchKernelGGL((outlier_side_kernel<B, G>), dim3((unsigned)((t + 255) / 256)), dim3(256), 0, s, W, N, K,
                       codes, meta, idx, n_out, side, status);
  return hipGetLastError();
}

hipError_t launch_pack_group_outlier(const float* W, int64_t N, int64_t K, int bits, int group, int n_out,
                                     uint32_t* codes, uint32_t* meta, uint16_t* side, int32_t* idx,
                                     void* ws, int* status, hipStream_t s) {
  uint32_t* score = static_cast<uint32_t*>(ws);
  uint32_t* zmask = score + ((K + 3) / 4) * 4;
#define CALL(b, g) pack_outlier_t<b, g>(W, N, K, n_out, codes, meta, side, idx, score, zmask, status, s)
  QG_DISPATCH_BG(bits, group, CALL)
#undef CALL
}

size_t pack_group_outlier_ws_bytes(int64_t K) {
  return (size_t)(((K + 3) / 4) * 4 + ((K + 31) / 32 + 3) / 4 * 4) * 4;
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

// ------------------------------------------------------- key-cache encoder
// Inner-product key quantizer ("70B en 4GB de VRAM...", section 3,
// TurboQuant): y = Pi x / |x| (random rotation), each coordinate to the
// nearest stored Lloyd-Max centroid (M bits, ties to the lower index), the
// residual r = y - c of the rotated unit vector, gamma = |r|, and the signs of
// S r (bit 1 <-> >= 0).  One 64-lane workgroup per 128-dimensional key; every
// sum runs in fp64 in increasing index order (contraction is off in this
// file), so the codes and signs are those of any IEEE implementation of the
// same steps.  Centroid k is delta * (e_k - 64), e_k the k-th byte of
// (tab_lo, tab_hi).  Outputs: codes [n][4][M] (units of 32 coordinates in
// the group-code layout), signs [n][4] (bit j of word w: coordinate 32w + j),
// norms [n] = fp16 |x| | fp16 gamma << 16.
// PROD = false: the reconstruction variant for values (M = 2..4 bits): codes
// and fp16 |x| only (no residual, no signs; norms' upper half 0).
template <int M, bool PROD>
__global__ __launch_bounds__(64) void tq_quant_kernel(const float* __restrict__ X, const double* __restrict__ Pi,
                                                      const double* __restrict__ S, double delta, uint4 tab,
                                                      uint32_t* __restrict__ codes, uint32_t* __restrict__ signs,
                                                      uint32_t* __restrict__ norms, int* status) {
  constexpr int D = 128, L = 1 << M;
  __shared__ double xs[D], rs[D], sh[2];
  __shared__ uint32_t cs[D], zs[D];
  const int64_t key = blockIdx.x;
  const int l = threadIdx.x;
  double cv[L];
#pragma unroll
  for (int k = 0; k < L; ++k) {
    const uint32_t tw = k < 4 ? tab.x : (k < 8 ? tab.y : (k < 12 ? tab.z : tab.w));
    const uint32_t e = (tw >> (8 * (k & 3))) & 0xFFu;
    cv[k] = delta * ((double)e - 64.0);
  }
  const float x0 = X[key * D + l], x1 = X[key * D + l + 64];
  if (!isfinite(x0) || !isfinite(x1)) atomicOr(status, 1);
  xs[l] = (double)x0;
  xs[l + 64] = (double)x1;
  __syncthreads();
  if (l == 0) {
    double a = 0.0;
    for (int j = 0; j < D; ++j) a = a + xs[j] * xs[j];
    sh[0] = sqrt(a);
  }
  __syncthreads();
  const double nrm = sh[0], safe = nrm > 0.0 ? nrm : 1.0;
  for (int h = 0; h < 2; ++h) {
    const int i = l + 64 * h;
    double a = 0.0;
    for (int j = 0; j < D; ++j) a = a + xs[j] * Pi[i * D + j];
    const double y = a / safe;
    int best = 0;
    double bd = fabs(y - cv[0]);
#pragma unroll
    for (int k = 1; k < L; ++k) {
      const double dd = fabs(y - cv[k]);
      if (dd < bd) { bd = dd; best = k; }
    }
    cs[i] = (uint32_t)best;
    rs[i] = y - cv[best];
  }
  __syncthreads();
  if constexpr (PROD) {
    if (l == 0) {
      double a = 0.0;
      for (int j = 0; j < D; ++j) a = a + rs[j] * rs[j];
      sh[1] = sqrt(a);
    }
    for (int h = 0; h < 2; ++h) {
      const int i = l + 64 * h;
      double a = 0.0;
      for (int j = 0; j < D; ++j) a = a + rs[j] * S[i * D + j];
      zs[i] = a >= 0.0 ? 1u : 0u;
    }
    __syncthreads();
  }
  if (l < 4) {
    uint32_t w[M];
#pragma unroll
    for (int i = 0; i < M; ++i) w[i] = 0u;
    uint32_t sg = 0u;
    for (int c = 0; c < 32; ++c) {
      place_code<M>(w, c, cs[32 * l + c]);
      if constexpr (PROD) sg |= zs[32 * l + c] << c;
    }
#pragma unroll
    for (int i = 0; i < M; ++i) codes[(key * 4 + l) * M + i] = w[i];
    if constexpr (PROD) signs[key * 4 + l] = sg;
  }
  if (l == 0) {
    bool bad = false;
    norms[key] = f16_rne_bits(sh[0], &bad) | (PROD ? f16_rne_bits(sh[1], &bad) << 16 : 0u);
    if (bad) atomicOr(status, 1);
  }
}

hipError_t launch_tq_quant(const float* X, int64_t n, int mbits, bool prod, const double* Pi, const double* S,
                           float delta, const uint32_t* tab, uint32_t* codes, uint32_t* signs, uint32_t* norms,
                           int* status, hipStream_t s) {
  const uint4 t4{tab[0], tab[1], tab[2], tab[3]};
#define L(MB, P)                                                                                                \
  hipLaunchKernelGGL((tq_quant_kernel<MB, P>), dim3((unsigned)n), dim3(64), 0, s, X, Pi, S, (double)delta, t4, \
                     codes, signs, norms, status)
  if (prod && mbits == 2) L(2, true);
  else if (prod && mbits == 3) L(3, true);
  else if (!prod && mbits == 2) L(2, false);
  else if (!prod && mbits == 3) L(3, false);
  else if (!prod && mbits == 4) L(4, false);
  else return hipErrorInvalidValue;
#undef L
  return hipGetLastError();
}

}  // namespace qg
