// Key-cache quantization with a random rotation, one Lloyd-Max codebook for
// the known coordinate law and a 1-bit QJL residual ("70B en 4GB de VRAM: la
// compresión neural de 2026, ¿es real?", section 3, TurboQuant): host set-up
// (centroids, rotation) and the attention-logit kernels.  The encoder lives
// with the other packers (pack.hip).
//
// Logits: for a query q, every stored key x of the same head gives the
// unbiased estimate
//   <q, x> ~ |x| (delta sum_j (e[code_j] - 64) (Pi q)_j
//                 + gamma sqrt(pi/2)/d sum_j sign_j (S Pi q)_j).
// A prep kernel forms Pi q and S Pi q = (S Pi) q once per query (fp32,
// rounded to bf16 and laid out as the operand pairs of the logit kernel); S Pi
// is formed once per (Pi, S) pair (qtq_project).  The logit
// kernel streams the keys: the centroid codes go through the codebook
// byte-permute decode (pairs 128 + e[code] in bf16) and the sign bits become
// bf16 +-1 pairs with one shift and one masked OR; the products with up to
// 16 queries (a grouped-query head's) run on the matrix cores, so a key is
// read once for all of them.
#include <math.h>

#include "codebook.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace qg {

// ------------------------------------------------------------ host set-up
// Lloyd-Max centroids of the coordinate law of a uniform unit vector in R^d,
// f(t) = C (1 - t^2)^((d-3)/2) on [-1, 1]: boundaries at midpoints,
// centroids at the conditional means; a cell's mass by composite Simpson
// quadrature, its first moment from the antiderivative
// -C (1 - t^2)^((d-1)/2) / (d - 1).
static double tq_logC(int d) { return lgamma(d / 2.0) - lgamma((d - 1) / 2.0) - 0.5 * log(3.14159265358979323846); }

static double tq_mass(int d, double a, double b) {
  const int n = 4096;   // even
  const double h = (b - a) / n, p = (d - 3) / 2.0, lc = tq_logC(d);
  auto f = [&](double t) {
    const double u = 1.0 - t * t;
    return u > 0.0 ? exp(lc + p * log(u)) : 0.0;
  };
  double s = f(a) + f(b);
  for (int i = 1; i < n; ++i) s += (i & 1 ? 4.0 : 2.0) * f(a + i * h);
  return s * h / 3.0;
}

static double tq_moment(int d, double a, double b) {
  auto F = [&](double t) {
    const double u = 1.0 - t * t;
    return u > 0.0 ? -exp(tq_logC(d) + (d - 1) / 2.0 * log(u)) / (d - 1) : 0.0;
  };
  return F(b) - F(a);
}

void tq_lloyd_max(int d, int m, double* c) {
  const int L = 1 << m;
  // start: evenly spaced in [-2/sqrt(d), 2/sqrt(d)]
  for (int k = 0; k < L; ++k) c[k] = (-1.0 + (2.0 * k + 1.0) / L) * 2.0 / sqrt((double)d);
  double e[17];
  for (int it = 0; it < 5000; ++it) {
    e[0] = -1.0;
    e[L] = 1.0;
    for (int k = 1; k < L; ++k) e[k] = 0.5 * (c[k - 1] + c[k]);
    double change = 0.0;
    for (int k = 0; k < L; ++k) {
      const double v = tq_moment(d, e[k], e[k + 1]) / tq_mass(d, e[k], e[k + 1]);
      change = fmax(change, fabs(v - c[k]));
      c[k] = v;
    }
    if (change < 1e-16) break;
  }
}

// Modified Gram-Schmidt on the columns of G (row-major d x d): the Q of
// G = QR with diag(R) > 0, written row-major to Pi.
void tq_rotation(int d, const double* G, double* Pi) {
  for (int i = 0; i < d * d; ++i) Pi[i] = G[i];
  for (int j = 0; j < d; ++j) {
    double nn = 0.0;
    for (int i = 0; i < d; ++i) nn += Pi[i * d + j] * Pi[i * d + j];
    const double inv = 1.0 / sqrt(nn);
    for (int i = 0; i < d; ++i) Pi[i * d + j] *= inv;
    for (int k = j + 1; k < d; ++k) {
      double dot = 0.0;
      for (int i = 0; i < d; ++i) dot += Pi[i * d + j] * Pi[i * d + k];
      for (int i = 0; i < d; ++i) Pi[i * d + k] -= dot * Pi[i * d + j];
    }
  }
}

// ------------------------------------------------------------ query prep
// SPi = S Pi, formed once per (Pi, S) pair: then Pi q and S Pi q = SPi q are
// independent products and one launch forms both.
__global__ __launch_bounds__(128) void tq_project_kernel(const double* __restrict__ S, const double* __restrict__ Pi,
                                                         double* __restrict__ SPi) {
  const int i = blockIdx.x, k = threadIdx.x;
  double a = 0.0;
  for (int j = 0; j < 128; ++j) a = __builtin_fma(S[i * 128 + j], Pi[j * 128 + k], a);
  SPi[i * 128 + k] = a;
}

// Per (query, head): qr = Pi q and u = SPi q, then for unit w and pair k:
// word w*32 + k = bf16 (qr[32w + ca], qr[32w + cb]) with (ca, cb) the code
// pair k of an M-bit unit; word w*32 + 16 + j = bf16 (u[32w + j],
// u[32w + j + 16]); float at 128 + w = the sum of the 32 bf16-rounded qr
// values of unit w (the 128-bias correction).  Grid (heads, 2 matrices, 4
// units): a workgroup stages the unit's 32 rows of its matrix in LDS as fp32
// (coalesced reads, 129-word pitch), multiplies them by every query of the
// head and writes that unit's words of its half (fp32 products, rounded once
// to bf16).
constexpr int kTqQueryWords = 132;
constexpr int kTqPitch = 129;

template <int M>
__global__ __launch_bounds__(256) void tq_prep_kernel(const float* __restrict__ Qv, int nq, const double* __restrict__ Pi,
                                                      const double* __restrict__ SPi, uint32_t* __restrict__ ws) {
  __shared__ float As[32][kTqPitch], v[16][128], res[16][32];
  const int h = blockIdx.x, mat = blockIdx.y, w = blockIdx.z, t = threadIdx.x;
  const double* A = mat ? SPi : Pi;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int e = t + 256 * k;                          // rows 32 w .. 32 w + 31
    As[e >> 7][e & 127] = (float)A[(size_t)(32 * w) * 128 + e];
  }
  for (int q0 = 0; q0 < nq; q0 += 16) {
    const int cnt = nq - q0 < 16 ? nq - q0 : 16;
    for (int i = t; i < cnt * 128; i += 256) v[i >> 7][i & 127] = Qv[((size_t)h * nq + q0) * 128 + i];
    __syncthreads();
    {
      const int r = t & 31;
      for (int j = t >> 5; j < cnt; j += 8) {
        float a0 = 0.f, a1 = 0.f;
#pragma unroll 8
        for (int c = 0; c < 128; c += 2) {
          a0 = __builtin_fmaf(As[r][c], v[j][c], a0);
          a1 = __builtin_fmaf(As[r][c + 1], v[j][c + 1], a1);
        }
        res[j][r] = a0 + a1;
      }
    }
    __syncthreads();
    for (int i = t; i < cnt * 17; i += 256) {
      const int j = i / 17, k = i % 17;
      uint32_t* out = ws + ((size_t)h * nq + q0 + j) * kTqQueryWords;
      if (mat == 0) {
        if (k < 16) {
          const PairInfo pi = Unit<M>::pair(k);
          out[w * 32 + k] = f32_to_bf16_rne(res[j][pi.ca]) | (f32_to_bf16_rne(res[j][pi.cb]) << 16);
        } else {
          float sum = 0.f;
          for (int c = 0; c < 32; ++c) sum += bf16_bits_to_f32(f32_to_bf16_rne(res[j][c]));
          out[128 + w] = __float_as_uint(sum);
        }
      } else if (k < 16) {
        out[w * 32 + 16 + k] = f32_to_bf16_rne(res[j][k]) | (f32_to_bf16_rne(res[j][k + 16]) << 16);
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------ logit kernel
// The logits of a wave step are a small matrix product: 16 keys x 128
// coordinates times up to 16 queries, on v_mfma_f32_16x16x32_bf16.  Lane l
// decodes unit l / 16 (32 coordinates) of key l % 16: its 16 code pairs
// (bf16 128 + e[code]) are the A operand of four K-steps (4 pair words each)
// and its 16 sign pairs (bf16 +-1) those of four more; lane l of the B
// operand holds the matching query pairs of query l % 16 for the same unit
// (the order of the contraction is free as long as A and B agree).  D lane l
// then holds keys 4 (l / 16) + i, i < 4, of query l % 16; the bias
// 192 sum(Pi q), delta, gamma sqrt(pi/2)/128 and |x| are applied per
// element.  Grid (blocks, heads, chunks of 16 queries); 4 waves per
// workgroup; grid-stride over the head's keys with TQ_DEPTH steps in flight.
#ifndef TQ_WAVES
#define TQ_WAVES 2048  // target waves per launch
#endif
#ifndef TQ_DEPTH
#define TQ_DEPTH 4    // key steps in flight per wave
#endif

template <int M, bool FULLN>
__global__ __launch_bounds__(256) void tq_logits_kernel(const uint32_t* __restrict__ codes,
                                                        const uint32_t* __restrict__ signs,
                                                        const uint32_t* __restrict__ norms, int n, int nq,
                                                        float delta, uint32_t tab_lo, uint32_t tab_hi,
                                                        const uint32_t* __restrict__ ws, float* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, kg = lane >> 4;             // A: key r, unit kg; B: query r, unit kg
  const int h = blockIdx.y, q = blockIdx.z * 16 + r;
  const bool qok = q < nq;
  u32x4_t qa[4], ua[4];
  float qsum = 0.f;
  {
    const uint32_t* src = ws + ((size_t)h * nq + (qok ? q : 0)) * kTqQueryWords;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qa[s][e] = qok ? src[kg * 32 + 4 * s + e] : 0u;
        ua[s][e] = qok ? src[kg * 32 + 16 + 4 * s + e] : 0u;
      }
    if (qok)
      for (int w = 0; w < 4; ++w) qsum += __uint_as_float(src[128 + w]);
  }
  const uint32_t T[4] = {tab_lo, tab_hi, 0u, 0u};
  const CbConst kc = cb_consts();
  uint32_t smask = 0x80008000u, sone = 0x3F803F80u;     // opaque: one v_and_or per sign pair
  asm volatile("" : "+v"(smask), "+v"(sone));
  const float gk = 1.2533141373155003f / 128.0f;        // sqrt(pi/2) / d
  const float bias = 192.0f * qsum;
  const size_t hk = (size_t)h * n;
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(codes + hk * 4 * M, (uint32_t)((size_t)n * 16 * M));
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(signs + hk * 4, (uint32_t)((size_t)n * 16));
  const __amdgpu_buffer_rsrc_t nrs = make_rsrc(norms + hk, (uint32_t)((size_t)n * 4));
  struct Raw { uint32_t c[M]; uint32_t s; uint32_t nm[4]; };
  // keys past n get offsets past every buffer (n * 64 < 2^32 - 256): zeros
  auto load = [&](int base, Raw& rw) {
    const int key = base + r;
    const uint32_t u = (uint32_t)key * 4 + (uint32_t)kg;
    const bool ok = key < n;
    buf_load_unit<M>(crs, ok ? u * (M * 4) : 0xFFFFFF00u, 0u, rw.c);
    rw.s = buf_load_u32(srs, ok ? u * 4 : 0xFFFFFF00u, 0u);
    // the norms of keys 4 kg .. 4 kg + 3 (the rows of D this lane holds): one
    // 16-byte load when the key count is a multiple of 4 (a group is then
    // whole or wholly past n), else one load per key.  The form is fixed per
    // instance, never chosen per lane, so every step issues the same number
    // of loads and the waits before a step's decode cover exactly its loads.
    const int k0 = base + 4 * kg;
    if constexpr (FULLN) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(nrs, k0 < n ? (uint32_t)k0 * 4 : 0xFFFFFF00u, 0u, kNT);
      rw.nm[0] = v[0]; rw.nm[1] = v[1]; rw.nm[2] = v[2]; rw.nm[3] = v[3];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = k0 + i;
        rw.nm[i] = buf_load_u32(nrs, kk < n ? (uint32_t)kk * 4 : 0xFFFFFF00u, 0u);
      }
    }
  };
  auto compute = [&](int base, const Raw& rw) {
    uint32_t pr[16];
    decode_unit_cb<M>(rw.c, T, pr, kc);
    const uint32_t ns = ~rw.s;
    f32x4_t dm = {0.f, 0.f, 0.f, 0.f}, ds = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4_t a, sg;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 4 * s + e;
        a[e] = pr[j];
        sg[e] = ((ns << (15 - j)) & smask) | sone;   // bits j, j + 16 -> bf16 +-1
      }
      dm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, qa[s]),
                                                   dm, 0, 0, 0);
      ds = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, sg),
                                                   __builtin_bit_cast(bf16x8_t, ua[s]), ds, 0, 0, 0);
    }
    if (qok) {
      float* orow = out + ((size_t)h * nq + q) * n;
      const int k0 = base + 4 * kg;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float nrm = f16_bits_to_f32(rw.nm[i] & 0xFFFFu), g = f16_bits_to_f32(rw.nm[i] >> 16) * gk;
        v[i] = nrm * (delta * (dm[i] - bias) + g * ds[i]);
      }
      if constexpr (FULLN) {   // rows 16-byte aligned (n % 4 == 0, out aligned): one store of 4 keys
        if (k0 < n) *reinterpret_cast<f32x4_t*>(orow + k0) = f32x4_t{v[0], v[1], v[2], v[3]};
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (k0 + i < n) orow[k0 + i] = v[i];
      }
    }
  };
  constexpr int DEPTH = TQ_DEPTH;
  const int stride = gridDim.x * 4 * 16;
  const int base0 = (blockIdx.x * 4 + wave) * 16;
  Raw rg[DEPTH];
#pragma unroll
  for (int t = 0; t < DEPTH - 1; ++t) load(base0 + t * stride, rg[t]);
  // loads past n read zeros; the last ring turn may decode such zero keys,
  // whose results are not stored
  for (int base = base0; base < n; base += DEPTH * stride) {   // wave-uniform
#pragma unroll
    for (int t = 0; t < DEPTH; ++t) {
      load(base + (t + DEPTH - 1) * stride, rg[(t + DEPTH - 1) % DEPTH]);
      __builtin_amdgcn_sched_barrier(0);
      compute(base + t * stride, rg[t]);
    }
  }
}

// ------------------------------------------------------------ value output
// Attention output over quantized values (the reconstruction variant):
//   o[h][q] = sum_i P[h][q][i] |v_i| Pi^T c[code_i].
// Pass 1 sums in the rotated domain on the matrix cores:
//   a[j][q] = sum_i (128 + e[code_ij]) w_q,i,  W_q = sum_i w_q,i,  w = P |v|.
// A wave takes 16 values per step.  Lane l decodes unit l / 16 of value l % 16
// (codebook byte-permute decode, bf16 128 + e) and writes its 32 coordinates
// into a per-wave LDS tile laid out [coordinate][value]; then
// v_mfma_f32_16x16x16_bf16 multiplies 8 tiles of 16 coordinates x 16 values
// (A, read back with one 8-byte LDS load per tile) by the weights of 16
// values x 16 queries (B, bf16 hi + lo, two MFMAs), lane l of B holding query
// l % 16 and values 4 (l / 16) .. + 3 straight from P and the norms.  The
// four waves of a workgroup meet in LDS and each workgroup leaves its
// partial sums in the workspace.  Pass 2 adds the partials, forms
// o_rot = delta (a - 192 W) and o = Pi^T o_rot (fp32).
constexpr int kTqPart = 129;             // floats per (workgroup, query): 128 sums + W
constexpr int kTqVPitch = 20;            // u16 per coordinate row of a wave's value tile (8-byte aligned rows)
typedef short s16x4_t __attribute__((ext_vector_type(4)));

template <int M, bool FULLN>
__global__ __launch_bounds__(256) void tq_attend_kernel(const uint32_t* __restrict__ codes,
                                                        const uint32_t* __restrict__ norms, int n, int nq,
                                                        const float* __restrict__ P, uint4 tab,
                                                        float* __restrict__ part) {
  __shared__ __align__(16) uint16_t vt[4][128 * kTqVPitch];
  __shared__ float red[4][16][129];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, kg = lane >> 4;            // decode: value r, unit kg; B: query r, values 4 kg ..
  const int h = blockIdx.y, q = blockIdx.z * 16 + r;
  const bool qok = q < nq;
  const uint32_t T[4] = {tab.x, tab.y, tab.z, tab.w};
  const CbConst kc = cb_consts();
  const size_t hk = (size_t)h * n;
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(codes + hk * 4 * M, (uint32_t)((size_t)n * 16 * M));
  const __amdgpu_buffer_rsrc_t nrs = make_rsrc(norms + hk, (uint32_t)((size_t)n * 4));
  const __amdgpu_buffer_rsrc_t prs = make_rsrc(P + ((size_t)h * nq + (qok ? q : 0)) * n, qok ? (uint32_t)((size_t)n * 4) : 0u);
  uint16_t* tile = vt[wave];
  f32x4_t acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  struct Raw { uint32_t c[M]; uint32_t nm[4]; uint32_t p[4]; };
  auto load = [&](int base, Raw& rw) {
    const int key = base + r;
    const uint32_t u = (uint32_t)key * 4 + (uint32_t)kg;
    buf_load_unit<M>(crs, key < n ? u * (M * 4) : 0xFFFFFF00u, 0u, rw.c);
    // norms and weights of values 4 kg .. 4 kg + 3: one 16-byte load each when
    // the value count is a multiple of 4 (a group is then whole or wholly
    // past n), else one load per value; fixed per instance, so every step
    // issues the same number of loads.
    const int k0 = base + 4 * kg;
    if constexpr (FULLN) {
      const uint32_t off = k0 < n ? (uint32_t)k0 * 4 : 0xFFFFFF00u;
      const auto vn = __builtin_amdgcn_raw_buffer_load_b128(nrs, off, 0u, kNT);
      const auto vp = __builtin_amdgcn_raw_buffer_load_b128(prs, off, 0u, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) { rw.nm[i] = vn[i]; rw.p[i] = vp[i]; }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = k0 + i;
        rw.nm[i] = buf_load_u32(nrs, kk < n ? (uint32_t)kk * 4 : 0xFFFFFF00u, 0u);
        rw.p[i] = buf_load_u32(prs, kk < n ? (uint32_t)kk * 4 : 0xFFFFFF00u, 0u);
      }
    }
  };
  auto compute = [&](const Raw& rw) {
    uint32_t pr[16];
    decode_unit_cb<M>(rw.c, T, pr, kc);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const PairInfo pi = Unit<M>::pair(k);
      tile[(32 * kg + pi.ca) * kTqVPitch + r] = (uint16_t)(pr[k] & 0xFFFFu);
      tile[(32 * kg + pi.cb) * kTqVPitch + r] = (uint16_t)(pr[k] >> 16);
    }
    // B: weights w = P |v| of values 4 kg .. 4 kg + 3 for query r, bf16 hi + lo
    float w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[i] = __uint_as_float(rw.p[i]) * f16_bits_to_f32(rw.nm[i] & 0xFFFFu);
      wsum += w[i];
    }
    const uint32_t h01 = cvt_pk_bf16(w[0], w[1]), h23 = cvt_pk_bf16(w[2], w[3]);
    const uint32_t l01 = cvt_pk_bf16(w[0] - bf16_lo_to_f32(h01), w[1] - bf16_hi_to_f32(h01));
    const uint32_t l23 = cvt_pk_bf16(w[2] - bf16_lo_to_f32(h23), w[3] - bf16_hi_to_f32(h23));
    const s16x4_t bh = __builtin_bit_cast(s16x4_t, (uint64_t)h01 | ((uint64_t)h23 << 32));
    const s16x4_t bl = __builtin_bit_cast(s16x4_t, (uint64_t)l01 | ((uint64_t)l23 << 32));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      // A: coordinate 16 t + r, values 4 kg .. 4 kg + 3
      const s16x4_t a = *reinterpret_cast<const s16x4_t*>(tile + (16 * t + r) * kTqVPitch + 4 * kg);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bh, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bl, acc[t], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  const int stride = gridDim.x * 4 * 16;
  int base = (blockIdx.x * 4 + wave) * 16;
  Raw ra{}, rb{};
  load(base, ra);
  while (base < n) {                                   // wave-uniform
    load(base + stride, rb);
    __builtin_amdgcn_sched_barrier(0);
    compute(ra);
    ra = rb;
    base += stride;
  }
  // lane l of tile t holds a[16 t + 4 (l / 16) + i][query l % 16]; W over the 4 lane groups
  wsum += __shfl_xor(wsum, 16);
  wsum += __shfl_xor(wsum, 32);
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][r][16 * t + 4 * kg + i] = acc[t][i];
  if (kg == 0) red[wave][r][128] = wsum;
  __syncthreads();
  float* dst = part + (((size_t)h * gridDim.z + blockIdx.z) * gridDim.x + blockIdx.x) * 16 * kTqPart;
  for (int i = threadIdx.x; i < 16 * kTqPart; i += 256) {
    const int qq = i / kTqPart, j = i % kTqPart;
    dst[i] = red[0][qq][j] + red[1][qq][j] + red[2][qq][j] + red[3][qq][j];
  }
}

// 256 threads: output i = t % 128, half t / 128 of the partials and of the
// Pi^T sum, halves combined in LDS.  The kernel is all latency (about 1 MB of
// partials in all), so loads go out in batches rather than one round trip at
// a time: the weight column W spread over all 256 threads (one block each)
// and reduced across the waves, the partial sums 16 at a time, then the
// thread's 64 entries of Pi in two batches of 32 (a wave can have at most 63
// loads outstanding), the first issued before the reduction's barriers.
__global__ __launch_bounds__(256) void tq_attend_finish_kernel(const float* __restrict__ part, int nblk, int nq,
                                                               const double* __restrict__ Pi, float delta,
                                                               float* __restrict__ out) {
  __shared__ float orot[128], half_a[128], half_o[128];
  __shared__ float wpart[4];
  const int h = blockIdx.x, q = blockIdx.y, t = threadIdx.x, i = t & 127, hh = t >> 7;
  const int nchunk = (nq + 15) / 16, ch = q / 16, qq = q % 16;
  const float* src = part + (((size_t)h * nchunk + ch) * nblk) * 16 * kTqPart + qq * kTqPart;
  const size_t bs = (size_t)16 * kTqPart;
  // W: block t now (consumed after the partial sums), further blocks after
  float w = t < nblk ? src[(size_t)t * bs + 128] : 0.f;
  float a[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) a[u] = 0.f;
  const int b0 = hh * ((nblk + 1) / 2), b1 = hh ? nblk : (nblk + 1) / 2;
  int b = b0;
  for (; b + 15 < b1; b += 16)
#pragma unroll
    for (int u = 0; u < 16; ++u) a[u] += src[(b + u) * bs + i];
  for (; b < b1; ++b) a[0] += src[b * bs + i];
  for (int c = t + 256; c < nblk; c += 256) w += src[c * bs + 128];
  float as = 0.f;
#pragma unroll
  for (int u = 0; u < 16; ++u) as += a[u];
  // Pi[j][i] for the first 32 of this thread's 64 j
  double pv[32];
#pragma unroll
  for (int u = 0; u < 32; ++u) pv[u] = Pi[(size_t)(64 * hh + u) * 128 + i];
  w = wave_sum(w);
  if (hh) half_a[i] = as;
  if ((t & 63) == 0) wpart[t >> 6] = w;
  __syncthreads();
  if (!hh) orot[i] = delta * (as + half_a[i] - 192.0f * ((wpart[0] + wpart[1]) + (wpart[2] + wpart[3])));
  __syncthreads();
  float o[4] = {0.f, 0.f, 0.f, 0.f};                   // (Pi^T o_rot)_i
#pragma unroll
  for (int u = 0; u < 32; ++u) o[u & 3] = __builtin_fmaf((float)pv[u], orot[64 * hh + u], o[u & 3]);
#pragma unroll
  for (int u = 0; u < 32; ++u) pv[u] = Pi[(size_t)(64 * hh + 32 + u) * 128 + i];
#pragma unroll
  for (int u = 0; u < 32; ++u) o[u & 3] = __builtin_fmaf((float)pv[u], orot[64 * hh + 32 + u], o[u & 3]);
  if (hh) half_o[i] = (o[0] + o[1]) + (o[2] + o[3]);
  __syncthreads();
  if (!hh) out[((size_t)h * nq + q) * 128 + i] = (o[0] + o[1]) + (o[2] + o[3]) + half_o[i];
}

// workgroups per head for the value pass (also sizes the workspace)
int64_t tq_attend_blocks(int64_t n, int64_t heads) {
  int64_t per_head = (TQ_WAVES / 4 + heads - 1) / heads;
  const int64_t need = (n + 63) / 64;
  if (per_head > need) per_head = need;
  return per_head < 1 ? 1 : per_head;
}

hipError_t launch_tq_attend(const uint32_t* codes, const uint32_t* norms, int64_t n, int64_t heads, int mbits,
                            float delta, const uint32_t* tab, const double* Pi, const float* P, int64_t nq,
                            float* out, float* part, hipStream_t s) {
  const int64_t nb = tq_attend_blocks(n, heads), nch = (nq + 15) / 16;
  const dim3 grid((unsigned)nb, (unsigned)heads, (unsigned)nch);
  const uint4 t4{tab[0], tab[1], tab[2], tab[3]};
  // weight rows 16-byte aligned when n % 4 == 0 and P is
  const bool full = n % 4 == 0 && (reinterpret_cast<uintptr_t>(P) & 15) == 0;
#define TQA(MB, F) \
  hipLaunchKernelGGL((tq_attend_kernel<MB, F>), grid, dim3(256), 0, s, codes, norms, (int)n, (int)nq, P, t4, part)
  if (mbits == 2) {
    if (full) TQA(2, true);
    else TQA(2, false);
  } else if (mbits == 3) {
    if (full) TQA(3, true);
    else TQA(3, false);
  } else if (mbits == 4) {
    if (full) TQA(4, true);
    else TQA(4, false);
  } else {
    return hipErrorInvalidValue;
  }
#undef TQA
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(tq_attend_finish_kernel, dim3((unsigned)heads, (unsigned)nq), dim3(256), 0, s, part, (int)nb,
                     (int)nq, Pi, delta, out);
  return hipGetLastError();
}

hipError_t launch_tq_project(const double* S, const double* Pi, double* SPi, hipStream_t s) {
  hipLaunchKernelGGL(tq_project_kernel, dim3(128), dim3(128), 0, s, S, Pi, SPi);
  return hipGetLastError();
}

hipError_t launch_tq_logits(const uint32_t* codes, const uint32_t* signs, const uint32_t* norms, int64_t n,
                            int64_t heads, int mbits, float delta, uint32_t tab_lo, uint32_t tab_hi,
                            const double* Pi, const double* SPi, const float* Qv, int64_t nq, float* out,
                            uint32_t* ws, hipStream_t s) {
  const dim3 pg((unsigned)heads, 2, 4);
  if (mbits == 2) hipLaunchKernelGGL((tq_prep_kernel<2>), pg, dim3(256), 0, s, Qv, (int)nq, Pi, SPi, ws);
  else if (mbits == 3) hipLaunchKernelGGL((tq_prep_kernel<3>), pg, dim3(256), 0, s, Qv, (int)nq, Pi, SPi, ws);
  else return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // about TQ_WAVES waves over all heads, at least one workgroup per head
  int64_t per_head = (TQ_WAVES / 4 + heads - 1) / heads;
  const int64_t need = (n + 63) / 64;
  if (per_head > need) per_head = need;
  if (per_head < 1) per_head = 1;
  const dim3 grid((unsigned)per_head, (unsigned)heads, (unsigned)((nq + 15) / 16));
  const bool full = n % 4 == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
#define TQL(MB, F)                                                                                             \
  hipLaunchKernelGGL((tq_logits_kernel<MB, F>), grid, dim3(256), 0, s, codes, signs, norms, (int)n, (int)nq, delta, \
                     tab_lo, tab_hi, ws, out)
  if (mbits == 2) {
    if (full) TQL(2, true);
    else TQL(2, false);
  } else {
    if (full) TQL(3, true);
    else TQL(3, false);
  }
#undef TQL
  return hipGetLastError();
}

}  // namespace qg
