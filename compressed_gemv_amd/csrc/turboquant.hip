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
// A prep kernel forms Pi q and S Pi q once per query (fp64 sums, rounded to
// bf16 and laid out as the dot-product pairs of the logit kernel).  The logit
// kernel streams the keys: four lanes per key, one 32-coordinate unit each;
// the centroid codes go through the codebook byte-permute decode (pairs
// 128 + e[code] in bf16) and the sign bits become bf16 +-1 pairs with one
// shift and one masked OR; v_dot2_f32_bf16 against the query pairs, a
// two-step DPP sum over the quad, and the per-key fp16 norms scale the
// result.  A key is read once for up to 4 queries (grouped-query heads).
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
// Per (query, head): qr = Pi q, u = S qr in fp64 (increasing index order),
// then for unit w and pair k: word w*32 + k = bf16 (qr[32w + ca], qr[32w + cb])
// with (ca, cb) the code pair k of an M-bit unit; word w*32 + 16 + j =
// bf16 (u[32w + j], u[32w + j + 16]); float at 128 + w = the sum of the 32
// bf16-rounded qr values of unit w (the 128-bias correction).
constexpr int kTqQueryWords = 132;

template <int M>
__global__ __launch_bounds__(128) void tq_prep_kernel(const float* __restrict__ Qv, int nq, const double* __restrict__ Pi,
                                                      const double* __restrict__ S, uint32_t* __restrict__ ws) {
  constexpr int D = 128;
  __shared__ double qs[D], qr[D];
  __shared__ uint32_t qb[D], ub[D];
  const int qi = blockIdx.x, h = blockIdx.y, i = threadIdx.x;
  const size_t row = (size_t)h * nq + qi;
  qs[i] = (double)Qv[row * D + i];
  __syncthreads();
  double a = 0.0;
  for (int j = 0; j < D; ++j) a = a + qs[j] * Pi[i * D + j];
  qr[i] = a;
  qb[i] = f32_to_bf16_rne((float)a);
  __syncthreads();
  double b = 0.0;
  for (int j = 0; j < D; ++j) b = b + qr[j] * S[i * D + j];
  ub[i] = f32_to_bf16_rne((float)b);
  __syncthreads();
  uint32_t* out = ws + row * kTqQueryWords;
  if (i < 64) {
    const int w = i / 16, k = i % 16;
    const PairInfo pi = Unit<M>::pair(k);
    out[w * 32 + k] = qb[32 * w + pi.ca] | (qb[32 * w + pi.cb] << 16);
    out[w * 32 + 16 + k] = ub[32 * w + k] | (ub[32 * w + k + 16] << 16);
  } else if (i < 68) {
    const int w = i - 64;
    float s = 0.f;
    for (int c = 0; c < 32; ++c) s += bf16_bits_to_f32(qb[32 * w + c]);
    out[128 + w] = __float_as_uint(s);
  }
}

// ------------------------------------------------------------ logit kernel
// Grid (blocks, heads, query chunks of Q); 4 waves per workgroup; a wave
// takes 16 keys per step (lane = 4 * key slot + unit), grid-stride over the
// head's n keys with the next step's loads issued before the current step is
// decoded.  Keys past n read zeros and are not stored.
template <int M, int Q>
__global__ __launch_bounds__(256) void tq_logits_kernel(const uint32_t* __restrict__ codes,
                                                        const uint32_t* __restrict__ signs,
                                                        const uint32_t* __restrict__ norms, int n, int nq,
                                                        float delta, uint32_t tab_lo, uint32_t tab_hi,
                                                        const uint32_t* __restrict__ ws, float* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int w = lane & 3, slot = lane >> 2;
  const int h = blockIdx.y, q0 = blockIdx.z * Q;
  uint32_t qp[Q][16], up[Q][16];
  float qsum[Q];
#pragma unroll
  for (int t = 0; t < Q; ++t) {
    const int qi = q0 + t < nq ? q0 + t : nq - 1;      // padded queries repeat the last one, never stored
    const uint32_t* src = ws + ((size_t)h * nq + qi) * kTqQueryWords;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      qp[t][k] = src[w * 32 + k];
      up[t][k] = src[w * 32 + 16 + k];
    }
    qsum[t] = __uint_as_float(src[128 + w]);
  }
  const uint32_t T[4] = {tab_lo, tab_hi, 0u, 0u};
  const CbConst kc = cb_consts();
  const float gk = 1.2533141373155003f / 128.0f;        // sqrt(pi/2) / d
  const size_t hk = (size_t)h * n;
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(codes + hk * 4 * M, (uint32_t)((size_t)n * 16 * M));
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(signs + hk * 4, (uint32_t)((size_t)n * 16));
  const __amdgpu_buffer_rsrc_t nrs = make_rsrc(norms + hk, (uint32_t)((size_t)n * 4));
  struct Raw { uint32_t c[M]; uint32_t s; uint32_t nm; };
  // keys past n get offsets past every buffer (n * 64 < 2^32 - 256): zeros
  auto load = [&](int key, Raw& r) {
    const bool ok = key < n;
    const uint32_t u = (uint32_t)key * 4 + (uint32_t)w;
    buf_load_unit<M>(crs, ok ? u * (M * 4) : 0xFFFFFF00u, 0u, r.c);
    r.s = buf_load_u32(srs, ok ? u * 4 : 0xFFFFFF00u, 0u);
    r.nm = buf_load_u32(nrs, ok ? (uint32_t)key * 4 : 0xFFFFFF00u, 0u);
  };
  auto compute = [&](int key, const Raw& r) {
    uint32_t pr[16];
    decode_unit_cb<M>(r.c, T, pr, kc);
    const uint32_t ns = ~r.s;
    uint32_t sp[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) sp[j] = ((ns << (15 - j)) & 0x80008000u) | 0x3F803F80u;
    const float nrm = f16_bits_to_f32(r.nm & 0xFFFFu), g = f16_bits_to_f32(r.nm >> 16) * gk;
#pragma unroll
    for (int t = 0; t < Q; ++t) {
      float a0 = -192.0f * qsum[t], a1 = 0.f, b0 = 0.f, b1 = 0.f;
#pragma unroll
      for (int k = 0; k < 16; k += 2) {
        a0 = dot2_bf16(pr[k], qp[t][k], a0);
        a1 = dot2_bf16(pr[k + 1], qp[t][k + 1], a1);
        b0 = dot2_bf16(sp[k], up[t][k], b0);
        b1 = dot2_bf16(sp[k + 1], up[t][k + 1], b1);
      }
      float part = delta * (a0 + a1) + g * (b0 + b1);
      part += dpp_f32<0xB1>(part);   // quad_perm [1,0,3,2]
      part += dpp_f32<0x4E>(part);   // quad_perm [2,3,0,1]
      if (w == 0 && key < n && q0 + t < nq) out[((size_t)h * nq + q0 + t) * n + key] = nrm * part;
    }
  };
  const int stride = gridDim.x * 4 * 16;
  int key = (blockIdx.x * 4 + wave) * 16 + slot;
  Raw ra{}, rb{};
  if (key - slot < n) load(key, ra);
  while (key - slot < n) {
    const int nxt = key + stride;
    const bool more = nxt - slot < n;                    // wave-uniform
    if (more) load(nxt, rb);
    __builtin_amdgcn_sched_barrier(0);
    compute(key, ra);
    ra = rb;
    key = nxt;
  }
}

hipError_t launch_tq_logits(const uint32_t* codes, const uint32_t* signs, const uint32_t* norms, int64_t n,
                            int64_t heads, int mbits, float delta, uint32_t tab_lo, uint32_t tab_hi,
                            const double* Pi, const double* S, const float* Qv, int64_t nq, float* out,
                            uint32_t* ws, hipStream_t s) {
  const dim3 pg((unsigned)nq, (unsigned)heads);
  if (mbits == 2) hipLaunchKernelGGL((tq_prep_kernel<2>), pg, dim3(128), 0, s, Qv, (int)nq, Pi, S, ws);
  else if (mbits == 3) hipLaunchKernelGGL((tq_prep_kernel<3>), pg, dim3(128), 0, s, Qv, (int)nq, Pi, S, ws);
  else return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // about 2048 waves over all heads, at least one workgroup per head
  const int Q = nq <= 1 ? 1 : (nq <= 2 ? 2 : 4);
  int64_t per_head = (2048 / 4 + heads - 1) / heads;
  const int64_t need = (n + 63) / 64;
  if (per_head > need) per_head = need;
  if (per_head < 1) per_head = 1;
  const dim3 grid((unsigned)per_head, (unsigned)heads, (unsigned)((nq + Q - 1) / Q));
#define L(MB, QQ)                                                                                       \
  hipLaunchKernelGGL((tq_logits_kernel<MB, QQ>), grid, dim3(256), 0, s, codes, signs, norms, (int)n, (int)nq, \
                     delta, tab_lo, tab_hi, ws, out)
  if (mbits == 2) { if (Q == 1) L(2, 1); else if (Q == 2) L(2, 2); else L(2, 4); }
  else { if (Q == 1) L(3, 1); else if (Q == 2) L(3, 2); else L(3, 4); }
#undef L
  return hipGetLastError();
}

}  // namespace qg
