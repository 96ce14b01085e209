// Prefill GEMM tile kernel, Y[M][N] = X[M][K] W_hat^T, for both weight
// formats (the launchers are in gemm_prefill.hip and gemm_prefill_outlier.hip).
//
// Prefill multiplies many token rows by the same weights, so unlike decode it
// is a dense contraction (arithmetic intensity of thousands of flops per
// weight byte) and belongs on the matrix cores.  A workgroup owns a TM x TN
// (tokens x outputs) tile, 128 x 256 with 8 waves or 256 x 256 with 4 waves,
// and walks K in steps of TK = 64:
//   * the X tile (bf16, optionally scaled by s2 and re-rounded) and the
//     decoded weight tile (bf16) are staged in LDS with a padded row pitch of
//     TK + 8 elements, so the 16-byte fragment reads of consecutive rows hit
//     distinct banks; two LDS buffers and two register stages: while the
//     matrix cores work on step i, the raw loads of step i+2 are in flight
//     and step i+1 is decoded and stored into the other LDS buffer, one
//     barrier per step;
//   * every thread decodes one or two 32-weight units per step: group RTN
//     unit -> fp16 subnormal q*2^(p-24) -> v_fma_mix_f32 s*q + o -> bf16
//     (round to nearest even); binary word -> +-1 (exact);
//   * each wave runs a 64 x 64 or 128 x 128 block of v_mfma_f32_32x32x16_bf16
//     tiles per 16-wide k slice, fp32 accumulation;
//   * workgroups are numbered so that the 8 XCDs each take a contiguous run
//     of tiles, N fastest: the concurrent tiles of one XCD share their X rows
//     in that XCD's L2.
// The binary format runs two passes ("70B en 4GB de VRAM...", section 1):
// T = bf16((X (.) s2) V) into the workspace, then Y = (T U^T) (.) s1.
#pragma once

#include "codebook.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace qg {


// Weight decoders.  load() fetches the raw bits of 32 consecutive k of weight
// row n starting at unit u (zero outside the matrix); decode() turns them
// into 16 bf16 pairs in k order.
template <int BITS, int G>
struct DecRTN {
  static constexpr int kDictWords = 0;     // no per-kernel table
  const uint32_t* codes; const uint32_t* meta; int N; int U;
  struct Raw { uint32_t w[BITS]; uint32_t m; };
  __device__ __forceinline__ void load(int n, int u, Raw& r) const {
    const int GN = U * 32 / G;
    const __amdgpu_buffer_rsrc_t crs = make_rsrc(codes, (uint32_t)((size_t)N * U * BITS * 4));
    const __amdgpu_buffer_rsrc_t mrs = make_rsrc(meta, (uint32_t)((size_t)N * GN * 4));
    const bool ok = n < N && u < U;
    const uint32_t co = ok ? (uint32_t)(n * U + u) * (BITS * 4) : 0xFFFFFF00u;
    const uint32_t mo = ok ? (uint32_t)(n * GN + (u * 32) / G) * 4 : 0xFFFFFF00u;
    buf_load_unit<BITS, 0>(crs, co, 0u, r.w);
    r.m = __builtin_amdgcn_raw_buffer_load_b32(mrs, mo, 0u, 0);
  }
  __device__ __forceinline__ void decode(const Raw& r, uint32_t (&outp)[16]) const {
    using UN = UnitH<BITS>;
    uint32_t pr[16];
    decode_unit_h<BITS>(r.w, pr);
    const float s = f16_bits_to_f32(r.m & 0xFFFFu), o = f16_bits_to_f32(r.m >> 16);
    float sp[UN::NCLS];
#pragma unroll
    for (int c = 0; c < UN::NCLS; ++c) sp[c] = s * (float)(1 << (24 - BITS * c));
    float wv[32];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const PairInfo pi = UN::pair(k);
      const int c = UN::p_of_pair(k) / BITS;
      wv[pi.ca] = __builtin_fmaf(f16_lo(pr[k]), sp[c], o);
      wv[pi.cb] = __builtin_fmaf(f16_hi(pr[k]), sp[c], o);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) outp[i] = cvt_pk_bf16(wv[2 * i], wv[2 * i + 1]);
  }
};

struct DecBIN {
  static constexpr int kDictWords = 0;
  const uint32_t* bits; int N; int Wn;   // rows, words per stored row
  struct Raw { uint32_t w; };
  __device__ __forceinline__ void load(int n, int u, Raw& r) const {
    const __amdgpu_buffer_rsrc_t brs = make_rsrc(bits, (uint32_t)((size_t)N * Wn * 4));
    const uint32_t off = (n < N && u < Wn) ? (uint32_t)(n * Wn + u) * 4u : 0xFFFFFF00u;
    r.w = __builtin_amdgcn_raw_buffer_load_b32(brs, off, 0u, 0);
  }
  __device__ __forceinline__ void decode(const Raw& r, uint32_t (&outp)[16]) const {
    // bit -> sign: 1 -> +1.0 (0x3F80), 0 -> -1.0 (0xBF80); bit 2i lands on
    // bit 15, bit 2i+1 on bit 31.  A zero word outside the matrix meets zero
    // activations.
    const uint32_t nw = ~r.w;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t lo = 2 * i <= 15 ? (nw << (15 - 2 * i)) : (nw >> (2 * i - 15));
      const uint32_t hi = nw << (30 - 2 * i);
      outp[i] = (lo & 0x00008000u) | (hi & 0x80000000u) | 0x3F803F80u;
    }
  }
};

// Group codes read through per-group books: the dictionary (<= 16 books of
// 2^BITS bytes) is staged in LDS once per workgroup (bind), each unit's book
// id is loaded with its meta word, and a unit decodes to
// fl32(s e[q] 2^(BITS-7) + o) rounded to bf16, as DecRTN does for s q + o.
template <int BITS, int G>
struct DecCB {
  static constexpr int kDictWords = 64;
  const uint32_t* codes; const uint32_t* meta; const uint8_t* ids; const uint8_t* dict; int nb; int N; int U;
  const uint32_t* lds_dict;
  CbConst kc;
  struct Raw { uint32_t w[BITS]; uint32_t m; uint32_t k; };
  // stage the dictionary (all threads of the workgroup; a barrier follows)
  __device__ __forceinline__ void bind(uint32_t* lds, int tid, int nt) {
    for (int t = tid; t < (nb << BITS); t += nt) reinterpret_cast<uint8_t*>(lds)[t] = dict[t];
    lds_dict = lds;
    kc = cb_consts();
  }
  __device__ __forceinline__ void load(int n, int u, Raw& r) const {
    const int GN = U * 32 / G;
    const __amdgpu_buffer_rsrc_t crs = make_rsrc(codes, (uint32_t)((size_t)N * U * BITS * 4));
    const __amdgpu_buffer_rsrc_t mrs = make_rsrc(meta, (uint32_t)((size_t)N * GN * 4));
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(ids, (uint32_t)((size_t)N * GN));
    const bool ok = n < N && u < U;
    const uint32_t co = ok ? (uint32_t)(n * U + u) * (BITS * 4) : 0xFFFFFF00u;
    const uint32_t go = ok ? (uint32_t)(n * GN + (u * 32) / G) : 0x3FFFFFC0u;
    buf_load_unit<BITS, 0>(crs, co, 0u, r.w);
    r.m = __builtin_amdgcn_raw_buffer_load_b32(mrs, go * 4, 0u, 0);
    r.k = __builtin_amdgcn_raw_buffer_load_b8(krs, go, 0u, 0);
  }
  __device__ __forceinline__ void decode(const Raw& r, uint32_t (&outp)[16]) const {
    uint32_t T[4] = {0u, 0u, 0u, 0u};
    const uint32_t* tp = lds_dict + ((r.k & 15u) << BITS) / 4;   // ids < 16 (packer)
#pragma unroll
    for (int i = 0; i < (1 << BITS) / 4; ++i) T[i] = tp[i];
    uint32_t pr[16];
    decode_unit_cb<BITS>(r.w, T, pr, kc);
    const float s = f16_bits_to_f32(r.m & 0xFFFFu) * (1.0f / (float)(1 << (7 - BITS)));
    const float o = f16_bits_to_f32(r.m >> 16);
    float wv[32];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const PairInfo pi = Unit<BITS>::pair(k);
      wv[pi.ca] = __builtin_fmaf(bf16_lo_to_f32(pr[k]) - 128.0f, s, o);
      wv[pi.cb] = __builtin_fmaf(bf16_hi_to_f32(pr[k]) - 128.0f, s, o);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) outp[i] = cvt_pk_bf16(wv[2 * i], wv[2 * i + 1]);
  }
};

// Tile configurations: block tile TM x TN, WM x WN waves, each wave
// (TM/WM) x (TN/WN) on 32x32x16 MFMAs; VPM VALU instructions are interleaved
// after each MFMA of a step.
// TK is the K step (a multiple of 32); LDS rows are TK + 8 bf16 apart.
struct TileSmall { static constexpr int TM = 128, TN = 256, TK = 64, WM = 2, WN = 4, VPM = 6; };   // 8 waves, 64 x 64
#ifndef QG_BIG_TK
#define QG_BIG_TK 64
#endif
#ifndef QG_BIG_VPM
#define QG_BIG_VPM 3
#endif
struct TileBig   { static constexpr int TM = 256, TN = 256, TK = QG_BIG_TK, WM = 2, WN = 2, VPM = QG_BIG_VPM; };   // 4 waves, 128 x 128

// AMODE 0: A = X (bf16).  AMODE 1: A = bf16(X * s2[k]).  KMASK: Kact % 8 != 0.
// oscale: per-column fp16 scale or null.  nbn: tiles along N.
// OUTL: outlier side columns (fp16 side[N][n_out] at input channels oidx[],
// 1 <= n_out <= TK) enter as one more K-step after the main loop, with A =
// X[m][oidx_j] and B = bf16(side[n][j]) (zero past n_out): the same bf16
// weight tiles as every other step.
template <typename Dec, int AMODE, bool KMASK, typename Cfg, bool OUTL>
__global__ __launch_bounds__(64 * Cfg::WM * Cfg::WN) void gemm_kernel(
    const uint16_t* __restrict__ A, int64_t lda, int M, int Kact, Dec dec, int N,
    const uint16_t* __restrict__ kscale, const uint16_t* __restrict__ oscale,
    void* __restrict__ Y, int64_t ldy, int y_bf16, int nbn,
    const uint16_t* __restrict__ side, const int32_t* __restrict__ oidx, int n_out) {
  constexpr int TM = Cfg::TM, TN = Cfg::TN, TK = Cfg::TK, LP = TK + 8, UPR = TK / 32;
  constexpr int NT = 64 * Cfg::WM * Cfg::WN;         // threads
  constexpr int FI = TM / Cfg::WM / 32, FJ = TN / Cfg::WN / 32;   // 32x32 tiles per wave
  constexpr int AC = TM * (TK / 8) / NT;              // 16-byte X chunks per thread and step
  constexpr int WU = TN * UPR / NT;                   // weight units per thread and step
  static_assert(AC >= 1 && WU >= 1 && NT % (TK / 8) == 0, "tile configuration");
  __shared__ __align__(16) uint16_t lds[2][(TM + TN) * LP];
  __shared__ __align__(16) uint32_t dict_lds[Dec::kDictWords > 0 ? Dec::kDictWords : 1];
  const int tid = threadIdx.x;
  if constexpr (Dec::kDictWords > 0) dec.bind(dict_lds, tid, NT);   // staged before the first decode
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
  int bid = blockIdx.x;
  const int nb = gridDim.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);   // XCD-contiguous runs
  const int m0 = (bid / nbn) * TM, n0 = (bid % nbn) * TN;
  f32x16_t acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  constexpr int AROWS = NT / (TK / 8);                // X rows covered per chunk round
  const int ar = tid / (TK / 8), ac = (tid % (TK / 8)) * 8;   // X: rows ar + AROWS i, 8 bf16 at ac
  const int nsteps = (Kact + TK - 1) / TK;
  // Branch-free loads through buffer resources based at this tile's first
  // row: rows past M are out of range and read 0, a chunk at or past Kact
  // gets an out-of-range offset.  (A chunk straddling Kact occurs only when
  // Kact % 8 != 0; KMASK then zeroes its tail after the load.)
  const int mrows = min(TM, M - m0);
  const __amdgpu_buffer_rsrc_t ars = make_rsrc(A + (size_t)m0 * lda, (uint32_t)((size_t)mrows * lda * 2));
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(kscale, (uint32_t)(AMODE == 1 ? (size_t)Kact * 2 : 0));
  struct Stage { u32x4_t a[AC]; u32x4_t sc; typename Dec::Raw w[WU]; };
  auto gload = [&](int step, Stage& st) {
    const int k = step * TK + ac;
#pragma unroll
    for (int i = 0; i < AC; ++i) {
      const uint32_t off = k < Kact ? (uint32_t)(((size_t)(ar + AROWS * i) * lda + k) * 2) : 0xFFFFFFF0u;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(ars, off, 0, 0);
      st.a[i] = u32x4_t{v[0], v[1], v[2], v[3]};
    }
    if constexpr (AMODE == 1) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(srs, k < Kact ? (uint32_t)k * 2 : 0xFFFFFFF0u, 0, 0);
      st.sc = u32x4_t{v[0], v[1], v[2], v[3]};
    }
#pragma unroll
    for (int j = 0; j < WU; ++j) {
      const int idx = tid + NT * j;                   // (row, unit) = (idx / UPR, idx % UPR)
      dec.load(n0 + idx / UPR, step * UPR + idx % UPR, st.w[j]);
    }
  };
  // scale (AMODE 1), decode and store one K-step into an LDS buffer
  auto lstore = [&](int step, Stage& st, int buf) {
    uint16_t* As = lds[buf];
    uint16_t* Bs = lds[buf] + TM * LP;
    if constexpr (KMASK) {
      const int k = step * TK + ac;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t keep = (k + 2 * e + 1 < Kact) ? 0xFFFFFFFFu : ((k + 2 * e < Kact) ? 0x0000FFFFu : 0u);
#pragma unroll
        for (int i = 0; i < AC; ++i) st.a[i][e] &= keep;
      }
    }
    if constexpr (AMODE == 1) {
      // A = bf16(X * s2[k]), re-rounded to nearest even
#pragma unroll
      for (int i = 0; i < AC; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          st.a[i][e] = cvt_pk_bf16(bf16_lo_to_f32(st.a[i][e]) * f16_bits_to_f32(st.sc[e] & 0xFFFFu),
                                   bf16_hi_to_f32(st.a[i][e]) * f16_bits_to_f32(st.sc[e] >> 16));
    }
#pragma unroll
    for (int i = 0; i < AC; ++i)
      *reinterpret_cast<u32x4_t*>(As + (ar + AROWS * i) * LP + ac) = st.a[i];
#pragma unroll
    for (int j = 0; j < WU; ++j) {
      const int idx = tid + NT * j;
      uint32_t v[16];
      dec.decode(st.w[j], v);
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(Bs + (idx / UPR) * LP + (idx % UPR) * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = u32x4_t{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
    }
  };
  // v_mfma_f32_32x32x16_bf16: lane l supplies row l % 32 and k = 8 (l / 32) .. +7
  // of each 32 x 16 operand; it sustains near-peak rate with few chains.
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  constexpr int WTM = TM / Cfg::WM, WTN = TN / Cfg::WN;
  auto mfma_step = [&](int buf) {
    const uint16_t* As = lds[buf];
    const uint16_t* Bs = lds[buf] + TM * LP;
    // fragments of k-slice s+1 are read before the MFMAs of slice s
    bf16x8_t af[2][FI], bfr[2][FJ];
    auto rd = [&](int kk, bf16x8_t (&a)[FI], bf16x8_t (&b)[FJ]) {
#pragma unroll
      for (int i = 0; i < FI; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(As + (wm * WTM + i * 32 + fr) * LP + kk + fk);
#pragma unroll
      for (int j = 0; j < FJ; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(Bs + (wn * WTN + j * 32 + fr) * LP + kk + fk);
    };
    rd(0, af[0], bfr[0]);
#pragma unroll
    for (int ks = 0; ks < TK / 16; ++ks) {
      if (ks + 1 < TK / 16) rd((ks + 1) * 16, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
#pragma unroll
      for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][i], bfr[ks & 1][j], acc[i][j], 0, 0, 0);
    }
  };
  // one half-iteration, a single basic block: issue the raw loads of step
  // s+2, run step s from LDS buffer `cur` on the matrix cores, decode and
  // store step s+1 (loaded one step earlier) into the other buffer, with the
  // decode interleaved between the MFMAs.  Steps past the end load zeros and
  // store into a buffer nobody reads.
  auto half = [&](int step, Stage& ld, Stage& st, int cur) {
    gload(step + 2, ld);
    mfma_step(cur);
    lstore(step + 1, st, cur ^ 1);
#pragma unroll
    for (int i = 0; i < FI * FJ * (TK / 16); ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, Cfg::VPM, 0);   // VALU
    }
    __syncthreads();
  };

  Stage s0, s1;
  gload(0, s0);
  gload(1, s1);
  if constexpr (Dec::kDictWords > 0) __syncthreads();   // dictionary staged
  lstore(0, s0, 0);
  __syncthreads();
  // Whole pairs of steps, so the loop has one exit: with an odd step count
  // the last half-step runs on a buffer of zeros (everything loaded past the
  // end is zero), which leaves the sums unchanged.
  for (int step = 0; step < nsteps; step += 2) {
    half(step, s0, s1, 0);            // s0 <- step + 2, s1 (step + 1) -> buffer 1
    half(step + 1, s1, s0, 1);        // s1 <- step + 3, s0 (step + 2) -> buffer 0
  }
  if constexpr (OUTL) {
    // the outlier K-step; the main loop is done with LDS (its last step
    // ended at a barrier)
    uint16_t* As = lds[0];
    uint16_t* Bs = lds[0] + TM * LP;
    for (int t = tid; t < TM * TK; t += NT) {
      const int r = t / TK, c = t % TK, m = m0 + r;
      As[r * LP + c] = (c < n_out && m < M) ? A[(size_t)m * lda + oidx[c]] : (uint16_t)0;
    }
    for (int t = tid; t < TN * TK; t += NT) {
      const int r = t / TK, c = t % TK, n = n0 + r;
      As[TM * LP + r * LP + c] = (c < n_out && n < N)
          ? (uint16_t)f32_to_bf16_rne(f16_bits_to_f32(side[(size_t)n * n_out + c])) : (uint16_t)0;
    }
    (void)Bs;
    __syncthreads();
    mfma_step(0);
  }
  // ---- epilogue: lane l holds D[8 (e / 4) + 4 (l / 32) + e % 4][l % 32] of each 32x32 tile
  const int col_l = lane & 31, row_l = (lane >> 5) * 4;
#pragma unroll
  for (int j = 0; j < FJ; ++j) {
    const int n = n0 + wn * WTN + j * 32 + col_l;
    if (n >= N) continue;
    const float sc = oscale ? f16_bits_to_f32(oscale[n]) : 1.0f;
#pragma unroll
    for (int i = 0; i < FI; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * WTM + i * 32 + 8 * (e >> 2) + row_l + (e & 3);
        if (m < M) {
          const float vout = acc[i][j][e] * sc;
          if (y_bf16) static_cast<uint16_t*>(Y)[(size_t)m * ldy + n] = (uint16_t)f32_to_bf16_rne(vout);
          else static_cast<float*>(Y)[(size_t)m * ldy + n] = vout;
        }
      }
    }
  }
}

struct SideCols { const uint16_t* vals; const int32_t* idx; int n; };   // outlier columns (n = 0: none)

template <typename Dec, int AMODE, bool KMASK, typename Cfg, bool OUTL = false>
static hipError_t gemm_launch(const uint16_t* A, int64_t lda, int64_t M, int64_t Kact, Dec dec, int64_t N,
                              const uint16_t* kscale, const uint16_t* oscale, void* Y, int64_t ldy,
                              int y_bf16, hipStream_t s, SideCols sc) {
  const int nbn = (int)((N + Cfg::TN - 1) / Cfg::TN);
  const dim3 grid((unsigned)(((M + Cfg::TM - 1) / Cfg::TM) * nbn));
  hipLaunchKernelGGL((gemm_kernel<Dec, AMODE, KMASK, Cfg, OUTL>), grid, dim3(64 * Cfg::WM * Cfg::WN), 0, s, A,
                     lda, (int)M, (int)Kact, dec, (int)N, kscale, oscale, Y, ldy, y_bf16, nbn, sc.vals, sc.idx, sc.n);
  return hipGetLastError();
}

// Either tile runs one workgroup per CU, and a 256 x 256 tile takes about
// 7/4 the time of a 128 x 256 one (fewer LDS reads and barriers per MFMA),
// so the choice compares whole rounds of workgroups over the CUs: the big
// tile wins once it has enough tiles to fill the GPU, the small one when
// its extra parallelism saves a round (short M, or the narrow first pass of
// the binary path).
#ifndef QG_GEMM_TILE
#define QG_GEMM_TILE 0    // 0 = by cost, 1 = small, 2 = big
#endif
static bool use_big_tile(int64_t M, int64_t N) {
  if (QG_GEMM_TILE) return QG_GEMM_TILE == 2;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const int64_t nbig = ((M + TileBig::TM - 1) / TileBig::TM) * ((N + TileBig::TN - 1) / TileBig::TN);
  const int64_t nsmall = ((M + TileSmall::TM - 1) / TileSmall::TM) * ((N + TileSmall::TN - 1) / TileSmall::TN);
  return 7 * ((nbig + cus - 1) / cus) <= 4 * ((nsmall + cus - 1) / cus);
}

template <typename Dec, int AMODE, bool KMASK, bool OUTL = false>
static hipError_t gemm_run(const uint16_t* A, int64_t lda, int64_t M, int64_t Kact, Dec dec, int64_t N,
                           const uint16_t* kscale, const uint16_t* oscale, void* Y, int64_t ldy,
                           int y_bf16, hipStream_t s, SideCols sc = SideCols{nullptr, nullptr, 0}) {
  if (use_big_tile(M, N))
    return gemm_launch<Dec, AMODE, KMASK, TileBig, OUTL>(A, lda, M, Kact, dec, N, kscale, oscale, Y, ldy, y_bf16,
                                                         s, sc);
  return gemm_launch<Dec, AMODE, KMASK, TileSmall, OUTL>(A, lda, M, Kact, dec, N, kscale, oscale, Y, ldy, y_bf16,
                                                         s, sc);
}

}  // namespace qg
