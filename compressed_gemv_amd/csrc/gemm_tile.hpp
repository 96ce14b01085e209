// Prefill GEMM tile kernel, Y[M][N] = X[M][K] W_hat^T, for both weight
// formats (the launchers are in gemm_prefill.hip and gemm_prefill_outlier.hip).
//
// Prefill multiplies many token rows by the same weights, so unlike decode it
// is a dense contraction (arithmetic intensity of thousands of flops per
// weight byte) and belongs on the matrix cores.  A workgroup owns a TM x TN
// (tokens x outputs) tile, 256 x 256 or 128 x 256 with 8 waves or 64 x 128
// with 4, and walks K in steps of TK = 64:
//   * the decoded weight tile (bf16) is staged in LDS with a padded row pitch
//     of TK + 8 elements, so the 16-byte fragment reads of consecutive rows
//     hit distinct banks; a plain bf16 X tile goes from memory straight into
//     LDS (unpadded rows, chunks placed by an XOR of the row so reads stay
//     conflict-free), an X tile scaled by s2 (binary first pass) or split
//     into hi + lo passes through registers; two LDS buffers: while the
//     matrix cores work on step i, the raw weight loads of a later step are
//     in flight and step i+1 is decoded and stored into the other buffer,
//     one barrier per step;
//   * every thread decodes one or two 32-weight units per step: group RTN
//     unit -> fp16 subnormal q*2^(p-24) -> v_fma_mix_f32 s*q + o -> bf16
//     (round to nearest even); binary word -> +-1 (exact);
//   * each wave runs a 32 x 64, 64 x 64 or 64 x 128 block of
//     v_mfma_f32_32x32x16_bf16 tiles per 16-wide k slice, fp32 accumulation;
//   * workgroups are numbered so that the 8 XCDs each take a contiguous run
//     of tiles, N fastest: the concurrent tiles of one XCD share their X rows
//     in that XCD's L2.
// The binary format runs two passes ("70B en 4GB de VRAM...", section 1):
// T = bf16((X (.) s2) V) into the workspace, then Y = (T U^T) (.) s1.
// Short reductions (K < 512) take a split-precision variant in which the
// operand that is not exact in bf16 enters as bf16 hi + lo (weights; X s2 and
// an fp32 T for the binary passes), so every output meets the same error
// bound as the long ones.
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
  static constexpr bool kExact = false;    // w_hat needs more bits than bf16
  // the 32 weights fl32(s q + o) (exact) in k order
  __device__ __forceinline__ void decode_f32(const Raw& r, float (&wv)[32]) const {
    using UN = UnitH<BITS>;
    uint32_t pr[16];
    decode_unit_h<BITS>(r.w, pr);
    const float s = f16_bits_to_f32(r.m & 0xFFFFu), o = f16_bits_to_f32(r.m >> 16);
    float sp[UN::NCLS];
#pragma unroll
    for (int c = 0; c < UN::NCLS; ++c) sp[c] = s * (float)(1 << (24 - BITS * c));
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const PairInfo pi = UN::pair(k);
      const int c = UN::p_of_pair(k) / BITS;
      wv[pi.ca] = __builtin_fmaf(f16_lo(pr[k]), sp[c], o);
      wv[pi.cb] = __builtin_fmaf(f16_hi(pr[k]), sp[c], o);
    }
  }
  __device__ __forceinline__ void decode(const Raw& r, uint32_t (&outp)[16]) const {
    float wv[32];
    decode_f32(r, wv);
#pragma unroll
    for (int i = 0; i < 16; ++i) outp[i] = cvt_pk_bf16(wv[2 * i], wv[2 * i + 1]);
  }
};

struct DecBIN {
  static constexpr int kDictWords = 0;
  static constexpr bool kExact = true;     // +-1 is exact in bf16
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
  static constexpr bool kExact = false;
  // the 32 weights fl32(s e[q] 2^(BITS-7) + o) (exact) in k order
  __device__ __forceinline__ void decode_f32(const Raw& r, float (&wv)[32]) const {
    uint32_t T[4] = {0u, 0u, 0u, 0u};
    const uint32_t* tp = lds_dict + ((r.k & 15u) << BITS) / 4;   // ids < 16 (packer)
#pragma unroll
    for (int i = 0; i < (1 << BITS) / 4; ++i) T[i] = tp[i];
    // entries as fp16 subnormals e * 2^-24: one v_fma_mix_f32 per weight
    uint32_t pr[16];
    decode_unit_cb<BITS, true>(r.w, T, pr, kc);
    const float s = f16_bits_to_f32(r.m & 0xFFFFu) * (float)(1 << (24 - (7 - BITS)));
    const float o = f16_bits_to_f32(r.m >> 16);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const PairInfo pi = Unit<BITS>::pair(k);
      wv[pi.ca] = __builtin_fmaf(f16_lo(pr[k]), s, o);
      wv[pi.cb] = __builtin_fmaf(f16_hi(pr[k]), s, o);
    }
  }
  __device__ __forceinline__ void decode(const Raw& r, uint32_t (&outp)[16]) const {
    float wv[32];
    decode_f32(r, wv);
#pragma unroll
    for (int i = 0; i < 16; ++i) outp[i] = cvt_pk_bf16(wv[2 * i], wv[2 * i + 1]);
  }
};

// Tile configurations: block tile TM x TN, WM x WN waves, each wave
// (TM/WM) x (TN/WN) on 32x32x16 MFMAs; VPM VALU instructions are interleaved
// after each MFMA of a step.
// TK is the K step (a multiple of 32); weight-tile LDS rows are TK + 8 bf16
// apart (a directly loaded X tile is unpadded, see DIRECT below).
struct TileSmall { static constexpr int TM = 128, TN = 256, TK = 64, WM = 2, WN = 4, VPM = 6; };   // 8 waves, 64 x 64
#ifndef QG_BIG_TK
#define QG_BIG_TK 64
#endif
#ifndef QG_DIRECT_A
#define QG_DIRECT_A 1     // bf16 X tiles loaded straight into LDS
#endif
#ifndef QG_BIG_VPM
#define QG_BIG_VPM 3
#endif
// 8 waves of 64 x 128: two waves per SIMD, so one wave's MFMAs run while the
// other waits at the step barrier or on its LDS reads (measured on MI355X
// against 4 waves of 128 x 128, 2 x 4 waves and 2-6 VALU per MFMA: ~10 %
// faster at M = 512 and 4096 for RTN, binary and codebook weights, although
// each step reads 50 % more LDS fragments).  Every instance fits the 256
// registers a wave has at two waves per SIMD; the plain and binary decoders
// run best at 3 VALU per MFMA (4-6 measured no faster).
struct TileBig   { static constexpr int TM = 256, TN = 256, TK = QG_BIG_TK, WM = 4, WN = 2, VPM = QG_BIG_VPM; };   // 8 waves, 64 x 128
// The outlier instances (one more K-step for the side columns) fit their
// registers at 4 VALU per MFMA (3 made the 5- and 6-bit ones spill).
struct TileBigO  { static constexpr int TM = 256, TN = 256, TK = QG_BIG_TK, WM = 4, WN = 2, VPM = 4; };
// The codebook decoder's byte-permute lookups are longer VALU chains: 6 VALU
// per MFMA (registers to spare once the X tile skips the registers) measured
// ~5 % faster than 3 at M = 512 and 4096; the other decoders gain nothing
// from more.
#ifndef QG_BIGC_VPM
#define QG_BIGC_VPM 6
#endif
struct TileBigC  { static constexpr int TM = 256, TN = 256, TK = QG_BIG_TK, WM = 4, WN = 2, VPM = QG_BIGC_VPM; };
// 64 x 128 with 4 waves: the split-precision kernel of short reductions (one
// operand carried as bf16 hi + lo tiles, three tiles per LDS buffer, which a
// smaller block keeps within the LDS), and the plain kernel of launches too
// small to fill the GPU with the larger tiles (two workgroups per CU).
struct TileSplit { static constexpr int TM = 64, TN = 128, TK = 64, WM = 2, WN = 2, VPM = 6; };      // 4 waves, 32 x 64

// AMODE 0: A = X (bf16).  AMODE 1: A = X * s2[k] (fp32, exact), rounded to
// bf16.  AMODE 2: A fp32 (the binary path's T in split precision; SPLIT
// only).  KMASK: Kact % 8 != 0.
// oscale: per-column fp16 scale or null.  nbn: tiles along N.
// OUTL: outlier side columns (fp16 side[N][n_out] at input channels oidx[],
// 1 <= n_out <= TK) enter as one more K-step after the main loop, with A =
// X[m][oidx_j] and B = side[n][j] (zero past n_out), rounded as the weight
// tiles of every other step.
// SPLIT: the inexact operand enters the matrix cores as bf16 hi + lo =
// bf16(v - hi) (2^-16 relative residual), two MFMAs per fragment pair:
// the fp32 A of AMODE 1 and 2, or, with AMODE 0, decoded weights that are
// not exact in bf16.  Used for short reductions, where one bf16 rounding of
// an operand (up to 2^-8 of sum |w||x|) could exceed the error budget.
template <typename Dec, int AMODE, bool KMASK, typename Cfg, bool OUTL, bool SPLIT>
__global__ __launch_bounds__(64 * Cfg::WM * Cfg::WN) void gemm_kernel(
    const void* __restrict__ A, int64_t lda, int M, int Kact, Dec dec, int N,
    const uint16_t* __restrict__ kscale, const uint16_t* __restrict__ oscale,
    void* __restrict__ Y, int64_t ldy, int y_bf16, int nbn,
    const uint16_t* __restrict__ side, const int32_t* __restrict__ oidx, int n_out) {
  static_assert(AMODE != 2 || SPLIT, "fp32 A comes with split precision");
  constexpr bool SPA = SPLIT && AMODE != 0;                  // A as hi + lo
  constexpr bool SPB = SPLIT && AMODE == 0 && !Dec::kExact;  // weights as hi + lo
  constexpr int ESZ = AMODE == 2 ? 4 : 2;                    // bytes per A element
  constexpr int TM = Cfg::TM, TN = Cfg::TN, TK = Cfg::TK, LP = TK + 8, UPR = TK / 32;
  constexpr int NT = 64 * Cfg::WM * Cfg::WN;         // threads
  constexpr int FI = TM / Cfg::WM / 32, FJ = TN / Cfg::WN / 32;   // 32x32 tiles per wave
  constexpr int AC = TM * (TK / 8) / NT;              // 8-element X chunks per thread and step
  constexpr int WU = TN * UPR / NT;                   // weight units per thread and step
  static_assert(AC >= 1 && WU >= 1 && NT % (TK / 8) == 0, "tile configuration");
  // DIRECT: the bf16 X tile goes from memory straight into LDS (buffer
  // loads with the LDS flag, no trip through registers), in unpadded rows of
  // TK elements whose 16-byte chunk c sits at slot c ^ (row % 8), so the
  // fragment reads below stay free of bank conflicts.
  constexpr bool DIRECT = QG_DIRECT_A && AMODE == 0 && !KMASK && !SPLIT && !OUTL;
  constexpr int AP = DIRECT ? TK : LP;                       // A row pitch
  // per buffer: A tile [, A lo tile] and B tile [, B lo tile], A and B in
  // separate arrays (the compiler then knows that reads of one buffer do not
  // wait on direct loads into the other)
  constexpr int AOFF_LO = TM * AP, ABUF = (SPA ? 2 : 1) * TM * AP;
  constexpr int BOFF_LO = TN * LP, BBUF = (SPB ? 2 : 1) * TN * LP;
  __shared__ __align__(16) uint16_t lds_a0[ABUF];
  __shared__ __align__(16) uint16_t lds_a1[ABUF];
  __shared__ __align__(16) uint16_t lds_b[2][BBUF];
  static_assert(!DIRECT || (TK == 64 && AC * (NT / 64) * 8 == TM), "direct X tiles: 1 KB (8 rows) per load");
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
  const int ar = tid / (TK / 8), ac = (tid % (TK / 8)) * 8;   // X: rows ar + AROWS i, 8 elements at ac
  const int nsteps = (Kact + TK - 1) / TK;
  // Branch-free loads through buffer resources based at this tile's first
  // row: rows past M are out of range and read 0, a chunk at or past Kact
  // gets an out-of-range offset.  (A chunk straddling Kact occurs only when
  // Kact % 8 != 0; KMASK then zeroes its tail after the load.)
  const int mrows = min(TM, M - m0);
  const __amdgpu_buffer_rsrc_t ars =
      make_rsrc(static_cast<const char*>(A) + (size_t)m0 * lda * ESZ, (uint32_t)((size_t)mrows * lda * ESZ));
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(kscale, (uint32_t)(AMODE == 1 ? (size_t)Kact * 2 : 0));
  // a: 8 bf16 (AMODE 0, 1) or the first 4 of 8 fp32 (AMODE 2, a2 the rest)
  struct Stage { u32x4_t a[AC]; u32x4_t a2[AMODE == 2 ? AC : 1]; u32x4_t sc; typename Dec::Raw w[WU]; };
  auto gload = [&](int step, Stage& st) {
    const int k = step * TK + ac;
#pragma unroll
    for (int i = 0; i < (DIRECT ? 0 : AC); ++i) {
      const uint32_t off = k < Kact ? (uint32_t)(((size_t)(ar + AROWS * i) * lda + k) * ESZ) : 0xFFFFFFE0u;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(ars, off, 0, 0);
      st.a[i] = u32x4_t{v[0], v[1], v[2], v[3]};
      if constexpr (AMODE == 2) {
        const auto v2 = __builtin_amdgcn_raw_buffer_load_b128(ars, off + 16u, 0, 0);
        st.a2[i] = u32x4_t{v2[0], v2[1], v2[2], v2[3]};
      }
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
    uint16_t* As = buf ? lds_a1 : lds_a0;
    uint16_t* Bs = lds_b[buf];
    if constexpr (KMASK) {
      const int k = step * TK + ac;
      if constexpr (AMODE == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t k0 = (k + e < Kact) ? 0xFFFFFFFFu : 0u, k1 = (k + 4 + e < Kact) ? 0xFFFFFFFFu : 0u;
#pragma unroll
          for (int i = 0; i < AC; ++i) { st.a[i][e] &= k0; st.a2[i][e] &= k1; }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t keep = (k + 2 * e + 1 < Kact) ? 0xFFFFFFFFu : ((k + 2 * e < Kact) ? 0x0000FFFFu : 0u);
#pragma unroll
          for (int i = 0; i < AC; ++i) st.a[i][e] &= keep;
        }
      }
    }
    if constexpr (AMODE == 0) {
      if constexpr (!DIRECT)
#pragma unroll
        for (int i = 0; i < AC; ++i)
          *reinterpret_cast<u32x4_t*>(As + (ar + AROWS * i) * LP + ac) = st.a[i];
    } else {
#pragma unroll
      for (int i = 0; i < AC; ++i) {
        // the 8 fp32 values of the chunk: X * s2 (exact: 8 x 11 significant
        // bits) or T; hi = bf16 (nearest even), lo = bf16(v - hi)
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (AMODE == 1) {
            v[2 * e] = bf16_lo_to_f32(st.a[i][e]) * f16_bits_to_f32(st.sc[e] & 0xFFFFu);
            v[2 * e + 1] = bf16_hi_to_f32(st.a[i][e]) * f16_bits_to_f32(st.sc[e] >> 16);
          } else {
            v[e] = __uint_as_float(st.a[i][e]);
            v[4 + e] = __uint_as_float(st.a2[i][e]);
          }
        }
        u32x4_t hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hi[e] = cvt_pk_bf16(v[2 * e], v[2 * e + 1]);
          if constexpr (SPA) lo[e] = cvt_pk_bf16(v[2 * e] - bf16_lo_to_f32(hi[e]), v[2 * e + 1] - bf16_hi_to_f32(hi[e]));
        }
        *reinterpret_cast<u32x4_t*>(As + (ar + AROWS * i) * LP + ac) = hi;
        if constexpr (SPA) *reinterpret_cast<u32x4_t*>(As + AOFF_LO + (ar + AROWS * i) * LP + ac) = lo;
      }
    }
#pragma unroll
    for (int j = 0; j < WU; ++j) {
      const int idx = tid + NT * j;
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(Bs + (idx / UPR) * LP + (idx % UPR) * 32);
      if constexpr (SPB) {
        float wv[32];
        dec.decode_f32(st.w[j], wv);
        u32x4_t* dlo = reinterpret_cast<u32x4_t*>(lds_b[buf] + BOFF_LO + (idx / UPR) * LP + (idx % UPR) * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x4_t hi, lo;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float w0 = wv[8 * i + 2 * e], w1 = wv[8 * i + 2 * e + 1];
            hi[e] = cvt_pk_bf16(w0, w1);
            lo[e] = cvt_pk_bf16(w0 - bf16_lo_to_f32(hi[e]), w1 - bf16_hi_to_f32(hi[e]));
          }
          dst[i] = hi;
          dlo[i] = lo;
        }
      } else {
        uint32_t v[16];
        dec.decode(st.w[j], v);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = u32x4_t{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
      }
    }
  };
  // v_mfma_f32_32x32x16_bf16: lane l supplies row l % 32 and k = 8 (l / 32) .. +7
  // of each 32 x 16 operand; it sustains near-peak rate with few chains.
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  constexpr int WTM = TM / Cfg::WM, WTN = TN / Cfg::WN;
  constexpr int NA = SPA ? 2 : 1, NB = SPB ? 2 : 1;   // A and B tiles (hi [, lo])
  auto mfma_step = [&](int buf) {
    const uint16_t* As = buf ? lds_a1 : lds_a0;
    const uint16_t* Bs = lds_b[buf];
    // fragments of k-slice s+1 are read before the MFMAs of slice s
    bf16x8_t af[2][NA][FI], bfr[2][NB][FJ];
    auto rd = [&](int kk, bf16x8_t (&a)[NA][FI], bf16x8_t (&b)[NB][FJ]) {
#pragma unroll
      for (int h = 0; h < NA; ++h)
#pragma unroll
        for (int i = 0; i < FI; ++i) {
          const int row = wm * WTM + i * 32 + fr;
          if constexpr (DIRECT)
            a[h][i] = *reinterpret_cast<const bf16x8_t*>(As + row * TK + 8 * (((kk + fk) >> 3) ^ (fr & 7)));
          else
            a[h][i] = *reinterpret_cast<const bf16x8_t*>(As + h * AOFF_LO + row * LP + kk + fk);
        }
#pragma unroll
      for (int h = 0; h < NB; ++h)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
          b[h][j] = *reinterpret_cast<const bf16x8_t*>(Bs + h * TN * LP + (wn * WTN + j * 32 + fr) * LP + kk + fk);
    };
    rd(0, af[0], bfr[0]);
#pragma unroll
    for (int ks = 0; ks < TK / 16; ++ks) {
      if (ks + 1 < TK / 16) rd((ks + 1) * 16, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
#pragma unroll
      for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][0][i], bfr[ks & 1][0][j], acc[i][j], 0, 0, 0);
          if constexpr (SPA)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][NA - 1][i], bfr[ks & 1][0][j], acc[i][j], 0,
                                                                0, 0);
          if constexpr (SPB)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][0][i], bfr[ks & 1][NB - 1][j], acc[i][j], 0,
                                                                0, 0);
        }
    }
  };
  // one half-iteration, a single basic block: issue the raw loads of step
  // s+2, run step s from LDS buffer `cur` on the matrix cores, decode and
  // store step s+1 (loaded one step earlier) into the other buffer, with the
  // decode interleaved between the MFMAs.  Steps past the end load zeros and
  // store into a buffer nobody reads.
  // DIRECT: the X tile of one step into an A buffer.  Wave w's load i
  // fills 1 KB of it, rows 8 (w AC + i) .. +7; lane l takes row l / 8 of
  // those and slot l % 8, i.e. chunk (l % 8) ^ (row % 8) of that row.
  // Rows past M and chunks at or past Kact read 0 (out-of-range offsets).
  auto adirect = [&](int step, int buf) {
    if constexpr (DIRECT) {
      uint16_t* base = buf ? lds_a1 : lds_a0;
      const int wv = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
      for (int i = 0; i < AC; ++i) {
        const int blk = wv * AC + i, r = blk * 8 + (lane >> 3);
        const int k = step * TK + 8 * ((lane & 7) ^ (r & 7));
        const uint32_t off = k < Kact ? (uint32_t)(((size_t)r * lda + k) * 2) : 0xFFFFFFE0u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (__attribute__((address_space(3))) void*)(base + blk * 512), 16,
                                                 off, 0, 0, 0);
      }
    }
  };
  // s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maximum): this
  // wave's direct loads have landed in LDS before the barrier
  auto adirect_wait = [&]() {
    if constexpr (DIRECT) __builtin_amdgcn_s_waitcnt(0x0F70);
  };
  auto half = [&](int step, Stage& ld, Stage& st, int cur) {
    adirect(step + 1, cur ^ 1);
    gload(step + 2, ld);
    // DIRECT waits for every load before the barrier, so the raw loads of
    // step s+2 go out first and have the whole step to arrive
    if constexpr (DIRECT) __builtin_amdgcn_sched_barrier(0);
    mfma_step(cur);
    lstore(step + 1, st, cur ^ 1);
#pragma unroll
    for (int i = 0; i < FI * FJ * (TK / 16) * (SPLIT ? 2 : 1); ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, Cfg::VPM, 0);   // VALU
    }
    adirect_wait();
    __syncthreads();
  };

  Stage s0, s1;
  adirect(0, 0);
  gload(0, s0);
  gload(1, s1);
  if constexpr (Dec::kDictWords > 0) __syncthreads();   // dictionary staged
  lstore(0, s0, 0);
  adirect_wait();
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
    // ended at a barrier).  X is bf16 here (AMODE 0).
    static_assert(AMODE == 0, "outlier columns come with the group format");
    const uint16_t* X = static_cast<const uint16_t*>(A);
    uint16_t* As = lds_a0;
    uint16_t* Bs = lds_b[0];
    for (int t = tid; t < TM * TK; t += NT) {
      const int r = t / TK, c = t % TK, m = m0 + r;
      As[r * LP + c] = (c < n_out && m < M) ? X[(size_t)m * lda + oidx[c]] : (uint16_t)0;
    }
    for (int t = tid; t < TN * TK; t += NT) {
      const int r = t / TK, c = t % TK, n = n0 + r;
      const float sv = (c < n_out && n < N) ? f16_bits_to_f32(side[(size_t)n * n_out + c]) : 0.f;
      const uint32_t hi = f32_to_bf16_rne(sv);
      Bs[r * LP + c] = (uint16_t)hi;
      // fp16 -> bf16 hi keeps 8 of 11 significant bits; lo holds the rest exactly
      if constexpr (SPB) Bs[TN * LP + r * LP + c] = (uint16_t)f32_to_bf16_rne(sv - bf16_bits_to_f32(hi));
    }
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

template <typename Dec, int AMODE, bool KMASK, typename Cfg, bool OUTL = false, bool SPLIT = false>
static hipError_t gemm_launch(const void* A, int64_t lda, int64_t M, int64_t Kact, Dec dec, int64_t N,
                              const uint16_t* kscale, const uint16_t* oscale, void* Y, int64_t ldy,
                              int y_bf16, hipStream_t s, SideCols sc) {
  const int nbn = (int)((N + Cfg::TN - 1) / Cfg::TN);
  const dim3 grid((unsigned)(((M + Cfg::TM - 1) / Cfg::TM) * nbn));
  hipLaunchKernelGGL((gemm_kernel<Dec, AMODE, KMASK, Cfg, OUTL, SPLIT>), grid, dim3(64 * Cfg::WM * Cfg::WN), 0, s,
                     A, lda, (int)M, (int)Kact, dec, (int)N, kscale, oscale, Y, ldy, y_bf16, nbn, sc.vals, sc.idx,
                     sc.n);
  return hipGetLastError();
}

// Reductions shorter than this take the split-precision kernel: with one
// bf16 rounding of an operand, the error of an output is a sum of K terms
// of up to 2^-8 |w||x| each that cancel like a random walk for long K
// (~2^-8 / sqrt(3K) of sum |w||x|) but can reach 2^-8 for short ones.
constexpr int64_t kSplitBelowK = 512;

// The two larger tiles run one workgroup per CU, the 64 x 128 tile two (its
// LDS allows two).  Counting a round as one tile per CU, a round of
// 256 x 256 tiles takes about 7/4 the time of a round of 128 x 256 ones and
// 7/2 that of a round of 64 x 128 ones (fewer LDS reads and barriers per
// MFMA in the larger tiles), so the choice compares whole rounds of tiles
// over the CUs: the big tile wins once
// it has enough tiles to fill the GPU, the smaller ones when their extra
// parallelism saves rounds (short M, narrow N such as k/v projections, the
// narrow first pass of the binary path).  Measured on MI355X over M = 64,
// 512, 4096 and N = 1024, 8192, 28672 (K = 8192): the model picks the
// fastest tile or one within 4 % of it; at equal cost the 64 x 128 tile
// measured faster than the 128 x 256 one.
#ifndef QG_GEMM_TILE
#define QG_GEMM_TILE 0    // 0 = by cost, 1 = small, 2 = big, 3 = 64 x 128
#endif
#ifndef QG_TINY_COST
#define QG_TINY_COST 2    // time of one round of 64 x 128 tiles, in the units of the model below
#endif
enum class TileChoice { Small, Big, Tiny };
static TileChoice pick_tile(int64_t M, int64_t N) {
  if (QG_GEMM_TILE) return QG_GEMM_TILE == 2 ? TileChoice::Big : (QG_GEMM_TILE == 3 ? TileChoice::Tiny : TileChoice::Small);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  auto rounds = [&](int tm, int tn) { return (((M + tm - 1) / tm) * ((N + tn - 1) / tn) + cus - 1) / cus; };
  const int64_t cbig = 7 * rounds(TileBig::TM, TileBig::TN), csmall = 4 * rounds(TileSmall::TM, TileSmall::TN);
  const int64_t ctiny = QG_TINY_COST * rounds(TileSplit::TM, TileSplit::TN);
  if (cbig <= csmall && cbig <= ctiny) return TileChoice::Big;
  return csmall < ctiny ? TileChoice::Small : TileChoice::Tiny;
}

template <typename Dec, int AMODE, bool KMASK, bool OUTL = false, bool SPLIT = false>
static hipError_t gemm_run(const void* A, int64_t lda, int64_t M, int64_t Kact, Dec dec, int64_t N,
                           const uint16_t* kscale, const uint16_t* oscale, void* Y, int64_t ldy,
                           int y_bf16, hipStream_t s, SideCols sc = SideCols{nullptr, nullptr, 0}) {
  if constexpr (SPLIT) {
    return gemm_launch<Dec, AMODE, KMASK, TileSplit, OUTL, true>(A, lda, M, Kact, dec, N, kscale, oscale, Y, ldy,
                                                                 y_bf16, s, sc);
  } else {
    const TileChoice tc = pick_tile(M, N);
    if (tc == TileChoice::Big) {
      if constexpr (OUTL)
        return gemm_launch<Dec, AMODE, KMASK, TileBigO, OUTL>(A, lda, M, Kact, dec, N, kscale, oscale, Y, ldy, y_bf16,
                                                              s, sc);
      else if constexpr (Dec::kDictWords > 0)
        return gemm_launch<Dec, AMODE, KMASK, TileBigC, OUTL>(A, lda, M, Kact, dec, N, kscale, oscale, Y, ldy, y_bf16,
                                                              s, sc);
      else
        return gemm_launch<Dec, AMODE, KMASK, TileBig, OUTL>(A, lda, M, Kact, dec, N, kscale, oscale, Y, ldy, y_bf16,
                                                             s, sc);
    }
    if (tc == TileChoice::Tiny)
      return gemm_launch<Dec, AMODE, KMASK, TileSplit, OUTL, false>(A, lda, M, Kact, dec, N, kscale, oscale, Y, ldy,
                                                                    y_bf16, s, sc);
    return gemm_launch<Dec, AMODE, KMASK, TileSmall, OUTL>(A, lda, M, Kact, dec, N, kscale, oscale, Y, ldy, y_bf16,
                                                           s, sc);
  }
}

}  // namespace qg
