// Group-RTN GEMV kernels for decode (templates shared by the plain, outlier,
// grouped and codebook entry points).
//
// A decode step reads every weight byte once and does two flops per weight,
// so it is bound by HBM bytes ("AirLLM corre un modelo 70B...", "Por qué es
// lento": time ~ bytes moved / bandwidth).  The kernels therefore stream the
// packed codes with coalesced vector loads, never write dequantized weights
// anywhere, and keep the per-weight ALU work small:
//
// Weight streams are read with nontemporal buffer loads (see common.hpp).
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
//  * 2 <= B <= 16 (MFMA): a wave owns RT 16-row tiles; each lane decodes
//    one unit per tile and K-step to fp32 w_hat = s*q + o (one v_fma_mix_f32
//    per weight from an fp16-subnormal decode), splits it into bf16 hi + lo
//    and feeds two v_mfma_f32_16x16x32_bf16 with the activations (bf16) as
//    the 16-column operand, fp32 accumulation.
#pragma once
#include "codebook.hpp"
#include "common.hpp"
#include "launch.hpp"


// Tile parameters of the B = 1 kernel.  UI = units per lane held in
// registers (a K-slice covers 2048*UI inputs), RPW = rows per pipeline
// stage, target waves per launch.  Measured on MI355X (repeated, interleaved
// runs over the Llama-70B layer shapes): bf16 activations run best with
// UI = 4, one row per stage and 1024 waves (one per SIMD, deep per-wave
// streams), except 3-bit codes (two rows per stage) and 2-bit codes (2048
// waves); fp32 activations (two bf16 halves per pair) use UI = 2, two rows
// per stage, 2048 waves.  QG_B1_UI / QG_B1_RPW / QG_B1_WAVES force one
// choice.
#ifndef QG_B1_UI
#define QG_B1_UI 0
#endif
#ifndef QG_B1_RPW
#define QG_B1_RPW 0       // 0 = by width (see above)
#endif
#ifndef QG_B1_WAVES
#define QG_B1_WAVES 0
#endif

namespace qg {

template <bool C, typename A, typename B> struct Pick { using T = A; };
template <typename A, typename B> struct Pick<false, A, B> { using T = B; };
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// ------------------------------------------------------------------ B = 1
// OUT: outlier side columns (fp16 side[N][n_out] at input channels oidx[],
// n_out <= 64): lane j < n_out of K-slice 0 adds side[row][j] * x[oidx[j]]
// to its share of the row before the wave reduction.
// MULTI: up to four matrices with the same K, width and group size, sharing
// x, in one launch (a layer's q/k/v or gate/up): launch row g belongs to
// matrix m with segs.start[m] <= g < segs.start[m + 1] (unused starts are
// INT_MAX) and is its row g - segs.start[m]; every row is wave-uniform, so
// the matrix's buffer resources and output are picked with scalar selects.
// CB: codes read through per-group books (decode_unit_cb); the dictionary
// is staged in LDS and each unit's book id is loaded with its meta word.
// Every code lands at mantissa bit 0, so there is a single landing class and
// the group scale takes the level grid's 2^(b-7).
template <int BITS, int G, bool XF32, int UI, int RPW, bool OUT, bool MULTI, bool CB = false>
__global__ __launch_bounds__(512) void gemv_b1_kernel(
    const uint32_t* __restrict__ codes, const uint32_t* __restrict__ meta, int N, int K,
    const void* __restrict__ xin, void* __restrict__ yout, int y_bf16, int S, int RS, int USL,
    int TMAX, const uint16_t* __restrict__ side, const int32_t* __restrict__ oidx, int n_out,
    MultiSegs segs, Books bk) {
  static_assert(!(CB && (OUT || MULTI)), "codebooks come without outlier columns or grouping");
  extern __shared__ float part[];
  __shared__ __align__(16) uint32_t dict[CB ? 64 : 1];
  if constexpr (CB) {
    for (int t = threadIdx.x; t < (bk.n << BITS); t += blockDim.x)
      reinterpret_cast<uint8_t*>(dict)[t] = bk.dict[t];
    __syncthreads();
  }
  constexpr int XS = XF32 ? 2 : 1;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
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
  uint32_t ka[RPW][UI], kb[RPW][UI];         // book id of each unit (CB)
  uint32_t sva[RPW], svb[RPW];               // side value of each row (OUT)
  // Weight loads go through buffer resources (row offset in soffset, the
  // lane's unit offset in voffset).  The hardware range check covers the
  // voffset only, so every load is kept inside its buffer by construction:
  // a row past N (the tail of the last stage) is loaded as row N - 1 and
  // never stored, and a lane without a unit (unit index past K/32) loads
  // its row's first unit, which meets zero activation pairs.  No branches
  // around loads, so the next stage stays in flight while the current one
  // is decoded.
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(codes, (uint32_t)((size_t)N * U * BITS * 4));
  const __amdgpu_buffer_rsrc_t mrs = make_rsrc(meta, (uint32_t)((size_t)N * GN * 4));
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(bk.ids, CB ? (uint32_t)((size_t)N * GN) : 0u);
  __amdgpu_buffer_rsrc_t mcrs[4], mmrs[4];
  if constexpr (MULTI) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t rows = segs.nrows[i];
      mcrs[i] = make_rsrc(segs.codes[i], (uint32_t)((size_t)rows * U * BITS * 4));
      mmrs[i] = make_rsrc(segs.meta[i], (uint32_t)((size_t)rows * GN * 4));
    }
  }
  auto seg_of = [&](uint32_t row) -> int {   // wave-uniform
    return (row >= (uint32_t)segs.start[1]) + (row >= (uint32_t)segs.start[2]) + (row >= (uint32_t)segs.start[3]);
  };
  auto pick = [](int i, const __amdgpu_buffer_rsrc_t (&a)[4]) {
    return i == 0 ? a[0] : (i == 1 ? a[1] : (i == 2 ? a[2] : a[3]));
  };
  // the output element of launch row `row`
  auto store = [&](int row, float v) {
    void* yb = yout;
    int lr = row;
    if constexpr (MULTI) {
      const int mi = seg_of((uint32_t)row);
      lr = row - segs.start[mi];
      yb = mi == 0 ? segs.y[0] : (mi == 1 ? segs.y[1] : (mi == 2 ? segs.y[2] : segs.y[3]));
    }
    if (y_bf16) static_cast<uint16_t*>(yb)[lr] = (uint16_t)f32_to_bf16_rne(v);
    else static_cast<float*>(yb)[lr] = v;
  };
  uint32_t cvoff[UI], mvoff[UI];
#pragma unroll
  for (int it = 0; it < UI; ++it) {
    const int u0 = sl * USL + it * 64 + lane;
    const int u = u0 < U ? u0 : 0;
    cvoff[it] = (uint32_t)u * (BITS * 4);
    mvoff[it] = (uint32_t)((u * 32) / G) * 4;
  }
  const uint32_t crow = (uint32_t)U * BITS * 4, mrow = (uint32_t)GN * 4;
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(side, OUT ? (uint32_t)((size_t)N * n_out * 2) : 0u);
  const uint32_t svoff = (OUT && sl == 0 && lane < n_out) ? (uint32_t)lane * 2u : 0xFFFFFF00u;
  auto load = [&](uint32_t (&w)[RPW][UI][BITS], uint32_t (&m)[RPW][UI], uint32_t (&sv)[RPW],
                  uint32_t (&kk)[RPW][UI], int row0) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      // wave-uniform; rows past N load row N - 1 (never stored)
      const uint32_t row = (uint32_t)min(row0 + r * nstreams, N - 1);
      if constexpr (MULTI) {
        const int mi = seg_of(row);
        const uint32_t lr = row - (uint32_t)segs.start[mi];
        const __amdgpu_buffer_rsrc_t c = pick(mi, mcrs), mm = pick(mi, mmrs);
#pragma unroll
        for (int it = 0; it < UI; ++it) {
          buf_load_unit<BITS>(c, cvoff[it], lr * crow, w[r][it]);
          m[r][it] = buf_load_u32(mm, mvoff[it], lr * mrow);
        }
      } else {
#pragma unroll
        for (int it = 0; it < UI; ++it) {
          buf_load_unit<BITS>(crs, cvoff[it], row * crow, w[r][it]);
          m[r][it] = buf_load_u32(mrs, mvoff[it], row * mrow);
          if constexpr (CB) kk[r][it] = __builtin_amdgcn_raw_buffer_load_b8(krs, mvoff[it] >> 2, row * (uint32_t)GN, kNT);
        }
      }
      if constexpr (OUT)
        sv[r] = __builtin_amdgcn_raw_buffer_load_b16(srs, svoff, row * (uint32_t)n_out * 2u, 0);
    }
  };
  // activations first (in-order vmcnt: waiting for them must not wait for
  // the weight stream), then the first weight stage, then the prep.  With
  // outlier columns the channel index comes before everything else, so its
  // wait covers nothing but itself, and the dependent activation load is
  // issued before the weight stream.
  int kout = 0;
  if constexpr (OUT) kout = oidx[lane < n_out ? lane : n_out - 1];   // branch-free (n_out >= 1)
  constexpr int XW = XF32 ? 8 : 4;   // 16-byte loads per unit of activations
  u32x4_t xraw[UI][XW];
#pragma unroll
  for (int it = 0; it < UI; ++it) {
    const int u = uidx[it] >= 0 ? uidx[it] : 0;
    const u32x4_t* src = XF32 ? reinterpret_cast<const u32x4_t*>(static_cast<const float*>(xin) + (size_t)u * 32)
                              : reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(xin) + (size_t)u * 32);
#pragma unroll
    for (int i = 0; i < XW; ++i) xraw[it][i] = src[i];
  }
  const int step = RPW * nstreams;
  const int nst = stream < N ? (N - stream + step - 1) / step : 0;   // stages of this stream
  if (nst > 0) load(wa, ma, sva, ka, stream);
  // activation of this lane's outlier channel (OUT, K-slice 0; 0 elsewhere),
  // requested after the first weight stage: its wait is for the index only
  float xo = 0.f;
  if constexpr (OUT) {
    __builtin_amdgcn_sched_barrier(0);
    xo = XF32 ? static_cast<const float*>(xin)[kout] : bf16_bits_to_f32(static_cast<const uint16_t*>(xin)[kout]);
    if (!(sl == 0 && lane < n_out)) xo = 0.f;
  }

  // Activation prep.  Pair k of a unit holds x[ca] (low bf16) and x[cb]
  // (high bf16), unscaled; codes that land on mantissa bit p are summed in
  // their own accumulator and rescaled by 2^-p once per unit, so the pairs
  // are plain byte permutes of the raw bf16 words.  Per class the
  // accumulator starts at -128 * (sum of its x), which cancels the 128 bias.
  // fp32 activations are split into bf16 hi + lo pairs (two dot2 per pair).
  using UN = Unit<BITS>;
  constexpr int NC = CB ? 1 : UN::NCLS;
  constexpr uint32_t kOnes = 0x3F803F80u;   // bf16 (1, 1)
  uint32_t xp[UI][16 * XS];
  float negC[UI][NC], xsum[UI];
#pragma unroll
  for (int it = 0; it < UI; ++it) {
    const bool v = uidx[it] >= 0;
    float cs[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) cs[c] = 0.f;
    if constexpr (!XF32) {
      uint32_t xr[16];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) xr[4 * i + j] = v ? xraw[it][i][j] : 0u;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const PairInfo pi = UN::pair(k);
        const uint32_t lo = (pi.ca & 1) ? (xr[pi.ca >> 1] >> 16) : (xr[pi.ca >> 1] & 0xFFFFu);
        const uint32_t hi = (pi.cb & 1) ? (xr[pi.cb >> 1] & 0xFFFF0000u) : (xr[pi.cb >> 1] << 16);
        xp[it][k] = lo | hi;
        const int c = CB ? 0 : UN::cls_of_p(pi.p);
        cs[c] = dot2_bf16(xp[it][k], kOnes, cs[c]);
      }
    } else {
      float xv[32];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) xv[4 * i + j] = v ? __uint_as_float(xraw[it][i][j]) : 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const PairInfo pi = UN::pair(k);
        const float a = xv[pi.ca], b = xv[pi.cb];
        const uint32_t ah = f32_to_bf16_rne(a), bh = f32_to_bf16_rne(b);
        const uint32_t al = f32_to_bf16_rne(a - bf16_bits_to_f32(ah));
        const uint32_t bl = f32_to_bf16_rne(b - bf16_bits_to_f32(bh));
        xp[it][2 * k] = ah | (bh << 16);
        xp[it][2 * k + 1] = al | (bl << 16);
        const int c = CB ? 0 : UN::cls_of_p(pi.p);
        cs[c] = dot2_bf16(xp[it][2 * k], kOnes, cs[c]);
        cs[c] = dot2_bf16(xp[it][2 * k + 1], kOnes, cs[c]);
      }
    }
    float xs = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      negC[it][c] = -128.0f * cs[c];
      xs += cs[c];
    }
    xsum[it] = xs;
  }

  const uint32_t bias = opaque_bias();
  CbConst kc{};
  if constexpr (CB) kc = cb_consts();
  auto compute = [&](const uint32_t (&w)[RPW][UI][BITS], const uint32_t (&m)[RPW][UI], const uint32_t (&sv)[RPW],
                     const uint32_t (&kk)[RPW][UI], int row0, int m0) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      float acc_row = 0.f;
#pragma unroll
      for (int it = 0; it < UI; ++it) {
        uint32_t pr[16];
        if constexpr (CB) {
          uint32_t T[4] = {0u, 0u, 0u, 0u};
          const uint32_t* tp = dict + ((kk[r][it] & 15u) << BITS) / 4;   // ids < 16 (packer)
          if constexpr (BITS == 4) {
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(tp);
            T[0] = v[0]; T[1] = v[1]; T[2] = v[2]; T[3] = v[3];
          } else {
#pragma unroll
            for (int i = 0; i < (1 << BITS) / 4; ++i) T[i] = tp[i];
          }
          decode_unit_cb<BITS>(w[r][it], T, pr, kc);
        } else {
          decode_unit<BITS>(w[r][it], pr, bias);
        }
        constexpr int NCH = NC > 1 ? NC : 2;   // independent dot2 chains
        float a[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) a[c] = c < NC ? negC[it][c] : 0.f;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int c = NC > 1 ? UN::cls_of_p(UN::pair(k).p) : (k & 1);
          a[c] = dot2_bf16(pr[k], xp[it][k * XS], a[c]);
          if constexpr (XF32) a[c] = dot2_bf16(pr[k], xp[it][k * XS + 1], a[c]);
        }
        float sq;
        if constexpr (CB) sq = (a[0] + a[1]) * (1.0f / (float)(1 << (7 - BITS)));
        else if constexpr (BITS == 2) sq = a[0] + 0.25f * a[1] + 0.0625f * a[2];
        else if constexpr (BITS == 3) sq = a[0] + 0.125f * a[1];
        else sq = a[0] + a[1];
        const float s = f16_bits_to_f32(m[r][it] & 0xFFFFu);
        const float o = f16_bits_to_f32(m[r][it] >> 16);
        acc_row = __builtin_fmaf(s, sq, __builtin_fmaf(o, xsum[it], acc_row));
      }
      // the side value is the stage's last load: used last, so the units
      // above are decoded while it is still in flight
      if constexpr (OUT) acc_row = __builtin_fmaf(f16_bits_to_f32(sv[r] & 0xFFFFu), xo, acc_row);
      const float total = wave_sum(acc_row);
      const int row = row0 + r * nstreams;
      if (row < N && lane == 0) {
        if (S == 1) {
          store(row, total);
        } else {
          part[((size_t)rs * TMAX + (m0 + r)) * S + sl] = total;
        }
      }
    }
  };

  // Stage st covers rows stream + (st*RPW + r)*nstreams.  Inside the loop
  // every load is unconditional, so the wait before decoding a stage covers
  // exactly that stage's loads and the next stage stays in flight.
  int st = 0;
  while (st + 2 < nst) {
    load(wb, mb, svb, kb, stream + (st + 1) * step);
    __builtin_amdgcn_sched_barrier(0);  // keep the stage's loads issued here
    compute(wa, ma, sva, ka, stream + st * step, st * RPW);
    load(wa, ma, sva, ka, stream + (st + 2) * step);
    __builtin_amdgcn_sched_barrier(0);  // keep the stage's loads issued here
    compute(wb, mb, svb, kb, stream + (st + 1) * step, (st + 1) * RPW);
    st += 2;
  }
  if (st + 1 < nst) {
    load(wb, mb, svb, kb, stream + (st + 1) * step);
    __builtin_amdgcn_sched_barrier(0);  // keep the stage's loads issued here
    compute(wa, ma, sva, ka, stream + st * step, st * RPW);
    compute(wb, mb, svb, kb, stream + (st + 1) * step, (st + 1) * RPW);
  } else if (st < nst) {
    compute(wa, ma, sva, ka, stream + st * step, st * RPW);
  }
  if (S > 1) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < RS * TMAX; idx += blockDim.x) {
      const int rs_ = idx / TMAX, m = idx % TMAX;
      const int row = blockIdx.x * RS + rs_ + m * nstreams;
      if (row < N) {
        float t = 0.f;
        for (int j = 0; j < S; ++j) t += part[(size_t)idx * S + j];
        store(row, t);
      }
    }
  }
}

// --------------------------------------------------------------- B = 2..16
// A workgroup owns RT 16-row tiles; its WPB waves split K (wave w takes unit
// quads w, w+WPB, ...), so the activation fragments a wave loads are reused
// by RT tiles.  Lane (r, kg) = (lane % 16, lane / 16) decodes unit 4*q + kg
// of row r of every tile; the 4 lane groups therefore cover 4 consecutive
// units (128 inputs) per MFMA quad, and the activation lane (b, kg) loads the
// matching 8-wide slices of x[b].  Dequantization: each code is decoded as
// the fp16 subnormal q*2^(p-24) (common.hpp, UnitH), and one v_fma_mix_f32
// per weight gives fl32(s*q + o); the MFMA takes it as bf16 hi + lo (two
// MFMAs, 2^-16 relative residual; SPLITW), or, for reductions of at least
// 512 inputs, rounded once to bf16 (one MFMA).  Partial sums of the WPB waves
// meet in LDS.
// PAIR (plain codes, one bf16 operand): a wave takes two quads (8 units) per
// step, and each weight load instruction reads those 8 units from 8 rows
// (lane (r, kg) of instruction h: row (r & 7) + 8h, unit kg + 4((r >> 3) ^ h))
// instead of 4 units from 16 rows, i.e. half as many cache lines per
// instruction, whole 128-byte lines for 4-bit codes.  The matrix-core layout
// is restored in registers: quad 0 is instruction 0's word for r < 8 and
// instruction 1's for r >= 8, quad 1 the other instruction's word 8 lanes
// away (a row rotation by 8, DPP).  Group words: g32 as the codes; g64 one
// load of the pair's 4 groups per row, spread by lane permutes.  The same
// products in the same order, so the results equal the one-quad form's.
// OUT: outlier side columns as in the B = 1 kernel, added to each output
// in the final reduction (the activations of the outlier channels are
// staged in LDS first).
// CB: codes read through per-group books; decode_unit_cb gives e[q] exactly
// as the fp16 subnormal e[q] 2^-24 and one v_fma_mix_f32 per weight gives
// fl32(s 2^(b-7) e[q] + o).
// MULTI: up to four matrices sharing K, width, group and x in one launch
// (a layer's q/k/v or gate/up): workgroup w belongs to matrix m with
// segs.start[m] <= w < segs.start[m + 1] (starts counted in workgroups,
// unused ones INT_MAX) and takes its tile w - segs.start[m]; the matrix's
// codes, group words, rows and output are picked with scalar selects.
template <int BITS, int G, int RT, int WPB, bool OUT, bool CB = false, bool SPLITW = true, bool PAIR = false,
          bool MULTI = false>
__global__ __launch_bounds__(64 * WPB) void gemv_mfma_kernel(
    const uint32_t* __restrict__ codes_in, const uint32_t* __restrict__ meta_in, int N_in, int K,
    const uint16_t* __restrict__ x, int B, void* __restrict__ yout_in, int y_bf16,
    const uint16_t* __restrict__ side, const int32_t* __restrict__ oidx, int n_out, Books bk, MultiSegs segs) {
  static_assert(!(CB && OUT), "codebooks come without outlier columns");
  static_assert(!(MULTI && (CB || OUT)), "grouped launches take plain codes");
  const uint32_t* codes = codes_in;
  const uint32_t* meta = meta_in;
  int N = N_in;
  void* yout = yout_in;
  int tile = blockIdx.x;
  if constexpr (MULTI) {
    const uint32_t w = blockIdx.x;
    const int mi = (w >= (uint32_t)segs.start[1]) + (w >= (uint32_t)segs.start[2]) + (w >= (uint32_t)segs.start[3]);
    codes = static_cast<const uint32_t*>(mi == 0 ? segs.codes[0] : (mi == 1 ? segs.codes[1] : (mi == 2 ? segs.codes[2] : segs.codes[3])));
    meta = static_cast<const uint32_t*>(mi == 0 ? segs.meta[0] : (mi == 1 ? segs.meta[1] : (mi == 2 ? segs.meta[2] : segs.meta[3])));
    yout = mi == 0 ? segs.y[0] : (mi == 1 ? segs.y[1] : (mi == 2 ? segs.y[2] : segs.y[3]));
    N = (int)(mi == 0 ? segs.nrows[0] : (mi == 1 ? segs.nrows[1] : (mi == 2 ? segs.nrows[2] : segs.nrows[3])));
    tile = (int)w - (mi == 0 ? segs.start[0] : (mi == 1 ? segs.start[1] : (mi == 2 ? segs.start[2] : segs.start[3])));
  }
  static_assert(!(PAIR && (CB || SPLITW)), "pair loads: plain codes, one bf16 weight operand");
  __shared__ float red[WPB][RT * 4][64];
  __shared__ float xo[OUT ? 16 * 64 : 1];
  __shared__ __align__(16) uint32_t dict[CB ? 64 : 1];
  if constexpr (CB) {
    for (int t = threadIdx.x; t < (bk.n << BITS); t += 64 * WPB)
      reinterpret_cast<uint8_t*>(dict)[t] = bk.dict[t];
  }
  if constexpr (OUT) {
    for (int t = threadIdx.x; t < B * n_out; t += 64 * WPB)
      xo[t] = bf16_bits_to_f32(x[(size_t)(t / n_out) * K + oidx[t % n_out]]);
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int row_base = tile * (16 * RT);
  const int r = lane & 15, kg = lane >> 4;
  const int U = K >> 5, GN = K / G;
  const int bcol = lane & 15;
  f32x4_t acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // one quad per step, or (PAIR) two: codes as loaded (instruction h of tile
  // t in w[t][h]) and meta as loaded (G = 32: as the codes; G = 64: one word)
  struct Buf1 { u32x4_t xb[4]; uint32_t w[RT][BITS]; uint32_t m[RT]; uint32_t k[RT]; };
  struct Buf2 { u32x4_t xb[2][4]; uint32_t w[RT][2][BITS]; uint32_t m[RT][2]; };
  using Buf = typename Pick<PAIR, Buf2, Buf1>::T;
  const bool lo8 = r < 8;
  // Branch-free loads through buffer resources.  Activations: a lane past B
  // reads a valid activation row (its column is never stored), a unit past K
  // gets an out-of-range offset and reads 0.  Weights: rows past N read 0
  // and are never stored; a unit past K meets a zero activation.
  const int bc = bcol < B ? bcol : B - 1;
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, (uint32_t)((size_t)B * K * 2));
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(codes, (uint32_t)((size_t)N * U * BITS * 4));
  const __amdgpu_buffer_rsrc_t mrs = make_rsrc(meta, (uint32_t)((size_t)N * GN * 4));
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(bk.ids, CB ? (uint32_t)((size_t)N * GN) : 0u);
  auto load = [&](Buf& b, int qi, bool even) {
    if constexpr (PAIR) {
      // qi is a pair of quads: units 8 qi .. 8 qi + 7.  Load instruction h
      // of tile t: lane (r, kg) takes row (r & 7) + 8 h of the tile and unit
      // 8 qi + kg + 4 ((r >> 3) ^ h), so each instruction reads 8 units in a
      // row from 8 rows (whole 128-byte lines for 4-bit codes).
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int u0 = 8 * qi + 4 * q + kg;
        const uint32_t xo = u0 < U ? (uint32_t)((bc * K + u0 * 32) * 2) : 0xFFFFFF00u;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const auto v = __builtin_amdgcn_raw_buffer_load_b128(xrs, xo + 16 * t, 0, 0);
          b.xb[q][t] = u32x4_t{v[0], v[1], v[2], v[3]};
        }
      }
#pragma unroll
      for (int t = 0; t < RT; ++t) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t row = (uint32_t)(row_base + 16 * t + (r & 7) + 8 * h);
          const uint32_t u = (uint32_t)(8 * qi + kg + 4 * ((r >> 3) ^ h));
          buf_load_unit<BITS, 0>(crs, (row * (uint32_t)U + u) * (BITS * 4), 0u, b.w[t][h]);
          if constexpr (G == 32) b.m[t][h] = __builtin_amdgcn_raw_buffer_load_b32(mrs, (row * (uint32_t)GN + u) * 4, 0u, 0);
        }
        if constexpr (G == 64) {
          // even steps load the group words of both pairs of their block (8
          // groups, 32 bytes of row r): lane (r, kg) takes groups
          // 4 qi + 2 kg and 4 qi + 2 kg + 1
          if (even) {
            const uint32_t row = (uint32_t)(row_base + 16 * t + r);
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(
                mrs, (row * (uint32_t)GN + (uint32_t)(4 * qi + 2 * kg)) * 4, 0u, 0);
            b.m[t][0] = v[0];
            b.m[t][1] = v[1];
          }
        }
      }
    } else {
    const int u0 = 4 * qi + kg;
    const uint32_t xo = u0 < U ? (uint32_t)((bc * K + u0 * 32) * 2) : 0xFFFFFF00u;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(xrs, xo + 16 * t, 0, 0);
      b.xb[t] = u32x4_t{v[0], v[1], v[2], v[3]};
    }
    // Default cache policy: the other half of each 128-byte code line and the
    // group constants (one dword serves up to 16 K-steps) are read again
    // shortly after, by this or a neighbouring wave.
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const uint32_t row = (uint32_t)(row_base + 16 * t + r);
      buf_load_unit<BITS, 0>(crs, (row * (uint32_t)U + (uint32_t)u0) * (BITS * 4), 0u, b.w[t]);
      b.m[t] = __builtin_amdgcn_raw_buffer_load_b32(mrs, (row * (uint32_t)GN + (uint32_t)((u0 * 32) / G)) * 4, 0u, 0);
      if constexpr (CB)
        b.k[t] = __builtin_amdgcn_raw_buffer_load_b8(krs, row * (uint32_t)GN + (uint32_t)((u0 * 32) / G), 0u, 0);
    }
    }
  };
  using UN = UnitH<BITS>;
  CbConst kc{};
  if constexpr (CB) kc = cb_consts();
  // one quad: codes w, group words m, book ids kk (CB) of the RT tiles and
  // the activation fragments xb
  auto quad = [&](const uint32_t (&bw)[RT][BITS], const uint32_t (&bm)[RT], const uint32_t (&bk_)[RT],
                  const u32x4_t (&bxb)[4]) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      uint32_t pr[16];
      const float s = f16_bits_to_f32(bm[t] & 0xFFFFu), o = f16_bits_to_f32(bm[t] >> 16);
      float wv[32];
      if constexpr (CB) {
        uint32_t T[4] = {0u, 0u, 0u, 0u};
        const uint32_t* tp = dict + ((bk_[t] & 15u) << BITS) / 4;   // ids < 16 (packer)
#pragma unroll
        for (int i = 0; i < (1 << BITS) / 4; ++i) T[i] = tp[i];
        // entries as fp16 subnormals e * 2^-24: one v_fma_mix_f32 per weight
        // gives fl32(s 2^(b-7) e + o), as for plain codes
        decode_unit_cb<BITS, true>(bw[t], T, pr, kc);
        const float sc = s * (float)(1 << (24 - (7 - BITS)));
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const PairInfo pi = UN::pair(k);
          wv[pi.ca] = __builtin_fmaf(f16_lo(pr[k]), sc, o);
          wv[pi.cb] = __builtin_fmaf(f16_hi(pr[k]), sc, o);
        }
      } else {
        decode_unit_h<BITS>(bw[t], pr);
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
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // SPLITW: w_hat = hi + lo, both bf16 (2^-16 relative residual), two
        // MFMAs; else w_hat rounded once to bf16 (nearest even), one MFMA
        u32x4_t hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float w0 = wv[8 * j + 2 * e], w1 = wv[8 * j + 2 * e + 1];
          hi[e] = cvt_pk_bf16(w0, w1);
          if constexpr (SPLITW) lo[e] = cvt_pk_bf16(w0 - bf16_lo_to_f32(hi[e]), w1 - bf16_hi_to_f32(hi[e]));
        }
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, hi),
                                                         __builtin_bit_cast(bf16x8_t, bxb[j]), acc[t], 0, 0, 0);
        if constexpr (SPLITW)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, lo),
                                                           __builtin_bit_cast(bf16x8_t, bxb[j]), acc[t], 0, 0, 0);
      }
    }
  };

  // s: the step's place in its pair block (G = 64 group words in mc)
  auto compute = [&](const Buf& b, int s_, const uint32_t (&mc)[RT][2]) {
    if constexpr (PAIR) {
      // to the matrix-core layout: quad 0 of the pair (lane (r, kg): unit kg
      // of row r) is instruction 0's word for r < 8 and instruction 1's for
      // r >= 8; quad 1 (unit 4 + kg) sits 8 lanes away in the other
      // instruction, brought over by a rotation by 8 inside each 16-lane row
      uint32_t w0[RT][BITS], w1[RT][BITS], m0[RT], m1[RT], k0[RT];
#pragma unroll
      for (int t = 0; t < RT; ++t) {
#pragma unroll
        for (int i = 0; i < BITS; ++i) {
          const uint32_t a = b.w[t][0][i], c = b.w[t][1][i];
          w0[t][i] = lo8 ? a : c;
          w1[t][i] = dpp_u32<0x128>(lo8 ? c : a);   // row_ror:8
        }
        if constexpr (G == 32) {
          m0[t] = lo8 ? b.m[t][0] : b.m[t][1];
          m1[t] = dpp_u32<0x128>(lo8 ? b.m[t][1] : b.m[t][0]);
        } else {
          // quad q of this step needs group 4 s + 2 q + kg / 2 of the block,
          // word kg / 2 of lane (r, 2 s + q)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int src = (r + 16 * (2 * s_ + q)) * 4;
            const uint32_t d0 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)mc[t][0]);
            const uint32_t d1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)mc[t][1]);
            (q ? m1 : m0)[t] = (kg >> 1) ? d1 : d0;
          }
        }
        k0[t] = 0u;
      }
      quad(w0, m0, k0, b.xb[0]);
      quad(w1, m1, k0, b.xb[1]);
    } else {
      quad(b.w, b.m, b.k, b.xb);
    }
  };

  // Steps of a wave: quads w, w + WPB, ...; with PAIR, pairs w, w + WPB, ...,
  // except for g64 groups (BLK), where wave w takes blocks of two adjacent
  // pairs, w, w + WPB, ... (step it is pair 2 (w + WPB (it / 2)) + it % 2), so
  // that b0 holds the even steps, which also load their block's group words,
  // and b1 the odd ones; an odd step past the last pair loads zero
  // activations.  (Blocks for g32 codes measured slower: the waves of a
  // workgroup then read pairs 0, 2, 4, 6 together rather than 0, 1, 2, 3.)
  constexpr bool BLK = PAIR && G == 64;
  const int nq = (U + 3) >> 2, npair = (nq + 1) >> 1, nblk = (npair + 1) >> 1;
  const int nunit = PAIR ? npair : nq;
  const int nit = BLK ? (wave < nblk ? 2 * ((nblk - wave + WPB - 1) / WPB) : 0)
                      : (wave < nunit ? (nunit - wave + WPB - 1) / WPB : 0);   // steps of this wave
  auto idx = [&](int st) { return BLK ? 2 * (wave + WPB * (st >> 1)) + (st & 1) : wave + WPB * st; };
  Buf b0, b1;
  uint32_t mc[RT][2];
#pragma unroll
  for (int t = 0; t < RT; ++t) mc[t][0] = mc[t][1] = 0u;
  auto keep = [&](const Buf& b) {   // the block's group words, for its odd step
    if constexpr (PAIR && G == 64)
#pragma unroll
      for (int t = 0; t < RT; ++t) { mc[t][0] = b.m[t][0]; mc[t][1] = b.m[t][1]; }
  };
  if (nit > 0) load(b0, idx(0), true);
  if constexpr (CB) __syncthreads();   // dictionary staged before the first decode
  int it = 0;
  while (it + 2 < nit) {
    load(b1, idx(it + 1), false);
    __builtin_amdgcn_sched_barrier(0);  // keep the stage's loads issued here
    keep(b0);
    compute(b0, 0, mc);
    load(b0, idx(it + 2), true);
    __builtin_amdgcn_sched_barrier(0);  // keep the stage's loads issued here
    compute(b1, 1, mc);
    it += 2;
  }
  if (it + 1 < nit) {
    load(b1, idx(it + 1), false);
    __builtin_amdgcn_sched_barrier(0);  // keep the stage's loads issued here
    keep(b0);
    compute(b0, 0, mc);
    compute(b1, 1, mc);
  } else if (it < nit) {
    keep(b0);
    compute(b0, 0, mc);
  }
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][t * 4 + i][lane] = acc[t][i];
  __syncthreads();
  // lane holds D[4*kg + i][bcol] of each tile: row 16t + 4kg + i, batch bcol
  for (int v = threadIdx.x; v < RT * 4 * 64; v += 64 * WPB) {
    const int ti = v / 64, ln = v % 64;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < WPB; ++w) sum += red[w][ti][ln];
    const int t = ti / 4, i = ti % 4;
    const int b = ln & 15, row = row_base + 16 * t + 4 * (ln >> 4) + i;
    if (b < B && row < N) {
      if constexpr (OUT)
        for (int j = 0; j < n_out; ++j)
          sum = __builtin_fmaf(f16_bits_to_f32(side[(size_t)row * n_out + j]), xo[b * n_out + j], sum);
      if (y_bf16) static_cast<uint16_t*>(yout)[(size_t)b * N + row] = (uint16_t)f32_to_bf16_rne(sum);
      else static_cast<float*>(yout)[(size_t)b * N + row] = sum;
    }
  }
}

// --------------------------------------------------------------- launchers
struct Side { const uint16_t* vals; const int32_t* idx; int n; };   // outlier columns (n = 0: none)

// CB: launch the codebook variant with the books in bk (sd and ms unused).
template <int BITS, int G, bool XF32, int UI, int RPW, bool CB = false>
static hipError_t gemv_b1_t(const uint32_t* codes, const uint32_t* meta, int64_t N, int64_t K,
                            const void* x, void* y, int y_bf16, hipStream_t s, int64_t waves, Side sd,
                            const MultiSegs* ms = nullptr, Books bk = Books{nullptr, nullptr, 0}) {
  const int64_t kTargetWaves = QG_B1_WAVES ? QG_B1_WAVES : waves;
  const int U = (int)(K / 32);
  int S = (U + 64 * UI - 1) / (64 * UI);
  if (S > 8) return hipErrorInvalidValue;
  // short matrices: split K further so the grid still has ~8 waves per CU
  while (S < 4 && N * S < kTargetWaves && (U + 2 * S - 1) / (2 * S) >= 64) S *= 2;
  const int RS = S <= 4 ? 4 / S : 1;   // 256 threads, or 64*S (<= 512) for long rows
  const int USL = (U + S - 1) / S;
  const int threads = 64 * S * RS;
  // rows per stream: a whole number of RPW-row stages
  const int64_t streams_target = kTargetWaves / S;
  const int64_t stages = (N + RPW * streams_target - 1) / (RPW * streams_target);
  const int64_t rows_per_stream = RPW * stages;
  int64_t blocks = ((N + rows_per_stream - 1) / rows_per_stream + RS - 1) / RS;
  if (blocks < 1) blocks = 1;
  const int64_t nstreams = blocks * RS;
  const int TMAX = (int)((N + nstreams - 1) / nstreams);
  const size_t lds = S > 1 ? (size_t)RS * TMAX * S * sizeof(float) : 0;
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  MultiSegs none{};
  if constexpr (CB)
    hipLaunchKernelGGL((gemv_b1_kernel<BITS, G, XF32, UI, RPW, false, false, true>), dim3((unsigned)blocks),
                       dim3(threads), lds, s, codes, meta, (int)N, (int)K, x, y, y_bf16, S, RS, USL,
                       TMAX, nullptr, nullptr, 0, none, bk);
  else if (ms)
    hipLaunchKernelGGL((gemv_b1_kernel<BITS, G, XF32, UI, RPW, false, true>), dim3((unsigned)blocks),
                       dim3(threads), lds, s, codes, meta, (int)N, (int)K, x, y, y_bf16, S, RS, USL,
                       TMAX, nullptr, nullptr, 0, *ms, bk);
  else if (sd.n > 0)
    hipLaunchKernelGGL((gemv_b1_kernel<BITS, G, XF32, UI, RPW, true, false>), dim3((unsigned)blocks),
                       dim3(threads), lds, s, codes, meta, (int)N, (int)K, x, y, y_bf16, S, RS, USL,
                       TMAX, sd.vals, sd.idx, sd.n, none, bk);
  else
    hipLaunchKernelGGL((gemv_b1_kernel<BITS, G, XF32, UI, RPW, false, false>), dim3((unsigned)blocks),
                       dim3(threads), lds, s, codes, meta, (int)N, (int)K, x, y, y_bf16, S, RS, USL,
                       TMAX, nullptr, nullptr, 0, none, bk);
  return hipGetLastError();
}

#ifndef QG_MB_PAIR
#define QG_MB_PAIR 1      // plain codes, K >= 512: two quads per step, 8-row load instructions
#endif
// Reductions of at least this many inputs take the weights as one bf16
// operand; shorter ones as bf16 hi + lo (the error argument is given with
// the tile choice below).
constexpr int64_t kGemvSplitBelowK = 512;

template <int BITS, int G, int RT, int WPB, bool CB = false>
static hipError_t gemv_mfma_launch(const uint32_t* codes, const uint32_t* meta, int64_t N, int64_t K,
                                   const uint16_t* x, int64_t B, void* y, int y_bf16, hipStream_t s, Side sd,
                                   Books bk = Books{nullptr, nullptr, 0}) {
  const int64_t tiles = (N + 16 * RT - 1) / (16 * RT);
  const dim3 grid((unsigned)tiles), block(64 * WPB);
#define MF(O, C, S, SV, SI, SN)                                                                               \
  hipLaunchKernelGGL((gemv_mfma_kernel<BITS, G, RT, WPB, O, C, S>), grid, block, 0, s, codes, meta, (int)N, (int)K, \
                     x, (int)B, y, y_bf16, SV, SI, SN, bk, MultiSegs{})
#define MFP(O, SV, SI, SN)                                                                                     \
  hipLaunchKernelGGL((gemv_mfma_kernel<BITS, G, RT, WPB, O, false, false, true>), grid, block, 0, s, codes, meta,   \
                     (int)N, (int)K, x, (int)B, y, y_bf16, SV, SI, SN, bk, MultiSegs{})
  const bool split = K < kGemvSplitBelowK;
  if constexpr (CB) {
    if (split) MF(false, true, true, nullptr, nullptr, 0);
    else MF(false, true, false, nullptr, nullptr, 0);
  } else if (sd.n > 0) {
    if (split) MF(true, false, true, sd.vals, sd.idx, sd.n);
    else if (QG_MB_PAIR) MFP(true, sd.vals, sd.idx, sd.n);
    else MF(true, false, false, sd.vals, sd.idx, sd.n);
  } else {
    if (split) MF(false, false, true, nullptr, nullptr, 0);
    else if (QG_MB_PAIR) MFP(false, nullptr, nullptr, 0);
    else MF(false, false, false, nullptr, nullptr, 0);
  }
#undef MF
#undef MFP
  return hipGetLastError();
}

// Tile choice, measured on MI355X at B = 2..16: 4 waves split K, and the
// row tiles per workgroup (reuse of the activation fragments) are picked
// from {1, 2, 4, 7} so that the workgroups spread evenly over the 256 CUs
// (mfma_row_tiles).  At N = 28672 that is 7 tiles
// (256 workgroups of 112 rows) instead of 4 (448 workgroups, so 192 CUs
// held two and 64 one): 8192 x 28672 4-bit g64 at B = 16 41.9 -> 36.7 us
// (with outlier columns 44.0 -> 39.6, codebooks 69.4 -> 62.8), 2-bit g32 at
// B = 8 36.2 -> 31.9 us; 3-bit g32 at B = 8 measured 40.1 -> 41.4 us, so
// 3-bit codes keep at most 4 tiles.  QG_MB_RT / QG_MB_WPB force one choice.
// Weight operand: rounding w_hat once to bf16 (unit roundoff 2^-8) moves a
// product by at most 2^-8 sum |w_hat||x| in the worst case, and by about
// 2^-8 / sqrt(3K) of it when the rounding errors are independent (below
// 1e-4 of the bound at K >= 512); for K < 512 the hi + lo split keeps every
// shape far inside the 2e-3 budget.
#ifndef QG_MB_RT
#define QG_MB_RT 0
#endif
#ifndef QG_MB_WPB
#define QG_MB_WPB 0
#endif
// Row tiles per workgroup of the B >= 2 kernel, among 1, 2, 4 and 7 (7 not
// for 3-bit codes): the least work on the busiest CU (256 CUs), counted as
// rounds of one workgroup per CU times (tiles + 1), the 1 standing for the
// activation loads a workgroup shares among its tiles; the larger tile on
// ties.
static inline int mfma_row_tiles(int64_t N, bool allow7) {
  constexpr int64_t kCUs = 256;
  int best = 1;
  int64_t best_cost = INT64_MAX;
  for (int rt : {1, 2, 4, 7}) {
    if (rt == 7 && !allow7) continue;
    const int64_t tiles = (N + 16 * rt - 1) / (16 * rt);
    const int64_t cost = (tiles + kCUs - 1) / kCUs * (rt + 1);
    if (cost <= best_cost) { best = rt; best_cost = cost; }
  }
  return best;
}

template <int BITS, int G, bool CB = false>
static hipError_t gemv_mfma_t(const uint32_t* codes, const uint32_t* meta, int64_t N, int64_t K,
                              const uint16_t* x, int64_t B, void* y, int y_bf16, hipStream_t s, Side sd,
                              Books bk = Books{nullptr, nullptr, 0}) {
#if QG_MB_RT && QG_MB_WPB
  return gemv_mfma_launch<BITS, G, QG_MB_RT, QG_MB_WPB, CB>(codes, meta, N, K, x, B, y, y_bf16, s, sd, bk);
#else
  constexpr bool kAllow7 = BITS != 3;
  const int rt = mfma_row_tiles(N, kAllow7), wpb = 4;
#define L(R, W) if (rt == R && wpb == W) return gemv_mfma_launch<BITS, G, R, W, CB>(codes, meta, N, K, x, B, y, y_bf16, s, sd, bk)
  if constexpr (kAllow7) L(7, 4);
  L(4, 4); L(2, 4); L(1, 4);
#undef L
  return hipErrorInvalidValue;
#endif
}

// Grouped launch for B >= 2: the matrices' tiles in one grid, the tile
// count chosen as for one matrix but over the matrices' tiles together.
template <int BITS, int G, int RT>
static hipError_t gemv_mfma_multi_launch(const MultiSegs& ms, int64_t K, const uint16_t* x, int64_t B, int y_bf16,
                                         hipStream_t s) {
  MultiSegs mt = ms;
  int64_t tiles = 0;
  for (int i = 0; i < 4; ++i) {
    if (i < ms.nseg) {
      mt.start[i] = (int)tiles;
      tiles += (ms.nrows[i] + 16 * RT - 1) / (16 * RT);
    } else {
      mt.start[i] = INT32_MAX;
    }
  }
  const dim3 grid((unsigned)tiles), block(64 * 4);
  const uint32_t* c0 = static_cast<const uint32_t*>(ms.codes[0]);
  const uint32_t* m0 = static_cast<const uint32_t*>(ms.meta[0]);
  const Books nob{nullptr, nullptr, 0};
  if (K < kGemvSplitBelowK)
    hipLaunchKernelGGL((gemv_mfma_kernel<BITS, G, RT, 4, false, false, true, false, true>), grid, block, 0, s, c0, m0,
                       (int)ms.nrows[0], (int)K, x, (int)B, ms.y[0], y_bf16, nullptr, nullptr, 0, nob, mt);
  else
    hipLaunchKernelGGL((gemv_mfma_kernel<BITS, G, RT, 4, false, false, false, true, true>), grid, block, 0, s, c0, m0,
                       (int)ms.nrows[0], (int)K, x, (int)B, ms.y[0], y_bf16, nullptr, nullptr, 0, nob, mt);
  return hipGetLastError();
}

template <int BITS, int G>
static hipError_t gemv_mfma_multi_t(const MultiSegs& ms, int64_t K, const uint16_t* x, int64_t B, int y_bf16,
                                    hipStream_t s) {
  constexpr bool kAllow7 = BITS != 3;
  constexpr int64_t kCUs = 256;
  int rt = 1;
  int64_t best = INT64_MAX;
  for (int r : {1, 2, 4, 7}) {
    if (r == 7 && !kAllow7) continue;
    int64_t tiles = 0;
    for (int i = 0; i < ms.nseg; ++i) tiles += (ms.nrows[i] + 16 * r - 1) / (16 * r);
    const int64_t cost = (tiles + kCUs - 1) / kCUs * (r + 1);
    if (cost <= best) { best = cost; rt = r; }
  }
  if constexpr (kAllow7)
    if (rt == 7) return gemv_mfma_multi_launch<BITS, G, 7>(ms, K, x, B, y_bf16, s);
  if (rt == 4) return gemv_mfma_multi_launch<BITS, G, 4>(ms, K, x, B, y_bf16, s);
  if (rt == 2) return gemv_mfma_multi_launch<BITS, G, 2>(ms, K, x, B, y_bf16, s);
  return gemv_mfma_multi_launch<BITS, G, 1>(ms, K, x, B, y_bf16, s);
}

}  // namespace qg
