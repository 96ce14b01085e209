// Binary low-rank GEMV, W ~ s1 (.) (U+-1 V+-1^T) (.) s2^T ("70B en 4GB de
// VRAM...", section 1, NanoQuant formulation), read right to left:
//   stage 1  t = V^T (s2 (.) x)       rows of VTbits, reduction over K
//   stage 2  y = s1 (.) (U t)         rows of Ubits,  reduction over r
// Both stages are one kernel: 16-row tiles of +-1 rows times a vector v on
// the matrix cores (v_mfma_f32_16x16x32_bf16), with
//   sum_k (2 b_k - 1) v_k = 2 * sum_k b_k v_k - sum_k v_k.
//
// A operand (the signs): bit j and bit 16+j of a 32-bit word form a pair;
// one masked OR into 0x4300 (bf16 128) turns it into the bf16x2
// 128 + b*2^p, p the mantissa bit the pair lands on (words pre-shifted by 7
// and 14 bring bits 7..15 down).  Exact in bf16.
// B operand (the vector): v is split into bf16 hi + lo (2^-16 relative
// residual), pre-scaled by 2^-p so every product b*2^p * v*2^-p is b*v, and
// laid out in a table in the order the A lanes hold their bits.  Column 0 of
// the 16 MFMA columns carries hi, column 1 lo (the others repeat them and
// are ignored).  Then D = sum_k (128 + b_k 2^p_k)(hi_k + lo_k) 2^-p_k
//                       = 128 C + sum_k b_k v~_k,  C = sum_k (hi_k + lo_k) 2^-p_k,
// and the row result is 2 (D - 128 C) - V with V = sum_k v~_k.
//
// Table layout (4 bytes per vector entry, 2 KB per 512-entry K-step): the
// 16-byte chunk ((s*16 + j)*2 + n)*4 + kg holds part n (0 hi, 1 lo) of the 8
// entries e = 2*e2 + h at k = 512 s + 32 (4 kg + e2) + 16 h + j.
//
// Stage 1 builds its table in LDS from x and s2, one chunk of 8192 entries at
// a time.  Its epilogue writes t already split and permuted into the stage-2
// table in the workspace, with per-workgroup partial sums of C and V, so a
// stage-2 workgroup only copies the table into LDS.
//
// Work split: a workgroup owns RT row tiles (16 RT rows) and NS waves that
// split the 512-bit K-steps.  Per table chunk a thread first issues its share
// of the table's loads (x and s2, or the stage-2 table: L2 hits), then all of
// its wave's sign words (HBM); loads return in issue order, so the table is
// built in LDS while the sign words are still on their way.  The NS partial
// sums meet in LDS.
#include "common.hpp"
#include "launch.hpp"
#include "qgemv.h"

#include <mutex>

namespace qg {

namespace {

constexpr int kTK = 8192;                 // vector entries per LDS table chunk
constexpr int kStepsPerChunk = kTK / 512; // 16 K-steps of 512 bits
constexpr int kMaxNS = 16;

// pair j of a word = bits (j, 16 + j); shift that brings it down, landing bit
__device__ __forceinline__ constexpr int bin_shift(int j) { return j < 7 ? 0 : (j < 14 ? 7 : 14); }
__device__ __forceinline__ constexpr int bin_p(int j) { return j - bin_shift(j); }
__device__ __forceinline__ int bin_p_rt(int j) { return j < 7 ? j : (j < 14 ? j - 7 : j - 14); }

// byte offset of entry k, part n, in a table
__device__ __forceinline__ uint32_t tab_off(int k, int n) {
  const int kl = k & 511;
  const int ent = ((((k >> 9) * 16 + (kl & 15)) * 2 + n) * 4) + ((kl >> 7) & 3);
  return (uint32_t)ent * 16u + (uint32_t)(((kl >> 5) & 3) * 2 + ((kl >> 4) & 1)) * 2u;
}

struct Stage2Out {         // where stage 1 leaves the stage-2 table
  uint16_t* tab;           // [B][steps2 * 2 KB / 2]
  float* part;             // [B][nparts][2] partial (C, V)
  int64_t tab_bstride;     // uint16 elements per batch row
  int64_t part_bstride;    // floats per batch row
};

// MODE 0: v = s2 * x (x bf16) -> stage-2 table
// MODE 1: v = s2 * x (x fp32) -> stage-2 table
// MODE 2: v from the stage-2 table -> y = s1 * dot (fp32 or bf16)
template <int MODE, int RT, int SPW, bool FULL>
__global__ __launch_bounds__(1024) void bin_mfma_kernel(
    const uint32_t* __restrict__ bits, int R, int Wn, int Lk, const void* __restrict__ vin,
    const uint16_t* __restrict__ vscale, const uint16_t* __restrict__ oscale,
    void* __restrict__ out, int y_bf16, int64_t in_bstride, int64_t out_bstride, int vec_ok,
    Stage2Out s2o, int nparts) {
  // SPW: max K-steps per wave and chunk (a power of two, SPW RT <= 8).
  // FULL: every chunk has exactly SPW steps per wave (so every slot and
  // table entry is in use), and in stage 1 the rows are 16-byte aligned and K
  // is a multiple of 512, so every group of 8 entries takes the fast path and
  // lies inside its chunk: no range tests, selects or element-wise path.
  static_assert(SPW * RT <= 8, "sign words held per wave");
  __shared__ u32x4_t tab[kStepsPerChunk * 16 * 2 * 4];   // 32 KB
  __shared__ float red[kMaxNS][RT * 16];
  __shared__ float sums[kMaxNS][2];
  __shared__ uint16_t junk[2];
  const int lane = threadIdx.x & 63;
  const int NS = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int b = blockIdx.y;
  const int row_base = blockIdx.x * 16 * RT;
  const int r16 = lane & 15, kg = lane >> 4;
  const int steps = (Wn + 15) >> 4;                 // 512-bit steps per row

  // Sign words through a buffer resource: rows past R and words past the
  // buffer read 0; words past Lk meet zero table entries.
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(bits, (uint32_t)((size_t)R * Wn * 4));
  uint32_t voff[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) voff[t] = ((uint32_t)(row_base + 16 * t + r16) * (uint32_t)Wn + 4u * kg) * 4u;

  f32x4_t acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float csum = 0.f, vsum = 0.f;                     // this thread's share of C and V
  const uint32_t bias = opaque_bias();
  float part_c = 0.f, part_v = 0.f;                 // stage 2: see below
  uint32_t s1_bits = 0;

  for (int c0 = 0; c0 < steps; c0 += kStepsPerChunk) {
    const int cs = min(kStepsPerChunk, steps - c0);
    // this wave's steps of the chunk: c0 + wave, c0 + wave + NS, ...
    const int my = wave < cs ? (cs - wave + NS - 1) / NS : 0;
    // Loads return in issue order, so the table's loads (L2 hits) go out
    // before the sign words (HBM): the table is written to LDS while the
    // signs are still in flight instead of after the last of them arrives.
    // The table's share of this thread is known exactly: a chunk has at most
    // SPW steps per wave, i.e. 2 SPW table entries (MODE 2) or SPW groups of
    // 8 vector entries (MODE 0/1) per thread.
    constexpr int CP = 2 * SPW;                     // MODE 2: table entries per thread
    constexpr int PG = SPW < 2 ? SPW : 2;           // MODE 0/1: groups per load batch
    u32x4_t pre[CP];
    u32x4_t rs[PG], ra[PG], rb[PG];                 // raw s2 and x of one batch of groups
    const int ncopy = cs * 128;
    const int ngr = cs * 64;
    // Unconditional buffer loads (reads past the range return 0), so no load
    // sits in a divergent branch; the fast path's tail test is applied where
    // the values are used.  With unaligned rows the range is empty and the
    // scalar path below reads the entries.  xrs covers this batch row of x
    // (stage 1) or this chunk of the stage-2 table (stage 2); srs covers s2.
    constexpr uint32_t esz = MODE == 0 ? 2u : 4u;
    const __amdgpu_buffer_rsrc_t xrs =
        make_rsrc(MODE == 2 ? static_cast<const void*>(s2o.tab + s2o.tab_bstride * b + c0 * 1024)
                            : static_cast<const void*>(static_cast<const char*>(vin) + in_bstride * b * esz),
                  MODE == 2 ? (uint32_t)ncopy * 16u : (vec_ok ? (uint32_t)Lk * esz : 0u));
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(vscale, vec_ok && MODE != 2 ? (uint32_t)Lk * 2u : 0u);
    auto fetch = [&](int g, int q) {
      const uint32_t k = (uint32_t)(c0 * 64 + g) * 8u;
      const auto sv = __builtin_amdgcn_raw_buffer_load_b128(srs, k * 2u, 0, 0);
      rs[q] = u32x4_t{sv[0], sv[1], sv[2], sv[3]};
      const auto av = __builtin_amdgcn_raw_buffer_load_b128(xrs, k * esz, 0, 0);
      ra[q] = u32x4_t{av[0], av[1], av[2], av[3]};
      if constexpr (MODE == 1) {
        const auto bv = __builtin_amdgcn_raw_buffer_load_b128(xrs, k * esz + 16u, 0, 0);
        rb[q] = u32x4_t{bv[0], bv[1], bv[2], bv[3]};
      }
    };
    if constexpr (MODE == 2) {
#pragma unroll
      for (int q = 0; q < CP; ++q) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(xrs, (threadIdx.x + q * blockDim.x) * 16u, 0, 0);
        pre[q] = u32x4_t{v[0], v[1], v[2], v[3]};
      }
    } else {
#pragma unroll
      for (int q = 0; q < PG; ++q) fetch(threadIdx.x + q * blockDim.x, q);
    }
    // keep the table's loads ahead of the sign words (neither the optimizer
    // nor the scheduler may move loads across this point)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // every slot is loaded (no branch, so the waits stay exact); slots past
    // this wave's steps read past the buffer, which returns 0 and fetches nothing
    u32x4_t w[SPW][RT];
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const uint32_t soff = (uint32_t)(c0 + wave + i * NS) * 64u;   // 16 words per step
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const uint32_t off = (FULL || i < my) ? voff[t] + soff : 0xFFFFFF00u;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(brs, off, 0, kNT);
        w[i][t] = u32x4_t{v[0], v[1], v[2], v[3]};
      }
    }
    if constexpr (MODE == 2) {
      // Stage 2's tail needs the (C, V) partials of stage 1 and s1 of the
      // rows: loaded behind the sign words (every chunk, so no branch), they
      // arrive while the matrix cores work instead of after them (buffer
      // loads: past the range they return 0)
      const __amdgpu_buffer_rsrc_t prs = make_rsrc(s2o.part + s2o.part_bstride * b, (uint32_t)nparts * 8u);
      const auto pv = __builtin_amdgcn_raw_buffer_load_b64(prs, threadIdx.x * 8u, 0, 0);
      part_c = __uint_as_float(pv[0]);
      part_v = __uint_as_float(pv[1]);
      const __amdgpu_buffer_rsrc_t ors = make_rsrc(oscale, (uint32_t)R * 2u);
      s1_bits = __builtin_amdgcn_raw_buffer_load_b16(ors, (uint32_t)(row_base + lane) * 2u, 0, 0);
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MODE == 2) {
      // this thread's entries of this chunk of the stage-2 table
#pragma unroll
      for (int q = 0; q < CP; ++q) {
        const int i = threadIdx.x + q * blockDim.x;
        if (FULL || i < ncopy) tab[i] = pre[q];
      }
    } else {
      // build the chunk from x and s2: group g of 8 consecutive entries
      // (16-byte loads) goes to thread g mod blockDim; the first batch uses
      // the loads issued above, in straight-line code so they stay ahead of
      // the sign words
      uint16_t* t16 = reinterpret_cast<uint16_t*>(tab);
      auto emit = [&](int g, int q) {
        const int k = (c0 * 64 + g) * 8;
        float v[8];
        const u32x4_t sc = rs[q];
        if constexpr (MODE == 0) {
          const u32x4_t a = ra[q];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[2 * e] = bf16_lo_to_f32(a[e]) * f16_bits_to_f32(sc[e] & 0xFFFFu);
            v[2 * e + 1] = bf16_hi_to_f32(a[e]) * f16_bits_to_f32(sc[e] >> 16);
          }
        } else {
          const u32x4_t a0 = ra[q], a1 = rb[q];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t xw = e < 4 ? a0[e] : a1[e - 4];
            const uint32_t sh = (e & 1) ? (sc[e / 2] >> 16) : (sc[e / 2] & 0xFFFFu);
            v[e] = __uint_as_float(xw) * f16_bits_to_f32(sh);
          }
        }
        if constexpr (!FULL) {
          // tails and unaligned rows replace the fast path's values entry by
          // entry
          const bool fast = vec_ok && g < ngr && k + 8 <= Lk;
          float sl[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          if (!fast) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              if (g < ngr && k + e < Lk) {
                float xv;
                if constexpr (MODE == 0) {
                  xv = bf16_bits_to_f32(static_cast<const uint16_t*>(vin)[in_bstride * b + k + e]);
                } else {
                  xv = static_cast<const float*>(vin)[in_bstride * b + k + e];
                }
                sl[e] = xv * f16_bits_to_f32(vscale[k + e]);
              }
            }
          }
          // the empty asm pins the selected values here, so the compiler
          // cannot fold the select into the branch and sink the fast path's
          // loads behind the sign words
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            v[e] = fast ? v[e] : sl[e];
            asm volatile("" : "+v"(v[e]));
          }
        }
        // groups past the chunk write to a junk slot and add nothing, so
        // this part has no branch either
        const bool valid = FULL || g < ngr;
        const int odd = g & 1;
        const int ep = ((g >> 2) & 3) * 2 + ((g >> 1) & 1);
        const int ent0 = (g >> 6) * 16 * 8 + ((g >> 4) & 3);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          // pair j = 8 odd + e (kl & 15) lands on bit j, j - 7 or j - 14
          const int p0 = odd ? (e < 6 ? e + 1 : e - 6) : e;
          const int p1 = odd ? (e + 1 < 6 ? e + 2 : e - 5) : (e + 1 < 7 ? e + 1 : 0);
          const float a0 = v[e] * __builtin_ldexpf(1.0f, -p0);     // exact
          const float a1 = v[e + 1] * __builtin_ldexpf(1.0f, -p1);
          const uint32_t hi = cvt_pk_bf16(a0, a1);
          const float h0 = bf16_lo_to_f32(hi), h1 = bf16_hi_to_f32(hi);
          const uint32_t lo = cvt_pk_bf16(a0 - h0, a1 - h1);
          const float l0 = bf16_lo_to_f32(lo), l1 = bf16_hi_to_f32(lo);
          const int j0 = 8 * odd + e;
          *(valid ? t16 + (ent0 + j0 * 8) * 8 + ep : junk) = (uint16_t)(hi & 0xFFFFu);
          *(valid ? t16 + (ent0 + j0 * 8 + 4) * 8 + ep : junk) = (uint16_t)(lo & 0xFFFFu);
          *(valid ? t16 + (ent0 + (j0 + 1) * 8) * 8 + ep : junk) = (uint16_t)(hi >> 16);
          *(valid ? t16 + (ent0 + (j0 + 1) * 8 + 4) * 8 + ep : junk) = (uint16_t)(lo >> 16);
          const float s0 = valid ? h0 + l0 : 0.f, s1 = valid ? h1 + l1 : 0.f;
          csum += s0 + s1;
          vsum = __builtin_fmaf(s0, __builtin_ldexpf(1.0f, p0), vsum);
          vsum = __builtin_fmaf(s1, __builtin_ldexpf(1.0f, p1), vsum);
        }
      };
#pragma unroll
      for (int q = 0; q < PG; ++q) emit(threadIdx.x + q * blockDim.x, q);
#pragma unroll
      for (int q0 = PG; q0 < SPW; q0 += PG) {
#pragma unroll
        for (int q = 0; q < PG; ++q) fetch(threadIdx.x + (q0 + q) * blockDim.x, q);
#pragma unroll
        for (int q = 0; q < PG; ++q) emit(threadIdx.x + (q0 + q) * blockDim.x, q);
      }
    }
    __syncthreads();
    const int n1 = r16 & 1;
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      if (FULL || i < my) {
        const int sl = wave + i * NS;                 // step within the chunk
        u32x4_t w7[RT], w14[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t) { w7[t] = w[i][t] >> 7u; w14[t] = w[i][t] >> 14u; }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const u32x4_t frag = tab[((sl * 16 + j) * 2 + n1) * 4 + kg];
          const uint32_t m = 0x00010001u << bin_p(j);
#pragma unroll
          for (int t = 0; t < RT; ++t) {
            const u32x4_t& src = bin_shift(j) == 0 ? w[i][t] : (bin_shift(j) == 7 ? w7[t] : w14[t]);
            u32x4_t a;
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] = (src[e] & m) | bias;
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                             __builtin_bit_cast(bf16x8_t, frag), acc[t], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();   // the next chunk overwrites the table
  }

  // C and V of the whole vector (every workgroup has the same sums)
  if constexpr (MODE == 2) {
    csum += part_c;
    vsum += part_v;
    const float* pp = s2o.part + s2o.part_bstride * b;
    for (int i = threadIdx.x + blockDim.x; i < nparts; i += blockDim.x) { csum += pp[2 * i]; vsum += pp[2 * i + 1]; }
  }
  csum = wave_sum(csum);
  vsum = wave_sum(vsum);
  if (lane == 0) { sums[wave][0] = csum; sums[wave][1] = vsum; }
  // lane (n, kg) holds D[4 kg + i][n]; hi (n = 0) + lo (n = 1) -> lane n = 0
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float d = acc[t][i] + dpp_f32<0x101>(acc[t][i]);   // row_shl:1 (lane l+1)
      if (r16 == 0) red[wave][t * 16 + 4 * kg + i] = d;
    }
  __syncthreads();
  if (wave == 0) {
    float dot = 0.f;
    const int row = row_base + lane;
    if (lane < 16 * RT) {
      float C = 0.f, V = 0.f, D = 0.f;
      for (int w2 = 0; w2 < NS; ++w2) { C += sums[w2][0]; V += sums[w2][1]; D += red[w2][lane]; }
      dot = 2.0f * (D - 128.0f * C) - V;
    }
    if constexpr (MODE == 2) {
      if (lane < 16 * RT && row < R) {
        const float yv = dot * f16_bits_to_f32(s1_bits & 0xFFFFu);
        if (y_bf16) static_cast<uint16_t*>(out)[out_bstride * b + row] = (uint16_t)f32_to_bf16_rne(yv);
        else static_cast<float*>(out)[out_bstride * b + row] = yv;
      }
    } else {
      // t_row -> stage-2 table entry `row`, plus this workgroup's share of
      // the stage-2 C and V; entries past R up to the end of the table's
      // last K-step are zero
      float cpart = 0.f, vpart = 0.f;
      uint16_t* t2 = s2o.tab + s2o.tab_bstride * b;
      const int kend = (R + 511) & ~511;
      if (lane < 16 * RT) {
        const int p = bin_p_rt(row & 15);
        const float a = (row < R ? dot : 0.f) * __builtin_ldexpf(1.0f, -p);
        const uint32_t hi = cvt_pk_bf16(a, 0.f);
        const float hf = bf16_lo_to_f32(hi);
        const uint32_t lo = cvt_pk_bf16(a - hf, 0.f);
        const float lf = bf16_lo_to_f32(lo);
        if (row < kend) {
          t2[tab_off(row, 0) / 2] = (uint16_t)(hi & 0xFFFFu);
          t2[tab_off(row, 1) / 2] = (uint16_t)(lo & 0xFFFFu);
        }
        cpart = hf + lf;
        vpart = (hf + lf) * __builtin_ldexpf(1.0f, p);
      }
      cpart = wave_sum(cpart);
      vpart = wave_sum(vpart);
      if (lane == 0) {
        s2o.part[s2o.part_bstride * b + 2 * blockIdx.x] = cpart;
        s2o.part[s2o.part_bstride * b + 2 * blockIdx.x + 1] = vpart;
      }
      if (blockIdx.x == gridDim.x - 1) {
        for (int k = row_base + 16 * RT + lane; k < kend; k += 64) {
          t2[tab_off(k, 0) / 2] = 0;
          t2[tab_off(k, 1) / 2] = 0;
        }
      }
    }
  }
}

// waves per workgroup: enough for ~2048 waves in all, never more waves than
// steps, and at most max_pw steps per wave and chunk (the sign words a wave
// holds in registers)
int64_t pick_ns(int64_t blocks, int64_t Wn, int max_pw) {
  const int64_t steps = (Wn + 15) / 16;
  const int64_t chunk_steps = steps < kStepsPerChunk ? steps : kStepsPerChunk;
  int64_t ns = 1;
  while (ns < kMaxNS && ns < chunk_steps && blocks * ns < 2048) ns *= 2;
  while ((chunk_steps + ns - 1) / ns > max_pw && ns < kMaxNS) ns *= 2;
  return (chunk_steps + ns - 1) / ns > max_pw ? -1 : ns;
}

template <int MODE, int RT>
hipError_t bin_launch(const uint32_t* bits, int64_t R, int64_t Wn, int64_t Lk, const void* vin,
                      const uint16_t* vscale, const uint16_t* oscale, void* out, int y_bf16,
                      int64_t B, int64_t in_bstride, int64_t out_bstride, Stage2Out s2o,
                      int nparts, hipStream_t s) {
  // stage 1 builds its table from registers loaded next to the sign words,
  // so it keeps fewer steps per wave than stage 2
  constexpr int kMaxPW = MODE == 2 ? 4 : 2;
  const int64_t blocks = (R + 16 * RT - 1) / (16 * RT);
  const int64_t ns = pick_ns(blocks, Wn, kMaxPW);
  if (ns < 0) return hipErrorInvalidValue;
  // 16-byte vector reads of the input vector and s2 need 16-byte aligned rows
  const size_t esz = MODE == 0 ? 2 : 4;
  const int vec_ok = MODE == 2 || ((reinterpret_cast<uintptr_t>(vin) % 16 == 0) && ((in_bstride * esz) % 16 == 0) &&
                                   reinterpret_cast<uintptr_t>(vscale) % 16 == 0);
  // steps per wave, rounded up to a power of two: the kernel holds exactly
  // that many sign-word slots and table loads per thread
  const int64_t steps = (Wn + 15) / 16;
  const int64_t chunk_steps = steps < kStepsPerChunk ? steps : kStepsPerChunk;
  const int64_t per_wave = (chunk_steps + ns - 1) / ns;
  const dim3 grid((unsigned)blocks, (unsigned)B), block((unsigned)(64 * ns));
  const bool full_ok = (MODE == 2 || (vec_ok && Lk % 512 == 0)) && steps % chunk_steps == 0;
  // (the FULL stage-2 kernel with one row tile and 4 steps per wave would
  // spill registers: that shape keeps the general kernel)
#define QG_BIN_LAUNCH(SPW_)                                                                                  \
  do {                                                                                                       \
    constexpr bool kFull = !(MODE == 2 && RT == 1 && (SPW_) == 4);                                           \
    if (full_ok && chunk_steps == (SPW_) * ns)                                                               \
      hipLaunchKernelGGL((bin_mfma_kernel<MODE, RT, SPW_, kFull>), grid, block, 0, s, bits, (int)R, (int)Wn,     \
                         (int)Lk, vin, vscale, oscale, out, y_bf16, in_bstride, out_bstride, vec_ok, s2o, nparts); \
    else                                                                                                     \
      hipLaunchKernelGGL((bin_mfma_kernel<MODE, RT, SPW_, false>), grid, block, 0, s, bits, (int)R, (int)Wn, \
                         (int)Lk, vin, vscale, oscale, out, y_bf16, in_bstride, out_bstride, vec_ok, s2o, nparts); \
  } while (0)
  if (per_wave <= 1) {
    QG_BIN_LAUNCH(1);
  } else if (per_wave <= 2 || kMaxPW == 2) {
    QG_BIN_LAUNCH(2);             // pick_ns keeps per_wave <= kMaxPW
  } else {
    QG_BIN_LAUNCH(kMaxPW);
  }
#undef QG_BIN_LAUNCH
  return hipGetLastError();
}

// row tiles per workgroup: 2 when there are >= 512 tiles to share the table
// over, else 1 (short matrices need the workgroups spread over the CUs)
int pick_rt(int64_t R) { return (R + 15) / 16 >= 512 ? 2 : 1; }

template <int MODE>
hipError_t bin_gemv_t(const uint32_t* bits, int64_t R, int64_t Wn, int64_t Lk, const void* vin,
                      const uint16_t* vscale, const uint16_t* oscale, void* out, int y_bf16,
                      int64_t B, int64_t in_bstride, int64_t out_bstride, Stage2Out s2o,
                      int nparts, hipStream_t s) {
  if (pick_rt(R) == 2)
    return bin_launch<MODE, 2>(bits, R, Wn, Lk, vin, vscale, oscale, out, y_bf16, B, in_bstride, out_bstride,
                               s2o, nparts, s);
  return bin_launch<MODE, 1>(bits, R, Wn, Lk, vin, vscale, oscale, out, y_bf16, B, in_bstride, out_bstride,
                             s2o, nparts, s);
}

int64_t pw(int64_t n) { return ((n + 31) / 32 + 3) / 4 * 4; }

}  // namespace

// Scratch for callers that cannot allocate (qgemv_binlr_noalloc): the
// binary GEMV's workspace as one device array per GPU, alive until the
// process ends.  Host code uses the address hipGetSymbolAddress returns for
// the current device, never the array's name.
static __device__ __align__(256) uint8_t scratch[Q_BINLR_NOALLOC_MAX_WS];

void* binlr_scratch_ptr(hipError_t* err) {
  static std::mutex mu;
  static void* ptrs[64] = {nullptr};
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= 64) { *err = hipErrorInvalidDevice; return nullptr; }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    ptrs[dev] = p;
  }
  *err = hipSuccess;
  return ptrs[dev];
}

int64_t binlr_ws_bytes_per_batch(int64_t r) {
  // stage-2 table (4 bytes per entry, whole 512-entry steps) + (C, V) partials
  // of at most one stage-1 workgroup per 16 rows of V^T
  const int64_t tab = (r + 511) / 512 * 2048;
  const int64_t part = ((r + 15) / 16) * 8;
  return (tab + part + 15) / 16 * 16;
}

hipError_t launch_gemv_binlr(const uint32_t* ubits, const uint32_t* vtbits,
                             const uint16_t* s1, const uint16_t* s2, int64_t N, int64_t K,
                             int64_t r, const void* x, int x_dtype, int64_t B, void* y,
                             int y_dtype, void* ws, hipStream_t s) {
  const int64_t wsb = binlr_ws_bytes_per_batch(r);
  Stage2Out o;
  o.tab = static_cast<uint16_t*>(ws);
  o.part = reinterpret_cast<float*>(static_cast<char*>(ws) + (r + 511) / 512 * 2048);
  o.tab_bstride = wsb / 2;
  o.part_bstride = wsb / 4;
  const int nparts = (int)((r + 16 * pick_rt(r) - 1) / (16 * pick_rt(r)));
  hipError_t e;
  if (x_dtype == 1)
    e = bin_gemv_t<0>(vtbits, r, pw(K), K, x, s2, nullptr, nullptr, 0, B, K, 0, o, 0, s);
  else
    e = bin_gemv_t<1>(vtbits, r, pw(K), K, x, s2, nullptr, nullptr, 0, B, K, 0, o, 0, s);
  if (e != hipSuccess) return e;
  return bin_gemv_t<2>(ubits, N, pw(r), r, nullptr, nullptr, s1, y, y_dtype == 1, B, 0, N, o, nparts, s);
}

}  // namespace qg
