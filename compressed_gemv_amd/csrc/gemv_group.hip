// Group-RTN GEMV for decode, y[b][n] = sum_k (s*q[n][k] + o) x[b][k].
//
// Kernels and launch templates: gemv_kernels.hpp.  This file holds the
// dispatch of the plain, outlier and grouped entry points.
#include "gemv_kernels.hpp"

namespace qg {

template <int BITS, int G>
static hipError_t gemv_dispatch(const uint32_t* codes, const uint32_t* meta, int64_t N,
                                int64_t K, const void* x, int x_dtype, int64_t B, void* y,
                                int y_bf16, hipStream_t s, Side sd, const MultiSegs* ms = nullptr) {
  if (B == 1) {
    if (x_dtype == 0) return gemv_b1_t<BITS, G, true, 2, 2>(codes, meta, N, K, x, y, y_bf16, s, 2048, sd, ms);
    constexpr int kRpw = QG_B1_RPW ? QG_B1_RPW : (BITS == 3 ? 2 : 1);
    const int64_t waves = BITS == 2 ? 2048 : 1024;
    if (QG_B1_UI == 2)
      return gemv_b1_t<BITS, G, false, 2, QG_B1_RPW ? QG_B1_RPW : 2>(codes, meta, N, K, x, y, y_bf16, s, 2048,
                                                                       sd, ms);
    return gemv_b1_t<BITS, G, false, 4, kRpw>(codes, meta, N, K, x, y, y_bf16, s, waves, sd, ms);
  }
  if (ms) return hipErrorInvalidValue;   // the grouped launch is for batch 1
  if (x_dtype != 1) return hipErrorInvalidValue;
  return gemv_mfma_t<BITS, G>(codes, meta, N, K, static_cast<const uint16_t*>(x), B, y, y_bf16, s, sd);
}

hipError_t launch_gemv_group(const uint32_t* codes, const uint32_t* meta, int64_t N,
                             int64_t K, int bits, int group, const void* x, int x_dtype,
                             int64_t B, void* y, int y_dtype, hipStream_t s, const uint16_t* side,
                             const int32_t* oidx, int n_out) {
  const int yb = y_dtype == 1;
  const Side sd{side, oidx, n_out};
#define CALL(b, g) gemv_dispatch<b, g>(codes, meta, N, K, x, x_dtype, B, y, yb, s, sd)
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

hipError_t launch_gemv_group_multi(const MultiSegs& ms, int64_t K, int bits, int group, const void* x,
                                   int x_dtype, int64_t B, void* y0, int y_dtype, hipStream_t s) {
  const int yb = y_dtype == 1;
  if (B > 1) {   // one matrix-core launch over the matrices' tiles
    if (x_dtype != 1) return hipErrorInvalidValue;
    const uint16_t* xb = static_cast<const uint16_t*>(x);
#define CALLB(b, g) gemv_mfma_multi_t<b, g>(ms, K, xb, B, yb, s)
    switch (bits * 100 + group) {
      case 232: return CALLB(2, 32); case 264: return CALLB(2, 64);
      case 332: return CALLB(3, 32); case 364: return CALLB(3, 64);
      case 432: return CALLB(4, 32); case 464: return CALLB(4, 64);
      case 532: return CALLB(5, 32); case 564: return CALLB(5, 64);
      case 632: return CALLB(6, 32); case 664: return CALLB(6, 64);
      default: return hipErrorInvalidValue;
    }
#undef CALLB
  }
  int64_t N = 0;
  for (int i = 0; i < ms.nseg; ++i) N += ms.nrows[i];
  const Side none{nullptr, nullptr, 0};
  const uint32_t* c0 = static_cast<const uint32_t*>(ms.codes[0]);
  const uint32_t* m0 = static_cast<const uint32_t*>(ms.meta[0]);
#define CALL(b, g) gemv_dispatch<b, g>(c0, m0, N, K, x, x_dtype, 1, y0, yb, s, none, &ms)
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
