// Prefill GEMM launchers: group RTN (one pass) and binary low-rank (two
// passes); the tile kernel is in gemm_tile.hpp, the outlier-column variant
// of the group path in gemm_prefill_outlier.hip.
#include "gemm_tile.hpp"

namespace qg {

template <int BITS, int G>
static hipError_t gemm_group_t(const uint32_t* codes, const uint32_t* meta, int64_t N, int64_t K,
                               const uint16_t* X, int64_t M, void* Y, int y_bf16, hipStream_t s, SideCols sc) {
  DecRTN<BITS, G> dec{codes, meta, (int)N, (int)(K / 32)};
  if (K < kSplitBelowK)
    return gemm_run<DecRTN<BITS, G>, 0, false, false, true>(X, K, M, K, dec, N, nullptr, nullptr, Y, N, y_bf16, s, sc);
  return gemm_run<DecRTN<BITS, G>, 0, false>(X, K, M, K, dec, N, nullptr, nullptr, Y, N, y_bf16, s, sc);
}

hipError_t launch_gemm_group(const uint32_t* codes, const uint32_t* meta, int64_t N,
                             int64_t K, int bits, int group, const uint16_t* X, int64_t M,
                             void* Y, int y_dtype, hipStream_t s, const uint16_t* side,
                             const int32_t* oidx, int n_out) {
  if (n_out > 0) return launch_gemm_group_outlier(codes, meta, N, K, bits, group, X, M, Y, y_dtype, s, side, oidx, n_out);
  const int yb = y_dtype == 1;
  const SideCols sc{nullptr, nullptr, 0};
#define CALL(b, g) gemm_group_t<b, g>(codes, meta, N, K, X, M, Y, yb, s, sc)
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

static int64_t pwords(int64_t n) { return ((n + 31) / 32 + 3) / 4 * 4; }

hipError_t launch_gemm_binlr(const uint32_t* ubits, const uint32_t* vtbits,
                             const uint16_t* s1, const uint16_t* s2, int64_t N, int64_t K,
                             int64_t r, const uint16_t* X, int64_t M, void* Y, int y_dtype,
                             void* T_ws, hipStream_t s) {
  const int64_t rp = pwords(r) * 32;
  const int yb = y_dtype == 1;
  DecBIN d1{vtbits, (int)r, (int)pwords(K)};   // pass 1: weight rows = VT rows (r of them)
  DecBIN d2{ubits, (int)N, (int)pwords(r)};    // pass 2: weight rows = U rows
  if (K < kSplitBelowK) {
    // split precision: T[M][rp] = (X * s2) V in fp32 from bf16 hi + lo parts
    // of X * s2, then Y = (T U^T) * s1 with T as bf16 hi + lo
    hipError_t e = gemm_run<DecBIN, 1, false, false, true>(X, K, M, K, d1, r, s2, nullptr, T_ws, rp, 0, s);
    if (e != hipSuccess) return e;
    if (r % 8) return gemm_run<DecBIN, 2, true, false, true>(T_ws, rp, M, r, d2, N, nullptr, s1, Y, N, yb, s);
    return gemm_run<DecBIN, 2, false, false, true>(T_ws, rp, M, r, d2, N, nullptr, s1, Y, N, yb, s);
  }
  // pass 1: T[M][rp] = bf16((X * s2) V)
  const hipError_t e = gemm_run<DecBIN, 1, false>(X, K, M, K, d1, r, s2, nullptr, T_ws, rp, 1, s);
  if (e != hipSuccess) return e;
  // pass 2: Y = (T U^T) * s1
  if (r % 8) return gemm_run<DecBIN, 0, true>(T_ws, rp, M, r, d2, N, nullptr, s1, Y, N, yb, s);
  return gemm_run<DecBIN, 0, false>(T_ws, rp, M, r, d2, N, nullptr, s1, Y, N, yb, s);
}

int64_t gemm_binlr_ws_bytes(int64_t M, int64_t K, int64_t r) {
  // T[M][rp]: bf16, or fp32 for the split-precision passes of short K
  return M * pwords(r) * 32 * (K < kSplitBelowK ? 4 : 2);
}

}  // namespace qg
