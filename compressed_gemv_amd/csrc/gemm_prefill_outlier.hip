// Prefill GEMM of the group format with outlier side columns (the mixed
// decomposition of "Métodos de cuantización de LLM...", opening and
// LLM.int8() paragraph): the tile kernel of gemm_tile.hpp with one more
// K-step for the side columns.  A translation unit of its own so the build
// compiles it in parallel with the plain instantiations.
#include "gemm_tile.hpp"

namespace qg {

template <int BITS, int G>
static hipError_t gemm_group_outl_t(const uint32_t* codes, const uint32_t* meta, int64_t N, int64_t K,
                                    const uint16_t* X, int64_t M, void* Y, int y_bf16, hipStream_t s,
                                    SideCols sc) {
  DecRTN<BITS, G> dec{codes, meta, (int)N, (int)(K / 32)};
  if (K < kSplitBelowK)
    return gemm_run<DecRTN<BITS, G>, 0, false, true, true>(X, K, M, K, dec, N, nullptr, nullptr, Y, N, y_bf16, s, sc);
  return gemm_run<DecRTN<BITS, G>, 0, false, true>(X, K, M, K, dec, N, nullptr, nullptr, Y, N, y_bf16, s, sc);
}

hipError_t launch_gemm_group_outlier(const uint32_t* codes, const uint32_t* meta, int64_t N, int64_t K,
                                     int bits, int group, const uint16_t* X, int64_t M, void* Y, int y_dtype,
                                     hipStream_t s, const uint16_t* side, const int32_t* oidx, int n_out) {
  const int yb = y_dtype == 1;
  const SideCols sc{side, oidx, n_out};
#define CALL(b, g) gemm_group_outl_t<b, g>(codes, meta, N, K, X, M, Y, yb, s, sc)
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
