// Prefill GEMM for group codes read through per-group books ("TurboQuant:
// cuantizar modelos grandes para que quepan en local", introduction and
// "Compresión por bloques"): the tiles of gemm_tile.hpp with the DecCB
// decoder, Y = X W_hat^T, w_hat = s e[book][q] / 2^(7-bits) + o.
#include "gemm_tile.hpp"

namespace qg {

template <int BITS, int G>
static hipError_t gemm_group_cb_t(const uint32_t* codes, const uint32_t* meta, const uint8_t* ids,
                                  const uint8_t* books, int nb, int64_t N, int64_t K, const uint16_t* X,
                                  int64_t M, void* Y, int y_bf16, hipStream_t s) {
  DecCB<BITS, G> dec{codes, meta, ids, books, nb, (int)N, (int)(K / 32), nullptr, CbConst{}};
  if (K < kSplitBelowK)
    return gemm_run<DecCB<BITS, G>, 0, false, false, true>(X, K, M, K, dec, N, nullptr, nullptr, Y, N, y_bf16, s);
  return gemm_run<DecCB<BITS, G>, 0, false>(X, K, M, K, dec, N, nullptr, nullptr, Y, N, y_bf16, s);
}

hipError_t launch_gemm_group_cb(const uint32_t* codes, const uint32_t* meta, const uint8_t* book_ids,
                                const uint8_t* books, int n_books, int64_t N, int64_t K, int bits, int group,
                                const uint16_t* X, int64_t M, void* Y, int y_dtype, hipStream_t s) {
  const int yb = y_dtype == 1;
#define CALL(b, g) gemm_group_cb_t<b, g>(codes, meta, book_ids, books, n_books, N, K, X, M, Y, yb, s)
  switch (bits * 100 + group) {
    case 232: return CALL(2, 32); case 264: return CALL(2, 64);
    case 332: return CALL(3, 32); case 364: return CALL(3, 64);
    case 432: return CALL(4, 32); case 464: return CALL(4, 64);
    default: return hipErrorInvalidValue;
  }
#undef CALL
}

}  // namespace qg
