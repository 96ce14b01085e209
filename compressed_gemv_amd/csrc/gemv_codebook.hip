// Decode GEMV for group codes read through per-group books of a shared
// dictionary ("TurboQuant: cuantizar modelos grandes para que quepan en
// local", introduction and "Compresión por bloques"):
// y[b][n] = sum_k (s * e[book][q[n][k]] / 2^(7-bits) + o) x[b][k].
// Kernels: the CB variants in gemv_kernels.hpp, with the tile choices of the
// plain codes.
#include "gemv_kernels.hpp"

// Tile choice of the B = 1 kernel for codebook decode.  The lookups about
// double the VALU work per code (4-bit: ~3 instructions per code against
// ~1.4), so two waves per SIMD (2048 waves) hide the dependent permute
// chains better than the plain kernel's one; rows per stage as for plain
// codes.  Measured on MI355X over the gate, q and down shapes (sums of the
// three, us): 4-bit 83.0 -> 73.3, 3-bit 71.2 -> 67.7, 2-bit 55.1 -> 55.0.
// QG_CB_WAVES / QG_CB_RPW force one choice.
#ifndef QG_CB_WAVES
#define QG_CB_WAVES 0
#endif
#ifndef QG_CB_RPW
#define QG_CB_RPW 0
#endif

namespace qg {

template <int BITS, int G>
static hipError_t gemv_cb_dispatch(const uint32_t* codes, const uint32_t* meta, Books bk, int64_t N,
                                   int64_t K, const void* x, int x_dtype, int64_t B, void* y, int y_bf16,
                                   hipStream_t s) {
  const Side none{nullptr, nullptr, 0};
  if (B == 1) {
    if (x_dtype == 0)
      return gemv_b1_t<BITS, G, true, 2, 2, true>(codes, meta, N, K, x, y, y_bf16, s, 2048, none, nullptr, bk);
    constexpr int kRpw = QG_CB_RPW ? QG_CB_RPW : (BITS == 3 ? 2 : 1);
    const int64_t waves = QG_CB_WAVES ? QG_CB_WAVES : 2048;
    return gemv_b1_t<BITS, G, false, 4, kRpw, true>(codes, meta, N, K, x, y, y_bf16, s, waves, none, nullptr, bk);
  }
  if (x_dtype != 1) return hipErrorInvalidValue;
  return gemv_mfma_t<BITS, G, true>(codes, meta, N, K, static_cast<const uint16_t*>(x), B, y, y_bf16, s, none, bk);
}

hipError_t launch_gemv_group_cb(const uint32_t* codes, const uint32_t* meta, const uint8_t* book_ids,
                                const uint8_t* books, int n_books, int64_t N, int64_t K, int bits, int group,
                                const void* x, int x_dtype, int64_t B, void* y, int y_dtype, hipStream_t s) {
  const int yb = y_dtype == 1;
  const Books bk{book_ids, books, n_books};
#define CALL(b, g) gemv_cb_dispatch<b, g>(codes, meta, bk, N, K, x, x_dtype, B, y, yb, s)
  switch (bits * 100 + group) {
    case 232: return CALL(2, 32); case 264: return CALL(2, 64);
    case 332: return CALL(3, 32); case 364: return CALL(3, 64);
    case 432: return CALL(4, 32); case 464: return CALL(4, 64);
    default: return hipErrorInvalidValue;
  }
#undef CALL
}

}  // namespace qg
