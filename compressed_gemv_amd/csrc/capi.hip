// C ABI of the compressed-weight product (declared in include/qgemv.h):
// argument validation, size queries, status codes, dispatch to the kernels.
// Validation runs on the host before any HIP call, so bad arguments are
// reported without touching the GPU.
#include "qgemv.h"

#include "launch.hpp"

#include <math.h>
#include <stdint.h>

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 30;
constexpr int64_t kMaxOutliers = 64;     // outlier side columns per matrix

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int group_args_ok(int64_t N, int64_t K, int bits, int group) {
  if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim) return Q_EINVAL;
  if (bits < 2 || bits > 6) return Q_EINVAL;
  if (group != 32 && group != 64) return Q_EINVAL;
  if (K % group) return Q_EINVAL;
  // the kernels address codes and meta through 32-bit buffer offsets
  if (N * K / 8 * bits >= ((int64_t)1 << 32)) return Q_EUNSUPPORTED;
  return Q_OK;
}

int64_t padded_words(int64_t n) { return ((n + 31) / 32 + 3) / 4 * 4; }

int hip_status(hipError_t e) { return e == hipSuccess ? Q_OK : Q_EHIP; }

int dtype_ok(int d) { return d == Q_F32 || d == Q_BF16; }

// B = 1 keeps a K-slice of activations in registers; at most 8 slices of
// 64 lanes x UI units x 32 inputs (UI = 4 for bf16 rows longer than 16384,
// 2 for fp32 activations).
int64_t gemv_b1_max_k(int x_dtype) { return x_dtype == Q_F32 ? 8 * 64 * 2 * 32 : 8 * 64 * 4 * 32; }

// The batched GEMV addresses a lane's activation slice as (row * K + unit
// * 32) * 2 bytes in 32-bit signed arithmetic: B * K * 2 must stay below
// 2^31.
int batched_x_ok(int64_t B, int64_t K) { return B > 1 && B * K * 2 >= ((int64_t)1 << 31) ? Q_EUNSUPPORTED : Q_OK; }

// Prefill tile loads address X (and the binary path's T) through 32-bit
// offsets from the tile's first row: 256 rows of K bf16 inputs, and of the
// padded rank in fp32 for T, must fit; the grid of 64 x 128 tiles must fit
// a signed 32-bit workgroup index.
int prefill_dims_ok(int64_t M, int64_t N, int64_t K, int64_t rp) {
  if (K * 256 * 2 >= ((int64_t)1 << 32) || rp * 256 * 4 >= ((int64_t)1 << 32)) return Q_EUNSUPPORTED;
  if (((M + 63) / 64) * ((N + 127) / 128) >= ((int64_t)1 << 31)) return Q_EUNSUPPORTED;
  return Q_OK;
}

// codebooks: 2..4-bit codes, 1..16 books
int cb_args_ok(int64_t N, int64_t K, int bits, int group, const uint8_t* books, int n_books) {
  const int st = group_args_ok(N, K, bits, group);
  if (st != Q_OK) return st;
  if (bits > 4 || !books || n_books < 1 || n_books > 16) return Q_EINVAL;
  return Q_OK;
}

}  // namespace

extern "C" {

int q_abi_version(void) { return Q_ABI_VERSION; }
int q_format_version(void) { return Q_FORMAT_VERSION; }

const char* q_status_str(int status) {
  switch (status) {
    case Q_OK: return "ok";
    case Q_EINVAL: return "invalid argument";
    case Q_EALIGN: return "misaligned buffer";
    case Q_EUNSUPPORTED: return "unsupported parameter combination";
    case Q_ERANGE: return "data out of range (non-finite weight, fp16 overflow or entry not +-1)";
    case Q_EWORKSPACE: return "workspace missing or too small";
    case Q_EHIP: return "HIP runtime or launch error";
    default: return "unknown status";
  }
}

int qgroup_sizes(int64_t N, int64_t K, int bits, int group, size_t* codes_bytes,
                 size_t* meta_bytes) {
  const int st = group_args_ok(N, K, bits, group);
  if (st != Q_OK) return st;
  if (codes_bytes) *codes_bytes = (size_t)(N * K / 8 * bits);
  if (meta_bytes) *meta_bytes = (size_t)(N * (K / group) * 4);
  return Q_OK;
}

int qpack_group(const float* W, int64_t N, int64_t K, int bits, int group, void* codes,
                void* meta, hipStream_t stream) {
  const int st = group_args_ok(N, K, bits, group);
  if (st != Q_OK) return st;
  if (!W || !codes || !meta) return Q_EINVAL;
  if (!aligned(W, 16) || !aligned(codes, 16) || !aligned(meta, 16)) return Q_EALIGN;
  hipError_t e;
  int* status = qg::pack_status_ptr(&e);
  if (!status) return Q_EHIP;
  if ((e = qg::launch_zero_status(status, stream)) != hipSuccess) return Q_EHIP;
  e = qg::launch_pack_group(W, N, K, bits, group, static_cast<uint32_t*>(codes),
                            static_cast<uint32_t*>(meta), status, stream);
  if (e != hipSuccess) return Q_EHIP;
  int host = 0;
  if (hipMemcpyAsync(&host, status, sizeof(int), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return Q_EHIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return Q_EHIP;
  return host ? Q_ERANGE : Q_OK;
}

int qunpack_group(const void* codes, const void* meta, int64_t N, int64_t K, int bits,
                  int group, uint8_t* q_out, float* w_out, hipStream_t stream) {
  const int st = group_args_ok(N, K, bits, group);
  if (st != Q_OK) return st;
  if (!codes || !meta || !q_out) return Q_EINVAL;
  if (!aligned(codes, 4) || !aligned(meta, 4) || !aligned(q_out, 4) || (w_out && !aligned(w_out, 4)))
    return Q_EALIGN;
  return hip_status(qg::launch_unpack_group(static_cast<const uint32_t*>(codes),
                                            static_cast<const uint32_t*>(meta), N, K, bits,
                                            group, q_out, w_out, stream));
}

int qgemv_group(const void* codes, const void* meta, int64_t N, int64_t K, int bits, int group,
                const void* x, int x_dtype, int64_t B, void* y, int y_dtype, hipStream_t stream) {
  const int st = group_args_ok(N, K, bits, group);
  if (st != Q_OK) return st;
  if (!codes || !meta || !x || !y) return Q_EINVAL;
  if (B < 1 || B > 16) return Q_EINVAL;
  if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return Q_EINVAL;
  if (!aligned(codes, 16) || !aligned(meta, 16) || !aligned(x, 16) || !aligned(y, 4))
    return Q_EALIGN;
  if (B == 1 && K > gemv_b1_max_k(x_dtype)) return Q_EUNSUPPORTED;
  if (batched_x_ok(B, K) != Q_OK) return Q_EUNSUPPORTED;
  if (B > 1 && x_dtype != Q_BF16) return Q_EUNSUPPORTED;
  if (N > INT32_MAX || K > INT32_MAX) return Q_EUNSUPPORTED;
  return hip_status(qg::launch_gemv_group(static_cast<const uint32_t*>(codes),
                                          static_cast<const uint32_t*>(meta), N, K, bits, group,
                                          x, x_dtype, B, y, y_dtype, stream));
}

int qgemv_group_multi(const qgroup_mat* mats, int count, int64_t K, int bits, int group,
                      const void* x, int x_dtype, int64_t B, int y_dtype, hipStream_t stream) {
  if (!mats || count < 1 || count > 4 || !x) return Q_EINVAL;
  if (B < 1 || B > 16) return Q_EINVAL;
  if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return Q_EINVAL;
  int64_t total = 0;
  for (int i = 0; i < count; ++i) {
    const int st = group_args_ok(mats[i].N, K, bits, group);
    if (st != Q_OK) return st;
    if (!mats[i].codes || !mats[i].meta || !mats[i].y) return Q_EINVAL;
    if (!aligned(mats[i].codes, 16) || !aligned(mats[i].meta, 16) || !aligned(mats[i].y, 4)) return Q_EALIGN;
    total += mats[i].N;
  }
  if (!aligned(x, 16)) return Q_EALIGN;
  if (B == 1 && K > gemv_b1_max_k(x_dtype)) return Q_EUNSUPPORTED;
  if (batched_x_ok(B, K) != Q_OK) return Q_EUNSUPPORTED;
  if (B > 1 && x_dtype != Q_BF16) return Q_EUNSUPPORTED;
  if (total > INT32_MAX || K > INT32_MAX) return Q_EUNSUPPORTED;
  qg::MultiSegs ms{};
  int start = 0;
  for (int i = 0; i < 4; ++i) {
    if (i < count) {
      ms.codes[i] = mats[i].codes; ms.meta[i] = mats[i].meta; ms.y[i] = mats[i].y;
      ms.nrows[i] = mats[i].N; ms.start[i] = start;
      start += (int)mats[i].N;
    } else {
      ms.codes[i] = mats[0].codes; ms.meta[i] = mats[0].meta; ms.y[i] = mats[0].y;
      ms.nrows[i] = 0; ms.start[i] = INT32_MAX;
    }
  }
  ms.nseg = count;
  return hip_status(qg::launch_gemv_group_multi(ms, K, bits, group, x, x_dtype, B, mats[0].y, y_dtype, stream));
}

int outlier_args_ok(int64_t K, int64_t n_out) {
  return (n_out >= 0 && n_out <= kMaxOutliers && n_out <= K) ? Q_OK : Q_EINVAL;
}

int qgroup_outlier_ws(int64_t K, int64_t n_out, size_t* ws_bytes) {
  if (!ws_bytes || K < 1 || K > kMaxDim) return Q_EINVAL;
  const int st = outlier_args_ok(K, n_out);
  if (st != Q_OK) return st;
  *ws_bytes = qg::pack_group_outlier_ws_bytes(K);
  return Q_OK;
}

int qpack_group_outlier(const float* W, int64_t N, int64_t K, int bits, int group, int64_t n_out,
                        void* codes, void* meta, uint16_t* side, int32_t* idx, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  int st = group_args_ok(N, K, bits, group);
  if (st != Q_OK) return st;
  if ((st = outlier_args_ok(K, n_out)) != Q_OK) return st;
  if (!W || !codes || !meta || (n_out > 0 && (!side || !idx))) return Q_EINVAL;
  if (!aligned(W, 16) || !aligned(codes, 16) || !aligned(meta, 16) || !aligned(side, 2) || !aligned(idx, 4))
    return Q_EALIGN;
  if (!ws || ws_bytes < qg::pack_group_outlier_ws_bytes(K)) return Q_EWORKSPACE;
  if (!aligned(ws, 16)) return Q_EALIGN;
  hipError_t e;
  int* status = qg::pack_status_ptr(&e);
  if (!status) return Q_EHIP;
  if ((e = qg::launch_zero_status(status, stream)) != hipSuccess) return Q_EHIP;
  e = qg::launch_pack_group_outlier(W, N, K, bits, group, (int)n_out, static_cast<uint32_t*>(codes),
                                    static_cast<uint32_t*>(meta), side, idx, ws, status, stream);
  if (e != hipSuccess) return Q_EHIP;
  int host = 0;
  if (hipMemcpyAsync(&host, status, sizeof(int), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return Q_EHIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return Q_EHIP;
  return host ? Q_ERANGE : Q_OK;
}

int qgemv_group_outlier(const void* codes, const void* meta, const uint16_t* side, const int32_t* idx,
                        int64_t n_out, int64_t N, int64_t K, int bits, int group, const void* x,
                        int x_dtype, int64_t B, void* y, int y_dtype, hipStream_t stream) {
  int st = group_args_ok(N, K, bits, group);
  if (st != Q_OK) return st;
  if ((st = outlier_args_ok(K, n_out)) != Q_OK) return st;
  if (n_out > 0 && (!side || !idx)) return Q_EINVAL;
  if (!aligned(side, 2) || !aligned(idx, 4)) return Q_EALIGN;
  if (!codes || !meta || !x || !y) return Q_EINVAL;
  if (B < 1 || B > 16) return Q_EINVAL;
  if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return Q_EINVAL;
  if (!aligned(codes, 16) || !aligned(meta, 16) || !aligned(x, 16) || !aligned(y, 4))
    return Q_EALIGN;
  if (B == 1 && K > gemv_b1_max_k(x_dtype)) return Q_EUNSUPPORTED;
  if (batched_x_ok(B, K) != Q_OK) return Q_EUNSUPPORTED;
  if (B > 1 && x_dtype != Q_BF16) return Q_EUNSUPPORTED;
  if (N > INT32_MAX || K > INT32_MAX || N * n_out > INT32_MAX) return Q_EUNSUPPORTED;
  return hip_status(qg::launch_gemv_group(static_cast<const uint32_t*>(codes),
                                          static_cast<const uint32_t*>(meta), N, K, bits, group,
                                          x, x_dtype, B, y, y_dtype, stream, side, idx, (int)n_out));
}

int qcodebook_default(int bits, uint8_t* books, int* n_books) {
  if (bits < 2 || bits > 4 || !books) return Q_EINVAL;
  // 8 monotone warps of the uniform grid c = j (j = 0..L-1, L = 2^bits):
  // uniform; centre-dense m(1 + sign(t)|t|^g), t = 2j/(L-1) - 1,
  // m = (L-1)/2, g = 1.5, 2, 3; minimum-dense (L-1) a^g, a = j/(L-1),
  // g = 1.5, 2.5; and their mirrors (L-1)(1 - (1-a)^g).  Entry =
  // c * 2^(7-bits) rounded to nearest, ties to even.
  const int L = 1 << bits;
  const double top = (double)(L - 1), m = top / 2.0, unit = (double)(1 << (7 - bits));
  const double gc[3] = {1.5, 2.0, 3.0}, gs[2] = {1.5, 2.5};
  for (int j = 0; j < L; ++j) {
    const double t = 2.0 * j / top - 1.0, a = j / top;
    double c[8];
    c[0] = j;
    for (int i = 0; i < 3; ++i) c[1 + i] = m * (1.0 + (t < 0 ? -1.0 : 1.0) * pow(fabs(t), gc[i]));
    for (int i = 0; i < 2; ++i) {
      c[4 + i] = top * pow(a, gs[i]);
      c[6 + i] = top * (1.0 - pow(1.0 - a, gs[i]));
    }
    for (int d = 0; d < 8; ++d) books[d * L + j] = (uint8_t)nearbyint(c[d] * unit);
  }
  if (n_books) *n_books = 8;
  return Q_OK;
}

int qpack_group_cb(const float* W, int64_t N, int64_t K, int bits, int group, const uint8_t* books, int n_books,
                   void* codes, void* meta, uint8_t* book_ids, hipStream_t stream) {
  const int st = cb_args_ok(N, K, bits, group, books, n_books);
  if (st != Q_OK) return st;
  if (!W || !codes || !meta || !book_ids) return Q_EINVAL;
  if (!aligned(W, 16) || !aligned(codes, 16) || !aligned(meta, 16)) return Q_EALIGN;
  hipError_t e;
  int* status = qg::pack_status_ptr(&e);
  if (!status) return Q_EHIP;
  if ((e = qg::launch_zero_status(status, stream)) != hipSuccess) return Q_EHIP;
  e = qg::launch_pack_group_cb(W, N, K, bits, group, books, n_books, static_cast<uint32_t*>(codes),
                               static_cast<uint32_t*>(meta), book_ids, status, stream);
  if (e != hipSuccess) return Q_EHIP;
  int host = 0;
  if (hipMemcpyAsync(&host, status, sizeof(int), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return Q_EHIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return Q_EHIP;
  return (host & 2) ? Q_EINVAL : (host ? Q_ERANGE : Q_OK);
}

int qgemv_group_cb(const void* codes, const void* meta, const uint8_t* book_ids, const uint8_t* books,
                   int n_books, int64_t N, int64_t K, int bits, int group, const void* x, int x_dtype,
                   int64_t B, void* y, int y_dtype, hipStream_t stream) {
  const int st = cb_args_ok(N, K, bits, group, books, n_books);
  if (st != Q_OK) return st;
  if (!codes || !meta || !book_ids || !x || !y) return Q_EINVAL;
  if (B < 1 || B > 16) return Q_EINVAL;
  if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return Q_EINVAL;
  if (!aligned(codes, 16) || !aligned(meta, 16) || !aligned(x, 16) || !aligned(y, 4))
    return Q_EALIGN;
  if (B == 1 && K > gemv_b1_max_k(x_dtype)) return Q_EUNSUPPORTED;
  if (batched_x_ok(B, K) != Q_OK) return Q_EUNSUPPORTED;
  if (B > 1 && x_dtype != Q_BF16) return Q_EUNSUPPORTED;
  if (N > INT32_MAX || K > INT32_MAX) return Q_EUNSUPPORTED;
  return hip_status(qg::launch_gemv_group_cb(static_cast<const uint32_t*>(codes),
                                             static_cast<const uint32_t*>(meta), book_ids, books, n_books,
                                             N, K, bits, group, x, x_dtype, B, y, y_dtype, stream));
}

int qtq_centroids(int d, int mbits, float* delta, uint8_t* table) {
  if (d < 3 || d > 65536 || mbits < 1 || mbits > 4 || !delta || !table) return Q_EINVAL;
  double c[16];
  qg::tq_lloyd_max(d, mbits, c);
  const int L = 1 << mbits;
  double cmax = 0.0;
  for (int k = 0; k < L; ++k) cmax = fmax(cmax, fabs(c[k]));
  const float dl = (float)(cmax / 63.0);
  for (int k = 0; k < L; ++k) {
    const double e = nearbyint(c[k] / (double)dl) + 64.0;
    if (e < 1.0 || e > 127.0) return Q_ERANGE;
    table[k] = (uint8_t)e;
  }
  *delta = dl;
  return Q_OK;
}

int qtq_rotation(int d, const double* G, double* Pi) {
  if (d < 1 || d > 4096 || !G || !Pi) return Q_EINVAL;
  qg::tq_rotation(d, G, Pi);
  for (int i = 0; i < d * d; ++i)
    if (!isfinite(Pi[i])) return Q_ERANGE;   // G was singular
  return Q_OK;
}

namespace {
constexpr int kTqDim = 128;
// one head's keys are addressed through 32-bit byte offsets (64 bytes of
// fp32 input per key half-row, 256 bytes of slack): n below this bound
constexpr int64_t kTqMaxKeys = (((int64_t)1 << 32) - 256) / 64;
// bits = stored bits per coordinate; the table has 2^m entries, m = bits - 1
// for keys (one sign bit) and m = bits for values
int tq_table_ok(int m, float delta, const uint8_t* table) {
  if (!table || !(delta > 0.0f) || !isfinite(delta)) return Q_EINVAL;
  for (int k = 0; k < (1 << m); ++k)
    if (table[k] < 1 || table[k] > 127) return Q_EINVAL;
  return Q_OK;
}
int tq_args_ok(int64_t n, int64_t heads, int bits, float delta, const uint8_t* table) {
  if (n < 1 || heads < 1 || bits < 3 || bits > 4 || !table) return Q_EINVAL;
  if (!(delta > 0.0f) || !isfinite(delta)) return Q_EINVAL;
  // keys of one head are addressed through 32-bit buffer offsets
  if (n >= kTqMaxKeys || heads > 65535 || n * heads > INT32_MAX) return Q_EUNSUPPORTED;
  const int L = 1 << (bits - 1);
  for (int k = 0; k < L; ++k)
    if (table[k] < 1 || table[k] > 127) return Q_EINVAL;
  return Q_OK;
}
void tq_table_words(const uint8_t* t, int L, uint32_t* w4) {
  for (int i = 0; i < 4; ++i) w4[i] = 0;
  for (int k = 0; k < L; ++k) w4[k >> 2] |= (uint32_t)t[k] << (8 * (k & 3));
}
}  // namespace

int qtq_sizes(int64_t n, int bits, size_t* codes_bytes, size_t* signs_bytes, size_t* norms_bytes) {
  if (n < 1 || bits < 3 || bits > 4) return Q_EINVAL;
  if (n >= kTqMaxKeys) return Q_EUNSUPPORTED;
  if (codes_bytes) *codes_bytes = (size_t)(n * kTqDim * (bits - 1) / 8);
  if (signs_bytes) *signs_bytes = (size_t)(n * kTqDim / 8);
  if (norms_bytes) *norms_bytes = (size_t)(n * 4);
  return Q_OK;
}

int qtq_quant_keys(const float* K, int64_t n, int bits, const double* Pi, const double* S, float delta,
                   const uint8_t* table, void* codes, uint32_t* signs, uint32_t* norms, hipStream_t stream) {
  const int st = tq_args_ok(n, 1, bits, delta, table);
  if (st != Q_OK) return st;
  if (!K || !Pi || !S || !codes || !signs || !norms) return Q_EINVAL;
  if (!aligned(K, 4) || !aligned(Pi, 8) || !aligned(S, 8) || !aligned(codes, 4) || !aligned(signs, 4) ||
      !aligned(norms, 4))
    return Q_EALIGN;
  uint32_t tw[4];
  tq_table_words(table, 1 << (bits - 1), tw);
  hipError_t e;
  int* status = qg::pack_status_ptr(&e);
  if (!status) return Q_EHIP;
  if ((e = qg::launch_zero_status(status, stream)) != hipSuccess) return Q_EHIP;
  e = qg::launch_tq_quant(K, n, bits - 1, true, Pi, S, delta, tw, static_cast<uint32_t*>(codes), signs, norms,
                          status, stream);
  if (e != hipSuccess) return Q_EHIP;
  int host = 0;
  if (hipMemcpyAsync(&host, status, sizeof(int), hipMemcpyDeviceToHost, stream) != hipSuccess) return Q_EHIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return Q_EHIP;
  return host ? Q_ERANGE : Q_OK;
}

int qtq_logits_ws(int64_t heads, int64_t nq, size_t* ws_bytes) {
  if (heads < 1 || nq < 1 || nq > 65535 || heads > 65535 || !ws_bytes) return Q_EINVAL;
  *ws_bytes = (size_t)(heads * nq * 132 * 4);
  return Q_OK;
}

int qtq_project(const double* S, const double* Pi, double* SPi, hipStream_t stream) {
  if (!S || !Pi || !SPi) return Q_EINVAL;
  if (!aligned(S, 8) || !aligned(Pi, 8) || !aligned(SPi, 8)) return Q_EALIGN;
  return hip_status(qg::launch_tq_project(S, Pi, SPi, stream));
}

int qtq_logits(const void* codes, const uint32_t* signs, const uint32_t* norms, int64_t n, int64_t heads,
               int bits, float delta, const uint8_t* table, const double* Pi, const double* SPi, const float* Qv,
               int64_t nq, float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = tq_args_ok(n, heads, bits, delta, table);
  if (st != Q_OK) return st;
  size_t need = 0;
  if ((st = qtq_logits_ws(heads, nq, &need)) != Q_OK) return st;
  if (!codes || !signs || !norms || !Pi || !SPi || !Qv || !out) return Q_EINVAL;
  if (!ws || ws_bytes < need) return Q_EWORKSPACE;
  if (!aligned(codes, 4) || !aligned(signs, 4) || !aligned(norms, 4) || !aligned(Pi, 8) || !aligned(SPi, 8) ||
      !aligned(Qv, 4) || !aligned(out, 4) || !aligned(ws, 16))
    return Q_EALIGN;
  if (heads * nq * n > ((int64_t)1 << 40)) return Q_EUNSUPPORTED;
  uint32_t tw[4];
  tq_table_words(table, 1 << (bits - 1), tw);
  return hip_status(qg::launch_tq_logits(static_cast<const uint32_t*>(codes), signs, norms, n, heads, bits - 1,
                                         delta, tw[0], tw[1], Pi, SPi, Qv, nq, out, static_cast<uint32_t*>(ws), stream));
}

int qtq_quant_values(const float* V, int64_t n, int bits, const double* Pi, float delta, const uint8_t* table,
                     void* codes, uint32_t* norms, hipStream_t stream) {
  if (n < 1 || bits < 2 || bits > 4) return Q_EINVAL;
  int st = tq_table_ok(bits, delta, table);
  if (st != Q_OK) return st;
  if (!V || !Pi || !codes || !norms) return Q_EINVAL;
  if (n >= kTqMaxKeys) return Q_EUNSUPPORTED;
  if (!aligned(V, 4) || !aligned(Pi, 8) || !aligned(codes, 4) || !aligned(norms, 4)) return Q_EALIGN;
  uint32_t tw[4];
  tq_table_words(table, 1 << bits, tw);
  hipError_t e;
  int* status = qg::pack_status_ptr(&e);
  if (!status) return Q_EHIP;
  if ((e = qg::launch_zero_status(status, stream)) != hipSuccess) return Q_EHIP;
  e = qg::launch_tq_quant(V, n, bits, false, Pi, nullptr, delta, tw, static_cast<uint32_t*>(codes), nullptr, norms,
                          status, stream);
  if (e != hipSuccess) return Q_EHIP;
  int host = 0;
  if (hipMemcpyAsync(&host, status, sizeof(int), hipMemcpyDeviceToHost, stream) != hipSuccess) return Q_EHIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return Q_EHIP;
  return host ? Q_ERANGE : Q_OK;
}

int qtq_attend_ws(int64_t n, int64_t heads, int64_t nq, size_t* ws_bytes) {
  if (n < 1 || heads < 1 || heads > 65535 || nq < 1 || nq > 65535 || !ws_bytes) return Q_EINVAL;
  if (n >= kTqMaxKeys) return Q_EUNSUPPORTED;
  *ws_bytes = (size_t)(heads * ((nq + 15) / 16) * qg::tq_attend_blocks(n, heads) * 16 * 129 * 4);
  return Q_OK;
}

int qtq_attend(const void* codes, const uint32_t* norms, int64_t n, int64_t heads, int bits, float delta,
               const uint8_t* table, const double* Pi, const float* P, int64_t nq, float* out, void* ws,
               size_t ws_bytes, hipStream_t stream) {
  if (bits < 2 || bits > 4) return Q_EINVAL;
  int st = tq_table_ok(bits, delta, table);
  if (st != Q_OK) return st;
  size_t need = 0;
  if ((st = qtq_attend_ws(n, heads, nq, &need)) != Q_OK) return st;
  if (!codes || !norms || !Pi || !P || !out) return Q_EINVAL;
  if (!ws || ws_bytes < need) return Q_EWORKSPACE;
  if (n * heads > INT32_MAX) return Q_EUNSUPPORTED;
  if (!aligned(codes, 4) || !aligned(norms, 4) || !aligned(Pi, 8) || !aligned(P, 4) || !aligned(out, 4) ||
      !aligned(ws, 16))
    return Q_EALIGN;
  uint32_t tw[4];
  tq_table_words(table, 1 << bits, tw);
  return hip_status(qg::launch_tq_attend(static_cast<const uint32_t*>(codes), norms, n, heads, bits, delta, tw, Pi, P,
                                         nq, out, static_cast<float*>(ws), stream));
}

int qbinlr_sizes(int64_t N, int64_t K, int64_t r, int64_t B, size_t* ubits_bytes,
                 size_t* vtbits_bytes, size_t* ws_bytes) {
  if (N < 1 || K < 1 || r < 1 || N > kMaxDim || K > kMaxDim || r > kMaxDim) return Q_EINVAL;
  if (B < 1 || B > 16) return Q_EINVAL;
  // sign words are addressed through 32-bit buffer offsets
  if (N * padded_words(r) * 4 >= ((int64_t)1 << 32) || r * padded_words(K) * 4 >= ((int64_t)1 << 32))
    return Q_EUNSUPPORTED;
  if (ubits_bytes) *ubits_bytes = (size_t)(N * padded_words(r) * 4);
  if (vtbits_bytes) *vtbits_bytes = (size_t)(r * padded_words(K) * 4);
  if (ws_bytes) *ws_bytes = (size_t)(B * qg::binlr_ws_bytes_per_batch(r));
  return Q_OK;
}

int qpack_binlr(const int8_t* U, const int8_t* V, int64_t N, int64_t K, int64_t r, void* ubits,
                void* vtbits, hipStream_t stream) {
  if (qbinlr_sizes(N, K, r, 1, nullptr, nullptr, nullptr) != Q_OK) return Q_EINVAL;
  if (!U || !V || !ubits || !vtbits) return Q_EINVAL;
  if (!aligned(ubits, 16) || !aligned(vtbits, 16)) return Q_EALIGN;
  hipError_t e;
  int* status = qg::pack_status_ptr(&e);
  if (!status) return Q_EHIP;
  if ((e = qg::launch_zero_status(status, stream)) != hipSuccess) return Q_EHIP;
  e = qg::launch_pack_binlr(U, V, N, K, r, static_cast<uint32_t*>(ubits),
                            static_cast<uint32_t*>(vtbits), status, stream);
  if (e != hipSuccess) return Q_EHIP;
  int host = 0;
  if (hipMemcpyAsync(&host, status, sizeof(int), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return Q_EHIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return Q_EHIP;
  return host ? Q_ERANGE : Q_OK;
}

int qunpack_binlr(const void* ubits, const void* vtbits, int64_t N, int64_t K, int64_t r,
                  int8_t* U_out, int8_t* V_out, hipStream_t stream) {
  if (qbinlr_sizes(N, K, r, 1, nullptr, nullptr, nullptr) != Q_OK) return Q_EINVAL;
  if (!ubits || !vtbits || (!U_out && !V_out)) return Q_EINVAL;
  if (!aligned(ubits, 4) || !aligned(vtbits, 4)) return Q_EALIGN;
  return hip_status(qg::launch_unpack_binlr(static_cast<const uint32_t*>(ubits),
                                            static_cast<const uint32_t*>(vtbits), N, K, r,
                                            U_out, V_out, stream));
}

int qgemv_binlr(const void* ubits, const void* vtbits, const uint16_t* s1, const uint16_t* s2,
                int64_t N, int64_t K, int64_t r, const void* x, int x_dtype, int64_t B, void* y,
                int y_dtype, void* ws, size_t ws_bytes, hipStream_t stream) {
  size_t need = 0;
  const int st = qbinlr_sizes(N, K, r, B, nullptr, nullptr, &need);
  if (st != Q_OK) return st;
  if (!ubits || !vtbits || !s1 || !s2 || !x || !y) return Q_EINVAL;
  if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return Q_EINVAL;
  if (!ws || ws_bytes < need) return Q_EWORKSPACE;
  if (!aligned(ubits, 16) || !aligned(vtbits, 16) || !aligned(ws, 16) || !aligned(x, 4) ||
      !aligned(y, 4) || !aligned(s1, 2) || !aligned(s2, 2))
    return Q_EALIGN;
  return hip_status(qg::launch_gemv_binlr(
      static_cast<const uint32_t*>(ubits), static_cast<const uint32_t*>(vtbits), s1, s2, N, K, r,
      x, x_dtype, B, y, y_dtype, ws, stream));
}

int qgemv_binlr_noalloc(const void* ubits, const void* vtbits, const uint16_t* s1, const uint16_t* s2,
                        int64_t N, int64_t K, int64_t r, const void* x, int x_dtype, int64_t B, void* y,
                        int y_dtype, hipStream_t stream) {
  size_t need = 0;
  const int st = qbinlr_sizes(N, K, r, B, nullptr, nullptr, &need);
  if (st != Q_OK) return st;
  if (!ubits || !vtbits || !s1 || !s2 || !x || !y) return Q_EINVAL;
  if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return Q_EINVAL;
  if (!aligned(ubits, 16) || !aligned(vtbits, 16) || !aligned(x, 4) || !aligned(y, 4) || !aligned(s1, 2) ||
      !aligned(s2, 2))
    return Q_EALIGN;
  if (need > Q_BINLR_NOALLOC_MAX_WS) return Q_EUNSUPPORTED;
  hipError_t e;
  void* ws = qg::binlr_scratch_ptr(&e);
  if (!ws) return Q_EHIP;
  return hip_status(qg::launch_gemv_binlr(
      static_cast<const uint32_t*>(ubits), static_cast<const uint32_t*>(vtbits), s1, s2, N, K, r,
      x, x_dtype, B, y, y_dtype, ws, stream));
}

int qstream_read(const void* buf, size_t bytes, uint32_t* out, hipStream_t stream) {
  if (!buf || !out || bytes == 0 || bytes % 16) return Q_EINVAL;
  if (!aligned(buf, 16) || !aligned(out, 4)) return Q_EALIGN;
  return hip_status(qg::launch_stream_read(buf, (uint64_t)bytes, out, stream));
}

int qgemm_prefill_ws(const qweight* w, int64_t M, size_t* ws_bytes) {
  if (!w || !ws_bytes || M < 1 || M > kMaxDim) return Q_EINVAL;
  if (w->format == Q_FMT_GROUP) {
    const int st = group_args_ok(w->N, w->K, w->bits, w->group);
    if (st != Q_OK) return st;
    *ws_bytes = 0;
    return Q_OK;
  }
  if (w->format == Q_FMT_BINLR) {
    const int st = qbinlr_sizes(w->N, w->K, w->r, 1, nullptr, nullptr, nullptr);
    if (st != Q_OK) return st;
    *ws_bytes = (size_t)qg::gemm_binlr_ws_bytes(M, w->K, w->r);
    return Q_OK;
  }
  return Q_EINVAL;
}

int qgemm_prefill(const qweight* w, const void* X, int x_dtype, int64_t M, void* Y, int y_dtype,
                  void* ws, size_t ws_bytes, hipStream_t stream) {
  size_t need = 0;
  const int st = qgemm_prefill_ws(w, M, &need);
  if (st != Q_OK) return st;
  if (!X || !Y) return Q_EINVAL;
  if (x_dtype != Q_BF16) return Q_EUNSUPPORTED;
  if (!dtype_ok(y_dtype)) return Q_EINVAL;
  if (!aligned(X, 16) || !aligned(Y, 4)) return Q_EALIGN;
  if (M > INT32_MAX) return Q_EUNSUPPORTED;
  if (prefill_dims_ok(M, w->N, w->K, w->format == Q_FMT_BINLR ? padded_words(w->r) * 32 : 0) != Q_OK)
    return Q_EUNSUPPORTED;
  if (w->format == Q_FMT_GROUP) {
    if (!w->codes || !w->meta) return Q_EINVAL;
    if (outlier_args_ok(w->K, w->n_out) != Q_OK || (w->n_out > 0 && (!w->side || !w->oidx))) return Q_EINVAL;
    if (!aligned(w->codes, 16) || !aligned(w->meta, 4) || !aligned(w->side, 2) || !aligned(w->oidx, 4))
      return Q_EALIGN;
    if (w->N * w->n_out > INT32_MAX) return Q_EUNSUPPORTED;
    if (w->books) {
      if (w->n_out > 0 || !w->book_ids) return Q_EINVAL;   // codebooks come without outlier columns
      const int cst = cb_args_ok(w->N, w->K, w->bits, w->group, w->books, w->n_books);
      if (cst != Q_OK) return cst;
      return hip_status(qg::launch_gemm_group_cb(static_cast<const uint32_t*>(w->codes),
                                                 static_cast<const uint32_t*>(w->meta), w->book_ids, w->books,
                                                 w->n_books, w->N, w->K, w->bits, w->group,
                                                 static_cast<const uint16_t*>(X), M, Y, y_dtype, stream));
    }
    return hip_status(qg::launch_gemm_group(static_cast<const uint32_t*>(w->codes),
                                            static_cast<const uint32_t*>(w->meta), w->N, w->K,
                                            w->bits, w->group, static_cast<const uint16_t*>(X),
                                            M, Y, y_dtype, stream, w->side, w->oidx, (int)w->n_out));
  }
  if (!w->ubits || !w->vtbits || !w->s1 || !w->s2) return Q_EINVAL;
  if (w->K % 8) return Q_EUNSUPPORTED;  // 16-byte row loads of X
  if (!ws || ws_bytes < need) return Q_EWORKSPACE;
  if (!aligned(ws, 16) || !aligned(w->ubits, 4) || !aligned(w->vtbits, 4)) return Q_EALIGN;
  return hip_status(qg::launch_gemm_binlr(
      static_cast<const uint32_t*>(w->ubits), static_cast<const uint32_t*>(w->vtbits), w->s1,
      w->s2, w->N, w->K, w->r, static_cast<const uint16_t*>(X), M, Y, y_dtype, ws, stream));
}

}  // extern "C"
