/*
 * qgemv.h - C ABI of the MI355X (gfx950) compressed-weight matrix product.
 *
 * Two weight formats:
 *   group RTN   b-bit codes (b = 2..6) in groups of g = 32 or 64 consecutive
 *               inputs, each group with an fp16 scale s and an fp16 offset o,
 *               w_hat = s*q + o.  Group-wise asymmetric round-to-nearest
 *               ("Métodos de cuantización de LLM para ejecutar un modelo de
 *               70B en una sola GPU", RTN paragraph; "TurboQuant: cuantizar
 *               modelos grandes para que quepan en local", "Compresión por
 *               bloques" and "Asignación de bits por capa").
 *   binary LR   W ~ s1 (.) (U+-1 . V+-1^T) (.) s2^T, U: N x r, V: K x r,
 *               s1 (N) and s2 (K) fp16 channel scales ("70B en 4GB de VRAM:
 *               la compresión neural de 2026, ¿es real?", section 1,
 *               NanoQuant, formulation bullet).
 *
 * Shapes: W has N outputs and K inputs and is stored output-major (the
 * reduction dimension K is contiguous).  Activations x/X are [B][K] or
 * [M][K] row-major; outputs y/Y are [B][N] or [M][N] row-major.
 *
 * Ownership: every data pointer is a DEVICE pointer owned by the caller.
 * The library never allocates or frees device memory.  Entry points that
 * need scratch take a caller-provided workspace whose size comes from the
 * matching *_sizes / *_ws query (host-only functions).
 *
 * Streams: compute calls are asynchronous on the caller's stream.  qpack_*
 * synchronize the stream to report data errors.  Device faults surface at
 * the caller's next synchronization.
 *
 * Errors: every entry point returns Q_OK (0) or a negative status; nothing
 * is launched when argument validation fails.  Launch failures are returned
 * as Q_EHIP.  No exception crosses the ABI.  Calls are reentrant, except
 * that qpack_* calls on one device share a device status word and must not
 * run concurrently with each other.
 *
 * Packed layout (format version 1):
 *   codes  row n is K/32 units of 32 codes; a unit is b little-endian u32
 *          words.  Each 16-bit half of a word holds floor(16/b) b-bit fields
 *          from bit 0 up; regular code c of a unit sits in word c/(2F), half
 *          (c%(2F))/F, field c%F (F = floor(16/b)).  The spare bits above
 *          the fields hold the remaining codes (b = 3, 5: codes 30, 31 with
 *          bit i in word i, bit 15 / bit 31; b = 6: codes 24..31, c = 24+4h+p,
 *          low 4 bits in word p bits 16h+12.., top 2 bits in word 4+p/2 bits
 *          16h+12+2(p%2)..).  N*K*b/8 bytes, no padding.
 *   meta   [N][K/g] u32: bits 0..15 fp16 scale s, bits 16..31 fp16 offset o.
 *   Ubits  [N][rw] u32, U[n][l] = +1 <-> bit (l%32) of word l/32 set.
 *   VTbits [r][Kw] u32, V[k][l] = +1 <-> bit (k%32) of word k/32 of row l.
 *          rw = ceil(r/32), Kw = ceil(K/32), each rounded up to a multiple of
 *          4 words; padding bits are 0 and contribute nothing.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  Q_OK = 0,
  Q_EINVAL = -1,        /* bad shape, null pointer, unsupported parameter value */
  Q_EALIGN = -2,        /* a buffer is not aligned as required below */
  Q_EUNSUPPORTED = -3,  /* valid but not implemented (dtype, size limit) */
  Q_ERANGE = -4,        /* data error: non-finite weight, fp16 overflow, entry not +-1 */
  Q_EWORKSPACE = -5,    /* workspace missing or smaller than the query said */
  Q_EHIP = -6           /* a HIP runtime call or kernel launch failed */
};
enum { Q_F32 = 0, Q_BF16 = 1, Q_F16 = 2 };
enum { Q_FMT_GROUP = 1, Q_FMT_BINLR = 2 };

#define Q_ABI_VERSION 3
#define Q_FORMAT_VERSION 1

int q_abi_version(void);
/* Format version of the packed buffers this library reads and writes. */
int q_format_version(void);
/* Static string for a status code; never NULL. */
const char* q_status_str(int status);

/* ---------------------------------------------------------------- group RTN
 * Byte sizes of the codes and meta buffers (host only, no GPU needed).
 * Requires N >= 1, K >= 1, K % group == 0, bits in 2..6, group in {32, 64}.
 */
int qgroup_sizes(int64_t N, int64_t K, int bits, int group,
                 size_t* codes_bytes, size_t* meta_bytes);

/* Quantize and pack W[N][K] (fp32, device) with group-wise RTN
 * ("Métodos de cuantización...", RTN paragraph; "TurboQuant...",
 * "Compresión por bloques"): per group o = largest fp16 <= min, s = smallest
 * fp16 >= (max - o)/(2^b - 1) (fp64), q = rint((w - o)/s) in fp64, ties to
 * even.  codes and meta must be 16-byte aligned and sized by qgroup_sizes.
 * Synchronizes `stream`; returns Q_ERANGE (buffers then undefined) if a
 * weight is non-finite or a constant leaves the fp16 range. */
int qpack_group(const float* W, int64_t N, int64_t K, int bits, int group,
                void* codes, void* meta, hipStream_t stream);

/* Inverse of the packing, for tests: q_out[N][K] (uint8 codes, required)
 * and, when w_out is not NULL, w_out[N][K] = s*q + o in fp32. Asynchronous. */
int qunpack_group(const void* codes, const void* meta, int64_t N, int64_t K,
                  int bits, int group, uint8_t* q_out, float* w_out,
                  hipStream_t stream);

/* Decode GEMV: y[b][n] = sum_k (s*q[n][k] + o) * x[b][k] for b < B
 * ("AirLLM corre un modelo 70B...", "Por qué es lento": a decode step moves
 * every weight byte once, so it is bound by the bytes read).
 * x: [B][K], x_dtype Q_BF16 or Q_F32; y: [B][N], y_dtype Q_F32 or Q_BF16;
 * accumulation in fp32.  1 <= B <= 16.  codes, meta and x must be 16-byte
 * aligned (the activations are read with 16-byte loads), y 4-byte aligned;
 * Q_EALIGN otherwise.  Batch 1 supports K <= 65536 (bf16 x) or 32768 (fp32
 * x); B > 1 takes bf16 x only and B * K < 2^30 (activation offsets are
 * 32-bit), Q_EUNSUPPORTED otherwise.  Asynchronous on `stream`. */
int qgemv_group(const void* codes, const void* meta, int64_t N, int64_t K,
                int bits, int group, const void* x, int x_dtype, int64_t B,
                void* y, int y_dtype, hipStream_t stream);

/* Several group-RTN matrices that share K, bits, group and the input x
 * (a decoder layer's q, k, v or its gate and up projections), multiplied in
 * one launch (for B > 1 one matrix-core launch over all the matrices' row
 * tiles; each y_i equals a qgemv_group call bit for bit): y_i = x W_i^T for
 * each entry of mats (a HOST array of 1..4 entries; each codes/meta/y as in
 * qgemv_group, y_i [B][N_i]).  Same limits, dtypes and alignment as
 * qgemv_group (x 16-byte aligned); the sum of the N_i is below 2^31.
 * Asynchronous. */
typedef struct qgroup_mat {
  const void* codes;
  const void* meta;
  int64_t N;
  void* y;
} qgroup_mat;
int qgemv_group_multi(const qgroup_mat* mats, int count, int64_t K, int bits, int group,
                      const void* x, int x_dtype, int64_t B, int y_dtype, hipStream_t stream);

/* ------------------------------------------- group RTN with outlier columns
 * Mixed decomposition ("Métodos de cuantización de LLM...", opening and
 * LLM.int8() paragraph: about 0.1 % of the hidden dimensions carry values up
 * to 20x larger; they run in FP16, the rest at low precision, and the two
 * results are added).  The n_out input channels with the largest
 * max_n |W[n][k]| (ties to the lower k) are the outliers, 0 <= n_out <= 64.
 * They are encoded as 0 by the group RTN above (codes and meta as usual),
 * and kept as fp16 columns side[n][j] = fp16(W[n][idx_j] - w_rest[n][idx_j]),
 * the true column minus what the codes reconstruct there (fp64, one
 * rounding to nearest even), so y = W_rest_hat x + side x[idx].
 *   side  [N][n_out] fp16 bits (uint16), row-major.
 *   idx   [n_out] int32, increasing.
 *
 * Workspace bytes of qpack_group_outlier (host only). */
int qgroup_outlier_ws(int64_t K, int64_t n_out, size_t* ws_bytes);

/* Choose the outlier channels, pack the rest as qpack_group does, and
 * write side and idx.  ws: device, >= the qgroup_outlier_ws value, 16-byte
 * aligned; side 2-byte and idx 4-byte aligned.  Synchronizes `stream`;
 * Q_ERANGE on a non-finite weight, an fp16 overflow of a group constant or
 * of a side value. */
int qpack_group_outlier(const float* W, int64_t N, int64_t K, int bits, int group, int64_t n_out,
                        void* codes, void* meta, uint16_t* side, int32_t* idx, void* ws,
                        size_t ws_bytes, hipStream_t stream);

/* qgemv_group plus the outlier term: y[b][n] = sum_k (s*q + o) x[b][k] +
 * sum_j side[n][j] x[b][idx[j]], fp32 accumulation; same arguments, limits
 * and alignment as qgemv_group (x 16-byte aligned; side 2-byte and idx
 * 4-byte aligned; n_out = 0 is qgemv_group).  Asynchronous. */
int qgemv_group_outlier(const void* codes, const void* meta, const uint16_t* side, const int32_t* idx,
                        int64_t n_out, int64_t N, int64_t K, int bits, int group, const void* x,
                        int x_dtype, int64_t B, void* y, int y_dtype, hipStream_t stream);

/* ------------------------------------------ group codes with codebooks
 * Per-group codebooks from a shared dictionary ("TurboQuant: cuantizar
 * modelos grandes para que quepan en local", introduction and "Compresión
 * por bloques": block compression with a shared dictionary; blocks of 32 or
 * 64 weights keep a scale and an offset and a compressed codebook per
 * group).  A dictionary holds n_books (1..16) books of 2^bits byte entries
 * e <= 127, bits = 2, 3 or 4, books[d][j] at byte d*2^bits + j.  Each group
 * stores s and o of the group RTN above and the index of one book in
 * book_ids[N][K/group] (bytes, row-major); code q stands for the level
 * e[q] / 2^(7-bits) in code units, w_hat = s * e[q] / 2^(7-bits) + o.  codes
 * and meta have the format-1 layout and sizes of qgroup_sizes.
 *
 * Default dictionary (host only): 8 books of 2^bits entries written to
 * books (8 * 2^bits bytes): the uniform grid e_j = j * 2^(7-bits) (book 0;
 * a dictionary of that book alone is qpack_group), three books denser near
 * the middle of the group's range, two denser near its minimum and their
 * two mirrors.  *n_books = 8 when n_books is not NULL. */
int qcodebook_default(int bits, uint8_t* books, int* n_books);
/* Encode W[N][K] (fp32, device): per group the RTN constants s, o,
 * u = (w - o)/s in fp64, for every book each weight's nearest level (ties
 * to the even, then the lower index) and the squared error summed in
 * increasing k in fp64; the least-error book (ties to the lower index) and
 * its codes.  books: device.  W, codes, meta 16-byte aligned.  Synchronizes
 * `stream`; Q_ERANGE as qpack_group, Q_EINVAL if a book entry exceeds 127
 * (outputs then undefined). */
int qpack_group_cb(const float* W, int64_t N, int64_t K, int bits, int group, const uint8_t* books,
                   int n_books, void* codes, void* meta, uint8_t* book_ids, hipStream_t stream);
/* Decode GEMV y[b][n] = sum_k (s * e[book][q] / 2^(7-bits) + o) x[b][k],
 * fp32 accumulation; same arguments, limits, dtypes and alignment as
 * qgemv_group (x 16-byte aligned) plus book_ids and books (device, entries
 * <= 127 as qpack_group_cb checks).  Asynchronous. */
int qgemv_group_cb(const void* codes, const void* meta, const uint8_t* book_ids, const uint8_t* books,
                   int n_books, int64_t N, int64_t K, int bits, int group, const void* x, int x_dtype,
                   int64_t B, void* y, int y_dtype, hipStream_t stream);
/* ------------------------------------------------ key-cache quantization
 * Inner-product quantizer for attention keys ("70B en 4GB de VRAM: la
 * compresión neural de 2026, ¿es real?", section 3, TurboQuant): a random
 * orthogonal rotation Pi makes every coordinate of a rotated unit vector
 * follow one known law, so one Lloyd-Max codebook serves all keys with no
 * per-block constants; one more bit per coordinate holds the signs of a
 * Gaussian projection S of the residual, which makes the inner-product
 * estimate unbiased.  Keys are 128-dimensional (d = 128).  bits = 3 or 4
 * bits per coordinate: m = bits - 1 codebook bits plus the sign bit.
 *   codes  [n][4][m] u32: per key, 4 units of 32 coordinates in the
 *          group-code layout of m-bit codes (format 1).
 *   signs  [n][4] u32: bit j of word w <-> coordinate 32w + j, 1 <-> >= 0.
 *   norms  [n] u32: fp16 |x| in bits 0..15, fp16 gamma = |r| in 16..31.
 * Centroid k = delta * (table[k] - 64) with table bytes 1..127 (a 7-bit
 * grid; table is a HOST array of 2^m bytes, delta > 0).  Pi and S are
 * row-major 128 x 128 fp64 DEVICE arrays.
 *
 * Lloyd-Max centroids of the coordinate law of a uniform unit vector in R^d,
 * f(t) ~ (1 - t^2)^((d-3)/2), on the 7-bit grid: delta = max|c| / 63 (fp32),
 * table[k] = nearest integer to c_k / delta, plus 64 (host only; 3 <= d,
 * 1 <= mbits <= 4, table holds 2^mbits bytes). */
int qtq_centroids(int d, int mbits, float* delta, uint8_t* table);
/* Q of G = QR with diag(R) > 0 (modified Gram-Schmidt; host, row-major d x
 * d); with G of i.i.d. N(0, 1) entries, a random rotation.  Q_ERANGE if G is
 * singular. */
int qtq_rotation(int d, const double* G, double* Pi);
/* Byte sizes of codes, signs and norms for n keys (host only).  Every
 * key-cache call takes n < 67108860 per head (one head's data is addressed
 * through 32-bit offsets) and returns Q_EUNSUPPORTED beyond. */
int qtq_sizes(int64_t n, int bits, size_t* codes_bytes, size_t* signs_bytes, size_t* norms_bytes);
/* Encode n keys K[n][128] (fp32, device): y = Pi x / |x|, each coordinate
 * to the nearest centroid (ties to the lower index), residual r = y - c,
 * gamma = |r|, signs of S r; every sum in fp64 in increasing index order,
 * norms rounded to fp16 (nearest even).  Synchronizes `stream`; Q_ERANGE on
 * a non-finite key or a norm beyond fp16. */
int qtq_quant_keys(const float* K, int64_t n, int bits, const double* Pi, const double* S, float delta,
                   const uint8_t* table, void* codes, uint32_t* signs, uint32_t* norms, hipStream_t stream);
/* SPi = S Pi (row-major 128 x 128 fp64, device), formed once per (Pi, S)
 * pair for qtq_logits: S Pi q is then one product.  Asynchronous. */
int qtq_project(const double* S, const double* Pi, double* SPi, hipStream_t stream);
/* Workspace bytes of qtq_logits for `heads` heads of nq queries (host). */
int qtq_logits_ws(int64_t heads, int64_t nq, size_t* ws_bytes);
/* Attention logits from quantized keys: for every head h < heads, query
 * i < nq (Qv[h][i][128], fp32, device) and key j < n of that head (the keys
 * of head h are rows h*n .. h*n + n - 1 of codes/signs/norms),
 *   out[h][i][j] = |x| (<Pi q, c[code]> + gamma sqrt(pi/2)/128 <S Pi q, sign>),
 * with Pi q and S Pi q = SPi q (SPi from qtq_project) formed in fp32 and
 * rounded once to bf16, products accumulated in fp32.  ws: device, >= the
 * qtq_logits_ws value, 16-byte aligned.  Asynchronous. */
int qtq_logits(const void* codes, const uint32_t* signs, const uint32_t* norms, int64_t n, int64_t heads,
               int bits, float delta, const uint8_t* table, const double* Pi, const double* SPi, const float* Qv,
               int64_t nq, float* out, void* ws, size_t ws_bytes, hipStream_t stream);
/* Values (the page's reconstruction variant): bits = 2, 3 or 4 codebook
 * bits per coordinate, no sign bits; codes [n][4][bits] as for keys, norms
 * [n] u32 = fp16 |v| (upper half 0); the table has 2^bits bytes.
 * Encode n values V[n][128] (fp32, device) as the keys' codebook part:
 * y = Pi v / |v|, nearest stored centroid, fp64 sums in increasing index
 * order.  Synchronizes `stream`; Q_ERANGE as qtq_quant_keys. */
int qtq_quant_values(const float* V, int64_t n, int bits, const double* Pi, float delta, const uint8_t* table,
                     void* codes, uint32_t* norms, hipStream_t stream);
/* Workspace bytes of qtq_attend (host); Q_EUNSUPPORTED for n >= 67108860. */
int qtq_attend_ws(int64_t n, int64_t heads, int64_t nq, size_t* ws_bytes);
/* Attention output over quantized values: for head h, query i < nq and
 * weights P[h][i][n] (fp32, device; e.g. the softmax of qtq_logits),
 *   out[h][i][:] = sum_j P[h][i][j] |v_j| Pi^T c[code_j]   (fp32, [heads][nq][128]).
 * Sums over the values in fp32 in the rotated domain, then one Pi^T product.
 * ws: device, >= the qtq_attend_ws value, 16-byte aligned.  Asynchronous. */
int qtq_attend(const void* codes, const uint32_t* norms, int64_t n, int64_t heads, int bits, float delta,
               const uint8_t* table, const double* Pi, const float* P, int64_t nq, float* out, void* ws,
               size_t ws_bytes, hipStream_t stream);
/* ------------------------------------------------------------- binary LR
 * Sizes of Ubits, VTbits and of the qgemv_binlr workspace for batch B
 * (host only).  r >= 1, N >= 1, K >= 1, 1 <= B <= 16. */
int qbinlr_sizes(int64_t N, int64_t K, int64_t r, int64_t B,
                 size_t* ubits_bytes, size_t* vtbits_bytes, size_t* ws_bytes);

/* Pack +-1 factors ("70B en 4GB de VRAM...", section 1, formulation):
 * U[N][r] and V[K][r] int8 (device) -> Ubits[N][rw], VTbits[r][Kw].
 * Synchronizes `stream`; Q_ERANGE if an entry is not +1 or -1. */
int qpack_binlr(const int8_t* U, const int8_t* V, int64_t N, int64_t K,
                int64_t r, void* ubits, void* vtbits, hipStream_t stream);

/* Inverse of qpack_binlr, for tests.  Asynchronous. */
int qunpack_binlr(const void* ubits, const void* vtbits, int64_t N, int64_t K,
                  int64_t r, int8_t* U_out, int8_t* V_out, hipStream_t stream);

/* Binary GEMV in two stages ("70B en 4GB de VRAM...", section 1: the
 * factored form read right to left): t[b] = V^T (s2 (.) x[b]) into the
 * workspace (as bf16 hi + lo parts laid out for the second stage, with
 * partial sums), then y[b] = s1 (.) (U t[b]).  s1, s2: fp16 bits (device).
 * x_dtype Q_BF16 or Q_F32, y_dtype Q_F32 or Q_BF16, 1 <= B <= 16.
 * ws: device, ws_bytes >= the qbinlr_sizes value, 16-byte aligned. */
int qgemv_binlr(const void* ubits, const void* vtbits, const uint16_t* s1,
                const uint16_t* s2, int64_t N, int64_t K, int64_t r,
                const void* x, int x_dtype, int64_t B, void* y, int y_dtype,
                void* ws, size_t ws_bytes, hipStream_t stream);

/* qgemv_binlr without a workspace argument, for callers that cannot
 * allocate device memory (code under stream/graph capture, tight serving
 * loops, harnesses that forbid allocation).  The workspace is a static
 * device array of Q_BINLR_NOALLOC_MAX_WS bytes that the library holds on
 * each GPU it runs on until the process ends; the call allocates nothing.
 * Same arguments, limits and results as qgemv_binlr; Q_EUNSUPPORTED when
 * the workspace qbinlr_sizes reports for (N, K, r, B) exceeds
 * Q_BINLR_NOALLOC_MAX_WS (e.g. r <= 16384 fits at B = 16).  Every call on
 * one GPU uses that GPU's array: calls that may overlap on one GPU (other
 * streams, other host threads) race and must be serialized by the caller.
 * No state carries from one call to the next. */
#define Q_BINLR_NOALLOC_MAX_WS ((size_t)2 << 20)
int qgemv_binlr_noalloc(const void* ubits, const void* vtbits, const uint16_t* s1,
                        const uint16_t* s2, int64_t N, int64_t K, int64_t r,
                        const void* x, int x_dtype, int64_t B, void* y, int y_dtype,
                        hipStream_t stream);

/* ------------------------------------------------------------ measurement
 * Reference for the decode kernels' bandwidth ("AirLLM corre un modelo
 * 70B...", "Por qué es lento": time per token ~ bytes / read speed): read
 * buf (device, 16-byte aligned, bytes a multiple of 16) once with 16-byte
 * nontemporal loads, as a plain read-only stream; *out (device, 4-byte
 * aligned) is written only in the unlikely case that the xor of all words
 * equals 0x9E3779B9, so callers pass a scratch word.  Asynchronous. */
int qstream_read(const void* buf, size_t bytes, uint32_t* out, hipStream_t stream);

/* --------------------------------------------------------------- prefill */
typedef struct qweight {
  int format;                 /* Q_FMT_GROUP or Q_FMT_BINLR */
  int64_t N, K;
  int bits, group;            /* Q_FMT_GROUP */
  const void* codes;
  const void* meta;
  int64_t r;                  /* Q_FMT_BINLR */
  const void* ubits;
  const void* vtbits;
  const uint16_t* s1;
  const uint16_t* s2;
  const uint16_t* side;       /* Q_FMT_GROUP outlier columns [N][n_out] fp16, or NULL */
  const int32_t* oidx;        /* their input channels [n_out] */
  int64_t n_out;              /* 0..64; 0 = none */
  const uint8_t* book_ids;    /* Q_FMT_GROUP with codebooks: [N][K/group] book per group, or NULL */
  const uint8_t* books;       /* the dictionary (n_books x 2^bits bytes), or NULL for plain codes */
  int n_books;                /* 1..16 when books is set (bits 2..4, n_out = 0) */
} qweight;

/* Workspace bytes qgemm_prefill needs for M token rows (host only). */
int qgemm_prefill_ws(const qweight* w, int64_t M, size_t* ws_bytes);

/* Prefill GEMM Y[M][N] = X[M][K] W_hat^T with X bf16 (x_dtype Q_BF16).
 * Group RTN with n_out > 0 adds X[:, oidx] side^T before the output
 * rounding; with books set, the codes are read through the per-group books
 * as in qgemv_group_cb.
 * Weight tiles are decoded to bf16 in LDS and fed to MFMA with fp32
 * accumulation.  Group RTN: one pass.  Binary: T = (X (.) s2) V into the
 * workspace as bf16, then Y = (T U^T) (.) s1 ("70B en 4GB de VRAM...",
 * section 1; the pages' GEMM kernels for this format).  y_dtype Q_F32 or
 * Q_BF16.  Tiles address X and T through 32-bit offsets: K < 2^23, the rank
 * padded to 128 below 2^22, and ceil(M/64) * ceil(N/128) < 2^31, else
 * Q_EUNSUPPORTED.  Asynchronous. */
int qgemm_prefill(const qweight* w, const void* X, int x_dtype, int64_t M,
                  void* Y, int y_dtype, void* ws, size_t ws_bytes,
                  hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* QGEMV_H */
