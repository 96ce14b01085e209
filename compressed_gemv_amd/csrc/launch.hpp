// Internal launchers (C++ linkage) called by the C ABI layer after argument
// validation.  Each returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

// Up to four group-RTN matrices with one K, width and group size that share
// x, multiplied in one launch; start[i] is the first launch row of matrix i
// (INT_MAX for i >= nseg).
struct MultiSegs {
  const void* codes[4];
  const void* meta[4];
  void* y[4];
  int64_t nrows[4];
  int start[4];
  int nseg;
};
hipError_t launch_gemv_group_multi(const MultiSegs& ms, int64_t K, int bits, int group, const void* x,
                                   int x_dtype, int64_t B, void* y0, int y_dtype, hipStream_t s);

// status word shared by the packers (per device)
int* pack_status_ptr(hipError_t* err);

hipError_t launch_pack_group(const float* W, int64_t N, int64_t K, int bits, int group,
                             uint32_t* codes, uint32_t* meta, int* status, hipStream_t s);
hipError_t launch_unpack_group(const uint32_t* codes, const uint32_t* meta, int64_t N,
                               int64_t K, int bits, int group, uint8_t* q, float* w,
                               hipStream_t s);
hipError_t launch_pack_binlr(const int8_t* U, const int8_t* V, int64_t N, int64_t K,
                             int64_t r, uint32_t* ubits, uint32_t* vtbits, int* status,
                             hipStream_t s);
hipError_t launch_unpack_binlr(const uint32_t* ubits, const uint32_t* vtbits, int64_t N,
                               int64_t K, int64_t r, int8_t* U, int8_t* V, hipStream_t s);
hipError_t launch_zero_status(int* status, hipStream_t s);

// Outlier side columns (side[N][n_out] fp16 bits at input channels oidx[];
// n_out = 0: none) are optional for the group GEMV and GEMM.
hipError_t launch_gemv_group(const uint32_t* codes, const uint32_t* meta, int64_t N,
                             int64_t K, int bits, int group, const void* x, int x_dtype,
                             int64_t B, void* y, int y_dtype, hipStream_t s,
                             const uint16_t* side = nullptr, const int32_t* oidx = nullptr, int n_out = 0);
hipError_t launch_pack_group_outlier(const float* W, int64_t N, int64_t K, int bits, int group, int n_out,
                                     uint32_t* codes, uint32_t* meta, uint16_t* side, int32_t* idx,
                                     void* ws, int* status, hipStream_t s);
size_t pack_group_outlier_ws_bytes(int64_t K);
hipError_t launch_pack_group_cb(const float* W, int64_t N, int64_t K, int bits, int group, const uint8_t* books,
                                int n_books, uint32_t* codes, uint32_t* meta, uint8_t* book_ids, int* status,
                                hipStream_t s);
void tq_lloyd_max(int d, int m, double* c);
void tq_rotation(int d, const double* G, double* Pi);
hipError_t launch_tq_quant(const float* X, int64_t n, int mbits, bool prod, const double* Pi, const double* S,
                           float delta, const uint32_t* tab, uint32_t* codes, uint32_t* signs, uint32_t* norms,
                           int* status, hipStream_t s);
int64_t tq_attend_blocks(int64_t n, int64_t heads);
hipError_t launch_tq_attend(const uint32_t* codes, const uint32_t* norms, int64_t n, int64_t heads, int mbits,
                            float delta, const uint32_t* tab, const double* Pi, const float* P, int64_t nq,
                            float* out, float* part, hipStream_t s);
hipError_t launch_tq_project(const double* S, const double* Pi, double* SPi, hipStream_t s);
hipError_t launch_tq_logits(const uint32_t* codes, const uint32_t* signs, const uint32_t* norms, int64_t n,
                            int64_t heads, int mbits, float delta, uint32_t tab_lo, uint32_t tab_hi,
                            const double* Pi, const double* SPi, const float* Qv, int64_t nq, float* out,
                            uint32_t* ws, hipStream_t s);
hipError_t launch_gemm_group_cb(const uint32_t* codes, const uint32_t* meta, const uint8_t* book_ids,
                                const uint8_t* books, int n_books, int64_t N, int64_t K, int bits, int group,
                                const uint16_t* X, int64_t M, void* Y, int y_dtype, hipStream_t s);
hipError_t launch_gemv_group_cb(const uint32_t* codes, const uint32_t* meta, const uint8_t* book_ids,
                                const uint8_t* books, int n_books, int64_t N, int64_t K, int bits, int group,
                                const void* x, int x_dtype, int64_t B, void* y, int y_dtype, hipStream_t s);

// Workspace bytes per batch row of qgemv_binlr: the stage-2 table and the
// stage-1 partial sums.
int64_t binlr_ws_bytes_per_batch(int64_t r);
// The per-device scratch array of qgemv_binlr_noalloc (Q_BINLR_NOALLOC_MAX_WS
// bytes): its device address on the current device, looked up once.
void* binlr_scratch_ptr(hipError_t* err);
hipError_t launch_gemv_binlr(const uint32_t* ubits, const uint32_t* vtbits,
                             const uint16_t* s1, const uint16_t* s2, int64_t N, int64_t K,
                             int64_t r, const void* x, int x_dtype, int64_t B, void* y,
                             int y_dtype, void* ws, hipStream_t s);

// Read `bytes` (a multiple of 16) once with 16-byte nontemporal loads.
hipError_t launch_stream_read(const void* buf, uint64_t bytes, uint32_t* out, hipStream_t s);

hipError_t launch_gemm_group(const uint32_t* codes, const uint32_t* meta, int64_t N,
                             int64_t K, int bits, int group, const uint16_t* X, int64_t M,
                             void* Y, int y_dtype, hipStream_t s,
                             const uint16_t* side = nullptr, const int32_t* oidx = nullptr, int n_out = 0);
hipError_t launch_gemm_group_outlier(const uint32_t* codes, const uint32_t* meta, int64_t N, int64_t K,
                                     int bits, int group, const uint16_t* X, int64_t M, void* Y, int y_dtype,
                                     hipStream_t s, const uint16_t* side, const int32_t* oidx, int n_out);
hipError_t launch_gemm_binlr(const uint32_t* ubits, const uint32_t* vtbits,
                             const uint16_t* s1, const uint16_t* s2, int64_t N, int64_t K,
                             int64_t r, const uint16_t* X, int64_t M, void* Y, int y_dtype,
                             void* T_ws, hipStream_t s);
// Bytes of the binary prefill workspace (T) for M token rows.
int64_t gemm_binlr_ws_bytes(int64_t M, int64_t K, int64_t r);

}  // namespace qg
