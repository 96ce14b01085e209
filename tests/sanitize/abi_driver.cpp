// Drives every entry point of the C ABI (include/qgemv.h) on the host, with
// the library's host code built under the address and undefined-behaviour
// sanitizers and linked against the host-only HIP stand-in (fake_hip.cpp):
//   - rejected arguments return the documented status and launch nothing;
//   - accepted arguments launch kernels whose grids, blocks and LDS sizes
//     fit a gfx950 launch, over shapes from one element to the largest the
//     ABI accepts;
//   - the size queries, fuzzed with random and extreme sizes, never overflow;
//   - the host-side fp64 routines (default codebooks, Lloyd-Max centroids,
//     Gram-Schmidt rotation) give the values their definitions fix.
// Device pointers are fake addresses the host code never dereferences.
// Exit status 0 when every check passes; the sanitizers abort on the first
// error they find.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "fake_hip.h"
#include "qgemv.h"

namespace {

int g_fail = 0;
int g_checks = 0;

#define CHECK(cond, ...)                                      \
  do {                                                        \
    ++g_checks;                                               \
    if (!(cond)) {                                            \
      ++g_fail;                                               \
      std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);                      \
      std::fprintf(stderr, "\n");                             \
    }                                                         \
  } while (0)

// distinct 256-byte aligned fake device addresses
void* dp(int i) { return reinterpret_cast<void*>((uintptr_t)0x10000000u + (uintptr_t)i * 0x1000000u); }
template <typename T>
T* dpt(int i) { return static_cast<T*>(dp(i)); }
void* odd(int i) { return static_cast<char*>(dp(i)) + 2; }

const hipStream_t S = nullptr;

// a call that must be rejected with `want` (or any negative status when
// want is 1) without launching a kernel
#define REJECT(want, call)                                                                       \
  do {                                                                                           \
    const long before = fake_hip_launches();                                                     \
    const int st = (call);                                                                       \
    CHECK((want) == 1 ? st < 0 : st == (want), "%s -> %d, expected %d", #call, st, (int)(want)); \
    CHECK(fake_hip_launches() == before, "%s launched a kernel (%s)", #call, fake_hip_last_kernel()); \
  } while (0)

// a call that must be accepted and launch at least one kernel, all in limits
#define ACCEPT(call)                                                                                   \
  do {                                                                                                 \
    const long before = fake_hip_launches(), bad = fake_hip_bad_launches();                            \
    const int st = (call);                                                                             \
    CHECK(st == Q_OK, "%s -> %d (%s)", #call, st, q_status_str(st));                                   \
    CHECK(fake_hip_launches() > before, "%s launched nothing", #call);                                 \
    CHECK(fake_hip_bad_launches() == bad, "%s: launch outside the limits (%s)", #call, fake_hip_last_kernel()); \
  } while (0)

uint64_t g_rng = 0x9E3779B97F4A7C15ull;
uint64_t next() {   // splitmix64
  uint64_t z = (g_rng += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
// sizes spread over every magnitude, negative and zero included
int64_t any_size() {
  const uint64_t r = next();
  switch (r % 8) {
    case 0: return -(int64_t)(next() % 1000);
    case 1: return (int64_t)(next() % 3);
    case 2: return INT64_MAX - (int64_t)(next() % 4);
    case 3: return ((int64_t)1 << (next() % 63)) + (int64_t)(next() % 3) - 1;
    default: return (int64_t)(next() >> (1 + next() % 63));
  }
}

void test_versions() {
  CHECK(q_abi_version() == Q_ABI_VERSION, "abi version");
  CHECK(q_format_version() == Q_FORMAT_VERSION, "format version");
  for (int s = -10; s <= 1; ++s) CHECK(q_status_str(s) != nullptr && std::strlen(q_status_str(s)) > 0, "status %d", s);
}

void test_size_queries() {
  size_t a = 0, b = 0, c = 0;
  for (int bits = 2; bits <= 6; ++bits)
    for (int g : {32, 64}) {
      CHECK(qgroup_sizes(7, 4 * g, bits, g, &a, &b) == Q_OK, "qgroup_sizes");
      CHECK(a == (size_t)7 * 4 * g * bits / 8 && b == (size_t)7 * 4 * 4, "qgroup_sizes values b=%d g=%d", bits, g);
    }
  CHECK(qgroup_sizes(1, 32, 1, 32, &a, &b) == Q_EINVAL, "bits 1");
  CHECK(qgroup_sizes(1, 32, 7, 32, &a, &b) == Q_EINVAL, "bits 7");
  CHECK(qgroup_sizes(1, 32, 4, 16, &a, &b) == Q_EINVAL, "group 16");
  CHECK(qgroup_sizes(1, 48, 4, 32, &a, &b) == Q_EINVAL, "K %% group");
  CHECK(qgroup_sizes(0, 32, 4, 32, &a, &b) == Q_EINVAL, "N 0");
  CHECK(qgroup_sizes((int64_t)1 << 30, (int64_t)1 << 30, 6, 64, &a, &b) == Q_EUNSUPPORTED, "32-bit offsets");
  CHECK(qbinlr_sizes(70, 300, 37, 1, &a, &b, &c) == Q_OK, "qbinlr_sizes");
  CHECK(a == 70 * 4 * 4 && b == 37 * 12 * 4 && c > 0, "qbinlr_sizes values %zu %zu %zu", a, b, c);
  CHECK(qbinlr_sizes(70, 300, 37, 17, &a, &b, &c) == Q_EINVAL, "B 17");
  CHECK(qtq_sizes(10, 4, &a, &b, &c) == Q_OK && a == 10 * 48 && b == 10 * 16 && c == 40, "qtq_sizes");
  // fuzz: every size query with sizes of every magnitude
  for (int it = 0; it < 200000; ++it) {
    const int64_t N = any_size(), K = any_size(), r = any_size(), B = any_size(), M = any_size();
    const int bits = (int)(next() % 9) - 1, group = (int)(16 << (next() % 4));
    qgroup_sizes(N, K, bits, group, &a, &b);
    qbinlr_sizes(N, K, r, B, &a, &b, &c);
    qtq_sizes(N, bits, &a, &b, &c);
    qtq_logits_ws(N, K, &a);
    qtq_attend_ws(N, K, r, &a);
    qgroup_outlier_ws(K, r, &a);
    qweight w{};
    w.format = (int)(next() % 3);
    w.N = N;
    w.K = K;
    w.bits = bits;
    w.group = group;
    w.r = r;
    qgemm_prefill_ws(&w, M, &a);
  }
}

void test_codebooks() {
  uint8_t books[8 * 16];
  int n = 0;
  for (int bits = 2; bits <= 4; ++bits) {
    std::memset(books, 0xFF, sizeof books);
    CHECK(qcodebook_default(bits, books, &n) == Q_OK && n == 8, "qcodebook_default %d", bits);
    const int L = 1 << bits, unit = 1 << (7 - bits);
    for (int j = 0; j < L; ++j) CHECK(books[j] == j * unit, "book 0 is the uniform grid (bits %d, j %d)", bits, j);
    for (int d = 0; d < 8; ++d) {
      CHECK(books[d * L] == 0 && books[d * L + L - 1] == (L - 1) * unit, "book %d spans the range", d);
      for (int j = 1; j < L; ++j) CHECK(books[d * L + j] >= books[d * L + j - 1], "book %d monotone", d);
      for (int j = 0; j < L; ++j) CHECK(books[d * L + j] <= 127, "7-bit grid");
    }
    // books 6, 7 mirror books 4, 5: e'[j] = top - e[L-1-j] (up to one rounding step)
    for (int p = 0; p < 2; ++p)
      for (int j = 0; j < L; ++j) {
        const int m = (L - 1) * unit - books[(4 + p) * L + L - 1 - j];
        CHECK(std::abs(books[(6 + p) * L + j] - m) <= 1, "mirror book %d j %d", 6 + p, j);
      }
  }
  REJECT(Q_EINVAL, qcodebook_default(1, books, &n));
  REJECT(Q_EINVAL, qcodebook_default(5, books, &n));
  REJECT(Q_EINVAL, qcodebook_default(3, nullptr, &n));
}

void test_centroids_and_rotation() {
  float delta = 0.0f;
  uint8_t table[16];
  for (int m = 1; m <= 4; ++m) {
    CHECK(qtq_centroids(128, m, &delta, table) == Q_OK, "qtq_centroids m=%d", m);
    const int L = 1 << m;
    CHECK(delta > 0.0f, "delta > 0");
    bool ext = false;
    for (int k = 0; k < L; ++k) {
      CHECK(table[k] >= 1 && table[k] <= 127, "table range");
      CHECK(table[k] + table[L - 1 - k] == 128, "centroids symmetric about 0 (m=%d k=%d)", m, k);
      if (k) CHECK(table[k] > table[k - 1], "increasing");
      ext |= table[k] == 1 || table[k] == 127;
    }
    CHECK(ext, "the largest centroid sits on the grid's end (delta = max|c| / 63)");
  }
  // one bit: the two centroids are +-E|t| = +-Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))
  CHECK(qtq_centroids(128, 1, &delta, table) == Q_OK, "m=1");
  const double c1 = std::exp(std::lgamma(64.0) - std::lgamma(64.5)) / std::sqrt(M_PI);
  CHECK(std::fabs(63.0 * delta - c1) < 1e-6 * c1, "one-bit centroid %.9f vs %.9f", 63.0 * delta, c1);
  REJECT(Q_EINVAL, qtq_centroids(2, 2, &delta, table));
  REJECT(Q_EINVAL, qtq_centroids(128, 0, &delta, table));
  REJECT(Q_EINVAL, qtq_centroids(128, 5, &delta, table));

  const int d = 128;
  std::vector<double> G(d * d), Q(d * d);
  for (auto& v : G) v = (double)(int64_t)(next() % 2000001) / 1e6 - 1.0;
  CHECK(qtq_rotation(d, G.data(), Q.data()) == Q_OK, "qtq_rotation");
  double worst = 0.0;
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) {
      double s = 0.0;
      for (int k = 0; k < d; ++k) s += Q[k * d + i] * Q[k * d + j];
      worst = std::fmax(worst, std::fabs(s - (i == j ? 1.0 : 0.0)));
    }
  CHECK(worst < 1e-10, "Q^T Q = I (%.3e)", worst);
  // R = Q^T G is upper triangular with a positive diagonal
  for (int i = 0; i < d; ++i)
    for (int j = 0; j <= i; ++j) {
      double s = 0.0;
      for (int k = 0; k < d; ++k) s += Q[k * d + i] * G[k * d + j];
      if (j < i) CHECK(std::fabs(s) < 1e-9, "R lower part (%d,%d) %.3e", i, j, s);
      else CHECK(s > 0.0, "R diagonal %d", i);
    }
  for (int i = 0; i < d; ++i) G[i * d + 5] = 0.0;   // a zero column: singular
  REJECT(Q_ERANGE, qtq_rotation(d, G.data(), Q.data()));
  REJECT(Q_EINVAL, qtq_rotation(0, G.data(), Q.data()));
}

// The batched GEMV's workgroup counts: row tiles per workgroup chosen so
// the workgroups spread evenly over 256 CUs (7 tiles of 16 rows at N = 28672,
// 4 for 3-bit codes, 2 at 8192, 1 at 1024; grouped launches count the
// matrices' tiles together), 4 waves each.
void test_tile_choice() {
  struct Case { int64_t N; int bits, g; unsigned grid; };
  for (const Case& c : {Case{28672, 4, 64, 256}, Case{28672, 2, 32, 256}, Case{28672, 3, 32, 448},
                        Case{8192, 6, 32, 256}, Case{1024, 4, 64, 64}, Case{28600, 4, 64, 256}}) {
    ACCEPT(qgemv_group(dp(2), dp(3), c.N, 8192, c.bits, c.g, dp(6), Q_BF16, 16, dp(7), Q_F32, S));
    CHECK(fake_hip_last_grid_x() == c.grid && fake_hip_last_block_x() == 256,
          "batched GEMV N %lld %d-bit: grid %u block %u, expected grid %u", (long long)c.N, c.bits,
          fake_hip_last_grid_x(), fake_hip_last_block_x(), c.grid);
  }
  qgroup_mat qkv[3] = {{dp(2), dp(3), 8192, dp(7)}, {dp(8), dp(9), 1024, dp(10)}, {dp(11), dp(12), 1024, dp(13)}};
  const long before = fake_hip_launches();
  ACCEPT(qgemv_group_multi(qkv, 3, 8192, 4, 64, dp(6), Q_BF16, 16, Q_F32, S));
  CHECK(fake_hip_launches() == before + 1, "grouped batched GEMV: %ld launches", fake_hip_launches() - before);
  CHECK(fake_hip_last_grid_x() == 160, "grouped q/k/v: grid %u, expected 160 (4 tiles each)", fake_hip_last_grid_x());
}

void test_group_paths() {
  for (int bits = 2; bits <= 6; ++bits)
    for (int g : {32, 64})
      for (int64_t N : {1, 7, 64, 1000, 28672})
        for (int64_t K : {(int64_t)g, (int64_t)3 * g, (int64_t)8192, (int64_t)28672, (int64_t)65536}) {
          if (K % g) continue;
          ACCEPT(qpack_group(dpt<float>(1), N, K, bits, g, dp(2), dp(3), S));
          ACCEPT(qunpack_group(dp(2), dp(3), N, K, bits, g, dpt<uint8_t>(4), dpt<float>(5), S));
          for (int64_t B : {1, 2, 5, 8, 16})
            for (int yd : {Q_F32, Q_BF16}) {
              if (B == 1 && K > 65536) continue;
              ACCEPT(qgemv_group(dp(2), dp(3), N, K, bits, g, dp(6), Q_BF16, B, dp(7), yd, S));
            }
          if (K <= 32768) ACCEPT(qgemv_group(dp(2), dp(3), N, K, bits, g, dp(6), Q_F32, 1, dp(7), Q_F32, S));
        }
  // rejected arguments
  REJECT(Q_EINVAL, qpack_group(nullptr, 8, 64, 4, 64, dp(2), dp(3), S));
  REJECT(Q_EALIGN, qpack_group(dpt<float>(1), 8, 64, 4, 64, odd(2), dp(3), S));
  REJECT(Q_EINVAL, qgemv_group(dp(2), dp(3), 8, 64, 4, 64, dp(6), Q_BF16, 0, dp(7), Q_F32, S));
  REJECT(Q_EINVAL, qgemv_group(dp(2), dp(3), 8, 64, 4, 64, dp(6), Q_BF16, 17, dp(7), Q_F32, S));
  REJECT(Q_EINVAL, qgemv_group(dp(2), dp(3), 8, 64, 4, 64, dp(6), 7, 1, dp(7), Q_F32, S));
  REJECT(Q_EALIGN, qgemv_group(dp(2), dp(3), 8, 64, 4, 64, static_cast<char*>(dp(6)) + 8, Q_BF16, 1, dp(7), Q_F32, S));
  REJECT(Q_EALIGN, qgemv_group(dp(2), dp(3), 8, 64, 4, 64, dp(6), Q_BF16, 1, static_cast<char*>(dp(7)) + 2, Q_F32, S));
  REJECT(Q_EUNSUPPORTED, qgemv_group(dp(2), dp(3), 8, 65536 + 64, 4, 64, dp(6), Q_BF16, 1, dp(7), Q_F32, S));
  REJECT(Q_EUNSUPPORTED, qgemv_group(dp(2), dp(3), 8, 32768 + 64, 4, 64, dp(6), Q_F32, 1, dp(7), Q_F32, S));
  REJECT(Q_EUNSUPPORTED, qgemv_group(dp(2), dp(3), 8, 64, 4, 64, dp(6), Q_F32, 2, dp(7), Q_F32, S));
  REJECT(Q_EINVAL, qgemv_group(dp(2), dp(3), 8, 96, 4, 64, dp(6), Q_BF16, 1, dp(7), Q_F32, S));
  REJECT(Q_EINVAL, qunpack_group(dp(2), dp(3), 8, 64, 4, 64, nullptr, nullptr, S));

  // several matrices sharing x
  qgroup_mat mats[4] = {{dp(2), dp(3), 8192, dp(7)}, {dp(8), dp(9), 1024, dp(10)},
                        {dp(11), dp(12), 1024, dp(13)}, {dp(14), dp(15), 28672, dp(16)}};
  for (int count = 1; count <= 4; ++count)
    for (int64_t B : {1, 4, 16}) ACCEPT(qgemv_group_multi(mats, count, 8192, 4, 64, dp(6), Q_BF16, B, Q_F32, S));
  REJECT(Q_EINVAL, qgemv_group_multi(mats, 0, 8192, 4, 64, dp(6), Q_BF16, 1, Q_F32, S));
  REJECT(Q_EINVAL, qgemv_group_multi(mats, 5, 8192, 4, 64, dp(6), Q_BF16, 1, Q_F32, S));
  qgroup_mat badm[2] = {{dp(2), dp(3), 64, dp(7)}, {dp(8), nullptr, 64, dp(10)}};
  REJECT(Q_EINVAL, qgemv_group_multi(badm, 2, 8192, 4, 64, dp(6), Q_BF16, 1, Q_F32, S));

  // outlier columns
  size_t ws = 0;
  for (int64_t n_out : {0, 1, 8, 64}) {
    CHECK(qgroup_outlier_ws(8192, n_out, &ws) == Q_OK, "qgroup_outlier_ws");
    ACCEPT(qpack_group_outlier(dpt<float>(1), 1000, 8192, 4, 64, n_out, dp(2), dp(3), dpt<uint16_t>(4),
                               dpt<int32_t>(5), dp(6), ws, S));
    for (int64_t B : {1, 3, 16})
      ACCEPT(qgemv_group_outlier(dp(2), dp(3), dpt<uint16_t>(4), dpt<int32_t>(5), n_out, 1000, 8192, 4, 64, dp(6),
                                 Q_BF16, B, dp(7), Q_F32, S));
  }
  REJECT(Q_EINVAL, qgroup_outlier_ws(8192, 65, &ws));
  REJECT(Q_EWORKSPACE, qpack_group_outlier(dpt<float>(1), 1000, 8192, 4, 64, 8, dp(2), dp(3), dpt<uint16_t>(4),
                                           dpt<int32_t>(5), dp(6), 16, S));
  REJECT(Q_EINVAL, qgemv_group_outlier(dp(2), dp(3), nullptr, dpt<int32_t>(5), 8, 1000, 8192, 4, 64, dp(6), Q_BF16, 1,
                                       dp(7), Q_F32, S));

  // codebooks (the books pointer is a device array; the host never reads it)
  for (int bits = 2; bits <= 4; ++bits)
    for (int nb : {1, 8, 16}) {
      ACCEPT(qpack_group_cb(dpt<float>(1), 1000, 8192, bits, 64, dpt<uint8_t>(20), nb, dp(2), dp(3),
                            dpt<uint8_t>(4), S));
      for (int64_t B : {1, 16})
        ACCEPT(qgemv_group_cb(dp(2), dp(3), dpt<uint8_t>(4), dpt<uint8_t>(20), nb, 1000, 8192, bits, 64, dp(6),
                              Q_BF16, B, dp(7), Q_BF16, S));
    }
  REJECT(Q_EINVAL, qgemv_group_cb(dp(2), dp(3), dpt<uint8_t>(4), dpt<uint8_t>(20), 17, 1000, 8192, 4, 64, dp(6), Q_BF16,
                                  1, dp(7), Q_F32, S));
  REJECT(Q_EINVAL, qpack_group_cb(dpt<float>(1), 1000, 8192, 5, 64, dpt<uint8_t>(20), 8, dp(2), dp(3),
                                  dpt<uint8_t>(4), S));
}

void test_binlr_paths() {
  size_t ub = 0, vb = 0, ws = 0;
  for (int64_t N : {1, 70, 4096, 28672})
    for (int64_t K : {1, 8, 300, 8192, 28672})
      for (int64_t r : {1, 31, 37, 512, 4096, 8192}) {
        CHECK(qbinlr_sizes(N, K, r, 16, &ub, &vb, &ws) == Q_OK, "qbinlr_sizes %lld %lld %lld", (long long)N,
              (long long)K, (long long)r);
        ACCEPT(qpack_binlr(dpt<int8_t>(1), dpt<int8_t>(2), N, K, r, dp(3), dp(4), S));
        ACCEPT(qunpack_binlr(dp(3), dp(4), N, K, r, dpt<int8_t>(1), dpt<int8_t>(2), S));
        for (int64_t B : {1, 2, 3, 8, 16})
          for (int xd : {Q_BF16, Q_F32}) {
            CHECK(qbinlr_sizes(N, K, r, B, nullptr, nullptr, &ws) == Q_OK, "ws");
            ACCEPT(qgemv_binlr(dp(3), dp(4), dpt<uint16_t>(5), dpt<uint16_t>(6), N, K, r, dp(7), xd, B, dp(8), Q_F32,
                               dp(9), ws, S));
            if (ws <= Q_BINLR_NOALLOC_MAX_WS)
              ACCEPT(qgemv_binlr_noalloc(dp(3), dp(4), dpt<uint16_t>(5), dpt<uint16_t>(6), N, K, r, dp(7), xd, B,
                                         dp(8), Q_BF16, S));
            else
              REJECT(Q_EUNSUPPORTED, qgemv_binlr_noalloc(dp(3), dp(4), dpt<uint16_t>(5), dpt<uint16_t>(6), N, K, r,
                                                         dp(7), xd, B, dp(8), Q_BF16, S));
          }
      }
  CHECK(qbinlr_sizes(70, 300, 37, 1, nullptr, nullptr, &ws) == Q_OK, "ws");
  REJECT(Q_EWORKSPACE, qgemv_binlr(dp(3), dp(4), dpt<uint16_t>(5), dpt<uint16_t>(6), 70, 300, 37, dp(7), Q_BF16, 1,
                                   dp(8), Q_F32, dp(9), ws - 16, S));
  REJECT(Q_EWORKSPACE, qgemv_binlr(dp(3), dp(4), dpt<uint16_t>(5), dpt<uint16_t>(6), 70, 300, 37, dp(7), Q_BF16, 1,
                                   dp(8), Q_F32, nullptr, ws, S));
  REJECT(Q_EALIGN, qgemv_binlr(odd(3), dp(4), dpt<uint16_t>(5), dpt<uint16_t>(6), 70, 300, 37, dp(7), Q_BF16, 1,
                               dp(8), Q_F32, dp(9), ws, S));
  REJECT(Q_EINVAL, qgemv_binlr(dp(3), dp(4), nullptr, dpt<uint16_t>(6), 70, 300, 37, dp(7), Q_BF16, 1, dp(8), Q_F32,
                               dp(9), ws, S));
  REJECT(Q_EINVAL, qgemv_binlr_noalloc(dp(3), dp(4), dpt<uint16_t>(5), dpt<uint16_t>(6), 70, 300, 37, dp(7), Q_BF16,
                                       0, dp(8), Q_F32, S));
  REJECT(Q_EUNSUPPORTED, qgemv_binlr_noalloc(dp(3), dp(4), dpt<uint16_t>(5), dpt<uint16_t>(6), 70, 300, 65536, dp(7),
                                             Q_BF16, 16, dp(8), Q_F32, S));
  REJECT(Q_EINVAL, qpack_binlr(dpt<int8_t>(1), dpt<int8_t>(2), 70, 300, 0, dp(3), dp(4), S));
}

void test_prefill_paths() {
  size_t ws = 0;
  for (int64_t M : {1, 17, 512, 4096, 65536})
    for (int64_t K : {64, 448, 576, 8192, 28672})
      for (int64_t N : {1, 130, 8192, 28672}) {
        qweight w{};
        w.format = Q_FMT_GROUP;
        w.N = N;
        w.K = K;
        w.bits = 4;
        w.group = 64;
        w.codes = dp(2);
        w.meta = dp(3);
        CHECK(qgemm_prefill_ws(&w, M, &ws) == Q_OK && ws == 0, "group prefill needs no workspace");
        for (int yd : {Q_F32, Q_BF16}) ACCEPT(qgemm_prefill(&w, dp(6), Q_BF16, M, dp(7), yd, nullptr, 0, S));
        w.side = dpt<uint16_t>(4);
        w.oidx = dpt<int32_t>(5);
        w.n_out = 8;
        ACCEPT(qgemm_prefill(&w, dp(6), Q_BF16, M, dp(7), Q_F32, nullptr, 0, S));
        w.side = nullptr;
        w.oidx = nullptr;
        w.n_out = 0;
        w.book_ids = dpt<uint8_t>(4);
        w.books = dpt<uint8_t>(20);
        w.n_books = 8;
        ACCEPT(qgemm_prefill(&w, dp(6), Q_BF16, M, dp(7), Q_F32, nullptr, 0, S));
        w.n_out = 8;
        REJECT(Q_EINVAL, qgemm_prefill(&w, dp(6), Q_BF16, M, dp(7), Q_F32, nullptr, 0, S));

        for (int64_t r : {8, 100, 4096}) {
          qweight b{};
          b.format = Q_FMT_BINLR;
          b.N = N;
          b.K = K;
          b.r = r;
          b.ubits = dp(2);
          b.vtbits = dp(3);
          b.s1 = dpt<uint16_t>(4);
          b.s2 = dpt<uint16_t>(5);
          CHECK(qgemm_prefill_ws(&b, M, &ws) == Q_OK && ws > 0, "binary prefill workspace");
          ACCEPT(qgemm_prefill(&b, dp(6), Q_BF16, M, dp(7), Q_F32, dp(8), ws, S));
          REJECT(Q_EWORKSPACE, qgemm_prefill(&b, dp(6), Q_BF16, M, dp(7), Q_F32, dp(8), ws - 1, S));
        }
      }
  qweight w{};
  w.format = Q_FMT_GROUP;
  w.N = 64;
  w.K = 64;
  w.bits = 4;
  w.group = 64;
  w.codes = dp(2);
  w.meta = dp(3);
  REJECT(Q_EUNSUPPORTED, qgemm_prefill(&w, dp(6), Q_F32, 4, dp(7), Q_F32, nullptr, 0, S));
  REJECT(Q_EALIGN, qgemm_prefill(&w, static_cast<char*>(dp(6)) + 8, Q_BF16, 4, dp(7), Q_F32, nullptr, 0, S));
  REJECT(Q_EINVAL, qgemm_prefill(&w, dp(6), Q_BF16, 0, dp(7), Q_F32, nullptr, 0, S));
  w.format = 9;
  REJECT(Q_EINVAL, qgemm_prefill(&w, dp(6), Q_BF16, 4, dp(7), Q_F32, nullptr, 0, S));
  qweight b{};
  b.format = Q_FMT_BINLR;
  b.N = 64;
  b.K = 100;   // not a multiple of 8
  b.r = 64;
  b.ubits = dp(2);
  b.vtbits = dp(3);
  b.s1 = dpt<uint16_t>(4);
  b.s2 = dpt<uint16_t>(5);
  size_t need = 0;
  CHECK(qgemm_prefill_ws(&b, 4, &need) == Q_OK, "ws");
  REJECT(Q_EUNSUPPORTED, qgemm_prefill(&b, dp(6), Q_BF16, 4, dp(7), Q_F32, dp(8), need, S));
}

void test_key_cache_paths() {
  float delta = 0.0f, vdelta = 0.0f;
  uint8_t table[16], vtable[16];
  CHECK(qtq_centroids(128, 3, &delta, table) == Q_OK, "centroids");
  CHECK(qtq_centroids(128, 3, &vdelta, vtable) == Q_OK, "centroids");
  for (int64_t n : {1, 3, 1000, 131072})
    for (int bits : {3, 4}) {
      uint8_t t[16];
      CHECK(qtq_centroids(128, bits - 1, &delta, t) == Q_OK, "centroids");
      ACCEPT(qtq_quant_keys(dpt<float>(1), n, bits, dpt<double>(2), dpt<double>(3), delta, t, dp(4),
                            dpt<uint32_t>(5), dpt<uint32_t>(6), S));
      for (int64_t H : {1, 8})
        for (int64_t nq : {1, 4, 16, 18}) {
          size_t ws = 0;
          CHECK(qtq_logits_ws(H, nq, &ws) == Q_OK, "logits ws");
          ACCEPT(qtq_logits(dp(4), dpt<uint32_t>(5), dpt<uint32_t>(6), n, H, bits, delta, t, dpt<double>(2),
                            dpt<double>(7), dpt<float>(8), nq, dpt<float>(9), dp(10), ws, S));
          REJECT(Q_EWORKSPACE, qtq_logits(dp(4), dpt<uint32_t>(5), dpt<uint32_t>(6), n, H, bits, delta, t,
                                          dpt<double>(2), dpt<double>(7), dpt<float>(8), nq, dpt<float>(9), dp(10),
                                          ws - 4, S));
        }
    }
  for (int vbits = 2; vbits <= 4; ++vbits) {
    uint8_t t[16];
    CHECK(qtq_centroids(128, vbits, &vdelta, t) == Q_OK, "value centroids");
    for (int64_t n : {1, 5, 20000, 131072}) {
      ACCEPT(qtq_quant_values(dpt<float>(1), n, vbits, dpt<double>(2), vdelta, t, dp(4), dpt<uint32_t>(6), S));
      for (int64_t H : {1, 8})
        for (int64_t nq : {1, 16, 18}) {
          size_t ws = 0;
          CHECK(qtq_attend_ws(n, H, nq, &ws) == Q_OK, "attend ws");
          ACCEPT(qtq_attend(dp(4), dpt<uint32_t>(6), n, H, vbits, vdelta, t, dpt<double>(2), dpt<float>(8), nq,
                            dpt<float>(9), dp(10), ws, S));
        }
    }
  }
  ACCEPT(qtq_project(dpt<double>(1), dpt<double>(2), dpt<double>(3), S));
  REJECT(Q_EALIGN, qtq_project(dpt<double>(1), reinterpret_cast<const double*>(static_cast<char*>(dp(2)) + 4),
                               dpt<double>(3), S));
  uint8_t bad[16];
  std::memcpy(bad, table, 16);
  bad[0] = 0;   // off the 7-bit grid
  REJECT(Q_EINVAL, qtq_quant_keys(dpt<float>(1), 10, 4, dpt<double>(2), dpt<double>(3), delta, bad, dp(4),
                                  dpt<uint32_t>(5), dpt<uint32_t>(6), S));
  REJECT(Q_EINVAL, qtq_quant_keys(dpt<float>(1), 10, 4, dpt<double>(2), dpt<double>(3), -1.0f, table, dp(4),
                                  dpt<uint32_t>(5), dpt<uint32_t>(6), S));
  REJECT(Q_EINVAL, qtq_quant_keys(dpt<float>(1), 10, 5, dpt<double>(2), dpt<double>(3), delta, table, dp(4),
                                  dpt<uint32_t>(5), dpt<uint32_t>(6), S));
}

void test_stream_read() {
  ACCEPT(qstream_read(dp(1), 132120576, dpt<uint32_t>(2), S));
  ACCEPT(qstream_read(dp(1), 16, dpt<uint32_t>(2), S));
  REJECT(Q_EINVAL, qstream_read(dp(1), 100, dpt<uint32_t>(2), S));
  REJECT(Q_EINVAL, qstream_read(dp(1), 0, dpt<uint32_t>(2), S));
  REJECT(Q_EALIGN, qstream_read(odd(1), 32, dpt<uint32_t>(2), S));
}

}  // namespace

int main() {
  test_versions();
  test_size_queries();
  test_codebooks();
  test_centroids_and_rotation();
  test_group_paths();
  test_tile_choice();
  test_binlr_paths();
  test_prefill_paths();
  test_key_cache_paths();
  test_stream_read();
  std::printf("%d checks, %d failed, %ld launches recorded, %ld outside the limits\n", g_checks, g_fail,
              fake_hip_launches(), fake_hip_bad_launches());
  return g_fail == 0 && fake_hip_bad_launches() == 0 ? 0 : 1;
}
