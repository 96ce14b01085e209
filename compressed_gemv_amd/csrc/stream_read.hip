// Streaming-read reference: the rate at which this GPU's HBM delivers a
// plain read-only stream to the same kind of load the GEMV kernels issue
// (16-byte nontemporal loads, one pass, nothing written back).  A decode step
// is bound by the bytes it reads ("AirLLM corre un modelo 70B...", "Por qué
// es lento": time per token ~ bytes / read speed), so this is the ceiling the
// decode kernels are compared with beside the HBM specification.
#include "common.hpp"
#include "launch.hpp"

namespace qg {

namespace {

// Each thread reads UNR 16-byte words per iteration of a grid-stride loop
// over n16 words and folds them with xor; the fold is stored only if it
// equals a constant no realistic buffer produces, so no load can be removed.
constexpr int kUnroll = 4;

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ p, uint64_t n16,
                                                          uint32_t* __restrict__ out) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9E3779B9u) out[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, uint64_t bytes, uint32_t* out, hipStream_t s) {
  // 1024 workgroups of 4 waves: four waves per SIMD on 256 CUs
  hipLaunchKernelGGL(stream_read_kernel, dim3(1024), dim3(256), 0, s, static_cast<const u32x4_t*>(buf), bytes / 16,
                     out);
  return hipGetLastError();
}

}  // namespace qg
