// Streaming-read reference: the rate at which this GPU's HBM delivers a
// plain read-only stream of the kind of load the GEMV kernels issue (16-byte
// nontemporal loads, one pass, nothing written back).  A decode step is
// bound by the bytes it reads ("AirLLM corre un modelo 70B...", "Por qué es
// lento": time per token ~ bytes / read speed), so this is the ceiling the
// decode kernels are compared with beside the HBM specification.
#include "common.hpp"
#include "launch.hpp"

namespace qg {

namespace {

// A grid-stride loop, one 16-byte load per thread and step, folded with
// xor; the fold is stored only if it equals a constant no realistic buffer
// produces, so no load can be removed.  Of the shapes measured on MI355X
// over 132 MB passes (1 to 16 loads in flight per thread, grid-stride or one
// contiguous span per wave, 256 to 4096 workgroups of 256 threads), this
// one (2048 workgroups, one load per step) read fastest: 19.9 us, 6.6 TB/s.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ p, uint64_t n16,
                                                          uint32_t* __restrict__ out) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const u32x4_t v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9E3779B9u) out[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, uint64_t bytes, uint32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(2048), dim3(256), 0, s, static_cast<const u32x4_t*>(buf), bytes / 16,
                     out);
  return hipGetLastError();
}

}  // namespace qg
