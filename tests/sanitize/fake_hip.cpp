// A host-only stand-in for the HIP runtime, so the library's host code (the
// C ABI's validation, size queries, dispatch and launch set-up, and the
// host-side fp64 routines) runs on a machine without a GPU under the address
// and undefined-behaviour sanitizers.
//
// Kernel launches are recorded, not run: each one's grid, block and dynamic
// LDS size are checked against the limits of a gfx950 launch, and the tests
// read the count to see that a call rejected by validation launched nothing.
// __device__ variables get host buffers, so hipGetSymbolAddress and the
// status read-back of the packers work on plain memory.  Device pointers
// passed to the library are never dereferenced by host code.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "fake_hip.h"

namespace {

struct Config {
  dim3 grid, block;
  size_t shmem;
  hipStream_t stream;
};

std::vector<Config> g_config;                         // push/pop stack of <<<...>>> configurations
std::map<const void*, std::string> g_kernels;         // host stub -> device name
std::map<const void*, std::vector<unsigned char>> g_vars;   // host shadow -> "device" memory
long g_launches = 0;
long g_bad_launches = 0;
std::string g_last_kernel;
dim3 g_last_grid, g_last_block;

constexpr size_t kMaxLds = 160 * 1024;

}  // namespace

extern "C" {

long fake_hip_launches(void) { return g_launches; }
long fake_hip_bad_launches(void) { return g_bad_launches; }
const char* fake_hip_last_kernel(void) { return g_last_kernel.c_str(); }
unsigned fake_hip_last_grid_x(void) { return g_last_grid.x; }
unsigned fake_hip_last_block_x(void) { return g_last_block.x; }

void** __hipRegisterFatBinary(const void*) {
  static void* handle = nullptr;
  return &handle;
}

void __hipUnregisterFatBinary(void**) {}

void __hipRegisterFunction(void**, const void* hostFunction, char*, const char* deviceName, unsigned int, void*,
                           void*, dim3*, dim3*, int*) {
  g_kernels[hostFunction] = deviceName;
}

void __hipRegisterVar(void**, void* var, char*, char*, int, size_t size, int, int) {
  g_vars[var].assign(size, 0);
}

hipError_t __hipPushCallConfiguration(dim3 grid, dim3 block, size_t shmem, hipStream_t stream) {
  g_config.push_back({grid, block, shmem, stream});
  return hipSuccess;
}

hipError_t __hipPopCallConfiguration(dim3* grid, dim3* block, size_t* shmem, hipStream_t* stream) {
  if (g_config.empty()) return hipErrorInvalidConfiguration;
  const Config c = g_config.back();
  g_config.pop_back();
  *grid = c.grid;
  *block = c.block;
  *shmem = c.shmem;
  *stream = c.stream;
  return hipSuccess;
}

hipError_t hipLaunchKernel(const void* f, dim3 grid, dim3 block, void** args, size_t shmem, hipStream_t) {
  ++g_launches;
  auto it = g_kernels.find(f);
  g_last_kernel = it == g_kernels.end() ? "<unregistered>" : it->second;
  g_last_grid = grid;
  g_last_block = block;
  const unsigned long long threads = (unsigned long long)block.x * block.y * block.z;
  const bool ok = it != g_kernels.end() && args != nullptr && grid.x >= 1 && grid.y >= 1 && grid.z >= 1 &&
                  grid.x <= 0x7fffffffu && grid.y <= 65535 && grid.z <= 65535 && threads >= 1 && threads <= 1024 &&
                  threads % 64 == 0 && shmem <= kMaxLds;
  if (!ok) {
    ++g_bad_launches;
    std::fprintf(stderr, "bad launch of %s: grid %u x %u x %u, block %u x %u x %u, lds %zu\n",
                 g_last_kernel.c_str(), grid.x, grid.y, grid.z, block.x, block.y, block.z, shmem);
    return hipErrorInvalidConfiguration;
  }
  return hipSuccess;
}

hipError_t hipGetLastError(void) { return hipSuccess; }

hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}

hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int) {
  if (attr != hipDeviceAttributeMultiprocessorCount) return hipErrorInvalidValue;
  *value = 256;
  return hipSuccess;
}

hipError_t hipGetSymbolAddress(void** ptr, const void* symbol) {
  auto it = g_vars.find(symbol);
  if (it == g_vars.end()) return hipErrorInvalidSymbol;
  *ptr = it->second.data();
  return hipSuccess;
}

hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind kind, hipStream_t) {
  // only the packers' status read-back: device status word -> host int
  if (kind != hipMemcpyDeviceToHost) return hipErrorInvalidValue;
  for (auto& v : g_vars) {
    const unsigned char* b = v.second.data();
    if (src >= (const void*)b && (const unsigned char*)src + n <= b + v.second.size()) {
      std::memcpy(dst, src, n);
      return hipSuccess;
    }
  }
  return hipErrorInvalidValue;
}

hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

}  // extern "C"
