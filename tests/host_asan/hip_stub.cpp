// Host stand-in for the HIP runtime, for the host-only sanitizer build of the library (test
// infrastructure).  Device memory is host memory, kernel launches are checked for sane launch shapes
// and counted but not run, events and streams are no-ops.  Nothing here touches a GPU.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>

namespace {
std::atomic<long> g_launches{0}, g_bad_launches{0}, g_allocs{0};
dim3 g_grid, g_block;
size_t g_shmem = 0;
}  // namespace

extern "C" long stub_launches() { return g_launches.load(); }
extern "C" long stub_bad_launches() { return g_bad_launches.load(); }
extern "C" long stub_live_allocs() { return g_allocs.load(); }

extern "C" void** __hipRegisterFatBinary(const void*) {
  static void* handle = nullptr;
  return &handle;
}
extern "C" void __hipRegisterFunction(void**, const void*, char*, const char*, unsigned int, void*, void*, dim3*,
                                      dim3*, int*) {}
extern "C" void __hipRegisterVar(void**, void*, char*, char*, int, size_t, int, int) {}
extern "C" void __hipUnregisterFatBinary(void**) {}
extern "C" hipError_t __hipPushCallConfiguration(dim3 grid, dim3 block, size_t shmem, hipStream_t) {
  g_grid = grid;
  g_block = block;
  g_shmem = shmem;
  return hipSuccess;
}
extern "C" hipError_t __hipPopCallConfiguration(dim3* grid, dim3* block, size_t* shmem, hipStream_t* stream) {
  *grid = g_grid;
  *block = g_block;
  *shmem = g_shmem;
  if (stream) *stream = nullptr;
  return hipSuccess;
}

hipError_t hipLaunchKernel(const void*, dim3 grid, dim3 block, void**, size_t shmem, hipStream_t) {
  ++g_launches;
  const unsigned long long threads = (unsigned long long)block.x * block.y * block.z;
  if (grid.x == 0 || grid.y == 0 || grid.z == 0 || grid.y > 65535 || grid.z > 65535 || threads == 0 ||
      threads > 1024 || shmem > 160 * 1024) {
    ++g_bad_launches;
    std::fprintf(stderr, "bad launch: grid %u %u %u block %u %u %u shmem %zu\n", grid.x, grid.y, grid.z, block.x,
                 block.y, block.z, shmem);
  }
  return hipSuccess;
}

hipError_t hipMalloc(void** p, size_t bytes) {
  if (!p) return hipErrorInvalidValue;
  *p = std::aligned_alloc(256, (bytes + 255) / 256 * 256 + 256);
  if (!*p) return hipErrorOutOfMemory;
  ++g_allocs;
  return hipSuccess;
}
hipError_t hipFree(void* p) {
  if (p) {
    std::free(p);
    --g_allocs;
  }
  return hipSuccess;
}
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind, hipStream_t) {
  std::memmove(dst, src, bytes);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t attr, int) {
  *v = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 1;
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "stub error"; }
hipError_t hipEventCreate(hipEvent_t* e) {
  *e = (hipEvent_t)std::malloc(16);
  return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t e) {
  std::free((void*)e);
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
  *ms = 1.0f;
  return hipSuccess;
}
hipError_t hipGetSymbolAddress(void** p, const void* symbol) {
  *p = (void*)symbol;   // host-only build: the symbol's host shadow stands in for its device copy
  return hipSuccess;
}
