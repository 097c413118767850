// The allocation-free attention entry: the attention workspace (key-split partials and redo marks, the
// layout of attention_workspace_bytes with a split capacity of 64) lives in this file's static device
// array, one per GPU (each device that loads the library holds its own copy until the process ends).
// Its device address is looked up once per device, with that device current; host code passes only that
// address to the kernels, never the array's name.
#include <mutex>

#include "common.h"
#include "launch.h"

namespace {

constexpr int64_t SCRATCH_SPLIT_CAP = 64;       // key-split workgroups of a last round
constexpr int64_t SCRATCH_MAX_UNITS = 16384;    // (batch, head, 256-query tile) units of one call
constexpr int64_t QTILE = 256;                  // queries per attention workgroup
constexpr int64_t SCRATCH_BYTES = SCRATCH_SPLIT_CAP * QTILE * (128 + 2) * 4 + 16 * (SCRATCH_MAX_UNITS + SCRATCH_SPLIT_CAP);
constexpr int SCRATCH_MAX_DEVICES = 64;

static __device__ __align__(256) char scratch[SCRATCH_BYTES];

std::mutex g_scratch_mu;
float* g_scratch_ptr[SCRATCH_MAX_DEVICES] = {};

}  // namespace

int64_t attention_scratch_max_units() { return SCRATCH_MAX_UNITS; }
int64_t attention_scratch_bytes() { return SCRATCH_BYTES; }

hipError_t attention_scratch(float** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = (float*)p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_attention_noalloc(const bf16_t* q, int64_t ldq, const bf16_t* k, int64_t ldk, const bf16_t* vt,
                                    int64_t ldv, bf16_t* o, int64_t ldo, int64_t B, int64_t Lq, int64_t Lkv, int nh,
                                    hipStream_t s) {
  if (B <= 0 || Lq <= 0) return hipSuccess;
  if (B * nh * ceil_div(Lq, QTILE) > SCRATCH_MAX_UNITS) return hipErrorInvalidValue;
  float* ws = nullptr;
  const hipError_t e = attention_scratch(&ws);
  if (e != hipSuccess) return e;
  return launch_attention(q, ldq, k, ldk, vt, ldv, o, ldo, B, Lq, Lkv, nh, Lq == Lkv, s, ws, SCRATCH_BYTES, false, false,
                          SCRATCH_SPLIT_CAP);
}
