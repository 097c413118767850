// MFMA throughput probe: the dense bf16 ceiling the forward's MFMA fractions are read against.
//
// Each 256-thread workgroup (one per CU at a time) fills 64 KB of LDS with operand values, then every wave
// repeats the inner loop of the large GEMM kernel without any global memory traffic: per round, 4
// k-substeps of 16 independent 32x32x16 bf16 MFMAs (4 A x 4 B fragments, 16 accumulators), the fragments
// of the next substep read from LDS while the current ones run.  The operand values decide how hard the chip throttles its clock: zeros draw the least
// power; random values drawn like the GEMM's (activations U(-1, 1), weights U(-0.05, 0.05)) show what dense
// bf16 work sustains on real data.
#include "common.h"
#include "launch.h"

namespace {

__device__ __forceinline__ unsigned short probe_val(unsigned i, unsigned seed, float scale) {
  unsigned x = i * 2654435761u ^ seed;
  x ^= x >> 13;
  x *= 0x5bd1e995u;
  x ^= x >> 15;
  const float f = (((int)(x & 0xFFFF) - 32768) / 32768.0f) * scale;
  return (unsigned short)(__float_as_uint(f) >> 16);
}

__global__ __launch_bounds__(256, 1) void k_mfma_probe(float* sink, int64_t rounds, int random_operands) {
  __shared__ __attribute__((aligned(1024))) unsigned short lds[32768];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, g = lane >> 5;
  for (int i = tid; i < 32768; i += 256)
    lds[i] = random_operands ? (i < 16384 ? probe_val(i, 11u, 1.0f) : probe_val(i, 22u, 0.05f)) : (unsigned short)0;
  __syncthreads();
  // the fragment layout of the large GEMM: 128-byte rows whose 16-byte chunks are XOR-swizzled by the
  // row (conflict-free reads of chunk 2 ks + g by 32 consecutive rows)
  const char* lx = (const char*)lds + (wave >> 1) * 16384;            // "activation" half
  const char* lw = (const char*)lds + 32768 + (wave & 1) * 16384;     // "weight" half
  const int swz = ((l32 >> 1) ^ (l32 << 2)) & 7;
  int foff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) foff[ks] = l32 * 128 + (((2 * ks + g) ^ swz) << 4);
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16){};
  // per round: 4 k-substeps of 16 MFMAs; the fragments of substep ks+1 are read while those of ks run
  for (int64_t r = 0; r < rounds; ++r) {
    u32x4 fa[2][4], fb[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[0][i] = *(const u32x4*)(lw + i * 4096 + foff[0]);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[0][j] = *(const u32x4*)(lx + j * 4096 + foff[0]);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int cur = ks & 1;
      if (ks < 3) {
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[cur ^ 1][i] = *(const u32x4*)(lw + i * 4096 + foff[ks + 1]);
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[cur ^ 1][j] = *(const u32x4*)(lx + j * 4096 + foff[ks + 1]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fa[cur][i]), as_bf16x8(fb[cur][j]), acc[i][j],
                                                              0, 0, 0);
    }
    // 8 fragment reads up front, then one read per 2 MFMAs, then the last 16 MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int q = 0; q < 24; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[i][j][e];
  sink[(int64_t)blockIdx.x * 256 + tid] = s;
}

}  // namespace

hipError_t launch_mfma_probe(float* sink, int blocks, int64_t rounds, int random_operands, hipStream_t s) {
  hipLaunchKernelGGL(k_mfma_probe, dim3((unsigned)blocks), dim3(256), 0, s, sink, rounds, random_operands);
  return hipGetLastError();
}
