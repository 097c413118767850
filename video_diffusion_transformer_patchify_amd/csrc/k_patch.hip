// Patchify gather, unpatchify scatter, dtype conversion and weight packing kernels.
//
// Patch layout (Wan2.1 walk-through page, section 5.1; diffusers WanPipeline notes, WanTransformer3DModel
// forward): Conv3d kernel = stride = (1,2,2) over the latent [B,C,F,H_z,W_z], output flattened over
// (F', H', W') so token n = (f*H' + h)*W' + w.  The patch vector follows the Conv3d weight
// [D, C, 1, 2, 2] flattened: column c*4 + 2i + j.  proj_out's columns follow the printed
// reshape(B,F',H',W',1,2,2,C_out): column (2i + j)*C_out + c.
#include "common.h"
#include "launch.h"

// One thread per (b, c, f, h, w-pair-of-tokens): reads 2 rows x 2 columns of the latent patch.
template <typename T>
__global__ void k_patchify(const T* __restrict__ x, int64_t B, int64_t C, int64_t F, int64_t Hz, int64_t Wz,
                           int64_t kp, bf16_t* __restrict__ p) {
  const int64_t Hp = Hz / 2, Wp = Wz / 2;
  const int64_t total = B * C * F * Hp * Wp;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    int64_t w = idx % Wp;
    int64_t r = idx / Wp;
    int64_t h = r % Hp; r /= Hp;
    int64_t f = r % F; r /= F;
    int64_t c = r % C;
    int64_t b = r / C;
    const T* src = x + (((b * C + c) * F + f) * Hz + 2 * h) * Wz + 2 * w;
    float v00, v01, v10, v11;
    if constexpr (sizeof(T) == 2) {
      v00 = bf16_to_f32(src[0]); v01 = bf16_to_f32(src[1]);
      v10 = bf16_to_f32(src[Wz]); v11 = bf16_to_f32(src[Wz + 1]);
    } else {
      v00 = src[0]; v01 = src[1]; v10 = src[Wz]; v11 = src[Wz + 1];
    }
    int64_t n = (f * Hp + h) * Wp + w;
    u32x2 o;
    o.x = pack_bf16x2(v00, v01);
    o.y = pack_bf16x2(v10, v11);
    *(u32x2*)(p + (b * F * Hp * Wp + n) * kp + c * 4) = o;
  }
}

// Zero the padding columns [4C, kp) of the patch matrix.
__global__ void k_patch_pad(bf16_t* __restrict__ p, int64_t rows, int64_t kp, int64_t k0) {
  const int64_t w = kp - k0;
  const int64_t total = rows * w;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    int64_t r = idx / w, c = idx % w;
    p[r * kp + k0 + c] = 0;
  }
}

// One thread per output element, x fastest so the stores are contiguous.
template <typename T>
__global__ void k_unpatchify(const float* __restrict__ z, int64_t ldz, int64_t B, int64_t C, int64_t F,
                             int64_t Hz, int64_t Wz, T* __restrict__ out) {
  const int64_t Hp = Hz / 2, Wp = Wz / 2;
  const int64_t total = B * C * F * Hz * Wz;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    int64_t xx = idx % Wz;
    int64_t r = idx / Wz;
    int64_t yy = r % Hz; r /= Hz;
    int64_t f = r % F; r /= F;
    int64_t c = r % C;
    int64_t b = r / C;
    int64_t n = (f * Hp + (yy >> 1)) * Wp + (xx >> 1);
    int64_t col = (2 * (yy & 1) + (xx & 1)) * C + c;
    float v = z[(b * F * Hp * Wp + n) * ldz + col];
    if constexpr (sizeof(T) == 2) out[idx] = f32_to_bf16(v);
    else out[idx] = v;
  }
}

// Denoising step fused into the unpatchify scatter (Wan2.1 walk-through page, section 7: the guided velocity
// v_u + s (v_c - v_u) and the Euler update x + (sigma_next - sigma) v; section 6.3 works one step by hand).
// z holds 2L proj_out rows, the conditional batch element first; x is the model input [1, C_x, F, Hz, Wz]
// whose first C channels are the noisy sample.  One thread per output element, fp32 arithmetic.
template <typename T>
__global__ void k_cfg_euler(const float* __restrict__ z, int64_t ldz, int64_t C, int64_t F, int64_t Hz, int64_t Wz,
                            const T* __restrict__ x, float scale, float dsigma, T* __restrict__ out) {
  const int64_t Hp = Hz / 2, Wp = Wz / 2, L = F * Hp * Wp;
  const int64_t total = C * F * Hz * Wz;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t xx = idx % Wz;
    int64_t r = idx / Wz;
    const int64_t yy = r % Hz; r /= Hz;
    const int64_t f = r % F;
    const int64_t c = r / F;
    const int64_t n = (f * Hp + (yy >> 1)) * Wp + (xx >> 1);
    const int64_t col = (2 * (yy & 1) + (xx & 1)) * C + c;
    const float vc = z[n * ldz + col], vu = z[(L + n) * ldz + col];
    const float v = fmaf(scale, vc - vu, vu);
    const int64_t xi = ((c * F + f) * Hz + yy) * Wz + xx;   // channel c < C of batch element 0 of the input
    float xv;
    if constexpr (sizeof(T) == 2) xv = bf16_to_f32(x[xi]);
    else xv = x[xi];
    const float o = fmaf(dsigma, v, xv);
    if constexpr (sizeof(T) == 2) out[idx] = f32_to_bf16(o);
    else out[idx] = o;
  }
}

// src (fp32 or bf16, rows x cols, leading dim lds) -> bf16 dst (leading dim ldd); columns
// [cols, ldd) of each written row are zero-filled.
template <typename T>
__global__ void k_pack_bf16(const T* __restrict__ src, int64_t rows, int64_t cols, int64_t lds,
                            bf16_t* __restrict__ dst, int64_t ldd) {
  const int64_t total = rows * ldd;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    int64_t r = idx / ldd, c = idx % ldd;
    bf16_t v = 0;
    if (c < cols) {
      if constexpr (sizeof(T) == 2) v = src[r * lds + c];
      else v = f32_to_bf16(src[r * lds + c]);
    }
    dst[idx] = v;
  }
}

template <typename T>
__global__ void k_pack_f32(const T* __restrict__ src, int64_t n, float* __restrict__ dst) {
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    if constexpr (sizeof(T) == 2) dst[idx] = bf16_to_f32(src[idx]);
    else dst[idx] = src[idx];
  }
}

static inline unsigned grid_for(int64_t total, int threads = 256) {
  int64_t g = ceil_div(total, threads);
  if (g > 65535LL * 16) g = 65535LL * 16;
  if (g < 1) g = 1;
  return (unsigned)g;
}

hipError_t launch_patchify(const void* x, int dtype, int64_t B, int64_t C, int64_t F, int64_t Hz, int64_t Wz,
                           int64_t kp, bf16_t* p, hipStream_t s) {
  int64_t total = B * C * F * (Hz / 2) * (Wz / 2);
  if (total > 0) {
    if (dtype == 1)
      hipLaunchKernelGGL(k_patchify<bf16_t>, dim3(grid_for(total)), dim3(256), 0, s, (const bf16_t*)x, B, C, F,
                         Hz, Wz, kp, p);
    else
      hipLaunchKernelGGL(k_patchify<float>, dim3(grid_for(total)), dim3(256), 0, s, (const float*)x, B, C, F, Hz,
                         Wz, kp, p);
  }
  int64_t rows = B * F * (Hz / 2) * (Wz / 2);
  if (kp > 4 * C && rows > 0)
    hipLaunchKernelGGL(k_patch_pad, dim3(grid_for(rows * (kp - 4 * C))), dim3(256), 0, s, p, rows, kp, 4 * C);
  return hipGetLastError();
}

hipError_t launch_unpatchify(const float* z, int64_t ldz, int64_t B, int64_t C, int64_t F, int64_t Hz, int64_t Wz,
                             void* out, int dtype, hipStream_t s) {
  int64_t total = B * C * F * Hz * Wz;
  if (total == 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL(k_unpatchify<bf16_t>, dim3(grid_for(total)), dim3(256), 0, s, z, ldz, B, C, F, Hz, Wz,
                       (bf16_t*)out);
  else
    hipLaunchKernelGGL(k_unpatchify<float>, dim3(grid_for(total)), dim3(256), 0, s, z, ldz, B, C, F, Hz, Wz,
                       (float*)out);
  return hipGetLastError();
}

hipError_t launch_cfg_euler(const float* z, int64_t ldz, int64_t C, int64_t F, int64_t Hz, int64_t Wz, const void* x,
                            int dtype, float scale, float sigma, float sigma_next, void* out, hipStream_t s) {
  const int64_t total = C * F * Hz * Wz;
  if (total == 0) return hipSuccess;
  const float ds = sigma_next - sigma;
  if (dtype == 1)
    hipLaunchKernelGGL(k_cfg_euler<bf16_t>, dim3(grid_for(total)), dim3(256), 0, s, z, ldz, C, F, Hz, Wz,
                       (const bf16_t*)x, scale, ds, (bf16_t*)out);
  else
    hipLaunchKernelGGL(k_cfg_euler<float>, dim3(grid_for(total)), dim3(256), 0, s, z, ldz, C, F, Hz, Wz,
                       (const float*)x, scale, ds, (float*)out);
  return hipGetLastError();
}

hipError_t launch_pack_bf16(const void* src, int dtype, int64_t rows, int64_t cols, int64_t lds, bf16_t* dst,
                            int64_t ldd, hipStream_t s) {
  int64_t total = rows * ldd;
  if (total == 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL(k_pack_bf16<bf16_t>, dim3(grid_for(total)), dim3(256), 0, s, (const bf16_t*)src, rows, cols,
                       lds, dst, ldd);
  else
    hipLaunchKernelGGL(k_pack_bf16<float>, dim3(grid_for(total)), dim3(256), 0, s, (const float*)src, rows, cols,
                       lds, dst, ldd);
  return hipGetLastError();
}

hipError_t launch_pack_f32(const void* src, int dtype, int64_t n, float* dst, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL(k_pack_f32<bf16_t>, dim3(grid_for(n)), dim3(256), 0, s, (const bf16_t*)src, n, dst);
  else
    hipLaunchKernelGGL(k_pack_f32<float>, dim3(grid_for(n)), dim3(256), 0, s, (const float*)src, n, dst);
  return hipGetLastError();
}
