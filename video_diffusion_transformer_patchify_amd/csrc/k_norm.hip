// Row-wise HBM-bound kernels: LayerNorm + modulation, QK RMSNorm + 3D RoPE, V transpose,
// RoPE angle tables, timestep sinusoid.
//
// Definitions (diffusers WanTransformerBlock.forward on the WanPipeline notes page; WanAnimate page,
// configuration section for eps, qk_norm = rms_norm_across_heads, cross_attn_norm; architecture
// section for the per-axis 3D RoPE):
//   LN(x) = (x - mean) / sqrt(var + eps), population variance, computed in fp32 from the fp32 residual.
//   modulate: LN(x) * (1 + scale) + shift with scale/shift = table[i] + timestep projection row.
//   RMS(u) = u / sqrt(mean(u^2) + eps) over the whole model width, times a learned gain.
//   RoPE rotates channel pairs (2m, 2m+1) of each 128-wide head by the token's angle for pair m:
//   pairs [0, pt) use the frame index, [pt, pt+ph) the row, [pt+ph, 64) the column.
#include "common.h"
#include "launch.h"

namespace {

// ---------------------------------------------------------------------------------------------------
// Residual add + LayerNorm + modulate / affine.  One wave per row; NV float4 per lane (D = 256 * NV).
// The row streams (x in and out, the branch output, y) are touched once per launch and are far larger
// than the caches, so they use non-temporal loads and stores; the small parameter vectors stay cached.
// The residual step folds the previous branch into the fp32 stream before normalising it:
//   res_mode 1: x += r            (cross-attention output, ungated)
//   res_mode 2: x += r * gate,    gate = res_tab[d] + res_src[row(m)][d]   (gate_msa, c_gate_msa)
// and writes x back; r is the bf16 output of the branch's last Linear.
// ---------------------------------------------------------------------------------------------------
struct LnArgs {
  float* x; int64_t rows; int64_t D; float eps;
  int mode;                       // 0: modulate, 1: affine
  const float* tab_shift;         // [D]
  const float* tab_scale;         // [D]
  const float* src; int64_t src_ld; int64_t src_shift_off; int64_t src_scale_off; int64_t rows_per_src;
  const float* gamma; const float* beta;
  int res_mode; const bf16_t* res; const float* res_tab; const float* res_src; int64_t res_ld;
  bf16_t* y;
};

template <int NV>
__global__ __launch_bounds__(256) void k_ln_mod(LnArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  float* xr = a.x + row * a.D;
  const int64_t sr = row / a.rows_per_src;
  f32x4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = __builtin_nontemporal_load((const f32x4*)(xr + 4 * (lane + 64 * i)));
  if (a.res_mode) {
    const bf16_t* rr = a.res + row * a.D;
    u32x2 rw[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) rw[i] = __builtin_nontemporal_load((const u32x2*)(rr + 4 * (lane + 64 * i)));
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = 4 * (lane + 64 * i);
      f32x4 r = {lo_bf16(rw[i].x), hi_bf16(rw[i].x), lo_bf16(rw[i].y), hi_bf16(rw[i].y)};
      if (a.res_mode == 2) r *= *(const f32x4*)(a.res_tab + c) + *(const f32x4*)(a.res_src + sr * a.res_ld + c);
      v[i] += r;
      __builtin_nontemporal_store(v[i], (f32x4*)(xr + c));
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  const float inv_d = 1.0f / (float)a.D;
  const float mean = wave_sum(s) * inv_d;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    f32x4 d = v[i] - mean;
    q += (d.x * d.x + d.y * d.y) + (d.z * d.z + d.w * d.w);
  }
  const float var = wave_sum(q) * inv_d;
  const float rstd = 1.0f / sqrtf(var + a.eps);
  bf16_t* yr = a.y + row * a.D;
  if (a.mode == 0) {
    const float* ssh = a.src + sr * a.src_ld + a.src_shift_off;
    const float* ssc = a.src + sr * a.src_ld + a.src_scale_off;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = 4 * (lane + 64 * i);
      f32x4 sc = *(const f32x4*)(a.tab_scale + c) + *(const f32x4*)(ssc + c);
      f32x4 sh = *(const f32x4*)(a.tab_shift + c) + *(const f32x4*)(ssh + c);
      f32x4 o = (v[i] - mean) * rstd * (1.0f + sc) + sh;
      u32x2 w; w.x = pack_bf16x2(o.x, o.y); w.y = pack_bf16x2(o.z, o.w);
      __builtin_nontemporal_store(w, (u32x2*)(yr + c));
    }
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = 4 * (lane + 64 * i);
      f32x4 o = (v[i] - mean) * rstd * *(const f32x4*)(a.gamma + c) + *(const f32x4*)(a.beta + c);
      u32x2 w; w.x = pack_bf16x2(o.x, o.y); w.y = pack_bf16x2(o.z, o.w);
      __builtin_nontemporal_store(w, (u32x2*)(yr + c));
    }
  }
}

// Two rows per wave (narrow rows, D <= 1536): both rows' loads are in flight before either is reduced,
// and the modulation / affine vectors are loaded once per sample and kept in registers.
template <int NV>
__device__ __forceinline__ void ln_load_params(const LnArgs& a, int64_t sr, int lane, f32x4 (&gt)[NV], f32x4 (&p0)[NV],
                                               f32x4 (&p1)[NV]) {
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = 4 * (lane + 64 * i);
    if (a.res_mode == 2) gt[i] = *(const f32x4*)(a.res_tab + c) + *(const f32x4*)(a.res_src + sr * a.res_ld + c);
    if (a.mode == 0) {
      p0[i] = 1.0f + (*(const f32x4*)(a.tab_scale + c) + *(const f32x4*)(a.src + sr * a.src_ld + a.src_scale_off + c));
      p1[i] = *(const f32x4*)(a.tab_shift + c) + *(const f32x4*)(a.src + sr * a.src_ld + a.src_shift_off + c);
    } else {
      p0[i] = *(const f32x4*)(a.gamma + c);
      p1[i] = *(const f32x4*)(a.beta + c);
    }
  }
}

template <int NV>
__global__ __launch_bounds__(256) void k_ln_mod2(LnArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 2;
  if (row0 >= a.rows) return;
  const int nr = row0 + 1 < a.rows ? 2 : 1;
  f32x4 v[2][NV];
  u32x2 rw[2][NV];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if (r < nr) {
      const float* xr = a.x + (row0 + r) * a.D;
#pragma unroll
      for (int i = 0; i < NV; ++i) v[r][i] = __builtin_nontemporal_load((const f32x4*)(xr + 4 * (lane + 64 * i)));
      if (a.res_mode) {
        const bf16_t* rr = a.res + (row0 + r) * a.D;
#pragma unroll
        for (int i = 0; i < NV; ++i) rw[r][i] = __builtin_nontemporal_load((const u32x2*)(rr + 4 * (lane + 64 * i)));
      }
    }
  }
  int64_t sr_cached = -1;
  f32x4 gt[NV], p0[NV], p1[NV];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if (r >= nr) break;
    const int64_t row = row0 + r;
    const int64_t sr = row / a.rows_per_src;
    if (sr != sr_cached) {
      ln_load_params<NV>(a, sr, lane, gt, p0, p1);
      sr_cached = sr;
    }
    float* xr = a.x + row * a.D;
    if (a.res_mode) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int c = 4 * (lane + 64 * i);
        f32x4 rv = {lo_bf16(rw[r][i].x), hi_bf16(rw[r][i].x), lo_bf16(rw[r][i].y), hi_bf16(rw[r][i].y)};
        if (a.res_mode == 2) rv *= gt[i];
        v[r][i] += rv;
        __builtin_nontemporal_store(v[r][i], (f32x4*)(xr + c));
      }
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) s += (v[r][i].x + v[r][i].y) + (v[r][i].z + v[r][i].w);
    const float inv_d = 1.0f / (float)a.D;
    const float mean = wave_sum(s) * inv_d;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      f32x4 d = v[r][i] - mean;
      q += (d.x * d.x + d.y * d.y) + (d.z * d.z + d.w * d.w);
    }
    const float rstd = 1.0f / sqrtf(wave_sum(q) * inv_d + a.eps);
    bf16_t* yr = a.y + row * a.D;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = 4 * (lane + 64 * i);
      // mode 0: (x - mean) rstd (1 + scale) + shift; mode 1: (x - mean) rstd gamma + beta
      f32x4 o = (v[r][i] - mean) * rstd * p0[i] + p1[i];
      u32x2 w; w.x = pack_bf16x2(o.x, o.y); w.y = pack_bf16x2(o.z, o.w);
      __builtin_nontemporal_store(w, (u32x2*)(yr + c));
    }
  }
}

// ---------------------------------------------------------------------------------------------------
// RMSNorm (+ RoPE) in place on bf16 rows.  One wave per row; NV 8-element chunks per lane per
// segment (D = 512 * NV).  Up to two segments (q and k) share a row.
// ---------------------------------------------------------------------------------------------------
struct RmsArgs {
  bf16_t* buf; int64_t ld; int64_t rows; int64_t D; float eps;
  int64_t off_a; const float* gamma_a; float scale_a;   // segment a's outputs are also multiplied by scale_a
  int64_t off_b; const float* gamma_b;   // gamma_b == nullptr: single segment
  const float* rope;                     // nullptr: no rotation.  Layout from launch_rope_table.
  int64_t L; int Hp, Wp; int pt, ph;     // tokens per sample, grid, pairs per axis (t, h)
  int64_t rope_h_off, rope_w_off, rope_sin_off;  // float offsets of the h / w tables and of the sin half
};

// Rotation coefficients of one token for the 4 pairs a lane owns: in every 8-element chunk of every head
// the lane holds channels 8 (lane % 16) .. +7 of the head, i.e. pairs m = 4 (lane % 16) .. +3, so the
// same 4 (cos, sin) serve all heads and both segments of the row.
struct RopeCoef {
  float cs[4], sn[4];
};

__device__ __forceinline__ RopeCoef rope_coef(const RmsArgs& a, int lane, int64_t tok_f, int64_t tok_h, int64_t tok_w) {
  RopeCoef rc;
  const int m0 = 4 * (lane & 15);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int m = m0 + e;
    int64_t off;
    if (m < a.pt) off = tok_f * a.pt + m;
    else if (m < a.pt + a.ph) off = a.rope_h_off + tok_h * a.ph + (m - a.pt);
    else off = a.rope_w_off + tok_w * (64 - a.pt - a.ph) + (m - a.pt - a.ph);
    rc.cs[e] = a.rope[off];
    rc.sn[e] = a.rope[a.rope_sin_off + off];
  }
  return rc;
}

// NT: non-temporal loads (the q/k pass streams 400 MB+ once; a single segment written by the GEMM just
// before is better served from the caches).
template <int NV, bool NT>
__device__ __forceinline__ void rms_load(const bf16_t* p, int lane, u32x4 (&raw)[NV]) {
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const u32x4* q = (const u32x4*)(p + 8 * (lane + 64 * i));
    raw[i] = NT ? __builtin_nontemporal_load(q) : *q;
  }
}

template <int NV, bool ROPE>
__device__ __forceinline__ void rms_finish(const RmsArgs& a, bf16_t* p, const float* gamma, float scale, int lane,
                                           const RopeCoef& rc, const u32x4 (&raw)[NV]) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float lo = lo_bf16(raw[i][e]), hi = hi_bf16(raw[i][e]);
      s += lo * lo + hi * hi;
    }
  const float rstd = scale / sqrtf(wave_sum(s) / (float)a.D + a.eps);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c0 = 8 * (lane + 64 * i);
    f32x4 g0 = *(const f32x4*)(gamma + c0), g1 = *(const f32x4*)(gamma + c0 + 4);
    float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x0 = lo_bf16(raw[i][e]) * rstd * gg[2 * e];
      float x1 = hi_bf16(raw[i][e]) * rstd * gg[2 * e + 1];
      if constexpr (ROPE) {
        const float r0 = x0 * rc.cs[e] - x1 * rc.sn[e];
        const float r1 = x0 * rc.sn[e] + x1 * rc.cs[e];
        x0 = r0; x1 = r1;
      }
      o[e] = pack_bf16x2(x0, x1);
    }
    *(u32x4*)(p + c0) = o;
  }
}

// TWO: q and k segments in one row (the self-attention pass); otherwise one segment.
template <int NV, bool TWO>
__global__ __launch_bounds__(256) void k_rms_rope(RmsArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  int64_t tf = 0, th = 0, tw = 0;
  if (a.rope) {
    const int64_t n = row % a.L;
    tw = n % a.Wp;
    th = (n / a.Wp) % a.Hp;
    tf = n / ((int64_t)a.Wp * a.Hp);
  }
  bf16_t* r = a.buf + row * a.ld;
  if constexpr (TWO) {
    // both segments' loads are in flight before either is reduced
    u32x4 ra[NV], rb[NV];
    rms_load<NV, true>(r + a.off_a, lane, ra);
    rms_load<NV, true>(r + a.off_b, lane, rb);
    if (a.rope) {
      const RopeCoef rc = rope_coef(a, lane, tf, th, tw);
      rms_finish<NV, true>(a, r + a.off_a, a.gamma_a, a.scale_a, lane, rc, ra);
      rms_finish<NV, true>(a, r + a.off_b, a.gamma_b, 1.0f, lane, rc, rb);
    } else {
      const RopeCoef rc = {};
      rms_finish<NV, false>(a, r + a.off_a, a.gamma_a, a.scale_a, lane, rc, ra);
      rms_finish<NV, false>(a, r + a.off_b, a.gamma_b, 1.0f, lane, rc, rb);
    }
  } else {
    u32x4 ra[NV];
    rms_load<NV, false>(r + a.off_a, lane, ra);
    if (a.rope) {
      const RopeCoef rc = rope_coef(a, lane, tf, th, tw);
      rms_finish<NV, true>(a, r + a.off_a, a.gamma_a, a.scale_a, lane, rc, ra);
    } else {
      const RopeCoef rc = {};
      rms_finish<NV, false>(a, r + a.off_a, a.gamma_a, a.scale_a, lane, rc, ra);
    }
  }
}

// ---------------------------------------------------------------------------------------------------
// V transpose: rows [B*L] x (nh*128) at column offset col_off -> vt[b][h][d][ldv], zero for tokens
// in [L, ldv).  One workgroup per (64-token tile, head, batch).
// ---------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_transpose_v(const bf16_t* __restrict__ src, int64_t ld, int64_t col_off,
                                                     int64_t L, int nh, bf16_t* __restrict__ vt, int64_t ldv) {
  __shared__ bf16_t t[64][128 + 2];
  const int tid = threadIdx.x;
  const int64_t l0 = (int64_t)blockIdx.x * 64;
  const int h = blockIdx.y, b = blockIdx.z;
  // load 64 tokens x 128 channels: 1024 chunks of 8 bf16, 4 per thread
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 4, col = (c & 15) * 8;
    const int64_t l = l0 + r;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (l < L) v = *(const u32x4*)(src + ((int64_t)b * L + l) * ld + col_off + (int64_t)h * 128 + col);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      t[r][col + 2 * e] = (bf16_t)(v[e] & 0xFFFF);
      t[r][col + 2 * e + 1] = (bf16_t)(v[e] >> 16);
    }
  }
  __syncthreads();
  // write 128 rows (d) x 64 tokens: 1024 chunks of 8 tokens, 4 per thread
  bf16_t* dst = vt + ((int64_t)b * nh + h) * 128 * ldv + l0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int d = c >> 3, j = (c & 7) * 8;
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (uint32_t)t[j + 2 * e][d] | ((uint32_t)t[j + 2 * e + 1][d] << 16);
    *(u32x4*)(dst + (int64_t)d * ldv + j) = o;
  }
}

// ---------------------------------------------------------------------------------------------------
// RoPE tables: cos then sin, each [Fp*pt | Hp*ph | Wp*pw] floats; angle = pos * theta^(-2j/d_axis),
// evaluated in double precision.
// ---------------------------------------------------------------------------------------------------
__global__ void k_rope_table(float* __restrict__ tab, int Fp, int Hp, int Wp, int dt, int dh, int dw, double theta) {
  const int pt = dt / 2, ph = dh / 2, pw = dw / 2;
  const int n_t = Fp * pt, n_h = Hp * ph, n_w = Wp * pw;
  const int total = n_t + n_h + n_w;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
    int pos, j, d;
    if (i < n_t) { pos = i / pt; j = i % pt; d = dt; }
    else if (i < n_t + n_h) { pos = (i - n_t) / ph; j = (i - n_t) % ph; d = dh; }
    else { pos = (i - n_t - n_h) / pw; j = (i - n_t - n_h) % pw; d = dw; }
    const double ang = (double)pos * pow(theta, -2.0 * (double)j / (double)d);
    tab[i] = (float)cos(ang);
    tab[total + i] = (float)sin(ang);
  }
}

// ---------------------------------------------------------------------------------------------------
// Timestep sinusoid: s[r] = [cos(t w_i), sin(t w_i)], w_i = 10000^(-i/half), evaluated in double.
// ---------------------------------------------------------------------------------------------------
__global__ void k_sinusoid(const float* __restrict__ t, int64_t rows, int freq_dim, float* __restrict__ s) {
  const int half = freq_dim / 2;
  const int64_t total = rows * half;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / half;
    const int j = (int)(i % half);
    const double ang = (double)t[r] * pow(10000.0, -(double)j / (double)half);
    s[r * freq_dim + j] = (float)cos(ang);
    s[r * freq_dim + half + j] = (float)sin(ang);
  }
}

}  // namespace

#define NV_CASES(X) X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) X(15) X(16) \
  X(17) X(18) X(19) X(20) X(21) X(22) X(23) X(24)

hipError_t launch_layernorm(float* x, int64_t rows, int64_t D, float eps, int mode, const float* tab_shift,
                            const float* tab_scale, const float* src, int64_t src_ld, int64_t src_shift_off,
                            int64_t src_scale_off, int64_t rows_per_src, const float* gamma, const float* beta,
                            int res_mode, const bf16_t* res, const float* res_tab, const float* res_src, int64_t res_ld,
                            bf16_t* y, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (D % 256 != 0 || D / 256 > 24) return hipErrorInvalidValue;
  LnArgs a{x, rows, D, eps, mode, tab_shift, tab_scale, src, src_ld, src_shift_off, src_scale_off,
           rows_per_src > 0 ? rows_per_src : 1, gamma, beta, res_mode, res, res_tab, res_src, res_ld, y};
  if (D / 256 <= 6) {
    dim3 grid((unsigned)ceil_div(rows, 8)), block(256);
    switch (D / 256) {
      case 1: hipLaunchKernelGGL(k_ln_mod2<1>, grid, block, 0, s, a); break;
      case 2: hipLaunchKernelGGL(k_ln_mod2<2>, grid, block, 0, s, a); break;
      case 3: hipLaunchKernelGGL(k_ln_mod2<3>, grid, block, 0, s, a); break;
      case 4: hipLaunchKernelGGL(k_ln_mod2<4>, grid, block, 0, s, a); break;
      case 5: hipLaunchKernelGGL(k_ln_mod2<5>, grid, block, 0, s, a); break;
      default: hipLaunchKernelGGL(k_ln_mod2<6>, grid, block, 0, s, a); break;
    }
    return hipGetLastError();
  }
  dim3 grid((unsigned)ceil_div(rows, 4)), block(256);
  switch (D / 256) {
#define X(n) case n: hipLaunchKernelGGL(k_ln_mod<n>, grid, block, 0, s, a); break;
    NV_CASES(X)
#undef X
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rms_rope(bf16_t* buf, int64_t ld, int64_t rows, int64_t D, float eps, int64_t off_a,
                           const float* gamma_a, int64_t off_b, const float* gamma_b, const float* rope, int64_t L,
                           int Fp, int Hp, int Wp, int dt, int dh, int dw, hipStream_t s, float scale_a) {
  if (rows <= 0) return hipSuccess;
  if (D % 512 != 0 || D / 512 > 24) return hipErrorInvalidValue;
  RmsArgs a;
  a.buf = buf; a.ld = ld; a.rows = rows; a.D = D; a.eps = eps;
  a.off_a = off_a; a.gamma_a = gamma_a; a.scale_a = scale_a; a.off_b = off_b; a.gamma_b = gamma_b;
  a.rope = rope; a.L = L > 0 ? L : 1; a.Hp = Hp; a.Wp = Wp; a.pt = dt / 2; a.ph = dh / 2;
  a.rope_h_off = (int64_t)Fp * (dt / 2);
  a.rope_w_off = a.rope_h_off + (int64_t)Hp * (dh / 2);
  a.rope_sin_off = a.rope_w_off + (int64_t)Wp * (dw / 2);
  dim3 grid((unsigned)ceil_div(rows, 4)), block(256);
  switch (D / 512) {
#define X(n)                                                                 \
  case n:                                                                    \
    if (gamma_b) hipLaunchKernelGGL((k_rms_rope<n, true>), grid, block, 0, s, a); \
    else hipLaunchKernelGGL((k_rms_rope<n, false>), grid, block, 0, s, a);       \
    break;
    NV_CASES(X)
#undef X
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_transpose_v(const bf16_t* src, int64_t ld, int64_t col_off, int64_t B, int64_t L, int nh, bf16_t* vt,
                              int64_t ldv, hipStream_t s) {
  if (B <= 0 || ldv <= 0) return hipSuccess;
  if (ldv % 64 != 0) return hipErrorInvalidValue;
  dim3 grid((unsigned)(ldv / 64), (unsigned)nh, (unsigned)B);
  hipLaunchKernelGGL(k_transpose_v, grid, dim3(256), 0, s, src, ld, col_off, L, nh, vt, ldv);
  return hipGetLastError();
}

int64_t rope_table_floats(int Fp, int Hp, int Wp, int dt, int dh, int dw) {
  return 2LL * ((int64_t)Fp * (dt / 2) + (int64_t)Hp * (dh / 2) + (int64_t)Wp * (dw / 2));
}

hipError_t launch_rope_table(float* tab, int Fp, int Hp, int Wp, int dt, int dh, int dw, double theta, hipStream_t s) {
  const int64_t n = rope_table_floats(Fp, Hp, Wp, dt, dh, dw) / 2;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_rope_table, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, tab, Fp, Hp, Wp, dt, dh, dw,
                     theta);
  return hipGetLastError();
}

hipError_t launch_sinusoid(const float* t, int64_t rows, int freq_dim, float* out, hipStream_t s) {
  const int64_t n = rows * (freq_dim / 2);
  if (n <= 0) return hipSuccess;
  int64_t g = ceil_div(n, 256);
  if (g > 65535) g = 65535;
  hipLaunchKernelGGL(k_sinusoid, dim3((unsigned)g), dim3(256), 0, s, t, rows, freq_dim, out);
  return hipGetLastError();
}
