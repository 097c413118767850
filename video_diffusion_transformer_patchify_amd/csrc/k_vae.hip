// Wan-VAE causal decoder kernels for gfx950: implicit-GEMM causal convolution, RMS norm + SiLU, latent
// preparation (per-channel un-normalisation + post-quant conv), weight packing.
//
// Operations (diffusers WanPipeline notes page, section "vae.decode"): WanCausalConv3d puts all temporal
// padding on the past side and takes the cached frames of earlier chunks in front of the chunk; the
// upsample modes double rows and columns (nearest) before a 3x3 Conv2d; upsample3d's (3,1,1) time conv
// doubles the channels, which become two frames; residual blocks apply RMS_norm and SiLU before each
// causal conv.  Frames use the padded layout of launch_vae.h.
//
// Convolution kernel (one 256-thread workgroup per CU):
//  * An output tile is 16 rows x 32 columns of one output frame x (32 * ncf) output channels; the four
//    waves own 4 rows each.  K runs over (time tap, 16-channel input block) stages; a stage holds the
//    input halo (18 x 34 pixels x 16 channels for 3x3 taps) and the stage's weights for all spatial taps
//    ([tap][c_out][16]), both brought global -> LDS by gfx950's direct loads (global_load_lds_dwordx4:
//    lane l of one instruction fills bytes 16 l .. 16 l + 15 of a 1 KB block), three stages in flight.
//  * The nine spatial taps read shifted windows of the one halo: the 32 pixels of an output row segment
//    and tap (dy, dx) are halo row r + dy, columns dx .. dx + 31, one 16-byte read per lane.
//  * MFMA 32x32x16 bf16 with the weights as the A operand (rows = output channels) and pixels as B:
//    each lane ends with 16 output channels (4 runs of 4 consecutive) of one pixel, stored as 8-byte
//    runs into the padded output frame, with the residual frame added in fp32 before the bf16 rounding.
//  * The frame border of zeros (and a zero frame for causal padding before the first frame) stands in
//    for all padding, so no load is masked; rows and columns past the frame edge are clamped on load
//    and not stored.  The nearest x2 upsample is a change of the load address: padded output row Y
//    reads padded input row (Y + 1) / 2.
//  * Workgroup ids are spread so that consecutive logical tiles (the output-channel tiles and output
//    frames of one spatial tile, which read the same input pixels) run on one XCD and share its L2.
#include "common.h"
#include "launch_vae.h"

typedef __attribute__((address_space(3))) void lds_void;

namespace {

constexpr int TH = 16, TW = 32;
constexpr int NSTG = 3;

template <int KS>
struct Halo {
  static constexpr int HR = TH + KS - 1, HC = TW + KS - 1;
  static constexpr int CHUNKS = HR * HC * 2;                   // 16-byte chunks (2 per pixel)
  static constexpr int BLOCKS = (CHUNKS + 255) / 256 * 4;      // 1 KB blocks, a multiple of the 4 waves
};

template <int KS, int NCF>
struct Wts {
  static constexpr int CHUNKS = KS * KS * NCF * 32 * 2;        // [tap][c_out][16 ci]: 2 chunks per c_out
  static constexpr int BLOCKS = (CHUNKS + 255) / 256 * 4;
  static constexpr int ELEMS = CHUNKS * 8;                     // bf16 elements of one stage
};

constexpr uint32_t vmcnt_imm(int n) { return 0x0F70u | (uint32_t)(n & 15) | ((uint32_t)(n >> 4) << 14); }

template <int KT, int KS, int UP, int NCF, bool VIDEO>
__global__ __launch_bounds__(256, 1) void k_vae_conv(const VaeConvArgs a) {
  using A_ = Halo<KS>;
  using B_ = Wts<KS, NCF>;
  constexpr int STAGE = (A_::BLOCKS + B_::BLOCKS) * 1024;
  constexpr int LA = A_::BLOCKS / 4, LB = B_::BLOCKS / 4;
  __shared__ __attribute__((aligned(1024))) char lds[NSTG * STAGE];

  const int total = a.tiles_x * a.tiles_y * a.nf * a.ntiles;
  const int per_xcd = gridDim.x >> 3;
  const int logical = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (logical >= total) return;
  const int n = logical % a.ntiles;
  int rem = logical / a.ntiles;
  const int j = rem % a.nf;
  const int tile = rem / a.nf;
  const int y0 = (tile / a.tiles_x) * TH, x0 = (tile % a.tiles_x) * TW;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, kh = lane >> 5;
  const int win_p = a.Win + 2;

  // per-lane byte offsets of the halo chunks inside one 16-channel block of the input frame
  uint32_t aoff[LA];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    int c = (4 * i + wave) * 64 + lane;
    if (c >= A_::CHUNKS) c = 0;                 // padding lanes of the last block fetch chunk 0
    const int px = c >> 1, half = c & 1;
    const int hr = px / A_::HC, hc = px % A_::HC;
    int row, col;
    if constexpr (UP) {
      row = (min(y0 + hr, a.H + 1) + 1) >> 1;
      col = (min(x0 + hc, a.W + 1) + 1) >> 1;
    } else if constexpr (KS == 3) {
      row = min(y0 + hr, a.H + 1);
      col = min(x0 + hc, a.W + 1);
    } else {
      row = min(y0 + hr + 1, a.H + 1);
      col = min(x0 + hc + 1, a.W + 1);
    }
    aoff[i] = (uint32_t)((row * win_p + col) * 32 + half * 16);
  }
  uint32_t boff[LB];
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    int c = (4 * i + wave) * 64 + lane;
    if (c >= B_::CHUNKS) c = 0;
    boff[i] = (uint32_t)(c * 16);
  }

  const int64_t plane_in = (int64_t)(a.Hin + 2) * win_p * 16;
  const int cinb = a.cin_blocks;
  const int nst = KT * cinb;
  const bf16_t* wbase = a.w + (int64_t)n * nst * B_::ELEMS;

  auto issue = [&](int st) {
    const int dt = st / cinb, cb = st - dt * cinb;
    const char* asrc = (const char*)(a.in[j][dt] + cb * plane_in);
    const char* bsrc = (const char*)(wbase + (int64_t)st * B_::ELEMS);
    char* dst = lds + (st % NSTG) * STAGE;
#pragma unroll
    for (int i = 0; i < LA; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(asrc + aoff[i]), (lds_void*)(dst + (4 * i + wave) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < LB; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(bsrc + boff[i]),
                                       (lds_void*)(dst + (A_::BLOCKS + 4 * i + wave) * 1024), 16, 0, 0);
  };

  // accumulators start at the bias: value v of lane (l32, kh) is output channel 8 (v / 4) + 4 kh + v % 4
  const int n0 = n * 32 * NCF;
  f32x16 acc[NCF][4];
#pragma unroll
  for (int f = 0; f < NCF; ++f) {
    f32x16 b;
#pragma unroll
    for (int v = 0; v < 16; ++v) b[v] = a.bias[n0 + f * 32 + 8 * (v >> 2) + 4 * kh + (v & 3)];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[f][r] = b;
  }

  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  issue(0);
  if (nst > 1) issue(1);
  for (int st = 0; st < nst; ++st) {
    if (st + 1 < nst) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LA + LB));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    block_sync();                                 // stage st visible; stage st - 1's buffer is free
    if (st + 2 < nst) issue(st + 2);
    const char* As = lds + (st % NSTG) * STAGE;
    const char* Bs = As + A_::BLOCKS * 1024;
    // Column tap dx uses 4 + KS - 1 halo rows and KS x NCF weight fragments.  The fragments of tap
    // dx + 1 are read while the MFMAs of tap dx run (two register sets), one read between every two
    // MFMAs, so a wave waits for LDS only at the start of a stage.
    constexpr int NP = 4 + KS - 1, NW = KS * NCF, NR = NP + NW, NM = KS * 4 * NCF;
    u32x4 pf[2][NP], wf[2][NW];
    auto read_tap = [&](int b, int dx) {
#pragma unroll
      for (int rr = 0; rr < NP; ++rr)
        pf[b][rr] = *(const u32x4*)(As + ((4 * wave + rr) * A_::HC + dx + l32) * 32 + kh * 16);
#pragma unroll
      for (int dy = 0; dy < KS; ++dy)
#pragma unroll
        for (int f = 0; f < NCF; ++f)
          wf[b][dy * NCF + f] = *(const u32x4*)(Bs + ((dy * KS + dx) * NCF * 32 + f * 32 + l32) * 32 + kh * 16);
    };
    read_tap(0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
    for (int dx = 0; dx < KS; ++dx) {
      const int b = dx & 1;
      if (dx + 1 < KS) read_tap(b ^ 1, dx + 1);
#pragma unroll
      for (int dy = 0; dy < KS; ++dy)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int f = 0; f < NCF; ++f)
            acc[f][r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(wf[b][dy * NCF + f]), as_bf16x8(pf[b][r + dy]),
                                                                 acc[f][r], 0, 0, 0);
      if (dx + 1 < KS) {
        constexpr int PER = NM / NR > 0 ? NM / NR : 1;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, NM - PER * NR > 0 ? NM - PER * NR : 0, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
      }
    }
  }

  const int x = x0 + l32;
  if constexpr (VIDEO) {
    // channels 0..2 are values 0..2 of the lanes with kh = 0 (tile 0 holds them)
    if (kh != 0 || n != 0 || x >= a.W) return;
    const int64_t hw = (int64_t)a.H * a.W;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int y = y0 + 4 * wave + r;
      if (y >= a.H) continue;
#pragma unroll
      for (int e = 0; e < 3; ++e) {
        const float v = fminf(fmaxf(acc[0][r][e], -1.0f), 1.0f);
        const int64_t idx = ((int64_t)e * a.video_T + a.video_t[j]) * hw + (int64_t)y * a.W + x;
        if (a.video_bf16) ((bf16_t*)a.video)[idx] = f32_to_bf16(v);
        else ((float*)a.video)[idx] = v;
      }
    }
  } else if (a.nout[j] != nullptr) {
    // one channel tile holds every channel of the lane's pixel: 16 per fragment in this lane, the other
    // 16 in lane l32 + 32 (1 - kh).  The norm is taken over the bf16-rounded outputs, as a separate
    // norm pass reading them back would take it.
    const int64_t wp = a.W + 2;
    const int64_t plane_out = (int64_t)(a.H + 2) * wp * 16;
    const bf16_t* rp = a.res[j];
    bf16_t* op = a.out[j];
    bf16_t* np = a.nout[j];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int y = y0 + 4 * wave + r;
      const bool ok = y < a.H && x < a.W;
      const int64_t pix = ((int64_t)(min(y, a.H - 1) + 1) * wp + (min(x, a.W - 1) + 1)) * 16;
      u32x2 o[NCF][4];
      float ss = 0.0f;
#pragma unroll
      for (int f = 0; f < NCF; ++f)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int co = f * 32 + 8 * q + 4 * kh;
          const int64_t off = (int64_t)(co >> 4) * plane_out + pix + (co & 15);
          float v0 = acc[f][r][4 * q], v1 = acc[f][r][4 * q + 1], v2 = acc[f][r][4 * q + 2], v3 = acc[f][r][4 * q + 3];
          if (rp) {
            const u32x2 rv = *(const u32x2*)(rp + off);
            v0 += lo_bf16(rv.x); v1 += hi_bf16(rv.x); v2 += lo_bf16(rv.y); v3 += hi_bf16(rv.y);
          }
          o[f][q].x = pack_bf16x2(v0, v1);
          o[f][q].y = pack_bf16x2(v2, v3);
          const float u0 = lo_bf16(o[f][q].x), u1 = hi_bf16(o[f][q].x), u2 = lo_bf16(o[f][q].y), u3 = hi_bf16(o[f][q].y);
          ss = fmaf(u0, u0, ss);
          ss = fmaf(u1, u1, ss);
          ss = fmaf(u2, u2, ss);
          ss = fmaf(u3, u3, ss);
        }
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
      ss = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);   // both halves, in the same order in both lanes
      const float rstd = 1.0f / sqrtf(fmaf(ss, 1.0f / (float)(32 * NCF), a.neps));
      if (!ok) continue;
#pragma unroll
      for (int f = 0; f < NCF; ++f)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int co = f * 32 + 8 * q + 4 * kh;
          const int64_t off = (int64_t)(co >> 4) * plane_out + pix + (co & 15);
          if (!a.nonly) *(u32x2*)(op + off) = o[f][q];
          const f32x4 g = *(const f32x4*)(a.ngamma + co);
          u32x2 w;
          w.x = pack_bf16x2(silu_f(lo_bf16(o[f][q].x) * rstd * g.x), silu_f(hi_bf16(o[f][q].x) * rstd * g.y));
          w.y = pack_bf16x2(silu_f(lo_bf16(o[f][q].y) * rstd * g.z), silu_f(hi_bf16(o[f][q].y) * rstd * g.w));
          *(u32x2*)(np + off) = w;
        }
    }
  } else {
    const int64_t wp = a.W + 2;
    const int64_t plane_out = (int64_t)(a.H + 2) * wp * 16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int y = y0 + 4 * wave + r;
      if (y >= a.H || x >= a.W) continue;
      const int64_t pix = ((int64_t)(y + 1) * wp + (x + 1)) * 16;
#pragma unroll
      for (int f = 0; f < NCF; ++f)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int co = n0 + f * 32 + 8 * q + 4 * kh;
          const int s = co / a.cpart;
          if (s >= a.split) continue;
          const int cl = co - s * a.cpart;
          const int64_t off = (int64_t)(cl >> 4) * plane_out + pix + (cl & 15);
          float v0 = acc[f][r][4 * q], v1 = acc[f][r][4 * q + 1], v2 = acc[f][r][4 * q + 2], v3 = acc[f][r][4 * q + 3];
          const bf16_t* rp = a.res[j * a.split + s];
          if (rp) {
            const u32x2 rv = *(const u32x2*)(rp + off);
            v0 += lo_bf16(rv.x); v1 += hi_bf16(rv.x); v2 += lo_bf16(rv.y); v3 += hi_bf16(rv.y);
          }
          u32x2 o;
          o.x = pack_bf16x2(v0, v1);
          o.y = pack_bf16x2(v2, v3);
          *(u32x2*)(a.out[j * a.split + s] + off) = o;
        }
    }
  }
}

struct VaeNormArgs {
  const bf16_t* in[VAE_MAXF];
  bf16_t* out[VAE_MAXF];
  const float* gamma;   // [cblocks * 16], zero beyond c
  int64_t H, W;
  int32_t cblocks;
  float inv_c, eps;
};

// Two lanes per pixel (channels 0..7 / 8..15 of every block), so each load instruction reads 32 whole
// 32-byte pixel runs.  CB > 0: the block count, the pixel's values kept in registers between the two
// passes; CB = 0: any count, the second pass reads the input again.
template <int CB>
__global__ __launch_bounds__(256) void k_vae_rms_silu(const VaeNormArgs a) {
  const int j = blockIdx.y;
  const int64_t p = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 1;
  const int half = threadIdx.x & 1;
  if (p >= a.H * a.W) return;
  const int64_t y = p / a.W, x = p - y * a.W;
  const int64_t wp = a.W + 2, plane = (a.H + 2) * wp * 16;
  const int64_t off = ((y + 1) * wp + x + 1) * 16 + half * 8;
  const bf16_t* src = a.in[j] + off;
  bf16_t* dst = a.out[j] + off;
  const int nb = CB > 0 ? CB : a.cblocks;
  u32x4 keep[CB > 0 ? CB : 1];
  float ss = 0.0f;
#pragma unroll
  for (int cb = 0; cb < (CB > 0 ? CB : 1); ++cb) keep[cb] = (u32x4){0, 0, 0, 0};
  for (int cb = 0; cb < nb; ++cb) {
    const u32x4 v = *(const u32x4*)(src + cb * plane);
    if constexpr (CB > 0) keep[cb] = v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = lo_bf16(v[e]), hi = hi_bf16(v[e]);
      ss = fmaf(lo, lo, ss);
      ss = fmaf(hi, hi, ss);
    }
  }
  ss += __shfl_xor(ss, 1, 64);
  const float rstd = 1.0f / sqrtf(fmaf(ss, a.inv_c, a.eps));
  for (int cb = 0; cb < nb; ++cb) {
    u32x4 v;
    if constexpr (CB > 0) v = keep[cb];
    else v = *(const u32x4*)(src + cb * plane);
    const float* g = a.gamma + cb * 16 + half * 8;
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = pack_bf16x2(silu_f(lo_bf16(v[e]) * rstd * g[2 * e]), silu_f(hi_bf16(v[e]) * rstd * g[2 * e + 1]));
    *(u32x4*)(dst + cb * plane) = o;
  }
}

struct VaePrepArgs {
  const void* z;
  bf16_t* out[VAE_MAXF];
  const float *mean, *std, *wq, *bq;
  int64_t F, H, W, f0;
};

template <typename T>
__global__ __launch_bounds__(256) void k_vae_prep(const VaePrepArgs a) {
  const int j = blockIdx.y;
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= a.H * a.W) return;
  const int64_t y = p / a.W, x = p - y * a.W;
  const T* z = (const T*)a.z;
  const int64_t hw = a.H * a.W;
  float u[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const T raw = z[(c * a.F + a.f0 + j) * hw + p];
    float v;
    if constexpr (sizeof(T) == 2) v = bf16_to_f32(raw);
    else v = raw;
    u[c] = fmaf(v, a.std[c], a.mean[c]);
  }
  uint32_t o[8];
#pragma unroll
  for (int co = 0; co < 16; co += 2) {
    float s0 = a.bq[co], s1 = a.bq[co + 1];
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      s0 = fmaf(a.wq[co * 16 + c], u[c], s0);
      s1 = fmaf(a.wq[(co + 1) * 16 + c], u[c], s1);
    }
    o[co / 2] = pack_bf16x2(s0, s1);
  }
  bf16_t* dst = a.out[j] + ((y + 1) * (a.W + 2) + x + 1) * 16;
  *(u32x4*)dst = (u32x4){o[0], o[1], o[2], o[3]};
  *(u32x4*)(dst + 8) = (u32x4){o[4], o[5], o[6], o[7]};
}

template <typename T>
__global__ void k_vae_pack_conv(const T* __restrict__ src, int64_t cout, int64_t cin, int kt, int ks, int ncf,
                                int64_t total, bf16_t* __restrict__ dst) {
  const int64_t cinb = (cin + 15) / 16, cols = 32 * ncf, taps = ks * ks;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = idx % 16;
    int64_t r = idx / 16;
    const int64_t col = r % cols; r /= cols;
    const int64_t tap = r % taps; r /= taps;
    const int64_t cb = r % cinb; r /= cinb;
    const int64_t dt = r % kt;
    const int64_t tl = r / kt;
    const int64_t co = tl * cols + col, ci = cb * 16 + e;
    bf16_t v = 0;
    if (co < cout && ci < cin) {
      const T s = src[((co * cin + ci) * kt + dt) * taps + tap];
      if constexpr (sizeof(T) == 2) v = s;
      else v = f32_to_bf16(s);
    }
    dst[idx] = v;
  }
}

__global__ void k_vae_zero(u32x4* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = (u32x4){0, 0, 0, 0};
}

unsigned grid_1d(int64_t total, int threads = 256) {
  int64_t g = (total + threads - 1) / threads;
  if (g > 65535LL * 16) g = 65535LL * 16;
  return (unsigned)(g < 1 ? 1 : g);
}

template <int KT, int KS, int UP, int NCF, bool VIDEO>
hipError_t run_conv(const VaeConvArgs& a, unsigned grid, hipStream_t s) {
  hipLaunchKernelGGL((k_vae_conv<KT, KS, UP, NCF, VIDEO>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int64_t vae_packed_conv_elems(int64_t cout, int64_t cin, int kt, int ks, int ncf) {
  const int64_t cols = 32 * ncf;
  return (cout + cols - 1) / cols * kt * ((cin + 15) / 16) * ks * ks * cols * 16;
}

hipError_t launch_vae_pack_conv(const void* src, int dtype, int64_t cout, int64_t cin, int kt, int ks, int ncf,
                                bf16_t* dst, hipStream_t s) {
  const int64_t total = vae_packed_conv_elems(cout, cin, kt, ks, ncf);
  if (dtype == 1)
    hipLaunchKernelGGL(k_vae_pack_conv<bf16_t>, dim3(grid_1d(total)), dim3(256), 0, s, (const bf16_t*)src, cout, cin,
                       kt, ks, ncf, total, dst);
  else
    hipLaunchKernelGGL(k_vae_pack_conv<float>, dim3(grid_1d(total)), dim3(256), 0, s, (const float*)src, cout, cin, kt,
                       ks, ncf, total, dst);
  return hipGetLastError();
}

hipError_t launch_vae_conv(const VaeConvArgs& a, int kt, int ks, int up, int ncf, bool video, hipStream_t s) {
  const int64_t total = (int64_t)a.tiles_x * a.tiles_y * a.nf * a.ntiles;
  if (total == 0) return hipSuccess;
  const unsigned grid = (unsigned)((total + 7) / 8 * 8);
#define VAE_CONV_CASE(KT_, KS_, UP_, NCF_, VID_)                                                   \
  if (kt == KT_ && ks == KS_ && up == UP_ && ncf == NCF_ && video == VID_)                          \
    return run_conv<KT_, KS_, UP_, NCF_, VID_>(a, grid, s);
  VAE_CONV_CASE(3, 3, 0, 3, false)
  VAE_CONV_CASE(3, 3, 0, 1, false)
  VAE_CONV_CASE(3, 3, 0, 1, true)
  VAE_CONV_CASE(3, 1, 0, 3, false)
  VAE_CONV_CASE(3, 1, 0, 1, false)
  VAE_CONV_CASE(1, 1, 0, 3, false)
  VAE_CONV_CASE(1, 1, 0, 1, false)
  VAE_CONV_CASE(1, 3, 1, 3, false)
  VAE_CONV_CASE(1, 3, 1, 1, false)
  VAE_CONV_CASE(1, 3, 0, 3, false)
  VAE_CONV_CASE(1, 3, 0, 1, false)
#undef VAE_CONV_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_vae_rms_silu(const bf16_t* const* in, bf16_t* const* out, int nf, int64_t c, int64_t cblocks,
                               int64_t H, int64_t W, const float* gamma, float eps, hipStream_t s) {
  if (nf <= 0 || H * W == 0) return hipSuccess;
  if (nf > VAE_MAXF) return hipErrorInvalidValue;
  VaeNormArgs a{};
  for (int j = 0; j < nf; ++j) {
    a.in[j] = in[j];
    a.out[j] = out[j];
  }
  a.gamma = gamma;
  a.H = H;
  a.W = W;
  a.cblocks = (int32_t)cblocks;
  a.inv_c = 1.0f / (float)c;
  a.eps = eps;
  const dim3 grid((unsigned)((H * W * 2 + 255) / 256), (unsigned)nf);
  switch (cblocks) {
    case 1: hipLaunchKernelGGL(k_vae_rms_silu<1>, grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_vae_rms_silu<2>, grid, dim3(256), 0, s, a); break;
    case 6: hipLaunchKernelGGL(k_vae_rms_silu<6>, grid, dim3(256), 0, s, a); break;
    case 12: hipLaunchKernelGGL(k_vae_rms_silu<12>, grid, dim3(256), 0, s, a); break;
    case 24: hipLaunchKernelGGL(k_vae_rms_silu<24>, grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(k_vae_rms_silu<0>, grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_vae_prep(const void* z, int dtype, int64_t F, int64_t H, int64_t W, int64_t f0, int n,
                           const float* mean, const float* std, const float* wq, const float* bq, bf16_t* const* out,
                           hipStream_t s) {
  if (n <= 0 || H * W == 0) return hipSuccess;
  if (n > VAE_MAXF) return hipErrorInvalidValue;
  VaePrepArgs a{};
  a.z = z;
  for (int j = 0; j < n; ++j) a.out[j] = out[j];
  a.mean = mean;
  a.std = std;
  a.wq = wq;
  a.bq = bq;
  a.F = F;
  a.H = H;
  a.W = W;
  a.f0 = f0;
  const dim3 grid((unsigned)((H * W + 255) / 256), (unsigned)n);
  if (dtype == 1) hipLaunchKernelGGL(k_vae_prep<bf16_t>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_vae_prep<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_vae_zero(void* p, int64_t bytes, hipStream_t s) {
  const int64_t n = bytes / 16;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_vae_zero, dim3(grid_1d(n)), dim3(256), 0, s, (u32x4*)p, n);
  return hipGetLastError();
}
