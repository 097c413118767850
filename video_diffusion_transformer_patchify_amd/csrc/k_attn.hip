// Flash-style attention forward for gfx950: O = softmax(Q K^T / sqrt(128)) V per (batch, head), no mask,
// head_dim 128, bf16 operands on 32x32x16 MFMAs, fp32 online softmax.
//
// Used for both attentions of the Wan block (Wan2.1 walk-through page, section 5.2: self-attention over
// all video tokens, cross-attention from video tokens to the text tokens; diffusers WanTransformerBlock
// printed on the WanPipeline notes page: attn1 with rotary_emb, attn2 on encoder_hidden_states).
//
// Layout and dataflow
//   * A workgroup owns 128 queries of one (batch, head): 4 waves x 32 queries.  Q stays in registers.
//   * Keys are consumed in tiles of 64, staged in LDS (double buffered): K as [key][d] and V from a
//     pre-transposed copy Vt[b][h][d][key] as [d][key].
//   * Scores are formed transposed, S^T = K Q^T: the accumulator's column is the lane's query, so the
//     probabilities P^T come out of the accumulator already in the B-operand layout of the PV MFMA
//     (O^T += V^T P^T) once the 32 key rows of a K fragment are loaded in the order pi(i), which swaps
//     bits 2 and 3 of i.  With that order, lane half g holds keys 8g..8g+7 (+16) of each 16-key step.
//   * Row max is shared between the two lane halves with one cross-lane exchange per tile; row sums
//     stay per lane half and are combined once at the end.
#include "common.h"
#include "launch.h"

namespace {

constexpr int KT = 64;              // keys per tile
constexpr int QW = 32;              // queries per wave
constexpr int QB = 4 * QW;          // queries per workgroup
constexpr int K_LD = 128 + 8;       // bf16 per LDS K row (272 B)
constexpr int V_LD = KT + 8;        // bf16 per LDS Vt row (144 B)

struct AttnArgs {
  const bf16_t* q; int64_t ldq;
  const bf16_t* k; int64_t ldk;
  const bf16_t* vt; int64_t ldv;
  bf16_t* o; int64_t ldo;
  int64_t Lq, Lkv;
  int nh, B;
  int q_tiles;
  float scale_log2;
};

__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int per = nb / 8, rem = nb % 8;
  const int xcd = b % 8, slot = b / 8;
  return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

__device__ __forceinline__ int key_perm(int i) { return (i & 0x13) | ((i & 4) << 1) | ((i & 8) >> 1); }

__global__ __launch_bounds__(256, 1) void k_flash_attn(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t lk[2][KT * K_LD];
  __shared__ __attribute__((aligned(16))) bf16_t lv[2][128 * V_LD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  // Workgroups of one (batch, head) are kept on one XCD so they share K/V in its L2.
  const int nb = a.q_tiles * a.nh * a.B;
  const int lid = xcd_remap(blockIdx.x, nb);
  const int qt = lid % a.q_tiles;
  const int bh = lid / a.q_tiles;
  const int h = bh % a.nh, b = bh / a.nh;

  // ---- Q fragments (B operand of S^T = K Q^T): query l32, d = 16 s + 8 g .. +7
  const int64_t qi = (int64_t)qt * QB + wave * QW + l32;
  const int64_t qrow = qi < a.Lq ? qi : a.Lq - 1;
  const bf16_t* qp = a.q + ((int64_t)b * a.Lq + qrow) * a.ldq + h * 128 + g * 8;
  u32x4 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) qf[s] = *(const u32x4*)(qp + 16 * s);

  // ---- global -> LDS staging: K tile 64 x 128 (4 chunks/thread), Vt tile 128 x 64 (4 chunks/thread)
  const bf16_t* kbase = a.k + (int64_t)b * a.Lkv * a.ldk + h * 128;
  const bf16_t* vbase = a.vt + ((int64_t)b * a.nh + h) * 128 * a.ldv;
  u32x4 ks[4], vs[4];
  const int n_tiles = (int)((a.Lkv + KT - 1) / KT);
  auto gload = [&](int t) {
    const int64_t key0 = (int64_t)t * KT;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int r = c >> 4, col = (c & 15) * 8;
      const int64_t key = key0 + r;
      if (key < a.Lkv) ks[i] = *(const u32x4*)(kbase + key * a.ldk + col);
      else ks[i] = (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int d = c >> 3, col = (c & 7) * 8;
      vs[i] = *(const u32x4*)(vbase + (int64_t)d * a.ldv + key0 + col);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      *(u32x4*)(&lk[buf][(c >> 4) * K_LD + (c & 15) * 8]) = ks[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      *(u32x4*)(&lv[buf][(c >> 3) * V_LD + (c & 7) * 8]) = vs[i];
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (f32x16){};
  float m_run = -INFINITY, l_run = 0.f;
  const int krow = key_perm(l32);

  gload(0);
  lstore(0);
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) gload(t + 1);

    // ---- S^T for two 32-key sub-tiles
    f32x16 sacc[2];
#pragma unroll
    for (int kt2 = 0; kt2 < 2; ++kt2) {
      sacc[kt2] = (f32x16){};
      const bf16_t* kr = &lk[buf][(32 * kt2 + krow) * K_LD + g * 8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        u32x4 kf = *(const u32x4*)(kr + 16 * s);
        sacc[kt2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(qf[s]), sacc[kt2], 0, 0, 0);
      }
    }
    // element r of sub-tile kt2 holds key 64 t + 32 kt2 + 16 (r/8) + 8 g + r%8
    const int64_t key_lim = a.Lkv - (int64_t)t * KT;   // keys >= key_lim are past the end
    float mx = -INFINITY;
#pragma unroll
    for (int kt2 = 0; kt2 < 2; ++kt2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = sacc[kt2][r] * a.scale_log2;
        if (key_lim < KT) {
          const int kk = 32 * kt2 + 16 * (r >> 3) + 8 * g + (r & 7);
          if (kk >= key_lim) v = -INFINITY;
        }
        sacc[kt2][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float ls = 0.f;
    u32x4 pf[4];
#pragma unroll
    for (int kt2 = 0; kt2 < 2; ++kt2)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(sacc[kt2][8 * hh + e] - m_new);
          ls += p[e];
        }
        u32x4 w;
        w.x = pack_bf16x2(p[0], p[1]); w.y = pack_bf16x2(p[2], p[3]);
        w.z = pack_bf16x2(p[4], p[5]); w.w = pack_bf16x2(p[6], p[7]);
        pf[2 * kt2 + hh] = w;
      }
    l_run = l_run * alpha + ls;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;

    // ---- O^T += V^T P^T: A = Vt rows d = 32 dt + l32, keys 16 j + 8 g .. +7
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const bf16_t* vr = &lv[buf][(32 * dt + l32) * V_LD + g * 8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 vf = *(const u32x4*)(vr + 16 * j);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pf[j]), o[dt], 0, 0, 0);
      }
    }
    if (t + 1 < n_tiles) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- normalise and store: o[dt] element r holds d = 32 dt + 8 (r/4) + 4 g + r%4 of query qi
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  if (qi < a.Lq) {
    bf16_t* op = a.o + ((int64_t)b * a.Lq + qi) * a.ldo + h * 128 + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        u32x2 w;
        w.x = pack_bf16x2(o[dt][4 * rg] * inv, o[dt][4 * rg + 1] * inv);
        w.y = pack_bf16x2(o[dt][4 * rg + 2] * inv, o[dt][4 * rg + 3] * inv);
        *(u32x2*)(op + 32 * dt + 8 * rg) = w;
      }
  }
}

}  // namespace

hipError_t launch_attention(const bf16_t* q, int64_t ldq, const bf16_t* k, int64_t ldk, const bf16_t* vt, int64_t ldv,
                            bf16_t* o, int64_t ldo, int64_t B, int64_t Lq, int64_t Lkv, int nh, hipStream_t s) {
  if (B <= 0 || Lq <= 0) return hipSuccess;
  if (Lkv <= 0 || ldv < round_up(Lkv, KT)) return hipErrorInvalidValue;
  AttnArgs a;
  a.q = q; a.ldq = ldq; a.k = k; a.ldk = ldk; a.vt = vt; a.ldv = ldv; a.o = o; a.ldo = ldo;
  a.Lq = Lq; a.Lkv = Lkv; a.nh = nh; a.B = (int)B;
  a.q_tiles = (int)ceil_div(Lq, QB);
  a.scale_log2 = (float)(1.4426950408889634 / sqrt(128.0));
  const int64_t nb = (int64_t)a.q_tiles * nh * B;
  hipLaunchKernelGGL(k_flash_attn, dim3((unsigned)nb), dim3(256), 0, s, a);
  return hipGetLastError();
}
