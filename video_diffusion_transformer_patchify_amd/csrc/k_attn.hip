// Flash-style attention forward for gfx950: O = softmax(Q K^T / sqrt(128)) V per (batch, head), no mask,
// head_dim 128, bf16 operands on 32x32x16 MFMAs, fp32 online softmax.
//
// Used for both attentions of the Wan block (Wan2.1 walk-through page, section 5.2: self-attention over
// all video tokens, cross-attention from video tokens to the text tokens; diffusers WanTransformerBlock
// printed on the WanPipeline notes page: attn1 with rotary_emb, attn2 on encoder_hidden_states).
//
// Layout and dataflow
//   * A workgroup owns 256 queries of one (batch, head): 4 waves x 64 queries, each wave as two
//     32-query blocks that share every K and V fragment it reads from LDS (half the LDS traffic per
//     MFMA of one block per wave).  Q stays in registers.
//   * Keys are consumed in tiles of 64.  K [key][d] and the pre-transposed V (Vt[b][h][d][key], so a
//     tile is [d][key]) are copied global -> LDS with gfx950's direct loads (global_load_lds_dwordx4:
//     lane l of an instruction fills bytes 16 l .. 16 l + 15 of a 1 KB LDS block), double buffered,
//     with no register staging.  The 16-byte chunks of each LDS row are XOR-swizzled so the fragment
//     reads are free of bank conflicts; the swizzle is applied by choosing which global chunk each
//     lane fetches.
//   * Scores are formed transposed, S^T = K Q^T: the accumulator's column is the lane's query, so the
//     probabilities P^T come out of the accumulator already in the B-operand layout of the PV MFMA
//     (O^T += V^T P^T) once the 32 key rows of a K fragment are taken in the order pi(i), which swaps
//     bits 2 and 3 of i.  With that order, lane half g holds keys 8g..8g+7 (+16) of each 16-key step.
//   * Softmax in base 2 with the 1/sqrt(128) scale folded into one FMA per score.  The running max is
//     only raised when a tile's max exceeds it by more than 8 (log2 units): until then the stale max is
//     kept (probabilities up to 2^8, exact after the final division because numerator and denominator
//     share it) and the O rescale is skipped.
//   * Row max is shared between the two lane halves with one cross-lane exchange per tile; row sums
//     stay per lane half and are combined once at the end.
//   * Only the last key tile can be partial; it runs a separately compiled copy of the tile body that
//     masks keys past the end, so full tiles carry no masking code.
#include "common.h"
#include "launch.h"

namespace {

constexpr int KT = 64;              // keys per tile
constexpr int QWAVE = 64;           // queries per wave (two 32-query blocks)
constexpr int QB = 4 * QWAVE;       // queries per workgroup
constexpr int K_TILE_BYTES = KT * 256;    // 64 rows of 128 bf16
constexpr int V_TILE_BYTES = 128 * KT * 2; // 128 rows of 64 bf16
constexpr float RESCALE_LOG2 = 8.0f;

typedef __attribute__((address_space(3))) void lds_void;

struct AttnArgs {
  const bf16_t* q; int64_t ldq;
  const bf16_t* k; int64_t ldk;
  const bf16_t* vt; int64_t ldv;
  bf16_t* o; int64_t ldo;
  int64_t Lq, Lkv;
  int nh, B;
  int q_tiles;
  float scale_log2;   // log2(e) / sqrt(128)
};

__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int per = nb / 8, rem = nb % 8;
  const int xcd = b % 8, slot = b / 8;
  return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

// Key order of the rows of a 32-key K fragment (swap bits 2 and 3; an involution).
__device__ __forceinline__ int key_perm(int i) { return (i & 0x13) | ((i & 4) << 1) | ((i & 8) >> 1); }
// Chunk swizzles: LDS chunk position = logical chunk ^ swz(row).
__device__ __forceinline__ int k_swz(int r) { return key_perm(r & 31) & 15; }
__device__ __forceinline__ int v_swz(int r) { return ((r >> 1) ^ (r << 2)) & 7; }

struct AttnState {
  f32x16 o[2][4];
  float m_run[2], l_run[2];
};

// One 64-key tile for both 32-query blocks of this wave.
template <bool MASK>
__device__ __forceinline__ void attn_tile(AttnState& st, const u32x4 (&qf)[2][8], const char* lk, const char* lv,
                                          int l32, int g, float c, float grow_thr, int key_lim) {
  // ---- S^T = K Q^T; each K fragment read once, used by both query blocks
  f32x16 sacc[2][2];
#pragma unroll
  for (int kt2 = 0; kt2 < 2; ++kt2) {
    sacc[0][kt2] = (f32x16){};
    sacc[1][kt2] = (f32x16){};
    const int row = 32 * kt2 + key_perm(l32);
    const char* kr = lk + row * 256;
    const int sw = k_swz(row);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 kf = *(const u32x4*)(kr + (((2 * s + g) ^ sw) << 4));
      sacc[0][kt2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(qf[0][s]), sacc[0][kt2], 0, 0, 0);
      sacc[1][kt2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(qf[1][s]), sacc[1][kt2], 0, 0, 0);
    }
  }
  // element r of sub-tile kt2 holds key 32 kt2 + 16 (r/8) + 8 g + r%8 of the tile
  if constexpr (MASK) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kt2 = 0; kt2 < 2; ++kt2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = 32 * kt2 + 16 * (r >> 3) + 8 * g + (r & 7);
          if (kk >= key_lim) sacc[qb][kt2][r] = -INFINITY;
        }
  }

  // ---- online softmax (base 2), per query block
  u32x4 pf[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float mx = sacc[qb][0][0];
#pragma unroll
    for (int kt2 = 0; kt2 < 2; ++kt2)
#pragma unroll
      for (int r = (kt2 == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, sacc[qb][kt2][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const bool grow = mx > st.m_run[qb] + grow_thr;
    if (__any(grow)) {
      const float m_new = grow ? mx : st.m_run[qb];
      const float alpha = __builtin_amdgcn_exp2f((st.m_run[qb] - m_new) * c);
      st.m_run[qb] = m_new;
      st.l_run[qb] *= alpha;
      // one 16-register accumulator at a time: the accumulators live in AGPRs and each multiply needs
      // VGPR temporaries
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        st.o[qb][dt] *= alpha;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const float mc = -st.m_run[qb] * c;
    float ls = 0.f;
#pragma unroll
    for (int kt2 = 0; kt2 < 2; ++kt2)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(fmaf(sacc[qb][kt2][8 * hh + e], c, mc));
          ls += p[e];
        }
        u32x4 w;
        w.x = pack_bf16x2(p[0], p[1]); w.y = pack_bf16x2(p[2], p[3]);
        w.z = pack_bf16x2(p[4], p[5]); w.w = pack_bf16x2(p[6], p[7]);
        pf[qb][2 * kt2 + hh] = w;
      }
    st.l_run[qb] += ls;
  }

  // ---- O^T += V^T P^T: A = Vt rows d = 32 dt + l32, keys 16 j + 8 g .. +7; each V fragment read once
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int row = 32 * dt + l32;
    const char* vr = lv + row * 128;
    const int sw = v_swz(row);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 vf = *(const u32x4*)(vr + (((2 * j + g) ^ sw) << 4));
      st.o[0][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pf[0][j]), st.o[0][dt], 0, 0, 0);
      st.o[1][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pf[1][j]), st.o[1][dt], 0, 0, 0);
    }
  }
}

// SELF selects the instantiation only (self- and cross-attention then show up as separate kernels in
// a trace); the code path is the same.
template <bool SELF>
__global__ __launch_bounds__(256, 1) void k_flash_attn(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[2][K_TILE_BYTES + V_TILE_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  // Workgroups of one (batch, head) are kept on one XCD so they share K/V in its L2.
  const int nb = a.q_tiles * a.nh * a.B;
  const int lid = xcd_remap(blockIdx.x, nb);
  const int qt = lid % a.q_tiles;
  const int bh = lid / a.q_tiles;
  const int h = bh % a.nh, b = bh / a.nh;

  // ---- Q fragments (B operand of S^T = K Q^T): query l32 of block qb, d = 16 s + 8 g .. +7
  int64_t qi[2];
  u32x4 qf[2][8];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    qi[qb] = (int64_t)qt * QB + wave * QWAVE + qb * 32 + l32;
    const int64_t qrow = qi[qb] < a.Lq ? qi[qb] : a.Lq - 1;
    const bf16_t* qp = a.q + ((int64_t)b * a.Lq + qrow) * a.ldq + h * 128 + g * 8;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[qb][s] = *(const u32x4*)(qp + 16 * s);
  }

  // ---- direct global -> LDS copies.  Each wave issues 4 K and 4 V instructions per tile.
  //   K: instruction I (= 4 wave + i) fills rows 4I .. 4I+3; lane -> row 4I + lane/16, position lane%16.
  //   V: instruction I fills rows 8I .. 8I+7; lane -> row 8I + lane/8, position lane%8.
  const bf16_t* kbase = a.k + (int64_t)b * a.Lkv * a.ldk + h * 128;
  const bf16_t* vbase = a.vt + ((int64_t)b * a.nh + h) * 128 * a.ldv;
  const int n_tiles = (int)((a.Lkv + KT - 1) / KT);
  int k_row[4], k_col[4], v_row[4], v_col[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int I = 4 * wave + i;
    k_row[i] = 4 * I + (lane >> 4);
    k_col[i] = ((lane & 15) ^ k_swz(k_row[i])) * 8;
    v_row[i] = 8 * I + (lane >> 3);
    v_col[i] = ((lane & 7) ^ v_swz(v_row[i])) * 8;
  }
  auto issue = [&](int t, int buf) {
    const int64_t key0 = (int64_t)t * KT;
    char* lk = lds[buf];
    char* lv = lds[buf] + K_TILE_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int64_t key = key0 + k_row[i];
      if (key > a.Lkv - 1) key = a.Lkv - 1;      // rows past the end are masked in the last tile
      __builtin_amdgcn_global_load_lds((const void*)(kbase + key * a.ldk + k_col[i]),
                                       (lds_void*)(lk + (4 * wave + i) * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_global_load_lds((const void*)(vbase + (int64_t)v_row[i] * a.ldv + key0 + v_col[i]),
                                       (lds_void*)(lv + (4 * wave + i) * 1024), 16, 0, 0);
    }
  };

  AttnState st;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) st.o[qb][i] = (f32x16){};
    st.m_run[qb] = -INFINITY;
    st.l_run[qb] = 0.f;
  }
  const float c = a.scale_log2;
  const float grow_thr = RESCALE_LOG2 / c;   // raw-score margin before the max is raised
  const int n_full = (int)(a.Lkv / KT);

  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = 0; t < n_full; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) issue(t + 1, buf ^ 1);
    attn_tile<false>(st, qf, lds[buf], lds[buf] + K_TILE_BYTES, l32, g, c, grow_thr, KT);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (n_full < n_tiles) {   // partial last tile, already in LDS
    const int buf = n_full & 1;
    attn_tile<true>(st, qf, lds[buf], lds[buf] + K_TILE_BYTES, l32, g, c, grow_thr, (int)(a.Lkv - (int64_t)n_full * KT));
  }

  // ---- normalise and store: o[qb][dt] element r holds d = 32 dt + 8 (r/4) + 4 g + r%4 of query qi[qb]
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l_tot = st.l_run[qb] + __shfl_xor(st.l_run[qb], 32, 64);
    const float inv = 1.0f / l_tot;
    if (qi[qb] < a.Lq) {
      bf16_t* op = a.o + ((int64_t)b * a.Lq + qi[qb]) * a.ldo + h * 128 + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          u32x2 w;
          w.x = pack_bf16x2(st.o[qb][dt][4 * rg] * inv, st.o[qb][dt][4 * rg + 1] * inv);
          w.y = pack_bf16x2(st.o[qb][dt][4 * rg + 2] * inv, st.o[qb][dt][4 * rg + 3] * inv);
          *(u32x2*)(op + 32 * dt + 8 * rg) = w;
        }
    }
  }
}

}  // namespace

hipError_t launch_attention(const bf16_t* q, int64_t ldq, const bf16_t* k, int64_t ldk, const bf16_t* vt, int64_t ldv,
                            bf16_t* o, int64_t ldo, int64_t B, int64_t Lq, int64_t Lkv, int nh, bool self_attn,
                            hipStream_t s) {
  if (B <= 0 || Lq <= 0) return hipSuccess;
  if (Lkv <= 0 || ldv < round_up(Lkv, KT)) return hipErrorInvalidValue;
  AttnArgs a;
  a.q = q; a.ldq = ldq; a.k = k; a.ldk = ldk; a.vt = vt; a.ldv = ldv; a.o = o; a.ldo = ldo;
  a.Lq = Lq; a.Lkv = Lkv; a.nh = nh; a.B = (int)B;
  a.q_tiles = (int)ceil_div(Lq, QB);
  a.scale_log2 = (float)(1.4426950408889634 / sqrt(128.0));
  const int64_t nb = (int64_t)a.q_tiles * nh * B;
  if (self_attn) hipLaunchKernelGGL(k_flash_attn<true>, dim3((unsigned)nb), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_flash_attn<false>, dim3((unsigned)nb), dim3(256), 0, s, a);
  return hipGetLastError();
}
