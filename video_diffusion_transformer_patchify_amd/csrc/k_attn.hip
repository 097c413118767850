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
//   * K [key][d] and the pre-transposed V (Vt[b][h][d][key], so a tile is [d][key]) are copied
//     global -> LDS in tiles of 64 keys with gfx950's direct loads (global_load_lds_dwordx4: lane l of
//     an instruction fills bytes 16 l .. 16 l + 15 of a 1 KB LDS block), no register staging, five
//     buffers (160 KB): one workgroup barrier per two tiles, each followed by the K copies of tiles
//     t+4, t+5 and the V copies of tiles t+3, t+4, so every load has at least four 32-key steps to
//     land.  The 16-byte
//     chunks of each LDS row are XOR-swizzled so the fragment reads are free of bank conflicts; the
//     swizzle is applied by choosing which global chunk each lane fetches.
//   * Scores are formed transposed, S^T = K Q^T: the accumulator's column is the lane's query, so the
//     probabilities P^T come out of the accumulator already in the B-operand layout of the PV MFMA
//     (O^T += V^T P^T) once the 32 key rows of a K fragment are taken in the order pi(i), which swaps
//     bits 2 and 3 of i.  With that order, lane half g holds keys 8g..8g+7 (+16) of each 16-key step.
//   * Keys are processed in 32-key sub-tiles j, software pipelined: the MFMAs of S(j+1) are issued
//     together with the exp / row-sum / bf16 packing of S(j), and the PV MFMAs of sub-tile j together
//     with the row max of S(j+1), so matrix and vector work of one wave overlap.
//   * Softmax in base 2 with the 1/sqrt(128) scale folded into one FMA per score.  The running max is
//     only raised when a sub-tile's max exceeds it by more than 8 (log2 units): until then the stale
//     max is kept (probabilities up to 2^8, exact after the final division because numerator and
//     denominator share it) and the O rescale is skipped.
//   * Row max is shared between the two lane halves with one cross-lane exchange per sub-tile; row
//     sums stay per lane half and are combined once at the end.
//   * Only the last sub-tile can be partial; its scores are masked in a peeled copy of the loop body.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace {

constexpr int KT = 64;              // keys per LDS tile
constexpr int KS = 32;              // keys per sub-tile
constexpr int NBUF = 5;             // LDS tile buffers
constexpr int QWAVE = 64;           // queries per wave (two 32-query blocks)
constexpr int QB = 4 * QWAVE;       // queries per workgroup
constexpr int K_TILE_BYTES = KT * 256;     // 64 rows of 128 bf16
constexpr int V_TILE_BYTES = 128 * KT * 2; // 128 rows of 64 bf16
constexpr int TILE_BYTES = K_TILE_BYTES + V_TILE_BYTES;
constexpr float RESCALE_LOG2 = 8.0f;
constexpr int64_t ATTN_SPLIT_MAX = 256;   // workgroups of a key-split launch (workspace size)

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
  int units;          // workgroups of the regular launch: units 0 .. units-1, unit = (b, h, query tile)
  // key-split launch: workgroup w works on unit units_base + w / split over keys
  // [chunk (w % split), chunk (w % split + 1)) and writes unnormalised partial results
  int split, units_base;
  int64_t chunk;
  float* part_o;      // [w][256 queries][128]: sum over the chunk's keys of p * v (p relative to m)
  float* part_ml;     // [w][256 queries][2]: running max m (raw score units) and row sum l
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
  float mc[2];   // -m_run * c, the exponent offset of the probabilities
};

// S^T for sub-tile `sub` (0 or 1) of an LDS tile, both query blocks; each K fragment read once.
__device__ __forceinline__ void scores(f32x16 (&s)[2], const u32x4 (&qf)[2][8], const char* lk, int sub, int l32,
                                       int g) {
  const int row = KS * sub + key_perm(l32);
  const char* kr = lk + row * 256;
  const int sw = k_swz(row);
  s[0] = (f32x16){};
  s[1] = (f32x16){};
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    u32x4 kf = *(const u32x4*)(kr + (((2 * st + g) ^ sw) << 4));
    s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(qf[0][st]), s[0], 0, 0, 0);
    s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(qf[1][st]), s[1], 0, 0, 0);
  }
}

// Scores of keys >= key_lim (sub-tile relative) become -inf.  Element r holds key 16 (r/8) + 8 g + r%8.
__device__ __forceinline__ void mask_scores(f32x16 (&s)[2], int g, int key_lim) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = 16 * (r >> 3) + 8 * g + (r & 7);
      if (kk >= key_lim) s[qb][r] = -INFINITY;
    }
}

// Row max of a sub-tile's scores for both query blocks (both lane halves agree).
__device__ __forceinline__ void row_max(f32x16 (&s)[2], float (&mx)[2]) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = s[qb][r];
      asm volatile("" : "+v"(x));   // one copy out of the accumulator registers, reused by probs()
      s[qb][r] = x;
    }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float m = fmaxf(s[qb][0], s[qb][1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) m = fmaxf(m, s[qb][r]);
    // lanes 0-31 and 32-63 hold the two key halves of the same queries: swap halves and combine
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    mx[qb] = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  }
}

// Raise the running max where a sub-tile's max passed it by more than the margin; rescale O and l.
__device__ __forceinline__ void maybe_rescale(AttnState& st, const float (&mx)[2], float c, float grow_thr) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const bool grow = mx[qb] > st.m_run[qb] + grow_thr;
    if (__any(grow)) {
      const float m_new = grow ? mx[qb] : st.m_run[qb];
      const float alpha = __builtin_amdgcn_exp2f((st.m_run[qb] - m_new) * c);
      st.m_run[qb] = m_new;
      st.mc[qb] = -m_new * c;
      st.l_run[qb] *= alpha;
      // one 16-register accumulator at a time: they live in AGPRs, each multiply needs VGPR temporaries
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        st.o[qb][dt] *= alpha;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

// P = exp2(s c - m c) as bf16 B-operand fragments (two 16-key steps per query block); l += row sums.
__device__ __forceinline__ void probs(AttnState& st, const f32x16 (&s)[2], u32x4 (&pf)[2][2], float c) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float mc = st.mc[qb];
    float ls;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(fmaf(s[qb][8 * hh + e], c, mc));
        ls = (hh == 0 && e == 0) ? p[e] : ls + p[e];
      }
      u32x4 w;
      w.x = pack_bf16x2(p[0], p[1]); w.y = pack_bf16x2(p[2], p[3]);
      w.z = pack_bf16x2(p[4], p[5]); w.w = pack_bf16x2(p[6], p[7]);
      pf[qb][hh] = w;
    }
    st.l_run[qb] += ls;
  }
}

// O^T += V^T P^T for sub-tile `sub` of an LDS tile: A = Vt rows d = 32 dt + l32, keys 32 sub + 16 jj + 8 g.
__device__ __forceinline__ void pv(AttnState& st, const u32x4 (&pf)[2][2], const char* lv, int sub, int l32, int g) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int row = 32 * dt + l32;
    const char* vr = lv + row * 128;
    const int sw = v_swz(row);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      u32x4 vf = *(const u32x4*)(vr + (((2 * (2 * sub + jj) + g) ^ sw) << 4));
      st.o[0][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pf[0][jj]), st.o[0][dt], 0, 0, 0);
      st.o[1][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pf[1][jj]), st.o[1][dt], 0, 0, 0);
    }
  }
}

// SELF selects the instantiation only (self- and cross-attention then show up as separate kernels in
// a trace); the code path is the same.  PART: one key chunk of a unit, unnormalised output (see
// AttnArgs); the last round of a launch that would leave most CUs idle is run this way.
template <bool SELF, bool PART>
__global__ __launch_bounds__(256, 1) void k_flash_attn(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[NBUF][TILE_BYTES];

  // the wave index is uniform: held in a scalar register, every direct load's LDS address (M0) is
  // scalar arithmetic instead of a vector add and a readfirstlane per load
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  // Workgroups of one (batch, head) are kept on one XCD so they share K/V in its L2.
  const int lid = PART ? a.units_base + (int)blockIdx.x / a.split : xcd_remap(blockIdx.x, a.units);
  const int64_t k_lo = PART ? (int64_t)((int)blockIdx.x % a.split) * a.chunk : 0;
  // keys of this workgroup: [k_lo, k_lo + Lkv) of its (batch, head)
  const int64_t Lkv = PART ? (a.Lkv - k_lo < a.chunk ? a.Lkv - k_lo : a.chunk) : a.Lkv;
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
    for (int s = 0; s < 8; ++s) {
      u32x4 v = *(const u32x4*)(qp + 16 * s);
      // MFMA source operands may come from AGPRs: Q lives there for the whole kernel, which leaves
      // the VGPRs to the score copies the softmax works on
      asm volatile("; q fragment %0" : "=a"(qf[qb][s]) : "0"(v));
    }
  }

  // ---- direct global -> LDS copies.  Each wave issues 4 K and 4 V instructions per tile.
  //   K: instruction I (= 4 wave + i) fills rows 4I .. 4I+3; lane -> row 4I + lane/16, position lane%16.
  //   V: instruction I fills rows 8I .. 8I+7; lane -> row 8I + lane/8, position lane%8.
  const bf16_t* kbase = a.k + ((int64_t)b * a.Lkv + k_lo) * a.ldk + h * 128;
  const bf16_t* vbase = a.vt + ((int64_t)b * a.nh + h) * 128 * a.ldv + k_lo;
  const int n_tiles = (int)((Lkv + KT - 1) / KT);
  const int n_sub = (int)((Lkv + KS - 1) / KS);
  // per-lane byte offsets inside a tile (K rows of the tile, Vt rows), fixed for the whole loop
  uint32_t k_off[4], v_off[4];
  int k_row[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int I = 4 * wave + i;
    k_row[i] = 4 * I + (lane >> 4);
    const int k_col = ((lane & 15) ^ k_swz(k_row[i])) * 8;
    k_off[i] = (uint32_t)(((int64_t)k_row[i] * a.ldk + k_col) * 2);
    const int v_row = 8 * I + (lane >> 3);
    const int v_col = ((lane & 7) ^ v_swz(v_row)) * 8;
    v_off[i] = (uint32_t)(((int64_t)v_row * a.ldv + v_col) * 2);
  }
  const bool tail_rows = (Lkv % KT) != 0;
  // half 0 of tile t: its 4 K instructions; half 1: its 4 V instructions
  auto issue = [&](int t, int part) {
    const int64_t key0 = (int64_t)t * KT;
    char* lk = lds[t % NBUF];
    if (part == 0) {
      const char* kt = (const char*)(kbase + key0 * a.ldk);
      if (tail_rows && t == n_tiles - 1) {
        // last, partial tile: rows past the end re-read the last valid row (their scores are masked)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t key = key0 + k_row[i] < Lkv ? k_row[i] : Lkv - 1 - key0;
          const uint32_t off = (uint32_t)(k_off[i] + (key - k_row[i]) * a.ldk * 2);
          __builtin_amdgcn_global_load_lds((const void*)(kt + off), (lds_void*)(lk + (4 * wave + i) * 1024), 16, 0, 0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __builtin_amdgcn_global_load_lds((const void*)(kt + k_off[i]), (lds_void*)(lk + (4 * wave + i) * 1024), 16, 0, 0);
      }
    } else {
      const char* vtb = (const char*)(vbase + key0);
      char* lv = lk + K_TILE_BYTES;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(vtb + v_off[i]), (lds_void*)(lv + (4 * wave + i) * 1024), 16, 0, 0);
    }
  };

  AttnState st;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) st.o[qb][i] = (f32x16){};
    st.m_run[qb] = -INFINITY;
    st.mc[qb] = INFINITY;
    st.l_run[qb] = 0.f;
  }
  const float c = a.scale_log2;
  const float grow_thr = RESCALE_LOG2 / c;   // raw-score margin before the max is raised
  const int last_lim = (int)(Lkv - (int64_t)(n_sub - 1) * KS);   // valid keys in the last sub-tile

  // vmcnt(n) for n in {0, 4, 8, 12, 16}, with or without lgkmcnt(0)
  auto wait_vm = [&](int n, auto lgkm0) {
    constexpr bool L0 = decltype(lgkm0)::value;
    if (n >= 16) __builtin_amdgcn_s_waitcnt(L0 ? 0x4070 : 0x4F70);
    else if (n >= 12) __builtin_amdgcn_s_waitcnt(L0 ? 0x007C : 0x0F7C);
    else if (n >= 8) __builtin_amdgcn_s_waitcnt(L0 ? 0x0078 : 0x0F78);
    else if (n >= 4) __builtin_amdgcn_s_waitcnt(L0 ? 0x0074 : 0x0F74);
    else __builtin_amdgcn_s_waitcnt(L0 ? 0x0070 : 0x0F70);
  };
  // ---- prologue: K0, then [K1 V0] [K2 V1] [K3 V2] (the batches the barriers of tiles -3..-1 would
  //      issue); tile 0 resident; scores and max of sub-tile 0
  // batches of the barriers of tiles -4 and -2: [K0 K1 V0] [K2 K3 V1 V2]
  issue(0, 0);
  if (1 < n_tiles) issue(1, 0);
  issue(0, 1);
#pragma unroll
  for (int b = 2; b <= 3; ++b)
    if (b < n_tiles) issue(b, 0);
#pragma unroll
  for (int b = 1; b <= 2; ++b)
    if (b < n_tiles) issue(b, 1);
  // own loads younger than V0: K2 K3 V1 V2
  wait_vm(4 * ((2 < n_tiles) + (3 < n_tiles) + (1 < n_tiles) + (2 < n_tiles)), std::false_type{});
  block_sync();
  f32x16 s_cur[2], s_next[2];
  float mx[2];
  scores(s_cur, qf, lds[0], 0, l32, g);
  if (n_sub == 1 && last_lim < KS) mask_scores(s_cur, g, last_lim);
  row_max(s_cur, mx);
  maybe_rescale(st, mx, c, grow_thr);

  // One pipelined step: S(j+1) with P(j); PV(j) with max(S(j+1)).  LAST: S(j+1) is the final sub-tile.
  // The second half of an even tile t opens with the workgroup barrier that covers the next four
  // steps, which read tiles t, t+1 and t+2 only: own loads of tiles t+1 and t+2 landed (both went out
  // at the previous barrier or in the prologue: vmcnt(0)), then every wave's.  Every wave is also past
  // its last read of K(t) (first half of tile t) and of V(t-1) (second half of tile t-1), so the K
  // regions of tiles <= t and the V regions of tiles <= t-1 take K(t+4), K(t+5), V(t+3), V(t+4).
  auto step = [&](int j, auto last_tag) {
    constexpr bool LAST = decltype(last_tag)::value;
    const int t = j >> 1, half = j & 1;
    if (half && !(t & 1)) {
      // tiles t+1 and t+2 landed (all issued at the previous barrier or before), then every wave's
      __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
      block_sync();
      // free: K regions of tiles <= t, V regions of tiles <= t-1
      if (t + 4 < n_tiles) issue(t + 4, 0);
      if (t + 5 < n_tiles) issue(t + 5, 0);
      if (t + 3 < n_tiles) issue(t + 3, 1);
      if (t + 4 < n_tiles) issue(t + 4, 1);
    }
    u32x4 pf[2][2];
    scores(s_next, qf, lds[((j + 1) >> 1) % NBUF], (j + 1) & 1, l32, g);
    probs(st, s_cur, pf, c);
    if constexpr (LAST) {
      if (last_lim < KS) mask_scores(s_next, g, last_lim);
    }
    pv(st, pf, lds[t % NBUF] + K_TILE_BYTES, half, l32, g);
    row_max(s_next, mx);
    maybe_rescale(st, mx, c, grow_thr);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) s_cur[qb] = s_next[qb];
  };
  int j = 0;
  for (; j + 2 < n_sub; ++j) step(j, std::false_type{});
  if (j + 1 < n_sub) {
    step(j, std::true_type{});
    ++j;
  }
  // ---- last sub-tile j = n_sub - 1
  {
    u32x4 pf[2][2];
    probs(st, s_cur, pf, c);
    pv(st, pf, lds[(j >> 1) % NBUF] + K_TILE_BYTES, j & 1, l32, g);
  }

  // ---- normalise and store: o[qb][dt] element r holds d = 32 dt + 8 (r/4) + 4 g + r%4 of query qi[qb]
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l_tot = st.l_run[qb] + __shfl_xor(st.l_run[qb], 32, 64);
    if constexpr (PART) {
      const int qloc = wave * QWAVE + qb * 32 + l32;
      float* po = a.part_o + ((int64_t)blockIdx.x * QB + qloc) * 128 + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg)
          *(f32x4*)(po + 32 * dt + 8 * rg) = (f32x4){st.o[qb][dt][4 * rg], st.o[qb][dt][4 * rg + 1],
                                                     st.o[qb][dt][4 * rg + 2], st.o[qb][dt][4 * rg + 3]};
      if (g == 0) *(f32x2*)(a.part_ml + ((int64_t)blockIdx.x * QB + qloc) * 2) = (f32x2){st.m_run[qb], l_tot};
      continue;
    }
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

// Merge of the key chunks of the split units: per query, m = max_c m_c, w_c = 2^((m_c - m) log2(e)/sqrt(128)),
// O = (sum_c w_c O_c) / (sum_c w_c l_c): the softmax over all keys, exactly as one pass would form it.
// One 256-thread workgroup per (unit, 2 queries), one thread per output element.
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a) {
  const int tu = (int)blockIdx.x / (QB / 2);
  const int q = ((int)blockIdx.x % (QB / 2)) * 2 + (int)(threadIdx.x >> 7), d = (int)threadIdx.x & 127;
  const int lid = a.units_base + tu;
  const int qt = lid % a.q_tiles, bh = lid / a.q_tiles;
  const int h = bh % a.nh, b = bh / a.nh;
  const int64_t qi = (int64_t)qt * QB + q;
  if (qi >= a.Lq) return;
  const int64_t w0 = (int64_t)tu * a.split;
  float m = -INFINITY;
  for (int c = 0; c < a.split; ++c) m = fmaxf(m, a.part_ml[((w0 + c) * QB + q) * 2]);
  float l = 0.f, acc = 0.f;
  for (int c = 0; c < a.split; ++c) {
    const int64_t r = (w0 + c) * QB + q;
    const float w = __builtin_amdgcn_exp2f((a.part_ml[r * 2] - m) * a.scale_log2);
    l = fmaf(a.part_ml[r * 2 + 1], w, l);
    acc = fmaf(a.part_o[r * 128 + d], w, acc);
  }
  a.o[((int64_t)b * a.Lq + qi) * a.ldo + h * 128 + d] = (bf16_t)(pack_bf16x2(acc / l, 0.f) & 0xFFFFu);
}

}  // namespace

int64_t attention_workspace_bytes() { return (int64_t)ATTN_SPLIT_MAX * QB * (128 + 2) * 4; }

hipError_t launch_attention(const bf16_t* q, int64_t ldq, const bf16_t* k, int64_t ldk, const bf16_t* vt, int64_t ldv,
                            bf16_t* o, int64_t ldo, int64_t B, int64_t Lq, int64_t Lkv, int nh, bool self_attn,
                            hipStream_t s, float* ws, int64_t ws_bytes) {
  if (B <= 0 || Lq <= 0) return hipSuccess;
  if (Lkv <= 0 || ldv < round_up(Lkv, KT)) return hipErrorInvalidValue;
  AttnArgs a;
  a.q = q; a.ldq = ldq; a.k = k; a.ldk = ldk; a.vt = vt; a.ldv = ldv; a.o = o; a.ldo = ldo;
  a.Lq = Lq; a.Lkv = Lkv; a.nh = nh; a.B = (int)B;
  a.q_tiles = (int)ceil_div(Lq, QB);
  a.scale_log2 = (float)(1.4426950408889634 / sqrt(128.0));
  a.split = 1; a.units_base = 0; a.chunk = Lkv; a.part_o = nullptr; a.part_ml = nullptr;
  const int64_t units = (int64_t)a.q_tiles * nh * B;
  // One workgroup per CU at a time: the last round holds units % CUs workgroups.  When it is at most half
  // full, its units are split over key chunks (multiples of 64 keys) so that it fills the chip, and a
  // merge pass forms their outputs.
  // CUs of the current device, asked per launch (the runtime keeps device attributes; devices may differ)
  int n_cu = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n_cu <= 0)
    n_cu = 256;
  const int64_t tail = units % n_cu;
  int64_t split = 1, chunk = Lkv;
  if (ws != nullptr && tail > 0 && 2 * tail <= n_cu) {
    chunk = round_up(ceil_div(Lkv, n_cu / tail), KT);
    split = ceil_div(Lkv, chunk);
    if (split < 2 || tail * split > ATTN_SPLIT_MAX || ws_bytes < attention_workspace_bytes()) split = 1;
  }
  auto launch = [&](auto self_tag, auto part_tag, int64_t grid) {
    constexpr bool SELF = decltype(self_tag)::value, PART = decltype(part_tag)::value;
    if (grid > 0) hipLaunchKernelGGL((k_flash_attn<SELF, PART>), dim3((unsigned)grid), dim3(256), 0, s, a);
  };
  using T = std::true_type;
  using F = std::false_type;
  a.units = (int)(split > 1 ? units - tail : units);
  if (self_attn) launch(T{}, F{}, a.units);
  else launch(F{}, F{}, a.units);
  if (split > 1) {
    a.split = (int)split; a.units_base = a.units; a.chunk = chunk;
    a.part_o = ws; a.part_ml = ws + (int64_t)ATTN_SPLIT_MAX * QB * 128;
    if (self_attn) launch(T{}, T{}, tail * split);
    else launch(F{}, T{}, tail * split);
    hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)(tail * (QB / 2))), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}
