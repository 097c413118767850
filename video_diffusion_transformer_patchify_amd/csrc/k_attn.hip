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
//     together with the exp / row-sum / bf16 packing of S(j), then the PV MFMAs of sub-tile j together
//     with the copy of S(j+1) out of the accumulator registers, so matrix and vector work of one wave
//     overlap.  The K and Vt fragments of a step are read from LDS during the step before it.
//   * Softmax in base 2: Q enters the score MFMAs multiplied by log2(e)/sqrt(128), so S is already in
//     log2 units and a probability is one exp2 of an accumulator value, with no offset at all: the row's
//     scores are not reduced to a running max while they stay in a safe range (any common offset of
//     numerator and denominator cancels in the final division).  Each lane's total probability sum is
//     checked against 2^64 after the last sub-tile (every probability is at most that sum, so nothing
//     overflowed on the way; an infinite or NaN probability fails the check too), and the first
//     sub-tile's row max against -60 (the largest probability stays a normal float); both checks are
//     branch-free, so the loop stays one block.  A wave whose rows leave that range drops its results
//     and marks its unit; the exact
//     kernel (same file, EXACT) then recomputes the marked units with the online softmax: a running
//     max, raised only when a sub-tile's max passes it by more than 8 (the stale max keeps
//     probabilities below 2^8), rescaling O and l when it is.
//   * Row sums (offset-free kernel) run on the matrix cores: v_mfma_f32_4x4x4_16b_bf16 with an all-ones
//     A operand adds each lane's own bf16 probabilities (the ones the PV MFMAs use) into an fp32
//     accumulator, 8 small MFMAs per step in place of 32 vector adds; the two lane halves of a row are
//     combined once at the end.  The exact kernel sums on the vector units (its sums are rescaled).
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
constexpr float SUM_LIMIT = 18446744073709551616.0f;   // 2^64: largest per-lane row sum, offset-free
constexpr float MAX_FLOOR = -60.0f;                    // smallest first-sub-tile row max, offset-free
constexpr float RESCALE_LOG2 = 8.0f;                   // exact path: margin before the running max is raised
constexpr int64_t ATTN_SPLIT_MAX = 256;   // workgroups of a key-split launch (default workspace size)

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
  float q_mul;        // factor applied to Q as it is loaded (1 when the caller stored Q pre-multiplied)
  int units;          // workgroups of the regular launch: units 0 .. units-1, unit = (b, h, query tile)
  // key-split launch: workgroup w works on unit units_base + w / split over keys
  // [chunk (w % split), chunk (w % split + 1)) and writes unnormalised partial results
  int split, units_base;
  int64_t chunk;
  float* part_o;      // [w][256 queries][128]: sum over the chunk's keys of p * v (p relative to m)
  float* part_ml;     // [w][256 queries][2]: exponent offset m (log2 units) and row sum l
  unsigned* flags;    // per workgroup, 4 wave flags: results dropped, recompute exactly (see k_flash_attn)
  int accumulate;     // 1: o += this attention's output (o holds another key set's normalised output)
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
  float l_run[2];   // this lane half's sum of the row's probabilities
  float m[2];       // exponent offset of the probabilities (log2 units): 0 offset-free, else the running max
  bool bad;         // offset-free kernel, wave-uniform: a row left the safe range (the unit is redone exactly)
  f32x4 lacc[2];    // offset-free kernel: this lane's sum of its bf16 probabilities (4 equal copies: the
                    // 4x4x4 MFMA's output rows)
};

typedef short s16x4 __attribute__((ext_vector_type(4)));   // 4 bf16: an operand of the 4x4x4 bf16 MFMA
__device__ __forceinline__ s16x4 as_s16x4(uint32_t a, uint32_t b) { return __builtin_bit_cast(s16x4, (u32x2){a, b}); }

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

// One copy of the scores out of the accumulator registers into the registers the softmax reads (the
// loop then carries them there: the prologue's and the loop's copies meet in the same registers).
__device__ __forceinline__ void to_vgprs(const f32x16 (&src)[2], f32x16 (&dst)[2]) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = src[qb][r];
      asm volatile("" : "+v"(x));
      dst[qb][r] = x;
    }
}

// Row max of one query block's sub-tile scores (both lane halves agree).
__device__ __forceinline__ float row_max(const f32x16& s) {
  float m = fmaxf(s[0], s[1]);
#pragma unroll
  for (int r = 2; r < 16; ++r) m = fmaxf(m, s[r]);
  // lanes 0-31 and 32-63 hold the two key halves of the same queries: swap halves and combine
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// P = exp2(s - m) as bf16 B-operand fragments (two 16-key steps per query block); OFFSET (the exact
// kernel) also this lane's fp32 sums.
template <bool OFFSET>
__device__ __forceinline__ void probs(const f32x16 (&s)[2], const float (&m)[2], u32x4 (&pf)[2][2], float (&ls)[2]) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float sum = 0.f;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(OFFSET ? s[qb][8 * hh + e] - m[qb] : s[qb][8 * hh + e]);
        if constexpr (OFFSET) sum = (hh == 0 && e == 0) ? p[e] : sum + p[e];
      }
      u32x4 w;
      w.x = pack_bf16x2(p[0], p[1]); w.y = pack_bf16x2(p[2], p[3]);
      w.z = pack_bf16x2(p[4], p[5]); w.w = pack_bf16x2(p[6], p[7]);
      pf[qb][hh] = w;
    }
    ls[qb] = sum;
  }
}

// Exact path: raise the running max where this sub-tile's max passed it by more than 8; rescale O, l.
__device__ __forceinline__ void raise_max(AttnState& st, const f32x16 (&s)[2]) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float mx = row_max(s[qb]);
    const bool grow = mx > st.m[qb] + RESCALE_LOG2;
    if (__any(grow)) {
      const float m_new = grow ? mx : st.m[qb];
      const float alpha = __builtin_amdgcn_exp2f(st.m[qb] - m_new);
      st.m[qb] = m_new;
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

// Probabilities of the current sub-tile into pf; their sums accumulate.  EXACT: against the running max,
// summed into l_run.  Otherwise offset-free, summed into lacc by MFMAs (the 4x4x4 MFMA's output column is
// the lane that holds the B operand's column, so with A = 1 each lane adds its own 4 values); finish_sums
// checks the totals.
template <bool EXACT>
__device__ __forceinline__ void softmax_step(AttnState& st, const f32x16 (&s)[2], u32x4 (&pf)[2][2]) {
  float ls[2];
  if constexpr (EXACT) {
    raise_max(st, s);
    probs<true>(s, st.m, pf, ls);
    st.l_run[0] += ls[0];
    st.l_run[1] += ls[1];
  } else {
    probs<false>(s, st.m, pf, ls);
    const s16x4 ones = as_s16x4(0x3F803F80u, 0x3F803F80u);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        st.lacc[qb] =
            __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ones, as_s16x4(pf[qb][hh].x, pf[qb][hh].y), st.lacc[qb], 0, 0, 0);
        st.lacc[qb] =
            __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ones, as_s16x4(pf[qb][hh].z, pf[qb][hh].w), st.lacc[qb], 0, 0, 0);
      }
  }
}
// Offset-free kernel, after the last step: the lane sums into l_run, and the wave is marked bad if any
// lane's sum left the safe range (above SUM_LIMIT, infinite or NaN).
__device__ __forceinline__ void finish_sums(AttnState& st) {
  st.l_run[0] = st.lacc[0][0];
  st.l_run[1] = st.lacc[1][0];
  st.bad |= __any(!(fmaxf(st.l_run[0], st.l_run[1]) <= SUM_LIMIT));
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

// K fragments of sub-tile `sub` of an LDS tile (rows in key_perm order), and the scores from them.
__device__ __forceinline__ void read_k(u32x4 (&kf)[8], const char* lk, int sub, int l32, int g) {
  const int row = KS * sub + key_perm(l32);
  const char* kr = lk + row * 256;
  const int sw = k_swz(row);
#pragma unroll
  for (int st = 0; st < 8; ++st) kf[st] = *(const u32x4*)(kr + (((2 * st + g) ^ sw) << 4));
}
__device__ __forceinline__ void scores_kf(f32x16 (&s)[2], const u32x4 (&qf)[2][8], const u32x4 (&kf)[8]) {
  s[0] = (f32x16){};
  s[1] = (f32x16){};
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[st]), as_bf16x8(qf[0][st]), s[0], 0, 0, 0);
    s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[st]), as_bf16x8(qf[1][st]), s[1], 0, 0, 0);
  }
}
// Vt fragments of sub-tile `sub` (the A operands of its PV MFMAs), and the PV MFMAs from them.
__device__ __forceinline__ void read_v(u32x4 (&vf)[4][2], const char* lv, int sub, int l32, int g) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int row = 32 * dt + l32;
    const char* vr = lv + row * 128;
    const int sw = v_swz(row);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) vf[dt][jj] = *(const u32x4*)(vr + (((2 * (2 * sub + jj) + g) ^ sw) << 4));
  }
}
__device__ __forceinline__ void pv_vf(AttnState& st, const u32x4 (&pf)[2][2], const u32x4 (&vf)[4][2]) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      st.o[0][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[dt][jj]), as_bf16x8(pf[0][jj]), st.o[0][dt], 0, 0, 0);
      st.o[1][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[dt][jj]), as_bf16x8(pf[1][jj]), st.o[1][dt], 0, 0, 0);
    }
}

// SELF selects the instantiation only (self- and cross-attention then show up as separate kernels in
// a trace); the code path is the same.  PART: one key chunk of a unit, unnormalised output (see
// AttnArgs); the last round of a launch that would leave most CUs idle is run this way.  EXACT: the
// online softmax with a running max.  The offset-free kernel (EXACT false) writes, per wave, whether
// its rows stayed in range to a.flags[4 w + wave] (w = the workgroup's unit, or its split workgroup)
// and drops the results of a wave that did not; the exact kernel launched after it with the same
// grid recomputes exactly the workgroups with a flag set and returns at once for the others.  With
// a.flags null the exact kernel computes every workgroup.
template <bool SELF, bool PART, bool EXACT>
__global__ __launch_bounds__(256, 1) void k_flash_attn(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[NBUF][TILE_BYTES];

  // the wave index is uniform: held in a scalar register, every direct load's LDS address (M0) is
  // scalar arithmetic instead of a vector add and a readfirstlane per load
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  // Workgroups of one (batch, head) are kept on one XCD so they share K/V in its L2.
  const int lid = PART ? a.units_base + (int)blockIdx.x / a.split : xcd_remap(blockIdx.x, a.units);
  const int wg = PART ? (int)blockIdx.x : lid;   // index of this workgroup's redo flags
  if constexpr (EXACT) {
    if (a.flags != nullptr) {
      const u32x4 f = *(const u32x4*)(a.flags + 4 * (int64_t)wg);
      if ((f.x | f.y | f.z | f.w) == 0u) return;   // whole workgroup, before any barrier
    }
  }
  const int64_t k_lo = PART ? (int64_t)((int)blockIdx.x % a.split) * a.chunk : 0;
  // keys of this workgroup: [k_lo, k_lo + Lkv) of its (batch, head)
  const int64_t Lkv = PART ? (a.Lkv - k_lo < a.chunk ? a.Lkv - k_lo : a.chunk) : a.Lkv;
  const int qt = lid % a.q_tiles;
  const int bh = lid / a.q_tiles;
  const int h = bh % a.nh, b = bh / a.nh;

  // ---- Q fragments (B operand of S^T = K Q^T): query l32 of block qb, d = 16 s + 8 g .. +7, times q_mul
  int64_t qi[2];
  u32x4 qf[2][8];
  const bool scale_q = a.q_mul != 1.0f;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    qi[qb] = (int64_t)qt * QB + wave * QWAVE + qb * 32 + l32;
    const int64_t qrow = qi[qb] < a.Lq ? qi[qb] : a.Lq - 1;
    const bf16_t* qp = a.q + ((int64_t)b * a.Lq + qrow) * a.ldq + h * 128 + g * 8;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 v = *(const u32x4*)(qp + 16 * s);
      if (scale_q) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = pack_bf16x2(lo_bf16(v[e]) * a.q_mul, hi_bf16(v[e]) * a.q_mul);
      }
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
    st.m[qb] = 0.f;
    st.l_run[qb] = 0.f;
    st.lacc[qb] = (f32x4){};
  }
  st.bad = false;
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
  // ---- prologue: batches of the barriers of tiles -4 and -2: [K0 K1 V0] [K2 K3 V1 V2]; tile 0
  //      resident; scores of sub-tile 0 and the offsets from their row max
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
  // Offset-free kernel: fragments are read one step ahead of their MFMAs, kf = K of the sub-tile whose
  // scores the next step forms, vf = Vt of the sub-tile whose PV it runs (the barrier schedule below
  // covers those reads too).  The exact kernel reads them where they are used (fewer live registers).
  constexpr bool AHEAD = !EXACT;
  u32x4 kf[8], vf[4][2];
  if constexpr (AHEAD) {
    read_k(kf, lds[0], 0, l32, g);
    scores_kf(s_next, qf, kf);
    if (n_sub > 1) read_k(kf, lds[0], 1, l32, g);
    read_v(vf, lds[0] + K_TILE_BYTES, 0, l32, g);
  } else {
    scores(s_next, qf, lds[0], 0, l32, g);
  }
  if (n_sub == 1 && last_lim < KS) mask_scores(s_next, g, last_lim);
  to_vgprs(s_next, s_cur);
  {
    // the first sub-tile holds at least one key, so its row max is finite.  Exact: the running max
    // starts there.  Offset-free: a row whose first sub-tile lies entirely below 2^-60 is out of range.
    const float mx0 = row_max(s_cur[0]), mx1 = row_max(s_cur[1]);
    if constexpr (EXACT) {
      st.m[0] = mx0;
      st.m[1] = mx1;
    } else {
      st.bad = __any(!(fminf(mx0, mx1) >= MAX_FLOOR));
    }
  }

  // One pipelined step j: head (barrier, loads, S(j+1)), the probabilities of sub-tile j, tail (PV(j)).
  // LAST: S(j+1) is the final sub-tile.
  // The second half of an even tile t opens with the workgroup barrier that covers the next four
  // steps, which read tiles t, t+1 and t+2 only: own loads of tiles t+1 and t+2 landed (both went out
  // at the previous barrier or in the prologue: vmcnt(0)), then every wave's.  Every wave is also past
  // its last read of K(t) (first half of tile t) and of V(t-1) (second half of tile t-1), so the K
  // regions of tiles <= t and the V regions of tiles <= t-1 take K(t+4), K(t+5), V(t+3), V(t+4).
  // Reading one step ahead stays inside that: the four steps then read K of sub-tiles 2t+3 .. 2t+6
  // (tiles t+1 .. t+3) and Vt of sub-tiles 2t+2 .. 2t+5 (tiles t+1, t+2); K(t+3) went out at the
  // previous barrier, so the vmcnt(0) + barrier here covers it as well.
  auto head = [&](int j, auto last_tag) {
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
    if constexpr (AHEAD) {
      scores_kf(s_next, qf, kf);
      if constexpr (!LAST) read_k(kf, lds[((j + 2) >> 1) % NBUF], (j + 2) & 1, l32, g);
    } else {
      scores(s_next, qf, lds[((j + 1) >> 1) % NBUF], (j + 1) & 1, l32, g);
    }
    if constexpr (LAST) {
      if (last_lim < KS) mask_scores(s_next, g, last_lim);
    }
  };
  // PV of sub-tile j; the next sub-tile's scores become current
  auto tail = [&](int j, const u32x4 (&pf)[2][2]) {
    if constexpr (AHEAD) {
      pv_vf(st, pf, vf);
      read_v(vf, lds[((j + 1) >> 1) % NBUF] + K_TILE_BYTES, (j + 1) & 1, l32, g);
    } else {
      pv(st, pf, lds[(j >> 1) % NBUF] + K_TILE_BYTES, j & 1, l32, g);
    }
    to_vgprs(s_next, s_cur);
  };
  int j = 0;
  for (; j + 2 < n_sub; ++j) {
    u32x4 pf[2][2];
    head(j, std::false_type{});
    softmax_step<EXACT>(st, s_cur, pf);
    tail(j, pf);
  }
  if (j + 1 < n_sub) {
    u32x4 pf[2][2];
    head(j, std::true_type{});
    softmax_step<EXACT>(st, s_cur, pf);
    tail(j, pf);
    ++j;
  }
  // ---- last sub-tile j = n_sub - 1
  {
    u32x4 pf[2][2];
    softmax_step<EXACT>(st, s_cur, pf);
    if constexpr (AHEAD) pv_vf(st, pf, vf);
    else pv(st, pf, lds[(j >> 1) % NBUF] + K_TILE_BYTES, j & 1, l32, g);
  }

  // ---- normalise and store: o[qb][dt] element r holds d = 32 dt + 8 (r/4) + 4 g + r%4 of query qi[qb]
  if constexpr (!EXACT) {
    finish_sums(st);
    if (lane == 0) a.flags[4 * (int64_t)wg + wave] = st.bad ? 1u : 0u;
    if (st.bad) return;
  } else {
    // redo pass: only the waves the offset-free kernel dropped store (the others' rows are in place,
    // and with accumulate they must not be added twice)
    if (a.flags != nullptr && a.flags[4 * (int64_t)wg + wave] == 0u) return;
  }
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
      if (g == 0) *(f32x2*)(a.part_ml + ((int64_t)blockIdx.x * QB + qloc) * 2) = (f32x2){st.m[qb], l_tot};
      continue;
    }
    const float inv = 1.0f / l_tot;
    if (qi[qb] < a.Lq) {
      bf16_t* op = a.o + ((int64_t)b * a.Lq + qi[qb]) * a.ldo + h * 128 + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          float v[4] = {st.o[qb][dt][4 * rg] * inv, st.o[qb][dt][4 * rg + 1] * inv, st.o[qb][dt][4 * rg + 2] * inv,
                        st.o[qb][dt][4 * rg + 3] * inv};
          if (a.accumulate) {
            const u32x2 prev = *(const u32x2*)(op + 32 * dt + 8 * rg);
            v[0] += lo_bf16(prev.x); v[1] += hi_bf16(prev.x); v[2] += lo_bf16(prev.y); v[3] += hi_bf16(prev.y);
          }
          u32x2 w;
          w.x = pack_bf16x2(v[0], v[1]);
          w.y = pack_bf16x2(v[2], v[3]);
          *(u32x2*)(op + 32 * dt + 8 * rg) = w;
        }
    }
  }
}

// Merge of the key chunks of the split units: per query, m = max_c m_c, w_c = 2^(m_c - m) (offsets in log2 units),
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
    const float w = __builtin_amdgcn_exp2f(a.part_ml[r * 2] - m);
    l = fmaf(a.part_ml[r * 2 + 1], w, l);
    acc = fmaf(a.part_o[r * 128 + d], w, acc);
  }
  bf16_t* op = a.o + ((int64_t)b * a.Lq + qi) * a.ldo + h * 128 + d;
  const float prev = a.accumulate ? bf16_to_f32(*op) : 0.f;
  *op = (bf16_t)(pack_bf16x2(acc / l + prev, 0.f) & 0xFFFFu);
}

// ---------------------------------------------------------------------------------------------------
// Cross-attention with the whole key set resident in LDS (at most RES_TILES * 64 keys: the text context).
// Persistent: one workgroup per CU walks a contiguous range of (batch, head, 256-query) units, loading a
// head's K and Vt tiles once (they stay for every query tile of that head it owns); each unit's Q is read
// into registers while the previous unit stores, and its output leaves through LDS as whole rows, so a
// unit costs its MFMA work and little else.  The probabilities are offset-free as in k_flash_attn, with
// the same redo marks: a wave whose rows leave the safe range stores nothing and marks its unit, and the
// exact k_flash_attn launched after it recomputes the marked units.
// ---------------------------------------------------------------------------------------------------
constexpr int RES_TILES = 4;

// One pass over the resident sub-tiles for the wave's two query blocks, software pipelined as in
// k_flash_attn (the scores of sub-tile j + 1 are formed with the probabilities of sub-tile j).
template <bool EXACT>
__device__ __forceinline__ void resident_pass(AttnState& st, const u32x4 (&qf)[2][8], char (*lds)[TILE_BYTES],
                                              int n_sub, int last_lim, int l32, int g) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) st.o[qb][i] = (f32x16){};
    st.m[qb] = 0.f;
    st.l_run[qb] = 0.f;
    st.lacc[qb] = (f32x4){};
  }
  st.bad = false;
  f32x16 s_cur[2], s_next[2];
  scores(s_next, qf, lds[0], 0, l32, g);
  if (n_sub == 1 && last_lim < KS) mask_scores(s_next, g, last_lim);
  to_vgprs(s_next, s_cur);
  {
    const float mx0 = row_max(s_cur[0]), mx1 = row_max(s_cur[1]);
    if constexpr (EXACT) {
      st.m[0] = mx0;
      st.m[1] = mx1;
    } else {
      st.bad = __any(!(fminf(mx0, mx1) >= MAX_FLOOR));
    }
  }
  int j = 0;
  for (; j + 2 < n_sub; ++j) {
    u32x4 pf[2][2];
    scores(s_next, qf, lds[(j + 1) >> 1], (j + 1) & 1, l32, g);
    softmax_step<EXACT>(st, s_cur, pf);
    pv(st, pf, lds[j >> 1] + K_TILE_BYTES, j & 1, l32, g);
    to_vgprs(s_next, s_cur);
  }
  if (j + 1 < n_sub) {
    u32x4 pf[2][2];
    scores(s_next, qf, lds[(j + 1) >> 1], (j + 1) & 1, l32, g);
    if (last_lim < KS) mask_scores(s_next, g, last_lim);
    softmax_step<EXACT>(st, s_cur, pf);
    pv(st, pf, lds[j >> 1] + K_TILE_BYTES, j & 1, l32, g);
    to_vgprs(s_next, s_cur);
    ++j;
  }
  {
    u32x4 pf[2][2];
    softmax_step<EXACT>(st, s_cur, pf);
    pv(st, pf, lds[j >> 1] + K_TILE_BYTES, j & 1, l32, g);
  }
  if constexpr (!EXACT) finish_sums(st);
}

constexpr int OSTAGE_BYTES = 32 * 256;   // one wave's 32 output rows of 128 bf16

__global__ __launch_bounds__(256, 1) void k_cross_attn(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[RES_TILES][TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char ostage[4][OSTAGE_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int64_t nwg = gridDim.x;
  const int u0 = (int)((int64_t)blockIdx.x * a.units / nwg), u1 = (int)((int64_t)(blockIdx.x + 1) * a.units / nwg);
  const int64_t Lkv = a.Lkv;
  const int n_tiles = (int)((Lkv + KT - 1) / KT);
  const int n_sub = (int)((Lkv + KS - 1) / KS);
  const int last_lim = (int)(Lkv - (int64_t)(n_sub - 1) * KS);
  // per-lane offsets of the direct loads, as in k_flash_attn
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
  const bool scale_q = a.q_mul != 1.0f;
  // Q of a unit (query l32 of block qb, d = 16 s + 8 g .. +7), read into registers.  The next unit's Q is
  // requested right after this unit's MFMAs and before its stores (the stores are unconditional, so the
  // wait for it at the next unit counts them and does not wait for them).
  const int qrow0 = wave * QWAVE + l32;
  u32x4 nq[2][8];
  auto load_q = [&](int u) {
    const int qt = u % a.q_tiles, bh = u / a.q_tiles;
    const int h = bh % a.nh, b = bh / a.nh;
    const char* qbase = (const char*)(a.q + ((int64_t)b * a.Lq + (int64_t)qt * QB) * a.ldq + h * 128);
    const int lim = (int)(a.Lq - 1 - (int64_t)qt * QB);   // rows past Lq re-read the last row
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int r = min(qrow0 + 32 * qb, lim);
      const uint32_t off = (uint32_t)((r * (int)a.ldq + g * 8) * 2);
#pragma unroll
      for (int s = 0; s < 8; ++s) nq[qb][s] = *(const u32x4*)(qbase + off + 32 * s);
    }
  };
  if (u0 < u1) load_q(u0);
  int cur_bh = -1;
  for (int u = u0; u < u1; ++u) {
    const int qt = u % a.q_tiles, bh = u / a.q_tiles;
    const int h = bh % a.nh, b = bh / a.nh;
    if (bh != cur_bh) {
      // a new head: every wave is past its reads of the previous one, then its K and Vt tiles come in
      block_sync();
      const bf16_t* kbase = a.k + (int64_t)b * a.Lkv * a.ldk + h * 128;
      const bf16_t* vbase = a.vt + ((int64_t)b * a.nh + h) * 128 * a.ldv;
      for (int t = 0; t < n_tiles; ++t) {
        const int64_t key0 = (int64_t)t * KT;
        const char* kt = (const char*)(kbase + key0 * a.ldk);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // rows past the last key re-read the last valid one (their scores are masked)
          const int64_t key = key0 + k_row[i] < Lkv ? k_row[i] : Lkv - 1 - key0;
          const uint32_t off = (uint32_t)(k_off[i] + (key - k_row[i]) * a.ldk * 2);
          __builtin_amdgcn_global_load_lds((const void*)(kt + off), (lds_void*)(lds[t] + (4 * wave + i) * 1024), 16,
                                           0, 0);
        }
        const char* vtb = (const char*)(vbase + key0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __builtin_amdgcn_global_load_lds((const void*)(vtb + v_off[i]),
                                           (lds_void*)(lds[t] + K_TILE_BYTES + (4 * wave + i) * 1024), 16, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
      block_sync();
      cur_bh = bh;
    }
    u32x4 qf[2][8];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        u32x4 v = nq[qb][s];
        if (scale_q) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = pack_bf16x2(lo_bf16(v[e]) * a.q_mul, hi_bf16(v[e]) * a.q_mul);
        }
        asm volatile("; q fragment %0" : "=a"(qf[qb][s]) : "0"(v));
      }
    }
    AttnState st;
    resident_pass<false>(st, qf, lds, n_sub, last_lim, l32, g);
    if (u + 1 < u1) load_q(u + 1);
    // a wave whose rows left the offset-free range marks its unit for the exact kernel and stores nothing
    if (lane == 0) a.flags[4 * (int64_t)u + wave] = st.bad ? 1u : 0u;
    if (st.bad) continue;
    // Normalise and store, one query block at a time through the wave's LDS stage: lane (l32, g) puts
    // its 4-value runs of row l32 into 16-byte chunk c = 4 dt + rg (8-byte half g) at position c ^ (l32 &
    // 15) (conflict-free), then 16 lanes per row read back the row's 16 chunks, so each store
    // instruction writes 4 whole 256-byte rows.
    char* stg = ostage[wave];
    const int c16 = lane & 15, r4 = lane >> 4;
    // a buffer resource covering this tile's valid rows: stores (and reads) of rows past Lq fall outside
    // it and the hardware drops them, so every lane issues the same memory operations
    const int64_t valid = a.Lq - (int64_t)qt * QB < QB ? a.Lq - (int64_t)qt * QB : QB;
    const auto orsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.o + ((int64_t)b * a.Lq + (int64_t)qt * QB) * a.ldo + h * 128), 0,
        (int)((valid - 1) * a.ldo * 2 + 256), 0x00020000);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float l_tot = st.l_run[qb] + __shfl_xor(st.l_run[qb], 32, 64);
      const float inv = 1.0f / l_tot;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          u32x2 w;
          w.x = pack_bf16x2(st.o[qb][dt][4 * rg] * inv, st.o[qb][dt][4 * rg + 1] * inv);
          w.y = pack_bf16x2(st.o[qb][dt][4 * rg + 2] * inv, st.o[qb][dt][4 * rg + 3] * inv);
          const int c = 4 * dt + rg;
          *(u32x2*)(stg + l32 * 256 + ((c ^ (l32 & 15)) << 4) + 8 * g) = w;
        }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the stage is written before any lane reads it
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 4 * i + r4;
        u32x4 d = *(const u32x4*)(stg + row * 256 + ((c16 ^ (row & 15)) << 4));
        const int off = ((wave * QWAVE + qb * 32 + row) * (int)a.ldo + 8 * c16) * 2;
        if (a.accumulate) {
          const u32x4 prev = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(orsrc, off, 0, 0));
#pragma unroll
          for (int e = 0; e < 4; ++e)
            d[e] = pack_bf16x2(lo_bf16(d[e]) + lo_bf16(prev[e]), hi_bf16(d[e]) + hi_bf16(prev[e]));
        }
        __builtin_amdgcn_raw_buffer_store_b128(d, orsrc, off, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // reads done before the next block overwrites the stage
      __builtin_amdgcn_wave_barrier();
    }
  }
}

}  // namespace

// Workspace: key-split partial outputs [split_cap][256][128] fp32, their (m, l) [split_cap][256][2], then the
// redo flags: 4 per workgroup of the regular launch and of the key-split launch.
int64_t attention_workspace_bytes(int64_t B, int64_t Lq, int nh, int64_t split_cap) {
  const int64_t units = B * nh * ceil_div(Lq, QB);
  return split_cap * QB * (128 + 2) * 4 + 16 * (units + split_cap);
}

hipError_t launch_attention(const bf16_t* q, int64_t ldq, const bf16_t* k, int64_t ldk, const bf16_t* vt, int64_t ldv,
                            bf16_t* o, int64_t ldo, int64_t B, int64_t Lq, int64_t Lkv, int nh, bool self_attn,
                            hipStream_t s, float* ws, int64_t ws_bytes, bool q_prescaled, bool accumulate,
                            int64_t split_cap) {
  if (B <= 0 || Lq <= 0) return hipSuccess;
  if (Lkv <= 0 || ldv < round_up(Lkv, KT)) return hipErrorInvalidValue;
  if (split_cap < 1) return hipErrorInvalidValue;
  if (ws != nullptr && ws_bytes < attention_workspace_bytes(B, Lq, nh, split_cap)) return hipErrorInvalidValue;
  AttnArgs a;
  a.q = q; a.ldq = ldq; a.k = k; a.ldk = ldk; a.vt = vt; a.ldv = ldv; a.o = o; a.ldo = ldo;
  a.Lq = Lq; a.Lkv = Lkv; a.nh = nh; a.B = (int)B;
  a.q_tiles = (int)ceil_div(Lq, QB);
  a.scale_log2 = (float)(1.4426950408889634 / sqrt(128.0));
  a.q_mul = q_prescaled ? 1.0f : a.scale_log2;
  a.split = 1; a.units_base = 0; a.chunk = Lkv; a.part_o = nullptr; a.part_ml = nullptr; a.flags = nullptr;
  a.accumulate = accumulate ? 1 : 0;
  const int64_t units = (int64_t)a.q_tiles * nh * B;
  // One workgroup per CU at a time: the last round holds units % CUs workgroups.  When it is at most half
  // full, its units are split over key chunks (multiples of 64 keys) so that it fills the chip, and a
  // merge pass forms their outputs.
  // CUs of the current device, asked per launch (the runtime keeps device attributes; devices may differ)
  int n_cu = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n_cu <= 0)
    n_cu = 256;
  if (!self_attn && Lkv <= RES_TILES * KT && ws != nullptr) {
    // keys resident in LDS: the persistent cross-attention kernel, then the exact kernel on the units it
    // marked (it returns at once for the others)
    a.units = (int)units;
    a.flags = (unsigned*)(ws + split_cap * QB * (128 + 2));
    hipLaunchKernelGGL(k_cross_attn, dim3((unsigned)(units < n_cu ? units : n_cu)), dim3(256), 0, s, a);
    hipLaunchKernelGGL((k_flash_attn<false, false, true>), dim3((unsigned)units), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const int64_t tail = units % n_cu;
  int64_t split = 1, chunk = Lkv;
  if (ws != nullptr && tail > 0 && 2 * tail <= n_cu) {
    chunk = round_up(ceil_div(Lkv, n_cu / tail), KT);
    split = ceil_div(Lkv, chunk);
    if (split < 2 || tail * split > split_cap) split = 1;
  }
  auto launch = [&](auto self_tag, auto part_tag, auto exact_tag, int64_t grid) {
    constexpr bool SELF = decltype(self_tag)::value, PART = decltype(part_tag)::value;
    constexpr bool EXACT = decltype(exact_tag)::value;
    if (grid > 0) hipLaunchKernelGGL((k_flash_attn<SELF, PART, EXACT>), dim3((unsigned)grid), dim3(256), 0, s, a);
  };
  // with a workspace: the offset-free kernel, then the exact kernel on the workgroups it flagged;
  // without one: the exact kernel alone
  auto run = [&](auto part_tag, int64_t grid) {
    using T = std::true_type;
    using F = std::false_type;
    if (a.flags != nullptr) {
      if (self_attn) launch(T{}, part_tag, F{}, grid);
      else launch(F{}, part_tag, F{}, grid);
    }
    if (self_attn) launch(T{}, part_tag, T{}, grid);
    else launch(F{}, part_tag, T{}, grid);
  };
  unsigned* flags = ws ? (unsigned*)(ws + split_cap * QB * (128 + 2)) : nullptr;
  a.units = (int)(split > 1 ? units - tail : units);
  a.flags = flags;
  run(std::false_type{}, a.units);
  if (split > 1) {
    a.split = (int)split; a.units_base = a.units; a.chunk = chunk;
    a.part_o = ws; a.part_ml = ws + split_cap * QB * 128;
    a.flags = flags + 4 * units;
    run(std::true_type{}, tail * split);
    hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)(tail * (QB / 2))), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

