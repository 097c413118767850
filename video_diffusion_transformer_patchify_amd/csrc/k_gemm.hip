// bf16 MFMA GEMM for gfx950 with fused epilogues, plus a small fp32 GEMM for the timestep MLP.
//
//   C[m, n] = sum_k X[m, k] * W[n, k]  (+ bias[n], then an epilogue)
//
// X is the activation (row-major, K contiguous), W an nn.Linear weight [N, K] (K contiguous), so both
// operands are read 16 bytes per lane straight into MFMA fragments.  The MFMA "A" operand is a W tile
// and the "B" operand an X tile, i.e. every 32x32 accumulator holds C^T: each lane then owns four
// consecutive output columns of one row, which makes the epilogue's stores 8- or 16-byte vector accesses.
//
// Epilogues (every nn.Linear of WanTransformerBlock.forward as printed on the WanPipeline notes page):
//   EPI_BF16       out_bf16 = acc + bias
//   EPI_GELU_BF16  out_bf16 = gelu_tanh(acc + bias)                       (FFN first Linear, text proj)
//   EPI_F32        out_f32  = acc + bias                                  (patch embed, proj_out)
//   EPI_RES_F32    out_f32 += acc + bias
//   EPI_GATE_F32   out_f32 += (acc + bias) * (gate_tab[n] + gate_src[row(m)][n])
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace {

constexpr int BK = 64;
constexpr int LDS_LD = BK + 8;  // bf16 per LDS row in the small kernel: 144 B rows, conflict-free reads

typedef __attribute__((address_space(3))) void lds_void;

struct GemmArgs {
  const bf16_t* x; int64_t ldx;
  const bf16_t* w; int64_t ldw;
  const float* bias;
  int64_t M, N, K;
  void* out; int64_t ldo;
  const float* gate_tab;   // [N] (already offset to the gate row)
  const float* gate_src;   // row-major, stride gate_ld, already offset to the gate column block
  int64_t gate_ld;
  int64_t rows_per_gate;   // tokens sharing one gate row (L for a per-sample timestep, 1 per-token)
  int tiles_m, tiles_n;
  // persistent kernel: tiles [0, dp_tiles) of the grouped order run whole, in full rounds.  The rest
  // (the stream-K tail: sk_tiles < one round) run as sk_split K chunks each, workgroup w < sk_tiles *
  // sk_split taking chunk w % sk_split of tail tile w / sk_split; each chunk writes its unbiased fp32
  // partial tile [256][256] to sk_part + 65536 w, and k_gemm_sk_fix sums them and applies the epilogue.
  int dp_tiles, sk_tiles, sk_split;
  float* sk_part;
};

// Dispatch order places consecutive workgroups on different XCDs (round robin over 8).  Renumber so
// that each XCD receives a contiguous range of logical tiles.
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int per = nb / 8, rem = nb % 8;
  const int xcd = b % 8, slot = b / 8;
  return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

// Epilogue of a wave's (32 TN) x (32 TM) output block.  acc[i][j] element r holds
// n = nb + 32 i + 8 (r/4) + 4 g + r%4, m = mb + 32 j + l32.  All bias fragments are loaded up front;
// for read-modify-write epilogues each row group's operands are fetched before any of it is used, so
// those loads are in flight together instead of one latency per 4 outputs.
template <int EPI, int TN, int TM>
__device__ __forceinline__ void store_tile(const GemmArgs& a, const f32x16 (&acc)[TN][TM], int64_t mb, int64_t nb, int l32,
                                           int g) {
  f32x4 bias[TN][4];
  const bool full_n = nb + 32 * TN <= a.N;
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      int64_t n = nb + 32 * i + 8 * rg + 4 * g;
      if (!full_n && n >= a.N) n = a.N - 4;
      bias[i][rg] = *(const f32x4*)(a.bias + n);
    }
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int64_t m = mb + 32 * j + l32;
    const bool row_ok = m < a.M;
    const int64_t mr = row_ok ? m : a.M - 1;
    f32x4 old[TN][4], gate[TN][4];
    if constexpr (EPI == EPI_RES_F32 || EPI == EPI_GATE_F32) {
      const int64_t gr = mr / a.rows_per_gate;
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          int64_t n = nb + 32 * i + 8 * rg + 4 * g;
          if (!full_n && n >= a.N) n = a.N - 4;
          old[i][rg] = *(const f32x4*)((const float*)a.out + mr * a.ldo + n);
          if constexpr (EPI == EPI_GATE_F32)
            gate[i][rg] = *(const f32x4*)(a.gate_tab + n) + *(const f32x4*)(a.gate_src + gr * a.gate_ld + n);
        }
    }
    if (!row_ok) continue;
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int64_t n = nb + 32 * i + 8 * rg + 4 * g;
        if (!full_n && n >= a.N) continue;
        f32x4 v = {acc[i][j][4 * rg], acc[i][j][4 * rg + 1], acc[i][j][4 * rg + 2], acc[i][j][4 * rg + 3]};
        v += bias[i][rg];
        if constexpr (EPI == EPI_BF16 || EPI == EPI_GELU_BF16) {
          if constexpr (EPI == EPI_GELU_BF16) {
            v.x = gelu_tanh_f(v.x); v.y = gelu_tanh_f(v.y); v.z = gelu_tanh_f(v.z); v.w = gelu_tanh_f(v.w);
          }
          u32x2 o;
          o.x = pack_bf16x2(v.x, v.y);
          o.y = pack_bf16x2(v.z, v.w);
          *(u32x2*)((bf16_t*)a.out + m * a.ldo + n) = o;
        } else if constexpr (EPI == EPI_F32) {
          *(f32x4*)((float*)a.out + m * a.ldo + n) = v;
        } else if constexpr (EPI == EPI_RES_F32) {
          *(f32x4*)((float*)a.out + m * a.ldo + n) = old[i][rg] + v;
        } else {
          *(f32x4*)((float*)a.out + m * a.ldo + n) = old[i][rg] + v * gate[i][rg];
        }
      }
  }
}

// ---------------------------------------------------------------------------------------------------
// Small-problem kernel: BM x BN workgroup tile, 4 waves of WM x WN, register-staged copies into padded
// LDS rows, double buffered.  M and N tails are clamped on load and guarded on store.
// ---------------------------------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(256, 2) void k_gemm_bf16(GemmArgs a) {
  static_assert((BM / WM) * (BN / WN) == 4, "4 waves");
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int XCH = BM * BK / 8 / 256;  // 16-byte chunks per thread for the X tile
  constexpr int WCH = BN * BK / 8 / 256;
  __shared__ __attribute__((aligned(16))) bf16_t lds[2][(BM + BN) * LDS_LD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = a.tiles_m * a.tiles_n;
  const int tile = xcd_remap(blockIdx.x, nb);
  const int tm = tile / a.tiles_n, tn = tile % a.tiles_n;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int wm0 = (wave / (BN / WN)) * WM, wn0 = (wave % (BN / WN)) * WN;
  const int l32 = lane & 31, g = lane >> 5;

  const bf16_t* xp[XCH];
  const bf16_t* wp[WCH];
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    int64_t r = m0 + (tid >> 3) + 32 * i;
    if (r > a.M - 1) r = a.M - 1;
    xp[i] = a.x + r * a.ldx + (tid & 7) * 8;
  }
#pragma unroll
  for (int i = 0; i < WCH; ++i) {
    int64_t r = n0 + (tid >> 3) + 32 * i;
    if (r > a.N - 1) r = a.N - 1;
    wp[i] = a.w + r * a.ldw + (tid & 7) * 8;
  }
  u32x4 xs[XCH], ws[WCH];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) xs[i] = *(const u32x4*)(xp[i] + kt * BK);
#pragma unroll
    for (int i = 0; i < WCH; ++i) ws[i] = *(const u32x4*)(wp[i] + kt * BK);
  };
  auto lstore = [&](int buf) {
    bf16_t* lx = lds[buf];
    bf16_t* lw = lds[buf] + BM * LDS_LD;
#pragma unroll
    for (int i = 0; i < XCH; ++i) *(u32x4*)(lx + ((tid >> 3) + 32 * i) * LDS_LD + (tid & 7) * 8) = xs[i];
#pragma unroll
    for (int i = 0; i < WCH; ++i) *(u32x4*)(lw + ((tid >> 3) + 32 * i) * LDS_LD + (tid & 7) * 8) = ws[i];
  };

  f32x16 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = (f32x16){};

  const int nk = (int)(a.K / BK);
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const bf16_t* lx = lds[buf];
    const bf16_t* lw = lds[buf] + BM * LDS_LD;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      u32x4 af[TN], bfr[TM];
#pragma unroll
      for (int i = 0; i < TN; ++i) af[i] = *(const u32x4*)(lw + (wn0 + 32 * i + l32) * LDS_LD + ks * 16 + g * 8);
#pragma unroll
      for (int j = 0; j < TM; ++j) bfr[j] = *(const u32x4*)(lx + (wm0 + 32 * j + l32) * LDS_LD + ks * 16 + g * 8);
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[i]), as_bf16x8(bfr[j]), acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }
  store_tile<EPI, TN, TM>(a, acc, m0 + wm0, n0 + wn0, l32, g);
}

// ---------------------------------------------------------------------------------------------------
// Large-problem kernel, persistent: 256 x 256 output tiles, 4 waves of 128 x 128, K in stages of 32.
//  * One workgroup per CU (160 KB of LDS: four 32 KB operand stages and a 32 KB epilogue buffer) walks
//    a contiguous range of its XCD's tiles in grouped order (GROUP_M tile rows at a time), so the
//    tiles that run together on one XCD share X rows and W rows in its L2.
//  * Operands go global -> LDS with gfx950's direct loads (global_load_lds_dwordx4: lane l of one
//    instruction fills bytes 16 l .. 16 l + 15 of a 1 KB LDS block), three to four stages ahead of
//    use.  The 8 direct loads of a stage sit between the MFMAs, one per 4, and the barrier waits only
//    for the stage about to be read, never for the whole queue.
//  * Each 64-byte LDS row (32 bf16 of K) holds its four 16-byte chunks XOR-swizzled by swz(row) so
//    fragment reads are free of bank conflicts; the swizzle is applied by choosing which global chunk
//    each lane fetches.
//  * The next tile's first stages are requested before the epilogue so their latency hides behind
//    it; bf16 epilogues pass through LDS and leave as whole 256-byte row segments.
// ---------------------------------------------------------------------------------------------------
constexpr int BIG = 256;
constexpr int GROUP_M = 2;
constexpr int BK4 = 32;                          // K per stage
constexpr int NSTAGE = 4;
constexpr int OPND_BYTES = BIG * BK4 * 2;        // one operand tile, 16 KB
constexpr int STAGE_BYTES = 2 * OPND_BYTES;      // X tile then W tile
constexpr int EPI_SLICE = 32 * 128 * 2;          // per-wave epilogue buffer: 32 rows x 128 bf16
constexpr int SLOTS_PER_XCD = 32;                // CUs per XCD: one persistent workgroup each

__device__ __forceinline__ int row_swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// Tile tt of the grouped order: GROUP_M tile rows at a time, column by column within a group.
__device__ __forceinline__ void tile_coords(const GemmArgs& a, int tt, int& tm, int& tn) {
  const int width = GROUP_M * a.tiles_n;
  const int first_m = (tt / width) * GROUP_M;
  const int gsz = min(a.tiles_m - first_m, GROUP_M);
  tm = first_m + (tt % width) % gsz;
  tn = (tt % width) / gsz;
}

// Stream-K chunk of a wave's 128 x 128 block: the raw fp32 sums into the partial tile [256][256]
// (element (m, n) of the tile at m * 256 + n).
__device__ __forceinline__ void store_partial(float* part, const f32x16 (&acc)[4][4], int wm0, int wn0, int l32, int g) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
        *(f32x4*)(part + (wm0 + 32 * j + l32) * BIG + wn0 + 32 * i + 8 * rg + 4 * g) =
            (f32x4){acc[i][j][4 * rg], acc[i][j][4 * rg + 1], acc[i][j][4 * rg + 2], acc[i][j][4 * rg + 3]};
}

// bf16 epilogue of one wave's 128 x 128 block (bias already in the accumulators) through its LDS slice,
// 32 rows at a time.  Writes: lane (l32, g) puts its 4 values of chunk c (= 8 output columns) of row l32
// into 16-byte position c ^ (l32 & 15), 8-byte half g ^ (l32 >> 4) (conflict-free); reads: 16 lanes per
// row take the row's 16 chunks, so each store instruction writes 4 whole 256-byte row segments.  Blocks
// wholly inside the output store without per-row checks, from a scalar row base and one 32-bit lane offset.
template <int EPI>
__device__ __forceinline__ void store_tile_lds(const GemmArgs& a, const f32x16 (&acc)[4][4], int64_t mb, int64_t nb,
                                               char* slice, int lane, int l32, int g) {
  const bool full = mb + 128 <= a.M && nb + 128 <= a.N;
  const int wrow = l32 * 256 + 8 * (g ^ (l32 >> 4));
  const int c16 = lane & 15, r4 = lane >> 4;
  const uint32_t loff = (uint32_t)((r4 * a.ldo + 8 * c16) * 2);
  char* const obase = (char*)a.out + (mb * a.ldo + nb) * 2;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        f32x4 v = {acc[i][j][4 * rg], acc[i][j][4 * rg + 1], acc[i][j][4 * rg + 2], acc[i][j][4 * rg + 3]};
        if constexpr (EPI == EPI_GELU_BF16) {
          v.x = gelu_tanh_f(v.x); v.y = gelu_tanh_f(v.y); v.z = gelu_tanh_f(v.z); v.w = gelu_tanh_f(v.w);
        }
        u32x2 o;
        o.x = pack_bf16x2(v.x, v.y);
        o.y = pack_bf16x2(v.z, v.w);
        const int c = 4 * i + rg;
        *(u32x2*)(slice + wrow + ((c ^ (l32 & 15)) << 4)) = o;
      }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the slice is written before any lane reads it
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int row = 4 * s + r4;
      u32x4 d = *(const u32x4*)(slice + row * 256 + ((c16 ^ (row & 15)) << 4));
      if (s >= 4) d = (u32x4){d.z, d.w, d.x, d.y};   // rows 16..31 hold their halves swapped
      char* const rowbase = obase + (int64_t)(32 * j + 4 * s) * a.ldo * 2;
      if (full) {
        *(u32x4*)(rowbase + loff) = d;
      } else {
        const int64_t m = mb + 32 * j + row, n = nb + 8 * c16;
        if (m < a.M && n < a.N) *(u32x4*)(rowbase + loff) = d;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): reads done before the next slab overwrites
    __builtin_amdgcn_wave_barrier();
  }
}

// SK: the stream-K launch.  Workgroup w takes K stages [kb, kb + nk) of chunk w % sk_split of tail tile
// dp_tiles + w / sk_split and writes the raw sums (no bias) to its partial tile.
template <int EPI, bool SK>
__global__ __launch_bounds__(256, 1) void k_gemm_big(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[NSTAGE * STAGE_BYTES + 4 * EPI_SLICE];
  // the wave index is uniform: read it into a scalar register so every LDS address of the direct
  // loads (written to M0) is scalar arithmetic, with no per-load readfirstlane
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int wm0 = (wave >> 1) * 128, wn0 = (wave & 1) * 128;

  // ---- this workgroup's tiles: XCD blockIdx % 8 owns tiles [lo, hi) of the first dp_tiles of the
  //      grouped order; its SLOTS_PER_XCD workgroups take every SLOTS_PER_XCD-th one
  const int per = (a.dp_tiles + 7) / 8;
  const int lo = (blockIdx.x % 8) * per;
  const int hi = min(a.dp_tiles, lo + per);
  int t = lo + (int)(blockIdx.x / 8);
  int kb = 0, nk = (int)(a.K / BK4);   // >= 4 (checked by the launcher)
  if constexpr (SK) {
    const int c = (int)blockIdx.x % a.sk_split;
    t = a.dp_tiles + (int)blockIdx.x / a.sk_split;
    kb = (int)((int64_t)c * nk / a.sk_split);
    nk = (int)((int64_t)(c + 1) * nk / a.sk_split) - kb;   // >= 4 (the launcher's split)
  } else {
    if (t >= hi) return;
  }

  int64_t m0, n0;
  uint32_t xo[4], wo[4];
  const char* xt;
  const char* wt;
  // tile t: origin, and per-lane direct-load offsets.  Instruction I = 4 wave + i covers tile rows
  // 16 I .. 16 I + 15: lane -> row 16 I + lane / 4, LDS chunk lane % 4, global chunk (lane % 4) ^ swz(row).
  // Rows past M or N repeat the last row (their results are never stored).
  // kb: first K stage (stream-K chunks)
  auto setup = [&](int tt, int kb) {
    int tm, tn;
    tile_coords(a, tt, tm, tn);
    m0 = (int64_t)tm * BIG;
    n0 = (int64_t)tn * BIG;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * (4 * wave + i) + (lane >> 2);
      const int cchunk = (lane & 3) ^ row_swz(r);
      int64_t rx = m0 + r, rw = n0 + r;
      if (rx > a.M - 1) rx = a.M - 1;
      if (rw > a.N - 1) rw = a.N - 1;
      xo[i] = (uint32_t)(((rx - m0) * a.ldx + cchunk * 8) * 2);
      wo[i] = (uint32_t)(((rw - n0) * a.ldw + cchunk * 8) * 2);
    }
    xt = (const char*)(a.x + m0 * a.ldx + (int64_t)kb * BK4);
    wt = (const char*)(a.w + n0 * a.ldw + (int64_t)kb * BK4);
  };
  // instruction i of half h of stage kt: h = 0 the X tile, h = 1 the W tile
  auto dma = [&](int kt, int h, int i) {
    char* dst = lds + (kt % NSTAGE) * STAGE_BYTES + h * OPND_BYTES + (4 * wave + i) * 1024;
    // scalar base + 32-bit lane offset: the load takes its address in saddr + voffset form
    const char* base = (h ? wt : xt) + kt * BK4 * 2;
    __builtin_amdgcn_global_load_lds((const void*)(base + (h ? wo[i] : xo[i])), (lds_void*)dst, 16, 0, 0);
  };
  // stages 0..2 whole and the first half of stage 3 (28 instructions)
  auto prologue = [&]() {
#pragma unroll
    for (int st = 0; st < 3; ++st)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) dma(st, h, i);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma(3, 0, i);
  };

  int foff[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) foff[ks] = l32 * 64 + (((2 * ks + g) ^ row_swz(l32)) << 4);

  f32x16 acc[4][4];
  u32x4 fa[2][4], fb[2][4];
  // bf16 epilogues: the accumulators start from the bias, written by one MFMA each at tile start:
  // A holds column n's bias split into bf16 hi + lo at k = 0, 1 (lane l32 of block i is column
  // wn0 + 32 i + l32), B holds 1 at k = 0, 1, so D[n][m] = hi + lo = bias[n] to ~2^-18 relative.
  // (stream-K chunks start from zero: k_gemm_sk_fix adds the bias once)
  constexpr bool FOLD = !SK && (EPI == EPI_BF16 || EPI == EPI_GELU_BF16);
  float bcol[4];
  auto bias_cols = [&](int64_t nb, int i) {   // bias of column nb + 32 i + l32 (clamped past N)
    const int64_t n = nb + 32 * i + l32;
    return a.bias[n < a.N ? n : a.N - 1];
  };
  // fragment q (0..7) of k-substep ks of stage kt: q < 4 -> W rows wn0 + 32 q, else X rows
  auto frag = [&](int kt, int ks, int q) {
    const char* base = lds + (kt % NSTAGE) * STAGE_BYTES;
    if (q < 4) fa[ks][q] = *(const u32x4*)(base + OPND_BYTES + (wn0 + q * 32) * 64 + foff[ks]);
    else fb[ks][q - 4] = *(const u32x4*)(base + (wm0 + (q - 4) * 32) * 64 + foff[ks]);
  };
  auto mma = [&](int ks, int q) {     // MFMAs 2q, 2q+1 of k-substep ks
    const int i = q >> 1, j0 = 2 * (q & 1);
    acc[i][j0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fa[ks][i]), as_bf16x8(fb[ks][j0]), acc[i][j0], 0, 0, 0);
    acc[i][j0 + 1] =
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fa[ks][i]), as_bf16x8(fb[ks][j0 + 1]), acc[i][j0 + 1], 0, 0, 0);
  };
  // One K step kt in two phases of 16 MFMAs, every 2 MFMAs followed by one fragment read and every 4 by
  // one direct load (sched_barrier keeps this order):
  //   A: MFMAs of substep 0 | fragments of substep 1 | second half of stage kt+3
  //   own part of stage kt+1 landed, every fragment read of stage kt returned, workgroup barrier
  //   B: MFMAs of substep 1 | substep-0 fragments of stage kt+1 | first half of stage kt+4, which goes
  //      into stage kt's buffer (free once every wave has passed the barrier)
  // WAIT = stages allowed in flight at the barrier (8 instructions each).
  //   BIAS (third-last step): the 4 bias loads of the next tile go out in phase A, after every direct
  //   load of this tile, so the barrier allows them in flight too (WAIT = 3: vmcnt(12)).
  int64_t bias_nb = 0;   // first column of this wave's block in the next tile
  auto step = [&](int kt, auto issue_a, auto issue_b, auto wait_n, auto next, auto bias_next) {
    constexpr bool IA = decltype(issue_a)::value, IB = decltype(issue_b)::value;
    constexpr bool NEXT = decltype(next)::value, BIAS = decltype(bias_next)::value;
    constexpr int WAIT = decltype(wait_n)::value;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      mma(0, q);
      frag(kt, 1, q);
      if (IA && (q & 1)) dma(kt + 3, 1, q >> 1);
      if (BIAS && q < 4) bcol[q] = bias_cols(bias_nb, q);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (NEXT) {
      if constexpr (WAIT == 3) __builtin_amdgcn_s_waitcnt(0x007C);        // vmcnt(12) lgkmcnt(0)
      else if constexpr (WAIT == 2) __builtin_amdgcn_s_waitcnt(0x4070);   // vmcnt(16) lgkmcnt(0)
      else if constexpr (WAIT == 1) __builtin_amdgcn_s_waitcnt(0x0078);   // vmcnt(8) lgkmcnt(0)
      else __builtin_amdgcn_s_waitcnt(0x0070);                            // vmcnt(0) lgkmcnt(0)
      block_sync();
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      mma(1, q);
      if (NEXT) frag(kt + 1, 0, q);
      if (IB && (q & 1)) dma(kt + 4, 0, q >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using T = std::true_type;
  using F = std::false_type;
  using W3 = std::integral_constant<int, 3>;
  using W2 = std::integral_constant<int, 2>;
  using W1 = std::integral_constant<int, 1>;
  using W0 = std::integral_constant<int, 0>;
  char* slice = lds + NSTAGE * STAGE_BYTES + wave * EPI_SLICE;

  setup(t, kb);
  if constexpr (FOLD) {
#pragma unroll
    for (int i = 0; i < 4; ++i) bcol[i] = bias_cols(n0 + wn0, i);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0), once per workgroup, before any direct load
  }
  prologue();
  while (true) {
    if constexpr (FOLD) {
      const u32x4 ones = {g ? 0u : 0x3F803F80u, 0u, 0u, 0u};   // bf16 1.0 at k = 0, 1
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float hi = lo_bf16(pack_bf16x2(bcol[i], 0.f));           // bias rounded to bf16
        const u32x4 bf = {g ? 0u : pack_bf16x2(bcol[i], bcol[i] - hi), 0u, 0u, 0u};   // hi, then the rest
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(bf), as_bf16x8(ones), (f32x16){}, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16){};
    }
    // stage 0 landed.  Outstanding: this tile's 28 direct loads, and possibly the previous tile's
    // epilogue stores (or loads issued after the 28).  Loads complete in order, so once at most 20
    // operations remain, the first 8 loads (stage 0) are done whatever the stores did.
    __builtin_amdgcn_s_waitcnt(0x4F74);   // vmcnt(20)
    block_sync();
#pragma unroll
    for (int q = 0; q < 8; ++q) frag(0, 0, q);
    const int tnext = t + SLOTS_PER_XCD;
    const bool more = !SK && tnext < hi;
    if constexpr (FOLD) {
      // the next tile's columns (after the last tile: this tile's again, loaded and never used)
      int tm, tn;
      tile_coords(a, more ? tnext : t, tm, tn);
      bias_nb = (int64_t)tn * BIG + wn0;
    }
    int kt = 0;
    for (; kt + 4 < nk; ++kt) step(kt, T{}, T{}, W2{}, T{}, F{});
    step(kt, T{}, F{}, W2{}, T{}, F{});
    if constexpr (FOLD) step(kt + 1, F{}, F{}, W3{}, T{}, T{});
    else step(kt + 1, F{}, F{}, W1{}, T{}, F{});
    step(kt + 2, F{}, F{}, W0{}, T{}, F{});
    step(kt + 3, F{}, F{}, W0{}, F{}, F{});
    const int64_t tm0 = m0, tn0 = n0;
    // every wave has read its last fragments before any wave refills the stages
    block_sync();
    if (more) {
      setup(tnext, 0);
      prologue();
    }
    if constexpr (SK)
      store_partial(a.sk_part + (int64_t)blockIdx.x * BIG * BIG, acc, wm0, wn0, l32, g);
    else if constexpr (EPI == EPI_BF16 || EPI == EPI_GELU_BF16)
      store_tile_lds<EPI>(a, acc, tm0 + wm0, tn0 + wn0, slice, lane, l32, g);
    else
      store_tile<EPI, 4, 4>(a, acc, tm0 + wm0, tn0 + wn0, l32, g);
    if (!more) break;
    t = tnext;
  }
}

// Stream-K fix-up: per tail tile, the sum of its sk_split fp32 partial tiles (in chunk order), plus the
// bias, through the epilogue.  64 workgroups per tile, each 4 rows x 256 columns, 4 columns per thread.
template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_sk_fix(GemmArgs a) {
  const int tl = (int)blockIdx.x / 64;
  int tm, tn;
  tile_coords(a, a.dp_tiles + tl, tm, tn);
  const int r = 4 * ((int)blockIdx.x % 64) + (int)(threadIdx.x >> 6), c = 4 * (int)(threadIdx.x & 63);
  const int64_t m = (int64_t)tm * BIG + r, n = (int64_t)tn * BIG + c;
  if (m >= a.M || n >= a.N) return;   // N is a multiple of 8: a thread's 4 columns are all in or all out
  const float* p = a.sk_part + (int64_t)tl * a.sk_split * BIG * BIG + r * BIG + c;
  f32x4 v = *(const f32x4*)(a.bias + n);
  for (int k = 0; k < a.sk_split; ++k) v += *(const f32x4*)(p + (int64_t)k * BIG * BIG);
  if constexpr (EPI == EPI_BF16 || EPI == EPI_GELU_BF16) {
    if constexpr (EPI == EPI_GELU_BF16) {
      v.x = gelu_tanh_f(v.x); v.y = gelu_tanh_f(v.y); v.z = gelu_tanh_f(v.z); v.w = gelu_tanh_f(v.w);
    }
    *(u32x2*)((bf16_t*)a.out + m * a.ldo + n) = (u32x2){pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
  } else {
    float* o = (float*)a.out + m * a.ldo + n;
    if constexpr (EPI == EPI_F32) {
      *(f32x4*)o = v;
    } else if constexpr (EPI == EPI_RES_F32) {
      *(f32x4*)o = *(const f32x4*)o + v;
    } else {
      const f32x4 gate = *(const f32x4*)(a.gate_tab + n) + *(const f32x4*)(a.gate_src + (m / a.rows_per_gate) * a.gate_ld + n);
      *(f32x4*)o = *(const f32x4*)o + v * gate;
    }
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_tile(int epi, GemmArgs& a, hipStream_t s) {
  a.tiles_m = (int)ceil_div(a.M, BM);
  a.tiles_n = (int)ceil_div(a.N, BN);
  dim3 grid(a.tiles_m * a.tiles_n), block(256);
  switch (epi) {
    case EPI_BF16: hipLaunchKernelGGL((k_gemm_bf16<BM, BN, WM, WN, EPI_BF16>), grid, block, 0, s, a); break;
    case EPI_GELU_BF16: hipLaunchKernelGGL((k_gemm_bf16<BM, BN, WM, WN, EPI_GELU_BF16>), grid, block, 0, s, a); break;
    case EPI_F32: hipLaunchKernelGGL((k_gemm_bf16<BM, BN, WM, WN, EPI_F32>), grid, block, 0, s, a); break;
    case EPI_RES_F32: hipLaunchKernelGGL((k_gemm_bf16<BM, BN, WM, WN, EPI_RES_F32>), grid, block, 0, s, a); break;
    case EPI_GATE_F32: hipLaunchKernelGGL((k_gemm_bf16<BM, BN, WM, WN, EPI_GATE_F32>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The persistent kernel runs one workgroup per CU slot (8 XCDs x 32), so a launch takes
// ceil(tiles / 256) rounds of whole tiles.  With a workspace and a last round at most half full, the
// tiles of that round are split along K instead (as many chunks as fill the slots, at least 4 stages
// each) and a fix-up pass sums them: the launch then costs its full rounds plus a fraction of one.
hipError_t launch_big(int epi, GemmArgs& a, float* ws, int64_t ws_bytes, hipStream_t s) {
  a.tiles_m = (int)ceil_div(a.M, BIG);
  a.tiles_n = (int)ceil_div(a.N, BIG);
  const int slots = 8 * SLOTS_PER_XCD;
  const int ntiles = a.tiles_m * a.tiles_n;
  const int tail = ntiles % slots;
  const int nk = (int)(a.K / BK4);
  int split = 0;
  if (ws != nullptr && tail > 0 && 2 * tail <= slots) {
    split = min(slots / tail, nk / 4);
    if (split < 2 || (int64_t)tail * split * BIG * BIG * 4 > ws_bytes) split = 0;
  }
  a.dp_tiles = split ? ntiles - tail : ntiles;
  a.sk_tiles = split ? tail : 0;
  a.sk_split = split ? split : 1;
  a.sk_part = split ? ws : nullptr;
  dim3 grid(slots), block(256);
  auto run = [&](auto epi_tag) {
    constexpr int E = decltype(epi_tag)::value;
    hipLaunchKernelGGL((k_gemm_big<E, false>), grid, block, 0, s, a);
    if (split) {
      hipLaunchKernelGGL((k_gemm_big<E, true>), dim3((unsigned)(tail * split)), block, 0, s, a);
      hipLaunchKernelGGL(k_gemm_sk_fix<E>, dim3((unsigned)(tail * 64)), block, 0, s, a);
    }
  };
  switch (epi) {
    case EPI_BF16: run(std::integral_constant<int, EPI_BF16>{}); break;
    case EPI_GELU_BF16: run(std::integral_constant<int, EPI_GELU_BF16>{}); break;
    case EPI_F32: run(std::integral_constant<int, EPI_F32>{}); break;
    case EPI_RES_F32: run(std::integral_constant<int, EPI_RES_F32>{}); break;
    case EPI_GATE_F32: run(std::integral_constant<int, EPI_GATE_F32>{}); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------------
// fp32 GEMM (timestep MLP, kept in fp32): C[m,n] = act_in(A)[m,:] . W[n,:] + bias[n], optional SiLU
// on the input elements and/or the output.  64x64 tile, 256 threads, 4x4 outputs per thread.
// ---------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gemm_f32(const float* __restrict__ A, int64_t lda, const float* __restrict__ W,
                                                  int64_t ldw, const float* __restrict__ bias, int64_t M, int64_t N,
                                                  int64_t K, float* __restrict__ C, int64_t ldc, int silu_in, int silu_out) {
  constexpr int T = 64, KB = 16;
  __shared__ float As[KB][T + 4];
  __shared__ float Ws[KB][T + 4];
  const int tid = threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.y * T, n0 = (int64_t)blockIdx.x * T;
  const int tr = tid / 16, tc = tid % 16;
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < K; k0 += KB) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = tid + 256 * i;
      int r = e / KB, kk = e % KB;
      int64_t gm = m0 + r, gn = n0 + r, gk = k0 + kk;
      float av = (gm < M && gk < K) ? A[gm * lda + gk] : 0.f;
      if (silu_in) av = silu_f(av);
      As[kk][r] = av;
      Ws[kk][r] = (gn < N && gk < K) ? W[gn * ldw + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) {
      float av[4], wv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { av[i] = As[kk][tr * 4 + i]; wv[i] = Ws[kk][tc * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], wv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int64_t m = m0 + tr * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int64_t n = n0 + tc * 4 + j;
      if (n >= N) continue;
      float v = acc[i][j] + bias[n];
      if (silu_out) v = silu_f(v);
      C[m * ldc + n] = v;
    }
  }
}

// fp32 GEMM on the fp32 matrix cores (v_mfma_f32_32x32x2_f32: fp32 products, fp32 accumulation), used
// for the timestep MLP when K is a multiple of 16.  128x128 workgroup tile, 4 waves of 64x64 (2x2 MFMA
// tiles), K in steps of 16 staged through registers into LDS rows padded to 17 floats (a column read by
// 32 consecutive rows then touches 32 distinct banks), double buffered.  SiLU of the input is applied on
// the way into LDS, bias and SiLU of the output in the epilogue.  Rows and columns past M and N load as
// zero and are not stored.
constexpr int F_TILE = 128, F_BK = 16, F_LD = F_BK + 1;

__global__ __launch_bounds__(256, 2) void k_gemm_f32m(const float* __restrict__ A, int64_t lda,
                                                      const float* __restrict__ W, int64_t ldw,
                                                      const float* __restrict__ bias, int64_t M, int64_t N, int64_t K,
                                                      float* __restrict__ C, int64_t ldc, int silu_in, int silu_out,
                                                      int tiles_n) {
  __shared__ float la[2][F_TILE * F_LD];
  __shared__ float lw[2][F_TILE * F_LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, g = lane >> 5;
  const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * F_TILE, n0 = (int64_t)(blockIdx.x % tiles_n) * F_TILE;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  // staging: thread -> row tid / 2 of each tile, 8 consecutive k at (tid % 2) * 8
  const int sr = tid >> 1, sk = (tid & 1) * 8;
  const bool a_ok = m0 + sr < M, w_ok = n0 + sr < N;
  const float* ap = A + (a_ok ? m0 + sr : 0) * lda + sk;
  const float* wp = W + (w_ok ? n0 + sr : 0) * ldw + sk;
  f32x4 ra[2], rw[2];
  auto load = [&](int64_t k0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ra[h] = a_ok ? *(const f32x4*)(ap + k0 + 4 * h) : (f32x4){};
      rw[h] = w_ok ? *(const f32x4*)(wp + k0 + 4 * h) : (f32x4){};
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float av = ra[h][e];
        la[buf][sr * F_LD + sk + 4 * h + e] = silu_in ? silu_f(av) : av;
        lw[buf][sr * F_LD + sk + 4 * h + e] = rw[h][e];
      }
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f32x16){};
  const int nk = (int)(K / F_BK);
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load((int64_t)(kt + 1) * F_BK);
#pragma unroll
    for (int kk = 0; kk < F_BK / 2; ++kk) {
      // A operand: output row (wm + 32 i + l32), k = 2 kk + g;  B operand: output column (wn + 32 j + l32)
      float fa[2], fw[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[i] = la[buf][(wm + 32 * i + l32) * F_LD + 2 * kk + g];
#pragma unroll
      for (int j = 0; j < 2; ++j) fw[j] = lw[buf][(wn + 32 * j + l32) * F_LD + 2 * kk + g];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i], fw[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }
  // acc[i][j] element r: row wm + 32 i + 8 (r/4) + 4 g + r%4, column wn + 32 j + l32
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = n0 + wn + 32 * j + l32;
    if (n >= N) continue;
    const float bn = bias[n];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
        if (m >= M) continue;
        const float v = acc[i][j][r] + bn;
        C[m * ldc + n] = silu_out ? silu_f(v) : v;
      }
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const bf16_t* x, int64_t ldx, const bf16_t* w, int64_t ldw, const float* bias, int64_t M,
                            int64_t N, int64_t K, int epi, void* out, int64_t ldo, const float* gate_tab,
                            const float* gate_src, int64_t gate_ld, int64_t rows_per_gate, hipStream_t s, float* ws,
                            int64_t ws_bytes) {
  if (M <= 0 || N <= 0) return hipSuccess;
  GemmArgs a;
  a.x = x; a.ldx = ldx; a.w = w; a.ldw = ldw; a.bias = bias;
  a.M = M; a.N = N; a.K = K; a.out = out; a.ldo = ldo;
  a.gate_tab = gate_tab; a.gate_src = gate_src; a.gate_ld = gate_ld;
  a.rows_per_gate = rows_per_gate > 0 ? rows_per_gate : 1;
  // Large problems: 256x256 tiles with direct LDS loads.  Small ones: 128x128 so the grid still covers
  // the chip.  The direct-load offsets are 32-bit: 256 rows of the larger leading dimension must fit.
  // The persistent kernel also needs 4+ K stages of 32 and, for its 16-byte bf16 stores, N, ldo and
  // the output address aligned to 8 elements.
  const int64_t big_tiles = ceil_div(M, 256) * ceil_div(N, 256);
  const bool offsets_fit = 256 * (ldx > ldw ? ldx : ldw) * 2 < (1LL << 31);
  const bool aligned = N % 8 == 0 && ldo % 8 == 0 && ((uintptr_t)out & 15) == 0;
  if (big_tiles >= 512 && offsets_fit && K % 32 == 0 && K >= 128 && aligned) return launch_big(epi, a, ws, ws_bytes, s);
  return launch_tile<128, 128, 64, 64>(epi, a, s);
}

int64_t gemm_workspace_bytes() { return (int64_t)8 * SLOTS_PER_XCD * BIG * BIG * 4; }

hipError_t launch_gemm_f32(const float* A, int64_t lda, const float* W, int64_t ldw, const float* bias, int64_t M,
                           int64_t N, int64_t K, float* C, int64_t ldc, int silu_in, int silu_out, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K % F_BK == 0 && lda % 4 == 0 && ldw % 4 == 0 && ((uintptr_t)A & 15) == 0 && ((uintptr_t)W & 15) == 0) {
    const int tiles_n = (int)ceil_div(N, F_TILE);
    const int64_t blocks = ceil_div(M, F_TILE) * tiles_n;
    hipLaunchKernelGGL(k_gemm_f32m, dim3((unsigned)blocks), dim3(256), 0, s, A, lda, W, ldw, bias, M, N, K, C, ldc,
                       silu_in, silu_out, tiles_n);
    return hipGetLastError();
  }
  dim3 grid((unsigned)ceil_div(N, 64), (unsigned)ceil_div(M, 64));
  hipLaunchKernelGGL(k_gemm_f32, grid, dim3(256), 0, s, A, lda, W, ldw, bias, M, N, K, C, ldc, silu_in, silu_out);
  return hipGetLastError();
}
