// bf16 MFMA GEMM for gfx950 with fused epilogues, plus a small fp32 GEMM for the timestep MLP.
//
//   C[m, n] = sum_k X[m, k] * W[n, k]  (+ bias[n], then an epilogue)
//
// X is the activation (row-major, K contiguous), W an nn.Linear weight [N, K] (K contiguous), so both
// operands are read 16 bytes per lane straight into MFMA fragments.  The MFMA "A" operand is a W tile
// and the "B" operand an X tile, i.e. every 32x32 accumulator holds C^T: each lane then owns four
// consecutive output columns of one row, which makes the epilogue's stores and the fp32 residual
// read-modify-write 16-byte vector accesses.
//
// Epilogues (diffusers WanTransformerBlock.forward as printed on the WanPipeline notes page):
//   EPI_BF16       out_bf16 = acc + bias                                  (QKV, cross Q/KV, text proj)
//   EPI_GELU_BF16  out_bf16 = gelu_tanh(acc + bias)                       (FFN first Linear, text proj)
//   EPI_F32        out_f32  = acc + bias                                  (patch embed, proj_out)
//   EPI_RES_F32    out_f32 += acc + bias                                  (ungated cross-attn residual)
//   EPI_GATE_F32   out_f32 += (acc + bias) * (gate_tab[n] + gate_src[row(m)][n])   (gate_msa, c_gate_msa)
#include "common.h"
#include "launch.h"

namespace {

constexpr int BK = 64;
constexpr int LDS_LD = BK + 8;  // bf16 per LDS row: 144 B rows keep ds_read_b128 conflict-free

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
};

// Dispatch order places consecutive workgroups on different XCDs (round robin over 8).  Renumber so
// that each XCD receives a contiguous range of logical tiles: tiles that share X rows then share
// that XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int per = nb / 8, rem = nb % 8;
  const int xcd = b % 8, slot = b / 8;
  return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

template <int EPI>
__device__ __forceinline__ void epilogue4(const GemmArgs& a, int64_t m, int64_t n, f32x4 v) {
  // v holds columns n..n+3 of row m; caller guarantees m < M and n + 3 < N.
  f32x4 b = *(const f32x4*)(a.bias + n);
  v += b;
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
    f32x4* p = (f32x4*)((float*)a.out + m * a.ldo + n);
    *p = *p + v;
  } else {  // EPI_GATE_F32
    const int64_t gr = m / a.rows_per_gate;
    f32x4 g = *(const f32x4*)(a.gate_tab + n) + *(const f32x4*)(a.gate_src + gr * a.gate_ld + n);
    f32x4* p = (f32x4*)((float*)a.out + m * a.ldo + n);
    *p = *p + v * g;
  }
}

// BM x BN workgroup tile, 4 waves arranged (BM/WM) x (BN/WN), each wave a WM x WN tile built from
// 32x32x16 bf16 MFMAs.  K must be a multiple of 64; M and N tails are clamped on load, guarded on store.
template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(256, (BM >= 256 ? 1 : 2)) void k_gemm_bf16(GemmArgs a) {
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

  // global load addressing: chunk c = tid + 256*i covers row c/8, 8 bf16 at column (c%8)*8
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

  // acc[i][j] element r: n = n0 + wn0 + 32i + 8(r/4) + 4g + r%4, m = m0 + wm0 + 32j + l32
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int64_t m = m0 + wm0 + 32 * j + l32;
    if (m >= a.M) continue;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int64_t n = n0 + wn0 + 32 * i + 8 * rg + 4 * g;
        if (n >= a.N) continue;
        f32x4 v = {acc[i][j][4 * rg], acc[i][j][4 * rg + 1], acc[i][j][4 * rg + 2], acc[i][j][4 * rg + 3]};
        epilogue4<EPI>(a, m, n, v);
      }
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
    // 64 rows x 16 k per operand = 1024 elements, 4 per thread
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

}  // namespace

hipError_t launch_gemm_bf16(const bf16_t* x, int64_t ldx, const bf16_t* w, int64_t ldw, const float* bias, int64_t M,
                            int64_t N, int64_t K, int epi, void* out, int64_t ldo, const float* gate_tab,
                            const float* gate_src, int64_t gate_ld, int64_t rows_per_gate, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  GemmArgs a;
  a.x = x; a.ldx = ldx; a.w = w; a.ldw = ldw; a.bias = bias;
  a.M = M; a.N = N; a.K = K; a.out = out; a.ldo = ldo;
  a.gate_tab = gate_tab; a.gate_src = gate_src; a.gate_ld = gate_ld;
  a.rows_per_gate = rows_per_gate > 0 ? rows_per_gate : 1;
  // Large problems: 256x256 tiles (each wave 128x128, 16 MFMA tiles in flight per LDS fragment set).
  // Small ones: 128x128 so the grid still covers the chip.
  const int64_t big_tiles = ceil_div(M, 256) * ceil_div(N, 256);
  if (big_tiles >= 512) return launch_tile<256, 256, 128, 128>(epi, a, s);
  return launch_tile<128, 128, 64, 64>(epi, a, s);
}

hipError_t launch_gemm_f32(const float* A, int64_t lda, const float* W, int64_t ldw, const float* bias, int64_t M,
                           int64_t N, int64_t K, float* C, int64_t ldc, int silu_in, int silu_out, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  dim3 grid((unsigned)ceil_div(N, 64), (unsigned)ceil_div(M, 64));
  hipLaunchKernelGGL(k_gemm_f32, grid, dim3(256), 0, s, A, lda, W, ldw, bias, M, N, K, C, ldc, silu_in, silu_out);
  return hipGetLastError();
}
