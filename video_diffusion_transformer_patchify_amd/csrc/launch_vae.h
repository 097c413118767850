// Internal launch functions of the Wan-VAE decoder kernels (not part of the C ABI).
//
// Frame layout ("padded frame"): one frame of C channels (C a multiple of 16) at H x W pixels is bf16
// [C / 16][H + 2][W + 2][16]: 16-channel blocks, each a row-major image with a one-pixel zero border.
// Kernels write only the interior, so the border stays zero once the buffer has been cleared.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;

constexpr int VAE_MAXF = 16;          // output frames per convolution / norm launch

inline int64_t vae_frame_elems(int64_t C, int64_t H, int64_t W) { return C * (H + 2) * (W + 2); }

struct VaeConvArgs {
  const bf16_t* in[VAE_MAXF][3];   // per output frame j, per time tap dt: padded input frame
  bf16_t* out[2 * VAE_MAXF];       // padded output frames, out[j * split + s]
  const bf16_t* res[2 * VAE_MAXF]; // residual frames added before rounding (may equal out), or null
  const bf16_t* w;                 // packed weights (vae_pack_conv)
  const float* bias;               // [ntiles * 32 * ncf], zero beyond c_out
  void* video;                     // video output (EPI video): [3, T, H, W] of one sample
  int32_t video_t[VAE_MAXF];       // video frame index of output frame j
  int32_t nf;                      // output frames
  int32_t H, W;                    // output frame size
  int32_t Hin, Win;                // input frame size (H / 2, W / 2 for the upsampling conv)
  int32_t cin_blocks;              // input channels / 16
  int32_t cpart;                   // channels of one output frame (split parts: c_out / split)
  int32_t split;                   // 1, or 2: channel part s of frame j goes to out[2 j + s]
  int32_t ntiles;                  // output-channel tiles of 32 * ncf
  int32_t tiles_x, tiles_y;
  int32_t video_T;                 // frames of the video output
  int32_t video_bf16;              // video dtype: 1 bf16, 0 fp32
  // fused RMS norm + SiLU of the (bf16-rounded) output over its 32 * ncf channels, for a launch with one
  // output-channel tile and no split: nout[j] = SiLU(ngamma * u / sqrt(mean(u^2) + neps)).  Null: none.
  bf16_t* nout[VAE_MAXF];
  const float* ngamma;             // [32 * ncf]
  float neps;
  int32_t nonly;                   // 1: only nout is written (out is not)
};

// kt: 1 or 3 time taps; ks: 1 or 3 (square) spatial taps; up: input is the half-size frame, read through
// a nearest x2 upsample (ks 3, kt 1); video: clamp to [-1, 1] and write channels 0..2 into a.video.
hipError_t launch_vae_conv(const VaeConvArgs& a, int kt, int ks, int up, int ncf, bool video, hipStream_t s);

// Packed weight elements of a conv [c_out, c_in, kt, ks, ks]: [ntiles][kt][c_in/16][ks*ks][32*ncf][16].
int64_t vae_packed_conv_elems(int64_t cout, int64_t cin, int kt, int ks, int ncf);
// src: fp32 or bf16 [c_out, c_in, kt, ks, ks] (dtype 0 / 1); c_in is padded to a multiple of 16.
hipError_t launch_vae_pack_conv(const void* src, int dtype, int64_t cout, int64_t cin, int kt, int ks, int ncf,
                                bf16_t* dst, hipStream_t s);

// out = SiLU(gamma * u / sqrt(mean_c(u^2) + eps)) per pixel over the first c channels of each frame.
hipError_t launch_vae_rms_silu(const bf16_t* const* in, bf16_t* const* out, int nf, int64_t c, int64_t cblocks,
                               int64_t H, int64_t W, const float* gamma, float eps, hipStream_t s);

// Latent frames [f0, f0 + n) of one sample [16, F, H, W] (fp32 / bf16) -> per channel z * std + mean, then
// the 1x1x1 post-quant conv (wq [16, 16] fp32, bq [16]) -> padded 16-channel frames out[j].
hipError_t launch_vae_prep(const void* z, int dtype, int64_t F, int64_t H, int64_t W, int64_t f0, int n,
                           const float* mean, const float* std, const float* wq, const float* bq, bf16_t* const* out,
                           hipStream_t s);

// Zero n 16-byte words (a fill kernel: safe inside a captured graph).
hipError_t launch_vae_zero(void* p, int64_t bytes, hipStream_t s);
