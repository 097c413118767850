/*
 * wan_vae.h - C ABI of the MI355X (gfx950) Wan-VAE causal video decoder.
 *
 * The decode computed here is the one the diffusers WanPipeline notes page prints in its "vae.decode"
 * section: post_quant_conv over the latent, then WanDecoder3d run on one latent frame at a time with a
 * feature cache of the last 2 input frames per causal convolution (CACHE_T = 2), the outputs
 * concatenated along time and clamped to [-1, 1].  WanDecoder3d: conv_in (16 -> 384), a mid block, four
 * up blocks (the printed ModuleList: three residual blocks each at 384, 384, 192, 96 channels; blocks
 * 0-1 end in an upsample3d, block 2 in an upsample2d), RMS_norm, SiLU, conv_out (96 -> 3).  Every
 * WanCausalConv3d pads time on the past side only.  The Wan2.1 walk-through page, section 3.1, gives the
 * shape relation: a latent [B, 16, F, H, W] decodes to a video [B, 3, 1 + 4 (F - 1), 8 H, 8 W].
 *
 * Where the pages leave a step open the library takes these readings:
 *   - RMS_norm(u) = gamma * u / sqrt(mean over channels of u^2 + eps), per pixel, no bias.
 *   - Residual block: h = conv1(SiLU(norm1(x))); h = conv2(SiLU(norm2(h))); out = h + shortcut(x), the
 *     shortcut being the identity or the printed 1x1x1 conv.
 *   - The mid block is two residual blocks at 384 channels (the 33 causal convolutions leave four for it).
 *   - conv_in / conv_out are 3x3x3 causal convs with spatial padding 1; post_quant_conv is 1x1x1.
 *   - Before post_quant_conv the latent is un-normalised per channel: z * latents_std + latents_mean.
 *   - upsample3d: the (3,1,1) time conv first, its output channel halves [0, C) and [C, 2C) becoming
 *     frames 2t and 2t + 1; the first latent frame skips it and does not enter its history.  Then the
 *     nearest x2 upsample and the 3x3 Conv2d, frame by frame.
 * Results do not depend on how the latent frames after the first are grouped into chunks: each output
 * value is computed by the same kernel arithmetic whatever the chunking.
 *
 * Conventions as in wan_dit.h: device pointers, caller-owned tensors, validation before any launch,
 * status returns, asynchronous launches on the given stream, one decode in flight per handle.
 */
#ifndef WAN_VAE_H
#define WAN_VAE_H

#include <stddef.h>
#include <stdint.h>

#include "wan_dit.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t z_dim;            /* latent channels: must be 16 */
  int32_t base_dim;         /* width of the last up block: 96 in Wan2.1 (stages use 4, 4, 2, 1 x base) */
  int32_t chunk_frames;     /* latent frames decoded per step after the first one, 1..4 (the pages: 1) */
  float eps;                /* RMS_norm epsilon (1e-6) */
  int64_t max_height;       /* latent H_z bound, >= 1 (the video is 8 H_z rows) */
  int64_t max_width;        /* latent W_z bound, >= 1 */
  int64_t reserved[2];
} wan_vae_config;

/* Weight names and shapes (ci / co per block from the layout above; all convs [c_out, c_in, kt, kh, kw]):
 *   latents_mean [16]   latents_std [16]                 post_quant_conv.weight [16, 16, 1, 1, 1]  .bias [16]
 *   decoder.conv_in.weight [4b, 16, 3, 3, 3]  .bias
 *   decoder.mid_block.resnets.{0,1}.* and decoder.up_blocks.{i}.resnets.{0,1,2}.*:
 *       norm1.gamma [ci]  conv1.weight [co, ci, 3, 3, 3] .bias [co]  norm2.gamma [co]
 *       conv2.weight [co, co, 3, 3, 3] .bias [co]   conv_shortcut.weight [co, ci, 1, 1, 1] .bias (ci != co only)
 *   decoder.up_blocks.{0,1}.upsamplers.0.time_conv.weight [8b, 4b, 3, 1, 1]  .bias [8b]
 *   decoder.up_blocks.{0,1,2}.upsamplers.0.resample.1.weight [c/2, c, 3, 3]  .bias [c/2]  (c = 4b, 4b, 2b)
 *   decoder.norm_out.gamma [b]   decoder.conv_out.weight [3, b, 3, 3, 3]  .bias [3]
 * with b = base_dim; block widths (ci -> co): mid 4b -> 4b; up 0: 4b -> 4b; up 1: 2b -> 4b, then 4b;
 * up 2: 2b -> 2b; up 3: b -> b.  Conv weights WAN_F32 or WAN_BF16 (used as bf16), the rest WAN_F32 or
 * WAN_BF16 (used as fp32). */

typedef struct wan_vae wan_vae;

/* Validate cfg and every weight (no missing, extra or duplicate names), pack the conv weights for the
 * convolution kernel (bf16, output-channel tiles of 96 or 32), copy the rest as fp32, and allocate the
 * per-convolution frame caches and stage buffers for max_height x max_width latents and chunk_frames.
 * Synchronises hip_stream before returning.  Errors: WAN_ERR_INVALID_ARG / WAN_ERR_UNSUPPORTED (config),
 * WAN_ERR_MISSING_WEIGHT, WAN_ERR_SHAPE / WAN_ERR_DTYPE (a weight), WAN_ERR_OOM, WAN_ERR_HIP. */
wan_status wan_vae_create(const wan_vae_config* cfg, const wan_weight* weights, size_t n_weights, void* hip_stream,
                          wan_vae** out);

/* Decode latents to videos.
 *   latent [B, 16, F, H_z, W_z] WAN_F32 or WAN_BF16, F >= 1, H_z <= max_height, W_z <= max_width
 *   video  [B, 3, 1 + 4 (F - 1), 8 H_z, 8 W_z] WAN_F32 or WAN_BF16, not aliasing the latent
 * Samples are decoded one after the other, each with fresh caches.  Allocates nothing; enqueues on
 * hip_stream and returns without synchronising.  A latent of another H_z x W_z than the previous call's
 * first clears the handle's frame buffers (a fill kernel on the stream). */
wan_status wan_vae_decode(wan_vae* h, const wan_tensor* latent, wan_tensor* video, void* hip_stream);

void wan_vae_destroy(wan_vae* h);

/* Text of the last wan_vae_* error on the calling thread ("" if none). */
const char* wan_vae_last_error(void);

/* Bytes of device memory the handle holds. */
int64_t wan_vae_device_bytes(const wan_vae* h);

/* Opt-in timing, for benchmarks, of the decode's 3x3x3 causal convolutions with 96-channel output tiles
 * (conv_in and the residual blocks' convolutions; not part of the computation).  max_launches > 0 creates
 * 2 * max_launches HIP events owned by the handle; later such launches of wan_vae_decode are bracketed
 * by an event pair recorded on the decode's stream until the pairs are used up.  0 releases the events
 * (wan_vae_destroy does too).  Errors: WAN_ERR_INVALID_ARG (NULL handle, max_launches outside
 * [0, 2^20], another current device), WAN_ERR_HIP (event creation; no events kept). */
wan_status wan_vae_time_convs(wan_vae* h, int64_t max_launches);

/* Sum in milliseconds of the convolution launches timed since the last call, their number and their
 * algorithmic FLOPs (2 x c_out x c_in x 27 per output pixel).  Host-synchronous; frees the pairs for
 * reuse.  Errors: WAN_ERR_INVALID_ARG (NULL argument, another current device), WAN_ERR_HIP. */
wan_status wan_vae_conv_time(wan_vae* h, double* total_ms, int64_t* launches, double* flops);

/* ---- one stage at a time (the kernels the decode runs), on padded frames ------------------------------
 * A padded frame of C channels (C a multiple of 16) at H x W is bf16 [C/16][H + 2][W + 2][16]: 16-channel
 * blocks, each a row-major image with a one-pixel border that must be zero.  The kernels write only the
 * interior. */

/* Elements (bf16) of the packed form of a conv weight [c_out, c_in, kt, ks, ks] (ks = 1 or 3). */
int64_t wan_vae_op_packed_conv_elems(int64_t c_out, int64_t c_in, int32_t kt, int32_t ks);

/* Pack a conv weight (WAN_F32 / WAN_BF16, [c_out, c_in, kt, ks, ks]) into dst (device, elements as above). */
wan_status wan_vae_op_pack_conv(const void* w, int32_t dtype, int64_t c_out, int64_t c_in, int32_t kt, int32_t ks,
                                void* dst, void* hip_stream);

/* One causal convolution launch over nf output frames (1 <= nf <= 16):
 *   out frame j (split = 1) or channel half s of it as frame 2 j + s (split = 2: c_out = 2 C, the time conv)
 *     = bias + sum over time taps dt < kt of conv_ks(in[j * kt + dt]) [+ res frame]
 * in: nf * kt padded input frames of c_in channels at H x W (H/2 x W/2 with up = 1: read through a
 * nearest x2 upsample; needs kt = 1, ks = 3); pass a zero frame where the causal padding falls.
 * w_packed: wan_vae_op_pack_conv output; bias [c_out] fp32.  out / res: nf * split padded frames of
 * c_out / split channels at H x W (res entries may be NULL, or equal the out entry for an in-place add).
 * c_in a multiple of 16; c_out a multiple of 32 (output-channel tiles of 96 when c_out is a multiple of
 * 96, else of 32). */
wan_status wan_vae_op_conv(const void* const* in, int32_t kt, int32_t ks, int32_t up, const void* w_packed,
                           const float* bias, int64_t c_in, int64_t c_out, int32_t split, int64_t H, int64_t W,
                           void* const* out, const void* const* res, int32_t nf, void* hip_stream);

/* out[j] = SiLU(RMS_norm(in[j])) over the first c channels (gamma [c] fp32) of nf padded frames of
 * round_up(c, 16) channels at H x W; out must not alias in. */
wan_status wan_vae_op_rms_silu(const void* const* in, void* const* out, int32_t nf, int64_t c, int64_t H, int64_t W,
                               const float* gamma, float eps, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* WAN_VAE_H */
