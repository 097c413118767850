/*
 * wan_dit.h - C ABI of the MI355X (gfx950) Wan-style video DiT denoiser forward.
 *
 * The forward computed here is the one the diffusers WanTransformer3DModel.forward prints on the
 * WanPipeline notes page (hk.pswp.cn "WanTransformer3DModel" / "WanTransformerBlock"), with the
 * block order of the Wan2.1 walk-through page (section 5.2) and the configuration defaults of the
 * WanAnimate page (configuration section: freq_dim 256, text_dim 4096, eps 1e-6,
 * qk_norm = rms_norm_across_heads, cross_attn_norm = True, rope_max_seq_len 1024):
 *
 *   latent [B,C_in,F,H_z,W_z] -> Conv3d (1,2,2) patch embed -> tokens [B, L=F*(H_z/2)*(W_z/2), D]
 *   timestep -> 256-d sinusoid -> time MLP -> temb [B,D] -> timestep_proj [B,6,D]
 *   text [B,Lt,4096] -> text projection -> ctx [B,Lt,D]
 *   N x WanTransformerBlock(x, ctx, timestep_proj, 3D RoPE)
 *   FP32 LayerNorm * (1 + scale) + shift (scale_shift_table + temb) -> proj_out -> unpatchify
 *
 * Conventions
 *   - All tensor data pointers are DEVICE pointers on the current HIP device, dense row-major.
 *   - The caller owns every tensor passed in.  wan_dit_create copies the weights into its own packed
 *     buffers, so the caller may free its weight tensors once create returns.
 *   - Every entry point validates all arguments before launching anything and returns a status; it
 *     never aborts.  On failure wan_dit_last_error() describes the problem.
 *   - Launches are asynchronous on the given stream (NULL = the default stream); the caller
 *     synchronises.  One handle must not be used by two forwards in flight at the same time (they
 *     share the handle's workspace).
 */
#ifndef WAN_DIT_H
#define WAN_DIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WAN_OK = 0,
  WAN_ERR_INVALID_ARG = 1,   /* null pointer, bad enum value, non-positive size */
  WAN_ERR_SHAPE = 2,         /* tensor shape does not match the configuration or the other tensors */
  WAN_ERR_DTYPE = 3,         /* dtype not accepted for this tensor */
  WAN_ERR_UNSUPPORTED = 4,   /* configuration outside what the kernels implement (e.g. head_dim != 128) */
  WAN_ERR_OOM = 5,           /* device allocation failed in wan_dit_create */
  WAN_ERR_HIP = 6,           /* a HIP runtime call or kernel launch failed */
  WAN_ERR_MISSING_WEIGHT = 7 /* a required weight name was not supplied (or supplied twice) */
} wan_status;

typedef enum { WAN_F32 = 0, WAN_BF16 = 1 } wan_dtype;

/* A dense row-major device tensor of up to 6 dimensions (shape[ndim..5] ignored). */
typedef struct {
  void* data;
  int32_t dtype; /* wan_dtype */
  int32_t ndim;
  int64_t shape[6];
} wan_tensor;

/* One named parameter.  Names and shapes (D = dim, Fd = ffn_dim, k = block index):
 *   patch_embedding.weight [D, C_in, 1, 2, 2]    patch_embedding.bias [D]
 *   time_embedder.linear_1.weight [D, freq_dim]  .bias [D]
 *   time_embedder.linear_2.weight [D, D]         .bias [D]
 *   time_proj.weight [6D, D]                     .bias [6D]
 *   text_embedder.linear_1.weight [D, text_dim]  .bias [D]
 *   text_embedder.linear_2.weight [D, D]         .bias [D]
 *   blocks.k.scale_shift_table [1, 6, D]
 *   blocks.k.attn{1,2}.to_{q,k,v,out}.weight [D, D]  .bias [D]
 *   blocks.k.attn{1,2}.norm_{q,k}.weight [D]
 *   blocks.k.norm2.weight [D]  blocks.k.norm2.bias [D]
 *   blocks.k.ffn.proj_in.weight [Fd, D] .bias [Fd]   blocks.k.ffn.proj_out.weight [D, Fd] .bias [D]
 *   scale_shift_table [1, 2, D]
 *   proj_out.weight [4*C_out, D]  proj_out.bias [4*C_out]
 * and, with max_image_len > 0 (the I2V image branch):
 *   image_embedder.linear_1.weight [D, image_dim] .bias [D]   image_embedder.linear_2.weight [D, D] .bias [D]
 *   blocks.k.attn2.add_k_proj.weight [D, D] .bias [D]   blocks.k.attn2.add_v_proj.weight [D, D] .bias [D]
 *   blocks.k.attn2.norm_added_k.weight [D]
 * Linear weights are nn.Linear layout [out, in].  Each may be WAN_F32 or WAN_BF16.
 */
typedef struct {
  const char* name;
  const void* data; /* device pointer */
  int32_t dtype;    /* wan_dtype */
  int32_t ndim;
  int64_t shape[6];
} wan_weight;

typedef struct {
  int32_t dim;            /* D; multiple of 512, = num_heads * head_dim */
  int32_t num_heads;
  int32_t head_dim;       /* must be 128 */
  int32_t ffn_dim;        /* multiple of 64 */
  int32_t num_layers;     /* >= 0 */
  int32_t in_channels;
  int32_t out_channels;
  int32_t text_dim;       /* 4096 in Wan; multiple of 64 */
  int32_t freq_dim;       /* 256 in Wan; multiple of 64 */
  int32_t patch_t, patch_h, patch_w; /* must be 1, 2, 2 */
  int32_t rope_dim_t, rope_dim_h, rope_dim_w; /* even, sum = head_dim; Wan: 44, 42, 42 */
  int32_t per_token_timestep; /* 1: forward also accepts timesteps [B, L] (workspace sized for it) */
  float eps;              /* LayerNorm / RMSNorm epsilon, 1e-6 in Wan */
  float reserved0;
  double rope_theta;      /* 10000 in Wan */
  int64_t max_batch;      /* workspace bounds checked by forward */
  int64_t max_tokens;     /* L per sample */
  int64_t max_text_len;   /* Lt */
  int64_t max_image_len;  /* CLIP image tokens of the I2V branch (Wan2.1 walk-through page, section 4: 257
                             tokens); 0 = no image branch (no image weights expected) */
  int32_t image_dim;      /* width of the image tokens (1280 on that page); multiple of 8 */
  int32_t reserved1;
} wan_dit_config;

typedef struct wan_dit wan_dit;

/* Validate cfg, check every weight named above against its shape (no extra, missing or duplicate
 * names), pack the weights into library-owned device buffers (GEMM weights as bf16, norms, tables
 * and the time MLP as fp32) and allocate all workspace for the max_* bounds.  Work is enqueued on
 * hip_stream and synchronised before returning.  On success *out receives the handle. */
wan_status wan_dit_create(const wan_dit_config* cfg, const wan_weight* weights, size_t n_weights, void* hip_stream,
                          wan_dit** out);

/* One DiT forward (one denoising step's velocity prediction).
 *   latent   [B, C_in, F, H_z, W_z]  WAN_F32 or WAN_BF16; H_z, W_z even; the token grid F x H_z/2 x W_z/2
 *            has at most 1024 positions per axis (F, H_z/2, W_z/2 <= 1024: the rotary tables)
 *   timestep [B] or [B, L] WAN_F32 (integer timesteps are passed as their float values); [B, L]
 *            needs cfg.per_token_timestep, with tokens in (f, h, w) order
 *   text_emb [B, Lt, text_dim] WAN_F32 or WAN_BF16
 *   out      [B, C_out, F, H_z, W_z] with the latent's dtype
 * Requires B <= max_batch, L <= max_tokens, 1 <= Lt <= max_text_len.  B == 0 is a no-op.
 * Allocates nothing; enqueues on hip_stream and returns without synchronising. */
wan_status wan_dit_forward(wan_dit* h, const wan_tensor* latent, const wan_tensor* timestep,
                           const wan_tensor* text_emb, wan_tensor* out, void* hip_stream);

/* The forward with CLIP image tokens (the I2V branch; Wan2.1 walk-through page, section 4: 257 image
 * tokens of width 1280 projected by an MLP to the model width and attended by a cross-attention of their
 * own; the WanPipeline notes' forward concatenates them in front of the text context).  Per block the
 * cross-attention output is softmax(q k_txt^T) v_txt + softmax(q k_img^T) v_img, with the image keys and
 * values from attn2.add_k_proj / add_v_proj (keys RMS-normalised with attn2.norm_added_k), before the
 * shared attn2.to_out projection.
 *   image_emb [B, Li, image_dim] WAN_F32 or WAN_BF16, 1 <= Li <= max_image_len (needs max_image_len > 0)
 * Everything else as wan_dit_forward. */
wan_status wan_dit_forward_image(wan_dit* h, const wan_tensor* latent, const wan_tensor* timestep,
                                 const wan_tensor* text_emb, const wan_tensor* image_emb, wan_tensor* out,
                                 void* hip_stream);

/* One guided flow-matching denoising step (Wan2.1 walk-through page, section 7: the guided velocity
 * v_u + s (v_c - v_u) and the update x_next = x + (sigma_next - sigma) v; section 6.3 works such a step by
 * hand).  Runs the forward as a batch of 2 on the same latent and timestep, with the conditional text
 * first and the unconditional (negative) text second, and fuses the guidance and the Euler update into
 * the unpatchify scatter:
 *   x_next[0, c, f, y, x] = latent[0, c, f, y, x] + (sigma_next - sigma) (v_u + guidance_scale (v_c - v_u)),
 *   c < out_channels (the first out_channels latent channels are the noisy sample; an I2V latent's
 *   condition and mask channels follow them).
 *   latent    [1, C_in, F, H_z, W_z] WAN_F32 or WAN_BF16     timestep [1] or [1, L] WAN_F32
 *   text_pair [2, Lt, text_dim]                                image_emb NULL, or [1, Li, image_dim]
 *   x_next    [1, C_out, F, H_z, W_z] with the latent's dtype, not aliasing the latent
 * sigma, sigma_next and the timestep are the caller's schedule (the pages leave the shifted schedule
 * open).  Needs max_batch >= 2.  Allocates nothing; asynchronous on hip_stream. */
wan_status wan_dit_denoise_step(wan_dit* h, const wan_tensor* latent, const wan_tensor* timestep,
                                const wan_tensor* text_pair, const wan_tensor* image_emb, float guidance_scale,
                                float sigma, float sigma_next, wan_tensor* x_next, void* hip_stream);

/* Release the handle's device buffers.  NULL is ignored. */
void wan_dit_destroy(wan_dit* h);

/* Opt-in timing of the self-attention kernel inside wan_dit_forward, for benchmarks (not part of the
 * computation: the softmax(Q K^T / sqrt(128)) V of every block runs the same either way).
 * max_launches > 0 creates 2 * max_launches HIP events on the handle's device, owned by the handle; every
 * later self-attention launch of wan_dit_forward is then bracketed by an event pair recorded on the
 * forward's stream, until max_launches pairs are in use (later launches run untimed).  max_launches == 0
 * turns the timing off and releases the events; wan_dit_destroy releases them too.  The forward still
 * allocates nothing.  Call it between forwards: events of a forward still running are released by it.
 * Errors: WAN_ERR_INVALID_ARG (NULL handle, max_launches outside [0, 2^20], current device not the
 * handle's), WAN_ERR_HIP (event creation failed; no events are kept). */
wan_status wan_dit_time_attention(wan_dit* h, int64_t max_launches);

/* Sum in milliseconds of the self-attention launches timed since the last call (or since
 * wan_dit_time_attention), and their number.  Host-synchronous: waits for the recorded events.  The
 * event pairs are free for reuse afterwards.  Errors: WAN_ERR_INVALID_ARG (NULL handle or output
 * pointer, current device not the handle's), WAN_ERR_HIP (an event query failed). */
wan_status wan_dit_attention_time(wan_dit* h, double* total_ms, int64_t* launches);

/* Text of the last error on the calling thread ("" if none); valid until the next call. */
const char* wan_dit_last_error(void);

/* Bytes of device memory the handle holds (packed weights + workspace). */
int64_t wan_dit_device_bytes(const wan_dit* h);

#ifdef __cplusplus
}
#endif
#endif /* WAN_DIT_H */
