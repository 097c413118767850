/*
 * wan_ops.h - per-stage entry points of the gfx950 Wan DiT forward.
 *
 * These run the exact kernels wan_dit_forward uses, one stage at a time, on caller-provided device
 * buffers, so each stage can be checked and timed on its own.  Conventions as in wan_dit.h: device
 * pointers, dense row-major, caller owns everything, asynchronous on `stream`, status return, no
 * allocation.  bf16 data is raw bf16 bits (uint16).
 */
#ifndef WAN_OPS_H
#define WAN_OPS_H

#include <stdint.h>

#include "wan_dit.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Patchify gather (Wan2.1 walk-through page, section 5.1; WanPipeline notes: Conv3d kernel = stride
 * = (1,2,2), flatten(2).transpose(1,2)).
 *   latent [B, C, F, H_z, W_z] (dtype WAN_F32 | WAN_BF16) -> p bf16 [B*L, kp],
 *   p[(b*L + n), c*4 + 2i + j] = latent[b, c, f, 2h+i, 2w+j], n = (f*H' + h)*W' + w,
 *   columns [4C, kp) zero.  kp >= 4C, multiple of 8.  H_z, W_z even. */
wan_status wan_op_patchify(const void* latent, int32_t dtype, int64_t B, int64_t C, int64_t F, int64_t H_z,
                           int64_t W_z, int64_t kp, void* p, void* stream);

/* Unpatchify scatter (WanPipeline notes: proj_out output reshape(B,F',H',W',1,2,2,C_out),
 * permute(0,7,1,4,2,5,3,6), flatten).
 *   z fp32 [B*L, ldz] (columns [0, 4C)) -> out [B, C, F, H_z, W_z] of out_dtype,
 *   out[b, c, f, 2h+i, 2w+j] = z[b*L + n, (2i + j)*C + c]; bf16 output rounds to nearest even. */
wan_status wan_op_unpatchify(const float* z, int64_t ldz, int64_t B, int64_t C, int64_t F, int64_t H_z, int64_t W_z,
                             void* out, int32_t out_dtype, void* stream);

/* Guided Euler step fused into the unpatchify scatter (Wan2.1 walk-through page, section 7):
 *   z fp32 [2L, ldz]: proj_out rows of the conditional batch element (rows [0, L)) then the
 *   unconditional one (rows [L, 2L)), columns as for wan_op_unpatchify;
 *   x [1, Cx, F, H_z, W_z] (dtype), Cx >= C: the model input, whose first C channels are the noisy sample;
 *   x_next[0, c, f, 2h+i, 2w+j] = x[0, c, f, 2h+i, 2w+j] + (sigma_next - sigma) (v_u + s (v_c - v_u)),
 *   v_c = z[n, (2i+j)*C + c], v_u = z[L + n, (2i+j)*C + c]; fp32 arithmetic, bf16 output rounds to nearest
 *   even.  x_next must not alias x. */
wan_status wan_op_cfg_euler(const float* z, int64_t ldz, int64_t C, int64_t F, int64_t H_z, int64_t W_z, const void* x,
                            int64_t Cx, int32_t dtype, float guidance_scale, float sigma, float sigma_next, void* x_next,
                            void* stream);

/* GEMM with fused epilogue (every nn.Linear of the block; WanPipeline notes, WanTransformerBlock):
 *   acc[m, n] = sum_k x[m, k] * w[n, k] + bias[n]   x bf16 [M, ldx], w bf16 [N, ldw], bias fp32 [N]
 *   epilogue 0: out bf16 [m, n] = acc                 1: out bf16 = gelu_tanh(acc)
 *            2: out fp32 = acc                        3: out fp32 += acc
 *            4: out fp32 += acc * (gate_tab[n] + gate_src[(m / rows_per_gate) * gate_ld + n])
 * K multiple of 64; N multiple of 4; ldx, ldw multiples of 8; ldo multiple of 4. */
wan_status wan_op_gemm(const void* x, int64_t ldx, const void* w, int64_t ldw, const float* bias, int64_t M, int64_t N,
                       int64_t K, int32_t epilogue, void* out, int64_t ldo, const float* gate_tab,
                       const float* gate_src, int64_t gate_ld, int64_t rows_per_gate, void* stream);

/* Size in bytes of wan_op_gemm_ws's workspace (fp32 partial tiles of at most one round of the
 * persistent kernel: 256 tiles of 256 x 256). */
int64_t wan_op_gemm_workspace_bytes(void);

/* wan_op_gemm with a caller-owned device workspace (16-byte aligned, at least
 * wan_op_gemm_workspace_bytes(); its contents on entry do not matter and are overwritten).  Same
 * arguments, result and errors as wan_op_gemm, plus WAN_ERR_INVALID_ARG for a missing, misaligned or
 * short workspace.  Where the persistent kernel's last round of 256 x 256 tiles would leave at least half
 * of the CUs idle, that round's tiles are split along K (stream-K): each chunk writes an fp32 partial
 * tile to the workspace and a fix-up pass adds them in chunk order, then the bias and the epilogue.
 * The sums then differ from wan_op_gemm's by fp32 rounding order only.  Calls that share a workspace
 * must be ordered (same stream). */
wan_status wan_op_gemm_ws(const void* x, int64_t ldx, const void* w, int64_t ldw, const float* bias, int64_t M, int64_t N,
                          int64_t K, int32_t epilogue, void* out, int64_t ldo, const float* gate_tab,
                          const float* gate_src, int64_t gate_ld, int64_t rows_per_gate, void* workspace,
                          int64_t workspace_bytes, void* stream);

/* Residual add + LayerNorm over D (population variance, eps) of fp32 rows x [rows, D] -> bf16 y [rows, D]
 * (WanPipeline notes, WanTransformerBlock: hidden_states + attn_output * gate_msa, + attn_output,
 * + ff_output * c_gate_msa, each followed by the next norm).  With r = res [rows, D] bf16 and
 * s = row / rows_per_src:
 *   res_mode 1: x += r;   res_mode 2: x += r * (res_tab[d] + res_src[s*res_ld + d]);   x is updated in place.
 * Then:
 *   mode 0 (norm1 / norm3 / norm_out + modulation; block and output head):
 *     y = LN(x) * (1 + tab_scale[d] + src[s*src_ld + src_scale_off + d])
 *               + tab_shift[d] + src[s*src_ld + src_shift_off + d]
 *   mode 1 (norm2 with affine, cross_attn_norm): y = LN(x) * gamma[d] + beta[d]
 * D multiple of 256, at most 6144. */
wan_status wan_op_layernorm(float* x, int64_t rows, int64_t D, float eps, int32_t mode, const float* tab_shift,
                            const float* tab_scale, const float* src, int64_t src_ld, int64_t src_shift_off,
                            int64_t src_scale_off, int64_t rows_per_src, const float* gamma, const float* beta,
                            int32_t res_mode, const void* res, const float* res_tab, const float* res_src, int64_t res_ld,
                            void* y, void* stream);

/* Size in floats of the RoPE angle table for a (Fp, Hp, Wp) token grid and head-dim split
 * (dt, dh, dw): 2 * (Fp*dt/2 + Hp*dh/2 + Wp*dw/2). */
int64_t wan_op_rope_table_floats(int32_t Fp, int32_t Hp, int32_t Wp, int32_t dt, int32_t dh, int32_t dw);

/* 3D RoPE angle table (WanAnimate page, architecture section: WanRotaryPosEmbed, one 1D rotary
 * frequency set per T/H/W axis, concatenated): cos then sin of pos * theta^(-2j/d_axis) for every
 * axis position; table must hold wan_op_rope_table_floats(...) floats. */
wan_status wan_op_rope_table(float* table, int32_t Fp, int32_t Hp, int32_t Wp, int32_t dt, int32_t dh, int32_t dw,
                             double theta, void* stream);

/* In-place QK RMSNorm (+ RoPE) on bf16 rows buf [rows, ld] (WanAnimate page, configuration section:
 * qk_norm = rms_norm_across_heads, eps):
 *   for each row and each segment s in {a, b (if gamma_b != NULL)}: u = buf[row, off_s : off_s + D],
 *   u <- u / sqrt(mean(u^2) + eps) * gamma_s; then, if table != NULL, every 128-wide head has its
 *   channel pairs (2m, 2m+1) rotated by the angle of pair m for token n = row % L, decoded as
 *   (f, h, w) on the Fp x Hp x Wp grid.  Segment a is also multiplied by scale_a (1 for the plain norm;
 *   the forward passes log2(e)/sqrt(128) for the queries, which its attention takes pre-multiplied), in
 *   fp32 before the one bf16 rounding.  D multiple of 512, at most 12288. */
wan_status wan_op_qk_norm_rope(void* buf, int64_t ld, int64_t rows, int64_t D, float eps, int64_t off_a,
                               const float* gamma_a, int64_t off_b, const float* gamma_b, const float* table,
                               int64_t L, int32_t Fp, int32_t Hp, int32_t Wp, int32_t dt, int32_t dh, int32_t dw,
                               float scale_a, void* stream);

/* V re-layout for the attention kernel: src bf16 rows [B*L, ld], heads at columns
 * col_off + 128h .. +127 -> vt bf16 [B, nh, 128, ldv] with vt[b,h,d,l] = src[b*L + l, col_off + 128h + d]
 * and zeros for l in [L, ldv).  ldv multiple of 64, >= L. */
wan_status wan_op_transpose_v(const void* src, int64_t ld, int64_t col_off, int64_t B, int64_t L, int32_t nh,
                              void* vt, int64_t ldv, void* stream);

/* Attention forward, head_dim 128, no mask (Wan2.1 walk-through page, section 5.2; WanPipeline notes
 * attn1 / attn2): for every batch b, head h, query i < Lq:
 *   o[b*Lq + i, 128h + :] = sum_j softmax_j(q_i . k_j / sqrt(128)) v_j
 *   q = q[b*Lq + i, 128h + :] (row stride ldq), k_j = k[b*Lkv + j, 128h + :] (row stride ldk),
 *   v_j = vt[b, h, :, j] from wan_op_transpose_v (ldv >= Lkv rounded up to 64).
 * bf16 in / out, fp32 softmax (online, with a running row max).  The queries are multiplied by
 * log2(e)/sqrt(128) and rounded to bf16 as the kernel loads them, so the scores come out in base-2 units. */
wan_status wan_op_attention(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* vt, int64_t ldv,
                            void* o, int64_t ldo, int64_t B, int64_t Lq, int64_t Lkv, int32_t nh, void* stream);

/* The same attention with a caller-owned device workspace of wan_op_attention_workspace_bytes(B, Lq, nh)
 * bytes (16-byte aligned; contents need no initialisation), the way the forward runs it:
 *   - The softmax first runs without any row max: probabilities are exp2 of the base-2 scores as they
 *     are (the common offset cancels in the final division).  A 64-row block of a wave whose scores
 *     leave the range where that is safe (a 16-key probability sum above 2^64, or a first 32-key block
 *     whose max is below -60) drops its results, and a second pass with the exact running-max softmax
 *     recomputes the (batch, head, 256-query) units marked so; it returns at once for every other unit.
 *     The marks live in the workspace.
 *   - Workgroups are (batch, head, 256-query tile) units, one per CU at a time; when the last round of
 *     units would occupy at most half of the CUs, its units are split into key chunks of a multiple of
 *     64 keys, each chunk writes its unnormalised output, exponent offset and row sum to the workspace,
 *     and a merge pass forms the softmax over all keys from them
 *     (o = sum_c 2^(m_c - m) O_c / sum_c 2^(m_c - m) l_c).
 * Results equal wan_op_attention's up to fp32 rounding.  The workspace is in use until the call's work on
 * `stream` completes; calls that overlap on one workspace race.  Errors: WAN_ERR_INVALID_ARG for a NULL,
 * misaligned or short workspace. */
wan_status wan_op_attention_ws(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* vt, int64_t ldv,
                               void* o, int64_t ldo, int64_t B, int64_t Lq, int64_t Lkv, int32_t nh, void* workspace,
                               int64_t workspace_bytes, void* stream);
/* Workspace bytes wan_op_attention_ws needs for B batches of Lq queries and nh heads (-1 for B or Lq
 * negative or nh <= 0). */
int64_t wan_op_attention_workspace_bytes(int64_t B, int64_t Lq, int32_t nh);

/* wan_op_attention_ws without a caller workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation): the workspace is a
 * static device array of the library, 8.8 MB on each GPU it runs on, held until the process ends.  Limits:
 * at most 16384 (batch, head, 256-query) units per call (B * nh * ceil(Lq / 256)), and a key-split last
 * round of at most 64 workgroups (otherwise the same softmax and merge as wan_op_attention_ws).  Larger
 * calls fail with WAN_ERR_UNSUPPORTED before any launch.  Allocates nothing.  Every call on a GPU uses that
 * GPU's one array: calls that overlap in time on one GPU (two streams, two threads) race.  Nothing in the
 * array needs clearing between calls (every value read is written earlier in the same call). */
wan_status wan_op_attention_noalloc(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* vt, int64_t ldv,
                                    void* o, int64_t ldo, int64_t B, int64_t Lq, int64_t Lkv, int32_t nh, void* stream);

/* Timestep embedding, fp32 throughout (WanAnimate page, configuration section: freq_dim 256, the
 * time embedder kept in fp32; WanPipeline notes: temb (B, D), timestep_proj (B, 6D)):
 *   s = [cos(t w_i), sin(t w_i)], w_i = 10000^(-i/(freq_dim/2))
 *   temb  = W2 silu(W1 s + b1) + b2                  [rows, D]
 *   tproj = Wp silu(temb) + bp                       [rows, 6D]
 * Weights fp32 [out, in].  work must hold rows * (freq_dim + D) floats. */
wan_status wan_op_time_embed(const float* t, int64_t rows, int32_t freq_dim, int64_t D, const float* w1,
                             const float* b1, const float* w2, const float* b2, const float* wp, const float* bp,
                             float* temb, float* tproj, float* work, void* stream);

/* Measurement aid, not a step of the forward: the dense bf16 MFMA ceiling that the forward's MFMA
 * fractions are read against.  `blocks` workgroups of 256 threads each run `rounds` rounds of 64
 * 32x32x16 bf16 MFMAs per wave (16 independent accumulators) on operands held in LDS, with no global
 * memory traffic; the work is blocks * 4 * rounds * 64 * 32768 FLOP.  random_operands = 0 uses zeros (least power drawn); 1 uses
 * values drawn like the GEMM operands (U(-1,1) and U(-0.05,0.05)), which shows what dense bf16 work
 * sustains once the clock settles.  sink: device fp32 [blocks * 256], receives per-thread sums (keeps the
 * work alive).  Time it with events on `stream`. */
wan_status wan_probe_mfma(float* sink, int32_t blocks, int64_t rounds, int32_t random_operands, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* WAN_OPS_H */
