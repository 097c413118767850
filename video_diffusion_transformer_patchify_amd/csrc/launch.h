// Internal launch functions of the gfx950 kernels (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;

enum { EPI_BF16 = 0, EPI_GELU_BF16 = 1, EPI_F32 = 2, EPI_RES_F32 = 3, EPI_GATE_F32 = 4 };

hipError_t launch_patchify(const void* x, int dtype, int64_t B, int64_t C, int64_t F, int64_t Hz, int64_t Wz,
                           int64_t kp, bf16_t* p, hipStream_t s);
hipError_t launch_unpatchify(const float* z, int64_t ldz, int64_t B, int64_t C, int64_t F, int64_t Hz, int64_t Wz,
                             void* out, int dtype, hipStream_t s);
// x_next = x[0, :C] + (sigma_next - sigma) (v_u + scale (v_c - v_u)), v_c / v_u from z rows [0, L) / [L, 2L);
// x has at least C channels (its first C are read)
hipError_t launch_cfg_euler(const float* z, int64_t ldz, int64_t C, int64_t F, int64_t Hz, int64_t Wz, const void* x,
                            int dtype, float scale, float sigma, float sigma_next, void* out, hipStream_t s);
hipError_t launch_pack_bf16(const void* src, int dtype, int64_t rows, int64_t cols, int64_t lds, bf16_t* dst,
                            int64_t ldd, hipStream_t s);
hipError_t launch_pack_f32(const void* src, int dtype, int64_t n, float* dst, hipStream_t s);

hipError_t launch_gemm_bf16(const bf16_t* x, int64_t ldx, const bf16_t* w, int64_t ldw, const float* bias, int64_t M,
                            int64_t N, int64_t K, int epi, void* out, int64_t ldo, const float* gate_tab,
                            const float* gate_src, int64_t gate_ld, int64_t rows_per_gate, hipStream_t s,
                            float* ws = nullptr, int64_t ws_bytes = 0);
// workspace of launch_gemm_bf16's stream-K tail: fp32 partial tiles of at most one round
int64_t gemm_workspace_bytes();
hipError_t launch_gemm_f32(const float* A, int64_t lda, const float* W, int64_t ldw, const float* bias, int64_t M,
                           int64_t N, int64_t K, float* C, int64_t ldc, int silu_in, int silu_out, hipStream_t s);

hipError_t launch_layernorm(float* x, int64_t rows, int64_t D, float eps, int mode, const float* tab_shift,
                            const float* tab_scale, const float* src, int64_t src_ld, int64_t src_shift_off,
                            int64_t src_scale_off, int64_t rows_per_src, const float* gamma, const float* beta,
                            int res_mode, const bf16_t* res, const float* res_tab, const float* res_src, int64_t res_ld,
                            bf16_t* y, hipStream_t s);
hipError_t launch_rms_rope(bf16_t* buf, int64_t ld, int64_t rows, int64_t D, float eps, int64_t off_a,
                           const float* gamma_a, int64_t off_b, const float* gamma_b, const float* rope, int64_t L,
                           int Fp, int Hp, int Wp, int dt, int dh, int dw, hipStream_t s, float scale_a = 1.0f);
// scale of the queries the attention kernels take pre-multiplied: log2(e) / sqrt(128)
inline float attention_q_scale() { return (float)(1.4426950408889634 / 11.313708498984761); }
hipError_t launch_transpose_v(const bf16_t* src, int64_t ld, int64_t col_off, int64_t B, int64_t L, int nh, bf16_t* vt,
                              int64_t ldv, hipStream_t s);
int64_t rope_table_floats(int Fp, int Hp, int Wp, int dt, int dh, int dw);
hipError_t launch_rope_table(float* tab, int Fp, int Hp, int Wp, int dt, int dh, int dw, double theta, hipStream_t s);
hipError_t launch_sinusoid(const float* t, int64_t rows, int freq_dim, float* out, hipStream_t s);

// ws (attention_workspace_bytes(B, Lq, nh) bytes, or null): runs the offset-free softmax kernel with the
// exact kernel redoing the workgroups whose scores left its range, and lets a launch whose last round of
// workgroups would leave most CUs idle split that round over key chunks and merge them (same result up to
// fp32 rounding).  Without it the exact kernel runs alone.
// q_prescaled: q holds the queries already multiplied by attention_q_scale() (log2(e) / sqrt(128)), as
// the QK-norm kernel writes them in the forward; otherwise the kernel multiplies them as it loads them.
// accumulate: o already holds the normalised output of another key set of the same queries (the text
// part of the I2V cross-attention); this one's output is added to it (fp32 sum, one bf16 rounding).
hipError_t launch_attention(const bf16_t* q, int64_t ldq, const bf16_t* k, int64_t ldk, const bf16_t* vt, int64_t ldv,
                            bf16_t* o, int64_t ldo, int64_t B, int64_t Lq, int64_t Lkv, int nh, bool self_attn,
                            hipStream_t s, float* ws = nullptr, int64_t ws_bytes = 0, bool q_prescaled = false,
                            bool accumulate = false, int64_t split_cap = 256);
// split_cap: most workgroups a key-split last round may use (the workspace holds their partial results)
int64_t attention_workspace_bytes(int64_t B, int64_t Lq, int nh, int64_t split_cap = 256);
// launch_attention with a workspace in the library's static device array (no allocation): at most
// attention_scratch_max_units() (batch, head, 256-query) units per call, a key split of at most 64
// workgroups; calls that overlap on one GPU share the array and race
hipError_t launch_attention_noalloc(const bf16_t* q, int64_t ldq, const bf16_t* k, int64_t ldk, const bf16_t* vt,
                                    int64_t ldv, bf16_t* o, int64_t ldo, int64_t B, int64_t Lq, int64_t Lkv, int nh,
                                    hipStream_t s);
int64_t attention_scratch_max_units();
int64_t attention_scratch_bytes();

hipError_t launch_mfma_probe(float* sink, int blocks, int64_t rounds, int random_operands, hipStream_t s);
