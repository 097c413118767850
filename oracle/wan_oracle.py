"""Plain float64 CPU oracle of the Wan-style video DiT denoiser forward.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the package entry module and the
CPU-baseline leg of the benchmark may import this module.  The GPU library never calls it and shares
no code with it; the two meet only through the seeded generator in ``wan_inputs``.

Every function evaluates the plain definition in float64 with numpy, in the order the pages give it:
no blocking, fusion or reordering beyond splitting attention into query chunks (which does not change
the mathematics).  Matrix products use the host BLAS.

Sources (page titles; sections / printed code):
  [W21]  "【VLA与模仿学习】Wan2.1框架与训练源码导读" - section 3.1 (VAE latent shapes), section 5.1
         (Patchify -> space-time tokens, L = F*(H_z/2)*(W_z/2)), section 5.2 (block order), section 5.3 (head).
  [DIF]  diffusers WanPipeline notes (hk.pswp.cn) - the printed WanTransformer3DModel.forward
         (rope, patch_embedding, flatten/transpose, condition_embedder, blocks, norm_out + shift/scale,
         proj_out, reshape/permute/flatten unpatchify) and WanTransformerBlock.forward (modulation chunk
         order, norm1/attn1/gate, norm2/attn2 ungated residual, norm3/ffn/gate).
  [ANI]  "Diffusers 中 WanAnimateTransformer3DModel 深度解析" - 架构全景 (3D RoPE built per T/H/W axis and
         concatenated), 配置参数全解 (freq_dim 256, text_dim 4096, qk_norm rms_norm_across_heads, eps 1e-6,
         cross_attn_norm True, rope_max_seq_len 1024, fp32-kept modules).

  [W21 6.3, 7] the flow-matching conventions: x_sigma = (1 - sigma) z + sigma eps, target velocity eps - z,
         the Euler update x_next = x + (sigma_next - sigma) v, and the CFG combine v_u + s (v_c - v_u).
  [W21 4]  the I2V CLIP branch: 257 image tokens of width 1280 projected to the model width by an MLP and
         attended by a cross-attention of their own; [DIF forward] concatenates them before the text.

Readings taken where the pages are silent (each one also listed in the design notes):
  sinusoid [cos, sin] with frequencies 10000^(-i/128); time MLP Lin-SiLU-Lin then SiLU-Lin(6D);
  text projection Lin-GELU_tanh-Lin; LayerNorm without affine for norm1/norm3/norm_out and with
  affine for norm2; QK RMSNorm over the whole model width with a learned gain, applied to q and k of
  both attentions, before RoPE; RoPE head-dim split 44/42/42 with theta 1e4 and adjacent pairs;
  attention scale 1/sqrt(head_dim), no masks; every Linear/Conv has a bias; the image MLP is
  Lin(image_dim -> D) - GELU_tanh - Lin(D -> D) like the text projection; the image tokens, first in the
  context, get their own key/value projections and key RMSNorm, their attention output is added to the
  text attention output before the shared output projection.

Parity status: every function here is pinned by a CPU test (closed forms, invariants, brute force or a
torch library routine); see tests/test_oracle_pins.py.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def _arr(w, name: str) -> np.ndarray:
    """Weight `name` as float64, from a dict of arrays or from an object with .f64(name)."""
    if hasattr(w, "f64"):
        return w.f64(name)
    return np.asarray(w[name], dtype=np.float64)


# ---------------------------------------------------------------------------------------------
# Shapes [W21 section 3.1, section 5.1; DIF latent-shape code]
# ---------------------------------------------------------------------------------------------


def vae_latent_shape(batch: int, frames: int, height: int, width: int, channels: int = 16,
                     t_stride: int = 4, s_stride: int = 8) -> tuple:
    """[B,3,T,H,W] -> [B,C,1+(T-1)/4,H/8,W/8]; T must be 4n+1 [W21 3.1]."""
    if (frames - 1) % t_stride != 0:
        raise ValueError(f"frame count {frames} is not {t_stride}n+1")
    if height % s_stride or width % s_stride:
        raise ValueError("spatial size not divisible by the VAE stride")
    return (batch, channels, 1 + (frames - 1) // t_stride, height // s_stride, width // s_stride)


def token_grid(frames: int, h_z: int, w_z: int, patch=(1, 2, 2)) -> tuple:
    """(F', H', W') after the (1,2,2) patch [W21 5.1]."""
    pt, ph, pw = patch
    if frames % pt or h_z % ph or w_z % pw:
        raise ValueError("latent size not divisible by the patch")
    return (frames // pt, h_z // ph, w_z // pw)


def num_tokens(frames: int, h_z: int, w_z: int, patch=(1, 2, 2)) -> int:
    """L = F x (H_z/2) x (W_z/2) [W21 5.1]."""
    f, h, w = token_grid(frames, h_z, w_z, patch)
    return f * h * w


# ---------------------------------------------------------------------------------------------
# Patchify / unpatchify [DIF forward: patch_embedding Conv3d(kernel=stride=(1,2,2)),
# flatten(2).transpose(1,2); proj_out, reshape(B,F',H',W',pt,ph,pw,-1), permute(0,7,1,4,2,5,3,6), flatten]
# ---------------------------------------------------------------------------------------------


def patchify(x: np.ndarray, patch=(1, 2, 2)) -> np.ndarray:
    """Latent [B,C,F,H_z,W_z] -> patch vectors [B, L, C*pt*ph*pw].

    Token n = (f*H' + h)*W' + w (flatten of the conv output's (F',H',W') grid); the patch vector is
    ordered like the Conv3d weight [D, C, pt, ph, pw] flattened, so channel is the slowest index.
    """
    b, c, f, hz, wz = x.shape
    pt, ph, pw = patch
    fp, hp, wp = f // pt, hz // ph, wz // pw
    v = x.reshape(b, c, fp, pt, hp, ph, wp, pw)
    v = v.transpose(0, 2, 4, 6, 1, 3, 5, 7)          # b, f', h', w', c, pt, ph, pw
    return np.ascontiguousarray(v.reshape(b, fp * hp * wp, c * pt * ph * pw))


def patch_embed(x: np.ndarray, w: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """Conv3d with kernel = stride = patch, written as patch vectors times the flattened kernel.

    x [B,C,F,H_z,W_z], w [D,C,pt,ph,pw], bias [D] -> tokens [B, L, D].
    """
    d = w.shape[0]
    patch = tuple(w.shape[2:])
    p = patchify(x, patch)
    return p @ w.reshape(d, -1).T + bias


def unpatchify(z: np.ndarray, frames: int, h_z: int, w_z: int, out_channels: int, patch=(1, 2, 2)) -> np.ndarray:
    """proj_out tokens [B, L, pt*ph*pw*C_out] -> latent [B, C_out, F, H_z, W_z].

    Follows the printed reshape (B,F',H',W',pt,ph,pw,C) -> permute(0,7,1,4,2,5,3,6) -> flatten.
    """
    b = z.shape[0]
    pt, ph, pw = patch
    fp, hp, wp = frames // pt, h_z // ph, w_z // pw
    v = z.reshape(b, fp, hp, wp, pt, ph, pw, out_channels)
    v = v.transpose(0, 7, 1, 4, 2, 5, 3, 6)
    return np.ascontiguousarray(v.reshape(b, out_channels, fp * pt, hp * ph, wp * pw))


# ---------------------------------------------------------------------------------------------
# Elementwise functions
# ---------------------------------------------------------------------------------------------


def silu(u: np.ndarray) -> np.ndarray:
    return u / (1.0 + np.exp(-u))


def gelu_tanh(u: np.ndarray) -> np.ndarray:
    """GELU, tanh approximation: u/2 * (1 + tanh(sqrt(2/pi) * (u + 0.044715 u^3)))."""
    return 0.5 * u * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (u + 0.044715 * u ** 3)))


def linear(u: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """nn.Linear: u @ w^T + b with w stored [out, in]."""
    return u @ w.T + b


def layer_norm(u: np.ndarray, eps: float, gamma=None, beta=None) -> np.ndarray:
    """LayerNorm over the last axis, population variance."""
    mu = u.mean(axis=-1, keepdims=True)
    var = ((u - mu) ** 2).mean(axis=-1, keepdims=True)
    y = (u - mu) / np.sqrt(var + eps)
    if gamma is not None:
        y = y * gamma
    if beta is not None:
        y = y + beta
    return y


def rms_norm(u: np.ndarray, eps: float, gamma=None) -> np.ndarray:
    """RMSNorm over the last axis: u / sqrt(mean(u^2) + eps) * gamma."""
    y = u / np.sqrt((u * u).mean(axis=-1, keepdims=True) + eps)
    if gamma is not None:
        y = y * gamma
    return y


# ---------------------------------------------------------------------------------------------
# Timestep sinusoid + MLP, text projection [ANI 配置参数全解: freq_dim 256, text_dim 4096;
# DIF forward: condition_embedder -> temb (B,D), timestep_proj (B,6D) -> unflatten (B,6,D), ctx (B,Lt,D)]
# ---------------------------------------------------------------------------------------------


def sinusoid(t: np.ndarray, dim: int = 256) -> np.ndarray:
    """[cos(t w_i), sin(t w_i)], w_i = 10000^(-i/(dim/2)), i = 0..dim/2-1."""
    half = dim // 2
    omega = np.power(10000.0, -np.arange(half, dtype=np.float64) / half)
    arg = np.asarray(t, dtype=np.float64)[..., None] * omega
    return np.concatenate([np.cos(arg), np.sin(arg)], axis=-1)


def time_embed(t: np.ndarray, w: dict, freq_dim: int = 256):
    """t [...] -> (temb [..., D], tproj [..., 6, D])."""
    s = sinusoid(t, freq_dim)
    temb = linear(silu(linear(s, _arr(w, "time_embedder.linear_1.weight"), _arr(w, "time_embedder.linear_1.bias"))),
                  _arr(w, "time_embedder.linear_2.weight"), _arr(w, "time_embedder.linear_2.bias"))
    tproj = linear(silu(temb), _arr(w, "time_proj.weight"), _arr(w, "time_proj.bias"))
    return temb, tproj.reshape(tproj.shape[:-1] + (6, temb.shape[-1]))


def text_embed(e: np.ndarray, w: dict) -> np.ndarray:
    """[B, Lt, 4096] -> [B, Lt, D]."""
    h = gelu_tanh(linear(e, _arr(w, "text_embedder.linear_1.weight"), _arr(w, "text_embedder.linear_1.bias")))
    return linear(h, _arr(w, "text_embedder.linear_2.weight"), _arr(w, "text_embedder.linear_2.bias"))


def image_embed(img: np.ndarray, w: dict) -> np.ndarray:
    """CLIP image tokens [B, Li, image_dim] -> [B, Li, D] [W21 4: 257 tokens of 1280 through an MLP]."""
    h = gelu_tanh(linear(img, _arr(w, "image_embedder.linear_1.weight"), _arr(w, "image_embedder.linear_1.bias")))
    return linear(h, _arr(w, "image_embedder.linear_2.weight"), _arr(w, "image_embedder.linear_2.bias"))


# ---------------------------------------------------------------------------------------------
# 3D rotary embedding [ANI 架构全景 / 关键子模块: WanRotaryPosEmbed, separate 1D RoPE per T/H/W,
# concatenated; DIF: rope table (1,1,L,64) complex for head_dim 128]
# ---------------------------------------------------------------------------------------------


def rope_angles(fp: int, hp: int, wp: int, head_dim: int = 128, dims=(44, 42, 42), theta: float = 1e4) -> np.ndarray:
    """Angle table [L, head_dim/2] for tokens in (f, h, w) order.

    Axis a with d_a channels uses frequencies theta^(-2j/d_a), j < d_a/2, at the token's integer
    position on that axis; the three per-axis angle lists are concatenated (t, then h, then w).
    """
    assert sum(dims) == head_dim
    per_axis = []
    for n, d_a in zip((fp, hp, wp), dims):
        omega = np.power(theta, -np.arange(0, d_a, 2, dtype=np.float64) / d_a)
        per_axis.append(np.outer(np.arange(n, dtype=np.float64), omega))
    ang_t, ang_h, ang_w = per_axis
    f_idx, h_idx, w_idx = np.meshgrid(np.arange(fp), np.arange(hp), np.arange(wp), indexing="ij")
    return np.concatenate([ang_t[f_idx.reshape(-1)], ang_h[h_idx.reshape(-1)], ang_w[w_idx.reshape(-1)]], axis=-1)


def apply_rope(u: np.ndarray, ang: np.ndarray) -> np.ndarray:
    """Rotate adjacent channel pairs (u[2m], u[2m+1]) by ang[..., m].

    u [L, H, head_dim] (ang broadcast over heads) or [L, head_dim]; ang [L, head_dim/2].
    """
    if u.ndim == 3:
        ang = ang[:, None, :]
    elif u.ndim != 2:
        raise ValueError("apply_rope expects [L, H, d] or [L, d]")
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = u[..., 0::2], u[..., 1::2]
    out = np.empty_like(u)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


# ---------------------------------------------------------------------------------------------
# Attention [W21 5.2: self-attention over all video tokens, cross-attention to text; DIF block]
# ---------------------------------------------------------------------------------------------


def _attn_one(q, k, v, scale, chunk):
    out = np.empty((q.shape[0], v.shape[1]))
    for s in range(0, q.shape[0], chunk):
        sc = (q[s:s + chunk] @ k.T) * scale
        sc -= sc.max(axis=1, keepdims=True)
        p = np.exp(sc)
        out[s:s + chunk] = (p @ v) / p.sum(axis=1, keepdims=True)
    return out


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float | None = None, chunk: int = 1024,
              workers: int = 1) -> np.ndarray:
    """softmax(q k^T * scale) v per head, no mask.

    q [Lq, H, d], k [Lk, H, d], v [Lk, H, d] -> [Lq, H, d].  scale defaults to 1/sqrt(d).
    """
    lq, nh, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.empty((lq, nh, v.shape[2]))

    def run(h):
        out[:, h, :] = _attn_one(np.ascontiguousarray(q[:, h]), np.ascontiguousarray(k[:, h]),
                                 np.ascontiguousarray(v[:, h]), scale, chunk)

    if workers > 1:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(run, range(nh)))
    else:
        for h in range(nh):
            run(h)
    return out


# ---------------------------------------------------------------------------------------------
# Transformer block [DIF WanTransformerBlock.forward; W21 5.2 order; ANI qk_norm, cross_attn_norm, eps]
# ---------------------------------------------------------------------------------------------


def modulation(table: np.ndarray, tproj: np.ndarray) -> list:
    """table (1,6,D) + timestep projection (B,6,D) or per token (B,L,6,D) -> six [B,1|L,D] arrays.

    Order as printed: shift_msa, scale_msa, gate_msa, c_shift_msa, c_scale_msa, c_gate_msa.
    """
    if tproj.ndim == 3:
        m = table + tproj                      # B,6,D
        return [m[:, i][:, None, :] for i in range(6)]
    m = table[None] + tproj                    # B,L,6,D
    return [m[:, :, i] for i in range(6)]


def _cross_attention(y2: np.ndarray, ctx: np.ndarray, w: dict, p: str, num_heads: int, eps: float, n_img: int,
                     workers: int) -> np.ndarray:
    """attn2 before its output projection: text keys/values (the context after its first n_img tokens),
    plus, with n_img > 0, an attention of its own over the leading image tokens, added."""
    b, l, d = y2.shape
    hd = d // num_heads
    q2 = rms_norm(linear(y2, _arr(w, p + "attn2.to_q.weight"), _arr(w, p + "attn2.to_q.bias")), eps, _arr(w, p + "attn2.norm_q.weight"))
    txt = ctx[:, n_img:]
    k2 = rms_norm(linear(txt, _arr(w, p + "attn2.to_k.weight"), _arr(w, p + "attn2.to_k.bias")), eps, _arr(w, p + "attn2.norm_k.weight"))
    v2 = linear(txt, _arr(w, p + "attn2.to_v.weight"), _arr(w, p + "attn2.to_v.bias"))
    lt = txt.shape[1]
    a2 = np.empty_like(q2)
    for bi in range(b):
        a2[bi] = attention(q2[bi].reshape(l, num_heads, hd), k2[bi].reshape(lt, num_heads, hd),
                           v2[bi].reshape(lt, num_heads, hd), workers=workers).reshape(l, d)
    if n_img > 0:
        img = ctx[:, :n_img]
        ki = rms_norm(linear(img, _arr(w, p + "attn2.add_k_proj.weight"), _arr(w, p + "attn2.add_k_proj.bias")), eps,
                      _arr(w, p + "attn2.norm_added_k.weight"))
        vi = linear(img, _arr(w, p + "attn2.add_v_proj.weight"), _arr(w, p + "attn2.add_v_proj.bias"))
        for bi in range(b):
            a2[bi] += attention(q2[bi].reshape(l, num_heads, hd), ki[bi].reshape(n_img, num_heads, hd),
                                vi[bi].reshape(n_img, num_heads, hd), workers=workers).reshape(l, d)
    return a2


def block_forward(x: np.ndarray, ctx: np.ndarray, tproj: np.ndarray, ang: np.ndarray, w: dict, prefix: str,
                  num_heads: int, eps: float = 1e-6, workers: int = 1, n_img: int = 0) -> np.ndarray:
    """One WanTransformerBlock.  x [B,L,D] (fp64), ctx [B,n_img+Lt,D] (image tokens first), tproj [B,6,D] or
    [B,L,6,D]."""
    p = prefix
    b, l, d = x.shape
    hd = d // num_heads
    sh1, sc1, g1, sh2, sc2, g2 = modulation(_arr(w, p + "scale_shift_table"), tproj)

    # 1. self-attention
    y = layer_norm(x, eps) * (1.0 + sc1) + sh1
    q = linear(y, _arr(w, p + "attn1.to_q.weight"), _arr(w, p + "attn1.to_q.bias"))
    k = linear(y, _arr(w, p + "attn1.to_k.weight"), _arr(w, p + "attn1.to_k.bias"))
    v = linear(y, _arr(w, p + "attn1.to_v.weight"), _arr(w, p + "attn1.to_v.bias"))
    q = rms_norm(q, eps, _arr(w, p + "attn1.norm_q.weight"))
    k = rms_norm(k, eps, _arr(w, p + "attn1.norm_k.weight"))
    a = np.empty_like(q)
    for bi in range(b):
        qh = apply_rope(q[bi].reshape(l, num_heads, hd), ang)
        kh = apply_rope(k[bi].reshape(l, num_heads, hd), ang)
        a[bi] = attention(qh, kh, v[bi].reshape(l, num_heads, hd), workers=workers).reshape(l, d)
    x = x + linear(a, _arr(w, p + "attn1.to_out.weight"), _arr(w, p + "attn1.to_out.bias")) * g1

    # 2. cross-attention (norm2 with affine; residual not gated)
    y2 = layer_norm(x, eps, _arr(w, p + "norm2.weight"), _arr(w, p + "norm2.bias"))
    a2 = _cross_attention(y2, ctx, w, p, num_heads, eps, n_img, workers)
    x = x + linear(a2, _arr(w, p + "attn2.to_out.weight"), _arr(w, p + "attn2.to_out.bias"))

    # 3. feed-forward with gated residual
    y3 = layer_norm(x, eps) * (1.0 + sc2) + sh2
    h = gelu_tanh(linear(y3, _arr(w, p + "ffn.proj_in.weight"), _arr(w, p + "ffn.proj_in.bias")))
    x = x + linear(h, _arr(w, p + "ffn.proj_out.weight"), _arr(w, p + "ffn.proj_out.bias")) * g2
    return x


def block_forward_rows(x: np.ndarray, ctx: np.ndarray, tproj: np.ndarray, ang: np.ndarray, w: dict, prefix: str,
                       num_heads: int, rows, eps: float = 1e-6, workers: int = 1, n_img: int = 0) -> np.ndarray:
    """block_forward restricted to the token rows `rows` of every batch element: [B, len(rows), D].

    Only self-attention mixes tokens, and only through its keys and values, so those come from every
    token; every other step (the queries, both attentions' outputs, the residuals, norms and FFN) is
    evaluated on the requested rows alone.  Same arithmetic as block_forward, row by row.
    """
    p = prefix
    rows = np.asarray(rows, dtype=np.int64)
    b, l, d = x.shape
    hd = d // num_heads
    tp = tproj if tproj.ndim == 3 else tproj[:, rows]
    sh1, sc1, g1, sh2, sc2, g2 = modulation(_arr(w, p + "scale_shift_table"), tp)
    mod_all = modulation(_arr(w, p + "scale_shift_table"), tproj)
    xr = x[:, rows]

    # 1. self-attention: keys and values of all tokens, queries of the rows
    y_all = layer_norm(x, eps) * (1.0 + mod_all[1]) + mod_all[0]
    k = rms_norm(linear(y_all, _arr(w, p + "attn1.to_k.weight"), _arr(w, p + "attn1.to_k.bias")), eps,
                 _arr(w, p + "attn1.norm_k.weight"))
    v = linear(y_all, _arr(w, p + "attn1.to_v.weight"), _arr(w, p + "attn1.to_v.bias"))
    del y_all
    y = layer_norm(xr, eps) * (1.0 + sc1) + sh1
    q = rms_norm(linear(y, _arr(w, p + "attn1.to_q.weight"), _arr(w, p + "attn1.to_q.bias")), eps,
                 _arr(w, p + "attn1.norm_q.weight"))
    a = np.empty_like(q)
    for bi in range(b):
        qh = apply_rope(q[bi].reshape(len(rows), num_heads, hd), ang[rows])
        kh = apply_rope(k[bi].reshape(l, num_heads, hd), ang)
        a[bi] = attention(qh, kh, v[bi].reshape(l, num_heads, hd), workers=workers).reshape(len(rows), d)
    del k, v
    xr = xr + linear(a, _arr(w, p + "attn1.to_out.weight"), _arr(w, p + "attn1.to_out.bias")) * g1

    # 2. cross-attention, 3. feed-forward: per token
    y2 = layer_norm(xr, eps, _arr(w, p + "norm2.weight"), _arr(w, p + "norm2.bias"))
    a2 = _cross_attention(y2, ctx, w, p, num_heads, eps, n_img, workers)
    xr = xr + linear(a2, _arr(w, p + "attn2.to_out.weight"), _arr(w, p + "attn2.to_out.bias"))
    y3 = layer_norm(xr, eps) * (1.0 + sc2) + sh2
    h = gelu_tanh(linear(y3, _arr(w, p + "ffn.proj_in.weight"), _arr(w, p + "ffn.proj_in.bias")))
    return xr + linear(h, _arr(w, p + "ffn.proj_out.weight"), _arr(w, p + "ffn.proj_out.bias")) * g2


def head_forward(x: np.ndarray, temb: np.ndarray, w: dict, eps: float = 1e-6) -> np.ndarray:
    """norm_out (no affine) + shift/scale from scale_shift_table (1,2,D) + temb, then proj_out.

    temb [B,D] (per-sample timestep) or [B,L,D] (per-token).  Returns z [B, L, N_out].
    """
    table = _arr(w, "scale_shift_table")
    if temb.ndim == 2:
        m = table + temb[:, None, :]           # B,2,D
        shift, scale = m[:, 0][:, None, :], m[:, 1][:, None, :]
    else:
        m = table[None] + temb[:, :, None, :]  # B,L,2,D
        shift, scale = m[:, :, 0], m[:, :, 1]
    y = layer_norm(x, eps) * (1.0 + scale) + shift
    return linear(y, _arr(w, "proj_out.weight"), _arr(w, "proj_out.bias"))


# ---------------------------------------------------------------------------------------------
# Full forward [DIF WanTransformer3DModel.forward]
# ---------------------------------------------------------------------------------------------


def _context(cfg, w, text, image):
    """Text context, with the projected image tokens concatenated in front when there are any [DIF forward]."""
    ctx = text_embed(np.asarray(text, dtype=np.float64), w)
    if image is None:
        return ctx, 0
    img = image_embed(np.asarray(image, dtype=np.float64), w)
    return np.concatenate([img, ctx], axis=1), img.shape[1]


def forward(cfg, weights, latent: np.ndarray, t: np.ndarray, text: np.ndarray, workers: int = 1,
            return_stages: bool = False, drop=None, checkpoint=None, image=None):
    """latent [B,C_in,F,H_z,W_z], t [B] or [B,L], text [B,Lt,4096] (and optionally CLIP image tokens
    [B,Li,image_dim]) -> velocity [B,C_out,F,H_z,W_z].

    cfg carries the geometry (dim, num_heads, num_layers, eps, rope split/theta, freq_dim, out_channels).
    weights: dict name -> array, or an object with .f64(name).  drop(prefix) is called after each block
    so lazily generated weights can be released.  checkpoint, if given, has load() -> (next_block, x) or
    None and save(next_block, x): a long run resumes from the token stream saved after its last finished
    block (it changes no arithmetic).
    """
    w = weights
    latent = np.asarray(latent, dtype=np.float64)
    b, _, f, hz, wz = latent.shape
    fp, hp, wp = token_grid(f, hz, wz, cfg.patch)
    x = patch_embed(latent, _arr(w, "patch_embedding.weight"), _arr(w, "patch_embedding.bias"))
    temb, tproj = time_embed(np.asarray(t, dtype=np.float64), w, cfg.freq_dim)
    ctx, n_img = _context(cfg, w, text, image)
    ang = rope_angles(fp, hp, wp, cfg.head_dim, cfg.rope_dims, cfg.rope_theta)
    stages = {"x0": x, "temb": temb, "tproj": tproj, "ctx": ctx, "ang": ang}
    start = 0
    if checkpoint is not None:
        saved = checkpoint.load()
        if saved is not None:
            start, x = saved
    for kb in range(start, cfg.num_layers):
        x = block_forward(x, ctx, tproj, ang, w, f"blocks.{kb}.", cfg.num_heads, cfg.eps, workers, n_img)
        if checkpoint is not None and kb + 1 < cfg.num_layers:
            checkpoint.save(kb + 1, x)
        if drop is not None:
            drop(f"blocks.{kb}.")
    z = head_forward(x, temb, w, cfg.eps)
    out = unpatchify(z, f, hz, wz, cfg.out_channels, cfg.patch)
    if return_stages:
        stages.update({"x_final": x, "z": z})
        return out, stages
    return out


def forward_rows(cfg, weights, latent: np.ndarray, t: np.ndarray, text: np.ndarray, rows, workers: int = 1,
                 image=None):
    """The forward's outputs of the token rows `rows` (same for every batch element), for a stack whose
    last block is the only one: z [B, len(rows), pt*ph*pw*C_out], the proj_out values of those tokens
    (unpatchify scatters token n's values to out[b, c, f, 2h+i, 2w+j]).

    Everything before the block runs on all tokens; the block runs through block_forward_rows; the
    head is per token.
    """
    if cfg.num_layers != 1:
        raise ValueError("forward_rows evaluates one-block stacks")
    w = weights
    rows = np.asarray(rows, dtype=np.int64)
    latent = np.asarray(latent, dtype=np.float64)
    b, _, f, hz, wz = latent.shape
    fp, hp, wp = token_grid(f, hz, wz, cfg.patch)
    x = patch_embed(latent, _arr(w, "patch_embedding.weight"), _arr(w, "patch_embedding.bias"))
    temb, tproj = time_embed(np.asarray(t, dtype=np.float64), w, cfg.freq_dim)
    ctx, n_img = _context(cfg, w, text, image)
    ang = rope_angles(fp, hp, wp, cfg.head_dim, cfg.rope_dims, cfg.rope_theta)
    xr = block_forward_rows(x, ctx, tproj, ang, w, "blocks.0.", cfg.num_heads, rows, cfg.eps, workers, n_img)
    del x
    return head_forward(xr, temb if temb.ndim == 2 else temb[:, rows], w, cfg.eps)


# ---------------------------------------------------------------------------------------------
# Denoising step around the forward [W21 6.3 hand-worked example, 7 inference: Euler update, CFG]
# ---------------------------------------------------------------------------------------------


def flow_noisy(z, eps, sigma):
    """The noised latent at noise level sigma: (1 - sigma) z + sigma eps."""
    return (1.0 - sigma) * np.asarray(z, dtype=np.float64) + sigma * np.asarray(eps, dtype=np.float64)


def flow_velocity(z, eps):
    """The velocity the DiT is trained to predict: eps - z (constant along the straight path)."""
    return np.asarray(eps, dtype=np.float64) - np.asarray(z, dtype=np.float64)


def cfg_combine(v_cond, v_uncond, scale):
    """Classifier-free guidance: v_u + s (v_c - v_u)."""
    v_u = np.asarray(v_uncond, dtype=np.float64)
    return v_u + scale * (np.asarray(v_cond, dtype=np.float64) - v_u)


def euler_step(x, v, sigma, sigma_next):
    """One Euler step of the flow ODE from sigma to sigma_next: x + (sigma_next - sigma) v."""
    return np.asarray(x, dtype=np.float64) + (sigma_next - sigma) * np.asarray(v, dtype=np.float64)


def denoise_step(cfg, weights, latent: np.ndarray, t, text_pair: np.ndarray, scale: float, sigma: float,
                 sigma_next: float, workers: int = 1, image=None):
    """One guided denoising step: the batch-2 forward of the same latent [1, C_in, F, H_z, W_z] under the
    conditional and the unconditional text (text_pair [2, Lt, 4096], conditional first; t [1] or [1, L]),
    CFG-combined and Euler-stepped.  The first C_out channels of the latent are the noisy sample x;
    returns x + (sigma_next - sigma) (v_u + s (v_c - v_u)) [1, C_out, F, H_z, W_z]."""
    latent = np.asarray(latent, dtype=np.float64)
    lat2 = np.concatenate([latent, latent], axis=0)
    t = np.asarray(t, dtype=np.float64)
    t2 = np.concatenate([t, t], axis=0)
    img2 = None if image is None else np.concatenate([image, image], axis=0)
    v = forward(cfg, weights, lat2, t2, text_pair, workers=workers, image=img2)
    x = latent[:, :cfg.out_channels]
    return euler_step(x, cfg_combine(v[:1], v[1:], scale), sigma, sigma_next)
