"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only).

Each test checks the oracle against something other than itself: numbers printed on the pages
(tests/golden/printed_facts.json, each entry with its citation), closed forms, invariants, brute force
on tiny inputs, or an independent library routine (torch CPU float64).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import wan_oracle as O
from wan_inputs import Weights, draw_inputs, get_config, param_count

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "printed_facts.json")))


def tiny_cfg(**kw):
    base = dict(dim=64, num_heads=2, head_dim=32, ffn_dim=96, num_layers=1, text_len=7, frames=3, height=4,
                width=6, batch=1, in_channels=4, out_channels=3, text_dim=16, freq_dim=16, rope_dims=(12, 10, 10),
                dtype="f32")
    base.update(kw)
    return get_config(1).replace(**base)


# ------------------------------------------------------------------------------------------------
# P-1 / P-2 / P-3: shapes and counts printed on the pages
# ------------------------------------------------------------------------------------------------


def test_printed_latent_shapes():
    for e in GOLDEN["vae_latents"]:
        if "rgb" in e:
            b, _, t, h, w = e["rgb"]
            stride = e.get("spatial_stride", 8)
            shp = O.vae_latent_shape(b, t, h, w, channels=e["latent"][1], s_stride=stride)
            assert list(shp) == e["latent"], e["cite"]
            if "rgb_elements" in e:
                assert int(np.prod(e["rgb"])) == e["rgb_elements"]
            if "latent_elements" in e:
                assert int(np.prod(shp)) == e["latent_elements"], e["cite"]
        else:
            shp = O.vae_latent_shape(1, e["frames"], 64, 64)
            assert shp[2] == e["latent_frames"], e["cite"]
    # frame counts that are not 4n+1 are rejected rather than silently floored
    with pytest.raises(ValueError):
        O.vae_latent_shape(1, 80, 480, 832)


def test_printed_token_counts():
    for e in GOLDEN["token_counts"]:
        f, h, w = e["latent_fhw"]
        assert O.num_tokens(f, h, w) == e["tokens"], e["cite"]
        if "per_frame" in e:
            assert O.num_tokens(1, h, w) == e["per_frame"], e["cite"]
    # the five workloads
    for cid, want in {1: 320, 2: 32760, 3: 7920, 4: 27280, 5: 75600}.items():
        c = get_config(cid)
        assert O.num_tokens(c.frames, c.height, c.width) == want


def test_printed_intermediate_shapes_1p3b():
    g = GOLDEN["intermediate_shapes_1p3b"]
    cfg = get_config(2).replace(batch=1, num_layers=0)
    w = Weights(cfg)
    rng = np.random.default_rng(0)
    lat = rng.standard_normal(cfg.latent_shape)
    x = O.patch_embed(lat, w.f64("patch_embedding.weight"), w.f64("patch_embedding.bias"))
    fp, hp, wp = O.token_grid(cfg.frames, cfg.height, cfg.width)
    assert [1, cfg.dim, fp, hp, wp] == g["patch_embedding"]
    assert list(x.shape) == g["tokens"]
    temb, tproj = O.time_embed(np.array([500.0]), w, cfg.freq_dim)
    assert list(temb.shape) == g["temb"]
    assert [1, int(np.prod(tproj.shape[1:]))] == g["timestep_proj"]
    assert list(tproj.shape) == g["timestep_proj_unflat"]
    ctx = O.text_embed(rng.standard_normal((1, 226, 4096)), w)
    assert list(ctx.shape) == g["ctx"]
    ang = O.rope_angles(fp, hp, wp)
    assert [1, 1] + list(ang.shape) == g["rope"]


def test_param_count_matches_model_sizes():
    """P-4: the block structure read from the pages gives the printed model sizes."""
    for e in GOLDEN["model_sizes"]:
        cid = 5 if e["dim"] == 5120 else 4
        c = get_config(cid)
        assert (c.dim, c.num_layers, c.num_heads) == (e["dim"], e["layers"], e["heads"])
        n = param_count(c)
        assert abs(n - e["params_approx"]) / e["params_approx"] < 0.03, (e["name"], n)
    # a three-matrix (gated) FFN would miss the 14B figure by more than 10%
    c = get_config(5)
    extra = c.num_layers * c.dim * c.ffn_dim
    assert (param_count(c) + extra - 14e9) / 14e9 > 0.10


# ------------------------------------------------------------------------------------------------
# P-5 / P-6: patchify, patch embedding, unpatchify
# ------------------------------------------------------------------------------------------------


def test_patchify_unpatchify_roundtrip_bitexact():
    rng = np.random.default_rng(1)
    for shape in [(1, 16, 5, 16, 16), (2, 3, 2, 6, 10), (1, 48, 3, 4, 8)]:
        x = rng.standard_normal(shape).astype(np.float32)
        p = O.patchify(x)
        b, l, k = p.shape
        c = shape[1]
        assert l == O.num_tokens(*shape[2:]) and k == 4 * c
        # conv-weight order (channel slowest) -> proj_out order (channel fastest)
        z = p.reshape(b, l, c, 4).transpose(0, 1, 3, 2).reshape(b, l, 4 * c)
        y = O.unpatchify(z, shape[2], shape[3], shape[4], c)
        assert y.dtype == x.dtype and np.array_equal(y, x)


def test_patch_embed_equals_direct_conv3d_loops():
    rng = np.random.default_rng(2)
    b, c, f, h, w, d = 2, 3, 2, 4, 6, 5
    x = rng.standard_normal((b, c, f, h, w))
    wt = rng.standard_normal((d, c, 1, 2, 2))
    bias = rng.standard_normal(d)
    got = O.patch_embed(x, wt, bias)
    fp, hp, wp = f, h // 2, w // 2
    ref = np.zeros((b, d, fp, hp, wp))
    for bi in range(b):
        for o in range(d):
            for ff in range(fp):
                for hh in range(hp):
                    for ww in range(wp):
                        s = bias[o]
                        for ci in range(c):
                            for i in range(2):
                                for j in range(2):
                                    s += wt[o, ci, 0, i, j] * x[bi, ci, ff, 2 * hh + i, 2 * ww + j]
                        ref[bi, o, ff, hh, ww] = s
    ref_tok = ref.reshape(b, d, -1).transpose(0, 2, 1)      # flatten(2).transpose(1,2)
    assert np.abs(got - ref_tok).max() <= 1e-12 * np.abs(ref_tok).max()


def test_patch_embed_equals_torch_conv3d():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 16, 5, 16, 16))
    wt = rng.standard_normal((32, 16, 1, 2, 2))
    bias = rng.standard_normal(32)
    ref = F.conv3d(torch.from_numpy(x), torch.from_numpy(wt), torch.from_numpy(bias), stride=(1, 2, 2))
    ref = ref.flatten(2).transpose(1, 2).numpy()
    got = O.patch_embed(x, wt, bias)
    assert np.abs(got - ref).max() < 1e-12 * np.abs(ref).max()


def test_unpatchify_index_map():
    """out[b,c,f,2h+i,2w+j] = z[b, n(f,h,w), (2i+j)*C_out + c] with n = (f*H'+h)*W'+w."""
    b, c, f, h, w = 2, 3, 2, 4, 6
    hp, wp = h // 2, w // 2
    z = np.arange(b * f * hp * wp * 4 * c, dtype=np.int64).reshape(b, f * hp * wp, 4 * c)
    out = O.unpatchify(z, f, h, w, c)
    for bi in range(b):
        for ci in range(c):
            for ff in range(f):
                for yy in range(h):
                    for xx in range(w):
                        n = (ff * hp + yy // 2) * wp + xx // 2
                        k = (2 * (yy % 2) + (xx % 2)) * c + ci
                        assert out[bi, ci, ff, yy, xx] == z[bi, n, k]


# ------------------------------------------------------------------------------------------------
# P-7: timestep sinusoid; activations
# ------------------------------------------------------------------------------------------------


def test_sinusoid_closed_forms():
    s0 = O.sinusoid(np.array([0.0]))
    assert np.array_equal(s0[0], np.concatenate([np.ones(128), np.zeros(128)]))
    t = np.array([0.5, 1.0, 37.25, 500.0, 999.9])
    s = O.sinusoid(t)
    assert s.shape == (5, 256)
    assert np.allclose((s * s).sum(-1), 128.0, rtol=0, atol=1e-12)
    # frequency index 64 is 10000^(-1/2) = 1/100: at t = 100 the angle is exactly 1 rad
    s100 = O.sinusoid(np.array([100.0]))[0]
    assert abs(s100[64] - math.cos(1.0)) < 1e-14 and abs(s100[128 + 64] - math.sin(1.0)) < 1e-14
    # frequency index 0 is 1: angle = t
    assert abs(s100[0] - math.cos(100.0)) < 1e-12


def test_gelu_tanh_and_silu_against_torch():
    u = np.linspace(-8, 8, 2001)
    ref = F.gelu(torch.from_numpy(u), approximate="tanh").numpy()
    assert np.abs(O.gelu_tanh(u) - ref).max() < 1e-14
    exact = F.gelu(torch.from_numpy(u)).numpy()      # erf form
    assert np.abs(O.gelu_tanh(u) - exact).max() < 1e-3
    assert O.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert np.abs(O.silu(u) - F.silu(torch.from_numpy(u)).numpy()).max() < 1e-14


# ------------------------------------------------------------------------------------------------
# P-8: norms
# ------------------------------------------------------------------------------------------------


def test_layer_norm_invariants_and_torch():
    rng = np.random.default_rng(4)
    u = rng.standard_normal((7, 1536)) * 3.0 + 1.5
    eps = 1e-6
    y = O.layer_norm(u, eps)
    var = u.var(axis=-1)
    assert np.abs(y.mean(-1)).max() < 1e-13
    assert np.allclose(y.var(-1), var / (var + eps), rtol=1e-12)
    g, b = rng.uniform(0.5, 1.5, 1536), rng.standard_normal(1536) * 0.02
    ref = F.layer_norm(torch.from_numpy(u), (1536,), torch.from_numpy(g), torch.from_numpy(b), eps).numpy()
    assert np.abs(O.layer_norm(u, eps, g, b) - ref).max() < 1e-12


def test_rms_norm_invariants_and_torch():
    rng = np.random.default_rng(5)
    u = rng.standard_normal((5, 3072)) * 0.1
    eps = 1e-6
    y = O.rms_norm(u, eps)
    m = (u * u).mean(-1)
    assert np.allclose((y * y).mean(-1), m / (m + eps), rtol=1e-12)
    g = rng.uniform(0.5, 1.5, 3072)
    ref = F.rms_norm(torch.from_numpy(u), (3072,), torch.from_numpy(g), eps).numpy()
    assert np.abs(O.rms_norm(u, eps, g) - ref).max() < 1e-12


# ------------------------------------------------------------------------------------------------
# P-9: 3D RoPE
# ------------------------------------------------------------------------------------------------


def test_rope_rotation_algebra():
    rng = np.random.default_rng(6)
    fp, hp, wp = 3, 4, 5
    ang = O.rope_angles(fp, hp, wp)
    l = fp * hp * wp
    assert ang.shape == (l, 64)
    u = rng.standard_normal((l, 2, 128))
    r = O.apply_rope(u, ang)
    pair = lambda a: a[..., 0::2] ** 2 + a[..., 1::2] ** 2  # noqa: E731
    assert np.allclose(pair(r), pair(u), rtol=1e-14)
    assert np.array_equal(r[0], u[0])                       # token (0,0,0): identity
    # R_a R_b = R_{a+b}
    ang2 = rng.uniform(-3, 3, ang.shape)
    assert np.allclose(O.apply_rope(O.apply_rope(u, ang), ang2), O.apply_rope(u, ang + ang2), atol=1e-13)
    # against complex multiplication of adjacent pairs (x0 + i x1) * e^{i phi}
    uc = torch.view_as_complex(torch.from_numpy(u).reshape(l, 2, 64, 2).contiguous())
    rc = uc * torch.polar(torch.ones(l, 1, 64, dtype=torch.float64), torch.from_numpy(ang)[:, None, :])
    assert np.abs(torch.view_as_real(rc).reshape(l, 2, 128).numpy() - r).max() < 1e-13


def test_rope_axis_split_and_relative_positions():
    fp, hp, wp = 4, 3, 5
    ang = O.rope_angles(fp, hp, wp)
    tok = lambda f, h, w: (f * hp + h) * wp + w  # noqa: E731
    # moving along w changes only the last 21 pairs, along h only the middle 21, along f only the first 22
    assert np.all(ang[tok(0, 0, 3), :43] == 0) and np.all(ang[tok(0, 0, 3), 43:] != 0)
    assert np.all(ang[tok(0, 2, 0), :22] == 0) and np.all(ang[tok(0, 2, 0), 22:43] != 0) \
        and np.all(ang[tok(0, 2, 0), 43:] == 0)
    assert np.all(ang[tok(3, 0, 0), :22] != 0) and np.all(ang[tok(3, 0, 0), 22:] == 0)
    # frequencies: first pair of every axis has frequency 1 (angle = position)
    assert ang[tok(3, 2, 4), 0] == 3 and ang[tok(3, 2, 4), 22] == 2 and ang[tok(3, 2, 4), 43] == 4
    # second t pair uses theta^(-2/44)
    assert abs(ang[tok(1, 0, 0), 1] - 1e4 ** (-2 / 44)) < 1e-15
    # scores q_i . k_j depend only on position differences: shift every f by +1
    rng = np.random.default_rng(7)
    q = rng.standard_normal((fp * hp * wp, 128))
    k = rng.standard_normal((fp * hp * wp, 128))
    big = O.rope_angles(fp + 1, hp, wp)
    shifted = big[hp * wp:]
    s1 = O.apply_rope(q, ang) @ O.apply_rope(k, ang).T
    s2 = O.apply_rope(q, shifted) @ O.apply_rope(k, shifted).T
    assert np.allclose(s1, s2, atol=1e-11)


# ------------------------------------------------------------------------------------------------
# P-11 / P-12: attention
# ------------------------------------------------------------------------------------------------


def test_attention_brute_force_tiny():
    rng = np.random.default_rng(8)
    for lq, lk in [(1, 1), (3, 8), (8, 5)]:
        q, k, v = rng.standard_normal((lq, 2, 4)), rng.standard_normal((lk, 2, 4)), rng.standard_normal((lk, 2, 3))
        got = O.attention(q, k, v)
        ref = np.zeros((lq, 2, 3))
        for h in range(2):
            for i in range(lq):
                e = [math.exp(sum(q[i, h, c] * k[j, h, c] for c in range(4)) / 2.0) for j in range(lk)]
                z = sum(e)
                for c in range(3):
                    ref[i, h, c] = sum(e[j] * v[j, h, c] for j in range(lk)) / z
        assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_attention_special_cases_and_torch():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((50, 3, 128)) * 4
    k_const = np.repeat(rng.standard_normal((1, 3, 128)), 40, axis=0)
    v = rng.standard_normal((40, 3, 128))
    assert np.allclose(O.attention(q, k_const, v), v.mean(0, keepdims=True), atol=1e-13)
    one = O.attention(q, k_const[:1], v[:1])
    assert np.allclose(one, np.broadcast_to(v[:1], one.shape), atol=1e-14)
    k = rng.standard_normal((333, 3, 128))
    v = rng.standard_normal((333, 3, 128))
    got = O.attention(q, k, v, chunk=16)
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(a).transpose(0, 1) for a in (q, k, v)))
    assert np.abs(got - ref.transpose(0, 1).numpy()).max() < 1e-12


# ------------------------------------------------------------------------------------------------
# P-10 / P-12 / P-13: block structure
# ------------------------------------------------------------------------------------------------


def _block_setup(cfg, seed=10):
    w = Weights(cfg)
    rng = np.random.default_rng(seed)
    l = cfg.tokens
    x = rng.standard_normal((cfg.batch, l, cfg.dim))
    ctx = rng.standard_normal((cfg.batch, cfg.text_len, cfg.dim))
    tproj = rng.standard_normal((cfg.batch, 6, cfg.dim)) * 0.3
    ang = O.rope_angles(cfg.post_f, cfg.post_h, cfg.post_w, cfg.head_dim, cfg.rope_dims)
    return w, x, ctx, tproj, ang


def _run_block(cfg, w, x, ctx, tproj, ang):
    return O.block_forward(x, ctx, tproj, ang, w, "blocks.0.", cfg.num_heads, cfg.eps)


def test_zero_gates_and_zero_cross_out_give_identity():
    cfg = tiny_cfg(batch=2)
    w, x, ctx, tproj, ang = _block_setup(cfg)
    d = cfg.dim
    tab = w.f64("blocks.0.scale_shift_table").copy()
    tproj[:, 2] = -tab[0, 2]
    tproj[:, 5] = -tab[0, 5]
    w.set("blocks.0.attn2.to_out.weight", np.zeros((d, d)))
    w.set("blocks.0.attn2.to_out.bias", np.zeros(d))
    y = _run_block(cfg, w, x, ctx, tproj, ang)
    assert np.array_equal(y, x)


def test_zero_gates_remove_self_attention_and_ffn():
    cfg = tiny_cfg()
    w, x, ctx, tproj, ang = _block_setup(cfg)
    tab = w.f64("blocks.0.scale_shift_table")
    tproj[:, 2] = -tab[0, 2]
    tproj[:, 5] = -tab[0, 5]
    y1 = _run_block(cfg, w, x, ctx, tproj, ang)
    rng = np.random.default_rng(11)
    for n in ("attn1.to_q.weight", "attn1.to_v.weight", "attn1.to_out.weight", "ffn.proj_in.weight",
              "ffn.proj_out.bias"):
        w.set("blocks.0." + n, rng.standard_normal(w.shape("blocks.0." + n)))
    y2 = _run_block(cfg, w, x, ctx, tproj, ang)
    assert np.array_equal(y1, y2)
    assert not np.allclose(y1, x)        # the ungated cross-attention residual still acts


def test_text_token_permutation_invariance():
    cfg = tiny_cfg()
    w, x, ctx, tproj, ang = _block_setup(cfg)
    perm = np.random.default_rng(12).permutation(cfg.text_len)
    y1 = _run_block(cfg, w, x, ctx, tproj, ang)
    y2 = _run_block(cfg, w, x, ctx[:, perm], tproj, ang)
    assert np.allclose(y1, y2, rtol=0, atol=1e-12)


def test_duplicated_batch_elements_match():
    cfg = tiny_cfg(batch=2)
    w = Weights(cfg)
    lat, t, txt = draw_inputs(cfg)
    lat, t, txt = lat.f64(), t.f64(), txt.f64()
    lat[1], t[1], txt[1] = lat[0], t[0], txt[0]
    out = O.forward(cfg, w, lat, t, txt)
    assert np.allclose(out[0], out[1], rtol=0, atol=1e-12)


def test_block_against_torch_library_composition():
    """The block assembled from torch's own layer_norm / rms_norm / linear / SDPA / gelu in float64."""
    cfg = tiny_cfg(batch=2)
    w, x, ctx, tproj, ang = _block_setup(cfg)
    got = _run_block(cfg, w, x, ctx, tproj, ang)
    T = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))  # noqa: E731
    W = lambda n: T(w.f64("blocks.0." + n))  # noqa: E731
    d, nh = cfg.dim, cfg.num_heads
    hd = d // nh
    xt = T(x)
    mod = (W("scale_shift_table") + T(tproj)).chunk(6, dim=1)
    sh1, sc1, g1, sh2, sc2, g2 = mod
    cos = T(np.cos(ang)).repeat_interleave(2, -1)
    sin = T(np.sin(ang)).repeat_interleave(2, -1)

    def rope(u):  # u [B, H, L, hd]; rotate-half written for adjacent pairs
        rot = torch.stack([-u[..., 1::2], u[..., 0::2]], dim=-1).flatten(-2)
        return u * cos + rot * sin

    def heads(u):
        return u.unflatten(-1, (nh, hd)).transpose(1, 2)

    y = F.layer_norm(xt, (d,), eps=cfg.eps) * (1 + sc1) + sh1
    q = F.rms_norm(F.linear(y, W("attn1.to_q.weight"), W("attn1.to_q.bias")), (d,), W("attn1.norm_q.weight"), cfg.eps)
    k = F.rms_norm(F.linear(y, W("attn1.to_k.weight"), W("attn1.to_k.bias")), (d,), W("attn1.norm_k.weight"), cfg.eps)
    v = F.linear(y, W("attn1.to_v.weight"), W("attn1.to_v.bias"))
    a = F.scaled_dot_product_attention(rope(heads(q)), rope(heads(k)), heads(v)).transpose(1, 2).flatten(2)
    xt = xt + F.linear(a, W("attn1.to_out.weight"), W("attn1.to_out.bias")) * g1
    y2 = F.layer_norm(xt, (d,), W("norm2.weight"), W("norm2.bias"), cfg.eps)
    ct = T(ctx)
    q2 = F.rms_norm(F.linear(y2, W("attn2.to_q.weight"), W("attn2.to_q.bias")), (d,), W("attn2.norm_q.weight"), cfg.eps)
    k2 = F.rms_norm(F.linear(ct, W("attn2.to_k.weight"), W("attn2.to_k.bias")), (d,), W("attn2.norm_k.weight"), cfg.eps)
    v2 = F.linear(ct, W("attn2.to_v.weight"), W("attn2.to_v.bias"))
    a2 = F.scaled_dot_product_attention(heads(q2), heads(k2), heads(v2)).transpose(1, 2).flatten(2)
    xt = xt + F.linear(a2, W("attn2.to_out.weight"), W("attn2.to_out.bias"))
    y3 = F.layer_norm(xt, (d,), eps=cfg.eps) * (1 + sc2) + sh2
    h = F.gelu(F.linear(y3, W("ffn.proj_in.weight"), W("ffn.proj_in.bias")), approximate="tanh")
    xt = xt + F.linear(h, W("ffn.proj_out.weight"), W("ffn.proj_out.bias")) * g2
    assert np.abs(got - xt.numpy()).max() < 1e-11


def test_per_token_modulation_matches_broadcast():
    """A per-token timestep projection with equal rows equals the per-sample one."""
    cfg = tiny_cfg()
    w, x, ctx, tproj, ang = _block_setup(cfg)
    tp_tok = np.repeat(tproj[:, None], cfg.tokens, axis=1)
    y1 = _run_block(cfg, w, x, ctx, tproj, ang)
    y2 = _run_block(cfg, w, x, ctx, tp_tok, ang)
    assert np.allclose(y1, y2, rtol=0, atol=1e-13)


def test_head_scale_minus_one_gives_constant_tokens():
    """(1 + scale) = 0 makes norm_out drop out: every token maps to shift @ W_out^T + b_out."""
    cfg = tiny_cfg()
    w = Weights(cfg)
    rng = np.random.default_rng(13)
    x = rng.standard_normal((1, cfg.tokens, cfg.dim))
    temb = rng.standard_normal((1, cfg.dim))
    tab = w.f64("scale_shift_table").copy()
    temb_fix = -1.0 - tab[0, 1]
    z = O.head_forward(x, temb_fix[None], w)
    assert np.allclose(z, z[:, :1], rtol=0, atol=1e-13)


def test_embedder_bias_only_paths():
    """Zero first-layer weights and biases make SiLU / GELU output zero: the second bias passes through."""
    cfg = tiny_cfg()
    w = Weights(cfg)
    d = cfg.dim
    for n, shp in (("time_embedder.linear_1", (d, cfg.freq_dim)), ("text_embedder.linear_1", (d, cfg.text_dim))):
        w.set(n + ".weight", np.zeros(shp))
        w.set(n + ".bias", np.zeros(d))
    temb, tproj = O.time_embed(np.array([123.0]), w, cfg.freq_dim)
    assert np.array_equal(temb[0], w.f64("time_embedder.linear_2.bias"))
    b_tp = w.f64("time_proj.bias").reshape(6, d)
    w_tp = w.f64("time_proj.weight")
    assert np.allclose(tproj[0], (w_tp @ O.silu(temb[0]) + w.f64("time_proj.bias")).reshape(6, d))
    assert tproj.shape == (1, 6, d) and not np.allclose(tproj[0], b_tp)
    ctx = O.text_embed(np.random.default_rng(0).standard_normal((1, 5, cfg.text_dim)), w)
    assert np.array_equal(ctx[0], np.broadcast_to(w.f64("text_embedder.linear_2.bias"), (5, d)))


# ------------------------------------------------------------------------------------------------
# Time and text embedders against torch's own layers, with non-zero weights (the Linear / SiLU /
# GELU composition is the reading; a dropped or misplaced activation changes the result)
# ------------------------------------------------------------------------------------------------


def _rand_weights(cfg, names, seed):
    w = Weights(cfg)
    rng = np.random.default_rng(seed)
    for n in names:
        w.set(n, rng.standard_normal(w.shape(n)) * 0.3)
    return w


def test_time_embed_against_torch_composition():
    cfg = tiny_cfg()
    names = [f"{m}.{k}" for m in ("time_embedder.linear_1", "time_embedder.linear_2", "time_proj")
             for k in ("weight", "bias")]
    w = _rand_weights(cfg, names, 21)
    t = np.array([0.0, 3.5, 500.0, 999.0])
    temb, tproj = O.time_embed(t, w, cfg.freq_dim)
    T = lambda n: torch.from_numpy(w.f64(n))  # noqa: E731
    half = cfg.freq_dim // 2
    freqs = torch.exp(-math.log(10000.0) * torch.arange(half, dtype=torch.float64) / half)
    arg = torch.from_numpy(t)[:, None] * freqs[None]
    s = torch.cat([torch.cos(arg), torch.sin(arg)], dim=-1)
    h = F.silu(F.linear(s, T("time_embedder.linear_1.weight"), T("time_embedder.linear_1.bias")))
    te = F.linear(h, T("time_embedder.linear_2.weight"), T("time_embedder.linear_2.bias"))
    tp = F.linear(F.silu(te), T("time_proj.weight"), T("time_proj.bias")).unflatten(1, (6, cfg.dim))
    assert np.abs(temb - te.numpy()).max() <= 1e-12 * max(1.0, np.abs(temb).max())
    assert np.abs(tproj - tp.numpy()).max() <= 1e-12 * max(1.0, np.abs(tproj).max())
    # without the inner SiLU, or without the one before time_proj, the values differ clearly
    te_nosilu = F.linear(F.linear(s, T("time_embedder.linear_1.weight"), T("time_embedder.linear_1.bias")),
                         T("time_embedder.linear_2.weight"), T("time_embedder.linear_2.bias"))
    assert np.abs(temb - te_nosilu.numpy()).max() > 1e-3


def test_text_embed_against_torch_composition():
    cfg = tiny_cfg()
    names = [f"text_embedder.linear_{i}.{k}" for i in (1, 2) for k in ("weight", "bias")]
    w = _rand_weights(cfg, names, 22)
    e = np.random.default_rng(23).standard_normal((2, 5, cfg.text_dim))
    got = O.text_embed(e, w)
    T = lambda n: torch.from_numpy(w.f64(n))  # noqa: E731
    h = F.gelu(F.linear(torch.from_numpy(e), T("text_embedder.linear_1.weight"), T("text_embedder.linear_1.bias")),
               approximate="tanh")
    ref = F.linear(h, T("text_embedder.linear_2.weight"), T("text_embedder.linear_2.bias")).numpy()
    assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())
    h_erf = F.gelu(F.linear(torch.from_numpy(e), T("text_embedder.linear_1.weight"), T("text_embedder.linear_1.bias")))
    ref_erf = F.linear(h_erf, T("text_embedder.linear_2.weight"), T("text_embedder.linear_2.bias")).numpy()
    assert np.abs(got - ref_erf).max() > 1e-6                     # the tanh form, not the erf one


# ------------------------------------------------------------------------------------------------
# Per-token timesteps through the whole forward (time MLP, modulation and head per token)
# ------------------------------------------------------------------------------------------------


def test_forward_per_token_timesteps_equal_broadcast():
    cfg = tiny_cfg(batch=2)
    w = Weights(cfg)
    lat, _, txt = draw_inputs(cfg)
    t_b = np.array([500.0, 137.0])
    out_b = O.forward(cfg, w, lat.f64(), t_b, txt.f64())
    t_tok = np.repeat(t_b[:, None], cfg.tokens, axis=1)
    out_tok = O.forward(cfg.replace(per_token_t=True), w, lat.f64(), t_tok, txt.f64())
    assert np.abs(out_tok - out_b).max() <= 1e-12 * np.abs(out_b).max()
    # and a token's own timestep matters: changing one token's t changes that token's output
    t_tok[0, 5] = 900.0
    out_one = O.forward(cfg.replace(per_token_t=True), w, lat.f64(), t_tok, txt.f64())
    assert np.abs(out_one - out_b).max() > 1e-3


def test_head_per_token_equal_rows_match_per_sample():
    cfg = tiny_cfg()
    w = Weights(cfg)
    rng = np.random.default_rng(24)
    x = rng.standard_normal((2, cfg.tokens, cfg.dim))
    temb = rng.standard_normal((2, cfg.dim))
    z2 = O.head_forward(x, temb, w)
    z3 = O.head_forward(x, np.repeat(temb[:, None], cfg.tokens, axis=1), w)
    assert np.abs(z3 - z2).max() <= 1e-13 * np.abs(z2).max()


# ------------------------------------------------------------------------------------------------
# Denoising step: the hand-worked flow-matching example and the CFG combine
# ------------------------------------------------------------------------------------------------


def test_flow_matching_worked_example():
    e = GOLDEN["flow_matching_example"]
    z, eps, sigma = e["z"], e["eps"], e["sigma"]
    x = O.flow_noisy(z, eps, sigma)
    assert x == e["x_sigma"]
    v = O.flow_velocity(z, eps)
    assert v == e["v_target"]
    assert (7.0 - v) ** 2 == 1.0                         # the printed squared error of a prediction of 7
    x1 = O.euler_step(x, v, sigma, 0.5)
    assert x1 == e["step_to_0p5"]
    assert O.euler_step(x1, v, 0.5, 0.0) == e["step_to_0"] == z   # the straight path lands on the data
    # stepping with the exact velocity from any sigma reaches the same point
    for s0, s1 in [(1.0, 0.25), (0.9, 0.3)]:
        assert abs(O.euler_step(O.flow_noisy(z, eps, s0), v, s0, s1) - O.flow_noisy(z, eps, s1)) < 1e-14


def test_cfg_combine_special_cases():
    rng = np.random.default_rng(25)
    vc, vu = rng.standard_normal((2, 3, 4, 5))
    assert np.allclose(O.cfg_combine(vc, vu, 1.0), vc, rtol=0, atol=1e-15)   # v_u + (v_c - v_u): one rounding
    assert np.array_equal(O.cfg_combine(vc, vu, 0.0), vu)
    assert np.allclose(O.cfg_combine(vc, vc, 6.0), vc, rtol=0, atol=1e-15)
    s = 6.0
    g = O.cfg_combine(vc, vu, s)
    assert np.allclose(g - vu, s * (vc - vu), rtol=1e-14, atol=1e-14)   # extrapolation along v_c - v_u
    assert np.allclose(O.cfg_combine(vc, vu, 2.0), 2 * vc - vu, rtol=1e-14, atol=1e-14)


def test_denoise_step_is_forward_then_cfg_then_euler():
    cfg = tiny_cfg(batch=2)
    w = Weights(cfg)
    lat, _, txt = draw_inputs(cfg.replace(batch=1))
    text_pair = np.random.default_rng(26).standard_normal((2, cfg.text_len, cfg.text_dim))
    lat1 = lat.f64()
    got = O.denoise_step(cfg, w, lat1, np.array([750.0]), text_pair, 5.0, 0.75, 0.5)
    v = O.forward(cfg, w, np.concatenate([lat1, lat1]), np.array([750.0, 750.0]), text_pair)
    ref = lat1[:, :cfg.out_channels] + (0.5 - 0.75) * (v[1:] + 5.0 * (v[:1] - v[1:]))
    assert np.abs(got - ref).max() <= 1e-13 * np.abs(ref).max()
    # the unconditional text only acts through the guidance: with s = 1 it drops out
    one = O.denoise_step(cfg, w, lat1, np.array([750.0]), text_pair, 1.0, 0.75, 0.5)
    other = text_pair.copy()
    other[1] = 0.0
    assert np.allclose(O.denoise_step(cfg, w, lat1, np.array([750.0]), other, 1.0, 0.75, 0.5), one,
                       rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------------------------
# I2V image branch: projected CLIP tokens first in the context, attended by their own keys/values
# ------------------------------------------------------------------------------------------------


def _i2v_cfg(**kw):
    base = dict(image_len=5, image_dim=12)
    base.update(kw)
    return tiny_cfg(**base)


def test_image_embed_shape_printed():
    e = GOLDEN["i2v_image_tokens"]
    cfg = get_config(3).replace(image_len=e["tokens"], num_layers=0)
    assert (cfg.image_len, cfg.image_dim, cfg.dim) == (e["tokens"], e["image_dim"], e["projected_dim"])
    assert cfg.in_channels == e["latent_channels"]["total"] == sum(
        e["latent_channels"][k] for k in ("noise", "condition", "mask"))
    w = Weights(cfg)
    img = np.random.default_rng(27).standard_normal((1, e["tokens"], e["image_dim"]))
    assert O.image_embed(img, w).shape == (1, e["tokens"], e["projected_dim"])


def test_image_branch_against_torch_composition():
    cfg = _i2v_cfg(batch=2)
    w, x, _, tproj, ang = _block_setup(cfg)
    rng = np.random.default_rng(28)
    ctx = rng.standard_normal((2, cfg.image_len + cfg.text_len, cfg.dim))
    got = O.block_forward(x, ctx, tproj, ang, w, "blocks.0.", cfg.num_heads, cfg.eps, n_img=cfg.image_len)
    # the block without image tokens plus the image attention's contribution, through torch
    T = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))  # noqa: E731
    W = lambda n: T(w.f64("blocks.0." + n))  # noqa: E731
    d, nh = cfg.dim, cfg.num_heads
    hd = d // nh
    heads = lambda u: u.unflatten(-1, (nh, hd)).transpose(1, 2)  # noqa: E731
    y2_fn = lambda xx: F.layer_norm(xx, (d,), W("norm2.weight"), W("norm2.bias"), cfg.eps)  # noqa: E731
    # x after the self-attention step, computed with the oracle's own first half (the text-only block
    # with zero cross output gives it), then the cross step in torch with both key sets
    w0 = Weights(cfg)
    for n in w.names():
        w0.set(n, w.f64(n))
    w0.set("blocks.0.attn2.to_out.weight", np.zeros((d, d)))
    w0.set("blocks.0.attn2.to_out.bias", np.zeros(d))
    w0.set("blocks.0.ffn.proj_out.weight", np.zeros((d, cfg.ffn_dim)))
    w0.set("blocks.0.ffn.proj_out.bias", np.zeros(d))
    x1 = T(O.block_forward(x, ctx[:, cfg.image_len:], tproj, ang, w0, "blocks.0.", nh, cfg.eps))
    y2 = y2_fn(x1)
    q2 = F.rms_norm(F.linear(y2, W("attn2.to_q.weight"), W("attn2.to_q.bias")), (d,), W("attn2.norm_q.weight"), cfg.eps)
    ct = T(ctx)
    img, txt = ct[:, :cfg.image_len], ct[:, cfg.image_len:]
    k2 = F.rms_norm(F.linear(txt, W("attn2.to_k.weight"), W("attn2.to_k.bias")), (d,), W("attn2.norm_k.weight"), cfg.eps)
    v2 = F.linear(txt, W("attn2.to_v.weight"), W("attn2.to_v.bias"))
    ki = F.rms_norm(F.linear(img, W("attn2.add_k_proj.weight"), W("attn2.add_k_proj.bias")), (d,),
                    W("attn2.norm_added_k.weight"), cfg.eps)
    vi = F.linear(img, W("attn2.add_v_proj.weight"), W("attn2.add_v_proj.bias"))
    a2 = (F.scaled_dot_product_attention(heads(q2), heads(k2), heads(v2))
          + F.scaled_dot_product_attention(heads(q2), heads(ki), heads(vi))).transpose(1, 2).flatten(2)
    x2 = x1 + F.linear(a2, W("attn2.to_out.weight"), W("attn2.to_out.bias"))
    mod = (W("scale_shift_table") + T(tproj)).chunk(6, dim=1)
    y3 = F.layer_norm(x2, (d,), eps=cfg.eps) * (1 + mod[4]) + mod[3]
    h = F.gelu(F.linear(y3, W("ffn.proj_in.weight"), W("ffn.proj_in.bias")), approximate="tanh")
    ref = x2 + F.linear(h, W("ffn.proj_out.weight"), W("ffn.proj_out.bias")) * mod[5]
    assert np.abs(got - ref.numpy()).max() < 1e-11


def test_image_branch_constant_keys_add_mean_of_image_values():
    cfg = _i2v_cfg()
    w, x, _, tproj, ang = _block_setup(cfg)
    d = cfg.dim
    w.set("blocks.0.attn2.add_k_proj.weight", np.zeros((d, d)))   # every image key equal
    rng = np.random.default_rng(29)
    ctx = rng.standard_normal((1, cfg.image_len + cfg.text_len, d))
    y2 = rng.standard_normal((1, cfg.tokens, d))
    with_img = O._cross_attention(y2, ctx, w, "blocks.0.", cfg.num_heads, cfg.eps, cfg.image_len, 1)
    text_only = O._cross_attention(y2, ctx[:, cfg.image_len:], w, "blocks.0.", cfg.num_heads, cfg.eps, 0, 1)
    vi = O.linear(ctx[:, :cfg.image_len], w.f64("blocks.0.attn2.add_v_proj.weight"),
                  w.f64("blocks.0.attn2.add_v_proj.bias"))
    assert np.allclose(with_img - text_only, vi.mean(axis=1, keepdims=True), rtol=0, atol=1e-12)


def test_image_tokens_permutation_invariance():
    cfg = _i2v_cfg()
    w, x, _, tproj, ang = _block_setup(cfg)
    rng = np.random.default_rng(30)
    ctx = rng.standard_normal((1, cfg.image_len + cfg.text_len, cfg.dim))
    perm = np.concatenate([rng.permutation(cfg.image_len), cfg.image_len + np.arange(cfg.text_len)])
    y1 = O.block_forward(x, ctx, tproj, ang, w, "blocks.0.", cfg.num_heads, cfg.eps, n_img=cfg.image_len)
    y2 = O.block_forward(x, ctx[:, perm], tproj, ang, w, "blocks.0.", cfg.num_heads, cfg.eps, n_img=cfg.image_len)
    assert np.allclose(y1, y2, rtol=0, atol=1e-12)
    # moving an image token into the text part changes the result (the split is by position)
    y3 = O.block_forward(x, ctx, tproj, ang, w, "blocks.0.", cfg.num_heads, cfg.eps, n_img=cfg.image_len - 1)
    assert np.abs(y3 - y1).max() > 1e-6


# ------------------------------------------------------------------------------------------------
# Row-restricted block and forward (the evaluation of the largest workload on sampled tokens)
# ------------------------------------------------------------------------------------------------


@pytest.mark.parametrize("per_token", [False, True])
def test_block_rows_equal_full_block(per_token):
    cfg = tiny_cfg(batch=2)
    w, x, ctx, tproj, ang = _block_setup(cfg)
    if per_token:
        tproj = np.random.default_rng(31).standard_normal((2, cfg.tokens, 6, cfg.dim)) * 0.3
    full = _run_block(cfg, w, x, ctx, tproj, ang)
    for rows in (np.array([0, 7, 3, cfg.tokens - 1]), np.arange(cfg.tokens)):
        got = O.block_forward_rows(x, ctx, tproj, ang, w, "blocks.0.", cfg.num_heads, rows, cfg.eps)
        assert np.abs(got - full[:, rows]).max() <= 1e-12 * np.abs(full).max()


def test_forward_rows_equal_full_forward():
    cfg = tiny_cfg(batch=1)
    w = Weights(cfg)
    lat, t, txt = draw_inputs(cfg)
    out = O.forward(cfg, w, lat.f64(), t.f64(), txt.f64())
    rows = np.array([1, 9, 12, cfg.tokens - 1])
    z = O.forward_rows(cfg, w, lat.f64(), t.f64(), txt.f64(), rows)
    hp, wp = cfg.post_h, cfg.post_w
    c_out = cfg.out_channels
    for r, n in enumerate(rows):
        f, hh, ww = n // (hp * wp), (n // wp) % hp, n % wp
        for i in range(2):
            for j in range(2):
                ref = out[0, :, f, 2 * hh + i, 2 * ww + j]
                got = z[0, r, (2 * i + j) * c_out:(2 * i + j + 1) * c_out]
                assert np.abs(got - ref).max() <= 1e-12 * np.abs(out).max()
