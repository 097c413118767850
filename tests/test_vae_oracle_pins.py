"""Pins of the fp64 Wan-VAE decoder oracle against what the pages and the mathematics fix (CPU only).

Each test checks the oracle against something other than itself: shapes and module lists printed on the
pages (tests/golden/printed_facts.json, tests/golden/vae_printed_modules.json, each with its citation),
an independent library routine (torch CPU float64 convolutions with the printed causal padding, torch's
nearest-exact interpolation), brute force on tiny inputs, invariants (causality, chunking) and special
cases with a closed form.
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import wan_vae_oracle as V
from wan_inputs.vae import (VaeConfig, VaeWeights, decoder_layout, draw_vae_latent, get_vae_config,
                            vae_weight_spec)

HERE = os.path.dirname(__file__)
FACTS = json.load(open(os.path.join(HERE, "golden", "printed_facts.json")))
MODULES = json.load(open(os.path.join(HERE, "golden", "vae_printed_modules.json")))


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _torch_causal(x, w, b):
    """The printed WanCausalConv3d padding (w_pad, w_pad, h_pad, h_pad, 2 t_pad, 0) with torch's conv3d."""
    kt, kh, kw = w.shape[2:]
    pad = (kw // 2, kw // 2, kh // 2, kh // 2, kt - 1, 0)
    xt = F.pad(torch.from_numpy(x)[None], pad)
    return F.conv3d(xt, torch.from_numpy(w), torch.from_numpy(b))[0].numpy()


# ------------------------------------------------------------------------------------------------
# Printed shapes and module list
# ------------------------------------------------------------------------------------------------
def test_decoded_video_shapes_match_printed_examples():
    """[B,16,F,H,W] -> [B,3,1+4(F-1),8H,8W] for every Wan2.1-VAE example the pages print."""
    n = 0
    for e in FACTS["vae_latents"]:
        if "rgb" not in e or e.get("spatial_stride", 8) != 8:
            continue
        b, c, f, h, w = e["latent"]
        assert c == 16
        cfg = VaeConfig(0, "x", frames=f, height=h, width=w, batch=b)
        assert list(cfg.out_shape) == e["rgb"], e["cite"]
        if "rgb_elements" in e:
            assert int(np.prod(cfg.out_shape)) == e["rgb_elements"]
            assert int(np.prod(cfg.latent_shape)) == e["latent_elements"]
        n += 1
    assert n == 3
    assert get_vae_config(13).out_shape == (1, 3, 33, 352, 640)
    assert get_vae_config(14).out_shape == (1, 3, 81, 480, 832)


def test_weight_list_matches_printed_modules():
    cfg = get_vae_config(14)
    spec = {n: s for n, s, _ in vae_weight_spec(cfg)}
    causal = [n for n, s in spec.items() if n.startswith("decoder.") and n.endswith(".weight") and len(s) == 5]
    assert len(causal) == MODULES["causal_conv3d_count"]
    assert spec["decoder.conv_in.weight"][0] == MODULES["after_conv_in_first_chunk"][1]
    for i, ub in enumerate(MODULES["up_blocks"]):
        p = f"decoder.up_blocks.{i}"
        for j, r in enumerate(ub["resnets"]):
            for conv in ("conv1", "conv2"):
                ci, co, k = r[conv]
                assert spec[f"{p}.resnets.{j}.{conv}.weight"] == (co, ci, *k)
            sc = f"{p}.resnets.{j}.conv_shortcut.weight"
            if r["shortcut"] is None:
                assert sc not in spec
            else:
                ci, co, k = r["shortcut"]
                assert spec[sc] == (co, ci, *k)
        rs = f"{p}.upsamplers.0.resample.1.weight"
        if ub["resample_conv2d"] is None:
            assert rs not in spec
        else:
            ci, co, k = ub["resample_conv2d"]
            assert spec[rs] == (co, ci, *k)
        tc = f"{p}.upsamplers.0.time_conv.weight"
        if ub["time_conv"] is None:
            assert tc not in spec
        else:
            ci, co, k = ub["time_conv"]
            assert spec[tc] == (co, ci, *k)


def test_chunk_shapes_match_printed_comments():
    """A later chunk's shape after each up block: the printed (C, frames) and x2 / x4 / x8 / x8 space."""
    cfg = VaeConfig(0, "shape-walk", frames=2, height=2, width=3)
    P = V.weights_f64(VaeWeights(cfg))
    z = draw_vae_latent(cfg).f64()[0]
    x = V.causal_conv3d(V.denormalize(z, P["latents_mean"], P["latents_std"]), P["post_quant_conv.weight"],
                        P["post_quant_conv.bias"])
    st = V._Stream(P, decoder_layout(cfg), cfg.eps)
    first, later = [], []
    st.chunk(x[:, :1], first)
    st.chunk(x[:, 1:2], later)
    lat = MODULES["latent_after_post_quant"]
    assert first[0][2][0] == MODULES["after_conv_in_first_chunk"][1] and first[0][2][1] == 1
    ends = [e for e in later if e[0] in ("up3d", "up2d")] + [later[-2]]   # up blocks 0-2, then block 3
    assert len(ends) == 4
    for (_, _, shp), want in zip(ends, MODULES["after_up_blocks_later_chunk"]):
        assert shp[0] == want[1] and shp[1] == want[2]
        assert shp[2] * lat[3] == cfg.height * want[3] and shp[3] * lat[4] == cfg.width * want[4]
    assert later[-1][2] == (3, 4, 16, 24)


# ------------------------------------------------------------------------------------------------
# Causal convolution
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("k", [(3, 3, 3), (3, 1, 1), (1, 1, 1), (1, 3, 3)])
def test_causal_conv_matches_torch_with_printed_padding(k):
    x = _rand((5, 4, 6, 7), 1)
    w = _rand((3, 5, *k), 2)
    b = _rand((3,), 3)
    np.testing.assert_allclose(V.causal_conv3d(x, w, b), _torch_causal(x, w, b), rtol=1e-12, atol=1e-12)


def test_causal_conv_brute_force():
    ci, co, T, H, W = 2, 3, 3, 3, 4
    x = _rand((ci, T, H, W), 4)
    w = _rand((co, ci, 3, 3, 3), 5)
    b = _rand((co,), 6)
    ref = np.zeros((co, T, H, W))
    for o in range(co):
        for t in range(T):
            for y in range(H):
                for xx in range(W):
                    s = b[o]
                    for i in range(ci):
                        for a in range(3):
                            for r in range(3):
                                for c in range(3):
                                    tt, yy, xc = t - 2 + a, y - 1 + r, xx - 1 + c
                                    if 0 <= tt < T and 0 <= yy < H and 0 <= xc < W:
                                        s += w[o, i, a, r, c] * x[i, tt, yy, xc]
                    ref[o, t, y, xx] = s
    np.testing.assert_allclose(V.causal_conv3d(x, w, b), ref, rtol=1e-12, atol=1e-12)


def test_causal_conv_is_causal():
    x = _rand((3, 6, 4, 5), 7)
    w = _rand((2, 3, 3, 3, 3), 8)
    b = _rand((2,), 9)
    y = V.causal_conv3d(x, w, b)
    x2 = x.copy()
    x2[:, 3] += 1.0
    y2 = V.causal_conv3d(x2, w, b)
    np.testing.assert_array_equal(y[:, :3], y2[:, :3])          # frames before the change: untouched
    for t in (3, 4, 5):                                          # the kernel reaches two frames back
        assert np.abs(y[:, t] - y2[:, t]).max() > 1e-3


@pytest.mark.parametrize("chunks", [[1, 1, 1, 1, 1, 1], [1, 2, 3], [1, 3, 2], [2, 4], [1, 5], [6]])
def test_cached_chunks_equal_whole_sequence(chunks):
    """The pages' feature cache (last 2 input frames, the previous cache's last frame in front of a
    1-frame chunk) gives the whole-sequence causal convolution for any chunking."""
    x = _rand((3, 6, 4, 5), 10)
    w = _rand((2, 3, 3, 3, 3), 11)
    b = _rand((2,), 12)
    whole = V.causal_conv3d(x, w, b)
    cache, outs, t0 = None, [], 0
    for n in chunks:
        xc = x[:, t0:t0 + n]
        new = V.next_cache(xc, cache)
        outs.append(V.causal_conv3d_step(xc, cache, w, b))
        cache, t0 = new, t0 + n
    np.testing.assert_allclose(np.concatenate(outs, axis=1), whole, rtol=1e-12, atol=1e-12)


def test_conv2d_frames_matches_torch():
    x = _rand((4, 3, 5, 6), 13)
    w = _rand((2, 4, 3, 3), 14)
    b = _rand((2,), 15)
    ref = F.conv2d(torch.from_numpy(x).permute(1, 0, 2, 3), torch.from_numpy(w), torch.from_numpy(b), padding=1)
    np.testing.assert_allclose(V.conv2d_frames(x, w, b), ref.permute(1, 0, 2, 3).numpy(), rtol=1e-12, atol=1e-12)


def test_upsample_matches_torch_nearest_exact():
    x = _rand((3, 2, 5, 7), 16)
    ref = F.interpolate(torch.from_numpy(x), scale_factor=(2.0, 2.0), mode="nearest-exact").numpy()
    np.testing.assert_array_equal(V.upsample_nearest2x(x), ref)


# ------------------------------------------------------------------------------------------------
# Norm, residual block, time upsampling
# ------------------------------------------------------------------------------------------------
def test_rms_norm_closed_forms():
    u = np.array([3.0, 4.0]).reshape(2, 1, 1, 1)
    y = V.rms_norm(u, np.array([1.0, 2.0]), 0.0)
    np.testing.assert_allclose(y.ravel(), [3.0 / np.sqrt(12.5), 8.0 / np.sqrt(12.5)], rtol=1e-15)
    x = _rand((6, 2, 3, 4), 17)
    g = np.ones(6)
    a = V.rms_norm(x, g, 1e-6)
    m = np.mean(x * x, axis=0)
    np.testing.assert_allclose(np.mean(a * a, axis=0), m / (m + 1e-6), rtol=1e-12)
    np.testing.assert_allclose(V.rms_norm(7.5 * x, g, 0.0), V.rms_norm(x, g, 0.0), rtol=1e-12)


def test_residual_block_with_zero_second_conv_is_identity():
    cfg = get_vae_config(11)
    P = V.weights_f64(VaeWeights(cfg))
    name = "decoder.up_blocks.3.resnets.0"
    P[f"{name}.conv2.weight"] = np.zeros_like(P[f"{name}.conv2.weight"])
    P[f"{name}.conv2.bias"] = np.zeros_like(P[f"{name}.conv2.bias"])
    x = _rand((cfg.base_dim, 3, 4, 5), 18)
    np.testing.assert_array_equal(V._res_whole(x, P, name, 1e-6), x)


def test_time_upsample_frame_order():
    """With an identity resample and a time conv whose channel block s copies s + 1 times the current
    frame, upsample3d gives frames x0, x1, 2 x1, x2, 2 x2, ... (each upsampled x2 in space)."""
    C, T = 2, 4
    x = _rand((C, T, 3, 4), 19)
    wt = np.zeros((2 * C, C, 3, 1, 1))
    for c in range(C):
        wt[c, c, 2] = 1.0
        wt[C + c, c, 2] = 2.0
    wr = np.zeros((C, C, 3, 3))
    for c in range(C):
        wr[c, c, 1, 1] = 1.0
    P = {"u.time_conv.weight": wt, "u.time_conv.bias": np.zeros(2 * C), "u.resample.1.weight": wr,
         "u.resample.1.bias": np.zeros(C)}
    y = V._up_whole(x, P, "u", time=True)
    assert y.shape == (C, 1 + 2 * (T - 1), 6, 8)
    want = [x[:, 0]] + [s * x[:, t] for t in range(1, T) for s in (1.0, 2.0)]
    for i, f in enumerate(want):
        np.testing.assert_allclose(y[:, i], np.repeat(np.repeat(f, 2, 1), 2, 2), rtol=1e-15)


def test_denormalize_inverts_the_encoder_normalisation():
    mu = _rand((16, 2, 3, 3), 20)
    mean, std = _rand(16, 21), np.abs(_rand(16, 22)) + 0.5
    normed = (mu - mean[:, None, None, None]) / std[:, None, None, None]
    np.testing.assert_allclose(V.denormalize(normed, mean, std), mu, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------------------------------------
# Whole decoder
# ------------------------------------------------------------------------------------------------
def _torch_decoder(z, P, layout, eps):
    """The decoder assembled from torch float64 library ops (conv3d with the printed causal padding,
    conv2d, nearest-exact interpolation, silu), one whole sequence per stage."""
    T = {k: torch.from_numpy(v) for k, v in P.items()}

    def cc(x, wn, bn):
        w = T[wn]
        kt, kh, kw = w.shape[2:]
        return F.conv3d(F.pad(x, (kw // 2, kw // 2, kh // 2, kh // 2, kt - 1, 0)), w, T[bn])

    def norm(x, g):
        return x * torch.rsqrt((x * x).mean(1, keepdim=True) + eps) * T[g].view(1, -1, 1, 1, 1)

    x = torch.from_numpy(z)[None] * T["latents_std"].view(1, -1, 1, 1, 1) + T["latents_mean"].view(1, -1, 1, 1, 1)
    x = cc(x, "post_quant_conv.weight", "post_quant_conv.bias")
    for kind, name, _, _ in layout:
        if kind == "conv_in":
            x = cc(x, f"{name}.weight", f"{name}.bias")
        elif kind == "res":
            h = cc(F.silu(norm(x, f"{name}.norm1.gamma")), f"{name}.conv1.weight", f"{name}.conv1.bias")
            h = cc(F.silu(norm(h, f"{name}.norm2.gamma")), f"{name}.conv2.weight", f"{name}.conv2.bias")
            if f"{name}.conv_shortcut.weight" in T:
                x = cc(x, f"{name}.conv_shortcut.weight", f"{name}.conv_shortcut.bias")
            x = x + h
        elif kind in ("up3d", "up2d"):
            if kind == "up3d":
                r = cc(x[:, :, 1:], f"{name}.time_conv.weight", f"{name}.time_conv.bias")
                b_, c2, t_, h_, w_ = r.shape
                r = r.view(b_, 2, c2 // 2, t_, h_, w_).permute(0, 2, 3, 1, 4, 5).reshape(b_, c2 // 2, 2 * t_, h_, w_)
                x = torch.cat([x[:, :, :1], r], 2)
            b_, c_, t_, h_, w_ = x.shape
            f = x.permute(0, 2, 1, 3, 4).reshape(b_ * t_, c_, h_, w_)
            f = F.interpolate(f, scale_factor=(2.0, 2.0), mode="nearest-exact")
            f = F.conv2d(f, T[f"{name}.resample.1.weight"], T[f"{name}.resample.1.bias"], padding=1)
            x = f.view(b_, t_, -1, 2 * h_, 2 * w_).permute(0, 2, 1, 3, 4)
        elif kind == "head":
            x = cc(F.silu(norm(x, f"{name}.norm_out.gamma")), f"{name}.conv_out.weight", f"{name}.conv_out.bias")
    return x.clamp(-1.0, 1.0)[0].numpy()


def test_decoder_matches_torch_library_assembly():
    cfg = get_vae_config(11)
    P = V.weights_f64(VaeWeights(cfg))
    z = draw_vae_latent(cfg).f64()[0]
    ours = V.decode_whole(z, P, decoder_layout(cfg), cfg.eps)
    ref = _torch_decoder(z, P, decoder_layout(cfg), cfg.eps)
    assert ours.shape == cfg.out_shape[1:]
    np.testing.assert_allclose(ours, ref, rtol=1e-10, atol=1e-10)
    assert 0.2 < ours.std() < 1.0 and 0.0 < np.mean(np.abs(ours) == 1.0) < 0.3   # not degenerate


@pytest.mark.parametrize("frames,chunks", [(3, None), (3, [2]), (5, [1, 3]), (5, [4]), (5, [2, 2])])
def test_streaming_decode_equals_whole_sequence(frames, chunks):
    cfg = VaeConfig(11, "vae-tiny", frames=frames, height=4, width=6, base_dim=8)
    P = V.weights_f64(VaeWeights(cfg))
    z = draw_vae_latent(cfg).f64()[0]
    whole = V.decode_whole(z, P, decoder_layout(cfg), cfg.eps)
    stream = V.decode_stream(z, P, decoder_layout(cfg), cfg.eps, chunks=chunks)
    np.testing.assert_allclose(stream, whole, rtol=1e-12, atol=1e-12)


def test_decoder_is_causal_in_latent_frames():
    """Latent frame k >= 1 decodes to output frames 4k - 3 .. 4k: changing it leaves every earlier output
    frame unchanged; frame 0 alone makes output frame 0."""
    cfg = VaeConfig(11, "vae-tiny", frames=4, height=3, width=4, base_dim=8)
    P = V.weights_f64(VaeWeights(cfg))
    lay = decoder_layout(cfg)
    z = draw_vae_latent(cfg).f64()[0]
    base = V.decode_whole(z, P, lay, cfg.eps, clamp=False)
    assert base.shape[1] == 13
    for k in range(4):
        z2 = z.copy()
        z2[:, k] += 0.5
        d = np.abs(V.decode_whole(z2, P, lay, cfg.eps, clamp=False) - base).max(axis=(0, 2, 3))
        first = 0 if k == 0 else 4 * k - 3
        assert np.all(d[:first] == 0.0), (k, d)
        assert np.all(d[first:first + (1 if k == 0 else 4)] > 1e-4), (k, d)
    one = VaeConfig(11, "vae-tiny", frames=1, height=3, width=4, base_dim=8)
    np.testing.assert_allclose(V.decode_whole(z[:, :1], P, lay, cfg.eps, clamp=False), base[:, :1], rtol=1e-12,
                               atol=1e-12)
    assert one.out_frames == 1


def test_decoder_flop_count_by_brute_force():
    """decoder_flops against counting 2 x (weight elements) x (output positions) conv by conv from the
    stage shapes of a traced run."""
    cfg = VaeConfig(11, "vae-tiny", frames=3, height=2, width=3, base_dim=8)
    spec = {n: s for n, s, _ in vae_weight_spec(cfg)}
    T, h, w = cfg.frames, cfg.height, cfg.width
    total = 2 * 16 * 16 * T * h * w
    for kind, name, ci, co in decoder_layout(cfg):
        convs = []
        if kind == "conv_in":
            convs = [(f"{name}.weight", T, h, w)]
        elif kind == "res":
            convs = [(f"{name}.conv1.weight", T, h, w), (f"{name}.conv2.weight", T, h, w)]
            if f"{name}.conv_shortcut.weight" in spec:
                convs.append((f"{name}.conv_shortcut.weight", T, h, w))
        elif kind == "up3d":
            convs = [(f"{name}.time_conv.weight", T - 1, h, w)]
            T, h, w = 2 * T - 1, 2 * h, 2 * w
            convs.append((f"{name}.resample.1.weight", T, h, w))
        elif kind == "up2d":
            h, w = 2 * h, 2 * w
            convs = [(f"{name}.resample.1.weight", T, h, w)]
        elif kind == "head":
            convs = [(f"{name}.conv_out.weight", T, h, w)]
        for wn, t_, h_, w_ in convs:
            total += 2 * int(np.prod(spec[wn])) * t_ * h_ * w_
    assert V.decoder_flops(cfg.frames, cfg.height, cfg.width, decoder_layout(cfg)) == total


def test_decoder_goldens_come_from_the_current_oracle():
    """tests/golden/vae_cfg*_first2.npz were written by this oracle (or one listed as arithmetic-equivalent),
    and their sample positions lie inside the first five frames of the workload's video."""
    import hashlib

    hashes = json.load(open(os.path.join(HERE, "golden", "oracle_hashes.json")))["vae"]
    src = hashlib.sha256(open(os.path.join(os.path.dirname(HERE), "oracle", "wan_vae_oracle.py"), "rb").read())
    assert hashes["current"] == src.hexdigest()[:16]
    ok = {hashes["current"], *hashes["equivalent"]}
    for cfg_id in (13, 14):
        g = np.load(os.path.join(HERE, "golden", f"vae_cfg{cfg_id}_first2.npz"))
        assert str(g["oracle"][0]) in ok
        cfg = get_vae_config(cfg_id)
        assert int(g["frames"][0]) == 5
        pos = g["positions"]
        hi = np.array([3, 5, cfg.out_shape[3], cfg.out_shape[4]])
        assert pos.min() >= 0 and np.all(pos.max(axis=0) < hi) and len(pos) > 30000
        assert len(np.unique(pos, axis=0)) == len(pos)
        assert np.all(np.abs(g["values"]) <= 1.0) and 0.3 < float(g["video_std"][0]) < 0.8
