"""End-to-end parity of wan_dit_forward (through the C ABI) against the fp64 oracle, plus properties
that hold at any size: run-to-run determinism, batch-duplicate equality, zero-gate identity.

Bars (applied to the final output): relative L2 <= 2e-2 and max abs <= 5e-2.
"""
import numpy as np
import pytest

from oracle import wan_oracle as O
from wan_inputs import Weights, draw_inputs, get_config

pytestmark = pytest.mark.gpu

REL_L2_BAR, MAX_ABS_BAR = 2e-2, 5e-2


@pytest.fixture(scope="module")
def G():
    import gpu_common

    return gpu_common


def run_gpu(G, cfg, weights, latent, t, text, **kw):
    import torch

    from video_diffusion_transformer_patchify_amd.harness import upload_weights

    n_layers = kw.get("num_layers", cfg.num_layers)
    names = [n for n in weights.names() if not n.startswith("blocks.") or int(n.split(".")[1]) < n_layers]
    wd = upload_weights(weights, names=names, drop=False)
    model = G.B.WanDiT(G.B.make_config(cfg, **kw), wd)
    del wd
    out = model.forward(G.to_device(latent), G.to_device(t), G.to_device(text))
    torch.cuda.synchronize()
    return model, out


def compare(G, got, ref):
    r = G.rel_l2(got, ref)
    m = G.max_abs(got, ref)
    print(f"rel_l2={r:.3e} max_abs={m:.3e} ref_std={ref.std():.3f}", flush=True)
    assert r <= REL_L2_BAR and m <= MAX_ABS_BAR, (r, m)


def test_forward_tiny_reference(G):
    """Config 1: 1 block, D=1536, 320 tokens, fp32 latent / text / weights."""
    G.note("forward tiny reference")
    cfg = get_config(1)
    w = Weights(cfg)
    lat, t, txt = draw_inputs(cfg)
    model, out = run_gpu(G, cfg, w, lat, t, txt)
    ref = O.forward(cfg, w, lat.f64(), t.f64(), txt.f64())
    compare(G, G.to_f64(out), ref)


def test_forward_two_blocks_batch2_bf16(G):
    """Tiny geometry, 2 blocks, batch 2, bf16 storage, ragged token count (3*10*7 = 210)."""
    G.note("forward 2 blocks batch 2 bf16")
    cfg = get_config(2).replace(num_layers=2, frames=3, height=20, width=14, text_len=100)
    w = Weights(cfg)
    lat, t, txt = draw_inputs(cfg)
    model, out = run_gpu(G, cfg, w, lat, t, txt)
    ref = O.forward(cfg, w, lat.f64(), t.f64(), txt.f64())
    compare(G, G.to_f64(out), ref)


@pytest.mark.parametrize("batch,frames,height,width,text_len", [
    (1, 1, 16, 16, 1),      # one latent frame (64 tokens) and a one-token text
    (3, 2, 18, 22, 512),    # batch 3, 2 x 9 x 11 = 198 tokens per sample, the longest text of the workloads
])
def test_forward_shape_extremes(G, batch, frames, height, width, text_len):
    """Forward against the oracle at shape extremes: a single frame, one text token, batch 3, 512 text tokens."""
    G.note(f"forward extremes B={batch} F={frames} H={height} W={width} Lt={text_len}")
    cfg = get_config(2).replace(num_layers=1, batch=batch, frames=frames, height=height, width=width,
                                text_len=text_len)
    w = Weights(cfg)
    lat, t, txt = draw_inputs(cfg)
    model, out = run_gpu(G, cfg, w, lat, t, txt)
    ref = O.forward(cfg, w, lat.f64(), t.f64(), txt.f64())
    compare(G, G.to_f64(out), ref)


def test_forward_per_token_timesteps(G):
    """Per-token timesteps [B, L] (the TI2V-5B geometry, reduced to 1 block and 4x22x20 tokens)."""
    G.note("forward per-token timesteps")
    cfg = get_config(4).replace(num_layers=1, frames=4, height=44, width=40, text_len=64)
    w = Weights(cfg)
    lat, t, txt = draw_inputs(cfg)
    model, out = run_gpu(G, cfg, w, lat, t, txt)
    ref = O.forward(cfg, w, lat.f64(), t.f64(), txt.f64())
    compare(G, G.to_f64(out), ref)


def test_forward_i2v_channels(G):
    """36 input channels -> 16 output channels, D=5120, 40 heads (the I2V stack geometry, 1 block, fewer tokens)."""
    G.note("forward I2V channels")
    cfg = get_config(3).replace(num_layers=1, frames=3, height=20, width=16, text_len=77)
    w = Weights(cfg)
    lat, t, txt = draw_inputs(cfg)
    model, out = run_gpu(G, cfg, w, lat, t, txt)
    ref = O.forward(cfg, w, lat.f64(), t.f64(), txt.f64())
    compare(G, G.to_f64(out), ref)


def test_determinism_and_batch_duplicates(G):
    import torch

    G.note("determinism + batch duplicates")
    cfg = get_config(2).replace(num_layers=2, frames=5, height=16, width=16, text_len=226)
    w = Weights(cfg)
    lat, t, txt = draw_inputs(cfg)
    lat.data.reshape(cfg.latent_shape)[1] = lat.data.reshape(cfg.latent_shape)[0]
    txt.data.reshape(cfg.text_shape)[1] = txt.data.reshape(cfg.text_shape)[0]
    model, out1 = run_gpu(G, cfg, w, lat, t, txt)
    out2 = model.forward(G.to_device(lat), G.to_device(t), G.to_device(txt))
    torch.cuda.synchronize()
    b1, b2 = G.bf16_bits(out1), G.bf16_bits(out2)
    assert np.array_equal(b1, b2)                  # run to run
    assert np.array_equal(b1[0], b1[1])            # duplicated batch element


def test_attention_timing(G):
    """wan_dit_time_attention / wan_dit_attention_time: one timed launch per block and forward up to the
    requested count, a reset after each query, timing off at 0, and the same output with and without."""
    import torch

    G.note("attention timing entry points")
    cfg = get_config(2).replace(num_layers=3, frames=3, height=16, width=16, text_len=64)
    w = Weights(cfg)
    lat, t, txt = draw_inputs(cfg)
    model, out0 = run_gpu(G, cfg, w, lat, t, txt)
    args = (G.to_device(lat), G.to_device(t), G.to_device(txt))
    model.time_attention(4)                      # room for 4 of the 6 launches of two forwards
    out1 = model.forward(*args)
    out2 = model.forward(*args)
    total, n = model.attention_time()
    assert n == 4 and total > 0.0, (n, total)
    assert model.attention_time() == (0.0, 0)    # counted once
    model.forward(*args)
    total, n = model.attention_time()            # the event pairs were free again
    assert n == 3 and total > 0.0, (n, total)
    model.time_attention(0)
    model.forward(*args)
    assert model.attention_time() == (0.0, 0)
    torch.cuda.synchronize()
    b0 = G.bf16_bits(out0)
    assert np.array_equal(b0, G.bf16_bits(out1)) and np.array_equal(b0, G.bf16_bits(out2))
    with pytest.raises(G.B.WanError):
        model.time_attention(-1)


def test_zero_gates_block_is_identity(G):
    """Gates exactly zero (table and time_proj rows) and a zero cross-attn output projection make every
    block the identity: N blocks give the same bits as 0 blocks."""
    import torch

    G.note("zero-gate identity")
    cfg = get_config(2).replace(num_layers=3, frames=2, height=12, width=16, text_len=50)
    w = Weights(cfg)
    D = cfg.dim
    for k in range(cfg.num_layers):
        tab = w.f64(f"blocks.{k}.scale_shift_table").copy()
        tab[0, 2] = 0.0
        tab[0, 5] = 0.0
        w.set(f"blocks.{k}.scale_shift_table", tab)
        w.set(f"blocks.{k}.attn2.to_out.weight", np.zeros((D, D)))
        w.set(f"blocks.{k}.attn2.to_out.bias", np.zeros(D))
    tpw = w.f64("time_proj.weight").copy()
    tpb = w.f64("time_proj.bias").copy()
    tpw[2 * D:3 * D] = 0.0
    tpw[5 * D:6 * D] = 0.0
    tpb[2 * D:3 * D] = 0.0
    tpb[5 * D:6 * D] = 0.0
    w.set("time_proj.weight", tpw)
    w.set("time_proj.bias", tpb)
    lat, t, txt = draw_inputs(cfg)
    _, out_n = run_gpu(G, cfg, w, lat, t, txt)
    _, out_0 = run_gpu(G, cfg, w, lat, t, txt, num_layers=0)
    torch.cuda.synchronize()
    assert np.array_equal(G.bf16_bits(out_n), G.bf16_bits(out_0))


def test_forward_rejects_bad_inputs(G):
    import torch

    G.note("forward argument errors")
    cfg = get_config(1)
    w = Weights(cfg)
    lat, t, txt = draw_inputs(cfg)
    model, _ = run_gpu(G, cfg, w, lat, t, txt)
    L, T, X = G.to_device(lat), G.to_device(t), G.to_device(txt)
    with pytest.raises(G.B.WanError) as e:
        model.forward(L[:, :8].contiguous(), T, X)                  # wrong channel count
    assert e.value.status == 2
    with pytest.raises(G.B.WanError) as e:
        model.forward(L, T, X[:, :, :100].contiguous())             # wrong text dim
    assert e.value.status == 2
    with pytest.raises(G.B.WanError) as e:
        model.forward(L, torch.zeros((1, 320), device="cuda"), X)    # per-token t not enabled in this config
    assert e.value.status == 4
    with pytest.raises(G.B.WanError) as e:
        model.forward(L, T.to(torch.bfloat16), X)                    # timestep dtype
    assert e.value.status == 3
    big = torch.zeros((1, 16, 5, 18, 16), device="cuda")             # 5*9*8 = 360 > max_tokens 320
    with pytest.raises(G.B.WanError) as e:
        model.forward(big, T, X)
    assert e.value.status == 2
    # empty batch is a no-op
    empty = model.forward(L[:0].contiguous(), T[:0].contiguous(), X[:0].contiguous())
    assert empty.shape[0] == 0
