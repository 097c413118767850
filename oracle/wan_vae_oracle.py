"""Plain float64 CPU oracle of the Wan-VAE causal video decoder.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the package entry module and the
CPU-baseline leg of the benchmark may import this module.  The GPU library never calls it and shares
no code with it; the two meet only through the seeded generator in ``wan_inputs``.

Every function evaluates the plain definition in float64 with numpy.  A convolution is written as its
definition, a sum over kernel taps of shifted inputs times that tap's [c_out, c_in] weight matrix (the
matrix product goes to the host BLAS).  Activations of one sample are [C, T, H, W] (channels, frames,
rows, columns), as the pages print them.

Sources (page titles; sections / printed code):
  [WP]   "diffusers WanPipeline notes" (the page that decodes the (1,16,21,60,104) latent), section
         "vae.decode": the loop over latent frames with the per-convolution feature cache (CACHE_T = 2),
         WanDecoder3d's forward, WanCausalConv3d (all temporal padding on the past side, cache frames
         concatenated in front), the upsample2d / upsample3d modes (nearest-exact x2 then a 3x3 Conv2d
         halving the channels; upsample3d adds a (3,1,1) causal time conv doubling them) and the printed
         up-block ModuleList (residual blocks: SiLU, RMS_norm, causal 3x3x3 convs, 1x1x1 shortcut).
  [W21]  "【VLA与模仿学习】Wan2.1框架与训练源码导读" - section 3.1 (T = 4n + 1 frames <-> 1 + (T-1)/4
         latent frames, x8 spatial), section 3.2 (causal convolution, feature cache, per-channel
         normalisation of the encoder's mean).

Readings where the pages leave a step open (each also stated where it is used):
  V1  RMS_norm over channels: u / sqrt(mean_c(u^2) + eps) * gamma, eps = 1e-6, no bias.
  V2  Residual block: h = conv1(SiLU(norm1(x))); h = conv2(SiLU(norm2(h))); out = h + shortcut(x)
      (dropout p = 0 is the identity); shortcut = identity, or the 1x1x1 conv where widths differ.
  V3  The mid block holds two residual blocks at the stage-A width: the count of 33 causal
      convolutions leaves exactly four for it, and nothing else in it is printed.
  V4  conv_in and conv_out are 3x3x3 causal convs with spatial padding 1 (the printed shapes keep H, W);
      conv_out gives 3 (RGB) channels; post_quant_conv is a 1x1x1 conv 16 -> 16.
  V5  Before post_quant_conv the latent is un-normalised per channel, z * std + mean (the inverse of the
      encoder's normalisation of its mean).
  V6  upsample3d: the time conv runs first (it takes the block's full width), its 2C output channels
      split into two frames (channels [0, C) first); the latent's first frame, decoded alone, passes
      the time conv by and does not enter its history, so the time conv sees zeros before the second
      chunk.  Then every frame is upsampled x2 (nearest) and goes through the 3x3 Conv2d.
  V7  The decoded video is clamped to [-1, 1].
"""
from __future__ import annotations

import numpy as np

CACHE_T = 2          # frames each causal convolution keeps from earlier chunks [WP]


# ----------------------------------------------------------------------------------------------------
# Building blocks
# ----------------------------------------------------------------------------------------------------
def denormalize(z: np.ndarray, mean: np.ndarray, std: np.ndarray) -> np.ndarray:
    """Reading V5: z [C, T, H, W] -> z * std_c + mean_c."""
    return z * std[:, None, None, None] + mean[:, None, None, None]


def silu(u: np.ndarray) -> np.ndarray:
    return u / (1.0 + np.exp(-u))


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """Reading V1: per position, over the channel axis 0."""
    ms = np.mean(x * x, axis=0, keepdims=True)
    return x / np.sqrt(ms + eps) * gamma.reshape((-1,) + (1,) * (x.ndim - 1))


def _conv_time_valid(xp: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Convolution over an input already padded in time: xp [Ci, T + kt - 1, H, W], w [Co, Ci, kt, kh, kw]
    (odd kh, kw) -> [Co, T, H, W], zero padding (kh // 2, kw // 2) on both sides in space, none in time.
    Written as the sum over taps (a, r, c) of w[:, :, a, r, c] @ (input shifted by that tap)."""
    co, ci, kt, kh, kw = w.shape
    T = xp.shape[1] - (kt - 1)
    H, W = xp.shape[2], xp.shape[3]
    ph, pw = kh // 2, kw // 2
    xs = np.pad(xp, ((0, 0), (0, 0), (ph, ph), (pw, pw)))
    out = np.zeros((co, T, H, W))
    for a in range(kt):
        for r in range(kh):
            for c in range(kw):
                sl = xs[:, a:a + T, r:r + H, c:c + W]
                out += np.tensordot(w[:, :, a, r, c], sl, axes=([1], [0]))
    return out + b[:, None, None, None]


def causal_conv3d(x: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """WanCausalConv3d over a whole frame sequence [WP]: the kt - 1 frames of temporal padding go on the
    past side (zeros before frame 0), spatial padding kh // 2, kw // 2 zeros on both sides."""
    kt = w.shape[2]
    xp = np.pad(x, ((0, 0), (kt - 1, 0), (0, 0), (0, 0)))
    return _conv_time_valid(xp, w, b)


def causal_conv3d_step(x: np.ndarray, cache: np.ndarray | None, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """One chunk of the streaming form [WP]: the cached frames of earlier chunks go in front of the chunk
    and replace as much of the past-side zero padding; the output has the chunk's frames."""
    kt = w.shape[2]
    pad_t = kt - 1
    if cache is not None and pad_t > 0:
        x = np.concatenate([cache, x], axis=1)
        pad_t -= cache.shape[1]
    xp = np.pad(x, ((0, 0), (pad_t, 0), (0, 0), (0, 0)))
    return _conv_time_valid(xp, w, b)


def next_cache(x: np.ndarray, cache: np.ndarray | None) -> np.ndarray:
    """The cache a convolution keeps for the next chunk [WP]: the last CACHE_T frames of its input; when
    the chunk is shorter than that, the last frame of the previous cache goes in front."""
    new = x[:, -CACHE_T:]
    if new.shape[1] < CACHE_T and cache is not None:
        new = np.concatenate([cache[:, -1:], new], axis=1)
    return new.copy()


def conv2d_frames(x: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Conv2d applied to every frame: w [Co, Ci, kh, kw], zero padding kh // 2 (the printed padding 1)."""
    return _conv_time_valid(x, w[:, :, None], b)


def upsample_nearest2x(x: np.ndarray) -> np.ndarray:
    """nearest-exact x2 in rows and columns: output (2i + r, 2j + c) = input (i, j)."""
    return np.repeat(np.repeat(x, 2, axis=2), 2, axis=3)


def time_to_frames(y: np.ndarray) -> np.ndarray:
    """Reading V6: [2C, T, H, W] -> [C, 2T, H, W], output frame 2t + s = channels [sC, (s + 1)C) at t."""
    c2, T, H, W = y.shape
    c = c2 // 2
    return y.reshape(2, c, T, H, W).transpose(1, 2, 0, 3, 4).reshape(c, 2 * T, H, W)


# ----------------------------------------------------------------------------------------------------
# Whole-sequence form: every causal convolution over all frames of its stage at once
# ----------------------------------------------------------------------------------------------------
def _res_whole(x, P, name, eps):
    h = causal_conv3d(silu(rms_norm(x, P[f"{name}.norm1.gamma"], eps)), P[f"{name}.conv1.weight"],
                      P[f"{name}.conv1.bias"])
    h = causal_conv3d(silu(rms_norm(h, P[f"{name}.norm2.gamma"], eps)), P[f"{name}.conv2.weight"],
                      P[f"{name}.conv2.bias"])
    sc = f"{name}.conv_shortcut.weight"
    if sc in P:
        x = causal_conv3d(x, P[sc], P[f"{name}.conv_shortcut.bias"])
    return h + x


def _up_whole(x, P, name, time: bool):
    if time:
        # reading V6: frame 0 (the first chunk) passes; the rest go through the time conv with zero past
        rest = causal_conv3d(x[:, 1:], P[f"{name}.time_conv.weight"], P[f"{name}.time_conv.bias"])
        x = np.concatenate([x[:, :1], time_to_frames(rest)], axis=1)
    return conv2d_frames(upsample_nearest2x(x), P[f"{name}.resample.1.weight"], P[f"{name}.resample.1.bias"])


def decode_whole(z: np.ndarray, P: dict, layout, eps: float = 1e-6, clamp: bool = True) -> np.ndarray:
    """Decoder of one sample, z [16, F, H, W] -> video [3, 1 + 4 (F - 1), 8H, 8W]; P: {name: float64 array};
    layout: wan_inputs.vae.decoder_layout(cfg)."""
    x = denormalize(z, P["latents_mean"], P["latents_std"])
    x = causal_conv3d(x, P["post_quant_conv.weight"], P["post_quant_conv.bias"])
    for kind, name, _, _ in layout:
        if kind == "conv_in":
            x = causal_conv3d(x, P[f"{name}.weight"], P[f"{name}.bias"])
        elif kind == "res":
            x = _res_whole(x, P, name, eps)
        elif kind in ("up3d", "up2d"):
            x = _up_whole(x, P, name, kind == "up3d")
        elif kind == "head":
            x = silu(rms_norm(x, P[f"{name}.norm_out.gamma"], eps))
            x = causal_conv3d(x, P[f"{name}.conv_out.weight"], P[f"{name}.conv_out.bias"])
    return np.clip(x, -1.0, 1.0) if clamp else x


# ----------------------------------------------------------------------------------------------------
# Streaming form: the pages' loop over latent frames, one feature cache per causal convolution
# ----------------------------------------------------------------------------------------------------
class _Stream:
    """The decoder run chunk by chunk with a feature cache per causal convolution (keyed by the
    convolution's name instead of the running index of the pages' list: the same 33 slots)."""

    def __init__(self, P: dict, layout, eps: float):
        self.P, self.layout, self.eps = P, layout, eps
        self.cache: dict[str, np.ndarray | None] = {}
        self.first_passed: set[str] = set()

    def conv(self, key: str, x: np.ndarray) -> np.ndarray:
        w, b = self.P[f"{key}.weight"], self.P[f"{key}.bias"]
        old = self.cache.get(key)
        new = next_cache(x, old)
        y = causal_conv3d_step(x, old, w, b)
        self.cache[key] = new
        return y

    def res(self, name: str, x: np.ndarray) -> np.ndarray:
        P, eps = self.P, self.eps
        h = self.conv(f"{name}.conv1", silu(rms_norm(x, P[f"{name}.norm1.gamma"], eps)))
        h = self.conv(f"{name}.conv2", silu(rms_norm(h, P[f"{name}.norm2.gamma"], eps)))
        if f"{name}.conv_shortcut.weight" in P:          # 1x1x1: no temporal padding, cache unused
            x = causal_conv3d(x, P[f"{name}.conv_shortcut.weight"], P[f"{name}.conv_shortcut.bias"])
        return h + x

    def up(self, name: str, x: np.ndarray, time: bool) -> np.ndarray:
        P = self.P
        if time:
            key = f"{name}.time_conv"
            if key not in self.first_passed:            # the first chunk: no time conv (reading V6)
                self.first_passed.add(key)
            else:
                x = time_to_frames(self.conv(key, x))
        return conv2d_frames(upsample_nearest2x(x), P[f"{name}.resample.1.weight"], P[f"{name}.resample.1.bias"])

    def chunk(self, x: np.ndarray, trace: list | None = None) -> np.ndarray:
        """One decoder call [WP]; trace, when given, receives (kind, name, shape) after every entry."""
        P, eps = self.P, self.eps
        for kind, name, _, _ in self.layout:
            if kind == "conv_in":
                x = self.conv(name, x)
            elif kind == "res":
                x = self.res(name, x)
            elif kind in ("up3d", "up2d"):
                x = self.up(name, x, kind == "up3d")
            elif kind == "head":
                x = self.conv(f"{name}.conv_out", silu(rms_norm(x, P[f"{name}.norm_out.gamma"], eps)))
            if trace is not None:
                trace.append((kind, name, x.shape))
        return x


def decode_stream(z: np.ndarray, P: dict, layout, eps: float = 1e-6, chunks=None, clamp: bool = True) -> np.ndarray:
    """The pages' decode [WP]: post_quant_conv over the latent, then the decoder on one latent frame at a
    time (chunks: optional list of chunk lengths after the first frame, e.g. [4, 4]; default one frame
    each), the outputs concatenated along time, then the clamp."""
    x = denormalize(z, P["latents_mean"], P["latents_std"])
    x = causal_conv3d(x, P["post_quant_conv.weight"], P["post_quant_conv.bias"])
    F = x.shape[1]
    bounds = [0, 1]
    for n in (chunks or [1] * (F - 1)):
        bounds.append(min(F, bounds[-1] + n))
    assert bounds[-1] == F, "chunks must cover the latent frames"
    st = _Stream(P, layout, eps)
    outs = [st.chunk(x[:, bounds[i]:bounds[i + 1]]) for i in range(len(bounds) - 1) if bounds[i + 1] > bounds[i]]
    out = np.concatenate(outs, axis=1)
    return np.clip(out, -1.0, 1.0) if clamp else out


def decode(latent: np.ndarray, P: dict, layout, eps: float = 1e-6, form: str = "whole") -> np.ndarray:
    """Batch of latents [B, 16, F, H, W] -> videos [B, 3, 1 + 4 (F - 1), 8H, 8W], each sample on its own."""
    f = decode_whole if form == "whole" else decode_stream
    return np.stack([f(latent[i], P, layout, eps) for i in range(latent.shape[0])])


def weights_f64(weights, names=None) -> dict:
    """{name: float64 array} from a wan_inputs.vae.VaeWeights (or any name -> Tensor mapping)."""
    return {n: weights[n].f64() for n in (names or weights.names())}


def decoder_flops(F: int, H: int, W: int, layout) -> int:
    """Multiply-add FLOPs (2 per MAC) of the decoder's convolutions for a latent of F x H x W, counting
    each causal convolution over every output frame with its full kernel (taps on zero padding included)."""
    fl = 2 * 16 * 16 * F * H * W                    # post_quant_conv
    T, h, w = F, H, W
    for kind, _, ci, co in layout:
        if kind in ("conv_in", "res"):
            fl += 2 * co * ci * 27 * T * h * w
            if kind == "res":
                fl += 2 * co * co * 27 * T * h * w
                if ci != co:
                    fl += 2 * co * ci * T * h * w
        elif kind == "up3d":
            fl += 2 * (2 * ci) * ci * 3 * (T - 1) * h * w
            T = 1 + 2 * (T - 1)
            h, w = 2 * h, 2 * w
            fl += 2 * co * ci * 9 * T * h * w
        elif kind == "up2d":
            h, w = 2 * h, 2 * w
            fl += 2 * co * ci * 9 * T * h * w
        elif kind == "head":
            fl += 2 * co * ci * 27 * T * h * w
    return fl
