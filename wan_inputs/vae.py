"""Wan-VAE causal decoder workloads: geometry, weight list and seeded synthetic draws.

Pure data plus integer shape bookkeeping; no model arithmetic lives here.

Geometry.  The decoder's module list and the per-frame decode loop are printed on the diffusers
WanPipeline notes page (section "vae.decode": the decode loop over latent frames, WanDecoder3d's
forward, WanCausalConv3d, the upsample modes and the printed up-block ModuleList).  The width ladder
384 / 192 / 96 and the 33 causal convolutions are the Wan2.1 decoder's; the base width is a parameter so
that small cases keep the same structure.  Shape facts: the Wan2.1 walk-through page, section 3.1,
relates a [B, 3, T, H, W] video with T = 4n + 1 to a [B, 16, 1 + (T - 1) / 4, H / 8, W / 8] latent and
works the 33 x 352 x 640 example; the WanPipeline notes decode a (1, 16, 21, 60, 104) latent.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass

import numpy as np

from .generate import ROOT_SEED, Tensor, _store


@dataclass(frozen=True)
class VaeConfig:
    cfg_id: int
    name: str
    frames: int          # latent frames F
    height: int          # latent height H_z
    width: int           # latent width W_z
    base_dim: int = 96   # width of the last up block (Wan2.1: 96)
    z_dim: int = 16
    batch: int = 1
    dtype: str = "bf16"  # storage type of the latent and of the conv weights
    eps: float = 1e-6
    notes: str = ""

    # ---- integer shape bookkeeping ----
    @property
    def dims(self) -> tuple:
        """Channel widths (stage A, B, C, D) = (4, 4, 2, 1) x base: 384, 384, 192, 96 for Wan2.1."""
        b = self.base_dim
        return (4 * b, 4 * b, 2 * b, b)

    @property
    def latent_shape(self) -> tuple:
        return (self.batch, self.z_dim, self.frames, self.height, self.width)

    @property
    def out_frames(self) -> int:
        """1 + 4 (F - 1): the first latent frame decodes to one frame, every later one to four."""
        return 1 + 4 * (self.frames - 1)

    @property
    def out_shape(self) -> tuple:
        return (self.batch, 3, self.out_frames, 8 * self.height, 8 * self.width)


VAE_CONFIGS = {
    11: VaeConfig(11, "vae-tiny", frames=3, height=4, width=6, base_dim=8,
                  notes="decoder structure at base width 8 (channels 32/32/16/8); oracle in milliseconds"),
    12: VaeConfig(12, "vae-realwidth-small", frames=3, height=5, width=7,
                  notes="Wan2.1 widths (384/384/192/96); ragged spatial tiles at every stage"),
    13: VaeConfig(13, "vae-dreamzero-33x352x640", frames=9, height=44, width=80,
                  notes="the DreamZero example: latent [1,16,9,44,80] -> video [1,3,33,352,640]"),
    14: VaeConfig(14, "vae-wan2.1-81x480x832", frames=21, height=60, width=104,
                  notes="the WanPipeline example: latent [1,16,21,60,104] -> video [1,3,81,480,832]"),
    15: VaeConfig(15, "vae-midsize", frames=3, height=12, width=20,
                  notes="Wan2.1 widths at 96 x 160 output pixels; several tiles per frame at every stage"),
}


def get_vae_config(cfg_id: int) -> VaeConfig:
    return VAE_CONFIGS[cfg_id]


def decoder_layout(cfg: VaeConfig):
    """The decoder's blocks in forward order, as (kind, name, c_in, c_out) entries.

    kinds: "conv_in", "res" (residual block), "up3d" (time conv + spatial upsample), "up2d", "head".
    Up block i holds three residual blocks; blocks 0 and 1 end with a 3D upsample, block 2 with a 2D one.
    """
    a, b, c, d = cfg.dims
    out = [("conv_in", "decoder.conv_in", cfg.z_dim, a)]
    out += [("res", f"decoder.mid_block.resnets.{j}", a, a) for j in range(2)]
    # up block 0: 384 -> 384, then upsample3d 384 -> 192
    out += [("res", f"decoder.up_blocks.0.resnets.{j}", a, a) for j in range(3)]
    out += [("up3d", "decoder.up_blocks.0.upsamplers.0", a, a // 2)]
    # up block 1: 192 -> 384 (first block has a 1x1x1 shortcut), then upsample3d 384 -> 192
    out += [("res", "decoder.up_blocks.1.resnets.0", a // 2, b)]
    out += [("res", f"decoder.up_blocks.1.resnets.{j}", b, b) for j in (1, 2)]
    out += [("up3d", "decoder.up_blocks.1.upsamplers.0", b, b // 2)]
    # up block 2: 192 -> 192, then upsample2d 192 -> 96
    out += [("res", f"decoder.up_blocks.2.resnets.{j}", c, c) for j in range(3)]
    out += [("up2d", "decoder.up_blocks.2.upsamplers.0", c, c // 2)]
    # up block 3: 96 -> 96, no upsampler
    out += [("res", f"decoder.up_blocks.3.resnets.{j}", d, d) for j in range(3)]
    out += [("head", "decoder", d, 3)]
    return out


def vae_weight_spec(cfg: VaeConfig):
    """[(name, shape, kind)] of every decoder tensor (diffusers-style names)."""
    spec = [("latents_mean", (cfg.z_dim,), "lat_mean"), ("latents_std", (cfg.z_dim,), "lat_std"),
            ("post_quant_conv.weight", (cfg.z_dim, cfg.z_dim, 1, 1, 1), "conv_w"),
            ("post_quant_conv.bias", (cfg.z_dim,), "bias")]
    for kind, name, ci, co in decoder_layout(cfg):
        if kind == "conv_in":
            spec += [(f"{name}.weight", (co, ci, 3, 3, 3), "conv_w"), (f"{name}.bias", (co,), "bias")]
        elif kind == "res":
            spec += [(f"{name}.norm1.gamma", (ci,), "gamma"),
                     (f"{name}.conv1.weight", (co, ci, 3, 3, 3), "conv_w"), (f"{name}.conv1.bias", (co,), "bias"),
                     (f"{name}.norm2.gamma", (co,), "gamma"),
                     (f"{name}.conv2.weight", (co, co, 3, 3, 3), "conv_w"), (f"{name}.conv2.bias", (co,), "bias")]
            if ci != co:
                spec += [(f"{name}.conv_shortcut.weight", (co, ci, 1, 1, 1), "conv_w"),
                         (f"{name}.conv_shortcut.bias", (co,), "bias")]
        elif kind == "up3d":
            spec += [(f"{name}.time_conv.weight", (2 * ci, ci, 3, 1, 1), "conv_w"),
                     (f"{name}.time_conv.bias", (2 * ci,), "bias"),
                     (f"{name}.resample.1.weight", (co, ci, 3, 3), "conv_w"),
                     (f"{name}.resample.1.bias", (co,), "bias")]
        elif kind == "up2d":
            spec += [(f"{name}.resample.1.weight", (co, ci, 3, 3), "conv_w"),
                     (f"{name}.resample.1.bias", (co,), "bias")]
        elif kind == "head":
            spec += [(f"{name}.norm_out.gamma", (ci,), "gamma"),
                     (f"{name}.conv_out.weight", (co, ci, 3, 3, 3), "conv_w"),
                     (f"{name}.conv_out.bias", (co,), "bias")]
    return spec


def vae_param_count(cfg: VaeConfig) -> int:
    return int(sum(np.prod(s) for _, s, _ in vae_weight_spec(cfg)))


def _rng(cfg_id: int, name: str, seed: int) -> np.random.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(cfg_id, zlib.crc32(name.encode())))
    return np.random.Generator(np.random.PCG64(ss))


def draw_vae_weight(cfg: VaeConfig, name: str, shape: tuple, kind: str, seed: int = ROOT_SEED) -> Tensor:
    """Distributions (the reading stated for the synthetic decoder):
      conv weights      N(0, 1 / fan_in)   (fan_in = c_in x kernel volume: activations stay O(1))
      conv biases       N(0, 0.02)
      RMS-norm gains    U[0.5, 1.5]
      latents_mean      N(0, 0.5^2);  latents_std U[0.5, 3.0]
    Conv weights are stored in the config's dtype, everything else in float32.
    """
    n = int(np.prod(shape))
    rng = _rng(cfg.cfg_id, name, seed)
    if kind == "conv_w":
        v = rng.standard_normal(n, dtype=np.float32)
        v *= np.float32(1.0 / np.sqrt(float(np.prod(shape[1:]))))
        dt = cfg.dtype
    elif kind == "bias":
        v = rng.standard_normal(n, dtype=np.float32) * np.float32(0.02)
        dt = "f32"
    elif kind == "gamma":
        v = rng.random(n, dtype=np.float32) + np.float32(0.5)
        dt = "f32"
    elif kind == "lat_mean":
        v = rng.standard_normal(n, dtype=np.float32) * np.float32(0.5)
        dt = "f32"
    elif kind == "lat_std":
        v = rng.random(n, dtype=np.float32) * np.float32(2.5) + np.float32(0.5)
        dt = "f32"
    else:
        raise ValueError(kind)
    return _store(name, dt, shape, v)


class VaeWeights:
    """Lazily drawn decoder weights (same interface as the DiT's Weights)."""

    def __init__(self, cfg: VaeConfig, seed: int = ROOT_SEED, overrides: dict | None = None):
        self.cfg, self.seed = cfg, seed
        self.spec = vae_weight_spec(cfg)
        self._kind = {n: (s, k) for n, s, k in self.spec}
        self._cache: dict[str, Tensor] = {}
        self._overrides = dict(overrides or {})

    def names(self):
        return [n for n, _, _ in self.spec]

    def shape(self, name):
        return self._kind[name][0]

    def __getitem__(self, name: str) -> Tensor:
        if name in self._overrides:
            return self._overrides[name]
        t = self._cache.get(name)
        if t is None:
            shape, kind = self._kind[name]
            t = draw_vae_weight(self.cfg, name, shape, kind, self.seed)
            self._cache[name] = t
        return t

    def set(self, name: str, values: np.ndarray, dtype: str | None = None):
        shape, kind = self._kind[name]
        dt = dtype or self[name].dtype
        self._overrides[name] = _store(name, dt, shape, np.asarray(values, dtype=np.float32))

    def drop(self, prefix: str = ""):
        for n in list(self._cache):
            if n.startswith(prefix):
                del self._cache[n]

    def f64(self, name: str) -> np.ndarray:
        return self[name].f64()


def draw_vae_latent(cfg: VaeConfig, seed: int = ROOT_SEED, frames: int | None = None) -> Tensor:
    """N(0, 1) latent [B, 16, F, H_z, W_z] in the config's dtype.  frames < F gives the first frames of the
    same draw (the draw is frame-major per channel, so it is cut, not redrawn)."""
    shape = cfg.latent_shape
    rng = _rng(cfg.cfg_id, "input.vae_latent", seed)
    v = rng.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if frames is not None:
        v = np.ascontiguousarray(v[:, :, :frames])
        shape = v.shape
    return _store("input.vae_latent", cfg.dtype, shape, v)
