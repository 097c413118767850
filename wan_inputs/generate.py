"""Seeded synthetic inputs and weights.

Every tensor gets its own random stream: numpy PCG64 seeded by
SeedSequence(root_seed, spawn_key=(cfg_id, crc32(name))).  Values are drawn in float32 and then,
for bf16 tensors, rounded to the nearest bf16 (ties to even) so that the oracle (which upcasts to
float64) and the GPU path (which consumes the raw bits) see identical numbers.

Distributions (the reading stated for the synthetic workload):
  Linear / Conv weights and biases  N(0, 0.02)
  modulation tables                 randn / sqrt(D)   (the init the diffusers block notes print)
  norm gains                        U[0.5, 1.5]       (a gain-indexing bug is visible, unlike gain == 1)
  norm biases                       N(0, 0.02)
  latent noise, text embedding      N(0, 1)           (the notes feed torch.randn text embeddings)
  CLIP image tokens (I2V branch)    N(0, 1)
  timestep                          500 per sample, or U[0, 1000) per token

This module holds no model arithmetic: only random draws, rounding to the storage type, and the
caching of large tensors.
"""
from __future__ import annotations

import zlib

import numpy as np

from .configs import WanConfig, weight_dtype, weight_spec

ROOT_SEED = 42


def _rng(cfg_id: int, name: str, seed: int = ROOT_SEED) -> np.random.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(cfg_id, zlib.crc32(name.encode())))
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16, ties to even; returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs: u + 0x8000 stays below 2^32, so uint32 arithmetic cannot wrap
    r = ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


class Tensor:
    """A host tensor in its storage type: dtype "f32" (float32 array) or "bf16" (uint16 bits)."""

    __slots__ = ("name", "dtype", "shape", "data")

    def __init__(self, name: str, dtype: str, shape: tuple, data: np.ndarray):
        self.name, self.dtype, self.shape, self.data = name, dtype, tuple(shape), data

    def f32(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.data).reshape(self.shape)
        return self.data.reshape(self.shape)

    def f64(self) -> np.ndarray:
        return self.f32().astype(np.float64)

    @property
    def nbytes(self) -> int:
        return self.data.nbytes


def _store(name: str, dtype: str, shape: tuple, vals_f32: np.ndarray) -> Tensor:
    vals_f32 = vals_f32.reshape(-1)
    if dtype == "bf16":
        return Tensor(name, "bf16", shape, f32_to_bf16_bits(vals_f32))
    return Tensor(name, "f32", shape, np.ascontiguousarray(vals_f32, dtype=np.float32))


def draw_weight(cfg: WanConfig, name: str, shape: tuple, kind: str, seed: int = ROOT_SEED) -> Tensor:
    n = int(np.prod(shape))
    rng = _rng(cfg.cfg_id, name, seed)
    if kind in ("linear_w", "linear_b", "conv_w", "beta"):
        v = rng.standard_normal(n, dtype=np.float32)
        v *= np.float32(0.02)
    elif kind == "table":
        v = rng.standard_normal(n, dtype=np.float32)
        v /= np.float32(np.sqrt(cfg.dim))
    elif kind == "gamma":
        v = rng.random(n, dtype=np.float32) + np.float32(0.5)
    else:
        raise ValueError(kind)
    return _store(name, weight_dtype(cfg, name, kind), shape, v)


class Weights:
    """Lazily drawn weights; each tensor is generated on first access and may be dropped again."""

    def __init__(self, cfg: WanConfig, seed: int = ROOT_SEED, overrides: dict | None = None):
        self.cfg, self.seed = cfg, seed
        self.spec = weight_spec(cfg)
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
            t = draw_weight(self.cfg, name, shape, kind, self.seed)
            self._cache[name] = t
        return t

    def set(self, name: str, values: np.ndarray, dtype: str | None = None):
        """Override one tensor (special-case tests: zero gates, unit gains, ...)."""
        shape, kind = self._kind[name]
        dt = dtype or weight_dtype(self.cfg, name, kind)
        self._overrides[name] = _store(name, dt, shape, np.asarray(values, dtype=np.float32))

    def drop(self, prefix: str = ""):
        for n in list(self._cache):
            if n.startswith(prefix):
                del self._cache[n]

    def f64(self, name: str) -> np.ndarray:
        return self[name].f64()


def draw_latent(cfg: WanConfig, seed: int = ROOT_SEED) -> Tensor:
    shape = cfg.latent_shape
    rng = _rng(cfg.cfg_id, "input.latent", seed)
    v = rng.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if cfg.in_channels == 36:
        # I2V layout: 16 noisy + 16 condition-latent stand-ins (both N(0,1)) + 4 mask channels that are
        # 1 on the first latent frame (the known image) and 0 elsewhere.
        v[:, 32:36] = 0.0
        v[:, 32:36, 0] = 1.0
    return _store("input.latent", cfg.dtype, shape, v)


def draw_text(cfg: WanConfig, seed: int = ROOT_SEED) -> Tensor:
    shape = cfg.text_shape
    rng = _rng(cfg.cfg_id, "input.text", seed)
    v = rng.standard_normal(int(np.prod(shape)), dtype=np.float32)
    return _store("input.text", cfg.dtype, shape, v)


def draw_image(cfg: WanConfig, seed: int = ROOT_SEED) -> Tensor:
    """CLIP image tokens [B, image_len, image_dim] N(0, 1), stand-ins for the encoder's features."""
    shape = cfg.image_shape
    rng = _rng(cfg.cfg_id, "input.image", seed)
    v = rng.standard_normal(int(np.prod(shape)), dtype=np.float32)
    return _store("input.image", cfg.dtype, shape, v)


def draw_timestep(cfg: WanConfig, seed: int = ROOT_SEED) -> Tensor:
    """Timesteps are always float32 values (integer timesteps are a special case of them)."""
    if cfg.per_token_t:
        rng = _rng(cfg.cfg_id, "input.timestep", seed)
        v = rng.random(int(np.prod(cfg.t_shape)), dtype=np.float32) * np.float32(1000.0)
        v = np.minimum(v, np.float32(np.nextafter(np.float32(1000.0), np.float32(0.0))))
        return Tensor("input.timestep", "f32", cfg.t_shape, v)
    return Tensor("input.timestep", "f32", cfg.t_shape, np.full(cfg.t_shape, 500.0, dtype=np.float32).reshape(-1))


def draw_inputs(cfg: WanConfig, seed: int = ROOT_SEED):
    return draw_latent(cfg, seed), draw_timestep(cfg, seed), draw_text(cfg, seed)


def draw_normal(cfg_id: int, name: str, shape: tuple, dtype: str = "bf16", scale: float = 1.0,
                seed: int = ROOT_SEED) -> Tensor:
    """Generic N(0, scale^2) tensor for per-stage tests."""
    rng = _rng(cfg_id, name, seed)
    v = rng.standard_normal(int(np.prod(shape)), dtype=np.float32)
    if scale != 1.0:
        v *= np.float32(scale)
    return _store(name, dtype, shape, v)


def draw_uniform(cfg_id: int, name: str, shape: tuple, lo: float, hi: float, dtype: str = "f32",
                 seed: int = ROOT_SEED) -> Tensor:
    rng = _rng(cfg_id, name, seed)
    v = rng.random(int(np.prod(shape)), dtype=np.float32) * np.float32(hi - lo) + np.float32(lo)
    return _store(name, dtype, shape, v)
