"""The five DiT geometries used as workloads, and the shape arithmetic of their inputs.

Pure data plus integer shape bookkeeping; no model arithmetic lives here.  Geometry figures
(width / heads / layers, latent channels, patch size) follow the Wan2.1 walk-through page
("Wan2.1框架与训练源码导读", section 10 model table and section 5.1 Patchify) and the diffusers
WanPipeline notes (the (1,16,21,60,104) latent of the 81x480x832 example).
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class WanConfig:
    cfg_id: int
    name: str
    batch: int
    in_channels: int
    out_channels: int
    frames: int          # latent frames F
    height: int          # latent height H_z
    width: int           # latent width W_z
    dim: int             # model width D
    num_heads: int
    ffn_dim: int
    num_layers: int
    text_len: int        # Lt
    dtype: str           # "f32" or "bf16": storage type of latent / text / Linear weights
    per_token_t: bool = False
    image_len: int = 0   # CLIP image tokens of the I2V branch (0: no image branch)
    image_dim: int = 1280
    head_dim: int = 128
    text_dim: int = 4096
    freq_dim: int = 256
    patch: tuple = (1, 2, 2)
    eps: float = 1e-6
    rope_dims: tuple = (44, 42, 42)
    rope_theta: float = 10000.0
    notes: str = field(default="", compare=False)

    # ---- integer shape bookkeeping ----
    @property
    def post_f(self) -> int:
        return self.frames // self.patch[0]

    @property
    def post_h(self) -> int:
        return self.height // self.patch[1]

    @property
    def post_w(self) -> int:
        return self.width // self.patch[2]

    @property
    def tokens(self) -> int:
        """L = F' * H' * W' tokens per sample."""
        return self.post_f * self.post_h * self.post_w

    @property
    def rows(self) -> int:
        """M = B * L token rows of the residual stream."""
        return self.batch * self.tokens

    @property
    def patch_k(self) -> int:
        return self.in_channels * self.patch[0] * self.patch[1] * self.patch[2]

    @property
    def out_k(self) -> int:
        return self.out_channels * self.patch[0] * self.patch[1] * self.patch[2]

    @property
    def latent_shape(self) -> tuple:
        return (self.batch, self.in_channels, self.frames, self.height, self.width)

    @property
    def out_shape(self) -> tuple:
        return (self.batch, self.out_channels, self.frames, self.height, self.width)

    @property
    def text_shape(self) -> tuple:
        return (self.batch, self.text_len, self.text_dim)

    @property
    def image_shape(self) -> tuple:
        return (self.batch, self.image_len, self.image_dim)

    @property
    def t_shape(self) -> tuple:
        return (self.batch, self.tokens) if self.per_token_t else (self.batch,)

    def with_layers(self, n: int) -> "WanConfig":
        """Same geometry with a different block count (used for reduced-depth parity runs)."""
        d = dict(self.__dict__)
        d["num_layers"] = n
        return WanConfig(**d)

    def replace(self, **kw) -> "WanConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return WanConfig(**d)


CONFIGS = {
    1: WanConfig(1, "tiny-ref", batch=1, in_channels=16, out_channels=16, frames=5, height=16, width=16,
                 dim=1536, num_heads=12, ffn_dim=8960, num_layers=1, text_len=226, dtype="f32",
                 notes="1 block + patch embed + head; 17 frames 128x128 -> 320 tokens; t=500"),
    2: WanConfig(2, "wan2.1-t2v-1.3b-cfg2", batch=2, in_channels=16, out_channels=16, frames=21, height=60,
                 width=104, dim=1536, num_heads=12, ffn_dim=8960, num_layers=30, text_len=226, dtype="bf16",
                 notes="81x480x832, CFG pair as batch 2 -> 32760 tokens per sample"),
    3: WanConfig(3, "dreamzero-i2v-stack", batch=1, in_channels=36, out_channels=16, frames=9, height=44,
                 width=80, dim=5120, num_heads=40, ffn_dim=13824, num_layers=4, text_len=512, dtype="bf16",
                 notes="16 noisy + 16 first-frame condition + 4 mask channels; 7920 tokens"),
    4: WanConfig(4, "wan2.2-ti2v-5b", batch=1, in_channels=48, out_channels=48, frames=31, height=44,
                 width=80, dim=3072, num_heads=24, ffn_dim=14336, num_layers=30, text_len=512, dtype="bf16",
                 per_token_t=True, notes="121 frames 704x1280, 16x spatial VAE; 27280 tokens; per-token t"),
    5: WanConfig(5, "wan-14b-720p", batch=1, in_channels=16, out_channels=16, frames=21, height=90,
                 width=160, dim=5120, num_heads=40, ffn_dim=13824, num_layers=40, text_len=512, dtype="bf16",
                 notes="81x720x1280 -> 75600 tokens"),
}


def get_config(cfg_id: int) -> WanConfig:
    return CONFIGS[cfg_id]


def weight_spec(cfg: WanConfig):
    """Ordered list of (name, shape, kind) for every parameter of the DiT.

    kind is one of "linear_w", "linear_b", "conv_w", "table", "gamma", "beta"; it selects the synthetic
    distribution only.  The inventory follows the module names the diffusers notes print
    (patch_embedding, condition_embedder / time_embedder, blocks[k].scale_shift_table, attn1, attn2,
    norm2, ffn, scale_shift_table, proj_out); the Linear structure inside the time and text embedders
    is the reading stated with the oracle.  With image tokens (the I2V branch) the image MLP and, per
    block, the image keys' and values' projections and key norm gain are added.
    """
    D, Fd = cfg.dim, cfg.ffn_dim
    spec = []

    def lin(name, n_out, n_in):
        spec.append((f"{name}.weight", (n_out, n_in), "linear_w"))
        spec.append((f"{name}.bias", (n_out,), "linear_b"))

    spec.append(("patch_embedding.weight", (D, cfg.in_channels) + tuple(cfg.patch), "conv_w"))
    spec.append(("patch_embedding.bias", (D,), "linear_b"))
    lin("time_embedder.linear_1", D, cfg.freq_dim)
    lin("time_embedder.linear_2", D, D)
    lin("time_proj", 6 * D, D)
    lin("text_embedder.linear_1", D, cfg.text_dim)
    lin("text_embedder.linear_2", D, D)
    if cfg.image_len:
        lin("image_embedder.linear_1", D, cfg.image_dim)
        lin("image_embedder.linear_2", D, D)
    for k in range(cfg.num_layers):
        p = f"blocks.{k}."
        spec.append((p + "scale_shift_table", (1, 6, D), "table"))
        for a in ("attn1", "attn2"):
            for proj in ("to_q", "to_k", "to_v", "to_out"):
                lin(p + f"{a}.{proj}", D, D)
            spec.append((p + f"{a}.norm_q.weight", (D,), "gamma"))
            spec.append((p + f"{a}.norm_k.weight", (D,), "gamma"))
        if cfg.image_len:
            lin(p + "attn2.add_k_proj", D, D)
            lin(p + "attn2.add_v_proj", D, D)
            spec.append((p + "attn2.norm_added_k.weight", (D,), "gamma"))
        spec.append((p + "norm2.weight", (D,), "gamma"))
        spec.append((p + "norm2.bias", (D,), "beta"))
        lin(p + "ffn.proj_in", Fd, D)
        lin(p + "ffn.proj_out", D, Fd)
    spec.append(("scale_shift_table", (1, 2, D), "table"))
    lin("proj_out", cfg.out_k, D)
    return spec


# Parameters the diffusers model keeps in fp32 regardless of the load dtype (time embedder,
# modulation tables, norms).  The synthetic weights for these stay fp32 in every config.
FP32_KEPT_PREFIXES = ("time_embedder.", "time_proj.")
FP32_KEPT_KINDS = ("table", "gamma", "beta")


def weight_dtype(cfg: WanConfig, name: str, kind: str) -> str:
    if kind in FP32_KEPT_KINDS or name.startswith(FP32_KEPT_PREFIXES):
        return "f32"
    return cfg.dtype


def param_count(cfg: WanConfig) -> int:
    n = 0
    for _, shape, _ in weight_spec(cfg):
        c = 1
        for s in shape:
            c *= s
        n += c
    return n
