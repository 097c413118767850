"""Write sampled fp64-oracle values of the Wan-VAE decode of the full-size workloads' first two latent frames.

By causality the first two latent frames decode to the first five video frames whatever follows them, so
these samples check the GPU's decode of the whole latent at full resolution.  Inputs and weights are
regenerated from the seeded generator on both sides; only the oracle's values are stored.  This script
calls only the oracle and the seeded generator.

usage: python tests/golden/make_vae_golden.py CFG_ID [--samples S]
"""
from __future__ import annotations

import argparse
import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import wan_vae_oracle as V  # noqa: E402
from wan_inputs.vae import VaeWeights, decoder_layout, draw_vae_latent, get_vae_config  # noqa: E402

LATENT_FRAMES = 2


def vae_oracle_hash() -> str:
    with open(os.path.join(ROOT, "oracle", "wan_vae_oracle.py"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def golden_path(cfg_id: int) -> str:
    return os.path.join(HERE, f"vae_cfg{cfg_id}_first2.npz")


def sample_positions(shape, n: int, seed: int) -> np.ndarray:
    """n distinct (c, t, y, x) positions: every corner and edge midpoint of every frame and channel, the
    rest uniform without replacement."""
    C, T, H, W = shape
    fixed = []
    for c in range(C):
        for t in range(T):
            for y in (0, H // 2, H - 1):
                for x in (0, W // 2, W - 1):
                    fixed.append((c, t, y, x))
    rng = np.random.default_rng(seed)
    flat = rng.choice(C * T * H * W, size=n, replace=False)
    rest = np.stack(np.unravel_index(flat, shape), axis=1)
    pos = np.unique(np.concatenate([np.array(fixed), rest]), axis=0)
    return pos.astype(np.int32)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("cfg_id", type=int)
    ap.add_argument("--samples", type=int, default=40000)
    a = ap.parse_args()
    cfg = get_vae_config(a.cfg_id)
    t0 = time.time()
    w = VaeWeights(cfg)
    P = V.weights_f64(w)
    z = draw_vae_latent(cfg, frames=LATENT_FRAMES).f64()[0]
    print(f"{cfg.name}: decoding latent {z.shape} with the oracle", flush=True)
    video = V.decode_whole(z, P, decoder_layout(cfg), cfg.eps)
    pos = sample_positions(video.shape, a.samples, seed=1000 + a.cfg_id)
    vals = video[pos[:, 0], pos[:, 1], pos[:, 2], pos[:, 3]]
    np.savez_compressed(golden_path(a.cfg_id), positions=pos, values=vals.astype(np.float64),
                        frames=np.array([video.shape[1]]), video_std=np.array([video.std()]),
                        oracle=np.array([vae_oracle_hash()]), seconds=np.array([time.time() - t0]))
    print(f"wrote {golden_path(a.cfg_id)}: {len(pos)} samples, video std {video.std():.4f}, "
          f"{time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main()
