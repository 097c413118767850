"""Write sampled fp64-oracle outputs of the full DiT forward for the large workloads.

The GPU end-to-end tests at full size compare the GPU output at these sampled positions (and the
output's overall L2 norm) with the oracle.  Inputs and weights are regenerated from the seeded
generator on both sides, so only the oracle's outputs are stored.  This script calls only the oracle
and the seeded generator.

usage: python tests/golden/make_forward_golden.py CFG_ID [--layers N] [--samples S] [--workers W]
                                                      [--checkpoint DIR] [--rows R] [--image LI]

With --image LI, the forward takes LI seeded CLIP image tokens (the I2V branch); the golden's name carries
an "i" after the workload id.

With --checkpoint, the token stream after each finished block is kept in DIR (one file per workload and
depth, tagged with the oracle's source hash) and an interrupted run resumes from it.

With --rows R (one-block stacks), the oracle evaluates only R seeded token rows plus the first and last
32 tokens (oracle.forward_rows: keys and values of every token, everything else on those rows) and the
golden holds all pt*ph*pw*C_out outputs of each of those tokens (the proj_out values z of those rows);
such a golden has no whole-output sum of squares (rows_only = 1).  This is how the workload too large for a whole fp64 forward on the host gets
its oracle comparison.
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

from oracle import wan_oracle as O  # noqa: E402
from wan_inputs import Weights, draw_image, draw_inputs, get_config  # noqa: E402


def oracle_hash() -> str:
    with open(os.path.join(ROOT, "oracle", "wan_oracle.py"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def golden_path(cfg_id: int, layers: int, image: bool = False) -> str:
    return os.path.join(HERE, f"forward_cfg{cfg_id}{'i' if image else ''}_L{layers}.npz")


class BlockCheckpoint:
    """Keeps the oracle's token stream after the last finished block in one .npy file (+ a small header)."""

    def __init__(self, directory: str, cfg_id: int, layers: int):
        os.makedirs(directory, exist_ok=True)
        stem = os.path.join(directory, f"forward_cfg{cfg_id}_L{layers}")
        self.data, self.head = stem + ".x.npy", stem + ".head.npz"
        self.tag = oracle_hash()

    def load(self):
        if not (os.path.exists(self.data) and os.path.exists(self.head)):
            return None
        h = np.load(self.head)
        if str(h["oracle"][0]) != self.tag:
            print("  checkpoint written by another oracle version: starting over", flush=True)
            return None
        nb = int(h["next_block"][0])
        print(f"  resuming at block {nb}", flush=True)
        return nb, np.load(self.data)

    def save(self, next_block: int, x: np.ndarray):
        np.save(self.data + ".tmp.npy", x)
        os.replace(self.data + ".tmp.npy", self.data)
        np.savez(self.head + ".tmp.npz", next_block=np.array([next_block]), oracle=np.array([self.tag]))
        os.replace(self.head + ".tmp.npz", self.head)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("cfg_id", type=int)
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--samples", type=int, default=32768)
    ap.add_argument("--workers", type=int, default=8)
    ap.add_argument("--checkpoint", default=None, help="directory for per-block resume state")
    ap.add_argument("--rows", type=int, default=0, help="evaluate only this many seeded token rows (+64 edge tokens)")
    ap.add_argument("--image", type=int, default=0, help="CLIP image tokens of the I2V branch (seeded N(0,1))")
    args = ap.parse_args()
    cfg = get_config(args.cfg_id)
    if args.layers is not None:
        cfg = cfg.with_layers(args.layers)
    if args.image:
        cfg = cfg.replace(image_len=args.image)
    w = Weights(cfg)
    lat, t, txt = draw_inputs(cfg)
    t0 = time.time()

    def drop(prefix):
        w.drop(prefix)
        print(f"  {prefix} done at {time.time() - t0:.0f}s", flush=True)

    if args.rows:
        rows_golden(cfg, args, w, lat, t, txt, t0)
        return
    ck = BlockCheckpoint(args.checkpoint, args.cfg_id, cfg.num_layers) if args.checkpoint else None
    img = draw_image(cfg).f64() if cfg.image_len else None
    out = O.forward(cfg, w, lat.f64(), t.f64(), txt.f64(), workers=args.workers, drop=drop, checkpoint=ck, image=img)
    elapsed = time.time() - t0
    rng = np.random.default_rng(12345)
    n = out.size
    idx = np.unique(np.concatenate([rng.integers(0, n, args.samples), np.arange(64), np.arange(n - 64, n)]))
    np.savez(golden_path(args.cfg_id, cfg.num_layers, bool(cfg.image_len)), index=idx.astype(np.int64), value=out.reshape(-1)[idx],
             sumsq=np.array([float((out * out).sum())]), shape=np.array(out.shape), seconds=np.array([elapsed]),
             oracle=np.array([oracle_hash()]), image_len=np.array([cfg.image_len]))
    print(f"cfg {args.cfg_id} layers {cfg.num_layers}: {elapsed:.0f}s, |out| = {np.sqrt((out * out).sum()):.4f}", flush=True)


def rows_golden(cfg, args, w, lat, t, txt, t0):
    """Oracle proj_out values of sampled token rows: z [B, T, pt*ph*pw*C_out] (float32 is ample for the
    comparison bars), with unpatchify's map out[b, c, f, 2h+i, 2w+j] = z[b, token n, (2i+j)*C_out + c]."""
    L = cfg.tokens
    rng = np.random.default_rng(12345)
    tokens = np.unique(np.concatenate([rng.integers(0, L, args.rows), np.arange(32), np.arange(L - 32, L)]))
    z = O.forward_rows(cfg, w, lat.f64(), t.f64(), txt.f64(), tokens, workers=args.workers)
    elapsed = time.time() - t0
    np.savez(golden_path(args.cfg_id, cfg.num_layers), tokens=tokens.astype(np.int32), z=z.astype(np.float32),
             rows_only=np.array([1]), shape=np.array(cfg.out_shape), seconds=np.array([elapsed]),
             oracle=np.array([oracle_hash()]))
    print(f"cfg {args.cfg_id} layers {cfg.num_layers}: {len(tokens)} token rows, {elapsed:.0f}s", flush=True)


if __name__ == "__main__":
    main()
