"""Shared helpers of the GPU parity tests (imported only by tests marked gpu)."""
import sys

import numpy as np
import torch

from video_diffusion_transformer_patchify_amd import binding as B  # noqa: F401  (fails loudly if not built)
from video_diffusion_transformer_patchify_amd.harness import bf16_bits, to_device, to_f64  # noqa: F401
from wan_inputs import draw_normal, draw_uniform  # noqa: F401

DEV = "cuda"


def note(msg: str):
    """Name the case on stdout before a GPU step, so a fault leaves a trace of which case ran."""
    print(msg, flush=True)
    sys.stdout.flush()


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.linalg.norm((got - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))


def max_abs(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.abs(got - ref).max()) if got.size else 0.0


def bf16_dev(shape, seed_name, scale=1.0, cfg_id=0):
    """A seeded N(0, scale^2) bf16 tensor on the GPU and its exact float64 host copy."""
    t = draw_normal(cfg_id, seed_name, tuple(shape), "bf16", scale)
    return to_device(t, DEV), t.f64()


def f32_dev(shape, seed_name, scale=1.0, cfg_id=0):
    t = draw_normal(cfg_id, seed_name, tuple(shape), "f32", scale)
    return to_device(t, DEV), t.f64()


def sync():
    torch.cuda.synchronize()
