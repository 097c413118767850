"""Host <-> device helpers for the seeded workloads (torch is used for device memory only).

Host tensors carry a storage dtype ("f32": float32 array, "bf16": uint16 bit patterns), a shape and
the data; these helpers move them to the GPU bit for bit and back.
"""
from __future__ import annotations

import numpy as np
import torch


def to_device(t, device="cuda") -> torch.Tensor:
    """Upload a host tensor with attributes dtype / shape / data (see wan_inputs.Tensor)."""
    if t.dtype == "bf16":
        cpu = torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).view(torch.bfloat16)
    else:
        cpu = torch.from_numpy(np.ascontiguousarray(t.data, dtype=np.float32))
    return cpu.reshape(t.shape).to(device)


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    """Raw uint16 bits of a bf16 tensor, on the host."""
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def to_f64(x: torch.Tensor) -> np.ndarray:
    return x.detach().float().cpu().numpy().astype(np.float64)


def upload_weights(weights, names=None, device="cuda", drop=True, threads=8) -> dict:
    """{name: device tensor} for every weight name; drops each host copy after upload when drop is set.

    Host tensors are produced by a small thread pool (numpy's generators release the GIL) a few names
    ahead of the upload.
    """
    from concurrent.futures import ThreadPoolExecutor

    names = list(names or weights.names())
    out = {}
    with ThreadPoolExecutor(threads) as ex:
        futs = [ex.submit(weights.__getitem__, n) for n in names[: 2 * threads]]
        for i, n in enumerate(names):
            host = futs[i].result()
            if i + 2 * threads < len(names):
                futs.append(ex.submit(weights.__getitem__, names[i + 2 * threads]))
            out[n] = to_device(host, device)
            futs[i] = None
            if drop and hasattr(weights, "drop"):
                weights.drop(n)
    return out
