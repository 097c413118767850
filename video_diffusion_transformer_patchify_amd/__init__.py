"""MI355X (gfx950) Wan-style video DiT denoiser forward: HIP kernels behind a C ABI.

The compute library is libwan_dit.so (built in-tree by ``build.py``); ``binding`` is its ctypes
binding and ``weights`` moves host weights to the device in the layout the C ABI expects.
"""
import os

PACKAGE_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PACKAGE_DIR, "libwan_dit.so")


def load():
    """Import the binding (raises ImportError if the HIP library has not been built)."""
    from . import binding

    return binding
