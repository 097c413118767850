"""The C ABI library loads, exports every declared symbol, and rejects bad arguments before touching the GPU.

CPU-only: no call here reaches a kernel launch (every call fails validation first).
"""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "video_diffusion_transformer_patchify_amd", "libwan_dit.so")



@pytest.fixture(scope="module", autouse=True)
def built_library():
    """The library this module checks: built here (hipcc cross-compiles for gfx950 without a GPU) when it
    is missing, so the C ABI is never left unchecked; a failed build fails the tests."""
    if not os.path.exists(LIB):
        from video_diffusion_transformer_patchify_amd.build import build

        build()
    assert os.path.exists(LIB)


def declared_functions():
    names = []
    for h in ("wan_dit.h", "wan_ops.h", "wan_vae.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:[A-Za-z_][\w\s\*]*?)\b(wan_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    lib = C.CDLL(LIB)
    names = declared_functions()
    assert len(names) >= 15, names
    for n in names:
        assert hasattr(lib, n), n


def test_binding_lists_every_declared_symbol():
    from video_diffusion_transformer_patchify_amd import binding

    assert sorted(binding.EXPORTED) == declared_functions()


def test_validation_errors_without_gpu():
    from video_diffusion_transformer_patchify_amd import binding as B

    # create: NULL config / NULL out
    h = C.c_void_p()
    assert B._create(None, None, 0, None, C.byref(h)) == 1
    assert "config" in B.last_error()
    cfg = B.WanDitConfig()
    assert B._create(C.byref(cfg), None, 0, None, None) == 1
    # unsupported head_dim
    from wan_inputs import get_config

    c = B.make_config(get_config(1))
    c.head_dim = 64
    assert B._create(C.byref(c), None, 0, None, C.byref(h)) == 4
    assert "head_dim" in B.last_error()
    c = B.make_config(get_config(1))
    c.patch_h = 4
    assert B._create(C.byref(c), None, 0, None, C.byref(h)) == 4
    # missing weights are reported by name
    c = B.make_config(get_config(1))
    assert B._create(C.byref(c), None, 0, None, C.byref(h)) == 7
    assert "patch_embedding.weight" in B.last_error()
    # forward on a NULL handle
    assert B._forward(None, None, None, None, None, None) == 1
    # op argument checks
    assert B._op_gemm(1, 64, 1, 64, 1, 10, 64, 60, 0, 1, 64, None, None, 0, 1, None) == 2      # K % 64
    assert B._op_gemm(1, 64, 1, 64, 1, 10, 64, 64, 9, 1, 64, None, None, 0, 1, None) == 1      # epilogue
    assert B._op_gemm(1, 64, 1, 64, 1, 10, 64, 64, 4, 1, 64, None, None, 0, 1, None) == 1      # gate missing
    assert B._op_patchify(1, 0, 1, 16, 5, 15, 16, 64, 1, None) == 2                             # odd height
    assert B._op_attention(1, 1536, 1, 1536, 1, 100, 1, 1536, 1, 320, 320, 12, None) == 2       # ldv < Lkv
    assert B._op_layernorm(1, 4, 1000, 1e-6, 0, 1, 1, 1, 0, 0, 0, 1, None, None, 0, None, None, None, 0, 1,
                           None) == 2                                                           # D % 256
    assert B._op_layernorm(1, 4, 1536, 1e-6, 0, 1, 1, 1, 0, 0, 0, 1, None, None, 2, 1, None, None, 0, 1,
                           None) == 1                                                           # gate missing
    assert B._op_qk_norm_rope(1, 4608, 4, 1536, 1e-6, 0, 1, 1536, 1, 1, 10, 2, 2, 2, 44, 42, 42, 1.0, None) == 2
    assert B._op_rope_table(1, 5, 8, 8, 44, 42, 40, 1e4, None) == 2                              # dims sum != 128


def test_vae_validation_errors_without_gpu():
    from video_diffusion_transformer_patchify_amd import binding as B
    from wan_inputs.vae import get_vae_config

    h = C.c_void_p()
    assert B._vae_create(None, None, 0, None, C.byref(h)) == 1
    c = B.make_vae_config(get_vae_config(14))
    c.z_dim = 48
    assert B._vae_create(C.byref(c), None, 0, None, C.byref(h)) == 4
    c = B.make_vae_config(get_vae_config(14), chunk_frames=5)
    assert B._vae_create(C.byref(c), None, 0, None, C.byref(h)) == 1
    assert "chunk_frames" in B._vae_last_error().decode()
    c = B.make_vae_config(get_vae_config(14))
    assert B._vae_create(C.byref(c), None, 0, None, C.byref(h)) == 7
    assert "latents_mean" in B._vae_last_error().decode()
    assert B._vae_decode(None, None, None, None) == 1
    assert B._vae_op_packed_elems(96, 96, 2, 3) == -1
    assert B._vae_op_packed_elems(96, 96, 3, 3) == 96 * 3 * 6 * 9 * 16
    assert B._vae_op_packed_elems(3, 96, 3, 3) == 32 * 3 * 6 * 9 * 16
    one = (C.c_void_p * 3)(1, 1, 1)
    outs = (C.c_void_p * 2)(1, 1)
    assert B._vae_op_conv(one, 3, 3, 0, 1, 1, 24, 96, 1, 8, 8, outs, None, 1, None) == 2        # c_in % 16
    assert B._vae_op_conv(one, 3, 3, 1, 1, 1, 96, 96, 1, 8, 8, outs, None, 1, None) == 1        # up needs kt 1
    assert B._vae_op_conv(one, 3, 3, 0, 1, 1, 96, 96, 2, 8, 8, outs, None, 1, None) == 4        # split: time conv
    assert B._vae_op_conv(one, 1, 3, 1, 1, 1, 96, 96, 1, 7, 8, outs, None, 1, None) == 2        # odd H with up
    assert B._vae_op_conv(one, 3, 3, 0, 1, 1, 96, 96, 1, 8, 8, outs, None, 17, None) == 1       # nf
    assert B._vae_op_rms_silu(one, one, 1, 96, 8, 8, 1, 1e-6, None) == 1                        # aliasing
