"""Host-only sanitizer run of the library (CPU): every source compiled for the host side only with
AddressSanitizer and UndefinedBehaviorSanitizer, the HIP runtime replaced by tests/host_asan/hip_stub.cpp
(device memory is host memory; kernel launches are checked for their launch shapes and skipped), then
tests/host_asan/driver.cpp drives the C ABI: weight matching (missing, duplicate, mis-shaped, mis-typed
weights), workspace planning and the whole launch sequence of the DiT forward (per-token timesteps, the
image branch, the denoising step, attention timing) and of the VAE decode (1, 2, 6 and 9 latent frames,
batch 2, a size change, frame rings), the argument checks, the allocation-free attention and the GEMM with a
workspace (its stream-K tail).  Leaks and
memory errors fail the run; so does a launch with an impossible shape.
"""
import os
import shutil
import subprocess

import pytest

from wan_inputs import get_config, weight_spec
from wan_inputs.configs import weight_dtype
from wan_inputs.vae import VaeConfig, vae_weight_spec

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "video_diffusion_transformer_patchify_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_asan")
CLANG = "/opt/rocm/llvm/bin/clang++"
SOURCES = ["k_patch", "k_gemm", "k_norm", "k_attn", "k_scratch", "k_probe", "wan_dit", "k_vae", "wan_vae"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
       "-fno-sanitize-recover=undefined"]


def _dit_spec(cfg, tag, max_batch, image_len=0):
    c = cfg.replace(image_len=image_len) if image_len else cfg
    fields = dict(dim=c.dim, num_heads=c.num_heads, head_dim=c.head_dim, ffn_dim=c.ffn_dim, num_layers=c.num_layers,
                  in_channels=c.in_channels, out_channels=c.out_channels, text_dim=c.text_dim, freq_dim=c.freq_dim,
                  rope_dim_t=c.rope_dims[0], rope_dim_h=c.rope_dims[1], rope_dim_w=c.rope_dims[2],
                  per_token_timestep=int(c.per_token_t), max_batch=max_batch, max_tokens=c.tokens,
                  max_text_len=c.text_len, max_image_len=image_len, image_dim=c.image_dim, frames=c.frames,
                  height=c.height, width=c.width)
    lines = ["DIT " + tag + " " + " ".join(f"{k}={v}" for k, v in fields.items())]
    for name, shape, kind in weight_spec(c):
        dt = 1 if weight_dtype(c, name, kind) == "bf16" else 0
        lines.append(f"W {name} {dt} {len(shape)} " + " ".join(str(d) for d in shape))
    return lines


def _vae_spec(cfg, tag, chunk):
    lines = [f"VAE {tag} base_dim={cfg.base_dim} chunk_frames={chunk} max_height={cfg.height} max_width={cfg.width}"]
    for name, shape, kind in vae_weight_spec(cfg):
        dt = 1 if (kind == "conv_w" and cfg.dtype == "bf16") else 0
        lines.append(f"W {name} {dt} {len(shape)} " + " ".join(str(d) for d in shape))
    return lines


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang is not installed")
def test_host_asan_run(tmp_path):
    objs = []
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    for s in SOURCES:
        o = str(tmp_path / f"{s}.o")
        cmd = [CLANG, "-x", "hip", "--offload-host-only", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
               *SAN, *inc, "-c", os.path.join(CSRC, s + ".hip"), "-o", o]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(o)
    for s in ("hip_stub", "driver"):
        o = str(tmp_path / f"{s}.o")
        cmd = [CLANG, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
               "-I", "/opt/rocm/include", *inc, "-c", os.path.join(HERE, s + ".cpp"), "-o", o]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(o)
    # the host-only objects name the device code objects they would register; nothing loads them here
    nm = subprocess.run(["nm", "-u", *objs], capture_output=True, text=True).stdout
    fatbins = sorted({ln.split()[-1] for ln in nm.splitlines() if "__hip_fatbin" in ln})
    stub_c = tmp_path / "fatbins.c"
    stub_c.write_text("".join(f"char {f}[16];\n" for f in fatbins))
    fo = str(tmp_path / "fatbins.o")
    assert subprocess.run([CLANG, "-x", "c", "-c", str(stub_c), "-o", fo]).returncode == 0
    exe = str(tmp_path / "driver")
    r = subprocess.run([CLANG, "-fsanitize=address,undefined", *objs, fo, "-o", exe, "-lstdc++", "-lm", "-lpthread"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    spec = []
    tiny = get_config(1)
    spec += _dit_spec(tiny, "tiny", 1)
    spec += _dit_spec(tiny.replace(per_token_t=True), "tiny-per-token-t", 2)
    spec += _dit_spec(tiny, "tiny-image", 2, image_len=5)
    spec += _vae_spec(VaeConfig(11, "vae-tiny", frames=3, height=4, width=6, base_dim=8), "vae-tiny", 4)
    spec += _vae_spec(VaeConfig(12, "vae-realwidth", frames=3, height=5, width=7), "vae-realwidth", 1)
    sp = tmp_path / "spec.txt"
    sp.write_text("\n".join(spec) + "\n")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, str(sp)], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout[-2000:])
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-5000:])
    assert "ALL OK" in r.stdout
