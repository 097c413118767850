"""ctypes binding of libwan_dit.so (include/wan_dit.h, include/wan_ops.h, include/wan_vae.h).

Argument marshalling only: every stage runs in the HIP library.  torch provides device memory and the
current stream.  If the library has not been built this module raises at import time; there is no
fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwan_dit.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m video_diffusion_transformer_patchify_amd.build`")
lib = C.CDLL(_LIB_PATH)

WAN_F32, WAN_BF16 = 0, 1
EPI_BF16, EPI_GELU_BF16, EPI_F32, EPI_RES_F32, EPI_GATE_F32 = range(5)
STATUS = {0: "WAN_OK", 1: "WAN_ERR_INVALID_ARG", 2: "WAN_ERR_SHAPE", 3: "WAN_ERR_DTYPE", 4: "WAN_ERR_UNSUPPORTED",
          5: "WAN_ERR_OOM", 6: "WAN_ERR_HIP", 7: "WAN_ERR_MISSING_WEIGHT"}


class WanError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class WanTensor(C.Structure):
    _fields_ = [("data", C.c_void_p), ("dtype", C.c_int32), ("ndim", C.c_int32), ("shape", C.c_int64 * 6)]


class WanWeight(C.Structure):
    _fields_ = [("name", C.c_char_p), ("data", C.c_void_p), ("dtype", C.c_int32), ("ndim", C.c_int32),
                ("shape", C.c_int64 * 6)]


class WanDitConfig(C.Structure):
    _fields_ = [("dim", C.c_int32), ("num_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn_dim", C.c_int32),
                ("num_layers", C.c_int32), ("in_channels", C.c_int32), ("out_channels", C.c_int32),
                ("text_dim", C.c_int32), ("freq_dim", C.c_int32), ("patch_t", C.c_int32), ("patch_h", C.c_int32),
                ("patch_w", C.c_int32), ("rope_dim_t", C.c_int32), ("rope_dim_h", C.c_int32),
                ("rope_dim_w", C.c_int32), ("per_token_timestep", C.c_int32), ("eps", C.c_float),
                ("reserved0", C.c_float), ("rope_theta", C.c_double), ("max_batch", C.c_int64),
                ("max_tokens", C.c_int64), ("max_text_len", C.c_int64), ("max_image_len", C.c_int64),
                ("image_dim", C.c_int32), ("reserved1", C.c_int32)]


_vp, _i64, _i32, _f32, _f64 = C.c_void_p, C.c_int64, C.c_int32, C.c_float, C.c_double


def _sig(name, args, res=C.c_int):
    f = getattr(lib, name)
    f.argtypes = args
    f.restype = res
    return f


_create = _sig("wan_dit_create", [C.POINTER(WanDitConfig), C.POINTER(WanWeight), C.c_size_t, _vp, C.POINTER(_vp)])
_forward = _sig("wan_dit_forward", [_vp, C.POINTER(WanTensor), C.POINTER(WanTensor), C.POINTER(WanTensor),
                                    C.POINTER(WanTensor), _vp])
_forward_image = _sig("wan_dit_forward_image", [_vp, C.POINTER(WanTensor), C.POINTER(WanTensor), C.POINTER(WanTensor),
                                                C.POINTER(WanTensor), C.POINTER(WanTensor), _vp])
_denoise_step = _sig("wan_dit_denoise_step", [_vp, C.POINTER(WanTensor), C.POINTER(WanTensor), C.POINTER(WanTensor),
                                              C.POINTER(WanTensor), _f32, _f32, _f32, C.POINTER(WanTensor), _vp])
_destroy = _sig("wan_dit_destroy", [_vp], None)
_last_error = _sig("wan_dit_last_error", [], C.c_char_p)
_device_bytes = _sig("wan_dit_device_bytes", [_vp], _i64)
_time_attention = _sig("wan_dit_time_attention", [_vp, _i64])
_attention_time = _sig("wan_dit_attention_time", [_vp, C.POINTER(C.c_double), C.POINTER(C.c_int64)])
_op_patchify = _sig("wan_op_patchify", [_vp, _i32, _i64, _i64, _i64, _i64, _i64, _i64, _vp, _vp])
_op_unpatchify = _sig("wan_op_unpatchify", [_vp, _i64, _i64, _i64, _i64, _i64, _i64, _vp, _i32, _vp])
_op_gemm = _sig("wan_op_gemm", [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i32, _vp, _i64, _vp, _vp, _i64, _i64,
                                _vp])
_op_gemm_ws = _sig("wan_op_gemm_ws", [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i32, _vp, _i64, _vp, _vp, _i64, _i64,
                                      _vp, _i64, _vp])
_op_gemm_ws_bytes = _sig("wan_op_gemm_workspace_bytes", [], C.c_int64)
_op_layernorm = _sig("wan_op_layernorm", [_vp, _i64, _i64, _f32, _i32, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp,
                                          _vp, _i32, _vp, _vp, _vp, _i64, _vp, _vp])
_op_rope_table_floats = _sig("wan_op_rope_table_floats", [_i32] * 6, _i64)
_op_rope_table = _sig("wan_op_rope_table", [_vp, _i32, _i32, _i32, _i32, _i32, _i32, _f64, _vp])
_op_qk_norm_rope = _sig("wan_op_qk_norm_rope", [_vp, _i64, _i64, _i64, _f32, _i64, _vp, _i64, _vp, _vp, _i64, _i32,
                                                _i32, _i32, _i32, _i32, _i32, _f32, _vp])
_op_cfg_euler = _sig("wan_op_cfg_euler", [_vp, _i64, _i64, _i64, _i64, _i64, _vp, _i64, _i32, _f32, _f32, _f32, _vp, _vp])
_op_transpose_v = _sig("wan_op_transpose_v", [_vp, _i64, _i64, _i64, _i64, _i32, _vp, _i64, _vp])
_op_attention = _sig("wan_op_attention", [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _i32, _vp])
_op_attention_ws = _sig("wan_op_attention_ws", [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _i32, _vp,
                                                _i64, _vp])
_op_attention_noalloc = _sig("wan_op_attention_noalloc", [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64,
                                                          _i32, _vp])
_op_attention_ws_bytes = _sig("wan_op_attention_workspace_bytes", [_i64, _i64, _i32], C.c_int64)
_op_time_embed = _sig("wan_op_time_embed", [_vp, _i64, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp])
_probe_mfma = _sig("wan_probe_mfma", [_vp, _i32, _i64, _i32, _vp])


class WanVaeConfig(C.Structure):
    _fields_ = [("z_dim", C.c_int32), ("base_dim", C.c_int32), ("chunk_frames", C.c_int32), ("eps", C.c_float),
                ("max_height", C.c_int64), ("max_width", C.c_int64), ("reserved", C.c_int64 * 2)]


_vae_create = _sig("wan_vae_create", [C.POINTER(WanVaeConfig), C.POINTER(WanWeight), C.c_size_t, _vp, C.POINTER(_vp)])
_vae_decode = _sig("wan_vae_decode", [_vp, C.POINTER(WanTensor), C.POINTER(WanTensor), _vp])
_vae_destroy = _sig("wan_vae_destroy", [_vp], None)
_vae_last_error = _sig("wan_vae_last_error", [], C.c_char_p)
_vae_device_bytes = _sig("wan_vae_device_bytes", [_vp], _i64)
_vae_time_convs = _sig("wan_vae_time_convs", [_vp, _i64])
_vae_conv_time = _sig("wan_vae_conv_time", [_vp, C.POINTER(C.c_double), C.POINTER(C.c_int64), C.POINTER(C.c_double)])
_vae_op_packed_elems = _sig("wan_vae_op_packed_conv_elems", [_i64, _i64, _i32, _i32], _i64)
_vae_op_pack_conv = _sig("wan_vae_op_pack_conv", [_vp, _i32, _i64, _i64, _i32, _i32, _vp, _vp])
_vae_op_conv = _sig("wan_vae_op_conv", [C.POINTER(_vp), _i32, _i32, _i32, _vp, _vp, _i64, _i64, _i32, _i64, _i64,
                                        C.POINTER(_vp), C.POINTER(_vp), _i32, _vp])
_vae_op_rms_silu = _sig("wan_vae_op_rms_silu", [C.POINTER(_vp), C.POINTER(_vp), _i32, _i64, _i64, _i64, _vp, _f32, _vp])

EXPORTED = ["wan_dit_create", "wan_dit_forward", "wan_dit_forward_image", "wan_dit_denoise_step", "wan_dit_destroy", "wan_dit_last_error", "wan_dit_device_bytes",
            "wan_dit_time_attention", "wan_dit_attention_time",
            "wan_op_patchify", "wan_op_unpatchify", "wan_op_cfg_euler", "wan_op_gemm", "wan_op_gemm_ws",
            "wan_op_gemm_workspace_bytes", "wan_op_layernorm", "wan_op_rope_table_floats",
            "wan_op_rope_table", "wan_op_qk_norm_rope", "wan_op_transpose_v", "wan_op_attention",
            "wan_op_attention_ws", "wan_op_attention_workspace_bytes", "wan_op_attention_noalloc",
            "wan_op_time_embed", "wan_probe_mfma",
            "wan_vae_create", "wan_vae_decode", "wan_vae_destroy", "wan_vae_last_error", "wan_vae_device_bytes",
            "wan_vae_time_convs", "wan_vae_conv_time",
            "wan_vae_op_packed_conv_elems", "wan_vae_op_pack_conv", "wan_vae_op_conv", "wan_vae_op_rms_silu"]


def last_error() -> str:
    return (_last_error() or b"").decode()


def _check(status: int):
    if status != 0:
        raise WanError(status, last_error())


def _check_vae(status: int):
    if status != 0:
        raise WanError(status, (_vae_last_error() or b"").decode())


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return WAN_F32
    if t.dtype == torch.bfloat16:
        return WAN_BF16
    raise WanError(3, f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def as_wan_tensor(t: torch.Tensor) -> WanTensor:
    if not t.is_contiguous():
        raise WanError(1, "tensors passed to the library must be contiguous")
    w = WanTensor()
    w.data = t.data_ptr()
    w.dtype = _dtype_code(t)
    w.ndim = t.dim()
    for i, s in enumerate(t.shape):
        w.shape[i] = s
    return w


def make_config(cfg, max_batch=None, max_tokens=None, max_text_len=None, num_layers=None) -> WanDitConfig:
    """Fill the C config from a geometry object with the wan_inputs.WanConfig attributes."""
    c = WanDitConfig()
    c.dim, c.num_heads, c.head_dim, c.ffn_dim = cfg.dim, cfg.num_heads, cfg.head_dim, cfg.ffn_dim
    c.num_layers = cfg.num_layers if num_layers is None else num_layers
    c.in_channels, c.out_channels, c.text_dim, c.freq_dim = cfg.in_channels, cfg.out_channels, cfg.text_dim, cfg.freq_dim
    c.patch_t, c.patch_h, c.patch_w = cfg.patch
    c.rope_dim_t, c.rope_dim_h, c.rope_dim_w = cfg.rope_dims
    c.per_token_timestep = 1 if cfg.per_token_t else 0
    c.eps = cfg.eps
    c.rope_theta = cfg.rope_theta
    c.max_batch = max_batch or cfg.batch
    c.max_tokens = max_tokens or cfg.tokens
    c.max_text_len = max_text_len or cfg.text_len
    c.max_image_len = getattr(cfg, "image_len", 0)
    c.image_dim = getattr(cfg, "image_dim", 1280)
    return c


def _weight_array(weights: dict):
    names = list(weights)
    arr = (WanWeight * len(names))()
    keep = []
    for i, n in enumerate(names):
        t = weights[n]
        if not t.is_cuda or not t.is_contiguous():
            raise WanError(1, f"weight {n} must be a contiguous device tensor")
        b = n.encode()
        keep.append(b)
        arr[i].name = b
        arr[i].data = t.data_ptr()
        arr[i].dtype = _dtype_code(t)
        arr[i].ndim = t.dim()
        for j, s in enumerate(t.shape):
            arr[i].shape[j] = s
    return arr, keep


class WanDiT:
    """Handle around wan_dit_create / wan_dit_forward / wan_dit_destroy."""

    def __init__(self, config: WanDitConfig, weights: dict, stream=None):
        arr, self._keep = _weight_array(weights)
        self.config = config
        h = C.c_void_p()
        _check(_create(C.byref(config), arr, len(arr), _stream(stream), C.byref(h)))
        self._h = h

    @property
    def device_bytes(self) -> int:
        return int(_device_bytes(self._h))

    def forward(self, latent: torch.Tensor, timestep: torch.Tensor, text: torch.Tensor, out: torch.Tensor = None,
                stream=None) -> torch.Tensor:
        if out is None:
            b, _, f, hz, wz = latent.shape
            out = torch.empty((b, self.config.out_channels, f, hz, wz), dtype=latent.dtype, device=latent.device)
        lt, tt, xt, ot = (as_wan_tensor(latent), as_wan_tensor(timestep), as_wan_tensor(text), as_wan_tensor(out))
        _check(_forward(self._h, C.byref(lt), C.byref(tt), C.byref(xt), C.byref(ot), _stream(stream)))
        return out

    def forward_image(self, latent: torch.Tensor, timestep: torch.Tensor, text: torch.Tensor, image: torch.Tensor,
                      out: torch.Tensor = None, stream=None) -> torch.Tensor:
        if out is None:
            b, _, f, hz, wz = latent.shape
            out = torch.empty((b, self.config.out_channels, f, hz, wz), dtype=latent.dtype, device=latent.device)
        lt, tt, xt, it, ot = (as_wan_tensor(latent), as_wan_tensor(timestep), as_wan_tensor(text), as_wan_tensor(image),
                              as_wan_tensor(out))
        _check(_forward_image(self._h, C.byref(lt), C.byref(tt), C.byref(xt), C.byref(it), C.byref(ot), _stream(stream)))
        return out

    def denoise_step(self, latent: torch.Tensor, timestep: torch.Tensor, text_pair: torch.Tensor, guidance_scale: float,
                     sigma: float, sigma_next: float, image: torch.Tensor = None, out: torch.Tensor = None,
                     stream=None) -> torch.Tensor:
        """x_next [1, C_out, F, H, W] = x + (sigma_next - sigma) (v_u + s (v_c - v_u)) (wan_dit_denoise_step)."""
        if out is None:
            _, _, f, hz, wz = latent.shape
            out = torch.empty((1, self.config.out_channels, f, hz, wz), dtype=latent.dtype, device=latent.device)
        lt, tt, xt, ot = as_wan_tensor(latent), as_wan_tensor(timestep), as_wan_tensor(text_pair), as_wan_tensor(out)
        it = as_wan_tensor(image) if image is not None else None
        _check(_denoise_step(self._h, C.byref(lt), C.byref(tt), C.byref(xt), C.byref(it) if it is not None else None,
                             guidance_scale, sigma, sigma_next, C.byref(ot), _stream(stream)))
        return out

    def time_attention(self, max_launches: int):
        """Bracket the next `max_launches` self-attention launches of forward() with HIP events (0: off)."""
        _check(_time_attention(self._h, int(max_launches)))

    def attention_time(self):
        """(total milliseconds, launches) of the self-attention launches timed since the last call."""
        ms, n = C.c_double(), C.c_int64()
        _check(_attention_time(self._h, C.byref(ms), C.byref(n)))
        return ms.value, int(n.value)

    def close(self):
        if getattr(self, "_h", None):
            _destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------------------------------------------
# per-stage ops (tensors are torch device tensors; bf16 tensors use torch.bfloat16)
# ------------------------------------------------------------------------------------------------


def op_patchify(latent: torch.Tensor, kp: int, out: torch.Tensor = None, stream=None) -> torch.Tensor:
    b, c, f, hz, wz = latent.shape
    rows = b * f * (hz // 2) * (wz // 2)
    if out is None:
        out = torch.empty((rows, kp), dtype=torch.bfloat16, device=latent.device)
    _check(_op_patchify(latent.data_ptr(), _dtype_code(latent), b, c, f, hz, wz, kp, out.data_ptr(), _stream(stream)))
    return out


def op_unpatchify(z: torch.Tensor, b: int, c: int, f: int, hz: int, wz: int, dtype=torch.float32, stream=None):
    out = torch.empty((b, c, f, hz, wz), dtype=dtype, device=z.device)
    _check(_op_unpatchify(z.data_ptr(), z.shape[1], b, c, f, hz, wz, out.data_ptr(), _dtype_code(out), _stream(stream)))
    return out


def op_gemm(x: torch.Tensor, w: torch.Tensor, bias: torch.Tensor, epilogue: int, out: torch.Tensor,
            gate_tab: torch.Tensor = None, gate_src: torch.Tensor = None, gate_ld: int = 0, rows_per_gate: int = 1,
            stream=None, workspace: torch.Tensor = None):
    """wan_op_gemm, or wan_op_gemm_ws with `workspace` (a device tensor of gemm_workspace_bytes() bytes)."""
    m, k = x.shape
    n = w.shape[0]
    args = (x.data_ptr(), x.stride(0), w.data_ptr(), w.stride(0), bias.data_ptr(), m, n, k, epilogue, out.data_ptr(),
            out.stride(0), _ptr(gate_tab), _ptr(gate_src), gate_ld, rows_per_gate)
    if workspace is None:
        _check(_op_gemm(*args, _stream(stream)))
    else:
        _check(_op_gemm_ws(*args, workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def gemm_workspace_bytes() -> int:
    return int(_op_gemm_ws_bytes())


def op_layernorm(x: torch.Tensor, eps: float, mode: int, out: torch.Tensor, tab_shift=None, tab_scale=None, src=None,
                 src_ld=0, src_shift_off=0, src_scale_off=0, rows_per_src=1, gamma=None, beta=None, res_mode=0,
                 res=None, res_tab=None, res_src=None, res_ld=0, stream=None):
    """x (fp32, updated in place when res_mode > 0) -> out (bf16)."""
    rows, d = x.shape
    _check(_op_layernorm(x.data_ptr(), rows, d, eps, mode, _ptr(tab_shift), _ptr(tab_scale), _ptr(src), src_ld,
                         src_shift_off, src_scale_off, rows_per_src, _ptr(gamma), _ptr(beta), res_mode, _ptr(res),
                         _ptr(res_tab), _ptr(res_src), res_ld, out.data_ptr(), _stream(stream)))
    return out


def op_rope_table(fp: int, hp: int, wp: int, dims=(44, 42, 42), theta: float = 1e4, device="cuda", stream=None):
    n = int(_op_rope_table_floats(fp, hp, wp, *dims))
    tab = torch.empty(n, dtype=torch.float32, device=device)
    _check(_op_rope_table(tab.data_ptr(), fp, hp, wp, *dims, theta, _stream(stream)))
    return tab


def op_qk_norm_rope(buf: torch.Tensor, d: int, eps: float, off_a: int, gamma_a: torch.Tensor, off_b: int = 0,
                    gamma_b: torch.Tensor = None, table: torch.Tensor = None, L: int = 1, grid=(1, 1, 1),
                    dims=(44, 42, 42), scale_a: float = 1.0, stream=None):
    rows = buf.shape[0]
    _check(_op_qk_norm_rope(buf.data_ptr(), buf.stride(0), rows, d, eps, off_a, gamma_a.data_ptr(), off_b,
                            _ptr(gamma_b), _ptr(table), L, *grid, *dims, scale_a, _stream(stream)))
    return buf


def op_cfg_euler(z: torch.Tensor, c: int, x: torch.Tensor, guidance_scale: float, sigma: float, sigma_next: float,
                 stream=None) -> torch.Tensor:
    """z fp32 [2L, >= 4c] (conditional rows first), x [1, Cx, F, H, W] -> x_next [1, c, F, H, W] (x's dtype)."""
    _, cx, f, hz, wz = x.shape
    out = torch.empty((1, c, f, hz, wz), dtype=x.dtype, device=x.device)
    _check(_op_cfg_euler(z.data_ptr(), z.stride(0), c, f, hz, wz, x.data_ptr(), cx, _dtype_code(x), guidance_scale, sigma,
                         sigma_next, out.data_ptr(), _stream(stream)))
    return out


def op_transpose_v(src: torch.Tensor, col_off: int, b: int, L: int, nh: int, ldv: int, stream=None):
    vt = torch.empty((b, nh, 128, ldv), dtype=torch.bfloat16, device=src.device)
    _check(_op_transpose_v(src.data_ptr(), src.stride(0), col_off, b, L, nh, vt.data_ptr(), ldv, _stream(stream)))
    return vt


def op_attention(q: torch.Tensor, k: torch.Tensor, vt: torch.Tensor, out: torch.Tensor, b: int, lq: int, lkv: int,
                 nh: int, stream=None):
    """q, k, out: 2-D views [b*L, >= 128*nh] (row stride from the tensor); vt [b, nh, 128, ldv]."""
    _check(_op_attention(q.data_ptr(), q.stride(0), k.data_ptr(), k.stride(0), vt.data_ptr(), vt.shape[3],
                         out.data_ptr(), out.stride(0), b, lq, lkv, nh, _stream(stream)))
    return out


def attention_workspace_bytes(b: int, lq: int, nh: int) -> int:
    return int(_op_attention_ws_bytes(b, lq, nh))


def op_attention_ws(q: torch.Tensor, k: torch.Tensor, vt: torch.Tensor, out: torch.Tensor, b: int, lq: int, lkv: int,
                    nh: int, workspace: torch.Tensor = None, stream=None):
    """op_attention with a device workspace (allocated here when not given), as the forward runs it:
    offset-free softmax with an exact redo pass, and the last round of workgroups possibly split over
    key chunks and merged."""
    if workspace is None:
        workspace = torch.empty((attention_workspace_bytes(b, lq, nh) + 3) // 4, dtype=torch.float32, device=q.device)
    _check(_op_attention_ws(q.data_ptr(), q.stride(0), k.data_ptr(), k.stride(0), vt.data_ptr(), vt.shape[3],
                            out.data_ptr(), out.stride(0), b, lq, lkv, nh, workspace.data_ptr(),
                            workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def op_attention_noalloc(q: torch.Tensor, k: torch.Tensor, vt: torch.Tensor, out: torch.Tensor, b: int, lq: int, lkv: int,
                         nh: int, stream=None):
    """op_attention_ws with the library's static workspace (wan_op_attention_noalloc: allocates nothing)."""
    _check(_op_attention_noalloc(q.data_ptr(), q.stride(0), k.data_ptr(), k.stride(0), vt.data_ptr(), vt.shape[3],
                                 out.data_ptr(), out.stride(0), b, lq, lkv, nh, _stream(stream)))
    return out


def op_time_embed(t: torch.Tensor, freq_dim: int, d: int, w1, b1, w2, b2, wp, bp, stream=None):
    rows = t.numel()
    temb = torch.empty((rows, d), dtype=torch.float32, device=t.device)
    tproj = torch.empty((rows, 6 * d), dtype=torch.float32, device=t.device)
    work = torch.empty(rows * (freq_dim + d), dtype=torch.float32, device=t.device)
    _check(_op_time_embed(t.data_ptr(), rows, freq_dim, d, w1.data_ptr(), b1.data_ptr(), w2.data_ptr(), b2.data_ptr(),
                          wp.data_ptr(), bp.data_ptr(), temb.data_ptr(), tproj.data_ptr(), work.data_ptr(),
                          _stream(stream)))
    return temb, tproj


def probe_mfma(blocks: int = 1024, rounds: int = 1000, random_operands: bool = True, reps: int = 3, stream=None) -> float:
    """Dense bf16 MFMA throughput (TFLOP/s) of the probe kernel: best of `reps` timed launches after one
    warm-up, HIP events on the stream it runs on."""
    s = stream or torch.cuda.current_stream()
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    flops = blocks * 4 * rounds * 64 * 32768
    best = 0.0
    for i in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        _check(_probe_mfma(sink.data_ptr(), blocks, rounds, int(random_operands), _stream(s)))
        e1.record(s)
        e1.synchronize()
        if i:
            best = max(best, flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return best


# ------------------------------------------------------------------------------------------------
# Wan-VAE causal decoder (include/wan_vae.h)
# ------------------------------------------------------------------------------------------------


def make_vae_config(cfg, chunk_frames: int = 4, max_height: int = None, max_width: int = None) -> WanVaeConfig:
    """Fill the C config from a wan_inputs.vae.VaeConfig."""
    c = WanVaeConfig()
    c.z_dim, c.base_dim, c.chunk_frames, c.eps = cfg.z_dim, cfg.base_dim, chunk_frames, cfg.eps
    c.max_height = max_height or cfg.height
    c.max_width = max_width or cfg.width
    return c


class WanVAE:
    """Handle around wan_vae_create / wan_vae_decode / wan_vae_destroy."""

    def __init__(self, config: WanVaeConfig, weights: dict, stream=None):
        arr, self._keep = _weight_array(weights)
        self.config = config
        h = C.c_void_p()
        _check_vae(_vae_create(C.byref(config), arr, len(arr), _stream(stream), C.byref(h)))
        self._h = h

    @property
    def device_bytes(self) -> int:
        return int(_vae_device_bytes(self._h))

    def decode(self, latent: torch.Tensor, video: torch.Tensor = None, dtype=None, stream=None) -> torch.Tensor:
        """latent [B, 16, F, H, W] -> video [B, 3, 1 + 4 (F - 1), 8H, 8W] (latent's dtype unless given)."""
        if video is None:
            b, _, f, h, w = latent.shape
            video = torch.empty((b, 3, 1 + 4 * (f - 1), 8 * h, 8 * w), dtype=dtype or latent.dtype, device=latent.device)
        lt, vt = as_wan_tensor(latent), as_wan_tensor(video)
        _check_vae(_vae_decode(self._h, C.byref(lt), C.byref(vt), _stream(stream)))
        return video

    def time_convs(self, max_launches: int):
        """Bracket the next `max_launches` 3x3x3 convolution launches (96-channel tiles) of decode() with HIP
        events (0: off)."""
        _check_vae(_vae_time_convs(self._h, int(max_launches)))

    def conv_time(self):
        """(total ms, launches, algorithmic FLOPs) of the convolution launches timed since the last call."""
        ms, n, fl = C.c_double(), C.c_int64(), C.c_double()
        _check_vae(_vae_conv_time(self._h, C.byref(ms), C.byref(n), C.byref(fl)))
        return ms.value, int(n.value), fl.value

    def close(self):
        if getattr(self, "_h", None):
            _vae_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def vae_packed_conv_elems(c_out: int, c_in: int, kt: int, ks: int) -> int:
    return int(_vae_op_packed_elems(c_out, c_in, kt, ks))


def op_vae_pack_conv(w: torch.Tensor, stream=None) -> torch.Tensor:
    """Conv weight [c_out, c_in, kt, ks, ks] (or [c_out, c_in, ks, ks]) -> packed bf16 device tensor."""
    if w.dim() == 4:
        w = w[:, :, None]
    co, ci, kt, ks, _ = w.shape
    out = torch.empty(vae_packed_conv_elems(co, ci, kt, ks), dtype=torch.bfloat16, device=w.device)
    _check_vae(_vae_op_pack_conv(w.contiguous().data_ptr(), _dtype_code(w), co, ci, kt, ks, out.data_ptr(),
                                 _stream(stream)))
    return out


def _ptrs(ts):
    arr = (_vp * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = None if t is None else t.data_ptr()
    return arr


def op_vae_conv(inputs, kt: int, ks: int, up: int, w_packed: torch.Tensor, bias: torch.Tensor, c_in: int, c_out: int,
                split: int, H: int, W: int, outputs, residuals=None, stream=None):
    """wan_vae_op_conv on padded frames: inputs [nf * kt] frame tensors (in[j * kt + dt]), outputs
    [nf * split], residuals None or [nf * split] (entries may be None)."""
    nf = len(outputs) // split
    res = _ptrs(residuals) if residuals is not None else None
    _check_vae(_vae_op_conv(_ptrs(inputs), kt, ks, up, w_packed.data_ptr(), bias.data_ptr(), c_in, c_out, split, H, W,
                            _ptrs(outputs), res, nf, _stream(stream)))


def op_vae_rms_silu(inputs, outputs, c: int, H: int, W: int, gamma: torch.Tensor, eps: float, stream=None):
    _check_vae(_vae_op_rms_silu(_ptrs(inputs), _ptrs(outputs), len(inputs), c, H, W, gamma.data_ptr(), eps,
                                _stream(stream)))
