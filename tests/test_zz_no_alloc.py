"""wan_op_attention_noalloc (the attention entry point that allocates nothing: its workspace is the
library's static device array) against wan_op_attention_ws with a caller workspace, on two calls in a
row, the second smaller, and against the fp64 oracle on sampled rows; plus its size limit."""
import ctypes as C

import numpy as np
import pytest

from oracle import wan_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    import gpu_common

    return gpu_common


def _noalloc(G, q, k, vt, out, b, lq, lkv, nh):
    import torch

    f = G.B.lib.wan_op_attention_noalloc
    vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int32
    f.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, i64, i64, i64, i32, vp]
    f.restype = C.c_int
    return f(q.data_ptr(), q.stride(0), k.data_ptr(), k.stride(0), vt.data_ptr(), vt.shape[3], out.data_ptr(),
             out.stride(0), b, lq, lkv, nh, torch.cuda.current_stream().cuda_stream)


def _case(G, B, L, nh, name, rows):
    import torch

    D = 128 * nh
    qkv, h = G.bf16_dev((B * L, 3 * D), name, 1.0)
    vt = G.B.op_transpose_v(qkv, 2 * D, B, L, nh, (L + 63) // 64 * 64)
    ref_ws = torch.empty((B * L, D), dtype=torch.bfloat16, device="cuda")
    G.B.op_attention_ws(qkv, qkv[:, D:], vt, ref_ws, B, L, L, nh)
    got = torch.full((B * L, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    assert _noalloc(G, qkv, qkv[:, D:], vt, got, B, L, L, nh) == 0, G.B.last_error()
    G.sync()
    g, r = G.to_f64(got), G.to_f64(ref_ws)
    assert np.isfinite(g).all()
    assert G.rel_l2(g, r) < 1e-2 and G.max_abs(g, r) < 2e-2 * max(1.0, np.abs(r).max())
    # and against the oracle (queries rounded as the entry points document: q * log2(e)/sqrt(128) in bf16)
    q, k, v = h[:, :D], h[:, D:2 * D], h[:, 2 * D:]
    for b in range(B):
        qb = q[b * L:(b + 1) * L][rows].reshape(len(rows), nh, 128)
        kb, vb = k[b * L:(b + 1) * L].reshape(L, nh, 128), v[b * L:(b + 1) * L].reshape(L, nh, 128)
        ref = O.attention(qb, kb, vb, workers=4).reshape(len(rows), D)
        gb = g[b * L:(b + 1) * L][rows]
        assert G.rel_l2(gb, ref) < 6e-3 and G.max_abs(gb, ref) < 2e-2 * max(1.0, np.abs(ref).max())


def test_noalloc_matches_workspace_entry_twice_then_smaller(G):
    # first call: 2 x 4000 tokens x 6 heads (192 units: a key-split last round); second: a smaller shape
    G.note("attention noalloc: first call B=2 L=4000 nh=6")
    _case(G, 2, 4000, 6, "na1", np.array([0, 1, 1999, 3999]))
    G.note("attention noalloc: second call B=1 L=777 nh=2")
    _case(G, 1, 777, 2, "na2", np.array([0, 300, 776]))


def test_noalloc_rejects_shapes_beyond_its_workspace(G):
    import torch

    G.note("attention noalloc: limit")
    t = torch.zeros((64, 128 * 40), dtype=torch.bfloat16, device="cuda")
    vt = torch.zeros((1, 40, 128, 64), dtype=torch.bfloat16, device="cuda")
    # 2 x 40 heads x ceil(60000/256) query tiles = 18800 units > 16384 (validation fails before any launch)
    rc = _noalloc(G, t, t, vt, t, 2, 60000, 64, 40)
    assert rc == 4 and "static workspace" in G.B.last_error()
