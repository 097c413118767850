"""Per-stage parity of the HIP kernels against the fp64 oracle, called through the C ABI.

Index kernels (patchify, unpatchify, V transpose) must match bit for bit.  Arithmetic kernels get
per-stage budgets derived from their last rounding step: a bf16 output carries at most 2^-9 relative
rounding error per element (rel-L2 about 1.1e-3 for random data), fp32 outputs only accumulation
error.
"""
import math

import numpy as np
import pytest

from oracle import wan_oracle as O
from wan_inputs import f32_to_bf16_bits

QSCALE = 1.4426950408889634 / math.sqrt(128.0)   # log2(e) / sqrt(128): the scale the attention applies to q

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    import gpu_common  # raises if the HIP library is missing: no fallback

    return gpu_common


def _round_up(a, b):
    return (a + b - 1) // b * b


# ------------------------------------------------------------------------------------------------
# patchify / unpatchify / V transpose: bit-exact
# ------------------------------------------------------------------------------------------------

PATCH_SHAPES = [
    ((1, 16, 5, 16, 16), "f32"),        # tiny reference (fp32 latent)
    ((2, 3, 3, 6, 10), "bf16"),         # ragged, kp padding
    ((2, 16, 21, 60, 104), "bf16"),     # Wan2.1 1.3B, CFG batch 2
    ((1, 36, 9, 44, 80), "bf16"),       # I2V stack
    ((1, 48, 31, 44, 80), "bf16"),      # TI2V-5B
    ((1, 16, 21, 90, 160), "bf16"),     # 14B 720p
]


@pytest.mark.parametrize("shape,dt", PATCH_SHAPES)
def test_patchify_bitexact(G, shape, dt):
    G.note(f"patchify {shape} {dt}")
    t = G.draw_normal(9, f"patch{shape}", shape, dt)
    x = G.to_device(t)
    kp = _round_up(4 * shape[1], 64)
    p = G.B.op_patchify(x, kp)
    G.sync()
    got = G.bf16_bits(p)
    ref = O.patchify(t.f32())                      # exact copy of the stored values, float32
    want = np.zeros((ref.shape[0] * ref.shape[1], kp), dtype=np.uint16)
    want[:, : ref.shape[2]] = f32_to_bf16_bits(ref.reshape(-1, ref.shape[2])).reshape(-1, ref.shape[2])
    assert np.array_equal(got, want)


@pytest.mark.parametrize("shape", [(1, 16, 5, 16, 16), (2, 3, 3, 6, 10), (2, 16, 21, 60, 104), (1, 48, 31, 44, 80)])
@pytest.mark.parametrize("out_dt", ["f32", "bf16"])
def test_unpatchify_bitexact(G, shape, out_dt):
    import torch

    G.note(f"unpatchify {shape} {out_dt}")
    b, c, f, hz, wz = shape
    L = f * (hz // 2) * (wz // 2)
    ldz = 4 * c + 4                                  # a padded row stride
    zt = G.draw_normal(9, f"z{shape}", (b * L, ldz), "f32")
    z = G.to_device(zt)
    out = G.B.op_unpatchify(z, b, c, f, hz, wz, torch.float32 if out_dt == "f32" else torch.bfloat16)
    G.sync()
    ref = O.unpatchify(zt.f32()[:, : 4 * c].reshape(b, L, 4 * c), f, hz, wz, c)
    if out_dt == "f32":
        assert np.array_equal(out.cpu().numpy(), ref)
    else:
        assert np.array_equal(G.bf16_bits(out), f32_to_bf16_bits(ref).reshape(ref.shape))


@pytest.mark.parametrize("B,L,nh,col_off,ld", [(2, 320, 12, 3072, 4608), (1, 1000, 3, 384, 768), (2, 226, 12, 1536, 3072),
                                               (2, 32760, 12, 3072, 4608)])
def test_transpose_v_bitexact(G, B, L, nh, col_off, ld):
    G.note(f"transpose_v B={B} L={L} nh={nh}")
    src, _ = G.bf16_dev((B * L, ld), f"tv{L}")
    ldv = _round_up(L, 64)
    vt = G.B.op_transpose_v(src, col_off, B, L, nh, ldv)
    G.sync()
    s = G.bf16_bits(src)
    want = np.zeros((B, nh, 128, ldv), dtype=np.uint16)
    want[:, :, :, :L] = s.reshape(B, L, ld)[:, :, col_off:col_off + 128 * nh].reshape(B, L, nh, 128).transpose(0, 2, 3, 1)
    assert np.array_equal(G.bf16_bits(vt), want)


# ------------------------------------------------------------------------------------------------
# GEMM + epilogues
# ------------------------------------------------------------------------------------------------

# The last three reach the persistent 256x256 kernel (>= 512 tiles): ragged M (37 rows into a tile) and N
# (8 columns into a tile) with a tile count that does not split evenly over the 8 XCDs; the minimum K of
# 128 (four K stages, no steady-state iteration); and the full block shape.
GEMM_CASES = [(1, 64, 64), (300, 192, 64), (4133, 1536, 1536), (452, 3072, 1536), (1000, 8960, 1536),
              (777, 1536, 8960), (4133, 8968, 1536), (9000, 4104, 128), (65520, 1536, 1536)]


@pytest.mark.parametrize("M,N,K", GEMM_CASES)
@pytest.mark.parametrize("epi", [0, 1, 2, 3, 4])
def test_gemm_epilogues(G, M, N, K, epi):
    import torch

    if M * N > 5e7 and epi not in (0, 4):
        pytest.skip("full-size shape checked with the bf16 and gated epilogues")
    G.note(f"gemm M={M} N={N} K={K} epi={epi}")
    x, xh = G.bf16_dev((M, K), f"gx{M}{K}")
    w, wh = G.bf16_dev((N, K), f"gw{N}{K}", 0.02)
    bt = G.draw_normal(0, f"gb{N}", (N,), "f32", 0.02)
    bias, bh = G.to_device(bt), bt.f64()
    rows = np.arange(M) if M <= 5000 else np.unique(np.concatenate([np.arange(64), np.arange(M - 200, M),
                                                                     np.random.default_rng(0).integers(0, M, 300)]))
    lin = xh[rows] @ wh.T + bh                     # oracle: nn.Linear in float64
    if epi in (0, 1):
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        G.B.op_gemm(x, w, bias, epi, out)
        G.sync()
        got = G.to_f64(out)[rows]
        ref = O.gelu_tanh(lin) if epi == 1 else lin
        # one bf16 rounding of the fp32 result
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5 * np.abs(ref).max())
        assert G.rel_l2(got, ref) < 3e-3
        return
    x0t = G.draw_normal(0, f"gx0{M}{N}", (M, N), "f32")
    out = G.to_device(x0t).clone()
    x0 = x0t.f64()[rows]
    if epi == 2:
        G.B.op_gemm(x, w, bias, epi, out)
        ref = lin
    elif epi == 3:
        G.B.op_gemm(x, w, bias, epi, out)
        ref = x0 + lin
    else:
        L = 100 if M > 100 else 1                 # tokens per gate row
        nsrc = (M + L - 1) // L
        tab_t = G.draw_normal(0, "gtab", (N,), "f32", 0.5)
        src_t = G.draw_normal(0, f"gsrc{nsrc}", (nsrc, 6 * N), "f32", 0.5)
        src = G.to_device(src_t)
        G.B.op_gemm(x, w, bias, epi, out, gate_tab=G.to_device(tab_t), gate_src=src[:, 2 * N:], gate_ld=6 * N,
                    rows_per_gate=L)
        gate = tab_t.f64()[None, :] + src_t.f64()[rows // L, 2 * N:3 * N]
        ref = x0 + lin * gate
    G.sync()
    got = G.to_f64(out)[rows]
    assert G.rel_l2(got - x0 if epi != 2 else got, ref - x0 if epi != 2 else ref) < 1e-5
    assert G.max_abs(got, ref) < 1e-4 * max(1.0, np.abs(ref).max())


# Stream-K tail (wan_op_gemm_ws): the persistent kernel's last round, when at most half full, runs split
# along K.  (9000, 4104, 256): 36 x 17 = 612 tiles, 100 in the tail, 2 chunks of the minimum 4 K stages,
# ragged M and N inside the tail tiles; (27280, 3072, 3072): the TI2V-5B output projections, 1284 tiles,
# 4 in the tail, 24 chunks; (7920, 5120, 13824): the I2V stack's FFN2, 620 tiles, 108 in the tail, 2 chunks
# of 216 stages.
SK_CASES = [(9000, 4104, 256), (27280, 3072, 3072), (7920, 5120, 13824)]


@pytest.mark.parametrize("M,N,K", SK_CASES)
@pytest.mark.parametrize("epi", [0, 1, 2, 3, 4])
def test_gemm_stream_k_tail(G, M, N, K, epi):
    import torch

    if M * K > 1e8 and epi not in (0, 4):
        pytest.skip("largest shape checked with the bf16 and gated epilogues")
    G.note(f"gemm_ws M={M} N={N} K={K} epi={epi}")
    ws = torch.empty(G.B.gemm_workspace_bytes() // 4, dtype=torch.float32, device="cuda")
    x, xh = G.bf16_dev((M, K), f"gx{M}{K}")
    w, wh = G.bf16_dev((N, K), f"gw{N}{K}", 0.02)
    bt = G.draw_normal(0, f"gb{N}", (N,), "f32", 0.02)
    bias, bh = G.to_device(bt), bt.f64()
    # every row of the last tile row (the tail tiles lie there) plus a sample of the rest
    tail_rows = np.arange((M - 1) // 256 * 256, M)
    rows = np.unique(np.concatenate([np.arange(64), tail_rows, np.random.default_rng(0).integers(0, M, 300)]))
    lin = xh[rows] @ wh.T + bh                     # oracle: nn.Linear in float64
    if epi in (0, 1):
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        G.B.op_gemm(x, w, bias, epi, out, workspace=ws)
        G.sync()
        got = G.to_f64(out)[rows]
        ref = O.gelu_tanh(lin) if epi == 1 else lin
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5 * np.abs(ref).max())
        assert G.rel_l2(got, ref) < 3e-3
        # the workspace path differs from the plain one by fp32 summation order only
        plain = torch.empty_like(out)
        G.B.op_gemm(x, w, bias, epi, plain)
        G.sync()
        assert G.rel_l2(G.to_f64(out), G.to_f64(plain)) < 2e-3
        return
    x0t = G.draw_normal(0, f"gx0{M}{N}", (M, N), "f32")
    out = G.to_device(x0t).clone()
    x0 = x0t.f64()[rows]
    if epi == 2:
        G.B.op_gemm(x, w, bias, epi, out, workspace=ws)
        ref = lin
    elif epi == 3:
        G.B.op_gemm(x, w, bias, epi, out, workspace=ws)
        ref = x0 + lin
    else:
        L = 100
        nsrc = (M + L - 1) // L
        tab_t = G.draw_normal(0, "gtab", (N,), "f32", 0.5)
        src_t = G.draw_normal(0, f"gsrc{nsrc}", (nsrc, 6 * N), "f32", 0.5)
        src = G.to_device(src_t)
        G.B.op_gemm(x, w, bias, epi, out, gate_tab=G.to_device(tab_t), gate_src=src[:, 2 * N:], gate_ld=6 * N,
                    rows_per_gate=L, workspace=ws)
        gate = tab_t.f64()[None, :] + src_t.f64()[rows // L, 2 * N:3 * N]
        ref = x0 + lin * gate
    G.sync()
    got = G.to_f64(out)[rows]
    assert G.rel_l2(got - x0 if epi != 2 else got, ref - x0 if epi != 2 else ref) < 1e-5
    assert G.max_abs(got, ref) < 1e-4 * max(1.0, np.abs(ref).max())


def test_gemm_ws_reused_across_calls(G):
    """One workspace, two calls in a row on one stream: a stream-K shape, then a smaller one whose tail
    takes fewer chunks; each matches the plain entry point to fp32 summation order."""
    import torch

    ws = torch.empty(G.B.gemm_workspace_bytes() // 4, dtype=torch.float32, device="cuda")
    for M, N, K in [(27280, 3072, 3072), (9000, 4104, 256)]:
        G.note(f"gemm_ws reuse M={M} N={N} K={K}")
        x, _ = G.bf16_dev((M, K), f"gx{M}{K}")
        w, _ = G.bf16_dev((N, K), f"gw{N}{K}", 0.02)
        bias = G.to_device(G.draw_normal(0, f"gb{N}", (N,), "f32", 0.02))
        out = torch.empty((M, N), dtype=torch.float32, device="cuda")
        plain = torch.empty_like(out)
        G.B.op_gemm(x, w, bias, 2, out, workspace=ws)
        G.B.op_gemm(x, w, bias, 2, plain)
        G.sync()
        assert G.rel_l2(G.to_f64(out), G.to_f64(plain)) < 1e-6
        assert G.max_abs(G.to_f64(out), G.to_f64(plain)) < 1e-5 * max(1.0, float(plain.abs().max()))


def test_gemm_ws_rejects_bad_workspace(G):
    import torch

    x = torch.zeros((1024, 256), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((1024, 256), dtype=torch.bfloat16, device="cuda")
    bias = torch.zeros(1024, dtype=torch.float32, device="cuda")
    out = torch.zeros((1024, 1024), dtype=torch.bfloat16, device="cuda")
    short = torch.empty(16, dtype=torch.float32, device="cuda")
    with pytest.raises(RuntimeError, match="workspace"):
        G.B.op_gemm(x, w, bias, 0, out, workspace=short)


# ------------------------------------------------------------------------------------------------
# LayerNorm + modulation
# ------------------------------------------------------------------------------------------------


@pytest.mark.parametrize("rows,D", [(300, 1536), (1000, 3072), (77, 5120), (65520, 1536)])
@pytest.mark.parametrize("mode", ["sample", "token", "affine", "head"])
def test_layernorm(G, rows, D, mode):
    import torch

    G.note(f"layernorm rows={rows} D={D} mode={mode}")
    xt = G.draw_normal(1, f"lnx{rows}{D}", (rows, D), "f32", 2.0)
    xh = xt.f64() + 0.75                          # non-zero mean
    x = torch.from_numpy(xh.astype(np.float32)).cuda()
    xh = xh.astype(np.float32).astype(np.float64)
    y = torch.empty((rows, D), dtype=torch.bfloat16, device="cuda")
    eps = 1e-6
    ln = O.layer_norm(xh, eps)
    if mode == "affine":
        g_t = G.draw_uniform(1, "lng", (D,), 0.5, 1.5)
        b_t = G.draw_normal(1, "lnb", (D,), "f32", 0.02)
        G.B.op_layernorm(x, eps, 1, y, gamma=G.to_device(g_t), beta=G.to_device(b_t))
        ref = ln * g_t.f64() + b_t.f64()
    else:
        nsl = 6 if mode != "head" else 1
        tab_t = G.draw_normal(1, "lntab", (nsl if mode != "head" else 2, D), "f32", 1.0 / math.sqrt(D))
        L = 1 if mode == "token" else 100
        nsrc = (rows + L - 1) // L
        src_t = G.draw_normal(1, f"lnsrc{nsrc}{D}", (nsrc, nsl * D), "f32", 0.3)
        tab, src = G.to_device(tab_t), G.to_device(src_t)
        if mode == "head":
            G.B.op_layernorm(x, eps, 0, y, tab_shift=tab[0], tab_scale=tab[1], src=src, src_ld=D, src_shift_off=0,
                             src_scale_off=0, rows_per_src=L)
            s = src_t.f64()[np.arange(rows) // L]
            shift, scale = tab_t.f64()[0] + s, tab_t.f64()[1] + s
        else:
            G.B.op_layernorm(x, eps, 0, y, tab_shift=tab[3], tab_scale=tab[4], src=src, src_ld=6 * D,
                             src_shift_off=3 * D, src_scale_off=4 * D, rows_per_src=L)
            s = src_t.f64()[np.arange(rows) // L]
            shift, scale = tab_t.f64()[3] + s[:, 3 * D:4 * D], tab_t.f64()[4] + s[:, 4 * D:5 * D]
        ref = ln * (1.0 + scale) + shift
    G.sync()
    got = G.to_f64(y)
    assert G.rel_l2(got, ref) < 3e-3
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4 * np.abs(ref).max())


# ------------------------------------------------------------------------------------------------
# QK RMSNorm + 3D RoPE
# ------------------------------------------------------------------------------------------------


def test_rope_table(G):
    G.note("rope table")
    fp, hp, wp = 21, 30, 52
    tab = G.B.op_rope_table(fp, hp, wp).cpu().numpy().astype(np.float64)
    ang = O.rope_angles(fp, hp, wp)
    n = fp * 22 + hp * 21 + wp * 21
    cos, sin = tab[:n], tab[n:]
    # rebuild the per-token angle table from the per-axis rows and compare with the oracle
    f_idx, h_idx, w_idx = np.meshgrid(np.arange(fp), np.arange(hp), np.arange(wp), indexing="ij")
    f_idx, h_idx, w_idx = f_idx.ravel(), h_idx.ravel(), w_idx.ravel()
    ct = cos[: fp * 22].reshape(fp, 22)
    ch = cos[fp * 22: fp * 22 + hp * 21].reshape(hp, 21)
    cw = cos[fp * 22 + hp * 21:].reshape(wp, 21)
    st = sin[: fp * 22].reshape(fp, 22)
    sh = sin[fp * 22: fp * 22 + hp * 21].reshape(hp, 21)
    sw = sin[fp * 22 + hp * 21:].reshape(wp, 21)
    c_all = np.concatenate([ct[f_idx], ch[h_idx], cw[w_idx]], axis=1)
    s_all = np.concatenate([st[f_idx], sh[h_idx], sw[w_idx]], axis=1)
    assert np.abs(c_all - np.cos(ang)).max() < 1e-7 and np.abs(s_all - np.sin(ang)).max() < 1e-7


@pytest.mark.parametrize("B,grid,D,scale_a", [(1, (5, 8, 8), 1536, 1.0), (2, (3, 6, 10), 3072, 1.0),
                                              (1, (9, 22, 40), 5120, 1.0), (2, (21, 30, 52), 1536, 1.0),
                                              (1, (5, 8, 8), 1536, QSCALE)])
def test_qk_norm_rope(G, B, grid, D, scale_a):
    G.note(f"qk_norm_rope B={B} grid={grid} D={D} scale_a={scale_a}")
    fp, hp, wp = grid
    L = fp * hp * wp
    rows = B * L
    buf, bh = G.bf16_dev((rows, 3 * D), f"qkb{rows}{D}", 0.05)
    gq_t, gk_t = G.draw_uniform(2, "gq", (D,), 0.5, 1.5), G.draw_uniform(2, "gk", (D,), 0.5, 1.5)
    v_before = G.bf16_bits(buf)[:, 2 * D:].copy()
    tab = G.B.op_rope_table(fp, hp, wp)
    G.B.op_qk_norm_rope(buf, D, 1e-6, 0, G.to_device(gq_t), D, G.to_device(gk_t), tab, L, grid, scale_a=scale_a)
    G.sync()
    out_bits = G.bf16_bits(buf)
    assert np.array_equal(out_bits[:, 2 * D:], v_before)        # V untouched
    got = G.to_f64(buf)
    sel = np.arange(rows) if rows <= 20000 else np.unique(np.random.default_rng(1).integers(0, rows, 2000))
    ang = O.rope_angles(fp, hp, wp)
    for seg, g_t in ((0, gq_t), (1, gk_t)):
        u = O.rms_norm(bh[sel, seg * D:(seg + 1) * D], 1e-6, g_t.f64()) * (scale_a if seg == 0 else 1.0)
        # rotate row by row with the oracle (each row has its own token position)
        ref = np.empty_like(u)
        for i in range(len(sel)):
            ref[i] = O.apply_rope(u[i].reshape(1, D // 128, 128), ang[[sel[i] % L]]).reshape(D)
        g = got[sel, seg * D:(seg + 1) * D]
        assert G.rel_l2(g, ref) < 3e-3
        assert np.all(np.abs(g - ref) <= 2.0 ** -8 * np.abs(ref) + 2e-3 * np.abs(ref).max())


def test_rms_norm_single_segment(G):
    G.note("rms single segment")
    D, rows = 5120, 1024
    buf, bh = G.bf16_dev((rows, 2 * D), "rms1", 0.05)
    g_t = G.draw_uniform(2, "g2", (D,), 0.5, 1.5)
    keep = G.bf16_bits(buf)[:, D:].copy()
    G.B.op_qk_norm_rope(buf, D, 1e-6, 0, G.to_device(g_t))
    G.sync()
    assert np.array_equal(G.bf16_bits(buf)[:, D:], keep)
    ref = O.rms_norm(bh[:, :D], 1e-6, g_t.f64())
    assert G.rel_l2(G.to_f64(buf)[:, :D], ref) < 3e-3


# ------------------------------------------------------------------------------------------------
# attention
# ------------------------------------------------------------------------------------------------


def _scaled_q_reference(q):
    """q * log2(e)/sqrt(128) rounded to bf16 (nearest even), expressed back in natural units."""
    from wan_inputs import bf16_bits_to_f32

    qs = (q * QSCALE).astype(np.float32)
    return bf16_bits_to_f32(f32_to_bf16_bits(qs)).astype(np.float64).reshape(q.shape) / QSCALE


def _attn_case(G, B, Lq, Lkv, nh, fused, name, scale=1.0, rows=None, split=False, q_round=False):
    import torch

    D = 128 * nh
    if fused:                                     # self-attention layout: q | k | v in one [B*L, 3D] buffer
        assert Lq == Lkv
        qkv, qh = G.bf16_dev((B * Lq, 3 * D), name, scale)
        q, k = qkv, qkv[:, D:]
        kh = qh[:, D:2 * D]
        vh = qh[:, 2 * D:]
        qh = qh[:, :D]
        vt = G.B.op_transpose_v(qkv, 2 * D, B, Lkv, nh, _round_up(Lkv, 64))
    else:                                         # cross layout: q [B*Lq, D], kv [B*Lkv, 2D]
        q, qh = G.bf16_dev((B * Lq, D), name + "q", scale)
        kv, kvh = G.bf16_dev((B * Lkv, 2 * D), name + "kv", scale)
        k = kv
        kh, vh = kvh[:, :D], kvh[:, D:]
        vt = G.B.op_transpose_v(kv, D, B, Lkv, nh, _round_up(Lkv, 64))
    out = torch.empty((B * Lq, D), dtype=torch.bfloat16, device="cuda")
    if split:
        G.B.op_attention_ws(q, k, vt, out, B, Lq, Lkv, nh)
    else:
        G.B.op_attention(q, k, vt, out, B, Lq, Lkv, nh)
    G.sync()
    got = G.to_f64(out)
    for b in range(B):
        sel = np.arange(Lq) if rows is None else rows
        qb = qh[b * Lq:(b + 1) * Lq][sel].reshape(len(sel), nh, 128)
        if q_round:
            qb = _scaled_q_reference(qb)
        kb = kh[b * Lkv:(b + 1) * Lkv].reshape(Lkv, nh, 128)
        vb = vh[b * Lkv:(b + 1) * Lkv].reshape(Lkv, nh, 128)
        ref = O.attention(qb, kb, vb, workers=4).reshape(len(sel), D)
        g = got[b * Lq:(b + 1) * Lq][sel]
        assert G.rel_l2(g, ref) < 6e-3, (b, G.rel_l2(g, ref))
        assert G.max_abs(g, ref) < 2e-2 * max(1.0, np.abs(ref).max())


@pytest.mark.parametrize("B,L,nh", [(1, 320, 12), (2, 1000, 3), (1, 64, 2), (1, 1, 1), (1, 100, 2), (2, 129, 4),
                                    (1, 7920, 2)])
def test_self_attention(G, B, L, nh):
    G.note(f"self attention B={B} L={L} nh={nh}")
    _attn_case(G, B, L, L, nh, True, f"sa{B}_{L}_{nh}")


@pytest.mark.parametrize("B,Lq,Lkv,nh", [(2, 320, 226, 12), (1, 1000, 512, 4), (2, 77, 1, 2), (1, 200, 64, 3),
                                          (1, 150, 70, 2)])
def test_cross_attention(G, B, Lq, Lkv, nh):
    G.note(f"cross attention B={B} Lq={Lq} Lkv={Lkv} nh={nh}")
    _attn_case(G, B, Lq, Lkv, nh, False, f"ca{B}_{Lq}_{Lkv}_{nh}")


# Key-split last round: every case below has fewer (batch, head, query-tile) units than half the CUs, so
# all of them run as key chunks (multiples of 64 keys, the last one ragged) merged by the combine pass.
@pytest.mark.parametrize("B,Lq,Lkv,nh,fused", [(1, 1000, 1000, 3, True), (2, 320, 320, 12, True), (1, 129, 129, 2, True),
                                               (1, 64, 64, 1, True), (2, 300, 226, 4, False), (1, 200, 70, 2, False),
                                               (1, 700, 1, 1, False)])
def test_attention_key_split(G, B, Lq, Lkv, nh, fused):
    G.note(f"attention key split B={B} Lq={Lq} Lkv={Lkv} nh={nh}")
    _attn_case(G, B, Lq, Lkv, nh, fused, f"ks{B}_{Lq}_{Lkv}_{nh}", split=True)


def test_cross_attention_resident_many_units(G):
    """More (batch, head, query-tile) units than CUs with the workspace path: the persistent cross kernel
    (text keys resident in LDS) walks several units per workgroup across head changes, with a ragged
    last query tile; sampled query rows of every batch element against the oracle."""
    G.note("cross attention resident, many units")
    rows = np.unique(np.concatenate([np.arange(0, 8200, 37), np.arange(8150, 8200)]))
    _attn_case(G, 2, 8200, 226, 12, False, "xres", rows=rows, split=True)
    _attn_case(G, 1, 2000, 256, 5, False, "xres256", split=True)


def test_attention_key_split_peaked(G):
    """Scores in the tens with chunked keys: the merge rescales chunks whose running maxima differ."""
    G.note("attention key split peaked")
    _attn_case(G, 1, 500, 500, 2, True, "kspeaked", scale=3.0, split=True)


def test_attention_out_of_range_scores_redone_exactly(G):
    """Scores of hundreds of base-2 units: the offset-free softmax leaves its range in every wave, so the
    workspace path drops those results and its exact running-max pass recomputes them (with and without a
    key-split last round); the plain entry point runs the exact kernel alone.  At such magnitudes the
    near one-hot softmax follows the one bf16 rounding of q * log2(e)/sqrt(128) the entry points apply
    (documented with them), so the reference takes the queries rounded that way."""
    G.note("attention out-of-range scores")
    for B, L, nh, split in ((1, 700, 3, True), (2, 2100, 4, True), (1, 500, 2, False)):
        _attn_case(G, B, L, L, nh, True, f"oor{B}_{L}", scale=8.0, split=split, q_round=True)
    _attn_case(G, 1, 300, 226, 2, False, "oorx", scale=8.0, split=True, q_round=True)


def test_attention_peaked_scores(G):
    """Large-magnitude q/k (scores in the tens): exercises the running max and rescaling."""
    G.note("attention peaked")
    _attn_case(G, 1, 500, 500, 2, True, "peaked", scale=3.0)


def test_self_attention_full_size_sampled(G):
    """Wan2.1-1.3B geometry: B=2, 12 heads, 32760 tokens; sampled query rows against the oracle."""
    G.note("self attention full size B=2 L=32760 nh=12")
    rows = np.unique(np.concatenate([np.arange(3), [32700, 32759], np.random.default_rng(3).integers(0, 32760, 8)]))
    _attn_case(G, 2, 32760, 32760, 12, True, "safull", rows=rows)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("L,nh", [(75600, 40), (27280, 24)])
def test_self_attention_largest_sampled(G, L, nh):
    """The largest self-attention shapes (Wan-14B 720p: 75600 tokens, 40 heads, 46 rounds of workgroups and
    64 more; TI2V-5B: 27280 tokens, 24 heads, 10 rounds and 8 more), launched with the workspace as the
    forward launches them, so the last round runs key-split; sampled query rows against the oracle."""
    G.note(f"self attention largest B=1 L={L} nh={nh} (key split)")
    rows = np.unique(np.concatenate([np.arange(2), [L - 300, L - 1], np.random.default_rng(5).integers(0, L, 6)]))
    _attn_case(G, 1, L, L, nh, True, f"salarge{L}", rows=rows, split=True)


# ------------------------------------------------------------------------------------------------
# timestep embedding (fp32)
# ------------------------------------------------------------------------------------------------


# Key counts around the 64-key LDS tile and the 32-key sub-tile, query counts around the 256-query
# workgroup; each through the plain entry point and through the one with a workspace, which splits
# these small launches into 64-key chunks (65 keys: a last chunk of one key).
_EDGE_CASES = [
    (1, 31, 31, 1, True), (1, 33, 33, 1, True), (1, 63, 63, 1, True), (1, 65, 65, 1, True),
    (1, 96, 96, 1, True), (1, 127, 127, 1, True), (1, 255, 255, 1, True), (1, 257, 257, 1, True),
    (2, 256, 256, 1, True), (1, 513, 513, 1, True),
    (1, 255, 2, 1, False), (1, 257, 32, 1, False), (2, 100, 33, 2, False), (1, 300, 95, 1, False),
    (1, 40, 97, 1, False), (1, 512, 321, 1, False), (1, 1, 129, 1, False),
]


@pytest.mark.parametrize("split", [False, True])
def test_attention_tile_edges(G, split):
    for i, (B, Lq, Lkv, nh, fused) in enumerate(_EDGE_CASES):
        G.note(f"attention edge case B={B} Lq={Lq} Lkv={Lkv} nh={nh} fused={fused} split={split}")
        _attn_case(G, B, Lq, Lkv, nh, fused, f"edge{i}", split=split)


@pytest.mark.parametrize("rows,D,per_token", [(2, 1536, False), (1, 5120, False), (2000, 3072, True)])
def test_time_embed(G, rows, D, per_token):
    import torch

    G.note(f"time embed rows={rows} D={D}")
    if per_token:
        t_t = G.draw_uniform(3, "tt", (rows,), 0.0, 999.9)
    else:
        t_t = None
    t_h = t_t.f64() if per_token else np.full(rows, 500.0)
    t = G.to_device(t_t) if per_token else torch.full((rows,), 500.0, device="cuda")
    ws = {}
    for n, shp in (("w1", (D, 256)), ("b1", (D,)), ("w2", (D, D)), ("b2", (D,)), ("wp", (6 * D, D)), ("bp", (6 * D,))):
        ws[n] = G.draw_normal(3, f"te{n}{D}", shp, "f32", 0.02)
    dev = {n: G.to_device(v) for n, v in ws.items()}
    temb, tproj = G.B.op_time_embed(t, 256, D, dev["w1"], dev["b1"], dev["w2"], dev["b2"], dev["wp"], dev["bp"])
    G.sync()
    w = {"time_embedder.linear_1.weight": ws["w1"].f64(), "time_embedder.linear_1.bias": ws["b1"].f64(),
         "time_embedder.linear_2.weight": ws["w2"].f64(), "time_embedder.linear_2.bias": ws["b2"].f64(),
         "time_proj.weight": ws["wp"].f64(), "time_proj.bias": ws["bp"].f64()}
    r_temb, r_tproj = O.time_embed(t_h, w)
    assert G.rel_l2(G.to_f64(temb), r_temb) < 1e-4
    assert G.rel_l2(G.to_f64(tproj), r_tproj.reshape(rows, 6 * D)) < 1e-4


@pytest.mark.parametrize("rows,D,res_mode,per_token", [(300, 1536, 1, False), (1000, 3072, 2, False),
                                                       (257, 5120, 2, True), (65520, 1536, 2, False),
                                                       (301, 1536, 2, True), (77, 512, 1, False)])
def test_layernorm_with_residual(G, rows, D, res_mode, per_token):
    """x += r (res_mode 1) or x += r * (tab + src[row]) (res_mode 2), then LN + modulation."""
    import torch

    G.note(f"layernorm residual rows={rows} D={D} res_mode={res_mode} per_token={per_token}")
    xt = G.draw_normal(4, f"lrx{rows}{D}", (rows, D), "f32", 1.5)
    x = G.to_device(xt).clone()
    r, rh = G.bf16_dev((rows, D), f"lrr{rows}{D}", 0.7)
    # 99 rows per sample: sample boundaries fall inside the row pairs of the two-rows-per-wave kernel
    L = 1 if per_token else 99
    nsrc = (rows + L - 1) // L
    tab_t = G.draw_normal(4, "lrtab", (6, D), "f32", 1.0 / math.sqrt(D))
    src_t = G.draw_normal(4, f"lrsrc{nsrc}{D}", (nsrc, 6 * D), "f32", 0.3)
    tab, src = G.to_device(tab_t), G.to_device(src_t)
    y = torch.empty((rows, D), dtype=torch.bfloat16, device="cuda")
    G.B.op_layernorm(x, 1e-6, 0, y, tab_shift=tab[0], tab_scale=tab[1], src=src, src_ld=6 * D, src_shift_off=0,
                     src_scale_off=D, rows_per_src=L, res_mode=res_mode, res=r, res_tab=tab[2],
                     res_src=src[:, 2 * D:], res_ld=6 * D)
    G.sync()
    s = src_t.f64()[np.arange(rows) // L]
    gate = tab_t.f64()[2] + s[:, 2 * D:3 * D]
    x_ref = xt.f64() + (rh * gate if res_mode == 2 else rh)
    x_got = G.to_f64(x)
    # fp32 update: one rounding of the sum
    assert np.abs(x_got - x_ref).max() <= 2.0 ** -22 * np.abs(x_ref).max()
    ref = O.layer_norm(x_ref, 1e-6) * (1.0 + tab_t.f64()[1] + s[:, D:2 * D]) + tab_t.f64()[0] + s[:, :D]
    got = G.to_f64(y)
    assert G.rel_l2(got, ref) < 3e-3


def test_mfma_probe(G):
    """The MFMA throughput probe runs, zero operands give exactly zero sums, random ones finite sums, and
    the measured rate is plausible for one device (below 3 PFLOP/s, above 100 TFLOP/s)."""
    import torch

    G.note("mfma probe")
    sink = torch.full((64 * 256,), float("nan"), dtype=torch.float32, device="cuda")
    assert G.B._probe_mfma(sink.data_ptr(), 64, 8, 0, G.B._stream(None)) == 0
    G.sync()
    assert torch.count_nonzero(sink).item() == 0
    assert G.B._probe_mfma(sink.data_ptr(), 64, 8, 1, G.B._stream(None)) == 0
    G.sync()
    assert torch.isfinite(sink).all().item() and torch.count_nonzero(sink).item() > 0
    tf = G.B.probe_mfma(blocks=256, rounds=50, random_operands=True, reps=1)
    assert 100.0 < tf < 3000.0, tf
    with pytest.raises(G.B.WanError):
        G.B._check(G.B._probe_mfma(sink.data_ptr(), 0, 8, 0, G.B._stream(None)))
