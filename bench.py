"""Benchmark of the Wan DiT forward on one MI355X.

A step is one wan_dit_forward: one denoising step's DiT work (patch embed, time/text embedding, all
blocks, head, unpatchify) on seeded synthetic inputs already resident in HBM.  Default workload: the
Wan2.1-T2V-1.3B geometry with the CFG pair as batch 2 (2 x 32760 tokens, 30 blocks, bf16).

Prints one JSON line.  `value` is the achieved throughput in TFLOP/s of algorithmic work (GEMM and
attention FLOPs) per step; `ms_per_step` the mean step time.  `roofline` reports the dominant kernel
(self-attention) timed with HIP events that the library records around each of its launches inside
the timed steps, on the stream the forward runs on (`wan_dit_time_attention`), and
`cpu_baseline` the fp64 oracle on a bounded sample of the same workload, scaled to a full step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def step_flops(cfg, B=None, L=None) -> dict:
    """Algorithmic FLOPs of one forward: 2*M*N*K per GEMM, 4*B*Lq*Lkv*D per attention."""
    B = B or cfg.batch
    L = L or cfg.tokens
    D, Fd, Lt, N = cfg.dim, cfg.ffn_dim, cfg.text_len, cfg.num_layers
    M = B * L
    R = M if cfg.per_token_t else B
    f = {}
    f["patch_embed"] = 2 * M * cfg.patch_k * D
    f["time_mlp_fp32"] = 2 * R * (cfg.freq_dim * D + D * D + 6 * D * D)
    f["text_proj"] = 2 * B * Lt * (cfg.text_dim * D + D * D)
    per_block = {
        "qkv": 2 * M * D * 3 * D, "o": 2 * M * D * D, "q2": 2 * M * D * D, "kv2": 2 * B * Lt * D * 2 * D,
        "o2": 2 * M * D * D, "ffn": 2 * 2 * M * D * Fd, "self_attn": 4 * B * L * L * D, "cross_attn": 4 * B * L * Lt * D,
    }
    for k, v in per_block.items():
        f[k] = v * N
    f["proj_out"] = 2 * M * D * cfg.out_k
    f["total"] = sum(f.values())
    return f


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "video_diffusion_transformer_patchify_amd", "csrc", n), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel_file: str):
    """HBM bytes per launch measured with rocprofv3 counters, if recorded for the current source."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p)).get(kernel_file)
    if not rec or rec.get("source_hash") != source_hash(kernel_file, "common.h"):
        return None
    return rec.get("bytes_per_launch")


def time_self_attention(B, cfg, reps, stream):
    """Average duration of the self-attention kernel at the workload's shape, HIP events on its stream; launched
    as the forward launches it (with its workspace, so a short last round of workgroups is key-split)."""
    import torch

    from video_diffusion_transformer_patchify_amd import binding as Bd

    D, nh, L = cfg.dim, cfg.num_heads, cfg.tokens
    g = torch.Generator(device="cuda").manual_seed(0)
    qkv = (torch.randn((B * L, 3 * D), generator=g, device="cuda") * 1.0).to(torch.bfloat16)
    ldv = (L + 63) // 64 * 64
    vt = Bd.op_transpose_v(qkv, 2 * D, B, L, nh, ldv, stream=stream)
    out = torch.empty((B * L, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((Bd.attention_workspace_bytes(B, L, nh) + 3) // 4, dtype=torch.float32, device="cuda")
    for _ in range(2):
        Bd.op_attention_ws(qkv, qkv[:, D:], vt, out, B, L, L, nh, workspace=ws, stream=stream)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(reps):
        Bd.op_attention_ws(qkv, qkv[:, D:], vt, out, B, L, L, nh, workspace=ws, stream=stream)
    ev1.record(stream)
    ev1.synchronize()
    ms = ev0.elapsed_time(ev1) / reps
    del qkv, vt, out, ws
    return ms


def cpu_baseline(cfg, budget_s: float):
    """fp64 oracle on a bounded sample of the workload's own seeded inputs, scaled to one full step.

    The embeddings (patch, time, text) run once in full.  A block costs a + b*L: the part over all L
    tokens that self-attention needs (LN1 and the keys and values with their norm and rotation: a,
    timed alone with the oracle's own functions) plus the per-token rest - the query, its self-attention
    over all keys, cross-attention, FFN (b per token, from oracle.block_forward_rows on R token rows of
    block 0, batch element 0, minus a).  The step is batch * (embeddings + blocks * (a + b*L)).  Each term
    is counted once."""
    import numpy as np

    from oracle import wan_oracle as O
    from wan_inputs import Weights, draw_inputs

    threads = len(os.sched_getaffinity(0))
    one = cfg.replace(batch=1, num_layers=1)
    w = Weights(one)
    lat, t, txt = draw_inputs(one)
    for n in w.names():
        w.f64(n)
    t0 = time.perf_counter()
    x = O.patch_embed(lat.f64(), w.f64("patch_embedding.weight"), w.f64("patch_embedding.bias"))
    temb, tproj = O.time_embed(t.f64(), w, one.freq_dim)
    ctx = O.text_embed(txt.f64(), w)
    ang = O.rope_angles(one.post_f, one.post_h, one.post_w, one.head_dim, one.rope_dims, one.rope_theta)
    t_embed = time.perf_counter() - t0
    L, D, nh, p = one.tokens, one.dim, one.num_heads, "blocks.0."
    # a: the all-token part, the same calls block_forward_rows makes for it
    t1 = time.perf_counter()
    sh1, sc1 = O.modulation(w.f64(p + "scale_shift_table"), tproj)[:2]
    y = O.layer_norm(x, one.eps) * (1.0 + sc1) + sh1
    k = O.rms_norm(O.linear(y, w.f64(p + "attn1.to_k.weight"), w.f64(p + "attn1.to_k.bias")), one.eps,
                   w.f64(p + "attn1.norm_k.weight"))
    O.linear(y, w.f64(p + "attn1.to_v.weight"), w.f64(p + "attn1.to_v.bias"))
    O.apply_rope(k[0].reshape(L, nh, D // nh), ang)
    a = time.perf_counter() - t1
    del y, k
    # a + b R: the block on R token rows
    r = min(2048, L)
    rows = np.sort(np.random.default_rng(0).choice(L, r, replace=False))
    t2 = time.perf_counter()
    O.block_forward_rows(x, ctx, tproj, ang, w, p, nh, rows, one.eps, workers=threads)
    t_rows = time.perf_counter() - t2
    b = max(t_rows - a, 0.0) / r
    est_step = cfg.batch * (t_embed + cfg.num_layers * (a + b * L))
    sample_s = t_embed + a + t_rows
    return est_step, sample_s, threads, (r, a, b, t_embed)


def probe(cfg):
    """One launch each of the kernels whose HBM traffic is read from rocprofv3 counters, plus a plain
    1 GiB device copy (read 1 GiB, write 1 GiB) that calibrates FETCH_SIZE / WRITE_SIZE."""
    import torch

    from video_diffusion_transformer_patchify_amd import binding as Bd

    torch.cuda.set_device(0)
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")        # 1 GiB
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    B, L, D, nh, Fd = cfg.batch, cfg.tokens, cfg.dim, cfg.num_heads, cfg.ffn_dim
    M = B * L
    g = torch.Generator(device="cuda").manual_seed(0)
    qkv = torch.randn((M, 3 * D), generator=g, device="cuda").to(torch.bfloat16)
    ldv = (L + 63) // 64 * 64
    vt = Bd.op_transpose_v(qkv, 2 * D, B, L, nh, ldv)
    out = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    Bd.op_attention_ws(qkv, qkv[:, D:], vt, out, B, L, L, nh)    # as the forward runs it
    torch.cuda.synchronize()
    x = torch.randn((M, D), generator=g, device="cuda")
    tab = torch.zeros((6, D), device="cuda")
    tsrc = torch.zeros((B, 6 * D), device="cuda")
    Bd.op_layernorm(x, 1e-6, 0, out, tab_shift=tab[0], tab_scale=tab[1], src=tsrc, src_ld=6 * D, src_shift_off=0,
                    src_scale_off=D, rows_per_src=L)
    torch.cuda.synchronize()
    w1 = (torch.randn((Fd, D), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    b1 = torch.zeros(Fd, device="cuda")
    h = torch.empty((M, Fd), dtype=torch.bfloat16, device="cuda")
    Bd.op_gemm(out, w1, b1, Bd.EPI_GELU_BF16, h)
    torch.cuda.synchronize()
    print("probe done", flush=True)


def vendor_reference(cfg):
    """Context, not part of the headline: the vendor libraries on the workload's shapes, same process.
    Each GEMM of the block runs through this library and through hipBLASLt (torch.matmul, bf16 out)
    on identical inputs; self-attention through this library and through torch's SDPA."""
    import torch

    from video_diffusion_transformer_patchify_amd import binding as Bd

    def timed(f, reps):
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    torch.cuda.set_device(0)
    B, L, D, nh, Fd = cfg.batch, cfg.tokens, cfg.dim, cfg.num_heads, cfg.ffn_dim
    M = B * L
    g = torch.Generator(device="cuda").manual_seed(0)
    res = {"gemm": [], "attention": {}}
    for name, N, K in (("qkv", 3 * D, D), ("o", D, D), ("ffn1", Fd, D), ("ffn2", D, Fd)):
        x = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
        w = (torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        wt = w.t()
        b = torch.zeros(N, device="cuda")
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        ours = timed(lambda: Bd.op_gemm(x, w, b, Bd.EPI_BF16, out), 10)
        blas = timed(lambda: torch.matmul(x, wt, out=out), 10)
        fl = 2.0 * M * N * K
        res["gemm"].append({"name": name, "M": M, "N": N, "K": K, "ours_ms": round(ours, 4),
                            "hipblaslt_ms": round(blas, 4), "ours_tflops": round(fl / ours / 1e9, 1),
                            "hipblaslt_tflops": round(fl / blas / 1e9, 1)})
        del x, w, wt, out
    fl = 4.0 * B * L * L * D
    qkv = torch.randn((M, 3 * D), generator=g, device="cuda").to(torch.bfloat16)
    ldv = (L + 63) // 64 * 64
    vt = Bd.op_transpose_v(qkv, 2 * D, B, L, nh, ldv)
    o = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")
    ours = timed(lambda: Bd.op_attention(qkv, qkv[:, D:], vt, o, B, L, L, nh), 5)
    res["attention"]["ours_ms"] = round(ours, 3)
    res["attention"]["ours_tflops"] = round(fl / ours / 1e9, 1)
    del qkv, vt, o
    q, k, v = (torch.randn((B, nh, L, 128), generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
    sdpa = timed(lambda: torch.nn.functional.scaled_dot_product_attention(q, k, v), 3)
    res["attention"]["torch_sdpa_ms"] = round(sdpa, 3)
    res["attention"]["torch_sdpa_tflops"] = round(fl / sdpa / 1e9, 1)
    print(json.dumps({"vendor_reference": res, "workload": cfg.name}), flush=True)


def vae_cpu_baseline(cfg, crop=(20, 26), frames=2):
    """fp64 oracle on a bounded sample of the decoder workload: the first `frames` latent frames of the
    workload's seeded latent, cropped to `crop` latent pixels, decoded whole; the decoder's work is
    convolutions of uniform cost per FLOP, so the full decode is estimated as its FLOPs at the sample's
    FLOP rate."""
    from oracle import wan_vae_oracle as V
    from wan_inputs.vae import VaeWeights, decoder_layout, draw_vae_latent

    threads = len(os.sched_getaffinity(0))
    w = VaeWeights(cfg)
    P = V.weights_f64(w)
    z = draw_vae_latent(cfg, frames=frames).f64()[0][:, :, :crop[0], :crop[1]]
    t0 = time.perf_counter()
    V.decode_whole(z, P, decoder_layout(cfg), cfg.eps)
    t = time.perf_counter() - t0
    fl = V.decoder_flops(frames, crop[0], crop[1], decoder_layout(cfg))
    return fl / t, t, threads


def vae_probe(cfg):
    """One launch each of the decoder kernels whose counters rocprofv3 reads, at the workload's stage-D
    shapes (96 channels, 8H x 8W, 16 frames: one chunk of 4 latent frames), plus the 1 GiB calibration copy."""
    import torch

    from video_diffusion_transformer_patchify_amd import binding as Bd

    torch.cuda.set_device(0)
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    C, H, W, nf = cfg.base_dim, 8 * cfg.height, 8 * cfg.width, 16
    g = torch.Generator(device="cuda").manual_seed(0)

    def frame():
        f = torch.zeros(((C + 15) // 16, H + 2, W + 2, 16), dtype=torch.bfloat16, device="cuda")
        f[:, 1:-1, 1:-1] = torch.randn((f.shape[0], H, W, 16), generator=g, device="cuda").to(torch.bfloat16)
        return f

    xs = [frame() for _ in range(nf + 2)]
    outs = [torch.zeros_like(xs[0]) for _ in range(nf)]
    w = (torch.randn((C, C, 3, 3, 3), generator=g, device="cuda") / (27 * C) ** 0.5).to(torch.bfloat16)
    wp = Bd.op_vae_pack_conv(w)
    b = torch.zeros(C, device="cuda")
    ins = [xs[j + dt] for j in range(nf) for dt in range(3)]
    torch.cuda.synchronize()
    Bd.op_vae_conv(ins, 3, 3, 0, wp, b, C, C, 1, H, W, outs)
    torch.cuda.synchronize()
    gam = torch.ones(C, device="cuda")
    Bd.op_vae_rms_silu(xs[:nf], outs, C, H, W, gam, 1e-6)
    torch.cuda.synchronize()
    print("vae probe done", flush=True)


def bench_vae(args):
    """A step is one wan_vae_decode of the whole latent (all latent frames, per-frame feature caches),
    inputs resident in HBM; value = the decoder's algorithmic convolution FLOPs per second."""
    import torch

    from oracle import wan_vae_oracle as V  # noqa: F401  (FLOP count only)
    from video_diffusion_transformer_patchify_amd import binding as Bd
    from video_diffusion_transformer_patchify_amd.harness import to_device, upload_weights
    from wan_inputs.vae import VaeWeights, decoder_layout, draw_vae_latent, get_vae_config

    cfg = get_vae_config(args.vae_config)
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    model = Bd.WanVAE(Bd.make_vae_config(cfg, chunk_frames=args.chunk_frames), upload_weights(VaeWeights(cfg)),
                      stream=stream)
    lat = to_device(draw_vae_latent(cfg))
    video = torch.empty(cfg.out_shape, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    print(f"# device bytes {model.device_bytes / 2**30:.2f} GiB", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        model.decode(lat, video, stream=stream)
    torch.cuda.synchronize()
    model.time_convs(4096)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        model.decode(lat, video, stream=stream)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    conv_ms, conv_n, conv_fl = model.conv_time()
    model.time_convs(0)
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    assert torch.isfinite(video.float()).all().item(), "non-finite video"
    fl = V.decoder_flops(cfg.frames, cfg.height, cfg.width, decoder_layout(cfg))
    tflops = fl / (ms * 1e-3) / 1e12
    conv_tf = conv_fl / (conv_ms * 1e-3) / 1e12
    print(f"# {ms:.2f} ms/decode = {tflops:.1f} TFLOP/s; 3x3x3 convs {conv_n} launches {conv_ms / conv_n:.3f} ms avg, "
          f"{conv_tf:.1f} TFLOP/s", file=sys.stderr, flush=True)
    res = {
        "metric": f"Wan-VAE decode TFLOP/s, latent {list(cfg.latent_shape)} -> video {list(cfg.out_shape)}, bf16",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 3), "ms_per_step_median": round(per_step[len(per_step) // 2], 3),
        "video_frames_per_s": round(cfg.out_frames * cfg.batch / (ms * 1e-3), 1),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) latent, N(0, 1/fan_in) random-init conv weights)",
        "config": {"workload": f"{cfg.name}: Wan2.1 VAE decoder (widths {list(cfg.dims)}), latent {list(cfg.latent_shape)}, "
                               f"chunks of {args.chunk_frames} latent frames after the first",
                   "global_batch": cfg.batch, "seq_len": cfg.out_frames, "parallelism": "single GPU"},
        "flops_per_step": fl,
        "mfma_frac_end_to_end": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": {"kernel": "k_vae_conv<3,3,0,3> (3x3x3 causal convs with 96-channel tiles: conv_in and the "
                               "residual-block convs)", "bound": "mfma", "achieved": round(conv_tf, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(conv_tf / PEAK_BF16_TFLOPS, 4),
                     "ms_per_launch": round(conv_ms / conv_n, 4), "flops_per_launch": round(conv_fl / conv_n),
                     "launches_timed": conv_n, "timed_where": "inside the timed decodes",
                     "traffic": traffic_for("k_vae.hip"),
                     "traffic_shape": "one stage-D launch (96 -> 96 channels, 16 frames of 480 x 832), "
                                      "rocprofv3 FETCH_SIZE / WRITE_SIZE of bench.py --workload vae --probe"},
    }
    model.close()
    del video, lat
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        rate, t, threads = vae_cpu_baseline(cfg)
        res["cpu_baseline"] = {
            "value": round(rate / 1e12, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "ms_per_step": round(fl / rate * 1e3, 1),
            "sample": f"fp64 numpy oracle decoding the workload's first 2 seeded latent frames cropped to 20 x 26 "
                      f"latent pixels ({t:.1f}s); the full decode estimated as its FLOPs at that rate",
        }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2, help="workload id (1..5); 2 = Wan2.1-1.3B, 2x32760 tokens")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=30.0)
    ap.add_argument("--probe", action="store_true", help="run the counter-calibration kernels only (for rocprofv3 --pmc)")
    ap.add_argument("--vendor-reference", action="store_true",
                    help="time hipBLASLt GEMMs and torch SDPA next to this library's kernels on the workload's shapes")
    ap.add_argument("--workload", choices=("dit", "vae"), default="dit",
                    help="dit: the DiT forward (default); vae: the Wan-VAE causal decoder")
    ap.add_argument("--vae-config", type=int, default=14, help="decoder workload id (11..15); 14 = 81 x 480 x 832")
    ap.add_argument("--chunk-frames", type=int, default=4, help="decoder: latent frames per chunk after the first")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 (no multi-GPU path)"}))
        sys.exit(2)
    if args.workload == "vae":
        if args.probe:
            from wan_inputs.vae import get_vae_config

            vae_probe(get_vae_config(args.vae_config))
        else:
            bench_vae(args)
        return
    if args.probe or args.vendor_reference:
        from wan_inputs import get_config

        (probe if args.probe else vendor_reference)(get_config(args.config))
        return

    import numpy as np  # noqa: F401
    import torch

    from video_diffusion_transformer_patchify_amd import binding as Bd
    from video_diffusion_transformer_patchify_amd.harness import to_device, upload_weights
    from wan_inputs import Weights, draw_inputs, get_config

    cfg = get_config(args.config)
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    t_setup = time.perf_counter()
    w = Weights(cfg)
    model = Bd.WanDiT(Bd.make_config(cfg), upload_weights(w, drop=True), stream=stream)
    torch.cuda.empty_cache()
    lat, t, txt = draw_inputs(cfg)
    latent, ts, text = to_device(lat), to_device(t), to_device(txt)
    out = torch.empty(cfg.out_shape, dtype=latent.dtype, device="cuda")
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    print(f"# setup {setup_s:.1f}s, device bytes {model.device_bytes / 2**30:.2f} GiB", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        model.forward(latent, ts, text, out, stream=stream)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    # the library brackets each self-attention launch of the timed steps with a HIP event pair
    model.time_attention(args.steps * cfg.num_layers)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        model.forward(latent, ts, text, out, stream=stream)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    attn_total_ms, attn_launches = model.attention_time()
    model.time_attention(0)
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    print(f"# timed {args.steps} steps: {ms:.2f} ms/step (wall {wall * 1e3 / args.steps:.2f})", file=sys.stderr, flush=True)
    assert torch.isfinite(out.float()).all().item(), "non-finite output"

    fl = step_flops(cfg)
    tflops = fl["total"] / (ms * 1e-3) / 1e12

    # dominant kernel: self-attention, its launches inside the timed steps (HIP events on the forward's
    # stream); also timed stand-alone on random operands, for reference
    assert attn_launches == args.steps * cfg.num_layers, attn_launches
    attn_ms = attn_total_ms / attn_launches
    attn_alone_ms = time_self_attention(cfg.batch, cfg, 10, stream)
    attn_flops = 4 * cfg.batch * cfg.tokens * cfg.tokens * cfg.dim
    attn_tf = attn_flops / (attn_ms * 1e-3) / 1e12
    print(f"# self-attention kernel in the timed steps {attn_ms:.3f} ms/launch = {attn_tf:.1f} TFLOP/s "
          f"({attn_launches} launches; stand-alone {attn_alone_ms:.3f} ms)", file=sys.stderr, flush=True)
    # measured dense bf16 MFMA ceiling on this device (MFMA-only probe kernel, no memory traffic)
    peak_zero = Bd.probe_mfma(random_operands=False, stream=stream)
    peak_rand = Bd.probe_mfma(random_operands=True, stream=stream)
    print(f"# MFMA probe: {peak_zero:.0f} TFLOP/s on zero operands, {peak_rand:.0f} on random bf16 operands",
          file=sys.stderr, flush=True)
    model.close()
    del latent, text, out
    torch.cuda.empty_cache()
    # measured HBM bandwidth on this device: a plain 1 GiB device-to-device copy (reads 1 GiB, writes 1 GiB)
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    e1.synchronize()
    copy_gbps = 2 * (1 << 30) * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    print(f"# HBM copy: {copy_gbps:.0f} GB/s (read + write)", file=sys.stderr, flush=True)
    del src, dst
    torch.cuda.empty_cache()

    res = {
        "metric": "DiT fwd ms/step + MFMA TFLOP/s, Wan-1.3B geometry, 32760 tokens bf16",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "ms_per_step_median": round(per_step[len(per_step) // 2], 3),
        "ms_per_step_min": round(per_step[0], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) latent/text, N(0,0.02) random-init weights)",
        "config": {"workload": f"{cfg.name}: B={cfg.batch}, latent {list(cfg.latent_shape)}, {cfg.tokens} tokens/sample, "
                               f"D={cfg.dim}, {cfg.num_heads} heads, FFN {cfg.ffn_dim}, {cfg.num_layers} blocks, "
                               f"text {cfg.text_len}x{cfg.text_dim}",
                   "global_batch": cfg.batch, "seq_len": cfg.tokens, "parallelism": "single GPU"},
        "mfma_frac_end_to_end": round(tflops / PEAK_BF16_TFLOPS, 4),
        "mfma_peak_measured": {"zero_operands": round(peak_zero, 1), "random_operands": round(peak_rand, 1),
                               "unit": "TFLOP/s", "kernel": "wan_probe_mfma (GEMM inner loop from LDS, 32x32x16 bf16)"},
        "mfma_frac_of_measured_random": round(tflops / peak_rand, 4),
        "hbm_peak_measured": {"copy": round(copy_gbps, 1), "unit": "GB/s", "vendor": 8000.0,
                              "kernel": "torch copy_ of 1 GiB (reads 1 GiB, writes 1 GiB)"},
        "flops_per_step": fl["total"],
        "roofline": {"kernel": "k_flash_attn<self> (self-attention)", "bound": "mfma", "achieved": round(attn_tf, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(attn_tf / PEAK_BF16_TFLOPS, 4),
                     "ms_per_launch": round(attn_ms, 3), "flops_per_launch": attn_flops,
                     "launches_timed": attn_launches, "timed_where": "inside the timed forward steps",
                     "ms_per_launch_standalone": round(attn_alone_ms, 3),
                     "traffic": traffic_for("k_attn.hip")},
    }
    if not args.no_cpu_baseline:
        est_step, sample_s, threads, (r, a, b, t_embed) = cpu_baseline(cfg, args.cpu_budget)
        res["cpu_baseline"] = {
            "value": round(fl["total"] / est_step / 1e12, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "ms_per_step": round(est_step * 1e3, 1),
            "sample": f"fp64 numpy oracle on the workload's seeded inputs, batch element 0: the embeddings in full "
                      f"({t_embed:.2f}s), the all-token part of block 0 (LN1, keys, values: {a:.2f}s) and block 0 on "
                      f"{r} token rows ({b * 1e3:.3f} ms per token beyond that part); step = {cfg.batch} x (embeddings "
                      f"+ {cfg.num_layers} blocks x ({a:.2f}s + {cfg.tokens} tokens x {b * 1e3:.3f} ms)); "
                      f"{sample_s:.1f}s measured",
        }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
