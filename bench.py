"""Throughput of the Stream Batch hot path on one MI355X.

A step is one push_frame (motion reduction, noise rate, entry noising) plus
one sd_stream_step (the whole stream-batched DiT forward over sink + window
KV, R-CFG, latent update, KV append, sink decision) on the 1.3B-shaped video
workload: 30 blocks, d 1536, 12 heads, FFN 8960, chunks of T=2 latent frames
of 16 x 60 x 104 (3120 tokens), 1560 sink + 9360 window tokens, n = 2 slots,
self-negative R-CFG, 77-token context, motion-aware noise on.  Inputs are
synthetic (seeded blob-motion latents, N(0,1) noise, N(0,0.02) weights) and
resident in device memory before timing starts.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--workload NAME] [--n-slots n] [--chunks B]
    python bench.py --workload video14b --sweep [--steps K]
    python bench.py --slo-fps F --chunks BMAX [--steps K]

Prints one JSON line (the sweep: one per (B, n) point, B chunks entering per
step and n denoising slots, so B*n rows per forward).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=6)
    ap.add_argument("--workload", default="video13b")
    ap.add_argument("--n-slots", type=int, default=2)
    ap.add_argument("--chunks", type=int, default=1, help="B: chunks entering (and leaving) per step")
    ap.add_argument("--batch-attn", action="store_true",
                    help="cross-frame batch attention: every row attends to the own tokens of all rows")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step as a captured HIP graph (the library runs on its own stream)")
    ap.add_argument("--io-stream", action="store_true",
                    help="pushes on a second stream (the IO queue), overlapped with the previous step's forward")
    ap.add_argument("--kv-recompute", action="store_true",
                    help="leaving chunks' cache entries from a clean-latent forward at timestep 0 (+B rows per step)")
    ap.add_argument("--sampler", choices=["ddim", "lcm"], default="ddim",
                    help="per-slot update: DDIM (re-noise with the guided prediction) or LCM-style fresh noise")
    ap.add_argument("--cfg", choices=["self", "onetime", "full"], default=None,
                    help="guidance variant (default: the workload's own, self-negative R-CFG for the video DiT)")
    ap.add_argument("--sweep", action="store_true",
                    help="one JSON line per (B, n) in {1,2,4,8} x {1,2,4}, weights shared (no CPU baseline)")
    ap.add_argument("--slo-fps", type=float, default=0.0,
                    help="run the SLO-aware batching loop for --steps steps with up to --chunks chunks per step "
                         "and report the batch sizes it chose (one JSON line)")
    ap.add_argument("--slo-plan", type=float, default=0.0, metavar="FPS",
                    help="measure steps at B in {1,2,4} x n in {1,2,4}, fit the latency per row and choose the "
                         "denoising steps n and chunks per step B for the target frame rate (one JSON line)")
    ap.add_argument("--vae", action="store_true",
                    help="measure the Stream-VAE instead: encode + decode of 4-frame chunks at the video shape")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-knee", action="store_true",
                    help="skip the below-the-knee leg (1.3B widths, 128-token chunks) of the default run")
    ap.add_argument("--cpu-blocks", type=int, default=2, help="DiT blocks in the oracle sample")
    ap.add_argument("--cpu-full", action="store_true",
                    help="time the CPU oracle alone, unsampled: the tiny workload's 16 steps (all threads and one "
                         "thread), one image-DiT step (one thread) and two full steps of the video DiT's pipeline "
                         "(n = 2, all 30 blocks, fp32); one JSON line, no GPU work (takes about ten minutes)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="after the run, copy MIB MiB device-to-device once (reference dispatch for HBM counters)")
    return ap.parse_args()


def slot_indices(n):
    return {1: (32,), 2: (32, 45), 3: (16, 32, 45), 4: (0, 16, 32, 45)}[n]


PMC_FILE = os.path.join(ROOT, "profiles", "attn_self_video13b_pmc.json")
ATTN_SOURCE = os.path.join(ROOT, "streaming_diffusion_amd", "csrc", "k_attn.hip")
PMC_FILE_KNEE = os.path.join(ROOT, "profiles", "gemm_ffn2_video13b_subknee_pmc.json")
GEMM_SOURCE = os.path.join(ROOT, "streaming_diffusion_amd", "csrc", "k_gemm_mfma.hip")


def measured_traffic(pmc_file=PMC_FILE, source=ATTN_SOURCE):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE runs, each scaled by what the counter
    read for a device copy of known size.  None when the kernel source
    changed since."""
    import hashlib
    try:
        rec = json.load(open(pmc_file))
        sha = hashlib.sha256(open(source, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != sha:
        return None
    cal = rec["copy_calibration"]
    f_scale = cal["bytes"] / (cal["fetch_kib"] * 1024.0)
    w_scale = cal["bytes"] / (cal["write_kib"] * 1024.0)
    return round(rec["fetch_kib_per_dispatch"] * 1024.0 * f_scale + rec["write_kib_per_dispatch"] * 1024.0 * w_scale)


def cpu_baseline(cfg, n_blocks_sample: int):
    """Time the CPU oracle on a bounded sample of the same workload: the full
    forward of one row through `n_blocks_sample` DiT blocks at the real shapes
    (3120 queries against a full 1560-sink + 9360-window cache plus its own
    tokens), fp32, then scale to one stream-batch step (n_blocks x rows)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle.dit import Denoiser
    from workloads import gen

    sample_cfg = cfg.replace(n_blocks=n_blocks_sample)
    w = gen.make_weights(sample_cfg)
    net = Denoiser(sample_cfg, w, dtype=np.float32)
    rng = np.random.default_rng(0)
    H, hd = cfg.n_heads, cfg.head_dim
    n_cache = cfg.sink_tokens + cfg.window_tokens
    cache = [(rng.standard_normal((n_cache, H, hd), dtype=np.float32),
              rng.standard_normal((n_cache, H, hd), dtype=np.float32)) for _ in range(n_blocks_sample)]
    ctx = gen.make_context(sample_cfg)
    ctx_kv = [net.cross_kv(ctx, b) for b in range(n_blocks_sample)] if ctx is not None else None
    x = gen.LatentSource(cfg).next()
    t0 = time.perf_counter()
    net.forward_row(x, 359, 0, cache, ctx_kv)
    dt = time.perf_counter() - t0
    rows = cfg.rows_per_step
    step_s = dt / n_blocks_sample * cfg.n_blocks * rows
    threads = 0
    blas = "unknown"
    for p in threadpool_info():
        if p.get("user_api") == "blas":
            threads = max(threads, int(p.get("num_threads", 0)))
            blas = f"{p.get('internal_api', '?')} {p.get('version', '')}".strip()
    cpu_model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": cfg.latent_t / step_s,
        "unit": "frames/s",
        "cores": threads or len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model,
        "blas": blas,
        "kind": "oracle",
        "sample": (f"one row through {n_blocks_sample} of {cfg.n_blocks} DiT blocks at full shape (fp32 NumPy, "
                   f"{dt:.2f} s), scaled x{cfg.n_blocks // n_blocks_sample * rows} to one {rows}-row step "
                   f"({step_s:.1f} s/step)"),
    }


def dominant_kind(cfg):
    """The kernel kind that bounds the step: self-attention at the video
    chunk sizes (MFMA-bound); below the roofline knee the FFN's second GEMM,
    which streams the largest weight matrix per launch (HBM-bound)."""
    return "gemm_ffn2" if cfg.tokens * cfg.rows_per_step <= 256 else "attn_self"


def measure(cfg, weights, steps: int, warmup: int, dev, io_stream: bool = False, graph: bool = False):
    """Warm up (fills the slots, the window and the sink), time `steps` steps
    with the inputs resident in device memory, then one untimed step with
    every kernel kind timed.  Returns the bench record without the CPU leg."""
    import torch

    from streaming_diffusion_amd.runner import StreamRunner
    from workloads import gen

    run = StreamRunner(cfg, weights, stream=torch.cuda.Stream() if graph else None)
    if graph:
        torch.cuda.synchronize()
        run.set_graph(True)
    if io_stream:
        run.set_io_stream(torch.cuda.Stream())        # inputs below are resident before the timed region
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    if cfg.ctx_len:
        ctx = torch.from_numpy(gen.make_context(cfg)).to(dev).to(tdt)
        ctx_neg = torch.from_numpy(gen.make_context(cfg, True)).to(dev).to(tdt) if cfg.cfg_type != "self" else None
        run.set_context(ctx, ctx_neg)
    B = cfg.chunks_per_step
    total = (warmup + (2 if graph else 1) * steps + 2) * B
    src, nz = gen.LatentSource(cfg), gen.NoiseSource(cfg)
    xs = [torch.from_numpy(src.next()).to(dev) for _ in range(total)]
    ns = [torch.from_numpy(gen.frame_noise(cfg, nz)).to(dev) for _ in range(total)]
    # SSF on images needs the frames; the uniform 1.0 never skips (u < p is
    # false for p <= 1), so the filter's reductions and decision run on every
    # push and every timed step has its chunks
    fs = None
    if cfg.ssf_on and cfg.ssf_kind == "u8":
        fsrc = gen.SSFFrameSource(cfg)
        fs = [torch.from_numpy(fsrc.next()).to(dev) for _ in range(total)]
    out = run.out
    torch.cuda.synchronize()
    k = 0

    def push_group():
        nonlocal k
        for _ in range(B):
            run.push(xs[k], ns[k], fs[k] if fs is not None else None, 1.0)
            k += 1

    # warm-up; time to first frame
    ttff_ms = None
    t_first = time.perf_counter()
    for _ in range(warmup):
        push_group()
        info = run.step(out)
        if info.has_output and ttff_ms is None:
            torch.cuda.synchronize()
            ttff_ms = (time.perf_counter() - t_first) * 1e3
    torch.cuda.synchronize()

    # timed region: the dominant kernel is timed live with events (with graph
    # replay, live events would turn replay off: it is timed over as many
    # extra launched steps right after)
    dom_kind = dominant_kind(cfg)
    if not graph:
        run.profile([dom_kind])
        run.profile_read()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    emitted = 0
    for _ in range(steps):
        push_group()
        info = run.step(out)
        emitted += info.n_out * cfg.latent_t
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if graph:
        graph_stats = run.graph_stats()
        run.profile([dom_kind])
        run.profile_read()
        for _ in range(steps):
            push_group()
            run.step(out)
        torch.cuda.synchronize()
    attn = run.profile_read().get(dom_kind)
    elapsed = t1 - t0
    ms_per_step = elapsed / steps * 1e3

    # untimed breakdown pass over every kernel kind (one step)
    run.profile(list(__import__("streaming_diffusion_amd._lib", fromlist=["PROF_KINDS"]).PROF_KINDS))
    push_group()
    run.step(out)
    breakdown = run.profile_read()
    run.profile([])
    run.close()

    roofline = None
    if attn and attn["launches"] and dom_kind == "attn_self":
        per_launch_ms = attn["ms"] / attn["launches"]
        per_launch_flop = attn["flops"] / attn["launches"]
        achieved = per_launch_flop / (per_launch_ms * 1e-3) / 1e12
        roofline = {"kernel": "attn_bf16_kernel<128, 0> (self-attention over sink + window + own)",
                    "bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                    "traffic": measured_traffic(),
                    "avg_launch_ms": round(per_launch_ms, 4), "flop_per_launch": per_launch_flop,
                    "algorithmic_bytes_per_launch": attn["bytes"] / attn["launches"],
                    "launches": attn["launches"]}
    elif attn and attn["launches"]:
        # below the knee: the FFN GEMMs stream the largest weights; bytes per
        # launch = W + A + the output pass (algorithmic), over the launch time
        per_launch_ms = attn["ms"] / attn["launches"]
        per_launch_bytes = attn["bytes"] / attn["launches"]
        achieved = per_launch_bytes / (per_launch_ms * 1e-3) / 1e9
        roofline = {"kernel": f"{dom_kind}: gemm_wstream_kernel + gemm_reduce_ln_kernel (weight-streaming GEMM, "
                              f"K split over the CUs; the reduction pass also runs the next block's LayerNorm)",
                    "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic(PMC_FILE_KNEE, GEMM_SOURCE) if dom_kind == "gemm_ffn2" else None,
                    "avg_launch_ms": round(per_launch_ms, 4), "algorithmic_bytes_per_launch": per_launch_bytes,
                    "launches": attn["launches"]}
    bd = {}
    for name, v in breakdown.items():
        if v["ms"] <= 0:
            continue
        bd[name] = {"ms": round(v["ms"], 3), "launches": v["launches"],
                    "tflops": round(v["flops"] / (v["ms"] * 1e-3) / 1e12, 1) if v["flops"] else None,
                    "gbs": round(v["bytes"] / (v["ms"] * 1e-3) / 1e9, 1)}
    return {
        "metric": "denoised latent frames/s, one Stream Batch step per call (1.3B-shaped video DiT)"
        if cfg.name == "video13b" else f"denoised latent frames/s, one Stream Batch step per call ({cfg.name})",
        "value": round(emitted / elapsed, 3),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.n_blocks} blocks d{cfg.d_model} h{cfg.n_heads} ffn{cfg.d_ffn}, "
                               f"chunk T={cfg.latent_t} {cfg.latent_c}x{cfg.latent_h}x{cfg.latent_w} "
                               f"({cfg.tokens} tokens), sink {cfg.sink_tokens} + window {cfg.window_tokens}, "
                               f"n={cfg.n_slots} slots, B={B} chunks per step, guidance {cfg.cfg_type}, "
                               f"ctx {cfg.ctx_len}, motion {'on' if cfg.motion_on else 'off'}"
                               + (", cross-frame batch attention" if cfg.batch_attn else "")
                               + (f", {cfg.sampler} sampler" if cfg.sampler != "ddim" else "")
                               + (", clean-latent KV recompute" if cfg.kv_recompute else ""),
                   "rows_per_step": cfg.rows_per_step, "tokens_per_row": cfg.tokens,
                   "frames_per_step": B * cfg.latent_t, "parallelism": "single GPU",
                   "io_stream": bool(io_stream), "graph": bool(graph)},
        "ttff_ms": round(ttff_ms, 2) if ttff_ms else None,
        "graph": {"captures": graph_stats[0], "replays": graph_stats[1]} if graph else None,
        "roofline": roofline,
        "breakdown_one_step": bd,
    }


def vae_conv_flops(L):
    """Algorithmic FLOP of one convolution layer: 2 x 27 Cin x Cout per output position."""
    return 2.0 * 27 * L["cin"] * L["cout"] * L["T"] * L["H"] * L["W"]


def vae_layers(v):
    T, h, w = v.latent_t, v.latent_h, v.latent_w
    Tp, H, W = 2 * T, 8 * h, 8 * w
    rows = [("e0", 8, v.c1, Tp, H, W), ("e1", v.c1, v.c2, Tp, H // 2, W // 2), ("e2", v.c2, v.c3, Tp, H // 4, W // 4),
            ("e3", v.c3, v.c3, T, h, w), ("e_out", v.c3, v.latent_c, T, h, w), ("d0", v.latent_c, v.c3, T, h, w),
            ("d1", v.c3, v.c3, Tp, H // 4, W // 4), ("d2", v.c3, v.c2, Tp, H // 2, W // 2),
            ("d3", v.c2, v.c1, Tp, H, W), ("d_out", v.c1, 3, Tp, H, W)]
    return [dict(name=n, cin=ci, cout=co, T=t, H=hh, W=ww) for n, ci, co, t, hh, ww in rows]


def vae_run(steps: int, warmup: int, dev, cpu: bool):
    """Stream-VAE at the video shape: `steps` chunks encoded and decoded back
    to back (pixels and latents resident), then every matrix-core layer timed
    alone at its real shape with HIP events on the library's stream."""
    import ctypes as C

    import numpy as np
    import torch

    import streaming_diffusion_amd._lib as L
    from streaming_diffusion_amd.runner import VAERunner, upload_vae_weights
    from workloads import gen, get_vae_config

    v = get_vae_config("video13b")
    w = gen.make_vae_weights(v)
    run = VAERunner(v, upload_vae_weights(v, w))
    src = gen.PixelSource(v)
    pix = [torch.from_numpy(np.ascontiguousarray(src.next())).to(dev) for _ in range(4)]
    lat = torch.empty(run.lat_shape, dtype=torch.float32, device=dev)
    out = torch.empty(run.pix_shape, dtype=torch.float32, device=dev)
    for k in range(warmup):
        run.encode(pix[k % 4], lat)
        run.decode(lat, out)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    enc_ms = dec_ms = 0.0
    t0 = time.perf_counter()
    for k in range(steps):
        ev[0].record()
        run.encode(pix[k % 4], lat)
        ev[1].record()
        run.decode(lat, out)
        ev[2].record()
        torch.cuda.synchronize()
        enc_ms += ev[0].elapsed_time(ev[1])
        dec_ms += ev[1].elapsed_time(ev[2])
    elapsed = time.perf_counter() - t0
    run.close()
    # each matrix-core convolution alone, random operands of its shape
    lib = L.load()
    stream = torch.cuda.current_stream()
    layers = []
    for Ly in vae_layers(v):
        T, H, W, ci, co = Ly["T"], Ly["H"], Ly["W"], Ly["cin"], Ly["cout"]
        x = torch.randn((T, H, W, ci), device=dev).to(torch.bfloat16)
        cache = torch.randn((2, H, W, ci), device=dev).to(torch.bfloat16)
        wt = (torch.randn((co, 27 * ci), device=dev) / np.sqrt(27 * ci)).to(torch.bfloat16)
        # the narrow last layers (latent and pixel projections) write fp32 channels-first
        narrow = co < 32
        y = torch.empty((T, co, H, W) if narrow else (T, H, W, co), dtype=torch.float32 if narrow else torch.bfloat16,
                        device=dev)
        call = lambda: lib.sd_k_conv3d(x.data_ptr(), cache.data_ptr(), wt.data_ptr(), None,
                                       None if narrow else y.data_ptr(), y.data_ptr() if narrow else None,
                                       T, H, W, ci, co, C.c_void_p(stream.cuda_stream))
        for _ in range(2):
            call()
        ev[0].record(stream)
        reps = 10
        for _ in range(reps):
            call()
        ev[1].record(stream)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / reps
        fl = vae_conv_flops(Ly)
        layers.append({"layer": Ly["name"], "cin": ci, "cout": co, "positions": T * H * W, "ms": round(ms, 4),
                       "tflops": round(fl / (ms * 1e-3) / 1e12, 1)})
        del x, cache, wt, y
    dom = max(layers, key=lambda r: r["ms"])
    Ldom = next(r for r in vae_layers(v) if r["name"] == dom["layer"])
    per_chunk_ms = (enc_ms + dec_ms) / steps
    res = {
        "metric": "Stream-VAE frames/s, encode + decode of one chunk per call (4 frames 480x832 <-> 2 x 16 x 60 x 104)",
        "value": round(steps * v.frames / ((enc_ms + dec_ms) * 1e-3), 2),
        "unit": "frames/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(per_chunk_ms, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"Stream-VAE video13b: chunk {v.frames} x 3 x {v.height} x {v.width} pixels, "
                               f"latent {v.latent_t} x {v.latent_c} x {v.latent_h} x {v.latent_w}, widths "
                               f"{v.c1}/{v.c2}/{v.c3}, causal 3x3x3 convolutions with 2-frame caches",
                   "parallelism": "single GPU"},
        "encode_ms_per_chunk": round(enc_ms / steps, 3), "decode_ms_per_chunk": round(dec_ms / steps, 3),
        "wall_ms_per_chunk": round(elapsed / steps * 1e3, 3),
        "roofline": {"kernel": f"sd_k_conv3d (layer {dom['layer']}, timed alone at its shape; halo-tiled "
                                "direct convolution for 4-frame layers)",
                     "bound": "mfma", "achieved": dom["tflops"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(dom["tflops"] / BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "avg_launch_ms": dom["ms"], "flop_per_launch": vae_conv_flops(Ldom)},
        "layers": layers,
    }
    if cpu:
        from threadpoolctl import threadpool_info

        from oracle import vae as ovae
        sv = ovae.StreamVAE(v, w)
        pix0 = src.next()
        t1 = time.perf_counter()
        sv.encode_chunk(pix0)
        dt = time.perf_counter() - t1
        fl_enc = sum(vae_conv_flops(r) for r in vae_layers(v) if r["name"].startswith("e"))
        fl_all = sum(vae_conv_flops(r) for r in vae_layers(v))
        chunk_s = dt * fl_all / fl_enc
        threads = max([int(p.get("num_threads", 0)) for p in threadpool_info() if p.get("user_api") == "blas"] or [0])
        res["cpu_baseline"] = {"value": round(v.frames / chunk_s, 4), "unit": "frames/s",
                               "cores": threads or len(os.sched_getaffinity(0)), "kind": "oracle",
                               "sample": f"one chunk through the encoder (fp64 NumPy, {dt:.1f} s), scaled by the "
                                         f"encode + decode / encode FLOP ratio {fl_all / fl_enc:.2f}"}
    return res


def cpu_full():
    """The oracle itself on whole steps of the workloads, no sampling."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle.stream import OracleStream
    from workloads import gen, get_config

    def run_steps(cfg, steps, dtype, threads=None):
        w = gen.make_weights(cfg)
        ctx = gen.make_context(cfg)
        neg = gen.make_context(cfg, True) if cfg.cfg_type != "self" else None
        orc = OracleStream(cfg, w, ctx, neg, dtype=dtype)
        src, nz, us = gen.LatentSource(cfg), gen.NoiseSource(cfg), gen.UniformSource()
        ssf = gen.SSFFrameSource(cfg) if cfg.ssf_on and cfg.ssf_kind == "u8" else None
        times = []
        with threadpool_limits(limits=threads):
            while len(times) < steps:
                t0 = time.perf_counter()
                po = orc.push_frame(src.next(), gen.frame_noise(cfg, nz), ssf.next() if ssf else None, us.next())
                if po.skipped:
                    continue
                orc.step()
                times.append(time.perf_counter() - t0)
                print(f"cpu-full: {cfg.name} step {len(times)}/{steps} {times[-1]:.2f} s", file=sys.stderr, flush=True)
        return times

    threads = max([int(p.get("num_threads", 0)) for p in threadpool_info() if p.get("user_api") == "blas"] or [0])
    res = {"metric": "CPU oracle, whole steps (no sampling)", "kind": "oracle", "cores": threads}
    t = run_steps(get_config("tiny"), 16, np.float64)
    res["tiny_fp64_16_steps"] = {"s_total": round(sum(t), 3), "ms_per_step": round(1e3 * sum(t) / 16, 2)}
    t = run_steps(get_config("tiny"), 16, np.float64, threads=1)
    res["tiny_fp64_16_steps_1_thread"] = {"s_total": round(sum(t), 3), "ms_per_step": round(1e3 * sum(t) / 16, 2)}
    t = run_steps(get_config("image", t_index=(32,)), 1, np.float64, threads=1)
    res["image_fp64_n1_one_step_1_thread"] = {"s": round(t[0], 2), "frames_per_s": round(1.0 / t[0], 4)}
    t = run_steps(get_config("image"), 8, np.float64)
    res["image_fp64_n2_8_steps"] = {"s_total": round(sum(t), 2), "ms_per_step": round(1e3 * sum(t) / 8, 1),
                                    "frames_per_s": round(8 / sum(t), 3)}
    t = run_steps(get_config("fourstep"), 4, np.float64)
    res["fourstep_fp64_n4_onetime_4_steps"] = {"s_total": round(sum(t), 2), "ms_per_step": round(1e3 * sum(t) / 4, 1),
                                               "frames_per_s": round(4 / sum(t), 4)}
    print(json.dumps(res), flush=True)
    cfg = get_config("video13b")
    t = run_steps(cfg, 2, np.float32)
    res["video13b_fp32_n2_two_steps"] = {
        "s_per_step": [round(x, 1) for x in t],
        "note": "step 1: one row (the entering chunk); step 2: two rows, the first chunk leaves (cache still empty, "
                "3120 keys per row); a steady-state step attends over 14040 keys"}
    return res


def slo_run(cfg, weights, target_fps: float, steps: int, dev):
    """The SLO-aware batching loop on the real pipeline with a backlog of
    input chunks: each step the scheduler picks how many enter; a step's
    latency counts only once the last n groups all had the same size (the
    latency depends on every group in flight)."""
    import torch

    from streaming_diffusion_amd.runner import StreamRunner
    from streaming_diffusion_amd.slo import SLOBatchScheduler
    from workloads import gen

    run = StreamRunner(cfg, weights)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    if cfg.ctx_len:
        neg = torch.from_numpy(gen.make_context(cfg, True)).to(dev).to(tdt) if cfg.cfg_type != "self" else None
        run.set_context(torch.from_numpy(gen.make_context(cfg)).to(dev).to(tdt), neg)
    src, nz = gen.LatentSource(cfg), gen.NoiseSource(cfg)
    pool = [(torch.from_numpy(src.next()).to(dev), torch.from_numpy(gen.frame_noise(cfg, nz)).to(dev))
            for _ in range(16)]
    sch = SLOBatchScheduler(cfg.latent_t, target_fps, cfg.chunks_per_step)
    n = cfg.n_slots
    sizes, trace = [], []
    k = 0
    for _ in range(steps):
        b = sch.choose(pending=cfg.chunks_per_step)
        for _ in range(b):
            x, e = pool[k % len(pool)]
            run.push(x, e)
            k += 1
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run.step(chunks=b)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        sizes.append(b)
        steady = len(sizes) >= n + 1 and all(v == b for v in sizes[-n:])
        if steady:
            sch.observe(b, dt)
        trace.append((b, round(dt * 1e3, 2), steady))
    run.close()
    b_final = sizes[-1]
    model = sch.model()
    return {"metric": "SLO-aware batching: chunks per step chosen from observed latency",
            "target_fps": target_fps, "b_max": cfg.chunks_per_step, "n_slots": n,
            "chosen_b": b_final,
            "predicted_fps_at_chosen_b": round(sch.rate(b_final, model), 2) if model else None,
            "latency_model_ms": {"fixed": round(model[0] * 1e3, 3), "per_chunk": round(model[1] * 1e3, 3)}
            if model else None,
            "observed_ms": {str(b): round(v * 1e3, 2) for b, v in sorted(sch.lat.items())},
            "trace": trace, "config": {"workload": cfg.name}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); multi-GPU sharding of this path is "
              "described in DESIGN.md and not run.", file=sys.stderr)
        sys.exit(2)

    if args.cpu_full:
        print(json.dumps(cpu_full()))
        return

    import torch

    from streaming_diffusion_amd.runner import random_device_weights
    from workloads import gen, get_config

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.vae:
        print(json.dumps(vae_run(args.steps, args.warmup, dev, not args.no_cpu_baseline)))
        return
    kw = {} if args.cfg is None else {"cfg_type": args.cfg}
    if args.batch_attn:
        kw["batch_attn"] = True
    if args.sampler != "ddim":
        kw["sampler"] = args.sampler
    if args.kv_recompute:
        kw["kv_recompute"] = True
    if args.slo_fps > 0:
        cfg = get_config(args.workload, t_index=slot_indices(args.n_slots), chunks_per_step=max(2, args.chunks), **kw)
        weights = random_device_weights(cfg, seed=gen.SEED_WEIGHTS)
        print(json.dumps(slo_run(cfg, weights, args.slo_fps, args.steps, dev)))
        return
    if args.slo_plan > 0:
        from streaming_diffusion_amd.slo import fit_rows_model, plan_steps_and_batch
        base = get_config(args.workload)
        weights = random_device_weights(base, seed=gen.SEED_WEIGHTS)
        table = {}
        for n in (1, 2, 4):
            for B in (1, 2, 4):
                cfg = get_config(args.workload, t_index=slot_indices(n), chunks_per_step=B, **kw)
                r = measure(cfg, weights, args.steps, max(args.warmup, n + 1), dev, graph=args.graph)
                table[(B, n)] = r["ms_per_step"] * 1e-3
        alpha, beta = fit_rows_model([(B * n, t) for (B, n), t in table.items()])
        plan = plan_steps_and_batch(lambda B, n: alpha + beta * B * n, base.latent_t, args.slo_plan, 4, (1, 2, 4))
        print(json.dumps({"metric": "SLO plan: denoising steps and chunks per step for a frame-rate target",
                          "target_fps": args.slo_plan, "workload": args.workload,
                          "measured_ms": {f"B{B}_n{n}": round(t * 1e3, 3) for (B, n), t in sorted(table.items())},
                          "latency_model_ms": {"fixed": round(alpha * 1e3, 3), "per_row": round(beta * 1e3, 3)},
                          "plan": {"n": plan[0], "B": plan[1],
                                   "predicted_fps": round(plan[1] * base.latent_t / (alpha + beta * plan[0] * plan[1]), 2)},
                          "graph": bool(args.graph)}))
        return
    if args.sweep:
        # weights do not depend on n or B
        base = get_config(args.workload)
        weights = random_device_weights(base, seed=gen.SEED_WEIGHTS)
        for n in (1, 2, 4):
            for B in (1, 2, 4, 8):
                cfg = get_config(args.workload, t_index=slot_indices(n), chunks_per_step=B, **kw)
                if cfg.rows_per_step > 40:          # beyond the rows one forward takes
                    continue
                res = measure(cfg, weights, args.steps, max(args.warmup, n + 1), dev)
                res["config"]["sweep"] = {"B": B, "n": n}
                print(json.dumps(res), flush=True)
        return
    cfg = get_config(args.workload, t_index=slot_indices(args.n_slots), chunks_per_step=args.chunks, **kw)
    weights = random_device_weights(cfg, seed=gen.SEED_WEIGHTS)
    res = measure(cfg, weights, args.steps, args.warmup, dev, args.io_stream, args.graph)
    plain = not (args.batch_attn or args.kv_recompute or args.io_stream or args.graph or args.cfg or
                 args.sampler != "ddim" or args.chunks != 1 or args.n_slots != 2)
    if cfg.name == "video13b" and plain and not args.no_knee:
        # the memory-bound side of the roofline: the same weights with one
        # latent frame of 8 x 16 tokens per chunk and one slot (128 tokens per
        # forward, below the knee), step replayed as a captured graph
        knee_cfg = get_config("video13b_subknee", t_index=slot_indices(1))
        knee = measure(knee_cfg, weights, max(args.steps, 20), args.warmup, dev, graph=True)
        res["roofline_below_knee"] = dict(knee["roofline"] or {}, workload=knee["config"]["workload"],
                                          ms_per_step=knee["ms_per_step"], frames_per_s=knee["value"])
    if args.calibrate_copy:
        n = args.calibrate_copy << 18          # float32 elements in MIB MiB
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, args.cpu_blocks)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
