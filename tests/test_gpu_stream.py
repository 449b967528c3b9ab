"""GPU parity of whole Stream Batch steps through the C ABI (sd_stream_*)
against the CPU oracle: denoiser outputs per row, emitted frames, SSF
decisions and every integer of the step state, KV ring contents and sink
decisions.  Shapes are reduced versions of the workloads (same code paths:
head dims, tile tails, cross-attention, onetime-negative rows, motion)."""
import numpy as np
import pytest
import torch

import streaming_diffusion_amd._lib as L
from oracle.stream import OracleStream
from streaming_diffusion_amd.runner import StreamRunner, upload_weights
from workloads import gen, get_config

from gpu_helpers import check_close, device, to_dev

pytestmark = pytest.mark.gpu


def reduced(name, **kw):
    base = {
        "tiny": {},
        "image": dict(n_blocks=2),
        "fourstep": dict(n_blocks=2, d_model=256, n_heads=4, d_ffn=1024),
        "video13b": dict(n_blocks=2, d_model=256, n_heads=2, d_ffn=512, latent_h=16, latent_w=24,
                         sink_tokens=96, window_tokens=576),
    }[name]
    base.update(kw)
    return get_config(name, **base)


def scene_cut(pushes, scale=-4.0):
    """Input transform of a crafted scene cut: the latents of the given
    pushes (0-based) are scaled by `scale`, which turns the chunk embedding
    away from the sink's (cosine about -0.9 instead of 0.93-0.99)."""
    return lambda k, x: x * np.float32(scale) if k in pushes else x


def run_parity(cfg, steps, check_ring=True, sizes=None, io_stream=False, transform=None, oracle_dtype=np.float64,
               progress=False, graph=False):
    """`sizes`: chunks entering at each step (cycled); default B every step.
    `io_stream`: inputs are produced and pushed on a second stream (the IO
    queue), overlapped with the steps on the main stream.  `transform(k, x0)`
    changes push k's clean latent on both sides.  The oracle's sink decisions
    that the GPU matched are kept in orc.sink_events as (sim, refreshed)."""
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    weights = gen.make_weights(cfg)
    ctx_pos = gen.make_context(cfg)
    ctx_neg = gen.make_context(cfg, negative=True) if cfg.cfg_type != "self" else None
    orc = OracleStream(cfg, weights, ctx_pos, ctx_neg, dtype=oracle_dtype)
    # graph replay needs a created stream: inputs are then produced on it too
    side = torch.cuda.Stream() if graph else None
    orc.sink_events = []
    orc.t0_trace = []
    run = StreamRunner(cfg, upload_weights(cfg, weights), stream=side)
    if graph:
        torch.cuda.synchronize()
        run.set_graph(True)
    if cfg.ctx_len:
        run.set_context(to_dev(ctx_pos, tdt), to_dev(ctx_neg, tdt) if ctx_neg is not None else None)
    io = torch.cuda.Stream() if io_stream else None
    if io is not None:
        run.set_io_stream(io)
    src, nz, us = gen.LatentSource(cfg), gen.NoiseSource(cfg), gen.UniformSource()
    ssf_src = gen.SSFFrameSource(cfg) if cfg.ssf_on and cfg.ssf_kind == "u8" else None
    lat = cfg.latent_elems
    B = cfg.chunks_per_step
    done = pushes = queued = 0
    worst = 0.0
    while done < steps:
        x0, e, u = src.next(), gen.frame_noise(cfg, nz), us.next()
        if transform is not None:
            x0 = transform(pushes, x0)
        frame = ssf_src.next() if ssf_src else None
        po = orc.push_frame(x0, e, frame, u)
        with torch.cuda.stream(io if io is not None else (side if side is not None else torch.cuda.current_stream())):
            pg = run.push(to_dev(x0, torch.float32), to_dev(e, torch.float32),
                          to_dev(frame, torch.uint8) if frame is not None else None, u)
        pushes += 1
        # SSF decision, probability and similarity: bit-exact
        assert bool(pg.skipped) == po.skipped, f"push {pushes}"
        assert pg.p == po.p and pg.sim == po.sim, (pushes, pg.p, po.p)
        if po.skipped:
            continue
        assert list(pg.taus)[:cfg.n_slots] == po.taus and pg.t0 == po.t0 and pg.s == po.s
        orc.t0_trace.append(po.t0)
        queued += 1
        want = sizes[done % len(sizes)] if sizes else B
        if queued < want:        # a step takes `want` pending chunks
            continue
        queued = 0
        out_o, so = orc.step(want)
        sg = run.step(chunks=want)
        torch.cuda.synchronize()
        assert (sg.has_output, sg.rows, sg.frame_id, sg.n_out) == (int(so.has_output), so.rows, so.frame_id,
                                                                   so.n_out)
        assert (sg.kv_ptr, sg.kv_valid, sg.sink_count, sg.rope_next) == (so.kv_ptr, so.kv_valid, so.sink_count,
                                                                         so.rope_next)
        eps = run.buffer(L.SD_BUF_EPS, torch.float32, (sg.rows, lat)).cpu().numpy()
        for r in range(sg.rows):
            worst = max(worst, check_close(eps[r], orc.last_eps[r].ravel(), cfg.dtype, f"step {done} eps row {r}"))
        if out_o is not None:
            got = run.out.cpu().numpy()
            if B > 1:
                got = got[:so.n_out]
            worst = max(worst, check_close(got, out_o, cfg.dtype, f"step {done} output"))
        if not np.isnan(so.sink_sim):
            si = run.sink_info()
            assert si.evaluated == 1 and si.entry == so.sink_entry
            if abs(so.sink_sim - cfg.sink_tau) > 1e-2:
                assert bool(si.refreshed) == so.sink_refreshed, (done, si.sim, so.sink_sim)
                orc.sink_events.append((so.sink_sim, so.sink_refreshed))
        done += 1
        if progress:
            print(f"  step {done}: {sg.rows} rows, kv_valid {sg.kv_valid}, worst error {worst:.3e}", flush=True)
    if check_ring and cfg.window_tokens:
        H, hd, W = cfg.n_heads, cfg.head_dim, cfg.window_tokens
        ringK = run.buffer(L.SD_BUF_RING_K, tdt, (cfg.n_blocks, H, W, hd)).float().cpu().numpy()
        ringV = run.buffer(L.SD_BUF_RING_V, tdt, (cfg.n_blocks, H, hd, W)).float().cpu().numpy()
        valid = [(orc.kv_ptr - orc.kv_valid + j) % W for j in range(orc.kv_valid)]
        for b in range(cfg.n_blocks):
            check_close(ringK[b].transpose(1, 0, 2)[valid], orc.ringK[b][valid], cfg.dtype, f"ring K block {b}",
                          stored_bf16=True)
            check_close(ringV[b].transpose(2, 0, 1)[valid], orc.ringV[b][valid], cfg.dtype, f"ring V block {b}",
                          stored_bf16=True)
    if check_ring and cfg.sink_tokens and orc.sink_count:
        H, hd, S = cfg.n_heads, cfg.head_dim, cfg.sink_tokens
        S8 = (S + 7) // 8 * 8
        used = orc.sink_count * (S // orc.M)
        sinkK = run.buffer(L.SD_BUF_SINK_K, tdt, (cfg.n_blocks, H, S8, hd)).float().cpu().numpy()
        sinkV = run.buffer(L.SD_BUF_SINK_V, tdt, (cfg.n_blocks, H, hd, S8)).float().cpu().numpy()
        for b in range(cfg.n_blocks):
            check_close(sinkK[b].transpose(1, 0, 2)[:used], orc.sinkK[b][:used], cfg.dtype, f"sink K block {b}",
                        stored_bf16=True)
            check_close(sinkV[b].transpose(2, 0, 1)[:used], orc.sinkV[b][:used], cfg.dtype, f"sink V block {b}",
                        stored_bf16=True)
    if graph:
        orc.graph_stats = run.graph_stats()
    print(f"{cfg.name}: {done} steps over {pushes} pushes, worst error {worst:.3e}", flush=True)
    run.close()
    return orc, run


def test_tiny_fp32_sixteen_steps_with_ssf():
    device()
    cfg = reduced("tiny")
    print("tiny fp32 16 steps", flush=True)
    orc, _ = run_parity(cfg, 16)
    assert orc.sink_count == 1


def test_tiny_fp32_without_ssf_three_slots_wide_window():
    device()
    cfg = reduced("tiny", ssf_on=False, t_index=(10, 32, 45), window_tokens=128)
    print("tiny fp32 n=3 W=128", flush=True)
    run_parity(cfg, 7)


def test_image_bf16_two_slots_cross_attention():
    device()
    cfg = reduced("image")
    print("image bf16 reduced", flush=True)
    run_parity(cfg, 5)


def test_image_bf16_single_slot():
    device()
    cfg = reduced("image", t_index=(32,))
    print("image bf16 n=1", flush=True)
    run_parity(cfg, 3)


def test_fourstep_bf16_onetime_negative_with_latent_ssf():
    device()
    cfg = reduced("fourstep")
    print("fourstep bf16 reduced", flush=True)
    run_parity(cfg, 6)


def test_video_bf16_motion_full_window():
    device()
    cfg = reduced("video13b")
    print("video bf16 reduced", flush=True)
    orc, _ = run_parity(cfg, 8)
    assert orc.kv_valid == cfg.window_tokens


def refresh_and_keep(orc, margin=1e-2):
    """Both sink outcomes occurred, each decided more than `margin` from tau
    (the GPU's decision was compared with the oracle's for each)."""
    tau = orc.cfg.sink_tau
    ref = [s for s, r in orc.sink_events if r and tau - s > margin]
    keep = [s for s, r in orc.sink_events if not r and s - tau > margin]
    assert ref and keep, orc.sink_events
    return len(ref), len(keep)


def test_video_bf16_sink_refresh_fires_after_a_scene_cut():
    """StreamDiffusionV2 summary, adaptive sink refresh: chunks 5 and 6 are a
    scene cut; their embeddings point away from the sink's, the entry is
    refreshed, and the following ordinary chunks are kept."""
    device()
    cfg = reduced("video13b")
    print("video bf16 reduced, scene cut at pushes 5-6", flush=True)
    orc, _ = run_parity(cfg, 10, transform=scene_cut({5, 6}))
    print("refresh / keep events:", refresh_and_keep(orc), flush=True)


def test_video_bf16_two_sink_entries_scene_cut():
    """M = 2 sink entries of 48 tokens: both fill from the first two leaving
    chunks, the least similar one is replaced after the cut."""
    device()
    cfg = reduced("video13b", sink_entries=2)
    print("video bf16 reduced, M = 2, scene cut", flush=True)
    orc, _ = run_parity(cfg, 10, transform=scene_cut({5, 6}))
    assert orc.sink_count == 2
    print("refresh / keep events:", refresh_and_keep(orc), flush=True)


def test_video_bf16_three_chunks_staged_sink_refresh():
    """B = 3: the cut chunk is the third of its group, so its refresh copies
    from its staged candidate slot (the ring already holds the later chunks)."""
    device()
    cfg = reduced("video13b", chunks_per_step=3, window_tokens=384)
    print("video bf16 reduced B=3, scene cut at push 5", flush=True)
    orc, _ = run_parity(cfg, 6, transform=scene_cut({5}))
    print("refresh / keep events:", refresh_and_keep(orc), flush=True)


def test_video_bf16_rope_reset_wraps_temporal_positions():
    """StreamDiffusionV2 summary, RoPE refresh: with the threshold at 3 and
    T = 2 frames per chunk the temporal base runs 0, 2, 0, 2, ...; keys cached
    before a wrap keep their old rotation."""
    device()
    cfg = reduced("video13b", rope_reset=3)
    print("video bf16 reduced, rope_reset 3", flush=True)
    orc, _ = run_parity(cfg, 8)
    assert orc.t0_trace == [0, 2] * 4


def test_tiny_fp32_rope_reset_wraps_temporal_positions():
    device()
    cfg = reduced("tiny", ssf_on=False, rope_reset=3)
    print("tiny fp32, rope_reset 3", flush=True)
    orc, _ = run_parity(cfg, 9)
    assert orc.t0_trace == [0, 1, 2, 3, 0, 1, 2, 3, 0]


def test_tiny_fp32_two_chunks_per_step():
    device()
    cfg = reduced("tiny", ssf_on=False, chunks_per_step=2)
    print("tiny fp32 B=2", flush=True)
    orc, _ = run_parity(cfg, 8)
    assert orc.sink_count == 1


def test_video_bf16_three_chunks_overflowing_window():
    """B = 3 chunks of 192 tokens leave per step into a 384-token window: the
    ring keeps the last two of them, and every sink decision after the first
    capture reads its chunk's staged copy."""
    device()
    cfg = reduced("video13b", chunks_per_step=3, window_tokens=384)
    print("video bf16 reduced B=3 W=384", flush=True)
    orc, _ = run_parity(cfg, 5)
    assert orc.kv_valid == cfg.window_tokens and orc.sink_count == 1


def test_fourstep_bf16_onetime_negative_two_chunks_per_step():
    device()
    cfg = reduced("fourstep", chunks_per_step=2, ssf_on=False)
    print("fourstep bf16 reduced B=2 onetime", flush=True)
    run_parity(cfg, 6)


def test_video_bf16_variable_group_sizes():
    """Steps take 1 to 3 chunks (capacity B = 3): groups keep their size through
    the slots, leave whole, and append / decide the sink in push order."""
    device()
    cfg = reduced("video13b", chunks_per_step=3, window_tokens=384)
    print("video bf16 reduced, group sizes 1,3,2,2,1,3,2,1", flush=True)
    run_parity(cfg, 8, sizes=[1, 3, 2, 2, 1, 3, 2, 1])


def test_tiny_fp32_full_cfg_with_context():
    device()
    cfg = reduced("tiny", ssf_on=False, ctx_len=12, cfg_type="full", gamma=1.8, delta=1.0)
    print("tiny fp32 full CFG", flush=True)
    orc, _ = run_parity(cfg, 6)
    assert orc.n_steps == 6


def test_image_bf16_full_cfg_four_rows():
    device()
    cfg = reduced("image", cfg_type="full", delta=0.8)
    print("image bf16 reduced full CFG", flush=True)
    run_parity(cfg, 4)


def test_video_bf16_full_cfg_two_chunks_per_step():
    device()
    cfg = reduced("video13b", cfg_type="full", chunks_per_step=2)
    print("video bf16 reduced full CFG B=2", flush=True)
    run_parity(cfg, 6)


def test_tiny_fp32_batch_attention():
    device()
    cfg = reduced("tiny", ssf_on=False, batch_attn=True, t_index=(10, 32, 45))
    print("tiny fp32 batch attention n=3", flush=True)
    run_parity(cfg, 7)


def test_image_bf16_batch_attention():
    device()
    cfg = reduced("image", batch_attn=True)
    print("image bf16 reduced batch attention", flush=True)
    run_parity(cfg, 4)


def test_video_bf16_batch_attention_two_chunks_per_step():
    device()
    cfg = reduced("video13b", batch_attn=True, chunks_per_step=2)
    print("video bf16 reduced batch attention B=2", flush=True)
    orc, _ = run_parity(cfg, 8)
    assert orc.kv_valid == cfg.window_tokens


def test_tiny_fp32_lcm_sampler_three_slots():
    device()
    cfg = reduced("tiny", ssf_on=False, sampler="lcm", t_index=(10, 32, 45))
    print("tiny fp32 LCM sampler n=3", flush=True)
    run_parity(cfg, 7)


def test_video_bf16_lcm_sampler_two_chunks_per_step():
    device()
    cfg = reduced("video13b", sampler="lcm", chunks_per_step=2)
    print("video bf16 reduced LCM sampler B=2", flush=True)
    run_parity(cfg, 6)


def test_tiny_fp32_clean_latent_kv_recompute():
    device()
    cfg = reduced("tiny", ssf_on=False, kv_recompute=True, t_index=(10, 32, 45))
    print("tiny fp32 clean-latent KV recompute n=3", flush=True)
    orc, _ = run_parity(cfg, 9)
    assert orc.sink_count == 1


def test_video_bf16_clean_latent_kv_recompute_two_chunks_per_step():
    device()
    cfg = reduced("video13b", kv_recompute=True, chunks_per_step=2)
    print("video bf16 reduced clean-latent KV recompute B=2", flush=True)
    orc, _ = run_parity(cfg, 8)
    assert orc.kv_valid == cfg.window_tokens


def test_video_bf16_pushes_on_an_io_stream_two_chunks_per_step():
    """Inputs produced and pushed on a second stream (motion reductions,
    entry noise into recycled frame records) overlapped with the steps: the
    same outputs, ring and sink as the oracle."""
    device()
    cfg = reduced("video13b", chunks_per_step=2)
    print("video bf16 reduced B=2, pushes on an IO stream", flush=True)
    orc, _ = run_parity(cfg, 10, io_stream=True)
    assert orc.kv_valid == cfg.window_tokens


def test_tiny_fp32_ssf_pushes_on_an_io_stream():
    device()
    cfg = reduced("tiny")
    print("tiny fp32 SSF, pushes on an IO stream", flush=True)
    run_parity(cfg, 12, io_stream=True)


def test_step_chunks_out_of_range():
    device()
    cfg = reduced("tiny", ssf_on=False, chunks_per_step=2)
    run = StreamRunner(cfg, upload_weights(cfg, gen.make_weights(cfg)))
    x = torch.zeros(run.lat_shape, device=device())
    run.push(x, x)
    for bad in (0, 3):
        with pytest.raises(L.SDError) as ei:
            run.step(chunks=bad)
        assert ei.value.code == L.SD_ERR_ARG
    with pytest.raises(L.SDError) as ei:
        run.step(chunks=2)                     # one chunk pending
    assert ei.value.code == L.SD_ERR_NOT_READY
    run.close()


def test_kv_reset_mid_stream_matches_oracle():
    device()
    cfg = reduced("tiny", ssf_on=False)
    weights = gen.make_weights(cfg)
    orc = OracleStream(cfg, weights)
    run = StreamRunner(cfg, upload_weights(cfg, weights))
    src, nz = gen.LatentSource(cfg), gen.NoiseSource(cfg)
    for k in range(6):
        if k == 3:
            orc.kv_reset()
            run.kv_reset()
        x0, e = src.next(), nz.next()
        po = orc.push_frame(x0, e)
        pg = run.push(to_dev(x0, torch.float32), to_dev(e, torch.float32))
        assert pg.t0 == po.t0
        out_o, so = orc.step()
        sg = run.step()
        torch.cuda.synchronize()
        assert (sg.kv_ptr, sg.kv_valid, sg.sink_count) == (so.kv_ptr, so.kv_valid, so.sink_count)
        if out_o is not None:
            check_close(run.out.cpu().numpy(), out_o, "f32", f"step {k}")
    run.close()


def test_step_errors():
    device()
    cfg = reduced("tiny", ssf_on=False)
    run = StreamRunner(cfg, upload_weights(cfg, gen.make_weights(cfg)))
    with pytest.raises(L.SDError) as ei:
        run.step()
    assert ei.value.code == L.SD_ERR_NOT_READY
    x = torch.zeros(run.lat_shape, device=device())
    for _ in range(4):
        run.push(x, x)
    with pytest.raises(L.SDError) as ei:
        run.push(x, x)
    assert ei.value.code == L.SD_ERR_STATE
    run.close()


# ------------------------------------------------------------------ graph replay of the step
def test_video_bf16_graph_replay_matches_oracle():
    """The step recorded once as a HIP graph and replayed with new rows, RoPE
    bases, window ranges and ring positions each step: the same outputs, ring
    and sink as the oracle; the steady state replays one graph."""
    device()
    cfg = reduced("video13b")
    print("video bf16 reduced, graph replay", flush=True)
    orc, _ = run_parity(cfg, 12, graph=True, transform=scene_cut({7}))
    cap, rep = orc.graph_stats
    print("graph captures / replays:", cap, rep, flush=True)
    assert rep >= 6 and cap <= 6


def test_fourstep_bf16_graph_replay_onetime_negative():
    device()
    cfg = reduced("fourstep", ssf_on=False)
    print("fourstep bf16 reduced, graph replay", flush=True)
    orc, _ = run_parity(cfg, 10, graph=True)
    cap, rep = orc.graph_stats
    assert rep >= 4


def test_video_bf16_graph_replay_variable_group_sizes():
    device()
    cfg = reduced("video13b", chunks_per_step=3, window_tokens=384)
    print("video bf16 reduced B=3, variable groups, graph replay", flush=True)
    orc, _ = run_parity(cfg, 12, graph=True, sizes=[1, 3, 2, 2, 1, 3, 2, 1])
    assert sum(orc.graph_stats) == 12
