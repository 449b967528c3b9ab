"""Pins for oracle.guidance and oracle.stream: R-CFG identities, the DDIM round
trip, the identity pipeline, the Stream Batch invariant and the integer
state machine."""
import numpy as np
import pytest

from oracle import guidance, schedule
from oracle.dit import Denoiser
from oracle.stream import NotReady, OracleStream, denoise_sequential
from workloads import gen, get_config


def vec(seed, n=50):
    return np.random.default_rng(seed).standard_normal(n)


# ------------------------------------------------------------------ R-CFG identities
def test_rcfg_gamma_one_returns_conditional():
    ec, ep = vec(0), vec(1)
    for delta in (0.0, 0.5, 1.0, 2.0):
        assert np.allclose(guidance.rcfg(ec, ep, 1.0, delta), ec, atol=1e-15)


def test_rcfg_delta_zero_scales_conditional():
    ec, ep = vec(0), vec(1)
    assert np.allclose(guidance.rcfg(ec, ep, 1.4, 0.0), 1.4 * ec, atol=1e-15)


def test_rcfg_is_extrapolation_away_from_the_negative():
    # eps_cfg - delta eps' = gamma (eps_c - delta eps'): the guidance direction
    ec, ep = vec(2), vec(3)
    g, dl = 1.4, 0.7
    assert np.allclose(guidance.rcfg(ec, ep, g, dl) - dl * ep, g * (ec - dl * ep), atol=1e-14)


def test_virtual_residual_at_entry_is_the_entry_noise():
    a, b = schedule.sched_coeffs(get_config("tiny"))
    x0, eps = vec(4), vec(5)
    for tau in (999, 359, 99, 0):
        x = guidance.entry_noise(x0, eps, a[tau], b[tau])
        assert np.allclose(guidance.virtual_residual(x, x0, a[tau], b[tau]), eps, atol=1e-12 / b[tau])


def test_true_noise_recovers_x0():
    a, b = schedule.sched_coeffs(get_config("tiny"))
    x0, eps = vec(6), vec(7)
    tau = 359
    x = guidance.entry_noise(x0, eps, a[tau], b[tau])
    assert np.allclose(guidance.predict_x0(x, eps, a[tau], b[tau]), x0, atol=1e-14)
    # renoise to a lower timestep with the same noise equals noising x0 there
    y = guidance.renoise(x0, eps, a[99], b[99])
    assert np.allclose(y, guidance.entry_noise(x0, eps, a[99], b[99]), atol=0)


# ------------------------------------------------------------------ identity pipeline
@pytest.mark.parametrize("t_index,cfg_type", [((32,), "self"), ((32, 45), "self"),
                                              ((0, 16, 32, 45), "self"), ((0, 16, 32, 45), "onetime"),
                                              ((0, 16, 32, 45), "full")])
def test_identity_pipeline_emits_inputs(t_index, cfg_type):
    """Denoiser replaced by eps_c := eps'.  With delta = 1 every slot has
    eps_cfg = eps' and x0_hat = x0*, so each frame leaves as it came in, in
    push order, n-1 steps after entering -- for any gamma."""
    cfg = get_config("tiny", t_index=t_index, cfg_type=cfg_type, gamma=3.7, delta=1.0, ssf_on=False)
    st = OracleStream(cfg, None, identity_denoiser=True)
    src, nz = gen.LatentSource(cfg), gen.NoiseSource(cfg)
    n = cfg.n_slots
    inputs, outs = [], []
    for k in range(10):
        x0 = src.next()
        inputs.append(x0)
        st.push_frame(x0, nz.next())
        out, info = st.step()
        assert info.has_output == (k >= n - 1)
        if out is not None:
            assert info.frame_id == k - (n - 1)
            outs.append(out)
    assert len(outs) == 10 - (n - 1)
    for k, o in enumerate(outs):
        assert np.allclose(o, inputs[k], atol=1e-11)


def test_step_without_push_is_not_ready():
    cfg = get_config("tiny", ssf_on=False)
    st = OracleStream(cfg, None, identity_denoiser=True)
    with pytest.raises(NotReady):
        st.step()


# ------------------------------------------------------------------ Stream Batch invariant
def small_cfg(**kw):
    base = dict(n_blocks=1, d_model=32, n_heads=2, d_ffn=64, d_freq=16, latent_h=8, latent_w=8,
                ssf_on=False, sink_tokens=4, window_tokens=48)
    base.update(kw)
    return get_config("tiny", **base)


@pytest.mark.parametrize("t_index", [(32, 45), (0, 16, 32, 45)])
def test_stream_batch_equals_sequential_with_frozen_cache(t_index):
    cfg = small_cfg(t_index=t_index)
    w = gen.make_weights(cfg)
    st = OracleStream(cfg, w, freeze_cache=True)
    net = Denoiser(cfg, w)
    a, b = schedule.sched_coeffs(cfg)
    src, nz = gen.LatentSource(cfg), gen.NoiseSource(cfg)
    frames = []
    outs = []
    for k in range(7):
        x0, e = src.next(), nz.next()
        info = st.push_frame(x0, e)
        frames.append((x0, e, info.t0))
        out, _ = st.step()
        if out is not None:
            outs.append(out)
    taus = schedule.taus_from_t_index(cfg)
    for k, o in enumerate(outs):
        x0, e, t0 = frames[k]
        ref = denoise_sequential(cfg, net, x0.astype(np.float64), e.astype(np.float64), taus, t0, a, b)
        assert np.array_equal(o, ref)          # bit-identical: same operations, same order


def test_stream_batch_equals_sequential_with_live_cache():
    """With the cache live, frame k's i-th step reads the snapshot of step
    k+i; replaying each frame alone against those snapshots gives the
    pipeline's output bit for bit."""
    cfg = small_cfg(t_index=(0, 16, 32, 45))
    w = gen.make_weights(cfg)
    st = OracleStream(cfg, w)
    net = Denoiser(cfg, w)
    a, b = schedule.sched_coeffs(cfg)
    src, nz = gen.LatentSource(cfg), gen.NoiseSource(cfg)
    frames, outs, snaps = [], [], []
    for k in range(8):
        x0, e = src.next(), nz.next()
        info = st.push_frame(x0, e)
        frames.append((x0, e, info.t0))
        snaps.append(st.cache_snapshot())
        out, _ = st.step()
        if out is not None:
            outs.append(out)
    assert st.kv_valid == cfg.window_tokens and st.sink_count == 1
    taus = schedule.taus_from_t_index(cfg)
    n = cfg.n_slots
    for k, o in enumerate(outs):
        x0, e, t0 = frames[k]
        ref = denoise_sequential(cfg, net, x0.astype(np.float64), e.astype(np.float64), taus, t0, a, b,
                                 snapshots=[snaps[k + i] for i in range(n)])
        assert np.array_equal(o, ref)


# ------------------------------------------------------------------ integer state
def test_ring_pointer_valid_and_sink_trace():
    cfg = small_cfg(t_index=(32, 45), window_tokens=40)     # L = 16 tokens per chunk
    st = OracleStream(cfg, gen.make_weights(cfg))
    src, nz = gen.LatentSource(cfg), gen.NoiseSource(cfg)
    trace = []
    for k in range(7):
        st.push_frame(src.next(), nz.next())
        _, info = st.step()
        trace.append((info.has_output, info.kv_ptr, info.kv_valid, info.sink_count))
    assert trace == [(False, 0, 0, 0), (True, 16, 16, 1), (True, 32, 32, 1), (True, 8, 40, 1),
                     (True, 24, 40, 1), (True, 0, 40, 1), (True, 16, 40, 1)]
    st.kv_reset()
    assert (st.kv_ptr, st.kv_valid, st.sink_count, st.rope_p) == (0, 0, 0, 0)


@pytest.mark.parametrize("T,reset,expect", [(1, 3, [0, 1, 2, 3, 0, 1, 2, 3, 0]),
                                           (2, 3, [0, 2, 0, 2, 0]),
                                           (2, 4, [0, 2, 0, 2, 0]),
                                           (2, 5, [0, 2, 4, 0, 2])])
def test_rope_temporal_positions_wrap(T, reset, expect):
    cfg = small_cfg(latent_t=T, rope_reset=reset)
    st = OracleStream(cfg, None, identity_denoiser=True)
    src, nz = gen.LatentSource(cfg), gen.NoiseSource(cfg)
    got = [st.push_frame(src.next(), nz.next()).t0 for _ in expect]
    assert got == expect


def test_ssf_skip_cap_trace():
    cfg = get_config("tiny", max_skip_frame=3)
    st = OracleStream(cfg, None, identity_denoiser=True)
    frame = np.full(cfg.ssf_shape, 9, np.uint8)             # identical frames: p = 1
    src, nz = gen.LatentSource(cfg), gen.NoiseSource(cfg)
    skipped = [st.push_frame(src.next(), nz.next(), frame, 0.0).skipped for _ in range(10)]
    assert skipped == [False, True, True, True, False, True, True, True, False, True]
    # u at or above p never skips (strict u < p)
    st2 = OracleStream(cfg, None, identity_denoiser=True)
    half = frame.copy()
    r = [st2.push_frame(src.next(), nz.next(), half, 0.999999).skipped for _ in range(3)]
    assert r == [False, True, True]            # p = 1 > 0.999999
    st3 = OracleStream(cfg, None, identity_denoiser=True)
    g = np.zeros(cfg.ssf_shape, np.uint8); g[0, 0, 0] = 5
    h = np.zeros(cfg.ssf_shape, np.uint8); h[0, 0, 1] = 5
    r = [st3.push_frame(src.next(), nz.next(), f, 0.0).skipped for f in (g, h, g)]
    assert r == [False, False, False]           # cos = 0 -> p = 0, u = 0 is not < 0


# ------------------------------------------------------------------ B > 1 chunks per step
@pytest.mark.parametrize("B,t_index,cfg_type", [(2, (32, 45), "self"), (3, (0, 16, 32, 45), "self"),
                                                (2, (0, 16, 32, 45), "onetime")])
def test_identity_pipeline_emits_inputs_b_chunks(B, t_index, cfg_type):
    """With B chunks per step the B frames of a group enter and leave
    together: each leaves unchanged (identity denoiser, delta = 1), in push
    order, n-1 steps after entering."""
    cfg = get_config("tiny", t_index=t_index, cfg_type=cfg_type, gamma=2.1, delta=1.0, ssf_on=False,
                     chunks_per_step=B)
    st = OracleStream(cfg, None, identity_denoiser=True)
    src, nz = gen.LatentSource(cfg), gen.NoiseSource(cfg)
    n = cfg.n_slots
    inputs, outs = [], []
    for k in range(6):
        for _ in range(B):
            x0 = src.next()
            inputs.append(x0)
            st.push_frame(x0, nz.next())
        out, info = st.step()
        assert info.has_output == (k >= n - 1) and info.n_out == (B if k >= n - 1 else 0)
        assert info.rows == B * min(k + 1, n) + (B if cfg_type == "onetime" else 0)
        if out is not None:
            assert out.shape == (B,) + inputs[0].shape
            assert info.frame_id == (k - (n - 1)) * B
            outs.extend(out)
    assert len(outs) == (6 - (n - 1)) * B
    for k, o in enumerate(outs):
        assert np.allclose(o, inputs[k], atol=1e-11)


def test_b_chunks_step_needs_b_pending_frames():
    cfg = get_config("tiny", ssf_on=False, chunks_per_step=2)
    st = OracleStream(cfg, None, identity_denoiser=True)
    src, nz = gen.LatentSource(cfg), gen.NoiseSource(cfg)
    st.push_frame(src.next(), nz.next())
    with pytest.raises(NotReady):
        st.step()


def test_stream_batch_equals_sequential_b_chunks_live_cache():
    """B = 2 with the cache live: each frame of a group, replayed alone
    against the snapshots of the steps it spent in the pipeline, gives the
    emitted latent bit for bit (frames of one group share their snapshots and
    do not attend to each other)."""
    cfg = small_cfg(t_index=(32, 45), chunks_per_step=2)
    w = gen.make_weights(cfg)
    st = OracleStream(cfg, w)
    net = Denoiser(cfg, w)
    a, b = schedule.sched_coeffs(cfg)
    src, nz = gen.LatentSource(cfg), gen.NoiseSource(cfg)
    frames, outs, snaps = [], [], []
    for k in range(5):
        for _ in range(2):
            x0, e = src.next(), nz.next()
            info = st.push_frame(x0, e)
            frames.append((x0, e, info.t0, k))
        snaps.append(st.cache_snapshot())
        out, _ = st.step()
        if out is not None:
            outs.extend(out)
    taus = schedule.taus_from_t_index(cfg)
    n = cfg.n_slots
    assert len(outs) == 8
    for j, o in enumerate(outs):
        x0, e, t0, k = frames[j]
        ref = denoise_sequential(cfg, net, x0.astype(np.float64), e.astype(np.float64), taus, t0, a, b,
                                 snapshots=[snaps[k + i] for i in range(n)])
        assert np.array_equal(o, ref)


def test_ring_pointer_and_sink_trace_b_chunks_overflowing_window():
    """B = 2 chunks of L = 16 tokens leave per step into a 24-token window:
    the two chunks append in order, so the window keeps the last 24 tokens
    (ptr advances by 32 mod 24); the first leaving chunk captures the sink."""
    cfg = small_cfg(t_index=(32, 45), window_tokens=24, chunks_per_step=2)
    st = OracleStream(cfg, gen.make_weights(cfg))
    src, nz = gen.LatentSource(cfg), gen.NoiseSource(cfg)
    trace = []
    for k in range(4):
        for _ in range(2):
            st.push_frame(src.next(), nz.next())
        _, info = st.step()
        trace.append((info.has_output, info.n_out, info.kv_ptr, info.kv_valid, info.sink_count))
    assert trace == [(False, 0, 0, 0, 0), (True, 2, 8, 24, 1), (True, 2, 16, 24, 1), (True, 2, 0, 24, 1)]


def test_identity_pipeline_variable_group_sizes():
    """Steps may take fewer chunks than the capacity B: each group keeps its
    size through the slots and leaves whole, frames in push order."""
    cfg = get_config("tiny", t_index=(0, 16, 32, 45), gamma=1.7, delta=1.0, ssf_on=False, chunks_per_step=3)
    st = OracleStream(cfg, None, identity_denoiser=True)
    src, nz = gen.LatentSource(cfg), gen.NoiseSource(cfg)
    sizes = [1, 3, 2, 2, 1, 3, 2, 1]
    inputs, outs, emitted_sizes = [], [], []
    for b in sizes:
        for _ in range(b):
            x0 = src.next()
            inputs.append(x0)
            st.push_frame(x0, nz.next())
        out, info = st.step(b)
        if out is not None:
            emitted_sizes.append(info.n_out)
            outs.extend(out)
    assert emitted_sizes == sizes[:len(sizes) - 3]          # a group leaves n - 1 = 3 steps after entering
    for k, o in enumerate(outs):
        assert np.allclose(o, inputs[k], atol=1e-11)
    with pytest.raises(ValueError):
        st.step(4)


# ------------------------------------------------------------------ full CFG (2n rows)
def full_cfg_run(cfg, w, ctx_pos, ctx_neg, steps, B=1):
    st = OracleStream(cfg, w, ctx_pos=ctx_pos, ctx_neg=ctx_neg)
    src, nz = gen.LatentSource(cfg), gen.NoiseSource(cfg)
    frames, outs, snaps, rows = [], [], [], []
    for k in range(steps):
        for _ in range(B):
            x0, e = src.next(), nz.next()
            info = st.push_frame(x0, e)
            frames.append((x0, e, info.t0))
        snaps.append(st.cache_snapshot())
        out, info = st.step()
        rows.append(info.rows)
        if out is not None:
            outs.extend([out] if B == 1 else list(out))
    return st, frames, outs, snaps, rows


def test_full_cfg_equals_textbook_guidance_replayed_per_frame():
    """Full CFG with delta = 1: each frame, replayed alone against the cache
    snapshots it read, with the standard guidance eps_u + gamma (eps_c - eps_u)
    from one forward under each prompt and the deterministic DDIM update."""
    cfg = small_cfg(t_index=(0, 16, 32, 45), ctx_len=6, cfg_type="full", gamma=1.7, delta=1.0)
    w = gen.make_weights(cfg)
    cp, cn = gen.make_context(cfg), gen.make_context(cfg, negative=True)
    st, frames, outs, snaps, rows = full_cfg_run(cfg, w, cp, cn, 8)
    n = cfg.n_slots
    assert rows == [2 * min(k + 1, n) for k in range(8)]
    net = Denoiser(cfg, w)
    kv_pos = [net.cross_kv(cp, b) for b in range(cfg.n_blocks)]
    kv_neg = [net.cross_kv(cn, b) for b in range(cfg.n_blocks)]
    a, b = schedule.sched_coeffs(cfg)
    taus = schedule.taus_from_t_index(cfg)
    assert len(outs) == 8 - (n - 1)
    for k, o in enumerate(outs):
        x0, e, t0 = frames[k]
        x = a[taus[0]] * x0.astype(np.float64) + b[taus[0]] * e.astype(np.float64)
        for i, tau in enumerate(taus):
            ec = net.forward_row(x, tau, t0, snaps[k + i], kv_pos)
            eu = net.forward_row(x, tau, t0, snaps[k + i], kv_neg)
            eps = eu + cfg.gamma * (ec - eu)
            x0h = (x - b[tau] * eps) / a[tau]
            if i + 1 < n:
                x = a[taus[i + 1]] * x0h + b[taus[i + 1]] * eps
        assert np.allclose(o, x0h, rtol=0, atol=1e-11 * max(1.0, np.abs(x0h).max()))


@pytest.mark.parametrize("B", [1, 2])
def test_full_cfg_with_the_same_prompt_twice_is_unguided(B):
    """With the negative prompt equal to the positive one, eps_u = eps_c and
    the guided prediction is eps_c for any gamma: the same stream as
    self-negative R-CFG at gamma = 1, whose residual term cancels."""
    base = dict(t_index=(32, 45), ctx_len=5, gamma=1.0, delta=1.0, chunks_per_step=B)
    cfg_s = small_cfg(cfg_type="self", **base)
    cfg_f = small_cfg(cfg_type="full", **{**base, "gamma": 2.9})
    w = gen.make_weights(cfg_s)
    cp = gen.make_context(cfg_s)
    _, _, outs_s, _, _ = full_cfg_run(cfg_s, w, cp, None, 5, B)
    _, _, outs_f, _, rows = full_cfg_run(cfg_f, w, cp, cp, 5, B)
    assert rows[-1] == 2 * B * cfg_f.n_slots
    assert len(outs_s) == len(outs_f) == 4 * B
    for o_s, o_f in zip(outs_s, outs_f):
        assert np.allclose(o_f, o_s, rtol=0, atol=1e-10)


def test_full_cfg_needs_a_negative_context():
    cfg = small_cfg(ctx_len=4, cfg_type="full")
    with pytest.raises(ValueError):
        OracleStream(cfg, gen.make_weights(cfg), ctx_pos=gen.make_context(cfg))


# ------------------------------------------------------------------ LCM-style re-noise
def lcm_noise(nz, n):
    return np.stack([nz.next() for _ in range(n)])


@pytest.mark.parametrize("t_index", [(32, 45), (0, 16, 32, 45)])
def test_lcm_identity_pipeline_emits_inputs(t_index):
    """With eps_c := eps' and delta = 1, x0_hat = x0 at every slot whatever
    noise the previous slot re-noised with."""
    cfg = get_config("tiny", t_index=t_index, sampler="lcm", gamma=2.3, delta=1.0, ssf_on=False)
    st = OracleStream(cfg, None, identity_denoiser=True)
    src, nz = gen.LatentSource(cfg), gen.NoiseSource(cfg)
    n, ins, outs = cfg.n_slots, [], []
    for _ in range(8):
        x0 = src.next()
        ins.append(x0)
        st.push_frame(x0, lcm_noise(nz, n))
        out, _ = st.step()
        if out is not None:
            outs.append(out)
    for k, o in enumerate(outs):
        assert np.allclose(o, ins[k], atol=1e-11)


def test_lcm_slots_hold_the_fresh_noise_closed_form():
    """After the first step the frame's slot-1 latent is exactly
    a1 x0_hat + b1 z1 (z1 the frame's second noise latent), not the DDIM
    a1 x0_hat + b1 eps_cfg."""
    cfg = small_cfg(t_index=(16, 45), sampler="lcm", window_tokens=0, sink_tokens=0)
    w = gen.make_weights(cfg)
    st = OracleStream(cfg, w)
    net = Denoiser(cfg, w)
    a, b = schedule.sched_coeffs(cfg)
    src, nz = gen.LatentSource(cfg), gen.NoiseSource(cfg)
    x0 = src.next()
    z = lcm_noise(nz, 2)
    info = st.push_frame(x0, z)
    st.step()
    t0, t1 = info.taus
    x = a[t0] * x0.astype(np.float64) + b[t0] * z[0].astype(np.float64)
    ec = net.forward_row(x, t0, info.t0)
    ep = (x - a[t0] * x0) / b[t0]
    eps = cfg.delta * ep + cfg.gamma * (ec - cfg.delta * ep)
    x0h = (x - b[t0] * eps) / a[t0]
    want = a[t1] * x0h + b[t1] * z[1].astype(np.float64)
    assert np.allclose(st.slots[0][0].x, want, rtol=0, atol=1e-12)
    assert not np.allclose(st.slots[0][0].x, a[t1] * x0h + b[t1] * eps, rtol=0, atol=1e-6)


def test_lcm_needs_n_noise_latents():
    cfg = get_config("tiny", sampler="lcm", ssf_on=False)
    st = OracleStream(cfg, None, identity_denoiser=True)
    src, nz = gen.LatentSource(cfg), gen.NoiseSource(cfg)
    with pytest.raises(ValueError):
        st.push_frame(src.next(), nz.next())


# ------------------------------------------------------------------ clean-latent KV recompute
def test_kv_recompute_appends_the_clean_forward():
    """The ring entries a leaving chunk appends are the per-block K/V of a
    forward of its emitted latent at tau = 0 against the step's snapshot,
    and the emitted frames are those of the stream without recompute up to
    the first step that reads a recomputed entry."""
    cfg = small_cfg(t_index=(16, 45), kv_recompute=True)
    w = gen.make_weights(cfg)
    net = Denoiser(cfg, w)
    st = OracleStream(cfg, w)
    ref = OracleStream(cfg.replace(kv_recompute=False), w)
    src, nz = gen.LatentSource(cfg), gen.NoiseSource(cfg)
    L, W = cfg.tokens, cfg.window_tokens
    for k in range(5):
        x0, e = src.next(), nz.next()
        info = st.push_frame(x0, e)
        ref.push_frame(x0, e)
        snap = st.cache_snapshot()
        ptr = st.kv_ptr
        out, si = st.step()
        out_r, _ = ref.step()
        if k < 2:                        # the first append is read from step 2 on
            assert (out is None and out_r is None) or np.array_equal(out, out_r)
        if out is not None:
            assert si.rows == cfg.n_slots + 1
            f0 = k - (cfg.n_slots - 1)
            t0 = f0 * cfg.latent_t       # RoPE base of the leaving frame (no wrap here)
            _, own, _ = net.forward_row(out, 0, t0, snap, None, collect=True)
            pos = [(ptr + j) % W for j in range(L)]
            for b in range(cfg.n_blocks):
                assert np.array_equal(st.ringK[b][pos], own[b][0])
                assert np.array_equal(st.ringV[b][pos], own[b][1])
    assert any(not np.array_equal(a, b) for a, b in [(st.ringK, ref.ringK)])


def test_kv_recompute_frozen_cache_changes_nothing_emitted():
    cfg = small_cfg(t_index=(0, 16, 32, 45), kv_recompute=True)
    w = gen.make_weights(cfg)
    a = OracleStream(cfg, w, freeze_cache=True)
    b = OracleStream(cfg.replace(kv_recompute=False), w, freeze_cache=True)
    src, nz = gen.LatentSource(cfg), gen.NoiseSource(cfg)
    for _ in range(6):
        x0, e = src.next(), nz.next()
        a.push_frame(x0, e)
        b.push_frame(x0, e)
        oa, ia = a.step()
        ob, ib = b.step()
        assert (oa is None) == (ob is None)
        if oa is not None:
            assert np.array_equal(oa, ob) and ia.rows == ib.rows + 1
