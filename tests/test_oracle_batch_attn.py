"""Pins for cross-frame batch attention in the oracle (Denoiser.forward_batch
and the stream's batch_attn switch): a batch of one row is forward_row bit for
bit; duplicating a row leaves its prediction unchanged (softmax over repeated
keys); the batch is permutation-equivariant; rows influence each other only
with the switch on; a one-row stream is unchanged by the switch."""
import numpy as np
import pytest

from oracle.dit import Denoiser
from oracle.stream import OracleStream
from workloads import gen, get_config


def cfg_(**kw):
    base = dict(n_blocks=2, d_model=32, n_heads=2, d_ffn=64, d_freq=16, latent_h=8, latent_w=8, ssf_on=False,
                sink_tokens=4, window_tokens=48, ctx_len=5)
    base.update(kw)
    return get_config("tiny", **base)


def setup(seed=0, **kw):
    cfg = cfg_(**kw)
    w = gen.make_weights(cfg)
    net = Denoiser(cfg, w)
    rng = np.random.default_rng(seed)
    H, hd = cfg.n_heads, cfg.head_dim
    cache = [(rng.standard_normal((20, H, hd)), rng.standard_normal((20, H, hd))) for _ in range(cfg.n_blocks)]
    ctx = [net.cross_kv(gen.make_context(cfg), b) for b in range(cfg.n_blocks)]
    lat = (cfg.latent_t, cfg.latent_c, cfg.latent_h, cfg.latent_w)
    rows = [(rng.standard_normal(lat), tau, t0) for tau, t0 in ((359, 0), (99, 1), (719, 3))]
    return cfg, net, cache, ctx, rows


def test_batch_of_one_row_is_forward_row():
    cfg, net, cache, ctx, rows = setup()
    x, tau, t0 = rows[0]
    got = net.forward_batch([rows[0]], cache, ctx, collect={0})[0]
    ref = net.forward_row(x, tau, t0, cache, ctx, collect=True)
    assert np.array_equal(got[0], ref[0])
    assert np.array_equal(got[2], ref[2])
    for (k1, v1), (k2, v2) in zip(got[1], ref[1]):
        assert np.array_equal(k1, k2) and np.array_equal(v1, v2)


def test_duplicated_row_keeps_its_prediction():
    """Two copies of a row and no cache: every key and value appears twice,
    the softmax weights halve and the attention output is unchanged."""
    cfg, net, cache, ctx, rows = setup()
    x, tau, t0 = rows[1]
    ref = net.forward_row(x, tau, t0, None, ctx)
    a, b = net.forward_batch([rows[1], rows[1]], None, ctx)
    assert np.allclose(a, ref, rtol=0, atol=1e-12) and np.allclose(b, ref, rtol=0, atol=1e-12)


def test_batch_is_permutation_equivariant():
    cfg, net, cache, ctx, rows = setup()
    out = net.forward_batch(rows, cache, ctx)
    perm = [2, 0, 1]
    outp = net.forward_batch([rows[i] for i in perm], cache, ctx)
    for j, i in enumerate(perm):
        assert np.allclose(outp[j], out[i], rtol=0, atol=1e-12)


def test_rows_see_each_other_only_in_a_batch():
    cfg, net, cache, ctx, rows = setup()
    out = net.forward_batch(rows, cache, ctx)
    x1, tau1, t01 = rows[1]
    changed = [rows[0], (x1 + 1.0, tau1, t01), rows[2]]
    out2 = net.forward_batch(changed, cache, ctx)
    assert np.abs(out2[0] - out[0]).max() > 1e-6          # row 0 reads row 1's tokens
    # without the batch, row 0 is forward_row whatever row 1 holds
    x0, tau0, t00 = rows[0]
    assert not np.allclose(out[0], net.forward_row(x0, tau0, t00, cache, ctx), rtol=0, atol=1e-9)


def test_one_row_stream_is_unchanged_by_batch_attention():
    outs = []
    for flag in (False, True):
        cfg = cfg_(t_index=(32,), batch_attn=flag)
        w = gen.make_weights(cfg)
        st = OracleStream(cfg, w, ctx_pos=gen.make_context(cfg))
        src, nz = gen.LatentSource(cfg), gen.NoiseSource(cfg)
        got = []
        for _ in range(4):
            st.push_frame(src.next(), nz.next())
            got.append(st.step()[0])
        outs.append(got)
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_batch_attention_stream_differs_and_needs_self_guidance():
    cfg = cfg_(t_index=(32, 45), batch_attn=True)
    w = gen.make_weights(cfg)
    res = []
    for flag in (False, True):
        st = OracleStream(cfg.replace(batch_attn=flag), w, ctx_pos=gen.make_context(cfg))
        src, nz = gen.LatentSource(cfg), gen.NoiseSource(cfg)
        for _ in range(3):
            st.push_frame(src.next(), nz.next())
            out, info = st.step()
        res.append(out)
        assert info.rows == 2
    assert np.abs(res[0] - res[1]).max() > 1e-6
    with pytest.raises(ValueError):
        OracleStream(cfg.replace(cfg_type="onetime"), w, ctx_pos=gen.make_context(cfg),
                     ctx_neg=gen.make_context(cfg, negative=True))
