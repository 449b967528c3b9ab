"""Pins for oracle.vae: the causal convolution against a pure-Python loop and
unit kernels, causality, chunked streaming against the whole video at once,
and the resampling round trip."""
import numpy as np
import pytest

from oracle import vae
from workloads import gen, get_vae_config


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_conv_matches_python_loop():
    T, H, W, Ci, Co = 3, 3, 4, 2, 3
    x, w, b, cache = rnd(0, T, H, W, Ci), rnd(1, Co, 3, 3, 3, Ci), rnd(2, Co), rnd(3, 2, H, W, Ci)
    y, new_cache = vae.causal_conv3d(x, w, b, cache)

    def src(t, yy, xx, c):
        if not (0 <= yy < H and 0 <= xx < W):
            return 0.0
        return cache[t + 2, yy, xx, c] if t < 0 else x[t, yy, xx, c]

    for t in range(T):
        for yy in range(H):
            for xx in range(W):
                for o in range(Co):
                    acc = b[o]
                    for dt in range(3):
                        for dy in range(3):
                            for dx in range(3):
                                for c in range(Ci):
                                    acc += w[o, dt, dy, dx, c] * src(t + dt - 2, yy + dy - 1, xx + dx - 1, c)
                    assert abs(y[t, yy, xx, o] - acc) < 1e-12
    assert np.array_equal(new_cache, x[1:])


@pytest.mark.parametrize("dt,shift", [(2, 0), (1, 1), (0, 2)])
def test_single_tap_kernel_shifts_in_time(dt, shift):
    """A kernel with one temporal tap dt and the spatial centre copies frame
    t - (2 - dt), reaching into the cache for frames before the chunk."""
    T, H, W, C = 4, 2, 3, 2
    x, cache = rnd(4, T, H, W, C), rnd(5, 2, H, W, C)
    w = np.zeros((C, 3, 3, 3, C))
    for c in range(C):
        w[c, dt, 1, 1, c] = 1.0
    y, _ = vae.causal_conv3d(x, w, np.zeros(C), cache)
    full = np.concatenate([cache, x])
    assert np.array_equal(y, full[2 - shift:2 - shift + T])


def test_convolution_is_causal():
    T, H, W, C = 4, 3, 3, 2
    x, w, b = rnd(6, T, H, W, C), rnd(7, C, 3, 3, 3, C), rnd(8, C)
    y, _ = vae.causal_conv3d(x, w, b)
    x2 = x.copy()
    x2[3] += 1.0
    y2, _ = vae.causal_conv3d(x2, w, b)
    assert np.array_equal(y[:3], y2[:3]) and not np.allclose(y[3], y2[3])


def test_chunked_streaming_equals_the_whole_video():
    v = get_vae_config("small")
    w = gen.make_vae_weights(v)
    src = gen.PixelSource(v)
    chunks = [src.next() for _ in range(3)]
    sv = vae.StreamVAE(v, w)
    lat = [sv.encode_chunk(c) for c in chunks]
    whole = vae.encode_video(v, w, np.concatenate(chunks))
    assert lat[0].shape == (v.latent_t, v.latent_c, v.latent_h, v.latent_w)
    assert np.allclose(np.concatenate(lat), whole, rtol=0, atol=1e-10)
    dec = [sv.decode_chunk(z) for z in lat]
    whole_dec = vae.decode_video(v, w, np.concatenate(lat))
    assert dec[0].shape == (v.frames, 3, v.height, v.width)
    assert np.allclose(np.concatenate(dec), whole_dec, rtol=0, atol=1e-10)
    # without the caches each chunk restarts from zeros: a different video
    fresh = vae.StreamVAE(v, w)
    fresh.encode_chunk(chunks[0])
    fresh.reset()
    assert not np.allclose(fresh.encode_chunk(chunks[1]), lat[1], rtol=0, atol=1e-6)


def test_pool_of_upsample_is_identity_and_norm_is_scale_free():
    x = rnd(9, 2, 3, 4, 5)
    for temporal in (False, True):
        assert np.array_equal(vae.avg_pool(vae.upsample(x, temporal), temporal), x)
    g = 1.0 + 0.1 * rnd(10, 5)
    assert np.allclose(vae.rms_norm_silu(3.0 * x, g, eps=0.0), vae.rms_norm_silu(x, g, eps=0.0), atol=1e-12)
