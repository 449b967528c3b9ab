"""Stream-VAE: chunked causal 3D-convolution encoder / decoder with per-layer
feature caches, written out plainly (test infrastructure: only tests/, the
smoke check and the CPU baseline of bench.py use it).

StreamDiffusionV2 summary, Stream-VAE: a low-latency video VAE variant for
streaming that encodes and decodes short chunks of frames (4 in the pages'
example) instead of a long sequence, and keeps intermediate features cached
inside every 3D convolution so that consecutive chunks stay temporally
coherent.  The pages give no architecture; the reading here (random weights):

* every convolution is causal in time, kernel 3 x 3 x 3, stride 1, spatial
  zero padding 1: output frame t reads input frames t-2, t-1, t; frames
  before the chunk come from the layer's cache, the last two input frames
  of the previous chunk (zeros at the start of the stream);
* after a convolution: RMS normalisation over the channels of each position
  (eps 1e-6, per-channel gain), then SiLU -- per position, so nothing mixes
  time beyond the convolutions;
* encoder: conv 8->c1 (RGB padded with zeros to 8 channels), 2x2 average
  pool, conv c1->c2, 2x2 pool, conv c2->c3, 2x2x2 pool (frame pairs 2j, 2j+1
  of the chunk), conv c3->c3, conv c3->16 (the latent, no norm);
* decoder: conv 16->c3, nearest 2x2x2 upsample, conv c3->c3, nearest 2x2,
  conv c3->c2, nearest 2x2, conv c2->c1, conv c1->3 (the pixels, no norm);
  so a chunk of 4 frames of H x W pixels is a latent of 2 x 16 x H/8 x W/8.

External layouts are channels-first ([T][C][H][W], as the denoiser's latent);
inside, tensors are channels-last [T][H][W][C].  Weights: conv "w" [Cout][3]
[3][3][Cin] (taps (dt, dy, dx)), "b" [Cout], norm gain "g" [Cout].

Pins (tests/test_oracle_vae.py): the convolution against a pure-Python loop;
a unit kernel reproduces its input; causality (a later frame never changes
an earlier output); chunked streaming equals the whole video run at once;
pool / upsample round trips.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Tuple

import numpy as np

KT = 3       # temporal taps; a layer caches KT - 1 = 2 input frames


def causal_conv3d(x, w, b, cache=None):
    """x [T][H][W][Cin], w [Cout][3][3][3][Cin], b [Cout], cache [2][H][W][Cin]
    or None (zeros).  Returns y [T][H][W][Cout] and the new cache (the last two
    frames of [cache | x])."""
    T, H, W, Cin = x.shape
    if cache is None:
        cache = np.zeros((KT - 1, H, W, Cin), x.dtype)
    xt = np.concatenate([cache, x], axis=0)                       # frames -2 .. T-1
    xp = np.pad(xt, ((0, 0), (1, 1), (1, 1), (0, 0)))             # spatial zero padding
    y = np.zeros((T, H, W, w.shape[0]), np.result_type(x, w))
    for dt in range(KT):
        for dy in range(3):
            for dx in range(3):
                y += xp[dt:dt + T, dy:dy + H, dx:dx + W, :] @ w[:, dt, dy, dx, :].T
    return y + b, xt[-(KT - 1):].copy()


def rms_norm_silu(x, g, eps: float = 1e-6):
    """Per position: x / sqrt(mean_c x^2 + eps) * g, then SiLU."""
    n = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g
    return n / (1.0 + np.exp(-n))


def avg_pool(x, temporal: bool):
    """2 x 2 spatial mean (and of frame pairs 2j, 2j+1 when temporal)."""
    T, H, W, C = x.shape
    y = x.reshape(T, H // 2, 2, W // 2, 2, C).mean(axis=(2, 4))
    if temporal:
        y = y.reshape(T // 2, 2, H // 2, W // 2, C).mean(axis=1)
    return y


def upsample(x, temporal: bool):
    """Nearest-neighbour 2x in y and x (and t when temporal)."""
    y = x.repeat(2, axis=1).repeat(2, axis=2)
    if temporal:
        y = y.repeat(2, axis=0)
    return y


# (layer name, Cin, Cout, resampling applied to the layer's input, norm after)
def encoder_layers(c1: int, c2: int, c3: int, zc: int):
    return [("e0", 8, c1, None, True), ("e1", c1, c2, "pool_s", True), ("e2", c2, c3, "pool_s", True),
            ("e3", c3, c3, "pool_st", True), ("e_out", c3, zc, None, False)]


def decoder_layers(c1: int, c2: int, c3: int, zc: int):
    return [("d0", zc, c3, None, True), ("d1", c3, c3, "up_st", True), ("d2", c3, c2, "up_s", True),
            ("d3", c2, c1, "up_s", True), ("d_out", c1, 3, None, False)]


def _resample(x, how):
    if how is None:
        return x
    if how.startswith("pool"):
        return avg_pool(x, how == "pool_st")
    return upsample(x, how == "up_st")


def _run(layers, weights, x, caches):
    """Run a layer list on a channels-last chunk; caches: dict name -> cache
    (updated in place), or None for a cache of zeros."""
    for name, cin, cout, how, norm in layers:
        x = _resample(x, how)
        c = None if caches is None else caches.get(name)
        x, new_cache = causal_conv3d(x, weights[name + ".w"], weights[name + ".b"], c)
        if caches is not None:
            caches[name] = new_cache
        if norm:
            x = rms_norm_silu(x, weights[name + ".g"])
    return x


def pixels_to_cl(pix):
    """[T][3][H][W] -> [T][H][W][8] (channels 3..7 zero)."""
    x = np.transpose(np.asarray(pix, np.float64), (0, 2, 3, 1))
    return np.pad(x, ((0, 0), (0, 0), (0, 0), (0, 8 - x.shape[-1])))


class StreamVAE:
    """Chunk-by-chunk encoder and decoder, each with its own per-layer caches."""

    def __init__(self, cfg, weights: Dict[str, np.ndarray]):
        self.cfg = cfg
        self.w = {k: np.asarray(v, np.float64) for k, v in weights.items()}
        self.enc = encoder_layers(cfg.c1, cfg.c2, cfg.c3, cfg.latent_c)
        self.dec = decoder_layers(cfg.c1, cfg.c2, cfg.c3, cfg.latent_c)
        self.reset()

    def reset(self):
        self.enc_cache: Dict[str, np.ndarray] = {}
        self.dec_cache: Dict[str, np.ndarray] = {}

    def encode_chunk(self, pix):
        """pix [Tp][3][H][W] -> latent [Tp/2][16][H/8][W/8]."""
        z = _run(self.enc, self.w, pixels_to_cl(pix), self.enc_cache)
        return np.transpose(z, (0, 3, 1, 2))

    def decode_chunk(self, lat):
        """latent [T][16][h][w] -> pixels [2T][3][8h][8w]."""
        x = _run(self.dec, self.w, np.transpose(np.asarray(lat, np.float64), (0, 2, 3, 1)), self.dec_cache)
        return np.transpose(x, (0, 3, 1, 2))


def encode_video(cfg, weights, pix):
    """The whole video at once (cache of zeros, every frame in one pass)."""
    w = {k: np.asarray(v, np.float64) for k, v in weights.items()}
    z = _run(encoder_layers(cfg.c1, cfg.c2, cfg.c3, cfg.latent_c), w, pixels_to_cl(pix), None)
    return np.transpose(z, (0, 3, 1, 2))


def decode_video(cfg, weights, lat):
    w = {k: np.asarray(v, np.float64) for k, v in weights.items()}
    x = _run(decoder_layers(cfg.c1, cfg.c2, cfg.c3, cfg.latent_c), w,
             np.transpose(np.asarray(lat, np.float64), (0, 2, 3, 1)), None)
    return np.transpose(x, (0, 3, 1, 2))
