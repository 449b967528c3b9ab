"""Seeded input generators (NumPy PCG64).

Seeds: weights 0, latents 1, entry noise 2, SSF uniforms 3, positive context 4,
negative context 5, SSF frames 6.  Every generator is deterministic in
(config, seed, index) and returns float32 (or uint8 for SSF frames).

Weights are drawn N(0, 0.02) tensor by tensor in the canonical order of
``param_specs``; for a bf16 configuration each value is rounded to the nearest
bf16 (ties to even) and kept as float32, so the CPU side and the device see the
same numbers.
"""
from __future__ import annotations

import numpy as np

from .configs import Config

SEED_WEIGHTS = 0
SEED_LATENT = 1
SEED_NOISE = 2
SEED_UNIFORM = 3
SEED_CTX_POS = 4
SEED_CTX_NEG = 5
SEED_SSF = 6
SEED_VAE_WEIGHTS = 7
SEED_VAE_PIXELS = 8

WEIGHT_STD = 0.02


# --------------------------------------------------------------------------
# parameter inventory
# --------------------------------------------------------------------------
GLOBAL_PARAMS_PRE = ("t_w1", "t_b1", "t_w2", "t_b2", "mod_w", "mod_b", "blk_mod", "pe_w", "pe_b")
BLOCK_PARAMS_SELF = ("qkv_w", "qkv_b", "o_w", "o_b")
BLOCK_PARAMS_CROSS = ("cq_w", "cq_b", "ckv_w", "ckv_b", "co_w", "co_b")
BLOCK_PARAMS_FFN = ("f1_w", "f1_b", "f2_w", "f2_b")
GLOBAL_PARAMS_POST = ("fin_w", "fin_b", "head_w", "head_b")


def param_specs(cfg: Config):
    """Canonical (name, shape) list.  Linear weights are [out, in]; per-block
    tensors carry a leading block axis.  The order is the draw order."""
    d, F, nb = cfg.d_model, cfg.d_ffn, cfg.n_blocks
    specs = [
        ("t_w1", (d, cfg.d_freq)), ("t_b1", (d,)),
        ("t_w2", (d, d)), ("t_b2", (d,)),
        ("mod_w", (6 * d, d)), ("mod_b", (6 * d,)),
        ("blk_mod", (nb, 6 * d)),
        ("pe_w", (d, cfg.patch_dim)), ("pe_b", (d,)),
        ("qkv_w", (nb, 3 * d, d)), ("qkv_b", (nb, 3 * d)),
        ("o_w", (nb, d, d)), ("o_b", (nb, d)),
    ]
    if cfg.ctx_len > 0:
        specs += [
            ("cq_w", (nb, d, d)), ("cq_b", (nb, d)),
            ("ckv_w", (nb, 2 * d, d)), ("ckv_b", (nb, 2 * d)),
            ("co_w", (nb, d, d)), ("co_b", (nb, d)),
        ]
    specs += [
        ("f1_w", (nb, F, d)), ("f1_b", (nb, F)),
        ("f2_w", (nb, d, F)), ("f2_b", (nb, d)),
        ("fin_w", (2 * d, d)), ("fin_b", (2 * d,)),
        ("head_w", (cfg.patch_dim, d)), ("head_b", (cfg.patch_dim,)),
    ]
    return specs


def param_count(cfg: Config) -> int:
    return int(sum(int(np.prod(s)) for _, s in param_specs(cfg)))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); the
    result is returned as float32 holding exactly representable values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def make_weights(cfg: Config, seed: int = SEED_WEIGHTS, std: float = WEIGHT_STD):
    """All denoiser parameters as a dict of float32 arrays."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name, shape in param_specs(cfg):
        w = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
        if cfg.dtype == "bf16":
            w = round_bf16(w)
        out[name] = w
    return out


def frame_noise(cfg: Config, nz: "NoiseSource"):
    """The noise one push takes: the entry noise, or for the LCM sampler the
    entry noise and then one latent per later slot ([n][T][C][H][W])."""
    if getattr(cfg, "sampler", "ddim") == "lcm":
        return np.stack([nz.next() for _ in range(cfg.n_slots)])
    return nz.next()


def make_context(cfg: Config, negative: bool = False):
    if cfg.ctx_len == 0:
        return None
    rng = np.random.Generator(np.random.PCG64(SEED_CTX_NEG if negative else SEED_CTX_POS))
    c = rng.standard_normal(size=(cfg.ctx_len, cfg.d_model), dtype=np.float32)
    return round_bf16(c) if cfg.dtype == "bf16" else c


# --------------------------------------------------------------------------
# per-push inputs
# --------------------------------------------------------------------------
def latent_shape(cfg: Config):
    return (cfg.latent_t, cfg.latent_c, cfg.latent_h, cfg.latent_w)


class LatentSource:
    """Sequence of clean input latents x0, one chunk [T][C][H][W] per call.

    tiny     : independent N(0,1) chunks.
    image    : random walk, x_{f+1} = x_f + N(0, 0.05^2).
    fourstep : alternating 32-frame segments, static (delta 0) then moving
               (delta ~ N(0, 0.3^2)), starting from N(0,1).
    video*   : per channel a sum of 8 Gaussian blobs (sigma 6 px, amplitude
               N(0,1)) translating at U[0,4] px/frame in a random direction,
               velocities redrawn every 30 chunks, a scene cut (new blobs)
               every 100 chunks, plus N(0, 0.05^2) per frame.
    """

    def __init__(self, cfg: Config, seed: int = SEED_LATENT, kind: str | None = None):
        self.cfg = cfg
        self.rng = np.random.Generator(np.random.PCG64(seed))
        self.kind = kind or {"tiny": "iid", "image": "walk", "fourstep": "segments"}.get(cfg.name, "blobs")
        self.i = 0
        self.prev = None
        self.shape = latent_shape(cfg)
        if self.kind == "blobs":
            self._new_scene()

    # blob scene state
    def _new_scene(self):
        c = self.cfg
        nb = 8
        self.bx = self.rng.uniform(0, c.latent_w, size=(c.latent_c, nb))
        self.by = self.rng.uniform(0, c.latent_h, size=(c.latent_c, nb))
        self.ba = self.rng.standard_normal(size=(c.latent_c, nb))
        self._new_velocity()

    def _new_velocity(self):
        c = self.cfg
        speed = self.rng.uniform(0.0, 4.0)
        ang = self.rng.uniform(0.0, 2 * np.pi)
        self.vx, self.vy = speed * np.cos(ang), speed * np.sin(ang)

    def _blob_frame(self):
        c = self.cfg
        yy = np.arange(c.latent_h, dtype=np.float64)[:, None]
        xx = np.arange(c.latent_w, dtype=np.float64)[None, :]
        out = np.zeros((c.latent_c, c.latent_h, c.latent_w))
        s2 = 2.0 * 6.0 ** 2
        for ch in range(c.latent_c):
            for j in range(self.bx.shape[1]):
                dx = (xx - self.bx[ch, j] + c.latent_w / 2) % c.latent_w - c.latent_w / 2
                dy = (yy - self.by[ch, j] + c.latent_h / 2) % c.latent_h - c.latent_h / 2
                out[ch] += self.ba[ch, j] * np.exp(-(dx * dx + dy * dy) / s2)
        out += 0.05 * self.rng.standard_normal(size=out.shape)
        self.bx += self.vx
        self.by += self.vy
        return out.astype(np.float32)

    def next(self) -> np.ndarray:
        c, k = self.cfg, self.kind
        if k == "iid":
            x = self.rng.standard_normal(size=self.shape, dtype=np.float32)
        elif k == "walk":
            if self.prev is None:
                x = self.rng.standard_normal(size=self.shape, dtype=np.float32)
            else:
                x = self.prev + np.float32(0.05) * self.rng.standard_normal(size=self.shape, dtype=np.float32)
        elif k == "segments":
            if self.prev is None:
                x = self.rng.standard_normal(size=self.shape, dtype=np.float32)
            elif (self.i // 32) % 2 == 0:
                x = self.prev.copy()
            else:
                x = self.prev + np.float32(0.3) * self.rng.standard_normal(size=self.shape, dtype=np.float32)
        else:
            if self.i > 0 and self.i % 100 == 0:
                self._new_scene()
            elif self.i > 0 and self.i % 30 == 0:
                self._new_velocity()
            x = np.stack([self._blob_frame() for _ in range(c.latent_t)])
        self.prev = x
        self.i += 1
        return np.ascontiguousarray(x, dtype=np.float32)


class NoiseSource:
    """Entry noise epsilon ~ N(0,1), one latent-shaped chunk per push."""

    def __init__(self, cfg: Config, seed: int = SEED_NOISE):
        self.rng = np.random.Generator(np.random.PCG64(seed))
        self.shape = latent_shape(cfg)

    def next(self) -> np.ndarray:
        return self.rng.standard_normal(size=self.shape, dtype=np.float32)


class UniformSource:
    """SSF uniforms u in [0,1), float64, one per push."""

    def __init__(self, seed: int = SEED_UNIFORM):
        self.rng = np.random.Generator(np.random.PCG64(seed))

    def next(self) -> float:
        return float(self.rng.random())


class SSFFrameSource:
    """uint8 frames [h][w][c]: a fixed uniform base image U{0..255} plus
    N(0, 3^2) per frame, rounded and clipped to [0, 255]."""

    def __init__(self, cfg: Config, seed: int = SEED_SSF, noise_std: float = 3.0):
        self.rng = np.random.Generator(np.random.PCG64(seed))
        self.base = self.rng.integers(0, 256, size=cfg.ssf_shape).astype(np.float64)
        self.std = noise_std

    def next(self) -> np.ndarray:
        f = self.base + self.std * self.rng.standard_normal(size=self.base.shape)
        return np.clip(np.rint(f), 0, 255).astype(np.uint8)


# --------------------------------------------------------------------------
# Stream-VAE
# --------------------------------------------------------------------------
def vae_param_specs(vcfg):
    """(name, shape) of every Stream-VAE parameter: conv weights
    [Cout][3][3][3][Cin], biases [Cout], norm gains [Cout]."""
    enc = [("e0", 8, vcfg.c1, True), ("e1", vcfg.c1, vcfg.c2, True), ("e2", vcfg.c2, vcfg.c3, True),
           ("e3", vcfg.c3, vcfg.c3, True), ("e_out", vcfg.c3, vcfg.latent_c, False)]
    dec = [("d0", vcfg.latent_c, vcfg.c3, True), ("d1", vcfg.c3, vcfg.c3, True), ("d2", vcfg.c3, vcfg.c2, True),
           ("d3", vcfg.c2, vcfg.c1, True), ("d_out", vcfg.c1, 3, False)]
    out = []
    for name, cin, cout, norm in enc + dec:
        out.append((name + ".w", (cout, 3, 3, 3, cin)))
        out.append((name + ".b", (cout,)))
        if norm:
            out.append((name + ".g", (cout,)))
    return out


def make_vae_weights(vcfg, seed: int = SEED_VAE_WEIGHTS):
    """bf16-representable float32 weights: conv weights N(0, 1/fan_in) (unit
    gain through a layer), biases N(0, 0.02^2), norm gains 1 + N(0, 0.1^2).
    The encoder's first layer sees zeros on input channels 3..7; its weights
    there are zero too."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name, shape in vae_param_specs(vcfg):
        if name.endswith(".w"):
            fan_in = int(np.prod(shape[1:]))
            w = rng.standard_normal(size=shape, dtype=np.float32) / np.float32(np.sqrt(fan_in))
            if name == "e0.w":
                w[..., 3:] = 0
        elif name.endswith(".b"):
            w = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(0.02)
        else:
            w = 1.0 + rng.standard_normal(size=shape, dtype=np.float32) * np.float32(0.1)
        out[name] = round_bf16(w.astype(np.float32))
    return out


class PixelSource:
    """Pixel chunks [2 latent_t][3][H][W] in [-1, 1]: a smooth moving pattern
    plus noise (bf16-representable), so consecutive chunks are correlated as
    video frames are."""

    def __init__(self, vcfg, seed: int = SEED_VAE_PIXELS):
        self.v = vcfg
        self.rng = np.random.Generator(np.random.PCG64(seed))
        self.t = 0

    def next(self):
        v = self.v
        T, H, W = v.frames, v.height, v.width
        yy, xx = np.meshgrid(np.linspace(0, 1, H), np.linspace(0, 1, W), indexing="ij")
        out = np.empty((T, 3, H, W), np.float32)
        for f in range(T):
            ph = 0.15 * (self.t + f)
            for c in range(3):
                out[f, c] = 0.6 * np.sin(6.0 * xx + 4.0 * yy + ph + 2.1 * c)
        self.t += T
        out += 0.2 * self.rng.standard_normal(size=out.shape, dtype=np.float32)
        return round_bf16(np.clip(out, -1.0, 1.0))


class VAELatentSource:
    """Latent chunks [latent_t][16][h][w], N(0, 1), bf16-representable."""

    def __init__(self, vcfg, seed: int = SEED_LATENT):
        self.v = vcfg
        self.rng = np.random.Generator(np.random.PCG64(seed))

    def next(self):
        v = self.v
        return round_bf16(self.rng.standard_normal(size=(v.latent_t, v.latent_c, v.latent_h, v.latent_w),
                                                   dtype=np.float32))
