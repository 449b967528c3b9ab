"""The five workload configurations, as plain data.

Shapes follow the workloads the pages measure on: 512x512-class image streams
(the SD-turbo / KohakuV2 rows of the StreamDiffusion project-intro performance
table, t_index [32, 45] from its usage example) and 480p video on 1.3B- and
14B-shaped DiTs at 1-4 denoise steps (StreamDiffusionV2 notes, experiment
section).  Where the pages leave a value open the choice is marked
``# reading`` and listed with its reason in the design notes.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Config:
    name: str
    dtype: str                      # "f32" or "bf16": storage/compute type of the denoiser
    # latent geometry of one chunk: [T][C][H][W]
    latent_c: int
    latent_t: int
    latent_h: int
    latent_w: int
    patch: int                      # spatial patch (temporal patch is 1)
    # denoiser
    n_blocks: int
    d_model: int
    n_heads: int
    d_ffn: int
    d_freq: int                     # sinusoidal timestep-embedding width
    ctx_len: int                    # 0 = no cross-attention
    # stream batch
    t_index: Tuple[int, ...]        # one entry per slot; n = len(t_index)
    cfg_type: str                   # "self" | "onetime" | "full"
    gamma: float = 1.4
    delta: float = 1.0
    chunks_per_step: int = 1        # B
    batch_attn: bool = False        # cross-frame batch attention (rows attend to every row's tokens)
    sampler: str = "ddim"           # "ddim" (re-noise with eps_cfg) | "lcm" (re-noise with fresh noise)
    kv_recompute: bool = False      # leaving chunks' cache entries from a clean-latent forward at tau = 0
    # KV cache (tokens)
    sink_tokens: int = 0
    window_tokens: int = 0
    sink_entries: int = 1           # M entries of sink_tokens / M tokens each
    sink_tau: float = 0.9           # reading: "tau should be large"
    rope_reset: int = 1024
    rope_base: float = 10000.0
    # schedule (scaled-linear)
    n_train_steps: int = 1000
    beta_start: float = 0.00085
    beta_end: float = 0.012
    # stochastic similarity filter
    ssf_on: bool = False
    ssf_kind: str = "u8"            # "u8" frames [h][w][c] or "latent" (quantised x0)
    ssf_shape: Tuple[int, ...] = ()
    ssf_eta: float = 0.98
    max_skip_frame: int = 10        # reading: pages give the name only
    # motion-aware noise
    motion_on: bool = False
    motion_k: int = 8
    motion_lambda: float = 0.3
    s_min: float = 0.3
    s_max: float = 0.9
    motion_sigma: float = 1.0
    # run length used by tests / bench
    frames: int = 16

    # ---- derived ----
    @property
    def n_slots(self) -> int:
        return len(self.t_index)

    @property
    def head_dim(self) -> int:
        return self.d_model // self.n_heads

    @property
    def tokens(self) -> int:
        return self.latent_t * (self.latent_h // self.patch) * (self.latent_w // self.patch)

    @property
    def latent_elems(self) -> int:
        return self.latent_t * self.latent_c * self.latent_h * self.latent_w

    @property
    def patch_dim(self) -> int:
        return self.patch * self.patch * self.latent_c

    @property
    def rows_per_step(self) -> int:
        pos = self.chunks_per_step * self.n_slots
        clean = self.chunks_per_step if self.kv_recompute else 0
        if self.cfg_type == "full":
            return 2 * pos + clean
        return pos + (self.chunks_per_step if self.cfg_type == "onetime" else 0) + clean

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    # Tiny stream batch, fp32: everything the oracle runs in seconds.
    "tiny": Config(
        name="tiny", dtype="f32",
        latent_c=4, latent_t=1, latent_h=16, latent_w=16, patch=2,
        n_blocks=2, d_model=128, n_heads=4, d_ffn=512, d_freq=128, ctx_len=0,
        t_index=(32, 45), cfg_type="self", gamma=1.4, delta=1.0,
        sink_tokens=4, window_tokens=64,
        ssf_on=True, ssf_kind="u8", ssf_shape=(64, 64, 3), ssf_eta=0.98,
        frames=16,
    ),
    # Image stream, bf16, 512x512-shaped latent (4x64x64), 12-block DiT.
    "image": Config(
        name="image", dtype="bf16",
        latent_c=4, latent_t=1, latent_h=64, latent_w=64, patch=2,
        n_blocks=12, d_model=768, n_heads=12, d_ffn=3072, d_freq=256, ctx_len=77,
        t_index=(32, 45), cfg_type="self",
        sink_tokens=4, window_tokens=1024,            # reading: tiny config's ratio
        frames=256,
    ),
    # Four-step stream batch with onetime-negative R-CFG and SSF on latents.
    "fourstep": Config(
        name="fourstep", dtype="bf16",
        latent_c=4, latent_t=1, latent_h=64, latent_w=64, patch=2,
        n_blocks=24, d_model=1024, n_heads=16, d_ffn=4096, d_freq=256, ctx_len=77,
        t_index=(0, 16, 32, 45), cfg_type="onetime",
        sink_tokens=4, window_tokens=1024,
        ssf_on=True, ssf_kind="latent", ssf_shape=(4, 64, 64), ssf_eta=0.95,
        frames=512,
    ),
    # Video-DiT chunk, 1.3B-shaped: 16ch latent 60x104 (480x832 / 8), T=2.
    "video13b": Config(
        name="video13b", dtype="bf16",
        latent_c=16, latent_t=2, latent_h=60, latent_w=104, patch=2,
        n_blocks=30, d_model=1536, n_heads=12, d_ffn=8960, d_freq=256, ctx_len=77,
        t_index=(32, 45), cfg_type="self",            # headline n=2
        sink_tokens=1560, window_tokens=9360,         # 1 sink frame, 3 chunks
        motion_on=True, motion_k=8, motion_lambda=0.3, s_min=0.3, s_max=0.9,
        motion_sigma=0.05,
        frames=300,
    ),
    # Diagnostic below the roofline knee (not one of the pages' workloads):
    # the 1.3B-shaped video DiT's weights with one small latent frame of
    # 16 x 32 latents (8 x 16 = 128 tokens) per chunk, so one forward holds
    # 128 tokens per slot -- far below the ~312 tokens per forward at which
    # streaming the weights from HBM stops being the bound.  Cache: one sink
    # frame and a window of three chunks, as in the video workload.
    "video13b_subknee": Config(
        name="video13b_subknee", dtype="bf16",
        latent_c=16, latent_t=1, latent_h=16, latent_w=32, patch=2,
        n_blocks=30, d_model=1536, n_heads=12, d_ffn=8960, d_freq=256, ctx_len=77,
        t_index=(32,), cfg_type="self",
        sink_tokens=128, window_tokens=384,
        motion_on=True, motion_k=8, motion_lambda=0.3, s_min=0.3, s_max=0.9,
        motion_sigma=0.05,
        frames=300,
    ),
    # Video-DiT chunk, 14B-shaped.
    "video14b": Config(
        name="video14b", dtype="bf16",
        latent_c=16, latent_t=2, latent_h=60, latent_w=104, patch=2,
        n_blocks=40, d_model=5120, n_heads=40, d_ffn=13824, d_freq=256, ctx_len=77,
        t_index=(32,), cfg_type="self",
        sink_tokens=1560, window_tokens=9360,
        motion_on=True, motion_k=8, motion_lambda=0.3, s_min=0.3, s_max=0.9,
        motion_sigma=0.05,
        frames=300,
    ),
}


def get_config(name: str, **overrides) -> Config:
    cfg = CONFIGS[name]
    return cfg.replace(**overrides) if overrides else cfg


# ---------------------------------------------------------------------------
# Stream-VAE shapes.  A chunk is latent_t latent frames (2 x latent_t pixel
# frames) of latent_h x latent_w latents (8x larger in pixels); c1..c3 are the
# channel widths from the pixel side inward.
@dataclass(frozen=True)
class VAEConfig:
    name: str
    latent_t: int = 2
    latent_c: int = 16
    latent_h: int = 60
    latent_w: int = 104
    c1: int = 64
    c2: int = 128
    c3: int = 256
    chunks: int = 3                 # chunks a test or bench streams

    @property
    def frames(self) -> int:
        return 2 * self.latent_t

    @property
    def height(self) -> int:
        return 8 * self.latent_h

    @property
    def width(self) -> int:
        return 8 * self.latent_w

    def replace(self, **kw) -> "VAEConfig":
        return dataclasses.replace(self, **kw)


VAE_CONFIGS = {
    # the 1.3B-shaped video workload's latent chunk: 4 frames of 480 x 832
    "video13b": VAEConfig(name="video13b"),
    # small enough for the oracle in seconds; every layer kind, ragged tiles
    "small": VAEConfig(name="small", latent_h=3, latent_w=5, c1=16, c2=32, c3=64),
}


def get_vae_config(name: str, **overrides) -> VAEConfig:
    return VAE_CONFIGS[name].replace(**overrides)
