"""Seeded synthetic workloads for the Stream Batch hot path.

This package holds configuration data (shapes and constants of the five
workload configurations) and seeded generators for every input the path
consumes: denoiser weights, latent sequences, entry noise, SSF frames,
uniforms and contexts.  It holds none of the method's arithmetic, so both the
CPU oracle and the GPU path may draw their inputs from it.
"""
from .configs import CONFIGS, VAE_CONFIGS, Config, VAEConfig, get_config, get_vae_config  # noqa: F401
from . import gen  # noqa: F401
