"""Noise schedule and per-slot timesteps.

Pinned by tests/test_oracle_schedule.py (endpoint values, linearity of
sqrt(beta), the cumulative-product recurrence, the t_index table).

Notation (StreamDiffusion paper notes, section 2 R-CFG): the pages write
x_tau = sqrt(alpha_tau) x0 + sqrt(beta_tau) eps.  Read here as
alpha_tau = prod_{s<=tau}(1 - beta_s) (often written alpha-bar) and
beta_tau = 1 - alpha_tau: the only reading under which the virtual residual
noise equation returns the noise that produced x_tau from x0.
"""
from __future__ import annotations

import math

import numpy as np


def betas(n_train: int = 1000, beta_start: float = 0.00085, beta_end: float = 0.012) -> np.ndarray:
    """Scaled-linear betas: sqrt(beta) is linear in t from sqrt(beta_start)
    to sqrt(beta_end) over t = 0..n_train-1."""
    t = np.arange(n_train, dtype=np.float64)
    s0, s1 = math.sqrt(beta_start), math.sqrt(beta_end)
    return (s0 + (s1 - s0) * t / (n_train - 1)) ** 2


def alphas_cumprod(n_train: int = 1000, beta_start: float = 0.00085, beta_end: float = 0.012) -> np.ndarray:
    """alpha_t = prod_{s<=t} (1 - beta_s)."""
    return np.cumprod(1.0 - betas(n_train, beta_start, beta_end))


def sched_coeffs(cfg):
    """Per-timestep (a_t, b_t) = (sqrt(alpha_t), sqrt(1 - alpha_t)) as fp64 arrays."""
    ab = alphas_cumprod(cfg.n_train_steps, cfg.beta_start, cfg.beta_end)
    return np.sqrt(ab), np.sqrt(1.0 - ab)


def taus_from_t_index(cfg, t_index=None):
    """Timestep per slot from t_index_list.

    The project intro's usage example passes t_index_list=[32, 45] without
    saying what the indices address.  Reading: positions on a 50-step grid of
    the n_train-step schedule, tau = (n_train - 1) - (n_train // 50) * k, so
    [32, 45] -> [359, 99] and [0, 16, 32, 45] -> [999, 679, 359, 99]."""
    t_index = cfg.t_index if t_index is None else t_index
    stride = cfg.n_train_steps // 50
    taus = [(cfg.n_train_steps - 1) - stride * int(k) for k in t_index]
    for t in taus:
        if not 0 <= t < cfg.n_train_steps:
            raise ValueError(f"t_index entry maps outside the schedule: {t}")
    return taus


def taus_from_noise_rate(s: float, n: int, n_train: int = 1000):
    """Timestep per slot from the motion-controlled noise rate s.

    Reading of the motion-aware noise scheduler (StreamDiffusionV2 summary):
    the noise rate s in [s_min, s_max] sets the first slot's timestep, the
    other slots are spaced evenly below it:
    tau_i = round_half_even(s * (n_train - 1) * (n - i) / n), i = 0..n-1,
    evaluated left to right in IEEE fp64."""
    out = []
    for i in range(n):
        v = s * float(n_train - 1) * float(n - i) / float(n)
        out.append(int(round(v)))        # Python round(): ties to even
    return out
