"""Pins for oracle.schedule (scaled-linear betas, cumulative alphas, timesteps)."""
import math

import numpy as np
import pytest

from oracle import schedule
from workloads import get_config


def test_beta_endpoints_are_the_configured_range():
    b = schedule.betas(1000, 0.00085, 0.012)
    assert b.shape == (1000,)
    assert abs(b[0] - 0.00085) < 1e-15
    assert abs(b[-1] - 0.012) < 1e-15


def test_sqrt_beta_is_linear_in_t():
    # "scaled-linear": sqrt(beta) -- not beta -- moves in equal steps
    s = np.sqrt(schedule.betas(1000, 0.00085, 0.012))
    d = np.diff(s)
    assert np.allclose(d, d[0], rtol=0, atol=1e-15)
    assert abs(d[0] - (math.sqrt(0.012) - math.sqrt(0.00085)) / 999) < 1e-16
    # beta itself is not linear
    assert not np.allclose(np.diff(schedule.betas()), np.diff(schedule.betas())[0])


def test_alpha_is_cumulative_product():
    b = schedule.betas()
    ab = schedule.alphas_cumprod()
    assert abs(ab[0] - (1 - 0.00085)) < 1e-15
    ratio = ab[1:] / ab[:-1]
    assert np.allclose(ratio, 1 - b[1:], rtol=1e-13, atol=0)
    assert np.all(np.diff(ab) < 0)


def test_alpha_known_values():
    # Widely used value of this schedule's last cumulative alpha (~0.00466),
    # plus the values at the grid timesteps the configurations use.
    ab = schedule.alphas_cumprod()
    assert abs(ab[999] - 0.0046601) < 5e-7
    assert abs(ab[679] - 0.0959839) < 5e-7
    assert abs(ab[359] - 0.4915004) < 5e-7
    assert abs(ab[99] - 0.8954628) < 5e-7


def test_t_index_table():
    cfg = get_config("tiny")
    assert schedule.taus_from_t_index(cfg, [32, 45]) == [359, 99]
    assert schedule.taus_from_t_index(cfg, [0, 16, 32, 45]) == [999, 679, 359, 99]
    assert schedule.taus_from_t_index(cfg, [49]) == [19]
    with pytest.raises(ValueError):
        schedule.taus_from_t_index(cfg, [50])


def test_noise_rate_timesteps():
    assert schedule.taus_from_noise_rate(0.9, 2) == [899, 450]     # 899.1, 449.55
    assert schedule.taus_from_noise_rate(0.5, 1) == [500]          # 499.5 ties to even
    assert schedule.taus_from_noise_rate(0.3, 4) == [300, 225, 150, 75]   # 299.7, 224.775, 149.85, 74.925
    t = schedule.taus_from_noise_rate(0.61, 3)
    assert t[0] > t[1] > t[2] >= 0
