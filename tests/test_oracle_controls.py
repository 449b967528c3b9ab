"""Pins for oracle.controls: SSF, motion-aware noise rate, sink refresh."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import controls
from workloads import gen, get_config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_ssf_golden():
    rows = []
    with open(os.path.join(GOLDEN, "ssf_worked_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b, eta, cos, p = [t.strip() for t in line.split(";")]
            rows.append(([int(v) for v in a.split(",")], [int(v) for v in b.split(",")],
                         float(eta), float(cos), float(p)))
    return rows


@pytest.mark.parametrize("a,b,eta,cos,p", load_ssf_golden())
def test_ssf_worked_examples(a, b, eta, cos, p):
    D, N1, N2 = controls.ssf_sums(np.array(a, np.uint8), np.array(b, np.uint8))
    sim = controls.cosine_from_sums(D, N1, N2)
    assert abs(sim - cos) < 1e-15
    assert abs(controls.skip_probability(sim, eta) - p) < 1e-12


def test_ssf_sums_exact_against_python_ints():
    r = np.random.default_rng(7)
    a = r.integers(0, 256, size=(64, 64, 3)).astype(np.uint8)
    b = r.integers(0, 256, size=(64, 64, 3)).astype(np.uint8)
    D, N1, N2 = controls.ssf_sums(a, b)
    al, bl = [int(v) for v in a.ravel()], [int(v) for v in b.ravel()]
    assert D == sum(x * y for x, y in zip(al, bl))
    assert N1 == sum(x * x for x in al) and N2 == sum(y * y for y in bl)
    # the fp64 tail equals the exact rational value to within one rounding chain
    exact = Fraction(D) / Fraction(math.isqrt(N1 * N2 * 10 ** 40), 10 ** 20)
    assert abs(controls.cosine_from_sums(D, N1, N2) - float(exact)) < 1e-15


def test_ssf_p_on_the_tiny_workload_is_high():
    # near-static frames (uniform base + N(0, 3^2) noise) give cos close to 1:
    # the filter is built to drop such frames most of the time.
    cfg = get_config("tiny")
    src = gen.SSFFrameSource(cfg)
    f0, f1 = src.next(), src.next()
    sim = controls.cosine_from_sums(*controls.ssf_sums(f1, f0))
    p = controls.skip_probability(sim, cfg.ssf_eta)
    assert 0.9 < p < 1.0


def test_quantiser():
    x = np.array([0.0, 1.0, -1.0, 2 ** -13, 3 * 2 ** -13, 1e9, -1e9, 0.123], np.float32)
    q = controls.quantise_latent(x)
    assert q.tolist()[:7] == [0, 4096, -4096, 0, 2, 1 << 20, -(1 << 20)]   # 0.5 -> 0, 1.5 -> 2: ties to even
    assert q[7] == round(float(np.float32(0.123)) * 4096)


# ------------------------------------------------------------------ motion
def test_motion_distance_is_rms():
    a = np.zeros(100, np.int64)
    b = np.full(100, 4096 * 3, np.int64)            # difference of 3.0 everywhere
    assert controls.motion_distance(controls.motion_sumsq(a, b), 100) == 3.0


def test_static_input_keeps_s_max():
    cfg = get_config("video13b")
    s = cfg.s_max
    win = []
    for _ in range(20):
        win = (win + [0.0])[-cfg.motion_k:]
        s = controls.motion_update(s, win, cfg)
        assert s == cfg.s_max


def test_constant_motion_gives_geometric_approach():
    cfg = get_config("video13b")
    d = 0.4 * cfg.motion_sigma
    target = cfg.s_max - (cfg.s_max - cfg.s_min) * 0.4
    s, s0 = cfg.s_max, cfg.s_max
    for t in range(1, 30):
        s = controls.motion_update(s, [d] * 5, cfg)
        assert abs(s - (target + (1 - cfg.motion_lambda) ** t * (s0 - target))) < 1e-14


def test_motion_saturates():
    cfg = get_config("video13b")
    s = 0.5
    s_big = controls.motion_update(s, [10 * cfg.motion_sigma], cfg)
    s_edge = controls.motion_update(s, [cfg.motion_sigma], cfg)
    assert s_big == s_edge == cfg.motion_lambda * cfg.s_min + (1 - cfg.motion_lambda) * s
    # the window is a mean: [2 sigma, 0] -> d_hat = 1
    assert controls.motion_update(s, [2 * cfg.motion_sigma, 0.0], cfg) == s_edge
    # empty window leaves s alone
    assert controls.motion_update(s, [], cfg) == s


def test_high_motion_lowers_the_noise_rate():
    cfg = get_config("video13b")
    lo = controls.motion_update(cfg.s_max, [0.1 * cfg.motion_sigma], cfg)
    hi = controls.motion_update(cfg.s_max, [0.9 * cfg.motion_sigma], cfg)
    assert hi < lo < cfg.s_max


# ------------------------------------------------------------------ sink refresh
def test_sink_never_refreshes_on_itself():
    h = np.random.default_rng(0).standard_normal(32)
    j, sim, ref = controls.sink_refresh_choice(h, [h.copy()], 0.9)
    assert j == 0 and abs(sim - 1) < 1e-15 and not ref
    j, sim, ref = controls.sink_refresh_choice(h, [3.0 * h], 0.999999)
    assert not ref


def test_sink_refreshes_orthogonal_and_picks_least_similar():
    e0 = np.array([1.0, 0, 0]); e1 = np.array([0, 1.0, 0]); e2 = np.array([1.0, 1.0, 0])
    h = np.array([1.0, 0.0, 0.0])
    j, sim, ref = controls.sink_refresh_choice(h, [e0, e1, e2], 0.9)
    assert j == 1 and sim == 0.0 and ref
    # ties pick the lowest index
    j, _, _ = controls.sink_refresh_choice(np.array([0, 0, 1.0]), [e0, e1, e2], 0.9)
    assert j == 0
    # zero vector has cosine 0
    assert controls.cosine(np.zeros(3), e0) == 0.0
    # strict comparison
    h2 = np.array([0.9, math.sqrt(1 - 0.81), 0.0])
    _, sim2, ref2 = controls.sink_refresh_choice(h2, [e0], sim2_tau := controls.cosine(h2, e0))
    assert not ref2
