"""SLO-aware batching (host logic, no GPU).  The expected choices come from
brute force over the true latency function of each synthetic regime: the
smallest batch whose rate b*T/L(b) meets the target, else the smallest batch
within the knee tolerance of the best reachable rate."""
import numpy as np
import pytest

from streaming_diffusion_amd.slo import SLOBatchScheduler


def brute_force(lat, T, target, cap, tol=0.05):
    rates = {b: b * T / lat(b) for b in range(1, cap + 1)}
    for b in range(1, cap + 1):
        if rates[b] >= target:
            return b
    best = max(rates.values())
    return min(b for b in rates if rates[b] >= (1 - tol) * best)


def run(lat, T, target, b_max, pending=lambda step: 64, steps=40, noise=0.0, seed=0):
    rng = np.random.default_rng(seed)
    sch = SLOBatchScheduler(T, target, b_max)
    trace = []
    for k in range(steps):
        b = sch.choose(pending(k))
        trace.append(b)
        sch.observe(b, lat(b) * (1.0 + noise * rng.standard_normal()))
    return trace


@pytest.mark.parametrize("target", [150.0, 400.0, 600.0])
def test_memory_bound_regime_converges_to_smallest_batch_meeting_the_target(target):
    # weight traffic fixed, activation traffic per chunk: L(b) = 10 ms + 2 ms * b
    lat = lambda b: 0.010 + 0.002 * b
    trace = run(lat, 2, target, 8)
    want = brute_force(lat, 2, target, 8)
    assert trace[-10:] == [want] * 10
    assert want == {150.0: 1, 400.0: 4, 600.0: 8}[target]


def test_compute_bound_regime_stays_at_the_knee():
    # every chunk costs the same: the rate does not depend on b, so batching
    # only adds latency, even with an unreachable target
    lat = lambda b: 0.040 * b
    trace = run(lat, 2, 80.0, 8)
    assert trace[-10:] == [1] * 10
    assert brute_force(lat, 2, 80.0, 8) == 1


def test_unreachable_target_stops_at_the_knee_of_a_saturating_curve():
    lat = lambda b: 0.030 + 0.010 * b           # rate -> 200 frames/s
    trace = run(lat, 2, 500.0, 8)
    want = brute_force(lat, 2, 500.0, 8)
    assert trace[-5:] == [want] * 5 and 1 < want < 8


def test_never_more_chunks_than_collected():
    lat = lambda b: 0.010 + 0.002 * b
    trace = run(lat, 2, 600.0, 8, pending=lambda k: 1 + k % 3)
    assert all(b <= 1 + k % 3 for k, b in enumerate(trace))


def test_noisy_latencies_still_settle():
    lat = lambda b: 0.010 + 0.002 * b
    trace = run(lat, 2, 400.0, 8, noise=0.03, steps=80)
    want = brute_force(lat, 2, 400.0, 8)
    assert sum(abs(b - want) <= 1 for b in trace[-20:]) == 20


def test_first_steps_measure_then_probe():
    sch = SLOBatchScheduler(2, 100.0, 8)
    assert sch.choose(8) == 1
    sch.observe(1, 0.04)
    assert sch.choose(8) == 2          # a second batch size to fix the slope
    sch.observe(2, 0.06)
    alpha, beta = sch.model()
    assert alpha == pytest.approx(0.02) and beta == pytest.approx(0.02)


def test_invalid_arguments():
    with pytest.raises(ValueError):
        SLOBatchScheduler(0, 30.0, 4)
    with pytest.raises(ValueError):
        SLOBatchScheduler(2, 0.0, 4)


# ------------------------------------------------------------------ denoising steps and batch together
from streaming_diffusion_amd.slo import fit_rows_model, plan_steps_and_batch


def brute_plan(lat, T, target, cap, ns, tol=0.05):
    ok = [(n, b) for n in ns for b in range(1, cap + 1) if b * T / lat(b, n) >= target]
    if ok:
        n = max(n for n, _ in ok)
        return n, min(b for m, b in ok if m == n)
    n = min(ns)
    rates = {b: b * T / lat(b, n) for b in range(1, cap + 1)}
    best = max(rates.values())
    return n, min(b for b in rates if rates[b] >= (1 - tol) * best)


REGIMES = {
    # below the knee: a fixed weight-streaming cost per step plus a cost per row
    "memory": lambda b, n: 0.012 + 0.0015 * b * n,
    # above the knee: every row costs the same (the video DiTs on one MI355X)
    "compute": lambda b, n: 0.020 * b * n,
    # in between
    "mixed": lambda b, n: 0.005 + 0.006 * b * n,
}


@pytest.mark.parametrize("regime", list(REGIMES))
@pytest.mark.parametrize("target", [10.0, 30.0, 60.0, 120.0, 400.0])
def test_plan_matches_brute_force(regime, target):
    lat = REGIMES[regime]
    got = plan_steps_and_batch(lat, 2, target, 8, (1, 2, 4))
    assert got == brute_plan(lat, 2, target, 8, (1, 2, 4))


def test_plan_prefers_more_steps_when_the_target_allows():
    lat = REGIMES["memory"]
    # 4 steps reach 30 frames/s with one chunk: 2 / (0.012 + 0.006) = 111 frames/s
    assert plan_steps_and_batch(lat, 2, 30.0, 8, (1, 2, 4)) == (4, 1)
    # compute-bound: frames/s = 2 / (0.02 n) does not depend on B; 60 frames/s needs n = 1
    assert plan_steps_and_batch(REGIMES["compute"], 2, 60.0, 8, (1, 2, 4)) == (1, 1)
    # unreachable: fewest steps, and B = 1 since batching never pays
    assert plan_steps_and_batch(REGIMES["compute"], 2, 500.0, 8, (1, 2, 4)) == (1, 1)


def test_rows_model_recovers_the_line_from_a_sweep():
    lat = REGIMES["mixed"]
    samples = [(b * n, lat(b, n)) for b in (1, 2, 4) for n in (1, 2, 4)]
    alpha, beta = fit_rows_model(samples)
    assert alpha == pytest.approx(0.005) and beta == pytest.approx(0.006)
    with pytest.raises(ValueError):
        fit_rows_model([(2, 0.1), (2, 0.11)])
