"""Per-frame control reductions: SSF, motion-aware noise rate, sink refresh.

Stochastic Similarity Filter (StreamDiffusion paper notes, section 3):
P(skip | I_t, I_ref) = max{0, (S_C(I_t, I_ref) - eta) / (1 - eta)} with S_C the
cosine similarity; the skip is drawn, not thresholded.  The project intro adds
a cap, max_skip_frame, on consecutive skipped frames.
Readings: frames are integers (uint8 images, or float latents quantised to
q = clamp(round_half_even(x * 2^12), +-2^20)); the three sums are exact
integers; the tail is IEEE fp64 (D / sqrt(N1 * N2)); skip iff u < p (strict)
for a host uniform u in [0, 1); both norms zero gives similarity 1, exactly one
zero gives 0.

Motion-aware noise scheduler (StreamDiffusionV2 summary): motion = L2 between
consecutive latent frames, normalised over a k-frame window by a scale sigma,
clipped to [0, 1]; the noise rate follows an EMA with rate lambda inside
[s_min, s_max]; high motion means more conservative denoising (less noise).
Readings: d = RMS of the difference of the 2^-12-quantised frames (exact
integer sum of squares, fp64 tail); d_bar = mean of the last <= k values;
target = s_max - (s_max - s_min) * clip(d_bar / sigma, 0, 1);
s <- lambda * target + (1 - lambda) * s, s starts at s_max.

Adaptive sink refresh (StreamDiffusionV2 summary): the new chunk embedding is
compared by cosine similarity with the sink set, and the least similar sink is
refreshed when its similarity falls below a threshold tau.
Readings: embedding = mean over the chunk's tokens of the last block's output;
j* = argmin (lowest index on ties); refresh iff sim_j* < tau (strict); a zero
vector has cosine 0.

Pins (tests/test_oracle_controls.py): identical frames give p = 1, disjoint
supports give p = 0, sim = eta gives p = 0, exact Python-integer brute force,
a hand-derived golden example; static input keeps s = s_max, a constant d_hat
gives the closed-form geometric approach, saturation; cos(h, h) = 1 never
refreshes, an orthogonal embedding refreshes, ties pick the lowest index.
"""
from __future__ import annotations

import math

import numpy as np

Q_SCALE = 4096.0          # 2^12
Q_CLAMP = 1 << 20


def quantise_latent(x):
    """Float latent -> int64 codes q = clamp(rint(x * 2^12), -2^20, 2^20).
    x * 2^12 is exact in fp64 for float32 x; rint rounds ties to even."""
    q = np.rint(np.asarray(x, dtype=np.float64) * Q_SCALE)
    return np.clip(q, -Q_CLAMP, Q_CLAMP).astype(np.int64)


def ssf_sums(a, b):
    """Exact (D, N1, N2) = (sum a*b, sum a*a, sum b*b) as Python ints."""
    a = np.asarray(a).astype(np.int64).ravel()
    b = np.asarray(b).astype(np.int64).ravel()
    return int(np.dot(a, b)), int(np.dot(a, a)), int(np.dot(b, b))


def cosine_from_sums(D: int, N1: int, N2: int) -> float:
    if N1 == 0 and N2 == 0:
        return 1.0
    if N1 == 0 or N2 == 0:
        return 0.0
    return float(D) / math.sqrt(float(N1) * float(N2))


def skip_probability(sim: float, eta: float) -> float:
    return max(0.0, (sim - eta) / (1.0 - eta))


def motion_sumsq(prev_q, cur_q) -> int:
    diff = np.asarray(cur_q, dtype=np.int64).ravel() - np.asarray(prev_q, dtype=np.int64).ravel()
    return int(np.dot(diff, diff))


def motion_distance(sumsq: int, n_elems: int) -> float:
    """RMS of the quantised difference, back in latent units."""
    return math.sqrt(float(sumsq) / float(n_elems)) / Q_SCALE


def motion_update(s: float, window, cfg):
    """One EMA step of the noise rate from the motion window (chronological
    list of distances, at most k long).  Returns the new s."""
    if len(window) == 0:
        return s
    tot = 0.0
    for v in window:
        tot += v
    d_bar = tot / float(len(window))
    d_hat = min(max(d_bar / cfg.motion_sigma, 0.0), 1.0)
    target = cfg.s_max - (cfg.s_max - cfg.s_min) * d_hat
    return cfg.motion_lambda * target + (1.0 - cfg.motion_lambda) * s


def cosine(h, e) -> float:
    h = np.asarray(h, dtype=np.float64)
    e = np.asarray(e, dtype=np.float64)
    nh, ne = float(np.sqrt(np.dot(h, h))), float(np.sqrt(np.dot(e, e)))
    if nh == 0.0 or ne == 0.0:
        return 0.0
    return float(np.dot(h, e)) / (nh * ne)


def sink_refresh_choice(h, embeddings, tau: float):
    """Return (j_star, sim_j_star, refresh?) for chunk embedding h against the
    sink embeddings (list of vectors)."""
    sims = [cosine(h, e) for e in embeddings]
    j = 0
    for i in range(1, len(sims)):
        if sims[i] < sims[j]:
            j = i
    return j, sims[j], sims[j] < tau
