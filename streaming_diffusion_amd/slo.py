"""SLO-aware batching: how many chunks enter each Stream Batch step.

StreamDiffusionV2 summary, SLO-aware batching scheduler: a step that takes b
chunks of T frames emits b*T frames after a latency L(b), so the achieved rate
is f(b) = b*T / L(b).  In the memory-bound regime the pages describe, the
latency is an affine function of the batch (activation traffic grows with b,
the weight traffic does not), so f rises with b towards the roofline knee and
flattens beyond it.  The scheduler adapts b from the latencies it observes:
the smallest b whose predicted rate meets the target frame rate (least
latency per frame), never more chunks than have been collected from the input
stream, and -- when the target is out of reach -- no further along the curve
than the knee, where a larger batch stops paying for its latency.

Host logic only: it drives `StreamRunner.step(chunks=b)` (the library's
sd_stream_step_chunks) and is exercised without a GPU by the tests.
"""
from __future__ import annotations

from typing import Dict, Optional, Tuple


class SLOBatchScheduler:
    def __init__(self, frames_per_chunk: int, target_fps: float, b_max: int, knee_tol: float = 0.05,
                 decay: float = 0.7):
        if frames_per_chunk < 1 or b_max < 1 or target_fps <= 0:
            raise ValueError("frames_per_chunk, b_max and target_fps must be positive")
        self.T = frames_per_chunk
        self.target = float(target_fps)
        self.b_max = b_max
        self.knee_tol = knee_tol
        self.decay = decay
        self.lat: Dict[int, float] = {}       # b -> smoothed step latency in seconds

    def observe(self, b: int, seconds: float) -> None:
        """Record the measured latency of a step that took b chunks."""
        prev = self.lat.get(b)
        self.lat[b] = seconds if prev is None else self.decay * prev + (1.0 - self.decay) * seconds

    def model(self) -> Optional[Tuple[float, float]]:
        """(alpha, beta) of L(b) = alpha + beta*b, least squares over the
        smoothed latencies; with a single batch size observed the latency is
        taken as proportional to b (no fixed part)."""
        pts = sorted(self.lat.items())
        if not pts:
            return None
        if len(pts) == 1:
            b, l = pts[0]
            return 0.0, l / b
        n = len(pts)
        mb = sum(b for b, _ in pts) / n
        ml = sum(l for _, l in pts) / n
        sbb = sum((b - mb) ** 2 for b, _ in pts)
        beta = sum((b - mb) * (l - ml) for b, l in pts) / sbb
        beta = max(beta, 1e-12)
        alpha = max(ml - beta * mb, 0.0)
        return alpha, beta

    def rate(self, b: int, model: Optional[Tuple[float, float]] = None) -> float:
        """Predicted frames per second of steps taking b chunks."""
        alpha, beta = model if model is not None else self.model()
        return b * self.T / (alpha + beta * b)

    def choose(self, pending: int) -> int:
        """Chunks for the next step, given `pending` collected chunks (>= 1)."""
        cap = max(1, min(self.b_max, pending))
        model = self.model()
        if model is None:
            return 1
        if len(self.lat) == 1 and cap >= 2 and 2 not in self.lat:
            return 2                          # a second batch size fixes the slope
        for b in range(1, cap + 1):
            if self.rate(b, model) >= self.target:
                return b
        best = max(self.rate(b, model) for b in range(1, cap + 1))
        for b in range(1, cap + 1):
            if self.rate(b, model) >= (1.0 - self.knee_tol) * best:
                return b
        return cap


def fit_rows_model(samples) -> Tuple[float, float]:
    """(alpha, beta) of L = alpha + beta * rows by least squares over measured
    (rows, seconds) pairs, rows = B * n per forward.  Every row of a Stream
    Batch forward costs the same (each is one chunk at one denoising slot), so
    a sweep over B and n collapses onto one line in rows; the intercept is the
    per-step cost that does not grow with the batch (in the pages' model, the
    weight traffic)."""
    pts = [(float(r), float(t)) for r, t in samples]
    if len(pts) < 2 or len({r for r, _ in pts}) < 2:
        raise ValueError("need latencies at two different row counts")
    n = len(pts)
    mr = sum(r for r, _ in pts) / n
    mt = sum(t for _, t in pts) / n
    beta = sum((r - mr) * (t - mt) for r, t in pts) / sum((r - mr) ** 2 for r, _ in pts)
    beta = max(beta, 1e-12)
    return max(mt - beta * mr, 0.0), beta


def plan_steps_and_batch(latency, frames_per_chunk: int, target_fps: float, b_max: int, n_options,
                         knee_tol: float = 0.05) -> Tuple[int, int]:
    """Denoising steps n and chunks per step B for a frame-rate target.

    StreamDiffusionV2 summary, SLO-aware batching: the scheduler sizes the
    stream batch from the target rate, and the denoising steps multiply the
    rows of every forward (B chunks at n slots each), so n trades image
    quality against rate.  Quality first: the largest n in n_options for
    which some B <= b_max reaches f(B, n) = B * T / L(B, n) >= target, with
    the smallest such B (least latency per frame).  When no pair reaches the
    target: the fewest steps, and on that curve the smallest B within
    knee_tol of its best rate.  `latency(B, n)` returns seconds per step."""
    if frames_per_chunk < 1 or b_max < 1 or target_fps <= 0 or not n_options:
        raise ValueError("frames_per_chunk, b_max, target_fps and n_options must be positive / non-empty")
    T = frames_per_chunk

    def rate(b, n):
        return b * T / latency(b, n)

    for n in sorted(n_options, reverse=True):
        for b in range(1, b_max + 1):
            if rate(b, n) >= target_fps:
                return n, b
    n = min(n_options)
    best = max(rate(b, n) for b in range(1, b_max + 1))
    for b in range(1, b_max + 1):
        if rate(b, n) >= (1.0 - knee_tol) * best:
            return n, b
    return n, b_max
