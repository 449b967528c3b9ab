"""The Stream Batch pipeline and its integer state machine, step by step.

Stream Batch (StreamDiffusion paper notes, section 1): with n denoise steps,
n frames sitting at n different steps form one batch of size n and a single
denoiser forward advances all of them; a frame that enters at step t is
finished n steps later.  Here a frame pushed before step s occupies slot 0 at
step s, slot i at step s+i, and leaves from slot n-1 at step s+n-1.  Slots
that are still empty during warm-up are not computed.

KV cache (StreamDiffusionV2 summary: sink-token guided rolling KV cache).
Readings:
* every row of a step reads the cache as it stood when the step began;
* after the forward the exiting chunk appends, at every block, the K/V it
  computed in that forward (K after RoPE) to a ring of W tokens at positions
  (ptr + j) mod W; then ptr <- (ptr + L) mod W, v <- min(W, v + L);
* the sink holds M entries of S/M tokens, filled from the first exiting
  chunks' leading tokens; it is a separate copy, so those keys also stay in the
  window until they roll out; once full, the adaptive refresh may overwrite
  the least similar entry;
* RoPE refresh: a host counter p gives a chunk of T frames temporal positions
  p..p+T-1; if p+T-1 would exceed the threshold, p restarts at 0 first.
* kv_reset clears ring, sink and the RoPE counter; frames in flight continue;
* with kv_recompute the K/V a leaving chunk appends (and the hidden state its
  sink decision uses) come instead from one more forward of its emitted
  x0_hat at timestep 0, against the same snapshot.

Pins (tests/test_oracle_stream.py): the identity pipeline returns every input
frame; with the cache frozen the pipelined output equals the same frame
denoised sequentially (bit-identical); the integer traces (slots, ring pointer
and valid count, sink count, RoPE wrap, skip counter) against hand-enumerated
tables.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from . import controls, guidance, schedule
from .dit import Denoiser


class NotReady(Exception):
    pass


@dataclass
class Frame:
    fid: int
    x0: np.ndarray            # clean input latent [T][C][H][W]
    x: np.ndarray             # current noisy latent of its slot
    taus: List[int]
    t0: int                   # temporal RoPE base
    x0_star: Optional[np.ndarray] = None
    renoise: Optional[List[np.ndarray]] = None   # LCM sampler: noise of slots 1 .. n-1


@dataclass
class PushInfo:
    skipped: bool
    p: float
    sim: float
    d: float
    s: float
    taus: List[int]
    t0: int


@dataclass
class StepInfo:
    step: int
    has_output: bool
    frame_id: int
    rows: int
    kv_ptr: int
    kv_valid: int
    sink_count: int
    sink_refreshed: bool
    sink_entry: int
    sink_sim: float
    rope_next: int
    n_out: int = 0            # frames emitted by the step (B when a slot group leaves)


class OracleStream:
    def __init__(self, cfg, weights, ctx_pos=None, ctx_neg=None, dtype=np.float64,
                 identity_denoiser=False, freeze_cache=False, sink_entries: Optional[int] = None):
        self.cfg = cfg
        self.dtype = dtype
        self.net = Denoiser(cfg, weights, dtype) if weights is not None else None
        self.a, self.b = schedule.sched_coeffs(cfg)
        self.identity = identity_denoiser
        self.freeze = freeze_cache
        if sink_entries is None:
            sink_entries = getattr(cfg, "sink_entries", 1)
        self.M = sink_entries
        if cfg.sink_tokens % sink_entries:
            raise ValueError("sink tokens must split evenly into entries")
        self.Se = cfg.sink_tokens // sink_entries
        self.ctx_kv = self._ctx(ctx_pos)
        self.ctx_kv_neg = self._ctx(ctx_neg)
        if cfg.cfg_type not in ("self", "onetime", "full"):
            raise ValueError("cfg_type must be self, onetime or full")
        if cfg.cfg_type != "self" and self.ctx_kv_neg is None and self.net is not None and cfg.ctx_len:
            raise ValueError("onetime-negative R-CFG and full CFG need a negative context")
        if getattr(cfg, "batch_attn", False) and cfg.cfg_type != "self":
            raise ValueError("batch attention is defined for self-negative R-CFG (rows of one prompt)")
        n = cfg.n_slots
        self.slots: List[Optional[List[Frame]]] = [None] * n      # slot groups of B frames
        self.pending: List[Frame] = []
        # SSF state
        self.ssf_ref = None
        self.skip_run = 0
        # motion state
        self.s = cfg.s_max
        self.motion_window: List[float] = []
        self.prev_q = None
        # counters
        self.n_pushed = 0
        self.n_steps = 0
        self.rope_p = 0
        self._alloc_cache()

    def _ctx(self, ctx):
        if ctx is None or self.net is None or self.cfg.ctx_len == 0:
            return None
        return [self.net.cross_kv(ctx, b) for b in range(self.cfg.n_blocks)]

    def _alloc_cache(self):
        cfg = self.cfg
        H, hd, W = cfg.n_heads, cfg.head_dim, cfg.window_tokens
        nb = cfg.n_blocks
        self.ringK = np.zeros((nb, W, H, hd), self.dtype)
        self.ringV = np.zeros((nb, W, H, hd), self.dtype)
        self.sinkK = np.zeros((nb, cfg.sink_tokens, H, hd), self.dtype)
        self.sinkV = np.zeros((nb, cfg.sink_tokens, H, hd), self.dtype)
        self.sink_emb = [None] * self.M
        self.sink_count = 0
        self.kv_ptr = 0
        self.kv_valid = 0

    # ------------------------------------------------------------------ API
    def kv_reset(self):
        self._alloc_cache()
        self.rope_p = 0

    def push_frame(self, x0, noise, ssf_frame=None, u: float = 0.0) -> PushInfo:
        cfg = self.cfg
        x0 = np.asarray(x0, np.float32)
        p = 0.0
        sim = 1.0
        if cfg.ssf_on:
            cur = (np.asarray(ssf_frame).astype(np.int64) if cfg.ssf_kind == "u8"
                   else controls.quantise_latent(x0))
            if self.ssf_ref is not None:
                D, N1, N2 = controls.ssf_sums(cur, self.ssf_ref)
                sim = controls.cosine_from_sums(D, N1, N2)
                p = controls.skip_probability(sim, cfg.ssf_eta)
                if self.skip_run < cfg.max_skip_frame and u < p:
                    self.skip_run += 1
                    return PushInfo(True, p, sim, 0.0, self.s, [], -1)
            self.skip_run = 0
            self.ssf_ref = cur
        d_last = 0.0
        if cfg.motion_on:
            qx = controls.quantise_latent(x0)
            frames = [qx[t] for t in range(qx.shape[0])]
            prev = self.prev_q
            for f in frames:
                if prev is not None:
                    d_last = controls.motion_distance(controls.motion_sumsq(prev, f), f.size)
                    self.motion_window.append(d_last)
                    if len(self.motion_window) > cfg.motion_k:
                        self.motion_window.pop(0)
                prev = f
            self.prev_q = frames[-1]
            self.s = controls.motion_update(self.s, self.motion_window, cfg)
            taus = schedule.taus_from_noise_rate(self.s, cfg.n_slots, cfg.n_train_steps)
        else:
            taus = schedule.taus_from_t_index(cfg)
        T = cfg.latent_t
        if self.rope_p + T - 1 > cfg.rope_reset:
            self.rope_p = 0
        t0 = self.rope_p
        self.rope_p += T
        a0, b0 = self.a[taus[0]], self.b[taus[0]]
        lcm = getattr(cfg, "sampler", "ddim") == "lcm"
        noise = np.asarray(noise, self.dtype)
        if lcm and noise.shape != (cfg.n_slots,) + x0.shape:
            raise ValueError("the LCM sampler takes n noise latents per frame (entry, then one per later slot)")
        x = guidance.entry_noise(x0.astype(self.dtype), noise[0] if lcm else noise, a0, b0)
        fr = Frame(self.n_pushed, x0.astype(self.dtype), x, taus, t0)
        if lcm:
            fr.renoise = [noise[i] for i in range(1, cfg.n_slots)]
        if cfg.cfg_type != "onetime":
            fr.x0_star = fr.x0
        self.pending.append(fr)
        self.n_pushed += 1
        return PushInfo(False, p, sim, d_last, self.s, taus, t0)

    def cache_snapshot(self):
        """Per block (K, V) arrays of the sink entries in use plus the valid
        window tokens, in an arbitrary but fixed order."""
        cfg = self.cfg
        W, v = cfg.window_tokens, self.kv_valid
        ns = self.sink_count * self.Se
        idx = [(self.kv_ptr - v + j) % W for j in range(v)] if W else []
        out = []
        for b in range(cfg.n_blocks):
            k = np.concatenate([self.sinkK[b, :ns], self.ringK[b, idx]], axis=0)
            vv = np.concatenate([self.sinkV[b, :ns], self.ringV[b, idx]], axis=0)
            out.append((k, vv))
        return out

    def _denoise(self, fr, tau, snapshot, ctx_kv, collect):
        if self.identity:
            return None
        return self.net.forward_row(fr.x, tau, fr.t0, snapshot, ctx_kv, collect=collect)

    def step(self, chunks: Optional[int] = None):
        """One Stream Batch step.  The `chunks` oldest pending frames (default
        and at most B = chunks_per_step) enter together as one slot group; all
        rows read the cache snapshot of the step start; the group in the last
        slot leaves, in push order, each frame appending its K/V and taking its
        sink decision in turn.  Returns (out, info): out is None when nothing
        leaves, the emitted latent when B = 1, else the [group size][latent]
        stack in push order."""
        cfg = self.cfg
        n = cfg.n_slots
        B = cfg.chunks_per_step
        b = B if chunks is None else chunks
        if not 1 <= b <= B:
            raise ValueError("chunks must be in [1, chunks_per_step]")
        if len(self.pending) < b:
            raise NotReady("fewer pending frames than chunks for this step")
        enter = [self.pending.pop(0) for _ in range(b)]
        self.slots = [enter] + self.slots[:n - 1]
        snapshot = None if self.identity else self.cache_snapshot()
        # forward rows: slot by slot, the frames of a slot in push order
        rows = [(i, f) for i, grp in enumerate(self.slots) if grp is not None for f in grp]
        # onetime-negative: one extra row per entering frame, with the negative prompt
        neg_eps = []
        if cfg.cfg_type == "onetime":
            for f in enter:
                tau0 = f.taus[0]
                a0, b0 = self.a[tau0], self.b[tau0]
                if self.identity:
                    eps_neg = (f.x - a0 * f.x0) / b0
                else:
                    eps_neg = self.net.forward_row(f.x, tau0, f.t0, snapshot, self.ctx_kv_neg)
                f.x0_star = guidance.predict_x0(f.x, eps_neg, a0, b0)
                neg_eps.append(eps_neg)
        if getattr(cfg, "batch_attn", False) and not self.identity:
            # cross-frame batch attention: one joint forward over the rows
            results = self.net.forward_batch([(f.x, f.taus[i], f.t0) for i, f in rows], snapshot, self.ctx_kv,
                                             collect={j for j, (i, _) in enumerate(rows) if i == n - 1})
        else:
            results = [self._denoise(f, f.taus[i], snapshot, self.ctx_kv, collect=(i == n - 1)) for i, f in rows]
        # full CFG (StreamDiffusion paper notes, section 2: standard CFG costs
        # 2n forwards): every row has a twin under the negative prompt, same
        # latent, timestep and cache; its prediction replaces eps'
        uncond = []
        if cfg.cfg_type == "full":
            for i, f in rows:
                tau = f.taus[i]
                if self.identity:
                    uncond.append(guidance.virtual_residual(f.x, f.x0, self.a[tau], self.b[tau]))
                else:
                    uncond.append(self.net.forward_row(f.x, tau, f.t0, snapshot, self.ctx_kv_neg))
        if not self.identity:
            # denoiser outputs in forward row order (slots, then the negative rows)
            self.last_eps = [res[0] if i == n - 1 else res for (i, _), res in zip(rows, results)]
            self.last_eps.extend(neg_eps)
            self.last_eps.extend(uncond)
        outs, exits = [], []
        for j, ((i, f), res) in enumerate(zip(rows, results)):
            tau = f.taus[i]
            a, b = self.a[tau], self.b[tau]
            eps_p = uncond[j] if uncond else guidance.virtual_residual(f.x, f.x0_star, a, b)
            exit_kv = exit_hidden = None
            if self.identity:
                eps_c = eps_p
            elif i == n - 1:
                eps_c, exit_kv, exit_hidden = res
            else:
                eps_c = res
            eps_cfg = guidance.rcfg(eps_c, eps_p, cfg.gamma, cfg.delta)
            x0_hat = guidance.predict_x0(f.x, eps_cfg, a, b)
            if i < n - 1:
                tn = f.taus[i + 1]
                # DDIM re-noises with the guided prediction, LCM with fresh noise
                z = eps_cfg if f.renoise is None else f.renoise[i]
                f.x = guidance.renoise(x0_hat, z, self.a[tn], self.b[tn])
            else:
                outs.append(x0_hat)
                exits.append((f, exit_kv, exit_hidden))
        n_rows = len(rows) + len(neg_eps) + len(uncond)
        if getattr(cfg, "kv_recompute", False) and exits and not self.identity:
            # clean-latent recompute: the leaving chunks' cache entries and sink
            # embeddings come from a forward of their emitted x0_hat at tau = 0
            # over the same snapshot; its eps is not used
            frames = [f for f, _, _ in exits]
            if getattr(cfg, "batch_attn", False):
                clean = self.net.forward_batch([(x, 0, f.t0) for f, x in zip(frames, outs)], snapshot,
                                               self.ctx_kv, collect=set(range(len(frames))))
            else:
                clean = [self.net.forward_row(x, 0, f.t0, snapshot, self.ctx_kv, collect=True)
                         for f, x in zip(frames, outs)]
            exits = [(f, kv, hidden) for f, (_, kv, hidden) in zip(frames, clean)]
            self.last_eps.extend(e for e, _, _ in clean)
            n_rows += len(clean)
        info = StepInfo(self.n_steps, bool(exits), exits[0][0].fid if exits else -1, n_rows,
                        0, 0, 0, False, -1, float("nan"), self.rope_p, len(exits))
        if exits:
            self.slots[n - 1] = None
            if not self.identity and not self.freeze:
                for _, kv, hidden in exits:
                    self._append(kv, hidden, info)
        info.kv_ptr, info.kv_valid, info.sink_count = self.kv_ptr, self.kv_valid, self.sink_count
        self.n_steps += 1
        if not outs:
            return None, info
        return (outs[0] if B == 1 else np.stack(outs)), info

    def _append(self, own_kv, hidden, info):
        cfg = self.cfg
        W, L = cfg.window_tokens, cfg.tokens
        h = hidden.mean(axis=0)
        if cfg.sink_tokens > 0:
            if self.sink_count < self.M:
                j = self.sink_count
                self._write_sink(j, own_kv, h)
                self.sink_count += 1
            else:
                j, sim, refresh = controls.sink_refresh_choice(h, self.sink_emb, cfg.sink_tau)
                info.sink_sim = sim
                info.sink_entry = j
                info.sink_refreshed = bool(refresh)       # the last leaving chunk's decision
                if refresh:
                    self._write_sink(j, own_kv, h)
        if W > 0:
            for b in range(cfg.n_blocks):
                k, v = own_kv[b]
                for j in range(L):
                    pos = (self.kv_ptr + j) % W
                    self.ringK[b, pos] = k[j]
                    self.ringV[b, pos] = v[j]
            self.kv_ptr = (self.kv_ptr + L) % W
            self.kv_valid = min(W, self.kv_valid + L)

    def _write_sink(self, j, own_kv, h):
        Se = self.Se
        for b in range(self.cfg.n_blocks):
            k, v = own_kv[b]
            self.sinkK[b, j * Se:(j + 1) * Se] = k[:Se]
            self.sinkV[b, j * Se:(j + 1) * Se] = v[:Se]
        self.sink_emb[j] = h.copy()


def denoise_sequential(cfg, net: Denoiser, x0, noise, taus, t0, a, b, snapshots=None, ctx_kv=None,
                       x0_star=None, ctx_kv_neg=None):
    """One frame denoised on its own, slot after slot, with no pipelining:
    the reference side of the Stream Batch invariant.  snapshots[i] is the
    cache the frame reads at its i-th step (None: no cache).  With
    ctx_kv_neg (full CFG) eps' is the prediction under that context."""
    x = guidance.entry_noise(x0, noise, a[taus[0]], b[taus[0]])
    xs = x0 if x0_star is None else x0_star
    n = len(taus)
    for i in range(n):
        tau = taus[i]
        snap = None if snapshots is None else snapshots[i]
        eps_c = net.forward_row(x, tau, t0, snap, ctx_kv)
        if ctx_kv_neg is not None:
            eps_p = net.forward_row(x, tau, t0, snap, ctx_kv_neg)
        else:
            eps_p = guidance.virtual_residual(x, xs, a[tau], b[tau])
        eps_cfg = guidance.rcfg(eps_c, eps_p, cfg.gamma, cfg.delta)
        x0_hat = guidance.predict_x0(x, eps_cfg, a[tau], b[tau])
        if i == n - 1:
            return x0_hat
        x = guidance.renoise(x0_hat, eps_cfg, a[taus[i + 1]], b[taus[i + 1]])
