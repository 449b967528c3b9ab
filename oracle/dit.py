"""The DiT denoiser, written out plainly.

The pages fix only the outline: a video DiT (Wan 2.1 / CausVid class) whose
attention reads a sink-token plus rolling-window KV cache, with RoPE
(StreamDiffusionV2 summary, adaptive sink and RoPE refresh), and
pre-computed prompt-side attention K/V (StreamDiffusion project intro,
feature 5).  Every network detail below is a reading chosen so the parameter
counts match the "1.3B-shaped" / "~28 GB" labels of the workloads:

* patchify with a 1 x p x p patch; tokens ordered (frame, y, x), a token's
  vector ordered (py, px, c);
* timestep embedding [cos(tau w_j), sin(tau w_j)], w_j = 10000^(-j/(D/2)),
  then Linear-SiLU-Linear -> c;
* adaLN: m = W_mod SiLU(c) + b_mod (6d, shared by all blocks); block b uses
  m + E_b split as (shift, scale, gate) for attention then for the MLP;
* block: x += g1 * Attn(mod(LN(x), s1, h1)); if a context is configured
  x += CrossAttn(LN(x), ctx) (no modulation, no gate);
  x += g2 * FFN(mod(LN(x), s2, h2)), FFN = Linear-GELU(erf)-Linear;
* LayerNorm without affine, eps 1e-6, population variance;
* final: (shift_f, scale_f) = W_f SiLU(c) + b_f; out = Linear(mod(LN(x)));
  unpatchify; the output is an epsilon prediction;
* attention scale 1/sqrt(hd), bidirectional within the row's own chunk,
  keys = sink + valid window + own; rows never see each other;
* 3D RoPE on q and k: head dim split (t, h, w) with h = w = 2*floor(hd/6),
  t the rest; interleaved pairs (x_2j, x_2j+1); base 10000; K is cached after
  RoPE.

Pins (tests/test_oracle_dit.py): LayerNorm and GELU against their scalar
definitions, linear against integer brute force, RoPE norm preservation,
relative-position property and the rotation of a unit pair, attention
against a pure-Python softmax loop and its special cases, modulation with
zero scale/shift reducing to LayerNorm, a block whose gates are zero being
the identity, the six modulation slots read off a one-token block in closed
form (shift, scale, gate for attention, then for the MLP), the final layer's
(shift, scale) order, and the cross-attention branch adding its projected
output without gate or modulation.  The composed forward is "parity unpinned" beyond its parts.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf


# ---------------------------------------------------------------- primitives
def silu(x):
    return x / (1.0 + np.exp(-x))


def gelu(x):
    """Exact GELU: x * Phi(x) with the standard normal CDF via erf."""
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def layer_norm(x, eps: float = 1e-6):
    """Normalise the last axis; population variance; no affine."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def modulate(xn, shift, scale):
    return xn * (1.0 + scale) + shift


def linear(x, w, b=None):
    """y = x W^T + b with W stored [out, in]."""
    y = x @ w.T
    return y if b is None else y + b


def timestep_embedding(tau: float, d_freq: int, dtype=np.float64):
    half = d_freq // 2
    j = np.arange(half, dtype=np.float64)
    w = 10000.0 ** (-j / half)
    arg = float(tau) * w
    return np.concatenate([np.cos(arg), np.sin(arg)]).astype(dtype)


# ---------------------------------------------------------------- layout
def patchify(lat, p: int):
    """[T][C][H][W] -> [T*(H/p)*(W/p), p*p*C], token order (t, y, x),
    vector order (py, px, c)."""
    T, C, H, W = lat.shape
    x = lat.reshape(T, C, H // p, p, W // p, p)          # t c y py x px
    x = x.transpose(0, 2, 4, 3, 5, 1)                    # t y x py px c
    return x.reshape(T * (H // p) * (W // p), p * p * C)


def unpatchify(tok, T: int, C: int, H: int, W: int, p: int):
    x = tok.reshape(T, H // p, W // p, p, p, C)          # t y x py px c
    x = x.transpose(0, 5, 1, 3, 2, 4)                    # t c y py x px
    return x.reshape(T, C, H, W)


def token_positions(T: int, Hp: int, Wp: int, t0: int):
    """Integer (temporal, y, x) position of every token; t0 is the chunk's
    temporal RoPE base."""
    t, y, x = np.meshgrid(np.arange(T), np.arange(Hp), np.arange(Wp), indexing="ij")
    return np.stack([t.ravel() + t0, y.ravel(), x.ravel()], axis=1)


# ---------------------------------------------------------------- RoPE
def rope_sections(hd: int):
    """(t, h, w) widths of the head dim: h = w = 2*floor(hd/6), t = rest."""
    hw = 2 * (hd // 6)
    return hd - 2 * hw, hw, hw


def rope_apply(x, pos, base: float = 10000.0):
    """Rotate x [L, H, hd] by token positions pos [L, 3].

    Each axis section of width D_a holds D_a/2 interleaved pairs; pair j of
    that section turns by angle pos_a * base^(-2j/D_a)."""
    L, H, hd = x.shape
    out = x.copy()
    off = 0
    for a, width in enumerate(rope_sections(hd)):
        for j in range(width // 2):
            theta = pos[:, a].astype(np.float64) * base ** (-2.0 * j / width)
            c = np.cos(theta)[:, None].astype(x.dtype)
            s = np.sin(theta)[:, None].astype(x.dtype)
            i0, i1 = off + 2 * j, off + 2 * j + 1
            x0, x1 = x[:, :, i0], x[:, :, i1]
            out[:, :, i0] = x0 * c - x1 * s
            out[:, :, i1] = x0 * s + x1 * c
        off += width
    return out


# ---------------------------------------------------------------- attention
def attention(q, k, v):
    """softmax(q k^T / sqrt(hd)) v per head.  q [Lq,H,hd], k/v [Lk,H,hd]."""
    hd = q.shape[-1]
    qh = q.transpose(1, 0, 2)
    kh = k.transpose(1, 0, 2)
    vh = v.transpose(1, 0, 2)
    s = qh @ kh.transpose(0, 2, 1) / math.sqrt(hd)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    pr = e / e.sum(axis=-1, keepdims=True)
    return (pr @ vh).transpose(1, 0, 2)


# ---------------------------------------------------------------- network
class Denoiser:
    """Holds the weights (as arrays of the working dtype) and the config."""

    def __init__(self, cfg, weights: dict, dtype=np.float64):
        self.cfg = cfg
        self.dtype = dtype
        self.w = {k: np.asarray(v, dtype=dtype) for k, v in weights.items()}

    # conditioning -----------------------------------------------------------
    def cond(self, tau):
        """Return (SiLU(c)) for timestep tau."""
        w = self.w
        e = timestep_embedding(tau, self.cfg.d_freq, self.dtype)
        h = silu(linear(e, w["t_w1"], w["t_b1"]))
        c = linear(h, w["t_w2"], w["t_b2"])
        return silu(c)

    def modulation(self, sc):
        """Shared 6d modulation vector from SiLU(c)."""
        return linear(sc, self.w["mod_w"], self.w["mod_b"])

    def block_mod(self, m, b):
        d = self.cfg.d_model
        mb = m + self.w["blk_mod"][b]
        return [mb[i * d:(i + 1) * d] for i in range(6)]  # h1 s1 g1 h2 s2 g2

    def cross_kv(self, ctx, b):
        """Prompt-side K/V of block b, computed once per context."""
        d = self.cfg.d_model
        kv = linear(np.asarray(ctx, self.dtype), self.w["ckv_w"][b], self.w["ckv_b"][b])
        H, hd = self.cfg.n_heads, self.cfg.head_dim
        return kv[:, :d].reshape(-1, H, hd), kv[:, d:].reshape(-1, H, hd)

    # one row ------------------------------------------------------------------
    def forward_row(self, x_lat, tau, t0, cache_kv=None, ctx_kv=None, collect=False):
        """Denoise one chunk.

        x_lat    : [T][C][H][W] noisy latent at timestep tau
        t0       : temporal RoPE base of the chunk
        cache_kv : per block (K_cache, V_cache) arrays [n, H, hd] holding the
                   sink and valid window keys/values (post-RoPE), or None
        ctx_kv   : per block (K_ctx, V_ctx) or None (no cross-attention)
        Returns eps [T][C][H][W]; with collect=True also the per-block own
        (K, V) [L, H, hd] and the last block's output hidden state [L, d].
        """
        cfg, w = self.cfg, self.w
        d, H, hd, p = cfg.d_model, cfg.n_heads, cfg.head_dim, cfg.patch
        T, C, Hl, Wl = x_lat.shape
        L = T * (Hl // p) * (Wl // p)
        pos = token_positions(T, Hl // p, Wl // p, t0)

        sc = self.cond(tau)
        m = self.modulation(sc)
        x = linear(patchify(np.asarray(x_lat, self.dtype), p), w["pe_w"], w["pe_b"])   # [L, d]
        own = []
        for b in range(cfg.n_blocks):
            h1, s1, g1, h2, s2, g2 = self.block_mod(m, b)
            # self-attention over sink + window + own
            xm = modulate(layer_norm(x), h1, s1)
            qkv = linear(xm, w["qkv_w"][b], w["qkv_b"][b])
            q = rope_apply(qkv[:, :d].reshape(L, H, hd), pos, cfg.rope_base)
            k = rope_apply(qkv[:, d:2 * d].reshape(L, H, hd), pos, cfg.rope_base)
            v = qkv[:, 2 * d:].reshape(L, H, hd)
            own.append((k, v))
            if cache_kv is not None and cache_kv[b][0].shape[0] > 0:
                kk = np.concatenate([cache_kv[b][0], k], axis=0)
                vv = np.concatenate([cache_kv[b][1], v], axis=0)
            else:
                kk, vv = k, v
            a = attention(q, kk, vv).reshape(L, d)
            x = x + g1 * linear(a, w["o_w"][b], w["o_b"][b])
            # cross-attention to the prompt
            if ctx_kv is not None:
                qc = linear(layer_norm(x), w["cq_w"][b], w["cq_b"][b]).reshape(L, H, hd)
                ac = attention(qc, ctx_kv[b][0], ctx_kv[b][1]).reshape(L, d)
                x = x + linear(ac, w["co_w"][b], w["co_b"][b])
            # feed-forward
            xm = modulate(layer_norm(x), h2, s2)
            hdn = gelu(linear(xm, w["f1_w"][b], w["f1_b"][b]))
            x = x + g2 * linear(hdn, w["f2_w"][b], w["f2_b"][b])
        hidden = x
        fm = linear(sc, w["fin_w"], w["fin_b"])
        out = linear(modulate(layer_norm(x), fm[:d], fm[d:]), w["head_w"], w["head_b"])
        eps = unpatchify(out, T, C, Hl, Wl, p)
        if collect:
            return eps, own, hidden
        return eps

    def forward_batch(self, rows, cache_kv=None, ctx_kv=None, collect=()):
        """Denoise the rows of one forward together with cross-frame batch
        attention (StreamDiffusion paper notes, section 1, temporal
        consistency: a row's queries attend to the keys and values of the
        whole batch).  Reading with the KV cache: each row attends to
        [cache | every row's own tokens, rows in batch order].  Everything
        else is forward_row's block, row by row.

        rows    : list of (x_lat, tau, t0)
        collect : indices of rows that return (eps, own, hidden) as
                  forward_row(collect=True) does; the others return eps.
        """
        cfg, w = self.cfg, self.w
        d, H, hd, p = cfg.d_model, cfg.n_heads, cfg.head_dim, cfg.patch
        st = []
        for x_lat, tau, t0 in rows:
            T, C, Hl, Wl = x_lat.shape
            sc = self.cond(tau)
            st.append({"shape": (T, C, Hl, Wl), "L": T * (Hl // p) * (Wl // p),
                       "pos": token_positions(T, Hl // p, Wl // p, t0), "sc": sc, "m": self.modulation(sc),
                       "x": linear(patchify(np.asarray(x_lat, self.dtype), p), w["pe_w"], w["pe_b"]), "own": []})
        for b in range(cfg.n_blocks):
            qs = []
            for r in st:
                L = r["L"]
                h1, s1, g1, h2, s2, g2 = self.block_mod(r["m"], b)
                xm = modulate(layer_norm(r["x"]), h1, s1)
                qkv = linear(xm, w["qkv_w"][b], w["qkv_b"][b])
                qs.append(rope_apply(qkv[:, :d].reshape(L, H, hd), r["pos"], cfg.rope_base))
                k = rope_apply(qkv[:, d:2 * d].reshape(L, H, hd), r["pos"], cfg.rope_base)
                r["own"].append((k, qkv[:, 2 * d:].reshape(L, H, hd)))
            kb = np.concatenate([r["own"][b][0] for r in st], axis=0)
            vb = np.concatenate([r["own"][b][1] for r in st], axis=0)
            if cache_kv is not None and cache_kv[b][0].shape[0] > 0:
                kk = np.concatenate([cache_kv[b][0], kb], axis=0)
                vv = np.concatenate([cache_kv[b][1], vb], axis=0)
            else:
                kk, vv = kb, vb
            for r, q in zip(st, qs):
                L = r["L"]
                h1, s1, g1, h2, s2, g2 = self.block_mod(r["m"], b)
                x = r["x"]
                a = attention(q, kk, vv).reshape(L, d)
                x = x + g1 * linear(a, w["o_w"][b], w["o_b"][b])
                if ctx_kv is not None:
                    qc = linear(layer_norm(x), w["cq_w"][b], w["cq_b"][b]).reshape(L, H, hd)
                    ac = attention(qc, ctx_kv[b][0], ctx_kv[b][1]).reshape(L, d)
                    x = x + linear(ac, w["co_w"][b], w["co_b"][b])
                xm = modulate(layer_norm(x), h2, s2)
                hdn = gelu(linear(xm, w["f1_w"][b], w["f1_b"][b]))
                r["x"] = x + g2 * linear(hdn, w["f2_w"][b], w["f2_b"][b])
        outs = []
        for j, r in enumerate(st):
            T, C, Hl, Wl = r["shape"]
            fm = linear(r["sc"], w["fin_w"], w["fin_b"])
            out = linear(modulate(layer_norm(r["x"]), fm[:d], fm[d:]), w["head_w"], w["head_b"])
            eps = unpatchify(out, T, C, Hl, Wl, p)
            outs.append((eps, r["own"], r["x"]) if j in collect else eps)
        return outs
