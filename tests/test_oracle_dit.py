"""Pins for oracle.dit: each part of the denoiser against a definition,
a textbook value, a mathematical property or brute force."""
import itertools
import math

import numpy as np
import pytest

from oracle import dit
from workloads import gen, get_config


def rng(seed=0):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ LayerNorm
def test_layernorm_moments_and_invariance():
    x = rng().standard_normal((5, 37)) * 3 + 1.5
    y = dit.layer_norm(x, eps=0.0)
    assert np.allclose(y.mean(-1), 0, atol=1e-14)
    # population variance (divide by n, not n-1) is exactly one
    assert np.allclose((y ** 2).mean(-1), 1, atol=1e-13)
    # invariant to shift and positive scale of the input
    assert np.allclose(dit.layer_norm(2.5 * x - 7.0, eps=0.0), y, atol=1e-12)


def test_layernorm_eps_enters_under_the_root():
    x = np.array([[-1.0, 1.0]])       # mean 0, population variance 1
    y = dit.layer_norm(x, eps=1e-6)
    assert np.allclose(y, x / math.sqrt(1 + 1e-6), rtol=0, atol=1e-15)


# ------------------------------------------------------------------ GELU / SiLU
def test_gelu_textbook_values():
    # GELU(x) = x * Phi(x); Phi(1) = 0.8413447460685429 (normal CDF table value)
    x = np.array([0.0, 1.0, -1.0, 2.0, 8.0])
    y = dit.gelu(x)
    assert y[0] == 0.0
    assert abs(y[1] - 0.8413447460685429) < 1e-15
    assert abs(y[2] + (1 - 0.8413447460685429)) < 1e-15
    assert abs(y[3] - 2 * 0.9772498680518208) < 1e-14
    assert abs(y[4] - 8.0) < 1e-12


def test_silu_values():
    assert dit.silu(np.array([0.0]))[0] == 0.0
    assert abs(dit.silu(np.array([1.0]))[0] - 1 / (1 + math.exp(-1))) < 1e-16


# ------------------------------------------------------------------ linear
def test_linear_integer_brute_force():
    r = rng(1)
    x = r.integers(-5, 6, size=(3, 4)).astype(np.float64)
    w = r.integers(-5, 6, size=(6, 4)).astype(np.float64)
    b = r.integers(-5, 6, size=6).astype(np.float64)
    y = dit.linear(x, w, b)
    for i in range(3):
        for o in range(6):
            assert y[i, o] == sum(int(x[i, k]) * int(w[o, k]) for k in range(4)) + int(b[o])


# ------------------------------------------------------------------ embedding
def test_timestep_embedding_layout():
    e = dit.timestep_embedding(0, 8)
    assert np.array_equal(e, [1, 1, 1, 1, 0, 0, 0, 0])
    e = dit.timestep_embedding(3.0, 8)
    assert abs(e[0] - math.cos(3.0)) < 1e-15 and abs(e[4] - math.sin(3.0)) < 1e-15
    # w_j = 10000^(-j/4): j = 2 -> 0.01
    assert abs(e[2] - math.cos(0.03)) < 1e-15 and abs(e[6] - math.sin(0.03)) < 1e-15


# ------------------------------------------------------------------ patchify
def test_patchify_index_map_and_round_trip():
    T, C, H, W, p = 2, 3, 4, 6, 2
    lat = np.arange(T * C * H * W, dtype=np.float64).reshape(T, C, H, W)
    tok = dit.patchify(lat, p)
    Hp, Wp = H // p, W // p
    assert tok.shape == (T * Hp * Wp, p * p * C)
    for t, y, x, py, px, c in itertools.product(range(T), range(Hp), range(Wp), range(p), range(p), range(C)):
        ti = (t * Hp + y) * Wp + x
        vi = (py * p + px) * C + c
        assert tok[ti, vi] == lat[t, c, y * p + py, x * p + px]
    assert np.array_equal(dit.unpatchify(tok, T, C, H, W, p), lat)


# ------------------------------------------------------------------ RoPE
@pytest.mark.parametrize("hd,expect", [(32, (12, 10, 10)), (64, (24, 20, 20)), (128, (44, 42, 42))])
def test_rope_sections(hd, expect):
    assert dit.rope_sections(hd) == expect


def test_rope_rotates_a_unit_pair_by_the_axis_frequency():
    hd = 32                                 # sections t=12, h=10, w=10
    x = np.zeros((1, 1, hd))
    # pair j=2 of the h section sits at offset 12 + 4
    x[0, 0, 16] = 1.0
    pos = np.array([[5, 3, 7]])
    y = dit.rope_apply(x, pos)
    th = 3 * 10000.0 ** (-2 * 2 / 10)
    assert abs(y[0, 0, 16] - math.cos(th)) < 1e-15
    assert abs(y[0, 0, 17] - math.sin(th)) < 1e-15
    assert np.count_nonzero(np.abs(y) > 1e-15) == 2
    # second element of a pair turns the other way round
    x2 = np.zeros((1, 1, hd)); x2[0, 0, 1] = 1.0      # pair 0 of the t section
    y2 = dit.rope_apply(x2, pos)
    assert abs(y2[0, 0, 0] + math.sin(5.0)) < 1e-15 and abs(y2[0, 0, 1] - math.cos(5.0)) < 1e-15


def test_rope_norm_and_relative_position():
    r = rng(2)
    hd, H = 64, 3
    q = r.standard_normal((4, H, hd))
    k = r.standard_normal((4, H, hd))
    pq = r.integers(0, 50, size=(4, 3))
    pk = r.integers(0, 50, size=(4, 3))
    rq, rk = dit.rope_apply(q, pq), dit.rope_apply(k, pk)
    assert np.allclose(np.linalg.norm(rq, axis=-1), np.linalg.norm(q, axis=-1), atol=1e-12)
    shift = np.array([[11, -3, 40]])
    rq2, rk2 = dit.rope_apply(q, pq + shift), dit.rope_apply(k, pk + shift)
    assert np.allclose(np.einsum("lhd,lhd->lh", rq, rk), np.einsum("lhd,lhd->lh", rq2, rk2), atol=1e-11)


# ------------------------------------------------------------------ attention
def attention_loops(q, k, v):
    """Plain per-query softmax with Python loops."""
    Lq, H, hd = q.shape
    out = np.zeros_like(q)
    for h in range(H):
        for i in range(Lq):
            s = [sum(q[i, h, e] * k[j, h, e] for e in range(hd)) / math.sqrt(hd) for j in range(k.shape[0])]
            mx = max(s)
            ex = [math.exp(t - mx) for t in s]
            z = sum(ex)
            for e in range(hd):
                out[i, h, e] = sum(ex[j] * v[j, h, e] for j in range(k.shape[0])) / z
    return out


def test_attention_brute_force():
    r = rng(3)
    q = r.standard_normal((5, 2, 4))
    k = r.standard_normal((7, 2, 4))
    v = r.standard_normal((7, 2, 4))
    assert np.allclose(dit.attention(q, k, v), attention_loops(q, k, v), atol=1e-13)


def test_attention_special_cases():
    r = rng(4)
    q = r.standard_normal((3, 2, 8))
    k1, v1 = r.standard_normal((1, 2, 8)), r.standard_normal((1, 2, 8))
    assert np.allclose(dit.attention(q, k1, v1), np.broadcast_to(v1, (3, 2, 8)), atol=1e-15)
    keq = np.repeat(k1, 5, axis=0)
    v5 = r.standard_normal((5, 2, 8))
    assert np.allclose(dit.attention(q, keq, v5), np.broadcast_to(v5.mean(0), (3, 2, 8)), atol=1e-14)
    k6, v6 = r.standard_normal((6, 2, 8)), r.standard_normal((6, 2, 8))
    perm = r.permutation(6)
    assert np.allclose(dit.attention(q, k6, v6), dit.attention(q, k6[perm], v6[perm]), atol=1e-14)


# ------------------------------------------------------------------ block structure
def tiny_net(**over):
    cfg = get_config("tiny", **over)
    w = gen.make_weights(cfg)
    return cfg, w


def test_zero_gate_blocks_are_identity():
    """With both gates of every block forced to zero (through the per-block
    table) the blocks pass x through, so eps only depends on the patch
    embedding and the final layer.  Checked against a network with no
    blocks at all."""
    cfg, w = tiny_net()
    net = dit.Denoiser(cfg, w)
    tau = 359
    m = net.modulation(net.cond(tau))
    d = cfg.d_model
    w2 = dict(w)
    bm = w["blk_mod"].astype(np.float64).copy()
    for b in range(cfg.n_blocks):
        bm[b, 2 * d:3 * d] = -m[2 * d:3 * d]
        bm[b, 5 * d:6 * d] = -m[5 * d:6 * d]
    w2["blk_mod"] = bm
    x = rng(5).standard_normal((1, 4, 16, 16))
    e_gated = dit.Denoiser(cfg, w2).forward_row(x, tau, 0)
    cfg0 = cfg.replace(n_blocks=0)
    w0 = {k: (v[:0] if v.ndim >= 1 and v.shape[0] == cfg.n_blocks and k not in ("t_w1", "t_b1") and
              k in ("blk_mod", "qkv_w", "qkv_b", "o_w", "o_b", "f1_w", "f1_b", "f2_w", "f2_b") else v)
          for k, v in w.items()}
    e0 = dit.Denoiser(cfg0, w0).forward_row(x, tau, 0)
    assert np.allclose(e_gated, e0, atol=1e-10)


def test_modulation_with_zero_scale_shift_is_layernorm():
    x = rng(6).standard_normal((4, 16))
    z = np.zeros(16)
    assert np.array_equal(dit.modulate(dit.layer_norm(x), z, z), dit.layer_norm(x))


# ------------------------------------------------------------------ modulation slots, final layer, cross branch
# One latent patch (4 x 2 x 2 with p = 2) is one token, so self-attention over
# the row's own chunk with no cache sees a single key and returns its value
# exactly; the block can then be read off in closed form.
def _one_token_net(n_blocks=1, ctx_len=0):
    cfg = get_config("tiny", n_blocks=n_blocks, ctx_len=ctx_len)
    w = {k: np.asarray(v, np.float64) for k, v in gen.make_weights(cfg).items()}
    return cfg, w


def _set_modulation(w, slots):
    """Make the shared modulation vector equal concat(slots) for every tau:
    zero projection, bias = the slots, zero per-block table."""
    w["mod_w"] = np.zeros_like(w["mod_w"])
    w["mod_b"] = np.concatenate(slots)
    w["blk_mod"] = np.zeros_like(w["blk_mod"])


def _patch_embed(w, x):
    # the single token of a 4 x 2 x 2 latent, vector order (py, px, c)
    tok = np.array([[x[0, c, py, px] for py in range(2) for px in range(2) for c in range(4)]])
    return tok @ w["pe_w"].T + w["pe_b"]


def test_block_modulation_slots_are_shift_scale_gate():
    """block_mod's split: slots 0..5 are (shift, scale, gate) for attention,
    then for the MLP.  With V and the output projection the identity, one
    token and the MLP gate zero, the block output is
    x + g1 * (LN(x) * (1 + s1) + h1) exactly; any other assignment of the six
    distinct random slot vectors changes it."""
    cfg, w = _one_token_net()
    d = cfg.d_model
    r = rng(11)
    h1, s1, g1, h2, s2 = (r.standard_normal(d) for _ in range(5))
    _set_modulation(w, [h1, s1, g1, h2, s2, np.zeros(d)])
    w["qkv_w"][0, 2 * d:] = np.eye(d)
    w["qkv_b"][0] = 0.0
    w["o_w"][0] = np.eye(d)
    w["o_b"][0] = 0.0
    x = r.standard_normal((1, 4, 2, 2))
    _, _, hidden = dit.Denoiser(cfg, w).forward_row(x, 359, 0, collect=True)
    x_pe = _patch_embed(w, x)
    mu = x_pe.mean()
    ln = (x_pe - mu) / math.sqrt(((x_pe - mu) ** 2).mean() + 1e-6)
    expect = x_pe + g1 * (ln * (1 + s1) + h1)
    assert np.allclose(hidden, expect, rtol=0, atol=1e-12)
    # a swapped split (shift <-> scale) would give a different hidden state
    assert not np.allclose(x_pe + g1 * (ln * (1 + h1) + s1), expect, atol=1e-3)


def test_final_layer_split_is_shift_then_scale():
    """The final layer's 2d vector is (shift, scale): with no blocks, the head
    picking the first p*p*C features and zero bias, eps is
    (LN(x) * (1 + s_f) + h_f)[:16] unpatchified."""
    cfg, w = _one_token_net()
    d = cfg.d_model
    r = rng(12)
    hf, sf = r.standard_normal(d), r.standard_normal(d)
    w["fin_w"] = np.zeros_like(w["fin_w"])
    w["fin_b"] = np.concatenate([hf, sf])
    w["head_w"] = np.eye(16, d)
    w["head_b"] = np.zeros(16)
    # zero both gates so the block passes x through
    m = np.zeros(6 * d)
    _set_modulation(w, [m[:d]] * 6)
    x = r.standard_normal((1, 4, 2, 2))
    eps = dit.Denoiser(cfg, w).forward_row(x, 99, 0)
    x_pe = _patch_embed(w, x)[0]
    mu = x_pe.mean()
    out = ((x_pe - mu) / math.sqrt(((x_pe - mu) ** 2).mean() + 1e-6) * (1 + sf) + hf)[:16]
    for py in range(2):
        for px in range(2):
            for c in range(4):
                assert abs(eps[0, c, py, px] - out[(py * 2 + px) * 4 + c]) < 1e-12


def test_cross_branch_is_ungated_and_adds_its_output():
    """Cross-attention adds its projected output to x with no gate and no
    modulation.  With zero query / key / value weights and biases the
    attention output is zero, so the block adds exactly co_b; with the value
    projection the identity and zero keys every prompt token gets weight
    1/77, so it adds mean(ctx) W_o^T + co_b.  Both gates are zero, so
    self-attention and the MLP add nothing."""
    cfg, w = _one_token_net(ctx_len=77)
    d, H, hd = cfg.d_model, cfg.n_heads, cfg.head_dim
    r = rng(13)
    _set_modulation(w, [np.zeros(d)] * 6)
    ctx = r.standard_normal((77, d))
    x = r.standard_normal((1, 4, 2, 2))
    x_pe = _patch_embed(w, x)
    co_b = r.standard_normal(d)
    for name in ("cq_w", "cq_b", "ckv_w", "ckv_b", "co_w"):
        w[name] = np.zeros_like(w[name])
    w["co_b"][0] = co_b
    net = dit.Denoiser(cfg, w)
    _, _, hidden = net.forward_row(x, 359, 0, ctx_kv=[net.cross_kv(ctx, 0)], collect=True)
    assert np.allclose(hidden, x_pe + co_b, rtol=0, atol=1e-12)
    # value projection = identity, zero keys (uniform weights), output = identity
    w["ckv_w"][0, d:] = np.eye(d)
    w["co_w"][0] = np.eye(d)
    w["cq_w"][0] = r.standard_normal((d, d))
    net = dit.Denoiser(cfg, w)
    _, _, hidden = net.forward_row(x, 359, 0, ctx_kv=[net.cross_kv(ctx, 0)], collect=True)
    assert np.allclose(hidden, x_pe + ctx.mean(0) + co_b, rtol=0, atol=1e-12)
