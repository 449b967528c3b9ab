"""GPU parity of single kernels through the C ABI (sd_k_*), against the CPU
oracle or exact integer arithmetic, at small ragged sizes and at the full
shapes of the 1.3B-shaped video workload."""
import ctypes as C

import numpy as np
import pytest
import torch

from oracle import controls
from oracle.dit import attention as oracle_attention
from workloads import gen, get_config

from gpu_helpers import (BF16_TOL, FP32_TOL, bf16_round, call, check_close, device, maxabs_over_rms, rel_inf,
                         stream_ptr, to_dev)

pytestmark = pytest.mark.gpu

import streaming_diffusion_amd._lib as sdlib


@pytest.fixture(scope="module")
def lib():
    device()
    return sdlib.load()


# ------------------------------------------------------------------ GEMM
@pytest.mark.parametrize("M,N,K", [(300, 200, 136), (64, 64, 16), (1, 8, 8), (257, 129, 1040), (400, 300, 128),
                                   (6240, 4608, 1536), (6240, 1536, 8960), (6240, 960, 1536)])
def test_gemm_bf16_exact_integers(lib, M, N, K):
    """Inputs k/16 with |k| <= 8 are exact in bf16 and every product and
    partial sum is exact in fp32, so the MFMA result must equal the integer
    matmul bit for bit (ragged M/N/K tails included)."""
    print(f"gemm exact M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(M * 7 + N)
    ai = rng.integers(-8, 9, size=(M, K))
    wi = rng.integers(-8, 9, size=(N, K))
    bi = rng.integers(-8, 9, size=N)
    A = to_dev(ai / 16.0, torch.bfloat16)
    W = to_dev(wi / 16.0, torch.bfloat16)
    b = to_dev(bi / 16.0, torch.bfloat16)
    out = torch.empty((M, N), dtype=torch.float32, device=device())
    call(lib.sd_k_gemm(1, A.data_ptr(), W.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, stream_ptr()))
    torch.cuda.synchronize()
    ref = (ai.astype(np.float64) @ wi.T.astype(np.float64)) / 256.0 + bi / 16.0
    assert np.array_equal(out.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("M,N,K", [(400, 300, 128), (64, 64, 64), (1, 8, 64), (300, 200, 136), (300, 200, 4096),
                                   (1000, 520, 2048), (1500, 700, 1600), (2048, 768, 3072), (6240, 1536, 1536),
                                   (6240, 1536, 8960), (3120, 5120, 5120), (6240, 1536, 960)])
def test_gemm_resid_bf16_exact_integers(lib, M, N, K):
    """Residual accumulation C += A W^T + b with integer-valued operands: every
    product, partial sum and the final sum are exact in fp32, so the result is
    the integer arithmetic bit for bit (ragged tiles, both DMA tile shapes, and
    K not a multiple of 64 included)."""
    print(f"gemm resid exact M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(M * 3 + N + K)
    ai = rng.integers(-8, 9, size=(M, K))
    wi = rng.integers(-8, 9, size=(N, K))
    bi = rng.integers(-8, 9, size=N)
    ci = rng.integers(-4096, 4097, size=(M, N))
    A = to_dev(ai / 16.0, torch.bfloat16)
    W = to_dev(wi / 16.0, torch.bfloat16)
    b = to_dev(bi / 16.0, torch.bfloat16)
    out = to_dev(ci / 256.0, torch.float32)
    call(lib.sd_k_gemm_resid(1, A.data_ptr(), W.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, stream_ptr()))
    torch.cuda.synchronize()
    ref = (ai.astype(np.float64) @ wi.T.astype(np.float64) + ci) / 256.0 + bi / 16.0
    assert np.array_equal(out.cpu().numpy().astype(np.float64), ref)


def test_gemm_resid_f32_matches_numpy(lib):
    M, N, K = 130, 70, 24
    rng = np.random.default_rng(9)
    a = rng.standard_normal((M, K)).astype(np.float32)
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    c = rng.standard_normal((M, N)).astype(np.float32)
    A, W, out = to_dev(a, torch.float32), to_dev(w, torch.float32), to_dev(c, torch.float32)
    call(lib.sd_k_gemm_resid(0, A.data_ptr(), W.data_ptr(), None, out.data_ptr(), M, N, K, stream_ptr()))
    torch.cuda.synchronize()
    ref = c.astype(np.float64) + a.astype(np.float64) @ w.T.astype(np.float64)
    assert rel_inf(out.cpu().numpy(), ref) < 1e-5


@pytest.mark.parametrize("M,N,K", [(130, 70, 24), (64, 384, 128), (128, 512, 512)])
def test_gemm_f32_matches_oracle(lib, M, N, K):
    print(f"gemm f32 M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(5)
    a = rng.standard_normal((M, K)).astype(np.float32)
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    out = torch.empty((M, N), dtype=torch.float32, device=device())
    A, W = to_dev(a, torch.float32), to_dev(w, torch.float32)
    call(lib.sd_k_gemm(0, A.data_ptr(), W.data_ptr(), None, out.data_ptr(), M, N, K, stream_ptr()))
    torch.cuda.synchronize()
    ref = a.astype(np.float64) @ w.T.astype(np.float64)
    assert rel_inf(out.cpu().numpy(), ref) < 1e-5


# ------------------------------------------------------------------ attention
def make_segments(rng, H, hd, R, L, sink_count, sink_cap, W, ring_start, ring_count, tdt):
    """Random K / V^T storage for sink, ring and own segments; returns the
    device tensors, the ctypes segment array and per-row key/value arrays in
    the oracle's [keys, H, hd] layout."""
    def kv(n):
        k = rng.standard_normal((H, n, hd)).astype(np.float32)
        v = rng.standard_normal((H, n, hd)).astype(np.float32)
        return k, v
    sk, sv = kv(sink_cap)
    sk[:, sink_count:] = 0
    sv[:, sink_count:] = 0
    rk, rv = kv(W)
    ok = rng.standard_normal((R, H, L, hd)).astype(np.float32)
    ov = rng.standard_normal((R, H, L, hd)).astype(np.float32)
    if tdt == torch.bfloat16:
        sk, sv, rk, rv, ok, ov = [bf16_round(x) for x in (sk, sv, rk, rv, ok, ov)]
    dev = dict(sk=to_dev(sk, tdt), svt=to_dev(sv.transpose(0, 2, 1), tdt), rk=to_dev(rk, tdt),
               rvt=to_dev(rv.transpose(0, 2, 1), tdt), ok=to_dev(ok, tdt), ovt=to_dev(ov.transpose(0, 1, 3, 2), tdt))
    segs = (sdlib.sd_kv_segment * 3)()
    segs[0] = sdlib.sd_kv_segment(dev["sk"].data_ptr(), dev["svt"].data_ptr(), sink_cap * hd, sink_cap * hd, 0, 0,
                              sink_cap, 0, sink_count, 0)
    segs[1] = sdlib.sd_kv_segment(dev["rk"].data_ptr(), dev["rvt"].data_ptr(), W * hd, W * hd, 0, 0, W, ring_start,
                              ring_count, 1)
    segs[2] = sdlib.sd_kv_segment(dev["ok"].data_ptr(), dev["ovt"].data_ptr(), L * hd, L * hd, H * L * hd, H * L * hd,
                              L, 0, L, 0)
    ring_idx = [(ring_start + j) % W for j in range(ring_count)]
    keys, vals = [], []
    for r in range(R):
        k = np.concatenate([sk[:, :sink_count], rk[:, ring_idx], ok[r]], axis=1).transpose(1, 0, 2)
        v = np.concatenate([sv[:, :sink_count], rv[:, ring_idx], ov[r]], axis=1).transpose(1, 0, 2)
        keys.append(k)
        vals.append(v)
    return dev, segs, keys, vals


@pytest.mark.parametrize("dtype,hd,L,sink_count,W,ring_start,ring_count,nsplit", [
    ("bf16", 64, 72, 4, 64, 40, 48, 1),        # ring wraps, sink padding, ragged queries
    ("bf16", 128, 200, 12, 160, 152, 160, 1),  # full ring starting at 152 (wraps)
    ("bf16", 32, 64, 0, 64, 0, 0, 1),          # empty sink and ring (plain self-attention)
    ("bf16", 128, 136, 8, 256, 0, 256, 1),
    ("bf16", 64, 72, 4, 64, 40, 48, 2),        # split over the keys, partial combine
    ("bf16", 128, 200, 12, 512, 136, 504, 3),
    ("bf16", 128, 136, 8, 256, 0, 256, 5),     # more splits than some key ranges fill
    ("bf16", 128, 296, 4, 640, 600, 600, 1),   # 256-query tiles, the second partial; 16 key tiles, every LDS stage reused
    ("bf16", 128, 8, 0, 64, 0, 0, 1),          # a single (partial) key tile
    ("bf16", 128, 520, 0, 448, 104, 448, 2),   # three query tiles, two key splits of odd tile counts
    ("bf16", 64, 72, 0, 64, 0, 0, 1),          # full key tile then a partial one (masked keys hold real data)
    ("bf16", 64, 72, 0, 64, 0, 64, 1),         # full ring tile, full own tile, partial own tile
    ("bf16", 64, 64, 8, 64, 0, 0, 1),          # partial sink tile (8 of 64), then the own tile
    ("bf16", 64, 8, 0, 128, 0, 128, 1),        # two full ring tiles, then 8 own keys
    ("f32", 32, 64, 4, 64, 40, 48, 1),
    ("f32", 16, 40, 3, 24, 16, 20, 1),
])
def test_attention_segments_match_oracle(lib, dtype, hd, L, sink_count, W, ring_start, ring_count, nsplit):
    print(f"attention {dtype} hd={hd} L={L} sink={sink_count} W={W} start={ring_start} count={ring_count}", flush=True)
    rng = np.random.default_rng(hd + L)
    H, R = 2, 2
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    sink_cap = max(8, (sink_count + 7) // 8 * 8)
    dev, segs, keys, vals = make_segments(rng, H, hd, R, L, sink_count, sink_cap, W, ring_start, ring_count, tdt)
    q = rng.standard_normal((R, H, L, hd)).astype(np.float32)
    if dtype == "bf16":
        q = bf16_round(q)
    qd = to_dev(q, tdt)
    o = torch.empty((R * L, H * hd), dtype=tdt, device=device())
    wsb = lib.sd_k_attention_workspace_bytes(R, H, L, hd, nsplit)
    ws = torch.empty(max(wsb, 1) + 256, dtype=torch.uint8, device=device())
    wsp = (ws.data_ptr() + 255) // 256 * 256 if wsb else None
    print(f"  nsplit={nsplit} workspace={wsb}", flush=True)
    call(lib.sd_k_attention(1 if dtype == "bf16" else 0, qd.data_ptr(), H * L * hd, L * hd, o.data_ptr(), R, H, L,
                            hd, 3, segs, nsplit, wsp, wsb, stream_ptr()))
    torch.cuda.synchronize()
    got = o.float().cpu().numpy().reshape(R, L, H, hd)
    for r in range(R):
        ref = oracle_attention(q[r].transpose(1, 0, 2).astype(np.float64), keys[r].astype(np.float64),
                               vals[r].astype(np.float64))
        check_close(got[r], ref, dtype, f"attention row {r}", stored_bf16=True)


def test_attention_full_video_shape_sampled(lib):
    """The 1.3B-shaped video attention: 3120 queries per row and head against
    a 1560-token sink, a wrapped 9360-token window and the row's own 3120
    tokens (hd 128).  Sampled queries are checked one by one on the CPU."""
    print("attention full video shape", flush=True)
    rng = np.random.default_rng(11)
    H, R, hd, L, S, W = 2, 2, 128, 3120, 1560, 9360
    dev, segs, keys, vals = make_segments(rng, H, hd, R, L, S, S, W, 3120, W, torch.bfloat16)
    q = bf16_round(rng.standard_normal((R, H, L, hd)).astype(np.float32))
    qd = to_dev(q, torch.bfloat16)
    o = torch.empty((R * L, H * hd), dtype=torch.bfloat16, device=device())
    nsplit = 5
    wsb = lib.sd_k_attention_workspace_bytes(R, H, L, hd, nsplit)
    ws = torch.empty(wsb + 256, dtype=torch.uint8, device=device())
    call(lib.sd_k_attention(1, qd.data_ptr(), H * L * hd, L * hd, o.data_ptr(), R, H, L, hd, 3, segs, nsplit,
                            (ws.data_ptr() + 255) // 256 * 256, wsb, stream_ptr()))
    torch.cuda.synchronize()
    got = o.float().cpu().numpy().reshape(R, L, H, hd)
    sample = np.concatenate([np.arange(0, 5), rng.integers(0, L, 40), np.arange(L - 5, L)])
    for r in range(R):
        ref = oracle_attention(q[r].transpose(1, 0, 2)[sample].astype(np.float64), keys[r].astype(np.float64),
                               vals[r].astype(np.float64))
        check_close(got[r][sample], ref, "bf16", f"row {r}", stored_bf16=True)


def _attn_call(lib, entry, qd, o, R, H, L, hd, segs, nsplit, extra=()):
    wsb = lib.sd_k_attention_workspace_bytes(R, H, L, hd, nsplit)
    ws = torch.empty(max(wsb, 1) + 256, dtype=torch.uint8, device=device())
    wsp = (ws.data_ptr() + 255) // 256 * 256 if wsb else None
    call(entry(1, qd.data_ptr(), H * L * hd, L * hd, o.data_ptr(), R, H, L, hd, 3, segs, nsplit, *extra, wsp, wsb,
               stream_ptr()))
    torch.cuda.synchronize()
    return o.float().cpu().numpy().reshape(R, L, H, hd).copy()


@pytest.mark.parametrize("H,hd,L,sink_count,W,ring_start,ring_count,nsplit,unsplit", [
    (3, 64, 72, 4, 64, 40, 48, 2, 1),          # ring wraps, ragged queries; one head whole, two split
    (3, 128, 200, 12, 512, 136, 504, 3, 2),
    (4, 128, 136, 8, 256, 0, 256, 5, 3),       # more splits than some key ranges fill
    (3, 32, 64, 0, 64, 0, 0, 2, 3),            # every head whole: no combine
])
def test_attention_plan_matches_oracle(lib, H, hd, L, sink_count, W, ring_start, ring_count, nsplit, unsplit):
    """A split plan (heads 0 .. unsplit-1 whole, the others split): every
    head bit for bit what sd_k_attention gives it unsplit or split, and all
    of them against the brute-force oracle attention."""
    print(f"attention plan H={H} hd={hd} L={L} nsplit={nsplit} unsplit={unsplit}", flush=True)
    rng = np.random.default_rng(hd + L + H)
    R = 2
    sink_cap = max(8, (sink_count + 7) // 8 * 8)
    dev, segs, keys, vals = make_segments(rng, H, hd, R, L, sink_count, sink_cap, W, ring_start, ring_count,
                                          torch.bfloat16)
    q = bf16_round(rng.standard_normal((R, H, L, hd)).astype(np.float32))
    qd = to_dev(q, torch.bfloat16)
    o = torch.empty((R * L, H * hd), dtype=torch.bfloat16, device=device())
    got = _attn_call(lib, lib.sd_k_attention_plan, qd, o, R, H, L, hd, segs, nsplit, (unsplit,))
    whole = _attn_call(lib, lib.sd_k_attention, qd, o, R, H, L, hd, segs, 1)
    split = _attn_call(lib, lib.sd_k_attention, qd, o, R, H, L, hd, segs, nsplit)
    assert np.array_equal(got[:, :, :unsplit], whole[:, :, :unsplit])
    assert np.array_equal(got[:, :, unsplit:], split[:, :, unsplit:])
    for r in range(R):
        ref = oracle_attention(q[r].transpose(1, 0, 2).astype(np.float64), keys[r].astype(np.float64),
                               vals[r].astype(np.float64))
        check_close(got[r], ref, "bf16", f"attention plan row {r}", stored_bf16=True)


def test_attention_plan_full_video_shape(lib):
    """The 1.3B-shaped video self-attention as the stream launches it: 12
    heads, 2 rows of 3120 queries, 1560 sink + wrapped 9360 window + 3120 own
    keys, with the plan the stream picks (10 heads whole, 2 split 5 ways).
    Every head bit for bit its unsplit or split result; sampled queries of a
    whole and a split head against the oracle."""
    print("attention plan full video shape", flush=True)
    rng = np.random.default_rng(12)
    H, R, hd, L, S, W = 12, 2, 128, 3120, 1560, 9360
    ns, hf = C.c_int32(), C.c_int32()
    call(lib.sd_k_attention_pick_plan(H, R * ((L + 127) // 128), (S + W + L + 63) // 64, 8, 512, C.byref(ns),
                                      C.byref(hf)))
    nsplit, unsplit = ns.value, hf.value
    print(f"  plan: {unsplit} heads whole, the rest split {nsplit} ways", flush=True)
    assert 0 < unsplit < H and nsplit > 1
    dev, segs, keys, vals = make_segments(rng, H, hd, R, L, S, S, W, 3120, W, torch.bfloat16)
    q = bf16_round(rng.standard_normal((R, H, L, hd)).astype(np.float32))
    qd = to_dev(q, torch.bfloat16)
    o = torch.empty((R * L, H * hd), dtype=torch.bfloat16, device=device())
    got = _attn_call(lib, lib.sd_k_attention_plan, qd, o, R, H, L, hd, segs, nsplit, (unsplit,))
    whole = _attn_call(lib, lib.sd_k_attention, qd, o, R, H, L, hd, segs, 1)
    assert np.array_equal(got[:, :, :unsplit], whole[:, :, :unsplit])
    del whole
    split = _attn_call(lib, lib.sd_k_attention, qd, o, R, H, L, hd, segs, nsplit)
    assert np.array_equal(got[:, :, unsplit:], split[:, :, unsplit:])
    del split
    sample = np.concatenate([np.arange(0, 3), rng.integers(0, L, 20), np.arange(L - 3, L)])
    for r in range(R):
        for h in (0, unsplit - 1, unsplit, H - 1):
            qh = q[r, h][sample].astype(np.float64)[:, None, :]
            ref = oracle_attention(qh, keys[r][:, h:h + 1].astype(np.float64), vals[r][:, h:h + 1].astype(np.float64))
            check_close(got[r][sample][:, h:h + 1], ref, "bf16", f"row {r} head {h}", stored_bf16=True)


# ------------------------------------------------------------------ SSF / motion reductions
def test_ssf_sums_bit_exact_u8(lib):
    cfg = get_config("tiny")
    src = gen.SSFFrameSource(cfg)
    frames = [src.next() for _ in range(4)]
    out = torch.zeros(3, dtype=torch.int64, device=device())
    for a, b in [(frames[0], frames[1]), (frames[2], frames[3]), (frames[0], frames[0])]:
        da, db = to_dev(a, torch.uint8), to_dev(b, torch.uint8)
        call(lib.sd_k_ssf_sums(0, da.data_ptr(), db.data_ptr(), a.size, out.data_ptr(), stream_ptr()))
        torch.cuda.synchronize()
        assert tuple(out.cpu().tolist()) == controls.ssf_sums(a, b)


def test_ssf_sums_bit_exact_latent(lib):
    rng = np.random.default_rng(3)
    a = rng.standard_normal((4, 64, 64)).astype(np.float32)
    b = (a + 0.3 * rng.standard_normal(a.shape)).astype(np.float32)
    b[0, 0, :4] = [1e6, -1e6, 2 ** -13, 3 * 2 ** -13]          # clamping and ties
    out = torch.zeros(3, dtype=torch.int64, device=device())
    da, db = to_dev(a, torch.float32), to_dev(b, torch.float32)      # keep both alive during the call
    call(lib.sd_k_ssf_sums(1, da.data_ptr(), db.data_ptr(), a.size, out.data_ptr(), stream_ptr()))
    torch.cuda.synchronize()
    assert tuple(out.cpu().tolist()) == controls.ssf_sums(controls.quantise_latent(a), controls.quantise_latent(b))


def test_motion_sums_bit_exact(lib):
    cfg = get_config("video13b")
    src = gen.LatentSource(cfg)
    c0, c1 = src.next(), src.next()
    n = c0[0].size
    out = torch.zeros(2, dtype=torch.int64, device=device())
    prev = to_dev(c0[1], torch.float32)
    cur = to_dev(c1, torch.float32)
    call(lib.sd_k_motion_sums(cur.data_ptr(), prev.data_ptr(), 2, n, out.data_ptr(), stream_ptr()))
    torch.cuda.synchronize()
    q = [controls.quantise_latent(x) for x in (c0[1], c1[0], c1[1])]
    assert out.cpu().tolist() == [controls.motion_sumsq(q[0], q[1]), controls.motion_sumsq(q[1], q[2])]
    call(lib.sd_k_motion_sums(cur.data_ptr(), None, 2, n, out.data_ptr(), stream_ptr()))
    torch.cuda.synchronize()
    assert out.cpu().tolist() == [0, controls.motion_sumsq(q[1], q[2])]
