"""GPU parity of the fused GEMM epilogues at the shapes and launch
configurations the 1.3B-shaped video step runs (two rows of 3120 tokens,
d 1536, 12 heads of 128, FFN 8960, 64-wide patches), through sd_k_gemm_epi
and sd_k_ln_mod.

Operands are k/16 with |k| <= 8, exact in bf16, so every accumulator is exact
in fp32.  Epilogues that only add, scatter or multiply exact values are then
compared bit for bit (with the oracle's own layouts: patchify / unpatchify,
per-head q / k, transposed v); RoPE and GELU are compared with the oracle's
fp64 rope_apply / gelu on the exact accumulators, within the bf16 rounding of
the stored result plus a bound on the fp32 arithmetic written in each test."""
import ctypes as C

import numpy as np
import pytest
import torch

import streaming_diffusion_amd._lib as sdlib
from oracle import dit

from gpu_helpers import bf16_round, call, device, stream_ptr, to_dev

pytestmark = pytest.mark.gpu

# the 1.3B-shaped video DiT, two rows (n = 2) of one T = 2 chunk
R, T, Hp, Wp = 2, 2, 30, 52
L = T * Hp * Wp                     # 3120 tokens
D, H, HD, F = 1536, 12, 128, 8960
PC, P, CH = 64, 2, 16               # patch vector 2*2*16
ROPE_POS = 1025                     # temporal positions of the table (reset threshold 1024)


@pytest.fixture(scope="module")
def lib():
    device()
    return sdlib.load()


def int_operands(M, N, K, seed):
    rng = np.random.default_rng(seed)
    ai = rng.integers(-8, 9, size=(M, K))
    wi = rng.integers(-8, 9, size=(N, K))
    bi = rng.integers(-8, 9, size=N)
    acc = (ai.astype(np.float64) @ wi.T.astype(np.float64)) / 256.0 + bi / 16.0     # exact
    A, W, b = to_dev(ai / 16.0, torch.bfloat16), to_dev(wi / 16.0, torch.bfloat16), to_dev(bi / 16.0, torch.bfloat16)
    return A, W, b, acc


def run(lib, A, W, M, N, K, e):
    call(lib.sd_k_gemm_epi(A.data_ptr(), W.data_ptr(), M, N, K, C.byref(e), stream_ptr()))
    torch.cuda.synchronize()


def rope_table(lib, hd, positions, hp, wp):
    n = lib.sd_k_rope_table_pairs(hd, positions, hp, wp)
    buf = np.zeros(2 * n, np.float32)
    call(lib.sd_k_rope_tables(hd, positions, hp, wp, 10000.0, buf.ctypes.data))
    return to_dev(buf, torch.float32)


# ------------------------------------------------------------------ q / k / v scatter with RoPE
def qkv_case(lib, rows, t, hp, wp, d, h, rope, t0s, kextra=0, seed=1):
    hd = d // h
    Lr = t * hp * wp
    M, N, K = rows * Lr, 3 * d, d
    print(f"qkv M={M} N={N} K={K} rope={rope} t0={t0s}", flush=True)
    A, W, b, acc = int_operands(M, N, K, seed)
    kstride, krows = Lr + kextra, rows + (1 if kextra else 0)
    q = torch.zeros((rows, h, Lr, hd), dtype=torch.bfloat16, device=device())
    k = torch.zeros((h, krows, kstride, hd), dtype=torch.bfloat16, device=device())
    vt = torch.zeros((h, hd, krows, kstride), dtype=torch.bfloat16, device=device())
    e = sdlib.sd_gemm_epi(mode=sdlib.SD_EPI_QKV, bias=b.data_ptr(), L=Lr, q=q.data_ptr(), k=k.data_ptr(),
                          vt=vt.data_ptr(), kstride=kstride, krows=krows, H=h, hd=hd, rope=int(rope), Hp=hp, Wp=wp)
    tab = None
    if rope:
        tab = rope_table(lib, hd, ROPE_POS, hp, wp)
        e.rope_table, e.rope_positions = tab.data_ptr(), ROPE_POS
        for r, v in enumerate(t0s):
            e.t0[r] = v
    run(lib, A, W, M, N, K, e)
    qg, kg, vg = q.float().cpu().numpy(), k.float().cpu().numpy(), vt.float().cpu().numpy()
    for r in range(rows):
        c = acc[r * Lr:(r + 1) * Lr].reshape(Lr, 3, h, hd)
        v_ref = c[:, 2]
        # v is stored unrotated: bit for bit the bf16 rounding of the exact value
        assert np.array_equal(vg[:, :, r, :Lr].transpose(2, 0, 1), bf16_round(v_ref)), f"v row {r}"
        for sec, got in ((0, qg[r].transpose(1, 0, 2)), (1, kg[:, r, :Lr].transpose(1, 0, 2))):
            x = c[:, sec]
            if not rope:
                assert np.array_equal(got, bf16_round(x)), f"section {sec} row {r}"
                continue
            ref = dit.rope_apply(x, dit.token_positions(t, hp, wp, t0s[r]))
            # pair magnitude |x0| + |x1| bounds the fp32 table and arithmetic error
            pair = np.abs(x[..., 0::2]) + np.abs(x[..., 1::2])
            pair = np.repeat(pair, 2, axis=-1)
            err = np.abs(got - ref) - 2.0 ** -8 * np.abs(ref) - 1e-6 * pair
            assert err.max() <= 0.0, f"section {sec} row {r}: excess {err.max():.3e}"
    if kextra:   # capacity beyond the rows / tokens written stays untouched
        assert not k[:, rows:].any() and not k[:, :, Lr:].any() and not vt[:, :, rows:].any()


def test_qkv_scatter_video13b_exact(lib):
    qkv_case(lib, R, T, Hp, Wp, D, H, rope=False, t0s=[0, 0])


def test_qkv_rope_video13b(lib):
    # second row's chunk ends on the last temporal position before the reset
    qkv_case(lib, R, T, Hp, Wp, D, H, rope=True, t0s=[6, 1023])


def test_qkv_rope_small_head_dims_and_strided_destination(lib):
    # hd 64 and 32 (RoPE sections 24/20/20 and 12/10/10), ragged tiles, a k / v^T capacity beyond the rows
    qkv_case(lib, 3, 1, 8, 10, 256, 4, rope=True, t0s=[0, 5, 17], kextra=16, seed=2)
    qkv_case(lib, 2, 2, 4, 6, 128, 4, rope=True, t0s=[1, 1000], kextra=8, seed=3)


def test_qkv_rope_ragged_160_row_tiles(lib):
    """1872-token rows: 3744 rows take 160-row tiles (2 rounds of 24 x 18
    tiles against 2 of 15 x 18 256-row tiles) and end in a tile of 64 rows."""
    qkv_case(lib, R, T, 24, 39, D, H, True, [0, 7])


def test_qkv_scatter_video14b_width_exact(lib):
    # d 5120, 40 heads, one row
    qkv_case(lib, 1, T, Hp, Wp, 5120, 40, rope=False, t0s=[0], seed=4)


# ------------------------------------------------------------------ FFN first layer with GELU
@pytest.mark.parametrize("M,N,K", [(R * L, F, D), (6100, F, D), (1000, 520, 256)])
def test_gelu_epilogue(lib, M, N, K):
    """224-row tiles (128 + 96 rows per wave row) at 6240 and 6100 rows (the
    latter ends in a tile of 52 rows); 128 x 128 tiles for the small case."""
    print(f"gelu M={M} N={N} K={K}", flush=True)
    A, W, b, acc = int_operands(M, N, K, 5)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=device())
    e = sdlib.sd_gemm_epi(mode=sdlib.SD_EPI_GELU, bias=b.data_ptr(), out=out.data_ptr(), ldo=N)
    run(lib, A, W, M, N, K, e)
    got = out.float().cpu().numpy()
    ref = dit.gelu(acc)
    # bf16 rounding of the stored value; the erf approximation (|error| <=
    # 1.5e-7) and the fp32 reciprocal / exponential add at most 2e-6 |v|
    err = np.abs(got - ref) - 2.0 ** -8 * np.abs(ref) - 2e-6 * np.abs(acc) - 1e-7
    assert err.max() <= 0.0, f"excess {err.max():.3e}"


# ------------------------------------------------------------------ gated residual (attention out, FFN out)
@pytest.mark.parametrize("M,N,K", [(R * L, D, D), (R * L, D, F), (6100, D, D), (6020, D, 960), (700, 136, 320)])
def test_gate_resid_epilogue_exact(lib, M, N, K):
    """resid += (mod[r][5d + n] + blk[5d + n]) * (A W^T + b)[m][n], r = m / L.
    Gates are multiples of 1/2 and the residual a multiple of 1/256: every
    product and sum is exact in fp32.  N = 1536 takes 160-row tiles (96 + 64
    rows per wave row); 6100 and 6020 rows end in a tile of 20 and 100 rows."""
    print(f"gate resid M={M} N={N} K={K}", flush=True)
    Lr = L if M % L == 0 else 100
    rows = M // Lr + (M % Lr > 0)
    A, W, b, acc = int_operands(M, N, K, 6)
    rng = np.random.default_rng(7)
    six_d = 6 * N
    off = 5 * N
    mod = rng.integers(-2, 3, size=(rows, six_d)) / 2.0
    blk = rng.integers(-1, 2, size=six_d) / 2.0
    c0 = rng.integers(-4096, 4097, size=(M, N)) / 256.0
    resid = to_dev(c0, torch.float32)
    mod_d, blk_d = to_dev(mod, torch.float32), to_dev(blk, torch.bfloat16)
    e = sdlib.sd_gemm_epi(mode=sdlib.SD_EPI_GATE_RESID, bias=b.data_ptr(), resid=resid.data_ptr(),
                          mod=mod_d.data_ptr(), blk=blk_d.data_ptr(), gate_off=off, six_d=six_d, L=Lr)
    run(lib, A, W, M, N, K, e)
    gate = mod[np.arange(M) // Lr, off:off + N] + blk[off:off + N]
    assert np.array_equal(resid.cpu().numpy().astype(np.float64), c0 + gate * acc)


# ------------------------------------------------------------------ patch embedding and head
def test_patch_embedding_epilogue_exact(lib):
    """The patch embedding of the video rows: K = 64 (a single 64-deep k-tile)
    writes the fp32 residual stream."""
    M, N, K = R * L, D, PC
    A, W, b, acc = int_operands(M, N, K, 8)
    resid = torch.full((M, N), 7.0, dtype=torch.float32, device=device())
    e = sdlib.sd_gemm_epi(mode=sdlib.SD_EPI_PATCH, bias=b.data_ptr(), resid=resid.data_ptr())
    run(lib, A, W, M, N, K, e)
    assert np.array_equal(resid.cpu().numpy().astype(np.float64), acc)


@pytest.mark.parametrize("rows,t,hp,wp,ch", [(R, T, Hp, Wp, CH), (3, 1, 8, 8, 4)])
def test_head_epilogue_unpatchifies_exactly(lib, rows, t, hp, wp, ch):
    Lr = t * hp * wp
    M, N, K = rows * Lr, P * P * ch, 256
    A, W, b, acc = int_operands(M, N, K, 9)
    eps = torch.zeros((rows, t, ch, hp * P, wp * P), dtype=torch.float32, device=device())
    e = sdlib.sd_gemm_epi(mode=sdlib.SD_EPI_HEAD, bias=b.data_ptr(), eps=eps.data_ptr(), L=Lr, C=ch, Hl=hp * P,
                          Wl=wp * P, p=P, T=t, Hp=hp, Wp=wp)
    run(lib, A, W, M, N, K, e)
    got = eps.cpu().numpy().astype(np.float64)
    for r in range(rows):
        ref = dit.unpatchify(acc[r * Lr:(r + 1) * Lr], t, ch, hp * P, wp * P, P)
        assert np.array_equal(got[r], ref), f"row {r}"


# ------------------------------------------------------------------ LayerNorm + adaLN modulation
@pytest.mark.parametrize("M,d,Lr", [(R * L, D, L), (L, 5120, L), (2048, 1024, 1024), (37, 128, 10), (128, D, 128),
                                    (300, 768, 100), (1024, 1024, 512), (3000, 2048, 1500), (2100, 1280, 700)])
def test_ln_mod_against_oracle(lib, M, d, Lr):
    """bf16 output of LN(x) * (1 + scale) + shift, scale / shift = the row's
    modulation slots plus the block table (the attention slots 0 and 1 of
    6d); register-resident rows of 4 (d <= 1024), 6 (1280, 1536), 8 (2048)
    and 20 (5120) vectors per lane, and up to 1024 rows of width 768 - 2048 a
    workgroup per row.  Bound: the stored bf16 rounding plus 1e-4 of the RMS."""
    print(f"ln_mod M={M} d={d}", flush=True)
    rng = np.random.default_rng(d + M)
    rows = (M + Lr - 1) // Lr
    x = rng.standard_normal((M, d)).astype(np.float32) * 3 + 0.5
    mod = (0.3 * rng.standard_normal((rows, 6 * d))).astype(np.float32)
    blk = bf16_round(0.02 * rng.standard_normal(6 * d))
    out = torch.empty((M, d), dtype=torch.bfloat16, device=device())
    xd, md, bd = to_dev(x, torch.float32), to_dev(mod, torch.float32), to_dev(blk, torch.bfloat16)
    call(lib.sd_k_ln_mod(sdlib.SD_DTYPE_BF16, xd.data_ptr(), out.data_ptr(), M, d, Lr, md.data_ptr(), bd.data_ptr(),
                         0, d, 6 * d, sdlib.SD_LN_PLAIN, stream_ptr()))
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    m = mod.astype(np.float64)[np.arange(M) // Lr] + blk.astype(np.float64)
    ref = dit.modulate(dit.layer_norm(x.astype(np.float64)), m[:, :d], m[:, d:2 * d])
    rms = np.sqrt(np.mean(ref * ref))
    excess = np.max(np.abs(got - ref) - 2.0 ** -8 * np.abs(ref)) / rms
    assert excess <= 1e-4, f"excess {excess:.3e}"


@pytest.mark.parametrize("M,d,Lr", [(R * L, D, L), (L, 5120, L), (128, D, 128), (256, 1024, 128)])
def test_ln_split_and_fp16_forms(lib, M, d, Lr):
    """The head's input as hi + lo bf16 pairs (SD_LN_SPLIT, with the final
    layer's (shift, scale) slots of a 2d vector) reconstructs the modulated
    LayerNorm to fp32 accuracy; the cross-attention's fp16 input (SD_LN_F16,
    no modulation) is within fp16 rounding (2^-11 relative)."""
    print(f"ln split / f16 M={M} d={d}", flush=True)
    rng = np.random.default_rng(d + 3 * M)
    x = rng.standard_normal((M, d)).astype(np.float32) * 2 - 0.3
    mod = (0.3 * rng.standard_normal((M // Lr, 2 * d))).astype(np.float32)
    xd, md = to_dev(x, torch.float32), to_dev(mod, torch.float32)
    ln = dit.layer_norm(x.astype(np.float64))
    split = torch.empty((M, 2 * d), dtype=torch.bfloat16, device=device())
    call(lib.sd_k_ln_mod(sdlib.SD_DTYPE_BF16, xd.data_ptr(), split.data_ptr(), M, d, Lr, md.data_ptr(), None, 0, d,
                         2 * d, sdlib.SD_LN_SPLIT, stream_ptr()))
    half = torch.empty((M, d), dtype=torch.float16, device=device())
    call(lib.sd_k_ln_mod(sdlib.SD_DTYPE_BF16, xd.data_ptr(), half.data_ptr(), M, d, Lr, None, None, 0, 0, 0,
                         sdlib.SD_LN_F16, stream_ptr()))
    torch.cuda.synchronize()
    m = mod.astype(np.float64)[np.arange(M) // Lr]
    ref = dit.modulate(ln, m[:, :d], m[:, d:])
    sp = split.float().cpu().numpy()
    hi, lo = sp[:, :d].astype(np.float64), sp[:, d:].astype(np.float64)
    # hi alone is the bf16 value (within its rounding of the reference)
    assert np.all(np.abs(hi - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5 * np.sqrt(np.mean(ref * ref)))
    rms = np.sqrt(np.mean(ref * ref))
    e_split = np.max(np.abs(hi + lo - ref) - 2.0 ** -16 * np.abs(ref)) / rms
    assert e_split <= 1e-5, f"split excess {e_split:.3e}"
    h = half.float().cpu().numpy()
    e_half = np.max(np.abs(h - ln) - 2.0 ** -11 * np.abs(ln)) / np.sqrt(np.mean(ln * ln))
    assert e_half <= 1e-5, f"fp16 excess {e_half:.3e}"


@pytest.mark.parametrize("M,N,K,mode", [(R * L, 960, D, "f32"), (R * L, D, 960, "resid"), (L, 3200, 5120, "f32"),
                                        (L, 5120, 3200, "resid"), (300, 200, 136, "resid")])
def test_fp16_gemm_exact_integers(lib, M, N, K, mode):
    """The folded cross-attention's fp16 GEMMs (scores: N = heads x 80
    prompt slots; output: K = heads x 80): k/16 operands are exact in fp16 as
    in bf16, so the result is the integer arithmetic bit for bit."""
    print(f"fp16 gemm {mode} M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(M + N + K)
    ai = rng.integers(-8, 9, size=(M, K))
    wi = rng.integers(-8, 9, size=(N, K))
    bi = rng.integers(-8, 9, size=N)
    A, W = to_dev(ai / 16.0, torch.float16), to_dev(wi / 16.0, torch.float16)
    b = to_dev(bi / 16.0, torch.bfloat16)
    ref = (ai.astype(np.float64) @ wi.T.astype(np.float64)) / 256.0 + bi / 16.0
    if mode == "f32":
        out = torch.empty((M, N), dtype=torch.float32, device=device())
        e = sdlib.sd_gemm_epi(mode=sdlib.SD_EPI_F32, bias=b.data_ptr(), out=out.data_ptr(), ldo=N, f16=1)
    else:
        c0 = rng.integers(-4096, 4097, size=(M, N)) / 256.0
        out = to_dev(c0, torch.float32)
        e = sdlib.sd_gemm_epi(mode=sdlib.SD_EPI_RESID, bias=b.data_ptr(), resid=out.data_ptr(), f16=1)
        ref = ref + c0
    run(lib, A, W, M, N, K, e)
    assert np.array_equal(out.cpu().numpy().astype(np.float64), ref)


# ------------------------------------------------------------------ few rows: the product split over K
def split_ws(nbytes=64 << 20):
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device())
    return ws, (ws.data_ptr() + 255) // 256 * 256, nbytes


@pytest.mark.parametrize("M,N,K", [(128, 4608, 1536), (256, 8960, 1536), (128, 1536, 8960), (256, 1536, 1536),
                                   (96, 200, 640), (2048, 768, 3072), (2048, 768, 768), (1000, 760, 1536)])
def test_split_k_epilogues_exact(lib, M, N, K):
    """Below the knee (M <= 256 rows: the sub-knee video diagnostic's 128 or
    256 tokens per forward; and up to 2048 rows when 128 x 128 tiles would
    leave most CUs idle, the image DiT's N = 768 GEMMs) the product is split
    over K into fp32 partials
    that a second pass sums in slice order before the epilogue; on exact
    operands the sums are exact, so F32 (also into rows not 16-byte
    aligned), RESID and the gated residual are bit for bit the integer
    arithmetic, STORE the bf16 rounding of it, and GELU within the bound of
    the full-size GELU test."""
    print(f"split-K M={M} N={N} K={K}", flush=True)
    A, W, b, acc = int_operands(M, N, K, 21)
    ws, wsp, wsb = split_ws()
    out = torch.empty((M, N), dtype=torch.float32, device=device())
    e = sdlib.sd_gemm_epi(mode=sdlib.SD_EPI_F32, bias=b.data_ptr(), out=out.data_ptr(), ldo=N, workspace=wsp,
                          workspace_bytes=wsb)
    run(lib, A, W, M, N, K, e)
    assert np.array_equal(out.cpu().numpy().astype(np.float64), acc)
    rng = np.random.default_rng(22)
    c0 = rng.integers(-4096, 4097, size=(M, N)) / 256.0
    Lr = M // 2 if M % 2 == 0 else M
    rows = M // Lr
    mod = rng.integers(-2, 3, size=(rows, 6 * N)) / 2.0
    blk = rng.integers(-1, 2, size=6 * N) / 2.0
    resid = to_dev(c0, torch.float32)
    mod_d, blk_d = to_dev(mod, torch.float32), to_dev(blk, torch.bfloat16)
    e = sdlib.sd_gemm_epi(mode=sdlib.SD_EPI_GATE_RESID, bias=b.data_ptr(), resid=resid.data_ptr(),
                          mod=mod_d.data_ptr(), blk=blk_d.data_ptr(), gate_off=2 * N, six_d=6 * N, L=Lr,
                          workspace=wsp, workspace_bytes=wsb)
    run(lib, A, W, M, N, K, e)
    gate = mod[np.arange(M) // Lr, 2 * N:3 * N] + blk[2 * N:3 * N]
    assert np.array_equal(resid.cpu().numpy().astype(np.float64), c0 + gate * acc)
    st = torch.empty((M, N), dtype=torch.bfloat16, device=device())
    e = sdlib.sd_gemm_epi(mode=sdlib.SD_EPI_STORE, bias=b.data_ptr(), out=st.data_ptr(), ldo=N, workspace=wsp,
                          workspace_bytes=wsb)
    run(lib, A, W, M, N, K, e)
    assert np.array_equal(st.float().cpu().numpy(), bf16_round(acc.astype(np.float32)))
    # the plain residual: resid += A W^T + b, exact
    resid = to_dev(c0, torch.float32)
    e = sdlib.sd_gemm_epi(mode=sdlib.SD_EPI_RESID, bias=b.data_ptr(), resid=resid.data_ptr(), workspace=wsp,
                          workspace_bytes=wsb)
    run(lib, A, W, M, N, K, e)
    assert np.array_equal(resid.cpu().numpy().astype(np.float64), c0 + acc)
    # GELU against the oracle's exact-erf GELU (bound as in test_gelu_epilogue)
    e = sdlib.sd_gemm_epi(mode=sdlib.SD_EPI_GELU, bias=b.data_ptr(), out=st.data_ptr(), ldo=N, workspace=wsp,
                          workspace_bytes=wsb)
    run(lib, A, W, M, N, K, e)
    ref = dit.gelu(acc)
    err = np.abs(st.float().cpu().numpy() - ref) - 2.0 ** -8 * np.abs(ref) - 2e-6 * np.abs(acc) - 1e-7
    assert err.max() <= 0.0, f"gelu excess {err.max():.3e}"
    # output rows two elements longer than N (not 16-byte aligned): element stores
    ld = N + 2
    wide = torch.full((M, ld), -1.0, dtype=torch.float32, device=device())
    e = sdlib.sd_gemm_epi(mode=sdlib.SD_EPI_F32, bias=b.data_ptr(), out=wide.data_ptr(), ldo=ld, workspace=wsp,
                          workspace_bytes=wsb)
    run(lib, A, W, M, N, K, e)
    wg = wide.cpu().numpy().astype(np.float64)
    assert np.array_equal(wg[:, :N], acc) and np.all(wg[:, N:] == -1.0)


def packed_copy(lib, W, N, K):
    n = lib.sd_k_pack_weight_bytes(N, K)
    assert n > 0
    buf = torch.empty(n // 2, dtype=W.dtype, device=device())
    call(lib.sd_k_pack_weight(W.data_ptr(), N, K, buf.data_ptr(), stream_ptr()))
    torch.cuda.synchronize()
    return buf


def test_pack_weight_layout(lib):
    """sd_k_pack_weight against its definition: chunk (nb, kt, kk, lane) is
    W[32 nb + lane % 32][64 kt + 16 kk + 8 (lane / 32) .. + 7], rows past N
    zero (N = 200 pads to 224)."""
    N, K = 200, 192
    rng = np.random.default_rng(31)
    wi = rng.integers(-200, 201, size=(N, K)).astype(np.float64)     # exact in bf16
    got = packed_copy(lib, to_dev(wi, torch.bfloat16), N, K).float().cpu().numpy().astype(np.float64)
    NB, KT = (N + 31) // 32, K // 64
    wp = np.zeros((NB * 32, K))
    wp[:N] = wi
    ref = wp.reshape(NB, 32, KT, 4, 2, 8).transpose(0, 2, 3, 4, 1, 5).reshape(-1)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("M,N,K", [(128, 4608, 1536), (128, 8960, 1536), (128, 1536, 8960), (256, 1536, 1536),
                                   (96, 200, 640)])
def test_split_k_packed_weights_exact(lib, M, N, K):
    """The few-row product reading W from its fragment-ordered copy (what the
    stream uses when every forward has at most 256 tokens): bit for bit the
    integer arithmetic, as with W read in place."""
    print(f"split-K packed M={M} N={N} K={K}", flush=True)
    A, W, b, acc = int_operands(M, N, K, 23)
    wp = packed_copy(lib, W, N, K)
    ws, wsp, wsb = split_ws()
    out = torch.empty((M, N), dtype=torch.float32, device=device())
    e = sdlib.sd_gemm_epi(mode=sdlib.SD_EPI_F32, bias=b.data_ptr(), out=out.data_ptr(), ldo=N, workspace=wsp,
                          workspace_bytes=wsb, wpack=wp.data_ptr())
    run(lib, A, W, M, N, K, e)
    assert np.array_equal(out.cpu().numpy().astype(np.float64), acc)
    rng = np.random.default_rng(24)
    c0 = rng.integers(-4096, 4097, size=(M, N)) / 256.0
    Lr = M // 2 if M % 2 == 0 else M
    mod = rng.integers(-2, 3, size=(M // Lr, 6 * N)) / 2.0
    blk = rng.integers(-1, 2, size=6 * N) / 2.0
    resid = to_dev(c0, torch.float32)
    mod_d, blk_d = to_dev(mod, torch.float32), to_dev(blk, torch.bfloat16)
    e = sdlib.sd_gemm_epi(mode=sdlib.SD_EPI_GATE_RESID, bias=b.data_ptr(), resid=resid.data_ptr(),
                          mod=mod_d.data_ptr(), blk=blk_d.data_ptr(), gate_off=5 * N, six_d=6 * N, L=Lr,
                          workspace=wsp, workspace_bytes=wsb, wpack=wp.data_ptr())
    run(lib, A, W, M, N, K, e)
    gate = mod[np.arange(M) // Lr, 5 * N:6 * N] + blk[5 * N:6 * N]
    assert np.array_equal(resid.cpu().numpy().astype(np.float64), c0 + gate * acc)


def test_split_k_qkv_rope_and_fp16(lib):
    """The q / k / v scatter with RoPE and the fp16 cross-attention products on
    the split path (one latent frame of 8 x 16 tokens per row, two rows)."""
    ws, wsp, wsb = split_ws()
    rows, t, hp, wp_, d, h = 2, 1, 8, 16, 1536, 12
    hd, Lr = d // h, t * hp * wp_
    M, N, K = rows * Lr, 3 * d, d
    A, W, b, acc = int_operands(M, N, K, 23)
    q = torch.zeros((rows, h, Lr, hd), dtype=torch.bfloat16, device=device())
    k = torch.zeros((h, rows, Lr, hd), dtype=torch.bfloat16, device=device())
    vt = torch.zeros((h, hd, rows, Lr), dtype=torch.bfloat16, device=device())
    tab = rope_table(lib, hd, ROPE_POS, hp, wp_)
    e = sdlib.sd_gemm_epi(mode=sdlib.SD_EPI_QKV, bias=b.data_ptr(), L=Lr, q=q.data_ptr(), k=k.data_ptr(),
                          vt=vt.data_ptr(), kstride=Lr, krows=rows, H=h, hd=hd, rope=1, Hp=hp, Wp=wp_,
                          rope_table=tab.data_ptr(), rope_positions=ROPE_POS, workspace=wsp, workspace_bytes=wsb)
    e.t0[0], e.t0[1] = 3, 1020
    run(lib, A, W, M, N, K, e)
    qg, kg, vg = q.float().cpu().numpy(), k.float().cpu().numpy(), vt.float().cpu().numpy()
    for r, t0 in enumerate((3, 1020)):
        c = acc[r * Lr:(r + 1) * Lr].reshape(Lr, 3, h, hd)
        assert np.array_equal(vg[:, :, r].transpose(2, 0, 1), bf16_round(c[:, 2]))
        for sec, got in ((0, qg[r].transpose(1, 0, 2)), (1, kg[:, r].transpose(1, 0, 2))):
            x = c[:, sec]
            ref = dit.rope_apply(x, dit.token_positions(t, hp, wp_, t0))
            pair = np.repeat(np.abs(x[..., 0::2]) + np.abs(x[..., 1::2]), 2, axis=-1)
            assert (np.abs(got - ref) - 2.0 ** -8 * np.abs(ref) - 1e-6 * pair).max() <= 0.0
    # fp16 operands (the folded cross-attention) on the split path
    rng = np.random.default_rng(24)
    M2, N2, K2 = 128, 960, 1536
    ai, wi = rng.integers(-8, 9, size=(M2, K2)), rng.integers(-8, 9, size=(N2, K2))
    out = torch.empty((M2, N2), dtype=torch.float32, device=device())
    e = sdlib.sd_gemm_epi(mode=sdlib.SD_EPI_F32, out=out.data_ptr(), ldo=N2, f16=1, workspace=wsp,
                          workspace_bytes=wsb)
    A2, W2 = to_dev(ai / 16.0, torch.float16), to_dev(wi / 16.0, torch.float16)
    call(lib.sd_k_gemm_epi(A2.data_ptr(), W2.data_ptr(), M2, N2, K2, C.byref(e), stream_ptr()))
    torch.cuda.synchronize()
    ref2 = (ai.astype(np.float64) @ wi.T) / 256.0
    assert np.array_equal(out.cpu().numpy().astype(np.float64), ref2)
    # the same from fragment-ordered copies of W (fp16, and the q / k / v product)
    out.zero_()
    wp2 = packed_copy(lib, W2, N2, K2)
    e.wpack = wp2.data_ptr()
    call(lib.sd_k_gemm_epi(A2.data_ptr(), W2.data_ptr(), M2, N2, K2, C.byref(e), stream_ptr()))
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), ref2)
    q2, k2, vt2 = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(vt)
    wp = packed_copy(lib, W, N, K)
    e = sdlib.sd_gemm_epi(mode=sdlib.SD_EPI_QKV, bias=b.data_ptr(), L=Lr, q=q2.data_ptr(), k=k2.data_ptr(),
                          vt=vt2.data_ptr(), kstride=Lr, krows=rows, H=h, hd=hd, rope=1, Hp=hp, Wp=wp_,
                          rope_table=tab.data_ptr(), rope_positions=ROPE_POS, workspace=wsp, workspace_bytes=wsb,
                          wpack=wp.data_ptr())
    e.t0[0], e.t0[1] = 3, 1020
    run(lib, A, W, M, N, K, e)
    assert torch.equal(q2, q) and torch.equal(k2, k) and torch.equal(vt2, vt)


@pytest.mark.parametrize("M,N,K,mode,form,with_blk", [
    (128, 1536, 8960, "gate", sdlib.SD_LN_PLAIN, True),    # FFN2 -> next block's attention LayerNorm
    (256, 1536, 1536, "gate", sdlib.SD_LN_SPLIT, False),   # last FFN2 -> the head's hi / lo input
    (128, 1536, 1536, "gate", sdlib.SD_LN_F16, False),     # O-projection -> cross-attention input
    (128, 1536, 960, "resid", sdlib.SD_LN_PLAIN, True),    # cross-attention out -> feed-forward LayerNorm
    (100, 1024, 1536, "resid", sdlib.SD_LN_PLAIN, True),   # ragged rows
    (128, 520, 640, "gate", sdlib.SD_LN_PLAIN, True),      # width not a multiple of 256: a separate pass
    (128, 1536, 960, "resid16", sdlib.SD_LN_PLAIN, True),  # fp16 operands (the folded cross-attention out)
])
def test_residual_gemm_with_layernorm(lib, M, N, K, mode, form, with_blk):
    """A residual GEMM that also writes the LayerNorm of the updated rows
    (sd_gemm_epi.ln_out; on the few-row path the reduction pass does both in
    one launch) gives bit for bit the residual and the LayerNorm output of
    the GEMM followed by sd_k_ln_mod."""
    print(f"gemm + LN M={M} N={N} K={K} {mode} form={form}", flush=True)
    rng = np.random.default_rng(M + N + K)
    f16 = mode == "resid16"
    A = to_dev(rng.standard_normal((M, K)), torch.float16 if f16 else torch.bfloat16)
    W = to_dev(0.02 * rng.standard_normal((N, K)), torch.float16 if f16 else torch.bfloat16)
    b = to_dev(0.1 * rng.standard_normal(N), torch.bfloat16)
    Lr = M // 2 if M % 2 == 0 else M
    rows = M // Lr
    c0 = (3 * rng.standard_normal((M, N)) + 0.5).astype(np.float32)
    gmod = to_dev(0.3 * rng.standard_normal((rows, 6 * N)), torch.float32)
    gblk = to_dev(0.02 * rng.standard_normal(6 * N), torch.bfloat16)
    lmod = to_dev(0.3 * rng.standard_normal((rows, 6 * N)), torch.float32) if form != sdlib.SD_LN_F16 else None
    lblk = to_dev(0.02 * rng.standard_normal(6 * N), torch.bfloat16) if with_blk else None
    ws, wsp, wsb = split_ws()
    width = 2 * N if form == sdlib.SD_LN_SPLIT else N
    odt = torch.float16 if form == sdlib.SD_LN_F16 else torch.bfloat16

    def epi(resid, ln_out):
        e = sdlib.sd_gemm_epi(mode=sdlib.SD_EPI_GATE_RESID if mode == "gate" else sdlib.SD_EPI_RESID,
                              bias=b.data_ptr(), resid=resid.data_ptr(), L=Lr, workspace=wsp, workspace_bytes=wsb,
                              f16=int(f16))
        if mode == "gate":
            e.mod, e.blk, e.gate_off, e.six_d = gmod.data_ptr(), gblk.data_ptr(), 5 * N, 6 * N
        if ln_out is not None:
            e.ln_out, e.ln_form = ln_out.data_ptr(), form
            if lmod is not None:
                e.ln_mod, e.ln_shift_off, e.ln_scale_off, e.ln_six_d = lmod.data_ptr(), 3 * N, 4 * N, 6 * N
                e.ln_blk = lblk.data_ptr() if lblk is not None else None
        return e

    r1 = to_dev(c0, torch.float32)
    y1 = torch.full((M, width), 7.0, dtype=odt, device=device())
    run(lib, A, W, M, N, K, epi(r1, y1))
    r2 = to_dev(c0, torch.float32)
    y2 = torch.full((M, width), 7.0, dtype=odt, device=device())
    run(lib, A, W, M, N, K, epi(r2, None))
    call(lib.sd_k_ln_mod(sdlib.SD_DTYPE_BF16, r2.data_ptr(), y2.data_ptr(), M, N, Lr,
                         lmod.data_ptr() if lmod is not None else None,
                         lblk.data_ptr() if lblk is not None else None, 3 * N, 4 * N, 6 * N, form, stream_ptr()))
    torch.cuda.synchronize()
    assert torch.equal(r1, r2), "residual differs"
    assert torch.equal(y1, y2), "LayerNorm output differs"
    assert not torch.equal(r1, to_dev(c0, torch.float32))


@pytest.mark.parametrize("M,H,Cp,K", [(128, 12, 80, 1536), (256, 12, 80, 1536), (96, 4, 40, 640)])
def test_score_gemm_with_grouped_softmax(lib, M, H, Cp, K):
    """The folded cross-attention's score product with its grouped softmax in
    the reduction pass (sd_gemm_epi.sm_out, few rows): bit for bit the
    probabilities of the product stored in fp32 followed by the softmax pass
    (taken here by giving the scores a wider row pitch), and within fp16
    rounding of the softmax of the exact products."""
    print(f"score gemm + softmax M={M} H={H} Cp={Cp} K={K}", flush=True)
    N = H * Cp
    A, W, b, acc = int_operands(M, N, K, 41)
    acc = acc - b.float().cpu().numpy().astype(np.float64)      # no bias on this product
    rng = np.random.default_rng(42)
    c = to_dev(rng.standard_normal(N), torch.float32)
    ws, wsp, wsb = split_ws()
    p1 = torch.full((M, N), 7.0, dtype=torch.float16, device=device())
    sc = torch.full((M, N), 7.0, dtype=torch.float32, device=device())
    e = sdlib.sd_gemm_epi(mode=sdlib.SD_EPI_F32, out=sc.data_ptr(), ldo=N, workspace=wsp, workspace_bytes=wsb,
                          sm_out=p1.data_ptr(), sm_bias=c.data_ptr(), sm_heads=H, sm_cp=Cp)
    run(lib, A, W, M, N, K, e)
    assert torch.all(sc == 7.0), "fused pass wrote the scores"
    p2 = torch.full((M, N), 7.0, dtype=torch.float16, device=device())
    e = sdlib.sd_gemm_epi(mode=sdlib.SD_EPI_F32, out=sc.data_ptr(), ldo=N, workspace=wsp, workspace_bytes=wsb)
    run(lib, A, W, M, N, K, e)
    assert np.array_equal(sc.cpu().numpy().astype(np.float64), acc)
    # the separate softmax pass on the stored scores, through a GEMM whose
    # output is the same scores but not split (no workspace)
    e = sdlib.sd_gemm_epi(mode=sdlib.SD_EPI_F32, out=sc.data_ptr(), ldo=N, sm_out=p2.data_ptr(),
                          sm_bias=c.data_ptr(), sm_heads=H, sm_cp=Cp)
    run(lib, A, W, M, N, K, e)
    assert torch.equal(p1, p2), "fused and separate softmax differ"
    z = (acc + c.cpu().numpy().astype(np.float64)).reshape(M, H, Cp)
    z = np.exp(z - z.max(axis=-1, keepdims=True))
    ref = (z / z.sum(axis=-1, keepdims=True)).reshape(M, N)
    got = p1.float().cpu().numpy()
    assert np.max(np.abs(got - ref) - 2.0 ** -11 * ref) <= 1e-6
