"""GPU parity of the Stream-VAE through the C ABI: single causal convolutions
(sd_k_conv3d) bit-exact on integer-valued operands at ragged sizes and
sampled at the video decoder's full shapes, and whole chunked encode /
decode streams (sd_vae_*) against the CPU oracle."""
import ctypes as C

import numpy as np
import pytest
import torch

import streaming_diffusion_amd._lib as L
from oracle import vae as ovae
from streaming_diffusion_amd.runner import VAERunner, upload_vae_weights
from workloads import gen, get_vae_config

from gpu_helpers import call, check_close, device, stream_ptr, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    device()
    return L.load()


def int_operands(seed, T, H, W, Ci, Co):
    """Operands k/8 (|k| <= 4) and weights k/16 (|k| <= 3): every product and
    partial sum is exact in fp32."""
    rng = np.random.default_rng(seed)
    x = rng.integers(-4, 5, (T, H, W, Ci)) / 8.0
    cache = rng.integers(-4, 5, (2, H, W, Ci)) / 8.0
    w = rng.integers(-3, 4, (Co, 3, 3, 3, Ci)) / 16.0
    b = rng.integers(-8, 9, Co) / 16.0
    return x, cache, w, b


def bf16_of(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)


@pytest.mark.parametrize("T,H,W,Ci,Co", [(4, 5, 7, 8, 16), (4, 9, 13, 24, 64), (2, 6, 10, 64, 132),
                                         (3, 16, 17, 128, 256), (4, 1, 1, 8, 4), (3, 7, 11, 16, 32),
                                         (2, 5, 6, 8, 20), (2, 8, 9, 40, 96), (2, 47, 97, 64, 256)])
def test_conv3d_bit_exact_on_integers(lib, T, H, W, Ci, Co):
    """Register-staged implicit GEMM at ragged small shapes; the last case
    (9118 positions, 256 channels) takes the DMA kernel's 128 x 64 tiles."""
    print(f"conv3d exact T={T} H={H} W={W} Cin={Ci} Cout={Co}", flush=True)
    x, cache, w, b = int_operands(T * 1000 + Co, T, H, W, Ci, Co)
    ref, _ = ovae.causal_conv3d(x, w, b, cache)
    dx, dc, dw, db = (to_dev(a, torch.bfloat16) for a in (x, cache, w, b))
    y = torch.empty((T, H, W, Co), dtype=torch.bfloat16, device=device())
    call(lib.sd_k_conv3d(dx.data_ptr(), dc.data_ptr(), dw.data_ptr(), db.data_ptr(), y.data_ptr(), None,
                         T, H, W, Ci, Co, stream_ptr()))
    torch.cuda.synchronize()
    # the exact sum, rounded once to bf16 (round to nearest even) by the kernel
    assert np.array_equal(y.float().cpu().numpy().astype(np.float64), bf16_of(ref))


@pytest.mark.parametrize("Co", [3, 16])
def test_conv3d_narrow_bit_exact_on_integers(lib, Co):
    T, H, W, Ci = 4, 6, 9, 24
    x, cache, w, b = int_operands(Co, T, H, W, Ci, Co)
    ref, _ = ovae.causal_conv3d(x, w, b, cache)
    dx, dc, dw, db = (to_dev(a, torch.bfloat16) for a in (x, cache, w, b))
    y = torch.empty((T, Co, H, W), dtype=torch.float32, device=device())
    call(lib.sd_k_conv3d(dx.data_ptr(), dc.data_ptr(), dw.data_ptr(), db.data_ptr(), None, y.data_ptr(),
                         T, H, W, Ci, Co, stream_ptr()))
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64), np.transpose(ref, (0, 3, 1, 2)))


@pytest.mark.parametrize("T,H,W,Ci,Co,cf", [(4, 13, 37, 64, 3, True), (4, 9, 20, 32, 16, False),
                                            (2, 10, 40, 96, 16, True), (2, 7, 19, 32, 8, False)])
def test_conv3d_narrow_halo_bit_exact_on_integers(lib, T, H, W, Ci, Co, cf):
    """At most 16 output channels with 32-channel input chunks: the narrow halo
    kernel (16 x 16 x 32 products, weights zero past Cout; 4 x 8 x 16 tiles for
    4 frames, 2 x 2 x 16 for 2), ragged frames, an odd number of chunks (96
    channels), fp32 channels-first or bf16 channels-last out."""
    print(f"conv3d narrow halo T={T} H={H} W={W} Cin={Ci} Cout={Co} cf={cf}", flush=True)
    x, cache, w, b = int_operands(T * 31 + Co + Ci, T, H, W, Ci, Co)
    ref, _ = ovae.causal_conv3d(x, w, b, cache)
    dx, dc, dw, db = (to_dev(a, torch.bfloat16) for a in (x, cache, w, b))
    if cf:
        y = torch.empty((T, Co, H, W), dtype=torch.float32, device=device())
        call(lib.sd_k_conv3d(dx.data_ptr(), dc.data_ptr(), dw.data_ptr(), db.data_ptr(), None, y.data_ptr(),
                             T, H, W, Ci, Co, stream_ptr()))
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().astype(np.float64), np.transpose(ref, (0, 3, 1, 2)))
    else:
        y = torch.empty((T, H, W, Co), dtype=torch.bfloat16, device=device())
        call(lib.sd_k_conv3d(dx.data_ptr(), dc.data_ptr(), dw.data_ptr(), db.data_ptr(), y.data_ptr(), None,
                             T, H, W, Ci, Co, stream_ptr()))
        torch.cuda.synchronize()
        assert np.array_equal(y.float().cpu().numpy().astype(np.float64), bf16_of(ref))


def test_conv3d_without_cache_is_zero_history(lib):
    T, H, W, Ci, Co = 3, 4, 5, 16, 8
    x, _, w, b = int_operands(7, T, H, W, Ci, Co)
    ref, _ = ovae.causal_conv3d(x, w, b, None)
    dx, dw, db = (to_dev(a, torch.bfloat16) for a in (x, w, b))
    y = torch.empty((T, H, W, Co), dtype=torch.bfloat16, device=device())
    call(lib.sd_k_conv3d(dx.data_ptr(), None, dw.data_ptr(), db.data_ptr(), y.data_ptr(), None, T, H, W, Ci, Co,
                         stream_ptr()))
    torch.cuda.synchronize()
    assert np.array_equal(y.float().cpu().numpy().astype(np.float64), bf16_of(ref))


def sampled_positions(rng, T, H, W, n=48):
    pts = {(0, 0, 0), (T - 1, H - 1, W - 1), (0, H - 1, 0), (1, 0, W - 1)}
    while len(pts) < n:
        pts.add((int(rng.integers(T)), int(rng.integers(H)), int(rng.integers(W))))
    return sorted(pts)


def conv_at(x, cache, w, b, t, i, j):
    """One output position of the causal convolution, from its definition."""
    T, H, W, Ci = x.shape
    acc = b.astype(np.float64).copy()
    for dt in range(3):
        for dy in range(3):
            for dx in range(3):
                tt, yy, xx = t + dt - 2, i + dy - 1, j + dx - 1
                if not (0 <= yy < H and 0 <= xx < W):
                    continue
                v = cache[tt + 2, yy, xx] if tt < 0 else x[tt, yy, xx]
                acc += w[:, dt, dy, dx, :] @ v.astype(np.float64)
    return acc


@pytest.mark.parametrize("T,H,W,Ci,Co", [(4, 128, 160, 64, 256), (4, 128, 256, 128, 128), (4, 256, 256, 128, 64),
                                         (4, 124, 200, 96, 192), (2, 256, 256, 64, 128), (3, 256, 352, 64, 64),
                                         (2, 60, 104, 256, 256), (4, 128, 256, 8, 64), (4, 124, 250, 8, 128)])
def test_conv3d_wide_paths_bit_exact_sampled(lib, T, H, W, Ci, Co):
    """The wide-layer kernels: 4-frame layers take the halo kernel (4 x 8 x 16
    output tiles, the 6 x 10 x 18 input halo per 32-channel chunk in LDS, all
    27 taps read from it; ragged 124 x 200 frame and 96 / 192 channels
    included), other layers with at least 512 tiles the DMA-fed implicit GEMM
    (256 x 128 and 512 x 64 tiles, 64-deep k-tiles inside one tap), the
    encoder's latent-resolution layer (2 x 60 x 104, 256 channels, too few
    tiles for both) its 128 x 64 tiles, 4-frame layers with 8 input
    channels the 16-byte-row halo kernel (two taps per product).  Integer
    operands: outputs at borders, cache frames and random positions equal the
    exact sum rounded once to bf16."""
    print(f"conv3d DMA path T={T} H={H} W={W} Cin={Ci} Cout={Co}", flush=True)
    x, cache, w, b = int_operands(T * 7 + Co, T, H, W, Ci, Co)
    dx, dc, dw, db = (to_dev(a, torch.bfloat16) for a in (x, cache, w, b))
    y = torch.empty((T, H, W, Co), dtype=torch.bfloat16, device=device())
    call(lib.sd_k_conv3d(dx.data_ptr(), dc.data_ptr(), dw.data_ptr(), db.data_ptr(), y.data_ptr(), None,
                         T, H, W, Ci, Co, stream_ptr()))
    torch.cuda.synchronize()
    yc = y.float().cpu().numpy().astype(np.float64)
    pts = sampled_positions(np.random.default_rng(5), T, H, W, n=64)
    got = np.stack([yc[t, i, j] for t, i, j in pts])
    ref = np.stack([conv_at(x, cache, w, b, t, i, j) for t, i, j in pts])
    assert np.array_equal(got, bf16_of(ref))


@pytest.mark.parametrize("T,H,W,Ci,Co", [(4, 128, 256, 32, 64), (4, 124, 200, 64, 192)])
def test_conv3d_upsampled_input_bit_exact_sampled(lib, T, H, W, Ci, Co):
    """sd_k_conv3d_up2: the halo kernel reading a half-size input (and cache)
    upsampled 2x2 (nearest) on the fly, as the decoder's upsampling layers do;
    against the definition on the explicitly upsampled operands (ragged
    124 x 200 frame, 192 channels included)."""
    print(f"conv3d up2 T={T} H={H} W={W} Cin={Ci} Cout={Co}", flush=True)
    x, cache, w, b = int_operands(T * 13 + Co, T, H // 2, W // 2, Ci, Co)
    dx, dc, dw, db = (to_dev(a, torch.bfloat16) for a in (x, cache, w, b))
    y = torch.empty((T, H, W, Co), dtype=torch.bfloat16, device=device())
    call(lib.sd_k_conv3d_up2(dx.data_ptr(), dc.data_ptr(), dw.data_ptr(), db.data_ptr(), y.data_ptr(),
                             T, H, W, Ci, Co, stream_ptr()))
    torch.cuda.synchronize()
    up = lambda a: np.repeat(np.repeat(a, 2, axis=1), 2, axis=2)
    xu, cu = up(x), up(cache)
    yc = y.float().cpu().numpy().astype(np.float64)
    pts = sampled_positions(np.random.default_rng(9), T, H, W, n=64)
    got = np.stack([yc[t, i, j] for t, i, j in pts])
    ref = np.stack([conv_at(xu, cu, w, b, t, i, j) for t, i, j in pts])
    assert np.array_equal(got, bf16_of(ref))


@pytest.mark.parametrize("layer", ["d3", "d_out"])
def test_conv3d_full_video_shape_sampled(lib, layer):
    """The video decoder's two full-resolution layers (4 x 480 x 832): d3
    (128 -> 64 channels, bf16 out) and d_out (64 -> 3, fp32 channels-first out,
    the narrow halo kernel),
    random bf16 operands, outputs sampled at borders, cache frames and random
    positions against the definition in fp64."""
    v = get_vae_config("video13b")
    T, H, W = v.frames, v.height, v.width
    Ci, Co = (v.c2, v.c1) if layer == "d3" else (v.c1, 3)
    print(f"conv3d full shape {layer}: T={T} H={H} W={W} Cin={Ci} Cout={Co}", flush=True)
    g = torch.Generator(device=device()).manual_seed(11)
    dx = torch.randn((T, H, W, Ci), generator=g, device=device()).to(torch.bfloat16)
    dc = torch.randn((2, H, W, Ci), generator=g, device=device()).to(torch.bfloat16)
    dw = (torch.randn((Co, 3, 3, 3, Ci), generator=g, device=device()) / np.sqrt(27 * Ci)).to(torch.bfloat16)
    db = (0.1 * torch.randn((Co,), generator=g, device=device())).to(torch.bfloat16)
    if layer == "d3":
        y = torch.empty((T, H, W, Co), dtype=torch.bfloat16, device=device())
        call(lib.sd_k_conv3d(dx.data_ptr(), dc.data_ptr(), dw.data_ptr(), db.data_ptr(), y.data_ptr(), None,
                             T, H, W, Ci, Co, stream_ptr()))
    else:
        y = torch.empty((T, Co, H, W), dtype=torch.float32, device=device())
        call(lib.sd_k_conv3d(dx.data_ptr(), dc.data_ptr(), dw.data_ptr(), db.data_ptr(), None, y.data_ptr(),
                             T, H, W, Ci, Co, stream_ptr()))
    torch.cuda.synchronize()
    x, c = dx.float().cpu().numpy(), dc.float().cpu().numpy()         # float32 copies, indexed per sample
    w, b = (t.float().cpu().numpy().astype(np.float64) for t in (dw, db))
    yc = y.float().cpu().numpy()
    pts = sampled_positions(np.random.default_rng(3), T, H, W)
    got = np.stack([yc[t, i, j] if layer == "d3" else yc[t, :, i, j] for t, i, j in pts])
    ref = np.stack([conv_at(x, c, w, b, t, i, j) for t, i, j in pts])
    check_close(got, ref, "bf16", f"{layer} sampled", stored_bf16=(layer == "d3"))


# Whole encoder / decoder chains: the bf16 bar of the path (2e-2 max-abs over
# RMS).  The chains store their activations in fp16 (2^-11 relative per
# rounding, 9 roundings on the decoder path through layers of unit gain), so
# the bar holds with margin; the RMS of the error stays near one rounding.
VAE_MAX_TOL = 2e-2
VAE_RMS_TOL = 5e-3


def check_vae(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    e_max = np.max(np.abs(got - ref)) / rms
    e_rms = np.sqrt(np.mean((got - ref) ** 2)) / rms
    print(f"  {what}: max-abs/RMS {e_max:.3e}, RMS {e_rms:.3e}", flush=True)
    assert e_max <= VAE_MAX_TOL and e_rms <= VAE_RMS_TOL, f"{what}: max-abs/RMS {e_max:.3e}, RMS {e_rms:.3e}"


def run_vae_stream(vcfg, chunks=3):
    w = gen.make_vae_weights(vcfg)
    orc = ovae.StreamVAE(vcfg, w)
    run = VAERunner(vcfg, upload_vae_weights(vcfg, w))
    src = gen.PixelSource(vcfg)
    worst = 0.0
    for k in range(chunks):
        pix = src.next()
        z_ref = orc.encode_chunk(pix)
        z = run.encode(to_dev(pix, torch.float32))
        x_ref = orc.decode_chunk(z_ref)
        x = run.decode(to_dev(z_ref, torch.float32))        # decode the oracle's latent: layers compared one by one
        torch.cuda.synchronize()
        check_vae(z.cpu().numpy(), z_ref, f"chunk {k} latent")
        check_vae(x.cpu().numpy(), x_ref, f"chunk {k} pixels")
        worst = max(worst, float(np.abs(x.cpu().numpy() - x_ref).max()))
    return orc, run, src, worst


def test_vae_small_stream_matches_oracle_over_chunks():
    device()
    v = get_vae_config("small")
    print("Stream-VAE small, 3 chunks", flush=True)
    orc, run, src, worst = run_vae_stream(v)
    # reset: both sides start a new video
    orc.reset()
    run.reset()
    pix = src.next()
    z = run.encode(to_dev(pix, torch.float32))
    torch.cuda.synchronize()
    check_vae(z.cpu().numpy(), orc.encode_chunk(pix), "after reset")
    run.close()


def test_vae_stream_three_latent_frames_wider_grid():
    device()
    v = get_vae_config("small", latent_h=6, latent_w=7, c1=32, c2=64, c3=128, latent_t=3)
    print("Stream-VAE medium, latent_t=3", flush=True)
    _, run, _, _ = run_vae_stream(v, chunks=2)
    run.close()


def test_vae_stream_full_resolution_layer_on_the_halo_path():
    """192 x 256 pixels, widths 128 / 128 / 256: the decoder's full-resolution
    128 -> 128 convolution (4 x 192 x 256 positions) runs on the halo kernel
    with 128-channel tiles and fp16 operands; two chunks against the oracle."""
    device()
    v = get_vae_config("small", latent_h=24, latent_w=32, c1=128, c2=128, c3=256)
    print("Stream-VAE 192 x 256, widths 128 / 128 / 256, 2 chunks", flush=True)
    _, run, _, _ = run_vae_stream(v, chunks=2)
    run.close()


def test_vae_stream_64_channel_full_resolution_layer_on_the_halo_path():
    """256 x 256 pixels, widths 64 / 128 / 256: the decoder's full-resolution
    128 -> 64 convolution (4 x 256 x 256 positions) runs on the halo kernel
    with 64-channel tiles and fp16 operands; one chunk against the oracle."""
    device()
    v = get_vae_config("small", latent_h=32, latent_w=32, c1=64, c2=128, c3=256)
    print("Stream-VAE 256 x 256, widths 64 / 128 / 256, 1 chunk", flush=True)
    _, run, _, _ = run_vae_stream(v, chunks=1)
    run.close()
