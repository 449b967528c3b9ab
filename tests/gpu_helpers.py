"""Shared helpers of the GPU parity tests (imported by test_gpu_*.py only)."""
import ctypes as C

import numpy as np
import torch

import streaming_diffusion_amd._lib as L


def device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def stream_ptr():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def to_dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device()).to(dtype).contiguous()


def bf16_round(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def maxabs_over_rms(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(got - ref)) / max(rms, 1e-30))


def rel_inf(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


# tolerances: fp32 1e-4 relative (max-abs over max-abs); bf16 2e-2 max-abs over RMS
FP32_TOL = 1e-4
BF16_TOL = 2e-2


def check_close(got, ref, dtype, what="", stored_bf16=False):
    """fp32: max|got-ref| / max|ref| <= 1e-4.  bf16: max|got-ref| / RMS(ref)
    <= 2e-2.  A tensor that the kernel itself stores in bf16 carries its own
    final rounding (up to 2^-8 relative per element, which alone can exceed
    2e-2 of the RMS when max|ref|/RMS > 5); for those the per-element rounding
    bound 2^-8 |ref| is subtracted before the 2e-2 bar is applied."""
    if dtype == "f32":
        e = rel_inf(got, ref)
        assert e <= FP32_TOL, f"{what}: fp32 relative error {e:.3e} > {FP32_TOL}"
    elif stored_bf16:
        g = np.asarray(got, np.float64)
        r = np.asarray(ref, np.float64)
        rms = max(float(np.sqrt(np.mean(r * r))), 1e-30)
        e = float(np.max(np.maximum(np.abs(g - r) - 2.0 ** -8 * np.abs(r), 0.0)) / rms)
        assert e <= BF16_TOL, f"{what}: bf16 (stored) excess max-abs/RMS {e:.3e} > {BF16_TOL}"
    else:
        e = maxabs_over_rms(got, ref)
        assert e <= BF16_TOL, f"{what}: bf16 max-abs/RMS {e:.3e} > {BF16_TOL}"
    return e


def call(code):
    if code != L.SD_OK:
        raise L.SDError(code)
