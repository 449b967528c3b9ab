"""The allocation-free attention entry point (sd_k_attention_noalloc) against
sd_k_attention with a caller workspace: the same kernels and split, so the
outputs must be identical, on two calls in a row (the second smaller, so the
shared scratch still holds the first call's partials)."""
import numpy as np
import pytest
import torch

import streaming_diffusion_amd._lib as sdlib

from gpu_helpers import bf16_round, call, device, stream_ptr, to_dev
from test_gpu_kernels import make_segments

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    device()
    return sdlib.load()


def one_case(lib, R, H, L, hd, S, W, start, count, nsplit, seed):
    print(f"noalloc attention R={R} H={H} L={L} hd={hd} S={S} W={W} nsplit={nsplit}", flush=True)
    rng = np.random.default_rng(seed)
    sink_cap = max(8, (S + 7) // 8 * 8)
    dev, segs, _, _ = make_segments(rng, H, hd, R, L, S, sink_cap, W, start, count, torch.bfloat16)
    q = to_dev(bf16_round(rng.standard_normal((R, H, L, hd)).astype(np.float32)), torch.bfloat16)
    o_ws = torch.empty((R * L, H * hd), dtype=torch.bfloat16, device=device())
    o_na = torch.empty_like(o_ws)
    wsb = lib.sd_k_attention_workspace_bytes(R, H, L, hd, nsplit)
    ws = torch.empty(max(wsb, 1) + 256, dtype=torch.uint8, device=device())
    wsp = (ws.data_ptr() + 255) // 256 * 256 if wsb else None
    call(lib.sd_k_attention(1, q.data_ptr(), H * L * hd, L * hd, o_ws.data_ptr(), R, H, L, hd, 3, segs, nsplit, wsp,
                            wsb, stream_ptr()))
    call(lib.sd_k_attention_noalloc(1, q.data_ptr(), H * L * hd, L * hd, o_na.data_ptr(), R, H, L, hd, 3, segs,
                                    nsplit, stream_ptr()))
    torch.cuda.synchronize()
    assert torch.equal(o_ws, o_na)
    assert torch.isfinite(o_na.float()).all()


def test_noalloc_matches_workspace_entry_point_on_two_calls(lib):
    # the video step's shape (5 splits, two rows, full sink and wrapped window), then a smaller ragged one
    one_case(lib, 2, 12, 3120, 128, 1560, 9360, 3120, 9360, 5, 1)
    one_case(lib, 2, 2, 200, 64, 12, 160, 152, 160, 3, 2)


def test_noalloc_without_split_and_oversize_request(lib):
    one_case(lib, 1, 2, 72, 64, 4, 64, 40, 48, 1, 3)
    seg = (sdlib.sd_kv_segment * 1)(sdlib.sd_kv_segment(k=8, vt=8, cap=64, start=0, count=64, wrap=0))
    assert lib.sd_k_attention_noalloc(1, 8, 0, 0, 8, 2, 12, 3120, 128, 1, seg, 8, stream_ptr()) == \
        sdlib.SD_ERR_WORKSPACE
