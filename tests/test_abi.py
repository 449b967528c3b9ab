"""CPU checks of the boundary: the library loads and exports every symbol the
headers declare, argument validation happens before any device call, and the
host state module's fp64 decisions equal the oracle's bit for bit."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from oracle import controls, schedule
from workloads import CONFIGS, get_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
L = pytest.importorskip("streaming_diffusion_amd._lib")


def header_symbols():
    syms = set()
    for h in ("sd_stream.h", "sd_kernels.h", "sd_vae.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        syms |= set(re.findall(r"\b(sd_(?:stream|k|vae)_\w+)\s*\(", src))
    return sorted(syms)


@pytest.fixture(scope="module")
def lib():
    return L.load()


@pytest.fixture(scope="module")
def state():
    return L.load_state()


def test_every_declared_symbol_is_exported(lib):
    syms = header_symbols()
    assert len(syms) >= 14
    for s in syms:
        assert hasattr(lib, s), s
    assert set(syms) == set(L.SIGNATURES), "binding and headers disagree"


def test_struct_sizes_match_a_c_compiler(tmp_path):
    """Compile a probe against the header and compare sizeof/offsetof with ctypes."""
    probe = tmp_path / "probe.c"
    fields = [f for f, _ in L.sd_stream_config._fields_]
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{ROOT}/include/sd_kernels.h"', "int main(void){"]
    lines.append('printf("%zu %zu %zu %zu %zu %zu\\n", sizeof(sd_stream_config), sizeof(sd_weights), '
                 'sizeof(sd_push_info), sizeof(sd_step_info), sizeof(sd_sink_info), sizeof(sd_kv_segment));')
    for f in fields:
        lines.append(f'printf("%zu\\n", offsetof(sd_stream_config, {f}));')
    lines.append("return 0;}")
    probe.write_text("\n".join(lines))
    exe = tmp_path / "probe"
    assert os.system(f"gcc -o {exe} {probe}") == 0
    out = os.popen(str(exe)).read().split()
    sizes = [int(v) for v in out[:6]]
    assert sizes == [C.sizeof(L.sd_stream_config), C.sizeof(L.sd_weights), C.sizeof(L.sd_push_info),
                     C.sizeof(L.sd_step_info), C.sizeof(L.sd_sink_info), C.sizeof(L.sd_kv_segment)]
    offs = [int(v) for v in out[6:]]
    assert offs == [getattr(L.sd_stream_config, f).offset for f in fields]


def cfg_struct(name, **kw):
    from streaming_diffusion_amd.runner import make_config
    return make_config(get_config(name, **kw))


@pytest.mark.parametrize("name", list(CONFIGS))
def test_workload_configs_validate(lib, state, name):
    c = cfg_struct(name)
    msg = C.create_string_buffer(256)
    assert state.sdstate_validate(C.byref(c), msg, 256) == 0, msg.value
    assert lib.sd_stream_workspace_bytes(C.byref(c)) > 0


@pytest.mark.parametrize("kw,code", [
    (dict(n_heads=5), L.SD_ERR_SHAPE),
    (dict(t_index=(32, 51)), L.SD_ERR_ARG),
    (dict(window_tokens=32), L.SD_ERR_ARG),          # window smaller than a chunk
    (dict(ssf_eta=1.0), L.SD_ERR_ARG),
    (dict(chunks_per_step=0), L.SD_ERR_ARG),
    (dict(chunks_per_step=9), L.SD_ERR_ARG),         # beyond SD_MAX_CHUNKS
    (dict(chunks_per_step=8, t_index=(0, 8, 16, 24, 32, 40)), L.SD_ERR_ARG),   # 48 rows > SD_MAX_ROWS
    (dict(cfg_type="onetime"), L.SD_ERR_ARG),        # tiny has no context
    (dict(cfg_type="full"), L.SD_ERR_ARG),
    (dict(cfg_type="onetime", ctx_len=8, batch_attn=True), L.SD_ERR_ARG),   # batch attention mixes prompts
    (dict(cfg_type="full", ctx_len=8, chunks_per_step=3, t_index=(0, 8, 16, 24, 32, 40, 45)), L.SD_ERR_ARG),  # 42 rows
    (dict(latent_h=15), L.SD_ERR_SHAPE),
    (dict(d_model=5184, n_heads=81), L.SD_ERR_SHAPE),  # beyond the register-resident LayerNorm rows
])
def test_invalid_configs_are_rejected(lib, state, kw, code):
    c = cfg_struct("tiny", **kw)
    assert state.sdstate_validate(C.byref(c), None, 0) == code
    assert lib.sd_stream_workspace_bytes(C.byref(c)) == 0


def test_create_rejects_bad_arguments_before_any_device_call(lib):
    c = cfg_struct("tiny")
    w = L.sd_weights()
    h = C.c_void_p()
    assert lib.sd_stream_create(None, C.byref(w), None, 0, None, C.byref(h)) == L.SD_ERR_ARG
    assert lib.sd_stream_create(C.byref(c), C.byref(w), C.c_void_p(256), 1 << 30, None, C.byref(h)) == L.SD_ERR_ARG
    for f in L.WEIGHT_FIELDS:
        setattr(w, f, 4096)
    assert lib.sd_stream_create(C.byref(c), C.byref(w), None, 1 << 30, None, C.byref(h)) == L.SD_ERR_WORKSPACE
    assert lib.sd_stream_create(C.byref(c), C.byref(w), C.c_void_p(4097), 1 << 30, None, C.byref(h)) == L.SD_ERR_WORKSPACE
    assert lib.sd_stream_create(C.byref(c), C.byref(w), C.c_void_p(4096), 16, None, C.byref(h)) == L.SD_ERR_WORKSPACE
    assert lib.sd_stream_push_frame(None, None, None, None, 0.0, None) == L.SD_ERR_ARG
    assert lib.sd_stream_step(None, None, None) == L.SD_ERR_ARG
    assert lib.sd_stream_kv_reset(None) == L.SD_ERR_ARG
    assert lib.sd_k_gemm(0, None, None, None, None, 1, 1, 8, None) == L.SD_ERR_ARG
    assert lib.sd_k_gemm(1, 8, 8, None, 8, 1, 1, 12, None) == L.SD_ERR_SHAPE
    assert lib.sd_k_gemm_resid(2, 8, 8, None, 8, 1, 1, 8, None) == L.SD_ERR_ARG
    assert lib.sd_k_gemm_resid(1, 8, None, None, 8, 1, 1, 8, None) == L.SD_ERR_ARG
    assert lib.sd_k_gemm_resid(1, 8, 8, None, 8, 1, 1, 60, None) == L.SD_ERR_SHAPE
    seg = L.sd_kv_segment(k=8, vt=8, cap=64, start=0, count=100, wrap=0)
    assert lib.sd_k_attention(1, 8, 0, 0, 8, 1, 1, 8, 64, 1, C.byref(seg), 1, None, 0, None) == L.SD_ERR_SHAPE
    assert lib.sd_k_attention(1, 8, 0, 0, 8, 1, 1, 8, 48, 1, C.byref(seg), 1, None, 0, None) == L.SD_ERR_SHAPE
    assert lib.sd_k_attention(1, 8, 0, 0, 8, 1, 1, 8, 64, 1, C.byref(seg), 2, None, 0, None) == L.SD_ERR_ARG
    assert lib.sd_k_attention(1, 8, 0, 0, 8, 1, 1, 8, 64, 1, C.byref(seg), 2, 256, 16, None) == L.SD_ERR_WORKSPACE
    assert lib.sd_k_attention_plan(1, 8, 0, 0, 8, 1, 2, 8, 64, 1, C.byref(seg), 2, 3, 256, 1 << 20,
                                   None) == L.SD_ERR_ARG       # unsplit heads > H
    assert lib.sd_k_attention_plan(1, 8, 0, 0, 8, 1, 2, 8, 64, 1, C.byref(seg), 2, -1, 256, 1 << 20,
                                   None) == L.SD_ERR_ARG
    ns, hf = C.c_int32(), C.c_int32()
    assert lib.sd_k_attention_pick_plan(0, 1, 1, 8, 512, C.byref(ns), C.byref(hf)) == L.SD_ERR_ARG
    assert lib.sd_k_attention_pick_plan(1, 1, 1, 8, 512, None, C.byref(hf)) == L.SD_ERR_ARG
    assert lib.sd_k_attention_workspace_bytes(2, 3, 40, 64, 1) == 0
    assert lib.sd_k_attention_workspace_bytes(2, 3, 40, 64, 3) == ((3 * 2 * 40 * 3 * 64 * 2 + 255) // 256 * 256
                                                                  + 3 * 2 * 3 * 40 * 8)


# ------------------------------------------------------------------ host state vs oracle, bit for bit
def test_schedule_bit_exact(state):
    c = cfg_struct("tiny")
    a = (C.c_double * 1000)()
    b = (C.c_double * 1000)()
    state.sdstate_schedule(C.byref(c), a, b)
    ab = schedule.alphas_cumprod()
    assert np.array_equal(np.frombuffer(a, np.float64), np.sqrt(ab))
    assert np.array_equal(np.frombuffer(b, np.float64), np.sqrt(1.0 - ab))


def test_timesteps_bit_exact(state):
    out = (C.c_int32 * 8)()
    c = cfg_struct("fourstep")
    state.sdstate_taus_t_index(C.byref(c), out)
    assert list(out)[:4] == schedule.taus_from_t_index(get_config("fourstep"))
    rng = np.random.default_rng(0)
    for s in list(rng.uniform(0.3, 0.9, 500)) + [0.5, 0.3, 0.9, 1.0 / 3.0]:
        for n in (1, 2, 3, 4):
            state.sdstate_taus_noise_rate(float(s), n, 1000, out)
            assert list(out)[:n] == schedule.taus_from_noise_rate(float(s), n)


def test_ssf_tail_bit_exact(state):
    rng = np.random.default_rng(1)
    for _ in range(300):
        a = rng.integers(0, 256, 500)
        b = np.clip(a + rng.integers(-9, 10, 500), 0, 255)
        D, N1, N2 = controls.ssf_sums(a, b)
        sim = state.sdstate_ssf_cosine(D, N1, N2)
        assert sim == controls.cosine_from_sums(D, N1, N2)
        for eta in (0.5, 0.95, 0.98):
            assert state.sdstate_ssf_probability(sim, eta) == controls.skip_probability(sim, eta)
    assert state.sdstate_ssf_cosine(0, 0, 0) == 1.0
    assert state.sdstate_ssf_cosine(0, 0, 5) == 0.0


def test_motion_bit_exact(state):
    cfg = get_config("video13b")
    c = cfg_struct("video13b")
    rng = np.random.default_rng(2)
    s = cfg.s_max
    win = []
    for _ in range(200):
        ss = int(rng.integers(0, 1 << 50))
        dist = state.sdstate_motion_distance(ss, 99840)
        assert dist == controls.motion_distance(ss, 99840)
        win = (win + [dist])[-cfg.motion_k:]
        arr = (C.c_double * len(win))(*win)
        s_c = state.sdstate_motion_update(s, arr, len(win), C.byref(c))
        s_o = controls.motion_update(s, win, cfg)
        assert s_c == s_o
        s = s_o


def test_unknown_sampler_and_batch_flag_are_rejected(lib, state):
    for field, value in (("sampler", 7), ("batch_attn", 2)):
        c = cfg_struct("tiny")
        setattr(c, field, value)
        assert state.sdstate_validate(C.byref(c), None, 0) == L.SD_ERR_ARG
        assert lib.sd_stream_workspace_bytes(C.byref(c)) == 0
    c = cfg_struct("tiny", sampler="lcm")
    assert state.sdstate_validate(C.byref(c), None, 0) == L.SD_OK


def test_vae_struct_sizes_match_a_c_compiler(tmp_path):
    probe = tmp_path / "probe.c"
    fields = [f for f, _ in L.sd_vae_config._fields_]
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{ROOT}/include/sd_vae.h"', "int main(void){",
             'printf("%zu %zu\\n", sizeof(sd_vae_config), sizeof(sd_vae_weights));']
    lines += [f'printf("%zu\\n", offsetof(sd_vae_config, {f}));' for f in fields]
    lines.append('printf("%d\\n", (int)SD_VAE_LAYERS); return 0;}')
    probe.write_text("\n".join(lines))
    exe = tmp_path / "probe"
    assert os.system(f"gcc -o {exe} {probe}") == 0
    out = [int(v) for v in os.popen(str(exe)).read().split()]
    assert out[:2] == [C.sizeof(L.sd_vae_config), C.sizeof(L.sd_vae_weights)]
    assert out[2:-1] == [getattr(L.sd_vae_config, f).offset for f in fields]
    assert out[-1] == L.SD_VAE_LAYERS


def vae_cfg(**kw):
    from streaming_diffusion_amd.runner import make_vae_config
    from workloads import get_vae_config
    return make_vae_config(get_vae_config("small", **kw))


@pytest.mark.parametrize("kw,ok", [({}, True), (dict(latent_t=1), False), (dict(latent_c=12), False),
                                   (dict(c2=48), False), (dict(latent_h=0), False)])
def test_vae_config_validation(lib, kw, ok):
    c = vae_cfg(**kw)
    assert (lib.sd_vae_workspace_bytes(C.byref(c)) > 0) == ok


def test_vae_and_conv_argument_errors(lib):
    c = vae_cfg()
    w = L.sd_vae_weights()
    h = C.c_void_p()
    assert lib.sd_vae_create(C.byref(c), C.byref(w), 256, 1 << 30, None, C.byref(h)) == L.SD_ERR_ARG   # null weights
    assert lib.sd_vae_encode(None, 8, 8) == L.SD_ERR_ARG
    assert lib.sd_k_conv3d(8, None, 8, None, 8, None, 1, 4, 4, 12, 8, None) == L.SD_ERR_SHAPE       # Cin % 8
    assert lib.sd_k_conv3d(8, None, 8, None, 8, None, 1, 4, 4, 8, 6, None) == L.SD_ERR_SHAPE        # Cout % 4
    assert lib.sd_k_conv3d(8, None, 8, None, None, 8, 1, 4, 4, 8, 17, None) == L.SD_ERR_SHAPE       # narrow > 16
    # the upsampled-input form takes only the halo kernel's shapes
    assert lib.sd_k_conv3d_up2(8, None, 8, None, 8, 3, 128, 256, 32, 64, None) == L.SD_ERR_SHAPE    # T != 4
    assert lib.sd_k_conv3d_up2(8, None, 8, None, 8, 4, 127, 256, 32, 64, None) == L.SD_ERR_SHAPE    # odd H
    assert lib.sd_k_conv3d_up2(8, None, 8, None, 8, 4, 128, 256, 24, 64, None) == L.SD_ERR_SHAPE    # Cin % 32
    assert lib.sd_k_conv3d_up2(8, None, 8, None, 8, 4, 16, 32, 32, 64, None) == L.SD_ERR_SHAPE      # too few tiles
    assert lib.sd_k_conv3d_up2(None, None, 8, None, 8, 4, 128, 256, 32, 64, None) == L.SD_ERR_ARG
    assert lib.sd_k_conv3d(None, None, 8, None, 8, None, 1, 4, 4, 8, 8, None) == L.SD_ERR_ARG


# ------------------------------------------------------------------ GEMM-epilogue and LN test entries
def test_gemm_epi_struct_matches_a_c_compiler(tmp_path):
    probe = tmp_path / "probe_epi.c"
    fields = [f for f, _ in L.sd_gemm_epi._fields_]
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{ROOT}/include/sd_kernels.h"', "int main(void){",
             'printf("%zu\\n", sizeof(sd_gemm_epi));']
    lines += [f'printf("%zu\\n", offsetof(sd_gemm_epi, {f}));' for f in fields]
    lines.append("return 0;}")
    probe.write_text("\n".join(lines))
    exe = tmp_path / "probe_epi"
    assert os.system(f"gcc -o {exe} {probe}") == 0
    out = [int(v) for v in os.popen(str(exe)).read().split()]
    assert out[0] == C.sizeof(L.sd_gemm_epi)
    assert out[1:] == [getattr(L.sd_gemm_epi, f).offset for f in fields]


def test_gemm_epi_and_ln_mod_reject_bad_arguments_before_any_device_call(lib):
    e = L.sd_gemm_epi(mode=L.SD_EPI_STORE, out=None, ldo=64)
    assert lib.sd_k_gemm_epi(8, 8, 64, 64, 64, C.byref(e), None) == L.SD_ERR_ARG        # no output
    e = L.sd_gemm_epi(mode=L.SD_EPI_STORE, out=8, ldo=32)
    assert lib.sd_k_gemm_epi(8, 8, 64, 64, 64, C.byref(e), None) == L.SD_ERR_ARG        # ldo < N
    assert lib.sd_k_gemm_epi(8, 8, 64, 64, 60, C.byref(e), None) == L.SD_ERR_SHAPE      # K % 8
    e = L.sd_gemm_epi(mode=99)
    assert lib.sd_k_gemm_epi(8, 8, 64, 64, 64, C.byref(e), None) == L.SD_ERR_ARG
    e = L.sd_gemm_epi(mode=L.SD_EPI_GATE_RESID, resid=8, mod=8, blk=8, L=16, gate_off=4, six_d=384)
    assert lib.sd_k_gemm_epi(8, 8, 64, 64, 64, C.byref(e), None) == L.SD_ERR_SHAPE      # unaligned gate offset
    e.gate_off = 336
    assert lib.sd_k_gemm_epi(8, 8, 64, 64, 64, C.byref(e), None) == L.SD_ERR_SHAPE      # gate beyond 6d
    # q | k | v widths must match the heads; rows must fit the k / v^T destination; RoPE positions in the table
    e = L.sd_gemm_epi(mode=L.SD_EPI_QKV, bias=8, q=8, k=8, vt=8, L=64, H=2, hd=32, kstride=64, krows=2)
    assert lib.sd_k_gemm_epi(8, 8, 128, 190, 64, C.byref(e), None) == L.SD_ERR_SHAPE
    assert lib.sd_k_gemm_epi(8, 8, 192, 192, 64, C.byref(e), None) == L.SD_ERR_SHAPE    # 3 rows > krows
    e.rope, e.rope_table, e.Hp, e.Wp, e.rope_positions = 1, 8, 8, 8, 4
    e.t0[0], e.t0[1] = 0, 4
    assert lib.sd_k_gemm_epi(8, 8, 128, 192, 64, C.byref(e), None) == L.SD_ERR_SHAPE    # position 4 not in table
    # the fused LayerNorm only after a residual epilogue, fp16 form without modulation, slots inside the rows
    e = L.sd_gemm_epi(mode=L.SD_EPI_F32, out=8, ldo=64, ln_out=8)
    assert lib.sd_k_gemm_epi(8, 8, 64, 64, 64, C.byref(e), None) == L.SD_ERR_ARG
    e = L.sd_gemm_epi(mode=L.SD_EPI_RESID, resid=8, ln_out=8, ln_form=L.SD_LN_F16, ln_mod=8, ln_six_d=384)
    assert lib.sd_k_gemm_epi(8, 8, 64, 64, 64, C.byref(e), None) == L.SD_ERR_ARG
    e = L.sd_gemm_epi(mode=L.SD_EPI_RESID, resid=8, ln_out=8, ln_form=3)
    assert lib.sd_k_gemm_epi(8, 8, 64, 64, 64, C.byref(e), None) == L.SD_ERR_ARG
    e = L.sd_gemm_epi(mode=L.SD_EPI_RESID, resid=8, ln_out=8, ln_mod=8, ln_shift_off=0, ln_scale_off=340,
                      ln_six_d=384)
    assert lib.sd_k_gemm_epi(8, 8, 64, 64, 64, C.byref(e), None) == L.SD_ERR_SHAPE      # scale beyond the row
    # the fused softmax only on F32 without bias, groups covering N, scores dense when not fused
    e = L.sd_gemm_epi(mode=L.SD_EPI_RESID, resid=8, sm_out=8, sm_bias=8, sm_heads=2, sm_cp=32)
    assert lib.sd_k_gemm_epi(8, 8, 64, 64, 64, C.byref(e), None) == L.SD_ERR_ARG
    e = L.sd_gemm_epi(mode=L.SD_EPI_F32, out=8, ldo=64, bias=8, sm_out=8, sm_bias=8, sm_heads=2, sm_cp=32)
    assert lib.sd_k_gemm_epi(8, 8, 64, 64, 64, C.byref(e), None) == L.SD_ERR_ARG
    e = L.sd_gemm_epi(mode=L.SD_EPI_F32, out=8, ldo=64, sm_out=8, sm_bias=8, sm_heads=3, sm_cp=32)
    assert lib.sd_k_gemm_epi(8, 8, 64, 64, 64, C.byref(e), None) == L.SD_ERR_SHAPE      # 3 x 32 != 64
    e = L.sd_gemm_epi(mode=L.SD_EPI_F32, out=8, ldo=72, sm_out=8, sm_bias=8, sm_heads=2, sm_cp=32)
    assert lib.sd_k_gemm_epi(8, 8, 64, 64, 64, C.byref(e), None) == L.SD_ERR_SHAPE      # unfused, ldo != N
    e = L.sd_gemm_epi(mode=L.SD_EPI_HEAD, bias=8, eps=8, L=64, C=4, p=2, T=1, Hp=8, Wp=8, Hl=16, Wl=15)
    assert lib.sd_k_gemm_epi(8, 8, 64, 16, 128, C.byref(e), None) == L.SD_ERR_SHAPE
    assert lib.sd_k_ln_mod(1, 8, 8, 4, 5124, 1, None, None, 0, 0, 0, 0, None) == L.SD_ERR_SHAPE
    assert lib.sd_k_ln_mod(1, 8, 8, 4, 128, 1, 8, 8, 0, 700, 768, 0, None) == L.SD_ERR_SHAPE
    assert lib.sd_k_ln_mod(3, 8, 8, 4, 128, 1, None, None, 0, 0, 0, 0, None) == L.SD_ERR_ARG
    assert lib.sd_k_ln_mod(0, 8, 8, 4, 128, 1, None, None, 0, 0, 0, L.SD_LN_SPLIT, None) == L.SD_ERR_ARG
    assert lib.sd_k_ln_mod(1, 8, 8, 4, 128, 1, 8, 8, 0, 128, 768, L.SD_LN_F16, None) == L.SD_ERR_ARG
    e = L.sd_gemm_epi(mode=L.SD_EPI_GELU, out=8, ldo=64, f16=1)
    assert lib.sd_k_gemm_epi(8, 8, 64, 64, 64, C.byref(e), None) == L.SD_ERR_ARG     # fp16: F32 / RESID only
    e = L.sd_gemm_epi(mode=L.SD_EPI_F32, out=8, ldo=64, wpack=24)
    assert lib.sd_k_gemm_epi(8, 8, 64, 64, 64, C.byref(e), None) == L.SD_ERR_ARG     # packed copy misaligned
    e.wpack = 32
    assert lib.sd_k_gemm_epi(8, 8, 64, 64, 96, C.byref(e), None) == L.SD_ERR_SHAPE   # packed: K % 64


def test_pack_weight_size_and_validation(lib):
    """The fragment-ordered weight copy: whole 32-row blocks of K/64 tiles of
    4 x 64 chunks of 16 bytes; rejected shapes and pointers never reach the
    device."""
    assert lib.sd_k_pack_weight_bytes(1536, 8960) == 1536 * 8960 * 2
    assert lib.sd_k_pack_weight_bytes(200, 640) == 224 * 640 * 2          # rows padded to 32
    assert lib.sd_k_pack_weight_bytes(64, 96) == 0
    assert lib.sd_k_pack_weight(None, 64, 64, 32, None) == L.SD_ERR_ARG
    assert lib.sd_k_pack_weight(32, 64, 96, 32, None) == L.SD_ERR_SHAPE
    assert lib.sd_k_pack_weight(32, 64, 64, 40, None) == L.SD_ERR_ARG       # output not 16-byte aligned


def test_rope_tables_are_cos_sin_of_the_section_angles(lib):
    """Host table of the RoPE epilogue: (cos, sin) of pos * base^(-2j/width)
    per section (t: hd - 2*dh, h = w: 2*floor(hd/6)), each value the fp64
    angle's cosine / sine rounded to fp32 (within one fp32 ulp of numpy's)."""
    hd, npos, Hp, Wp, base = 128, 7, 5, 6, 10000.0
    n = lib.sd_k_rope_table_pairs(hd, npos, Hp, Wp)
    dh = 2 * (hd // 6)
    dt = hd - 2 * dh
    assert n == npos * dt // 2 + Hp * dh // 2 + Wp * dh // 2
    buf = np.zeros(2 * n, np.float32)
    assert lib.sd_k_rope_tables(hd, npos, Hp, Wp, base, buf.ctypes.data) == L.SD_OK
    got = buf.reshape(-1, 2)
    ref = []
    for npos_a, width in ((npos, dt), (Hp, dh), (Wp, dh)):
        for p in range(npos_a):
            for j in range(width // 2):
                th = p * base ** (-2.0 * j / width)
                ref.append((np.cos(th), np.sin(th)))
    ref = np.array(ref, np.float32)
    assert np.all(np.abs(got - ref) <= np.spacing(np.abs(ref)))


def test_attention_noalloc_rejects_before_any_device_call(lib):
    seg = L.sd_kv_segment(k=8, vt=8, cap=64, start=0, count=64, wrap=0)
    # 8 splits of 2 rows x 12 heads x 3120 queries x hd 128 need more than the fixed scratch
    need = lib.sd_k_attention_workspace_bytes(2, 12, 3120, 128, 8)
    assert need > L.SD_ATTENTION_NOALLOC_SCRATCH_BYTES
    assert lib.sd_k_attention_noalloc(1, 8, 0, 0, 8, 2, 12, 3120, 128, 1, C.byref(seg), 8, None) == L.SD_ERR_WORKSPACE
    assert lib.sd_k_attention_noalloc(0, 8, 0, 0, 8, 1, 1, 8, 64, 1, C.byref(seg), 2, None) == L.SD_ERR_ARG   # fp32 split
    assert lib.sd_k_attention_noalloc(1, 8, 0, 0, 8, 1, 1, 8, 48, 1, C.byref(seg), 1, None) == L.SD_ERR_SHAPE
    assert lib.sd_k_attention_noalloc(1, None, 0, 0, 8, 1, 1, 8, 64, 1, C.byref(seg), 1, None) == L.SD_ERR_ARG
    # the video step's own split (5 splits, 2 rows) fits
    assert lib.sd_k_attention_workspace_bytes(2, 12, 3120, 128, 5) <= L.SD_ATTENTION_NOALLOC_SCRATCH_BYTES


# ------------------------------------------------------------------ attention split plan (host only)
def _greedy_finish(jobs, slots):
    """Workgroups started in grid order on the earliest free of `slots`
    resident slots; jobs = list of (count, length)."""
    import heapq
    free = [0] * slots
    end = 0
    for n, length in jobs:
        for _ in range(n):
            t = heapq.heappop(free) + length
            heapq.heappush(free, t)
            end = max(end, t)
    return end


@pytest.mark.parametrize("H,uph,tiles,cap,slots", [(12, 50, 221, 8, 512), (12, 1, 10, 8, 512),
                                                   (40, 25, 221, 8, 512), (16, 8, 40, 8, 512),
                                                   (12, 25, 74, 8, 512), (12, 100, 221, 4, 512)])
def test_attention_split_plan(lib, H, uph, tiles, cap, slots):
    """The plan is within 5 % of the best greedy schedule over every
    (unsplit heads, splits) pair, never splits more than asked, and with few
    query tiles (fewer than the resident slots) splits every head."""
    ns, hf = C.c_int32(), C.c_int32()
    assert lib.sd_k_attention_pick_plan(H, uph, tiles, cap, slots, C.byref(ns), C.byref(hf)) == L.SD_OK
    ns, hf = ns.value, hf.value
    assert 1 <= ns <= cap and 0 <= hf < H

    def finish(h, s):
        return _greedy_finish([(h * uph, tiles), ((H - h) * uph * s, -(-tiles // s))], slots)

    best = min(finish(h, s) for h in range(H) for s in range(1, cap + 1))
    assert finish(hf, ns) <= 1.05 * best
    if H * uph <= slots:
        assert hf == 0
    if (H, uph, tiles) == (12, 50, 221):      # the 1.3B-shaped video step: 10 heads whole, 2 split in 5
        assert (hf, ns) == (10, 5)
