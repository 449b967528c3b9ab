"""ctypes binding of libsdstream.so: the C ABI of include/sd_stream.h and
include/sd_kernels.h with the same names.  Argument marshalling only.

Loading fails loudly when the library has not been built: there is no
fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsdstream.so")
STATE_LIB_PATH = os.path.join(PKG, "libsdstate.so")

SD_ABI_VERSION = 4
SD_MAX_SLOTS = 8
SD_MAX_ROWS = 40
SD_MAX_SINK = 8
SD_ATTENTION_NOALLOC_SCRATCH_BYTES = 128 << 20

SD_OK, SD_ERR_ARG, SD_ERR_SHAPE, SD_ERR_STATE, SD_ERR_WORKSPACE, SD_ERR_HIP, SD_ERR_NOT_READY = 0, -1, -2, -3, -4, -5, -6
STATUS_NAMES = {0: "SD_OK", -1: "SD_ERR_ARG", -2: "SD_ERR_SHAPE", -3: "SD_ERR_STATE", -4: "SD_ERR_WORKSPACE",
                -5: "SD_ERR_HIP", -6: "SD_ERR_NOT_READY"}
SD_DTYPE_F32, SD_DTYPE_BF16 = 0, 1
SD_CFG_SELF, SD_CFG_ONETIME, SD_CFG_FULL = 0, 1, 2
SD_SSF_U8, SD_SSF_LATENT = 0, 1
SD_SAMPLER_DDIM, SD_SAMPLER_LCM = 0, 1
SD_BUF_EPS, SD_BUF_RING_K, SD_BUF_RING_V, SD_BUF_SINK_K, SD_BUF_SINK_V, SD_BUF_RESID, SD_BUF_MOD = range(7)


class sd_stream_config(C.Structure):
    _fields_ = [
        ("abi_version", C.c_uint32), ("dtype", C.c_int32),
        ("latent_t", C.c_int32), ("latent_c", C.c_int32), ("latent_h", C.c_int32), ("latent_w", C.c_int32),
        ("patch", C.c_int32),
        ("n_blocks", C.c_int32), ("d_model", C.c_int32), ("n_heads", C.c_int32), ("d_ffn", C.c_int32),
        ("d_freq", C.c_int32), ("ctx_len", C.c_int32),
        ("n_slots", C.c_int32), ("t_index", C.c_int32 * SD_MAX_SLOTS), ("chunks_per_step", C.c_int32),
        ("cfg_type", C.c_int32), ("gamma", C.c_double), ("delta", C.c_double),
        ("sink_tokens", C.c_int32), ("sink_entries", C.c_int32), ("window_tokens", C.c_int32),
        ("sink_tau", C.c_double), ("rope_reset", C.c_int32), ("rope_base", C.c_double),
        ("n_train_steps", C.c_int32), ("beta_start", C.c_double), ("beta_end", C.c_double),
        ("ssf_on", C.c_int32), ("ssf_kind", C.c_int32), ("ssf_h", C.c_int32), ("ssf_w", C.c_int32),
        ("ssf_c", C.c_int32), ("ssf_eta", C.c_double), ("max_skip_frame", C.c_int32),
        ("motion_on", C.c_int32), ("motion_k", C.c_int32), ("motion_lambda", C.c_double), ("s_min", C.c_double),
        ("s_max", C.c_double), ("motion_sigma", C.c_double), ("batch_attn", C.c_int32),
        ("sampler", C.c_int32), ("kv_recompute", C.c_int32),
    ]


WEIGHT_FIELDS = ["t_w1", "t_b1", "t_w2", "t_b2", "mod_w", "mod_b", "blk_mod", "pe_w", "pe_b", "qkv_w", "qkv_b",
                 "o_w", "o_b", "cq_w", "cq_b", "ckv_w", "ckv_b", "co_w", "co_b", "f1_w", "f1_b", "f2_w", "f2_b",
                 "fin_w", "fin_b", "head_w", "head_b"]


class sd_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in WEIGHT_FIELDS]


class sd_push_info(C.Structure):
    _fields_ = [("skipped", C.c_int32), ("t0", C.c_int32), ("frame_id", C.c_int64), ("sim", C.c_double),
                ("p", C.c_double), ("d", C.c_double), ("s", C.c_double), ("taus", C.c_int32 * SD_MAX_SLOTS)]


class sd_step_info(C.Structure):
    _fields_ = [("step", C.c_int64), ("has_output", C.c_int32), ("rows", C.c_int32), ("frame_id", C.c_int64),
                ("kv_ptr", C.c_int32), ("kv_valid", C.c_int32), ("sink_count", C.c_int32), ("rope_next", C.c_int32),
                ("n_out", C.c_int32)]


class sd_sink_info(C.Structure):
    _fields_ = [("evaluated", C.c_int32), ("entry", C.c_int32), ("refreshed", C.c_int32), ("sim", C.c_float)]


class sd_kernel_stat(C.Structure):
    _fields_ = [("kind", C.c_int32), ("reserved", C.c_int32), ("launches", C.c_int64), ("ms", C.c_double),
                ("flops", C.c_double), ("bytes", C.c_double)]


PROF_KINDS = ["attn_self", "attn_cross", "gemm_qkv", "gemm_o", "gemm_ffn1", "gemm_ffn2", "gemm_cross", "other",
              "ln_mod", "gemv", "kv_cache", "epilogue", "controls", "attn_combine"]


class sd_kv_segment(C.Structure):
    _fields_ = [("k", C.c_void_p), ("vt", C.c_void_p), ("k_head_stride", C.c_int64), ("vt_head_stride", C.c_int64),
                ("k_row_stride", C.c_int64), ("vt_row_stride", C.c_int64), ("cap", C.c_int32), ("start", C.c_int32),
                ("count", C.c_int32), ("wrap", C.c_int32)]


SD_EPI_STORE, SD_EPI_GELU, SD_EPI_GATE_RESID, SD_EPI_RESID, SD_EPI_PATCH, SD_EPI_QKV, SD_EPI_HEAD = range(7)
SD_EPI_F32 = 8


class sd_gemm_epi(C.Structure):
    _fields_ = [("mode", C.c_int32), ("bias", C.c_void_p), ("out", C.c_void_p), ("ldo", C.c_int32),
                ("resid", C.c_void_p), ("mod", C.c_void_p), ("blk", C.c_void_p), ("gate_off", C.c_int32),
                ("six_d", C.c_int32), ("L", C.c_int32), ("q", C.c_void_p), ("k", C.c_void_p), ("vt", C.c_void_p),
                ("kstride", C.c_int32), ("krows", C.c_int32), ("H", C.c_int32), ("hd", C.c_int32),
                ("rope", C.c_int32), ("Hp", C.c_int32), ("Wp", C.c_int32), ("rope_table", C.c_void_p),
                ("rope_positions", C.c_int32), ("t0", C.c_int32 * SD_MAX_ROWS), ("eps", C.c_void_p),
                ("C", C.c_int32), ("Hl", C.c_int32), ("Wl", C.c_int32), ("p", C.c_int32), ("T", C.c_int32),
                ("f16", C.c_int32), ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t),
                ("wpack", C.c_void_p), ("ln_out", C.c_void_p), ("ln_mod", C.c_void_p), ("ln_blk", C.c_void_p),
                ("ln_shift_off", C.c_int32), ("ln_scale_off", C.c_int32), ("ln_six_d", C.c_int32),
                ("ln_form", C.c_int32), ("sm_out", C.c_void_p), ("sm_bias", C.c_void_p), ("sm_heads", C.c_int32),
                ("sm_cp", C.c_int32)]


SD_LN_PLAIN, SD_LN_F16, SD_LN_SPLIT = 0, 1, 2


SD_VAE_ABI_VERSION = 1
SD_VAE_LAYERS = 10
VAE_LAYER_NAMES = ["e0", "e1", "e2", "e3", "e_out", "d0", "d1", "d2", "d3", "d_out"]


class sd_vae_config(C.Structure):
    _fields_ = [("abi_version", C.c_uint32), ("latent_t", C.c_int32), ("latent_c", C.c_int32),
                ("latent_h", C.c_int32), ("latent_w", C.c_int32), ("c1", C.c_int32), ("c2", C.c_int32),
                ("c3", C.c_int32)]


class sd_vae_weights(C.Structure):
    _fields_ = [("w", C.c_void_p * SD_VAE_LAYERS), ("b", C.c_void_p * SD_VAE_LAYERS),
                ("g", C.c_void_p * SD_VAE_LAYERS)]


# name -> (restype, argtypes)
SIGNATURES = {
    "sd_stream_workspace_bytes": (C.c_size_t, [C.POINTER(sd_stream_config)]),
    "sd_stream_create": (C.c_int, [C.POINTER(sd_stream_config), C.POINTER(sd_weights), C.c_void_p, C.c_size_t,
                                   C.c_void_p, C.POINTER(C.c_void_p)]),
    "sd_stream_set_context": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p]),
    "sd_stream_push_frame": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_double,
                                       C.POINTER(sd_push_info)]),
    "sd_stream_set_io_stream": (C.c_int, [C.c_void_p, C.c_void_p]),
    "sd_stream_set_graph": (C.c_int, [C.c_void_p, C.c_int32]),
    "sd_stream_graph_stats": (C.c_int, [C.c_void_p, C.POINTER(C.c_int64), C.POINTER(C.c_int64)]),
    "sd_stream_step": (C.c_int, [C.c_void_p, C.c_void_p, C.POINTER(sd_step_info)]),
    "sd_stream_step_chunks": (C.c_int, [C.c_void_p, C.c_int32, C.c_void_p, C.POINTER(sd_step_info)]),
    "sd_stream_kv_reset": (C.c_int, [C.c_void_p]),
    "sd_stream_sink_info": (C.c_int, [C.c_void_p, C.POINTER(sd_sink_info)]),
    "sd_stream_buffer": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_void_p), C.POINTER(C.c_size_t)]),
    "sd_stream_profile": (C.c_int, [C.c_void_p, C.c_uint32]),
    "sd_stream_profile_read": (C.c_int, [C.c_void_p, C.POINTER(sd_kernel_stat), C.c_int32, C.POINTER(C.c_int32)]),
    "sd_stream_destroy": (None, [C.c_void_p]),
    "sd_stream_last_error": (C.c_char_p, [C.c_void_p]),
    "sd_k_gemm": (C.c_int, [C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32,
                            C.c_int32, C.c_void_p]),
    "sd_k_gemm_resid": (C.c_int, [C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32,
                                  C.c_int32, C.c_void_p]),
    "sd_k_gemm_epi": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.POINTER(sd_gemm_epi),
                                C.c_void_p]),
    "sd_k_pack_weight_bytes": (C.c_size_t, [C.c_int32, C.c_int32]),
    "sd_k_pack_weight": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]),
    "sd_k_rope_table_pairs": (C.c_size_t, [C.c_int32, C.c_int32, C.c_int32, C.c_int32]),
    "sd_k_rope_tables": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_double, C.c_void_p]),
    "sd_k_ln_mod": (C.c_int, [C.c_int32, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p,
                              C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_void_p]),
    "sd_k_attention": (C.c_int, [C.c_int32, C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_int32, C.c_int32,
                                 C.c_int32, C.c_int32, C.c_int32, C.POINTER(sd_kv_segment), C.c_int32, C.c_void_p,
                                 C.c_size_t, C.c_void_p]),
    "sd_k_attention_workspace_bytes": (C.c_size_t, [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32]),
    "sd_k_attention_plan": (C.c_int, [C.c_int32, C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_int32, C.c_int32,
                                      C.c_int32, C.c_int32, C.c_int32, C.POINTER(sd_kv_segment), C.c_int32, C.c_int32,
                                      C.c_void_p, C.c_size_t, C.c_void_p]),
    "sd_k_attention_pick_plan": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                           C.POINTER(C.c_int32), C.POINTER(C.c_int32)]),
    "sd_k_attention_noalloc": (C.c_int, [C.c_int32, C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_int32,
                                         C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.POINTER(sd_kv_segment),
                                         C.c_int32, C.c_void_p]),
    "sd_k_ssf_sums": (C.c_int, [C.c_int32, C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p]),
    "sd_k_motion_sums": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_int64, C.c_void_p, C.c_void_p]),
    "sd_k_conv3d": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32,
                              C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_void_p]),
    "sd_k_conv3d_up2": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32,
                                  C.c_int32, C.c_int32, C.c_int32, C.c_void_p]),
    "sd_vae_workspace_bytes": (C.c_size_t, [C.POINTER(sd_vae_config)]),
    "sd_vae_create": (C.c_int, [C.POINTER(sd_vae_config), C.POINTER(sd_vae_weights), C.c_void_p, C.c_size_t,
                                C.c_void_p, C.POINTER(C.c_void_p)]),
    "sd_vae_encode": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p]),
    "sd_vae_decode": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p]),
    "sd_vae_reset": (C.c_int, [C.c_void_p]),
    "sd_vae_destroy": (None, [C.c_void_p]),
    "sd_vae_last_error": (C.c_char_p, [C.c_void_p]),
}

STATE_SIGNATURES = {
    "sdstate_validate": (C.c_int, [C.POINTER(sd_stream_config), C.c_char_p, C.c_int]),
    "sdstate_schedule": (None, [C.POINTER(sd_stream_config), C.POINTER(C.c_double), C.POINTER(C.c_double)]),
    "sdstate_taus_noise_rate": (None, [C.c_double, C.c_int, C.c_int, C.POINTER(C.c_int32)]),
    "sdstate_taus_t_index": (None, [C.POINTER(sd_stream_config), C.POINTER(C.c_int32)]),
    "sdstate_ssf_cosine": (C.c_double, [C.c_int64, C.c_int64, C.c_int64]),
    "sdstate_ssf_probability": (C.c_double, [C.c_double, C.c_double]),
    "sdstate_motion_distance": (C.c_double, [C.c_int64, C.c_int64]),
    "sdstate_motion_update": (C.c_double, [C.c_double, C.POINTER(C.c_double), C.c_int,
                                           C.POINTER(sd_stream_config)]),
}

_lib = None
_state = None


def _bind(lib, sigs):
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def load():
    """The HIP library.  Raises if it is missing: there is no CPU path."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libsdstream.so not found at {LIB_PATH}; build it with "
                               "`python -m streaming_diffusion_amd.build`")
        _lib = _bind(C.CDLL(LIB_PATH), SIGNATURES)
    return _lib


def load_state():
    """The host-only state module (no device code)."""
    global _state
    if _state is None:
        if not os.path.exists(STATE_LIB_PATH):
            raise RuntimeError(f"libsdstate.so not found at {STATE_LIB_PATH}; run the build first")
        _state = _bind(C.CDLL(STATE_LIB_PATH), STATE_SIGNATURES)
    return _state


class SDError(RuntimeError):
    def __init__(self, code, msg=""):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


def check(code, handle=None):
    if code != SD_OK:
        msg = ""
        if handle is not None:
            m = load().sd_stream_last_error(handle)
            msg = m.decode() if m else ""
        raise SDError(code, msg)
