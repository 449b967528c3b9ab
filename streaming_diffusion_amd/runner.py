"""Thin driver around the C ABI: turns a workload configuration into an
sd_stream_config, places weights and workspace in device memory with torch,
and forwards push/step calls.  All computation happens in libsdstream.
"""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import _lib as L


def make_config(cfg) -> L.sd_stream_config:
    c = L.sd_stream_config()
    c.abi_version = L.SD_ABI_VERSION
    c.dtype = L.SD_DTYPE_BF16 if cfg.dtype == "bf16" else L.SD_DTYPE_F32
    c.latent_t, c.latent_c, c.latent_h, c.latent_w = cfg.latent_t, cfg.latent_c, cfg.latent_h, cfg.latent_w
    c.patch = cfg.patch
    c.n_blocks, c.d_model, c.n_heads, c.d_ffn = cfg.n_blocks, cfg.d_model, cfg.n_heads, cfg.d_ffn
    c.d_freq, c.ctx_len = cfg.d_freq, cfg.ctx_len
    c.n_slots = cfg.n_slots
    for i, k in enumerate(cfg.t_index):
        c.t_index[i] = int(k)
    c.chunks_per_step = cfg.chunks_per_step
    c.cfg_type = {"self": L.SD_CFG_SELF, "onetime": L.SD_CFG_ONETIME, "full": L.SD_CFG_FULL}[cfg.cfg_type]
    c.gamma, c.delta = cfg.gamma, cfg.delta
    c.sink_tokens = cfg.sink_tokens
    c.sink_entries = getattr(cfg, "sink_entries", 1) if cfg.sink_tokens else 0
    c.window_tokens = cfg.window_tokens
    c.sink_tau = cfg.sink_tau
    c.rope_reset, c.rope_base = cfg.rope_reset, cfg.rope_base
    c.n_train_steps, c.beta_start, c.beta_end = cfg.n_train_steps, cfg.beta_start, cfg.beta_end
    c.ssf_on = int(cfg.ssf_on)
    c.ssf_kind = L.SD_SSF_U8 if cfg.ssf_kind == "u8" else L.SD_SSF_LATENT
    if cfg.ssf_on and cfg.ssf_kind == "u8":
        c.ssf_h, c.ssf_w, c.ssf_c = cfg.ssf_shape
    c.ssf_eta, c.max_skip_frame = cfg.ssf_eta, cfg.max_skip_frame
    c.motion_on, c.motion_k = int(cfg.motion_on), cfg.motion_k
    c.motion_lambda, c.s_min, c.s_max, c.motion_sigma = cfg.motion_lambda, cfg.s_min, cfg.s_max, cfg.motion_sigma
    c.batch_attn = int(cfg.batch_attn)
    c.sampler = {"ddim": L.SD_SAMPLER_DDIM, "lcm": L.SD_SAMPLER_LCM}[cfg.sampler]
    c.kv_recompute = int(cfg.kv_recompute)
    return c


def torch_dtype(cfg):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def upload_weights(cfg, weights: dict, device="cuda") -> dict:
    """Host float32 arrays (already bf16-representable for bf16 configs) ->
    contiguous device tensors of the config's element type."""
    dt = torch_dtype(cfg)
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(device=device).to(dt).contiguous()
            for k, v in weights.items()}


def random_device_weights(cfg, seed: int = 0, std: float = 0.02, device="cuda") -> dict:
    """N(0, std) weights drawn on the device (for timing runs of large shapes)."""
    from workloads.gen import param_specs
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    dt = torch_dtype(cfg)
    out = {}
    for name, shape in param_specs(cfg):
        out[name] = (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std).to(dt)
    return out


def ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


class StreamRunner:
    """One sd_stream handle plus the device memory it needs."""

    def __init__(self, cfg, dev_weights: dict, device="cuda", stream=None):
        self.lib = L.load()
        self.cfg = cfg
        self.device = device
        self.c = make_config(cfg)
        ws = self.lib.sd_stream_workspace_bytes(C.byref(self.c))
        if ws == 0:
            raise L.SDError(L.SD_ERR_ARG, "invalid configuration")
        self.ws_bytes = ws
        self._ws = torch.empty(ws + 256, dtype=torch.uint8, device=device)
        base = ptr(self._ws)
        self.ws_ptr = (base + 255) & ~255
        self.weights = dev_weights
        self.w = L.sd_weights()
        for name in L.WEIGHT_FIELDS:
            t = dev_weights.get(name)
            setattr(self.w, name, ptr(t) if t is not None else None)
        self.stream = stream if stream is not None else torch.cuda.current_stream(device)
        h = C.c_void_p()
        L.check(self.lib.sd_stream_create(C.byref(self.c), C.byref(self.w), C.c_void_p(self.ws_ptr), ws,
                                          C.c_void_p(self.stream.cuda_stream), C.byref(h)))
        self.h = h
        self.lat_shape = (cfg.latent_t, cfg.latent_c, cfg.latent_h, cfg.latent_w)
        # a step emits B latents ([B][T][C][H][W]); with B = 1 the leading axis is dropped
        self.out_shape = self.lat_shape if cfg.chunks_per_step == 1 else (cfg.chunks_per_step,) + self.lat_shape
        self.out = torch.empty(self.out_shape, dtype=torch.float32, device=device)

    def close(self):
        if getattr(self, "h", None):
            self.lib.sd_stream_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_context(self, ctx_pos, ctx_neg=None):
        self._ctx = (ctx_pos, ctx_neg)
        L.check(self.lib.sd_stream_set_context(self.h, C.c_void_p(ptr(ctx_pos)), C.c_void_p(ptr(ctx_neg))), self.h)

    def push(self, x0, noise, ssf_frame=None, u: float = 0.0) -> L.sd_push_info:
        info = L.sd_push_info()
        L.check(self.lib.sd_stream_push_frame(self.h, C.c_void_p(ptr(x0)), C.c_void_p(ptr(noise)),
                                              C.c_void_p(ptr(ssf_frame)), float(u), C.byref(info)), self.h)
        return info

    def step(self, out=None, chunks=None) -> L.sd_step_info:
        """Advance one step with a group of `chunks` entering (default B);
        the emitted latents (info.n_out of them) land in out (default
        self.out), shaped [B][T][C][H][W] (no leading axis when B = 1)."""
        info = L.sd_step_info()
        o = self.out if out is None else out
        if o.numel() < int(np.prod(self.out_shape)):
            raise ValueError("out holds fewer elements than the B latents a step emits")
        if chunks is None:
            L.check(self.lib.sd_stream_step(self.h, C.c_void_p(ptr(o)), C.byref(info)), self.h)
        else:
            L.check(self.lib.sd_stream_step_chunks(self.h, int(chunks), C.c_void_p(ptr(o)), C.byref(info)), self.h)
        return info

    def kv_reset(self):
        L.check(self.lib.sd_stream_kv_reset(self.h), self.h)

    def set_io_stream(self, stream=None):
        """Run pushes on `stream` (a torch.cuda.Stream on which the caller also
        produces the inputs), overlapped with the steps; None: the main stream."""
        self.io_stream = stream
        L.check(self.lib.sd_stream_set_io_stream(self.h, C.c_void_p(stream.cuda_stream if stream else None)), self.h)

    def set_graph(self, enable: bool = True):
        """Replay each step as a captured HIP graph (the runner's stream must
        be a created stream, not the default one)."""
        L.check(self.lib.sd_stream_set_graph(self.h, int(enable)), self.h)

    def graph_stats(self):
        cap, rep = C.c_int64(), C.c_int64()
        L.check(self.lib.sd_stream_graph_stats(self.h, C.byref(cap), C.byref(rep)), self.h)
        return cap.value, rep.value

    def sink_info(self) -> L.sd_sink_info:
        info = L.sd_sink_info()
        L.check(self.lib.sd_stream_sink_info(self.h, C.byref(info)), self.h)
        return info

    def profile(self, kinds):
        """Time every launch of the named kinds (see _lib.PROF_KINDS) with HIP events."""
        mask = 0
        for k in kinds:
            mask |= 1 << L.PROF_KINDS.index(k)
        L.check(self.lib.sd_stream_profile(self.h, mask), self.h)

    def profile_read(self) -> dict:
        """Per-kind totals since the last read: {kind: dict(launches, ms, flops, bytes)}."""
        arr = (L.sd_kernel_stat * len(L.PROF_KINDS))()
        n = C.c_int32()
        L.check(self.lib.sd_stream_profile_read(self.h, arr, len(L.PROF_KINDS), C.byref(n)), self.h)
        return {L.PROF_KINDS[a.kind]: dict(launches=a.launches, ms=a.ms, flops=a.flops, bytes=a.bytes)
                for a in arr[:n.value]}

    def buffer(self, which: int, dtype, shape):
        """A torch view of an internal device buffer (no copy)."""
        p = C.c_void_p()
        n = C.c_size_t()
        L.check(self.lib.sd_stream_buffer(self.h, which, C.byref(p), C.byref(n)), self.h)
        count = int(np.prod(shape))
        esz = torch.tensor([], dtype=dtype).element_size()
        if count * esz > n.value:
            raise ValueError("view larger than the buffer")
        return _wrap_device(p.value, dtype, shape, self.device, self._ws)


def _wrap_device(addr, dtype, shape, device, owner):
    """View device memory at addr (inside owner's allocation) as a tensor."""
    base = owner.data_ptr()
    off = addr - base
    esz = torch.tensor([], dtype=dtype).element_size()
    count = int(np.prod(shape))
    if off < 0 or off + count * esz > owner.numel() * owner.element_size():
        raise ValueError("address outside the workspace")
    return owner[off:off + count * esz].view(dtype).view(*shape)


# --------------------------------------------------------------------------
# Stream-VAE
# --------------------------------------------------------------------------
def make_vae_config(vcfg) -> "L.sd_vae_config":
    c = L.sd_vae_config()
    c.abi_version = L.SD_VAE_ABI_VERSION
    c.latent_t, c.latent_c, c.latent_h, c.latent_w = vcfg.latent_t, vcfg.latent_c, vcfg.latent_h, vcfg.latent_w
    c.c1, c.c2, c.c3 = vcfg.c1, vcfg.c2, vcfg.c3
    return c


def upload_vae_weights(vcfg, weights: dict, device="cuda") -> dict:
    """Host float32 arrays (bf16-representable) -> contiguous bf16 device tensors."""
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(device=device).to(torch.bfloat16).contiguous()
            for k, v in weights.items()}


class VAERunner:
    """Owns the workspace and weight table of one sd_vae; encode / decode take
    and return fp32 device tensors in the channels-first layouts."""

    def __init__(self, vcfg, dev_weights: dict, device="cuda", stream=None):
        self.lib = L.load()
        self.v = vcfg
        self.cfg = make_vae_config(vcfg)
        self.weights = dev_weights
        self.wt = L.sd_vae_weights()
        for i, name in enumerate(L.VAE_LAYER_NAMES):
            self.wt.w[i] = dev_weights[name + ".w"].data_ptr()
            self.wt.b[i] = dev_weights[name + ".b"].data_ptr()
            g = dev_weights.get(name + ".g")
            self.wt.g[i] = g.data_ptr() if g is not None else None
        nbytes = self.lib.sd_vae_workspace_bytes(C.byref(self.cfg))
        if nbytes == 0:
            raise ValueError("invalid Stream-VAE configuration")
        self.ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        base = self.ws.data_ptr()
        off = (-base) % 256
        self.h = C.c_void_p()
        s = stream.cuda_stream if stream is not None else torch.cuda.current_stream().cuda_stream
        L.check(self.lib.sd_vae_create(C.byref(self.cfg), C.byref(self.wt), C.c_void_p(base + off),
                                       C.c_size_t(nbytes), C.c_void_p(s), C.byref(self.h)))
        self.lat_shape = (vcfg.latent_t, vcfg.latent_c, vcfg.latent_h, vcfg.latent_w)
        self.pix_shape = (vcfg.frames, 3, vcfg.height, vcfg.width)

    def _check(self, code):
        if code != L.SD_OK:
            m = self.lib.sd_vae_last_error(self.h)
            raise L.SDError(code, m.decode() if m else "")

    def encode(self, pixels, out=None):
        if tuple(pixels.shape) != self.pix_shape or pixels.dtype != torch.float32 or not pixels.is_contiguous():
            raise ValueError(f"pixels must be contiguous fp32 {self.pix_shape}")
        out = torch.empty(self.lat_shape, dtype=torch.float32, device=pixels.device) if out is None else out
        self._check(self.lib.sd_vae_encode(self.h, C.c_void_p(pixels.data_ptr()), C.c_void_p(out.data_ptr())))
        return out

    def decode(self, latent, out=None):
        if tuple(latent.shape) != self.lat_shape or latent.dtype != torch.float32 or not latent.is_contiguous():
            raise ValueError(f"latent must be contiguous fp32 {self.lat_shape}")
        out = torch.empty(self.pix_shape, dtype=torch.float32, device=latent.device) if out is None else out
        self._check(self.lib.sd_vae_decode(self.h, C.c_void_p(latent.data_ptr()), C.c_void_p(out.data_ptr())))
        return out

    def reset(self):
        self._check(self.lib.sd_vae_reset(self.h))

    def close(self):
        if self.h:
            self.lib.sd_vae_destroy(self.h)
            self.h = C.c_void_p()
