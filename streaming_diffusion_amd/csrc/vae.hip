// sd_vae_*: the Stream-VAE runtime (see include/sd_vae.h).  Per chunk the
// layers run in order on the caller's stream.  Every layer owns two input
// buffers and uses them on alternate chunks: its convolution reads the
// chunk's frames from one and the previous chunk's last two input frames --
// the layer's cache -- straight from the other, so no frames are copied.
// The layer before writes (or resamples) into the buffer of this chunk's
// parity.  Activations, caches and the
// convolution weights (copied at create from the caller's bf16) are fp16:
// the chain stores its activations nine times on the decoder path, and
// fp16's three extra mantissa bits keep the accumulated rounding an order
// below bf16's at the same matrix-core rate (all values are bounded: inputs
// of unit scale, RMS-normalised activations, unit-gain convolutions).
#include <algorithm>
#include <cstring>
#include <string>

#include "../../include/sd_vae.h"
#include "kernels.h"

namespace {

struct VaeLayer {
  int cin, cout;
  int mode;          // resampling of the layer's input: -1 none, else sdk::resample's mode
  bool norm;
  int T, H, W;       // shape of the convolution's input (after resampling)
  bool up;           // input kept at H/2 x W/2, upsampled 2x2 by the convolution's reads
  void* in[2];       // fp16 [T][H][W][cin] (H/2, W/2 with up): this chunk's input / the previous chunk's
  int par;           // which of in[] the next chunk uses
  void* w16;         // fp16 copy of the weights [cout][27 cin]
};

bool width_ok(int c) { return c == 16 || c == 32 || c == 64 || c == 128 || c == 256; }

int validate(const sd_vae_config& c, std::string* err) {
  auto fail = [&](const char* m) {
    if (err) *err = m;
    return (int)SD_ERR_ARG;
  };
  if (c.abi_version != SD_VAE_ABI_VERSION) return fail("abi_version mismatch");
  if (c.latent_t < 2) return fail("latent_t must be at least 2 (the caches hold two frames)");
  if (c.latent_c < 8 || c.latent_c > 16 || (c.latent_c & 7)) return fail("latent_c must be 8 or 16");
  if (c.latent_h < 1 || c.latent_w < 1 || c.latent_h > 512 || c.latent_w > 512) return fail("latent grid out of range");
  if (!width_ok(c.c1) || !width_ok(c.c2) || !width_ok(c.c3)) return fail("c1, c2, c3 must be 16, 32, 64, 128 or 256");
  return SD_OK;
}

void layers_of(const sd_vae_config& c, VaeLayer* L) {
  const int T = c.latent_t, h = c.latent_h, w = c.latent_w, z = c.latent_c;
  const int Tp = 2 * T, H = 8 * h, W = 8 * w;
  L[SD_VAE_E0] = {8, c.c1, -1, true, Tp, H, W, false, {nullptr, nullptr}, 0, nullptr};
  L[SD_VAE_E1] = {c.c1, c.c2, 0, true, Tp, H / 2, W / 2, false, {nullptr, nullptr}, 0, nullptr};
  L[SD_VAE_E2] = {c.c2, c.c3, 0, true, Tp, H / 4, W / 4, false, {nullptr, nullptr}, 0, nullptr};
  L[SD_VAE_E3] = {c.c3, c.c3, 1, true, T, h, w, false, {nullptr, nullptr}, 0, nullptr};
  L[SD_VAE_E_OUT] = {c.c3, z, -1, false, T, h, w, false, {nullptr, nullptr}, 0, nullptr};
  L[SD_VAE_D0] = {z, c.c3, -1, true, T, h, w, false, {nullptr, nullptr}, 0, nullptr};
  L[SD_VAE_D1] = {c.c3, c.c3, 3, true, Tp, H / 4, W / 4, false, {nullptr, nullptr}, 0, nullptr};
  L[SD_VAE_D2] = {c.c3, c.c2, 2, true, Tp, H / 2, W / 2, false, {nullptr, nullptr}, 0, nullptr};
  L[SD_VAE_D3] = {c.c2, c.c1, 2, true, Tp, H, W, false, {nullptr, nullptr}, 0, nullptr};
  L[SD_VAE_D_OUT] = {c.c1, 3, -1, false, Tp, H, W, false, {nullptr, nullptr}, 0, nullptr};
  // 2x2 nearest upsampling folded into the next convolution's input reads
  // where its kernel can do it: the layer stores its input at half size
  for (int i = 0; i < SD_VAE_LAYERS; ++i)
    L[i].up = L[i].mode == 2 && sdk::conv3d_upsample_ok(L[i].T, L[i].H, L[i].W, L[i].cin, L[i].cout);
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// bytes of the staging buffer: the largest convolution output that is
// resampled before the next layer
size_t act_bytes(const VaeLayer* L) {
  size_t m = 0;
  for (int i = 0; i + 1 < SD_VAE_LAYERS; ++i)
    if (L[i + 1].mode >= 0 && !L[i + 1].up) m = std::max(m, (size_t)L[i].T * L[i].H * L[i].W * L[i].cout);
  return align256(m * 2);
}

size_t input_frame(const VaeLayer& l) { return (size_t)(l.up ? l.H / 2 : l.H) * (l.up ? l.W / 2 : l.W) * l.cin; }
size_t input_bytes(const VaeLayer& l) { return align256((size_t)l.T * input_frame(l) * 2); }
size_t weight_bytes(const VaeLayer& l) { return align256((size_t)27 * l.cin * l.cout * 2); }

}  // namespace

struct sd_vae {
  sd_vae_config cfg;
  sd_vae_weights w;
  VaeLayer L[SD_VAE_LAYERS];
  hipStream_t st = nullptr;
  void* act = nullptr;             // staging of a convolution output that is resampled
  void* cache_base = nullptr;      // the layers' input buffers
  size_t cache_total = 0;
  std::string err;
};

namespace {

sd_status set_err(sd_vae* v, sd_status code, const std::string& m) {
  if (v) v->err = m;
  return code;
}

#define VHIP(expr)                                                                  \
  do {                                                                              \
    hipError_t _e = (expr);                                                         \
    if (_e != hipSuccess) return set_err(v, SD_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(_e)); \
  } while (0)

// layers [first, last] on the chunk already in L[first].in[par] (16-bit
// channels-last); the last layer is narrow and writes fp32 channels-first to
// out
sd_status run_layers(sd_vae* v, int first, int last, float* out) {
  for (int li = first; li <= last; ++li) {
    VaeLayer& l = v->L[li];
    VaeLayer* nx = li < last ? &v->L[li + 1] : nullptr;
    // this layer's output: the next layer's input buffer of this chunk, or
    // the staging buffer when the next layer resamples it first
    const bool stage = nx && nx->mode >= 0 && !nx->up;
    void* dst = nx ? (stage ? v->act : nx->in[nx->par]) : nullptr;
    const size_t frame = input_frame(l);
    sdk::ConvArgs a;
    a.up = l.up;
    a.x = (const bf16*)l.in[l.par];
    a.cache = (const bf16*)((const char*)l.in[l.par ^ 1] + (size_t)(l.T - 2) * frame * 2);
    a.w = (const bf16*)l.w16;
    a.h16 = true;
    a.b = (const bf16*)v->w.b[li];
    a.y = (bf16*)dst;
    a.ycf = nx ? nullptr : out;
    a.T = l.T;
    a.H = l.H;
    a.W = l.W;
    a.Cin = l.cin;
    a.Cout = l.cout;
    VHIP(sdk::conv3d(v->st, a));
    // the input just read is the next chunk's cache
    l.par ^= 1;
    if (!nx) break;
    if (l.norm && stage && nx->mode <= 1) {
      // the encoder's norm and pooling in one pass: only the pooled values are written
      VHIP(sdk::norm_silu_pool(v->st, v->act, v->w.g[li], nx->in[nx->par], l.T, l.H, l.W, l.cout, nx->mode == 1,
                               1e-6f, true));
      continue;
    }
    if (l.norm)
      VHIP(sdk::norm_silu(v->st, dst, v->w.g[li], (int64_t)l.T * l.H * l.W, l.cout, 1e-6f, true));
    if (stage) VHIP(sdk::resample(v->st, v->act, nx->in[nx->par], l.T, l.H, l.W, l.cout, nx->mode, true));
  }
  return SD_OK;
}

}  // namespace

extern "C" {

size_t sd_vae_workspace_bytes(const sd_vae_config* cfg) {
  if (!cfg || validate(*cfg, nullptr) != SD_OK) return 0;
  VaeLayer L[SD_VAE_LAYERS];
  layers_of(*cfg, L);
  size_t n = act_bytes(L);
  for (int i = 0; i < SD_VAE_LAYERS; ++i) n += 2 * input_bytes(L[i]) + weight_bytes(L[i]);
  return n;
}

sd_status sd_vae_create(const sd_vae_config* cfg, const sd_vae_weights* w, void* workspace, size_t workspace_bytes,
                        void* hip_stream, sd_vae** out) {
  if (!cfg || !w || !out) return SD_ERR_ARG;
  *out = nullptr;
  std::string err;
  if (validate(*cfg, &err) != SD_OK) return SD_ERR_ARG;
  for (int i = 0; i < SD_VAE_LAYERS; ++i) {
    const bool norm = i != SD_VAE_E_OUT && i != SD_VAE_D_OUT;
    if (!w->w[i] || !w->b[i] || (norm && !w->g[i])) return SD_ERR_ARG;
    if (((uintptr_t)w->w[i] | (uintptr_t)w->b[i] | (uintptr_t)(norm ? w->g[i] : nullptr)) & 15) return SD_ERR_ARG;
  }
  const size_t need = sd_vae_workspace_bytes(cfg);
  if (!workspace || ((uintptr_t)workspace & 255) || workspace_bytes < need) return SD_ERR_WORKSPACE;
  sd_vae* v = new sd_vae();
  v->cfg = *cfg;
  v->w = *w;
  v->st = (hipStream_t)hip_stream;
  layers_of(*cfg, v->L);
  char* p = (char*)workspace;
  v->act = p;
  p += act_bytes(v->L);
  v->cache_base = p;
  for (int i = 0; i < SD_VAE_LAYERS; ++i)
    for (int k = 0; k < 2; ++k) {
      v->L[i].in[k] = p;
      p += input_bytes(v->L[i]);
    }
  v->cache_total = (size_t)(p - (char*)v->cache_base);
  for (int i = 0; i < SD_VAE_LAYERS; ++i) {
    v->L[i].w16 = p;
    p += weight_bytes(v->L[i]);
    if (sdk::cast_to_h16(v->st, w->w[i], v->L[i].w16, (int64_t)27 * v->L[i].cin * v->L[i].cout) != hipSuccess) {
      delete v;
      return SD_ERR_HIP;
    }
  }
  const sd_status r = sd_vae_reset(v);
  if (r != SD_OK) {
    delete v;
    return r;
  }
  *out = v;
  return SD_OK;
}

sd_status sd_vae_reset(sd_vae* v) {
  if (!v) return SD_ERR_ARG;
  // both input buffers of every layer: the first chunk's caches read zeros
  VHIP(sdk::fill_zero(v->st, v->cache_base, v->cache_total));
  for (int i = 0; i < SD_VAE_LAYERS; ++i) v->L[i].par = 0;
  return SD_OK;
}

sd_status sd_vae_encode(sd_vae* v, const float* pixels, float* latent) {
  if (!v) return SD_ERR_ARG;
  if (!pixels || !latent) return set_err(v, SD_ERR_ARG, "null pixels or latent");
  const sd_vae_config& c = v->cfg;
  const int Tp = 2 * c.latent_t, H = 8 * c.latent_h, W = 8 * c.latent_w;
  VaeLayer& l0 = v->L[SD_VAE_E0];
  VHIP(sdk::to_channels_last(v->st, pixels, l0.in[l0.par], Tp, 3, H * W, 8, true));
  return run_layers(v, SD_VAE_E0, SD_VAE_E_OUT, latent);
}

sd_status sd_vae_decode(sd_vae* v, const float* latent, float* pixels) {
  if (!v) return SD_ERR_ARG;
  if (!pixels || !latent) return set_err(v, SD_ERR_ARG, "null pixels or latent");
  const sd_vae_config& c = v->cfg;
  VaeLayer& l0 = v->L[SD_VAE_D0];
  VHIP(sdk::to_channels_last(v->st, latent, l0.in[l0.par], c.latent_t, c.latent_c, c.latent_h * c.latent_w,
                             c.latent_c, true));
  return run_layers(v, SD_VAE_D0, SD_VAE_D_OUT, pixels);
}

void sd_vae_destroy(sd_vae* v) { delete v; }

const char* sd_vae_last_error(const sd_vae* v) { return v ? v->err.c_str() : "null handle"; }

}  // extern "C"
