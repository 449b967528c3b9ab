// sd_vae_*: the Stream-VAE runtime (see include/sd_vae.h).  Per chunk the
// layers run in order on the caller's stream; each convolution reads its
// cache (the previous chunk's last two input frames) and then replaces it
// with the last two frames of its own input.
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
  void* cache;       // bf16 [2][H][W][cin]
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
  L[SD_VAE_E0] = {8, c.c1, -1, true, Tp, H, W, nullptr};
  L[SD_VAE_E1] = {c.c1, c.c2, 0, true, Tp, H / 2, W / 2, nullptr};
  L[SD_VAE_E2] = {c.c2, c.c3, 0, true, Tp, H / 4, W / 4, nullptr};
  L[SD_VAE_E3] = {c.c3, c.c3, 1, true, T, h, w, nullptr};
  L[SD_VAE_E_OUT] = {c.c3, z, -1, false, T, h, w, nullptr};
  L[SD_VAE_D0] = {z, c.c3, -1, true, T, h, w, nullptr};
  L[SD_VAE_D1] = {c.c3, c.c3, 3, true, Tp, H / 4, W / 4, nullptr};
  L[SD_VAE_D2] = {c.c3, c.c2, 2, true, Tp, H / 2, W / 2, nullptr};
  L[SD_VAE_D3] = {c.c2, c.c1, 2, true, Tp, H, W, nullptr};
  L[SD_VAE_D_OUT] = {c.c1, 3, -1, false, Tp, H, W, nullptr};
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// bytes of one activation buffer: the largest convolution input or output
size_t act_bytes(const VaeLayer* L) {
  size_t m = 0;
  for (int i = 0; i < SD_VAE_LAYERS; ++i) {
    const size_t pos = (size_t)L[i].T * L[i].H * L[i].W;
    m = std::max(m, pos * (size_t)std::max(L[i].cin, L[i].cout));
  }
  return align256(m * 2);
}

size_t cache_bytes(const VaeLayer& l) { return align256((size_t)2 * l.H * l.W * l.cin * 2); }

}  // namespace

struct sd_vae {
  sd_vae_config cfg;
  sd_vae_weights w;
  VaeLayer L[SD_VAE_LAYERS];
  hipStream_t st = nullptr;
  void* act[2] = {nullptr, nullptr};
  void* cache_base = nullptr;
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

// layers [first, last] on the channels-last chunk in act[cur] (shape T, H, W,
// C); the last layer is narrow and writes fp32 channels-first to out
sd_status run_layers(sd_vae* v, int first, int last, int cur, int T, int H, int W, int C, float* out) {
  for (int li = first; li <= last; ++li) {
    VaeLayer& l = v->L[li];
    int in = cur;
    if (l.mode >= 0) {
      VHIP(sdk::resample(v->st, v->act[cur], v->act[cur ^ 1], T, H, W, C, l.mode));
      in = cur ^ 1;
    }
    sdk::ConvArgs a;
    a.x = (const bf16*)v->act[in];
    a.cache = (const bf16*)l.cache;
    a.w = (const bf16*)v->w.w[li];
    a.b = (const bf16*)v->w.b[li];
    a.y = li == last ? nullptr : (bf16*)v->act[in ^ 1];
    a.ycf = li == last ? out : nullptr;
    a.T = l.T;
    a.H = l.H;
    a.W = l.W;
    a.Cin = l.cin;
    a.Cout = l.cout;
    VHIP(sdk::conv3d(v->st, a));
    // this chunk's last two input frames become the layer's cache
    const size_t frame = (size_t)l.H * l.W * l.cin;
    VHIP(hipMemcpyAsync(l.cache, (const char*)v->act[in] + (size_t)(l.T - 2) * frame * 2, 2 * frame * 2,
                        hipMemcpyDeviceToDevice, v->st));
    if (li == last) break;
    if (l.norm) VHIP(sdk::norm_silu(v->st, v->act[in ^ 1], v->w.g[li], (int64_t)l.T * l.H * l.W, l.cout, 1e-6f));
    cur = in ^ 1;
    T = l.T;
    H = l.H;
    W = l.W;
    C = l.cout;
  }
  return SD_OK;
}

}  // namespace

extern "C" {

size_t sd_vae_workspace_bytes(const sd_vae_config* cfg) {
  if (!cfg || validate(*cfg, nullptr) != SD_OK) return 0;
  VaeLayer L[SD_VAE_LAYERS];
  layers_of(*cfg, L);
  size_t n = 2 * act_bytes(L);
  for (int i = 0; i < SD_VAE_LAYERS; ++i) n += cache_bytes(L[i]);
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
  const size_t ab = act_bytes(v->L);
  v->act[0] = p;
  v->act[1] = p + ab;
  p += 2 * ab;
  v->cache_base = p;
  for (int i = 0; i < SD_VAE_LAYERS; ++i) {
    v->L[i].cache = p;
    p += cache_bytes(v->L[i]);
  }
  v->cache_total = (size_t)(p - (char*)v->cache_base);
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
  VHIP(sdk::fill_zero(v->st, v->cache_base, v->cache_total));
  return SD_OK;
}

sd_status sd_vae_encode(sd_vae* v, const float* pixels, float* latent) {
  if (!v) return SD_ERR_ARG;
  if (!pixels || !latent) return set_err(v, SD_ERR_ARG, "null pixels or latent");
  const sd_vae_config& c = v->cfg;
  const int Tp = 2 * c.latent_t, H = 8 * c.latent_h, W = 8 * c.latent_w;
  VHIP(sdk::to_channels_last(v->st, pixels, v->act[0], Tp, 3, H * W, 8));
  return run_layers(v, SD_VAE_E0, SD_VAE_E_OUT, 0, Tp, H, W, 8, latent);
}

sd_status sd_vae_decode(sd_vae* v, const float* latent, float* pixels) {
  if (!v) return SD_ERR_ARG;
  if (!pixels || !latent) return set_err(v, SD_ERR_ARG, "null pixels or latent");
  const sd_vae_config& c = v->cfg;
  VHIP(sdk::to_channels_last(v->st, latent, v->act[0], c.latent_t, c.latent_c, c.latent_h * c.latent_w, c.latent_c));
  return run_layers(v, SD_VAE_D0, SD_VAE_D_OUT, 0, c.latent_t, c.latent_h, c.latent_w, c.latent_c, pixels);
}

void sd_vae_destroy(sd_vae* v) { delete v; }

const char* sd_vae_last_error(const sd_vae* v) { return v ? v->err.c_str() : "null handle"; }

}  // extern "C"
