// Host-side state machine; see host_state.h.  Built with -ffp-contract=off.
#include "host_state.h"

#include <cmath>
#include <cstdio>

namespace sd {

static int fail(std::string* err, int code, const char* msg) {
  if (err) *err = msg;
  return code;
}

int validate_config(const sd_stream_config& c, std::string* err) {
  if (c.abi_version != SD_ABI_VERSION) return fail(err, SD_ERR_ARG, "abi_version mismatch");
  if (c.dtype != SD_DTYPE_F32 && c.dtype != SD_DTYPE_BF16) return fail(err, SD_ERR_ARG, "dtype must be F32 or BF16");
  if (c.latent_t < 1 || c.latent_c < 1 || c.latent_h < 1 || c.latent_w < 1 || c.patch < 1)
    return fail(err, SD_ERR_SHAPE, "latent dims and patch must be >= 1");
  if (c.latent_t > 64) return fail(err, SD_ERR_SHAPE, "at most 64 latent frames per chunk");
  if (c.latent_h % c.patch || c.latent_w % c.patch) return fail(err, SD_ERR_SHAPE, "latent H/W must be multiples of patch");
  if ((c.patch * c.patch * c.latent_c) % 8) return fail(err, SD_ERR_SHAPE, "patch*patch*C must be a multiple of 8");
  if (c.n_blocks < 0 || c.d_model < 8 || c.n_heads < 1 || c.d_model % c.n_heads)
    return fail(err, SD_ERR_SHAPE, "d_model must be a positive multiple of n_heads");
  const int hd = c.d_model / c.n_heads;
  if (hd % 8 || hd > 128 || hd < 16) return fail(err, SD_ERR_SHAPE, "head dim must be a multiple of 8 in [16, 128]");
  if (c.d_model % 64) return fail(err, SD_ERR_SHAPE, "d_model must be a multiple of 64");
  if (c.d_model > 5120) return fail(err, SD_ERR_SHAPE, "d_model must be at most 5120");
  if (c.d_ffn < 8 || c.d_ffn % 64) return fail(err, SD_ERR_SHAPE, "d_ffn must be a positive multiple of 64");
  if (c.d_freq < 2 || c.d_freq % 8) return fail(err, SD_ERR_SHAPE, "d_freq must be a positive multiple of 8");
  if (c.ctx_len < 0 || c.ctx_len > 4096) return fail(err, SD_ERR_SHAPE, "ctx_len out of range");
  if (c.n_slots < 1 || c.n_slots > SD_MAX_SLOTS) return fail(err, SD_ERR_ARG, "n_slots out of range");
  if (c.chunks_per_step < 1 || c.chunks_per_step > SD_MAX_CHUNKS)
    return fail(err, SD_ERR_ARG, "chunks_per_step must be in [1, 8]");
  if (c.cfg_type != SD_CFG_SELF && c.cfg_type != SD_CFG_ONETIME && c.cfg_type != SD_CFG_FULL)
    return fail(err, SD_ERR_ARG, "unknown cfg_type");
  if (c.cfg_type != SD_CFG_SELF && c.ctx_len == 0)
    return fail(err, SD_ERR_ARG, "onetime-negative R-CFG and full CFG need a (negative) context");
  if (!std::isfinite(c.gamma) || !std::isfinite(c.delta)) return fail(err, SD_ERR_ARG, "gamma/delta must be finite");
  if (c.batch_attn != 0 && c.batch_attn != 1) return fail(err, SD_ERR_ARG, "batch_attn must be 0 or 1");
  if (c.sampler != SD_SAMPLER_DDIM && c.sampler != SD_SAMPLER_LCM) return fail(err, SD_ERR_ARG, "unknown sampler");
  if (c.kv_recompute != 0 && c.kv_recompute != 1) return fail(err, SD_ERR_ARG, "kv_recompute must be 0 or 1");
  if (c.batch_attn && c.cfg_type != SD_CFG_SELF)
    return fail(err, SD_ERR_ARG, "batch attention needs self-negative R-CFG (all rows under one prompt)");
  if (c.n_train_steps < 50 || c.n_train_steps > 100000) return fail(err, SD_ERR_ARG, "n_train_steps out of range");
  if (!(c.beta_start > 0) || !(c.beta_end > 0) || !(c.beta_end < 1)) return fail(err, SD_ERR_ARG, "betas out of range");
  if (!c.motion_on) {
    const int stride = c.n_train_steps / 50;
    for (int i = 0; i < c.n_slots; ++i) {
      const int t = (c.n_train_steps - 1) - stride * c.t_index[i];
      if (c.t_index[i] < 0 || t < 0 || t >= c.n_train_steps) return fail(err, SD_ERR_ARG, "t_index out of range");
    }
  }
  const int64_t L = tokens_per_chunk(c);
  if (L < 1 || L > (1 << 20)) return fail(err, SD_ERR_SHAPE, "tokens per chunk out of range");
  if (c.sink_tokens < 0 || c.window_tokens < 0) return fail(err, SD_ERR_ARG, "negative cache size");
  if (c.sink_tokens > 0) {
    if (c.sink_entries < 1 || c.sink_entries > SD_MAX_SINK || c.sink_tokens % c.sink_entries)
      return fail(err, SD_ERR_ARG, "sink_tokens must split evenly into 1..SD_MAX_SINK entries");
    if (c.sink_tokens / c.sink_entries > L) return fail(err, SD_ERR_ARG, "a sink entry cannot exceed one chunk");
    if (c.window_tokens < L) return fail(err, SD_ERR_ARG, "a sink needs a window of at least one chunk");
  }
  if (c.window_tokens > 0 && c.window_tokens < L) return fail(err, SD_ERR_ARG, "window must hold at least one chunk");
  if (c.dtype == SD_DTYPE_BF16 && (L % 8 || c.window_tokens % 8))
    return fail(err, SD_ERR_SHAPE, "bf16 streams need tokens per chunk and window in multiples of 8");
  if (c.dtype == SD_DTYPE_BF16 && hd != 32 && hd != 64 && hd != 128)
    return fail(err, SD_ERR_SHAPE, "bf16 streams need head dim 32, 64 or 128");
  if (c.dtype == SD_DTYPE_F32 && hd != 16 && hd != 32 && hd != 64 && hd != 128)
    return fail(err, SD_ERR_SHAPE, "fp32 streams need head dim 16, 32, 64 or 128");
  if (c.window_tokens > (1 << 22)) return fail(err, SD_ERR_ARG, "window too large");
  if (c.rope_reset < 0 || !(c.rope_base > 1.0)) return fail(err, SD_ERR_ARG, "rope_reset/rope_base out of range");
  if (c.ssf_on) {
    if (c.ssf_kind != SD_SSF_U8 && c.ssf_kind != SD_SSF_LATENT) return fail(err, SD_ERR_ARG, "unknown ssf_kind");
    if (c.ssf_kind == SD_SSF_U8 && (c.ssf_h < 1 || c.ssf_w < 1 || c.ssf_c < 1))
      return fail(err, SD_ERR_SHAPE, "ssf frame dims must be >= 1");
    if (!(c.ssf_eta < 1.0) || !(c.ssf_eta >= -1.0)) return fail(err, SD_ERR_ARG, "ssf_eta must be in [-1, 1)");
    if (c.max_skip_frame < 0) return fail(err, SD_ERR_ARG, "max_skip_frame must be >= 0");
  }
  if (c.motion_on) {
    if (c.motion_k < 1 || c.motion_k > 1024) return fail(err, SD_ERR_ARG, "motion_k out of range");
    if (!(c.motion_lambda > 0 && c.motion_lambda < 1)) return fail(err, SD_ERR_ARG, "motion_lambda must be in (0,1)");
    if (!(c.s_min >= 0 && c.s_min <= c.s_max && c.s_max <= 1)) return fail(err, SD_ERR_ARG, "need 0 <= s_min <= s_max <= 1");
    if (!(c.motion_sigma > 0)) return fail(err, SD_ERR_ARG, "motion_sigma must be > 0");
  }
  if (rows_max(c) > SD_MAX_ROWS) return fail(err, SD_ERR_ARG, "too many rows per forward");
  return SD_OK;
}

void make_schedule(const sd_stream_config& c, std::vector<double>& a, std::vector<double>& b) {
  const int T = c.n_train_steps;
  a.resize(T);
  b.resize(T);
  const double s0 = std::sqrt(c.beta_start), s1 = std::sqrt(c.beta_end);
  double prod = 1.0;
  for (int t = 0; t < T; ++t) {
    const double r = s0 + (s1 - s0) * (double)t / (double)(T - 1);
    const double beta = r * r;
    prod *= (1.0 - beta);
    a[t] = std::sqrt(prod);
    b[t] = std::sqrt(1.0 - prod);
  }
}

void taus_from_t_index(const sd_stream_config& c, int32_t* taus) {
  const int stride = c.n_train_steps / 50;
  for (int i = 0; i < c.n_slots; ++i) taus[i] = (c.n_train_steps - 1) - stride * c.t_index[i];
}

void taus_from_noise_rate(double s, int n, int n_train, int32_t* taus) {
  for (int i = 0; i < n; ++i) {
    volatile double v = s * (double)(n_train - 1);
    v = v * (double)(n - i);
    v = v / (double)n;
    taus[i] = (int32_t)std::nearbyint(v);   // default rounding mode: ties to even
  }
}

double ssf_cosine(int64_t D, int64_t N1, int64_t N2) {
  if (N1 == 0 && N2 == 0) return 1.0;
  if (N1 == 0 || N2 == 0) return 0.0;
  volatile double prod = (double)N1 * (double)N2;
  return (double)D / std::sqrt(prod);
}

double ssf_probability(double sim, double eta) {
  const double p = (sim - eta) / (1.0 - eta);
  return p > 0.0 ? p : 0.0;
}

double motion_distance(int64_t sumsq, int64_t n_elems) {
  return std::sqrt((double)sumsq / (double)n_elems) / 4096.0;
}

double motion_update(double s, const double* w, int n, const sd_stream_config& c) {
  if (n == 0) return s;
  double tot = 0.0;
  for (int i = 0; i < n; ++i) tot += w[i];
  const double d_bar = tot / (double)n;
  double d_hat = d_bar / c.motion_sigma;
  d_hat = d_hat < 0.0 ? 0.0 : (d_hat > 1.0 ? 1.0 : d_hat);
  volatile double span = (c.s_max - c.s_min) * d_hat;
  const double target = c.s_max - span;
  volatile double t1 = c.motion_lambda * target;
  volatile double t2 = (1.0 - c.motion_lambda) * s;
  return t1 + t2;
}

bool ssf_decide(Controls& st, const sd_stream_config& c, int64_t D, int64_t N1, int64_t N2, double u,
                double* sim, double* p) {
  *sim = 1.0;
  *p = 0.0;
  if (!st.has_ref) {
    st.skip_run = 0;
    st.has_ref = true;
    return false;
  }
  *sim = ssf_cosine(D, N1, N2);
  *p = ssf_probability(*sim, c.ssf_eta);
  if (st.skip_run < c.max_skip_frame && u < *p) {
    st.skip_run += 1;
    return true;
  }
  st.skip_run = 0;
  return false;
}

double motion_push(Controls& st, const sd_stream_config& c, const double* dists, int n) {
  for (int i = 0; i < n; ++i) {
    st.window.push_back(dists[i]);
    if ((int)st.window.size() > c.motion_k) st.window.erase(st.window.begin());
  }
  st.s = motion_update(st.s, st.window.data(), (int)st.window.size(), c);
  return st.s;
}

int32_t rope_assign(Controls& st, int32_t T, int32_t reset) {
  if (st.rope_p + T - 1 > reset) st.rope_p = 0;
  const int32_t t0 = st.rope_p;
  st.rope_p += T;
  return t0;
}

}  // namespace sd

// ---------------------------------------------------------------------------
// Host-only entry points of the state module (no device code), so the CPU
// test suite can check the fp64 decisions against the oracle bit for bit.
extern "C" {

int sdstate_validate(const sd_stream_config* c, char* msg, int msg_len) {
  std::string err;
  const int rc = sd::validate_config(*c, &err);
  if (msg && msg_len > 0) std::snprintf(msg, msg_len, "%s", err.c_str());
  return rc;
}

void sdstate_schedule(const sd_stream_config* c, double* a, double* b) {
  std::vector<double> va, vb;
  sd::make_schedule(*c, va, vb);
  for (size_t i = 0; i < va.size(); ++i) { a[i] = va[i]; b[i] = vb[i]; }
}

void sdstate_taus_noise_rate(double s, int n, int n_train, int32_t* taus) { sd::taus_from_noise_rate(s, n, n_train, taus); }
void sdstate_taus_t_index(const sd_stream_config* c, int32_t* taus) { sd::taus_from_t_index(*c, taus); }
double sdstate_ssf_cosine(int64_t D, int64_t N1, int64_t N2) { return sd::ssf_cosine(D, N1, N2); }
double sdstate_ssf_probability(double sim, double eta) { return sd::ssf_probability(sim, eta); }
double sdstate_motion_distance(int64_t sumsq, int64_t n) { return sd::motion_distance(sumsq, n); }
double sdstate_motion_update(double s, const double* w, int n, const sd_stream_config* c) {
  return sd::motion_update(s, w, n, *c);
}

}  // extern "C"
