// Host-side state machine of the stream: configuration checks, the noise
// schedule, timesteps, the SSF decision, the motion-aware noise rate and the
// RoPE counter.  Plain C++ with no device code; every floating-point step is
// IEEE fp64 evaluated in the written order (built without FMA contraction), so
// integer decisions derived from it are reproducible.
#pragma once
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/sd_stream.h"

namespace sd {

// Returns SD_OK or an error code with a message in *err.
int validate_config(const sd_stream_config& c, std::string* err);

inline int64_t tokens_per_chunk(const sd_stream_config& c) {
  return (int64_t)c.latent_t * (c.latent_h / c.patch) * (c.latent_w / c.patch);
}
inline int64_t latent_elems(const sd_stream_config& c) {
  return (int64_t)c.latent_t * c.latent_c * c.latent_h * c.latent_w;
}
inline int rows_max(const sd_stream_config& c) {
  const int pos = c.chunks_per_step * c.n_slots;
  const int clean = c.kv_recompute ? c.chunks_per_step : 0;
  if (c.cfg_type == SD_CFG_FULL) return 2 * pos + clean;
  return pos + (c.cfg_type == SD_CFG_ONETIME ? c.chunks_per_step : 0) + clean;
}

// Scaled-linear schedule: sqrt(beta_t) linear in t; alpha_t = prod(1 - beta).
// a[t] = sqrt(alpha_t), b[t] = sqrt(1 - alpha_t).
void make_schedule(const sd_stream_config& c, std::vector<double>& a, std::vector<double>& b);

// tau_i = (n_train - 1) - (n_train / 50) * t_index[i]
void taus_from_t_index(const sd_stream_config& c, int32_t* taus);
// tau_i = round_half_even(s * (n_train - 1) * (n - i) / n)
void taus_from_noise_rate(double s, int n, int n_train, int32_t* taus);

// SSF tail: cosine from exact integer sums; skip probability.
double ssf_cosine(int64_t D, int64_t N1, int64_t N2);
double ssf_probability(double sim, double eta);

// Motion: RMS distance of 2^-12-quantised frames from the exact sum of squares.
double motion_distance(int64_t sumsq, int64_t n_elems);
// One EMA step of the noise rate from a chronological window of distances.
double motion_update(double s, const double* window, int n, const sd_stream_config& c);

struct Controls {
  // SSF
  bool has_ref = false;
  int32_t skip_run = 0;
  // motion
  double s = 0.0;
  std::vector<double> window;
  bool has_prev = false;
  // RoPE
  int32_t rope_p = 0;
};

// Decide whether a frame is skipped given the exact sums against the
// reference.  Updates skip_run.  has_ref=false means first frame.
bool ssf_decide(Controls& st, const sd_stream_config& c, int64_t D, int64_t N1, int64_t N2, double u,
                double* sim, double* p);

// Append the chunk's motion distances, update s and return it.
double motion_push(Controls& st, const sd_stream_config& c, const double* dists, int n);

// Temporal RoPE base for a chunk of T frames; restarts at 0 when the chunk's
// last position would exceed the threshold.
int32_t rope_assign(Controls& st, int32_t T, int32_t reset);

}  // namespace sd
