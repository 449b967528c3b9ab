// Memory-bound kernels of the step: entry noising, the fused R-CFG / update
// epilogue, patch gathering, LayerNorm + adaLN modulation, the timestep
// embedding and its GEMVs, KV ring append and sink copies, and the exact
// reductions of the per-frame controls (SSF, motion, sink cosine).
#include <cmath>

#include "kernels.h"
#include "kv_append.h"
#include "ln_row.h"

namespace sdk {

static inline unsigned grid1(int64_t n, int block) { return (unsigned)((n + block - 1) / block); }

// ---------------------------------------------------------------------------
// Entry noising of a new frame (x_tau0 = a x0 + b eps): the start of a frame's
// trajectory through the slots.
__global__ void entry_noise_kernel(const float* __restrict__ x0, const float* __restrict__ noise,
                                   float* __restrict__ xs, float* __restrict__ x0s, int64_t n, float a, float b) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float v = x0[i];
  xs[i] = a * v + b * noise[i];
  if (x0s) x0s[i] = v;
}

hipError_t entry_noise(hipStream_t s, const float* x0, const float* noise, float* xs, float* x0s, int64_t n,
                       float a, float b) {
  if (n == 0) return hipSuccess;
  entry_noise_kernel<<<grid1(n, 256), 256, 0, s>>>(x0, noise, xs, x0s, n, a, b);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Residual CFG (StreamDiffusion paper notes, section 2): virtual residual
// noise eps' = (x - a x0*) / b, eps_cfg = delta eps' + gamma (eps_c - delta eps'),
// then x0_hat = (x - b eps_cfg) / a and either re-noise to the next slot's
// timestep (DDIM: with eps_cfg; LCM sampler: with the frame's noise record
// zrow) or emit x0_hat (to output position oidx of the step).  For
// onetime-negative R-CFG an entering row first turns its negative row's output
// into its x0* estimate; under full CFG eps' is the twin row's output.
__global__ void rcfg_update_kernel(const RowTable* __restrict__ rt, float* __restrict__ store_x,
                                   float* __restrict__ store_x0s, const float* __restrict__ eps,
                                   const float* __restrict__ store_z, float* __restrict__ out, int64_t lat, float gamma,
                                   float delta) {
  const int r = blockIdx.y;
  const RowInfo ri = rt->r[r];
  if (ri.kind != 0) return;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= lat) return;
  const int64_t off = (int64_t)ri.frame * lat + i;
  const float x = store_x[off];
  float ep;
  if (ri.pair >= 0) {
    ep = eps[(int64_t)ri.pair * lat + i];
  } else {
    float x0s;
    if (ri.neg >= 0) {
      const float en = eps[(int64_t)ri.neg * lat + i];
      x0s = (x - ri.b0 * en) / ri.a0;
      store_x0s[off] = x0s;
    } else {
      x0s = store_x0s[off];
    }
    ep = (x - ri.a * x0s) / ri.b;
  }
  const float ec = eps[(int64_t)r * lat + i];
  const float ecfg = delta * ep + gamma * (ec - delta * ep);
  const float x0h = (x - ri.b * ecfg) / ri.a;
  if (ri.last) {
    out[(int64_t)ri.oidx * lat + i] = x0h;
    if (ri.keep) store_x[off] = x0h;
  } else {
    // DDIM re-noises with the guided prediction, the LCM sampler with the
    // frame's fresh noise for the next slot
    const float z = ri.zrow >= 0 ? store_z[(int64_t)ri.zrow * lat + i] : ecfg;
    store_x[off] = ri.an * x0h + ri.bn * z;
  }
}

hipError_t rcfg_update(hipStream_t s, const RowTable* rt, int R, float* store_x, float* store_x0s, const float* eps,
                       const float* store_z, float* out, int64_t lat, float gamma, float delta) {
  if (R == 0) return hipSuccess;
  dim3 g(grid1(lat, 256), R);
  rcfg_update_kernel<<<g, 256, 0, s>>>(rt, store_x, store_x0s, eps, store_z, out, lat, gamma, delta);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Patch gather: token (t, y, x) of row r gets the p x p x C patch in
// (py, px, c) order.  SPLIT (bf16): a token's row holds the P values as
// hi = bf16(v), then lo = bf16(v - hi) (row pitch 2P), for a patch embedding
// over K = 2P against [W | W] that sees the fp32 latent to about 16 bits.
template <typename T, bool SPLIT = false>
__global__ void patchify_kernel(const RowTable* __restrict__ rt, const float* __restrict__ store_x, T* __restrict__ out,
                                int64_t lat, int Tn, int C, int Hl, int Wl, int p) {
  const int r = blockIdx.y;
  const int Hp = Hl / p, Wp = Wl / p;
  const int P = p * p * C;
  const int64_t per_row = (int64_t)Tn * Hp * Wp * P;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= per_row) return;
  const int v = (int)(i % P);
  const int64_t tok = i / P;
  const int xq = (int)(tok % Wp), yq = (int)((tok / Wp) % Hp), f = (int)(tok / ((int64_t)Wp * Hp));
  const int c = v % C, px = (v / C) % p, py = v / (C * p);
  const float* src = store_x + (int64_t)rt->r[r].frame * lat;
  const float val = src[(((int64_t)f * C + c) * Hl + (yq * p + py)) * Wl + (xq * p + px)];
  if constexpr (SPLIT) {
    const T hi = from_f<T>(val);
    T* o = out + ((int64_t)r * Tn * Hp * Wp + tok) * 2 * P + v;
    o[0] = hi;
    o[P] = from_f<T>(val - (float)hi);
  } else {
    out[(int64_t)r * per_row + i] = from_f<T>(val);
  }
}

hipError_t patchify(hipStream_t s, bool bf, const RowTable* rt, int R, const float* store_x, void* out, int64_t lat,
                    int T, int C, int Hl, int Wl, int p, bool split) {
  const int64_t per_row = (int64_t)T * (Hl / p) * (Wl / p) * p * p * C;
  if (R == 0) return hipSuccess;
  dim3 g(grid1(per_row, 256), R);
  if (split && !bf) return hipErrorInvalidValue;
  if (split)
    patchify_kernel<bf16, true><<<g, 256, 0, s>>>(rt, store_x, (bf16*)out, lat, T, C, Hl, Wl, p);
  else if (bf)
    patchify_kernel<bf16><<<g, 256, 0, s>>>(rt, store_x, (bf16*)out, lat, T, C, Hl, Wl, p);
  else
    patchify_kernel<float><<<g, 256, 0, s>>>(rt, store_x, (float*)out, lat, T, C, Hl, Wl, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// LayerNorm + adaLN modulation, one wave per token row.  The row is read
// once into registers (NV float4 per lane, d <= 256 NV); mean and variance
// are two passes over the registers (population variance).  Shift / scale
// vectors (per forward row, cache resident) load four at a time; outputs
// store four at a time.
constexpr int LN_MAXV = 20;     // largest NV: d up to 5120

// SPLIT (bf16): the row of 2d outputs holds hi = bf16(y) in [0, d) and
// lo = bf16(y - hi) in [d, 2d), so hi + lo carries y to about 16 bits; a GEMM
// over K = 2d against the weights stored twice ([W | W]) then sees y itself.
template <typename T, int NV, bool SPLIT = false>
__global__ __launch_bounds__(256) void ln_mod_kernel(const float* __restrict__ x, T* __restrict__ out, int M, int d,
                                                     int L, const float* __restrict__ mod, const T* __restrict__ blk,
                                                     int shift_off, int scale_off, int six_d, float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float4* xr = (const float4*)(x + (int64_t)row * d);
  const int nv = d >> 2;
  float4 v[NV];
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = lane + 64 * i;
    v[i] = j < nv ? xr[j] : make_float4(0.f, 0.f, 0.f, 0.f);
    sum += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  }
  const float mu = wave_sum(sum) / (float)d;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (lane + 64 * i < nv) {
      const float a = v[i].x - mu, b = v[i].y - mu, c = v[i].z - mu, e = v[i].w - mu;
      sq += (a * a + b * b) + (c * c + e * e);
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(sq) / (float)d + eps);
  const int r = row / L;
  const float* mr = mod ? mod + (int64_t)r * six_d : nullptr;
  T* orow = out + (int64_t)row * (SPLIT ? 2 * d : d);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = lane + 64 * i;
    if (j >= nv) continue;
    float o[4] = {(v[i].x - mu) * rstd, (v[i].y - mu) * rstd, (v[i].z - mu) * rstd, (v[i].w - mu) * rstd};
    if (mr) {
      float sh[4], sc[4];
      load4(mr + shift_off + 4 * j, sh);
      load4(mr + scale_off + 4 * j, sc);
      if (blk) {
        float bs[4], bc[4];
        load4(blk + shift_off + 4 * j, bs);
        load4(blk + scale_off + 4 * j, bc);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          sh[q] += bs[q];
          sc[q] += bc[q];
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = o[q] * (1.0f + sc[q]) + sh[q];
    }
    store4<T>(orow + 4 * j, o);
    if constexpr (SPLIT) {
      float lo[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) lo[q] = o[q] - (float)(T)o[q];
      store4<T>(orow + d + 4 * j, lo);
    }
  }
}

// The same LayerNorm + modulation for few rows (the chunks below the batch
// knee): one workgroup of d / 4 threads per row, one float4 per thread, so
// the row, its shift / scale vectors and the block table are all requested
// at once and the reductions span the workgroup (wave sums, then the waves
// through LDS).  With 128 rows the one-wave-per-row form leaves most of the
// chip idle and runs its loads, its two reductions and the modulation reads
// one after another.
template <typename T, bool SPLIT = false>
__global__ __launch_bounds__(512) void ln_mod_row_kernel(const float* __restrict__ x, T* __restrict__ out, int d,
                                                         int L, const float* __restrict__ mod,
                                                         const T* __restrict__ blk, int shift_off, int scale_off,
                                                         int six_d, float eps) {
  __shared__ float red[2][8];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int j = tid;                                     // float4 index in the row (blockDim = d / 4)
  const float4 v = ((const float4*)(x + (int64_t)row * d))[j];
  const float* mr = mod ? mod + (int64_t)(row / L) * six_d : nullptr;
  float sh[4] = {0.f, 0.f, 0.f, 0.f}, sc[4] = {0.f, 0.f, 0.f, 0.f};
  if (mr) ln_row_mod(mr, blk, shift_off, scale_off, j, sh, sc);
  float o[4];
  ln_row(v, d, eps, mr != nullptr, sh, sc, red, nw, lane, wave, o);
  ln_row_store<T, SPLIT>(out + (int64_t)row * (SPLIT ? 2 * d : d), d, j, o);
}

void rope_table_fill(float2* out, int npos, int width, double base) {
  const int np = width / 2;
  for (int p = 0; p < npos; ++p) {
    if (np == 0) out[p] = float2{1.f, 0.f};
    for (int j = 0; j < np; ++j) {
      const double th = (double)p * std::pow(base, -2.0 * j / (double)width);
      out[(size_t)p * np + j] = float2{(float)std::cos(th), (float)std::sin(th)};
    }
  }
}

hipError_t ln_mod(hipStream_t s, bool bf, const float* x, void* out, int M, int d, int L, const float* mod,
                  const void* blk, int shift_off, int scale_off, int six_d, float eps, int form) {
  if (M == 0) return hipSuccess;
  if ((d & 3) || d > 4 * 64 * LN_MAXV || (shift_off & 3) || (scale_off & 3) || (six_d & 3)) return hipErrorInvalidValue;
  if (form != LN_PLAIN && !bf) return hipErrorInvalidValue;
  if (form == LN_F16 && mod) return hipErrorInvalidValue;
  // few rows: a workgroup per row (d / 4 threads, whole waves, at most 512)
  if (M <= 1024 && d % 256 == 0 && d <= 2048) {
    const unsigned g = (unsigned)M, nt = (unsigned)(d / 4);
    if (form == LN_F16)
      ln_mod_row_kernel<f16><<<g, nt, 0, s>>>(x, (f16*)out, d, L, nullptr, nullptr, 0, 0, six_d, eps);
    else if (form == LN_SPLIT)
      ln_mod_row_kernel<bf16, true><<<g, nt, 0, s>>>(x, (bf16*)out, d, L, mod, (const bf16*)blk, shift_off,
                                                      scale_off, six_d, eps);
    else if (bf)
      ln_mod_row_kernel<bf16><<<g, nt, 0, s>>>(x, (bf16*)out, d, L, mod, (const bf16*)blk, shift_off, scale_off,
                                               six_d, eps);
    else
      ln_mod_row_kernel<float><<<g, nt, 0, s>>>(x, (float*)out, d, L, mod, (const float*)blk, shift_off,
                                                scale_off, six_d, eps);
    return hipGetLastError();
  }
  const unsigned g = (unsigned)((M + 3) / 4);
#define SD_LN_LAUNCH(NV)                                                                                           \
  do {                                                                                                             \
    if (form == LN_F16)                                                                                            \
      ln_mod_kernel<f16, NV><<<g, 256, 0, s>>>(x, (f16*)out, M, d, L, nullptr, nullptr, 0, 0, six_d, eps);         \
    else if (form == LN_SPLIT)                                                                                     \
      ln_mod_kernel<bf16, NV, true><<<g, 256, 0, s>>>(x, (bf16*)out, M, d, L, mod, (const bf16*)blk, shift_off,    \
                                                      scale_off, six_d, eps);                                      \
    else if (bf)                                                                                                   \
      ln_mod_kernel<bf16, NV><<<g, 256, 0, s>>>(x, (bf16*)out, M, d, L, mod, (const bf16*)blk, shift_off, scale_off, \
                                                six_d, eps);                                                       \
    else                                                                                                           \
      ln_mod_kernel<float, NV><<<g, 256, 0, s>>>(x, (float*)out, M, d, L, mod, (const float*)blk, shift_off,       \
                                                 scale_off, six_d, eps);                                           \
  } while (0)
  if (d <= 1024)
    SD_LN_LAUNCH(4);
  else if (d <= 1536)
    SD_LN_LAUNCH(6);
  else if (d <= 2048)
    SD_LN_LAUNCH(8);
  else
    SD_LN_LAUNCH(LN_MAXV);
#undef SD_LN_LAUNCH
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Sinusoidal timestep embedding in fp64: e = [cos(tau w_j), sin(tau w_j)],
// w_j = 10000^(-j / (D/2)).
__global__ void temb_embed_kernel(const RowTable* __restrict__ rt, float* __restrict__ out, int d_freq) {
  const int r = blockIdx.x;
  const int half = d_freq / 2;
  for (int j = threadIdx.x; j < half; j += blockDim.x) {
    const double w = pow(10000.0, -(double)j / (double)half);
    const double arg = (double)rt->r[r].tau * w;
    out[(int64_t)r * d_freq + j] = (float)cos(arg);
    out[(int64_t)r * d_freq + half + j] = (float)sin(arg);
  }
}

hipError_t temb_embed(hipStream_t s, const RowTable* rt, int R, float* out, int d_freq) {
  if (R == 0) return hipSuccess;
  temb_embed_kernel<<<R, 128, 0, s>>>(rt, out, d_freq);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Small-batch GEMV y[r][n] = act(x[r] . W[n] + b[n]) for all R rows, the
// weight matrix streamed from HBM once.  Each wave owns GN consecutive
// output features: per iteration every lane loads 8 weights (16 B bf16) of
// each of the GN weight rows, so GN independent loads are in flight, and
// applies them to the R input rows (read once per iteration, shared by the
// GN features, cache resident).  RB >= R bounds the row loop at compile time.
template <typename T>
SD_DEV void load8(const T* p, float* w);
template <>
SD_DEV void load8<bf16>(const bf16* p, float* w) {
  const bf16x8 v = *(const bf16x8*)p;
#pragma unroll
  for (int q = 0; q < 8; ++q) w[q] = (float)v[q];
}
template <>
SD_DEV void load8<float>(const float* p, float* w) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

constexpr int GEMV_GN = 4;

template <typename T, int RB>
__global__ __launch_bounds__(256) void gemv_kernel(const float* __restrict__ x, const T* __restrict__ W,
                                                   const T* __restrict__ bias, float* __restrict__ y, int R, int N,
                                                   int K, int act) {
  constexpr int GN = GEMV_GN;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nw = gridDim.x * 4;
  const int K8 = K >> 3;
  for (int n0 = wave * GN; n0 < N; n0 += nw * GN) {
    float acc[GN][RB];
#pragma unroll
    for (int g = 0; g < GN; ++g)
#pragma unroll
      for (int r = 0; r < RB; ++r) acc[g][r] = 0.f;
#pragma unroll 4
    for (int c = lane; c < K8; c += 64) {
      float w[GN][8];
#pragma unroll
      for (int g = 0; g < GN; ++g) {
        const int n = min(n0 + g, N - 1);      // a tail group repeats the last feature (not stored)
        load8<T>(W + (int64_t)n * K + 8 * c, w[g]);
      }
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        if (r < R) {
          const float4* xr = (const float4*)(x + (int64_t)r * K + 8 * c);
          const float4 a = xr[0], b = xr[1];
#pragma unroll
          for (int g = 0; g < GN; ++g)
            acc[g][r] += w[g][0] * a.x + w[g][1] * a.y + w[g][2] * a.z + w[g][3] * a.w + w[g][4] * b.x +
                         w[g][5] * b.y + w[g][6] * b.z + w[g][7] * b.w;
        }
      }
    }
#pragma unroll
    for (int g = 0; g < GN; ++g) {
      const int n = n0 + g;
      if (n >= N) break;
      const float bn = bias ? to_f(bias[n]) : 0.f;
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        if (r < R) {
          float v = wave_sum(acc[g][r]) + bn;
          if (act == 1) v = v / (1.0f + expf(-v));
          if (lane == 0) y[(int64_t)r * N + n] = v;
        }
      }
    }
  }
}

template <typename T>
static void launch_gemv(hipStream_t s, const float* x, const T* W, const T* b, float* y, int R, int N, int K, int act) {
  const int groups = (N + GEMV_GN - 1) / GEMV_GN;
  const int blocks = (groups + 3) / 4 < 2048 ? (groups + 3) / 4 : 2048;
  if (R <= 2)
    gemv_kernel<T, 2><<<blocks, 256, 0, s>>>(x, W, b, y, R, N, K, act);
  else if (R <= 4)
    gemv_kernel<T, 4><<<blocks, 256, 0, s>>>(x, W, b, y, R, N, K, act);
  else if (R <= 8)
    gemv_kernel<T, 8><<<blocks, 256, 0, s>>>(x, W, b, y, R, N, K, act);
  else if (R <= 16)
    gemv_kernel<T, 16><<<blocks, 256, 0, s>>>(x, W, b, y, R, N, K, act);
  else
    gemv_kernel<T, SD_MAX_ROWS><<<blocks, 256, 0, s>>>(x, W, b, y, R, N, K, act);
}

hipError_t gemv(hipStream_t s, bool bf, const float* x, const void* W, const void* b, float* y, int R, int N, int K,
                int act) {
  if (R < 1 || R > SD_MAX_ROWS || N < 1 || K < 8 || (K & 7)) return hipErrorInvalidValue;
  if (bf)
    launch_gemv<bf16>(s, x, (const bf16*)W, (const bf16*)b, y, R, N, K, act);
  else
    launch_gemv<float>(s, x, (const float*)W, (const float*)b, y, R, N, K, act);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// KV ring append: the exiting chunk's own K (head h: [L][hd] at kown + h k_hs)
// and V^T (row (h, e): [L] at vtown + (h hd + e) vt_ps) go to ring positions
// (ptr + t) mod W; its first Se tokens optionally become a sink entry.
template <typename T>
__global__ void kv_append_kernel(const T* __restrict__ kown, const T* __restrict__ vtown, int64_t k_hs, int64_t vt_ps,
                                 T* __restrict__ ringK, T* __restrict__ ringVT, int H, int hd, int L, int W, int ptr,
                                 T* __restrict__ sinkK, T* __restrict__ sinkVT, int S8, int sink_off, int Se,
                                 const int* __restrict__ ptr_dev) {
  if (ptr_dev) ptr = *ptr_dev;
  const int64_t per_head = (int64_t)L * hd;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= per_head * H) return;
  const int h = (int)(i / per_head);
  const int64_t j = i % per_head;
  // K element (t, e)
  {
    const int t = (int)(j / hd), e = (int)(j % hd);
    const T v = kown[h * k_hs + j];
    if (W > 0) ringK[((int64_t)h * W + (ptr + t) % W) * hd + e] = v;
    if (sinkK && t < Se) sinkK[((int64_t)h * S8 + sink_off + t) * hd + e] = v;
  }
  // V^T element (e, t)
  {
    const int e = (int)(j / L), t = (int)(j % L);
    const T v = vtown[((int64_t)h * hd + e) * vt_ps + t];
    if (W > 0) ringVT[((int64_t)h * hd + e) * W + (ptr + t) % W] = v;
    if (sinkVT && t < Se) sinkVT[((int64_t)h * hd + e) * S8 + sink_off + t] = v;
  }
}

// bf16 with every token range a multiple of 8 and L <= W: 16-byte chunks (8
// head-dim elements of one K row, or 8 consecutive tokens of one V^T row), one
// conditional wrap per chunk (kv_append_chunk).
__global__ void kv_append_vec_kernel(KvAppendArgs a) {
  kv_append_chunk(a, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

bool kv_append_vec_ok(bool bf, int64_t k_hs, int64_t vt_ps, int H, int hd, int L, int W, int ptr, const void* sinkK,
                      int S8, int sink_off, int Se) {
  return bf && (hd % 8) == 0 && (L % 8) == 0 && (W % 8) == 0 && (ptr % 8) == 0 && ptr < (W > 0 ? W : 1) &&
         (W == 0 || L <= W) && (k_hs % 8) == 0 && (vt_ps % 8) == 0 && k_hs >= (int64_t)L * hd && vt_ps >= L &&
         (!sinkK || ((S8 % 8) == 0 && (sink_off % 8) == 0 && (Se % 8) == 0));
}

hipError_t kv_append(hipStream_t s, bool bf, const void* kown, const void* vtown, int64_t k_hs, int64_t vt_ps,
                     void* ringK, void* ringVT, int H, int hd, int L, int W, int ptr, void* sinkK, void* sinkVT, int S8,
                     int sink_off, int Se, const int* ptr_dev) {
  const int64_t n = (int64_t)H * L * hd;
  if (k_hs < (int64_t)L * hd || vt_ps < L) return hipErrorInvalidValue;
  if (kv_append_vec_ok(bf, k_hs, vt_ps, H, hd, L, W, ptr, sinkK, S8, sink_off, Se)) {
    const int64_t chunks = 2 * (n / 8);
    const KvAppendArgs a{(const bf16*)kown, (const bf16*)vtown, k_hs, vt_ps, (bf16*)ringK, (bf16*)ringVT, H, hd, L,
                         W, ptr, (bf16*)sinkK, (bf16*)sinkVT, S8, sink_off, Se, ptr_dev};
    kv_append_vec_kernel<<<grid1(chunks, 256), 256, 0, s>>>(a);
    return hipGetLastError();
  }
  if (bf)
    kv_append_kernel<bf16><<<grid1(n, 256), 256, 0, s>>>((const bf16*)kown, (const bf16*)vtown, k_hs, vt_ps,
                                                         (bf16*)ringK, (bf16*)ringVT, H, hd, L, W, ptr, (bf16*)sinkK,
                                                         (bf16*)sinkVT, S8, sink_off, Se, ptr_dev);
  else
    kv_append_kernel<float><<<grid1(n, 256), 256, 0, s>>>((const float*)kown, (const float*)vtown, k_hs, vt_ps,
                                                          (float*)ringK, (float*)ringVT, H, hd, L, W, ptr,
                                                          (float*)sinkK, (float*)sinkVT, S8, sink_off, Se, ptr_dev);
  return hipGetLastError();
}

// Sink refresh copy: entry flag[1] <- ring tokens (ptr_old + t) mod W, t < Se,
// at every block, when flag[0] is set by sink_score.
template <typename T>
__global__ void sink_copy_kernel(const int* __restrict__ flag, const T* __restrict__ ringK,
                                 const T* __restrict__ ringVT, T* __restrict__ sinkK, T* __restrict__ sinkVT, int nb,
                                 int H, int hd, int W, int S8, int ptr_old, int Se, const int* __restrict__ ptr_dev) {
  if (flag[0] == 0) return;
  if (ptr_dev) ptr_old = *ptr_dev;
  const int j = flag[1];
  const int64_t per = (int64_t)Se * hd;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= per * H * nb) return;
  const int64_t bh = i / per;          // block * H + head
  const int64_t w = i % per;
  {
    const int t = (int)(w / hd), e = (int)(w % hd);
    sinkK[(bh * S8 + j * Se + t) * hd + e] = ringK[(bh * W + (ptr_old + t) % W) * hd + e];
  }
  {
    const int e = (int)(w / Se), t = (int)(w % Se);
    sinkVT[(bh * hd + e) * S8 + j * Se + t] = ringVT[(bh * hd + e) * W + (ptr_old + t) % W];
  }
}

hipError_t sink_copy(hipStream_t s, bool bf, const int* flag, const void* ringK, const void* ringVT, void* sinkK,
                     void* sinkVT, int nb, int H, int hd, int W, int S8, int ptr_old, int Se, const int* ptr_dev) {
  const int64_t n = (int64_t)nb * H * Se * hd;
  if (n == 0) return hipSuccess;
  if (bf)
    sink_copy_kernel<bf16><<<grid1(n, 256), 256, 0, s>>>(flag, (const bf16*)ringK, (const bf16*)ringVT,
                                                         (bf16*)sinkK, (bf16*)sinkVT, nb, H, hd, W, S8, ptr_old, Se,
                                                         ptr_dev);
  else
    sink_copy_kernel<float><<<grid1(n, 256), 256, 0, s>>>(flag, (const float*)ringK, (const float*)ringVT,
                                                          (float*)sinkK, (float*)sinkVT, nb, H, hd, W, S8, ptr_old,
                                                          Se, ptr_dev);
  return hipGetLastError();
}

// The step's dynamic values, by value in the kernel arguments, to device memory.
__global__ __launch_bounds__(256) void dyn_write_kernel(StepDyn d, StepDyn* __restrict__ dst) {
  constexpr int NW = (int)(sizeof(StepDyn) / 4);
  const uint32_t* src = (const uint32_t*)&d;
  uint32_t* out = (uint32_t*)dst;
  for (int i = threadIdx.x; i < NW; i += blockDim.x) out[i] = src[i];
}

hipError_t dyn_write(hipStream_t s, const StepDyn& d, StepDyn* dst) {
  static_assert(sizeof(StepDyn) % 4 == 0 && sizeof(StepDyn) <= 4000, "step values must fit the kernel arguments");
  dyn_write_kernel<<<1, 256, 0, s>>>(d, dst);
  return hipGetLastError();
}

__global__ void fill_zero_kernel(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t fill_zero(hipStream_t s, void* p, size_t bytes) {
  const int64_t n = (int64_t)(bytes / 4);
  if (n == 0) return hipSuccess;
  fill_zero_kernel<<<grid1(n, 256), 256, 0, s>>>((uint32_t*)p, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Stochastic Similarity Filter sums (StreamDiffusion paper notes, section 3):
// exact int64 dot products of integer frames, one workgroup, fixed order.
SD_DEV long long ssf_code(int kind, const void* p, int64_t i) {
  if (kind == 0) return (long long)((const uint8_t*)p)[i];
  const double v = rint((double)((const float*)p)[i] * 4096.0);
  const double c = v < -1048576.0 ? -1048576.0 : (v > 1048576.0 ? 1048576.0 : v);
  return (long long)c;
}

__global__ __launch_bounds__(1024) void ssf_sums_kernel(int kind, const void* __restrict__ a,
                                                        const void* __restrict__ b, int64_t n,
                                                        long long* __restrict__ out) {
  __shared__ long long red[3][16];
  long long d = 0, n1 = 0, n2 = 0;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const long long x = ssf_code(kind, a, i), y = ssf_code(kind, b, i);
    d += x * y;
    n1 += x * x;
    n2 += y * y;
  }
  d = wave_sum_i64(d);
  n1 = wave_sum_i64(n1);
  n2 = wave_sum_i64(n2);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][w] = d;
    red[1][w] = n1;
    red[2][w] = n2;
  }
  __syncthreads();
  if (threadIdx.x < 3) {
    long long t = 0;
    for (int k = 0; k < (int)(blockDim.x >> 6); ++k) t += red[threadIdx.x][k];
    out[threadIdx.x] = t;
  }
}

hipError_t ssf_sums(hipStream_t s, int kind, const void* a, const void* b, int64_t n, long long* out3) {
  ssf_sums_kernel<<<1, 1024, 0, s>>>(kind, a, b, n, out3);
  return hipGetLastError();
}

// Motion (StreamDiffusionV2 summary, motion-aware noise scheduler): exact
// sum of squared differences of consecutive 2^-12-quantised latent frames.
__global__ __launch_bounds__(1024) void motion_sums_kernel(const float* __restrict__ cur,
                                                           const float* __restrict__ prev_last, int64_t n,
                                                           long long* __restrict__ out) {
  __shared__ long long red[16];
  const int t = blockIdx.x;
  const float* a = (t == 0) ? prev_last : cur + (int64_t)(t - 1) * n;
  const float* b = cur + (int64_t)t * n;
  long long acc = 0;
  if (a) {
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
      const long long x = ssf_code(1, a, i), y = ssf_code(1, b, i);
      acc += (y - x) * (y - x);
    }
  }
  acc = wave_sum_i64(acc);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    long long s = 0;
    for (int k = 0; k < (int)(blockDim.x >> 6); ++k) s += red[k];
    out[t] = s;
  }
}

hipError_t motion_sums(hipStream_t s, const float* cur, const float* prev_last, int T, int64_t n, long long* out) {
  motion_sums_kernel<<<T, 1024, 0, s>>>(cur, prev_last, n, out);
  return hipGetLastError();
}

// Adaptive sink refresh (StreamDiffusionV2 summary): chunk embedding h = token
// mean of the last block's output; cosine against each sink embedding; the
// least similar entry is refreshed when its cosine is below tau.
#define SINK_PARTS 64
// The token mean, the embeddings and the cosines are kept in fp64, and the
// decision compares against tau in fp64, as the rule is stated.
__global__ __launch_bounds__(256) void sink_partial_kernel(const float* __restrict__ x, double* __restrict__ part,
                                                           int L, int d) {
  const int g = blockIdx.y;
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= d) return;
  const int per = (L + SINK_PARTS - 1) / SINK_PARTS;
  const int t0 = g * per, t1 = min(L, t0 + per);
  double s = 0.0;
  for (int t = t0; t < t1; ++t) s += (double)x[(int64_t)t * d + c];
  part[(int64_t)g * d + c] = s;
}

__global__ __launch_bounds__(1024) void sink_decide_kernel(const double* __restrict__ part, int L, int d,
                                                           double* __restrict__ emb, int M, int capture_entry,
                                                           double tau, int* __restrict__ flag,
                                                           double* __restrict__ sim_out) {
  extern __shared__ double h[];
  __shared__ double red[3][16];
  __shared__ double sims[SD_MAX_SINK];
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    double s = 0.0;
    for (int g = 0; g < SINK_PARTS; ++g) s += part[(int64_t)g * d + c];
    h[c] = s / (double)L;
  }
  __syncthreads();
  if (capture_entry >= 0) {
    for (int c = threadIdx.x; c < d; c += blockDim.x) emb[(int64_t)capture_entry * d + c] = h[c];
    if (threadIdx.x == 0) {
      flag[0] = 0;
      flag[1] = capture_entry;
      flag[2] = 0;
      sim_out[0] = 1.0;
    }
    return;
  }
  for (int j = 0; j < M; ++j) {
    double dot = 0, hh = 0, ee = 0;
    for (int c = threadIdx.x; c < d; c += blockDim.x) {
      const double a = h[c], b = emb[(int64_t)j * d + c];
      dot += a * b;
      hh += a * a;
      ee += b * b;
    }
    dot = wave_sum_d(dot);
    hh = wave_sum_d(hh);
    ee = wave_sum_d(ee);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
      red[0][w] = dot;
      red[1][w] = hh;
      red[2][w] = ee;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      double D = 0, A = 0, B = 0;
      for (int k = 0; k < (int)(blockDim.x >> 6); ++k) {
        D += red[0][k];
        A += red[1][k];
        B += red[2][k];
      }
      sims[j] = (A == 0.0 || B == 0.0) ? 0.0 : D / (sqrt(A) * sqrt(B));
    }
    __syncthreads();
  }
  __shared__ int jstar;
  if (threadIdx.x == 0) {
    int js = 0;
    for (int j = 1; j < M; ++j)
      if (sims[j] < sims[js]) js = j;
    jstar = js;
    const int refresh = sims[js] < tau ? 1 : 0;
    flag[0] = refresh;
    flag[1] = js;
    flag[2] = 1;
    sim_out[0] = sims[js];
  }
  __syncthreads();
  if (sims[jstar] < tau)
    for (int c = threadIdx.x; c < d; c += blockDim.x) emb[(int64_t)jstar * d + c] = h[c];
}

hipError_t sink_score(hipStream_t s, const float* x, double* partial, int L, int d, double* emb, int M,
                      int capture_entry, double tau, int* flag, double* sim) {
  dim3 g1((d + 255) / 256, SINK_PARTS);
  sink_partial_kernel<<<g1, 256, 0, s>>>(x, partial, L, d);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  sink_decide_kernel<<<1, 1024, d * sizeof(double), s>>>(partial, L, d, emb, M, capture_entry, tau, flag, sim);
  return hipGetLastError();
}

}  // namespace sdk
