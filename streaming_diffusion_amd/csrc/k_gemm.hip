// GEMMs of the denoiser, C[m][n] = sum_k A[m][k] W[n][k], with the fused
// epilogues of the DiT block (bias, GELU, gate * (.) + residual, q|k|v split
// with 3D RoPE and per-head scatter, unpatchify).  bf16 problems go to the
// matrix-core kernel (k_gemm_mfma.hip); this file holds the fp32 path, a
// vector-ALU tiled kernel (64 x 64 tile, 4 x 4 outputs per thread) used by the
// fp32 configuration, and the dispatch.
#include <cmath>

#include "kernels.h"

namespace sdk {

// ---------------------------------------------------------------------------
// Epilogue.  acc is C[m][n] (fp32); partner is C[m][n ^ 1] (the other half of
// a RoPE pair).  T is the element type of the GEMM.
template <typename T>
SD_DEV float bias_at(const Epi& E, int n) {
  return E.bias ? to_f(((const T*)E.bias)[n]) : 0.f;
}

template <typename T, int MODE>
SD_DEV void epi_apply(const Epi& E, int m, int n, int N, float acc, float partner) {
  switch (MODE) {
    case EPI_STORE: {
      const float v = acc + bias_at<T>(E, n);
      ((T*)E.out)[(int64_t)m * E.ldo + n] = from_f<T>(v);
      break;
    }
    case EPI_F32: {
      const float v = acc + bias_at<T>(E, n);
      ((float*)E.out)[(int64_t)m * E.ldo + n] = v;
      break;
    }
    case EPI_GELU: {
      const float v = acc + bias_at<T>(E, n);
      const float g = 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
      ((T*)E.out)[(int64_t)m * E.ldo + n] = from_f<T>(g);
      break;
    }
    case EPI_GATE_RESID: {
      const int r = m / E.L;
      const float v = acc + bias_at<T>(E, n);
      const float g = E.mod[(int64_t)r * E.six_d + E.gate_off + n] + to_f(((const T*)E.blk)[E.gate_off + n]);
      E.resid[(int64_t)m * N + n] += g * v;
      break;
    }
    case EPI_RESID: {
      const float v = acc + bias_at<T>(E, n);
      E.resid[(int64_t)m * N + n] += v;
      break;
    }
    case EPI_PATCH: {
      E.resid[(int64_t)m * N + n] = acc + bias_at<T>(E, n);
      break;
    }
    case EPI_QKV:
    case EPI_CTXKV: {
      const int which = n / E.d;
      const int nn = n - which * E.d;
      const int h = nn / E.hd, e = nn - h * E.hd;
      float v = acc + bias_at<T>(E, n);
      const int r = m / E.L, t = m - r * E.L;
      const int sec = (MODE == EPI_CTXKV) ? which + 1 : which;   // 0 q, 1 k, 2 v
      if (E.rope && sec < 2) {
        const float pv = partner + bias_at<T>(E, n ^ 1);
        const int hw = E.Hp * E.Wp;
        const int f = t / hw, y = (t / E.Wp) % E.Hp, x = t % E.Wp;
        float2 cs;
        if (e < E.dt)
          cs = E.rope_t[((E.t0_dev ? E.t0_dev[r] : E.t0[r]) + f) * (E.dt >> 1) + (e >> 1)];
        else if (e < E.dt + E.dh)
          cs = E.rope_h[y * (E.dh >> 1) + ((e - E.dt) >> 1)];
        else
          cs = E.rope_w[x * ((E.hd - E.dt - E.dh) >> 1) + ((e - E.dt - E.dh) >> 1)];
        v = (e & 1) ? (pv * cs.y + v * cs.x) : (v * cs.x - pv * cs.y);
      }
      if (sec == 0)
        ((T*)E.q)[(((int64_t)r * E.H + h) * E.L + t) * E.hd + e] = from_f<T>(v);
      else if (sec == 1)
        ((T*)E.k)[(((int64_t)h * E.krows + r) * E.kstride + t) * E.hd + e] = from_f<T>(v);
      else
        ((T*)E.vt)[(((int64_t)h * E.hd + e) * E.krows + r) * E.kstride + t] = from_f<T>(v);
      break;
    }
    case EPI_HEAD: {
      const int r = m / E.L, t = m - r * E.L;
      const int hw = E.Hp * E.Wp;
      const int f = t / hw, y = (t / E.Wp) % E.Hp, x = t % E.Wp;
      const int c = n % E.C, px = (n / E.C) % E.p, py = n / (E.C * E.p);
      const int64_t lat = (int64_t)E.T * E.C * E.Hl * E.Wl;
      const float v = acc + bias_at<T>(E, n);
      E.eps[r * lat + (((int64_t)f * E.C + c) * E.Hl + y * E.p + py) * E.Wl + x * E.p + px] = v;
      break;
    }
    default:
      break;
  }
}

// ---------------------------------------------------------------------------
// fp32 vector-ALU GEMM: 64 x 64 tile, BK = 16, 4 x 4 outputs per thread.
template <int MODE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ W,
                                                       int M, int N, int K, Epi E, int tiles_m) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  const int tid = threadIdx.x;
  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * 256, row = c >> 4, kk = c & 15;
      const int gm = m0 + row, gn = n0 + row, gk = k0 + kk;
      As[kk][row] = (gm < M && gk < K) ? A[(int64_t)gm * K + gk] : 0.f;
      Bs[kk][row] = (gn < N && gk < K) ? W[(int64_t)gn * K + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m < M && n < N) epi_apply<float, MODE>(E, m, n, N, acc[i][j], acc[i][j ^ 1]);
    }
}

template <int MODE>
static hipError_t gemm_f32_mode(hipStream_t s, const void* A, const void* W, int M, int N, int K, const Epi& E) {
  const int tm = (M + 63) / 64, tn = (N + 63) / 64;
  gemm_f32_kernel<MODE><<<tm * tn, 256, 0, s>>>((const float*)A, (const float*)W, M, N, K, E, tm);
  return hipGetLastError();
}

hipError_t gemm(hipStream_t s, bool bf, const void* A, const void* W, int M, int N, int K, const Epi& E) {
  if (M == 0 || N == 0) return hipSuccess;
  if (bf) return gemm_mfma(s, A, W, M, N, K, E);
  switch (E.mode) {
    case EPI_STORE: return gemm_f32_mode<EPI_STORE>(s, A, W, M, N, K, E);
    case EPI_GELU: return gemm_f32_mode<EPI_GELU>(s, A, W, M, N, K, E);
    case EPI_GATE_RESID: return gemm_f32_mode<EPI_GATE_RESID>(s, A, W, M, N, K, E);
    case EPI_RESID: return gemm_f32_mode<EPI_RESID>(s, A, W, M, N, K, E);
    case EPI_PATCH: return gemm_f32_mode<EPI_PATCH>(s, A, W, M, N, K, E);
    case EPI_QKV: return gemm_f32_mode<EPI_QKV>(s, A, W, M, N, K, E);
    case EPI_HEAD: return gemm_f32_mode<EPI_HEAD>(s, A, W, M, N, K, E);
    case EPI_CTXKV: return gemm_f32_mode<EPI_CTXKV>(s, A, W, M, N, K, E);
    case EPI_F32: return gemm_f32_mode<EPI_F32>(s, A, W, M, N, K, E);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sdk
