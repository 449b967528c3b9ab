// Stream-VAE kernels (StreamDiffusionV2 summary, Stream-VAE: short chunks,
// intermediate features cached inside every 3D convolution).  Activations are
// bf16 channels-last [T][H][W][C]; a causal 3x3x3 convolution reads input
// frames t-2, t-1, t, taking frames before the chunk from the layer's cache
// (the last two input frames of the previous chunk), with spatial zero
// padding.  Weights [Cout][3][3][3][Cin] (taps (dt, dy, dx)), i.e. a row of
// K = 27 Cin per output channel.
#include "kernels.h"

namespace sdk {

// k index -> (tap, channel): 16-byte chunks of 8 channels never straddle a
// tap because Cin is a multiple of 8.
SD_DEV const bf16* conv_src(const ConvArgs& a, int t, int y, int x, int k, int HW) {
  const int tap = k / a.Cin, ci = k - tap * a.Cin;
  const int dt = tap / 9, dy = (tap / 3) % 3, dx = tap % 3;
  const int t2 = t + dt - 2, y2 = y + dy - 1, x2 = x + dx - 1;
  if ((unsigned)y2 >= (unsigned)a.H || (unsigned)x2 >= (unsigned)a.W) return nullptr;
  if (t2 < 0) return a.cache ? a.cache + ((int64_t)(t2 + 2) * HW + (int64_t)y2 * a.W + x2) * a.Cin + ci : nullptr;
  return a.x + ((int64_t)t2 * HW + (int64_t)y2 * a.W + x2) * a.Cin + ci;
}

// ---------------------------------------------------------------------------
// Implicit-GEMM convolution on the matrix cores: C^T[n][m] = sum_k W[n][k]
// A[m][k], m an output position, n an output channel, A the gathered input
// (im2col on the fly).  Workgroup tile 128 positions x BN channels, k-tiles
// of 32, 4 waves: 2 x 2 (each 64 positions x BN/2 channels) for BN >= 64,
// 4 x 1 (each 32 positions x 32 channels) for the narrow BN = 32, operands
// staged global -> registers -> LDS (double buffered, one barrier per
// k-tile); LDS rows are 64 bytes with their four 16-byte chunks XOR-swizzled
// by row.  The weights are the A operand, so a lane holds one position and
// four runs of 4 consecutive channels: 8-byte bf16 stores channels-last, or
// fp32 stores channels-first (the pixel / latent outputs, where consecutive
// lanes write consecutive positions of one channel).
constexpr int CV_BM = 128;
constexpr int CV_BK = 32;     // k-tile width used by the dispatch

// 16-byte chunk swizzle of a row of BK elements: the 16 lanes of one
// ds_read_b128 pass (16 consecutive rows, one logical chunk) land on 16
// distinct 16-byte bank groups
template <int BK>
SD_DEV int cv_swz(int row) {
  return (row / (128 / BK)) & (BK / 8 - 1);
}

template <int BN, int BK>
__global__ __launch_bounds__(256) void conv3d_mfma_kernel(ConvArgs a) {
  constexpr int WMW = BN >= 64 ? 2 : 4, WNW = 4 / WMW;   // waves along positions / channels
  constexpr int TMP = CV_BM / WMW, TNC = BN / WNW;      // wave tile: positions x channels
  constexpr int MB = TMP / 32, NB = TNC / 32;           // 32 x 32 blocks per wave
  constexpr int CPR = BK / 8, RPP = 256 / CPR;          // chunks per row, rows per pass of 256 threads
  constexpr int RA = CV_BM / RPP;                       // input chunks per thread per k-tile
  constexpr int RB = (BN + RPP - 1) / RPP;              // weight chunks per thread per k-tile
  static_assert(MB >= 1 && NB >= 1 && RA >= 1, "wave tile");
  __shared__ __attribute__((aligned(16))) bf16 As[2][CV_BM * BK];
  __shared__ __attribute__((aligned(16))) bf16 Bs[2][BN * BK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave / WMW, wm = wave % WMW;
  const int HW = a.H * a.W;
  const int M = a.T * HW;
  const int K = 27 * a.Cin;
  const int KT = (K + BK - 1) / BK;
  const int tiles_m = (M + CV_BM - 1) / CV_BM;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int tm = lid % tiles_m, tn = lid / tiles_m;
  const int m0 = tm * CV_BM, n0 = tn * BN;

  // staged chunks of this thread: input rows r0 + RPP i, weight rows
  // r0 + RPP i, all at chunk ck of the k-tile
  const int ck = tid % CPR, r0 = tid / CPR;
  int pt[RA], py[RA], px[RA];
  bool pv[RA];
#pragma unroll
  for (int i = 0; i < RA; ++i) {
    const int p = m0 + r0 + RPP * i;
    pv[i] = p < M;
    const int pp = pv[i] ? p : 0;
    pt[i] = pp / HW;
    const int rem = pp - pt[i] * HW;
    py[i] = rem / a.W;
    px[i] = rem - py[i] * a.W;
  }
  const bf16x8 zero8 = {};
  bf16x8 ra[RA], rb[RB];
  auto load = [&](int kt) {
    const int k = kt * BK + ck * 8;
    const bool kv = k < K;
#pragma unroll
    for (int i = 0; i < RA; ++i) {
      const bf16* src = (kv && pv[i]) ? conv_src(a, pt[i], py[i], px[i], k, HW) : nullptr;
      ra[i] = src ? *(const bf16x8*)src : zero8;
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int n = n0 + r0 + RPP * i;
      rb[i] = (kv && r0 + RPP * i < BN && n < a.Cout) ? *(const bf16x8*)(a.w + (int64_t)n * K + k) : zero8;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < RA; ++i) {
      const int r = r0 + RPP * i;
      *(bf16x8*)&As[buf][r * BK + ((ck ^ cv_swz<BK>(r)) * 8)] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int r = r0 + RPP * i;
      if (r < BN) *(bf16x8*)&Bs[buf][r * BK + ((ck ^ cv_swz<BK>(r)) * 8)] = rb[i];
    }
  };

  f32x16 acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  const int lr = lane & 31, lh = lane >> 5;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) load(kt + 1);            // in flight during this k-tile's MFMAs
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int c = s * 2 + lh;
      bf16x8 fw[NB], fp[MB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int row = wn * TNC + i * 32 + lr;
        fw[i] = *(const bf16x8*)&Bs[buf][row * BK + ((c ^ cv_swz<BK>(row)) * 8)];
      }
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const int row = wm * TMP + j * 32 + lr;
        fp[j] = *(const bf16x8*)&As[buf][row * BK + ((c ^ cv_swz<BK>(row)) * 8)];
      }
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[i], fp[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) store(buf ^ 1);
    __syncthreads();
  }

  // lane: position column lr of each 32-position block; channel rows
  // 8 (q / 4) + 4 lh + (q % 4) of each 32-channel block
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    const int p = m0 + wm * TMP + j * 32 + lr;
    if (p >= M) continue;
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * TNC + i * 32 + 8 * g + 4 * lh;
        if (n >= a.Cout) continue;
        if (a.ycf) {
          const int t = p / HW, hw = p - t * HW;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < a.Cout)
              a.ycf[((int64_t)t * a.Cout + n + e) * HW + hw] = acc[i][j][4 * g + e] + (a.b ? (float)a.b[n + e] : 0.f);
        } else {
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (bf16)(acc[i][j][4 * g + e] + (a.b ? (float)a.b[n + e] : 0.f));
          *(bf16x4*)(a.y + (int64_t)p * a.Cout + n) = o;
        }
      }
  }
}

hipError_t conv3d(hipStream_t s, const ConvArgs& a) {
  if (a.Cin < 8 || (a.Cin & 7) || a.Cout < 1 || a.T < 1 || a.H < 1 || a.W < 1) return hipErrorInvalidValue;
  if (a.ycf ? false : (!a.y || (a.Cout & 3))) return hipErrorInvalidValue;
  const int64_t M = (int64_t)a.T * a.H * a.W;
  if (M * a.Cout >= (1ll << 31) || M * a.Cin >= (1ll << 31) || 27ll * a.Cin * a.Cout >= (1ll << 31))
    return hipErrorInvalidValue;
  const int tiles_m = (int)((M + CV_BM - 1) / CV_BM);
  if (a.Cout <= 32) {
    conv3d_mfma_kernel<32, CV_BK><<<tiles_m * ((a.Cout + 31) / 32), 256, 0, s>>>(a);
  } else if (a.Cout <= 64) {
    conv3d_mfma_kernel<64, CV_BK><<<tiles_m * ((a.Cout + 63) / 64), 256, 0, s>>>(a);
  } else {
    conv3d_mfma_kernel<128, CV_BK><<<tiles_m * ((a.Cout + 127) / 128), 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// RMS norm over the C channels of a position, gain g, then SiLU, in place.
// C / 8 lanes per position, 8 channels each; the sum of squares is reduced
// with butterfly shuffles inside the lane group (every lane takes part).
template <int C>
__global__ __launch_bounds__(256) void norm_silu_kernel(bf16* __restrict__ x, const bf16* __restrict__ g, int64_t P,
                                                        float eps) {
  constexpr int LP = C / 8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t p = gid / LP;
  const int c0 = (int)(gid % LP) * 8;
  const bool ok = p < P;
  bf16x8 v = {};
  if (ok) v = *(const bf16x8*)(x + p * C + c0);
  float f[8], ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    f[e] = (float)v[e];
    ss = fmaf(f[e], f[e], ss);
  }
#pragma unroll
  for (int off = LP / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, LP);
  const float r = 1.0f / sqrtf(ss / (float)C + eps);
  if (!ok) return;
  const bf16x8 gv = *(const bf16x8*)(g + c0);
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float n = f[e] * r * (float)gv[e];
    o[e] = (bf16)(n / (1.0f + __expf(-n)));
  }
  *(bf16x8*)(x + p * C + c0) = o;
}

hipError_t norm_silu(hipStream_t s, void* x, const void* g, int64_t P, int C, float eps) {
  const int64_t n = P * (C / 8);
  const unsigned grid = (unsigned)((n + 255) / 256);
  switch (C) {
    case 16: norm_silu_kernel<16><<<grid, 256, 0, s>>>((bf16*)x, (const bf16*)g, P, eps); break;
    case 32: norm_silu_kernel<32><<<grid, 256, 0, s>>>((bf16*)x, (const bf16*)g, P, eps); break;
    case 64: norm_silu_kernel<64><<<grid, 256, 0, s>>>((bf16*)x, (const bf16*)g, P, eps); break;
    case 128: norm_silu_kernel<128><<<grid, 256, 0, s>>>((bf16*)x, (const bf16*)g, P, eps); break;
    case 256: norm_silu_kernel<256><<<grid, 256, 0, s>>>((bf16*)x, (const bf16*)g, P, eps); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 2 x 2 (x 2 in time) average pooling and nearest 2x upsampling, one thread
// per 8-channel chunk of an output position.
__global__ void pool_kernel(const bf16* __restrict__ x, bf16* __restrict__ y, int T, int H, int W, int C,
                            int temporal) {
  const int To = temporal ? T / 2 : T, Ho = H / 2, Wo = W / 2, C8 = C / 8;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)To * Ho * Wo * C8) return;
  const int c = (int)(i % C8) * 8;
  int64_t r = i / C8;
  const int xo = (int)(r % Wo);
  r /= Wo;
  const int yo = (int)(r % Ho);
  const int to = (int)(r / Ho);
  float acc[8] = {};
  const int nt = temporal ? 2 : 1;
  for (int dt = 0; dt < nt; ++dt)
    for (int dy = 0; dy < 2; ++dy)
      for (int dx = 0; dx < 2; ++dx) {
        const int t = temporal ? 2 * to + dt : to;
        const bf16x8 v = *(const bf16x8*)(x + (((int64_t)t * H + 2 * yo + dy) * W + 2 * xo + dx) * C + c);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += (float)v[e];
      }
  const float sc = temporal ? 0.125f : 0.25f;
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (bf16)(acc[e] * sc);
  *(bf16x8*)(y + i * 8) = o;
}

__global__ void upsample_kernel(const bf16* __restrict__ x, bf16* __restrict__ y, int T, int H, int W, int C,
                                int temporal) {
  const int To = temporal ? 2 * T : T, Ho = 2 * H, Wo = 2 * W, C8 = C / 8;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)To * Ho * Wo * C8) return;
  const int c = (int)(i % C8) * 8;
  int64_t r = i / C8;
  const int xo = (int)(r % Wo);
  r /= Wo;
  const int yo = (int)(r % Ho);
  const int to = (int)(r / Ho);
  const int t = temporal ? to / 2 : to;
  *(bf16x8*)(y + i * 8) = *(const bf16x8*)(x + (((int64_t)t * H + yo / 2) * W + xo / 2) * C + c);
}

hipError_t resample(hipStream_t s, const void* x, void* y, int T, int H, int W, int C, int mode) {
  // mode 0 pool 2x2, 1 pool 2x2x2, 2 upsample 2x2, 3 upsample 2x2x2
  if ((C & 7) || T < 1 || H < 1 || W < 1 || mode < 0 || mode > 3) return hipErrorInvalidValue;
  const bool pool = mode < 2, temporal = mode & 1;
  int64_t n;
  if (pool) {
    if ((H & 1) || (W & 1) || (temporal && (T & 1))) return hipErrorInvalidValue;
    n = (int64_t)(temporal ? T / 2 : T) * (H / 2) * (W / 2) * (C / 8);
  } else {
    n = (int64_t)(temporal ? 2 * T : T) * (2 * H) * (2 * W) * (C / 8);
  }
  const unsigned g = (unsigned)((n + 255) / 256);
  if (pool)
    pool_kernel<<<g, 256, 0, s>>>((const bf16*)x, (bf16*)y, T, H, W, C, temporal);
  else
    upsample_kernel<<<g, 256, 0, s>>>((const bf16*)x, (bf16*)y, T, H, W, C, temporal);
  return hipGetLastError();
}

// fp32 channels-first [T][C][H][W] -> bf16 channels-last [T][H][W][Cp],
// channels C .. Cp-1 zero; one thread per (position, 8-channel chunk).
__global__ void to_channels_last_kernel(const float* __restrict__ x, bf16* __restrict__ y, int T, int C, int HW,
                                        int Cp) {
  const int C8 = Cp / 8;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * HW * C8) return;
  const int c0 = (int)(i % C8) * 8;
  const int64_t pos = i / C8;
  const int t = (int)(pos / HW), hw = (int)(pos % HW);
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = c0 + e;
    o[e] = (bf16)(c < C ? x[((int64_t)t * C + c) * HW + hw] : 0.f);
  }
  *(bf16x8*)(y + i * 8) = o;
}

hipError_t to_channels_last(hipStream_t s, const float* x, void* y, int T, int C, int HW, int Cp) {
  if (Cp < C || (Cp & 7) || T < 1 || HW < 1) return hipErrorInvalidValue;
  const int64_t n = (int64_t)T * HW * (Cp / 8);
  to_channels_last_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(x, (bf16*)y, T, C, HW, Cp);
  return hipGetLastError();
}

}  // namespace sdk
