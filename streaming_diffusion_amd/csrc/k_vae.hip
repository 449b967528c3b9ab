// Stream-VAE kernels (StreamDiffusionV2 summary, Stream-VAE: short chunks,
// intermediate features cached inside every 3D convolution).  Activations are
// bf16 channels-last [T][H][W][C]; a causal 3x3x3 convolution reads input
// frames t-2, t-1, t, taking frames before the chunk from the layer's cache
// (the last two input frames of the previous chunk), with spatial zero
// padding.  Weights [Cout][3][3][3][Cin] (taps (dt, dy, dx)), i.e. a row of
// K = 27 Cin per output channel.
#include "kernels.h"

namespace sdk {

// 16-bit activation element: bf16, or fp16 (H16) for the Stream-VAE's own
// chain, whose values are bounded (normalised activations, unit-gain
// convolutions) and gain three mantissa bits in fp16 at the same matrix-core
// rate.  Data movement treats both as raw 16-bit words.
template <bool H16>
SD_DEV bf16 to16(float v) {
  if constexpr (H16) return __builtin_bit_cast(bf16, (f16)v);
  else return (bf16)v;
}
template <bool H16>
SD_DEV float from16(bf16 v) {
  if constexpr (H16) return (float)__builtin_bit_cast(f16, v);
  else return (float)v;
}

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

template <int BN, int BK, bool H16>
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
        for (int j = 0; j < MB; ++j) {
          if constexpr (H16)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, fw[i]),
                                                               __builtin_bit_cast(f16x8, fp[j]), acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[i], fp[j], acc[i][j], 0, 0, 0);
        }
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
          for (int e = 0; e < 4; ++e) o[e] = to16<H16>(acc[i][j][4 * g + e] + (a.b ? (float)a.b[n + e] : 0.f));
          *(bf16x4*)(a.y + (int64_t)p * a.Cout + n) = o;
        }
      }
  }
}

// ---------------------------------------------------------------------------
// The same implicit GEMM for the wide layers (Cin and Cout multiples of 64,
// enough positions to fill the chip): workgroup tile BM positions x BN
// channels, 8 waves (WMW along positions x 8 / WMW along channels, each a
// 64 x 64 block of outputs), k-tiles of 64 that lie inside one tap
// (Cin % 64 == 0), so the tap's (dt, dy, dx) shift is uniform per k-tile.
// Both operands go global -> LDS by DMA (global_load_lds, 16 bytes per lane,
// no register staging) into NS stages: the DMA of k-tile t + NS - 1 leaves
// while tile t is multiplied.  A gathered input row whose tap falls outside
// the frame (or before the chunk without a cache) reads a 16-byte zero row in
// device memory instead.  256 x 128 tiles with 3 stages for 128-channel
// outputs, 512 x 64 with 2 stages for 64-channel outputs.
static __device__ __attribute__((aligned(64))) bf16 conv_zero_row[8];

template <int n>
SD_DEV void conv_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(n) : "memory");
}

template <int BM, int BN, int WMW, int NS, bool H16>
__global__ __launch_bounds__(512) void conv3d_dma_kernel(ConvArgs a) {
  constexpr int BK = 64;
  constexpr int WNW = 8 / WMW;                          // waves along positions / channels
  constexpr int TMP = BM / WMW, TNC = BN / WNW;         // wave tile: positions x channels
  constexpr int MB = TMP / 32, NB = TNC / 32;           // 32 x 32 blocks per wave
  constexpr int AQ = BM / 64, BQ = BN / 64;             // DMA instructions per wave per k-tile (8 rows each)
  constexpr int DQ = AQ + BQ;
  constexpr int STAGE = (BM + BN) * BK;
  static_assert(NB >= 1 && MB >= 1 && BQ >= 1 && (NS == 2 || NS == 3), "tile shape");
  __shared__ __attribute__((aligned(1024))) bf16 smem[NS * STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave / WMW, wm = wave % WMW;
  const int HW = a.H * a.W;
  const int M = a.T * HW;
  const int K = 27 * a.Cin;
  const int KT = K / BK;
  const int tiles_m = (M + BM - 1) / BM;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int tm = lid % tiles_m, tn = lid / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const bf16* const zero = conv_zero_row;

  // this lane's DMA rows: row (wave * Q + q) * 8 + lane / 8 of the tile, its
  // 16-byte LDS slot lane % 8 holds logical chunk (lane % 8) ^ swz(row)
  const int lrow = lane >> 3, lpos = lane & 7;
  int pt[AQ], py[AQ], px[AQ], ach[AQ];
  bool pv[AQ];
#pragma unroll
  for (int q = 0; q < AQ; ++q) {
    const int row = (wave * AQ + q) * 8 + lrow;
    const int p = m0 + row;
    pv[q] = p < M;
    const int pp = pv[q] ? p : 0;
    pt[q] = pp / HW;
    const int rem = pp - pt[q] * HW;
    py[q] = rem / a.W;
    px[q] = rem - py[q] * a.W;
    ach[q] = (lpos ^ cv_swz<BK>(row)) * 8;
  }
  const bf16* wsrc[BQ];
#pragma unroll
  for (int q = 0; q < BQ; ++q) {
    const int row = (wave * BQ + q) * 8 + lrow;
    const int n = n0 + row;
    wsrc[q] = n < a.Cout ? a.w + (int64_t)n * K + (lpos ^ cv_swz<BK>(row)) * 8 : nullptr;
  }
  auto dma = [](const bf16* src, bf16* lds) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
  };
  auto issue = [&](int kt, int buf) {
    const int k0 = kt * BK;
    const int tap = k0 / a.Cin, ci0 = k0 - tap * a.Cin;
    const int dt = tap / 9, dy = (tap / 3) % 3, dx = tap % 3;
    bf16* as = smem + buf * STAGE;
    bf16* bs = as + BM * BK;
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
      const int t2 = pt[q] + dt - 2, y2 = py[q] + dy - 1, x2 = px[q] + dx - 1;
      const bf16* src = zero;
      if (pv[q] && (unsigned)y2 < (unsigned)a.H && (unsigned)x2 < (unsigned)a.W) {
        if (t2 >= 0)
          src = a.x + ((int64_t)t2 * HW + (int64_t)y2 * a.W + x2) * a.Cin + ci0 + ach[q];
        else if (a.cache)
          src = a.cache + ((int64_t)(t2 + 2) * HW + (int64_t)y2 * a.W + x2) * a.Cin + ci0 + ach[q];
      }
      dma(src, as + (wave * AQ + q) * 8 * BK);
    }
#pragma unroll
    for (int q = 0; q < BQ; ++q) dma(wsrc[q] ? wsrc[q] + k0 : zero, bs + (wave * BQ + q) * 8 * BK);
  };

  f32x16 acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  const int lr = lane & 31, lh = lane >> 5;
  issue(0, 0);
  if (NS == 3 && KT > 1) issue(1, 1);
  for (int kt = 0; kt < KT; ++kt) {
    // k-tile kt has landed in every wave (with 3 stages kt + 1 may stay in
    // flight) and every wave is done with the stage the next DMA overwrites
    if (NS == 3 && kt + 1 < KT) conv_wait_barrier<DQ>();
    else conv_wait_barrier<0>();
    if (kt + NS - 1 < KT) issue(kt + NS - 1, (kt + NS - 1) % NS);
    const bf16* as = smem + (kt % NS) * STAGE;
    const bf16* bs = as + BM * BK;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int c = ks * 2 + lh;
      bf16x8 fw[NB], fp[MB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int row = wn * TNC + i * 32 + lr;
        fw[i] = *(const bf16x8*)&bs[row * BK + ((c ^ cv_swz<BK>(row)) * 8)];
      }
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const int row = wm * TMP + j * 32 + lr;
        fp[j] = *(const bf16x8*)&as[row * BK + ((c ^ cv_swz<BK>(row)) * 8)];
      }
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j) {
          if constexpr (H16)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, fw[i]),
                                                               __builtin_bit_cast(f16x8, fp[j]), acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[i], fp[j], acc[i][j], 0, 0, 0);
        }
    }
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
          for (int e = 0; e < 4; ++e) o[e] = to16<H16>(acc[i][j][4 * g + e] + (a.b ? (float)a.b[n + e] : 0.f));
          *(bf16x4*)(a.y + (int64_t)p * a.Cout + n) = o;
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Direct convolution for the layers of a whole 4-frame chunk: a workgroup
// computes all 4 output frames x 8 rows x 16 columns (512 positions) x BN
// output channels.  The input it reads -- frames t-2 .. t+3 (the two before
// the chunk from the cache), one row and one column beyond the tile on each
// side -- is a halo of 6 x 10 x 18 positions.  Per chunk of 32 input channels
// the halo is DMA'd into LDS once (64-byte rows, 16-byte chunks XOR-swizzled
// by row; positions outside the frame read a zero row), and all 27 taps read
// their operand rows from it at their (dt, dy, dx) offsets: each input
// element crosses from L2 once per output tile instead of once per tap.  The
// next chunk's halo loads into the second buffer while this chunk's 27 x 2
// products run.  Weight fragments (the first matrix-core operand) come from
// device memory straight into registers, one tap ahead.  8 waves: WMW along
// positions x 8 / WMW along channels.
template <int BN, int WMW, bool H16>
__global__ __launch_bounds__(512) void conv3d_halo_kernel(ConvArgs a) {
  constexpr int TT = 4, TY = 8, TX = 16;                // output tile: frames x rows x columns
  constexpr int HY = TY + 2, HX = TX + 2, HT = TT + 2;  // halo
  constexpr int HROWS = HT * HY * HX;                   // 1080
  constexpr int CK = 32;                                // input channels per chunk: 64-byte rows
  constexpr int HINS = (HROWS + 15) / 16;               // DMA instructions per halo (16 rows each)
  constexpr int HQ = (HINS + 7) / 8;                    // per wave
  constexpr int HBUF = HINS * 16 * CK;                  // elements per halo buffer
  constexpr int WNW = 8 / WMW;
  constexpr int TMP = TT * TY * TX / WMW, TNC = BN / WNW;
  constexpr int MB = TMP / 32, NB = TNC / 32;
  static_assert(MB >= 1 && NB >= 1 && WMW * WNW == 8, "wave layout");
  // two halo buffers as separate arrays: the compiler can then tell that the
  // DMA into one does not write what the products read from the other
  __shared__ __attribute__((aligned(1024))) bf16 halo0[HBUF];
  __shared__ __attribute__((aligned(1024))) bf16 halo1[HBUF];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WMW, wn = wave / WMW;
  const int HW = a.H * a.W;
  const int K = 27 * a.Cin;
  const int tiles_x = (a.W + TX - 1) / TX, tiles_n = a.Cout / BN;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  // channel tiles of one spatial tile are neighbours: they read the same halo
  const int tn = lid % tiles_n, txy = lid / tiles_n;
  const int y0 = (txy / tiles_x) * TY, x0 = (txy % tiles_x) * TX, n0 = tn * BN;
  const bf16* const zero = conv_zero_row;

  // this lane's halo rows: row (wave * HQ + q) * 16 + lane / 4; its 16-byte
  // LDS slot lane % 4 holds logical chunk (lane % 4) ^ swz(row).  With an
  // upsampled input the row (y, x) is read from (y / 2, x / 2) of the
  // half-size frames.
  const int us = a.up ? 1 : 0;
  const int Ws = a.W >> us, HWs = (a.H >> us) * Ws;
  const bf16* hsrc[HQ];
#pragma unroll
  for (int q = 0; q < HQ; ++q) {
    const int ins = wave * HQ + q;
    const int row = ins * 16 + (lane >> 2);
    const bf16* src = nullptr;
    if (ins < HINS && row < HROWS) {
      const int ft = row / (HY * HX), hy = (row / HX) % HY, hx = row % HX;
      const int ti = ft - 2, y = y0 + hy - 1, x = x0 + hx - 1;
      if ((unsigned)y < (unsigned)a.H && (unsigned)x < (unsigned)a.W) {
        const int64_t sp = (int64_t)(y >> us) * Ws + (x >> us);
        if (ti >= 0)
          src = a.x + ((int64_t)ti * HWs + sp) * a.Cin;
        else if (a.cache)
          src = a.cache + ((int64_t)(ti + 2) * HWs + sp) * a.Cin;
      }
      if (src) src += ((lane & 3) ^ cv_swz<CK>(row)) * 8;
    }
    hsrc[q] = src;
  }
  auto issue_halo = [&](int cc, bf16* buf) {
#pragma unroll
    for (int q = 0; q < HQ; ++q) {
      const int ins = wave * HQ + q;
      if (ins < HINS)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(hsrc[q] ? hsrc[q] + cc * CK : zero),
            (__attribute__((address_space(3))) void*)(buf + ins * 16 * CK), 16, 0, 0);
    }
  };
  // halo row of tap (0, 0, 0) for each of this lane's position blocks
  const int lr = lane & 31, lh = lane >> 5;
  int hbase[MB];
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    const int pw = wm * TMP + j * 32 + lr;
    const int tf = pw / (TY * TX), r = (pw / TX) % TY, c = pw % TX;
    hbase[j] = (tf * HY + r) * HX + c;
  }
  // weight fragments of (chunk cc, tap): rows n0 + wn TNC + 32 i + l % 32
  const bf16* wrow[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) wrow[i] = a.w + (int64_t)(n0 + wn * TNC + i * 32 + lr) * K + lh * 8;
  auto load_w = [&](int cc, int tap, bf16x8 (&wf)[2][NB]) {
    const int k = tap * a.Cin + cc * CK;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < NB; ++i) wf[ks][i] = *(const bf16x8*)(wrow[i] + k + ks * 16);
  };

  f32x16 acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  const int NC = a.Cin / CK;
  bf16x8 wcur[2][NB], wnxt[2][NB];
  // one chunk: products from the halo in rd while the next chunk's halo
  // streams into wr
  auto chunk = [&](int cc, const bf16* rd, bf16* wr) {
    // the halo of chunk cc and the weights of (cc, tap 0) have landed in
    // every wave; every wave is done with the buffer the next halo
    // overwrites.  (A wait the compiler sees: otherwise the first products
    // after the next halo's DMA would wait for that DMA too.)
    __builtin_amdgcn_s_waitcnt(0x0070);               // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    if (cc + 1 < NC) issue_halo(cc + 1, wr);
    __builtin_amdgcn_sched_barrier(0);
    for (int tap = 0; tap < 27; ++tap) {
      if (tap < 26) load_w(cc, tap + 1, wnxt);
      else if (cc + 1 < NC) load_w(cc + 1, 0, wnxt);
      const int dt = tap / 9, dy = (tap / 3) % 3, dx = tap % 3;
      const int toff = (dt * HY + dy) * HX + dx;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int c = ks * 2 + lh;
        bf16x8 fp[MB];
#pragma unroll
        for (int j = 0; j < MB; ++j) {
          const int row = hbase[j] + toff;
          fp[j] = *(const bf16x8*)(rd + row * CK + ((c ^ cv_swz<CK>(row)) * 8));
        }
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int j = 0; j < MB; ++j) {
            if constexpr (H16)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, wcur[ks][i]),
                                                                 __builtin_bit_cast(f16x8, fp[j]), acc[i][j], 0, 0, 0);
            else
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wcur[ks][i], fp[j], acc[i][j], 0, 0, 0);
          }
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < NB; ++i) wcur[ks][i] = wnxt[ks][i];
    }
  };
  issue_halo(0, halo0);
  __builtin_amdgcn_sched_barrier(0);
  load_w(0, 0, wcur);
  for (int cc = 0; cc < NC; cc += 2) {
    chunk(cc, halo0, halo1);
    if (cc + 1 < NC) chunk(cc + 1, halo1, halo0);
  }

  // lane: position column lr of each 32-position block; channel rows
  // 8 (q / 4) + 4 lh + (q % 4) of each 32-channel block
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    const int pw = wm * TMP + j * 32 + lr;
    const int tf = pw / (TY * TX), y = y0 + (pw / TX) % TY, x = x0 + pw % TX;
    if (y >= a.H || x >= a.W) continue;
    const int64_t p = (int64_t)tf * HW + (int64_t)y * a.W + x;
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * TNC + i * 32 + 8 * g + 4 * lh;
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = to16<H16>(acc[i][j][4 * g + e] + (a.b ? (float)a.b[n + e] : 0.f));
        *(bf16x4*)(a.y + p * a.Cout + n) = o;
      }
  }
}

// The same halo scheme for layers with at most 16 output channels (the
// encoder's latent projection, 16 channels, and the decoder's pixel
// projection, 3): 16 x 16 x 32 matrix-core products, the weights (zero rows
// past Cout) as the first operand -- one 16-byte fragment per lane covers a
// whole 32-channel chunk of one tap, so all 27 taps of a chunk sit in
// registers, loaded while the previous chunk runs -- and 16 output positions
// along x as the second, read from the halo.  NW waves, each 1 / NW of the
// TT x TY x 16 positions.  A product reads as many halo bytes as it does
// work, so these layers are bound by the LDS reads, which is still far less
// traffic than gathering every tap's input from memory.  Output: fp32
// channels-first (ycf) or 16-bit channels-last (Cout a multiple of 4).
//
// NBUF = 1 keeps a single halo buffer (the next chunk's halo is DMA'd after
// every wave is done with this one), so two workgroups fit on a CU and one
// computes while the other waits for its halo.
template <int TT, int TY, int NW, int NBUF, bool H16>
__global__ __launch_bounds__(64 * NW, NBUF == 1 ? 2 : 1) void conv3d_halo16_kernel(ConvArgs a) {
  constexpr int TX = 16;
  constexpr int HY = TY + 2, HX = TX + 2, HT = TT + 2;
  constexpr int HROWS = HT * HY * HX;
  constexpr int CK = 32;
  constexpr int HINS = (HROWS + 15) / 16;               // DMA instructions per halo (16 rows each)
  constexpr int HQ = (HINS + NW - 1) / NW;              // per wave
  constexpr int HBUF = HINS * 16 * CK;
  constexpr int PW = TT * TY * TX / NW, MB = PW / 16;   // positions per wave, blocks of 16
  static_assert(MB >= 1 && PW % 16 == 0 && (NBUF == 1 || NBUF == 2), "wave tile");
  __shared__ __attribute__((aligned(1024))) bf16 halo0[HBUF];
  __shared__ __attribute__((aligned(1024))) bf16 halo1[NBUF == 2 ? HBUF : 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int HW = a.H * a.W;
  const int K = 27 * a.Cin;
  const int tiles_x = (a.W + TX - 1) / TX;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int y0 = (lid / tiles_x) * TY, x0 = (lid % tiles_x) * TX;
  const bf16* const zero = conv_zero_row;

  // this lane's halo rows as 32-bit element offsets (registers are tight):
  // >= 0 into x, <= -2 into the cache (-2 - offset), -1 the zero row
  int hoff[HQ];
#pragma unroll
  for (int q = 0; q < HQ; ++q) {
    const int ins = wave * HQ + q;
    const int row = ins * 16 + (lane >> 2);
    int off = -1;
    if (ins < HINS && row < HROWS) {
      const int ft = row / (HY * HX), hy = (row / HX) % HY, hx = row % HX;
      const int ti = ft - 2, y = y0 + hy - 1, x = x0 + hx - 1;
      const int sw = ((lane & 3) ^ cv_swz<CK>(row)) * 8;
      if ((unsigned)y < (unsigned)a.H && (unsigned)x < (unsigned)a.W) {
        if (ti >= 0)
          off = (ti * HW + y * a.W + x) * a.Cin + sw;
        else if (a.cache)
          off = -2 - (((ti + 2) * HW + y * a.W + x) * a.Cin + sw);
      }
    }
    hoff[q] = off;
  }
  auto issue_halo = [&](int cc, bf16* buf) {
#pragma unroll
    for (int q = 0; q < HQ; ++q) {
      const int ins = wave * HQ + q;
      const int off = hoff[q];
      const bf16* src = off >= 0 ? a.x + off + cc * CK : (off == -1 ? zero : a.cache + (-2 - off) + cc * CK);
      if (ins < HINS)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                         (__attribute__((address_space(3))) void*)(buf + ins * 16 * CK), 16, 0, 0);
    }
  };
  // second operand: lane -> position (block base + lane % 16), channels
  // 8 (lane / 16) .. + 7 of the chunk; halo row of tap (0, 0, 0) per block
  const int l16 = lane & 15, lq = lane >> 4;
  int hbase[MB];
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    const int pw = wave * PW + j * 16 + l16;
    const int tf = pw / (TY * TX), r = (pw / TX) % TY, c = pw % TX;
    hbase[j] = (tf * HY + r) * HX + c;
  }
  // first operand: lane -> output channel lane % 16 (zero past Cout), the
  // same 8 channels of the chunk, every tap
  const bool wlive = l16 < a.Cout;
  const bf16* const wrow = a.w + (int64_t)(wlive ? l16 : 0) * K + lq * 8;
  bf16x8 wt[27];
  auto load_w = [&](int cc) {
#pragma unroll
    for (int tap = 0; tap < 27; ++tap) {
      bf16x8 v = {};
      if (wlive) v = *(const bf16x8*)(wrow + tap * a.Cin + cc * CK);
      wt[tap] = v;
    }
  };

  f32x4 acc[MB];
#pragma unroll
  for (int j = 0; j < MB; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[j][q] = 0.f;

  const int NC = a.Cin / CK;
  auto chunk = [&](int cc, const bf16* rd, bf16* wr) {
    // halo and weights of chunk cc landed in every wave; every wave is done
    // with the buffer the next halo overwrites
    __builtin_amdgcn_s_waitcnt(0x0070);               // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    if (NBUF == 2 && cc + 1 < NC) issue_halo(cc + 1, wr);
    __builtin_amdgcn_sched_barrier(0);
    // halo fragments one tap ahead of the products (two register sets); a
    // scheduling fence per tap keeps the compiler from hoisting every tap's
    // reads, which would not fit in registers
    auto read_tap = [&](int tap, bf16x8* fp) {
      const int dt = tap / 9, dy = (tap / 3) % 3, dx = tap % 3;
      const int toff = (dt * HY + dy) * HX + dx;
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const int row = hbase[j] + toff;
        fp[j] = *(const bf16x8*)(rd + row * CK + ((lq ^ cv_swz<CK>(row)) * 8));
      }
    };
    // the 27 x MB swizzled read addresses do not change between chunks; left
    // to itself the compiler keeps them all in registers across the chunk
    // loop and spills, so they are recomputed per tap
#pragma unroll
    for (int j = 0; j < MB; ++j) asm volatile("" : "+v"(hbase[j]));
    // (with one halo buffer two workgroups share the CU and hide each
    // other's read latency: a single register set)
    constexpr int NF = NBUF == 2 ? MB : 1;
    bf16x8 fa[MB], fb[NF];
    read_tap(0, fa);
#pragma unroll
    for (int tap = 0; tap < 27; ++tap) {
      bf16x8* cur = fa;
      if constexpr (NBUF == 2) {
        cur = (tap & 1) ? fb : fa;
        if (tap < 26) read_tap(tap + 1, (tap & 1) ? fa : fb);
      } else if (tap > 0) {
        read_tap(tap, fa);
      }
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        if constexpr (H16)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, wt[tap]),
                                                          __builtin_bit_cast(f16x8, cur[j]), acc[j], 0, 0, 0);
        else
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wt[tap], cur[j], acc[j], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the next chunk's weights (and with one buffer its halo, once every
    // wave is done reading this one), in flight across the next barrier
    __builtin_amdgcn_sched_barrier(0);
    if (cc + 1 < NC) {
      if constexpr (NBUF == 1) {
        __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0): this wave's halo reads are done
        __builtin_amdgcn_s_barrier();
        issue_halo(cc + 1, wr);
      }
      load_w(cc + 1);
    }
  };
  issue_halo(0, halo0);
  load_w(0);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (NBUF == 1) {
    for (int cc = 0; cc < NC; ++cc) chunk(cc, halo0, halo0);
  } else {
    for (int cc = 0; cc < NC; cc += 2) {
      chunk(cc, halo0, halo1);
      if (cc + 1 < NC) chunk(cc + 1, halo1, halo0);
    }
  }

  // lane: position l % 16 of each block, output channels 4 (l / 16) + 0..3
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    const int pw = wave * PW + j * 16 + l16;
    const int tf = pw / (TY * TX), y = y0 + (pw / TX) % TY, x = x0 + pw % TX;
    if (y >= a.H || x >= a.W) continue;
    const int n = 4 * lq;
    if (n >= a.Cout) continue;
    if (a.ycf) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < a.Cout)
          a.ycf[(((int64_t)tf * a.Cout + n + e) * a.H + y) * a.W + x] = acc[j][e] + (a.b ? (float)a.b[n + e] : 0.f);
    } else {
      bf16x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = to16<H16>(acc[j][e] + (a.b ? (float)a.b[n + e] : 0.f));
      *(bf16x4*)(a.y + ((int64_t)tf * HW + (int64_t)y * a.W + x) * a.Cout + n) = o;
    }
  }
}

// The halo scheme for the first encoder layer, whose input has 8 channels
// (RGB and zero padding): the halo rows are 16 bytes (all channels of a
// position) and one 32 x 32 x 16 product covers two taps -- lanes 0-31
// supply tap 2s, lanes 32-63 tap 2s + 1 (the 28th tap is zero weights) -- so
// a tile needs 14 products per 32 x 32 block and its whole weight slice (14
// fragments) stays in registers.  One halo, one DMA round: 4 x 8 x 16
// positions x BN channels per workgroup of 8 waves (4 along positions x 2
// along channels).
template <int BN, bool H16>
__global__ __launch_bounds__(512) void conv3d_halo8_kernel(ConvArgs a) {
  constexpr int TT = 4, TY = 8, TX = 16;
  constexpr int HY = TY + 2, HX = TX + 2, HT = TT + 2;
  constexpr int HROWS = HT * HY * HX;                   // 1080 rows of 16 bytes
  constexpr int HINS = (HROWS + 63) / 64;               // DMA instructions (64 rows each)
  constexpr int HQ = (HINS + 7) / 8;
  constexpr int WMW = 4, WNW = 2;
  constexpr int TMP = TT * TY * TX / WMW, TNC = BN / WNW;
  constexpr int MB = TMP / 32, NB = TNC / 32, KS = 14;
  static_assert(MB >= 1 && NB >= 1, "wave tile");
  __shared__ __attribute__((aligned(1024))) bf16 halo[HINS * 64 * 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WMW, wn = wave / WMW;
  const int HW = a.H * a.W;
  const int tiles_x = (a.W + TX - 1) / TX, tiles_n = a.Cout / BN;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int tn = lid % tiles_n, txy = lid / tiles_n;
  const int y0 = (txy / tiles_x) * TY, x0 = (txy % tiles_x) * TX, n0 = tn * BN;
  const bf16* const zero = conv_zero_row;
#pragma unroll
  for (int q = 0; q < HQ; ++q) {
    const int ins = wave * HQ + q;
    const int row = ins * 64 + lane;
    if (ins < HINS) {
      const bf16* src = zero;
      if (row < HROWS) {
        const int ft = row / (HY * HX), hy = (row / HX) % HY, hx = row % HX;
        const int ti = ft - 2, y = y0 + hy - 1, x = x0 + hx - 1;
        if ((unsigned)y < (unsigned)a.H && (unsigned)x < (unsigned)a.W) {
          if (ti >= 0)
            src = a.x + ((int64_t)ti * HW + (int64_t)y * a.W + x) * 8;
          else if (a.cache)
            src = a.cache + ((int64_t)(ti + 2) * HW + (int64_t)y * a.W + x) * 8;
        }
      }
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(halo + ins * 64 * 8), 16, 0, 0);
    }
  }
  // weights: lane -> output channel (l % 32) of each block, tap 2 s + l / 32
  const int lr = lane & 31, lh = lane >> 5;
  bf16x8 wf[KS][NB];
#pragma unroll
  for (int s2 = 0; s2 < KS; ++s2) {
    const int tap = 2 * s2 + lh;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      bf16x8 v = {};
      if (tap < 27) v = *(const bf16x8*)(a.w + (int64_t)(n0 + wn * TNC + i * 32 + lr) * 216 + tap * 8);
      wf[s2][i] = v;
    }
  }
  int hbase[MB];
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    const int pw = wm * TMP + j * 32 + lr;
    const int tf = pw / (TY * TX), r = (pw / TX) % TY, c = pw % TX;
    hbase[j] = (tf * HY + r) * HX + c;
  }
  f32x16 acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  __builtin_amdgcn_s_waitcnt(0x0070);                   // vmcnt(0) lgkmcnt(0): halo and weights landed
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int s2 = 0; s2 < KS; ++s2) {
    const int tap = min(2 * s2 + lh, 26);               // tap 27 reads a real row against zero weights
    const int dt = tap / 9, dy = (tap / 3) % 3, dx = tap % 3;
    const int toff = (dt * HY + dy) * HX + dx;
    bf16x8 fp[MB];
#pragma unroll
    for (int j = 0; j < MB; ++j) fp[j] = *(const bf16x8*)(halo + (hbase[j] + toff) * 8);
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        if constexpr (H16)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, wf[s2][i]),
                                                             __builtin_bit_cast(f16x8, fp[j]), acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[s2][i], fp[j], acc[i][j], 0, 0, 0);
      }
  }
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    const int pw = wm * TMP + j * 32 + lr;
    const int tf = pw / (TY * TX), y = y0 + (pw / TX) % TY, x = x0 + pw % TX;
    if (y >= a.H || x >= a.W) continue;
    const int64_t p = (int64_t)tf * HW + (int64_t)y * a.W + x;
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * TNC + i * 32 + 8 * g + 4 * lh;
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = to16<H16>(acc[i][j][4 * g + e] + (a.b ? (float)a.b[n + e] : 0.f));
        *(bf16x4*)(a.y + p * a.Cout + n) = o;
      }
  }
}

bool conv3d_upsample_ok(int T, int H, int W, int Cin, int Cout) {
  if (T != 4 || Cin % 32 || Cout % 64 || (H & 1) || (W & 1)) return false;
  const int64_t tiles = (int64_t)((H + 7) / 8) * ((W + 15) / 16) * (Cout / (Cout % 128 == 0 ? 128 : 64));
  return tiles >= 256;
}

hipError_t conv3d(hipStream_t s, const ConvArgs& a) {
  if (a.Cin < 8 || (a.Cin & 7) || a.Cout < 1 || a.T < 1 || a.H < 1 || a.W < 1) return hipErrorInvalidValue;
  if (a.up && (a.ycf || !conv3d_upsample_ok(a.T, a.H, a.W, a.Cin, a.Cout))) return hipErrorInvalidValue;
  if (a.ycf ? false : (!a.y || (a.Cout & 3))) return hipErrorInvalidValue;
  const int64_t M = (int64_t)a.T * a.H * a.W;
  if (M * a.Cout >= (1ll << 31) || M * a.Cin >= (1ll << 31) || 27ll * a.Cin * a.Cout >= (1ll << 31))
    return hipErrorInvalidValue;
  const int tiles_m = (int)((M + CV_BM - 1) / CV_BM);
#define SD_CONV_LAUNCH(BN)                                                                  \
  do {                                                                                      \
    const unsigned g = (unsigned)(tiles_m * ((a.Cout + BN - 1) / BN));                      \
    if (a.h16) conv3d_mfma_kernel<BN, CV_BK, true><<<g, 256, 0, s>>>(a);                    \
    else conv3d_mfma_kernel<BN, CV_BK, false><<<g, 256, 0, s>>>(a);                         \
  } while (0)
  // 4-frame layers with 32-channel input chunks and 64- or 128-channel
  // output tiles: the halo kernel, when its tiles fill the chip
  if (a.T == 4 && !a.ycf && a.Cin % 32 == 0 && a.Cout % 64 == 0) {
    const bool wide = a.Cout % 128 == 0;
    const int64_t tiles = (int64_t)((a.H + 7) / 8) * ((a.W + 15) / 16) * (a.Cout / (wide ? 128 : 64));
    if (tiles >= 256) {
      const unsigned g = (unsigned)tiles;
      if (wide) {
        if (a.h16) conv3d_halo_kernel<128, 4, true><<<g, 512, 0, s>>>(a);
        else conv3d_halo_kernel<128, 4, false><<<g, 512, 0, s>>>(a);
      } else {
        if (a.h16) conv3d_halo_kernel<64, 4, true><<<g, 512, 0, s>>>(a);
        else conv3d_halo_kernel<64, 4, false><<<g, 512, 0, s>>>(a);
      }
      return hipGetLastError();
    }
  }
  // 4-frame layers with 8 input channels (the first encoder layer): one
  // halo of 16-byte rows, two taps per product
  if (a.T == 4 && a.Cin == 8 && !a.ycf && a.Cout % 64 == 0 &&
      (int64_t)((a.H + 7) / 8) * ((a.W + 15) / 16) * (a.Cout / 64) >= 256) {
    const unsigned g = (unsigned)(((a.H + 7) / 8) * ((a.W + 15) / 16) * (a.Cout / 64));
    if (a.h16) conv3d_halo8_kernel<64, true><<<g, 512, 0, s>>>(a);
    else conv3d_halo8_kernel<64, false><<<g, 512, 0, s>>>(a);
    return hipGetLastError();
  }
  // layers with at most 16 output channels (latent and pixel projections):
  // the narrow halo kernel, 4 x 8 x 16 tiles for 4 frames, 2 x 2 x 16 for 2
  if (a.Cout <= 16 && a.Cin % 32 == 0 && (a.T == 4 || a.T == 2)) {
    if (a.T == 4) {
      const unsigned g = (unsigned)(((a.H + 3) / 4) * ((a.W + 15) / 16));
      if (a.h16) conv3d_halo16_kernel<4, 4, 4, 1, true><<<g, 256, 0, s>>>(a);
      else conv3d_halo16_kernel<4, 4, 4, 1, false><<<g, 256, 0, s>>>(a);
    } else {
      const unsigned g = (unsigned)(((a.H + 1) / 2) * ((a.W + 15) / 16));
      if (a.h16) conv3d_halo16_kernel<2, 2, 4, 2, true><<<g, 256, 0, s>>>(a);
      else conv3d_halo16_kernel<2, 2, 4, 2, false><<<g, 256, 0, s>>>(a);
    }
    return hipGetLastError();
  }
  // wide layers with enough tiles to fill the chip twice take the DMA
  // kernel: 256 x 128 tiles when the output channels are a multiple of 128,
  // else 512 x 64
  if (a.Cin % 64 == 0 && a.Cout % 64 == 0) {
    const bool wide = a.Cout % 128 == 0;
    const int64_t tiles = wide ? ((M + 255) / 256) * (a.Cout / 128) : ((M + 511) / 512) * (a.Cout / 64);
    if (tiles >= 512) {
      const unsigned g = (unsigned)tiles;
      if (wide) {
        if (a.h16) conv3d_dma_kernel<256, 128, 4, 3, true><<<g, 512, 0, s>>>(a);
        else conv3d_dma_kernel<256, 128, 4, 3, false><<<g, 512, 0, s>>>(a);
      } else {
        if (a.h16) conv3d_dma_kernel<512, 64, 8, 2, true><<<g, 512, 0, s>>>(a);
        else conv3d_dma_kernel<512, 64, 8, 2, false><<<g, 512, 0, s>>>(a);
      }
      return hipGetLastError();
    }
    // the latent-resolution layers (12 480 positions): 128 x 64 tiles, two
    // workgroups per CU, so the grid still covers the chip
    const int64_t t64 = ((M + 127) / 128) * (a.Cout / 64);
    if (t64 >= 256) {
      const unsigned g = (unsigned)t64;
      if (a.h16) conv3d_dma_kernel<128, 64, 4, 3, true><<<g, 512, 0, s>>>(a);
      else conv3d_dma_kernel<128, 64, 4, 3, false><<<g, 512, 0, s>>>(a);
      return hipGetLastError();
    }
  }
  if (a.Cout <= 32) SD_CONV_LAUNCH(32);
  else if (a.Cout <= 64) SD_CONV_LAUNCH(64);
  else SD_CONV_LAUNCH(128);
#undef SD_CONV_LAUNCH
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// RMS norm over the C channels of a position, gain g, then SiLU, in place.
// C / 8 lanes per position, 8 channels each; the sum of squares is reduced
// with butterfly shuffles inside the lane group (every lane takes part).
template <int C, bool H16>
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
    f[e] = from16<H16>(v[e]);
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
    // SiLU n sigmoid(n) with the hardware reciprocal (1 ulp, far below the
    // 16-bit rounding of the stored value): n -> -inf gives -0, n -> +inf n
    const float n = f[e] * r * (float)gv[e];
    o[e] = to16<H16>(n * __builtin_amdgcn_rcpf(1.0f + __expf(-n)));
  }
  *(bf16x8*)(x + p * C + c0) = o;
}

hipError_t norm_silu(hipStream_t s, void* x, const void* g, int64_t P, int C, float eps, bool h16) {
  const int64_t n = P * (C / 8);
  const unsigned grid = (unsigned)((n + 255) / 256);
#define SD_NS(CC)                                                                                 \
  case CC:                                                                                        \
    if (h16) norm_silu_kernel<CC, true><<<grid, 256, 0, s>>>((bf16*)x, (const bf16*)g, P, eps);   \
    else norm_silu_kernel<CC, false><<<grid, 256, 0, s>>>((bf16*)x, (const bf16*)g, P, eps);      \
    break;
  switch (C) {
    SD_NS(16)
    SD_NS(32)
    SD_NS(64)
    SD_NS(128)
    SD_NS(256)
    default: return hipErrorInvalidValue;
  }
#undef SD_NS
  return hipGetLastError();
}

// RMS norm + SiLU of every input position followed by the 2 x 2 (x 2 in
// time) average pooling of the normalised values, in one pass: the encoder's
// layer outputs are read once and only the pooled quarter (eighth) is
// written.  C / 8 lanes per pooled position, 8 channels each; for each of
// its 4 (8) input positions the group reduces the sum of squares with
// butterfly shuffles, normalises its 8 channels and adds them in.
template <int C, bool H16, bool TEMPORAL>
__global__ __launch_bounds__(256) void norm_silu_pool_kernel(const bf16* __restrict__ x, const bf16* __restrict__ g,
                                                             bf16* __restrict__ y, int T, int H, int W, float eps) {
  constexpr int LP = C / 8;
  const int To = TEMPORAL ? T / 2 : T, Ho = H / 2, Wo = W / 2;
  const int64_t P = (int64_t)To * Ho * Wo;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t po = gid / LP;
  const int c0 = (int)(gid % LP) * 8;
  const bool ok = po < P;
  const int64_t pc = ok ? po : 0;
  const int xo = (int)(pc % Wo), yo = (int)((pc / Wo) % Ho), to = (int)(pc / ((int64_t)Wo * Ho));
  const bf16x8 gv = *(const bf16x8*)(g + c0);
  float acc[8] = {};
  constexpr int NT = TEMPORAL ? 2 : 1;
#pragma unroll
  for (int dt = 0; dt < NT; ++dt)
#pragma unroll
    for (int dy = 0; dy < 2; ++dy)
#pragma unroll
      for (int dx = 0; dx < 2; ++dx) {
        const int t = TEMPORAL ? 2 * to + dt : to;
        const bf16x8 v = *(const bf16x8*)(x + (((int64_t)t * H + 2 * yo + dy) * W + 2 * xo + dx) * C + c0);
        float f[8], ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          f[e] = from16<H16>(v[e]);
          ss = fmaf(f[e], f[e], ss);
        }
#pragma unroll
        for (int off = LP / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, LP);
        const float r = 1.0f / sqrtf(ss / (float)C + eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float n = f[e] * r * (float)gv[e];
          acc[e] += n * __builtin_amdgcn_rcpf(1.0f + __expf(-n));
        }
      }
  if (!ok) return;
  constexpr float sc = TEMPORAL ? 0.125f : 0.25f;
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = to16<H16>(acc[e] * sc);
  *(bf16x8*)(y + po * C + c0) = o;
}

hipError_t norm_silu_pool(hipStream_t s, const void* x, const void* g, void* y, int T, int H, int W, int C,
                          bool temporal, float eps, bool h16) {
  if ((H & 1) || (W & 1) || (temporal && (T & 1)) || T < 1 || H < 2 || W < 2) return hipErrorInvalidValue;
  const int64_t n = (int64_t)(temporal ? T / 2 : T) * (H / 2) * (W / 2) * (C / 8);
  const unsigned grid = (unsigned)((n + 255) / 256);
#define SD_NSP(CC)                                                                                          \
  case CC:                                                                                                  \
    if (h16 && temporal)                                                                                    \
      norm_silu_pool_kernel<CC, true, true><<<grid, 256, 0, s>>>((const bf16*)x, (const bf16*)g, (bf16*)y, T, H, W, eps); \
    else if (h16)                                                                                           \
      norm_silu_pool_kernel<CC, true, false><<<grid, 256, 0, s>>>((const bf16*)x, (const bf16*)g, (bf16*)y, T, H, W, eps); \
    else if (temporal)                                                                                      \
      norm_silu_pool_kernel<CC, false, true><<<grid, 256, 0, s>>>((const bf16*)x, (const bf16*)g, (bf16*)y, T, H, W, eps); \
    else                                                                                                    \
      norm_silu_pool_kernel<CC, false, false><<<grid, 256, 0, s>>>((const bf16*)x, (const bf16*)g, (bf16*)y, T, H, W, eps); \
    break;
  switch (C) {
    SD_NSP(16)
    SD_NSP(32)
    SD_NSP(64)
    SD_NSP(128)
    SD_NSP(256)
    default: return hipErrorInvalidValue;
  }
#undef SD_NSP
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 2 x 2 (x 2 in time) average pooling and nearest 2x upsampling, one thread
// per 8-channel chunk of an output position.
template <bool H16>
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
        for (int e = 0; e < 8; ++e) acc[e] += from16<H16>(v[e]);
      }
  const float sc = temporal ? 0.125f : 0.25f;
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = to16<H16>(acc[e] * sc);
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

hipError_t resample(hipStream_t s, const void* x, void* y, int T, int H, int W, int C, int mode, bool h16) {
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
  if (pool && h16)
    pool_kernel<true><<<g, 256, 0, s>>>((const bf16*)x, (bf16*)y, T, H, W, C, temporal);
  else if (pool)
    pool_kernel<false><<<g, 256, 0, s>>>((const bf16*)x, (bf16*)y, T, H, W, C, temporal);
  else
    upsample_kernel<<<g, 256, 0, s>>>((const bf16*)x, (bf16*)y, T, H, W, C, temporal);
  return hipGetLastError();
}

// fp32 channels-first [T][C][H][W] -> bf16 channels-last [T][H][W][Cp],
// channels C .. Cp-1 zero; one thread per (position, 8-channel chunk).
template <bool H16>
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
    o[e] = to16<H16>(c < C ? x[((int64_t)t * C + c) * HW + hw] : 0.f);
  }
  *(bf16x8*)(y + i * 8) = o;
}

hipError_t to_channels_last(hipStream_t s, const float* x, void* y, int T, int C, int HW, int Cp, bool h16) {
  if (Cp < C || (Cp & 7) || T < 1 || HW < 1) return hipErrorInvalidValue;
  const int64_t n = (int64_t)T * HW * (Cp / 8);
  if (h16)
    to_channels_last_kernel<true><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(x, (bf16*)y, T, C, HW, Cp);
  else
    to_channels_last_kernel<false><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(x, (bf16*)y, T, C, HW, Cp);
  return hipGetLastError();
}

// bf16 -> fp16, n elements (the Stream-VAE's weights, once at create)
__global__ void cast_h16_kernel(const bf16* __restrict__ x, f16* __restrict__ y, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = (f16)(float)x[i];
}

hipError_t cast_to_h16(hipStream_t s, const void* x, void* y, int64_t n) {
  if (n <= 0) return hipSuccess;
  cast_h16_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>((const bf16*)x, (f16*)y, n);
  return hipGetLastError();
}

}  // namespace sdk
