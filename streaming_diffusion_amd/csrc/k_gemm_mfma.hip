// bf16 GEMM on the matrix cores: C[m][n] = sum_k A[m][k] W[n][k], both
// operands K-contiguous, fp32 accumulation, fused DiT epilogues.
//
// Tiles of BM x BN (256x256, 256x128 or 128x128) per workgroup of 4 waves
// (2 x 2); each wave owns a (BM/2) x (BN/2) block of v_mfma_f32_32x32x16_bf16
// tiles.  BK = 64; A and W tiles are staged in LDS (rows padded by 16 bytes),
// two stages, with the next k-tile prefetched into registers while the
// current one is multiplied.
//
// Epilogue: the accumulators leave through LDS in strips of 64 rows, so every
// global store is a 16-byte vector: row-major outputs, the per-head Q/K
// layouts (8 consecutive head-dim elements of one token, RoPE applied to the
// pairs in registers) and the transposed V layout (8 consecutive tokens of one
// head-dim element).
#include <algorithm>
#include <cmath>

#include <type_traits>

#include "kernels.h"
#include "ln_row.h"

namespace sdk {

// Launch-bound-checked helpers shared with the epilogue.
// GELU(v) = v * Phi(v) = 0.5 v (1 + erf(v / sqrt 2)), with erf from the
// Abramowitz-Stegun rational approximation 7.1.26 (absolute error <= 1.5e-7,
// far below the bf16 rounding of the stored result) and no branches:
// erf(z) = 1 - e, e = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2),
// t = 1 / (1 + p z), z = |v| / sqrt 2; for v < 0, 1 + erf = e exactly.
SD_DEV float gelu_f(float v) {
  const float z = fabsf(v) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
  float poly = fmaf(t, 1.061405429f, -1.453152027f);
  poly = fmaf(t, poly, 1.421413741f);
  poly = fmaf(t, poly, -0.284496736f);
  poly = fmaf(t, poly, 0.254829592f);
  const float e = poly * t * __builtin_amdgcn_exp2f(-z * z * 1.4426950408889634f);
  return 0.5f * v * (v >= 0.f ? 2.0f - e : e);
}

// One 32x32x16 matrix-core product; with H16 the 16-bit operands are
// IEEE half precision (same layout and rate as bf16, 3 more mantissa bits).
template <bool H16>
SD_DEV f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (H16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                  0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

SD_DEV void load8_bf16(const bf16* p, float* o) {
  const bf16x8 v = *(const bf16x8*)p;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (float)v[i];
}

SD_DEV void store8_bf16(bf16* p, const float* v) {
  bf16x8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (bf16)v[i];
  *(bf16x8*)p = o;
}

// Row table of a 64-row strip: for the q/k/v scatters (row << 20 | token)
// and the token's offsets into the RoPE frame, row and column tables; for
// the gated residual the forward row of each token.
template <int MODE>
SD_DEV void epi_rows(const Epi& E, int4* rowtab, int m_base, int M, int tid, const int* t0s) {
  if constexpr (MODE == EPI_GATE_RESID) {
    if (tid < 64) rowtab[tid] = make_int4(min(m_base + tid, M - 1) / E.L, 0, 0, 0);
  }
  if constexpr (MODE == EPI_QKV || MODE == EPI_CTXKV) {
    if (tid < 64) {
      const int m = min(m_base + tid, M - 1);
      const int r = m / E.L, t = m - r * E.L;
      int4 v = make_int4((r << 20) | t, 0, 0, 0);
      if (E.rope) {
        const int hw = E.Hp * E.Wp;
        const int f = t / hw, y = (t / E.Wp) % E.Hp, x = t % E.Wp;
        v.y = (t0s[r] + f) * (E.dt >> 1);
        v.z = y * (E.dh >> 1);
        v.w = x * ((E.hd - E.dt - E.dh) >> 1);
      }
      rowtab[tid] = v;
    }
  }
}

template <int BN, int NT, int MODE>
SD_DEV void epi_strip(const Epi& E, const float* stg, int LC, int m_base, int n0, int M, int N, int tid,
                      const int4* rowtab) {
  constexpr int G = BN / 8;       // 8-column groups per row
  if constexpr (MODE == EPI_HEAD) {
    for (int idx = tid; idx < 64 * BN; idx += NT) {
      const int row = idx / BN, col = idx % BN;
      const int m = m_base + row, n = n0 + col;
      if (m >= M || n >= N) continue;
      const int r = m / E.L, t = m - r * E.L;
      const int hw = E.Hp * E.Wp;
      const int f = t / hw, y = (t / E.Wp) % E.Hp, x = t % E.Wp;
      const int c = n % E.C, px = (n / E.C) % E.p, py = n / (E.C * E.p);
      const int64_t lat = (int64_t)E.T * E.C * E.Hl * E.Wl;
      E.eps[r * lat + (((int64_t)f * E.C + c) * E.Hl + y * E.p + py) * E.Wl + x * E.p + px] =
          stg[row * LC + col] + (float)((const bf16*)E.bias)[n];
    }
    return;
  }
  if constexpr (MODE == EPI_QKV || MODE == EPI_CTXKV) {
    // Row facts come from the strip's row table, column facts are fixed per
    // thread (the thread -> column mapping repeats every NT groups).
    // q and k sections: groups of 8 head-dim elements of one token
    static_assert(NT % G == 0 && (64 * G) % NT == 0, "q/k thread mapping");
    {
      const int cg = tid % G, n = n0 + cg * 8;
      const int which = n / E.d;
      const int sec = (MODE == EPI_CTXKV) ? which + 1 : which;     // 0 q, 1 k, 2 v
      if (n < N && sec != 2) {
        const int nn = n - which * E.d, h = nn / E.hd, e0 = nn - h * E.hd;
        float b[8];
        load8_bf16((const bf16*)E.bias + n, b);
        // RoPE section (0 t, 1 h, 2 w) and in-section pair index of each pair
        int tp[4], jp[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int e = e0 + 2 * p;
          tp[p] = e < E.dt ? 0 : (e < E.dt + E.dh ? 1 : 2);
          jp[p] = (tp[p] == 0 ? e : (tp[p] == 1 ? e - E.dt : e - E.dt - E.dh)) >> 1;
        }
        bf16* const dst = sec == 0 ? (bf16*)E.q : (bf16*)E.k;
        constexpr int IT = 64 * G / NT;
        // phase 1: every (cos, sin) of the strip (table reads are not
        // ordered behind the stores of phase 2)
        float2 cs[IT][4];
        if (E.rope) {
#pragma unroll
          for (int it = 0; it < IT; ++it) {
            const int4 ri = rowtab[tid / G + it * (NT / G)];
#pragma unroll
            for (int p = 0; p < 4; ++p)
              cs[it][p] = tp[p] == 0 ? E.rope_t[ri.y + jp[p]]
                                     : (tp[p] == 1 ? E.rope_h[ri.z + jp[p]] : E.rope_w[ri.w + jp[p]]);
          }
        }
        // phase 2: rotate and store
#pragma unroll
        for (int it = 0; it < IT; ++it) {
          const int row = tid / G + it * (NT / G);
          if (m_base + row >= M) continue;
          const int rt = rowtab[row].x;
          const int r = rt >> 20, t = rt & 0xFFFFF;
          float v[8];
          const float4* sp = (const float4*)(stg + row * LC + cg * 8);
          const float4 v0 = sp[0], v1 = sp[1];
          v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w; v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] += b[i];
          if (E.rope) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const float x0 = v[2 * p], x1 = v[2 * p + 1];
              v[2 * p] = x0 * cs[it][p].x - x1 * cs[it][p].y;
              v[2 * p + 1] = x0 * cs[it][p].y + x1 * cs[it][p].x;
            }
          }
          const int64_t tok = sec == 0 ? ((int64_t)r * E.H + h) * E.L + t : ((int64_t)h * E.krows + r) * E.kstride + t;
          store8_bf16(dst + tok * E.hd + e0, v);
        }
      }
    }
    // v section: groups of 8 tokens of one head-dim element (transposed store)
    static_assert(NT % BN == 0 && (8 * BN) % NT == 0, "v thread mapping");
    {
      const int col = tid % BN, n = n0 + col;
      const int which = n / E.d;
      const int sec = (MODE == EPI_CTXKV) ? which + 1 : which;
      if (n < N && sec == 2) {
        const int nn = n - which * E.d, h = nn / E.hd, e = nn - h * E.hd;
        const float bn = (float)((const bf16*)E.bias)[n];
#pragma unroll
        for (int it = 0; it < 8 * BN / NT; ++it) {
          const int rg = tid / BN + it * (NT / BN);
          const int m = m_base + rg * 8;
          if (m >= M) continue;
          const int4 ri = rowtab[rg * 8];
          const int r = ri.x >> 20, t = ri.x & 0xFFFFF;
          if (m + 8 <= M && t + 8 <= E.L) {
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = stg[(rg * 8 + i) * LC + col] + bn;
            store8_bf16((bf16*)E.vt + (((int64_t)h * E.hd + e) * E.krows + r) * E.kstride + t, v);
          } else {
            for (int i = 0; i < 8 && m + i < M; ++i) {
              const int rx = rowtab[rg * 8 + i].x;
              bf16* di = (bf16*)E.vt + (((int64_t)h * E.hd + e) * E.krows + (rx >> 20)) * E.kstride + (rx & 0xFFFFF);
              *di = (bf16)(stg[(rg * 8 + i) * LC + col] + bn);
            }
          }
        }
      }
    }
    return;
  }
  // row-major modes: groups of 8 consecutive columns of one row.  A thread's
  // columns are fixed (bias and block gate load once); all global loads of
  // the strip are issued before any store, since a store to the residual
  // would otherwise order the next group's load behind it.
  static_assert(NT % G == 0 && (64 * G) % NT == 0, "row-major thread mapping");
  constexpr int IT = 64 * G / NT;
  const int cg = tid % G, n = n0 + cg * 8;
  if (n >= N) return;
  if (n + 8 > N || (E.ldo & 7) || (N & 7)) {
    // ragged right edge or unaligned rows: element by element
    for (int it = 0; it < IT; ++it) {
      const int row = tid / G + it * (NT / G), m = m_base + row;
      if (m >= M) continue;
      for (int i = 0; i < 8 && n + i < N; ++i) {
        float v = stg[row * LC + cg * 8 + i] + (E.bias ? (float)((const bf16*)E.bias)[n + i] : 0.f);
        if constexpr (MODE == EPI_STORE) {
          ((bf16*)E.out)[(int64_t)m * E.ldo + n + i] = (bf16)v;
        } else if constexpr (MODE == EPI_GELU) {
          ((bf16*)E.out)[(int64_t)m * E.ldo + n + i] = (bf16)gelu_f(v);
        } else if constexpr (MODE == EPI_F32) {
          ((float*)E.out)[(int64_t)m * E.ldo + n + i] = v;
        } else if constexpr (MODE == EPI_PATCH) {
          E.resid[(int64_t)m * N + n + i] = v;
        } else if constexpr (MODE == EPI_RESID || MODE == EPI_GATE_RESID) {
          if constexpr (MODE == EPI_GATE_RESID)
            v *= E.mod[(int64_t)(m / E.L) * E.six_d + E.gate_off + n + i] +
                 (float)((const bf16*)E.blk)[E.gate_off + n + i];
          E.resid[(int64_t)m * N + n + i] += v;
        }
      }
    }
    return;
  }
  float b[8];
  if (E.bias) {
    load8_bf16((const bf16*)E.bias + n, b);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = 0.f;
  }
  constexpr bool RES = MODE == EPI_RESID || MODE == EPI_GATE_RESID;
  float gb[8];
  if constexpr (MODE == EPI_GATE_RESID) load8_bf16((const bf16*)E.blk + E.gate_off + n, gb);
  float4 rin[IT][2], gin[IT][2];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int row = tid / G + it * (NT / G), m = m_base + row;
    if (m >= M) continue;
    if constexpr (RES) {
      const float4* o = (const float4*)(E.resid + (int64_t)m * N + n);
      rin[it][0] = o[0];
      rin[it][1] = o[1];
    }
    if constexpr (MODE == EPI_GATE_RESID) {
      const float4* gm = (const float4*)(E.mod + (int64_t)rowtab[row].x * E.six_d + E.gate_off + n);
      gin[it][0] = gm[0];
      gin[it][1] = gm[1];
    }
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int row = tid / G + it * (NT / G), m = m_base + row;
    if (m >= M) continue;
    float v[8];
    const float4* sp = (const float4*)(stg + row * LC + cg * 8);
    const float4 v0 = sp[0], v1 = sp[1];
    v[0] = v0.x + b[0]; v[1] = v0.y + b[1]; v[2] = v0.z + b[2]; v[3] = v0.w + b[3];
    v[4] = v1.x + b[4]; v[5] = v1.y + b[5]; v[6] = v1.z + b[6]; v[7] = v1.w + b[7];
    if constexpr (MODE == EPI_STORE) {
      store8_bf16((bf16*)E.out + (int64_t)m * E.ldo + n, v);
    } else if constexpr (MODE == EPI_GELU) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = gelu_f(v[i]);
      store8_bf16((bf16*)E.out + (int64_t)m * E.ldo + n, v);
    } else if constexpr (MODE == EPI_F32) {
      float4* o = (float4*)((float*)E.out + (int64_t)m * E.ldo + n);
      o[0] = make_float4(v[0], v[1], v[2], v[3]);
      o[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else if constexpr (MODE == EPI_PATCH) {
      float4* o = (float4*)(E.resid + (int64_t)m * N + n);
      o[0] = make_float4(v[0], v[1], v[2], v[3]);
      o[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else if constexpr (RES) {
      if constexpr (MODE == EPI_GATE_RESID) {
        const float4 g0 = gin[it][0], g1 = gin[it][1];
        v[0] *= g0.x + gb[0]; v[1] *= g0.y + gb[1]; v[2] *= g0.z + gb[2]; v[3] *= g0.w + gb[3];
        v[4] *= g1.x + gb[4]; v[5] *= g1.y + gb[5]; v[6] *= g1.z + gb[6]; v[7] *= g1.w + gb[7];
      }
      float4 r0 = rin[it][0], r1 = rin[it][1];
      r0.x += v[0]; r0.y += v[1]; r0.z += v[2]; r0.w += v[3];
      r1.x += v[4]; r1.y += v[5]; r1.z += v[6]; r1.w += v[7];
      float4* o = (float4*)(E.resid + (int64_t)m * N + n);
      o[0] = r0;
      o[1] = r1;
    }
  }
}

template <int BM, int BN, int NW, int MODE, bool H16 = false>
__global__ __launch_bounds__(64 * NW) void gemm_mfma_kernel(const bf16* __restrict__ A, const bf16* __restrict__ W,
                                                        int M, int N, int K, Epi E) {
  constexpr int BK = 64, PAD = 8, LDK = BK + PAD;
  constexpr int NT = 64 * NW, WN = NW / 2;          // waves arranged 2 x WN
  constexpr int TM = BM / 2, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  constexpr int CA = BM * (BK / 8) / NT, CB = BN * (BK / 8) / NT;
  constexpr int STAGE = (BM + BN) * LDK;                 // bf16 elements per LDS stage
  constexpr int LC = BN + 4;                             // fp32 pitch of the epilogue strip
  static_assert(64 * LC * 4 <= 2 * STAGE * 2, "epilogue strip must fit in the stage buffers");
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * STAGE];
  __shared__ int t0s[SD_MAX_ROWS];     // per-row temporal RoPE base (read with a dynamic row index)
  __shared__ int4 rowtab[64];          // per-strip row facts of the q/k/v scatters

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  // XCD-contiguous logical ids; groups of GM tile-rows walked column by column
  constexpr int GM = 4;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = lid / (GM * tiles_n), first_m = grp * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int within = lid - grp * GM * tiles_n;
  const int tm = first_m + within % gm, tn = within / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // Global -> register staging.  Rows beyond M (N) are clamped to the last
  // row: they only feed output rows/columns that are never stored, so full
  // k-tiles load without branches; only a ragged last k-tile checks K.
  uint32_t a_off[CA], b_off[CB];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int c = tid + i * NT, row = c >> 3, kc = (c & 7) * 8;
    a_off[i] = (uint32_t)min(m0 + row, M - 1) * (uint32_t)K + kc;
  }
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int c = tid + i * NT, row = c >> 3, kc = (c & 7) * 8;
    b_off[i] = (uint32_t)min(n0 + row, N - 1) * (uint32_t)K + kc;
  }
  const int KT = (K + BK - 1) / BK;
  const bool ragged = (K % BK) != 0;
  const bf16x8 zero8 = {};
  auto gload = [&](bf16x8* ra, bf16x8* rb, int kt) {
    const uint32_t k0 = (uint32_t)kt * BK;
    if (!ragged || kt + 1 < KT) {
#pragma unroll
      for (int i = 0; i < CA; ++i) ra[i] = *(const bf16x8*)(A + a_off[i] + k0);
#pragma unroll
      for (int i = 0; i < CB; ++i) rb[i] = *(const bf16x8*)(W + b_off[i] + k0);
    } else {
#pragma unroll
      for (int i = 0; i < CA; ++i) {
        const int kc = ((tid + i * NT) & 7) * 8;
        ra[i] = ((int)k0 + kc < K) ? *(const bf16x8*)(A + a_off[i] + k0) : zero8;
      }
#pragma unroll
      for (int i = 0; i < CB; ++i) {
        const int kc = ((tid + i * NT) & 7) * 8;
        rb[i] = ((int)k0 + kc < K) ? *(const bf16x8*)(W + b_off[i] + k0) : zero8;
      }
    }
  };
  auto sstore = [&](const bf16x8* ra, const bf16x8* rb, int buf) {
    bf16* as = smem + buf * STAGE;
    bf16* bs = as + BM * LDK;
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = tid + i * NT, row = c >> 3, kc = (c & 7) * 8;
      *(bf16x8*)(as + row * LDK + kc) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = tid + i * NT, row = c >> 3, kc = (c & 7) * 8;
      *(bf16x8*)(bs + row * LDK + kc) = rb[i];
    }
  };
  const int lr = lane & 31, lk = (lane >> 5) * 8;
  // The fragments of k-step kk+1 are read from LDS before the MFMAs of step
  // kk are issued, so LDS latency hides behind matrix-core work; the
  // scheduling barriers keep the compiler from regrouping the reads.
  auto compute = [&](int buf) {
    const bf16* as = smem + buf * STAGE + (wm * TM + lr) * LDK + lk;
    const bf16* bs = smem + buf * STAGE + BM * LDK + (wn * TN + lr) * LDK + lk;
    bf16x8 fa[2][FM], fb[2][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[0][i] = *(const bf16x8*)(as + i * 32 * LDK);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[0][j] = *(const bf16x8*)(bs + j * 32 * LDK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int cur = ks & 1, nxt = cur ^ 1;
      if (ks + 1 < BK / 16) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[nxt][i] = *(const bf16x8*)(as + i * 32 * LDK + (ks + 1) * 16);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[nxt][j] = *(const bf16x8*)(bs + j * 32 * LDK + (ks + 1) * 16);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = mfma32<H16>(fa[cur][i], fb[cur][j], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if constexpr (MODE == EPI_QKV) {
    if (tid == 0) {
#pragma unroll
      for (int i = 0; i < SD_MAX_ROWS; ++i) t0s[i] = E.t0_dev ? E.t0_dev[i] : E.t0[i];
    }
  }
  // One register stage, two LDS stages: the loads of k-tile t+1 are issued
  // before tile t is multiplied and stored to the free LDS stage after it.
  bf16x8 ra[CA], rb[CB];
  gload(ra, rb, 0);
  sstore(ra, rb, 0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(ra, rb, kt + 1);
    compute(buf);
    if (kt + 1 < KT) sstore(ra, rb, buf ^ 1);
    __syncthreads();
  }

  // epilogue through LDS, 64 rows at a time.  C layout of a 32x32 tile: lane
  // holds column lane%32, rows 8*(q/4) + 4*(lane/32) + q%4.
  float* stg = (float*)smem;
  constexpr int SPW = TM / 64;          // strips per wave-row
#pragma unroll
  for (int s = 0; s < BM / 64; ++s) {
    if (wm == s / SPW) {
      const int i0 = (s % SPW) * 2;
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int row = ii * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
            const int col = wn * TN + j * 32 + (lane & 31);
            stg[row * LC + col] = acc[i0 + ii][j][q];
          }
    }
    epi_rows<MODE>(E, rowtab, m0 + s * 64, M, tid, t0s);
    __syncthreads();
    epi_strip<BN, NT, MODE>(E, stg, LC, m0 + s * 64, n0, M, N, tid, rowtab);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Direct-to-LDS variant (K a multiple of BK).  Operand tiles move from global
// memory into LDS with global_load_lds_dwordx4: one wave instruction fills
// 1 KB of a stage (1024 / (2 BK) rows of BK bf16), lane l landing at byte
// 16*l.  No registers are involved, so the wave's instruction stream carries
// only the DMA issue, the LDS fragment reads and the MFMAs.  Rows are stored
// unpadded with an XOR swizzle of their 16-byte chunks: chunk c of row r sits
// at position c ^ ((r / RP) % CPR), CPR = BK / 8 chunks per row, RP = 128 / BK
// rows per 256 bytes, which keeps the 16-lane passes of the MFMA fragment
// reads on distinct banks.  NS stages: the DMA of k-tile t + NS - 1 is issued
// right after the barrier that retires tile t - 1, and the wait before tile t
// leaves the later tiles' DMA in flight.
template <int BK>
SD_DEV int swz(int row) {
  return (row / (128 / BK)) & (BK / 8 - 1);
}

// wait until at most n of this wave's vector-memory operations are in flight,
// then meet the workgroup at a barrier (no fence: the DMA writes are ordered
// by the wait, the LDS reads of the previous tile were consumed by its MFMAs)
template <int n>
SD_DEV void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(n) : "memory");
}

//
// TM0 < BM / 2 splits the tile rows unevenly between the two wave rows (TM0
// and BM - TM0 rows, both multiples of 32): a 160-row tile as 96 + 64.  Wave
// w then takes wave row w / WN, so each SIMD (waves w and w + 4) holds one
// wave of each row and gets the same number of products per k-step as the
// others; the A rows of a k-tile need not divide evenly over the waves
// (DMA block b goes to wave b % NW).
template <int BM, int BN, int NW, int BK, int NS, bool SPREAD, int MODE, bool H16 = false, int TM0 = BM / 2,
          int GM = 8>
__global__ __launch_bounds__(64 * NW) void gemm_dma_kernel(const bf16* __restrict__ A, const bf16* __restrict__ W,
                                                          int M, int N, int K, Epi E) {
  constexpr bool EVEN = TM0 * 2 == BM;
  constexpr int NT = 64 * NW, WN = NW / 2;
  constexpr int TN = BN / WN, FM = TM0 / 32, FM1 = (BM - TM0) / 32, FN = TN / 32;
  constexpr int CPR = BK / 8, RPB = 64 / CPR;             // chunks per row, rows per DMA block
  constexpr int ABLK = BM / RPB;                          // A DMA blocks per k-tile
  constexpr int AQ = (ABLK + NW - 1) / NW, BQ = BN / RPB / NW;   // DMA blocks per wave per k-tile (A: at most)
  constexpr int DQ = AQ + BQ;
  constexpr int STAGE = (BM + BN) * BK;                   // bf16 elements per stage
  constexpr int LC = BN + 4;
  static_assert(TM0 % 32 == 0 && TM0 * 2 >= BM && FM1 >= 1, "wave rows");
  static_assert(BQ >= 1 && ABLK * RPB == BM && BQ * RPB * NW == BN, "tile shape");
  // uneven tiles: the first AX waves issue one A block more per k-tile
  constexpr int AX = ABLK % NW, DQ_LO = ABLK / NW + BQ;
  static_assert(NS >= 2 && NS <= 5 && DQ * (NS - 2) < 64, "stages");
  static_assert(64 * LC * 4 <= NS * STAGE * 2, "epilogue strip must fit in the stage buffers");
  // one LDS block with the stage buffers at offset 0 (the row table and the
  // per-row RoPE bases follow them): left to the compiler, the placement of
  // the small arrays could move the stage buffers off offset 0, which costs
  // up to half the throughput of the gated-residual kernels.  (160 x 256
  // tiles with three stages: 156 KB of stages + 1.2 KB of tables.)
  constexpr int SMEM_BYTES = NS * STAGE * 2;
  static_assert(SMEM_BYTES + 64 * 16 + SD_MAX_ROWS * 4 <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[SMEM_BYTES + 64 * 16 + SD_MAX_ROWS * 4];
  bf16* const smem = (bf16*)lds;
  int4* const rowtab = (int4*)(lds + SMEM_BYTES);
  int* const t0s = (int*)(lds + SMEM_BYTES + 64 * 16);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = EVEN ? (wave & 1) : wave / WN, wn = EVEN ? (wave >> 1) : wave % WN;
  const int row0 = wm * TM0;                               // first tile row of this wave row
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  // XCD-contiguous logical ids walked in groups of GM tile-rows, column by
  // column, so the A rows and W columns of neighbouring tiles meet in one
  // L2 (8 rows measured 1-2 % faster than 4 on the video step's QKV, FFN2
  // and cross GEMMs, 1.5 % slower on FFN1)
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = lid / (GM * tiles_n), first_m = grp * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int within = lid - grp * GM * tiles_n;
  const int tm = first_m + within % gm, tn = within / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // per-lane source offsets (elements) of this wave's DMA blocks, k-tile 0;
  // rows beyond M / N are clamped (they feed outputs that are never stored)
  auto ablk = [&](int q) { return EVEN ? wave * AQ + q : q * NW + wave; };
  uint32_t a_src[AQ], b_src[BQ];
  const int lrow = lane / CPR, lpos = lane % CPR;
#pragma unroll
  for (int q = 0; q < AQ; ++q) {
    const int r = min(ablk(q), ABLK - 1) * RPB + lrow;
    a_src[q] = (uint32_t)min(m0 + r, M - 1) * (uint32_t)K + (uint32_t)((lpos ^ swz<BK>(r)) * 8);
  }
#pragma unroll
  for (int q = 0; q < BQ; ++q) {
    const int r = (wave * BQ + q) * RPB + lrow;
    b_src[q] = (uint32_t)min(n0 + r, N - 1) * (uint32_t)K + (uint32_t)((lpos ^ swz<BK>(r)) * 8);
  }
  // DMA of k-tile kt into stage buf; part < 0 issues every block of this
  // wave, part p in [0, BK/16) only the blocks j with j * (BK/16) / DQ == p
  auto issue = [&](int kt, int buf, int part) {
    const uint32_t k0 = (uint32_t)kt * BK;
    bf16* as = smem + buf * STAGE;
    bf16* bs = as + BM * BK;
#pragma unroll
    for (int q = 0; q < AQ; ++q)
      if ((EVEN || ablk(q) < ABLK) && (part < 0 || q * (BK / 16) / DQ == part))
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(A + a_src[q] + k0),
                                         (__attribute__((address_space(3))) void*)(as + ablk(q) * RPB * BK),
                                         16, 0, 0);
#pragma unroll
    for (int q = 0; q < BQ; ++q)
      if (part < 0 || (AQ + q) * (BK / 16) / DQ == part)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(W + b_src[q] + k0),
                                         (__attribute__((address_space(3))) void*)(bs + (wave * BQ + q) * RPB * BK),
                                         16, 0, 0);
  };
  // fragment rows of this lane and their swizzle
  const int lr = lane & 31, lh = lane >> 5;
  // MFMAs over stage buf for a wave row of FR fragment rows; with SPREAD and
  // WI the DMA of k-tile nkt into stage nbuf is issued a part per 16-wide k
  // step
  auto compute_rows = [&](int buf, int nkt, int nbuf, auto wi, auto fr) {
    constexpr int FR = decltype(fr)::value;
    const bf16* as = smem + buf * STAGE;
    const bf16* bs = as + BM * BK;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if constexpr (SPREAD && decltype(wi)::value) issue(nkt, nbuf, ks);
      const int c = ks * 2 + lh;           // logical 16-byte chunk of this lane
      bf16x8 fa[FR], fb[FN];
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        const int row = row0 + i * 32 + lr;
        fa[i] = *(const bf16x8*)(as + row * BK + ((c ^ swz<BK>(row)) * 8));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = wn * TN + j * 32 + lr;
        fb[j] = *(const bf16x8*)(bs + row * BK + ((c ^ swz<BK>(row)) * 8));
      }
#pragma unroll
      for (int i = 0; i < FR; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = mfma32<H16>(fa[i], fb[j], acc[i][j]);
    }
  };
  auto compute = [&](int buf, int nkt, int nbuf, auto wi) {
    if constexpr (EVEN) {
      compute_rows(buf, nkt, nbuf, wi, std::integral_constant<int, FM>{});
    } else {
      if (wm == 0) compute_rows(buf, nkt, nbuf, wi, std::integral_constant<int, FM>{});
      else compute_rows(buf, nkt, nbuf, wi, std::integral_constant<int, FM1>{});
    }
  };

  if constexpr (MODE == EPI_QKV) {
    if (tid == 0) {
#pragma unroll
      for (int i = 0; i < SD_MAX_ROWS; ++i) t0s[i] = E.t0_dev ? E.t0_dev[i] : E.t0[i];
    }
  }
  const int KT = K / BK;
#pragma unroll
  for (int t = 0; t < NS - 1; ++t)
    if (t < KT) issue(t, t, -1);
  // one k-tile: tiles kt+1 .. kt+NS-2 may stay in flight; tile kt must have
  // landed in every wave, and every wave must be done reading tile kt-1.  WI:
  // k-tile kt+NS-1 exists and its DMA goes out during this tile's MFMAs.
  auto wait_tiles = [](int ahead, auto dq) {
    constexpr int D = decltype(dq)::value;
    if constexpr (NS >= 5) {
      if (ahead >= 3) return wait_vm_barrier<D * 3>();
    }
    if constexpr (NS >= 4) {
      if (ahead >= 2) return wait_vm_barrier<D * 2>();
    }
    if constexpr (NS >= 3) {
      if (ahead >= 1) return wait_vm_barrier<D>();
    }
    wait_vm_barrier<0>();
  };
  auto step = [&](int kt, auto wi) {
    // leave this wave's blocks of the next `ahead` k-tiles in flight
    const int ahead = min(NS - 2, KT - 1 - kt);
    // (a scalar branch: the two arms hold barriers, which must not both run
    // under a partial exec mask)
    if (EVEN || __builtin_amdgcn_readfirstlane(wave) < AX) wait_tiles(ahead, std::integral_constant<int, DQ>{});
    else wait_tiles(ahead, std::integral_constant<int, DQ_LO>{});
    const int nkt = kt + NS - 1;
    if constexpr (!SPREAD && decltype(wi)::value) issue(nkt, nkt % NS, -1);
    compute(kt % NS, nkt, nkt % NS, wi);
  };
  int kt = 0;
  for (; kt + NS - 1 < KT; ++kt) step(kt, std::true_type{});
  for (; kt < KT; ++kt) step(kt, std::false_type{});
  __syncthreads();

  // epilogue in 64-row strips staged through LDS; a strip gathers the
  // 32-row fragment rows of whichever waves hold them (a wave row may hold
  // 96 or 64 rows); the last strip of a 160-row tile is half full, and rows
  // past the tile (mt) are not stored
  float* stg = (float*)smem;
  const int mt = min(M, m0 + BM);
  const int fm = (EVEN || wm == 0) ? FM : FM1;
#pragma unroll
  for (int s = 0; s < (BM + 63) / 64; ++s) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int rb = row0 + i * 32;
      if (i < fm && rb / 64 == s) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int row = rb % 64 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
            const int col = wn * TN + j * 32 + (lane & 31);
            stg[row * LC + col] = acc[i][j][q];
          }
      }
    }
    epi_rows<MODE>(E, rowtab, m0 + s * 64, mt, tid, t0s);
    __syncthreads();
    epi_strip<BN, NT, MODE>(E, stg, LC, m0 + s * 64, n0, mt, N, tid, rowtab);
    __syncthreads();
  }
}

// Second pass of the weight-streaming product.  Its partials are stored in
// accumulator order, float4 granules [slice][tile][feature block][row block]
// [g][lane] (tile = 128 features x 128 rows, blocks of 32; lane l of
// feature block i, row block j holds row 32 j + l % 32, features
// 32 i + 8 g + 4 (l / 32) + 0..3), so both passes move whole 1 KB wave rows.
// One workgroup takes one tile, one 64-row strip and one feature block: it
// sums the K slices in slice order (fixed, so results do not depend on
// scheduling) and runs the epilogue of MODE on the 64 x 32 strip -- the
// row-major modes straight from the sums, the scatters through LDS.
template <int MODE>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(int M, int N, Epi E) {
  constexpr int BN = 32, NT = 256, LC = BN + 4;
  __shared__ __attribute__((aligned(16))) float stg[64 * LC];
  __shared__ int4 rowtab[64];
  __shared__ int t0s[SD_MAX_ROWS];
  const int tid = threadIdx.x;
  const int tiles_n = (N + 127) / 128, tiles = tiles_n * ((M + 127) / 128);
  const int tile = blockIdx.x / 8, sp = (blockIdx.x / 4) % 2, i = blockIdx.x % 4;
  const int m_base = (tile / tiles_n) * 128 + sp * 64, n0 = (tile % tiles_n) * 128 + i * 32;
  if (m_base >= M || n0 >= N) return;                     // uniform over the workgroup
  if constexpr (MODE == EPI_QKV) {
    if (tid < SD_MAX_ROWS) t0s[tid] = E.t0_dev ? E.t0_dev[tid] : E.t0[tid];
  }
  const int g = tid / 64, ln = tid % 64;
  // Row-major epilogues run straight from the sums: this thread's outputs are
  // features n0 + 8 g + 4 (ln / 32) + 0..3 of rows m_base + 32 h + ln % 32,
  // and every epilogue operand (bias, gates, residual) is requested before
  // the partial sums, so the pass takes one memory round trip
  constexpr bool DIRECT = MODE == EPI_F32 || MODE == EPI_RESID || MODE == EPI_GATE_RESID ||
                          MODE == EPI_STORE || MODE == EPI_GELU;
  const int nf = n0 + 8 * g + 4 * (ln / 32);
  const int mr[2] = {m_base + ln % 32, m_base + 32 + ln % 32};
  float bq[4] = {0.f, 0.f, 0.f, 0.f}, gq[4] = {0.f, 0.f, 0.f, 0.f};
  float4 rin[2], gin[2];
  if constexpr (DIRECT) {
    if (nf < N) {
      if (E.bias) {
        const bf16x4 bv = *(const bf16x4*)((const bf16*)E.bias + nf);
#pragma unroll
        for (int e = 0; e < 4; ++e) bq[e] = (float)bv[e];
      }
      if constexpr (MODE == EPI_GATE_RESID) {
        const bf16x4 gv = *(const bf16x4*)((const bf16*)E.blk + E.gate_off + nf);
#pragma unroll
        for (int e = 0; e < 4; ++e) gq[e] = (float)gv[e];
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (mr[h] >= M) continue;
        if constexpr (MODE == EPI_RESID || MODE == EPI_GATE_RESID)
          rin[h] = *(const float4*)(E.resid + (int64_t)mr[h] * N + nf);
        if constexpr (MODE == EPI_GATE_RESID)
          gin[h] = *(const float4*)(E.mod + (int64_t)(mr[h] / E.L) * E.six_d + E.gate_off + nf);
      }
    }
  }
  const int64_t slice_st = (int64_t)tiles * 4 * 16 * 64;  // float4 granules per slice
  // both granules of the thread, eight slices at a time: 16 loads in flight
  // per thread (the pass is latency-bound), each sum still in slice order
  const float4* src0 = (const float4*)E.part + (((int64_t)tile * 4 + i) * 16 + (2 * sp) * 4 + g) * 64 + ln;
  const float4* src1 = src0 + 4 * 64;
  float4 acc[2] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
  int sl = 0;
  for (; sl + 8 <= E.ksplit; sl += 8) {
    float4 v[2][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      v[0][u] = src0[(sl + u) * slice_st];
      v[1][u] = src1[(sl + u) * slice_st];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        acc[h].x += v[h][u].x;
        acc[h].y += v[h][u].y;
        acc[h].z += v[h][u].z;
        acc[h].w += v[h][u].w;
      }
  }
  if (sl + 4 <= E.ksplit) {
    float4 v[2][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v[0][u] = src0[(sl + u) * slice_st];
      v[1][u] = src1[(sl + u) * slice_st];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        acc[h].x += v[h][u].x;
        acc[h].y += v[h][u].y;
        acc[h].z += v[h][u].z;
        acc[h].w += v[h][u].w;
      }
    sl += 4;
  }
  for (; sl < E.ksplit; ++sl) {
    const float4 v0 = src0[sl * slice_st], v1 = src1[sl * slice_st];
    acc[0].x += v0.x;
    acc[0].y += v0.y;
    acc[0].z += v0.z;
    acc[0].w += v0.w;
    acc[1].x += v1.x;
    acc[1].y += v1.y;
    acc[1].z += v1.z;
    acc[1].w += v1.w;
  }
  if constexpr (DIRECT) {
    if (nf >= N) return;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (mr[h] >= M) continue;
      float v[4] = {acc[h].x + bq[0], acc[h].y + bq[1], acc[h].z + bq[2], acc[h].w + bq[3]};
      if constexpr (MODE == EPI_F32) {
        float* const o = (float*)E.out + (int64_t)mr[h] * E.ldo + nf;
        if (E.ldo & 3) {          // rows not 16-byte aligned: element by element
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = v[e];
        } else {
          *(float4*)o = make_float4(v[0], v[1], v[2], v[3]);
        }
      } else if constexpr (MODE == EPI_STORE || MODE == EPI_GELU) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (bf16)(MODE == EPI_GELU ? gelu_f(v[e]) : v[e]);
        bf16* const o = (bf16*)E.out + (int64_t)mr[h] * E.ldo + nf;
        if (E.ldo & 3) {
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = ov[e];
        } else {
          *(bf16x4*)o = ov;
        }
      } else {
        if constexpr (MODE == EPI_GATE_RESID) {
          v[0] *= gin[h].x + gq[0];
          v[1] *= gin[h].y + gq[1];
          v[2] *= gin[h].z + gq[2];
          v[3] *= gin[h].w + gq[3];
        }
        float4 r = rin[h];
        r.x += v[0];
        r.y += v[1];
        r.z += v[2];
        r.w += v[3];
        *(float4*)(E.resid + (int64_t)mr[h] * N + nf) = r;
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) *(float4*)(stg + (h * 32 + ln % 32) * LC + 8 * g + 4 * (ln / 32)) = acc[h];
    __syncthreads();
    epi_rows<MODE>(E, rowtab, m_base, M, tid, t0s);
    __syncthreads();
    epi_strip<BN, NT, MODE>(E, stg, LC, m_base, n0, M, N, tid, rowtab);
  }
}

// The reduction pass of a residual GEMM fused with the LayerNorm that reads
// the residual next: one workgroup per row, thread j owns features
// 4 j .. 4 j + 3, read from row-major partials (the streaming kernel stores
// them so with part_rows; in the fragment order a row is 16 bytes of every
// 128-byte line, eight times the traffic).  It
// sums the K slices in slice order and applies the epilogue exactly as
// gemm_reduce_kernel does (the same residual values), stores the row, then
// normalises and modulates it as the LayerNorm row kernel does (ln_row), so
// the output is the one the separate passes would give.  Saves a launch and
// the residual's read-back per block below the knee.  N a multiple of 256,
// at most 2048 (blockDim = N / 4, at most 8 waves).
template <int MODE, typename T, bool SPLIT>
__global__ __launch_bounds__(512) void gemm_reduce_ln_kernel(int M, int N, Epi E) {
  __shared__ float red[2][8];
  const int m = blockIdx.x, j = threadIdx.x, lane = j & 63, wave = j >> 6, nw = blockDim.x >> 6;
  const int n = 4 * j;
  // row-major partials (part_rows): slice sl of this float4 at sl M N + m N + n
  const float4* src = (const float4*)(E.part + (int64_t)m * N + n);
  const int64_t slice_st = (int64_t)M * N / 4;
  // epilogue and LayerNorm operands, requested before the partial sums
  float bq[4] = {0.f, 0.f, 0.f, 0.f}, gq[4] = {0.f, 0.f, 0.f, 0.f};
  if (E.bias) {
    const bf16x4 bv = *(const bf16x4*)((const bf16*)E.bias + n);
#pragma unroll
    for (int e = 0; e < 4; ++e) bq[e] = (float)bv[e];
  }
  float4 gin = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (MODE == EPI_GATE_RESID) {
    const bf16x4 gv = *(const bf16x4*)((const bf16*)E.blk + E.gate_off + n);
#pragma unroll
    for (int e = 0; e < 4; ++e) gq[e] = (float)gv[e];
    gin = *(const float4*)(E.mod + (int64_t)(m / E.L) * E.six_d + E.gate_off + n);
  }
  const float4 rin = *(const float4*)(E.resid + (int64_t)m * N + n);
  const float* mr = E.ln_mod ? E.ln_mod + (int64_t)(m / E.L) * E.ln_six : nullptr;
  float sh[4] = {0.f, 0.f, 0.f, 0.f}, sc[4] = {0.f, 0.f, 0.f, 0.f};
  if (mr) ln_row_mod(mr, (const T*)E.ln_blk, E.ln_shift, E.ln_scale, j, sh, sc);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  int sl = 0;
  for (; sl + 8 <= E.ksplit; sl += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[(sl + u) * slice_st];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      acc.x += v[u].x;
      acc.y += v[u].y;
      acc.z += v[u].z;
      acc.w += v[u].w;
    }
  }
  for (; sl < E.ksplit; ++sl) {
    const float4 v = src[sl * slice_st];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  float v[4] = {acc.x + bq[0], acc.y + bq[1], acc.z + bq[2], acc.w + bq[3]};
  if constexpr (MODE == EPI_GATE_RESID) {
    v[0] *= gin.x + gq[0];
    v[1] *= gin.y + gq[1];
    v[2] *= gin.z + gq[2];
    v[3] *= gin.w + gq[3];
  }
  float4 r = rin;
  r.x += v[0];
  r.y += v[1];
  r.z += v[2];
  r.w += v[3];
  *(float4*)(E.resid + (int64_t)m * N + n) = r;
  float o[4];
  ln_row(r, N, E.ln_eps, mr != nullptr, sh, sc, red, nw, lane, wave, o);
  ln_row_store<T, SPLIT>((T*)E.ln_out + (int64_t)m * (SPLIT ? 2 * N : N), N, j, o);
}

// The reduction pass of the folded cross-attention's score product fused
// with its grouped softmax: 16 lanes per (row, group of sm_cp columns), each
// lane summing the K slices (row-major partials, slice order, as the other
// reduction) of columns l, l + 16, ... and then the softmax of the folded
// attention (max, exponentials, sum, scale) on them, written in fp16; the
// scores themselves are not stored.
__global__ __launch_bounds__(256) void gemm_reduce_softmax_kernel(int M, int N, Epi E) {
  const int64_t g = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int l = threadIdx.x & 15;
  if (g >= (int64_t)M * E.sm_heads) return;        // whole 16-lane groups leave together
  const int64_t m = g / E.sm_heads;
  const int h = (int)(g - m * E.sm_heads), Cp = E.sm_cp;
  const float* const src = E.part + m * N + (int64_t)h * Cp;
  const int64_t slice_st = (int64_t)M * N;
  // four slices' loads in flight at a time, each sum in slice order
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int sl = 0;
  for (; sl + 4 <= E.ksplit; sl += 4) {
    float t[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) t[u][i] = l + 16 * i < Cp ? src[(sl + u) * slice_st + l + 16 * i] : 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] += t[u][i];
  }
  for (; sl < E.ksplit; ++sl) {
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = l + 16 * i < Cp ? src[sl * slice_st + l + 16 * i] : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] += t[i];
  }
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = l + 16 * i;
    v[i] = j < Cp ? v[i] + E.sm_bias[h * Cp + j] : -INFINITY;
    mx = fmaxf(mx, v[i]);
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 16));
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = l + 16 * i < Cp ? __expf(v[i] - mx) : 0.f;
    sum += v[i];
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 16);
  const float inv = 1.0f / sum;
  f16* const out = E.sm_out + m * N + (int64_t)h * Cp;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = l + 16 * i;
    if (j < Cp) out[j] = (f16)(v[i] * inv);
  }
}

// compute units of the current device (queried once; 256 on MI355X)
static int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

template <int BM, int BN, int NW, int BK, int NS, bool SPREAD, int MODE, bool H16 = false, int TM0 = BM / 2,
          int GM = 8>
hipError_t launch_dma(hipStream_t s, const bf16* A, const bf16* W, int M, int N, int K, const Epi& E) {
  const unsigned grid = (unsigned)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
  gemm_dma_kernel<BM, BN, NW, BK, NS, SPREAD, MODE, H16, TM0, GM><<<grid, 64 * NW, 0, s>>>(A, W, M, N, K, E);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Weight-streaming product for few rows (tiles of up to 128 rows), the regime
// below the knee where reading W from HBM bounds the GEMM.  C^T = W A^T per
// workgroup tile of 128 output features x 128 rows over one K slice of KT
// k-tiles of 64.  Wave w owns features 32 w .. 32 w + 31 of the tile and all
// 128 rows.  At kernel start every lane issues its share of the A slice (rows
// shared by the four waves, staged through registers into swizzled LDS rows)
// and then its wave's W fragments for the whole slice straight into registers
// (the MFMA A operand: W never passes through LDS), so the slice is in flight
// at once -- one memory round trip per workgroup.  The products of k-tile t
// wait only for that k-tile's W fragments (register loads, which the
// compiler's counters track exactly), so they start while later k-tiles are
// still arriving from HBM.  The fp32 accumulators leave as they are, in
// fragment order, for gemm_reduce_kernel (which sums the K slices and runs
// the epilogue).  Workgroups are ordered slice-major, so the tiles that read
// one A slice share an XCD and its L2.
template <int KT, bool H16, bool PACKED>
__global__ __launch_bounds__(256) void gemm_wstream_kernel(const bf16* __restrict__ A, const bf16* __restrict__ W,
                                                           int M, int N, int K, Epi E) {
  constexpr int BN = 128, BK = 64;
  constexpr int ATILE = 128 * BK;                         // bf16 elements of one k-tile of A
  constexpr int RL = 132;                                 // fp32 row pitch of the row-major staging
  constexpr int AS = KT * ATILE > 64 * RL * 2 ? KT * ATILE : 64 * RL * 2;
  __shared__ __attribute__((aligned(1024))) bf16 as[AS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tiles_n = (N + BN - 1) / BN, tiles = tiles_n * ((M + 127) / 128);
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int slice = lid / tiles, tile = lid % tiles;
  const int n0 = (tile % tiles_n) * BN, m0 = (tile / tiles_n) * 128;
  const int kbase = slice * KT * BK;                      // dispatch: K = ksplit * KT * 64
  // A slice: 16-byte chunks, 8 lanes per 128-byte row piece (rows past M
  // read row M - 1: finite values in accumulators the reduction drops)
  const int crow = tid >> 3, cc = tid & 7;
  bf16x8 ast[4 * KT];
#pragma unroll
  for (int t = 0; t < KT; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      ast[t * 4 + u] = *(const bf16x8*)(A + (int64_t)min(m0 + u * 32 + crow, M - 1) * K + kbase + t * BK + cc * 8);
  // W fragments: lane l holds feature n0 + 32 w + l % 32, k offsets 16 j + 8 (l / 32) .. + 7;
  // from the fragment-ordered copy (PACKED) each fragment is one contiguous
  // 1 KB wave load, from [N][K] it is 32 rows x 32 bytes
  const int lr = lane & 31, lh = lane >> 5;
  bf16x8 wf[4 * KT];
  if constexpr (PACKED) {
    const int nblk = min((n0 >> 5) + wave, ((N + 31) >> 5) - 1);
    const bf16* const wp = (const bf16*)E.wpack + (((int64_t)nblk * (K >> 6) + (kbase >> 6)) * 4) * 512 + lane * 8;
#pragma unroll
    for (int j = 0; j < 4 * KT; ++j) wf[j] = *(const bf16x8*)(wp + j * 512);
  } else {
    const bf16* const wrow = W + (int64_t)min(n0 + wave * 32 + lr, N - 1) * K + kbase + lh * 8;
#pragma unroll
    for (int j = 0; j < 4 * KT; ++j) wf[j] = *(const bf16x8*)(wrow + j * 16);
  }
#pragma unroll
  for (int t = 0; t < KT; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = u * 32 + crow;
      *(bf16x8*)(as + t * ATILE + row * BK + ((cc ^ swz<BK>(row)) * 8)) = ast[t * 4 + u];
    }
  __syncthreads();
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[j][q] = 0.f;
#pragma unroll
  for (int t = 0; t < KT; ++t)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = kk * 2 + lh;
      bf16x8 bfr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = j * 32 + lr;
        bfr[j] = *(const bf16x8*)(as + t * ATILE + row * BK + ((c ^ swz<BK>(row)) * 8));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = mfma32<H16>(wf[t * 4 + kk], bfr[j], acc[j]);
    }
  if (E.part_rows) {
    // row-major partials [slice][M][N], 64 rows at a time through LDS (the A
    // slice has been consumed), each row's 128 features one 512-byte store
    float* const st = (float*)as;
    float* const dst = E.part + (int64_t)slice * M * N;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      __syncthreads();
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(float4*)(st + (32 * jj + lr) * RL + 32 * wave + 8 * g + 4 * lh) =
              make_float4(acc[2 * h + jj][4 * g], acc[2 * h + jj][4 * g + 1], acc[2 * h + jj][4 * g + 2],
                          acc[2 * h + jj][4 * g + 3]);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = tid / 32 + 8 * i, m = m0 + 64 * h + row, n = n0 + 4 * (tid % 32);
        if (m < M && n < N) *(float4*)(dst + (int64_t)m * N + n) = *(const float4*)(st + row * RL + 4 * (tid % 32));
      }
    }
    return;
  }
  // granules [slice][tile][feature block = wave][row block j][g][lane]: lane l
  // holds row 32 j + l % 32, features 32 w + 8 g + 4 (l / 32) + 0..3
  float4* dst = (float4*)E.part + ((((int64_t)slice * tiles + tile) * 4 + wave) * 16) * 64 + lane;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      dst[(j * 4 + g) * 64] = make_float4(acc[j][4 * g], acc[j][4 * g + 1], acc[j][4 * g + 2], acc[j][4 * g + 3]);
}

template <int KT, bool H16>
hipError_t launch_wstream(hipStream_t s, const bf16* A, const bf16* W, int M, int N, int K, const Epi& E) {
  const unsigned grid = (unsigned)(((M + 127) / 128) * ((N + 127) / 128)) * E.ksplit;
  if (E.wpack)
    gemm_wstream_kernel<KT, H16, true><<<grid, 256, 0, s>>>(A, W, M, N, K, E);
  else
    gemm_wstream_kernel<KT, H16, false><<<grid, 256, 0, s>>>(A, W, M, N, K, E);
  return hipGetLastError();
}

// W [N][K] -> fragment order: 16-byte chunk (nb, kt, kk, lane) holds
// W[32 nb + lane % 32][64 kt + 16 kk + 8 (lane / 32) .. + 7], rows past N zero.
__global__ __launch_bounds__(256) void pack_weight_kernel(const bf16* __restrict__ W, int N, int K,
                                                          bf16* __restrict__ out, int64_t chunks) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  const int lane = (int)(c & 63), kk = (int)((c >> 6) & 3);
  const int64_t rest = c >> 8;
  const int kt = (int)(rest % (K >> 6)), nb = (int)(rest / (K >> 6));
  const int n = nb * 32 + (lane & 31), k = kt * 64 + kk * 16 + (lane >> 5) * 8;
  bf16x8 v;
  if (n < N) {
    v = *(const bf16x8*)(W + (int64_t)n * K + k);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (bf16)0.f;
  }
  *(bf16x8*)(out + c * 8) = v;
}

size_t pack_weight_bytes(int N, int K) { return (size_t)((N + 31) / 32) * 32 * (size_t)K * 2; }

hipError_t pack_weight(hipStream_t s, const void* W, int N, int K, void* out) {
  if (N < 1 || K < 64 || K % 64) return hipErrorInvalidValue;
  const int64_t chunks = (int64_t)pack_weight_bytes(N, K) / 16;
  pack_weight_kernel<<<(unsigned)((chunks + 255) / 256), 256, 0, s>>>((const bf16*)W, N, K, (bf16*)out, chunks);
  return hipGetLastError();
}

// Few rows (M <= 256, below the knee where streaming W from HBM bounds the
// product): gemm_wstream_kernel over 128 x 128 tiles with K split into ks
// slices of KT k-tiles (K = 64 ks KT), then gemm_reduce_kernel.  KT is chosen
// by a small cost model: one memory round trip per workgroup plus the bytes
// of W and A over the bandwidth the workgroups can draw, plus the partials'
// write and read-back when ks > 1.  Up to 2048 rows it also takes products
// whose 128 x 128 tiles would occupy at most half of the CUs (the image
// DiT's N = 768 GEMMs: 96 tiles), with the matrix-core time of a slice in the
// model.  0 when the shape does not take this path (more rows, K % 64, no
// partial buffer, N % 4).
static int stream_pick_kt(int M, int N, int K, const Epi& E0) {
  if (M > 2048 || K % 64 || (N & 3) || M < 1) return 0;
  const int KT64 = K / 64;
  const int64_t tiles = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
  const bool few_rows = M <= 256;
  // above 256 rows only the row-major epilogues (the scatters through the
  // reduction's LDS strips measured slower there than the one-pass tile)
  if (!few_rows && (tiles * 2 > device_cus() || E0.mode == EPI_QKV || E0.mode == EPI_CTXKV ||
                    E0.mode == EPI_HEAD || E0.mode == EPI_PATCH))
    return 0;
  const double w_bytes = 2.0 * N * K, a_bytes = 2.0 * M * K * ((N + 127) / 128);
  int best_kt = 0;
  double best_t = 1e30;
  for (int kt = 8; kt >= 1; --kt) {
    if (KT64 % kt) continue;
    const int64_t ks = KT64 / kt;
    if (ks > 64) continue;
    if (!E0.part || ks * tiles * 128 * 128 > E0.part_cap) continue;
    const int64_t wgs = tiles * ks;
    const double rounds = (double)((wgs + 255) / 256);
    const double bw = std::min(8.0e12 * 0.8, (double)std::min<int64_t>(wgs, 256) * 40.0e9);   // bytes/s
    double t = rounds * 2.0e-6 + (w_bytes + a_bytes) / bw;
    if (!few_rows) t += rounds * kt * (64.0 * 128 * 128 * 2) / 4.0e12;     // a slice's products per CU
    if (ks > 1) t += 3.0e-6 + 2.0 * ks * M * N * 4.0 / 10.0e12;
    if (t < best_t * 0.999) {
      best_t = t;
      best_kt = kt;
    }
  }
  return best_kt;
}

// the reduction pass also runs the LayerNorm of the updated rows (residual
// modes, a workgroup of N / 4 threads per row, at most 8 waves)
static bool ln_fusable(int M, int N, int K, const Epi& E) {
  if (!E.ln_out || (E.mode != EPI_RESID && E.mode != EPI_GATE_RESID)) return false;
  if (N % 256 || N > 2048 || E.ln_form < 0 || E.ln_form > 2) return false;
  return stream_pick_kt(M, N, K, E) > 0;
}

bool gemm_fuses_ln(int M, int N, int K, const Epi& E) { return ln_fusable(M, N, K, E); }

// the reduction pass also runs the grouped softmax of the product (F32
// without a bias, groups of at most 128 columns covering N)
static bool sm_fusable(int M, int N, int K, const Epi& E) {
  if (!E.sm_out || E.mode != EPI_F32 || E.bias || E.sm_cp < 1 || E.sm_cp > 128 || E.sm_heads * E.sm_cp != N)
    return false;
  return stream_pick_kt(M, N, K, E) > 0;
}

bool gemm_fuses_softmax(int M, int N, int K, const Epi& E) { return sm_fusable(M, N, K, E); }

template <int MODE, bool H16>
bool launch_stream(hipStream_t s, const bf16* A, const bf16* W, int M, int N, int K, const Epi& E0, hipError_t* err) {
  const int best_kt = stream_pick_kt(M, N, K, E0);
  if (!best_kt) return false;
  const int KT64 = K / 64;
  const int64_t tiles = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
  Epi E = E0;
  E.ksplit = KT64 / best_kt;
  E.part_rows = 0;
  if constexpr (MODE == EPI_RESID || MODE == EPI_GATE_RESID) E.part_rows = ln_fusable(M, N, K, E0) ? 1 : 0;
  if constexpr (MODE == EPI_F32) E.part_rows = sm_fusable(M, N, K, E0) ? 1 : 0;
  switch (best_kt) {
    case 1: *err = launch_wstream<1, H16>(s, A, W, M, N, K, E); break;
    case 2: *err = launch_wstream<2, H16>(s, A, W, M, N, K, E); break;
    case 3: *err = launch_wstream<3, H16>(s, A, W, M, N, K, E); break;
    case 4: *err = launch_wstream<4, H16>(s, A, W, M, N, K, E); break;
    case 5: *err = launch_wstream<5, H16>(s, A, W, M, N, K, E); break;
    case 6: *err = launch_wstream<6, H16>(s, A, W, M, N, K, E); break;
    case 7: *err = launch_wstream<7, H16>(s, A, W, M, N, K, E); break;
    default: *err = launch_wstream<8, H16>(s, A, W, M, N, K, E); break;
  }
  if (*err == hipSuccess) {
    if constexpr (MODE == EPI_RESID || MODE == EPI_GATE_RESID) {
      if (E.part_rows) {
        const unsigned nt = (unsigned)(N / 4);
        if (E.ln_form == 1)
          gemm_reduce_ln_kernel<MODE, f16, false><<<(unsigned)M, nt, 0, s>>>(M, N, E);
        else if (E.ln_form == 2)
          gemm_reduce_ln_kernel<MODE, bf16, true><<<(unsigned)M, nt, 0, s>>>(M, N, E);
        else
          gemm_reduce_ln_kernel<MODE, bf16, false><<<(unsigned)M, nt, 0, s>>>(M, N, E);
        *err = hipGetLastError();
        return true;
      }
    }
    if constexpr (MODE == EPI_F32) {
      if (E.part_rows) {
        const int64_t groups = (int64_t)M * E.sm_heads;
        gemm_reduce_softmax_kernel<<<(unsigned)((groups + 15) / 16), 256, 0, s>>>(M, N, E);
        *err = hipGetLastError();
        return true;
      }
    }
    gemm_reduce_kernel<MODE><<<(unsigned)(tiles * 8), 256, 0, s>>>(M, N, E);
    *err = hipGetLastError();
  }
  return true;
}

template <int MODE, bool H16 = false>
hipError_t gemm_mfma_mode(hipStream_t s, const bf16* A, const bf16* W, int M, int N, int K, const Epi& E) {
  // pick the tile that minimises (rounds of resident workgroups) x (cost per
  // tile); larger tiles cost less per flop.  256 x 256 with 8 waves keeps two
  // waves per SIMD; the 4-wave tiles run one.
  struct Opt { int bm, bn, per_cu; double eff; };
  const Opt opts[3] = {{256, 256, 1, 1.0}, {256, 128, 1, 0.85}, {128, 128, 2, 0.7}};
  int best = 0;
  double best_t = 1e30;
  for (int i = 0; i < 3; ++i) {
    const int64_t tiles = (int64_t)((M + opts[i].bm - 1) / opts[i].bm) * ((N + opts[i].bn - 1) / opts[i].bn);
    const int64_t slots = 256 * opts[i].per_cu;
    const int64_t rounds = (tiles + slots - 1) / slots;
    const double t = (double)rounds * opts[i].bm * opts[i].bn / (opts[i].eff * opts[i].per_cu);
    if (t < best_t * 0.999) {
      best_t = t;
      best = i;
    }
  }
  {
    hipError_t err = hipSuccess;
    if (launch_stream<MODE, H16>(s, A, W, M, N, K, E, &err)) return err;
  }
  if (K % 64 == 0) {
    // direct-to-LDS, DMA spread over the MFMAs, one workgroup per CU, tiles of
    // 256 columns and 256, 224, 192 or 160 rows (224 and 160 split unevenly
    // over the two wave rows: 128 + 96 and 96 + 64), whichever needs the
    // fewest (rounds of resident tiles) x (tile rows), ties to the larger
    // tile; the 160-row tile is charged 8 % (more operand traffic per flop,
    // a half-empty last epilogue strip: the video QKV measured 5 % slower on
    // 3 rounds of 160 rows than on 2 of 256).  Measured at the video shapes
    // (6240 rows, normal operands, one box): QKV 130.5 us on 256-row tiles
    // (450 tiles, 1.76 rounds) vs 104.3 on 224 (504, 1.97); FFN1 221.8 on
    // 192 vs 204.9 on 224; N = 1536 (FFN2) 179.0 on 192 (198 tiles) vs 165.9
    // on 160 (234).
    const int64_t cus = device_cus();
    const int64_t tn = (N + 255) / 256;
    auto cost = [&](int bm) { return ((M + bm - 1) / bm * tn + cus - 1) / cus * bm; };
    const int64_t t192 = (int64_t)((M + 191) / 192) * tn;
    // small problems: when even the 192-row tiles would occupy fewer than 60 %
    // of the CUs, 128 x 128 tiles (4 waves, two workgroups per CU) spread the
    // work over more of them (measured faster on every GEMM of the 12- and
    // 24-block image DiTs, slower on the video DiT's 198-tile N = 1536 GEMMs)
    if (t192 * 10 < cus * 6) return launch_dma<128, 128, 4, 64, 2, true, MODE, H16>(s, A, W, M, N, K, E);
    const int64_t c256 = cost(256), c224 = cost(224), c192 = cost(192), c160 = cost(160) * 108 / 100;
    const int64_t best = std::min(std::min(c256, c224), std::min(c192, c160));
    if (c256 == best) return launch_dma<256, 256, 8, 64, 2, true, MODE, H16>(s, A, W, M, N, K, E);
    if (c224 == best) return launch_dma<224, 256, 8, 64, 2, true, MODE, H16, 128>(s, A, W, M, N, K, E);
    if (c192 == best) return launch_dma<192, 256, 8, 64, 2, true, MODE, H16>(s, A, W, M, N, K, E);
    return launch_dma<160, 256, 8, 64, 3, true, MODE, H16, 96>(s, A, W, M, N, K, E);
  }
  const int bm = opts[best].bm, bn = opts[best].bn;
  const unsigned grid = (unsigned)(((M + bm - 1) / bm) * ((N + bn - 1) / bn));
  if (best == 0)
    gemm_mfma_kernel<256, 256, 8, MODE, H16><<<grid, 512, 0, s>>>(A, W, M, N, K, E);
  else if (best == 1)
    gemm_mfma_kernel<256, 128, 4, MODE, H16><<<grid, 256, 0, s>>>(A, W, M, N, K, E);
  else
    gemm_mfma_kernel<128, 128, 4, MODE, H16><<<grid, 256, 0, s>>>(A, W, M, N, K, E);
  return hipGetLastError();
}

hipError_t gemm_mfma(hipStream_t s, const void* A, const void* W, int M, int N, int K, const Epi& E) {
  // operand offsets are 32-bit
  if ((uint64_t)M * K >= (1ull << 32) || (uint64_t)N * K >= (1ull << 32)) return hipErrorInvalidValue;
  const bf16* a = (const bf16*)A;
  const bf16* w = (const bf16*)W;
  switch (E.mode) {
    case EPI_STORE: return gemm_mfma_mode<EPI_STORE>(s, a, w, M, N, K, E);
    case EPI_GELU: return gemm_mfma_mode<EPI_GELU>(s, a, w, M, N, K, E);
    case EPI_GATE_RESID: return gemm_mfma_mode<EPI_GATE_RESID>(s, a, w, M, N, K, E);
    case EPI_RESID: return gemm_mfma_mode<EPI_RESID>(s, a, w, M, N, K, E);
    case EPI_PATCH: return gemm_mfma_mode<EPI_PATCH>(s, a, w, M, N, K, E);
    case EPI_QKV: return gemm_mfma_mode<EPI_QKV>(s, a, w, M, N, K, E);
    case EPI_HEAD: return gemm_mfma_mode<EPI_HEAD>(s, a, w, M, N, K, E);
    case EPI_CTXKV: return gemm_mfma_mode<EPI_CTXKV>(s, a, w, M, N, K, E);
    case EPI_F32: return gemm_mfma_mode<EPI_F32>(s, a, w, M, N, K, E);
    default: return hipErrorInvalidValue;
  }
}

hipError_t gemm_mfma_f16(hipStream_t s, const void* A, const void* W, int M, int N, int K, const Epi& E) {
  if ((uint64_t)M * K >= (1ull << 32) || (uint64_t)N * K >= (1ull << 32)) return hipErrorInvalidValue;
  if (M == 0 || N == 0) return hipSuccess;
  const bf16* a = (const bf16*)A;
  const bf16* w = (const bf16*)W;
  switch (E.mode) {
    case EPI_RESID: return gemm_mfma_mode<EPI_RESID, true>(s, a, w, M, N, K, E);
    case EPI_F32: return gemm_mfma_mode<EPI_F32, true>(s, a, w, M, N, K, E);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sdk
