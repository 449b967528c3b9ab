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
#include <cmath>

#include <type_traits>

#include "kernels.h"

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

template <int BM, int BN, int NW, int MODE>
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
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if constexpr (MODE == EPI_QKV) {
    if (tid == 0) {
#pragma unroll
      for (int i = 0; i < SD_MAX_ROWS; ++i) t0s[i] = E.t0[i];
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

template <int BM, int BN, int NW, int BK, int NS, bool SPREAD, int MODE>
__global__ __launch_bounds__(64 * NW) void gemm_dma_kernel(const bf16* __restrict__ A, const bf16* __restrict__ W,
                                                          int M, int N, int K, Epi E) {
  constexpr int NT = 64 * NW, WN = NW / 2;
  constexpr int TM = BM / 2, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  constexpr int CPR = BK / 8, RPB = 64 / CPR;             // chunks per row, rows per DMA block
  constexpr int AQ = BM / RPB / NW, BQ = BN / RPB / NW;   // DMA blocks per wave per k-tile
  constexpr int DQ = AQ + BQ;
  constexpr int STAGE = (BM + BN) * BK;                   // bf16 elements per stage
  constexpr int LC = BN + 4;
  static_assert(AQ >= 1 && BQ >= 1 && AQ * RPB * NW == BM && BQ * RPB * NW == BN, "tile shape");
  static_assert(NS >= 2 && NS <= 4 && DQ * (NS - 2) < 64, "stages");
  static_assert(64 * LC * 4 <= NS * STAGE * 2, "epilogue strip must fit in the stage buffers");
  // one LDS block with the stage buffers at offset 0 (the row table and the
  // per-row RoPE bases follow them): left to the compiler, the placement of
  // the small arrays could move the stage buffers off offset 0, which costs
  // up to half the throughput of the gated-residual kernels
  constexpr int SMEM_BYTES = NS * STAGE * 2;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[SMEM_BYTES + 64 * 16 + SD_MAX_ROWS * 4];
  bf16* const smem = (bf16*)lds;
  int4* const rowtab = (int4*)(lds + SMEM_BYTES);
  int* const t0s = (int*)(lds + SMEM_BYTES + 64 * 16);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
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

  // per-lane source offsets (elements) of this wave's DMA blocks, k-tile 0;
  // rows beyond M / N are clamped (they feed outputs that are never stored)
  uint32_t a_src[AQ], b_src[BQ];
  const int lrow = lane / CPR, lpos = lane % CPR;
#pragma unroll
  for (int q = 0; q < AQ; ++q) {
    const int r = (wave * AQ + q) * RPB + lrow;
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
      if (part < 0 || q * (BK / 16) / DQ == part)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(A + a_src[q] + k0),
                                         (__attribute__((address_space(3))) void*)(as + (wave * AQ + q) * RPB * BK),
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
  // MFMAs over stage buf; with SPREAD and WI the DMA of k-tile nkt into stage
  // nbuf is issued a part per 16-wide k step
  auto compute = [&](int buf, int nkt, int nbuf, auto wi) {
    const bf16* as = smem + buf * STAGE;
    const bf16* bs = as + BM * BK;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if constexpr (SPREAD && decltype(wi)::value) issue(nkt, nbuf, ks);
      const int c = ks * 2 + lh;           // logical 16-byte chunk of this lane
      bf16x8 fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm * TM + i * 32 + lr;
        fa[i] = *(const bf16x8*)(as + row * BK + ((c ^ swz<BK>(row)) * 8));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = wn * TN + j * 32 + lr;
        fb[j] = *(const bf16x8*)(bs + row * BK + ((c ^ swz<BK>(row)) * 8));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  };

  if constexpr (MODE == EPI_QKV) {
    if (tid == 0) {
#pragma unroll
      for (int i = 0; i < SD_MAX_ROWS; ++i) t0s[i] = E.t0[i];
    }
  }
  const int KT = K / BK;
#pragma unroll
  for (int t = 0; t < NS - 1; ++t)
    if (t < KT) issue(t, t, -1);
  // one k-tile: tiles kt+1 .. kt+NS-2 may stay in flight; tile kt must have
  // landed in every wave, and every wave must be done reading tile kt-1.  WI:
  // k-tile kt+NS-1 exists and its DMA goes out during this tile's MFMAs.
  auto step = [&](int kt, auto wi) {
    const int ahead = min(NS - 2, KT - 1 - kt);
    if constexpr (NS >= 4) {
      if (ahead >= 2) wait_vm_barrier<DQ * 2>();
      else if (ahead == 1) wait_vm_barrier<DQ>();
      else wait_vm_barrier<0>();
    } else if constexpr (NS == 3) {
      if (ahead >= 1) wait_vm_barrier<DQ>();
      else wait_vm_barrier<0>();
    } else {
      wait_vm_barrier<0>();
    }
    const int nkt = kt + NS - 1;
    if constexpr (!SPREAD && decltype(wi)::value) issue(nkt, nkt % NS, -1);
    compute(kt % NS, nkt, nkt % NS, wi);
  };
  int kt = 0;
  for (; kt + NS - 1 < KT; ++kt) step(kt, std::true_type{});
  for (; kt < KT; ++kt) step(kt, std::false_type{});
  __syncthreads();

  // epilogue in 64-row strips staged through LDS; a strip gathers the
  // 32-row fragment rows of whichever waves hold them (TM may be 96)
  float* stg = (float*)smem;
#pragma unroll
  for (int s = 0; s < BM / 64; ++s) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int rb = wm * TM + i * 32;
      if (rb / 64 == s) {
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
    epi_rows<MODE>(E, rowtab, m0 + s * 64, M, tid, t0s);
    __syncthreads();
    epi_strip<BN, NT, MODE>(E, stg, LC, m0 + s * 64, n0, M, N, tid, rowtab);
    __syncthreads();
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

template <int BM, int BN, int NW, int BK, int NS, bool SPREAD, int MODE>
hipError_t launch_dma(hipStream_t s, const bf16* A, const bf16* W, int M, int N, int K, const Epi& E) {
  const unsigned grid = (unsigned)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
  gemm_dma_kernel<BM, BN, NW, BK, NS, SPREAD, MODE><<<grid, 64 * NW, 0, s>>>(A, W, M, N, K, E);
  return hipGetLastError();
}

template <int MODE>
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
  if (K % 64 == 0) {
    // direct-to-LDS, DMA spread over the MFMAs, one workgroup per CU: 256 x 256
    // or 192 x 256 tiles, whichever needs the smaller (rounds of resident
    // tiles) x (tile area); 192-row tiles fill more CUs when the 256-row
    // grid leaves many idle (N = 1536: 150 vs 198 tiles on 256 CUs)
    const int64_t cus = device_cus();
    const int64_t t256 = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
    const int64_t t192 = (int64_t)((M + 191) / 192) * ((N + 255) / 256);
    const int64_t c256 = (t256 + cus - 1) / cus * 256, c192 = (t192 + cus - 1) / cus * 192;
    // small problems: when even the 192-row tiles would occupy fewer than 60 %
    // of the CUs, 128 x 128 tiles (4 waves, two workgroups per CU) spread the
    // work over more of them (measured faster on every GEMM of the 12- and
    // 24-block image DiTs, slower on the video DiT's 198-tile N = 1536 GEMMs)
    if (t192 * 10 < cus * 6) return launch_dma<128, 128, 4, 64, 2, true, MODE>(s, A, W, M, N, K, E);
    if (c192 < c256) return launch_dma<192, 256, 8, 64, 2, true, MODE>(s, A, W, M, N, K, E);
    return launch_dma<256, 256, 8, 64, 2, true, MODE>(s, A, W, M, N, K, E);
  }
  const int bm = opts[best].bm, bn = opts[best].bn;
  const unsigned grid = (unsigned)(((M + bm - 1) / bm) * ((N + bn - 1) / bn));
  if (best == 0)
    gemm_mfma_kernel<256, 256, 8, MODE><<<grid, 512, 0, s>>>(A, W, M, N, K, E);
  else if (best == 1)
    gemm_mfma_kernel<256, 128, 4, MODE><<<grid, 256, 0, s>>>(A, W, M, N, K, E);
  else
    gemm_mfma_kernel<128, 128, 4, MODE><<<grid, 256, 0, s>>>(A, W, M, N, K, E);
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

}  // namespace sdk
