// Four-element loads and stores of the LayerNorm kernels, and the
// LayerNorm + modulation of one row held as one float4 per thread (the
// workgroup spans the row).  Shared by the LayerNorm kernels and the
// few-row GEMM reduction that normalises the residual it has just updated,
// so both produce the same values from the same row.
#pragma once
#include "common.h"

namespace sdk {

template <typename T>
SD_DEV void store4(T* p, const float* o);
template <>
SD_DEV void store4<float>(float* p, const float* o) { *(float4*)p = make_float4(o[0], o[1], o[2], o[3]); }
template <>
SD_DEV void store4<bf16>(bf16* p, const float* o) {
  bf16x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = (bf16)o[q];
  *(bf16x4*)p = v;
}
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
template <>
SD_DEV void store4<f16>(f16* p, const float* o) {
  f16x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = (f16)o[q];
  *(f16x4*)p = v;
}
SD_DEV void load4(const float* p, float* o) {
  const float4 v = *(const float4*)p;
  o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
SD_DEV void load4(const bf16* p, float* o) {
  const bf16x4 v = *(const bf16x4*)p;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = (float)v[q];
}
SD_DEV void load4(const f16* p, float* o) {
  const f16x4 v = *(const f16x4*)p;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = (float)v[q];
}


// Shift and scale of float4 j of a row: the row's modulation slots mr[off + .]
// plus the block table blk[off + .] (blk may be NULL).
template <typename T>
SD_DEV void ln_row_mod(const float* mr, const T* blk, int shift_off, int scale_off, int j, float* sh, float* sc) {
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
}

// LayerNorm (population variance, eps) of the row whose float4 j = threadIdx.x
// this thread holds in v (blockDim = d / 4, nw waves), then, with `mod`,
// o * (1 + sc) + sh.  red: LDS scratch [2][8] (nw <= 8).  Two workgroup
// barriers.
SD_DEV void ln_row(const float4 v, int d, float eps, bool mod, const float* sh, const float* sc, float (*red)[8],
                   int nw, int lane, int wave, float* o) {
  const float s1 = wave_sum((v.x + v.y) + (v.z + v.w));
  if (lane == 0) red[0][wave] = s1;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < nw; ++w) tot += red[0][w];
  const float mu = tot / (float)d;
  const float a0 = v.x - mu, a1 = v.y - mu, a2 = v.z - mu, a3 = v.w - mu;
  const float s2 = wave_sum((a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3));
  if (lane == 0) red[1][wave] = s2;
  __syncthreads();
  float sq = 0.f;
  for (int w = 0; w < nw; ++w) sq += red[1][w];
  const float rstd = 1.0f / sqrtf(sq / (float)d + eps);
  o[0] = a0 * rstd;
  o[1] = a1 * rstd;
  o[2] = a2 * rstd;
  o[3] = a3 * rstd;
  if (mod) {
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = o[q] * (1.0f + sc[q]) + sh[q];
  }
}

// Store of the normalised values: T [d] per row, or with SPLIT the bf16
// hi / lo pair, row pitch 2d (hi in [0, d), lo in [d, 2d)).
template <typename T, bool SPLIT>
SD_DEV void ln_row_store(T* orow, int d, int j, const float* o) {
  store4<T>(orow + 4 * j, o);
  if constexpr (SPLIT) {
    float lo[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) lo[q] = o[q] - (float)(T)o[q];
    store4<T>(orow + d + 4 * j, lo);
  }
}

}  // namespace sdk
