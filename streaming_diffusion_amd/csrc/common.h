// Shared device-side definitions for the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sd_stream.h"

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define SD_DEV __device__ __forceinline__

SD_DEV float to_f(float x) { return x; }
SD_DEV float to_f(bf16 x) { return (float)x; }
template <typename T> SD_DEV T from_f(float x);
template <> SD_DEV float from_f<float>(float x) { return x; }
template <> SD_DEV bf16 from_f<bf16>(float x) { return (bf16)x; }

SD_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
SD_DEV double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
SD_DEV long long wave_sum_i64(long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// MI355X dispatches consecutive workgroups of a launch round-robin over its
// 8 XCDs, each with a private L2.  xcd_remap turns the hardware workgroup id
// into a logical id such that each XCD receives one contiguous range of
// logical ids (a bijection on [0, n)); neighbouring logical work items --
// which share operands -- then meet in the same L2.
#define SD_NUM_XCD 8
SD_DEV int xcd_remap(int pid, int n) {
  const int xcd = pid % SD_NUM_XCD, k = pid / SD_NUM_XCD;
  const int base = n / SD_NUM_XCD, rem = n % SD_NUM_XCD;
  return (xcd < rem ? xcd * (base + 1) : rem * (base + 1) + (xcd - rem) * base) + k;
}

// Per-row description of one forward.  Passed by value as a kernel argument.
struct RowInfo {
  int32_t frame;      // frame-store record of the row's latent
  int32_t tau;        // timestep
  int32_t t0;         // temporal RoPE base
  int32_t kind;       // 0 = denoise slot, 1 = negative-prompt row (onetime R-CFG, full CFG)
  int32_t last;       // 1 if this slot is the last (the frame leaves)
  int32_t ctx;        // 0 = positive context, 1 = negative
  float a, b;         // sqrt(alpha_tau), sqrt(1 - alpha_tau)
  float an, bn;       // coefficients of the next slot's timestep
  float a0, b0;       // entry timestep coefficients (negative row)
  int32_t oidx;       // last slot: position of the frame among the step's outputs
  int32_t neg;        // entering frame with onetime R-CFG: its negative row, else -1
  int32_t pair;       // full CFG: the row's twin under the negative prompt, else -1
  int32_t zrow;       // LCM sampler, not the last slot: record of the re-noise latent, else -1
  int32_t keep;       // last slot with clean-latent recompute: x0_hat also stays in the frame record
};
struct RowTable {
  int32_t R;
  RowInfo r[SD_MAX_ROWS];
};

// Everything of a forward that changes from step to step while the launch
// sequence stays the same: the rows, their RoPE bases, the self-attention's
// sink / window ranges and the ring positions of the leaving chunks' appends.
// Written to device memory by one small kernel before the forward, so that a
// captured graph of the forward can be replayed with new values.
struct StepDyn {
  RowTable rt;
  int32_t t0[SD_MAX_ROWS];
  int32_t seg[4];                 // sink start, sink count, window start, window count
  int32_t kv_pos[SD_MAX_CHUNKS];  // ring position of leaving chunk k's append
  int32_t ptr_old;                // ring position of the first leaving chunk
};

// GEMM epilogue modes: C[m][n] = sum_k A[m][k] * W[n][k], then:
enum EpiMode {
  EPI_STORE = 0,      // out[m][n] = T(acc + bias[n])
  EPI_GELU = 1,       // out[m][n] = T(gelu(acc + bias[n]))
  EPI_GATE_RESID = 2, // resid[m][n] += gate[r][n] * (acc + bias[n])
  EPI_RESID = 3,      // resid[m][n] += acc + bias[n]
  EPI_PATCH = 4,      // resid[m][n] = acc + bias[n]
  EPI_QKV = 5,        // split q|k|v, RoPE on q,k, scatter to per-head layouts
  EPI_HEAD = 6,       // eps[r][unpatchify(m, n)] = acc + bias[n]   (fp32)
  EPI_CTXKV = 7,      // split k|v of a context to per-head cache layouts
  EPI_F32 = 8         // outf[m][n] = acc + bias[n]  (fp32 out, tests)
};

struct Epi {
  int mode;
  const void* bias;     // [N], element type of the GEMM (may be null)
  void* out;            // EPI_STORE / EPI_GELU / EPI_F32 output, leading dim ldo
  int ldo;
  float* resid;         // fp32 [M][N]
  const float* mod;     // [R][6d] shared modulation (gate source)
  const void* blk;      // [6d] block table (element type of the GEMM)
  int gate_off;         // offset of the gate inside 6d
  int six_d;            // 6d
  int L;                // tokens per row
  // EPI_QKV / EPI_CTXKV destinations (element type of the GEMM); k and vt
  // are head-major so that one head's keys of all rows are contiguous
  void* q;              // [R][H][L][hd]
  void* k;              // [H][krows][kstride][hd]
  void* vt;             // [H][hd][krows][kstride]   (V stored transposed)
  int kstride;          // token capacity of the k/vt destination per (row, head)
  int krows;            // rows of the k/vt destination (1 for a context)
  int H, hd, d;
  int rope;             // apply RoPE to q and k
  int Hp, Wp;           // token grid of one latent frame
  int dt, dh;           // RoPE section widths (t, h); w = hd - dt - dh
  const float2* rope_t; // [positions][dt/2] (cos, sin)
  const float2* rope_h; // [Hp][dh/2]
  const float2* rope_w; // [Wp][dw/2]
  int t0[SD_MAX_ROWS];
  const int* t0_dev;    // when set, the RoPE bases are read from device memory instead of t0
  // EPI_HEAD
  float* eps;           // [R][T][C][Hl][Wl]
  int C, Hl, Wl, p, T;
  // split over K for few rows: fp32 partials of ksplit slices, each
  // ceil(M/128) ceil(N/128) tiles of 128 x 128 in accumulator order (capacity
  // part_cap floats; null: no split); ksplit is set by the dispatch
  float* part;
  int64_t part_cap;
  int ksplit;
  int part_rows;        // partials row-major [slice][M][N] instead (for the fused LayerNorm pass)
  // the same W in fragment order (pack_weight), read by the few-row product
  // when set (null: W is read as [N][K])
  const void* wpack;
  // EPI_RESID / EPI_GATE_RESID on the few-row path: when ln_out is set the
  // reduction pass also writes the LayerNorm (+ modulation) of each updated
  // residual row to ln_out (form 0 plain in the GEMM's type, 1 fp16 without
  // modulation, 2 bf16 hi / lo pair), the computation of the LayerNorm
  // kernel; gemm_fuses_ln() says whether a call takes that path
  void* ln_out;
  const float* ln_mod;  // [R][ln_six] modulation rows (null: none)
  const void* ln_blk;   // [ln_six] block table (null: none)
  int ln_shift, ln_scale, ln_six, ln_form;
  float ln_eps;
  // EPI_F32 on the few-row path: when sm_out is set the reduction pass writes
  // softmax over each of the sm_heads groups of sm_cp columns of (C + sm_bias)
  // to sm_out in fp16 instead of C itself (the folded cross-attention's
  // probabilities); gemm_fuses_softmax() says whether a call does
  f16* sm_out;
  const float* sm_bias;
  int sm_heads, sm_cp;
};
