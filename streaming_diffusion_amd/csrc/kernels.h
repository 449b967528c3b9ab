// Launchers of the gfx950 kernels.  Every launcher enqueues on the given
// stream and returns the launch status; shapes are checked by the caller.
#pragma once
#include "common.h"

namespace sdk {

// ---------------------------------------------------------------- elementwise
// xs = a*x0 + b*noise; x0s = x0 (when x0s != nullptr).
hipError_t entry_noise(hipStream_t s, const float* x0, const float* noise, float* xs, float* x0s, int64_t n,
                       float a, float b);
// R-CFG, x0 prediction and re-noise for every denoise row of the device row
// table rt (R rows).
hipError_t rcfg_update(hipStream_t s, const RowTable* rt, int R, float* store_x, float* store_x0s, const float* eps,
                       const float* store_z, float* out, int64_t lat, float gamma, float delta);
// Gather patches of each row's latent into [R*L][p*p*C] (element type by bf);
// split (bf16): [R*L][2*p*p*C], each token's values as hi then lo parts.
hipError_t patchify(hipStream_t s, bool bf, const RowTable* rt, int R, const float* store_x, void* out, int64_t lat,
                    int T, int C, int Hl, int Wl, int p, bool split = false);
// LayerNorm (no affine, population variance) then optional modulation
// x*(1+scale)+shift with scale/shift = mod[r][off] + blk[off]; output element
// type by bf (form LN_PLAIN), fp16 without modulation (LN_F16), or bf16 as a
// hi / lo pair per element, row pitch 2d (LN_SPLIT).
enum { LN_PLAIN = 0, LN_F16 = 1, LN_SPLIT = 2 };
hipError_t ln_mod(hipStream_t s, bool bf, const float* x, void* out, int M, int d, int L, const float* mod,
                  const void* blk, int shift_off, int scale_off, int six_d, float eps, int form = LN_PLAIN);
// Sinusoidal timestep embedding per row: [cos(tau w_j), sin(tau w_j)], fp64 math.
hipError_t temb_embed(hipStream_t s, const RowTable* rt, int R, float* out, int d_freq);
// Copy the step's dynamic values to device memory (one small launch).
hipError_t dyn_write(hipStream_t s, const StepDyn& d, StepDyn* dst);
// y[r][n] = act(sum_k x[r][k] W[n][k] + b[n]); act 0 = none, 1 = SiLU.
hipError_t gemv(hipStream_t s, bool bf, const float* x, const void* W, const void* b, float* y, int R, int N, int K,
                int act);
// Append the exiting row's own K / V^T to the ring; optionally capture its
// first Se tokens as sink entry (sink_off .. sink_off+Se).
// kown: head h's [L][hd] keys start at kown + h * k_hs; vtown: the V^T row of
// (h, e) starts at vtown + (h * hd + e) * vt_ps.
// ptr_dev (nullable): the ring position is read from device memory instead
// of ptr (then ptr only selects the kernel: any multiple of 8 below W).
hipError_t kv_append(hipStream_t s, bool bf, const void* kown, const void* vtown, int64_t k_hs, int64_t vt_ps,
                     void* ringK, void* ringVT, int H, int hd, int L, int W, int ptr, void* sinkK, void* sinkVT, int S8,
                     int sink_off, int Se, const int* ptr_dev = nullptr);
// Predicated sink refresh copy over all blocks (flag[0] != 0 -> entry flag[1]).
hipError_t sink_copy(hipStream_t s, bool bf, const int* flag, const void* ringK, const void* ringVT, void* sinkK,
                     void* sinkVT, int nb, int H, int hd, int W, int S8, int ptr_old, int Se,
                     const int* ptr_old_dev = nullptr);
hipError_t fill_zero(hipStream_t s, void* p, size_t bytes);
// Host: one section of the 3D RoPE table, (cos, sin) of pos * base^(-2j/width)
// for pos < npos, j < width/2, written as npos * max(1, width/2) pairs
// (width 0: a single identity pair per position).
void rope_table_fill(float2* out, int npos, int width, double base);
// cross-attention with folded prompt projections (k_attn.hip): the folded
// score / output matrices of one block and context, and the grouped softmax
// kv: the context's fp32 K | V projections, token-major [C][2d]; the folded
// matrices are fp16 (score and output GEMMs run on fp16 operands)
hipError_t cross_fold(hipStream_t s, const float* kv, const bf16* Wq, const bf16* bq, const bf16* Wo, f16* wq_f,
                      float* cq, f16* wo_f, int d, int H, int hd, int C, int Cp);
hipError_t ctx_softmax(hipStream_t s, const float* S, const float* c, f16* P, int64_t M, int H, int Cp);

// ---------------------------------------------------------------- reductions
// Exact int64 (sum a*b, sum a*a, sum b*b); kind 0 = uint8, 1 = fp32 latents
// quantised to rint(x * 2^12) clamped to +-2^20.
hipError_t ssf_sums(hipStream_t s, int kind, const void* a, const void* b, int64_t n, long long* out3);
// Exact int64 sum of squared differences of quantised frames for each of the
// T frame pairs (prev_last, cur[0]), (cur[0], cur[1]), ...; pair 0 skipped
// (written 0) when prev_last is null.
hipError_t motion_sums(hipStream_t s, const float* cur, const float* prev_last, int T, int64_t n, long long* out);
// Chunk embedding (token mean of x [L][d]) and cosine decision against the
// sink embeddings.  capture_entry >= 0 stores h as that entry instead.
hipError_t sink_score(hipStream_t s, const float* x, double* partial, int L, int d, double* emb, int M,
                      int capture_entry, double tau, int* flag, double* sim);

// ---------------------------------------------------------------- GEMM
// C = A[M][K] * W[N][K]^T with epilogue E; element type by bf (bf16 on MFMA,
// fp32 on the vector ALUs).
hipError_t gemm(hipStream_t s, bool bf, const void* A, const void* W, int M, int N, int K, const Epi& E);
// bf16 matrix-core path of gemm() (K a multiple of 8).
hipError_t gemm_mfma(hipStream_t s, const void* A, const void* W, int M, int N, int K, const Epi& E);
// Whether gemm_mfma / gemm_mfma_f16 with these arguments runs the LayerNorm
// of E.ln_out itself (the few-row path, residual modes, row width a multiple
// of 256 up to 4096); when false the caller runs ln_mod after the GEMM.
bool gemm_fuses_ln(int M, int N, int K, const Epi& E);
// Whether a call with E.sm_out set writes the grouped softmax itself (the
// few-row path); when false the caller stores C and runs ctx_softmax.
bool gemm_fuses_softmax(int M, int N, int K, const Epi& E);
// The same with fp16 operands A and W (bias stays bf16); EPI_F32 and EPI_RESID.
hipError_t gemm_mfma_f16(hipStream_t s, const void* A, const void* W, int M, int N, int K, const Epi& E);
// A weight W [N][K] (16-bit elements, K a multiple of 64) rearranged for the
// few-row product (Epi::wpack): 16-byte chunk (nb, kt, kk, lane) holds
// W[32 nb + lane % 32][64 kt + 16 kk + 8 (lane / 32) .. + 7], rows past N zero.
size_t pack_weight_bytes(int N, int K);
hipError_t pack_weight(hipStream_t s, const void* W, int N, int K, void* out);

// ---------------------------------------------------------------- attention
struct KvSeg {
  const void* k;          // K   [.][cap][hd]  (head stride k_hs, row stride k_rs)
  const void* vt;         // V^T [.][hd][cap]  (head stride vt_hs, row stride vt_rs)
  long long k_hs, vt_hs, k_rs, vt_rs;
  int cap;                // token capacity (V^T row pitch, ring modulus)
  int start;              // position of the first valid token
  int count;              // valid tokens
  int wrap;               // positions are taken modulo cap
};
struct AttnArgs {
  const void* q;          // q(r,h,t) = q + r*q_rs + h*q_hs + t*hd
  long long q_rs, q_hs;
  void* o;                // token-major [R*L][d]
  int R, H, L, hd, d;
  int r0;                 // first row of this launch (rows r0 .. r0+R-1)
  int nseg;
  KvSeg seg[3];
  float scale;            // 1/sqrt(hd)
  // split over the key sequence (bf16 path): nsplit workgroups share one
  // query tile, each writes unnormalised O (bf16) and its (max, sum) to
  // part_o [nsplit][rows*L][d] / part_ml [nsplit][rows][H][L] (row index
  // absolute, strides part_so / part_sml elements), then a combine pass
  // normalises.  nsplit = 1 writes O directly.
  int nsplit;
  // heads [0, h_full) are not split: each of their query tiles is one
  // workgroup over the whole key sequence that writes O directly; only heads
  // [h_full, H) are split nsplit ways (and combined).  The unsplit
  // workgroups come first in the grid, so they are dispatched first and the
  // short split pieces fill the slots they leave.
  int h_full;
  bf16* part_o;
  float2* part_ml;
  long long part_so, part_sml;
  // bf16 path: when set, (start, count) of segments 0 and 1 are read from
  // dyn_seg[0..3] in device memory instead of seg[0], seg[1]
  const int* dyn_seg;
};
// With combine = false a split launch leaves its partials for a separate
// attention_combine() call (so the two passes can be timed apart).
hipError_t attention(hipStream_t s, bool bf, const AttnArgs& a, bool combine = true);
hipError_t attention_combine(hipStream_t s, const AttnArgs& a);
// The combine pass of a split launch (none when nothing was split) and the
// vectorised KV append k in one launch (k must satisfy kv_append_vec_ok).
struct KvAppendArgs;
hipError_t attention_combine_append(hipStream_t s, const AttnArgs& a, const KvAppendArgs& k);
bool kv_append_vec_ok(bool bf, int64_t k_hs, int64_t vt_ps, int H, int hd, int L, int W, int ptr, const void* sinkK,
                      int S8, int sink_off, int Se);
// Queries per attention workgroup and resident attention workgroups per CU.
int attention_q_tile(bool bf, int hd);
int attention_wg_per_cu(bool bf, int hd);
// Split count that best fills `concurrent` resident workgroups for `units`
// query tiles over `tiles` key tiles (1 .. max_split).
int attention_pick_split(int units, int tiles, int max_split, int concurrent);
// Split plan for `heads` heads of `units_per_head` query tiles each over
// `tiles` key tiles: the first *h_full heads unsplit, the others split
// *nsplit ways (*h_full = 0: every head split, *nsplit = 1: none).
void attention_pick_plan(int heads, int units_per_head, int tiles, int max_split, int concurrent, int* nsplit,
                         int* h_full);

// ---------------------------------------------------------------- Stream-VAE
// Causal 3x3x3 convolution: x bf16 [T][H][W][Cin], cache bf16 [2][H][W][Cin]
// (input frames -2, -1; null = zeros), w bf16 [Cout][27 Cin], b bf16 [Cout]
// (null = 0); output bf16 channels-last y [T][H][W][Cout] (Cout a multiple of
// 4) or, when ycf is set, fp32 channels-first ycf [T][Cout][H][W] (any Cout).
// Cin a multiple of 8.
struct ConvArgs {
  const bf16* x;
  const bf16* cache;
  const bf16* w;
  const bf16* b;
  bf16* y;
  float* ycf;
  int T, H, W, Cin, Cout;
  bool h16;             // x, cache, w and y hold fp16 words (b stays bf16)
  // x and cache hold the input at half the height and width ([.][H/2][W/2]
  // [Cin]); the convolution reads it upsampled 2x2 (nearest).  Only where
  // conv3d_upsample_ok() holds.
  bool up = false;
};
hipError_t conv3d(hipStream_t s, const ConvArgs& a);
// whether conv3d can read its input upsampled (the halo kernel's shapes)
bool conv3d_upsample_ok(int T, int H, int W, int Cin, int Cout);
// In place on [P][C] (bf16, or fp16 with h16): RMS norm over C (gain g bf16
// [C]) then SiLU.
hipError_t norm_silu(hipStream_t s, void* x, const void* g, int64_t P, int C, float eps, bool h16 = false);
// RMS norm + SiLU as above, then 2 x 2 (x 2 in time with temporal) average
// pooling: x [T][H][W][C] -> y [T'][H/2][W/2][C] (T' = T / 2 with temporal).
hipError_t norm_silu_pool(hipStream_t s, const void* x, const void* g, void* y, int T, int H, int W, int C,
                          bool temporal, float eps, bool h16);
// bf16 channels-last resampling: mode 0 pool 2x2, 1 pool 2x2x2, 2 nearest
// upsample 2x2, 3 nearest upsample 2x2x2; (T, H, W) is the input's shape.
hipError_t resample(hipStream_t s, const void* x, void* y, int T, int H, int W, int C, int mode, bool h16 = false);
// fp32 [T][C][H*W] -> bf16 (fp16 with h16) [T][H*W][Cp], channels C .. Cp-1 zero.
hipError_t to_channels_last(hipStream_t s, const float* x, void* y, int T, int C, int HW, int Cp, bool h16 = false);
// bf16 -> fp16 elementwise
hipError_t cast_to_h16(hipStream_t s, const void* x, void* y, int64_t n);

}  // namespace sdk
