/*
 * sd_kernels.h -- single-kernel entry points of libsdstream.
 *
 * The same kernels that sd_stream_step() enqueues, callable one at a time so
 * that each step of the path can be checked against the CPU oracle and timed
 * at full size.  Pointers are device pointers owned by the caller; every call
 * is asynchronous on the given hipStream_t (NULL = default stream); arguments
 * are validated before any HIP call and a failed check returns SD_ERR_ARG or
 * SD_ERR_SHAPE without launching anything.
 */
#ifndef SD_KERNELS_H
#define SD_KERNELS_H

#include "sd_stream.h"

#ifdef __cplusplus
extern "C" {
#endif

/* C[m][n] = sum_k A[m][k] W[n][k] + bias[n], fp32 out.  A [M][K], W [N][K] of
 * dtype (bf16 as uint16); bias may be NULL.  K must be a multiple of 8.
 * The dense contraction of every linear layer of the denoiser. */
sd_status sd_k_gemm(int32_t dtype, const void* A, const void* W, const void* bias, float* C, int32_t M, int32_t N,
                    int32_t K, void* stream);

/* C[m][n] += sum_k A[m][k] W[n][k] + bias[n]: the update that closes the
 * attention and FFN sub-layers of a denoiser block, adding the projected
 * output to the fp32 residual stream.  Operand rules as sd_k_gemm; C is read
 * and written in place; C must not alias A, W or bias. */
sd_status sd_k_gemm_resid(int32_t dtype, const void* A, const void* W, const void* bias, float* C, int32_t M,
                          int32_t N, int32_t K, void* stream);

/* Epilogue modes of the denoiser's bf16 GEMMs: each fuses the step that
 * follows a linear layer of a DiT block (StreamDiffusionV2 notes, 实现细节:
 * the Wan-shaped video DiT; the block layout is the reading written in the
 * oracle's denoiser).  C[m][n] = sum_k A[m][k] W[n][k] + bias[n], then
 *   SD_EPI_STORE      out[m][n] = bf16(C)
 *   SD_EPI_GELU       out[m][n] = bf16(GELU(C))            (FFN first layer)
 *   SD_EPI_GATE_RESID resid[m][n] += gate[m/L][n] * C      (attention out / FFN out)
 *                     with gate[r][n] = mod[r*six_d + gate_off + n] + blk[gate_off + n]
 *   SD_EPI_RESID      resid[m][n] += C                     (cross-attention out)
 *   SD_EPI_PATCH      resid[m][n] = C                      (patch embedding)
 *   SD_EPI_QKV        N = 3*H*hd: q | k | v per token, RoPE on q and k when
 *                     rope != 0, q to [rows][H][L][hd], k to
 *                     [H][krows][kstride][hd], v transposed to
 *                     [H][hd][krows][kstride] (row r = m / L, token t = m % L)
 *   SD_EPI_HEAD       eps[r] (fp32 [T][C][Hl][Wl]) = unpatchify(C) of row r
 *   SD_EPI_F32        out[m][n] = C in fp32 */
enum { SD_EPI_STORE = 0, SD_EPI_GELU = 1, SD_EPI_GATE_RESID = 2, SD_EPI_RESID = 3, SD_EPI_PATCH = 4,
       SD_EPI_QKV = 5, SD_EPI_HEAD = 6, SD_EPI_F32 = 8 };

typedef struct {
  int32_t mode;                /* SD_EPI_* */
  const void* bias;            /* bf16 [N]; NULL = 0 (row-major modes only) */
  void* out;                   /* STORE / GELU: bf16 [M][ldo]; F32: fp32 [M][ldo] */
  int32_t ldo;
  float* resid;                /* GATE_RESID / RESID / PATCH: fp32 [M][N] */
  const float* mod;            /* GATE_RESID: fp32 [M/L][six_d] */
  const void* blk;             /* GATE_RESID: bf16 [six_d] */
  int32_t gate_off, six_d;
  int32_t L;                   /* tokens per row; M must be a multiple of L for QKV and HEAD */
  void* q;                     /* QKV destinations (bf16) */
  void* k;
  void* vt;
  int32_t kstride, krows;      /* k / vt token capacity per (head, row) and rows (krows >= M/L) */
  int32_t H, hd;               /* heads and head dim (QKV) */
  int32_t rope;                /* QKV: rotate q and k by 3D RoPE */
  int32_t Hp, Wp;              /* token grid of one latent frame (QKV with RoPE, HEAD) */
  const void* rope_table;      /* device copy of the sd_k_rope_tables() table */
  int32_t rope_positions;      /* temporal positions the table holds */
  int32_t t0[SD_MAX_ROWS];     /* temporal RoPE base of each row */
  float* eps;                  /* HEAD: fp32 [M/L][T][C][Hl][Wl] */
  int32_t C, Hl, Wl, p, T;     /* HEAD: latent geometry and patch (Hl = Hp*p, Wl = Wp*p, L = T*Hp*Wp) */
  int32_t f16;                 /* A and W are IEEE fp16 (F32 and RESID only; bias stays bf16) */
  void* workspace;             /* optional device scratch (256-byte aligned): with M <= 256 the
                                  product is split over K into fp32 partials held here */
  size_t workspace_bytes;
  const void* wpack;           /* optional: W rearranged by sd_k_pack_weight(); with M <= 256 and a
                                  workspace the product reads W from here (NULL: from W) */
  void* ln_out;                /* optional, GATE_RESID / RESID of a bf16 product: after the update,
                                  the LayerNorm of each residual row as sd_k_ln_mod() computes it
                                  (form ln_form, modulation ln_mod / ln_blk at ln_shift_off /
                                  ln_scale_off of ln_six_d, row r = m / L), written here; on the
                                  few-row path the reduction pass does it in the same launch
                                  (N a multiple of 256, at most 2048), otherwise a LayerNorm pass
                                  follows.  NULL: none. */
  const float* ln_mod;
  const void* ln_blk;
  int32_t ln_shift_off, ln_scale_off, ln_six_d, ln_form;
  void* sm_out;                /* optional, F32 without bias: fp16 [M][N] softmax over each of the
                                  sm_heads groups of sm_cp (<= 128) columns of C + sm_bias (fp32
                                  [N]), N = sm_heads * sm_cp (the folded cross-attention's
                                  probabilities); on the few-row path the reduction pass writes it
                                  and out is not written, otherwise C goes to out (ldo = N, else
                                  SD_ERR_SHAPE) and a softmax pass follows.  NULL: none. */
  const float* sm_bias;
  int32_t sm_heads, sm_cp;
} sd_gemm_epi;

/* One bf16 GEMM with the epilogue e->mode, on the kernels and launch
 * configuration sd_stream_step() uses for the same (M, N, K).  A [M][K],
 * W [N][K] bf16, K a multiple of 8.  Destinations must not alias operands. */
sd_status sd_k_gemm_epi(const void* A, const void* W, int32_t M, int32_t N, int32_t K, const sd_gemm_epi* e,
                        void* stream);

/* W [N][K] (bf16 or fp16, K a multiple of 64) rearranged for the few-row
 * product of sd_k_gemm_epi (sd_gemm_epi.wpack): 16-byte chunk
 * (nb, kt, kk, lane), nb = 0 .. ceil(N/32)-1, kt = 0 .. K/64-1, kk = 0 .. 3,
 * lane = 0 .. 63, holds W[32 nb + lane % 32][64 kt + 16 kk + 8 (lane / 32) .. + 7],
 * rows past N zero, so that each 32 x 16 matrix-core operand of a wave is one
 * contiguous 1 KB load.  Below the batch knee the product is bound by reading
 * W (StreamDiffusionV2 summary, SLO-aware batching scheduler: latency model);
 * sd_stream_create() keeps such a copy of the block weights when every forward
 * has at most 256 tokens.  out: device, sd_k_pack_weight_bytes() bytes,
 * 16-byte aligned, not overlapping W.  Enqueued on stream. */
size_t sd_k_pack_weight_bytes(int32_t N, int32_t K);
sd_status sd_k_pack_weight(const void* W, int32_t N, int32_t K, void* out, void* stream);

/* Elements (float pairs) of the 3D RoPE table for head dim hd: the temporal
 * section (positions x dt/2), then height (Hp x dh/2), then width (Wp x dw/2),
 * with dh = dw = 2*floor(hd/6) and dt = hd - 2*dh (StreamDiffusionV2 summary,
 * adaptive sink and RoPE refresh: positions restart below a threshold, so the
 * temporal section has a fixed length). */
size_t sd_k_rope_table_pairs(int32_t hd, int32_t positions, int32_t Hp, int32_t Wp);
/* Fill host memory `out` (2 * sd_k_rope_table_pairs() floats) with
 * (cos, sin) of pos * base^(-2j/width) for every section; the same table
 * sd_stream_create() builds.  Host only, no HIP call. */
sd_status sd_k_rope_tables(int32_t hd, int32_t positions, int32_t Hp, int32_t Wp, double base, float* out);

/* LayerNorm over d (no affine, population variance, eps) of fp32 x [M][d],
 * then x * (1 + scale) + shift with scale / shift = mod[r*six_d + off + c] +
 * blk[off + c], r = m / L (mod NULL: no modulation; blk NULL: 0).  d a
 * multiple of 4, at most 5120.  The adaLN-modulated normalisation in front of
 * a block's attention and MLP.  Output by form:
 *   SD_LN_PLAIN  dtype (bf16 or fp32) [M][d]
 *   SD_LN_F16    fp16 [M][d], no modulation (the cross-attention input)
 *   SD_LN_SPLIT  bf16 [M][2d]: hi = bf16(y) in [0, d), lo = bf16(y - hi) in
 *                [d, 2d) (the head's input, read against doubled weights) */
enum { SD_LN_PLAIN = 0, SD_LN_F16 = 1, SD_LN_SPLIT = 2 };
sd_status sd_k_ln_mod(int32_t dtype, const float* x, void* out, int32_t M, int32_t d, int32_t L, const float* mod,
                      const void* blk, int32_t shift_off, int32_t scale_off, int32_t six_d, int32_t form,
                      void* stream);

/* One causal 3x3x3 convolution of the Stream-VAE (StreamDiffusionV2 summary,
 * Stream-VAE: features cached inside every 3D convolution), bf16 channels-last:
 * x [T][H][W][Cin], cache [2][H][W][Cin] (the two input frames before the
 * chunk; NULL = zeros), w [Cout][3][3][3][Cin], bias [Cout] (NULL = 0);
 * y[t][i][j][o] = bias[o] + sum w[o][dt][dy][dx][c] x'[t+dt-2][i+dy-1][j+dx-1][c]
 * with x' = [cache | x] in time and zero outside the frame.  Cin a multiple of
 * 8, Cout a multiple of 4 (y bf16 [T][H][W][Cout]) or, with y_f32_cf != NULL
 * and Cout <= 16, fp32 channels-first [T][Cout][H][W] to y_f32_cf instead. */
sd_status sd_k_conv3d(const void* x, const void* cache, const void* w, const void* bias, void* y, float* y_f32_cf,
                      int32_t T, int32_t H, int32_t W, int32_t Cin, int32_t Cout, void* stream);

/* The same convolution reading its input upsampled 2x2 (nearest): x bf16
 * [T][H/2][W/2][Cin] and cache [2][H/2][W/2][Cin] stand for
 * x'[t][i][j] = x[t][i/2][j/2] at the output size H x W, as the Stream-VAE
 * decoder's upsampling layers use it (the upsampled tensor is never
 * written).  y bf16 [T][H][W][Cout].  Only the shapes of the halo kernel:
 * T = 4, H and W even, Cin a multiple of 32, Cout of 64, at least 256
 * output tiles of 4 x 8 x 16 positions x 64 or 128 channels; else
 * SD_ERR_SHAPE. */
sd_status sd_k_conv3d_up2(const void* x, const void* cache, const void* w, const void* bias, void* y, int32_t T,
                          int32_t H, int32_t W, int32_t Cin, int32_t Cout, void* stream);

/* One key segment of an attention call.  K is [cap][hd] per (row, head), V is
 * stored transposed [hd][cap]; a head starts head_stride elements after the
 * previous one and a query row row_stride elements after the previous one
 * (0 = shared by all rows).  Valid tokens are positions start .. start+count-1,
 * taken modulo cap when wrap != 0 (the rolling window).  For bf16, start, count
 * (when wrap != 0) and cap must be multiples of 8 and storage between count and
 * the next multiple of 8 must hold finite values. */
typedef struct {
  const void* k;
  const void* vt;
  int64_t k_head_stride, vt_head_stride, k_row_stride, vt_row_stride;
  int32_t cap, start, count, wrap;
} sd_kv_segment;

/* O = softmax(Q K^T / sqrt(hd)) V over the concatenation of up to three
 * segments (sink, window, own chunk), per query row r < R and head h < H.
 * q(r,h,t) = q + r*q_row_stride + h*q_head_stride + t*hd; o is token-major
 * [R*L][H*hd].  StreamDiffusionV2 summary: sink-token guided rolling KV cache.
 * nsplit > 1 (bf16 only) splits every query tile's key sequence over nsplit
 * workgroups whose partial results are combined in a second pass; it needs
 * sd_k_attention_workspace_bytes() bytes of device workspace (256-byte
 * aligned), otherwise workspace may be NULL. */
sd_status sd_k_attention(int32_t dtype, const void* q, int64_t q_row_stride, int64_t q_head_stride, void* o,
                         int32_t R, int32_t H, int32_t L, int32_t hd, int32_t nseg, const sd_kv_segment* segs,
                         int32_t nsplit, void* workspace, size_t workspace_bytes, void* stream);
size_t sd_k_attention_workspace_bytes(int32_t R, int32_t H, int32_t L, int32_t hd, int32_t nsplit);

/* sd_k_attention with a split plan: the query tiles of heads
 * 0 .. unsplit_heads-1 each run as one workgroup over the whole key sequence
 * (O written directly), and only heads unsplit_heads .. H-1 are split nsplit
 * ways and combined.  The unsplit workgroups are dispatched first, so the
 * short split pieces fill the compute units they leave free (the plan the
 * stream uses for self-attention when the query tiles outnumber the resident
 * workgroups).  0 <= unsplit_heads <= H, else SD_ERR_ARG; unsplit_heads = 0
 * is sd_k_attention; with nsplit = 1 it is ignored.  Workspace as for
 * sd_k_attention with the same nsplit.  Results per head equal
 * sd_k_attention's with nsplit 1 (unsplit heads) or nsplit (split heads). */
sd_status sd_k_attention_plan(int32_t dtype, const void* q, int64_t q_row_stride, int64_t q_head_stride, void* o,
                              int32_t R, int32_t H, int32_t L, int32_t hd, int32_t nseg, const sd_kv_segment* segs,
                              int32_t nsplit, int32_t unsplit_heads, void* workspace, size_t workspace_bytes,
                              void* stream);

/* The plan the stream picks for H heads of units_per_head query tiles over
 * `tiles` key tiles of 64, at most max_split splits and `concurrent`
 * resident workgroups: a greedy schedule of the workgroups in grid order
 * over the resident slots, the split share charged 4 % for its partials and
 * combine pass.  Host-only (no HIP call).  SD_ERR_ARG on a non-positive
 * argument or a NULL output. */
sd_status sd_k_attention_pick_plan(int32_t H, int32_t units_per_head, int32_t tiles, int32_t max_split,
                                   int32_t concurrent, int32_t* nsplit, int32_t* unsplit_heads);

/* sd_k_attention without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The split partials use a fixed array of
 * SD_ATTENTION_NOALLOC_SCRATCH_BYTES (128 MiB) in the library's code object,
 * one per device, held until the process ends; the call allocates nothing.
 * A split whose sd_k_attention_workspace_bytes() exceeds that size returns
 * SD_ERR_WORKSPACE before any HIP call.  Results equal sd_k_attention's with
 * the same arguments.  Calls that overlap on one device (different streams,
 * threads or processes' kernels in flight together) share the array and
 * race; calls ordered on one stream do not. */
#define SD_ATTENTION_NOALLOC_SCRATCH_BYTES (128u << 20)
sd_status sd_k_attention_noalloc(int32_t dtype, const void* q, int64_t q_row_stride, int64_t q_head_stride, void* o,
                                 int32_t R, int32_t H, int32_t L, int32_t hd, int32_t nseg,
                                 const sd_kv_segment* segs, int32_t nsplit, void* stream);

/* Exact int64 sums (sum a*b, sum a*a, sum b*b) of two frames: kind SD_SSF_U8
 * (uint8) or SD_SSF_LATENT (fp32 quantised to rint(x*2^12) clamped to +-2^20).
 * out_dev is a device int64[3].  StreamDiffusion paper notes, section 3 (SSF). */
sd_status sd_k_ssf_sums(int32_t kind, const void* a, const void* b, int64_t n, int64_t* out_dev, void* stream);

/* Exact int64 sum of squared differences of consecutive quantised frames:
 * pair 0 = (prev_last, cur[0]) (written 0 when prev_last is NULL), pair t =
 * (cur[t-1], cur[t]).  cur is fp32 [T][n].  StreamDiffusionV2 summary,
 * motion-aware noise scheduler. */
sd_status sd_k_motion_sums(const float* cur, const float* prev_last, int32_t T, int64_t n, int64_t* out_dev,
                           void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SD_KERNELS_H */
