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
