// sd_k_* : single-kernel entry points (see include/sd_kernels.h).
#include <cmath>
#include <cstring>

#include "../../include/sd_kernels.h"
#include "kernels.h"

extern "C" {

static sd_status gemm_call(int32_t dtype, const void* A, const void* W, const void* bias, float* C, int32_t M,
                           int32_t N, int32_t K, void* stream, int mode) {
  if (dtype != SD_DTYPE_F32 && dtype != SD_DTYPE_BF16) return SD_ERR_ARG;
  if (!A || !W || !C || M < 0 || N < 0 || K < 1) return SD_ERR_ARG;
  if (K % 8) return SD_ERR_SHAPE;
  Epi E;
  std::memset(&E, 0, sizeof(E));
  E.mode = mode;
  E.bias = bias;
  E.out = C;
  E.resid = C;
  E.ldo = N;
  E.L = 1;
  return sdk::gemm((hipStream_t)stream, dtype == SD_DTYPE_BF16, A, W, M, N, K, E) == hipSuccess ? SD_OK
                                                                                             : SD_ERR_HIP;
}

sd_status sd_k_gemm(int32_t dtype, const void* A, const void* W, const void* bias, float* C, int32_t M, int32_t N,
                    int32_t K, void* stream) {
  return gemm_call(dtype, A, W, bias, C, M, N, K, stream, EPI_F32);
}

sd_status sd_k_gemm_resid(int32_t dtype, const void* A, const void* W, const void* bias, float* C, int32_t M,
                          int32_t N, int32_t K, void* stream) {
  return gemm_call(dtype, A, W, bias, C, M, N, K, stream, EPI_RESID);
}

static size_t part_o_bytes(int32_t R, int32_t H, int32_t L, int32_t hd, int32_t nsplit) {
  return (((size_t)nsplit * R * L * H * hd * 2) + 255) & ~(size_t)255;
}

size_t sd_k_attention_workspace_bytes(int32_t R, int32_t H, int32_t L, int32_t hd, int32_t nsplit) {
  if (R < 1 || H < 1 || L < 1 || hd < 1 || nsplit < 1) return 0;
  if (nsplit == 1) return 0;
  return part_o_bytes(R, H, L, hd, nsplit) + (size_t)nsplit * R * H * L * 8;
}

sd_status sd_k_attention(int32_t dtype, const void* q, int64_t q_row_stride, int64_t q_head_stride, void* o,
                         int32_t R, int32_t H, int32_t L, int32_t hd, int32_t nseg, const sd_kv_segment* segs,
                         int32_t nsplit, void* workspace, size_t workspace_bytes, void* stream) {
  if (nsplit < 1 || nsplit > 64) return SD_ERR_ARG;
  if (nsplit > 1) {
    if (dtype != SD_DTYPE_BF16 || !workspace || ((uintptr_t)workspace & 255)) return SD_ERR_ARG;
    if (workspace_bytes < sd_k_attention_workspace_bytes(R, H, L, hd, nsplit)) return SD_ERR_WORKSPACE;
  }
  if (dtype != SD_DTYPE_F32 && dtype != SD_DTYPE_BF16) return SD_ERR_ARG;
  if (!q || !o || !segs || nseg < 1 || nseg > 3 || R < 0 || H < 1 || L < 0) return SD_ERR_ARG;
  const bool bf = dtype == SD_DTYPE_BF16;
  if (bf && hd != 32 && hd != 64 && hd != 128) return SD_ERR_SHAPE;
  if (!bf && hd != 16 && hd != 32 && hd != 64 && hd != 128) return SD_ERR_SHAPE;
  sdk::AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.q_rs = q_row_stride;
  a.q_hs = q_head_stride;
  a.o = o;
  a.R = R;
  a.H = H;
  a.L = L;
  a.hd = hd;
  a.d = H * hd;
  a.nseg = nseg;
  a.scale = 1.0f / std::sqrt((float)hd);
  for (int i = 0; i < nseg; ++i) {
    const sd_kv_segment& g = segs[i];
    if (g.count < 0 || g.cap < 0 || g.start < 0) return SD_ERR_ARG;
    if (g.count > 0 && (!g.k || !g.vt)) return SD_ERR_ARG;
    if (g.count > 0 && g.cap < 1) return SD_ERR_ARG;
    if (!g.wrap && g.start + g.count > g.cap) return SD_ERR_SHAPE;
    if (g.wrap && g.count > g.cap) return SD_ERR_SHAPE;
    if (bf && (g.cap % 8 || g.start % 8 || (g.wrap && g.count % 8))) return SD_ERR_SHAPE;
    if (bf && !g.wrap && g.start + ((g.count + 7) & ~7) > g.cap) return SD_ERR_SHAPE;
    sdk::KvSeg& s = a.seg[i];
    s.k = g.k;
    s.vt = g.vt;
    s.k_hs = g.k_head_stride;
    s.vt_hs = g.vt_head_stride;
    s.k_rs = g.k_row_stride;
    s.vt_rs = g.vt_row_stride;
    s.cap = g.cap;
    s.start = g.start;
    s.count = g.count;
    s.wrap = g.wrap;
  }
  a.nsplit = nsplit;
  if (nsplit > 1) {
    a.part_o = (bf16*)workspace;
    a.part_ml = (float2*)((char*)workspace + part_o_bytes(R, H, L, hd, nsplit));
    a.part_so = (long long)R * L * H * hd;
    a.part_sml = (long long)R * H * L;
  }
  return sdk::attention((hipStream_t)stream, bf, a) == hipSuccess ? SD_OK : SD_ERR_HIP;
}

sd_status sd_k_conv3d(const void* x, const void* cache, const void* w, const void* bias, void* y, float* y_f32_cf,
                      int32_t T, int32_t H, int32_t W, int32_t Cin, int32_t Cout, void* stream) {
  if (!x || !w || T < 1 || H < 1 || W < 1 || Cin < 8 || Cout < 1) return SD_ERR_ARG;
  if (Cin % 8) return SD_ERR_SHAPE;
  if ((int64_t)T * H * W * (Cin > Cout ? Cin : Cout) >= (1ll << 31)) return SD_ERR_SHAPE;
  sdk::ConvArgs a;
  a.x = (const bf16*)x;
  a.cache = (const bf16*)cache;
  a.w = (const bf16*)w;
  a.b = (const bf16*)bias;
  a.y = (bf16*)y;
  a.ycf = y_f32_cf;
  a.T = T;
  a.H = H;
  a.W = W;
  a.Cin = Cin;
  a.Cout = Cout;
  if (y_f32_cf) {
    if (Cout > 16) return SD_ERR_SHAPE;
    a.y = nullptr;
    return sdk::conv3d((hipStream_t)stream, a) == hipSuccess ? SD_OK : SD_ERR_HIP;
  }
  if (!y) return SD_ERR_ARG;
  if (Cout % 4) return SD_ERR_SHAPE;
  return sdk::conv3d((hipStream_t)stream, a) == hipSuccess ? SD_OK : SD_ERR_HIP;
}

sd_status sd_k_ssf_sums(int32_t kind, const void* a, const void* b, int64_t n, int64_t* out_dev, void* stream) {
  if ((kind != SD_SSF_U8 && kind != SD_SSF_LATENT) || !a || !b || !out_dev || n < 0) return SD_ERR_ARG;
  return sdk::ssf_sums((hipStream_t)stream, kind, a, b, n, (long long*)out_dev) == hipSuccess ? SD_OK : SD_ERR_HIP;
}

sd_status sd_k_motion_sums(const float* cur, const float* prev_last, int32_t T, int64_t n, int64_t* out_dev,
                           void* stream) {
  if (!cur || !out_dev || T < 1 || T > 64 || n < 1) return SD_ERR_ARG;
  return sdk::motion_sums((hipStream_t)stream, cur, prev_last, T, n, (long long*)out_dev) == hipSuccess ? SD_OK
                                                                                                       : SD_ERR_HIP;
}

}  // extern "C"
