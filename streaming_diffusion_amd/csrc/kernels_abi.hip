// sd_k_* : single-kernel entry points (see include/sd_kernels.h).
#include <cmath>
#include <cstring>
#include <mutex>

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

static void rope_split(int hd, int* dt, int* dh, int* dw) {
  *dh = 2 * (hd / 6);
  *dw = *dh;
  *dt = hd - 2 * *dh;
}

static size_t pairs_of(int npos, int width) { return (size_t)npos * (size_t)(width / 2 > 1 ? width / 2 : 1); }

size_t sd_k_rope_table_pairs(int32_t hd, int32_t positions, int32_t Hp, int32_t Wp) {
  if (hd < 2 || positions < 1 || Hp < 1 || Wp < 1) return 0;
  int dt, dh, dw;
  rope_split(hd, &dt, &dh, &dw);
  return pairs_of(positions, dt) + pairs_of(Hp, dh) + pairs_of(Wp, dw);
}

sd_status sd_k_rope_tables(int32_t hd, int32_t positions, int32_t Hp, int32_t Wp, double base, float* out) {
  if (!out || hd < 2 || (hd & 1) || positions < 1 || Hp < 1 || Wp < 1 || !(base > 1.0)) return SD_ERR_ARG;
  int dt, dh, dw;
  rope_split(hd, &dt, &dh, &dw);
  float2* o = (float2*)out;
  sdk::rope_table_fill(o, positions, dt, base);
  o += pairs_of(positions, dt);
  sdk::rope_table_fill(o, Hp, dh, base);
  o += pairs_of(Hp, dh);
  sdk::rope_table_fill(o, Wp, dw, base);
  return SD_OK;
}

sd_status sd_k_gemm_epi(const void* A, const void* W, int32_t M, int32_t N, int32_t K, const sd_gemm_epi* e,
                        void* stream) {
  if (!A || !W || !e || M < 0 || N < 1 || K < 8) return SD_ERR_ARG;
  if (K % 8) return SD_ERR_SHAPE;
  Epi E;
  std::memset(&E, 0, sizeof(E));
  E.mode = e->mode;
  E.bias = e->bias;
  E.L = e->L > 0 ? e->L : 1;
  E.ldo = N;
  if (e->f16 && e->mode != SD_EPI_F32 && e->mode != SD_EPI_RESID) return SD_ERR_ARG;
  if (e->workspace && ((uintptr_t)e->workspace & 255)) return SD_ERR_ARG;
  switch (e->mode) {
    case SD_EPI_STORE:
    case SD_EPI_GELU:
    case SD_EPI_F32:
      if (!e->out || e->ldo < N) return SD_ERR_ARG;
      E.out = e->out;
      E.ldo = e->ldo;
      break;
    case SD_EPI_GATE_RESID:
      if (!e->resid || !e->mod || !e->blk || e->L < 1) return SD_ERR_ARG;
      if (e->gate_off < 0 || e->gate_off % 8 || e->six_d % 8 || e->gate_off + N > e->six_d) return SD_ERR_SHAPE;
      E.resid = e->resid;
      E.mod = e->mod;
      E.blk = e->blk;
      E.gate_off = e->gate_off;
      E.six_d = e->six_d;
      break;
    case SD_EPI_RESID:
    case SD_EPI_PATCH:
      if (!e->resid) return SD_ERR_ARG;
      E.resid = e->resid;
      break;
    case SD_EPI_QKV: {
      if (!e->q || !e->k || !e->vt || !e->bias || e->L < 1 || e->H < 1 || e->hd < 8) return SD_ERR_ARG;
      const int rows = M / e->L;
      if (e->hd % 8 || N != 3 * e->H * e->hd || M % e->L || e->L % 8 || rows > SD_MAX_ROWS) return SD_ERR_SHAPE;
      if (e->krows < rows || e->kstride < e->L || e->kstride % 8) return SD_ERR_SHAPE;
      E.q = e->q;
      E.k = e->k;
      E.vt = e->vt;
      E.kstride = e->kstride;
      E.krows = e->krows;
      E.H = e->H;
      E.hd = e->hd;
      E.d = e->H * e->hd;
      E.rope = e->rope ? 1 : 0;
      if (E.rope) {
        if (!e->rope_table || e->Hp < 1 || e->Wp < 1 || e->rope_positions < 1) return SD_ERR_ARG;
        const int hw = e->Hp * e->Wp;
        if (e->L % hw) return SD_ERR_SHAPE;
        for (int r = 0; r < rows; ++r)
          if (e->t0[r] < 0 || e->t0[r] + e->L / hw > e->rope_positions) return SD_ERR_SHAPE;
        int dt, dh, dw;
        rope_split(e->hd, &dt, &dh, &dw);
        E.Hp = e->Hp;
        E.Wp = e->Wp;
        E.dt = dt;
        E.dh = dh;
        E.rope_t = (const float2*)e->rope_table;
        E.rope_h = E.rope_t + pairs_of(e->rope_positions, dt);
        E.rope_w = E.rope_h + pairs_of(e->Hp, dh);
        for (int r = 0; r < rows; ++r) E.t0[r] = e->t0[r];
      }
      break;
    }
    case SD_EPI_HEAD: {
      if (!e->eps || !e->bias || e->L < 1 || e->C < 1 || e->p < 1 || e->T < 1 || e->Hp < 1 || e->Wp < 1)
        return SD_ERR_ARG;
      if (N != e->p * e->p * e->C || e->Hl != e->Hp * e->p || e->Wl != e->Wp * e->p ||
          e->L != e->T * e->Hp * e->Wp || M % e->L)
        return SD_ERR_SHAPE;
      E.eps = e->eps;
      E.C = e->C;
      E.Hl = e->Hl;
      E.Wl = e->Wl;
      E.p = e->p;
      E.T = e->T;
      E.Hp = e->Hp;
      E.Wp = e->Wp;
      break;
    }
    default:
      return SD_ERR_ARG;
  }
  if (e->workspace && e->workspace_bytes >= 4) {
    E.part = (float*)e->workspace;
    E.part_cap = (int64_t)(e->workspace_bytes / 4);
  }
  if (e->wpack) {
    if ((uintptr_t)e->wpack & 15) return SD_ERR_ARG;
    if (K % 64) return SD_ERR_SHAPE;
    E.wpack = e->wpack;
  }
  if (e->ln_out) {
    if (e->mode != SD_EPI_GATE_RESID && e->mode != SD_EPI_RESID) return SD_ERR_ARG;
    if (e->ln_form != SD_LN_PLAIN && e->ln_form != SD_LN_F16 && e->ln_form != SD_LN_SPLIT) return SD_ERR_ARG;
    if (e->ln_form == SD_LN_F16 && e->ln_mod) return SD_ERR_ARG;
    if (N % 4 || N > 5120) return SD_ERR_SHAPE;
    if (e->ln_mod && (e->ln_shift_off < 0 || e->ln_scale_off < 0 || e->ln_shift_off % 4 || e->ln_scale_off % 4 ||
                      e->ln_six_d % 4 || e->ln_shift_off + N > e->ln_six_d || e->ln_scale_off + N > e->ln_six_d))
      return SD_ERR_SHAPE;
    E.ln_out = e->ln_out;
    E.ln_mod = e->ln_mod;
    E.ln_blk = e->ln_mod ? e->ln_blk : nullptr;
    E.ln_shift = e->ln_shift_off;
    E.ln_scale = e->ln_scale_off;
    E.ln_six = e->ln_mod ? e->ln_six_d : 4;
    E.ln_form = e->ln_form;
    E.ln_eps = 1e-6f;
  }
  if (e->sm_out) {
    if (e->mode != SD_EPI_F32 || e->bias || !e->sm_bias) return SD_ERR_ARG;
    if (e->sm_cp < 1 || e->sm_cp > 128 || e->sm_heads < 1 || e->sm_heads * e->sm_cp != N) return SD_ERR_SHAPE;
    E.sm_out = (f16*)e->sm_out;
    E.sm_bias = e->sm_bias;
    E.sm_heads = e->sm_heads;
    E.sm_cp = e->sm_cp;
  }
  const bool sm_fused = E.sm_out && sdk::gemm_fuses_softmax(M, N, K, E);
  if (E.sm_out && !sm_fused) {
    if (E.ldo != N) return SD_ERR_SHAPE;          // the softmax pass reads C densely
    E.sm_out = nullptr;
  }
  const bool fused = E.ln_out && sdk::gemm_fuses_ln(M, N, K, E);
  hipError_t r = e->f16 ? sdk::gemm_mfma_f16((hipStream_t)stream, A, W, M, N, K, E)
                        : sdk::gemm_mfma((hipStream_t)stream, A, W, M, N, K, E);
  if (r == hipSuccess && e->sm_out && !sm_fused) {
    r = sdk::ctx_softmax((hipStream_t)stream, (const float*)E.out, e->sm_bias, (f16*)e->sm_out, M, e->sm_heads,
                         e->sm_cp);
  }
  if (r == hipSuccess && E.ln_out && !fused)
    r = sdk::ln_mod((hipStream_t)stream, true, E.resid, E.ln_out, M, N, E.L, E.ln_mod, E.ln_blk, E.ln_shift,
                    E.ln_scale, E.ln_six, E.ln_eps, E.ln_form);
  return r == hipSuccess ? SD_OK : SD_ERR_HIP;
}

size_t sd_k_pack_weight_bytes(int32_t N, int32_t K) {
  if (N < 1 || K < 64 || K % 64) return 0;
  return sdk::pack_weight_bytes(N, K);
}

sd_status sd_k_pack_weight(const void* W, int32_t N, int32_t K, void* out, void* stream) {
  if (!W || !out || N < 1 || K < 1) return SD_ERR_ARG;
  if (K % 64) return SD_ERR_SHAPE;
  if ((uintptr_t)out & 15) return SD_ERR_ARG;
  return sdk::pack_weight((hipStream_t)stream, W, N, K, out) == hipSuccess ? SD_OK : SD_ERR_HIP;
}

sd_status sd_k_ln_mod(int32_t dtype, const float* x, void* out, int32_t M, int32_t d, int32_t L, const float* mod,
                      const void* blk, int32_t shift_off, int32_t scale_off, int32_t six_d, int32_t form,
                      void* stream) {
  if (dtype != SD_DTYPE_F32 && dtype != SD_DTYPE_BF16) return SD_ERR_ARG;
  if (form != SD_LN_PLAIN && form != SD_LN_F16 && form != SD_LN_SPLIT) return SD_ERR_ARG;
  if (form != SD_LN_PLAIN && dtype != SD_DTYPE_BF16) return SD_ERR_ARG;
  if (form == SD_LN_F16 && mod) return SD_ERR_ARG;
  if (!x || !out || M < 0 || d < 4 || L < 1) return SD_ERR_ARG;
  if (d % 4 || d > 5120) return SD_ERR_SHAPE;
  if (mod && (shift_off < 0 || scale_off < 0 || shift_off % 4 || scale_off % 4 || six_d % 4 ||
              shift_off + d > six_d || scale_off + d > six_d))
    return SD_ERR_SHAPE;
  return sdk::ln_mod((hipStream_t)stream, dtype == SD_DTYPE_BF16, x, out, M, d, L, mod, mod ? blk : nullptr,
                     shift_off, scale_off, mod ? six_d : 4, 1e-6f, form) == hipSuccess
             ? SD_OK
             : SD_ERR_HIP;
}

static size_t part_o_bytes(int32_t R, int32_t H, int32_t L, int32_t hd, int32_t nsplit) {
  return (((size_t)nsplit * R * L * H * hd * 2) + 255) & ~(size_t)255;
}

size_t sd_k_attention_workspace_bytes(int32_t R, int32_t H, int32_t L, int32_t hd, int32_t nsplit) {
  if (R < 1 || H < 1 || L < 1 || hd < 1 || nsplit < 1) return 0;
  if (nsplit == 1) return 0;
  return part_o_bytes(R, H, L, hd, nsplit) + (size_t)nsplit * R * H * L * 8;
}

// Validation and argument packing shared by the attention entry points; no
// HIP call.  The split partials are attached by the caller.
static sd_status attention_prepare(int32_t dtype, const void* q, int64_t q_row_stride, int64_t q_head_stride,
                                   void* o, int32_t R, int32_t H, int32_t L, int32_t hd, int32_t nseg,
                                   const sd_kv_segment* segs, int32_t nsplit, sdk::AttnArgs* out, bool* bf_out) {
  if (nsplit < 1 || nsplit > 64) return SD_ERR_ARG;
  if (nsplit > 1 && dtype != SD_DTYPE_BF16) return SD_ERR_ARG;
  if (dtype != SD_DTYPE_F32 && dtype != SD_DTYPE_BF16) return SD_ERR_ARG;
  if (!q || !o || !segs || nseg < 1 || nseg > 3 || R < 0 || H < 1 || L < 0) return SD_ERR_ARG;
  const bool bf = dtype == SD_DTYPE_BF16;
  if (bf && hd != 32 && hd != 64 && hd != 128) return SD_ERR_SHAPE;
  if (!bf && hd != 16 && hd != 32 && hd != 64 && hd != 128) return SD_ERR_SHAPE;
  sdk::AttnArgs& a = *out;
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
    sdk::KvSeg& sg = a.seg[i];
    sg.k = g.k;
    sg.vt = g.vt;
    sg.k_hs = g.k_head_stride;
    sg.vt_hs = g.vt_head_stride;
    sg.k_rs = g.k_row_stride;
    sg.vt_rs = g.vt_row_stride;
    sg.cap = g.cap;
    sg.start = g.start;
    sg.count = g.count;
    sg.wrap = g.wrap;
  }
  a.nsplit = nsplit;
  *bf_out = bf;
  return SD_OK;
}

static void attach_partials(sdk::AttnArgs& a, void* workspace) {
  if (a.nsplit < 2) return;
  a.part_o = (bf16*)workspace;
  a.part_ml = (float2*)((char*)workspace + part_o_bytes(a.R, a.H, a.L, a.hd, a.nsplit));
  a.part_so = (long long)a.R * a.L * a.H * a.hd;
  a.part_sml = (long long)a.R * a.H * a.L;
}

sd_status sd_k_attention(int32_t dtype, const void* q, int64_t q_row_stride, int64_t q_head_stride, void* o,
                         int32_t R, int32_t H, int32_t L, int32_t hd, int32_t nseg, const sd_kv_segment* segs,
                         int32_t nsplit, void* workspace, size_t workspace_bytes, void* stream) {
  return sd_k_attention_plan(dtype, q, q_row_stride, q_head_stride, o, R, H, L, hd, nseg, segs, nsplit, 0, workspace,
                             workspace_bytes, stream);
}

sd_status sd_k_attention_plan(int32_t dtype, const void* q, int64_t q_row_stride, int64_t q_head_stride, void* o,
                              int32_t R, int32_t H, int32_t L, int32_t hd, int32_t nseg, const sd_kv_segment* segs,
                              int32_t nsplit, int32_t unsplit_heads, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (nsplit < 1 || nsplit > 64) return SD_ERR_ARG;
  if (unsplit_heads < 0 || unsplit_heads > H) return SD_ERR_ARG;
  if (nsplit > 1) {
    if (dtype != SD_DTYPE_BF16 || !workspace || ((uintptr_t)workspace & 255)) return SD_ERR_ARG;
    if (workspace_bytes < sd_k_attention_workspace_bytes(R, H, L, hd, nsplit)) return SD_ERR_WORKSPACE;
  }
  sdk::AttnArgs a;
  bool bf = false;
  const sd_status st = attention_prepare(dtype, q, q_row_stride, q_head_stride, o, R, H, L, hd, nseg, segs, nsplit,
                                         &a, &bf);
  if (st != SD_OK) return st;
  a.h_full = nsplit > 1 ? unsplit_heads : 0;
  attach_partials(a, workspace);
  return sdk::attention((hipStream_t)stream, bf, a) == hipSuccess ? SD_OK : SD_ERR_HIP;
}

sd_status sd_k_attention_pick_plan(int32_t H, int32_t units_per_head, int32_t tiles, int32_t max_split,
                                   int32_t concurrent, int32_t* nsplit, int32_t* unsplit_heads) {
  if (H < 1 || units_per_head < 1 || tiles < 1 || max_split < 1 || concurrent < 1 || !nsplit || !unsplit_heads)
    return SD_ERR_ARG;
  int ns = 1, hf = 0;
  sdk::attention_pick_plan(H, units_per_head, tiles, max_split, concurrent, &ns, &hf);
  *nsplit = ns;
  *unsplit_heads = hf;
  return SD_OK;
}

// ---------------------------------------------------------------------------
// Allocation-free attention.  The split partials live in `scratch`, a
// fixed-size array in the code object (each device that loads the library
// holds its own copy until the process ends).  Host code never passes the
// array's name to a kernel: that is a host-side stand-in.  The device address
// of each device's copy is looked up once, with that device current, and
// kept per device.  Every split partial is written before the combine reads
// it, so nothing needs clearing between calls.
static __device__ __attribute__((aligned(256))) unsigned char scratch[SD_ATTENTION_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of this device's scratch copy (nullptr on failure)
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

sd_status sd_k_attention_noalloc(int32_t dtype, const void* q, int64_t q_row_stride, int64_t q_head_stride, void* o,
                                 int32_t R, int32_t H, int32_t L, int32_t hd, int32_t nseg,
                                 const sd_kv_segment* segs, int32_t nsplit, void* stream) {
  sdk::AttnArgs a;
  bool bf = false;
  const sd_status st = attention_prepare(dtype, q, q_row_stride, q_head_stride, o, R, H, L, hd, nseg, segs, nsplit,
                                         &a, &bf);
  if (st != SD_OK) return st;
  if (nsplit > 1) {
    if (sd_k_attention_workspace_bytes(R, H, L, hd, nsplit) > (size_t)SD_ATTENTION_NOALLOC_SCRATCH_BYTES)
      return SD_ERR_WORKSPACE;
    void* ws = device_scratch();
    if (!ws) return SD_ERR_HIP;
    attach_partials(a, ws);
  }
  return sdk::attention((hipStream_t)stream, bf, a) == hipSuccess ? SD_OK : SD_ERR_HIP;
}

sd_status sd_k_conv3d(const void* x, const void* cache, const void* w, const void* bias, void* y, float* y_f32_cf,
                      int32_t T, int32_t H, int32_t W, int32_t Cin, int32_t Cout, void* stream) {
  if (!x || !w || T < 1 || H < 1 || W < 1 || Cin < 8 || Cout < 1) return SD_ERR_ARG;
  if (Cin % 8) return SD_ERR_SHAPE;
  if ((int64_t)T * H * W * (Cin > Cout ? Cin : Cout) >= (1ll << 31)) return SD_ERR_SHAPE;
  sdk::ConvArgs a;
  a.h16 = false;
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

sd_status sd_k_conv3d_up2(const void* x, const void* cache, const void* w, const void* bias, void* y, int32_t T,
                          int32_t H, int32_t W, int32_t Cin, int32_t Cout, void* stream) {
  if (!x || !w || !y || T < 1 || H < 1 || W < 1 || Cin < 8 || Cout < 1) return SD_ERR_ARG;
  if ((int64_t)T * H * W * (Cin > Cout ? Cin : Cout) >= (1ll << 31)) return SD_ERR_SHAPE;
  if (!sdk::conv3d_upsample_ok(T, H, W, Cin, Cout)) return SD_ERR_SHAPE;
  sdk::ConvArgs a;
  a.h16 = false;
  a.up = true;
  a.x = (const bf16*)x;
  a.cache = (const bf16*)cache;
  a.w = (const bf16*)w;
  a.b = (const bf16*)bias;
  a.y = (bf16*)y;
  a.ycf = nullptr;
  a.T = T;
  a.H = H;
  a.W = W;
  a.Cin = Cin;
  a.Cout = Cout;
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
