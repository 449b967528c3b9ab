// sd_stream_* : the Stream Batch runtime.  Holds the integer state machine
// (frame store, slots, KV ring pointer and valid count, sink entries, RoPE
// counter, SSF and motion state) and enqueues the kernels of one step.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <deque>
#include <string>
#include <vector>

#include "host_state.h"
#include "kernels.h"
#include "kv_append.h"

using sdk::AttnArgs;
using sdk::KvSeg;

namespace {

// pending chunks accepted before a step must run: at least 4, at least 2 B
int pending_max(int B) { return B * 2 > 4 ? B * 2 : 4; }

struct FrameRec {
  bool used = false;
  int64_t fid = -1;
  int32_t taus[SD_MAX_SLOTS] = {};
  int32_t t0 = 0;
};

}  // namespace

struct sd_stream {
  sd_stream_config cfg;
  sd_weights w;
  hipStream_t st = nullptr;
  std::string err;
  bool bf = false;
  size_t es = 4;  // element size of weights / activations
  // dims
  int L = 0, d = 0, H = 0, hd = 0, F = 0, nb = 0, P = 0, Tn = 0, Hp = 0, Wp = 0;
  int64_t lat = 0, frame_elems = 0;
  int S = 0, S8 = 0, Se = 0, Ment = 0, Wt = 0, ctx8 = 0, Rmax = 0, n = 0, NF = 0;
  int B = 1, pend_max = 4;        // chunks per step, pending-queue capacity
  int Cc = 0;                     // sink-candidate tokens per (block, head) (B > 1 with a sink)
  int dt = 0, dh = 0, dw = 0, rope_pos = 0;
  std::vector<double> a, b;
  // device regions
  float *fx = nullptr, *fx0s = nullptr;
  float* fz = nullptr;          // LCM sampler: per frame record, the n-1 re-noise latents
  void* ssf_ref = nullptr;
  long long* sums = nullptr;      // [0..2] ssf, [4..4+T) motion
  float* mprev = nullptr;
  float *emb = nullptr, *h1 = nullptr, *sc = nullptr, *mod = nullptr, *fmod = nullptr;
  float* resid = nullptr;
  void *xm = nullptr, *q = nullptr, *kown = nullptr, *vtown = nullptr, *ao = nullptr, *hid = nullptr;
  float* eps = nullptr;
  void *ringK = nullptr, *ringVT = nullptr, *sinkK = nullptr, *sinkVT = nullptr;
  // B > 1: the first S_e tokens' K / V^T of each leaving chunk, staged at
  // append time for its sink decision (the ring may already hold later
  // chunks at those positions); [nb][H][Cc][hd] and [nb][H][hd][Cc]
  void *candK = nullptr, *candVT = nullptr;
  void *ctxK = nullptr, *ctxVT = nullptr;
  // bf16: cross-attention runs on folded projections (k_attn.hip): per block
  // and context wq_f [H Cp][d], wo_f [d][H Cp] fp16 and the score bias [H Cp]
  bool fold = false;
  // bf16: the patch embedding and the head see their fp32 inputs as hi + lo
  // bf16 pairs (K doubled); their weights are kept twice side by side,
  // pe2 [d][2P] = [pe_w | pe_w], head2 [P][2d] = [head_w | head_w], copied
  // from the caller's weights at create
  void *pe2 = nullptr, *head2 = nullptr;
  // bf16 with short chunks (L <= 256): fp32 partials of GEMMs split over K
  // when a forward has few rows (kernels.h, Epi::part)
  float* gpart = nullptr;
  int64_t gpart_cap = 0;
  // with short chunks, fragment-ordered copies of the block weights for the
  // few-row product (kernels.h, pack_weight; null where K % 64 != 0): made
  // at create from the caller's weights, the folded cross-attention ones at
  // set_context
  void *wp_qkv = nullptr, *wp_o = nullptr, *wp_f1 = nullptr, *wp_f2 = nullptr, *wp_cq = nullptr, *wp_co = nullptr;
  void *wp_fq = nullptr, *wp_fo = nullptr;
  // the step's dynamic values in device memory: [0] the forward, [1] the
  // clean-latent forward of kv_recompute
  StepDyn* dyn = nullptr;
  // graph replay of the step's forward and update (sd_stream_set_graph): a
  // few instantiated graphs keyed by the launch sequence's static arguments
  struct GraphEntry {
    std::vector<int64_t> key;
    hipGraphExec_t exec = nullptr;
    uint64_t used = 0;
  };
  bool graph_on = false;
  std::vector<GraphEntry> graphs;
  uint64_t graph_clock = 0;
  int64_t graph_captures = 0, graph_replays = 0;
  void *fold_q = nullptr, *fold_o = nullptr;
  float* fold_c = nullptr;
  double *sink_emb = nullptr, *sink_part = nullptr, *sink_sim = nullptr;
  int* sink_flag = nullptr;
  float2 *rope_t = nullptr, *rope_h = nullptr, *rope_w = nullptr;
  // split-KV partials of the self-attention
  int attn_split_max = 1;
  bf16* part_o = nullptr;         // split-KV partial outputs (unnormalised, bf16)
  float2* part_ml = nullptr;
  int cus = 256;                // compute units of the device
  size_t ws_used = 0;
  // host state
  std::vector<FrameRec> frames;
  std::deque<int> pending;
  int slots[SD_MAX_SLOTS * SD_MAX_CHUNKS];   // frame per (slot, lane), slot-major
  sd::Controls ctl;
  int64_t n_pushed = 0, n_steps = 0;
  int kv_ptr = 0, kv_valid = 0, sink_count = 0;
  bool ctx_set = false;
  bool has_ref_frame = false;
  // live kernel timing (HIP events on the stream), per kind
  uint32_t prof_mask = 0;
  struct ProfRec { int kind; int ev; double flops, bytes; };
  std::vector<hipEvent_t> ev_pool;
  int ev_used = 0;
  std::vector<ProfRec> prof_pending;
  sd_kernel_stat prof_acc[SD_PROF_KINDS];
  hipStream_t pst = nullptr;            // stream the profiling events go to (st, or io during a push)
  // IO queue: pushes on io; ev_push marks the last push, rec_ev[f] the end of
  // the step that last read frame record f
  hipStream_t io = nullptr;
  hipEvent_t ev_push = nullptr;
  bool push_pending = false;
  std::vector<hipEvent_t> rec_ev;
  std::vector<char> rec_ev_set;
  ~sd_stream() {
    if (io) (void)hipStreamSynchronize(io);
    if (st) (void)hipStreamSynchronize(st);
    for (GraphEntry& g : graphs)
      if (g.exec) (void)hipGraphExecDestroy(g.exec);
    for (hipEvent_t e : ev_pool) (void)hipEventDestroy(e);
    for (hipEvent_t e : rec_ev) (void)hipEventDestroy(e);
    if (ev_push) (void)hipEventDestroy(ev_push);
  }
};

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Carver {
  char* base;
  size_t off = 0;
  template <typename T>
  T* take(size_t bytes) {
    T* p = base ? (T*)(base + off) : nullptr;
    off += align256(bytes);
    return p;
  }
};

void dims(sd_stream* s) {
  const sd_stream_config& c = s->cfg;
  s->bf = c.dtype == SD_DTYPE_BF16;
  s->es = s->bf ? 2 : 4;
  s->L = (int)sd::tokens_per_chunk(c);
  s->d = c.d_model;
  s->H = c.n_heads;
  s->hd = c.d_model / c.n_heads;
  s->F = c.d_ffn;
  s->nb = c.n_blocks;
  s->P = c.patch * c.patch * c.latent_c;
  s->Tn = c.latent_t;
  s->Hp = c.latent_h / c.patch;
  s->Wp = c.latent_w / c.patch;
  s->lat = sd::latent_elems(c);
  s->frame_elems = (int64_t)c.latent_c * c.latent_h * c.latent_w;
  s->S = c.sink_tokens;
  s->S8 = (c.sink_tokens + 7) & ~7;
  s->Ment = c.sink_tokens > 0 ? c.sink_entries : 0;
  s->Se = c.sink_tokens > 0 ? c.sink_tokens / c.sink_entries : 0;
  s->Wt = c.window_tokens;
  s->ctx8 = (c.ctx_len + 7) & ~7;
  s->Rmax = sd::rows_max(c);
  s->n = c.n_slots;
  s->B = c.chunks_per_step;
  s->pend_max = pending_max(s->B);
  s->NF = c.n_slots * s->B + s->pend_max + 1;
  s->Cc = (s->B > 1 && s->S > 0) ? ((s->B * s->Se + 7) & ~7) : 0;
  s->dh = 2 * (s->hd / 6);
  s->dw = s->dh;
  s->dt = s->hd - 2 * s->dh;
  s->rope_pos = std::max(c.rope_reset, s->Tn - 1) + 1;
}

// bytes of one fragment-ordered weight copy [N][K] (K % 64 == 0)
size_t packed_bytes(int N, int K) { return sdk::pack_weight_bytes(N, K); }

// Lay out (or, with base == nullptr, measure) the workspace.
size_t carve(sd_stream* s, char* base) {
  const sd_stream_config& c = s->cfg;
  Carver cv{base};
  const size_t es = s->es;
  const int64_t M = (int64_t)s->Rmax * s->L;
  const int nctx = c.cfg_type != SD_CFG_SELF ? 2 : 1;
  s->fx = cv.take<float>((size_t)s->NF * s->lat * 4);
  s->fx0s = cv.take<float>((size_t)s->NF * s->lat * 4);
  if (c.sampler == SD_SAMPLER_LCM && s->n > 1) s->fz = cv.take<float>((size_t)s->NF * (s->n - 1) * s->lat * 4);
  if (c.ssf_on) {
    const size_t rb = c.ssf_kind == SD_SSF_U8 ? (size_t)c.ssf_h * c.ssf_w * c.ssf_c : (size_t)s->lat * 4;
    s->ssf_ref = cv.take<void>(rb);
  }
  s->sums = cv.take<long long>(sizeof(long long) * (4 + s->Tn));
  if (c.motion_on) s->mprev = cv.take<float>((size_t)s->frame_elems * 4);
  s->emb = cv.take<float>((size_t)s->Rmax * c.d_freq * 4);
  s->h1 = cv.take<float>((size_t)s->Rmax * s->d * 4);
  s->sc = cv.take<float>((size_t)s->Rmax * s->d * 4);
  s->mod = cv.take<float>((size_t)s->Rmax * 6 * s->d * 4);
  s->fmod = cv.take<float>((size_t)s->Rmax * 2 * s->d * 4);
  s->resid = cv.take<float>((size_t)M * s->d * 4);
  s->xm = cv.take<void>((size_t)M * std::max(s->d, s->P) * (s->bf ? 2 : 1) * es);
  s->q = cv.take<void>((size_t)M * s->d * es);
  s->kown = cv.take<void>((size_t)M * s->d * es);
  s->vtown = cv.take<void>((size_t)M * s->d * es);
  s->ao = cv.take<void>((size_t)M * s->d * es);
  s->hid = cv.take<void>((size_t)M * s->F * es);
  s->eps = cv.take<float>((size_t)s->Rmax * s->lat * 4);
  s->ringK = cv.take<void>((size_t)s->nb * s->H * s->Wt * s->hd * es);
  s->ringVT = cv.take<void>((size_t)s->nb * s->H * s->Wt * s->hd * es);
  s->sinkK = cv.take<void>((size_t)s->nb * s->H * s->S8 * s->hd * es);
  s->sinkVT = cv.take<void>((size_t)s->nb * s->H * s->S8 * s->hd * es);
  if (s->Cc > 0) {
    s->candK = cv.take<void>((size_t)s->nb * s->H * s->Cc * s->hd * es);
    s->candVT = cv.take<void>((size_t)s->nb * s->H * s->Cc * s->hd * es);
  }
  if (c.ctx_len > 0) {
    s->ctxK = cv.take<void>((size_t)s->nb * nctx * s->H * s->ctx8 * s->hd * es);
    s->ctxVT = cv.take<void>((size_t)s->nb * nctx * s->H * s->ctx8 * s->hd * es);
    // folding trades the d x d Q and O projections for two d x H Cp GEMMs: it
    // pays only when H Cp <= d.  The step's scores (fp32) and probabilities
    // (bf16) live in the FFN buffer.
    const size_t ncol = (size_t)s->H * s->ctx8;
    s->fold = s->bf && s->ctx8 <= 128 && ncol <= (size_t)s->d && ncol * 3 <= (size_t)s->F &&
              (size_t)c.ctx_len * 2 * s->d * 4 <= (size_t)M * s->F * es;
    if (s->fold) {
      s->fold_q = cv.take<void>((size_t)s->nb * nctx * ncol * s->d * es);
      s->fold_o = cv.take<void>((size_t)s->nb * nctx * s->d * ncol * es);
      s->fold_c = cv.take<float>((size_t)s->nb * nctx * ncol * 4);
    }
  }
  // fp32 partials of the products split over K: every GEMM of a forward of
  // at most 256 tokens, and those of at most 2048 tokens whose tiles would
  // leave most of the chip idle (rows of up to 2048 tokens)
  if (s->bf && s->L <= 2048) {
    s->gpart_cap = (int64_t)16 << 20;          // 64 MiB
    s->gpart = cv.take<float>((size_t)s->gpart_cap * 4);
  }
  if (s->bf && s->L <= 256) {
    const int d = s->d, F = s->F, nb = s->nb;
    auto take_packed = [&](int N, int K, int count) -> void* {
      return K % 64 ? nullptr : cv.take<void>(packed_bytes(N, K) * count);
    };
    s->wp_qkv = take_packed(3 * d, d, nb);
    s->wp_o = take_packed(d, d, nb);
    s->wp_f1 = take_packed(F, d, nb);
    s->wp_f2 = take_packed(d, F, nb);
    if (c.ctx_len > 0 && !s->fold) {
      s->wp_cq = take_packed(d, d, nb);
      s->wp_co = take_packed(d, d, nb);
    }
    if (s->fold) {
      const int ncol = s->H * s->ctx8;
      s->wp_fq = take_packed(ncol, d, nb * nctx);
      s->wp_fo = take_packed(d, ncol, nb * nctx);
    }
  }
  if (s->bf) {
    s->pe2 = cv.take<void>((size_t)s->d * 2 * s->P * es);
    s->head2 = cv.take<void>((size_t)s->P * 2 * s->d * es);
  }
  s->dyn = cv.take<StepDyn>(2 * sizeof(StepDyn));
  s->sink_emb = cv.take<double>((size_t)std::max(1, s->Ment) * s->d * 8);
  s->sink_part = cv.take<double>((size_t)64 * s->d * 8);
  s->sink_flag = cv.take<int>(16);
  s->sink_sim = cv.take<double>(16);
  s->rope_t = cv.take<float2>((size_t)s->rope_pos * std::max(1, s->dt / 2) * sizeof(float2));
  s->rope_h = cv.take<float2>((size_t)s->Hp * std::max(1, s->dh / 2) * sizeof(float2));
  s->rope_w = cv.take<float2>((size_t)s->Wp * std::max(1, s->dw / 2) * sizeof(float2));
  if (s->bf) {
    // split-KV partials, at most 8 splits and 1 GiB
    const size_t per = (size_t)M * s->d * 4 + (size_t)M * s->H * sizeof(float2);
    s->attn_split_max = (int)std::max<size_t>(1, std::min<size_t>(8, ((size_t)1 << 30) / per));
    if (s->attn_split_max > 1) {
      s->part_o = cv.take<bf16>((size_t)s->attn_split_max * M * s->d * 2);
      s->part_ml = cv.take<float2>((size_t)s->attn_split_max * M * s->H * sizeof(float2));
    }
  }
  return cv.off;
}

sd_status set_err(sd_stream* s, sd_status code, const std::string& msg) {
  if (s) s->err = msg;
  return code;
}

#define PROF(kind, flops, bytes, expr)              \
  do {                                              \
    const int _ev = prof_begin(s, kind);            \
    HIP_TRY(expr);                                  \
    prof_end(s, kind, _ev, (flops), (bytes));       \
  } while (0)

#define HIP_TRY(expr)                                                              \
  do {                                                                             \
    hipError_t _e = (expr);                                                        \
    if (_e != hipSuccess)                                                          \
      return set_err(s, SD_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(_e)); \
  } while (0)

const char* P(const void* base, int64_t elem_off, size_t es) { return (const char*)base + elem_off * (int64_t)es; }
char* Pm(void* base, int64_t elem_off, size_t es) { return (char*)base + elem_off * (int64_t)es; }

void rope_tables(const sd_stream* s, std::vector<float2>& t, std::vector<float2>& h, std::vector<float2>& w) {
  const double base = s->cfg.rope_base;
  auto fill = [&](std::vector<float2>& out, int npos, int width) {
    out.assign((size_t)npos * std::max(1, width / 2), float2{1.f, 0.f});
    sdk::rope_table_fill(out.data(), npos, width, base);
  };
  fill(t, s->rope_pos, s->dt);
  fill(h, s->Hp, s->dh);
  fill(w, s->Wp, s->dw);
}

// block (or block-and-context) b of a fragment-ordered copy, null if none
const void* packed_at(const void* base, int b, int N, int K) {
  return base ? (const char*)base + (int64_t)b * (int64_t)packed_bytes(N, K) : nullptr;
}

Epi epi_base(const sd_stream* s, int mode) {
  Epi E;
  std::memset(&E, 0, sizeof(E));
  E.mode = mode;
  E.L = s->L;
  E.six_d = 6 * s->d;
  E.H = s->H;
  E.hd = s->hd;
  E.d = s->d;
  E.Hp = s->Hp;
  E.Wp = s->Wp;
  E.dt = s->dt;
  E.dh = s->dh;
  E.rope_t = s->rope_t;
  E.rope_h = s->rope_h;
  E.rope_w = s->rope_w;
  E.C = s->cfg.latent_c;
  E.Hl = s->cfg.latent_h;
  E.Wl = s->cfg.latent_w;
  E.p = s->cfg.patch;
  E.T = s->Tn;
  E.krows = 1;
  E.part = s->gpart;
  E.part_cap = s->gpart_cap;
  return E;
}

// Ask the residual GEMM described by E to also write the LayerNorm that
// reads the residual next (into xm: form, modulation mod / blk at shift /
// scale of six).  True when the GEMM's launch does it in its reduction pass
// (few rows, bf16); otherwise the caller runs the LayerNorm itself.
static bool fuse_ln(const sd_stream* s, Epi& E, int M, int N, int K, const float* mod, const void* blk, int shift,
                    int scale, int six, int form) {
  if (!s->bf) return false;
  E.ln_out = s->xm;
  E.ln_mod = mod;
  E.ln_blk = mod ? blk : nullptr;
  E.ln_shift = shift;
  E.ln_scale = scale;
  E.ln_six = mod ? six : 4;
  E.ln_form = form;
  E.ln_eps = 1e-6f;
  if (sdk::gemm_fuses_ln(M, N, K, E)) return true;
  E.ln_out = nullptr;
  return false;
}

// Start timing a launch of `kind` (returns -1 when that kind is not profiled).
int prof_begin(sd_stream* s, int kind) {
  if (!(s->prof_mask & (1u << kind))) return -1;
  while ((int)s->ev_pool.size() < s->ev_used + 2) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return -1;
    s->ev_pool.push_back(e);
  }
  const int ev = s->ev_used;
  s->ev_used += 2;
  if (hipEventRecord(s->ev_pool[ev], s->pst) != hipSuccess) return -1;
  return ev;
}

void prof_end(sd_stream* s, int kind, int ev, double flops, double bytes) {
  if (ev < 0) return;
  if (hipEventRecord(s->ev_pool[ev + 1], s->pst) != hipSuccess) return;
  s->prof_pending.push_back({kind, ev, flops, bytes});
}

double gflop(int64_t M, int64_t N, int64_t K) { return 2.0 * M * N * K; }
// algorithmic bytes of a GEMM: both operands once plus the output traffic
double gbytes(int64_t M, int64_t N, int64_t K, size_t es, double out_bytes) {
  return (double)(M * K + N * K) * es + (double)M * N * out_bytes;
}

int free_frame(sd_stream* s) {
  for (int i = 0; i < s->NF; ++i)
    if (!s->frames[i].used) return i;
  return -1;
}

}  // namespace

extern "C" {

size_t sd_stream_workspace_bytes(const sd_stream_config* cfg) {
  if (!cfg) return 0;
  if (sd::validate_config(*cfg, nullptr) != SD_OK) return 0;
  sd_stream tmp;
  tmp.cfg = *cfg;
  dims(&tmp);
  return carve(&tmp, nullptr);
}

sd_status sd_stream_create(const sd_stream_config* cfg, const sd_weights* w, void* workspace, size_t ws_bytes,
                           void* hip_stream, sd_stream** out) {
  if (!cfg || !w || !out) return SD_ERR_ARG;
  *out = nullptr;
  std::string err;
  const int rc = sd::validate_config(*cfg, &err);
  if (rc != SD_OK) return (sd_status)rc;
  const void* need[] = {w->t_w1, w->t_b1, w->t_w2, w->t_b2, w->mod_w, w->mod_b, w->blk_mod, w->pe_w,
                        w->pe_b, w->qkv_w, w->qkv_b, w->o_w, w->o_b, w->f1_w, w->f1_b, w->f2_w,
                        w->f2_b, w->fin_w, w->fin_b, w->head_w, w->head_b};
  for (const void* p : need)
    if (!p) return SD_ERR_ARG;
  if (cfg->ctx_len > 0 && (!w->cq_w || !w->cq_b || !w->ckv_w || !w->ckv_b || !w->co_w || !w->co_b))
    return SD_ERR_ARG;
  if (!workspace || ((uintptr_t)workspace & 255)) return SD_ERR_WORKSPACE;
  sd_stream* s = new sd_stream();
  s->cfg = *cfg;
  s->w = *w;
  s->st = (hipStream_t)hip_stream;
  s->pst = s->st;
  dims(s);
  const size_t need_ws = carve(s, nullptr);
  if (ws_bytes < need_ws) {
    delete s;
    return SD_ERR_WORKSPACE;
  }
  s->ws_used = carve(s, (char*)workspace);
  sd::make_schedule(s->cfg, s->a, s->b);
  s->frames.assign(s->NF, FrameRec());
  s->rec_ev.assign(s->NF, nullptr);
  s->rec_ev_set.assign(s->NF, 0);
  for (int i = 0; i < s->NF; ++i)
    if (hipEventCreateWithFlags(&s->rec_ev[i], hipEventDisableTiming) != hipSuccess) {
      delete s;
      return SD_ERR_HIP;
    }
  if (hipEventCreateWithFlags(&s->ev_push, hipEventDisableTiming) != hipSuccess) {
    delete s;
    return SD_ERR_HIP;
  }
  for (int i = 0; i < SD_MAX_SLOTS * SD_MAX_CHUNKS; ++i) s->slots[i] = -1;
  s->ctl.s = s->cfg.s_max;
  std::memset(s->prof_acc, 0, sizeof(s->prof_acc));
  {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
      s->cus = cus;
  }
  // zero the caches (padding keys must stay finite) and upload RoPE tables
  std::vector<float2> rt, rh, rw;
  rope_tables(s, rt, rh, rw);
  hipError_t e = hipSuccess;
  const size_t cache_bytes[] = {(size_t)s->nb * s->H * s->Wt * s->hd * s->es,
                                (size_t)s->nb * s->H * s->S8 * s->hd * s->es};
  if (e == hipSuccess) e = sdk::fill_zero(s->st, s->ringK, cache_bytes[0]);
  if (e == hipSuccess) e = sdk::fill_zero(s->st, s->ringVT, cache_bytes[0]);
  if (e == hipSuccess) e = sdk::fill_zero(s->st, s->sinkK, cache_bytes[1]);
  if (e == hipSuccess) e = sdk::fill_zero(s->st, s->sinkVT, cache_bytes[1]);
  if (e == hipSuccess) e = sdk::fill_zero(s->st, s->sink_emb, (size_t)std::max(1, s->Ment) * s->d * 8);
  if (e == hipSuccess) e = sdk::fill_zero(s->st, s->sink_flag, 16);
  if (s->bf)
    for (int half = 0; half < 2 && e == hipSuccess; ++half) {
      e = hipMemcpy2DAsync(Pm(s->pe2, (int64_t)half * s->P, s->es), 2 * s->P * s->es, w->pe_w, s->P * s->es,
                           s->P * s->es, s->d, hipMemcpyDeviceToDevice, s->st);
      if (e == hipSuccess)
        e = hipMemcpy2DAsync(Pm(s->head2, (int64_t)half * s->d, s->es), 2 * s->d * s->es, w->head_w, s->d * s->es,
                             s->d * s->es, s->P, hipMemcpyDeviceToDevice, s->st);
    }
  {
    const int d = s->d, F = s->F;
    auto pack = [&](void* dst, const void* src, int N, int K) {
      if (!dst) return;
      for (int b = 0; b < s->nb && e == hipSuccess; ++b)
        e = sdk::pack_weight(s->st, P(src, (int64_t)b * N * K, s->es), N, K, Pm(dst, (int64_t)b * packed_bytes(N, K), 1));
    };
    pack(s->wp_qkv, w->qkv_w, 3 * d, d);
    pack(s->wp_o, w->o_w, d, d);
    pack(s->wp_f1, w->f1_w, F, d);
    pack(s->wp_f2, w->f2_w, d, F);
    pack(s->wp_cq, w->cq_w, d, d);
    pack(s->wp_co, w->co_w, d, d);
  }
  if (e == hipSuccess) e = hipMemcpyAsync(s->rope_t, rt.data(), rt.size() * sizeof(float2), hipMemcpyHostToDevice, s->st);
  if (e == hipSuccess) e = hipMemcpyAsync(s->rope_h, rh.data(), rh.size() * sizeof(float2), hipMemcpyHostToDevice, s->st);
  if (e == hipSuccess) e = hipMemcpyAsync(s->rope_w, rw.data(), rw.size() * sizeof(float2), hipMemcpyHostToDevice, s->st);
  if (e == hipSuccess) e = hipStreamSynchronize(s->st);
  if (e != hipSuccess) {
    delete s;
    return SD_ERR_HIP;
  }
  s->ctx_set = (cfg->ctx_len == 0);
  *out = s;
  return SD_OK;
}

sd_status sd_stream_set_context(sd_stream* s, const void* ctx_pos, const void* ctx_neg) {
  if (!s) return SD_ERR_ARG;
  const sd_stream_config& c = s->cfg;
  if (c.ctx_len == 0) return set_err(s, SD_ERR_STATE, "no cross-attention configured (ctx_len == 0)");
  if (!ctx_pos) return set_err(s, SD_ERR_ARG, "ctx_pos is null");
  if (c.cfg_type != SD_CFG_SELF && !ctx_neg)
    return set_err(s, SD_ERR_ARG, "onetime-negative R-CFG and full CFG need ctx_neg");
  const int nctx = c.cfg_type != SD_CFG_SELF ? 2 : 1;
  const size_t per = (size_t)s->H * s->ctx8 * s->hd;   // elements per (block, context)
  HIP_TRY(sdk::fill_zero(s->st, s->ctxK, (size_t)s->nb * nctx * per * s->es));
  HIP_TRY(sdk::fill_zero(s->st, s->ctxVT, (size_t)s->nb * nctx * per * s->es));
  for (int b = 0; b < s->nb; ++b)
    for (int ci = 0; ci < nctx; ++ci) {
      Epi E = epi_base(s, EPI_CTXKV);
      E.bias = P(s->w.ckv_b, (int64_t)b * 2 * s->d, s->es);
      E.L = c.ctx_len;
      E.k = Pm(s->ctxK, ((int64_t)b * nctx + ci) * per, s->es);
      E.vt = Pm(s->ctxVT, ((int64_t)b * nctx + ci) * per, s->es);
      E.kstride = s->ctx8;
      E.rope = 0;
      HIP_TRY(sdk::gemm(s->st, s->bf, ci == 0 ? ctx_pos : ctx_neg, P(s->w.ckv_w, (int64_t)b * 2 * s->d * s->d, s->es),
                        c.ctx_len, 2 * s->d, s->d, E));
    }
  if (s->fold) {
    // the prompt K | V in fp32 (scratch: the FFN buffer, free between steps),
    // folded into fp16 score / output matrices
    const int64_t ncol = (int64_t)s->H * s->ctx8, d = s->d;
    float* kv = (float*)s->hid;
    for (int b = 0; b < s->nb; ++b)
      for (int ci = 0; ci < nctx; ++ci) {
        const int64_t bc = (int64_t)b * nctx + ci;
        Epi E = epi_base(s, EPI_F32);
        E.bias = P(s->w.ckv_b, (int64_t)b * 2 * d, s->es);
        E.out = kv;
        E.ldo = 2 * s->d;
        HIP_TRY(sdk::gemm(s->st, s->bf, ci == 0 ? ctx_pos : ctx_neg, P(s->w.ckv_w, (int64_t)b * 2 * d * d, s->es),
                          c.ctx_len, 2 * s->d, s->d, E));
        HIP_TRY(sdk::cross_fold(s->st, kv, (const bf16*)P(s->w.cq_w, (int64_t)b * d * d, s->es),
                                (const bf16*)P(s->w.cq_b, (int64_t)b * d, s->es),
                                (const bf16*)P(s->w.co_w, (int64_t)b * d * d, s->es),
                                (f16*)Pm(s->fold_q, bc * ncol * d, s->es), s->fold_c + bc * ncol,
                                (f16*)Pm(s->fold_o, bc * d * ncol, s->es), s->d, s->H, s->hd, c.ctx_len, s->ctx8));
        if (s->wp_fq)
          HIP_TRY(sdk::pack_weight(s->st, P(s->fold_q, bc * ncol * d, s->es), (int)ncol, (int)d,
                                   Pm(s->wp_fq, bc * (int64_t)packed_bytes((int)ncol, (int)d), 1)));
        if (s->wp_fo)
          HIP_TRY(sdk::pack_weight(s->st, P(s->fold_o, bc * d * ncol, s->es), (int)d, (int)ncol,
                                   Pm(s->wp_fo, bc * (int64_t)packed_bytes((int)d, (int)ncol), 1)));
      }
  }
  s->ctx_set = true;
  return SD_OK;
}

sd_status sd_stream_push_frame(sd_stream* s, const float* x0, const float* noise, const void* ssf_frame, double u,
                               sd_push_info* info) {
  if (!s) return SD_ERR_ARG;
  const sd_stream_config& c = s->cfg;
  if (!x0 || !noise || !info) return set_err(s, SD_ERR_ARG, "null x0, noise or info");
  if (c.ssf_on && c.ssf_kind == SD_SSF_U8 && !ssf_frame) return set_err(s, SD_ERR_ARG, "ssf_frame is null");
  if (!(u >= 0.0 && u <= 1.0)) return set_err(s, SD_ERR_ARG, "u must be in [0, 1]");
  if ((int)s->pending.size() >= s->pend_max) return set_err(s, SD_ERR_STATE, "pending queue full; call step()");
  std::memset(info, 0, sizeof(*info));
  info->t0 = -1;
  info->frame_id = -1;
  info->sim = 1.0;
  info->s = s->ctl.s;
  // all of the push runs on the IO stream when one is set
  const hipStream_t ps = s->io ? s->io : s->st;
  s->pst = ps;
  struct RestorePst {
    sd_stream* s;
    ~RestorePst() { s->pst = s->st; }
  } restore_pst{s};
  // device reductions for the SSF and motion decisions, one read-back
  const void* ssf_cur = c.ssf_kind == SD_SSF_U8 ? ssf_frame : (const void*)x0;
  const int64_t ssf_n = c.ssf_kind == SD_SSF_U8 ? (int64_t)c.ssf_h * c.ssf_w * c.ssf_c : s->lat;
  const bool do_ssf = c.ssf_on && s->ctl.has_ref;
  long long hs[4 + 64] = {};
  if (do_ssf)
    PROF(SD_PROF_CONTROLS, 0.0, 2.0 * ssf_n * (c.ssf_kind == SD_SSF_U8 ? 1 : 4),
         sdk::ssf_sums(ps, c.ssf_kind, ssf_cur, s->ssf_ref, ssf_n, s->sums));
  if (c.motion_on)
    PROF(SD_PROF_CONTROLS, 0.0, 4.0 * (s->Tn + 1) * s->frame_elems,
         sdk::motion_sums(ps, x0, s->ctl.has_prev ? s->mprev : nullptr, s->Tn, s->frame_elems, s->sums + 4));
  if (do_ssf || c.motion_on) {
    HIP_TRY(hipMemcpyAsync(hs, s->sums, sizeof(long long) * (4 + s->Tn), hipMemcpyDeviceToHost, ps));
    HIP_TRY(hipStreamSynchronize(ps));
  }
  if (c.ssf_on) {
    double sim = 1.0, p = 0.0;
    const bool skip = sd::ssf_decide(s->ctl, c, hs[0], hs[1], hs[2], u, &sim, &p);
    info->sim = sim;
    info->p = p;
    if (skip) {
      info->skipped = 1;
      return SD_OK;
    }
    const size_t rb = c.ssf_kind == SD_SSF_U8 ? (size_t)ssf_n : (size_t)ssf_n * 4;
    HIP_TRY(hipMemcpyAsync(s->ssf_ref, ssf_cur, rb, hipMemcpyDeviceToDevice, ps));
  }
  const int f = free_frame(s);
  if (f < 0) return set_err(s, SD_ERR_STATE, "frame store full");
  FrameRec& fr = s->frames[f];
  if (c.motion_on) {
    double dist[64];
    int nd = 0;
    for (int t = (s->ctl.has_prev ? 0 : 1); t < s->Tn; ++t) dist[nd++] = sd::motion_distance(hs[4 + t], s->frame_elems);
    sd::motion_push(s->ctl, c, dist, nd);
    if (nd > 0) info->d = dist[nd - 1];
    HIP_TRY(hipMemcpyAsync(s->mprev, x0 + (int64_t)(s->Tn - 1) * s->frame_elems, s->frame_elems * 4,
                           hipMemcpyDeviceToDevice, ps));
    s->ctl.has_prev = true;
    sd::taus_from_noise_rate(s->ctl.s, s->n, c.n_train_steps, fr.taus);
  } else {
    sd::taus_from_t_index(c, fr.taus);
  }
  info->s = s->ctl.s;
  fr.t0 = sd::rope_assign(s->ctl, s->Tn, c.rope_reset);
  fr.fid = s->n_pushed++;
  fr.used = true;
  const int tau0 = fr.taus[0];
  // the record's previous reader (a step on the main stream) must be done
  if (s->io && s->rec_ev_set[f]) HIP_TRY(hipStreamWaitEvent(ps, s->rec_ev[f], 0));
  PROF(SD_PROF_EPILOGUE, 2.0 * s->lat, 16.0 * s->lat,
       sdk::entry_noise(ps, x0, noise, s->fx + (int64_t)f * s->lat, s->fx0s + (int64_t)f * s->lat, s->lat,
                        (float)s->a[tau0], (float)s->b[tau0]));
  if (s->fz)
    HIP_TRY(hipMemcpyAsync(s->fz + (int64_t)f * (s->n - 1) * s->lat, noise + s->lat,
                           (size_t)(s->n - 1) * s->lat * 4, hipMemcpyDeviceToDevice, ps));
  if (s->io) {
    HIP_TRY(hipEventRecord(s->ev_push, ps));
    s->push_pending = true;
  }
  s->pending.push_back(f);
  info->t0 = fr.t0;
  info->frame_id = fr.fid;
  for (int i = 0; i < s->n; ++i) info->taus[i] = fr.taus[i];
  return SD_OK;
}

// Which rows of a forward leave the pipeline and take the cache updates: in
// push order, row rows[k] appends its K / V^T at ring position ptr_old + k L
// (and fills sink entry cap_entry[k], or stages a refresh candidate), then
// takes its sink decision after the last block.
struct ExitPlan {
  int n;
  const int* rows;
  const int* cap_entry;
  int ptr_old;
};

// One denoiser forward over the rows of rt (rows [0, R_pos) under the
// positive prompt, the nneg after them under the negative one): conditioning,
// patch embedding, the blocks, the final layer; eps_out receives eps of row r
// at eps_out + r * lat.  With xp the leaving rows update the KV cache and the
// sink; without it the cache is only read.
extern "C++" {
// Per-step device values of a forward over rt (see StepDyn), from the cache
// state as it stands at the start of the step.
static StepDyn make_dyn(const sd_stream* s, const RowTable& rt, int nexit, int ptr_old) {
  StepDyn d;
  std::memset(&d, 0, sizeof(d));
  d.rt = rt;
  for (int r = 0; r < rt.R; ++r) d.t0[r] = rt.r[r].t0;
  d.seg[0] = 0;
  d.seg[1] = s->sink_count * s->Se;
  d.seg[2] = s->Wt > 0 ? (s->kv_ptr - s->kv_valid + s->Wt) % s->Wt : 0;
  d.seg[3] = s->kv_valid;
  for (int k = 0; k < nexit; ++k)
    d.kv_pos[k] = s->Wt > 0 ? (int)(((int64_t)ptr_old + (int64_t)k * s->L) % s->Wt) : 0;
  d.ptr_old = ptr_old;
  return d;
}

// Graph replay applies to bf16 steps on a created stream with no IO queue,
// no live profiling and no clean-latent recompute (its second forward's rows
// depend on the exits).
static bool graph_eligible(const sd_stream* s) {
  return s->graph_on && s->bf && s->st != nullptr && s->io == nullptr && s->prof_mask == 0 && !s->cfg.kv_recompute;
}

// Launch the graph recorded for `key`, capturing it from `body` the first
// time; at most four are kept (least recently used evicted).
template <typename F>
static sd_status graph_run(sd_stream* s, const std::vector<int64_t>& key, F&& body) {
  sd_stream::GraphEntry* ge = nullptr;
  for (auto& g : s->graphs)
    if (g.key == key) ge = &g;
  if (!ge) {
    HIP_TRY(hipStreamBeginCapture(s->st, hipStreamCaptureModeThreadLocal));
    const sd_status fs = body();
    hipGraph_t graph = nullptr;
    const hipError_t ce = hipStreamEndCapture(s->st, &graph);
    if (fs != SD_OK) {
      if (graph) (void)hipGraphDestroy(graph);
      return fs;
    }
    if (ce != hipSuccess || !graph) return set_err(s, SD_ERR_HIP, std::string("graph capture: ") + hipGetErrorString(ce));
    hipGraphExec_t exec = nullptr;
    const hipError_t ie = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (ie != hipSuccess) return set_err(s, SD_ERR_HIP, std::string("graph instantiate: ") + hipGetErrorString(ie));
    if (s->graphs.size() >= 4) {
      auto lru = s->graphs.begin();
      for (auto it = s->graphs.begin(); it != s->graphs.end(); ++it)
        if (it->used < lru->used) lru = it;
      (void)hipGraphExecDestroy(lru->exec);
      s->graphs.erase(lru);
    }
    s->graphs.push_back({key, exec, 0});
    ge = &s->graphs.back();
    ++s->graph_captures;
  } else {
    ++s->graph_replays;
  }
  ge->used = ++s->graph_clock;
  HIP_TRY(hipGraphLaunch(ge->exec, s->st));
  return SD_OK;
}
}  // extern "C++"

// The forward over rows rt (host copy, for shapes and launch decisions); the
// kernels read the per-step values from dd, the device copy written before.
static sd_status run_forward(sd_stream* s, const RowTable& rt, const StepDyn* dd, int R_pos, int nneg,
                             const ExitPlan* xp, float* eps_out) {
  const sd_stream_config& c = s->cfg;
  const int R = rt.R;
  const int L = s->L, d = s->d, H = s->H, hd = s->hd, M = R * L;
  const size_t es = s->es;
  const bool bf = s->bf;
  hipStream_t st = s->st;
  const int nexit = xp ? xp->n : 0;
  const int* exit_rows = xp ? xp->rows : nullptr;
  const int* cap_entry = xp ? xp->cap_entry : nullptr;
  const int ptr_old = xp ? xp->ptr_old : 0;

  // ---- conditioning: timestep embedding -> MLP -> SiLU(c) -> adaLN vectors
  PROF(SD_PROF_GEMV, 0.0, 4.0 * R * c.d_freq, sdk::temb_embed(st, &dd->rt, R, s->emb, c.d_freq));
  PROF(SD_PROF_GEMV, 2.0 * R * d * c.d_freq, (double)d * c.d_freq * es,
       sdk::gemv(st, bf, s->emb, s->w.t_w1, s->w.t_b1, s->h1, R, d, c.d_freq, 1));
  PROF(SD_PROF_GEMV, 2.0 * R * d * d, (double)d * d * es, sdk::gemv(st, bf, s->h1, s->w.t_w2, s->w.t_b2, s->sc, R, d, d, 1));
  PROF(SD_PROF_GEMV, 12.0 * R * d * d, 6.0 * d * d * es,
       sdk::gemv(st, bf, s->sc, s->w.mod_w, s->w.mod_b, s->mod, R, 6 * d, d, 0));
  PROF(SD_PROF_GEMV, 4.0 * R * d * d, 2.0 * d * d * es,
       sdk::gemv(st, bf, s->sc, s->w.fin_w, s->w.fin_b, s->fmod, R, 2 * d, d, 0));

  // ---- patch embedding into the fp32 residual stream
  // (bf16: hi + lo input pairs against the doubled weights, K = 2P)
  const int KP = bf ? 2 * s->P : s->P;
  PROF(SD_PROF_OTHER, 0.0, (4.0 + es * KP / s->P) * R * s->lat,
       sdk::patchify(st, bf, &dd->rt, R, s->fx, s->xm, s->lat, s->Tn, c.latent_c, c.latent_h, c.latent_w, c.patch,
                     bf));
  {
    Epi E = epi_base(s, EPI_PATCH);
    E.bias = s->w.pe_b;
    E.resid = s->resid;
    PROF(SD_PROF_OTHER, gflop(M, d, KP), gbytes(M, d, KP, es, 4),
         sdk::gemm(st, bf, s->xm, bf ? s->pe2 : s->w.pe_w, M, d, KP, E));
  }

  const int nctx = c.cfg_type != SD_CFG_SELF ? 2 : 1;
  // q is [R][H][L][hd]; the own K / V^T are head-major, [H][R][L][hd] and
  // [H][hd][R][L], so that one head's keys of every row are contiguous (the
  // key range of cross-frame batch attention)
  const int64_t own_stride = (int64_t)H * L * hd;
  const int64_t kv_hs = (int64_t)R * L * hd;
  // set when the residual GEMM before a LayerNorm already wrote its output
  // into xm (fuse_ln)
  bool ln_ready = false;
  for (int b = 0; b < s->nb; ++b) {
    const void* blk = P(s->w.blk_mod, (int64_t)b * 6 * d, es);
    // self-attention
    AttnArgs combine_args;
    bool combine_pending = false;
    if (!ln_ready)
      PROF(SD_PROF_LN, 0.0, (4.0 + es) * M * d,
           sdk::ln_mod(st, bf, s->resid, s->xm, M, d, L, s->mod, blk, 0, d, 6 * d, 1e-6f));
    ln_ready = false;
    {
      Epi E = epi_base(s, EPI_QKV);
      E.bias = P(s->w.qkv_b, (int64_t)b * 3 * d, es);
      E.q = s->q;
      E.k = s->kown;
      E.vt = s->vtown;
      E.kstride = L;
      E.krows = R;
      E.rope = 1;
      for (int r = 0; r < R; ++r) E.t0[r] = rt.r[r].t0;
      E.t0_dev = dd->t0;
      E.wpack = packed_at(s->wp_qkv, b, 3 * d, d);
      PROF(SD_PROF_GEMM_QKV, gflop(M, 3 * d, d), gbytes(M, 3 * d, d, es, es),
           sdk::gemm(st, bf, s->xm, P(s->w.qkv_w, (int64_t)b * 3 * d * d, es), M, 3 * d, d, E));
    }
    {
      AttnArgs A;
      std::memset(&A, 0, sizeof(A));
      A.q = s->q;
      A.q_rs = own_stride;
      A.q_hs = (int64_t)L * hd;
      A.o = s->ao;
      A.R = R;
      A.H = H;
      A.L = L;
      A.hd = hd;
      A.d = d;
      A.scale = 1.0f / std::sqrt((float)hd);
      int ns = 0;
      KvSeg& sk = A.seg[ns++];
      sk.k = P(s->sinkK, (int64_t)b * H * s->S8 * hd, es);
      sk.vt = P(s->sinkVT, (int64_t)b * H * s->S8 * hd, es);
      sk.k_hs = sk.vt_hs = (int64_t)s->S8 * hd;
      sk.cap = std::max(8, s->S8);
      sk.start = 0;
      sk.count = s->sink_count * s->Se;
      KvSeg& sw = A.seg[ns++];
      sw.k = P(s->ringK, (int64_t)b * H * s->Wt * hd, es);
      sw.vt = P(s->ringVT, (int64_t)b * H * s->Wt * hd, es);
      sw.k_hs = sw.vt_hs = (int64_t)s->Wt * hd;
      sw.cap = std::max(8, s->Wt);
      sw.count = s->kv_valid;
      sw.start = s->Wt > 0 ? (s->kv_ptr - s->kv_valid + s->Wt) % s->Wt : 0;
      sw.wrap = 1;
      // own tokens: this row's (row stride L tokens), or with batch attention
      // every row's (row stride 0, R L tokens)
      KvSeg& so = A.seg[ns++];
      so.k = s->kown;
      so.vt = s->vtown;
      so.k_rs = c.batch_attn ? 0 : (int64_t)L * hd;
      so.vt_rs = c.batch_attn ? 0 : L;
      so.k_hs = so.vt_hs = kv_hs;
      so.cap = R * L;
      so.count = c.batch_attn ? R * L : L;
      A.nseg = ns;
      if (bf) A.dyn_seg = dd->seg;
      if (s->attn_split_max > 1) {
        const int nk = ((sk.count + 7) & ~7) + sw.count + so.count;
        const int qt = sdk::attention_q_tile(bf, hd);
        sdk::attention_pick_plan(H, R * ((L + qt - 1) / qt), (nk + 63) / 64, s->attn_split_max,
                                 s->cus * sdk::attention_wg_per_cu(bf, hd), &A.nsplit, &A.h_full);
        A.part_o = s->part_o;
        A.part_ml = s->part_ml;
        A.part_so = (long long)s->Rmax * L * d;
        A.part_sml = (long long)s->Rmax * H * L;
      }
      const double shared = (double)sk.count + sw.count;
      PROF(SD_PROF_ATTN_SELF, 4.0 * R * L * (shared + so.count) * d,
           (double)es * d * (2.0 * R * L + 2.0 * shared + 2.0 * R * L), sdk::attention(st, bf, A, false));
      if (A.nsplit > 1 && A.h_full < H) {
        combine_args = A;
        combine_pending = true;
      }
    }
    // the combine pass of the split heads (run below, in the append's launch
    // when a single chunk leaves)
    const double comb_bytes =
        combine_pending ? (double)(H - combine_args.h_full) / H *
                              ((double)combine_args.nsplit * R * L * (d * 2.0 + H * 8.0) + (double)R * L * d * es)
                        : 0.0;
    // the leaving chunks append their K / V^T in push order (ring positions
    // ptr_old + k L); a capturing chunk also fills its sink entry, with B > 1
    // a refresh candidate stages its first S_e tokens
    for (int k = 0; k < nexit; ++k) {
      void *dK = nullptr, *dVT = nullptr;
      int dcap = s->S8, doff = 0;
      if (cap_entry[k] >= 0) {
        const int64_t cb = (int64_t)b * H * s->S8 * hd;
        dK = Pm(s->sinkK, cb, es);
        dVT = Pm(s->sinkVT, cb, es);
        doff = cap_entry[k] * s->Se;
      } else if (s->Cc > 0) {
        const int64_t cb = (int64_t)b * H * s->Cc * hd;
        dK = Pm(s->candK, cb, es);
        dVT = Pm(s->candVT, cb, es);
        dcap = s->Cc;
        doff = k * s->Se;
      }
      if (s->Wt == 0 && !dK) continue;
      const int pk = s->Wt > 0 ? (int)(((int64_t)ptr_old + (int64_t)k * L) % s->Wt) : 0;
      if (combine_pending && nexit == 1 &&
          sdk::kv_append_vec_ok(bf, kv_hs, (int64_t)R * L, H, hd, L, s->Wt, pk, dK, dcap, doff, s->Se)) {
        const sdk::KvAppendArgs ka{(const bf16*)P(s->kown, (int64_t)exit_rows[k] * L * hd, es),
                                   (const bf16*)P(s->vtown, (int64_t)exit_rows[k] * L, es), kv_hs, (int64_t)R * L,
                                   (bf16*)Pm(s->ringK, (int64_t)b * H * s->Wt * hd, es),
                                   (bf16*)Pm(s->ringVT, (int64_t)b * H * s->Wt * hd, es), H, hd, L, s->Wt, pk,
                                   (bf16*)dK, (bf16*)dVT, dcap, doff, s->Se, &dd->kv_pos[k]};
        PROF(SD_PROF_ATTN_COMBINE, 0.0, comb_bytes + 4.0 * L * d * es,
             sdk::attention_combine_append(st, combine_args, ka));
        combine_pending = false;
        continue;
      }
      PROF(SD_PROF_KV, 0.0, 4.0 * L * d * es,
           sdk::kv_append(st, bf, P(s->kown, (int64_t)exit_rows[k] * L * hd, es), P(s->vtown, (int64_t)exit_rows[k] * L, es),
                          kv_hs, (int64_t)R * L,
                          Pm(s->ringK, (int64_t)b * H * s->Wt * hd, es), Pm(s->ringVT, (int64_t)b * H * s->Wt * hd, es),
                          H, hd, L, s->Wt, pk, dK, dVT, dcap, doff, s->Se, &dd->kv_pos[k]));
    }
    if (combine_pending) {
      PROF(SD_PROF_ATTN_COMBINE, 0.0, comb_bytes, sdk::attention_combine(st, combine_args));
      combine_pending = false;
    }
    {
      Epi E = epi_base(s, EPI_GATE_RESID);
      E.bias = P(s->w.o_b, (int64_t)b * d, es);
      E.resid = s->resid;
      E.mod = s->mod;
      E.blk = blk;
      E.gate_off = 2 * d;
      E.wpack = packed_at(s->wp_o, b, d, d);
      // the LayerNorm after it: the cross-attention input (fp16 when folded),
      // or the feed-forward one when there is no prompt
      if (c.ctx_len > 0)
        ln_ready = fuse_ln(s, E, M, d, d, nullptr, nullptr, 0, 0, 6 * d, s->fold ? sdk::LN_F16 : sdk::LN_PLAIN);
      else
        ln_ready = fuse_ln(s, E, M, d, d, s->mod, blk, 3 * d, 4 * d, 6 * d, sdk::LN_PLAIN);
      PROF(SD_PROF_GEMM_O, gflop(M, d, d), gbytes(M, d, d, es, 8) + (ln_ready ? (double)M * d * es : 0.0),
           sdk::gemm(st, bf, s->ao, P(s->w.o_w, (int64_t)b * d * d, es), M, d, d, E));
    }
    // cross-attention to the pre-computed prompt K/V
    if (c.ctx_len > 0 && s->fold) {
      if (!ln_ready)
        PROF(SD_PROF_LN, 0.0, (4.0 + es) * M * d,
             sdk::ln_mod(st, bf, s->resid, s->xm, M, d, L, nullptr, nullptr, 0, 0, 6 * d, 1e-6f, sdk::LN_F16));
      ln_ready = false;
      const int ncol = H * s->ctx8;
      float* sc = (float*)s->hid;
      f16* pc = (f16*)((char*)s->hid + (size_t)M * ncol * 4);
      // rows [0, R_pos) read the positive context, [R_pos, R_pos + nneg) the negative one
      for (int part = 0; part < (nneg > 0 ? 2 : 1); ++part) {
        const int64_t t0 = (int64_t)(part == 0 ? 0 : R_pos) * L, Mp = (int64_t)(part == 0 ? R_pos : nneg) * L;
        const int64_t bc = (int64_t)b * nctx + part;
        bool sm_fused = false;
        {
          Epi E = epi_base(s, EPI_F32);
          E.out = sc + t0 * ncol;
          E.ldo = ncol;
          E.wpack = packed_at(s->wp_fq, (int)bc, ncol, d);
          // few rows: the reduction pass writes the probabilities itself
          E.sm_out = pc + t0 * ncol;
          E.sm_bias = s->fold_c + bc * ncol;
          E.sm_heads = H;
          E.sm_cp = s->ctx8;
          sm_fused = sdk::gemm_fuses_softmax((int)Mp, ncol, d, E);
          if (!sm_fused) E.sm_out = nullptr;
          PROF(SD_PROF_GEMM_CROSS, gflop(Mp, ncol, d), gbytes(Mp, ncol, d, es, sm_fused ? 2 : 4),
               sdk::gemm_mfma_f16(st, P(s->xm, t0 * d, es), P(s->fold_q, bc * ncol * d, es), (int)Mp, ncol, d, E));
        }
        if (!sm_fused)
          PROF(SD_PROF_ATTN_CROSS, 4.0 * Mp * ncol, 6.0 * Mp * ncol,
               sdk::ctx_softmax(st, sc + t0 * ncol, s->fold_c + bc * ncol, pc + t0 * ncol, Mp, H, s->ctx8));
        {
          Epi E = epi_base(s, EPI_RESID);
          E.bias = P(s->w.co_b, (int64_t)b * d, es);
          E.resid = s->resid + t0 * d;
          E.wpack = packed_at(s->wp_fo, (int)bc, d, ncol);
          // one context: the feed-forward LayerNorm of every row follows
          if (nneg == 0) ln_ready = fuse_ln(s, E, (int)Mp, d, ncol, s->mod, blk, 3 * d, 4 * d, 6 * d, sdk::LN_PLAIN);
          PROF(SD_PROF_GEMM_CROSS, gflop(Mp, d, ncol), gbytes(Mp, d, ncol, es, 8) + (ln_ready ? (double)Mp * d * es : 0.0),
               sdk::gemm_mfma_f16(st, pc + t0 * ncol, P(s->fold_o, bc * d * ncol, es), (int)Mp, d, ncol, E));
        }
      }
    } else if (c.ctx_len > 0) {
      if (!ln_ready)
        PROF(SD_PROF_LN, 0.0, (4.0 + es) * M * d,
             sdk::ln_mod(st, bf, s->resid, s->xm, M, d, L, nullptr, nullptr, 0, 0, 6 * d, 1e-6f));
      ln_ready = false;
      {
        Epi E = epi_base(s, EPI_QKV);
        E.bias = P(s->w.cq_b, (int64_t)b * d, es);
        E.q = s->q;
        E.rope = 0;
        E.wpack = packed_at(s->wp_cq, b, d, d);
        PROF(SD_PROF_GEMM_CROSS, gflop(M, d, d), gbytes(M, d, d, es, es),
             sdk::gemm(st, bf, s->xm, P(s->w.cq_w, (int64_t)b * d * d, es), M, d, d, E));
      }
      const size_t per = (size_t)H * s->ctx8 * hd;
      for (int part = 0; part < (nneg > 0 ? 2 : 1); ++part) {
        AttnArgs A;
        std::memset(&A, 0, sizeof(A));
        A.q = s->q;
        A.q_rs = own_stride;
        A.q_hs = (int64_t)L * hd;
        A.o = s->ao;
        A.r0 = part == 0 ? 0 : R_pos;
        A.R = part == 0 ? R_pos : nneg;
        A.H = H;
        A.L = L;
        A.hd = hd;
        A.d = d;
        A.scale = 1.0f / std::sqrt((float)hd);
        A.nseg = 1;
        KvSeg& g = A.seg[0];
        g.k = P(s->ctxK, ((int64_t)b * nctx + part) * per, es);
        g.vt = P(s->ctxVT, ((int64_t)b * nctx + part) * per, es);
        g.k_hs = g.vt_hs = (int64_t)s->ctx8 * hd;
        g.cap = s->ctx8;
        g.count = c.ctx_len;
        PROF(SD_PROF_ATTN_CROSS, 4.0 * A.R * L * c.ctx_len * d, (double)es * d * (2.0 * A.R * L + 2.0 * c.ctx_len),
             sdk::attention(st, bf, A));
      }
      {
        Epi E = epi_base(s, EPI_RESID);
        E.bias = P(s->w.co_b, (int64_t)b * d, es);
        E.resid = s->resid;
        E.wpack = packed_at(s->wp_co, b, d, d);
        ln_ready = fuse_ln(s, E, M, d, d, s->mod, blk, 3 * d, 4 * d, 6 * d, sdk::LN_PLAIN);
        PROF(SD_PROF_GEMM_CROSS, gflop(M, d, d), gbytes(M, d, d, es, 8) + (ln_ready ? (double)M * d * es : 0.0),
             sdk::gemm(st, bf, s->ao, P(s->w.co_w, (int64_t)b * d * d, es), M, d, d, E));
      }
    }
    // feed-forward
    if (!ln_ready)
      PROF(SD_PROF_LN, 0.0, (4.0 + es) * M * d,
           sdk::ln_mod(st, bf, s->resid, s->xm, M, d, L, s->mod, blk, 3 * d, 4 * d, 6 * d, 1e-6f));
    ln_ready = false;
    {
      Epi E = epi_base(s, EPI_GELU);
      E.bias = P(s->w.f1_b, (int64_t)b * s->F, es);
      E.out = s->hid;
      E.ldo = s->F;
      E.wpack = packed_at(s->wp_f1, b, s->F, d);
      PROF(SD_PROF_GEMM_FFN1, gflop(M, s->F, d), gbytes(M, s->F, d, es, es),
           sdk::gemm(st, bf, s->xm, P(s->w.f1_w, (int64_t)b * s->F * d, es), M, s->F, d, E));
    }
    {
      Epi E = epi_base(s, EPI_GATE_RESID);
      E.bias = P(s->w.f2_b, (int64_t)b * d, es);
      E.resid = s->resid;
      E.mod = s->mod;
      E.blk = blk;
      E.gate_off = 5 * d;
      E.wpack = packed_at(s->wp_f2, b, d, s->F);
      // the next block's attention LayerNorm, or after the last block the
      // final layer's (hi / lo pairs in bf16)
      if (b + 1 < s->nb)
        ln_ready = fuse_ln(s, E, M, d, s->F, s->mod, P(s->w.blk_mod, (int64_t)(b + 1) * 6 * d, es), 0, d, 6 * d,
                           sdk::LN_PLAIN);
      else
        ln_ready = fuse_ln(s, E, M, d, s->F, s->fmod, nullptr, 0, d, 2 * d, sdk::LN_SPLIT);
      // (with the LayerNorm fused: its output too, hi / lo pairs after the last block)
      PROF(SD_PROF_GEMM_FFN2, gflop(M, d, s->F),
           gbytes(M, d, s->F, es, 8) + (ln_ready ? (double)M * d * es * (b + 1 < s->nb ? 1 : 2) : 0.0),
           sdk::gemm(st, bf, s->hid, P(s->w.f2_w, (int64_t)b * d * s->F, es), M, d, s->F, E));
    }
  }

  // ---- adaptive sink: embedding of the exiting chunk, decision, predicated copy
  // one leaving chunk after the other, so that each decision sees the
  // embeddings the previous one left; the K / V^T of a refresh come from the
  // ring (B = 1: the chunk just appended at ptr_old) or from its staged copy
  for (int k = 0; k < nexit && s->S > 0; ++k) {
    PROF(SD_PROF_CONTROLS, 0.0, 4.0 * L * d,
         sdk::sink_score(st, s->resid + (int64_t)exit_rows[k] * L * d, s->sink_part, L, d, s->sink_emb, s->Ment,
                         cap_entry[k], c.sink_tau, s->sink_flag, s->sink_sim));
    if (cap_entry[k] < 0) {
      const bool staged = s->Cc > 0;
      PROF(SD_PROF_KV, 0.0, 4.0 * s->nb * s->Se * d * es,
           sdk::sink_copy(st, bf, s->sink_flag, staged ? s->candK : s->ringK, staged ? s->candVT : s->ringVT,
                          s->sinkK, s->sinkVT, s->nb, H, hd, staged ? s->Cc : s->Wt, s->S8,
                          staged ? k * s->Se : ptr_old, s->Se, staged ? nullptr : &dd->ptr_old));
    }
  }

  // ---- final layer and unpatchify -> eps_c
  // (bf16: the normalised rows as hi + lo pairs against the doubled head, K = 2d)
  const int KH = bf ? 2 * d : d;
  if (!ln_ready)
    PROF(SD_PROF_LN, 0.0, (4.0 + es * KH / d) * M * d,
         sdk::ln_mod(st, bf, s->resid, s->xm, M, d, L, s->fmod, nullptr, 0, d, 2 * d, 1e-6f,
                     bf ? sdk::LN_SPLIT : sdk::LN_PLAIN));
  {
    Epi E = epi_base(s, EPI_HEAD);
    E.bias = s->w.head_b;
    E.eps = eps_out;
    PROF(SD_PROF_OTHER, gflop(M, s->P, KH), gbytes(M, s->P, KH, es, 4),
         sdk::gemm(st, bf, s->xm, bf ? s->head2 : s->w.head_w, M, s->P, KH, E));
  }
  return SD_OK;
}

sd_status sd_stream_step(sd_stream* s, float* out_latent, sd_step_info* info) {
  if (!s) return SD_ERR_ARG;
  return sd_stream_step_chunks(s, s->B, out_latent, info);
}

sd_status sd_stream_step_chunks(sd_stream* s, int32_t chunks, float* out_latent, sd_step_info* info) {
  if (!s) return SD_ERR_ARG;
  const sd_stream_config& c = s->cfg;
  if (!info) return set_err(s, SD_ERR_ARG, "info is null");
  const int n = s->n, B = s->B;
  if (chunks < 1 || chunks > B) return set_err(s, SD_ERR_ARG, "chunks must be in [1, chunks_per_step]");
  if ((int)s->pending.size() < chunks) return set_err(s, SD_ERR_NOT_READY, "fewer pending chunks than requested");
  if (!s->ctx_set) return set_err(s, SD_ERR_STATE, "set_context() must be called first");
  const bool will_exit = (n == 1) || (s->slots[(n - 2) * B] >= 0);
  if (will_exit && !out_latent) return set_err(s, SD_ERR_ARG, "out_latent is null but frames leave this step");
  std::memset(info, 0, sizeof(*info));
  if (s->push_pending) {
    HIP_TRY(hipStreamWaitEvent(s->st, s->ev_push, 0));   // the entering chunks' records are written
    s->push_pending = false;
  }

  // ---- slot-group shift (the B oldest pending chunks enter slot 0) and row
  // table: slot by slot, the chunks of a slot in push order
  for (int i = n - 1; i >= 1; --i)
    for (int k = 0; k < B; ++k) s->slots[i * B + k] = s->slots[(i - 1) * B + k];
  for (int k = 0; k < B; ++k) {
    if (k < chunks) {
      s->slots[k] = s->pending.front();
      s->pending.pop_front();
    } else {
      s->slots[k] = -1;       // a smaller group leaves its upper lanes empty
    }
  }
  RowTable rt;
  std::memset(&rt, 0, sizeof(rt));
  int R = 0, nexit = 0;
  int exit_rows[SD_MAX_CHUNKS];
  for (int i = 0; i < n; ++i) {
    for (int k = 0; k < B; ++k) {
      const int f = s->slots[i * B + k];
      if (f < 0) continue;
      const FrameRec& fr = s->frames[f];
      RowInfo& ri = rt.r[R];
      ri.frame = f;
      ri.tau = fr.taus[i];
      ri.t0 = fr.t0;
      ri.kind = 0;
      ri.last = (i == n - 1);
      ri.ctx = 0;
      ri.a = (float)s->a[ri.tau];
      ri.b = (float)s->b[ri.tau];
      if (i + 1 < n) {
        ri.an = (float)s->a[fr.taus[i + 1]];
        ri.bn = (float)s->b[fr.taus[i + 1]];
      }
      ri.a0 = (float)s->a[fr.taus[0]];
      ri.b0 = (float)s->b[fr.taus[0]];
      ri.oidx = ri.last ? nexit : 0;
      ri.neg = -1;
      ri.pair = -1;
      ri.zrow = (s->fz && i + 1 < n) ? f * (n - 1) + i : -1;
      ri.keep = (i == n - 1 && c.kv_recompute) ? 1 : 0;
      if (ri.last) exit_rows[nexit++] = R;
      ++R;
    }
  }
  const int R_pos = R;
  int nneg = 0;
  if (c.cfg_type == SD_CFG_ONETIME) {
    // one negative-prompt row per entering chunk (rows 0 .. chunks-1 are slot 0)
    for (int k = 0; k < chunks; ++k) {
      rt.r[R] = rt.r[k];
      rt.r[R].kind = 1;
      rt.r[R].last = 0;
      rt.r[R].ctx = 1;
      rt.r[R].neg = -1;
      rt.r[k].neg = R;
      ++R;
      ++nneg;
    }
  } else if (c.cfg_type == SD_CFG_FULL) {
    // full CFG: a twin of every row under the negative prompt, same order
    for (int k = 0; k < R_pos; ++k) {
      rt.r[R] = rt.r[k];
      rt.r[R].kind = 1;
      rt.r[R].last = 0;
      rt.r[R].ctx = 1;
      rt.r[k].pair = R;
      ++R;
      ++nneg;
    }
  }
  rt.R = R;
  const int L = s->L;
  hipStream_t st = s->st;
  // sink plan of the leaving chunks, in push order: while entries are empty a
  // chunk captures the next one; later chunks take a refresh decision
  int cap_entry[SD_MAX_CHUNKS];
  int sink_count_after = s->sink_count;
  for (int k = 0; k < nexit; ++k)
    cap_entry[k] = (s->S > 0 && sink_count_after < s->Ment) ? sink_count_after++ : -1;
  const int ptr_old = s->kv_ptr;

  const ExitPlan plan{nexit, exit_rows, cap_entry, ptr_old};
  HIP_TRY(sdk::dyn_write(st, make_dyn(s, rt, nexit, ptr_old), s->dyn));
  // the forward (with clean-latent recompute it only reads the cache), then
  // R-CFG, x0 prediction, re-noise / emit
  auto forward_update = [&]() -> sd_status {
    const sd_status fs = run_forward(s, rt, s->dyn, R_pos, nneg, c.kv_recompute ? nullptr : &plan, s->eps);
    if (fs != SD_OK) return fs;
    PROF(SD_PROF_EPILOGUE, 12.0 * R * s->lat, 16.0 * R * s->lat,
         sdk::rcfg_update(st, &s->dyn->rt, R, s->fx, s->fx0s, s->eps, s->fz, out_latent, s->lat, (float)c.gamma,
                          (float)c.delta));
    return SD_OK;
  };
  if (graph_eligible(s)) {
    // everything the launch sequence depends on besides the device values
    std::vector<int64_t> key = {R, R_pos, nneg, nexit, chunks, s->sink_count, s->kv_valid,
                                (int64_t)(uintptr_t)out_latent};
    for (int k = 0; k < nexit; ++k) {
      key.push_back(exit_rows[k]);
      key.push_back(cap_entry[k]);
    }
    const sd_status gs = graph_run(s, key, forward_update);
    if (gs != SD_OK) return gs;
  } else {
    const sd_status fs = forward_update();
    if (fs != SD_OK) return fs;
  }

  // ---- clean-latent recompute: the leaving chunks' emitted latents (kept in
  // their frame records) go through one more forward at timestep 0 against
  // the same cache; its leaving rows take the cache and sink updates and its
  // eps lands after the main forward's rows
  int clean_rows = 0;
  if (c.kv_recompute && nexit > 0) {
    RowTable rc;
    std::memset(&rc, 0, sizeof(rc));
    int rows_c[SD_MAX_CHUNKS];
    for (int k = 0; k < nexit; ++k) {
      RowInfo& ri = rc.r[k];
      ri = rt.r[exit_rows[k]];
      ri.tau = 0;
      ri.a = (float)s->a[0];
      ri.b = (float)s->b[0];
      ri.neg = ri.pair = ri.zrow = -1;
      ri.keep = 0;
      rows_c[k] = k;
    }
    rc.R = nexit;
    const ExitPlan cplan{nexit, rows_c, cap_entry, ptr_old};
    HIP_TRY(sdk::dyn_write(st, make_dyn(s, rc, nexit, ptr_old), s->dyn + 1));
    const sd_status fs = run_forward(s, rc, s->dyn + 1, nexit, 0, &cplan, s->eps + (int64_t)R * s->lat);
    if (fs != SD_OK) return fs;
    clean_rows = nexit;
  }

  // ---- host bookkeeping
  info->step = s->n_steps++;
  info->rows = R + clean_rows;
  info->frame_id = -1;
  if (nexit > 0) {
    info->has_output = 1;
    info->n_out = nexit;
    info->frame_id = s->frames[s->slots[(n - 1) * B]].fid;
    for (int k = 0; k < B; ++k) {
      const int f = s->slots[(n - 1) * B + k];
      if (f >= 0) {
        s->frames[f].used = false;
        // a later push on the IO stream rewrites the record only after this step
        HIP_TRY(hipEventRecord(s->rec_ev[f], st));
        s->rec_ev_set[f] = 1;
      }
      s->slots[(n - 1) * B + k] = -1;
    }
    if (s->Wt > 0) {
      s->kv_ptr = (int)(((int64_t)s->kv_ptr + (int64_t)nexit * L) % s->Wt);
      s->kv_valid = std::min(s->Wt, s->kv_valid + nexit * L);
    }
    s->sink_count = sink_count_after;
  }
  info->kv_ptr = s->kv_ptr;
  info->kv_valid = s->kv_valid;
  info->sink_count = s->sink_count;
  info->rope_next = s->ctl.rope_p;
  return SD_OK;
}

sd_status sd_stream_set_graph(sd_stream* s, int32_t enable) {
  if (!s) return SD_ERR_ARG;
  if (enable && !s->st) return set_err(s, SD_ERR_STATE, "graph replay needs a created stream (not the null stream)");
  if (!enable) {
    HIP_TRY(hipStreamSynchronize(s->st));
    for (auto& g : s->graphs) (void)hipGraphExecDestroy(g.exec);
    s->graphs.clear();
  }
  s->graph_on = enable != 0;
  return SD_OK;
}

sd_status sd_stream_graph_stats(sd_stream* s, int64_t* captures, int64_t* replays) {
  if (!s || !captures || !replays) return SD_ERR_ARG;
  *captures = s->graph_captures;
  *replays = s->graph_replays;
  return SD_OK;
}

sd_status sd_stream_kv_reset(sd_stream* s) {
  if (!s) return SD_ERR_ARG;
  s->kv_ptr = 0;
  s->kv_valid = 0;
  s->sink_count = 0;
  s->ctl.rope_p = 0;
  return SD_OK;
}

sd_status sd_stream_sink_info(sd_stream* s, sd_sink_info* info) {
  if (!s || !info) return SD_ERR_ARG;
  int fl[4] = {};
  double sim = 0.0;
  HIP_TRY(hipMemcpyAsync(fl, s->sink_flag, sizeof(int) * 3, hipMemcpyDeviceToHost, s->st));
  HIP_TRY(hipMemcpyAsync(&sim, s->sink_sim, sizeof(double), hipMemcpyDeviceToHost, s->st));
  HIP_TRY(hipStreamSynchronize(s->st));
  info->refreshed = fl[0];
  info->entry = fl[1];
  info->evaluated = fl[2];
  info->sim = (float)sim;
  return SD_OK;
}

sd_status sd_stream_buffer(sd_stream* s, int32_t which, void** ptr, size_t* bytes) {
  if (!s || !ptr || !bytes) return SD_ERR_ARG;
  const size_t es = s->es;
  switch (which) {
    case SD_BUF_EPS: *ptr = s->eps; *bytes = (size_t)s->Rmax * s->lat * 4; break;
    case SD_BUF_RING_K: *ptr = s->ringK; *bytes = (size_t)s->nb * s->H * s->Wt * s->hd * es; break;
    case SD_BUF_RING_V: *ptr = s->ringVT; *bytes = (size_t)s->nb * s->H * s->Wt * s->hd * es; break;
    case SD_BUF_SINK_K: *ptr = s->sinkK; *bytes = (size_t)s->nb * s->H * s->S8 * s->hd * es; break;
    case SD_BUF_SINK_V: *ptr = s->sinkVT; *bytes = (size_t)s->nb * s->H * s->S8 * s->hd * es; break;
    case SD_BUF_RESID: *ptr = s->resid; *bytes = (size_t)s->Rmax * s->L * s->d * 4; break;
    case SD_BUF_MOD: *ptr = s->mod; *bytes = (size_t)s->Rmax * 6 * s->d * 4; break;
    default: return set_err(s, SD_ERR_ARG, "unknown buffer");
  }
  return SD_OK;
}

sd_status sd_stream_profile(sd_stream* s, uint32_t kind_mask) {
  if (!s) return SD_ERR_ARG;
  s->prof_mask = kind_mask;
  return SD_OK;
}

sd_status sd_stream_profile_read(sd_stream* s, sd_kernel_stat* out, int32_t n_max, int32_t* n_out) {
  if (!s || !out || !n_out || n_max < 1) return SD_ERR_ARG;
  if (s->io) HIP_TRY(hipStreamSynchronize(s->io));
  HIP_TRY(hipStreamSynchronize(s->st));
  for (int k = 0; k < SD_PROF_KINDS; ++k) s->prof_acc[k].kind = k;
  for (const auto& r : s->prof_pending) {
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, s->ev_pool[r.ev], s->ev_pool[r.ev + 1]));
    sd_kernel_stat& a = s->prof_acc[r.kind];
    a.launches += 1;
    a.ms += ms;
    a.flops += r.flops;
    a.bytes += r.bytes;
  }
  s->prof_pending.clear();
  s->ev_used = 0;
  int n = 0;
  for (int k = 0; k < SD_PROF_KINDS && n < n_max; ++k)
    if (s->prof_acc[k].launches > 0) out[n++] = s->prof_acc[k];
  *n_out = n;
  std::memset(s->prof_acc, 0, sizeof(s->prof_acc));
  return SD_OK;
}

sd_status sd_stream_set_io_stream(sd_stream* s, void* io_stream) {
  if (!s) return SD_ERR_ARG;
  if (s->io && (hipStream_t)io_stream != s->io) {
    // later steps no longer wait on ev_push: let the switch wait for the old queue
    HIP_TRY(hipStreamSynchronize(s->io));
  }
  s->io = (hipStream_t)io_stream;
  return SD_OK;
}

void sd_stream_destroy(sd_stream* s) { delete s; }

const char* sd_stream_last_error(const sd_stream* s) { return s ? s->err.c_str() : "null stream"; }

}  // extern "C"
