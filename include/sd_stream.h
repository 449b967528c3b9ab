/*
 * sd_stream.h -- C ABI of the Stream Batch denoising library for MI355X (gfx950).
 *
 * One Stream Batch iteration (StreamDiffusion paper notes, section 1 "Stream
 * Batch"): n frames that sit at n different denoising steps are stacked into
 * one batch and advanced by a single denoiser forward; a frame that enters at
 * step t leaves n steps later.  The denoiser is a DiT whose self-attention
 * reads a sink-token plus rolling-window KV cache with a RoPE phase reset
 * (StreamDiffusionV2 summary: "sink-token guided rolling KV cache",
 * "adaptive sink and RoPE refresh").  The forward is followed by the Residual
 * CFG estimate and the per-slot latent update (StreamDiffusion paper notes,
 * section 2 "R-CFG"), and the per-frame controls: the Stochastic Similarity
 * Filter (section 3 "SSF"; the max_skip_frame cap of the project intro's usage
 * section), the motion-aware noise rate (StreamDiffusionV2 summary, "motion-aware
 * noise scheduler") and the adaptive sink refresh.
 *
 * The calls mirror the pages' problem statement: a stream is prepared once
 * (create + set_context: the project intro's prepare(prompt), with the
 * prompt-side attention K/V pre-computed, feature 5 "Pre-Computation for
 * KV-Caches"), then frames are pushed one at a time (the intro's stream(image))
 * and each step advances the pipeline by one denoising step.
 *
 * Conventions
 * -----------
 * - Every call returns sd_status (0 = OK, < 0 = error); no exceptions cross
 *   the ABI.  After an error, sd_stream_last_error() describes it.
 * - Arguments are validated before any HIP call; a failed validation leaves
 *   the stream unchanged.
 * - Memory: the caller allocates all device memory (weights, workspace,
 *   inputs, outputs) and keeps it alive for the lifetime of the handle (weights,
 *   workspace) or the call (inputs, outputs).  The library allocates no device
 *   memory; it owns only the opaque host-side handle.
 * - Streams: all device work is ordered on the hipStream_t given at create.
 *   push_frame synchronises that stream once to read back a few bytes (SSF
 *   sums, motion sums); step never synchronises.
 * - Latents cross the boundary as fp32 [T][C][H][W]; internal precision
 *   follows config.dtype.
 * - A handle is not thread-safe; separate handles are independent.
 */
#ifndef SD_STREAM_H
#define SD_STREAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SD_ABI_VERSION 4
#define SD_MAX_SLOTS 8       /* n, denoising steps in flight */
#define SD_MAX_ROWS 40       /* rows per step: B*n (+B onetime-negative, 2*B*n full CFG; +B kv_recompute) */
#define SD_MAX_CHUNKS 8      /* chunks per step (B) */
#define SD_MAX_SINK 8        /* sink entries M */

typedef enum {
  SD_OK = 0,
  SD_ERR_ARG = -1,        /* null pointer, out-of-range value */
  SD_ERR_SHAPE = -2,      /* inconsistent dimensions */
  SD_ERR_STATE = -3,      /* call not valid in the current state (e.g. queue full) */
  SD_ERR_WORKSPACE = -4,  /* workspace too small or misaligned */
  SD_ERR_HIP = -5,        /* a HIP runtime call failed */
  SD_ERR_NOT_READY = -6   /* step() with no pending frame */
} sd_status;

typedef enum { SD_DTYPE_F32 = 0, SD_DTYPE_BF16 = 1 } sd_dtype;
/* Guidance variants (StreamDiffusion paper notes, section 2): self-negative
 * R-CFG uses the frame's own input latent as x0*; onetime-negative R-CFG adds
 * one forward of the entering frame under the negative prompt and uses its x0
 * estimate; full CFG, the standard guidance R-CFG replaces, gives every row a
 * twin under the negative prompt (2n rows) whose prediction takes the place of
 * the virtual residual (with delta = 1: eps_u + gamma (eps_c - eps_u)). */
typedef enum { SD_CFG_SELF = 0, SD_CFG_ONETIME = 1, SD_CFG_FULL = 2 } sd_cfg_type;
typedef enum { SD_SSF_U8 = 0, SD_SSF_LATENT = 1 } sd_ssf_kind;
/* Per-slot latent update.  The pages name no sampler.  DDIM (eta = 0) hands
 * the next slot a_next x0_hat + b_next eps_cfg; the LCM-style update (the
 * pages pair the pipeline with LCM models) re-noises with fresh noise,
 * a_next x0_hat + b_next z, z given with the frame for each later slot. */
typedef enum { SD_SAMPLER_DDIM = 0, SD_SAMPLER_LCM = 1 } sd_sampler;

typedef struct {
  uint32_t abi_version;            /* must be SD_ABI_VERSION */
  int32_t dtype;                   /* sd_dtype: weights, activations, KV cache */
  /* latent chunk geometry [T][C][H][W]; patch is 1 x patch x patch */
  int32_t latent_t, latent_c, latent_h, latent_w, patch;
  /* denoiser */
  int32_t n_blocks, d_model, n_heads, d_ffn, d_freq;
  int32_t ctx_len;                 /* prompt tokens; 0 = no cross-attention */
  /* stream batch */
  int32_t n_slots;                 /* n = number of denoising steps in flight */
  int32_t t_index[SD_MAX_SLOTS];   /* 50-step grid index per slot: tau = 999 - 20 k */
  int32_t chunks_per_step;         /* B in [1, SD_MAX_CHUNKS]: chunks that enter (and leave)
                                      together; B*n rows (+B for onetime R-CFG, x2 for
                                      full CFG) <= SD_MAX_ROWS */
  int32_t cfg_type;                /* sd_cfg_type */
  double gamma, delta;             /* R-CFG guidance scale and residual weight */
  /* KV cache, in tokens */
  int32_t sink_tokens;             /* S, split into sink_entries entries */
  int32_t sink_entries;            /* M >= 1 when S > 0 */
  int32_t window_tokens;           /* W (0 or >= tokens per chunk) */
  double sink_tau;                 /* refresh iff cosine < sink_tau */
  int32_t rope_reset;              /* temporal RoPE position restarts past this */
  double rope_base;
  /* scaled-linear schedule */
  int32_t n_train_steps;
  double beta_start, beta_end;
  /* stochastic similarity filter */
  int32_t ssf_on, ssf_kind;        /* sd_ssf_kind */
  int32_t ssf_h, ssf_w, ssf_c;     /* uint8 frame shape [h][w][c] for SD_SSF_U8 */
  double ssf_eta;                  /* similarity threshold eta < 1 */
  int32_t max_skip_frame;          /* at most this many consecutive skips */
  /* motion-aware noise rate */
  int32_t motion_on, motion_k;
  double motion_lambda, s_min, s_max, motion_sigma;
  /* cross-frame batch attention (StreamDiffusion paper notes, section 1,
   * temporal consistency): every row's queries attend to [sink | window |
   * the own tokens of every row of the forward] instead of [sink | window |
   * its own tokens].  Self-negative R-CFG only (the rows share one prompt). */
  int32_t batch_attn;
  int32_t sampler;                 /* sd_sampler */
  /* clean-latent KV recompute: the K/V a leaving chunk appends to the cache
   * (and the hidden state of its sink decision) come from one more forward of
   * its emitted latent at timestep 0 against the same cache, instead of from
   * its last denoising forward; + B rows per step */
  int32_t kv_recompute;
} sd_stream_config;

/*
 * Denoiser weights: device pointers owned by the caller, element type =
 * config.dtype (fp32, or bf16 stored as uint16).  Linear weights are
 * [out][in] row-major; tensors marked [nb] hold all blocks contiguously.
 * Cross-attention pointers may be NULL when ctx_len == 0.
 */
typedef struct {
  const void *t_w1, *t_b1;     /* [d][d_freq], [d]   timestep MLP, layer 1 */
  const void *t_w2, *t_b2;     /* [d][d], [d]        timestep MLP, layer 2 */
  const void *mod_w, *mod_b;   /* [6d][d], [6d]      shared adaLN projection */
  const void *blk_mod;         /* [nb][6d]           per-block modulation table */
  const void *pe_w, *pe_b;     /* [d][p*p*C], [d]    patch embedding */
  const void *qkv_w, *qkv_b;   /* [nb][3d][d], [nb][3d] */
  const void *o_w, *o_b;       /* [nb][d][d], [nb][d] */
  const void *cq_w, *cq_b;     /* [nb][d][d], [nb][d]      cross-attention query */
  const void *ckv_w, *ckv_b;   /* [nb][2d][d], [nb][2d]    prompt-side K/V */
  const void *co_w, *co_b;     /* [nb][d][d], [nb][d]      cross-attention output */
  const void *f1_w, *f1_b;     /* [nb][F][d], [nb][F] */
  const void *f2_w, *f2_b;     /* [nb][d][F], [nb][d] */
  const void *fin_w, *fin_b;   /* [2d][d], [2d]      final (shift, scale) */
  const void *head_w, *head_b; /* [p*p*C][d], [p*p*C] */
} sd_weights;

typedef struct {
  int32_t skipped;             /* 1: frame dropped by the SSF, nothing queued */
  int32_t t0;                  /* temporal RoPE base assigned to the chunk (-1 if skipped) */
  int64_t frame_id;            /* id of the queued frame (-1 if skipped) */
  double sim;                  /* SSF cosine similarity to the reference (1 if first) */
  double p;                    /* SSF skip probability */
  double d;                    /* last motion distance (RMS, latent units) */
  double s;                    /* noise rate after this push */
  int32_t taus[SD_MAX_SLOTS];  /* timestep per slot for this frame */
} sd_push_info;

typedef struct {
  int64_t step;                /* index of this step */
  int32_t has_output;          /* 1 if a frame left the pipeline */
  int32_t rows;                /* rows in the forward */
  int64_t frame_id;            /* id of the emitted frame (-1 if none) */
  int32_t kv_ptr, kv_valid;    /* ring write position and valid tokens after the step */
  int32_t sink_count;          /* filled sink entries after the step */
  int32_t rope_next;           /* next temporal RoPE base */
  int32_t n_out;               /* frames emitted: B when a slot group leaves, else 0;
                                  frame_id is the first, the others follow in push order */
} sd_step_info;

/* Result of the last adaptive sink decision (read back on request). */
typedef struct {
  int32_t evaluated;           /* 1 if the last exiting chunk met a full sink set */
  int32_t entry;               /* least similar entry j* */
  int32_t refreshed;           /* 1 if entry j* was overwritten */
  float sim;                   /* cosine of entry j* */
} sd_sink_info;

typedef struct sd_stream sd_stream;

/* Bytes of device workspace the stream needs (256-byte aligned base). 0 on an
 * invalid config. */
size_t sd_stream_workspace_bytes(const sd_stream_config* cfg);

/* Validate cfg, carve the workspace, build the schedule and RoPE tables and
 * zero the state.  hip_stream is a hipStream_t (NULL = default stream).
 * In bf16 the workspace also receives copies of some weights made here: the
 * patch-embedding and head weights side by side twice (their fp32 inputs are
 * read as hi + lo bf16 pairs), and, when a chunk has at most 256 tokens, the
 * block weights rearranged for the few-row product (sd_k_pack_weight).  A
 * caller that changes the weights afterwards creates the stream again. */
sd_status sd_stream_create(const sd_stream_config* cfg, const sd_weights* w, void* workspace,
                           size_t workspace_bytes, void* hip_stream, sd_stream** out);

/* Pre-compute the prompt-side cross-attention K/V of every block from the
 * positive (and, for onetime-negative, negative) context, [ctx_len][d] device
 * arrays of config.dtype.  Required before the first step when ctx_len > 0. */
sd_status sd_stream_set_context(sd_stream* s, const void* ctx_pos, const void* ctx_neg);

/* Offer one chunk.  x0 and noise are device fp32 [T][C][H][W] (noise ~ N(0,1),
 * the entry noise of this frame; with SD_SAMPLER_LCM noise is [n][T][C][H][W]:
 * the entry noise, then the noise slots 1 .. n-1 re-noise with, copied into
 * the frame store); ssf_frame is a device uint8 [h][w][c] image
 * for SD_SSF_U8 (ignored otherwise); u is the host uniform in [0,1) for the
 * SSF draw.  A skipped frame changes nothing but the skip counter. */
sd_status sd_stream_push_frame(sd_stream* s, const float* x0, const float* noise,
                               const void* ssf_frame, double u, sd_push_info* info);

/* IO queue (StreamDiffusion project intro: input and output queues that decouple
 * frame arrival from the denoising loop).  With io_stream set (a hipStream_t of
 * default priority), push_frame reads its inputs and runs all of its work there:
 * the SSF / motion reductions (the only part the host waits for), the reference
 * copies and the entry noise into a frame record.  The write of a frame record
 * first waits, on the device, for the step that last read that record, and the
 * next step waits for the push, so the pushes of the next chunk overlap the
 * forward of the current step on one GPU.  The caller produces x0, noise and
 * ssf_frame on io_stream (or before the call) and keeps io_stream alive while
 * it is set.  NULL (the default) runs pushes on the stream given at create;
 * switching queues first waits for the old one. */
sd_status sd_stream_set_io_stream(sd_stream* s, void* io_stream);

/* Graph replay of the step (StreamDiffusion project intro and StreamDiffusionV2
 * summary, system-level co-design: the denoising loop runs as one launch
 * sequence that the host re-issues every step).  With enable != 0, the forward
 * and the latent update of a step are captured once as a HIP graph and then
 * replayed: the values that change from step to step (the rows, their RoPE
 * bases, the window range, the ring positions of the appends) are written to
 * device memory by one small kernel first and read there by the kernels, so
 * a replay launches the whole step at once.  A graph is recorded per launch
 * sequence (rows, exits, sink state, window fill, output buffer); up to four
 * are kept.  Applies to bf16 configurations without kv_recompute, with no IO
 * queue set and no live profiling (otherwise the step is launched as usual);
 * needs a created stream (SD_ERR_STATE on the null stream).  Results equal
 * those of the launched step.  enable == 0 (the default) waits for the stream
 * and frees the graphs. */
sd_status sd_stream_set_graph(sd_stream* s, int32_t enable);
/* Steps that recorded a new graph and steps that replayed one. */
sd_status sd_stream_graph_stats(sd_stream* s, int64_t* captures, int64_t* replays);

/* Advance the pipeline by one denoising step (Stream Batch: the B oldest
 * pending chunks enter slot 0, every slot advances one timestep, the slot
 * group in the last slot leaves).  SD_ERR_NOT_READY while fewer than B chunks
 * are pending.  When a group leaves, the clean latent estimates of its B
 * chunks are written to out_latent (device fp32 [B][T][C][H][W], push order);
 * out_latent may be NULL on steps that emit nothing. */
sd_status sd_stream_step(sd_stream* s, float* out_latent, sd_step_info* info);

/* sd_stream_step with a group of `chunks` (1 <= chunks <= chunks_per_step)
 * entering instead of B: groups of different sizes travel through the slots
 * and each leaves whole (n_out = its size), so a host scheduler can change
 * the batch from step to step (StreamDiffusionV2 summary, SLO-aware batching
 * scheduler).  SD_ERR_NOT_READY while fewer than `chunks` are pending;
 * SD_ERR_ARG for chunks outside the range.  out_latent holds at least
 * chunks_per_step latents. */
sd_status sd_stream_step_chunks(sd_stream* s, int32_t chunks, float* out_latent, sd_step_info* info);

/* Clear the ring, the sink and the RoPE counter (frames in flight continue). */
sd_status sd_stream_kv_reset(sd_stream* s);

/* Synchronise the stream and report the last adaptive sink decision. */
sd_status sd_stream_sink_info(sd_stream* s, sd_sink_info* info);

/* Device views of internal buffers, for inspection by tests. */
typedef enum {
  SD_BUF_EPS = 0,      /* fp32 [rows][T*C*H*W] denoiser output of the last step, row order of the forward */
  SD_BUF_RING_K = 1,   /* [nb][H][W][hd] dtype, token at ring position w */
  SD_BUF_RING_V = 2,   /* [nb][H][hd][W] dtype (V stored transposed) */
  SD_BUF_SINK_K = 3,   /* [nb][H][S8][hd] dtype, S8 = S rounded up to 8, entry j at j*S/M */
  SD_BUF_SINK_V = 4,   /* [nb][H][hd][S8] dtype */
  SD_BUF_RESID = 5,    /* fp32 [rows*L][d] residual stream after the last block */
  SD_BUF_MOD = 6       /* fp32 [rows][6d] shared modulation of the last step */
} sd_buffer;
sd_status sd_stream_buffer(sd_stream* s, int32_t which, void** ptr, size_t* bytes);

/* Live kernel timing.  For every kernel kind whose bit is set in kind_mask,
 * each launch is bracketed by HIP events on the stream; profile_read
 * synchronises, returns per-kind totals (launches, milliseconds and the
 * algorithmic flops and bytes of those launches) since the previous read, and
 * resets them.  Events are created on first use and reused. */
typedef enum {
  SD_PROF_ATTN_SELF = 0, SD_PROF_ATTN_CROSS = 1, SD_PROF_GEMM_QKV = 2, SD_PROF_GEMM_O = 3,
  SD_PROF_GEMM_FFN1 = 4, SD_PROF_GEMM_FFN2 = 5, SD_PROF_GEMM_CROSS = 6, SD_PROF_OTHER = 7,
  SD_PROF_LN = 8, SD_PROF_GEMV = 9, SD_PROF_KV = 10, SD_PROF_EPILOGUE = 11, SD_PROF_CONTROLS = 12,
  SD_PROF_ATTN_COMBINE = 13, SD_PROF_KINDS = 14
} sd_prof_kind;
typedef struct {
  int32_t kind;
  int32_t reserved;
  int64_t launches;
  double ms;                   /* summed event time */
  double flops;                /* summed algorithmic flops */
  double bytes;                /* summed algorithmic bytes */
} sd_kernel_stat;
sd_status sd_stream_profile(sd_stream* s, uint32_t kind_mask);
sd_status sd_stream_profile_read(sd_stream* s, sd_kernel_stat* out, int32_t n_max, int32_t* n_out);

void sd_stream_destroy(sd_stream* s);
const char* sd_stream_last_error(const sd_stream* s);

#ifdef __cplusplus
}
#endif
#endif /* SD_STREAM_H */
