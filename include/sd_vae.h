/* Stream-VAE: chunked causal video encoder / decoder for gfx950
 * (StreamDiffusionV2 summary, Stream-VAE: a low-latency VAE variant that
 * processes short chunks of frames and caches intermediate features inside
 * every 3D convolution to keep consecutive chunks temporally coherent).
 *
 * Network (the pages give no architecture; the reading, with random weights):
 * every convolution is causal 3x3x3 (output frame t reads input frames t-2,
 * t-1, t; frames before the chunk come from the layer's cache of the previous
 * chunk's last two input frames, zeros after create / reset), followed on the
 * inner layers by RMS normalisation over channels (gain) and SiLU.
 *   encoder: conv 8->c1 | pool 2x2, conv c1->c2 | pool 2x2, conv c2->c3 |
 *            pool 2x2x2, conv c3->c3 | conv c3->latent_c
 *   decoder: conv latent_c->c3 | up 2x2x2, conv c3->c3 | up 2x2, conv c3->c2 |
 *            up 2x2, conv c2->c1 | conv c1->3
 * A chunk is 2*latent_t frames of (8 latent_h) x (8 latent_w) RGB pixels and
 * latent_t x latent_c x latent_h x latent_w latents.
 *
 * Memory: the library allocates nothing; the caller provides weights (device,
 * bf16) and a workspace of sd_vae_workspace_bytes() (device, 256-byte
 * aligned), which holds two input buffers per layer (used on alternate
 * chunks: the other one still holds the previous chunk's frames, which are
 * the layer's cache), a staging buffer and an fp16 copy of the convolution
 * weights made at create (activations and caches are stored in fp16; the
 * weights must not change while the handle lives).  Calls are
 * asynchronous on the stream given at create; encode and decode keep separate
 * caches and must each be fed the chunks of one stream in order.
 */
#ifndef SD_VAE_H
#define SD_VAE_H

#include <stddef.h>
#include <stdint.h>

#include "sd_stream.h"

#ifdef __cplusplus
extern "C" {
#endif

#define SD_VAE_ABI_VERSION 1

/* conv layers, in the order of the weight arrays */
typedef enum {
  SD_VAE_E0 = 0, SD_VAE_E1, SD_VAE_E2, SD_VAE_E3, SD_VAE_E_OUT,
  SD_VAE_D0, SD_VAE_D1, SD_VAE_D2, SD_VAE_D3, SD_VAE_D_OUT,
  SD_VAE_LAYERS
} sd_vae_layer;

typedef struct {
  uint32_t abi_version;            /* must be SD_VAE_ABI_VERSION */
  int32_t latent_t;                /* latent frames per chunk, >= 2 (pixel frames 2 latent_t) */
  int32_t latent_c;                /* latent channels: a multiple of 8, at most 16 */
  int32_t latent_h, latent_w;      /* latent grid (pixels 8x larger), >= 1 */
  int32_t c1, c2, c3;              /* channel widths from the pixel side in: 16, 32, 64, 128 or 256 */
} sd_vae_config;

/* Per layer: w [Cout][3][3][3][Cin] (taps (dt, dy, dx)), b [Cout], g [Cout]
 * (norm gain; NULL for SD_VAE_E_OUT and SD_VAE_D_OUT), all bf16 device
 * arrays, 16-byte aligned.  The encoder's first layer has Cin = 8: the input
 * RGB is padded with 5 zero channels. */
typedef struct {
  const void* w[SD_VAE_LAYERS];
  const void* b[SD_VAE_LAYERS];
  const void* g[SD_VAE_LAYERS];
} sd_vae_weights;

typedef struct sd_vae sd_vae;

/* 0 if cfg is invalid. */
size_t sd_vae_workspace_bytes(const sd_vae_config* cfg);

/* Validate, carve the workspace, zero the caches.  hip_stream is a
 * hipStream_t (NULL = default stream). */
sd_status sd_vae_create(const sd_vae_config* cfg, const sd_vae_weights* w, void* workspace, size_t workspace_bytes,
                        void* hip_stream, sd_vae** out);

/* One chunk: pixels fp32 [2 latent_t][3][8 latent_h][8 latent_w] (device) ->
 * latent fp32 [latent_t][latent_c][latent_h][latent_w] (device). */
sd_status sd_vae_encode(sd_vae* v, const float* pixels, float* latent);

/* One chunk: latent fp32 [latent_t][latent_c][latent_h][latent_w] ->
 * pixels fp32 [2 latent_t][3][8 latent_h][8 latent_w]. */
sd_status sd_vae_decode(sd_vae* v, const float* latent, float* pixels);

/* Zero both sets of caches (a new video starts). */
sd_status sd_vae_reset(sd_vae* v);

void sd_vae_destroy(sd_vae* v);
const char* sd_vae_last_error(const sd_vae* v);

#ifdef __cplusplus
}
#endif
#endif
