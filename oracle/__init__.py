"""CPU oracle for the Stream Batch hot path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct NumPy implementation of what one Stream
Batch denoising iteration computes, written from the pages:

* StreamDiffusion paper notes ("StreamDiffusion: A Pipeline-level Solution
  for Real-time Interactive Generation"): section 1 Stream Batch, section 2
  R-CFG (virtual residual noise and the combine equation, self- and
  onetime-negative), section 3 SSF (skip probability).
* StreamDiffusion project intro ("StreamDiffusion 完全解析"): the usage example
  (t_index_list, cfg_type, max_skip_frame) and the KV pre-computation feature.
* StreamDiffusionV2 summary pages: sink-token rolling KV cache, adaptive sink
  and RoPE refresh, motion-aware noise scheduler.

Floating point is fp64 unless a caller asks for fp32 (large video shapes).
Integer decisions (SSF skip, timestep indices, ring bookkeeping) are exact.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never does, and this
package never imports the GPU library: they share nothing but the seeded
input generators in ``workloads``.

Parity status per function is listed in each module's header.  The whole
denoiser forward (``dit.forward_row``) is "parity unpinned" as a whole: the
pages print no worked example and the weights are random; its parts are
pinned one by one (LayerNorm, GELU, linear, RoPE, attention, modulation).
"""
