// One 16-byte chunk of the KV append (bf16, token ranges multiples of 8):
// chunk i < H L hd / 8 copies 8 head-dim elements of one K row of the own
// chunk to the ring (and the sink entry being captured), the rest 8
// consecutive tokens of one V^T row.  Shared by the append kernel and the
// launch that runs the append beside the attention's combine pass.
#pragma once
#include "common.h"

namespace sdk {

struct KvAppendArgs {
  const bf16* kown;
  const bf16* vtown;
  int64_t k_hs, vt_ps;
  bf16* ringK;
  bf16* ringVT;
  int H, hd, L, W, ptr;
  bf16* sinkK;
  bf16* sinkVT;
  int S8, sink_off, Se;
  const int* ptr_dev;   // when set, the ring position is read from here
};

SD_DEV void kv_append_chunk(const KvAppendArgs& a, int64_t i) {
  const int ptr = a.ptr_dev ? *a.ptr_dev : a.ptr;
  const int64_t nk = (int64_t)a.H * a.L * (a.hd / 8);
  if (i >= 2 * nk) return;
  if (i < nk) {
    const int c = (int)(i % (a.hd / 8));
    const int64_t ht = i / (a.hd / 8);
    const int h = (int)(ht / a.L), t = (int)(ht % a.L);
    const bf16x8 v = *(const bf16x8*)(a.kown + h * a.k_hs + (int64_t)t * a.hd + c * 8);
    if (a.W > 0) {
      int p = ptr + t;
      if (p >= a.W) p -= a.W;
      *(bf16x8*)(a.ringK + ((int64_t)h * a.W + p) * a.hd + c * 8) = v;
    }
    if (a.sinkK && t < a.Se) *(bf16x8*)(a.sinkK + ((int64_t)h * a.S8 + a.sink_off + t) * a.hd + c * 8) = v;
  } else {
    i -= nk;
    const int tc = (int)(i % (a.L / 8));
    const int64_t he = i / (a.L / 8);          // h * hd + e
    const int t = tc * 8;
    const bf16x8 v = *(const bf16x8*)(a.vtown + he * a.vt_ps + t);
    if (a.W > 0) {
      int p = ptr + t;
      if (p >= a.W) p -= a.W;
      *(bf16x8*)(a.ringVT + he * a.W + p) = v;
    }
    if (a.sinkVT && t < a.Se) *(bf16x8*)(a.sinkVT + he * a.S8 + a.sink_off + t) = v;
  }
}

}  // namespace sdk
