// Attention over the sink + rolling-window KV cache (StreamDiffusionV2
// summary: sink-token guided rolling KV cache), flash-style online softmax.
//
// The keys of one (row, head) form a virtual sequence made of up to three
// segments -- sink, valid ring window, the row's own chunk (or the prompt
// context for cross-attention).  Each segment is padded to a multiple of 8
// keys; padding keys are masked.  A segment may wrap (the ring).  K is stored
// [pos][hd], V transposed [hd][pos].
//
// bf16 path: one workgroup = 4 waves = 128 queries of one (row, head); key
// tiles of 64 staged in LDS (double buffered).  Scores are computed
// transposed, S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so each lane owns one
// query's scores and the softmax statistics stay in-lane (one cross-half
// shuffle per tile).  K rows are loaded in a permuted order (bits 2 and 3 of
// the row index swapped) so that the score accumulators are directly the B
// operand of O^T = V^T P^T with 8 consecutive keys per lane.
// fp32 path: one thread per query on the vector ALUs.
#include <cmath>

#include "kernels.h"

namespace sdk {

struct SegRt {
  int begin[3];     // virtual index where the segment starts
  int count[3];
  int end[3];       // begin + padded count
};

SD_DEV SegRt seg_layout(const AttnArgs& a) {
  SegRt s;
  int v = 0;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int c = i < a.nseg ? a.seg[i].count : 0;
    s.begin[i] = v;
    s.count[i] = c;
    v += (c + 7) & ~7;
    s.end[i] = v;
  }
  return s;
}

SD_DEV bool key_valid(const SegRt& s, int j) {
  return (j < s.begin[0] + s.count[0]) || (j >= s.begin[1] && j < s.begin[1] + s.count[1]) ||
         (j >= s.begin[2] && j < s.begin[2] + s.count[2]);
}

// Physical position and segment of virtual key j (j inside a segment's padded range).
SD_DEV int key_seg(const SegRt& s, int j) { return j < s.end[0] ? 0 : (j < s.end[1] ? 1 : 2); }

// Segment s of the launch, selected without dynamic indexing of the argument.
SD_DEV KvSeg seg_pick(const AttnArgs& a, int s) { return s == 0 ? a.seg[0] : (s == 1 ? a.seg[1] : a.seg[2]); }

SD_DEV int key_pos(const KvSeg& g, int u) {
  const int p = g.start + u;
  return g.wrap ? p % g.cap : p;
}

// ---------------------------------------------------------------------------
// ONESEG = 1 instantiates the same code for single-segment calls (the
// prompt cross-attention), so that profiles tell the two uses apart.
template <int HD, int ONESEG>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnArgs a) {
  constexpr int BQ = 128, KB = 64, PK = 8, PV = 8;
  constexpr int LK = HD + PK, LV = KB + PV;
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][KB * LK];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][HD * LV];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // logical order (row, head, q-tile) with q-tiles fastest; all q-tiles of a
  // (row, head) share its keys, so they are kept on one XCD
  const int nqt = (a.L + BQ - 1) / BQ;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  // order (row, head, split, q-tile): the workgroups resident on one XCD at
  // a time are q-tiles of the same key range, which then streams through L2
  const int qt = lid % nqt, sp = (lid / nqt) % a.nsplit;
  const int h = (lid / (nqt * a.nsplit)) % a.H, r = a.r0 + lid / (nqt * a.nsplit * a.H);
  const int q0 = qt * BQ;
  const SegRt sr = seg_layout(a);
  const int NK = sr.end[2];
  const int NT_all = (NK + KB - 1) / KB;
  const int tps = (NT_all + a.nsplit - 1) / a.nsplit;
  const int T0 = min(NT_all, sp * tps), NT = min(NT_all, T0 + tps);   // this split's key tiles [T0, NT)

  // Q fragments (B operand): lane -> query q0 + wave*32 + lane%32, hd block
  // kk*16 + 8*(lane/32).
  const int myq = q0 + wave * 32 + (lane & 31);
  bf16x8 qf[HD / 16];
  {
    const bf16* qp = (const bf16*)a.q + (int64_t)r * a.q_rs + (int64_t)h * a.q_hs + (int64_t)myq * HD;
    const bf16x8 z = {};
#pragma unroll
    for (int kk = 0; kk < HD / 16; ++kk)
      qf[kk] = (myq < a.L) ? *(const bf16x8*)(qp + kk * 16 + 8 * (lane >> 5)) : z;
  }

  // Tile loaders: K tile KB x HD (HD/8 chunks per key), V^T tile HD x KB
  // (KB/8 chunks per hd row).  Chunks per thread:
  constexpr int CK = KB * (HD / 8) / 256, CV = HD * (KB / 8) / 256;
  bf16x8 rk[CK > 0 ? CK : 1], rv[CV > 0 ? CV : 1];
  auto gload = [&](int tile) {
    const bf16x8 z = {};
    // Fast path (all but a few tiles of a row): the whole tile is valid keys
    // of one segment at contiguous positions.  Everything below is uniform
    // over the workgroup.
    {
      const int jb = tile * KB;
      const int s0 = key_seg(sr, jb);
      const int b0 = s0 == 0 ? sr.begin[0] : (s0 == 1 ? sr.begin[1] : sr.begin[2]);
      const KvSeg g = seg_pick(a, s0);
      const int u0 = jb - b0;
      int p0 = g.start + u0;
      if (g.wrap && p0 >= g.cap) p0 -= g.cap;
      if (u0 + KB <= g.count && p0 + KB <= g.cap) {
        const bf16* kb = (const bf16*)g.k + (int64_t)r * g.k_rs + (int64_t)h * g.k_hs + (int64_t)p0 * HD;
        const bf16* vb = (const bf16*)g.vt + (int64_t)r * g.vt_rs + (int64_t)h * g.vt_hs + p0;
#pragma unroll
        for (int i = 0; i < CK; ++i) {
          const int c = tid + i * 256, key = c / (HD / 8), e0 = (c % (HD / 8)) * 8;
          rk[i] = *(const bf16x8*)(kb + key * HD + e0);
        }
#pragma unroll
        for (int i = 0; i < CV; ++i) {
          const int c = tid + i * 256, e = c / (KB / 8), k0 = (c % (KB / 8)) * 8;
          rv[i] = *(const bf16x8*)(vb + (int64_t)e * g.cap + k0);
        }
        return;
      }
    }
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      const int c = tid + i * 256, key = c / (HD / 8), e0 = (c % (HD / 8)) * 8;
      const int j = tile * KB + key;
      bf16x8 v = z;
      if (j < NK) {
        const int s = key_seg(sr, j);
        const KvSeg g = seg_pick(a, s);
        const int u = j - (s == 0 ? sr.begin[0] : (s == 1 ? sr.begin[1] : sr.begin[2]));
        // padding keys are never loaded (their scores are masked)
        if (u < g.count) {
          const int pos = key_pos(g, u);
          const bf16* kp = (const bf16*)g.k + (int64_t)r * g.k_rs + (int64_t)h * g.k_hs;
          v = *(const bf16x8*)(kp + (int64_t)pos * HD + e0);
        }
      }
      rk[i] = v;
    }
#pragma unroll
    for (int i = 0; i < CV; ++i) {
      const int c = tid + i * 256, e = c / (KB / 8), k0 = (c % (KB / 8)) * 8;
      const int j = tile * KB + k0;
      bf16x8 v = z;
      if (j < NK) {
        const int s = key_seg(sr, j);
        const KvSeg g = seg_pick(a, s);
        const int u = j - (s == 0 ? sr.begin[0] : (s == 1 ? sr.begin[1] : sr.begin[2]));
        // a chunk that starts inside the valid range may end in the zero-filled
        // padding of its segment's storage (capacity is a multiple of 8)
        if (u < g.count) {
          const int pos = key_pos(g, u);
          const bf16* vp = (const bf16*)g.vt + (int64_t)r * g.vt_rs + (int64_t)h * g.vt_hs;
          v = *(const bf16x8*)(vp + (int64_t)e * g.cap + pos);
        }
      }
      rv[i] = v;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      const int c = tid + i * 256, key = c / (HD / 8), e0 = (c % (HD / 8)) * 8;
      *(bf16x8*)&Ks[buf][key * LK + e0] = rk[i];
    }
#pragma unroll
    for (int i = 0; i < CV; ++i) {
      const int c = tid + i * 256, e = c / (KB / 8), k0 = (c % (KB / 8)) * 8;
      *(bf16x8*)&Vs[buf][e * LV + k0] = rv[i];
    }
  };

  f32x16 o[HD / 32];
#pragma unroll
  for (int t = 0; t < HD / 32; ++t)
#pragma unroll
    for (int q = 0; q < 16; ++q) o[t][q] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * 1.4426950408889634f;
  const int half = lane >> 5;
  // permuted key row read by this lane for the S^T A operand
  const int rho = lane & 31;
  const int krow = (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);

  if (T0 < NT) {
    gload(T0);
    sstore(0);
  }
  __syncthreads();
  for (int tile = T0; tile < NT; ++tile) {
    const int buf = (tile - T0) & 1;
    if (tile + 1 < NT) gload(tile + 1);
    // S^T for two 32-key halves of the tile
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int q = 0; q < 16; ++q) s[kt][q] = 0.f;
      const bf16* kp = &Ks[buf][(kt * 32 + krow) * LK + 8 * half];
#pragma unroll
      for (int kk = 0; kk < HD / 16; ++kk) {
        const bf16x8 ka = *(const bf16x8*)(kp + kk * 16);
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], s[kt], 0, 0, 0);
      }
    }
    // accumulator q of half kt holds key kt*32 + 16*(q/8) + 8*half + (q%8)
    const int jb = tile * KB;
    const bool full = (jb + KB <= sr.begin[0] + sr.count[0]) ||
                      (jb >= sr.begin[1] && jb + KB <= sr.begin[1] + sr.count[1]) ||
                      (jb >= sr.begin[2] && jb + KB <= sr.begin[2] + sr.count[2]);
    // running max in raw score units (the scale is positive); the scale and
    // the log2(e) factor are folded into one FMA in front of exp2
    float mx = -INFINITY;
    if (!full) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int j = jb + kt * 32 + 16 * (q >> 3) + 8 * half + (q & 7);
          if (!key_valid(sr, j)) s[kt][q] = -INFINITY;
        }
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int q = 0; q < 16; ++q) mx = fmaxf(mx, s[kt][q]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * sl2);
    const float moff = -m_use * sl2;
    float psum = 0.f;
    bf16x8 pb[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][q], sl2, moff));   // v_exp_f32: tiny results flush to 0
        psum += p;
        pb[kt * 2 + (q >> 3)][q & 7] = (bf16)p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // rescale only when some query of the wave raised its maximum (exact:
    // alpha is 1 otherwise)
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int t = 0; t < HD / 32; ++t)
#pragma unroll
        for (int q = 0; q < 16; ++q) o[t][q] *= alpha;
    }
    // O^T += V^T P^T over 4 key blocks of 16
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int t = 0; t < HD / 32; ++t) {
        const bf16x8 va = *(const bf16x8*)&Vs[buf][(t * 32 + (lane & 31)) * LV + kb * 16 + 8 * half];
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kb], o[t], 0, 0, 0);
      }
    }
    if (tile + 1 < NT) sstore(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (a.nsplit > 1) {
    // partial result of this key range: unnormalised O and (max, sum)
    const int tq = q0 + wave * 32 + (lane & 31);
    if (tq < a.L) {
      float* po = a.part_o + sp * a.part_so + ((int64_t)r * a.L + tq) * a.d + (int64_t)h * HD;
#pragma unroll
      for (int t = 0; t < HD / 32; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(float4*)(po + t * 32 + 8 * g + 4 * half) =
              make_float4(o[t][4 * g], o[t][4 * g + 1], o[t][4 * g + 2], o[t][4 * g + 3]);
      if (half == 0) a.part_ml[sp * a.part_sml + ((int64_t)r * a.H + h) * a.L + tq] = make_float2(m_run, l_tot);
    }
    return;
  }
  // normalise and write O (token-major) through LDS: Os[query][hd]
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  bf16* Os = &Ks[0][0];                // BQ x (HD + PK) fits in one K stage
  constexpr int LO = HD + PK;
  static_assert(BQ * LO <= 2 * KB * LK, "O staging must fit in the K buffers");
  const int ql = wave * 32 + (lane & 31);
#pragma unroll
  for (int t = 0; t < HD / 32; ++t)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int e = t * 32 + 8 * (q >> 2) + 4 * half + (q & 3);
      Os[ql * LO + e] = (bf16)(o[t][q] * inv);
    }
  __syncthreads();
  constexpr int CO = BQ * (HD / 8) / 256;
#pragma unroll
  for (int i = 0; i < CO; ++i) {
    const int c = tid + i * 256, qq = c / (HD / 8), e0 = (c % (HD / 8)) * 8;
    const int t = q0 + qq;
    if (t < a.L) {
      bf16* op = (bf16*)a.o + ((int64_t)r * a.L + t) * a.d + (int64_t)h * HD + e0;
      *(bf16x8*)op = *(const bf16x8*)&Os[qq * LO + e0];
    }
  }
}

// ---------------------------------------------------------------------------
// fp32: one thread per query, keys staged 64 at a time in LDS.
template <int HD>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  constexpr int KB = 64;
  __shared__ float Ks[KB][HD + 1];
  __shared__ float Vs[HD][KB + 1];
  const int tid = threadIdx.x;
  const int h = blockIdx.y, r = a.r0 + blockIdx.z;
  const int t = blockIdx.x * 64 + tid;
  const SegRt sr = seg_layout(a);
  const int NK = sr.end[2];
  float q[HD], o[HD];
  const float* qp = (const float*)a.q + (int64_t)r * a.q_rs + (int64_t)h * a.q_hs + (int64_t)t * HD;
#pragma unroll
  for (int e = 0; e < HD; ++e) {
    q[e] = (t < a.L) ? qp[e] * a.scale : 0.f;
    o[e] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  for (int jb = 0; jb < NK; jb += KB) {
    __syncthreads();
    for (int c = tid; c < KB * HD; c += 64) {
      const int key = c / HD, e = c % HD;
      const int j = jb + key;
      float kv = 0.f, vv = 0.f;
      if (j < NK && key_valid(sr, j)) {
        const int s = key_seg(sr, j);
        const KvSeg g = seg_pick(a, s);
        const int pos = key_pos(g, j - (s == 0 ? sr.begin[0] : (s == 1 ? sr.begin[1] : sr.begin[2])));
        kv = ((const float*)g.k)[(int64_t)r * g.k_rs + (int64_t)h * g.k_hs + (int64_t)pos * HD + e];
        vv = ((const float*)g.vt)[(int64_t)r * g.vt_rs + (int64_t)h * g.vt_hs + (int64_t)e * g.cap + pos];
      }
      Ks[key][e] = kv;
      Vs[e][key] = vv;
    }
    __syncthreads();
    float sc[KB];
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      float v = -INFINITY;
      if (jb + k < NK && key_valid(sr, jb + k)) {
        v = 0.f;
#pragma unroll
        for (int e = 0; e < HD; ++e) v += q[e] * Ks[k][e];
      }
      sc[k] = v;
      mx = fmaxf(mx, v);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = expf(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int e = 0; e < HD; ++e) o[e] *= alpha;
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const float p = expf(sc[k] - m_use);
      l_run += p;
#pragma unroll
      for (int e = 0; e < HD; ++e) o[e] += p * Vs[e][k];
    }
    m_run = m_new;
  }
  if (t < a.L) {
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    float* op = (float*)a.o + ((int64_t)r * a.L + t) * a.d + (int64_t)h * HD;
#pragma unroll
    for (int e = 0; e < HD; ++e) op[e] = o[e] * inv;
  }
}

// ---------------------------------------------------------------------------
// Combine of split-KV partials: O = sum_s w_s O_s / sum_s w_s l_s with
// w_s = 2^((m_s - max_s m_s) * scale * log2 e).  One thread per 4 head-dim
// elements of one (token, head).
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int hd4 = a.hd / 4;
  const int64_t per_tok = (int64_t)a.H * hd4;
  if (i >= (int64_t)a.R * a.L * per_tok) return;
  const int64_t tok = i / per_tok;                // r_rel * L + t
  const int h = (int)((i % per_tok) / hd4), e = (int)(i % hd4) * 4;
  const int rr = (int)(tok / a.L), t = (int)(tok % a.L);
  const int r = a.r0 + rr;
  const float sl2 = a.scale * 1.4426950408889634f;
  float mmax = -INFINITY;
  for (int sp = 0; sp < a.nsplit; ++sp)
    mmax = fmaxf(mmax, a.part_ml[sp * a.part_sml + ((int64_t)r * a.H + h) * a.L + t].x);
  float l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int sp = 0; sp < a.nsplit; ++sp) {
    const float2 ml = a.part_ml[sp * a.part_sml + ((int64_t)r * a.H + h) * a.L + t];
    if (ml.x == -INFINITY) continue;
    const float w = exp2f((ml.x - mmax) * sl2);
    l += w * ml.y;
    const float4 v = *(const float4*)(a.part_o + sp * a.part_so + ((int64_t)r * a.L + t) * a.d + (int64_t)h * a.hd + e);
    acc.x += w * v.x;
    acc.y += w * v.y;
    acc.z += w * v.z;
    acc.w += w * v.w;
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  bf16x4 ov;
  ov[0] = (bf16)(acc.x * inv);
  ov[1] = (bf16)(acc.y * inv);
  ov[2] = (bf16)(acc.z * inv);
  ov[3] = (bf16)(acc.w * inv);
  *(bf16x4*)((bf16*)a.o + ((int64_t)r * a.L + t) * a.d + (int64_t)h * a.hd + e) = ov;
}

int attention_pick_split(int units, int tiles, int max_split, int concurrent) {
  int best = 1;
  double best_cost = (double)((units + concurrent - 1) / concurrent);
  for (int sp = 2; sp <= max_split; ++sp) {
    if (tiles / sp < 4) break;
    const double rounds = (double)(((int64_t)units * sp + concurrent - 1) / concurrent);
    const double cost = rounds / sp * 1.04;     // 4% for the partial traffic and the combine pass
    if (cost < best_cost * 0.98) {
      best_cost = cost;
      best = sp;
    }
  }
  return best;
}

hipError_t attention_combine(hipStream_t s, const AttnArgs& a) {
  if (a.nsplit <= 1 || a.R == 0 || a.L == 0) return hipSuccess;
  const int64_t n = (int64_t)a.R * a.L * a.H * (a.hd / 4);
  attn_combine_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t attention(hipStream_t s, bool bf, const AttnArgs& args, bool combine) {
  if (args.R == 0 || args.L == 0) return hipSuccess;
  AttnArgs a = args;
  if (a.nsplit < 1 || !bf) a.nsplit = 1;
  if (bf) {
    const int nsplit = a.nsplit;
    const dim3 g(((a.L + 127) / 128) * a.H * a.R * nsplit);
    switch (a.hd) {
      case 32:
        if (a.nseg == 1) attn_bf16_kernel<32, 1><<<g, 256, 0, s>>>(a);
        else attn_bf16_kernel<32, 0><<<g, 256, 0, s>>>(a);
        break;
      case 64:
        if (a.nseg == 1) attn_bf16_kernel<64, 1><<<g, 256, 0, s>>>(a);
        else attn_bf16_kernel<64, 0><<<g, 256, 0, s>>>(a);
        break;
      case 128:
        if (a.nseg == 1) attn_bf16_kernel<128, 1><<<g, 256, 0, s>>>(a);
        else attn_bf16_kernel<128, 0><<<g, 256, 0, s>>>(a);
        break;
      default: return hipErrorInvalidValue;
    }
    if (nsplit > 1 && combine) {
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      return attention_combine(s, a);
    }
  } else {
    dim3 g((a.L + 63) / 64, a.H, a.R);
    switch (a.hd) {
      case 16: attn_f32_kernel<16><<<g, 64, 0, s>>>(a); break;
      case 32: attn_f32_kernel<32><<<g, 64, 0, s>>>(a); break;
      case 64: attn_f32_kernel<64><<<g, 64, 0, s>>>(a); break;
      case 128: attn_f32_kernel<128><<<g, 64, 0, s>>>(a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace sdk
