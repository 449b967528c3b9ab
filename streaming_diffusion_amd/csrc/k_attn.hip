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
#include <algorithm>
#include <cmath>
#include <queue>
#include <vector>

#include "kernels.h"
#include "kv_append.h"

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

// Branch-free: each segment is one unsigned range test, combined with
// bitwise ors (no short-circuit control flow inside the masking loops).
SD_DEV bool key_valid(const SegRt& s, int j) {
  const bool v0 = (unsigned)(j - s.begin[0]) < (unsigned)s.count[0];
  const bool v1 = (unsigned)(j - s.begin[1]) < (unsigned)s.count[1];
  const bool v2 = (unsigned)(j - s.begin[2]) < (unsigned)s.count[2];
  return v0 | v1 | v2;
}

// Physical position and segment of virtual key j (j inside a segment's padded range).
SD_DEV int key_seg(const SegRt& s, int j) { return j < s.end[0] ? 0 : (j < s.end[1] ? 1 : 2); }

// Segment s of the launch, selected without dynamic indexing of the argument.
SD_DEV KvSeg seg_pick(const AttnArgs& a, int s) { return s == 0 ? a.seg[0] : (s == 1 ? a.seg[1] : a.seg[2]); }

SD_DEV int key_pos(const KvSeg& g, int u) {
  const int p = g.start + u;
  return g.wrap ? p % g.cap : p;
}

// One of three values, chosen by value (a conditional over lvalues would
// select an address and force its operands into memory)
template <typename T>
SD_DEV T pick3(bool first, bool second, T x, T y, T z) {
  return first ? x : (second ? y : z);
}

// ---------------------------------------------------------------------------
// K and V^T tiles move from global memory straight into LDS
// (global_load_lds_dwordx4: 16 bytes per lane, a wave instruction fills 1 KB,
// lane l at byte 16*l); no register staging.  LDS rows are unpadded and their
// 16-byte chunks XOR-swizzled by row (chunk c of row r at c ^ chunk_swz<W>(r),
// W the row width in elements) so that the 16-lane passes of the MFMA
// fragment reads fall on distinct banks.
template <int W>
SD_DEV int chunk_swz(int row) {
  return (row / (128 / W)) & (W / 8 - 1);
}

SD_DEV void dma16(const bf16* src, bf16* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// this wave's loads have landed; meet the workgroup (no fence: the wait
// orders the DMA writes, the LDS reads of the previous tile were consumed)
SD_DEV void dma_wait_barrier() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// max / sum of a lane's value and the value of lane ^ 32
SD_DEV float halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
SD_DEV float halves_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// bf16 path.  The keys of one (row, head) are walked segment by segment in
// tiles of 64 that never straddle two segments (a segment's last tile is
// partial and masked), so the segment, its base pointers and its ring wrap
// are uniform per tile and every per-lane address is plain arithmetic.
// One workgroup = 4 waves = 128 queries; two workgroups share a CU.
//
// ONESEG = 1 instantiates the same code for single-segment calls (the
// prompt cross-attention), so that profiles tell the two uses apart.
template <int HD, int ONESEG>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnArgs a) {
  constexpr int BQ = 128, KB = 64;
  constexpr int CKR = HD / 8, RK = 64 / CKR;              // K: chunks per key row, key rows per DMA
  constexpr int IK = KB / RK / 4, IV = HD / 8 / 4;        // DMA instructions per wave per tile (K, V^T)
  constexpr int KT_EL = KB * HD, STAGE = 2 * KB * HD;     // bf16 elements: K tile, K + V^T tile
  constexpr int LO = HD + 8;
  static_assert(IK >= 1 && IV >= 1, "tile shape");
  static_assert(BQ * LO <= 2 * STAGE, "output staging must fit in the stages");
  // growth of the running maximum (in exp2 units) that forces a rescale, so
  // probabilities stay below 2^8 between rescales
  constexpr float RESCALE_LOG2 = 8.0f;
  __shared__ __attribute__((aligned(1024))) bf16 smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nqt = (a.L + BQ - 1) / BQ;
  // The first nfull workgroups take the query tiles of heads [0, h_full)
  // whole, the rest the split pieces of heads [h_full, H); each class is
  // mapped XCD-contiguously on its own.  Order (head, split, row, q-tile):
  // the workgroups resident on one XCD at a time are the q-tiles of every
  // row for the same key range -- the rows share the sink and the window,
  // which then stream through that XCD's L2 once for all of them.
  const int nfull = a.h_full * nqt * a.R;
  const bool whole = (int)blockIdx.x < nfull;
  const int nsp = whole ? 1 : a.nsplit;
  const int lid = whole ? xcd_remap(blockIdx.x, nfull) : xcd_remap(blockIdx.x - nfull, gridDim.x - nfull);
  const int qt = lid % nqt, r = a.r0 + (lid / nqt) % a.R;
  const int sp = (lid / (nqt * a.R)) % nsp, h = (whole ? 0 : a.h_full) + lid / (nqt * a.R * nsp);
  const int q0 = qt * BQ;

  // segments of this (row, head) as plain scalars, uniform over the
  // workgroup (unused segments have no keys)
  const int* const dyn = a.dyn_seg;
  const int c0 = a.nseg > 0 ? (dyn ? dyn[1] : a.seg[0].count) : 0;
  const int c1 = a.nseg > 1 ? (dyn ? dyn[3] : a.seg[1].count) : 0;
  const int c2 = a.nseg > 2 ? a.seg[2].count : 0;
  const int nt0 = (c0 + KB - 1) / KB, nt1 = (c1 + KB - 1) / KB, nt2 = (c2 + KB - 1) / KB;
  const int NT_all = nt0 + nt1 + nt2;
  const int tps = (NT_all + nsp - 1) / nsp;
  const int T0 = min(NT_all, sp * tps), NT = min(NT_all, T0 + tps);   // this split's key tiles [T0, NT)
  const bf16* const kbase0 = (const bf16*)a.seg[0].k + (int64_t)r * a.seg[0].k_rs + (int64_t)h * a.seg[0].k_hs;
  const bf16* const kbase1 = (const bf16*)a.seg[1].k + (int64_t)r * a.seg[1].k_rs + (int64_t)h * a.seg[1].k_hs;
  const bf16* const kbase2 = (const bf16*)a.seg[2].k + (int64_t)r * a.seg[2].k_rs + (int64_t)h * a.seg[2].k_hs;
  const bf16* const vbase0 = (const bf16*)a.seg[0].vt + (int64_t)r * a.seg[0].vt_rs + (int64_t)h * a.seg[0].vt_hs;
  const bf16* const vbase1 = (const bf16*)a.seg[1].vt + (int64_t)r * a.seg[1].vt_rs + (int64_t)h * a.seg[1].vt_hs;
  const bf16* const vbase2 = (const bf16*)a.seg[2].vt + (int64_t)r * a.seg[2].vt_rs + (int64_t)h * a.seg[2].vt_hs;
  const int cap0 = a.seg[0].cap, cap1 = a.seg[1].cap, cap2 = a.seg[2].cap;
  const int st0 = dyn ? dyn[0] : a.seg[0].start, st1 = dyn ? dyn[2] : a.seg[1].start, st2 = a.seg[2].start;
  const int wr0 = a.seg[0].wrap, wr1 = a.seg[1].wrap, wr2 = a.seg[2].wrap;

  // tile t -> its segment's bases, the position of its first key, the
  // segment's capacity and ring flag, and the number of valid keys in it
  struct TileRef {
    const bf16* kb;
    const bf16* vb;
    int p0, cap, wrap, nvalid;
  };
  auto tile_ref = [=](int t) {
    const bool in0 = t < nt0, in1 = !in0 && t < nt0 + nt1;
    const int u0 = (t - pick3(in0, in1, 0, nt0, nt0 + nt1)) * KB;
    TileRef f;
    f.kb = pick3(in0, in1, kbase0, kbase1, kbase2);
    f.vb = pick3(in0, in1, vbase0, vbase1, vbase2);
    f.cap = pick3(in0, in1, cap0, cap1, cap2);
    f.wrap = pick3(in0, in1, wr0, wr1, wr2);
    f.nvalid = min(KB, pick3(in0, in1, c0, c1, c2) - u0);
    int p0 = pick3(in0, in1, st0, st1, st2) + u0;
    if (f.wrap && p0 >= f.cap) p0 -= f.cap;
    f.p0 = p0;
    return f;
  };

  // Q fragments (B operand): lane -> query q0 + wave*32 + lane%32, hd block
  // kk*16 + 8*(lane/32).
  const int half = lane >> 5;
  const int myq = q0 + wave * 32 + (lane & 31);
  bf16x8 qf[HD / 16];
  {
    const bf16* qp = (const bf16*)a.q + (int64_t)r * a.q_rs + (int64_t)h * a.q_hs + (int64_t)min(myq, a.L - 1) * HD;
#pragma unroll
    for (int kk = 0; kk < HD / 16; ++kk) qf[kk] = *(const bf16x8*)(qp + kk * 16 + 8 * half);
  }
  // the Q fragments have landed (a wait the compiler sees: without it, the
  // first MFMA of every tile would wait for all outstanding tile DMA)
  __builtin_amdgcn_s_waitcnt(0x0F70);       // vmcnt(0), expcnt and lgkmcnt unconstrained

  // DMA of key tile t into stage buf.  This lane moves K key row
  // kr = wave*(KB/4) + i*RK + lane/CKR (logical chunk kc) and V^T head-dim row
  // ve = wave*(HD/4) + i*8 + lane/8 (logical 8-key group vc).  Keys past the
  // segment's count are read from the tile's first key: finite data whose
  // scores are masked.  An 8-key group that starts inside the valid range may
  // end in the zero-filled padding of the segment's storage (positions up to
  // the next multiple of 8 exist).
  // per-lane byte offsets of this lane's K rows inside a contiguous tile
  uint32_t koff[IK];
#pragma unroll
  for (int i = 0; i < IK; ++i) {
    const int kr = wave * (KB / 4) + i * RK + lane / CKR;
    koff[i] = (uint32_t)((kr * HD + ((lane % CKR) ^ chunk_swz<HD>(kr)) * 8) * 2);
  }
  auto issue = [&](int t, int buf) {
    bf16* ks = smem + buf * STAGE;
    bf16* vs = ks + KT_EL;
    const TileRef f = tile_ref(t);
    if (f.nvalid == KB && (!f.wrap || f.p0 + KB <= f.cap)) {
      // whole tile of valid keys at contiguous positions: uniform base plus
      // a per-lane 32-bit offset
      const char* kb = (const char*)(f.kb + (int64_t)f.p0 * HD);
      const char* vb = (const char*)(f.vb + f.p0);
#pragma unroll
      for (int i = 0; i < IK; ++i) dma16((const bf16*)(kb + koff[i]), ks + (wave * (KB / 4) + i * RK) * HD);
#pragma unroll
      for (int i = 0; i < IV; ++i) {
        const int ve = wave * (HD / 4) + i * 8 + lane / 8;
        const uint32_t vo = (uint32_t)(ve * f.cap + ((lane % 8) ^ chunk_swz<KB>(ve)) * 8) * 2u;
        dma16((const bf16*)(vb + vo), vs + (wave * (HD / 4) + i * 8) * KB);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < IK; ++i) {
      const int kr = wave * (KB / 4) + i * RK + lane / CKR;
      const int kc = (lane % CKR) ^ chunk_swz<HD>(kr);
      int pos = f.p0 + (kr < f.nvalid ? kr : 0);
      if (f.wrap && pos >= f.cap) pos -= f.cap;
      dma16(f.kb + (int64_t)pos * HD + kc * 8, ks + (wave * (KB / 4) + i * RK) * HD);
    }
#pragma unroll
    for (int i = 0; i < IV; ++i) {
      const int ve = wave * (HD / 4) + i * 8 + lane / 8;
      const int vc = (lane % 8) ^ chunk_swz<KB>(ve);
      int pos = f.p0 + (vc * 8 < f.nvalid ? vc * 8 : 0);
      if (f.wrap && pos >= f.cap) pos -= f.cap;
      dma16(f.vb + (int64_t)ve * f.cap + pos, vs + (wave * (HD / 4) + i * 8) * KB);
    }
  };

  f32x16 o[HD / 32];
#pragma unroll
  for (int t = 0; t < HD / 32; ++t)
#pragma unroll
    for (int q = 0; q < 16; ++q) o[t][q] = 0.f;
  // m_run: reference maximum (raw score units) of the exponentials; it is
  // raised only when a score exceeds it by RESCALE_LOG2 in exp2 units
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * 1.4426950408889634f;
  const float grow = RESCALE_LOG2 / sl2;
  // permuted key row read by this lane for the S^T A operand (bits 2 and 3
  // swapped), so that the accumulators are the B operand of O^T = V^T P^T
  const int rho = lane & 31;
  const int krow = (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
  const int vrow = lane & 31;

  if (T0 < NT) issue(T0, 0);
  for (int tile = T0; tile < NT; ++tile) {
    const int buf = (tile - T0) & 1;
    dma_wait_barrier();                               // tile landed everywhere; tile-1 retired
    if (tile + 1 < NT) issue(tile + 1, buf ^ 1);
    const bf16* ks = smem + buf * STAGE;
    const bf16* vs = ks + KT_EL;
    // S^T for two 32-key halves of the tile.  Every K fragment read is
    // issued before the first product: while the next tile's DMA is in
    // flight each LDS wait drains all outstanding reads, so reads issued one
    // product ahead would put an LDS round trip in front of every MFMA.
    bf16x8 ka[2][HD / 16];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int row = kt * 32 + krow;
      const bf16* kp = ks + row * HD;
      const int sw = chunk_swz<HD>(row);
#pragma unroll
      for (int kk = 0; kk < HD / 16; ++kk) ka[kt][kk] = *(const bf16x8*)(kp + (((kk * 2 + half) ^ sw) * 8));
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int q = 0; q < 16; ++q) s[kt][q] = 0.f;
#pragma unroll
    for (int kk = 0; kk < HD / 16; ++kk)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kt][kk], qf[kk], s[kt], 0, 0, 0);
    // the V^T fragments of the PV product, read while the softmax runs
    bf16x8 va[4][HD / 32];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int t = 0; t < HD / 32; ++t) {
        const int row = t * 32 + vrow;
        va[kb][t] = *(const bf16x8*)(vs + row * KB + (((kb * 2 + half) ^ chunk_swz<KB>(row)) * 8));
      }
    __builtin_amdgcn_sched_barrier(0);
    // accumulator q of half kt holds tile key kt*32 + 16*(q/8) + 8*half + (q%8)
    const int nvalid = tile_ref(tile).nvalid;
    if (__builtin_expect(nvalid < KB, 0)) {
      asm volatile("");      // keeps the masking out of line (a segment's last tile only)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int q = 0; q < 16; ++q)
          s[kt][q] = kt * 32 + 16 * (q >> 3) + 8 * half + (q & 7) < nvalid ? s[kt][q] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int q = 0; q < 16; ++q) mx = fmaxf(mx, s[kt][q]);
    mx = halves_max(mx);
    // raise the reference maximum (and rescale O and l) only when some query
    // of the wave outgrew it by the threshold; a lane whose maximum is -inf
    // keeps m_run, so -inf - -inf never occurs
    if (__builtin_amdgcn_ballot_w64(mx > m_run + grow)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f((m_run - m_new) * sl2);
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < HD / 32; ++t)
#pragma unroll
        for (int q = 0; q < 16; ++q) o[t][q] *= alpha;
      m_run = m_new;
    }
    const float moff = m_run == -INFINITY ? 0.f : -m_run * sl2;
    bf16x8 pb[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int q = 0; q < 16; ++q)     // v_exp_f32: tiny results flush to 0
        pb[kt * 2 + (q >> 3)][q & 7] = (bf16)__builtin_amdgcn_exp2f(fmaf(s[kt][q], sl2, moff));
    // the row sum of the bf16 probabilities (the values the PV product
    // uses), two at a time with v_dot2c_f32_bf16 against (1, 1)
    {
      const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
      float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 8; i += 4) {
          ps0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[kb][i], pb[kb][i + 1]}, ones, ps0, false);
          ps1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[kb][i + 2], pb[kb][i + 3]}, ones, ps1, false);
        }
      l_run += ps0 + ps1;
    }
    // O^T += V^T P^T over 4 key blocks of 16
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int t = 0; t < HD / 32; ++t) o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kb][t], pb[kb], o[t], 0, 0, 0);
  }

  const float l_tot = halves_sum(l_run);
  if (nsp > 1) {
    // partial result of this key range: unnormalised O and (reference max, sum)
    if (myq < a.L) {
      bf16* po = a.part_o + sp * a.part_so + ((int64_t)r * a.L + myq) * a.d + (int64_t)h * HD;
#pragma unroll
      for (int t = 0; t < HD / 32; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (bf16)o[t][4 * g + e];
          *(bf16x4*)(po + t * 32 + 8 * g + 4 * half) = v;
        }
      if (half == 0) a.part_ml[sp * a.part_sml + ((int64_t)r * a.H + h) * a.L + myq] = make_float2(m_run, l_tot);
    }
    return;
  }
  // normalise and write O (token-major) through LDS: Os[query][hd]
  __syncthreads();
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  bf16* Os = smem;
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
// Cross-attention with the prompt projections folded in (one context).  The
// prompt K / V are fixed for the whole stream, so per block and head h
//   scores_h = (x W_q,h^T + b_q,h) K_h^T s = x (s K_h W_q,h)^T + s K_h b_q,h
//   output   = sum_h P_h (V_h W_oc,h^T) + b_oc
// with s = 1/sqrt(hd), W_q,h the rows h hd .. h hd + hd - 1 of W_q and W_oc,h
// the same columns of W_oc.  The folded matrices are built once per context;
// a step then runs a GEMM to the scores (N = H Cp), a softmax over each head's
// Cp columns and a GEMM back to the residual (K = H Cp), in place of the Q
// projection, the attention over the prompt keys and the O projection.
// Context slots C .. Cp - 1 get zero weight rows and a score bias of -inf.
// The folds read the prompt K / V in fp32 ([C][2d], token-major, before any
// rounding) and store the folded matrices, the step's normalised input and
// its probabilities in fp16: every value there is bounded (LayerNorm output,
// probabilities, products of weights with the prompt projections), and fp16
// carries three more mantissa bits than bf16 at the same matrix-core rate.
// W_q, W_oc [d][d] (out x in).

// wq_f[h Cp + j][k] = s sum_e K[j][h hd + e] W_q[h hd + e][k];  cq[h Cp + j] = s K[j][h hd ..] . b_q[h hd ..]
// (K, V: the fp32 prompt projections, token-major [C][2d], K in [0, d), V in [d, 2d))
__global__ __launch_bounds__(256) void fold_q_kernel(const float* __restrict__ kv, const bf16* __restrict__ Wq,
                                                     const bf16* __restrict__ bq, f16* __restrict__ wq_f,
                                                     float* __restrict__ cq, int d, int hd, int C, int Cp, float scale) {
  const int row = blockIdx.y, h = row / Cp, j = row - h * Cp;
  const int k = blockIdx.x * 256 + threadIdx.x;
  const float* kr = kv + (int64_t)min(j, C - 1) * 2 * d + h * hd;
  if (k < d) {
    float acc = 0.f;
    if (j < C)
      for (int e = 0; e < hd; ++e) acc += kr[e] * (float)Wq[(int64_t)(h * hd + e) * d + k];
    wq_f[(int64_t)row * d + k] = (f16)(acc * scale);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    float acc = 0.f;
    for (int e = 0; e < hd; ++e) acc += kr[e] * (float)bq[h * hd + e];
    cq[row] = j < C ? acc * scale : -INFINITY;
  }
}

// wo_f[n][h Cp + j] = sum_e V[j][h hd + e] W_oc[n][h hd + e]
__global__ __launch_bounds__(256) void fold_o_kernel(const float* __restrict__ kv, const bf16* __restrict__ Wo,
                                                     f16* __restrict__ wo_f, int d, int H, int hd, int C, int Cp) {
  const int n = blockIdx.x, ncol = H * Cp;
  for (int col = threadIdx.x; col < ncol; col += 256) {
    const int h = col / Cp, j = col - h * Cp;
    float acc = 0.f;
    if (j < C) {
      const float* vr = kv + (int64_t)j * 2 * d + d + h * hd;
      for (int e = 0; e < hd; ++e) acc += vr[e] * (float)Wo[(int64_t)n * d + h * hd + e];
    }
    wo_f[(int64_t)n * ncol + col] = (f16)acc;
  }
}

// P[m][h Cp + j] = softmax over j of (S[m][h Cp + j] + c[h Cp + j]); 16 lanes
// per (row, head), Cp <= 128
__global__ __launch_bounds__(256) void ctx_softmax_kernel(const float* __restrict__ S, const float* __restrict__ c,
                                                          f16* __restrict__ P, int64_t M, int H, int Cp) {
  const int64_t g = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int l = threadIdx.x & 15;
  if (g >= M * H) return;           // whole 16-lane groups leave together
  const int64_t m = g / H;
  const int h = (int)(g - m * H);
  const int64_t base = m * (int64_t)H * Cp + (int64_t)h * Cp;
  float v[8];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = l + 16 * i;
    v[i] = j < Cp ? S[base + j] + c[h * Cp + j] : -INFINITY;
    mx = fmaxf(mx, v[i]);
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 16));
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = l + 16 * i < Cp ? __expf(v[i] - mx) : 0.f;
    sum += v[i];
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 16);
  const float inv = 1.0f / sum;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = l + 16 * i;
    if (j < Cp) P[base + j] = (f16)(v[i] * inv);
  }
}

hipError_t cross_fold(hipStream_t s, const float* kv, const bf16* Wq, const bf16* bq, const bf16* Wo, f16* wq_f,
                      float* cq, f16* wo_f, int d, int H, int hd, int C, int Cp) {
  if (C < 1 || C > Cp || Cp > 128 || H * Cp > 65535) return hipErrorInvalidValue;
  fold_q_kernel<<<dim3((d + 255) / 256, H * Cp), 256, 0, s>>>(kv, Wq, bq, wq_f, cq, d, hd, C, Cp,
                                                              1.0f / std::sqrt((float)hd));
  fold_o_kernel<<<d, 256, 0, s>>>(kv, Wo, wo_f, d, H, hd, C, Cp);
  return hipGetLastError();
}

hipError_t ctx_softmax(hipStream_t s, const float* S, const float* c, f16* P, int64_t M, int H, int Cp) {
  if (Cp < 1 || Cp > 128) return hipErrorInvalidValue;
  const int64_t groups = M * H;
  if (groups == 0) return hipSuccess;
  ctx_softmax_kernel<<<(unsigned)((groups + 15) / 16), 256, 0, s>>>(S, c, P, M, H, Cp);
  return hipGetLastError();
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
// Combine of split partials (heads h_full .. H-1): O = sum_s w_s O_s / sum_s w_s l_s with
// w_s = 2^((m_s - max_s m_s) * scale * log2 e) (a split without keys has
// m_s = -inf and weight 0).  One thread per 8 head-dim elements of one
// (token, head); NS > 0 fixes the split count so every split's loads are in
// flight together, NS = 0 loops over a.nsplit.  The host guarantees that
// R * L * H * hd / 8 fits in 31 bits.
template <int NS>
SD_DEV void combine_one(const AttnArgs& a, int i) {
  const int c8 = a.hd >> 3, per_tok = (a.H - a.h_full) * c8;
  if (i >= a.R * a.L * per_tok) return;
  const int tok = i / per_tok, rem = i - tok * per_tok;
  const int h = a.h_full + rem / c8, e = (rem - (h - a.h_full) * c8) * 8;
  const int rr = tok / a.L, t = tok - rr * a.L;
  const int r = a.r0 + rr;
  const float sl2 = a.scale * 1.4426950408889634f;
  const float2* ml = a.part_ml + ((int64_t)r * a.H + h) * a.L + t;
  const bf16* po = a.part_o + ((int64_t)r * a.L + t) * a.d + (int64_t)h * a.hd + e;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  if constexpr (NS > 0) {
    float2 m[NS];
    bf16x8 x[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      m[s] = ml[s * a.part_sml];
      x[s] = *(const bf16x8*)(po + s * a.part_so);
    }
    float mmax = -INFINITY;
#pragma unroll
    for (int s = 0; s < NS; ++s) mmax = fmaxf(mmax, m[s].x);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const float w = m[s].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m[s].x - mmax) * sl2);
      l += w * m[s].y;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += w * (float)x[s][j];
    }
  } else {
    float mmax = -INFINITY;
    for (int s = 0; s < a.nsplit; ++s) mmax = fmaxf(mmax, ml[s * a.part_sml].x);
    for (int s = 0; s < a.nsplit; ++s) {
      const float2 m = ml[s * a.part_sml];
      if (m.x == -INFINITY) continue;
      const float w = __builtin_amdgcn_exp2f((m.x - mmax) * sl2);
      l += w * m.y;
      const bf16x8 x = *(const bf16x8*)(po + s * a.part_so);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += w * (float)x[j];
    }
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  bf16x8 ov;
#pragma unroll
  for (int j = 0; j < 8; ++j) ov[j] = (bf16)(acc[j] * inv);
  *(bf16x8*)((bf16*)a.o + ((int64_t)r * a.L + t) * a.d + (int64_t)h * a.hd + e) = ov;
}

template <int NS>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  combine_one<NS>(a, blockIdx.x * 256 + threadIdx.x);
}

// The combine pass and the KV append of the leaving chunk in one launch
// (both only wait for the attention; the append may overwrite ring entries
// the attention has just read): workgroups [0, ncomb) combine, the rest
// append.
template <int NS>
__global__ __launch_bounds__(256) void attn_combine_append_kernel(AttnArgs a, KvAppendArgs k, int ncomb) {
  if ((int)blockIdx.x < ncomb)
    combine_one<NS>(a, blockIdx.x * 256 + threadIdx.x);
  else
    kv_append_chunk(k, (int64_t)(blockIdx.x - ncomb) * 256 + threadIdx.x);
}

int attention_q_tile(bool bf, int hd) { return !bf ? 64 : 128; }

int attention_wg_per_cu(bool bf, int hd) { return !bf ? 1 : 2; }

int attention_pick_split(int units, int tiles, int max_split, int concurrent) {
  // cost ~ rounds of resident workgroups x key tiles per workgroup, plus 4%
  // per split launch for the partial traffic and the combine pass; ties go
  // to fewer splits
  int best = 1;
  double best_cost = (double)((units + concurrent - 1) / concurrent) * tiles;
  for (int sp = 2; sp <= max_split && sp <= tiles; ++sp) {
    const double rounds = (double)(((int64_t)units * sp + concurrent - 1) / concurrent);
    const double cost = rounds * ((tiles + sp - 1) / sp) * 1.04;
    if (cost < best_cost * 0.98) {
      best_cost = cost;
      best = sp;
    }
  }
  return best;
}

// Greedy list schedule of n_long workgroups of len_long key tiles followed
// by n_short of len_short on `slots` resident slots (each workgroup starts
// on the earliest free slot, in grid order): the finishing time.
static int64_t list_makespan(int64_t n_long, int64_t len_long, int64_t n_short, int64_t len_short, int slots) {
  std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> free_at;
  for (int i = 0; i < slots; ++i) free_at.push(0);
  int64_t end = 0;
  auto place = [&](int64_t n, int64_t len) {
    for (int64_t j = 0; j < n; ++j) {
      const int64_t t = free_at.top() + len;
      free_at.pop();
      free_at.push(t);
      end = std::max(end, t);
    }
  };
  place(n_long, len_long);
  place(n_short, len_short);
  return end;
}

void attention_pick_plan(int heads, int units_per_head, int tiles, int max_split, int concurrent, int* nsplit,
                         int* h_full) {
  // remembered per arguments (the step asks with the same ones every block)
  static thread_local int memo[7] = {-1, -1, -1, -1, -1, 1, 0};
  if (memo[0] == heads && memo[1] == units_per_head && memo[2] == tiles && memo[3] == max_split &&
      memo[4] == concurrent) {
    *nsplit = memo[5];
    *h_full = memo[6];
    return;
  }
  const int units = heads * units_per_head;
  int best_ns = attention_pick_split(units, tiles, max_split, concurrent), best_hf = 0;
  // the uniform plan, priced by the same schedule, with 4 % for the split's
  // partial traffic and combine pass in proportion to the heads it splits
  double best_cost = (double)list_makespan(0, 0, (int64_t)units * best_ns, (tiles + best_ns - 1) / best_ns,
                                           concurrent) * (best_ns > 1 ? 1.04 : 1.0);
  if (units > concurrent && best_ns > 1) {
    // whole heads filling the first full rounds, the rest split
    const int hf_max = std::min(heads - 1, (units / concurrent) * concurrent / std::max(1, units_per_head));
    // (most whole heads first: on a tie they leave the least to combine)
    for (int hf = hf_max; hf >= std::max(1, hf_max - 2); --hf)
      for (int ns = 2; ns <= max_split && ns <= tiles; ++ns) {
        const int64_t n_short = (int64_t)(heads - hf) * units_per_head * ns;
        const double cost = (double)list_makespan((int64_t)hf * units_per_head, tiles, n_short, (tiles + ns - 1) / ns,
                                                  concurrent) * (1.0 + 0.04 * (heads - hf) / heads);
        if (cost < best_cost * 0.995) {
          best_cost = cost;
          best_ns = ns;
          best_hf = hf;
        }
      }
  }
  const int v[7] = {heads, units_per_head, tiles, max_split, concurrent, best_ns, best_hf};
  std::copy(v, v + 7, memo);
  *nsplit = best_ns;
  *h_full = best_hf;
}

hipError_t attention_combine(hipStream_t s, const AttnArgs& a) {
  if (a.nsplit <= 1 || a.R == 0 || a.L == 0 || a.h_full >= a.H) return hipSuccess;
  const int64_t n = (int64_t)a.R * a.L * (a.H - a.h_full) * (a.hd / 8);
  if (a.hd % 8 || n > 0x7fffffff) return hipErrorInvalidValue;
  const unsigned g = (unsigned)((n + 255) / 256);
  switch (a.nsplit) {
    case 2: attn_combine_kernel<2><<<g, 256, 0, s>>>(a); break;
    case 3: attn_combine_kernel<3><<<g, 256, 0, s>>>(a); break;
    case 4: attn_combine_kernel<4><<<g, 256, 0, s>>>(a); break;
    case 5: attn_combine_kernel<5><<<g, 256, 0, s>>>(a); break;
    case 6: attn_combine_kernel<6><<<g, 256, 0, s>>>(a); break;
    case 7: attn_combine_kernel<7><<<g, 256, 0, s>>>(a); break;
    case 8: attn_combine_kernel<8><<<g, 256, 0, s>>>(a); break;
    default: attn_combine_kernel<0><<<g, 256, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

hipError_t attention_combine_append(hipStream_t s, const AttnArgs& a, const KvAppendArgs& k) {
  const int64_t n = a.nsplit > 1 && a.h_full < a.H ? (int64_t)a.R * a.L * (a.H - a.h_full) * (a.hd / 8) : 0;
  const int64_t chunks = 2 * ((int64_t)k.H * k.L * k.hd / 8);
  if (a.hd % 8 || n > 0x7fffffff) return hipErrorInvalidValue;
  const int64_t gc = (n + 255) / 256, ga = (chunks + 255) / 256;
  if (gc + ga == 0) return hipSuccess;
  const unsigned g = (unsigned)(gc + ga);
  switch (a.nsplit) {
    case 2: attn_combine_append_kernel<2><<<g, 256, 0, s>>>(a, k, (int)gc); break;
    case 3: attn_combine_append_kernel<3><<<g, 256, 0, s>>>(a, k, (int)gc); break;
    case 4: attn_combine_append_kernel<4><<<g, 256, 0, s>>>(a, k, (int)gc); break;
    case 5: attn_combine_append_kernel<5><<<g, 256, 0, s>>>(a, k, (int)gc); break;
    case 6: attn_combine_append_kernel<6><<<g, 256, 0, s>>>(a, k, (int)gc); break;
    case 7: attn_combine_append_kernel<7><<<g, 256, 0, s>>>(a, k, (int)gc); break;
    case 8: attn_combine_append_kernel<8><<<g, 256, 0, s>>>(a, k, (int)gc); break;
    default: attn_combine_append_kernel<0><<<g, 256, 0, s>>>(a, k, (int)gc); break;
  }
  return hipGetLastError();
}

hipError_t attention(hipStream_t s, bool bf, const AttnArgs& args, bool combine) {
  if (args.R == 0 || args.L == 0) return hipSuccess;
  AttnArgs a = args;
  if (a.nsplit < 1 || !bf) a.nsplit = 1;
  if (a.nsplit == 1 || a.h_full < 0 || a.h_full > a.H) a.h_full = 0;
  if (bf) {
    const int nsplit = a.nsplit;
    const int64_t per_head = (int64_t)((a.L + 127) / 128) * a.R;
    const dim3 g((unsigned)(per_head * (a.h_full + (int64_t)(a.H - a.h_full) * nsplit)));
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
    if (nsplit > 1 && a.h_full < a.H && combine) {
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
