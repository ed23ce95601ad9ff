// Flash-style attention kernels of the MC-Sparse hot path for gfx950.
//
// One wavefront owns one query group of C = 64 queries (PDDP groups on the sparse
// path, consecutive token blocks on the dense path) and walks that group's key
// list 32 keys at a time:
//   * gather-sparse (MC-Sparse summary page, grouping paragraph): the key list is
//     the group's row of int32 indices; every K/V row is fetched straight from
//     global memory by index (no block repacking), so a group's keys may lie
//     anywhere in the sequence;
//   * dense (limitations paragraph: anchors still run full attention): the key
//     list is 0..N-1.
// Per 32-key step the wave computes S^T = K_step * Q_group^T with
// v_mfma_f32_32x32x16_bf16 (fp32 inputs: 32x32x2_f32), so each lane owns one
// query column and the online softmax needs a single cross-half exchange
// (v_permlane32_swap); then O += P * V_step on the same MFMA shape.  P never
// leaves registers: the accumulator layout of S^T is already the A-operand
// layout of the PV product once the step's key order is fixed accordingly.
//
// Epilogues (residual paragraph): plain O, O + cached residual (reuse step),
// or dense output minus O (the anchor's residual).  A variant without the PV
// product produces the per-row softmax statistics (selection pass 1).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "ldstile.hpp"

namespace mcs {

namespace {

// Lane-level tile bookkeeping of one 32-key step.
//   A-row m of S^T (lane m%32 loads its K row) holds step entry
//     e(m) = 16*((m/4)%2) + 4*(m/8) + m%4,
//   which makes accumulator register r of lane half hf hold entry 16*hf + r.
//   The PV product then consumes registers 8*ks..8*ks+7 as its k-slots, and the
//   V operand of lane half hf needs entries 16*hf + 8*ks + t: 16 consecutive
//   entries per lane half.
__device__ __forceinline__ int a_row_entry(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }

template <typename T, int D>
struct Tile {
  static constexpr bool F32 = std::is_same<T, float>::value;
  static constexpr int ES = sizeof(T);
  static constexpr int ROWB = D * ES;
  // K/Q operand: each lane holds half a row (bf16: dims 16s+8hf..+7 for step s;
  // fp32: dims (D/2)*hf + s), fetched as 16-byte chunks.
  static constexpr int KCH = ROWB / 2 / 16;          // 16-byte chunks per lane
  static constexpr int KSTRIDE = F32 ? 16 : 32;      // byte stride between chunks
  static constexpr int QK_STEPS = F32 ? D / 2 : D / 16;
  // V operand: each lane fetches VEC consecutive dims of each of its 16 entries.
  static constexpr int VEC = D / 32;
  static constexpr int VBYTES = VEC * ES;
  static constexpr int VW = VBYTES / 4;              // dwords per V fetch
  static_assert(VW == 1 || VW == 2 || VW == 4, "V fetch width");

  __device__ static uint32_t khalf_off(int hf) { return F32 ? (uint32_t)(D / 2 * 4 * hf) : (uint32_t)(16 * hf); }
};

template <int VW>
struct VRaw;
template <> struct VRaw<1> { uint32_t w[1]; };
template <> struct VRaw<2> { uint32_t w[2]; };
template <> struct VRaw<4> { uint32_t w[4]; };

template <typename T, int D>
struct KV {
  using TL = Tile<T, D>;
  u32x4 k[TL::KCH];
  VRaw<TL::VW> v[16];
};

struct Idx {
  int k;       // key of this lane's A-row
  int v[16];   // keys of entries 16*hf + 0..15
};

template <int VW>
__device__ __forceinline__ VRaw<VW> vload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  VRaw<VW> x;
  if constexpr (VW == 1) {
    x.w[0] = bload32(r, off);
  } else if constexpr (VW == 2) {
    u32x2 t = bload64(r, off);
    x.w[0] = t[0];
    x.w[1] = t[1];
  } else {
    u32x4 t = bload128(r, off);
    x.w[0] = t[0]; x.w[1] = t[1]; x.w[2] = t[2]; x.w[3] = t[3];
  }
  return x;
}

// Keys of the step's entries.  No clamping: an entry past K holds -1 (or lies past
// kpad, where the index buffer reads as 0), and key * row_bytes of -1 wraps to an
// offset past the end of the K/V buffers, which the buffer loads return as zeros;
// those entries' scores are masked to -inf anyway.
template <bool GATHER>
__device__ __forceinline__ void load_idx(Idx& ix, __amdgpu_buffer_rsrc_t ridx, int t0, int lm, int hf) {
  if constexpr (GATHER) {
    ix.k = (int)bload32(ridx, (uint32_t)(t0 + a_row_entry(lm)) * 4u);
    const int ev = t0 + 16 * hf;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4 w = bload128(ridx, (uint32_t)(ev + 4 * c) * 4u);
#pragma unroll
      for (int j = 0; j < 4; ++j) ix.v[4 * c + j] = (int)w[j];
    }
  } else {
    ix.k = t0 + a_row_entry(lm);
#pragma unroll
    for (int j = 0; j < 16; ++j) ix.v[j] = t0 + 16 * hf + j;
  }
}

template <typename T, int D>
__device__ __forceinline__ void load_k(KV<T, D>& b, const Idx& ix, __amdgpu_buffer_rsrc_t rk, int hf) {
  using TL = Tile<T, D>;
  const uint32_t kb = (uint32_t)ix.k * TL::ROWB + TL::khalf_off(hf);
#pragma unroll
  for (int c = 0; c < TL::KCH; ++c) b.k[c] = bload128(rk, kb + c * TL::KSTRIDE);
}

template <typename T, int D>
__device__ __forceinline__ void load_v(KV<T, D>& b, const Idx& ix, __amdgpu_buffer_rsrc_t rv, int lm) {
  using TL = Tile<T, D>;
  const uint32_t lo = (uint32_t)lm * TL::VBYTES;
#pragma unroll
  for (int j = 0; j < 16; ++j) b.v[j] = vload<TL::VW>(rv, (uint32_t)ix.v[j] * TL::ROWB + lo);
}

// Component c (0..VEC-1) of fetched V data as a 16-bit (bf16) half-word source.
template <int VW>
__device__ __forceinline__ uint32_t vword(const VRaw<VW>& x, int c) { return x.w[c >> 1]; }

template <typename T, int D, bool PV>
struct State {
  using TL = Tile<T, D>;
  f32x16 o[2][TL::VEC];
  float m[2];   // running offset, log2 units (scaled max), per query column
  float l[2];   // running sum of exp2(s*c - m) that normalises O
  float lx[2];  // exact fp32 sum of the unrounded probabilities, kept for the row
                // statistics when l sums the bf16-rounded ones (see row_sums)
};

// Row sums of one step's probabilities.  O is normalised by the sum of exactly
// the values the PV product multiplies: for bf16 those are the probabilities
// rounded to bf16, summed with v_dot2_f32_bf16 against ones, so a row whose
// mass sits on one key returns that key's V row without a 2^-9 scale error.  The
// row statistics (logsumexp, the offset and 1/sum that selection pass 2 reads)
// need the exact fp32 sum of the unrounded values: with STATS both are kept,
// the exact one in lx.  Without PV there is only the exact sum, in l.
template <bool PV, bool F32, bool STATS>
__device__ __forceinline__ void row_sums(float& l, float& lx, const f32x16& p, const uint32_t (&pk)[8]) {
  constexpr bool PACKED = PV && !F32;
  constexpr bool EXACT = !PACKED || STATS;
  if constexpr (PACKED) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    float ls = l;
#pragma unroll
    for (int i = 0; i < 8; ++i) ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[i]), one, ls, false);
    l = ls;
  }
  if constexpr (EXACT) {
    float ls = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) ls += p[r];
    if constexpr (PACKED)
      lx += ls;
    else
      l += ls;
  }
}

// The sum the row statistics are taken from (see row_sums).
template <bool PV, bool F32, bool STATS>
__device__ __forceinline__ float stat_sum(float l, float lx) {
  return (PV && !F32 && STATS) ? lx : l;
}

// S^T of one 32-key step (rows: the step's keys, columns: the group's 64 queries).
template <typename T, int D>
__device__ __forceinline__ void qk(f32x16 (&s)[2], const KV<T, D>& b, const u32x4 (&q)[2][Tile<T, D>::KCH]) {
  using TL = Tile<T, D>;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    s[nt] = f32x16{};
    if constexpr (TL::F32) {
#pragma unroll
      for (int c = 0; c < TL::KCH; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          s[nt] = mfma_f32(__uint_as_float(b.k[c][j]), __uint_as_float(q[nt][c][j]), s[nt]);
    } else {
#pragma unroll
      for (int ks = 0; ks < TL::QK_STEPS; ++ks) s[nt] = mfma_bf16(as_bf16x8(b.k[ks]), as_bf16x8(q[nt][ks]), s[nt]);
    }
  }
}

template <int RB>
__device__ __forceinline__ void mask_tail(f32x16 (&s)[2], int t0, int nkeys, int hf) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (t0 + 16 * hf + r >= nkeys) s[nt][r] = -INFINITY;
}

// Probabilities exp2(s*c - m) with the offsets m fixed, their bf16 packing for the
// PV product, and the row sums.
template <typename T, int D, bool PV, bool STATS>
__device__ __forceinline__ void probs(State<T, D, PV>& st, f32x16 (&s)[2], uint32_t (&pk)[2][8], float c) {
  using TL = Tile<T, D>;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float moff = st.m[nt];
#pragma unroll
    for (int r = 0; r < 16; ++r) s[nt][r] = fast_exp2(__builtin_fmaf(s[nt][r], c, -moff));
    if constexpr (!TL::F32) {
#pragma unroll
      for (int i = 0; i < 8; ++i) pk[nt][i] = pack_bf16x2(s[nt][2 * i], s[nt][2 * i + 1]);
    }
    row_sums<PV, TL::F32, STATS>(st.l[nt], st.lx[nt], s[nt], pk[nt]);
  }
}

// Masking of entries past the key count and the online softmax update; leaves
// the step's probabilities exp2(s*c - m) in s.
template <typename T, int D, bool PV, bool STATS, bool MASK>
__device__ __forceinline__ void softmax(State<T, D, PV>& st, f32x16 (&s)[2], uint32_t (&pk)[2][8], int t0, int nkeys,
                                        float c, int hf) {
  using TL = Tile<T, D>;
  if constexpr (MASK) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (t0 + 16 * hf + r >= nkeys) s[nt][r] = -INFINITY;
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float mx = s[nt][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[nt][r]);
    mx = pair_max(mx) * c;
    // Lazy rescaling: the offset only moves when the maximum grows by more than
    // 2^8, so probabilities stay below 256 and the rescale of O is rare.
    const bool need = mx > st.m[nt] + 8.0f;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float mnew = need ? mx : st.m[nt];
      const float alpha = need ? fast_exp2(st.m[nt] - mnew) : 1.0f;
      st.l[nt] *= alpha;
      st.lx[nt] *= alpha;
      st.m[nt] = mnew;
      if constexpr (PV) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float ar = lane_read(alpha, 8 * (r >> 2) + 4 * hf + (r & 3));
#pragma unroll
          for (int cc = 0; cc < TL::VEC; ++cc) st.o[nt][cc][r] *= ar;
        }
      }
    }
    const float moff = st.m[nt] == -INFINITY ? 0.0f : st.m[nt];
#pragma unroll
    for (int r = 0; r < 16; ++r) s[nt][r] = fast_exp2(__builtin_fmaf(s[nt][r], c, -moff));
    if constexpr (!TL::F32) {
#pragma unroll
      for (int i = 0; i < 8; ++i) pk[nt][i] = pack_bf16x2(s[nt][2 * i], s[nt][2 * i + 1]);
    }
    row_sums<PV, TL::F32, STATS>(st.l[nt], st.lx[nt], s[nt], pk[nt]);
  }
}

// O += P * V_step.
template <typename T, int D, bool PV>
__device__ __forceinline__ void pv(State<T, D, PV>& st, const f32x16 (&p)[2], const uint32_t (&pk)[2][8],
                                   const KV<T, D>& b) {
  using TL = Tile<T, D>;
  if constexpr (TL::F32) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int kk = 0; kk < 16; ++kk)
#pragma unroll
        for (int cc = 0; cc < TL::VEC; ++cc)
          st.o[nt][cc] = mfma_f32(p[nt][kk], __uint_as_float(b.v[kk].w[cc]), st.o[nt][cc]);
  } else {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 pa[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pk[nt][4 * ks + i];
        pa[nt] = as_bf16x8(w);
      }
#pragma unroll
      for (int cc = 0; cc < TL::VEC; ++cc) {
        const uint32_t sel = (cc & 1) ? 0x07060302u : 0x05040100u;
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w[i] = __builtin_amdgcn_perm(vword(b.v[8 * ks + 2 * i + 1], cc), vword(b.v[8 * ks + 2 * i], cc), sel);
        const bf16x8 vb = as_bf16x8(w);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) st.o[nt][cc] = mfma_bf16(pa[nt], vb, st.o[nt][cc]);
      }
    }
  }
}

// Per-wave context of one query group.
template <typename T, int D, bool GATHER>
struct Ctx {
  __amdgpu_buffer_rsrc_t rk, rv, ridx;
  int nkeys, lm, hf;
  float c;
};

// Fixed-offset pass over the group's key list.  Each query's offset is the
// maximum of its first 32 logits plus kMargin (log2 units); every later
// probability is exp2(s*c - offset) with no running maximum and no rescaling of
// O, so a step is one straight basic block of MFMAs and VALU work.  A logit more
// than 2^(127 - kMargin) above the first tile's maximum overflows the row sum,
// which the caller detects and answers with the online pass below.
constexpr float kMargin = 16.0f;

template <typename T, int D, bool GATHER, bool PV>
__device__ __forceinline__ void fixed_step(State<T, D, PV>& st, const Ctx<T, D, GATHER>& x,
                                           const u32x4 (&q)[2][Tile<T, D>::KCH], KV<T, D>& b, const Idx& inext,
                                           Idx& ilater, int it) {
  // Step `it` with K/V already in flight in b; inext holds the keys of step it+1,
  // ilater receives those of step it+2.  The index loads are issued first so
  // that waiting for them never waits for this step's K/V gathers (the vector
  // memory counter retires in order).
  constexpr bool STATS = !GATHER;
  load_idx<GATHER>(ilater, x.ridx, (it + 2) * 32, x.lm, x.hf);
  f32x16 s[2];
  uint32_t pk[2][8];
  __builtin_amdgcn_sched_barrier(0);
  qk<T, D>(s, b, q);
  load_k<T, D>(b, inext, x.rk, x.hf);
  // keep the gathers where they are: sinking them toward the end of the step
  // (which the scheduler does to shorten live ranges) exposes their latency
  __builtin_amdgcn_sched_barrier(0);
  probs<T, D, PV, STATS>(st, s, pk, x.c);
  if constexpr (PV) {
    pv<T, D, PV>(st, s, pk, b);
    load_v<T, D>(b, inext, x.rv, x.lm);
  }
}

template <typename T, int D, bool GATHER, bool PV>
__device__ __forceinline__ void pass_fixed(State<T, D, PV>& st, const Ctx<T, D, GATHER>& x,
                                           const u32x4 (&q)[2][Tile<T, D>::KCH]) {
  constexpr bool STATS = !GATHER;
  Idx ia, ib;
  KV<T, D> b;
  const int nsteps = (x.nkeys + 31) >> 5;
  load_idx<GATHER>(ia, x.ridx, 0, x.lm, x.hf);
  load_k<T, D>(b, ia, x.rk, x.hf);
  if constexpr (PV) load_v<T, D>(b, ia, x.rv, x.lm);
  load_idx<GATHER>(ia, x.ridx, 32, x.lm, x.hf);
  load_idx<GATHER>(ib, x.ridx, 64, x.lm, x.hf);
  {  // first step: fixes the offsets
    f32x16 s[2];
    uint32_t pk[2][8];
    qk<T, D>(s, b, q);
    if (nsteps > 1) load_k<T, D>(b, ia, x.rk, x.hf);
    if (nsteps == 1) mask_tail<0>(s, 0, x.nkeys, x.hf);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float mx = s[nt][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[nt][r]);
      st.m[nt] = pair_max(mx) * x.c + kMargin;
    }
    probs<T, D, PV, STATS>(st, s, pk, x.c);
    if constexpr (PV) {
      pv<T, D, PV>(st, s, pk, b);
      if (nsteps > 1) load_v<T, D>(b, ia, x.rv, x.lm);
    }
  }
  ia = ib;
  // Middle steps: no masking, no branches around the prefetches (reads past the
  // key list return zeros or valid rows that are never used).  ia holds the keys
  // of step it+1; the step loads those of it+2 into ib first thing, so the copy
  // at the end waits only for that load, not for the K/V gathers issued after it.
#pragma unroll 1
  for (int it = 1; it + 1 < nsteps; ++it) {
    fixed_step<T, D, GATHER, PV>(st, x, q, b, ia, ib, it);
    ia = ib;
  }
  if (nsteps > 1) {
    f32x16 s[2];
    uint32_t pk[2][8];
    qk<T, D>(s, b, q);
    mask_tail<0>(s, (nsteps - 1) * 32, x.nkeys, x.hf);
    probs<T, D, PV, STATS>(st, s, pk, x.c);
    if constexpr (PV) pv<T, D, PV>(st, s, pk, b);
  }
}

// Q operand of the group: lane half hf of query column lm + 32*nt holds the
// dims of its half of every k-chunk.
template <typename T, int D>
__device__ __forceinline__ void load_q(__amdgpu_buffer_rsrc_t rq, const int (&tokq)[2], int hf,
                                       u32x4 (&q)[2][Tile<T, D>::KCH]) {
  using TL = Tile<T, D>;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const uint32_t qb = (uint32_t)tokq[nt] * TL::ROWB + TL::khalf_off(hf);
#pragma unroll
    for (int c = 0; c < TL::KCH; ++c) q[nt][c] = bload128(rq, qb + c * TL::KSTRIDE);
  }
}

// Online pass with a running maximum and lazy rescaling (the offset moves only
// when the maximum grows by more than 2^8).  Used only for groups whose
// fixed-offset pass overflowed.
template <typename T, int D, bool GATHER, bool PV, bool STATS>
__device__ __attribute__((noinline)) void pass_online(State<T, D, PV>& st, const Ctx<T, D, GATHER>& x,
                                                      __amdgpu_buffer_rsrc_t rq, int tok0, int tok1) {
  // Q is reloaded here rather than passed in: an array argument of a
  // non-inlined call would force the caller's copy into scratch memory.
  const int tokq[2] = {tok0, tok1};
  u32x4 q[2][Tile<T, D>::KCH];
  load_q<T, D>(rq, tokq, x.hf, q);
  Idx ix;
  KV<T, D> b;
  const int nsteps = (x.nkeys + 31) >> 5;
  for (int it = 0; it < nsteps; ++it) {
    load_idx<GATHER>(ix, x.ridx, it * 32, x.lm, x.hf);
    load_k<T, D>(b, ix, x.rk, x.hf);
    if constexpr (PV) load_v<T, D>(b, ix, x.rv, x.lm);
    f32x16 s[2];
    uint32_t pk[2][8];
    qk<T, D>(s, b, q);
    if (it + 1 == nsteps)
      softmax<T, D, PV, STATS, true>(st, s, pk, it * 32, x.nkeys, x.c, x.hf);
    else
      softmax<T, D, PV, STATS, false>(st, s, pk, it * 32, x.nkeys, x.c, x.hf);
    if constexpr (PV) pv<T, D, PV>(st, s, pk, b);
  }
}

template <typename T, int D, bool PV>
__device__ __forceinline__ void state_init(State<T, D, PV>& st) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    st.m[nt] = -INFINITY;
    st.l[nt] = 0.0f;
    st.lx[nt] = 0.0f;
    if constexpr (PV) {
#pragma unroll
      for (int cc = 0; cc < Tile<T, D>::VEC; ++cc) st.o[nt][cc] = f32x16{};
    }
  }
}

// Row statistics, normalisation and the epilogue stores of one group.
template <typename T, int D, int EPI, bool PV, bool STATS>
__device__ __forceinline__ void finish(const State<T, D, PV>& st, const AttnArgs& a, int h, const int (&tokq)[2],
                                       const bool (&qvalid)[2], int lm, int hf) {
  using TL = Tile<T, D>;
  const int N = a.N;
  float inv[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float lt = pair_sum(st.l[nt]);
    const float ls = pair_sum(stat_sum<PV, TL::F32, STATS>(st.l[nt], st.lx[nt]));
    inv[nt] = 1.0f / lt;
    if (hf == 0 && qvalid[nt]) {
      const size_t ri = (size_t)h * N + tokq[nt];
      if (a.stats) a.stats[ri] = make_float2(st.m[nt], 1.0f / ls);
      if (a.lse) a.lse[ri] = (st.m[nt] + __log2f(ls)) * kLn2;
    }
  }
  if constexpr (PV) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = 8 * (r >> 2) + 4 * hf + (r & 3);  // query row within this nt half
        const float ir = lane_read(inv[nt], qi);
        const int tok = lane_read_i(tokq[nt], qi);
        const int ok = lane_read_i(qvalid[nt] ? 1 : 0, qi);
        if (!ok) continue;  // padding slot of the last group, or an invalid perm entry
        const size_t base = ((size_t)h * N + tok) * D + (size_t)lm * TL::VEC;
        float vals[TL::VEC];
#pragma unroll
        for (int cc = 0; cc < TL::VEC; ++cc) vals[cc] = st.o[nt][cc][r] * ir;
        if constexpr (TL::F32) {
          const float* rin = (const float*)a.rin;
          float* out = (float*)a.o + base;
#pragma unroll
          for (int cc = 0; cc < TL::VEC; ++cc) {
            float v = vals[cc];
            if constexpr (EPI == EPI_ADD) v += rin[base + cc];
            if constexpr (EPI == EPI_RESID) v = rin[base + cc] - v;
            out[cc] = v;
          }
        } else {
          const __bf16* rin = (const __bf16*)a.rin;
          if constexpr (EPI != EPI_PLAIN) {
#pragma unroll
            for (int cc = 0; cc < TL::VEC; ++cc) {
              const float rv2 = (float)rin[base + cc];
              vals[cc] = EPI == EPI_ADD ? vals[cc] + rv2 : rv2 - vals[cc];
            }
          }
          uint32_t w[TL::VEC / 2];
#pragma unroll
          for (int i = 0; i < TL::VEC / 2; ++i) w[i] = pack_bf16x2(vals[2 * i], vals[2 * i + 1]);
          uint32_t* out = (uint32_t*)((__bf16*)a.o + base);
#pragma unroll
          for (int i = 0; i < TL::VEC / 2; ++i) out[i] = w[i];
        }
      }
    }
  }
}

template <typename T, int D, bool GATHER, int EPI, bool PV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_kernel(AttnArgs a) {
  using TL = Tile<T, D>;
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int hf = lane >> 5, lm = lane & 31;
  const int items = a.H * a.G;
  const int blk = xcd_remap(blockIdx.x, (items + 3) >> 2, a.xcd_chunk);
  if (blk < 0) return;
  const int item = blk * 4 + wid;
  if (item >= items) return;  // no block-level synchronisation below
  const int h = item / a.G, g = item - h * a.G;
  const int N = a.N;
  const size_t head_off = (size_t)h * N * TL::ROWB;
  const uint32_t head_bytes = (uint32_t)((size_t)N * TL::ROWB);
  const auto rq = make_rsrc((const char*)a.q + head_off, head_bytes);
  Ctx<T, D, GATHER> x;
  x.rk = make_rsrc((const char*)a.k + head_off, head_bytes);
  x.rv = make_rsrc((const char*)a.v + head_off, head_bytes);
  x.ridx = GATHER ? make_rsrc(a.idx + ((size_t)h * a.G + g) * a.kpad, (uint32_t)a.kpad * 4u) : make_rsrc(nullptr, 0);
  x.nkeys = a.nkeys;
  x.lm = lm;
  x.hf = hf;
  x.c = a.c;

  // This lane's two query columns (queries lm and lm + 32 of the group).
  int tokq[2];
  bool qvalid[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int slot = g * 64 + lm + 32 * nt;
    qvalid[nt] = slot < N;
    tokq[nt] = qvalid[nt] ? (a.perm ? a.perm[(size_t)h * N + slot] : slot) : 0;
    if (tokq[nt] < 0 || tokq[nt] >= N) {  // not a token (corrupt perm): compute nothing for it
      qvalid[nt] = false;
      tokq[nt] = 0;
    }
  }
  u32x4 q[2][TL::KCH];
  load_q<T, D>(rq, tokq, hf, q);

  State<T, D, PV> st;
  state_init<T, D, PV>(st);
  pass_fixed<T, D, GATHER, PV>(st, x, q);
  const bool ok = __builtin_isfinite(st.l[0]) && __builtin_isfinite(st.l[1]);
  if (__builtin_amdgcn_ballot_w64(!ok)) {
    State<T, D, PV> so;
    state_init<T, D, PV>(so);
    pass_online<T, D, GATHER, PV, !GATHER>(so, x, rq, tokq[0], tokq[1]);
    finish<T, D, EPI, PV, !GATHER>(so, a, h, tokq, qvalid, lm, hf);
  } else {
    finish<T, D, EPI, PV, !GATHER>(st, a, h, tokq, qvalid, lm, hf);
  }
}

// ---------------------------------------------------------------------------
// bf16 path with K/V staged through LDS.
//
// Fetching a K row straight into the MFMA operand layout puts a different row
// in every lane of a quad, which costs the texture-address unit four cycles per
// quad: the gathers of a step, not the MFMAs, set the pace.  Here every step's
// 32 K rows and 32 V rows are copied global -> LDS with buffer_load ... lds,
// each lane quad reading 64 contiguous bytes of one row (one cycle per quad),
// and the operands are read from LDS: K with ds_read_b128, V with the gfx950
// transposing read ds_read_b64_tr_b16, which hands every lane one dimension of
// four keys, i.e. the PV B-operand layout, with no register shuffles.
//
// Tile geometry (one K or V tile = the 32 rows of one step):
//   a DMA instruction moves 1 KiB = RPI rows; lane j of instruction i fetches
//   16-byte chunk (j % LPR) ^ swz(g) of step entry NI*g + i, g = j / LPR, and it
//   lands at LDS offset i*BLK + 16*j.  So entry e sits in block e % NI, row
//   e / NI, and its chunk x at position x ^ swz(e / NI).  The 32-byte skew
//   between blocks and the XOR swizzle inside 64-byte groups spread the rows a
//   ds_read touches together over the LDS banks; the swizzle never leaves a
//   64-byte group, so a quad still reads one contiguous 64-byte piece.
//   Entry e of the step is row e of S^T, so the accumulator register r of lane
//   half hf holds entry 8*(r/4) + 4*hf + r%4.
// Two stages (separate LDS arrays, so the compiler's wait counting can tell the
// in-flight copy of step i+1 from the one step i reads) alternate.

template <int D>
struct LKeys {
  int k[LT<D>::NI];
};

template <int D, bool PV>
struct LState {
  f32x16 o[2][LT<D>::VT];
  float m[2];
  float l[2];   // normaliser of O (see row_sums)
  float lx[2];  // exact sum for the row statistics when l is the packed one
};

// Keys of the NI entries this lane copies (entries NI*g + 0..NI-1 of the step).
template <int D, bool GATHER>
__device__ __forceinline__ void lkeys(LKeys<D>& kk, __amdgpu_buffer_rsrc_t ridx, int t0, int ebase) {
  using L = LT<D>;
  if constexpr (GATHER) {
#pragma unroll
    for (int c = 0; c < L::NI / 4; ++c) {
      const u32x4 w = bload128(ridx, (uint32_t)(t0 + ebase + 4 * c) * 4u);
#pragma unroll
      for (int j = 0; j < 4; ++j) kk.k[4 * c + j] = (int)w[j];
    }
  } else {
#pragma unroll
    for (int i = 0; i < L::NI; ++i) kk.k[i] = t0 + ebase + i;
  }
}

// Start the copies of one step's K (and V) rows into a stage.  A key of -1 (a
// padding entry) or past the sequence gives an offset beyond the buffer, which
// the buffer unit answers with zeros; those entries are masked anyway.
template <int D, bool PV>
__device__ __forceinline__ void ldma(LDSP char* stage, const LKeys<D>& kk, __amdgpu_buffer_rsrc_t rk,
                                     __amdgpu_buffer_rsrc_t rv, uint32_t goff) {
  using L = LT<D>;
#pragma unroll
  for (int i = 0; i < L::NI; ++i) {
    const uint32_t vo = (uint32_t)kk.k[i] * (uint32_t)L::ROWB + goff;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (LDSP void*)(stage + i * L::BLK), 16, vo, 0, 0, 0);
    if constexpr (PV)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (LDSP void*)(stage + L::TILE + i * L::BLK), 16, vo, 0, 0, 0);
  }
}

template <int D>
__device__ __forceinline__ void lkread(u32x4 (&ka)[LT<D>::KCH], const LDSP char* stage, const int (&kaddr)[2]) {
#pragma unroll
  for (int ks = 0; ks < LT<D>::KCH; ++ks) ka[ks] = *(const LDSP u32x4*)(stage + kaddr[ks & 1] + 64 * (ks >> 1));
}

template <int D>
__device__ __forceinline__ void lqk(f32x16 (&s)[2], const u32x4 (&ka)[LT<D>::KCH], const u32x4 (&q)[2][LT<D>::KCH]) {
  s[0] = f32x16{};
  s[1] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < LT<D>::KCH; ++ks)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) s[nt] = mfma_bf16(as_bf16x8(ka[ks]), as_bf16x8(q[nt][ks]), s[nt]);
}

__device__ __forceinline__ void lmask(f32x16 (&s)[2], int t0, int nkeys, int hf) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (t0 + 8 * (r >> 2) + 4 * hf + (r & 3) >= nkeys) s[nt][r] = -INFINITY;
}

template <int D, bool PV, bool STATS>
__device__ __forceinline__ void lprobs(LState<D, PV>& st, f32x16 (&s)[2], uint32_t (&pk)[2][8], float c) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float moff = st.m[nt];
#pragma unroll
    for (int r = 0; r < 16; ++r) s[nt][r] = fast_exp2(__builtin_fmaf(s[nt][r], c, -moff));
    if constexpr (PV) {
#pragma unroll
      for (int i = 0; i < 8; ++i) pk[nt][i] = pack_bf16x2(s[nt][2 * i], s[nt][2 * i + 1]);
    }
    row_sums<PV, false, STATS>(st.l[nt], st.lx[nt], s[nt], pk[nt]);
  }
}

// V operands of one step: for key chunk kc and output tile n, two transposing
// reads give a lane dimension 32*n + lane%32 of the 8 keys its k-slots name.
template <int D>
__device__ __forceinline__ void lvread(bf16x8 (&vb)[2][LT<D>::VT], const LDSP char* stage, const int (&vaddr)[2][2]) {
  using L = LT<D>;
  typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
  const LDSP char* vt = stage + L::TILE;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int n = 0; n < L::VT; ++n) {
      const bf4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDSP bf4*)(vt + vaddr[kc][0] + 64 * n));
      const bf4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDSP bf4*)(vt + vaddr[kc][1] + 64 * n));
      vb[kc][n] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

template <int D>
__device__ __forceinline__ void lpv(LState<D, true>& st, const uint32_t (&pk)[2][8], const bf16x8 (&vb)[2][LT<D>::VT]) {
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    bf16x8 pa[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = pk[nt][4 * kc + i];
      pa[nt] = as_bf16x8(w);
    }
#pragma unroll
    for (int n = 0; n < LT<D>::VT; ++n)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) st.o[nt][n] = mfma_bf16(pa[nt], vb[kc][n], st.o[nt][n]);
  }
}

// Per-lane context of the LDS path.
template <int D>
struct LCtx {
  __amdgpu_buffer_rsrc_t rk, rv, ridx;
  int nkeys, hf, ebase;
  uint32_t goff;
  int kaddr[2];
  int vaddr[2][2];
  float c;
};


// One step on stage `cur`.  DMA_NEXT: start the copies of step it+1 into `nxt`
// (keys in kn) and load the keys of step it+2 into kn; FIRST: fix the offsets
// from this step's maxima; LAST: mask entries past the key count.
template <int D, bool GATHER, bool PV, bool STATS, bool FIRST, bool LAST, bool DMA_NEXT>
__device__ __forceinline__ void lstep(LState<D, PV>& st, const LCtx<D>& x, const u32x4 (&q)[2][LT<D>::KCH],
                                      const LDSP char* cur, LDSP char* nxt, const LKeys<D>& kcur, LKeys<D>& knext,
                                      int it) {
  constexpr int NKL = GATHER ? LT<D>::NI / 4 : 0;        // key loads per step
  constexpr int NDMA = (PV ? 2 : 1) * LT<D>::NI;         // copy instructions per step
  // The copies of step it+1 (keys in kcur) and the key load of step it+2 go out
  // before waiting for this step's copies, so two steps of rows are in flight
  // while the wave waits: the gathers are bound by the cache hierarchy's
  // latency, and one step in flight per wave is too little to cover it.
  if constexpr (DMA_NEXT) {
    lkeys<D, GATHER>(knext, x.ridx, (it + 2) * 32, x.ebase);
    ldma<D, PV>(nxt, kcur, x.rk, x.rv, x.goff);
    // this step's copies landed once at most those two batches remain
    wait_vm<NKL + NDMA>();
  } else {
    wait_vm<0>();
  }
  __builtin_amdgcn_sched_barrier(0);
  u32x4 ka[LT<D>::KCH];
  lkread<D>(ka, cur, x.kaddr);
  __builtin_amdgcn_sched_barrier(0);
  f32x16 s[2];
  uint32_t pk[2][8];
  lqk<D>(s, ka, q);
  __builtin_amdgcn_sched_barrier(0);
  bf16x8 vb[2][LT<D>::VT];
  if constexpr (PV) lvread<D>(vb, cur, x.vaddr);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (LAST) lmask(s, it * 32, x.nkeys, x.hf);
  if constexpr (FIRST) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float mx = s[nt][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[nt][r]);
      st.m[nt] = pair_max(mx) * x.c + kMargin;
    }
  }
  lprobs<D, PV, STATS>(st, s, pk, x.c);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (PV) lpv<D>(st, pk, vb);
}

// The whole key list: first step, a branch-free middle of step pairs on the two
// stages (no masking; the key prefetch may read past the list, which returns
// zeros or unused entries), then at most one more middle step and the masked
// last step.  Step j's rows live in stage j % 2; the keys of steps alternate
// between ka and kb the same way.
//
// FRESH: the pass starts the softmax (its first step fixes the offsets); false
// when steps over other keys of the same queries came before it.
template <int D, bool GATHER, bool PV, bool STATS, bool FRESH = true>
__device__ __forceinline__ void lpass(LState<D, PV>& st, const LCtx<D>& x, const u32x4 (&q)[2][LT<D>::KCH],
                                      LDSP char* s0, LDSP char* s1) {
  const int nsteps = (x.nkeys + 31) >> 5;
  LKeys<D> ka, kb;
  lkeys<D, GATHER>(ka, x.ridx, 0, x.ebase);
  ldma<D, PV>(s0, ka, x.rk, x.rv, x.goff);
  lkeys<D, GATHER>(kb, x.ridx, 32, x.ebase);
  if (nsteps == 1) {
    lstep<D, GATHER, PV, STATS, FRESH, true, false>(st, x, q, s0, s1, kb, ka, 0);
    return;
  }
  lstep<D, GATHER, PV, STATS, FRESH, false, true>(st, x, q, s0, s1, kb, ka, 0);
  int it = 1;
  for (; it + 2 < nsteps; it += 2) {
    lstep<D, GATHER, PV, STATS, false, false, true>(st, x, q, s1, s0, ka, kb, it);
    lstep<D, GATHER, PV, STATS, false, false, true>(st, x, q, s0, s1, kb, ka, it + 1);
  }
  // it is odd: stage s1 holds step it
  if (it + 1 < nsteps) {
    lstep<D, GATHER, PV, STATS, false, false, true>(st, x, q, s1, s0, ka, kb, it);
    lstep<D, GATHER, PV, STATS, false, true, false>(st, x, q, s0, s1, kb, ka, it + 1);
  } else {
    lstep<D, GATHER, PV, STATS, false, true, false>(st, x, q, s1, s0, ka, kb, it);
  }
}

// Normalisation, statistics and epilogue of the LDS path.  O goes through LDS
// (fp32, SROWS query rows at a time; buf holds SROWS * OPITCH bytes) so that every
// lane stores 16 contiguous bytes of one output row, and the residual is added in
// fp32 before the single rounding to bf16.
template <int D, int EPI, bool PV, bool STATS, int SROWS = 32>
__device__ __forceinline__ void lfinish(const LState<D, PV>& st, const AttnArgs& a, int h, const int (&tokq)[2],
                                        const bool (&qvalid)[2], int lane, LDSP char* buf) {
  using L = LT<D>;
  const int N = a.N, hf = lane >> 5, lm = lane & 31;
  float inv[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float lt = pair_sum(st.l[nt]);
    const float ls = pair_sum(stat_sum<PV, false, STATS>(st.l[nt], st.lx[nt]));
    inv[nt] = 1.0f / lt;
    if (hf == 0 && qvalid[nt]) {
      const size_t ri = (size_t)h * N + tokq[nt];
      if (a.stats) a.stats[ri] = make_float2(st.m[nt], 1.0f / ls);
      if (a.lse) a.lse[ri] = (st.m[nt] + __log2f(ls)) * kLn2;
    }
  }
  if constexpr (PV) {
    constexpr int LPO = D / 8;        // lanes per output row (8 dims each)
    constexpr int RPO = 64 / LPO;     // rows per pass
    static_assert(SROWS % 8 == 0 && 32 % SROWS == 0 && SROWS % RPO == 0, "staging rows");
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int tok_l = tokq[nt], ok_l = qvalid[nt] ? 1 : 0;
      const int ch = lane % LPO;
#pragma unroll
      for (int hb = 0; hb < 32 / SROWS; ++hb) {
        // accumulator register r holds row 8*(r/4) + 4*hf + r%4; the rows of this
        // round are [hb*SROWS, (hb+1)*SROWS).  A wave's LDS accesses are done in
        // order, so the next round's writes follow this round's reads.
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if ((8 * (r >> 2)) / SROWS != hb) continue;
          const int qi = 8 * (r >> 2) + 4 * hf + (r & 3);
          const float ir = lane_read(inv[nt], qi);
#pragma unroll
          for (int n = 0; n < L::VT; ++n)
            *(LDSP float*)(buf + (qi - hb * SROWS) * L::OPITCH + (32 * n + lm) * 4) = st.o[nt][n][r] * ir;
        }
#pragma unroll
        for (int p = 0; p < SROWS / RPO; ++p) {
          const int qr = p * RPO + lane / LPO;
          const int qi = hb * SROWS + qr;
          const LDSP char* src = buf + qr * L::OPITCH + ch * 32;
          const f32x4 v0 = *(const LDSP f32x4*)src;
          const f32x4 v1 = *(const LDSP f32x4*)(src + 16);
          const int tok = lane_read_i(tok_l, qi);
          const int ok = lane_read_i(ok_l, qi);
          float vals[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
          if (ok) {
            const size_t base = ((size_t)h * N + tok) * D + (size_t)ch * 8;
            if constexpr (EPI != EPI_PLAIN) {
              const u32x4 rw = *(const u32x4*)((const __bf16*)a.rin + base);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float r0 = bf16lo(rw[i]), r1 = bf16hi(rw[i]);
                vals[2 * i] = EPI == EPI_ADD ? vals[2 * i] + r0 : r0 - vals[2 * i];
                vals[2 * i + 1] = EPI == EPI_ADD ? vals[2 * i + 1] + r1 : r1 - vals[2 * i + 1];
              }
            }
            u32x4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(vals[2 * i], vals[2 * i + 1]);
            *(u32x4*)((__bf16*)a.o + base) = w;
          }
        }
      }
    }
  }
}

// Per-lane context of group g of head h: buffer descriptors of K, V and the
// group's key list, and the LDS addresses of this lane's copy chunk and MFMA
// operands.
template <int D, bool GATHER>
__device__ __forceinline__ void lctx_init(LCtx<D>& x, const AttnArgs& a, int h, int g, int lane) {
  using L = LT<D>;
  const int hf = lane >> 5, lm = lane & 31;
  const size_t head_off = (size_t)h * a.N * L::ROWB;
  const uint32_t head_bytes = (uint32_t)((size_t)a.N * L::ROWB);
  x.rk = make_rsrc((const char*)a.k + head_off, head_bytes);
  x.rv = make_rsrc((const char*)a.v + head_off, head_bytes);
  x.ridx = GATHER ? make_rsrc(a.idx + ((size_t)h * a.G + g) * a.kpad, (uint32_t)a.kpad * 4u) : make_rsrc(nullptr, 0);
  x.nkeys = a.nkeys;
  x.hf = hf;
  x.c = a.c;
  {
    const int gd = lane / L::LPR, cj = lane % L::LPR;
    x.goff = 16u * (uint32_t)(cj ^ L::swz(gd));
    x.ebase = L::NI * gd;
    // K operand: lane row m = lm (entry m), chunk 2*ks + hf
#pragma unroll
    for (int v = 0; v < 2; ++v) x.kaddr[v] = L::off(lm, 2 * v + hf);
    // V operand (transposing read): lane i of its 16-lane group supplies the
    // address of 4 dims of one key; see lpv for the resulting layout
    const int g16 = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int sr = 0; sr < 2; ++sr) {
        const int e = 16 * kc + 8 * sr + 4 * (g16 >> 1) + (i16 >> 2);
        const int xch = 2 * (g16 & 1) + ((i16 & 3) >> 1);
        x.vaddr[kc][sr] = L::off(e, xch) + 8 * (i16 & 1);
      }
  }
}

// Token ids (through perm) and validity of the lane's two query columns, and
// the group's Q operands (kept in registers for the whole pass).
template <int D>
__device__ __forceinline__ void lqueries(int (&tokq)[2], bool (&qvalid)[2], u32x4 (&q)[2][LT<D>::KCH],
                                         const AttnArgs& a, __amdgpu_buffer_rsrc_t rq, int h, int g, int lane) {
  using L = LT<D>;
  const int N = a.N, hf = lane >> 5, lm = lane & 31;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int slot = g * 64 + lm + 32 * nt;
    qvalid[nt] = slot < N;
    tokq[nt] = qvalid[nt] ? (a.perm ? a.perm[(size_t)h * N + slot] : slot) : 0;
    if (tokq[nt] < 0 || tokq[nt] >= N) {
      qvalid[nt] = false;
      tokq[nt] = 0;
    }
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const uint32_t qb = (uint32_t)tokq[nt] * L::ROWB + 16u * hf;
#pragma unroll
    for (int c = 0; c < L::KCH; ++c) q[nt][c] = bload128(rq, qb + c * 32);
  }
}

// Bytes of one stage: K and V tiles (also the epilogue's O buffer) with the PV
// product, the K tile alone without it.
template <int D, bool PV>
constexpr int stage_bytes() { return PV ? LT<D>::STAGE : LT<D>::TILE; }

// Stages start zeroed: a padding entry's copy may leave its slot untouched,
// and a masked probability times a stale non-finite value would poison O.
template <int D, bool PV = true>
__device__ __forceinline__ void lzero(LDSP char* s0, LDSP char* s1, int lane) {
  for (int o = lane * 16; o < stage_bytes<D, PV>(); o += 64 * 16) {
    *(LDSP u32x4*)(s0 + o) = u32x4{0, 0, 0, 0};
    *(LDSP u32x4*)(s1 + o) = u32x4{0, 0, 0, 0};
  }
  // The copies that follow land in LDS through the texture path, not in order
  // behind these stores: the stores must be done before the first copy is issued.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

template <int D, bool PV>
__device__ __forceinline__ void lstate_init(LState<D, PV>& st) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    st.m[nt] = 0.0f;
    st.l[nt] = 0.0f;
    st.lx[nt] = 0.0f;
    if constexpr (PV) {
#pragma unroll
      for (int n = 0; n < LT<D>::VT; ++n) st.o[nt][n] = f32x16{};
    }
  }
}

// Normalise and store, or, if a logit far above its query's first-tile maximum
// overflowed the fixed offset, redo the group with the online pass (direct
// global loads over the whole key list of x.ridx).
template <int D, bool GATHER, int EPI, bool PV, bool STATS, int SROWS = 32>
__device__ __forceinline__ void lend(const LState<D, PV>& st, const LCtx<D>& x, const AttnArgs& a,
                                     __amdgpu_buffer_rsrc_t rq, int h, const int (&tokq)[2],
                                     const bool (&qvalid)[2], int lane, LDSP char* buf) {
  const int hf = lane >> 5, lm = lane & 31;
  const bool ok = __builtin_isfinite(st.l[0]) && __builtin_isfinite(st.l[1]);
  if (__builtin_amdgcn_ballot_w64(!ok)) {
    Ctx<__bf16, D, GATHER> xo;
    xo.rk = x.rk;
    xo.rv = x.rv;
    xo.ridx = x.ridx;
    xo.nkeys = x.nkeys;
    xo.lm = lm;
    xo.hf = hf;
    xo.c = x.c;
    State<__bf16, D, PV> so;
    state_init<__bf16, D, PV>(so);
    pass_online<__bf16, D, GATHER, PV, STATS>(so, xo, rq, tokq[0], tokq[1]);
    finish<__bf16, D, EPI, PV, STATS>(so, a, h, tokq, qvalid, lm, hf);
  } else {
    lfinish<D, EPI, PV, STATS, SROWS>(st, a, h, tokq, qvalid, lane, buf);
  }
}

// STATS (dense with PV only): also keep the exact row sums for the statistics;
// the other variants have one sum (see row_sums).
// Without the PV product (selection pass 1, sparse logsumexp) a stage holds only
// the K tile, so two blocks fit a CU: a wave issues in order and its own MFMAs
// and VALU do not overlap, but a second wave per SIMD runs its exponentials
// beside the first one's MFMAs.
template <int D, bool GATHER, int EPI, bool PV, bool STATS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(PV ? 1 : 2, PV ? 1 : 2)))
void attn_lds_kernel(AttnArgs a) {
  using L = LT<D>;
  __shared__ __attribute__((aligned(16))) char stage0[4][stage_bytes<D, PV>()];
  __shared__ __attribute__((aligned(16))) char stage1[4][stage_bytes<D, PV>()];
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int items = a.H * a.G;
  const int blk = xcd_remap(blockIdx.x, (items + 3) >> 2, a.xcd_chunk);
  if (blk < 0) return;
  const int item = blk * 4 + wid;
  if (item >= items) return;  // waves are independent: no block-level synchronisation
  const int h = item / a.G, g = item - h * a.G;
  const auto rq = make_rsrc((const char*)a.q + (size_t)h * a.N * L::ROWB, (uint32_t)((size_t)a.N * L::ROWB));
  LDSP char* s0 = (LDSP char*)&stage0[wid][0];
  LDSP char* s1 = (LDSP char*)&stage1[wid][0];

  LCtx<D> x;
  lctx_init<D, GATHER>(x, a, h, g, lane);
  int tokq[2];
  bool qvalid[2];
  u32x4 q[2][L::KCH];
  lqueries<D>(tokq, qvalid, q, a, rq, h, g, lane);
  lzero<D, PV>(s0, s1, lane);
  LState<D, PV> st;
  lstate_init<D, PV>(st);
  if (x.nkeys > 0) lpass<D, GATHER, PV, STATS>(st, x, q, s0, s1);
  lend<D, GATHER, EPI, PV, STATS>(st, x, a, rq, h, tokq, qvalid, lane, s0);
}

// ---------------------------------------------------------------------------
// Gather sharing between neighbouring groups.  Groups 2p and 2p+1 of a head are
// adjacent leaves of the PDDP tree (similar queries), and their kept-key sets
// overlap: on the 75,600-token workload at density 0.2 about 40% of a group's
// keys are also kept by its neighbour.  The gather of a K/V row into LDS is the
// bound of this kernel, and the MFMA work per gathered row is fixed by C, so a
// row that both groups keep is gathered once and consumed by both.
//
// The pair plan (mcs_pair_plan) reorders each group's list as [nc keys common to
// both groups, ascending | the group's other keys, ascending], nc a multiple of
// 128.  One block of two waves takes one pair.  Over the common prefix the waves
// move in macro-steps of two tiles: each wave copies one 32-key tile into its own
// stage and both waves consume both tiles (one block barrier per macro-step, so
// each copied row feeds 128 queries).  Then each wave walks its private keys
// alone with the ordinary two-stage pass.  Every group still attends to exactly
// its own K keys; only the order of the softmax sums differs from the plain
// kernel.
// ---------------------------------------------------------------------------

// The MFMA work of one tile already in LDS (no copies, no waits).
template <int D, bool FIRST>
__device__ __forceinline__ void lcompute(LState<D, true>& st, const LCtx<D>& x, const u32x4 (&q)[2][LT<D>::KCH],
                                         const LDSP char* cur) {
  // keep the two tiles of a macro-step apart: overlapping them costs registers
  __builtin_amdgcn_sched_barrier(0);
  u32x4 ka[LT<D>::KCH];
  lkread<D>(ka, cur, x.kaddr);
  __builtin_amdgcn_sched_barrier(0);
  f32x16 s[2];
  uint32_t pk[2][8];
  lqk<D>(s, ka, q);
  __builtin_amdgcn_sched_barrier(0);
  bf16x8 vb[2][LT<D>::VT];
  lvread<D>(vb, cur, x.vaddr);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (FIRST) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float mx = s[nt][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[nt][r]);
      st.m[nt] = pair_max(mx) * x.c + kMargin;
    }
  }
  lprobs<D, true, false>(st, s, pk, x.c);
  __builtin_amdgcn_sched_barrier(0);
  lpv<D>(st, pk, vb);
  __builtin_amdgcn_sched_barrier(0);
}

// One macro-step over the common prefix: t0 / t1 are the tiles the two waves
// copied (wave 0's, wave 1's stage).  ISSUE: start this wave's copy of the next
// macro-step into own_next (keys in kn) and load the keys of the one after that
// (list entry entry_nn) into knn.
template <int D, bool FIRST, bool ISSUE>
__device__ __forceinline__ void lmacro(LState<D, true>& st, const LCtx<D>& x, const u32x4 (&q)[2][LT<D>::KCH],
                                       const LDSP char* t0, const LDSP char* t1, LDSP char* own_next,
                                       const LKeys<D>& kn, LKeys<D>& knn, int entry_nn) {
  // Drain this wave's loads: the current tiles' copies and the keys of the next
  // copy, all issued a macro-step ago.  A count that spares the key loads would
  // rely on their issue order, which the compiler is free to change (it hoists
  // key loads above earlier copies), and a copy still in flight would then be
  // read by both waves.  The barrier makes the partner's copies visible too,
  // and tells that both waves finished reading the stages of the macro-step
  // before (the ones the copies below overwrite).
  wait_vm<0>();
  block_barrier();
  if constexpr (ISSUE) {
    ldma<D, true>(own_next, kn, x.rk, x.rv, x.goff);
    lkeys<D, true>(knn, x.ridx, entry_nn, x.ebase);
  }
  lcompute<D, FIRST>(st, x, q, t0);
  lcompute<D, false>(st, x, q, t1);
  // both tiles' LDS reads are complete before this wave reaches the next barrier
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

template <int D, int EPI>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_pairs_kernel(AttnArgs a, const int32_t* ncommon) {
  using L = LT<D>;
  __shared__ __attribute__((aligned(16))) char stage0[2][L::STAGE];
  __shared__ __attribute__((aligned(16))) char stage1[2][L::STAGE];
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int P = (a.G + 1) >> 1;
  const int blk = xcd_remap(blockIdx.x, a.H * P, a.xcd_chunk);
  if (blk < 0) return;
  const int h = blk / P, p = blk - h * P;
  const int g = 2 * p + wid;
  if (g >= a.G) return;  // the last pair of an odd G has one group (and shares nothing)
  // A count that is not a multiple of 128 within [0, K], or a lone group, falls
  // back to no sharing: each row still lists all of its group's keys.
  int nc = __builtin_amdgcn_readfirstlane(ncommon[(size_t)h * P + p]);
  if (2 * p + 1 >= a.G || nc < 0 || nc > a.nkeys || (nc & 127) != 0) nc = 0;
  const auto rq = make_rsrc((const char*)a.q + (size_t)h * a.N * L::ROWB, (uint32_t)((size_t)a.N * L::ROWB));
  LDSP char* own0 = (LDSP char*)&stage0[wid][0];
  LDSP char* own1 = (LDSP char*)&stage1[wid][0];

  LCtx<D> x;
  lctx_init<D, true>(x, a, h, g, lane);
  int tokq[2];
  bool qvalid[2];
  u32x4 q[2][L::KCH];
  lqueries<D>(tokq, qvalid, q, a, rq, h, g, lane);
  lzero<D>(own0, own1, lane);
  LState<D, true> st;
  lstate_init<D, true>(st);

  const int ns = nc >> 6;  // macro-steps (even)
  if (ns > 0) {
    const LDSP char* a0 = (const LDSP char*)&stage0[0][0];
    const LDSP char* b0 = (const LDSP char*)&stage0[1][0];
    const LDSP char* a1 = (const LDSP char*)&stage1[0][0];
    const LDSP char* b1 = (const LDSP char*)&stage1[1][0];
    // copy c of this wave is list entries 32*(2c + wid) .. +31, into stage c % 2
    LKeys<D> ka, kb;
    lkeys<D, true>(ka, x.ridx, 32 * wid, x.ebase);
    ldma<D, true>(own0, ka, x.rk, x.rv, x.goff);
    lkeys<D, true>(kb, x.ridx, 32 * (2 + wid), x.ebase);
    lmacro<D, true, true>(st, x, q, a0, b0, own1, kb, ka, 32 * (4 + wid));
    int m = 1;
    for (; m + 2 < ns; m += 2) {
      lmacro<D, false, true>(st, x, q, a1, b1, own0, ka, kb, 32 * (2 * (m + 2) + wid));
      lmacro<D, false, true>(st, x, q, a0, b0, own1, kb, ka, 32 * (2 * (m + 3) + wid));
    }
    lmacro<D, false, false>(st, x, q, a1, b1, own0, ka, kb, 0);
    // both waves are done with every stage before the private passes refill them
    block_barrier();
  }
  const int npriv = a.nkeys - nc;
  if (npriv > 0) {
    LCtx<D> xp = x;
    xp.ridx = make_rsrc(a.idx + ((size_t)h * a.G + g) * a.kpad + nc, (uint32_t)(a.kpad - nc) * 4u);
    xp.nkeys = npriv;
    if (ns == 0)
      lpass<D, true, true, false, true>(st, xp, q, own0, own1);
    else
      lpass<D, true, true, false, false>(st, xp, q, own0, own1);
  }
  lend<D, true, EPI, true, false>(st, x, a, rq, h, tokq, qvalid, lane, own0);
}

// ---------------------------------------------------------------------------
// Dense attention at two waves per SIMD.  Within a step a wave's softmax needs its
// QK product and its PV product needs the softmax, so at one wave per SIMD a step
// costs the MFMA time and the VALU time one after the other.
// Here a block's waves (eight at D = 128, one block per CU; four at D = 64, two
// blocks per CU) take consecutive 64-query groups of one head and share a ring of
// kDenseStages K/V stages (every group of a head reads every key in the same
// order): each wave issues its share of each step's copies, and one block barrier
// per step marks "this step's copies landed everywhere, the stage read in the step
// before is free".  With the K and V operands read from LDS a few chunks ahead
// of the MFMAs that use them (not all eight chunks at once), a wave fits in 256
// registers, and the two waves of a SIMD run one's exponentials beside the other's
// MFMAs.  Per query the arithmetic is that of the one-wave-per-SIMD kernel, in the
// same order.
constexpr int kDenseStages = 4;
// Waves per block: one copy instruction of each tile per wave and step.
template <int D>
constexpr int dense_waves() { return LT<D>::NI >= 8 ? 8 : 4; }
// LDS operand reads in flight ahead of the MFMAs: K chunks of the QK product,
// V chunk pairs of the PV product.  With one read in flight each MFMA pair waits
// a full LDS round trip.
constexpr int kDenseKAhead = 3;
constexpr int kDenseVAhead = 2;

// This wave's share of the copies of step j (K and V tiles) into its ring stage.
template <int D, int NS>
__device__ __forceinline__ void ring_copy(LDSP char* ring0, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                          int j, int ebase, uint32_t goff, int wid) {
  constexpr int NC = LT<D>::NI / dense_waves<D>();
  LDSP char* stg = ring0 + (j % NS) * LT<D>::STAGE;
  tile_copy_dense<D, NC>(stg, rk, j, ebase, goff, wid * NC);
  tile_copy_dense<D, NC>(stg + LT<D>::TILE, rv, j, ebase, goff, wid * NC);
}

// One step of a 64-query wave on stage `cur` (no waits).  The step's ring
// copies (step it + NS - 1) go out right after its last V read: the compiler
// waits for every copy in flight before a stage's first transposing read, so a
// copy issued in this step has a whole step to land before it is waited for.
template <int D, bool STATS, bool FIRST, bool LAST, int NS>
__device__ __forceinline__ void rstep(LState<D, true>& st, const LCtx<D>& x, const u32x4 (&q)[2][LT<D>::KCH],
                                      const LDSP char* cur, int it, LDSP char* ring0, int wid) {
  using L = LT<D>;
  typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
  constexpr int KCH = L::KCH, KA = kDenseKAhead, VA = kDenseVAhead, NV = 2 * L::VT;
  static_assert(KA <= KCH && VA <= NV, "read-ahead depth");
  // QK: chunk ks + KA is read while the MFMAs of chunk ks run
  f32x16 s[2] = {f32x16{}, f32x16{}};
  u32x4 ka[KCH];
#pragma unroll
  for (int ks = 0; ks < KA; ++ks) ka[ks] = *(const LDSP u32x4*)(cur + x.kaddr[ks & 1] + 64 * (ks >> 1));
  __builtin_amdgcn_sched_group_barrier(0x100, KA, 0);  // DS reads
#pragma unroll
  for (int ks = 0; ks < KCH; ++ks) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) s[nt] = mfma_bf16(as_bf16x8(ka[ks]), as_bf16x8(q[nt][ks]), s[nt]);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMAs
    if (ks + KA < KCH) {
      ka[ks + KA] = *(const LDSP u32x4*)(cur + x.kaddr[(ks + KA) & 1] + 64 * ((ks + KA) >> 1));
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (LAST) lmask(s, it * 32, x.nkeys, x.hf);
  if constexpr (FIRST) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float mx = s[nt][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[nt][r]);
      st.m[nt] = pair_max(mx) * x.c + kMargin;
    }
  }
  uint32_t pk[2][8];
  lprobs<D, true, STATS>(st, s, pk, x.c);
  __builtin_amdgcn_sched_barrier(0);
  // PV: operand c = (key chunk c / VT, output tile c % VT); two transposing
  // reads give the operand, read VA operands ahead
  const LDSP char* vt = cur + L::TILE;
  bf16x8 vb[NV];
  auto vread = [&](int c) {
    const int kc = c / L::VT, n = c % L::VT;
    const bf4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDSP bf4*)(vt + x.vaddr[kc][0] + 64 * n));
    const bf4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDSP bf4*)(vt + x.vaddr[kc][1] + 64 * n));
    vb[c] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
#pragma unroll
  for (int c = 0; c < VA; ++c) vread(c);
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * VA, 0);
#pragma unroll
  for (int c = 0; c < NV; ++c) {
    const int kc = c / L::VT, n = c % L::VT;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = pk[nt][4 * kc + i];
      st.o[nt][n] = mfma_bf16(as_bf16x8(w), vb[c], st.o[nt][n]);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    if (c + VA < NV) {
      vread(c + VA);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    if (c + VA == NV) {
      ring_copy<D, NS>(ring0, x.rk, x.rv, it + NS - 1, x.ebase, x.goff, wid);
      __builtin_amdgcn_sched_group_barrier(0x020, 2 * (L::NI / dense_waves<D>()), 0);  // VMEM reads
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int D, bool STATS>
__global__ __launch_bounds__((64 * dense_waves<D>())) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_dense_ring_kernel(AttnArgs a) {
  using L = LT<D>;
  constexpr int NS = kDenseStages, W = dense_waves<D>();
  constexpr int NC = L::NI / W;
  // the epilogue stages SROWS query rows per wave in the ring
  constexpr int SROWS = W == 8 ? 16 : 32;
  static_assert(NC >= 1 && NC * W == L::NI, "copies per wave");
  static_assert(NS * L::STAGE >= W * SROWS * L::OPITCH, "epilogue staging fits the ring");
  __shared__ __attribute__((aligned(16))) char ring[NS][L::STAGE];
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int bph = (a.G + W - 1) / W;  // blocks per head
  const int blk = xcd_remap(blockIdx.x, a.H * bph, a.xcd_chunk);
  if (blk < 0) return;  // the whole block
  const int h = blk / bph;
  const int g = (blk - h * bph) * W + wid;
  const bool active = g < a.G;
  const int gc = active ? g : a.G - 1;  // a wave past the last group computes that group and stores nothing
  const auto rq = make_rsrc((const char*)a.q + (size_t)h * a.N * L::ROWB, (uint32_t)((size_t)a.N * L::ROWB));
  LCtx<D> x;
  lctx_init<D, false>(x, a, h, gc, lane);
  int tokq[2];
  bool qvalid[2];
  u32x4 q[2][L::KCH];
  lqueries<D>(tokq, qvalid, q, a, rq, h, gc, lane);
  if (!active) qvalid[0] = qvalid[1] = false;
  // zero the ring before any copy lands (see lzero)
  for (int o = (wid * 64 + lane) * 16; o < NS * L::STAGE; o += 64 * W * 16)
    *(LDSP u32x4*)((LDSP char*)&ring[0][0] + o) = u32x4{0, 0, 0, 0};
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  block_barrier();
  LState<D, true> st;
  lstate_init<D, true>(st);
  const int nsteps = (x.nkeys + 31) >> 5;
  LDSP char* ring0 = (LDSP char*)&ring[0][0];
  for (int j = 0; j < NS - 1; ++j) ring_copy<D, NS>(ring0, x.rk, x.rv, j, x.ebase, x.goff, wid);
  // Iteration i: this wave's copies of step i landed (those of the NS - 2 later
  // steps may still be in flight), then the barrier: everyone's have, and
  // everyone is done with step i-1, whose stage takes step i+NS-1 (copied inside
  // step i, after its V reads).  Copies run past the last step (rows past N read
  // as zeros), so the count in flight is fixed.
#define MCS_RING_BEGIN()                                                     \
  __builtin_amdgcn_sched_barrier(0);                                         \
  wait_vm<(NS - 2) * 2 * NC>();                                              \
  block_barrier();                                                           \
  __builtin_amdgcn_sched_barrier(0);
  if (nsteps == 1) {
    MCS_RING_BEGIN()
    rstep<D, STATS, true, true, NS>(st, x, q, ring0, 0, ring0, wid);
  } else {
    MCS_RING_BEGIN()
    rstep<D, STATS, true, false, NS>(st, x, q, ring0, 0, ring0, wid);
    int it = 1;
#pragma unroll 1
    for (; it + 1 < nsteps; ++it) {
      MCS_RING_BEGIN()
      rstep<D, STATS, false, false, NS>(st, x, q, ring0 + (it % NS) * L::STAGE, it, ring0, wid);
    }
    MCS_RING_BEGIN()
    rstep<D, STATS, false, true, NS>(st, x, q, ring0 + (it % NS) * L::STAGE, it, ring0, wid);
  }
#undef MCS_RING_BEGIN
  wait_vm<0>();
  block_barrier();  // every wave is done with the ring before it holds the epilogue's rows
  if (!active) return;
  lend<D, false, EPI_PLAIN, true, STATS, SROWS>(st, x, a, rq, h, tokq, qvalid, lane,
                                               ring0 + wid * SROWS * L::OPITCH);
}

// ---------------------------------------------------------------------------
// Row statistics over all keys (selection pass 1) with the dense ring: eight waves
// of a block take eight consecutive 64-query groups of one head and share each K
// tile (no V tile, no output).  Without O a wave needs about 128 registers, so
// two blocks share a CU at four waves per SIMD, and each wave issues one copy
// instruction per step.  Per query the arithmetic is that of attn_lds_kernel
// without the PV product, in the same order.
constexpr int kLseWaves = 8;

// Copy instruction `wid` of the K tile of step j (waves past the tile's
// instructions copy nothing).  The body exists only in the device pass: the host
// pass of this file rejects this instantiation of tile_copy_dense (its parameter
// substitution fails there), though the device code is the same as ring_copy's.
template <int D, int NS>
__device__ __forceinline__ void lse_ring_copy(LDSP char* ring0, __amdgpu_buffer_rsrc_t rk, int j, int ebase,
                                              uint32_t goff, int wid) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NC = LT<D>::NI >= kLseWaves ? LT<D>::NI / kLseWaves : 1;
  LDSP char* stg = ring0 + (j % NS) * LT<D>::TILE;
  if (wid * NC < LT<D>::NI) tile_copy_dense<D, NC>(stg, rk, j, ebase, goff, wid * NC);
#endif
}

// One step: the barrier, the copies of step it + NS - 1 into the stage read in the
// step before, QK with the K chunks read ahead of the MFMAs, the probabilities.
template <int D, bool FIRST, bool LAST, int NS>
__device__ __forceinline__ void lse_ring_step(LState<D, false>& st, const LCtx<D>& x,
                                              const u32x4 (&q)[2][LT<D>::KCH], LDSP char* ring0, int it, int wid) {
  using L = LT<D>;
  constexpr int NC = L::NI >= kLseWaves ? L::NI / kLseWaves : 1;
  constexpr int KCH = L::KCH, KA = kDenseKAhead;
  __builtin_amdgcn_sched_barrier(0);
  // this wave's copies of step it landed once at most those of the NS - 2 later steps remain
  wait_vm<(NS - 2) * NC>();
  block_barrier();
  lse_ring_copy<D, NS>(ring0, x.rk, it + NS - 1, x.ebase, x.goff, wid);
  __builtin_amdgcn_sched_barrier(0);
  const LDSP char* cur = ring0 + (it % NS) * L::TILE;
  f32x16 s[2] = {f32x16{}, f32x16{}};
  u32x4 ka[KCH];
#pragma unroll
  for (int ks = 0; ks < KA; ++ks) ka[ks] = *(const LDSP u32x4*)(cur + x.kaddr[ks & 1] + 64 * (ks >> 1));
  __builtin_amdgcn_sched_group_barrier(0x100, KA, 0);
#pragma unroll
  for (int ks = 0; ks < KCH; ++ks) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) s[nt] = mfma_bf16(as_bf16x8(ka[ks]), as_bf16x8(q[nt][ks]), s[nt]);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    if (ks + KA < KCH) {
      ka[ks + KA] = *(const LDSP u32x4*)(cur + x.kaddr[(ks + KA) & 1] + 64 * ((ks + KA) >> 1));
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (LAST) lmask(s, it * 32, x.nkeys, x.hf);
  if constexpr (FIRST) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float mx = s[nt][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[nt][r]);
      st.m[nt] = pair_max(mx) * x.c + kMargin;
    }
  }
  uint32_t pk[2][8];
  lprobs<D, false, false>(st, s, pk, x.c);
}

template <int D>
__global__ __launch_bounds__(64 * kLseWaves) __attribute__((amdgpu_waves_per_eu(4, 4)))
void attn_lse_ring_kernel(AttnArgs a) {
  using L = LT<D>;
  constexpr int NS = kDenseStages, W = kLseWaves;
  __shared__ __attribute__((aligned(16))) char ring[NS][L::TILE];
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int bph = (a.G + W - 1) / W;  // blocks per head
  const int blk = xcd_remap(blockIdx.x, a.H * bph, a.xcd_chunk);
  if (blk < 0) return;  // the whole block
  const int h = blk / bph;
  const int g = (blk - h * bph) * W + wid;
  const bool active = g < a.G;
  const int gc = active ? g : a.G - 1;  // a wave past the last group computes that group and stores nothing
  const auto rq = make_rsrc((const char*)a.q + (size_t)h * a.N * L::ROWB, (uint32_t)((size_t)a.N * L::ROWB));
  LCtx<D> x;
  lctx_init<D, false>(x, a, h, gc, lane);
  int tokq[2];
  bool qvalid[2];
  u32x4 q[2][L::KCH];
  lqueries<D>(tokq, qvalid, q, a, rq, h, gc, lane);
  if (!active) qvalid[0] = qvalid[1] = false;
  LDSP char* ring0 = (LDSP char*)&ring[0][0];
  // zero the ring before any copy lands (see lzero)
  for (int o = (wid * 64 + lane) * 16; o < NS * L::TILE; o += 64 * W * 16)
    *(LDSP u32x4*)(ring0 + o) = u32x4{0, 0, 0, 0};
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  block_barrier();
  LState<D, false> st;
  lstate_init<D, false>(st);
  const int nsteps = (x.nkeys + 31) >> 5;
  for (int j = 0; j < NS - 1; ++j) lse_ring_copy<D, NS>(ring0, x.rk, j, x.ebase, x.goff, wid);
  // copies run past the last step (rows past N read as zeros), so the count in
  // flight is fixed
  if (nsteps == 1) {
    lse_ring_step<D, true, true, NS>(st, x, q, ring0, 0, wid);
  } else {
    lse_ring_step<D, true, false, NS>(st, x, q, ring0, 0, wid);
    int it = 1;
#pragma unroll 1
    for (; it + 1 < nsteps; ++it) lse_ring_step<D, false, false, NS>(st, x, q, ring0, it, wid);
    lse_ring_step<D, false, true, NS>(st, x, q, ring0, it, wid);
  }
  wait_vm<0>();  // the copies past the last step land before the block's LDS is released
  if (!active) return;
  lend<D, false, EPI_PLAIN, false, false>(st, x, a, rq, h, tokq, qvalid, lane, ring0);
}

template <int D>
hipError_t launch_lse_ring(const AttnArgs& a, hipStream_t s) {
  const int blocks = xcd_grid(a.H * ((a.G + kLseWaves - 1) / kLseWaves));
  hipLaunchKernelGGL((attn_lse_ring_kernel<D>), dim3(blocks), dim3(64 * kLseWaves), 0, s, a);
  return hipGetLastError();
}

template <int D, bool STATS>
hipError_t launch_dense_ring(const AttnArgs& a, hipStream_t s) {
  constexpr int W = dense_waves<D>();
  const int blocks = xcd_grid(a.H * ((a.G + W - 1) / W));
  hipLaunchKernelGGL((attn_dense_ring_kernel<D, STATS>), dim3(blocks), dim3(64 * W), 0, s, a);
  return hipGetLastError();
}

template <int D, bool GATHER, int EPI, bool PV, bool STATS = false>
hipError_t launch_lds(const AttnArgs& a, hipStream_t s) {
  const int items = a.H * a.G;
  const int blocks = xcd_grid((items + 3) / 4);
  hipLaunchKernelGGL((attn_lds_kernel<D, GATHER, EPI, PV, STATS>), dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D, int EPI>
hipError_t launch_pairs_d(const AttnArgs& a, const int32_t* ncommon, hipStream_t s) {
  const int blocks = xcd_grid(a.H * ((a.G + 1) / 2));
  hipLaunchKernelGGL((attn_pairs_kernel<D, EPI>), dim3(blocks), dim3(128), 0, s, a, ncommon);
  return hipGetLastError();
}

template <int D>
hipError_t launch_pairs_e(const AttnArgs& a, const int32_t* ncommon, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_ADD: return launch_pairs_d<D, EPI_ADD>(a, ncommon, s);
    case EPI_RESID: return launch_pairs_d<D, EPI_RESID>(a, ncommon, s);
    default: return launch_pairs_d<D, EPI_PLAIN>(a, ncommon, s);
  }
}

template <typename T, int D, bool GATHER, int EPI, bool PV>
hipError_t launch_t(const AttnArgs& a, hipStream_t s) {
  const int items = a.H * a.G;
  const int blocks = xcd_grid((items + 3) / 4);
  hipLaunchKernelGGL((attn_kernel<T, D, GATHER, EPI, PV>), dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const AttnArgs& a, bool gather, int epi, bool pv, hipStream_t s) {
  if constexpr (std::is_same<T, __bf16>::value) {
    if (!pv) return gather ? launch_lds<D, true, EPI_PLAIN, false>(a, s) : launch_lse_ring<D>(a, s);
    if (gather) {
      switch (epi) {
        case EPI_ADD: return launch_lds<D, true, EPI_ADD, true>(a, s);
        case EPI_RESID: return launch_lds<D, true, EPI_RESID, true>(a, s);
        default: return launch_lds<D, true, EPI_PLAIN, true>(a, s);
      }
    }
    // dense: the exact row sums are kept only when statistics are written
    return (a.stats || a.lse) ? launch_dense_ring<D, true>(a, s) : launch_dense_ring<D, false>(a, s);
  } else {
    if (!pv) return gather ? launch_t<T, D, true, EPI_PLAIN, false>(a, s) : launch_t<T, D, false, EPI_PLAIN, false>(a, s);
    if (gather) {
      switch (epi) {
        case EPI_ADD: return launch_t<T, D, true, EPI_ADD, true>(a, s);
        case EPI_RESID: return launch_t<T, D, true, EPI_RESID, true>(a, s);
        default: return launch_t<T, D, true, EPI_PLAIN, true>(a, s);
      }
    }
    return launch_t<T, D, false, EPI_PLAIN, true>(a, s);
  }
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int dtype, int head_dim, bool gather, int epi, bool pv,
                            hipStream_t s) {
  if (dtype == DT_BF16) {
    return head_dim == 128 ? launch_d<__bf16, 128>(a, gather, epi, pv, s) : launch_d<__bf16, 64>(a, gather, epi, pv, s);
  }
  return head_dim == 128 ? launch_d<float, 128>(a, gather, epi, pv, s) : launch_d<float, 64>(a, gather, epi, pv, s);
}

hipError_t launch_attention_pairs(const AttnArgs& a, const int32_t* ncommon, int head_dim, int epi,
                                  hipStream_t s) {
  return head_dim == 128 ? launch_pairs_e<128>(a, ncommon, epi, s) : launch_pairs_e<64>(a, ncommon, epi, s);
}

}  // namespace mcs
