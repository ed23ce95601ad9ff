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
  float l[2];   // running sum of exp2(s*c - m)
};

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
template <typename T, int D, bool PV, bool EXACT_SUM>
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
    if constexpr (EXACT_SUM || TL::F32) {
      float ls = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) ls += s[nt][r];
      st.l[nt] += ls;
    } else {
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
      float ls = st.l[nt];
#pragma unroll
      for (int i = 0; i < 8; ++i) ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[nt][i]), one, ls, false);
      st.l[nt] = ls;
    }
  }
}

// Masking of entries past the key count and the online softmax update; leaves
// the step's probabilities exp2(s*c - m) in s.
template <typename T, int D, bool PV, bool EXACT_SUM, bool MASK>
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
    if constexpr (EXACT_SUM || TL::F32) {
      // fp32 row sums: the row statistics / logsumexp are consumed by selection
      float ls = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) ls += s[nt][r];
      st.l[nt] += ls;
    } else {
      // sum of the bf16-rounded probabilities that the PV product uses, so the
      // normalisation matches the numerator (v_dot2_f32_bf16 against ones)
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
      float ls = st.l[nt];
#pragma unroll
      for (int i = 0; i < 8; ++i) ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[nt][i]), one, ls, false);
      st.l[nt] = ls;
    }
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
  constexpr bool EXACT = !GATHER;
  load_idx<GATHER>(ilater, x.ridx, (it + 2) * 32, x.lm, x.hf);
  f32x16 s[2];
  uint32_t pk[2][8];
  __builtin_amdgcn_sched_barrier(0);
  qk<T, D>(s, b, q);
  load_k<T, D>(b, inext, x.rk, x.hf);
  // keep the gathers where they are: sinking them toward the end of the step
  // (which the scheduler does to shorten live ranges) exposes their latency
  __builtin_amdgcn_sched_barrier(0);
  probs<T, D, PV, EXACT>(st, s, pk, x.c);
  if constexpr (PV) {
    pv<T, D, PV>(st, s, pk, b);
    load_v<T, D>(b, inext, x.rv, x.lm);
  }
}

template <typename T, int D, bool GATHER, bool PV>
__device__ __forceinline__ void pass_fixed(State<T, D, PV>& st, const Ctx<T, D, GATHER>& x,
                                           const u32x4 (&q)[2][Tile<T, D>::KCH]) {
  constexpr bool EXACT = !GATHER;
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
    probs<T, D, PV, EXACT>(st, s, pk, x.c);
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
    probs<T, D, PV, EXACT>(st, s, pk, x.c);
    if constexpr (PV) pv<T, D, PV>(st, s, pk, b);
  }
}

// Online pass with a running maximum and lazy rescaling (the offset moves only
// when the maximum grows by more than 2^8).  Used only for groups whose
// fixed-offset pass overflowed.
template <typename T, int D, bool GATHER, bool PV>
__device__ __attribute__((noinline)) void pass_online(State<T, D, PV>& st, const Ctx<T, D, GATHER>& x,
                                                      const u32x4 (&q)[2][Tile<T, D>::KCH]) {
  constexpr bool EXACT = !GATHER;
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
      softmax<T, D, PV, EXACT, true>(st, s, pk, it * 32, x.nkeys, x.c, x.hf);
    else
      softmax<T, D, PV, EXACT, false>(st, s, pk, it * 32, x.nkeys, x.c, x.hf);
    if constexpr (PV) pv<T, D, PV>(st, s, pk, b);
  }
}

template <typename T, int D, bool PV>
__device__ __forceinline__ void state_init(State<T, D, PV>& st) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    st.m[nt] = -INFINITY;
    st.l[nt] = 0.0f;
    if constexpr (PV) {
#pragma unroll
      for (int cc = 0; cc < Tile<T, D>::VEC; ++cc) st.o[nt][cc] = f32x16{};
    }
  }
}

// Row statistics, normalisation and the epilogue stores of one group.
template <typename T, int D, int EPI, bool PV>
__device__ __forceinline__ void finish(const State<T, D, PV>& st, const AttnArgs& a, int h, int g, const int (&tokq)[2],
                                       const bool (&qvalid)[2], int lm, int hf) {
  using TL = Tile<T, D>;
  const int N = a.N;
  float inv[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float lt = pair_sum(st.l[nt]);
    inv[nt] = 1.0f / lt;
    if (hf == 0 && qvalid[nt]) {
      const size_t ri = (size_t)h * N + tokq[nt];
      if (a.stats) a.stats[ri] = make_float2(st.m[nt], inv[nt]);
      if (a.lse) a.lse[ri] = (st.m[nt] + __log2f(lt)) * kLn2;
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
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const uint32_t qb = (uint32_t)tokq[nt] * TL::ROWB + TL::khalf_off(hf);
#pragma unroll
    for (int c = 0; c < TL::KCH; ++c) q[nt][c] = bload128(rq, qb + c * TL::KSTRIDE);
  }

  State<T, D, PV> st;
  state_init<T, D, PV>(st);
  pass_fixed<T, D, GATHER, PV>(st, x, q);
  const bool ok = __builtin_isfinite(st.l[0]) && __builtin_isfinite(st.l[1]);
  if (__builtin_amdgcn_ballot_w64(!ok)) {
    State<T, D, PV> so;
    state_init<T, D, PV>(so);
    pass_online<T, D, GATHER, PV>(so, x, q);
    finish<T, D, EPI, PV>(so, a, h, g, tokq, qvalid, lm, hf);
  } else {
    finish<T, D, EPI, PV>(st, a, h, g, tokq, qvalid, lm, hf);
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

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int dtype, int head_dim, bool gather, int epi, bool pv,
                            hipStream_t s) {
  if (dtype == DT_BF16) {
    return head_dim == 128 ? launch_d<__bf16, 128>(a, gather, epi, pv, s) : launch_d<__bf16, 64>(a, gather, epi, pv, s);
  }
  return head_dim == 128 ? launch_d<float, 128>(a, gather, epi, pv, s) : launch_d<float, 64>(a, gather, epi, pv, s);
}

}  // namespace mcs
