// Two-pass exact top-K selection of the MC-Sparse hot path for gfx950
// (MC-Sparse summary page, selection paragraph: per query group, keep the K keys
// with the largest summed attention weight; flash attention hides the logits, so
// a second QK pass recomputes them).
//
// Pass 1 (row statistics) is the PV-less variant of the attention kernel.
// Pass 2 (this file): one wavefront per query group recomputes S = Q_g K^T for
// all keys, 32 at a time (v_mfma_f32_32x32x16_bf16 with the group's queries as
// the A operand, so each lane owns one key column), normalises each logit with
// its row statistics and sums the 64 probabilities per key: mass[g][j].
// While the row is produced, a 2048-bin histogram of its values (exponent and
// top mantissa bits over a window of binades, see hist_bin) is built in LDS and
// stored beside the row when the loop ends.
// Top-K (a second kernel, four waves per SIMD so that the row reads overlap):
// one wavefront per row finds the bin of the K-th largest mass from the stored
// histogram, then reads the row once.  Every entry above that bin, and every
// entry in it (a candidate, flagged), goes to a provisional ascending list that
// overwrites the row's head, while the candidates' values go to LDS.  The exact
// threshold is resolved among the candidates, and a pass over the provisional
// list (about K entries, not N) writes the kept key ids in ascending order, ties
// at the threshold going to the lowest ids.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "ldstile.hpp"

namespace mcs {

namespace {

template <typename T, int D>
struct QTile {
  static constexpr bool F32 = std::is_same<T, float>::value;
  static constexpr int ROWB = D * (int)sizeof(T);
  static constexpr int KCH = ROWB / 2 / 16;
  static constexpr int KSTRIDE = F32 ? 16 : 32;
  static constexpr int QK_STEPS = F32 ? D / 2 : D / 16;
  __device__ static uint32_t khalf_off(int hf) { return F32 ? (uint32_t)(D / 2 * 4 * hf) : (uint32_t)(16 * hf); }
};

// The loop's histogram of a row's masses (non-negative floats, whose bit
// patterns order like their values): bin = exponent and top six mantissa bits
// (bits 30..17, 1/64 of a binade) over the 32 binades [2^-27, 2^5), values
// outside that window counted in the end bins.  A row's masses around its K-th
// largest span a binade or two, so the threshold's bin holds a few hundred
// entries, which the top-K resolves among themselves after a single read of the
// row; coarser bins (the top 11 bits) held thousands and cost a second read
// nearly every time.  A threshold in an end bin is refined from the top bits.
constexpr int kHistBins = kMassHistBins;
constexpr int kHistKeyShift = 17;              // a 15-bit key: bits 31..17 (bit 31 clear)
constexpr int kHistKeyBase = (127 - 27) << 6;  // key of 2^-27: bin 0
constexpr int kHistPerLane = kHistBins / 64;
static_assert(kHistBins == 32 * 64, "32 binades of 64 bins");
__device__ __forceinline__ uint32_t hist_bin(float mass) {
  const int key = (int)(__float_as_uint(mass) >> kHistKeyShift) - kHistKeyBase;
  return (uint32_t)min(max(key, 0), kHistBins - 1);
}
// Per-wave shared memory of the top-K: a 256-bin histogram for refining the
// threshold, and the values of the candidates (entries of the threshold's bin),
// in ascending key order.
constexpr int kCandCap = 2048;
struct WaveTopk {
  uint32_t hist[256];
  uint32_t cand_bits[kCandCap];
};

// LDS atomic add issued through inline asm.  The compiler cannot tell LDS that a
// pending buffer_load ... lds copy writes from any other LDS, so before an
// ordinary LDS atomic it waits for every such copy in flight; in the selection
// loop that wait drained the whole K pipeline at every step.  The asm add is not
// seen by that analysis.  LDS operations of a wave complete in order, so the
// compiler's own lgkmcnt waits stay sufficient, and the histogram is read only
// after an explicit s_waitcnt lgkmcnt(0).
__device__ __forceinline__ void lds_add_u32(uint32_t* p, uint32_t v) {
  const uint32_t addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint32_t*)p;
  asm volatile("ds_add_u32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}

// Ranks of this lane's flagged entries among the flagged entries of a 64 x 4
// block ordered lane-major, then by j: rank[j] = flagged entries before (lane, j).
// Returns the block's total.  Ballots and mbcnt, no cross-lane shuffles: the
// shuffle-based scans these replace were latency bound (one wave per SIMD).
__device__ __forceinline__ uint32_t flag_ranks(const bool (&f)[4], uint32_t (&rank)[4]) {
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint64_t m = __builtin_amdgcn_ballot_w64(f[j]);
    before = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, before));
    total += (uint32_t)__builtin_popcountll(m);
  }
  uint32_t within = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    rank[j] = before + within;
    within += f[j] ? 1u : 0u;
  }
  return total;
}

// Digit (from the top) holding the kr-th largest entry of a wave-private histogram
// of `bins` bins (a multiple of 64); returns the digit, leaves in kr the rank
// inside it and in cnt its population.  Lane l owns bins [l*bins/64, (l+1)*bins/64).
__device__ uint32_t pick_digit(const uint32_t* hist, int bins, uint32_t& kr, uint32_t& cnt) {
  const int lane = threadIdx.x & 63;
  const int per = bins / 64;
  uint32_t t = 0;
  for (int j = 0; j < per; ++j) t += hist[lane * per + j];
  uint32_t above = 0;
  int L = 0;
  for (int l = 63; l >= 0; --l) {
    const uint32_t tl = (uint32_t)__builtin_amdgcn_readlane((int)t, l);
    if (above + tl >= kr || l == 0) {
      L = l;
      break;
    }
    above += tl;
  }
  int d = L * per;
  cnt = 0;
  for (int j = per - 1; j >= 0; --j) {
    const uint32_t c = hist[L * per + j];
    if (above + c >= kr || j == 0) {
      d = L * per + j;
      cnt = c;
      break;
    }
    above += c;
  }
  kr -= above;
  return (uint32_t)d;
}

constexpr int kMassStages = 4;  // K tiles in flight in the bf16 pass-2 loop
constexpr int kUnroll = 4;
constexpr int kBatch = 256 * kUnroll;

// Entries [base, base + kBatch) of a row: lane l gets entries base + 256*u + 4*l + j.
// Entries past N read as 0 (they are masked by the callers).
__device__ __forceinline__ void load_batch(const uint32_t* rb, int N, int base, uint32_t (&b)[kUnroll][4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int i0 = base + 256 * u + 4 * lane;
    if (i0 + 3 < N) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(rb + i0);
      b[u][0] = v[0]; b[u][1] = v[1]; b[u][2] = v[2]; b[u][3] = v[3];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) b[u][j] = i0 + j < N ? rb[i0 + j] : 0u;
    }
  }
}

// Visit a row in batches of kBatch entries, the loads of batch n+1 in flight
// while batch n is processed.  f(base, b) sees entries base + 256*u + 4*lane + j.
// (Latency is hidden mostly by the other waves of the SIMD: the top-K kernel
// runs four per SIMD.)
template <typename F>
__device__ __forceinline__ void scan_row(const uint32_t* rb, int N, F&& f) {
  uint32_t ba[kUnroll][4], bb[kUnroll][4];
  load_batch(rb, N, 0, ba);
  int base = 0;
  for (; base + kBatch < N; base += 2 * kBatch) {
    load_batch(rb, N, base + kBatch, bb);
    f(base, ba);
    if (base + 2 * kBatch < N) load_batch(rb, N, base + 2 * kBatch, ba);
    f(base + kBatch, bb);
  }
  if (base < N) f(base, ba);
}

// Bin (from the top) of a stored histogram that holds the kr-th largest entry
// (1-based); leaves in kr the rank inside that bin and in cnt its population.
// Lane l sums its kHistPerLane consecutive bins; suffix sums over the lanes find
// the lane, then over that lane's bins the bin.
__device__ uint32_t pick_top_bin(const uint32_t* gh, uint32_t& kr, uint32_t& cnt) {
  const int lane = threadIdx.x & 63;
  auto suffix = [&](uint32_t x) {  // inclusive: sum over lanes >= this one
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = (uint32_t)__shfl_down((int)x, o, 64);
      if (lane + o < 64) x += y;
    }
    return x;
  };
  const u32x4* p = reinterpret_cast<const u32x4*>(gh + kHistPerLane * lane);
  uint32_t t = 0;
#pragma unroll
  for (int i = 0; i < kHistPerLane / 4; ++i) {
    const u32x4 v = p[i];
    t += v[0] + v[1] + v[2] + v[3];
  }
  uint32_t inc = suffix(t);
  // exactly one lane has inc >= kr > inc - t (the histogram holds N >= K entries)
  uint64_t m = __builtin_amdgcn_ballot_w64(inc >= kr && inc - t < kr);
  const int L = m ? __builtin_ctzll(m) : 0;
  uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)(inc - t), L);
  const uint32_t c = lane < kHistPerLane ? gh[kHistPerLane * L + lane] : 0u;
  inc = suffix(c) + above;
  m = __builtin_amdgcn_ballot_w64(inc >= kr && inc - c < kr);
  const int j = m ? __builtin_ctzll(m) : 0;
  cnt = (uint32_t)__builtin_amdgcn_readlane((int)c, j);
  kr -= (uint32_t)__builtin_amdgcn_readlane((int)(inc - c), j);
  return (uint32_t)(kHistPerLane * L + j);
}

// Exact top-K of one mass row by one wavefront, ascending ids, ties to the lower
// id.  gh is the row's stored histogram.  The row's head is overwritten by the
// provisional list.
__device__ void wave_topk(float* row, const uint32_t* gh, int N, int K, int kpad, int32_t* out, WaveTopk* w) {
  const int lane = threadIdx.x & 63;
  uint32_t* rb = reinterpret_cast<uint32_t*>(row);
  uint32_t kr = (uint32_t)K, cnt = 0;
  const uint32_t bin = pick_top_bin(gh, kr, cnt);
  // The threshold's entries share the top bits of `prefix` under `pmask`; the
  // bits below `shift` are still open.
  uint32_t prefix, pmask;
  int shift;
  if (bin == 0 || bin == (uint32_t)kHistBins - 1) {
    // an end bin also counts the values outside the window: start from the top
    kr = (uint32_t)K;
    cnt = (uint32_t)N;
    prefix = 0;
    pmask = 0;
    shift = 32;
  } else {
    prefix = (bin + (uint32_t)kHistKeyBase) << kHistKeyShift;
    pmask = 0x7fffu << kHistKeyShift;
    shift = kHistKeyShift;
  }
  // Refine the prefix while too many entries share it, 8 bits per pass (a
  // threshold in an end bin, or a crowd of nearly equal masses).  The row is read
  // in the same batches as below.
  while (cnt > (uint32_t)kCandCap && shift > 0) {
    const int nshift = shift >= 8 ? shift - 8 : 0;
    const int bins = 1 << (shift - nshift);
    for (int j = lane; j < 256; j += 64) w->hist[j] = 0;
    __builtin_amdgcn_s_waitcnt(0);
    scan_row(rb, N, [&](int base, const uint32_t (&b)[kUnroll][4]) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = base + 256 * u + 4 * lane + j;
          if (i < N && (b[u][j] & pmask) == prefix)
            atomicAdd(&w->hist[(b[u][j] >> nshift) & (uint32_t)(bins - 1)], 1u);
        }
    });
    __builtin_amdgcn_s_waitcnt(0);
    const uint32_t d = pick_digit(w->hist, 256, kr, cnt);
    prefix |= d << nshift;
    pmask |= (uint32_t)(bins - 1) << nshift;
    shift = nshift;
  }
  // One pass over the row: entries whose masked bits exceed the prefix are kept
  // for sure, entries equal to it are candidates.  Both go, in id order, to the
  // provisional list at the row's head (id, bit 31 set for a candidate); the
  // candidates' values go to LDS.  The list position of an entry never exceeds
  // its own index, and the batch read ahead lies past the current one, so no
  // store lands on an entry not yet read.
  uint32_t nsel = 0, nc = 0;
  scan_row(rb, N, [&](int base, const uint32_t (&b)[kUnroll][4]) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i0 = base + 256 * u + 4 * lane;
      bool sel[4], cand[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t mb = b[u][j] & pmask;
        sel[j] = i0 + j < N && mb >= prefix;
        cand[j] = i0 + j < N && mb == prefix;
      }
      uint32_t rs[4], rc[4];
      const uint32_t ts = flag_ranks(sel, rs);
      const uint32_t tc = flag_ranks(cand, rc);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (sel[j]) rb[nsel + rs[j]] = (uint32_t)(i0 + j) | (cand[j] ? 0x80000000u : 0u);
        if (cand[j] && nc + rc[j] < (uint32_t)kCandCap) w->cand_bits[nc + rc[j]] = b[u][j];
      }
      nsel += ts;
      nc += tc;
    }
  });
  if (nc > (uint32_t)kCandCap) nc = kCandCap;  // the refinement above keeps nc within the cap
  // The list's stores have landed in L2, and this CU's L1 (which holds the row
  // lines just read) is invalidated, before the list is read back.
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  // Resolve the remaining low bits among the candidates, 8 at a time.
  while (shift > 0) {
    const int nshift = shift >= 8 ? shift - 8 : 0;
    const int bins = 1 << (shift - nshift);
    for (int j = lane; j < 256; j += 64) w->hist[j] = 0;
    __builtin_amdgcn_s_waitcnt(0);
    for (uint32_t c = lane; c < nc; c += 64) {
      const uint32_t b = w->cand_bits[c];
      if ((b & pmask) == prefix) atomicAdd(&w->hist[(b >> nshift) & (uint32_t)(bins - 1)], 1u);
    }
    __builtin_amdgcn_s_waitcnt(0);
    const uint32_t d = pick_digit(w->hist, 256, kr, cnt);
    prefix |= d << nshift;
    pmask |= (uint32_t)(bins - 1) << nshift;
    shift = nshift;
  }
  const uint32_t tau = prefix;  // the K-th largest bit pattern; keep kr of its ties
  // Ascending compaction of the provisional list: sure entries are kept; a
  // candidate (the c-th, in id order) is kept if its value exceeds tau, or equals
  // it and is among the first kr such.  The kept ids go out through a buffer
  // descriptor covering exactly K entries, one store instruction per (u, j)
  // whatever is kept (the rest aim past the range and are dropped).
  const auto rout = make_rsrc(out, (uint32_t)K * 4u);
  uint32_t written = 0, eq_seen = 0, cand_seen = 0;
  scan_row(rb, (int)nsel, [&](int base, const uint32_t (&bb)[kUnroll][4]) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i0 = base + 256 * u + 4 * lane;
      bool isc[4], eq[4], keep[4];
      uint32_t cb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) isc[j] = i0 + j < (int)nsel && (bb[u][j] >> 31) != 0;
      uint32_t crank[4];
      const uint32_t ctot = flag_ranks(isc, crank);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // a candidate past the LDS cap exists only when the refinement ran down
        // to the last bit (more than kCandCap entries share one value): it equals tau
        const uint32_t ci = cand_seen + crank[j];
        cb[j] = isc[j] ? (ci < nc ? w->cand_bits[ci] : tau) : 0u;
        eq[j] = isc[j] && cb[j] == tau;
      }
      uint32_t eq_rank[4];
      const uint32_t eq_tot = flag_ranks(eq, eq_rank);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        keep[j] = i0 + j < (int)nsel && (!isc[j] || cb[j] > tau || (eq[j] && eq_seen + eq_rank[j] < kr));
      uint32_t rank[4];
      const uint32_t sel_tot = flag_ranks(keep, rank);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t off = keep[j] ? (written + rank[j]) * 4u : 0xfffffff0u;  // exactly K are kept overall
        asm volatile("" : "+v"(off));  // opaque: keeps the store out of a branch on keep[j]
        __builtin_amdgcn_raw_buffer_store_b32(bb[u][j] & 0x7fffffffu, rout, off, 0, 0);
      }
      written += sel_tot;
      eq_seen += eq_tot;
      cand_seen += ctot;
    }
  });
  for (int j = K + lane; j < kpad; j += 64) out[j] = -1;
}

// Top-K of rows [0, hcount*G) of a pass: one wavefront per row, four per SIMD.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void topk_rows_kernel(MassArgs a) {
  __shared__ WaveTopk s_w[4];
  const int wid = wave_id();
  const int item = blockIdx.x * 4 + wid;
  if (item >= a.hcount * a.G) return;  // no block-level synchronisation below
  const int hl = item / a.G, g = item - hl * a.G;
  wave_topk(a.mass + (size_t)item * a.ldm, a.hist + (size_t)item * kHistBins, a.N, a.K, a.kpad,
            a.idx + ((size_t)(a.h0 + hl) * a.G + g) * a.kpad, &s_w[wid]);
}

// Store a wave's LDS histogram to its row's slot: 16 consecutive bytes per lane.
__device__ __forceinline__ void store_hist(const uint32_t* hist, uint32_t* gh) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < kHistBins / 256; ++i) {
    const int e = 4 * (64 * i + lane);
    *reinterpret_cast<u32x4*>(gh + e) = *reinterpret_cast<const u32x4*>(hist + e);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void group_mass_kernel(MassArgs a) {
  using TL = QTile<T, D>;
  __shared__ uint32_t s_hist[4][kHistBins];
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int hf = lane >> 5, lm = lane & 31;
  const int items = a.hcount * a.G;
  const int blk = xcd_remap(blockIdx.x, (items + 3) >> 2, a.xcd_chunk);
  if (blk < 0) return;
  const int item = blk * 4 + wid;
  if (item >= items) return;  // no block-level synchronisation below
  uint32_t* hist = s_hist[wid];
  const int hl = item / a.G, g = item - hl * a.G;
  const int h = a.h0 + hl;
  const int N = a.N;
  const size_t head_off = (size_t)h * N * TL::ROWB;
  const uint32_t head_bytes = (uint32_t)((size_t)N * TL::ROWB);
  const auto rq = make_rsrc((const char*)a.q + head_off, head_bytes);
  const auto rk = make_rsrc((const char*)a.k + head_off, head_bytes);
  for (int j = lane; j < kHistBins; j += 64) hist[j] = 0;

  // Query rows of this group: lane lm holds queries lm and lm + 32 (A operand).
  int tokq[2];
  bool qvalid[2];
  u32x4 q[2][TL::KCH];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int slot = g * 64 + lm + 32 * nt;
    qvalid[nt] = slot < N;
    tokq[nt] = qvalid[nt] ? a.perm[(size_t)h * N + slot] : 0;
    if (tokq[nt] < 0 || tokq[nt] >= N) {  // not a token: treat as padding
      qvalid[nt] = false;
      tokq[nt] = 0;
    }
    const uint32_t qb = (uint32_t)tokq[nt] * TL::ROWB + TL::khalf_off(hf);
#pragma unroll
    for (int c = 0; c < TL::KCH; ++c) q[nt][c] = bload128(rq, qb + c * TL::KSTRIDE);
  }
  // Row statistics of the 32 accumulator rows this lane sees:
  // p = exp2(s*c - m) * w, with (m, w) = (offset, 1/sum) from pass 1, or
  // (lse*log2(e), 1) from a caller-supplied natural-log logsumexp.
  float rm[2][16], rw[2][16];
  float my_m[2], my_w[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    if (!qvalid[nt]) {
      my_m[nt] = INFINITY;  // exp2(-inf) = 0: padding rows add nothing
      my_w[nt] = 0.0f;
    } else if (a.stats) {
      const float2 st = a.stats[(size_t)h * N + tokq[nt]];
      my_m[nt] = st.x;
      my_w[nt] = st.y;
    } else {
      my_m[nt] = a.lse[(size_t)h * N + tokq[nt]] * kLog2e;
      my_w[nt] = 1.0f;
    }
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int src = 8 * (r >> 2) + 4 * hf + (r & 3);
      rm[nt][r] = lane_read(my_m[nt], src);
      rw[nt][r] = lane_read(my_w[nt], src);
    }

  float* out = a.mass + ((size_t)hl * a.G + g) * (size_t)a.ldm;  // rows 16-byte aligned
  const float c = a.c;
  const int nsteps = (N + 31) >> 5;
  auto load_keys = [&](u32x4 (&kb)[TL::KCH], int t0) {
    // keys past N read as zeros (buffer range check); their mass is never stored
    const uint32_t base = (uint32_t)(t0 + lm) * TL::ROWB + TL::khalf_off(hf);
#pragma unroll
    for (int cc = 0; cc < TL::KCH; ++cc) kb[cc] = bload128(rk, base + cc * TL::KSTRIDE);
  };
  auto qk = [&](f32x16 (&s)[2], const u32x4 (&kb)[TL::KCH]) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      s[nt] = f32x16{};
      if constexpr (TL::F32) {
#pragma unroll
        for (int ks = 0; ks < TL::QK_STEPS; ++ks)
          s[nt] = mfma_f32(__uint_as_float(q[nt][ks >> 2][ks & 3]), __uint_as_float(kb[ks >> 2][ks & 3]), s[nt]);
      } else {
#pragma unroll
        for (int ks = 0; ks < TL::QK_STEPS; ++ks) s[nt] = mfma_bf16(as_bf16x8(q[nt][ks]), as_bf16x8(kb[ks]), s[nt]);
      }
    }
  };
  auto reduce_store = [&](const f32x16 (&s)[2], int t0) {
    float acc = 0.0f;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        acc = __builtin_fmaf(fast_exp2(__builtin_fmaf(s[nt][r], c, -rm[nt][r])), rw[nt][r], acc);
    acc = pair_sum(acc);
    if (hf == 0 && t0 + lm < N) {
      out[t0 + lm] = acc;
      atomicAdd(&hist[hist_bin(acc)], 1u);
    }
  };
  // Software pipeline: the MFMAs of step i+1 are issued before the exponentials
  // of step i, so the matrix core and the VALU overlap; the single K buffer is
  // refilled for step i+2 as soon as the step i+1 MFMAs have read it.
  u32x4 kb[TL::KCH];
  f32x16 sa[2], sb[2];
  load_keys(kb, 0);
  qk(sa, kb);
  load_keys(kb, 32);
  int it = 0;
  for (; it + 2 < nsteps; it += 2) {
    qk(sb, kb);
    load_keys(kb, (it + 2) * 32);
    reduce_store(sa, it * 32);
    qk(sa, kb);
    load_keys(kb, (it + 3) * 32);
    reduce_store(sb, (it + 1) * 32);
  }
  if (it + 1 < nsteps) {
    qk(sb, kb);
    reduce_store(sa, it * 32);
    reduce_store(sb, (it + 1) * 32);
  } else {
    reduce_store(sa, it * 32);
  }
  __builtin_amdgcn_s_waitcnt(0);  // the histogram's LDS atomics are done
  store_hist(hist, a.hist + (size_t)item * kHistBins);
}

// bf16 pass 2 with K staged through LDS.  Every group scans all keys in the
// same order, so the four waves of a block take four consecutive groups of one
// head and share each K tile: every wave issues a quarter of the tile's copies
// and one block barrier per step separates "copies landed / previous tile
// consumed" from the reads.  This cuts the address work of the K fetches by
// 16x (quad-contiguous copies, a quarter each) and the L2 traffic by 4x.
//
// A wave issues in order, so its own MFMAs and VALU do not overlap: two blocks
// per CU (two waves per SIMD, from blocks with no barrier between them) let one
// wave's exponentials run beside the other's MFMAs.  That caps a block at 64 KB
// of LDS: four 8 KiB stages, copied four steps ahead, after the four waves'
// 8 KiB histograms.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void group_mass_lds_kernel(MassArgs a) {
  using L = LT<D>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int hf = lane >> 5, lm = lane & 31;
  const int gb = (a.G + 3) >> 2;
  const int blk = xcd_remap(blockIdx.x, a.hcount * gb, a.xcd_chunk);
  if (blk < 0) return;  // the whole block
  const int hl = blk / gb;
  const int g = (blk - hl * gb) * 4 + wid;
  const bool active = g < a.G;  // a wave past the last group only helps copy
  uint32_t* hist = (uint32_t*)smem + wid * kHistBins;
  LDSP char* lbase = (LDSP char*)smem + 4 * kHistBins * sizeof(uint32_t);
  constexpr int NS = kMassStages;
  auto stage = [&](int j) -> LDSP char* { return lbase + j * L::TILE; };
  const int h = a.h0 + hl;
  const int N = a.N;
  const size_t head_off = (size_t)h * N * L::ROWB;
  const uint32_t head_bytes = (uint32_t)((size_t)N * L::ROWB);
  const auto rq = make_rsrc((const char*)a.q + head_off, head_bytes);
  const auto rk = make_rsrc((const char*)a.k + head_off, head_bytes);
  for (int j = lane; j < kHistBins; j += 64) hist[j] = 0;

  // Query rows of this group: lane lm holds queries lm and lm + 32 (A operand).
  int tokq[2];
  bool qvalid[2];
  u32x4 q[2][L::KCH];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int slot = g * 64 + lm + 32 * nt;
    qvalid[nt] = active && slot < N;
    tokq[nt] = qvalid[nt] ? a.perm[(size_t)h * N + slot] : 0;
    if (tokq[nt] < 0 || tokq[nt] >= N) {
      qvalid[nt] = false;
      tokq[nt] = 0;
    }
    const uint32_t qb = (uint32_t)tokq[nt] * L::ROWB + 16u * hf;
#pragma unroll
    for (int c = 0; c < L::KCH; ++c) q[nt][c] = bload128(rq, qb + c * 32);
  }
  float rm[2][16], rw[2][16];
  float my_m[2], my_w[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    if (!qvalid[nt]) {
      my_m[nt] = INFINITY;
      my_w[nt] = 0.0f;
    } else if (a.stats) {
      const float2 st = a.stats[(size_t)h * N + tokq[nt]];
      my_m[nt] = st.x;
      my_w[nt] = st.y;
    } else {
      my_m[nt] = a.lse[(size_t)h * N + tokq[nt]] * kLog2e;
      my_w[nt] = 1.0f;
    }
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int src = 8 * (r >> 2) + 4 * hf + (r & 3);
      rm[nt][r] = lane_read(my_m[nt], src);
      rw[nt][r] = lane_read(my_w[nt], src);
    }

  float* out = a.mass + ((size_t)hl * a.G + (active ? g : 0)) * (size_t)a.ldm;
  // Mass stores go through a buffer descriptor so that every wave issues exactly
  // one store instruction per step (lanes with nothing to store, and every lane
  // of a wave past the last group, aim past the range and are dropped): the
  // per-step wait below then knows that exactly one store follows the copies.
  const auto rout = make_rsrc(out, active ? (uint32_t)a.ldm * 4u : 0u);
  const float c = a.c;
  const int nsteps = (N + 31) >> 5;
  const uint32_t goff = tile_goff<D>(lane);
  const int ebase = tile_ebase<D>(lane);
  int kaddr[2];
  tile_kaddr<D>(kaddr, lm, hf);
  constexpr int NC = L::NI / 4;

  auto qk = [&](f32x16 (&s)[2], const LDSP char* tile) {
    u32x4 kb[L::KCH];
    tile_kread<D>(kb, tile, kaddr);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      s[nt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < L::KCH; ++ks) s[nt] = mfma_bf16(as_bf16x8(q[nt][ks]), as_bf16x8(kb[ks]), s[nt]);
    }
  };
  auto reduce_store = [&](const f32x16 (&s)[2], int t0) {
    float acc = 0.0f;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        acc = __builtin_fmaf(fast_exp2(__builtin_fmaf(s[nt][r], c, -rm[nt][r])), rw[nt][r], acc);
    acc = pair_sum(acc);
    const bool keep = active && hf == 0 && t0 + lm < N;
    uint32_t soff = keep ? (uint32_t)(t0 + lm) * 4u : 0xfffffff0u;
    asm volatile("" : "+v"(soff));  // opaque: keeps the store out of the branch on `keep`
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc), rout, soff, 0, 0);
    if (keep) lds_add_u32(&hist[hist_bin(acc)], 1u);
  };
  // Iteration i: barrier (every wave's copy of K(i+1) landed, every wave done
  // with K(i)'s stage), copy K(i+NS) into that stage, QK of step i+1, then the
  // exponentials of step i (they overlap the MFMAs).  K(j) lives in stage j % NS.
  // Copies run past the last step (those rows read as zeros and are never used),
  // so every iteration issues NC copies and one store, and the number of vector
  // memory operations issued after this wave's copy of K(i+1) is fixed: the
  // copies of the NS - 2 steps after it (from the prologue, or one iteration
  // each), plus one store per iteration since the prologue, at most NS - 1.
  auto iter = [&](f32x16 (&sc)[2], f32x16 (&sn)[2], int i) {
    __builtin_amdgcn_sched_barrier(0);
    if (i >= NS - 1)
      wait_vm<(NS - 2) * NC + NS - 1>();
    else
      wait_vm<(NS - 2) * NC>();  // fewer stores so far: wait a little longer
    block_barrier();
    tile_copy_dense<D, NC>(stage(i % NS), rk, i + NS, ebase, goff, wid * NC);
    __builtin_amdgcn_sched_barrier(0);
    qk(sn, stage((i + 1) % NS));
    reduce_store(sc, i * 32);
  };
  f32x16 sa[2], sb[2];
  for (int j = 0; j < NS; ++j) tile_copy_dense<D, NC>(stage(j), rk, j, ebase, goff, wid * NC);
  wait_vm<(NS - 1) * NC>();
  block_barrier();
  qk(sa, stage(0));
  int it = 0;
  for (; it + 2 < nsteps; it += 2) {
    iter(sa, sb, it);
    iter(sb, sa, it + 1);
  }
  if (it + 1 < nsteps) {
    iter(sa, sb, it);
    reduce_store(sb, (it + 1) * 32);
  } else {
    reduce_store(sa, it * 32);
  }
  // The copies past the last step land before the block's LDS is released.
  wait_vm<0>();
  if (!active) return;
  __builtin_amdgcn_s_waitcnt(0);  // the histogram's LDS atomics are done
  store_hist(hist, a.hist + ((size_t)hl * a.G + g) * kHistBins);
}

template <int D>
hipError_t launch_mass_lds(const MassArgs& a, hipStream_t s) {
  const int blocks = xcd_grid(a.hcount * ((a.G + 3) / 4));
  const size_t lds = 4 * kHistBins * sizeof(uint32_t) + kMassStages * LT<D>::TILE;
  hipError_t e = hipFuncSetAttribute((const void*)group_mass_lds_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((group_mass_lds_kernel<D>), dim3(blocks), dim3(256), lds, s, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_mass_t(const MassArgs& a, hipStream_t s) {
  const int items = a.hcount * a.G;
  const int blocks = xcd_grid((items + 3) / 4);
  hipLaunchKernelGGL((group_mass_kernel<T, D>), dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_group_mass(const MassArgs& a, int dtype, int head_dim, hipStream_t s) {
  if (dtype == DT_BF16) return head_dim == 128 ? launch_mass_lds<128>(a, s) : launch_mass_lds<64>(a, s);
  return head_dim == 128 ? launch_mass_t<float, 128>(a, s) : launch_mass_t<float, 64>(a, s);
}

hipError_t launch_topk(const MassArgs& a, hipStream_t s) {
  const int rows = a.hcount * a.G;
  hipLaunchKernelGGL(topk_rows_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mcs
