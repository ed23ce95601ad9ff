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
// Top-K: one workgroup per (head, group) row finds the K-th largest mass by an
// MSB-first radix select on the fp32 bit pattern (non-negative floats order like
// their bits), then writes the kept key ids in ascending order, ties at the
// threshold going to the lowest ids.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

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

template <typename T, int D>
__global__ __launch_bounds__(256) void group_mass_kernel(MassArgs a) {
  using TL = QTile<T, D>;
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int hf = lane >> 5, lm = lane & 31;
  const int items = a.hcount * a.G;
  const int blk = xcd_remap(blockIdx.x, (items + 3) >> 2, a.xcd_chunk);
  if (blk < 0) return;
  const int item = blk * 4 + wid;
  if (item >= items) return;  // no block-level synchronisation below
  const int hl = item / a.G, g = item - hl * a.G;
  const int h = a.h0 + hl;
  const int N = a.N;
  const size_t head_off = (size_t)h * N * TL::ROWB;
  const uint32_t head_bytes = (uint32_t)((size_t)N * TL::ROWB);
  const auto rq = make_rsrc((const char*)a.q + head_off, head_bytes);
  const auto rk = make_rsrc((const char*)a.k + head_off, head_bytes);

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

  float* out = a.mass + ((size_t)hl * a.G + g) * (size_t)N;
  const float c = a.c;
  const int nsteps = (N + 31) >> 5;
  u32x4 kb[TL::KCH];
  auto load_keys = [&](int t0) {
    const int key = t0 + lm < N ? t0 + lm : 0;
    const uint32_t base = (uint32_t)key * TL::ROWB + TL::khalf_off(hf);
#pragma unroll
    for (int cc = 0; cc < TL::KCH; ++cc) kb[cc] = bload128(rk, base + cc * TL::KSTRIDE);
  };
  load_keys(0);
  for (int it = 0; it < nsteps; ++it) {
    const int t0 = it * 32;
    f32x16 s[2];
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
    if (it + 1 < nsteps) load_keys(t0 + 32);
    float acc = 0.0f;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc = __builtin_fmaf(fast_exp2(__builtin_fmaf(s[nt][r], c, -rm[nt][r])), rw[nt][r], acc);
    acc = pair_sum(acc);
    if (hf == 0 && t0 + lm < N) out[t0 + lm] = acc;
  }
}

// ---------------------------------------------------------------------------
// Top-K of one mass row per workgroup.
// ---------------------------------------------------------------------------

constexpr int kTopkThreads = 256;
constexpr int kTopkWaves = kTopkThreads / 64;

// Add 1 to hist[d] for every active lane, one LDS atomic per distinct digit in the
// wave (the first radix digits of a mass row take few distinct values, so plain
// per-lane atomics would serialise on a handful of bins).
__device__ __forceinline__ void hist_add(uint32_t* hist, bool active, uint32_t d) {
  uint64_t todo = __builtin_amdgcn_ballot_w64(active);
  while (todo) {
    const int leader = __builtin_ctzll(todo);
    const uint32_t ld = (uint32_t)__builtin_amdgcn_readlane((int)d, leader);
    const uint64_t same = __builtin_amdgcn_ballot_w64(active && d == ld);
    if ((threadIdx.x & 63) == leader) atomicAdd(&hist[ld], (uint32_t)__builtin_popcountll(same));
    todo &= ~same;
  }
}

// Inclusive prefix sum over the 256 threads of the block; returns the block total.
__device__ __forceinline__ uint32_t block_scan(uint32_t x, uint32_t* wsum, uint32_t& incl) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t v = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) wsum[wid] = v;
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const uint32_t t = wsum[w];
    if (w < wid) before += t;
    total += t;
  }
  __syncthreads();
  incl = v + before;
  return total;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wsum[kTopkWaves];
  __shared__ uint32_t sel_state[3];
  const int row = blockIdx.x;
  const int N = a.N, K = a.K;
  const uint32_t* m = reinterpret_cast<const uint32_t*>(a.mass + (size_t)row * N);
  int32_t* out = a.idx + (size_t)row * a.kpad;
  const int tid = threadIdx.x;

  // Radix select of the K-th largest bit pattern, 8 bits per pass, MSB first.
  uint32_t prefix = 0, pmask = 0;
  uint32_t kr = (uint32_t)K;  // rank (1-based, from the top) still to locate
  uint32_t eq_total = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int base = 0; base < N; base += kTopkThreads) {
      const int i = base + tid;
      uint32_t bits = i < N ? m[i] : 0u;
      const bool act = i < N && (bits & pmask) == prefix;
      hist_add(hist, act, (bits >> shift) & 255u);
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t above = 0;
      int d = 255;
      for (; d > 0; --d) {
        if (above + hist[d] >= kr) break;
        above += hist[d];
      }
      sel_state[0] = (uint32_t)d;
      sel_state[1] = kr - above;
      sel_state[2] = hist[d];
    }
    __syncthreads();
    prefix |= sel_state[0] << shift;
    pmask |= 255u << shift;
    kr = sel_state[1];
    eq_total = sel_state[2];
    __syncthreads();
  }
  const uint32_t tau = prefix;
  // kr of the eq_total entries equal to tau are kept (the lowest ids).
  const bool all_ties = kr == eq_total;

  // Ascending compaction, 16 consecutive entries per thread per tile.
  constexpr int E = 16;
  uint32_t written = 0, eq_seen = 0;
  for (int base = 0; base < N; base += kTopkThreads * E) {
    const int i0 = base + tid * E;
    uint32_t bits[E];
#pragma unroll
    for (int e = 0; e < E; ++e) bits[e] = i0 + e < N ? m[i0 + e] : 0u;
    uint32_t ne = 0, ngt = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool in = i0 + e < N;
      ngt += (in && bits[e] > tau) ? 1u : 0u;
      ne += (in && bits[e] == tau) ? 1u : 0u;
    }
    uint32_t eq_before = 0;
    if (!all_ties) {
      uint32_t incl;
      const uint32_t tot = block_scan(ne, wsum, incl);
      eq_before = eq_seen + incl - ne;
      eq_seen += tot;
    }
    // entries kept by this thread
    uint32_t take_eq = ne;
    if (!all_ties) {
      const uint32_t room = kr > eq_before ? kr - eq_before : 0u;
      take_eq = ne < room ? ne : room;
    }
    const uint32_t nsel = ngt + take_eq;
    uint32_t incl;
    const uint32_t tot = block_scan(nsel, wsum, incl);
    uint32_t pos = written + incl - nsel;
    uint32_t eq_left = take_eq;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool in = i0 + e < N;
      bool keep = in && bits[e] > tau;
      if (in && bits[e] == tau && eq_left > 0) {
        keep = true;
        --eq_left;
      }
      if (keep) {
        if (pos < (uint32_t)K) out[pos] = i0 + e;  // exactly K are kept; stay inside the row regardless
        ++pos;
      }
    }
    written += tot;
  }
  for (int j = K + tid; j < a.kpad; j += kTopkThreads) out[j] = -1;
}

}  // namespace

hipError_t launch_group_mass(const MassArgs& a, int dtype, int head_dim, hipStream_t s) {
  const int items = a.hcount * a.G;
  const int blocks = xcd_grid((items + 3) / 4);
  if (dtype == DT_BF16) {
    if (head_dim == 128)
      hipLaunchKernelGGL((group_mass_kernel<__bf16, 128>), dim3(blocks), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((group_mass_kernel<__bf16, 64>), dim3(blocks), dim3(256), 0, s, a);
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL((group_mass_kernel<float, 128>), dim3(blocks), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((group_mass_kernel<float, 64>), dim3(blocks), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(a.rows), dim3(kTopkThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mcs
