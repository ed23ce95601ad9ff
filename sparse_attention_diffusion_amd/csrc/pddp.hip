// PDDP query grouping of the MC-Sparse hot path for gfx950 (MC-Sparse summary
// page, grouping paragraph: project a node's queries onto its principal
// direction, cut at the median, repeat until every group holds exactly C).
//
// The split tree's shape depends only on N and C (a node of n queries holds
// g = ceil(n/C) groups and its left child takes floor(g/2)*C of them), so every
// node is a contiguous slot range of perm known before any data is seen, and
// node k of level l is found by walking the l bits of k from the root.  The
// tree is processed one level at a time, all heads and all nodes of the level
// in one launch per stage:
//   1. stats   : per node, shifted sums  s = sum(x - r),  S = sum (x - r)(x - r)^T
//                with r the node's first query (exact zero for identical queries,
//                and no large-mean cancellation).  bf16 input: S on the bf16 MFMA
//                from a two-plane split of x - r (exact products); fp32 input: S
//                on v_mfma_f32_32x32x2_f32.  Big nodes are split over several
//                blocks that write partials.
//   2. power   : mean mu = r + s/n, covariance  C = S - n*m*m^T  (m = s/n), then a
//                fixed number of power steps from ones/sqrt(D) (stop only if
//                |C v| = 0); fused into stage 1 when one block holds the node
//                (bf16: on the covariance as the MFMA left it, in registers).
//   3. project : p = (x - mu) . v for every slot, as an order-preserving uint32.
//   4. split   : per node, radix select of the rank-cut element of the 64-bit
//                composite (projection key, token id), then a stable partition of
//                the node's slots: smaller composites to the left child.
#include "common.hpp"
#include "kernels.hpp"
#include "ldstile.hpp"

#include <type_traits>

namespace mcs {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxParts = 64;  // blocks per node at the top levels
constexpr int kStatsAhead = 2; // tiles of gathered rows in flight per bf16 statistics block

struct Node {
  int start, n;
  bool internal;
};

__host__ __device__ inline Node walk_node(int N, int C, int level, int k) {
  Node nd{0, N, false};
  for (int d = 0; d < level; ++d) {
    const int g = (nd.n + C - 1) / C;
    if (g <= 1) return Node{0, 0, false};
    const int cut = (g / 2) * C;
    if ((k >> (level - 1 - d)) & 1) {
      nd.start += cut;
      nd.n -= cut;
    } else {
      nd.n = cut;
    }
  }
  nd.internal = (nd.n + C - 1) / C >= 2;
  return nd;
}

// One level of the tree as launched: `nodes` blocks (times `parts`) per head.
// With `list`, block j of a head takes node list[j] (the level's internal nodes,
// listed on the device when the level also holds leaves); otherwise node j.
struct Level {
  int level, nodes, parts;
  const int32_t* list;
};

// Workspace carve-up (all offsets 256-byte aligned).
struct Ws {
  int32_t* tmp_perm;   // [H][N]
  uint32_t* keys;      // [H][N]
  float* partials;     // [H][kMaxParts][D + D*D]
  float* node_param;   // [H][max_nodes][2*D]   (mu, v)
  int32_t* node_list;  // [max_nodes]: the internal nodes of the current level
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline int level_count(int N, int C) {
  const int G = (N + C - 1) / C;
  int L = 0;
  while ((1 << L) < G) ++L;  // ceil(log2 G)
  return L;
}

inline int max_nodes(int N, int C) {
  const int L = level_count(N, C);
  return L == 0 ? 1 : (1 << (L - 1));
}

// Blocks per node: about one per 1024 rows, with at most kMaxParts partials per
// head in total (nodes * parts <= kMaxParts); one block per node from level 6 on.
inline int parts_for(int N, int level) {
  int p = (N >> level) / 1024;
  const int cap = kMaxParts >> level;
  if (p > cap) p = cap;
  return p < 1 ? 1 : p;
}

inline Ws carve(void* base, int H, int N, int D, int C) {
  char* p = (char*)base;
  Ws w;
  w.tmp_perm = (int32_t*)p;
  p += align256((size_t)H * N * 4);
  w.keys = (uint32_t*)p;
  p += align256((size_t)H * N * 4);
  w.partials = (float*)p;
  p += align256((size_t)H * kMaxParts * (D + (size_t)D * D) * 4);
  w.node_param = (float*)p;
  p += align256((size_t)H * max_nodes(N, C) * 2 * D * 4);
  w.node_list = (int32_t*)p;
  return w;
}

template <typename T>
__device__ __forceinline__ float ldf(const T* p) { return (float)*p; }

// Wave sum on DPP and permlane swaps (no LDS round trips).  Every step adds two
// partners whose values are each already uniform over their own half, and IEEE
// addition is commutative, so all 64 lanes end with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum_dpp(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  x += dpp_mov<0x141>(x);  // row_half_mirror: quad 0 <-> quad 1 of each 8 lanes
  x += dpp_mov<0x140>(x);  // row_mirror: the two halves of each 16-lane row
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);  // rows 0 <-> 1, 2 <-> 3
  return pair_sum(x);                                 // the two 32-lane halves
}

// Accumulated statistics of one block: fp32 MFMA tiles of S = sum (x - r)(x - r)^T.
// D = 128: 4 x 4 tiles of 32 x 32, wave w owns tile row w; D = 64: 2 x 2, one per wave.
template <typename T, int D>
struct StatsAcc {
  static constexpr int NT = D / 32;
  static constexpr int TPW = NT * NT / 4;  // output tiles per wave
  static constexpr int LDX = D + 32;       // padded LDS row stride (floats): rows 2s, 2s+1 hit disjoint banks
  static constexpr int TILE_ROWS = 64;     // rows staged per iteration (32 MFMA k-steps)
  static constexpr int CH = D * (int)sizeof(T) / 16;  // 16-byte chunks per row
  static constexpr int EPC = 16 / (int)sizeof(T);     // elements per chunk
  f32x16 acc[TPW];
};

// Accumulator tiles of wave `wid`: a-tile ta, b-tiles tb0 .. tb0 + TPW - 1.
template <int D>
__device__ __forceinline__ int acc_ta(int wid) { return D == 128 ? wid : (wid >> 1); }
template <int D>
__device__ __forceinline__ int acc_tb0(int wid) { return D == 128 ? 0 : (wid & 1); }

// LDS of the power iteration (floats): partial products [2][D/32][D], one copy of
// the direction per wave [4][D], then ref[D] (the node's first query) and m[D]
// (mean of x - ref).
template <int D>
struct PowLds {
  static constexpr int PART = 0;
  static constexpr int VW = PART + 2 * (D / 32) * D;
  static constexpr int VEC = VW + 4 * D;
  static constexpr int FLOATS = VEC + 2 * D;
};

// Floats of LDS of the fp32 statistics kernel: the row tile, then the power region.
template <typename T, int D>
constexpr int stats_f32_lds_floats() {
  return StatsAcc<T, D>::TILE_ROWS * StatsAcc<T, D>::LDX + PowLds<D>::FLOATS;
}

template <typename T>
__device__ __forceinline__ void chunk_to_f32(u32x4 w, float* out);
template <>
__device__ __forceinline__ void chunk_to_f32<__bf16>(u32x4 w, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = bf16lo(w[i]);
    out[2 * i + 1] = bf16hi(w[i]);
  }
}
template <>
__device__ __forceinline__ void chunk_to_f32<float>(u32x4 w, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(w[i]);
}

// n consecutive elements (n * sizeof(T) a multiple of 8 bytes, naturally aligned)
// as floats, with 16- or 8-byte loads.
template <typename T, int n>
__device__ __forceinline__ void load_dims(const T* p, float* out) {
  if constexpr (sizeof(T) * n % 16 == 0) {
#pragma unroll
    for (int c = 0; c < (int)(sizeof(T) * n / 16); ++c)
      chunk_to_f32<T>(reinterpret_cast<const u32x4*>(p)[c], out + c * (16 / (int)sizeof(T)));
  } else {
    static_assert(sizeof(T) * n == 8, "8-byte piece");
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    if constexpr (sizeof(T) == 2) {
      out[0] = bf16lo(w[0]);
      out[1] = bf16hi(w[0]);
      out[2] = bf16lo(w[1]);
      out[3] = bf16hi(w[1]);
    } else {
      out[0] = __uint_as_float(w[0]);
      out[1] = __uint_as_float(w[1]);
    }
  }
}

// Projection keys of slots [r0, r1): key = float_key((x - mu) . v), 16 lanes per
// row, D/16 consecutive dims per lane.  Each thread has the perm entries and then
// the rows of kRowsInFlight slots in flight before it reduces any of them (one
// slot at a time left the pass bound by the perm -> row load latency).
constexpr int kRowsInFlight = 4;
template <typename T, int D>
__device__ __forceinline__ void project_rows(const T* qh, const int32_t* permh, uint32_t* keys, int r0, int r1,
                                             const float (&mu)[D / 16], const float (&v)[D / 16]) {
  constexpr int DPL = D / 16;
  constexpr int RSTEP = kThreads / 16;
  constexpr int U = kRowsInFlight;
  const int tid = threadIdx.x, sub = tid & 15, rgrp = tid >> 4;
  for (int row0 = r0 + rgrp; row0 < r1; row0 += U * RSTEP) {
    int tok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = row0 + u * RSTEP;
      tok[u] = row < r1 ? permh[row] : 0;  // past the range: any row of the head, not stored
    }
    float x[U][DPL];
#pragma unroll
    for (int u = 0; u < U; ++u) load_dims<T, DPL>(qh + (size_t)tok[u] * D + sub * DPL, x[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float p = 0.0f;
#pragma unroll
      for (int j = 0; j < DPL; ++j) p = __builtin_fmaf(x[u][j] - mu[j], v[j], p);
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) p += __shfl_xor(p, o, 16);
      const int row = row0 + u * RSTEP;
      if (sub == 0 && row < r1) keys[row] = float_key(p);
    }
  }
}

// Accumulate the shifted sums of rows [r0, r1) of a node (slots, mapped through
// perm) into colsum (threads tid < D own one column) and the MFMA tiles.
template <typename T, int D>
__device__ void stats_rows(const T* qh, const int32_t* permh, const float* ref, int r0, int r1, float* xs,
                           StatsAcc<T, D>& sa, float& colsum) {
  using SA = StatsAcc<T, D>;
  const int tid = threadIdx.x, lane = tid & 63, wid = wave_id(), hf = lane >> 5, lm = lane & 31;
  for (int t = 0; t < SA::TPW; ++t) sa.acc[t] = f32x16{};
  colsum = 0.0f;
  for (int base = r0; base < r1; base += SA::TILE_ROWS) {
    const int nrows = min(SA::TILE_ROWS, r1 - base);
    __syncthreads();  // previous tile fully consumed
    for (int e = tid; e < SA::TILE_ROWS * SA::CH; e += kThreads) {
      const int rr = e / SA::CH, ch = e - rr * SA::CH;
      float x[SA::EPC];
      if (rr < nrows) {
        const int tok = permh[base + rr];
        const u32x4 w = *reinterpret_cast<const u32x4*>(qh + (size_t)tok * D + ch * SA::EPC);
        chunk_to_f32<T>(w, x);
#pragma unroll
        for (int i = 0; i < SA::EPC; ++i) x[i] -= ref[ch * SA::EPC + i];
      } else {
#pragma unroll
        for (int i = 0; i < SA::EPC; ++i) x[i] = 0.0f;
      }
#pragma unroll
      for (int i = 0; i < SA::EPC; ++i) xs[rr * SA::LDX + ch * SA::EPC + i] = x[i];
    }
    __syncthreads();
    if (tid < D) {
      for (int rr = 0; rr < nrows; ++rr) colsum += xs[rr * SA::LDX + tid];
    }
    // S += X^T X: k-step s covers rows 2s (lanes 0-31) and 2s+1 (lanes 32-63).
    const int ksteps = (nrows + 1) >> 1;
    for (int s = 0; s < ksteps; ++s) {
      const float* row = xs + (2 * s + hf) * SA::LDX;
      if constexpr (D == 128) {
        const float av = row[lm + 32 * wid];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) sa.acc[tb] = mfma_f32(av, row[lm + 32 * tb], sa.acc[tb]);
      } else {
        const int ta = wid >> 1, tb = wid & 1;
        sa.acc[0] = mfma_f32(row[lm + 32 * ta], row[lm + 32 * tb], sa.acc[0]);
      }
    }
  }
}

// Row-major D x D store of accumulator tiles (a = 32*ta + row of the tile,
// b = 32*tb + lane % 32).
template <int D, int TPW>
__device__ void store_acc(const f32x16 (&acc)[TPW], int ta, int tb0, float* dst) {
  const int lane = threadIdx.x & 63, hf = lane >> 5, lm = lane & 31;
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int a = 32 * ta + 8 * (r >> 2) + 4 * hf + (r & 3);
      const int b = 32 * (tb0 + t) + lm;
      dst[a * D + b] = acc[t][r];
    }
}

// Power iteration on C = S - n m m^T, with S in MFMA accumulator tiles: lane l of
// a wave holds S[a][b] for b = 32*(tb0 + t) + l % 32 and the 16 a = 32*ta +
// 8*(r/4) + 4*(l/32) + r%4 (r = accumulator register).  pl is the PowLds region,
// with ref and m filled in and visible to the whole block.
//
// C is symmetric, so (C v)[b] = sum_a C[a][b] v[a]: summed within the lane, then
// over the two lane halves, then over the a-tiles through LDS (one barrier per
// step; the partial buffers alternate, and a buffer is rewritten only after the
// next barrier).  Every wave forms the whole new vector from the same data in the
// same order, so all waves hold bitwise equal copies and take the zero-norm exit
// together; each keeps its own copy, which is left in pl + VW + wave*D.  Wave 0
// writes {mu = ref + m, v} to out.
template <int D, int TPW>
__device__ __forceinline__ void power_regs(f32x16 (&acc)[TPW], int ta, int tb0, int n, int iters, float* pl,
                                           float* out) {
  constexpr int NTA = D / 32;
  const int lane = threadIdx.x & 63, wid = wave_id(), hf = lane >> 5, lm = lane & 31;
  float* partb = pl + PowLds<D>::PART;
  float* vwave = pl + PowLds<D>::VW + wid * D;
  const float* vec = pl + PowLds<D>::VEC;
  {
    float ma[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) ma[r] = vec[D + 32 * ta + 8 * (r >> 2) + 4 * hf + (r & 3)];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const float mb = vec[D + 32 * (tb0 + t) + lm];
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] -= (float)n * ma[r] * mb;
    }
  }
  for (int e = lane; e < D; e += 64) vwave[e] = 1.0f / sqrtf((float)D);
  for (int it = 0; it < iters; ++it) {
    float va[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 v4 = *(const f32x4*)(vwave + 32 * ta + 8 * j + 4 * hf);
#pragma unroll
      for (int i = 0; i < 4; ++i) va[4 * j + i] = v4[i];
    }
    float* pw = partb + (it & 1) * NTA * D;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      float p = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) p = __builtin_fmaf(acc[t][r], va[r], p);
      p = pair_sum(p);
      if (hf == 0) pw[ta * D + 32 * (tb0 + t) + lm] = p;
    }
    __syncthreads();
    constexpr int PER = D / 64;
    float wv[PER];
    float sq = 0.0f;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      float s = 0.0f;
#pragma unroll
      for (int t2 = 0; t2 < NTA; ++t2) s += pw[t2 * D + lane + 64 * j];
      wv[j] = s;
      sq = __builtin_fmaf(s, s, sq);
    }
    sq = wave_sum_dpp(sq);
    if (sq == 0.0f) break;
    const float inv = 1.0f / sqrtf(sq);
#pragma unroll
    for (int j = 0; j < PER; ++j) vwave[lane + 64 * j] = wv[j] * inv;
  }
  if (wid == 0) {
    for (int e = lane; e < D; e += 64) {
      out[e] = vec[e] + vec[D + e];  // mu
      out[D + e] = vwave[e];         // v
    }
  }
}

// After power_regs: projections of the node's slots with this wave's copy of v.
template <typename T, int D>
__device__ __forceinline__ void project_node(const T* qh, const int32_t* permh, uint32_t* keys, int r0, int r1,
                                             const float* pl) {
  constexpr int DPL = D / 16;
  const int sub = threadIdx.x & 15;
  const float* vwave = pl + PowLds<D>::VW + wave_id() * D;
  const float* vec = pl + PowLds<D>::VEC;
  float mu[DPL], v[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) {
    mu[j] = vec[sub * DPL + j] + vec[D + sub * DPL + j];
    v[j] = vwave[sub * DPL + j];
  }
  project_rows<T, D>(qh, permh, keys, r0, r1, mu, v);
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void pddp_stats_kernel(PddpArgs a, Ws w, Level lv) {
  extern __shared__ float smem[];
  using SA = StatsAcc<T, D>;
  const int P = lv.parts;
  const int per_head = lv.nodes * P;
  const int h = blockIdx.x / per_head;
  const int rem = blockIdx.x - h * per_head;
  const int kk = rem / P, part = rem - kk * P;  // kk: launch index, k: node id
  const int k = lv.list ? lv.list[kk] : kk;
  const Node nd = walk_node(a.N, a.C, lv.level, k);
  if (!nd.internal) return;
  const int chunk = (nd.n + P - 1) / P;
  const int r0 = nd.start + part * chunk;
  const int r1 = min(nd.start + nd.n, r0 + chunk);
  const T* qh = (const T*)a.q + (size_t)h * a.N * D;
  const int32_t* permh = a.perm + (size_t)h * a.N;

  float* tile = smem;                                       // row tile
  float* pl = smem + SA::TILE_ROWS * SA::LDX;               // power region
  float* vec = pl + PowLds<D>::VEC;                         // ref[D], m[D]
  const int tid = threadIdx.x, wid = wave_id();
  const int tok0 = permh[nd.start];
  if (tid < D) vec[tid] = ldf(qh + (size_t)tok0 * D + tid);
  __syncthreads();
  SA sa;
  float colsum;
  stats_rows<T, D>(qh, permh, vec, r0, max(r1, r0), tile, sa, colsum);
  if (P > 1) {
    float* dst = w.partials + ((size_t)h * kMaxParts + (size_t)kk * P + part) * (D + (size_t)D * D);
    if (tid < D) dst[tid] = colsum;
    store_acc<D, SA::TPW>(sa.acc, acc_ta<D>(wid), acc_tb0<D>(wid), dst + D);
    return;
  }
  if (tid < D) vec[D + tid] = colsum / (float)nd.n;
  __syncthreads();
  const int maxn = 1 << lv.level;
  power_regs<D, SA::TPW>(sa.acc, acc_ta<D>(wid), acc_tb0<D>(wid), nd.n, a.iters, pl,
                         w.node_param + ((size_t)h * maxn + k) * 2 * D);
  project_node<T, D>(qh, permh, w.keys + (size_t)h * a.N, nd.start, nd.start + nd.n, pl);
}

// Nodes split over several statistics blocks: fixed-order sums of their partials
// (column sums, then S straight into the accumulator layout), then power_regs.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void pddp_power_kernel(PddpArgs a, Ws w, Level lv) {
  extern __shared__ float smem[];  // PowLds<D>
  constexpr int TPW = (D / 32) * (D / 32) / 4;
  const int h = blockIdx.x / lv.nodes;
  const int kk = blockIdx.x - h * lv.nodes;  // launch index; k: node id
  const int k = lv.list ? lv.list[kk] : kk;
  const Node nd = walk_node(a.N, a.C, lv.level, k);
  if (!nd.internal) return;
  const int P = lv.parts;
  const T* qh = (const T*)a.q + (size_t)h * a.N * D;
  const int32_t* permh = a.perm + (size_t)h * a.N;
  const int tid = threadIdx.x, lane = tid & 63, wid = wave_id(), hf = lane >> 5, lm = lane & 31;
  const size_t stride = D + (size_t)D * D;
  const float* src = w.partials + ((size_t)h * kMaxParts + (size_t)kk * P) * stride;
  float* vec = smem + PowLds<D>::VEC;
  if (tid < D) {
    float s = 0.0f;
#pragma unroll 8
    for (int p = 0; p < P; ++p) s += src[p * stride + tid];
    vec[D + tid] = s / (float)nd.n;
    vec[tid] = ldf(qh + (size_t)permh[nd.start] * D + tid);
  }
  const int ta = acc_ta<D>(wid), tb0 = acc_tb0<D>(wid);
  f32x16 acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = f32x16{};
  for (int p = 0; p < P; ++p) {
    const float* sp = src + p * stride + D;
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] += sp[(32 * ta + 8 * (r >> 2) + 4 * hf + (r & 3)) * D + 32 * (tb0 + t) + lm];
  }
  __syncthreads();
  const int maxn = 1 << lv.level;
  power_regs<D, TPW>(acc, ta, tb0, nd.n, a.iters, smem, w.node_param + ((size_t)h * maxn + k) * 2 * D);
}

// ---------------------------------------------------------------------------
// bf16 statistics on the bf16 MFMA.
//
// A node's shifted rows d = x - r (x, r bf16; d exact in fp32) are staged in LDS
// as two bf16 planes, hi = bf16(d) and lo = bf16(d - hi).  hi + lo = d exactly
// when |x| and |r| are within a factor 2^7 of each other, and to about 2^-17
// relative otherwise.  Then
//   S = sum d d^T = sum (hi hi^T + hi lo^T + lo hi^T + lo lo^T),
// four v_mfma_f32_32x32x16_bf16 per 16 rows and 32x32 tile: every product is
// exact in fp32 and the sums are fp32, as on the fp32 MFMA, at a quarter of its
// issue cost.  Wave w owns accumulator tiles (ta, tb): ta = w, tb = 0..3 at
// D = 128; (w / 2, w % 2) at D = 64.
//
// The MFMA operands of S = X^T X are columns of X (one dimension per lane, 8 rows
// per lane in its k-slots), read from the row-major planes with the gfx950
// transposing read ds_read_b64_tr_b16: within a 16-lane group, lane j receives
// element j % 4 of the 8-byte pieces addressed by lanes 4t + j / 4, t = 0..3.
// Lane m of group q addresses row 4*(q / 2) + m / 4 (+ 8 for the second read) and
// dims 16*(q % 2) + 4*(m % 4) of the tile, so lane l ends up with dimension l % 32
// of row 8*s + 4*(l / 32) + t in k-slot 4*s + t (s = read, t = 0..3).  A and B
// use the same slot -> row map, and the 16 rows of a k-step each appear once.
//
// Plane rows are 2D bytes with the 32-byte units of row r XOR-ed by r % 4, so the
// four rows one 16-lane group reads fall in four different 32-byte units.
template <int D>
struct BStats {
  static constexpr int TR = 32;                // rows per tile: two 16-row k-steps
  static constexpr int ROWB = 2 * D;           // bytes per plane row
  static constexpr int PLANE = TR * ROWB;
  static constexpr int BUF = 2 * PLANE;        // hi plane, then lo plane
  static constexpr int CH = D / 8;             // 16-byte chunks per row
  static constexpr int RSTEP = kThreads / CH;  // rows between the chunks one thread stages
  static constexpr int ITEMS = TR / RSTEP;     // chunks staged per thread per tile
  static constexpr int NTA = D / 32;           // 32-dim tiles per side
  static constexpr int TPW = NTA * NTA / 4;    // accumulator tiles per wave
  // LDS carve-up (bytes): two tile buffers, then the power region.  The
  // column-sum partials reuse the tile buffers after the last tile.
  static constexpr int OFF_POW = 2 * BUF;
  static constexpr int BYTES = OFF_POW + PowLds<D>::FLOATS * 4;
  static_assert(RSTEP * D * 4 <= 2 * BUF, "column-sum partials fit the tile buffers");
  static_assert(ITEMS * RSTEP == TR, "tile rows split evenly over the staging threads");
  __device__ static int off(int row, int c) { return row * ROWB + (((c >> 1) ^ (row & 3)) << 5) + ((c & 1) << 4); }
};

// Lane byte offset (within a plane, first k-step) of the transposing reads of
// 32-dim tile `tile`.
template <int D>
__device__ __forceinline__ int tr_lane_off(int lane, int tile) {
  const int q = lane >> 4, m = lane & 15;
  const int row = 4 * (q >> 1) + (m >> 2);  // row % 4 == m / 4
  return row * BStats<D>::ROWB + (((2 * tile + (q & 1)) ^ (m >> 2)) << 5) + 8 * (m & 3);
}

// One MFMA operand: dimension lane % 32 of the lane's 8 rows.
template <int D>
__device__ __forceinline__ bf16x8 tr_read(const LDSP char* p) {
  typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
  const bf4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDSP bf4*)p);
  const bf4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDSP bf4*)(p + 8 * BStats<D>::ROWB));
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3)))
void pddp_stats_bf16_kernel(PddpArgs a, Ws w, Level lv) {
  using B = BStats<D>;
  extern __shared__ float smem[];
  const int P = lv.parts;
  const int per_head = lv.nodes * P;
  const int h = blockIdx.x / per_head;
  const int rem = blockIdx.x - h * per_head;
  const int kk = rem / P, part = rem - kk * P;  // kk: launch index, k: node id
  const int k = lv.list ? lv.list[kk] : kk;
  const Node nd = walk_node(a.N, a.C, lv.level, k);
  if (!nd.internal) return;
  const int chunk = (nd.n + P - 1) / P;
  const int r0 = nd.start + part * chunk;
  const int r1 = min(nd.start + nd.n, r0 + chunk);
  const int ntiles = r1 > r0 ? (r1 - r0 + B::TR - 1) / B::TR : 0;
  const bf16* qh = (const bf16*)a.q + (size_t)h * a.N * D;
  const int32_t* permh = a.perm + (size_t)h * a.N;
  const int tid = threadIdx.x, lane = tid & 63, wid = wave_id();
  LDSP char* lds = (LDSP char*)smem;

  // Staging: thread tid converts chunk c of rows rbase + RSTEP*j of each tile.
  const int c = tid % B::CH, rbase = tid / B::CH;
  const int tok0 = permh[nd.start];
  float refc[8];
  chunk_to_f32<bf16>(*reinterpret_cast<const u32x4*>(qh + (size_t)tok0 * D + 8 * c), refc);
  float cs[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) cs[i] = 0.0f;

  // Rows past the part read its last row (in bounds for any tile index, padding
  // tiles included: r1 - 1 >= nd.start) and are staged as zeros.
  auto load_toks = [&](int tile, int (&tk)[B::ITEMS]) {
#pragma unroll
    for (int j = 0; j < B::ITEMS; ++j) tk[j] = permh[min(r0 + tile * B::TR + rbase + B::RSTEP * j, r1 - 1)];
  };
  auto load_rows = [&](const int (&tk)[B::ITEMS], u32x4 (&xv)[B::ITEMS]) {
#pragma unroll
    for (int j = 0; j < B::ITEMS; ++j) xv[j] = *reinterpret_cast<const u32x4*>(qh + (size_t)tk[j] * D + 8 * c);
  };
  auto stage = [&](LDSP char* buf, int tile, const u32x4 (&xv)[B::ITEMS]) {
#pragma unroll
    for (int j = 0; j < B::ITEMS; ++j) {
      float x[8];
      chunk_to_f32<bf16>(xv[j], x);
      const bool ok = r0 + tile * B::TR + rbase + B::RSTEP * j < r1;  // rows past the part contribute zero
      u32x4 hw, lw;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float d0 = ok ? x[2 * i] - refc[2 * i] : 0.0f;
        const float d1 = ok ? x[2 * i + 1] - refc[2 * i + 1] : 0.0f;
        cs[2 * i] += d0;
        cs[2 * i + 1] += d1;
        hw[i] = pack_bf16x2(d0, d1);
        lw[i] = pack_bf16x2(d0 - bf16lo(hw[i]), d1 - bf16hi(hw[i]));
      }
      const int off = B::off(rbase + B::RSTEP * j, c);
      *(LDSP u32x4*)(buf + off) = hw;
      *(LDSP u32x4*)(buf + B::PLANE + off) = lw;
    }
  };

  const int ta = D == 128 ? wid : (wid >> 1);
  const int tb0 = D == 128 ? 0 : (wid & 1);
  const int aoff = tr_lane_off<D>(lane, ta);
  int boff[B::TPW];
#pragma unroll
  for (int t = 0; t < B::TPW; ++t) boff[t] = tr_lane_off<D>(lane, tb0 + t);
  f32x16 acc[B::TPW];
#pragma unroll
  for (int t = 0; t < B::TPW; ++t) acc[t] = f32x16{};

  auto mma_tile = [&](const LDSP char* buf) {
#pragma unroll
    for (int ks = 0; ks < B::TR / 16; ++ks) {
      const LDSP char* base = buf + 16 * ks * B::ROWB;
      const bf16x8 ah = tr_read<D>(base + aoff), al = tr_read<D>(base + B::PLANE + aoff);
      bf16x8 bh[B::TPW], bl[B::TPW];
#pragma unroll
      for (int t = 0; t < B::TPW; ++t) {
        bh[t] = tr_read<D>(base + boff[t]);
        bl[t] = tr_read<D>(base + B::PLANE + boff[t]);
      }
#pragma unroll
      for (int t = 0; t < B::TPW; ++t) acc[t] = mfma_bf16(ah, bh[t], acc[t]);
#pragma unroll
      for (int t = 0; t < B::TPW; ++t) acc[t] = mfma_bf16(ah, bl[t], acc[t]);
#pragma unroll
      for (int t = 0; t < B::TPW; ++t) acc[t] = mfma_bf16(al, bh[t], acc[t]);
#pragma unroll
      for (int t = 0; t < B::TPW; ++t) acc[t] = mfma_bf16(al, bl[t], acc[t]);
    }
  };

  // Tile t is read from LDS buffer t % 2 while tile t + 1 is converted into the
  // other one; one barrier per tile.  The gathered row loads run kStatsAhead
  // tiles ahead: register slot s holds the rows of tiles s, s + A, s + 2A, ...
  // (A = kStatsAhead), and their perm entries are read A tiles before the rows,
  // so a wait for a tile's rows leaves the next A - 1 tiles' loads in flight
  // (one tile in flight left the deep levels bound by the gather latency).
  // The tile count is padded to a multiple of A with empty tiles, which stage
  // as zeros and add nothing, so every step issues the same loads.
  constexpr int A = kStatsAhead;
  const int npad = (ntiles + A - 1) / A * A;
  int tk[A][B::ITEMS];
  u32x4 xv[A][B::ITEMS];
#pragma unroll
  for (int s = 0; s < A; ++s) load_toks(s, tk[s]);
#pragma unroll
  for (int s = 0; s < A; ++s) {
    load_rows(tk[s], xv[s]);
    load_toks(s + A, tk[s]);
  }
  stage(lds, 0, xv[0]);
  load_rows(tk[0], xv[0]);
  load_toks(2 * A, tk[0]);
  __syncthreads();
  for (int t0 = 0; t0 < npad; t0 += A) {
#pragma unroll
    for (int u = 0; u < A; ++u) {
      const int t = t0 + u, s = (u + 1) % A;  // slot of tile t + 1
      mma_tile(lds + (t & 1) * B::BUF);
      stage(lds + ((t + 1) & 1) * B::BUF, t + 1, xv[s]);
      load_rows(tk[s], xv[s]);
      load_toks(t + 1 + 2 * A, tk[s]);
      __syncthreads();
    }
  }

  // Column sums: per-thread partials (tile buffers are free now), then one
  // fixed-order sum per dimension.
  float* csp = smem;
#pragma unroll
  for (int i = 0; i < 8; ++i) csp[rbase * D + 8 * c + i] = cs[i];
  __syncthreads();
  float colsum = 0.0f;
  if (tid < D)
    for (int rr = 0; rr < B::RSTEP; ++rr) colsum += csp[rr * D + tid];

  if (P > 1) {
    float* dst = w.partials + ((size_t)h * kMaxParts + (size_t)kk * P + part) * (D + (size_t)D * D);
    if (tid < D) dst[tid] = colsum;
    store_acc<D, B::TPW>(acc, ta, tb0, dst + D);
    return;
  }

  const int maxn = 1 << lv.level;
  float* pl = smem + B::OFF_POW / 4;
  float* vec = pl + PowLds<D>::VEC;
  if (tid < D) vec[D + tid] = colsum / (float)nd.n;
  if (tid < B::CH)
#pragma unroll
    for (int i = 0; i < 8; ++i) vec[8 * c + i] = refc[i];
  __syncthreads();
  power_regs<D, B::TPW>(acc, ta, tb0, nd.n, a.iters, pl, w.node_param + ((size_t)h * maxn + k) * 2 * D);
  project_node<bf16, D>(qh, permh, w.keys + (size_t)h * a.N, nd.start, nd.start + nd.n, pl);
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void pddp_project_kernel(PddpArgs a, Ws w, Level lv) {
  const int P = lv.parts;
  const int per_head = lv.nodes * P;
  const int h = blockIdx.x / per_head;
  const int rem = blockIdx.x - h * per_head;
  const int kk = rem / P, part = rem - kk * P;  // kk: launch index, k: node id
  const int k = lv.list ? lv.list[kk] : kk;
  const Node nd = walk_node(a.N, a.C, lv.level, k);
  if (!nd.internal) return;
  const int chunk = (nd.n + P - 1) / P;
  const int r0 = nd.start + part * chunk;
  const int r1 = min(nd.start + nd.n, r0 + chunk);
  const int maxn = 1 << lv.level;
  const float* prm = w.node_param + ((size_t)h * maxn + k) * 2 * D;
  const T* qh = (const T*)a.q + (size_t)h * a.N * D;
  const int32_t* permh = a.perm + (size_t)h * a.N;
  // 16 lanes per row, D/16 consecutive dims per lane.
  constexpr int DPL = D / 16;
  const int sub = threadIdx.x & 15;
  float mu[DPL], v[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) {
    mu[j] = prm[sub * DPL + j];
    v[j] = prm[D + sub * DPL + j];
  }
  project_rows<T, D>(qh, permh, w.keys + (size_t)h * a.N, r0, r1, mu, v);
}

// Histogram add of digit d for the active lanes: one LDS atomic for the wave when
// every active lane has the same digit (the usual case for the high digits of a
// node's keys), else one per lane.
__device__ __forceinline__ void hist_add(uint32_t* hist, bool active, uint32_t d) {
  const uint64_t act = __builtin_amdgcn_ballot_w64(active);
  if (act == 0) return;
  const int leader = __builtin_ctzll(act);
  const uint32_t ld = (uint32_t)__builtin_amdgcn_readlane((int)d, leader);
  const uint64_t same = __builtin_amdgcn_ballot_w64(active && d == ld);
  if (same == act) {
    if ((threadIdx.x & 63) == leader) atomicAdd(&hist[ld], (uint32_t)__builtin_popcountll(act));
  } else if (active) {
    atomicAdd(&hist[d], 1u);
  }
}

// Inclusive block scan of x over NT threads; returns the block total.
template <int NT>
__device__ __forceinline__ uint32_t block_scan(uint32_t x, uint32_t* wsum, uint32_t& incl) {
  const int lane = threadIdx.x & 63, wid = wave_id();
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
  for (int ww = 0; ww < NT / 64; ++ww) {
    const uint32_t t = wsum[ww];
    if (ww < wid) before += t;
    total += t;
  }
  __syncthreads();
  incl = v + before;
  return total;
}

// One radix pass over the node: histogram of digit `shift` of the selected word
// among entries whose already-fixed bits match; returns the digit holding rank kr
// (0-based, ascending) and updates kr to the rank inside that digit.  The digit is
// the bin whose inclusive prefix count first exceeds kr, found by a block scan of
// the 256 bins.
template <int NT>
__device__ uint32_t radix_pass(const uint32_t* keys, const int32_t* toks, int start, int n, bool use_tok,
                               uint32_t hi_val, uint32_t prefix, uint32_t pmask, int shift, uint32_t& kr,
                               uint32_t* hist, uint32_t* wsum, uint32_t* bcast) {
  const int tid = threadIdx.x;
  for (int i = tid; i < 256; i += NT) hist[i] = 0;
  __syncthreads();
  for (int b = 0; b < n; b += NT) {
    const int i = b + tid;
    bool act = i < n;
    uint32_t word = 0;
    if (act) {
      const uint32_t hk = keys[start + i];
      if (use_tok) {
        act = hk == hi_val;
        word = (uint32_t)toks[start + i];
      } else {
        word = hk;
      }
      act = act && (word & pmask) == prefix;
    }
    hist_add(hist, act, (word >> shift) & 255u);
  }
  __syncthreads();
  const uint32_t cnt = tid < 256 ? hist[tid] : 0u;
  uint32_t incl;
  block_scan<NT>(cnt, wsum, incl);  // its barriers also order the hist reads before the next clear
  if (tid < 256 && incl > kr && incl - cnt <= kr) {  // exactly one bin, as kr < the pass's count
    bcast[0] = (uint32_t)tid;
    bcast[1] = kr - (incl - cnt);
  }
  __syncthreads();
  const uint32_t d = bcast[0];
  kr = bcast[1];
  return d;  // bcast is rewritten only after the next pass's barriers
}

template <int NT>
__global__ __launch_bounds__(NT) void pddp_split_kernel(PddpArgs a, Ws w, Level lv) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wsum[NT / 64];
  __shared__ uint32_t bcast[2];
  const int h = blockIdx.x / lv.nodes;
  const int kk = blockIdx.x - h * lv.nodes;  // launch index; k: node id
  const int k = lv.list ? lv.list[kk] : kk;
  const Node nd = walk_node(a.N, a.C, lv.level, k);
  if (!nd.internal) return;
  const int g = (nd.n + a.C - 1) / a.C;
  const uint32_t cut = (uint32_t)((g / 2) * a.C);
  const uint32_t* keys = w.keys + (size_t)h * a.N;
  const int32_t* src = w.tmp_perm + (size_t)h * a.N;  // this level's input order
  int32_t* dst = a.perm + (size_t)h * a.N;

  // Rank-cut element of the composite (key, token) in ascending order.
  uint32_t kr = cut, prefix = 0, pmask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    const uint32_t d = radix_pass<NT>(keys, src, nd.start, nd.n, false, 0, prefix, pmask, shift, kr, hist, wsum, bcast);
    prefix |= d << shift;
    pmask |= 255u << shift;
  }
  const uint32_t thi = prefix;
  uint32_t ttok = 0;
  const bool need_tok = kr > 0;  // some entries equal to thi go left: split them by token id
  if (need_tok) {
    prefix = 0;
    pmask = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
      const uint32_t d = radix_pass<NT>(keys, src, nd.start, nd.n, true, thi, prefix, pmask, shift, kr, hist, wsum, bcast);
      prefix |= d << shift;
      pmask |= 255u << shift;
    }
    ttok = prefix;
  }

  // Stable partition of the node's slots.
  constexpr int E = 8;
  const int tid = threadIdx.x;
  uint32_t left_done = 0, right_done = 0;
  for (int b = 0; b < nd.n; b += NT * E) {
    const int i0 = b + tid * E;
    int32_t tk[E];
    bool lf[E];
    uint32_t nl = 0, nr = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = i0 + e;
      lf[e] = false;
      tk[e] = 0;
      if (i < nd.n) {
        const uint32_t hk = keys[nd.start + i];
        tk[e] = src[nd.start + i];
        lf[e] = hk < thi || (need_tok && hk == thi && (uint32_t)tk[e] < ttok);
        nl += lf[e] ? 1u : 0u;
        nr += lf[e] ? 0u : 1u;
      }
    }
    uint32_t incl;
    const uint32_t packed = nl | (nr << 16);
    const uint32_t tot = block_scan<NT>(packed, wsum, incl);
    uint32_t pl = left_done + (incl & 0xffffu) - nl;
    uint32_t pr = right_done + (incl >> 16) - nr;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (i0 + e >= nd.n) continue;
      // the threshold puts exactly `cut` entries left; the bounds keep every
      // store inside this node's slots regardless
      if (lf[e]) {
        if (pl < cut) dst[nd.start + pl] = tk[e];
        ++pl;
      } else {
        if (pr < (uint32_t)nd.n - cut) dst[nd.start + cut + pr] = tk[e];
        ++pr;
      }
    }
    left_done += tot & 0xffffu;
    right_done += tot >> 16;
  }
}

// The internal nodes of `level` (those still holding two or more groups) in
// ascending order, for a level that also holds leaves: one block.
__global__ __launch_bounds__(1024) void pddp_list_kernel(int N, int C, int level, int32_t* list) {
  __shared__ uint32_t wsum[1024 / 64];
  const int nodes = 1 << level;
  uint32_t done = 0;
  for (int b = 0; b < nodes; b += 1024) {
    const int k = b + (int)threadIdx.x;
    const bool f = k < nodes && walk_node(N, C, level, k).internal;
    uint32_t incl;
    const uint32_t tot = block_scan<1024>(f ? 1u : 0u, wsum, incl);
    if (f) list[done + incl - 1] = k;
    done += tot;
  }
}

__global__ void iota_kernel(int32_t* perm, int H, int N) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < (size_t)H * N) perm[i] = (int32_t)(i % (size_t)N);
}

template <typename T, int D>
hipError_t run_levels(const PddpArgs& a, hipStream_t s) {
  Ws w = carve(a.ws, a.H, a.N, D, a.C);
  const size_t total = (size_t)a.H * a.N;
  hipLaunchKernelGGL(iota_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a.perm, a.H, a.N);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int L = level_count(a.N, a.C);
  const size_t lds_f32 = (size_t)stats_f32_lds_floats<T, D>() * sizeof(float);
  const size_t lds_pow = (size_t)PowLds<D>::FLOATS * sizeof(float);
  for (int l = 0; l < L; ++l) {
    // internal nodes of the level, counted on the host (the tree depends only on N, C)
    int internal = 0;
    for (int k = 0; k < (1 << l); ++k) internal += walk_node(a.N, a.C, l, k).internal ? 1 : 0;
    Level lv{l, 1 << l, parts_for(a.N, l), nullptr};
    if (internal < lv.nodes) {  // the level also holds leaves: launch its internal nodes only
      hipLaunchKernelGGL(pddp_list_kernel, dim3(1), dim3(1024), 0, s, a.N, a.C, l, w.node_list);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      lv.nodes = internal;
      lv.list = w.node_list;
    }
    if (lv.nodes == 0) continue;
    const unsigned nb = (unsigned)(a.H * lv.nodes * lv.parts);
    if constexpr (std::is_same<T, __bf16>::value)
      hipLaunchKernelGGL((pddp_stats_bf16_kernel<D>), dim3(nb), dim3(kThreads), BStats<D>::BYTES, s, a, w, lv);
    else
      hipLaunchKernelGGL((pddp_stats_kernel<T, D>), dim3(nb), dim3(kThreads), lds_f32, s, a, w, lv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (lv.parts > 1) {
      hipLaunchKernelGGL((pddp_power_kernel<T, D>), dim3(a.H * lv.nodes), dim3(kThreads), lds_pow, s, a, w, lv);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (lv.parts > 1) {  // single-block nodes project inside the statistics kernel
      hipLaunchKernelGGL((pddp_project_kernel<T, D>), dim3(nb), dim3(kThreads), 0, s, a, w, lv);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = hipMemcpyAsync(w.tmp_perm, a.perm, total * 4, hipMemcpyDeviceToDevice, s)) != hipSuccess) return e;
    // few nodes (the top levels): 1024 threads per node
    if (lv.nodes <= 4)
      hipLaunchKernelGGL((pddp_split_kernel<1024>), dim3(a.H * lv.nodes), dim3(1024), 0, s, a, w, lv);
    else
      hipLaunchKernelGGL((pddp_split_kernel<kThreads>), dim3(a.H * lv.nodes), dim3(kThreads), 0, s, a, w, lv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

size_t pddp_workspace_bytes(int H, int N, int D, int C) {
  return align256((size_t)H * N * 4) * 2 + align256((size_t)H * kMaxParts * (D + (size_t)D * D) * 4) +
         align256((size_t)H * max_nodes(N, C) * 2 * D * 4) + align256((size_t)max_nodes(N, C) * 4);
}

hipError_t launch_pddp(const PddpArgs& a, int dtype, hipStream_t s) {
  if (dtype == DT_BF16) return a.D == 128 ? run_levels<__bf16, 128>(a, s) : run_levels<__bf16, 64>(a, s);
  return a.D == 128 ? run_levels<float, 128>(a, s) : run_levels<float, 64>(a, s);
}

}  // namespace mcs
