// Pair plan of the kept-key lists (gather sharing between neighbouring groups).
//
// Groups 2p and 2p+1 of a head are adjacent leaves of the PDDP tree, i.e. two
// sets of similar queries (MC-Sparse summary page, grouping paragraph), and the
// key sets the selection keeps for them overlap.  The paired attention kernel
// gathers a row both groups keep once for both, so the plan rewrites each pair's
// two rows as
//   [ the nc lowest keys common to both groups, ascending | the group's other keys, ascending ]
// with nc = 128 * floor(|common| / 128) (whole macro-steps of the kernel), and
// stores nc per pair.  Each row still holds exactly its group's kept set, so any
// consumer that treats a row as a set (the plain gather kernel, the oracle) sees
// the same selection.  A lone last group (odd G) keeps its list, nc = 0.
//
// One block per pair: both rows become bitmaps in LDS (one atomic OR per kept
// key), a block scan of the common-bit counts fixes nc and which common bits are
// shared, three more scans place each word's keys, and every thread writes the
// keys of its contiguous run of words.  Both rows are read in full before either
// is written, so the plan may be built in place (pidx == idx).
#include "common.hpp"
#include "kernels.hpp"

namespace mcs {

namespace {

constexpr int kPlanThreads = 256;
constexpr int kPlanWaves = kPlanThreads / 64;

__device__ __forceinline__ uint32_t incl_scan64(uint32_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// Exclusive prefix sum of x over the block (thread order) and the block total.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* tot, uint32_t& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t incl = incl_scan64(x);
  if (lane == 63) tot[wid] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int v = 0; v < kPlanWaves; ++v) {
    const uint32_t t = tot[v];
    if (v < wid) before += t;
    all += t;
  }
  __syncthreads();  // tot is rewritten by the next scan
  total = all;
  return before + incl - x;
}

// The bits of word cm whose rank among all common bits (cum of them come before
// this word) is below nc.
__device__ __forceinline__ uint32_t take_low(uint32_t cm, uint32_t cum, uint32_t nc) {
  if (cum >= nc) return 0u;
  const uint32_t cnt = (uint32_t)__builtin_popcount(cm);
  if (cum + cnt <= nc) return cm;
  uint32_t r = nc - cum, out = 0u;
  while (r--) {
    const uint32_t low = cm & (0u - cm);
    out |= low;
    cm ^= low;
  }
  return out;
}

__device__ __forceinline__ void emit(int32_t* row, uint32_t& pos, uint32_t bits, int w) {
  while (bits) {
    row[pos++] = 32 * w + __builtin_ctz(bits);
    bits &= bits - 1u;
  }
}

__global__ __launch_bounds__(kPlanThreads) void pair_plan_kernel(const int32_t* idx, int32_t* pidx, int32_t* ncommon,
                                                                  int N, int G, int K, int kpad, int W) {
  extern __shared__ uint32_t bm[];  // 2 * W words: the bitmap of group 2p, then of group 2p+1
  __shared__ uint32_t tot[kPlanWaves];
  const int P = (G + 1) / 2;
  const int h = blockIdx.x / P, p = blockIdx.x - h * P;
  const int t = threadIdx.x;
  const int32_t* ra = idx + ((size_t)h * G + 2 * p) * kpad;
  int32_t* oa = pidx + ((size_t)h * G + 2 * p) * kpad;
  if (2 * p + 1 >= G) {
    if (oa != ra)
      for (int j = t; j < kpad; j += kPlanThreads) oa[j] = ra[j];
    if (t == 0) ncommon[(size_t)h * P + p] = 0;
    return;
  }
  const int32_t* rb = ra + kpad;
  int32_t* ob = oa + kpad;
  uint32_t* A = bm;
  uint32_t* B = bm + W;
  for (int w = t; w < 2 * W; w += kPlanThreads) bm[w] = 0u;
  __syncthreads();
  for (int j = t; j < K; j += kPlanThreads) {
    const int ka = ra[j], kb = rb[j];
    if (ka >= 0 && ka < N) atomicOr(&A[ka >> 5], 1u << (ka & 31));
    if (kb >= 0 && kb < N) atomicOr(&B[kb >> 5], 1u << (kb & 31));
  }
  __syncthreads();
  // thread t owns words [w0, w1)
  const int cw = (W + kPlanThreads - 1) / kPlanThreads;
  const int w0 = min(W, t * cw), w1 = min(W, w0 + cw);
  uint32_t c = 0;
  for (int w = w0; w < w1; ++w) c += (uint32_t)__builtin_popcount(A[w] & B[w]);
  uint32_t ctot;
  const uint32_t cbefore = block_excl_scan(c, tot, ctot);
  const uint32_t nc = ctot / 128u * 128u;
  uint32_t na = 0, nb = 0, nsh = 0;
  {
    uint32_t cum = cbefore;
    for (int w = w0; w < w1; ++w) {
      const uint32_t cm = A[w] & B[w];
      const uint32_t sh = take_low(cm, cum, nc);
      cum += (uint32_t)__builtin_popcount(cm);
      nsh += (uint32_t)__builtin_popcount(sh);
      na += (uint32_t)__builtin_popcount(A[w] & ~sh);
      nb += (uint32_t)__builtin_popcount(B[w] & ~sh);
    }
  }
  uint32_t stot, atot, btot;
  const uint32_t sb = block_excl_scan(nsh, tot, stot);
  const uint32_t ab = block_excl_scan(na, tot, atot);
  const uint32_t bb = block_excl_scan(nb, tot, btot);
  {
    uint32_t cum = cbefore, ps = sb, psb = sb, pa = nc + ab, pb = nc + bb;
    for (int w = w0; w < w1; ++w) {
      const uint32_t cm = A[w] & B[w];
      const uint32_t sh = take_low(cm, cum, nc);
      cum += (uint32_t)__builtin_popcount(cm);
      emit(oa, ps, sh, w);
      emit(ob, psb, sh, w);
      emit(oa, pa, A[w] & ~sh, w);
      emit(ob, pb, B[w] & ~sh, w);
    }
  }
  for (uint32_t j = nc + atot + t; j < (uint32_t)kpad; j += kPlanThreads) oa[j] = -1;
  for (uint32_t j = nc + btot + t; j < (uint32_t)kpad; j += kPlanThreads) ob[j] = -1;
  if (t == 0) ncommon[(size_t)h * P + p] = (int32_t)nc;
}

}  // namespace

size_t pair_plan_lds_bytes(int N) { return (size_t)2 * ((N + 31) / 32) * sizeof(uint32_t); }

hipError_t launch_pair_plan(const int32_t* idx, int32_t* pidx, int32_t* ncommon, int H, int N, int G, int K, int kpad,
                            hipStream_t s) {
  const int W = (N + 31) / 32;
  const size_t lds = pair_plan_lds_bytes(N);
  hipError_t e =
      hipFuncSetAttribute((const void*)pair_plan_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int blocks = H * ((G + 1) / 2);
  hipLaunchKernelGGL(pair_plan_kernel, dim3((unsigned)blocks), dim3(kPlanThreads), lds, s, idx, pidx, ncommon, N, G,
                     K, kpad, W);
  return hipGetLastError();
}

}  // namespace mcs
