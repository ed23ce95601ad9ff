// Vanilla block-sparse selection, the baseline the matched-density comparison
// measures MC-Sparse against (MC-Sparse summary page, block-sparsity paragraph:
// training-free systems cut Q and K into tile blocks and score them by their
// mean-pooled vectors).  Blocks are runs of C = 64 consecutive token ids, so the
// query blocks are the groups of an identity perm and the selection is a list of
// whole key blocks per query block, expanded to ascending key ids: the same idx
// layout as the token-level selection, consumed by the same gather kernel.
//
//   1. block means: mq[h][b] = mean of Q rows 64b .. 64b+63, mk likewise (fp32);
//   2. per (head, query block b): score_j = scale * mq[b] . mk[j] for every key
//      block j (fp32), the kb = K / 64 blocks of highest score (ties to the lower
//      block id), expanded ascending.
// Both are small next to attention: the means read Q and K once (HBM-bound),
// the scores are 2 G^2 D flops per head.
#include "blocksel.hpp"
#include "common.hpp"

namespace mcs {

namespace {

constexpr int kMeanThreads = 128;
constexpr int kSelThreads = 256;

// One block per (head, block, tensor): thread t sums dimension t (and t + 128
// for wider rows) over the 64 rows of the block.
template <typename T>
__global__ __launch_bounds__(kMeanThreads) void block_means_kernel(const T* q, const T* k, float* mq, float* mk,
                                                                    int N, int D) {
  const int G = N / 64;
  const int hb = blockIdx.x;  // h * G + b
  const int h = hb / G, b = hb - h * G;
  const T* src = (blockIdx.y == 0 ? q : k) + ((size_t)h * N + (size_t)b * 64) * D;
  float* dst = (blockIdx.y == 0 ? mq : mk) + (size_t)hb * D;
  for (int c = threadIdx.x; c < D; c += kMeanThreads) {
    float acc = 0.0f;
#pragma unroll 8
    for (int r = 0; r < 64; ++r) acc += (float)src[(size_t)r * D + c];
    dst[c] = acc * (1.0f / 64.0f);
  }
}

// Descending score, then ascending block id, as one ascending 64-bit key.
__device__ __forceinline__ uint64_t score_key(float s, int j) {
  return ((uint64_t)(~float_key(s)) << 32) | (uint32_t)j;
}

// One block per (head, query block).  LDS: the query block's mean, the G sort
// keys padded to a power of two, and one flag per key block.
__global__ __launch_bounds__(kSelThreads) void block_topk_kernel(const float* mq, const float* mk, int32_t* idx,
                                                                  int N, int D, int kb, int kpad, float scale,
                                                                  int gpow) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int G = N / 64;
  const int hb = blockIdx.x;
  const int h = hb / G;
  float* qm = (float*)smem;                                   // D floats
  uint64_t* keys = (uint64_t*)(smem + ((D * 4 + 15) & ~15));  // gpow keys
  uint32_t* flag = (uint32_t*)(keys + gpow);                  // G flags, then 4 wave totals
  uint32_t* tot = flag + G;
  const int t = threadIdx.x;
  for (int c = t; c < D; c += kSelThreads) qm[c] = mq[(size_t)hb * D + c];
  for (int j = t; j < G; j += kSelThreads) flag[j] = 0u;
  __syncthreads();
  const float* kh = mk + (size_t)h * G * D;
  for (int j = t; j < gpow; j += kSelThreads) {
    uint64_t key = ~(uint64_t)0;
    if (j < G) {
      const float* kr = kh + (size_t)j * D;
      float s = 0.0f;
      for (int c = 0; c < D; ++c) s = __builtin_fmaf(qm[c], kr[c], s);
      key = score_key(s * scale, j);
    }
    keys[j] = key;
  }
  __syncthreads();
  // bitonic sort, ascending
  for (int size = 2; size <= gpow; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = t; i < gpow; i += kSelThreads) {
        const int p = i ^ stride;
        if (p > i) {
          const uint64_t a = keys[i], c = keys[p];
          const bool up = (i & size) == 0;
          if ((a > c) == up) {
            keys[i] = c;
            keys[p] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int r = t; r < kb; r += kSelThreads) flag[(int)(uint32_t)keys[r]] = 1u;
  __syncthreads();
  // position of each kept block among the kept blocks (ascending id): block
  // scan over contiguous runs of flags, one run per thread
  const int run = (G + kSelThreads - 1) / kSelThreads;
  const int j0 = min(G, t * run), j1 = min(G, j0 + run);
  uint32_t cnt = 0;
  for (int j = j0; j < j1; ++j) cnt += flag[j];
  const int lane = t & 63, wid = t >> 6;
  uint32_t incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) tot[wid] = incl;
  __syncthreads();
  uint32_t pos = incl - cnt;
  for (int v = 0; v < wid; ++v) pos += tot[v];
  int32_t* row = idx + (size_t)hb * kpad;
  for (int j = j0; j < j1; ++j) {
    if (flag[j]) {
      for (int e = 0; e < 64; ++e) row[pos * 64 + e] = j * 64 + e;
      ++pos;
    }
  }
  for (int e = kb * 64 + t; e < kpad; e += kSelThreads) row[e] = -1;
}

int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

size_t topk_lds(int N, int D) {
  const int G = N / 64;
  return (size_t)((D * 4 + 15) & ~15) + (size_t)pow2_at_least(G) * 8 + (size_t)G * 4 + 16;
}

}  // namespace

size_t block_select_ws_bytes(int H, int N, int D) { return (size_t)2 * H * (N / 64) * D * sizeof(float); }

bool block_select_fits(int N, int D) { return topk_lds(N, D) <= 160u * 1024u; }

hipError_t launch_block_select(const void* q, const void* k, int dtype, int H, int N, int D, int kb, int kpad,
                               float scale, int32_t* idx, void* ws, hipStream_t s) {
  const int G = N / 64;
  float* mq = (float*)ws;
  float* mk = mq + (size_t)H * G * D;
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(block_means_kernel<__bf16>, dim3((unsigned)(H * G), 2), dim3(kMeanThreads), 0, s,
                       (const __bf16*)q, (const __bf16*)k, mq, mk, N, D);
  else
    hipLaunchKernelGGL(block_means_kernel<float>, dim3((unsigned)(H * G), 2), dim3(kMeanThreads), 0, s,
                       (const float*)q, (const float*)k, mq, mk, N, D);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = topk_lds(N, D);
  e = hipFuncSetAttribute((const void*)block_topk_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(block_topk_kernel, dim3((unsigned)(H * G)), dim3(kSelThreads), lds, s, mq, mk, idx, N, D, kb,
                     kpad, scale, pow2_at_least(G));
  return hipGetLastError();
}

}  // namespace mcs
