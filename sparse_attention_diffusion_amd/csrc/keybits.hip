// Compact form of the meta-cache's kept-key lists (MC-Sparse summary page,
// residual paragraph: inactive cache entries move to host memory, and the
// residual-plus-index traffic has to hide behind compute).
//
// A group's kept keys are an ascending list of K ids in [0, N) padded with -1 to
// kpad entries.  The same set is a bitmap of W = ceil(N/32) words: bit b of word
// w is set when key 32*w + b is kept.  At density 0.15 of 118,800 tokens that is
// 14.9 KB per group instead of 71.3 KB, so the host copies of an offloaded cache
// entry shrink about 2.8x (the residual then dominates).  Both directions are one
// block per (head, group) and bound by HBM: encode reads the list and writes the
// bitmap, decode reads the bitmap and writes the list.
#include "common.hpp"
#include "kernels.hpp"

namespace mcs {

namespace {

constexpr int kBitsThreads = 256;

// List -> bitmap: the row's bitmap is built in LDS (zeroed, one atomic OR per
// kept key; keys outside [0, N), i.e. the -1 padding, are skipped), then
// written out whole.
__global__ __launch_bounds__(kBitsThreads) void idx_to_bits_kernel(const int32_t* idx, uint32_t* bits, int N, int K,
                                                                     int kpad, int W) {
  extern __shared__ uint32_t wbits[];  // W words
  const size_t row = blockIdx.x;       // h * G + g
  const int32_t* ir = idx + row * (size_t)kpad;
  uint32_t* br = bits + row * (size_t)W;
  for (int w = threadIdx.x; w < W; w += kBitsThreads) wbits[w] = 0u;
  __syncthreads();
  constexpr int U = 16;  // list loads in flight per thread
  for (int j0 = threadIdx.x; j0 < K; j0 += U * kBitsThreads) {
    int key[U];
#pragma unroll
    for (int u = 0; u < U; ++u) key[u] = j0 + u * kBitsThreads < K ? ir[j0 + u * kBitsThreads] : -1;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (key[u] >= 0 && key[u] < N) atomicOr(&wbits[key[u] >> 5], 1u << (key[u] & 31));
  }
  __syncthreads();
  for (int w = threadIdx.x; w < W; w += kBitsThreads) br[w] = wbits[w];
}

// Inclusive prefix sum of x over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

constexpr int kDecWaves = kBitsThreads / 64;
constexpr int kDecChunk = kBitsThreads;  // words per chunk: one per thread
constexpr int kDecRegs = 8;              // chunks whose words are loaded at once
constexpr int kDecStage = 64 * 32;       // keys one wave's 64 words can hold

// Bitmap -> list.  The words are read 8 chunks of 256 at a time (one word per
// thread and chunk, coalesced), all loads issued before any key is written, so
// that the list stores never hold up a load.  Each wave scans its lanes' bit
// counts for all 8 chunks and publishes its 8 totals in LDS; after one barrier
// every wave knows where the keys of each of its chunks start in the list
// (running total over chunks, then over the waves before it).  Per chunk, each
// lane expands its word's keys into the wave's LDS staging area at its scanned
// position, and the wave copies that contiguous run of keys out with consecutive
// lanes (coalesced stores).  Keys past the K-th are dropped (a chunk starting at
// or past K is skipped), bits at or past N in the last word are ignored, and
// positions from min(total, K) to kpad get -1.
__global__ __launch_bounds__(kBitsThreads) void bits_to_idx_kernel(const uint32_t* bits, int32_t* idx, int N, int K,
                                                                     int kpad, int W) {
  __shared__ uint32_t wtot[kDecRegs][kDecWaves];
  __shared__ int32_t stage[kDecWaves][kDecStage];
  const size_t row = blockIdx.x;
  const uint32_t* br = bits + row * (size_t)W;
  int32_t* ir = idx + row * (size_t)kpad;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t tail = (N & 31) ? ((1u << (N & 31)) - 1u) : 0xffffffffu;  // valid bits of the last word
  int32_t* st = stage[wid];
  const auto rsrc = make_rsrc(br, (uint32_t)W * 4u);  // words past the row read as 0
  uint32_t done = 0;  // keys of the words before w0 (the same in every thread)
  for (int w0 = 0; w0 < W && done < (uint32_t)K; w0 += kDecRegs * kDecChunk) {
    uint32_t wr[kDecRegs], excl[kDecRegs];
#pragma unroll
    for (int r = 0; r < kDecRegs; ++r) wr[r] = bload32(rsrc, (uint32_t)(w0 + r * kDecChunk + (int)threadIdx.x) * 4u);
#pragma unroll
    for (int r = 0; r < kDecRegs; ++r) {
      const int w = w0 + r * kDecChunk + (int)threadIdx.x;
      if (w == W - 1) wr[r] &= tail;
      const uint32_t cnt = (uint32_t)__builtin_popcount(wr[r]);
      const uint32_t incl = wave_incl_scan(cnt);
      excl[r] = incl - cnt;
      if (lane == 63) wtot[r][wid] = incl;
    }
    __syncthreads();
    uint32_t run = done;  // keys before chunk r
#pragma unroll
    for (int r = 0; r < kDecRegs; ++r) {
      uint32_t before = 0, total = 0;
#pragma unroll
      for (int v = 0; v < kDecWaves; ++v) {
        const uint32_t t = wtot[r][v];
        if (v < wid) before += t;
        total += t;
      }
      const uint32_t base = run + before;  // this wave's first position in chunk r
      run += total;
      if (base >= (uint32_t)K) continue;   // the same in every lane of the wave
      const int w = w0 + r * kDecChunk + (int)threadIdx.x;
      uint32_t b = wr[r], p = excl[r];
      while (b) {
        st[p++] = 32 * w + __builtin_ctz(b);
        b &= b - 1u;
      }
      // the staging writes of every lane must land before the wave reads them back
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      const uint32_t mine = wtot[r][wid];  // this wave's key count
      for (uint32_t j = lane; j < mine; j += 64) {
        if (base + j < (uint32_t)K) ir[base + j] = st[j];
      }
      // and the reads must be done before the next chunk's writes
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    done = run;
    __syncthreads();  // wtot is rewritten by the next 8 chunks
  }
  const int first_pad = (int)min(done, (uint32_t)K);
  for (int j = first_pad + (int)threadIdx.x; j < kpad; j += kBitsThreads) ir[j] = -1;
}

}  // namespace

size_t keybits_lds_bytes(int N) { return (size_t)((N + 31) / 32) * sizeof(uint32_t); }

hipError_t launch_idx_to_bits(const int32_t* idx, uint32_t* bits, int rows, int N, int K, int kpad,
                              hipStream_t s) {
  const int W = (N + 31) / 32;
  const size_t lds = keybits_lds_bytes(N);
  hipError_t e = hipFuncSetAttribute((const void*)idx_to_bits_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(idx_to_bits_kernel, dim3((unsigned)rows), dim3(kBitsThreads), lds, s, idx, bits, N, K, kpad, W);
  return hipGetLastError();
}

hipError_t launch_bits_to_idx(const uint32_t* bits, int32_t* idx, int rows, int N, int K, int kpad,
                              hipStream_t s) {
  const int W = (N + 31) / 32;
  hipLaunchKernelGGL(bits_to_idx_kernel, dim3((unsigned)rows), dim3(kBitsThreads), 0, s, bits, idx, N, K, kpad, W);
  return hipGetLastError();
}

}  // namespace mcs
