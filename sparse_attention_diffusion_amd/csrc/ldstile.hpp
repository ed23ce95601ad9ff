// LDS staging of 32-row K/V tiles for the bf16 kernels of the MC-Sparse hot
// path on gfx950 (shared by attention and the selection pass).
//
// Fetching a K row straight into the MFMA operand layout puts a different row in
// every lane of a quad, which costs the texture-address unit four cycles per
// quad.  Instead a step's 32 rows are copied global -> LDS with
// buffer_load ... lds, each lane quad reading 64 contiguous bytes of one row (one
// cycle per quad), and the MFMA operands are read from LDS.
//
// Tile geometry (one tile = the 32 rows of one step):
//   a copy instruction moves 1 KiB = RPI rows; lane j of instruction i fetches
//   16-byte chunk (j % LPR) ^ swz(g) of step entry NI*g + i, g = j / LPR, and it
//   lands at LDS offset i*BLK + 16*j.  So entry e sits in block e % NI, row
//   e / NI, and its chunk x at position x ^ swz(e / NI).  The 32-byte skew
//   between blocks and the XOR swizzle inside 64-byte groups spread the rows a
//   ds_read touches together over the LDS banks; the swizzle never leaves a
//   64-byte group, so a quad still reads one contiguous 64-byte piece.
#pragma once

#include "common.hpp"

namespace mcs {

#define LDSP __attribute__((address_space(3)))

template <int D>
struct LT {
  static constexpr int ROWB = D * 2;
  static constexpr int LPR = ROWB / 16;   // lanes per row in a DMA
  static constexpr int RPI = 64 / LPR;    // rows per DMA instruction
  static constexpr int NI = 32 / RPI;     // DMA instructions per tile
  static constexpr int BLK = 1024 + 32;
  static constexpr int TILE = NI * BLK;
  static constexpr int KCH = D / 16;      // QK k-chunks of 16 dims
  static constexpr int VT = D / 32;       // PV output tiles of 32 dims
  // epilogue: half of the group's O (32 queries, fp32) with a 16-byte row skew
  static constexpr int OPITCH = D * 4 + 16;
  static constexpr int STAGE = (2 * TILE > 32 * OPITCH) ? 2 * TILE : 32 * OPITCH;
  __device__ static int swz(int g) { return (g * ROWB / 256) & 3; }
  __device__ static int off(int e, int x) { return (e % NI) * BLK + (e / NI) * ROWB + 16 * (x ^ swz(e / NI)); }
};


// Explicit wait on the vector memory counter.  The compiler's own tracking of
// the LDS copies is not relied on: across a loop back-edge it has been seen to
// drop the wait a stage read needs.  Loads retire in order, so vmcnt(n) means
// "everything but the last n vector memory instructions has landed".
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Block barrier without the memory fence of __syncthreads(): that fence waits for
// every outstanding global store (vmcnt(0)), which would expose a store's write
// latency at every step.  Shared tiles need no fence: each wave waits for its
// own copies (wait_vm) before the barrier, and its reads of the previous tile
// were consumed before it arrives.  The "memory" clobber keeps the compiler from
// moving LDS accesses across the barrier.
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Lane constants of the tile copies: the byte offset of this lane's 16-byte
// chunk within a row, and the first step entry this lane copies.
template <int D>
__device__ __forceinline__ uint32_t tile_goff(int lane) {
  using L = LT<D>;
  return 16u * (uint32_t)((lane % L::LPR) ^ L::swz(lane / L::LPR));
}
template <int D>
__device__ __forceinline__ int tile_ebase(int lane) {
  return LT<D>::NI * (lane / LT<D>::LPR);
}

// Byte offsets (within a tile) of the MFMA operand chunks of lane row m = lm:
// chunk 2*ks + hf of entry lm is at kaddr[ks & 1] + 64*(ks >> 1).
template <int D>
__device__ __forceinline__ void tile_kaddr(int (&kaddr)[2], int lm, int hf) {
#pragma unroll
  for (int v = 0; v < 2; ++v) kaddr[v] = LT<D>::off(lm, 2 * v + hf);
}

template <int D>
__device__ __forceinline__ void tile_kread(u32x4 (&ka)[LT<D>::KCH], const LDSP char* tile, const int (&kaddr)[2]) {
#pragma unroll
  for (int ks = 0; ks < LT<D>::KCH; ++ks) ka[ks] = *(const LDSP u32x4*)(tile + kaddr[ks & 1] + 64 * (ks >> 1));
}

// Copy instructions i0 .. i0+NCOPY-1 of the tile of keys step*32 + e (a dense
// key list).  Keys past the buffer read as zeros.
template <int D, int NCOPY>
__device__ __forceinline__ void tile_copy_dense(LDSP char* tile, __amdgpu_buffer_rsrc_t r, int step, int ebase,
                                                uint32_t goff, int i0) {
  using L = LT<D>;
  const uint32_t base = (uint32_t)(step * 32 + ebase + i0) * (uint32_t)L::ROWB + goff;
#pragma unroll
  for (int j = 0; j < NCOPY; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDSP void*)(tile + (i0 + j) * L::BLK), 16, base + j * L::ROWB, 0, 0,
                                             0);
}

}  // namespace mcs
