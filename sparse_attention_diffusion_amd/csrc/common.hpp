// Device helpers shared by the MC-Sparse HIP kernels (gfx950 / CDNA4 only).
//
// Wave size is 64.  Matrix work uses the CDNA4 MFMA builtins:
//   v_mfma_f32_32x32x16_bf16 : A 32x16, B 16x32, C 32x32 (8 bf16 per lane per operand)
//   v_mfma_f32_32x32x2_f32   : A 32x2,  B 2x32,  C 32x32 (1 fp32 per lane per operand)
// For both, lane l supplies A[row = l%32][k = (l/32)*kw + t] and B[k = (l/32)*kw + t][col = l%32];
// accumulator register r of lane l holds C[row = 8*(r/4) + 4*(l/32) + r%4][col = l%32].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mcs {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kNumXcd = 8;

// Raw buffer descriptor over [base, base + bytes); out-of-range loads return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 bload64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bload32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Index of this wavefront in its workgroup, as a wave-uniform (scalar) value so
// that everything derived from it (head, group, buffer descriptors) stays in SGPRs.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Pack two floats into a dword of two bf16 (round to nearest even), lo first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// v_permlane32_swap exchanges the upper half of one register with the lower half of
// another.  Fed the same value twice, the two results hold {x[l%32], x[l%32+32]} in
// every lane (which of the two comes first does not matter for max / sum), so one
// instruction combines the two wave halves.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // IEEE addition is commutative, so both halves get the same bits
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Read `x` from lane `src` (0..63) of the wave.
__device__ __forceinline__ float lane_read(float x, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
}
__device__ __forceinline__ int lane_read_i(int x, int src) {
  return __builtin_amdgcn_ds_bpermute(src << 2, x);
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Workgroups are dealt round-robin to the 8 XCDs (each with its own 4 MB L2), and
// all XCDs share the MALL.  Map hardware block b (XCD b % 8, local slot b / 8) so
// that each XCD runs `chunk` consecutive logical blocks at a time while the 8 XCDs
// together sweep one window of 8*chunk consecutive blocks: neighbouring query
// groups (which pick overlapping keys) share an L2, and the blocks in flight
// across the chip stay within about one head's K/V (MALL-resident).  The last
// partial window keeps the identity mapping.  Returns -1 for padding blocks.
__device__ __forceinline__ int xcd_remap(int hw_block, int n_logical, int chunk) {
  if (hw_block >= n_logical) return -1;
  if (chunk <= 0) return hw_block;
  const int window = kNumXcd * chunk;
  const int full = (n_logical / window) * window;
  if (hw_block >= full) return hw_block;
  const int x = hw_block % kNumXcd, j = hw_block / kNumXcd;
  return (j / chunk) * window + x * chunk + (j % chunk);
}
inline int xcd_grid(int n_logical) { return n_logical; }

// Order-preserving map of a float onto uint32 (ascending floats -> ascending keys).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

}  // namespace mcs
