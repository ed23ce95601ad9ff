// Internal launcher interface between the C-ABI layer (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mcs {

enum { DT_F32 = 0, DT_BF16 = 1 };
enum { EPI_PLAIN = 0, EPI_ADD = 1, EPI_RESID = 2 };

// Blocks per XCD per scheduling window of the block-to-XCD mapping (see
// xcd_remap).  Window sizes from 0 to 148 blocks per XCD changed the sparse
// kernel's time by under 2%, so this is a fixed constant, not a tunable.
constexpr int kXcdChunk = 32;

// Attention over query groups of 64 (one wavefront each).
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* perm;  // [H][N] slot -> token, or null (slot == token)
  const int32_t* idx;   // [H][G][kpad] kept keys of each group, or null (all N keys)
  const void* rin;      // EPI_ADD: cached residual; EPI_RESID: dense output
  void* o;              // [H][N][D] output (token order)
  float2* stats;        // optional [H][N] {offset m (log2 units), 1 / sum exp2(s*c - m)}
  float* lse;           // optional [H][N] natural-log logsumexp of scale * q.k
  int H, N, G, nkeys, kpad;
  float c;              // scale * log2(e)
  int xcd_chunk;        // blocks per XCD per window of the block-to-XCD mapping
};
hipError_t launch_attention(const AttnArgs& a, int dtype, int head_dim, bool gather, int epi, bool pv,
                            hipStream_t s);
// bf16 gather-sparse attention over pair-planned lists: groups 2p and 2p+1 share
// the gathers of their first ncommon[h][p] keys (see launch_pair_plan).
hipError_t launch_attention_pairs(const AttnArgs& a, const int32_t* ncommon, int head_dim, int epi,
                                  hipStream_t s);

// Pair plan of kept-key lists: for each pair of groups (2p, 2p+1) of a head,
// rewrite both rows as [common keys | own keys], the common prefix nc a multiple
// of 128 (written to ncommon[h][p]); a lone last group keeps its list (nc = 0).
size_t pair_plan_lds_bytes(int N);
hipError_t launch_pair_plan(const int32_t* idx, int32_t* pidx, int32_t* ncommon, int H, int N, int G, int K, int kpad,
                            hipStream_t s);

// Selection pass 2 with the per-group top-K fused into its epilogue: summed
// normalised probabilities of every key per query group (written to `mass`),
// then the K keys of largest mass per group, ascending, -1 padded to kpad.
constexpr int kMassHistBins = 2048;  // bins of a mass row's histogram (top 11 value bits)
struct MassArgs {
  const void* q;
  const void* k;
  const int32_t* perm;     // [H][N]
  const float2* stats;     // [H][N] row statistics from pass 1 (or null: use lse)
  const float* lse;        // [H][N] natural-log logsumexp (used when stats is null)
  float* mass;             // [hcount][G][ldm] scratch rows
  uint32_t* hist;          // [hcount][G][kMassHistBins] scratch: each row's histogram of its top value bits
  int ldm;                 // row stride of mass: N rounded up to a multiple of 4
  int32_t* idx;            // [H][G][kpad] output
  int h0, hcount, N, G, K, kpad;
  float c;                 // scale * log2(e)
  int xcd_chunk;
};
// Pass 2: the mass rows and their histograms of heads h0 .. h0+hcount-1.
hipError_t launch_group_mass(const MassArgs& a, int dtype, int head_dim, hipStream_t s);
// Exact top-K of those rows into idx (reads the rows and histograms; overwrites the rows).
hipError_t launch_topk(const MassArgs& a, hipStream_t s);

// PDDP grouping.
struct PddpArgs {
  const void* q;        // [H][N][D]
  int32_t* perm;        // [H][N] output
  void* ws;             // workspace (see pddp_workspace_bytes)
  int H, N, D, C, iters;
};
size_t pddp_workspace_bytes(int H, int N, int D, int C);
hipError_t launch_pddp(const PddpArgs& a, int dtype, hipStream_t s);

// Kept-key lists <-> per-group key bitmaps (`rows` = H * G rows of kpad ids /
// ceil(N/32) words).  The encoder holds one row's bitmap in LDS.
size_t keybits_lds_bytes(int N);
hipError_t launch_idx_to_bits(const int32_t* idx, uint32_t* bits, int rows, int N, int K, int kpad, hipStream_t s);
hipError_t launch_bits_to_idx(const uint32_t* bits, int32_t* idx, int rows, int N, int K, int kpad, hipStream_t s);

}  // namespace mcs
