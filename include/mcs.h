/*
 * mcs.h - C ABI of the MC-Sparse hot path on AMD Instinct MI355X (gfx950).
 *
 * MC-Sparse ("MC-Sparse: Deconstructing and Closing the Dense-Sparse Attention
 * Gap in Diffusion Transformers", summary page of arXiv 2610.06801) replaces a
 * DiT attention call by meta-cached token-level sparse attention:
 *   - anchor step: group the queries into PDDP groups of exactly C, select per
 *     group the K keys of largest summed softmax mass (two-pass exact top-K),
 *     run dense attention and cache the dense-minus-sparse output residual;
 *   - reuse step: run gather-sparse attention on the current Q/K/V with the
 *     cached groups and indices and add the cached residual.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors live in device memory, row-major, batch folded into heads:
 *   q, k, v, o, resid : [H][N][D], element type d->dtype (fp32 or bf16)
 *   perm              : int32 [H][N]; perm[h][s] is the token held by slot s.
 *                       Group g of head h is slots [g*C, min((g+1)*C, N)).
 *                       An entry outside [0, N) marks an empty slot: selection
 *                       gives it no weight and attention writes no output for
 *                       it (so a perm holding one token per group makes
 *                       mcs_select a per-query top-K for those tokens).
 *   idx               : int32 [H][G][kpad], G = ceil(N/C); row (h, g) lists
 *                       the K kept key ids of group g in ascending order, then
 *                       kpad - K entries of -1.
 *   lse               : fp32 [H][N] natural-log logsumexp of scale * q_i . k_j
 *                       over all keys, indexed by token.
 * Logits are scale * q . k (q and k are stored unscaled).
 * q, k, v, o, resid must be 16-byte aligned; perm, idx, lse 4-byte aligned.
 *
 * Ownership: the caller allocates every buffer (device memory; pinned host
 * memory for mcs_copy_async).  The library allocates nothing, keeps no pointer
 * after a call returns and has no global state except a per-thread error string.
 * All compute entry points are asynchronous on `stream`: buffers must stay valid
 * until the stream has executed the work.  Calls on different streams that share
 * output or workspace buffers race.
 *
 * Errors: every function returns MCS_OK or a negative code.  Arguments are
 * validated on the host before anything is enqueued (MCS_EINVAL,
 * MCS_EUNSUPPORTED, MCS_EWORKSPACE); a launch failure returns MCS_EHIP.  Faults
 * inside kernels surface asynchronously at the caller's next synchronisation.
 * mcs_last_error() describes the last failure on the calling thread.
 */
#ifndef MCS_H
#define MCS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MCS_ABI_VERSION 1

enum mcs_status {
  MCS_OK = 0,
  MCS_EINVAL = -1,       /* null / misaligned pointer, inconsistent or out-of-range sizes */
  MCS_EUNSUPPORTED = -2, /* C != 64, D not in {64, 128}, unknown dtype */
  MCS_EWORKSPACE = -3,   /* workspace missing or smaller than the minimum */
  MCS_EHIP = -4          /* a HIP launch or copy failed; see mcs_last_error() */
};

enum mcs_dtype { MCS_F32 = 0, MCS_BF16 = 1 };

enum mcs_op { MCS_OP_GROUP = 1, MCS_OP_SELECT = 2, MCS_OP_ANCHOR = 3, MCS_OP_BLOCK_SELECT = 4 };

enum mcs_copy_kind { MCS_COPY_H2D = 1, MCS_COPY_D2H = 2, MCS_COPY_D2D = 3 };

typedef struct mcs_dims {
  int32_t heads;       /* H >= 1: independent heads (batch folded in) */
  int32_t n;           /* N >= 1: tokens per head; N * D * elemsize < 2^31 bytes */
  int32_t head_dim;    /* D: 64 or 128 */
  int32_t group;       /* C: queries per group; must be 64 (one MFMA tile) */
  int32_t topk;        /* K: kept keys per group, 1 <= K <= N */
  int32_t kpad;        /* row stride of idx; kpad >= K and a multiple of 32 */
  int32_t dtype;       /* MCS_F32 or MCS_BF16: type of q, k, v, o, resid */
  int32_t power_iters; /* PDDP power-iteration steps, 1..1024 (32 recommended) */
  float scale;         /* softmax scale, > 0 (1/sqrt(D) for standard attention) */
} mcs_dims;

/* MCS_ABI_VERSION of the loaded library. */
int32_t mcs_abi_version(void);

/* Message of the last failed call on this thread ("" if none). Never NULL. */
const char* mcs_last_error(void);

/* Workspace needed by op (MCS_OP_GROUP / SELECT / ANCHOR / BLOCK_SELECT) when up to
 * heads_per_pass heads of the selection mass are processed at once
 * (0 = all heads).  The selection stores one fp32 mass row of N entries and an
 * 8 KB histogram per group for each head of a pass, so heads_per_pass bounds
 * the memory.  Any
 * workspace at least as large as the heads_per_pass = 1 figure is accepted by
 * the calls below; larger ones process more heads per pass. */
int mcs_workspace_bytes(const mcs_dims* d, int32_t op, int32_t heads_per_pass, size_t* bytes);

/* PDDP grouping (summary page, grouping paragraph): for every head, split the
 * queries recursively - centre the node, take its principal direction by
 * d->power_iters power steps from ones/sqrt(D), order the node by (projection,
 * token id) and give the left child floor(g/2)*C queries, g = ceil(n/C) - until
 * each node holds one group.  Writes perm (leaves in depth-first, left-first
 * order): every group has exactly C queries except the last, which has N mod C
 * when C does not divide N.  Reads q only.  Needs workspace (op GROUP). */
int mcs_group(const mcs_dims* d, const void* q, int32_t* perm, void* ws, size_t ws_bytes, hipStream_t stream);

/* Two-pass exact top-K selection (summary page, selection paragraph).  Pass 1
 * (skipped when lse is non-NULL) computes each query's logsumexp; pass 2 sums,
 * for every key j, the softmax probabilities exp(scale*q_i.k_j - lse_i) over the
 * queries i of each group of perm; each group keeps the K keys of largest
 * summed mass (ties to the lower key id) in ascending order, -1 padded to kpad.
 * Writes idx.  Needs workspace (op SELECT). */
int mcs_select(const mcs_dims* d, const void* q, const void* k, const int32_t* perm, const float* lse,
               int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream);

/* mcs_select without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same result as mcs_select (bit for bit); the row
 * statistics and mass rows live in a static device array of MCS_SCRATCH_BYTES
 * that each GPU the library runs on holds until the process ends.  Processes
 * ceil(H / hpp) passes of hpp heads, hpp as large as the scratch allows.
 * Workloads needing more than MCS_SCRATCH_BYTES for one head (8*H*N bytes of
 * statistics plus about N*N/16 of mass rows and N/8 KB of histograms, padded)
 * are rejected with
 * MCS_EUNSUPPORTED before any HIP call.  The scratch belongs to the current
 * device (hipSetDevice), which must be the device of `stream` and of every
 * buffer.  Every call on one GPU shares that GPU's scratch: calls that overlap
 * in time on one GPU (other streams, other threads) race.  Allocates nothing:
 * no hipMalloc, hipFree or allocating library routine. */
#define MCS_SCRATCH_BYTES ((size_t)128 << 20)
int mcs_select_noalloc(const mcs_dims* d, const void* q, const void* k, const int32_t* perm, const float* lse,
                       int32_t* idx, hipStream_t stream);

/* Dense softmax attention (summary page, limitations paragraph: anchors run full
 * attention): o[h][i] = sum_j softmax_j(scale*q_i.k_j) v[h][j].  Writes o and,
 * when lse is non-NULL, the row logsumexp. */
int mcs_dense_attn(const mcs_dims* d, const void* q, const void* k, const void* v, void* o, float* lse,
                   hipStream_t stream);

/* Gather-sparse attention (summary page, grouping paragraph): every query of
 * group g attends, with a softmax renormalised over the kept keys, to the K keys
 * listed in idx[h][g]; K/V rows are gathered by index.  Output rows are written
 * in token order.  With resid_add non-NULL the result plus resid_add[h][i] is
 * written (residual paragraph: a reuse step adds the cached residual). */
int mcs_sparse_attn(const mcs_dims* d, const void* q, const void* k, const void* v, const int32_t* perm,
                    const int32_t* idx, const void* resid_add, void* o, hipStream_t stream);

/* Anchor step (summary page, residual paragraph): perm = PDDP(q); o_dense =
 * dense attention (with its logsumexp); idx = top-K selection on perm reusing
 * the dense pass's row statistics; resid = o_dense - sparse attention(perm,
 * idx).  The anchor's attention output is o_dense.  lse may be NULL.  Needs
 * workspace: with at least the op ANCHOR figure for heads_per_pass 1 (the
 * grouping's and the selection's regions side by side), grouping runs on a
 * library-owned side stream of the current device (default priority, created on
 * first use, kept until the process ends) beside dense attention, forked from
 * and joined back into `stream` with events before selection; with less, but
 * at least max(op GROUP, op SELECT with heads_per_pass 1), the steps run in
 * turn on `stream`.  Both give the same bits. */
int mcs_anchor(const mcs_dims* d, const void* q, const void* k, const void* v, int32_t* perm, int32_t* idx,
               void* resid, void* o_dense, float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/* Residual of a supplied selection (summary page, residual paragraph: the
 * residual is the dense output minus the sparse output on the same step):
 * resid = o_dense - gather-sparse attention of q/k/v with perm and idx as for
 * mcs_sparse_attn, formed in fp32 and rounded once to d->dtype.  o_dense is the
 * dense output of the same q/k/v (mcs_dense_attn), read-only; resid may not
 * alias it.  mcs_anchor forms its residual the same way with its own perm and
 * idx; this entry point serves selections made elsewhere (for example block
 * selections, mcs_block_select with an identity perm). */
int mcs_residual(const mcs_dims* d, const void* q, const void* k, const void* v, const int32_t* perm,
                 const int32_t* idx, const void* o_dense, void* resid, hipStream_t stream);

/* Reuse step (summary page, selection and residual paragraphs): o = sparse
 * attention of the current q/k/v with the cached perm and idx, plus the cached
 * resid.  No regrouping, no reselection. */
int mcs_reuse(const mcs_dims* d, const void* q, const void* k, const void* v, const int32_t* perm,
              const int32_t* idx, const void* resid, void* o, hipStream_t stream);

/* Compact kept-key sets for the meta-cache (summary page, residual paragraph:
 * the residual-plus-index traffic of offloaded entries must hide behind
 * compute).  bits: uint32 [H][G][W], W = ceil(N/32); bit b of word w of row
 * (h, g) is set when key 32*w + b is in that group's kept set.  About N/8 bytes
 * per group instead of 4*kpad.
 *
 * mcs_idx_to_bits: encode idx (the first K entries of every row; entries
 * outside [0, N) are ignored) into bits.  Every word of bits is written.
 * mcs_bits_to_idx: decode bits into idx: the set bits of each row as ascending
 * key ids, then -1 up to kpad.  A row with more than K set bits keeps its K
 * lowest keys; one with fewer is -1 padded from its last key on (a bitmap from
 * mcs_idx_to_bits of a list with K distinct keys has exactly K).
 * Both: d gives heads, n, group (64), topk and kpad as for idx; head_dim,
 * dtype and scale must hold valid values but are not used.  N <=
 * MCS_BITS_MAX_N (MCS_EUNSUPPORTED otherwise); idx and bits 4-byte aligned;
 * bounded by HBM bandwidth. */
#define MCS_BITS_MAX_N (1 << 20)
int mcs_idx_to_bits(const mcs_dims* d, const int32_t* idx, uint32_t* bits, hipStream_t stream);
int mcs_bits_to_idx(const mcs_dims* d, const uint32_t* bits, int32_t* idx, hipStream_t stream);

/* Matched-density comparison (summary page, block-sparsity and gap
 * paragraphs: training-free block sparsity scores tile blocks of Q and K by
 * their mean-pooled vectors and keeps whole key blocks; the gap to the dense
 * output is measured at equal density).
 *
 * mcs_block_select: vanilla block sparsity.  Blocks are runs of 64 consecutive
 * token ids (N must be a multiple of 64: MCS_EUNSUPPORTED otherwise).  For
 * every head and query block b, score each key block j by scale * mean(q over
 * b) . mean(k over j) (fp32), keep the K / 64 key blocks of highest score (ties
 * to the lower block id; K must be a multiple of 64: MCS_EINVAL), and write
 * their keys ascending to idx[h][b] (-1 padded to kpad).  With perm = the
 * identity (slot = token), idx is a selection for mcs_sparse_attn, so block and
 * token-level selections run through the same gather kernel.  Needs workspace
 * (op MCS_OP_BLOCK_SELECT: the block means); q, k 16-byte aligned.
 *
 * mcs_sparse_lse: the natural-log logsumexp of each query's logits
 * scale * q_i . k_j over its group's kept keys (perm, idx as for
 * mcs_sparse_attn), written to lse [H][N] in token order.  With the dense
 * logsumexp L_i (mcs_dense_attn), exp(lse_i - L_i) is the share of query i's
 * dense softmax mass that its kept keys capture. */
int mcs_block_select(const mcs_dims* d, const void* q, const void* k, int32_t* idx, void* ws, size_t ws_bytes,
                     hipStream_t stream);
int mcs_sparse_lse(const mcs_dims* d, const void* q, const void* k, const int32_t* perm, const int32_t* idx, float* lse,
                   hipStream_t stream);

/* Gather sharing between neighbouring groups (summary page, grouping paragraph:
 * PDDP cuts similar queries into groups, so adjacent leaves of its tree keep
 * overlapping key sets; the gather of K/V rows by index bounds the sparse
 * kernel).  Groups 2p and 2p+1 of each head form pair p, P = ceil(G/2) pairs.
 *
 * mcs_pair_plan: from kept-key lists idx [H][G][kpad] (as mcs_select writes
 * them: K distinct keys in [0, N) per row, -1 padded), write pidx [H][G][kpad]
 * and ncommon int32 [H][P].  Both rows of pair p become [nc keys kept by both
 * groups (the lowest such ids, ascending) | the group's other keys, ascending],
 * -1 padded, with nc = 128 * floor(|common| / 128) stored in ncommon[h][p]; a
 * lone last group (odd G) keeps its list and gets nc = 0.  Every row still holds
 * exactly its group's kept set.  pidx may equal idx (in place).  N <=
 * MCS_PAIRS_MAX_N (MCS_EUNSUPPORTED otherwise); idx and pidx 16-byte aligned.
 *
 * mcs_sparse_attn_pairs: the same result as mcs_sparse_attn on pidx (up to the
 * order of the softmax sums), with each key of a pair's common prefix gathered
 * once for both groups.  pidx and ncommon must come from mcs_pair_plan with the
 * same d; an ncommon entry that is not a multiple of 128 in [0, K] is treated
 * as 0 (no sharing, still exact).  resid_add as for mcs_sparse_attn (so this
 * is also the reuse step on a pair-planned cache).  fp32 inputs run the plain
 * gather kernel on pidx. */
#define MCS_PAIRS_MAX_N (1 << 19)
int mcs_pair_plan(const mcs_dims* d, const int32_t* idx, int32_t* pidx, int32_t* ncommon, hipStream_t stream);
int mcs_sparse_attn_pairs(const mcs_dims* d, const void* q, const void* k, const void* v, const int32_t* perm,
                          const int32_t* pidx, const int32_t* ncommon, const void* resid_add, void* o,
                          hipStream_t stream);

/* Meta-cache transfer helper (summary page, residual paragraph: inactive cache
 * entries move to host memory and the next layer is prefetched): enqueue a copy
 * of `bytes` bytes on `stream` (kind MCS_COPY_H2D / D2H / D2D; host buffers
 * should be pinned for the copy to be asynchronous) and, if done is non-NULL,
 * record `done` on the stream after it. */
int mcs_copy_async(void* dst, const void* src, size_t bytes, int32_t kind, hipStream_t stream, hipEvent_t done);

#ifdef __cplusplus
}
#endif

#endif /* MCS_H */
