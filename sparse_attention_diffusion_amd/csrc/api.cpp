// C ABI of the MC-Sparse hot path: host-side validation, workspace carve-up and
// the composition of the kernels into the anchor and reuse steps.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/mcs.h"
#include "blocksel.hpp"
#include "kernels.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MCS_EHIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int elem_size(int32_t dtype) { return dtype == MCS_BF16 ? 2 : 4; }

int groups_of(const mcs_dims* d) { return (d->n + d->group - 1) / d->group; }

// Shape checks shared by every op.  need_topk: K/kpad are used by the op.
int check_dims(const mcs_dims* d, bool need_topk) {
  if (!d) return fail(MCS_EINVAL, "dims is NULL");
  if (d->heads < 1 || d->n < 1) return fail(MCS_EINVAL, "heads (%d) and n (%d) must be >= 1", d->heads, d->n);
  if (d->dtype != MCS_F32 && d->dtype != MCS_BF16) return fail(MCS_EUNSUPPORTED, "unknown dtype %d", d->dtype);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(MCS_EUNSUPPORTED, "head_dim %d not supported (64 or 128)", d->head_dim);
  if (d->group != 64) return fail(MCS_EUNSUPPORTED, "group size %d not supported (must be 64)", d->group);
  if (!(d->scale > 0.0f) || !isfinite(d->scale)) return fail(MCS_EINVAL, "scale must be finite and > 0");
  const size_t head_bytes = (size_t)d->n * d->head_dim * elem_size(d->dtype);
  if (head_bytes >= ((size_t)1 << 31)) return fail(MCS_EINVAL, "one head of q/k/v exceeds 2 GiB");
  if ((size_t)d->heads * (size_t)groups_of(d) >= ((size_t)1 << 31)) return fail(MCS_EINVAL, "too many groups");
  if (need_topk) {
    if (d->topk < 1 || d->topk > d->n) return fail(MCS_EINVAL, "topk %d outside [1, n=%d]", d->topk, d->n);
    if (d->kpad < d->topk || d->kpad % 32 != 0)
      return fail(MCS_EINVAL, "kpad %d must be >= topk (%d) and a multiple of 32", d->kpad, d->topk);
  }
  return MCS_OK;
}

int check_ptr(const void* p, size_t align, const char* name) {
  if (!p) return fail(MCS_EINVAL, "%s is NULL", name);
  if (((uintptr_t)p) % align != 0) return fail(MCS_EINVAL, "%s is not %zu-byte aligned", name, align);
  return MCS_OK;
}

#define CHECK(x)               \
  do {                         \
    int _rc = (x);             \
    if (_rc != MCS_OK) return _rc; \
  } while (0)

size_t stats_bytes(const mcs_dims* d) { return align256((size_t)d->heads * d->n * 8); }
int mass_ld(const mcs_dims* d) { return (d->n + 3) & ~3; }
size_t mass_rows_bytes_per_head(const mcs_dims* d) { return align256((size_t)groups_of(d) * mass_ld(d) * 4); }
constexpr size_t kHistBytesPerGroup = (size_t)mcs::kMassHistBins * 4;  // a mass row's histogram
size_t mass_bytes_per_head(const mcs_dims* d) {
  return mass_rows_bytes_per_head(d) + align256((size_t)groups_of(d) * kHistBytesPerGroup);
}
size_t group_ws(const mcs_dims* d) { return mcs::pddp_workspace_bytes(d->heads, d->n, d->head_dim, d->group); }
size_t select_ws(const mcs_dims* d, int hpp) { return stats_bytes(d) + (size_t)hpp * mass_bytes_per_head(d); }
// The anchor keeps the grouping's workspace beside the selection's, so that
// grouping can run while dense attention writes the row statistics.
size_t anchor_ws(const mcs_dims* d, int hpp) { return align256(group_ws(d)) + select_ws(d, hpp); }

mcs::AttnArgs attn_args(const mcs_dims* d, const void* q, const void* k, const void* v) {
  mcs::AttnArgs a{};
  a.xcd_chunk = mcs::kXcdChunk;
  a.q = q;
  a.k = k;
  a.v = v;
  a.H = d->heads;
  a.N = d->n;
  a.G = groups_of(d);
  a.nkeys = d->n;
  a.kpad = d->kpad;
  a.c = (float)((double)d->scale * 1.4426950408889634);
  return a;
}

// Selection pass 2 and the top-K over all heads, hpp heads of mass rows at a
// time: the loop writes the rows and their histograms, then the top-K reads
// them.  (Running each pass's top-K on a second stream beside the next pass's
// loop, with double-buffered rows, measured about 1 ms slower on the 40-head
// benchmark layer: the top-K's memory traffic slows the loop more than it hides.)
int run_select(const mcs_dims* d, const void* q, const void* k, const int32_t* perm, const float2* stats,
               const float* lse, int32_t* idx, float* mass, int hpp, hipStream_t s) {
  const int G = groups_of(d);
  for (int h0 = 0; h0 < d->heads; h0 += hpp) {
    mcs::MassArgs m{};
    m.q = q;
    m.k = k;
    m.perm = perm;
    m.stats = stats;
    m.lse = lse;
    m.mass = mass;
    // the histograms follow the mass rows of hpp heads
    m.hist = (uint32_t*)((char*)mass + (size_t)hpp * mass_rows_bytes_per_head(d));
    m.ldm = mass_ld(d);
    m.h0 = h0;
    m.hcount = d->heads - h0 < hpp ? d->heads - h0 : hpp;
    m.N = d->n;
    m.G = G;
    m.c = (float)((double)d->scale * 1.4426950408889634);
    m.xcd_chunk = mcs::kXcdChunk;
    m.idx = idx;
    m.K = d->topk;
    m.kpad = d->kpad;
    hipError_t e = mcs::launch_group_mass(m, d->dtype, d->head_dim, s);
    if (e != hipSuccess) return hip_fail(e, "selection pass 2 launch");
    if ((e = mcs::launch_topk(m, s)) != hipSuccess) return hip_fail(e, "top-K launch");
  }
  return MCS_OK;
}

int heads_per_pass(const mcs_dims* d, size_t ws_bytes) {
  const size_t fixed = stats_bytes(d), per = mass_bytes_per_head(d);
  if (ws_bytes < fixed + per) return 0;
  size_t hpp = (ws_bytes - fixed) / per;
  return hpp > (size_t)d->heads ? d->heads : (int)hpp;
}

// Device-resident scratch of mcs_select_noalloc (for callers that cannot
// allocate).  In host code `scratch` names a host-side stand-in, not device
// memory: only the address hipGetSymbolAddress returns for the current device
// is ever handed to a kernel.  Each GPU the library runs on holds its own copy
// until the process ends.
static __device__ __align__(256) unsigned char scratch[MCS_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device.
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MCS_EUNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(MCS_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MCS_OK;
}

// One stream per device for work that runs beside the caller's stream inside
// a call (grouping beside dense attention in mcs_anchor).  Created on first
// use with the default priority; it lives until the process ends.
std::mutex g_side_mu;
hipStream_t g_side[kMaxDevices] = {};

int side_stream(hipStream_t* out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MCS_EUNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_side_mu);
  if (!g_side[dev]) {
    hipStream_t s = nullptr;
    e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
    if (e != hipSuccess) return hip_fail(e, "hipStreamCreateWithFlags");
    g_side[dev] = s;
  }
  *out = g_side[dev];
  return MCS_OK;
}

}  // namespace

extern "C" {

int32_t mcs_abi_version(void) { return MCS_ABI_VERSION; }

const char* mcs_last_error(void) { return g_err.c_str(); }

int mcs_workspace_bytes(const mcs_dims* d, int32_t op, int32_t hpp, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(MCS_EINVAL, "bytes is NULL");
  CHECK(check_dims(d, false));
  if (hpp < 0) return fail(MCS_EINVAL, "heads_per_pass must be >= 0");
  const int h = (hpp == 0 || hpp > d->heads) ? d->heads : hpp;
  switch (op) {
    case MCS_OP_GROUP: *bytes = group_ws(d); return MCS_OK;
    case MCS_OP_SELECT: *bytes = select_ws(d, h); return MCS_OK;
    case MCS_OP_ANCHOR: *bytes = anchor_ws(d, h); return MCS_OK;
    case MCS_OP_BLOCK_SELECT: *bytes = align256(mcs::block_select_ws_bytes(d->heads, d->n, d->head_dim)); return MCS_OK;
    default: return fail(MCS_EINVAL, "unknown op %d", op);
  }
}

int mcs_group(const mcs_dims* d, const void* q, int32_t* perm, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err.clear();
  CHECK(check_dims(d, false));
  if (d->power_iters < 1 || d->power_iters > 1024) return fail(MCS_EINVAL, "power_iters %d outside [1, 1024]", d->power_iters);
  CHECK(check_ptr(q, 16, "q"));
  CHECK(check_ptr(perm, 4, "perm"));
  CHECK(check_ptr(ws, 256, "workspace"));
  if (ws_bytes < group_ws(d)) return fail(MCS_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, group_ws(d));
  mcs::PddpArgs a{q, perm, ws, d->heads, d->n, d->head_dim, d->group, d->power_iters};
  hipError_t e = mcs::launch_pddp(a, d->dtype, stream);
  if (e != hipSuccess) return hip_fail(e, "pddp launch");
  return MCS_OK;
}

int mcs_select(const mcs_dims* d, const void* q, const void* k, const int32_t* perm, const float* lse,
               int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err.clear();
  CHECK(check_dims(d, true));
  CHECK(check_ptr(q, 16, "q"));
  CHECK(check_ptr(k, 16, "k"));
  CHECK(check_ptr(perm, 4, "perm"));
  CHECK(check_ptr(idx, 16, "idx"));
  if (lse) CHECK(check_ptr(lse, 4, "lse"));
  CHECK(check_ptr(ws, 256, "workspace"));
  const int hpp = heads_per_pass(d, ws_bytes);
  if (hpp < 1) return fail(MCS_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, select_ws(d, 1));
  float2* stats = (float2*)ws;
  float* mass = (float*)((char*)ws + stats_bytes(d));
  if (!lse) {
    mcs::AttnArgs a = attn_args(d, q, k, nullptr);
    a.stats = stats;
    hipError_t e = mcs::launch_attention(a, d->dtype, d->head_dim, false, mcs::EPI_PLAIN, false, stream);
    if (e != hipSuccess) return hip_fail(e, "selection pass 1 launch");
  }
  return run_select(d, q, k, perm, lse ? nullptr : stats, lse, idx, mass, hpp, stream);
}

int mcs_select_noalloc(const mcs_dims* d, const void* q, const void* k, const int32_t* perm, const float* lse,
                       int32_t* idx, hipStream_t stream) {
  g_err.clear();
  CHECK(check_dims(d, true));
  CHECK(check_ptr(q, 16, "q"));
  CHECK(check_ptr(k, 16, "k"));
  CHECK(check_ptr(perm, 4, "perm"));
  CHECK(check_ptr(idx, 16, "idx"));
  if (lse) CHECK(check_ptr(lse, 4, "lse"));
  // sizes first: a workload the scratch cannot hold is rejected before any HIP call
  const size_t need = select_ws(d, 1);
  if (need > (size_t)MCS_SCRATCH_BYTES)
    return fail(MCS_EUNSUPPORTED, "selection of n=%d needs %zu bytes of scratch for one head, above the %zu the "
                "library holds (use mcs_select with a workspace)", d->n, need, (size_t)MCS_SCRATCH_BYTES);
  void* ws = nullptr;
  CHECK(scratch_address(&ws));
  // Every byte the kernels read from the scratch is written earlier in the same
  // call (row statistics by pass 1 for every token, each mass row and its
  // histogram by the pass-2 loop before the top-K reads them), so nothing left
  // by an earlier call needs clearing.
  return mcs_select(d, q, k, perm, lse, idx, ws, (size_t)MCS_SCRATCH_BYTES, stream);
}

int mcs_dense_attn(const mcs_dims* d, const void* q, const void* k, const void* v, void* o, float* lse,
                   hipStream_t stream) {
  g_err.clear();
  CHECK(check_dims(d, false));
  CHECK(check_ptr(q, 16, "q"));
  CHECK(check_ptr(k, 16, "k"));
  CHECK(check_ptr(v, 16, "v"));
  CHECK(check_ptr(o, 16, "o"));
  if (lse) CHECK(check_ptr(lse, 4, "lse"));
  mcs::AttnArgs a = attn_args(d, q, k, v);
  a.o = o;
  a.lse = lse;
  hipError_t e = mcs::launch_attention(a, d->dtype, d->head_dim, false, mcs::EPI_PLAIN, true, stream);
  if (e != hipSuccess) return hip_fail(e, "dense attention launch");
  return MCS_OK;
}

int mcs_sparse_attn(const mcs_dims* d, const void* q, const void* k, const void* v, const int32_t* perm,
                    const int32_t* idx, const void* resid_add, void* o, hipStream_t stream) {
  g_err.clear();
  CHECK(check_dims(d, true));
  CHECK(check_ptr(q, 16, "q"));
  CHECK(check_ptr(k, 16, "k"));
  CHECK(check_ptr(v, 16, "v"));
  CHECK(check_ptr(perm, 4, "perm"));
  CHECK(check_ptr(idx, 16, "idx"));
  CHECK(check_ptr(o, 16, "o"));
  if (resid_add) CHECK(check_ptr(resid_add, 16, "resid_add"));
  mcs::AttnArgs a = attn_args(d, q, k, v);
  a.perm = perm;
  a.idx = idx;
  a.nkeys = d->topk;
  a.rin = resid_add;
  a.o = o;
  hipError_t e = mcs::launch_attention(a, d->dtype, d->head_dim, true, resid_add ? mcs::EPI_ADD : mcs::EPI_PLAIN,
                                       true, stream);
  if (e != hipSuccess) return hip_fail(e, "sparse attention launch");
  return MCS_OK;
}

int mcs_anchor(const mcs_dims* d, const void* q, const void* k, const void* v, int32_t* perm, int32_t* idx,
               void* resid, void* o_dense, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err.clear();
  CHECK(check_dims(d, true));
  if (d->power_iters < 1 || d->power_iters > 1024) return fail(MCS_EINVAL, "power_iters %d outside [1, 1024]", d->power_iters);
  CHECK(check_ptr(q, 16, "q"));
  CHECK(check_ptr(k, 16, "k"));
  CHECK(check_ptr(v, 16, "v"));
  CHECK(check_ptr(perm, 4, "perm"));
  CHECK(check_ptr(idx, 16, "idx"));
  CHECK(check_ptr(resid, 16, "resid"));
  CHECK(check_ptr(o_dense, 16, "o_dense"));
  if (lse) CHECK(check_ptr(lse, 4, "lse"));
  CHECK(check_ptr(ws, 256, "workspace"));
  if (ws_bytes < group_ws(d)) return fail(MCS_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, group_ws(d));
  // With room for both workspaces, grouping runs on a side stream beside dense
  // attention (they share only q); otherwise one after the other.
  const bool overlap = ws_bytes >= anchor_ws(d, 1);
  const size_t sel_off = overlap ? align256(group_ws(d)) : 0;
  const int hpp = heads_per_pass(d, ws_bytes - sel_off);
  if (hpp < 1) return fail(MCS_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, select_ws(d, 1));
  char* sel_ws = (char*)ws + sel_off;
  mcs::PddpArgs pa{q, perm, ws, d->heads, d->n, d->head_dim, d->group, d->power_iters};
  // 2. dense attention; its row statistics double as selection pass 1
  float2* stats = (float2*)sel_ws;
  float* mass = (float*)(sel_ws + stats_bytes(d));
  mcs::AttnArgs a = attn_args(d, q, k, v);
  a.o = o_dense;
  a.lse = lse;
  a.stats = stats;
  hipError_t e;
  if (overlap) {
    hipStream_t side = nullptr;
    CHECK(side_stream(&side));
    hipEvent_t fork = nullptr, join = nullptr;
    if ((e = hipEventCreateWithFlags(&fork, hipEventDisableTiming)) != hipSuccess) return hip_fail(e, "hipEventCreate");
    if ((e = hipEventCreateWithFlags(&join, hipEventDisableTiming)) != hipSuccess) {
      hipEventDestroy(fork);
      return hip_fail(e, "hipEventCreate");
    }
    // 1. grouping on the side stream, after everything queued on `stream` so far
    hipError_t eg = hipEventRecord(fork, stream);
    if (eg == hipSuccess) eg = hipStreamWaitEvent(side, fork, 0);
    if (eg == hipSuccess) eg = mcs::launch_pddp(pa, d->dtype, side);
    const hipError_t ed = mcs::launch_attention(a, d->dtype, d->head_dim, false, mcs::EPI_PLAIN, true, stream);
    // join before anything else is queued on `stream`, whatever failed
    hipError_t ej = hipEventRecord(join, side);
    if (ej == hipSuccess) ej = hipStreamWaitEvent(stream, join, 0);
    hipEventDestroy(fork);
    hipEventDestroy(join);
    if (eg != hipSuccess) return hip_fail(eg, "pddp launch on the side stream");
    if (ed != hipSuccess) return hip_fail(ed, "dense attention launch");
    if (ej != hipSuccess) return hip_fail(ej, "side stream join");
  } else {
    // 1. grouping
    e = mcs::launch_pddp(pa, d->dtype, stream);
    if (e != hipSuccess) return hip_fail(e, "pddp launch");
    e = mcs::launch_attention(a, d->dtype, d->head_dim, false, mcs::EPI_PLAIN, true, stream);
    if (e != hipSuccess) return hip_fail(e, "dense attention launch");
  }
  // 3. selection pass 2 and top-K
  CHECK(run_select(d, q, k, perm, stats, nullptr, idx, mass, hpp, stream));
  // 4. residual = dense - sparse
  mcs::AttnArgs sa = attn_args(d, q, k, v);
  sa.perm = perm;
  sa.idx = idx;
  sa.nkeys = d->topk;
  sa.rin = o_dense;
  sa.o = resid;
  e = mcs::launch_attention(sa, d->dtype, d->head_dim, true, mcs::EPI_RESID, true, stream);
  if (e != hipSuccess) return hip_fail(e, "residual launch");
  return MCS_OK;
}

int mcs_residual(const mcs_dims* d, const void* q, const void* k, const void* v, const int32_t* perm,
                 const int32_t* idx, const void* o_dense, void* resid, hipStream_t stream) {
  g_err.clear();
  CHECK(check_dims(d, true));
  CHECK(check_ptr(q, 16, "q"));
  CHECK(check_ptr(k, 16, "k"));
  CHECK(check_ptr(v, 16, "v"));
  CHECK(check_ptr(perm, 4, "perm"));
  CHECK(check_ptr(idx, 16, "idx"));
  CHECK(check_ptr(o_dense, 16, "o_dense"));
  CHECK(check_ptr(resid, 16, "resid"));
  if (resid == o_dense) return fail(MCS_EINVAL, "resid may not alias o_dense");
  mcs::AttnArgs sa = attn_args(d, q, k, v);
  sa.perm = perm;
  sa.idx = idx;
  sa.nkeys = d->topk;
  sa.rin = o_dense;
  sa.o = resid;
  hipError_t e = mcs::launch_attention(sa, d->dtype, d->head_dim, true, mcs::EPI_RESID, true, stream);
  if (e != hipSuccess) return hip_fail(e, "residual launch");
  return MCS_OK;
}

int mcs_reuse(const mcs_dims* d, const void* q, const void* k, const void* v, const int32_t* perm,
              const int32_t* idx, const void* resid, void* o, hipStream_t stream) {
  g_err.clear();
  if (!resid) return fail(MCS_EINVAL, "resid is NULL");
  return mcs_sparse_attn(d, q, k, v, perm, idx, resid, o, stream);
}

int mcs_pair_plan(const mcs_dims* d, const int32_t* idx, int32_t* pidx, int32_t* ncommon, hipStream_t stream) {
  g_err.clear();
  CHECK(check_dims(d, true));
  CHECK(check_ptr(idx, 16, "idx"));
  CHECK(check_ptr(pidx, 16, "pidx"));
  CHECK(check_ptr(ncommon, 4, "ncommon"));
  if (d->n > MCS_PAIRS_MAX_N) return fail(MCS_EUNSUPPORTED, "n %d above %d for pair plans", d->n, MCS_PAIRS_MAX_N);
  hipError_t e = mcs::launch_pair_plan(idx, pidx, ncommon, d->heads, d->n, groups_of(d), d->topk, d->kpad, stream);
  if (e != hipSuccess) return hip_fail(e, "pair plan launch");
  return MCS_OK;
}

int mcs_sparse_attn_pairs(const mcs_dims* d, const void* q, const void* k, const void* v, const int32_t* perm,
                          const int32_t* pidx, const int32_t* ncommon, const void* resid_add, void* o,
                          hipStream_t stream) {
  g_err.clear();
  CHECK(check_dims(d, true));
  CHECK(check_ptr(q, 16, "q"));
  CHECK(check_ptr(k, 16, "k"));
  CHECK(check_ptr(v, 16, "v"));
  CHECK(check_ptr(perm, 4, "perm"));
  CHECK(check_ptr(pidx, 16, "pidx"));
  CHECK(check_ptr(ncommon, 4, "ncommon"));
  CHECK(check_ptr(o, 16, "o"));
  if (resid_add) CHECK(check_ptr(resid_add, 16, "resid_add"));
  mcs::AttnArgs a = attn_args(d, q, k, v);
  a.perm = perm;
  a.idx = pidx;
  a.nkeys = d->topk;
  a.rin = resid_add;
  a.o = o;
  const int epi = resid_add ? mcs::EPI_ADD : mcs::EPI_PLAIN;
  // fp32 has no LDS-staged kernel to share: every row is its group's whole kept
  // set, so the plain gather kernel gives the same attention
  hipError_t e = d->dtype == MCS_BF16 ? mcs::launch_attention_pairs(a, ncommon, d->head_dim, epi, stream)
                                      : mcs::launch_attention(a, d->dtype, d->head_dim, true, epi, true, stream);
  if (e != hipSuccess) return hip_fail(e, "paired sparse attention launch");
  return MCS_OK;
}

int mcs_block_select(const mcs_dims* d, const void* q, const void* k, int32_t* idx, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  g_err.clear();
  CHECK(check_dims(d, true));
  CHECK(check_ptr(q, 16, "q"));
  CHECK(check_ptr(k, 16, "k"));
  CHECK(check_ptr(idx, 4, "idx"));
  CHECK(check_ptr(ws, 256, "workspace"));
  if (d->n % 64 != 0) return fail(MCS_EUNSUPPORTED, "block selection needs n (%d) to be a multiple of 64", d->n);
  if (d->topk % 64 != 0) return fail(MCS_EINVAL, "topk %d is not a whole number of 64-token blocks", d->topk);
  if (!mcs::block_select_fits(d->n, d->head_dim))
    return fail(MCS_EUNSUPPORTED, "n %d: too many blocks for one selection block", d->n);
  const size_t need = mcs::block_select_ws_bytes(d->heads, d->n, d->head_dim);
  if (ws_bytes < need) return fail(MCS_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  hipError_t e = mcs::launch_block_select(q, k, d->dtype, d->heads, d->n, d->head_dim, d->topk / 64, d->kpad,
                                          d->scale, idx, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "block selection launch");
  return MCS_OK;
}

int mcs_sparse_lse(const mcs_dims* d, const void* q, const void* k, const int32_t* perm, const int32_t* idx, float* lse,
                   hipStream_t stream) {
  g_err.clear();
  CHECK(check_dims(d, true));
  CHECK(check_ptr(q, 16, "q"));
  CHECK(check_ptr(k, 16, "k"));
  CHECK(check_ptr(perm, 4, "perm"));
  CHECK(check_ptr(idx, 16, "idx"));
  CHECK(check_ptr(lse, 4, "lse"));
  mcs::AttnArgs a = attn_args(d, q, k, nullptr);
  a.perm = perm;
  a.idx = idx;
  a.nkeys = d->topk;
  a.lse = lse;
  hipError_t e = mcs::launch_attention(a, d->dtype, d->head_dim, true, mcs::EPI_PLAIN, false, stream);
  if (e != hipSuccess) return hip_fail(e, "sparse logsumexp launch");
  return MCS_OK;
}

int mcs_idx_to_bits(const mcs_dims* d, const int32_t* idx, uint32_t* bits, hipStream_t stream) {
  g_err.clear();
  CHECK(check_dims(d, true));
  CHECK(check_ptr(idx, 4, "idx"));
  CHECK(check_ptr(bits, 4, "bits"));
  if (d->n > MCS_BITS_MAX_N) return fail(MCS_EUNSUPPORTED, "n %d above %d for key bitmaps", d->n, MCS_BITS_MAX_N);
  hipError_t e = mcs::launch_idx_to_bits(idx, bits, d->heads * groups_of(d), d->n, d->topk, d->kpad, stream);
  if (e != hipSuccess) return hip_fail(e, "key bitmap encode launch");
  return MCS_OK;
}

int mcs_bits_to_idx(const mcs_dims* d, const uint32_t* bits, int32_t* idx, hipStream_t stream) {
  g_err.clear();
  CHECK(check_dims(d, true));
  CHECK(check_ptr(bits, 4, "bits"));
  CHECK(check_ptr(idx, 4, "idx"));
  if (d->n > MCS_BITS_MAX_N) return fail(MCS_EUNSUPPORTED, "n %d above %d for key bitmaps", d->n, MCS_BITS_MAX_N);
  hipError_t e = mcs::launch_bits_to_idx(bits, idx, d->heads * groups_of(d), d->n, d->topk, d->kpad, stream);
  if (e != hipSuccess) return hip_fail(e, "key bitmap decode launch");
  return MCS_OK;
}

int mcs_copy_async(void* dst, const void* src, size_t bytes, int32_t kind, hipStream_t stream, hipEvent_t done) {
  g_err.clear();
  if (!dst || !src) return fail(MCS_EINVAL, "dst/src is NULL");
  hipMemcpyKind k;
  switch (kind) {
    case MCS_COPY_H2D: k = hipMemcpyHostToDevice; break;
    case MCS_COPY_D2H: k = hipMemcpyDeviceToHost; break;
    case MCS_COPY_D2D: k = hipMemcpyDeviceToDevice; break;
    default: return fail(MCS_EINVAL, "unknown copy kind %d", kind);
  }
  if (bytes) {
    hipError_t e = hipMemcpyAsync(dst, src, bytes, k, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
  }
  if (done) {
    hipError_t e = hipEventRecord(done, stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  }
  return MCS_OK;
}

}  // extern "C"
