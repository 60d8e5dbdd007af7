// The C ABI of include/mha_fwd.h: argument validation (before any HIP call),
// the per-(device, stream) scheduler workspace, and dispatch to the compiled
// kernel variants.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "kernels.h"
#include "mha_fwd.h"

namespace mha {

const Variant* find_variant(int dtype, int dn, int dr, int dv) {
  switch (dtype) {
    case MHA_DTYPE_F32:
      return find_variant_f32(dn, dr, dv);
    case MHA_DTYPE_BF16:
      return find_variant_bf16(dn, dr, dv);
    case MHA_DTYPE_FP8_E4M3:
      return find_variant_fp8(dn, dr, dv, false);
    case MHA_DTYPE_FP8_E4M3_FASTACC:
      return find_variant_fp8(dn, dr, dv, true);
    default:
      return nullptr;
  }
}

}  // namespace mha

namespace {

thread_local std::string g_err;
// measurement hook (mha_fwd_set_kernel_events): events recorded around the
// attention kernel of each mha_fwd call made by this host thread
thread_local hipEvent_t g_ev_start = nullptr;
thread_local hipEvent_t g_ev_stop = nullptr;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int fail_hip(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return MHA_ERR_HIP;
}

// Scheduler workspace: [SchedState | table (16-byte entries x capacity) | scratch (int x groups)]
struct Workspace {
  char* buf = nullptr;
  size_t bytes = 0;
};

std::mutex g_mu;
std::map<std::pair<int, void*>, Workspace> g_ws;

// mha_fwd_noalloc's workspace: a file-scope device array (one copy per GPU,
// held until the process ends).  Host code never uses its name as an
// address: each device's copy is located once with hipGetSymbolAddress, on
// that device's first call, and that pointer is what the kernels get.
constexpr size_t kNoAllocBytes = size_t(16) << 20;
static __device__ __align__(256) char scratch[kNoAllocBytes];
constexpr int kMaxDevices = 64;
char* g_noalloc_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (dev is the current device).
hipError_t noalloc_workspace(int dev, char** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_noalloc_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_noalloc_ptr[dev] = static_cast<char*>(ptr);
  }
  *out = g_noalloc_ptr[dev];
  return hipSuccess;
}

constexpr size_t kStateBytes = (sizeof(mha::SchedState) + 255) / 256 * 256;
static_assert(alignof(mha::SchedState) <= 256, "workspace base is 256-byte aligned");

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Returns the workspace of (dev, stream) with at least `need` bytes.  A
// workspace that must grow is freed only after the stream has drained, since
// kernels already queued on it may still read it.
hipError_t get_workspace(int dev, hipStream_t stream, size_t need, char** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  Workspace& ws = g_ws[{dev, (void*)stream}];
  if (ws.bytes < need) {
    if (ws.buf) {
      hipError_t e = hipStreamSynchronize(stream);
      if (e != hipSuccess) return e;
      e = hipFree(ws.buf);
      if (e != hipSuccess) return e;
      ws.buf = nullptr;
      ws.bytes = 0;
    }
    size_t bytes = align_up(need < (1u << 20) ? (1u << 20) : need, 1u << 20);
    hipError_t e = hipMalloc(&ws.buf, bytes);
    if (e != hipSuccess) return e;
    ws.bytes = bytes;
  }
  *out = ws.buf;
  return hipSuccess;
}

int cu_count(int dev) {
  static int counts[64] = {0};
  if (dev < 0 || dev >= 64) return 256;
  if (counts[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < 1)
      n = 256;
    counts[dev] = n;
  }
  return counts[dev];
}

struct Plan {
  int capacity;  // work-table entries (upper bound on items)
  int groups;    // batch * num_kv_heads
  size_t bytes;  // workspace size
};

// float32 calls with at most this many sequences (and at most one work item
// per workgroup of a full launch) skip the scheduler: see `direct` below
constexpr int kDirectMaxBatch = 64;

int make_plan(int batch, int max_seqlen, int num_heads, int num_kv_heads, int block_m,
              int num_splits, Plan* plan) {
  long long tiles = ((long long)max_seqlen + block_m - 1) / block_m;
  long long cap = (long long)num_heads * batch * tiles * num_splits;
  if (tiles >= mha::kMaxQTilesPerSeq || cap > INT_MAX / 2)
    return fail(MHA_ERR_INVALID_ARG, "problem too large for the work table");
  long long groups = (long long)batch * num_kv_heads;
  if (groups > INT_MAX / 2) return fail(MHA_ERR_INVALID_ARG, "batch * num_kv_heads too large");
  plan->capacity = (int)cap;
  plan->groups = (int)groups;
  plan->bytes = kStateBytes + align_up((size_t)cap * sizeof(mha::i32x4), 256) +
                align_up((size_t)groups * sizeof(int), 256);
  return MHA_OK;
}

int check_scalars(int32_t batch, int32_t max_seqlen, int32_t num_heads,
                  int32_t num_kv_heads) {
  if (batch < 1 || batch >= mha::kMaxBatch)
    return fail(MHA_ERR_INVALID_ARG, "batch must be in [1, 2^24)");
  if (max_seqlen < 0) return fail(MHA_ERR_INVALID_ARG, "max_seqlen must be >= 0");
  if (num_heads < 1 || num_kv_heads < 1)
    return fail(MHA_ERR_INVALID_ARG, "num_heads and num_kv_heads must be >= 1");
  if (num_heads % num_kv_heads != 0)
    return fail(MHA_ERR_INVALID_ARG, "num_heads must be a multiple of num_kv_heads");
  if (num_heads >= mha::kMaxHeads) return fail(MHA_ERR_INVALID_ARG, "num_heads too large");
  return MHA_OK;
}

// Key splits for mha_fwd.  With every sequence taken at max_seqlen (an upper
// bound the host can compute without reading cu_seqlens), the run lasts at
// least as long as the longest item (nb blocks) and as the average work per
// CU; when the longest item exceeds that average by more than a quarter, its
// keys are split so that a split is about 0.83 of the average (the
// scheduler then has pieces to even the CUs out with, and the merge reads
// few partials), with at least 8 blocks per split, at most 8 splits, and at
// most 1 GiB of partials.  (Splits of half the average measured 6-9% slower
// whole-step on causal B1 S16384 with 4 and with 2 heads.)
int auto_splits(long long batch, long long max_seqlen, long long num_heads, int causal,
                long long v_dim, int bm, int bn, int cus) {
  if (batch < 1 || max_seqlen < 1 || num_heads < 1 || cus < 1) return 1;
  const long long tiles = (max_seqlen + bm - 1) / bm;
  const long long nb = (max_seqlen + bn - 1) / bn;
  long long per_tile_sum = 0;  // blocks of one (sequence, head)'s q-tiles
  if (causal) {
    const long long full = std::min(tiles, nb * bn / bm);  // tiles whose keys do not reach past the end
    per_tile_sum = (bm / bn) * full * (full + 1) / 2 + (tiles - full) * nb;
  } else {
    per_tile_sum = tiles * nb;
  }
  const long long total = batch * num_heads * per_tile_sum;
  const long long per_cu = (total + cus - 1) / cus;
  if (4 * nb <= 5 * per_cu) return 1;
  long long sp = (6 * nb + 5 * per_cu - 1) / std::max(1LL, 5 * per_cu);  // ceil(1.2 nb / per_cu)
  sp = std::min({sp, 8LL, nb / 8});
  const long long tokens = batch * max_seqlen;
  while (sp > 1 && (sp * tokens * num_heads * v_dim * 4 > (1LL << 30) || tokens > INT_MAX / 2)) --sp;
  return sp > 1 ? (int)sp : 1;
}

}  // namespace

extern "C" {

const char* mha_fwd_last_error(void) { return g_err.c_str(); }

int mha_fwd_auto_splits(int32_t batch, int32_t max_seqlen, int32_t num_heads, int32_t causal,
                        int32_t v_dim, int32_t cus) {
  return auto_splits(batch, max_seqlen, num_heads, causal, v_dim, mha::kBlockM_Mfma,
                     mha::kBlockN_Mfma, cus);
}

int mha_fwd_supported(int32_t dtype, int32_t head_dim_nope, int32_t head_dim_rope,
                      int32_t v_dim) {
  return mha::find_variant(dtype, head_dim_nope, head_dim_rope, v_dim) != nullptr;
}

}  // extern "C"

namespace {

// mha_fwd, and the first half of mha_fwd_splitkv (num_splits > 1: partial
// results to o_part / lse_part, which the caller has checked).
int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse,
             const int32_t* cu_seqlens, int32_t batch, int32_t max_seqlen, int32_t num_heads,
             int32_t num_kv_heads, int32_t head_dim_nope, int32_t head_dim_rope, int32_t v_dim,
             const void* q_rope, const void* k_rope, int32_t causal, float softmax_scale,
             int32_t dtype, const float* q_scale, const float* k_scale, int32_t total_tokens,
             int32_t num_splits, float* o_part, float* lse_part, void* stream,
             bool noalloc = false) {
  int rc = check_scalars(batch, max_seqlen, num_heads, num_kv_heads);
  if (rc) return rc;
  if (head_dim_nope < 1 || head_dim_rope < 0 || v_dim < 1)
    return fail(MHA_ERR_INVALID_ARG, "head dims must be positive (rope >= 0)");
  if (causal != 0 && causal != 1) return fail(MHA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (dtype != MHA_DTYPE_F32 && dtype != MHA_DTYPE_BF16 && dtype != MHA_DTYPE_FP8_E4M3 &&
      dtype != MHA_DTYPE_FP8_E4M3_FASTACC)
    return fail(MHA_ERR_INVALID_ARG, "unknown dtype");
  if (std::isnan(softmax_scale) || std::isinf(softmax_scale))
    return fail(MHA_ERR_INVALID_ARG, "softmax_scale must be finite");
  const mha::Variant* var = mha::find_variant(dtype, head_dim_nope, head_dim_rope, v_dim);
  if (!var) return fail(MHA_ERR_UNSUPPORTED, "no compiled kernel for this (dtype, Dn, Dr, Dv)");
  // every sequence empty: nothing is read, written or launched (empty
  // tensors may come with NULL data pointers)
  if (max_seqlen == 0) return MHA_OK;
  if (!q || !k || !v || !o || !lse || !cu_seqlens)
    return fail(MHA_ERR_INVALID_ARG, "q, k, v, o, lse, cu_seqlens must be non-NULL");
  if (num_splits > 1 && !var->launch_split)
    return fail(MHA_ERR_UNSUPPORTED, "split-KV runs on the bf16 / fp8 kernels only");
  if ((q_rope == nullptr) != (k_rope == nullptr))
    return fail(MHA_ERR_INVALID_ARG, "q_rope and k_rope must both be given or both NULL");
  if ((head_dim_rope > 0) != (q_rope != nullptr))
    return fail(MHA_ERR_INVALID_ARG, "rope pointers must be given iff head_dim_rope > 0");
  const bool fp8 = dtype == MHA_DTYPE_FP8_E4M3 || dtype == MHA_DTYPE_FP8_E4M3_FASTACC;
  if (fp8 != (q_scale != nullptr) || fp8 != (k_scale != nullptr))
    return fail(MHA_ERR_INVALID_ARG, "q_scale and k_scale must be given iff dtype is FP8_E4M3");
  auto misaligned = [](const void* ptr, uintptr_t a) {
    return reinterpret_cast<uintptr_t>(ptr) % a != 0;
  };
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) ||
      misaligned(q_rope, 16) || misaligned(k_rope, 16))
    return fail(MHA_ERR_INVALID_ARG, "q, k, v, o, q_rope, k_rope must be 16-byte aligned");
  if (misaligned(lse, 4) || misaligned(cu_seqlens, 4) || misaligned(q_scale, 4) ||
      misaligned(k_scale, 4))
    return fail(MHA_ERR_INVALID_ARG, "lse, cu_seqlens, q_scale, k_scale must be 4-byte aligned");

  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  // mha_fwd: key splits of its own where the longest items would set the
  // run time, partials in the workspace (laid out for batch x max_seqlen
  // tokens; the merge stops at the real total, cu_seqlens[batch]), the O
  // partials in bfloat16 (half the bytes of float32 for the split kernel to
  // write and for the merge to read)
  // (also under mha_fwd_splitkv with num_splits = 1, which is mha_fwd exactly;
  // its partial buffers are not used then)
  // (not under mha_fwd_noalloc, whose workspace holds no partials)
  const bool auto_split = num_splits == 1 && var->launch_split != nullptr && !noalloc;
  size_t part_bytes = 0;
  if (auto_split) {
    const int sp = auto_splits(batch, max_seqlen, num_heads, causal, v_dim, var->block_m,
                               var->block_n, cu_count(dev));
    if (sp > 1) {
      num_splits = sp;
      total_tokens = (int32_t)((long long)batch * max_seqlen);  // auto_splits keeps this within int
      part_bytes = align_up((size_t)sp * total_tokens * num_heads * v_dim * sizeof(uint16_t), 256) +
                   align_up((size_t)sp * num_heads * total_tokens * sizeof(float), 256);
    }
  }
  const bool split_here = auto_split && num_splits > 1;

  Plan plan;
  rc = make_plan(batch, max_seqlen, num_heads, num_kv_heads, var->block_m, num_splits, &plan);
  if (rc) return rc;

  const float sigma =
      softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)(head_dim_nope + head_dim_rope));
  // float32 problems small enough for one workgroup per work item (the
  // (sequence, head, q-tile) grid of max_seqlen) map item = workgroup
  // directly: no work table, no prepass launch, no queue round trips (the
  // kernel reads cu_seqlens, and refuses lengths as the prepass would)
  const long long full_grid = (long long)cu_count(dev) * var->blocks_per_cu();
  const bool direct = dtype == MHA_DTYPE_F32 && num_splits == 1 && !split_here &&
                      plan.capacity <= full_grid && batch <= kDirectMaxBatch;
  char* ws = nullptr;
  if (direct) {
    // (nothing to stage)
  } else if (noalloc) {
    if (plan.bytes > kNoAllocBytes)
      return fail(MHA_ERR_INVALID_ARG,
                  "mha_fwd_noalloc: the work table needs " + std::to_string(plan.bytes) +
                      " bytes; its fixed workspace holds " + std::to_string(kNoAllocBytes));
    e = noalloc_workspace(dev, &ws);
    if (e != hipSuccess) return fail_hip(e, "mha_fwd_noalloc: workspace lookup");
  } else {
    e = get_workspace(dev, s, plan.bytes + part_bytes, &ws);
    if (e != hipSuccess) return fail_hip(e, "workspace allocation");
  }
  if (split_here && !direct) {
    o_part = reinterpret_cast<float*>(ws + plan.bytes);
    lse_part = reinterpret_cast<float*>(
        ws + plan.bytes +
        align_up((size_t)num_splits * total_tokens * num_heads * v_dim * sizeof(uint16_t), 256));
  }
  auto* st = direct ? nullptr : reinterpret_cast<mha::SchedState*>(ws);
  auto* table = direct ? nullptr : reinterpret_cast<mha::i32x4*>(ws + kStateBytes);
  if (!direct) {
    auto* gwork = reinterpret_cast<int*>(ws + kStateBytes +
                                         align_up((size_t)plan.capacity * sizeof(mha::i32x4), 256));
    const int chunk = mha::prepass_chunk(causal, num_heads / num_kv_heads,
                                         (max_seqlen + var->block_m - 1) / var->block_m);
    e = mha::launch_prepass(cu_seqlens, batch, max_seqlen, num_heads, num_kv_heads, causal,
                            var->block_m, var->block_n, num_splits, plan.capacity, chunk, table,
                            st, gwork, s);
    if (e != hipSuccess) return fail_hip(e, "scheduler prepass launch");
  }

  mha::AttnParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.q_rope = q_rope;
  p.k_rope = k_rope;
  p.q_scale = q_scale;
  p.k_scale = k_scale;
  p.cu_seqlens = cu_seqlens;
  p.table = table;
  p.sched = st;
  p.batch = batch;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = num_heads / num_kv_heads;
  p.causal = causal;
  p.scale_log2 = sigma * 1.4426950408889634f;
  p.num_splits = num_splits;
  p.part_tokens = total_tokens;
  p.o_part = num_splits > 1 ? o_part : nullptr;
  p.lse_part = num_splits > 1 ? lse_part : nullptr;
  p.max_seqlen = max_seqlen;
  p.part_bf16 = split_here ? 1 : 0;

  // direct: exactly one workgroup per item of the grid (none when
  // max_seqlen is 0: every sequence is then empty or the call is refused,
  // and either way nothing is written)
  long long grid = direct ? plan.capacity : full_grid;
  if (!direct && grid > plan.capacity) grid = plan.capacity;
  if (!direct && grid < 1) grid = 1;
  if (g_ev_start) {
    e = hipEventRecord(g_ev_start, s);
    if (e != hipSuccess) return fail_hip(e, "hipEventRecord (start)");
  }
  if (grid > 0) {
    e = (num_splits > 1 ? var->launch_split : var->launch)(p, (int)grid, s);
    if (e != hipSuccess) return fail_hip(e, "attention kernel launch");
  }
  if (g_ev_stop) {
    e = hipEventRecord(g_ev_stop, s);
    if (e != hipSuccess) return fail_hip(e, "hipEventRecord (stop)");
  }
  if (num_splits > 1) {
    // (a refused call writes no partial; the merge then writes nothing)
    e = mha::launch_combine(o_part, split_here, lse_part, num_splits, total_tokens,
                            split_here ? cu_seqlens + batch : nullptr, num_heads, v_dim,
                            dtype != MHA_DTYPE_F32, o, lse, st, s);
    if (e != hipSuccess) return fail_hip(e, "split-KV merge launch");
  }
  return MHA_OK;
}

}  // namespace

extern "C" {

int mha_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
            const int32_t* cu_seqlens, int32_t batch, int32_t max_seqlen, int32_t num_heads,
            int32_t num_kv_heads, int32_t head_dim_nope, int32_t head_dim_rope, int32_t v_dim,
            const void* q_rope, const void* k_rope, int32_t causal, float softmax_scale,
            int32_t dtype, const float* q_scale, const float* k_scale, void* stream) {
  g_err.clear();
  return fwd_impl(q, k, v, o, lse, cu_seqlens, batch, max_seqlen, num_heads, num_kv_heads,
                  head_dim_nope, head_dim_rope, v_dim, q_rope, k_rope, causal, softmax_scale,
                  dtype, q_scale, k_scale, 0, 1, nullptr, nullptr, stream);
}

int mha_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu_seqlens, int32_t batch, int32_t max_seqlen,
                    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim_nope,
                    int32_t head_dim_rope, int32_t v_dim, const void* q_rope, const void* k_rope,
                    int32_t causal, float softmax_scale, int32_t dtype, const float* q_scale,
                    const float* k_scale, void* stream) {
  g_err.clear();
  return fwd_impl(q, k, v, o, lse, cu_seqlens, batch, max_seqlen, num_heads, num_kv_heads,
                  head_dim_nope, head_dim_rope, v_dim, q_rope, k_rope, causal, softmax_scale,
                  dtype, q_scale, k_scale, 0, 1, nullptr, nullptr, stream, true);
}

int mha_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu_seqlens, int32_t batch, int32_t max_seqlen,
                    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim_nope,
                    int32_t head_dim_rope, int32_t v_dim, const void* q_rope, const void* k_rope,
                    int32_t causal, float softmax_scale, int32_t dtype, const float* q_scale,
                    const float* k_scale, int32_t total_tokens, int32_t num_splits,
                    float* o_partial, float* lse_partial, void* stream) {
  g_err.clear();
  if (num_splits < 1 || num_splits > mha::kMaxSplits)
    return fail(MHA_ERR_INVALID_ARG, "num_splits must be in [1, 64]");
  if (total_tokens < 0) return fail(MHA_ERR_INVALID_ARG, "total_tokens must be >= 0");
  if (dtype == MHA_DTYPE_F32)
    return fail(MHA_ERR_UNSUPPORTED, "split-KV runs on the bf16 / fp8 kernels only");
  if (num_splits > 1 && max_seqlen > 0 && (!o_partial || !lse_partial))
    return fail(MHA_ERR_INVALID_ARG, "o_partial and lse_partial must be non-NULL");
  if (num_splits > 1 && max_seqlen > 0 &&
      (reinterpret_cast<uintptr_t>(o_partial) % 16 != 0 ||
       reinterpret_cast<uintptr_t>(lse_partial) % 4 != 0))
    return fail(MHA_ERR_INVALID_ARG, "o_partial must be 16-byte and lse_partial 4-byte aligned");
  return fwd_impl(q, k, v, o, lse, cu_seqlens, batch, max_seqlen, num_heads, num_kv_heads,
                  head_dim_nope, head_dim_rope, v_dim, q_rope, k_rope, causal, softmax_scale,
                  dtype, q_scale, k_scale, total_tokens, num_splits, o_partial, lse_partial,
                  stream);
}

int mha_combine_splits(const float* o_partial, const float* lse_partial, int32_t num_splits,
                       int32_t total_tokens, int32_t num_heads, int32_t v_dim, int32_t out_dtype,
                       void* o, float* lse, void* stream) {
  g_err.clear();
  if (num_splits < 1 || num_splits > mha::kMaxSplits)
    return fail(MHA_ERR_INVALID_ARG, "num_splits must be in [1, 64]");
  if (total_tokens < 0 || num_heads < 1)
    return fail(MHA_ERR_INVALID_ARG, "total_tokens must be >= 0 and num_heads >= 1");
  if (v_dim != 64 && v_dim != 128) return fail(MHA_ERR_UNSUPPORTED, "v_dim must be 64 or 128");
  if (out_dtype != MHA_DTYPE_F32 && out_dtype != MHA_DTYPE_BF16)
    return fail(MHA_ERR_INVALID_ARG, "out_dtype must be MHA_DTYPE_F32 or MHA_DTYPE_BF16");
  if (total_tokens == 0) return MHA_OK;
  if (!o_partial || !lse_partial || !o || !lse)
    return fail(MHA_ERR_INVALID_ARG, "o_partial, lse_partial, o, lse must be non-NULL");
  if (reinterpret_cast<uintptr_t>(o_partial) % 16 != 0 || reinterpret_cast<uintptr_t>(o) % 16 != 0)
    return fail(MHA_ERR_INVALID_ARG, "o_partial and o must be 16-byte aligned");
  hipError_t e = mha::launch_combine(o_partial, false, lse_partial, num_splits, total_tokens, nullptr,
                                     num_heads, v_dim, out_dtype == MHA_DTYPE_BF16, o, lse,
                                     nullptr, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail_hip(e, "split-KV merge launch");
  return MHA_OK;
}

int mha_fwd_set_kernel_events(void* start_event, void* stop_event) {
  g_err.clear();
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(MHA_ERR_INVALID_ARG, "start_event and stop_event must both be given or both NULL");
  g_ev_start = static_cast<hipEvent_t>(start_event);
  g_ev_stop = static_cast<hipEvent_t>(stop_event);
  return MHA_OK;
}

int mha_fwd_kernel_info(int32_t dtype, int32_t head_dim_nope, int32_t head_dim_rope,
                        int32_t v_dim, int32_t* block_m, int32_t* blocks_per_cu, int32_t* grid,
                        int32_t* lds_bytes) {
  g_err.clear();
  const mha::Variant* var = mha::find_variant(dtype, head_dim_nope, head_dim_rope, v_dim);
  if (!var) return fail(MHA_ERR_UNSUPPORTED, "no compiled kernel for this (dtype, Dn, Dr, Dv)");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  const int bpc = var->blocks_per_cu();
  if (block_m) *block_m = var->block_m;
  if (blocks_per_cu) *blocks_per_cu = bpc;
  if (grid) *grid = cu_count(dev) * bpc;
  if (lds_bytes) *lds_bytes = var->lds_bytes;
  return MHA_OK;
}

int mha_sched_visit(const int32_t* cu_seqlens, int32_t batch, int32_t max_seqlen,
                    int32_t num_heads, int32_t num_kv_heads, int32_t causal, int32_t block_m,
                    int32_t grid, int32_t protocol, int32_t* visits, void* stream) {
  g_err.clear();
  int rc = check_scalars(batch, max_seqlen, num_heads, num_kv_heads);
  if (rc) return rc;
  if (protocol != 0 && protocol != 1) return fail(MHA_ERR_INVALID_ARG, "protocol must be 0 or 1");
  if (!cu_seqlens) return fail(MHA_ERR_INVALID_ARG, "cu_seqlens is NULL");
  if (!visits) return fail(MHA_ERR_INVALID_ARG, "visits is NULL");
  if (causal != 0 && causal != 1) return fail(MHA_ERR_INVALID_ARG, "causal must be 0 or 1");
  int block_n;
  if (block_m == mha::kBlockM_Mfma)
    block_n = mha::kBlockN_Mfma;
  else if (block_m == mha::kBlockM_F32)
    block_n = mha::kBlockN_F32;
  else
    return fail(MHA_ERR_INVALID_ARG, "block_m must be 32 or 256");
  if (grid < 0) return fail(MHA_ERR_INVALID_ARG, "grid must be >= 0");
  if (max_seqlen == 0) return MHA_OK;
  Plan plan;
  rc = make_plan(batch, max_seqlen, num_heads, num_kv_heads, block_m, 1, &plan);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  char* ws = nullptr;
  e = get_workspace(dev, s, plan.bytes, &ws);
  if (e != hipSuccess) return fail_hip(e, "workspace allocation");
  auto* st = reinterpret_cast<mha::SchedState*>(ws);
  auto* table = reinterpret_cast<mha::i32x4*>(ws + kStateBytes);
  auto* gwork = reinterpret_cast<int*>(ws + kStateBytes + align_up((size_t)plan.capacity * sizeof(mha::i32x4), 256));
  const int chunk = mha::prepass_chunk(causal, num_heads / num_kv_heads,
                                       (max_seqlen + block_m - 1) / block_m);
  e = mha::launch_prepass(cu_seqlens, batch, max_seqlen, num_heads, num_kv_heads, causal, block_m,
                          block_n, 1, plan.capacity, chunk, table, st, gwork, s);
  if (e != hipSuccess) return fail_hip(e, "scheduler prepass launch");
  if (grid == 0) grid = cu_count(dev) * 2;
  const int tiles = (int)(((long long)max_seqlen + block_m - 1) / block_m);
  e = mha::launch_sched_visit(batch, num_heads, tiles, protocol, table, st, visits, grid, s);
  if (e != hipSuccess) return fail_hip(e, "visit kernel launch");
  return MHA_OK;
}

int mha_quantize_fp8(const void* x, int32_t x_dtype, int64_t rows, int32_t cols,
                     uint8_t* codes, float* scales, void* stream) {
  g_err.clear();
  if (x_dtype != MHA_DTYPE_F32 && x_dtype != MHA_DTYPE_BF16)
    return fail(MHA_ERR_INVALID_ARG, "x_dtype must be MHA_DTYPE_F32 or MHA_DTYPE_BF16");
  if (rows < 0 || rows > INT_MAX) return fail(MHA_ERR_INVALID_ARG, "rows must be in [0, 2^31)");
  if (cols < 8 || cols > 512 || cols % 8 != 0)
    return fail(MHA_ERR_INVALID_ARG, "cols must be a multiple of 8 in [8, 512]");
  if (rows == 0) return MHA_OK;
  if (!x || !codes || !scales)
    return fail(MHA_ERR_INVALID_ARG, "x, codes, scales must be non-NULL");
  if (reinterpret_cast<uintptr_t>(x) % 16 != 0 || reinterpret_cast<uintptr_t>(codes) % 8 != 0 ||
      reinterpret_cast<uintptr_t>(scales) % 4 != 0)
    return fail(MHA_ERR_INVALID_ARG, "x must be 16-byte, codes 8-byte, scales 4-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (g_ev_start && (e = hipEventRecord(g_ev_start, s)) != hipSuccess)
    return fail_hip(e, "hipEventRecord");
  e = mha::launch_fp8_quant(x, x_dtype == MHA_DTYPE_BF16, rows, cols, codes, scales, s);
  if (e != hipSuccess) return fail_hip(e, "quantiser launch");
  if (g_ev_stop && (e = hipEventRecord(g_ev_stop, s)) != hipSuccess)
    return fail_hip(e, "hipEventRecord");
  return MHA_OK;
}

}  // extern "C"
