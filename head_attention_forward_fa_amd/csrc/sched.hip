// Persistent tile scheduler: the prepass that builds the work table and the
// diagnostic visit kernel.
//
// The pages describe the scheduler as a trait (MHATileScheduler: "maps work
// tiles to thread blocks, advances the per-CTA state through the work grid
// across kernel iterations, and reports the grid dimensions required for
// launch"), generic over an optional pointer of per-batch sequence-length
// offsets (Required methods: get_current_work_info, ValidLengthType), with
// a shared-memory slot that publishes the active work index to the block
// (initial_state) and an advance() that reports whether work remains.  The
// MI355X version:
//
//   * a one-workgroup prepass turns cu_seqlens into a table of work items
//     (b, h, q-tile).  Items are grouped by (sequence, KV head), so that the
//     query heads sharing a KV head and every q-tile of that sequence sit
//     next to each other; groups are dealt to 8 queues, one per XCD, largest
//     first in a snake order so the queues carry equal work; inside a group
//     the q-tiles run longest first (causal cost grows with the tile index).
//   * the attention kernel is launched with about (CUs x resident
//     workgroups) workgroups; each pops items from queue blockIdx % 8 with
//     one atomic add, then helps the other queues once its own is empty.
//
// Cost of an item, in BN-key blocks: causal ceil(min(L, (qt+1)*BM) / BN),
// non-causal ceil(L / BN).
#include "common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr int kPrepassThreads = 1024;
constexpr int kSortedMax = 2048;  // groups ranked in LDS up to this count

__device__ __forceinline__ long long group_cost(int L, int bm, int bn, int causal) {
  if (L <= 0) return 0;
  long long nqt = (L + bm - 1) / bm;
  long long last = (L + bn - 1) / bn;
  if (!causal) return nqt * last;
  return (long long)(bm / bn) * (nqt - 1) * nqt / 2 + last;
}

__device__ __forceinline__ int snake_bin(int r) {
  int p = r / kNumXcd, j = r % kNumXcd;
  return (p & 1) ? (kNumXcd - 1 - j) : j;
}

__global__ __launch_bounds__(kPrepassThreads) void sched_prepass_kernel(
    const int32_t* __restrict__ cu, int batch, int num_heads, int num_kv_heads, int causal,
    int bm, int bn, int capacity, int2* __restrict__ table, SchedState* __restrict__ st,
    int* __restrict__ scratch) {
  __shared__ long long s_cost[kSortedMax];
  __shared__ int s_items[kSortedMax];
  __shared__ int s_order[kSortedMax];   // rank -> group
  __shared__ int s_bin[kSortedMax];     // group -> queue
  __shared__ int s_off[kSortedMax];     // group -> offset inside its queue
  __shared__ int s_fill[kNumXcd];
  __shared__ unsigned long long s_total;  // 64-bit: garbage lengths must not wrap
  __shared__ int s_bad;

  const int tid = threadIdx.x;
  const int group = num_heads / num_kv_heads;
  const int n = batch * num_kv_heads;
  const bool sorted = n <= kSortedMax;
  if (tid == 0) {
    s_total = 0ull;
    s_bad = 0;
  }
  if (tid < kNumXcd) s_fill[tid] = 0;
  __syncthreads();

  // A: per-group cost and item count
  for (int i = tid; i < n; i += kPrepassThreads) {
    int b = i / num_kv_heads;
    int L = cu[b + 1] - cu[b];
    int nqt = L > 0 ? (L + bm - 1) / bm : 0;
    if (L < 0 || nqt >= kMaxQTilesPerSeq) atomicOr(&s_bad, 1);
    int items = nqt * group;
    atomicAdd(&s_total, (unsigned long long)items);
    if (sorted) {
      s_cost[i] = group_cost(L, bm, bn, causal) * group;
      s_items[i] = items;
    } else {
      scratch[i] = items;
    }
  }
  __syncthreads();
  if (s_bad || s_total > (unsigned long long)capacity) {
    if (tid < kNumXcd) {
      st->counters[tid] = 0;
      st->base[tid] = 0;
      st->count[tid] = 0;
    }
    if (tid == 0) {
      st->status = 1;
      st->total = 0;
    }
    return;
  }

  if (sorted) {
    // B: rank groups by cost, largest first (ties by index), snake-deal to queues
    for (int i = tid; i < n; i += kPrepassThreads) {
      long long c = s_cost[i];
      int rank = 0;
      for (int j = 0; j < n; ++j) {
        long long cj = s_cost[j];
        rank += (cj > c) || (cj == c && j < i);
      }
      s_order[rank] = i;
    }
    __syncthreads();
    for (int r = tid; r < n; r += kPrepassThreads) {
      int bin = snake_bin(r);
      int off = 0;
      for (int r2 = bin; r2 < r; ++r2)
        if (snake_bin(r2) == bin) off += s_items[s_order[r2]];
      int g = s_order[r];
      s_bin[g] = bin;
      s_off[g] = off;
      atomicAdd(&s_fill[bin], s_items[g]);
    }
    __syncthreads();
  } else {
    // B': contiguous index ranges per queue; offsets from an exclusive scan
    // of the item counts in index order (scratch[i] <- prefix before i)
    __shared__ int s_carry;
    __shared__ int s_scan[kPrepassThreads];
    if (tid == 0) s_carry = 0;
    __syncthreads();
    for (int c0 = 0; c0 < n; c0 += kPrepassThreads) {
      int i = c0 + tid;
      int v = i < n ? scratch[i] : 0;
      s_scan[tid] = v;
      __syncthreads();
      for (int d = 1; d < kPrepassThreads; d <<= 1) {
        int add = tid >= d ? s_scan[tid - d] : 0;
        __syncthreads();
        s_scan[tid] += add;
        __syncthreads();
      }
      if (i < n) scratch[i] = s_carry + s_scan[tid] - v;
      __syncthreads();
      if (tid == kPrepassThreads - 1) s_carry += s_scan[tid];
      __syncthreads();
    }
  }

  // C: queue slices
  if (tid == 0) {
    int base = 0;
    for (int x = 0; x < kNumXcd; ++x) {
      int cnt;
      if (sorted) {
        cnt = s_fill[x];
      } else {
        int lo = (int)((long long)x * n / kNumXcd), hi = (int)((long long)(x + 1) * n / kNumXcd);
        int plo = lo < n ? scratch[lo] : (int)s_total;
        int phi = hi < n ? scratch[hi] : (int)s_total;
        cnt = phi - plo;
      }
      st->base[x] = base;
      st->count[x] = cnt;
      st->counters[x] = 0;
      base += cnt;
    }
    st->status = 0;
    st->total = (int)s_total;
  }
  __syncthreads();

  // D: write the items of each group, q-tiles longest first, heads inner
  for (int i = tid; i < n; i += kPrepassThreads) {
    int b = i / num_kv_heads;
    int g = i % num_kv_heads;
    int L = cu[b + 1] - cu[b];
    int nqt = L > 0 ? (L + bm - 1) / bm : 0;
    int pos;
    if (sorted) {
      int base = 0;
      for (int x = 0; x < s_bin[i]; ++x) base += s_fill[x];
      pos = base + s_off[i];
    } else {
      pos = scratch[i];  // queues are contiguous in index order
    }
    for (int qt = nqt - 1; qt >= 0; --qt)
      for (int hh = 0; hh < group; ++hh)
        table[pos++] = make_int2(b, ((g * group + hh) << 20) | qt);
  }
}

__global__ __launch_bounds__(256) void sched_visit_kernel(const int32_t* __restrict__ cu,
                                                           int batch, int num_heads, int tiles,
                                                           const int2* __restrict__ table,
                                                           SchedState* __restrict__ st,
                                                           int* __restrict__ visits) {
  __shared__ int2 s_slot[2];
  int queue = blockIdx.x % kNumXcd, tried = 0;
  for (int it = 0;; ++it) {
    if (threadIdx.x == 0) {
      int2 e;
      s_slot[it & 1] = fetch_item(st, table, queue, tried, e) ? e : make_int2(-1, 0);
    }
    __syncthreads();
    int2 e = s_slot[it & 1];
    if (e.x < 0) break;
    WorkItem w = decode_item(e);
    if (threadIdx.x == 0 && w.b < batch && w.h < num_heads && w.qt < tiles)
      atomicAdd(&visits[(w.h * batch + w.b) * tiles + w.qt], 1);
  }
}

}  // namespace

hipError_t launch_prepass(const int32_t* cu, int batch, int num_heads, int num_kv_heads,
                          int causal, int bm, int bn, int capacity, int2* table,
                          SchedState* st, int* scratch, hipStream_t stream) {
  hipLaunchKernelGGL(sched_prepass_kernel, dim3(1), dim3(kPrepassThreads), 0, stream, cu, batch,
                     num_heads, num_kv_heads, causal, bm, bn, capacity, table, st, scratch);
  return hipGetLastError();
}

hipError_t launch_sched_visit(const int32_t* cu, int batch, int num_heads, int tiles,
                              const int2* table, SchedState* st, int* visits, int grid,
                              hipStream_t stream) {
  hipLaunchKernelGGL(sched_visit_kernel, dim3(grid), dim3(256), 0, stream, cu, batch, num_heads,
                     tiles, table, st, visits);
  return hipGetLastError();
}

}  // namespace mha
