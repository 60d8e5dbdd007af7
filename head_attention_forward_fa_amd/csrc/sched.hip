// Persistent tile scheduler: the prepass that builds the work table and the
// diagnostic visit kernel.
//
// The pages give the scheduler as a trait (MHATileScheduler): it assigns
// work tiles to thread blocks, steps each block's state through the work
// across iterations of a persistent kernel, reports the launch grid, and is
// generic over an optional pointer to per-batch sequence-length offsets
// (Required methods: get_current_work_info, ValidLengthType); the active
// work index is published to the block through shared memory
// (initial_state), and advance() tells whether work remains.  The MI355X
// version:
//
//   * a one-workgroup prepass turns cu_seqlens into a table of work items
//     {s0, L, h, q-tile, b} (times the key splits under split-KV: one item
//     per split, next to each other).  Items are grouped by (sequence, KV head), so
//     that the query heads sharing a KV head and every q-tile of that
//     sequence sit next to each other; groups are dealt to 8 queues, one per
//     XCD, largest first in a snake order so the queues carry equal work;
//     inside a group the q-tiles run longest first (causal cost grows with
//     the tile index).
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
    int bm, int bn, int num_splits, int capacity, i32x4* __restrict__ table,
    SchedState* __restrict__ st, int* __restrict__ scratch) {
  __shared__ long long s_cost[kSortedMax];
  __shared__ int s_items[kSortedMax];   // group -> item count
  __shared__ int s_irank[kSortedMax];   // rank -> item count
  __shared__ int s_grank[kSortedMax];   // group -> rank
  __shared__ int s_off[kSortedMax];     // rank -> offset inside its queue
  __shared__ int s_fill[kNumXcd];
  __shared__ int s_base[kNumXcd];
  __shared__ int s_bad;

  const int tid = threadIdx.x;
  const int group = num_heads / num_kv_heads;
  const int n = batch * num_kv_heads;
  const bool sorted = n <= kSortedMax;
  if (tid == 0) s_bad = 0;
  __syncthreads();

  // A: per-group cost and item count; the item total by a block reduction
  // (in 64 bits: garbage lengths must not wrap past the capacity check)
  long long my_items = 0;
  for (int i = tid; i < n; i += kPrepassThreads) {
    const int b = i / num_kv_heads;
    const int L = cu[b + 1] - cu[b];
    const int nqt = L > 0 ? (L + bm - 1) / bm : 0;
    if (L < 0 || nqt >= kMaxQTilesPerSeq) s_bad = 1;
    const int items = nqt * group * num_splits;
    my_items += items;
    if (sorted) {
      s_cost[i] = group_cost(L, bm, bn, causal) * group;
      s_items[i] = items;
    } else {
      scratch[i] = items;
    }
  }
  for (int d = kWave / 2; d > 0; d >>= 1) my_items += __shfl_down(my_items, d);
  __shared__ long long s_wsum[kPrepassThreads / kWave];
  if ((tid & (kWave - 1)) == 0) s_wsum[tid / kWave] = my_items;
  __syncthreads();
  long long total = 0;
  for (int w = 0; w < kPrepassThreads / kWave; ++w) total += s_wsum[w];
  if (s_bad || total > (long long)capacity) {
    if (tid < kNumXcd) {
      st->q[tid].counter = 0;
      st->q[tid].base = 0;
      st->q[tid].count = 0;
    }
    if (tid == 0) {
      st->status = 1;
      st->total = 0;
    }
    return;
  }

  if (sorted) {
    // B: rank groups by cost, largest first (ties by index)
    for (int i = tid; i < n; i += kPrepassThreads) {
      const long long c = s_cost[i];
      int rank = 0;
#pragma unroll 8
      for (int j = 0; j < n; ++j) {
        const long long cj = s_cost[j];
        rank += (cj > c) || (cj == c && j < i);
      }
      s_grank[i] = rank;
      s_irank[rank] = s_items[i];
    }
    __syncthreads();
    // C: snake-deal ranks to queues (rank r -> queue snake_bin(r)); queue x
    // holds ranks x, 15-x, 16+x, 31-x, ...  One thread per queue walks its
    // ranks in order and lays them out back to back.
    if (tid < kNumXcd) {
      int off = 0;
      for (int r0 = 0; r0 < n; r0 += 2 * kNumXcd) {
        const int ra = r0 + tid, rb = r0 + 2 * kNumXcd - 1 - tid;
        if (ra < n) {
          s_off[ra] = off;
          off += s_irank[ra];
        }
        if (rb < n) {
          s_off[rb] = off;
          off += s_irank[rb];
        }
      }
      s_fill[tid] = off;
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
      const int i = c0 + tid;
      const int v = i < n ? scratch[i] : 0;
      s_scan[tid] = v;
      __syncthreads();
      for (int d = 1; d < kPrepassThreads; d <<= 1) {
        const int add = tid >= d ? s_scan[tid - d] : 0;
        __syncthreads();
        s_scan[tid] += add;
        __syncthreads();
      }
      if (i < n) scratch[i] = s_carry + s_scan[tid] - v;
      __syncthreads();
      if (tid == kPrepassThreads - 1) s_carry += s_scan[tid];
      __syncthreads();
    }
    if (tid < kNumXcd) {
      const int lo = (int)((long long)tid * n / kNumXcd);
      const int hi = (int)((long long)(tid + 1) * n / kNumXcd);
      const int plo = lo < n ? scratch[lo] : (int)total;
      const int phi = hi < n ? scratch[hi] : (int)total;
      s_fill[tid] = phi - plo;
    }
    __syncthreads();
  }

  // D: queue slices
  if (tid == 0) {
    int base = 0;
    for (int x = 0; x < kNumXcd; ++x) {
      s_base[x] = base;
      st->q[x].base = base;
      st->q[x].count = s_fill[x];
      st->q[x].counter = 0;
      base += s_fill[x];
    }
    st->status = 0;
    st->total = (int)total;
  }
  __syncthreads();

  // E: write the items of each group, q-tiles longest first, heads inner
  for (int i = tid; i < n; i += kPrepassThreads) {
    const int b = i / num_kv_heads;
    const int g = i % num_kv_heads;
    const int s0 = cu[b];
    const int L = cu[b + 1] - s0;
    const int nqt = L > 0 ? (L + bm - 1) / bm : 0;
    int pos;
    if (sorted) {
      const int r = s_grank[i];
      pos = s_base[snake_bin(r)] + s_off[r];
    } else {
      pos = scratch[i];  // queues are contiguous in index order
    }
    for (int qt = nqt - 1; qt >= 0; --qt)
      for (int hh = 0; hh < group; ++hh)
        for (int sp = 0; sp < num_splits; ++sp)
          table[pos++] = i32x4{s0, L, ((g * group + hh) << 20) | qt, (sp << 24) | b};
  }
}

__global__ __launch_bounds__(256) void sched_visit_kernel(int batch, int num_heads, int tiles,
                                                           const i32x4* __restrict__ table,
                                                           SchedState* __restrict__ st,
                                                           int* __restrict__ visits) {
  __shared__ i32x4 s_item[2];
  Fetcher fetch;
  const bool w0 = threadIdx.x < kWave;
  if (w0) {
    fetch.init(st);
    const i32x4 e0 = fetch.take(st, table);
    if (threadIdx.x == 0) s_item[0] = e0;
  }
  for (int it = 0;; ++it) {
    __syncthreads();
    const i32x4 e = s_item[it & 1];
    if (e[1] < 0) break;
    if (w0) {
      const i32x4 nxt = fetch.take(st, table);
      if (threadIdx.x == 0) {
        s_item[(it + 1) & 1] = nxt;
        const WorkItem w = decode_item(e);
        if (w.b < batch && w.h < num_heads && w.qt < tiles)
          atomicAdd(&visits[(w.h * batch + w.b) * tiles + w.qt], 1);
      }
    }
  }
}

}  // namespace

hipError_t launch_prepass(const int32_t* cu, int batch, int num_heads, int num_kv_heads,
                          int causal, int bm, int bn, int num_splits, int capacity,
                          i32x4* table, SchedState* st, int* scratch, hipStream_t stream) {
  hipLaunchKernelGGL(sched_prepass_kernel, dim3(1), dim3(kPrepassThreads), 0, stream, cu, batch,
                     num_heads, num_kv_heads, causal, bm, bn, num_splits, capacity, table, st,
                     scratch);
  return hipGetLastError();
}

hipError_t launch_sched_visit(int batch, int num_heads, int tiles, const i32x4* table,
                              SchedState* st, int* visits, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(sched_visit_kernel, dim3(grid), dim3(256), 0, stream, batch, num_heads,
                     tiles, table, st, visits);
  return hipGetLastError();
}

}  // namespace mha
