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
//     per split, next to each other).  Groups are (sequence, KV head): the
//     query heads sharing a KV head sit next to each other.  Groups are
//     ranked by cost (bitonic sort in LDS) and dealt to 8 queues, one per
//     XCD, largest first in a snake order so the queues carry equal work.
//     A queue runs chunk by chunk (a chunk: consecutive groups), a chunk in
//     rounds: round k holds the k-th longest q-tile of each of its groups
//     (causal cost grows with the tile index).  Causal: chunks of 8
//     groups (8 / query heads per KV head with GQA, so that a chunk holds
//     about as many items), so each chunk, and the queue, drains with short
//     items and the CUs finish close together.  Non-causal: one group per chunk (equal
//     costs; a group's items share their K/V in the XCD's L2).
//   * the attention kernel is launched with about (CUs x resident
//     workgroups) workgroups; each pops items from queue blockIdx % 8 with
//     one atomic add, then helps the other queues once its own is empty.
//
// Cost of an item, in BN-key blocks: causal ceil(min(L, (qt+1)*BM) / BN),
// non-causal ceil(L / BN).
#include <climits>

#include "common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr int kPrepassThreads = 1024;
constexpr int kSortedMax = 2048;  // groups ranked in LDS up to this count
constexpr int kRankDirect = 384;  // up to this many: rank by counting (else sort)

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
// rank of the group at position j of queue x under the snake deal
__device__ __forceinline__ int queue_rank(int x, int j) {
  return 2 * kNumXcd * (j >> 1) + ((j & 1) ? 2 * kNumXcd - 1 - x : x);
}

__global__ __launch_bounds__(kPrepassThreads) void sched_prepass_kernel(
    const int32_t* __restrict__ cu, int batch, int max_seqlen, int num_heads, int num_kv_heads,
    int causal, int bm, int bn, int num_splits, int capacity, int chunk,
    i32x4* __restrict__ table, SchedState* __restrict__ st, int* __restrict__ scratch) {
  __shared__ long long s_cost[kSortedMax];
  __shared__ int s_items[kSortedMax];   // group -> item count
  __shared__ int s_irank[kSortedMax];   // rank -> item count
  __shared__ int s_grank[kSortedMax];   // group -> rank
  __shared__ int s_off[kSortedMax];     // rank -> offset inside its queue
  __shared__ int s_gidx[kSortedMax];    // rank -> group (after the sort)
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
  // (in 64 bits: garbage lengths must not wrap past the capacity check).  A
  // length above max_seqlen refuses the call: the split-KV partials are laid
  // out for batch x max_seqlen tokens.
  long long my_items = 0;
  int my_rmax = 0;  // most q-tiles of a group
  for (int i = tid; i < n; i += kPrepassThreads) {
    const int b = i / num_kv_heads;
    const int L = cu[b + 1] - cu[b];
    const int nqt = L > 0 ? (L + bm - 1) / bm : 0;
    if (L < 0 || L > max_seqlen || nqt >= kMaxQTilesPerSeq) s_bad = 1;
    const long long items64 = (long long)nqt * group * num_splits;
    // (stored as int only for use after the capacity check, where it fits)
    const int items = (int)min(items64, (long long)INT_MAX);
    my_items += items64;
    my_rmax = max(my_rmax, nqt);
    if (sorted) {
      s_cost[i] = group_cost(L, bm, bn, causal) * group;
      s_items[i] = items;
    } else {
      scratch[i] = items;
    }
  }
  for (int d = kWave / 2; d > 0; d >>= 1) {
    my_items += __shfl_down(my_items, d);
    my_rmax = max(my_rmax, __shfl_down(my_rmax, d));
  }
  __shared__ long long s_wsum[kPrepassThreads / kWave];
  __shared__ int s_wmax[kPrepassThreads / kWave];
  if ((tid & (kWave - 1)) == 0) {
    s_wsum[tid / kWave] = my_items;
    s_wmax[tid / kWave] = my_rmax;
  }
  __syncthreads();
  long long total = 0;
  int rmax = 0;
  for (int w = 0; w < kPrepassThreads / kWave; ++w) {
    total += s_wsum[w];
    rmax = max(rmax, s_wmax[w]);
  }
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
    // B: rank groups by cost, largest first (ties by index).  Equal costs
    // (a uniform batch): the index order.  Up to kRankDirect groups: each
    // group counts the groups ahead of it.  More: bitonic sort of (cost,
    // index) in LDS, padded to a power of two with cost -1.
    __shared__ int s_uniform;
    if (tid == 0) s_uniform = 1;
    __syncthreads();
    for (int i = tid + 1; i < n; i += kPrepassThreads)
      if (s_cost[i] != s_cost[0]) s_uniform = 0;
    __syncthreads();
    const bool direct = s_uniform || n <= kRankDirect;
    int np = 1;
    while (np < n) np <<= 1;
    for (int i = tid; i < np; i += kPrepassThreads) {
      if (i >= n) s_cost[i] = -1;
      s_gidx[i] = i;
    }
    __syncthreads();
    if (direct && !s_uniform) {
      for (int i = tid; i < n; i += kPrepassThreads) {
        const long long c = s_cost[i];
        int rank = 0;
#pragma unroll 8
        for (int j = 0; j < n; ++j) {
          const long long cj = s_cost[j];
          rank += (cj > c) || (cj == c && j < i);
        }
        s_gidx[rank] = i;
      }
      __syncthreads();
    }
    for (int k = 2; k <= (direct ? 1 : np); k <<= 1)
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int t = tid; t < np; t += kPrepassThreads) {
          const int u = t ^ j;
          if (u > t) {
            const long long ct = s_cost[t], cu2 = s_cost[u];
            const int it = s_gidx[t], iu = s_gidx[u];
            const bool t_first = ct > cu2 || (ct == cu2 && it < iu);
            if (((t & k) == 0) != t_first) {  // (t & k) == 0: this run goes in final order
              s_cost[t] = cu2;
              s_cost[u] = ct;
              s_gidx[t] = iu;
              s_gidx[u] = it;
            }
          }
        }
        __syncthreads();
      }
    for (int r = tid; r < n; r += kPrepassThreads) {
      const int i = s_gidx[r];
      s_grank[i] = r;
      s_irank[r] = s_items[i];
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

  // E: write the items of each group: per q-tile, its query heads (and
  // their key splits) next to each other.  Sorted path: a queue is cut into
  // chunks of `chunk` consecutive groups; a chunk runs in rounds, round k
  // holding the k-th longest q-tile of each of its groups that has one, in
  // queue order.  The queue's groups come in non-increasing q-tile count
  // (cost order implies it), so round k is the chunk's first C_k groups,
  // and the rounds before it hold sum_j min(nqt_j, k) q-tiles.  Unsorted
  // path: each group's q-tiles back to back, longest first.
  // One (group, round) pair per thread and step: a group's rounds spread
  // over the threads.
  const int u = group * num_splits;  // items per (group, q-tile)
  const int qlen = 2 * ((n + 2 * kNumXcd - 1) / (2 * kNumXcd));  // queue positions, upper bound
  const long long npairs = (long long)n * rmax;
  for (long long t = tid; t < npairs; t += kPrepassThreads) {
    const int i = (int)(t / rmax);
    const int k = (int)(t % rmax);
    const int b = i / num_kv_heads;
    const int g = i % num_kv_heads;
    const int s0 = cu[b];
    const int L = cu[b + 1] - s0;
    const int nqt = L > 0 ? (L + bm - 1) / bm : 0;
    if (k >= nqt) continue;
    const int qt = nqt - 1 - k;
    long long pos;
    if (sorted) {
      const int r = s_grank[i];
      const int x = snake_bin(r);
      const int jq = 2 * (r / (2 * kNumXcd)) + (r % (2 * kNumXcd) < kNumXcd ? 0 : 1);
      // the chunk [c0, c1) of queue positions holding this group
      const int c0 = jq - jq % chunk;
      const int c1 = min(c0 + chunk, qlen);
      // items at queue positions < j (positions past the queue's end map to
      // ranks >= n)
      auto prefix = [&](int j) -> long long {
        const int rr = queue_rank(x, j);
        return rr < n ? s_off[rr] : s_fill[x];
      };
      // C_k: the first chunk position whose group has at most k q-tiles
      // (none before this group's position: those have at least as many)
      const long long lim = (long long)k * u;
      int lo = jq + 1, hi = c1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const int rm = queue_rank(x, mid);
        const long long a = rm < n ? s_irank[rm] : 0;
        if (a > lim)
          lo = mid + 1;
        else
          hi = mid;
      }
      pos = s_base[x] + prefix(c0) + lim * (lo - c0) + (prefix(c1) - prefix(lo)) +
            (long long)(jq - c0) * u;
    } else {
      pos = scratch[i] + (long long)k * u;  // queues are contiguous in index order
    }
    for (int hh = 0; hh < group; ++hh)
      for (int sp = 0; sp < num_splits; ++sp, ++pos)
        if (pos < total)
          table[pos] = i32x4{s0, L, ((g * group + hh) << 20) | qt, (sp << 24) | b};
  }
}

// protocol 0: the next item reserved when the current one starts and its
// entry read after a workgroup barrier (the float32 kernel's placement);
// protocol 1: reserve() and resolve() at the places the matrix-core
// attention kernel uses them: an item of nb key blocks (here nb = qt % 5, so
// that items with no blocks occur too) reserves at block max(0, nb - 3) and
// reads the entry at block max(0, nb - 1), with a workgroup barrier per block;
// an item with no blocks does both after its (empty) block loop.
__global__ __launch_bounds__(256) void sched_visit_kernel(int batch, int num_heads, int tiles,
                                                           int protocol,
                                                           const i32x4* __restrict__ table,
                                                           SchedState* __restrict__ st,
                                                           int* __restrict__ visits) {
  __shared__ i32x4 s_item[2];
  Fetcher fetch;
  const bool w0 = threadIdx.x < kWave;
  if (w0) {
    fetch.init(st);
    const i32x4 e0 = fetch.resolve(st, table);
    if (threadIdx.x == 0) s_item[0] = e0;
  }
  for (int it = 0;; ++it) {
    __syncthreads();
    const i32x4 e = s_item[it & 1];
    if (e[1] < 0) break;
    const WorkItem w = decode_item(e);
    i32x4 nxt = {0, -1, 0, 0};
    if (protocol == 0) {
      if (w0) fetch.reserve(st);
      __syncthreads();
      if (w0) nxt = fetch.resolve(st, table);
    } else {
      const int nb = w.qt % 5;
      const int j_res = max(0, nb - 3), j_get = max(0, nb - 1);
      for (int j = 0; j < nb; ++j) {
        if (w0) {
          if (j == j_res) fetch.reserve(st);
          if (j == j_get) nxt = fetch.resolve(st, table);
        }
        __syncthreads();
      }
      if (w0 && nb <= 0) {
        fetch.reserve(st);
        nxt = fetch.resolve(st, table);
      }
    }
    if (threadIdx.x == 0) {
      s_item[(it + 1) & 1] = nxt;
      if (w.b < batch && w.h < num_heads && w.qt < tiles)
        atomicAdd(&visits[(w.h * batch + w.b) * tiles + w.qt], 1);
    }
  }
}

}  // namespace

hipError_t launch_prepass(const int32_t* cu, int batch, int max_seqlen, int num_heads,
                          int num_kv_heads, int causal, int bm, int bn, int num_splits,
                          int capacity, int chunk, i32x4* table, SchedState* st, int* scratch,
                          hipStream_t stream) {
  if (chunk < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sched_prepass_kernel, dim3(1), dim3(kPrepassThreads), 0, stream, cu, batch,
                     max_seqlen, num_heads, num_kv_heads, causal, bm, bn, num_splits, capacity,
                     chunk, table, st, scratch);
  return hipGetLastError();
}

hipError_t launch_sched_visit(int batch, int num_heads, int tiles, int protocol,
                              const i32x4* table, SchedState* st, int* visits, int grid,
                              hipStream_t stream) {
  hipLaunchKernelGGL(sched_visit_kernel, dim3(grid), dim3(256), 0, stream, batch, num_heads,
                     tiles, protocol, table, st, visits);
  return hipGetLastError();
}

}  // namespace mha
