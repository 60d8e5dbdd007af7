// Device-side building blocks shared by the attention kernels and the
// scheduler: vector types, bf16 packing, cross-lane reductions, kernel
// parameter block.  gfx950 (CDNA4) only; wave size 64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mha {

constexpr int kWave = 64;
constexpr int kNumXcd = 8;          // MI355X: 8 accelerator complex dies, each with its own L2
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// A work item of the persistent scheduler: query tile qt of query head h
// over sequence b, whose tokens are s0 .. s0 + L - 1, against key split
// `split` of the tile's keys (split-KV; 0 when the keys are not split).  A
// table entry is the 16-byte vector {s0, L, (h << 20) | qt, (split << 24) |
// b}; L = -1 marks "no work left".
struct WorkItem {
  int s0, L, h, qt, b, split;
};
__device__ __forceinline__ WorkItem decode_item(const i32x4& e) {
  return WorkItem{e[0], e[1], (int)((unsigned)e[2] >> 20), e[2] & 0xFFFFF, e[3] & 0xFFFFFF,
                  (int)((unsigned)e[3] >> 24)};
}
constexpr int kMaxQTilesPerSeq = 1 << 20;
constexpr int kMaxHeads = 1 << 11;
constexpr int kMaxBatch = 1 << 24;
constexpr int kMaxSplits = 64;

// Scheduler state kept in device memory (the library workspace).  Each
// queue (one per XCD) sits on its own 256-byte line, so that the atomic
// adds of different queues never meet on one cache line.
//   counter      next index to hand out from the queue
//   base, count  the queue's slice of the work table
//   status       nonzero when the prepass refused the problem
struct alignas(256) SchedQueue {
  int counter;
  int base;
  int count;
  int pad[61];
};
struct SchedState {
  SchedQueue q[kNumXcd];
  int status;
  int total;
  int pad[62];
};

// Kernel parameters (one struct so the launch signature stays the same for
// every instantiation).
struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const void* q_rope;
  const void* k_rope;
  const float* q_scale;
  const float* k_scale;
  const int32_t* cu_seqlens;
  const i32x4* table;
  SchedState* sched;
  int batch;
  int num_heads;
  int num_kv_heads;
  int group;          // num_heads / num_kv_heads
  int causal;
  float scale_log2;   // sigma * log2(e)
  // split-KV: the keys of every query tile are cut into num_splits ranges
  // of whole key blocks; with o_part set, a work item writes its range's
  // partial result (float32 O normalised over the range, and its LSE) to
  // o_part [num_splits, T, Hq, Dv] / lse_part [num_splits, Hq, T] instead of
  // o / lse.
  int num_splits;
  int part_tokens;    // T of the partial layouts (rows past it are not written)
  float* o_part;
  float* lse_part;
  int max_seqlen;     // the caller's bound on every sequence length
  int part_bf16;      // o_part holds bfloat16 values instead of float32
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (lo in bits 0..15), round to nearest even
// (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// acc + a.lo + a.hi for a packed bf16 pair (v_dot2_f32_bf16 against 1.0).
__device__ __forceinline__ float add_bf16x2(uint32_t a, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), one, acc, false);
}

// Buffer resource over [base, base + bytes): loads at offsets past the end
// return zeros, with no branch (raw buffer, stride 0; gfx9 dword3 config).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ i32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// Combine a value across the two 32-lane halves of the wave (lanes i and
// i ^ 32 hold the same query row in the MFMA output layout).
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second; with both operands equal to x, every lane ends
// with the pair {x[i % 32], x[i % 32 + 32]}, so both lanes of a pair compute
// the same combination in the same order.
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // the operands are scores or -inf, never NaN: a plain v_max_f32 (fmaxf
  // would first quiet both operands, two more vector ops)
  float m;
  asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(__uint_as_float(r[0])), "v"(__uint_as_float(r[1])));
  return m;
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) {
  return __builtin_amdgcn_ballot_w64(p) != 0;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Work-item source of one workgroup, driven by one wave (all its lanes take
// the same path; only lane 0 touches the counters).  Queue choice is
// XCD-aware: workgroup i is dispatched to XCD i % 8, so it drains queue
// i % 8 first (whose items share K/V and therefore that XCD's L2), then the
// others that still have work.  It is driven in two steps, reserve() (an
// atomic add whose result is not waited for) and resolve() (the entry of
// the reserved index), which a kernel places apart inside its current item
// so that neither memory round trip sits between two items: the bf16 / fp8
// kernel near the item's end (the next item is then chosen late, and the
// queue deals like a list scheduler over the queue order), the float32
// kernel at the item's start and after its key blocks.
struct Fetcher {
  int queue, cnt, base;  // wave-uniform
  int pend;              // lane 0: the reserved index (in flight until resolved)

  __device__ __forceinline__ void open_queue(const SchedState* st) {
    cnt = __builtin_amdgcn_readfirstlane(st->q[queue].count);
    base = __builtin_amdgcn_readfirstlane(st->q[queue].base);
  }
  __device__ __forceinline__ void reserve(SchedState* st) {
    pend = 0;
    if (__lane_id() == 0) pend = atomicAdd(&st->q[queue].counter, 1);
  }
  __device__ __forceinline__ void init(SchedState* st) {
    queue = blockIdx.x % kNumXcd;
    open_queue(st);
    reserve(st);
  }
  // The first queue after the current one (in queue order, wrapping round
  // to the current one last) whose counter has not reached its count, or -1
  // when every queue is drained.  All queues are read at once (lane i reads
  // queue + 1 + i), with loads that go past the compute unit's cache to the
  // L2 where the atomic adds happen, so a drained workgroup finds the work
  // left, or that there is none, in one round trip instead of visiting the
  // queues one by one.
  __device__ __forceinline__ int next_open_queue(SchedState* st) {
    const int lane = __lane_id();
    bool open = false;
    if (lane < kNumXcd) {
      const int qq = (queue + 1 + lane) % kNumXcd;
      const int c = __hip_atomic_load(&st->q[qq].counter, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
      open = c < st->q[qq].count;
    }
    const uint64_t b = __builtin_amdgcn_ballot_w64(open);
    if (b == 0) return -1;
    return (queue + 1 + (int)__builtin_ctzll(b)) % kNumXcd;
  }
  // Entry of the reserved index; while the queue is exhausted, moves to the
  // next queue that has work left (and reserves there); L = -1 when every
  // queue is drained.  A reservation that loses the race for a queue's last
  // items only moves that counter past its count, so the scan ends.
  __device__ __forceinline__ i32x4 resolve(SchedState* st, const i32x4* table) {
    for (;;) {
      const int idx = __builtin_amdgcn_readfirstlane(pend);
      if (idx < cnt) return table[base + idx];
      const int nq = next_open_queue(st);
      if (nq < 0) return i32x4{0, -1, 0, 0};
      queue = nq;
      open_queue(st);
      reserve(st);
    }
  }
};

}  // namespace mha
