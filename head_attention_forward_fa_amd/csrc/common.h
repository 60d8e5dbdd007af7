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

// A work item of the persistent scheduler: sequence b, query head h, query
// tile qt.  Packed as {b, (h << 20) | qt}.
struct WorkItem {
  int b, h, qt;
};
__device__ __forceinline__ WorkItem decode_item(int2 e) {
  return WorkItem{e.x, (int)((unsigned)e.y >> 20), e.y & 0xFFFFF};
}
constexpr int kMaxQTilesPerSeq = 1 << 20;
constexpr int kMaxHeads = 1 << 11;

// Scheduler state kept in device memory (the library workspace).
//   counters[x]  next index to hand out from queue x (one queue per XCD)
//   base[x], count[x]  queue x's slice of the work table
//   status       nonzero when the prepass refused the problem
struct SchedState {
  int counters[kNumXcd];
  int base[kNumXcd];
  int count[kNumXcd];
  int status;
  int total;
  int pad[6];
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
  const int2* table;
  SchedState* sched;
  int batch;
  int num_heads;
  int num_kv_heads;
  int group;          // num_heads / num_kv_heads
  int causal;
  float scale_log2;   // sigma * log2(e)
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
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) {
  return __builtin_amdgcn_ballot_w64(p) != 0;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Fetch the next work item for this workgroup.  Queue choice is XCD-aware:
// workgroup i is dispatched to XCD i % 8, so it drains queue i % 8 first
// (whose items share K/V and therefore that XCD's L2), then the others.
// Called by one thread; returns false when every queue is empty.
__device__ __forceinline__ bool fetch_item(SchedState* s, const int2* table, int& queue,
                                           int& tried, int2& out) {
  while (tried < kNumXcd) {
    int cnt = s->count[queue];
    if (cnt > 0) {
      int idx = atomicAdd(&s->counters[queue], 1);
      if (idx < cnt) {
        out = table[s->base[queue] + idx];
        return true;
      }
    }
    queue = (queue + 1) % kNumXcd;
    ++tried;
  }
  return false;
}

}  // namespace mha
