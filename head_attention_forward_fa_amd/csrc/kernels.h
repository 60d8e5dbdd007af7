// Host-side launchers of the device kernels (internal to the library; the
// public C ABI is include/mha_fwd.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace mha {

// Query-tile heights of the two kernel families (rows of Q per work item).
constexpr int kBlockM_Mfma = 256;
constexpr int kBlockN_Mfma = 64;
constexpr int kBlockM_F32 = 32;
constexpr int kBlockN_F32 = 32;

// chunk: groups per chunk of a queue (>= 1), see prepass_chunk.
// Refuses (status 1, empty queues) when a length is negative or above
// max_seqlen, or when the items exceed `capacity`.
hipError_t launch_prepass(const int32_t* cu, int batch, int max_seqlen, int num_heads,
                          int num_kv_heads, int causal, int bm, int bn, int num_splits,
                          int capacity, int chunk, i32x4* table, SchedState* st, int* scratch,
                          hipStream_t stream);

// Groups per queue chunk.  Causal: 8 groups (their longest q-tiles first:
// the CUs then finish close together; measured against the whole queue as
// one chunk, equal on causal B4 H32 S4096 and 3.7% faster on causal B16 H32
// S1024, where fewer groups in flight share the XCD's L2 better).
// Non-causal: one group (all its q-tiles cost the same; consecutive items of
// one group share their K/V in the L2, measured 6-8% faster than
// interleaving the groups).
// causal: 8 groups per chunk for MHA; with GQA a group holds `group` query
// heads' items, so the chunk shrinks to keep about as many items per chunk
// (ragged GQA causal, Hq 32 / Hkv 8: +1.4%).  Sequences of more than 16
// query tiles (`tiles` = ceil(max_seqlen / block_m)) shrink it by (16 /
// tiles)^2 more: a group's K/V then spans several L2s' worth, and fewer
// groups in flight per XCD keep their re-reads in the L2 (nope+rope causal
// B2 H16 S8192: chunks of 2 instead of 8, L2 fills from 1.21 GB to 0.62 GB
// per launch at the same speed; ragged GQA and B1 H32 S16384 unchanged).
inline int prepass_chunk(int causal, int group, int tiles) {
  int c = causal ? (group >= 8 ? 1 : 8 / group) : 1;
  if (causal && tiles > 16) c = c * 256 / (tiles * tiles);
  return c < 1 ? 1 : c;
}

// protocol: 0 reserve() / resolve() placed as the float32 kernel places
// them, 1 as the bf16 / fp8 kernel does (see sched_visit_kernel)
hipError_t launch_sched_visit(int batch, int num_heads, int tiles, int protocol,
                              const i32x4* table, SchedState* st, int* visits, int grid,
                              hipStream_t stream);

// Per-row fp8 quantisation (quant.hip): rows x cols input (bf16 bits or
// float32), cols % 8 == 0, 8 <= cols <= 512.
hipError_t launch_fp8_quant(const void* x, bool bf16, int64_t rows, int cols, uint8_t* codes,
                            float* scales, hipStream_t stream);

// Split-KV merge (combine.hip): o_part [num_splits, T, H, Dv] (float32, or
// bfloat16 with part16) and lse_part [num_splits, H, T] -> o [T, H, Dv] (bf16
// or float32), lse [H, T].  With `sched` set, nothing is written when the
// prepass refused the call.
hipError_t launch_combine(const void* o_part, bool part16, const float* lse_part, int num_splits,
                          int T, const int32_t* t_out, int H, int dv, bool bf16_out, void* o,
                          float* lse, const SchedState* sched, hipStream_t stream);

// A kernel variant: its launcher and its occupancy (resident workgroups per
// CU at its LDS and register footprint, computed once per device).
struct Variant {
  hipError_t (*launch)(const AttnParams& p, int grid, hipStream_t stream);
  int (*blocks_per_cu)();
  int block_m;
  int block_n;
  int lds_bytes;
  // split-KV instantiation (partial results per key range); null if none
  hipError_t (*launch_split)(const AttnParams& p, int grid, hipStream_t stream);
};

// Lookup of the compiled variant for (dtype, Dn, Dr, Dv); nullptr if none.
const Variant* find_variant(int dtype, int dn, int dr, int dv);

// Per-family tables (defined next to each kernel family).
const Variant* find_variant_f32(int dn, int dr, int dv);
const Variant* find_variant_bf16(int dn, int dr, int dv);
const Variant* find_variant_fp8(int dn, int dr, int dv, bool fast);

}  // namespace mha
