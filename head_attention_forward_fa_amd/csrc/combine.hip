// Split-KV merge: the partial results of a query row over disjoint key
// ranges (float32 O normalised over its range, and that range's LSE) add up
// through their exponential sums:
//
//   LSE = log sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s
//
// evaluated with the largest LSE_s factored out; a partial with LSE_s = -inf
// (no visible key in its range) weighs nothing, and a row whose partials are
// all empty gets O = 0, LSE = -inf.  The pages keep the running softmax
// statistics of a row in a per-row correction buffer (SM100AttentionSMem,
// Methods: correction_smem) and name the split count (comptime members:
// MiscMBarsType takes the config's splitk_partitions); the merge itself is
// this library's.
//
// HBM-bound: per (token, head) row, num_splits x (Dv x 4 + 4) bytes read,
// Dv x {2, 4} + 4 written.  A row is spread over Dv / 4 lanes (16 bytes of
// each partial per lane); the split loop reads the partials' LSEs first (the
// same few bytes for all lanes of a row) and then streams the O rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr int kCombineThreads = 256;

// T: tokens of the partials' layout; t_out (device, may be null): tokens of
// the output when fewer (the rest of the partial rows are not merged), else T;
// sched (may be null): the scheduler state of the split attention call, whose
// refusal (status != 0: no partial was written) leaves o and lse untouched
template <int DV, bool BF16>
__global__ __launch_bounds__(kCombineThreads) void combine_splits_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part, int num_splits, int T,
    const int32_t* __restrict__ t_out, int H, void* __restrict__ o, float* __restrict__ lse,
    const SchedState* __restrict__ sched) {
  if (sched && sched->status != 0) return;
  constexpr int LPR = DV / 4;  // lanes per row
  constexpr int RPB = kCombineThreads / LPR;
  const int c = threadIdx.x % LPR;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;  // row = t * H + h
  if (row >= (long long)T * H) return;
  const int t = (int)(row / H), h = (int)(row % H);
  const int Tn = t_out ? min(*t_out, T) : T;
  if (t >= Tn) return;
  const size_t split_stride_o = (size_t)T * H * DV;
  const size_t split_stride_l = (size_t)H * T;
  const float* lp = lse_part + (size_t)h * T + t;
  float m = -INFINITY;
  for (int sp = 0; sp < num_splits; ++sp) m = fmaxf(m, lp[sp * split_stride_l]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float total = 0.f;
  if (m > -INFINITY) {
    // four partials' loads in flight at a time; an empty partial (LSE -inf)
    // is loaded too but selected away, so whatever it holds adds nothing
    const float* op = o_part + (size_t)row * DV + 4 * c;
    for (int sp0 = 0; sp0 < num_splits; sp0 += 4) {
      f32x4 x[4];
      float wgt[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int sp = sp0 + u;
        x[u] = sp < num_splits ? *reinterpret_cast<const f32x4*>(op + sp * split_stride_o)
                               : f32x4{0.f, 0.f, 0.f, 0.f};
        const float ls = sp < num_splits ? lp[sp * split_stride_l] : -INFINITY;
        wgt[u] = ls > -INFINITY ? __expf(ls - m) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        total += wgt[u];
        if (wgt[u] > 0.f) acc += wgt[u] * x[u];
      }
    }
  }
  const float inv = total > 0.f ? 1.f / total : 0.f;
  acc *= inv;
  if constexpr (BF16) {
    const uint32_t lo = pack_bf16x2(acc[0], acc[1]), hi = pack_bf16x2(acc[2], acc[3]);
    *reinterpret_cast<i32x2*>(static_cast<uint16_t*>(o) + (size_t)row * DV + 4 * c) =
        i32x2{(int)lo, (int)hi};
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(o) + (size_t)row * DV + 4 * c) = acc;
  }
  if (c == 0) lse[(size_t)h * Tn + t] = total > 0.f ? m + __logf(total) : -INFINITY;
}

template <int DV, bool BF16>
hipError_t launch_dv(const float* o_part, const float* lse_part, int num_splits, int T,
                     const int32_t* t_out, int H, void* o, float* lse, const SchedState* sched,
                     hipStream_t stream) {
  constexpr int RPB = kCombineThreads / (DV / 4);
  const long long rows = (long long)T * H;
  const long long blocks = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((combine_splits_kernel<DV, BF16>), dim3((unsigned)blocks),
                     dim3(kCombineThreads), 0, stream, o_part, lse_part, num_splits, T, t_out, H,
                     o, lse, sched);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const float* o_part, const float* lse_part, int num_splits, int T,
                          const int32_t* t_out, int H, int dv, bool bf16_out, void* o, float* lse,
                          const SchedState* sched, hipStream_t stream) {
  if (dv == 64)
    return bf16_out ? launch_dv<64, true>(o_part, lse_part, num_splits, T, t_out, H, o, lse,
                                          sched, stream)
                    : launch_dv<64, false>(o_part, lse_part, num_splits, T, t_out, H, o, lse,
                                           sched, stream);
  if (dv == 128)
    return bf16_out ? launch_dv<128, true>(o_part, lse_part, num_splits, T, t_out, H, o, lse,
                                           sched, stream)
                    : launch_dv<128, false>(o_part, lse_part, num_splits, T, t_out, H, o, lse,
                                            sched, stream);
  return hipErrorInvalidValue;
}

}  // namespace mha
