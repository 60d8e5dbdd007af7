// Split-KV merge: the partial results of a query row over disjoint key
// ranges (O normalised over its range, float32 or bfloat16, and that range's
// LSE) add up through their exponential sums:
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
// HBM-bound: per (token, head) row, num_splits x (Dv x {4, 2} + 4) bytes
// read, Dv x {2, 4} + 4 written.  A row is spread over Dv / 4 (float32
// partials) or Dv / 8 (bfloat16) lanes, 16 bytes of each partial per lane; the
// split loop reads the partials' LSEs first (the same few bytes for all lanes
// of a row) and then streams the O rows.
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
// refusal (status != 0: no partial was written) leaves o and lse untouched;
// PART16: the partial O rows are bfloat16.  Each lane takes 16 bytes of each
// partial row: 4 float32 or 8 bfloat16 values.
template <bool PART16>
constexpr int values_per_lane() {
  return PART16 ? 8 : 4;
}
template <int DV, bool BF16, bool PART16>
__global__ __launch_bounds__(kCombineThreads) void combine_splits_kernel(
    const void* __restrict__ o_part, const float* __restrict__ lse_part, int num_splits, int T,
    const int32_t* __restrict__ t_out, int H, void* __restrict__ o, float* __restrict__ lse,
    const SchedState* __restrict__ sched) {
  if (sched && sched->status != 0) return;
  constexpr int VPL = values_per_lane<PART16>();
  constexpr int LPR = DV / VPL;  // lanes per row
  constexpr int RPB = kCombineThreads / LPR;
  const int c = threadIdx.x % LPR;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;  // row = t * H + h
  if (row >= (long long)T * H) return;
  const int t = (int)(row / H), h = (int)(row % H);
  const int Tn = t_out ? min(*t_out, T) : T;
  if (t >= Tn) return;
  constexpr int EB = PART16 ? 2 : 4;  // bytes per partial value
  const size_t split_stride_o = (size_t)T * H * DV * EB;
  const size_t split_stride_l = (size_t)H * T;
  const float* lp = lse_part + (size_t)h * T + t;
  float m = -INFINITY;
  for (int sp = 0; sp < num_splits; ++sp) m = fmaxf(m, lp[sp * split_stride_l]);
  float acc[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) acc[i] = 0.f;
  float total = 0.f;
  if (m > -INFINITY) {
    // four partials' loads in flight at a time; an empty partial (LSE -inf)
    // is loaded too but selected away, so whatever it holds adds nothing
    const char* op = static_cast<const char*>(o_part) + ((size_t)row * DV + VPL * c) * EB;
    for (int sp0 = 0; sp0 < num_splits; sp0 += 4) {
      i32x4 x[4];
      float wgt[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int sp = sp0 + u;
        x[u] = sp < num_splits ? *reinterpret_cast<const i32x4*>(op + sp * split_stride_o)
                               : i32x4{0, 0, 0, 0};
        const float ls = sp < num_splits ? lp[sp * split_stride_l] : -INFINITY;
        wgt[u] = ls > -INFINITY ? __expf(ls - m) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        total += wgt[u];
        if (wgt[u] > 0.f) {
#pragma unroll
          for (int i = 0; i < VPL; ++i) {
            // (bfloat16 -> float32: the bits in the upper half)
            const uint32_t d = (uint32_t)x[u][PART16 ? i / 2 : i];
            const float val = !PART16 ? __uint_as_float(d)
                                      : __uint_as_float(i % 2 ? d & 0xFFFF0000u : d << 16);
            acc[i] += wgt[u] * val;
          }
        }
      }
    }
  }
  const float inv = total > 0.f ? 1.f / total : 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) acc[i] *= inv;
  if constexpr (BF16) {
    uint16_t* dst = static_cast<uint16_t*>(o) + (size_t)row * DV + VPL * c;
    if constexpr (VPL == 8)
      *reinterpret_cast<i32x4*>(dst) =
          i32x4{(int)pack_bf16x2(acc[0], acc[1]), (int)pack_bf16x2(acc[2], acc[3]),
                (int)pack_bf16x2(acc[4], acc[5]), (int)pack_bf16x2(acc[6], acc[7])};
    else
      *reinterpret_cast<i32x2*>(dst) =
          i32x2{(int)pack_bf16x2(acc[0], acc[1]), (int)pack_bf16x2(acc[2], acc[3])};
  } else {
    float* dst = static_cast<float*>(o) + (size_t)row * DV + VPL * c;
#pragma unroll
    for (int i = 0; i < VPL; i += 4)
      *reinterpret_cast<f32x4*>(dst + i) = f32x4{acc[i], acc[i + 1], acc[i + 2], acc[i + 3]};
  }
  if (c == 0) lse[(size_t)h * Tn + t] = total > 0.f ? m + __logf(total) : -INFINITY;
}

template <int DV, bool BF16, bool PART16>
hipError_t launch_dv(const void* o_part, const float* lse_part, int num_splits, int T,
                     const int32_t* t_out, int H, void* o, float* lse, const SchedState* sched,
                     hipStream_t stream) {
  constexpr int RPB = kCombineThreads / (DV / values_per_lane<PART16>());
  const long long rows = (long long)T * H;
  const long long blocks = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((combine_splits_kernel<DV, BF16, PART16>), dim3((unsigned)blocks),
                     dim3(kCombineThreads), 0, stream, o_part, lse_part, num_splits, T, t_out, H,
                     o, lse, sched);
  return hipGetLastError();
}

template <int DV>
hipError_t launch_dv(const void* o_part, bool part16, const float* lse_part, int num_splits,
                     int T, const int32_t* t_out, int H, bool bf16_out, void* o, float* lse,
                     const SchedState* sched, hipStream_t stream) {
  if (part16)
    return bf16_out ? launch_dv<DV, true, true>(o_part, lse_part, num_splits, T, t_out, H, o, lse,
                                                sched, stream)
                    : launch_dv<DV, false, true>(o_part, lse_part, num_splits, T, t_out, H, o, lse,
                                                 sched, stream);
  return bf16_out ? launch_dv<DV, true, false>(o_part, lse_part, num_splits, T, t_out, H, o, lse,
                                               sched, stream)
                  : launch_dv<DV, false, false>(o_part, lse_part, num_splits, T, t_out, H, o, lse,
                                                sched, stream);
}

}  // namespace

hipError_t launch_combine(const void* o_part, bool part16, const float* lse_part, int num_splits,
                          int T, const int32_t* t_out, int H, int dv, bool bf16_out, void* o,
                          float* lse, const SchedState* sched, hipStream_t stream) {
  if (dv == 64)
    return launch_dv<64>(o_part, part16, lse_part, num_splits, T, t_out, H, bf16_out, o, lse,
                         sched, stream);
  if (dv == 128)
    return launch_dv<128>(o_part, part16, lse_part, num_splits, T, t_out, H, bf16_out, o, lse,
                          sched, stream);
  return hipErrorInvalidValue;
}

}  // namespace mha
