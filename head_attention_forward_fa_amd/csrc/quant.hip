// Per-token fp8 quantisation of Q / K rows: one float32 scale per row of D
// elements and the row's OCP E4M3 codes.  This is the step in front of the
// fp8 attention path, whose Q and K come as 8-bit codes with a per-token
// scale (SM100AttentionSMem, Parameters: scale_dtype_; Methods q_scale_smem /
// k_scale_smem).  Reading of how the codes are made (the pages leave it
// open):
//
//   scale = amax(|row|) / 448        (448 = largest finite E4M3; scale 1 for a
//                                     row of zeros)
//   code  = round-to-nearest-even E4M3 of clamp(x / scale, -448, 448)
//
// with IEEE float32 division, so the codes are exact functions of the input
// (computed as a reciprocal product where that provably rounds the same way,
// see the kernel).
//
// HBM-bound: each row is read once (D bf16 or float32 elements) and written
// once (D codes + 4 bytes of scale).  A row is spread over LPR lanes (8
// consecutive elements per lane, one 16- or 32-byte load), its amax is a
// reduction over those lanes by DPP moves and lane swaps (no LDS round
// trips), and each lane writes its 8 codes as one 8-byte store, so a wave
// moves 64 x 16 (bf16) contiguous bytes per load instruction.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr float kE4M3Max = 448.0f;
constexpr int kQuantThreads = 256;

// Two float32 values of magnitude below 464 -> two E4M3 codes in the low 16
// bits (first value in the low byte): v_cvt_pk_fp8_f32, round to nearest
// even, OCP E4M3 on gfx950.
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Max over each aligned group of LPR lanes (8 to 64), in every lane of the
// group: within a row of 16 lanes by DPP moves (swap neighbours, swap pairs,
// mirror the half-row, mirror the row), across rows by v_permlane16_swap
// and v_permlane32_swap.  The values are magnitudes (>= 0).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}
template <int LPR>
__device__ __forceinline__ float group_max(float x) {
  static_assert(LPR == 8 || LPR == 16 || LPR == 32 || LPR == 64, "lane group");
  x = fmaxf(x, dpp_mov<0xB1>(x));   // quad_perm [1, 0, 3, 2]
  x = fmaxf(x, dpp_mov<0x4E>(x));   // quad_perm [2, 3, 0, 1]
  x = fmaxf(x, dpp_mov<0x141>(x));  // row_half_mirror
  if constexpr (LPR >= 16) x = fmaxf(x, dpp_mov<0x140>(x));  // row_mirror
  if constexpr (LPR >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  if constexpr (LPR >= 64) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return x;
}

template <bool BF16>
__device__ __forceinline__ void load8(const void* x, size_t elem, float (&v)[8]) {
  if constexpr (BF16) {
    // (input read once, codes written once: streaming accesses, which keep
    // them from displacing what the L2 holds for other work)
    const i32x4 w =
        __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(x) + elem));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __builtin_bit_cast(float, (uint32_t)w[i] << 16);
      v[2 * i + 1] = __builtin_bit_cast(float, (uint32_t)w[i] & 0xFFFF0000u);
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + elem);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
}

// LPR lanes per row (a power of two, LPR * 8 >= cols); each group of LPR
// lanes takes NR rows, NR x 256 / LPR rows per workgroup, and issues the NR
// rows' loads before any arithmetic, so that more bytes are in flight per
// lane than one load's worth.
template <bool BF16, int LPR, int NR>
__global__ __launch_bounds__(kQuantThreads) void fp8_quant_rows_kernel(const void* __restrict__ x,
                                                                      int64_t rows, int cols,
                                                                      uint8_t* __restrict__ codes,
                                                                      float* __restrict__ scales) {
  constexpr int RPB = kQuantThreads / LPR;  // row groups per workgroup
  const int c = threadIdx.x % LPR;          // 8-element chunk of the row
  const int64_t row0 = ((int64_t)blockIdx.x * RPB + threadIdx.x / LPR) * NR;
  float v[NR][8];
  bool live[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    live[r] = row0 + r < rows && c * 8 < cols;
    if (live[r]) load8<BF16>(x, (size_t)(row0 + r) * cols + c * 8, v[r]);
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    float amax = 0.f;
    if (live[r]) {
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[r][i]));
    }
    amax = group_max<LPR>(amax);
    const float scale = amax > 0.f ? amax / kE4M3Max : 1.0f;
    if (!live[r]) continue;
    // x / scale, as its E4M3 rounding needs it: q = x * rcp(scale) is within
    // a few float32 ulps of the correctly rounded quotient, and for |q| >=
    // 2^-5 (E4M3 normals) the E4M3 rounding of q only depends on whether the
    // 20 mantissa bits below E4M3's 3 lie above or below their midpoint
    // 0x80000.  So q gives the same code as the quotient unless those bits
    // lie within 16 of the midpoint, or |q| < 2^-5; then the lane's eight
    // quotients are the IEEE divisions themselves.
    // (a scale below 2^-100 takes the divisions too: its reciprocal may not
    // be a normal float32)
    const float rs = __builtin_amdgcn_rcpf(scale);
    float q[8];
    bool exact = !(scale >= 7.888609052e-31f);  // 2^-100
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      q[i] = v[r][i] * rs;
      const uint32_t low = __builtin_bit_cast(uint32_t, q[i]) & 0xFFFFFu;
      exact = exact || !(fabsf(q[i]) >= 0.03125f) || (low - (0x80000u - 16u)) <= 32u;
    }
    if (exact) {
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = v[r][i] / scale;
    }
    // (no clamp to [-448, 448]: |x| <= amax makes |q| at most a few ulps
    // above 448, below the midpoint 464 to the next binade, so such q
    // round to +-448 as the clamped value would)
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const uint32_t p = cvt2(q[i], q[i + 1]);
      if (i < 4)
        lo |= p << (8 * i);
      else
        hi |= p << (8 * (i - 4));
    }
    __builtin_nontemporal_store(i32x2{(int)lo, (int)hi},
                                reinterpret_cast<i32x2*>(codes + (size_t)(row0 + r) * cols + c * 8));
    if (c == 0) scales[row0 + r] = scale;
  }
}

template <bool BF16, int LPR>
hipError_t launch_lpr(const void* x, int64_t rows, int cols, uint8_t* codes, float* scales,
                      hipStream_t stream) {
  constexpr int NR = 4;  // rows per lane group
  constexpr int RPB = kQuantThreads / LPR * NR;
  const int64_t blocks = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((fp8_quant_rows_kernel<BF16, LPR, NR>), dim3((unsigned)blocks),
                     dim3(kQuantThreads), 0, stream, x, rows, cols, codes, scales);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dtype(const void* x, int64_t rows, int cols, uint8_t* codes, float* scales,
                        hipStream_t stream) {
  const int chunks = cols / 8;
  if (chunks <= 8) return launch_lpr<BF16, 8>(x, rows, cols, codes, scales, stream);
  if (chunks <= 16) return launch_lpr<BF16, 16>(x, rows, cols, codes, scales, stream);
  if (chunks <= 32) return launch_lpr<BF16, 32>(x, rows, cols, codes, scales, stream);
  return launch_lpr<BF16, 64>(x, rows, cols, codes, scales, stream);
}

}  // namespace

hipError_t launch_fp8_quant(const void* x, bool bf16, int64_t rows, int cols, uint8_t* codes,
                            float* scales, hipStream_t stream) {
  return bf16 ? launch_dtype<true>(x, rows, cols, codes, scales, stream)
              : launch_dtype<false>(x, rows, cols, codes, scales, stream);
}

}  // namespace mha
