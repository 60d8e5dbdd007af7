// float32 attention forward: the exact-precision variant.
//
// Plain fp32 vector arithmetic (no matrix cores): four lanes own one query
// row, each holding every fourth element of q and of the output row; K and V
// blocks of 32 keys are staged in LDS and read as broadcasts.  The running
// softmax statistics (row max m and row sum l, both in the log2 domain) are
// corrected once per key block -- the online-softmax rescale that the pages
// stage in a per-row "correction" buffer (SM100AttentionSMem, Methods:
// correction_smem); here it lives in registers.  Work items come from the
// persistent scheduler (sched.hip) with 64-row query tiles.
#include "common.h"
#include "kernels.h"

namespace mha {
namespace {

constexpr int kThreads = 256;
constexpr int BM = kBlockM_F32;   // 64 query rows per item, 4 lanes per row
constexpr int BN = kBlockN_F32;   // 32 keys per block

template <int DN, int DR, int DV>
__global__ __launch_bounds__(kThreads) void attn_fwd_f32_kernel(AttnParams p) {
  constexpr int DQK = DN + DR;
  static_assert(DN % 4 == 0 && DR % 4 == 0 && DV % 4 == 0, "depths must be multiples of 4");
  constexpr int NQ = DQK / 4, NO = DV / 4;

  __shared__ float s_k[BN][DQK];
  __shared__ float s_v[BN][DV];
  __shared__ i32x4 s_item[2];

  const int tid = threadIdx.x;
  const int sub = tid & 3;
  const int row = tid >> 2;
  const float* __restrict__ q = static_cast<const float*>(p.q);
  const float* __restrict__ k = static_cast<const float*>(p.k);
  const float* __restrict__ v = static_cast<const float*>(p.v);
  const float* __restrict__ qr = static_cast<const float*>(p.q_rope);
  const float* __restrict__ kr = static_cast<const float*>(p.k_rope);
  float* __restrict__ o = static_cast<float*>(p.o);
  const int T = p.cu_seqlens[p.batch];

  // wave 0 runs the work-item source; the next item's entry is published at
  // the end of the current item
  Fetcher fetch;
  const bool w0 = __builtin_amdgcn_readfirstlane(tid >> 6) == 0;
  if (w0) {
    fetch.init(p.sched);
    const i32x4 e0 = fetch.take(p.sched, p.table);
    if (tid == 0) s_item[0] = e0;
  }
  for (int it = 0;; ++it) {
    __syncthreads();
    const WorkItem w = decode_item(s_item[it & 1]);
    if (w.L < 0) break;
    i32x4 nxt;
    if (w0) nxt = fetch.take(p.sched, p.table);
    const int s0 = w.s0;
    const int L = w.L;
    const int g = w.h / p.group;
    const int qi = w.qt * BM + row;  // query row inside the sequence
    const bool qvalid = qi < L;

    float qv[NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      int d = sub + 4 * i;
      float x = 0.f;
      if (qvalid) {
        if (d < DN)
          x = q[((size_t)(s0 + qi) * p.num_heads + w.h) * DN + d];
        else
          x = qr[((size_t)(s0 + qi) * p.num_heads + w.h) * DR + (d - DN)];
      }
      qv[i] = x;
    }
    float acc[NO];
#pragma unroll
    for (int i = 0; i < NO; ++i) acc[i] = 0.f;
    float m = -INFINITY, l = 0.f;

    const int n_kv = p.causal ? min(L, (w.qt + 1) * BM) : L;
    for (int kb = 0; kb < n_kv; kb += BN) {
      // stage K (nope | rope) and V rows kb .. kb+BN-1; rows past L are zero
      for (int c = tid; c < BN * DQK; c += kThreads) {
        int r = c / DQK, d = c % DQK, key = kb + r;
        float x = 0.f;
        if (key < L) {
          size_t t = (size_t)(s0 + key) * p.num_kv_heads + g;
          x = d < DN ? k[t * DN + d] : kr[t * DR + (d - DN)];
        }
        s_k[r][d] = x;
      }
      for (int c = tid; c < BN * DV; c += kThreads) {
        int r = c / DV, d = c % DV, key = kb + r;
        s_v[r][d] = key < L ? v[((size_t)(s0 + key) * p.num_kv_heads + g) * DV + d] : 0.f;
      }
      __syncthreads();

      float s[BN];
      float mblk = -INFINITY;
#pragma unroll
      for (int j = 0; j < BN; ++j) {
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < NQ; ++i) part = fmaf(qv[i], s_k[j][sub + 4 * i], part);
        part += __shfl_xor(part, 1);
        part += __shfl_xor(part, 2);
        int key = kb + j;
        bool vis = key < L && (!p.causal || key <= qi);
        s[j] = vis ? part * p.scale_log2 : -INFINITY;
        mblk = fmaxf(mblk, s[j]);
      }
      const float m_new = fmaxf(m, mblk);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      float lsum = 0.f;
#pragma unroll
      for (int j = 0; j < BN; ++j) {
        s[j] = fast_exp2(s[j] - m_use);
        lsum += s[j];
      }
      l = l * alpha + lsum;
      m = m_new;
#pragma unroll
      for (int i = 0; i < NO; ++i) {
        float a = acc[i] * alpha;
#pragma unroll
        for (int j = 0; j < BN; ++j) a = fmaf(s[j], s_v[j][sub + 4 * i], a);
        acc[i] = a;
      }
      __syncthreads();
    }

    if (qvalid) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      float* orow = o + ((size_t)(s0 + qi) * p.num_heads + w.h) * DV;
#pragma unroll
      for (int i = 0; i < NO; ++i) orow[sub + 4 * i] = acc[i] * inv;
      if (sub == 0)
        p.lse[(size_t)w.h * T + s0 + qi] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
    }
    if (tid == 0) s_item[(it + 1) & 1] = nxt;
  }
}

template <int DN, int DR, int DV>
hipError_t launch_f32(const AttnParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_f32_kernel<DN, DR, DV>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int DN, int DR, int DV>
int blocks_f32() {
  static int cached = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_fwd_f32_kernel<DN, DR, DV>,
                                                     kThreads, 0) != hipSuccess || n < 1)
      n = 1;
    return n;
  }();
  return cached;
}

const Variant kF32[] = {
    {launch_f32<64, 0, 64>, blocks_f32<64, 0, 64>, BM, BN, (int)sizeof(float) * BN * (64+0+64)},
    {launch_f32<128, 0, 128>, blocks_f32<128, 0, 128>, BM, BN, (int)sizeof(float) * BN * (128+0+128)},
    {launch_f32<128, 64, 128>, blocks_f32<128, 64, 128>, BM, BN, (int)sizeof(float) * BN * (128+64+128)},
};

}  // namespace

const Variant* find_variant_f32(int dn, int dr, int dv) {
  if (dn == 64 && dr == 0 && dv == 64) return &kF32[0];
  if (dn == 128 && dr == 0 && dv == 128) return &kF32[1];
  if (dn == 128 && dr == 64 && dv == 128) return &kF32[2];
  return nullptr;
}

}  // namespace mha
