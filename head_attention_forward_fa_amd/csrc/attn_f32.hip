// float32 attention forward: the exact-precision variant, on the matrix cores.
//
// Both products run on v_mfma_f32_32x32x2_f32 (float32 operands, float32
// accumulation): the same 32x32 tile shapes as the bf16 kernel, at the
// float32 matrix rate.  One work item = one (sequence, query head, 32-row
// query tile).  The four waves of a workgroup share the tile's 32 query
// rows and split its 32-key blocks round robin (wave w takes blocks w,
// w + 4, ...); each wave keeps its own running max, row sum and O over its
// blocks, and the four partial results are merged through LDS at the end
// of the item, with the same rescaling that combines key splits.  A short
// sequence's item therefore costs about a quarter of its blocks in series,
// not all of them.
//
// Per wave and 32-key block:
//   S^T = K Q^T: keys along the MFMA M axis, queries along N, so lane i
//         holds 16 keys of query row i % 32 (lane i ^ 32 the other 16).
//         Operands come straight from global memory (L2): lane i reads K row
//         i % 32 and Q row i % 32, the lane half's contiguous half of the
//         depth (nope, then rope), one depth element per product.
//   mask, online softmax in the log2 domain (running max m of
//         sigma log2(e) S, P = 2^(sigma log2(e) S - m), the O / l correction
//         of the pages' per-row correction buffer: SM100AttentionSMem,
//         Methods correction_smem), all in float32.
//   O^T += V^T P^T: P^T is already the B operand (product s takes element s
//         of each lane), V^T's A operand is one float of V per lane and
//         product, 32 consecutive columns of two key rows per instruction.
// Rows past a sequence's end are read from its last row (the scores of such
// keys are masked, so their P is 0 against finite V).
#include "common.h"
#include "kernels.h"

namespace mha {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int BM = kBlockM_F32;  // 32 query rows per item
constexpr int BN = kBlockN_F32;  // 32 keys per block
static_assert(BM == 32 && BN == 32, "one 32x32 tile per wave and block");

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int DN, int DR, int DV>
__global__ __launch_bounds__(kThreads) void attn_fwd_f32_kernel(AttnParams p) {
  static_assert(DN % 8 == 0 && DR % 8 == 0 && DV % 32 == 0, "depth multiples");
  constexpr int HN = DN / 2, HR = DR / 2;  // depth elements per lane half
  constexpr int DVT = DV / 32;             // O^T tiles
  constexpr int OP = DV + 4;               // merge staging row pitch (floats)

  __shared__ __attribute__((aligned(16))) float s_o[kWaves][BM][OP];
  __shared__ float s_m[kWaves][BM];
  __shared__ float s_l[kWaves][BM];
  __shared__ i32x4 s_item[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const float* __restrict__ q = static_cast<const float*>(p.q);
  const float* __restrict__ k = static_cast<const float*>(p.k);
  const float* __restrict__ v = static_cast<const float*>(p.v);
  const float* __restrict__ qr = static_cast<const float*>(p.q_rope);
  const float* __restrict__ kr = static_cast<const float*>(p.k_rope);
  float* __restrict__ o = static_cast<float*>(p.o);
  const int T = p.cu_seqlens[p.batch];
  const int H = p.num_heads, Hkv = p.num_kv_heads;

  // wave 0 runs the work-item source: the next item is reserved when an
  // item starts and its entry read after the wave's key blocks, so neither
  // round trip delays the wave's products; the entry is published at the
  // end of the current item.  Without a table (direct mapping, small
  // problems) the workgroup's only item is item blockIdx.x of the
  // (sequence, head, q-tile) grid the launch covers, read from cu_seqlens
  // here; a length below 0 or above max_seqlen refuses the call in every
  // workgroup, as the prepass does.
  const bool direct = p.table == nullptr;
  Fetcher fetch;
  if (wave == 0) {
    i32x4 e0 = {0, -1, 0, 0};
    if (direct) {
      bool bad = false;
      for (int b = lane; b < p.batch; b += kWave) {
        const int Lb = p.cu_seqlens[b + 1] - p.cu_seqlens[b];
        bad = bad || Lb < 0 || Lb > p.max_seqlen;
      }
      const int tiles = (p.max_seqlen + BM - 1) / BM;
      const int idx = (int)blockIdx.x;
      const int qt = idx % tiles, bh = idx / tiles;
      const int h = bh % H, b = bh / H;
      if (!wave_any(bad) && b < p.batch) {
        const int s0 = p.cu_seqlens[b], Lb = p.cu_seqlens[b + 1] - s0;
        if (qt * BM < Lb) e0 = i32x4{s0, Lb, (h << 20) | qt, b};
      }
    } else {
      fetch.init(p.sched);
      e0 = fetch.resolve(p.sched, p.table);
    }
    if (lane == 0) s_item[0] = e0;
  }
  for (int it = 0;; ++it) {
    __syncthreads();
    const WorkItem w = decode_item(i32x4{__builtin_amdgcn_readfirstlane(s_item[it & 1][0]),
                                         __builtin_amdgcn_readfirstlane(s_item[it & 1][1]),
                                         __builtin_amdgcn_readfirstlane(s_item[it & 1][2]),
                                         __builtin_amdgcn_readfirstlane(s_item[it & 1][3])});
    if (w.L < 0) break;
    if (wave == 0 && !direct) fetch.reserve(p.sched);
    const int s0 = w.s0, L = w.L;
    const int g = w.h / p.group;
    const int q0 = w.qt * BM;
    const int qi = q0 + l32;  // this lane's query row
    const bool qvalid = qi < L;

    // Q: the lane half's half of the depth, as B operands
    float qn[HN], qrp[HR > 0 ? HR : 1];
    {
      const size_t row = (size_t)(s0 + (qvalid ? qi : L - 1)) * H + w.h;
      const f32x4* src = reinterpret_cast<const f32x4*>(q + row * DN + hf * HN);
#pragma unroll
      for (int c = 0; c < HN / 4; ++c) {
        const f32x4 x = src[c];
#pragma unroll
        for (int e = 0; e < 4; ++e) qn[4 * c + e] = x[e];
      }
      if constexpr (DR > 0) {
        const f32x4* srr = reinterpret_cast<const f32x4*>(qr + row * DR + hf * HR);
#pragma unroll
        for (int c = 0; c < HR / 4; ++c) {
          const f32x4 x = srr[c];
#pragma unroll
          for (int e = 0; e < 4; ++e) qrp[4 * c + e] = x[e];
        }
      }
    }

    f32x16 acc[DVT];
#pragma unroll
    for (int t = 0; t < DVT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
    float m = -INFINITY, l = 0.f;
    const float c2 = p.scale_log2;

    const int n_kv = p.causal ? min(L, q0 + BM) : L;
    const int nblk = (n_kv + BN - 1) / BN;
    const int lim = p.causal ? min(L - 1, qi) : L - 1;  // last key visible to this lane
    for (int j = wave; j < nblk; j += kWaves) {
      const int kb = j * BN;
      // S^T of keys kb .. kb + 31 (rows past the end read the last row)
      const size_t krow = (size_t)(s0 + min(kb + l32, L - 1)) * Hkv + g;
      f32x16 st;
#pragma unroll
      for (int r = 0; r < 16; ++r) st[r] = 0.f;
      {
        const f32x4* src = reinterpret_cast<const f32x4*>(k + krow * DN + hf * HN);
#pragma unroll
        for (int c = 0; c < HN / 4; ++c) {
          const f32x4 x = src[c];
#pragma unroll
          for (int e = 0; e < 4; ++e) st = mfma_f32(x[e], qn[4 * c + e], st);
        }
        if constexpr (DR > 0) {
          const f32x4* srr = reinterpret_cast<const f32x4*>(kr + krow * DR + hf * HR);
#pragma unroll
          for (int c = 0; c < HR / 4; ++c) {
            const f32x4 x = srr[c];
#pragma unroll
            for (int e = 0; e < 4; ++e) st = mfma_f32(x[e], qrp[4 * c + e], st);
          }
        }
      }
      // V^T operands: element s of the lane is key kb + 8(s/4) + 4 hf + s%4,
      // column 32 t + lane % 32 (issued before the softmax, used after it)
      float va[DVT][16];
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const int key = min(kb + 8 * (s >> 2) + 4 * hf + (s & 3), L - 1);
        const float* vr = v + ((size_t)(s0 + key) * Hkv + g) * DV + l32;
#pragma unroll
        for (int t = 0; t < DVT; ++t) va[t][s] = vr[32 * t];
      }
      // mask (element e is key kb + 8(e/4) + 4 hf + e%4), then the softmax
      float x = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kb + 8 * (e >> 2) + 4 * hf + (e & 3);
        st[e] = key <= lim ? st[e] * c2 : -INFINITY;
        x = fmaxf(x, st[e]);
      }
      const float m_new = fmaxf(m, half_max(x));
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);  // 0 while m = -inf
      float ls = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        st[e] = fast_exp2(st[e] - m_use);
        ls += st[e];
      }
      l = l * alpha + ls;
      m = m_new;
#pragma unroll
      for (int t = 0; t < DVT; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] *= alpha;
#pragma unroll
        for (int s = 0; s < 16; ++s) acc[t] = mfma_f32(va[t][s], st[s], acc[t]);
      }
    }

    i32x4 nxt = {0, -1, 0, 0};
    if (wave == 0 && !direct) nxt = fetch.resolve(p.sched, p.table);

    // merge the four waves' partial results: O = sum_w 2^(m_w - M) O_w /
    // sum_w 2^(m_w - M) l_w, M = max_w m_w
    {
      const float lt = half_sum(l);
#pragma unroll
      for (int t = 0; t < DVT; ++t)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const f32x4 y = {acc[t][4 * a4], acc[t][4 * a4 + 1], acc[t][4 * a4 + 2],
                           acc[t][4 * a4 + 3]};
          *reinterpret_cast<f32x4*>(&s_o[wave][l32][32 * t + 8 * a4 + 4 * hf]) = y;
        }
      if (hf == 0) {
        s_m[wave][l32] = m;
        s_l[wave][l32] = lt;
      }
    }
    __syncthreads();
    {
      constexpr int TPR = kThreads / BM;  // threads per output row
      constexpr int NPT = DV / TPR;       // columns per thread
      const int r = tid / TPR, c0 = (tid % TPR) * NPT;
      const int row = q0 + r;
      if (row < L) {
        float M = -INFINITY;
#pragma unroll
        for (int u = 0; u < kWaves; ++u) M = fmaxf(M, s_m[u][r]);
        const float Mu = M == -INFINITY ? 0.f : M;
        float a[kWaves], lt = 0.f;
#pragma unroll
        for (int u = 0; u < kWaves; ++u) {
          a[u] = fast_exp2(s_m[u][r] - Mu);  // 0 for a wave with no visible key
          lt += a[u] * s_l[u][r];
        }
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        float* dst = o + ((size_t)(s0 + row) * H + w.h) * DV + c0;
#pragma unroll
        for (int c = 0; c < NPT; c += 4) {
          f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int u = 0; u < kWaves; ++u) {
            const f32x4 z = *reinterpret_cast<const f32x4*>(&s_o[u][r][c0 + c]);
            y += a[u] * z;
          }
          *reinterpret_cast<f32x4*>(dst + c) = y * inv;
        }
        if (c0 == 0) p.lse[(size_t)w.h * T + s0 + row] = lt > 0.f ? (M + log2f(lt)) * kLn2 : -INFINITY;
      }
    }
    if (wave == 0 && lane == 0) s_item[(it + 1) & 1] = nxt;
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

constexpr int lds_f32(int dv) { return (int)sizeof(float) * kWaves * BM * (dv + 4 + 2); }

const Variant kF32[] = {
    {launch_f32<64, 0, 64>, blocks_f32<64, 0, 64>, BM, BN, lds_f32(64)},
    {launch_f32<128, 0, 128>, blocks_f32<128, 0, 128>, BM, BN, lds_f32(128)},
    {launch_f32<128, 64, 128>, blocks_f32<128, 64, 128>, BM, BN, lds_f32(128)},
};

}  // namespace

const Variant* find_variant_f32(int dn, int dr, int dv) {
  if (dn == 64 && dr == 0 && dv == 64) return &kF32[0];
  if (dn == 128 && dr == 0 && dv == 128) return &kF32[1];
  if (dn == 128 && dr == 64 && dv == 128) return &kF32[2];
  return nullptr;
}

}  // namespace mha
