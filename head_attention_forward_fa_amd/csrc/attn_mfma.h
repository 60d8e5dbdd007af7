// Matrix-core attention forward for bf16 and fp8 (E4M3) Q/K on gfx950.
//
// One work item = one (sequence, query head, 128-row query tile).  A
// workgroup is 4 waves; wave w owns query rows 32w .. 32w+31 of the tile.
// The tile of Q stays in registers for the whole item; K and V stream past
// in 64-key blocks through a two-stage LDS ring (the "Q-stationary" tiling
// with staged K/V buffers of the pages: SM100AttentionSMem, comptime
// members q_bytes and k_stage_bytes / v_stage_bytes; TMAProducerPipeline,
// acquire / commit_step).
//
// Per 64-key block, per wave:
//   S^T = K Q^T on the matrix cores (v_mfma_f32_32x32x16_bf16, or for fp8
//         v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales).  Keys run
//         along the MFMA M axis and queries along N, so in the 32x32 output
//         layout lane i holds 16 keys of ONE query row (i % 32); lanes i and
//         i ^ 32 hold the other 16.  Row max / row sum are therefore 15
//         in-lane operations plus one v_permlane32_swap.
//   fp8:  S_ij *= k_scale_j (and q_scale_i is folded into the exponent
//         multiplier), after the product, as the per-token scales are staged
//         per tile on the pages (SM100AttentionSMem, Methods q_scale_smem,
//         k_scale_smem).
//   mask: only in blocks that cross the causal diagonal or the sequence end.
//   online softmax in the log2 domain: m_i is the running row max of
//         sigma*log2(e)*S; P = 2^(sigma*log2(e)*S - m) via v_exp_f32.  The
//         correction of O and l (the pages' per-row correction buffer,
//         SM100AttentionSMem Methods: correction_smem) is applied lazily: only
//         when some row's max grows by more than 8 (a factor 256), so almost
//         every block skips it.  Both O and l always use the same stale m, so
//         the final O/l and LSE = (m + log2 l) ln 2 are unchanged.
//   O^T += V^T P^T on the matrix cores.  P^T is already in the B-operand
//         layout of the next MFMA (lane = query, 8 consecutive k-slots), so it
//         goes from the S registers to the PV product with only a bf16 pack.
//         V^T (the "mn-major" V tile of TMAProducerPipeline) is written to LDS
//         transposed by the loader, with keys permuted inside each group of
//         16 so that every A-operand fragment is one 16-byte LDS read.
// Epilogue: O / l, bf16 round-to-nearest-even, staged through LDS for
// coalesced 16-byte stores (the pages reuse the Q region for this,
// SM100AttentionSMem Methods: o_smem), and LSE in natural log.
#pragma once

#include "common.h"
#include "kernels.h"

namespace mha {

template <int DN_, int DR_, int DV_, bool FP8_>
struct MfmaCfg {
  static constexpr int DN = DN_, DR = DR_, DV = DV_;
  static constexpr bool FP8 = FP8_;
  static constexpr int BM = kBlockM_Mfma;  // 128 query rows per item
  static constexpr int BN = kBlockN_Mfma;  // 64 keys per block
  static constexpr int WAVES = BM / 32;
  static constexpr int THREADS = WAVES * kWave;
  static constexpr int EB = FP8 ? 1 : 2;               // bytes per Q/K nope element
  static constexpr int NOPE_BYTES = DN * EB;           // per K row in HBM
  static constexpr int ROPE_BYTES = DR * 2;
  static constexpr int K_ROW = NOPE_BYTES + ROPE_BYTES + 16;  // LDS K row stride (+16 B pad)
  static constexpr int K_STAGE = BN * K_ROW;
  static constexpr int KS_STAGE = FP8 ? BN * 4 : 0;    // k_scale of the block's keys
  static constexpr int V_ROW = BN * 2 + 16;            // LDS V^T row: BN keys + 16 B pad
  static constexpr int V_STAGE = DV * V_ROW;
  static constexpr int STAGE = K_STAGE + KS_STAGE + V_STAGE;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int O_ROW = DV * 2 + 16;            // epilogue staging row stride
  static constexpr int K_CHUNKS_ROW = (NOPE_BYTES + ROPE_BYTES) / 16;
  static constexpr int K_CHUNKS = BN * K_CHUNKS_ROW;
  static constexpr int K_PER_THREAD = (K_CHUNKS + THREADS - 1) / THREADS;
  static constexpr int V_GROUPS = (DV / 8) * (BN / 4);  // 4 keys x 8 columns each
  static constexpr int V_PER_THREAD = (V_GROUPS + THREADS - 1) / THREADS;
  static constexpr int QK_STEPS = FP8 ? DN / 64 : (DN + DR) / 16;
  static constexpr int DV_TILES = DV / 32;

  static_assert(!FP8 || DR == 0, "fp8 Q/K carry no rope part");
  static_assert(DN % 64 == 0 && DR % 16 == 0 && DV % 32 == 0, "unsupported depths");
  static_assert(NOPE_BYTES % 16 == 0 && ROPE_BYTES % 16 == 0, "16-byte rows");
  static_assert(WAVES * 32 * O_ROW <= LDS, "epilogue staging must fit in the ring");
  static_assert(LDS <= 160 * 1024, "LDS per workgroup");
};

// Position of key k (0..BN-1) inside a V^T LDS row: bits 2 and 3 swapped.
// The PV B-operand slot (lane half hf, element i) of MFMA u holds key
// 16u + 8(i/4) + 4hf + (i%4) (from the 32x32 output layout of S^T); with this
// permutation the 8 keys of a slot group are contiguous: 16u + 8hf + i.
__device__ __forceinline__ int vt_pos(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

template <class C>
struct MfmaKernel {
  using QFrag = typename std::conditional<C::FP8, i32x8, bf16x8>::type;

  struct Prefetch {
    i32x4 k[C::K_PER_THREAD];
    i32x4 v[C::V_PER_THREAD][4];
    float ks;
  };

  static __device__ __forceinline__ void load_block(const AttnParams& p, Prefetch& pf, int tid,
                                                    int s0, int L, int g, int kbase) {
    const char* __restrict__ kp = static_cast<const char*>(p.k);
    const char* __restrict__ krp = static_cast<const char*>(p.k_rope);
    const char* __restrict__ vp = static_cast<const char*>(p.v);
    const int Hkv = p.num_kv_heads;
#pragma unroll
    for (int i = 0; i < C::K_PER_THREAD; ++i) {
      const int c = tid + i * C::THREADS;
      i32x4 x = {0, 0, 0, 0};
      if (C::K_CHUNKS % C::THREADS == 0 || c < C::K_CHUNKS) {
        const int r = c / C::K_CHUNKS_ROW, cc = c % C::K_CHUNKS_ROW, key = kbase + r;
        if (key < L) {
          const size_t row = (size_t)(s0 + key) * Hkv + g;
          const int off = cc * 16;
          const char* src = (C::DR == 0 || off < C::NOPE_BYTES)
                                ? kp + row * C::NOPE_BYTES + off
                                : krp + row * C::ROPE_BYTES + (off - C::NOPE_BYTES);
          x = *reinterpret_cast<const i32x4*>(src);
        }
      }
      pf.k[i] = x;
    }
#pragma unroll
    for (int i = 0; i < C::V_PER_THREAD; ++i) {
      const int c = tid + i * C::THREADS;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) pf.v[i][rr] = i32x4{0, 0, 0, 0};
      if (C::V_GROUPS % C::THREADS == 0 || c < C::V_GROUPS) {
        const int dg = c % (C::DV / 8), kg = c / (C::DV / 8);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int key = kbase + 4 * kg + rr;
          if (key < L)
            pf.v[i][rr] = *reinterpret_cast<const i32x4*>(
                vp + (((size_t)(s0 + key) * Hkv + g) * C::DV + dg * 8) * 2);
        }
      }
    }
    if (C::FP8) {
      pf.ks = 0.f;
      if (tid < C::BN && kbase + tid < L) pf.ks = p.k_scale[(size_t)(s0 + kbase + tid) * Hkv + g];
    }
  }

  static __device__ __forceinline__ void store_block(char* stage, const Prefetch& pf, int tid) {
#pragma unroll
    for (int i = 0; i < C::K_PER_THREAD; ++i) {
      const int c = tid + i * C::THREADS;
      if (C::K_CHUNKS % C::THREADS == 0 || c < C::K_CHUNKS) {
        const int r = c / C::K_CHUNKS_ROW, cc = c % C::K_CHUNKS_ROW;
        *reinterpret_cast<i32x4*>(stage + r * C::K_ROW + cc * 16) = pf.k[i];
      }
    }
    char* vt = stage + C::K_STAGE + C::KS_STAGE;
#pragma unroll
    for (int i = 0; i < C::V_PER_THREAD; ++i) {
      const int c = tid + i * C::THREADS;
      if (C::V_GROUPS % C::THREADS == 0 || c < C::V_GROUPS) {
        const int dg = c % (C::DV / 8), kg = c / (C::DV / 8);
        const int pos = vt_pos(4 * kg);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int w = j >> 1;
          uint32_t e0 = (uint32_t)pf.v[i][0][w], e1 = (uint32_t)pf.v[i][1][w];
          uint32_t e2 = (uint32_t)pf.v[i][2][w], e3 = (uint32_t)pf.v[i][3][w];
          uint32_t lo, hi;
          if (j & 1) {
            lo = (e0 >> 16) | (e1 & 0xFFFF0000u);
            hi = (e2 >> 16) | (e3 & 0xFFFF0000u);
          } else {
            lo = (e0 & 0xFFFFu) | (e1 << 16);
            hi = (e2 & 0xFFFFu) | (e3 << 16);
          }
          *reinterpret_cast<i32x2*>(vt + (dg * 8 + j) * C::V_ROW + pos * 2) =
              i32x2{(int)lo, (int)hi};
        }
      }
    }
    if (C::FP8 && tid < C::BN) reinterpret_cast<float*>(stage + C::K_STAGE)[tid] = pf.ks;
  }

  static __device__ __forceinline__ f32x16 mfma_qk(const QFrag& a, const QFrag& b, f32x16 acc) {
    if constexpr (C::FP8)
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
    else
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }

  static __device__ void run(const AttnParams& p, char* smem) {
    __shared__ int2 s_slot[2];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int lane32 = lane & 31;
    const int hf = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = p.cu_seqlens[p.batch];
    const char* __restrict__ qp = static_cast<const char*>(p.q);
    const char* __restrict__ qrp = static_cast<const char*>(p.q_rope);
    char* __restrict__ op = static_cast<char*>(p.o);

    int queue = blockIdx.x % kNumXcd, tried = 0;
    for (int it = 0;; ++it) {
      if (tid == 0) {
        int2 e;
        s_slot[it & 1] = fetch_item(p.sched, p.table, queue, tried, e) ? e : make_int2(-1, 0);
      }
      __syncthreads();
      const int2 e = s_slot[it & 1];
      if (e.x < 0) break;
      const WorkItem w = decode_item(e);
      const int s0 = p.cu_seqlens[w.b];
      const int L = p.cu_seqlens[w.b + 1] - s0;
      const int g = w.h / p.group;
      const int q0 = w.qt * C::BM;           // first query row of the tile
      const int wq0 = q0 + wave * 32;        // first query row of this wave
      const int qi = wq0 + lane32;           // this lane's query row
      const bool qvalid = qi < L;
      const size_t qrow = (size_t)(s0 + qi) * p.num_heads + w.h;

      // Q fragments (B operand): lane -> query qi, 8 (bf16) or 32 (fp8)
      // consecutive depth elements per step and lane half.
      QFrag qf[C::QK_STEPS];
#pragma unroll
      for (int s = 0; s < C::QK_STEPS; ++s) {
        if constexpr (C::FP8) {
          i32x8 x = {0, 0, 0, 0, 0, 0, 0, 0};
          if (qvalid) {
            const i32x4* src =
                reinterpret_cast<const i32x4*>(qp + qrow * C::DN + s * 64 + 32 * hf);
            i32x4 a0 = src[0], a1 = src[1];
            x = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          }
          qf[s] = x;
        } else {
          i32x4 x = {0, 0, 0, 0};
          if (qvalid) {
            const int d = s * 16 + 8 * hf;
            const char* src = d < C::DN ? qp + (qrow * C::DN + d) * 2
                                        : qrp + (qrow * C::DR + (d - C::DN)) * 2;
            x = *reinterpret_cast<const i32x4*>(src);
          }
          qf[s] = __builtin_bit_cast(bf16x8, x);
        }
      }
      // multiplier of S in the exponent (log2 domain); kept >= FLT_MIN so
      // that a masked -inf score stays -inf (a zero q_scale row then gives
      // the uniform distribution over its visible keys, as 0 * S does)
      float cq = p.scale_log2;
      if (C::FP8 && qvalid) cq *= p.q_scale[qrow];
      if (!(cq >= 1.17549435e-38f)) cq = 1.17549435e-38f;

      f32x16 o[C::DV_TILES];
#pragma unroll
      for (int t = 0; t < C::DV_TILES; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
      float m = -INFINITY;  // running max (log2 domain), same in lanes i, i^32
      float l = 0.f;        // this lane's partial row sum (its 32 keys of each block)

      const int n_kv = p.causal ? min(L, q0 + C::BM) : L;
      const int nblocks = (n_kv + C::BN - 1) / C::BN;

      Prefetch pf;
      load_block(p, pf, tid, s0, L, g, 0);
      store_block(smem, pf, tid);
      __syncthreads();

      for (int kb = 0; kb < nblocks; ++kb) {
        const int kbase = kb * C::BN;
        const bool more = kb + 1 < nblocks;
        if (more) load_block(p, pf, tid, s0, L, g, kbase + C::BN);
        char* stage = smem + (kb & 1) * C::STAGE;

        if (!p.causal || kbase <= wq0 + 31) {
          // ---- S^T = K Q^T : two 32-key tiles
          f32x16 st[2];
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            f32x16 acc;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.f;
            const char* krow = stage + (kt * 32 + lane32) * C::K_ROW;
#pragma unroll
            for (int s = 0; s < C::QK_STEPS; ++s) {
              QFrag a;
              if constexpr (C::FP8) {
                const i32x4* src = reinterpret_cast<const i32x4*>(krow + s * 64 + 32 * hf);
                i32x4 a0 = src[0], a1 = src[1];
                a = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
              } else {
                a = *reinterpret_cast<const bf16x8*>(krow + (s * 16 + 8 * hf) * 2);
              }
              acc = mfma_qk(a, qf[s], acc);
            }
            st[kt] = acc;
          }

          // ---- per-key scale (fp8), mask, block row max
          if constexpr (C::FP8) {
            const float* ksl = reinterpret_cast<const float*>(stage + C::K_STAGE);
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
              for (int a4 = 0; a4 < 4; ++a4) {
                const f32x4 ks = *reinterpret_cast<const f32x4*>(ksl + kt * 32 + 8 * a4 + 4 * hf);
#pragma unroll
                for (int r = 0; r < 4; ++r) st[kt][4 * a4 + r] *= ks[r];
              }
          }
          const bool need_mask =
              (kbase + C::BN > L) || (p.causal && kbase + C::BN - 1 > wq0);
          if (need_mask) {
            const int lim = p.causal ? min(L - 1, qi) : L - 1;  // last visible key
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int key = kbase + kt * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
                if (key > lim) st[kt][r] = -INFINITY;
              }
          }
          float mx = -INFINITY;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[kt][r]);
          mx = half_max(mx) * cq;

          // ---- lazy correction of the running statistics
          if (wave_any(mx > m + 8.0f)) {
            const float m_new = fmaxf(m, mx);
            const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m - m_new);
            l *= alpha;
#pragma unroll
            for (int t = 0; t < C::DV_TILES; ++t)
#pragma unroll
              for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
            m = m_new;
          }
          const float m_use = m == -INFINITY ? 0.f : m;

          // ---- P = 2^(cq*S - m), row sums, bf16 B-operand fragments
          bf16x8 pb[4];
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float pv = fast_exp2(fmaf(st[kt][r], cq, -m_use));
              st[kt][r] = pv;
              l += pv;
            }
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              i32x4 x;
#pragma unroll
              for (int j = 0; j < 4; ++j)
                x[j] = (int)pack_bf16x2(st[kt][8 * hh + 2 * j], st[kt][8 * hh + 2 * j + 1]);
              pb[2 * kt + hh] = __builtin_bit_cast(bf16x8, x);
            }
          }

          // ---- O^T += V^T P^T
          const char* vt = stage + C::K_STAGE + C::KS_STAGE;
#pragma unroll
          for (int t = 0; t < C::DV_TILES; ++t) {
            const char* vrow = vt + (t * 32 + lane32) * C::V_ROW;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const bf16x8 a = *reinterpret_cast<const bf16x8*>(vrow + (16 * u + 8 * hf) * 2);
              o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[u], o[t], 0, 0, 0);
            }
          }
        }

        if (more) store_block(smem + ((kb + 1) & 1) * C::STAGE, pf, tid);
        __syncthreads();
      }

      // ---- epilogue
      const float lt = half_sum(l);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      char* ost = smem + wave * 32 * C::O_ROW + lane32 * C::O_ROW;
#pragma unroll
      for (int t = 0; t < C::DV_TILES; ++t)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int dv0 = t * 32 + 8 * a4 + 4 * hf;
          const uint32_t lo = pack_bf16x2(o[t][4 * a4 + 0] * inv, o[t][4 * a4 + 1] * inv);
          const uint32_t hi = pack_bf16x2(o[t][4 * a4 + 2] * inv, o[t][4 * a4 + 3] * inv);
          *reinterpret_cast<i32x2*>(ost + dv0 * 2) = i32x2{(int)lo, (int)hi};
        }
      if (hf == 0 && qvalid)
        p.lse[(size_t)w.h * T + s0 + qi] = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
      __syncthreads();
      constexpr int CPR = C::DV * 2 / 16;  // 16-byte chunks per output row
#pragma unroll
      for (int i = 0; i < 32 * CPR / kWave; ++i) {
        const int c = lane + i * kWave;
        const int r = c / CPR, cc = c % CPR;
        const int row = wq0 + r;
        if (row < L) {
          const i32x4 x =
              *reinterpret_cast<const i32x4*>(smem + (wave * 32 + r) * C::O_ROW + cc * 16);
          *reinterpret_cast<i32x4*>(op + (((size_t)(s0 + row) * p.num_heads + w.h) * C::DV) * 2 +
                                    cc * 16) = x;
        }
      }
    }
  }
};

template <class C>
__global__ __launch_bounds__(C::THREADS, 2) void attn_fwd_mfma_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  MfmaKernel<C>::run(p, smem);
}

template <class C>
hipError_t launch_mfma(const AttnParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(attn_fwd_mfma_kernel<C>, dim3(grid), dim3(C::THREADS), 0, stream, p);
  return hipGetLastError();
}

template <class C>
int blocks_mfma() {
  static int cached = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_fwd_mfma_kernel<C>, C::THREADS,
                                                     0) != hipSuccess ||
        n < 1)
      n = 1;
    return n;
  }();
  return cached;
}

}  // namespace mha
