// Matrix-core attention forward for bf16 and fp8 (E4M3) Q/K on gfx950.
//
// One work item = one (sequence, query head, 128-row query tile).  A
// workgroup is 4 waves; wave w owns query rows 32w .. 32w+31 of the tile.
// The tile of Q stays in registers for the whole item; K and V stream past
// in 64-key blocks through a two-stage LDS ring (the Q-stationary tiling
// with staged K/V buffers of the pages: SM100AttentionSMem, comptime
// members q_bytes, k_stage_bytes, v_stage_bytes; TMAProducerPipeline,
// acquire / commit_step).
//
// Staging.  K, K_rope, V (and the fp8 k_scale) of block j+1 are copied
// HBM -> LDS by buffer_load ... lds while block j is computed: each lane
// moves 16 bytes straight into LDS (lane i of an instruction lands at byte
// 16 i of a 1 KiB run), with no register staging and no VALU work.  The
// buffer resource of a block ends at the sequence's last key, so rows past
// the end arrive as zeros.  Rows are stored as 16-byte chunks in
// XOR-swizzled order (the global side picks which chunk each lane fetches),
// so the matrix-core operand reads below are free of LDS bank conflicts.
//
// Per 64-key block, per wave:
//   S^T = K Q^T on the matrix cores (v_mfma_f32_32x32x16_bf16, or for fp8
//         v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales).  Keys run
//         along the MFMA M axis and queries along N, so in the 32x32 output
//         layout lane i holds 16 keys of ONE query row (i % 32); lanes i and
//         i ^ 32 hold the other 16.  Row max is 15 in-lane operations plus
//         one v_permlane32_swap; row sums stay per lane until the end.
//   fp8:  S_ij *= k_scale_j, with q_scale_i folded into the exponent
//         multiplier, after the product (per-token scales staged per tile:
//         SM100AttentionSMem, Methods q_scale_smem, k_scale_smem).
//   mask: only in blocks that cross the causal diagonal or the sequence end.
//   online softmax in the log2 domain: m_i is the running row max of
//         sigma*log2(e)*S; P = 2^(sigma*log2(e)*S - m) via v_exp_f32.  The
//         correction of O and l (the per-row correction buffer of
//         SM100AttentionSMem, Methods: correction_smem) is applied lazily,
//         only when some row's max grows by more than 8 (a factor 256), so
//         almost every block skips it; O and l always share the same stale m,
//         so O / l and LSE = (m + log2 l) ln 2 are unchanged.
//   O^T += V^T P^T on the matrix cores.  P^T is already in the B-operand
//         layout (lane = query, 8 k-slots), so it goes from the S registers to
//         the PV product with one v_cvt_pk_bf16_f32 per pair.  V stays
//         row-major in LDS ("mn-major" V of TMAProducerPipeline); the
//         A-operand V^T fragments come from ds_read_b64_tr_b16, which hands
//         each lane 4 keys of one V column.
// Epilogue: O / l, bf16 round-to-nearest-even, staged through LDS for
// coalesced 16-byte stores (the pages reuse the Q region for this,
// SM100AttentionSMem Methods: o_smem), and LSE in natural log.
#pragma once

#include "common.h"
#include "kernels.h"

namespace mha {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

template <int DN_, int DR_, int DV_, bool FP8_>
struct MfmaCfg {
  static constexpr int DN = DN_, DR = DR_, DV = DV_;
  static constexpr bool FP8 = FP8_;
  static constexpr int BM = kBlockM_Mfma;  // 128 query rows per item
  static constexpr int BN = kBlockN_Mfma;  // 64 keys per block
  static constexpr int WAVES = BM / 32;
  static constexpr int THREADS = WAVES * kWave;
  static constexpr int EB = FP8 ? 1 : 2;    // bytes per Q/K nope element
  static constexpr int K_RB = DN * EB;      // bytes per K nope row
  static constexpr int R_RB = DR * 2;       // bytes per K rope row
  static constexpr int V_RB = DV * 2;       // bytes per V row
  // stage layout: K nope | K rope | V | k_scale  (the first three are whole KiB)
  static constexpr int K_OFF = 0;
  static constexpr int R_OFF = K_OFF + BN * K_RB;
  static constexpr int V_OFF = R_OFF + BN * R_RB;
  static constexpr int KS_OFF = V_OFF + BN * V_RB;
  static constexpr int STAGE = KS_OFF + (FP8 ? BN * 4 : 0);
  static constexpr int LDS = 2 * STAGE;
  static constexpr int O_ROW = DV * 2 + 16;  // epilogue staging row stride
  static constexpr int QK_STEPS = FP8 ? DN / 64 : DN / 16;  // nope MFMA k-steps
  static constexpr int ROPE_STEPS = DR / 16;
  static constexpr int DV_TILES = DV / 32;

  static_assert(!FP8 || DR == 0, "fp8 Q/K carry no rope part");
  static_assert(K_RB == 128 || K_RB == 256, "K rows of 128 or 256 bytes");
  static_assert(DR == 0 || R_RB == 128, "rope rows of 128 bytes");
  static_assert(V_RB == 128 || V_RB == 256, "V rows of 128 or 256 bytes");
  static_assert((BN * K_RB / 1024) % WAVES == 0 && (BN * R_RB / 1024) % WAVES == 0 &&
                    (BN * V_RB / 1024) % WAVES == 0,
                "DMA instructions split evenly over the waves");
  static_assert(WAVES * 32 * O_ROW <= LDS, "epilogue staging must fit in the ring");
  static_assert(LDS <= 160 * 1024, "LDS per workgroup");
};

// Chunk swizzles (position of 16-byte chunk c of row r = c ^ swz(r)).
// K regions are read as A operands: 16 lanes (or 8 on a 32-bank LDS) read
// the same chunk of 16 (8) consecutive rows in one cycle, which the XOR
// spreads over distinct banks.
__device__ __forceinline__ int swz_k256(int r) { return r & 15; }
__device__ __forceinline__ int swz_k128(int r) { return (r & 7) ^ ((r >> 3) & 1); }
// V rows are read by ds_read_b64_tr_b16: one instruction touches 4 (per 16
// lanes) or 8 consecutive keys at 2 or 4 chunks each; the XOR keeps both the
// 16- and the 32-lane groups on distinct banks.
__device__ __forceinline__ int swz_v256(int k) {
  return (4 * (k & 3)) ^ (((k ^ (k >> 1)) & 1) << 1);
}
__device__ __forceinline__ int swz_v128(int k) { return 2 * (k & 3); }

template <int RB>
__device__ __forceinline__ int swz_k(int r) {
  return RB == 256 ? swz_k256(r) : swz_k128(r);
}
template <int RB>
__device__ __forceinline__ int swz_v(int k) {
  return RB == 256 ? swz_v256(k) : swz_v128(k);
}

template <class C>
struct MfmaKernel {
  using QFrag = typename std::conditional<C::FP8, i32x8, bf16x8>::type;

  // One 16-byte-per-lane DMA instruction: buffer_load_dwordx4 ... lds writes
  // lane i's 16 bytes at LDS address m0 + 16 i.  (m0 is set here; nothing
  // else in these kernels keeps a value in m0.)  Issued from inline assembly
  // so that the compiler does not treat it as a pending write to every LDS
  // address (it would otherwise wait for it before each LDS read of the
  // other stage); completion is awaited explicitly with vmcnt(0) before the
  // barrier that publishes the stage.
  static __device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t lds_addr,
                                               uint32_t voff) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(lds_addr), "v"(voff), "s"(rsrc)
        : "memory");
  }
  static __device__ __forceinline__ void dma4(const i32x4& rsrc, uint32_t lds_addr,
                                              uint32_t voff) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dword %1, %2, 0 offen lds"
        :
        : "s"(lds_addr), "v"(voff), "s"(rsrc)
        : "memory");
  }
  // Raw buffer resource (stride 0) over [base, base + bytes) in SGPRs.
  static __device__ __forceinline__ i32x4 rsrc_of(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu)),
                 __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
  }
  static __device__ __forceinline__ uint32_t lds_addr_of(const char* p) {
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)p);
  }

  // Issue this wave's share of the DMA of one row-major region of BN rows
  // of RB bytes into LDS.  Instruction n covers rows RPI*n .. RPI*n+RPI-1;
  // lane i fills position i % CPR of row RPI*n + i / CPR with the chunk
  // that the swizzle puts there.
  template <int RB, bool VREGION>
  static __device__ __forceinline__ void dma_region(const char* lds_region, const i32x4& rsrc,
                                                    int row_stride_bytes, int wave, int lane) {
    constexpr int CPR = RB / 16, RPI = 1024 / RB;
    constexpr int INSTS = C::BN * RB / 1024;
    constexpr int PER_WAVE = INSTS / C::WAVES;
    const uint32_t base = lds_addr_of(lds_region);
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int n = wave * PER_WAVE + j;
      const int row = RPI * n + lane / CPR;
      const int pos = lane % CPR;
      const int chunk = pos ^ (VREGION ? swz_v<RB>(row) : swz_k<RB>(row));
      dma16(rsrc, __builtin_amdgcn_readfirstlane(base + 1024 * n),
            (uint32_t)(row * row_stride_bytes + chunk * 16));
    }
  }

  static __device__ __forceinline__ void load_block(const AttnParams& p, const char* stage,
                                                    int wave, int lane, int s0, int L, int g,
                                                    int kbase) {
    const int Hkv = p.num_kv_heads;
    const int rows = min(L - kbase, C::BN);  // >= 1
    const size_t row0 = (size_t)(s0 + kbase) * Hkv + g;
    const uint32_t span = (uint32_t)((rows - 1) * Hkv + 1);  // [T, Hkv] rows touched
    dma_region<C::K_RB, false>(
        stage + C::K_OFF, rsrc_of(static_cast<const char*>(p.k) + row0 * C::K_RB, span * C::K_RB),
        Hkv * C::K_RB, wave, lane);
    if constexpr (C::DR > 0)
      dma_region<C::R_RB, false>(
          stage + C::R_OFF,
          rsrc_of(static_cast<const char*>(p.k_rope) + row0 * C::R_RB, span * C::R_RB),
          Hkv * C::R_RB, wave, lane);
    dma_region<C::V_RB, true>(
        stage + C::V_OFF, rsrc_of(static_cast<const char*>(p.v) + row0 * C::V_RB, span * C::V_RB),
        Hkv * C::V_RB, wave, lane);
    if constexpr (C::FP8) {
      if (wave == 0)
        dma4(rsrc_of(p.k_scale + row0, span * 4),
             __builtin_amdgcn_readfirstlane(lds_addr_of(stage + C::KS_OFF)),
             (uint32_t)(lane * Hkv * 4));
    }
  }

  static __device__ __forceinline__ f32x16 mfma_qk(const QFrag& a, const QFrag& b, f32x16 acc) {
    if constexpr (C::FP8)
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
    else
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }

  // A-operand fragment of K for key row r (0..BN-1), depth step s, lane half hf.
  static __device__ __forceinline__ QFrag k_frag(const char* stage, int r, int s, int hf) {
    const char* row = stage + C::K_OFF + r * C::K_RB;
    const int sw = swz_k<C::K_RB>(r);
    if constexpr (C::FP8) {
      const int c0 = 4 * s + 2 * hf;  // 32 bytes = chunks c0, c0 + 1
      const i32x4 a0 = *reinterpret_cast<const i32x4*>(row + 16 * (c0 ^ sw));
      const i32x4 a1 = *reinterpret_cast<const i32x4*>(row + 16 * ((c0 + 1) ^ sw));
      return i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    } else {
      return *reinterpret_cast<const bf16x8*>(row + 16 * ((2 * s + hf) ^ sw));
    }
  }
  static __device__ __forceinline__ bf16x8 krope_frag(const char* stage, int r, int s, int hf) {
    const char* row = stage + C::R_OFF + r * C::R_RB;
    return *reinterpret_cast<const bf16x8*>(row + 16 * ((2 * s + hf) ^ swz_k<C::R_RB>(r)));
  }
  // A-operand fragment of V^T for dv tile t and keys 16u .. 16u+15: slot
  // (lane half h, element i) holds key 16u + 8(i/4) + 4h + i%4 of column
  // 32t + lane % 32, matching the P^T B-operand slots.  Within each group of
  // 16 lanes, ds_read_b64_tr_b16 gives lane i, element k, the element i % 4
  // of the 8 bytes addressed by lane 4k + i/4; so lane s of the group
  // addresses key (base + s/4) at columns 4(s%4) .. 4(s%4)+3.
  static __device__ __forceinline__ bf16x8 v_frag(const char* stage, int t, int u, int lane) {
    const int grp = lane >> 4, s = lane & 15;
    const int h = grp >> 1;
    const int dv = t * 32 + 16 * (grp & 1) + 4 * (s & 3);  // first of this lane's 4 columns
    const int c = dv >> 3, sub = (dv & 7) * 2;               // chunk and byte inside it
    const int k1 = 16 * u + 4 * h + (s >> 2), k2 = k1 + 8;
    const char* v = stage + C::V_OFF;
    const char* a1 = v + k1 * C::V_RB + 16 * (c ^ swz_v<C::V_RB>(k1)) + sub;
    const char* a2 = v + k2 * C::V_RB + 16 * (c ^ swz_v<C::V_RB>(k2)) + sub;
    const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a1));
    const i16x4 r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a2));
    const i16x8 r = {r1[0], r1[1], r1[2], r1[3], r2[0], r2[1], r2[2], r2[3]};
    return __builtin_bit_cast(bf16x8, r);
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
      // the item is the same for the whole workgroup: keep it in SGPRs
      const int2 e = make_int2(__builtin_amdgcn_readfirstlane(s_slot[it & 1].x),
                               __builtin_amdgcn_readfirstlane(s_slot[it & 1].y));
      if (e.x < 0) break;
      const WorkItem w = decode_item(e);
      const int s0 = __builtin_amdgcn_readfirstlane(p.cu_seqlens[w.b]);
      const int L = __builtin_amdgcn_readfirstlane(p.cu_seqlens[w.b + 1]) - s0;
      const int g = w.h / p.group;
      const int q0 = w.qt * C::BM;     // first query row of the tile
      const int wq0 = q0 + wave * 32;  // first query row of this wave
      const int qi = wq0 + lane32;     // this lane's query row
      const bool qvalid = qi < L;
      const size_t qrow = (size_t)(s0 + qi) * p.num_heads + w.h;

      const int n_kv = p.causal ? min(L, q0 + C::BM) : L;
      const int nblocks = (n_kv + C::BN - 1) / C::BN;
      load_block(p, smem, wave, lane, s0, L, g, 0);

      // Q fragments (B operand): lane -> query qi, 8 (bf16) or 32 (fp8)
      // consecutive depth elements per step and lane half.
      QFrag qf[C::QK_STEPS];
      bf16x8 qr[C::ROPE_STEPS > 0 ? C::ROPE_STEPS : 1];
#pragma unroll
      for (int s = 0; s < C::QK_STEPS; ++s) {
        if constexpr (C::FP8) {
          i32x8 x = {0, 0, 0, 0, 0, 0, 0, 0};
          if (qvalid) {
            const i32x4* src =
                reinterpret_cast<const i32x4*>(qp + qrow * C::DN + s * 64 + 32 * hf);
            const i32x4 a0 = src[0], a1 = src[1];
            x = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          }
          qf[s] = x;
        } else {
          i32x4 x = {0, 0, 0, 0};
          if (qvalid) x = *reinterpret_cast<const i32x4*>(qp + (qrow * C::DN + s * 16 + 8 * hf) * 2);
          qf[s] = __builtin_bit_cast(bf16x8, x);
        }
      }
#pragma unroll
      for (int s = 0; s < C::ROPE_STEPS; ++s) {
        i32x4 x = {0, 0, 0, 0};
        if (qvalid) x = *reinterpret_cast<const i32x4*>(qrp + (qrow * C::DR + s * 16 + 8 * hf) * 2);
        qr[s] = __builtin_bit_cast(bf16x8, x);
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

      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMA of block 0 landed
      __syncthreads();

      // Causal: this wave sees keys up to wq0 + 31 only, so its last
      // blocks may be fully masked; it then only keeps the DMA/barrier
      // rhythm of the workgroup (a separate loop, so that the accumulators
      // never flow through a skip path).
      const int wave_nblocks =
          p.causal ? min(nblocks, ((wq0 + 31) >> 6) + 1) : nblocks;
      int kb = 0;
      for (; kb < wave_nblocks; ++kb) {
        const int kbase = kb * C::BN;
        const char* stage = smem + (kb & 1) * C::STAGE;
        if (kb + 1 < nblocks)
          load_block(p, smem + ((kb + 1) & 1) * C::STAGE, wave, lane, s0, L, g, kbase + C::BN);
        // ---- S^T = K Q^T : two 32-key tiles
        f32x16 st[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          f32x16 acc;
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r] = 0.f;
          const int r = kt * 32 + lane32;
#pragma unroll
          for (int s = 0; s < C::QK_STEPS; ++s) acc = mfma_qk(k_frag(stage, r, s, hf), qf[s], acc);
#pragma unroll
          for (int s = 0; s < C::ROPE_STEPS; ++s)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(krope_frag(stage, r, s, hf), qr[s],
                                                          acc, 0, 0, 0);
          st[kt] = acc;
        }

        // ---- per-key scale (fp8), mask, block row max
        if constexpr (C::FP8) {
          const float* ksl = reinterpret_cast<const float*>(stage + C::KS_OFF);
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
              const f32x4 ks = *reinterpret_cast<const f32x4*>(ksl + kt * 32 + 8 * a4 + 4 * hf);
#pragma unroll
              for (int r = 0; r < 4; ++r) st[kt][4 * a4 + r] *= ks[r];
            }
        }
        const bool need_mask = (kbase + C::BN > L) || (p.causal && kbase + C::BN - 1 > wq0);
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

        // ---- P = 2^(cq*S - m) -> bf16 B-operand fragments
        bf16x8 pb[4];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            st[kt][r] = fast_exp2(fmaf(st[kt][r], cq, -m_use));
            l += st[kt][r];
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
#pragma unroll
        for (int t = 0; t < C::DV_TILES; ++t)
#pragma unroll
          for (int u = 0; u < 4; ++u)
            o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_frag(stage, t, u, lane), pb[u],
                                                           o[t], 0, 0, 0);

        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMA of the next block landed
        __syncthreads();
      }
      for (; kb < nblocks; ++kb) {
        if (kb + 1 < nblocks)
          load_block(p, smem + ((kb + 1) & 1) * C::STAGE, wave, lane, s0, L, g,
                     (kb + 1) * C::BN);
        __builtin_amdgcn_s_waitcnt(0x0F70);
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
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
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
