// Matrix-core attention forward for bf16 and fp8 (E4M3) Q/K on gfx950.
//
// One work item = one (sequence, query head, 128-row query tile).  A
// workgroup is 4 waves; wave w owns query rows 32w .. 32w+31 of the tile.
// The tile of Q stays in registers for the whole item; K and V stream past
// in 64-key blocks through LDS rings (the Q-stationary tiling with staged
// K/V buffers of the pages: SM100AttentionSMem, comptime members q_bytes,
// k_stage_bytes, v_stage_bytes; TMAProducerPipeline, acquire / commit_step).
//
// Staging.  K (+ K_rope, + the fp8 k_scale) and V of coming blocks are
// copied HBM -> LDS by buffer_load ... lds while the current block is
// computed: each lane moves 16 bytes straight into LDS (lane i of an
// instruction lands at byte 16 i of a 1 KiB run), with no register staging
// and no VALU work.  The buffer resource of a block ends at the sequence's
// last key, so rows past the end arrive as zeros.  Rows are stored as
// 16-byte chunks in XOR-swizzled order (the global side picks which chunk
// each lane fetches), so the matrix-core operand reads are free of LDS bank
// conflicts.  The K ring runs one block ahead of the V ring.
//
// Math per 64-key block j, per wave:
//   S^T = K Q^T on the matrix cores (v_mfma_f32_32x32x16_bf16, or for fp8
//         v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales).  Keys run
//         along the MFMA M axis and queries along N, so in the 32x32 output
//         layout lane i holds 16 keys of ONE query row (i % 32); lanes i and
//         i ^ 32 hold the other 16.  Row max is in-lane v_max3 plus one
//         v_permlane32_swap; row sums stay per lane until the end.
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
//         A-operand V^T fragments come from ds_read_b64_tr_b16.
//
// Schedule.  A 32x32x16 MFMA occupies the matrix pipe for ~32 cycles, of
// which ~16-18 can overlap VALU work issued by the same wave (measured on
// MI355X).  Each block is therefore written as two explicit software-
// pipelined phases, slot by slot, with its operand read issued two slots
// ahead:
//   phase A  the S products of block j+1, each followed by a share of block
//            j's exponentials, row sums and bf16 packing;
//   phase B  block j's P V products, in the second half each followed by a
//            share of block j+1's (fp8 k_scale and) row max.
// Epilogue: O / l, bf16 round-to-nearest-even, staged through LDS for
// coalesced 16-byte stores (the pages reuse the Q region for this,
// SM100AttentionSMem Methods: o_smem), and LSE in natural log.
#pragma once

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mha {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

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
  // LDS: a K ring and a V ring of two slots each.
  //   K slot: K nope rows | K rope rows | k_scale (fp8)      V slot: V rows
  //   [K0 | K1 | V0 | V1]
  static constexpr int K_OFF = 0;                      // inside a K slot
  static constexpr int R_OFF = BN * K_RB;              // inside a K slot
  static constexpr int KS_OFF = R_OFF + BN * R_RB;     // inside a K slot
  static constexpr int KSLOT = KS_OFF + (FP8 ? 256 : 0);  // 64 floats, padded to 256 B
  static constexpr int VSLOT = BN * V_RB;
  static constexpr int V_BASE = 2 * KSLOT;
  static constexpr int LDS = V_BASE + 2 * VSLOT;
  // two workgroups per CU when the rings fit twice in 160 KiB
  static constexpr int OCC = 2 * LDS + 64 <= 160 * 1024 ? 2 : 1;
  static constexpr int O_ROW = DV * 2 + 16;  // epilogue staging row stride
  static constexpr int QK_STEPS = FP8 ? DN / 64 : DN / 16;  // nope MFMA k-steps
  static constexpr int ROPE_STEPS = DR / 16;
  static constexpr int S_STEPS = QK_STEPS + ROPE_STEPS;   // per 32-key tile
  static constexpr int NA = 2 * S_STEPS;                  // S products per block
  static constexpr int DV_TILES = DV / 32;
  static constexpr int NB = 4 * DV_TILES;                 // P V products per block

  static_assert(!FP8 || DR == 0, "fp8 Q/K carry no rope part");
  static_assert(K_RB == 128 || K_RB == 256, "K rows of 128 or 256 bytes");
  static_assert(DR == 0 || R_RB == 128, "rope rows of 128 bytes");
  static_assert(V_RB == 128 || V_RB == 256, "V rows of 128 or 256 bytes");
  static_assert((BN * K_RB / 1024) % WAVES == 0 && (BN * R_RB / 1024) % WAVES == 0 &&
                    (BN * V_RB / 1024) % WAVES == 0,
                "DMA instructions split evenly over the waves");
  static_assert(KSLOT % 256 == 0 && VSLOT % 256 == 0, "slots keep 256-byte row alignment");
  static_assert(WAVES * 32 * O_ROW <= LDS, "epilogue staging must fit in the rings");
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

// Keep the compiler from moving anything across this point (the explicit
// pipeline slots below are laid out in source order).
#define MHA_SLOT_FENCE() __builtin_amdgcn_sched_barrier(0)

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

template <class C>
struct MfmaKernel {
  using QFrag = typename std::conditional<C::FP8, i32x8, bf16x8>::type;

  // ------------------------------------------------------------ staging

  // One 16-byte-per-lane DMA instruction: buffer_load_dwordx4 ... lds writes
  // lane i's 16 bytes at LDS address m0 + 16 i.  (m0 is set here; nothing
  // else in these kernels keeps a value in m0.)  Issued from inline assembly
  // so that the compiler does not treat it as a pending write to every LDS
  // address (it would otherwise wait for it before each LDS read of the
  // other slots); completion is awaited explicitly with vmcnt(0) before the
  // barrier that publishes the slot.
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

  // This wave's share of the DMA of one row-major region of BN rows of RB
  // bytes.  Instruction n covers rows RPI*n .. RPI*n+RPI-1; lane i fills
  // position i % CPR of row RPI*n + i / CPR with the chunk that the swizzle
  // puts there.
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

  struct Rows {
    size_t row0;    // first [T, Hkv] row of the block
    uint32_t span;  // [T, Hkv] rows touched by the block's keys
  };
  static __device__ __forceinline__ Rows block_rows(const AttnParams& p, int s0, int L, int g,
                                                   int kbase) {
    const int rows = min(L - kbase, C::BN);  // >= 1
    return Rows{(size_t)(s0 + kbase) * p.num_kv_heads + g,
                (uint32_t)((rows - 1) * p.num_kv_heads + 1)};
  }
  // K, K rope and the fp8 k_scale of the block at kbase into a K slot.
  static __device__ __forceinline__ void load_k(const AttnParams& p, const char* kslot, int wave,
                                                int lane, int s0, int L, int g, int kbase) {
    const Rows b = block_rows(p, s0, L, g, kbase);
    const int Hkv = p.num_kv_heads;
    dma_region<C::K_RB, false>(
        kslot + C::K_OFF,
        rsrc_of(static_cast<const char*>(p.k) + b.row0 * C::K_RB, b.span * C::K_RB),
        Hkv * C::K_RB, wave, lane);
    if constexpr (C::DR > 0)
      dma_region<C::R_RB, false>(
          kslot + C::R_OFF,
          rsrc_of(static_cast<const char*>(p.k_rope) + b.row0 * C::R_RB, b.span * C::R_RB),
          Hkv * C::R_RB, wave, lane);
    if constexpr (C::FP8) {
      if (wave == 0)
        dma4(rsrc_of(p.k_scale + b.row0, b.span * 4),
             __builtin_amdgcn_readfirstlane(lds_addr_of(kslot + C::KS_OFF)),
             (uint32_t)(lane * Hkv * 4));
    }
  }
  // V of the block at kbase into a V slot.
  static __device__ __forceinline__ void load_v(const AttnParams& p, const char* vslot, int wave,
                                                int lane, int s0, int L, int g, int kbase) {
    const Rows b = block_rows(p, s0, L, g, kbase);
    dma_region<C::V_RB, true>(
        vslot, rsrc_of(static_cast<const char*>(p.v) + b.row0 * C::V_RB, b.span * C::V_RB),
        p.num_kv_heads * C::V_RB, wave, lane);
  }

  // ------------------------------------------------------------ operands

  // A operand of S product a of a block: 32-key tile kt = a % 2 (the two
  // tiles alternate, so consecutive products are independent), depth step
  // a / 2 (nope steps first, then rope steps).
  static __device__ __forceinline__ QFrag s_frag(const char* kslot, int a, int lane32, int hf) {
    const int kt = a & 1, s = a >> 1;
    const int r = kt * 32 + lane32;
    if constexpr (C::FP8) {
      const char* row = kslot + C::K_OFF + r * C::K_RB;
      const int sw = swz_k<C::K_RB>(r);
      const int c0 = 4 * s + 2 * hf;  // 32 bytes = chunks c0, c0 + 1
      const i32x4 a0 = *reinterpret_cast<const i32x4*>(row + 16 * (c0 ^ sw));
      const i32x4 a1 = *reinterpret_cast<const i32x4*>(row + 16 * ((c0 + 1) ^ sw));
      return i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    } else {
      if (s < C::QK_STEPS) {
        const char* row = kslot + C::K_OFF + r * C::K_RB;
        return *reinterpret_cast<const bf16x8*>(row + 16 * ((2 * s + hf) ^ swz_k<C::K_RB>(r)));
      }
      const int sr = s - C::QK_STEPS;
      const char* row = kslot + C::R_OFF + r * C::R_RB;
      return *reinterpret_cast<const bf16x8*>(row + 16 * ((2 * sr + hf) ^ swz_k<C::R_RB>(r)));
    }
  }
  static __device__ __forceinline__ f32x16 s_mfma(const QFrag& a, const QFrag& b, f32x16 acc) {
    if constexpr (C::FP8)
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
    else
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }

  // A operand of P V product b of a block: dv tile t = b % DV_TILES, keys
  // 16u .. 16u+15 with u = b / DV_TILES.  Slot (lane half h, element i)
  // holds key 16u + 8(i/4) + 4h + i%4 of column 32t + lane % 32, matching the
  // P^T B-operand slots.  Within each group of 16 lanes, ds_read_b64_tr_b16
  // gives lane i, element k, the element i % 4 of the 8 bytes addressed by
  // lane 4k + i/4; so lane s of the group addresses key (base + s/4) at
  // columns 4(s%4) .. 4(s%4)+3.
  static __device__ __forceinline__ bf16x8 v_frag(const char* vslot, int b, int lane) {
    const int t = b % C::DV_TILES, u = b / C::DV_TILES;
    const int grp = lane >> 4, s = lane & 15;
    const int h = grp >> 1;
    const int dv = t * 32 + 16 * (grp & 1) + 4 * (s & 3);  // first of this lane's 4 columns
    const int c = dv >> 3, sub = (dv & 7) * 2;               // chunk and byte inside it
    const int k1 = 16 * u + 4 * h + (s >> 2), k2 = k1 + 8;
    const char* a1 = vslot + k1 * C::V_RB + 16 * (c ^ swz_v<C::V_RB>(k1)) + sub;
    const char* a2 = vslot + k2 * C::V_RB + 16 * (c ^ swz_v<C::V_RB>(k2)) + sub;
    const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a1));
    const i16x4 r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a2));
    const i16x8 r = {r1[0], r1[1], r1[2], r1[3], r2[0], r2[1], r2[2], r2[3]};
    return __builtin_bit_cast(bf16x8, r);
  }

  // ------------------------------------------------------------ pieces

  // Per-wave state of one work item.
  struct State {
    f32x16 o[C::DV_TILES];  // O^T accumulator (lane = query, 16 dv rows per tile)
    f32x16 st[2];           // S^T of the current block (fp8: k_scale applied)
    float mx;               // cq * row max of st (valid unless the block is masked)
    float m;                // running max (log2 domain), same in lanes i and i ^ 32
    float l;                // this lane's partial row sum
  };

  static __device__ __forceinline__ void scale_and_max(const char* kslot, int hf, float cq,
                                                       f32x16 (&st)[2], float& mx) {
    if constexpr (C::FP8) {
      const float* ks = reinterpret_cast<const float*>(kslot + C::KS_OFF);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const f32x4 k4 = *reinterpret_cast<const f32x4*>(ks + kt * 32 + 8 * a4 + 4 * hf);
#pragma unroll
          for (int r = 0; r < 4; ++r) st[kt][4 * a4 + r] *= k4[r];
        }
    }
    float x = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) x = fmaxf(x, st[kt][r]);
    mx = half_max(x) * cq;
  }

  // Plain (not pipelined) S of one block from a K slot, with the fp8
  // k_scale and the row max: used for block 0.
  static __device__ __forceinline__ void s_block(const char* kslot, const QFrag* qf, int lane32,
                                                 int hf, float cq, State& w) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) w.st[kt][r] = 0.f;
#pragma unroll
    for (int a = 0; a < C::NA; ++a)
      w.st[a & 1] = s_mfma(s_frag(kslot, a, lane32, hf), qf[a >> 1], w.st[a & 1]);
    scale_and_max(kslot, hf, cq, w.st, w.mx);
  }

  // Mask of a block that crosses the causal diagonal or the sequence end
  // (hidden keys -> -inf) and its row max.
  static __device__ __forceinline__ void mask_block(State& w, int kbase, int lim, int hf,
                                                    float cq) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kbase + kt * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (key > lim) w.st[kt][r] = -INFINITY;
      }
    float x = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) x = fmaxf(x, w.st[kt][r]);
    w.mx = half_max(x) * cq;
  }

  // Lazy correction of the running statistics; returns the exponent offset.
  static __device__ __forceinline__ float correct(State& w) {
    if (wave_any(w.mx > w.m + 8.0f)) {
      const float m_new = fmaxf(w.m, w.mx);
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(w.m - m_new);
      w.l *= alpha;
#pragma unroll
      for (int t = 0; t < C::DV_TILES; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) w.o[t][r] *= alpha;
      w.m = m_new;
    }
    return w.m == -INFINITY ? 0.f : w.m;
  }

  // Exponentials of elements [LO, HI) of the 32 S values of a lane (element
  // e is st[e / 16][e % 16]), with each finished pair packed to bf16.
  template <int LO, int HI>
  static __device__ __forceinline__ void exp_chunk(f32x16 (&st)[2], float cq, float m_use,
                                                   uint32_t (&pw)[16], float (&ls)[2]) {
#pragma unroll
    for (int e = LO; e < HI; ++e) {
      st[e >> 4][e & 15] = fast_exp2(fmaf(st[e >> 4][e & 15], cq, -m_use));
      ls[e & 1] += st[e >> 4][e & 15];
      if (e & 1) pw[e >> 1] = pack_bf16x2(st[(e - 1) >> 4][(e - 1) & 15], st[e >> 4][e & 15]);
    }
  }

  // One pipelined block.  NEXT: compute S of the following block (K slot
  // kn) alongside.  On entry w.st holds this block's S (scaled, masked) and
  // w.mx its row max; on exit they hold the next block's.
  template <bool NEXT>
  static __device__ __forceinline__ void block(State& w, const char* kn, const char* vslot,
                                               const QFrag* qf, int lane, int lane32, int hf,
                                               float cq) {
    const float m_use = correct(w);
    uint32_t pw[16];  // P as packed bf16 pairs: pw[4u + i] = dword i of B operand u
    float ls[2] = {0.f, 0.f};
    f32x16 sn[2];
    MHA_SLOT_FENCE();

    // ---- phase A: S products of the next block + exponentials of this one
    if constexpr (NEXT) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) sn[kt][r] = 0.f;
      QFrag kf[3];
      kf[0] = s_frag(kn, 0, lane32, hf);
      kf[1] = s_frag(kn, 1, lane32, hf);
      static_for<0, C::NA>([&](auto ac) {
        constexpr int a = decltype(ac)::value;
        if constexpr (a + 2 < C::NA) kf[(a + 2) % 3] = s_frag(kn, a + 2, lane32, hf);
        sn[a & 1] = s_mfma(kf[a % 3], qf[a >> 1], sn[a & 1]);
        exp_chunk<a * 32 / C::NA, (a + 1) * 32 / C::NA>(w.st, cq, m_use, pw, ls);
        MHA_SLOT_FENCE();
      });
    } else {
      exp_chunk<0, 32>(w.st, cq, m_use, pw, ls);
    }

    // ---- phase B: P V products (+ next block's scale and max)
    bf16x8 pb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      pb[u] = __builtin_bit_cast(
          bf16x8, i32x4{(int)pw[4 * u], (int)pw[4 * u + 1], (int)pw[4 * u + 2], (int)pw[4 * u + 3]});
    float mxp = -INFINITY;
    const float* ks = reinterpret_cast<const float*>(kn + C::KS_OFF);
    bf16x8 vf[3];
    vf[0] = v_frag(vslot, 0, lane);
    vf[1] = v_frag(vslot, 1, lane);
    static_for<0, C::NB>([&](auto bc) {
      constexpr int b = decltype(bc)::value;
      if constexpr (b + 2 < C::NB) vf[(b + 2) % 3] = v_frag(vslot, b + 2, lane);
      w.o[b % C::DV_TILES] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          vf[b % 3], pb[b / C::DV_TILES], w.o[b % C::DV_TILES], 0, 0, 0);
      // next block's k_scale and row max over the second half of the slots
      if constexpr (NEXT && 2 * b >= C::NB) {
        constexpr int H = C::NB / 2, q = b - C::NB / 2;
#pragma unroll
        for (int e = q * 32 / H; e < (q + 1) * 32 / H; ++e) {
          if constexpr (C::FP8)
            sn[e >> 4][e & 15] *= ks[(e >> 4) * 32 + 8 * ((e & 15) >> 2) + 4 * hf + (e & 3)];
          mxp = fmaxf(mxp, sn[e >> 4][e & 15]);
        }
      }
      MHA_SLOT_FENCE();
    });
    w.l += ls[0] + ls[1];
    if constexpr (NEXT) {
      w.st[0] = sn[0];
      w.st[1] = sn[1];
      w.mx = half_max(mxp) * cq;
    }
  }

  // ------------------------------------------------------------ kernel body

  static __device__ void run(const AttnParams& p, char* smem) {
    __shared__ i32x4 s_item[2];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int lane32 = lane & 31;
    const int hf = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = p.cu_seqlens[p.batch];
    const char* __restrict__ qp = static_cast<const char*>(p.q);
    const char* __restrict__ qrp = static_cast<const char*>(p.q_rope);
    char* __restrict__ op = static_cast<char*>(p.o);

    // wave 0 runs the work-item source; the next item's table entry is read
    // while the current item's first blocks load and published at the first
    // barrier after that
    Fetcher fetch;
    if (wave == 0) {
      fetch.init(p.sched);
      const i32x4 e0 = fetch.take(p.sched, p.table);
      if (tid == 0) s_item[0] = e0;
    }
    for (int it = 0;; ++it) {
      __syncthreads();
      // the item is the same for the whole workgroup: keep it in SGPRs
      const WorkItem wi = decode_item(i32x4{__builtin_amdgcn_readfirstlane(s_item[it & 1][0]),
                                            __builtin_amdgcn_readfirstlane(s_item[it & 1][1]),
                                            __builtin_amdgcn_readfirstlane(s_item[it & 1][2]),
                                            __builtin_amdgcn_readfirstlane(s_item[it & 1][3])});
      if (wi.L < 0) break;
      i32x4 nxt;
      if (wave == 0) nxt = fetch.take(p.sched, p.table);
      const int s0 = wi.s0;
      const int L = wi.L;
      const int g = wi.h / p.group;
      const int q0 = wi.qt * C::BM;    // first query row of the tile
      const int wq0 = q0 + wave * 32;  // first query row of this wave
      const int qi = wq0 + lane32;     // this lane's query row
      const bool qvalid = qi < L;
      const size_t qrow = (size_t)(s0 + qi) * p.num_heads + wi.h;

      const int n_kv = p.causal ? min(L, q0 + C::BM) : L;
      const int nblocks = (n_kv + C::BN - 1) / C::BN;
      // blocks this wave computes (causal: keys up to wq0 + 31 only), and the
      // leading ones among them that need no mask
      const int wave_nblocks = p.causal ? min(nblocks, ((wq0 + 31) >> 6) + 1) : nblocks;
      const int n_full = (p.causal ? min(L, wq0 + 1) : L) / C::BN;
      const int lim = p.causal ? min(L - 1, qi) : L - 1;  // last key visible to this lane

      load_k(p, smem, wave, lane, s0, L, g, 0);
      load_v(p, smem + C::V_BASE, wave, lane, s0, L, g, 0);

      // Q fragments (B operand): lane -> query qi, 8 (bf16) or 32 (fp8)
      // consecutive depth elements per step and lane half; rope steps follow
      // the nope steps.
      QFrag qf[C::S_STEPS];
#pragma unroll
      for (int s = 0; s < C::S_STEPS; ++s) {
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
          if (qvalid) {
            const char* src = s < C::QK_STEPS
                                  ? qp + (qrow * C::DN + s * 16 + 8 * hf) * 2
                                  : qrp + (qrow * C::DR + (s - C::QK_STEPS) * 16 + 8 * hf) * 2;
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

      State w;
#pragma unroll
      for (int t = 0; t < C::DV_TILES; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) w.o[t][r] = 0.f;
      w.m = -INFINITY;
      w.l = 0.f;

      // prologue: block 0's K and V (and the next item's entry) land; S_0;
      // K_1 lands
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMA landed
      if (tid == 0) s_item[(it + 1) & 1] = nxt;
      __syncthreads();
      s_block(smem, qf, lane32, hf, cq, w);
      if (nblocks > 1) load_k(p, smem + C::KSLOT, wave, lane, s0, L, g, C::BN);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();

      // Block j: K_{j+2} -> K slot j%2 and V_{j+1} -> V slot (j+1)%2 go out
      // first (both slots were last read in block j-1); the block then reads
      // K slot (j+1)%2 and V slot j%2; every wave ends it at one barrier.
      // The slot parity is a template argument (blocks are taken in pairs),
      // so every LDS operand address is a per-lane offset plus a constant.
      auto issue = [&](auto par, int j) {
        constexpr int P = decltype(par)::value;
        if (j + 2 < nblocks) load_k(p, smem + P * C::KSLOT, wave, lane, s0, L, g, (j + 2) * C::BN);
        if (j + 1 < nblocks)
          load_v(p, smem + C::V_BASE + (1 - P) * C::VSLOT, wave, lane, s0, L, g, (j + 1) * C::BN);
      };
      auto finish = [&]() {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMA landed
        __syncthreads();
      };
      auto step = [&](auto next, auto par, int j) {
        constexpr bool NEXT = decltype(next)::value;
        constexpr int P = decltype(par)::value;
        issue(par, j);
        if (j >= n_full) mask_block(w, j * C::BN, lim, hf, cq);
        block<NEXT>(w, smem + (1 - P) * C::KSLOT, smem + C::V_BASE + P * C::VSLOT, qf, lane,
                    lane32, hf, cq);
        finish();
      };
      using Even = std::integral_constant<int, 0>;
      using Odd = std::integral_constant<int, 1>;
      using Yes = std::true_type;
      using No = std::false_type;
      int j = 0;
      for (; j + 2 < wave_nblocks; j += 2) {
        step(Yes{}, Even{}, j);
        step(Yes{}, Odd{}, j + 1);
      }
      if (j + 1 < wave_nblocks) {
        step(Yes{}, Even{}, j);
        ++j;
      }
      // this wave's last block: no next S
      if (j & 1)
        step(No{}, Odd{}, j);
      else
        step(No{}, Even{}, j);
      ++j;
      // causal: blocks past this wave's last visible key -- keep the
      // workgroup's DMA / barrier rhythm only
      for (; j < nblocks; ++j) {
        if (j & 1)
          issue(Odd{}, j);
        else
          issue(Even{}, j);
        finish();
      }

      // ---- epilogue
      const float lt = half_sum(w.l);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      char* ost = smem + wave * 32 * C::O_ROW + lane32 * C::O_ROW;
#pragma unroll
      for (int t = 0; t < C::DV_TILES; ++t)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int dv0 = t * 32 + 8 * a4 + 4 * hf;
          const uint32_t lo = pack_bf16x2(w.o[t][4 * a4 + 0] * inv, w.o[t][4 * a4 + 1] * inv);
          const uint32_t hi = pack_bf16x2(w.o[t][4 * a4 + 2] * inv, w.o[t][4 * a4 + 3] * inv);
          *reinterpret_cast<i32x2*>(ost + dv0 * 2) = i32x2{(int)lo, (int)hi};
        }
      if (hf == 0 && qvalid)
        p.lse[(size_t)wi.h * T + s0 + qi] = lt > 0.f ? (w.m + log2f(lt)) * kLn2 : -INFINITY;
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
          *reinterpret_cast<i32x4*>(op + (((size_t)(s0 + row) * p.num_heads + wi.h) * C::DV) * 2 +
                                    cc * 16) = x;
        }
      }
    }
  }
};

template <class C>
__global__ __launch_bounds__(C::THREADS, C::OCC) void attn_fwd_mfma_kernel(AttnParams p) {
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
