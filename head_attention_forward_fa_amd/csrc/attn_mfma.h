// Matrix-core attention forward for bf16 and fp8 (E4M3) Q/K on gfx950.
//
// One work item = one (sequence, query head, 256-row query tile).  A
// workgroup is 8 waves (two per SIMD); wave w owns query rows 32w .. 32w+31
// of the tile.  The tile of Q stays in registers for the whole item; K and V
// stream past in 64-key blocks through LDS rings (the Q-stationary tiling
// with staged K/V buffers of the pages: SM100AttentionSMem, comptime members
// q_bytes, k_stage_bytes, v_stage_bytes; TMAProducerPipeline, acquire /
// commit_step).
//
// Staging.  K (+ K_rope, + the fp8 k_scale) and V of coming blocks are
// copied HBM -> LDS by buffer_load ... lds: each lane moves 16 bytes straight
// into LDS (lane i of an instruction lands at byte 16 i of a 1 KiB run), with
// no register staging.  The K ring has 4 slots (3 with a rope part) and the
// V ring 4, so block j+3's K and block j+2's V are requested while block j
// is computed, two blocks before they are needed (exact fp8 without rope:
// the fp8 K rows are staged four blocks ahead and decoded to bf16 K slots
// by the whole workgroup two blocks ahead); each wave spreads its few DMA instructions
// over the matrix-core slots of the block's first step instead of issuing
// them in one burst.  A block's buffer resource ends at the sequence's last
// key, so rows past the end arrive as zeros.  K rows are stored at a pitch of
// row + 16 bytes (consecutive rows start 4 banks apart, so the rows that one
// operand read touches at a time fall on distinct banks, and every K operand
// address is a per-lane base plus an immediate); V rows are unpadded, with
// their 16-byte chunks in XOR-swizzled order for the transposed reads.
//
// Math per 32-key sub-tile i, per wave:
//   S^T = K Q^T on the matrix cores (v_mfma_f32_32x32x16_bf16, or for fp8
//         v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales).  Keys run
//         along the MFMA M axis and queries along N, so in the 32x32 output
//         layout lane i holds 16 keys of ONE query row (i % 32); lanes i and
//         i ^ 32 hold the other 16.  Row max is in-lane v_max3 plus one
//         v_permlane32_swap; row sums stay per lane until the end.
//   fp8:  S_ij *= k_scale_j, with q_scale_i folded into the exponent
//         multiplier, after the product (per-token scales staged per tile:
//         SM100AttentionSMem, Methods q_scale_smem, k_scale_smem).
//   mask: only the wave's last sub-tile can cross the causal diagonal or the
//         sequence end (sub-tiles and wave rows are both 32-aligned).
//   online softmax in the log2 domain: m is a running row max of
//         sigma*log2(e)*S; P = 2^(sigma*log2(e)*S - m) via v_exp_f32.  The
//         correction of O and l (the per-row correction buffer of
//         SM100AttentionSMem, Methods: correction_smem) is applied lazily:
//         P is computed against the current m, and only when a lane's sum of
//         P exceeds 2^32 (or at an item's first sub-tile) is the row max
//         taken, O and l corrected and P recomputed, so almost every
//         sub-tile spends no vector work on maxima; O and l always share the
//         same stale m, so O / l and LSE = (m + log2 l) ln 2 are unchanged.
//   O^T += V^T P^T on the matrix cores.  P^T is already in the B-operand
//         layout (lane = query, 8 k-slots), so it goes from the S registers to
//         the PV product with one v_cvt_pk_bf16_f32 per pair.  V stays
//         row-major in LDS ("mn-major" V of TMAProducerPipeline); the
//         A-operand V^T fragments come from ds_read_b64_tr_b16.
//
// Schedule.  Each sub-tile step is two software-pipelined phases, written
// slot by slot with operand reads issued two slots ahead:
//   phase A  the S products of sub-tile i+1 and sub-tile i's exponentials,
//            row sums and bf16 packing;
//   phase B  sub-tile i's P V products and sub-tile i+1's (fp8 k_scale and)
//            row max.
// The machine scheduler interleaves the independent vector work with the
// matrix-core ops inside a step; the two waves that share a SIMD overlap
// one's softmax with the other's products.
// Pipelining at 32 keys keeps only two 32x32 S tiles live, which leaves the
// registers for O, Q and the operand buffers within 256 VGPRs (two waves per
// SIMD).  One barrier per 64-key block publishes the DMA'd slots.
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

// FP8_: Q/K nope parts are OCP E4M3 codes with per-token scales.  F8MMA_:
// their products run on the fp8 matrix instruction, whose accumulation keeps
// only about 13 bits below the largest of the 64 products of one
// instruction (measured on gfx950: error up to 2^-13 of the sum of the
// products' magnitudes, where a bf16 product of the same values errs by
// 2^-22); without it the codes are decoded to bfloat16 (exact: E4M3 has 3
// mantissa bits and exponents well inside bfloat16's range) and the
// products run on the bf16 instruction with float32-grade accumulation.
template <int DN_, int DR_, int DV_, bool FP8_, bool F8MMA_ = FP8_>
struct MfmaCfg {
  static constexpr int DN = DN_, DR = DR_, DV = DV_;
  static constexpr bool FP8 = FP8_;
  static constexpr bool F8MMA = FP8_ && F8MMA_;
  // fp8 nope with a bfloat16 rope part: the per-token scales multiply the
  // nope product only, so the two products accumulate separately
  static constexpr bool MIXED = FP8 && DR > 0;
  static constexpr int BM = kBlockM_Mfma;  // 256 query rows per item
  static constexpr int BN = kBlockN_Mfma;  // 64 keys per block
  static constexpr int WAVES = BM / 32;    // 8 waves, two per SIMD
  static constexpr int THREADS = WAVES * kWave;
  // SD: exact fp8 decodes each K block once, for the whole workgroup: the
  // fp8 nope rows land in a staging ring and are written back as bfloat16
  // rows into the K ring, which the products then read as in the bf16
  // kernel.  With a rope part (SDR) the K block is staged by depth: the
  // nope depth through the staging ring and the decode, the bfloat16 rope
  // depth straight into its K slot one block later (the depth-staged K of
  // the pages' TMAProducerPipeline, K staged in num_qk_stages chunks), so
  // that the decoded ring fits in 160 KiB (see NSS, JUNK).
  static constexpr bool SD = FP8 && !F8MMA;
  static constexpr bool SDR = SD && DR > 0;
  static constexpr int EB = FP8 ? 1 : 2;   // bytes per Q/K nope element
  static constexpr int K_HB = DN * EB;     // bytes per K nope row in HBM
  static constexpr int K_RB = SD ? DN * 2 : K_HB;  // bytes per K nope row in a K slot
  static constexpr int R_RB = DR * 2;      // bytes per K rope row
  static constexpr int V_RB = DV * 2;      // bytes per V row
  // LDS: [K slots | V slots | sink]; block b lives in K slot b % NKS and V
  // slot b % NVS.
  //   K slot: K nope rows | K rope rows | k_scale (fp8)      V slot: V rows
  static constexpr int NVS = 4;
  static constexpr int K_RP = K_RB + 16;               // padded K row pitch
  static constexpr int R_RP = DR > 0 ? R_RB + 16 : 0;  // padded rope row pitch
  static constexpr int K_OFF = 0;                      // inside a K slot
  static constexpr int R_OFF = BN * K_RP;              // inside a K slot
  static constexpr int KS_OFF = R_OFF + BN * R_RP;     // inside a K slot
  static constexpr int KSLOT = (KS_OFF + (FP8 ? 256 : 0) + 255) / 256 * 256;
  static constexpr int VSLOT = BN * V_RB;
  // SD staging slot: fp8 rows (unpadded), k_scale.  3 slots (staged four
  // blocks ahead); SDR: 2 (staged three blocks ahead, two slots being what
  // fits next to the decoded K ring with its rope rows and the V ring)
  static constexpr int NSS = SD ? (SDR ? 2 : 3) : 0;
  static constexpr int SSLOT = SD ? BN * K_HB + 256 : 0;
  // 4 K slots when they fit next to the V ring, else 3 (the rope layout);
  // SD: 3 (a decoded block is written one block before its first use)
  static constexpr int NKS =
      SD ? 3 : 4 * KSLOT + NVS * BN * V_RB + 1024 + 64 <= 160 * 1024 ? 4 : 3;
  // blocks between a K block's request and its use (SD: the staged rows'
  // request and their decode); RLEAD: the same for the rope rows, which
  // SDR requests into their K slot directly
  static constexpr int KLEAD = SD ? (SDR ? 3 : 4) : NKS - 1;
  static constexpr int RLEAD = SDR ? 2 : KLEAD;
  // batch j's K-side DMA may still be in flight at barrier j (its data is
  // first used, or decoded, after barrier j + 1)
  static constexpr bool K_SLACK = KLEAD >= 3 && !SDR;
  static constexpr int S_BASE = NKS * KSLOT;
  static constexpr int V_BASE = S_BASE + NSS * SSLOT;
  // 1 KiB sink for DMA ops past a region's end.  SDR has none (160 KiB):
  // such ops repeat the region's last instruction, the same bytes to the
  // same place, and the k_scale op of every wave is wave 0's.
  static constexpr bool NOJUNK = SDR;
  static constexpr int JUNK = V_BASE + NVS * VSLOT;
  static constexpr int LDS = JUNK + (NOJUNK ? 0 : 1024);
  static constexpr int OCC = 1;              // one workgroup (8 waves) per CU
  static constexpr int O_ROW = DV * 2 + 16;  // epilogue staging row stride
  static constexpr int QK_STEPS = F8MMA ? DN / 64 : DN / 16;  // nope MFMA k-steps
  static constexpr int ROPE_STEPS = DR / 16;
  static constexpr int S_STEPS = QK_STEPS + ROPE_STEPS;  // S products per sub-tile
  static constexpr int DV_TILES = DV / 32;
  static constexpr int NPV = 2 * DV_TILES;  // P V products per sub-tile
  static constexpr int G_AHEAD = 2;         // products between an operand read and its use
  // The first KPF S operand fragments of a product half-step are read at
  // the start of the softmax half-step before it, whose vector work then
  // covers their latency (a wave reads LDS at a limited rate, and does not
  // read it at all in its softmax half-steps otherwise).  Two measured best
  // on the bf16 layouts (three and four gained less); the others keep none.
  static constexpr int KPF = (!FP8 && DR == 0) ? 2 : 0;
  // 1 KiB DMA instructions per block and region.  The waves of group 0
  // (DW of them, one per SIMD) issue them: wave w takes instructions w,
  // w + DW, ... of each region (the fp8 k_scale: wave 0, one dword per
  // lane).  Each of them issues the same N_OPS instructions per block: the
  // ones past a region's end and another wave's k_scale read nothing and
  // land in the JUNK sink (NOJUNK: they repeat an existing instruction), and
  // those of a block that does not exist read nothing (empty buffer range),
  // so one vmcnt(N_OPS) wait fits every wave and every block.
  static constexpr int DW = WAVES / 2;
  static constexpr int K_INST = SD ? BN * K_HB / 1024 : BN * K_RP / 1024;
  static constexpr int R_INST = BN * R_RP / 1024;
  static constexpr int V_INST = BN * V_RB / 1024;
  static constexpr int K_DMA = (K_INST + DW - 1) / DW;
  static constexpr int R_DMA = (R_INST + DW - 1) / DW;
  static constexpr int KS_DMA = FP8 ? 1 : 0;
  static constexpr int V_DMA = V_INST / DW;
  static constexpr int N_OPS = K_DMA + R_DMA + KS_DMA + V_DMA;

  static_assert(K_RB == 128 || K_RB == 256, "K rows of 128 or 256 bytes");
  static_assert(DR == 0 || R_RB == 128, "rope rows of 128 bytes");
  static_assert(V_RB == 128 || V_RB == 256, "V rows of 128 or 256 bytes");
  static_assert(K_INST * 1024 == (SD ? BN * K_HB : BN * K_RP) && R_INST * 1024 == BN * R_RP &&
                    V_INST * 1024 == BN * V_RB,
                "regions are whole KiB");
  static_assert(V_DMA * DW == V_INST && V_DMA >= 1, "V DMA splits evenly over the waves");
  static_assert(N_OPS <= 15, "vmcnt immediates");
  static_assert(V_BASE % 256 == 0 && VSLOT % 256 == 0, "V rows keep 256-byte alignment");
  static_assert(!SD || (SSLOT % 256 == 0 && BN * (K_HB / 16) == WAVES * kWave),
                "SD: one 16-byte chunk of a staged block per thread");
  static_assert(WAVES * 32 * O_ROW <= LDS, "epilogue staging must fit in the rings");
  static_assert(LDS + 64 <= 160 * 1024, "LDS per workgroup");
};

// XOR swizzle of V rows (position of 16-byte chunk c of key row k =
// c ^ swz_v(k)).  ds_read_b64_tr_b16 touches 4 (per 16 lanes) or 8
// consecutive keys at 2 or 4 chunks each; the XOR keeps both the 16- and
// the 32-lane groups on distinct banks.
__device__ __forceinline__ int swz_v256(int k) {
  return (4 * (k & 3)) ^ (((k ^ (k >> 1)) & 1) << 1);
}
__device__ __forceinline__ int swz_v128(int k) { return 2 * (k & 3); }
template <int RB>
__device__ __forceinline__ int swz_v(int k) {
  return RB == 256 ? swz_v256(k) : swz_v128(k);
}

// Keep the compiler from moving anything across this point (step
// boundaries; inside a step the machine scheduler interleaves the
// independent softmax work with the matrix-core ops).
#define MHA_SLOT_FENCE() __builtin_amdgcn_sched_barrier(0)

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// s_waitcnt with only the vector-memory counter: vmcnt(N), N < 16.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

template <class C>
struct MfmaKernel {
  using QFrag = typename std::conditional<C::F8MMA, i32x8, bf16x8>::type;

  // ------------------------------------------------------------ staging

  // One 16-byte-per-lane DMA instruction: buffer_load_dwordx4 ... lds writes
  // lane i's 16 bytes at LDS address m0 + 16 i.  (m0 is set here; nothing
  // else in these kernels keeps a value in m0.)  Issued from inline assembly
  // so that the compiler does not treat it as a pending write to every LDS
  // address (it would otherwise wait for it before each LDS read of the
  // other slots); completion is awaited explicitly with vmcnt before the
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
  // Wait for this wave's DMA down to N outstanding instructions, then the
  // workgroup barrier (no fence: the compiler would add a vmcnt(0) wait).
  // SD: the block's decoded K rows are plain LDS writes, so the wait also
  // covers this wave's LDS operations (lgkmcnt(0)).
  template <int N>
  static __device__ __forceinline__ void publish() {
    if constexpr (C::SD) {
      static_assert(N >= 0 && N < 16, "vmcnt immediate");
      __builtin_amdgcn_s_waitcnt(0x0070 | N);
    } else {
      wait_vm<N>();
    }
    asm volatile("s_barrier" ::: "memory");
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

  // Per-lane source offset of DMA instruction n of a K region of BN rows of
  // RB bytes stored at pitch RB + 16: lane i fills 16-byte unit 64n + i of
  // the region, i.e. chunk (64n + i) % (RB/16 + 1) of row (64n + i) /
  // (RB/16 + 1); the pad unit gets an offset past every buffer (zeros).
  template <int RB>
  static __device__ __forceinline__ uint32_t dma_k_lane_off(int n, int lane, int row_stride) {
    constexpr int UPR = RB / 16 + 1;  // 16-byte units per padded row
    const int q = 64 * n + lane;
    const int row = q / UPR, chunk = q % UPR;
    return chunk == UPR - 1 ? 0x80000000u : (uint32_t)(row * row_stride + chunk * 16);
  }
  // SD staging order: 16-byte unit u of a staged block (u = 64 n + i for
  // lane i of DMA instruction n, and thread u of the decode) holds chunk
  // sd_chunk(u) of row sd_row(u): each group of 8 units is one chunk of 8
  // consecutive rows, and units 8 apart take chunks 4 apart.  The decode's
  // 16-byte writes to the padded K rows (pitch K_HB * 2 + 16) then fall on
  // distinct banks within every 8 and every 16 lanes, and its reads are
  // consecutive.
  static __device__ __forceinline__ int sd_row(int u) { return 8 * (u >> 6) + (u & 7); }
  static __device__ __forceinline__ int sd_chunk(int u) {
    const int j = (u >> 3) & 7;
    return (j >> 1) | ((j & 1) << 2);
  }
  // Per-lane source offset of DMA instruction n of an unpadded K staging
  // region (SD): lane i fills unit 64n + i (see sd_row, sd_chunk).
  static __device__ __forceinline__ uint32_t dma_s_lane_off(int n, int lane, int row_stride) {
    static_assert(!C::SD || C::K_HB == 128, "SD staging: 8 chunks of 16 bytes per row");
    const int u = 64 * n + lane;
    return (uint32_t)(sd_row(u) * row_stride + sd_chunk(u) * 16);
  }
  // Per-lane source offset of DMA instruction n of an unpadded, swizzled V
  // region: instruction n covers rows RPI*n .. RPI*n+RPI-1; lane i fills
  // position i % CPR of row RPI*n + i / CPR with the chunk that the swizzle
  // puts there.
  template <int RB>
  static __device__ __forceinline__ uint32_t dma_v_lane_off(int n, int lane, int row_stride) {
    constexpr int CPR = RB / 16, RPI = 1024 / RB;
    const int row = RPI * n + lane / CPR;
    const int chunk = (lane % CPR) ^ swz_v<RB>(row);
    return (uint32_t)(row * row_stride + chunk * 16);
  }

  // This wave's DMA source offsets (fixed for the kernel: they depend on the
  // head stride only).  An instruction index past a region's end gets rows
  // past every block (all lanes out of range, zeros); another wave's k_scale
  // instruction gets lanes out of range too.  NOJUNK: both repeat an
  // existing instruction instead (the rope region's last one, wave 0's
  // k_scale).
  struct DmaLanes {
    uint32_t k[C::K_DMA];
    uint32_t r[C::R_DMA > 0 ? C::R_DMA : 1];
    uint32_t v[C::V_DMA];
    uint32_t ks;
  };
  static __device__ __forceinline__ DmaLanes dma_lanes(const AttnParams& p, int wave, int lane) {
    DmaLanes d;
    const int Hkv = p.num_kv_heads;
#pragma unroll
    for (int i = 0; i < C::K_DMA; ++i)
      d.k[i] = C::SD ? dma_s_lane_off(wave + C::DW * i, lane, Hkv * C::K_HB)
                     : dma_k_lane_off<C::K_HB>(wave + C::DW * i, lane, Hkv * C::K_HB);
    if constexpr (C::R_DMA > 0) {
#pragma unroll
      for (int i = 0; i < C::R_DMA; ++i) {
        const int n = wave + C::DW * i;
        d.r[i] = dma_k_lane_off<C::R_RB>(C::NOJUNK && n >= C::R_INST ? C::R_INST - 1 : n, lane,
                                         Hkv * C::R_RB);
      }
    }
#pragma unroll
    for (int i = 0; i < C::V_DMA; ++i)
      d.v[i] = dma_v_lane_off<C::V_RB>(wave + C::DW * i, lane, Hkv * C::V_RB);
    d.ks = wave == 0 || C::NOJUNK ? (uint32_t)(lane * Hkv * 4) : 0x80000000u;
    return d;
  }

  // Per-item DMA sources: this (sequence, KV head)'s first row of each
  // tensor, the bytes one block advances, and the range of a full and of the
  // last block (one row of a block every Hkv rows of [T, Hkv]).
  struct DmaSrc {
    const char* k;
    const char* r;
    const char* ks;
    const char* v;
    uint32_t rows_stride;        // [T, Hkv] rows per block: BN * Hkv
    uint32_t span_full, span_last;  // [T, Hkv] rows a full / the last block spans
    int nblocks;                 // blocks of the tile's visible keys
    int jlo, jhi;                // the blocks this item loads (its key split)
  };
  static __device__ __forceinline__ DmaSrc dma_src(const AttnParams& p, int s0, int L, int g,
                                                  int nblocks, int jlo, int jhi) {
    const uint32_t Hkv = (uint32_t)p.num_kv_heads;
    const size_t row0 = (size_t)s0 * Hkv + (uint32_t)g;
    DmaSrc d;
    d.k = static_cast<const char*>(p.k) + row0 * C::K_HB;
    d.r = static_cast<const char*>(p.k_rope) + row0 * C::R_RB;
    d.ks = reinterpret_cast<const char*>(p.k_scale + row0);
    d.v = static_cast<const char*>(p.v) + row0 * C::V_RB;
    d.rows_stride = C::BN * Hkv;
    d.span_full = (C::BN - 1) * Hkv + 1;
    d.span_last = (uint32_t)(min(L - (nblocks - 1) * C::BN, C::BN) - 1) * Hkv + 1;
    d.nblocks = nblocks;
    d.jlo = jlo;
    d.jhi = jhi;
    return d;
  }

  // One batch of the DMA pipeline: the K side of block kblk (its rope rows:
  // of block rblk) and the V of block vblk (different blocks).  A block that
  // does not exist gets empty ranges and still its own slot, which nobody
  // reads while it is written.
  struct BlockDma {
    i32x4 k, r, ks, v;         // buffer resources
    uint32_t kdst, rdst, vdst;  // this wave's 1 KiB run in the K (SD: staging) / rope's K / V slot
  };
  template <int RB>
  static __device__ __forceinline__ i32x4 block_rsrc(const char* base, const DmaSrc& d, int blk,
                                                    uint32_t span) {
    return rsrc_of(base + (size_t)((uint32_t)blk * d.rows_stride) * RB, span * RB);
  }
  // rows a block spans in [T, Hkv] (0: the block is outside the item's range)
  template <bool SPLIT>
  static __device__ __forceinline__ uint32_t block_span(const DmaSrc& d, int blk) {
    if constexpr (SPLIT)
      return blk >= d.jlo && blk < d.jhi ? (blk < d.nblocks - 1 ? d.span_full : d.span_last) : 0u;
    else  // the range is [0, nblocks)
      return blk >= 0 && blk < d.nblocks ? (blk < d.nblocks - 1 ? d.span_full : d.span_last) : 0u;
  }
  template <bool SPLIT>
  static __device__ __forceinline__ BlockDma block_dma(const DmaSrc& d, uint32_t sbase, int wave,
                                                      int kblk, int rblk, int vblk) {
    const uint32_t kspan = block_span<SPLIT>(d, kblk), vspan = block_span<SPLIT>(d, vblk);
    const int kb = kspan ? kblk : 0, vb = vspan ? vblk : 0;  // keep addresses in range
    BlockDma b;
    b.k = block_rsrc<C::K_HB>(d.k, d, kb, kspan);
    if constexpr (C::DR > 0) {
      const uint32_t rspan = C::SDR ? block_span<SPLIT>(d, rblk) : kspan;
      b.r = block_rsrc<C::R_RB>(d.r, d, rspan ? rblk : 0, rspan);
    }
    if constexpr (C::FP8) b.ks = block_rsrc<4>(d.ks, d, kb, kspan);
    b.v = block_rsrc<C::V_RB>(d.v, d, vb, vspan);
    b.kdst = (C::SD ? sbase + C::S_BASE + (uint32_t)(kblk % C::NSS) * C::SSLOT
                    : sbase + (uint32_t)(kblk % C::NKS) * C::KSLOT) +
             1024u * (uint32_t)wave;
    // (rblk >= -KLEAD: the first batches of an item name blocks before it)
    b.rdst = sbase + (uint32_t)((rblk + 4 * C::NKS) % C::NKS) * C::KSLOT + 1024u * (uint32_t)wave;
    b.vdst = sbase + C::V_BASE + (uint32_t)(vblk & (C::NVS - 1)) * C::VSLOT +
             1024u * (uint32_t)wave;
    return b;
  }
  // DMA op OP of this wave (K nope, K rope, fp8 k_scale, V, in that order).
  // An instruction index past its region's end (for this wave) and another
  // wave's k_scale instruction write their zeros into the JUNK sink
  // (NOJUNK: they repeat the region's last instruction and wave 0's k_scale
  // instruction, identical bytes to the same place).
  template <int OP>
  static __device__ __forceinline__ void dma_op(const BlockDma& b, const DmaLanes& d,
                                                uint32_t junk, int wave) {
    if constexpr (OP < C::K_DMA) {
      constexpr uint32_t OFF = C::K_OFF + 1024u * C::DW * OP;
      uint32_t m0 = b.kdst + OFF;
      if constexpr ((OP + 1) * C::DW > C::K_INST) {
        static_assert(!C::NOJUNK, "K regions of whole instructions per wave");
        m0 = wave + C::DW * OP < C::K_INST ? m0 : junk;
      }
      dma16(b.k, m0, d.k[OP]);
    } else if constexpr (OP < C::K_DMA + C::R_DMA) {
      constexpr int I = OP - C::K_DMA;
      constexpr uint32_t OFF = C::R_OFF + 1024u * C::DW * I;
      uint32_t m0 = b.rdst + OFF;
      if constexpr ((I + 1) * C::DW > C::R_INST) {
        const uint32_t last = b.rdst - 1024u * (uint32_t)wave + C::R_OFF + 1024u * (C::R_INST - 1);
        m0 = wave + C::DW * I < C::R_INST ? m0 : (C::NOJUNK ? last : junk);
      }
      dma16(b.r, m0, d.r[I]);
    } else if constexpr (OP < C::K_DMA + C::R_DMA + C::KS_DMA) {
      // wave 0's run starts at its slot's k_scale area
      const uint32_t ks0 = b.kdst - 1024u * (uint32_t)wave + (C::SD ? C::BN * C::K_HB : C::KS_OFF);
      dma4(b.ks, wave == 0 || C::NOJUNK ? ks0 : junk, d.ks);
    } else {
      constexpr int I = OP - C::K_DMA - C::R_DMA - C::KS_DMA;
      dma16(b.v, b.vdst + 1024u * C::DW * I, d.v[I]);
    }
  }
  template <int OP0, int OP1>
  static __device__ __forceinline__ void dma_ops(const BlockDma& b, const DmaLanes& d,
                                                 uint32_t junk, int wave) {
    static_for<OP0, OP1>([&](auto oc) { dma_op<decltype(oc)::value>(b, d, junk, wave); });
  }

  // ------------------------------------------------------------ operands

  // LDS byte addresses.  Operand addresses are a per-lane part (fixed for
  // the kernel) plus the slot of the step plus an immediate; the sum of the
  // first two is made opaque once per step, so that the compiler neither
  // hoists one address register per immediate out of the loop nor loses the
  // immediate offsets of the reads.
  typedef __attribute__((address_space(3))) char lchar;
  static __device__ __forceinline__ const lchar* lp(uint32_t a) {
    return reinterpret_cast<const lchar*>(static_cast<uintptr_t>(a));
  }
  static __device__ __forceinline__ uint32_t opaque(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
  }
  struct Lanes {
    uint32_t k;               // K nope operand: row lane32, this lane half's bytes
    uint32_t r;               // K rope operand
    uint32_t v[C::DV_TILES];  // V^T operand of dv tile t (see v_frag)
  };
  static __device__ __forceinline__ Lanes lanes_of(int lane) {
    const int lane32 = lane & 31, hf = lane >> 5;
    Lanes ln;
    ln.k = lane32 * C::K_RP + (C::F8MMA ? 32 : (C::FP8 && !C::SD) ? 8 : 16) * hf;
    ln.r = lane32 * C::R_RP + 16 * hf;
    const int grp = lane >> 4, s = lane & 15;
    const int k1 = 4 * (grp >> 1) + (s >> 2);  // key row of the first read (u = 0)
#pragma unroll
    for (int t = 0; t < C::DV_TILES; ++t) {
      const int dv = t * 32 + 16 * (grp & 1) + 4 * (s & 3);  // first of this lane's 4 columns
      const int c = dv >> 3, sub = (dv & 7) * 2;               // chunk and byte inside it
      ln.v[t] = k1 * C::V_RB + 16 * (c ^ swz_v<C::V_RB>(k1)) + sub;
    }
    return ln;
  }

  // A operand of S product s of a 32-key sub-tile, from the per-lane K
  // (nope) and rope addresses of the sub-tile: nope steps first, then rope
  // steps.  Row pitch is K_RP.
  // 8 E4M3 codes (depth order) -> 8 bfloat16 values, exactly
  static __device__ __forceinline__ bf16x8 dec8(i32x2 x) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.f, true);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  }
  static __device__ __forceinline__ QFrag s_frag(uint32_t kt, uint32_t rt, int s) {
    if constexpr (C::FP8 && !C::F8MMA && !C::SD) {
      // E4M3 rows at pitch K_RP: step s covers depth 16 s .. 16 s + 15, 8
      // bytes per lane half
      if (s < C::QK_STEPS) {
        const i32x2 x =
            *reinterpret_cast<const __attribute__((address_space(3))) i32x2*>(lp(kt) + 16 * s);
        return dec8(x);
      }
      return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
          lp(rt) + 32 * (s - C::QK_STEPS));
    } else if constexpr (C::F8MMA) {
      const i32x4 a0 = *reinterpret_cast<const __attribute__((address_space(3))) i32x4*>(
          lp(kt) + 64 * s);
      const i32x4 a1 = *reinterpret_cast<const __attribute__((address_space(3))) i32x4*>(
          lp(kt) + 64 * s + 16);
      return i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    } else {
      if (s < C::QK_STEPS)
        return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(lp(kt) +
                                                                                  32 * s);
      return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
          lp(rt) + 32 * (s - C::QK_STEPS));
    }
  }
  // A operand of rope step s of the mixed layout (bf16 rows at pitch R_RP)
  static __device__ __forceinline__ bf16x8 r_frag(uint32_t rt, int s) {
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(lp(rt) + 32 * s);
  }
  static __device__ __forceinline__ f32x16 r_mfma(const bf16x8& a, const bf16x8& b, f32x16 acc) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16 s_mfma(const QFrag& a, const QFrag& b, f32x16 acc) {
    if constexpr (C::F8MMA)
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
    else
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }

  // A operand of P V product b of a sub-tile, from the per-lane V addresses
  // of the sub-tile (one per dv tile): dv tile t = b % DV_TILES, keys 16u ..
  // 16u+15 with u = b / DV_TILES.  Slot (lane half h, element i) holds key
  // 16u + 8(i/4) + 4h + i%4 of column 32t + lane % 32, matching the P^T
  // B-operand slots.  Within each group of 16 lanes, ds_read_b64_tr_b16
  // gives lane i, element k, the element i % 4 of the 8 bytes addressed by
  // lane 4k + i/4; so lane s of the group addresses key (base + s/4) at
  // columns 4(s%4) .. 4(s%4)+3.  The swizzle depends on key % 4 only, so the
  // keys 16u and 16u + 8 are immediate offsets.
  static __device__ __forceinline__ bf16x8 v_frag(const uint32_t (&vh)[C::DV_TILES], int b) {
    const int t = b % C::DV_TILES, u = b / C::DV_TILES;
    const lchar* a1 = lp(vh[t]) + 16 * u * C::V_RB;
    const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a1));
    const i16x4 r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a1 + 8 * C::V_RB));
    const i16x8 r = {r1[0], r1[1], r1[2], r1[3], r2[0], r2[1], r2[2], r2[3]};
    return __builtin_bit_cast(bf16x8, r);
  }

  // SD: the staged fp8 rows of block blk, decoded to bfloat16 into its K
  // slot (rows at pitch K_RP, as the bf16 kernel stores them), and its
  // k_scale copied there.  One 16-byte unit (16 codes) per thread, in the
  // staging order of sd_row / sd_chunk.
  static __device__ __forceinline__ void decode_block(uint32_t sbase, int blk, int tid) {
    typedef __attribute__((address_space(3))) i32x4 li32x4;
    typedef __attribute__((address_space(3))) bf16x8 lbf16x8;
    const uint32_t src = sbase + C::S_BASE + (uint32_t)(blk % C::NSS) * C::SSLOT;
    const uint32_t dst = sbase + (uint32_t)(blk % C::NKS) * C::KSLOT;
    const int row = sd_row(tid), ch = sd_chunk(tid);
    const i32x4 x = *reinterpret_cast<const li32x4*>(lp(src + tid * 16));
    lchar* d = const_cast<lchar*>(lp(dst + row * C::K_RP + ch * 32));
    *reinterpret_cast<lbf16x8*>(d) = dec8(i32x2{x[0], x[1]});
    *reinterpret_cast<lbf16x8*>(d + 16) = dec8(i32x2{x[2], x[3]});
    if (tid < C::BN / 4) {
      const i32x4 k4 =
          *reinterpret_cast<const li32x4*>(lp(src + C::BN * C::K_HB + 16 * tid));
      *reinterpret_cast<li32x4*>(const_cast<lchar*>(lp(dst + C::KS_OFF + 16 * tid))) = k4;
    }
  }

  // ------------------------------------------------------------ pieces

  // Per-wave state of one work item.
  struct State {
    f32x16 o[C::DV_TILES];  // O^T accumulator (lane = query, 16 dv rows per tile)
    f32x16 st;              // S^T of the sub-tile awaiting its softmax half-step
    f32x16 sr;              // its rope part (mixed layout only)
    uint32_t pw[8];         // P of the sub-tile awaiting its product half-step,
                            // packed bf16 pairs: pw[4u + i] = dword i of B operand u
    float m;                // running max (log2 domain), same in lanes i and i ^ 32
    float l;                // this lane's partial row sum
  };

  // Plain S of one sub-tile (the item's first).
  static __device__ __forceinline__ void s_tile(uint32_t kt, uint32_t rt, const QFrag* qf,
                                                const bf16x8* qr, State& w) {
#pragma unroll
    for (int r = 0; r < 16; ++r) w.st[r] = 0.f;
    if constexpr (C::MIXED) {
#pragma unroll
      for (int s = 0; s < C::QK_STEPS; ++s) w.st = s_mfma(s_frag(kt, rt, s), qf[s], w.st);
#pragma unroll
      for (int r = 0; r < 16; ++r) w.sr[r] = 0.f;
#pragma unroll
      for (int s = 0; s < C::ROPE_STEPS; ++s) w.sr = r_mfma(r_frag(rt, s), qr[s], w.sr);
    } else {
      (void)qr;
#pragma unroll
      for (int s = 0; s < C::S_STEPS; ++s) w.st = s_mfma(s_frag(kt, rt, s), qf[s], w.st);
    }
  }

  // Exponentials of a sub-tile's scores against the running max m (S in
  // w.st, left unchanged): P = 2^(cq S - m) packed as bf16 pairs into w.pw;
  // returns this lane's float32 sum of the unrounded P.
  static __device__ __forceinline__ float exp_pack(State& w, float cq, float m) {
    float ls[2];
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float p0 = fast_exp2(fmaf(w.st[e], cq, -m));
      const float p1 = fast_exp2(fmaf(w.st[e + 1], cq, -m));
      ls[0] = e == 0 ? p0 : ls[0] + p0;  // no add of the zero start
      ls[1] = e == 0 ? p1 : ls[1] + p1;
      w.pw[e >> 1] = pack_bf16x2(p0, p1);
    }
    // (two sum chains, and computed even when the caller will redo them:
    // no branch around the common path)
    asm volatile("" : "+v"(ls[0]), "+v"(ls[1]), "+v"(w.pw[0]), "+v"(w.pw[1]), "+v"(w.pw[2]),
                 "+v"(w.pw[3]), "+v"(w.pw[4]), "+v"(w.pw[5]), "+v"(w.pw[6]), "+v"(w.pw[7]));
    return ls[0] + ls[1];
  }

  // Softmax half-step of a sub-tile whose S is in w.st: fp8 k_scale, the mask
  // when it is the wave's last sub-tile (keys past `rel` in lane-relative
  // numbering hidden), exponentials, row sums and the bf16 packing of P into
  // w.pw.  Element e of a lane is key 8(e/4) + 4 hf + e%4 of the sub-tile.
  //
  // The running max is lazy (the per-row correction buffer of
  // SM100AttentionSMem, Methods: correction_smem, applied rarely): P is
  // computed against the current m first, and only when a lane's sum of P
  // exceeds 2^kLazy (so some P may exceed 2^(kLazy - 4), or be infinite),
  // or at the item's first sub-tile (`first`, no max yet), is the row max
  // taken, O and l corrected and P recomputed.  Otherwise
  // every P <= 2^kLazy: bf16 P, the float32 row sums and O keep their
  // relative precision at any such scale, and O / l and LSE = (m + log2 l)
  // ln 2 do not depend on which m they share.  This spends no vector work on
  // row maxima in the common case.
  template <int OP0, int OP1, bool MAYMASK>
  static __device__ __forceinline__ void xphase(State& w, bool first, const float* ks, int hf,
                                                float cq_in, float crope, bool mask, int rel,
                                                const BlockDma& bd, const DmaLanes& dl,
                                                uint32_t junk, int wave) {
    MHA_SLOT_FENCE();
    // this half-step's share of the block's DMA ops
    dma_ops<OP0, OP1>(bd, dl, junk, wave);
    // mixed layout: the score goes straight to the log2 domain here
    // (q_scale k_scale S_nope and S_rope at their own multipliers); the
    // rest of the half-step then runs with multiplier 1
    const float cq = C::MIXED ? 1.f : cq_in;
    (void)crope;
    if constexpr (C::MIXED || C::FP8) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if constexpr (C::MIXED)
          w.st[e] = fmaf(w.st[e] * ks[8 * (e >> 2) + 4 * hf + (e & 3)], cq_in, w.sr[e] * crope);
        else
          w.st[e] *= ks[8 * (e >> 2) + 4 * hf + (e & 3)];
      }
    }
    if (MAYMASK && mask) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (8 * (e >> 2) + (e & 3) > rel) w.st[e] = -INFINITY;
    }
    constexpr float kLazyMax = 4294967296.f;  // 2^kLazy, kLazy = 32 (log2 units)
    float ls = exp_pack(w, cq, w.m);
    // (checked half-steps: also any row still without a visible key, whose
    // m = -inf gives no usable P)
    // (bitwise or: every term is evaluated, no branch around the check)
    const bool big = (int)wave_any(ls > kLazyMax) | (int)first |
                     (int)(MAYMASK && wave_any(w.m == -INFINITY));
    if (big) {
      float x = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) x = fmaxf(x, w.st[e]);
      const float mx = half_max(x) * cq;
      const float m_new = fmaxf(w.m, mx);
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(w.m - m_new);
      w.l *= alpha;
#pragma unroll
      for (int t = 0; t < C::DV_TILES; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) w.o[t][r] *= alpha;
      w.m = m_new;
      // rows with no visible key yet keep m = -inf, P = 0
      ls = exp_pack(w, cq, m_new == -INFINITY ? 0.f : m_new);
    }
    w.l += ls;
    MHA_SLOT_FENCE();
  }

  // Matrix-core half-step: P V of sub-tile i (P in w.pw, V rows in half VH
  // of the V block at vb) and S of sub-tile i+1 (K rows in half KH of the K
  // block at kb / rb, the first KPF of its fragments already in kpre) into
  // w.st; the S of a sub-tile past the wave's last is computed from
  // whatever the slot holds and never used.
  template <int KH, int VH>
  static __device__ __forceinline__ void gphase(State& w, uint32_t kb, uint32_t rb,
                                                const uint32_t (&vb)[C::DV_TILES],
                                                const QFrag* qf, const bf16x8* qr,
                                                const QFrag* kpre) {
    // K rows of half KH of the K block, V rows of half VH of the V block
    const uint32_t kn = kb + KH * 32 * C::K_RP, rn = rb + KH * 32 * C::R_RP;
    uint32_t vh[C::DV_TILES];
#pragma unroll
    for (int t = 0; t < C::DV_TILES; ++t) vh[t] = vb[t] + VH * 32 * C::V_RB;
    constexpr int NS = C::S_STEPS + C::NPV;  // matrix-core slots
    MHA_SLOT_FENCE();
    bf16x8 pb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
      pb[u] = __builtin_bit_cast(bf16x8, i32x4{(int)w.pw[4 * u], (int)w.pw[4 * u + 1],
                                               (int)w.pw[4 * u + 2], (int)w.pw[4 * u + 3]});
    f32x16 sn, srn;
#pragma unroll
    for (int r = 0; r < 16; ++r) sn[r] = 0.f;
    if constexpr (C::MIXED) {
#pragma unroll
      for (int r = 0; r < 16; ++r) srn[r] = 0.f;
    }
    // products alternate between the P V and the S streams while both last
    static_for<0, NS>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      constexpr int NPAIR = C::NPV < C::S_STEPS ? C::NPV : C::S_STEPS;
      constexpr bool PV = k < 2 * NPAIR ? (k % 2 == 0) : (C::NPV > C::S_STEPS);
      constexpr int idx = k < 2 * NPAIR ? k / 2 : k - NPAIR;
      if constexpr (PV) {
        w.o[idx % C::DV_TILES] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            v_frag(vh, idx), pb[idx / C::DV_TILES], w.o[idx % C::DV_TILES], 0, 0, 0);
      } else if constexpr (C::MIXED && idx >= C::QK_STEPS) {
        srn = r_mfma(r_frag(rn, idx - C::QK_STEPS), qr[idx - C::QK_STEPS], srn);
      } else {
        if constexpr (idx < C::KPF)
          sn = s_mfma(kpre[idx], qf[idx], sn);
        else
          sn = s_mfma(s_frag(kn, rn, idx), qf[idx], sn);
      }
    });
    // Slot shape for the machine scheduler: each product's operands are
    // read G_AHEAD products ahead (not all at the start, which would hold 16
    // operand fragments in registers at once).
    constexpr int RA = C::G_AHEAD;
    static_for<0, NS + RA>([&](auto kc) {
      constexpr int k = decltype(kc)::value;  // reads for product k, then product k - RA
      constexpr int NPAIR = C::NPV < C::S_STEPS ? C::NPV : C::S_STEPS;
      if constexpr (k < NS) {
        constexpr bool PV = k < 2 * NPAIR ? (k % 2 == 0) : (C::NPV > C::S_STEPS);
        constexpr int idx = k < 2 * NPAIR ? k / 2 : k - NPAIR;
        if constexpr (PV || idx >= C::KPF)
          __builtin_amdgcn_sched_group_barrier(
              0x100, PV ? 2 : (C::F8MMA && idx < C::QK_STEPS ? 2 : 1), 0);
      }
      if constexpr (k >= RA) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    });
    w.st = sn;
    if constexpr (C::MIXED) w.sr = srn;
    MHA_SLOT_FENCE();
  }

  // ------------------------------------------------------------ kernel body

  // SPLIT: split-KV work items (a key range of the tile, partial results
  // to o_part / lse_part); without it the range is the whole tile and the
  // split arithmetic folds away.
  template <bool SPLIT>
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
    const DmaLanes dl = dma_lanes(p, wave, lane);
    const Lanes ln = lanes_of(lane);
    const uint32_t sbase = lds_addr_of(smem);
    const uint32_t junk = sbase + C::JUNK;

    // wave FW runs the work-item source.  It belongs to group 1, which
    // issues no DMA, so its vector-memory counter holds only its own loads.
    // The next item is reserved three blocks before the current item's end
    // and its table entry read one block before it: the choice is made
    // late (list scheduling over the queue order, so the CUs finish close
    // together) and neither round trip sits between two items.
    constexpr int FW = C::WAVES / 2;
    Fetcher fetch;
    if (wave == FW) {
      fetch.init(p.sched);
      const i32x4 e0 = fetch.resolve(p.sched, p.table);
      if (lane == 0) s_item[0] = e0;
    }
    // Q fragments (B operand): lane -> query qi, 8 (bf16) or 32 (fp8)
    // consecutive depth elements per step and lane half; rope steps follow
    // the nope steps.  cq: the multiplier of S in the exponent (log2
    // domain), kept >= FLT_MIN so that a masked -inf score stays -inf (a
    // zero q_scale row then gives the uniform distribution over its visible
    // keys, as 0 * S does).
    constexpr int NQF = C::MIXED ? C::QK_STEPS : C::S_STEPS;
    constexpr int NQR = C::MIXED ? C::ROPE_STEPS : 1;  // mixed layout: the rope steps
    auto load_q = [&](const WorkItem& wi, QFrag* qf, bf16x8* qr, float& cq) {
      const int qi = wi.qt * C::BM + wave * 32 + lane32;
      const bool qvalid = qi < wi.L;
      const size_t qrow = (size_t)(wi.s0 + qi) * p.num_heads + wi.h;
#pragma unroll
      for (int s = 0; s < C::S_STEPS; ++s) {
        if constexpr (C::MIXED) {
          if (s >= C::QK_STEPS) {
            i32x4 x = {0, 0, 0, 0};
            if (qvalid)
              x = *reinterpret_cast<const i32x4*>(
                  qrp + (qrow * C::DR + (s - C::QK_STEPS) * 16 + 8 * hf) * 2);
            qr[s - C::QK_STEPS] = __builtin_bit_cast(bf16x8, x);
            continue;
          }
        }
        if constexpr (C::FP8 && !C::F8MMA) {
          i32x2 x = {0, 0};
          if (qvalid) x = *reinterpret_cast<const i32x2*>(qp + qrow * C::DN + s * 16 + 8 * hf);
          qf[s] = dec8(x);
        } else if constexpr (C::FP8) {
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
      cq = p.scale_log2;
      if (C::FP8 && qvalid) cq *= p.q_scale[qrow];
      if (!(cq >= 1.17549435e-38f)) cq = 1.17549435e-38f;
    };
    // Without a rope part, the next item's Q loads are issued as soon as
    // the next item is known (after the current item's last products),
    // ahead of the current item's output stores, so that their latency
    // overlaps the epilogue.  (With a rope part the longer live range
    // costs more than it saves.)
    constexpr bool EARLY_Q = C::DR == 0;
    // (the fragments live across items only when they are loaded early)
    QFrag qf_x[EARLY_Q ? NQF : 1];
    bf16x8 qr_x[EARLY_Q ? NQR : 1];
    float cq_x = 0.f;
    // bf16: the early Q loads read whole rows (RPI rows of QRB bytes per
    // instruction, a few cache lines each, instead of one 16-byte piece of
    // each of 32 rows) into the fragment registers themselves, and the rows
    // are rearranged into the
    // fragment layout through this wave's 32 QRB-byte part of the V ring,
    // which is idle between two items (chunk c of row r at chunk position
    // c ^ (r % QCPR), so that neither the writes nor the fragment reads
    // meet on a bank)
    constexpr bool QROWS = EARLY_Q && !C::FP8;
    constexpr int QRB = C::DN * 2, QCPR = QRB / 16, QRPI = kWave / QCPR;
    static_assert(!QROWS || (32 / QRPI == C::QK_STEPS && 8 * 32 * QRB <= C::NVS * C::VSLOT),
                  "a wave's Q rows fit its part of the V ring, one instruction per step");
    const uint32_t qarea = sbase + C::V_BASE + (uint32_t)wave * (32 * QRB);
    // (the per-lane offsets are recomputed at each call, from a lane index
    // the compiler cannot see through, rather than kept in registers across
    // the block loop)
    auto load_q_rows = [&](const WorkItem& nw) {
      const int r0 = nw.qt * C::BM + wave * 32;
      const int ql = (int)opaque((uint32_t)lane);
#pragma unroll
      for (int i = 0; i < C::QK_STEPS; ++i) {
        const int r = QRPI * i + ql / QCPR, c = ql % QCPR;
        i32x4 x = {0, 0, 0, 0};
        if (r0 + r < nw.L)
          // (read once per item: a streaming load, as for the output)
          x = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(
              qp + (((size_t)(nw.s0 + r0 + r) * p.num_heads + nw.h) * C::DN) * 2 + c * 16));
        if constexpr (QROWS) qf_x[i] = __builtin_bit_cast(bf16x8, x);
      }
      cq_x = p.scale_log2;
      if (!(cq_x >= 1.17549435e-38f)) cq_x = 1.17549435e-38f;
    };
    auto place_q_rows = [&]() {
      typedef __attribute__((address_space(3))) i32x4 li32x4;
      const int ql = (int)opaque((uint32_t)lane);
      const int ql32 = ql & 31, qhf = ql >> 5;
      const uint32_t qa = opaque(qarea);
#pragma unroll
      for (int i = 0; i < C::QK_STEPS; ++i) {
        const int r = QRPI * i + ql / QCPR, c = ql % QCPR;
        if constexpr (QROWS)
          *reinterpret_cast<li32x4*>(const_cast<lchar*>(
              lp(qa + r * QRB + 16 * (c ^ (r % QCPR))))) = __builtin_bit_cast(i32x4, qf_x[i]);
      }
      if constexpr (QROWS) {
#pragma unroll
        for (int s = 0; s < C::QK_STEPS; ++s)
          qf_x[s] = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const li32x4*>(
                          lp(qa + ql32 * QRB + 16 * ((2 * s + qhf) ^ (ql32 % QCPR)))));
      }
    };
    for (int it = 0;; ++it) {
      __syncthreads();
      // the item is the same for the whole workgroup: keep it in SGPRs
      const WorkItem wi = decode_item(i32x4{__builtin_amdgcn_readfirstlane(s_item[it & 1][0]),
                                            __builtin_amdgcn_readfirstlane(s_item[it & 1][1]),
                                            __builtin_amdgcn_readfirstlane(s_item[it & 1][2]),
                                            __builtin_amdgcn_readfirstlane(s_item[it & 1][3])});
      if (wi.L < 0) break;
      const int s0 = wi.s0;
      const int L = wi.L;
      const int g = wi.h / p.group;
      const int q0 = wi.qt * C::BM;    // first query row of the tile
      const int wq0 = q0 + wave * 32;  // first query row of this wave
      // (fast fp8 with a rope part: the lane-derived values of an item come
      // from a lane index the compiler cannot see through, so that they are
      // recomputed per item instead of kept, and spilled, across the loop)
      constexpr bool OPQ = C::MIXED && C::F8MMA;
      const int ol = OPQ ? (int)opaque((uint32_t)lane) : 0;
      const int qi = wq0 + (OPQ ? (ol & 31) : lane32);  // this lane's query row
      const bool qvalid = qi < L;
      const size_t qrow = (size_t)(s0 + qi) * p.num_heads + wi.h;

      const int n_kv = p.causal ? min(L, q0 + C::BM) : L;
      const int nblocks = (n_kv + C::BN - 1) / C::BN;
      // this item's key blocks: split wi.split of num_splits (all of them
      // without split-KV)
      const int per = SPLIT ? (nblocks + p.num_splits - 1) / p.num_splits : nblocks;
      const int jlo = SPLIT ? min(nblocks, wi.split * per) : 0;
      const int jhi = SPLIT ? min(nblocks, jlo + per) : nblocks;
      // 32-key sub-tiles this wave computes (causal: keys up to wq0 + 31
      // only; none when all its rows are past the end); only the last can
      // need the mask
      const int n_sub_all = wq0 >= L ? 0
                            : p.causal ? min((L + 31) >> 5, (wq0 >> 5) + 1)
                                       : (L + 31) >> 5;
      const int last_sub = n_sub_all - 1;                // the one that takes the mask
      const int n_sub = SPLIT ? min(n_sub_all, 2 * jhi) : n_sub_all;  // sub-tiles 2 jlo .. n_sub - 1 here
      const bool has_sub = n_sub > 2 * jlo;
      const int j_res = max(jlo, jhi - 3), j_get = max(jlo, jhi - 1);
      i32x4 nxt = {0, -1, 0, 0};
      const int lim = p.causal ? min(L - 1, qi) : L - 1;  // last key visible to this lane

      // Q fragments (B operand): lane -> query qi, 8 (bf16) or 32 (fp8)
      // consecutive depth elements per step and lane half; rope steps follow
      // the nope steps.  cq: see load_q.
      QFrag qf_i[EARLY_Q ? 1 : NQF];
      bf16x8 qr_i[EARLY_Q ? 1 : NQR];
      QFrag* qf = EARLY_Q ? qf_x : qf_i;
      bf16x8* qr = EARLY_Q ? qr_x : qr_i;
      if (EARLY_Q && it == 0) load_q(wi, qf_x, qr_x, cq_x);
      if constexpr (!EARLY_Q) {
#pragma unroll
        for (int s = 0; s < C::S_STEPS; ++s) {
          if constexpr (C::MIXED) {
            if (s >= C::QK_STEPS) {
              i32x4 x = {0, 0, 0, 0};
              if (qvalid)
                x = *reinterpret_cast<const i32x4*>(
                    qrp + (qrow * C::DR + (s - C::QK_STEPS) * 16 + 8 * (OPQ ? (ol >> 5) : hf)) * 2);
              qr_i[s - C::QK_STEPS] = __builtin_bit_cast(bf16x8, x);
              continue;
            }
          }
          if constexpr (C::FP8 && !C::F8MMA) {
            i32x2 x = {0, 0};
            if (qvalid) x = *reinterpret_cast<const i32x2*>(qp + qrow * C::DN + s * 16 + 8 * (OPQ ? (ol >> 5) : hf));
            qf_i[s] = dec8(x);
          } else if constexpr (C::FP8) {
            i32x8 x = {0, 0, 0, 0, 0, 0, 0, 0};
            if (qvalid) {
              const i32x4* src =
                  reinterpret_cast<const i32x4*>(qp + qrow * C::DN + s * 64 + 32 * (OPQ ? (ol >> 5) : hf));
              const i32x4 a0 = src[0], a1 = src[1];
              x = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            }
            qf_i[s] = x;
          } else {
            i32x4 x = {0, 0, 0, 0};
            if (qvalid) {
              const char* src = s < C::QK_STEPS
                                    ? qp + (qrow * C::DN + s * 16 + 8 * (OPQ ? (ol >> 5) : hf)) * 2
                                    : qrp + (qrow * C::DR + (s - C::QK_STEPS) * 16 + 8 * (OPQ ? (ol >> 5) : hf)) * 2;
              x = *reinterpret_cast<const i32x4*>(src);
            }
            qf_i[s] = __builtin_bit_cast(bf16x8, x);
          }
        }
      }
      float cq = cq_x;
      if constexpr (!EARLY_Q) {
        cq = p.scale_log2;
        if (C::FP8 && qvalid) cq *= p.q_scale[qrow];
        if (!(cq >= 1.17549435e-38f)) cq = 1.17549435e-38f;
      }

      State w;
#pragma unroll
      for (int t = 0; t < C::DV_TILES; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) w.o[t][r] = 0.f;
      w.m = -INFINITY;
      w.l = 0.f;

      // The DMA pipeline: batch t is {K_{t+KLEAD} (SDR: its rope rows
      // K_{t+RLEAD}), V_{t+2}}, and block j issues batch j.  The prologue
      // issues the batches before block 0: those needed in block 0 are
      // waited for here together with the Q loads (the compiler's own wait
      // for those could not tell the DMA apart anyway); with 4 K slots the
      // last one goes out after the first S.  SDR: the staged rows of block
      // jlo + 2 go to the staging slot of block jlo, so they are requested
      // after that block's decode, and waited for before block jlo.
      const int grp = wave >> 2;  // group 0 issues the DMA
      const DmaSrc dsrc = dma_src(p, s0, L, g, nblocks, jlo, jhi);
      auto blk = [&](int t) {
        return block_dma<SPLIT>(dsrc, sbase, wave, t + C::KLEAD, t + C::RLEAD, t + 2);
      };
      constexpr int OP_R = C::K_DMA, OP_KS = OP_R + C::R_DMA, OP_V = OP_KS + C::KS_DMA;
      if (grp == 0) {
        for (int t = jlo - C::KLEAD; t < jlo + (C::KLEAD >= 3 ? -1 : 0); ++t)
          dma_ops<0, C::N_OPS>(blk(t), dl, junk, wave);
        if constexpr (C::SDR) {
          const BlockDma b = blk(jlo - 1);
          dma_ops<OP_R, OP_KS>(b, dl, junk, wave);
          dma_ops<OP_V, C::N_OPS>(b, dl, junk, wave);
        }
      }
      wait_vm<0>();
      __syncthreads();
      if constexpr (C::SD) {
        // the first two blocks are decoded here, the third in block jlo
        decode_block(sbase, jlo, tid);
        decode_block(sbase, jlo + 1, tid);
        __syncthreads();
      }
      if constexpr (C::SDR)
        if (grp == 0) {
          const BlockDma b = blk(jlo - 1);
          dma_ops<0, OP_R>(b, dl, junk, wave);
          dma_ops<OP_KS, OP_V>(b, dl, junk, wave);
        }
      if (has_sub) {
        const uint32_t ks0 = sbase + (uint32_t)(jlo % C::NKS) * C::KSLOT;
        s_tile(opaque(ks0 + C::K_OFF + ln.k), opaque(ks0 + C::R_OFF + ln.r), qf, qr, w);
      }
      if constexpr (C::SDR) {
        wait_vm<0>();
        __syncthreads();
      } else if constexpr (C::KLEAD >= 3) {
        if (grp == 0) dma_ops<0, C::N_OPS>(blk(jlo - 1), dl, junk, wave);
      }

      // Per wave the sub-tiles run as alternating half-steps X_0 G_0 X_1
      // G_1 ...: X_i is sub-tile i's softmax (vector ALU), G_i its P V and
      // the next sub-tile's S (matrix cores).  Waves w and w + 4 share a
      // SIMD.  Every wave runs X_{2j} G_{2j} X_{2j+1} G_{2j+1} per block, but
      // group 1 (waves 4-7) takes the block's barrier before G_{2j+1} and
      // group 0 after it: between two barriers group 0 runs X G X G and
      // group 1 G X G X, so on every SIMD one wave's softmax overlaps the
      // other's products (the ping-pong of the pages' two softmax warp
      // groups).  Group 1 reads V_j after barrier j, hence 4 V slots.  At
      // each barrier j, K_{j+2} and V_{j+1} must have landed.
      constexpr int OPH = C::N_OPS / 2;  // DMA ops issued in the block's first softmax half-step
      // softmax half-step of sub-tile i = 2j + H (k_scale from K block j);
      // group 0 also issues its share of the block's DMA.  CHK: the sub-tile
      // may be missing or be the wave's last (masked).
      QFrag kpre[C::KPF > 0 ? C::KPF : 1];
      auto xh = [&](auto grpc, auto chk, auto part, int i, int j, const BlockDma& bd) {
        constexpr int H = decltype(part)::value;
        if constexpr (C::KPF > 0) {
          // the next product half-step's first S operands: half 1 of K block
          // j after X_{2j}, half 0 of block j + 1 after X_{2j+1}
          const int jk = H == 0 ? j : j + 1;
          const uint32_t kn = opaque(sbase + (uint32_t)(jk % C::NKS) * C::KSLOT + C::K_OFF + ln.k) +
                              (H == 0 ? 32 * C::K_RP : 0);
#pragma unroll
          for (int s = 0; s < C::KPF; ++s) kpre[s] = s_frag(kn, 0u, s);
        }
        constexpr bool DMA = decltype(grpc)::value == 0;
        constexpr int O0 = !DMA ? 0 : H == 0 ? 0 : OPH;
        constexpr int O1 = !DMA ? 0 : H == 0 ? OPH : C::N_OPS;
        constexpr bool CHK = decltype(chk)::value;
        const float* ks =
            reinterpret_cast<const float*>(smem + (j % C::NKS) * C::KSLOT + C::KS_OFF) + 32 * H;
        if (!CHK || i < n_sub)
          xphase<O0, O1, CHK>(w, i == 2 * jlo, ks, OPQ ? (ol >> 5) : hf, cq, p.scale_log2,
                              SPLIT ? i == last_sub : i == n_sub - 1,
                              lim - 32 * i - 4 * (OPQ ? (ol >> 5) : hf), bd,
                              dl, junk, wave);
        else
          dma_ops<O0, O1>(bd, dl, junk, wave);
      };
      // product half-step of sub-tile i: V of block j (half VH), K of block
      // jk (half KH)
      auto gh = [&](auto chk, auto kh, auto vh_, int i, int j, int jk) {
        if (!decltype(chk)::value || i < n_sub) {
          const uint32_t ks = sbase + (uint32_t)(jk % C::NKS) * C::KSLOT;
          const uint32_t vs = sbase + C::V_BASE + (uint32_t)(j & (C::NVS - 1)) * C::VSLOT;
          uint32_t vb[C::DV_TILES];
#pragma unroll
          for (int t = 0; t < C::DV_TILES; ++t) vb[t] = opaque(vs + ln.v[t]);
          gphase<decltype(kh)::value, decltype(vh_)::value>(
              w, opaque(ks + C::K_OFF + ln.k), C::DR > 0 ? opaque(ks + C::R_OFF + ln.r) : 0u, vb,
              qf, qr, kpre);
        }
      };
      using P0 = std::integral_constant<int, 0>;
      using P1 = std::integral_constant<int, 1>;
      using Y = std::true_type;
      using N = std::false_type;
      auto publish_block = [&]() {
        if constexpr (C::K_SLACK)
          publish<C::N_OPS>();  // batch j may stay in flight
        else
          publish<C::V_DMA>();  // batch j's K part must be in too
      };
      // One block of a group: X_{2j} G_{2j} X_{2j+1} G_{2j+1}, the barrier
      // after it (group 0) or before its last product half-step (group 1).
      auto block = [&](auto grpc, auto chk, int j) {
        constexpr int GRP = decltype(grpc)::value;
        BlockDma bd;
        if constexpr (GRP == 0) bd = blk(j);
        // SD: block j + 2 (staged by batch j - 2, published at barrier j - 1)
        // is decoded into the slot that block j - 1 freed; barrier j
        // publishes it before block j + 1 first reads it
        if constexpr (C::SD) decode_block(sbase, j + 2, tid);
        xh(grpc, chk, P0{}, 2 * j, j, bd);
        gh(chk, P1{}, P0{}, 2 * j, j, j);
        xh(grpc, chk, P1{}, 2 * j + 1, j, bd);
        if constexpr (GRP == 1) publish_block();
        gh(chk, P0{}, P1{}, 2 * j + 1, j, j + 1);
        if constexpr (GRP == 0) publish_block();
      };
      // blocks whose four half-steps all exist and need no mask, then the rest
      const int j_steady = max(jlo, min(jhi, last_sub > 0 ? last_sub / 2 : 0));
      if (grp == 0) {
        int j = jlo;
        for (; j < j_steady; ++j) block(P0{}, N{}, j);
        for (; j < jhi; ++j) block(P0{}, Y{}, j);
      } else {
        auto fetch_at = [&](int j) {
          if (wave == FW) {
            if (j == j_res) fetch.reserve(p.sched);
            if (j == j_get) nxt = fetch.resolve(p.sched, p.table);
          }
        };
        int j = jlo;
        for (; j < j_steady; ++j) {
          fetch_at(j);
          block(P1{}, N{}, j);
        }
        for (; j < jhi; ++j) {
          fetch_at(j);
          block(P1{}, Y{}, j);
        }
        if (wave == FW) {
          if (jhi <= jlo) {  // no blocks in this item (an empty key range)
            fetch.reserve(p.sched);
            nxt = fetch.resolve(p.sched, p.table);
          }
          if (lane == 0) s_item[(it + 1) & 1] = nxt;
        }
      }
      // the last batches requested nothing; drain, and let group 1 finish
      // its last products, before the rings are reused for the output
      // staging
      wait_vm<0>();
      __syncthreads();
      if constexpr (EARLY_Q) {
        const WorkItem nw =
            decode_item(i32x4{__builtin_amdgcn_readfirstlane(s_item[(it + 1) & 1][0]),
                              __builtin_amdgcn_readfirstlane(s_item[(it + 1) & 1][1]),
                              __builtin_amdgcn_readfirstlane(s_item[(it + 1) & 1][2]),
                              __builtin_amdgcn_readfirstlane(s_item[(it + 1) & 1][3])});
        if (nw.L >= 0) {
          if constexpr (QROWS)
            load_q_rows(nw);
          else
            load_q(nw, qf_x, qr_x, cq_x);
        }
      }

      // ---- epilogue
      const float lt = half_sum(w.l);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      if constexpr (SPLIT) {
        // split-KV partial: O over this item's key range (zero where the
        // range holds no visible key), float32 or rounded to bfloat16, and
        // its LSE (-inf there), straight from the registers: each lane
        // writes runs of 4 values of its row
        const int sl = OPQ ? (int)opaque((uint32_t)lane) : 0;
        if ((OPQ ? wq0 + (sl & 31) < L : qvalid) &&
            s0 + (OPQ ? wq0 + (sl & 31) : qi) < p.part_tokens) {
          const size_t prow = ((size_t)wi.split * p.part_tokens + s0 +
                               (OPQ ? wq0 + (sl & 31) : qi)) * p.num_heads + wi.h;
          float* dst = p.o_part + prow * C::DV;
          uint16_t* dst16 = reinterpret_cast<uint16_t*>(p.o_part) + prow * C::DV;
#pragma unroll
          for (int t = 0; t < C::DV_TILES; ++t)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
              const f32x4 x = {w.o[t][4 * a4 + 0] * inv, w.o[t][4 * a4 + 1] * inv,
                               w.o[t][4 * a4 + 2] * inv, w.o[t][4 * a4 + 3] * inv};
              const int col = t * 32 + 8 * a4 + 4 * (OPQ ? sl >> 5 : hf);
              if (p.part_bf16)
                *reinterpret_cast<i32x2*>(dst16 + col) =
                    i32x2{(int)pack_bf16x2(x[0], x[1]), (int)pack_bf16x2(x[2], x[3])};
              else
                *reinterpret_cast<f32x4*>(dst + col) = x;
            }
          if ((OPQ ? sl >> 5 : hf) == 0)
            p.lse_part[((size_t)wi.split * p.num_heads + wi.h) * p.part_tokens + s0 +
                       (OPQ ? wq0 + (sl & 31) : qi)] =
                lt > 0.f ? (w.m + log2f(lt)) * kLn2 : -INFINITY;
        }
        if constexpr (QROWS) place_q_rows();
        continue;
      }
      // SDR: the staging addresses are recomputed per item, from a lane index
      // the compiler cannot see through, instead of hoisted out of the item
      // loop as constants that would not fit in the registers beside the
      // loop's state
      const int el = C::SDR || OPQ ? (int)opaque((uint32_t)lane) : lane;
      const int el32 = el & 31, ehf = el >> 5;
      char* ost = smem + wave * 32 * C::O_ROW + el32 * C::O_ROW;
#pragma unroll
      for (int t = 0; t < C::DV_TILES; ++t)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int dv0 = t * 32 + 8 * a4 + 4 * ehf;
          const uint32_t lo = pack_bf16x2(w.o[t][4 * a4 + 0] * inv, w.o[t][4 * a4 + 1] * inv);
          const uint32_t hi = pack_bf16x2(w.o[t][4 * a4 + 2] * inv, w.o[t][4 * a4 + 3] * inv);
          *reinterpret_cast<i32x2*>(ost + dv0 * 2) = i32x2{(int)lo, (int)hi};
        }
      if (OPQ ? ehf == 0 && wq0 + el32 < L : hf == 0 && qvalid)
        p.lse[(size_t)wi.h * T + s0 + (OPQ ? wq0 + el32 : qi)] =
            lt > 0.f ? (w.m + log2f(lt)) * kLn2 : -INFINITY;
      __syncthreads();
      constexpr int CPR = C::DV * 2 / 16;  // 16-byte chunks per output row
#pragma unroll
      for (int i = 0; i < 32 * CPR / kWave; ++i) {
        const int c = el + i * kWave;
        const int r = c / CPR, cc = c % CPR;
        const int row = wq0 + r;
        if (row < L) {
          const i32x4 x =
              *reinterpret_cast<const i32x4*>(smem + (wave * 32 + r) * C::O_ROW + cc * 16);
          // (write-once output: a streaming store, which leaves the L2 to
          // the K/V blocks that later items of the same head read again)
          __builtin_nontemporal_store(
              x, reinterpret_cast<i32x4*>(
                     op + (((size_t)(s0 + row) * p.num_heads + wi.h) * C::DV) * 2 + cc * 16));
        }
      }
      if constexpr (QROWS) place_q_rows();
    }
  }
};

template <class C, bool SPLIT>
__global__ __launch_bounds__(C::THREADS, C::OCC) void attn_fwd_mfma_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  MfmaKernel<C>::template run<SPLIT>(p, smem);
}

template <class C, bool SPLIT = false>
hipError_t launch_mfma(const AttnParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_mfma_kernel<C, SPLIT>), dim3(grid), dim3(C::THREADS), 0, stream,
                     p);
  return hipGetLastError();
}

template <class C>
int blocks_mfma() {
  static int cached = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_fwd_mfma_kernel<C, false>, C::THREADS,
                                                     0) != hipSuccess ||
        n < 1)
      n = 1;
    return n;
  }();
  return cached;
}

}  // namespace mha
