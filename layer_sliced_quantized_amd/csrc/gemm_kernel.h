// Batched (2..16 tokens) Q4_0 / Q8_0 matrix products on the int8 matrix cores.
//
// Same work split as the single-token GEMV (64-row group per wave, K tiles over
// the waves of a workgroup and over split-K workgroups, waves summed in LDS in
// wave order, splits in split order) and the same fp32 operations per (row,
// token, block), so every token's result is bitwise the single-token one.  Only
// the exact integer block sums come from the matrix cores.
//
// Operand layout (checked on gfx950) of v_mfma_i32_16x16x64_i8: lane l holds
// row/column l % 16 and the 16-byte k-group l / 16 of A and of B alike; output
// register i of lane l is C[4 (l / 16) + i][l % 16].
//
// The activation record of a block (MFMA layout, see Act) holds its digits as
// chunks: Q4_0 chunk 4p + g is digit 2p of elements 16 (g & 1) .. +15 for g < 2
// and 16 x digit 2p+1 of those elements for g >= 2 (one 64-deep MFMA takes a
// digit pair, P_p = C_2p + 16 C_2p+1); Q8_0 chunk 2p + h is digit p of
// elements 16 h .. +15.  The block sum is exact in int32: Q4_0
// D = P_0 + 256 (P_1 + 256 P_2) (|D| <= 32 * 8 * 7829367 < 2^31), and (float)D
// is the single rounding of D the GEMV's fused two-part sum also gives; Q8_0
// is combined like the GEMV (digit 2 times 65536 fused with digit 1 * 256 +
// digit 0).
//
// Two uses of the matrix cores, by batch size:
//
// Block-diagonal (2..8 tokens).  A is the wave's own weights, lane l = row l,
// so k-group g of A row m is weight row 16 g + m; B column n = 4 s + t is token
// t of a group of four, and its only nonzero k-group is g = s.  Then
// C[m][4 s + t] = row (16 s + m) . digits of token t: 64 rows x 4 tokens per
// MFMA with no data movement for the weights.  Lane l ends with rows
// 16 ((l & 15) >> 2) + 4 (l >> 4) + i, i = 0..3, of token 4 group + (l & 3).
//
// Dense (9..16 tokens).  One MFMA multiplies 16 weight rows (A) by all 16
// token slots (B) of one block: A's k-groups 0 and 1 hold the row's elements
// 0..15 and 16..31 as int8, k-groups 2 and 3 repeat them (Q4_0) or are zero
// (Q8_0); B's k-groups are the record's chunks of the digit (pair).  A wave's
// 64 rows are 4 row tiles of 16, three MFMAs each per block; each block's rows
// (as int8) pass through a small per-wave LDS buffer so that lane l can take
// row 16 r + l % 16, and the tile's row scales are staged there once per
// tile.  Lane l ends with rows 16 r + 4 (l / 16) + i (r, i = 0..3) of token
// slot l % 16.
//
// In both, the weights stream into registers one tile ahead, lane = row, as in
// the GEMV but block by block into one register set (each block's registers
// are refilled with the next tile's block as soon as they are used), and the
// records of the blocks in use come into a ring of block slots in the wave's
// LDS by buffer loads into LDS (4 slots, four blocks ahead, block-diagonal; 2
// slots, dense).  Each ring wait is an explicit vmcnt that leaves the later
// weight refills and record copies in flight, so no read of the ring waits
// for them.
#pragma once
#include "gemv_kernel.h"

namespace slq {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

// LDS of one ring slot: chunks x tp token slots x 16 B, then the 16 token
// scales.
__host__ __device__ constexpr int gemm_slot(int qt, int tp) { return mx_chunks(qt) * tp * 16 + 64; }
// copy instructions (64 lanes x 16 B) per block
__host__ __device__ constexpr int gemm_dpb(int qt, int tp) { return (gemm_slot(qt, tp) / 16 + 63) / 64; }
// The block-diagonal kernel keeps a ring of 4 block slots per wave: the
// records are L2-resident, so copies four blocks ahead arrive in time, and a
// small ring lets more workgroups share a CU.  The dense kernel's records are
// 3 KB (Q4_0), and LDS bounds its resident waves, so it keeps 2.
constexpr int RING = 4;
constexpr int DENSE_RING = 2;
// Block-diagonal LDS per wave: the ring, the tile's row scales as fp32
// [8 blocks][64 rows], and a zero area as large as one slot's digits (read by
// the B lanes outside the diagonal), placed 64 B further on so that its
// broadcast reads fall in other banks than the chunks read by the lanes
// inside the diagonal.
__host__ __device__ constexpr int gemm_zero(int qt, int tp) { return RING * gemm_slot(qt, tp) + 2048 + 64; }
__host__ __device__ constexpr int diag_region(int qt, int tp) {
  return gemm_zero(qt, tp) + mx_chunks(qt) * tp * 16 > 4096 ? gemm_zero(qt, tp) + mx_chunks(qt) * tp * 16 : 4096;
}
// Dense LDS per wave (16 token slots): the ring, then the block's int8 rows
// as two planes (elements 0..15 and 16..31) [2][64][16 B], the tile's row
// scales [8 blocks][64 rows] fp32 and 16 zero bytes.
constexpr int DENSE_TP = 16;
__host__ __device__ constexpr int dense_abuf(int qt) { return DENSE_RING * gemm_slot(qt, DENSE_TP); }
__host__ __device__ constexpr int dense_region(int qt) { return dense_abuf(qt) + 64 * 32 + TB * 64 * 4 + 16; }
// Either kernel's epilogue reuses the start of each wave's region for
// 16 tokens x 64 rows of sums.
__host__ __device__ constexpr int gemm_region(int qt, int T) {
  return T <= 8 ? diag_region(qt, (T + 3) & ~3) : (dense_region(qt) > 4096 ? dense_region(qt) : 4096);
}
constexpr int GEMM_LDS_MAX = 160 * 1024;
// at most 8 waves (256 registers each: the explicit wait counts rely on the
// kernel never spilling to scratch), a whole number of waves per token group,
// and the LDS of every wave's ring
__host__ __device__ constexpr bool gemm_fits(int qt, int T, int waves) {
  return T >= 1 && T <= MAX_PASS && waves <= 8 && waves % gemm_groups(T) == 0 &&
         waves * gemm_region(qt, T) <= GEMM_LDS_MAX;
}

// s_waitcnt immediate on gfx9: wait until at most n vector-memory operations
// are outstanding (expcnt and lgkmcnt left at their maxima).
__host__ __device__ constexpr unsigned vmcnt_imm(int n) {
  return (unsigned)((n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14));
}

// Byte-addressed buffer descriptor of x's MFMA records (reads past the last
// block return zeros).  Copies go through buffer (not global) loads into LDS:
// the compiler's wait tracking takes a global->LDS load as touching two
// address spaces and then turns every later register wait into a full drain,
// while buffer loads keep the ordinary in-order counting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t mx_rsrc(const Act& x, int qt, int grp = 0) {
  return __builtin_amdgcn_make_buffer_rsrc(x.mxd + (size_t)grp * x.nblk * (mx_block_bytes(qt) / 4), 0,
                                           x.nblk * mx_block_bytes(qt), 0x00020000);
}

// 16 bytes per lane from byte off + 16-byte-piece voff of the buffer straight
// into LDS at dst + 16 * lane (dst and off are the same for the whole wave).
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, unsigned voff, unsigned off, void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)dst, 16, voff, off, 0, 0);
}

// Four two's-complement nibbles in the low halves of the bytes of t (high
// halves zero) -> four int8: ((t ^ 8) + 0x78) ^ 0x80 per byte, no carries.
__device__ __forceinline__ uint32_t sext_nibbles(uint32_t t) {
  return ((t ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u;
}

#define SLQ_COMPILER_FENCE() asm volatile("" ::: "memory")

// The exact block sum of three digit-pair products, D = P0 + 256 (P1 + 256 P2),
// as two shift-adds: the empty asm keeps the compiler from distributing the
// outer shift over the inner sum (which takes three instructions).
__device__ __forceinline__ int digit_sum3(int p0, int p1, int p2) {
  int t = p1 + (p2 << 8);
  asm volatile("" : "+v"(t));
  return p0 + (t << 8);
}

// Digits (token slots 0..tp-1) and scales of block blk into a ring slot:
// piece q < NCH*tp is chunk q / tp, slot q % tp; the last 4 pieces are the
// block's 16 scales.  Exactly DPB instructions (lane 0 is always active).
template <int QT, int DPB>
__device__ __forceinline__ void dma_block(__amdgpu_buffer_rsrc_t rs, int blk, int tp, uint8_t* slot) {
  constexpr int NCH = QT == QT_Q4 ? 12 : 6;
  const int lane = threadIdx.x & 63;
  const int nd = NCH * tp;
  const unsigned rec = (unsigned)blk * (unsigned)mx_block_bytes(QT);
#pragma unroll
  for (int i = 0; i < DPB; ++i) {
    const int q = 64 * i + lane;
    if (q < nd + 4) {
      const unsigned voff =
          q < nd ? (unsigned)(((q / tp) * MX_SLOTS + q % tp) * 16) : (unsigned)(mx_scale_off(QT) + 16 * (q - nd));
      load_lds16(rs, voff, rec, slot + 1024 * i);
    }
  }
}

// One tile: for each block wait for its record's ring slot (b mod 4),
// multiply and fold into acc[group][i]; then (one step) refill the block's
// weight registers with the same block of the next tile and the ring slot
// with the record four blocks on (b + 4 of this tile, or b - 4 of the next).
// The next tile's weights thus arrive one block at a time, a tile ahead of
// their use, in the one register set.  kb: first block of this tile; nb: its
// blocks; ntile, nbn: the next tile's bytes and blocks (nbn = 0: none).
template <int QT, int NG>
__device__ __forceinline__ void tile_diag(TileRegs<QT>& r, int kb, int nb, __amdgpu_buffer_rsrc_t rs,
                                          const uint8_t* ntile, int kb_next, int nbn, int T, uint8_t* ring,
                                          float (&acc)[NG][4]) {
  constexpr int NCH = QT == QT_Q4 ? 12 : 6;
  constexpr int NH = TileRegs<QT>::NH;
  constexpr int TP = 4 * NG;
  constexpr int SLOT = gemm_slot(QT, TP);
  constexpr int DPB = gemm_dpb(QT, TP);
  static_assert(3 * (NH + DPB) + 1 <= 63, "vmcnt holds at most 63 outstanding loads");
  const int lane = threadIdx.x & 63;
  const bool bvalid = ((lane & 15) >> 2) == (lane >> 4);   // B lane inside the diagonal
  const int rbase = 16 * ((lane & 15) >> 2) + 4 * (lane >> 4);
  const uint8_t* zero = ring + gemm_zero(QT, TP);
  // the tile's scales, transposed: sct[b][row] (one 16-byte read per block
  // gives this lane's four rows)
  float* sct = reinterpret_cast<float*>(ring + RING * SLOT);
#pragma unroll
  for (int b = 0; b < TB; ++b) sct[b * 64 + lane] = scale_of(r.sc, b);
  SLQ_COMPILER_FENCE();
  r.sc = load_scales_fixed(ntile, lane, nbn, NH);
  SLQ_COMPILER_FENCE();
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    if (b < nb) {
      // Block b's record was copied (DPB loads, always) at the end of the step
      // after block b - 4 (of the previous tile for b < 4).  Issued later: the
      // next three steps (NH weight and DPB copy loads each, always) and, for
      // b < 4, this tile's scale load.  Loads complete in issue order, so the
      // record has landed once at most 3 (NH + DPB) (+ 1 for b < 4) are
      // outstanding.  (In a wave's first tile the prologue copied blocks 0..3
      // before the tile's weights, so more loads follow those copies: the wait
      // is longer than needed there, never shorter.)
      if (b < 4) __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * (NH + DPB) + 1));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * (NH + DPB)));
      SLQ_COMPILER_FENCE();
      const uint8_t* slot = ring + (b % RING) * SLOT;
      const i32x4 z = {0, 0, 0, 0};
      u32x4 a0, a1;   // A operands: elements 0..15 and 16..31 of the lane's row
      if constexpr (QT == QT_Q4) {
        const u32x4 c = r.c[b];
        a0.x = sext_nibbles(c.x & 0x0F0F0F0Fu);
        a0.y = sext_nibbles(c.y & 0x0F0F0F0Fu);
        a0.z = sext_nibbles(c.z & 0x0F0F0F0Fu);
        a0.w = sext_nibbles(c.w & 0x0F0F0F0Fu);
        a1.x = sext_nibbles((c.x >> 4) & 0x0F0F0F0Fu);
        a1.y = sext_nibbles((c.y >> 4) & 0x0F0F0F0Fu);
        a1.z = sext_nibbles((c.z >> 4) & 0x0F0F0F0Fu);
        a1.w = sext_nibbles((c.w >> 4) & 0x0F0F0F0Fu);
      } else {
        a0 = r.c[2 * b];
        a1 = r.c[2 * b + 1];
      }
      const i32x4 A0 = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w};
      const i32x4 A1 = {(int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      float d[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = sct[b * 64 + rbase + i];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        SLQ_COMPILER_FENCE();
        const int t = 4 * g + (lane & 3);
        const float xs = t < T ? reinterpret_cast<const float*>(slot + NCH * TP * 16)[t] : 0.0f;
        // B operand lanes: token t's chunks inside the diagonal, zeros outside
        const uint8_t* bsrc = bvalid ? slot + t * 16 : zero;
        i32x4 P[3];
#pragma unroll
        for (int p = 0; p < 3; ++p) {
          if constexpr (QT == QT_Q4) {
            i32x4 bq[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) bq[k] = *reinterpret_cast<const i32x4*>(bsrc + (4 * p + k) * TP * 16);
            i32x4 C = __builtin_amdgcn_mfma_i32_16x16x64_i8(A0, bq[0], z, 0, 0, 0);
            C = __builtin_amdgcn_mfma_i32_16x16x64_i8(A1, bq[1], C, 0, 0, 0);
            C = __builtin_amdgcn_mfma_i32_16x16x64_i8(A0, bq[2], C, 0, 0, 0);
            P[p] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A1, bq[3], C, 0, 0, 0);
          } else {
            i32x4 bq[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) bq[k] = *reinterpret_cast<const i32x4*>(bsrc + (2 * p + k) * TP * 16);
            const i32x4 C = __builtin_amdgcn_mfma_i32_16x16x64_i8(A0, bq[0], z, 0, 0, 0);
            P[p] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A1, bq[1], C, 0, 0, 0);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float bf;
          if constexpr (QT == QT_Q4) {
            bf = (float)digit_sum3(P[0][i], P[1][i], P[2][i]);
          } else {
            bf = __builtin_fmaf((float)P[2][i], 65536.0f, (float)(P[0][i] + (P[1][i] << 8)));
          }
          acc[g][i] = __builtin_fmaf(bf, d[i] * xs, acc[g][i]);
          // keep the fold here: otherwise the compiler sinks every block's
          // fold to the end of the tile and keeps all MFMA results live
          asm volatile("" : "+v"(acc[g][i]));
        }
      }
    }
    // the step: block b of the next tile into the registers just used, and
    // the record four blocks on into slot b mod 4; where there is none, dummy
    // loads (the last block again, or block 0's record into the unused slot)
    // keep the load count fixed
    SLQ_COMPILER_FENCE();
    load_block_fixed<QT>(ntile, lane, nbn, b, r);
    const int nxt = b < 4 ? (b + 4 < nb ? kb + b + 4 : 0) : (b - 4 < nbn ? kb_next + b - 4 : 0);
    dma_block<QT, DPB>(rs, nxt, TP, ring + (b % RING) * SLOT);
    SLQ_COMPILER_FENCE();
  }
}

// One tile: for each block wait for its record's ring slot (b mod
// DENSE_RING), stage the block's rows, multiply, fold into acc[r][i]; then
// (one step) refill the block's weight registers with the same block of the
// next tile and the ring slot with the record DENSE_RING blocks on (in this
// tile or the next).  kb: first block of this tile; nb: its blocks; ntile,
// nbn: the next tile's bytes and blocks (nbn = 0: none).
template <int QT, int TP, bool NT>
__device__ __forceinline__ void tile_dense(TileRegs<QT>& w, int kb, int nb, __amdgpu_buffer_rsrc_t rs,
                                           const uint8_t* ntile, int kb_next, int nbn, uint8_t* ring,
                                           float (&acc)[4][4]) {
  constexpr int NCH = QT == QT_Q4 ? 12 : 6;
  constexpr int NH = TileRegs<QT>::NH;
  constexpr int SLOT = gemm_slot(QT, TP);
  constexpr int DPB = gemm_dpb(QT, TP);
  constexpr int DR = DENSE_RING;
  static_assert(TB % DR == 0 && (DR - 1) * (NH + DPB) + 1 <= 63, "ring depth");
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, s = lane & 15;         // k-group and token slot (row in the tile) of this lane
  uint8_t* abuf = ring + dense_abuf(QT);
  float* sct = reinterpret_cast<float*>(abuf + 64 * 32);
  const uint8_t* zero16 = abuf + 64 * 32 + TB * 64 * 4;
  // this lane's A source in row tile r: row 16 r + s, elements 16 (g & 1) ..
  // (plane g & 1 of the staged rows; 16 lanes read 256 contiguous bytes)
  const uint8_t* asrc = (QT == QT_Q8 && g >= 2) ? zero16 : abuf + (g & 1) * 64 * 16 + s * 16;
  const int astep = (QT == QT_Q8 && g >= 2) ? 0 : 16 * 16;
  // this lane's B chunk for digit (pair) p is c0 + p * cstep
  const int c0 = QT == QT_Q4 ? g : (g & 1);
  constexpr int cstep = QT == QT_Q4 ? 4 : 2;
  // the tile's scales, transposed: sct[b][row]; then w.sc takes the next
  // tile's
#pragma unroll
  for (int b = 0; b < TB; ++b) sct[b * 64 + lane] = scale_of(w.sc, b);
  SLQ_COMPILER_FENCE();
  w.sc = load_scales_fixed<NT>(ntile, lane, nbn, NH);
  SLQ_COMPILER_FENCE();
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    if (b < nb) {
      // Block b's record was copied (DPB loads, always) at the end of the step
      // after block b - DR (of the previous tile for b < DR).  Issued later:
      // the next DR - 1 steps (NH weight and DPB copy loads each, always) and,
      // for b < DR, this tile's scale load.  Loads complete in issue order, so
      // the record has landed once at most (DR - 1)(NH + DPB) (+ 1 for b < DR)
      // are outstanding.  (In a wave's first tile the prologue copied blocks
      // 0..DR-1 before the tile's weights, so more loads follow those copies:
      // the wait is longer than needed there, never shorter.)
      if (b < DR) __builtin_amdgcn_s_waitcnt(vmcnt_imm((DR - 1) * (NH + DPB) + 1));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm((DR - 1) * (NH + DPB)));
      SLQ_COMPILER_FENCE();
      // stage row `lane` of block b: elements 0..31 as int8
      u32x4 lo, hi;
      if constexpr (QT == QT_Q4) {
        const u32x4 c = w.c[b];
        lo.x = sext_nibbles(c.x & 0x0F0F0F0Fu);
        lo.y = sext_nibbles(c.y & 0x0F0F0F0Fu);
        lo.z = sext_nibbles(c.z & 0x0F0F0F0Fu);
        lo.w = sext_nibbles(c.w & 0x0F0F0F0Fu);
        hi.x = sext_nibbles((c.x >> 4) & 0x0F0F0F0Fu);
        hi.y = sext_nibbles((c.y >> 4) & 0x0F0F0F0Fu);
        hi.z = sext_nibbles((c.z >> 4) & 0x0F0F0F0Fu);
        hi.w = sext_nibbles((c.w >> 4) & 0x0F0F0F0Fu);
      } else {
        lo = w.c[2 * b];
        hi = w.c[2 * b + 1];
      }
      reinterpret_cast<u32x4*>(abuf)[lane] = lo;
      reinterpret_cast<u32x4*>(abuf + 64 * 16)[lane] = hi;
      // (LDS accesses of one wave take effect in program order: the reads
      // below see these writes)
      const uint8_t* slot = ring + (b % DR) * SLOT;
      i32x4 bq[3];
#pragma unroll
      for (int p = 0; p < 3; ++p) bq[p] = *reinterpret_cast<const i32x4*>(slot + ((c0 + p * cstep) * TP + s) * 16);
      const float xs = reinterpret_cast<const float*>(slot + NCH * TP * 16)[s];
      const i32x4 z = {0, 0, 0, 0};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const i32x4 A = *reinterpret_cast<const i32x4*>(asrc + r * astep);
        float dd[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) dd[i] = sct[b * 64 + 16 * r + 4 * g + i];
        const i32x4 P0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, bq[0], z, 0, 0, 0);
        const i32x4 P1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, bq[1], z, 0, 0, 0);
        const i32x4 P2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, bq[2], z, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float bf;
          if constexpr (QT == QT_Q4) {
            bf = (float)digit_sum3(P0[i], P1[i], P2[i]);
          } else {
            bf = __builtin_fmaf((float)P2[i], 65536.0f, (float)(P0[i] + (P1[i] << 8)));
          }
          acc[r][i] = __builtin_fmaf(bf, dd[i] * xs, acc[r][i]);
        }
      }
    }
    // the step: block b of the next tile into the registers just used, and
    // the record DR blocks on into slot b mod DR; where there is none, dummy
    // loads (the last block again, or block 0's record into the unused slot)
    // keep the load count fixed
    SLQ_COMPILER_FENCE();
    load_block_fixed<QT, NT>(ntile, lane, nbn, b, w);
    const int nxt = b < TB - DR ? (b + DR < nb ? kb + b + DR : 0) : (b + DR - TB < nbn ? kb_next + b + DR - TB : 0);
    dma_block<QT, DPB>(rs, nxt, TP, ring + (b % DR) * SLOT);
    SLQ_COMPILER_FENCE();
  }
}

// Epilogue of token j for the 64 rows of group rg; lane = row, a = sum over K.
// pre: the token's RMSNorm factor (STORE, SWIGLU) or its residual entry h
// (RESID), fetched at kernel start; nw_row: next RMSNorm weight of the row.
template <int QT, int EPI>
__device__ __forceinline__ void gemm_epi(const Packed& W, const GemvOut& out, int rg, int j, float a, float pre,
                                         float nw_row) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)rg * RG + lane;
  const bool rv = row < W.rows;
  if constexpr (EPI == EPI_STORE) {
    if (rv) out.y[(size_t)j * out.y_tstride + row] = a * pre;
  } else if constexpr (EPI == EPI_SWIGLU) {
    // lanes 0..31: gate rows, lanes 32..63: the matching up rows
    const float v = a * pre;
    const float up = xor_lane<32>(v);   // row lane ^ 32
    const float m = (v / (1.0f + expf(-v))) * up;
    if (out.y && lane < 32) out.y[(size_t)j * out.y_tstride + rg * 32 + lane] = m;
    put_digits(out.next, out.next_qt, j, rg, m, lane < 32);
  } else {  // EPI_RESID
    const float hn = rv ? pre + a : 0.0f;
    resid_tail_w(j, rg, (int)W.rows, hn, nw_row, out.y, out.y_tstride, out.next_qt, out.next, out.ssq_out, W.nrg());
  }
}

// What token j's epilogue reads besides the sum: its RMSNorm factor (STORE,
// SWIGLU) or this row's residual entry (RESID); 1 / 0 for j >= T.
template <int EPI>
__device__ __forceinline__ float epi_input(const GemvOut& out, const NormIn& nin, int64_t row, bool rv, int j, int T) {
  if constexpr (EPI == EPI_RESID) return (j < T && rv) ? out.y[(size_t)j * out.y_tstride + row] : 0.0f;
  else return j < T ? rnorm_from(nin, j) : 1.0f;
}

// The same in two steps, so that the loads fly under the first tile: fetch
// this row's residual entry (RESID) or the token's sum-of-squares partials,
// two per lane (STORE, SWIGLU), and after the main loop fold them into the
// RMSNorm factor with the additions of rnorm_from (bitwise the same value).
struct EpiRaw {
  float a, b;
};
template <int EPI>
__device__ __forceinline__ EpiRaw epi_fetch(const GemvOut& out, const NormIn& nin, int64_t row, bool rv, int j, int T) {
  if constexpr (EPI == EPI_RESID) {
    return {(j < T && rv) ? out.y[(size_t)j * out.y_tstride + row] : 0.0f, 0.0f};
  } else {
    if (j >= T) return {0.0f, 0.0f};
    const RnRaw r = rnorm_fetch(nin, j);
    return {r.a, r.b};
  }
}
template <int EPI>
__device__ __forceinline__ float epi_finish(const EpiRaw& r, const NormIn& nin, int j, int T) {
  if constexpr (EPI == EPI_RESID) {
    return r.a;
  } else {
    if (j >= T) return 1.0f;
    return rnorm_finish(RnRaw{r.a, r.b}, nin, j);
  }
}

template <int QT, int EPI, int NG>
__global__ __launch_bounds__(512) void k_gemm_diag(Packed W, Act x, NormIn nin, GemvOut out, int ksplit, int T) {
  constexpr int TBY = tile_bytes(QT);
  constexpr int TP = 4 * NG;
  constexpr int REGION = diag_region(QT, TP);
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int nw = blockDim.x >> 6;
  const int rg = blockIdx.x / ksplit, ks = blockIdx.x % ksplit;
  const int nblk = W.nblk(), ntiles = W.ntiles(), full = nblk / TB;
  const int w0 = ntiles * ks / ksplit, w1 = ntiles * (ks + 1) / ksplit;
  const int t0 = __builtin_amdgcn_readfirstlane(w0 + (w1 - w0) * wave / nw);
  const int t1 = __builtin_amdgcn_readfirstlane(w0 + (w1 - w0) * (wave + 1) / nw);
  const uint8_t* base = W.w + (size_t)rg * rg_bytes(QT, W.cols);
  uint8_t* ring = lds + (size_t)wave * REGION;
  auto nb_of = [&](int t) { return t < full ? TB : nblk - full * TB; };
  {
    constexpr int NZ = (QT == QT_Q4 ? 12 : 6) * TP;   // 16-byte pieces of the zero area
    u32x4* zero = reinterpret_cast<u32x4*>(ring + gemm_zero(QT, TP));
    for (int i = lane; i < NZ; i += 64) zero[i] = u32x4{0u, 0u, 0u, 0u};
  }

  float acc[NG][4];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[g][i] = 0.0f;

  const __amdgpu_buffer_rsrc_t rs = mx_rsrc(x, QT);
  TileRegs<QT> R;
  if (t0 < t1) {
    // prologue: the records of tile t0's first 4 blocks into the ring (block
    // 0 again past a ragged tile's end), then the tile's weights
#pragma unroll
    for (int b = 0; b < RING; ++b)
      dma_block<QT, gemm_dpb(QT, TP)>(rs, b < nb_of(t0) ? t0 * TB + b : 0, TP, ring + b * gemm_slot(QT, TP));
    SLQ_COMPILER_FENCE();
    load_tile_fixed<QT>(base + (size_t)t0 * TBY, lane, nb_of(t0), R);
    SLQ_COMPILER_FENCE();
  }

  // The first four tokens this wave finishes (j = wave + nw q): what their
  // epilogues read is requested now, behind the first tile, so its latency
  // hides under the weights.
  const int64_t erow = (int64_t)rg * RG + lane;
  const bool erv = erow < W.rows;
  EpiRaw raw[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) raw[q] = epi_fetch<EPI>(out, nin, erow, erv, wave + nw * q, T);
  const float nw_row = EPI == EPI_RESID ? (erv ? out.norm_w[erow] : 0.0f) : 0.0f;
  SLQ_COMPILER_FENCE();

  if (t0 < t1) {
    // each tile refills the registers with the next tile's weights (lane-
    // uniform dummies after the wave's last tile).  The first tile runs
    // before the loop, so the loop is entered in the same state as it loops
    // back, and the compiler's waits on the refilled registers stay exact
    // instead of draining every load at the top of each tile.
    auto one = [&](int t) {
      const bool n1 = t + 1 < t1;
      tile_diag<QT, NG>(R, t * TB, nb_of(t), rs, base + (size_t)(n1 ? t + 1 : t) * TBY, (t + 1) * TB,
                        n1 ? nb_of(t + 1) : 0, T, ring, acc);
    };
    one(t0);
    for (int t = t0 + 1; t < t1; ++t) one(t);
    // the dummy refills of the last tile still write the ring, which the
    // reduction below reuses
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }

  float pre[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) pre[q] = epi_finish<EPI>(raw[q], nin, wave + nw * q, T);

  // Waves meet in LDS: red[token][row] in each wave's own region.  Token j is
  // finished by wave j % nw, which adds the waves in wave order.
  __syncthreads();
  {
    float* red = reinterpret_cast<float*>(ring);
    const int rbase = 16 * ((lane & 15) >> 2) + 4 * (lane >> 4);
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[(4 * g + (lane & 3)) * RG + rbase + i] = acc[g][i];
  }
  __syncthreads();
  // token j of this wave: sum of the waves' values in wave order
  auto wave_sum_of = [&](int j) {
    float a = reinterpret_cast<const float*>(lds)[(size_t)j * RG + lane];
    for (int w = 1; w < nw; ++w) a += reinterpret_cast<const float*>(lds + (size_t)w * REGION)[(size_t)j * RG + lane];
    return a;
  };
  auto pre_of = [&](int q, int j) {
    return q == 0 ? pre[0] : q == 1 ? pre[1] : q == 2 ? pre[2] : q == 3 ? pre[3] : epi_input<EPI>(out, nin, erow, erv, j, T);
  };
  if (ksplit == 1) {
    for (int q = 0, j = wave; j < T; ++q, j += nw) gemm_epi<QT, EPI>(W, out, rg, j, wave_sum_of(j), pre_of(q, j), nw_row);
    return;
  }

  // Same exchange as the GEMV: partials move through agent-scope atomics,
  // every wave's stores are complete before the workgroup takes its ticket,
  // and the last split adds them in split order.
  for (int j = wave; j < T; j += nw)
    __hip_atomic_store(out.part + (((size_t)rg * ksplit + ks) * T + j) * RG + lane, wave_sum_of(j), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  unsigned* tk = reinterpret_cast<unsigned*>(lds);
  if (threadIdx.x == 0) tk[0] = __hip_atomic_fetch_add(out.cnt + rg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const unsigned ticket = tk[0];
  if (ticket != (unsigned)(ksplit - 1)) return;
  const float* all = out.part + (size_t)rg * ksplit * T * RG;
  for (int q = 0, j = wave; j < T; ++q, j += nw) {
    float pv[16];   // all splits' loads in flight together
#pragma unroll
    for (int k2 = 0; k2 < 16; ++k2)
      pv[k2] = k2 < ksplit ? __hip_atomic_load(all + ((size_t)k2 * T + j) * RG + lane, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)
                           : 0.0f;
    float sum = 0.0f;
#pragma unroll
    for (int k2 = 0; k2 < 16; ++k2)
      if (k2 < ksplit) sum += pv[k2];
    gemm_epi<QT, EPI>(W, out, rg, j, sum, pre_of(q, j), nw_row);
  }
  if (threadIdx.x == 0) __hip_atomic_store(out.cnt + rg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// NGR token groups (prompt passes of 17..64 tokens): wave w multiplies group
// w % NGR over K part w / NGR of the split, so the waves of one K part read
// the same weight tiles: with ordinary loads (not nontemporal ones) L2 keeps
// a tile for the other groups' waves, and HBM delivers it once; tokens of
// group g are summed over the K parts in order.  NGR = 1 is the 9..16-token
// form (nontemporal weight loads).
template <int QT, int EPI, int NGR>
__global__ __launch_bounds__(512) void k_gemm_dense(Packed W, Act x, NormIn nin, GemvOut out, int ksplit, int T) {
  constexpr int TBY = tile_bytes(QT);
  constexpr int TP = DENSE_TP;
  constexpr int REGION = dense_region(QT) > 4096 ? dense_region(QT) : 4096;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int nw = blockDim.x >> 6;
  const int grp = wave % NGR, kw = wave / NGR, nkw = nw / NGR;
  const int rg = blockIdx.x / ksplit, ks = blockIdx.x % ksplit;
  const int nblk = W.nblk(), ntiles = W.ntiles(), full = nblk / TB;
  const int w0 = ntiles * ks / ksplit, w1 = ntiles * (ks + 1) / ksplit;
  const int t0 = __builtin_amdgcn_readfirstlane(w0 + (w1 - w0) * kw / nkw);
  const int t1 = __builtin_amdgcn_readfirstlane(w0 + (w1 - w0) * (kw + 1) / nkw);
  const uint8_t* base = W.w + (size_t)rg * rg_bytes(QT, W.cols);
  uint8_t* ring = lds + (size_t)wave * REGION;
  auto nb_of = [&](int t) { return t < full ? TB : nblk - full * TB; };
  if (lane == 0) *reinterpret_cast<u32x4*>(ring + dense_abuf(QT) + 64 * 32 + TB * 64 * 4) = u32x4{0u, 0u, 0u, 0u};

  float acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[r][i] = 0.0f;

  const __amdgpu_buffer_rsrc_t rs = mx_rsrc(x, QT, grp);
  TileRegs<QT> R;
  if (t0 < t1) {
    // prologue: the records of tile t0's first DENSE_RING blocks into the
    // ring (block 0 again past a ragged tile's end), then the tile's weights
#pragma unroll
    for (int b = 0; b < DENSE_RING; ++b)
      dma_block<QT, gemm_dpb(QT, TP)>(rs, b < nb_of(t0) ? t0 * TB + b : 0, TP, ring + b * gemm_slot(QT, TP));
    SLQ_COMPILER_FENCE();
    load_tile_fixed<QT, NGR == 1>(base + (size_t)t0 * TBY, lane, nb_of(t0), R);
    SLQ_COMPILER_FENCE();
  }

  // The first four tokens this wave finishes (j = wave + nw q): what their
  // epilogues read is requested now, behind the first tile, so its latency
  // hides under the weights.
  const int64_t erow = (int64_t)rg * RG + lane;
  const bool erv = erow < W.rows;
  EpiRaw raw[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) raw[q] = epi_fetch<EPI>(out, nin, erow, erv, wave + nw * q, T);
  const float nw_row = EPI == EPI_RESID ? (erv ? out.norm_w[erow] : 0.0f) : 0.0f;
  SLQ_COMPILER_FENCE();

  if (t0 < t1) {
    // each tile refills the registers with the next tile's weights (lane-
    // uniform dummies after the wave's last tile); the first tile runs before
    // the loop, as in the block-diagonal form
    auto one = [&](int t) {
      const bool n1 = t + 1 < t1;
      tile_dense<QT, TP, NGR == 1>(R, t * TB, nb_of(t), rs, base + (size_t)(n1 ? t + 1 : t) * TBY, (t + 1) * TB,
                                   n1 ? nb_of(t + 1) : 0, ring, acc);
    };
    one(t0);
    for (int t = t0 + 1; t < t1; ++t) one(t);
    // the dummy refills of the last tile still write the ring, which the
    // reduction below reuses
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }

  float pre[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) pre[q] = epi_finish<EPI>(raw[q], nin, wave + nw * q, T);

  // Waves meet in LDS: red[token][row] in each wave's own region.  Token j is
  // finished by wave j % nw, which adds the waves in wave order.
  __syncthreads();
  {
    // lane l holds rows 16 r + 4 (l / 16) + i of token slot l % 16 (slots
    // past T hold nothing of use and are never read)
    float* red = reinterpret_cast<float*>(ring) + (lane & 15) * RG + 4 * (lane >> 4);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      *reinterpret_cast<float4*>(red + 16 * r) = float4{acc[r][0], acc[r][1], acc[r][2], acc[r][3]};
  }
  __syncthreads();
  // token j: slot j % 16 of the waves of group j / 16, added in K-part order
  auto wave_sum_of = [&](int j) {
    const int g = j / MX_SLOTS, sl = j % MX_SLOTS;
    float a = reinterpret_cast<const float*>(lds + (size_t)g * REGION)[(size_t)sl * RG + lane];
    for (int k = 1; k < nkw; ++k)
      a += reinterpret_cast<const float*>(lds + (size_t)(k * NGR + g) * REGION)[(size_t)sl * RG + lane];
    return a;
  };
  auto pre_of = [&](int q, int j) {
    return q == 0 ? pre[0] : q == 1 ? pre[1] : q == 2 ? pre[2] : q == 3 ? pre[3] : epi_input<EPI>(out, nin, erow, erv, j, T);
  };
  if (ksplit == 1) {
    for (int q = 0, j = wave; j < T; ++q, j += nw) gemm_epi<QT, EPI>(W, out, rg, j, wave_sum_of(j), pre_of(q, j), nw_row);
    return;
  }

  // Same exchange as the GEMV: partials move through agent-scope atomics,
  // every wave's stores are complete before the workgroup takes its ticket,
  // and the last split adds them in split order.
  for (int j = wave; j < T; j += nw)
    __hip_atomic_store(out.part + (((size_t)rg * ksplit + ks) * T + j) * RG + lane, wave_sum_of(j), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  unsigned* tk = reinterpret_cast<unsigned*>(lds);
  if (threadIdx.x == 0) tk[0] = __hip_atomic_fetch_add(out.cnt + rg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const unsigned ticket = tk[0];
  if (ticket != (unsigned)(ksplit - 1)) return;
  const float* all = out.part + (size_t)rg * ksplit * T * RG;
  for (int q = 0, j = wave; j < T; ++q, j += nw) {
    float pv[16];   // all splits' loads in flight together
#pragma unroll
    for (int k2 = 0; k2 < 16; ++k2)
      pv[k2] = k2 < ksplit ? __hip_atomic_load(all + ((size_t)k2 * T + j) * RG + lane, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)
                           : 0.0f;
    float sum = 0.0f;
#pragma unroll
    for (int k2 = 0; k2 < 16; ++k2)
      if (k2 < ksplit) sum += pv[k2];
    gemm_epi<QT, EPI>(W, out, rg, j, sum, pre_of(q, j), nw_row);
  }
  if (threadIdx.x == 0) __hip_atomic_store(out.cnt + rg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int QT, int EPI>
hipError_t gemm_inst(const Packed& W, int T, Act x, NormIn nin, GemvOut out, int ksplit, int waves,
                     hipStream_t s) {
  if (!x.mxd || ksplit < 1 || ksplit > 16 || waves < 1 || !gemm_fits(QT, T, waves))
    return hipErrorInvalidValue;
  if (ksplit > 1 && (!out.part || !out.cnt)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(W.nrg() * ksplit)), block(64 * waves);
  const size_t lds = (size_t)waves * gemm_region(QT, T);
  if (T <= 4) k_gemm_diag<QT, EPI, 1><<<grid, block, lds, s>>>(W, x, nin, out, ksplit, T);
  else if (T <= 8) k_gemm_diag<QT, EPI, 2><<<grid, block, lds, s>>>(W, x, nin, out, ksplit, T);
  else if (T <= MX_SLOTS) k_gemm_dense<QT, EPI, 1><<<grid, block, lds, s>>>(W, x, nin, out, ksplit, T);
  else if (gemm_groups(T) == 2) k_gemm_dense<QT, EPI, 2><<<grid, block, lds, s>>>(W, x, nin, out, ksplit, T);
  else k_gemm_dense<QT, EPI, 4><<<grid, block, lds, s>>>(W, x, nin, out, ksplit, T);
  return hipGetLastError();
}

#define SLQ_DECLARE_GEMM(QT, EPI) \
  extern template hipError_t gemm_inst<QT, EPI>(const Packed&, int, Act, NormIn, GemvOut, int, int, hipStream_t);
SLQ_DECLARE_GEMM(QT_Q4, EPI_STORE) SLQ_DECLARE_GEMM(QT_Q4, EPI_SWIGLU) SLQ_DECLARE_GEMM(QT_Q4, EPI_RESID)
SLQ_DECLARE_GEMM(QT_Q8, EPI_STORE) SLQ_DECLARE_GEMM(QT_Q8, EPI_SWIGLU) SLQ_DECLARE_GEMM(QT_Q8, EPI_RESID)
#undef SLQ_DECLARE_GEMM

}  // namespace slq
