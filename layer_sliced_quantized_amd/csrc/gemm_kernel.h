// Batched (2..16 tokens) Q4_0 / Q8_0 matrix products on the int8 matrix cores.
//
// Each token's result is bitwise the one the single-token GEMV gives.  The
// single-token GEMV splits the K tiles of a 64-row group over ks workgroups and
// w waves ("units" u = split * w + wave), adds the waves of a split in wave order
// and the splits in split order, and applies the same fp32 operations to every
// block.  This kernel keeps every unit's tile range and block order and the
// order of the final sums; only the exact integer block sums come from the
// matrix cores:
//
//   Q4_0: v_mfma_i32_16x16x64_i8, A = digits of 16 token slots (activation
//         layout fmt 1: 64 k-entries = digit 2p of the 32 elements and 16 x digit
//         2p+1 of them), B = 16 weight rows, each 4-bit code widened to int8.
//         Three MFMAs give P_p = C_2p + 16 C_2p+1 (C_d = codes . digit d); the
//         block sum D = P_0 + 256 (P_1 + 256 P_2) is exact in int32 (|D| <= 32 *
//         8 * 7829367 < 2^31), and (float)D is the single rounding of D that
//         the GEMV's two-part fma also produces.
//   Q8_0: v_mfma_i32_16x16x32_i8 per base-256 digit; combined exactly like the
//         GEMV (digit 2 times 65536 fused with digit 1 * 256 + digit 0).
//
// Operand layout (checked on gfx950): lane l holds row/column l % 16 and
// k-group l / 16 of A and of B alike; output register i of lane l is
// C[4 (l / 16) + i][l % 16].  Here C rows are tokens and columns weight rows.
//
// Work split: a workgroup of R waves takes R consecutive row groups (one per
// wave) and one unit u, so all its waves walk the same K tiles.  The
// activation digits of a tile (only the token slots in use, rounded up to 4)
// are copied once per workgroup into LDS with direct global->LDS loads one
// tile ahead, next to each wave's next weight tile (registers), so no load has
// to wait for a later-issued one.  Every unit publishes its partial sums; the
// last unit of a row group (atomic ticket) adds them in the GEMV's order and
// runs the epilogue.
#pragma once
#include "gemv_kernel.h"

namespace slq {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

constexpr int GEMM_R = 4;                       // row groups (waves) per workgroup
constexpr int GEMM_STAGE = 3072;                // per wave: 2 KB staged codes + 1 KB tile scales
constexpr int GEMM_MAX_UNITS = 64;              // split-K workgroups x waves of the single-token plan
// bytes of one row of chunk slots per block in LDS: 12 chunks x tp slots x (16 or 8) B
__host__ __device__ constexpr int gemm_blk_lds(int qt, int tp) { return 12 * tp * (qt == QT_Q4 ? 16 : 8); }
// LDS of one tile of digits (tp slots) + its scales (16 slots)
__host__ __device__ constexpr int gemm_act_tile(int qt, int tp) { return TB * gemm_blk_lds(qt, tp) + TB * MX_SLOTS * 4; }
__host__ __device__ constexpr int gemm_lds_bytes(int qt, int tp) {
  return 2 * gemm_act_tile(qt, tp) + GEMM_R * GEMM_STAGE > GEMM_R * 4096 ? 2 * gemm_act_tile(qt, tp) + GEMM_R * GEMM_STAGE
                                                                         : GEMM_R * 4096;
}

// 16 bytes per lane from global memory straight into LDS at dst + 16 * lane
// (dst is the same for the whole wave).
__device__ __forceinline__ void load_lds16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)dst, 16, 0, 0);
}

// Four two's-complement nibbles in the low halves of the bytes of t (high
// halves zero) -> four int8: ((t ^ 8) + 0x78) ^ 0x80 per byte, no carries.
__device__ __forceinline__ uint32_t sext_nibbles(uint32_t t) {
  return ((t ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u;
}

#define SLQ_COMPILER_FENCE() asm volatile("" ::: "memory")
#define SLQ_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// Copy the digits of tile blocks kb .. kb+nb-1, token slots 0 .. tp-1, into
// LDS as [block][chunk][slot] (tp slots), then the block scales [block][16].
// Every wave of the workgroup takes a share of the 16-byte pieces.
template <int QT>
__device__ __forceinline__ void stage_act(const Act& x, int kb, int nb, int tp, uint8_t* dst, int wave, int R) {
  constexpr int PB = QT == QT_Q4 ? 16 : 8;       // bytes per slot of a chunk
  constexpr int SPP = 16 / PB;                   // slots per 16-byte piece
  const int lane = threadIdx.x & 63;
  const uint8_t* src = reinterpret_cast<const uint8_t*>(x.xd);
  const int ppc = tp / SPP;                      // pieces per chunk
  const int n16 = nb * 12 * ppc;
  for (int i = wave * 64; i < n16; i += R * 64) {
    const int q = i + lane;
    if (q < n16) {
      const int b = q / (12 * ppc), c = (q / ppc) % 12, m = (q % ppc) * SPP;
      load_lds16(src + ((((size_t)(kb + b) * 12 + c) * MX_SLOTS + m) * PB), dst + (size_t)i * 16);
    }
  }
  if (wave == R - 1 && lane < nb * (MX_SLOTS / 4))
    load_lds16(reinterpret_cast<const uint8_t*>(x.xs + (size_t)kb * MX_SLOTS) + lane * 16,
               dst + TB * gemm_blk_lds(QT, tp));
}

// All blocks of one tile: stage the weights, multiply, fold into acc[s][i]
// (row 16 s + (lane & 15), token 4 (lane >> 4) + i).  act: the tile's digits
// (tp slots) and scales in LDS.
template <int QT>
__device__ __forceinline__ void tile_mma(const TileRegs<QT>& r, int nb, const uint8_t* act, int T, int tp,
                                         uint8_t* my, float (&acc)[4][4]) {
  constexpr int PB = QT == QT_Q4 ? 16 : 8;
  const int BL = gemm_blk_lds(QT, tp);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const bool slot_ok = n < T;   // A operand: this lane carries token slot n
  u32x4* sc_lds = reinterpret_cast<u32x4*>(my + 2048);
  sc_lds[lane] = r.sc;
  SLQ_COMPILER_FENCE();
  u32x4 scw[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) scw[s] = sc_lds[16 * s + n];
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    if (b < nb) {
      SLQ_SCHED_FENCE();
      // chunk c = 4p + g, slot n of block b
      const uint8_t* ab = act + (size_t)b * BL + ((size_t)g * tp + n) * PB;
      const float4 s4 = reinterpret_cast<const float4*>(act + TB * BL)[b * (MX_SLOTS / 4) + g];
      const float xs[4] = {4 * g + 0 < T ? s4.x : 0.0f, 4 * g + 1 < T ? s4.y : 0.0f, 4 * g + 2 < T ? s4.z : 0.0f,
                           4 * g + 3 < T ? s4.w : 0.0f};
      if constexpr (QT == QT_Q4) {
        const u32x4 c = r.c[b];
        u32x4 lo, hi;
        lo.x = sext_nibbles(c.x & 0x0F0F0F0Fu);
        lo.y = sext_nibbles(c.y & 0x0F0F0F0Fu);
        lo.z = sext_nibbles(c.z & 0x0F0F0F0Fu);
        lo.w = sext_nibbles(c.w & 0x0F0F0F0Fu);
        hi.x = sext_nibbles((c.x >> 4) & 0x0F0F0F0Fu);
        hi.y = sext_nibbles((c.y >> 4) & 0x0F0F0F0Fu);
        hi.z = sext_nibbles((c.z >> 4) & 0x0F0F0F0Fu);
        hi.w = sext_nibbles((c.w >> 4) & 0x0F0F0F0Fu);
        u32x4* st = reinterpret_cast<u32x4*>(my);
        st[lane] = lo;        // weights j of row `lane`
        st[RG + lane] = hi;   // weights j + 16
      } else {
        u32x4* st = reinterpret_cast<u32x4*>(my);
        st[2 * lane] = r.c[2 * b];
        st[2 * lane + 1] = r.c[2 * b + 1];
      }
      SLQ_COMPILER_FENCE();
      const i32x4 z = {0, 0, 0, 0};
      if constexpr (QT == QT_Q4) {
        i32x4 a[3];
#pragma unroll
        for (int p = 0; p < 3; ++p) a[p] = slot_ok ? *reinterpret_cast<const i32x4*>(ab + (size_t)p * 4 * tp * PB) : z;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float d = scale_of(scw[s], b);
          const u32x4 wu = reinterpret_cast<const u32x4*>(my)[(g & 1) * RG + 16 * s + n];
          const i32x4 wv = {(int)wu.x, (int)wu.y, (int)wu.z, (int)wu.w};
          const i32x4 C0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[0], wv, z, 0, 0, 0);
          const i32x4 C1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[1], wv, z, 0, 0, 0);
          const i32x4 C2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[2], wv, z, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int D = C0[i] + ((C1[i] + (C2[i] << 8)) << 8);
            acc[s][i] = __builtin_fmaf((float)D, d * xs[i], acc[s][i]);
            // keep the fold here: otherwise the compiler sinks every block's
            // fold to the end of the tile and keeps all MFMA results live
            asm volatile("" : "+v"(acc[s][i]));
          }
        }
      } else {
        long a[3];
#pragma unroll
        for (int p = 0; p < 3; ++p) a[p] = slot_ok ? *reinterpret_cast<const long*>(ab + (size_t)p * 4 * tp * PB) : 0;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float d = scale_of(scw[s], b);
          const long wv = reinterpret_cast<const long*>(my)[(16 * s + n) * 4 + g];
          const i32x4 C0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(a[0], wv, z, 0, 0, 0);
          const i32x4 C1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(a[1], wv, z, 0, 0, 0);
          const i32x4 C2 = __builtin_amdgcn_mfma_i32_16x16x32_i8(a[2], wv, z, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int l = C0[i] + (C1[i] << 8);
            const float bf = __builtin_fmaf((float)C2[i], 65536.0f, (float)l);
            acc[s][i] = __builtin_fmaf(bf, d * xs[i], acc[s][i]);
            asm volatile("" : "+v"(acc[s][i]));
          }
        }
      }
      SLQ_COMPILER_FENCE();
    }
  }
}

// Epilogue of token j for the 64 rows of group rg; lane = row, a = sum over K.
// pre: the token's RMSNorm factor (STORE, SWIGLU) or its residual entry h
// (RESID); nw_row: next RMSNorm weight of the row (RESID).
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
    const float up = __shfl(v, (lane + 32) & 63, 64);
    const float m = (v / (1.0f + expf(-v))) * up;
    if (out.y && lane < 32) out.y[(size_t)j * out.y_tstride + rg * 32 + lane] = m;
    put_digits(out.next, out.next_qt, j, rg, m, lane < 32);
  } else {  // EPI_RESID
    const float hn = rv ? pre + a : 0.0f;
    resid_tail_w(j, rg, (int)W.rows, hn, nw_row, out.y, out.y_tstride, out.next_qt, out.next, out.ssq_out, W.nrg());
  }
}

// What token j's epilogue reads besides the sum: its RMSNorm factor (STORE,
// SWIGLU) or residual entry (RESID).  Loads for all tokens are issued before
// the first is used.
template <int EPI>
__device__ __forceinline__ void epi_inputs(const Packed& W, const GemvOut& out, const NormIn& nin, int rg, int T,
                                           float (&pre)[MX_SLOTS]) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)rg * RG + lane;
  if constexpr (EPI == EPI_RESID) {
#pragma unroll
    for (int j = 0; j < MX_SLOTS; ++j) pre[j] = (j < T && row < W.rows) ? out.y[(size_t)j * out.y_tstride + row] : 0.0f;
  } else if (!nin.ssq) {
#pragma unroll
    for (int j = 0; j < MX_SLOTS; ++j) pre[j] = 1.0f;
  } else {
    // n_part <= 128 partial sums per token: two loads per lane
    float a0[MX_SLOTS], a1[MX_SLOTS];
#pragma unroll
    for (int j = 0; j < MX_SLOTS; ++j) {
      const float* s = nin.ssq + (size_t)j * nin.n_part;
      a0[j] = (j < T && lane < nin.n_part) ? s[lane] : 0.0f;
      a1[j] = (j < T && lane + 64 < nin.n_part) ? s[lane + 64] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < MX_SLOTS; ++j) {
      const float a = wave_sum(a0[j] + a1[j]);
      pre[j] = 1.0f / sqrtf(a * nin.inv_n + nin.eps);
    }
  }
}

// Units' partials of tokens j0 .. j0+NJ-1 added in the single-token GEMV's
// order (per split its waves in wave order, then the splits in split order,
// from 0.0f when there are several).  NJ * U_MAX loads in flight together.
template <int U_MAX, int NJ>
__device__ __forceinline__ void sum_units(const float* all, int ksplit, int wsplit, int T, int j0, float (&v)[NJ]) {
  const int lane = threadIdx.x & 63;
  const int units = ksplit * wsplit;
  float pv[NJ][U_MAX];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
    for (int k = 0; k < U_MAX; ++k)
      pv[jj][k] = (k < units && j0 + jj < T)
                      ? __hip_atomic_load(all + ((size_t)k * T + j0 + jj) * RG + lane, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT)
                      : 0.0f;
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) {
    float tot = 0.0f, s = pv[jj][0];
    int wj = 0;
#pragma unroll
    for (int k = 1; k < U_MAX; ++k) {
      if (k < units) {
        wj = wj + 1 == wsplit ? 0 : wj + 1;
        if (wj == 0) {   // unit k starts the next split
          tot = tot + s;
          s = pv[jj][k];
        } else {
          s += pv[jj][k];
        }
      }
    }
    v[jj] = ksplit > 1 ? tot + s : s;
  }
}

template <int QT, int EPI, int U_MAX, int NJ>
__device__ __forceinline__ void finish_units(const Packed& W, const GemvOut& out, const float* all, int ksplit,
                                             int wsplit, int T, int rg, const float (&pre)[MX_SLOTS],
                                             float nw_row) {
#pragma unroll
  for (int j0 = 0; j0 < MX_SLOTS; j0 += NJ) {
    if (j0 < T) {
      float v[NJ];
      sum_units<U_MAX, NJ>(all, ksplit, wsplit, T, j0, v);
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj)
        if (j0 + jj < T) gemm_epi<QT, EPI>(W, out, rg, j0 + jj, v[jj], pre[j0 + jj], nw_row);
    }
  }
}

template <int QT, int EPI>
__global__ __launch_bounds__(GEMM_R * 64) void k_gemm(Packed W, Act x, NormIn nin, GemvOut out, int ksplit,
                                                       int wsplit, int T, int tp) {
  constexpr int TBY = tile_bytes(QT);
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int ACTB = gemm_act_tile(QT, tp);
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int R = blockDim.x >> 6;
  const int units = ksplit * wsplit;
  const int u = blockIdx.x % units, grp = blockIdx.x / units;
  const int ks_i = u / wsplit, w_j = u % wsplit;
  const int nrg = W.nrg();
  const int rg = grp * R + wave;
  const bool live = rg < nrg;
  const int nblk = W.nblk(), ntiles = W.ntiles(), full = nblk / TB;
  // the single-token GEMV's tile range of unit (ks_i, w_j)
  const int w0 = ntiles * ks_i / ksplit, w1 = ntiles * (ks_i + 1) / ksplit;
  const int t0 = w0 + (w1 - w0) * w_j / wsplit, t1 = w0 + (w1 - w0) * (w_j + 1) / wsplit;
  const uint8_t* base = W.w + (size_t)(live ? rg : 0) * rg_bytes(QT, W.cols);
  uint8_t* act0 = lds;
  uint8_t* act1 = lds + ACTB;
  uint8_t* my = lds + 2 * ACTB + (size_t)wave * GEMM_STAGE;
  auto nb_of = [&](int t) { return t < full ? TB : nblk - full * TB; };

  float acc[4][4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[s][i] = 0.0f;

  if (t0 < t1) {
    TileRegs<QT> A, B;
    stage_act<QT>(x, t0 * TB, nb_of(t0), tp, act0, wave, R);
    if (live) load_tile<QT>(base + (size_t)t0 * TBY, lane, nb_of(t0), A);
    for (int t = t0; t < t1; t += 2) {
      // tile t: weights in A, digits in act0; tile t+1 is requested meanwhile
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (t + 1 < t1) {
        stage_act<QT>(x, (t + 1) * TB, nb_of(t + 1), tp, act1, wave, R);
        if (live) load_tile<QT>(base + (size_t)(t + 1) * TBY, lane, nb_of(t + 1), B);
      }
      if (live) tile_mma<QT>(A, nb_of(t), act0, T, tp, my, acc);
      if (t + 1 >= t1) break;
      // tile t+1: weights in B, digits in act1
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (t + 2 < t1) {
        stage_act<QT>(x, (t + 2) * TB, nb_of(t + 2), tp, act0, wave, R);
        if (live) load_tile<QT>(base + (size_t)(t + 2) * TBY, lane, nb_of(t + 2), A);
      }
      if (live) tile_mma<QT>(B, nb_of(t + 1), act1, T, tp, my, acc);
    }
  }
  __syncthreads();   // every wave is done with the digit buffers
  if (!live) return;
  const int64_t erow = (int64_t)rg * RG + lane;
  const float nw_row = (EPI == EPI_RESID && erow < W.rows) ? out.norm_w[erow] : 0.0f;
  const int g = lane >> 4, n = lane & 15;

  if (units == 1) {
    // the whole sum is here: to lane = row through the wave's own 4 KB
    float pre[MX_SLOTS];
    epi_inputs<EPI>(W, out, nin, rg, T, pre);
    float* red = reinterpret_cast<float*>(lds + (size_t)wave * 4096);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[(4 * g + i) * RG + 16 * s + n] = acc[s][i];
    SLQ_COMPILER_FENCE();
#pragma unroll
    for (int j = 0; j < MX_SLOTS; ++j)
      if (j < T) gemm_epi<QT, EPI>(W, out, rg, j, red[j * RG + lane], pre[j], nw_row);
    return;
  }

  // publish this unit's partial sums [rg][u][token][row], take a ticket
  float* mine = out.part + ((size_t)rg * units + u) * T * RG;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * g + i < T)
        __hip_atomic_store(mine + (size_t)(4 * g + i) * RG + 16 * s + n, acc[s][i], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  unsigned ticket = 0;
  if (lane == 0) ticket = __hip_atomic_fetch_add(out.cnt + rg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  ticket = __shfl(ticket, 0, 64);
  if (ticket != (unsigned)(units - 1)) return;
  float pre[MX_SLOTS];
  epi_inputs<EPI>(W, out, nin, rg, T, pre);
  const float* all = out.part + (size_t)rg * units * T * RG;
  if (units <= 16) finish_units<QT, EPI, 16, 4>(W, out, all, ksplit, wsplit, T, rg, pre, nw_row);
  else if (units <= 32) finish_units<QT, EPI, 32, 2>(W, out, all, ksplit, wsplit, T, rg, pre, nw_row);
  else finish_units<QT, EPI, GEMM_MAX_UNITS, 1>(W, out, all, ksplit, wsplit, T, rg, pre, nw_row);
  if (lane == 0) __hip_atomic_store(out.cnt + rg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int QT, int EPI>
hipError_t gemm_inst(const Packed& W, int T, Act x, NormIn nin, GemvOut out, int ksplit, int waves,
                     hipStream_t s) {
  if (T < 1 || T > MX_SLOTS || ksplit < 1 || waves < 1 || waves > 8 || ksplit * waves > GEMM_MAX_UNITS)
    return hipErrorInvalidValue;
  const int units = ksplit * waves;
  if (units > 1 && (!out.part || !out.cnt)) return hipErrorInvalidValue;
  const int tp = (T + 3) & ~3;
  const int ngrp = (W.nrg() + GEMM_R - 1) / GEMM_R;
  k_gemm<QT, EPI><<<dim3((unsigned)(ngrp * units)), dim3(GEMM_R * 64), gemm_lds_bytes(QT, tp), s>>>(
      W, x, nin, out, ksplit, waves, T, tp);
  return hipGetLastError();
}

}  // namespace slq
