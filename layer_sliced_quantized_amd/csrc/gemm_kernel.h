// Batched (2..16 tokens) Q4_0 / Q8_0 matrix products on the int8 matrix cores.
//
// Same work split as the streaming GEMV (64-row groups, K tiles spread over
// waves and split-K workgroups, waves summed in LDS in wave order, splits summed
// in split order) and the same fp32 operations per (row, token, block), so a
// token's result is bitwise the one the single-token GEMV gives.  Only the
// exact integer block sums come from a different unit:
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
// A wave's 64 rows arrive one row per lane (the GEMV's packed layout); each
// block is staged through the wave's own LDS area so that lane (g, n) can read
// row 16 s + n of sub-tile s.
#pragma once
#include "gemv_kernel.h"

namespace slq {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int GEMM_LDS_PER_WAVE = 3072;   // 2 KB staged codes + 1 KB tile scales

template <int QT>
struct MxRegs;
template <>
struct MxRegs<QT_Q4> {
  i32x4 a[3];
  float s[4];
};
template <>
struct MxRegs<QT_Q8> {
  long a[3];
  float s[4];
};

// Digit operands of block blk for this lane's token slot (lane & 15) and
// k-group (lane >> 4), and the scales of the tokens this lane's outputs hold
// (4 (lane >> 4) + i).  Slots >= T read as zero.
template <int QT>
__device__ __forceinline__ void load_mx(const Act& x, int blk, int T, MxRegs<QT>& r) {
  const int lane = threadIdx.x & 63;
  const int m = lane & 15, g = lane >> 4;
  if constexpr (QT == QT_Q4) {
    const i32x4* X = reinterpret_cast<const i32x4*>(x.xd) + (size_t)blk * 12 * MX_SLOTS + lane;
#pragma unroll
    for (int p = 0; p < 3; ++p) r.a[p] = m < T ? X[p * 4 * MX_SLOTS] : i32x4{0, 0, 0, 0};
  } else {
    const long* X = reinterpret_cast<const long*>(x.xd) + (size_t)blk * 12 * MX_SLOTS + lane;
#pragma unroll
    for (int p = 0; p < 3; ++p) r.a[p] = m < T ? X[p * 4 * MX_SLOTS] : 0;
  }
  const float4 s4 = reinterpret_cast<const float4*>(x.xs)[(size_t)blk * (MX_SLOTS / 4) + g];
  r.s[0] = 4 * g + 0 < T ? s4.x : 0.0f;
  r.s[1] = 4 * g + 1 < T ? s4.y : 0.0f;
  r.s[2] = 4 * g + 2 < T ? s4.z : 0.0f;
  r.s[3] = 4 * g + 3 < T ? s4.w : 0.0f;
}

// Four two's-complement nibbles in the low halves of the bytes of t (high
// halves zero) -> four int8: ((t ^ 8) + 0x78) ^ 0x80 per byte, no carries.
__device__ __forceinline__ uint32_t sext_nibbles(uint32_t t) {
  return ((t ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u;
}

#define SLQ_COMPILER_FENCE() asm volatile("" ::: "memory")
#define SLQ_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// All blocks of one tile: stage, multiply, and fold into acc[s][i] (row
// 16 s + (lane & 15), token 4 (lane >> 4) + i).  `cur` holds the operands of
// block kb on entry and of the block after the tile on exit.
template <int QT>
__device__ __forceinline__ void tile_mma(const TileRegs<QT>& r, int nb, int kb, int kend, const Act& x, int T,
                                         uint8_t* my, MxRegs<QT>& cur, float (&acc)[4][4]) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
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
      MxRegs<QT> nxt;
      const bool more = kb + b + 1 < kend;
      if (more) load_mx<QT>(x, kb + b + 1, T, nxt);
      SLQ_COMPILER_FENCE();
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
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float d = scale_of(scw[s], b);
        const i32x4 z = {0, 0, 0, 0};
        i32x4 C0, C1, C2;
        if constexpr (QT == QT_Q4) {
          const u32x4 wu = reinterpret_cast<const u32x4*>(my)[(g & 1) * RG + 16 * s + n];
          const i32x4 wv = {(int)wu.x, (int)wu.y, (int)wu.z, (int)wu.w};
          C0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(cur.a[0], wv, z, 0, 0, 0);
          C1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(cur.a[1], wv, z, 0, 0, 0);
          C2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(cur.a[2], wv, z, 0, 0, 0);
        } else {
          const long wv = reinterpret_cast<const long*>(my)[(16 * s + n) * 4 + g];
          C0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(cur.a[0], wv, z, 0, 0, 0);
          C1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(cur.a[1], wv, z, 0, 0, 0);
          C2 = __builtin_amdgcn_mfma_i32_16x16x32_i8(cur.a[2], wv, z, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float bf;
          if constexpr (QT == QT_Q4) {
            const int D = C0[i] + ((C1[i] + (C2[i] << 8)) << 8);
            bf = (float)D;
          } else {
            const int l = C0[i] + (C1[i] << 8);
            bf = __builtin_fmaf((float)C2[i], 65536.0f, (float)l);
          }
          const float dsx = d * cur.s[i];
          acc[s][i] = __builtin_fmaf(bf, dsx, acc[s][i]);
          // keep the fold here: otherwise the compiler sinks every block's
          // fold to the end of the tile and keeps all MFMA results live
          asm volatile("" : "+v"(acc[s][i]));
        }
      }
      SLQ_COMPILER_FENCE();
      if (more) cur = nxt;
    }
  }
}

// Epilogue of token j for the 64 rows of group rg; lane = row, a = sum over K.
template <int QT, int EPI>
__device__ __forceinline__ void gemm_epi(const Packed& W, const GemvOut& out, const NormIn& nin, int rg, int j,
                                         float a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)rg * RG + lane;
  const bool rv = row < W.rows;
  if constexpr (EPI == EPI_STORE) {
    const float rn = rnorm_from(nin, j);
    if (rv) out.y[(size_t)j * out.y_tstride + row] = a * rn;
  } else if constexpr (EPI == EPI_SWIGLU) {
    // lanes 0..31: gate rows, lanes 32..63: the matching up rows
    const float rn = rnorm_from(nin, j);
    const float v = a * rn;
    const float up = __shfl(v, (lane + 32) & 63, 64);
    const float m = (v / (1.0f + expf(-v))) * up;
    if (out.y && lane < 32) out.y[(size_t)j * out.y_tstride + rg * 32 + lane] = m;
    put_digits(out.next, out.next_qt, j, rg, m, lane < 32);
  } else {  // EPI_RESID
    const float hn = rv ? out.y[(size_t)j * out.y_tstride + row] + a : 0.0f;
    resid_tail(j, rg, (int)W.rows, hn, out.y, out.y_tstride, out.norm_w, out.next_qt, out.next, out.ssq_out,
               W.nrg());
  }
}

template <int QT, int EPI>
__global__ __launch_bounds__(512) void k_gemm(Packed W, Act x, NormIn nin, GemvOut out, int ksplit, int T) {
  constexpr int TBY = tile_bytes(QT);
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int nw = blockDim.x >> 6;
  const int rg = blockIdx.x / ksplit, ks = blockIdx.x % ksplit;
  const int nblk = W.nblk(), ntiles = W.ntiles(), full = nblk / TB;
  const int w0 = ntiles * ks / ksplit, w1 = ntiles * (ks + 1) / ksplit;
  const int t0 = __builtin_amdgcn_readfirstlane(w0 + (w1 - w0) * wave / nw);
  const int t1 = __builtin_amdgcn_readfirstlane(w0 + (w1 - w0) * (wave + 1) / nw);
  const int kend = t1 * TB < nblk ? t1 * TB : nblk;
  const uint8_t* base = W.w + (size_t)rg * rg_bytes(QT, W.cols);
  uint8_t* my = lds + (size_t)wave * GEMM_LDS_PER_WAVE;

  float acc[4][4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[s][i] = 0.0f;

  MxRegs<QT> cur;
  if (t0 < t1) load_mx<QT>(x, t0 * TB, T, cur);
  const int te = t1 < full ? t1 : full;
  if (t0 < te) {
    TileRegs<QT> A, B;
    load_tile<QT>(base + (size_t)t0 * TBY, lane, TB, A);
    for (int t = t0; t < te; t += 2) {
      if (t + 1 < te) load_tile<QT>(base + (size_t)(t + 1) * TBY, lane, TB, B);
      tile_mma<QT>(A, TB, t * TB, kend, x, T, my, cur, acc);
      if (t + 1 < te) {
        if (t + 2 < te) load_tile<QT>(base + (size_t)(t + 2) * TBY, lane, TB, A);
        tile_mma<QT>(B, TB, (t + 1) * TB, kend, x, T, my, cur, acc);
      }
    }
  }
  if (t1 > full) {   // the ragged last tile, owned by the wave whose range ends there
    const int nb = nblk - full * TB;
    TileRegs<QT> A;
    load_tile<QT>(base + (size_t)full * TBY, lane, nb, A);
    tile_mma<QT>(A, nb, full * TB, kend, x, T, my, cur, acc);
  }

  // Waves meet in LDS, eight tokens at a time: red[wave][token - 8 ps][row].
  // Token j is finished by wave j % nw, which adds the waves in wave order.
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);
  const int g = lane >> 4, n = lane & 15;
  for (int ps = 0; ps * 8 < T; ++ps) {
    if ((g >> 1) == ps) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[((size_t)wave * 8 + 4 * (g & 1) + i) * RG + 16 * s + n] = acc[s][i];
    }
    __syncthreads();
    const int jend = T < 8 * ps + 8 ? T : 8 * ps + 8;
    for (int j = 8 * ps + wave; j < jend; j += nw) {
      const int jj = j - 8 * ps;
      float v = red[(size_t)jj * RG + lane];
      for (int w = 1; w < nw; ++w) v += red[((size_t)w * 8 + jj) * RG + lane];
      if (ksplit == 1) gemm_epi<QT, EPI>(W, out, nin, rg, j, v);
      else
        __hip_atomic_store(out.part + (((size_t)rg * ksplit + ks) * T + j) * RG + lane, v, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
  }

  if (ksplit > 1) {
    // Same exchange as the GEMV: partials move through agent-scope atomics,
    // every wave's stores are complete before the workgroup takes its ticket,
    // and the last split adds them in split order.
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
    for (int j = wave; j < T; j += nw) {
      float pv[16];
#pragma unroll
      for (int k2 = 0; k2 < 16; ++k2)
        pv[k2] = k2 < ksplit ? __hip_atomic_load(all + ((size_t)k2 * T + j) * RG + lane, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT)
                             : 0.0f;
      float sum = 0.0f;
#pragma unroll
      for (int k2 = 0; k2 < 16; ++k2)
        if (k2 < ksplit) sum += pv[k2];
      gemm_epi<QT, EPI>(W, out, nin, rg, j, sum);
    }
    if (threadIdx.x == 0) __hip_atomic_store(out.cnt + rg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int QT, int EPI>
hipError_t gemm_inst(const Packed& W, int T, Act x, NormIn nin, GemvOut out, int ksplit, int waves,
                     hipStream_t s) {
  if (T < 1 || T > MX_SLOTS || ksplit > 16 || waves > 8) return hipErrorInvalidValue;
  dim3 grid((unsigned)(W.nrg() * ksplit)), block(64 * waves);
  k_gemm<QT, EPI><<<grid, block, (size_t)waves * GEMM_LDS_PER_WAVE, s>>>(W, x, nin, out, ksplit, T);
  return hipGetLastError();
}

}  // namespace slq
