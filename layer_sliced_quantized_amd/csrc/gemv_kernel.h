// Streaming GEMV kernel template (included by the per-format instantiation units).
//
// Each lane owns one output row of a 64-row group and streams whole blocks of
// that row with one 128-bit load per block; the activation is wave-uniform and
// comes from scalar registers as integer digits, so every block's dot product
// is an exact int32 sum (v_dot8c_i32_i4 for Q4_0, v_dot4c_i32_i8 for Q8_0) and
// only the per-block scales are applied in fp32.  The waves of a workgroup split
// K and are summed in LDS in wave order; every token of a batched call goes
// through the same operations as a batch-1 call.
#pragma once
#include "dev.h"

namespace slq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int QT>
struct TileRegs {
  static constexpr int NH = QT == QT_Q4 ? 1 : 2;
  u32x4 c[TB * NH];
  u32x4 sc;
};

template <int QT>
__device__ __forceinline__ void load_tile(const uint8_t* tile, int lane, int nb, TileRegs<QT>& r) {
  constexpr int NH = TileRegs<QT>::NH;
  const u32x4* cp = reinterpret_cast<const u32x4*>(tile) + lane;
#pragma unroll
  for (int b = 0; b < TB * NH; ++b)
    if (b < nb * NH) r.c[b] = __builtin_nontemporal_load(cp + b * RG);
  r.sc = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(tile + (size_t)nb * NH * RG * 16) + lane);
}

// One 16-byte weight load: nontemporal (streamed past the caches, the usual
// case: every weight is read once) or, NT = false, an ordinary load that L2
// keeps for other waves reading the same tile soon after.
template <bool NT>
__device__ __forceinline__ u32x4 ld_w(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// A tile's weights into registers with always TB * NH + 1 loads, whatever the
// tile: the codes of a ragged tile (nb < TB) repeat its last block, and nb = 0
// (no tile) reads the first 16 bytes at tile from every lane.  Every path thus
// issues the same loads, which keeps the compiler's own waits on these
// registers (and the explicit ring waits) exact.
template <int QT, bool NT = true>
__device__ __forceinline__ void load_tile_fixed(const uint8_t* tile, int lane, int nb, TileRegs<QT>& r) {
  constexpr int NH = TileRegs<QT>::NH;
  const int nc = nb * NH;
  const u32x4* cp = reinterpret_cast<const u32x4*>(tile) + (nb ? lane : 0);
#pragma unroll
  for (int b = 0; b < TB * NH; ++b) r.c[b] = ld_w<NT>(cp + (nb ? (b < nc ? b : nc - 1) : 0) * RG);
  r.sc = ld_w<NT>(nb ? reinterpret_cast<const u32x4*>(tile + (size_t)nc * RG * 16) + lane : cp);
}

// One block's codes of a tile (r.c[b * NH + h], h < NH) with always NH loads,
// and the tile's scales (r.sc) with always one, choosing their sources as
// load_tile_fixed does; together they issue its loads one block at a time.
template <int QT, bool NT = true>
__device__ __forceinline__ void load_block_fixed(const uint8_t* tile, int lane, int nb, int b, TileRegs<QT>& r) {
  constexpr int NH = TileRegs<QT>::NH;
  const int nc = nb * NH;
  const u32x4* cp = reinterpret_cast<const u32x4*>(tile) + (nb ? lane : 0);
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int i = b * NH + h;
    r.c[i] = ld_w<NT>(cp + (nb ? (i < nc ? i : nc - 1) : 0) * RG);
  }
}
template <bool NT = true>
__device__ __forceinline__ u32x4 load_scales_fixed(const uint8_t* tile, int lane, int nb, int nh) {
  const u32x4* cp = reinterpret_cast<const u32x4*>(tile) + (nb ? lane : 0);
  return ld_w<NT>(nb ? reinterpret_cast<const u32x4*>(tile + (size_t)nb * nh * RG * 16) + lane : cp);
}

__device__ __forceinline__ float scale_of(const u32x4& sc, int b) {
  const uint32_t w = b < 2 ? sc.x : b < 4 ? sc.y : b < 6 ? sc.z : sc.w;
  const unsigned short hb = (unsigned short)((b & 1) ? (w >> 16) : (w & 0xffff));
  return __half2float(__ushort_as_half(hb));
}

// Digits and scale of one activation block of one token (wave-uniform: SGPRs).
struct XRegs {
  int32_t d[XW];
  float s;
};

__device__ __forceinline__ void load_x(const Act& x, int j, int blk, XRegs& r) {
  const int32_t* X = x.xd + ((size_t)j * x.nblk + blk) * XW;
#pragma unroll
  for (int i = 0; i < XW; ++i) r.d[i] = X[i];
  r.s = x.xs[(size_t)j * x.nblk + blk];
}

// Exact integer dot product of one block's codes with one token's digits, as
// fp32.  The digit sums are combined Horner-style inside the accumulator:
// ((a2 * 16) + a1) * 16 + a0 is a2*256 + a1*16 + a0 exactly.
template <int QT>
__device__ __forceinline__ float block_dot(const TileRegs<QT>& r, int b, const XRegs& X) {
  if constexpr (QT == QT_Q4) {
    const u32x4 c = r.c[b];
    int h = __builtin_amdgcn_sdot8((int)c.x, X.d[20], 0, false);
    h = __builtin_amdgcn_sdot8((int)c.y, X.d[21], h, false);
    h = __builtin_amdgcn_sdot8((int)c.z, X.d[22], h, false);
    h = __builtin_amdgcn_sdot8((int)c.w, X.d[23], h, false);
    int l = __builtin_amdgcn_sdot8((int)c.x, X.d[8], 0, false);
    l = __builtin_amdgcn_sdot8((int)c.y, X.d[9], l, false);
    l = __builtin_amdgcn_sdot8((int)c.z, X.d[10], l, false);
    l = __builtin_amdgcn_sdot8((int)c.w, X.d[11], l, false);
    h *= 16;
    l *= 16;
    h = __builtin_amdgcn_sdot8((int)c.x, X.d[16], h, false);
    h = __builtin_amdgcn_sdot8((int)c.y, X.d[17], h, false);
    h = __builtin_amdgcn_sdot8((int)c.z, X.d[18], h, false);
    h = __builtin_amdgcn_sdot8((int)c.w, X.d[19], h, false);
    l = __builtin_amdgcn_sdot8((int)c.x, X.d[4], l, false);
    l = __builtin_amdgcn_sdot8((int)c.y, X.d[5], l, false);
    l = __builtin_amdgcn_sdot8((int)c.z, X.d[6], l, false);
    l = __builtin_amdgcn_sdot8((int)c.w, X.d[7], l, false);
    h *= 16;
    l *= 16;
    h = __builtin_amdgcn_sdot8((int)c.x, X.d[12], h, false);
    h = __builtin_amdgcn_sdot8((int)c.y, X.d[13], h, false);
    h = __builtin_amdgcn_sdot8((int)c.z, X.d[14], h, false);
    h = __builtin_amdgcn_sdot8((int)c.w, X.d[15], h, false);
    l = __builtin_amdgcn_sdot8((int)c.x, X.d[0], l, false);
    l = __builtin_amdgcn_sdot8((int)c.y, X.d[1], l, false);
    l = __builtin_amdgcn_sdot8((int)c.z, X.d[2], l, false);
    l = __builtin_amdgcn_sdot8((int)c.w, X.d[3], l, false);
    return __builtin_fmaf((float)h, 4096.0f, (float)l);
  } else {
    const u32x4 c0 = r.c[2 * b], c1 = r.c[2 * b + 1];
    int a = 0, l;
    // a2
    a = __builtin_amdgcn_sdot4((int)c0.x, X.d[16], a, false);
    a = __builtin_amdgcn_sdot4((int)c0.y, X.d[17], a, false);
    a = __builtin_amdgcn_sdot4((int)c0.z, X.d[18], a, false);
    a = __builtin_amdgcn_sdot4((int)c0.w, X.d[19], a, false);
    a = __builtin_amdgcn_sdot4((int)c1.x, X.d[20], a, false);
    a = __builtin_amdgcn_sdot4((int)c1.y, X.d[21], a, false);
    a = __builtin_amdgcn_sdot4((int)c1.z, X.d[22], a, false);
    a = __builtin_amdgcn_sdot4((int)c1.w, X.d[23], a, false);
    // a1 * 256 + a0
    l = __builtin_amdgcn_sdot4((int)c0.x, X.d[8], 0, false);
    l = __builtin_amdgcn_sdot4((int)c0.y, X.d[9], l, false);
    l = __builtin_amdgcn_sdot4((int)c0.z, X.d[10], l, false);
    l = __builtin_amdgcn_sdot4((int)c0.w, X.d[11], l, false);
    l = __builtin_amdgcn_sdot4((int)c1.x, X.d[12], l, false);
    l = __builtin_amdgcn_sdot4((int)c1.y, X.d[13], l, false);
    l = __builtin_amdgcn_sdot4((int)c1.z, X.d[14], l, false);
    l = __builtin_amdgcn_sdot4((int)c1.w, X.d[15], l, false);
    l *= 256;
    l = __builtin_amdgcn_sdot4((int)c0.x, X.d[0], l, false);
    l = __builtin_amdgcn_sdot4((int)c0.y, X.d[1], l, false);
    l = __builtin_amdgcn_sdot4((int)c0.z, X.d[2], l, false);
    l = __builtin_amdgcn_sdot4((int)c0.w, X.d[3], l, false);
    l = __builtin_amdgcn_sdot4((int)c1.x, X.d[4], l, false);
    l = __builtin_amdgcn_sdot4((int)c1.y, X.d[5], l, false);
    l = __builtin_amdgcn_sdot4((int)c1.z, X.d[6], l, false);
    l = __builtin_amdgcn_sdot4((int)c1.w, X.d[7], l, false);
    return __builtin_fmaf((float)a, 65536.0f, (float)l);
  }
}

// All blocks of one tile for T tokens.  The digits of the next (block, token)
// are requested before the current one is used, so the scalar loads overlap
// the dot products.
template <int QT, int T>
__device__ __forceinline__ void tile_math(const TileRegs<QT>& r, int nb, int kb, const Act& x,
                                          float (&acc)[T]) {
  XRegs cur, nxt;
  load_x(x, 0, kb, cur);
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    if (b < nb) {
      const float d = scale_of(r.sc, b);
#pragma unroll
      for (int j = 0; j < T; ++j) {
        const bool more = (j + 1 < T) || (b + 1 < nb);
        const float dsx = d * cur.s;
        if (more) load_x(x, j + 1 < T ? j + 1 : 0, j + 1 < T ? kb + b : kb + b + 1, nxt);
        const float bf = block_dot<QT>(r, b, cur);
        acc[j] = __builtin_fmaf(bf, dsx, acc[j]);
        if (more) cur = nxt;
      }
    }
  }
}

// Tile range [t0, t1) of wave `wave` of `nw` in split ks of ksplit (uniform:
// readfirstlane keeps the loop and the digit addresses in scalar registers).
__device__ __forceinline__ void wave_tiles(int ntiles, int ks, int ksplit, int wave, int nw, int& t0, int& t1) {
  const int w0 = ntiles * ks / ksplit, w1 = ntiles * (ks + 1) / ksplit;
  t0 = __builtin_amdgcn_readfirstlane(w0 + (w1 - w0) * wave / nw);
  t1 = __builtin_amdgcn_readfirstlane(w0 + (w1 - w0) * (wave + 1) / nw);
}

// The waves of a workgroup meet in LDS, summed in wave order; wave 0 ends
// with the workgroup's sums.
template <int T>
__device__ __forceinline__ void reduce_waves(float (&acc)[T], float (*red)[RG], int wave, int nw, int lane) {
#pragma unroll
  for (int j = 0; j < T; ++j) {
    if (nw > 1) {
      red[wave][lane] = acc[j];
      __syncthreads();
      if (wave == 0) {
        float s = red[0][lane];
        for (int w = 1; w < nw; ++w) s += red[w][lane];
        acc[j] = s;
      }
      __syncthreads();
    }
  }
}

// Split-K exchange, called by wave 0 of every split of row group rg when
// ksplit > 1.  Each split publishes its sums and takes a ticket; the last
// split of the row group adds all of them in split order (so the result does
// not depend on arrival order), resets the ticket and returns true; the
// others return false.  Partials and the ticket move only through
// agent-scope atomic accesses (global stores / loads with sc1 on gfx950,
// which write through to and read from the point where all XCDs agree);
// waiting for the stores to complete (vmcnt 0) before the ticket is taken
// orders them before it, so the split that sees the last ticket reads every
// partial in full.  No cache-wide write-back or invalidate is needed.
template <int T>
__device__ __forceinline__ bool split_exchange(float (&acc)[T], const GemvOut& out, int rg, int ks, int ksplit,
                                               int lane) {
  float* my = out.part + ((size_t)rg * ksplit + ks) * T * RG;
#pragma unroll
  for (int j = 0; j < T; ++j)
    __hip_atomic_store(my + j * RG + lane, acc[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  unsigned ticket = 0;
  if (lane == 0) ticket = __hip_atomic_fetch_add(out.cnt + rg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  ticket = __shfl(ticket, 0, 64);
  if (ticket != (unsigned)(ksplit - 1)) return false;
  const float* all = out.part + (size_t)rg * ksplit * T * RG;
#pragma unroll
  for (int j = 0; j < T; ++j) {
    // all loads in flight before the first add; the adds run in split order
    float pv[16];
#pragma unroll
    for (int k2 = 0; k2 < 16; ++k2)
      pv[k2] = k2 < ksplit ? __hip_atomic_load(all + ((size_t)k2 * T + j) * RG + lane, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)
                           : 0.0f;
    float s = 0.0f;
#pragma unroll
    for (int k2 = 0; k2 < 16; ++k2)
      if (k2 < ksplit) s += pv[k2];
    acc[j] = s;
  }
  if (lane == 0) __hip_atomic_store(out.cnt + rg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// Epilogue of row group rg (wave 0, whole K summed): store y, or the SwiGLU
// of lane pairs (row, row + 32) and the digits of the product, or the
// residual update with the next RMSNorm's statistics and digits.  COH: the
// results are read by later workgroups of the same kernel (coherent stores,
// and the residual read coherently).
template <int QT, int T, int EPI, bool COH>
__device__ __forceinline__ void gemv_epilogue(const float (&acc)[T], const float (&rn)[T], const Packed& W,
                                              const GemvOut& out, int rg, int lane) {
  const int64_t row = (int64_t)rg * RG + lane;
  const bool rv = row < W.rows;
#pragma unroll
  for (int j = 0; j < T; ++j) {
    if constexpr (EPI == EPI_STORE) {
      if (rv) st_<COH>(out.y + (size_t)j * out.y_tstride + row, acc[j] * rn[j]);
    } else if constexpr (EPI == EPI_SWIGLU) {
      // lanes 0..31: gate rows, lanes 32..63: the matching up rows
      const float v = acc[j] * rn[j];
      const float up = xor_lane<32>(v);   // row lane ^ 32
      const float m = (v / (1.0f + expf(-v))) * up;
      if (out.y && lane < 32) st_<COH>(out.y + (size_t)j * out.y_tstride + rg * 32 + lane, m);
      put_digits<COH>(out.next, out.next_qt, j, rg, m, lane < 32);
    } else {  // EPI_RESID, whole K in this workgroup
      const float hn = rv ? ld_<COH>(out.y + (size_t)j * out.y_tstride + row) + acc[j] : 0.0f;
      resid_tail<COH>(j, rg, (int)W.rows, hn, out.y, out.y_tstride, out.norm_w, out.next_qt, out.next,
                      out.ssq_out, W.nrg());
    }
  }
}

template <int QT, int T, int EPI>
__global__ __launch_bounds__(512) void k_gemv(Packed W, Act x, NormIn nin, GemvOut out, int ksplit) {
  constexpr int TBY = tile_bytes(QT);
  __shared__ float red[8][RG];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int nw = blockDim.x >> 6;
  const int rg = blockIdx.x / ksplit, ks = blockIdx.x % ksplit;
  const int nblk = W.nblk(), ntiles = W.ntiles(), full = nblk / TB;
  int t0, t1;
  wave_tiles(ntiles, ks, ksplit, wave, nw, t0, t1);
  const uint8_t* base = W.w + (size_t)rg * rg_bytes(QT, W.cols);

  float acc[T];
#pragma unroll
  for (int j = 0; j < T; ++j) acc[j] = 0.0f;
  // RMSNorm factor of the input (STORE / SWIGLU): its partial sums are
  // requested now and summed after the main loop, so waiting for them does
  // not hold back wave 0's first weight loads
  RnRaw rr[T];
#pragma unroll
  for (int j = 0; j < T; ++j) rr[j] = (EPI != EPI_RESID && wave == 0) ? rnorm_fetch(nin, j) : RnRaw{0.0f, 0.0f};

  // full tiles, two register sets in turn so the next tile's loads overlap this tile's math
  const int te = t1 < full ? t1 : full;
  if (t0 < te) {
    TileRegs<QT> A, B;
    load_tile<QT>(base + (size_t)t0 * TBY, lane, TB, A);
    for (int t = t0; t < te; t += 2) {
      if (t + 1 < te) load_tile<QT>(base + (size_t)(t + 1) * TBY, lane, TB, B);
      tile_math<QT, T>(A, TB, t * TB, x, acc);
      if (t + 1 < te) {
        if (t + 2 < te) load_tile<QT>(base + (size_t)(t + 2) * TBY, lane, TB, A);
        tile_math<QT, T>(B, TB, (t + 1) * TB, x, acc);
      }
    }
  }
  // the ragged last tile (< 8 blocks), owned by whichever wave's range ends there
  if (t1 > full) {
    const int nb = nblk - full * TB;
    TileRegs<QT> A;
    load_tile<QT>(base + (size_t)full * TBY, lane, nb, A);
    tile_math<QT, T>(A, nb, full * TB, x, acc);
  }

  float rn[T];
#pragma unroll
  for (int j = 0; j < T; ++j) rn[j] = (EPI != EPI_RESID && wave == 0) ? rnorm_finish(rr[j], nin, j) : 1.0f;

  reduce_waves<T>(acc, red, wave, nw, lane);
  if (wave != 0) return;
  if (ksplit > 1 && !split_exchange<T>(acc, out, rg, ks, ksplit, lane)) return;
  gemv_epilogue<QT, T, EPI, false>(acc, rn, W, out, rg, lane);
}


template <int QT, int EPI>
hipError_t gemv_inst(const Packed& W, int T, Act x, NormIn nin, GemvOut out, int ksplit, int waves,
                     hipStream_t s) {
  dim3 grid((unsigned)(W.nrg() * ksplit)), block(64 * waves);
  switch (T) {
#define SLQ_T(n) case n: k_gemv<QT, n, EPI><<<grid, block, 0, s>>>(W, x, nin, out, ksplit); break;
    SLQ_T(1) SLQ_T(2) SLQ_T(3) SLQ_T(4) SLQ_T(5) SLQ_T(6) SLQ_T(7) SLQ_T(8)
    SLQ_T(9) SLQ_T(10) SLQ_T(11) SLQ_T(12) SLQ_T(13) SLQ_T(14) SLQ_T(15) SLQ_T(16)
#undef SLQ_T
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

#define SLQ_DECLARE_GEMV(QT, EPI) \
  extern template hipError_t gemv_inst<QT, EPI>(const Packed&, int, Act, NormIn, GemvOut, int, int, hipStream_t);
SLQ_DECLARE_GEMV(QT_Q4, EPI_STORE) SLQ_DECLARE_GEMV(QT_Q4, EPI_SWIGLU) SLQ_DECLARE_GEMV(QT_Q4, EPI_RESID)
SLQ_DECLARE_GEMV(QT_Q8, EPI_STORE) SLQ_DECLARE_GEMV(QT_Q8, EPI_SWIGLU) SLQ_DECLARE_GEMV(QT_Q8, EPI_RESID)
#undef SLQ_DECLARE_GEMV

}  // namespace slq
