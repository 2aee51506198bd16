// Device helpers shared by the kernels of libslq.
#pragma once
#include "slq.h"

namespace slq {

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Lane l ^ M's value, exchanged in the vector ALU (no LDS round trip): DPP
// quad permutes for M = 1 and 2; for M = 4 the row shifts by 4 (left where bit
// 2 of the lane is clear, right where it is set); a rotate by 8 within 16-lane
// rows for M = 8; gfx950's permlane16 / permlane32 swaps for M = 16 and 32.
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "xor partner");
  const int x = __float_as_int(v);
  if constexpr (M == 1) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xB1 /* quad_perm 1,0,3,2 */, 0xf, 0xf, false));
  if constexpr (M == 2) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x4E /* quad_perm 2,3,0,1 */, 0xf, 0xf, false));
  if constexpr (M == 4) {
    const int up = __builtin_amdgcn_update_dpp(0, x, 0x104 /* row_shl:4 */, 0xf, 0xf, false);
    const int dn = __builtin_amdgcn_update_dpp(0, x, 0x114 /* row_shr:4 */, 0xf, 0xf, false);
    return __int_as_float((threadIdx.x & 4) ? dn : up);
  }
  if constexpr (M == 8) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x128 /* row_ror:8 */, 0xf, 0xf, false));
  if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
    return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
  }
  if constexpr (M == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
  }
  return v;
}

// Butterfly reductions: every lane ends with the same value, and the value does
// not depend on the lane (each level adds commutative pairs).
__device__ __forceinline__ float wave_sum(float v) {
  v += xor_lane<32>(v);
  v += xor_lane<16>(v);
  v += xor_lane<8>(v);
  v += xor_lane<4>(v);
  v += xor_lane<2>(v);
  v += xor_lane<1>(v);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, xor_lane<32>(v));
  v = fmaxf(v, xor_lane<16>(v));
  v = fmaxf(v, xor_lane<8>(v));
  v = fmaxf(v, xor_lane<4>(v));
  v = fmaxf(v, xor_lane<2>(v));
  v = fmaxf(v, xor_lane<1>(v));
  return v;
}
// over each 32-lane half separately
__device__ __forceinline__ float half_max(float v) {
  v = fmaxf(v, xor_lane<16>(v));
  v = fmaxf(v, xor_lane<8>(v));
  v = fmaxf(v, xor_lane<4>(v));
  v = fmaxf(v, xor_lane<2>(v));
  v = fmaxf(v, xor_lane<1>(v));
  return v;
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }

// Stores and loads of values that workgroups of the same kernel hand to each
// other (COH = true): agent-scope relaxed atomics, which gfx950 issues as
// global stores / loads with the sc1 bit (written through to, and read from,
// the point where all XCDs see the same value).  With COH = false, plain
// accesses (the kernel boundary makes them visible).
template <bool COH, class V>
__device__ __forceinline__ void st_(V* p, V v) {
  if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
template <bool COH, class V>
__device__ __forceinline__ V ld_(const V* p) {
  if constexpr (COH) return __hip_atomic_load(const_cast<V*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}

// RMSNorm factor from a producer's partial sums of squares: one load per lane
// (all in flight together), then a butterfly sum, so every wave that calls
// this gets the same value.
__device__ __forceinline__ float rnorm_from(const NormIn& n, int t) {
  if (!n.ssq) return 1.0f;
  const int lane = threadIdx.x & 63;
  const float* s = n.ssq + (size_t)t * n.n_part;
  float a = 0.0f;
  for (int i = lane; i < n.n_part; i += 64) a += s[i];
  a = wave_sum(a);
  return 1.0f / sqrtf(a * n.inv_n + n.eps);
}

// rnorm_from in two steps, so that the loads go out early and the wave-wide
// sum is taken later: rnorm_fetch takes this lane's (at most two) partial
// sums, rnorm_finish adds them with rnorm_from's additions (bitwise the same
// value; more than 128 partials fall back to rnorm_from).  Every lane of the
// wave must call rnorm_finish.
struct RnRaw {
  float a, b;
};
template <bool COH = false>
__device__ __forceinline__ RnRaw rnorm_fetch(const NormIn& n, int t) {
  const int lane = threadIdx.x & 63;
  if (!n.ssq || n.n_part > 128) return {0.0f, 0.0f};
  const float* s = n.ssq + (size_t)t * n.n_part;
  return {lane < n.n_part ? ld_<COH>(s + lane) : 0.0f, lane + 64 < n.n_part ? ld_<COH>(s + lane + 64) : 0.0f};
}
__device__ __forceinline__ float rnorm_finish(const RnRaw& r, const NormIn& n, int t) {
  if (!n.ssq) return 1.0f;
  if (n.n_part > 128) return rnorm_from(n, t);
  const float a = wave_sum(r.a + r.b);
  return 1.0f / sqrtf(a * n.inv_n + n.eps);
}

// Integer form of one block of 32 activations held one per lane by a 32-lane
// half of the wave (element e = lane & 31):
//   s = max|x| / M,  x_int = rint(x / s)  (|x_int| <= M),  u = x_int + OFF
// with OFF = 0x888888 (Q4_0) or 0x808080 (Q8_0), so that the balanced digits
// are ((u >> 4d) & 15) - 8 (six base-16 digits) or ((u >> 8d) & 255) - 128
// (three base-256 digits).  Returns u and sets `scale` to s.  A block holding
// an infinity or NaN gets scale NaN (digits 0), so every product that reads
// it is NaN, as the exact sums would be; a block whose s underflows to zero
// (max|x| below ~1e-38) is flushed to zero.  Every lane of the wave must call
// this (cross-lane exchanges).
template <int QT>
__device__ __forceinline__ uint32_t quant_int(float v, float& scale) {
  const float M = QT == QT_Q4 ? M_Q4 : M_Q8;
  const int Mi = QT == QT_Q4 ? 7829367 : 8355711;
  const float a = fabsf(v);
  const float amax = half_max(a);                       // fmaxf skips NaN entries
  const unsigned long long bad = __ballot(!(a <= 3.402823466e38f));   // NaN or infinity
  const bool any_bad = (bad >> (threadIdx.x & 32)) & 0xffffffffull;
  const float s = amax / M;
  int xi = 0;
  if (!any_bad && s > 0.0f) xi = min(max((int)rintf(v / s), -Mi), Mi);
  scale = any_bad ? __builtin_nanf("") : (s > 0.0f ? s : 0.0f);
  return (uint32_t)(xi + (QT == QT_Q4 ? 0x888888 : 0x808080));
}

// Layout fmt 0, in the order the weight codes of format QT are packed:
//   Q4_0: nibble 2k of dword (d, m) <- digit d of element 4m+k, nibble 2k+1 <- of
//         element 4m+k+16  (byte j of a Q4_0 block holds weights j, j+16)
//   Q8_0: byte k of dword (d, m) <- digit d of element 4m+k
template <int QT, bool COH = false>
__device__ __forceinline__ void quant_block_half(float v, int32_t* xd, float* xs, bool write) {
  const int lane = threadIdx.x & 63;
  const int e = lane & 31;
  const int base = lane & 32;
  float sc;
  const uint32_t u = quant_int<QT>(v, sc);
  uint32_t word = 0;
  if (QT == QT_Q4) {
    const int d = (e >> 2) % 6, m = e & 3;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t ul = (uint32_t)__shfl((int)u, base + 4 * m + k, 64);
      const uint32_t uh = (uint32_t)__shfl((int)u, base + 4 * m + k + 16, 64);
      const uint32_t nl = ((ul >> (4 * d)) & 15u) ^ 8u;
      const uint32_t nh = ((uh >> (4 * d)) & 15u) ^ 8u;
      word |= (nl | (nh << 4)) << (8 * k);
    }
  } else {
    const int d = (e >> 3) % 3, m = e & 7;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t uk = (uint32_t)__shfl((int)u, base + 4 * m + k, 64);
      word |= (((uk >> (8 * d)) & 255u) ^ 0x80u) << (8 * k);
    }
  }
  if (write) {
    if (e < XW) st_<COH>(xd + e, (int32_t)word);
    if (e == 0) st_<COH>(xs, sc);
  }
}

// MFMA layout (see Act): the same x_int and scale as the lane-row layout.
template <int QT>
__device__ __forceinline__ void quant_block_mx(float v, const Act& a, int tok, int blk, bool write) {
  const int lane = threadIdx.x & 63;
  const int e = lane & 31;
  const int base = lane & 32;
  // token group tok / 16 has a record of its own per block; t is the slot in it
  int32_t* rec = a.mxd + ((size_t)(tok / MX_SLOTS) * a.nblk + blk) * (mx_block_bytes(QT) / 4);
  const int t = tok % MX_SLOTS;
  float sc;
  const uint32_t u = quant_int<QT>(v, sc);
  if (QT == QT_Q4) {
    // 48 dwords: chunk c = w >> 2 (p = c >> 2, g = c & 3), dword q = w & 3;
    // lane e makes dword e and, for e < 16, dword e + 32
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int w = e + 32 * r;
      const int c = (w >> 2) % 12, q = w & 3, p = c >> 2, g = c & 3;
      const int d = 2 * p + (g >> 1);
      uint32_t word = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t uk = (uint32_t)__shfl((int)u, base + 16 * (g & 1) + 4 * q + k, 64);
        int dig = (int)((uk >> (4 * d)) & 15u) - 8;
        if (g >= 2) dig *= 16;
        word |= ((uint32_t)dig & 255u) << (8 * k);
      }
      if (write && w < 48) rec[(c * MX_SLOTS + t) * 4 + q] = (int32_t)word;
    }
  } else {
    // 24 dwords: w = e < 24, chunk c = w >> 2 (p = c >> 1, h = c & 1), dword q = w & 3
    const int w = e % 24;
    const int c = w >> 2, q = w & 3, p = c >> 1, h = c & 1;
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t uk = (uint32_t)__shfl((int)u, base + 16 * h + 4 * q + k, 64);
      word |= (((uk >> (8 * p)) & 255u) ^ 0x80u) << (8 * k);
    }
    if (write && e < 24) rec[(c * MX_SLOTS + t) * 4 + q] = (int32_t)word;
  }
  if (write && e == 0) reinterpret_cast<float*>(rec + mx_scale_off(QT) / 4)[t] = sc;
}

// Digits of block blk of token t of `a`, in the lane-row layout and, when a
// has one, the MFMA layout.  Every lane of the wave must call this; `write`
// selects which 32-lane halves store.
template <bool COH = false>
__device__ __forceinline__ void put_digits(const Act& a, int qt, int t, int blk, float v, bool write) {
  int32_t* xd = a.xd + ((size_t)t * a.nblk + blk) * XW;
  float* xs = a.xs + (size_t)t * a.nblk + blk;
  if (qt == QT_Q4) quant_block_half<QT_Q4, COH>(v, xd, xs, write);
  else quant_block_half<QT_Q8, COH>(v, xd, xs, write);
  if (a.mxd) {
    if (qt == QT_Q4) quant_block_mx<QT_Q4>(v, a, t, blk, write);
    else quant_block_mx<QT_Q8>(v, a, t, blk, write);
  }
}

// Shared tail of every producer of a residual-stream vector: lane holds h_new
// for row rg*64+lane (0 beyond H).  Writes h, the sum of squares of the 64 rows,
// and the digits of norm_w*h for blocks 2rg and 2rg+1.
// `w` is norm_w of this lane's row (0 beyond H).
template <bool COH = false>
__device__ __forceinline__ void resid_tail_w(int t, int rg, int H, float hn, float w, float* h, int64_t h_ts, int qt,
                                             const Act& next, float* ssq_out, int nrg) {
  const int lane = threadIdx.x & 63;
  const int row = rg * RG + lane;
  if (row < H) st_<COH>(h + (size_t)t * h_ts + row, hn);
  const float ss = wave_sum(hn * hn);
  if (lane == 0) st_<COH>(ssq_out + (size_t)t * nrg + rg, ss);
  const int blk = 2 * rg + (lane >> 5);
  put_digits<COH>(next, qt, t, blk, w * hn, blk < next.nblk);
}
template <bool COH = false>
__device__ __forceinline__ void resid_tail(int t, int rg, int H, float hn, float* h, int64_t h_ts,
                                           const float* norm_w, int qt, const Act& next,
                                           float* ssq_out, int nrg) {
  const int row = rg * RG + (int)(threadIdx.x & 63);
  const float w = row < H ? norm_w[row] : 0.0f;
  resid_tail_w<COH>(t, rg, H, hn, w, h, h_ts, qt, next, ssq_out, nrg);
}

}  // namespace slq
