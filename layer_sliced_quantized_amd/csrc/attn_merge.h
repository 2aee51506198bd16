// The merge of a decode attention head's split partials by one wave, shared
// by the combine kernel (attn.hip) and the chained decode kernel (chain.hip),
// so both give the same bits.
#pragma once
#include "dev.h"

namespace slq {

// Merge of at most 64 partials of (token t, head h, dims d0 .. d0 + 63) by one
// wave (lane = dimension): every partial's max and sum (lane c) and the first
// VPRE partials' values are requested in one round, then M = max m_c,
// L = sum l_c e^(m_c - M), O = sum_c e^(m_c - M) o_c in partial order,
// o = O / L, the gate sigmoid(g), and the output digits.  wsh: 64 floats of
// the wave's own.  COH: the digits are read later in the same kernel
// (coherent stores).
template <bool COH>
__device__ __forceinline__ void merge_wave(const AttnParams& p, int t, int h, int d0, int nc, float* wsh) {
  constexpr int VPRE = 32;   // partials whose values are requested with the statistics
  const int lane = threadIdx.x & 63;
  const int d = d0 + lane;
  const float gz = p.off_g >= 0 ? p.y[(size_t)t * p.y_stride + p.off_g + h * p.hd + d] : 0.0f;
  const int stride = p.hd + 2;
  const float* base = p.part + ((size_t)t * p.q_heads + h) * p.nchunk * stride;
  float m0 = -INFINITY, l0 = 0.0f;
  if (lane < nc) {
    m0 = base[(size_t)lane * stride];
    l0 = base[(size_t)lane * stride + 1];
  }
  float v0[VPRE];
#pragma unroll
  for (int u = 0; u < VPRE; ++u) v0[u] = u < nc ? base[(size_t)u * stride + 2 + d] : 0.0f;
  const float M = wave_max(m0);
  const float wt = lane < nc ? __expf(m0 - M) : 0.0f;
  const float L = wave_sum((lane < nc ? l0 : 0.0f) * wt);
  if (lane < nc) wsh[lane] = wt;   // LDS operations of one wave take effect in order
  float o = 0.0f;
#pragma unroll
  for (int u = 0; u < VPRE; ++u)
    if (u < nc) o = __builtin_fmaf(v0[u], wsh[u], o);
  for (int c0 = VPRE; c0 < nc; c0 += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = c0 + u < nc ? base[(size_t)(c0 + u) * stride + 2 + d] : 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (c0 + u < nc) o = __builtin_fmaf(v[u], wsh[c0 + u], o);
  }
  o = o / L;
  if (p.off_g >= 0) o = o * sigmoidf_(gz);
  const int nu = p.q_heads * p.hd;
  if (p.u_out) p.u_out[(size_t)t * nu + h * p.hd + d] = o;
  const int blk = (h * p.hd + d) / QK;
  if (p.next.xd) put_digits<COH>(p.next, p.next_qt, t, blk, o, true);
}

}  // namespace slq
