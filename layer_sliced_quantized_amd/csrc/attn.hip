// GQA decode / verify attention over an fp16 KV cache, split along the keys.
//
// Attention layers of both model kinds (ChatTorrent README, "What it can
// run"): Llama-style GQA with RoPE, and the hybrid's full-attention layers with
// partial RoPE, QK-norm and a sigmoid output gate.  Each stage keeps its own
// KV cache ("Unstable Legion", section "Splitting the workload").
//
// Three kernels per layer:
//   prep:    per query/KV head: RMSNorm (if QK-norm), RoPE on the first
//            rope_dims entries (angle pos * theta^(-2i/r) taken in fp64),
//            q scaled by 1/sqrt(head_dim); K/V row p+t rounded to fp16 and
//            appended to the cache.
//   split:   one workgroup per (KV head, 64-row chunk); scores of the group's
//            query heads against the chunk, chunk-local max / sum of exp and
//            the unnormalised P V.  Query t (position p+t) sees rows <= p+t.
//   combine: per (token, query head): merge the chunks' partials, apply the
//            gate sigmoid(g), and quantise the result for the output GEMV.
// Chunk boundaries are absolute (multiples of 64), so query t of a verify
// pass is computed with exactly the operations a decode at p+t would use.
//
// K cache layout: [kv][pos/64][head_dim/8][64 pos][8] (a wave reads 64 rows'
// 16-byte pieces as one contiguous 1 KiB); V cache: [kv][pos][head_dim].
#include "dev.h"

namespace slq {

__device__ __forceinline__ size_t kidx(int g, int pos, int d, int max_seq, int hd) {
  const int ntile = max_seq / 64;
  return ((((size_t)g * ntile + pos / 64) * (hd / 8) + d / 8) * 64 + (pos % 64)) * 8 + (d % 8);
}

__global__ __launch_bounds__(256) void k_attn_prep(AttnParams p) {
  __shared__ float buf[256];
  __shared__ float wred[4];
  const int nh = p.q_heads + p.kv_heads;
  const int t = blockIdx.x / nh, hh = blockIdx.x % nh;
  const int d = threadIdx.x;
  const int pos = p.ctrl->pos + t;
  const float* y = p.y + (size_t)t * p.y_stride;
  const bool isq = hh < p.q_heads;
  const int kvh = hh - p.q_heads;
  float x = isq ? y[p.off_q + hh * p.hd + d] : y[p.off_k + kvh * p.hd + d];
  if (p.qk_norm) {
    const float ss = wave_sum(x * x);
    if ((d & 63) == 0) wred[d >> 6] = ss;
    __syncthreads();
    float tot = 0.0f;
    for (int w = 0; w < (p.hd >> 6); ++w) tot += wred[w];
    const float rn = 1.0f / sqrtf(tot / (float)p.hd + p.eps);
    x = x * rn * (isq ? p.q_norm[d] : p.k_norm[d]);
  }
  buf[d] = x;
  __syncthreads();
  if (d < p.rope_dims) {
    const int half = p.rope_dims / 2;
    const int i = d % half;
    const double ang = (double)pos * pow(p.rope_theta, -2.0 * (double)i / (double)p.rope_dims);
    const float c = (float)cos(ang), sn = (float)sin(ang);
    if (d < half) x = buf[d] * c - buf[d + half] * sn;
    else x = buf[d] * c + buf[d - half] * sn;
  }
  if (isq) {
    p.qhat[((size_t)t * p.q_heads + hh) * p.hd + d] = x * (1.0f / sqrtf((float)p.hd));
  } else {
    p.kc[kidx(kvh, pos, d, p.max_seq, p.hd)] = __float2half_rn(x);
    p.vc[((size_t)kvh * p.max_seq + pos) * p.hd + d] = __float2half_rn(y[p.off_v + kvh * p.hd + d]);
  }
}

// One workgroup per (KV head g, 64-row chunk c), 4 waves.  Scores: wave w
// takes rows 16w..16w+15 of the chunk, 4 lanes per row each over a quarter of
// the head dimensions, summed with two butterfly steps.  P V: one thread per
// head dimension over the chunk's rows.
template <int GRP, int HD>
__global__ __launch_bounds__(256) void k_attn_split(AttnParams p, int T) {
  constexpr int C = ATT_CHUNK;
  __shared__ __attribute__((aligned(16))) float pl[GRP][C];
  __shared__ __attribute__((aligned(16))) float qsh[GRP * HD];
  __shared__ float wm[4][GRP];
  const int g = blockIdx.x / p.nchunk, c = blockIdx.x % p.nchunk;
  const int p0 = p.ctrl->pos;
  const int r0 = c * C;
  if (r0 > p0 + T - 1) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_id();
  const int rr = wave * 16 + (lane & 15);      // row of this lane inside the chunk
  const int dq = lane >> 4;                    // quarter of the head dimensions
  constexpr int NC = HD / 32;                  // 8-dim pieces per quarter of the head
  const int r = r0 + rr;
  for (int t = 0; t < T; ++t) {
    const int P = p0 + t;
    const int nvalid = min(C, P + 1 - r0);
    if (nvalid <= 0) continue;
    {
      const float* qg = p.qhat + ((size_t)t * p.q_heads + g * GRP) * p.hd;
      float qv[GRP];
#pragma unroll
      for (int h = 0; h < GRP; ++h) qv[h] = tid < HD ? qg[h * HD + tid] : 0.0f;
#pragma unroll
      for (int h = 0; h < GRP; ++h)
        if (tid < HD) qsh[h * HD + tid] = qv[h];
    }
    __syncthreads();
    float s[GRP];
#pragma unroll
    for (int h = 0; h < GRP; ++h) s[h] = 0.0f;
    if (rr < nvalid) {
      // this lane's NC pieces of the key row, all requested before any math
      uint4 kw[NC];
#pragma unroll
      for (int i = 0; i < NC; ++i)
        kw[i] = *reinterpret_cast<const uint4*>(p.kc + kidx(g, r, (dq * NC + i) * 8, p.max_seq, HD));
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int dc = dq * NC + i;
        float kf[8];
        const uint32_t ws[4] = {kw[i].x, kw[i].y, kw[i].z, kw[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kf[2 * e] = __half2float(__ushort_as_half((unsigned short)(ws[e] & 0xffff)));
          kf[2 * e + 1] = __half2float(__ushort_as_half((unsigned short)(ws[e] >> 16)));
        }
#pragma unroll
        for (int h = 0; h < GRP; ++h) {
          const float4 qa = *reinterpret_cast<const float4*>(qsh + h * HD + dc * 8);
          const float4 qb = *reinterpret_cast<const float4*>(qsh + h * HD + dc * 8 + 4);
          s[h] = __builtin_fmaf(kf[0], qa.x, s[h]);
          s[h] = __builtin_fmaf(kf[1], qa.y, s[h]);
          s[h] = __builtin_fmaf(kf[2], qa.z, s[h]);
          s[h] = __builtin_fmaf(kf[3], qa.w, s[h]);
          s[h] = __builtin_fmaf(kf[4], qb.x, s[h]);
          s[h] = __builtin_fmaf(kf[5], qb.y, s[h]);
          s[h] = __builtin_fmaf(kf[6], qb.z, s[h]);
          s[h] = __builtin_fmaf(kf[7], qb.w, s[h]);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      s[h] += __shfl_xor(s[h], 16, 64);
      s[h] += __shfl_xor(s[h], 32, 64);
    }
    // chunk max per head
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      const float v = wave_max(rr < nvalid ? s[h] : -INFINITY);
      if (lane == 0) wm[wave][h] = v;
    }
    __syncthreads();
    float m[GRP];
#pragma unroll
    for (int h = 0; h < GRP; ++h) m[h] = fmaxf(fmaxf(wm[0][h], wm[1][h]), fmaxf(wm[2][h], wm[3][h]));
    __syncthreads();
    float l[GRP];
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      const float e = rr < nvalid ? __expf(s[h] - m[h]) : 0.0f;
      if (dq == 0) pl[h][rr] = e;
      // each row's weight appears on 4 lanes; count it once
      const float v = wave_sum(dq == 0 ? e : 0.0f);
      if (lane == 0) wm[wave][h] = v;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < GRP; ++h) l[h] = (wm[0][h] + wm[1][h]) + (wm[2][h] + wm[3][h]);
    // P V: thread = dimension
    if (tid < HD) {
      float o[GRP];
#pragma unroll
      for (int h = 0; h < GRP; ++h) o[h] = 0.0f;
      const __half* vrow = p.vc + ((size_t)g * p.max_seq + r0) * HD + tid;
      // rows past nvalid have weight 0 and lie inside the cache (r0 + C <= max_seq)
      for (int q0 = 0; q0 < nvalid; q0 += 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = __half2float(vrow[(size_t)(q0 + u) * HD]);
#pragma unroll
        for (int u = 0; u < 16; u += 4) {
#pragma unroll
          for (int h = 0; h < GRP; ++h) {
            const float4 w4 = *reinterpret_cast<const float4*>(&pl[h][q0 + u]);
            o[h] = __builtin_fmaf(w4.x, v[u], o[h]);
            o[h] = __builtin_fmaf(w4.y, v[u + 1], o[h]);
            o[h] = __builtin_fmaf(w4.z, v[u + 2], o[h]);
            o[h] = __builtin_fmaf(w4.w, v[u + 3], o[h]);
          }
        }
      }
#pragma unroll
      for (int h = 0; h < GRP; ++h) {
        float* dst = p.part + (((size_t)t * p.q_heads + g * GRP + h) * p.nchunk + c) * (HD + 2);
        dst[2 + tid] = o[h];
        if (tid == 0) { dst[0] = m[h]; dst[1] = l[h]; }
      }
    }
    __syncthreads();
  }
}

// One workgroup per (token, query head, 64 dimensions): merge the chunks,
// normalise, apply the gate and quantise the two 32-dim blocks.  Lane c loads
// chunk c's max and sum (several rounds beyond 64 chunks), the weights
// exp(m_c - M) go through LDS, and every lane then folds its dimension.
__global__ __launch_bounds__(64) void k_attn_combine(AttnParams p) {
  __shared__ float wsh[1024];
  const int ndg = p.hd / 64;
  const int t = blockIdx.x / (p.q_heads * ndg);
  const int h = (blockIdx.x / ndg) % p.q_heads;
  const int lane = threadIdx.x;
  const int d = (blockIdx.x % ndg) * 64 + lane;
  const int P = p.ctrl->pos + t;
  const int nc = P / ATT_CHUNK + 1;
  const int stride = p.hd + 2;
  const float* base = p.part + ((size_t)t * p.q_heads + h) * p.nchunk * stride;
  float M = -INFINITY;
  for (int c = lane; c < nc; c += 64) M = fmaxf(M, base[(size_t)c * stride]);
  M = wave_max(M);
  float L = 0.0f;
  for (int c0 = 0; c0 < nc; c0 += 64) {
    const int c = c0 + lane;
    float w = 0.0f, l = 0.0f;
    if (c < nc) {
      w = __expf(base[(size_t)c * stride] - M);
      l = base[(size_t)c * stride + 1];
    }
    L += wave_sum(l * w);
    if (c < nc && c < 1024) wsh[c] = w;
  }
  __syncthreads();
  float o = 0.0f;
  for (int c0 = 0; c0 < nc; c0 += 8) {
    // eight loads in flight, then the adds in chunk order
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = c0 + u < nc ? base[(size_t)(c0 + u) * stride + 2 + d] : 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = c0 + u;
      if (c < nc) {
        const float w = c < 1024 ? wsh[c] : __expf(base[(size_t)c * stride] - M);
        o = __builtin_fmaf(v[u], w, o);
      }
    }
  }
  o = o / L;
  if (p.off_g >= 0) o = o * sigmoidf_(p.y[(size_t)t * p.y_stride + p.off_g + h * p.hd + d]);
  const int nu = p.q_heads * p.hd;
  if (p.u_out) p.u_out[(size_t)t * nu + h * p.hd + d] = o;
  const int blk = (h * p.hd + d) / QK;
  put_digits(p.next, p.next_qt, t, blk, o, true);
}

hipError_t launch_attention(const AttnParams& p, int T, hipStream_t s) {
  if (p.hd % 64 || p.hd > 256 || p.rope_dims % 2 || p.rope_dims > p.hd || p.max_seq % 64 ||
      p.q_heads % p.kv_heads)
    return hipErrorInvalidValue;
  k_attn_prep<<<T * (p.q_heads + p.kv_heads), p.hd, 0, s>>>(p);
  const int grp = p.q_heads / p.kv_heads;
  const unsigned grid = (unsigned)(p.kv_heads * p.nchunk);
#define SLQ_G(n, hd) case n: k_attn_split<n, hd><<<grid, 256, 0, s>>>(p, T); break;
#define SLQ_HD(hd)                                                                        \
  case hd:                                                                                \
    switch (grp) {                                                                        \
      SLQ_G(1, hd) SLQ_G(2, hd) SLQ_G(3, hd) SLQ_G(4, hd) SLQ_G(5, hd) SLQ_G(6, hd)       \
      SLQ_G(7, hd) SLQ_G(8, hd)                                                           \
      default: return hipErrorInvalidValue;                                               \
    }                                                                                     \
    break;
  switch (p.hd) {
    SLQ_HD(64) SLQ_HD(128) SLQ_HD(192) SLQ_HD(256)
    default: return hipErrorInvalidValue;
  }
#undef SLQ_HD
#undef SLQ_G
  k_attn_combine<<<T * p.q_heads * (p.hd / 64), 64, 0, s>>>(p);
  return hipGetLastError();
}

// Canonical [kv][rows][hd] fp16 <-> cache layouts.
__global__ void k_kv_io(__half* kc, __half* vc, int kvh, int max_seq, int hd, uint16_t* k, uint16_t* v,
                        int rows, int to_device) {
  const size_t n = (size_t)kvh * rows * hd;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int g = (int)(idx / ((size_t)rows * hd));
  const int rem = (int)(idx % ((size_t)rows * hd));
  const int pos = rem / hd, d = rem % hd;
  unsigned short* K = reinterpret_cast<unsigned short*>(kc);
  unsigned short* V = reinterpret_cast<unsigned short*>(vc);
  const size_t ki = kidx(g, pos, d, max_seq, hd);
  const size_t vi = ((size_t)g * max_seq + pos) * hd + d;
  if (to_device) { K[ki] = k[idx]; V[vi] = v[idx]; }
  else { k[idx] = K[ki]; v[idx] = V[vi]; }
}

hipError_t launch_kv_io(__half* kc, __half* vc, int kv_heads, int max_seq, int hd, uint16_t* k, uint16_t* v,
                        int rows, int to_device, hipStream_t s) {
  const size_t n = (size_t)kv_heads * rows * hd;
  if (n == 0) return hipSuccess;
  k_kv_io<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(kc, vc, kv_heads, max_seq, hd, k, v, rows, to_device);
  return hipGetLastError();
}

}  // namespace slq
