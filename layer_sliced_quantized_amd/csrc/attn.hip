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
//   split:   one workgroup per (KV head, 256-row chunk); scores of the group's
//            query heads against the chunk, chunk-local max / sum of exp and
//            the unnormalised P V.  Query t (position p+t) sees rows <= p+t.
//   combine: per (token, query head): merge the chunks' partials, apply the
//            gate sigmoid(g), and quantise the result for the output GEMV.
// Chunk boundaries are absolute (multiples of 256), so query t of a verify
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

template <int GRP>
__global__ __launch_bounds__(256) void k_attn_split(AttnParams p, int T) {
  constexpr int C = ATT_CHUNK;
  __shared__ float pl[GRP][C];
  __shared__ float wm[4][GRP];
  const int g = blockIdx.x / p.nchunk, c = blockIdx.x % p.nchunk;
  const int p0 = p.ctrl->pos;
  const int r0 = c * C;
  if (r0 > p0 + T - 1) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_id();
  const int r = r0 + tid;
  for (int t = 0; t < T; ++t) {
    const int P = p0 + t;
    const int nvalid = min(C, P + 1 - r0);
    if (nvalid <= 0) continue;
    const float* qh = p.qhat + ((size_t)t * p.q_heads + g * GRP) * p.hd;
    float s[GRP];
#pragma unroll
    for (int h = 0; h < GRP; ++h) s[h] = 0.0f;
    if (tid < nvalid) {
      for (int dc = 0; dc < p.hd / 8; ++dc) {
        const uint4 kw = *reinterpret_cast<const uint4*>(p.kc + kidx(g, r, dc * 8, p.max_seq, p.hd));
        float kf[8];
        const uint32_t ws[4] = {kw.x, kw.y, kw.z, kw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kf[2 * e] = __half2float(__ushort_as_half((unsigned short)(ws[e] & 0xffff)));
          kf[2 * e + 1] = __half2float(__ushort_as_half((unsigned short)(ws[e] >> 16)));
        }
#pragma unroll
        for (int h = 0; h < GRP; ++h) {
          const float* q = qh + (size_t)h * p.hd + dc * 8;
#pragma unroll
          for (int e = 0; e < 8; ++e) s[h] = __builtin_fmaf(kf[e], q[e], s[h]);
        }
      }
    }
    // chunk max per head
    float m[GRP];
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      const float v = wave_max(tid < nvalid ? s[h] : -INFINITY);
      if (lane == 0) wm[wave][h] = v;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      float v = wm[0][h];
      for (int w = 1; w < 4; ++w) v = fmaxf(v, wm[w][h]);
      m[h] = v;
    }
    __syncthreads();
    float l[GRP];
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      const float e = tid < nvalid ? __expf(s[h] - m[h]) : 0.0f;
      pl[h][tid] = e;
      const float v = wave_sum(e);
      if (lane == 0) wm[wave][h] = v;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < GRP; ++h) l[h] = wm[0][h] + wm[1][h] + wm[2][h] + wm[3][h];
    // P V: thread = dimension
    if (tid < p.hd) {
      float o[GRP];
#pragma unroll
      for (int h = 0; h < GRP; ++h) o[h] = 0.0f;
      const __half* vrow = p.vc + ((size_t)g * p.max_seq + r0) * p.hd + tid;
      for (int rr = 0; rr < nvalid; ++rr) {
        const float v = __half2float(vrow[(size_t)rr * p.hd]);
#pragma unroll
        for (int h = 0; h < GRP; ++h) o[h] = __builtin_fmaf(pl[h][rr], v, o[h]);
      }
#pragma unroll
      for (int h = 0; h < GRP; ++h) {
        float* dst = p.part + (((size_t)t * p.q_heads + g * GRP + h) * p.nchunk + c) * (p.hd + 2);
        dst[2 + tid] = o[h];
        if (tid == 0) { dst[0] = m[h]; dst[1] = l[h]; }
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void k_attn_combine(AttnParams p) {
  const int t = blockIdx.x / p.q_heads, h = blockIdx.x % p.q_heads;
  const int d = threadIdx.x;
  const int P = p.ctrl->pos + t;
  const int nc = P / ATT_CHUNK + 1;
  const float* base = p.part + ((size_t)t * p.q_heads + h) * p.nchunk * (p.hd + 2);
  float M = -INFINITY;
  for (int c = 0; c < nc; ++c) M = fmaxf(M, base[(size_t)c * (p.hd + 2)]);
  float L = 0.0f, o = 0.0f;
  for (int c = 0; c < nc; ++c) {
    const float* pc = base + (size_t)c * (p.hd + 2);
    const float w = __expf(pc[0] - M);
    L = __builtin_fmaf(pc[1], w, L);
    o = __builtin_fmaf(pc[2 + d], w, o);
  }
  o = o / L;
  if (p.off_g >= 0) o = o * sigmoidf_(p.y[(size_t)t * p.y_stride + p.off_g + h * p.hd + d]);
  const int nu = p.q_heads * p.hd;
  if (p.u_out) p.u_out[(size_t)t * nu + h * p.hd + d] = o;
  const int blk = (h * p.hd + d) / QK;
  quant_block_half_qt(p.next_qt, o, p.next.xd + ((size_t)t * p.next.nblk + blk) * XW,
                      p.next.xs + (size_t)t * p.next.nblk + blk, true);
}

hipError_t launch_attention(const AttnParams& p, int T, hipStream_t s) {
  if (p.hd % 64 || p.hd > 256 || p.rope_dims % 2 || p.rope_dims > p.hd || p.max_seq % 64 ||
      p.q_heads % p.kv_heads)
    return hipErrorInvalidValue;
  k_attn_prep<<<T * (p.q_heads + p.kv_heads), p.hd, 0, s>>>(p);
  const int grp = p.q_heads / p.kv_heads;
  const unsigned grid = (unsigned)(p.kv_heads * p.nchunk);
  switch (grp) {
#define SLQ_G(n) case n: k_attn_split<n><<<grid, 256, 0, s>>>(p, T); break;
    SLQ_G(1) SLQ_G(2) SLQ_G(3) SLQ_G(4) SLQ_G(5) SLQ_G(6) SLQ_G(7) SLQ_G(8)
#undef SLQ_G
    default: return hipErrorInvalidValue;
  }
  k_attn_combine<<<T * p.q_heads, p.hd, 0, s>>>(p);
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
