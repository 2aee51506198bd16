// GQA decode / verify attention over an fp16 KV cache, split along the keys.
//
// Attention layers of both model kinds (ChatTorrent README, "What it can
// run"): Llama-style GQA with RoPE, and the hybrid's full-attention layers with
// partial RoPE, QK-norm and a sigmoid output gate.  Each stage keeps its own
// KV cache ("Unstable Legion", section "Splitting the workload").
//
// Two kernels per layer:
//   split:   one workgroup per (KV head, 32-row chunk).  It first appends the
//            K/V rows of this step that fall in its chunk (RMSNorm if QK-norm,
//            RoPE on the first rope_dims entries with the angle
//            pos * theta^(-2i/r) taken in fp64, fp16 rounding), then prepares
//            its query heads the same way (q also scaled by 1/sqrt(head_dim)),
//            and computes the chunk-local max / sum of exp and the
//            unnormalised P V.  Query t (position p+t) sees rows <= p+t.
//   combine: per (token, query head): merge the chunks' partials, apply the
//            gate sigmoid(g), and quantise the result for the output GEMV.
// Chunk boundaries are absolute (multiples of 32), so query t of a verify
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

// Table of the RoPE rotations, built once at load: entry (pos, i) holds cos
// and sin of the angle pos * theta^(-2i/r), taken in fp64.
__global__ void k_rope_table(float* cs, int max_seq, int rope_dims, double theta) {
  const int half = rope_dims / 2;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)max_seq * half) return;
  const int pos = (int)(idx / half), i = (int)(idx % half);
  const double ang = (double)pos * pow(theta, -2.0 * (double)i / (double)rope_dims);
  cs[2 * idx] = (float)cos(ang);
  cs[2 * idx + 1] = (float)sin(ang);
}

hipError_t launch_rope_table(float* cs, int max_seq, int rope_dims, double theta, hipStream_t s) {
  const size_t n = (size_t)max_seq * (rope_dims / 2);
  if (n == 0) return hipSuccess;
  k_rope_table<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(cs, max_seq, rope_dims, theta);
  return hipGetLastError();
}

// Rotation of entry d at position pos (identity past rope_dims).
__device__ __forceinline__ void rope_cs(const AttnParams& p, int d, int pos, float& c, float& sn) {
  c = 1.0f;
  sn = 0.0f;
  if (d < p.rope_dims) {
    const int half = p.rope_dims / 2;
    const float* e = p.rope_cs + 2 * ((size_t)pos * half + d % half);
    c = e[0];
    sn = e[1];
  }
}

// RMSNorm (when enabled) and RoPE of NH head vectors held one entry per
// thread (x[h] = entry d of head h for d < hd, 0 elsewhere), all rotated by
// (c, sn) of entry d.  Every thread of the workgroup calls it: buf (NH * hd
// floats) and wred (4 x NH floats) are LDS, free again on return.
template <int NH>
__device__ __forceinline__ void heads_prep(float (&x)[NH], int d, const AttnParams& p, const float* norm_w, float c,
                                           float sn, float* buf, float (*wred)[8]) {
  const bool act = d < p.hd;
  if (p.qk_norm) {
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const float ss = wave_sum(x[h] * x[h]);
      if ((d & 63) == 0) wred[d >> 6][h] = ss;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      float tot = 0.0f;
      for (int w = 0; w < (p.hd >> 6); ++w) tot += wred[w][h];
      const float rn = 1.0f / sqrtf(tot / (float)p.hd + p.eps);
      x[h] = act ? x[h] * rn * norm_w[d] : 0.0f;
    }
  }
#pragma unroll
  for (int h = 0; h < NH; ++h)
    if (act) buf[h * p.hd + d] = x[h];
  __syncthreads();
  if (act && d < p.rope_dims) {
    const int half = p.rope_dims / 2;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const float* b = buf + h * p.hd;
      x[h] = d < half ? b[d] * c - b[d + half] * sn : b[d] * c + b[d - half] * sn;
    }
  }
  __syncthreads();
}

// One workgroup per (KV head g, group of HPW of its query heads, 32-row chunk
// c), 4 waves.  Scores: thread
// (row rr = tid / 8, part = tid % 8) takes an eighth of the head dimensions
// of key row rr, the eight parts meeting with three butterfly steps.  P V:
// one thread per head dimension over the chunk's rows.  The chunk's keys and
// values are requested once, before the query preparation, and serve every
// token of the pass.
template <int GRP, int HD>   // GRP: query heads per workgroup
__global__ __launch_bounds__(256) void k_attn_split(AttnParams p, int T) {
  constexpr int C = ATT_CHUNK;
  constexpr int NC = HD / 64;   // 8-dim pieces per eighth of the head
  __shared__ __attribute__((aligned(16))) float qsh[GRP * HD];
  __shared__ __attribute__((aligned(16))) float pl[GRP][C];
  __shared__ float buf[GRP * HD];
  __shared__ float wred[4][8];
  __shared__ float wm[4][GRP];
  const int nsub = p.q_heads / p.kv_heads / GRP;   // query-head groups per KV head
  const int g = blockIdx.x / (nsub * p.nchunk);
  const int sub = (blockIdx.x / p.nchunk) % nsub, c = blockIdx.x % p.nchunk;
  const int h0 = (g * nsub + sub) * GRP;            // first query head of this workgroup
  const int p0 = p.ctrl->pos;
  const int r0 = c * C;
  if (r0 > p0 + T - 1) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_id();
  const bool dact = tid < HD;

  // this step's K/V rows inside the chunk: positions p0 + t in [r0, r0 + C).
  // Every query-head group of the chunk computes and stores them itself
  // (the same bits), so each reads them back after its own stores.
  // (each token's k and v are requested one token ahead)
  const int ta = max(0, r0 - p0), tb = min(T, r0 + C - p0);
  float kn = 0.0f, vn = 0.0f;
  if (ta < tb && dact) {
    const float* y = p.y + (size_t)ta * p.y_stride;
    kn = y[p.off_k + g * HD + tid];
    vn = y[p.off_v + g * HD + tid];
  }
  for (int t = ta; t < tb; ++t) {
    const int pos = p0 + t;
    float k[1] = {kn};
    const float vx = vn;
    if (t + 1 < tb && dact) {
      const float* y = p.y + (size_t)(t + 1) * p.y_stride;
      kn = y[p.off_k + g * HD + tid];
      vn = y[p.off_v + g * HD + tid];
    }
    float c, sn;
    rope_cs(p, tid, pos, c, sn);
    heads_prep<1>(k, tid, p, p.k_norm, c, sn, buf, wred);
    if (dact) {
      p.kc[kidx(g, pos, tid, p.max_seq, HD)] = __float2half_rn(k[0]);
      p.vc[((size_t)g * p.max_seq + pos) * HD + tid] = __float2half_rn(vx);
    }
  }
  if (tb > ta) {
    __threadfence_block();
    __syncthreads();
  }

  // the chunk's keys (this thread's eighth of row rr) and values (dimension
  // tid of every row); rows past the valid ones lie inside the cache and get
  // weight 0
  const int rr = tid >> 3, part = tid & 7;
  const int r = r0 + rr;
  uint4 kw[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i)
    kw[i] = *reinterpret_cast<const uint4*>(p.kc + kidx(g, r, (part * NC + i) * 8, p.max_seq, HD));
  unsigned short vv[C];
  {
    const unsigned short* vrow =
        reinterpret_cast<const unsigned short*>(p.vc) + ((size_t)g * p.max_seq + r0) * HD + (dact ? tid : 0);
#pragma unroll
    for (int q = 0; q < C; ++q) vv[q] = vrow[(size_t)q * HD];
  }

  // tokens from the first whose position reaches this chunk; each token's
  // query values are requested one token ahead
  const int tq = max(0, r0 - p0);
  float qn[GRP];
#pragma unroll
  for (int h = 0; h < GRP; ++h) qn[h] = dact && tq < T ? p.y[(size_t)tq * p.y_stride + p.off_q + (h0 + h) * HD + tid] : 0.0f;
  for (int t = tq; t < T; ++t) {
    const int P = p0 + t;
    const int nvalid = min(C, P + 1 - r0);
    {
      float qx[GRP];
#pragma unroll
      for (int h = 0; h < GRP; ++h) qx[h] = qn[h];
      if (t + 1 < T && dact) {
        const float* y = p.y + (size_t)(t + 1) * p.y_stride;
#pragma unroll
        for (int h = 0; h < GRP; ++h) qn[h] = y[p.off_q + (h0 + h) * HD + tid];
      }
      float c, sn;
      rope_cs(p, tid, P, c, sn);
      heads_prep<GRP>(qx, tid, p, p.q_norm, c, sn, buf, wred);
#pragma unroll
      for (int h = 0; h < GRP; ++h)
        if (dact) qsh[h * HD + tid] = qx[h] * (1.0f / sqrtf((float)HD));
    }
    __syncthreads();
    float s[GRP];
#pragma unroll
    for (int h = 0; h < GRP; ++h) s[h] = 0.0f;
    if (rr < nvalid) {
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int dc = part * NC + i;
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
        asm volatile("" ::: "memory");   // one piece's query values in registers at a time
      }
    }
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      s[h] += __shfl_xor(s[h], 1, 64);
      s[h] += __shfl_xor(s[h], 2, 64);
      s[h] += __shfl_xor(s[h], 4, 64);
    }
    // chunk max per head (each wave holds 8 rows)
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
      if (part == 0) pl[h][rr] = e;
      // each row's weight appears on 8 lanes; count it once
      const float v = wave_sum(part == 0 ? e : 0.0f);
      if (lane == 0) wm[wave][h] = v;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < GRP; ++h) l[h] = (wm[0][h] + wm[1][h]) + (wm[2][h] + wm[3][h]);
    if (dact) {
      float o[GRP];
#pragma unroll
      for (int h = 0; h < GRP; ++h) o[h] = 0.0f;
#pragma unroll
      for (int q = 0; q < C; q += 4) {
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = q + u < nvalid ? __half2float(__ushort_as_half(vv[q + u])) : 0.0f;
#pragma unroll
        for (int h = 0; h < GRP; ++h) {
          const float4 w = *reinterpret_cast<const float4*>(&pl[h][q]);
          o[h] = __builtin_fmaf(w.x, v[0], o[h]);
          o[h] = __builtin_fmaf(w.y, v[1], o[h]);
          o[h] = __builtin_fmaf(w.z, v[2], o[h]);
          o[h] = __builtin_fmaf(w.w, v[3], o[h]);
        }
        asm volatile("" ::: "memory");   // four rows' weights in registers at a time
      }
#pragma unroll
      for (int h = 0; h < GRP; ++h) {
        float* dst = p.part + (((size_t)t * p.q_heads + h0 + h) * p.nchunk + c) * (HD + 2);
        dst[2 + tid] = o[h];
        if (tid == 0) { dst[0] = m[h]; dst[1] = l[h]; }
      }
    }
    __syncthreads();   // qsh, pl and wm are rewritten by the next token
  }
}

// One workgroup per (token, query head, 64 dimensions): merge the chunks,
// normalise, apply the gate and quantise the two 32-dim blocks.  Lane c loads
// chunk c's max and sum (several rounds beyond 64 chunks), the weights
// exp(m_c - M) go through LDS, and every lane then folds its dimension.
__global__ __launch_bounds__(64) void k_attn_combine(AttnParams p) {
  __shared__ float wsh[2048];
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
    if (c < nc && c < 2048) wsh[c] = w;
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
        const float w = c < 2048 ? wsh[c] : __expf(base[(size_t)c * stride] - M);
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
      p.nchunk * ATT_CHUNK < p.max_seq || (p.rope_dims && !p.rope_cs) ||
      p.q_heads % p.kv_heads)
    return hipErrorInvalidValue;
  // query heads per split workgroup: at most 2 of a KV head's group, so that
  // the work of a chunk spreads over several workgroups
  const int grp = p.q_heads / p.kv_heads;
  const int hpw = grp % 2 == 0 ? 2 : 1;
  const unsigned grid = (unsigned)(p.kv_heads * (grp / hpw) * p.nchunk);
#define SLQ_G(n, hd) case n: k_attn_split<n, hd><<<grid, 256, 0, s>>>(p, T); break;
#define SLQ_HD(hd)                                          \
  case hd:                                                  \
    switch (hpw) {                                          \
      SLQ_G(1, hd) SLQ_G(2, hd)                             \
      default: return hipErrorInvalidValue;                 \
    }                                                       \
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
