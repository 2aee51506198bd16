// GQA decode / verify attention over an fp16 KV cache, split along the keys.
//
// Attention layers of both model kinds (ChatTorrent README, "What it can
// run"): Llama-style GQA with RoPE, and the hybrid's full-attention layers with
// partial RoPE, QK-norm and a sigmoid output gate.  Each stage keeps its own
// KV cache ("Unstable Legion", section "Splitting the workload").
//
// Two kernels per layer:
//   split:   one workgroup per (KV head, group of query heads, 32-row chunk);
//            for one token on a long cache (k_attn_split_range) one workgroup
//            per (KV head, range of chunks) with all the KV head's query heads.
//            It first appends the K/V rows of this step that fall in its
//            chunk (RMSNorm if QK-norm, RoPE on the first rope_dims entries
//            with the angle pos * theta^(-2i/r) taken in fp64, fp16
//            rounding), then prepares its query heads the same way (q also
//            scaled by 1/sqrt(head_dim)), and computes the chunk-local max /
//            sum of exp and the unnormalised P V for every token of the pass.
//            Query t (position p+t) sees rows <= p+t.
//   combine: per (token, query head): merge the chunks' partials, apply the
//            gate sigmoid(g), and quantise the result for the output GEMV.
// Chunk boundaries are absolute (multiples of 32), so query t of a verify
// pass is computed with exactly the operations a decode at p+t would use.
//
// K cache layout: [kv][pos/64][head_dim/8][64 pos][8] (a wave reads 64 rows'
// 16-byte pieces as one contiguous 1 KiB); V cache: [kv][pos][head_dim].
#include "attn_merge.h"
#include <algorithm>

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

// RMSNorm (when enabled) and RoPE of one head vector held by one wave: lane l
// holds entries l + 64 k, k < NC.  The sum of squares is a butterfly inside
// the wave; the rotation pairs (d, d +- rope_dims/2) meet through the wave's
// own LDS row rb (LDS operations of one wave take effect in program order), so
// no workgroup barrier is needed.
template <int NC>
__device__ __forceinline__ void head_prep(float (&x)[NC], const AttnParams& p, const float* norm_w, int pos,
                                          float* rb) {
  const int lane = threadIdx.x & 63;
  if (p.qk_norm) {
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < NC; ++k) ss += x[k] * x[k];
    ss = wave_sum(ss);
    const float rn = 1.0f / sqrtf(ss / (float)(64 * NC) + p.eps);
#pragma unroll
    for (int k = 0; k < NC; ++k) x[k] = x[k] * rn * norm_w[lane + 64 * k];
  }
  if (p.rope_dims) {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int k = 0; k < NC; ++k) rb[lane + 64 * k] = x[k];
    asm volatile("" ::: "memory");
    const int half = p.rope_dims / 2;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int d = lane + 64 * k;
      if (d < p.rope_dims) {
        float c, sn;
        rope_cs(p, d, pos, c, sn);
        x[k] = d < half ? rb[d] * c - rb[d + half] * sn : rb[d] * c + rb[d - half] * sn;
      }
    }
    asm volatile("" ::: "memory");
  }
}

// Values of a 32-row chunk.  Thread (dim group vg = tid / 8, row quarter vq =
// tid % 8) holds dims 8 vg .. 8 vg + 7 of rows 4 vq .. 4 vq + 3: four 16-byte
// loads, one per row (a wave's load covers 8 rows x 64 dims, 8 whole lines).
__device__ __forceinline__ void v_request(const AttnParams& p, int g, int r0, int hd, uint4 (&vw)[4]) {
  const int vg = (int)threadIdx.x >> 3, vq = (int)threadIdx.x & 7;
  const __half* base = p.vc + ((size_t)g * p.max_seq + r0 + 4 * vq) * hd + 8 * (8 * vg < hd ? vg : 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) vw[j] = *reinterpret_cast<const uint4*>(base + (size_t)j * hd);
}
// fp32 values; rows at or past nvmax (past the pass's last position) are 0
__device__ __forceinline__ void v_convert(const uint4 (&vw)[4], int nvmax, float (&vf)[4][8]) {
  const int vq = (int)threadIdx.x & 7;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w4[4] = {vw[j].x, vw[j].y, vw[j].z, vw[j].w};
    const bool ok = 4 * vq + j < nvmax;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vf[j][2 * e] = ok ? __half2float(__ushort_as_half((unsigned short)(w4[e] & 0xffff))) : 0.0f;
      vf[j][2 * e + 1] = ok ? __half2float(__ushort_as_half((unsigned short)(w4[e] >> 16))) : 0.0f;
    }
  }
}
// The dimension whose chunk sum this thread ends with in pv_sum.
__device__ __forceinline__ int pv_dim() {
  const int t = (int)threadIdx.x;
  return 8 * (t >> 3) + 4 * (t & 1) + 2 * ((t >> 1) & 1) + ((t >> 2) & 1);
}
// P V of one (token, head) over a chunk: this thread's 8 dims over its 4 rows
// (weights w[4 vq .. 4 vq + 3]), then the 8 row quarters of a dim group (lanes
// l ^ 1, l ^ 2, l ^ 4) are summed in three exchange steps, each lane handing
// on half of its sums and keeping the other half, so that lane l ends with
// the whole sum of dim pv_dim().  A fixed order: the same bits wherever it runs.
__device__ __forceinline__ float pv_sum(const float* w, const float (&vf)[4][8]) {
  const int t = (int)threadIdx.x;
  const float4 p4 = *reinterpret_cast<const float4*>(w + 4 * (t & 7));
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float x = p4.x * vf[0][e];
    x = __builtin_fmaf(p4.y, vf[1][e], x);
    x = __builtin_fmaf(p4.z, vf[2][e], x);
    o[e] = __builtin_fmaf(p4.w, vf[3][e], x);
  }
  const bool b0 = t & 1, b1 = t & 2, b2 = t & 4;
  float a[4], b[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {   // keep dims 4 b0 + i
    const float send = b0 ? o[i] : o[4 + i];
    a[i] = (b0 ? o[4 + i] : o[i]) + xor_lane<1>(send);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {   // keep dims 4 b0 + 2 b1 + i
    const float send = b1 ? a[i] : a[2 + i];
    b[i] = (b1 ? a[2 + i] : a[i]) + xor_lane<2>(send);
  }
  const float send = b2 ? b[0] : b[1];
  return (b2 ? b[1] : b[0]) + xor_lane<4>(send);
}

// One workgroup per (KV head g, group of GRP of its query heads, range of cpw
// consecutive 32-row chunks), 4 waves, for all T (<= TM) tokens of the pass:
//   1. the pass's K/V rows that fall in the range are prepared (wave w takes
//      tokens w, w + 4, ...) and appended to the cache;
//   2. the first chunk's keys (thread (row rr = tid / 8, part = tid % 8): an
//      eighth of the head dimensions of key row rr) and values (v_request: 8
//      dims of 4 rows per thread) are requested;
//   3. every (token, query head) that reaches the range is prepared into LDS
//      once (wave w takes pairs w, w + 4, ...) while those loads are in flight;
//   then chunk after chunk, with the next chunk's keys and values requested
//   as soon as the current ones are in registers:
//   4. scores for every (token, head): the eight parts meet in three butterfly
//      steps; then one wave per (token, head) takes the chunk max, the
//      weights exp(s - max) and their sum;
//   5. P V per (token, head) (pv_sum: each dimension's sum ends in one
//      thread), merged into the range's output.
// Each chunk's (max, sum, P V) is computed by exactly the operations of
// k_attn_split below.  The chunks of a range are then merged in order into
// one partial per (token, head): M' = max(M, m_c), L = L e^(M - M') + l_c
// e^(m_c - M'), O likewise, from M = -inf, L = O = 0; with one chunk per
// range that is the chunk's own partial bit for bit (both factors are exp(0)
// = 1 and 0 * 0 = 0).  The range size comes from the cache size alone, so a
// decode step (all query heads of a KV head per workgroup) and a verify pass
// (two) merge the same chunks in the same order and give the same bits.
// Every group of query heads of a range appends the same rows itself (the
// same bits), so each reads them back after its own stores.
template <int GRP, int HD, int TM>   // GRP: query heads per workgroup; TM: most tokens
__global__ __launch_bounds__(256) void k_attn_split_range(AttnParams p, int T, int cpw) {
  constexpr int C = ATT_CHUNK;
  constexpr int NC = HD / 64;   // entries per lane of a head vector; 8-dim pieces per eighth of the head
  constexpr int TW = (TM + 3) / 4;   // tokens per wave in step 1
  // prepared queries; every 32 floats of a row are followed by 4 of padding,
  // so the eight key parts of a score step (32 floats apart) read 16-byte
  // pieces in eight different bank groups instead of two
  constexpr int QW = HD + HD / 8;
  __shared__ __attribute__((aligned(16))) float qsh[TM][GRP][QW];
  __shared__ __attribute__((aligned(16))) float pl[TM][GRP][C];
  __shared__ float rbuf[4][HD];
  __shared__ float ml[TM][GRP][2];
  __shared__ float run[TM][GRP][2];   // running max and sum of the range
  __shared__ float fac[TM][GRP][2];   // this chunk's rescaling of the running output and of its own
  const int nsub = p.q_heads / p.kv_heads / GRP;   // query-head groups per KV head
  const int nrange = (p.nchunk + cpw - 1) / cpw;
  // Workgroups go to the XCDs round robin by index.  The nsub workgroups that
  // read the same (KV head, range) pair take indices 8 apart, i.e. one XCD and
  // close in time, so the later ones find its keys and values in that XCD's
  // L2: pairs come in groups of 8, each group once per query-head group.
  const int pair = ((int)blockIdx.x / (8 * nsub)) * 8 + (int)blockIdx.x % 8;
  const int sub = ((int)blockIdx.x / 8) % nsub;
  if (pair >= p.kv_heads * nrange) return;
  const int g = pair / nrange, rng = pair % nrange;
  const int cb = rng * cpw;
  const int h0 = (g * nsub + sub) * GRP;            // first query head of this workgroup
  const int p0 = (p.ctrl ? p.ctrl->pos : p.pos) + p.pos_off;
  if (cb * C > p0 + T - 1) return;
  const int ce = min(min(cb + cpw, p.nchunk), (p0 + T - 1) / C + 1);   // chunks [cb, ce) hold visible rows
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_id();
  const bool dact = tid < HD;
  float* rb = rbuf[wave];

  // 1. this pass's K/V rows inside the range: positions p0 + t in [cb C, ce C);
  // wave w takes tokens ta + w + 4 m, all its loads first
  {
    const int ta = max(0, cb * C - p0), tb = min(T, ce * C - p0);
    if (tb > ta) {
      float k[TW][NC], v[TW][NC];
#pragma unroll
      for (int m = 0; m < TW; ++m) {
        const int t = ta + wave + 4 * m;
        if (t < tb) {
          const float* y = p.y + (size_t)t * p.y_stride;
#pragma unroll
          for (int e = 0; e < NC; ++e) {
            k[m][e] = y[p.off_k + g * HD + lane + 64 * e];
            v[m][e] = y[p.off_v + g * HD + lane + 64 * e];
          }
        }
      }
#pragma unroll
      for (int m = 0; m < TW; ++m) {
        const int t = ta + wave + 4 * m;
        if (t < tb) {
          const int pos = p0 + t;
          head_prep<NC>(k[m], p, p.k_norm, pos, rb);
#pragma unroll
          for (int e = 0; e < NC; ++e) {
            const int d = lane + 64 * e;
            p.kc[kidx(g, pos, d, p.max_seq, HD)] = __float2half_rn(k[m][e]);
            p.vc[((size_t)g * p.max_seq + pos) * HD + d] = __float2half_rn(v[m][e]);
          }
        }
      }
      __threadfence_block();
      __syncthreads();
    }
  }

  // 2. the first chunk's keys (this thread's eighth of row rr) and values (8
  // dims of 4 rows); rows past the pass's last position lie inside the cache,
  // get weight 0 and a value of 0
  const int rr = tid >> 3, part = tid & 7;
  uint4 kw[NC];
  uint4 vw[4];
  auto request = [&](int c) {
    const int r = c * C + rr;
#pragma unroll
    for (int i = 0; i < NC; ++i)
      kw[i] = *reinterpret_cast<const uint4*>(p.kc + kidx(g, r, (part * NC + i) * 8, p.max_seq, HD));
    v_request(p, g, c * C, HD, vw);
  };
  request(cb);

  // 3. queries of tokens tq0.. (those whose position reaches the range):
  // pair q = (t - tq0) GRP + h, wave w takes pairs w + 4 m, all its loads first
  const int tq0 = max(0, cb * C - p0);
  float orun[TM][GRP];   // this thread's dimension of the range's output, per (token, head)
#pragma unroll
  for (int t = 0; t < TM; ++t)
#pragma unroll
    for (int h = 0; h < GRP; ++h) orun[t][h] = 0.0f;
  if (tid < TM * GRP) {
    run[tid / GRP][tid % GRP][0] = -INFINITY;
    run[tid / GRP][tid % GRP][1] = 0.0f;
  }
  {
    const int npair = (T - tq0) * GRP;
    constexpr int MQ = (TM * GRP + 3) / 4;
    float x[MQ][NC];
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
      const int q = wave + 4 * m;
      if (q < npair) {
        const float* y = p.y + (size_t)(tq0 + q / GRP) * p.y_stride + p.off_q + (h0 + q % GRP) * HD;
#pragma unroll
        for (int e = 0; e < NC; ++e) x[m][e] = y[lane + 64 * e];
      }
    }
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
      const int q = wave + 4 * m;
      if (q < npair) {
        const int t = tq0 + q / GRP, h = q % GRP;
        head_prep<NC>(x[m], p, p.q_norm, p0 + t, rb);
#pragma unroll
        for (int e = 0; e < NC; ++e) {
          const int d = lane + 64 * e;
          qsh[t][h][d + (d >> 5) * 4] = x[m][e] * (1.0f / sqrtf((float)HD));
        }
      }
    }
  }
  __syncthreads();

  for (int c = cb; c < ce; ++c) {
    const int r0 = c * C;
    const int nvmax = min(C, p0 + T - r0);   // rows valid for the pass's last token
    float kf[NC][8];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const uint32_t ws[4] = {kw[i].x, kw[i].y, kw[i].z, kw[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[i][2 * e] = __half2float(__ushort_as_half((unsigned short)(ws[e] & 0xffff)));
        kf[i][2 * e + 1] = __half2float(__ushort_as_half((unsigned short)(ws[e] >> 16)));
      }
    }
    float vf[4][8];
    v_convert(vw, nvmax, vf);
    if (c + 1 < ce) request(c + 1);
    const int tq = max(0, r0 - p0);
    const int npair = (T - tq) * GRP;

    // 4. scores, then per (token, head) the max, weights and their sum
    for (int t = tq; t < T; ++t) {
      const int nvalid = min(C, p0 + t + 1 - r0);
#pragma unroll
      for (int h = 0; h < GRP; ++h) {
        float sc = 0.0f;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
          const int dc = part * NC + i;
          const int q8 = dc * 8 + (dc >> 2) * 4;   // dims dc*8 .. dc*8+7 lie in one padded group of 32
          const float4 qa = *reinterpret_cast<const float4*>(&qsh[t][h][q8]);
          const float4 qb = *reinterpret_cast<const float4*>(&qsh[t][h][q8 + 4]);
          sc = __builtin_fmaf(kf[i][0], qa.x, sc);
          sc = __builtin_fmaf(kf[i][1], qa.y, sc);
          sc = __builtin_fmaf(kf[i][2], qa.z, sc);
          sc = __builtin_fmaf(kf[i][3], qa.w, sc);
          sc = __builtin_fmaf(kf[i][4], qb.x, sc);
          sc = __builtin_fmaf(kf[i][5], qb.y, sc);
          sc = __builtin_fmaf(kf[i][6], qb.z, sc);
          sc = __builtin_fmaf(kf[i][7], qb.w, sc);
        }
        sc += xor_lane<1>(sc);
        sc += xor_lane<2>(sc);
        sc += xor_lane<4>(sc);
        if (part == 0) pl[t][h][rr] = rr < nvalid ? sc : -INFINITY;
      }
    }
    __syncthreads();
    for (int q = wave; q < npair; q += 4) {
      const int t = tq + q / GRP, h = q % GRP;
      const int nvalid = min(C, p0 + t + 1 - r0);
      const float sc = lane < C ? pl[t][h][lane] : -INFINITY;
      const float m = wave_max(sc);
      const float e = lane < nvalid ? __expf(sc - m) : 0.0f;
      if (lane < C) pl[t][h][lane] = e;
      const float l = wave_sum(e);
      if (lane == 0) {
        // merge into the range: running max M' and the two rescaling factors
        const float M = run[t][h][0];
        const float Mn = fmaxf(M, m);
        const float fa = __expf(M - Mn), fb = __expf(m - Mn);
        fac[t][h][0] = fa;
        fac[t][h][1] = fb;
        run[t][h][0] = Mn;
        run[t][h][1] = __builtin_fmaf(run[t][h][1], fa, l * fb);
      }
    }
    __syncthreads();

    // 5. P V, merged into the range's output (this thread: dim pv_dim())
    if (dact) {
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        if (t < tq || t >= T) continue;
#pragma unroll
        for (int h = 0; h < GRP; ++h) {
          const float o = pv_sum(pl[t][h], vf);
          orun[t][h] = __builtin_fmaf(orun[t][h], fac[t][h][0], o * fac[t][h][1]);
        }
      }
    }
    __syncthreads();   // pl, ml and fac are rewritten by the next chunk
  }

  // the range's partial for every (token, head) that reached it
  if (dact) {
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      if (t < tq0 || t >= T) continue;
#pragma unroll
      for (int h = 0; h < GRP; ++h) {
        float* dst = p.part + (((size_t)t * p.q_heads + h0 + h) * p.nchunk + rng) * (HD + 2);
        dst[2 + pv_dim()] = orun[t][h];
        if (tid == 0) { dst[0] = run[t][h][0]; dst[1] = run[t][h][1]; }
      }
    }
  }
}

// One workgroup per (KV head g, group of GRP of its query heads, 32-row chunk
// c), 4 waves, for all T tokens of the pass at once:
//   1. the pass's K/V rows that fall in the chunk are prepared (wave w takes
//      tokens w, w + 4, ...) and appended to the cache;
//   2. the chunk's keys (thread (row rr = tid / 8, part = tid % 8): an eighth
//      of the head dimensions of key row rr) and values (v_request: 8 dims of
//      4 rows per thread) are requested once;
//   3. every (token, query head) is prepared into LDS (wave w takes pairs w,
//      w + 4, ...) while those loads are in flight;
//   4. scores for every (token, head): the eight parts meet in three butterfly
//      steps; then one wave per (token, head) takes the chunk max, the
//      weights exp(s - max) and their sum;
//   5. P V per (token, head) (pv_sum: each dimension's sum ends in one thread).
// Four workgroup barriers in all, whatever T.  Every group of query heads of
// the chunk appends the same rows itself (the same bits), so each reads them
// back after its own stores.
template <int GRP, int HD>   // GRP: query heads per workgroup
__global__ __launch_bounds__(256) void k_attn_split(AttnParams p, int T) {
  constexpr int C = ATT_CHUNK;
  constexpr int NC = HD / 64;   // entries per lane of a head vector; 8-dim pieces per eighth of the head
  // prepared queries; every 32 floats of a row are followed by 4 of padding,
  // so the eight key parts of a score step (32 floats apart) read 16-byte
  // pieces in eight different bank groups instead of two
  constexpr int QW = HD + HD / 8;
  __shared__ __attribute__((aligned(16))) float qsh[MAX_T][GRP][QW];
  __shared__ __attribute__((aligned(16))) float pl[MAX_T][GRP][C];
  __shared__ float rbuf[4][HD];
  __shared__ float ml[MAX_T][GRP][2];
  const int nsub = p.q_heads / p.kv_heads / GRP;   // query-head groups per KV head
  // Workgroups go to the XCDs round robin by index.  The nsub workgroups that
  // read the same (KV head, chunk) pair take indices 8 apart, i.e. one XCD and
  // close in time, so the later ones find its keys and values in that XCD's
  // L2: pairs come in groups of 8, each group once per query-head group.
  const int pair = ((int)blockIdx.x / (8 * nsub)) * 8 + (int)blockIdx.x % 8;
  const int sub = ((int)blockIdx.x / 8) % nsub;
  if (pair >= p.kv_heads * p.nchunk) return;
  const int g = pair / p.nchunk, c = pair % p.nchunk;
  const int h0 = (g * nsub + sub) * GRP;            // first query head of this workgroup
  const int p0 = (p.ctrl ? p.ctrl->pos : p.pos) + p.pos_off;
  const int r0 = c * C;
  if (r0 > p0 + T - 1) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_id();
  const bool dact = tid < HD;
  float* rb = rbuf[wave];

  // 1. this pass's K/V rows inside the chunk: positions p0 + t in [r0, r0 + C);
  // wave w takes tokens ta + w + 4 m, all its loads first
  const int ta = max(0, r0 - p0), tb = min(T, r0 + C - p0);
  if (tb > ta) {
    float k[MAX_T / 4][NC], v[MAX_T / 4][NC];
#pragma unroll
    for (int m = 0; m < MAX_T / 4; ++m) {
      const int t = ta + wave + 4 * m;
      if (t < tb) {
        const float* y = p.y + (size_t)t * p.y_stride;
#pragma unroll
        for (int e = 0; e < NC; ++e) {
          k[m][e] = y[p.off_k + g * HD + lane + 64 * e];
          v[m][e] = y[p.off_v + g * HD + lane + 64 * e];
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MAX_T / 4; ++m) {
      const int t = ta + wave + 4 * m;
      if (t < tb) {
        const int pos = p0 + t;
        head_prep<NC>(k[m], p, p.k_norm, pos, rb);
#pragma unroll
        for (int e = 0; e < NC; ++e) {
          const int d = lane + 64 * e;
          p.kc[kidx(g, pos, d, p.max_seq, HD)] = __float2half_rn(k[m][e]);
          p.vc[((size_t)g * p.max_seq + pos) * HD + d] = __float2half_rn(v[m][e]);
        }
      }
    }
    __threadfence_block();
    __syncthreads();
  }

  // 2. the chunk's keys (this thread's eighth of row rr) and values (8 dims
  // of 4 rows) are requested now and converted after the queries are
  // prepared; rows past the pass's last position lie inside the cache, get
  // weight 0 and a value of 0
  const int rr = tid >> 3, part = tid & 7;
  const int r = r0 + rr;
  uint4 kw[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i)
    kw[i] = *reinterpret_cast<const uint4*>(p.kc + kidx(g, r, (part * NC + i) * 8, p.max_seq, HD));
  const int nvmax = min(C, p0 + T - r0);   // rows valid for the pass's last token
  uint4 vw[4];
  v_request(p, g, r0, HD, vw);

  // 3. queries of tokens tq.. (those whose position reaches this chunk):
  // pair q = (t - tq) GRP + h, wave w takes pairs w + 4 m, all its loads first
  const int tq = max(0, r0 - p0);
  const int npair = (T - tq) * GRP;
  {
    constexpr int MQ = MAX_T * GRP / 4;
    float x[MQ][NC];
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
      const int q = wave + 4 * m;
      if (q < npair) {
        const float* y = p.y + (size_t)(tq + q / GRP) * p.y_stride + p.off_q + (h0 + q % GRP) * HD;
#pragma unroll
        for (int e = 0; e < NC; ++e) x[m][e] = y[lane + 64 * e];
      }
    }
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
      const int q = wave + 4 * m;
      if (q < npair) {
        const int t = tq + q / GRP, h = q % GRP;
        head_prep<NC>(x[m], p, p.q_norm, p0 + t, rb);
#pragma unroll
        for (int e = 0; e < NC; ++e) {
          const int d = lane + 64 * e;
          qsh[t][h][d + (d >> 5) * 4] = x[m][e] * (1.0f / sqrtf((float)HD));
        }
      }
    }
  }
  __syncthreads();
  float kf[NC][8];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const uint32_t ws[4] = {kw[i].x, kw[i].y, kw[i].z, kw[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kf[i][2 * e] = __half2float(__ushort_as_half((unsigned short)(ws[e] & 0xffff)));
      kf[i][2 * e + 1] = __half2float(__ushort_as_half((unsigned short)(ws[e] >> 16)));
    }
  }
  float vf[4][8];
  v_convert(vw, nvmax, vf);

  // 4. scores, then per (token, head) the max, weights and their sum
  for (int t = tq; t < T; ++t) {
    const int nvalid = min(C, p0 + t + 1 - r0);
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      float sc = 0.0f;
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int dc = part * NC + i;
        const int q8 = dc * 8 + (dc >> 2) * 4;   // dims dc*8 .. dc*8+7 lie in one padded group of 32
        const float4 qa = *reinterpret_cast<const float4*>(&qsh[t][h][q8]);
        const float4 qb = *reinterpret_cast<const float4*>(&qsh[t][h][q8 + 4]);
        sc = __builtin_fmaf(kf[i][0], qa.x, sc);
        sc = __builtin_fmaf(kf[i][1], qa.y, sc);
        sc = __builtin_fmaf(kf[i][2], qa.z, sc);
        sc = __builtin_fmaf(kf[i][3], qa.w, sc);
        sc = __builtin_fmaf(kf[i][4], qb.x, sc);
        sc = __builtin_fmaf(kf[i][5], qb.y, sc);
        sc = __builtin_fmaf(kf[i][6], qb.z, sc);
        sc = __builtin_fmaf(kf[i][7], qb.w, sc);
      }
      sc += xor_lane<1>(sc);
      sc += xor_lane<2>(sc);
      sc += xor_lane<4>(sc);
      if (part == 0) pl[t][h][rr] = rr < nvalid ? sc : -INFINITY;
    }
  }
  __syncthreads();
  for (int q = wave; q < npair; q += 4) {
    const int t = tq + q / GRP, h = q % GRP;
    const int nvalid = min(C, p0 + t + 1 - r0);
    const float sc = lane < C ? pl[t][h][lane] : -INFINITY;
    const float m = wave_max(sc);
    const float e = lane < nvalid ? __expf(sc - m) : 0.0f;
    if (lane < C) pl[t][h][lane] = e;
    const float l = wave_sum(e);
    if (lane == 0) { ml[t][h][0] = m; ml[t][h][1] = l; }
  }
  __syncthreads();

  // 5. P V (this thread: dim pv_dim())
  if (dact) {
    for (int t = tq; t < T; ++t) {
#pragma unroll
      for (int h = 0; h < GRP; ++h) {
        const float o = pv_sum(pl[t][h], vf);
        float* dst = p.part + (((size_t)t * p.q_heads + h0 + h) * p.nchunk + c) * (HD + 2);
        dst[2 + pv_dim()] = o;
        if (tid == 0) { dst[0] = ml[t][h][0]; dst[1] = ml[t][h][1]; }
      }
    }
  }
}

// One workgroup of CW waves per (token, query head, 64 dimensions): merge the
// chunks, normalise, apply the gate and quantise the two 32-dim blocks.
//
// Up to 64 chunks (2048 rows) wave 0 does it alone: lane c loads chunk c's max
// and sum, the weights exp(m_c - M) go through LDS, and every lane then folds
// its dimension over the chunks in order.  The gate input, the statistics and
// the first 32 chunks' values are all requested before the statistics are
// used, so this costs one memory round trip after the position is read.
//
// Beyond 64 chunks wave w of the NW = blockDim / 64 waves takes the
// contiguous chunk range [nc w / NW, nc (w+1) / NW): the waves' maxima, their
// sums of weighted chunk sums and their partial outputs meet in LDS in wave
// order, and wave 0 finishes.  32 value loads per wave are in flight at a
// time.  The launch takes CW waves when the cache holds more than 64
// partials (chunks, or ranges of chunks on long caches), else one (the long
// branch is then never taken), so a slice's decode and verify steps always
// sum in the same order.
constexpr int CW = 8;
__global__ __launch_bounds__(64 * CW) void k_attn_combine(AttnParams p) {
  __shared__ float wsh[2048];
  __shared__ float red[CW][64];
  __shared__ float mred[CW], lred[CW];
  const int ndg = p.hd / 64;
  const int t = blockIdx.x / (p.q_heads * ndg);
  const int h = (blockIdx.x / ndg) % p.q_heads;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int d = (blockIdx.x % ndg) * 64 + lane;
  const int P = (p.ctrl ? p.ctrl->pos : p.pos) + p.pos_off + t;
  const int nc = P / ATT_CHUNK / p.rchunks + 1;   // partials that token t reaches
  if (nc <= 64) {   // one wave
    if (w == 0) merge_wave<false>(p, t, h, (blockIdx.x % ndg) * 64, nc, wsh);
    return;
  }
  // the gate input does not depend on the position
  const float gz = p.off_g >= 0 && w == 0 ? p.y[(size_t)t * p.y_stride + p.off_g + h * p.hd + d] : 0.0f;
  const int stride = p.hd + 2;
  const float* base = p.part + ((size_t)t * p.q_heads + h) * p.nchunk * stride;
  float o = 0.0f, L = 0.0f;
  {
    const int c_lo = nc * w / nw, c_hi = nc * (w + 1) / nw;
    float mw = -INFINITY;
    for (int c = c_lo + lane; c < c_hi; c += 64) mw = fmaxf(mw, base[(size_t)c * stride]);
    mw = wave_max(mw);
    if (lane == 0) mred[w] = mw;
    __syncthreads();
    float M = mred[0];
#pragma unroll
    for (int x = 1; x < CW; ++x)
      if (x < nw) M = fmaxf(M, mred[x]);
    float lw = 0.0f;
    for (int c0 = c_lo; c0 < c_hi; c0 += 64) {
      const int c = c0 + lane;
      float wt = 0.0f, l = 0.0f;
      if (c < c_hi) {
        wt = __expf(base[(size_t)c * stride] - M);
        l = base[(size_t)c * stride + 1];
      }
      lw += wave_sum(l * wt);
      if (c < c_hi && c < 2048) wsh[c] = wt;
    }
    if (lane == 0) lred[w] = lw;
    __syncthreads();
    // the wave's weighted values in chunk order
    for (int c0 = c_lo; c0 < c_hi; c0 += 32) {
      float v[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) v[u] = c0 + u < c_hi ? base[(size_t)(c0 + u) * stride + 2 + d] : 0.0f;
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int c = c0 + u;
        if (c < c_hi) o = __builtin_fmaf(v[u], c < 2048 ? wsh[c] : __expf(base[(size_t)c * stride] - M), o);
      }
    }
    red[w][lane] = o;
    __syncthreads();
    if (w != 0) return;
    L = lred[0];
    o = red[0][lane];
#pragma unroll
    for (int x = 1; x < CW; ++x)
      if (x < nw) {
        L += lred[x];
        o += red[x][lane];
      }
  }
  o = o / L;
  if (p.off_g >= 0) o = o * sigmoidf_(gz);
  const int nu = p.q_heads * p.hd;
  if (p.u_out) p.u_out[(size_t)t * nu + h * p.hd + d] = o;
  const int blk = (h * p.hd + d) / QK;
  if (p.next.xd) put_digits(p.next, p.next_qt, t, blk, o, true);
}

hipError_t launch_attention(const AttnParams& p, int T, hipStream_t s) {
  if (p.hd % 64 || p.hd > 256 || p.rope_dims % 2 || p.rope_dims > p.hd || p.max_seq % 64 ||
      p.nchunk * ATT_CHUNK < p.max_seq || (p.rope_dims && !p.rope_cs) ||
      p.q_heads % p.kv_heads || T < 1 || T > MAX_T || (p.split_only && (T != 1 || p.nchunk > 64)))
    return hipErrorInvalidValue;
  // Chunks per partial, from the cache size alone (decode and verify must
  // merge alike): one up to 1024 (KV head, chunk) pairs, beyond that enough
  // that about 512 ranges remain (a sweep of 256 to 4096 at 32768 rows on
  // MI355X: 512 is the fastest for one query, 51 us, and for sixteen, 460 us;
  // the decode grid then fits the machine's resident workgroups at once).  A
  // partial is 4 (hd + 2) bytes per token and head: per 32-row chunk that is
  // three times its K/V for 16 tokens, so long caches merge their chunks in the
  // split kernel.
  const int grp = p.q_heads / p.kv_heads;
  const int npairs = p.kv_heads * p.nchunk;
  const int R = npairs > 1024 ? std::min(16, (npairs + 511) / 512) : 1;
  if (p.split_only && R != 1) return hipErrorInvalidValue;
  AttnParams q = p;
  q.rchunks = R;
  // Query heads per split workgroup: with one token on a cache of at least
  // 512 pairs, all of a KV head's group (its keys and values are then read
  // once per chunk: 100.6 -> 71.9 us at 32768 rows, 22.3 -> 17.2 at 4096 on
  // MI355X); otherwise at most 2 (more workgroups for a short cache, 9.6
  // against 11.6 us at 512 rows; and the prepared queries of 16 tokens fill
  // LDS).  The range kernel runs whenever chunks are merged or all heads go
  // to one workgroup; the per-chunk kernel otherwise.
  const bool all_heads = T == 1 && npairs >= 512 &&
                         (grp == 1 || grp == 2 || grp == 3 || grp == 4 || grp == 6 || grp == 8);
  const bool range = R > 1 || all_heads;
  const int hpw = all_heads ? grp : (grp % 2 == 0 ? 2 : 1);
  const int nsub = grp / hpw;
  const int nrange = (p.nchunk + R - 1) / R;
  const int pairs = p.kv_heads * (range ? nrange : p.nchunk);   // padded to groups of 8
  const unsigned grid = (unsigned)(((pairs + 7) / 8) * 8 * nsub);
#define SLQ_R1(n, hd) case n: k_attn_split_range<n, hd, 1><<<grid, 256, 0, s>>>(q, T, R); break;
#define SLQ_RT(n, hd) case n: k_attn_split_range<n, hd, MAX_T><<<grid, 256, 0, s>>>(q, T, R); break;
#define SLQ_G(n, hd) case n: k_attn_split<n, hd><<<grid, 256, 0, s>>>(q, T); break;
#define SLQ_HD(hd)                                                                  \
  case hd:                                                                          \
    if (range && T == 1) {                                                          \
      switch (hpw) {                                                                \
        SLQ_R1(1, hd) SLQ_R1(2, hd) SLQ_R1(3, hd) SLQ_R1(4, hd) SLQ_R1(6, hd) SLQ_R1(8, hd) \
        default: return hipErrorInvalidValue;                                       \
      }                                                                             \
    } else if (range) {                                                             \
      switch (hpw) {                                                                \
        SLQ_RT(1, hd) SLQ_RT(2, hd)                                                 \
        default: return hipErrorInvalidValue;                                       \
      }                                                                             \
    } else {                                                                        \
      switch (hpw) {                                                                \
        SLQ_G(1, hd) SLQ_G(2, hd)                                                   \
        default: return hipErrorInvalidValue;                                       \
      }                                                                             \
    }                                                                               \
    break;
  switch (p.hd) {
    SLQ_HD(64) SLQ_HD(128) SLQ_HD(192) SLQ_HD(256)
    default: return hipErrorInvalidValue;
  }
#undef SLQ_HD
#undef SLQ_G
#undef SLQ_RT
#undef SLQ_R1
  // the chained decode kernel merges (merge_wave) what the split leaves
  if (!p.split_only) k_attn_combine<<<T * p.q_heads * (p.hd / 64), nrange > 64 ? 64 * CW : 64, 0, s>>>(q);
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
