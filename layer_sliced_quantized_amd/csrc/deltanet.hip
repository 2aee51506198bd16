// Gated DeltaNet recurrent update for decode, verify and prompt ingestion.
//
// The hybrid model's linear-attention layers are Gated DeltaNet (ChatTorrent
// README, "What it can run").  Each head carries a state S (d_v x d_k, fp32)
// that is updated once per token, one token after the other (the pages name
// this serial recurrence as the reason prompt ingestion is slow; SwarmLLM
// README, bench paragraph):
//     S' = alpha S (I - beta k k^T) + beta v k^T,   o = S' q
// with q, k divided by sqrt(sum of squares + 1e-6).  Row i of S only needs the
// whole k and q plus v_i, so rows are independent:
//     u_i = S_i . k,   S'_ij = alpha S_ij + beta (v_i - alpha u_i) k_j,   o_i = S'_i . q
// Eight lanes of one wave own one row i, each with an eighth of the j range
// (the state lives in registers across the tokens of a verify pass), and
// meet in three butterfly steps, so a token needs no workgroup barrier.
//
// State layout in HBM: [slot][head][i / 8][jj][part][i % 8] with
// j = part * (d_k / 8) + jj, so that for one jj a wave's 64 lanes (8 parts x
// 8 rows) load and store 256 contiguous bytes.  Decode updates slot `cur` in
// place; verify writes the state after token t to slot (cur + 1 + t) mod
// nslots and never touches slot `cur`, which is what makes rollback exact.
// Prompt ingestion takes the chunked form further down (k_deltanet_chunk).
#include "deltanet.h"

namespace slq {

template <int DKP>
__global__ __launch_bounds__(256) void k_deltanet(DnParams p, int T) {
  deltanet_rows<DKP, MAX_T, false>(p, T, (int)blockIdx.x);
}

// Prompt ingestion: the T tokens of a pass at once (chunked form).
//
// Unrolling the row recurrence above over a chunk of T tokens, with
// g(t, s) = alpha_{s+1} ... alpha_t (g(t, t) = 1) and gamma_t = alpha_0 ... alpha_t,
// every state in the chunk is S0 plus rank-one terms:
//     S_t = gamma_t S0 + sum_{s<=t} g(t, s) c_s k_s^T,
// and the increments c_t (one value per row) solve a unit lower-triangular
// system that is the same for all rows of a head:
//     c_t + beta_t sum_{s<t} g(t, s) (k_t . k_s) c_s = beta_t (v_t - gamma_t S0 k_t).
// Then o_t = gamma_t S0 q_t + sum_{s<=t} g(t, s) (k_s . q_t) c_s.  This is the
// chunkwise (UT-transform) form of the delta rule published for DeltaNet and
// Gated DeltaNet (Yang et al., "Parallelizing Linear Transformers with the
// Delta Rule over Sequence Length", 2024; "Gated Delta Networks", 2025), here
// solved by forward substitution per row.  Only the final state is stored
// (slot cur, in place); a row's 2T dot products with S0 meet in one set of
// butterflies instead of 2T dependent ones, and no state is written per token.
// The result equals the recurrence up to rounding order, not bit for bit.
template <int DKP>
__global__ __launch_bounds__(1024) void k_deltanet_chunk(DnParams p, int T) {
  constexpr int DK = 8 * DKP;
  constexpr int DKS = DK + 4;          // padded LDS row: rows of different tokens start in different banks
  constexpr int JQ = DK / 4;           // key range of one coefficient partial
  constexpr int JJ = DKP / 4;          // state entries a lane finalises
  // Tokens T..MAX_T-1 are padding with q = k = v = 0, alpha = 1, beta = 0:
  // their increments are zero and they change neither the outputs of real
  // tokens nor the final state, so the loops run over MAX_T tokens.
  __shared__ float qs[MAX_T][DKS], ksh[MAX_T][DKS];
  __shared__ float vsh[MAX_T][32], zsh[MAX_T][32];
  __shared__ float al[MAX_T], be[MAX_T];
  __shared__ float pk[4][MAX_T * MAX_T], pq[4][MAX_T * MAX_T];   // k_t.k_s, k_s.q_t over key quarters
  __shared__ float Am[MAX_T][MAX_T];   // beta_t g(t, s) k_t.k_s for s < t, else 0
  __shared__ float Mm[MAX_T][MAX_T];   // g(t, s) k_s.q_t for s <= t, else 0
  __shared__ float wkl[MAX_T][32], wql[MAX_T][32];   // S0_i . k_t, S0_i . q_t
  __shared__ float csh[MAX_T][32];     // c_t
  __shared__ float osh[MAX_T][32];
  const int nib = p.dv / 32;
  const int h = blockIdx.x / nib, ib = blockIdx.x % nib;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int rg = w & 3, tg = w >> 2;   // rows 8 rg .. 8 rg + 7; tokens (and state entries) of quarter tg
  const int part = lane >> 3, r = lane & 7;
  const int ii = rg * 8 + r;
  const int i = ib * 32 + ii;
  const int cur = p.ctrl ? p.ctrl->cur : 0;
  const size_t hs = (size_t)DK * p.dv;
  float* Sp = p.state + ((size_t)cur * p.heads + h) * hs;
  const int j0 = part * DKP;
  const size_t sbase = dn_off(i, j0, DKP);

  float S[DKP];
#pragma unroll
  for (int jj = 0; jj < DKP; ++jj) S[jj] = Sp[sbase + (size_t)jj * 64];

  // wave w normalises q, k of token w; v (threads 0..511) and z (512..1023)
  // of token (tid / 32) % 16, row tid % 32; gates of token tid
  {
    float q0 = 0.0f, q1 = 0.0f, k0 = 0.0f, k1 = 0.0f;
    if (w < T) {
      const float* y = p.y + (size_t)w * p.y_stride;
      if (lane < DK) { q0 = y[p.off_q + h * DK + lane]; k0 = y[p.off_k + h * DK + lane]; }
      if (lane + 64 < DK) { q1 = y[p.off_q + h * DK + lane + 64]; k1 = y[p.off_k + h * DK + lane + 64]; }
    }
    const int t2 = (tid >> 5) & 15, row = tid & 31;
    float x = 0.0f;
    if (t2 < T) x = p.y[(size_t)t2 * p.y_stride + (tid < 512 ? p.off_v : p.off_z) + h * p.dv + ib * 32 + row];
    if (tid < 512) vsh[t2][row] = x;
    else zsh[t2][row] = x;
    if (tid < MAX_T) {
      float a_ = 1.0f, b_ = 0.0f;
      if (tid < T) {
        const float* y = p.y + (size_t)tid * p.y_stride;
        a_ = sigmoidf_(p.a_scale * y[p.off_a + h] + p.a_bias);
        b_ = sigmoidf_(p.b_scale * y[p.off_b + h]);
      }
      al[tid] = a_;
      be[tid] = b_;
    }
    const float sq = wave_sum(q0 * q0 + q1 * q1), sk = wave_sum(k0 * k0 + k1 * k1);
    const float rq = 1.0f / sqrtf(sq + 1e-6f), rk = 1.0f / sqrtf(sk + 1e-6f);
    if (lane < DK) { qs[w][lane] = q0 * rq; ksh[w][lane] = k0 * rk; }
    if (lane + 64 < DK) { qs[w][lane + 64] = q1 * rq; ksh[w][lane + 64] = k1 * rk; }
  }
  __syncthreads();

  // decays: gamma_t = alpha_0 ... alpha_t, g(T-1, t) = alpha_{t+1} ... alpha_{MAX_T-1}
  float a[MAX_T], gam[MAX_T], gend[MAX_T];
#pragma unroll
  for (int t = 0; t < MAX_T; ++t) a[t] = al[t];
  gam[0] = a[0];
#pragma unroll
  for (int t = 1; t < MAX_T; ++t) gam[t] = gam[t - 1] * a[t];
  gend[MAX_T - 1] = 1.0f;
#pragma unroll
  for (int t = MAX_T - 2; t >= 0; --t) gend[t] = gend[t + 1] * a[t + 1];

  // partial k_t.k_s and k_s.q_t: thread (quarter, t, s) = (tid / 256, (tid / 16) % 16, tid % 16)
  {
    const int pr = tid & 255, qq = tid >> 8;
    const int t = pr >> 4, s2 = pr & 15;
    float kk = 0.0f, kq = 0.0f;
#pragma unroll 8
    for (int j = qq * JQ; j < qq * JQ + JQ; ++j) {
      const float ks = ksh[s2][j];
      kk = __builtin_fmaf(ksh[t][j], ks, kk);
      kq = __builtin_fmaf(ks, qs[t][j], kq);
    }
    pk[qq][pr] = kk;
    pq[qq][pr] = kq;
  }
  // S0_i . k_t and S0_i . q_t for the wave's four tokens: partial dots, then
  // the eight parts of the row meet
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int t = tg * 4 + m;
    float a_ = 0.0f, b_ = 0.0f;
#pragma unroll
    for (int jj = 0; jj < DKP; ++jj) {
      a_ = __builtin_fmaf(S[jj], ksh[t][j0 + jj], a_);
      b_ = __builtin_fmaf(S[jj], qs[t][j0 + jj], b_);
    }
    a_ = row_sum8(a_);
    b_ = row_sum8(b_);
    if (part == 0) {
      wkl[t][ii] = a_;
      wql[t][ii] = b_;
    }
  }
  __syncthreads();

  // the head's coefficients (decay products formed directly: a ratio of
  // cumulative products could underflow)
  if (tid < MAX_T * MAX_T) {
    const int t = tid >> 4, s2 = tid & 15;
    float g = 1.0f;
#pragma unroll
    for (int x = 1; x < MAX_T; ++x) g *= (x > s2 && x <= t) ? a[x] : 1.0f;
    const float kk = ((pk[0][tid] + pk[1][tid]) + pk[2][tid]) + pk[3][tid];
    const float kq = ((pq[0][tid] + pq[1][tid]) + pq[2][tid]) + pq[3][tid];
    Am[t][s2] = s2 < t ? be[t] * g * kk : 0.0f;
    Mm[t][s2] = s2 <= t ? g * kq : 0.0f;
  }
  __syncthreads();

  // increments by forward substitution, one lane per row
  if (tid < 32) {
    float c[MAX_T];
#pragma unroll
    for (int t = 0; t < MAX_T; ++t) {
      float x = be[t] * (vsh[t][tid] - gam[t] * wkl[t][tid]);
#pragma unroll
      for (int s2 = 0; s2 < t; ++s2) x = __builtin_fmaf(-Am[t][s2], c[s2], x);
      c[t] = x;
      csh[t][tid] = x;
    }
  }
  __syncthreads();

  // gated outputs: thread (token, row) = (tid / 32, tid % 32) for tid < 512
  if (tid < MAX_T * 32) {
    const int t = tid >> 5, row = tid & 31;
    float o = gam[t] * wql[t][row];
#pragma unroll
    for (int s2 = 0; s2 < MAX_T; ++s2) o = __builtin_fmaf(Mm[t][s2], csh[s2][row], o);
    osh[t][row] = o * sigmoidf_(p.z_scale * zsh[t][row]);
  }
  // final state, in place: the wave's quarter of each lane's entries
  {
    float cc[MAX_T];
#pragma unroll
    for (int t = 0; t < MAX_T; ++t) cc[t] = csh[t][ii] * gend[t];
    const float gall = gam[MAX_T - 1];
#pragma unroll
    for (int jj = 0; jj < DKP; ++jj) {
      if (jj / JJ != tg) continue;
      float x = gall * S[jj];
#pragma unroll
      for (int t = 0; t < MAX_T; ++t) x = __builtin_fmaf(cc[t], ksh[t][j0 + jj], x);
      Sp[sbase + (size_t)jj * 64] = x;
    }
  }

  __syncthreads();

  // digits: token w by wave w; lanes l and l + 32 hold row l's value
  if (w < T) {
    const int blk = (h * p.dv + ib * 32) / QK;
    const float uo = osh[w][lane & 31];
    if (p.u_out && lane < 32) p.u_out[(size_t)w * (p.heads * p.dv) + h * p.dv + ib * 32 + lane] = uo;
    if (p.next.xd) put_digits(p.next, p.next_qt, w, blk, uo, lane < 32);
  }
}

// The qwen3_5 form (DnParams::variant = 1): one workgroup per value head h,
// dv / 8 waves with eight lanes per row of S as in deltanet_rows, the T
// tokens in order.  Per token:
//   1. conv: thread c < 2 dk + dv owns channel c of this head's q | k | v
//      (q, k of query/key head kh = h / (heads / k_heads)); it keeps the
//      channel's last conv - 1 inputs, applies the taps to them (oldest
//      first) and to the new input, then SiLU.  Every value head keeps its own
//      copy of the q and k windows, so no two workgroups share state.  The
//      windows go to the conv-state slot of the token (decode: slot cur in
//      place; verify: slot (cur + 1 + t), slot cur untouched).
//   2. q and k L2-normalised (one wave each), q scaled by 1/sqrt(dk); alpha =
//      exp(-exp(A_log) softplus(a_scale a + dt_bias)), beta = sigmoid(b_scale b);
//   3. the row update of deltanet_rows;
//   4. rmsnorm of the head's output over its dv rows, times the weights and
//      silu(z_scale z), quantised into the output digits.
// Conv-state slot layout: [head][2 dk + dv channels][conv - 1], oldest first.
template <int DKP>
__global__ __launch_bounds__(1024) void k_deltanet_q35(DnParams p, int T) {
  constexpr int DK = 8 * DKP;
  __shared__ float qraw[DK], kraw[DK], qs[DK], ksh[DK];
  __shared__ float vsh[128], zsh[128], osh[128];
  __shared__ float sc[3];
  const int h = blockIdx.x;
  const int kh = h / (p.heads / p.k_heads);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int part = lane >> 3, r = lane & 7;
  const int i = wave * 8 + r;     // row of S (value index); the launch has dv / 8 waves
  const int K = p.conv;
  const int nch = 2 * DK + p.dv;  // this head's conv channels
  const int nv = p.heads * p.dv;
  const int cur = p.ctrl ? p.ctrl->cur : 0;

  // 1. this thread's conv channel: taps, window, and where its input lies in y
  int yoff = -1;
  if (tid < DK) yoff = p.off_q + kh * DK + tid;
  else if (tid < 2 * DK) yoff = p.off_k + kh * DK + (tid - DK);
  else if (tid < nch) yoff = p.off_v + h * p.dv + (tid - 2 * DK);
  const int cglob = tid < DK ? kh * DK + tid
                  : tid < 2 * DK ? p.k_heads * DK + kh * DK + (tid - DK)
                                 : 2 * p.k_heads * DK + h * p.dv + (tid - 2 * DK);
  const size_t cst = ((size_t)h * nch + tid) * (K - 1);   // this channel's window inside a slot
  float win[3] = {0.0f, 0.0f, 0.0f}, taps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (yoff >= 0) {
    const float* st = p.conv_state + (size_t)cur * p.conv_slot + cst;
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (j < K - 1) win[j] = st[j];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < K) taps[j] = p.conv_w[(size_t)cglob * K + j];
  }
  const size_t hs = (size_t)DK * p.dv;
  const float* S_in = p.state + ((size_t)cur * p.heads + h) * hs;
  const int j0 = part * DKP;
  const size_t sbase = dn_off(i, j0, DKP);
  float S[DKP];
#pragma unroll
  for (int jj = 0; jj < DKP; ++jj) S[jj] = S_in[sbase + (size_t)jj * 64];
  const float wn = tid < p.dv ? p.norm_w[tid] : 0.0f;
  const float a_coef = expf(p.a_log[h]), dtb = p.dt_bias[h];

  for (int t = 0; t < T; ++t) {
    const float* y = p.y + (size_t)t * p.y_stride;
    if (yoff >= 0) {
      const float x = y[yoff];
      float c = 0.0f;
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (j < K - 1) c = __builtin_fmaf(taps[j], win[j], c);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j == K - 1) c = __builtin_fmaf(taps[j], x, c);
      const float sv = c / (1.0f + expf(-c));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (j + 1 < K - 1) win[j] = win[j + 1];
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (j == K - 2) win[j] = x;
      float* dst = p.conv_state + (size_t)(p.mode == DN_VERIFY ? (cur + 1 + t) % p.nslots : cur) * p.conv_slot + cst;
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (j < K - 1) dst[j] = win[j];
      if (tid < DK) qraw[tid] = sv;
      else if (tid < 2 * DK) kraw[tid - DK] = sv;
      else vsh[tid - 2 * DK] = sv;
    }
    if (tid < p.dv) zsh[tid] = p.z_scale * y[p.off_z + h * p.dv + tid];
    if (tid == 0) {
      const float av = p.a_scale * y[p.off_a + h] + dtb;
      const float spl = av > 20.0f ? av : log1pf(expf(av));
      sc[0] = expf(-a_coef * spl);
      sc[1] = sigmoidf_(p.b_scale * y[p.off_b + h]);
    }
    __syncthreads();
    // 2. q (wave 0) and k (wave 1) normalised
    if (wave < 2) {
      const float* src = wave == 0 ? qraw : kraw;
      const float a0 = lane < DK ? src[lane] : 0.0f, a1 = lane + 64 < DK ? src[lane + 64] : 0.0f;
      const float ss = wave_sum(a0 * a0 + a1 * a1);
      float rn = 1.0f / sqrtf(ss + 1e-6f);
      if (wave == 0) rn *= 1.0f / sqrtf((float)DK);
      float* dst = wave == 0 ? qs : ksh;
      if (lane < DK) dst[lane] = a0 * rn;
      if (lane + 64 < DK) dst[lane + 64] = a1 * rn;
    }
    __syncthreads();
    // 3. the rows of S
    const float alpha = sc[0], beta = sc[1];
    float up = 0.0f;
#pragma unroll
    for (int jj = 0; jj < DKP; ++jj) up = __builtin_fmaf(S[jj], ksh[j0 + jj], up);
    up = row_sum8(up);
    const float cc = beta * (vsh[i] - alpha * up);
    float op = 0.0f;
#pragma unroll
    for (int jj = 0; jj < DKP; ++jj) {
      S[jj] = __builtin_fmaf(cc, ksh[j0 + jj], alpha * S[jj]);
      op = __builtin_fmaf(S[jj], qs[j0 + jj], op);
    }
    op = row_sum8(op);
    if (part == 0) osh[i] = op;
    float* S_out = p.mode == DN_VERIFY ? p.state + ((size_t)((cur + 1 + t) % p.nslots) * p.heads + h) * hs
                            : const_cast<float*>(S_in);
#pragma unroll
    for (int jj = 0; jj < DKP; ++jj) S_out[sbase + (size_t)jj * 64] = S[jj];
    __syncthreads();
    // 4. gated RMSNorm of the head's output, then its digits (half-wave per 32 rows)
    if (wave == 0) {
      const float a0 = lane < p.dv ? osh[lane] : 0.0f, a1 = lane + 64 < p.dv ? osh[lane + 64] : 0.0f;
      const float ss = wave_sum(a0 * a0 + a1 * a1);
      if (lane == 0) sc[2] = 1.0f / sqrtf(ss / (float)p.dv + p.eps);
    }
    __syncthreads();
    if (tid < (p.dv + 63) / 64 * 64) {
      const bool valid = tid < p.dv;
      float uo = 0.0f;
      if (valid) {
        const float zz = zsh[tid];
        uo = osh[tid] * sc[2] * wn * (zz / (1.0f + expf(-zz)));
      }
      if (p.u_out && valid) p.u_out[(size_t)t * nv + h * p.dv + tid] = uo;
      if (p.next.xd) put_digits(p.next, p.next_qt, t, (h * p.dv + (tid & ~31)) / QK, uo, valid);
    }
    __syncthreads();
  }
}

hipError_t launch_deltanet(const DnParams& p, int T, hipStream_t s) {
  if (p.dk % 32 || p.dk > 128 || p.dv % 32 || T < 1 || T > MAX_T) return hipErrorInvalidValue;
  if (p.mode != DN_DECODE && p.mode != DN_VERIFY && p.mode != DN_CHUNK) return hipErrorInvalidValue;
  if (p.variant) {
    if (p.mode == DN_CHUNK || p.dv > 128 || 7 * p.dv < 2 * p.dk || p.conv < 2 || p.conv > 4 || p.k_heads <= 0 ||
        p.heads % p.k_heads ||
        !p.conv_w || !p.a_log || !p.dt_bias || !p.norm_w || !p.conv_state)
      return hipErrorInvalidValue;
    const unsigned block = (unsigned)(p.dv / 8) * 64;   // 8 lanes per row of S
    switch (p.dk) {
      case 32: k_deltanet_q35<4><<<p.heads, block, 0, s>>>(p, T); break;
      case 64: k_deltanet_q35<8><<<p.heads, block, 0, s>>>(p, T); break;
      case 96: k_deltanet_q35<12><<<p.heads, block, 0, s>>>(p, T); break;
      case 128: k_deltanet_q35<16><<<p.heads, block, 0, s>>>(p, T); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const unsigned grid = (unsigned)(p.heads * (p.dv / 32));
  const bool chunk = p.mode == DN_CHUNK;
  switch (p.dk) {
#define SLQ_DN(DKP)                                            \
  if (chunk) k_deltanet_chunk<DKP><<<grid, 1024, 0, s>>>(p, T); \
  else k_deltanet<DKP><<<grid, 256, 0, s>>>(p, T);             \
  break;
    case 32: SLQ_DN(4)
    case 64: SLQ_DN(8)
    case 96: SLQ_DN(12)
    case 128: SLQ_DN(16)
#undef SLQ_DN
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Canonical [head][i][j] <-> the device layout of the current slot.
__global__ void k_state_io(float* state, int nslots, const Ctrl* ctrl, int heads, int dk, int dv,
                           float* canon, int to_device) {
  const size_t n = (size_t)heads * dk * dv;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int h = (int)(idx / ((size_t)dk * dv));
  const int rem = (int)(idx % ((size_t)dk * dv));
  const int i = rem / dk, j = rem % dk;     // canonical index (h, i, j)
  float* dev = state + (size_t)(ctrl ? ctrl->cur : 0) * n + (size_t)h * dk * dv + dn_off(i, j, dk / 8);
  if (to_device) *dev = canon[idx];
  else canon[idx] = *dev;
  (void)nslots;
}

hipError_t launch_state_io(float* state, int nslots, const Ctrl* ctrl, int heads, int dk, int dv,
                           float* canon, int to_device, hipStream_t s) {
  const size_t n = (size_t)heads * dk * dv;
  k_state_io<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(state, nslots, ctrl, heads, dk, dv, canon, to_device);
  return hipGetLastError();
}

}  // namespace slq
