// Gated DeltaNet recurrent update for decode and verify.
//
// The hybrid model's linear-attention layers are Gated DeltaNet (ChatTorrent
// README, "What it can run").  Each head carries a state S (d_v x d_k, fp32)
// that is updated once per token, one token after the other (the pages note
// that this recurrence cannot be parallelised over tokens; SwarmLLM README,
// bench paragraph):
//     S' = alpha S (I - beta k k^T) + beta v k^T,   o = S' q
// with q, k divided by sqrt(sum of squares + 1e-6).  Row i of S only needs the
// whole k and q plus v_i, so rows are independent:
//     u_i = S_i . k,   S'_ij = alpha S_ij + beta (v_i - alpha u_i) k_j,   o_i = S'_i . q
// Eight threads own one row i, each with an eighth of the j range (the state
// lives in registers across the tokens of a verify pass), and meet in LDS.
//
// State layout in HBM: [slot][head][j][i] (i fastest) so that a wave's loads
// and stores of one j are contiguous.  Decode updates slot `cur` in place;
// verify writes the state after token t to slot (cur + 1 + t) mod nslots and
// never touches slot `cur`, which is what makes rollback exact.
#include "dev.h"

namespace slq {

// One workgroup of 4 waves per (head, 32 rows of S).  Thread (part, ii)
// owns row i = 32 ib + ii over the key range [part*DKP, part*DKP + DKP),
// part = 0..7; a half-wave (one part) reads 32 consecutive rows of one j as
// 128 contiguous bytes.  The parts of a row meet in LDS and are added in part
// order, so the two reductions per token are deterministic.
//
// Every token's inputs are requested together before the first update (the
// recurrence itself runs token after token): the waves normalise q and k of
// tokens wave, wave + 4, ... into LDS, and (for several tokens) the v, z,
// decay and gate inputs go to LDS as well, so no token waits on a global
// load inside the loop.  The
// two reductions of a token use separate LDS areas, which leaves two
// workgroup barriers per token.  Wave 0 quantises the 32 outputs of each
// token (one digit block).
template <int DKP>
__global__ __launch_bounds__(256) void k_deltanet(DnParams p, int T) {
  constexpr int DK = 8 * DKP;
  __shared__ float qs[MAX_T][DK], ksh[MAX_T][DK];
  __shared__ float vsh[MAX_T][32], zsh[MAX_T][32];
  __shared__ float ab[MAX_T][2];
  __shared__ float red_u[8][32], red_o[8][32];
  const int nib = p.dv / 32;
  const int h = blockIdx.x / nib, ib = blockIdx.x % nib;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int part = tid >> 5, ii = tid & 31;
  const int i = ib * 32 + ii;
  const int cur = p.ctrl->cur;
  const size_t hs = (size_t)DK * p.dv;
  const float* S_in = p.state + ((size_t)cur * p.heads + h) * hs;
  const int j0 = part * DKP;

  float S[DKP];
#pragma unroll
  for (int jj = 0; jj < DKP; ++jj) S[jj] = S_in[(size_t)(j0 + jj) * p.dv + i];

  // q, k of head h for tokens wave + 4m: lanes hold entries lane and lane + 64
  {
    float q0[4], q1[4], k0[4], k1[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int t = wave + 4 * m;
      q0[m] = q1[m] = k0[m] = k1[m] = 0.0f;
      if (t < T) {
        const float* y = p.y + (size_t)t * p.y_stride;
        if (lane < DK) { q0[m] = y[p.off_q + h * DK + lane]; k0[m] = y[p.off_k + h * DK + lane]; }
        if (lane + 64 < DK) { q1[m] = y[p.off_q + h * DK + lane + 64]; k1[m] = y[p.off_k + h * DK + lane + 64]; }
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int t = wave + 4 * m;
      if (t < T) {
        const float sq = wave_sum(q0[m] * q0[m] + q1[m] * q1[m]), sk = wave_sum(k0[m] * k0[m] + k1[m] * k1[m]);
        const float rq = 1.0f / sqrtf(sq + 1e-6f), rk = 1.0f / sqrtf(sk + 1e-6f);
        if (lane < DK) { qs[t][lane] = q0[m] * rq; ksh[t][lane] = k0[m] * rk; }
        if (lane + 64 < DK) { qs[t][lane + 64] = q1[m] * rq; ksh[t][lane + 64] = k1[m] * rk; }
      }
    }
  }
  // v, z, decay and gate: with one token every thread takes its own from
  // global memory (no LDS hop on the decode path); with several, v and z of
  // rows 32 ib + (tid % 32) for tokens tid / 32 and tid / 32 + 8, and the
  // gates of token tid, go to LDS
  const bool one = T == 1;
  float v1 = 0.0f, z1 = 0.0f, a1 = 0.0f, b1 = 0.0f;
  if (one) {
    v1 = p.y[p.off_v + h * p.dv + i];
    z1 = p.y[p.off_z + h * p.dv + i];
    a1 = sigmoidf_(p.a_scale * p.y[p.off_a + h] + p.a_bias);
    b1 = sigmoidf_(p.b_scale * p.y[p.off_b + h]);
  } else {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int t = tid / 32 + 8 * m;
      if (t < T) {
        const float* y = p.y + (size_t)t * p.y_stride;
        vsh[t][ii] = y[p.off_v + h * p.dv + i];
        zsh[t][ii] = y[p.off_z + h * p.dv + i];
      }
    }
    if (tid < T) {
      const float* y = p.y + (size_t)tid * p.y_stride;
      ab[tid][0] = sigmoidf_(p.a_scale * y[p.off_a + h] + p.a_bias);
      ab[tid][1] = sigmoidf_(p.b_scale * y[p.off_b + h]);
    }
  }
  __syncthreads();

  for (int t = 0; t < T; ++t) {
    const float alpha = one ? a1 : ab[t][0], beta = one ? b1 : ab[t][1];
    const float vi = one ? v1 : vsh[t][ii];
    float up = 0.0f;
#pragma unroll
    for (int jj = 0; jj < DKP; ++jj) up = __builtin_fmaf(S[jj], ksh[t][j0 + jj], up);
    red_u[part][ii] = up;
    __syncthreads();
    float u = red_u[0][ii];
#pragma unroll
    for (int k = 1; k < 8; ++k) u += red_u[k][ii];
    const float c = beta * (vi - alpha * u);
    float op = 0.0f;
#pragma unroll
    for (int jj = 0; jj < DKP; ++jj) {
      S[jj] = __builtin_fmaf(c, ksh[t][j0 + jj], alpha * S[jj]);
      op = __builtin_fmaf(S[jj], qs[t][j0 + jj], op);
    }
    red_o[part][ii] = op;

    float* S_out = p.verify ? p.state + ((size_t)((cur + 1 + t) % p.nslots) * p.heads + h) * hs
                            : const_cast<float*>(S_in);
#pragma unroll
    for (int jj = 0; jj < DKP; ++jj) S_out[(size_t)(j0 + jj) * p.dv + i] = S[jj];
    // Every thread has read red_u (before writing red_o), so the next token
    // may overwrite it after this barrier; wave 0 reads red_o before it
    // reaches the next token's barrier, so red_o is not overwritten early.
    __syncthreads();
    if (tid < 64) {
      // lanes ii and ii + 32 of wave 0 both hold row i's output; the first
      // half stores it
      float o = red_o[0][ii];
#pragma unroll
      for (int k = 1; k < 8; ++k) o += red_o[k][ii];
      const float uo = o * sigmoidf_(p.z_scale * (one ? z1 : zsh[t][ii]));
      const int nv = p.heads * p.dv;
      if (p.u_out && lane < 32) p.u_out[(size_t)t * nv + h * p.dv + i] = uo;
      const int blk = (h * p.dv + ib * 32) / QK;
      put_digits(p.next, p.next_qt, t, blk, uo, lane < 32);
    }
  }
}

hipError_t launch_deltanet(const DnParams& p, int T, hipStream_t s) {
  if (p.dk % 32 || p.dk > 128 || p.dv % 32 || T < 1 || T > MAX_T) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)(p.heads * (p.dv / 32));
  switch (p.dk) {
    case 32: k_deltanet<4><<<grid, 256, 0, s>>>(p, T); break;
    case 64: k_deltanet<8><<<grid, 256, 0, s>>>(p, T); break;
    case 96: k_deltanet<12><<<grid, 256, 0, s>>>(p, T); break;
    case 128: k_deltanet<16><<<grid, 256, 0, s>>>(p, T); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Canonical [head][i][j] <-> device [head][j][i] of the current slot.
__global__ void k_state_io(float* state, int nslots, const Ctrl* ctrl, int heads, int dk, int dv,
                           float* canon, int to_device) {
  const size_t n = (size_t)heads * dk * dv;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int h = (int)(idx / ((size_t)dk * dv));
  const int rem = (int)(idx % ((size_t)dk * dv));
  const int i = rem / dk, j = rem % dk;     // canonical index (h, i, j)
  float* dev = state + (size_t)ctrl->cur * n + (size_t)h * dk * dv + (size_t)j * dv + i;
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
