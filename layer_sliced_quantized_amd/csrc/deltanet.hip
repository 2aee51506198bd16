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
// order, so the two reductions per token are deterministic.  Wave 0 also
// normalises q and k into LDS and quantises the 32 outputs (one digit block).
template <int DKP>
__global__ __launch_bounds__(256) void k_deltanet(DnParams p, int T) {
  __shared__ float qs[8 * DKP], ksh[8 * DKP];
  __shared__ float red[8][32];
  const int nib = p.dv / 32;
  const int h = blockIdx.x / nib, ib = blockIdx.x % nib;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int part = tid >> 5, ii = tid & 31;
  const int i = ib * 32 + ii;
  const int dk = 8 * DKP;
  const int cur = p.ctrl->cur;
  const size_t hs = (size_t)dk * p.dv;
  const float* S_in = p.state + ((size_t)cur * p.heads + h) * hs;
  const int j0 = part * DKP;

  float S[DKP];
#pragma unroll
  for (int jj = 0; jj < DKP; ++jj) S[jj] = S_in[(size_t)(j0 + jj) * p.dv + i];

  for (int t = 0; t < T; ++t) {
    const float* y = p.y + (size_t)t * p.y_stride;
    if (tid < 64) {
      // q, k of head h: lanes hold entries lane and lane + 64
      float q0 = 0.0f, q1 = 0.0f, k0 = 0.0f, k1 = 0.0f;
      if (lane < dk) { q0 = y[p.off_q + h * dk + lane]; k0 = y[p.off_k + h * dk + lane]; }
      if (lane + 64 < dk) { q1 = y[p.off_q + h * dk + lane + 64]; k1 = y[p.off_k + h * dk + lane + 64]; }
      const float sq = wave_sum(q0 * q0 + q1 * q1), sk = wave_sum(k0 * k0 + k1 * k1);
      const float rq = 1.0f / sqrtf(sq + 1e-6f), rk = 1.0f / sqrtf(sk + 1e-6f);
      if (lane < dk) { qs[lane] = q0 * rq; ksh[lane] = k0 * rk; }
      if (lane + 64 < dk) { qs[lane + 64] = q1 * rq; ksh[lane + 64] = k1 * rk; }
    }
    const float alpha = sigmoidf_(p.a_scale * y[p.off_a + h] + p.a_bias);
    const float beta = sigmoidf_(p.b_scale * y[p.off_b + h]);
    const float vi = y[p.off_v + h * p.dv + i];
    const float zi = y[p.off_z + h * p.dv + i];
    __syncthreads();

    float up = 0.0f;
#pragma unroll
    for (int jj = 0; jj < DKP; ++jj) up = __builtin_fmaf(S[jj], ksh[j0 + jj], up);
    red[part][ii] = up;
    __syncthreads();
    float u = red[0][ii];
#pragma unroll
    for (int k = 1; k < 8; ++k) u += red[k][ii];
    const float c = beta * (vi - alpha * u);
    float op = 0.0f;
#pragma unroll
    for (int jj = 0; jj < DKP; ++jj) {
      S[jj] = __builtin_fmaf(c, ksh[j0 + jj], alpha * S[jj]);
      op = __builtin_fmaf(S[jj], qs[j0 + jj], op);
    }
    __syncthreads();   // every thread has read red
    red[part][ii] = op;

    float* S_out = p.verify ? p.state + ((size_t)((cur + 1 + t) % p.nslots) * p.heads + h) * hs
                            : const_cast<float*>(S_in);
#pragma unroll
    for (int jj = 0; jj < DKP; ++jj) S_out[(size_t)(j0 + jj) * p.dv + i] = S[jj];
    __syncthreads();
    if (tid < 64) {
      // lanes ii and ii + 32 of wave 0 both hold row i's output; the first
      // half stores it
      float o = red[0][ii];
#pragma unroll
      for (int k = 1; k < 8; ++k) o += red[k][ii];
      const float uo = o * sigmoidf_(p.z_scale * zi);
      const int nv = p.heads * p.dv;
      if (p.u_out && lane < 32) p.u_out[(size_t)t * nv + h * p.dv + i] = uo;
      const int blk = (h * p.dv + ib * 32) / QK;
      put_digits(p.next, p.next_qt, t, blk, uo, lane < 32);
    }
    __syncthreads();   // qs, ksh and red are rewritten by the next token
  }
}

hipError_t launch_deltanet(const DnParams& p, int T, hipStream_t s) {
  if (p.dk % 32 || p.dk > 128 || p.dv % 32) return hipErrorInvalidValue;
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
