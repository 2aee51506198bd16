// Gated DeltaNet recurrent update for decode and verify.
//
// The hybrid's linear-attention layers (ChatTorrent README, "What it can run":
// "Gated DeltaNet linear-attention layers") carry a per-head state S (d_v x
// d_k, fp32) updated once per token, serially ("the DeltaNet recurrence is
// serial", SwarmLLM README, bench paragraph):
//     S' = alpha S (I - beta k k^T) + beta v k^T,   o = S' q
// with q, k divided by sqrt(sum of squares + 1e-6).  Row i of S only needs the
// whole k and q plus v_i, so rows are independent:
//     u_i = S_i . k,   S'_ij = alpha S_ij + beta (v_i - alpha u_i) k_j,   o_i = S'_i . q
// Each lane owns one row i and 32 consecutive j of it (the state lives in
// registers across the tokens of a verify pass); the waves of a workgroup
// cover the j range and meet in LDS in a fixed order.
//
// State layout in HBM: [slot][head][j][i] (i fastest) so that a wave's loads
// and stores of one j are contiguous.  Decode updates slot `cur` in place;
// verify writes the state after token t to slot (cur + 1 + t) mod nslots and
// never touches slot `cur`, which is what makes rollback exact.
#include "dev.h"

namespace slq {

__global__ __launch_bounds__(256) void k_deltanet(DnParams p, int T) {
  __shared__ float qs[128], ksh[128];
  __shared__ float red[4][RG];
  __shared__ float red2[4][2];
  const int nic = (p.dv + RG - 1) / RG;
  const int h = blockIdx.x / nic, ic = blockIdx.x % nic;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int nw = blockDim.x >> 6;          // == dk / 32
  const int i = ic * RG + lane;
  const bool iv = i < p.dv;
  const int cur = p.ctrl->cur;
  const size_t hs = (size_t)p.dk * p.dv;
  const float* S_in = p.state + ((size_t)cur * p.heads + h) * hs;
  const int j0 = wave * 32;

  float S[32];
#pragma unroll
  for (int jj = 0; jj < 32; ++jj) S[jj] = iv ? S_in[(size_t)(j0 + jj) * p.dv + i] : 0.0f;

  for (int t = 0; t < T; ++t) {
    const float* y = p.y + (size_t)t * p.y_stride;
    float qv = 0.0f, kv = 0.0f;
    if ((int)threadIdx.x < p.dk) {
      qv = y[p.off_q + h * p.dk + threadIdx.x];
      kv = y[p.off_k + h * p.dk + threadIdx.x];
    }
    const float sq = wave_sum(qv * qv), sk = wave_sum(kv * kv);
    if (lane == 0) { red2[wave][0] = sq; red2[wave][1] = sk; }
    __syncthreads();
    float Sq = 0.0f, Sk = 0.0f;
    for (int w = 0; w < nw; ++w) { Sq += red2[w][0]; Sk += red2[w][1]; }
    const float rq = 1.0f / sqrtf(Sq + 1e-6f), rk = 1.0f / sqrtf(Sk + 1e-6f);
    if ((int)threadIdx.x < p.dk) { qs[threadIdx.x] = qv * rq; ksh[threadIdx.x] = kv * rk; }
    const float alpha = sigmoidf_(p.a_scale * y[p.off_a + h] + p.a_bias);
    const float beta = sigmoidf_(p.b_scale * y[p.off_b + h]);
    const float vi = iv ? y[p.off_v + h * p.dv + i] : 0.0f;
    const float zi = iv ? y[p.off_z + h * p.dv + i] : 0.0f;
    __syncthreads();

    float up = 0.0f;
#pragma unroll
    for (int jj = 0; jj < 32; ++jj) up = __builtin_fmaf(S[jj], ksh[j0 + jj], up);
    red[wave][lane] = up;
    __syncthreads();
    float u = 0.0f;
    for (int w = 0; w < nw; ++w) u += red[w][lane];
    const float c = beta * (vi - alpha * u);
    float op = 0.0f;
#pragma unroll
    for (int jj = 0; jj < 32; ++jj) {
      S[jj] = __builtin_fmaf(c, ksh[j0 + jj], alpha * S[jj]);
      op = __builtin_fmaf(S[jj], qs[j0 + jj], op);
    }
    __syncthreads();
    red[wave][lane] = op;
    __syncthreads();
    float o = 0.0f;
    for (int w = 0; w < nw; ++w) o += red[w][lane];

    float* S_out = p.verify ? p.state + ((size_t)((cur + 1 + t) % p.nslots) * p.heads + h) * hs
                            : const_cast<float*>(S_in);
    if (iv) {
#pragma unroll
      for (int jj = 0; jj < 32; ++jj) S_out[(size_t)(j0 + jj) * p.dv + i] = S[jj];
    }
    if (wave == 0) {
      const float uo = o * sigmoidf_(p.z_scale * zi);
      const int nv = p.heads * p.dv;
      if (p.u_out && iv) p.u_out[(size_t)t * nv + h * p.dv + i] = uo;
      const int blk = (h * p.dv + ic * RG) / QK + (lane >> 5);
      const bool wr = (ic * RG + (lane & 32)) < p.dv;
      quant_block_half_qt(p.next_qt, iv ? uo : 0.0f, p.next.xd + ((size_t)t * p.next.nblk + blk) * XW,
                          p.next.xs + (size_t)t * p.next.nblk + blk, wr);
    }
    __syncthreads();
  }
}

hipError_t launch_deltanet(const DnParams& p, int T, hipStream_t s) {
  if (p.dk % 32 || p.dk > 128 || p.dv % 32) return hipErrorInvalidValue;
  const int nic = (p.dv + RG - 1) / RG;
  k_deltanet<<<p.heads * nic, 64 * (p.dk / 32), 0, s>>>(p, T);
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
