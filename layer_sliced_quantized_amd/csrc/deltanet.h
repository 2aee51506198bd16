// Gated DeltaNet decode rows: the per-workgroup body shared by the DeltaNet
// kernel and the chained decode products (the method and the state layout
// are described in deltanet.hip).
#pragma once
#include "dev.h"

namespace slq {

// Sum over the eight lanes l, l ^ 8, ..., l ^ 56 that hold the parts of one
// row, with the additions in the order x + x[l^8], then + [l^16], then
// + [l^32], so every lane gets the same bits.
__device__ __forceinline__ float row_sum8(float v) {
  v += xor_lane<8>(v);
  v += xor_lane<16>(v);
  v += xor_lane<32>(v);
  return v;
}

// Offset of S[i][j] inside one head's state (d_k = 8 dkp).
__host__ __device__ inline size_t dn_off(int i, int j, int dkp) {
  return ((size_t)((i >> 3) * dkp + j % dkp) * 8 + j / dkp) * 8 + (i & 7);
}

// One workgroup of 4 waves per (head, 32 rows of S); wave w owns rows
// 32 ib + 8 w + r, lane (part, r) = (lane / 8, lane % 8) the key range
// [part*DKP, part*DKP + DKP) of its row.  The eight parts of a row meet in a
// butterfly over lanes r, r + 8, ..., r + 56 (row_sum8: a fixed order, so the
// sums are deterministic).
//
// Every token's inputs are requested together before the first update (the
// recurrence itself runs token after token): the waves normalise q and k of
// tokens wave, wave + 4, ... into LDS, and (for several tokens) the v, z,
// decay and gate inputs go to LDS as well, so no token waits on a global
// load inside the loop.  The outputs of all tokens are quantised after the
// loop, one digit block of 32 rows per token, by wave t mod 4.
//
// deltanet_rows is the body of one workgroup (block = head * dv / 32 + row
// block), for at most TM tokens; COH makes the output digits coherent stores,
// for a consumer inside the same kernel (the chained decode products).
//
// With an active Wait (one token only) the inputs are written earlier in the
// same kernel: the state rows are requested first, then wait() (uniform over
// the workgroup; false: give up and return false), then the inputs are read
// with coherent loads.  The arithmetic is the same either way.
struct NoWait {
  static constexpr bool active = false;
  __device__ bool operator()() const { return true; }
};
template <int DKP, int TM, bool COH, class Wait = NoWait>
__device__ __forceinline__ bool deltanet_rows(const DnParams& p, int T, int block, const Wait& wait = Wait{}) {
  constexpr bool AFTER = Wait::active;
  static_assert(!AFTER || TM == 1, "a waiting update takes one token");
  constexpr int DK = 8 * DKP;
  constexpr int NM = TM > 4 ? 4 : TM;   // tokens per wave
  __shared__ float qs[TM][DK], ksh[TM][DK];
  __shared__ float vsh[TM][32], zsh[TM][32];
  __shared__ float ab[TM][2];
  __shared__ float osh[TM][32];
  const int nib = p.dv / 32;
  const int h = block / nib, ib = block % nib;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int part = lane >> 3, r = lane & 7;
  const int ii = wave * 8 + r;          // row within the workgroup's 32
  const int i = ib * 32 + ii;
  const bool one = TM == 1 || T == 1;
  // Vector inputs first (q, k of tokens wave + 4m, lanes holding entries lane
  // and lane + 64; with one token also this lane's v and z): none of them
  // depends on the state slot, so their latency overlaps the read of the slot
  // index below.  (The gate inputs are uniform, so they come through scalar
  // loads; requested here they would hold up the slot index, so they follow
  // the state loads.)
  float q0[NM], q1[NM], k0[NM], k1[NM];
  float v1 = 0.0f, z1 = 0.0f;
  auto inputs = [&]() {
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int t = wave + 4 * m;
      q0[m] = q1[m] = k0[m] = k1[m] = 0.0f;
      if (t < T) {
        const float* y = p.y + (size_t)t * p.y_stride;
        if (lane < DK) { q0[m] = ld_<AFTER>(y + p.off_q + h * DK + lane); k0[m] = ld_<AFTER>(y + p.off_k + h * DK + lane); }
        if (lane + 64 < DK) {
          q1[m] = ld_<AFTER>(y + p.off_q + h * DK + lane + 64);
          k1[m] = ld_<AFTER>(y + p.off_k + h * DK + lane + 64);
        }
      }
    }
    if (one) {
      v1 = ld_<AFTER>(p.y + p.off_v + h * p.dv + i);
      z1 = ld_<AFTER>(p.y + p.off_z + h * p.dv + i);
    }
  };
  if constexpr (!AFTER) inputs();

  const int cur = p.ctrl ? p.ctrl->cur : 0;
  const size_t hs = (size_t)DK * p.dv;
  const float* S_in = p.state + ((size_t)cur * p.heads + h) * hs;
  const int j0 = part * DKP;
  // this lane's state entries: jj = 0..DKP-1 at a stride of 64 floats
  const size_t sbase = dn_off(i, j0, DKP);

  float S[DKP];
#pragma unroll
  for (int jj = 0; jj < DKP; ++jj) S[jj] = S_in[sbase + (size_t)jj * 64];
  if constexpr (AFTER) {
    if (!wait()) return false;
    inputs();
  }

  // normalised q, k into LDS
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const int t = wave + 4 * m;
    if (t < T) {
      const float sq = wave_sum(q0[m] * q0[m] + q1[m] * q1[m]), sk = wave_sum(k0[m] * k0[m] + k1[m] * k1[m]);
      const float rq = 1.0f / sqrtf(sq + 1e-6f), rk = 1.0f / sqrtf(sk + 1e-6f);
      if (lane < DK) { qs[t][lane] = q0[m] * rq; ksh[t][lane] = k0[m] * rk; }
      if (lane + 64 < DK) { qs[t][lane + 64] = q1[m] * rq; ksh[t][lane + 64] = k1[m] * rk; }
    }
  }
  // decay and gate: with one token every lane keeps its own (no LDS hop on
  // the decode path); with several, v and z of rows 32 ib + (tid % 32) for
  // tokens tid / 32 and tid / 32 + 8, and the gates of token tid, go to LDS
  float a1 = 0.0f, b1 = 0.0f;
  if (one) {
    a1 = sigmoidf_(p.a_scale * ld_<AFTER>(p.y + p.off_a + h) + p.a_bias);
    b1 = sigmoidf_(p.b_scale * ld_<AFTER>(p.y + p.off_b + h));
  } else {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int t = tid / 32 + 8 * m;
      if (t < T && t < TM) {
        const float* y = p.y + (size_t)t * p.y_stride;
        vsh[t][tid & 31] = y[p.off_v + h * p.dv + ib * 32 + (tid & 31)];
        zsh[t][tid & 31] = y[p.off_z + h * p.dv + ib * 32 + (tid & 31)];
      }
    }
    if (tid < T && tid < TM) {
      const float* y = p.y + (size_t)tid * p.y_stride;
      ab[tid][0] = sigmoidf_(p.a_scale * y[p.off_a + h] + p.a_bias);
      ab[tid][1] = sigmoidf_(p.b_scale * y[p.off_b + h]);
    }
  }
  __syncthreads();

  for (int t = 0; t < T && t < TM; ++t) {
    const float alpha = one ? a1 : ab[t][0], beta = one ? b1 : ab[t][1];
    const float vi = one ? v1 : vsh[t][ii];
    float up = 0.0f;
#pragma unroll
    for (int jj = 0; jj < DKP; ++jj) up = __builtin_fmaf(S[jj], ksh[t][j0 + jj], up);
    up = row_sum8(up);
    const float c = beta * (vi - alpha * up);
    float op = 0.0f;
#pragma unroll
    for (int jj = 0; jj < DKP; ++jj) {
      S[jj] = __builtin_fmaf(c, ksh[t][j0 + jj], alpha * S[jj]);
      op = __builtin_fmaf(S[jj], qs[t][j0 + jj], op);
    }
    op = row_sum8(op);
    if (part == 0) osh[t][ii] = op * sigmoidf_(p.z_scale * (one ? z1 : zsh[t][ii]));

    float* S_out = p.mode == DN_VERIFY ? p.state + ((size_t)((cur + 1 + t) % p.nslots) * p.heads + h) * hs
                            : const_cast<float*>(S_in);
#pragma unroll
    for (int jj = 0; jj < DKP; ++jj) S_out[sbase + (size_t)jj * 64] = S[jj];
  }
  __syncthreads();

  // outputs: token t by wave t mod 4; lanes l and l + 32 hold row l's value,
  // the first half stores it
  const int blk = (h * p.dv + ib * 32) / QK;
  const int nv = p.heads * p.dv;
  for (int t = wave; t < T && t < TM; t += 4) {
    const float uo = osh[t][lane & 31];
    if (p.u_out && lane < 32) p.u_out[(size_t)t * nv + h * p.dv + ib * 32 + lane] = uo;
    if (p.next.xd) put_digits<COH>(p.next, p.next_qt, t, blk, uo, lane < 32);
  }
  return true;
}

}  // namespace slq
