// Boundary conversion, step control, embedding lookup and greedy argmax.
//
// A stage hands one token's hidden state on (5,120 x f16 on the pages' wire,
// SwarmLLM README, bench paragraph); the first stage owns the embedding and
// the last one the head and the sampling ("Unstable Legion", section
// "Splitting the workload").  Sampling here is greedy, as in the pages'
// benchmark table (SwarmLLM README).
#include "dev.h"

namespace slq {

// h fp32 [T][H] -> boundary vector (fp16 round-to-nearest-even, or fp32 copy).
__global__ void k_store_out(const float* __restrict__ h, int n, void* out, int fp32, Ctrl* ctrl,
                            int advance) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (!out) out = ctrl->out;
  if (i < n) {
    if (fp32) reinterpret_cast<float*>(out)[i] = h[i];
    else reinterpret_cast<__half*>(out)[i] = __float2half_rn(h[i]);
  }
  if (advance && i == 0) ctrl->pos += advance;
}

hipError_t launch_store_out(const float* h, int T, int H, void* out, int fp32, Ctrl* ctrl, int advance,
                            hipStream_t s) {
  const int n = T * H;
  k_store_out<<<(n + 255) / 256, 256, 0, s>>>(h, n, out, fp32, ctrl, advance);
  return hipGetLastError();
}

__global__ void k_fill_zero_u32(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

hipError_t launch_fill_zero_u32(uint32_t* p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t nb = (n + 255) / 256;
  const unsigned grid = (unsigned)(nb < 1024 ? nb : 1024);
  k_fill_zero_u32<<<grid, 256, 0, s>>>(p, n);
  return hipGetLastError();
}

// Streaming read of n16 16-byte words, each read once with a nontemporal
// load (as the GEMVs read weights), sixteen loads in flight per lane (the
// fastest of 2 to 16 loads and 1024 to 16384 workgroups over 4 GiB on
// MI355X: 6.9 TB/s).  The words are folded by XOR into one value per wave,
// stored to sink, so that no load can be dropped; sink needs gridDim.x * 4
// entries.
typedef uint32_t rp_u32x4 __attribute__((ext_vector_type(4)));
constexpr int RP_LOADS = 16;

__global__ __launch_bounds__(256) void k_read_probe(const rp_u32x4* __restrict__ p, size_t n16, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  rp_u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (RP_LOADS - 1) * stride < n16; i += RP_LOADS * stride) {
    rp_u32x4 v[RP_LOADS];
#pragma unroll
    for (int u = 0; u < RP_LOADS; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < RP_LOADS; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
  uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
  for (int o = 32; o > 0; o >>= 1) v ^= __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = v;
}

// grid: at most max_grid workgroups, fewer for a buffer under max_grid full
// rounds of sixteen loads per lane
hipError_t launch_read_probe(const void* p, size_t n16, uint32_t* sink, unsigned max_grid, hipStream_t s) {
  const size_t per = (size_t)RP_LOADS * 256;
  const size_t want = (n16 + per - 1) / per;
  const unsigned grid = (unsigned)(want < max_grid ? (want ? want : 1) : max_grid);
  k_read_probe<<<grid, 256, 0, s>>>(reinterpret_cast<const rp_u32x4*>(p), n16, sink);
  return hipGetLastError();
}

__global__ void k_ctrl_io(Ctrl* c, const void* in, void* out) {
  c->in = in;
  c->out = out;
}

hipError_t launch_ctrl_io(Ctrl* c, const void* in, void* out, hipStream_t s) {
  k_ctrl_io<<<1, 1, 0, s>>>(c, in, out);
  return hipGetLastError();
}

__global__ void k_ctrl_set(Ctrl* c, int pos, int cur) {
  c->pos = pos;
  c->cur = cur;
}

hipError_t launch_ctrl_set(Ctrl* c, int pos, int cur, hipStream_t s) {
  k_ctrl_set<<<1, 1, 0, s>>>(c, pos, cur);
  return hipGetLastError();
}

// Dequantise row *tok of a packed embedding table into a boundary vector.
template <int QT>
__global__ void k_embed(Packed E, const int32_t* __restrict__ tok, void* out, int fp32) {
  constexpr int NH = QT == QT_Q4 ? 1 : 2;
  const int b = blockIdx.x * blockDim.x + threadIdx.x;   // block along the row
  const int nblk = E.nblk();
  if (b >= nblk) return;
  int64_t r = *tok;
  if (r < 0 || r >= E.rows) r = 0;
  const int64_t rg = r / RG;
  const int lane = (int)(r % RG);
  const int t = b / TB, bi = b % TB;
  const int nb_t = min(TB, nblk - t * TB);
  const uint8_t* tile = E.w + rg * rg_bytes(QT, E.cols) + (size_t)t * tile_bytes(QT);
  const uint8_t* sc = tile + (size_t)nb_t * NH * RG * 16 + lane * 16 + bi * 2;
  const float d = __half2float(__ushort_as_half((unsigned short)(sc[0] | (sc[1] << 8))));
  float v[QK];
  for (int h = 0; h < NH; ++h) {
    const uint8_t* c = tile + (size_t)(bi * NH + h) * RG * 16 + lane * 16;
    for (int j = 0; j < 16; ++j) {
      if (QT == QT_Q4) {
        v[j] = (float)((int)((c[j] & 15) ^ 8) - 8) * d;
        v[j + 16] = (float)((int)((c[j] >> 4) ^ 8) - 8) * d;
      } else {
        v[h * 16 + j] = (float)(int8_t)c[j] * d;
      }
    }
  }
  for (int j = 0; j < QK; ++j) {
    const int64_t i = (int64_t)b * QK + j;
    if (fp32) reinterpret_cast<float*>(out)[i] = v[j];
    else reinterpret_cast<__half*>(out)[i] = __float2half_rn(v[j]);
  }
}

hipError_t launch_embed(const Packed& E, const int32_t* tok, void* out, int fp32, hipStream_t s) {
  const int nblk = E.nblk();
  if (E.qt == QT_Q4) k_embed<QT_Q4><<<(nblk + 63) / 64, 64, 0, s>>>(E, tok, out, fp32);
  else k_embed<QT_Q8><<<(nblk + 63) / 64, 64, 0, s>>>(E, tok, out, fp32);
  return hipGetLastError();
}

// The draft head's input digits.  Workgroup 0 takes the embedding row *tok
// (dequantised from the packed table, as k_embed), workgroup 1 the boundary
// vector h; each RMS-normalises its H values with its own weights (sum of
// squares in a fixed order: per thread, then per wave, then waves in order)
// and writes the digits of its half of the 2H-wide input: blocks 0..H/32-1
// the embedding side, H/32.. the hidden side.  MTP_THREADS threads each.
constexpr int MTP_THREADS = 1024;
template <int QT>
__global__ __launch_bounds__(MTP_THREADS) void k_mtp_in(Packed E, const int32_t* __restrict__ tok, const void* hin,
                                                int fp32, const float* __restrict__ w_e,
                                                const float* __restrict__ w_h, float eps, Act x) {
  constexpr int NH = QT == QT_Q4 ? 1 : 2;
  extern __shared__ float sv[];          // [H] values, then [MTP_THREADS / 64] wave sums
  const int H = (int)E.cols;
  const int half = blockIdx.x;
  const int tid = threadIdx.x;
  float ss = 0.0f;
  if (half == 0) {
    int64_t r = *tok;
    if (r < 0 || r >= E.rows) r = 0;
    const int64_t rg = r / RG;
    const int lane = (int)(r % RG);
    const int nblk = E.nblk();
    for (int i = tid; i < H; i += MTP_THREADS) {
      const int b = i / QK, j = i % QK;
      const int t = b / TB, bi = b % TB;
      const int nb_t = min(TB, nblk - t * TB);
      const uint8_t* tile = E.w + rg * rg_bytes(QT, E.cols) + (size_t)t * tile_bytes(QT);
      const uint8_t* sc = tile + (size_t)nb_t * NH * RG * 16 + lane * 16 + bi * 2;
      const float d = __half2float(__ushort_as_half((unsigned short)(sc[0] | (sc[1] << 8))));
      float v;
      if (QT == QT_Q4) {
        const uint8_t c = tile[(size_t)bi * RG * 16 + lane * 16 + (j & 15)];
        v = (float)((int)(((j < 16 ? c : c >> 4) & 15) ^ 8) - 8) * d;
      } else {
        v = (float)(int8_t)tile[(size_t)(bi * NH + (j >> 4)) * RG * 16 + lane * 16 + (j & 15)] * d;
      }
      sv[i] = v;
      ss += v * v;
    }
  } else {
    for (int i = tid; i < H; i += MTP_THREADS) {
      const float v = fp32 ? reinterpret_cast<const float*>(hin)[i]
                           : __half2float(reinterpret_cast<const __half*>(hin)[i]);
      sv[i] = v;
      ss += v * v;
    }
  }
  ss = wave_sum(ss);
  const int wave = wave_id(), lane = tid & 63;
  if (lane == 0) sv[H + wave] = ss;
  __syncthreads();
  float tot = sv[H];
  for (int w = 1; w < MTP_THREADS / 64; ++w) tot += sv[H + w];   // waves in order
  const float rn = 1.0f / sqrtf(tot / (float)H + eps);
  const float* w = half == 0 ? w_e : w_h;
  const int nb = H / QK;
  for (int rg = wave; 2 * rg < nb; rg += MTP_THREADS / 64) {
    const int i = rg * RG + lane;
    const bool ok = i < H;
    const float v = ok ? (sv[i] * rn) * w[i] : 0.0f;
    const int blk = 2 * rg + (lane >> 5);
    put_digits(x, QT, 0, half * nb + blk, v, blk < nb);
  }
}

hipError_t launch_mtp_input(const Packed& E, const int32_t* tok, const void* hin, int fp32, const float* w_e,
                            const float* w_h, float eps, Act x, hipStream_t s) {
  const int H = (int)E.cols;
  if (H % QK || x.nblk != 2 * H / QK || x.mxd) return hipErrorInvalidValue;
  const size_t lds = ((size_t)H + MTP_THREADS / 64) * 4;
  if (E.qt == QT_Q4) k_mtp_in<QT_Q4><<<2, MTP_THREADS, lds, s>>>(E, tok, hin, fp32, w_e, w_h, eps, x);
  else k_mtp_in<QT_Q8><<<2, MTP_THREADS, lds, s>>>(E, tok, hin, fp32, w_e, w_h, eps, x);
  return hipGetLastError();
}

// Greedy argmax in two passes; the larger value wins, the lower index wins a tie.
__device__ __forceinline__ void better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

__device__ __forceinline__ void block_argmax(float& bv, int& bi) {
  __shared__ float sv[16];
  __shared__ int si[16];
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(bv, m, 64);
    const int oi = __shfl_xor(bi, m, 64);
    better(bv, bi, ov, oi);
  }
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if ((threadIdx.x & 63) == 0) { sv[w] = bv; si[w] = bi; }
  __syncthreads();
  bv = sv[0]; bi = si[0];
  for (int k = 1; k < nw; ++k) better(bv, bi, sv[k], si[k]);
}

__global__ void k_argmax_part(const float* __restrict__ x, int n, float* pv, int* pi) {
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    better(bv, bi, x[i], i);
  block_argmax(bv, bi);
  if (threadIdx.x == 0) { pv[blockIdx.x] = bv; pi[blockIdx.x] = bi; }
}

__global__ void k_argmax_final(const float* __restrict__ pv, const int* __restrict__ pi, int np,
                               int32_t* tok) {
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = threadIdx.x; i < np; i += blockDim.x) better(bv, bi, pv[i], pi[i]);
  block_argmax(bv, bi);
  if (threadIdx.x == 0) *tok = bi == 0x7fffffff ? 0 : bi;
}

hipError_t launch_argmax(const float* logits, int n, float* part_v, int* part_i, int nparts, int32_t* tok,
                         hipStream_t s) {
  k_argmax_part<<<nparts, 256, 0, s>>>(logits, n, part_v, part_i);
  k_argmax_final<<<1, 256, 0, s>>>(part_v, part_i, nparts, tok);
  return hipGetLastError();
}

}  // namespace slq
