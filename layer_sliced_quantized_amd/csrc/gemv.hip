// Q4_0 / Q8_0 matrix-vector products for gfx950.
//
// In the pages' decode kernel (SwarmLLM README, architecture paragraph) every
// weight is read once per token: a 64-thread group walks one row of Q4_0
// blocks, dequantises in registers and reduces through shared memory.  On
// CDNA4 this kernel keeps the 64-lane sweep but turns it 90
// degrees: each lane owns one output row of a 64-row group and streams whole
// blocks of that row with one 128-bit load per block (the load-time repack puts
// 64 rows' 16-byte code chunks side by side, so a wave's load is 1 KiB
// contiguous).  The activation is the same for every row, so it lives in scalar
// registers as integer digits (see quant_block_half): each block's dot product
// is exact in int32 via v_dot8c_i32_i4 (Q4_0) or v_dot4c_i32_i8 (Q8_0), and the
// per-block scales d * s_x are applied in fp32.  Waves of a workgroup split K
// and meet in LDS in a fixed order; nothing uses float atomics, so results are
// the same on every run and for every batch size.
//
// Packed layout of one 64-row group, tile by tile along K (8 blocks per tile):
//   codes  [blocks in tile][NH][64 rows][16 B]  (NH = 1 for Q4_0, 2 for Q8_0;
//          Q4_0 nibbles stored XOR 8, i.e. as signed 4-bit q-8)
//   scales [64 rows][8] fp16
#include "gemv_kernel.h"

namespace slq {

// ------------------------------------------------------------------- repack

// One thread per (source row, block).  map_kind 0: dst row = row_off + r;
// map_kind 1: dst row = (r/32)*64 + r%32 + row_off (interleaves two matrices
// 32 rows at a time, used for the fused SwiGLU gate/up projection).
template <int QT>
__global__ void k_repack(const uint8_t* __restrict__ raw, int64_t rows, int64_t cols,
                         uint8_t* __restrict__ packed, int map_kind, int64_t row_off) {
  constexpr int BB = QT == QT_Q4 ? 18 : 34;
  constexpr int NH = QT == QT_Q4 ? 1 : 2;
  const int nblk = (int)(cols / QK);
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * nblk) return;
  const int64_t r = idx / nblk;
  const int b = (int)(idx % nblk);
  const int64_t R = map_kind == 0 ? row_off + r : (r / 32) * 64 + (r % 32) + row_off;
  const int64_t rg = R / RG;
  const int lane = (int)(R % RG);
  const int t = b / TB, bi = b % TB;
  const int nb_t = min(TB, nblk - t * TB);
  uint8_t* tile = packed + rg * rg_bytes(QT, cols) + (size_t)t * tile_bytes(QT);
  const uint8_t* src = raw + idx * BB;
  for (int h = 0; h < NH; ++h) {
    uint8_t* dst = tile + (size_t)(bi * NH + h) * RG * 16 + lane * 16;
    for (int j = 0; j < 16; ++j) {
      uint8_t c = src[2 + h * 16 + j];
      dst[j] = QT == QT_Q4 ? (uint8_t)(c ^ 0x88) : c;
    }
  }
  uint8_t* sc = tile + (size_t)nb_t * NH * RG * 16 + lane * 16 + bi * 2;
  sc[0] = src[0];
  sc[1] = src[1];
}

hipError_t launch_repack(int qt, const uint8_t* raw, int64_t rows, int64_t cols, uint8_t* packed,
                         int64_t dst_rows, int map_kind, int64_t row_off, hipStream_t s) {
  (void)dst_rows;
  const int64_t n = rows * (cols / QK);
  if (n == 0) return hipSuccess;
  const int bs = 256;
  const unsigned grid = (unsigned)((n + bs - 1) / bs);
  if (qt == QT_Q4) k_repack<QT_Q4><<<grid, bs, 0, s>>>(raw, rows, cols, packed, map_kind, row_off);
  else k_repack<QT_Q8><<<grid, bs, 0, s>>>(raw, rows, cols, packed, map_kind, row_off);
  return hipGetLastError();
}

// ------------------------------------------------------------------ dequant

template <int QT>
__global__ void k_dequant(Packed W, float* __restrict__ out) {
  constexpr int NH = QT == QT_Q4 ? 1 : 2;
  const int nblk = W.nblk();
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= W.rows * nblk) return;
  const int64_t r = idx / nblk;
  const int b = (int)(idx % nblk);
  const int64_t rg = r / RG;
  const int lane = (int)(r % RG);
  const int t = b / TB, bi = b % TB;
  const int nb_t = min(TB, nblk - t * TB);
  const uint8_t* tile = W.w + rg * rg_bytes(QT, W.cols) + (size_t)t * tile_bytes(QT);
  const uint8_t* sc = tile + (size_t)nb_t * NH * RG * 16 + lane * 16 + bi * 2;
  const float d = __half2float(__ushort_as_half((unsigned short)(sc[0] | (sc[1] << 8))));
  float* o = out + r * W.cols + (int64_t)b * QK;
  for (int h = 0; h < NH; ++h) {
    const uint8_t* c = tile + (size_t)(bi * NH + h) * RG * 16 + lane * 16;
    for (int j = 0; j < 16; ++j) {
      if (QT == QT_Q4) {
        const int lo = (int)((c[j] & 15) ^ 8) - 8;    // signed nibble = q - 8
        const int hi = (int)((c[j] >> 4) ^ 8) - 8;
        o[j] = (float)lo * d;
        o[j + 16] = (float)hi * d;
      } else {
        o[h * 16 + j] = (float)(int8_t)c[j] * d;
      }
    }
  }
}

hipError_t launch_dequant(const Packed& W, float* out, hipStream_t s) {
  const int64_t n = W.rows * W.nblk();
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (W.qt == QT_Q4) k_dequant<QT_Q4><<<grid, 256, 0, s>>>(W, out);
  else k_dequant<QT_Q8><<<grid, 256, 0, s>>>(W, out);
  return hipGetLastError();
}

// ------------------------------------------------------- activation digits

// x [T][n] fp32 -> digits.  One wave quantises two blocks.
__global__ void k_quant_act(int qt, const float* __restrict__ x, int n, int64_t x_ts, Act a) {
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int blk = (blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * 2 + (lane >> 5);
  const int i = blk * QK + (lane & 31);
  const float v = (blk < a.nblk && i < n) ? x[(size_t)t * x_ts + i] : 0.0f;
  const int bsafe = blk < a.nblk ? blk : 0;
  put_digits(a, qt, t, bsafe, v, blk < a.nblk);
}

hipError_t launch_quant_act(int qt, const float* x, int T, int n, int64_t x_ts, Act a, hipStream_t s) {
  const int waves = (a.nblk + 1) / 2;
  const int wpb = 4;
  dim3 grid((waves + wpb - 1) / wpb, T);
  k_quant_act<<<grid, 64 * wpb, 0, s>>>(qt, x, n, x_ts, a);
  return hipGetLastError();
}

// --------------------------------------------------------------------- GEMV

hipError_t launch_gemv(const Packed& W, int T, Act x, NormIn nin, GemvOut out, int ksplit, int waves,
                       hipStream_t s) {
  if (waves < 1 || waves > 8 || ksplit < 1) return hipErrorInvalidValue;
  if (ksplit > 1 && (!out.part || !out.cnt)) return hipErrorInvalidValue;
  if (x.mxd && T >= (x.min_t ? x.min_t : gemm_min_tokens(W.qt, waves)) && gemm_usable(W.qt, T, waves))
    return launch_gemm(W, T, x, nin, out, ksplit, waves, s);
  const bool q4 = W.qt == QT_Q4;
  switch (out.kind) {
    case EPI_STORE: return q4 ? gemv_inst<QT_Q4, EPI_STORE>(W, T, x, nin, out, ksplit, waves, s)
                              : gemv_inst<QT_Q8, EPI_STORE>(W, T, x, nin, out, ksplit, waves, s);
    case EPI_SWIGLU: return q4 ? gemv_inst<QT_Q4, EPI_SWIGLU>(W, T, x, nin, out, ksplit, waves, s)
                               : gemv_inst<QT_Q8, EPI_SWIGLU>(W, T, x, nin, out, ksplit, waves, s);
    case EPI_RESID: return q4 ? gemv_inst<QT_Q4, EPI_RESID>(W, T, x, nin, out, ksplit, waves, s)
                              : gemv_inst<QT_Q8, EPI_RESID>(W, T, x, nin, out, ksplit, waves, s);
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------- boundary vector -> h

// h = boundary input (fp16 or fp32); then digits of norm_w*h and sums of squares.
__global__ void k_resid_finish(int in_kind, const void* in, const Ctrl* ctrl, int64_t in_ts, int T, int H,
                               float* h, const float* __restrict__ norm_w, int qt, Act next, float* ssq_out) {
  const int rg = blockIdx.x;
  const int t = blockIdx.y;
  const int lane = threadIdx.x;
  const int row = rg * RG + lane;
  if (!in) in = ctrl->in;
  float hn = 0.0f;
  if (row < H) {
    if (in_kind == 1) hn = __half2float(reinterpret_cast<const __half*>(in)[(size_t)t * in_ts + row]);
    else hn = reinterpret_cast<const float*>(in)[(size_t)t * in_ts + row];
  }
  resid_tail(t, rg, H, hn, h, H, norm_w, qt, next, ssq_out, (H + RG - 1) / RG);
}

hipError_t launch_resid_finish(int in_kind, const void* in, const Ctrl* ctrl, int64_t in_ts, int T, int H,
                               float* h, const float* norm_w, int qt, Act next, float* ssq_out, hipStream_t s) {
  dim3 grid((unsigned)((H + RG - 1) / RG), T);
  k_resid_finish<<<grid, 64, 0, s>>>(in_kind, in, ctrl, in_ts, T, H, h, norm_w, qt, next, ssq_out);
  return hipGetLastError();
}

}  // namespace slq
