// Internal declarations shared by the HIP sources of libslq (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>
#include <stddef.h>

namespace slq {

constexpr int QK = 32;          // weights per block
constexpr int TB = 8;           // blocks per tile along K
constexpr int RG = 64;          // rows per row group: one row per lane of a wave64
constexpr int XW = 24;          // digit dwords per activation block (both formats)
constexpr int MAX_T = 16;       // tokens per batched pass (verify, the mixers' kernels)
constexpr int MAX_PASS = 64;    // tokens per prompt pass (products in token groups of 16)
constexpr int QT_Q4 = 2;
constexpr int QT_Q8 = 8;

// Bytes of one row's codes for one block in the packed layout.
__host__ __device__ constexpr int code_bytes(int qt) { return qt == QT_Q4 ? 16 : 32; }
// Bytes of one full tile: 8 blocks x 64 rows of codes + 64 rows x 8 fp16 scales.
__host__ __device__ constexpr int tile_bytes(int qt) { return TB * RG * code_bytes(qt) + RG * TB * 2; }

struct Packed {
  const uint8_t* w;   // packed bytes
  int64_t rows, cols;
  int qt;
  __host__ __device__ int nblk() const { return (int)(cols / QK); }
  __host__ __device__ int ntiles() const { return (nblk() + TB - 1) / TB; }
  __host__ __device__ int nrg() const { return (int)((rows + RG - 1) / RG); }
};

// Bytes of one 64-row group (all tiles along K; the last tile may hold < 8 blocks).
__host__ __device__ inline size_t rg_bytes(int qt, int64_t cols) {
  int nb = (int)(cols / QK);
  int full = nb / TB, tail = nb % TB;
  size_t b = (size_t)full * tile_bytes(qt);
  if (tail) b += (size_t)tail * RG * code_bytes(qt) + RG * TB * 2;
  return b;
}
inline size_t packed_bytes(int qt, int64_t rows, int64_t cols) {
  return (size_t)((rows + RG - 1) / RG) * rg_bytes(qt, cols);
}

// ---------------------------------------------------------------- activations
// An activation vector of n = 32*nblk floats is handed to a GEMV as integer
// digits: per block b, scale s_b = max|x| / M and x_int = rint(x / s_b), split
// into balanced digits (Q4_0: six base-16 digits in [-8,7]; Q8_0: three base-256
// digits in [-128,127]) and packed in the order the weight codes use, so the
// GEMV takes exact integer dot products of codes and digits.
//
// Two layouts of the same digits (a producer writes both when mxd is set):
//   lane-row layout (single-token GEMV): xd [T][nblk][24 dwords], xs [T][nblk].
//   MFMA layout (batched products, 16 token slots): one record per block of
//     NCH chunks of 16 slots x 16 bytes (slot = token), then the 16 token
//     scales (fp32), so that one buffer holds everything a block needs.
//     Q4_0 (NCH 12): c = 4p + g, p = 0..2 digit pair, g = 0..3; byte j of chunk
//           (p, g) is digit 2p of element 16(g&1)+j for g < 2 and 16 * digit 2p+1
//           of that element for g >= 2 (one 64-deep int8 MFMA takes two digits).
//     Q8_0 (NCH 6): c = 2p + h, p = 0..2 digit; byte j is digit p of element 16h+j.
struct Act {
  int32_t* xd;
  float* xs;
  int nblk;      // blocks per token
  int32_t* mxd;  // MFMA layout records, or nullptr (not written); tokens 16 g .. 16 g + 15
                 // of block b in the record at mxd + (g nblk + b) mx_block_bytes / 4
  int min_t;     // calls with at least this many tokens use the MFMA products (when they
                 // fit); 0: the measured default, gemm_min_tokens
};
constexpr int MX_SLOTS = 16;
// Token groups of 16 a batched product multiplies at once: past 16 tokens
// (prompt passes) the dense form gives each of 2 or 4 groups its own waves (a
// group past the last token multiplies whatever its records hold and is never
// read), so the records of every such group must exist.
__host__ __device__ constexpr int gemm_groups(int T) { return T <= MX_SLOTS ? 1 : T <= 2 * MX_SLOTS ? 2 : 4; }
__host__ __device__ constexpr int mx_chunks(int qt) { return qt == QT_Q4 ? 12 : 6; }
// Bytes of one block's MFMA-layout record: digits, then the token scales at
// byte mx_scale_off(qt).
__host__ __device__ constexpr int mx_scale_off(int qt) { return mx_chunks(qt) * MX_SLOTS * 16; }
__host__ __device__ constexpr int mx_block_bytes(int qt) { return mx_scale_off(qt) + MX_SLOTS * 4; }

constexpr float M_Q4 = 7829367.0f;   // 7 * 0x111111
constexpr float M_Q8 = 8355711.0f;   // 127 * 0x010101

// RMSNorm statistic handed from a producer to a consumer GEMV: per token,
// n_part partial sums of squares; rnorm = 1 / sqrt(sum / n + eps).
struct NormIn {
  const float* ssq;   // [T][n_part] or nullptr (no normalisation)
  int n_part;
  float inv_n, eps;
};

// GEMV epilogues
enum Epi {
  EPI_STORE = 0, EPI_SWIGLU = 2, EPI_RESID = 3,
  EPI_DN = 7,          // chained DeltaNet decode phase
  EPI_ATT_COMB = 9     // chained attention merge (four (head, 64-dim) merges per workgroup)
};

// With ksplit > 1 the K tiles of a 64-row group are spread over ksplit
// workgroups; each publishes its partial sums, and the last one to finish
// (atomic ticket per row group) adds them in split order and runs the epilogue.
struct GemvOut {
  int kind;
  float* y;            // STORE: [T][rows]; SWIGLU: m [T][rows/2] (nullable);
                       // RESID: residual h [T][rows] updated in place
  int64_t y_tstride;   // token stride of y in floats
  Act next;            // SWIGLU/RESID: digits of the next GEMV input
  int next_qt;
  float* ssq_out;      // RESID: [T][nrg] sums of squares of h
  const float* norm_w; // RESID: weights of the next RMSNorm (digits are of w*h)
  float* part;         // ksplit > 1: partial sums [nrg][ksplit][T][64]
  unsigned* cnt;       // ksplit > 1: one ticket counter per row group, zero before and after
};

struct Ctrl {         // device-resident step control
  int pos;            // decode position p
  int cur;            // current DeltaNet state slot
  const void* in;     // boundary input of the step being run
  void* out;          // boundary output of the step being run
  int err;            // non-zero: a bounded wait inside a kernel gave up
  int pad[57];
};

// -------------------------------------------------------------------- launchers
// All return hipError_t from the launch.
hipError_t launch_repack(int qt, const uint8_t* raw, int64_t rows, int64_t cols, uint8_t* packed,
                         int64_t dst_rows, int map_kind, int64_t row_off, hipStream_t s);
hipError_t launch_dequant(const Packed& W, float* out, hipStream_t s);
// x fp32 [T][n] -> digits; optional ssq partials [T][nrg] of x (not of w*x).
hipError_t launch_quant_act(int qt, const float* x, int T, int n, int64_t x_tstride, Act a,
                            hipStream_t s);
// The int8-MFMA product when x carries MFMA-layout digits, T >= x.min_t and
// its LDS fits; otherwise the one-row-per-lane GEMV.  Same results either way.
hipError_t launch_gemv(const Packed& W, int T, Act x, NormIn nin, GemvOut out, int ksplit,
                       int waves, hipStream_t s);
hipError_t launch_gemm(const Packed& W, int T, Act x, NormIn nin, GemvOut out, int ksplit,
                       int waves, hipStream_t s);
bool gemm_usable(int qt, int T, int waves);
// Fewest tokens for which the MFMA products beat the per-token integer dot
// products (measured on MI355X over the slice's shapes): Q8_0 from 2 tokens;
// Q4_0 from 4 tokens with at most 4 waves per workgroup, from 8 with more
// (the batched kernels stream fewer tiles per wave as waves are added).
int gemm_min_tokens(int qt, int waves);
// h [T][H] = boundary input, then digits of norm_w*h and ssq partials.
// in_kind: 1 = fp16 input, 2 = fp32 input; with in == nullptr the input pointer
// is read from ctrl->in.
hipError_t launch_resid_finish(int in_kind, const void* in, const Ctrl* ctrl, int64_t in_tstride,
                               int T, int H, float* h, const float* norm_w, int qt, Act next,
                               float* ssq_out, hipStream_t s);
// out == nullptr: write to ctrl->out.  advance_pos: added to ctrl->pos.
hipError_t launch_store_out(const float* h, int T, int H, void* out, int fp32, Ctrl* ctrl,
                            int advance_pos, hipStream_t s);
hipError_t launch_ctrl_io(Ctrl* c, const void* in, void* out, hipStream_t s);
// p[0..n) = 0 with a kernel (usable where a memset node is not wanted)
hipError_t launch_fill_zero_u32(uint32_t* p, size_t n, hipStream_t s);
hipError_t launch_read_probe(const void* p, size_t n16, uint32_t* sink, unsigned grid, hipStream_t s);
hipError_t launch_ctrl_set(Ctrl* c, int pos, int cur, hipStream_t s);
hipError_t launch_embed(const Packed& E, const int32_t* tok, void* out, int fp32, hipStream_t s);
// digits of [RMSNorm(E[*tok]) w_e ; RMSNorm(hin) w_h] (x: 2 H / 32 blocks, one token)
hipError_t launch_mtp_input(const Packed& E, const int32_t* tok, const void* hin, int fp32, const float* w_e,
                            const float* w_h, float eps, Act x, hipStream_t s);
hipError_t launch_argmax(const float* logits, int n, float* part_v, int* part_i, int nparts,
                         int32_t* tok, hipStream_t s);


// DeltaNet update modes: DN_DECODE updates slot cur in place (one token);
// DN_VERIFY writes the state after token t to slot (cur+1+t) % nslots and
// leaves slot cur intact; DN_CHUNK takes all tokens at once in the chunked
// form and leaves only the final state, in slot cur.
enum { DN_DECODE = 0, DN_VERIFY = 1, DN_CHUNK = 2 };

struct DnParams {
  const float* y;        // G1 output [T][y_stride]
  int64_t y_stride;
  int off_q, off_k, off_v, off_a, off_b, off_z;
  int heads, dk, dv;
  float a_scale, a_bias, b_scale, z_scale;
  float* state;          // slot 0 of this layer: [nslots][heads][dv/8][dk/8][8][8] (see k_deltanet)
  int nslots;
  int mode;              // DN_DECODE, DN_VERIFY or DN_CHUNK (below)
  const Ctrl* ctrl;      // state slot index ctrl->cur; nullptr: slot 0
  float* u_out;          // [T][heads*dv] (nullable)
  Act next; int next_qt; // digits of the output (next.xd == nullptr: none)
  // qwen3_5 form (variant 1): conv over q | k | v (k_heads query/key heads of
  // dk, heads value heads of dv), decay exp(-exp(a_log) softplus(.)), gated norm
  int variant, k_heads, conv;
  float eps;                  // gated-norm epsilon
  const float* conv_w;        // [conv_dim][conv]
  const float* a_log;         // [heads]
  const float* dt_bias;       // [heads]
  const float* norm_w;        // [dv]
  float* conv_state;          // slot 0: [nslots][conv_dim][conv - 1]
  int64_t conv_slot;          // floats per slot
};
hipError_t launch_deltanet(const DnParams& p, int T, hipStream_t s);
hipError_t launch_state_io(float* state, int nslots, const Ctrl* ctrl, int heads, int dk, int dv,
                           float* canon, int to_device, hipStream_t s);

struct AttnParams {
  const float* y;        // G1 output [T][y_stride]
  int64_t y_stride;
  int off_q, off_g, off_k, off_v;   // off_g < 0: no gate
  int q_heads, kv_heads, hd, rope_dims;
  double rope_theta;
  const float* rope_cs;  // [max_seq][rope_dims / 2][2]: cos, sin of the RoPE angle
  int qk_norm;
  const float* q_norm; const float* k_norm;
  float eps;
  __half* kc;            // K cache, tiled: [kv][max_seq/64][hd/8][64][8]
  __half* vc;            // V cache: [kv][max_seq][hd]
  int max_seq;
  const Ctrl* ctrl;      // position ctrl->pos; nullptr: pos below
  int pos;
  int pos_off;           // added to that position (token t sits at position + pos_off + t)
  float* part;           // [T][q_heads][nchunk][hd + 2]: one partial per rchunks chunks
  int nchunk;            // max_seq / chunk
  int rchunks;           // chunks per partial (set by launch_attention from the cache size)
  float* u_out;          // [T][q_heads*hd] (nullable)
  Act next; int next_qt; // digits of the output (next.xd == nullptr: none)
  int split_only;        // 1: one token on at most 64 partials, merged later by the chained decode
                         // kernel's first phase (launch_attention runs the split only)
};
constexpr int ATT_CHUNK = 32;    // KV rows per split-attention workgroup
hipError_t launch_attention(const AttnParams& p, int T, hipStream_t s);
hipError_t launch_rope_table(float* cs, int max_seq, int rope_dims, double theta, hipStream_t s);
hipError_t launch_kv_io(__half* kc, __half* vc, int kv_heads, int max_seq, int hd,
                        uint16_t* k, uint16_t* v, int rows, int to_device, hipStream_t s);

// ------------------------------------------------------- chained single-token GEMVs
// One kernel runs up to CHAIN_MAX_PHASES dependent phases of a decode step,
// in step order and across layers: a DeltaNet layer's recurrent update
// (EPI_DN), its mixer output projection, the gate/up projection, the down
// projection, the next layer's input projections, then the next DeltaNet
// layer's update, and so on.  A phase's workgroups first request what does
// not depend on the phase before (a GEMV its first weight tile, an update
// its state rows), then wait until every row group of the phase before has
// finished, then compute exactly what the separate kernel computes
// (chain.hip).
constexpr int CHAIN_MAX_PHASES = 20;
// split-K partial and ticket regions, taken in turn by the phases of a launch
constexpr int CHAIN_PART_BUFS = 5;
// per phase of a chain launch: 33 counter lines, then 64 ready-flag lines
constexpr int CHAIN_PHASE_LINES = 33 + 64;
constexpr int CHAIN_PHASE_SYNC_BYTES = CHAIN_PHASE_LINES * 128;
struct ChainPhase {   // one GEMV of the chain; lives in device memory
  // every location is a byte offset: weights and norm weights into the
  // weights buffer, everything else into the workspace.  EPI_DN: y_off is
  // the layer's state (slot 0), nd_off / ns_off its output digits; the rest
  // of the update's parameters come from ChainArgs::dn.  EPI_ATT_COMB: nd_off / ns_off
  // its output digits; the rest from ChainArgs::att
  int64_t w_off, rows, cols;          // packed matrix
  int64_t xd_off, xs_off;             // input digits and their block scales
  int64_t ssq_off;                    // RMSNorm partial sums of the input (-1: none)
  int64_t y_off, y_tstride;           // STORE: y; RESID: h; SWIGLU: -1
  int64_t nd_off, ns_off;             // SWIGLU / RESID: output digits and scales
  int64_t ssq_out_off;                // RESID: sums of squares of h
  int64_t norm_w_off;                 // RESID: weights of the next RMSNorm
  int64_t part_off, cnt_off;          // split-K partials and tickets
  int x_nblk, n_nblk;                 // blocks per token of the input / output digits
  int n_part;                         // partial sums per token of the input statistics
  float inv_n, eps;                   // RMSNorm of the input: 1 / width, epsilon
  int qt;                             // weight format (also of the output digits)
  int ksplit;                         // split-K workgroups per row group
  int nwg;                            // workgroups of this phase: row groups x ksplit
  int epi;                            // EPI_STORE, EPI_SWIGLU, EPI_RESID, or EPI_DN / EPI_ATT_COMB (rows = nwg workgroups)
  int w;                              // waves of the product (<= 4; the others idle)
};
// Kernel arguments of one chained launch (by value, so the workgroups read
// their product's descriptor without a dependent memory load).
struct ChainArgs {
  ChainPhase ph[CHAIN_MAX_PHASES];
  int nph;
  int first_wg[CHAIN_MAX_PHASES + 1];   // workgroup index where product p starts; [nph] = grid
  int gsize[CHAIN_MAX_PHASES];          // row groups per completion group of product p
  DnParams dn;                          // the EPI_DN phases: one decode token (T = 1); state and
                                        // output digits per phase (ChainPhase)
  int dn_dkp;                           // its d_k / 8
  AttnParams att;                       // the EPI_ATT_COMB phases: one decode token; output digits
                                        // per phase (ChainPhase)
};
// sync region of one chain launch (nph * CHAIN_PHASE_SYNC_BYTES, zero before
// its first launch), each counter and flag in its own 128-byte line (u32
// index), in block p = 32 * CHAIN_PHASE_LINES * p of product p:
//   [block + 32 g], g < 32: row groups of group g of product p finished (over
//                    all launches); g = 32: groups of product p finished;
//   [block + 32 (33 + c)]: copy c of product p's ready flag, the last launch
//                    (1, 2, ...) whose product p is complete.
hipError_t launch_chain(int qt, const ChainArgs& args, unsigned grid, const uint8_t* weights, uint8_t* ws,
                        unsigned* sync, Ctrl* ctrl, hipStream_t s);
// ctrl->err = 0 and the sync regions cleared (n_u32 words)
hipError_t launch_chain_reset(unsigned* sync, size_t n_u32, Ctrl* ctrl, hipStream_t s);


}  // namespace slq
