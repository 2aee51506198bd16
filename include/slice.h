/*
 * slice.h -- C ABI of libslq: single-token decode of a contiguous slice of
 * transformer layers with Q4_0 / Q8_0 block-quantised weights, on AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed.  A pipeline stage owns a contiguous range of layers and
 * its own attention cache; per token it takes one hidden state in and hands
 * one hidden state on ("Unstable Legion: the peer-to-peer ChatGPT", sections
 * "Splitting the workload" and "The runtime: legion-stage-runtime").  The
 * hidden state on the wire is 5,120 x f16 for the
 * hybrid model (SwarmLLM README, bench paragraph).  Layers are either
 * Llama-style attention blocks or the qwen3_5 hybrid's Gated DeltaNet and
 * gated full-attention blocks (ChatTorrent README, "What it can run").  Weights
 * are block-quantised (Q4_0: 4-bit codes, one fp16 scale per 32) and each
 * weight is read once per token (SwarmLLM README, architecture paragraph).  Drafts are verified in one batched pass with exact
 * rollback of the recurrent state (same paragraph and feature list).
 *
 * Conventions for every entry point:
 *   - Device pointers are plain HIP device addresses on the current device;
 *     the caller allocates and frees them (the library never allocates or frees
 *     weights, workspace, inputs or outputs).  The caller keeps them alive
 *     until slice_free (or, for the slq_* kernels, until the stream has run).
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *     Work is enqueued asynchronously on it; nothing synchronises the host
 *     unless stated.
 *   - Return value: SLICE_OK (0) or a negative slice_status.  No call throws.
 *     slice_last_error() gives a thread-local message for the last failure.
 *   - Matrices are row-major, y = W x, W has `rows` outputs and `cols` inputs;
 *     cols is a multiple of 32 (one quantisation block).
 */
#ifndef LAYER_SLICE_H
#define LAYER_SLICE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SLICE_OK = 0,
    SLICE_EINVAL = -1,   /* bad argument or configuration                     */
    SLICE_ESHAPE = -2,   /* shape the kernels do not support                  */
    SLICE_ERANGE = -3,   /* position would pass max_seq, or k > max_verify    */
    SLICE_ESTATE = -4,   /* call not allowed in the current state             */
    SLICE_EHIP = -5,     /* a HIP runtime call failed (message has the detail) */
    SLICE_ENOSYS = -6    /* not implemented for this configuration            */
} slice_status;

/* GGUF tensor-type ids of the two weight formats.
 *   Q4_0: 18 bytes per 32 weights: fp16 d (little endian), 16 code bytes;
 *         byte j: weight j in the low nibble, weight j+16 in the high nibble;
 *         value = (nibble - 8) * d.
 *   Q8_0: 34 bytes per 32 weights: fp16 d, 32 int8 codes; value = code * d.  */
enum { SLICE_Q4_0 = 2, SLICE_Q8_0 = 8 };

/* ------------------------------------------------------------------------ */
/* Kernel-level entry points (one matrix at a time)                          */
/* ------------------------------------------------------------------------ */

/* Bytes of the device layout that slq_repack writes for a rows x cols matrix
 * (same bytes per weight as the GGUF blocks, padded to 64-row groups).
 * Returns 0 for an unsupported qtype or cols % 32 != 0.                      */
size_t slq_packed_bytes(int qtype, int64_t rows, int64_t cols);

/* Re-lay GGUF blocks for the GEMV.  raw_dev: rows x (cols/32) blocks exactly as
 * in a GGUF file (device memory).  packed_dev: slq_packed_bytes() bytes.  The
 * repacked layout groups 64 rows x 8 blocks into 16-byte-aligned tiles (codes
 * apart from scales) so that every lane streams whole blocks with 128-bit
 * loads; it holds the same codes and fp16 scales, nothing is rounded.        */
int slq_repack(int qtype, const void *raw_dev, int64_t rows, int64_t cols,
               void *packed_dev, void *stream);

/* Decode a packed matrix to fp32, out_dev: rows x cols.  Every value
 * (q-8)*d or q*d is exact in fp32, so this equals the GGUF decode bit for bit. */
int slq_dequant(int qtype, const void *packed_dev, int64_t rows, int64_t cols,
                float *out_dev, void *stream);

/* Workspace bytes slq_gemv needs for `batch` right-hand sides.               */
size_t slq_gemv_workspace_bytes(int qtype, int64_t rows, int64_t cols, int batch);

/* Y = W X for batch right-hand sides (1 <= batch <= 16): x_dev fp32
 * [batch][cols], y_dev fp32 [batch][rows], ws_dev at least
 * slq_gemv_workspace_bytes() bytes and zero-filled before its first use (the
 * calls leave the counters in it at zero again, so a workspace can be reused
 * without clearing; calls that share one workspace must not overlap).  Each
 * weight is read once for all right-hand sides.  Two kernel launches, no
 * memory set, so the call can be captured in a HIP graph.                   */
int slq_gemv(int qtype, const void *packed_dev, int64_t rows, int64_t cols, int batch,
             const float *x_dev, float *y_dev, void *ws_dev, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* Slice executor                                                            */
/* ------------------------------------------------------------------------ */

typedef struct slice slice_t;   /* opaque: positions, state-slot indices, HIP graphs */

typedef struct slice_config {
    int32_t hidden;                 /* H: width of the hidden state                     */
    int32_t n_layers;               /* layers of the whole model                        */
    int32_t layer_begin, layer_end; /* this slice runs layers [begin, end)              */
    int32_t attn_period;            /* 0: every layer is attention; P > 0: layer l is
                                       attention iff l % P == P-1, else Gated DeltaNet  */
    int32_t dn_heads, dn_dk, dn_dv; /* DeltaNet heads and key / value widths            */
    int32_t q_heads, kv_heads, head_dim, rope_dims;
    double  rope_theta;
    int32_t qk_norm;                /* RMSNorm per head on q and k before RoPE          */
    int32_t attn_gate;              /* output multiplied by sigmoid(W_g x)              */
    float   eps;                    /* RMSNorm epsilon                                  */
    float   dn_a_scale, dn_a_bias;  /* alpha = sigmoid(a_scale * (W_a x) + a_bias)      */
    float   dn_b_scale;             /* beta  = sigmoid(b_scale * (W_b x))               */
    float   dn_z_scale;             /* gate  = sigmoid(z_scale * (W_z x))               */
    int32_t ffn;                    /* SwiGLU width; 0 = the layer has no FFN           */
    int32_t vocab, has_embed, has_head, tied_head;
    int32_t max_seq;                /* KV rows per attention layer                      */
    int32_t max_verify;             /* largest k for slice_verify (<= 16)               */
    int32_t qtype;                  /* SLICE_Q4_0 or SLICE_Q8_0                         */
    int32_t io_fp32;                /* boundary vectors: 0 = fp16, 1 = fp32             */
} slice_config;

/* Tensor ids for slice_set_tensor.  Matrices take raw GGUF blocks
 * (rows x cols/32 blocks, device); vectors take fp32 (device).
 *   layer tensors: attention layers use WQ, WG (if attn_gate), WK, WV, WO,
 *   Q_NORM/K_NORM (if qk_norm); DeltaNet layers use DN_Q/K/V ([heads*dk or
 *   heads*dv] x H), DN_A/DN_B ([heads] x H), DN_Z ([heads*dv] x H), DN_OUT
 *   (H x [heads*dv]); every layer uses ATTN_NORM, and FFN_NORM, W_GATE, W_UP
 *   (ffn x H), W_DOWN (H x ffn) if ffn > 0.
 *   global tensors (layer argument ignored): EMBED (vocab x H), HEAD (if not
 *   tied), OUT_NORM.                                                         */
enum {
    SLICE_T_ATTN_NORM = 0, SLICE_T_FFN_NORM = 1,
    SLICE_T_DN_Q = 10, SLICE_T_DN_K = 11, SLICE_T_DN_V = 12, SLICE_T_DN_A = 13,
    SLICE_T_DN_B = 14, SLICE_T_DN_Z = 15, SLICE_T_DN_OUT = 16,
    SLICE_T_WQ = 20, SLICE_T_WG = 21, SLICE_T_WK = 22, SLICE_T_WV = 23, SLICE_T_WO = 24,
    SLICE_T_Q_NORM = 25, SLICE_T_K_NORM = 26,
    SLICE_T_W_GATE = 30, SLICE_T_W_UP = 31, SLICE_T_W_DOWN = 32,
    SLICE_T_EMBED = 40, SLICE_T_HEAD = 41, SLICE_T_OUT_NORM = 42
};

/* Bytes of the weights buffer (packed layout of every tensor of the slice)
 * and of the workspace (KV caches, DeltaNet state slots, activations, the
 * RoPE rotation table).  0 means the configuration is invalid (see
 * slice_last_error).                                                        */
size_t slice_weights_bytes(const slice_config *cfg);
size_t slice_workspace_bytes(const slice_config *cfg);

/* Bind a slice to caller-owned device buffers (weights_dev: weights_bytes,
 * workspace_dev: workspace_bytes, both 256-byte aligned).  Validates the
 * configuration, carves the workspace, zeroes it and builds the RoPE table
 * in it on `stream`.  Weights are filled afterwards with slice_set_tensor.
 * Position 0, state slot 0.  The caller does not write to either buffer
 * while the slice is loaded, except through these calls.                   */
int slice_load(const slice_config *cfg, void *weights_dev, void *workspace_dev,
               void *stream, slice_t **out);

/* Repack / copy one tensor into the weights buffer (see the tensor ids). */
int slice_set_tensor(slice_t *s, int layer, int tensor_id, const void *src_dev, void *stream);

/* Set the decode position to kv_len (rows [0, kv_len) of every KV cache are
 * the context) and drop any uncommitted verify.  DeltaNet states are left as
 * they are. */
int slice_reset(slice_t *s, int kv_len, void *stream);

/* One decode step at the current position p: hid_in_dev [H] -> hid_out_dev [H]
 * (fp16 or fp32 per io_fp32).  Appends K/V row p, updates every DeltaNet state
 * in place, then p <- p + 1.  ESTATE while a verify is uncommitted, ERANGE if
 * p + 1 > max_seq.  One graph launch per call. */
int slice_decode(slice_t *s, const void *hid_in_dev, void *hid_out_dev, void *stream);

/* Op kinds reported by slice_decode_profiled. */
enum {
    SLICE_OP_ENTRY = 0,      /* boundary vector in, first RMSNorm statistics          */
    SLICE_OP_DN_IN = 1,      /* DeltaNet input projections [q|k|v|a|b|z] (GEMV)        */
    SLICE_OP_DELTANET = 2,   /* DeltaNet state update and gated output                */
    SLICE_OP_DN_OUT = 3,     /* DeltaNet output projection + residual (GEMV)          */
    SLICE_OP_ATT_IN = 4,     /* attention input projections [q|g|k|v] (GEMV)          */
    SLICE_OP_ATTENTION = 5,  /* QK-norm, RoPE, KV append, split attention, combine    */
    SLICE_OP_ATT_OUT = 6,    /* attention output projection + residual (GEMV)         */
    SLICE_OP_FFN_IN = 7,     /* RMSNorm + fused gate/up projection + SwiGLU (GEMV)    */
    SLICE_OP_FFN_OUT = 8,    /* down projection + residual (GEMV)                     */
    SLICE_OP_EXIT = 9        /* boundary vector out                                   */
};

/* Same as slice_decode, but launched op by op (no graph) with a HIP event on
 * `stream` at every op boundary; waits for the step to finish.  Writes, in
 * order, the kind and the duration in ms of each op (at most max_ops) and
 * returns how many were written (>= 0) or a negative slice_status. */
int slice_decode_profiled(slice_t *s, const void *hid_in_dev, void *hid_out_dev,
                          int *op_kind, float *op_ms, int max_ops, void *stream);

/* Launch, back to back on `stream`, the GEMV of one op kind (SLICE_OP_DN_IN,
 * _DN_OUT, _ATT_IN, _ATT_OUT, _FFN_IN or _FFN_OUT) for every layer of the
 * slice that has it, on the activations the last decode left in the
 * workspace; nothing else runs.  For timing one kernel in isolation.  The
 * residual-update kinds (_OUT) modify the workspace copy of h, which the next
 * decode overwrites; DeltaNet states, KV caches and the position are not
 * touched. */
int slice_run_gemv_op(slice_t *s, int op_kind, void *stream);

/* Batched verify of k inputs at positions p .. p+k-1: hid_in_dev [k][H] ->
 * hid_out_dev [k][H].  Output t equals what slice_decode would give after the
 * first t inputs.  The weights are read once for all k tokens.  The DeltaNet
 * state before the call is kept intact; the state after each token goes to its
 * own slot.  Must be followed by slice_commit before the next decode/verify.  */
int slice_verify(slice_t *s, int k, const void *hid_in_dev, void *hid_out_dev, void *stream);

/* Prompt ingestion of k inputs (1..max_verify) at positions p .. p+k-1:
 * hid_in_dev [k][H] -> hid_out_dev [k][H] (caller-owned device buffers in the
 * boundary format), then p <- p + k (no commit).  The result is that of k
 * slice_decode calls up to floating-point rounding, not bit for bit: the
 * DeltaNet layers take all k tokens at once in the chunked form of the
 * recurrence and keep only the final state (the pages name the serial
 * recurrence as what makes prefill slow; SwarmLLM README, bench paragraph),
 * and the products use launch shapes of their own, so their sums run in
 * another order.  For a bit-exact pass use slice_verify + slice_commit(k).
 * Errors: SLICE_EINVAL for a null argument, SLICE_ESTATE while a verify is
 * pending, SLICE_ERANGE for k or positions out of range; nothing is enqueued
 * then.  */
int slice_prefill(slice_t *s, int k, const void *hid_in_dev, void *hid_out_dev, void *stream);

/* Accept the first `accepted` (0..k) tokens of the pending verify: the state
 * becomes exactly the state after that many plain steps (a slot switch; no
 * values are recomputed) and p <- p + accepted.  Enqueues one tiny kernel.  */
int slice_commit(slice_t *s, int accepted, void *stream);

/* First stage: hid_out_dev [H] <- dequantised embedding row *tok_dev. */
int slice_embed(slice_t *s, const int32_t *tok_dev, void *hid_out_dev, void *stream);

/* Last stage: final RMSNorm, logits = W_head x (W_head = EMBED if tied),
 * greedy token = argmax (lowest index wins an exact tie).  logits_dev
 * ([vocab] fp32) may be NULL. */
int slice_head_argmax(slice_t *s, const void *hid_in_dev, int32_t *tok_dev,
                      float *logits_dev, void *stream);

int  slice_position(const slice_t *s);
void slice_free(slice_t *s);        /* releases host objects and graphs only */
const char *slice_last_error(void);

/* ---- state access for tests and synthetic prior context ----
 * DeltaNet state of `layer` in canonical layout fp32 [dn_heads][dv][dk]
 * (S[h][i][j]: i indexes values, j keys), current slot.                   */
int slice_dbg_set_state(slice_t *s, int layer, const float *src_dev, void *stream);
int slice_dbg_get_state(slice_t *s, int layer, float *dst_dev, void *stream);
/* KV rows [0, rows) of attention `layer`, canonical fp16 [kv_heads][rows][head_dim]. */
int slice_dbg_set_kv(slice_t *s, int layer, const uint16_t *k_dev, const uint16_t *v_dev,
                     int rows, void *stream);
int slice_dbg_get_kv(slice_t *s, int layer, uint16_t *k_dev, uint16_t *v_dev,
                     int rows, void *stream);

/* fp32 residual stream h [k][hidden] at the end of the last decode (k = 1) or
 * verify (k tokens) step, before the boundary conversion.  For checking
 * results when the boundary is fp16 and |h| passes the fp16 range. */
int slice_dbg_get_hidden(slice_t *s, float *dst_dev, int k, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* LAYER_SLICE_H */
