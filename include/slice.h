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
 * Returns 0 for an unsupported qtype or cols % 32 != 0.  The weights are the
 * GGUF Q4_0 / Q8_0 blocks the pages' models ship in (SwarmLLM README, model
 * table; its repo layout has the GGUF reader repack quantised blocks at load). */
size_t slq_packed_bytes(int qtype, int64_t rows, int64_t cols);

/* Re-lay GGUF blocks for the GEMV.  raw_dev: rows x (cols/32) blocks exactly as
 * in a GGUF file (device memory).  packed_dev: slq_packed_bytes() bytes.  The
 * repacked layout groups 64 rows x 8 blocks into 16-byte-aligned tiles (codes
 * apart from scales) so that every lane streams whole blocks with 128-bit
 * loads; it holds the same codes and fp16 scales, nothing is rounded.        */
int slq_repack(int qtype, const void *raw_dev, int64_t rows, int64_t cols,
               void *packed_dev, void *stream);

/* Decode a packed matrix to fp32, out_dev: rows x cols.  Every value
 * (q-8)*d or q*d is exact in fp32, so this equals the GGUF decode bit for bit
 * (the 4-bit blocks with fp16 scales of the SwarmLLM README, engine paragraph).
 * Test access: the dequantised weights are compared with the oracle's.        */
int slq_dequant(int qtype, const void *packed_dev, int64_t rows, int64_t cols,
                float *out_dev, void *stream);

/* Workspace bytes slq_gemv needs for `batch` right-hand sides (0 for an
 * unsupported qtype, shape, or batch outside 1..16).                        */
size_t slq_gemv_workspace_bytes(int qtype, int64_t rows, int64_t cols, int batch);

/* Y = W X for batch right-hand sides (1 <= batch <= 16): the weight-streaming
 * product that dominates decode, where every token reads every weight once
 * (SwarmLLM README, engine paragraph); batch > 1 is the batched form a verify
 * pass uses (same README, feature list).  x_dev fp32
 * [batch][cols], y_dev fp32 [batch][rows], ws_dev at least
 * slq_gemv_workspace_bytes() bytes and zero-filled before its first use (the
 * calls leave the counters in it at zero again, so a workspace can be reused
 * without clearing; calls that share one workspace must not overlap).  Each
 * weight is read once for all right-hand sides.  Two kernel launches, no
 * memory set, so the call can be captured in a HIP graph.                   */
int slq_gemv(int qtype, const void *packed_dev, int64_t rows, int64_t cols, int batch,
             const float *x_dev, float *y_dev, void *ws_dev, size_t ws_bytes, void *stream);

/* Bytes of the static device scratch of slq_gemv_noalloc (16 MiB per GPU). */
#define SLQ_GEMV_NOALLOC_SCRATCH_BYTES (16u << 20)

/* slq_gemv for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, kernels and results (bit for bit) as slq_gemv, but the
 * workspace is a file-scope device array of SLQ_GEMV_NOALLOC_SCRATCH_BYTES
 * that the library holds on every GPU it runs on until the process ends; no
 * call allocates or frees memory.  SLICE_ESHAPE when the shape needs more
 * scratch than that (slq_gemv_workspace_bytes() > the limit; every shape with
 * rows <= 262144 and cols <= 32768 fits at any batch), or for an unsupported
 * qtype, shape or batch; SLICE_EINVAL for a null pointer; SLICE_EHIP if the
 * scratch's device address cannot be obtained.  Three kernel launches: the
 * row-group tickets are cleared by a fill kernel, then the two of slq_gemv.
 * All calls on one GPU share its scratch, which keeps the last call's
 * contents: calls that overlap in time on one GPU (different streams or
 * threads without ordering between them) race and give wrong results.     */
int slq_gemv_noalloc(int qtype, const void *packed_dev, int64_t rows, int64_t cols, int batch,
                     const float *x_dev, float *y_dev, void *stream);

/* Streaming-read ceiling of the device: reads `bytes` (a multiple of 16) at
 * buf_dev once, as the GEMVs read weights (nontemporal 16-byte loads, sixteen
 * in flight per lane, up to SLQ_READ_PROBE_GRID workgroups of 256), and
 * stores an XOR fold of what it read to sink_dev (SLQ_READ_PROBE_GRID * 4
 * uint32; the XOR of all of them is the XOR of every 32-bit word read).  The
 * pages judge their decode against the read bandwidth they measured on their
 * device (SwarmLLM README, bench paragraph); timing this call over a buffer
 * well beyond the last-level cache gives that ceiling here.  SLICE_EINVAL for
 * a null pointer or a size that is not a positive multiple of 16.           */
#define SLQ_READ_PROBE_GRID 16384
int slq_read_probe(const void *buf_dev, size_t bytes, uint32_t *sink_dev, void *stream);

/* ------------------------------------------------------------------------ */
/* Mixers on caller buffers (kernel level)                                   */
/* ------------------------------------------------------------------------ */

/* Gated DeltaNet, the hybrid's linear-attention layers (ChatTorrent README,
 * "What it can run"), one token after the other as the pages' engine runs
 * the recurrence (SwarmLLM README, bench paragraph).  Per head h and token t:
 *   q^ = q / sqrt(sum q^2 + 1e-6), k^ likewise; alpha = sigmoid(a),
 *   beta = sigmoid(b); S <- alpha S (I - beta k^ k^T) + beta v k^T;
 *   o = S q^; out = o * sigmoid(z) elementwise.
 * in_dev: fp32 [T][ q (heads x dk) | k (heads x dk) | v (heads x dv) |
 *   a (heads) | b (heads) | z (heads x dv) ]: the pre-activations of the decay,
 *   write strength and output gate are inputs here (in a slice they come from
 *   the layer's projections).  state_dev: fp32 heads x dv x dk in the
 *   library's layout (slq_dn_state_layout converts), read and updated in place
 *   to the state after token T-1.  out_dev: fp32 [T][heads x dv].
 * T in 1..16; dk in {32, 64, 96, 128}; dv a multiple of 32.  The same kernel
 * as a slice's decode step.  Errors: SLICE_ESHAPE, SLICE_ERANGE (T),
 * SLICE_EINVAL (null pointer); nothing is enqueued then.                     */
int slq_dn_step(int heads, int dk, int dv, int T, const float *in_dev, float *state_dev, float *out_dev,
                void *stream);

/* Convert a DeltaNet state between canonical fp32 [heads][dv][dk] (S[h][i][j]:
 * i indexes values, j keys) and the library's layout used by slq_dn_step.
 * to_lib != 0: canon_dev -> lib_dev, else lib_dev -> canon_dev.             */
int slq_dn_state_layout(int heads, int dk, int dv, float *canon_dev, float *lib_dev, int to_lib, void *stream);

/* Decode attention over an fp16 KV cache: the hybrid's full-attention layers
 * (QK-norm, RoPE on part of each head, sigmoid output gate) or Llama-style GQA
 * (ChatTorrent README, "What it can run"), each stage keeping its own cache
 * ("Unstable Legion", "Splitting the workload").                          */
typedef struct slq_attn_desc {
    int32_t q_heads, kv_heads, head_dim; /* query head h reads KV head h / (q_heads / kv_heads) */
    int32_t rope_dims;                   /* entries 0..rope_dims-1 rotated in pairs (i, i + rope_dims/2) */
    double  rope_theta;                  /* angle pos * theta^(-2i / rope_dims), fp64            */
    int32_t qk_norm;                     /* RMSNorm of every q and k head before RoPE           */
    int32_t has_gate;                    /* output multiplied by sigmoid(g)                      */
    float   eps;                         /* QK-norm epsilon                                      */
    int32_t max_seq;                     /* cache rows (multiple of 64)                          */
    const float *q_norm_dev, *k_norm_dev;/* [head_dim] fp32 norm weights (qk_norm only)          */
} slq_attn_desc;

/* Workspace for T tokens (the RoPE table, then split partials); 0 for an
 * invalid descriptor or T outside 1..16.                                    */
size_t slq_attn_workspace_bytes(const slq_attn_desc *d, int T);

/* Build the RoPE table at the start of ws_dev (once per workspace). */
int slq_attn_prepare(const slq_attn_desc *d, void *ws_dev, size_t ws_bytes, void *stream);

/* T tokens at positions pos .. pos+T-1: in_dev fp32 [T][ q (q_heads x hd) |
 * g (q_heads x hd, if has_gate) | k (kv_heads x hd) | v (kv_heads x hd) ].
 * Appends the T new K/V rows (QK-norm, RoPE, fp16 rounding) to the caches at
 * pos .. pos+T-1; query t attends causally to rows 0 .. pos+t with scale
 * 1/sqrt(head_dim).  out_dev: fp32 [T][q_heads x hd] (o, or o * sigmoid(g)).
 * k_cache_dev / v_cache_dev: kv_heads x max_seq x head_dim fp16 each, in the
 * library's layout (slq_kv_layout converts).  ws_dev: slq_attn_workspace_bytes
 * bytes, prepared by slq_attn_prepare for this descriptor.  Errors:
 * SLICE_ESHAPE (descriptor), SLICE_ERANGE (T or positions), SLICE_EINVAL.    */
int slq_attn_decode(const slq_attn_desc *d, int T, int pos, const float *in_dev, uint16_t *k_cache_dev,
                    uint16_t *v_cache_dev, float *out_dev, void *ws_dev, size_t ws_bytes, void *stream);

/* Copy rows [0, rows) between canonical fp16 [kv_heads][rows][head_dim] K and
 * V arrays and caches in the library's layout (to_cache != 0: into the
 * caches).                                                                   */
int slq_kv_layout(int kv_heads, int max_seq, int head_dim, int rows, uint16_t *k_canon_dev, uint16_t *v_canon_dev,
                  uint16_t *k_cache_dev, uint16_t *v_cache_dev, int to_cache, void *stream);

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
    /* The qwen3_5 form of the Gated DeltaNet layers (ChatTorrent README, "What
     * it can run", names the layer kind; the form is the published mixer):
     * dn_variant = 1 runs a depthwise causal conv of width dn_conv (2..4) over
     * the q | k | v projections, then SiLU; dn_k_heads query/key heads are
     * shared by the dn_heads value heads (dn_heads % dn_k_heads == 0); q is
     * L2-normalised then scaled by 1/sqrt(dn_dk); alpha = exp(-exp(A_log) *
     * softplus(a_scale * (W_a x) + dt_bias)), beta = sigmoid(b_scale * (W_b x));
     * each head's output o becomes rmsnorm(o) * w * silu(z_scale * (W_z x)).
     * dn_a_bias is unused then.  dn_variant = 0: the form described above. */
    int32_t dn_variant;
    int32_t dn_k_heads;             /* 0: dn_heads                                      */
    int32_t dn_conv;                /* conv width (dn_variant = 1)                      */
    /* 1: the slice is a draft head (see slice_mtp_input): it also holds the
     * input projection MTP_FC and the norms MTP_NORM_E / MTP_NORM_H, and
     * needs has_embed.  Its layers are normally one attention layer
     * (attn_period 0, layer range [0, 1)), OUT_NORM is the head's own final
     * norm and the head matrix the model's LM head.                       */
    int32_t has_mtp;
    /* Tokens a slice_prefill pass may carry: 0 = max_verify; up to 64 (more
     * than 16 needs dn_variant 0).  The activation buffers are sized for
     * max(max_verify, max_prefill) tokens.                                   */
    int32_t max_prefill;
} slice_config;

/* Tensor ids for slice_set_tensor.  Matrices take raw GGUF blocks
 * (rows x cols/32 blocks, device); vectors take fp32 (device).
 *   layer tensors: attention layers use WQ, WG (if attn_gate), WK, WV, WO,
 *   Q_NORM/K_NORM (if qk_norm); DeltaNet layers use DN_Q/K ([k_heads*dk] x H,
 *   k_heads = dn_k_heads or dn_heads), DN_V ([heads*dv] x H), DN_A/DN_B
 *   ([heads] x H), DN_Z ([heads*dv] x H), DN_OUT (H x [heads*dv]), and with
 *   dn_variant = 1 also DN_CONV, DN_ALOG, DN_DTB, DN_NORM (below); every
 *   layer uses ATTN_NORM, and FFN_NORM, W_GATE, W_UP
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
    SLICE_T_EMBED = 40, SLICE_T_HEAD = 41, SLICE_T_OUT_NORM = 42,
    /* DeltaNet layers with dn_variant = 1 (fp32): DN_CONV [conv_dim][dn_conv]
     * taps (conv_dim = 2*dn_k_heads*dn_dk + dn_heads*dn_dv channels in the
     * order q | k | v, tap dn_conv-1 on the current input), DN_ALOG and DN_DTB
     * [dn_heads], DN_NORM [dn_dv] (gated-norm weights, shared by the heads) */
    SLICE_T_DN_CONV = 17, SLICE_T_DN_ALOG = 18, SLICE_T_DN_DTB = 19, SLICE_T_DN_NORM = 28,
    /* draft head (has_mtp; global, layer argument ignored): MTP_FC (H x 2H,
     * columns 0..H-1 read the embedding side), MTP_NORM_E and MTP_NORM_H
     * (fp32 [H]) */
    SLICE_T_MTP_FC = 43, SLICE_T_MTP_NORM_E = 44, SLICE_T_MTP_NORM_H = 45
};

/* A stage owns the weights, cache and recurrent state of its own layer range
 * ("Unstable Legion", sections "Splitting the workload" and "The runtime:
 * legion-stage-runtime").
 *
 * Bytes of the weights buffer (packed layout of every tensor of the slice)
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

/* Expected source of one tensor for a configuration (host only; no GPU call):
 * a quantised matrix of *rows x *cols weights as GGUF blocks in the slice's
 * format (*kind = cfg->qtype, *src_bytes = rows * cols/32 * 18 or 34), or an
 * fp32 vector of *rows entries (*kind = 0, *cols = 1, *src_bytes = 4 * rows).
 * Any output pointer may be NULL.  SLICE_EINVAL for an invalid configuration
 * or a tensor the slice does not hold (layer outside [begin, end), a tensor
 * of the other layer kind, a gate or FFN the configuration has not).  A loader
 * checks a file's tensors with this before it uploads anything (a stage loads
 * only its own layer range: "Unstable Legion", "Splitting the workload").  */
int slice_tensor_info(const slice_config *cfg, int layer, int tensor_id, int64_t *rows, int64_t *cols,
                      int32_t *kind, size_t *src_bytes);

/* Repack / copy one tensor into the weights buffer (see the tensor ids).
 * src_dev holds src_bytes bytes of device memory: GGUF blocks or fp32
 * values, exactly slice_tensor_info's *src_bytes.  A different byte count
 * returns SLICE_ESHAPE and a tensor the slice does not hold SLICE_EINVAL,
 * both before anything is enqueued, so a mis-shaped file cannot make the
 * repack read past its source.  Asynchronous on `stream`; src_dev must stay
 * valid until the stream has run the copy. */
int slice_set_tensor(slice_t *s, int layer, int tensor_id, const void *src_dev, size_t src_bytes,
                     void *stream);

/* Set the decode position to kv_len (rows [0, kv_len) of every KV cache are
 * the context) and drop any uncommitted verify; clears the condition that
 * slice_sync_check reports.  DeltaNet states are left as they are.  The stage's prior context is its own cache ("Unstable Legion",
 * "Splitting the workload").  SLICE_ERANGE if kv_len is outside 0..max_seq. */
int slice_reset(slice_t *s, int kv_len, void *stream);

/* One decode step at the current position p, activation in, activation out
 * ("Unstable Legion", "The runtime: legion-stage-runtime"; one submission per
 * token as in the SwarmLLM README, engine paragraph): hid_in_dev [H] -> hid_out_dev [H]
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
    SLICE_OP_EXIT = 9,       /* boundary vector out                                   */
    SLICE_OP_CHAIN = 10      /* one chained kernel: the phases of consecutive layers
                                up to the next attention layer (DeltaNet update,
                                mixer output + residual, gate/up + SwiGLU, down +
                                residual, next layer's input projections)          */
};

/* Measurement (the pages' engine ships tok/s harnesses and a kernel-family
 * profiler: SwarmLLM README, repo layout).
 * Same as slice_decode, but launched op by op (no graph) with a HIP event on
 * `stream` at every op boundary; waits for the step to finish.  Writes, in
 * order, the kind and the duration in ms of each op (at most max_ops) and
 * returns how many were written (>= 0) or a negative slice_status. */
int slice_decode_profiled(slice_t *s, const void *hid_in_dev, void *hid_out_dev,
                          int *op_kind, float *op_ms, int max_ops, void *stream);

/* Measurement, as above.
 * Launch, back to back on `stream`, the GEMV of one op kind (SLICE_OP_DN_IN,
 * _DN_OUT, _ATT_IN, _ATT_OUT, _FFN_IN or _FFN_OUT; or SLICE_OP_CHAIN, the
 * chained-product kernel decode uses) for every layer of the
 * slice that has it, on the activations the last decode left in the
 * workspace; nothing else runs.  For timing one kernel in isolation.  The
 * residual-update kinds (_OUT) modify the workspace copy of h, which the next
 * decode overwrites; DeltaNet states, KV caches and the position are not
 * touched. */
int slice_run_gemv_op(slice_t *s, int op_kind, void *stream);

/* Drafts are checked in one batched pass and the recurrent state is rolled
 * back exactly on rejection (SwarmLLM README, feature list and engine
 * paragraph).
 * Batched verify of k inputs at positions p .. p+k-1: hid_in_dev [k][H] ->
 * hid_out_dev [k][H].  Output t equals what slice_decode would give after the
 * first t inputs.  The weights are read once for all k tokens.  The DeltaNet
 * state before the call is kept intact; the state after each token goes to its
 * own slot.  Must be followed by slice_commit before the next decode/verify.  */
int slice_verify(slice_t *s, int k, const void *hid_in_dev, void *hid_out_dev, void *stream);

/* Prompt ingestion of k inputs (1..max(max_verify, max_prefill), at most 64)
 * at positions p .. p+k-1 (the pages batch 16 prompt tokens per round trip,
 * SwarmLLM README, feature list; a stage can take more at once):
 * hid_in_dev [k][H] -> hid_out_dev [k][H] (caller-owned device buffers in the
 * boundary format), then p <- p + k (no commit).  The result is that of k
 * slice_decode calls up to floating-point rounding, not bit for bit: the
 * DeltaNet layers take the tokens in the chunked form of the recurrence, 16
 * at a time, and keep only the final state (the pages name the serial
 * recurrence as what makes prefill slow; SwarmLLM README, bench paragraph),
 * and the products use launch shapes of their own, so their sums run in
 * another order.  Past 16 tokens every product still reads its weights once
 * for all k tokens; the mixers run in sub-passes of 16 tokens, in order.  For
 * a bit-exact pass use slice_verify + slice_commit(k) (k <= 16).
 * Errors: SLICE_EINVAL for a null argument, SLICE_ESTATE while a verify is
 * pending, SLICE_ERANGE for k or positions out of range; nothing is enqueued
 * then.  */
int slice_prefill(slice_t *s, int k, const void *hid_in_dev, void *hid_out_dev, void *stream);

/* Exact rollback of the recurrent state after a verify pass (SwarmLLM README,
 * feature list).  Accept the first `accepted` (0..k) tokens of the pending
 * verify: the state becomes exactly the state after that many plain steps (a
 * slot switch; no values are recomputed) and p <- p + accepted.  Enqueues one
 * tiny kernel on `stream` (the device-side position and slot index), so later
 * work on that stream sees the committed state.  SLICE_ESTATE when no verify
 * is pending, SLICE_ERANGE for accepted outside 0..k.  */
int slice_commit(slice_t *s, int accepted, void *stream);

/* The first stage owns the embedding ("Unstable Legion", "Splitting the
 * workload").  hid_out_dev [H] (boundary format) <- dequantised embedding row
 * *tok_dev (int32 on the device; an id outside 0..vocab-1 reads row 0).
 * SLICE_EINVAL if the slice has no embedding. */
int slice_embed(slice_t *s, const int32_t *tok_dev, void *hid_out_dev, void *stream);

/* The last stage owns the head and the sampling ("Unstable Legion",
 * "Splitting the workload"); sampling is greedy as in the SwarmLLM README's
 * benchmark table.  Final RMSNorm, logits = W_head x (W_head = EMBED if tied),
 * greedy token = argmax (lowest index wins an exact tie) into *tok_dev (int32,
 * device).  hid_in_dev is in the boundary format; logits_dev ([vocab] fp32)
 * may be NULL.  SLICE_EINVAL if the slice has no head. */
int slice_head_argmax(slice_t *s, const void *hid_in_dev, int32_t *tok_dev,
                      float *logits_dev, void *stream);

/* The draft head's input (SwarmLLM README, pipeline diagram: the last stage's
 * draft head guesses the token after the one it just sampled; the form is the
 * published multi-token-prediction module of the model family the engine
 * follows).  x_out_dev [H] <- W_fc [RMSNorm(E[*tok_dev]) * w_e ;
 * RMSNorm(hid_in_dev) * w_h], embedding side first, each RMSNorm over its
 * own H entries with the slice's eps.  tok_dev: int32 on the device (an id
 * outside 0..vocab-1 reads row 0, as slice_embed); hid_in_dev: the hidden
 * state the token was sampled from (before the final norm); both vectors in
 * the boundary format.  x_out_dev then goes to slice_decode of the same
 * slice, whose output goes to slice_head_argmax for the draft token and, with
 * the draft, back in here for the next draft.  Stream-ordered; touches no
 * position or state.  SLICE_EINVAL if the slice is not a draft head or an
 * argument is NULL.  */
int slice_mtp_input(slice_t *s, const int32_t *tok_dev, const void *hid_in_dev, void *x_out_dev, void *stream);

/* Decode steps run the products and DeltaNet updates of consecutive layers as
 * one kernel whose workgroups wait, with a bounded wait, for the phase before
 * theirs (the pages' engine submits one command buffer per token: SwarmLLM
 * README, engine paragraph).  Synchronises `stream`, then returns SLICE_EHIP if such
 * a wait gave up since the last slice_reset (the step's outputs are then
 * invalid), else SLICE_OK. */
int slice_sync_check(slice_t *s, void *stream);

/* Host-side position p (-1 for NULL). */
int  slice_position(const slice_t *s);
/* Releases host objects and graphs only; the caller frees its buffers. */
void slice_free(slice_t *s);
/* Thread-local message of the last failed call on this thread. */
const char *slice_last_error(void);

/* Launch-shape overrides for tests and tuning sweeps (the pages' engine
 * tunes kernels per device: SwarmLLM README, repo layout, autotune).  Names:
 * "KS_<kind>" / "W_<kind>" (split-K workgroups / waves per workgroup; kinds
 * G1, G2, F1, F2, HEAD, GEMV, and G1P, G2P, F1P, F2P for prompt passes),
 * "MFMA_MIN_T" (fewest tokens sent to the matrix-core products), "EAGER"
 * (1: slices launch op by op instead of replaying graphs), "CHAIN" (0: decode
 * launches every product as its own kernel; the results are the same bits),
 * "CHAIN_MAX" (1..20: phases per chained kernel), "CHAIN_DN" / "CHAIN_ATT" /
 * "CHAIN_G1" (0: the DeltaNet update / the attention merge / the first
 * layer's input projections as kernels of their own instead of phases of the
 * chained kernel).  value < 0 removes
 * the override.  Process-wide; slices take them at slice_load, slq_gemv at
 * each call.  Nothing else (no environment variable) changes a launch shape,
 * and so the summation order.  SLICE_EINVAL for an unknown name. */
int slq_debug_override(const char *name, int value);

/* ---- state access for tests and synthetic prior context ----
 * (every optimisation of the pages' engine is gated on golden tests: SwarmLLM
 * README, feature list; these calls give the tests the state to compare)
 * DeltaNet state of `layer` in canonical layout fp32 [dn_heads][dv][dk]
 * (S[h][i][j]: i indexes values, j keys), current slot.                   */
int slice_dbg_set_state(slice_t *s, int layer, const float *src_dev, void *stream);
int slice_dbg_get_state(slice_t *s, int layer, float *dst_dev, void *stream);
/* KV rows [0, rows) of attention `layer`, canonical fp16 [kv_heads][rows][head_dim]. */
int slice_dbg_set_kv(slice_t *s, int layer, const uint16_t *k_dev, const uint16_t *v_dev,
                     int rows, void *stream);
int slice_dbg_get_kv(slice_t *s, int layer, uint16_t *k_dev, uint16_t *v_dev,
                     int rows, void *stream);

/* Conv state of DeltaNet `layer` (dn_variant = 1): the last dn_conv - 1 inputs
 * of every conv channel, canonical fp32 [conv_dim][dn_conv - 1], oldest
 * first, current slot (rolled back with the recurrent state).               */
int slice_dbg_set_conv(slice_t *s, int layer, const float *src_dev, void *stream);
int slice_dbg_get_conv(slice_t *s, int layer, float *dst_dev, void *stream);

/* fp32 residual stream h [k][hidden] at the end of the last decode (k = 1) or
 * verify (k tokens) step, before the boundary conversion.  For checking
 * results when the boundary is fp16 and |h| passes the fp16 range. */
int slice_dbg_get_hidden(slice_t *s, float *dst_dev, int k, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* LAYER_SLICE_H */
