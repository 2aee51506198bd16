// Host side of libslq: the C ABI declared in include/slice.h.
//
// A slice is the layer range [begin, end) of a decoder: one pipeline stage
// owns a contiguous run of layers and its own cache, and maps one hidden state
// to the next ("Unstable Legion", sections "Splitting the workload" and "The
// runtime").  One decode step is one HIP graph launch, where the pages' WebGPU
// engine submits one command buffer per token (SwarmLLM README, architecture
// paragraph).  The verify
// pass for k drafts uses the same kernels with k right-hand sides and writes
// each token's DeltaNet state to its own slot, so commit(j) is a slot switch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <map>
#include <string>
#include <vector>

#include "slice.h"
#include "slq.h"

using namespace slq;

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define HIPCHK(x)                                                                              \
  do {                                                                                         \
    hipError_t e_ = (x);                                                                       \
    if (e_ != hipSuccess) return fail(SLICE_EHIP, std::string(#x) + ": " + hipGetErrorString(e_)); \
  } while (0)

inline size_t al256(size_t x) { return (x + 255) & ~size_t(255); }
inline hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return v && *v ? atoi(v) : dflt;
}

// Launch shape of one GEMV: `ks` workgroups share the K tiles of each 64-row
// group (their partial sums meet through atomics), `w` waves per workgroup.
// Defaults come from kernel-trace sweeps on MI355X at hidden 5120 (all Q4_0):
//   input projections (16448/14336 x 5120): ks 4, w 4
//   gate/up + SwiGLU (34816 x 5120):        ks 2, w 4
//   down projection (5120 x 17408):         ks 8, w 4
//   mixer output (5120 x 4096 / 6144):      ks 4, w 4
// (one token: within 1 % of the best shape for every kind; at most 4 waves
// per workgroup also lets a verify pass of 4 tokens use the MFMA products)
// Other shapes: enough splits for ~1000 workgroups, about two tiles per wave,
// at most 4 waves per workgroup.
// SLQ_KS_<kind> / SLQ_W_<kind> override (kinds G1, G2, F1, F2, HEAD, GEMV).
struct Plan {
  int ks, w;
};

int clampi(int v, int lo, int hi) { return v < lo ? lo : v > hi ? hi : v; }

// Fewest tokens per call that go to the int8-MFMA products: 0 leaves the
// choice to gemm_min_tokens (by format and waves per workgroup);
// SLQ_MFMA_MIN_T sets a fixed count instead.
int mfma_min_tokens() { return clampi(env_int("SLQ_MFMA_MIN_T", 0), 0, MAX_T + 1); }

Plan plan_gemv(const char* kind, int64_t rows, int64_t cols) {
  const int nrg = (int)((rows + RG - 1) / RG);
  const int ntiles = (int)((cols / QK + TB - 1) / TB);
  const std::string k(kind);
  Plan p;
  if (k == "G2" && nrg <= 128) {
    // few row groups: four splits of four waves (fewer where K is short)
    p.ks = clampi(4, 1, ntiles);
    p.w = clampi(ntiles / p.ks, 1, 4);
  } else {
    p.ks = clampi((1024 + nrg - 1) / nrg, 1, ntiles < 16 ? ntiles : 16);
    if (k == "F1") p.ks = clampi(p.ks, 1, 2);
    if (k == "F2" || k == "G1") p.ks = clampi(p.ks, 1, k == "F2" ? 8 : 4);
    // at most 4 waves: one token is as fast as with 8 (LM head 248320 x 5120:
    // 114.8 against 115.1 us) and the batched products fit and stream longer
    // per wave (16 tokens: 474 against 874 us)
    p.w = clampi(k == "GEMV" || k == "HEAD" ? (ntiles / p.ks + 1) / 2 : 4, 1, 4);
  }
  p.ks = clampi(env_int(("SLQ_KS_" + k).c_str(), p.ks), 1, 16);
  p.w = clampi(env_int(("SLQ_W_" + k).c_str(), p.w), 1, 8);
  return p;
}

// Launch shape of the products of a prompt pass (slice_prefill), which need
// not sum in decode's order: four waves per workgroup and splits for about
// 2048 waves in all, at least one tile per wave.  At 16 tokens on MI355X this
// is the fastest shape, or within 6 % of it, for every product of the
// hidden-5120 hybrid in Q4_0 and Q8_0 (standalone sweep; e.g. gate/up 53.5
// against 57.1 us with the decode shape, attention input 31.1 against 39.2).
// SLQ_KS_<kind>P / SLQ_W_<kind>P override.
Plan plan_pass(const char* kind, int64_t rows, int64_t cols) {
  const int nrg = (int)((rows + RG - 1) / RG);
  const int ntiles = (int)((cols / QK + TB - 1) / TB);
  const std::string k(kind);
  Plan p;
  p.w = clampi(ntiles, 1, 4);
  p.ks = clampi((4096 + p.w * nrg) / (2 * p.w * nrg), 1, std::max(1, ntiles / p.w));   // round(2048 / (w nrg))
  p.ks = clampi(env_int(("SLQ_KS_" + k + "P").c_str(), p.ks), 1, 16);
  p.w = clampi(env_int(("SLQ_W_" + k + "P").c_str(), p.w), 1, 8);
  return p;
}

struct Mat {
  size_t off = 0;      // into the weights buffer
  int64_t rows = 0, cols = 0;
  bool present = false;
};

struct LayerLayout {
  bool attn = false;
  Mat g1, g2, f1, f2;
  Plan pg1{1, 1}, pg2{1, 1}, pf1{1, 1}, pf2{1, 1};   // GEMV splits, fixed at load
  Plan qg1{1, 1}, qg2{1, 1}, qf1{1, 1}, qf2{1, 1};   // the same for prompt passes
  size_t attn_norm = 0, ffn_norm = 0, q_norm = 0, k_norm = 0;
  // row offsets inside g1
  int off_q = 0, off_k = 0, off_v = 0, off_a = 0, off_b = 0, off_z = 0, off_g = -1;
  int dn_index = -1, attn_index = -1;
};

struct Layout {
  std::vector<LayerLayout> layers;   // index l - begin
  Mat embed, head;
  Plan phead{1, 1};
  size_t out_norm = 0;
  size_t wbytes = 0;
  // workspace
  size_t ctrl = 0, h = 0, xa_d = 0, xa_s = 0, xu_d = 0, xu_s = 0, xm_d = 0, xm_s = 0, ssq = 0, y1 = 0,
         xa_md = 0, xu_md = 0, xm_md = 0,
         part = 0, cnt = 0, apart = 0, rope = 0, logits = 0, amax_v = 0, amax_i = 0, kv = 0, dn = 0;
  size_t kv_layer_bytes = 0, dn_layer_bytes = 0;
  size_t wsbytes = 0;
  int64_t g1_rows_max = 0;
  int nu = 0;              // width of the mixer output (G2 input)
  int nchunk = 0, n_dn = 0, n_attn = 0, nslots = 0, mt = 1, amax_parts = 256;
};

std::string validate(const slice_config& c) {
  if (c.qtype != SLICE_Q4_0 && c.qtype != SLICE_Q8_0) return "qtype must be 2 (Q4_0) or 8 (Q8_0)";
  if (c.hidden <= 0 || c.hidden % 64) return "hidden must be a positive multiple of 64";
  if (c.layer_begin < 0 || c.layer_end < c.layer_begin || c.layer_end > c.n_layers) return "bad layer range";
  if (c.attn_period < 0) return "attn_period must be >= 0";
  if (c.max_verify < 1 || c.max_verify > MAX_T) return "max_verify must be in 1..16";
  if (c.ffn < 0 || c.ffn % 32) return "ffn must be a multiple of 32";
  if (!(c.eps >= 0)) return "eps must be >= 0";
  bool any_attn = false, any_dn = false;
  for (int l = c.layer_begin; l < c.layer_end; ++l) {
    bool a = c.attn_period == 0 || (l % c.attn_period) == c.attn_period - 1;
    any_attn |= a;
    any_dn |= !a;
  }
  if (any_attn) {
    if (c.q_heads <= 0 || c.kv_heads <= 0 || c.q_heads % c.kv_heads) return "q_heads must be a multiple of kv_heads";
    if (c.q_heads / c.kv_heads > 8) return "at most 8 query heads per KV head";
    if (c.head_dim % 64 || c.head_dim > 256 || c.head_dim <= 0) return "head_dim must be 64, 128, 192 or 256";
    if (c.rope_dims < 0 || c.rope_dims % 2 || c.rope_dims > c.head_dim) return "bad rope_dims";
    if (c.max_seq <= 0 || c.max_seq % 64) return "max_seq must be a positive multiple of 64";
  }
  if (any_dn) {
    if (c.dn_heads <= 0 || c.dn_dk % 32 || c.dn_dk > 128 || c.dn_dk <= 0 || c.dn_dv % 32 || c.dn_dv <= 0)
      return "DeltaNet needs dk in {32,64,96,128} and dv a multiple of 32";
  }
  if ((c.has_embed || c.has_head) && c.vocab <= 0) return "vocab must be > 0 with an embedding or head";
  return "";
}

Layout make_layout(const slice_config& c) {
  Layout L;
  const int qt = c.qtype;
  const int H = c.hidden;
  size_t w = 0;
  auto mat = [&](int64_t rows, int64_t cols) {
    Mat m;
    m.off = w;
    m.rows = rows;
    m.cols = cols;
    m.present = true;
    w = al256(w + packed_bytes(qt, rows, cols));
    return m;
  };
  auto vec = [&](int64_t n) {
    size_t o = w;
    w = al256(w + (size_t)n * 4);
    return o;
  };
  L.mt = c.max_verify;
  L.nslots = c.max_verify + 1;
  const int nkd = c.dn_heads * c.dn_dk, nvd = c.dn_heads * c.dn_dv;
  const int nq = c.q_heads * c.head_dim, nkv = c.kv_heads * c.head_dim;
  for (int l = c.layer_begin; l < c.layer_end; ++l) {
    LayerLayout ll;
    ll.attn = c.attn_period == 0 || (l % c.attn_period) == c.attn_period - 1;
    if (ll.attn) {
      ll.off_q = 0;
      int r = nq;
      if (c.attn_gate) { ll.off_g = r; r += nq; }
      ll.off_k = r; r += nkv;
      ll.off_v = r; r += nkv;
      ll.g1 = mat(r, H);
      ll.g2 = mat(H, nq);
      ll.attn_index = L.n_attn++;
      if (nq > L.nu) L.nu = nq;
    } else {
      ll.off_q = 0;
      ll.off_k = nkd;
      ll.off_v = 2 * nkd;
      ll.off_a = 2 * nkd + nvd;
      ll.off_b = ll.off_a + c.dn_heads;
      ll.off_z = ll.off_b + c.dn_heads;
      ll.g1 = mat(ll.off_z + nvd, H);
      ll.g2 = mat(H, nvd);
      ll.dn_index = L.n_dn++;
      if (nvd > L.nu) L.nu = nvd;
    }
    if (ll.g1.rows > L.g1_rows_max) L.g1_rows_max = ll.g1.rows;
    if (c.ffn) {
      ll.f1 = mat(2 * (int64_t)c.ffn, H);
      ll.f2 = mat(H, c.ffn);
    }
    ll.attn_norm = vec(H);
    ll.ffn_norm = vec(H);
    if (ll.attn) {
      ll.q_norm = vec(c.head_dim);
      ll.k_norm = vec(c.head_dim);
    }
    L.layers.push_back(ll);
  }
  if (c.has_embed || (c.has_head && c.tied_head)) L.embed = mat(c.vocab, H);
  if (c.has_head && !c.tied_head) L.head = mat(c.vocab, H);
  L.out_norm = vec(H);
  L.wbytes = w;

  // workspace
  const int mt = L.mt;
  const int nblkH = H / QK;
  const int nblkU = (L.nu + QK - 1) / QK;
  const int nblkM = c.ffn / QK;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t r = o;
    o = al256(o + bytes);
    return r;
  };
  L.ctrl = take(sizeof(Ctrl));
  L.h = take((size_t)mt * H * 4);
  // activation digits: the lane-row layout for every step, and the 16-slot
  // MFMA layout for steps of several tokens
  auto digits = [&](int nblk) { return (size_t)mt * XW * 4 * (nblk ? nblk : 1); };
  auto scales = [&](int nblk) { return (size_t)mt * (nblk ? nblk : 1) * 4; };
  auto mdigits = [&](int nblk) { return mt > 1 ? (size_t)mx_block_bytes(c.qtype) * (nblk ? nblk : 1) : 0; };
  L.xa_d = take(digits(nblkH));
  L.xa_s = take(scales(nblkH));
  L.xu_d = take(digits(nblkU));
  L.xu_s = take(scales(nblkU));
  L.xm_d = take(digits(nblkM));
  L.xm_s = take(scales(nblkM));
  L.xa_md = take(mdigits(nblkH));
  L.xu_md = take(mdigits(nblkU));
  L.xm_md = take(mdigits(nblkM));
  L.ssq = take((size_t)mt * (H / RG) * 4);
  L.y1 = take((size_t)mt * (L.g1_rows_max ? L.g1_rows_max : 1) * 4);
  // split-K scratch: any GEMV of the slice with up to 16 splits
  // (one partial per split-K workgroup and token)
  int64_t rg_max = 0;
  size_t part_floats = 0;
  auto upd = [&](const Mat& m, Plan& p, Plan* q, const char* kind) {
    if (!m.present) return;
    p = plan_gemv(kind, m.rows, m.cols);
    const int64_t nrg = (m.rows + RG - 1) / RG;
    rg_max = std::max<int64_t>(rg_max, nrg);
    part_floats = std::max<size_t>(part_floats, (size_t)nrg * p.ks * mt * RG);
    if (q) {
      *q = plan_pass(kind, m.rows, m.cols);
      part_floats = std::max<size_t>(part_floats, (size_t)nrg * q->ks * mt * RG);
    }
  };
  for (LayerLayout& ll : L.layers) {
    upd(ll.g1, ll.pg1, &ll.qg1, "G1");
    upd(ll.g2, ll.pg2, &ll.qg2, "G2");
    upd(ll.f1, ll.pf1, &ll.qf1, "F1");
    upd(ll.f2, ll.pf2, &ll.qf2, "F2");
  }
  if (c.has_head) upd(c.tied_head ? L.embed : L.head, L.phead, nullptr, "HEAD");
  L.part = take(part_floats * 4);
  L.cnt = take((size_t)std::max<int64_t>(rg_max, 1) * 4);
  if (L.n_attn) {
    L.nchunk = (c.max_seq + ATT_CHUNK - 1) / ATT_CHUNK;
    L.apart = take((size_t)mt * c.q_heads * L.nchunk * (c.head_dim + 2) * 4);
    L.rope = take((size_t)c.max_seq * (c.rope_dims / 2 > 0 ? c.rope_dims / 2 : 1) * 8);
  }
  if (c.has_head) {
    L.logits = take((size_t)c.vocab * 4);
    L.amax_v = take((size_t)L.amax_parts * 4);
    L.amax_i = take((size_t)L.amax_parts * 4);
  }
  L.kv_layer_bytes = al256((size_t)2 * c.kv_heads * c.max_seq * c.head_dim * 2);
  L.kv = take((size_t)L.n_attn * L.kv_layer_bytes);
  L.dn_layer_bytes = al256((size_t)L.nslots * c.dn_heads * c.dn_dk * c.dn_dv * 4);
  L.dn = take((size_t)L.n_dn * L.dn_layer_bytes);
  L.wsbytes = o;
  return L;
}

}  // namespace

// Optional per-op timing: an event is recorded at every op boundary.
struct Prof {
  std::vector<hipEvent_t> ev;
  std::vector<int> kind;   // kind of the op that ends at ev[i+1]
  int mark(int k, hipStream_t st) {
    hipEvent_t e;
    HIPCHK(hipEventCreate(&e));
    ev.push_back(e);
    if (ev.size() > 1) kind.push_back(k);
    HIPCHK(hipEventRecord(e, st));
    return SLICE_OK;
  }
  void destroy() {
    for (hipEvent_t e : ev) hipEventDestroy(e);
    ev.clear();
    kind.clear();
  }
};

struct slice {
  slice_config cfg;
  Layout L;
  uint8_t* w = nullptr;
  uint8_t* ws = nullptr;
  int pos = 0, cur = 0, pending = 0;   // pending: k of an uncommitted verify, else 0
  const void* last_in = nullptr;
  void* last_out = nullptr;
  bool eager = false;
  hipStream_t cap = nullptr;
  std::map<int, hipGraphExec_t> graphs;   // key: decode 0, verify k k, prefill k 100 + k
  Ctrl* ctrl() const { return reinterpret_cast<Ctrl*>(ws + L.ctrl); }
  template <class X> X* wsp(size_t off) const { return reinterpret_cast<X*>(ws + off); }
  Packed packed(const Mat& m) const { return Packed{w + m.off, m.rows, m.cols, cfg.qtype}; }
  int mx_min_t = 0;   // GEMVs with at least this many tokens use the MFMA products (0: by format and plan)
  // digits of a step of T tokens; the MFMA layout is written when it may be used
  Act act(size_t d, size_t s_, size_t md, int nblk, int T) const {
    const bool mx = T >= (mx_min_t ? mx_min_t : 2) && L.mt > 1;
    return Act{wsp<int32_t>(d), wsp<float>(s_), nblk, mx ? wsp<int32_t>(md) : nullptr, mx_min_t};
  }
  Act act_a(int T) const { return act(L.xa_d, L.xa_s, L.xa_md, cfg.hidden / QK, T); }
  Act act_u(int T) const { return act(L.xu_d, L.xu_s, L.xu_md, (L.nu + QK - 1) / QK, T); }
  Act act_m(int T) const { return act(L.xm_d, L.xm_s, L.xm_md, cfg.ffn / QK, T); }
  NormIn norm_h() const {
    return NormIn{wsp<float>(L.ssq), cfg.hidden / RG, 1.0f / (float)cfg.hidden, cfg.eps};
  }
};

// One step with T tokens: entry, every layer, exit.  Reads the input/output
// pointers from the control block so a captured graph serves any buffers.
// only >= 0: enqueue just the GEMV op of that kind for every layer (no entry,
// mixers or exit), reading the activations the last step left in the workspace.
static int enqueue_step(slice* s, int T, int mode, hipStream_t st, Prof* prof = nullptr, int only = -1) {
#define SLQ_MARK(k) do { if (prof) { int r_ = prof->mark(k, st); if (r_) return r_; } } while (0)
  const bool decode = mode == DN_DECODE;
  const bool pass = mode == DN_CHUNK;   // prompt pass: its own product shapes
  const slice_config& c = s->cfg;
  const Layout& L = s->L;
  const int H = c.hidden;
  const int qt = c.qtype;
  float* h = s->wsp<float>(L.h);
  float* ssq = s->wsp<float>(L.ssq);
  float* y1 = s->wsp<float>(L.y1);
  Ctrl* ctrl = s->ctrl();
  const int nlay = (int)L.layers.size();
  // norm weights of the RMSNorm in front of layer i (past the last layer the
  // digits are not consumed; any valid vector will do)
  auto attn_norm_of = [&](int i) -> const float* {
    if (i < nlay) return reinterpret_cast<const float*>(s->w + L.layers[i].attn_norm);
    return reinterpret_cast<const float*>(s->w + L.out_norm);
  };
  // entry: boundary vector -> h, digits of attn_norm(first layer) * h
  SLQ_MARK(-1);
  if (only < 0) HIPCHK(launch_resid_finish(c.io_fp32 ? 2 : 1, nullptr, ctrl, H, T, H, h, attn_norm_of(0), qt, s->act_a(T), ssq, st));
  SLQ_MARK(SLICE_OP_ENTRY);
  float* part = s->wsp<float>(L.part);
  unsigned* cnt = s->wsp<unsigned>(L.cnt);
  for (int i = 0; i < nlay; ++i) {
    const LayerLayout& ll = L.layers[i];
    const int k_in = ll.attn ? SLICE_OP_ATT_IN : SLICE_OP_DN_IN;
    const int k_mix = ll.attn ? SLICE_OP_ATTENTION : SLICE_OP_DELTANET;
    const int k_out = ll.attn ? SLICE_OP_ATT_OUT : SLICE_OP_DN_OUT;
    // mixer input projections: G1 = [q|k|v|a|b|z] or [q|g|k|v] of RMSNorm(h)
    if (only < 0 || only == k_in) {
      const Packed W = s->packed(ll.g1);
      GemvOut o{};
      o.kind = EPI_STORE;
      o.y = y1;
      o.y_tstride = W.rows;
      o.part = part;
      o.cnt = cnt;
      const Plan pl = pass ? ll.qg1 : ll.pg1;
      HIPCHK(launch_gemv(W, T, s->act_a(T), s->norm_h(), o, pl.ks, pl.w, st));
      SLQ_MARK(ll.attn ? SLICE_OP_ATT_IN : SLICE_OP_DN_IN);
    }
    if (only >= 0 && only != k_mix) {
    } else if (ll.attn) {
      AttnParams p{};
      p.y = y1;
      p.y_stride = ll.g1.rows;
      p.off_q = ll.off_q; p.off_g = ll.off_g; p.off_k = ll.off_k; p.off_v = ll.off_v;
      p.q_heads = c.q_heads; p.kv_heads = c.kv_heads; p.hd = c.head_dim; p.rope_dims = c.rope_dims;
      p.rope_theta = c.rope_theta;
      p.rope_cs = s->wsp<float>(L.rope);
      p.qk_norm = c.qk_norm;
      p.q_norm = reinterpret_cast<const float*>(s->w + ll.q_norm);
      p.k_norm = reinterpret_cast<const float*>(s->w + ll.k_norm);
      p.eps = c.eps;
      uint8_t* kvb = s->ws + L.kv + (size_t)ll.attn_index * L.kv_layer_bytes;
      p.kc = reinterpret_cast<__half*>(kvb);
      p.vc = reinterpret_cast<__half*>(kvb + (size_t)c.kv_heads * c.max_seq * c.head_dim * 2);
      p.max_seq = c.max_seq;
      p.ctrl = ctrl;
      p.part = s->wsp<float>(L.apart);
      p.nchunk = L.nchunk;
      p.u_out = nullptr;
      p.next = s->act_u(T);
      p.next_qt = qt;
      HIPCHK(launch_attention(p, T, st));
      SLQ_MARK(SLICE_OP_ATTENTION);
    } else {
      DnParams p{};
      p.y = y1;
      p.y_stride = ll.g1.rows;
      p.off_q = ll.off_q; p.off_k = ll.off_k; p.off_v = ll.off_v;
      p.off_a = ll.off_a; p.off_b = ll.off_b; p.off_z = ll.off_z;
      p.heads = c.dn_heads; p.dk = c.dn_dk; p.dv = c.dn_dv;
      p.a_scale = c.dn_a_scale; p.a_bias = c.dn_a_bias; p.b_scale = c.dn_b_scale; p.z_scale = c.dn_z_scale;
      p.state = reinterpret_cast<float*>(s->ws + L.dn + (size_t)ll.dn_index * L.dn_layer_bytes);
      p.nslots = L.nslots;
      p.mode = mode;
      p.ctrl = ctrl;
      p.u_out = nullptr;
      p.next = s->act_u(T);
      p.next_qt = qt;
      HIPCHK(launch_deltanet(p, T, st));
      SLQ_MARK(SLICE_OP_DELTANET);
    }
    // residual update after the mixer: h += W_o u, then digits for the next RMSNorm
    const float* nw_after_mixer = c.ffn ? reinterpret_cast<const float*>(s->w + ll.ffn_norm) : attn_norm_of(i + 1);
    auto residual = [&](const Mat& m, Act in, const float* next_norm, const Plan& pl) -> int {
      const Packed W = s->packed(m);
      GemvOut o{};
      o.kind = EPI_RESID;
      o.y = h;
      o.y_tstride = H;
      o.next = s->act_a(T);
      o.next_qt = qt;
      o.ssq_out = ssq;
      o.norm_w = next_norm;
      o.part = part;
      o.cnt = cnt;
      HIPCHK(launch_gemv(W, T, in, NormIn{nullptr, 0, 0.f, 0.f}, o, pl.ks, pl.w, st));
      return SLICE_OK;
    };
    int rc = (only < 0 || only == k_out) ? residual(ll.g2, s->act_u(T), nw_after_mixer, pass ? ll.qg2 : ll.pg2) : SLICE_OK;
    if (rc) return rc;
    SLQ_MARK(k_out);
    if (c.ffn && (only < 0 || only == SLICE_OP_FFN_IN)) {
      const Packed W = s->packed(ll.f1);
      GemvOut o{};
      o.kind = EPI_SWIGLU;
      o.y = nullptr;
      o.y_tstride = c.ffn;
      o.next = s->act_m(T);
      o.next_qt = qt;
      o.part = part;
      o.cnt = cnt;
      const Plan pl = pass ? ll.qf1 : ll.pf1;
      HIPCHK(launch_gemv(W, T, s->act_a(T), s->norm_h(), o, pl.ks, pl.w, st));
      SLQ_MARK(SLICE_OP_FFN_IN);
    }
    if (c.ffn && (only < 0 || only == SLICE_OP_FFN_OUT)) {
      rc = residual(ll.f2, s->act_m(T), attn_norm_of(i + 1), pass ? ll.qf2 : ll.pf2);
      if (rc) return rc;
      SLQ_MARK(SLICE_OP_FFN_OUT);
    }
  }
  // decode and prefill move the position on the device; a verify waits for commit
  const int advance = decode ? 1 : mode == DN_CHUNK ? T : 0;
  if (only < 0) HIPCHK(launch_store_out(h, T, H, nullptr, c.io_fp32, ctrl, advance, st));
  SLQ_MARK(SLICE_OP_EXIT);
  return SLICE_OK;
#undef SLQ_MARK
}

static int run_step(slice* s, int T, int mode, const void* in, void* out, hipStream_t st) {
  if (in != s->last_in || out != s->last_out) {
    HIPCHK(launch_ctrl_io(s->ctrl(), in, out, st));
    s->last_in = in;
    s->last_out = out;
  }
  if (s->eager) return enqueue_step(s, T, mode, st);
  const int key = mode == DN_DECODE ? 0 : mode == DN_CHUNK ? 100 + T : T;
  auto it = s->graphs.find(key);
  if (it == s->graphs.end()) {
    HIPCHK(hipStreamBeginCapture(s->cap, hipStreamCaptureModeThreadLocal));
    int rc = enqueue_step(s, T, mode, s->cap);
    hipGraph_t g = nullptr;
    hipError_t e = hipStreamEndCapture(s->cap, &g);
    if (rc) {
      if (g) hipGraphDestroy(g);
      return rc;
    }
    if (e != hipSuccess) return fail(SLICE_EHIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(e));
    hipGraphExec_t ex = nullptr;
    e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
    hipGraphDestroy(g);
    if (e != hipSuccess) return fail(SLICE_EHIP, std::string("hipGraphInstantiate: ") + hipGetErrorString(e));
    it = s->graphs.emplace(key, ex).first;
  }
  HIPCHK(hipGraphLaunch(it->second, st));
  return SLICE_OK;
}

// ====================================================================== ABI

extern "C" {

const char* slice_last_error(void) { return g_err.c_str(); }

size_t slq_packed_bytes(int qtype, int64_t rows, int64_t cols) {
  if ((qtype != SLICE_Q4_0 && qtype != SLICE_Q8_0) || rows < 0 || cols <= 0 || cols % QK) return 0;
  return packed_bytes(qtype, rows, cols);
}

int slq_repack(int qtype, const void* raw_dev, int64_t rows, int64_t cols, void* packed_dev, void* stream) {
  const size_t n = slq_packed_bytes(qtype, rows, cols);
  if (!n) return fail(SLICE_ESHAPE, "slq_repack: bad qtype or shape");
  if (!raw_dev || !packed_dev) return fail(SLICE_EINVAL, "slq_repack: null pointer");
  HIPCHK(hipMemsetAsync(packed_dev, 0, n, S(stream)));
  HIPCHK(launch_repack(qtype, static_cast<const uint8_t*>(raw_dev), rows, cols, static_cast<uint8_t*>(packed_dev),
                       rows, 0, 0, S(stream)));
  return SLICE_OK;
}

int slq_dequant(int qtype, const void* packed_dev, int64_t rows, int64_t cols, float* out_dev, void* stream) {
  if (!slq_packed_bytes(qtype, rows, cols)) return fail(SLICE_ESHAPE, "slq_dequant: bad qtype or shape");
  if (!packed_dev || !out_dev) return fail(SLICE_EINVAL, "slq_dequant: null pointer");
  HIPCHK(launch_dequant(Packed{static_cast<const uint8_t*>(packed_dev), rows, cols, qtype}, out_dev, S(stream)));
  return SLICE_OK;
}

// Standalone GEMV workspace: activation digits (room for both layouts), their
// scales, split-K partials, ticket counters.
// Standalone GEMV workspace, in order: lane-row digits [batch][nblk][24],
// their scales, MFMA-layout block records, split-K partials
// [nrg][ks][batch][64], ticket counters [nrg].
struct GemvWs {
  size_t dig, sc, mdig, part, cnt, total;
};
static GemvWs gemv_ws(int qtype, int64_t rows, int64_t cols, int batch) {
  const int nblk = (int)(cols / QK);
  const int64_t nrg = (rows + RG - 1) / RG;
  const Plan p = plan_gemv("GEMV", rows, cols);
  GemvWs w{};
  size_t o = 0;
  w.dig = o; o += al256((size_t)batch * nblk * XW * 4);
  w.sc = o; o += al256((size_t)batch * nblk * 4);
  w.mdig = o; o += al256((size_t)nblk * mx_block_bytes(qtype));
  w.part = o; o += al256((size_t)nrg * p.ks * batch * RG * 4);
  w.cnt = o; o += al256((size_t)nrg * 4);
  w.total = o;
  return w;
}

size_t slq_gemv_workspace_bytes(int qtype, int64_t rows, int64_t cols, int batch) {
  if (!slq_packed_bytes(qtype, rows, cols) || batch < 1 || batch > MAX_T) return 0;
  return gemv_ws(qtype, rows, cols, batch).total;
}

int slq_gemv(int qtype, const void* packed_dev, int64_t rows, int64_t cols, int batch, const float* x_dev,
             float* y_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  const size_t need = slq_gemv_workspace_bytes(qtype, rows, cols, batch);
  if (!need) return fail(SLICE_ESHAPE, "slq_gemv: bad qtype, shape or batch (1..16)");
  if (ws_bytes < need) return fail(SLICE_EINVAL, "slq_gemv: workspace too small");
  if (!packed_dev || !x_dev || !y_dev || !ws_dev) return fail(SLICE_EINVAL, "slq_gemv: null pointer");
  const int nblk = (int)(cols / QK);
  uint8_t* ws = static_cast<uint8_t*>(ws_dev);
  const GemvWs L = gemv_ws(qtype, rows, cols, batch);
  const int min_t = mfma_min_tokens();
  const bool mx = batch >= (min_t ? min_t : 2);
  Act a{reinterpret_cast<int32_t*>(ws + L.dig), reinterpret_cast<float*>(ws + L.sc), nblk,
        mx ? reinterpret_cast<int32_t*>(ws + L.mdig) : nullptr, min_t};
  float* part = reinterpret_cast<float*>(ws + L.part);
  unsigned* cnt = reinterpret_cast<unsigned*>(ws + L.cnt);
  HIPCHK(launch_quant_act(qtype, x_dev, batch, (int)cols, cols, a, S(stream)));
  const Plan pl = plan_gemv("GEMV", rows, cols);
  const Packed W{static_cast<const uint8_t*>(packed_dev), rows, cols, qtype};
  GemvOut o{};
  o.kind = EPI_STORE;
  o.y = y_dev;
  o.y_tstride = rows;
  o.part = part;
  o.cnt = cnt;
  HIPCHK(launch_gemv(W, batch, a, NormIn{nullptr, 0, 0.f, 0.f}, o, pl.ks, pl.w, S(stream)));
  return SLICE_OK;
}

size_t slice_weights_bytes(const slice_config* cfg) {
  if (!cfg) return 0;
  std::string e = validate(*cfg);
  if (!e.empty()) { fail(SLICE_EINVAL, e); return 0; }
  return make_layout(*cfg).wbytes;
}

size_t slice_workspace_bytes(const slice_config* cfg) {
  if (!cfg) return 0;
  std::string e = validate(*cfg);
  if (!e.empty()) { fail(SLICE_EINVAL, e); return 0; }
  return make_layout(*cfg).wsbytes;
}

int slice_load(const slice_config* cfg, void* weights_dev, void* workspace_dev, void* stream, slice_t** out) {
  if (!cfg || !out) return fail(SLICE_EINVAL, "slice_load: null argument");
  *out = nullptr;
  std::string e = validate(*cfg);
  if (!e.empty()) return fail(SLICE_EINVAL, e);
  if (!weights_dev || !workspace_dev) return fail(SLICE_EINVAL, "slice_load: null buffer");
  if ((reinterpret_cast<uintptr_t>(weights_dev) | reinterpret_cast<uintptr_t>(workspace_dev)) & 255)
    return fail(SLICE_EINVAL, "slice_load: buffers must be 256-byte aligned");
  slice* s = new slice();
  s->cfg = *cfg;
  s->L = make_layout(*cfg);
  s->w = static_cast<uint8_t*>(weights_dev);
  s->ws = static_cast<uint8_t*>(workspace_dev);
  s->eager = env_int("SLQ_EAGER", 0) != 0;
  s->mx_min_t = mfma_min_tokens();
  hipError_t he = hipMemsetAsync(s->w, 0, s->L.wbytes, S(stream));
  if (he == hipSuccess) he = hipMemsetAsync(s->ws, 0, s->L.wsbytes, S(stream));
  if (he == hipSuccess && s->L.n_attn && cfg->rope_dims > 0)
    he = launch_rope_table(s->wsp<float>(s->L.rope), cfg->max_seq, cfg->rope_dims, cfg->rope_theta, S(stream));
  if (he == hipSuccess) he = hipStreamCreate(&s->cap);
  if (he != hipSuccess) {
    delete s;
    return fail(SLICE_EHIP, std::string("slice_load: ") + hipGetErrorString(he));
  }
  *out = s;
  return SLICE_OK;
}

int slice_set_tensor(slice_t* s, int layer, int tid, const void* src, void* stream) {
  if (!s || !src) return fail(SLICE_EINVAL, "slice_set_tensor: null argument");
  const slice_config& c = s->cfg;
  const Layout& L = s->L;
  const int qt = c.qtype;
  const hipStream_t st = S(stream);
  auto repack = [&](const Mat& m, int64_t rows, int64_t cols, int map_kind, int64_t row_off) -> int {
    if (!m.present) return fail(SLICE_EINVAL, "slice_set_tensor: tensor not in this slice");
    HIPCHK(launch_repack(qt, static_cast<const uint8_t*>(src), rows, cols, s->w + m.off, m.rows, map_kind, row_off, st));
    return SLICE_OK;
  };
  auto copyv = [&](size_t off, int64_t n) -> int {
    HIPCHK(hipMemcpyAsync(s->w + off, src, (size_t)n * 4, hipMemcpyDeviceToDevice, st));
    return SLICE_OK;
  };
  if (tid == SLICE_T_EMBED) {
    if (!L.embed.present) return fail(SLICE_EINVAL, "slice has no embedding");
    return repack(L.embed, c.vocab, c.hidden, 0, 0);
  }
  if (tid == SLICE_T_HEAD) {
    if (!L.head.present) return fail(SLICE_EINVAL, "slice has no untied head");
    return repack(L.head, c.vocab, c.hidden, 0, 0);
  }
  if (tid == SLICE_T_OUT_NORM) return copyv(L.out_norm, c.hidden);
  if (layer < c.layer_begin || layer >= c.layer_end) return fail(SLICE_ERANGE, "slice_set_tensor: layer outside the slice");
  const LayerLayout& ll = L.layers[layer - c.layer_begin];
  const int H = c.hidden;
  const int nkd = c.dn_heads * c.dn_dk, nvd = c.dn_heads * c.dn_dv;
  const int nq = c.q_heads * c.head_dim, nkv = c.kv_heads * c.head_dim;
  switch (tid) {
    case SLICE_T_ATTN_NORM: return copyv(ll.attn_norm, H);
    case SLICE_T_FFN_NORM: return c.ffn ? copyv(ll.ffn_norm, H) : fail(SLICE_EINVAL, "no FFN in this slice");
    case SLICE_T_W_GATE: return c.ffn ? repack(ll.f1, c.ffn, H, 1, 0) : fail(SLICE_EINVAL, "no FFN");
    case SLICE_T_W_UP: return c.ffn ? repack(ll.f1, c.ffn, H, 1, 32) : fail(SLICE_EINVAL, "no FFN");
    case SLICE_T_W_DOWN: return c.ffn ? repack(ll.f2, H, c.ffn, 0, 0) : fail(SLICE_EINVAL, "no FFN");
    default: break;
  }
  if (ll.attn) {
    switch (tid) {
      case SLICE_T_WQ: return repack(ll.g1, nq, H, 0, ll.off_q);
      case SLICE_T_WG: return c.attn_gate ? repack(ll.g1, nq, H, 0, ll.off_g) : fail(SLICE_EINVAL, "no attention gate");
      case SLICE_T_WK: return repack(ll.g1, nkv, H, 0, ll.off_k);
      case SLICE_T_WV: return repack(ll.g1, nkv, H, 0, ll.off_v);
      case SLICE_T_WO: return repack(ll.g2, H, nq, 0, 0);
      case SLICE_T_Q_NORM: return copyv(ll.q_norm, c.head_dim);
      case SLICE_T_K_NORM: return copyv(ll.k_norm, c.head_dim);
      default: return fail(SLICE_EINVAL, "slice_set_tensor: not an attention-layer tensor");
    }
  }
  switch (tid) {
    case SLICE_T_DN_Q: return repack(ll.g1, nkd, H, 0, ll.off_q);
    case SLICE_T_DN_K: return repack(ll.g1, nkd, H, 0, ll.off_k);
    case SLICE_T_DN_V: return repack(ll.g1, nvd, H, 0, ll.off_v);
    case SLICE_T_DN_A: return repack(ll.g1, c.dn_heads, H, 0, ll.off_a);
    case SLICE_T_DN_B: return repack(ll.g1, c.dn_heads, H, 0, ll.off_b);
    case SLICE_T_DN_Z: return repack(ll.g1, nvd, H, 0, ll.off_z);
    case SLICE_T_DN_OUT: return repack(ll.g2, H, nvd, 0, 0);
    default: return fail(SLICE_EINVAL, "slice_set_tensor: not a DeltaNet-layer tensor");
  }
}

int slice_reset(slice_t* s, int kv_len, void* stream) {
  if (!s) return fail(SLICE_EINVAL, "null slice");
  if (kv_len < 0 || (s->L.n_attn && kv_len > s->cfg.max_seq)) return fail(SLICE_ERANGE, "kv_len out of range");
  HIPCHK(launch_ctrl_set(s->ctrl(), kv_len, s->cur, S(stream)));
  s->pos = kv_len;
  s->pending = 0;
  return SLICE_OK;
}

int slice_decode(slice_t* s, const void* in, void* out, void* stream) {
  if (!s || !in || !out) return fail(SLICE_EINVAL, "slice_decode: null argument");
  if (s->pending) return fail(SLICE_ESTATE, "slice_decode: a verify is waiting for slice_commit");
  if (s->L.n_attn && s->pos + 1 > s->cfg.max_seq) return fail(SLICE_ERANGE, "slice_decode: position reached max_seq");
  int rc = run_step(s, 1, DN_DECODE, in, out, S(stream));
  if (rc) return rc;
  s->pos += 1;
  return SLICE_OK;
}

int slice_decode_profiled(slice_t* s, const void* in, void* out, int* op_kind, float* op_ms, int max_ops,
                          void* stream) {
  if (!s || !in || !out || !op_kind || !op_ms) return fail(SLICE_EINVAL, "slice_decode_profiled: null argument");
  if (s->pending) return fail(SLICE_ESTATE, "slice_decode_profiled: a verify is waiting for slice_commit");
  if (s->L.n_attn && s->pos + 1 > s->cfg.max_seq) return fail(SLICE_ERANGE, "slice_decode_profiled: position reached max_seq");
  const hipStream_t st = S(stream);
  if (in != s->last_in || out != s->last_out) {
    HIPCHK(launch_ctrl_io(s->ctrl(), in, out, st));
    s->last_in = in;
    s->last_out = out;
  }
  Prof prof;
  int rc = enqueue_step(s, 1, DN_DECODE, st, &prof);
  int n = 0;
  if (!rc) {
    hipError_t e = hipEventSynchronize(prof.ev.back());
    if (e != hipSuccess) rc = fail(SLICE_EHIP, std::string("hipEventSynchronize: ") + hipGetErrorString(e));
    for (size_t i = 0; !rc && i < prof.kind.size() && n < max_ops; ++i, ++n) {
      op_kind[n] = prof.kind[i];
      e = hipEventElapsedTime(&op_ms[n], prof.ev[i], prof.ev[i + 1]);
      if (e != hipSuccess) rc = fail(SLICE_EHIP, std::string("hipEventElapsedTime: ") + hipGetErrorString(e));
    }
  }
  for (hipEvent_t e : prof.ev) hipEventDestroy(e);
  if (rc) return rc;
  s->pos += 1;
  return n;
}

int slice_run_gemv_op(slice_t* s, int op_kind, void* stream) {
  if (!s) return fail(SLICE_EINVAL, "null slice");
  if (op_kind != SLICE_OP_DN_IN && op_kind != SLICE_OP_DN_OUT && op_kind != SLICE_OP_ATT_IN &&
      op_kind != SLICE_OP_ATT_OUT && op_kind != SLICE_OP_FFN_IN && op_kind != SLICE_OP_FFN_OUT)
    return fail(SLICE_EINVAL, "slice_run_gemv_op: not a GEMV op kind");
  if (s->pending) return fail(SLICE_ESTATE, "slice_run_gemv_op: a verify is waiting for slice_commit");
  return enqueue_step(s, 1, DN_DECODE, S(stream), nullptr, op_kind);
}

int slice_verify(slice_t* s, int k, const void* in, void* out, void* stream) {
  if (!s || !in || !out) return fail(SLICE_EINVAL, "slice_verify: null argument");
  if (s->pending) return fail(SLICE_ESTATE, "slice_verify: a verify is waiting for slice_commit");
  if (k < 1 || k > s->cfg.max_verify) return fail(SLICE_ERANGE, "slice_verify: k outside 1..max_verify");
  if (s->L.n_attn && s->pos + k > s->cfg.max_seq) return fail(SLICE_ERANGE, "slice_verify: positions pass max_seq");
  int rc = run_step(s, k, DN_VERIFY, in, out, S(stream));
  if (rc) return rc;
  s->pending = k;
  return SLICE_OK;
}

int slice_prefill(slice_t* s, int k, const void* in, void* out, void* stream) {
  if (!s || !in || !out) return fail(SLICE_EINVAL, "slice_prefill: null argument");
  if (s->pending) return fail(SLICE_ESTATE, "slice_prefill: a verify is waiting for slice_commit");
  if (k < 1 || k > s->cfg.max_verify) return fail(SLICE_ERANGE, "slice_prefill: k outside 1..max_verify");
  if (s->L.n_attn && s->pos + k > s->cfg.max_seq) return fail(SLICE_ERANGE, "slice_prefill: positions pass max_seq");
  int rc = run_step(s, k, DN_CHUNK, in, out, S(stream));
  if (rc) return rc;
  s->pos += k;
  return SLICE_OK;
}

int slice_commit(slice_t* s, int accepted, void* stream) {
  if (!s) return fail(SLICE_EINVAL, "null slice");
  if (!s->pending) return fail(SLICE_ESTATE, "slice_commit: no verify pending");
  if (accepted < 0 || accepted > s->pending) return fail(SLICE_ERANGE, "slice_commit: accepted outside 0..k");
  const int cur = (s->cur + accepted) % s->L.nslots;
  HIPCHK(launch_ctrl_set(s->ctrl(), s->pos + accepted, cur, S(stream)));
  s->pos += accepted;
  s->cur = cur;
  s->pending = 0;
  return SLICE_OK;
}

int slice_embed(slice_t* s, const int32_t* tok, void* out, void* stream) {
  if (!s || !tok || !out) return fail(SLICE_EINVAL, "slice_embed: null argument");
  if (!s->L.embed.present || !s->cfg.has_embed) return fail(SLICE_EINVAL, "slice_embed: slice has no embedding");
  HIPCHK(launch_embed(s->packed(s->L.embed), tok, out, s->cfg.io_fp32, S(stream)));
  return SLICE_OK;
}

int slice_head_argmax(slice_t* s, const void* in, int32_t* tok, float* logits, void* stream) {
  if (!s || !in || !tok) return fail(SLICE_EINVAL, "slice_head_argmax: null argument");
  if (!s->cfg.has_head) return fail(SLICE_EINVAL, "slice_head_argmax: slice has no head");
  const slice_config& c = s->cfg;
  const Layout& L = s->L;
  const hipStream_t st = S(stream);
  float* lg = logits ? logits : s->wsp<float>(L.logits);
  HIPCHK(launch_resid_finish(c.io_fp32 ? 2 : 1, in, nullptr, c.hidden, 1, c.hidden, s->wsp<float>(L.h),
                             reinterpret_cast<const float*>(s->w + L.out_norm), c.qtype, s->act_a(1),
                             s->wsp<float>(L.ssq), st));
  const Packed W = s->packed(c.tied_head ? L.embed : L.head);
  GemvOut o{};
  o.kind = EPI_STORE;
  o.y = lg;
  o.y_tstride = W.rows;
  o.part = s->wsp<float>(L.part);
  o.cnt = s->wsp<unsigned>(L.cnt);
  const Plan pl = L.phead;
  HIPCHK(launch_gemv(W, 1, s->act_a(1), s->norm_h(), o, pl.ks, pl.w, st));
  HIPCHK(launch_argmax(lg, c.vocab, s->wsp<float>(L.amax_v), s->wsp<int>(L.amax_i), L.amax_parts, tok, st));
  return SLICE_OK;
}

int slice_position(const slice_t* s) { return s ? s->pos : -1; }

void slice_free(slice_t* s) {
  if (!s) return;
  for (auto& kv : s->graphs) hipGraphExecDestroy(kv.second);
  if (s->cap) hipStreamDestroy(s->cap);
  delete s;
}

int slice_dbg_set_state(slice_t* s, int layer, const float* src, void* stream) {
  if (!s || !src) return fail(SLICE_EINVAL, "null argument");
  const slice_config& c = s->cfg;
  if (layer < c.layer_begin || layer >= c.layer_end) return fail(SLICE_ERANGE, "layer outside the slice");
  const LayerLayout& ll = s->L.layers[layer - c.layer_begin];
  if (ll.attn) return fail(SLICE_EINVAL, "not a DeltaNet layer");
  float* st = reinterpret_cast<float*>(s->ws + s->L.dn + (size_t)ll.dn_index * s->L.dn_layer_bytes);
  HIPCHK(launch_state_io(st, s->L.nslots, s->ctrl(), c.dn_heads, c.dn_dk, c.dn_dv, const_cast<float*>(src), 1, S(stream)));
  return SLICE_OK;
}

int slice_dbg_get_state(slice_t* s, int layer, float* dst, void* stream) {
  if (!s || !dst) return fail(SLICE_EINVAL, "null argument");
  const slice_config& c = s->cfg;
  if (layer < c.layer_begin || layer >= c.layer_end) return fail(SLICE_ERANGE, "layer outside the slice");
  const LayerLayout& ll = s->L.layers[layer - c.layer_begin];
  if (ll.attn) return fail(SLICE_EINVAL, "not a DeltaNet layer");
  float* st = reinterpret_cast<float*>(s->ws + s->L.dn + (size_t)ll.dn_index * s->L.dn_layer_bytes);
  HIPCHK(launch_state_io(st, s->L.nslots, s->ctrl(), c.dn_heads, c.dn_dk, c.dn_dv, dst, 0, S(stream)));
  return SLICE_OK;
}

static int kv_io(slice_t* s, int layer, uint16_t* k, uint16_t* v, int rows, int to_device, void* stream) {
  if (!s || !k || !v) return fail(SLICE_EINVAL, "null argument");
  const slice_config& c = s->cfg;
  if (layer < c.layer_begin || layer >= c.layer_end) return fail(SLICE_ERANGE, "layer outside the slice");
  const LayerLayout& ll = s->L.layers[layer - c.layer_begin];
  if (!ll.attn) return fail(SLICE_EINVAL, "not an attention layer");
  if (rows < 0 || rows > c.max_seq) return fail(SLICE_ERANGE, "rows outside 0..max_seq");
  uint8_t* kvb = s->ws + s->L.kv + (size_t)ll.attn_index * s->L.kv_layer_bytes;
  __half* kc = reinterpret_cast<__half*>(kvb);
  __half* vc = reinterpret_cast<__half*>(kvb + (size_t)c.kv_heads * c.max_seq * c.head_dim * 2);
  HIPCHK(launch_kv_io(kc, vc, c.kv_heads, c.max_seq, c.head_dim, k, v, rows, to_device, S(stream)));
  return SLICE_OK;
}

int slice_dbg_get_hidden(slice_t* s, float* dst, int k, void* stream) {
  if (!s || !dst) return fail(SLICE_EINVAL, "null argument");
  if (k < 1 || k > s->L.mt) return fail(SLICE_ERANGE, "k outside 1..max_verify");
  HIPCHK(hipMemcpyAsync(dst, s->ws + s->L.h, (size_t)k * s->cfg.hidden * 4, hipMemcpyDeviceToDevice, S(stream)));
  return SLICE_OK;
}

int slice_dbg_set_kv(slice_t* s, int layer, const uint16_t* k, const uint16_t* v, int rows, void* stream) {
  return kv_io(s, layer, const_cast<uint16_t*>(k), const_cast<uint16_t*>(v), rows, 1, stream);
}

int slice_dbg_get_kv(slice_t* s, int layer, uint16_t* k, uint16_t* v, int rows, void* stream) {
  return kv_io(s, layer, k, v, rows, 0, stream);
}

}  // extern "C"
