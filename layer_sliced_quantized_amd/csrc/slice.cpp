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
#include <mutex>
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

// Launch-shape overrides for tests and tuning sweeps, set only through
// slq_debug_override (never read from the environment, so a process cannot
// change a product's summation order by inheriting a variable).  Slices take
// them at slice_load; the standalone GEMV at each call.
std::mutex g_ovr_mu;
std::map<std::string, int> g_ovr;

int override_int(const std::string& name, int dflt) {
  std::lock_guard<std::mutex> lk(g_ovr_mu);
  auto it = g_ovr.find(name);
  return it == g_ovr.end() ? dflt : it->second;
}

bool override_name_ok(const std::string& n) {
  if (n == "MFMA_MIN_T" || n == "EAGER" || n == "CHAIN" || n == "CHAIN_MAX" || n == "CHAIN_DN" || n == "CHAIN_ATT" ||
      n == "CHAIN_G1")
    return true;
  static const char* kinds[] = {"G1", "G2", "F1", "F2", "HEAD", "GEMV", "G1P", "G2P", "F1P", "F2P",
                                "G1W", "G2W", "F1W", "F2W"};
  for (const char* k : kinds)
    if (n == std::string("KS_") + k || n == std::string("W_") + k) return true;
  return false;
}

// Launch shape of one GEMV: `ks` workgroups share the K tiles of each 64-row
// group (their partial sums meet through atomics), `w` waves per workgroup.
// Defaults come from kernel-trace sweeps on MI355X at hidden 5120 (all Q4_0):
//   input projections (16448/14336 x 5120): ks 4, w 4
//   gate/up + SwiGLU (34816 x 5120):        ks 2, w 4
//   down projection (5120 x 17408):         ks 8, w 4
//   mixer output (5120 x 4096 / 6144):      ks 4, w 4
// (one token: within 1 % of the best shape for every kind; at most 4 waves
// per workgroup also lets a verify pass of 4 tokens use the MFMA products).
// Q8_0 input projections take 2 splits: their tiles carry twice the bytes
// (64-layer Q8_0 slice in chained decode: 182.4 against 180.5 tok/s with 4,
// 169.7 with 1).
// Other shapes: enough splits for ~1000 workgroups, about two tiles per wave,
// at most 4 waves per workgroup.
// Overrides KS_<kind> / W_<kind> (kinds G1, G2, F1, F2, HEAD, GEMV) through
// slq_debug_override.
struct Plan {
  int ks, w;
};

int clampi(int v, int lo, int hi) { return v < lo ? lo : v > hi ? hi : v; }

// Fewest tokens per call that go to the int8-MFMA products: 0 leaves the
// choice to gemm_min_tokens (by format and waves per workgroup); the override
// MFMA_MIN_T sets a fixed count instead.
int mfma_min_tokens() { return clampi(override_int("MFMA_MIN_T", 0), 0, MAX_T + 1); }

Plan plan_gemv(const char* kind, int64_t rows, int64_t cols, int qt = QT_Q4) {
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
    if (k == "F2" || k == "G1") p.ks = clampi(p.ks, 1, k == "F2" ? 8 : qt == QT_Q8 ? 2 : 4);
    // at most 4 waves: one token is as fast as with 8 (LM head 248320 x 5120:
    // 114.8 against 115.1 us) and the batched products fit and stream longer
    // per wave (16 tokens: 474 against 874 us)
    p.w = clampi(k == "GEMV" || k == "HEAD" ? (ntiles / p.ks + 1) / 2 : 4, 1, 4);
  }
  p.ks = clampi(override_int("KS_" + k, p.ks), 1, 16);
  p.w = clampi(override_int("W_" + k, p.w), 1, 8);
  return p;
}

// Launch shape of the products of a prompt pass (slice_prefill), which need
// not sum in decode's order: four waves per workgroup and splits for about
// 2048 waves in all, at least one tile per wave.  At 16 tokens on MI355X this
// is the fastest shape, or within 6 % of it, for every product of the
// hidden-5120 hybrid in Q4_0 and Q8_0 (standalone sweep; e.g. gate/up 53.5
// against 57.1 us with the decode shape, attention input 31.1 against 39.2).
// Overrides KS_<kind>P / W_<kind>P.
Plan plan_pass(const char* kind, int64_t rows, int64_t cols) {
  const int nrg = (int)((rows + RG - 1) / RG);
  const int ntiles = (int)((cols / QK + TB - 1) / TB);
  const std::string k(kind);
  Plan p;
  p.w = clampi(ntiles, 1, 4);
  p.ks = clampi((4096 + p.w * nrg) / (2 * p.w * nrg), 1, std::max(1, ntiles / p.w));   // round(2048 / (w nrg))
  p.ks = clampi(override_int("KS_" + k + "P", p.ks), 1, 16);
  p.w = clampi(override_int("W_" + k + "P", p.w), 1, 8);
  return p;
}

// Launch shape of the products of prompt passes of 17..64 tokens (token
// groups of 16, each group its own waves): four waves per workgroup (one K
// part of four groups, or two of two) and splits for about 512 workgroups, at
// most one per tile (64 tokens, 8 layers at hidden 5120 on MI355X: 4.32 ms
// per pass against 4.61 with about 1024).  Overrides KS_<kind>W.
Plan plan_wide(const char* kind, int64_t rows, int64_t cols) {
  const int nrg = (int)((rows + RG - 1) / RG);
  const int ntiles = (int)((cols / QK + TB - 1) / TB);
  Plan p;
  p.w = 4;
  p.ks = clampi((512 + nrg / 2) / nrg, 1, std::min(16, std::max(1, ntiles)));
  p.ks = clampi(override_int(std::string("KS_") + kind + "W", p.ks), 1, 16);
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
  Plan wg1{1, 1}, wg2{1, 1}, wf1{1, 1}, wf2{1, 1};   // ... of more than 16 tokens
  size_t attn_norm = 0, ffn_norm = 0, q_norm = 0, k_norm = 0;
  // row offsets inside g1
  int off_q = 0, off_k = 0, off_v = 0, off_a = 0, off_b = 0, off_z = 0, off_g = -1;
  size_t dn_conv_w = 0, dn_alog = 0, dn_dtb = 0, dn_normw = 0;   // qwen3_5-form DeltaNet vectors
  int dn_index = -1, attn_index = -1;
  // chained decode: the digits this layer's phases hand on (the update's
  // output, the FFN input, the SwiGLU output, the next mixer input), each
  // layer its own so that a launch over several layers writes every digit
  // buffer once
  size_t cxu_d = 0, cxu_s = 0, cxa_d = 0, cxa_s = 0, cxm_d = 0, cxm_s = 0, cxb_d = 0, cxb_s = 0;
};

struct Layout {
  std::vector<LayerLayout> layers;   // index l - begin
  Mat embed, head;
  Plan phead{1, 1};
  Mat mtp_fc;                         // draft head: input projection [H][2H]
  Plan pmtp{1, 1};
  size_t mtp_ne = 0, mtp_nh = 0;      // ... and the norms of its two inputs
  size_t out_norm = 0;
  size_t wbytes = 0;
  // workspace
  size_t ctrl = 0, h = 0, xa_d = 0, xa_s = 0, xu_d = 0, xu_s = 0, xm_d = 0, xm_s = 0, ssq = 0, y1 = 0,
         xa_md = 0, xu_md = 0, xm_md = 0,
         part = 0, cnt = 0, apart = 0, rope = 0, logits = 0, amax_v = 0, amax_i = 0, kv = 0, dn = 0;
  // chained decode: digits and statistics of the mixer inputs (the FFN input
  // keeps xa / ssq), per-product split-K regions, per-layer descriptors and
  // sync regions
  size_t xb_d = 0, xb_s = 0, ssq_b = 0, chain_sync = 0;
  size_t xe_d = 0, xe_s = 0, mtp_y = 0;   // draft head: input digits (2H wide) and projection
  size_t cpart[CHAIN_PART_BUFS] = {}, ccnt[CHAIN_PART_BUFS] = {};
  size_t chain_sync_bytes = 0;
  size_t ccnt_n = 0;      // u32 tickets in each ccnt region
  size_t kv_layer_bytes = 0, dn_layer_bytes = 0;
  size_t conv = 0, conv_layer_bytes = 0;   // qwen3_5-form DeltaNet conv states
  int64_t conv_slot = 0;                   // floats per conv-state slot
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
  if (c.max_prefill < 0 || c.max_prefill > MAX_PASS) return "max_prefill must be in 0..64";
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
    if (c.dn_variant != 0 && c.dn_variant != 1) return "dn_variant must be 0 or 1";
    if (c.dn_variant) {
      if (c.dn_conv < 2 || c.dn_conv > 4) return "dn_conv must be in 2..4";
      if (c.dn_k_heads < 0 || (c.dn_k_heads && c.dn_heads % c.dn_k_heads)) return "dn_heads must be a multiple of dn_k_heads";
      if (c.dn_dv > 128 || 7 * c.dn_dv < 2 * c.dn_dk)
        return "the qwen3_5 DeltaNet form needs dv <= 128 and 7 dv >= 2 dk (a thread per conv channel)";
    }
  }
  if ((c.has_embed || c.has_head) && c.vocab <= 0) return "vocab must be > 0 with an embedding or head";
  if (c.has_mtp != 0 && c.has_mtp != 1) return "has_mtp must be 0 or 1";
  if (c.max_prefill > MAX_T && c.dn_variant && any_dn)
    return "prompt passes of more than 16 tokens need the chunked DeltaNet (dn_variant 0)";
  if (c.has_mtp && !c.has_embed) return "a draft head (has_mtp) needs has_embed";
  if (c.has_mtp && c.hidden > 8192) return "a draft head needs hidden <= 8192";
  return "";
}

// Query/key heads of the DeltaNet layers, and the conv channels of the qwen3_5 form.
int dn_kh(const slice_config& c) { return c.dn_variant && c.dn_k_heads > 0 ? c.dn_k_heads : c.dn_heads; }
int dn_conv_dim(const slice_config& c) { return 2 * dn_kh(c) * c.dn_dk + c.dn_heads * c.dn_dv; }

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
  L.mt = std::max(c.max_verify, c.max_prefill);   // tokens a step may carry
  L.nslots = c.max_verify + 1;
  const int nkd = dn_kh(c) * c.dn_dk, nvd = c.dn_heads * c.dn_dv;
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
    } else if (c.dn_variant) {
      ll.dn_conv_w = vec((int64_t)dn_conv_dim(c) * c.dn_conv);
      ll.dn_alog = vec(c.dn_heads);
      ll.dn_dtb = vec(c.dn_heads);
      ll.dn_normw = vec(c.dn_dv);
    }
    L.layers.push_back(ll);
  }
  if (c.has_embed || (c.has_head && c.tied_head)) L.embed = mat(c.vocab, H);
  if (c.has_head && !c.tied_head) L.head = mat(c.vocab, H);
  L.out_norm = vec(H);
  if (c.has_mtp) {
    L.mtp_fc = mat(H, 2 * (int64_t)H);
    L.mtp_ne = vec(H);
    L.mtp_nh = vec(H);
  }
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
  auto mdigits = [&](int nblk) {
    return mt > 1 ? (size_t)mx_block_bytes(c.qtype) * (nblk ? nblk : 1) * gemm_groups(mt) : 0;
  };
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
    p = plan_gemv(kind, m.rows, m.cols, c.qtype);
    const int64_t nrg = (m.rows + RG - 1) / RG;
    rg_max = std::max<int64_t>(rg_max, nrg);
    part_floats = std::max<size_t>(part_floats, (size_t)nrg * p.ks * mt * RG);
    if (q) {
      *q = plan_pass(kind, m.rows, m.cols);
      part_floats = std::max<size_t>(part_floats, (size_t)nrg * q->ks * mt * RG);
    }
  };
  auto updw = [&](const Mat& m, Plan& p, const char* kind) {
    if (!m.present || mt <= MAX_T) return;
    p = plan_wide(kind, m.rows, m.cols);
    part_floats = std::max<size_t>(part_floats, (size_t)((m.rows + RG - 1) / RG) * p.ks * mt * RG);
  };
  for (LayerLayout& ll : L.layers) {
    upd(ll.g1, ll.pg1, &ll.qg1, "G1");
    upd(ll.g2, ll.pg2, &ll.qg2, "G2");
    upd(ll.f1, ll.pf1, &ll.qf1, "F1");
    upd(ll.f2, ll.pf2, &ll.qf2, "F2");
    updw(ll.g1, ll.wg1, "G1");
    updw(ll.g2, ll.wg2, "G2");
    updw(ll.f1, ll.wf1, "F1");
    updw(ll.f2, ll.wf2, "F2");
  }
  if (c.has_head) upd(c.tied_head ? L.embed : L.head, L.phead, nullptr, "HEAD");
  if (c.has_mtp) upd(L.mtp_fc, L.pmtp, nullptr, "F2");
  L.part = take(part_floats * 4);
  L.cnt = take((size_t)std::max<int64_t>(rg_max, 1) * 4);
  if (!L.layers.empty()) {
    L.xb_d = take((size_t)XW * 4 * nblkH);
    L.xb_s = take((size_t)4 * nblkH);
    L.ssq_b = take((size_t)(H / RG) * 4);
    size_t cpf = 0;
    for (const LayerLayout& ll : L.layers)
      for (const auto& mp : {std::make_pair(&ll.g1, &ll.pg1), std::make_pair(&ll.g2, &ll.pg2),
                             std::make_pair(&ll.f1, &ll.pf1), std::make_pair(&ll.f2, &ll.pf2)})
        if (mp.first->present) cpf = std::max<size_t>(cpf, (size_t)((mp.first->rows + RG - 1) / RG) * mp.second->ks * RG);
    L.ccnt_n = (size_t)std::max<int64_t>(rg_max, 1);
    for (int p = 0; p < CHAIN_PART_BUFS; ++p) {
      L.cpart[p] = take(cpf * 4);
      L.ccnt[p] = take(L.ccnt_n * 4);
    }
    // at most five phases per layer (update, mixer output, gate/up, down, next input projections)
    // (and the first layer's input projections)
    L.chain_sync_bytes = (L.layers.size() * 5 + 1) * CHAIN_PHASE_SYNC_BYTES;
    L.chain_sync = take(L.chain_sync_bytes);
    for (LayerLayout& ll : L.layers) {
      ll.cxu_d = take((size_t)XW * 4 * nblkU);
      ll.cxu_s = take((size_t)4 * nblkU);
      ll.cxa_d = take((size_t)XW * 4 * nblkH);
      ll.cxa_s = take((size_t)4 * nblkH);
      if (nblkM) {
        ll.cxm_d = take((size_t)XW * 4 * nblkM);
        ll.cxm_s = take((size_t)4 * nblkM);
      }
      ll.cxb_d = take((size_t)XW * 4 * nblkH);
      ll.cxb_s = take((size_t)4 * nblkH);
    }
  }
  if (L.n_attn) {
    L.nchunk = (c.max_seq + ATT_CHUNK - 1) / ATT_CHUNK;
    L.apart = take((size_t)std::min(mt, MAX_T) * c.q_heads * L.nchunk * (c.head_dim + 2) * 4);
    L.rope = take((size_t)c.max_seq * (c.rope_dims / 2 > 0 ? c.rope_dims / 2 : 1) * 8);
  }
  if (c.has_mtp) {
    L.xe_d = take((size_t)XW * 4 * (2 * H / QK));
    L.xe_s = take((size_t)4 * (2 * H / QK));
    L.mtp_y = take((size_t)H * 4);
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
  if (c.dn_variant && L.n_dn) {
    // every value head keeps its own q / k windows: [head][2 dk + dv][conv - 1]
    L.conv_slot = (int64_t)c.dn_heads * (2 * c.dn_dk + c.dn_dv) * (c.dn_conv - 1);
    L.conv_layer_bytes = al256((size_t)L.nslots * L.conv_slot * 4);
    L.conv = take((size_t)L.n_dn * L.conv_layer_bytes);
  }
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
  bool chain = false;                 // decode steps run the chained GEMV kernels
  bool chain_dn = false;              // ... with each DeltaNet layer's update as a phase
  bool chain_att = false;             // ... and each attention layer's merge as the first phase of
                                      // the launch after its split kernel
  bool chain_g1_first = false;        // ... and the first layer's input projections (a DeltaNet layer)
                                      // as the first phase of the first launch
  struct ChainLaunch {
    int layer;                        // the layer whose mixer it follows
    ChainArgs args;                   // descriptors (kernel arguments)
    unsigned grid;                    // workgroups
    size_t sync;                      // sync region (workspace offset)
  };
  std::vector<ChainLaunch> chain_launch;   // in step order
  Act act_b() const { return Act{wsp<int32_t>(L.xb_d), wsp<float>(L.xb_s), cfg.hidden / QK, nullptr, mx_min_t}; }
  NormIn norm_b() const { return NormIn{wsp<float>(L.ssq_b), cfg.hidden / RG, 1.0f / (float)cfg.hidden, cfg.eps}; }
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

// Norm weights of the RMSNorm in front of layer i (past the last layer the
// digits are not consumed; any valid vector will do): offset in the weights.
static size_t attn_norm_off(const slice* s, int i) {
  const Layout& L = s->L;
  return i < (int)L.layers.size() ? L.layers[i].attn_norm : L.out_norm;
}

// The mixer of layer i (DeltaNet update or attention) on the G1 output y1;
// its output digits go to xu.
// The DeltaNet update of layer i for T tokens in `mode`.
static DnParams dn_params(slice* s, int i, int T, int mode) {
  const slice_config& c = s->cfg;
  const Layout& L = s->L;
  const LayerLayout& ll = L.layers[i];
  DnParams p{};
  p.y = s->wsp<float>(L.y1);
  p.y_stride = ll.g1.rows;
  p.off_q = ll.off_q; p.off_k = ll.off_k; p.off_v = ll.off_v;
  p.off_a = ll.off_a; p.off_b = ll.off_b; p.off_z = ll.off_z;
  p.heads = c.dn_heads; p.dk = c.dn_dk; p.dv = c.dn_dv;
  p.a_scale = c.dn_a_scale; p.a_bias = c.dn_a_bias; p.b_scale = c.dn_b_scale; p.z_scale = c.dn_z_scale;
  p.state = reinterpret_cast<float*>(s->ws + L.dn + (size_t)ll.dn_index * L.dn_layer_bytes);
  p.nslots = L.nslots;
  p.mode = mode;
  p.ctrl = s->ctrl();
  p.u_out = nullptr;
  p.next = s->act_u(T);
  p.next_qt = c.qtype;
  if (c.dn_variant) {
    p.variant = 1;
    p.k_heads = dn_kh(c);
    p.conv = c.dn_conv;
    p.eps = c.eps;
    p.conv_w = reinterpret_cast<const float*>(s->w + ll.dn_conv_w);
    p.a_log = reinterpret_cast<const float*>(s->w + ll.dn_alog);
    p.dt_bias = reinterpret_cast<const float*>(s->w + ll.dn_dtb);
    p.norm_w = reinterpret_cast<const float*>(s->w + ll.dn_normw);
    p.conv_state = reinterpret_cast<float*>(s->ws + L.conv + (size_t)ll.dn_index * L.conv_layer_bytes);
    p.conv_slot = L.conv_slot;
  }
  return p;
}

// The same activations seen from token t0 on (t0 a multiple of 16: token
// group t0 / 16 starts a record of its own in the MFMA layout).
static Act act_from(const Act& a, int t0, int qt) {
  Act r = a;
  r.xd += (size_t)t0 * a.nblk * XW;
  r.xs += (size_t)t0 * a.nblk;
  if (r.mxd) r.mxd += (size_t)(t0 / MX_SLOTS) * a.nblk * (mx_block_bytes(qt) / 4);
  return r;
}

// Attention parameters of layer i for tokens t0 .. of a step of Tall tokens.
static AttnParams attn_params(slice* s, int i, int Tall, int t0) {
  const slice_config& c = s->cfg;
  const Layout& L = s->L;
  const LayerLayout& ll = L.layers[i];
  AttnParams p{};
  p.y = s->wsp<float>(L.y1) + (size_t)t0 * ll.g1.rows;
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
  p.ctrl = s->ctrl();
  p.part = s->wsp<float>(L.apart);
  p.nchunk = L.nchunk;
  p.rchunks = 1;
  p.u_out = nullptr;
  p.pos_off = t0;
  p.next = act_from(s->act_u(Tall), t0, c.qtype);
  p.next_qt = c.qtype;
  return p;
}

// Layer i's mixer for tokens t0 .. t0 + T - 1 of a step of Tall tokens.
static int enqueue_mixer_part(slice* s, int i, int Tall, int t0, int T, int mode, hipStream_t st) {
  const slice_config& c = s->cfg;
  const Layout& L = s->L;
  const LayerLayout& ll = L.layers[i];
  float* y1 = s->wsp<float>(L.y1) + (size_t)t0 * ll.g1.rows;
  if (ll.attn) {
    const AttnParams p = attn_params(s, i, Tall, t0);
    HIPCHK(launch_attention(p, T, st));
  } else {
    DnParams p = dn_params(s, i, T, mode);
    p.y = y1;
    p.next = act_from(s->act_u(Tall), t0, c.qtype);
    HIPCHK(launch_deltanet(p, T, st));
  }
  return SLICE_OK;
}

// A prompt pass of more than 16 tokens runs each mixer in sub-passes of 16
// (tokens t0 .. t0 + 15 at positions pos + t0 ..): attention appends and
// attends causally in order, the chunked DeltaNet carries its state from one
// sub-pass to the next; the products around the mixers take all tokens at once.
static int enqueue_mixer(slice* s, int i, int T, int mode, hipStream_t st) {
  if (T <= MAX_T) return enqueue_mixer_part(s, i, T, 0, T, mode, st);
  if (mode != DN_CHUNK) return fail(SLICE_EINVAL, "more than 16 tokens only in a prompt pass");
  for (int t0 = 0; t0 < T; t0 += MAX_T) {
    int rc = enqueue_mixer_part(s, i, T, t0, std::min(MAX_T, T - t0), mode, st);
    if (rc) return rc;
  }
  return SLICE_OK;
}

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
  auto norm_at = [&](size_t off) { return reinterpret_cast<const float*>(s->w + off); };
  float* part = s->wsp<float>(L.part);
  unsigned* cnt = s->wsp<unsigned>(L.cnt);
  auto g1_out = [&]() {
    GemvOut o{};
    o.kind = EPI_STORE;
    o.y = y1;
    o.part = part;
    o.cnt = cnt;
    return o;
  };

  if (decode && s->chain && nlay > 0 && (only < 0 || only == SLICE_OP_CHAIN)) {
    // Chained decode: entry, the first layer's input projections, then per
    // layer its mixer and one kernel for the products after it (mixer output,
    // gate/up, down, the next layer's input projections), then the exit.
    if (only < 0) {
      SLQ_MARK(-1);
      HIPCHK(launch_resid_finish(c.io_fp32 ? 2 : 1, nullptr, ctrl, H, 1, H, h, norm_at(attn_norm_off(s, 0)), qt,
                                 s->act_b(), s->wsp<float>(L.ssq_b), st));
      SLQ_MARK(SLICE_OP_ENTRY);
      if (!s->chain_g1_first) {   // else the first chained launch starts with them
        const LayerLayout& l0 = L.layers[0];
        GemvOut o = g1_out();
        o.y_tstride = l0.g1.rows;
        HIPCHK(launch_gemv(s->packed(l0.g1), 1, s->act_b(), s->norm_b(), o, l0.pg1.ks, l0.pg1.w, st));
        SLQ_MARK(l0.attn ? SLICE_OP_ATT_IN : SLICE_OP_DN_IN);
      }
    }
    for (int i = 0; i < nlay; ++i) {
      if (only < 0 && L.layers[i].attn && s->chain_att) {
        // the split only: the next chained launch merges it first
        AttnParams p = attn_params(s, i, 1, 0);
        p.split_only = 1;
        HIPCHK(launch_attention(p, 1, st));
        SLQ_MARK(SLICE_OP_ATTENTION);
      } else if (only < 0 && (L.layers[i].attn || !s->chain_dn)) {
        int rc = enqueue_mixer(s, i, 1, DN_DECODE, st);
        if (rc) return rc;
        SLQ_MARK(L.layers[i].attn ? SLICE_OP_ATTENTION : SLICE_OP_DELTANET);
      }
      for (const slice::ChainLaunch& cl : s->chain_launch) {
        if (cl.layer != i) continue;
        HIPCHK(launch_chain(qt, cl.args, cl.grid, s->w, s->ws, reinterpret_cast<unsigned*>(s->ws + cl.sync), ctrl, st));
        SLQ_MARK(SLICE_OP_CHAIN);
      }
    }
    if (only < 0) HIPCHK(launch_store_out(h, 1, H, nullptr, c.io_fp32, ctrl, 1, st));
    SLQ_MARK(SLICE_OP_EXIT);
    return SLICE_OK;
  }
  if (only == SLICE_OP_CHAIN) return fail(SLICE_EINVAL, "the slice does not run chained products");

  // entry: boundary vector -> h, digits of attn_norm(first layer) * h
  SLQ_MARK(-1);
  if (only < 0) HIPCHK(launch_resid_finish(c.io_fp32 ? 2 : 1, nullptr, ctrl, H, T, H, h, norm_at(attn_norm_off(s, 0)), qt, s->act_a(T), ssq, st));
  SLQ_MARK(SLICE_OP_ENTRY);
  for (int i = 0; i < nlay; ++i) {
    const LayerLayout& ll = L.layers[i];
    const int k_in = ll.attn ? SLICE_OP_ATT_IN : SLICE_OP_DN_IN;
    const int k_mix = ll.attn ? SLICE_OP_ATTENTION : SLICE_OP_DELTANET;
    const int k_out = ll.attn ? SLICE_OP_ATT_OUT : SLICE_OP_DN_OUT;
    // mixer input projections: G1 = [q|k|v|a|b|z] or [q|g|k|v] of RMSNorm(h)
    if (only < 0 || only == k_in) {
      const Packed W = s->packed(ll.g1);
      GemvOut o = g1_out();
      o.y_tstride = W.rows;
      const Plan pl = pass ? (T > MAX_T ? ll.wg1 : ll.qg1) : ll.pg1;
      HIPCHK(launch_gemv(W, T, s->act_a(T), s->norm_h(), o, pl.ks, pl.w, st));
      SLQ_MARK(k_in);
    }
    if (only < 0 || only == k_mix) {
      int rc = enqueue_mixer(s, i, T, mode, st);
      if (rc) return rc;
      SLQ_MARK(k_mix);
    }
    // residual update after the mixer: h += W_o u, then digits for the next RMSNorm
    const size_t nw_after_mixer = c.ffn ? ll.ffn_norm : attn_norm_off(s, i + 1);
    auto residual = [&](const Mat& m, Act in, size_t next_norm, const Plan& pl) -> int {
      const Packed W = s->packed(m);
      GemvOut o{};
      o.kind = EPI_RESID;
      o.y = h;
      o.y_tstride = H;
      o.next = s->act_a(T);
      o.next_qt = qt;
      o.ssq_out = ssq;
      o.norm_w = norm_at(next_norm);
      o.part = part;
      o.cnt = cnt;
      HIPCHK(launch_gemv(W, T, in, NormIn{nullptr, 0, 0.f, 0.f}, o, pl.ks, pl.w, st));
      return SLICE_OK;
    };
    int rc = (only < 0 || only == k_out)
                 ? residual(ll.g2, s->act_u(T), nw_after_mixer, pass ? (T > MAX_T ? ll.wg2 : ll.qg2) : ll.pg2)
                 : SLICE_OK;
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
      const Plan pl = pass ? (T > MAX_T ? ll.wf1 : ll.qf1) : ll.pf1;
      HIPCHK(launch_gemv(W, T, s->act_a(T), s->norm_h(), o, pl.ks, pl.w, st));
      SLQ_MARK(SLICE_OP_FFN_IN);
    }
    if (c.ffn && (only < 0 || only == SLICE_OP_FFN_OUT)) {
      rc = residual(ll.f2, s->act_m(T), attn_norm_off(s, i + 1), pass ? (T > MAX_T ? ll.wf2 : ll.qf2) : ll.pf2);
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

// Descriptors of the chained decode phases (one token), in step order: per
// layer [DeltaNet update (DeltaNet layers, when chained), mixer output (+
// residual), gate/up + SwiGLU, down (+ residual), next layer's input
// projections], with the launch shapes of the separate kernels, so that
// results are the same bit for bit.  A launch runs the phases of consecutive
// layers up to the next layer whose mixer is a kernel of its own (attention,
// or every mixer when the updates are not chained), at most CHAIN_MAX phases
// (a layer whose phases do not fit starts the next launch).  Each layer's
// phases hand on digits through buffers of its own (cxu, cxa, cxm, cxb), and
// the statistics through ssq (FFN input) and ssq_b (next mixer input), so a
// launch writes every digit buffer once.
static void build_chains(slice* s) {
  const slice_config& c = s->cfg;
  const Layout& L = s->L;
  const int H = c.hidden, nblkH = H / QK;
  const int nlay = (int)L.layers.size();
  s->chain_launch.clear();
  // phases per chained kernel (tuning; CHAIN_MAX_PHASES at most)
  const int per = clampi(override_int("CHAIN_MAX", CHAIN_MAX_PHASES), 1, CHAIN_MAX_PHASES);
  const int nblkU = (L.nu + QK - 1) / QK;
  struct Step {
    ChainPhase ph;
    int layer;   // the layer whose step the phase belongs to (the next input projections: the layer before)
  };
  std::vector<Step> open;   // phases of the launch being built
  size_t sync = L.chain_sync;
  auto close = [&]() {
    if (open.empty()) return;
    slice::ChainLaunch cl{};
    cl.layer = open[0].layer;
    cl.args.nph = (int)open.size();
    cl.args.first_wg[0] = 0;
    int dn_layer = -1, att_layer = -1;
    for (int k = 0; k < cl.args.nph; ++k) {
      ChainPhase q = open[k].ph;
      // split-K regions in turn: a phase runs only after the one before has
      // completed, so phase k + CHAIN_PART_BUFS finds phase k's regions free
      q.part_off = (int64_t)L.cpart[k % CHAIN_PART_BUFS];
      q.cnt_off = (int64_t)L.ccnt[k % CHAIN_PART_BUFS];
      cl.args.ph[k] = q;
      cl.args.first_wg[k + 1] = cl.args.first_wg[k] + q.nwg;
      const int nrg = (int)((q.rows + RG - 1) / RG);
      cl.args.gsize[k] = (nrg + 31) / 32;   // at most 32 completion groups
      if (q.epi == EPI_DN && dn_layer < 0) dn_layer = open[k].layer;
      if (q.epi == EPI_ATT_COMB && att_layer < 0) att_layer = open[k].layer;
    }
    cl.grid = (unsigned)cl.args.first_wg[cl.args.nph];
    if (dn_layer >= 0) {
      // shared by the launch's updates; state and output digits come per phase
      cl.args.dn = dn_params(s, dn_layer, 1, DN_DECODE);
      cl.args.dn_dkp = c.dn_dk / 8;
    }
    if (att_layer >= 0) cl.args.att = attn_params(s, att_layer, 1, 0);   // output digits come per phase
    cl.sync = sync;
    sync += (size_t)cl.args.nph * CHAIN_PHASE_SYNC_BYTES;
    s->chain_launch.push_back(cl);
    open.clear();
  };
  for (int i = 0; i < nlay; ++i) {
    const LayerLayout& ll = L.layers[i];
    const bool dn_phase = s->chain_dn && !ll.attn;
    // a mixer that runs as a kernel of its own comes between two launches
    if (!dn_phase) close();
    std::vector<ChainPhase> ph;
    ph.reserve(6);   // add() hands out references into it
    auto add = [&](const Mat& m, const Plan& pl, int epi) -> ChainPhase& {
      ChainPhase q{};
      q.w_off = (int64_t)m.off;
      q.rows = m.rows;
      q.cols = m.cols;
      q.ssq_off = q.y_off = q.nd_off = q.ns_off = q.ssq_out_off = q.norm_w_off = -1;
      q.qt = c.qtype;
      q.ksplit = pl.ks;
      q.nwg = (int)((m.rows + RG - 1) / RG) * pl.ks;
      q.epi = epi;
      q.w = pl.w;
      ph.push_back(q);
      return ph.back();
    };
    auto input = [&](ChainPhase& q, size_t d, size_t sc, int nblk, int64_t ssq) {
      q.xd_off = (int64_t)d;
      q.xs_off = (int64_t)sc;
      q.x_nblk = nblk;
      q.ssq_off = ssq;
      q.n_part = H / RG;
      q.inv_n = 1.0f / (float)H;
      q.eps = c.eps;
    };
    auto resid = [&](ChainPhase& q, size_t nd, size_t ns, size_t ssq_out, size_t norm_w) {
      q.y_off = (int64_t)L.h;
      q.y_tstride = H;
      q.nd_off = (int64_t)nd;
      q.ns_off = (int64_t)ns;
      q.n_nblk = nblkH;
      q.ssq_out_off = (int64_t)ssq_out;
      q.norm_w_off = (int64_t)norm_w;
    };
    if (i == 0 && s->chain_g1_first) {
      // the first layer's input projections, from the entry kernel's digits
      ChainPhase& g1 = add(ll.g1, ll.pg1, EPI_STORE);
      input(g1, L.xb_d, L.xb_s, nblkH, (int64_t)L.ssq_b);
      g1.y_off = (int64_t)L.y1;
      g1.y_tstride = ll.g1.rows;
    }
    if (dn_phase) {
      // the layer's DeltaNet update: one workgroup per 32 state rows of a head
      ChainPhase d{};
      d.epi = EPI_DN;
      d.nwg = c.dn_heads * (c.dn_dv / 32);
      d.rows = (int64_t)d.nwg * RG;   // counted as nwg row groups
      d.ksplit = 1;
      d.w = 4;
      d.qt = c.qtype;
      d.xd_off = d.xs_off = d.ssq_off = d.ssq_out_off = d.norm_w_off = -1;
      d.y_off = (int64_t)(L.dn + (size_t)ll.dn_index * L.dn_layer_bytes);
      d.nd_off = (int64_t)ll.cxu_d;
      d.ns_off = (int64_t)ll.cxu_s;
      ph.push_back(d);
    }
    const bool merge_phase = s->chain_att && ll.attn;
    if (merge_phase) {
      // the layer's attention merge, four (head, 64 dims) per workgroup, into this layer's digits
      ChainPhase m{};
      m.epi = EPI_ATT_COMB;
      m.nwg = (c.q_heads * (c.head_dim / 64) + 3) / 4;
      m.rows = (int64_t)m.nwg * RG;   // counted as nwg row groups
      m.ksplit = 1;
      m.w = 4;
      m.qt = c.qtype;
      m.xd_off = m.xs_off = m.ssq_off = m.ssq_out_off = m.y_off = m.norm_w_off = -1;
      m.nd_off = (int64_t)ll.cxu_d;
      m.ns_off = (int64_t)ll.cxu_s;
      ph.push_back(m);
    }
    ChainPhase& g2 = add(ll.g2, ll.pg2, EPI_RESID);
    // the update's or the merge's digits, or the separate mixer's (written before the launch)
    if (dn_phase || merge_phase) input(g2, ll.cxu_d, ll.cxu_s, nblkU, -1);
    else input(g2, L.xu_d, L.xu_s, nblkU, -1);
    if (c.ffn) {
      resid(g2, ll.cxa_d, ll.cxa_s, L.ssq, ll.ffn_norm);
      ChainPhase& f1 = add(ll.f1, ll.pf1, EPI_SWIGLU);
      input(f1, ll.cxa_d, ll.cxa_s, nblkH, (int64_t)L.ssq);
      f1.nd_off = (int64_t)ll.cxm_d;
      f1.ns_off = (int64_t)ll.cxm_s;
      f1.n_nblk = c.ffn / QK;
      ChainPhase& f2 = add(ll.f2, ll.pf2, EPI_RESID);
      input(f2, ll.cxm_d, ll.cxm_s, c.ffn / QK, -1);
      resid(f2, ll.cxb_d, ll.cxb_s, L.ssq_b, attn_norm_off(s, i + 1));
    } else {
      resid(g2, ll.cxb_d, ll.cxb_s, L.ssq_b, attn_norm_off(s, i + 1));
    }
    if (i + 1 < nlay) {
      const LayerLayout& nx = L.layers[i + 1];
      ChainPhase& g1 = add(nx.g1, nx.pg1, EPI_STORE);
      input(g1, ll.cxb_d, ll.cxb_s, nblkH, (int64_t)L.ssq_b);
      g1.y_off = (int64_t)L.y1;
      g1.y_tstride = nx.g1.rows;
    }
    // a layer whose phases do not fit the open launch starts the next one
    if (open.size() + ph.size() > (size_t)per) close();
    for (const ChainPhase& q : ph) {
      if (open.size() == (size_t)per) close();
      open.push_back(Step{q, i});
    }
  }
  close();
}

// Chained decode needs every product's plan within the chain kernel's four
// waves per workgroup.
static bool chains_possible(const slice* s) {
  // the RMSNorm statistics must fit the coherent two-load fetch (rnorm_fetch)
  if (s->cfg.hidden / RG > 128) return false;
  for (const LayerLayout& ll : s->L.layers)
    for (const Plan* p : {&ll.pg1, &ll.pg2, &ll.pf1, &ll.pf2})
      if (p->w > 4) return false;
  return !s->L.layers.empty();
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

// Shape of tensor `tid` of `layer` for config c: rows x cols blocks of the
// slice's format (kind = qtype) or an fp32 vector of rows entries (kind 0,
// cols 1).  Returns "" or the reason the tensor is not part of the slice.
namespace {

std::string tensor_shape(const slice_config& c, int layer, int tid, int64_t& rows, int64_t& cols, int& kind) {
  const int H = c.hidden;
  const int nkd = dn_kh(c) * c.dn_dk, nvd = c.dn_heads * c.dn_dv;
  const int nq = c.q_heads * c.head_dim, nkv = c.kv_heads * c.head_dim;
  auto mat = [&](int64_t r, int64_t cc) { rows = r; cols = cc; kind = c.qtype; return std::string(); };
  auto vec = [&](int64_t n) { rows = n; cols = 1; kind = 0; return std::string(); };
  if (tid == SLICE_T_EMBED) {
    if (!(c.has_embed || (c.has_head && c.tied_head))) return "slice has no embedding";
    return mat(c.vocab, H);
  }
  if (tid == SLICE_T_HEAD) {
    if (!c.has_head || c.tied_head) return "slice has no untied head";
    return mat(c.vocab, H);
  }
  if (tid == SLICE_T_OUT_NORM) return vec(H);
  if (tid == SLICE_T_MTP_FC || tid == SLICE_T_MTP_NORM_E || tid == SLICE_T_MTP_NORM_H) {
    if (!c.has_mtp) return "slice is not a draft head";
    return tid == SLICE_T_MTP_FC ? mat(H, 2 * (int64_t)H) : vec(H);
  }
  if (layer < c.layer_begin || layer >= c.layer_end) return "layer outside the slice";
  const bool attn = c.attn_period == 0 || (layer % c.attn_period) == c.attn_period - 1;
  switch (tid) {
    case SLICE_T_ATTN_NORM: return vec(H);
    case SLICE_T_FFN_NORM: return c.ffn ? vec(H) : "no FFN in this slice";
    case SLICE_T_W_GATE:
    case SLICE_T_W_UP: return c.ffn ? mat(c.ffn, H) : "no FFN in this slice";
    case SLICE_T_W_DOWN: return c.ffn ? mat(H, c.ffn) : "no FFN in this slice";
    default: break;
  }
  if (attn) {
    switch (tid) {
      case SLICE_T_WQ: return mat(nq, H);
      case SLICE_T_WG: return c.attn_gate ? mat(nq, H) : "no attention gate";
      case SLICE_T_WK:
      case SLICE_T_WV: return mat(nkv, H);
      case SLICE_T_WO: return mat(H, nq);
      case SLICE_T_Q_NORM:
      case SLICE_T_K_NORM: return vec(c.head_dim);
      default: return "not an attention-layer tensor";
    }
  }
  switch (tid) {
    case SLICE_T_DN_Q:
    case SLICE_T_DN_K: return mat(nkd, H);
    case SLICE_T_DN_V:
    case SLICE_T_DN_Z: return mat(nvd, H);
    case SLICE_T_DN_A:
    case SLICE_T_DN_B: return mat(c.dn_heads, H);
    case SLICE_T_DN_OUT: return mat(H, nvd);
    case SLICE_T_DN_CONV: return c.dn_variant ? vec((int64_t)dn_conv_dim(c) * c.dn_conv) : "dn_variant is 0";
    case SLICE_T_DN_ALOG:
    case SLICE_T_DN_DTB: return c.dn_variant ? vec(c.dn_heads) : "dn_variant is 0";
    case SLICE_T_DN_NORM: return c.dn_variant ? vec(c.dn_dv) : "dn_variant is 0";
    default: return "not a DeltaNet-layer tensor";
  }
}

size_t tensor_src_bytes(int64_t rows, int64_t cols, int kind) {
  if (kind == 0) return (size_t)rows * 4;
  return (size_t)rows * (size_t)(cols / QK) * (kind == SLICE_Q4_0 ? 18 : 34);
}

}  // namespace

// Scratch of the allocation-free standalone GEMV (slq_gemv_noalloc): one
// file-scope device array, which every GPU the library runs on holds until the
// process ends.  Host code never uses its name as an address: the device
// address is taken once per device with hipGetSymbolAddress (with that device
// current) and kept here.
static __device__ __align__(256) uint8_t scratch[SLQ_GEMV_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
std::map<int, uint8_t*> g_scratch_ptr;   // device id -> address of `scratch` on it

int scratch_on_current_device(uint8_t** out) {
  int dev = 0;
  HIPCHK(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SLICE_EHIP, std::string("slq_gemv_noalloc: hipGetSymbolAddress: ") + hipGetErrorString(e));
    it = g_scratch_ptr.emplace(dev, static_cast<uint8_t*>(p)).first;
  }
  *out = it->second;
  return SLICE_OK;
}

}  // namespace

namespace {

std::string attn_desc_error(const slq_attn_desc* d) {
  if (!d) return "null descriptor";
  if (d->q_heads <= 0 || d->kv_heads <= 0 || d->q_heads % d->kv_heads) return "q_heads must be a multiple of kv_heads";
  if (d->q_heads / d->kv_heads > 8) return "at most 8 query heads per KV head";
  if (d->head_dim <= 0 || d->head_dim % 64 || d->head_dim > 256) return "head_dim must be 64, 128, 192 or 256";
  if (d->rope_dims < 0 || d->rope_dims % 2 || d->rope_dims > d->head_dim) return "bad rope_dims";
  if (d->max_seq <= 0 || d->max_seq % 64) return "max_seq must be a positive multiple of 64";
  if (d->qk_norm && (!d->q_norm_dev || !d->k_norm_dev)) return "qk_norm needs both norm weight vectors";
  return "";
}

// attention workspace: the RoPE table, then the split partials [T][q_heads][nchunk][head_dim + 2]
size_t attn_rope_bytes(const slq_attn_desc* d) {
  return al256((size_t)d->max_seq * (d->rope_dims / 2 > 0 ? d->rope_dims / 2 : 1) * 8);
}

}  // namespace

// ====================================================================== ABI

extern "C" {

const char* slice_last_error(void) { return g_err.c_str(); }

int slq_debug_override(const char* name, int value) {
  if (!name) return fail(SLICE_EINVAL, "slq_debug_override: null name");
  const std::string n(name);
  if (!override_name_ok(n)) return fail(SLICE_EINVAL, "slq_debug_override: unknown name " + n);
  std::lock_guard<std::mutex> lk(g_ovr_mu);
  if (value < 0) g_ovr.erase(n);
  else g_ovr[n] = value;
  return SLICE_OK;
}

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

// Standalone GEMV workspace, in order: lane-row digits [batch][nblk][24],
// their scales, MFMA-layout block records, split-K partials
// [nrg][ks][batch][64] (only when the plan splits K), ticket counters [nrg].
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
  w.part = o; o += p.ks > 1 ? al256((size_t)nrg * p.ks * batch * RG * 4) : 0;
  w.cnt = o; o += al256((size_t)nrg * 4);
  w.total = o;
  return w;
}

// The two launches of a standalone GEMV on a workspace laid out by gemv_ws:
// activation digits, then the product.
static int run_gemv(int qtype, const void* packed_dev, int64_t rows, int64_t cols, int batch, const float* x_dev,
                    float* y_dev, uint8_t* ws, const GemvWs& L, hipStream_t st) {
  const int nblk = (int)(cols / QK);
  const int min_t = mfma_min_tokens();
  const bool mx = batch >= (min_t ? min_t : 2);
  Act a{reinterpret_cast<int32_t*>(ws + L.dig), reinterpret_cast<float*>(ws + L.sc), nblk,
        mx ? reinterpret_cast<int32_t*>(ws + L.mdig) : nullptr, min_t};
  HIPCHK(launch_quant_act(qtype, x_dev, batch, (int)cols, cols, a, st));
  const Plan pl = plan_gemv("GEMV", rows, cols);
  const Packed W{static_cast<const uint8_t*>(packed_dev), rows, cols, qtype};
  GemvOut o{};
  o.kind = EPI_STORE;
  o.y = y_dev;
  o.y_tstride = rows;
  o.part = reinterpret_cast<float*>(ws + L.part);
  o.cnt = reinterpret_cast<unsigned*>(ws + L.cnt);
  HIPCHK(launch_gemv(W, batch, a, NormIn{nullptr, 0, 0.f, 0.f}, o, pl.ks, pl.w, st));
  return SLICE_OK;
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
  return run_gemv(qtype, packed_dev, rows, cols, batch, x_dev, y_dev, static_cast<uint8_t*>(ws_dev),
                  gemv_ws(qtype, rows, cols, batch), S(stream));
}

int slq_gemv_noalloc(int qtype, const void* packed_dev, int64_t rows, int64_t cols, int batch, const float* x_dev,
                     float* y_dev, void* stream) {
  const size_t need = slq_gemv_workspace_bytes(qtype, rows, cols, batch);
  if (!need) return fail(SLICE_ESHAPE, "slq_gemv_noalloc: bad qtype, shape or batch (1..16)");
  if (need > SLQ_GEMV_NOALLOC_SCRATCH_BYTES)
    return fail(SLICE_ESHAPE, "slq_gemv_noalloc: this shape needs " + std::to_string(need) +
                                  " bytes of scratch; the static scratch holds " +
                                  std::to_string((size_t)SLQ_GEMV_NOALLOC_SCRATCH_BYTES) + " (use slq_gemv)");
  if (!packed_dev || !x_dev || !y_dev) return fail(SLICE_EINVAL, "slq_gemv_noalloc: null pointer");
  uint8_t* ws = nullptr;
  int rc = scratch_on_current_device(&ws);
  if (rc) return rc;
  const GemvWs L = gemv_ws(qtype, rows, cols, batch);
  // the row-group tickets must start at zero: a fill kernel (no memset node,
  // no allocation), then the same two launches as slq_gemv
  HIPCHK(launch_fill_zero_u32(reinterpret_cast<uint32_t*>(ws + L.cnt), (size_t)((rows + RG - 1) / RG), S(stream)));
  return run_gemv(qtype, packed_dev, rows, cols, batch, x_dev, y_dev, ws, L, S(stream));
}

// ------------------------------------------------ mixers on caller buffers

int slq_read_probe(const void* buf_dev, size_t bytes, uint32_t* sink_dev, void* stream) {
  if (!buf_dev || !sink_dev) return fail(SLICE_EINVAL, "slq_read_probe: null pointer");
  if (bytes == 0 || bytes % 16) return fail(SLICE_EINVAL, "slq_read_probe: bytes must be a positive multiple of 16");
  HIPCHK(launch_read_probe(buf_dev, bytes / 16, sink_dev, SLQ_READ_PROBE_GRID, S(stream)));
  return SLICE_OK;
}

int slq_dn_state_layout(int heads, int dk, int dv, float* canon_dev, float* lib_dev, int to_lib, void* stream) {
  if (heads <= 0 || dk <= 0 || dk % 32 || dk > 128 || dv <= 0 || dv % 32)
    return fail(SLICE_ESHAPE, "slq_dn_state_layout: heads > 0, dk in {32, 64, 96, 128}, dv a multiple of 32");
  if (!canon_dev || !lib_dev) return fail(SLICE_EINVAL, "slq_dn_state_layout: null pointer");
  HIPCHK(launch_state_io(lib_dev, 1, nullptr, heads, dk, dv, canon_dev, to_lib ? 1 : 0, S(stream)));
  return SLICE_OK;
}

int slq_dn_step(int heads, int dk, int dv, int T, const float* in_dev, float* state_dev, float* out_dev,
                void* stream) {
  if (heads <= 0 || dk <= 0 || dk % 32 || dk > 128 || dv <= 0 || dv % 32)
    return fail(SLICE_ESHAPE, "slq_dn_step: heads > 0, dk in {32, 64, 96, 128}, dv a multiple of 32");
  if (T < 1 || T > MAX_T) return fail(SLICE_ERANGE, "slq_dn_step: T outside 1..16");
  if (!in_dev || !state_dev || !out_dev) return fail(SLICE_EINVAL, "slq_dn_step: null pointer");
  DnParams p{};
  p.y = in_dev;
  p.off_q = 0;
  p.off_k = heads * dk;
  p.off_v = 2 * heads * dk;
  p.off_a = p.off_v + heads * dv;
  p.off_b = p.off_a + heads;
  p.off_z = p.off_b + heads;
  p.y_stride = p.off_z + heads * dv;
  p.heads = heads; p.dk = dk; p.dv = dv;
  p.a_scale = 1.0f; p.a_bias = 0.0f; p.b_scale = 1.0f; p.z_scale = 1.0f;
  p.state = state_dev;
  p.nslots = 1;
  p.mode = DN_DECODE;     // one token after the other, the state updated in place
  p.ctrl = nullptr;
  p.u_out = out_dev;
  HIPCHK(launch_deltanet(p, T, S(stream)));
  return SLICE_OK;
}

size_t slq_attn_workspace_bytes(const slq_attn_desc* d, int T) {
  if (!attn_desc_error(d).empty() || T < 1 || T > MAX_T) return 0;
  const size_t nchunk = (size_t)(d->max_seq + ATT_CHUNK - 1) / ATT_CHUNK;
  return attn_rope_bytes(d) + al256((size_t)T * d->q_heads * nchunk * (d->head_dim + 2) * 4);
}

int slq_attn_prepare(const slq_attn_desc* d, void* ws_dev, size_t ws_bytes, void* stream) {
  const std::string e = attn_desc_error(d);
  if (!e.empty()) return fail(SLICE_ESHAPE, "slq_attn_prepare: " + e);
  if (!ws_dev) return fail(SLICE_EINVAL, "slq_attn_prepare: null workspace");
  if (ws_bytes < attn_rope_bytes(d)) return fail(SLICE_EINVAL, "slq_attn_prepare: workspace too small");
  HIPCHK(launch_rope_table(static_cast<float*>(ws_dev), d->max_seq, d->rope_dims, d->rope_theta, S(stream)));
  return SLICE_OK;
}

int slq_attn_decode(const slq_attn_desc* d, int T, int pos, const float* in_dev, uint16_t* k_cache_dev,
                    uint16_t* v_cache_dev, float* out_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  const std::string e = attn_desc_error(d);
  if (!e.empty()) return fail(SLICE_ESHAPE, "slq_attn_decode: " + e);
  if (T < 1 || T > MAX_T) return fail(SLICE_ERANGE, "slq_attn_decode: T outside 1..16");
  if (pos < 0 || pos + T > d->max_seq) return fail(SLICE_ERANGE, "slq_attn_decode: positions outside the cache");
  if (!in_dev || !k_cache_dev || !v_cache_dev || !out_dev || !ws_dev) return fail(SLICE_EINVAL, "slq_attn_decode: null pointer");
  if (ws_bytes < slq_attn_workspace_bytes(d, T)) return fail(SLICE_EINVAL, "slq_attn_decode: workspace too small");
  const int nq = d->q_heads * d->head_dim, nkv = d->kv_heads * d->head_dim;
  AttnParams p{};
  p.y = in_dev;
  p.off_q = 0;
  p.off_g = d->has_gate ? nq : -1;
  p.off_k = d->has_gate ? 2 * nq : nq;
  p.off_v = p.off_k + nkv;
  p.y_stride = p.off_v + nkv;
  p.q_heads = d->q_heads; p.kv_heads = d->kv_heads; p.hd = d->head_dim; p.rope_dims = d->rope_dims;
  p.rope_theta = d->rope_theta;
  p.rope_cs = static_cast<const float*>(ws_dev);
  p.qk_norm = d->qk_norm;
  p.q_norm = d->q_norm_dev;
  p.k_norm = d->k_norm_dev;
  p.eps = d->eps;
  p.kc = reinterpret_cast<__half*>(k_cache_dev);
  p.vc = reinterpret_cast<__half*>(v_cache_dev);
  p.max_seq = d->max_seq;
  p.ctrl = nullptr;
  p.pos = pos;
  p.part = reinterpret_cast<float*>(static_cast<uint8_t*>(ws_dev) + attn_rope_bytes(d));
  p.nchunk = (d->max_seq + ATT_CHUNK - 1) / ATT_CHUNK;
  p.u_out = out_dev;
  HIPCHK(launch_attention(p, T, S(stream)));
  return SLICE_OK;
}

int slq_kv_layout(int kv_heads, int max_seq, int head_dim, int rows, uint16_t* k_canon_dev, uint16_t* v_canon_dev,
                  uint16_t* k_cache_dev, uint16_t* v_cache_dev, int to_cache, void* stream) {
  if (kv_heads <= 0 || head_dim <= 0 || head_dim % 64 || head_dim > 256 || max_seq <= 0 || max_seq % 64)
    return fail(SLICE_ESHAPE, "slq_kv_layout: bad kv_heads, head_dim or max_seq");
  if (rows < 0 || rows > max_seq) return fail(SLICE_ERANGE, "slq_kv_layout: rows outside 0..max_seq");
  if (!k_canon_dev || !v_canon_dev || !k_cache_dev || !v_cache_dev) return fail(SLICE_EINVAL, "slq_kv_layout: null pointer");
  HIPCHK(launch_kv_io(reinterpret_cast<__half*>(k_cache_dev), reinterpret_cast<__half*>(v_cache_dev), kv_heads, max_seq,
                      head_dim, k_canon_dev, v_canon_dev, rows, to_cache ? 1 : 0, S(stream)));
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
  s->eager = override_int("EAGER", 0) != 0;
  s->mx_min_t = mfma_min_tokens();
  hipError_t he = hipMemsetAsync(s->w, 0, s->L.wbytes, S(stream));
  if (he == hipSuccess) he = hipMemsetAsync(s->ws, 0, s->L.wsbytes, S(stream));
  if (he == hipSuccess && s->L.n_attn && cfg->rope_dims > 0)
    he = launch_rope_table(s->wsp<float>(s->L.rope), cfg->max_seq, cfg->rope_dims, cfg->rope_theta, S(stream));
  s->chain = chains_possible(s) && override_int("CHAIN", 1) != 0;
  // the qwen3_5 form's update takes a workgroup per head, too wide for the chain
  s->chain_dn = s->chain && !cfg->dn_variant && override_int("CHAIN_DN", 1) != 0;
  // the chained merge takes one token's partials of single chunks, at most 64
  s->chain_g1_first = s->chain_dn && !s->L.layers.empty() && !s->L.layers[0].attn &&
                      override_int("CHAIN_G1", 1) != 0;
  s->chain_att = s->chain && s->L.n_attn > 0 && s->L.nchunk <= 64 && (int64_t)cfg->kv_heads * s->L.nchunk <= 1024 &&
                 override_int("CHAIN_ATT", 1) != 0;
  if (s->chain) build_chains(s);
  if (he == hipSuccess) he = hipStreamCreate(&s->cap);
  if (he != hipSuccess) {
    delete s;
    return fail(SLICE_EHIP, std::string("slice_load: ") + hipGetErrorString(he));
  }
  *out = s;
  return SLICE_OK;
}

int slice_tensor_info(const slice_config* cfg, int layer, int tid, int64_t* rows, int64_t* cols, int32_t* kind,
                      size_t* src_bytes) {
  if (!cfg) return fail(SLICE_EINVAL, "slice_tensor_info: null config");
  std::string e = validate(*cfg);
  if (!e.empty()) return fail(SLICE_EINVAL, e);
  int64_t r = 0, c = 0;
  int k = 0;
  e = tensor_shape(*cfg, layer, tid, r, c, k);
  if (!e.empty()) return fail(SLICE_EINVAL, "slice_tensor_info: " + e);
  if (rows) *rows = r;
  if (cols) *cols = c;
  if (kind) *kind = k;
  if (src_bytes) *src_bytes = tensor_src_bytes(r, c, k);
  return SLICE_OK;
}

int slice_set_tensor(slice_t* s, int layer, int tid, const void* src, size_t src_bytes, void* stream) {
  if (!s || !src) return fail(SLICE_EINVAL, "slice_set_tensor: null argument");
  {
    int64_t r = 0, cc = 0;
    int k = 0;
    const std::string e = tensor_shape(s->cfg, layer, tid, r, cc, k);
    if (!e.empty()) return fail(SLICE_EINVAL, "slice_set_tensor: " + e);
    const size_t need = tensor_src_bytes(r, cc, k);
    if (src_bytes != need)
      return fail(SLICE_ESHAPE, "slice_set_tensor: tensor " + std::to_string(tid) + " of layer " + std::to_string(layer) +
                                    " needs " + std::to_string(need) + " source bytes (" + std::to_string(r) + " x " +
                                    std::to_string(cc) + (k ? " blocks" : " fp32") + "), got " + std::to_string(src_bytes));
  }
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
  if (tid == SLICE_T_MTP_FC) return repack(L.mtp_fc, c.hidden, 2 * (int64_t)c.hidden, 0, 0);
  if (tid == SLICE_T_MTP_NORM_E) return copyv(L.mtp_ne, c.hidden);
  if (tid == SLICE_T_MTP_NORM_H) return copyv(L.mtp_nh, c.hidden);
  if (layer < c.layer_begin || layer >= c.layer_end) return fail(SLICE_ERANGE, "slice_set_tensor: layer outside the slice");
  const LayerLayout& ll = L.layers[layer - c.layer_begin];
  const int H = c.hidden;
  const int nkd = dn_kh(c) * c.dn_dk, nvd = c.dn_heads * c.dn_dv;
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
    case SLICE_T_DN_CONV: return copyv(ll.dn_conv_w, (int64_t)dn_conv_dim(c) * c.dn_conv);
    case SLICE_T_DN_ALOG: return copyv(ll.dn_alog, c.dn_heads);
    case SLICE_T_DN_DTB: return copyv(ll.dn_dtb, c.dn_heads);
    case SLICE_T_DN_NORM: return copyv(ll.dn_normw, c.dn_dv);
    default: return fail(SLICE_EINVAL, "slice_set_tensor: not a DeltaNet-layer tensor");
  }
}

int slice_reset(slice_t* s, int kv_len, void* stream) {
  if (!s) return fail(SLICE_EINVAL, "null slice");
  if (kv_len < 0 || (s->L.n_attn && kv_len > s->cfg.max_seq)) return fail(SLICE_ERANGE, "kv_len out of range");
  HIPCHK(launch_ctrl_set(s->ctrl(), kv_len, s->cur, S(stream)));
  if (s->chain) {
    HIPCHK(launch_chain_reset(reinterpret_cast<unsigned*>(s->ws + s->L.chain_sync), s->L.chain_sync_bytes / 4,
                              s->ctrl(), S(stream)));
    // split-K tickets of the chained products (zero unless a wait gave up mid-exchange)
    for (int p = 0; p < CHAIN_PART_BUFS; ++p)
      HIPCHK(launch_fill_zero_u32(reinterpret_cast<uint32_t*>(s->ws + s->L.ccnt[p]), s->L.ccnt_n, S(stream)));
  }
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
      op_kind != SLICE_OP_ATT_OUT && op_kind != SLICE_OP_FFN_IN && op_kind != SLICE_OP_FFN_OUT &&
      op_kind != SLICE_OP_CHAIN)
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
  if (k < 1 || k > s->L.mt)
    return fail(SLICE_ERANGE, "slice_prefill: k outside 1..max(max_verify, max_prefill)");
  if (s->L.n_attn && s->pos + k > s->cfg.max_seq) return fail(SLICE_ERANGE, "slice_prefill: positions pass max_seq");
  if (s->cfg.dn_variant && s->L.n_dn) {
    // the qwen3_5 form has no chunked update: a verify pass whose k tokens are all kept
    int rc = run_step(s, k, DN_VERIFY, in, out, S(stream));
    if (rc) return rc;
    const int cur = (s->cur + k) % s->L.nslots;
    HIPCHK(launch_ctrl_set(s->ctrl(), s->pos + k, cur, S(stream)));
    s->cur = cur;
    s->pos += k;
    return SLICE_OK;
  }
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

int slice_mtp_input(slice_t* s, const int32_t* tok, const void* in, void* out, void* stream) {
  if (!s || !tok || !in || !out) return fail(SLICE_EINVAL, "slice_mtp_input: null argument");
  const slice_config& c = s->cfg;
  const Layout& L = s->L;
  if (!c.has_mtp || !L.mtp_fc.present) return fail(SLICE_EINVAL, "slice_mtp_input: slice is not a draft head");
  const hipStream_t st = S(stream);
  const int H = c.hidden;
  const Act x{s->wsp<int32_t>(L.xe_d), s->wsp<float>(L.xe_s), 2 * H / QK, nullptr, 0};
  HIPCHK(launch_mtp_input(s->packed(L.embed), tok, in, c.io_fp32,
                          reinterpret_cast<const float*>(s->w + L.mtp_ne),
                          reinterpret_cast<const float*>(s->w + L.mtp_nh), c.eps, x, st));
  GemvOut o{};
  o.kind = EPI_STORE;
  o.y = c.io_fp32 ? static_cast<float*>(out) : s->wsp<float>(L.mtp_y);
  o.y_tstride = H;
  o.part = s->wsp<float>(L.part);
  o.cnt = s->wsp<unsigned>(L.cnt);
  HIPCHK(launch_gemv(s->packed(L.mtp_fc), 1, x, NormIn{nullptr, 0, 0.0f, 0.0f}, o, L.pmtp.ks, L.pmtp.w, st));
  if (!c.io_fp32) HIPCHK(launch_store_out(s->wsp<float>(L.mtp_y), 1, H, out, 0, s->ctrl(), 0, st));
  return SLICE_OK;
}

int slice_position(const slice_t* s) { return s ? s->pos : -1; }

int slice_sync_check(slice_t* s, void* stream) {
  if (!s) return fail(SLICE_EINVAL, "null slice");
  HIPCHK(hipStreamSynchronize(S(stream)));
  int err = 0;
  HIPCHK(hipMemcpy(&err, &s->ctrl()->err, sizeof(int), hipMemcpyDeviceToHost));
  if (err)
    return fail(SLICE_EHIP, "a bounded wait between chained products gave up; outputs since the last "
                            "slice_reset are invalid (slice_reset clears the condition)");
  return SLICE_OK;
}

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

static int conv_io(slice_t* s, int layer, float* buf, int to_device, void* stream) {
  if (!s || !buf) return fail(SLICE_EINVAL, "null argument");
  const slice_config& c = s->cfg;
  if (layer < c.layer_begin || layer >= c.layer_end) return fail(SLICE_ERANGE, "layer outside the slice");
  const LayerLayout& ll = s->L.layers[layer - c.layer_begin];
  if (ll.attn || !c.dn_variant) return fail(SLICE_EINVAL, "not a DeltaNet layer of the qwen3_5 form");
  // canonical [conv_dim][conv - 1] (q | k | v channels) <-> the slot's
  // [head][q of its key head | k of its key head | its v][conv - 1]
  float* slot = reinterpret_cast<float*>(s->ws + s->L.conv + (size_t)ll.dn_index * s->L.conv_layer_bytes) +
                (size_t)s->cur * s->L.conv_slot;
  const int kh = dn_kh(c), ratio = c.dn_heads / kh, w = c.dn_conv - 1, dk = c.dn_dk, dv = c.dn_dv;
  const size_t per_head = (size_t)(2 * dk + dv) * w;
  auto mv = [&](size_t canon_off, size_t dev_off, size_t n) -> int {
    float* a = buf + canon_off * w;
    float* b = slot + dev_off;
    HIPCHK(hipMemcpyAsync(to_device ? b : a, to_device ? a : b, n * w * 4, hipMemcpyDeviceToDevice, S(stream)));
    return SLICE_OK;
  };
  for (int h = 0; h < c.dn_heads; ++h) {
    const int g = h / ratio;
    const size_t base = (size_t)h * per_head;
    int rc = SLICE_OK;
    if (to_device || h % ratio == 0) {   // the copies of a key head's windows are identical
      rc = mv((size_t)g * dk, base, dk);
      if (!rc) rc = mv((size_t)kh * dk + (size_t)g * dk, base + (size_t)dk * w, dk);
    }
    if (!rc) rc = mv((size_t)2 * kh * dk + (size_t)h * dv, base + (size_t)2 * dk * w, dv);
    if (rc) return rc;
  }
  return SLICE_OK;
}

int slice_dbg_set_conv(slice_t* s, int layer, const float* src, void* stream) {
  return conv_io(s, layer, const_cast<float*>(src), 1, stream);
}

int slice_dbg_get_conv(slice_t* s, int layer, float* dst, void* stream) { return conv_io(s, layer, dst, 0, stream); }

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
  if (k < 1 || k > s->L.mt) return fail(SLICE_ERANGE, "k outside 1..max(max_verify, max_prefill)");
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
