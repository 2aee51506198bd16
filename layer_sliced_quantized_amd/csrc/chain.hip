// Chained single-token GEMVs: several dependent products of one decode step
// in one kernel.
//
// A decode step reads every weight once (SwarmLLM README, engine paragraph),
// and the products of a layer depend on each other one after the other:
// the mixer output projection updates h, the gate/up projection needs the
// RMSNorm of all of h, the down projection needs all of the SwiGLU output,
// the next layer's input projections all of h again.  As separate kernels,
// each product pays a launch, a ramp-up before its first weights arrive, and
// a tail (the last tiles, the split-K exchange, the epilogue) during which
// the memory system idles.  Here the workgroups of product p + 1 start while
// product p is still running: they request their first weight tiles at once,
// wait for product p to finish, then run the same arithmetic as the separate
// kernel (k_gemv), so results are the same bit for bit.
//
// Forward progress.  The workgroups of product 0 come first in index order,
// then those of product 1, and so on, and a workgroup of product p waits only
// for product p - 1.  The hardware hands a launch's workgroups to the XCDs in
// turn and each XCD starts its share in index order, so when a workgroup of
// product p is running, every workgroup of product p - 1 on its own XCD has
// started, and on every other XCD the ones not yet started come before any of
// product p there; by induction over the products the launch always drains.
// Every wait is also bounded: past CHAIN_SPIN_LIMIT polls (about a second) it
// sets ctrl->err and the workgroup leaves, as do the workgroups that then find
// ctrl->err set, so the kernel always ends, and slice_sync_check reports it.
// (A single ticket counter taken by every workgroup would not need the
// dispatch order, but its atomics, serialised on one address, cost more than
// the chaining saves.)
//
// Launches.  The counters are never reset between launches: launch k (from 1)
// waits for product p - 1's ready flag to reach k and the count of finished
// row groups to reach k times the row groups.  Each workgroup reads k - 1 from
// the last product's ready flag when it starts: that flag moves to k only once
// the last product is complete, which needs every workgroup of the launch to
// have run.
//
// Visibility.  Whatever a product hands to a later one inside the kernel
// (the residual h, the RMSNorm partial sums, the activation digits, split-K
// partials, the input projections a DeltaNet update reads) is stored with
// agent-scope atomic stores (global stores with sc1 on gfx950, written
// through to the level that every XCD reads), and h, the partial sums and
// the update's inputs are read back with agent-scope atomic loads.  The last
// workgroup of each row group waits for its stores to complete (vmcnt 0)
// before it counts the row group as finished; the workgroup that finishes
// the product's last row group then sets the product's ready flags.  The
// digits are read by scalar loads; each digit buffer is written once per
// kernel (every layer of a launch has its own) and read only after its ready
// flag, so no cache of the reading XCD can hold an older copy of it from this
// kernel, and the kernel boundary drops copies from earlier kernels.
#include "gemv_kernel.h"
#include "deltanet.h"
#include "attn_merge.h"

namespace slq {

constexpr unsigned CHAIN_SPIN_LIMIT = 1u << 20;

constexpr int CHAIN_COPIES = 64;   // copies of each ready flag (pollers spread over 64 lines)
constexpr int CHAIN_GROUPS = 32;   // completion groups per product
static_assert(CHAIN_PHASE_LINES == CHAIN_GROUPS + 1 + CHAIN_COPIES, "sync lines per phase");
// kernel arguments are passed in a 4 KiB segment
static_assert(sizeof(ChainArgs) <= 4096, "chain launch arguments");
__device__ __forceinline__ unsigned* chain_count(unsigned* sync, int p, int g) {
  return sync + 32 * (CHAIN_PHASE_LINES * p + g);
}
__device__ __forceinline__ unsigned* chain_ready(unsigned* sync, int p, int c) {
  return sync + 32 * (CHAIN_PHASE_LINES * p + CHAIN_GROUPS + 1 + c);
}

// Poll one copy of a ready flag until it reaches `epoch` (wrap-safe compare).
// Returns false when the wait gives up (ctrl->err set here or elsewhere).
__device__ __forceinline__ bool chain_wait(const unsigned* flag, unsigned epoch, Ctrl* ctrl) {
  unsigned n = 0;
  while ((int)(__hip_atomic_load(const_cast<unsigned*>(flag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - epoch) < 0) {
    __builtin_amdgcn_s_sleep(2);
    if ((++n & 31) == 0) {
      if (__hip_atomic_load(&ctrl->err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return false;
      if (n >= CHAIN_SPIN_LIMIT) {
        __hip_atomic_store(&ctrl->err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
      }
    }
  }
  return true;
}

// Row group rg of product p is done (wave 0, after its stores completed).
// Row groups count in groups of gsize (one counter line each); the workgroup
// that completes a group counts it on the product's line, and the one that
// completes the last group sets the product's ready flags, so that no counter
// line takes more than about 32 increments per launch.
__device__ __forceinline__ void chain_complete(int p, int rg, int nrg, int gsize, unsigned* sync,
                                               const unsigned& epoch_v, int lane) {
  const unsigned epoch = __builtin_amdgcn_readfirstlane(epoch_v);
  const int g = rg / gsize;
  const int ngroups = (nrg + gsize - 1) / gsize;
  const unsigned in_group = (unsigned)min(gsize, nrg - g * gsize);
  unsigned old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(chain_count(sync, p, g), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __builtin_amdgcn_readfirstlane(old);   // the whole wave is active here: lane 0's value
  if (old + 1u != epoch * in_group) return;
  if (lane == 0)
    old = __hip_atomic_fetch_add(chain_count(sync, p, CHAIN_GROUPS), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __builtin_amdgcn_readfirstlane(old);
  // the workgroup that completes the product sets its ready flags, one copy per lane
  if (old + 1u == epoch * (unsigned)ngroups)
    __hip_atomic_store(chain_ready(sync, p, lane % CHAIN_COPIES), epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The restrict-qualified bases tell the compiler which memory this workgroup
// only reads; every pointer is formed from a base and a descriptor offset.
template <int QT, int EPI>
__device__ __forceinline__ void chain_phase(const ChainPhase& ph, int p, int id, int gsize,
                                            const uint8_t* __restrict__ wts, const uint8_t* __restrict__ dig,
                                            uint8_t* __restrict__ ws, unsigned* __restrict__ sync,
                                            Ctrl* __restrict__ ctrl, const unsigned& epoch_v, float (*red)[RG],
                                            int* s_ok) {
  constexpr int TBY = tile_bytes(QT);
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  // the product's own wave count (the separate kernel's launch shape); waves
  // past it have no tiles and only take part in the barriers
  const int nw = ph.w;
  const Packed W{wts + ph.w_off, ph.rows, ph.cols, QT};
  const int ksplit = ph.ksplit;
  const int rg = id / ksplit, ks = id % ksplit;
  const int nblk = W.nblk(), ntiles = W.ntiles(), full = nblk / TB;
  int t0 = 0, t1 = 0;
  if (wave < nw) wave_tiles(ntiles, ks, ksplit, wave, nw, t0, t1);
  const uint8_t* base = W.w + (size_t)rg * rg_bytes(QT, W.cols);
  const int te = t1 < full ? t1 : full;

  // the first tile is requested before the wait: weights depend on nothing.
  // (Two tiles per wave in flight would put so many bytes in the memory
  // queues that the previous product's synchronisation round trips, queued
  // behind them, would slow down more than the prefetch gains.)
  TileRegs<QT> A, B;
  if (t0 < te) load_tile<QT>(base + (size_t)t0 * TBY, lane, TB, A);

  if (p > 0) {
    if (threadIdx.x == 0)
      *s_ok = chain_wait(chain_ready(sync, p - 1, blockIdx.x % CHAIN_COPIES),
                         __builtin_amdgcn_readfirstlane(epoch_v), ctrl) ? 1 : 0;
    __syncthreads();
    if (!*s_ok) return;
  }

  // the residual rows this row group updates: final once the product is
  // released (the earlier products that wrote them are complete), so they are
  // requested now rather than in the epilogue
  float hprev = 0.0f;
  if constexpr (EPI == EPI_RESID) {
    const int64_t row = (int64_t)rg * RG + lane;
    if (wave == 0 && row < W.rows) hprev = ld_<true>(reinterpret_cast<const float*>(ws + ph.y_off) + row);
  }

  // When a product is released every wave's first weights are already in
  // registers, so the digits are what it waits for, and the scalar loads in
  // tile_math ask for them one block ahead.  The workgroup first pulls its
  // split's whole digit range [kb0, kb1) into L2 with one batch of vector
  // loads (one memory round trip), so those scalar loads hit L2.
  {
    const int kb0 = (ntiles * ks / ksplit) * TB;
    const int kb1 = min((ntiles * (ks + 1) / ksplit) * TB, nblk);
    const uint8_t* xb = dig + ph.xd_off + (size_t)kb0 * XW * 4;
    const int nbytes = (kb1 - kb0) * XW * 4;
    unsigned v = 0;
    for (int i = threadIdx.x * 64; i < nbytes; i += blockDim.x * 64) v ^= *reinterpret_cast<const unsigned*>(xb + i);
    const uint8_t* sb = dig + ph.xs_off + (size_t)kb0 * 4;
    if (threadIdx.x * 64 < (kb1 - kb0) * 4) v ^= *reinterpret_cast<const unsigned*>(sb + threadIdx.x * 64);
    red[4][threadIdx.x & 63] = __uint_as_float(v);   // keeps the loads; the slot is rewritten before it is read
  }
  const NormIn nin{ph.ssq_off >= 0 ? reinterpret_cast<const float*>(ws + ph.ssq_off) : nullptr, ph.n_part, ph.inv_n,
                   ph.eps};
  float acc[1] = {0.0f};
  RnRaw rr = (EPI != EPI_RESID && wave == 0) ? rnorm_fetch<true>(nin, 0) : RnRaw{0.0f, 0.0f};
  const Act x{const_cast<int32_t*>(reinterpret_cast<const int32_t*>(dig + ph.xd_off)),
              const_cast<float*>(reinterpret_cast<const float*>(dig + ph.xs_off)), ph.x_nblk, nullptr, 0};
  for (int t = t0; t < te; t += 2) {
    if (t + 1 < te) load_tile<QT>(base + (size_t)(t + 1) * TBY, lane, TB, B);
    tile_math<QT, 1>(A, TB, t * TB, x, acc);
    if (t + 1 < te) {
      if (t + 2 < te) load_tile<QT>(base + (size_t)(t + 2) * TBY, lane, TB, A);
      tile_math<QT, 1>(B, TB, (t + 1) * TB, x, acc);
    }
  }
  if (t1 > full) {
    const int nb = nblk - full * TB;
    TileRegs<QT> R;
    load_tile<QT>(base + (size_t)full * TBY, lane, nb, R);
    tile_math<QT, 1>(R, nb, full * TB, x, acc);
  }
  float rn[1] = {(EPI != EPI_RESID && wave == 0) ? rnorm_finish(rr, nin, 0) : 1.0f};

  reduce_waves<1>(acc, red, wave, nw, lane);
  if (wave != 0) return;
  GemvOut out{};
  out.kind = EPI;
  out.y = ph.y_off >= 0 ? reinterpret_cast<float*>(ws + ph.y_off) : nullptr;
  out.y_tstride = ph.y_tstride;
  out.next = Act{ph.nd_off >= 0 ? reinterpret_cast<int32_t*>(ws + ph.nd_off) : nullptr,
                 ph.ns_off >= 0 ? reinterpret_cast<float*>(ws + ph.ns_off) : nullptr, ph.n_nblk, nullptr, 0};
  out.next_qt = QT;
  out.ssq_out = ph.ssq_out_off >= 0 ? reinterpret_cast<float*>(ws + ph.ssq_out_off) : nullptr;
  out.norm_w = ph.norm_w_off >= 0 ? reinterpret_cast<const float*>(wts + ph.norm_w_off) : nullptr;
  out.part = reinterpret_cast<float*>(ws + ph.part_off);
  out.cnt = reinterpret_cast<unsigned*>(ws + ph.cnt_off);
  if (ksplit > 1 && !split_exchange<1>(acc, out, rg, ks, ksplit, lane)) return;
  if constexpr (EPI == EPI_RESID) {
    // gemv_epilogue's residual update, with the rows read earlier
    const bool rv = (int64_t)rg * RG + lane < W.rows;
    resid_tail<true>(0, rg, (int)W.rows, rv ? hprev + acc[0] : 0.0f, out.y, out.y_tstride, out.norm_w, out.next_qt,
                     out.next, out.ssq_out, W.nrg());
  } else {
    gemv_epilogue<QT, 1, EPI, true>(acc, rn, W, out, rg, lane);
  }

  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  chain_complete(p, rg, (int)W.nrg(), gsize, sync, epoch_v, lane);
}

// The wait of a DeltaNet update that follows another phase: thread 0 polls
// the phase before's ready flag, and the workgroup learns the outcome at a
// barrier.
struct ChainWait {
  static constexpr bool active = true;
  const unsigned* flag;
  unsigned epoch;
  Ctrl* ctrl;
  int* s_ok;
  __device__ bool operator()() const {
    if (threadIdx.x == 0) *s_ok = chain_wait(flag, epoch, ctrl) ? 1 : 0;
    __syncthreads();
    return *s_ok != 0;
  }
};

// A DeltaNet layer's recurrent update (one decode token): the separate
// kernel's workgroup body, with the output digits stored coherently for the
// mixer output projection that follows in this kernel.  As the launch's
// first phase it reads inputs written before the launch; after another phase
// (the layer's input projections, earlier in the same launch) it requests
// its state rows, waits for that phase, then reads the inputs coherently.
// Each workgroup (a head's 32 state rows) counts as one row group once the
// stores of all its waves have completed.
template <int DKP>
__device__ __forceinline__ void chain_dn_phase(const ChainArgs& args, int p, int id, unsigned* __restrict__ sync,
                                               Ctrl* __restrict__ ctrl, uint8_t* __restrict__ ws,
                                               const unsigned& epoch_v, int* s_ok) {
  const ChainPhase& ph = args.ph[p];
  DnParams dn = args.dn;
  dn.state = reinterpret_cast<float*>(ws + ph.y_off);
  dn.next.xd = reinterpret_cast<int32_t*>(ws + ph.nd_off);
  dn.next.xs = reinterpret_cast<float*>(ws + ph.ns_off);
  if (p == 0) {
    deltanet_rows<DKP, 1, true>(dn, 1, id);
  } else {
    const ChainWait w{chain_ready(sync, p - 1, blockIdx.x % CHAIN_COPIES), (unsigned)__builtin_amdgcn_readfirstlane(epoch_v),
                      ctrl, s_ok};
    if (!deltanet_rows<DKP, 1, true>(dn, 1, id, w)) return;
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (wave_id() != 0) return;
  chain_complete(p, id, args.ph[p].nwg, args.gsize[p], sync, epoch_v, (int)(threadIdx.x & 63));
}

// An attention layer's merge (one decode token) as the first phase of the
// launch after its split kernel: wave w of workgroup id merges (head, 64 dims)
// number 4 id + w over the partials the token reaches (merge_wave, as the
// combine kernel does; the partials and the gate input were written before
// the launch), the output digits stored coherently for the mixer output
// projection that follows.  Each workgroup counts as one row group.
__device__ __forceinline__ void chain_att_merge_phase(const ChainArgs& args, int p, int id, uint8_t* __restrict__ ws,
                                                      unsigned* __restrict__ sync, const unsigned& epoch_v,
                                                      float (*red)[RG]) {
  const ChainPhase& ph = args.ph[p];
  AttnParams a = args.att;
  a.next.xd = reinterpret_cast<int32_t*>(ws + ph.nd_off);
  a.next.xs = reinterpret_cast<float*>(ws + ph.ns_off);
  const int wave = wave_id();
  const int ndg = a.hd / 64;
  const int job = 4 * id + wave;
  const int pos = (a.ctrl ? a.ctrl->pos : a.pos) + a.pos_off;
  if (job < a.q_heads * ndg) merge_wave<true>(a, 0, job / ndg, (job % ndg) * 64, pos / ATT_CHUNK + 1, red[wave]);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (wave != 0) return;
  chain_complete(p, id, ph.nwg, args.gsize[p], sync, epoch_v, (int)(threadIdx.x & 63));
}

template <int QT>
__global__ __launch_bounds__(256) void k_chain(const ChainArgs args, const uint8_t* __restrict__ wts,
                                               const uint8_t* __restrict__ dig, uint8_t* __restrict__ ws,
                                               unsigned* __restrict__ sync, Ctrl* __restrict__ ctrl) {
  __shared__ float red[8][RG];
  __shared__ int s_ok;
  // this launch's number: one more than the last product's ready flag (read
  // now, used only at the first wait or the publication, so its latency is
  // not in front of the first weight requests)
  const unsigned epoch_v =
      __hip_atomic_load(chain_ready(sync, args.nph - 1, blockIdx.x % CHAIN_COPIES), __ATOMIC_RELAXED,
                        __HIP_MEMORY_SCOPE_AGENT) + 1u;
  const int b = (int)blockIdx.x;
  int p = 0;
  while (p + 1 < args.nph && b >= args.first_wg[p + 1]) ++p;
  const int id = b - args.first_wg[p];
  switch (args.ph[p].epi) {
    case EPI_DN:
      switch (args.dn_dkp) {
        case 4: chain_dn_phase<4>(args, p, id, sync, ctrl, ws, epoch_v, &s_ok); break;
        case 8: chain_dn_phase<8>(args, p, id, sync, ctrl, ws, epoch_v, &s_ok); break;
        case 12: chain_dn_phase<12>(args, p, id, sync, ctrl, ws, epoch_v, &s_ok); break;
        default: chain_dn_phase<16>(args, p, id, sync, ctrl, ws, epoch_v, &s_ok); break;
      }
      break;
    case EPI_ATT_COMB:
      chain_att_merge_phase(args, p, id, ws, sync, epoch_v, red);
      break;
    case EPI_STORE:
      chain_phase<QT, EPI_STORE>(args.ph[p], p, id, args.gsize[p], wts, dig, ws, sync, ctrl, epoch_v, red, &s_ok);
      break;
    case EPI_SWIGLU:
      chain_phase<QT, EPI_SWIGLU>(args.ph[p], p, id, args.gsize[p], wts, dig, ws, sync, ctrl, epoch_v, red, &s_ok);
      break;
    default:
      chain_phase<QT, EPI_RESID>(args.ph[p], p, id, args.gsize[p], wts, dig, ws, sync, ctrl, epoch_v, red, &s_ok);
      break;
  }
}

hipError_t launch_chain(int qt, const ChainArgs& args, unsigned grid, const uint8_t* weights, uint8_t* ws,
                        unsigned* sync, Ctrl* ctrl, hipStream_t s) {
  if (args.nph < 1 || args.nph > CHAIN_MAX_PHASES || grid == 0 || (int)grid != args.first_wg[args.nph])
    return hipErrorInvalidValue;
  // a DeltaNet phase has one workgroup per 32 state rows
  for (int p = 0; p < args.nph; ++p)
    if (args.ph[p].epi == EPI_DN &&
        (args.ph[p].nwg != args.dn.heads * (args.dn.dv / 32) || args.dn.dv % 32 ||
         args.dn.dk != 8 * args.dn_dkp || (args.dn_dkp != 4 && args.dn_dkp != 8 && args.dn_dkp != 12 &&
                                           args.dn_dkp != 16) || args.dn.mode != DN_DECODE))
      return hipErrorInvalidValue;
  // an attention merge comes first (its split ran as the kernel before), one
  // workgroup per four (head, 64 dims), at most 64 partials of one chunk each
  for (int p = 0; p < args.nph; ++p) {
    if (args.ph[p].epi != EPI_ATT_COMB) continue;
    const AttnParams& a = args.att;
    if (p != 0 || a.hd % 64 || a.hd > 256 || a.q_heads <= 0 || a.nchunk > 64 ||
        args.ph[p].nwg != (a.q_heads * (a.hd / 64) + 3) / 4)
      return hipErrorInvalidValue;
  }
  if (qt == QT_Q4) k_chain<QT_Q4><<<grid, 256, 0, s>>>(args, weights, ws, ws, sync, ctrl);
  else k_chain<QT_Q8><<<grid, 256, 0, s>>>(args, weights, ws, ws, sync, ctrl);
  return hipGetLastError();
}

__global__ void k_chain_reset(unsigned* sync, size_t n, Ctrl* ctrl) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) sync[i] = 0u;
  if (blockIdx.x == 0 && threadIdx.x == 0) ctrl->err = 0;
}

hipError_t launch_chain_reset(unsigned* sync, size_t n_u32, Ctrl* ctrl, hipStream_t s) {
  const size_t nb = (n_u32 + 255) / 256;
  k_chain_reset<<<(unsigned)(nb < 1024 ? (nb ? nb : 1) : 1024), 256, 0, s>>>(sync, n_u32, ctrl);
  return hipGetLastError();
}

}  // namespace slq
