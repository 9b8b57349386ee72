// C ABI of libssd: argument validation, workspace layout and dispatch to the
// gfx950 kernels.  Declarations and the contract are in include/ssd.h.
//
// Everything here runs on the host.  Validation is complete before the first
// launch, so an invalid call writes nothing.  No allocation, no
// synchronisation.  The only global state is the per-device address of the
// static scratch that ssd_chunk_scan_noalloc uses, set once per device.
#include "ssd.h"

#include <float.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "ssd_launch.h"

namespace {

constexpr size_t kAlign = 256;

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

inline size_t io_size(int32_t dt) { return dt == SSD_BF16 ? 2 : 4; }

// Checked product of non-negative int64 values; false on overflow.
inline bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

inline Range range_of(const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + (uintptr_t)bytes};
}

inline bool overlap(Range a, Range b) {
  if (a.lo == a.hi || b.lo == b.hi || a.lo == 0 || b.lo == 0) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

inline bool limits_ok(float lo, float hi) { return !isnan(lo) && !isnan(hi) && lo <= hi; }

struct ScanSizes {
  int64_t Nc = 0;
  bool chain = false;
  bool cb_bf16 = false;
  int64_t n_x = 0, n_dt = 0, n_bc = 0, n_state = 0;  // element counts
  size_t ws_state_bytes = 0, ws_alpha_bytes = 0, ws_cb_bytes = 0, ws_bt_bytes = 0, ws_hb_bytes = 0,
         ws_total = 0;
};

// force_phased: size (and run) the phased schedule even where the chain one
// would be chosen (the gradients read the per-chunk states it leaves).
// cb_f32: keep C B^T in float32 with bfloat16 io as well (the gradients read
// it); otherwise the bfloat16 scan holds it in bfloat16.
ssd_status check_scan_desc(const ssd_scan_desc* d, ScanSizes* s, bool force_phased = false,
                           bool cb_f32 = false) {
  if (!d) return SSD_ERR_INVALID_ARG;
  if (d->io_dtype != SSD_F32 && d->io_dtype != SSD_BF16) return SSD_ERR_DTYPE;
  if (d->batch < 0 || d->seqlen < 0 || d->nheads <= 0 || d->headdim <= 0 || d->dstate <= 0 ||
      d->ngroups <= 0 || d->chunk <= 0)
    return SSD_ERR_SHAPE;
  if (d->nheads % d->ngroups != 0) return SSD_ERR_SHAPE;
  if (!limits_ok(d->dt_min, d->dt_max)) return SSD_ERR_INVALID_ARG;
  if (!ssd::scan_shape_supported(d->headdim, d->dstate, d->chunk, d->io_dtype == SSD_BF16))
    return SSD_ERR_UNSUPPORTED;
  const int64_t Nc = (d->seqlen + d->chunk - 1) / d->chunk;
  int64_t bt = 0, bth = 0, bh = 0, pn = 0, tmp = 0;
  if (!mul_ok(d->batch, d->seqlen, &bt) || !mul_ok(bt, d->nheads, &bth) ||
      !mul_ok(bth, d->headdim, &s->n_x) || !mul_ok(bt, d->ngroups, &tmp) ||
      !mul_ok(tmp, d->dstate, &s->n_bc) || !mul_ok(d->batch, d->nheads, &bh) ||
      !mul_ok(d->headdim, d->dstate, &pn) || !mul_ok(bh, pn, &s->n_state))
    return SSD_ERR_UNSUPPORTED;
  s->n_dt = bth;
  s->Nc = Nc;
  int64_t units = 0, ws_elems = 0;
  if (!mul_ok(bh, Nc, &units) || !mul_ok(units, pn, &ws_elems) || !mul_ok(ws_elems, 4, &tmp))
    return SSD_ERR_UNSUPPORTED;
  // one workgroup per (batch, chunk, head): the grid must fit a 32-bit x-dimension
  if (units > INT32_MAX || s->n_x > (INT64_MAX / 8)) return SSD_ERR_UNSUPPORTED;
  int64_t bcg = 0, ll = 0, cb_elems = 0;
  if (!mul_ok(d->batch, Nc, &bcg) || !mul_ok(bcg, d->ngroups, &bcg) ||
      !mul_ok(d->chunk, d->chunk, &ll) || !mul_ok(bcg, ll, &cb_elems) ||
      !mul_ok(cb_elems, 4, &tmp))
    return SSD_ERR_UNSUPPORTED;
  s->chain = !force_phased && ssd::scan_uses_chain(d->batch, d->nheads, d->headdim, d->dstate,
                                                   d->chunk, d->io_dtype == SSD_BF16);
  // the chain schedule keeps states on chip; the phased one needs S_c and alpha_c
  s->ws_state_bytes = s->chain ? 0 : round_up((size_t)ws_elems * 4, kAlign);
  s->ws_alpha_bytes = s->chain ? 0 : round_up((size_t)units * 4, kAlign);
  int64_t bt_elems = 0;
  if (!mul_ok(bcg, d->dstate, &bt_elems) || !mul_ok(bt_elems, d->chunk, &bt_elems) ||
      !mul_ok(bt_elems, 2, &tmp))
    return SSD_ERR_UNSUPPORTED;
  s->cb_bf16 = d->io_dtype == SSD_BF16 && !cb_f32;
  s->ws_cb_bytes = round_up((size_t)cb_elems * (s->cb_bf16 ? 2 : 4), kAlign);
  const bool use_bt = s->chain || (d->io_dtype == SSD_BF16 &&
                                ssd::phased_prepass(d->headdim, d->dstate, d->chunk));
  s->ws_bt_bytes = use_bt ? round_up((size_t)bt_elems * 2, kAlign) : 0;
  // the bfloat16 phased schedule hands the entering states to its output kernel in bf16
  s->ws_hb_bytes = (!s->chain && d->io_dtype == SSD_BF16) ? round_up((size_t)ws_elems * 2, kAlign) : 0;
  s->ws_total = s->ws_state_bytes + s->ws_alpha_bytes + s->ws_cb_bytes + s->ws_bt_bytes +
                s->ws_hb_bytes;
  return SSD_OK;
}

ssd_status scan_impl(const ssd_scan_desc* desc, const void* x, const float* dt,
                     const float* dt_bias, const float* A, const void* B, const void* C,
                     const float* D, const float* initial_state, void* y, float* final_state,
                     void* workspace, size_t workspace_bytes, hipStream_t stream,
                     hipEvent_t* events, int n_events, bool states_only = false,
                     bool force_phased = false, bool keep_f32_states = false,
                     int32_t variant = SSD_VARIANT_DEFAULT) {
  ScanSizes s;
  // a states-only run serves the gradients, which read C B^T in float32
  ssd_status st = check_scan_desc(desc, &s, force_phased, states_only);
  if (st != SSD_OK) return st;
  if (variant != SSD_VARIANT_DEFAULT) {
    if (variant != SSD_VARIANT_BF16_DECAY && variant != SSD_VARIANT_LOADED_MASK)
      return SSD_ERR_INVALID_ARG;
    // compiled for the 130M / 2.7B / 1.3B head shape at chunks up to 256; the
    // loaded-mask variant exists in the bfloat16 output path only
    if (!ssd::ablation_shape(desc->headdim, desc->dstate) || desc->chunk > 256 ||
        (variant == SSD_VARIANT_LOADED_MASK && desc->io_dtype != SSD_BF16))
      return SSD_ERR_UNSUPPORTED;
  }
  // phases 0-2 alone (entering states and C B^T left in the workspace, no y):
  // phased schedule only
  if (states_only && s.chain) return SSD_ERR_UNSUPPORTED;
  if (events) {
    if (n_events < SSD_SCAN_PHASES + 1) return SSD_ERR_INVALID_ARG;
    for (int k = 0; k <= SSD_SCAN_PHASES; ++k)
      if (!events[k]) return SSD_ERR_INVALID_ARG;
  }
  const bool work = desc->batch > 0 && desc->seqlen > 0;
  if (work && (!x || !dt || !A || !B || !C || (!y && !states_only))) return SSD_ERR_INVALID_ARG;
  if (!work && desc->batch > 0 && !A) return SSD_ERR_INVALID_ARG;
  // tensors read or written in 16-byte vectors, and per-token/per-head scalars
  const void* vec[] = {x, B, C, initial_state, y, final_state, workspace};
  for (const void* p : vec)
    if (p && !aligned16(p)) return SSD_ERR_ALIGNMENT;
  const void* scal[] = {dt, dt_bias, A, D};
  for (const void* p : scal)
    if (p && !aligned4(p)) return SSD_ERR_ALIGNMENT;
  if (work && (!workspace || workspace_bytes < s.ws_total)) return SSD_ERR_WORKSPACE;

  // outputs must not overlap any input, the workspace or each other
  const int64_t es = (int64_t)io_size(desc->io_dtype);
  const Range r_y = work && y ? range_of(y, s.n_x * es) : Range{0, 0};
  const Range r_f = final_state ? range_of(final_state, s.n_state * 4) : Range{0, 0};
  const Range ins[] = {
      range_of(x, work ? s.n_x * es : 0), range_of(dt, work ? s.n_dt * 4 : 0),
      range_of(dt_bias, desc->nheads * 4), range_of(A, desc->nheads * 4),
      range_of(B, work ? s.n_bc * es : 0), range_of(C, work ? s.n_bc * es : 0),
      range_of(D, desc->nheads * 4), range_of(initial_state, s.n_state * 4),
      range_of(workspace, work ? (int64_t)s.ws_total : 0)};
  for (const Range& r : ins)
    if (overlap(r_y, r) || overlap(r_f, r)) return SSD_ERR_INVALID_ARG;
  if (overlap(r_y, r_f)) return SSD_ERR_INVALID_ARG;

  if (desc->batch == 0) return SSD_OK;
  if (!work) {
    // empty sequence: the final state is the initial state (or zeros)
    if (final_state) {
      if (events) {
        for (int k = 0; k <= SSD_SCAN_PHASES; ++k)
          if (hipEventRecord(events[k], stream) != hipSuccess) return SSD_ERR_HIP;
      }
      if (ssd::launch_copy_or_zero(final_state, initial_state, s.n_state, stream) != hipSuccess)
        return SSD_ERR_HIP;
    }
    return SSD_OK;
  }

  ssd::ScanArgs a;
  a.x = x; a.dt = dt; a.dt_bias = dt_bias; a.A = A; a.B = B; a.C = C; a.D = D;
  a.h0 = initial_state; a.y = y; a.final_state = final_state;
  a.ws_state = static_cast<float*>(workspace);
  a.ws_alpha = reinterpret_cast<float*>(static_cast<char*>(workspace) + s.ws_state_bytes);
  a.ws_cb = reinterpret_cast<float*>(static_cast<char*>(workspace) + s.ws_state_bytes +
                                     s.ws_alpha_bytes);
  a.ws_bt = static_cast<char*>(workspace) + s.ws_state_bytes + s.ws_alpha_bytes + s.ws_cb_bytes;
  a.ws_hb = static_cast<char*>(a.ws_bt) + s.ws_bt_bytes;
  a.Bt = desc->batch; a.T = desc->seqlen; a.H = desc->nheads; a.G = desc->ngroups;
  a.L = desc->chunk; a.Nc = s.Nc;
  a.softplus = desc->dt_softplus ? 1 : 0;
  a.dt_min = desc->dt_min; a.dt_max = desc->dt_max;
  a.chain = s.chain ? 1 : 0;
  a.states_only = states_only ? 1 : 0;
  a.keep_f32_states = keep_f32_states ? 1 : 0;
  a.variant = variant;
  a.cb_bf16 = s.cb_bf16 ? 1 : 0;
  hipError_t e = desc->io_dtype == SSD_BF16
                     ? ssd::launch_scan_bf16(a, (int)desc->headdim, (int)desc->dstate, stream, events)
                     : ssd::launch_scan_f32(a, (int)desc->headdim, (int)desc->dstate, stream, events);
  return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

}  // namespace

namespace ssd {
bool scan_shape_supported(int64_t P, int64_t N, int64_t L, bool bf16) {
  // bfloat16 matrix-core steps contract 32 state elements at a time
  const bool pn = (P == 16 || P == 32 || P == 64 || P == 128) &&
                  ((N == 16 && !bf16) || N == 32 || N == 64 || N == 128);
  return pn && L >= 32 && L <= 512 && L % 32 == 0 && P * L <= 32768;
}

bool scan_uses_chain(int64_t batch, int64_t nheads, int64_t P, int64_t N, int64_t L, bool bf16) {
  return bf16 && chain_variant(P, N) && L <= 256 && batch * nheads >= kChainMinChains;
}
}  // namespace ssd

namespace {

struct ConvSizes {
  int64_t n_x = 0, n_state = 0, n_w = 0, es = 4;
};

ssd_status check_conv_desc(const ssd_conv_desc* d, bool step, ConvSizes* s) {
  if (!d) return SSD_ERR_INVALID_ARG;
  if (d->io_dtype != SSD_F32 && d->io_dtype != SSD_BF16) return SSD_ERR_DTYPE;
  const int64_t T = step ? 1 : d->seqlen;
  if (d->batch < 0 || T < 0 || d->channels <= 0 || d->width <= 0) return SSD_ERR_SHAPE;
  if (!ssd::conv_width_supported(d->width)) return SSD_ERR_UNSUPPORTED;
  int64_t bt = 0, bd = 0;
  if (!mul_ok(d->batch, T, &bt) || !mul_ok(bt, d->channels, &s->n_x) ||
      !mul_ok(d->batch, d->channels, &bd) || !mul_ok(bd, d->width - 1, &s->n_state) ||
      !mul_ok(d->channels, d->width, &s->n_w))
    return SSD_ERR_UNSUPPORTED;
  if (!ssd::conv_shape_supported(d->batch, T, d->channels)) return SSD_ERR_UNSUPPORTED;
  s->es = (int64_t)io_size(d->io_dtype);
  return SSD_OK;
}

ssd::ConvArgs conv_args(const ssd_conv_desc* d, int64_t T) {
  ssd::ConvArgs a;
  a.Bt = d->batch; a.T = T; a.D = d->channels;
  a.K = (int32_t)d->width;
  a.silu = d->silu ? 1 : 0;
  return a;
}

}  // namespace

namespace {

// ---------------------------------------------------------------------------
// Backward pass: descriptors of the three internal scans and the workspace.
// ---------------------------------------------------------------------------
enum BwdRegion {
  kScanWs, kScanWsR1, kWd, kCum, kRscale, kDtr1, kR1x, kR1b, kR1c, kR1h0, kR1y, kR1final, kMix, kQrow,
  kQcol, kUv, kDbcPart, kDdin, kDdp, kPart, kNumRegions
};

struct BwdPlan {
  ssd_scan_desc fw, r1;        // forward state scan and reversed scan R1 (io type, phased)
  size_t scan_ws = 0;          // F0's workspace (entering states, decays, C B^T)
  size_t scan_ws_r1 = 0;       // R1's own (its entering states are read with F0's)
  size_t fwd_cb_off = 0;       // offset of C B^T in F0's workspace (after states and decays)
  int64_t pad = 0;             // empty leading positions of R1
  int32_t NB = 0, LP = 0, HS = 1, hpw = 1, HSD = 1, hpwd = 1, NS = 1;
  size_t off[kNumRegions] = {0};
  size_t total = 0;
};

// Splits of a group's heads over workgroups: enough workgroups to fill the
// device (`target`), each with at least one head.
// Heads of a group dealt to `splits` workgroups of `per` heads each: as many
// splits as fit in one round of `slots` resident workgroups (so that no
// second, nearly empty round follows), one split when the units alone fill
// the round.
inline void head_split_round(int64_t hpg, int64_t units, int64_t slots, int32_t* splits,
                             int32_t* per) {
  int64_t want = units > 0 ? slots / units : 1;
  if (want < 1) want = 1;
  if (want > hpg) want = hpg;
  const int64_t p = (hpg + want - 1) / want;
  *per = (int32_t)p;
  *splits = (int32_t)((hpg + p - 1) / p);
}

ssd_status plan_backward(const ssd_scan_desc* d, BwdPlan* pl) {
  ScanSizes s0, s1, sf;
  ssd_status st = check_scan_desc(d, &s0);
  if (st != SSD_OK) return st;
  // the kernels of the gradient stage one chunk per workgroup of 256 threads
  // and index (batch, token, head) rows in 32 bits
  if (d->chunk > 256 || s0.n_dt > (int64_t)INT32_MAX) return SSD_ERR_UNSUPPORTED;
  // both scans run the phased schedule of the io type and keep float32
  // entering states in their workspaces
  pl->fw = *d;
  const int64_t Nc = (d->seqlen + d->chunk - 1) / d->chunk;
  pl->pad = Nc * d->chunk - d->seqlen;
  // R1 reads Delta' directly: no softplus, no bias, no clip
  pl->r1 = pl->fw;
  pl->r1.seqlen = d->seqlen + pl->pad;
  pl->r1.dt_softplus = 0;
  pl->r1.dt_min = 0.0f;
  pl->r1.dt_max = FLT_MAX;
  if ((st = check_scan_desc(&pl->fw, &sf, true, true)) != SSD_OK) return st;
  if ((st = check_scan_desc(&pl->r1, &s1, true)) != SSD_OK) return st;
  pl->scan_ws = sf.ws_total;
  pl->scan_ws_r1 = s1.ws_total;
  pl->fwd_cb_off = sf.ws_state_bytes + sf.ws_alpha_bytes;

  const int64_t Bt = d->batch, T = d->seqlen, H = d->nheads, G = d->ngroups, N = d->dstate;
  const int64_t hpg = H / G;
  pl->NB = (int32_t)((d->chunk + 63) / 64);
  pl->LP = 64 * pl->NB;
  pl->NS = N > 64 ? (int32_t)(N / 64) : 1;
  const int64_t nbt = (int64_t)pl->NB * (pl->NB + 1) / 2;
  const int64_t bcg = Bt * Nc * G;
  // k_bwd_mix: three resident workgroups per compute unit (of 256) for
  // bfloat16 rows of P <= 64, two otherwise (LDS and registers);
  // k_bwd_dcdb: the same, three workgroups per compute unit at P <= 64
  head_split_round(hpg, bcg * nbt, 256 * ((d->io_dtype == SSD_BF16 && d->headdim <= 64) ? 3 : 2),
                   &pl->HS, &pl->hpw);
  head_split_round(hpg, bcg * 2 * pl->NS * pl->NB, 256 * (d->headdim <= 64 ? 3 : 2), &pl->HSD,
                   &pl->hpwd);

  const size_t es = io_size(d->io_dtype);
  const size_t nst = (size_t)s0.n_state, nbc = (size_t)s0.n_bc;
  const size_t ndt = (size_t)s0.n_dt;
  const size_t nx1 = (size_t)s1.n_x, nbc1 = (size_t)s1.n_bc, ndt1 = (size_t)s1.n_dt;  // R1, padded
  const size_t LP = (size_t)pl->LP, NB = (size_t)pl->NB;
  size_t sizes[kNumRegions];
  sizes[kScanWs] = pl->scan_ws;
  sizes[kScanWsR1] = pl->scan_ws_r1;
  sizes[kWd] = ndt * 4;
  sizes[kCum] = ndt * 8;
  sizes[kRscale] = 2 * ndt * 4;
  sizes[kDtr1] = ndt1 * 4;
  sizes[kR1x] = nx1 * es;
  sizes[kR1b] = nbc1 * es;
  sizes[kR1c] = nbc1 * es;
  sizes[kR1h0] = nst * 4;
  sizes[kR1y] = nx1 * es;
  sizes[kR1final] = nst * 4;
  sizes[kMix] = (size_t)bcg * pl->HS * LP * LP * 4;
  sizes[kQrow] = (size_t)(Bt * Nc * H) * NB * NB * 128 * 4;
  sizes[kQcol] = sizes[kQrow];
  sizes[kUv] = 2 * (size_t)pl->NS * ndt * 4;
  sizes[kDbcPart] = pl->HSD > 1 ? 2 * (size_t)pl->HSD * nbc * 4 : 0;
  sizes[kDdin] = ndt * 4;
  sizes[kDdp] = ndt * 4;
  sizes[kPart] = 4 * (size_t)(Bt * Nc * H) * 4;
  size_t at = 0;
  for (int k = 0; k < kNumRegions; ++k) {
    pl->off[k] = at;
    at += round_up(sizes[k], kAlign);
  }
  pl->total = at;
  return SSD_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// Scratch of ssd_chunk_scan_noalloc: a file-scope device array, one copy per
// GPU (allocated when the library's code object is loaded on it, held until
// the process ends).  Host code never passes `scratch` itself to a kernel (in
// host code the name is only a stand-in for the symbol): its address on a
// device comes from hipGetSymbolAddress, taken once per device with that
// device current and kept below.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)SSD_NOALLOC_MAX_WORKSPACE;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The scratch address on the device `stream` runs on, which must be the
// current device (the symbol's address is taken with its device current).
ssd_status scratch_of_stream(hipStream_t stream, void** out) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return SSD_ERR_HIP;
  if (stream) {
    hipDevice_t sd = -1;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return SSD_ERR_HIP;
    if ((int)sd != cur) return SSD_ERR_INVALID_ARG;
  }
  if (cur < 0 || cur >= kMaxDevices) return SSD_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[cur].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[cur].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SSD_ERR_HIP;
      g_scratch_ptr[cur].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SSD_OK;
}

}  // namespace

extern "C" {

size_t ssd_chunk_scan_workspace_bytes(const ssd_scan_desc* desc) {
  ScanSizes s;
  if (check_scan_desc(desc, &s) != SSD_OK) return 0;
  return s.ws_total;
}

int32_t ssd_chunk_scan_schedule(const ssd_scan_desc* desc) {
  ScanSizes s;
  const ssd_status st = check_scan_desc(desc, &s);
  if (st != SSD_OK) return -(int32_t)st;
  return s.chain ? SSD_SCHEDULE_CHAIN : SSD_SCHEDULE_PHASED;
}

ssd_status ssd_chunk_scan(const ssd_scan_desc* desc, const void* x, const float* dt,
                          const float* dt_bias, const float* A, const void* B, const void* C,
                          const float* D, const float* initial_state, void* y,
                          float* final_state, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  return scan_impl(desc, x, dt, dt_bias, A, B, C, D, initial_state, y, final_state, workspace,
                   workspace_bytes, stream, nullptr, 0);
}

ssd_status ssd_chunk_scan_timed(const ssd_scan_desc* desc, const void* x, const float* dt,
                                const float* dt_bias, const float* A, const void* B,
                                const void* C, const float* D, const float* initial_state,
                                void* y, float* final_state, void* workspace,
                                size_t workspace_bytes, hipStream_t stream,
                                hipEvent_t* phase_events, int n_events) {
  return scan_impl(desc, x, dt, dt_bias, A, B, C, D, initial_state, y, final_state, workspace,
                   workspace_bytes, stream, phase_events, n_events);
}

ssd_status ssd_chunk_scan_ablation(const ssd_scan_desc* desc, int32_t variant, const void* x,
                                   const float* dt, const float* dt_bias, const float* A,
                                   const void* B, const void* C, const float* D,
                                   const float* initial_state, void* y, float* final_state,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return scan_impl(desc, x, dt, dt_bias, A, B, C, D, initial_state, y, final_state, workspace,
                   workspace_bytes, stream, nullptr, 0, false, false, false, variant);
}

ssd_status ssd_chunk_scan_noalloc(const ssd_scan_desc* desc, const void* x, const float* dt,
                                  const float* dt_bias, const float* A, const void* B,
                                  const void* C, const float* D, const float* initial_state,
                                  void* y, float* final_state, hipStream_t stream) {
  ScanSizes s;
  const ssd_status st = check_scan_desc(desc, &s);
  if (st != SSD_OK) return st;
  if (s.ws_total > kScratchBytes) return SSD_ERR_WORKSPACE;
  void* ws = nullptr;
  if (desc->batch > 0 && desc->seqlen > 0) {
    const ssd_status sst = scratch_of_stream(stream, &ws);
    if (sst != SSD_OK) return sst;
  }
  return scan_impl(desc, x, dt, dt_bias, A, B, C, D, initial_state, y, final_state, ws,
                   kScratchBytes, stream, nullptr, 0);
}

ssd_status ssd_step(const ssd_step_desc* d, float* state, const void* x_t, const float* dt_t,
                    const float* dt_bias, const float* A, const void* B_t, const void* C_t,
                    const float* D, void* y_t, hipStream_t stream) {
  if (!d) return SSD_ERR_INVALID_ARG;
  if (d->io_dtype != SSD_F32 && d->io_dtype != SSD_BF16) return SSD_ERR_DTYPE;
  if (d->batch < 0 || d->nheads <= 0 || d->headdim <= 0 || d->dstate <= 0 || d->ngroups <= 0)
    return SSD_ERR_SHAPE;
  if (d->nheads % d->ngroups != 0) return SSD_ERR_SHAPE;
  if (!limits_ok(d->dt_min, d->dt_max)) return SSD_ERR_INVALID_ARG;
  if (!ssd::step_shape_supported(d->headdim, d->dstate)) return SSD_ERR_UNSUPPORTED;
  int64_t bh = 0, pn = 0, n_state = 0, n_x = 0, bg = 0, n_bc = 0;
  if (!mul_ok(d->batch, d->nheads, &bh) || !mul_ok(d->headdim, d->dstate, &pn) ||
      !mul_ok(bh, pn, &n_state) || !mul_ok(bh, d->headdim, &n_x) ||
      !mul_ok(d->batch, d->ngroups, &bg) || !mul_ok(bg, d->dstate, &n_bc) || bh > INT32_MAX)
    return SSD_ERR_UNSUPPORTED;
  if (d->batch == 0) return SSD_OK;
  if (!state || !x_t || !dt_t || !A || !B_t || !C_t || !y_t) return SSD_ERR_INVALID_ARG;
  const void* vec[] = {state, x_t, B_t, C_t, y_t};
  for (const void* p : vec)
    if (p && !aligned16(p)) return SSD_ERR_ALIGNMENT;
  const void* scal[] = {dt_t, dt_bias, A, D};
  for (const void* p : scal)
    if (p && !aligned4(p)) return SSD_ERR_ALIGNMENT;
  const int64_t es = (int64_t)io_size(d->io_dtype);
  const Range r_y = range_of(y_t, n_x * es);
  const Range others[] = {range_of(state, n_state * 4), range_of(x_t, n_x * es),
                          range_of(dt_t, bh * 4), range_of(dt_bias, d->nheads * 4),
                          range_of(A, d->nheads * 4), range_of(B_t, n_bc * es),
                          range_of(C_t, n_bc * es), range_of(D, d->nheads * 4)};
  for (const Range& r : others)
    if (overlap(r_y, r)) return SSD_ERR_INVALID_ARG;
  const Range r_s = others[0];
  for (int k = 1; k < 8; ++k)
    if (overlap(r_s, others[k])) return SSD_ERR_INVALID_ARG;

  ssd::StepArgs a;
  a.state = state; a.x = x_t; a.dt = dt_t; a.dt_bias = dt_bias; a.A = A;
  a.B = B_t; a.C = C_t; a.D = D; a.y = y_t;
  a.Bt = d->batch; a.H = d->nheads; a.G = d->ngroups;
  a.P = (int32_t)d->headdim; a.N = (int32_t)d->dstate;
  a.softplus = d->dt_softplus ? 1 : 0;
  a.dt_min = d->dt_min; a.dt_max = d->dt_max;
  hipError_t e = d->io_dtype == SSD_BF16 ? ssd::launch_step_bf16(a, stream)
                                         : ssd::launch_step_f32(a, stream);
  return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

ssd_status ssd_conv1d(const ssd_conv_desc* d, const void* x, const float* w, const float* bias,
                      const void* state_in, void* y, void* state_out, hipStream_t stream) {
  ConvSizes s;
  const ssd_status st = check_conv_desc(d, false, &s);
  if (st != SSD_OK) return st;
  if (d->batch == 0 || (d->seqlen == 0 && !state_out)) return SSD_OK;
  if (!w || (d->seqlen > 0 && (!x || !y))) return SSD_ERR_INVALID_ARG;
  const void* vec[] = {x, y, state_in, state_out};
  for (const void* p : vec)
    if (p && !aligned16(p)) return SSD_ERR_ALIGNMENT;
  if (!aligned4(w) || (bias && !aligned4(bias))) return SSD_ERR_ALIGNMENT;
  const Range r_x = range_of(x, s.n_x * s.es), r_y = range_of(y, s.n_x * s.es);
  const Range r_w = range_of(w, s.n_w * 4), r_b = range_of(bias, d->channels * 4);
  const Range r_si = range_of(state_in, s.n_state * s.es);
  const Range r_so = range_of(state_out, s.n_state * s.es);
  const Range for_y[] = {r_x, r_w, r_b, r_si, r_so};
  for (const Range& r : for_y)
    if (overlap(r_y, r)) return SSD_ERR_INVALID_ARG;
  const Range for_so[] = {r_x, r_w, r_b};
  for (const Range& r : for_so)
    if (overlap(r_so, r)) return SSD_ERR_INVALID_ARG;
  if (state_out != state_in && overlap(r_so, r_si)) return SSD_ERR_INVALID_ARG;

  ssd::ConvArgs a = conv_args(d, d->seqlen);
  a.x = x; a.w = w; a.bias = bias; a.state_in = state_in; a.y = y; a.state_out = state_out;
  const hipError_t e = ssd::launch_conv(a, d->io_dtype == SSD_BF16, false, stream);
  return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

ssd_status ssd_conv1d_step(const ssd_conv_desc* d, void* state, const void* x_t, const float* w,
                           const float* bias, void* y_t, hipStream_t stream) {
  ConvSizes s;
  const ssd_status st = check_conv_desc(d, true, &s);
  if (st != SSD_OK) return st;
  if (d->batch == 0) return SSD_OK;
  if (!state || !x_t || !w || !y_t) return SSD_ERR_INVALID_ARG;
  const void* vec[] = {state, x_t, y_t};
  for (const void* p : vec)
    if (!aligned16(p)) return SSD_ERR_ALIGNMENT;
  if (!aligned4(w) || (bias && !aligned4(bias))) return SSD_ERR_ALIGNMENT;
  const Range r_s = range_of(state, s.n_state * s.es), r_y = range_of(y_t, s.n_x * s.es);
  const Range inputs[] = {range_of(x_t, s.n_x * s.es), range_of(w, s.n_w * 4),
                          range_of(bias, d->channels * 4)};
  for (const Range& r : inputs)
    if (overlap(r_y, r) || overlap(r_s, r)) return SSD_ERR_INVALID_ARG;
  if (overlap(r_y, r_s)) return SSD_ERR_INVALID_ARG;

  ssd::ConvArgs a = conv_args(d, 1);
  a.x = x_t; a.w = w; a.bias = bias; a.state_in = state; a.y = y_t; a.state_out = state;
  const hipError_t e = ssd::launch_conv(a, d->io_dtype == SSD_BF16, true, stream);
  return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

size_t ssd_chunk_scan_backward_workspace_bytes(const ssd_scan_desc* desc) {
  BwdPlan pl;
  if (plan_backward(desc, &pl) != SSD_OK) return 0;
  return pl.total;
}

ssd_status ssd_chunk_scan_backward(const ssd_scan_desc* d, const void* x, const float* dt,
                                   const float* dt_bias, const float* A, const void* B,
                                   const void* C, const float* D, const float* initial_state,
                                   const void* dy, const float* dfinal_state, float* dx,
                                   float* ddt, float* dA, float* dB, float* dC, float* dD,
                                   float* ddt_bias, float* dinitial_state, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  BwdPlan pl;
  ssd_status st = plan_backward(d, &pl);
  if (st != SSD_OK) return st;
  ScanSizes s;
  check_scan_desc(d, &s);
  const bool tokens = d->batch > 0 && d->seqlen > 0;
  if (d->batch > 0 && (!A || !dA)) return SSD_ERR_INVALID_ARG;
  if (tokens && (!x || !dt || !B || !C || !dy || !dx || !ddt || !dB || !dC))
    return SSD_ERR_INVALID_ARG;
  const void* vec[] = {x, B, C, initial_state, dy, dfinal_state, dx, dB, dC, dinitial_state,
                       workspace};
  for (const void* p : vec)
    if (p && !aligned16(p)) return SSD_ERR_ALIGNMENT;
  const void* scal[] = {dt, dt_bias, A, D, ddt, dA, dD, ddt_bias};
  for (const void* p : scal)
    if (p && !aligned4(p)) return SSD_ERR_ALIGNMENT;
  if (tokens && (!workspace || workspace_bytes < pl.total)) return SSD_ERR_WORKSPACE;
  // gradients must not overlap any input, the workspace or each other
  const int64_t es = (int64_t)io_size(d->io_dtype), H = d->nheads;
  const Range outs[] = {range_of(dx, tokens ? s.n_x * 4 : 0),
                        range_of(ddt, tokens ? s.n_dt * 4 : 0), range_of(dA, H * 4),
                        range_of(dB, tokens ? s.n_bc * 4 : 0),
                        range_of(dC, tokens ? s.n_bc * 4 : 0), range_of(dD, H * 4),
                        range_of(ddt_bias, H * 4), range_of(dinitial_state, s.n_state * 4)};
  const Range ins[] = {range_of(x, tokens ? s.n_x * es : 0),
                       range_of(dt, tokens ? s.n_dt * 4 : 0), range_of(dt_bias, H * 4),
                       range_of(A, H * 4), range_of(B, tokens ? s.n_bc * es : 0),
                       range_of(C, tokens ? s.n_bc * es : 0), range_of(D, H * 4),
                       range_of(initial_state, s.n_state * 4),
                       range_of(dy, tokens ? s.n_x * es : 0),
                       range_of(dfinal_state, s.n_state * 4),
                       range_of(workspace, tokens ? (int64_t)pl.total : 0)};
  const int nouts = (int)(sizeof(outs) / sizeof(outs[0]));
  for (int i = 0; i < nouts; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return SSD_ERR_INVALID_ARG;
    for (int j = i + 1; j < nouts; ++j)
      if (overlap(outs[i], outs[j])) return SSD_ERR_INVALID_ARG;
  }
  if (d->batch == 0) {
    if (!dA && !dD && !ddt_bias) return SSD_OK;
    if (!dA) return SSD_ERR_INVALID_ARG;
    return ssd::launch_backward_zero_heads(dA, ddt_bias, dD, H, stream) == hipSuccess
               ? SSD_OK : SSD_ERR_HIP;
  }
  if (!tokens) {
    // no token: the parameters get no gradient, the initial state passes dfinal on
    if (ssd::launch_backward_zero_heads(dA, ddt_bias, dD, H, stream) != hipSuccess)
      return SSD_ERR_HIP;
    if (dinitial_state &&
        ssd::launch_copy_or_zero(dinitial_state, dfinal_state, s.n_state, stream) != hipSuccess)
      return SSD_ERR_HIP;
    return SSD_OK;
  }

  char* w = static_cast<char*>(workspace);
  auto at = [&](int k) { return static_cast<void*>(w + pl.off[k]); };
  auto atf = [&](int k) { return reinterpret_cast<float*>(w + pl.off[k]); };

  ssd::BwdArgs a;
  a.x = x; a.dt = dt; a.dt_bias = dt_bias; a.A = A; a.B = B; a.C = C; a.D = D;
  a.h0 = initial_state; a.dy = dy; a.dfinal = dfinal_state;
  const bool bf = d->io_dtype == SSD_BF16;
  a.wd = atf(kWd); a.cum = reinterpret_cast<double*>(w + pl.off[kCum]);
  a.rscale = atf(kRscale); a.dtr1 = atf(kDtr1);
  a.r1_x = at(kR1x); a.r1_b = at(kR1b); a.r1_c = at(kR1c); a.r1_h0 = atf(kR1h0);
  a.r1_y = at(kR1y); a.r1_final = atf(kR1final);
  a.fwd_state = atf(kScanWs);
  a.fwd_cb = reinterpret_cast<const float*>(w + pl.off[kScanWs] + pl.fwd_cb_off);
  a.r1_state = atf(kScanWsR1);
  a.mix = atf(kMix); a.qrow = atf(kQrow); a.qcol = atf(kQcol); a.uv = atf(kUv);
  a.dbc_part = pl.HSD > 1 ? atf(kDbcPart) : nullptr;
  a.ddin = atf(kDdin); a.dDp = atf(kDdp); a.part = atf(kPart);
  a.dx = dx; a.ddt = ddt; a.dA = dA; a.dB = dB; a.dC = dC; a.dD = dD;
  a.ddt_bias_out = ddt_bias; a.dh0 = dinitial_state;
  a.Bt = d->batch; a.T = d->seqlen; a.H = d->nheads; a.G = d->ngroups;
  a.L = d->chunk; a.Nc = s.Nc; a.pad = pl.pad;
  a.P = (int32_t)d->headdim; a.N = (int32_t)d->dstate;
  a.NB = pl.NB; a.LP = pl.LP; a.HS = pl.HS; a.hpw = pl.hpw; a.HSD = pl.HSD; a.hpwd = pl.hpwd;
  a.NS = pl.NS;
  a.softplus = d->dt_softplus ? 1 : 0;
  a.dt_min = d->dt_min; a.dt_max = d->dt_max;

  if (ssd::launch_backward_phase(a, bf, 0, stream) != hipSuccess) return SSD_ERR_HIP;
  // forward states (phased schedule of the io type): C B^T and the float32
  // state entering each chunk
  st = scan_impl(&pl.fw, x, dt, dt_bias, A, B, C, D, initial_state, nullptr, nullptr,
                 at(kScanWs), pl.scan_ws, stream, nullptr, 0, true, true, true);
  if (st != SSD_OK) return st;
  // R1: sum_n G B over reversed time; its entering states are the adjoint at
  // the forward chunk boundaries and its final state dL/dh_{-1} / abar_0
  st = scan_impl(&pl.r1, a.r1_x, a.dtr1, nullptr, A, a.r1_b, a.r1_c, nullptr, a.r1_h0,
                 at(kR1y), atf(kR1final), at(kScanWsR1), pl.scan_ws_r1, stream, nullptr, 0,
                 false, true, true);
  if (st != SSD_OK) return st;
  if (ssd::launch_backward_phase(a, bf, 1, stream) != hipSuccess) return SSD_ERR_HIP;
  return SSD_OK;
}

const char* ssd_status_string(ssd_status s) {
  switch (s) {
    case SSD_OK: return "SSD_OK";
    case SSD_ERR_INVALID_ARG: return "SSD_ERR_INVALID_ARG: null, aliased or otherwise invalid argument";
    case SSD_ERR_SHAPE: return "SSD_ERR_SHAPE: non-positive size or heads not a multiple of groups";
    case SSD_ERR_DTYPE: return "SSD_ERR_DTYPE: unknown io dtype";
    case SSD_ERR_ALIGNMENT: return "SSD_ERR_ALIGNMENT: device pointer below its required alignment";
    case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED: shape without a compiled gfx950 variant";
    case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE: workspace missing or too small";
    case SSD_ERR_HIP: return "SSD_ERR_HIP: a HIP launch failed";
  }
  return "unknown ssd_status";
}

int32_t ssd_abi_version(void) { return SSD_ABI_VERSION; }

}  // extern "C"
