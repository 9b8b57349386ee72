// Pieces shared by the chunked-scan kernels of both io types.
//
// Source: "Compiler-First State Space Duality and Portable O(1)
// Autoregressive Caching", Background (Eq. 3 and the inter-chunk recurrence
// after it) and SSD properties ("diagonal state matrix": the decay over a
// chunk is the exponential of a segment-wise prefix sum of A*Delta).
#pragma once

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {
namespace prefill {

constexpr int kThreads = 256;  // 4 wavefronts per workgroup
constexpr int kMaxL = 512;

// Step Delta_l and the inclusive prefix sum cum_l of a_l = Delta_l A[h] over
// the chunk's L tokens.  Tokens at or past T get Delta = 0 (so the sum stays
// flat there).  Each thread owns tokens 2*tid and 2*tid+1.  The work is split
// in two stages around a barrier so that a kernel can overlap the first stage
// with other work; every kernel runs the same operations in the same order,
// so all of them get bit-identical Delta and cum values.  Products and sums
// are written with explicit rounding so the compiler cannot fuse them
// differently from one kernel to another.
struct DeltaScan {
  float d0, d1, a0, a1, local, incl;
};

// Raw dt of this thread's two tokens.  Tokens past the chunk or past T
// re-read the chunk's last token: unconditional loads and no select on the
// loaded values (a select would wait for them at once); stage 1 gives those
// tokens Delta = 0.
__device__ __forceinline__ float2 chunk_dt_load(const ScanArgs& a, int64_t b, int64_t c,
                                                int64_t h) {
  const int l0 = 2 * opaque_tid(), l1 = l0 + 1;
  const int64_t t0 = c * a.L;
  const int last = (int)min<int64_t>(a.L, a.T - t0) - 1;   // last token of the chunk
  const float* dg = a.dt + (b * a.T + t0) * a.H + h;        // uniform base, 32-bit lane offsets
  const uint32_t hs = (uint32_t)a.H;
  const float v0 = *off32(dg, (uint32_t)min(l0, last) * hs);
  const float v1 = *off32(dg, (uint32_t)min(l1, last) * hs);
  return make_float2(v0, v1);
}

// A and the dt bias of head h.  A kernel that walks several chunks of one
// head loads them once: a load inside the walk would be waited for next to
// the loads of the following chunk.
struct HeadConsts {
  float A, bias;
};
__device__ __forceinline__ HeadConsts head_consts(const ScanArgs& a, int64_t h) {
  return HeadConsts{a.A[h], a.dt_bias ? a.dt_bias[h] : 0.0f};
}

// Stage 1: Delta, a and the wavefront-inclusive scan; publishes each
// wavefront's total in s_wsum[wave].  No barrier inside.
__device__ __forceinline__ DeltaScan chunk_scan_stage1(const ScanArgs& a, int64_t c,
                                                       HeadConsts hc, float2 dtv,
                                                       float* s_wsum) {
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int l0 = 2 * tid, l1 = l0 + 1;
  const int64_t t0 = c * a.L;
  const float Ah = hc.A;
  const float bias = hc.bias;
  DeltaScan s;
  s.d0 = (l0 < a.L && t0 + l0 < a.T)
             ? delta_of(__fadd_rn(dtv.x, bias), a.softplus, a.dt_min, a.dt_max) : 0.0f;
  s.d1 = (l1 < a.L && t0 + l1 < a.T)
             ? delta_of(__fadd_rn(dtv.y, bias), a.softplus, a.dt_min, a.dt_max) : 0.0f;
  s.a0 = __fmul_rn(s.d0, Ah);
  s.a1 = __fmul_rn(s.d1, Ah);
  s.local = __fadd_rn(s.a0, s.a1);
  s.incl = wave_inclusive_scan(s.local, lane);
  if (lane == 63) s_wsum[wave] = s.incl;
  return s;
}
__device__ __forceinline__ DeltaScan chunk_scan_stage1(const ScanArgs& a, int64_t c, int64_t h,
                                                       float2 dtv, float* s_wsum) {
  return chunk_scan_stage1(a, c, head_consts(a, h), dtv, s_wsum);
}

// Stage 2 (after a barrier that follows stage 1): cross-wavefront offsets;
// writes s_d and s_cum for this thread's tokens.  No barrier inside.
__device__ __forceinline__ void chunk_scan_stage2(const ScanArgs& a, const DeltaScan& s,
                                                  const float* s_wsum, float* s_d, float* s_cum) {
  const int tid = opaque_tid(), wave = tid >> 6;
  const int l0 = 2 * tid, l1 = l0 + 1;
  float off = 0.0f;
  for (int w = 0; w < wave; ++w) off = __fadd_rn(off, s_wsum[w]);
  const float excl = __fadd_rn(off, __fsub_rn(s.incl, s.local));
  const float c0 = __fadd_rn(excl, s.a0);
  if (l0 < a.L) { s_d[l0] = s.d0; s_cum[l0] = c0; }
  if (l1 < a.L) { s_d[l1] = s.d1; s_cum[l1] = __fadd_rn(c0, s.a1); }
}

// Both stages with their barriers: s_d and s_cum are ready for every thread
// on return.  Every thread of the block must call this.
__device__ __forceinline__ void chunk_delta_cumsum(const ScanArgs& a, int64_t b, int64_t c,
                                                   int64_t h, float* s_d, float* s_cum,
                                                   float* s_wsum) {
  const DeltaScan s = chunk_scan_stage1(a, c, h, chunk_dt_load(a, b, c, h), s_wsum);
  __syncthreads();
  chunk_scan_stage2(a, s, s_wsum, s_d, s_cum);
  __syncthreads();
}

// Row tiles of 16 tokens are dealt to the 4 wavefronts in a snake order
// (0 1 2 3 3 2 1 0 0 1 ...), which balances the triangular intra-chunk work.
__device__ __forceinline__ int row_tile_of(int wave, int k) {
  return 4 * k + ((k & 1) ? 3 - wave : wave);
}

// Number of valid tokens in chunk c.
__device__ __forceinline__ int chunk_len(const ScanArgs& a, int64_t c) {
  return (int)min<int64_t>(a.L, a.T - c * a.L);
}

// 16 bytes = one fragment chunk of a lane.
__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
// Branch-free masked load: `p` must be a valid address whether or not `ok`
// (callers clamp the row); the value is replaced by zeros when !ok.  A plain
// `ok ? load : 0` becomes one exec-masked branch, and a wait, per load.
__device__ __forceinline__ float4 ld4_masked(const float* p, bool ok) {
  const float4 v = ld4(p);
  return ok ? v : make_float4(0.f, 0.f, 0.f, 0.f);
}
__device__ __forceinline__ void st4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
__device__ __forceinline__ float get(const float4& v, int k) {
  return k == 0 ? v.x : (k == 1 ? v.y : (k == 2 ? v.z : v.w));
}

}  // namespace prefill
}  // namespace ssd
