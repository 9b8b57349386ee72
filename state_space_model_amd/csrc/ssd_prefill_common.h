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
// the chunk's L tokens, into LDS.  Tokens at or past T get Delta = 0 (so the
// sum stays flat there).  Every thread of the block must call this; it ends
// with a barrier.  Each thread owns tokens 2*tid and 2*tid+1; the wavefront
// scan and the cross-wave offsets run in a fixed order, so every kernel that
// calls this gets bit-identical values.
__device__ __forceinline__ void chunk_delta_cumsum(const ScanArgs& a, int64_t b, int64_t c,
                                                   int64_t h, float* s_d, float* s_cum,
                                                   float* s_wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = (int)a.L;
  const int64_t t0 = c * a.L;
  const float Ah = a.A[h];
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
  const int l0 = 2 * tid, l1 = 2 * tid + 1;
  float d0 = 0.0f, d1 = 0.0f;
  if (l0 < L && t0 + l0 < a.T)
    d0 = delta_of(a.dt[(b * a.T + t0 + l0) * a.H + h] + bias, a.softplus, a.dt_min, a.dt_max);
  if (l1 < L && t0 + l1 < a.T)
    d1 = delta_of(a.dt[(b * a.T + t0 + l1) * a.H + h] + bias, a.softplus, a.dt_min, a.dt_max);
  const float a0 = d0 * Ah, a1 = d1 * Ah;
  const float local = a0 + a1;
  const float incl = wave_inclusive_scan(local);
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  float off = 0.0f;
  for (int w = 0; w < wave; ++w) off += s_wsum[w];
  const float excl = off + (incl - local);
  if (l0 < L) { s_d[l0] = d0; s_cum[l0] = excl + a0; }
  if (l1 < L) { s_d[l1] = d1; s_cum[l1] = excl + a0 + a1; }
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
__device__ __forceinline__ void st4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
__device__ __forceinline__ float get(const float4& v, int k) {
  return k == 0 ? v.x : (k == 1 ? v.y : (k == 2 ? v.z : v.w));
}

}  // namespace prefill
}  // namespace ssd
