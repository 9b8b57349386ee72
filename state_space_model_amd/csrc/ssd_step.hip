// One decode step of the SSD recurrence for gfx950, state updated in place.
//
// Source: "Compiler-First State Space Duality and Portable O(1)
// Autoregressive Caching", O(1) cache section (the fixed-size state
// (B,H,P,N) summarises the prefix; the next token needs one step
// h_t = Abar h_{t-1} + Bbar x_t) and Results (decode reads and writes the same
// state whatever the prefix length, so it is bound by memory bandwidth).
//
// Per (b, h):  d = clip(softplus(dt + dt_bias)),  alpha = exp(d A[h])
//   h'[p,n] = alpha h[p,n] + d x[p] B[n];   y[p] = sum_n C[n] h'[p,n] + D[h] x[p]
// A workgroup streams the (b, h) state slice, or a run of its rows: every
// lane moves 16-byte vectors, a wavefront instruction covers 1 KB of
// contiguous state, each element is read once and written once, and the row
// sums over n are reduced across the N/4 lanes that hold one row.  The state is touched exactly once
// per step, so its loads and stores are non-temporal (no cache allocation for
// a stream that will not be re-read before it is evicted); this alone raised
// the measured rate at batch 64 from 53% to 65% of the HBM peak.  The
// workgroup shape (threads x vectors per lane, workgroups per slice) is
// chosen per batch size from measurements (launch_step).
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;  // block size of the helper kernels

__device__ __forceinline__ float4 ld_stream(const float4* p) {
  const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ void st_stream(float4* p, float4 v) {
  __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4*>(p));
}

// THREADS lanes per workgroup, BATCH float4 loads in flight per lane.
//
// EXACT = true: the token's x, B and C and the state vectors of the first
// pass are all issued before anything is computed, and every load is issued
// on every path (indexes clamped), so the wait before each state vector
// covers exactly that vector.  EXACT = false: the state loads go first and
// each vector's x is loaded next to its use; the wait for that x also waits
// for the previous vector's store (loads and stores share one counter), which
// spaces out the stores.  Measured at the 2.7B shape: exact waits took batch
// 64 from 57.8 to 56.1 us and batch 1 from 4.74 to 4.28 us; at batch 16 the
// spaced stores are faster (15.4 against 17.1 us).
//
// PS workgroups share one (b, h) slice, each taking P / PS consecutive rows:
// the rows are independent (row p needs x[p] and the whole of B and C), so the
// split changes no arithmetic and every element is computed exactly as with
// one workgroup per slice.
template <typename T, int THREADS, int BATCH, bool EXACT, int PS = 1>
__global__ __launch_bounds__(THREADS) void k_step(StepArgs a) {
  const int64_t bh = blockIdx.x / PS;
  const int ps = (int)(blockIdx.x % PS);
  const int P = a.P / PS, N = a.N, NQ = N / 4;   // P: rows of this workgroup
  const int nq_shift = __builtin_ctz(NQ);   // N / 4 is a power of two
  const int tid = threadIdx.x;
  const int total = P * NQ;  // float4 elements of the rows, a multiple of 64
  float4* st = reinterpret_cast<float4*>(a.state + (bh * PS + ps) * (int64_t)P * N);
  const int64_t b = bh / a.H, h = bh % a.H, g = h / (a.H / a.G);
  const T* xg = reinterpret_cast<const T*>(a.x) + (bh * PS + ps) * P;
  const T* Bg = reinterpret_cast<const T*>(a.B) + (b * a.G + g) * N;
  const T* Cg = reinterpret_cast<const T*>(a.C) + (b * a.G + g) * N;
  T* yg = reinterpret_cast<T*>(a.y) + (bh * PS + ps) * P;
  // the n-quad of this lane is the same for every row it visits (NQ | THREADS)
  const int n4 = tid % NQ;

  float4 s[BATCH];
  T xraw[BATCH], braw[4], craw[4];
  auto load_pass = [&](int base) {
    if constexpr (EXACT) {
#pragma unroll
      for (int k = 0; k < BATCH; ++k) xraw[k] = xg[min(base + k * THREADS + tid, total - 1) >> nq_shift];
#pragma unroll
      for (int k = 0; k < BATCH; ++k) s[k] = ld_stream(&st[min(base + k * THREADS + tid, total - 1)]);
    } else {
#pragma unroll
      for (int k = 0; k < BATCH; ++k) {
        const int f = base + k * THREADS + tid;
        if (f < total) s[k] = ld_stream(&st[f]);   // uniform per wavefront
      }
    }
    // keep the loads ahead of the conversions that consume them
    __builtin_amdgcn_sched_barrier(0);
  };
  if constexpr (EXACT) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      braw[k] = Bg[4 * n4 + k];
      craw[k] = Cg[4 * n4 + k];
    }
  }
  load_pass(0);
  if constexpr (!EXACT) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      braw[k] = Bg[4 * n4 + k];
      craw[k] = Cg[4 * n4 + k];
    }
  }
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
  const float d = delta_of(a.dt[bh] + bias, a.softplus, a.dt_min, a.dt_max);
  const float alpha = expf(d * a.A[h]);
  const float Dh = a.D ? a.D[h] : 0.0f;
  float bv[4], cv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    bv[k] = to_f32(braw[k]);
    cv[k] = to_f32(craw[k]);
  }
  for (int base = 0; base < total; base += THREADS * BATCH) {
    if (base > 0) load_pass(base);
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int f = base + k * THREADS + tid;
      if (f < total) {  // uniform per wavefront: total is a multiple of 64
        const int p = f >> nq_shift;
        const float xp = to_f32(EXACT ? xraw[k] : xg[p]);
        const float dx = d * xp;
        float4 v = s[k];
        v.x = alpha * v.x + dx * bv[0];
        v.y = alpha * v.y + dx * bv[1];
        v.z = alpha * v.z + dx * bv[2];
        v.w = alpha * v.w + dx * bv[3];
        st_stream(&st[f], v);
        float part = cv[0] * v.x + cv[1] * v.y + cv[2] * v.z + cv[3] * v.w;
        part = group_sum(part, NQ);
        if (n4 == 0) yg[p] = to_io<T>(part + Dh * xp);
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_copy_or_zero(float4* dst, const float4* src, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n4) dst[i] = src ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

template <typename T>
hipError_t launch_step(const StepArgs& a, hipStream_t stream) {
  const int64_t slices = a.Bt * a.H;
  // Shapes measured at the 2.7B shape (P N = 8192, 1024 steps from one HIP
  // graph).  Batch 1 (80 slices) and batch 64: each slice's rows split over
  // four workgroups of 256 lanes, two vectors each (batch 1: 4.05 -> 3.54 us,
  // more compute units streaming at once; batch 64: 56.6 -> 55.5 us).  Batch
  // 16 (1280 slices): one workgroup of 256 lanes x 8 vectors per slice with
  // spaced stores (16.0 us; every split or exact-wait shape tried was
  // 16.2-18.8 us).  P N >= 8192 makes every split's rows a multiple of 64
  // vectors and a whole number of 512-vector passes.  The split grid must
  // also fit the 32-bit grid dimension (the whole-slice grid always does: the
  // ABI refuses more than INT32_MAX slices).
  if (a.P * a.N >= 8192 && (slices >= 2048 || slices < 512) && slices <= INT32_MAX / 4) {
    hipLaunchKernelGGL((k_step<T, 256, 2, true, 4>), dim3((unsigned)(slices * 4)), dim3(256), 0,
                       stream, a);
  } else {
    hipLaunchKernelGGL((k_step<T, 256, 8, false>), dim3((unsigned)slices), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

bool step_shape_supported(int64_t P, int64_t N) {
  return (P == 16 || P == 32 || P == 64 || P == 128) && (N == 16 || N == 32 || N == 64 || N == 128);
}

hipError_t launch_step_f32(const StepArgs& a, hipStream_t s) { return launch_step<float>(a, s); }
hipError_t launch_step_bf16(const StepArgs& a, hipStream_t s) { return launch_step<bf16>(a, s); }

hipError_t launch_copy_or_zero(float* dst, const float* src, int64_t n, hipStream_t stream) {
  const int64_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  const int64_t blocks = (n4 + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(k_copy_or_zero, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     reinterpret_cast<float4*>(dst), reinterpret_cast<const float4*>(src), n4);
  return hipGetLastError();
}

}  // namespace ssd
