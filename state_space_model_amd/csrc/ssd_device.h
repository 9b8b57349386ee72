// Device-side building blocks of the gfx950 SSD kernels: io types, matrix-core
// (MFMA) fragments, the Delta activation and wavefront reductions/scans.
//
// gfx950 (CDNA4) only.  Wavefronts are 64 lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// exp(x) on the hardware base-2 exponential: exp(x) = 2^(x log2 e).
// Results below the float32 normal range flush to zero, which is harmless
// here: every argument is a (non-positive) accumulated decay.
__device__ __forceinline__ float fast_exp(float x) {
  return __builtin_amdgcn_exp2f(x * kLog2e);
}

constexpr float kLn2 = 0.6931471805599453f;

// softplus(z) = max(z, 0) + log1p(exp(-|z|)), which never overflows, on the
// hardware base-2 exponential and logarithm.  log1p(e) for e = exp(-|z|) in
// (0, 1] is formed as log(u) e / (u - 1) with u = 1 + e rounded to float32
// (Goldberg, "What every computer scientist should know about floating-point
// arithmetic", 1991, Theorem 4): the quotient e / (u - 1) cancels the rounding
// of u, so the result keeps a few-ulp relative error for tiny e as well; when
// u rounds to 1, log1p(e) = e to working precision.
__device__ __forceinline__ float softplus_of(float z) {
  const float e = __builtin_amdgcn_exp2f(-fabsf(z) * kLog2e);
  const float u = 1.0f + e;
  const float l = u == 1.0f ? e
                            : __builtin_amdgcn_logf(u) * kLn2 * e * __builtin_amdgcn_rcpf(u - 1.0f);
  return fmaxf(z, 0.0f) + l;
}

// Delta = clip(softplus(dt + dt_bias), lo, hi)  ("Compiler-First State Space
// Duality ...", Implementation: einsum shaping names softplus and clip).
// Every kernel forms Delta through this one function, so all of them see the
// same bits for a token.
__device__ __forceinline__ float delta_of(float z, int softplus, float lo, float hi) {
  float d = softplus ? softplus_of(z) : z;
  return fminf(fmaxf(d, lo), hi);
}

// ---------------------------------------------------------------------------
// Matrix-core fragments.
//
// Both instructions used here compute a 16x16 float32 tile D += A * B with
// the same register layout for A, B and D:
//   lane l holds A[i = l % 16][k-slots of group q = l / 16]
//   lane l holds B[k-slots of group q][j = l % 16]
//   register r of lane l holds D[i = 4 (l / 16) + r][j = l % 16]
// float32:  v_mfma_f32_16x16x4_f32, 1 k-slot per lane  (K = 4 per instruction)
// bfloat16: v_mfma_f32_16x16x32_bf16, 8 k-slots per lane (K = 32)
// The reduction runs over all K slots, so any assignment of contraction
// indices to (group, slot) works as long as A and B use the same one.
// ---------------------------------------------------------------------------
template <typename T> struct Mfma;

template <> struct Mfma<float> {
  using frag = float;
  static constexpr int KPL = 1;   // k-slots per lane
  static constexpr int K = 4;     // k per instruction
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<bf16> {
  using frag = bf16x8;
  static constexpr int KPL = 8;
  static constexpr int K = 32;
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <typename T> __device__ __forceinline__ T to_io(float v);
template <> __device__ __forceinline__ float to_io<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 to_io<bf16>(float v) { return (bf16)v; }  // RNE

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

// Load KPL consecutive io elements (one fragment) from LDS or global memory.
// The address must be aligned to the fragment size (4 B float, 16 B bf16x8).
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag load_frag(const T* p) {
  return *reinterpret_cast<const typename Mfma<T>::frag*>(p);
}

// ---------------------------------------------------------------------------
// Wavefront helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// The thread index through an opaque copy.  Inside a kernel's long loop the
// indices and addresses derived from it are then formed where they are used
// instead of being hoisted out of the loop and held in (or spilled from)
// registers across it.
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// base + elems elements, the offset formed in 32 bits (bytes): with a
// wavefront-uniform base the load or store can take the scalar-base address
// form (base in scalar registers, a 32-bit offset per lane) instead of a
// 64-bit address computed per lane.  elems * sizeof(T) must fit in 32 bits.
template <typename T>
__device__ __forceinline__ T* off32(T* base, uint32_t elems) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + (elems * (uint32_t)sizeof(T)));
}
template <typename T>
__device__ __forceinline__ const T* off32(const T* base, uint32_t elems) {
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) +
                                    (elems * (uint32_t)sizeof(T)));
}

// Inclusive prefix sum across the 64 lanes of a wavefront (Hillis-Steele,
// log2(64) = 6 shuffle steps; a fixed order, so the result is reproducible).
// `lane` is the caller's lane index; a caller in a loop passes an opaque copy
// so that the six source-lane addresses are formed at each use rather than
// held in registers across the loop.
__device__ __forceinline__ float wave_inclusive_scan(float v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    // lanes below `off` read some lane and discard it
    const float o = __int_as_float(__builtin_amdgcn_ds_bpermute((lane - off) << 2,
                                                                __float_as_int(v)));
    if (lane >= off) v += o;
  }
  return v;
}
__device__ __forceinline__ float wave_inclusive_scan(float v) {
  return wave_inclusive_scan(v, lane_id());
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int off = width >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Workgroups are dealt round-robin to the 8 XCDs of an MI355X (block b runs
// on XCD b % 8).  Re-number blocks so that consecutive logical units land on
// the same XCD and share its L2 (e.g. the heads of one chunk read the same
// B/C rows).  Valid for any grid size: the last partial round keeps its
// round-robin order.
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t nblocks) {
  constexpr int64_t kXcd = 8;
  const int64_t full = (nblocks / kXcd) * kXcd;
  if (bid >= full) return bid;
  const int64_t per = full / kXcd;
  return (bid % kXcd) * per + bid / kXcd;
}

}  // namespace ssd
