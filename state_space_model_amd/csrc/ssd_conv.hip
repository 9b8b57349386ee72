// Depthwise causal convolution over time for gfx950: a whole sequence with
// its cached window carried in and out, and one token from the window.
//
// Source: "Compiler-First State Space Duality and Portable O(1)
// Autoregressive Caching", O(1) cache section (each channel is convolved over
// a sliding window of its k-1 previous inputs, cached with shape
// (B, D_conv, k-1); the decode body updates that window) and Setup (k = 4).
//
// Per batch row b and channel c, xp = (window[b][c][0..k-2], x[b][0..T-1][c]):
//   z[t] = bias[c] + sum_{i<k} w[c][i] xp[t+i]      (fused multiply-adds, i = 0..k-1)
//   y[b][t][c] = silu ? z / (1 + exp(-z)) : z
//
// k multiply-adds per element moved: the layer is bound by memory bandwidth.
// A thread owns VEC adjacent channels, 16 bytes of one token row (4 float32
// or 8 bfloat16), so one wavefront instruction moves 1 KB of a row.  In the
// sequence kernel the thread also owns a run of R tokens: it issues the loads
// of the k-1 inputs before the run and of the whole run at once, then
// computes and stores R rows.  The k-1 inputs before a run are re-read by its
// thread (R = 16 makes that 3/16 of the reads, served mostly by the caches).
// Only the thread of the first run of (b, channels) touches the window: it
// reads it before anything else and writes the outgoing window last, so the
// window may be updated in place.  Channel counts that are not a multiple of
// VEC (or rows that are therefore not 16-byte aligned) run with VEC = 1.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

constexpr int kConvThreads = 256;
constexpr int kConvRun = 16;  // tokens per thread in the sequence kernel

template <typename T, int VEC>
__device__ __forceinline__ void load_vec(const T* p, float (&v)[VEC]) {
  if constexpr (VEC == 1) {
    v[0] = to_f32(p[0]);
  } else if constexpr (sizeof(T) == 4) {
    static_assert(VEC == 4, "float32 rows move as float4");
    const float4 f = *reinterpret_cast<const float4*>(p);
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  } else {
    static_assert(VEC == 8, "bfloat16 rows move as 8-element vectors");
    const bf16x8 h = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)h[e];
  }
}

template <typename T, int VEC>
__device__ __forceinline__ void store_vec(T* p, const float (&v)[VEC]) {
  if constexpr (VEC == 1) {
    p[0] = to_io<T>(v[0]);
  } else if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    bf16x8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = (bf16)v[e];  // round to nearest even
    *reinterpret_cast<bf16x8*>(p) = h;
  }
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// z = bias + sum_i w[i] * win(i), i = 0..K-1 in this order: shared by both
// kernels so that a token gives the same bits through either.
template <int K, int VEC>
__device__ __forceinline__ void conv_point(const float (&w)[VEC][K], const float (&bs)[VEC],
                                           const float (*xp)[VEC], int silu_on, float (&out)[VEC]) {
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    float z = bs[v];
#pragma unroll
    for (int i = 0; i < K; ++i) z = __fmaf_rn(w[v][i], xp[i][v], z);
    out[v] = silu_on ? silu(z) : z;
  }
}

template <int K, int VEC>
__device__ __forceinline__ void load_weights(const ConvArgs& a, int64_t c0, float (&w)[VEC][K],
                                             float (&bs)[VEC]) {
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
#pragma unroll
    for (int i = 0; i < K; ++i) w[v][i] = a.w[(c0 + v) * K + i];
    bs[v] = a.bias ? a.bias[c0 + v] : 0.0f;
  }
}

// grid: ceil(Bt * NR * NG / 256) blocks; thread -> (b, run of R tokens, VEC channels)
template <typename T, int K, int VEC, int R>
__global__ __launch_bounds__(kConvThreads) void k_conv(ConvArgs a, int64_t NG, int64_t NR) {
  static_assert(R >= K - 1, "only the first run may reach into the cached window");
  const int64_t gid = (int64_t)blockIdx.x * kConvThreads + threadIdx.x;
  if (gid >= a.Bt * NR * NG) return;
  const int64_t g = gid % NG, rest = gid / NG, run = rest % NR, b = rest / NR;
  const int64_t c0 = g * VEC, D = a.D, nT = a.T;
  const int64_t t0 = run * R;
  const int tn = (int)(nT - t0 < R ? nT - t0 : R);  // tokens of this run (0 only when nT == 0)
  const T* xb = reinterpret_cast<const T*>(a.x) + b * nT * D + c0;
  const T* win = a.state_in ? reinterpret_cast<const T*>(a.state_in) + (b * D + c0) * (K - 1)
                            : nullptr;

  float xp[K - 1 + R][VEC];
  // the k-1 inputs before the run: earlier tokens, or the cached window
#pragma unroll
  for (int j = 0; j < K - 1; ++j) {
    const int64_t tt = t0 - (K - 1) + j;
    if (tt >= 0) {
      load_vec<T, VEC>(xb + tt * D, xp[j]);
    } else {
#pragma unroll
      for (int v = 0; v < VEC; ++v) xp[j][v] = win ? to_f32(win[v * (K - 1) + (K - 1) + tt]) : 0.0f;
    }
  }
  if (tn > 0) {
    // the run: tokens past the end re-read the last one and are not stored
#pragma unroll
    for (int t = 0; t < R; ++t) {
      const int tc = t < tn ? t : tn - 1;
      load_vec<T, VEC>(xb + (t0 + tc) * D, xp[K - 1 + t]);
    }
  }
  float w[VEC][K], bs[VEC];
  load_weights<K, VEC>(a, c0, w, bs);
  T* yb = reinterpret_cast<T*>(a.y) + b * nT * D + c0;
#pragma unroll
  for (int t = 0; t < R; ++t) {
    if (t < tn) {
      float out[VEC];
      conv_point<K, VEC>(w, bs, &xp[t], a.silu, out);
      store_vec<T, VEC>(yb + (t0 + t) * D, out);
    }
  }
  // outgoing window: inputs T-(k-1) .. T-1, written by the first run's thread
  // after its reads of the incoming one
  if (run == 0 && a.state_out) {
    T* so = reinterpret_cast<T*>(a.state_out) + (b * D + c0) * (K - 1);
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
      const int64_t tt = nT - (K - 1) + j;
      float v4[VEC];
      if (tt >= 0) {
        load_vec<T, VEC>(xb + tt * D, v4);
      } else {
        // nT < k-1: entry nT + j of the incoming window, already in registers
#pragma unroll
        for (int v = 0; v < VEC; ++v) v4[v] = 0.0f;
#pragma unroll
        for (int jj = 0; jj < K - 1; ++jj)
          if (jj == nT + j) {
#pragma unroll
            for (int v = 0; v < VEC; ++v) v4[v] = xp[jj][v];
          }
      }
#pragma unroll
      for (int v = 0; v < VEC; ++v) so[v * (K - 1) + j] = to_io<T>(v4[v]);
    }
  }
}

// grid: ceil(Bt * NG / 256) blocks; thread -> (b, VEC channels)
template <typename T, int K, int VEC>
__global__ __launch_bounds__(kConvThreads) void k_conv_step(ConvArgs a, int64_t NG) {
  const int64_t gid = (int64_t)blockIdx.x * kConvThreads + threadIdx.x;
  if (gid >= a.Bt * NG) return;
  const int64_t g = gid % NG, b = gid / NG;
  const int64_t c0 = g * VEC, D = a.D;
  T* st = reinterpret_cast<T*>(a.state_out) + (b * D + c0) * (K - 1);  // VEC*(K-1) contiguous
  // window element e = v*(K-1) + j, moved in VEC-element pieces
  float flat[K - 1][VEC];
#pragma unroll
  for (int m = 0; m < K - 1; ++m) load_vec<T, VEC>(st + m * VEC, flat[m]);
  float xp[K][VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v)
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
      const int e = v * (K - 1) + j;
      xp[j][v] = flat[e / VEC][e % VEC];
    }
  load_vec<T, VEC>(reinterpret_cast<const T*>(a.x) + b * D + c0, xp[K - 1]);
  float w[VEC][K], bs[VEC];
  load_weights<K, VEC>(a, c0, w, bs);
  float out[VEC];
  conv_point<K, VEC>(w, bs, xp, a.silu, out);
  store_vec<T, VEC>(reinterpret_cast<T*>(a.y) + b * D + c0, out);
  // shift: the oldest input drops out, x_t enters as the newest
#pragma unroll
  for (int v = 0; v < VEC; ++v)
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
      const int e = v * (K - 1) + j;
      flat[e / VEC][e % VEC] = xp[j + 1][v];
    }
#pragma unroll
  for (int m = 0; m < K - 1; ++m) store_vec<T, VEC>(st + m * VEC, flat[m]);
}

inline unsigned blocks_for(int64_t threads) {
  return (unsigned)((threads + kConvThreads - 1) / kConvThreads);
}

template <typename T, int K, int VEC>
hipError_t launch_kv(const ConvArgs& a, bool step, hipStream_t stream) {
  const int64_t NG = (a.D + VEC - 1) / VEC;
  if (step) {
    hipLaunchKernelGGL((k_conv_step<T, K, VEC>), dim3(blocks_for(a.Bt * NG)), dim3(kConvThreads),
                       0, stream, a, NG);
  } else {
    const int64_t NR = a.T > 0 ? (a.T + kConvRun - 1) / kConvRun : 1;
    hipLaunchKernelGGL((k_conv<T, K, VEC, kConvRun>), dim3(blocks_for(a.Bt * NR * NG)),
                       dim3(kConvThreads), 0, stream, a, NG, NR);
  }
  return hipGetLastError();
}

template <typename T, int K>
hipError_t launch_k(const ConvArgs& a, bool step, hipStream_t stream) {
  constexpr int VEC = 16 / sizeof(T);
  if (a.D % VEC == 0) return launch_kv<T, K, VEC>(a, step, stream);
  return launch_kv<T, K, 1>(a, step, stream);
}

template <typename T>
hipError_t launch_t(const ConvArgs& a, bool step, hipStream_t stream) {
  switch (a.K) {
    case 2: return launch_k<T, 2>(a, step, stream);
    case 3: return launch_k<T, 3>(a, step, stream);
    case 4: return launch_k<T, 4>(a, step, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool conv_width_supported(int64_t K) { return K >= 2 && K <= 4; }

hipError_t launch_conv(const ConvArgs& a, bool io_bf16, bool step, hipStream_t stream) {
  return io_bf16 ? launch_t<bf16>(a, step, stream) : launch_t<float>(a, step, stream);
}

}  // namespace ssd
