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
// A thread owns VEC = 4 adjacent channels of a token row (16 bytes of float32,
// 8 of bfloat16), so one wavefront instruction moves 1 KB or 512 bytes of a
// row.  In the sequence kernel the thread also owns a run of R = 8 tokens: it
// issues the loads of the k-1 inputs before the run and of the whole run at
// once, keeps them packed, then computes and stores R rows through a rolling
// window of k unpacked inputs.  The k-1 inputs before a run are re-read by
// its thread; the HBM read counters show 7-13% above the bytes of x for it.
// Measured on the 2.7B-shaped layer (4096 x 5376 bfloat16) against runs of
// 1, 2, 4, 16 and 32 tokens, 8 channels per lane, and a variant that issues
// the next run's loads before computing the current one, this was fastest.
// Only the thread of the first run of (b, channels) touches the window: it
// reads it before anything else and writes the outgoing window last, so the
// window may be updated in place.  Channel counts that are not a multiple of
// 4 (whose rows are then not aligned to the vectors) run with VEC = 1.
#include <type_traits>

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

constexpr int kConvThreads = 256;
constexpr int kConvRun = 8;  // tokens per thread in the sequence kernel
// Workgroup of the one-token kernel: 64 lanes.  At batch 64 of the 2.7B
// shape (5376 channels, 1344 lanes per row) one step is one short round of
// dependent loads and stores; 1344 workgroups of one wavefront spread it over
// every compute unit (4.52 -> 4.03 us per step from a HIP graph against 384
// workgroups of 256 lanes; 128 and 192 lanes: 4.09-4.11 us).
constexpr int kConvStepThreads = 64;

// VEC elements of T as they move: float4 (16 bytes), 4 x bfloat16 (8 bytes),
// or one T.
template <typename T, int VEC>
using raw_t = std::conditional_t<VEC == 1, T, std::conditional_t<sizeof(T) == 4, float4, bf16x4>>;

template <typename T, int VEC>
__device__ __forceinline__ raw_t<T, VEC> load_raw(const T* p) {
  static_assert(VEC == 1 || VEC == 4, "rows move in pieces of 4 channels");
  return *reinterpret_cast<const raw_t<T, VEC>*>(p);
}

template <typename T, int VEC>
__device__ __forceinline__ void unpack(const raw_t<T, VEC>& r, float (&v)[VEC]) {
  if constexpr (VEC == 1) {
    v[0] = to_f32(r);
  } else if constexpr (sizeof(T) == 4) {
    v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (float)r[e];
  }
}

template <typename T, int VEC>
__device__ __forceinline__ void load_vec(const T* p, float (&v)[VEC]) {
  unpack<T, VEC>(load_raw<T, VEC>(p), v);
}

template <typename T, int VEC>
__device__ __forceinline__ void store_vec(T* p, const float (&v)[VEC]) {
  if constexpr (VEC == 1) {
    p[0] = to_io<T>(v[0]);
  } else if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    bf16x4 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = (bf16)v[e];  // round to nearest even
    *reinterpret_cast<bf16x4*>(p) = h;
  }
}

// The same for y, which nothing re-reads: non-temporal stores (no cache
// allocation for the stream).
template <typename T, int VEC>
__device__ __forceinline__ void store_vec_stream(T* p, const float (&v)[VEC]) {
  if constexpr (VEC == 1) {
    __builtin_nontemporal_store(to_io<T>(v[0]), p);
  } else if constexpr (sizeof(T) == 4) {
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(p));
  } else {
    bf16x4 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = (bf16)v[e];  // round to nearest even
    __builtin_nontemporal_store(__builtin_bit_cast(uint64_t, h), reinterpret_cast<uint64_t*>(p));
  }
}

// silu(z) = z * logistic(z), logistic(z) = 1 / (1 + 2^(-z log2 e)) on the
// hardware base-2 exponential and reciprocal (about 1 ulp each; the
// accurate library exp and IEEE division cost some 30 instructions per
// element and made the layer bound by vector arithmetic instead of memory).
// Large negative z: 2^(+big) = inf, reciprocal 0, result -0; large positive
// z: the exponential flushes to 0 and the result is z.
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

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

// grid (ceil(NG / 64), ceil(NR / 4), Bt), 256 threads: lane -> VEC channels,
// wavefront -> run of R tokens; no integer division on the device
template <typename T, int K, int VEC, int R>
__global__ __launch_bounds__(kConvThreads) void k_conv(ConvArgs a, int32_t NG, int32_t NR) {
  static_assert(R >= K - 1, "only the first run may reach into the cached window");
  const int32_t g = (int32_t)blockIdx.x * 64 + (threadIdx.x & 63);
  const int32_t run = (int32_t)blockIdx.y * (kConvThreads / 64) + (threadIdx.x >> 6);
  if (g >= NG || run >= NR) return;
  const int64_t b = blockIdx.z;
  const int64_t c0 = (int64_t)g * VEC, D = a.D, nT = a.T;
  const int64_t t0 = (int64_t)run * R;
  const int tn = (int)(nT - t0 < R ? nT - t0 : R);  // tokens of this run (0 only when nT == 0)
  const T* xb = reinterpret_cast<const T*>(a.x) + b * nT * D + c0;
  const T* win = a.state_in ? reinterpret_cast<const T*>(a.state_in) + (b * D + c0) * (K - 1)
                            : nullptr;

  // the k-1 inputs before the run: earlier tokens, or the cached window
  raw_t<T, VEC> rh[K - 1];
  float hf[K - 1][VEC];
#pragma unroll
  for (int j = 0; j < K - 1; ++j) {
    const int64_t tt = t0 - (K - 1) + j;
    if (tt >= 0) {
      rh[j] = load_raw<T, VEC>(xb + tt * D);
    } else {
#pragma unroll
      for (int v = 0; v < VEC; ++v) hf[j][v] = win ? to_f32(win[v * (K - 1) + (K - 1) + tt]) : 0.0f;
    }
  }
  // An empty sequence launches one run with no tokens, which only hands the
  // window on: it reads no x and writes no y.
  if (tn > 0) {
    // the run, issued at once and kept packed until used: tokens past the
    // end re-read the last one and are not stored
    raw_t<T, VEC> rx[R];
#pragma unroll
    for (int t = 0; t < R; ++t) rx[t] = load_raw<T, VEC>(xb + (t0 + (t < tn ? t : tn - 1)) * D);
    float w[VEC][K], bs[VEC];
    load_weights<K, VEC>(a, c0, w, bs);
    // rolling window of K unpacked inputs
    float xw[K][VEC];
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
      if (t0 - (K - 1) + j >= 0) unpack<T, VEC>(rh[j], hf[j]);
#pragma unroll
      for (int v = 0; v < VEC; ++v) xw[j][v] = hf[j][v];
    }
    T* yb = reinterpret_cast<T*>(a.y) + b * nT * D + c0;
    // The first token needs no condition (tn >= 1 here), so every path waits
    // for the loads there and the later tokens issue stores only.  (With the
    // first token under the condition, the compiler waited again before each
    // token, and such a wait counts the previous token's store too: 23 -> 20
    // us at 4096 x 5376.)
#pragma unroll
    for (int t = 0; t < R; ++t) {
      if (t == 0 || t < tn) {
        unpack<T, VEC>(rx[t], xw[K - 1]);
        float out[VEC];
        conv_point<K, VEC>(w, bs, xw, a.silu, out);
        store_vec_stream<T, VEC>(yb + (t0 + t) * D, out);
#pragma unroll
        for (int jj = 0; jj < K - 1; ++jj)
#pragma unroll
          for (int v = 0; v < VEC; ++v) xw[jj][v] = xw[jj + 1][v];
      }
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
            for (int v = 0; v < VEC; ++v) v4[v] = hf[jj][v];
          }
      }
#pragma unroll
      for (int v = 0; v < VEC; ++v) so[v * (K - 1) + j] = to_io<T>(v4[v]);
    }
  }
}

// grid (ceil(NG / 256), Bt): thread -> VEC channels of batch row b
template <typename T, int K, int VEC>
__global__ __launch_bounds__(kConvStepThreads) void k_conv_step(ConvArgs a, int32_t NG) {
  const int32_t g = (int32_t)blockIdx.x * kConvStepThreads + threadIdx.x;
  if (g >= NG) return;
  const int64_t b = blockIdx.y;
  const int64_t c0 = (int64_t)g * VEC, D = a.D;
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
  store_vec_stream<T, VEC>(reinterpret_cast<T*>(a.y) + b * D + c0, out);
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

template <typename T, int K, int VEC>
hipError_t launch_kv(const ConvArgs& a, bool step, hipStream_t stream) {
  const int64_t NG = (a.D + VEC - 1) / VEC;
  if (step) {
    const dim3 grid((unsigned)((NG + kConvStepThreads - 1) / kConvStepThreads), (unsigned)a.Bt);
    hipLaunchKernelGGL((k_conv_step<T, K, VEC>), grid, dim3(kConvStepThreads), 0, stream, a,
                       (int32_t)NG);
  } else {
    const int64_t NR = a.T > 0 ? (a.T + kConvRun - 1) / kConvRun : 1;
    const dim3 grid((unsigned)((NG + 63) / 64), (unsigned)((NR + 3) / 4), (unsigned)a.Bt);
    hipLaunchKernelGGL((k_conv<T, K, VEC, kConvRun>), grid, dim3(kConvThreads), 0, stream, a,
                       (int32_t)NG, (int32_t)NR);
  }
  return hipGetLastError();
}

template <typename T, int K>
hipError_t launch_k(const ConvArgs& a, bool step, hipStream_t stream) {
  constexpr int VEC = 4;
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

// grid limits: batch rows and groups of 4 runs index the 16-bit y/z grid
// dimensions, channel groups and run indices fit 32 bits
bool conv_shape_supported(int64_t Bt, int64_t T, int64_t D) {
  constexpr int64_t kMaxYZ = 65535;
  const int64_t NR = (T + kConvRun - 1) / kConvRun;
  return Bt <= kMaxYZ && (NR + 3) / 4 <= kMaxYZ && D <= (int64_t)INT32_MAX;
}

hipError_t launch_conv(const ConvArgs& a, bool io_bf16, bool step, hipStream_t stream) {
  return io_bf16 ? launch_t<bf16>(a, step, stream) : launch_t<float>(a, step, stream);
}

}  // namespace ssd
