// Chunked SSD scan (prefill) for gfx950, bfloat16 x/B/C/y: first version.
//
// Source: "Compiler-First State Space Duality and Portable O(1)
// Autoregressive Caching", Background (Eq. 3 and the inter-chunk recurrence
// after it), SSD properties ("diagonal state matrix": the decay over a chunk
// is the exponential of a segment-wise prefix sum of A*Delta; "chunked
// recurrence": parallel matrix work inside a chunk of L tokens, a light scan
// across chunks) and Implementation ("static masking": prefix sum,
// subtraction, mask and exponentiation fused around the contractions).
//
// Per (batch b, chunk c, head h), with d the clipped softplus step, a = d*A,
// cum_l = sum_{k<=l} a_k inside the chunk and X, B, C the chunk's rows:
//   phase 0  S_c   = sum_l exp(cum_last - cum_l) d_l x_l (x) B_l     [P x N]
//            alpha_c = exp(cum_last)
//   phase 1  h_c   = alpha_c h_{c-1} + S_c    (sequential over c; the state
//            entering chunk c, h_{c-1}, replaces S_c in the workspace)
//   phase 2  y_l   = sum_{j<=l} (C_l . B_j) exp(cum_l - cum_j) d_j x_j
//                  + exp(cum_l) C_l h_{c-1}^T + D x_l
// Contractions run on the matrix cores (MFMA); the decay matrix
// exp(cum_i - cum_j) is formed in registers, tile by tile, with the causal
// mask applied as a select before the exponential; nothing L x L is stored.
//
// Included once per io type by ssd_prefill_f32.hip / ssd_prefill_bf16.hip.
#pragma once

#include "ssd_prefill_common.h"

namespace ssd {
namespace prefill {
namespace {  // each io-type translation unit keeps its own copy

struct Unit {
  int64_t b, c, h, g;
};

__device__ __forceinline__ Unit unit_of(const ScanArgs& a) {
  // heads fastest, then chunks, then batch; XCD-aware so the heads of one
  // chunk (which share the chunk's B and C rows) run on the same XCD
  const int64_t u = xcd_remap(blockIdx.x, gridDim.x);
  Unit r;
  r.h = u % a.H;
  const int64_t bc = u / a.H;
  r.c = bc % a.Nc;
  r.b = bc / a.Nc;
  r.g = r.h / (a.H / a.G);
  return r;
}

// ---------------------------------------------------------------------------
// Phase 0: chunk summary states S_c = X^T diag(w) B, w_l = d_l exp(cum_last - cum_l)
// ---------------------------------------------------------------------------
template <typename T, int P, int N>
__global__ __launch_bounds__(kThreads) void k_chunk_state(ScanArgs a) {
  using M = Mfma<T>;
  constexpr int KB = 64;            // tokens per LDS stage
  constexpr int XS = KB + 8;        // LDS row stride (elements), keeps 16-byte alignment
  constexpr int TP = P / 16, TN = N / 16, TT = TP * TN;
  constexpr int TPW = (TT + 3) / 4; // output tiles per wavefront
  __shared__ float s_d[kMaxL], s_cum[kMaxL], s_w[kMaxL], s_wsum[4];
  __shared__ __attribute__((aligned(16))) T s_xt[P * XS];   // [p][token]
  __shared__ __attribute__((aligned(16))) T s_bt[N * XS];   // [n][token]

  const Unit u = unit_of(a);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  chunk_delta_cumsum(a, u.b, u.c, u.h, s_d, s_cum, s_wsum);
  const int64_t t0 = u.c * a.L;
  const int Lc = (int)min<int64_t>(a.L, a.T - t0);
  const float cum_last = s_cum[Lc - 1];
  for (int l = tid; l < (int)a.L; l += kThreads)
    s_w[l] = (l < Lc) ? s_d[l] * fast_exp(cum_last - s_cum[l]) : 0.0f;
  if (tid == 0) a.ws_alpha[(u.b * a.H + u.h) * a.Nc + u.c] = fast_exp(cum_last);
  __syncthreads();

  f32x4 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const T* xg = reinterpret_cast<const T*>(a.x);
  const T* Bg = reinterpret_cast<const T*>(a.B);
  const int q = lane >> 4, r16 = lane & 15;
  for (int kb0 = 0; kb0 < Lc; kb0 += KB) {
    // stage the token block transposed: s_xt[p][k] = x[t0+kb0+k][p] * w, s_bt[n][k] = B[..][n]
    for (int e = tid; e < KB * P; e += kThreads) {
      const int k = e / P, p = e % P;
      float v = 0.0f;
      if (kb0 + k < Lc)
        v = to_f32(xg[((u.b * a.T + t0 + kb0 + k) * a.H + u.h) * P + p]) * s_w[kb0 + k];
      s_xt[p * XS + k] = to_io<T>(v);
    }
    for (int e = tid; e < KB * N; e += kThreads) {
      const int k = e / N, n = e % N;
      T v = to_io<T>(0.0f);
      if (kb0 + k < Lc) v = Bg[((u.b * a.T + t0 + kb0 + k) * a.G + u.g) * N + n];
      s_bt[n * XS + k] = v;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KB; ks += M::K) {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int tile = wave * TPW + i;
        if (tile < TT) {
          const int pt = tile / TN, nt = tile % TN;
          const auto fa = load_frag<T>(&s_xt[(pt * 16 + r16) * XS + ks + q * M::KPL]);
          const auto fb = load_frag<T>(&s_bt[(nt * 16 + r16) * XS + ks + q * M::KPL]);
          acc[i] = M::mma(fa, fb, acc[i]);
        }
      }
    }
    __syncthreads();
  }
  float* out = a.ws_state + ((u.b * a.H + u.h) * a.Nc + u.c) * (int64_t)(P * N);
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tile = wave * TPW + i;
    if (tile < TT) {
      const int pt = tile / TN, nt = tile % TN;
#pragma unroll
      for (int r = 0; r < 4; ++r) out[(pt * 16 + 4 * q + r) * N + nt * 16 + r16] = acc[i][r];
    }
  }
}

// ---------------------------------------------------------------------------
// Phase 2: chunk outputs.
//   y_i = exp(cum_i) C_i h_{c-1}^T + sum_{j<=i} (C_i . B_j) exp(cum_i - cum_j) d_j x_j + D x_i
// Row tiles of 16 tokens are dealt to the 4 wavefronts in a snake order
// (0 1 2 3 3 2 1 0 ...) so that the triangular work is balanced.  The score
// tile is computed transposed (S^T = B C^T) so that its accumulator layout is
// directly the A operand of the following (S o decay) X product.
// ---------------------------------------------------------------------------
template <typename T, int P, int N, int RT>
__global__ __launch_bounds__(kThreads) void k_chunk_out(ScanArgs a) {
  using M = Mfma<T>;
  constexpr int JB = 64;            // key tokens per LDS stage
  constexpr int TP = P / 16;
  constexpr int HS = N + 8;         // row strides (elements), 16-byte aligned rows
  constexpr int BS = N + 8;
  constexpr int XS = JB + 8;
  constexpr int NK = N / M::K;      // MFMA k-steps over the state dimension
  __shared__ float s_d[kMaxL], s_cum[kMaxL], s_wsum[4];
  __shared__ __attribute__((aligned(16))) T s_h[P * HS];    // h_{c-1}[p][n]
  __shared__ __attribute__((aligned(16))) T s_b[JB * BS];   // B[j][n]
  __shared__ __attribute__((aligned(16))) T s_xt[P * XS];   // x[j][p] transposed

  const Unit u = unit_of(a);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  chunk_delta_cumsum(a, u.b, u.c, u.h, s_d, s_cum, s_wsum);
  const int64_t t0 = u.c * a.L;
  const int Lc = (int)min<int64_t>(a.L, a.T - t0);
  const int nrt = (Lc + 15) / 16;

  const float* hp = a.ws_state + ((u.b * a.H + u.h) * a.Nc + u.c) * (int64_t)(P * N);
  for (int e = tid; e < P * N; e += kThreads) s_h[(e / N) * HS + e % N] = to_io<T>(hp[e]);
  __syncthreads();

  const T* xg = reinterpret_cast<const T*>(a.x);
  const T* Bg = reinterpret_cast<const T*>(a.B);
  const T* Cg = reinterpret_cast<const T*>(a.C);
  // C rows of token t (this chunk), as a k-fragment at state offset ks
  auto c_frag = [&](int row, int ks) -> typename M::frag {
    if (row < Lc) return load_frag<T>(&Cg[((u.b * a.T + t0 + row) * a.G + u.g) * N + ks + q * M::KPL]);
    typename M::frag z;
    if constexpr (M::KPL == 1) z = 0.0f; else for (int s = 0; s < M::KPL; ++s) z[s] = to_io<T>(0.0f);
    return z;
  };

  f32x4 acc[RT][TP];
  // inter-chunk term: acc = exp(cum_i) * (C_i . h_{c-1}[p])
#pragma unroll
  for (int k = 0; k < RT; ++k) {
    const int I = row_tile_of(wave, k);
#pragma unroll
    for (int pt = 0; pt < TP; ++pt) acc[k][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (I < nrt) {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const auto fc = c_frag(16 * I + r16, kk * M::K);
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) {
          const auto fh = load_frag<T>(&s_h[(pt * 16 + r16) * HS + kk * M::K + q * M::KPL]);
          acc[k][pt] = M::mma(fc, fh, acc[k][pt]);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * q + r;
        const float sc = (i < Lc) ? fast_exp(s_cum[i]) : 0.0f;
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) acc[k][pt][r] *= sc;
      }
    }
  }

  // intra-chunk term, one block of JB key tokens at a time
  const int njb = (Lc + JB - 1) / JB;
  for (int jb = 0; jb < njb; ++jb) {
    const int j_base = jb * JB;
    __syncthreads();
    for (int e = tid; e < JB * N; e += kThreads) {
      const int j = e / N, n = e % N;
      T v = to_io<T>(0.0f);
      if (j_base + j < Lc) v = Bg[((u.b * a.T + t0 + j_base + j) * a.G + u.g) * N + n];
      s_b[j * BS + n] = v;
    }
    for (int e = tid; e < JB * P; e += kThreads) {
      const int j = e / P, p = e % P;
      T v = to_io<T>(0.0f);
      if (j_base + j < Lc) v = xg[((u.b * a.T + t0 + j_base + j) * a.H + u.h) * P + p];
      s_xt[p * XS + j] = v;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < RT; ++k) {
      const int I = row_tile_of(wave, k);
      if (I >= nrt || 16 * I + 15 < j_base) continue;
      typename M::frag fc[NK];
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) fc[kk] = c_frag(16 * I + r16, kk * M::K);
      const int i = 16 * I + r16;           // this lane's query row in the score tiles
      const float cum_i = s_cum[i < Lc ? i : Lc - 1];
#pragma unroll
      for (int jp = 0; jp < JB / 32; ++jp) {
        const int j0 = j_base + jp * 32;    // first key of the pair of 16-wide tiles
        if (j0 > 16 * I + 15) continue;     // whole pair above the diagonal
        f32x4 st0 = {0.f, 0.f, 0.f, 0.f}, st1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          const auto fb0 = load_frag<T>(&s_b[(jp * 32 + r16) * BS + kk * M::K + q * M::KPL]);
          const auto fb1 = load_frag<T>(&s_b[(jp * 32 + 16 + r16) * BS + kk * M::K + q * M::KPL]);
          st0 = M::mma(fb0, fc[kk], st0);   // st0[r] = S[i][j0 + 4q + r]
          st1 = M::mma(fb1, fc[kk], st1);   // st1[r] = S[i][j0 + 16 + 4q + r]
        }
        float m0[4], m1[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ja = j0 + 4 * q + r, jc = j0 + 16 + 4 * q + r;
          m0[r] = (ja <= i) ? st0[r] * fast_exp(cum_i - s_cum[ja]) * s_d[ja] : 0.0f;
          m1[r] = (jc <= i) ? st1[r] * fast_exp(cum_i - s_cum[jc]) * s_d[jc] : 0.0f;
        }
        const int jo = jp * 32 + 4 * q;     // column of x^T holding key j0 + 4q
        if constexpr (M::KPL == 8) {
          bf16x8 fa;
#pragma unroll
          for (int r = 0; r < 4; ++r) { fa[r] = (bf16)m0[r]; fa[4 + r] = (bf16)m1[r]; }
#pragma unroll
          for (int pt = 0; pt < TP; ++pt) {
            const T* row = &s_xt[(pt * 16 + r16) * XS];
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + jo);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + jo + 16);
            bf16x8 fx;
#pragma unroll
            for (int r = 0; r < 4; ++r) { fx[r] = lo[r]; fx[4 + r] = hi[r]; }
            acc[k][pt] = M::mma(fa, fx, acc[k][pt]);
          }
        } else {
#pragma unroll
          for (int pt = 0; pt < TP; ++pt) {
            const T* row = &s_xt[(pt * 16 + r16) * XS];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              acc[k][pt] = M::mma(m0[r], row[jo + r], acc[k][pt]);
              acc[k][pt] = M::mma(m1[r], row[jo + 16 + r], acc[k][pt]);
            }
          }
        }
      }
    }
  }

  // skip term and store
  const float Dh = a.D ? a.D[u.h] : 0.0f;
  T* yg = reinterpret_cast<T*>(a.y);
#pragma unroll
  for (int k = 0; k < RT; ++k) {
    const int I = row_tile_of(wave, k);
    if (I >= nrt) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * I + 4 * q + r;
      if (i >= Lc) continue;
      const int64_t rowoff = ((u.b * a.T + t0 + i) * a.H + u.h) * P;
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) {
        const int p = pt * 16 + r16;
        const float v = acc[k][pt][r] + Dh * to_f32(xg[rowoff + p]);
        yg[rowoff + p] = to_io<T>(v);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side launch
// ---------------------------------------------------------------------------
template <typename T, int P, int N>
hipError_t launch_pn(const ScanArgs& a, hipStream_t stream, hipEvent_t* ev) {
  hipError_t e;
  auto rec = [&](int k) -> hipError_t { return ev ? hipEventRecord(ev[k], stream) : hipSuccess; };
  const int64_t units = a.Bt * a.Nc * a.H;
  // phase 0 (C B^T) is computed inside the output kernel on this path
  if ((e = rec(0)) != hipSuccess) return e;
  if ((e = rec(1)) != hipSuccess) return e;
  hipLaunchKernelGGL((k_chunk_state<T, P, N>), dim3((unsigned)units), dim3(kThreads), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = rec(2)) != hipSuccess) return e;
  if ((e = launch_state_pass(a, P, N, stream)) != hipSuccess) return e;
  if ((e = rec(3)) != hipSuccess) return e;
  const int rt_needed = (int)((a.L + 63) / 64);
  if (rt_needed <= 4) {
    hipLaunchKernelGGL((k_chunk_out<T, P, N, 4>), dim3((unsigned)units), dim3(kThreads), 0, stream, a);
  } else {
    if constexpr (P <= 64) {
      hipLaunchKernelGGL((k_chunk_out<T, P, N, 8>), dim3((unsigned)units), dim3(kThreads), 0, stream, a);
    } else {
      return hipErrorInvalidValue;
    }
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return rec(4);
}

template <typename T, int P>
hipError_t launch_p(const ScanArgs& a, int N, hipStream_t s, hipEvent_t* ev) {
  switch (N) {
    case 16:
      if constexpr (Mfma<T>::K <= 16) return launch_pn<T, P, 16>(a, s, ev);
      else return hipErrorInvalidValue;
    case 32: return launch_pn<T, P, 32>(a, s, ev);
    case 64: return launch_pn<T, P, 64>(a, s, ev);
    case 128: return launch_pn<T, P, 128>(a, s, ev);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_scan(const ScanArgs& a, int P, int N, hipStream_t s, hipEvent_t* ev) {
  switch (P) {
    case 16: return launch_p<T, 16>(a, N, s, ev);
    case 32: return launch_p<T, 32>(a, N, s, ev);
    case 64: return launch_p<T, 64>(a, N, s, ev);
    case 128: return launch_p<T, 128>(a, N, s, ev);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace prefill
}  // namespace ssd
