// Gradients of the chunked scan for gfx950: the element-wise, transform and
// reduction kernels around the scans that ssd_chunk_scan_backward runs.
//
// Source: "Compiler-First State Space Duality and Portable O(1)
// Autoregressive Caching", Background (Eq. 2-3: the recurrence and its
// chunked dual form) and Implementation (softplus and clip on Delta).
//
// The adjoint G_t = dL/dh_t of h_t = abar_t h_{t-1} + d_t x_t (x) B_t,
// y_t = h_t C_t + D x_t runs backwards in time:
//   G_t = dy_t (x) C_t + abar_{t+1} G_{t+1},   G_{T-1} = dfinal + dy_{T-1} (x) C_{T-1}.
// Every product of G with B_t or x_t is therefore the same chunked scan run
// over reversed time, with the decay of step t+1 at reversed position T-1-t
// and the input divided by that decay step's Delta (the scan multiplies its
// input by its Delta).  The host launches:
//   forward F0 in float32 (the entering states H_c and C B^T stay in its workspace)
//   scan R1 (reversed, float32): input dy/Delta', B' = C, C' = B  -> sum_n G[p,n] B_t[n];
//        pad = Nc L - T empty leading positions align its chunks with F0's, so that
//        its entering states are G at the forward chunk boundaries
//   scan F2 (forward):   input B (per head), B'' = x, C'' = dy   -> sum_p dy_t[p] h_t[p,n]
//   scan R3 (reversed):  input C/Delta', B''' = dy, C''' = x     -> sum_p G[p,n] x_t[p]
// and these kernels form the rest:
//   dx_t = d_t (R1)_t + D dy_t;  dB = sum over a group's heads of d_t (R3)_t;
//   dC = sum over a group's heads of (F2)_t;  dD = sum_t dy_t . x_t;
//   dL/d(d_t A) = abar_t sum_{p,n} G_t h_{t-1}, per forward chunk c (token t,
//   chunk-local cumulative log-decay cum, in double):
//     sum_{i >= t > j in c} Q_ij                 Q_ij = (dy_i.x_j)(C_i.B_j) e^{cum_i - cum_j} d_j
//   + sum_{i >= t in c} e^{cum_i} dy_i . (C_i H_c^T)
//   + sum_{j < t in c} d_j e^{cum_last - cum_j} x_j . (B_j Ghat_c^T)
//   + e^{cum_last} <Ghat_c, H_c>,                Ghat_c = dL/dh at the end of chunk c
//   (no term of this sum cancels against another across the sequence);
//   dd_t = A dL/d(d_t A) + x_t . (R1)_t;  ddt_t = dd_t softplus'(z_t) where Delta
//   is not clipped;  dA = sum_t d_t dL/d(d_t A);  dh0 = abar_0 (final state of R1).
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

constexpr int kBwdThreads = 256;

template <typename T>
__device__ __forceinline__ T io_of(float v) { return to_io<T>(v); }

__device__ __forceinline__ float delta_at(const BwdArgs& a, int64_t b, int64_t t, int64_t h) {
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
  return delta_of(a.dt[(b * a.T + t) * a.H + h] + bias, a.softplus, a.dt_min, a.dt_max);
}

// One wavefront per (b, t, h) row: Delta, the reversed Delta', and the
// reversed / replicated / rescaled inputs of the three scans.  The pad
// positions of R1 are zeroed by k_bwd_zero_pad.
template <typename T>
__global__ __launch_bounds__(kBwdThreads) void k_bwd_prep(BwdArgs a) {
  const uint32_t row32 = blockIdx.x * (kBwdThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if ((int64_t)row32 >= a.Bt * a.T * a.H) return;
  // rows fit 32 bits (checked on the host): 32-bit divisions
  const uint32_t H32 = (uint32_t)a.H, T32 = (uint32_t)a.T, hpg32 = (uint32_t)(a.H / a.G);
  const uint32_t bt32 = row32 / H32;
  const int64_t row = row32, h = row32 - bt32 * H32, t = bt32 % T32, b = bt32 / T32;
  const int64_t hpg = hpg32, g = (uint32_t)h / hpg32;
  const int64_t tr = a.T - 1 - t;                     // reversed position of token t (R3)
  const int64_t T1 = a.T + a.pad, tr1 = a.pad + tr;    // R1: after pad empty positions
  const int P = a.P, N = a.N;
  const float d = delta_at(a, b, t, h);
  const bool has_next = t + 1 < a.T;
  const float dn = has_next ? delta_at(a, b, t + 1, h) : 1.0f;
  if (lane == 0) {
    a.wd[row] = d;
    // Delta' at reversed position T - t is d_t (positions 1..T-1); position 0 gets 0
    if (t >= 1) a.dtr[(b * a.T + (a.T - t)) * a.H + h] = d;
    else a.dtr[(b * a.T + 0) * a.H + h] = 0.0f;
    // R1: the same one position later than its pad; the pad and its first position get 0
    if (t >= 1) a.dtr1[(b * T1 + (a.pad + a.T - t)) * a.H + h] = d;
    else
      for (int64_t k = 0; k <= a.pad; ++k) a.dtr1[(b * T1 + k) * a.H + h] = 0.0f;
  }
  const T* x = reinterpret_cast<const T*>(a.x);
  const T* dy = reinterpret_cast<const T*>(a.dy);
  const T* Bm = reinterpret_cast<const T*>(a.B);
  const T* Cm = reinterpret_cast<const T*>(a.C);
  const int64_t rp = ((b * a.T + t) * a.H + h) * P, rpr = ((b * a.T + tr) * a.H + h) * P;
  const int64_t rpr1 = ((b * T1 + tr1) * a.H + h) * P;
  const int64_t rn = ((b * a.T + t) * a.H + h) * N, rnr = ((b * a.T + tr) * a.H + h) * N;
  const int64_t gn = ((b * a.T + t) * a.G + g) * N;
  const int64_t gnr1 = ((b * T1 + tr1) * a.G + g) * N;
  for (int p = lane; p < P; p += 64) {
    const float v = to_f32(dy[rp + p]);
    // input of R1 at reversed position T-1-t: dy_t / Delta_{t+1} (0 for t = T-1)
    a.r1_x[rpr1 + p] = has_next ? v / dn : 0.0f;
    reinterpret_cast<T*>(a.r3_b)[rpr + p] = dy[rp + p];
    reinterpret_cast<T*>(a.r3_c)[rpr + p] = x[rp + p];
    if (a.x32) a.x32[rp + p] = to_f32(x[rp + p]);
  }
  for (int n = lane; n < N; n += 64) {
    const T bv = Bm[gn + n], cv = Cm[gn + n];
    reinterpret_cast<T*>(a.f2_x)[rn + n] = bv;
    reinterpret_cast<T*>(a.r3_x)[rnr + n] = io_of<T>(has_next ? to_f32(cv) / dn : 0.0f);
    if (h % hpg == 0) {
      a.r1_b[gnr1 + n] = to_f32(cv);
      a.r1_c[gnr1 + n] = to_f32(bv);
      if (a.b32) {
        a.b32[gn + n] = to_f32(bv);
        a.c32[gn + n] = to_f32(cv);
      }
    }
  }
}

// Initial states of the reversed scans (dfinal + dy_{T-1} (x) C_{T-1}, as
// [P][N] for R1 and [N][P] for R3) and of F2 (initial_state transposed).
template <typename T>
__global__ __launch_bounds__(kBwdThreads) void k_bwd_init_states(BwdArgs a) {
  const int64_t e = (int64_t)blockIdx.x * kBwdThreads + threadIdx.x;
  const int P = a.P, N = a.N;
  if (e >= a.Bt * a.H * P * N) return;
  const int64_t n = e % N, p = (e / N) % P, bh = e / ((int64_t)P * N);
  const int64_t h = bh % a.H, b = bh / a.H, g = h / (a.H / a.G);
  const int64_t tl = a.T - 1;
  const float dyv = to_f32(reinterpret_cast<const T*>(a.dy)[((b * a.T + tl) * a.H + h) * P + p]);
  const float cv = to_f32(reinterpret_cast<const T*>(a.C)[((b * a.T + tl) * a.G + g) * N + n]);
  const float v = __fmaf_rn(dyv, cv, a.dfinal ? a.dfinal[e] : 0.0f);
  a.r1_h0[e] = v;
  const int64_t et = (bh * N + n) * P + p;   // [b][h][n][p]
  a.r3_h0[et] = v;
  if (a.h0) a.f2_h0[et] = a.h0[e];
}

// One wavefront per (b, t, h): dx, the input-scale part of the Delta gradient
// (x . R1) and the per-token part of dD.
template <typename T>
__global__ __launch_bounds__(kBwdThreads) void k_bwd_dx(BwdArgs a) {
  const int64_t row = (int64_t)blockIdx.x * (kBwdThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.Bt * a.T * a.H) return;
  const int64_t h = row % a.H, bt = row / a.H, t = bt % a.T, b = bt / a.T;
  const int P = a.P;
  const float d = a.wd[row];
  const float Dh = a.D ? a.D[h] : 0.0f;
  const int64_t rp = row * P;
  const int64_t rpr1 = ((b * (a.T + a.pad) + (a.pad + a.T - 1 - t)) * a.H + h) * P;
  const T* x = reinterpret_cast<const T*>(a.x);
  const T* dy = reinterpret_cast<const T*>(a.dy);
  float s_din = 0.0f, s_dd = 0.0f;
  for (int p = lane; p < P; p += 64) {
    const float xv = to_f32(x[rp + p]), dyv = to_f32(dy[rp + p]);
    const float gb = a.r1_y[rpr1 + p];               // sum_n G[p,n] B_t[n]
    a.dx[rp + p] = __fmaf_rn(Dh, dyv, d * gb);
    s_din = __fmaf_rn(xv, gb, s_din);
    s_dd = __fmaf_rn(dyv, xv, s_dd);
  }
  s_din = group_sum(s_din, 64);
  s_dd = group_sum(s_dd, 64);
  if (lane == 0) {
    a.ddin[row] = s_din;
    a.dDp[row] = s_dd;
  }
}

// One workgroup per (b, h): the dt gradient and this (b, h)'s parts of dA,
// ddt_bias and dD (block sums in a fixed order).
__global__ __launch_bounds__(kBwdThreads) void k_bwd_dt(BwdArgs a) {
  const int64_t bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float Ah = a.A[h];
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
  __shared__ float red[3][kBwdThreads / 64];
  float pA = 0.0f, pB = 0.0f, pD = 0.0f;
  for (int64_t t = tid; t < a.T; t += kBwdThreads) {
    const int64_t row = (b * a.T + t) * a.H + h;
    const float da = a.dlda[row];
    const float z = a.dt[row] + bias;
    const float pre = a.softplus ? (fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z)))) : z;
    float gate = (pre >= a.dt_min && pre <= a.dt_max) ? 1.0f : 0.0f;
    if (a.softplus) gate *= 1.0f / (1.0f + expf(-z));
    const float g = __fmaf_rn(Ah, da, a.ddin[row]) * gate;
    a.ddt[row] = g;
    pA = __fmaf_rn(a.wd[row], da, pA);
    pB += g;
    pD += a.dDp[row];
  }
  pA = group_sum(pA, 64);
  pB = group_sum(pB, 64);
  pD = group_sum(pD, 64);
  if (lane == 0) {
    red[0][wave] = pA;
    red[1][wave] = pB;
    red[2][wave] = pD;
  }
  __syncthreads();
  if (tid < 3) {
    float s = 0.0f;
    for (int w = 0; w < kBwdThreads / 64; ++w) s += red[tid][w];
    a.part[tid * a.Bt * a.H + bh] = s;
  }
}

// Inclusive prefix sum over the 256 threads of a workgroup (fixed order).
__device__ __forceinline__ float block_inclusive_scan(float v, float* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float inc = wave_inclusive_scan(v);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  float before = 0.0f;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  __syncthreads();
  return inc + before;
}

template <typename T>
__device__ __forceinline__ float4 ld4_io(const T* p, bool ok) {
  if constexpr (sizeof(T) == 4) {
    return ok ? *reinterpret_cast<const float4*>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
  } else {
    if (!ok) return make_float4(0.f, 0.f, 0.f, 0.f);
    const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
    return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
  }
}

__device__ __forceinline__ f32x4 mfma4(float4 a, float4 b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, c, 0, 0, 0);
}

// One workgroup per (b, forward chunk c, h): dL/d(Delta_t A) of the chunk's
// tokens (the four terms in the header).  Matrix-core tiles (16x16x4 fp32,
// lane l: A[l%16][k], B[k][l%16], D[4(l/16)+r][l%16], k = 16 blk + 4(l/16) + kk):
//   dy x^T over P for Q, C H_c^T and B Ghat_c^T over N for the state terms.
// Row sums of Q are kept per (row tile, column tile) and added in column
// order; column sums are owned by one wavefront per column tile: the result
// does not depend on scheduling.
template <typename T, int P, int N>
__global__ __launch_bounds__(kBwdThreads) void k_bwd_dlda(BwdArgs a) {
  constexpr int LMAX = kBwdThreads, NRT = LMAX / 16;
  __shared__ double s_cum[LMAX];
  __shared__ double s_dw[kBwdThreads / 64];
  __shared__ float s_d[LMAX];
  __shared__ float s_rowp[NRT][NRT][16];
  __shared__ float s_col[LMAX], s_q[LMAX], s_r[LMAX];
  __shared__ float s_w[kBwdThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, q = lane >> 4, r16 = lane & 15;
  const int64_t u = blockIdx.x;
  const int64_t h = u % a.H, bc = u / a.H, c = bc % a.Nc, b = bc / a.Nc;
  const int64_t g = h / (a.H / a.G);
  const int64_t L = a.L, t0 = c * L;
  const int Lc = (int)(a.T - t0 < L ? a.T - t0 : L);
  const int nrt = (Lc + 15) / 16;
  const float Ah = a.A[h];

  // Delta and the chunk's cumulative log-decay, in double
  {
    const float dv = tid < Lc ? a.wd[(b * a.T + t0 + tid) * a.H + h] : 0.0f;
    s_d[tid] = dv;
    double v = (double)dv * (double)Ah;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double o = __shfl_up(v, off, 64);
      if (lane >= off) v += o;
    }
    if (lane == 63) s_dw[wave] = v;
    __syncthreads();
    double before = 0.0;
    for (int w = 0; w < wave; ++w) before += s_dw[w];
    s_cum[tid] = v + before;
    s_col[tid] = 0.0f;
    s_q[tid] = 0.0f;
    s_r[tid] = 0.0f;
  }
  __syncthreads();
  const double cum_last = s_cum[Lc - 1];

  const T* xg = reinterpret_cast<const T*>(a.x) + ((b * a.T + t0) * a.H + h) * P;
  const T* dyg = reinterpret_cast<const T*>(a.dy) + ((b * a.T + t0) * a.H + h) * P;
  const T* Bg = reinterpret_cast<const T*>(a.B) + ((b * a.T + t0) * a.G + g) * N;
  const T* Cg = reinterpret_cast<const T*>(a.C) + ((b * a.T + t0) * a.G + g) * N;
  const int64_t xrs = a.H * P, brs = a.G * N;

  // ---- Q_ij, i > j: row sums per (I, J) tile, column sums per column tile ----
  const float* S = a.fwd_cb + ((b * a.Nc + c) * a.G + g) * L * L;
  for (int J = wave; J < nrt; J += kBwdThreads / 64) {
    const int j = 16 * J + r16;
    const bool jok = j < Lc;
    const float dj = jok ? s_d[j] : 0.0f;
    const double cj = s_cum[jok ? j : 0];
    // this lane's x row (column j of the tiles), loaded once for the column tile
    float4 xr[P / 16];
#pragma unroll
    for (int pb = 0; pb < P / 16; ++pb)
      xr[pb] = ld4_io<T>(xg + (jok ? j : Lc - 1) * xrs + 16 * pb + 4 * q, jok);
    float colacc = 0.0f;
    for (int I = J; I < nrt; ++I) {
      const int ia = 16 * I + r16;
      float4 dr[P / 16];
#pragma unroll
      for (int pb = 0; pb < P / 16; ++pb)
        dr[pb] = ld4_io<T>(dyg + (ia < Lc ? ia : Lc - 1) * xrs + 16 * pb + 4 * q, ia < Lc);
      float sv[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int i = 16 * I + 4 * q + rr;
        sv[rr] = (jok && i > j && i < Lc) ? S[(int64_t)i * L + j] : 0.0f;
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int pb = 0; pb < P / 16; ++pb) acc = mfma4(dr[pb], xr[pb], acc);
      float colpart = 0.0f;
      float rowv[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int i = 16 * I + 4 * q + rr;
        float qv = 0.0f;
        if (jok && i > j && i < Lc) {
          const float dec = expf((float)(s_cum[i] - cj));
          qv = acc[rr] * sv[rr] * dec * dj;
        }
        rowv[rr] = qv;
        colpart += qv;
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) rowv[rr] = group_sum(rowv[rr], 16);
      if (r16 == 0) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) s_rowp[I][J][4 * q + rr] = rowv[rr];
      }
      colpart += __shfl_xor(colpart, 16, 64);
      colpart += __shfl_xor(colpart, 32, 64);
      colacc += colpart;
    }
    if (q == 0 && jok) s_col[j] = colacc;
  }

  // ---- state terms: C H_c^T against dy, B Ghat_c^T against x ----
  constexpr int64_t PN = (int64_t)P * N;
  const float* Hc = a.fwd_state + ((b * a.H + h) * a.Nc + c) * PN;
  const float* Gh = nullptr;
  float gs = 1.0f;
  if (c + 1 < a.Nc) {
    Gh = a.r1_state + ((b * a.H + h) * a.Nc + (a.Nc - 1 - c)) * PN;
    gs = expf(a.wd[(b * a.T + t0 + L) * a.H + h] * Ah);   // abar of the next chunk's first token
  } else if (a.dfinal) {
    Gh = a.dfinal + (b * a.H + h) * PN;
  }
  for (int I = wave; I < nrt; I += kBwdThreads / 64) {
    const int ia = 16 * I + r16;
    const bool iok = ia < Lc;
    // this lane's C and B rows (row i = 16 I + r16), loaded once for all p tiles
    float4 cr[N / 16], br[N / 16];
#pragma unroll
    for (int nb = 0; nb < N / 16; ++nb) {
      cr[nb] = ld4_io<T>(Cg + (iok ? ia : Lc - 1) * brs + 16 * nb + 4 * q, iok);
      br[nb] = ld4_io<T>(Bg + (iok ? ia : Lc - 1) * brs + 16 * nb + 4 * q, iok);
    }
    float qp[4] = {0.f, 0.f, 0.f, 0.f}, rp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int pt = 0; pt < P / 16; ++pt) {
      f32x4 ay = {0.f, 0.f, 0.f, 0.f}, ag = {0.f, 0.f, 0.f, 0.f};
      const float* hrow = Hc + (16 * pt + r16) * N + 4 * q;
#pragma unroll
      for (int nb = 0; nb < N / 16; ++nb)
        ay = mfma4(cr[nb], *reinterpret_cast<const float4*>(hrow + 16 * nb), ay);
      if (Gh) {
        const float* grow = Gh + (16 * pt + r16) * N + 4 * q;
#pragma unroll
        for (int nb = 0; nb < N / 16; ++nb)
          ag = mfma4(br[nb], *reinterpret_cast<const float4*>(grow + 16 * nb), ag);
      }
      // lane holds rows i = 16 I + 4 q + rr, column p = 16 pt + r16
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int i = 16 * I + 4 * q + rr;
        if (i < Lc) {
          qp[rr] = __fmaf_rn(ay[rr], to_f32(dyg[(int64_t)i * xrs + 16 * pt + r16]), qp[rr]);
          rp[rr] = __fmaf_rn(ag[rr], to_f32(xg[(int64_t)i * xrs + 16 * pt + r16]), rp[rr]);
        }
      }
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      qp[rr] = group_sum(qp[rr], 16);
      rp[rr] = group_sum(rp[rr], 16);
    }
    if (r16 == 0) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int i = 16 * I + 4 * q + rr;
        if (i < Lc) {
          s_q[i] = (float)exp(s_cum[i]) * qp[rr];
          s_r[i] = s_d[i] * gs * (float)exp(cum_last - s_cum[i]) * rp[rr];
        }
      }
    }
  }
  // s_c = e^{cum_last} <Ghat_c, H_c>
  float sc = 0.0f;
  if (Gh)
    for (int e = tid; e < P * N; e += kBwdThreads) sc = __fmaf_rn(Gh[e], Hc[e], sc);
  sc = group_sum(sc, 64);
  if (lane == 0) s_w[wave] = sc;
  __syncthreads();
  float s_c = 0.0f;
  for (int w = 0; w < kBwdThreads / 64; ++w) s_c += s_w[w];
  s_c *= gs * (float)exp(cum_last);
  __syncthreads();

  // ---- assemble: R_t = sum_{v<t} (col_v - row_v), suffix of q, prefix of r ----
  const int l = tid;
  float rowsum = 0.0f;
  if (l < Lc) {
    const int I = l >> 4;
    for (int J = 0; J <= I; ++J) rowsum += s_rowp[I][J][l & 15];
  }
  const float dv = l < Lc ? s_col[l] - rowsum : 0.0f;
  const float qv = s_q[l], rv = s_r[l];
  const float inc_d = block_inclusive_scan(dv, s_w);
  const float inc_q = block_inclusive_scan(qv, s_w);
  const float inc_r = block_inclusive_scan(rv, s_w);
  // totals: the last thread's inclusive sums
  __shared__ float s_tot;
  if (tid == kBwdThreads - 1) s_tot = inc_q;
  __syncthreads();
  if (l < Lc) {
    const float R = inc_d - dv;                 // sum over v < t
    const float Sq = s_tot - (inc_q - qv);      // sum over i >= t
    const float Pr = inc_r - rv;                // sum over j < t
    a.dlda[(b * a.T + t0 + l) * a.H + h] = R + Sq + Pr + s_c;
  }
}

// The pad positions of R1 (reversed positions 0 .. pad-1) hold no token.
__global__ __launch_bounds__(kBwdThreads) void k_bwd_zero_pad(BwdArgs a, int64_t per_b) {
  const int64_t e = (int64_t)blockIdx.x * kBwdThreads + threadIdx.x;
  if (e >= a.Bt * per_b) return;
  const int64_t b = e / per_b, r = e % per_b;
  const int64_t T1 = a.T + a.pad;
  if (r < a.pad * a.H * a.P) a.r1_x[b * T1 * a.H * a.P + r] = 0.0f;
  if (r < a.pad * a.G * a.N) {
    a.r1_b[b * T1 * a.G * a.N + r] = 0.0f;
    a.r1_c[b * T1 * a.G * a.N + r] = 0.0f;
  }
}

// dA, ddt_bias, dD: sums over the batch of the (b, h) parts (fixed order).
__global__ __launch_bounds__(kBwdThreads) void k_bwd_reduce_heads(BwdArgs a) {
  const int64_t h = (int64_t)blockIdx.x * kBwdThreads + threadIdx.x;
  if (h >= a.H) return;
  float s[3] = {0.0f, 0.0f, 0.0f};
  for (int64_t b = 0; b < a.Bt; ++b)
    for (int k = 0; k < 3; ++k) s[k] += a.part[k * a.Bt * a.H + b * a.H + h];
  a.dA[h] = s[0];
  if (a.ddt_bias_out) a.ddt_bias_out[h] = s[1];
  if (a.dD) a.dD[h] = s[2];
}

// dB and dC: sums over a group's heads (fixed order) of d_t R3 and of F2.
template <typename T>
__global__ __launch_bounds__(kBwdThreads) void k_bwd_dbdc(BwdArgs a) {
  const int64_t e = (int64_t)blockIdx.x * kBwdThreads + threadIdx.x;
  const int N = a.N;
  if (e >= a.Bt * a.T * a.G * N) return;
  const int64_t n = e % N, btg = e / N, g = btg % a.G, bt = btg / a.G, t = bt % a.T, b = bt / a.T;
  const int64_t hpg = a.H / a.G;
  const int64_t tr = a.T - 1 - t;
  const T* f2 = reinterpret_cast<const T*>(a.f2_y);
  const T* r3 = reinterpret_cast<const T*>(a.r3_y);
  float sb = 0.0f, sc = 0.0f;
  for (int64_t h = g * hpg; h < (g + 1) * hpg; ++h) {
    sc += to_f32(f2[((b * a.T + t) * a.H + h) * N + n]);
    sb = __fmaf_rn(a.wd[(b * a.T + t) * a.H + h], to_f32(r3[((b * a.T + tr) * a.H + h) * N + n]), sb);
  }
  a.dB[e] = sb;
  a.dC[e] = sc;
}

// dh0 = abar_0 * (final state of R1).
__global__ __launch_bounds__(kBwdThreads) void k_bwd_dh0(BwdArgs a) {
  const int64_t e = (int64_t)blockIdx.x * kBwdThreads + threadIdx.x;
  const int64_t PN = (int64_t)a.P * a.N;
  if (e >= a.Bt * a.H * PN) return;
  const int64_t bh = e / PN, h = bh % a.H, b = bh / a.H;
  const float ab0 = expf(a.wd[(b * a.T) * a.H + h] * a.A[h]);
  a.dh0[e] = ab0 * a.r1_final[e];
}

inline unsigned blocks_of(int64_t n, int64_t per) { return (unsigned)((n + per - 1) / per); }

template <typename T>
hipError_t launch_phase(const BwdArgs& a, int phase, hipStream_t s) {
  const int64_t rows = a.Bt * a.T * a.H;
  switch (phase) {
    case 0:
      hipLaunchKernelGGL(k_bwd_prep<T>, dim3(blocks_of(rows, kBwdThreads / 64)), dim3(kBwdThreads),
                         0, s, a);
      if (a.pad > 0) {
        const int64_t hp = a.pad * a.H * a.P, gn = a.pad * a.G * a.N;
        const int64_t per_b = hp > gn ? hp : gn;
        hipLaunchKernelGGL(k_bwd_zero_pad, dim3(blocks_of(a.Bt * per_b, kBwdThreads)),
                           dim3(kBwdThreads), 0, s, a, per_b);
      }
      hipLaunchKernelGGL(k_bwd_init_states<T>,
                         dim3(blocks_of(a.Bt * a.H * (int64_t)a.P * a.N, kBwdThreads)),
                         dim3(kBwdThreads), 0, s, a);
      break;
    case 1: {
      const dim3 grid((unsigned)(a.Bt * a.Nc * a.H));
      hipError_t e = hipErrorInvalidValue;
#define SSD_BWD_DLDA(PP, NN)                                                          \
  if (a.P == PP && a.N == NN) {                                                       \
    hipLaunchKernelGGL((k_bwd_dlda<T, PP, NN>), grid, dim3(kBwdThreads), 0, s, a);     \
    e = hipSuccess;                                                                   \
  }
      SSD_BWD_DLDA(16, 16) SSD_BWD_DLDA(16, 32) SSD_BWD_DLDA(16, 64) SSD_BWD_DLDA(16, 128)
      SSD_BWD_DLDA(32, 16) SSD_BWD_DLDA(32, 32) SSD_BWD_DLDA(32, 64) SSD_BWD_DLDA(32, 128)
      SSD_BWD_DLDA(64, 16) SSD_BWD_DLDA(64, 32) SSD_BWD_DLDA(64, 64) SSD_BWD_DLDA(64, 128)
      SSD_BWD_DLDA(128, 16) SSD_BWD_DLDA(128, 32) SSD_BWD_DLDA(128, 64) SSD_BWD_DLDA(128, 128)
#undef SSD_BWD_DLDA
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(k_bwd_dx<T>, dim3(blocks_of(rows, kBwdThreads / 64)), dim3(kBwdThreads),
                         0, s, a);
      hipLaunchKernelGGL(k_bwd_dt, dim3((unsigned)(a.Bt * a.H)), dim3(kBwdThreads), 0, s, a);
      hipLaunchKernelGGL(k_bwd_reduce_heads, dim3(blocks_of(a.H, kBwdThreads)), dim3(kBwdThreads),
                         0, s, a);
      if (a.dh0)
        hipLaunchKernelGGL(k_bwd_dh0, dim3(blocks_of(a.Bt * a.H * (int64_t)a.P * a.N, kBwdThreads)),
                           dim3(kBwdThreads), 0, s, a);
      break;
    }
    case 2:
      hipLaunchKernelGGL(k_bwd_dbdc<T>, dim3(blocks_of(a.Bt * a.T * a.G * (int64_t)a.N, kBwdThreads)),
                         dim3(kBwdThreads), 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward_phase(const BwdArgs& a, bool io_bf16, int phase, hipStream_t s) {
  return io_bf16 ? launch_phase<bf16>(a, phase, s) : launch_phase<float>(a, phase, s);
}

// Zero gradients of the per-head parameters when there is no token (or no row).
__global__ __launch_bounds__(kBwdThreads) void k_bwd_zero_heads(float* dA, float* ddt_bias,
                                                                float* dD, int64_t H) {
  const int64_t h = (int64_t)blockIdx.x * kBwdThreads + threadIdx.x;
  if (h >= H) return;
  dA[h] = 0.0f;
  if (ddt_bias) ddt_bias[h] = 0.0f;
  if (dD) dD[h] = 0.0f;
}

hipError_t launch_backward_zero_heads(float* dA, float* ddt_bias, float* dD, int64_t H,
                                      hipStream_t s) {
  hipLaunchKernelGGL(k_bwd_zero_heads, dim3(blocks_of(H, kBwdThreads)), dim3(kBwdThreads), 0, s,
                     dA, ddt_bias, dD, H);
  return hipGetLastError();
}

}  // namespace ssd
