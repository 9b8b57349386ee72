// Gradients of the chunked scan for gfx950 (ssd_chunk_scan_backward): the
// kernels around the two scans the host runs.
//
// Source: "Compiler-First State Space Duality and Portable O(1)
// Autoregressive Caching", Background (Eq. 2-3: the recurrence and its
// chunked dual form) and Implementation (softplus and clip on Delta).
//
// Per (b, h), with Delta d_t, a_t = d_t A, abar_t = e^{a_t}, the recurrence
// h_t = abar_t h_{t-1} + d_t x_t (x) B_t, y_t = h_t C_t + D x_t has the adjoint
//   G_t = dL/dh_t = dy_t (x) C_t + abar_{t+1} G_{t+1},  G_{T-1} = dfinal + dy_{T-1} (x) C_{T-1}.
// In forward chunk c (local tokens i, j; cum = chunk-local inclusive prefix
// sum of a; H_c = state entering the chunk; Ghat_c = abar of the next
// chunk's first token times G there, dfinal for the last chunk):
//   h_i = e^{cum_i} H_c + sum_{j<=i} e^{cum_i - cum_j} d_j x_j (x) B_j
//   G_j = sum_{i>=j} e^{cum_i - cum_j} dy_i (x) C_i + e^{cum_last - cum_j} Ghat_c
// The gradients, with M^h_ij = (dy_i . x_j) e^{cum_i - cum_j} d_j for j <= i
// and M = sum of M^h over a group's heads (the heads share B and C, so the
// products with B and C are taken once per group):
//   dx_j = d_j G_j B_j + D dy_j                       (G_j B_j from R1, below)
//   dC_i = sum_{j<=i} M_ij B_j + sum_h e^{cum_i} dy_i H_c
//   dB_j = sum_{i>=j} M_ij C_i + sum_h d_j e^{cum_last - cum_j} x_j Ghat_c
//   dL/da_t = sum_{i>=t>j} Q_ij + sum_{i>=t} u_i + sum_{j<t} v_j + e^{cum_last} <Ghat_c, H_c>
//     Q_ij = M^h_ij (C_i . B_j),  u_i = C_i . (e^{cum_i} dy_i H_c),
//     v_j = B_j . (d_j e^{cum_last - cum_j} x_j Ghat_c)
//   (sums inside the chunk only: no term cancels against another across the sequence)
//   dd_t = A dL/da_t + x_t . (G_t B_t),  ddt_t = dd_t softplus'(z_t) where Delta is not clipped,
//   dA = sum_t d_t dL/da_t,  dD = sum_t dy_t . x_t,  dh0 = abar_0 G_0.
// The host runs the forward scan's state phases (H_c, kept in float32, and
// C B^T stay in its workspace) and R1, the scan itself over reversed time, both
// with the phased kernels of the io type: reversed
// position T-1-t has the decay of step t+1 and the input dy_t / d_{t+1} (the
// scan multiplies its input by its Delta), with B and C exchanged, so its
// outputs are G_t B_t and its entering states the G at chunk boundaries; pad =
// Nc L - T empty leading positions align its chunks with the forward ones.
//
// Matrix-core tiles: v_mfma_f32_16x16x4_f32, lane l holds A[l%16][k],
// B[k][l%16] and D[4(l/16)+r][l%16]; the contraction index of four
// consecutive instructions is k = 16 blk + 4 (l/16) + e, e = 0..3, so each
// lane reads one float4 of a row-major operand per four instructions.
#include <type_traits>

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

constexpr int kBwdThreads = 256;

__device__ __forceinline__ float delta_at(const BwdArgs& a, int64_t b, int64_t t, int64_t h) {
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
  return delta_of(a.dt[(b * a.T + t) * a.H + h] + bias, a.softplus, a.dt_min, a.dt_max);
}

__device__ __forceinline__ int chunk_tokens(const BwdArgs& a, int64_t c) {
  const int64_t t0 = c * a.L;
  return (int)(a.T - t0 < a.L ? a.T - t0 : a.L);
}

// Branch-free masked loads: `p` must be a valid address whether or not `ok`
// (callers clamp rows to the chunk); the value is replaced by zeros when !ok.
// A plain `ok ? load : 0` becomes one exec-masked branch, and a wait, per load.
template <typename T>
__device__ __forceinline__ float4 ld4_io(const T* p, bool ok) {
  float4 v;
  if constexpr (sizeof(T) == 4) {
    v = *reinterpret_cast<const float4*>(p);
  } else {
    const bf16x4 w = *reinterpret_cast<const bf16x4*>(p);
    v = make_float4((float)w[0], (float)w[1], (float)w[2], (float)w[3]);
  }
  return ok ? v : make_float4(0.f, 0.f, 0.f, 0.f);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// KK consecutive elements (KK = 1, 2 or 4; aligned to KK elements) as float32.
template <int KK, typename T>
__device__ __forceinline__ void ldk(const T* p, bool ok, float (&v)[KK]) {
  if constexpr (KK == 4) {
    const float4 f = ld4_io<T>(p, ok);
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  } else if constexpr (KK == 2) {
    float2 f;
    if constexpr (sizeof(T) == 4) {
      f = *reinterpret_cast<const float2*>(p);
    } else {
      const bf16x2 w = *reinterpret_cast<const bf16x2*>(p);
      f = make_float2((float)w[0], (float)w[1]);
    }
    v[0] = ok ? f.x : 0.f;
    v[1] = ok ? f.y : 0.f;
  } else {
    const float f = to_f32(p[0]);
    v[0] = ok ? f : 0.f;
  }
}

// 16 bytes of io elements (8 bfloat16 or 4 float32) as float32, and back.
template <typename T>
__device__ __forceinline__ void ld16_io(const T* p, float (&v)[16 / sizeof(T)]) {
  if constexpr (sizeof(T) == 4) {
    const float4 f = *reinterpret_cast<const float4*>(p);
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  } else {
    const bf16x8 w = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = (float)w[k];
  }
}
template <typename T>
__device__ __forceinline__ void st16_io(T* p, const float (&v)[16 / sizeof(T)]) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    bf16x8 w;
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = (bf16)v[k];
    *reinterpret_cast<bf16x8*>(p) = w;
  }
}

// Four consecutive elements to memory in the io type (aligned to 4 elements).
template <typename T>
__device__ __forceinline__ void st4_io(T* p, float4 v) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<float4*>(p) = v;
  } else {
    bf16x4 w;
    w[0] = (bf16)v.x; w[1] = (bf16)v.y; w[2] = (bf16)v.z; w[3] = (bf16)v.w;
    *reinterpret_cast<bf16x4*>(p) = w;
  }
}

__device__ __forceinline__ f32x4 mma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma4(float4 a, float4 b, f32x4 c) {
  c = mma(a.x, b.x, c);
  c = mma(a.y, b.y, c);
  c = mma(a.z, b.z, c);
  return mma(a.w, b.w, c);
}

// Sum over each aligned group of 16 lanes (a DPP row), returned to all 16,
// with data-parallel moves instead of LDS permutes: lane pairs xor 1 and xor
// 2 (quad permutes), then the mirrored half row and the mirrored row.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF,
                                                            0xF, false));
}
__device__ __forceinline__ float sum16(float v) {
  v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);   // row_half_mirror
  v += dpp_mov<0x140>(v);   // row_mirror
  return v;
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

// Sum over the 256 threads of a workgroup (fixed order), returned to all.
__device__ __forceinline__ float block_sum(float v, float* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = group_sum(v, 64);
  if (lane == 0) wsum[wave] = v;
  __syncthreads();
  const float s = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  __syncthreads();
  return s;
}

// ---------------------------------------------------------------------------
// Phase 0
// ---------------------------------------------------------------------------

// One thread per four head columns of a (b, t, h) row: R1's input
// dy_t / Delta_{t+1} (0 for the last token) at R1 position pad + T-1-t, in the
// io type (R1 runs the scan kernels of that type).  `sh` = log2(P/4).
template <typename T>
__global__ __launch_bounds__(kBwdThreads) void k_bwd_prep_x(BwdArgs a, int sh) {
  constexpr int EPT = 16 / sizeof(T);   // elements per thread: one 16-byte vector
  const uint32_t e = blockIdx.x * kBwdThreads + threadIdx.x;
  const uint32_t row32 = e >> sh, pq = e & ((1u << sh) - 1u);
  if ((int64_t)row32 >= a.Bt * a.T * a.H) return;
  const uint32_t H32 = (uint32_t)a.H, T32 = (uint32_t)a.T;
  const uint32_t bt32 = row32 / H32;
  const int64_t h = row32 - bt32 * H32, t = bt32 % T32, b = bt32 / T32;
  const int64_t T1 = a.T + a.pad, tr1 = a.pad + (a.T - 1 - t);
  const int P = a.P;
  const int64_t rp = (int64_t)row32 * P + EPT * pq;
  const bool has_next = t + 1 < a.T;
  const float wn = a.wd[has_next ? row32 + (uint32_t)a.H : row32];   // a valid row either way
  // dy_t / Delta_{t+1}, as dy_t times the reciprocal (one division per row)
  const float rn = has_next ? 1.0f / wn : 0.0f;
  float v[EPT];
  ld16_io<T>(reinterpret_cast<const T*>(a.dy) + rp, v);
#pragma unroll
  for (int k = 0; k < EPT; ++k) v[k] *= rn;
  st16_io<T>(reinterpret_cast<T*>(a.r1_x) + ((b * T1 + tr1) * a.H + h) * P + EPT * pq, v);
}

// One thread per four state columns of a (b, t, g) row: R1's B and C (C and
// B, reversed), copied in the io type.  `sh` = log2(N/4).
template <typename T>
__device__ __forceinline__ void bwd_prep_bc(const BwdArgs& a, int sh, int64_t bid) {
  const uint32_t e = (uint32_t)bid * kBwdThreads + threadIdx.x;
  const uint32_t row32 = e >> sh, nq = e & ((1u << sh) - 1u);
  if ((int64_t)row32 >= a.Bt * a.T * a.G) return;
  const uint32_t G32 = (uint32_t)a.G, T32 = (uint32_t)a.T;
  const uint32_t bt32 = row32 / G32;
  const int64_t g = row32 - bt32 * G32, t = bt32 % T32, b = bt32 / T32;
  const int64_t T1 = a.T + a.pad, tr1 = a.pad + (a.T - 1 - t);
  const int N = a.N;
  const int64_t rn = (int64_t)row32 * N + 4 * nq;
  const int64_t rn1 = ((b * T1 + tr1) * a.G + g) * N + 4 * nq;
  using V = typename std::conditional<sizeof(T) == 4, float4, bf16x4>::type;
  const V bv = *reinterpret_cast<const V*>(reinterpret_cast<const T*>(a.B) + rn);
  const V cv = *reinterpret_cast<const V*>(reinterpret_cast<const T*>(a.C) + rn);
  *reinterpret_cast<V*>(reinterpret_cast<T*>(a.r1_b) + rn1) = cv;
  *reinterpret_cast<V*>(reinterpret_cast<T*>(a.r1_c) + rn1) = bv;
}

// The pad positions of R1 (reversed positions 0 .. pad-1) hold no token.
template <typename T>
__device__ __forceinline__ void bwd_zero_pad(const BwdArgs& a, int64_t per_b, int64_t bid) {
  const int64_t e = bid * kBwdThreads + threadIdx.x;
  if (e >= a.Bt * per_b) return;
  const int64_t b = e / per_b, r = e % per_b;
  const int64_t T1 = a.T + a.pad;
  const T z = to_io<T>(0.0f);
  if (r < a.pad * a.H * a.P) reinterpret_cast<T*>(a.r1_x)[b * T1 * a.H * a.P + r] = z;
  if (r < a.pad * a.G * a.N) {
    reinterpret_cast<T*>(a.r1_b)[b * T1 * a.G * a.N + r] = z;
    reinterpret_cast<T*>(a.r1_c)[b * T1 * a.G * a.N + r] = z;
  }
}

// Initial state of R1: dfinal + dy_{T-1} (x) C_{T-1}.
template <typename T>
__device__ __forceinline__ void bwd_init_states(const BwdArgs& a, int64_t bid) {
  const int64_t e = bid * kBwdThreads + threadIdx.x;
  const int P = a.P, N = a.N;
  if (e >= a.Bt * a.H * P * N) return;
  const int64_t n = e % N, p = (e / N) % P, bh = e / ((int64_t)P * N);
  const int64_t h = bh % a.H, b = bh / a.H, g = h / (a.H / a.G);
  const int64_t tl = a.T - 1;
  const float dyv = to_f32(reinterpret_cast<const T*>(a.dy)[((b * a.T + tl) * a.H + h) * P + p]);
  const float cv = to_f32(reinterpret_cast<const T*>(a.C)[((b * a.T + tl) * a.G + g) * N + n]);
  a.r1_h0[e] = __fmaf_rn(dyv, cv, a.dfinal ? a.dfinal[e] : 0.0f);
}

// Delta and R1's Delta' (d_t at R1 position pad + T - t; the pad and
// position pad get 0), then the chunk-local inclusive prefix sum of Delta A
// in double and the row scales of the dC / dB inter-chunk products.  One
// workgroup per (b, c, block of 16 heads): thread (g, hh) forms Delta of
// tokens 16g .. 16g+15 of head hb + hh and their serial prefix sum (the 16
// heads of a token are adjacent in memory, so every access is a 64-byte run),
// then adds the totals of the token groups before it, in order, from LDS.
__device__ __forceinline__ void bwd_cum_delta(const BwdArgs& a, int64_t bid) {
  constexpr int kHB = 16, kTG = kBwdThreads / kHB;   // heads per block, token groups (L <= 256)
  __shared__ double s_tot[kTG][kHB];
  __shared__ double s_last[kHB];
  const int hh = threadIdx.x % kHB, g = threadIdx.x / kHB;
  const int64_t nhb = (a.H + kHB - 1) / kHB;
  const int64_t hb = (bid % nhb) * kHB, bc = bid / nhb, c = bc % a.Nc, b = bc / a.Nc;
  const int64_t h = min(hb + hh, (int64_t)a.H - 1);   // heads past H repeat the last and store nothing
  const bool hok = hb + hh < a.H;
  const int64_t t0 = c * a.L, T1 = a.T + a.pad;
  const int Lc = chunk_tokens(a, c);
  const double Ah = (double)a.A[h];
  float wdv[16];   // tokens past the chunk repeat its last one and store nothing
#pragma unroll
  for (int k = 0; k < 16; ++k) wdv[k] = delta_at(a, b, t0 + min(16 * g + k, Lc - 1), h);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int l = 16 * g + k;
    if (hok && l < Lc) {
      const int64_t t = t0 + l;
      a.wd[(b * a.T + t) * a.H + h] = wdv[k];
      if (t >= 1) {
        a.dtr1[(b * T1 + (a.pad + a.T - t)) * a.H + h] = wdv[k];
      } else {
        for (int64_t z = 0; z <= a.pad; ++z) a.dtr1[(b * T1 + z) * a.H + h] = 0.0f;
      }
    }
  }
  double cv[16];
  double run = 0.0;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    run += 16 * g + k < Lc ? (double)wdv[k] * Ah : 0.0;
    cv[k] = run;
  }
  s_tot[g][hh] = run;
  __syncthreads();
  double off = 0.0;
  for (int j = 0; j < g; ++j) off += s_tot[j][hh];
  const int last = Lc - 1;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    cv[k] += off;
    const int l = 16 * g + k;
    if (hok && l < Lc) a.cum[(b * a.T + t0 + l) * a.H + h] = cv[k];
    if (l == last) s_last[hh] = cv[k];
  }
  __syncthreads();
  // the row scales (the same float operations the products' kernel would
  // apply to the prefix sums)
  const double clast = s_last[hh];
  const int64_t n = a.Bt * a.T * a.H;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int l = 16 * g + k;
    if (hok && l < Lc) {
      const int64_t row = (b * a.T + t0 + l) * a.H + h;
      a.rscale[row] = fast_exp((float)cv[k]);
      a.rscale[n + row] = wdv[k] * fast_exp((float)(clast - cv[k]));
    }
  }
}

// Phase 0 but R1's input rows: the blocks of one launch are dealt, in order,
// to Delta and its prefix sums, R1's B and C, R1's pad rows and R1's initial
// state (independent work; fewer launches).
struct Prep0Grid {
  int64_t n_cd, n_bc, n_pad;
  int64_t per_b;
  int sh_bc;
};
template <typename T>
__global__ __launch_bounds__(kBwdThreads) void k_bwd_prep0(BwdArgs a, Prep0Grid pg) {
  int64_t bid = blockIdx.x;
  if (bid < pg.n_cd) {
    bwd_cum_delta(a, bid);
    return;
  }
  bid -= pg.n_cd;
  if (bid < pg.n_bc) {
    bwd_prep_bc<T>(a, pg.sh_bc, bid);
    return;
  }
  bid -= pg.n_bc;
  if (bid < pg.n_pad) {
    bwd_zero_pad<T>(a, pg.per_b, bid);
    return;
  }
  bid -= pg.n_pad;
  bwd_init_states<T>(a, bid);
}

// ---------------------------------------------------------------------------
// Phase 1
// ---------------------------------------------------------------------------

// One workgroup per (b, c, g, head split, 64x64 block (I, J) of the chunk's
// token pairs, J <= I).  For each head of the split: S = dy_I x_J^T on the
// matrix cores, M^h = S o e^{cum_i - cum_j} o d_j (j <= i), the block's part
// of M = sum_h M^h, and the row and column sums of Q = M^h o C B^T (j < i)
// over the block's halves.  Wavefront (wr, wc) owns rows 32 wr .. +31 and
// columns 32 wc .. +31 of the block.  Nothing is shared between wavefronts:
// every partial sum has one writer, and the consumers add them in a fixed
// order.
template <typename T, int P>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(3))) void k_bwd_mix(BwdArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int NB = a.NB, nbt = NB * (NB + 1) / 2;
  // the blocks of one (b, c, g, head split) read the same rows: same XCD, same L2
  int64_t u = xcd_remap(blockIdx.x, gridDim.x);
  const int blk = (int)(u % nbt);
  u /= nbt;
  const int hs = (int)(u % a.HS);
  u /= a.HS;
  const int64_t g = u % a.G, bc = u / a.G, c = bc % a.Nc, b = bc / a.Nc;
  int I = 0;
  while ((I + 1) * (I + 2) / 2 <= blk) ++I;
  const int J = blk - I * (I + 1) / 2;
  const int64_t L = a.L, t0 = c * L;
  const int Lc = chunk_tokens(a, c);
  if (64 * I >= Lc) return;
  const int64_t hpg = a.H / a.G;
  const int64_t hb = g * hpg + (int64_t)hs * a.hpw;
  const int64_t he = min(hb + (int64_t)a.hpw, (g + 1) * hpg);

  int ia[2], jb[2];        // A-operand rows (dy) and B-operand / output columns (x)
  int io[2][4];            // output rows
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    ia[s] = 64 * I + 32 * wr + 16 * s + r16;
    jb[s] = 64 * J + 32 * wc + 16 * s + r16;
#pragma unroll
    for (int r = 0; r < 4; ++r) io[s][r] = 64 * I + 32 * wr + 16 * s + 4 * q + r;
  }
  const int64_t xrs = a.H * P;
  const T* xg = reinterpret_cast<const T*>(a.x) + (b * a.T + t0) * xrs;
  const T* dyg = reinterpret_cast<const T*>(a.dy) + (b * a.T + t0) * xrs;
  const double* cumg = a.cum + (b * a.T + t0) * a.H;
  const float* wdg = a.wd + (b * a.T + t0) * a.H;

  // C B^T of this lane's outputs where j < i (the products Q need), else 0
  const float* cb = a.fwd_cb + ((b * a.Nc + c) * a.G + g) * L * L;
  float cbv[2][2][4];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = io[s][r], j = jb[v];
        const float cv = cb[(int64_t)min(i, Lc - 1) * L + min(j, Lc - 1)];
        // one select (not a short-circuit branch) keeps the 16 loads together
        cbv[s][v][r] = ((i < Lc) & (j < i)) ? cv : 0.0f;
      }

  f32x4 mv[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int v = 0; v < 2; ++v) mv[s][v] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t bch = (b * a.Nc + c) * a.H;
  // The block's dy rows (I) and x rows (J) of one head go through LDS,
  // double-buffered: each is read by two wavefronts, and the next head's rows
  // are loaded into registers while this head's are consumed.  Rows past the
  // chunk read its last row: finite values whose products the causal select
  // below discards.
  // bfloat16 rows (P a multiple of 32) go to the bf16 matrix cores as they
  // are: products of two bf16 values are exact in float32, so S is the same
  // up to the order of its sums.  Otherwise they are staged as float32.
  constexpr bool kB = sizeof(T) == 2 && P % 32 == 0;
  using ST = typename std::conditional<kB, bf16, float>::type;
  // native vectors (not HIP's struct vector types): the staging registers
  // must stay in VGPRs across process(), and the struct types were kept on
  // the stack
  using VT = typename std::conditional<kB, bf16x8, f32x4>::type;
  constexpr int EPV = kB ? 8 : 4;                 // elements per 16-byte vector
  constexpr int XS = P + EPV;                     // padded LDS row
  constexpr int RQ = P / EPV;                     // vectors per row
  constexpr int SL = 2 * 64 * RQ / kBwdThreads;   // vectors per thread per head
  __shared__ __attribute__((aligned(16))) ST s_op[2][2 * 64 * XS];
  auto load_stage = [&](int64_t h, VT (&st)[SL]) {
#pragma unroll
    for (int k = 0; k < SL; ++k) {
      const int e = tid + k * kBwdThreads, which = e / (64 * RQ), rem = e % (64 * RQ);
      const int row = rem / RQ, p4 = rem % RQ;
      const int grow = min((which ? 64 * J : 64 * I) + row, Lc - 1);
      const T* src = (which ? xg : dyg) + (int64_t)grow * xrs + h * P + EPV * p4;
      if constexpr (kB) {
        st[k] = *reinterpret_cast<const bf16x8*>(src);
      } else {
        const float4 v = ld4_io<T>(src, true);
        st[k] = f32x4{v.x, v.y, v.z, v.w};
      }
    }
  };
  auto store_stage = [&](int buf, const VT (&st)[SL]) {
#pragma unroll
    for (int k = 0; k < SL; ++k) {
      const int e = tid + k * kBwdThreads, which = e / (64 * RQ), rem = e % (64 * RQ);
      const int row = rem / RQ, p4 = rem % RQ;
      *reinterpret_cast<VT*>(&s_op[buf][(which * 64 + row) * XS + EPV * p4]) = st[k];
    }
  };
  // The prefix sums of the block's rows (I) and columns (J) and Delta of its
  // columns go through LDS with the operand rows (a register copy per lane
  // of its ten values, for this head and the next, held the kernel to two
  // wavefronts per SIMD).  Every thread loads one of each (rows past the
  // chunk read its last token); threads 0..127 store the prefix sums, 128..191
  // the Deltas.
  __shared__ double s_cum[2][128];
  __shared__ float s_dj[2][64];
  struct Tok {
    double cv;
    float wv;
  };
  auto load_tok = [&](int64_t h, Tok& o) {
    const int rrow = tid < 64 ? 64 * I + tid : 64 * J + (tid & 63);
    o.cv = cumg[(int64_t)min(rrow, Lc - 1) * a.H + h];
    o.wv = wdg[(int64_t)min(64 * J + (tid & 63), Lc - 1) * a.H + h];   // masked with the decay
  };
  auto store_tok = [&](int buf, const Tok& o) {
    if (tid < 128) s_cum[buf][tid] = o.cv;
    else if (tid < 192) s_dj[buf][tid - 128] = o.wv;
  };
  struct Dec {
    double ci[2][4], cj[2];
    float dj[2];
  };
  auto read_dec = [&](int buf, Dec& o) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int r = 0; r < 4; ++r) o.ci[s][r] = s_cum[buf][32 * wr + 16 * s + 4 * q + r];
      o.cj[s] = s_cum[buf][64 + 32 * wc + 16 * s + r16];
      o.dj[s] = s_dj[buf][32 * wc + 16 * s + r16];
    }
  };
  auto process = [&](int64_t h, const ST* so, const Dec& o) {
    f32x4 sv[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int v = 0; v < 2; ++v) sv[s][v] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (kB) {
      // v_mfma_f32_16x16x32_bf16: lane (q, r16) holds k-slots 32 kb + 8 q .. +7
#pragma unroll
      for (int kb = 0; kb < P / 32; ++kb) {
        bf16x8 dv[2], xv[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          dv[s] = *reinterpret_cast<const bf16x8*>(&so[(32 * wr + 16 * s + r16) * XS + 32 * kb + 8 * q]);
          xv[s] = *reinterpret_cast<const bf16x8*>(
              &so[(64 + 32 * wc + 16 * s + r16) * XS + 32 * kb + 8 * q]);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int v = 0; v < 2; ++v)
            sv[s][v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dv[s], xv[v], sv[s][v], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int pb = 0; pb < P / 16; ++pb) {
        float4 dv[2], xv[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          dv[s] = *reinterpret_cast<const float4*>(&so[(32 * wr + 16 * s + r16) * XS + 16 * pb + 4 * q]);
          xv[s] = *reinterpret_cast<const float4*>(
              &so[(64 + 32 * wc + 16 * s + r16) * XS + 16 * pb + 4 * q]);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int v = 0; v < 2; ++v) sv[s][v] = mfma4(dv[s], xv[v], sv[s][v]);
      }
    }
    float rowp[2][4], colp[2] = {0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        rowp[s][r] = 0.0f;
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          const int i = io[s][r], j = jb[v];
          // causal mask selected before the exponential
          const bool ok = i < Lc && j <= i;
          const float e = ok ? fast_exp((float)(o.ci[s][r] - o.cj[v])) : 0.0f;
          const float m = sv[s][v][r] * e * o.dj[v];
          mv[s][v][r] += m;
          const float qv = m * cbv[s][v][r];
          rowp[s][r] += qv;
          colp[v] += qv;
        }
      }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r) rowp[s][r] = sum16(rowp[s][r]);
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      colp[v] += __shfl_xor(colp[v], 16, 64);
      colp[v] += __shfl_xor(colp[v], 32, 64);
    }
    const int64_t qo = (((bch + h) * NB + I) * NB + J) * 128;
    if (r16 == 0) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) a.qrow[qo + 64 * wc + 32 * wr + 16 * s + 4 * q + r] = rowp[s][r];
    }
    if (q == 0) {
#pragma unroll
      for (int v = 0; v < 2; ++v) a.qcol[qo + 64 * wr + 32 * wc + 16 * v + r16] = colp[v];
    }
  };
  {
    VT st[SL];
    Tok tk;
    load_stage(hb, st);
    load_tok(hb, tk);
    store_stage(0, st);
    store_tok(0, tk);
    __syncthreads();
    int buf = 0;
    // the next head's loads are issued on every path (the last head re-reads
    // itself into the buffer nobody reads again): a conditional load kept
    // the staging registers in scratch memory across process()
#pragma unroll 1
    for (int64_t h = hb; h < he; ++h) {
      const int64_t hn = h + 1 < he ? h + 1 : h;   // uniform
      load_stage(hn, st);
      load_tok(hn, tk);
      Dec cur;
      read_dec(buf, cur);
      process(h, s_op[buf], cur);
      store_stage(buf ^ 1, st);
      store_tok(buf ^ 1, tk);
      __syncthreads();
      buf ^= 1;
    }
  }
  // this head split's part of M (zeros outside j <= i < Lc)
  const int64_t LP = a.LP;
  float* mp = a.mix + (((b * a.Nc + c) * a.G + g) * a.HS + hs) * LP * LP;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int r = 0; r < 4; ++r) mp[(int64_t)io[s][r] * LP + jb[v]] = mv[s][v][r];
}

// One workgroup per (b, c, g, head split, role, column split, 64-row block):
// role 0 forms dC for the block's tokens, role 1 dB, over NW = 16 KK of the
// N state columns.  Wavefront w owns the block's rows 16 w .. +15; lane
// (q, r16) holds outputs of rows 4q + r and columns KK r16 .. +KK-1 (the
// KK accumulator tiles interleave their columns, so that the state rows are
// read as KK-wide vectors).
//   inter-chunk part, per head of the split: (scale_i row_i) . Z, with
//     role 0: row = dy_i, scale = e^{cum_i}, Z = H_c;
//     role 1: row = x_j, scale = d_j e^{cum_last - cum_j}, Z = Ghat_c;
//     its dot with C_i (role 0) or B_j (role 1) is u_i or v_j (this split's columns);
//   intra-chunk part: M B (role 0, j <= i) or M^T C (role 1, i >= j), its 16-token
//     blocks dealt out over the head splits.
template <typename T, int P, int KK>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(3))) void k_bwd_dcdb(BwdArgs a) {
  constexpr int NW = 16 * KK;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NB = a.NB;
  // the row blocks of one (b, c, g, head split, role, column split) read the
  // same state slices: same XCD, same L2
  int64_t u = xcd_remap(blockIdx.x, gridDim.x);
  const int rb = (int)(u % NB);
  u /= NB;
  const int ns = (int)(u % a.NS);
  u /= a.NS;
  const int role = (int)(u % 2);
  u /= 2;
  const int hsd = (int)(u % a.HSD);
  u /= a.HSD;
  const int64_t g = u % a.G, bc = u / a.G, c = bc % a.Nc, b = bc / a.Nc;
  const int64_t L = a.L, t0 = c * L;
  const int Lc = chunk_tokens(a, c);
  if (64 * rb >= Lc) return;
  const int N = a.N;
  const int n0 = ns * NW + KK * r16;          // this lane's columns
  const int ia = 64 * rb + 16 * wave + r16;   // A-operand row
  const bool iok = ia < Lc;
  const int iac = iok ? ia : Lc - 1;
  int io[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) io[r] = 64 * rb + 16 * wave + 4 * q + r;
  const int64_t grs = a.G * N;
  const T* Bg = reinterpret_cast<const T*>(a.B) + ((b * a.T + t0) * a.G + g) * N;
  const T* Cg = reinterpret_cast<const T*>(a.C) + ((b * a.T + t0) * a.G + g) * N;
  const T* dotm = role ? Bg : Cg;
  float dvec[4][KK];
#pragma unroll
  for (int r = 0; r < 4; ++r)
    ldk<KK, T>(dotm + (int64_t)min(io[r], Lc - 1) * grs + n0, io[r] < Lc, dvec[r]);

  f32x4 acc[KK];
#pragma unroll
  for (int k = 0; k < KK; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t hpg = a.H / a.G;
  const int64_t hb = g * hpg + (int64_t)hsd * a.hpwd;
  const int64_t he = min(hb + (int64_t)a.hpwd, (g + 1) * hpg);
  const int64_t PN = (int64_t)P * N;
  const int64_t BtT = a.Bt * a.T;
  // u / v are stored token-contiguous per (b, h): [2][NS][Bt,H,T]
  float* uvo = a.uv + (int64_t)(role * a.NS + ns) * BtT * a.H + b * a.H * a.T + t0;
  // Z = H_c (role 0) or Ghat_c / abar (role 1; null for the last chunk without dfinal)
  auto zptr = [&](int64_t h) -> const float* {
    if (role == 0) return a.fwd_state + ((b * a.H + h) * a.Nc + c) * PN;
    if (c + 1 < a.Nc) return a.r1_state + ((b * a.H + h) * a.Nc + (a.Nc - 1 - c)) * PN;
    return a.dfinal ? a.dfinal + (b * a.H + h) * PN : nullptr;
  };
  // The workgroup's NW columns of Z are shared by its four wavefronts: they
  // go through LDS, double-buffered, the next head's slice loaded into
  // registers while this head's is consumed.  Each wavefront reads its own A
  // rows directly.
  //
  // bfloat16 inputs (kB): A (dy or x) holds bf16 values, exact as
  // matrix-core operands, so the per-row scale is applied to the products
  // instead of to A, and Z (float32) is split into two bf16 parts
  // Z = Zh + Zl (Zh = bf16(Z), Zl = bf16(Z - Zh)): A Zh + A Zl on
  // v_mfma_f32_16x16x32_bf16 is A Z to within the rounding of Zl (2^-16
  // relative), at an eighth of the float32 matrix-core time.  Z is staged
  // transposed, [n][p] bf16 (the contraction index p contiguous, as the
  // operand wants it), its 16-byte units XOR-swizzled by the row's lane
  // index so that the 8 lanes of a read group hit distinct banks.
  constexpr bool kB = sizeof(T) == 2 && P % 32 == 0 && KK == 4;
  constexpr int ZS = NW + 4;                        // padded LDS row
  constexpr int ZQ = NW / 4;                        // float4 per Z row
  constexpr int ZL = (P * ZQ + kBwdThreads - 1) / kBwdThreads;
  constexpr int ZU = (P / 8 < 8 ? P / 8 : 8) - 1;   // swizzle mask of a [n][p] row's units
  __shared__ __attribute__((aligned(16))) float s_z[2][kB ? 4 : P * ZS];
  __shared__ __attribute__((aligned(16))) bf16 s_zt[2][kB ? 2 * NW * P : 8];
  // Z's loads are issued on every path (a missing Z reads the forward states
  // and is zeroed when stored): a load under a condition leaves a different
  // number of loads in flight on each path, and the compiler's wait after the
  // merge then also covers loads issued after the ones it needs
  // kB: thread (g, cq) = (tid / ZQ, tid % ZQ) holds rows ZL g .. ZL g + ZL-1
  // of column quad cq, so that each of its four columns goes to the
  // transposed LDS copy as one packed store of ZL consecutive p; otherwise
  // rows tid / ZQ + k kBwdThreads / ZQ
  auto z_row = [&](int k) -> int {
    if constexpr (kB) return ZL * (tid / ZQ) + k;
    return min((tid + k * kBwdThreads) / ZQ, P - 1);
  };
  auto load_z = [&](int64_t h, float4 (&zr)[ZL]) {
    const float* Z = zptr(h);
    const float* Zs = Z != nullptr ? Z : a.fwd_state;   // a valid address either way
    const int cq = tid % ZQ;
#pragma unroll
    for (int k = 0; k < ZL; ++k)
      zr[k] = *reinterpret_cast<const float4*>(Zs + (int64_t)z_row(k) * N + ns * NW + 4 * cq);
  };
  auto store_z = [&](int buf, int64_t h, float4 (&zr)[ZL]) {
    if (zptr(h) == nullptr) {   // uniform
#pragma unroll
      for (int k = 0; k < ZL; ++k) zr[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if constexpr (kB) {
      // column n = 4 cq + cc: ZL consecutive p (one aligned run inside a
      // 16-byte unit), hi and lo parts, one store each
      using Pack = typename std::conditional<ZL == 2, bf16x2,
                   typename std::conditional<ZL == 4, bf16x4, bf16x8>::type>::type;
      const int cq = tid % ZQ, pr0 = z_row(0);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const int n = 4 * cq + cc;
        Pack hi, lo;
#pragma unroll
        for (int k = 0; k < ZL; ++k) {
          const float v = cc == 0 ? zr[k].x : cc == 1 ? zr[k].y : cc == 2 ? zr[k].z : zr[k].w;
          hi[k] = (bf16)v;
          lo[k] = (bf16)__fsub_rn(v, (float)hi[k]);
        }
        const int at = n * P + 8 * ((pr0 >> 3) ^ ((n >> 2) & ZU)) + (pr0 & 7);
        *reinterpret_cast<Pack*>(&s_zt[buf][at]) = hi;
        *reinterpret_cast<Pack*>(&s_zt[buf][NW * P + at]) = lo;
      }
    } else {
#pragma unroll
      for (int k = 0; k < ZL; ++k) {
        const int e = tid + k * kBwdThreads, pr = e / ZQ, cq = e % ZQ;
        if (e < P * ZQ) *reinterpret_cast<float4*>(&s_z[buf][pr * ZS + 4 * cq]) = zr[k];
      }
    }
  };
  // A rows stay in their io type until used: converting bf16 as it arrives
  // put a wait for the next head's rows right after their loads (2.7B-shaped
  // backward 0.66 -> 0.64 ms)
  using RawA = typename std::conditional<sizeof(T) == 4, float4, bf16x4>::type;
  // kB: the A fragments of the bf16 products (8 consecutive p per lane) and
  // the prefix sums and Delta of the lane's four output rows
  struct Arow {
    RawA av[kB ? 1 : P / 16];
    bf16x8 avb[kB ? P / 32 : 1];
    float sc[kB ? 4 : 1];   // the row scale of the role (output rows io[r], or row ia)
    float wn, Ah;
  };
  const T* amat = reinterpret_cast<const T*>(role ? a.x : a.dy);
  const float* rsc = a.rscale + (role ? a.Bt * a.T * a.H : 0);
  auto load_a = [&](int64_t h, Arow& o) {
    const int64_t rowi = (b * a.T + t0 + iac) * a.H + h;
    const T* arow = amat + rowi * P;
    if constexpr (kB) {
#pragma unroll
      for (int kb = 0; kb < P / 32; ++kb)
        o.avb[kb] = *reinterpret_cast<const bf16x8*>(arow + 32 * kb + 8 * q);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t ro = (b * a.T + t0 + min(io[r], Lc - 1)) * a.H + h;
        o.sc[r] = rsc[ro];
      }
    } else {
#pragma unroll
      for (int pb = 0; pb < P / 16; ++pb) o.av[pb] = *reinterpret_cast<const RawA*>(arow + 16 * pb + 4 * q);
      o.sc[0] = rsc[rowi];
    }
    // Delta of the next chunk's first token (role 1; a valid row is read on
    // every path and the value is dropped where it does not apply)
    o.wn = a.wd[(b * a.T + min(t0 + L, a.T - 1)) * a.H + h];
    // A of the head with the rest of its values: loaded where it is used, it
    // was the newest load in flight, and its wait covered every load before it
    o.Ah = a.A[h];
  };
  auto process_h = [&](int64_t h, const Arow& o, const float* sz, const bf16* szt) {
    f32x4 ah[KK];
#pragma unroll
    for (int k = 0; k < KK; ++k) ah[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (kB) {
      // lane (q, r16): A[row r16][p = 32 kb + 8q ..], Z[p][n = KK r16 + kk]
#pragma unroll
      for (int kb = 0; kb < P / 32; ++kb) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const int n = KK * r16 + kk;
          const int at = n * P + 8 * ((4 * kb + q) ^ (r16 & ZU));
          const bf16x8 zh = *reinterpret_cast<const bf16x8*>(szt + at);
          const bf16x8 zl = *reinterpret_cast<const bf16x8*>(szt + NW * P + at);
          ah[kk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.avb[kb], zh, ah[kk], 0, 0, 0);
          ah[kk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.avb[kb], zl, ah[kk], 0, 0, 0);
        }
      }
      // the row scale of output row io[r] (0 past the chunk)
      const float gs = (role == 1 && c + 1 < a.Nc) ? expf(o.wn * o.Ah) : 1.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = io[r] < Lc;
        const float sc = ok ? (role == 0 ? o.sc[r] : gs * o.sc[r]) : 0.0f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) ah[kk][r] *= sc;
      }
    } else {
    float scale;
    if (role == 0) {
      scale = iok ? o.sc[0] : 0.0f;
    } else {
      // abar of the next chunk's first token turns R1's entering state into Ghat_c
      const float gs = c + 1 < a.Nc ? expf(o.wn * o.Ah) : 1.0f;
      scale = iok ? gs * o.sc[0] : 0.0f;
    }
#pragma unroll
    for (int pb = 0; pb < P / 16; ++pb) {
      float4 avf;
      if constexpr (sizeof(T) == 4) {
        avf = o.av[pb];
      } else {
        avf = make_float4((float)o.av[pb][0], (float)o.av[pb][1], (float)o.av[pb][2],
                          (float)o.av[pb][3]);
      }
      const float av[4] = {avf.x * scale, avf.y * scale, avf.z * scale, avf.w * scale};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float* zrow = sz + (16 * pb + 4 * q + e) * ZS + KK * r16;
        float zv[KK];
        if constexpr (KK == 4) {
          const float4 v = *reinterpret_cast<const float4*>(zrow);
          zv[0] = v.x; zv[1] = v.y; zv[2] = v.z; zv[3] = v.w;
        } else if constexpr (KK == 2) {
          const float2 v = *reinterpret_cast<const float2*>(zrow);
          zv[0] = v.x; zv[1] = v.y;
        } else {
          zv[0] = zrow[0];
        }
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) ah[kk] = mma(av[e], zv[kk], ah[kk]);
      }
    }
    }
    // u_i (role 0) or v_j (role 1) over this split's columns
    float ds[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float sum = 0.0f;
#pragma unroll
      for (int k = 0; k < KK; ++k) sum = __fmaf_rn(dvec[r][k], ah[k][r], sum);
      ds[r] = sum16(sum);
    }
    if (r16 == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (io[r] < Lc) uvo[h * a.T + io[r]] = ds[r];
    }
#pragma unroll
    for (int k = 0; k < KK; ++k) acc[k] += ah[k];
  };
  {
    float4 zr[ZL];
    Arow cur, nxt;
    load_z(hb, zr);
    load_a(hb, cur);
    store_z(0, hb, zr);
    __syncthreads();
    int buf = 0;
    // the next head's loads are issued on every path (the last head re-reads
    // itself into the buffer nobody reads again)
#pragma unroll 1
    for (int64_t h = hb; h < he; ++h) {
      const int64_t hn = h + 1 < he ? h + 1 : h;   // uniform
      load_z(hn, zr);
      load_a(hn, nxt);
      process_h(h, cur, s_z[buf], s_zt[buf]);
      store_z(buf ^ 1, hn, zr);
      __syncthreads();
      cur = nxt;
      buf ^= 1;
    }
  }

  // intra-chunk part: its 16-token blocks are dealt out over the head splits
  // (whose parts are summed afterwards), so every workgroup gets a share
  {
    const int64_t LP = a.LP, LP2 = LP * LP;
    const float* mp = a.mix + ((b * a.Nc + c) * a.G + g) * (int64_t)a.HS * LP2;
    const int kend = (Lc + 15) / 16;
    if (role == 0) {
      // dC_i += sum_{j <= i} M[i][j] B_j
      const int kb1 = min(4 * (rb + 1), kend);
      for (int kb = hsd; kb < kb1; kb += a.HSD) {
        float4 m4 = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int s = 0; s < a.HS; ++s) {
          const float4 v =
              *reinterpret_cast<const float4*>(mp + s * LP2 + (int64_t)ia * LP + 16 * kb + 4 * q);
          m4.x += v.x; m4.y += v.y; m4.z += v.z; m4.w += v.w;
        }
        float bv[4][KK];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // M[i][j] = 0 for j >= Lc: the clamped row needs no mask
          const int j = 16 * kb + 4 * q + e;
          ldk<KK, T>(Bg + (int64_t)min(j, Lc - 1) * grs + n0, true, bv[e]);
        }
#pragma unroll
        for (int k = 0; k < KK; ++k) {
          acc[k] = mma(m4.x, bv[0][k], acc[k]);
          acc[k] = mma(m4.y, bv[1][k], acc[k]);
          acc[k] = mma(m4.z, bv[2][k], acc[k]);
          acc[k] = mma(m4.w, bv[3][k], acc[k]);
        }
      }
    } else {
      // dB_j += sum_{i >= j} M[i][j] C_i
      for (int kb = 4 * rb + hsd; kb < kend; kb += a.HSD) {
        float m4[4] = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < a.HS; ++s) {
#pragma unroll
          for (int e = 0; e < 4; ++e) m4[e] += mp[s * LP2 + (int64_t)(16 * kb + 4 * q + e) * LP + ia];
        }
        float cv[4][KK];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // M[i][j] = 0 for i >= Lc: the clamped row needs no mask
          const int i = 16 * kb + 4 * q + e;
          ldk<KK, T>(Cg + (int64_t)min(i, Lc - 1) * grs + n0, true, cv[e]);
        }
#pragma unroll
        for (int k = 0; k < KK; ++k) {
          acc[k] = mma(m4[0], cv[0][k], acc[k]);
          acc[k] = mma(m4[1], cv[1][k], acc[k]);
          acc[k] = mma(m4[2], cv[2][k], acc[k]);
          acc[k] = mma(m4[3], cv[3][k], acc[k]);
        }
      }
    }
  }

  float* out = a.HSD > 1 ? a.dbc_part + (int64_t)(role * a.HSD + hsd) * BtT * a.G * N
                         : (role ? a.dB : a.dC);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (io[r] >= Lc) continue;
    float* o = out + ((b * a.T + t0 + io[r]) * a.G + g) * N + n0;
    if constexpr (KK == 4) {
      *reinterpret_cast<float4*>(o) = make_float4(acc[0][r], acc[1][r], acc[2][r], acc[3][r]);
    } else if constexpr (KK == 2) {
      *reinterpret_cast<float2*>(o) = make_float2(acc[0][r], acc[1][r]);
    } else {
      o[0] = acc[0][r];
    }
  }
}

// dC, dB: sums over the head splits of their parts (fixed order).
__device__ __forceinline__ void bwd_dcdb_reduce(const BwdArgs& a, int64_t bid) {
  const int64_t n = a.Bt * a.T * a.G * a.N;
  const int64_t e = bid * kBwdThreads + threadIdx.x;
  if (e >= 2 * n) return;
  const int role = e >= n ? 1 : 0;
  const int64_t k = e - role * n;
  float s = 0.0f;
  for (int p = 0; p < a.HSD; ++p) s += a.dbc_part[(int64_t)(role * a.HSD + p) * n + k];
  (role ? a.dB : a.dC)[k] = s;
}

// One thread per four head columns of a (b, t, h) row (the P/4 threads of a
// row are adjacent lanes of one wavefront): dx, the input-scale part of the
// Delta gradient (x . G B) and the per-token part of dD.  `sh` = log2(P/4).
template <typename T>
__device__ __forceinline__ void bwd_dx(const BwdArgs& a, int sh, int64_t bid) {
  constexpr int EPT = 16 / sizeof(T);   // elements per thread: one 16-byte vector of each input
  const uint32_t e = (uint32_t)bid * kBwdThreads + threadIdx.x;
  const uint32_t row32 = e >> sh, pq = e & ((1u << sh) - 1u);
  const bool ok = (int64_t)row32 < a.Bt * a.T * a.H;
  const uint32_t rowc = ok ? row32 : 0u;
  const uint32_t H32 = (uint32_t)a.H, T32 = (uint32_t)a.T;
  const uint32_t bt32 = rowc / H32;
  const int64_t h = rowc - bt32 * H32, t = bt32 % T32, b = bt32 / T32;
  const int P = a.P;
  const float d = a.wd[rowc];
  const float Dh = a.D ? a.D[h] : 0.0f;
  const int64_t rp = (int64_t)rowc * P + EPT * pq;
  const int64_t rpr1 = ((b * (a.T + a.pad) + (a.pad + a.T - 1 - t)) * a.H + h) * P + EPT * pq;
  // threads past the last row read row 0 and store nothing
  float xv[EPT], dyv[EPT], gb[EPT];   // gb = sum_n G[p,n] B_t[n]
  ld16_io<T>(reinterpret_cast<const T*>(a.x) + rp, xv);
  ld16_io<T>(reinterpret_cast<const T*>(a.dy) + rp, dyv);
  ld16_io<T>(reinterpret_cast<const T*>(a.r1_y) + rpr1, gb);
  if (ok) {
#pragma unroll
    for (int k = 0; k < EPT; k += 4)
      *reinterpret_cast<float4*>(a.dx + rp + k) =
          make_float4(__fmaf_rn(Dh, dyv[k], d * gb[k]), __fmaf_rn(Dh, dyv[k + 1], d * gb[k + 1]),
                      __fmaf_rn(Dh, dyv[k + 2], d * gb[k + 2]), __fmaf_rn(Dh, dyv[k + 3], d * gb[k + 3]));
  }
  float s_din = xv[0] * gb[0];
#pragma unroll
  for (int k = 1; k < EPT; ++k) s_din = __fmaf_rn(xv[k], gb[k], s_din);
  float s_dd = dyv[0] * xv[0];
#pragma unroll
  for (int k = 1; k < EPT; ++k) s_dd = __fmaf_rn(dyv[k], xv[k], s_dd);
  const int width = 1 << sh;
  s_din = group_sum(s_din, width);
  s_dd = group_sum(s_dd, width);
  if (ok && pq == 0) {
    // token-contiguous per (b, h), as the assembly reads them
    const int64_t o = (b * a.H + h) * a.T + t;
    a.ddin[o] = s_din;
    a.dDp[o] = s_dd;
  }
}

// One workgroup per (b, c, h), one token per thread (L <= 256): dL/da_t from
// the block sums of Q and the per-token u, v (prefix and suffix sums within
// the chunk), the dt gradient, and this chunk's parts of dA, ddt_bias, dD.
// Every global load is issued before the first value is used (rows, blocks
// and splits that do not apply read a valid clamped address and are dropped
// by a select), so the workgroup waits for memory once instead of once per
// dependent step; the chunk-boundary dot <Ghat_c, H_c> comes formed.
__global__ __launch_bounds__(kBwdThreads) void k_bwd_assemble(BwdArgs a) {
  constexpr int kMaxNB = 4;   // 64-token blocks of a chunk (L <= 256)
  constexpr int kMaxNS = 2;   // 64-column splits of N (N <= 128)
  __shared__ float s_w[kBwdThreads / 64];
  const int l = threadIdx.x;
  const int64_t u = blockIdx.x;
  const int64_t h = u % a.H, bc = u / a.H, c = bc % a.Nc, b = bc / a.Nc;
  const int64_t L = a.L, t0 = c * L;
  const int Lc = chunk_tokens(a, c);
  const int NB = a.NB, nbc = (Lc + 63) / 64;
  const bool ok = l < Lc;
  const int lc = ok ? l : 0;
  const int64_t row = (b * a.T + t0 + lc) * a.H + h;
  const int64_t BtT = a.Bt * a.T;

  // per-token and per-head scalars
  const int64_t rowt = (b * a.H + h) * a.T + t0 + lc;   // the token-contiguous buffers
  const float dt_raw = a.dt[row], wd_t = a.wd[row], ddin_t = a.ddin[rowt], dDp_t = a.dDp[rowt];
  const float Ah = a.A[h];
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
  const double clast = a.cum[(b * a.T + t0 + Lc - 1) * a.H + h];
  const bool has_next = c + 1 < a.Nc;
  const float wd_next = a.wd[(b * a.T + min(t0 + L, a.T - 1)) * a.H + h];
  // Q's block row sums (blocks (K, Jb), Jb <= K) and column sums (blocks (Ib, K), K <= Ib < nbc)
  const int K = lc >> 6, s = lc & 63;
  const float* qr = a.qrow + ((b * a.Nc + c) * a.H + h) * (int64_t)NB * NB * 128;
  const float* qc = a.qcol + ((b * a.Nc + c) * a.H + h) * (int64_t)NB * NB * 128;
  float qrv[kMaxNB][2], qcv[kMaxNB][2];
#pragma unroll
  for (int k = 0; k < kMaxNB; ++k) {
    const int jb = min(k, K);
    const int ib = min(max(k, K), nbc - 1);
    qrv[k][0] = qr[(K * NB + jb) * 128 + s];
    qrv[k][1] = qr[(K * NB + jb) * 128 + 64 + s];
    qcv[k][0] = qc[(ib * NB + K) * 128 + s];
    qcv[k][1] = qc[(ib * NB + K) * 128 + 64 + s];
  }
  float uvv[kMaxNS][2];
#pragma unroll
  for (int k = 0; k < kMaxNS; ++k) {
    const int ns = min(k, a.NS - 1);
    uvv[k][0] = a.uv[(int64_t)ns * BtT * a.H + rowt];
    uvv[k][1] = a.uv[(int64_t)(a.NS + ns) * BtT * a.H + rowt];
  }
  // <Ghat_c, H_c>, formed beside dx (bwd_ghat_dot)
  const int64_t nbch = a.Bt * a.Nc * a.H;
  float sc = a.part[3 * nbch + (b * a.Nc + c) * a.H + h];
  float dv = 0.0f, uu = 0.0f, vv = 0.0f;
  if (ok) {
    // R_t = sum_{s<t} (column sum of s below the diagonal - row sum of s left of it)
    float rs = 0.0f, cs = 0.0f;
#pragma unroll
    for (int k = 0; k < kMaxNB; ++k) rs += k <= K ? qrv[k][0] + qrv[k][1] : 0.0f;
#pragma unroll
    for (int k = 0; k < kMaxNB; ++k) cs += (k >= K && k < nbc) ? qcv[k][0] + qcv[k][1] : 0.0f;
    dv = cs - rs;
#pragma unroll
    for (int k = 0; k < kMaxNS; ++k) {
      uu += k < a.NS ? uvv[k][0] : 0.0f;
      vv += k < a.NS ? uvv[k][1] : 0.0f;
    }
  }
  const float inc_d = block_inclusive_scan(dv, s_w);
  const float inc_v = block_inclusive_scan(vv, s_w);
  const float inc_u = block_inclusive_scan(uu, s_w);
  const float tot_u = block_sum(uu, s_w);
  const float gs = has_next ? expf(wd_next * Ah) : 1.0f;
  sc *= gs * (float)exp(clast);

  float pA = 0.0f, pB = 0.0f, pD = 0.0f;
  if (ok) {
    const float da = (inc_d - dv) + (tot_u - (inc_u - uu)) + (inc_v - vv) + sc;
    const float z = dt_raw + bias;
    const float pre = a.softplus ? softplus_of(z) : z;   // as in delta_of: the same clip decision
    float gate = (pre >= a.dt_min && pre <= a.dt_max) ? 1.0f : 0.0f;
    if (a.softplus) gate *= 1.0f / (1.0f + expf(-z));
    const float gd = __fmaf_rn(Ah, da, ddin_t) * gate;
    a.ddt[row] = gd;
    pA = wd_t * da;
    pB = gd;
    pD = dDp_t;
  }
  pA = block_sum(pA, s_w);
  pB = block_sum(pB, s_w);
  pD = block_sum(pD, s_w);
  if (l == 0) {
    const int64_t n = a.Bt * a.Nc * a.H, k = (b * a.Nc + c) * a.H + h;
    a.part[k] = pA;
    a.part[n + k] = pB;
    a.part[2 * n + k] = pD;
  }
}

// dA, ddt_bias, dD: sums over the batch and the chunks of the parts (fixed order).
__device__ __forceinline__ void bwd_reduce_heads(const BwdArgs& a, int64_t bid) {
  const int64_t h = bid * kBwdThreads + threadIdx.x;
  if (h >= a.H) return;
  const int64_t n = a.Bt * a.Nc;
  float s[3] = {0.0f, 0.0f, 0.0f};
  // 16 parts of each sum in flight, added in order (rows past n re-read the last)
  for (int64_t k0 = 0; k0 < n; k0 += 16) {
    float v[3][16];
#pragma unroll
    for (int m = 0; m < 3; ++m)
#pragma unroll
      for (int k = 0; k < 16; ++k) v[m][k] = a.part[(m * n + min(k0 + k, n - 1)) * a.H + h];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (k0 + k < n)
#pragma unroll
        for (int m = 0; m < 3; ++m) s[m] += v[m][k];
  }
  a.dA[h] = s[0];
  if (a.ddt_bias_out) a.ddt_bias_out[h] = s[1];
  if (a.dD) a.dD[h] = s[2];
}

// dh0 = abar_0 * (final state of R1).
__device__ __forceinline__ void bwd_dh0(const BwdArgs& a, int64_t bid) {
  const int64_t e = bid * kBwdThreads + threadIdx.x;
  const int64_t PN = (int64_t)a.P * a.N;
  if (e >= a.Bt * a.H * PN) return;
  const int64_t bh = e / PN, h = bh % a.H, b = bh / a.H;
  const float ab0 = expf(a.wd[(b * a.T) * a.H + h] * a.A[h]);
  a.dh0[e] = ab0 * a.r1_final[e];
}

// <Ghat_c, H_c> of one (b, c, h), for the assembly of the decay gradient:
// Ghat_c is R1's state at the next chunk (times that chunk's first abar, which
// the assembly applies) or dfinal for the last chunk; without either the term
// is 0 (the loads then read H_c twice).  Stored after the three parts.
__device__ __forceinline__ void bwd_ghat_dot(const BwdArgs& a, int64_t bid) {
  __shared__ float s_w[kBwdThreads / 64];
  const int l = threadIdx.x;
  const int64_t h = bid % a.H, bc = bid / a.H, c = bc % a.Nc, b = bc / a.Nc;
  const int64_t PN = (int64_t)a.P * a.N;
  const bool has_next = c + 1 < a.Nc;
  const float* Hc = a.fwd_state + ((b * a.H + h) * a.Nc + c) * PN;
  const float* Gh = has_next ? a.r1_state + ((b * a.H + h) * a.Nc + (a.Nc - 1 - c)) * PN
                             : (a.dfinal ? a.dfinal + (b * a.H + h) * PN : nullptr);
  const bool has_g = Gh != nullptr;
  float sc = 0.0f;
  {
    // float4 vectors, eight of each operand in flight per thread; vectors past
    // the state re-read its last one and are dropped
    const float4* g4 = reinterpret_cast<const float4*>(has_g ? Gh : Hc);
    const float4* h4 = reinterpret_cast<const float4*>(Hc);
    const int n4 = (int)(PN / 4);
    for (int e0 = 0; e0 < n4; e0 += 8 * kBwdThreads) {
      float4 gv[8], hv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int e = min(e0 + k * kBwdThreads + l, n4 - 1);
        gv[k] = g4[e];
        hv[k] = h4[e];
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (e0 + k * kBwdThreads + l < n4) {
          sc = __fmaf_rn(gv[k].x, hv[k].x, sc);
          sc = __fmaf_rn(gv[k].y, hv[k].y, sc);
          sc = __fmaf_rn(gv[k].z, hv[k].z, sc);
          sc = __fmaf_rn(gv[k].w, hv[k].w, sc);
        }
      }
    }
    if (!has_g) sc = 0.0f;
  }
  sc = block_sum(sc, s_w);
  if (l == 0) a.part[3 * a.Bt * a.Nc * a.H + bid] = sc;
}

// Independent work in one launch each: the chunk-boundary dots, dx (with the
// per-token parts of the Delta and D gradients) and the sum of the dC / dB
// head-split parts; the per-head sums beside d(initial state).
template <typename T>
__global__ __launch_bounds__(kBwdThreads) void k_bwd_dx_reduce(BwdArgs a, int sh, int64_t n_dot,
                                                               int64_t n_dx) {
  int64_t bid = blockIdx.x;
  if (bid < n_dot) {
    bwd_ghat_dot(a, bid);
    return;
  }
  bid -= n_dot;
  if (bid < n_dx) bwd_dx<T>(a, sh, bid);
  else bwd_dcdb_reduce(a, bid - n_dx);
}
__global__ __launch_bounds__(kBwdThreads) void k_bwd_finish(BwdArgs a, int64_t n_heads) {
  const int64_t bid = blockIdx.x;
  if (bid < n_heads) bwd_reduce_heads(a, bid);
  else bwd_dh0(a, bid - n_heads);
}

inline unsigned blocks_of(int64_t n, int64_t per) { return (unsigned)((n + per - 1) / per); }

inline int log2_of(int v) {   // v a power of two
  int k = 0;
  while ((1 << k) < v) ++k;
  return k;
}

template <typename T, int P>
hipError_t launch_mix_dcdb(const BwdArgs& a, hipStream_t s) {
  const int64_t bcg = a.Bt * a.Nc * a.G;
  const int64_t nbt = (int64_t)a.NB * (a.NB + 1) / 2;
  hipLaunchKernelGGL((k_bwd_mix<T, P>), dim3((unsigned)(bcg * a.HS * nbt)), dim3(kBwdThreads), 0,
                     s, a);
  const dim3 grid((unsigned)(bcg * a.HSD * 2 * a.NS * a.NB));
  switch (a.N) {
    case 16: hipLaunchKernelGGL((k_bwd_dcdb<T, P, 1>), grid, dim3(kBwdThreads), 0, s, a); break;
    case 32: hipLaunchKernelGGL((k_bwd_dcdb<T, P, 2>), grid, dim3(kBwdThreads), 0, s, a); break;
    case 64:
    case 128: hipLaunchKernelGGL((k_bwd_dcdb<T, P, 4>), grid, dim3(kBwdThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_phase(const BwdArgs& a, int phase, hipStream_t s) {
  const int64_t rows = a.Bt * a.T * a.H;
  switch (phase) {
    case 0: {
      Prep0Grid pg;
      pg.n_cd = a.Bt * a.Nc * ((a.H + 15) / 16);
      pg.n_bc = blocks_of(a.Bt * a.T * a.G * (int64_t)(a.N / 4), kBwdThreads);
      pg.sh_bc = log2_of(a.N / 4);
      const int64_t hp = a.pad * a.H * a.P, gn = a.pad * a.G * a.N;
      pg.per_b = hp > gn ? hp : gn;
      pg.n_pad = a.pad > 0 ? blocks_of(a.Bt * pg.per_b, kBwdThreads) : 0;
      const int64_t n_init = blocks_of(a.Bt * a.H * (int64_t)a.P * a.N, kBwdThreads);
      hipLaunchKernelGGL(k_bwd_prep0<T>, dim3((unsigned)(pg.n_cd + pg.n_bc + pg.n_pad + n_init)),
                         dim3(kBwdThreads), 0, s, a, pg);
      // R1's input rows read Delta of the next token
      hipLaunchKernelGGL(k_bwd_prep_x<T>,
                         dim3(blocks_of(rows * (a.P / (16 / (int)sizeof(T))), kBwdThreads)),
                         dim3(kBwdThreads), 0, s, a, log2_of(a.P / (16 / (int)sizeof(T))));
      break;
    }
    case 1: {
      hipError_t e;
      switch (a.P) {
        case 16: e = launch_mix_dcdb<T, 16>(a, s); break;
        case 32: e = launch_mix_dcdb<T, 32>(a, s); break;
        case 64: e = launch_mix_dcdb<T, 64>(a, s); break;
        case 128: e = launch_mix_dcdb<T, 128>(a, s); break;
        default: e = hipErrorInvalidValue;
      }
      if (e != hipSuccess) return e;
      {
        const int64_t n_dx = blocks_of(rows * (a.P / (16 / (int)sizeof(T))), kBwdThreads);
        const int64_t n_red = a.HSD > 1 ? blocks_of(2 * a.Bt * a.T * a.G * (int64_t)a.N, kBwdThreads) : 0;
        const int64_t n_dot = a.Bt * a.Nc * a.H;
        hipLaunchKernelGGL(k_bwd_dx_reduce<T>, dim3((unsigned)(n_dot + n_dx + n_red)),
                           dim3(kBwdThreads), 0, s, a, log2_of(a.P / (16 / (int)sizeof(T))), n_dot,
                           n_dx);
      }
      hipLaunchKernelGGL(k_bwd_assemble, dim3((unsigned)(a.Bt * a.Nc * a.H)), dim3(kBwdThreads),
                         0, s, a);
      {
        const int64_t n_heads = blocks_of(a.H, kBwdThreads);
        const int64_t n_dh0 = a.dh0 ? blocks_of(a.Bt * a.H * (int64_t)a.P * a.N, kBwdThreads) : 0;
        hipLaunchKernelGGL(k_bwd_finish, dim3((unsigned)(n_heads + n_dh0)), dim3(kBwdThreads), 0, s,
                           a, n_heads);
      }
      break;
    }
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
