// Chunked SSD scan (prefill) for gfx950, bfloat16 x/B/C/y.
//
// Source: "Compiler-First State Space Duality and Portable O(1)
// Autoregressive Caching", Background (Eq. 3, inter-chunk recurrence), SSD
// properties ("diagonal state matrix", "chunked recurrence") and
// Implementation ("static masking"; "precision management": decay kept in
// float32 and exponentiated at compute time, bfloat16 only for the io
// tensors).
//
// Same four phases as the float32 path (C B^T per chunk, chunk states,
// inter-chunk recurrence, outputs).  Matrix products run on
// v_mfma_f32_16x16x32_bf16: lane l holds 8 consecutive k-slots of row l%16
// of A (and of column l%16 of B) in group l/16, and the four outputs
// D[4(l/16)+r][l%16].  Decay, states, C B^T and accumulation stay float32;
// operands are rounded to bfloat16 (round to nearest even) right before a
// matrix instruction: the decayed scores (S o decay), the state h_{c-1} in the
// inter-chunk term and x w in the chunk states.
//
// Contractions over tokens (the chunk state X^T diag(w) B and the
// intra-chunk product (S o decay) X) need token-contiguous operands, so x and
// B are transposed on their way into LDS: every thread loads an 8 x 8 block
// (8 rows of 16 bytes) and writes it back as 8 columns of 16 bytes.
#include "ssd_prefill_common.h"

namespace ssd {
namespace prefill {
namespace {

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float4 zero4() { return make_float4(0.f, 0.f, 0.f, 0.f); }

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (bf16)0.0f;
  return z;
}

__device__ __forceinline__ bf16x8 ld8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ void st8(bf16* p, bf16x8 v) { *reinterpret_cast<bf16x8*>(p) = v; }
__device__ __forceinline__ bf16x4 ld4b(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }

__device__ __forceinline__ bf16x8 cat(bf16x4 lo, bf16x4 hi) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) { r[i] = lo[i]; r[4 + i] = hi[i]; }
  return r;
}

// 8 x 8 transpose of bf16: out[c][r] = in[r][c]
__device__ __forceinline__ void transpose8(const bf16x8 (&in)[8], bf16x8 (&out)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 8; ++r) out[c][r] = in[r][c];
}

// ---------------------------------------------------------------------------
// Phase 0: S = C B^T (float32) for the causal 16x16 tiles of every (b, c, g).
// One wavefront computes one tile (I, J), J <= I.
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ void cb_tile_bf16(const ScanArgs& a, int ntiles, int64_t block) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, q = lane >> 4, r16 = lane & 15;
  const int64_t item = block * 4 + wave;
  const int64_t bcg = item / ntiles;
  if (bcg >= a.Bt * a.Nc * a.G) return;
  const int t = (int)(item % ntiles);
  int I = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((I + 1) * (I + 2) / 2 <= t) ++I;
  while (I * (I + 1) / 2 > t) --I;
  const int J = t - I * (I + 1) / 2;
  const int64_t g = bcg % a.G, bc = bcg / a.G, c = bc % a.Nc, b = bc / a.Nc;
  const int64_t t0 = c * a.L;
  const int Lc = chunk_len(a, c);
  if (16 * I >= Lc) return;
  const bf16* Cg = reinterpret_cast<const bf16*>(a.C) + ((b * a.T + t0) * a.G + g) * N + 8 * q;
  const bf16* Bg = reinterpret_cast<const bf16*>(a.B) + ((b * a.T + t0) * a.G + g) * N + 8 * q;
  const int64_t rs = a.G * N;
  const int ri = 16 * I + r16, rj = 16 * J + r16;
  bf16x8 cf[N / 32], bf[N / 32];
#pragma unroll
  for (int nb = 0; nb < N / 32; ++nb) {
    cf[nb] = ri < Lc ? ld8(Cg + ri * rs + nb * 32) : zero8();
    bf[nb] = rj < Lc ? ld8(Bg + rj * rs + nb * 32) : zero8();
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nb = 0; nb < N / 32; ++nb) acc = mma(cf[nb], bf[nb], acc);
  float* S = a.ws_cb + bcg * a.L * a.L;
#pragma unroll
  for (int r = 0; r < 4; ++r) S[(int64_t)(16 * I + 4 * q + r) * a.L + 16 * J + r16] = acc[r];
}

// ---------------------------------------------------------------------------
// Phase 1: chunk summary states S_c[p][n] = sum_l (x_l[p] w_l) B_l[n],
// w_l = Delta_l exp(cum_last - cum_l).  Tokens are staged 64 at a time,
// transposed (token-contiguous rows), double-buffered in LDS.
// ---------------------------------------------------------------------------
template <int P, int N>
struct ChunkStateShapeB {
  static constexpr int KB = 64;
  static constexpr int TS = KB + 8;   // LDS row stride (elements) of the transposed blocks
};

template <int P, int N>
__device__ __forceinline__ void chunk_state_bf16(const ScanArgs& a, int64_t block, int64_t nblocks,
                                                 float* s_d, float* s_cum, float* s_w,
                                                 float* s_wsum, bf16* s_x0, bf16* s_x1,
                                                 bf16* s_b0, bf16* s_b1) {
  using Sh = ChunkStateShapeB<P, N>;
  constexpr int KB = Sh::KB, TS = Sh::TS;
  constexpr int TP = P / 16, TN = N / 16, TT = TP * TN;
  constexpr int TPW = TT >= 4 ? TT / 4 : 1;          // output tiles per wavefront
  constexpr int NNT = TPW < TN ? TPW : TN;
  constexpr int NPT = TPW / NNT;
  // 8 x 8 transpose blocks of one stage: x (KB/8 x P/8), B (KB/8 x N/8)
  constexpr int XBLK = (KB / 8) * (P / 8), BBLK = (KB / 8) * (N / 8);
  constexpr int NB8 = (XBLK + BBLK + kThreads - 1) / kThreads;  // blocks per thread

  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t u = xcd_remap(block, nblocks);
  const int64_t h = u % a.H, bc = u / a.H, c = bc % a.Nc, b = bc / a.Nc;
  const int64_t g = h / (a.H / a.G);
  const int64_t t0 = c * a.L;
  const int Lc = chunk_len(a, c);
  const bf16* xg = reinterpret_cast<const bf16*>(a.x) + ((b * a.T + t0) * a.H + h) * P;
  const bf16* Bg = reinterpret_cast<const bf16*>(a.B) + ((b * a.T + t0) * a.G + g) * N;
  const int64_t xstride = a.H * P, bstride = a.G * N;

  // this thread's 8x8 blocks: id < XBLK -> x block, else B block
  auto load_block = [&](int kb0, bf16x8 (&v)[NB8][8]) {
#pragma unroll
    for (int i = 0; i < NB8; ++i) {
      const int id = tid + i * kThreads;
      if (id < XBLK) {
        const int lb = id / (P / 8), cb = id % (P / 8);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int l = kb0 + 8 * lb + r;
          v[i][r] = l < Lc ? ld8(xg + l * xstride + 8 * cb) : zero8();
        }
      } else if (id < XBLK + BBLK) {
        const int id2 = id - XBLK, lb = id2 / (N / 8), cb = id2 % (N / 8);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int l = kb0 + 8 * lb + r;
          v[i][r] = l < Lc ? ld8(Bg + l * bstride + 8 * cb) : zero8();
        }
      }
    }
  };
  auto store_block = [&](int kb0, const bf16x8 (&v)[NB8][8], bf16* sx, bf16* sb) {
#pragma unroll
    for (int i = 0; i < NB8; ++i) {
      const int id = tid + i * kThreads;
      bf16x8 tr[8];
      if (id < XBLK) {
        const int lb = id / (P / 8), cb = id % (P / 8);
        bf16x8 in[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float w = s_w[kb0 + 8 * lb + r];
#pragma unroll
          for (int e = 0; e < 8; ++e) in[r][e] = (bf16)((float)v[i][r][e] * w);
        }
        transpose8(in, tr);
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) st8(sx + (8 * cb + cc) * TS + 8 * lb, tr[cc]);
      } else if (id < XBLK + BBLK) {
        const int id2 = id - XBLK, lb = id2 / (N / 8), cb = id2 % (N / 8);
        transpose8(v[i], tr);
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) st8(sb + (8 * cb + cc) * TS + 8 * lb, tr[cc]);
      }
    }
  };
  bf16x8 vA[NB8][8];
  load_block(0, vA);   // in flight during the prologue

  chunk_delta_cumsum(a, b, c, h, s_d, s_cum, s_wsum);
  const float cum_last = s_cum[Lc - 1];
  for (int l = tid; l < (int)a.L; l += kThreads)
    s_w[l] = (l < Lc) ? s_d[l] * fast_exp(cum_last - s_cum[l]) : 0.0f;
  if (tid == 0) a.ws_alpha[(b * a.H + h) * a.Nc + c] = fast_exp(cum_last);
  __syncthreads();

  const bool active = TT >= 4 || wave < TT;
  const int tile0 = wave * TPW;
  const int pt0 = tile0 / TN, nt0 = tile0 % TN;
  f32x4 acc[NPT][NNT];
#pragma unroll
  for (int ip = 0; ip < NPT; ++ip)
#pragma unroll
    for (int in = 0; in < NNT; ++in) acc[ip][in] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const bf16* sx, const bf16* sb) {
    if (!active) return;
#pragma unroll
    for (int ks = 0; ks < KB; ks += 32) {
      bf16x8 av[NPT], bv[NNT];
#pragma unroll
      for (int ip = 0; ip < NPT; ++ip) av[ip] = ld8(sx + ((pt0 + ip) * 16 + r16) * TS + ks + 8 * q);
#pragma unroll
      for (int in = 0; in < NNT; ++in) bv[in] = ld8(sb + ((nt0 + in) * 16 + r16) * TS + ks + 8 * q);
#pragma unroll
      for (int ip = 0; ip < NPT; ++ip)
#pragma unroll
        for (int in = 0; in < NNT; ++in) acc[ip][in] = mma(av[ip], bv[in], acc[ip][in]);
    }
  };
  int buf = 0;
  for (int kb0 = 0; kb0 < Lc; kb0 += KB, buf ^= 1) {
    bf16* sx = buf ? s_x1 : s_x0;
    bf16* sb = buf ? s_b1 : s_b0;
    store_block(kb0, vA, sx, sb);
    __syncthreads();
    if (kb0 + KB < Lc) load_block(kb0 + KB, vA);
    compute(sx, sb);
  }
  if (active) {
    float* out = a.ws_state + ((b * a.H + h) * a.Nc + c) * (int64_t)(P * N);
#pragma unroll
    for (int ip = 0; ip < NPT; ++ip)
#pragma unroll
      for (int in = 0; in < NNT; ++in)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          out[((pt0 + ip) * 16 + 4 * q + r) * N + (nt0 + in) * 16 + r16] = acc[ip][in][r];
  }
}

template <int P, int N>
__global__ __launch_bounds__(kThreads) void k_cb_and_chunk_state_bf16(ScanArgs a, int ntiles,
                                                                      int64_t ncb) {
  using Sh = ChunkStateShapeB<P, N>;
  __shared__ float s_d[kMaxL], s_cum[kMaxL], s_w[kMaxL], s_wsum[4];
  __shared__ __attribute__((aligned(16))) bf16 s_x[2][P * Sh::TS];
  __shared__ __attribute__((aligned(16))) bf16 s_b[2][N * Sh::TS];
  if ((int64_t)blockIdx.x < ncb) {
    cb_tile_bf16<N>(a, ntiles, blockIdx.x);
    return;
  }
  chunk_state_bf16<P, N>(a, blockIdx.x - ncb, gridDim.x - ncb, s_d, s_cum, s_w, s_wsum, s_x[0],
                         s_x[1], s_b[0], s_b[1]);
}

// ---------------------------------------------------------------------------
// Phase 3: chunk outputs, one workgroup per (b, c, h).  Wavefront w owns the
// 16-row tiles row_tile_of(w, k), k < RT, and keeps all their accumulators.
// x is staged transposed (x^T[p][j]) for the whole chunk.  Decay factors as
// in the float32 path: factored through the 64-token block boundary for
// earlier blocks, masked exponentials inside the row tile's own block.
// ---------------------------------------------------------------------------
template <int P, int N, int LMAX>
__global__ __launch_bounds__(kThreads) void k_chunk_out_bf16(ScanArgs a) {
  constexpr int TP = P / 16;
  constexpr int NBLK = LMAX / 64, RT = NBLK;
  constexpr int XTS = LMAX + 8;          // row stride of x^T (elements)
  __shared__ __attribute__((aligned(16))) float s_d[LMAX];
  __shared__ __attribute__((aligned(16))) float s_cum[LMAX];
  __shared__ float s_wsum[4];
  __shared__ __attribute__((aligned(16))) float s_w[(NBLK - 1) * LMAX];
  __shared__ __attribute__((aligned(16))) bf16 s_xt[P * XTS];

  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t u = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t h = u % a.H, bc = u / a.H, c = bc % a.Nc, b = bc / a.Nc;
  const int64_t g = h / (a.H / a.G);
  const int64_t t0 = c * a.L;
  const int Lc = chunk_len(a, c);
  const int nrt = (Lc + 15) / 16;
  const bf16* xg = reinterpret_cast<const bf16*>(a.x) + ((b * a.T + t0) * a.H + h) * P;
  const int64_t xstride = a.H * P;

  // stage x^T: 8x8 blocks, loads of a batch issued before the transposes/stores
  {
    const int nblk8 = ((nrt * 16) / 8) * (P / 8);
    for (int e0 = 0; e0 < nblk8; e0 += kThreads) {
      const int id = e0 + tid;
      const int lb = id / (P / 8), cb = id % (P / 8);
      bf16x8 in[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int l = 8 * lb + r;
        in[r] = (id < nblk8 && l < Lc) ? ld8(xg + l * xstride + 8 * cb) : zero8();
      }
      if (id < nblk8) {
        bf16x8 tr[8];
        transpose8(in, tr);
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) st8(s_xt + (8 * cb + cc) * XTS + 8 * lb, tr[cc]);
      }
    }
  }
  chunk_delta_cumsum(a, b, c, h, s_d, s_cum, s_wsum);  // ends with a barrier
  for (int e = tid; e < (NBLK - 1) * LMAX; e += kThreads) {
    const int R = e / LMAX + 1, j = e % LMAX;
    const int r = min(64 * R, Lc - 1);
    s_w[e] = (j < r) ? fast_exp(s_cum[r] - s_cum[j]) * s_d[j] : 0.0f;
  }
  __syncthreads();

  int Ik[RT];
  bool vk[RT];
  float cumk[RT];
#pragma unroll
  for (int k = 0; k < RT; ++k) {
    Ik[k] = row_tile_of(wave, k);
    vk[k] = Ik[k] < nrt;
    cumk[k] = s_cum[min(16 * Ik[k] + r16, Lc - 1)];
  }
  f32x4 acc[RT][TP];
#pragma unroll
  for (int k = 0; k < RT; ++k)
#pragma unroll
    for (int pt = 0; pt < TP; ++pt) acc[k][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- inter-chunk term: acc[k] = exp(cum_i) * sum_n C[i][n] h_{c-1}[p][n] ----
  {
    const bf16* Cg = reinterpret_cast<const bf16*>(a.C) + ((b * a.T + t0) * a.G + g) * N + 8 * q;
    const int64_t crs = a.G * N;
    const float* hp = a.ws_state + ((b * a.H + h) * a.Nc + c) * (int64_t)(P * N) +
                      (int64_t)r16 * N + 8 * q;
#pragma unroll 1
    for (int nb = 0; nb < N / 32; ++nb) {
      float4 hv[TP][2];
      bf16x8 cv[RT];
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) {
        hv[pt][0] = ld4(hp + pt * 16 * N + nb * 32);
        hv[pt][1] = ld4(hp + pt * 16 * N + nb * 32 + 4);
      }
#pragma unroll
      for (int k = 0; k < RT; ++k) {
        const int ri = 16 * Ik[k] + r16;
        cv[k] = (vk[k] && ri < Lc) ? ld8(Cg + ri * crs + nb * 32) : zero8();
      }
      bf16x8 hb[TP];
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) {
        hb[pt][0] = (bf16)hv[pt][0].x; hb[pt][1] = (bf16)hv[pt][0].y;
        hb[pt][2] = (bf16)hv[pt][0].z; hb[pt][3] = (bf16)hv[pt][0].w;
        hb[pt][4] = (bf16)hv[pt][1].x; hb[pt][5] = (bf16)hv[pt][1].y;
        hb[pt][6] = (bf16)hv[pt][1].z; hb[pt][7] = (bf16)hv[pt][1].w;
      }
#pragma unroll
      for (int k = 0; k < RT; ++k) {
        if (!vk[k]) continue;
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) acc[k][pt] = mma(cv[k], hb[pt], acc[k][pt]);
      }
    }
    // decay from the chunk start: rows 16 I + 4q + r of the accumulators
#pragma unroll
    for (int k = 0; k < RT; ++k) {
      if (!vk[k]) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * Ik[k] + 4 * q + r;
        const float sc = i < Lc ? fast_exp(s_cum[i]) : 0.0f;
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) acc[k][pt][r] *= sc;
      }
    }
  }

  // ---- intra-chunk term: row tile by row tile, 64 keys (two 32-key slots) at a time ----
  const float* S = a.ws_cb + ((b * a.Nc + c) * a.G + g) * a.L * a.L;
#pragma unroll
  for (int k = 0; k < RT; ++k) {
    if (!vk[k]) continue;
    const int I = Ik[k], R = I >> 2;
    const int ri = 16 * I + r16;
    const float cum_i = cumk[k];
    const float* sr = S + (int64_t)ri * a.L + 4 * q;
    // a 64-key block is 4 key tiles; tile t of the block is read as S[ri][16t + 4q .. +3]
    auto load_s = [&](int jb, float4 (&st)[4]) {
#pragma unroll
      for (int t = 0; t < 4; ++t) st[t] = ld4(sr + 64 * jb + 16 * min(t, I - 4 * jb));
    };
    const float u_i = R > 0 ? fast_exp(cum_i - s_cum[64 * R]) : 0.0f;
    auto block = [&](int jb, const float4 (&st)[4]) {
      // k-slots of a 32-key half (tiles 2s, 2s+1): slot e<4 -> key 16(2s)+4q+e,
      // slot e>=4 -> key 16(2s+1)+4q+e-4
      const bf16* xq = s_xt + (int64_t)r16 * XTS + 64 * jb + 4 * q;
      if (jb < R) {
        const float* wrow = &s_w[(R - 1) * LMAX + 64 * jb + 4 * q];
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
          const float4 w0 = ld4(wrow + 32 * sh), w1 = ld4(wrow + 32 * sh + 16);
          const float4 s0 = st[2 * sh], s1 = st[2 * sh + 1];
          bf16x8 m;
          m[0] = (bf16)(s0.x * u_i * w0.x); m[1] = (bf16)(s0.y * u_i * w0.y);
          m[2] = (bf16)(s0.z * u_i * w0.z); m[3] = (bf16)(s0.w * u_i * w0.w);
          m[4] = (bf16)(s1.x * u_i * w1.x); m[5] = (bf16)(s1.y * u_i * w1.y);
          m[6] = (bf16)(s1.z * u_i * w1.z); m[7] = (bf16)(s1.w * u_i * w1.w);
#pragma unroll
          for (int pt = 0; pt < TP; ++pt) {
            const bf16* xr = xq + pt * 16 * XTS + 32 * sh;
            acc[k][pt] = mma(m, cat(ld4b(xr), ld4b(xr + 16)), acc[k][pt]);
          }
        }
      } else {
        const int nt = I - 4 * R + 1;          // key tiles up to the diagonal (uniform)
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
          if (2 * sh < nt) {
            const int j0 = 64 * jb + 32 * sh + 4 * q;   // keys j0..j0+3 and j0+16..j0+19
            const float4 c0 = ld4(&s_cum[j0]), c1 = ld4(&s_cum[j0 + 16]);
            const float4 d0 = ld4(&s_d[j0]), d1 = ld4(&s_d[j0 + 16]);
            const float4 s0 = st[2 * sh], s1 = st[2 * sh + 1];
            const bool hi = 2 * sh + 1 < nt;
            bf16x8 m;
            m[0] = (bf16)((j0 + 0 <= ri) ? s0.x * fast_exp(cum_i - c0.x) * d0.x : 0.0f);
            m[1] = (bf16)((j0 + 1 <= ri) ? s0.y * fast_exp(cum_i - c0.y) * d0.y : 0.0f);
            m[2] = (bf16)((j0 + 2 <= ri) ? s0.z * fast_exp(cum_i - c0.z) * d0.z : 0.0f);
            m[3] = (bf16)((j0 + 3 <= ri) ? s0.w * fast_exp(cum_i - c0.w) * d0.w : 0.0f);
            m[4] = (bf16)((hi && j0 + 16 <= ri) ? s1.x * fast_exp(cum_i - c1.x) * d1.x : 0.0f);
            m[5] = (bf16)((hi && j0 + 17 <= ri) ? s1.y * fast_exp(cum_i - c1.y) * d1.y : 0.0f);
            m[6] = (bf16)((hi && j0 + 18 <= ri) ? s1.z * fast_exp(cum_i - c1.z) * d1.z : 0.0f);
            m[7] = (bf16)((hi && j0 + 19 <= ri) ? s1.w * fast_exp(cum_i - c1.w) * d1.w : 0.0f);
            // the upper key tile may lie past the staged rows: never read it then
            // (uninitialised LDS could hold a NaN pattern, and 0 * NaN = NaN)
            bf16x4 z4;
#pragma unroll
            for (int e = 0; e < 4; ++e) z4[e] = (bf16)0.0f;
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) {
              const bf16* xr = xq + pt * 16 * XTS + 32 * sh;
              acc[k][pt] = mma(m, cat(ld4b(xr), hi ? ld4b(xr + 16) : z4), acc[k][pt]);
            }
          }
        }
      }
    };
    float4 sa[4], sb[4];
    load_s(0, sa);
    for (int jb = 0; jb <= R; jb += 2) {
      if (jb + 1 <= R) load_s(jb + 1, sb);
      block(jb, sa);
      if (jb + 1 > R) break;
      if (jb + 2 <= R) load_s(jb + 2, sa);
      block(jb + 1, sb);
    }
  }

  // ---- skip term and store ----
  const float Dh = a.D ? a.D[h] : 0.0f;
  bf16* yg = reinterpret_cast<bf16*>(a.y);
#pragma unroll
  for (int k = 0; k < RT; ++k) {
    if (!vk[k]) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * Ik[k] + 4 * q + r;
      if (i < Lc) {
        const int64_t row = ((b * a.T + t0 + i) * a.H + h) * P;
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) {
          const int p = pt * 16 + r16;
          yg[row + p] = (bf16)(acc[k][pt][r] + Dh * (float)s_xt[p * XTS + i]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------
template <int P, int N>
hipError_t launch_pn(const ScanArgs& a, hipStream_t stream, hipEvent_t* ev) {
  hipError_t e;
  auto rec = [&](int k) -> hipError_t { return ev ? hipEventRecord(ev[k], stream) : hipSuccess; };
  if ((e = rec(0)) != hipSuccess) return e;
  if ((e = rec(1)) != hipSuccess) return e;
  const int nrt = (int)((a.L + 15) / 16), ntiles = nrt * (nrt + 1) / 2;
  const int64_t items = a.Bt * a.Nc * a.G * ntiles;
  const int64_t ncb = ((items + 3) / 4 + 7) / 8 * 8;
  const int64_t units = a.Bt * a.Nc * a.H;
  hipLaunchKernelGGL((k_cb_and_chunk_state_bf16<P, N>), dim3((unsigned)(ncb + units)),
                     dim3(kThreads), 0, stream, a, ntiles, ncb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = rec(2)) != hipSuccess) return e;
  if ((e = launch_state_pass(a, P, N, stream)) != hipSuccess) return e;
  if ((e = rec(3)) != hipSuccess) return e;
  if (a.L <= 256) {
    hipLaunchKernelGGL((k_chunk_out_bf16<P, N, 256>), dim3((unsigned)units), dim3(kThreads), 0,
                       stream, a);
  } else {
    if constexpr (P <= 64) {
      hipLaunchKernelGGL((k_chunk_out_bf16<P, N, 512>), dim3((unsigned)units), dim3(kThreads), 0,
                         stream, a);
    } else {
      return hipErrorInvalidValue;
    }
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return rec(4);
}

template <int P>
hipError_t launch_p(const ScanArgs& a, int N, hipStream_t s, hipEvent_t* ev) {
  switch (N) {
    case 32: return launch_pn<P, 32>(a, s, ev);
    case 64: return launch_pn<P, 64>(a, s, ev);
    case 128: return launch_pn<P, 128>(a, s, ev);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace prefill

hipError_t launch_scan_bf16(const ScanArgs& a, int P, int N, hipStream_t s, hipEvent_t* ev) {
  switch (P) {
    case 16: return prefill::launch_p<16>(a, N, s, ev);
    case 32: return prefill::launch_p<32>(a, N, s, ev);
    case 64: return prefill::launch_p<64>(a, N, s, ev);
    case 128: return prefill::launch_p<128>(a, N, s, ev);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssd
