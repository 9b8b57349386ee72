// Chunked SSD scan (prefill) for gfx950, float32 x/B/C/y.
//
// Source: "Compiler-First State Space Duality and Portable O(1)
// Autoregressive Caching", Background (Eq. 3, inter-chunk recurrence), SSD
// properties ("diagonal state matrix", "chunked recurrence") and
// Implementation ("static masking": prefix sum, subtraction, mask and
// exponentiation fused around the contractions; "precision management": the
// highest matmul precision -- here full float32 matrix-core products, there is
// no reduced-precision float32 mode on gfx950).
//
// Per (batch b, chunk c of L tokens, head h; g = B/C group of h), with
// Delta_l the clipped softplus step, cum_l = sum_{k<=l} Delta_k A[h]:
//   phase 0  S   = C_c B_c^T                       (once per (b, c, g), causal tiles)
//   phase 1  S_c = sum_l exp(cum_last - cum_l) Delta_l x_l (x) B_l,  alpha_c = exp(cum_last)
//   phase 2  h_{c-1} for every chunk               (ssd_state_pass.hip)
//   phase 3  y_i = exp(cum_i) C_i h_{c-1}^T
//                + sum_{j<=i} S[i][j] exp(cum_i - cum_j) Delta_j x_j + D x_i
// The decay factor exp(cum_i - cum_j) is formed in registers as each score
// tile is consumed; the causal mask is a select taken before the exponential.
//
// Matrix-core layout (v_mfma_f32_16x16x4_f32): lane l holds one A element
// A[l%16][k], one B element B[k][l%16] and four outputs D[4(l/16)+r][l%16].
// The contraction index is free to permute, so for contractions over a
// contiguous dimension (n in C B^T and C h^T, j in S x) lane l uses
// k = 16*blk + 4*(l/16) + kk, kk = 0..3: each lane then reads one float4 of
// plain row-major data per four instructions.
#include "ssd_prefill_common.h"

namespace ssd {
namespace prefill {
namespace {

__device__ __forceinline__ f32x4 mma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float4 zero4() { return make_float4(0.f, 0.f, 0.f, 0.f); }

// ---------------------------------------------------------------------------
// Phase 0: S = C B^T for the causal 16x16 tiles of every (b, c, g).
// One wavefront computes tile t of (b, c, g) = bcg: (I, J), J <= I.  The
// tiles are shared out among the chunk-state workgroups of the same
// (b, c, g), which compute them after their own state.
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ void cb_tile_f32(const ScanArgs& a, int64_t bcg, int t) {
  const int lane = threadIdx.x & 63, q = lane >> 4, r16 = lane & 15;
  // triangular index t -> (I, J), 0 <= J <= I
  int I = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((I + 1) * (I + 2) / 2 <= t) ++I;
  while (I * (I + 1) / 2 > t) --I;
  const int J = t - I * (I + 1) / 2;
  const int64_t g = bcg % a.G, bc = bcg / a.G, c = bc % a.Nc, b = bc / a.Nc;
  const int64_t t0 = c * a.L;
  const int Lc = chunk_len(a, c);
  if (16 * I >= Lc) return;
  const float* Cg = reinterpret_cast<const float*>(a.C) + ((b * a.T + t0) * a.G + g) * N + 4 * q;
  const float* Bg = reinterpret_cast<const float*>(a.B) + ((b * a.T + t0) * a.G + g) * N + 4 * q;
  const int64_t rs = a.G * N;
  const int ri = 16 * I + r16, rj = 16 * J + r16;
  float4 cf[N / 16], bf[N / 16];
#pragma unroll
  for (int nb = 0; nb < N / 16; ++nb) {
    cf[nb] = ld4_masked(Cg + min(ri, Lc - 1) * rs + nb * 16, ri < Lc);
    bf[nb] = ld4_masked(Bg + min(rj, Lc - 1) * rs + nb * 16, rj < Lc);
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nb = 0; nb < N / 16; ++nb) {
    acc = mma(cf[nb].x, bf[nb].x, acc);
    acc = mma(cf[nb].y, bf[nb].y, acc);
    acc = mma(cf[nb].z, bf[nb].z, acc);
    acc = mma(cf[nb].w, bf[nb].w, acc);
  }
  float* S = a.ws_cb + bcg * a.L * a.L;
#pragma unroll
  for (int r = 0; r < 4; ++r) S[(int64_t)(16 * I + 4 * q + r) * a.L + 16 * J + r16] = acc[r];
}

// ---------------------------------------------------------------------------
// Phase 1: chunk summary states S_c[p][n] = sum_l (x_l[p] w_l) B_l[n],
// w_l = Delta_l exp(cum_last - cum_l), computed as tiles of S_c^T (rows n) so
// that each lane stores four consecutive n of one p.  A workgroup covers NW
// of the N state columns.  Tokens go through LDS in double-buffered blocks of KB: the global
// loads of block k+1 are in flight while block k feeds the matrix cores.
// ---------------------------------------------------------------------------
template <int P, int N, int NW>
struct ChunkStateShape {
  static constexpr int KB = 32;
  static constexpr int XS = P + 4, BS = NW + 4;  // = 4 (mod 8): conflict-free fragment reads
};

template <int P, int N, int NW>
__device__ __forceinline__ void chunk_state_f32(const ScanArgs& a, int ntiles, int64_t block,
                                                int64_t nblocks,
                                                float* s_d, float* s_cum, float* s_w, float* s_wsum,
                                                float* s_x0, float* s_x1, float* s_b0, float* s_b1) {
  using Sh = ChunkStateShape<P, N, NW>;
  constexpr int NSPLIT = N / NW;
  constexpr int KB = Sh::KB, XS = Sh::XS, BS = Sh::BS;
  constexpr int TP = P / 16, TN = NW / 16, TT = TP * TN;
  // output tiles of one wavefront: NPT p-tiles x NNT n-tiles
  constexpr int TPW = TT >= 4 ? TT / 4 : 1;
  constexpr int NNT = TPW < TN ? TPW : TN;
  constexpr int NPT = TPW / NNT;
  constexpr int XQ = P / 4, BQ = NW / 4;                  // float4 per staged row
  constexpr int XL = (KB * XQ + kThreads - 1) / kThreads;  // float4 loads per thread
  constexpr int BL = (KB * BQ + kThreads - 1) / kThreads;

  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t u = xcd_remap(block, nblocks);
  const int ns = (int)(u % NSPLIT);
  const int64_t u2 = u / NSPLIT;
  const int64_t h = u2 % a.H, bc = u2 / a.H, c = bc % a.Nc, b = bc / a.Nc;
  const int64_t g = h / (a.H / a.G);
  const int64_t t0 = c * a.L;
  const int Lc = chunk_len(a, c);
  const float* xg = reinterpret_cast<const float*>(a.x) + ((b * a.T + t0) * a.H + h) * P;
  const float* Bg = reinterpret_cast<const float*>(a.B) + ((b * a.T + t0) * a.G + g) * N + ns * NW;
  const int64_t xstride = a.H * P, bstride = a.G * N;

  auto load_block = [&](int kb0, float4 (&xr)[XL], float4 (&br)[BL]) {
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      const int e = tid + i * kThreads, l = e / XQ, m = e % XQ;
      xr[i] = ld4_masked(&xg[min(kb0 + l, Lc - 1) * xstride + 4 * m], e < KB * XQ && kb0 + l < Lc);
    }
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      const int e = tid + i * kThreads, l = e / BQ, m = e % BQ;
      br[i] = ld4_masked(&Bg[min(kb0 + l, Lc - 1) * bstride + 4 * m], e < KB * BQ && kb0 + l < Lc);
    }
  };
  auto store_block = [&](int kb0, const float4 (&xr)[XL], const float4 (&br)[BL], float* sx,
                         float* sb) {
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      const int e = tid + i * kThreads, l = e / XQ, m = e % XQ;
      if (e < KB * XQ) {
        const float w = s_w[kb0 + l];
        float4 v = xr[i];
        v.x *= w; v.y *= w; v.z *= w; v.w *= w;
        st4(&sx[l * XS + 4 * m], v);
      }
    }
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      const int e = tid + i * kThreads, l = e / BQ, m = e % BQ;
      if (e < KB * BQ) st4(&sb[l * BS + 4 * m], br[i]);
    }
  };
  // Two token blocks are always in flight ahead of the one being consumed.
  // The loads are unconditional (rows past the chunk's end are clamped and
  // zeroed), so every path has the same loads in flight and each wait covers
  // exactly the block about to be staged.
  const float2 dtv = chunk_dt_load(a, b, c, h);
  float4 xA[XL], bA[BL], xB[XL], bB[BL];
  load_block(0, xA, bA);
  load_block(KB, xB, bB);

  {
    const DeltaScan ds = chunk_scan_stage1(a, c, h, dtv, s_wsum);
    __syncthreads();
    chunk_scan_stage2(a, ds, s_wsum, s_d, s_cum);
    __syncthreads();
  }
  const float cum_last = s_cum[Lc - 1];
  for (int l = tid; l < (int)a.L; l += kThreads)
    s_w[l] = (l < Lc) ? s_d[l] * fast_exp(cum_last - s_cum[l]) : 0.0f;
  if (tid == 0 && ns == 0) a.ws_alpha[(b * a.H + h) * a.Nc + c] = fast_exp(cum_last);
  __syncthreads();

  const bool active = TT >= 4 || wave < TT;   // uniform per wavefront
  const int tile0 = wave * TPW;
  const int pt0 = tile0 / TN, nt0 = tile0 % TN;
  f32x4 acc[NPT][NNT];
#pragma unroll
  for (int ip = 0; ip < NPT; ++ip)
#pragma unroll
    for (int in = 0; in < NNT; ++in) acc[ip][in] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const float* sx, const float* sb) {
    if (!active) return;
    // token of k-slot (ks, q, kk) = ks + 4q + kk; all fragments of the block are
    // read before its MFMAs, so the LDS latency is paid once per block
    const float* xa = &sx[4 * q * XS + pt0 * 16 + r16];
    const float* xb = &sb[4 * q * BS + nt0 * 16 + r16];
    float av[KB / 4][NPT], bv[KB / 4][NNT];
#pragma unroll
    for (int k = 0; k < KB / 4; ++k) {
      const int row = (k / 4) * 16 + (k % 4);
#pragma unroll
      for (int ip = 0; ip < NPT; ++ip) av[k][ip] = xa[row * XS + ip * 16];
#pragma unroll
      for (int in = 0; in < NNT; ++in) bv[k][in] = xb[row * BS + in * 16];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < KB / 4; ++k)
#pragma unroll
      for (int ip = 0; ip < NPT; ++ip)
#pragma unroll
        for (int in = 0; in < NNT; ++in) acc[ip][in] = mma(bv[k][in], av[k][ip], acc[ip][in]);
  };
  for (int kb0 = 0; kb0 < Lc; kb0 += 2 * KB) {
    store_block(kb0, xA, bA, s_x0, s_b0);
    __syncthreads();
    load_block(kb0 + 2 * KB, xA, bA);
    compute(s_x0, s_b0);
    if (kb0 + KB >= Lc) break;
    store_block(kb0 + KB, xB, bB, s_x1, s_b1);
    __syncthreads();
    load_block(kb0 + 3 * KB, xB, bB);
    compute(s_x1, s_b1);
  }
  if (active) {
    // tiles are S_c^T [n][p]: lane holds S_c[p = 16 pt + r16][n = 16 nt + 4q .. +3]
    float* out = a.ws_state + ((b * a.H + h) * a.Nc + c) * (int64_t)(P * N) + ns * NW;
#pragma unroll
    for (int ip = 0; ip < NPT; ++ip)
#pragma unroll
      for (int in = 0; in < NNT; ++in) {
        const f32x4 v = acc[ip][in];
        st4(out + ((pt0 + ip) * 16 + r16) * N + (nt0 + in) * 16 + 4 * q,
            make_float4(v[0], v[1], v[2], v[3]));
      }
  }
  // this workgroup's share of the causal C B^T tiles of (b, c, g)
  {
    const int hpg = (int)(a.H / a.G);
    const int nwg = hpg * NSPLIT;                       // chunk-state workgroups of (b, c, g)
    const int wi = (int)(h % hpg) * NSPLIT + ns;
    const int64_t bcg = (b * a.Nc + c) * a.G + g;
    for (int t = wi * 4 + wave; t < ntiles; t += nwg * 4) cb_tile_f32<N>(a, bcg, t);
  }
}

// Phases 0 and 1 share one launch: every chunk-state workgroup also computes
// its share of the C B^T tiles of its (b, c, g) once its state is stored (a
// few tiles each; separate short workgroups ahead of the chunk-state ones
// would hold their slots and delay them).
template <int P, int N, int NW>
__global__ __launch_bounds__(kThreads) void k_cb_and_chunk_state_f32(ScanArgs a, int ntiles) {
  using Sh = ChunkStateShape<P, N, NW>;
  __shared__ float s_d[kMaxL], s_cum[kMaxL], s_w[kMaxL], s_wsum[4];
  __shared__ __attribute__((aligned(16))) float s_x[2][Sh::KB * Sh::XS];
  __shared__ __attribute__((aligned(16))) float s_b[2][Sh::KB * Sh::BS];
  chunk_state_f32<P, N, NW>(a, ntiles, blockIdx.x, gridDim.x, s_d, s_cum, s_w, s_wsum, s_x[0],
                            s_x[1], s_b[0], s_b[1]);
}

// ---------------------------------------------------------------------------
// Phase 3: chunk outputs.  A workgroup covers PW of the P head columns of one
// (b, c, h).  Wavefront w owns the 16-token column tiles row_tile_of(w, k),
// k < RT, of y^T (tiles [p][i]) and keeps all their accumulators live, so
// every h and x fragment it loads serves all of its tiles.  Computing y^T
// rather than y puts four consecutive head columns of one token in each lane:
// the skip term and the store are float4 accesses.
//
// Order: the inter-chunk term needs only h_{c-1} and C, the staging (prefix
// sum, x into LDS, decay tables) only dt and x, so they run in either order
// (below); the inter-chunk decay exp(cum_i) is applied to the accumulators
// once both are done, and then the intra-chunk term runs.  A wavefront's
// loads complete in issue order, so a workgroup that starts with the
// inter-chunk term issues its x loads only after it: issued first, they
// would hold back the h and C loads behind them.
//
// Decay factors.  For a token in 64-token block R > 0 and a key j in an
// earlier block, exp(cum_i - cum_j) = exp(cum_i - cum_r) * exp(cum_r - cum_j)
// with r = 64 R the first token of block R; both factors are <= 1.  The key
// factors exp(cum_r - cum_j) Delta_j are tabulated in LDS once per workgroup
// (one row per block boundary), the row factor is one exponential per lane
// and column tile.  Inside the token's own block the decay is exponentiated
// element by element, with the causal mask selected first.
// ---------------------------------------------------------------------------
// VAR 1 (the decay-precision ablation, ssd_chunk_scan_ablation): every decay
// factor of the output path is rounded to bfloat16 before use.
template <int VAR>
__device__ __forceinline__ float decay_f32(float e) {
  if constexpr (VAR == 1) return (float)(__bf16)e;
  return e;
}

template <int P, int N, int PW, int LMAX, int VAR>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3)))
void k_chunk_out_f32(ScanArgs a) {
  constexpr int PSPLIT = P / PW, TP = PW / 16;
  constexpr int XS = PW + 4;   // = 4 (mod 8): conflict-free x^T-fragment reads
  constexpr int NBLK = LMAX / 64;
  constexpr int RT = NBLK;     // column tiles per wavefront
  __shared__ __attribute__((aligned(16))) float s_d[LMAX];
  __shared__ __attribute__((aligned(16))) float s_cum[LMAX];
  __shared__ float s_wsum[4];
  __shared__ __attribute__((aligned(16))) float s_w[(NBLK - 1) * LMAX];  // key factors
  __shared__ __attribute__((aligned(16))) float s_x[LMAX * XS];

  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t u = xcd_remap(blockIdx.x, gridDim.x);
  const int ps = (int)(u % PSPLIT);
  const int64_t u2 = u / PSPLIT;
  const int64_t h = u2 % a.H, bc = u2 / a.H, c = bc % a.Nc, b = bc / a.Nc;
  const int64_t g = h / (a.H / a.G);
  const int64_t t0 = c * a.L;
  const int Lc = chunk_len(a, c);
  const int nrt = (Lc + 15) / 16;
  const int p0 = ps * PW;
  const float* xg = reinterpret_cast<const float*>(a.x);

  // column tiles of this wavefront (uniform)
  int Ik[RT];
  bool vk[RT];
#pragma unroll
  for (int k = 0; k < RT; ++k) {
    Ik[k] = row_tile_of(wave, k);
    vk[k] = Ik[k] < nrt;
  }

  // x of this workgroup's PW columns for every chunk row, loaded into
  // registers ahead of the staging that writes it to LDS
  constexpr int XQ = PW / 4;
  constexpr int XLB = (LMAX * XQ + kThreads - 1) / kThreads;
  const int nx = nrt * 16 * XQ;
  float4 xv_stage[XLB];
  auto load_x = [&]() {
#pragma unroll
    for (int i = 0; i < XLB; ++i) {
      const int e = i * kThreads + tid, j = e / XQ, m = e % XQ;
      xv_stage[i] = ld4_masked(&xg[((b * a.T + t0 + min(j, Lc - 1)) * a.H + h) * P + p0 + 4 * m],
                               e < nx && j < Lc);
    }
  };

  const float2 dtv = chunk_dt_load(a, b, c, h);

  f32x4 acc[RT][TP];
#pragma unroll
  for (int k = 0; k < RT; ++k)
#pragma unroll
    for (int pt = 0; pt < TP; ++pt) acc[k][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- inter-chunk term: acc[k][pt] = sum_n h_{c-1}[p][n] C[i][n] ----
  auto inter = [&]() {
    const float* Cg = reinterpret_cast<const float*>(a.C) + ((b * a.T + t0) * a.G + g) * N + 4 * q;
    const int64_t crs = a.G * N;
    const float* hp = a.ws_state + ((b * a.H + h) * a.Nc + c) * (int64_t)(P * N) +
                      (int64_t)(p0 + r16) * N + 4 * q;
    auto load_nb = [&](int nb, float4 (&hv)[TP], float4 (&cv)[RT]) {
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) hv[pt] = ld4(hp + pt * 16 * N + nb * 16);
#pragma unroll
      for (int k = 0; k < RT; ++k) {
        const int ri = 16 * Ik[k] + r16;
        cv[k] = ld4_masked(Cg + min(ri, Lc - 1) * crs + nb * 16, vk[k] && ri < Lc);
      }
    };
    auto mma_nb = [&](const float4 (&hv)[TP], const float4 (&cv)[RT]) {
#pragma unroll
      for (int k = 0; k < RT; ++k) {
        if (!vk[k]) continue;
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) {
          acc[k][pt] = mma(hv[pt].x, cv[k].x, acc[k][pt]);
          acc[k][pt] = mma(hv[pt].y, cv[k].y, acc[k][pt]);
          acc[k][pt] = mma(hv[pt].z, cv[k].z, acc[k][pt]);
          acc[k][pt] = mma(hv[pt].w, cv[k].w, acc[k][pt]);
        }
      }
    };
    // Unrolled, so that the same loads are in flight on every path: the
    // compiler then waits for exactly the n-block being consumed (after a
    // conditional load it waits for every load).
    float4 hs[2][TP], cs[2][RT];
    load_nb(0, hs[0], cs[0]);
#pragma unroll
    for (int nb = 0; nb < N / 16; ++nb) {
      if (nb + 1 < N / 16) load_nb(nb + 1, hs[(nb + 1) & 1], cs[(nb + 1) & 1]);
      mma_nb(hs[nb & 1], cs[nb & 1]);
    }
  };

  // ---- prefix sum, x staging, decay tables (ends with a barrier) ----
  auto stage = [&]() {
    const DeltaScan ds = chunk_scan_stage1(a, c, h, dtv, s_wsum);
    __syncthreads();
    chunk_scan_stage2(a, ds, s_wsum, s_d, s_cum);
#pragma unroll
    for (int i = 0; i < XLB; ++i) {
      const int e = i * kThreads + tid, j = e / XQ, m = e % XQ;
      if (e < nx) st4(&s_x[j * XS + 4 * m], xv_stage[i]);
    }
    __syncthreads();
    for (int e = tid; e < (NBLK - 1) * LMAX; e += kThreads) {
      const int R = e / LMAX + 1, j = e % LMAX;
      const int r = min(64 * R, Lc - 1);
      s_w[e] = (j < r) ? decay_f32<VAR>(fast_exp(s_cum[r] - s_cum[j])) * s_d[j] : 0.0f;
    }
    __syncthreads();
  };

  // The workgroups sharing a compute unit start together; alternating the
  // order of the two independent phases lets one workgroup's staging (LDS
  // and vector work, waits) overlap another's inter-chunk term (matrix
  // cores).  Workgroups are dealt to the 256 compute units in rounds of 256
  // (blockIdx % 8 picks the XCD, the rest the unit), so the round's parity
  // is what differs between the workgroups of one unit.
  if ((blockIdx.x >> 8) & 1) {
    load_x();
    stage();
    inter();
  } else {
    inter();
    load_x();
    stage();
  }

  // decay from the chunk start: column i = 16 I + r16 of every accumulator
  float cumk[RT];
#pragma unroll
  for (int k = 0; k < RT; ++k) {
    const int ri = 16 * Ik[k] + r16;
    cumk[k] = s_cum[min(ri, Lc - 1)];
    const float sc = (vk[k] && ri < Lc) ? decay_f32<VAR>(fast_exp(cumk[k])) : 0.0f;
#pragma unroll
    for (int pt = 0; pt < TP; ++pt)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[k][pt][r] *= sc;
  }

  // ---- intra-chunk term: column tile by column tile, one block of 64 keys at a time ----
  const float* S = a.ws_cb + ((b * a.Nc + c) * a.G + g) * a.L * a.L;
  const float* xq = &s_x[4 * q * XS + r16];   // + key * XS + pt * 16
#pragma unroll
  for (int k = 0; k < RT; ++k) {
    if (!vk[k]) continue;                      // uniform
    const int I = Ik[k], R = k;   // row_tile_of deals tile k of a wavefront from block k
    const int ri = 16 * I + r16;
    const float cum_i = cumk[k];
    const float* sr = S + (int64_t)ri * a.L + 4 * q;
    auto load_s = [&](int jb, float4 (&st)[4]) {
#pragma unroll
      for (int t = 0; t < 4; ++t) st[t] = ld4(sr + 64 * jb + 16 * min(t, I - 4 * jb));
    };
    const float u_i = R > 0 ? decay_f32<VAR>(fast_exp(cum_i - s_cum[64 * R])) : 0.0f;
    auto block = [&](int jb, const float4 (&st)[4]) {
      float xv[4][4][TP];   // [key tile][kk][pt]
      if (jb < R) {
        // earlier key block: factored decay u_i * s_w[R-1][j]
        const float* wrow = &s_w[(R - 1) * LMAX + 64 * jb + 4 * q];
        float4 w4[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          w4[t] = ld4(wrow + 16 * t);
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) xv[t][kk][pt] = xq[(64 * jb + 16 * t + kk) * XS + pt * 16];
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float m0 = st[t].x * u_i * w4[t].x, m1 = st[t].y * u_i * w4[t].y;
          const float m2 = st[t].z * u_i * w4[t].z, m3 = st[t].w * u_i * w4[t].w;
#pragma unroll
          for (int pt = 0; pt < TP; ++pt) {
            acc[k][pt] = mma(xv[t][0][pt], m0, acc[k][pt]);
            acc[k][pt] = mma(xv[t][1][pt], m1, acc[k][pt]);
            acc[k][pt] = mma(xv[t][2][pt], m2, acc[k][pt]);
            acc[k][pt] = mma(xv[t][3][pt], m3, acc[k][pt]);
          }
        }
      } else {
        // the column tile's own block, up to the diagonal: masked exponentials
        const int nt = I - 4 * R + 1;           // key tiles up to the diagonal (uniform)
        float4 cj[4], dj[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (t < nt) {
            const int j0 = 64 * jb + 16 * t + 4 * q;
            cj[t] = ld4(&s_cum[j0]);
            dj[t] = ld4(&s_d[j0]);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
              for (int pt = 0; pt < TP; ++pt) xv[t][kk][pt] = xq[(64 * jb + 16 * t + kk) * XS + pt * 16];
          }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (t < nt) {
            const int j0 = 64 * jb + 16 * t + 4 * q;
            const float m0 = (j0 + 0 <= ri) ? st[t].x * decay_f32<VAR>(fast_exp(cum_i - cj[t].x)) * dj[t].x : 0.0f;
            const float m1 = (j0 + 1 <= ri) ? st[t].y * decay_f32<VAR>(fast_exp(cum_i - cj[t].y)) * dj[t].y : 0.0f;
            const float m2 = (j0 + 2 <= ri) ? st[t].z * decay_f32<VAR>(fast_exp(cum_i - cj[t].z)) * dj[t].z : 0.0f;
            const float m3 = (j0 + 3 <= ri) ? st[t].w * decay_f32<VAR>(fast_exp(cum_i - cj[t].w)) * dj[t].w : 0.0f;
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) {
              acc[k][pt] = mma(xv[t][0][pt], m0, acc[k][pt]);
              acc[k][pt] = mma(xv[t][1][pt], m1, acc[k][pt]);
              acc[k][pt] = mma(xv[t][2][pt], m2, acc[k][pt]);
              acc[k][pt] = mma(xv[t][3][pt], m3, acc[k][pt]);
            }
          }
        }
      }
    };
    // Score tiles double-buffered in two register sets.  R is a compile-time
    // constant here, so the loop unrolls and every wait is for exactly the
    // block being consumed; the scheduling barrier keeps the next block's
    // loads ahead of this block's work instead of next to their use.
    float4 sbuf[2][4];
    load_s(0, sbuf[0]);
#pragma unroll
    for (int jb = 0; jb <= R; ++jb) {
      if (jb + 1 <= R) load_s(jb + 1, sbuf[(jb + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      block(jb, sbuf[jb & 1]);
    }
  }

  // ---- skip term and store: lane holds y[i][p..p+3], p = p0 + 16 pt + 4q ----
  const float Dh = a.D ? a.D[h] : 0.0f;
  float* yg = reinterpret_cast<float*>(a.y);
#pragma unroll
  for (int k = 0; k < RT; ++k) {
    if (!vk[k]) continue;
    const int i = 16 * Ik[k] + r16;
    if (i < Lc) {
      float* row = yg + ((b * a.T + t0 + i) * a.H + h) * P + p0;
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) {
        const float4 xv4 = ld4(&s_x[i * XS + 16 * pt + 4 * q]);
        const f32x4 v = acc[k][pt];
        // y is not read again by the scan: stream it past the caches
        __builtin_nontemporal_store(
            f32x4{v[0] + Dh * xv4.x, v[1] + Dh * xv4.y, v[2] + Dh * xv4.z, v[3] + Dh * xv4.w},
            reinterpret_cast<f32x4*>(row + 16 * pt + 4 * q));
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
  // phases 0 and 1 (C B^T, chunk states) in one launch
  if ((e = rec(0)) != hipSuccess) return e;
  if ((e = rec(1)) != hipSuccess) return e;
  const int nrt = (int)((a.L + 15) / 16), ntiles = nrt * (nrt + 1) / 2;
  constexpr int NW = N < 64 ? N : 64;
  const int64_t units1 = a.Bt * a.Nc * a.H * (N / NW);
  hipLaunchKernelGGL((k_cb_and_chunk_state_f32<P, N, NW>), dim3((unsigned)units1),
                     dim3(kThreads), 0, stream, a, ntiles);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // phase 2: inter-chunk recurrence
  if ((e = rec(2)) != hipSuccess) return e;
  if ((e = launch_state_pass(a, P, N, stream, false)) != hipSuccess) return e;
  // phase 3: outputs (skipped when only the entering states are wanted)
  if ((e = rec(3)) != hipSuccess) return e;
  if (a.states_only) return rec(4);
  constexpr int PW = P < 32 ? P : 32;
  const int64_t units3 = a.Bt * a.Nc * a.H * (P / PW);
  if (a.variant != 0) {
    // the decay-precision ablation: the 130M / 2.7B head shape at chunks up to 256 only
    if constexpr (ablation_shape(P, N)) {
      if (a.variant != 1 || a.L > 256) return hipErrorInvalidValue;
      hipLaunchKernelGGL((k_chunk_out_f32<P, N, PW, 256, 1>), dim3((unsigned)units3),
                         dim3(kThreads), 0, stream, a);
    } else {
      return hipErrorInvalidValue;
    }
  } else if (a.L <= 256) {
    hipLaunchKernelGGL((k_chunk_out_f32<P, N, PW, 256, 0>), dim3((unsigned)units3), dim3(kThreads),
                       0, stream, a);
  } else {
    hipLaunchKernelGGL((k_chunk_out_f32<P, N, PW, 512, 0>), dim3((unsigned)units3), dim3(kThreads),
                       0, stream, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return rec(4);
}

template <int P>
hipError_t launch_p(const ScanArgs& a, int N, hipStream_t s, hipEvent_t* ev) {
  switch (N) {
    case 16: return launch_pn<P, 16>(a, s, ev);
    case 32: return launch_pn<P, 32>(a, s, ev);
    case 64: return launch_pn<P, 64>(a, s, ev);
    case 128: return launch_pn<P, 128>(a, s, ev);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace prefill

hipError_t launch_scan_f32(const ScanArgs& a, int P, int N, hipStream_t s, hipEvent_t* ev) {
  switch (P) {
    case 16: return prefill::launch_p<16>(a, N, s, ev);
    case 32: return prefill::launch_p<32>(a, N, s, ev);
    case 64: return prefill::launch_p<64>(a, N, s, ev);
    case 128: return prefill::launch_p<128>(a, N, s, ev);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssd
