// Chunked SSD scan (prefill) for gfx950, bfloat16 x/B/C/y.
//
// Source: "Compiler-First State Space Duality and Portable O(1)
// Autoregressive Caching", Background (Eq. 3, inter-chunk recurrence), SSD
// properties ("diagonal state matrix", "chunked recurrence") and
// Implementation ("static masking"; "precision management": decay kept in
// float32 and exponentiated at compute time, bfloat16 only for the io
// tensors).
//
// Two schedules compute the same numbers, bit for bit:
//
//  * phased: C B^T per chunk, chunk summary states S_c, the inter-chunk
//    recurrence over S_c (state pass), then the outputs, one workgroup per
//    (batch, chunk, head).  Parallel over chunks; the states make three trips
//    through memory.
//  * chain: after a pre-pass (C B^T and a transposed copy of B per chunk,
//    shared by the heads of a group), one workgroup per (batch, head) walks
//    its chunks in order.  The float32 state never leaves the matrix-core
//    accumulators; it reaches LDS only as the bfloat16 operand of the next
//    chunk's inter-chunk term.  Used when batch x heads alone fill the GPU.
//
// Both run the same matrix-core instructions on the same operands in the same
// order for every output and state element, so a row of a batch gets the same
// bits whichever schedule its batch size selects:
//   S_c       = sum over 32-token steps of  (B^T w)_bf16 x        (tile [n][p])
//   h_c       = fma(alpha_c, h_{c-1}, S_c)
//   y^T[p][i] = exp(cum_i) * sum_n bf16(h_{c-1})[p][n] C[i][n]
//               + sum_j x^T[p][j] bf16(S[i][j] decay(i,j) Delta_j)   + D x
// Matrix products run on v_mfma_f32_16x16x32_bf16: lane l holds 8
// consecutive k-slots of row l%16 of A (and of column l%16 of B) in group
// l/16, and the four outputs D[4(l/16)+r][l%16].  Decay, states, C B^T and
// accumulation stay float32; operands are rounded to bfloat16 (round to
// nearest even) right before a matrix instruction.
//
// Contractions over tokens need token-contiguous operands, so x (and B in the
// phased chunk states) is transposed on its way into LDS: every thread loads
// an 8 x 8 block (8 rows of 16 bytes) and writes it back as 8 columns of 16
// bytes.
#include "ssd_prefill_common.h"

namespace ssd {
namespace prefill {
namespace {

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (bf16)0.0f;
  return z;
}

__device__ __forceinline__ bf16x8 ld8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
// Branch-free masked load: `p` must be a valid address whether or not `ok`
// (callers clamp the row); the value is replaced by zeros when !ok.  A plain
// `ok ? load : 0` becomes one exec-masked branch (and a wait) per load.
// The select works on the four packed dwords (a per-element select would
// unpack every bf16 into a register of its own).
__device__ __forceinline__ bf16x8 ld8_masked(const bf16* p, bool ok) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  v.x = ok ? v.x : 0u;
  v.y = ok ? v.y : 0u;
  v.z = ok ? v.z : 0u;
  v.w = ok ? v.w : 0u;
  return __builtin_bit_cast(bf16x8, v);
}

// Pin a loaded fragment in its registers as loaded: work that depends on it
// cannot be moved above this point (keeps a prefetch a prefetch: otherwise
// the compiler may consume the load, and wait for it, right where it is
// issued).
__device__ __forceinline__ void pin(bf16x8& v) {
  uint4 u = __builtin_bit_cast(uint4, v);
  asm volatile("" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w));
  v = __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ void st8(bf16* p, bf16x8 v) { *reinterpret_cast<bf16x8*>(p) = v; }
__device__ __forceinline__ bf16x4 ld4b(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
__device__ __forceinline__ void st4b(bf16* p, bf16x4 v) { *reinterpret_cast<bf16x4*>(p) = v; }

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

// (bf16)(v[e] * w[e]) for 8 slots: the rounding point of B^T w.
__device__ __forceinline__ bf16x8 scale8(bf16x8 v, float4 w0, float4 w1) {
  bf16x8 r;
  r[0] = (bf16)__fmul_rn((float)v[0], w0.x); r[1] = (bf16)__fmul_rn((float)v[1], w0.y);
  r[2] = (bf16)__fmul_rn((float)v[2], w0.z); r[3] = (bf16)__fmul_rn((float)v[3], w0.w);
  r[4] = (bf16)__fmul_rn((float)v[4], w1.x); r[5] = (bf16)__fmul_rn((float)v[5], w1.y);
  r[6] = (bf16)__fmul_rn((float)v[6], w1.z); r[7] = (bf16)__fmul_rn((float)v[7], w1.w);
  return r;
}

// ---------------------------------------------------------------------------
// S = C B^T (float32) for the causal 16x16 tiles of every (b, c, g).
// One wavefront computes tile t of (b, c, g) = bcg: (I, J), J <= I.
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ void cb_tile_bf16(const ScanArgs& a, int64_t bcg, int t) {
  const int lane = threadIdx.x & 63, q = lane >> 4, r16 = lane & 15;
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
    cf[nb] = ld8_masked(Cg + min(ri, Lc - 1) * rs + nb * 32, ri < Lc);
    bf[nb] = ld8_masked(Bg + min(rj, Lc - 1) * rs + nb * 32, rj < Lc);
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nb = 0; nb < N / 32; ++nb) acc = mma(cf[nb], bf[nb], acc);
  float* S = a.ws_cb + bcg * a.L * a.L;
#pragma unroll
  for (int r = 0; r < 4; ++r) S[(int64_t)(16 * I + 4 * q + r) * a.L + 16 * J + r16] = acc[r];
}

// Number of causal 16x16 tiles of one chunk and the C B^T blocks of a grid
// that gives them workgroups of their own (4 tiles per block, rounded up to
// whole rounds of the 8 XCDs).
inline int cb_tiles(const ScanArgs& a) {
  const int nrt = (int)((a.L + 15) / 16);
  return nrt * (nrt + 1) / 2;
}
inline int64_t cb_blocks(const ScanArgs& a) {
  const int64_t items = a.Bt * a.Nc * a.G * cb_tiles(a);
  return ((items + 3) / 4 + 7) / 8 * 8;
}
// Tile work of C B^T block `block` (4 tiles, one per wavefront).
template <int N>
__device__ __forceinline__ void cb_block_bf16(const ScanArgs& a, int ntiles, int64_t block) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t item = block * 4 + wave;
  const int64_t bcg = item / ntiles;
  if (bcg >= a.Bt * a.Nc * a.G) return;
  cb_tile_bf16<N>(a, bcg, (int)(item % ntiles));
}

// ---------------------------------------------------------------------------
// Shared per-chunk pieces.
// ---------------------------------------------------------------------------

// x of one chunk, in 8 x 8 blocks (8 token rows x 8 head columns): block id
// -> token block id / (P/8), column block id % (P/8).  Rows past the chunk's
// end are zeros.  NXB blocks per thread cover LMAX rows.
template <int P, int LMAX>
struct XStage {
  static constexpr int NBLK8 = (LMAX / 8) * (P / 8);
  static constexpr int NXB = (NBLK8 + kThreads - 1) / kThreads;
  bf16x8 v[NXB][8];

  __device__ __forceinline__ void load(const ScanArgs& a, int64_t b, int64_t c, int64_t h) {
    const int tid = threadIdx.x;
    const int64_t t0 = c * a.L;
    const int Lc = chunk_len(a, c);
    const bf16* xg = reinterpret_cast<const bf16*>(a.x) + ((b * a.T + t0) * a.H + h) * P;
    const int64_t xs = a.H * P;
#pragma unroll
    for (int i = 0; i < NXB; ++i) {
      const int id = min(tid + i * kThreads, NBLK8 - 1);
      const int lb = id / (P / 8), cb = id % (P / 8);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int l = 8 * lb + r;
        v[i][r] = ld8_masked(xg + min(l, Lc - 1) * xs + 8 * cb, l < Lc);
      }
    }
  }
  // x^T[p][l] into s_xt (row stride XTS)
  __device__ __forceinline__ void store(bf16* s_xt) {
    constexpr int XTS = LMAX + 8;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NXB; ++i)
#pragma unroll
      for (int r = 0; r < 8; ++r) pin(v[i][r]);
#pragma unroll
    for (int i = 0; i < NXB; ++i) {
      const int id = tid + i * kThreads;
      if (id < NBLK8) {
        const int lb = id / (P / 8), cb = id % (P / 8);
        bf16x8 tr[8];
        transpose8(v[i], tr);
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) st8(s_xt + (8 * cb + cc) * XTS + 8 * lb, tr[cc]);
      }
    }
  }
};

// Factored-decay table: for a query block R >= 1 (queries 64R..) and a key
// j of an earlier block, decay(i, j) Delta_j = u_i * s_w[(R-1)*LMAX + j] with
// u_i = exp(cum_i - cum_r), r = 64R (both factors <= 1 since cum falls).
template <int LMAX>
__device__ __forceinline__ void factored_table(int Lc, const float* s_d, const float* s_cum,
                                               float* s_w) {
  constexpr int NBLK = LMAX / 64;
  for (int e = threadIdx.x; e < (NBLK - 1) * LMAX; e += kThreads) {
    const int R = e / LMAX + 1, j = e % LMAX;
    const int r = min(64 * R, Lc - 1);
    s_w[e] = (j < r) ? __fmul_rn(fast_exp(__fsub_rn(s_cum[r], s_cum[j])), s_d[j]) : 0.0f;
  }
}

// State weights w_l = Delta_l exp(cum_last - cum_l) of the chunk summary state.
template <int LMAX>
__device__ __forceinline__ void state_weights(int Lc, const float* s_d, const float* s_cum,
                                              float* s_ws) {
  const float cum_last = s_cum[Lc - 1];
  for (int l = threadIdx.x; l < LMAX; l += kThreads)
    s_ws[l] = (l < Lc) ? __fmul_rn(s_d[l], fast_exp(__fsub_rn(cum_last, s_cum[l]))) : 0.0f;
}

// Outputs of one chunk, y^T tiles [p][i]: wavefront w owns the 16-token
// column tiles row_tile_of(w, k), k < LMAX/64, and all P/16 head tiles,
// processed KP column tiles per pass.
//   s_h   bf16(h_{c-1})[p][n] (row stride N + 8): the inter-chunk operand
//   s_xt  bf16 x^T[p][j]     (row stride LMAX + 8), zero past the chunk
//   s_d, s_cum, s_w: Delta, cum and the factored-decay table of the chunk
// S (C B^T) and C come from global memory (L2: shared by all heads of a
// group).  A pass's C fragments and the first S block of each of its column
// tiles are loaded ahead (prefetch()), so that their latency hides behind
// other work: the next pass's behind this pass's intra-chunk term, the first
// pass's behind whatever the kernel does between prefetch() and run().
// Every accumulator sees the same instruction sequence whatever KP is.
template <int P, int N, int LMAX, int KP>
struct ChunkOut {
  static constexpr int TP = P / 16;
  static constexpr int RT = LMAX / 64;
  static constexpr int NPASS = RT / KP;
  static constexpr int XTS = LMAX + 8, HS = N + 8;
  static_assert(RT % KP == 0, "passes must cover the column tiles");

  const ScanArgs& a;
  int64_t b, c, h, g;
  int Lc;
  bf16x8 cf[N / 32][KP];   // C[i][32 nb + 8q ..] of the pass's column tiles
  float4 s0[KP][4];        // first 64-key block of S for each column tile

  __device__ __forceinline__ ChunkOut(const ScanArgs& a_, int64_t b_, int64_t c_, int64_t h_,
                                      int64_t g_, int Lc_)
      : a(a_), b(b_), c(c_), h(h_), g(g_), Lc(Lc_) {}

  // Lane index through an opaque copy: inside the chain kernel's chunk loop
  // the many lane-dependent addresses are then formed where they are used
  // instead of being hoisted out of the loop and held in registers.
  __device__ __forceinline__ static int lane_opaque() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t & 63;
  }
  __device__ __forceinline__ static int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  }
  __device__ __forceinline__ int nrt() const { return (Lc + 15) / 16; }

  // S[ri][16t + 4q ..] of 64-key block jb, tile t (tiles past the diagonal
  // tile are never written: the diagonal one is read instead)
  __device__ __forceinline__ void load_s(int I, int jb, float4 (&st)[4]) const {
    const int lane = lane_opaque(), q = lane >> 4, r16 = lane & 15;
    const float* sr = a.ws_cb + ((b * a.Nc + c) * a.G + g) * a.L * a.L +
                      (int64_t)(16 * I + r16) * a.L + 4 * q;
#pragma unroll
    for (int t = 0; t < 4; ++t) st[t] = ld4(sr + 64 * jb + 16 * min(t, I - 4 * jb));
  }

  // C fragments and first S blocks of a pass.  The C rows are loaded with no
  // zeroing select (rows past the chunk read its last row: they only feed
  // output columns that are never stored): with the select the compiler
  // waited for these loads right after issuing them, which left nothing in
  // flight behind the intra-chunk term (chain schedule 1.92 -> 1.85 ms at
  // 8 x 16384).
  __device__ __forceinline__ void prefetch(int pass) {
    const int lane = lane_opaque(), q = lane >> 4, r16 = lane & 15;
    const int wave = wave_id(), n_rt = nrt();
    const bf16* Cg = reinterpret_cast<const bf16*>(a.C) + ((b * a.T + c * a.L) * a.G + g) * N + 8 * q;
    const int64_t crs = a.G * N;
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int I = row_tile_of(wave, pass * KP + k);
      const bool v = I < n_rt;
      const int i = 16 * I + r16;
#pragma unroll
      for (int nb = 0; nb < N / 32; ++nb)
        cf[nb][k] = ld8(Cg + min(i, Lc - 1) * crs + nb * 32);
      load_s(v ? I : n_rt - 1, 0, s0[k]);   // unconditional: exact waits
    }
  }

  // All passes; pass 0 must have been prefetched.
  __device__ __forceinline__ void run(const float* s_d, const float* s_cum, const float* s_w,
                                      const bf16* s_xt, const bf16* s_h) {
    const int lane = lane_opaque(), q = lane >> 4, r16 = lane & 15;
    const int wave = wave_id(), n_rt = nrt();
    const int64_t t0 = c * a.L;
    const float Dh = a.D ? a.D[h] : 0.0f;
    bf16* yg = reinterpret_cast<bf16*>(a.y);

#pragma unroll 1
    for (int pass = 0; pass < NPASS; ++pass) {
      int Ik[KP];
      bool vk[KP];
#pragma unroll
      for (int k = 0; k < KP; ++k) {
        Ik[k] = row_tile_of(wave, pass * KP + k);
        vk[k] = Ik[k] < n_rt;
      }
      // later passes hold later (snake-ordered) tiles only when this one does
      if (!vk[0]) break;
      const bool more = pass + 1 < NPASS && row_tile_of(wave, (pass + 1) * KP) < n_rt;
      f32x4 acc[KP][TP];
#pragma unroll
      for (int k = 0; k < KP; ++k)
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) acc[k][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

      // ---- inter-chunk term: acc[k] = exp(cum_i) * sum_n h_{c-1}[p][n] C[i][n] ----
#pragma unroll
      for (int nb = 0; nb < N / 32; ++nb) {
        bf16x8 hf[TP];
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) hf[pt] = ld8(s_h + (16 * pt + r16) * HS + 32 * nb + 8 * q);
#pragma unroll
        for (int k = 0; k < KP; ++k) {
          if (!vk[k]) continue;
#pragma unroll
          for (int pt = 0; pt < TP; ++pt) acc[k][pt] = mma(hf[pt], cf[nb][k], acc[k][pt]);
        }
      }
      // decay from the chunk start: column i = 16 I + r16 of every accumulator
#pragma unroll
      for (int k = 0; k < KP; ++k) {
        if (!vk[k]) continue;
        const int i = 16 * Ik[k] + r16;
        const float sc = i < Lc ? fast_exp(s_cum[i]) : 0.0f;
#pragma unroll
        for (int pt = 0; pt < TP; ++pt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[k][pt][r] = __fmul_rn(acc[k][pt][r], sc);
      }

      // ---- intra-chunk term: column tile by column tile, 64 keys (two 32-key slots) at a time ----
#pragma unroll
      for (int k = 0; k < KP; ++k) {
        if (!vk[k]) continue;
        const int I = Ik[k], R = I >> 2;
        const int ri = 16 * I + r16;
        const float cum_i = s_cum[min(ri, Lc - 1)];
        const float u_i = R > 0 ? fast_exp(__fsub_rn(cum_i, s_cum[64 * R])) : 0.0f;
        auto block = [&](int jb, const float4 (&st)[4]) {
          // k-slots of a 32-key half (key tiles 2s, 2s+1): slot e < 4 -> key
          // 16(2s) + 4q + e, slot e >= 4 -> key 16(2s+1) + 4q + e - 4
          const bf16* xq = s_xt + (int64_t)r16 * XTS + 64 * jb + 4 * q;
          if (jb < R) {
            const float* wrow = &s_w[(R - 1) * LMAX + 64 * jb + 4 * q];
#pragma unroll
            for (int sh = 0; sh < 2; ++sh) {
              const float4 w0 = ld4(wrow + 32 * sh), w1 = ld4(wrow + 32 * sh + 16);
              const float4 t0v = st[2 * sh], t1v = st[2 * sh + 1];
              bf16x8 m;
              m[0] = (bf16)__fmul_rn(__fmul_rn(t0v.x, u_i), w0.x);
              m[1] = (bf16)__fmul_rn(__fmul_rn(t0v.y, u_i), w0.y);
              m[2] = (bf16)__fmul_rn(__fmul_rn(t0v.z, u_i), w0.z);
              m[3] = (bf16)__fmul_rn(__fmul_rn(t0v.w, u_i), w0.w);
              m[4] = (bf16)__fmul_rn(__fmul_rn(t1v.x, u_i), w1.x);
              m[5] = (bf16)__fmul_rn(__fmul_rn(t1v.y, u_i), w1.y);
              m[6] = (bf16)__fmul_rn(__fmul_rn(t1v.z, u_i), w1.z);
              m[7] = (bf16)__fmul_rn(__fmul_rn(t1v.w, u_i), w1.w);
#pragma unroll
              for (int pt = 0; pt < TP; ++pt) {
                const bf16* xr = xq + pt * 16 * XTS + 32 * sh;
                acc[k][pt] = mma(cat(ld4b(xr), ld4b(xr + 16)), m, acc[k][pt]);
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
                const float4 t0v = st[2 * sh], t1v = st[2 * sh + 1];
                const bool hi = 2 * sh + 1 < nt;
                auto dec = [&](bool on, float sv, float cj, float dj) {
                  return on ? __fmul_rn(__fmul_rn(sv, fast_exp(__fsub_rn(cum_i, cj))), dj) : 0.0f;
                };
                bf16x8 m;
                m[0] = (bf16)dec(j0 + 0 <= ri, t0v.x, c0.x, d0.x);
                m[1] = (bf16)dec(j0 + 1 <= ri, t0v.y, c0.y, d0.y);
                m[2] = (bf16)dec(j0 + 2 <= ri, t0v.z, c0.z, d0.z);
                m[3] = (bf16)dec(j0 + 3 <= ri, t0v.w, c0.w, d0.w);
                m[4] = (bf16)dec(hi && j0 + 16 <= ri, t1v.x, c1.x, d1.x);
                m[5] = (bf16)dec(hi && j0 + 17 <= ri, t1v.y, c1.y, d1.y);
                m[6] = (bf16)dec(hi && j0 + 18 <= ri, t1v.z, c1.z, d1.z);
                m[7] = (bf16)dec(hi && j0 + 19 <= ri, t1v.w, c1.w, d1.w);
                // the upper key tile may lie past the staged rows of a ragged
                // chunk's x^T: never read it then
                bf16x4 z4;
#pragma unroll
                for (int e = 0; e < 4; ++e) z4[e] = (bf16)0.0f;
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) {
                  const bf16* xr = xq + pt * 16 * XTS + 32 * sh;
                  acc[k][pt] = mma(cat(ld4b(xr), hi ? ld4b(xr + 16) : z4), m, acc[k][pt]);
                }
              }
            }
          }
        };
        float4 sa[4], sb[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) sa[t] = s0[k][t];
        // the C fragments are dead now: the next pass's are loaded behind this intra term
        if (k == 0 && more) {
          const bf16* Cg = reinterpret_cast<const bf16*>(a.C) + ((b * a.T + t0) * a.G + g) * N + 8 * q;
          const int64_t crs = a.G * N;
#pragma unroll
          for (int kk = 0; kk < KP; ++kk) {
            const int In = row_tile_of(wave, (pass + 1) * KP + kk);
            const int i = 16 * In + r16;
#pragma unroll
            for (int nb = 0; nb < N / 32; ++nb)
              cf[nb][kk] = ld8(Cg + min(i, Lc - 1) * crs + nb * 32);   // see prefetch
          }
        }
        for (int jb = 0; jb <= R; jb += 2) {
          if (jb + 1 <= R) load_s(I, jb + 1, sb);
          block(jb, sa);
          if (jb + 1 > R) break;
          if (jb + 2 <= R) load_s(I, jb + 2, sa);
          block(jb + 1, sb);
        }
        // this column tile's first S block is consumed: load the next pass's
        if (more) {
          const int In = row_tile_of(wave, (pass + 1) * KP + k);
          if (In < n_rt) load_s(In, 0, s0[k]);
        }
      }

      // ---- skip term and store: lane holds y[i][p..p+3], p = 16 pt + 4q ----
#pragma unroll
      for (int k = 0; k < KP; ++k) {
        if (!vk[k]) continue;
        const int i = 16 * Ik[k] + r16;
        if (i < Lc) {
          bf16* row = yg + ((b * a.T + t0 + i) * a.H + h) * P;
#pragma unroll
          for (int pt = 0; pt < TP; ++pt) {
            const int p0 = 16 * pt + 4 * q;
            bf16x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r)
              o[r] = (bf16)__fmaf_rn(Dh, (float)s_xt[(p0 + r) * XTS + i], acc[k][pt][r]);
            st4b(row + p0, o);
          }
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Phased schedule, phase 1: chunk summary states S_c = sum_l B_l^T w_l x_l,
// tile [n][p] (stored to the workspace as [p][n]), w_l = Delta_l exp(cum_last
// - cum_l).  Tokens are staged 64 at a time, transposed (token-contiguous
// rows), double-buffered in LDS; B^T is scaled by w_l as it is staged.
// ---------------------------------------------------------------------------
template <int P, int N>
struct ChunkStateShapeB {
  static constexpr int KB = 64;
  static constexpr int TS = KB;       // LDS row (elements) of the transposed blocks: 128 bytes
  // 16-byte unit u (8 tokens) of row r lives at unit u ^ key(r), key(r) =
  // (r ^ (r >> 3)) & 7.  The transposing stores vary r in steps of 8 across
  // lanes and the fragment reads vary r by 1: the key differs across any 8
  // such lanes, so each group of 8 lanes covers 32 distinct banks either way.
  // A padded stride of 72 elements put the stores' 8 lanes in one bank group;
  // the swizzle took the 2.7B-shaped chunk-state kernel from 52 to 47 us.
  static_assert(KB == 64, "8 units per row");
  __device__ __forceinline__ static int at(int r, int u) {
    return r * TS + 8 * (u ^ ((r ^ (r >> 3)) & 7));
  }
};

template <int P, int N>
__device__ __forceinline__ void chunk_state_bf16(const ScanArgs& a, int ntiles, int64_t block,
                                                 int64_t nblocks,
                                                 float* s_d, float* s_cum, float* s_w,
                                                 float* s_wsum, bf16* s_x0, bf16* s_x1,
                                                 bf16* s_b0, bf16* s_b1) {
  using Sh = ChunkStateShapeB<P, N>;
  constexpr int KB = Sh::KB;
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

  // this thread's 8x8 blocks: id < XBLK -> x block, else B block.  Rows past
  // the chunk read its last row unmasked: B is scaled by w_l = 0 there, so
  // those finite rows add nothing.  (A zeroing select let the compiler wait
  // for the whole block right after issuing it, before the prologue: 42 ->
  // 37 us on the 2.7B shape.)
  auto load_block = [&](int kb0, bf16x8 (&v)[NB8][8]) {
#pragma unroll
    for (int i = 0; i < NB8; ++i) {
      const int id = tid + i * kThreads;
      if (id < XBLK) {
        const int lb = id / (P / 8), cb = id % (P / 8);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int l = kb0 + 8 * lb + r;
          v[i][r] = ld8(xg + min(l, Lc - 1) * xstride + 8 * cb);
        }
      } else if (id < XBLK + BBLK) {
        const int id2 = id - XBLK, lb = id2 / (N / 8), cb = id2 % (N / 8);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int l = kb0 + 8 * lb + r;
          v[i][r] = ld8(Bg + min(l, Lc - 1) * bstride + 8 * cb);
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
        transpose8(v[i], tr);
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) st8(sx + Sh::at(8 * cb + cc, lb), tr[cc]);
      } else if (id < XBLK + BBLK) {
        const int id2 = id - XBLK, lb = id2 / (N / 8), cb = id2 % (N / 8);
        bf16x8 in[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float w = s_w[kb0 + 8 * lb + r];
#pragma unroll
          for (int e = 0; e < 8; ++e) in[r][e] = (bf16)__fmul_rn((float)v[i][r][e], w);
        }
        transpose8(in, tr);
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) st8(sb + Sh::at(8 * cb + cc, lb), tr[cc]);
      }
    }
  };
  bf16x8 vA[NB8][8];
  load_block(0, vA);   // in flight during the prologue

  chunk_delta_cumsum(a, b, c, h, s_d, s_cum, s_wsum);
  state_weights<kMaxL>(Lc, s_d, s_cum, s_w);
  if (tid == 0) a.ws_alpha[(b * a.H + h) * a.Nc + c] = fast_exp(s_cum[Lc - 1]);
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
      for (int ip = 0; ip < NPT; ++ip) av[ip] = ld8(sx + Sh::at((pt0 + ip) * 16 + r16, ks / 8 + q));
#pragma unroll
      for (int in = 0; in < NNT; ++in) bv[in] = ld8(sb + Sh::at((nt0 + in) * 16 + r16, ks / 8 + q));
#pragma unroll
      for (int ip = 0; ip < NPT; ++ip)
#pragma unroll
        for (int in = 0; in < NNT; ++in) acc[ip][in] = mma(bv[in], av[ip], acc[ip][in]);
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
    // lane holds S[n = 16 nt + 4q + r][p = 16 pt + r16]: 4 consecutive n of one p
    float* out = a.ws_state + ((b * a.H + h) * a.Nc + c) * (int64_t)(P * N);
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
    const int wi = (int)(h % hpg);
    const int64_t bcg = (b * a.Nc + c) * a.G + g;
    for (int t = wi * 4 + wave; t < ntiles; t += hpg * 4) cb_tile_bf16<N>(a, bcg, t);
  }
}

// Every chunk-state workgroup also computes its share of the C B^T tiles of
// its (b, c, g) once its state is stored.
template <int P, int N>
__global__ __launch_bounds__(kThreads) void k_cb_and_chunk_state_bf16(ScanArgs a, int ntiles) {
  using Sh = ChunkStateShapeB<P, N>;
  __shared__ float s_d[kMaxL], s_cum[kMaxL], s_w[kMaxL], s_wsum[4];
  __shared__ __attribute__((aligned(16))) bf16 s_x[2][P * Sh::TS];
  __shared__ __attribute__((aligned(16))) bf16 s_b[2][N * Sh::TS];
  chunk_state_bf16<P, N>(a, ntiles, blockIdx.x, gridDim.x, s_d, s_cum, s_w, s_wsum, s_x[0],
                         s_x[1], s_b[0], s_b[1]);
}

// ---------------------------------------------------------------------------
// Phased schedule, phase 3: chunk outputs, one workgroup per (b, c, h).  The
// entering state h_{c-1} (rounded to bf16 by the state pass) is copied to
// LDS, x is staged transposed, then the shared ChunkOut runs.
// ---------------------------------------------------------------------------
constexpr int kOutPass = 2;     // column tiles per output pass, phased schedule
constexpr int kChainPass = 1;   // and chain schedule (which holds more besides)

template <int P, int N, int LMAX>
__global__ __launch_bounds__(kThreads) void k_chunk_out_bf16(ScanArgs a) {
  constexpr int NBLK = LMAX / 64;
  constexpr int XTS = LMAX + 8, HS = N + 8;
  __shared__ __attribute__((aligned(16))) float s_d[LMAX];
  __shared__ __attribute__((aligned(16))) float s_cum[LMAX];
  __shared__ float s_wsum[4];
  __shared__ __attribute__((aligned(16))) float s_w[(NBLK - 1) * LMAX + 4];
  __shared__ __attribute__((aligned(16))) bf16 s_xt[P * XTS];
  __shared__ __attribute__((aligned(16))) bf16 s_h[P * HS];

  const int tid = threadIdx.x;
  const int64_t u = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t h = u % a.H, bc = u / a.H, c = bc % a.Nc, b = bc / a.Nc;
  const int64_t g = h / (a.H / a.G);
  const int Lc = chunk_len(a, c);

  // every global load of the staging is issued before the first barrier
  XStage<P, LMAX> xs;
  xs.load(a, b, c, h);
  constexpr int HV = P * N / 8;                 // 8-element groups of the state
  constexpr int NHV = (HV + kThreads - 1) / kThreads;
  const bf16* hp = reinterpret_cast<const bf16*>(a.ws_hb) +
                   ((b * a.H + h) * a.Nc + c) * (int64_t)(P * N);
  bf16x8 hv[NHV];
#pragma unroll
  for (int i = 0; i < NHV; ++i) hv[i] = ld8(hp + min(tid + i * kThreads, HV - 1) * 8);
  ChunkOut<P, N, LMAX, kOutPass> out(a, b, c, h, g, Lc);
  out.prefetch(0);
  chunk_delta_cumsum(a, b, c, h, s_d, s_cum, s_wsum);  // ends with a barrier
  factored_table<LMAX>(Lc, s_d, s_cum, s_w);
  xs.store(s_xt);
#pragma unroll
  for (int i = 0; i < NHV; ++i) {
    const int e = tid + i * kThreads;
    if (e < HV) st8(s_h + ((e * 8) / N) * HS + (e * 8) % N, hv[i]);
  }
  __syncthreads();
  out.run(s_d, s_cum, s_w, s_xt, s_h);
}

// ---------------------------------------------------------------------------
// Chain schedule.
// Pre-pass: C B^T tiles (first ncb blocks) and the transposed copy of B:
// ws_bt[(b, c, g)][n][l] = B[b, cL + l, g, n], zero past the chunk's end.
// One thread per 8 x 8 block (8 tokens x 8 state columns); consecutive
// threads take consecutive token blocks, so a row of ws_bt is written by
// consecutive threads.
// ---------------------------------------------------------------------------
template <int N>
__global__ __launch_bounds__(kThreads) void k_cb_and_bt_bf16(ScanArgs a, int ntiles, int64_t ncb) {
  if ((int64_t)blockIdx.x < ncb) {
    cb_block_bf16<N>(a, ntiles, blockIdx.x);
    return;
  }
  const int LB = (int)(a.L / 8);
  const int64_t per = (int64_t)LB * (N / 8);
  const int64_t id = ((int64_t)blockIdx.x - ncb) * kThreads + threadIdx.x;
  const int64_t unit = id / per;
  if (unit >= a.Bt * a.Nc * a.G) return;
  const int e = (int)(id % per);
  const int lb = e % LB, nb = e / LB;
  const int64_t g = unit % a.G, bc = unit / a.G, c = bc % a.Nc, b = bc / a.Nc;
  const int Lc = chunk_len(a, c);
  const bf16* Bg = reinterpret_cast<const bf16*>(a.B) + ((b * a.T + c * a.L) * a.G + g) * N + 8 * nb;
  const int64_t rs = a.G * N;
  bf16x8 in[8], tr[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int l = 8 * lb + r;
    in[r] = ld8_masked(Bg + min(l, Lc - 1) * rs, l < Lc);
  }
  transpose8(in, tr);
  bf16* dst = reinterpret_cast<bf16*>(a.ws_bt) + unit * N * a.L + (int64_t)(8 * nb) * a.L + 8 * lb;
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) st8(dst + cc * a.L, tr[cc]);
}

// Chain kernel: one workgroup per (b, h), chunks in order.  Wavefront w keeps
// the float32 state tiles [n][p] of n-tiles NTW*w .. NTW*w + NTW-1 (all p) in
// matrix-core accumulators for the whole sequence; LDS holds only bf16(h) as
// the inter-chunk operand.  Per chunk c:
//   stage:   Delta/cum, x^T and bf16(h_{c-1}) into LDS, decay tables
//   outputs: ChunkOut (inter-chunk term from the LDS copy)
//   state:   S_c = sum_ks (B^T w)_bf16 x into a fresh accumulator, then
//            h_c = fma(alpha_c, h_{c-1}, S_c)
// Load order (memory counters retire loads in order, so a wait for a load
// also waits for every older one): the state step's B^T fragments first,
// then the next chunk's x and dt (consumed after the next barrier); the next
// chunk's first output-pass operands right after that barrier, so they fly
// during the staging.
template <int P, int N, int LMAX>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void k_chain_bf16(ScanArgs a) {
  constexpr int TP = P / 16, TN = N / 16, NTW = TN / 4;
  constexpr int NBLK = LMAX / 64, NKS = LMAX / 32;
  constexpr int XTS = LMAX + 8, HS = N + 8;
  static_assert(TN % 4 == 0, "N must give every wavefront whole n-tiles");
  using Out = ChunkOut<P, N, LMAX, kChainPass>;
  __shared__ __attribute__((aligned(16))) float s_d[LMAX];
  __shared__ __attribute__((aligned(16))) float s_cum[LMAX];
  __shared__ __attribute__((aligned(16))) float s_ws[LMAX];
  __shared__ float s_wsum[4];
  __shared__ __attribute__((aligned(16))) float s_w[(NBLK - 1) * LMAX + 4];
  __shared__ __attribute__((aligned(16))) bf16 s_xt[P * XTS];
  __shared__ __attribute__((aligned(16))) bf16 s_h[P * HS];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t u = xcd_remap(blockIdx.x, gridDim.x);   // heads of a batch row share an XCD
  const int64_t h = u % a.H, b = u / a.H;
  const int64_t g = h / (a.H / a.G);
  const int64_t sbase = (b * a.H + h) * (int64_t)(P * N);

  Out out(a, b, 0, h, g, chunk_len(a, 0));
  XStage<P, LMAX> xs;
  xs.load(a, b, 0, h);
  float2 dtv = chunk_dt_load(a, b, 0, h);
  out.prefetch(0);

  // state tiles: acc_h[in][pt] holds h[p = 16 pt + r16][n = 16 (NTW w + in) + 4q + r]
  f32x4 acc_h[NTW][TP];
  {
    const int lane = Out::lane_opaque(), q = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int in = 0; in < NTW; ++in)
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) {
        if (a.h0) {
          const float4 v =
              ld4(a.h0 + sbase + (16 * pt + r16) * N + 16 * (NTW * wave + in) + 4 * q);
          acc_h[in][pt] = f32x4{v.x, v.y, v.z, v.w};
        } else {
          acc_h[in][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
  }

  for (int64_t c = 0; c < a.Nc; ++c) {
    const int Lc = chunk_len(a, c);
    // ---- stage chunk c ----
    const DeltaScan ds = chunk_scan_stage1(a, c, h, dtv, s_wsum);
    __syncthreads();   // every wavefront is done with chunk c-1's LDS; s_wsum published
    if (c > 0) {
      // first output pass of this chunk: younger than x, which the staging
      // below waits for anyway, and in flight during the staging
      out.c = c;
      out.Lc = Lc;
      out.prefetch(0);
    }
    chunk_scan_stage2(a, ds, s_wsum, s_d, s_cum);
    xs.store(s_xt);
    {
      const int lane = Out::lane_opaque(), q = lane >> 4, r16 = lane & 15;
#pragma unroll
      for (int in = 0; in < NTW; ++in)
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) {
          bf16x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = (bf16)acc_h[in][pt][r];
          st4b(s_h + (16 * pt + r16) * HS + 16 * (NTW * wave + in) + 4 * q, v);
        }
    }
    __syncthreads();
    factored_table<LMAX>(Lc, s_d, s_cum, s_w);
    state_weights<LMAX>(Lc, s_d, s_cum, s_ws);
    const float alpha = fast_exp(s_cum[Lc - 1]);
    __syncthreads();

    // ---- outputs of chunk c ----
    out.run(s_d, s_cum, s_w, s_xt, s_h);

    // ---- chunk summary state S_c, then h_c = fma(alpha, h_{c-1}, S_c) ----
    // steps st = (ks, in): one x^T fragment per (ks, pt) serves every n-tile
    // of the wavefront.  B^T fragments stream through a ring of RING register
    // sets, RING steps ahead; the next chunk's x and dt are issued once the
    // last fragment load is out.
    {
      const int nks = (Lc + 31) / 32;
      const int lane = Out::lane_opaque(), q = lane >> 4, r16 = lane & 15;
      const bf16* btc = reinterpret_cast<const bf16*>(a.ws_bt) +
                        ((b * a.Nc + c) * a.G + g) * (int64_t)(N * a.L) + 8 * q;
      constexpr int NSTEP = NKS * NTW, RING = 4;
      bf16x8 ring[RING];
      auto issue = [&](int st) {
        const int ks = st / NTW, in = st % NTW;
        if (ks < nks)
          ring[st % RING] = ld8(btc + (int64_t)(16 * (NTW * wave + in) + r16) * a.L + 32 * ks);
      };
      f32x4 t[NTW][TP];
#pragma unroll
      for (int in = 0; in < NTW; ++in)
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) t[in][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < RING && st < NSTEP; ++st) issue(st);
      bf16x8 xf[TP];
#pragma unroll
      for (int st = 0; st < NSTEP; ++st) {
        const int ks = st / NTW, in = st % NTW;
        const bf16x8 frag = ring[st % RING];
        if (st + RING < NSTEP) issue(st + RING);
        if (st + RING == NSTEP - 1 || (st == 0 && NSTEP <= RING)) {
          if (c + 1 < a.Nc) {
            xs.load(a, b, c + 1, h);
            dtv = chunk_dt_load(a, b, c + 1, h);
          }
        }
        if (ks < nks) {
          const int l0 = 32 * ks + 8 * q;
          if (in == 0) {
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) xf[pt] = ld8(s_xt + (16 * pt + r16) * XTS + l0);
          }
          const bf16x8 bw = scale8(frag, ld4(&s_ws[l0]), ld4(&s_ws[l0 + 4]));
#pragma unroll
          for (int pt = 0; pt < TP; ++pt) t[in][pt] = mma(bw, xf[pt], t[in][pt]);
        }
      }
#pragma unroll
      for (int in = 0; in < NTW; ++in)
#pragma unroll
        for (int pt = 0; pt < TP; ++pt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc_h[in][pt][r] = __fmaf_rn(alpha, acc_h[in][pt][r], t[in][pt][r]);
    }
  }

  if (a.final_state) {
    const int lane = Out::lane_opaque(), q = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int in = 0; in < NTW; ++in)
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) {
        const f32x4 v = acc_h[in][pt];
        st4(a.final_state + sbase + (16 * pt + r16) * N + 16 * (NTW * wave + in) + 4 * q,
            make_float4(v[0], v[1], v[2], v[3]));
      }
  }
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------
template <int P, int N>
hipError_t launch_phased(const ScanArgs& a, hipStream_t stream, hipEvent_t* ev) {
  hipError_t e;
  auto rec = [&](int k) -> hipError_t { return ev ? hipEventRecord(ev[k], stream) : hipSuccess; };
  if ((e = rec(0)) != hipSuccess) return e;
  if ((e = rec(1)) != hipSuccess) return e;
  const int64_t units = a.Bt * a.Nc * a.H;
  hipLaunchKernelGGL((k_cb_and_chunk_state_bf16<P, N>), dim3((unsigned)units), dim3(kThreads), 0,
                     stream, a, cb_tiles(a));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = rec(2)) != hipSuccess) return e;
  if ((e = launch_state_pass(a, P, N, stream, true)) != hipSuccess) return e;
  if ((e = rec(3)) != hipSuccess) return e;
  if (a.states_only) return rec(4);   // entering states and C B^T only
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

template <int P, int N>
hipError_t launch_chain(const ScanArgs& a, hipStream_t stream, hipEvent_t* ev) {
  if constexpr (chain_variant(P, N)) {
    hipError_t e;
    auto rec = [&](int k) -> hipError_t { return ev ? hipEventRecord(ev[k], stream) : hipSuccess; };
    if ((e = rec(0)) != hipSuccess) return e;
    const int64_t ncb = cb_blocks(a);
    const int64_t nbt = (a.Bt * a.Nc * a.G * (a.L / 8) * (N / 8) + kThreads - 1) / kThreads;
    hipLaunchKernelGGL((k_cb_and_bt_bf16<N>), dim3((unsigned)(ncb + nbt)), dim3(kThreads), 0,
                       stream, a, cb_tiles(a), ncb);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = rec(1)) != hipSuccess) return e;
    if ((e = rec(2)) != hipSuccess) return e;
    if ((e = rec(3)) != hipSuccess) return e;
    const unsigned chains = (unsigned)(a.Bt * a.H);
    if (a.L <= 128) {
      hipLaunchKernelGGL((k_chain_bf16<P, N, 128>), dim3(chains), dim3(kThreads), 0, stream, a);
    } else {
      hipLaunchKernelGGL((k_chain_bf16<P, N, 256>), dim3(chains), dim3(kThreads), 0, stream, a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return rec(4);
  } else {
    return hipErrorInvalidValue;
  }
}

template <int P, int N>
hipError_t launch_pn(const ScanArgs& a, hipStream_t stream, hipEvent_t* ev) {
  return a.chain ? launch_chain<P, N>(a, stream, ev) : launch_phased<P, N>(a, stream, ev);
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
