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
#include <type_traits>

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

// x of a chunk sits in LDS row-major, x[token][p] with row stride P + 16, and
// the matrix-core operands that contract over tokens (x^T rows p, k = token)
// are read with the transposing LDS read ds_read_b64_tr_b16: within each
// group of 16 lanes, lane j addresses 4 elements and receives element j % 4
// of the vectors addressed by lanes j / 4, 4 + j / 4, 8 + j / 4, 12 + j / 4
// (checked on gfx950 with an in-bounds probe of every lane).  So when lane j
// of group q addresses x[t + j / 4][p0 + 4 (j % 4)], it receives
// x[t .. t+3][p0 + j]: the operand layout of lane (row p0 + j, k-slots of
// group q).
constexpr int x_row_stride(int P) { return P + 16; }
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<bf16*>(p)));
  return __builtin_bit_cast(bf16x4, v);
}
// The lane's part of a transposed read: x[j / 4 + QM q][4 (j % 4)] for lane j
// of 16-lane group q, whose first token is QM q past the fragment's.  Reads
// then add only the fragment's uniform token and column offsets (immediate
// offsets where those are compile-time constants).
template <int P, int QM>
__device__ __forceinline__ const bf16* xt_lane(const bf16* s_x, int lane) {
  const int j = lane & 15, q = lane >> 4;
  return s_x + ((j >> 2) + QM * q) * x_row_stride(P) + 4 * (j & 3);
}
// x^T[p0 + j][t + QM q .. + 3] for lane j of group q (base from xt_lane)
template <int P>
__device__ __forceinline__ bf16x4 xt_at4(const bf16* base, int t, int p0) {
  return lds_read_tr4(base + t * x_row_stride(P) + p0);
}
// x^T[p0 + j][t + QM q .. + 7] (the 8 k-slots of a 32-deep operand)
template <int P>
__device__ __forceinline__ bf16x8 xt_at8(const bf16* base, int t, int p0) {
  const bf16x4 lo = xt_at4<P>(base, t, p0), hi = xt_at4<P>(base, t + 4, p0);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
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
// S = C B^T for the causal 16x16 tiles of every (b, c, g), float32
// accumulation.  The forward scan keeps S in bfloat16 (a.cb_bf16): it is only
// ever a matrix-core operand after its decay factor is applied, and half the
// bytes halve the rows each column tile streams; the gradients' recompute of
// the forward states keeps float32 (their own products read it).
// One wavefront computes tile t of (b, c, g) = bcg: (I, J), J <= I, as
// S^T = B_J C_I^T, so that a lane holds 4 consecutive keys of one query row.
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
  for (int nb = 0; nb < N / 32; ++nb) acc = mma(bf[nb], cf[nb], acc);
  // lane holds S[16I + r16][16J + 4q + r], r = 0..3
  const int64_t at = bcg * a.L * a.L + (int64_t)(16 * I + r16) * a.L + 16 * J + 4 * q;
  if (a.cb_bf16) {
    bf16x4 v;
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = (bf16)acc[r];
    st4b(reinterpret_cast<bf16*>(a.ws_cb) + at, v);
  } else {
    st4(a.ws_cb + at, make_float4(acc[0], acc[1], acc[2], acc[3]));
  }
}

// Number of causal 16x16 tiles of one chunk.
inline int cb_tiles(const ScanArgs& a) {
  const int nrt = (int)((a.L + 15) / 16);
  return nrt * (nrt + 1) / 2;
}

// ---------------------------------------------------------------------------
// Shared per-chunk pieces.
// ---------------------------------------------------------------------------

// x of one chunk, in blocks of 8 token rows x CW head columns (CW = 8, or 4
// when the workgroup has threads enough for the smaller blocks): block id ->
// token block id / (P/CW), column block id % (P/CW).  NXB blocks per thread
// cover LMAX rows.  Rows past the chunk's end repeat its last row (finite
// values: they meet only zero scores and zero state weights).
template <int P, int LMAX, int NTH = kThreads>
struct XStage {
  static constexpr int CW = (LMAX / 8) * (P / 8) >= NTH ? 8 : 4;
  static constexpr int NCB = P / CW;
  static constexpr int NBLK = (LMAX / 8) * NCB;
  static constexpr int NXB = (NBLK + NTH - 1) / NTH;
  typedef __bf16 vrow __attribute__((ext_vector_type(CW)));
  vrow v[NXB][8];
  int Lc = 0;

  // block id -> (token block, column block), column blocks fastest: the
  // lanes of a token block load and store whole rows
  __device__ __forceinline__ static void block_of(int id, int& lb, int& cb) {
    cb = id % NCB;
    lb = id / NCB;
  }

  __device__ __forceinline__ void load(const ScanArgs& a, int64_t b, int64_t c, int64_t h) {
    const int tid = opaque_tid();
    const int64_t t0 = c * a.L;
    Lc = chunk_len(a, c);
    const bf16* xg = reinterpret_cast<const bf16*>(a.x) + ((b * a.T + t0) * a.H + h) * P;
    const uint32_t xs = (uint32_t)(a.H * P);
#pragma unroll
    for (int i = 0; i < NXB; ++i) {
      int lb, cb;
      block_of(min(tid + i * NTH, NBLK - 1), lb, cb);
#pragma unroll
      for (int r = 0; r < 8; ++r)
        v[i][r] = *reinterpret_cast<const vrow*>(
            off32(xg, (uint32_t)min(8 * lb + r, Lc - 1) * xs + CW * cb));
    }
  }
  // x[l][p] into s_x (row stride x_row_stride(P))
  __device__ __forceinline__ void store(bf16* s_x) {
    constexpr int XRS = x_row_stride(P);
    const int tid = opaque_tid();
#pragma unroll
    for (int i = 0; i < NXB; ++i) {
      const int id = tid + i * NTH;
      if (id < NBLK) {
        int lb, cb;
        block_of(id, lb, cb);
#pragma unroll
        for (int r = 0; r < 8; ++r) *reinterpret_cast<vrow*>(s_x + (8 * lb + r) * XRS + CW * cb) = v[i][r];
      }
    }
  }
};

// Variants of the output path, chosen at compile time:
//   kDecayF32    decay factors in float32 (the library's path)
//   kDecayBf16   every decay factor of the output path rounded to bfloat16
//                before use (the decay-precision ablation)
//   kMaskLoaded  the causal mask of the diagonal tiles read from a stored
//                lower-triangular bit table instead of formed from an index
//                comparison (the mask-placement ablation; same bits)
enum : int { kDecayF32 = 0, kDecayBf16 = 1, kMaskLoaded = 2 };

template <int VAR>
__device__ __forceinline__ float decay_factor(float e) {
  if constexpr (VAR == kDecayBf16) return (float)(bf16)e;
  return e;
}

// Lower-triangular mask of a kMaxL x kMaxL chunk as bits: bit b of word
// [i][wd] is set iff key 32 wd + b <= query i.  Read by the loaded-mask
// variant only.
struct TrilBits {
  uint32_t w[kMaxL * (kMaxL / 32)];
};
constexpr TrilBits make_tril_bits() {
  TrilBits t{};
  for (int i = 0; i < kMaxL; ++i)
    for (int wd = 0; wd < kMaxL / 32; ++wd) {
      const int k = i - 32 * wd;
      t.w[i * (kMaxL / 32) + wd] = k < 0 ? 0u : (k >= 31 ? 0xffffffffu : ((2u << k) - 1u));
    }
  return t;
}
__device__ const TrilBits kTrilBits = make_tril_bits();

// Per-column-tile decay tables.  Column tile I >= 1 (queries 16I .. 16I+15)
// takes token r = 16I as its reference: for a key j < r,
//   decay(i, j) Delta_j = exp(cum_i - cum_r) * W_I[j],   W_I[j] = exp(cum_r - cum_j) Delta_j,
// both factors <= 1 since cum falls.  Row I holds its 16I entries at 8 I (I-1);
// only the rows of the chunk's tiles are written.
constexpr int tile_table_size(int LMAX) { return 8 * (LMAX / 16) * (LMAX / 16 - 1); }

template <int VAR, int NTH, int LMAX>
__device__ __forceinline__ void tile_decay_table(int Lc, const float* s_d, const float* s_cum,
                                                 float* s_w) {
  constexpr int NT = LMAX / 16, NW = NTH / 64;
  const int nrt = (Lc + 15) / 16;
  auto entry = [&](int I, int j) {
    s_w[8 * I * (I - 1) + j] =
        __fmul_rn(decay_factor<VAR>(fast_exp(__fsub_rn(s_cum[16 * I], s_cum[j]))), s_d[j]);
  };
  if constexpr (NW == NT / 2) {
    // wavefront w > 0 fills rows w and NT - w (16 NT entries together),
    // wavefront 0 row NT/2: every wavefront the same 16 NT / 64 sweeps
    const int tid = opaque_tid();
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int I1 = w > 0 ? w : NT / 2, I2 = w > 0 ? NT - w : 0;
    const int n1 = I1 < nrt ? 16 * I1 : 0, n2 = I2 > 0 && I2 < nrt ? 16 * I2 : 0;
    for (int e = lane; e < n1 + n2; e += 64) {
      if (e < n1) entry(I1, e);
      else entry(I2, e - n1);
    }
  } else {
    const int n = 8 * nrt * (nrt - 1);
    for (int e = opaque_tid(); e < n; e += NTH) {
      int I = (int)(0.5f + sqrtf(0.25f + 0.125f * (float)e));   // row: 8 I (I-1) <= e
      if (8 * I * (I - 1) > e) --I;
      else if (8 * I * (I + 1) <= e) ++I;
      entry(I, e - 8 * I * (I - 1));
    }
  }
}

// State weights w_l = Delta_l exp(cum_last - cum_l) of the chunk summary state.
template <int LMAX, int NTH = kThreads>
__device__ __forceinline__ void state_weights(int Lc, const float* s_d, const float* s_cum,
                                              float* s_ws) {
  const float cum_last = s_cum[Lc - 1];
  for (int l = opaque_tid(); l < LMAX; l += NTH)
    s_ws[l] = (l < Lc) ? __fmul_rn(s_d[l], fast_exp(__fsub_rn(cum_last, s_cum[l]))) : 0.0f;
}

__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// Column tile k of wavefront w of NW: the tiles are dealt in a snake order
// (0 1 .. NW-1 NW-1 .. 1 0), which balances the triangular work.
template <int NW>
__device__ __forceinline__ int col_tile_of(int wave, int k) {
  return NW * k + ((k & 1) ? NW - 1 - wave : wave);
}

// Outputs of one chunk, y^T tiles [p][i]: wavefront w of NW owns the one or
// two 16-query column tiles col_tile_of<NW>(w, k) and all P/16 head tiles.
// For column tile I (reference token r = 16I, query i = 16I + lane%16):
//   acc  = exp(cum_r) * sum_n bf16(h_{c-1})[p][n] C[i][n]          inter-chunk term
//   acc += sum_{j < r} x^T[p][j] bf16(S[i][j] W_I[j])               earlier key tiles
//   acc *= exp(cum_i - cum_r)
//   acc += sum_{r <= j <= i} x^T[p][j] bf16(S[i][j] exp(cum_i - cum_j) Delta_j)
//   acc += sum_k x^T[p][16I + k] E_m[k][i - 16I],  m = 1..3  (the skip term D x:
//          E_m = d_m I with D = d_1 + d_2 + d_3 split exactly into three
//          bfloat16 parts, so each product is exact in float32)
//   y[i][p] = bf16(acc)
// so an earlier key costs one multiply (the exponentials are in the table)
// and only the 16 x 16 diagonal tile takes exponentials and the causal
// select (made before the exponential's result is used).  Earlier keys go 32
// at a time through v_mfma_f32_16x16x32_bf16 (lane: 8 consecutive keys 8q ..);
// a 16-key remainder and the diagonal tile through v_mfma_f32_16x16x16_bf16
// (lane: keys 4q ..).
//   s_h   bf16(h_{c-1})[p][n] (row stride N + 8): the inter-chunk operand
//   s_xt  bf16 x[j][p]       (row stride P + 16), read transposed (xt_at4/8)
//   s_d, s_cum, s_w: Delta, cum and the per-tile decay tables of the chunk
// S (C B^T, bfloat16) and C come from global memory (L2: shared by all heads
// of a group).  The S rows of every 32-key step a wavefront needs are
// requested at once by prefetch() (one round trip instead of one per key
// step), together with the first tile's C: tile 0's steps fill sf from the
// front, tile 1's from the back (their counts add up to NS), so every
// register index is static.  The two 16-key blocks of a tile (before and on
// the diagonal) are requested at the tile's start.
// C_AHEAD: the second tile's C is loaded behind the first tile's intra term
// (else at the second tile's start, 16 registers fewer).
template <int P, int N, int LMAX, int NW, int VAR = kDecayF32, bool C_AHEAD = true>
struct ChunkOut {
  static constexpr int TP = P / 16;
  static constexpr int NT = LMAX / 16;   // 16-query column tiles of a chunk
  static constexpr int CT = NT / NW;     // column tiles per wavefront
  static_assert(NT % NW == 0 && (CT == 1 || CT == 2), "one or two column tiles per wavefront");
  // 32-key steps before the wavefront's tiles: tile w has w/2, and with a
  // second tile 2NW-1-w the two add up to NW-1
  static constexpr int NS = CT == 2 ? NW - 1 : (NW - 1) / 2;
  static constexpr int HS = N + 8;

  const ScanArgs& a;
  int64_t b, c, h, g;
  int Lc;
  float Dh;                       // D of head h (0 without D)
  f32x4 yacc[TP];                 // y of the last tile run() computed, not yet stored
  int yrow;                       // its token (per lane; >= Lc: nothing to store)
  bf16x8 cf[N / 32];              // C[i][32 nb + 8q ..] of the tile about to run
  bf16x8 sf[NS > 0 ? NS : 1];     // S[i][32 ks + 8q ..] of the 32-key steps

  __device__ __forceinline__ ChunkOut(const ScanArgs& a_, int64_t b_, int64_t c_, int64_t h_,
                                      int64_t g_, int Lc_)
      : a(a_), b(b_), c(c_), h(h_), g(g_), Lc(Lc_), Dh(a_.D ? a_.D[h_] : 0.0f), yrow(0) {}

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

  // C fragments of column tile I (rows past the chunk read its last row, with
  // no zeroing select: they feed only output columns that are never stored)
  __device__ __forceinline__ void load_c(int I) {
    const int lane = lane_opaque(), q = lane >> 4, r16 = lane & 15;
    // chunk base (uniform) + a 32-bit lane offset: the loads take the
    // scalar-base form, with no 64-bit address arithmetic per lane
    const bf16* Cg = reinterpret_cast<const bf16*>(a.C) + ((b * a.T + c * a.L) * a.G + g) * N;
    const uint32_t i = (uint32_t)min(16 * I + r16, Lc - 1);
    const uint32_t rs = (uint32_t)(a.G * N);
#pragma unroll
    for (int nb = 0; nb < N / 32; ++nb) cf[nb] = ld8(off32(Cg, i * rs + nb * 32 + 8 * q));
  }

  // The first tile's C and every S row the wavefront's tiles need.  Each load
  // is issued on every path (exact waits): a tile past the chunk, or a step a
  // tile does not have, reads the first keys of the chunk's last tile.
  __device__ __forceinline__ void prefetch() {
    const int lane = lane_opaque(), q = lane >> 4, r16 = lane & 15;
    const int wave = wave_id(), n_rt = nrt();
    load_c(min(col_tile_of<NW>(wave, 0), n_rt - 1));
    const bf16* S = reinterpret_cast<const bf16*>(a.ws_cb) + ((b * a.Nc + c) * a.G + g) * a.L * a.L;
    uint32_t row[CT];
    int nf[CT];
#pragma unroll
    for (int k = 0; k < CT; ++k) {
      const int I = col_tile_of<NW>(wave, k);
      const bool v = I < n_rt;
      const int Ic = v ? I : n_rt - 1;
      row[k] = (uint32_t)(16 * Ic + r16) * (uint32_t)a.L + 8 * q;
      nf[k] = v ? I >> 1 : 0;
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      uint32_t src;
      if constexpr (CT == 2) {
        const int ks1 = NS - 1 - j;
        src = j < nf[0] ? row[0] + 32 * j : (ks1 < nf[1] ? row[1] + 32 * ks1 : row[1]);
      } else {
        src = j < nf[0] ? row[0] + 32 * j : row[0];
      }
      sf[j] = ld8(off32(S, src));
    }
  }

  // y of the pending tile: lane holds y[yrow][p..p+3], p = 16 pt + 4q.
  // Stores and loads share one in-order completion counter, so a store issued
  // ahead of a load makes every wait for that load wait for the store too:
  // each tile's store is issued after the next tile's loads, and the last
  // one by the caller, after the loads it issues next.  The stores are issued
  // on every path, also by lanes with no row to store (rows past the chunk,
  // or no tile run): a store issued on some paths only is counted as absent
  // by the waits that follow it, so a wait for a load issued just before it
  // would wait for the store too.  Those lanes write their meaningless values
  // into the chunk's C B^T tile (0, L/16 - 1), strictly above the diagonal,
  // which the scan never writes or reads (all of their stores to one place).
  __device__ __forceinline__ void store_pending() {
    const int lane = lane_opaque(), q = lane >> 4, r16 = lane & 15;
    const bool ok = yrow < Lc;
    bf16* yg = reinterpret_cast<bf16*>(a.y) + ((b * a.T + c * a.L) * a.H + h) * P;
    bf16* tg = reinterpret_cast<bf16*>(a.ws_cb) + ((b * a.Nc + c) * a.G + g) * a.L * a.L;
    const uint32_t ry = (uint32_t)yrow * (uint32_t)(a.H * P) + 4 * q;
    const uint32_t rt = (uint32_t)r16 * (uint32_t)a.L + (uint32_t)(a.L - 16) + 4 * q;
    bf16* dst = ok ? off32(yg, ry) : off32(tg, rt);
    const uint32_t step = ok ? 16u : 0u;
#pragma unroll
    for (int pt = 0; pt < TP; ++pt) {
      bf16x4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = (bf16)yacc[pt][r];
      st4b(off32(dst, step * pt), o);
    }
  }

  // Both tiles; prefetch() must have been called, and store_pending() must
  // follow.
  __device__ __forceinline__ void run(const float* s_d, const float* s_cum, const float* s_w,
                                      const bf16* s_xt, const bf16* s_h) {
    const int lane = lane_opaque(), q = lane >> 4, r16 = lane & 15;
    const int wave = wave_id(), n_rt = nrt();
    const bf16* xb8 = xt_lane<P, 8>(s_xt, lane);   // 32-key steps: 8 tokens per group
    const bf16* xb4 = xt_lane<P, 4>(s_xt, lane);   // 16-key steps: 4 tokens per group
    yrow = Lc;   // nothing pending unless a tile runs
    // skip-term operands: D = d1 + d2 + d3 exactly (bfloat16 parts of the
    // float32 value and of its remainders), on the diagonal of a 16 x 16 block
    bf16x4 e1, e2, e3;
    {
      const bf16 d1 = (bf16)Dh;
      const float r1 = __fsub_rn(Dh, (float)d1);
      const bf16 d2 = (bf16)r1;
      const bf16 d3 = (bf16)__fsub_rn(r1, (float)d2);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool on = 4 * q + e == r16;
        e1[e] = on ? d1 : (bf16)0.0f;
        e2[e] = on ? d2 : (bf16)0.0f;
        e3[e] = on ? d3 : (bf16)0.0f;
      }
    }

#pragma unroll
    for (int k = 0; k < CT; ++k) {
      const int I = col_tile_of<NW>(wave, k);
      if (I >= n_rt) break;                 // later tiles lie further on
      if (!C_AHEAD && k > 0) load_c(I);
      const int ri = 16 * I + r16;
      // the 16-key block before the diagonal (re-reading the diagonal one when
      // I is even) and the diagonal block: consumed after the 32-key steps
      const bf16* sch = reinterpret_cast<const bf16*>(a.ws_cb) +
                        ((b * a.Nc + c) * a.G + g) * a.L * a.L;
      const uint32_t srow = (uint32_t)ri * (uint32_t)a.L + 4 * q;
      const bf16x4 sod = ld4b(off32(sch, srow + 16 * (I - (I & 1))));
      const bf16x4 sdg = ld4b(off32(sch, srow + 16 * I));
      if (k > 0) store_pending();   // the previous tile's y, behind this tile's loads
      f32x4 acc[TP];
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};

      // ---- inter-chunk term, then the decay from the chunk start to the
      // tile's reference token ----
#pragma unroll
      for (int nb = 0; nb < N / 32; ++nb) {
        bf16x8 hf[TP];
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) hf[pt] = ld8(s_h + (16 * pt + r16) * HS + 32 * nb + 8 * q);
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) acc[pt] = mma(hf[pt], cf[nb], acc[pt]);
      }
      // the C fragments are dead now: the next tile's fly behind this one's intra term
      if (C_AHEAD && k + 1 < CT) load_c(min(col_tile_of<NW>(wave, k + 1), n_rt - 1));
      {
        const float er = decay_factor<VAR>(fast_exp(s_cum[16 * I]));
#pragma unroll
        for (int pt = 0; pt < TP; ++pt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[pt][r] = __fmul_rn(acc[pt][r], er);
      }

      // ---- earlier key tiles: 32-key steps, then the odd 16-key one ----
      const float* wI = s_w + 8 * I * (I - 1);
      const float* wq = wI + 8 * q;
      const int nfull = I >> 1;
#pragma unroll
      for (int ks = 0; ks < NS; ++ks) {
        if (ks < nfull) {
          const bf16x8 st = sf[k == 0 ? ks : NS - 1 - ks];
          const float4 w0 = ld4(wq + 32 * ks), w1 = ld4(wq + 32 * ks + 4);
          bf16x8 m;
          m[0] = (bf16)__fmul_rn((float)st[0], w0.x);
          m[1] = (bf16)__fmul_rn((float)st[1], w0.y);
          m[2] = (bf16)__fmul_rn((float)st[2], w0.z);
          m[3] = (bf16)__fmul_rn((float)st[3], w0.w);
          m[4] = (bf16)__fmul_rn((float)st[4], w1.x);
          m[5] = (bf16)__fmul_rn((float)st[5], w1.y);
          m[6] = (bf16)__fmul_rn((float)st[6], w1.z);
          m[7] = (bf16)__fmul_rn((float)st[7], w1.w);
#pragma unroll
          for (int pt = 0; pt < TP; ++pt)
            acc[pt] = mma(xt_at8<P>(xb8, 32 * ks, 16 * pt), m, acc[pt]);
        }
      }
      if (I & 1) {   // the key tile just before the diagonal one
        const int k0 = 16 * (I - 1) + 4 * q;
        const float4 w = ld4(wI + k0);
        const bf16x4 st = sod;
        bf16x4 m;
        m[0] = (bf16)__fmul_rn((float)st[0], w.x);
        m[1] = (bf16)__fmul_rn((float)st[1], w.y);
        m[2] = (bf16)__fmul_rn((float)st[2], w.z);
        m[3] = (bf16)__fmul_rn((float)st[3], w.w);
#pragma unroll
        for (int pt = 0; pt < TP; ++pt)
          acc[pt] = mma16(xt_at4<P>(xb4, 16 * (I - 1), 16 * pt), m, acc[pt]);
      }
      // decay from the reference token to the query
      const float cum_i = s_cum[ri];
      {
        const float u = decay_factor<VAR>(fast_exp(__fsub_rn(cum_i, s_cum[16 * I])));
#pragma unroll
        for (int pt = 0; pt < TP; ++pt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[pt][r] = __fmul_rn(acc[pt][r], u);
      }
      // ---- diagonal tile: keys j0 .. j0+3, causal select before the result is used ----
      {
        const int j0 = 16 * I + 4 * q;
        const float4 cj = ld4(s_cum + j0), dj = ld4(s_d + j0);
        const bf16x4 st = sdg;
        bool mk[4];
        if constexpr (VAR == kMaskLoaded) {
          const uint32_t bits = kTrilBits.w[ri * (kMaxL / 32) + (j0 >> 5)] >> (j0 & 31);
#pragma unroll
          for (int e = 0; e < 4; ++e) mk[e] = (bits >> e) & 1u;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) mk[e] = j0 + e <= ri;
        }
        auto dec = [&](bool on, float sv, float cjv, float djv) {
          return on ? (bf16)__fmul_rn(__fmul_rn(sv, decay_factor<VAR>(fast_exp(__fsub_rn(cum_i, cjv)))), djv)
                    : (bf16)0.0f;
        };
        bf16x4 m;
        m[0] = dec(mk[0], (float)st[0], cj.x, dj.x);
        m[1] = dec(mk[1], (float)st[1], cj.y, dj.y);
        m[2] = dec(mk[2], (float)st[2], cj.z, dj.z);
        m[3] = dec(mk[3], (float)st[3], cj.w, dj.w);
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) {
          const bf16x4 xd = xt_at4<P>(xb4, 16 * I, 16 * pt);
          acc[pt] = mma16(xd, m, acc[pt]);
          // the skip term D x of the tile's own tokens, on the same x^T fragment
          acc[pt] = mma16(xd, e1, acc[pt]);
          acc[pt] = mma16(xd, e2, acc[pt]);
          acc[pt] = mma16(xd, e3, acc[pt]);
        }
      }

      // ---- y of this tile: stored later (store_pending) ----
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) yacc[pt] = acc[pt];
      yrow = ri;
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
// The output kernels run LMAX/32 wavefronts per workgroup (two 16-query
// column tiles each; the chain kernel 8): two workgroups share a compute unit
// (LDS), so each SIMD keeps four wavefronts to cover the latency of the rows
// they read from L2.  Delta and its prefix sum are formed by the first 256
// threads with the same arithmetic as every other kernel of the scan
// (bit-identical values).
constexpr int kOutThreads = 512;   // the chain kernel, and the phased one at chunks <= 256
constexpr int kOutWaves = kOutThreads / 64;

// Delta and the chunk-local prefix sum for a workgroup of more than kThreads
// threads: the first kThreads compute (as chunk_delta_cumsum), all wait.
__device__ __forceinline__ void chunk_delta_cumsum_wide(const ScanArgs& a, int64_t b, int64_t c,
                                                        int64_t h, float* s_d, float* s_cum,
                                                        float* s_wsum) {
  const bool on = threadIdx.x < kThreads;
  DeltaScan ds{};
  if (on) ds = chunk_scan_stage1(a, c, h, chunk_dt_load(a, b, c, h), s_wsum);
  __syncthreads();
  if (on) chunk_scan_stage2(a, ds, s_wsum, s_d, s_cum);
  __syncthreads();
}

template <int P, int N, int LMAX, int VAR>
__global__ __launch_bounds__(2 * LMAX) __attribute__((amdgpu_waves_per_eu(LMAX <= 256 ? 4 : 2)))
void k_chunk_out_bf16(ScanArgs a) {
  constexpr int HS = N + 8;
  constexpr int NTH = 2 * LMAX, NW = NTH / 64;
  __shared__ __attribute__((aligned(16))) float s_d[LMAX];
  __shared__ __attribute__((aligned(16))) float s_cum[LMAX];
  __shared__ float s_wsum[4];
  __shared__ __attribute__((aligned(16))) float s_w[tile_table_size(LMAX) + 4];
  __shared__ __attribute__((aligned(16))) bf16 s_xt[LMAX * x_row_stride(P)];
  __shared__ __attribute__((aligned(16))) bf16 s_h[P * HS];

  const int tid = threadIdx.x;
  const int64_t u = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t h = u % a.H, bc = u / a.H, c = bc % a.Nc, b = bc / a.Nc;
  const int64_t g = h / (a.H / a.G);
  const int Lc = chunk_len(a, c);

  // every global load of the staging is issued before the first barrier
  XStage<P, LMAX, NTH> xs;
  xs.load(a, b, c, h);
  constexpr int HV = P * N / 8;                 // 8-element groups of the state
  constexpr int NHV = (HV + NTH - 1) / NTH;
  const bf16* hp = reinterpret_cast<const bf16*>(a.ws_hb) +
                   ((b * a.H + h) * a.Nc + c) * (int64_t)(P * N);
  bf16x8 hv[NHV];
#pragma unroll
  for (int i = 0; i < NHV; ++i) hv[i] = ld8(hp + min(tid + i * NTH, HV - 1) * 8);
  ChunkOut<P, N, LMAX, NW, VAR> out(a, b, c, h, g, Lc);
  out.prefetch();
  chunk_delta_cumsum_wide(a, b, c, h, s_d, s_cum, s_wsum);  // ends with a barrier
  tile_decay_table<VAR, NTH, LMAX>(Lc, s_d, s_cum, s_w);
  xs.store(s_xt);
#pragma unroll
  for (int i = 0; i < NHV; ++i) {
    const int e = tid + i * NTH;
    if (e < HV) st8(s_h + ((e * 8) / N) * HS + (e * 8) % N, hv[i]);
  }
  __syncthreads();
  out.run(s_d, s_cum, s_w, s_xt, s_h);
  out.store_pending();
}

// ---------------------------------------------------------------------------
// Pre-pass of the chain's head shapes (chunks up to 256), both schedules.
// Blocks [0, ncb): C B^T of one (b, c, g) per workgroup of 8 wavefronts.  B of
// the chunk is staged in LDS, zero past the chunk's end, rows padded to N + 8
// elements so that the 16 rows one fragment read touches fall in distinct
// banks; wavefront w computes the tiles (I, J <= I) of its row tiles
// I = col_tile_of<8>(w, k) (16 - I + 1 + I + 1 tiles whatever w: balanced)
// with the C fragments of the row tile held in registers.  B and C are read
// from memory once per chunk (one tile per wavefront had read each row once
// per tile it enters: 4.6 times the bytes of B and C at 8 x 16384).  The
// products are those of cb_tile_bf16, in the same order.
// The transposed copy of B, ws_bt[(b, c, g)][n][l] = B[b, cL + l, g, n], zero
// past the chunk's end: one thread per 8 x 8 block (8 tokens x 8 state
// columns), consecutive threads on consecutive token blocks, so a row of
// ws_bt is written by consecutive threads; from the staged rows in the
// workgroup-per-chunk mode, else in blocks from ncb.
// ---------------------------------------------------------------------------
constexpr int kPrepThreads = 512;

template <int N>
__device__ __forceinline__ void cb_chunk_bf16(const ScanArgs& a, int64_t bcg, bf16* s_b) {
  constexpr int BS = N + 8, NU = N / 8;
  constexpr int NS8 = 256 * NU / kPrepThreads;    // 16-byte units of B per thread
  const int tid = opaque_tid();
  const int64_t g = bcg % a.G, bc = bcg / a.G, c = bc % a.Nc, b = bc / a.Nc;
  const int Lc = chunk_len(a, c);
  const int64_t rs = a.G * N;
  const bf16* Bg = reinterpret_cast<const bf16*>(a.B) + ((b * a.T + c * a.L) * a.G + g) * N;
  const bf16* Cg = reinterpret_cast<const bf16*>(a.C) + ((b * a.T + c * a.L) * a.G + g) * N;
  {
    bf16x8 v[NS8];
#pragma unroll
    for (int k = 0; k < NS8; ++k) {
      const int e = tid + k * kPrepThreads, l = e / NU, u = e % NU;
      v[k] = ld8(Bg + min(l, Lc - 1) * rs + 8 * u);
    }
#pragma unroll
    for (int k = 0; k < NS8; ++k) {
      const int e = tid + k * kPrepThreads, l = e / NU, u = e % NU;
      st8(s_b + l * BS + 8 * u, l < Lc ? v[k] : bf16x8{});
    }
  }
  __syncthreads();
  // the transposed copy ws_bt of the chunk, from the staged rows (zero past
  // the chunk's end as staged): 8 x 8 blocks, consecutive threads on
  // consecutive token blocks, as the B^T blocks of the tile-per-wavefront mode
  {
    const int LB = (int)(a.L / 8);
    bf16* bt = reinterpret_cast<bf16*>(a.ws_bt) + bcg * N * a.L;
    for (int e = tid; e < LB * (N / 8); e += kPrepThreads) {
      const int lb = e % LB, nb = e / LB;
      bf16x8 in[8], tr[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) in[r] = ld8(s_b + (8 * lb + r) * BS + 8 * nb);
      transpose8(in, tr);
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) st8(bt + (int64_t)(8 * nb + cc) * a.L + 8 * lb, tr[cc]);
    }
  }
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int n_rt = (Lc + 15) / 16;
#pragma unroll 1
  for (int k = 0; k < 2; ++k) {
    const int I = col_tile_of<8>(wave, k);
    if (I >= n_rt) continue;                  // uniform
    const int ri = 16 * I + r16;
    bf16x8 cf[N / 32];
#pragma unroll
    for (int nb = 0; nb < N / 32; ++nb)
      cf[nb] = ld8_masked(Cg + min(ri, Lc - 1) * rs + nb * 32 + 8 * q, ri < Lc);
#pragma unroll 2
    for (int J = 0; J <= I; ++J) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nb = 0; nb < N / 32; ++nb)
        acc = mma(ld8(s_b + (16 * J + r16) * BS + nb * 32 + 8 * q), cf[nb], acc);
      // lane holds S[16I + r16][16J + 4q + r], r = 0..3
      const int64_t at = bcg * a.L * a.L + (int64_t)(16 * I + r16) * a.L + 16 * J + 4 * q;
      if (a.cb_bf16) {
        bf16x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = (bf16)acc[r];
        st4b(reinterpret_cast<bf16*>(a.ws_cb) + at, o);
      } else {
        st4(a.ws_cb + at, make_float4(acc[0], acc[1], acc[2], acc[3]));
      }
    }
  }
}

// per_chunk = 0 (too few chunks to fill the GPU): block k of [0, ncb) gives
// its 8 wavefronts the tiles 8k .. 8k+7 of the chunks' tile list, one each
// (cb_tile_bf16, the same products).
template <int N>
__global__ __launch_bounds__(kPrepThreads) void k_cb_and_bt_bf16(ScanArgs a, int64_t ncb,
                                                                 int per_chunk, int ntiles) {
  __shared__ __attribute__((aligned(16))) bf16 s_b[256 * (N + 8)];
  if ((int64_t)blockIdx.x < ncb) {
    if (per_chunk) {
      cb_chunk_bf16<N>(a, blockIdx.x, s_b);
    } else {
      const int64_t item = (int64_t)blockIdx.x * kOutWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
      if (item < a.Bt * a.Nc * a.G * ntiles) cb_tile_bf16<N>(a, item / ntiles, (int)(item % ntiles));
    }
    return;
  }
  const int LB = (int)(a.L / 8);
  const int64_t per = (int64_t)LB * (N / 8);
  const int64_t id = ((int64_t)blockIdx.x - ncb) * kPrepThreads + threadIdx.x;
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

// Launch of the pre-pass (both schedules, chain shapes, L <= 256): a
// workgroup per chunk once the chunks fill the GPU (two workgroups per
// compute unit), else a wavefront per tile.
constexpr int64_t kPrepChunkMin = 256;
template <int N>
hipError_t launch_prepass(const ScanArgs& a, hipStream_t stream) {
  const int64_t chunks = a.Bt * a.Nc * a.G;
  const int ntiles = cb_tiles(a);
  const int per_chunk = chunks >= kPrepChunkMin ? 1 : 0;
  const int64_t ncb = per_chunk ? chunks : (chunks * ntiles + kOutWaves - 1) / kOutWaves;
  // (a workgroup per chunk writes the chunk's B^T itself)
  const int64_t nbt =
      per_chunk ? 0 : (chunks * (a.L / 8) * (N / 8) + kPrepThreads - 1) / kPrepThreads;
  hipLaunchKernelGGL((k_cb_and_bt_bf16<N>), dim3((unsigned)(ncb + nbt)), dim3(kPrepThreads), 0,
                     stream, a, ncb, per_chunk, ntiles);
  return hipGetLastError();
}

// Chunk summary state of one wavefront's tiles, from zero, in 32-token
// steps: t[ip][n = 16 nt + 4q + r][p = 16 (pt0 + ip) + lane%16] = sum over the
// chunk of (B^T w)_bf16 x, with B^T w the wavefront's B^T fragment (n-tile
// nt, from the pre-pass copy ws_bt) scaled by the state weights in LDS and
// x^T from LDS.  state_bt_load requests every fragment of the chunk at once
// (steps past the chunk re-read its last); state_tiles consumes them.  The
// chain kernel and the phased chunk-state kernel share both, so they form
// S_c with the same instructions in the same order.
template <int N, int LMAX>
__device__ __forceinline__ void state_bt_load(const ScanArgs& a, int64_t b, int64_t c, int64_t g,
                                              int nt, int Lc, bf16x8 (&bt)[LMAX / 32]) {
  const int nks = (Lc + 31) / 32;
  const int lane = opaque_tid() & 63, q = lane >> 4, r16 = lane & 15;
  const bf16* btc = reinterpret_cast<const bf16*>(a.ws_bt) +
                    ((b * a.Nc + c) * a.G + g) * (int64_t)(N * a.L);
  const uint32_t row = (uint32_t)(16 * nt + r16) * (uint32_t)a.L + 8 * q;
#pragma unroll
  for (int ks = 0; ks < LMAX / 32; ++ks) bt[ks] = ld8(off32(btc, row + 32 * min(ks, nks - 1)));
}

template <int P, int LMAX, int TPW>
__device__ __forceinline__ void state_tiles(const bf16x8 (&bt)[LMAX / 32], int pt0, int Lc,
                                            const bf16* s_xt, const float* s_ws,
                                            f32x4 (&t)[TPW]) {
  constexpr int NKS = LMAX / 32;
  const int nks = (Lc + 31) / 32;
  const int lane = opaque_tid() & 63, q = lane >> 4;
  const bf16* xb8 = xt_lane<P, 8>(s_xt, lane);
  const float* wq = s_ws + 8 * q;
#pragma unroll
  for (int ip = 0; ip < TPW; ++ip) t[ip] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if (ks < nks) {
      const bf16x8 bw = scale8(bt[ks], ld4(wq + 32 * ks), ld4(wq + 32 * ks + 4));
#pragma unroll
      for (int ip = 0; ip < TPW; ++ip)
        t[ip] = mma(bw, xt_at8<P>(xb8, 32 * ks, 16 * (pt0 + ip)), t[ip]);
    }
  }
}

// Wavefronts per state n-tile and p-tiles per wavefront when 8 wavefronts
// share the P x N state of a head.
template <int P, int N>
struct StateSplit {
  static constexpr int TP = P / 16, TN = N / 16, NW = 8;
  static constexpr int WPN = NW / TN;
  static constexpr int TPW = TP / WPN;
  static_assert(TN <= NW && NW % TN == 0 && TP % WPN == 0, "whole state tiles per wavefront");
};

// Phased schedule, phase 1 for the chain shapes (chain_variant, L <= 256):
// chunk summary states S_c from the pre-pass's B^T (k_cb_and_bt_bf16, which
// also forms C B^T), one workgroup of 8 wavefronts per (b, c, g) and run of
// `per` consecutive heads of group g.  The wavefront's B^T fragments are the
// same for every head of the group and stay in registers; the next head's x
// and dt are requested before the current head's products, so their latency
// hides behind them (the last head, peeled, requests nothing).  Stored as
// [p][n] to ws_state; exp(cum_last) to ws_alpha.
template <int P, int N>
__global__ __launch_bounds__(kOutThreads) __attribute__((amdgpu_waves_per_eu(4)))
void k_chunk_state_bf16(ScanArgs a, int per, int splits) {
  constexpr int LMAX = 256, NTH = kOutThreads;
  using SP = StateSplit<P, N>;
  __shared__ __attribute__((aligned(16))) float s_d[LMAX];
  __shared__ __attribute__((aligned(16))) float s_cum[LMAX];
  __shared__ __attribute__((aligned(16))) float s_ws[LMAX];
  __shared__ float s_wsum[4];
  __shared__ __attribute__((aligned(16))) bf16 s_xt[LMAX * x_row_stride(P)];

  const int tid = threadIdx.x;
  const bool scan_thread = tid < kThreads;   // Delta and its prefix sum
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nt = wave % SP::TN, pt0 = (wave / SP::TN) * SP::TPW;
  // the runs of one (b, c, g) are consecutive: they share an XCD and B^T in its L2
  const int64_t u = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t sp = u % splits, bcg = u / splits;
  const int64_t g = bcg % a.G, bc = bcg / a.G, c = bc % a.Nc, b = bc / a.Nc;
  const int64_t hpg = a.H / a.G;
  const int64_t h_lo = g * hpg + sp * per;
  const int64_t h_hi = min<int64_t>(h_lo + per, (g + 1) * hpg);
  const int Lc = chunk_len(a, c);
  const int lane = tid & 63, q = lane >> 4, r16 = lane & 15;

  // every global load of the first head is issued before the first wait
  bf16x8 bt[LMAX / 32];
  state_bt_load<N, LMAX>(a, b, c, g, nt, Lc, bt);
  float2 dtv = scan_thread ? chunk_dt_load(a, b, c, h_lo) : make_float2(0.f, 0.f);
  HeadConsts hc = head_consts(a, h_lo);
  XStage<P, LMAX, NTH> xs;
  xs.load(a, b, c, h_lo);

  auto head = [&](int64_t h, auto more) {
    DeltaScan ds{};
    if (scan_thread) ds = chunk_scan_stage1(a, c, hc, dtv, s_wsum);
    __syncthreads();
    if (scan_thread) chunk_scan_stage2(a, ds, s_wsum, s_d, s_cum);
    __syncthreads();
    xs.store(s_xt);
    state_weights<LMAX, NTH>(Lc, s_d, s_cum, s_ws);
    if (tid == 0) a.ws_alpha[(b * a.H + h) * a.Nc + c] = fast_exp(s_cum[Lc - 1]);
    __syncthreads();
    if constexpr (decltype(more)::value) {
      // the next head's operands, behind this head's products
      if (scan_thread) dtv = chunk_dt_load(a, b, c, h + 1);
      hc = head_consts(a, h + 1);
      xs.load(a, b, c, h + 1);
    }
    f32x4 t[SP::TPW];
    state_tiles<P, LMAX, SP::TPW>(bt, pt0, Lc, s_xt, s_ws, t);
    // lane holds S[n = 16 nt + 4q + r][p = 16 (pt0 + ip) + r16]: 4 consecutive n of one p
    float* out = a.ws_state + ((b * a.H + h) * a.Nc + c) * (int64_t)(P * N);
#pragma unroll
    for (int ip = 0; ip < SP::TPW; ++ip)
      st4(out + (16 * (pt0 + ip) + r16) * N + 16 * nt + 4 * q,
          make_float4(t[ip][0], t[ip][1], t[ip][2], t[ip][3]));
    // s_d, s_cum and s_wsum are next written after the next head's stage-1
    // barrier, s_xt and s_ws after its stage-2 one: every wavefront has left
    // this head's products by then
  };
  for (int64_t h = h_lo; h + 1 < h_hi; ++h) head(h, std::true_type{});
  head(h_hi - 1, std::false_type{});
}

// Chain kernel: one workgroup of 8 wavefronts per (b, h), chunks in order.
// The float32 state [n][p] lives in matrix-core accumulators for the whole
// sequence: wavefront w keeps n-tile w % (N/16) and P/16 / (8 / (N/16))
// p-tiles of it; LDS holds only bf16(h) as the inter-chunk operand.  Delta
// and its prefix sum run one chunk ahead, in double-buffered LDS, so a chunk
// takes two barriers:
//   stage:   x^T and bf16(h_{c-1}) into LDS; the first tile's C and S rows
//            requested; chunk c's decay tables and state weights (from its
//            prefix, formed during chunk c-1); stage 1 of chunk c+1's prefix
//            sum (wavefronts 0-3); barrier
//   then:    stage 2 of chunk c+1's prefix sum (wavefronts 0-3, into the
//            other buffer); outputs (ChunkOut); S_c = sum_ks (B^T w)_bf16 x
//            into a fresh accumulator, h_c = fma(alpha_c, h_{c-1}, S_c), the
//            next chunk's x requested; barrier
// Load order (memory counters retire loads in order): dt two chunks ahead
// before the outputs; the state step's B^T fragments, then the next chunk's
// x; the first output-pass operands before the first barrier.
template <int P, int N, int LMAX, int VAR>
__global__ __launch_bounds__(kOutThreads) __attribute__((amdgpu_waves_per_eu(4)))
void k_chain_bf16(ScanArgs a) {
  constexpr int NTH = kOutThreads, NW = kOutWaves;
  constexpr int TN = StateSplit<P, N>::TN, TPW = StateSplit<P, N>::TPW;
  constexpr int HS = N + 8;
  using Out = ChunkOut<P, N, LMAX, NW, VAR, false>;
  __shared__ __attribute__((aligned(16))) float s_d[2][LMAX];
  __shared__ __attribute__((aligned(16))) float s_cum[2][LMAX];
  __shared__ __attribute__((aligned(16))) float s_ws[LMAX];
  __shared__ float s_wsum[4];
  __shared__ __attribute__((aligned(16))) float s_w[tile_table_size(LMAX) + 4];
  __shared__ __attribute__((aligned(16))) bf16 s_xt[LMAX * x_row_stride(P)];
  __shared__ __attribute__((aligned(16))) bf16 s_h[P * HS];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool scan_thread = threadIdx.x < kThreads;   // Delta and its prefix sum
  const int nt = wave % TN, pt0 = (wave / TN) * TPW;
  const int64_t u = xcd_remap(blockIdx.x, gridDim.x);   // heads of a batch row share an XCD
  const int64_t h = u % a.H, b = u / a.H;
  const int64_t g = h / (a.H / a.G);
  const int64_t sbase = (b * a.H + h) * (int64_t)(P * N);

  const HeadConsts hc = head_consts(a, h);
  // chunk 0's prefix into buffer 0; chunk 1's dt
  {
    DeltaScan ds{};
    if (scan_thread) ds = chunk_scan_stage1(a, 0, hc, chunk_dt_load(a, b, 0, h), s_wsum);
    __syncthreads();
    if (scan_thread) chunk_scan_stage2(a, ds, s_wsum, s_d[0], s_cum[0]);
  }
  float2 dtv = scan_thread ? chunk_dt_load(a, b, a.Nc > 1 ? 1 : 0, h) : make_float2(0.f, 0.f);
  Out out(a, b, 0, h, g, chunk_len(a, 0));
  XStage<P, LMAX, NTH> xs;
  xs.load(a, b, 0, h);

  // state tiles: acc_h[ip] holds h[p = 16 (pt0 + ip) + r16][n = 16 nt + 4q + r]
  f32x4 acc_h[TPW];
  {
    const int lane = Out::lane_opaque(), q = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int ip = 0; ip < TPW; ++ip) {
      if (a.h0) {
        const float4 v = ld4(a.h0 + sbase + (16 * (pt0 + ip) + r16) * N + 16 * nt + 4 * q);
        acc_h[ip] = f32x4{v.x, v.y, v.z, v.w};
      } else {
        acc_h[ip] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
  __syncthreads();   // chunk 0's prefix

  for (int64_t c = 0; c < a.Nc; ++c) {
    const int Lc = chunk_len(a, c);
    const int buf = (int)(c & 1);
    const bool next = c + 1 < a.Nc;   // uniform
    // ---- stage chunk c ----
    xs.store(s_xt);
    {
      const int lane = Out::lane_opaque(), q = lane >> 4, r16 = lane & 15;
#pragma unroll
      for (int ip = 0; ip < TPW; ++ip) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (bf16)acc_h[ip][r];
        st4b(s_h + (16 * (pt0 + ip) + r16) * HS + 16 * nt + 4 * q, v);
      }
    }
    out.c = c;
    out.Lc = Lc;
    out.prefetch();
    tile_decay_table<VAR, NTH, LMAX>(Lc, s_d[buf], s_cum[buf], s_w);
    state_weights<LMAX, NTH>(Lc, s_d[buf], s_cum[buf], s_ws);
    const float alpha = fast_exp(s_cum[buf][Lc - 1]);
    DeltaScan ds{};
    if (scan_thread && next) ds = chunk_scan_stage1(a, c + 1, hc, dtv, s_wsum);
    __syncthreads();
    if (scan_thread && next) chunk_scan_stage2(a, ds, s_wsum, s_d[buf ^ 1], s_cum[buf ^ 1]);

    // dt two chunks ahead (the last chunks re-read the last), ahead of the
    // state step's loads so that the next staging does not wait behind them
    if (scan_thread) dtv = chunk_dt_load(a, b, c + 2 < a.Nc ? c + 2 : a.Nc - 1, h);

    // ---- outputs of chunk c ----
    out.run(s_d[buf], s_cum[buf], s_w, s_xt, s_h);

    // ---- chunk summary state S_c, then h_c = fma(alpha, h_{c-1}, S_c) ----
    // the next chunk's x is issued right behind the state step's fragments
    // (the last chunk re-reads itself: the same loads on every path)
    {
      bf16x8 bt[LMAX / 32];
      state_bt_load<N, LMAX>(a, b, c, g, nt, Lc, bt);
      xs.load(a, b, next ? c + 1 : c, h);
      out.store_pending();
      f32x4 t[TPW];
      state_tiles<P, LMAX, TPW>(bt, pt0, Lc, s_xt, s_ws, t);
#pragma unroll
      for (int ip = 0; ip < TPW; ++ip)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc_h[ip][r] = __fmaf_rn(alpha, acc_h[ip][r], t[ip][r]);
    }
    __syncthreads();   // every wavefront is done with s_xt, s_h, s_w, s_ws and buffer buf
  }

  if (a.final_state) {
    const int lane = Out::lane_opaque(), q = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int ip = 0; ip < TPW; ++ip) {
      const f32x4 v = acc_h[ip];
      st4(a.final_state + sbase + (16 * (pt0 + ip) + r16) * N + 16 * nt + 4 * q,
          make_float4(v[0], v[1], v[2], v[3]));
    }
  }
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------
// Heads per chunk-state workgroup.  The heads of a compute unit run one after
// another whether they share a workgroup or not, so the unit with the most
// heads sets the time: with `per` heads per workgroup and the workgroups dealt
// round-robin over the 256 compute units, that is ceil(workgroups / 256) *
// per heads.  The smallest such load wins, and of equal loads the longest
// runs (B^T loaded once per run, each head's loads behind the previous head's
// products): on the 2.7B shape (16 chunks x 80 heads) 5 heads per workgroup,
// 256 workgroups, 32.5 -> 29 us against one head per workgroup.
inline void state_runs(int64_t bcg, int64_t hpg, int& per, int& splits) {
  constexpr int64_t kCUs = 256;
  int64_t best = -1;
  for (int64_t p = 1; p <= hpg; ++p) {
    const int64_t sp = (hpg + p - 1) / p;
    const int64_t load = (bcg * sp + kCUs - 1) / kCUs * p;
    if (best < 0 || load <= best) {
      best = load;
      per = (int)p;
      splits = (int)sp;
    }
  }
}

template <int P, int N>
hipError_t launch_phased(const ScanArgs& a, hipStream_t stream, hipEvent_t* ev) {
  hipError_t e;
  auto rec = [&](int k) -> hipError_t { return ev ? hipEventRecord(ev[k], stream) : hipSuccess; };
  if ((e = rec(0)) != hipSuccess) return e;
  const int64_t units = a.Bt * a.Nc * a.H;
  if (phased_prepass(P, N, a.L)) {
    // C B^T and B^T of every (b, c, g), then the chunk states from B^T
    if ((e = launch_prepass<N>(a, stream)) != hipSuccess) return e;
    if ((e = rec(1)) != hipSuccess) return e;
    if constexpr (chain_variant(P, N)) {
      int per = 1, splits = 1;
      state_runs(a.Bt * a.Nc * a.G, a.H / a.G, per, splits);
      hipLaunchKernelGGL((k_chunk_state_bf16<P, N>), dim3((unsigned)(a.Bt * a.Nc * a.G * splits)),
                         dim3(kOutThreads), 0, stream, a, per, splits);
    }
  } else {
    if ((e = rec(1)) != hipSuccess) return e;
    hipLaunchKernelGGL((k_cb_and_chunk_state_bf16<P, N>), dim3((unsigned)units), dim3(kThreads), 0,
                       stream, a, cb_tiles(a));
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = rec(2)) != hipSuccess) return e;
  if ((e = launch_state_pass(a, P, N, stream, true)) != hipSuccess) return e;
  if ((e = rec(3)) != hipSuccess) return e;
  if (a.states_only) return rec(4);   // entering states and C B^T only
  if (a.variant != kDecayF32) {
    // ablation variants: the 2.7B / 1.3B head shape at chunks up to 256 only
    if constexpr (ablation_shape(P, N)) {
      if (a.L > 256) return hipErrorInvalidValue;
      if (a.variant == kDecayBf16)
        hipLaunchKernelGGL((k_chunk_out_bf16<P, N, 256, kDecayBf16>), dim3((unsigned)units),
                           dim3(512), 0, stream, a);
      else
        hipLaunchKernelGGL((k_chunk_out_bf16<P, N, 256, kMaskLoaded>), dim3((unsigned)units),
                           dim3(512), 0, stream, a);
    } else {
      return hipErrorInvalidValue;
    }
  } else if (a.L <= 256) {
    hipLaunchKernelGGL((k_chunk_out_bf16<P, N, 256, kDecayF32>), dim3((unsigned)units),
                       dim3(512), 0, stream, a);
  } else {
    if constexpr (P <= 64) {
      hipLaunchKernelGGL((k_chunk_out_bf16<P, N, 512, kDecayF32>), dim3((unsigned)units),
                         dim3(1024), 0, stream, a);
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
    if ((e = launch_prepass<N>(a, stream)) != hipSuccess) return e;
    if ((e = rec(1)) != hipSuccess) return e;
    if ((e = rec(2)) != hipSuccess) return e;
    if ((e = rec(3)) != hipSuccess) return e;
    const unsigned chains = (unsigned)(a.Bt * a.H);
    if (a.variant != kDecayF32) {
      if constexpr (ablation_shape(P, N)) {
        if (a.L > 256) return hipErrorInvalidValue;
        if (a.variant == kDecayBf16)
          hipLaunchKernelGGL((k_chain_bf16<P, N, 256, kDecayBf16>), dim3(chains),
                             dim3(kOutThreads), 0, stream, a);
        else
          hipLaunchKernelGGL((k_chain_bf16<P, N, 256, kMaskLoaded>), dim3(chains),
                             dim3(kOutThreads), 0, stream, a);
      } else {
        return hipErrorInvalidValue;
      }
    } else if (a.L <= 128) {
      hipLaunchKernelGGL((k_chain_bf16<P, N, 128, kDecayF32>), dim3(chains), dim3(kOutThreads),
                         0, stream, a);
    } else {
      hipLaunchKernelGGL((k_chain_bf16<P, N, 256, kDecayF32>), dim3(chains), dim3(kOutThreads),
                         0, stream, a);
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
