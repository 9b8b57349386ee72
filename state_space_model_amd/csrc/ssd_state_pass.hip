// Inter-chunk state recurrence of the chunked SSD scan (both io types).
//
// Source: "Compiler-First State Space Duality and Portable O(1)
// Autoregressive Caching", Background: across chunks, a sequential
// recurrence over chunk-level summary states whose FLOP count is small next
// to the intra-chunk matrix products.
//
//   h_c = alpha_c h_{c-1} + S_c,   h_{-1} = initial state (or 0)
//
// computed as one fused multiply-add per element (the same operation the
// bfloat16 chain kernel applies to its on-chip state).
//
// Element-wise over the P x N state of every (batch, head), sequential over
// chunks.  The workspace holds S_c on entry; the state entering chunk c,
// h_{c-1}, is written over it in float32 or, for the bfloat16 output kernel
// (which only uses it rounded to bfloat16), to a separate bf16 region (and,
// when asked, in float32 over it too); the last state goes to final_state.  One lane owns one
// float4 of a state and keeps it in registers across all chunks; the chunk
// states it reads are issued in batches of 16 so their latency overlaps.
#include "ssd_prefill_common.h"

namespace ssd {
namespace prefill {
namespace {

constexpr int kBatch = 16;

// Every memory operation of a batch is issued on every path: the counter that
// tracks loads and stores together is then counted exactly, and the wait for
// chunk k's state waits for that load alone.  (With the stores of the last,
// partial batch and of the optional float32 copy under runtime conditions,
// the compiler counted them as absent and each step waited for the stores
// before it as well.)  Whole batches first, the last Nc % 16 chunks one at
// a time.
template <bool BF16_OUT, bool KEEP_F32>
__global__ __launch_bounds__(kThreads) void k_state_pass(float* ws_state, const float* ws_alpha,
                                                         bf16* ws_hb, const float* h0,
                                                         float* final_state, int64_t BH,
                                                         int64_t Nc, int PN) {
  const int PN4 = PN / 4;
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= BH * PN4) return;
  const int64_t bh = gid / PN4;
  const int e4 = (int)(gid % PN4);
  float4* st = reinterpret_cast<float4*>(ws_state + bh * Nc * PN) + e4;
  bf16x4* hb = nullptr;
  if constexpr (BF16_OUT) hb = reinterpret_cast<bf16x4*>(ws_hb + bh * Nc * PN) + e4;
  const float* al = ws_alpha + bh * Nc;
  float4 hc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (h0) hc = reinterpret_cast<const float4*>(h0 + bh * PN)[e4];
  // h_{c-1} to chunk c's slots, then h_c = fma(alpha_c, h_{c-1}, S_c)
  auto step = [&](int64_t c, float4 sc, float a) {
    if constexpr (BF16_OUT) {
      bf16x4 v;
      v[0] = (bf16)hc.x; v[1] = (bf16)hc.y; v[2] = (bf16)hc.z; v[3] = (bf16)hc.w;
      hb[c * PN4] = v;
      if constexpr (KEEP_F32) st[c * PN4] = hc;   // S_c is already loaded
    } else {
      st[c * PN4] = hc;
    }
    hc.x = __fmaf_rn(a, hc.x, sc.x);
    hc.y = __fmaf_rn(a, hc.y, sc.y);
    hc.z = __fmaf_rn(a, hc.z, sc.z);
    hc.w = __fmaf_rn(a, hc.w, sc.w);
  };
  int64_t c0 = 0;
  for (; c0 + kBatch <= Nc; c0 += kBatch) {
    float4 s[kBatch];
    float al_c[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      s[k] = st[(c0 + k) * PN4];
      al_c[k] = al[c0 + k];
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) step(c0 + k, s[k], al_c[k]);
  }
  for (; c0 < Nc; ++c0) step(c0, st[c0 * PN4], al[c0]);
  if (final_state) reinterpret_cast<float4*>(final_state + bh * PN)[e4] = hc;
}

}  // namespace
}  // namespace prefill

hipError_t launch_state_pass(const ScanArgs& a, int P, int N, hipStream_t stream, bool bf16_out) {
  const int PN = P * N;
  const int64_t threads = a.Bt * a.H * (PN / 4);
  const int64_t blocks = (threads + prefill::kThreads - 1) / prefill::kThreads;
  const dim3 grid((unsigned)blocks), block(prefill::kThreads);
  const float* alpha = a.ws_alpha;
  bf16* hb = reinterpret_cast<bf16*>(a.ws_hb);
  if (bf16_out && a.keep_f32_states) {
    hipLaunchKernelGGL((prefill::k_state_pass<true, true>), grid, block, 0, stream, a.ws_state,
                       alpha, hb, a.h0, a.final_state, a.Bt * a.H, a.Nc, PN);
  } else if (bf16_out) {
    hipLaunchKernelGGL((prefill::k_state_pass<true, false>), grid, block, 0, stream, a.ws_state,
                       alpha, hb, a.h0, a.final_state, a.Bt * a.H, a.Nc, PN);
  } else {
    hipLaunchKernelGGL((prefill::k_state_pass<false, false>), grid, block, 0, stream, a.ws_state,
                       alpha, nullptr, a.h0, a.final_state, a.Bt * a.H, a.Nc, PN);
  }
  return hipGetLastError();
}

}  // namespace ssd
