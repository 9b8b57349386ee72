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

template <bool BF16_OUT>
__global__ __launch_bounds__(kThreads) void k_state_pass(float* ws_state, const float* ws_alpha,
                                                         bf16* ws_hb, const float* h0,
                                                         float* final_state, int64_t BH,
                                                         int64_t Nc, int PN, int keep_f32) {
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
  for (int64_t c0 = 0; c0 < Nc; c0 += kBatch) {
    const int n = (int)min<int64_t>(kBatch, Nc - c0);
    // every load of the batch is issued unconditionally (indices clamped in range)
    float4 s[kBatch];
    float al_c[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int64_t cc = min<int64_t>(c0 + k, Nc - 1);
      s[k] = st[cc * PN4];
      al_c[k] = al[cc];
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (k < n) {
        if constexpr (BF16_OUT) {
          bf16x4 v;
          v[0] = (bf16)hc.x; v[1] = (bf16)hc.y; v[2] = (bf16)hc.z; v[3] = (bf16)hc.w;
          hb[(c0 + k) * PN4] = v;
          if (keep_f32) st[(c0 + k) * PN4] = hc;   // this batch's S_c are already loaded
        } else {
          st[(c0 + k) * PN4] = hc;
        }
        const float a = al_c[k];
        hc.x = __fmaf_rn(a, hc.x, s[k].x);
        hc.y = __fmaf_rn(a, hc.y, s[k].y);
        hc.z = __fmaf_rn(a, hc.z, s[k].z);
        hc.w = __fmaf_rn(a, hc.w, s[k].w);
      }
    }
  }
  if (final_state) reinterpret_cast<float4*>(final_state + bh * PN)[e4] = hc;
}

}  // namespace
}  // namespace prefill

hipError_t launch_state_pass(const ScanArgs& a, int P, int N, hipStream_t stream, bool bf16_out) {
  const int PN = P * N;
  const int64_t threads = a.Bt * a.H * (PN / 4);
  const int64_t blocks = (threads + prefill::kThreads - 1) / prefill::kThreads;
  if (bf16_out) {
    hipLaunchKernelGGL(prefill::k_state_pass<true>, dim3((unsigned)blocks), dim3(prefill::kThreads),
                       0, stream, a.ws_state, (const float*)a.ws_alpha,
                       reinterpret_cast<bf16*>(a.ws_hb), a.h0, a.final_state, a.Bt * a.H, a.Nc,
                       PN, a.keep_f32_states);
  } else {
    hipLaunchKernelGGL(prefill::k_state_pass<false>, dim3((unsigned)blocks),
                       dim3(prefill::kThreads), 0, stream, a.ws_state, (const float*)a.ws_alpha,
                       nullptr, a.h0, a.final_state, a.Bt * a.H, a.Nc, PN, 0);
  }
  return hipGetLastError();
}

}  // namespace ssd
