// Internal interface between the C ABI (ssd_api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

// Arguments of the chunked scan, after validation.  Device pointers.
struct ScanArgs {
  const void* x;          // [Bt,T,H,P] io
  const float* dt;        // [Bt,T,H]
  const float* dt_bias;   // [H] or null
  const float* A;         // [H]
  const void* B;          // [Bt,T,G,N] io
  const void* C;          // [Bt,T,G,N] io
  const float* D;         // [H] or null
  const float* h0;        // [Bt,H,P,N] or null
  void* y;                // [Bt,T,H,P] io
  float* final_state;     // [Bt,H,P,N] or null
  float* ws_state;        // [Bt,H,Nc,P,N]: chunk summary states, then entering states
  float* ws_alpha;        // [Bt,H,Nc]: exp(total decay of the chunk)
  float* ws_cb;           // [Bt,Nc,G,L,L]: C B^T of each chunk (causal 16x16 tiles); bf16
                          // elements when cb_bf16
  void* ws_bt;            // [Bt,Nc,G,N,L] bf16: B of each chunk, transposed (token-contiguous)
  void* ws_hb;            // [Bt,H,Nc,P,N] bf16: entering states, rounded (bf16 phased schedule)
  int64_t Bt, T, H, G, L, Nc;
  int32_t softplus;
  float dt_min, dt_max;
  int32_t chain;          // 1: chain schedule (bfloat16 only), 0: phased
  int32_t states_only;    // 1: phases 0-2 only (C B^T, chunk and entering states; no y)
  int32_t keep_f32_states; // bf16 phased: the state pass also writes the float32 entering
                           // states over ws_state (the gradients read them)
  int32_t cb_bf16 = 0;     // ws_cb holds bfloat16 (the bfloat16 forward scan) instead of float32
  int32_t variant = 0;     // bf16 output path: 0 float32 decay and in-register mask; 1 decay
                           // factors rounded to bf16; 2 mask loaded from a stored table
};

struct StepArgs {
  float* state;           // [Bt,H,P,N] in/out
  const void* x;          // [Bt,H,P] io
  const float* dt;        // [Bt,H]
  const float* dt_bias;   // [H] or null
  const float* A;         // [H]
  const void* B;          // [Bt,G,N] io
  const void* C;          // [Bt,G,N] io
  const float* D;         // [H] or null
  void* y;                // [Bt,H,P] io
  int64_t Bt, H, G;
  int32_t P, N;
  int32_t softplus;
  float dt_min, dt_max;
};

struct ConvArgs {
  const void* x;          // [Bt,T,D] io (the step: x_t [Bt,D])
  const float* w;         // [D,K]
  const float* bias;      // [D] or null
  const void* state_in;   // [Bt,D,K-1] io or null (the step: the in/out window)
  void* y;                // [Bt,T,D] io (the step: y_t [Bt,D])
  void* state_out;        // [Bt,D,K-1] io or null (the step: the in/out window)
  int64_t Bt, T, D;
  int32_t K;
  int32_t silu;
};

// Arguments of the kernels of the scan's backward pass (ssd_backward.hip).
// Device pointers.
struct BwdArgs {
  // inputs of the forward scan and the cotangents
  const void* x;            // [Bt,T,H,P] io
  const float* dt;          // [Bt,T,H]
  const float* dt_bias;     // [H] or null
  const float* A;           // [H]
  const void* B;            // [Bt,T,G,N] io
  const void* C;            // [Bt,T,G,N] io
  const float* D;           // [H] or null
  const float* h0;          // [Bt,H,P,N] or null
  const void* dy;           // [Bt,T,H,P] io
  const float* dfinal;      // [Bt,H,P,N] or null
  // Delta, its chunk-local prefix, and the operands and results of the reversed scan R1
  // (in the io type: R1 runs the scan kernels of that type)
  float* wd;                // [Bt,T,H] Delta
  double* cum;              // [Bt,T,H] sum of Delta A from the chunk start to the token (inclusive)
  float* rscale;            // [2,Bt,T,H] row scales of the dC / dB inter-chunk products:
                            // e^{cum_t} and Delta_t e^{cum_last - cum_t}
  float* dtr1;              // [Bt,T+pad,H] Delta' of R1: d_t at reversed position pad+T-t
  void* r1_x;               // [Bt,T+pad,H,P] io  reversed dy_t / Delta_{t+1}
  void* r1_b;               // [Bt,T+pad,G,N] io  reversed C
  void* r1_c;               // [Bt,T+pad,G,N] io  reversed B
  float* r1_h0;             // [Bt,H,P,N]     dfinal + dy_{T-1} (x) C_{T-1}
  const void* r1_y;         // [Bt,T+pad,H,P] io  sum_n G B (reversed positions)
  const float* r1_final;    // [Bt,H,P,N]     dL/dh_{-1} / abar_0
  // entering states (float32) and C B^T tiles the two scans leave in their workspaces
  const float* fwd_state;   // [Bt,H,Nc,P,N] state entering forward chunk c (H_c)
  const float* fwd_cb;      // [Bt,Nc,G,L,L] C B^T of each forward chunk
  const float* r1_state;    // [Bt,H,Nc,P,N] state entering reversed chunk c' (G at (Nc-c')L)
  // intermediate results
  float* mix;               // [Bt,Nc,G,HS,LP,LP] per head split: sum_h (dy x^T) o decay o Delta_j
  float* qrow;              // [Bt,Nc,H,NB,NB,2,64] row sums of the decay-gradient products
  float* qcol;              // [Bt,Nc,H,NB,NB,2,64] column sums of the same
  float* uv;                // [2][NS][Bt,H,T] per-token state terms of the decay gradient
  float* dbc_part;          // [2][HSD][Bt,T,G,N] head-split parts of dC, dB (HSD > 1)
  float* ddin;              // [Bt,H,T]  x_t . (sum_n G B)
  float* dDp;               // [Bt,H,T]  dy_t . x_t
  float* part;              // [4][Bt,Nc,H] parts of dA, ddt_bias, dD; <Ghat_c, H_c>
  // gradients
  float* dx;                // [Bt,T,H,P]
  float* ddt;               // [Bt,T,H]
  float* dA;                // [H]
  float* dB;                // [Bt,T,G,N]
  float* dC;                // [Bt,T,G,N]
  float* dD;                // [H] or null
  float* ddt_bias_out;      // [H] or null
  float* dh0;               // [Bt,H,P,N] or null
  int64_t Bt, T, H, G;
  int64_t L, Nc;            // chunk and chunks of the forward partition
  int64_t pad;              // leading empty positions of the reversed scan R1 (Nc L - T)
  int32_t P, N;
  int32_t NB, LP;           // 64-token blocks per chunk, and NB * 64
  int32_t HS, hpw;          // head splits of the mix kernel and heads per split
  int32_t HSD, hpwd;        // head splits of the dC/dB kernel and heads per split
  int32_t NS;               // column splits of N in the dC/dB kernel
  int32_t softplus;
  float dt_min, dt_max;
};

// Compiled shape variants.
bool scan_shape_supported(int64_t P, int64_t N, int64_t L, bool bf16);

// Head/state sizes with compiled ablation variants of the bfloat16 output path
// (ssd_chunk_scan_ablation), at chunks up to 256.
constexpr bool ablation_shape(int64_t P, int64_t N) { return P == 64 && N == 128; }

// Head/state sizes with a compiled chain kernel (bfloat16 io, L <= 256).
constexpr bool chain_variant(int64_t P, int64_t N) {
  return (P == 32 || P == 64) && (N == 64 || N == 128);
}
// The phased bfloat16 schedule of the chain shapes at chunks up to 256 also
// starts with the C B^T / B^T pre-pass and forms its chunk states from B^T.
constexpr bool phased_prepass(int64_t P, int64_t N, int64_t L) {
  return chain_variant(P, N) && L <= 256;
}

// The chain schedule runs one workgroup per (batch, head) for the whole
// sequence; it is chosen once batch x heads alone fill the GPU's 256 compute
// units (two workgroups per unit at most).  Both schedules give bit-identical
// results, so the choice never changes an answer.
constexpr int64_t kChainMinChains = 256;
bool scan_uses_chain(int64_t batch, int64_t nheads, int64_t P, int64_t N, int64_t L, bool bf16);
bool step_shape_supported(int64_t P, int64_t N);

// Launch the whole scan (Bt*T > 0) on `stream`.  `events` (may be null) gets
// one record before each of the 4 phases and one after the last.
hipError_t launch_scan_f32(const ScanArgs& a, int P, int N, hipStream_t stream, hipEvent_t* events);
hipError_t launch_scan_bf16(const ScanArgs& a, int P, int N, hipStream_t stream, hipEvent_t* events);

// Inter-chunk recurrence over the workspace states (both io types).  The
// entering states go to ws_state in float32, or, when bf16_out, to ws_hb
// rounded to bfloat16 (the only form the bfloat16 output kernel uses).
hipError_t launch_state_pass(const ScanArgs& a, int P, int N, hipStream_t stream, bool bf16_out);

hipError_t launch_step_f32(const StepArgs& a, hipStream_t stream);
hipError_t launch_step_bf16(const StepArgs& a, hipStream_t stream);

// Depthwise causal convolution: the sequence kernel (step == false) or the
// one-token kernel (step == true, window in state_out, updated in place).
bool conv_width_supported(int64_t K);
bool conv_shape_supported(int64_t Bt, int64_t T, int64_t D);
hipError_t launch_conv(const ConvArgs& a, bool io_bf16, bool step, hipStream_t stream);

// Backward pass pieces: phase 0 prepares Delta, its chunk-local prefix and the
// reversed operands and initial state of R1; phase 1 (after the forward state
// scan and R1) forms every gradient.
hipError_t launch_backward_phase(const BwdArgs& a, bool io_bf16, int phase, hipStream_t stream);
hipError_t launch_backward_zero_heads(float* dA, float* ddt_bias, float* dD, int64_t H,
                                      hipStream_t stream);

// dst[i] = src ? src[i] : 0 for i < n (float4 granularity; n % 4 == 0).
hipError_t launch_copy_or_zero(float* dst, const float* src, int64_t n, hipStream_t stream);

}  // namespace ssd
