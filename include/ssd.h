/*
 * ssd.h -- C ABI of the MI355X (gfx950) Mamba-2 SSD library (libssd.so).
 *
 * Operations, following "Compiler-First State Space Duality and Portable
 * O(1) Autoregressive Caching" (arXiv 2603.09555):
 *
 *   ssd_chunk_scan  the chunked state-space-duality scan over a whole
 *                   sequence (prefill): Background, Eq. 3 and the inter-chunk
 *                   recurrence described after it; SSD properties "diagonal
 *                   state matrix", "chunked recurrence", "static control flow".
 *   ssd_step        one token of the recurrence from a fixed-size state held
 *                   on the device (decode): the O(1) cache section.
 *   ssd_conv1d, ssd_conv1d_step
 *                   the depthwise causal convolution that precedes the scan
 *                   in a Mamba-2 block, over a sequence and for one token
 *                   from its cached window (O(1) cache section; Setup: k = 4).
 *   ssd_chunk_scan_backward
 *                   the gradients of ssd_chunk_scan with respect to all of
 *                   its inputs (the backward pass of a training step).
 *
 * Both compute, for every batch row b and head h (g = h / (H/G) is the B/C
 * group of head h), the selective diagonal SSM
 *
 *   d_t      = clip(softplus(dt[b,t,h] + dt_bias[h]), dt_min, dt_max)
 *              (softplus skipped when dt_softplus == 0; dt_bias NULL -> 0)
 *   h_t[p,n] = exp(d_t * A[h]) * h_{t-1}[p,n] + d_t * x[b,t,h,p] * B[b,t,g,n]
 *   y[b,t,h,p] = sum_n C[b,t,g,n] * h_t[p,n] + D[h] * x[b,t,h,p]
 *
 * i.e. Abar = exp(Delta*A), Bbar = Delta*B (Background, Eq. 2; the page names
 * zero-order hold but its equation is lost, and this is the form whose
 * unrolled kernel is the decay-only lower-triangular matrix of Eq. 3).
 * A[h] is the (negative) decay itself, not its logarithm: a caller holding
 * log-space decay parameters (Implementation, precision management) passes
 * -exp(A_log) computed in float32.
 *
 * Conventions shared by every call
 *  - Pointers are DEVICE pointers (hipMalloc'd or equivalent) except the
 *    descriptor, which is a host pointer read during the call only.
 *  - Tensors are dense, contiguous, row-major, in the layouts listed per call.
 *    x, B, C, y and every state (and the workspace) must be 16-byte aligned;
 *    dt, dt_bias, A, D and the convolution weights and bias 4-byte aligned.
 *  - x, B, C and y share one dtype (desc->io_dtype: SSD_F32 or SSD_BF16);
 *    dt, dt_bias, A, D and every SSM state are float32 (the convolution
 *    window holds past inputs and keeps io_dtype).  All arithmetic inside is
 *    float32 (decay, exponentials, states, accumulation); bfloat16 appears
 *    only as matrix-core operands and at the output store (round to nearest
 *    even).
 *  - The caller owns every buffer, including the workspace.  The library never
 *    allocates, frees or synchronises; calls are asynchronous on `stream`
 *    (0 = the null stream) and results are valid once the stream has reached
 *    them.  The library keeps no mutable global state other than the
 *    per-device address of ssd_chunk_scan_noalloc's static scratch.
 *  - Errors: arguments are validated before anything is launched; on any error
 *    other than SSD_ERR_HIP nothing has been written.  SSD_ERR_HIP means a
 *    launch failed (hipGetLastError); outputs are then undefined.  No C++
 *    exception crosses this interface.
 *  - Shapes supported by the compiled gfx950 kernels: headdim P in
 *    {16, 32, 64, 128}, dstate N in {16, 32, 64, 128} (N = 16 with float32
 *    io only), chunk L a multiple of 32 in [32, 512] with P*L <= 32768
 *    (ssd_step: the same P, and N for either dtype).  Other positive shapes
 *    return SSD_ERR_UNSUPPORTED.  seqlen need not be a multiple of the
 *    chunk: the last chunk may be shorter.  batch == 0 or seqlen == 0 is valid.
 */
#ifndef SSD_MI355X_H
#define SSD_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 5

typedef enum {
  SSD_OK = 0,
  SSD_ERR_INVALID_ARG = 1, /* NULL required pointer, NaN/inverted dt limits, aliasing */
  SSD_ERR_SHAPE = 2,       /* non-positive size, heads not a multiple of groups */
  SSD_ERR_DTYPE = 3,       /* io_dtype not one of ssd_dtype */
  SSD_ERR_ALIGNMENT = 4,   /* a device pointer below its required alignment */
  SSD_ERR_UNSUPPORTED = 5, /* valid shape without a compiled gfx950 variant */
  SSD_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than the query returned */
  SSD_ERR_HIP = 7          /* a HIP launch failed */
} ssd_status;

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

/* Problem description of a chunked scan (prefill). */
typedef struct {
  int64_t batch;     /* Bt >= 0 */
  int64_t seqlen;    /* T >= 0 */
  int64_t nheads;    /* H >= 1, a multiple of ngroups */
  int64_t headdim;   /* P */
  int64_t dstate;    /* N */
  int64_t ngroups;   /* G >= 1: heads h share B/C group h / (H/G) */
  int64_t chunk;     /* L: tokens per chunk of the dual form */
  int32_t io_dtype;  /* ssd_dtype of x, B, C and y */
  int32_t dt_softplus; /* 1: d = softplus(dt + dt_bias) before clipping; 0: d = dt + dt_bias */
  float dt_min, dt_max; /* clip limits of d, dt_min <= dt_max (e.g. 1e-4 and 0.5) */
} ssd_scan_desc;

/* Problem description of one decode step. */
typedef struct {
  int64_t batch, nheads, headdim, dstate, ngroups;
  int32_t io_dtype;
  int32_t dt_softplus;
  float dt_min, dt_max;
} ssd_step_desc;

/*
 * Workspace bytes ssd_chunk_scan needs for `desc` (0 if desc is invalid).
 * Both schedules (see ssd_chunk_scan_schedule) hold the L x L matrix C B^T
 * of every (batch, chunk, group), in the io dtype: s*Bt*ceil(T/L)*G*L*L
 * bytes with s = 4 (float32) or 2 (bfloat16).  The
 * phased schedule adds one float32 P x N state and one float32 decay per
 * (batch, head, chunk): 4*Bt*ceil(T/L)*H*(P*N+1) bytes, and with bfloat16 io
 * a bfloat16 copy of the entering states: 2*Bt*ceil(T/L)*H*P*N bytes; the
 * chain schedule adds a bfloat16 transposed copy of B per (batch, chunk,
 * group): 2*Bt*ceil(T/L)*G*N*L bytes.  Each region is rounded up to 256
 * bytes.
 */
size_t ssd_chunk_scan_workspace_bytes(const ssd_scan_desc* desc);

/*
 * Which schedule ssd_chunk_scan runs for `desc`; a negative ssd_status if the
 * descriptor is invalid.  Both compute bit-identical results (the same
 * matrix-core instructions on the same operands in the same order for every
 * element), so the choice, which depends on the batch size, never changes an
 * answer; the pages' batch-size invariance holds across it.
 *   SSD_SCHEDULE_PHASED  one workgroup per (batch, chunk, head) and phase:
 *                        C B^T, chunk states, state pass, outputs
 *   SSD_SCHEDULE_CHAIN   bfloat16 io, P in {32, 64}, N in {64, 128}, L <= 256
 *                        and batch*heads >= 256: a C B^T / B^T pre-pass, then
 *                        one workgroup per (batch, head) walks the chunks in
 *                        order with its state on chip
 */
#define SSD_SCHEDULE_PHASED 0
#define SSD_SCHEDULE_CHAIN 1
int32_t ssd_chunk_scan_schedule(const ssd_scan_desc* desc);

/*
 * Chunked SSD scan over a whole sequence (prefill).
 *
 * Source: "Compiler-First State Space Duality and Portable O(1) Autoregressive
 * Caching", Background (Eq. 3: within a chunk of L tokens, y = (L o C B^T) X
 * with L the lower-triangular matrix of exponentiated segment sums of A*Delta;
 * across chunks, a sequential recurrence over chunk summary states) and the
 * O(1) cache section (prefill hands its final state to the decode cache).
 *
 *   x   [Bt,T,H,P] io_dtype     dt  [Bt,T,H] f32 (pre-activation)
 *   A   [H] f32 (A < 0)         dt_bias [H] f32 or NULL
 *   B,C [Bt,T,G,N] io_dtype     D   [H] f32 or NULL (no skip term)
 *   initial_state [Bt,H,P,N] f32 or NULL (zeros)
 *   y   [Bt,T,H,P] io_dtype (written)
 *   final_state [Bt,H,P,N] f32 (written) or NULL (not returned)
 *   workspace: device buffer of at least ssd_chunk_scan_workspace_bytes(desc)
 *
 * y and final_state must not overlap any input or each other.  The result does
 * not depend on the run (no atomics in any reduction): repeated calls on the
 * same inputs are bitwise identical.
 */
ssd_status ssd_chunk_scan(const ssd_scan_desc* desc, const void* x, const float* dt,
                          const float* dt_bias, const float* A, const void* B, const void* C,
                          const float* D, const float* initial_state, void* y,
                          float* final_state, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * Gradients of ssd_chunk_scan (same descriptor and inputs) for the loss
 * L = sum(dy * y) + sum(dfinal_state * final_state), with respect to every
 * input: the backward pass of a training step over the recurrence of
 * "Compiler-First State Space Duality and Portable O(1) Autoregressive
 * Caching", Background, Eq. 2-3.
 *
 * The adjoint state G_t = dL/dh_t obeys the same recurrence backwards in
 * time (G_t = dy_t (x) C_t + abar_{t+1} G_{t+1}).  The library recomputes the
 * forward chunk states and C B^T, runs the scan itself over reversed time
 * with B and C exchanged (G_t B_t for dx, and the adjoint at chunk
 * boundaries), both with the scan kernels of the io type (float32 states),
 * and forms dB, dC and the Delta gradient chunk by chunk with float32
 * matrix-core products: per group, M = sum over its heads of (dy x^T) o
 * decay o Delta is built once, dC = M B + dy H, dB = M^T C + x Ghat, and
 * dL/d(Delta A) comes from sums inside each chunk only (no sum over the
 * sequence cancels).  With bfloat16 io the reversed scan's input dy / Delta
 * and its output G B are rounded to bfloat16, as in the forward scan.  No
 * atomics: results are deterministic.
 *
 *   inputs as ssd_chunk_scan; dy [Bt,T,H,P] io_dtype;
 *   dfinal_state [Bt,H,P,N] f32 or NULL (zero)
 *   gradients, all float32 (written): dx [Bt,T,H,P]; ddt [Bt,T,H] with
 *   respect to the pre-activation dt (zero where Delta is clipped); dA [H];
 *   dB, dC [Bt,T,G,N]; dD [H] or NULL; ddt_bias [H] or NULL;
 *   dinitial_state [Bt,H,P,N] or NULL (not returned)
 *   workspace: at least ssd_chunk_scan_backward_workspace_bytes(desc)
 *
 * Shapes: those of ssd_chunk_scan with chunk <= 256 and batch * seqlen *
 * nheads <= INT32_MAX; other valid shapes return SSD_ERR_UNSUPPORTED (and a
 * workspace size of 0).  Gradients may not overlap any input, the workspace
 * or each other.  batch == 0 writes zeros to dA, dD and ddt_bias; seqlen == 0
 * also copies dfinal_state (or zeros) to dinitial_state.
 */
size_t ssd_chunk_scan_backward_workspace_bytes(const ssd_scan_desc* desc);
ssd_status ssd_chunk_scan_backward(const ssd_scan_desc* desc, const void* x, const float* dt,
                                   const float* dt_bias, const float* A, const void* B,
                                   const void* C, const float* D, const float* initial_state,
                                   const void* dy, const float* dfinal_state, float* dx,
                                   float* ddt, float* dA, float* dB, float* dC, float* dD,
                                   float* ddt_bias, float* dinitial_state, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * ssd_chunk_scan with timing instrumentation: when `phase_events` is not NULL
 * it must hold `n_events` created HIP events; event k is recorded on `stream`
 * before phase k and event n_phases after the last one (n_phases =
 * SSD_SCAN_PHASES).  Used by the benchmark to time each kernel of the scan on
 * the stream it runs on.  n_events < SSD_SCAN_PHASES + 1, or a NULL event among
 * the first SSD_SCAN_PHASES + 1, is SSD_ERR_INVALID_ARG.
 * Phases: 0 C B^T per chunk, 1 chunk states, 2 state passing, 3 chunk outputs
 * (a phase may be empty on some paths: its two events then coincide).  On
 * the chain schedule phase 0 is the C B^T / B^T pre-pass, phases 1 and 2 are
 * empty and phase 3 is the chain kernel (states, recurrence and outputs).
 */
#define SSD_SCAN_PHASES 4
ssd_status ssd_chunk_scan_timed(const ssd_scan_desc* desc, const void* x, const float* dt,
                                const float* dt_bias, const float* A, const void* B,
                                const void* C, const float* D, const float* initial_state,
                                void* y, float* final_state, void* workspace,
                                size_t workspace_bytes, hipStream_t stream,
                                hipEvent_t* phase_events, int n_events);

/*
 * ssd_chunk_scan with a variant of its output path, for the two ablations of
 * "Compiler-First State Space Duality and Portable O(1) Autoregressive
 * Caching", Implementation choices:
 *
 *   SSD_VARIANT_BF16_DECAY   every decay factor of the output path (the
 *                            exponentials of segment sums of A*Delta that
 *                            weight C B^T, and those of the inter-chunk term)
 *                            rounded to bfloat16 before use, instead of kept
 *                            in float32 ("precision management": the decay
 *                            held in bfloat16 costs accuracy)
 *   SSD_VARIANT_LOADED_MASK  the causal mask of the diagonal tiles read from a
 *                            stored lower-triangular bit table in device
 *                            memory instead of formed by an index comparison
 *                            in registers ("static masking": where the mask
 *                            lives changes the speed, not the bits); bfloat16
 *                            io only; the output is bitwise that of
 *                            ssd_chunk_scan
 *   SSD_VARIANT_DEFAULT      ssd_chunk_scan itself
 *
 * Arguments, layouts, ownership and errors as ssd_chunk_scan.  Supported for
 * P = 64, N = 128 and chunk <= 256 (the 130M, 2.7B and 1.3B head shapes);
 * other shapes return SSD_ERR_UNSUPPORTED, an unknown variant
 * SSD_ERR_INVALID_ARG.  The chunk states and the recurrence are those of
 * ssd_chunk_scan in every variant.
 */
#define SSD_VARIANT_DEFAULT 0
#define SSD_VARIANT_BF16_DECAY 1
#define SSD_VARIANT_LOADED_MASK 2
ssd_status ssd_chunk_scan_ablation(const ssd_scan_desc* desc, int32_t variant, const void* x,
                                   const float* dt, const float* dt_bias, const float* A,
                                   const void* B, const void* C, const float* D,
                                   const float* initial_state, void* y, float* final_state,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * ssd_chunk_scan without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  It calls no allocating routine: its
 * workspace is a static device array of SSD_NOALLOC_MAX_WORKSPACE bytes
 * that the library holds on every GPU it runs on, until the process ends.
 *
 * Arguments, layouts, results and errors as ssd_chunk_scan, less the
 * workspace.  A problem whose ssd_chunk_scan_workspace_bytes exceeds
 * SSD_NOALLOC_MAX_WORKSPACE returns SSD_ERR_WORKSPACE before anything is
 * launched (96 MiB holds the 130M- and 2.7B-shaped 4096-token layers and
 * the 8 x 16384-token batch of 64 heads; larger problems must use
 * ssd_chunk_scan with a workspace of their own).  `stream`
 * must belong to the current device (0: the current device's null stream),
 * else SSD_ERR_INVALID_ARG.  The first call on a device looks up the array's
 * address on that device (SSD_ERR_HIP if that fails).
 *
 * Every call on one GPU uses that GPU's one array, and nothing in it needs
 * to start at zero: calls on one GPU that may overlap in time (on different
 * streams, or from several host threads without ordering) race on it and
 * give undefined results; calls ordered on one stream are safe.
 */
#define SSD_NOALLOC_MAX_WORKSPACE (96u << 20)
ssd_status ssd_chunk_scan_noalloc(const ssd_scan_desc* desc, const void* x, const float* dt,
                                  const float* dt_bias, const float* A, const void* B,
                                  const void* C, const float* D, const float* initial_state,
                                  void* y, float* final_state, hipStream_t stream);

/*
 * One decode step of the recurrence, the state updated in place.
 *
 * Source: "Compiler-First State Space Duality and Portable O(1) Autoregressive
 * Caching", O(1) cache section: the fixed-size state (B,H,P,N) summarises the
 * prefix, and the next token needs one recurrence step h_t = Abar h_{t-1} +
 * Bbar x_t, O(1) in the prefix length; Results: each decode step reads and
 * writes the same state whatever the prefix length.
 *
 *   state [Bt,H,P,N] f32, read and overwritten with the new state
 *   x_t   [Bt,H,P] io_dtype        dt_t [Bt,H] f32 (pre-activation)
 *   A [H] f32, dt_bias [H] f32 or NULL, D [H] f32 or NULL
 *   B_t, C_t [Bt,G,N] io_dtype
 *   y_t   [Bt,H,P] io_dtype (written; must not overlap the state or inputs)
 *
 * Each state element is read once and written once.
 */
ssd_status ssd_step(const ssd_step_desc* desc, float* state, const void* x_t, const float* dt_t,
                    const float* dt_bias, const float* A, const void* B_t, const void* C_t,
                    const float* D, void* y_t, hipStream_t stream);

/* Problem description of a depthwise causal convolution (prefill or step). */
typedef struct {
  int64_t batch;     /* Bt >= 0 */
  int64_t seqlen;    /* T >= 0 (ssd_conv1d); not used by ssd_conv1d_step */
  int64_t channels;  /* D >= 1 */
  int64_t width;     /* k: taps per channel, the current input and k-1 cached ones */
  int32_t io_dtype;  /* ssd_dtype of x, y and the cached window */
  int32_t silu;      /* 1: y = z * logistic(z) of the convolution z; 0: y = z */
} ssd_conv_desc;

/*
 * Depthwise causal convolution over a sequence, carrying the window of the
 * k-1 previous inputs in and out.
 *
 * Source: "Compiler-First State Space Duality and Portable O(1) Autoregressive
 * Caching", O(1) cache section (each channel is convolved over a sliding
 * window of its k-1 previous inputs, cached with shape (B, D_conv, k-1);
 * prefill initialises that cache) and Setup (kernel size k = 4).  Per batch
 * row b and channel c, with xp = (state_in[b][c][0..k-2], x[b][0..T-1][c]):
 *
 *   z[t] = bias[c] + sum_{i<k} w[c][i] * xp[t+i]     (w[c][k-1]: current input)
 *   y[b][t][c] = silu ? z[t] * logistic(z[t]) : z[t]
 *   state_out[b][c][j] = xp[T+j], j < k-1             (the last k-1 inputs)
 *
 *   x     [Bt,T,D] io_dtype       w    [D,k] f32      bias [D] f32 or NULL
 *   state_in  [Bt,D,k-1] io_dtype, oldest input first, or NULL (zeros)
 *   y     [Bt,T,D] io_dtype (written)
 *   state_out [Bt,D,k-1] io_dtype (written) or NULL; it may be state_in
 *             itself (updated in place) but may not overlap it otherwise.
 *
 * The sum is float32 fused multiply-adds in the order i = 0..k-1 starting
 * from the bias, the same in ssd_conv1d_step, so a sequence split anywhere
 * (each part seeded with the previous part's state_out) or run token by
 * token gives bitwise the same outputs.  The window is kept in io_dtype: it
 * holds past inputs, which that type represents exactly.  Supported: k in
 * {2, 3, 4}; any D (a multiple of 4 takes the vector path, 4 channels per
 * lane); batch <= 65535 and T <= 2097120 (grid limits).
 * y may not overlap any input or state.
 */
ssd_status ssd_conv1d(const ssd_conv_desc* desc, const void* x, const float* w,
                      const float* bias, const void* state_in, void* y, void* state_out,
                      hipStream_t stream);

/*
 * One token of the depthwise causal convolution from its cached window, the
 * window updated in place (O(1) cache section: the decode body updates the
 * convolution window, then runs one recurrence step).
 *
 *   state [Bt,D,k-1] io_dtype, read and overwritten: the oldest input drops
 *         out and x_t enters as the newest
 *   x_t   [Bt,D] io_dtype         w [D,k] f32      bias [D] f32 or NULL
 *   y_t   [Bt,D] io_dtype (written; must not overlap the state or inputs)
 *
 * y_t[b][c] = act(bias[c] + sum_{i<k-1} w[c][i] * state[b][c][i] + w[c][k-1] * x_t[b][c]),
 * bitwise equal to ssd_conv1d over the one token.  desc->seqlen is not read.
 */
ssd_status ssd_conv1d_step(const ssd_conv_desc* desc, void* state, const void* x_t,
                           const float* w, const float* bias, void* y_t, hipStream_t stream);

/* Static description of a status code (never NULL). */
const char* ssd_status_string(ssd_status status);

/* SSD_ABI_VERSION of the built library. */
int32_t ssd_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSD_MI355X_H */
