/*
 * ssmscan.h -- C ABI of libssmscan, the selective-SSM (Mamba-1) scan on AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (pages: "Mamba и State Space Models", nareshka.ru, sections
 * "Ключевая инновация: input-dependent parameters" and "Selective Scan (core
 * algorithm)"; "State Space Models: Mamba и альтернатива Transformer",
 * johe.ru, MambaBlock "_scan" code for the D skip; "Модуль 8. Альтернативы
 * Transformer", vladkulikov.com, section 6 for softplus and sections 7 and 14
 * for the recurrent decode step and the shape of ssm_state):
 *
 *   for every batch row b and channel d, from a zero state h = 0:
 *     dt  = softplus(delta[b,t,d] + bias[d])     (or delta + bias without SSM_SOFTPLUS)
 *     h[n] = exp(dt * A[d,n]) * h[n] + dt * B[b,t,n] * x[b,t,d]     n < d_state
 *     y   = sum_n C[b,t,n] * h[n] + D[d] * x[b,t,d]
 *     out[b,t,d] = y * z[b,t,d] * sigmoid(z[b,t,d])                  (SiLU gate)
 *   softplus(u) = log(1 + e^u).  y is read after the update of step t.
 *
 * Layouts (all row-major, last index fastest, no strides):
 *   x, delta, z, out : [batch, seqlen, d_inner]
 *   B, C             : [batch, seqlen, d_state]  (one B_t, C_t per batch row
 *                                                 and step, shared by every channel)
 *   A                : [d_inner, d_state] fp32   (the caller passes A itself,
 *                                                 e.g. A = -exp(A_log))
 *   D, delta_bias    : [d_inner] fp32
 *   last_state, state: [batch, d_inner, d_state] fp32
 *
 * Precision: x, delta, z, B and C are all fp32 or all bf16 (in_dtype); the
 * state and every intermediate are fp32; out is fp32 or bf16 (out_dtype,
 * rounded to nearest even).
 *
 * Ownership: every pointer is a device pointer owned by the caller.  A scan
 * over more than one time chunk (and the backward, and a chunked Mamba-2
 * scan) takes a temporary workspace, stream-ordered on `stream` and freed on
 * it before the call returns.  Workspaces come from a memory pool that the
 * library keeps per device: memory a call frees stays reserved for later
 * calls (at most the largest set of workspaces in use at one time), so a call
 * after a synchronisation does not map its workspace again;
 * ssm_trim_workspace() returns it to the system.  Under stream capture the
 * workspace comes from hipMallocAsync on the stream instead, and the graph
 * owns it.  ssm_scan_fwd_noalloc uses a fixed array instead (below).
 *
 * Errors: every argument is checked on the host before anything is enqueued.
 * A non-OK status means nothing was enqueued and no output was written;
 * ssm_last_error() then holds a message for the calling thread.  Calls are
 * asynchronous on `stream` (a hipStream_t; NULL is the null stream): faults
 * during execution surface at the caller's next synchronisation.  Results
 * are bitwise reproducible for identical inputs and plan (no atomics).
 *
 * Graph capture: a call enqueues only kernels on `stream` (zero fills and
 * state copies are kernels, not memset or memcpy nodes), plus the
 * stream-ordered workspace allocation above, so it may be captured in a HIP
 * graph and replayed; the host checks run at capture time.
 */
#ifndef SSMSCAN_H
#define SSMSCAN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 10

/*
 * Bits of the step-flags argument (named `softplus` in the calls below):
 *   SSM_SOFTPLUS  dt = softplus(delta + bias); without it dt = delta + bias
 *                 as given (the caller guarantees a meaningful step).
 *   SSM_ZOH       the exact zero-order-hold input coefficient: the update adds
 *                 (e^{dt A[d,n]} - 1) / A[d,n] * B_t[n] * x in place of
 *                 dt * B_t[n] * x, with its limit dt where A[d,n] = 0 (page
 *                 "Модуль 8. Альтернативы Transformer", vladkulikov.com,
 *                 section 4: the input is held constant over the step, so its
 *                 coefficient is the integral of e^{sA} over [0, dt]; section 5
 *                 shows the two coefficients differ by 10 % at dt A = -0.19).
 *                 Forward calls only; the backward rejects it.
 * Any other bit is rejected with SSM_ERR_UNSUPPORTED.
 */
#define SSM_SOFTPLUS 1
#define SSM_ZOH 2

typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype;

typedef enum {
  SSM_OK = 0,
  SSM_ERR_NULL_ARG = 1,    /* a required pointer is NULL                                   */
  SSM_ERR_BAD_SHAPE = 2,   /* a size is negative or the element count overflows int64      */
  SSM_ERR_UNSUPPORTED = 3, /* dtype, d_state, alignment, aliasing or plan not supported    */
  SSM_ERR_HIP = 4          /* the HIP runtime refused an allocation or a launch            */
} ssm_status;

/*
 * Forward scan (prefill / training forward) from a zero state.
 *
 * Required: x, delta, A, B, C, out (a required pointer may be NULL only when
 * its tensor has no elements, as PyTorch gives empty tensors).  Optional (NULL
 * turns the term off):
 *   D           -- no skip term;
 *   z           -- no gate (out = y);
 *   delta_bias  -- bias 0;
 *   last_state  -- final state h after step seqlen-1 is not stored.
 * softplus: step flags, SSM_SOFTPLUS and/or SSM_ZOH (0: dt = delta + bias as
 *   given, with the dt input coefficient).
 * Sizes: batch, seqlen, d_inner >= 0 (a zero size is a valid empty call;
 *   with seqlen == 0 a non-NULL last_state is set to zero); d_state == 16.
 * Alignment: every pointer 16-byte aligned.
 * Aliasing: out and last_state must not overlap any input or each other.
 */
ssm_status ssm_scan_fwd(const void* x, const void* delta, const float* A, const void* B,
                        const void* C, const float* D, const void* z, const float* delta_bias,
                        int softplus, void* out, float* last_state, int64_t batch, int64_t seqlen,
                        int64_t d_inner, int64_t d_state, ssm_dtype in_dtype, ssm_dtype out_dtype,
                        void* stream);

/*
 * Single-token decode: one step of the same recurrence for every (b, d),
 * continuing from `state`, which is read and overwritten in place.
 *   state          : [batch, d_inner, d_state] fp32, in/out
 *   x, delta, z, out: [batch, d_inner]; B, C: [batch, d_state]
 * Optional arguments, sizes, alignment and errors as for ssm_scan_fwd; out
 * must not overlap state or any input.  Running seqlen steps from a zero
 * state gives the same outputs and final state as one ssm_scan_fwd call.
 */
ssm_status ssm_state_update(float* state, const void* x, const void* delta, const float* A,
                            const void* B, const void* C, const float* D, const void* z,
                            const float* delta_bias, int softplus, void* out, int64_t batch,
                            int64_t d_inner, int64_t d_state, ssm_dtype in_dtype,
                            ssm_dtype out_dtype, void* stream);

/*
 * Execution plan of a scan: how many of the d_state states one wavefront
 * carries per channel (states_per_wave in {1, 2, 4, 8, 16}; a workgroup
 * holds d_state / states_per_wave wavefronts on the same 64 channels), and the
 * time-chunk length (chunk_len >= 1; the sequence is cut into
 * ceil(seqlen / chunk_len) chunks scanned in parallel and joined by the
 * affine-pair carry pass).  ssm_scan_plan reports the plan ssm_scan_fwd picks;
 * ssm_scan_fwd_plan runs with a given plan (tests and tuning).  Any valid plan
 * computes the same function; only rounding order and speed differ.
 */
typedef struct {
  int32_t states_per_wave;
  int32_t reserved0;
  int64_t chunk_len;
  int64_t n_chunks;      /* output of ssm_scan_plan; ignored on input */
  int64_t reserved[4];
} ssm_plan;

ssm_status ssm_scan_plan(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                         ssm_plan* plan);

ssm_status ssm_scan_fwd_plan(const void* x, const void* delta, const float* A, const void* B,
                             const void* C, const float* D, const void* z,
                             const float* delta_bias, int softplus, void* out, float* last_state,
                             int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                             ssm_dtype in_dtype, ssm_dtype out_dtype, void* stream,
                             const ssm_plan* plan);

/*
 * Forward scan continuing from a stored state: the recurrence starts from
 * h = initial_state instead of zero, which continues a sequence scanned
 * earlier (chunked prefill, or a prompt after a cached prefix; pages
 * "Модуль 8. Альтернативы Transformer", sections 7 and 14: the inference cache
 * holds ssm_state [batch, d_inner, d_state], and the scan is the same
 * recurrence run from it).  Scanning L1 steps and then L2 steps from the
 * returned last_state gives the same outputs as one scan of L1 + L2 steps.
 *   initial_state: [batch, d_inner, d_state] fp32, or NULL for a zero state.
 * last_state may be the same buffer as initial_state (the state is then
 * replaced in place), but must not overlap it otherwise; out must not overlap
 * it.  plan may be NULL (the planner's choice).  With seqlen == 0 a non-NULL
 * last_state receives the initial state.  Everything else as for
 * ssm_scan_fwd.
 */
ssm_status ssm_scan_fwd_from(const void* x, const void* delta, const float* A, const void* B,
                             const void* C, const float* D, const void* z,
                             const float* delta_bias, int softplus, const float* initial_state,
                             void* out, float* last_state, int64_t batch, int64_t seqlen,
                             int64_t d_inner, int64_t d_state, ssm_dtype in_dtype,
                             ssm_dtype out_dtype, void* stream, const ssm_plan* plan);

/*
 * ssm_scan_fwd_from for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and checks as ssm_scan_fwd_from, and
 * the same kernels; it calls no hipMalloc, hipMallocAsync,
 * hipMallocFromPoolAsync or hipFree.  A plan
 * with more than one time chunk keeps its carry workspace (about
 * batch * n_chunks * d_inner * 68 bytes, plus the state when initial_state
 * is last_state) in a fixed array of SSM_NOALLOC_SCRATCH_BYTES bytes that
 * every GPU the library runs on holds from the first use until the process
 * ends.  A plan that needs more returns SSM_ERR_UNSUPPORTED (nothing
 * enqueued); ssm_scan_plan gives the planner's chunks.  All calls on one GPU
 * share that GPU's array and leave their contents in it: calls that overlap
 * in time on one GPU (different streams, or different host threads without
 * ordering) race and give wrong results.  The first call on a device looks
 * up the array's address (no allocation).
 */
#define SSM_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)
ssm_status ssm_scan_fwd_noalloc(const void* x, const void* delta, const float* A, const void* B,
                                const void* C, const float* D, const void* z,
                                const float* delta_bias, int softplus, const float* initial_state,
                                void* out, float* last_state, int64_t batch, int64_t seqlen,
                                int64_t d_inner, int64_t d_state, ssm_dtype in_dtype,
                                ssm_dtype out_dtype, void* stream, const ssm_plan* plan);

/*
 * Backward of the scan: the gradients of a loss L with respect to every input
 * of ssm_scan_fwd_from, given dout = dL/dout (and optionally dlast_state =
 * dL/dlast_state).  The pages give the forward recurrence only; the gradients
 * are its chain rule in reverse time:
 *   dh_t = C_t dy_t + exp(dt_{t+1} A) dh_{t+1}  (dh after the last step = dlast_state),
 *   with dy_t = dout_t SiLU(z_t) (or dout_t), and from it dx, ddelta, dz, dA,
 *   dB, dC, dD, ddelta_bias and dinitial_state.
 * The forward inputs (x .. softplus, initial_state) are those of the forward
 * call (step flags: SSM_SOFTPLUS or 0; SSM_ZOH is rejected); the forward
 * outputs are not needed (the states are recomputed).
 *   dout          : [batch, seqlen, d_inner] in grad_dtype
 *   dlast_state   : [batch, d_inner, d_state] fp32, or NULL (zero)
 *   dx, ddelta, dz: [batch, seqlen, d_inner] in grad_dtype (dz iff z != NULL)
 *   dB, dC        : [batch, seqlen, d_state] in grad_dtype
 *   dA            : [d_inner, d_state] fp32;  dD, ddelta_bias: [d_inner] fp32,
 *                   required exactly when D, delta_bias are given
 *   dinitial_state: [batch, d_inner, d_state] fp32 or NULL (not computed)
 * Every gradient is overwritten (not accumulated).  Reductions (dB, dC over
 * channels; dA, dD, ddelta_bias over rows) run in a fixed order: results are
 * bitwise reproducible for a given plan (below).  A workspace of about
 * batch * seqlen * d_inner * 8 + batch * seqlen * ceil(d_inner / 64) * 128
 * bytes (the states entering every 8-step tile, and per-block dB, dC) is taken
 * on `stream` as described under Ownership.  With few
 * channel blocks the sequence is cut into time chunks (ssm_scan_bwd_plan).
 * Outputs must not overlap any input or each other.  Sizes, dtypes, alignment
 * and errors as for ssm_scan_fwd (grad_dtype in place of out_dtype).
 */
ssm_status ssm_scan_bwd(const void* x, const void* delta, const float* A, const void* B,
                        const void* C, const float* D, const void* z, const float* delta_bias,
                        int softplus, const float* initial_state, const void* dout,
                        const float* dlast_state, void* dx, void* ddelta, float* dA, void* dB,
                        void* dC, float* dD, void* dz, float* ddelta_bias, float* dinitial_state,
                        int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                        ssm_dtype in_dtype, ssm_dtype grad_dtype, void* stream);

/*
 * Plans of the backward.  With fewer 64-channel blocks (batch *
 * ceil(d_inner / 64)) than compute units, ssm_scan_bwd cuts the sequence into
 * time chunks that run in parallel: each chunk's entering state comes from the
 * forward's chunk carry (vladkulikov.com, "Модуль 8. Альтернативы
 * Transformer", section 7: the affine pairs (exp(A S), end state) composed in
 * time order), and the gradient arriving at its end from the same pair
 * operator composed in reverse order (the reverse recurrence over a chunk is
 * affine in the gradient that arrives at its end, with the same decay
 * exp(A S)).  ssm_scan_bwd_plan_query reports the plan ssm_scan_bwd picks;
 * ssm_scan_bwd_plan runs with a given one (tests and tuning).
 * plan->states_per_wave must be 4; plan->chunk_len >= 1, and a multiple of 8
 * whenever it is below seqlen; at most 65535 chunks.  Any valid plan computes
 * the same gradients up to rounding order.  A chunked run takes
 * batch * n_chunks * d_inner * (3 * d_state + 2) * 4 more bytes of workspace.
 * Otherwise as for ssm_scan_bwd.
 */
ssm_status ssm_scan_bwd_plan_query(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                                   ssm_plan* plan);

ssm_status ssm_scan_bwd_plan(const void* x, const void* delta, const float* A, const void* B,
                             const void* C, const float* D, const void* z,
                             const float* delta_bias, int softplus, const float* initial_state,
                             const void* dout, const float* dlast_state, void* dx, void* ddelta,
                             float* dA, void* dB, void* dC, float* dD, void* dz,
                             float* ddelta_bias, float* dinitial_state, int64_t batch,
                             int64_t seqlen, int64_t d_inner, int64_t d_state, ssm_dtype in_dtype,
                             ssm_dtype grad_dtype, void* stream, const ssm_plan* plan);

/*
 * The backward's checkpoints from the forward.  ssm_scan_bwd first runs the
 * forward again to store the state entering every 8-step tile; a training
 * step that has just run the forward can keep those states instead
 * (vladkulikov.com, "Модуль 8. Альтернативы Transformer", section 7: the
 * forward's recurrence gives the state at every step; the backward is the
 * chain rule over the same recurrence).
 *   ssm_scan_ckpt_bytes : size of the checkpoint buffer for these sizes:
 *                         batch * ceil(d_inner / 64) * ceil(seqlen / 8) *
 *                         1024 * 4 bytes (the Mamba-2.8B-like layer: 671 MB).
 *   ssm_scan_fwd_ckpt   : ssm_scan_fwd_from (the planner's plan) that also
 *                         stores the checkpoints in ckpt (device memory, 16-byte
 *                         aligned, overlapping nothing else).  SSM_ZOH is
 *                         rejected (so is it by the backward).  out and
 *                         last_state are bitwise those of ssm_scan_fwd_from.
 *   ssm_scan_bwd_ckpt   : ssm_scan_bwd reading those checkpoints instead of
 *                         computing them; ckpt must come from
 *                         ssm_scan_fwd_ckpt over the same inputs, initial state
 *                         and step flags.  The gradients equal ssm_scan_bwd's
 *                         to rounding, and bitwise where neither call's plan
 *                         cuts the sequence into time chunks (chunked plans
 *                         join chunks at different steps, so their states
 *                         differ in rounding).
 * The buffer's layout is the library's own; it is read and written only by
 * these calls.  Otherwise as for ssm_scan_fwd_from and ssm_scan_bwd.
 */
ssm_status ssm_scan_ckpt_bytes(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state, int64_t* bytes);

ssm_status ssm_scan_fwd_ckpt(const void* x, const void* delta, const float* A, const void* B, const void* C,
                             const float* D, const void* z, const float* delta_bias, int softplus,
                             const float* initial_state, void* out, float* last_state, float* ckpt, int64_t batch,
                             int64_t seqlen, int64_t d_inner, int64_t d_state, ssm_dtype in_dtype,
                             ssm_dtype out_dtype, void* stream);

ssm_status ssm_scan_bwd_ckpt(const void* x, const void* delta, const float* A, const void* B, const void* C,
                             const float* D, const void* z, const float* delta_bias, int softplus,
                             const float* initial_state, const void* dout, const float* dlast_state,
                             const float* ckpt, void* dx, void* ddelta, float* dA, void* dB, void* dC, float* dD,
                             void* dz, float* ddelta_bias, float* dinitial_state, int64_t batch, int64_t seqlen,
                             int64_t d_inner, int64_t d_state, ssm_dtype in_dtype, ssm_dtype grad_dtype,
                             void* stream);

/*
 * The block's short causal depthwise convolution that feeds the scan (page
 * "Mamba и State Space Models", nareshka.ru, section "Реализация MambaBlock":
 * a Conv1d with one width-d_conv filter per channel and padding d_conv - 1,
 * cut to the sequence length; page "State Space Models: Mamba и альтернатива
 * Transformer", johe.ru, MambaBlock: SiLU after it):
 *
 *   out[b,t,d] = act(bias[d] + sum_{k < d_conv} weight[d,k] * x[b, t-d_conv+1+k, d])
 *
 * act is SiLU when `silu` is nonzero, else the identity.  Inputs before t = 0
 * are taken from conv_state_in, or are zero when it is NULL.
 *   x, out          : [batch, seqlen, d_inner] (in_dtype / out_dtype)
 *   weight          : [d_inner, d_conv] fp32;  bias: [d_inner] fp32 or NULL
 *   conv_state_in   : [batch, d_inner, d_conv] in in_dtype, or NULL: the d_conv
 *                     most recent earlier inputs of each channel, oldest first
 *                     (page "Модуль 8", sections 6 and 14: the decode cache keeps
 *                     the last d_conv inputs of the convolution branch)
 *   conv_state_out  : same layout, or NULL: receives the d_conv most recent
 *                     inputs after this call (zero-padded, or taken from
 *                     conv_state_in, when seqlen < d_conv); it may be the same
 *                     buffer as conv_state_in.
 * d_conv is 2, 3 or 4 (else SSM_ERR_UNSUPPORTED).  Pointers 16-byte aligned;
 * out and conv_state_out must not overlap any input or each other (except the
 * in-place cache).  Errors and asynchrony as for ssm_scan_fwd.
 */
ssm_status ssm_conv1d_fwd(const void* x, const float* weight, const float* bias, int silu,
                          const void* conv_state_in, void* out, void* conv_state_out,
                          int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_conv,
                          ssm_dtype in_dtype, ssm_dtype out_dtype, void* stream);

/*
 * One decode step of the convolution: for every (b, d) the cache conv_state
 * [batch, d_inner, d_conv] (in_dtype, read and overwritten in place) drops its
 * oldest input and appends x[b, d]; out[b, d] is the filter applied to the
 * updated cache, plus bias, through SiLU when `silu` is nonzero.  Running
 * seqlen steps from a zero cache gives the outputs and the cache of one
 * ssm_conv1d_fwd call.  x, out: [batch, d_inner].  Other arguments and errors
 * as for ssm_conv1d_fwd; out must not overlap conv_state or any input.
 */
ssm_status ssm_conv1d_update(void* conv_state, const void* x, const float* weight, const float* bias,
                             int silu, void* out, int64_t batch, int64_t d_inner, int64_t d_conv,
                             ssm_dtype in_dtype, ssm_dtype out_dtype, void* stream);

/*
 * Mamba-2 (SSD) form of the scan (page "Mamba и State Space Models",
 * nareshka.ru, section "Mamba-2: State Space Duality": A is one scalar per
 * head; page "Модуль 8. Альтернативы Transformer", vladkulikov.com, section 7:
 * with the transition a_t I the scan is the semi-separable matrix
 * M_ij = C_i^T B_j prod_{r=j+1..i} a_r applied to dt x, computed chunk by chunk
 * with matrix products and the state passed between chunks; section 14: the
 * state is [batch, nheads, headdim, d_state] and the input term is dt B x).
 * Channels are heads x headdim; the heads are split into ngroups contiguous
 * blocks that share B and C:
 *
 *   for batch row b, head h (group g = h / (nheads / ngroups)), channel p:
 *     dt  = softplus(dt_in[b,t,h] + dt_bias[h])   (or dt_in + dt_bias)
 *     s[p,n] = exp(dt * A[h]) * s[p,n] + dt * B[b,t,g,n] * x[b,t,h,p]
 *     out[b,t,h,p] = (sum_n C[b,t,g,n] s[p,n] + D[h*headdim + p] x) * SiLU(z)
 *
 * Layouts (row-major, last index fastest):
 *   x, z, out             : [batch, seqlen, nheads, headdim]
 *   dt                    : [batch, seqlen, nheads]
 *   B, C                  : [batch, seqlen, ngroups, d_state]
 *   A, dt_bias            : [nheads] fp32;  D: [nheads * headdim] fp32
 *   initial/last_state    : [batch, nheads, headdim, d_state] fp32
 * Supported: in_dtype bf16 (x, dt, z, B, C; the chunk products run on bf16
 * matrix cores with fp32 accumulation), out fp32 or bf16; headdim 64;
 * d_state 64 or 128; nheads a multiple of ngroups and at most 65535.
 * softplus: 0 or SSM_SOFTPLUS.  Optional (NULL): D, z, dt_bias, initial_state (zero),
 * last_state.  last_state may be the same buffer as initial_state; no other
 * overlap of an output with anything is allowed.  Every pointer 16-byte
 * aligned, except dt (element alignment).  The chunk form sums in a
 * different order than the recurrence:
 * results agree with it to rounding, not bitwise.
 */
ssm_status ssm_ssd_fwd(const void* x, const void* dt, const float* A, const void* B, const void* C,
                       const float* D, const void* z, const float* dt_bias, int softplus,
                       const float* initial_state, void* out, float* last_state, int64_t batch, int64_t seqlen,
                       int64_t nheads, int64_t headdim, int64_t ngroups, int64_t d_state, ssm_dtype in_dtype,
                       ssm_dtype out_dtype, void* stream);

/*
 * Plans of the Mamba-2 scan.  A workgroup walks one (batch row, head) through
 * the sequence; with at most 1.75 of them per compute unit, ssm_ssd_fwd cuts
 * the sequence into time chunks that run in parallel.  A head's decay over a
 * chunk is the scalar exp(A * sum of dt), so each chunk reduces to the pair
 * (decay, end state from zero), and the pairs compose in time order into each
 * chunk's entering state (vladkulikov.com, "Модуль 8. Альтернативы
 * Transformer", section 7: the affine pair operator of the chunked scan).
 * ssm_ssd_plan_query reports the plan ssm_ssd_fwd picks; ssm_ssd_fwd_plan
 * runs with a given one (tests and tuning): plan->chunk_len >= 1, and a
 * multiple of 32 whenever it is below seqlen; at most 65535 chunks;
 * states_per_wave is ignored.  A chunked run takes
 * batch * n_chunks * nheads * (headdim * d_state + 1) * 4 bytes of workspace
 * (plus a copy of an in-place initial state), taken as described under Ownership.
 * Any valid plan computes the same function up to rounding order.  Otherwise
 * as for ssm_ssd_fwd.
 */
ssm_status ssm_ssd_plan_query(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                              int64_t ngroups, int64_t d_state, ssm_plan* plan);

ssm_status ssm_ssd_fwd_plan(const void* x, const void* dt, const float* A, const void* B,
                            const void* C, const float* D, const void* z, const float* dt_bias,
                            int softplus, const float* initial_state, void* out, float* last_state,
                            int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                            int64_t ngroups, int64_t d_state, ssm_dtype in_dtype,
                            ssm_dtype out_dtype, void* stream, const ssm_plan* plan);

/*
 * One Mamba-2 decode step for every (b, h, p), continuing from `state`
 * [batch, nheads, headdim, d_state] fp32, read and overwritten in place
 * (pages as above; "Модуль 8", section 7: decode is the recurrent step with a
 * fixed-size state).  x, z, out: [batch, nheads, headdim]; dt: [batch, nheads];
 * B, C: [batch, ngroups, d_state].  in_dtype fp32 or bf16; any headdim >= 1;
 * nheads <= 65535; d_state 64 or 128; other rules as for ssm_ssd_fwd.
 */
ssm_status ssm_ssd_state_update(float* state, const void* x, const void* dt, const float* A, const void* B,
                                const void* C, const float* D, const void* z, const float* dt_bias, int softplus,
                                void* out, int64_t batch, int64_t nheads, int64_t headdim, int64_t ngroups,
                                int64_t d_state, ssm_dtype in_dtype, ssm_dtype out_dtype, void* stream);

/*
 * The affine-pair operator on its own, for checking the carry pass's combine
 * (page "Модуль 8. Альтернативы Transformer", section 7: the step h -> a h + b
 * is the pair (a, b), and (a2, b2) o (a1, b1) = (a2 a1, a2 b1 + b2), the later
 * step first).  Given n pairs (a[k], b[k]) in time order (device arrays, fp32),
 * writes the exclusive prefix: out_b[k] = state after pairs 0..k-1 applied to
 * h = 0 (out_b[0] = 0) and out_a[k] = product of a[0..k-1] (out_a[0] = 1).
 * Runs the same wavefront scan the carry pass uses.  n >= 0.
 */
ssm_status ssm_affine_exclusive_scan(const float* a, const float* b, float* out_a, float* out_b,
                                     int64_t n, void* stream);

/* Static string for a status code. */
const char* ssm_status_string(ssm_status s);
/* Message for the calling thread's last non-OK status ("" if none). */
const char* ssm_last_error(void);
/* SSM_ABI_VERSION of the loaded library. */
int ssm_abi_version(void);

/*
 * Returns the workspace memory that the library's pool on the current device
 * holds and no call is using to the system (hipMemPoolTrimTo).  Call it after
 * synchronising the streams the library ran on; the next call that needs a
 * workspace maps it again.  SSM_OK also when the pool was never created.
 */
ssm_status ssm_trim_workspace(void);

#ifdef __cplusplus
}
#endif

#endif /* SSMSCAN_H */
