/*
 * efla.h -- C ABI of libefla.so: Error-Free Linear Attention (EFLA) on AMD Instinct MI355X (gfx950).
 *
 * The operator (per batch b, head h, token t; S is d_k x d_v, k v^T is d_k x d_v):
 *   lambda_t = ||k_t||^2
 *   alpha_t  = (1 - e^{-beta_t lambda_t}) / lambda_t           (alpha_t = beta_t when lambda_t = 0)
 *   S_t      = (I - alpha_t k_t k_t^T) S_{t-1} + alpha_t k_t v_t^T
 *   o_t      = S_t^T q_t                                       (read after the update)
 * Sources: "Exact Flow Linear Attention: Exact Solution from Continuous-Time Dynamics" (gist.science),
 * Metodologia items 1-3 (ZOH ODE, closed-form rank-1 exponential, update rule and coefficient);
 * "Error-Free Linear Attention is a Free Lunch" (howistudyai.com), Steps 1-4 and the pipeline summary
 * (alpha from ||k||^2, exact update, readout o = S^T q, chunkwise parallel form with state passing).
 * Keys are used as given: nothing here normalises k (its norm is the gate).
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE pointers (memory from hipMalloc / a PyTorch CUDA tensor) unless stated.
 *     The library never allocates or frees device memory, and keeps no state between calls apart from
 *     a thread-local copy of the last HIP error text and, per device, the address of the fixed scratch
 *     array of efla_chunk_fwd_noalloc.  Calls that need scratch memory take a caller-owned workspace
 *     and say how large it must be (efla_chunk_fwd_noalloc uses the library's array instead).
 *   - Layouts are contiguous row-major.  q, k: [B,H,L,d_k]; v, o: [B,H,L,d_v]; beta: [B,H,L];
 *     state: [B,H,d_k,d_v] (S as the update writes it: row i is key dimension i).
 *     efla_chunk_fwd_layout and efla_chunk_bwd_layout also take strided views and packed sequences
 *     (efla_layout).
 *   - q, k, v, o use the storage type `dtype` (fp32 or bf16).  beta, alpha and the state are fp32.
 *     Arithmetic is fp32 (bf16 operands are multiplied on bf16 matrix cores with fp32 accumulation).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only enqueues work and returns;
 *     results are valid once the stream has been synchronised.
 *   - All arguments are checked BEFORE anything is enqueued.  On any error nothing is launched and
 *     no output is touched.  A failed launch returns EFLA_ERR_HIP (text: efla_last_error()).
 *     Faults of running kernels surface at the caller's next synchronisation.
 *   - Supported sizes: d_k, d_v in {16, 32, 64, 128}; chunk in {16, 32, 64}; any L >= 0 (a short
 *     last chunk is handled).  Tensor pointers must be 16-byte aligned, beta/alpha 4-byte aligned.
 *   - Preconditions not checked on the device: beta >= 0 and finite inputs (NaN propagates).
 */
#ifndef EFLA_H
#define EFLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    EFLA_OK = 0,
    EFLA_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, negative size, overlapping buffers, bad enum */
    EFLA_ERR_UNSUPPORTED = 2,   /* d_k, d_v, chunk or dtype combination this build does not provide    */
    EFLA_ERR_WORKSPACE = 3,     /* workspace / output buffer missing, misaligned or smaller than needed */
    EFLA_ERR_NO_DEVICE = 4,     /* no HIP device is visible to the process                             */
    EFLA_ERR_HIP = 5,           /* a HIP runtime call or kernel launch failed                          */
    EFLA_STATUS_RANGE_MIN_ = -0x7FFFFFFF - 1,   /* never returned: with these two bounds every 32-bit int */
    EFLA_STATUS_RANGE_MAX_ = 0x7FFFFFFF         /* is a value of the type, so a C caller's bad value is   */
} efla_status;                                  /* defined and reaches the argument checks               */

typedef enum {
    EFLA_F32 = 0,
    EFLA_BF16 = 1,
    EFLA_DTYPE_RANGE_MIN_ = -0x7FFFFFFF - 1,    /* never valid: every 32-bit int is a value of the type */
    EFLA_DTYPE_RANGE_MAX_ = 0x7FFFFFFF          /* (an invalid one is rejected as EFLA_ERR_INVALID_ARG)  */
} efla_dtype;

/*
 * Gates.  The calls below use the exact coefficient alpha_t.  Their *_gate variants take an `int gate`
 * that selects the coefficient of another integrator of the same per-token dynamics
 * dS/dt = -k k^T S + k v^T over a step beta, with every kernel and layout unchanged:
 *   EFLA_GATE_EXACT (0)     the exact flow, alpha = (1 - e^{-beta lambda}) / lambda
 *   p in 1 .. EFLA_GATE_MAX_ORDER
 *                           one p-th order Runge-Kutta step.  For this rank-1 dynamics it has the same
 *                           update form, with alpha_p = sum_{n=1}^{p} (-1)^{n-1} beta^n lambda^{n-1} / n!
 *                           (the degree-p Taylor polynomial of the exponential, reduced with
 *                           (k k^T)^n = lambda^{n-1} k k^T).  p = 1 (EFLA_GATE_DELTANET) is the explicit
 *                           Euler step, the delta rule's alpha = beta; alpha_p -> alpha as p grows.
 * ("Error-Free Linear Attention guida completa" (mauroscia.it), the section on RK-infinity: Euler and
 * Runge-Kutta steps of rising order approach the exact solution; "Error-Free Linear Attention is a Free
 * Lunch" (howistudyai.com), building blocks "Delta Rule" and "Runge-Kutta Methods".)  A gate outside
 * 0 .. EFLA_GATE_MAX_ORDER is EFLA_ERR_INVALID_ARG.  alpha_p is evaluated in fp32 by Horner's scheme;
 * for large beta*lambda it grows like (beta lambda)^{p-1} (the explicit schemes are not stable there).
 */
#define EFLA_GATE_EXACT 0
#define EFLA_GATE_DELTANET 1
#define EFLA_GATE_MAX_ORDER 16

/*
 * efla_alpha -- the exact gate alpha_t for n_tokens keys.
 * "Error-Free Linear Attention is a Free Lunch" (howistudyai.com), Step 1; "Exact Flow Linear
 * Attention" (gist.science), Metodologia item 3 (the effective coefficient).
 *   k     [n_tokens, d_k] in k_dtype (device), read only
 *   beta  [n_tokens] fp32 (device), read only
 *   alpha [n_tokens] fp32 (device), written; must not overlap k or beta
 * Evaluated as -expm1(-beta*lambda)/lambda in fp32 with lambda summed in fp32; beta when
 * beta*lambda == 0.  n_tokens == 0 is a no-op.  d_k may be any of 16, 32, 64, 128.
 */
efla_status efla_alpha(const void* k, efla_dtype k_dtype, const float* beta, float* alpha,
                       int64_t n_tokens, int d_k, void* stream);
/* efla_alpha with a gate (see "Gates" above); efla_alpha is gate EFLA_GATE_EXACT. */
efla_status efla_alpha_gate(const void* k, efla_dtype k_dtype, const float* beta, float* alpha,
                            int64_t n_tokens, int d_k, int gate, void* stream);

/*
 * efla_chunk_fwd -- the whole sequence forward: every o_t and (optionally) the final state.
 * Chunkwise-parallel form ("Exact Flow Linear Attention", Metodologia item 3: the update keeps the
 * rank-1 delta-rule structure, so the WY/UT chunk scheme applies; "Error-Free Linear Attention is a
 * Free Lunch", Step 4 and the pipeline summary: within-chunk transforms in parallel, chunks joined by
 * passing the state, "for each token (or for each chunk in parallel)").
 * Per chunk of C tokens with state S entering it:
 *   A = strict_lower(diag(alpha) K K^T),  T = (I + A)^{-1},  R = V - K S,  Delta = T diag(alpha) R,
 *   O = Q S + lower_incl(Q K^T) Delta,    S <- S + K^T Delta
 * which is the token recurrence above, regrouped; the result does not depend on `chunk` beyond
 * rounding.
 *   q, k          [B,H,L,d_k] dtype, read only
 *   v             [B,H,L,d_v] dtype, read only
 *   beta          [B,H,L] fp32, read only
 *   o             [B,H,L,d_v] dtype, written; must not overlap any other argument
 *   initial_state [B,H,d_k,d_v] fp32 or NULL (= zeros), read only
 *   final_state   [B,H,d_k,d_v] fp32 or NULL (= not written).  May be the same pointer as
 *                 initial_state (in-place state passing); any other overlap is rejected.
 *   chunk         16, 32 or 64 tokens per chunk
 *   workspace     device memory of at least efla_chunk_fwd_workspace_size(B, H, L, d_k, d_v, chunk, dtype)
 *                 bytes, 256-byte aligned, overlapping no other argument; may be NULL when that size is 0.
 *                 Smaller, NULL or misaligned when needed: EFLA_ERR_WORKSPACE.  Its contents on return are
 *                 unspecified; calls that share a workspace must be ordered on one stream.
 * The library picks the form for the sizes (efla_chunk_fwd_form reports it; every form gives the same result
 * up to rounding, and the same form always gives bit-identical results):
 *   EFLA_FWD_SCAN        few (batch, head) pairs and long sequences (one segment's state pass would occupy at
 *                        most a quarter of the compute units): the segment-parallel form of efla_chunk_fwd_scan
 *                        with the library's segment count;
 *   EFLA_FWD_ONE_LAUNCH  otherwise, bf16 with d_k >= 32 and 64-token chunks: one kernel whose workgroups form
 *                        the chunks' T diag(alpha) themselves (efla_chunk_fwd_slab); no workspace;
 *   EFLA_FWD_SPLIT       otherwise: the UT transform of every chunk into the workspace, then the state pass
 *                        (efla_chunk_fwd_split).
 * The state is carried in fp32 for the whole sequence.  L == 0 copies initial_state (or zeros) to
 * final_state.  q, k, v, beta and o may be NULL only when L == 0.
 */
efla_status efla_chunk_fwd(const void* q, const void* k, const void* v, const float* beta,
                           efla_dtype dtype, void* o, const float* initial_state, float* final_state,
                           int B, int H, int L, int d_k, int d_v, int chunk,
                           void* workspace, size_t workspace_bytes, void* stream);
/* efla_chunk_fwd with a gate (see "Gates" above); efla_chunk_fwd is gate EFLA_GATE_EXACT. */
efla_status efla_chunk_fwd_gate(const void* q, const void* k, const void* v, const float* beta,
                                efla_dtype dtype, void* o, const float* initial_state, float* final_state,
                                int B, int H, int L, int d_k, int d_v, int chunk, int gate,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * efla_chunk_fwd_workspace_size -- bytes of workspace efla_chunk_fwd needs for these sizes (host only, no
 * device needed): 0 for the one-launch form; the UT output for the split form; the UT output and the
 * segments' states for the scan form.  Sizes efla_chunk_fwd would reject give 0 (the call itself then
 * returns the error).
 */
size_t efla_chunk_fwd_workspace_size(int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype dtype);

/* The forms efla_chunk_fwd chooses between (see there). */
typedef enum {
    EFLA_FWD_ONE_LAUNCH = 0,
    EFLA_FWD_SPLIT = 1,
    EFLA_FWD_SCAN = 2,
    EFLA_FWD_FORM_RANGE_MIN_ = -0x7FFFFFFF - 1,   /* never reported (32-bit range, as efla_dtype) */
    EFLA_FWD_FORM_RANGE_MAX_ = 0x7FFFFFFF
} efla_fwd_form;

/*
 * efla_chunk_fwd_form -- the form efla_chunk_fwd takes for these sizes, its segment count (1 unless
 * EFLA_FWD_SCAN) and its workspace bytes (host only).  Any output pointer may be NULL.  Returns the error
 * efla_chunk_fwd would return for the sizes alone, else EFLA_OK.
 */
efla_status efla_chunk_fwd_form(int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype dtype,
                                int* form, int* segments, size_t* workspace_bytes);

/*
 * efla_chunk_fwd_noalloc -- efla_chunk_fwd_gate for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same forms, kernels and results
 * (bit-identical to efla_chunk_fwd_gate with a workspace of its own), with the workspace taken from a scratch
 * array of EFLA_NOALLOC_SCRATCH_BYTES that the library holds in device memory on every GPU it runs on, from its
 * code's load until the process ends.  The call allocates nothing: no hipMalloc, no hipFree, no allocating
 * library routine.  The caller still passes every input and output.
 *   Sizes whose efla_chunk_fwd_workspace_size exceeds EFLA_NOALLOC_SCRATCH_BYTES: EFLA_ERR_WORKSPACE, nothing
 *   enqueued.  The forms that need no workspace (the one-launch form) never touch the scratch.
 *   Every call on one GPU uses that GPU's one scratch array, which keeps what the last call left there: calls
 *   that may run at the same time on one GPU (other streams, other threads) race and give wrong results; order
 *   them on one stream.  Nothing in the scratch needs to start at any value (each call writes what it reads).
 *   The device is the calling thread's current HIP device; its scratch address is looked up once per device.
 * Other arguments and errors as efla_chunk_fwd_gate.
 */
#define EFLA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
efla_status efla_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* beta,
                                   efla_dtype dtype, void* o, const float* initial_state, float* final_state,
                                   int B, int H, int L, int d_k, int d_v, int chunk, int gate, void* stream);

/*
 * efla_chunk_fwd_slab -- the forward in one launch and without workspace, with an explicit split of the d_v
 * columns of the state across workgroups: each workgroup owns `dv_slab` columns (16, 32 or 64, dividing d_v;
 * 0 = the library's choice).  For bf16, d_k >= 32 and 64-token chunks the kernel is the one of efla_chunk_fwd's
 * one-launch form (each workgroup runs the state pass and, on waves of its own, the chunks' UT transform);
 * otherwise a fused kernel that repeats every chunk's UT transform in each of its head's workgroups.  Columns of
 * S evolve independently, so every valid split gives the same result up to rounding.  Same arguments and errors
 * as efla_chunk_fwd otherwise (there is no workspace).
 */
efla_status efla_chunk_fwd_slab(const void* q, const void* k, const void* v, const float* beta,
                                efla_dtype dtype, void* o, const float* initial_state, float* final_state,
                                int B, int H, int L, int d_k, int d_v, int chunk, int dv_slab, void* stream);
/* efla_chunk_fwd_slab with a gate (see "Gates" above): alpha_t of every token is the gate's. */
efla_status efla_chunk_fwd_slab_gate(const void* q, const void* k, const void* v, const float* beta,
                                     efla_dtype dtype, void* o, const float* initial_state, float* final_state,
                                     int B, int H, int L, int d_k, int d_v, int chunk, int dv_slab, int gate,
                                     void* stream);

/*
 * efla_recurrent_step -- one decode token for NH independent (sequence, head) states, in place.
 * "Error-Free Linear Attention is a Free Lunch" (howistudyai.com), pipeline summary ("for each
 * token": alpha, update S, emit o = S^T q); "Exact Flow Linear Attention", Metodologia item 3.
 * Per state (a = S^T k and b = S^T q taken before the update):
 *   S <- S + alpha k (v - a)^T,   o = b + alpha (k^T q) (v - a)      (= S_new^T q)
 *   q, k  [NH, d_k] dtype, read only
 *   v     [NH, d_v] dtype, read only
 *   beta  [NH] fp32, read only
 *   state [NH, d_k, d_v] fp32, read and overwritten in place
 *   o     [NH, d_v] dtype, written; must not overlap state or the inputs
 * NH == 0 is a no-op.
 */
efla_status efla_recurrent_step(const void* q, const void* k, const void* v, const float* beta,
                                efla_dtype dtype, float* state, void* o,
                                int64_t NH, int d_k, int d_v, void* stream);
/* efla_recurrent_step with a gate (see "Gates" above). */
efla_status efla_recurrent_step_gate(const void* q, const void* k, const void* v, const float* beta,
                                     efla_dtype dtype, float* state, void* o,
                                     int64_t NH, int d_k, int d_v, int gate, void* stream);

/*
 * efla_chunk_split_workspace_size -- bytes of the workspace efla_chunk_fwd_split needs, which is also the
 * size of the efla_ut_transform output: ceil(L / chunk) * (chunk/16)(chunk/16 + 1)/2 * 256 elements of
 * the storage type per (batch, head).  Host only.  Fills *bytes and returns EFLA_OK, or INVALID_ARG
 * (negative size, bad dtype, NULL bytes) / UNSUPPORTED (chunk).
 */
efla_status efla_chunk_split_workspace_size(int B, int H, int L, int chunk, efla_dtype dtype, size_t* bytes);

/*
 * efla_ut_transform -- the intra-chunk UT transform alone: for every chunk of C = chunk tokens of every
 * (batch, head), with alpha the exact gate of its tokens,
 *   A = strict_lower(diag(alpha) K K^T),  T = (I + A)^{-1},  output T diag(alpha)  (C x C, lower).
 * "Error-Free Linear Attention is a Free Lunch" (howistudyai.com), Step 4 (precompute the within-chunk
 * transforms in parallel); "Exact Flow Linear Attention" (gist.science), Metodologia item 3 (the update
 * keeps the delta-rule rank-1 form, so the WY/UT representation applies).  A short last chunk is padded
 * with zero keys and zero beta, so its missing rows and columns of T diag(alpha) are zero.
 *   k      [B,H,L,d_k] dtype, read only;  beta [B,H,L] fp32, read only
 *   t_out  written, t_out_bytes >= efla_chunk_split_workspace_size(...) (else EFLA_ERR_WORKSPACE), 16-byte
 *          aligned, no overlap with k or beta.  Layout, in the storage type, per (bh, chunk c): the
 *          (C/16)(C/16+1)/2 lower 16x16 blocks (rb, kb), kb <= rb, in the order rb (rb+1)/2 + kb, each as
 *          256 elements [lane][j] with lane = 16 g + r holding (T diag(alpha))[16 rb + r][16 kb + 4 g + j]
 *          (the matrix-core operand layout in which efla_chunk_fwd_split consumes it).
 * The substitution runs in fp32; the bf16 build rounds the result to bf16.  L == 0 is a no-op.
 */
efla_status efla_ut_transform(const void* k, const float* beta, efla_dtype dtype, void* t_out, size_t t_out_bytes,
                              int B, int H, int L, int d_k, int chunk, void* stream);
/* efla_ut_transform with a gate (see "Gates" above): alpha in A and in T diag(alpha) is the gate's. */
efla_status efla_ut_transform_gate(const void* k, const float* beta, efla_dtype dtype, void* t_out,
                                   size_t t_out_bytes, int B, int H, int L, int d_k, int chunk, int gate,
                                   void* stream);

/*
 * efla_chunk_fwd_split -- efla_chunk_fwd as two launches on `stream`: efla_ut_transform of every chunk into
 * `workspace`, then the inter-chunk state pass, which reads T diag(alpha) from it.  Same operator, arguments,
 * aliasing rules and errors as efla_chunk_fwd_slab, plus:
 *   workspace        device memory of at least efla_chunk_split_workspace_size(B, H, L, chunk, dtype) bytes,
 *                    16-byte aligned, overlapping no other argument (else EFLA_ERR_WORKSPACE /
 *                    EFLA_ERR_INVALID_ARG); its contents on return are the UT output described above,
 *                    except that with bf16 inputs, d_k >= 32 and chunk 64 only the blocks (rb, kb) with
 *                    rb / 2 == kb / 2 (the two diagonal 32 x 32 blocks of each chunk, all the state pass reads
 *                    there) are written; the other four blocks of each chunk are left as they were.
 * The UT launch spreads over all (batch*head, chunk) pairs, so the serial state pass carries only the
 * state-dependent products.  Calls that share a workspace must be ordered on one stream.
 */
efla_status efla_chunk_fwd_split(const void* q, const void* k, const void* v, const float* beta,
                                 efla_dtype dtype, void* o, const float* initial_state, float* final_state,
                                 int B, int H, int L, int d_k, int d_v, int chunk, int dv_slab,
                                 void* workspace, size_t workspace_bytes, void* stream);
/* efla_chunk_fwd_split with a gate (see "Gates" above).  The state pass itself does not depend on the
 * gate (it reads T diag(alpha) from the workspace), so efla_chunk_state_pass serves every gate. */
efla_status efla_chunk_fwd_split_gate(const void* q, const void* k, const void* v, const float* beta,
                                      efla_dtype dtype, void* o, const float* initial_state, float* final_state,
                                      int B, int H, int L, int d_k, int d_v, int chunk, int dv_slab, int gate,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * efla_chunk_state_pass -- the inter-chunk state pass alone, from a UT output made beforehand by
 * efla_ut_transform (same k, beta, B, H, L, d_k, chunk, dtype).  For each (batch, head), S starts at
 * initial_state (or 0) and, chunk after chunk, with Ta = T diag(alpha) read from t_in:
 *   Delta = Ta (V - K S),  O = Q S + lower_incl(Q K^T) Delta,  S <- S + K^T Delta
 * ("Error-Free Linear Attention is a Free Lunch" (howistudyai.com), Step 4: chunks joined by passing the
 * state; Step 3: o_t = S_t^T q_t after each token's update).  efla_chunk_fwd_split is efla_ut_transform
 * followed by this call, and gives bit-identical results.
 *   t_in  read only, t_in_bytes >= efla_chunk_split_workspace_size(...) (else EFLA_ERR_WORKSPACE), 16-byte
 *         aligned, overlapping no output.  Other arguments as efla_chunk_fwd_slab (there is no beta).
 */
efla_status efla_chunk_state_pass(const void* q, const void* k, const void* v, const void* t_in, size_t t_in_bytes,
                                  efla_dtype dtype, void* o, const float* initial_state, float* final_state,
                                  int B, int H, int L, int d_k, int d_v, int chunk, int dv_slab, void* stream);

/*
 * efla_chunk_fwd_scan -- efla_chunk_fwd for few (batch, head) pairs and long sequences: the chunks of each
 * sequence are cut into `segments` consecutive segments that are processed at the same time.  The state
 * recurrence is affine in the state ("Exact Flow Linear Attention" (gist.science), Metodologia item 3: the
 * update is linear in S; "Error-Free Linear Attention is a Free Lunch" (howistudyai.com), Step 4: chunks are
 * joined by passing the state), so over a segment S_out = M S_in + S_out(0), with M the product of the chunk
 * transitions I - K^T T diag(alpha) K.  Launches, all on `stream`: the UT transform of every chunk; a state pass
 * over every segment from a zero state, on the state augmented with d_k columns that start as the identity
 * and see zero values (they end as M); a scan S_in[g+1] = M_g S_in[g] + S_g(0) from initial_state; a state pass
 * over every segment from its S_in that writes the outputs and the last segment's final state.  About three
 * times the state-pass work of efla_chunk_fwd_split, spread over `segments` times as many workgroups.
 * Same operator, arguments, aliasing rules and errors as efla_chunk_fwd_split_gate, plus:
 *   segments   0 = the library's choice (efla_chunk_scan_plan), else the number of segments wanted (at most
 *              one per chunk; the count actually used is ceil(chunks / ceil(chunks / segments)))
 *   workspace  device memory of at least efla_chunk_scan_plan(...)'s workspace_bytes, 256-byte aligned,
 *              overlapping no other argument; with one segment this is the efla_chunk_fwd_split workspace.
 */
efla_status efla_chunk_fwd_scan(const void* q, const void* k, const void* v, const float* beta,
                                efla_dtype dtype, void* o, const float* initial_state, float* final_state,
                                int B, int H, int L, int d_k, int d_v, int chunk, int segments, int gate,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Launch shape and workspace of efla_chunk_fwd_scan for these sizes (host only): segments used, chunks per
 * segment, state slab width (of the pass that writes the outputs; the first pass, which carries d_v + d_k
 * columns, takes slabs of 128 at d_k = d_v = 128 with bf16 and 64-token chunks when that still gives every
 * compute unit a workgroup) and workspace bytes.  Errors as efla_chunk_fwd_scan would return for the sizes.
 * With segments = 0 the library cuts sequences only when one segment's state pass would run at most 64
 * workgroups (a quarter of the compute units): the count G starts at 1 and doubles while 2G segments' second
 * pass stays within 256 workgroups and the sequence holds at least 32 G chunks; otherwise one segment. */
efla_status efla_chunk_scan_plan(int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype dtype, int segments,
                                 int* nseg, int* seg_chunks, int* slab_width, size_t* workspace_bytes);

/*
 * Token layouts of efla_chunk_fwd_layout.  The pages place the method as a drop-in replacement inside
 * existing chunked delta-rule pipelines ("Error-Free Linear Attention guida completa" (mauroscia.it),
 * section "Chunkwise parallelism"), so the forward reads the tensors as a model layer holds them instead of
 * requiring transposed copies.
 *
 * Every stride counts elements (not bytes).  Element (b, h, t, i) of q is q[b*q[0] + h*q[1] + t*q[2] + i]
 * (feature index i contiguous); likewise k, v and o; beta(b, h, t) = beta[b*beta[0] + h*beta[1] + t*beta[2]].
 * [B,H,L,d] contiguous is {H*L*d, L*d, d}; [B,L,H,d] is {L*H*d, d, H*d}.
 *
 * cu_seqlens (device memory, B + 1 int32, or NULL): packed sequences.  Then B counts sequences, L is the
 * packed token count, sequence b is tokens [cu_seqlens[b], cu_seqlens[b+1]) of every head, the batch strides
 * are ignored, and every sequence starts from its own initial state and ends in its own final state
 * ([B,H,d_k,d_v]).  The offsets are read sanitised: each clamped to [0, L], then replaced by the largest of
 * itself and the entries before it (so an out-of-order or out-of-range entry gives shorter or empty
 * sequences, never overlapping ones nor an access outside [0, L)).  An empty sequence passes its initial
 * state through.
 */
typedef struct efla_layout {
    int64_t q[3], k[3], v[3], o[3]; /* batch, head, token strides */
    int64_t beta[3];                /* batch, head, token strides */
    const int32_t* cu_seqlens;      /* device, B + 1 entries, or NULL */
} efla_layout;

/*
 * efla_chunk_fwd_layout -- the forward over tensors in the layout described by `layout` (NULL: contiguous
 * [B,H,L,d]), in the form efla_chunk_fwd_gate would take: the one-launch kernel for bf16 with d_k >= 32 and
 * 64-token chunks when one segment is used (then bit-identical to that kernel on contiguous copies), else
 * efla_chunk_fwd_split_gate or efla_chunk_fwd_scan.  Same operator, gate, states, aliasing rules and errors, plus:
 *   strides    all >= 0; those of q, k, v, o multiples of 16 bytes / element size (8 for bf16, 4 for fp32);
 *              token strides at least the row (d_k for q and k, d_v for v) and 1 for beta, and below
 *              2^31 / (64 * element size); the rows of o must not overlap one another (sorted by stride,
 *              each stride at least the extent of the dimensions inside it); else EFLA_ERR_INVALID_ARG.
 *              Overlap checks between arguments use each tensor's address extent.
 *   segments   as efla_chunk_fwd_scan (0 = the library's choice); with cu_seqlens only 0 or 1 (one segment).
 *   workspace  device memory of at least efla_chunk_layout_plan(...)'s workspace_bytes, 256-byte aligned,
 *              overlapping no other argument.  With cu_seqlens it holds the sanitised token offsets and the
 *              sequences' chunk offsets (made on `stream` by this call), then the UT output of
 *              sum_b ceil(len_b / chunk) chunks per head.
 */
efla_status efla_chunk_fwd_layout(const void* q, const void* k, const void* v, const float* beta,
                                  efla_dtype dtype, void* o, const float* initial_state, float* final_state,
                                  int B, int H, int L, int d_k, int d_v, int chunk, int segments, int gate,
                                  const efla_layout* layout, void* workspace, size_t workspace_bytes, void* stream);

/* Segments used and workspace bytes of efla_chunk_fwd_layout for these sizes (host only); varlen != 0 when
 * cu_seqlens will be given.  Errors as efla_chunk_fwd_layout would return for the sizes. */
efla_status efla_chunk_layout_plan(int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype dtype, int varlen,
                                   int segments, int* nseg, size_t* workspace_bytes);

/*
 * efla_chunk_bwd -- gradients of the chunked forward (efla_chunk_fwd_split_gate with the same q, k, v, beta,
 * initial_state, chunk and gate): given d_o = dLoss/do and d_final = dLoss/dS_L, writes dLoss/dq, /dk, /dv,
 * /dbeta and /dinitial_state.  The pages train every model they report but print no backward pass ("Exact
 * Flow Linear Attention" (gist.science), Risultati Sperimentali item 4; "Error-Free Linear Attention is a
 * Free Lunch" (howistudyai.com), the language-modelling results), so this is the adjoint of the chunked form
 * of Step 4, with d alpha / d beta and d alpha / d lambda of the gate in use (gate as in "Gates" above).
 *   q, k, v, beta, initial_state   the forward's inputs (initial_state NULL = zeros), read only
 *   d_o            [B,H,L,d_v] dtype, read only (required when L > 0)
 *   d_final        [B,H,d_k,d_v] fp32 or NULL (= zeros), read only
 *   dq, dk         [B,H,L,d_k] dtype, written;  dv [B,H,L,d_v] dtype, written;  dbeta [B,H,L] fp32, written
 *   d_initial      [B,H,d_k,d_v] fp32, written, or NULL (not written)
 *   workspace      device memory of at least efla_chunk_bwd_workspace_size(...) bytes, 256-byte aligned:
 *                  the chunks' T diag(alpha), the state entering and the state gradient leaving every chunk
 *                  (2 B H ceil(L/chunk) d_k d_v elements: bf16 where all three passes below run on bf16 matrix
 *                  cores -- bf16, d_k >= 32, 64-token chunks, d_v a multiple of 32 -- else fp32; 0.54 GB of the
 *                  0.65 GB for B8 H16 L4096 d128), and for bf16 with d_k >= 32, chunks of 32 or 64 and d_v a
 *                  multiple of 32 each chunk's T^T (bf16)
 * Outputs must not overlap one another, any input or the workspace (EFLA_ERR_INVALID_ARG).  Launches, all on
 * `stream`: the UT transform, the state pass again (keeping every chunk's entering state), the state
 * gradient backwards over the chunks (dv, d_initial), and one launch over all (head, chunk) pairs (dq, dk,
 * dbeta).  Arithmetic: bf16 inputs with d_k >= 32 take every product on bf16 matrix cores with fp32
 * accumulation (operands, the per-chunk states included, rounded to bf16) where the sizes above allow, fp32
 * matrix cores otherwise; fp32 inputs are fp32 throughout.  No kernel accumulates with atomics: the same
 * inputs give the same bits.  Sizes as efla_chunk_fwd.
 */
efla_status efla_chunk_bwd(const void* q, const void* k, const void* v, const float* beta, efla_dtype dtype,
                           const float* initial_state, const void* d_o, const float* d_final,
                           void* dq, void* dk, void* dv, float* dbeta, float* d_initial,
                           int B, int H, int L, int d_k, int d_v, int chunk, int gate,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes efla_chunk_bwd needs for these sizes (host only). */
efla_status efla_chunk_bwd_workspace_size(int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype dtype,
                                          size_t* bytes);

/*
 * efla_chunk_bwd_layout -- efla_chunk_bwd over tensors in the layout described by `layout` (NULL: contiguous
 * [B,H,L,d], exactly efla_chunk_bwd): the gradients of efla_chunk_fwd_layout's operator, for model layers that
 * hold q, k, v as [B,L,H,d] views, slices of a fused projection or packed sequences ("Error-Free Linear
 * Attention guida completa" (mauroscia.it), section "Chunkwise parallelism": the method drops into existing
 * chunked pipelines, whose training runs the backward over the same tensors).
 *   layout     as efla_chunk_fwd_layout's (same stride rules), with o's strides describing d_o.  dq, dk, dv and
 *              dbeta are written with the strides of q, k, v and beta (e.g. slices of one fused gradient buffer
 *              when q, k, v are slices of a fused projection); no two of their rows (elements, for dbeta) may
 *              share memory, else EFLA_ERR_INVALID_ARG.
 *   cu_seqlens packed sequences (layout->cu_seqlens, read sanitised as in efla_chunk_fwd_layout): B counts
 *              sequences, every sequence starts from its own initial state, and initial_state, d_final and
 *              d_initial hold one [d_k,d_v] state per (sequence, head).  Gradients of tokens outside every
 *              sequence are not written.
 *   workspace  at least efla_chunk_bwd_layout_workspace_size(...) bytes, 256-byte aligned, overlapping no other
 *              argument; with cu_seqlens it begins with the sanitised offsets, made on `stream` by this call.
 * Arithmetic, launches and errors as efla_chunk_bwd; a layout changes only where the kernels read and write, so
 * the results equal efla_chunk_bwd's on contiguous copies of the tensors bit for bit, and for packed sequences
 * those of separate calls, one per sequence (no kernel of the backward accumulates with atomics: the same inputs
 * give the same bits).  Overlap checks use each tensor's address extent, except that two tensors of the same
 * element size, sizes and strides may share an extent when their rows provably miss one another, as slices of
 * one fused buffer do: with the dimensions sorted by stride and those contiguous with the row merged into a block
 * of m elements, every other stride a multiple of the smallest, s, and the bases' distance d (elements) with
 * m <= d mod s <= s - m.
 */
efla_status efla_chunk_bwd_layout(const void* q, const void* k, const void* v, const float* beta, efla_dtype dtype,
                                  const float* initial_state, const void* d_o, const float* d_final,
                                  void* dq, void* dk, void* dv, float* dbeta, float* d_initial,
                                  int B, int H, int L, int d_k, int d_v, int chunk, int gate,
                                  const efla_layout* layout, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes efla_chunk_bwd_layout needs for these sizes (host only); varlen != 0 when cu_seqlens will be
 * given (then the bound H (ceil(L / chunk) + B) on the sequences' chunks sizes it).  Errors as
 * efla_chunk_bwd_layout would return for the sizes. */
efla_status efla_chunk_bwd_layout_workspace_size(int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype dtype,
                                                 int varlen, size_t* bytes);

/* Like efla_chunk_fwd_plan, for the state-pass launch of efla_chunk_fwd_split / efla_chunk_state_pass. */
efla_status efla_chunk_fwd_split_plan(int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype dtype,
                                      int dv_slab, int* workgroups, int* slab_width, int* lds_bytes);

/* Workgroups and d_v slab width efla_chunk_fwd would launch for these sizes (host only, no device
 * needed).  Returns EFLA_OK and fills the outputs, or the error efla_chunk_fwd would return for
 * the sizes alone. */
efla_status efla_chunk_fwd_plan(int B, int H, int L, int d_k, int d_v, int chunk, efla_dtype dtype,
                                int dv_slab, int* workgroups, int* slab_width, int* lds_bytes);

/* Static description of a status code (never NULL). */
const char* efla_status_string(efla_status s);

/* Text of the last HIP error seen by a call on this thread ("" if none). */
const char* efla_last_error(void);

/* ABI version of this library (major * 10000 + minor * 100 + patch). */
int efla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EFLA_H */
