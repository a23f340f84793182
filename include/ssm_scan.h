/*
 * ssm_scan.h -- C ABI of libssmscan.so, the MI355X (gfx950) selective-scan
 * library.
 *
 * Every entry point takes plain pointers and sizes.  Unless stated otherwise
 * a tensor pointer is a DEVICE pointer to a contiguous row-major array (last
 * index fastest) owned by the caller; the library never allocates device
 * memory, never frees caller memory and keeps no state between calls.  Work
 * is enqueued on `stream` (a hipStream_t; NULL means the default stream) and
 * the call returns without synchronising.  Arguments are validated on the
 * host before anything is enqueued; a rejected call has no side effects.
 * No entry point aborts the process: every failure is a status code.
 *
 * Notation follows the pages: B sequences (batch), L tokens, D channels
 * (d_inner), N states per channel (d_state); for Mamba-2 SSD, H heads of P
 * channels each and G groups of heads sharing B and C.
 *
 * Sources (page title, then the part of it that states the fact):
 * [mamba#285]  "Adding Initial Value Support to Selective Scan Forward Kernel"
 *              (state-spaces/mamba issue 285): the recurrence
 *              h_t = dA*h_{t-1} + Bx, the scan pair (exp(delta*A), state), and
 *              an initial state h0 of shape (B, D, N) entering as the pair
 *              (1, h0) -- the opening question and the running-prefix replies.
 * [ggml#6758]  "ggml : add GPU support for Mamba models" (llama.cpp issue
 *              6758): the SSM_SCAN op ggml_ssm_scan(s, x, dt, A, B, C) with
 *              tensors s {d_state, d_inner, n_seqs}, x/dt {d_inner,
 *              n_seq_tokens, n_seqs}, A {d_state, d_inner}, B/C {d_state,
 *              n_seq_tokens, n_seqs} (compilade's test patch, fastest
 *              dimension first); the ssm_d {d_inner} skip term (ctx_layer
 *              diff); silu(z) applied to the z half (jploski's silu report);
 *              inputs left unmodified with the final state returned as an
 *              output (compilade's follow-up); non-contiguous x/z views as a
 *              source of wrong results (slaren's ggml_cont diff).
 * [megatron#6444] "Clean up SSM ops directory structure - #6444": the decode
 *              op selective_state_update, the Mamba-2 state-space-duality
 *              kernels ssd_bmm, ssd_chunk_state, ssd_state_passing,
 *              ssd_chunk_scan, ssd_combined, the short causal
 *              convolution's causal_conv1d_update, the slot-indexed state
 *              gather/scatter (intermediate_extraction) and the
 *              batch-invariant decode.
 * [fastllm#333] "Tensor-parallel SSM #333": head groups (repeat_interleave of
 *              groups to heads) for Mamba-2.
 * [mixer2-tp]  "Current Implementation of TP in MambaMixer2": the number of
 *              groups divides the number of heads.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage dtype of x, delta (dt), z, Bm, Cm and y.  A, D_skip, h0, h_final
 * and the decode state are always fp32; arithmetic is fp32 throughout. */
typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype;

typedef enum {
    SSM_OK = 0,
    SSM_ERR_INVALID_ARG = 1, /* negative size, NULL required pointer, aliasing */
    SSM_ERR_UNSUPPORTED = 2, /* size outside what the kernels are built for   */
    SSM_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than required        */
    SSM_ERR_HIP = 4          /* a HIP launch failed (see hipGetLastError)      */
} ssm_status;

/* Kernel-variant selection for ssm_scan_fwd.  Pass NULL for the defaults.
 * The default schedule's results depend only on (L, D, N) -- never on B or
 * on the device -- so a sequence gives bitwise the same result whatever
 * batch it is part of.  (Within the channel-sequential schedule the
 * automatic choice also looks at the alignment of Bm and Cm, at B and at
 * the device's CU count; variants 1, 3 and 4 give bitwise identical
 * results.)  */
typedef struct {
    int32_t variant;   /* 0 = automatic; 1 = channel-sequential, a workgroup
                          per 64-channel tile whose waves split the N states;
                          2 = chunked over L (segment summaries, carry pass,
                          output pass); 3 = channel-sequential, the N states
                          of a channel split over 1, 2 or 4 lanes of one wave
                          (N in {4, 8, 16, 32, 64} and Bm, Cm 16-byte
                          aligned, else SSM_ERR_UNSUPPORTED); 4 = variant 3
                          with some waves' tokens cut in two at a 32-token
                          cycle, the second half continuing from the state
                          the first hands over through the workspace (also
                          L >= 64, else SSM_ERR_UNSUPPORTED; asked for
                          explicitly it cuts half of the 64-channel tiles).
                          Automatic: variant 3 where it applies, else 1,
                          when L <= 256 or D >= 4096 -- variant 4 instead of
                          3 when the waves exceed the device's SIMDs by at
                          most half their count, cutting just the excess so
                          every SIMD carries the same work; variant 2
                          otherwise. */
    int32_t chunk_len; /* variant 2: tokens per segment (multiple of 8,
                          >= 8); 0 = automatic (a multiple of 32).  With a
                          multiple of 32, states_per_lane 0 and the
                          conditions of variant 3, the segment passes run
                          on the lane-split kernel of variant 3, else on the
                          workgroup kernel of variant 1; the two give
                          bitwise the same result. */
    int32_t states_per_lane; /* 0 = automatic; else 2, 4, 8 or 16: each lane
                          keeps this many of a channel's N states and
                          ceil(N / states_per_lane) waves (1, 2, 4 or 8)
                          share a channel tile (the workgroup kernel) */
    int32_t reserved[5]; /* must be zero */
} ssm_tuning;

/* Optional transform of the step size before it enters the recurrence:
 * delta' = delta + bias[c] (bias may be NULL), then softplus(delta') =
 * log(1 + e^delta') when softplus == 1 -- Mamba's dt-projection bias and
 * softplus fused into the scan (the bias exists as a model tensor on the
 * llama.cpp page, [ggml#6758]).  c is the channel d for the Mamba-1 scan and
 * decode step, the head h for SSD.  Tokens past the end of a sequence are not
 * affected.  NULL options = delta used as given. */
typedef struct {
    const float *bias;   /* device pointer: (D) fp32, (H) for SSD; or NULL */
    int32_t softplus;    /* 0 or 1 */
    int32_t reserved[3]; /* must be zero */
} ssm_delta_opts;

/* Largest N the Mamba-1 kernels (scan and decode) are built for. */
#define SSM_SCAN_MAX_N 64
/* Largest N the SSD kernels are built for. */
#define SSM_SSD_MAX_N 256

/*
 * ssm_scan_fwd -- Mamba-1 selective scan over a prefill of L tokens.
 *
 * For every sequence b, channel d and state n ([mamba#285]):
 *   dA_t  = exp(delta[b,t,d] * A[d,n])
 *   dBx_t = delta[b,t,d] * Bm[b,t,n] * x[b,t,d]
 *   h_t   = dA_t * h_{t-1} + dBx_t,   h_0 = h0[b,d,n] (zeros if h0 == NULL)
 *   y[b,t,d] = (sum_n Cm[b,t,n] * h_t[n] + D_skip[d] * x[b,t,d])
 *              * silu(z[b,t,d])       (skip term only if D_skip != NULL,
 *                                      gate only if z != NULL; [ggml#6758])
 *   h_final[b,d,n] = h_L[n]
 * y_t uses the state after token t (inclusive scan).
 *
 * x, delta, z, y : (B, L, D), dtype `dt`
 * Bm, Cm         : (B, L, N), dtype `dt`
 * A              : (D, N) fp32;   D_skip : (D) fp32 or NULL
 * h0, h_final    : (B, D, N) fp32; either may be NULL (h_final NULL = not
 *                  returned).  h_final must not overlap h0 or any input.
 * y must not overlap any input.  Inputs are never modified.
 * workspace      : device scratch of at least ssm_scan_fwd_workspace_size()
 *                  bytes (may be NULL when that size is 0, which it is for
 *                  variants 1 and 3): the segment summaries of the chunked
 *                  schedule, the handed-over states and flags of variant 4.
 *                  Contents on entry are ignored (variant 4 clears its
 *                  flags with a kernel of its own); it must not overlap any
 *                  argument, and two calls that overlap in time must not
 *                  share it.
 * Sizes: B, L, D, N >= 0; N <= SSM_SCAN_MAX_N; one sequence's x plane
 * (L + 64) * D * sizeof(dtype) and B/C plane (L + 64) * N * sizeof(dtype)
 * below 2^31 bytes (else SSM_ERR_UNSUPPORTED).  L == 0 writes h_final = h0
 * (or zeros); B or D == 0 is a no-op; N == 0 leaves y = D_skip x silu(z).
 * Returns SSM_OK, SSM_ERR_INVALID_ARG, SSM_ERR_UNSUPPORTED,
 * SSM_ERR_WORKSPACE or SSM_ERR_HIP.
 */
ssm_status ssm_scan_fwd(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype dt,
                        const void *x, const void *delta, const float *A,
                        const void *Bm, const void *Cm, const float *D_skip,
                        const void *z, const float *h0, void *y, float *h_final,
                        void *workspace, size_t workspace_bytes,
                        const ssm_tuning *tuning, void *stream);

/* ssm_scan_fwd with the step-size transform of ssm_delta_opts (NULL = none).
 * The bias must not overlap y or h_final. */
ssm_status ssm_scan_fwd_ex(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype dt,
                           const void *x, const void *delta, const float *A,
                           const void *Bm, const void *Cm, const float *D_skip,
                           const void *z, const float *h0, void *y, float *h_final,
                           void *workspace, size_t workspace_bytes,
                           const ssm_tuning *tuning, const ssm_delta_opts *dopts,
                           void *stream);

/*
 * ssm_scan_fwd_noalloc -- ssm_scan_fwd_ex for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, results and schedule choice as
 * ssm_scan_fwd_ex, bitwise, without the workspace: where the chosen schedule
 * needs one (the chunked schedule's segment summaries, variant 4's state
 * handoff), it uses a device
 * scratch array that the library holds on every GPU it runs on, for the life
 * of the process.  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); the caller still passes inputs and outputs.
 *   limit : schedules needing more than 16 MiB of workspace
 *           (ssm_scan_fwd_workspace_size > 16777216) return
 *           SSM_ERR_WORKSPACE with nothing enqueued.
 *   races : every call on one GPU shares that GPU's scratch, which keeps the
 *           last call's contents (each call writes the entries it reads, so
 *           nothing needs clearing); calls that overlap in time on one GPU
 *           (other streams, other threads) race and must be serialised by the
 *           caller.
 * Errors as ssm_scan_fwd_ex; SSM_ERR_HIP if the scratch address cannot be
 * looked up on the current device.
 */
ssm_status ssm_scan_fwd_noalloc(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype dt,
                                const void *x, const void *delta, const float *A,
                                const void *Bm, const void *Cm, const float *D_skip,
                                const void *z, const float *h0, void *y, float *h_final,
                                const ssm_tuning *tuning, const ssm_delta_opts *dopts,
                                void *stream);

/*
 * ssm_scan_fwd_train -- ssm_scan_fwd_ex for a training step: also writes
 * h_ckpt (B, ceil(L/8), D, N) fp32, the state entering every 8-token segment
 * (segment 0: h0), which ssm_scan_bwd then reads instead of recomputing
 * them (the mamba page's backward recomputes the forward states; here the
 * forward keeps them at segment boundaries).  Always the lane-split
 * schedule: N in {4, 8, 16, 32, 64}, Bm and Cm 16-byte aligned, x, delta, z,
 * y aligned to two elements, D even, h_ckpt 16-byte aligned (else
 * SSM_ERR_UNSUPPORTED).  y and h_final are bitwise those of ssm_scan_fwd_ex
 * with tuning variant 3.  h_ckpt must not overlap any other argument.
 */
ssm_status ssm_scan_fwd_train(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype dt,
                              const void *x, const void *delta, const float *A,
                              const void *Bm, const void *Cm, const float *D_skip,
                              const void *z, const float *h0, void *y, float *h_final,
                              float *h_ckpt, const ssm_delta_opts *dopts, void *stream);

/* Device workspace ssm_scan_fwd needs for these sizes and tuning (bytes);
 * it may depend on the current device (variant 4 is chosen from its CU
 * count). */
size_t ssm_scan_fwd_workspace_size(int64_t B, int64_t L, int64_t D, int64_t N,
                                   const ssm_tuning *tuning);

/*
 * ssm_state_update -- one decode step for S independent sequences
 * (selective_state_update, [megatron#6444]): the ssm_scan_fwd body with
 * L = 1, the state read and written IN PLACE.
 *
 * state          : (S, D, N) fp32, in/out
 * x, delta, z, y : (S, D), dtype `dt`;  Bm, Cm : (S, N), dtype `dt`
 * A              : (D, N) fp32;  D_skip : (D) fp32 or NULL;  z may be NULL.
 * y must not overlap any input or the state.  Sizes as ssm_scan_fwd.
 */
ssm_status ssm_state_update(int64_t S, int64_t D, int64_t N, ssm_dtype dt,
                            float *state, const void *x, const void *delta,
                            const float *A, const void *Bm, const void *Cm,
                            const float *D_skip, const void *z, void *y,
                            void *stream);

/* ssm_state_update with the step-size transform of ssm_delta_opts. */
ssm_status ssm_state_update_ex(int64_t S, int64_t D, int64_t N, ssm_dtype dt,
                               float *state, const void *x, const void *delta,
                               const float *A, const void *Bm, const void *Cm,
                               const float *D_skip, const void *z, void *y,
                               const ssm_delta_opts *dopts, void *stream);

/*
 * ssm_scan_bwd -- gradients of ssm_scan_fwd_ex (training).
 *
 * The backward of [mamba#285] (replies on the backward kernel): the states
 * are recomputed forward, the gradient of the state is carried backwards by
 * a reverse scan fed with dy * C and decayed by exp(delta * A) from token to
 * token, and the gradient of the initial state is exp(delta_0 * A) times the
 * carried gradient at the first token.  With y the gated output of
 * ssm_scan_fwd_ex and h_final its final state, for the loss gradients dy
 * (B, L, D) and dh_final (B, D, N) (NULL = zero) this returns the outputs
 * below.  h_ckpt: the segment states ssm_scan_fwd_train wrote for the same
 * inputs (16-byte aligned), or NULL to recompute them here (into the
 * workspace, by the prefill scan's kernel where it takes the shape: even D,
 * x and delta aligned to two elements, Bm and the workspace 16-byte
 * aligned; the gradients are then bitwise those computed from
 * ssm_scan_fwd_train's states; otherwise by the backward kernel itself).
 *   dx, ddelta, dz : (B, L, D) dtype `dt` (ddelta is the gradient of the
 *                    delta INPUT, i.e. through bias and softplus when dopts
 *                    asks for them; dz only with z, else must be NULL)
 *   dA             : (D, N) fp32;   dB, dC : (B, L, N) fp32
 *   dD             : (D) fp32, written when D_skip and dD are both non-NULL
 *   dh0            : (B, D, N) fp32 or NULL (not returned)
 *   d_delta_bias   : (D) fp32 or NULL (not returned): the sum of ddelta
 * Every output is overwritten (not accumulated).  Sums over channels and
 * over tokens are taken in a fixed order: results are run-to-run
 * reproducible.  Inputs as ssm_scan_fwd_ex (dy in dtype `dt`); A, h0,
 * dh_final, dh0 and the workspace 16-byte aligned.  N in {4, 8, 16, 32, 64}
 * (else SSM_ERR_UNSUPPORTED).  Outputs must not overlap inputs, the
 * workspace or each other.
 * workspace : at least ssm_scan_bwd_workspace_size_ex(B, L, D, N,
 *             h_ckpt != NULL) bytes: the states entering every 8-token
 *             segment (B * ceil(L/8) * D * N fp32, 1.34 GB at B=8, L=4096,
 *             D=5120, N=16; left out when h_ckpt is given) plus
 *             per-channel-tile partial sums; contents on entry are ignored.
 */
ssm_status ssm_scan_bwd(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype dt,
                        const void *x, const void *delta, const float *A,
                        const void *Bm, const void *Cm, const float *D_skip,
                        const void *z, const float *h0, const void *dy,
                        const float *dh_final, const float *h_ckpt, void *dx,
                        void *ddelta, void *dz,
                        float *dA, float *dB, float *dC, float *dD, float *dh0,
                        float *d_delta_bias, const ssm_delta_opts *dopts,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Device workspace ssm_scan_bwd needs when it recomputes the segment states
 * (h_ckpt == NULL); bytes, 0 for unsupported N.  Equal to
 * ssm_scan_bwd_workspace_size_ex(B, L, D, N, 0). */
size_t ssm_scan_bwd_workspace_size(int64_t B, int64_t L, int64_t D, int64_t N);

/* Device workspace ssm_scan_bwd needs; saved_states = 1 when the call passes
 * the forward's segment states (h_ckpt != NULL), which then take no
 * workspace; 0 otherwise.  0 for unsupported N or a saved_states other than
 * 0 or 1. */
size_t ssm_scan_bwd_workspace_size_ex(int64_t B, int64_t L, int64_t D, int64_t N,
                                      int32_t saved_states);

/*
 * ssm_decode_steps -- T decode tokens for each of S sequences whose states
 * live in a pool of rows (the slot-indexed state gather/scatter of prefix
 * caching, intermediate_extraction, and the batch-invariant decode of
 * [megatron#6444]).  Sequence s reads and writes the state row
 * slot_idx[s] of state_pool IN PLACE; its T tokens go through the decode
 * step in order with the state kept on chip between them, so T = 1 is one
 * decode step and T > 1 reads and writes the state once for T tokens.  For
 * T <= 4 the results are bitwise those of T successive ssm_state_update
 * calls; longer calls run the prefill scan's kernels (bitwise ssm_scan_fwd
 * with tuning variant 1 and h0 = h_final = the gathered rows).  A sequence's
 * results do not depend on which other sequences share the call.
 *
 * state_pool : (pool_rows, D, N) fp32, in/out
 * slot_idx   : (S) int32 DEVICE array, or NULL for slot s = s (then
 *              pool_rows >= S).  Slots outside [0, pool_rows) skip the
 *              sequence (its y rows are not written); with pool_rows == 0
 *              every sequence is skipped and nothing is enqueued.
 *              Non-negative slots must be distinct: two sequences on one
 *              row race.
 * x, delta, z, y : (S, T, D) dtype `dt`;  Bm, Cm : (S, T, N) dtype `dt`
 * A : (D, N) fp32;  D_skip : (D) or NULL;  z may be NULL;  dopts as
 * ssm_scan_fwd_ex.  y must not overlap the inputs or the pool; the pool must
 * not overlap the inputs.  Sizes as ssm_scan_fwd with L = T.
 */
ssm_status ssm_decode_steps(int64_t S, int64_t T, int64_t D, int64_t N, ssm_dtype dt,
                            float *state_pool, int64_t pool_rows, const int32_t *slot_idx,
                            const void *x, const void *delta, const float *A,
                            const void *Bm, const void *Cm, const float *D_skip,
                            const void *z, void *y, const ssm_delta_opts *dopts,
                            void *stream);

/*
 * ssm_ssd_fwd -- Mamba-2 state-space-duality (SSD) chunked scan
 * (ssd_combined and the kernels it drives, [megatron#6444]).
 *
 * Per sequence b, head h, channel p < P and state n, with group
 * g = h / (H / G) ([fastllm#333], [mixer2-tp]):
 *   dA_t  = exp(dt[b,t,h] * A[h])                  (scalar per head)
 *   h_t[p,n] = dA_t * h_{t-1}[p,n] + dt[b,t,h] * Bm[b,t,g,n] * x[b,t,h,p]
 *   y[b,t,h,p] = (sum_n Cm[b,t,g,n] h_t[p,n] + D_skip[h] x[b,t,h,p])
 *                * silu(z[b,t,h,p])
 * Two paths, chosen from the shape alone:
 *  - matrix cores: bf16 inputs, P == 64, N a multiple of 32 (32 .. 256),
 *    chunk in {64, 128, 256}, and x, Bm, Cm, h0, h_final and the workspace
 *    16-byte aligned.  Computed chunk by chunk (`chunk` tokens):
 *    intra-chunk products on the matrix cores with computed operands split
 *    into bf16 hi + lo, chunk states passed sequentially in fp32 from h0.
 *    Needs ssm_ssd_fwd_workspace_size() bytes of workspace.
 *  - every other shape with N <= SSM_SSD_MAX_N (fp32 inputs, any P, any
 *    N, any chunk >= 1, any alignment): the recurrence token by token on
 *    the vector ALU in fp32; the result does not depend on `chunk`; no
 *    workspace (workspace may be NULL).
 * x, z, y   : (B, L, H, P) dtype `dt`;  dt_in : (B, L, H) dtype `dt`
 * Bm, Cm    : (B, L, G, N) dtype `dt`;  A, D_skip : (H) fp32 (D_skip may be NULL)
 * h0, h_final : (B, H, P, N) fp32 or NULL.  z may be NULL.
 * SSM_ERR_UNSUPPORTED: N > SSM_SSD_MAX_N, chunk < 1, H % G != 0.  Any
 * L >= 0 (a ragged last chunk is handled).
 */
ssm_status ssm_ssd_fwd(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                       int64_t N, int64_t chunk, ssm_dtype dt, const void *x,
                       const void *dt_in, const float *A, const void *Bm,
                       const void *Cm, const float *D_skip, const void *z,
                       const float *h0, void *y, float *h_final,
                       void *workspace, size_t workspace_bytes, void *stream);

/* ssm_ssd_fwd with the step-size transform of ssm_delta_opts (bias per head). */
ssm_status ssm_ssd_fwd_ex(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                          int64_t N, int64_t chunk, ssm_dtype dt, const void *x,
                          const void *dt_in, const float *A, const void *Bm,
                          const void *Cm, const float *D_skip, const void *z,
                          const float *h0, void *y, float *h_final,
                          void *workspace, size_t workspace_bytes,
                          const ssm_delta_opts *dopts, void *stream);

/* Workspace of the matrix-core path for these sizes (bytes); 0 where that
 * path does not apply (the token-by-token path needs none). */
size_t ssm_ssd_fwd_workspace_size(int64_t B, int64_t L, int64_t H, int64_t P,
                                  int64_t G, int64_t N, int64_t chunk);

/*
 * ssm_conv1d_fwd -- the short causal convolution that precedes the scan
 * (ggml's SSM_CONV, [ggml#6758]: ggml_ssm_conv(s, x, c) with the state s
 * holding each channel's d_conv - 1 previous inputs and the conv bias
 * ssm_conv1d_b), over a prefill of L tokens.  For every b, d, with
 * xp = [state_in[b,d,:], x[b,0,d], ..., x[b,L-1,d]]:
 *   y[b,t,d] = act(sum_{k<K} w[d,k] * xp[t+k] + bias[d])
 *   state_out[b,d,j] = xp[L + j],  j < K - 1   (the last K - 1 entries)
 * act is the identity (activation == 0) or SiLU (activation == 1).
 *
 * x, y           : (B, L, D), dtype `dt`
 * w              : (D, K) fp32;  bias : (D) fp32 or NULL
 * state_in       : (B, D, K-1) fp32, oldest first, or NULL (zeros)
 * state_out      : (B, D, K-1) fp32 or NULL (not returned)
 * y must not overlap x, w, bias or the states; state_out must not overlap
 * state_in (the segments of L run in parallel).  2 <= K <= 8.  L == 0 only
 * writes state_out.  Sizes as ssm_scan_fwd (the (L + 64) * D plane limit).
 */
ssm_status ssm_conv1d_fwd(int64_t B, int64_t L, int64_t D, int64_t K, ssm_dtype dt,
                          const void *x, const float *w, const float *bias,
                          const float *state_in, int32_t activation, void *y,
                          float *state_out, void *stream);

/*
 * ssm_conv1d_update -- one decode step of the causal convolution for S
 * sequences (causal_conv1d_update, [megatron#6444]): window = [state, x],
 * y = act(sum_k w[d,k] window[k] + bias[d]), and the state drops its oldest
 * entry and appends x, IN PLACE.
 *
 * state : (S, D, K-1) fp32 in/out;  x, y : (S, D) dtype `dt`
 * w : (D, K) fp32;  bias : (D) fp32 or NULL.  y must not overlap the other
 * arguments.  2 <= K <= 8 and S <= 65535 (else SSM_ERR_UNSUPPORTED).
 */
ssm_status ssm_conv1d_update(int64_t S, int64_t D, int64_t K, ssm_dtype dt, float *state,
                             const void *x, const float *w, const float *bias,
                             int32_t activation, void *y, void *stream);

/* Static description of a status code. */
const char *ssm_status_string(ssm_status s);

/* Library version, major*10000 + minor*100 + patch. */
int ssm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H */
