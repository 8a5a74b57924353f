/*
 * ssm_mi355x.h -- C ABI of the MI355X (gfx950) selective-scan + causal-conv1d library.
 *
 * The library computes a Mamba-2-style selective state-space scan with an explicit initial
 * state in and the final state out, fused with its causal depthwise conv1d front end that
 * carries a K-1 input history, plus the two decode-time updates.  Sources, cited by page
 * title and section:
 *
 *   [LG] "Understanding and Improving Length Generalization in Recurrent Models" -- reading
 *        notes on arXiv:2507.02782v2.  Sec. 2.1, Eq. (1): h_t = A_t h_{t-1} + B_t x_t,
 *        y_t = C_t^T h_t with initial state h_{-1}.  Sec. 2.5, Eq. (4): the unrolling with a
 *        non-zero h_{-1} and the note that the transition enters in log space.  Sec. 2.6:
 *        State Passing / TBTT (the final state of one call is the initial state of the next).
 *   [CC] Causal-conv1d tutorial, chapter 7 "State, chunking and incremental inference":
 *        "defining the state through the extended sequence" (u = [S, x], z_t, F);
 *        "chunked training and truncated backprop" (S_B = F_A); "single-token update
 *        maths"; "the physical cache may exceed the minimal history" (state_len, circular
 *        mode through cache_seqlens); "state indices for continuous batching"
 *        (conv_state_indices); "packed-sequence boundaries" (seq_idx).
 *
 * Conventions shared by every call
 *   - All array arguments are DEVICE pointers owned by the caller, laid out contiguously
 *     (row-major) exactly as stated, unless explicit strides are given.  Inputs are const.
 *   - The library allocates nothing per call and keeps no state between calls except the
 *     loaded kernels, the thread-local error text and the optional timing events.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default stream) and
 *     never synchronises.  Host-side argument errors return a status and enqueue nothing.
 *   - dtype is the storage type of the activations (x, B, C, conv states, outputs):
 *     SSM_F32 or SSM_BF16.  Weights, bias, dt and A are fp32; SSM states are fp32.
 *     Floating point outputs are rounded once to the storage type (round to nearest even).
 *   - Integer index arrays are int32.  Sizes are int64.
 *   - Permitted aliasing: final_state == initial_state (in-place state passing), for the
 *     conv pair and for the SSM pair.  Pools are updated in place.  No other aliasing.
 *   - Nothing throws, aborts or prints.  ssm_last_error() gives the detail of the last
 *     failure on the calling thread.
 */
#ifndef SSM_MI355X_H
#define SSM_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 4

/* hipStream_t is `struct ihipStream_t*`; this typedef is the same type. */
struct ihipStream_t;
typedef struct ihipStream_t* ssm_stream_t;

typedef enum {
    SSM_OK = 0,
    SSM_ERR_INVALID_ARG = 1, /* NULL required pointer, bad size, bad enum, H % G != 0 ... */
    SSM_ERR_UNSUPPORTED = 2, /* valid arguments outside what the kernels implement */
    SSM_ERR_ALIGNMENT = 3,   /* a pointer not aligned to its element size */
    SSM_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than the query returned */
    SSM_ERR_HIP = 5          /* a HIP launch/runtime error; see ssm_last_error() */
} ssm_status_t;

/* Element type codes.  The parameter type is a plain 32-bit integer, not the enum, so that a
   caller may pass any value and get SSM_ERR_INVALID_ARG back for one outside the list (an enum
   object holding a value outside its enumerators' range is undefined behaviour in C++). */
enum { SSM_F32 = 0, SSM_BF16 = 1 };
typedef int32_t ssm_dtype_t;

/* phi of [CC] "single-token update maths": identity or SiLU(z) = z / (1 + exp(-z)).  A plain
   32-bit integer for the same reason as ssm_dtype_t. */
enum { SSM_ACT_NONE = 0, SSM_ACT_SILU = 1 };
typedef int32_t ssm_act_t;

/* Library ABI version (SSM_ABI_VERSION of the build). */
int ssm_abi_version(void);
/* Static English text for a status code; "unknown status" for any other integer. */
const char* ssm_status_string(int32_t status);
/* Detail of the last failure on the calling thread ("" if none).  Valid until the next call
 * on the same thread. */
const char* ssm_last_error(void);

/* ---------------------------------------------------------------------------------------
 * ssm_conv1d_fwd -- causal depthwise conv1d with state in / out.
 * Defined in [CC] "defining the state through the extended sequence": with
 * u = [S_0 .. S_{K-2}, x_0 .. x_{L-1}] (S oldest first, zeros when absent),
 *     out_t = phi(bias + sum_{k<K} w_k u_{t+k}),     F = u[L : L+K-1]  (raw copy).
 * seq_idx ([CC] "packed-sequence boundaries"): a tap contributes only when its token has
 * the same id as the output token (S carries the id of token 0); F stays unmasked.
 *
 *   x             [batch, seqlen, channels]   dtype, channel-last
 *   w             [channels, width]           fp32 (w[c][width-1] multiplies x_t)
 *   bias          [channels]                  fp32, or NULL (= 0)
 *   initial_state [batch, channels, width-1]  dtype, or NULL (= zeros)
 *   final_state   [batch, channels, width-1]  dtype, or NULL (not written); may alias
 *                                             initial_state
 *   seq_idx       [batch, seqlen]             int32, or NULL (one sequence per row)
 *   out           [batch, seqlen, channels]   dtype
 * width in [2, 8]; seqlen = 0 is legal (final_state = initial_state); batch = 0 is a no-op.
 * ------------------------------------------------------------------------------------- */
ssm_status_t ssm_conv1d_fwd(const void* x, const float* w, const float* bias,
                            const void* initial_state, void* final_state,
                            const int32_t* seq_idx, void* out, int64_t batch, int64_t seqlen,
                            int64_t channels, int64_t width, ssm_dtype_t dtype, ssm_act_t act,
                            ssm_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * ssm_conv1d_update -- decode-time update of the conv state pool, n_new >= 1 new tokens.
 * Defined in [CC] "single-token update maths", "the physical cache may exceed the minimal
 * history" and "state indices for continuous batching".  Row b uses pool slot
 * s = conv_state_indices[b] (b when NULL).  The K-1 history values are read before
 * anything is overwritten:
 *   circular (cache_seqlens != NULL, p = cache_seqlens[b]): history j steps back is slot
 *       (p - j) mod state_len (non-negative remainder); new token i goes to slot
 *       (p + i) mod state_len;
 *   linear (cache_seqlens == NULL): the row holds the newest state_len inputs, oldest
 *       first; the history is its last K-1 entries; afterwards the row is the last
 *       state_len entries of (old row ++ new tokens).
 * out_i = phi(bias + sum_k w_k u_{i+k}) over u = [history, new tokens].  The pool stores
 * the raw inputs, never the outputs.  cache_seqlens is read, never advanced: the caller
 * adds n_new afterwards.
 *
 *   x                  [batch, channels, n_new]           dtype
 *   conv_state         [n_slots, channels, state_len]     dtype, in / out
 *   w, bias            as ssm_conv1d_fwd
 *   conv_state_indices [batch] int32, or NULL
 *   cache_seqlens      [batch] int32 (>= 0), or NULL (linear mode)
 *   out                [batch, channels, n_new]           dtype
 * state_len >= width-1.  A row whose slot is outside [0, n_slots) is skipped: its out row
 * is zero-filled and the pool is not touched.  Two rows on the same slot: undefined (a
 * caller-contract error); a reused slot must have been initialised by the caller.
 * ------------------------------------------------------------------------------------- */
ssm_status_t ssm_conv1d_update(const void* x, void* conv_state, const float* w,
                               const float* bias, const int32_t* conv_state_indices,
                               const int32_t* cache_seqlens, void* out, int64_t batch,
                               int64_t channels, int64_t n_new, int64_t width,
                               int64_t state_len, int64_t n_slots, ssm_dtype_t dtype,
                               ssm_act_t act, ssm_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * Workspace bytes that ssm_scan_fwd / ssm_conv_scan_fwd need for these sizes (0 if none).
 * ------------------------------------------------------------------------------------- */
size_t ssm_scan_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                               int64_t ngroups, int64_t dstate, ssm_dtype_t dtype);

/* ---------------------------------------------------------------------------------------
 * ssm_scan_fwd -- selective scan with initial state in, final state out.
 * Defined in [LG] Sec. 2.1 Eq. (1) and Sec. 2.5 Eq. (4), per head h (group
 * g = h / (nheads / ngroups)) and channel p:
 *     a_t = exp(dt[t,h] * A[h])
 *     state_t[p,:] = a_t * state_{t-1}[p,:] + dt[t,h] * x[t,h,p] * B[t,g,:]
 *     y[t,h,p] = C[t,g,:] . state_t[p,:]
 * starting from state_{-1} = initial_state (zeros when NULL); final_state = state_{L-1}.
 * seq_idx: the state restarts from zero where seq_idx[b,t] != seq_idx[b,t-1].
 *
 *   x             [batch, seqlen, nheads, headdim]   dtype
 *   dt            [batch, seqlen, nheads]            fp32 (used as given, no softplus)
 *   A             [nheads]                           fp32
 *   Bm, Cm        [batch, seqlen, ngroups, dstate]   dtype
 *   initial_state [batch, nheads, headdim, dstate]   fp32, or NULL
 *   final_state   [batch, nheads, headdim, dstate]   fp32, or NULL; may alias initial_state
 *   seq_idx       [batch, seqlen] int32, or NULL
 *   y             [batch, seqlen, nheads, headdim]   dtype
 *   workspace     device scratch of >= ssm_scan_workspace_size(...) bytes (NULL if 0)
 * bf16 with headdim 64 and dstate 128 runs chunked on the matrix cores when x, Bm and Cm are
 * 16-byte and y 8-byte aligned (the workspace is then required); other shapes, fp32 and
 * other alignments run token-sequentially (same results to rounding).
 * ------------------------------------------------------------------------------------- */
ssm_status_t ssm_scan_fwd(const void* x, const float* dt, const float* A, const void* Bm,
                          const void* Cm, const float* initial_state, float* final_state,
                          const int32_t* seq_idx, void* y, int64_t batch, int64_t seqlen,
                          int64_t nheads, int64_t headdim, int64_t ngroups, int64_t dstate,
                          ssm_dtype_t dtype, void* workspace, size_t workspace_bytes,
                          ssm_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * ssm_decode_step -- one decode step of a layer on its pools: ssm_conv1d_update over the
 * x | B | C channels of x_new, then ssm_step reading the channel ranges of that conv output.
 * [CC] "single-token update maths" (the ring cache, the K-1 inputs before position p) and
 * "state indices for continuous batching"; [LG] Sec. 2.1 Eq. (1) for the state update.
 * Results are exactly those of the two calls in sequence (same roundings, same bits).
 *
 *   x_new              [batch, C, n_new]  dtype, C = nheads*headdim + 2*ngroups*dstate
 *   conv_state         [n_conv_slots, C, state_len]  dtype, updated in place as by
 *                      ssm_conv1d_update (circular with cache_seqlens, else linear)
 *   conv_w, conv_bias  [C, width], [C] fp32 (bias may be NULL)
 *   conv_state_indices [batch] int32 slot of each row in conv_state, or NULL (= row)
 *   cache_seqlens      [batch] int32 ring positions, or NULL (linear layout); read only
 *   dt                 [batch, n_new, nheads] fp32;  A  [nheads] fp32
 *   ssm_state          [n_ssm_slots, nheads, headdim, dstate] fp32, 16-byte aligned,
 *                      updated in place
 *   state_indices      [batch] int32 slot of each row in ssm_state, or NULL (= the conv
 *                      slot, conv_state_indices)
 *   conv_out           [batch, C, n_new] dtype, written (the conv outputs)
 *   y                  [batch, n_new, nheads, headdim] dtype
 * Rows whose slot lies outside a pool are handled as by the two calls (zero conv outputs /
 * zero y, that pool untouched).  Two rows naming one slot of a pool race (caller contract).
 * Runs the two kernels of those calls back to back on `stream` (one entry, one argument
 * check); the conv output is the step's input, so conv_out is required.
 * ------------------------------------------------------------------------------------- */
ssm_status_t ssm_decode_step(const void* x_new, void* conv_state, const float* conv_w,
                             const float* conv_bias, const int32_t* conv_state_indices,
                             const int32_t* cache_seqlens, const float* dt, const float* A,
                             float* ssm_state, const int32_t* state_indices, void* conv_out,
                             void* y, int64_t batch, int64_t n_new, int64_t nheads,
                             int64_t headdim, int64_t ngroups, int64_t dstate, int64_t width,
                             int64_t state_len, int64_t n_conv_slots, int64_t n_ssm_slots,
                             ssm_dtype_t dtype, ssm_act_t act, ssm_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * ssm_scan_fwd_vector_decay -- the scan with a diagonal transition, one decay per state
 * dimension ([LG] Sec. 2.1 Eq. (1) with A_t = diag(a_t); Sec. 2.5, the diagonal case taken
 * from log transition coefficients), per head h, channel p and state dimension n:
 *     state[p][n] <- a_t[n] state[p][n] + u_t x_t[p] B_t[n],   y_t[p] = C_t . state[p][:]
 * with log a_t[n] = log_decay[b][t][h][n] (data-dependent gates) or dt_t[h] A_vec[h][n] (a
 * fixed rate per dimension), and u_t = dt_t[h] (1 when dt is NULL).  Initial / final state
 * and seq_idx resets as ssm_scan_fwd.
 *
 *   x, y           [batch, seqlen, nheads, headdim]   dtype
 *   dt             [batch, seqlen, nheads] fp32, or NULL (= 1; not with A_vec)
 *   log_decay      [batch, seqlen, nheads, dstate] fp32 (<= 0 for a contraction), or NULL
 *   A_vec          [nheads, dstate] fp32, or NULL -- exactly one of log_decay, A_vec
 *   B, C           [batch, seqlen, ngroups, dstate]   dtype
 *   initial_state, final_state  [batch, nheads, headdim, dstate] fp32, 16-byte aligned, or
 *                  NULL; final_state may alias initial_state
 *   seq_idx        [batch, seqlen] int32, or NULL
 * dstate = 4 * 2^k <= 256, headdim * dstate <= 16384.  The gate form (log_decay) with bf16,
 * headdim 64, dstate 128, contiguous 16-byte aligned rows and states runs chunked on the
 * matrix cores (64-token chunks, [LG] Sec. 2.5: the decay over a span is the exponential of
 * a sum of log coefficients; a chunk whose summed log decay leaves +-40 runs token by
 * token); other bf16 shapes with headdim 64 and dstate 64 or 128 (and the A_vec form) run a
 * token-sequential long-row kernel, the rest the general token-sequential one (all agree to
 * rounding).  seqlen = 0: final_state = initial_state (or zero).
 * ------------------------------------------------------------------------------------- */
ssm_status_t ssm_scan_fwd_vector_decay(const void* x, const float* dt, const float* log_decay,
                                       const float* A_vec, const void* B, const void* C,
                                       const float* initial_state, float* final_state,
                                       const int32_t* seq_idx, void* y, int64_t batch,
                                       int64_t seqlen, int64_t nheads, int64_t headdim,
                                       int64_t ngroups, int64_t dstate, ssm_dtype_t dtype,
                                       ssm_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * ssm_conv_scan_fwd -- the fused prefill: ssm_conv1d_fwd over the channels of xBC (with
 * phi; its output rounded to dtype exactly as the standalone call would store it), split
 * into x | B | C channel ranges, then ssm_scan_fwd.  One pass over HBM for x.  The conv is
 * the extended-sequence definition with its carried state ([CC] ch. 7, "defining the state
 * through the extended sequence"); the scan is [LG] Sec. 2.1 Eq. (1) started from the
 * initial state (Sec. 2.5 Eq. (4)) and returning the final state (Sec. 2.6 State Passing).
 *
 *   xBC                [batch, seqlen, nheads*headdim + 2*ngroups*dstate]  dtype;
 *                      channels [0, H*P) are x (head-major), then B (group-major), then C
 *   conv_w, conv_bias  [C_conv, width], [C_conv] fp32 (bias may be NULL)
 *   conv_initial_state, conv_final_state   [batch, C_conv, width-1] dtype, or NULL
 *   dt, A, initial_state, final_state, seq_idx, y, workspace: as ssm_scan_fwd
 *   (seq_idx also masks the conv taps as in ssm_conv1d_fwd)
 * ------------------------------------------------------------------------------------- */
ssm_status_t ssm_conv_scan_fwd(const void* xBC, const float* conv_w, const float* conv_bias,
                               const void* conv_initial_state, void* conv_final_state,
                               const float* dt, const float* A, const float* initial_state,
                               float* final_state, const int32_t* seq_idx, void* y,
                               int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                               int64_t ngroups, int64_t dstate, int64_t width,
                               ssm_dtype_t dtype, ssm_act_t act, void* workspace,
                               size_t workspace_bytes, ssm_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * ssm_conv_scan_fwd_noalloc -- ssm_conv_scan_fwd for callers that cannot allocate device
 * memory (code under stream/graph capture, tight serving loops, hosts that forbid
 * hipMalloc): the same operation, arguments and results, minus the workspace, which is a
 * static device array of the library, ssm_noalloc_scratch_bytes() = 32 MiB per GPU, created
 * when the library is first used on that GPU and held until the process ends.  The call
 * allocates nothing: no hipMalloc / hipFree, no allocating library routine, and no timing
 * events even while ssm_timing_enable is on.
 *   - Sizes whose ssm_scan_workspace_size exceeds the scratch return SSM_ERR_WORKSPACE.  On
 *     the matrix-core path that is 48 KiB per 64-token chunk per row and group, plus the
 *     segment states of rows split across blocks (1.3B-like layer, batch 4 x 8192 tokens:
 *     24 MiB; batch 1 x 8192: 14 MiB; one 131072-token row: 104 MiB, rejected).
 *   - The scratch belongs to the current device (hipGetDevice); `stream` must be a stream of
 *     that device.  The first call on a device looks its address up (hipGetSymbolAddress).
 *   - Every call on one GPU shares that GPU's scratch: calls that may overlap in time on one
 *     GPU (different streams, or several host threads) race and give wrong results; order
 *     them on one stream.  No part of the scratch needs clearing between calls: each call
 *     writes every byte it reads before reading it.
 * ------------------------------------------------------------------------------------- */
size_t ssm_noalloc_scratch_bytes(void);
ssm_status_t ssm_conv_scan_fwd_noalloc(const void* xBC, const float* conv_w,
                                       const float* conv_bias, const void* conv_initial_state,
                                       void* conv_final_state, const float* dt, const float* A,
                                       const float* initial_state, float* final_state,
                                       const int32_t* seq_idx, void* y, int64_t batch,
                                       int64_t seqlen, int64_t nheads, int64_t headdim,
                                       int64_t ngroups, int64_t dstate, int64_t width,
                                       ssm_dtype_t dtype, ssm_act_t act, ssm_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * ssm_conv_scan_fwd_pooled -- the fused prefill reading its initial states from, and writing
 * its final states to, the decode pools, so a request moves from prefill to decode (or to its
 * next prefill chunk) without dense state copies.  [CC] "the physical cache may exceed the
 * minimal history", "state indices for continuous batching" and the chapter's closing
 * distinction between choosing another request's history (the slot), blocking history across
 * packed samples (seq_idx) and continuing one request's history (the ring position).
 * Row b uses slot s = state_indices[b] (b when NULL):
 *   conv history = ssm_conv1d_update's: circular (cache_seqlens != NULL, p = cache_seqlens[b])
 *     slots (p - j) mod state_len, j = K-1 .. 1 (oldest first); linear: the row's last K-1;
 *   SSM initial state = ssm_state[s];
 *   then ssm_conv_scan_fwd over the row's L tokens, and afterwards, as ssm_conv1d_update
 *   would leave them: circular: token i in slot (p + i) mod state_len; linear: the row is the
 *   last state_len entries of (old row ++ new tokens); ssm_state[s] = the final state.
 * cache_seqlens is read, never advanced (the caller adds seqlen).  A row whose slot is outside
 * [0, n_slots) runs from zero states and stores nothing; two rows on one slot: undefined.
 *
 *   xBC, conv_w, conv_bias, dt, A, seq_idx, y    as ssm_conv_scan_fwd
 *   conv_state      [n_slots, C_conv, state_len]     dtype, in / out (state_len >= width-1)
 *   ssm_state       [n_slots, nheads, headdim, dstate] fp32, in / out
 *   state_indices   [batch] int32, or NULL;  cache_seqlens [batch] int32 (>= 0), or NULL
 *   workspace       ssm_conv_scan_fwd_pooled_workspace_size bytes, 256-byte aligned
 * ------------------------------------------------------------------------------------- */
size_t ssm_conv_scan_fwd_pooled_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads,
                                               int64_t headdim, int64_t ngroups, int64_t dstate,
                                               int64_t width, ssm_dtype_t dtype);
ssm_status_t ssm_conv_scan_fwd_pooled(const void* xBC, const float* conv_w,
                                      const float* conv_bias, const float* dt, const float* A,
                                      void* conv_state, float* ssm_state,
                                      const int32_t* state_indices, const int32_t* cache_seqlens,
                                      const int32_t* seq_idx, void* y, int64_t batch,
                                      int64_t seqlen, int64_t nheads, int64_t headdim,
                                      int64_t ngroups, int64_t dstate, int64_t width,
                                      int64_t state_len, int64_t n_slots, ssm_dtype_t dtype,
                                      ssm_act_t act, void* workspace, size_t workspace_bytes,
                                      ssm_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * ssm_step -- decode-time scan update on a state pool, n_new >= 1 tokens per request.
 * Same recurrence as ssm_scan_fwd ([LG] Eq. (1)), token by token, on pool slot
 * s = state_indices[b] (b when NULL); the state is kept in fp32 registers across the n_new
 * tokens and written back once.  A row whose slot is outside [0, n_slots) is skipped: its
 * y rows are zero-filled and the pool is not touched.  Two rows on one slot: undefined.
 *
 *   x   element (b, t, h, p) at x[b*x_sb + t*x_st + (h*headdim + p)*x_sc]     dtype
 *   Bm  element (b, t, g, n) at Bm[b*B_sb + t*B_st + (g*dstate + n)*B_sc]     dtype
 *   Cm  element (b, t, g, n) at Cm[b*C_sb + t*C_st + (g*dstate + n)*C_sc]     dtype
 *       (strides in elements: contiguous [batch, n_new, ...] inputs and the
 *       [batch, channels, n_new] output of ssm_conv1d_update both fit)
 *   dt     [batch, n_new, nheads] fp32;   A [nheads] fp32
 *   state  [n_slots, nheads, headdim, dstate] fp32, in / out
 *   state_indices [batch] int32, or NULL
 *   y      [batch, n_new, nheads, headdim] dtype
 * ------------------------------------------------------------------------------------- */
ssm_status_t ssm_step(const void* x, int64_t x_sb, int64_t x_st, int64_t x_sc, const float* dt,
                      const float* A, const void* Bm, int64_t B_sb, int64_t B_st, int64_t B_sc,
                      const void* Cm, int64_t C_sb, int64_t C_st, int64_t C_sc, float* state,
                      const int32_t* state_indices, void* y, int64_t batch, int64_t n_new,
                      int64_t nheads, int64_t headdim, int64_t ngroups, int64_t dstate,
                      int64_t n_slots, ssm_dtype_t dtype, ssm_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * ssm_conv1d_bwd -- backward of ssm_conv1d_fwd with state gradients.
 * Defined in [CC] "backward with states, a unified derivation": over the extended sequence
 * u = [S, x], with delta_t = dL/dz_t = dout_t * phi'(z_t) (z recomputed from x, S, w, bias),
 *     du_j = sum_t sum_k delta_t w_k [j = t + k] + [L <= j < L+K-1] dF_{j-L},
 *     dS = du[0 : K-1],  dx = du[K-1 : K-1+L],
 *     dw_k = sum_{b,t} delta_t u_{t+k},  dbias = sum_{b,t} delta_t.
 * With seq_idx the taps are masked exactly as in the forward; dF reaches the last K-1 inputs
 * directly (F is their raw copy).  Chunked training ([CC] "chunked training and truncated
 * back-propagation"): with S_B = F_A, passing chunk B's dS as chunk A's dF reproduces the
 * whole sequence's gradients.
 *
 *   x, initial_state, seq_idx, w, bias   as ssm_conv1d_fwd (initial_state may be NULL)
 *   dout            [batch, seqlen, channels]   dtype: dL/d(out)
 *   dfinal_state    [batch, channels, width-1]  dtype: dL/dF, or NULL (= 0)
 *   dx              [batch, seqlen, channels]   dtype
 *   dinitial_state  [batch, channels, width-1]  dtype, or NULL (not written)
 *   dw              [channels, width]           fp32 (summed over the batch)
 *   dbias           [channels]                  fp32, or NULL (not written)
 *   workspace       ssm_conv1d_bwd_workspace_size bytes (per-run partial sums of dw, dbias)
 * Outputs must not overlap inputs.  dw and dbias are deterministic (a fixed summation
 * order).  seqlen = 0: dinitial_state = dfinal_state, dw = dbias = 0.  batch = 0: no-op.
 * ------------------------------------------------------------------------------------- */
size_t ssm_conv1d_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t channels,
                                     int64_t width);
ssm_status_t ssm_conv1d_bwd(const void* x, const float* w, const float* bias,
                            const void* initial_state, const int32_t* seq_idx, const void* dout,
                            const void* dfinal_state, void* dx, void* dinitial_state, float* dw,
                            float* dbias, void* workspace, size_t workspace_bytes, int64_t batch,
                            int64_t seqlen, int64_t channels, int64_t width, ssm_dtype_t dtype,
                            ssm_act_t act, ssm_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * ssm_scan_bwd_initial_state -- gradient of the loss with respect to the scan's initial
 * state.  [LG] Sec. 2.5 Eq. (4): h_{-1} reaches y_t only through
 * C_t^T (prod_{tau<=t} a_tau) h_{-1} and the final state through (prod_{tau<L} a_tau) h_{-1},
 * a_tau = exp(dt_tau A_h), so
 *     dh_{-1}[p][n] = sum_t dy_t[p] (prod_{tau<=t} a_tau) C_t[n] + (prod_{tau<L} a_tau) dF[p][n].
 * With seq_idx the state is zeroed where the id changes, so only tokens before the first
 * change reach h_{-1}, and dF does only when the row has no change.  Chunked training
 * (Sec. 2.6): chunk B's result, passed as chunk A's dfinal_state, gives the whole sequence's.
 *
 *   dt               [batch, seqlen, nheads]            fp32
 *   A                [nheads]                           fp32
 *   C                [batch, seqlen, ngroups, dstate]   dtype
 *   dy               [batch, seqlen, nheads, headdim]   dtype: dL/dy
 *   seq_idx          [batch, seqlen] int32, or NULL
 *   dfinal_state     [batch, nheads, headdim, dstate]   fp32, or NULL (= 0)
 *   dinitial_state   [batch, nheads, headdim, dstate]   fp32; may alias dfinal_state
 * headdim 64 / dstate 128 / bf16 run on the matrix cores (16-byte aligned C and dy); other
 * shapes on a per-element loop.  Tokens after the decay product underflows to zero are not
 * read (their terms are exactly zero).  batch = 0: no-op.
 * ------------------------------------------------------------------------------------- */
ssm_status_t ssm_scan_bwd_initial_state(const float* dt, const float* A, const void* C,
                                        const void* dy, const int32_t* seq_idx,
                                        const float* dfinal_state, float* dinitial_state,
                                        int64_t batch, int64_t seqlen, int64_t nheads,
                                        int64_t headdim, int64_t ngroups, int64_t dstate,
                                        ssm_dtype_t dtype, ssm_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * Initial-state distributions for training ([LG] Sec. 2.6: the four interventions -- Random
 * Noise, Fitted Noise, State Passing, TBTT -- and the Fitted Noise update, Eqs. (5)-(6)).
 * Random numbers: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
 * easy as 1, 2, 3", SC 2011), key (seed, purpose), counter (block, offset, 0, 0).  The same
 * (seed, offset) always gives the same draws; a training step passes its own offset.
 * Gaussian initial states are for training only: [LG] evaluates from the zero state.
 * ------------------------------------------------------------------------------------- */

/* ssm_state_stats_update -- the Fitted Noise statistics, per head h:
 *   mean[h] <- (1 - beta) Mean(h_T) + beta mean[h],  var[h] <- (1 - beta) Var(h_T) + beta var[h]
 * ([LG] Eqs. (5)-(6), beta = 0.1 there: the new batch carries weight 1 - beta).  Mean and Var
 * are taken over the head's batch rows, channels and state dimension; Var is the population
 * variance (mean squared deviation), both accumulated in double (two passes).
 *   final_state  [batch, nheads, headdim, dstate]   fp32
 *   mean, var    [nheads]                           fp32, in / out (the caller initialises)
 * batch = 0: no-op (nothing observed).  Deterministic (fixed reduction order).
 * ------------------------------------------------------------------------------------- */
ssm_status_t ssm_state_stats_update(const float* final_state, int64_t batch, int64_t nheads,
                                    int64_t headdim, int64_t dstate, float beta, float* mean,
                                    float* var, ssm_stream_t stream);

/* ssm_initial_state_noise -- noise initial states: with mean and var (Fitted Noise) element
 * (b, h, p, n) is drawn from N(mean[h], var[h]); with both NULL (Random Noise) from
 * N(0, sigma^2).  Element e (flat index) reads word j = (e % 8) / 2 of Philox block e / 8
 * (purpose 0): u1 = (bits 40-63, plus 1) 2^-24 in (0, 1], u2 = (bits 8-31) 2^-24 in [0, 1),
 * r = sqrt(-2 ln u1) (Box-Muller), and z = r cos(2 pi u2) for even e, r sin(2 pi u2) for
 * odd e.  fp32 arithmetic.
 *   out       [batch, nheads, headdim, dstate]   fp32
 *   mean, var [nheads] fp32 (var >= 0), or both NULL
 * batch = 0: no-op.
 * ------------------------------------------------------------------------------------- */
ssm_status_t ssm_initial_state_noise(float* out, int64_t batch, int64_t nheads, int64_t headdim,
                                     int64_t dstate, const float* mean, const float* var,
                                     float sigma, uint64_t seed, uint64_t offset,
                                     ssm_stream_t stream);

/* ssm_state_reset -- State Passing's occasional reset ([LG] Sec. 2.6): row b of a carried
 * state (any tensor whose leading dimension is the batch row: the SSM state, the conv
 * state) is zeroed with probability p, else copied.  The decision for row b is word b % 4 of
 * Philox block b / 4 (purpose 1): zero iff its top 32 bits < floor(p 2^32) (p clipped to
 * [0, 1]).  It depends only on (seed, offset, b), so the SSM and conv states of one row,
 * reset with the same seed and offset, are zeroed together.
 *   src        [batch, row_bytes]   any type, row_bytes even, 2-byte aligned
 *   dst        [batch, row_bytes]   may alias src (then kept rows are not rewritten)
 *   reset_mask [batch] uint8, or NULL: 1 for a zeroed row
 * batch = 0: no-op.  p NaN: SSM_ERR_INVALID_ARG.
 * ------------------------------------------------------------------------------------- */
ssm_status_t ssm_state_reset(const void* src, void* dst, uint8_t* reset_mask, int64_t batch,
                             int64_t row_bytes, double p, uint64_t seed, uint64_t offset,
                             ssm_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * Measurement support (does not change any result).  When enabled, every launch of the
 * chunked-scan main kernel (the dominant kernel of ssm_scan_fwd / ssm_conv_scan_fwd) is
 * bracketed by a pair of HIP events recorded on the call's stream.  ssm_timing_read waits
 * for the recorded events, returns the summed kernel time in milliseconds and the number of
 * launches, and clears the record.  Event pairs are created the first time they are needed
 * and kept for reuse after a read, so a timed loop creates events only until its first read.
 * Not thread-safe with concurrent calls on other threads.
 * ------------------------------------------------------------------------------------- */
ssm_status_t ssm_timing_enable(int enable);
ssm_status_t ssm_timing_read(double* total_ms, int64_t* launches);

/* ssm_stream_copy -- a plain device-to-device copy of `bytes` bytes with non-temporal 16-byte
 * accesses (byte accesses for a tail, or when either pointer is not 16-byte aligned).  Not
 * part of the method: it is the streaming reference the benchmark reports beside the HBM
 * peak, since a copy with these accesses outruns the runtime's own device copy on this GPU.
 *   src, dst   device memory, must not overlap (SSM_ERR_INVALID_ARG if they do)
 * bytes = 0: no-op (pointers may be NULL).  bytes < 0: SSM_ERR_INVALID_ARG.
 * ------------------------------------------------------------------------------------- */
ssm_status_t ssm_stream_copy(const void* src, void* dst, int64_t bytes, ssm_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_MI355X_H */
