/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention library.
 *
 * The operation is the gated delta rule with a per-channel decay on the key
 * axis ("atlas_core/kimi_k3/kda.rs" page, module doc "Recurrence"), per
 * sequence n and head h, with a K x V fp32 state S:
 *     S <- diag(exp(g_t)) S
 *     d <- beta_t * (v_t - S^T k_t)
 *     S <- S + k_t d^T
 *     o_t <- scale * S^T q_t
 * with q, k optionally L2-normalised (eps 1e-6), beta optionally a logit and
 * g optionally computed in kernel from a raw gate input.  The argument set
 * follows the chunk_kda operator boundary of the "K3/kda/ops/api.py" page
 * (q, k, v, g, beta, A_log, dt_bias, scale, initial_state,
 * output_final_state, use_qk_l2norm_in_kernel, use_gate_in_kernel,
 * use_beta_sigmoid_in_kernel, safe_gate, lower_bound, chunk_size) without its
 * backend switch, plus packed variable-length sequences.
 *
 * Conventions shared by every entry point
 *   - Plain C types only.  Every tensor pointer is a DEVICE pointer unless
 *     stated otherwise; the args structs themselves live on the host and are
 *     read during the call only.
 *   - The caller owns every buffer.  The library never allocates or frees
 *     device memory and keeps no global mutable state; scratch memory is a
 *     caller-provided workspace whose size the *_workspace queries return.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL is the default
 *     stream) and the call returns without synchronising.
 *   - Every argument is validated on the host before anything is launched;
 *     on any error nothing is launched.  Device-resident index data
 *     (cu_seqlens) cannot be checked on the host: kernels clamp it so that
 *     no access leaves the tensors, but results for malformed offsets are
 *     unspecified.
 *   - Outputs must not alias inputs, except the documented in/out states of
 *     kda_recurrent_step.
 *   - Layouts are row-major with the last index fastest:
 *       q, k, g [rows, H, K]   v, o [rows, H, V]   beta [rows, H]
 *       states  [N, H, K, V]   (key index major)
 *     rows = B*T for dense input (sequence n is rows n*T .. n*T+T-1), or the
 *     packed token count T with B = 1 for variable-length input (sequence n is
 *     rows cu_seqlens[n] .. cu_seqlens[n+1]-1).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, bad flag value */
    KDA_ERR_UNSUPPORTED = 2,   /* dtype, chunk size, K/V/D outside the built set */
    KDA_ERR_MISSING_PARAM = 3, /* A_log absent with an in-kernel gate, or lower_bound
                                  absent with the safe gate (the two ValueErrors of
                                  the api.py boundary) */
    KDA_ERR_WORKSPACE = 4,     /* workspace pointer NULL or smaller than required */
    KDA_ERR_HIP = 5            /* a kernel launch reported an error */
} kda_status;

/* Element types.  The args structs hold them (like the flags and the gate
 * mode) in plain int fields, so that any value a caller stores is a valid
 * object in both C and C++; the library rejects values outside this set. */
typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* How g is turned into the per-channel log-decay (api.py chunk_kda gate
 * branch; kda.rs bounded_gate):
 *   KDA_GATE_LOGDECAY  g is the log-decay itself (use_gate_in_kernel=False).
 *   KDA_GATE_SAFE      g_eff = lower_bound * sigmoid(exp(A_log_h) * (g + dt_bias))
 *                      (use_gate_in_kernel=True, safe_gate=True).
 *   KDA_GATE_SOFTPLUS  g_eff = -exp(A_log_h) * softplus(g + dt_bias)
 *                      (use_gate_in_kernel=True, safe_gate=False). */
typedef enum { KDA_GATE_LOGDECAY = 0, KDA_GATE_SAFE = 1, KDA_GATE_SOFTPLUS = 2 } kda_gate_mode;

/* Arguments of the chunked forward / backward. */
typedef struct {
    /* sizes */
    int B, T, H, K, V;
    /* Variable-length packing: device int32 [N+1] prefix offsets with
     * cu_seqlens[0] = 0 and cu_seqlens[N] = T, non-decreasing; requires B = 1.
     * NULL means dense input with N = B sequences of length T.  The values
     * are read on the device only: offsets that break these rules are
     * clamped so that every access stays inside the tensors and the
     * workspace, and the results are then unspecified. */
    const int32_t *cu_seqlens;
    int N;
    /* inputs */
    int qkv_dtype;           /* kda_dtype of q, k, v (and o, dq, dk, dv, dO) */
    const void *q, *k, *v;
    const float *g;          /* [rows, H, K] log-decay or raw gate input (see gate_mode) */
    const float *beta;       /* [rows, H] value, or logit when use_beta_sigmoid */
    const float *A_log;      /* [H]; required for SAFE / SOFTPLUS, ignored otherwise */
    const float *dt_bias;    /* [H*K] or NULL (= 0); SAFE / SOFTPLUS only */
    float scale;             /* <= 0 or NaN means K^-1/2 */
    float lower_bound;       /* NaN means "none".  Required for SAFE (the gate's
                                floor); not read in the other modes, where any
                                log-decay is handled by the run-time per-block
                                span check of the kernels. */
    int gate_mode;           /* kda_gate_mode */
    int use_qk_l2norm;       /* q <- q (sum q^2 + 1e-6)^-1/2, same for k.  With 0 the
                                caller must supply well-scaled keys: the api.py
                                boundary warns that un-normalised keys can drive the
                                exact result to inf. */
    int use_beta_sigmoid;    /* beta <- sigmoid(beta) */
    int chunk_size;          /* >= 1: a tiling request.  The chunked form is exact for any
                                chunk size, and the api.py dispatch maps the request to
                                each backend's own tiling (a divisor of T for its
                                reference, 32 or 64 for its Triton kernels); these
                                kernels always tile with 64 rows, so every request
                                gives the same result.  <= 0 is KDA_ERR_INVALID_ARG. */
    /* state */
    const float *initial_state; /* [N, H, K, V] or NULL (zeros) */
    int output_final_state;
    /* outputs */
    void *o;                 /* [rows, H, V] in qkv_dtype */
    float *final_state;      /* [N, H, K, V]; written when output_final_state != 0 */
    /* resources */
    void *workspace;
    size_t workspace_bytes;
    void *stream;            /* hipStream_t */
    /* Save-for-backward (0 or 1).  0: the forward keeps only its own per-chunk
     * operands in the workspace (kda_chunk_fwd_workspace bytes) and a later
     * kda_chunk_bwd recomputes them and every chunk's entry state.  1: the
     * forward also writes what the backward's stages 0 and 1 would compute (the
     * backward's per-chunk operands and each chunk's entry state) into a
     * workspace of kda_chunk_bwd_workspace bytes (kda_chunk_fwd_workspace then
     * returns that size), and a backward called with the flag set and the same
     * workspace reads them instead, its stages 0 and 1 doing nothing.  Between
     * the two calls the caller keeps the workspace and every input unchanged;
     * the library cannot check this. */
    int keep_for_backward;
    /* Fused full-rank output gate (forward only; the "atlas_core/kimi_k3/kda.rs"
     * page, full_rank_output_gate).  With out_gate given, o receives, per row
     * and head, y = sigmoid(out_gate) * o / sqrt(mean_v(o^2) + eps) over the
     * head's V values -- kda_output_gate applied to the output.  With at least
     * 256 (sequence, head) chains the state pass computes it before each row
     * is stored (one workgroup per chain, o never written ungated); with
     * fewer, the state pass writes o and the gate runs over it in place within
     * the same call (the split state pass fills the chip better; o is then
     * rounded to its element type before the gate, as with kda_output_gate).
     * out_gate is [rows, H, V] in out_gate_dtype, 16-byte aligned.  Inference
     * only: keep_for_backward must be 0 and kda_chunk_bwd rejects a set
     * out_gate (KDA_ERR_INVALID_ARG); training calls the forward without it
     * and kda_output_gate / kda_output_gate_bwd. */
    const void *out_gate;     /* [rows, H, V] gate input, or NULL (o is the plain output) */
    int out_gate_dtype;       /* kda_dtype of out_gate */
    float out_gate_eps;       /* NaN means 1e-5; must be >= 0 */
} kda_chunk_args;

/* Gradients for kda_chunk_bwd.  dq, dk, dv are in qkv_dtype; the others fp32.
 * dg and dbeta are taken with respect to the tensors AS PASSED: the raw gate
 * input in SAFE / SOFTPLUS mode, the logit when use_beta_sigmoid is set. */
typedef struct {
    const void *dO;              /* [rows, H, V], required */
    const float *d_final_state;  /* [N, H, K, V] or NULL (= 0) */
    void *dq, *dk, *dv;          /* required */
    float *dg;                   /* [rows, H, K], required */
    float *dbeta;                /* [rows, H], required */
    float *d_initial_state;      /* [N, H, K, V] or NULL (not written) */
    float *dA_log;               /* [H] or NULL; SAFE / SOFTPLUS only */
    float *ddt_bias;             /* [H*K] or NULL; SAFE / SOFTPLUS only */
} kda_chunk_grads;

/* Chunked forward (64-row chunks): writes o and, if requested, final_state.
 * Computes exactly the recurrence above, in chunkwise-parallel form
 * (api.py chunk_kda; the chunk form's use of I + tril(A_kk * beta) is named in
 * its l2-norm warning).  K = V in {32, 64, 128} for KDA_BF16 q/k/v and
 * {32, 64} for KDA_F32 (the fp32 operand tiles of K = 128 exceed the 160 KiB
 * of LDS a workgroup can hold), and the narrow-key pair K = 32, V = 64 of the
 * "KDA <=> FLA Parity in Primus" page's 300M configuration (key head dim 32,
 * value head dim 64) in both dtypes; anything else is KDA_ERR_UNSUPPORTED.
 * An empty sequence writes final_state = initial_state. */
kda_status kda_chunk_fwd(const kda_chunk_args *a);
size_t kda_chunk_fwd_workspace(const kda_chunk_args *a);

/* Chunked forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Identical to kda_chunk_fwd, except that its workspace is the
 * library's own device array of KDA_NOALLOC_SCRATCH_BYTES bytes, one per GPU,
 * held from the library's load on that GPU until the process ends;
 * a->workspace and a->workspace_bytes are ignored.  It calls no hipMalloc,
 * hipFree or other allocating routine.
 *   - If kda_chunk_fwd_workspace(a) exceeds KDA_NOALLOC_SCRATCH_BYTES the call
 *     returns KDA_ERR_WORKSPACE and launches nothing (192 MiB holds, e.g.,
 *     the packed 8192-token, 16-head, K = V = 128 bf16 prefill).
 *   - keep_for_backward must be 0 (else KDA_ERR_INVALID_ARG): the array is
 *     shared by every call on the GPU, so saved operands would not survive.
 *   - Every call on a GPU shares that GPU's array, which keeps the last
 *     call's contents (nothing in it needs to start at zero).  Calls that
 *     overlap in time on one GPU (unordered streams or threads) race on it
 *     and their results are undefined; calls ordered on one stream are safe.
 *   - The first call on each device looks up the array's device address
 *     (hipGetSymbolAddress, not a stream operation); later calls reuse it.
 *     A failure of that lookup returns KDA_ERR_HIP. */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)192 << 20)
kda_status kda_chunk_fwd_noalloc(const kda_chunk_args *a);

/* Stage-split forward, for profilers that time each kernel with stream
 * events.  Calling stage 0 then stage 1 with the same arguments (and the
 * same workspace) on one stream is identical to kda_chunk_fwd:
 *   stage 0  per-chunk preparation (fully parallel over chunk x head);
 *   stage 1  sequential state pass and output (parallel over sequence x head
 *            x value-column block).
 * Other stage numbers return KDA_ERR_INVALID_ARG. */
kda_status kda_chunk_fwd_stage(const kda_chunk_args *a, int stage);

/* Chunked backward: gradients of <o, dO> + <final_state, d_final_state>.
 * Uses the same args as the forward (o and final_state are not read). */
kda_status kda_chunk_bwd(const kda_chunk_args *a, const kda_chunk_grads *gr);
size_t kda_chunk_bwd_workspace(const kda_chunk_args *a);

/* Stage-split backward, for per-kernel timing (see kda_chunk_fwd_stage).
 * Stages 0 .. kda_chunk_bwd_stages()-1 called in order with the same
 * arguments and workspace equal one kda_chunk_bwd call:
 *   0  per-chunk preparation (as the forward's, plus (I + A)^-1 and the
 *      un-scaled k-k scores);
 *   1  forward state pass, storing every chunk's entry state;
 *   2  reverse state pass, storing every chunk's exit-state gradient and
 *      writing d_initial_state;
 *   3  per chunk: dv and the value-summed operand gradients;
 *   4  per chunk: dq, dk, dg, dbeta, and the reduction of dA_log / ddt_bias.
 * Other stage numbers return KDA_ERR_INVALID_ARG. */
kda_status kda_chunk_bwd_stage(const kda_chunk_args *a, const kda_chunk_grads *gr, int stage);
int kda_chunk_bwd_stages(void);

/* One decode token per sequence ("atlas_core/kimi_k3/kda.rs" page,
 * kda_decode_token = conv_update followed by kda_recurrent_step):
 *   for each of the 3*H*D channels c of x = [q | k | v]:
 *       window[c] shifts left one slot (slot 0 leaves), x[c] enters slot W-1,
 *       y[c] = SiLU(sum_j conv_w[c, j] * window[c, j])   (no bias)
 *   then per head the recurrence step above on (q, k, v) = y, writing
 *   o [N, H*D] (fp32) and updating state in place.
 * With out_gate set, o receives the full-rank output gate of the step's
 * output instead (kda_output_gate below, same page: full_rank_output_gate),
 * computed in the same kernel.
 * Slot-indexed states (resuming sequences from saved snapshots, the
 * prefix-hit restore of the same page's test prefix_hit_wrong_slot_diverges):
 * with state_slots given, state is a pool [S, H, D, D] and conv_state a pool
 * [S, 3*H*D, W] (S = n_slots), and sequence n reads and updates slot
 * state_slots[n]; x, g, beta, out_gate and o stay indexed by n.  Slots must
 * be distinct within a call: the library does not check this (the indices are
 * device data), and two sequences on one slot race, leaving that slot's
 * states and both outputs undefined.  A slot outside
 * [0, S) leaves every state unchanged and sets that sequence's o to NaN. */
typedef struct {
    int N, H, D, W;          /* D = head dim (K = V = D) in {32, 64, 128}; 1 <= W <= 8 */
    int x_dtype;             /* kda_dtype: KDA_F32 or KDA_BF16 */
    const void *x_qkv;       /* [N, 3*H*D] pre-conv inputs, [q | k | v] */
    const float *conv_w;     /* [3*H*D, W], slot 0 oldest */
    float *conv_state;       /* [N, 3*H*D, W] in/out, oldest -> newest */
    const float *g;          /* [N, H*D] log-decay or raw gate input (gate_mode) */
    const float *beta;       /* [N, H] */
    const float *A_log;      /* [H] (SAFE / SOFTPLUS) */
    const float *dt_bias;    /* [H*D] or NULL */
    float lower_bound;       /* NaN = none; required for SAFE */
    int gate_mode;
    int use_qk_l2norm;       /* kda.rs always normalises; 1 is the usual setting */
    int use_beta_sigmoid;    /* kda.rs passes a logit; 1 is the usual setting */
    float scale;             /* <= 0 or NaN means D^-1/2 */
    float *state;            /* [N, H, D, D] in/out, key index major */
    float *o;                /* [N, H*D] fp32 */
    void *stream;            /* hipStream_t */
    const void *out_gate;    /* [N, H*D] in x_dtype, or NULL: o is the plain output */
    float out_gate_eps;      /* NaN means 1e-5; must be >= 0 */
    const int32_t *state_slots; /* device [N] or NULL; see below */
    int n_slots;             /* pool size S when state_slots is given */
} kda_step_args;

kda_status kda_recurrent_step(const kda_step_args *a);

/* Stateful prefill of the short convolution: the conv_update of the
 * "atlas_core/kimi_k3/kda.rs" page applied to every row of a sequence in
 * order, carrying the window state in and out, so that a prompt primed here
 * continues exactly in kda_recurrent_step (the prime -> decode hand-off of the
 * "memra-engine kda_fixture_gpu.rs" page, GATE 2 and GATE 3).  For each
 * sequence n and each of the C = 3*H*D channels c, over its rows t in order:
 *     the window shifts left one slot, x[t, c] enters slot W-1,
 *     y[t, c] = SiLU(sum_j conv_w[c, j] * window[j])   (no bias)
 * The window starts as conv_state[n, c, :] (all zeros when conv_state is
 * NULL) and, on return, conv_state[n, c, :] holds the window after the last
 * row (unchanged for an empty sequence).  y is written split by channel block
 * as the [rows, H, D] inputs of kda_chunk_fwd:
 *     q = y[:, 0 : H*D],  k = y[:, H*D : 2*H*D],  v = y[:, 2*H*D : 3*H*D].
 * The final states of that forward (output_final_state) and this conv state
 * are the decode state of kda_recurrent_step.
 * Every pointer must be 16-byte aligned; q, k and v must not overlap x_qkv or
 * each other.  Errors as for the other entry points (nothing is launched). */
typedef struct {
    int B, T, H, D, W;         /* D in {32, 64, 128}; 1 <= W <= 8 */
    const int32_t *cu_seqlens; /* device [N+1] for packed input (B = 1), or NULL (dense, N = B) */
    int N;
    int x_dtype;               /* kda_dtype: KDA_F32 or KDA_BF16 */
    const void *x_qkv;         /* [rows, 3*H*D] pre-conv inputs, [q | k | v] */
    const float *conv_w;       /* [3*H*D, W], slot 0 oldest */
    float *conv_state;         /* [N, 3*H*D, W] in/out, oldest -> newest; or NULL */
    int y_dtype;               /* kda_dtype: KDA_F32 or KDA_BF16, element type of q, k, v */
    void *q, *k, *v;           /* [rows, H, D] each */
    void *stream;              /* hipStream_t */
} kda_conv_args;

kda_status kda_conv_prefill(const kda_conv_args *a);

/* Full-rank output gate (full_rank_output_gate of the
 * "atlas_core/kimi_k3/kda.rs" page), per head of every row:
 *     r = 1 / sqrt(mean_v(o[v]^2) + eps),   y[v] = sigmoid(g[v]) * o[v] * r
 * over the V values of the head (no weight).  The gated output norm of the
 * "memra-engine kda_fixture_gpu.rs" page uses eps = 1e-5, the default here.
 * o is the output of kda_chunk_fwd or kda_recurrent_step; y feeds the output
 * projection.  y may be o (in place); any other overlap is not allowed.
 * Every pointer must be 16-byte aligned.  Nothing is launched on error. */
typedef struct {
    int rows, H, V;            /* V in {32, 64, 128, 256}; rows >= 0 */
    int o_dtype;               /* kda_dtype: KDA_F32 or KDA_BF16, for o, y (and dy, dO) */
    int g_dtype;               /* kda_dtype: KDA_F32 or KDA_BF16, for g (and dg) */
    float eps;                 /* NaN means 1e-5; must be >= 0 */
    const void *o;             /* [rows, H, V] */
    const void *g;             /* [rows, H, V] gate input (before the sigmoid) */
    void *y;                   /* [rows, H, V] */
    void *stream;              /* hipStream_t */
} kda_gate_args;

kda_status kda_output_gate(const kda_gate_args *a);

/* Reverse mode of kda_output_gate (the chain rule written out; no page prints
 * it): with a = sigmoid(g) and r as above, for the upstream gradient dy,
 *     dg[v] = dy[v] * o[v] * r * a[v] * (1 - a[v])
 *     dO[v] = r * a[v] * dy[v] - (r^3 / V) * o[v] * sum_u a[u] * dy[u] * o[u].
 * a->y is not read.  dy and dO have o_dtype, dg has g_dtype; dO may be dy and
 * dg may be g (in place); no other overlap.  dO is the dO of kda_chunk_bwd. */
kda_status kda_output_gate_bwd(const kda_gate_args *a, const void *dy, void *dO, void *dg);

/* Static description of a status code.  Thread-safe. */
const char *kda_status_string(kda_status s);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
