/*
 * sdm.h -- C ABI of the Sparse Delta Memory (SDM) hot path on AMD Instinct
 * MI355X (gfx950).
 *
 * The method (cited by page title and section):
 *   [P] "Sparse Delta Memory: Scaling the State of Linear RNNs through
 *       Sparsity"
 *       Sec. 2, Product-Key Memories: N = n_sub^2 slot scores are the outer
 *               sum of two half-score vectors; top-k is found without
 *               materialising the N scores.
 *       Sec. 3.1, step 1 (Sparse Key Selection), step 2 (Gated Delta Write,
 *               Eq. 4), step 3 (Sparse Read), "Learned Initial State".
 *       Sec. 4, SDM Configuration: read and write activations use softmax
 *               normalisation.
 *   [B] "Sparse Delta Memory: Scaling Linear RNN States to 1M Tokens via
 *       Sparsity", Methodology, item 2 (Gated Delta Updates):
 *       M_t[i] <- a_t M_{t-1}[i] + b_t k^(i) (v_t - a_t M_{t-1}^T k_t).
 *
 * Conventions shared by every call:
 *   - Layouts are row-major and contiguous.  A "token-head" is one (b, t, h).
 *       k, q       [B, T, H, d_k]        bf16 (in_dtype SDM_BF16) or fp32
 *       v          [B, T, H, d_v]        same dtype as k
 *       C_w, C_r   [H, 2, n_sub, d_k/2]  sub-key codebooks (half 0, half 1)
 *       a, b       [B, T, H]             fp32 forget gate a_t and input gate b_t
 *       widx, wwt  [B, T, H, W]          int32 write slots, fp32 weights
 *       ridx, rwt  [B, T, H, R]          int32 read slots, fp32 weights
 *       M          [B, H, N, d_v]        fp32 memory state, N = n_sub^2
 *       M0         [H, N, d_v]           fp32 learned initial state
 *       o          [B, T, H, d_v]        fp32 read-out
 *   - Slot numbering: slot = i1 * n_sub + i2, i1 from half 0 of the key.
 *   - Slot lists are sorted by score descending, ties to the lower slot; a
 *     half score is an fp32 dot product and a slot score is the fp32 sum of
 *     its two half scores.  Weights are the softmax of the selected scores.
 *   - All pointers are device pointers (hipMalloc'd or equivalent) unless
 *     stated.  The caller owns every buffer; the library keeps no pointer
 *     after a call returns and allocates no device memory.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *     default stream).  Arguments are validated on the host before anything
 *     is launched; on a validation error nothing is written.  A launch
 *     failure returns SDM_ERR_HIP.  No C++ exception crosses this boundary.
 *   - A call with no work (B = 0, or T = 0 where a call takes T) returns
 *     SDM_OK once dims are valid, touches no buffer and launches nothing;
 *     its pointers may then be NULL (as empty torch tensors give).
 *   - Calls that overlap on the same buffers race; order them on one stream.
 *   - sdm_last_error() returns a per-thread message describing the last
 *     non-OK status.
 */
#ifndef SDM_H_
#define SDM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SDM_OK = 0,
    SDM_ERR_INVALID_ARG = -1, /* bad pointer, size or dimension */
    SDM_ERR_UNSUPPORTED = -2, /* legal for the method, outside what the kernels implement */
    SDM_ERR_HIP = -3          /* the HIP runtime reported an error */
} sdm_status;

typedef enum { SDM_F32 = 0, SDM_BF16 = 1 } sdm_dtype;

typedef void *sdm_stream_t; /* a hipStream_t */

typedef struct {
    int64_t B;       /* sequences */
    int64_t T;       /* tokens per sequence in this call (1 for sdm_decode_step) */
    int64_t H;       /* SDM heads */
    int64_t d_k;     /* key/query width, even; each half is d_k/2 */
    int64_t n_sub;   /* sub-keys per half; N = n_sub^2 slots per head */
    int64_t d_v;     /* value / memory row width */
    int64_t k_prime; /* candidates kept per half before the merge */
    int64_t W;       /* write slots per token */
    int64_t R;       /* read slots per token */
    int32_t in_dtype;/* sdm_dtype of k, q, v, C_w, C_r */
    int32_t reserved;/* must be 0 */
} sdm_dims;

/* Limits of this implementation (SDM_ERR_UNSUPPORTED beyond them):
 *   B < 2^31;  W, R <= 64;  k_prime <= 64;  k_prime <= n_sub <= 2048;
 *   d_v a multiple of 32 and <= 1024;  n_sub^2 * d_v * 4 <= 2 GiB (one (b, h) memory);
 *   bf16: d_k/2 a multiple of 32, d_k <= 512;
 *   fp32: d_k <= 512.
 * Method constraints (SDM_ERR_INVALID_ARG): d_k even; 1 <= W, R <= k_prime^2. */

/* ---------------------------------------------------------------------------
 * sdm_state_init -- [P] Sec. 3.1 "Learned Initial State"; [B] item 3.
 * Copies the learned initial memory into every sequence: M[b][h] = M0[h].
 *   M  [B,H,N,d_v] fp32, written.   M0 [H,N,d_v] fp32, read.
 * Only B, H, n_sub and d_v of dims are used.  M and M0 must not overlap.
 * ------------------------------------------------------------------------- */
sdm_status sdm_state_init(float *M, const float *M0, const sdm_dims *dims, sdm_stream_t stream);

/* ---------------------------------------------------------------------------
 * sdm_pkm_address -- [P] Sec. 2 (PKM) and Sec. 3.1 step 1; softmax of Sec. 4.
 * For every token-head and each kind (write: x = k against C_w, read: x = q
 * against C_r):
 *   s_c[u] = <x[c*d_k/2 : (c+1)*d_k/2], C[h][c][u]>   c = 0, 1   (fp32 result)
 *   top-k_prime of s_0 and of s_1; the k_prime^2 outer-sum candidates
 *   s_0[i1] + s_1[i2] at slot i1*n_sub + i2; the top W (write) / R (read)
 *   of those, sorted; weights = softmax of their scores.
 * With k_prime >= W (resp. R) the result is the exact top-W over all N slots.
 * C_r may equal C_w (one shared codebook).  Outputs: widx, wwt [B,T,H,W];
 * ridx, rwt [B,T,H,R].  Uses B, T, H, d_k, n_sub, k_prime, W, R, in_dtype.
 * ------------------------------------------------------------------------- */
sdm_status sdm_pkm_address(const void *k, const void *q, const void *C_w, const void *C_r,
                           const sdm_dims *dims, int32_t *widx, float *wwt, int32_t *ridx,
                           float *rwt, sdm_stream_t stream);

/* ---------------------------------------------------------------------------
 * sdm_pkm_address_overlapped -- sdm_pkm_address with the same arguments and
 * results (bit for bit), launched so that each compute unit holds at most
 * one of its workgroups: the rest of the CU's LDS and wave slots stay free
 * for a kernel running at the same time on another stream.  For a prefill
 * pipelined over chunks of tokens: the addressing of chunk c + 1 (this call,
 * on a second stream) overlaps the scan of chunk c (sdm_scan_forward, whose
 * chunks give the same results as one call over all tokens).  Alone it runs
 * about half as fast as sdm_pkm_address.
 * ------------------------------------------------------------------------- */
sdm_status sdm_pkm_address_overlapped(const void *k, const void *q, const void *C_w, const void *C_r,
                                      const sdm_dims *dims, int32_t *widx, float *wwt, int32_t *ridx,
                                      float *rwt, sdm_stream_t stream);

/* ---------------------------------------------------------------------------
 * sdm_scan_workspace_size -- bytes of device workspace sdm_scan_forward needs
 * for these dims (0 if none).  Host-only; never fails (returns 0 on bad dims).
 * ------------------------------------------------------------------------- */
size_t sdm_scan_workspace_size(const sdm_dims *dims);

/* ---------------------------------------------------------------------------
 * sdm_scan_forward -- [P] Sec. 3.1 steps 2-3 (Eq. 4) and [B] item 2.
 * For every (b, h), tokens t = 0..T-1 in order, on the state M in place:
 *   p   = sum_j wwt_j M[widx_j]                    (rows before this write)
 *   M[widx_j] = a_t M[widx_j] + b_t wwt_j (v_t - a_t p)   for all j at once
 *   o_t = sum_j rwt_j M[ridx_j]                    (rows after this write)
 * Rows not in widx are untouched.  Write slots of one token must be distinct
 * and every slot must lie in [0, N); out-of-range slots are dropped by the
 * hardware bounds check of the buffer access instead of faulting (results
 * are then undefined, never out-of-bounds memory traffic).
 * workspace: device memory of at least sdm_scan_workspace_size(dims) bytes
 * (may be NULL when that is 0); its contents on entry are ignored.
 * o must not alias M, the slot lists or the weights.
 * Uses B, T, H, n_sub, d_v, W, R, in_dtype (v's dtype).
 * ------------------------------------------------------------------------- */
sdm_status sdm_scan_forward(float *M, const int32_t *widx, const float *wwt, const int32_t *ridx,
                            const float *rwt, const void *v, const float *a, const float *b,
                            float *o, void *workspace, size_t workspace_bytes,
                            const sdm_dims *dims, sdm_stream_t stream);

/* ---------------------------------------------------------------------------
 * sdm_scan_forward_gated -- sdm_scan_forward with the gates applied inside
 * its preparation pass ([P] Sec. 3.1 step 2 and Sec. 4, as sdm_gates):
 *   a_t = exp(-A[h] softplus(a_raw + dt_bias[h])),  b_t = sigmoid(b_raw)
 * a_raw, b_raw [B,T,H] fp32 (the gates' pre-activations) take the place of
 * a, b; A, dt_bias [H] fp32 (A >= 0, the decay rate itself).  The results
 * are those of sdm_gates followed by sdm_scan_forward, bit for bit, without
 * the separate pass over the gates.  Same workspace, dims, layout and rules
 * as sdm_scan_forward; A and dt_bias must not overlap M, o or the workspace
 * (SDM_ERR_INVALID_ARG).
 * ------------------------------------------------------------------------- */
sdm_status sdm_scan_forward_gated(float *M, const int32_t *widx, const float *wwt, const int32_t *ridx,
                                  const float *rwt, const void *v, const float *a_raw, const float *b_raw,
                                  const float *A, const float *dt_bias, float *o, void *workspace,
                                  size_t workspace_bytes, const sdm_dims *dims, sdm_stream_t stream);

/* ---------------------------------------------------------------------------
 * sdm_scan_forward_noalloc -- sdm_scan_forward for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): same arguments without the
 * workspace, same kernels and results, bit for bit.  The preparation
 * streams live in a static scratch array of SDM_NOALLOC_SCRATCH_BYTES
 * (128 MiB) that each GPU the library runs on holds until the process ends;
 * its device address is looked up once per device, on the first call with
 * that device current.  The call allocates nothing (no hipMalloc, no
 * hipFree).  Dims with sdm_scan_workspace_size(dims) above
 * SDM_NOALLOC_SCRATCH_BYTES give SDM_ERR_UNSUPPORTED before anything is
 * launched (split T or B, or use sdm_scan_forward).  Every call on one GPU
 * shares that GPU's scratch: calls that overlap in time on one GPU (other
 * streams, other host threads) race and must not be issued; calls in order
 * on one stream are safe.  Nothing needs clearing between calls (the scan
 * reads only scratch bytes its preparation pass wrote in the same call).
 * ------------------------------------------------------------------------- */
#define SDM_NOALLOC_SCRATCH_BYTES ((size_t)134217728)
sdm_status sdm_scan_forward_noalloc(float *M, const int32_t *widx, const float *wwt, const int32_t *ridx,
                                    const float *rwt, const void *v, const float *a, const float *b,
                                    float *o, const sdm_dims *dims, sdm_stream_t stream);

/* ---------------------------------------------------------------------------
 * sdm_scan_forward_save -- sdm_scan_forward that also saves, for the
 * backward pass, the rows each token used:
 *   xsave [B,H,T,d_v/4,W,4] fp32: the write rows before the token's write;
 *   zsave [B,H,T,d_v/4,R,4] fp32: the read rows after it (what o_t sums);
 *   both in 4-column chunks, the list positions of a chunk adjacent, so
 *   that the lanes of one token store and load consecutive bytes.
 * Everything else as sdm_scan_forward (same results, bit for bit).  One
 * (sequence, head) of xsave or zsave must stay below 2 GiB
 * (SDM_ERR_UNSUPPORTED otherwise; split T into chunks).
 * ------------------------------------------------------------------------- */
sdm_status sdm_scan_forward_save(float *M, const int32_t *widx, const float *wwt, const int32_t *ridx,
                                 const float *rwt, const void *v, const float *a, const float *b,
                                 float *o, float *xsave, float *zsave, void *workspace,
                                 size_t workspace_bytes, const sdm_dims *dims, sdm_stream_t stream);

/* ---------------------------------------------------------------------------
 * sdm_scan_backward_workspace_size -- bytes of device workspace
 * sdm_scan_backward needs for these dims (uses B, T, H, W, R, d_v,
 * in_dtype).  0 when the dims are invalid, or when they fall outside the
 * lane-parallel backward (one (sequence, head) of its streams, of xsave or
 * of the per-chunk partial sums would reach 2 GiB, or T * H * d_v * 4 does):
 * sdm_scan_backward then runs its token-serial kernels, which take no
 * workspace.  Host-only.
 * ------------------------------------------------------------------------- */
size_t sdm_scan_backward_workspace_size(const sdm_dims *dims);

/* ---------------------------------------------------------------------------
 * sdm_scan_backward -- reverse-mode gradients of sdm_scan_forward ([P]
 * Sec. 3.1 steps 2-3, Eq. 4, differentiated; the pages print no backward
 * pass).  For a loss L with dL/do_t = dout [B,T,H,d_v] fp32 and dL/dM after
 * the call = dM on entry ([B,H,N,d_v] fp32; zeros if L does not see the
 * final state), writes
 *   dM  <- dL/dM before the call (in place),
 *   dv [B,T,H,d_v], da, db [B,T,H], dw [B,T,H,W], dr [B,T,H,R]  (fp32),
 * the gradients with respect to v, the gates and the write and read weights.
 * xsave, zsave: from sdm_scan_forward_save of the same call.  Same slot
 * lists, weights, v, a, b as the forward.  Per token, in reverse:
 *   dr_i = <do, Z_i>;  G[r_i] += r_i do;  dY_j = G[s_j];  p = sum_j w_j X_j;
 *   u = v - a p;  du = b sum_j w_j dY_j;  dv = du;  dp = -a du;
 *   da = sum_j <dY_j, X_j> - <p, du>;  db = sum_j w_j <dY_j, u>;
 *   dw_j = b <dY_j, u> + <dp, X_j>;  G[s_j] = a dY_j + w_j dp.
 * A read slot may appear at several positions of one token: each position
 * adds its r_i do to G (the positions are merged, their weights summed in
 * list order).  Write slots of one token must be distinct, as in the
 * forward.  fp32 arithmetic, every sum in a fixed order (deterministic).
 * Uses B, T, H, n_sub, d_v (<= 256), W, R, in_dtype.
 * workspace: at least sdm_scan_backward_workspace_size(dims) bytes, 16-byte
 * aligned, owned by the caller; it holds the forwarding codes and repacked
 * inputs of the lane-parallel pass and its per-chunk partial sums, and is
 * overwritten.  workspace = NULL with workspace_bytes = 0 selects the
 * token-serial kernels, which need none (same results up to the order of
 * fp32 sums; slower: one token of a chain at a time), for callers that
 * cannot provide it.  dM, the outputs and the workspace must not overlap
 * each other or any input (SDM_ERR_INVALID_ARG).
 * ------------------------------------------------------------------------- */
sdm_status sdm_scan_backward(float *dM, const int32_t *widx, const float *wwt, const int32_t *ridx,
                             const float *rwt, const void *v, const float *a, const float *b,
                             const float *dout, const float *xsave, const float *zsave, float *dv,
                             float *da, float *db, float *dw, float *dr, void *workspace,
                             size_t workspace_bytes, const sdm_dims *dims, sdm_stream_t stream);

/* ---------------------------------------------------------------------------
 * sdm_address_backward_workspace_size -- bytes of device workspace
 * sdm_address_backward needs for these dims (0 on bad dims).  Host-only.
 * ------------------------------------------------------------------------- */
size_t sdm_address_backward_workspace_size(const sdm_dims *dims);

/* ---------------------------------------------------------------------------
 * sdm_address_backward -- gradients of sdm_pkm_address with the selected
 * slots held fixed (the selection is piecewise constant): [P] Sec. 2 (slot
 * score = the sum of the two half scores, each a dot product with a
 * sub-key) and Sec. 4 (softmax over the selected scores), differentiated:
 *   dsc_j = w_j (dw_j - sum_k w_k dw_k)
 *   dx[half c] += dsc_j C[h][c][i_c],   dC[h][c][i_c] += dsc_j x[half c]
 * with i_0 = slot / n_sub, i_1 = slot % n_sub, for the write lists (x = k,
 * C = C_w, dw = dL/dwwt) and the read lists (x = q, C = C_r, dr = dL/drwt).
 *   widx, wwt, ridx, rwt: the forward's lists and weights;
 *   dk, dq [B,T,H,d_k] fp32 written;
 *   dC_w, dC_r [H,2,n_sub,d_k/2] fp32 written (sums over every token); they
 *   may be the same buffer (a shared codebook): it then receives the sum.
 * workspace: at least sdm_address_backward_workspace_size(dims) bytes,
 * 16-byte aligned.  fp32 arithmetic, every sum in a fixed order.  The
 * outputs and the workspace must not overlap each other (except dC_w ==
 * dC_r) or any input (SDM_ERR_INVALID_ARG).
 * ------------------------------------------------------------------------- */
sdm_status sdm_address_backward(const void *k, const void *q, const void *C_w, const void *C_r,
                                const int32_t *widx, const float *wwt, const int32_t *ridx,
                                const float *rwt, const float *dw, const float *dr,
                                const sdm_dims *dims, float *dk, float *dq, float *dC_w, float *dC_r,
                                void *workspace, size_t workspace_bytes, sdm_stream_t stream);

/* ---------------------------------------------------------------------------
 * sdm_decode_step -- one new token for each of B sequences: the addressing of
 * sdm_pkm_address and one step of sdm_scan_forward fused in one launch
 * ([P] Sec. 3.1 steps 1-3 for T = 1).
 *   M [B,H,N,d_v] in/out;  k, q [B,H,d_k];  v [B,H,d_v];  a, b [B,H];
 *   o [B,H,d_v] written;  widx_out [B,H,W], ridx_out [B,H,R] optional (NULL
 *   skips them) -- the selected slots, for inspection.
 * dims->T must be 1.  Results equal sdm_pkm_address followed by
 * sdm_scan_forward on the same token.
 * ------------------------------------------------------------------------- */
sdm_status sdm_decode_step(float *M, const void *k, const void *q, const void *C_w,
                           const void *C_r, const void *v, const float *a, const float *b,
                           float *o, int32_t *widx_out, int32_t *ridx_out, const sdm_dims *dims,
                           sdm_stream_t stream);

/* ---------------------------------------------------------------------------
 * Copy-on-write state for decode ([P] Sec. 3.1 "Learned Initial State": every
 * sequence starts from the shared M0).  Instead of copying M0 into every
 * sequence (sdm_state_init: B x |M0| bytes written), each (b, h) keeps a
 * bitmap of the slots it has written; a row whose bit is clear is read from
 * M0.  A decode step touches at most W rows per (b, h), so after a few
 * thousand steps most of a large memory is still M0's.
 *   touched [B][H][ceil(N/32)] uint32 (bit s % 32 of word s / 32: slot s of
 *   that (b, h) has been written and lives in M).  Bytes:
 *   sdm_cow_bitmap_bytes(dims).
 * ------------------------------------------------------------------------- */
size_t sdm_cow_bitmap_bytes(const sdm_dims *dims);

/* sdm_cow_reset -- every sequence starts from M0: clears the bitmap (a fill
 * kernel, safe under graph capture).  Uses B, H, n_sub of dims. */
sdm_status sdm_cow_reset(uint32_t *touched, const sdm_dims *dims, sdm_stream_t stream);

/* sdm_decode_step_cow -- sdm_decode_step on a copy-on-write state: the rows
 * it gathers are taken from M where their bit is set and from M0 [H,N,d_v]
 * otherwise; the rows it writes go to M and get their bit set.  M needs no
 * initialisation.  Outputs and the rows written are bit-identical to
 * sdm_state_init followed by sdm_decode_step.  M0, M, the bitmap and o must
 * not overlap (SDM_ERR_INVALID_ARG); other arguments as sdm_decode_step.
 * Calls that overlap on one bitmap race. */
sdm_status sdm_decode_step_cow(float *M, const float *M0, uint32_t *touched, const void *k,
                               const void *q, const void *C_w, const void *C_r, const void *v,
                               const float *a, const float *b, float *o, int32_t *widx_out,
                               int32_t *ridx_out, const sdm_dims *dims, sdm_stream_t stream);

/* sdm_cow_materialize -- turns a copy-on-write state into a plain one: every
 * row whose bit is clear takes M0's values, then every bit is set (so further
 * copy-on-write steps read M only).  After it, M is exactly the state that
 * sdm_state_init and the same plain steps would have produced.  Uses B, H,
 * n_sub, d_v of dims. */
sdm_status sdm_cow_materialize(float *M, const float *M0, uint32_t *touched, const sdm_dims *dims,
                               sdm_stream_t stream);

/* ---------------------------------------------------------------------------
 * sdm_gates -- the scan's gates from their pre-activations: [P] Sec. 3.1
 * step 2 (per-head forget gate a_t with a learnable decay A, input gate
 * b_t) with the Gated DeltaNet parameterisation that [P] Sec. 4 initialises
 * A and the time-step bias for (the pages print no formula; this is the
 * reading the library implements):
 *   a[b,t,h] = exp(-A[h] * softplus(a_raw[b,t,h] + dt_bias[h]))
 *   b[b,t,h] = 1 / (1 + exp(-b_raw[b,t,h]))        softplus(z) = ln(1 + e^z)
 *   a_raw, b_raw [B,T,H] fp32 (the token's gate projections);
 *   A [H] fp32, >= 0 (the decay rate itself, not its logarithm);
 *   dt_bias [H] fp32;  a, b [B,T,H] fp32 written.
 * fp32 arithmetic.  a may be the same buffer as a_raw and b as b_raw (in
 * place); any other overlap is SDM_ERR_INVALID_ARG.  Negative A or
 * non-finite inputs are not checked (the results are then unspecified).
 * Uses B, T, H of dims.
 * ------------------------------------------------------------------------- */
sdm_status sdm_gates(const float *a_raw, const float *b_raw, const float *A, const float *dt_bias,
                     const sdm_dims *dims, float *a, float *b, sdm_stream_t stream);

/* ---------------------------------------------------------------------------
 * sdm_output_norm_gate -- [P] Sec. 3.1 step 4: the read-out of each
 * token-head is RMS-normalised over its d_v features with a learned gain and
 * gated element-wise, before the head-mixing projection (reading: the
 * Gated DeltaNet output gate, silu(g) = g / (1 + e^-g)):
 *   y[b,t,h,c] = o[b,t,h,c] / sqrt(mean_c' o[b,t,h,c']^2 + eps) * gamma[c] * silu(g[b,t,h,c])
 *   o [B,T,H,d_v] fp32 (sdm_scan_forward's read-out), 16-byte aligned;
 *   g [B,T,H,d_v] in_dtype (the output-gate projection);
 *   gamma [d_v] fp32, 16-byte aligned;  eps finite, >= 0;
 *   y [B,T,H,d_v] in_dtype written (bf16: rounded to nearest even), must
 *   not overlap o, g or gamma.
 * fp32 arithmetic.  Uses B, T, H, d_v (a multiple of 32, <= 1024), in_dtype.
 * ------------------------------------------------------------------------- */
sdm_status sdm_output_norm_gate(const float *o, const void *g, const float *gamma, float eps,
                                const sdm_dims *dims, void *y, sdm_stream_t stream);

/* ---------------------------------------------------------------------------
 * sdm_gates_backward -- reverse mode of sdm_gates (the chain rule through
 * the same formulas): given da = dL/da and db = dL/db [B,T,H] fp32,
 *   da_raw = da * a * (-A[h]) * sigmoid(a_raw + dt_bias[h])
 *   db_raw = db * b * (1 - b)
 *   dA[h]       = sum over (b,t) of da * a * (-softplus(a_raw + dt_bias[h]))
 *   ddt_bias[h] = sum over (b,t) of da_raw
 *   a_raw, b_raw, A, dt_bias: the forward's inputs;
 *   da_raw, db_raw [B,T,H] fp32 written;  dA, ddt_bias [H] fp32 written.
 * workspace: at least sdm_gates_backward_workspace_size(dims) bytes, 4-byte
 * aligned.  fp32 arithmetic; the per-head sums use a fixed order (the same
 * bits on every run).  No output may overlap an input, another output or
 * the workspace (SDM_ERR_INVALID_ARG).  Uses B, T, H of dims.
 * ------------------------------------------------------------------------- */
sdm_status sdm_gates_backward(const float *a_raw, const float *b_raw, const float *A,
                              const float *dt_bias, const float *da, const float *db,
                              const sdm_dims *dims, float *da_raw, float *db_raw, float *dA,
                              float *ddt_bias, void *workspace, size_t workspace_bytes,
                              sdm_stream_t stream);

/* Workspace bytes of sdm_gates_backward for these dims (at most 4 KiB per
 * head: per-part sums of dA and ddt_bias); 0 for invalid dims or no work. */
size_t sdm_gates_backward_workspace_size(const sdm_dims *dims);

/* Workspace bytes of sdm_output_norm_gate_backward for these dims (at most
 * 4 MiB: 1024 partial rows of d_v floats); 0 for invalid dims. */
size_t sdm_output_norm_gate_backward_workspace_size(const sdm_dims *dims);

/* ---------------------------------------------------------------------------
 * sdm_output_norm_gate_backward -- reverse mode of sdm_output_norm_gate.
 * With n = o / sqrt(mean(o^2) + eps) per row, s = sigmoid(g) and
 * q = dy * gamma * g * s:
 *   dout   = (q - n * <q, n> / d_v) / sqrt(mean(o^2) + eps)
 *   dg     = dy * gamma * n * s * (1 + g * (1 - s))
 *   dgamma = sum over the rows of dy * n * g * s
 *   o, g, gamma, eps: the forward's inputs (same layout and alignment);
 *   dy [B,T,H,d_v] fp32 (dL/dy), 16-byte aligned;
 *   dout, dg [B,T,H,d_v] fp32 written, 16-byte aligned;  dgamma [d_v] fp32.
 * workspace: at least sdm_output_norm_gate_backward_workspace_size(dims)
 * bytes, 16-byte aligned.  fp32 arithmetic; dgamma is summed in a fixed
 * order.  No output may overlap an input, another output or the workspace
 * (SDM_ERR_INVALID_ARG).  Uses B, T, H, d_v (a multiple of 32, <= 1024),
 * in_dtype.
 * ------------------------------------------------------------------------- */
sdm_status sdm_output_norm_gate_backward(const float *o, const void *g, const float *gamma,
                                         float eps, const float *dy, const sdm_dims *dims,
                                         float *dout, float *dg, float *dgamma, void *workspace,
                                         size_t workspace_bytes, sdm_stream_t stream);

/* ---------------------------------------------------------------------------
 * sdm_gdn_dense_forward -- the dense Gated DeltaNet recurrence, [P] Sec. 2
 * Eq. 2, which [P] Sec. 3.1 ("Connection to GDN") states the sparse memory
 * reduces to when every slot is selected with a dense key:
 *   S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t
 * for every (b, h), tokens t = 0..T-1 in order, on S in place.  S is stored
 * transposed, like the sparse memory with N = d_k slots:
 *   S [B,H,d_k,d_v] fp32 in/out (row j for key dimension j);
 *   k, q [B,T,H,d_k] and v [B,T,H,d_v] in_dtype (k, q 16-byte aligned);
 *   a, b [B,T,H] fp32;  o [B,T,H,d_v] fp32 written.
 * The same function as sdm_scan_forward with W = R = N = d_k, slot lists
 * 0..N-1 and weights k_t (write) and q_t (read).  fp32 arithmetic; o and S
 * must not overlap each other or the inputs.  Uses B, T, H, d_k (16, 32,
 * 64, 128 or 256), d_v, in_dtype.
 * ------------------------------------------------------------------------- */
sdm_status sdm_gdn_dense_forward(float *S, const void *k, const void *q, const void *v,
                                 const float *a, const float *b, float *o, const sdm_dims *dims,
                                 sdm_stream_t stream);

/* Static description of a status code. */
const char *sdm_status_string(sdm_status status);

/* Per-thread detail message of the last non-OK status ("" if none). */
const char *sdm_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int sdm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SDM_H_ */
