/*
 * gdn_cpr.h - C ABI of libgdn_cpr.so: Chunkwise-Parallel Recurrent (CPR) Gated DeltaNet
 * on AMD Instinct MI355X (gfx950).
 *
 * The library computes the gated delta rule, per sequence n, value head h and state row i:
 *     S_t = a_t * S_{t-1} * (I - b_t k_t k_t^T) + b_t v_t k_t^T,      o_t = S_t q_t
 * (Yang, Kautz & Hatamizadeh, "Gated Delta Networks", ICLR 2025), through the three cases
 * that the IsoExec pages name - trainer forward, engine prefill and decode - which must
 * give bitwise identical results (IsoExec, agentlenshq.com: section on the contract
 * structure, cases and regions; section "Chunkwise-Parallel Recurrent (CPR) Gated
 * DeltaNet", including its table where all three CPR stages are bitwise exact).
 *
 * EXECUTION CONTRACT (hashed by gdn_contract_identity; see gdn_contract_string).
 * Each row s = S[i, :] (d_k binary32 values) absorbs token t in this exact order:
 *     x_e = a * s_e                      binary32 multiply, round to nearest even
 *     u   = dot(x, k)                    contract dot product, below
 *     d   = b * (v_i - u)                subtract, then multiply
 *     s_e = fmaf(d, k_e, x_e)            one fused multiply-add per element
 *     o_i = dot(s, q)                    read out from the updated state
 * dot(x, y): GDN_CPR_LEAVES = 16 leaves of d_k/16 contiguous elements; a leaf starts with
 * the rounded product of its first pair and adds the others with fmaf in ascending index;
 * the 16 leaf sums are added pairwise in natural order ((0+1),(2+3),...; then pairs of
 * those; four levels). Binary32 throughout, denormals kept, no fusion other than these
 * fmaf. The fixed binary tree with fp32 accumulation follows the IsoExec page's section on
 * achieving parallel invariance; the per-(region, case) pinning of accumulation dtype and
 * reduction decomposition follows its section on contract structure. The update order,
 * leaf width and pairing are this library's reading of the rule and are part of the
 * identity. q/k head of value head h is h / (Hv / Hk). bf16 inputs are widened exactly.
 * The chunk size C selects only which states are emitted; it changes no output bits.
 *
 * LAYOUTS (row-major, element offsets; all device pointers unless stated otherwise):
 *   cu_seqlens  int32 [N+1], cu_seqlens[0] = 0, nondecreasing, cu_seqlens[N] = T
 *   q, k        [T, Hk, d_k]   binary32 or bfloat16 (gdn_shape_t.qkv_dtype)
 *   v           [T, Hv, d_v]   same dtype as q and k
 *   a, b        float [T, Hv]  decay and write strength, used as given
 *   o           float [T, Hv, d_v]
 *   states      float [.., Hv, d_v, d_k]  (row i of S is d_k contiguous floats)
 * Sequence n owns tokens cu_seqlens[n] .. cu_seqlens[n+1]-1 of the packed batch.
 *
 * OWNERSHIP, STREAMS, ERRORS. The caller allocates every buffer; the library allocates
 * and frees no device memory and keeps no state between calls other than a per-device
 * cache of the compute-unit count, read once. Work is enqueued on the
 * hipStream_t passed as `stream` (NULL = the null stream) of the current HIP device; the
 * calls return before the work finishes. All argument checks run on the host before
 * anything is enqueued, so a non-GDN_OK status means nothing was launched, except
 * GDN_E_DEVICE (a launch error reported by HIP). Device-side values (cu_seqlens contents,
 * pos) cannot be checked on the host: kernels clamp token ranges to [0, T) and skip
 * chunk-state writes past total_chunks, so bad contents give wrong numbers, never
 * out-of-bounds accesses. Outputs must not alias inputs (except the documented in/out
 * state of decode). gdn_last_error() returns text for the calling thread's last error.
 * All functions are thread-safe.
 *
 * TUNING. How many lanes of a wavefront share one state row is chosen per call from the
 * number of rows: 16 when that gives at most two wavefronts per SIMD, 8 when 8 lanes give
 * at most one, 4 otherwise (decode: 32 for d_k >= 32, two rows per group of 32 lanes, else
 * 16; the backward's reverse pass over dL/dS: the widest that keeps at most two wavefronts
 * per SIMD). The environment variable GDN_CPR_LANES_PER_ROW (16, 8 or 4; 32 for decode
 * only) overrides the choice. With two wavefronts per SIMD at
 * 16 lanes, bf16 inputs and d_v a multiple of 32 a scan workgroup has 512 threads
 * (GDN_CPR_SCAN_THREADS=256 keeps 256); at 4 lanes, where rows fill two 32-row wavefronts
 * on every SIMD, each group of 4 lanes holds two rows (GDN_CPR_ROWS_PER_GROUP=1 or 2
 * overrides); and the backward picks its schedule by the number
 * of (sequence, head, row block) units (GDN_CPR_BWD_SCHEDULE=sequences or chunks
 * overrides). The contract makes every admitted choice give the same bits, which the
 * tests check.
 */
#ifndef GDN_CPR_H
#define GDN_CPR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_CPR_ABI_VERSION 3
#define GDN_CPR_LEAVES 16
#define GDN_CPR_IDENTITY_BYTES 32

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_E_NULL = 1,        /* a required pointer is NULL                                */
  GDN_E_SHAPE = 2,       /* sizes are negative, inconsistent or too large             */
  GDN_E_UNSUPPORTED = 3, /* chunk, d_k, d_v or dtype outside the admitted values      */
  GDN_E_IDENTITY = 4,    /* expected_identity differs from this library's contract    */
  GDN_E_DEVICE = 5       /* HIP reported an error when launching                      */
} gdn_status_t;

typedef enum gdn_dtype { GDN_DTYPE_F32 = 0, GDN_DTYPE_BF16 = 1 } gdn_dtype_t;

/* Host struct. Admitted values (claims checked on every call):
 *   num_seqs >= 0; num_qk_heads >= 1; num_v_heads a multiple of num_qk_heads;
 *   d_k in {16, 32, 64, 128}; 1 <= d_v <= 1024; chunk in {16, 32, 64, 128, 256};
 *   num_v_heads * max(d_k, d_v) <= 2^20 (GDN_E_SHAPE otherwise);
 *   qkv_dtype GDN_DTYPE_F32 or GDN_DTYPE_BF16. */
typedef struct gdn_shape {
  int32_t num_seqs;     /* N  */
  int32_t num_qk_heads; /* Hk */
  int32_t num_v_heads;  /* Hv */
  int32_t d_k;
  int32_t d_v;
  int32_t chunk; /* C  */
  int32_t qkv_dtype;
} gdn_shape_t;

/* Library utility (it implements no passage of the pages): the ABI version of the loaded
 * library, GDN_CPR_ABI_VERSION, so that a caller built against another header can refuse
 * it. Host only; cannot fail. */
int32_t gdn_abi_version(void);

/* Canonical contract text for (chunk, d_k): ASCII lines "key=value\n" fixing the rule,
 * operation order, reduction tree, dtypes, rounding, head mapping, chunk boundaries and
 * resync rule. Writes at most buf_len bytes (NUL-terminated when it fits) and the full
 * length, without the NUL, to *out_len. buf may be NULL when buf_len is 0. The text is
 * copied into caller memory rather than returned as a pointer into the library, so its
 * lifetime is the caller's and the call stays thread-safe; ask with buf_len 0 for the size.
 * Host only. Errors: GDN_E_NULL (out_len NULL), GDN_E_UNSUPPORTED (chunk or d_k not
 * admitted), GDN_E_SHAPE (buffer too small; *out_len still set).
 * Identity by content digest follows IsoExec (aihirek.info, section on the contract and
 * common model; agentlenshq.com, section on contract structure: SHA-256 identities). */
gdn_status_t gdn_contract_string(int32_t chunk, int32_t d_k, char *buf, size_t buf_len,
                                 size_t *out_len);

/* SHA-256 (FIPS 180-4) of gdn_contract_string(chunk, d_k) into digest[32] (host memory).
 * Every compute entry point takes this digest as expected_identity and refuses to run
 * when it differs. Host only. Errors: GDN_E_NULL, GDN_E_UNSUPPORTED. */
gdn_status_t gdn_contract_identity(int32_t chunk, int32_t d_k, uint8_t digest[32]);

/* Library utility: SHA-256 (FIPS 180-4) of len bytes at msg (host memory) into
 * digest[32] (host memory); the routine behind gdn_contract_identity, exported so that a
 * caller can hash a contract text it holds and compare identities itself. Host only.
 * Errors: GDN_E_NULL (digest NULL, or msg NULL with len > 0). */
gdn_status_t gdn_sha256(const void *msg, size_t len, uint8_t digest[32]);

/* trainer_fwd: the recurrence over a packed batch, writing o for every token and the state
 * at every C-token chunk boundary (IsoExec, agentlenshq.com, section "Chunkwise-Parallel
 * Recurrent (CPR) Gated DeltaNet"; the trainer-forward case of the contract).
 *   shape, expected_identity : host pointers, required (identity: 32 bytes)
 *   cu_seqlens [N+1], total_tokens T (0 <= T < 2^31)
 *   q, k, v, a, b            : inputs, layouts above
 *   initial_state            : [N, Hv, d_v, d_k] or NULL for zeros
 *   o                        : [T, Hv, d_v] output
 *   chunk_states             : [total_chunks, Hv, d_v, d_k] output; the state after
 *                              in-sequence token j with (j+1) % C == 0, boundary by
 *                              boundary, sequence by sequence: sequence n writes
 *                              floor(T_n / C) states starting at sum_{m<n} floor(T_m / C).
 *                              May be NULL only when total_chunks == 0.
 *   total_chunks             : sum_n floor(T_n / C), 0 <= total_chunks < 2^31
 *   stream                   : hipStream_t or NULL.
 * There is no chunk-offsets argument: each workgroup derives its sequence's first state
 * index, sum_{m<n} floor(T_m / C), from cu_seqlens on the device (64-bit sums, clamped to
 * total_chunks). A caller-supplied copy of those prefix sums could only disagree with
 * cu_seqlens, and the host cannot read device memory to check it. */
gdn_status_t gdn_cpr_trainer_fwd(const gdn_shape_t *shape, const uint8_t *expected_identity,
                                 const int32_t *cu_seqlens, int64_t total_tokens,
                                 const void *q, const void *k, const void *v, const float *a,
                                 const float *b, const float *initial_state, float *o,
                                 float *chunk_states, int64_t total_chunks, void *stream);

/* engine_prefill: the same recurrence over a packed batch of prompts, writing o for every
 * token and the final state of every sequence (IsoExec, agentlenshq.com, section
 * "Chunkwise-Parallel Recurrent (CPR) Gated DeltaNet"; the engine-prefill case).
 *   initial_state [N, Hv, d_v, d_k] or NULL for zeros; o [T, Hv, d_v];
 *   final_state [N, Hv, d_v, d_k] (required; may be the same buffer as initial_state, which
 *   is then updated in place). Other arguments as for gdn_cpr_trainer_fwd. */
gdn_status_t gdn_cpr_prefill(const gdn_shape_t *shape, const uint8_t *expected_identity,
                             const int32_t *cu_seqlens, int64_t total_tokens, const void *q,
                             const void *k, const void *v, const float *a, const float *b,
                             const float *initial_state, float *o, float *final_state,
                             void *stream);

/* engine_decode: one token for each of N sequences, streaming the binary32 state through
 * HBM; at every C-token boundary the new state is also written as the resync checkpoint,
 * equal bit for bit to the trainer's chunk state at that boundary (IsoExec,
 * agentlenshq.com, section "Chunkwise-Parallel Recurrent (CPR) Gated DeltaNet": decode
 * resynchronises the hidden state every C tokens).
 *   pos            int32 [N]: tokens already absorbed by state[n]; the step applies token
 *                  pos[n]; pos[n] < 0 marks an idle slot, whose state, o and resync rows
 *                  are left untouched
 *   q, k [N, Hk, d_k]; v [N, Hv, d_v]; a, b float [N, Hv]
 *   state          float [N, Hv, d_v, d_k], in/out
 *   o              float [N, Hv, d_v] output
 *   resync_states  float [N, Hv, d_v, d_k] or NULL; row block n is written iff
 *                  (pos[n] + 1) % C == 0
 * Other arguments as for gdn_cpr_trainer_fwd. */
gdn_status_t gdn_cpr_decode_step(const gdn_shape_t *shape, const uint8_t *expected_identity,
                                 const int32_t *pos, const void *q, const void *k,
                                 const void *v, const float *a, const float *b, float *state,
                                 float *o, float *resync_states, void *stream);

/* Bytes of device workspace that gdn_cpr_trainer_bwd needs for this shape, total_tokens
 * and total_chunks, into *bytes (host). Host only. Errors: GDN_E_NULL, GDN_E_UNSUPPORTED
 * (chunk not 16, 32, 64, 128 or 256), GDN_E_SHAPE (sizes outside the claims of gdn_cpr_trainer_bwd). */
gdn_status_t gdn_cpr_trainer_bwd_workspace(const gdn_shape_t *shape, int64_t total_tokens,
                                           int64_t total_chunks, size_t *bytes);

/* trainer_bwd: gradients of a scalar loss L through gdn_cpr_trainer_fwd, given dL/do and
 * dL/d(final state), in a fixed operation order, so the same inputs give the same bits on
 * every launch (the backward half of the trainer's forward+backward step in the IsoExec
 * table of stage costs, agentlenshq.com, section "Chunkwise-Parallel Recurrent (CPR) Gated
 * DeltaNet"; the fixed reduction tree with binary32 accumulation follows that page's
 * section on achieving parallel invariance). The pages give no backward arithmetic; this
 * library's order, hashed into the contract identity, is, per row i and token t in reverse
 * order, with sh = dL/dS_t[i, :] (starting from d_final_state, or zeros), g = d_o[t, h, i],
 * s and s_prev the row after and before token t, x = a*s_prev, and u, d as in the forward:
 *     sh_e = fmaf(g, q_e, sh_e)        pq_e = g * s_e
 *     dh = dot(sh, k)   dv_i = b*dh    pb = dh * (v_i - u)
 *     xh_e = fmaf(-dv_i, k_e, sh_e)    pk_e = fmaf(-dv_i, x_e, d * sh_e)
 *     pa = dot(xh, s_prev)             sh_e = a * xh_e
 * dv[t, h, i] = dv_i; d_initial_state[n, h, i, :] = sh after the sequence's first token.
 * dq[t, hk, e], dk[t, hk, e], da[t, h] and db[t, h] sum pq_e, pk_e, pa and pb over the rows
 * i = 0 .. d_v-1 by a pairwise tree in natural order, where at every level a pair whose
 * second member holds no row passes its first member on unchanged; then dq and dk add the
 * value heads of the q/k group hk in ascending order, left to right.
 * Arguments:
 *   shape, expected_identity, cu_seqlens, total_tokens, q, k, v, a, b, initial_state:
 *                    as passed to the gdn_cpr_trainer_fwd call being differentiated;
 *                    (every admitted chunk; C changes no bit of the gradients)
 *   chunk_states     [total_chunks, Hv, d_v, d_k]: that call's output (read only); NULL
 *                    only when total_chunks == 0
 *   total_chunks     sum_n floor(T_n / C), as for gdn_cpr_trainer_fwd
 *   d_o              float [T, Hv, d_v]: dL/do (required when T > 0)
 *   d_final_state    float [N, Hv, d_v, d_k]: dL/d(state after each sequence's last token),
 *                    or NULL for zeros
 *   dq, dk           float [T, Hk, d_k] outputs; dv float [T, Hv, d_v]; da, db float [T, Hv]
 *                    (required when T > 0)
 *   d_initial_state  float [N, Hv, d_v, d_k] output, written whether or not initial_state
 *                    is NULL (required when N > 0)
 *   workspace        device memory of at least gdn_cpr_trainer_bwd_workspace() bytes,
 *                    256-byte aligned, owned by the caller; its contents on entry do not
 *                    matter and are overwritten. Calls that share a workspace must not run
 *                    concurrently.
 *   stream           hipStream_t or NULL.
 * Outputs must not alias inputs, each other or the workspace. Errors: as for
 * gdn_cpr_trainer_fwd; GDN_E_UNSUPPORTED for chunk 128 or 256; GDN_E_NULL for a missing
 * required pointer or workspace; GDN_E_SHAPE for total_chunks outside [0, T / C], a
 * workspace smaller than reported or misaligned, or a grid too large. */
gdn_status_t gdn_cpr_trainer_bwd(const gdn_shape_t *shape, const uint8_t *expected_identity,
                                 const int32_t *cu_seqlens, int64_t total_tokens,
                                 const void *q, const void *k, const void *v, const float *a,
                                 const float *b, const float *initial_state,
                                 const float *chunk_states, int64_t total_chunks,
                                 const float *d_o, const float *d_final_state, float *dq,
                                 float *dk, float *dv, float *da, float *db,
                                 float *d_initial_state, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory - code under HIP graph capture, tight
 * serving or training loops, harnesses that forbid allocation: gdn_cpr_trainer_bwd with the
 * workspace taken from a fixed device array inside the library instead of the caller.
 * Arguments, outputs, bits and errors as for gdn_cpr_trainer_bwd (which it shares every
 * kernel with), without workspace and workspace_bytes. The call allocates nothing: the
 * array, GDN_CPR_BWD_NOALLOC_MAX_BYTES bytes, is part of the library's device code, one per
 * GPU the library runs on, held until the process ends; its address on a device is looked
 * up on the first call there. Sizes whose workspace (gdn_cpr_trainer_bwd_workspace) exceeds
 * GDN_CPR_BWD_NOALLOC_MAX_BYTES are refused with GDN_E_SHAPE before anything is launched.
 * All calls on one GPU share that GPU's array: calls that overlap on one GPU (other
 * streams, other threads) race and must be ordered by the caller. The array's contents
 * between calls do not matter; every call writes what it reads. Host only. */
#define GDN_CPR_BWD_NOALLOC_MAX_BYTES ((size_t)128 << 20)
gdn_status_t gdn_cpr_trainer_bwd_noalloc(const gdn_shape_t *shape,
                                         const uint8_t *expected_identity,
                                         const int32_t *cu_seqlens, int64_t total_tokens,
                                         const void *q, const void *k, const void *v,
                                         const float *a, const float *b,
                                         const float *initial_state, const float *chunk_states,
                                         int64_t total_chunks, const float *d_o,
                                         const float *d_final_state, float *dq, float *dk,
                                         float *dv, float *da, float *db,
                                         float *d_initial_state, void *stream);

/* Host struct of the linear region: Y [m, n] = X [m, k] W [k, n], all row-major.
 * Admitted: 0 <= m, n < 2^31; k a positive multiple of 512 up to 2^24; x_dtype and w_dtype
 * GDN_DTYPE_F32 or GDN_DTYPE_BF16. */
typedef struct gdn_linear_shape {
  int64_t m, n, k;
  int32_t x_dtype, w_dtype;
} gdn_linear_shape_t;

/* linear: Y = X W in which every output is the contract dot of a row of X and a column of
 * W, so its bits depend on that row and column only: not on m (batch invariance), the tile
 * or the schedule. This is the second region of the contract: the IsoExec pages make a
 * tensor-parallel matrix product invariant by splitting K into contiguous leaves, each
 * accumulated in binary32 on the matrix units in a fixed schedule, combined in a fixed
 * order (agentlenshq.com, section on achieving parallel invariance: tensor parallelism).
 * Here the 16 leaves of k/16 run on gfx950's binary32 matrix instructions, whose every
 * step is a fused multiply-add in ascending k, and are added by the dot's pairwise tree.
 *   shape, expected_identity : host pointers; the identity of any admitted (chunk, d_k),
 *                              one- or two-level (the linear rule is in every contract text)
 *   x  [m, k], w [k, n]      : binary32, or bfloat16 widened exactly; 16-byte aligned
 *   y  [m, n]                : binary32 output, 4-byte aligned; must not alias x or w
 *   stream                   : hipStream_t or NULL.
 * Errors: GDN_E_NULL, GDN_E_IDENTITY, GDN_E_SHAPE (sizes, alignment),
 * GDN_E_UNSUPPORTED (k or dtype not admitted), GDN_E_DEVICE. m == 0 or n == 0 does
 * nothing. */
gdn_status_t gdn_linear_fwd(const gdn_linear_shape_t *shape, const uint8_t *expected_identity,
                            const void *x, const void *w, float *y, void *stream);

/* ------------------------------------------------------------------------------------
 * TWO-LEVEL READING of CPR. The IsoExec pages describe CPR as the recurrence made primary
 * but parallelised across chunks, with decode resynchronising its hidden state every C
 * tokens (agentlenshq.com, section "Chunkwise-Parallel Recurrent (CPR) Gated DeltaNet").
 * Read literally, the state at each chunk boundary comes from a chunkwise transition and
 * the outputs from the recurrence restarted at each boundary, all chunks in parallel. The
 * rows' update over a full chunk of C tokens is affine, S_end = S_start A_c + B_c, where
 *   A_c [d_k, d_k]: unit rows e_j that absorb the chunk's tokens with v = +0,
 *   B_c [d_v, d_k]: +0 rows that absorb them with the chunk's v,
 * both through the contract row update above. Then, per sequence and value head,
 *   S_0 = initial state;  S_{c+1}[i, j] = B_c[i, j] + sum_k S_c[i, k] A_c[k, j]
 * as one fused multiply-add per k, k ascending, starting from B_c[i, j] (on gfx950's
 * binary32 matrix instructions); the outputs of chunk c are those of rows that restart from
 * S_c and absorb its tokens; the final state is S after the last full chunk when T_n is a
 * multiple of C, else the restarted rows after the last token. Decode runs the rows from
 * the boundary state token by token, keeps the chunk's tokens in a C-slot cache, and after
 * a chunk's last token rebuilds A_c and B_c from the cache and sets the running state, the
 * boundary state and the resync checkpoint to S_{c+1}. The three cases give the same bits
 * (outputs, boundary states, final state) as one another, not as the one-level calls: the
 * reading has its own contract text and identity. Admitted d_k: 32, 64 or 128.
 * ------------------------------------------------------------------------------------ */

/* Contract text and SHA-256 identity of the two-level reading for (chunk, d_k): the
 * canonical text with its "cpr=" line replaced by the two-level lines. Host only. Errors
 * as for gdn_contract_string / gdn_contract_identity; GDN_E_UNSUPPORTED also for d_k 16. */
gdn_status_t gdn_cpr2_contract_string(int32_t chunk, int32_t d_k, char *buf, size_t buf_len,
                                      size_t *out_len);
gdn_status_t gdn_cpr2_contract_identity(int32_t chunk, int32_t d_k, uint8_t digest[32]);

/* Bytes of device workspace that the two-level calls need, into *bytes (host). decode == 0:
 * for gdn_cpr2_trainer_fwd and gdn_cpr2_prefill over total_tokens tokens and total_chunks
 * full chunks (the prefill figure also holds its boundary states, so it is the larger);
 * decode != 0: for gdn_cpr2_decode_step (total_tokens, total_chunks ignored). Host only.
 * Errors: GDN_E_NULL, GDN_E_SHAPE. */
gdn_status_t gdn_cpr2_workspace(const gdn_shape_t *shape, int64_t total_tokens,
                                int64_t total_chunks, int32_t decode, size_t *bytes);

/* trainer_fwd, two-level: o for every token and chunk_states [total_chunks, Hv, d_v, d_k]
 * = S_1, S_2, ... of every sequence, laid out as for gdn_cpr_trainer_fwd.
 *   expected_identity : gdn_cpr2_contract_identity(chunk, d_k)
 *   workspace         : device, 256-byte aligned, at least gdn_cpr2_workspace(decode = 0)
 *                       bytes; its contents on entry do not matter
 * Other arguments and errors as for gdn_cpr_trainer_fwd, plus GDN_E_SHAPE when the
 * workspace is short or misaligned. Launches four kernels on the stream: the chunk plan,
 * the transitions of all full chunks, the boundary sweep, the outputs. */
gdn_status_t gdn_cpr2_trainer_fwd(const gdn_shape_t *shape, const uint8_t *expected_identity,
                                  const int32_t *cu_seqlens, int64_t total_tokens,
                                  const void *q, const void *k, const void *v, const float *a,
                                  const float *b, const float *initial_state, float *o,
                                  float *chunk_states, int64_t total_chunks, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* engine_prefill, two-level: o for every token and final_state [N, Hv, d_v, d_k]
 * (required unless N == 0; must not alias initial_state). total_chunks =
 * sum_n floor(T_n / C) sizes the boundary states, which live in the workspace. Other
 * arguments as for gdn_cpr2_trainer_fwd. */
gdn_status_t gdn_cpr2_prefill(const gdn_shape_t *shape, const uint8_t *expected_identity,
                              const int32_t *cu_seqlens, int64_t total_tokens, const void *q,
                              const void *k, const void *v, const float *a, const float *b,
                              const float *initial_state, float *o, float *final_state,
                              int64_t total_chunks, void *workspace, size_t workspace_bytes,
                              void *stream);

/* engine_decode, two-level: one token for each of N sequences.
 *   pos                 int32 [N], tokens already absorbed (pos[n] < 0: idle slot, nothing
 *                       of it is read or written)
 *   q, k, v, a, b       the step's token, layouts as for gdn_cpr_decode_step
 *   state               float [N, Hv, d_v, d_k], in/out: the running rows
 *   boundary            float [N, Hv, d_v, d_k], in/out: S_c of the chunk in progress
 *   cache_k [N, C, Hk, d_k], cache_v [N, C, Hv, d_v] (qkv dtype), cache_a, cache_b
 *                       float [N, C, Hv]: in/out, the chunk's tokens so far (slot pos % C);
 *                       contents before a sequence's first step do not matter
 *   o                   float [N, Hv, d_v] output
 *   resync_states       float [N, Hv, d_v, d_k] or NULL: written with S_{c+1} iff
 *                       (pos[n] + 1) % C == 0
 *   workspace           device, 256-byte aligned, gdn_cpr2_workspace(decode != 0) bytes
 * A sequence starts with pos = 0 and state = boundary = its initial state; to continue
 * after a two-level prefill of P tokens, set state = its final state, boundary = the last
 * chunk state S_{floor(P/C)} (gdn_cpr2_trainer_fwd's, or the initial state if P < C) and
 * cache slots 0 .. P % C - 1 = the tokens after that boundary. After a step
 * with (pos[n] + 1) % C == 0, state = boundary = resync = S_{c+1}, equal bit for bit to
 * gdn_cpr2_trainer_fwd's chunk state there. Overlapping calls that share the workspace
 * race. Errors as for gdn_cpr_decode_step, plus the workspace and cache checks. */
gdn_status_t gdn_cpr2_decode_step(const gdn_shape_t *shape, const uint8_t *expected_identity,
                                  const int32_t *pos, const void *q, const void *k,
                                  const void *v, const float *a, const float *b, float *state,
                                  float *boundary, void *cache_k, void *cache_v,
                                  float *cache_a, float *cache_b, float *o,
                                  float *resync_states, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* Library utility: text describing the calling thread's last non-GDN_OK status ("" if
 * none). The pointer stays valid until the thread's next call into the library. Host only;
 * cannot fail. */
const char *gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_CPR_H */
