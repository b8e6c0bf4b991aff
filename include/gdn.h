/*
 * gdn.h -- C ABI of the chunked gated delta rule forward pass (GDN prefill)
 * for AMD Instinct MI355X (gfx950).
 *
 * Operation (per sequence n and value head j, key head jk = j / (HV/H)):
 *
 *   S <- S0[n, j]                                   (K x V, zero if absent)
 *   for each token t of the sequence, in order:
 *     qh, kh = q[t, jk], k[t, jk]                   (optionally L2-normalised:
 *                                                    x / sqrt(sum x^2 + 1e-6))
 *     S      = exp(g[t, j]) S
 *     S      = S + kh (beta[t, j] (v[t, j] - S^T kh))^T
 *     out[t, j] = scale S^T qh
 *   final_state[n, j] = S
 *
 * This is the gated delta rule of the Gated Delta Networks paper
 * (arXiv:2412.06464), which the page "NPU Training Operators - GDN" cites in its
 * section on the operator's semantics, computed with the 64-token chunked WY
 * algorithm that the same section lists step by step and that the page
 * "[Qwen3.5][Feature] support fla triton kernel for qwen3.5" (FastDeploy PR
 * #7024) names as the prefill path in its Motivation section.  The argument
 * list mirrors the prefill call in that PR's "Usage or Command" section, item 1
 * (q, k, v, g, beta, scale, initial_state, output_final_state,
 * use_qk_l2norm_in_kernel) plus the FlashAttention-style cu_seqlens that the
 * NPU page's tiling section and the LightLLM page "gdn.py"
 * (_gdn_prefill_kernel) pass for packed variable-length batches.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers to contiguous row-major memory.
 *   - The caller owns every buffer (including the workspace).  The library
 *     never allocates device memory, frees or keeps pointers, and never
 *     synchronises the host (the timing hook below aside):
 *     work is enqueued on `stream` and runs asynchronously.
 *   - All argument checks happen on the host before anything is enqueued; on
 *     error a negative gdn_status is returned and nothing was launched.
 *   - Device-side preconditions (documented, not checked): cu_seqlens is
 *     non-decreasing with cu_seqlens[0] == 0 and cu_seqlens[N] == T;
 *     g <= 0; beta in [0, 1]; no NaN/Inf in the inputs.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_NULL = -1,        /* a required pointer is NULL */
    GDN_ERR_SHAPE = -2,       /* sizes negative or inconsistent (e.g. N != B without cu_seqlens,
                                 B != 1 with cu_seqlens) */
    GDN_ERR_DTYPE = -3,       /* unknown dtype code */
    GDN_ERR_UNSUPPORTED = -4, /* K or V not in {64, 128}, or HV not a multiple of H */
    GDN_ERR_WORKSPACE = -5,   /* workspace NULL, misaligned or too small where required (gdn_chunk_bwd) */
    GDN_ERR_LAUNCH = -6,      /* the HIP runtime reported an error at launch */
    GDN_ERR_ALIGN = -7,       /* a pointer lacks the alignment its argument requires */
    GDN_ERR_SCRATCH = -8      /* gdn_chunk_fwd_noalloc: the sizes need more than the static scratch */
} gdn_status;

/* Element type of q, k, v and out.  g, beta and both states are always fp32.
 * GDN_F32 is a check mode: the same algorithm with fp32 operands everywhere. */
typedef enum gdn_dtype { GDN_BF16 = 0, GDN_F32 = 1 } gdn_dtype;

/* Problem sizes.
 *   B, T  : batch rows and tokens per row of q/k/v/out ([B, T, ...]).  With
 *           cu_seqlens, B must be 1 and T is the total packed token count.
 *   H, HV : key/query heads and value heads; HV % H == 0, value head j uses
 *           key head j / (HV/H) (contiguous groups).
 *   K, V  : key and value head dimensions, each 64 or 128.
 *   N     : number of sequences: N == B without cu_seqlens, else the length
 *           of cu_seqlens minus one.  States are [N, HV, K, V].
 *   dtype : gdn_dtype of q, k, v and out. */
typedef struct gdn_shape {
    int32_t B, T, H, HV, K, V, N;
    int32_t dtype;
} gdn_shape;

/* Bytes of device workspace that let gdn_chunk_fwd (and gdn_chunk_fwd_gated,
 * gdn_chunk_fwd_pool) split long sequences or order a packed batch for
 * `shape`; depends only on the sizes and the dtype.  0 means no workspace is
 * used; invalid shapes also give 0, and gdn_chunk_fwd reports why.
 *
 * The order: a packed batch (cu_seqlens, B = 1) of 2 to 1024 sequences asks
 * for one int32 per sequence (rounded up to 256 bytes).  A one-workgroup
 * kernel ranks the sequences by chunk count, longest first, and the prefill
 * kernel's workgroups take the sequences in that order, so that a long
 * sequence never starts last and sets the tail of the launch (greedy
 * longest-first list scheduling over the CUs).  Results are identical with or
 * without it: only which workgroup computes which sequence changes.
 *
 * The split: a batch of few equal-length sequences (B * HV * V/64 <= 64
 * workgroups, T >= 2048) is too narrow to fill the GPU, so each sequence is
 * cut into 2-8 segments that run side by side.  The recurrence below is linear
 * in S, so a segment's end state is F + M h for a segment started from h, with
 * F its end state from zero and M its K x K transfer map (what the same
 * recurrence computes from the identity with v = 0).  Every segment runs
 * twice without outputs (from zero, and for its map), the segments' starting
 * states follow in order, and every segment runs once more from its starting
 * state, writing the outputs and end states.  Results equal the unsplit pass
 * up to rounding.  The workspace holds the segments' starting states, end
 * states and maps, 4 * B * S * HV * K * (2 V + K) bytes plus small tables:
 * 48 MiB for one sequence of any length with HV = 32, K = V = 128 (S = 8). */
size_t gdn_chunk_fwd_workspace_bytes(const gdn_shape *shape);

/* Chunked gated delta rule forward pass (prefill).
 *
 *   q, k          [B, T, H, K]   dtype          read
 *   v             [B, T, HV, V]  dtype          read
 *   g             [B, T, HV]     fp32           read; log-space forget gate (<= 0)
 *   beta          [B, T, HV]     fp32           read; delta-rule write strength
 *   scale         output scale (the Python binding maps None to 1/sqrt(K))
 *   use_l2norm    non-zero: normalise every q and k row in-kernel
 *   initial_state [N, HV, K, V]  fp32 or NULL   read; NULL = zero state, not read
 *   cu_seqlens    [N+1] int32 or NULL           read on the device only (never
 *                 copied to the host); NULL = B equal-length sequences of T
 *   out           [B, T, HV, V]  dtype          written (every element)
 *   final_state   [N, HV, K, V]  fp32 or NULL   written; NULL = not produced.
 *                 May alias initial_state exactly (in-place state update);
 *                 must not overlap any other argument.
 *   shape         sizes, see gdn_shape (host pointer)
 *   workspace     device scratch of gdn_chunk_fwd_workspace_bytes bytes
 *                 (256-byte aligned), or NULL: long sequences are split, and
 *                 a packed batch ordered, only when it is given and large
 *                 enough, and otherwise run unsplit or in index order (never
 *                 an error); contents on entry are ignored
 *   stream        hipStream_t to enqueue on (NULL = the default stream)
 *
 * `out` must not overlap any input.  Sequences of length 0 produce no rows and
 * their final state equals their initial state (or zero).
 * q, k, v, out, initial_state and final_state must be 16-byte aligned and g,
 * beta and cu_seqlens 4-byte aligned (GDN_ERR_ALIGN otherwise): the kernels
 * move the tensors in 16-byte pieces.
 * Returns GDN_OK or a negative gdn_status (see above). */
int gdn_chunk_fwd(const void *q, const void *k, const void *v,
                  const float *g, const float *beta,
                  float scale, int use_l2norm,
                  const float *initial_state, const int32_t *cu_seqlens,
                  void *out, float *final_state,
                  const gdn_shape *shape, void *workspace, size_t workspace_bytes,
                  void *stream);

/* Bytes of the static device scratch that gdn_chunk_fwd_noalloc uses (one
 * array per GPU the library runs on, held until the process ends). */
#define GDN_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/* gdn_chunk_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, serving loops that keep allocation out of the step,
 * harnesses that forbid hipMalloc.  Same arguments, checks and results as
 * gdn_chunk_fwd given a workspace, minus the workspace: where gdn_chunk_fwd
 * would split long sequences (gdn_chunk_fwd_workspace_bytes(shape) > 0) this
 * call uses the library's static scratch array instead, and neither it nor any
 * routine it calls allocates.  Every split the library plans fits in
 * GDN_STATIC_SCRATCH_BYTES (at most about 50 MiB: the workspace grows with
 * the heads and segments, not with T); a split that did not would be refused
 * with GDN_ERR_SCRATCH before anything is enqueued.  A packed batch of 2 to
 * 1024 sequences keeps its longest-first order there (4 bytes per sequence);
 * other sizes use no scratch.
 *
 * The first call for a device looks up that device's address of the array
 * (hipGetSymbolAddress, with the device of `stream` made current for the
 * lookup); later calls reuse it.  The array keeps whatever the last call left
 * in it; every call writes each part of it before reading it, so nothing
 * needs clearing.  All calls on one GPU share the one array: two calls that
 * use it (a split, or an ordered packed batch) and can run at the same time on
 * one GPU (on different streams, or on unordered streams of different host
 * threads) race and give wrong results; enqueue them on one stream.
 * Returns the statuses of gdn_chunk_fwd and GDN_ERR_SCRATCH. */
int gdn_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                          const float *g, const float *beta,
                          float scale, int use_l2norm,
                          const float *initial_state, const int32_t *cu_seqlens,
                          void *out, float *final_state,
                          const gdn_shape *shape, void *stream);

/* Sizes of a decode step (one token per sequence).
 *   N         : sequences in the step (rows of q/k/v/out)
 *   H, HV     : key/query heads and value heads, as in gdn_shape
 *   K, V      : head dimensions, each 64 or 128
 *   pool_size : slots in the state pool
 *   dtype     : gdn_dtype of q, k, v and out */
typedef struct gdn_decode_shape {
    int32_t N, H, HV, K, V, pool_size;
    int32_t dtype;
} gdn_decode_shape;

/* Fused recurrent decode step with an in-place, pool-indexed state: for every
 * sequence n with a valid slot s = state_indices[n] and every value head j,
 * one token of the recurrence above is applied to pool[s, j]:
 *
 *   S = pool[s, j];  S = exp(g[n, j]) S;  S = S + kh (beta[n, j] (v[n, j] - S^T kh))^T
 *   out[n, j] = scale S^T qh;  pool[s, j] = S
 *
 * This is the decode path that the FastDeploy PR #7024 page lists as its
 * fused recurrent kernel (file table: standard and pool-index interfaces with
 * a PAD_SLOT_ID = -1 sentinel) and calls in "Usage or Command", item 2
 * (q, k, v, g, beta, ssm_pool [max_seqs, HV, K, V] updated in place,
 * ssm_indices [N] int32); the LightLLM page "gdn.py" calls the same operation
 * with ssm_state_indices and an in-place final state (_gdn_decode_kernel).
 *
 *   q, k          [N, H, K]      dtype    read (a [B, 1, H, K] prefill layout with B = N)
 *   v             [N, HV, V]     dtype    read
 *   g, beta       [N, HV]        fp32     read
 *   scale, use_l2norm            as for gdn_chunk_fwd
 *   state_pool    [pool_size, HV, K, V]  fp32  read and written in place
 *                 (16-byte aligned: the state moves in 16-byte pieces)
 *   state_indices [N] int32               read on the device; an entry outside
 *                 [0, pool_size) (the sentinel -1 included) marks a padding row:
 *                 its pool slot is neither read nor written and its out row is
 *                 written as zeros.  Two valid rows must not name the same slot.
 *   out           [N, HV, V]     dtype    written (every element)
 *   shape         sizes (host pointer); stream as for gdn_chunk_fwd
 *
 * No workspace.  out must not overlap any input or the pool.
 * Returns GDN_OK or a negative gdn_status (GDN_ERR_NULL, GDN_ERR_SHAPE for
 * negative sizes or pool_size < 1 with N > 0, GDN_ERR_DTYPE,
 * GDN_ERR_UNSUPPORTED as for gdn_chunk_fwd, GDN_ERR_ALIGN for a state_pool
 * that is not 16-byte aligned, GDN_ERR_LAUNCH). */
int gdn_recurrent_update(const void *q, const void *k, const void *v,
                         const float *g, const float *beta,
                         float scale, int use_l2norm,
                         float *state_pool, const int32_t *state_indices,
                         void *out, const gdn_decode_shape *shape, void *stream);

/* Raw gate inputs, for the entry points that compute the gates themselves:
 *
 *   g    = -exp(A_log[j]) * softplus(a[r, j] + dt_bias[j])
 *   beta = sigmoid(b[r, j])
 *
 * per row r (token) and value head j, in fp32: the fused gating operator of
 * the FastDeploy PR #7024 page (file table and "Usage or Command", item 5),
 * which the LightLLM page "gdn.py" also hands to its decode kernel as A_log,
 * dt_bias, a_raw, b_raw.  softplus(x) = ln(1 + e^x), sigmoid(x) = 1/(1 + e^-x).
 *
 *   A_log, dt_bias  [HV]       fp32   read (device pointers)
 *   a, b            [rows, HV] dtype  read (device pointers; the dtype of the
 *                   call's q/k/v: bf16, or fp32 in the check mode), 4-byte
 *                   aligned */
typedef struct gdn_gates {
    const float *A_log;
    const float *dt_bias;
    const void *a;
    const void *b;
} gdn_gates;

/* The stand-alone gate computation: g and beta [rows, HV] fp32 (written, every
 * element) from `gates` with a, b of type `dtype`.  For callers that keep the
 * gates as tensors (the un-fused prefill of the LightLLM page calls the gating
 * operator, then the chunked kernel).
 * Returns GDN_OK, GDN_ERR_NULL (gates, a pointer of it, g or beta NULL with
 * rows > 0), GDN_ERR_SHAPE (rows < 0, HV <= 0, rows * HV beyond 2^62),
 * GDN_ERR_DTYPE, GDN_ERR_LAUNCH. */
int gdn_gating(const gdn_gates *gates, int64_t rows, int32_t HV, int32_t dtype,
               float *g, float *beta, void *stream);

/* Bytes of device workspace gdn_gating_bwd needs for rows x HV (two floats per
 * head and 64-row block); 0 for invalid sizes or when rows == 0. */
size_t gdn_gating_bwd_workspace_bytes(int64_t rows, int32_t HV);

/* Backward of gdn_gating (training): the gradients of the raw gate inputs,
 * given dg and dbeta [rows, HV] fp32 (the gradients of g and beta, as
 * gdn_chunk_bwd writes them).  By the chain rule through the two gate
 * definitions above (softplus' = sigmoid, sigmoid' = sigmoid (1 - sigmoid)):
 *
 *   da[r, j]    = dg[r, j] * (-exp(A_log[j])) * sigmoid(a[r, j] + dt_bias[j])
 *   db[r, j]    = dbeta[r, j] * beta (1 - beta),   beta = sigmoid(b[r, j])
 *   dA_log[j]   = sum_r dg[r, j] * g[r, j]
 *   ddt_bias[j] = sum_r da[r, j]
 *
 *   gates         A_log, dt_bias [HV] fp32 and a, b [rows, HV] of dtype (read)
 *   dg, dbeta     [rows, HV] fp32 (read)
 *   da, db        [rows, HV] dtype, written (every element; fp32 arithmetic,
 *                 rounded once to dtype)
 *   dA_log, ddt_bias  [HV] fp32, written (zero when rows == 0)
 *   workspace     gdn_gating_bwd_workspace_bytes bytes, 16-byte aligned
 *                 (may be NULL when that is 0); contents on entry ignored
 *
 * The sums over rows are taken in a fixed order (per 64-row block, then over
 * the blocks), so the result is the same on every call.  Returns GDN_OK,
 * GDN_ERR_SHAPE, GDN_ERR_DTYPE, GDN_ERR_NULL (a required pointer NULL: A_log,
 * dt_bias, dA_log, ddt_bias always, the rest when rows > 0), GDN_ERR_ALIGN (a, b
 * not 4-byte aligned), GDN_ERR_WORKSPACE, GDN_ERR_LAUNCH. */
int gdn_gating_bwd(const gdn_gates *gates, int64_t rows, int32_t HV, int32_t dtype,
                   const float *dg, const float *dbeta,
                   void *da, void *db, float *dA_log, float *ddt_bias,
                   void *workspace, size_t workspace_bytes, void *stream);

/* gdn_chunk_fwd with the gates computed in the kernel from `gates` (rows =
 * B * T) instead of read from g and beta: the same result as gdn_gating
 * followed by gdn_chunk_fwd, up to rounding, with no g / beta tensors in
 * memory and one launch.  All other arguments as for gdn_chunk_fwd.  With bf16
 * inputs HV must be even (GDN_ERR_UNSUPPORTED otherwise: the kernel reads
 * each bf16 gate input through the aligned 4-byte word that holds it); a and
 * b must be 4-byte aligned (GDN_ERR_ALIGN). */
int gdn_chunk_fwd_gated(const void *q, const void *k, const void *v,
                        const gdn_gates *gates,
                        float scale, int use_l2norm,
                        const float *initial_state, const int32_t *cu_seqlens,
                        void *out, float *final_state,
                        const gdn_shape *shape, void *workspace, size_t workspace_bytes,
                        void *stream);

/* gdn_recurrent_update with the gates computed in the kernel from `gates`
 * (rows = N; a padding row's inputs are not read), as the LightLLM page's
 * decode call does.  All other arguments as for gdn_recurrent_update. */
int gdn_recurrent_update_gated(const void *q, const void *k, const void *v,
                               const gdn_gates *gates,
                               float scale, int use_l2norm,
                               float *state_pool, const int32_t *state_indices,
                               void *out, const gdn_decode_shape *shape, void *stream);

/* A state pool: the recurrent states of the sequences a server keeps, one
 * slot per sequence, read and updated in place by prefill and decode (the
 * ssm_pool / ssm_indices interface of the FastDeploy PR #7024 page, "Usage or
 * Command" item 2, and the ssm_states buffer with b_ssm_buffer_idx and a
 * bf16 or fp32 state type of the LightLLM page "gdn.py").
 *
 *   data          [pool_size, HV, K, V] of dtype (device); 16-byte aligned in
 *                 fp32, 8-byte in bf16 (GDN_ERR_ALIGN otherwise)
 *   indices       [N] int32 (device): the slot of sequence n.  A slot outside
 *                 [0, pool_size) (the PAD_SLOT_ID -1 of the FastDeploy page
 *                 included) gives the sequence no state: prefill runs it from
 *                 zero and stores nothing, decode writes a zero output row.
 *                 Two sequences must not name the same slot.
 *   pool_size     slots in the pool (>= 1 when N > 0)
 *   dtype         GDN_F32, or GDN_BF16: states are read as bf16 and the
 *                 updated state is rounded to bf16 (nearest even) when stored;
 *                 the arithmetic stays fp32
 *   read_initial  prefill only: non-zero = each sequence starts from its
 *                 slot's state; 0 = from zero (the slot is only written), so
 *                 no dummy zero state is ever read (the FastDeploy page's
 *                 review comments ask for exactly this flag) */
typedef struct gdn_state_pool {
    void *data;
    const int32_t *indices;
    int32_t pool_size;
    int32_t dtype;
    int32_t read_initial;
} gdn_state_pool;

/* Prefill with the states in a pool: as gdn_chunk_fwd (or, when gates is
 * non-NULL, gdn_chunk_fwd_gated, g and beta then unused), with sequence n's
 * initial state read from and its final state written to slot indices[n] of
 * the pool, in place.  Returns the statuses of those calls, and GDN_ERR_NULL
 * (no pool, or no data / indices), GDN_ERR_DTYPE (pool dtype), GDN_ERR_SHAPE
 * (pool_size < 1) and GDN_ERR_ALIGN for the pool. */
int gdn_chunk_fwd_pool(const void *q, const void *k, const void *v,
                       const float *g, const float *beta, const gdn_gates *gates,
                       float scale, int use_l2norm,
                       const gdn_state_pool *pool, const int32_t *cu_seqlens, void *out,
                       const gdn_shape *shape, void *workspace, size_t workspace_bytes,
                       void *stream);

/* Decode with a pool of either state type: as gdn_recurrent_update (or, when
 * gates is non-NULL, gdn_recurrent_update_gated) on pool->data at the slots
 * pool->indices; shape->pool_size must equal pool->pool_size (GDN_ERR_SHAPE);
 * read_initial is ignored (decode always continues the slot's state). */
int gdn_recurrent_update_pool(const void *q, const void *k, const void *v,
                              const float *g, const float *beta, const gdn_gates *gates,
                              float scale, int use_l2norm,
                              const gdn_state_pool *pool, void *out,
                              const gdn_decode_shape *shape, void *stream);

/* Bytes of device workspace gdn_chunk_bwd needs for `shape` (0 for invalid
 * shapes).  The backward pass keeps, per 64-token chunk and value head, the
 * chunk-start state and its gradient (2 K V floats) and three 64 x 64 fp32
 * matrices that are zero above their diagonal 16 x 16 blocks (stored as the
 * ten blocks on and below it), and per token and value head 2 V + 2 K + 1
 * floats: about 2.24 GiB at B = 4, T = 4096, HV = 32, K = V = 128.  Chunk slots are
 * counted for packed sequences (ceil(T/64) + N) when B == 1, else B ceil(T/64). */
size_t gdn_chunk_bwd_workspace_bytes(const gdn_shape *shape);

/* Backward pass of gdn_chunk_fwd (training).  The page "NPU Training
 * Operators - GDN" lists the backward operators next to the forward ones in its
 * operator-semantics section: the gradients of q, k, v, of the gates g and
 * beta (the one of g by a reverse cumulative sum over each chunk) and of the
 * initial state.  Given the forward inputs and the gradients of the forward
 * outputs, it writes the gradients of the forward inputs:
 *
 *   q, k, v, g, beta, scale, use_l2norm, initial_state, cu_seqlens, shape
 *                 exactly as given to gdn_chunk_fwd (read)
 *   dout          [B, T, HV, V]  dtype          read; gradient of out
 *   dht           [N, HV, K, V]  fp32 or NULL   read; gradient of final_state
 *                 (NULL: the final state is not used, gradient zero)
 *   dq, dk        [B, T, H, K]   dtype          written (every element); with
 *                 use_l2norm these are gradients of the raw (unnormalised) rows
 *   dv            [B, T, HV, V]  dtype          written (every element)
 *   dg, dbeta     [B, T, HV]     fp32           written (every element)
 *   dh0           [N, HV, K, V]  fp32 or NULL   written; gradient of
 *                 initial_state (NULL = not produced)
 *   workspace     device scratch of gdn_chunk_bwd_workspace_bytes bytes,
 *                 256-byte aligned (required: GDN_ERR_WORKSPACE otherwise);
 *                 contents on entry are ignored
 *   stream        hipStream_t to enqueue on (NULL = the default stream)
 *
 * q, k, v, dout, dq, dk, dv and the three states must be 16-byte aligned
 * (GDN_ERR_ALIGN otherwise).  Outputs must not overlap each other, the inputs
 * or the workspace.  All
 * arithmetic is fp32 whatever dtype is (bf16 inputs are widened, bf16 outputs
 * rounded to nearest even at the end).  Returns GDN_OK or a negative
 * gdn_status; checks run on the host before anything is enqueued. */
int gdn_chunk_bwd(const void *q, const void *k, const void *v,
                  const float *g, const float *beta,
                  const void *dout, const float *dht,
                  float scale, int use_l2norm,
                  const float *initial_state, const int32_t *cu_seqlens,
                  void *dq, void *dk, void *dv, float *dg, float *dbeta, float *dh0,
                  const gdn_shape *shape, void *workspace, size_t workspace_bytes,
                  void *stream);

/* Kernel timing hook, for measurement.  While enabled, every call of the
 * entry points above records HIP events on its stream just before
 * and just after each kernel it enqueues (events are created on first use and
 * reused).
 * gdn_profile_enable(1) starts recording, gdn_profile_enable(0) stops; both
 * discard what was accumulated so far.  Returns GDN_OK. */
int gdn_profile_enable(int enable);

/* Waits for the recorded events, adds the duration of each recorded launch to
 * its kernel's total and reports, for up to max_kinds kernel kinds of the
 * library: a static name, the accumulated milliseconds and the number of
 * launches.  Any output pointer may be NULL.  Returns the number of kernel
 * kinds.  Host-blocking (it synchronises on the
 * events), so call it outside a timed region. */
int gdn_profile_read(int max_kinds, const char **names, double *total_ms, int64_t *launches);

/* Static, human-readable name of a status code (never NULL). */
const char *gdn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
