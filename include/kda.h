/*
 * kda.h -- C ABI of the MI355X (gfx950) chunkwise-parallel KDA forward pass.
 *
 * Kimi Delta Attention (KDA) is a gated delta-rule recurrence with a
 * per-channel decay.  Per sequence and head, with state S (d_k x d_v):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t                         alpha_t = exp(log_alpha_t)
 *
 * (ogis-ri NLP primer on Kimi K3, §3.1 "KDA（Kimi Delta Attention）": state and
 * operand shapes, the decay / probe / delta / write decomposition, and the
 * read-out).  The library evaluates it chunk by chunk (same page, §3.1, the
 * chunkwise form and "chunk 内の減衰と、その数値範囲"), relying on the bounded
 * log-decay log_alpha >= -5 so that every 16-token diagonal sub-tile is an
 * ordinary dense matrix product (orkas.ai "Kimi K3 architecture",
 * §"GPU のコードパスを一本消した「下界」").
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers on the current HIP device,
 *     contiguous, token-major with heads interleaved:
 *         q, k, log_alpha : [total_tokens, n_heads, d_k]   (dtype dt)
 *         v, o            : [total_tokens, n_heads, d_v]   (dtype dt)
 *         beta            : [total_tokens, n_heads]        (dtype dt)
 *         S0, S_T         : [n_seqs, n_heads, d_k, d_v]    (float32, row = key channel)
 *         cu_seqlens      : [n_seqs + 1] int32, cu[0] = 0, nondecreasing,
 *                           cu[n_seqs] = total_tokens (packed variable-length
 *                           batch); NULL = n_seqs equal lengths.
 *     Each sequence starts from its own S0[n] (zeros if S0 == NULL); there is
 *     no leakage across sequences.  o has the input dtype (rounded to nearest
 *     even for bf16); S_T is float32.
 *   - The caller owns every buffer, including the workspace.  The library
 *     never allocates device memory, frees or synchronises; work is enqueued
 *     on `stream` and the call returns once it is queued.  Library-held
 *     state is limited to one side stream per device with its events
 *     (created on first use, default priority, guarded by a mutex; see
 *     kda_chunk_fwd) and the array of kda_chunk_fwd_noalloc; concurrent
 *     calls on different workspaces are safe.
 *   - Argument errors are detected on the host before anything is enqueued;
 *     on error nothing is written.  Value ranges are not checked: log_alpha
 *     must lie in [-5, 0] and beta in [0, 1] for the documented accuracy
 *     (values outside give unspecified results, possibly inf or NaN: below
 *     -5 the in-chunk decay factors can overflow; never a memory
 *     access outside the buffers described here).  Device-side cu_seqlens
 *     that break the rules above give unspecified results but every access
 *     stays inside the buffers.
 *   - Supported by every entry point (the tuned sizes): chunk == 64 and
 *     d_k == d_v, with dt == KDA_BF16 at d in {64, 128} or dt == KDA_F32 at
 *     d == 64; total_tokens < 2^31; n_heads <= 65535.  kda_chunk_fwd,
 *     kda_chunk_fwd_profile and kda_chunk_fwd_noalloc also take chunk in
 *     {16, 32, 64, 128} with any d_k, d_v in {64, 128} and either dtype; the
 *     sizes outside the tuned ones run untuned fp32 kernels (see
 *     kda_chunk_fwd).  Anything else returns KDA_ERR_UNSUPPORTED.
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
    KDA_ERR_NULL = 1,          /* a required pointer is NULL */
    KDA_ERR_SHAPE = 2,         /* inconsistent sizes (e.g. total_tokens not divisible by n_seqs) */
    KDA_ERR_DTYPE = 3,         /* unknown dtype code */
    KDA_ERR_UNSUPPORTED = 4,   /* valid but unsupported sizes */
    KDA_ERR_WORKSPACE = 5,     /* workspace NULL, too small or misaligned */
    KDA_ERR_HIP = 6            /* a kernel launch failed (hipGetLastError) */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* Bytes of device workspace kda_chunk_fwd needs for these sizes (0 if the
 * sizes are invalid or unsupported).  The workspace must be 256-byte aligned. */
size_t kda_chunk_fwd_workspace_size(int64_t total_tokens, int32_t n_seqs, int32_t n_heads,
                                    int32_t d_k, int32_t d_v, int32_t chunk, kda_dtype dt);

/* Chunkwise-parallel KDA forward: o and (optionally) the final per-sequence
 * states S_T for the recurrence above (ogis-ri NLP primer on Kimi K3, §3.1
 * "KDA"), over a packed batch of n_seqs sequences.
 *   q, k, v, beta, log_alpha : inputs, layouts above (read only)
 *   S0         : initial states or NULL (zeros)
 *   cu_seqlens : device int32 [n_seqs+1] or NULL (equal lengths)
 *   o          : output [total_tokens, n_heads, d_v], dtype dt (required)
 *   S_T        : output [n_seqs, n_heads, d_k, d_v] float32, or NULL
 *   workspace  : >= kda_chunk_fwd_workspace_size(...) bytes of device memory
 *   stream     : HIP stream (hipStream_t) the work is queued on; NULL = default
 * total_tokens == 0 is valid: o is empty and S_T (if given) receives S0
 * (or zeros).  Every tensor pointer must be 16-byte aligned (KDA_ERR_SHAPE
 * otherwise).
 * Chunk size and head dims: the result does not depend on the chunk size
 * (up to rounding: the chunked form is an exact regrouping of the
 * recurrence).  Chunk 64 with d_k == d_v (bf16 at 64 or 128, fp32 at 64)
 * runs the tuned kernels (bf16 MFMA operands at bf16, fp32 at fp32); every
 * other supported size -- chunk 16, 32 or 128, d_k != d_v, fp32 at 128 --
 * runs generic kernels in fp32 arithmetic (fp32 operands, fp32 matrix
 * cores), correct to the same bars but several times slower than the tuned
 * path.  Their workspace is fp32: about
 * 4 (3 d_k + 2 chunk + d_k / chunk) bytes per (token, head).
 * Launch shapes (results do not depend on them): the sequential pass takes
 * 32 value columns per workgroup when the (sequence, head) chains at 16
 * columns would outnumber the device's CUs, else 16.  Equal-length bf16
 * batches of at least 2048 chunks per sequence whose 16-column chains fill
 * at most half of the CUs are pipelined by token blocks: the chunk-parallel
 * stage of the next block runs on the library's side stream beside the
 * sequential pass of this one (on a 256-CU device on XCDs 4..7 and 0..3
 * respectively); `stream` waits for all of it before any later work. */
kda_status kda_chunk_fwd(kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads,
                         int32_t d_k, int32_t d_v, int32_t chunk,
                         const void* q, const void* k, const void* v,
                         const void* beta, const void* log_alpha,
                         const float* S0, const int32_t* cu_seqlens,
                         void* o, float* S_T,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Size of the device array that kda_chunk_fwd_noalloc uses as its workspace
 * (64 MiB: about 60,000 (token, head) pairs at d_k = d_v = 128, e.g. 3,584
 * tokens x 16 heads). */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)

/* kda_chunk_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, kernels and results, minus the workspace, which is a
 * fixed device array of KDA_NOALLOC_SCRATCH_BYTES inside this library (one
 * per GPU, held until the process ends; its address is looked up once per
 * GPU, with that GPU current, on the first call there).  The call allocates
 * nothing and never uses a second stream.
 * Errors: as kda_chunk_fwd; KDA_ERR_WORKSPACE when
 * kda_chunk_fwd_workspace_size(...) exceeds KDA_NOALLOC_SCRATCH_BYTES;
 * KDA_ERR_HIP if the array's address cannot be found.
 * All calls on one GPU share the array: calls that overlap in time on one
 * GPU (on different streams, or from several threads without ordering)
 * race and give wrong results.  Calls on one stream are ordered and safe.
 * Nothing in the array needs to start at zero (each call writes every
 * region it later reads). */
kda_status kda_chunk_fwd_noalloc(kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads,
                                 int32_t d_k, int32_t d_v, int32_t chunk,
                                 const void* q, const void* k, const void* v,
                                 const void* beta, const void* log_alpha,
                                 const float* S0, const int32_t* cu_seqlens,
                                 void* o, float* S_T, void* stream);

/* Bytes of the state-checkpoint buffer kda_chunk_fwd_ckpt writes into for a
 * given `every`: floor((floor(total_tokens / 64) + n_seqs) / every) slots x
 * n_heads x d_k x d_v float32 -- an upper bound on the checkpoints any
 * split of total_tokens into n_seqs sequences produces (0 if the sizes are
 * invalid or every < 1). */
size_t kda_chunk_ckpt_size(int64_t total_tokens, int32_t n_seqs, int32_t n_heads, int32_t d_k, int32_t d_v,
                           int32_t every);

/* kda_chunk_fwd that also emits the recurrent state at chosen chunk
 * boundaries, the prefix-cache checkpoints of the serving side (orkas.ai
 * "Kimi K3 architecture", §"請求書はサービング側に回ってくる": prefixes are
 * hashed in 512-token units and the recurrent state is checkpointed only at a
 * sparse subset of those ends).  Same arguments, results and errors as
 * kda_chunk_fwd, plus:
 *   every        : >= 1; after chunk j of a sequence (0-based, 64 tokens
 *                  each, the last one possibly partial) with (j + 1) % every
 *                  == 0 -- i.e. after its first min(64 (j + 1), len) tokens
 *                  -- the state is written (every = 8: every 512 tokens)
 *   S_ckpt       : device float32 [slots][n_heads][d_k][d_v]; the state after
 *                  chunk j of sequence n goes to slot ck0(n) + (j + 1) / every
 *                  - 1, where ck0(n) is the sum of floor(ceil(len_m / 64) /
 *                  every) over the sequences m < n (the checkpoints are
 *                  packed: slot i holds the i-th checkpoint in sequence
 *                  order); slots past the last checkpoint are not written.
 *                  The same values as kda_chunk_fwd's S_T of that prefix.
 *   S_ckpt_bytes : size of S_ckpt; at least
 *                  kda_chunk_ckpt_size(total_tokens, n_seqs, n_heads, d_k,
 *                  d_v, every).
 * KDA_ERR_SHAPE if every < 1, KDA_ERR_NULL if S_ckpt is NULL,
 * KDA_ERR_WORKSPACE if S_ckpt_bytes is too small, and KDA_ERR_UNSUPPORTED
 * for KDA_F32. */
kda_status kda_chunk_fwd_ckpt(kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads,
                              int32_t d_k, int32_t d_v, int32_t chunk,
                              const void* q, const void* k, const void* v,
                              const void* beta, const void* log_alpha,
                              const float* S0, const int32_t* cu_seqlens,
                              void* o, float* S_T, int32_t every, float* S_ckpt, size_t S_ckpt_bytes,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Measurement entry point: the same work as kda_chunk_fwd (same arguments,
 * same results), with a HIP event recorded on `stream` before and after each
 * kernel launch.  Unlike kda_chunk_fwd it BLOCKS until the pass has finished
 * (it synchronises on its last event), then writes each launch's duration in
 * milliseconds to stage_ms[0 .. kda_profile_num_stages()-1] (host memory,
 * required).  It creates and destroys its events; it allocates no device
 * memory.  Errors as for kda_chunk_fwd; KDA_ERR_NULL if stage_ms is NULL.
 * On the generic sizes stage 1 ("k_prep") times the two chunk-parallel
 * kernels together and stage 2 ("k_recur") the sequential one. */
kda_status kda_chunk_fwd_profile(kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads,
                                 int32_t d_k, int32_t d_v, int32_t chunk,
                                 const void* q, const void* k, const void* v,
                                 const void* beta, const void* log_alpha,
                                 const float* S0, const int32_t* cu_seqlens,
                                 void* o, float* S_T,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 float* stage_ms);

/* Transition matrices of a packed batch: for each sequence n and head h,
 *     P[n, h] = prod over its tokens, last first, of (I - beta_t k_t k_t^T) Diag(alpha_t)
 * so that the sequence maps an incoming state S to P S + Z, Z being its
 * zero-start final state (kda_chunk_fwd with S0 = NULL).  This is the
 * segment transition of sequence-parallel state passing (orkas.ai "Kimi K3
 * architecture", §"請求書はサービング側に回ってくる"): with a long sequence cut into
 * segments, the states entering the segments follow from every segment's
 * (P, Z) by kda_compose_states, after which each segment's outputs are
 * kda_chunk_fwd from its incoming state.  Computed by the chunked pass with
 * v = 0 from S0 = I (no output is produced).
 *   k, beta, log_alpha, cu_seqlens : as for kda_chunk_fwd (q and v are not used)
 *   P : output [n_seqs, n_heads, d_k, d_k] float32
 *   workspace : >= kda_chunk_fwd_workspace_size(total_tokens, n_seqs, n_heads,
 *               d_k, d_k, chunk, dt) bytes
 * Supported: dt == KDA_BF16, d_k in {64, 128}, chunk == 64; otherwise as
 * kda_chunk_fwd.  Enqueued on `stream`, never synchronises. */
kda_status kda_chunk_transition(kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads,
                                int32_t d_k, int32_t chunk,
                                const void* k, const void* beta, const void* log_alpha,
                                const int32_t* cu_seqlens, float* P,
                                void* workspace, size_t workspace_bytes, void* stream);

/* State composition of sequence-parallel state passing: for n_segments
 * consecutive segments of one sequence with transitions P[g] and zero-start
 * states Z[g] (per head), the states entering the segments:
 *     S_in[0] = S0 (zeros if NULL),  S_in[g+1] = P[g] S_in[g] + Z[g]
 * (S_in[n_segments] is the final state).  fp32 throughout.
 *   P    : [n_segments, n_heads, d, d]       Z : [n_segments, n_heads, d, d]
 *   S0   : [n_heads, d, d] or NULL           S_in : output [n_segments + 1, n_heads, d, d]
 * Supported: d in {64, 128}; n_segments >= 1.  S_in must not overlap P, Z
 * or S0.  Enqueued on `stream`, never synchronises. */
kda_status kda_compose_states(int32_t n_segments, int32_t n_heads, int32_t d, const float* P,
                              const float* Z, const float* S0, float* S_in, void* stream);

/* Token-by-token KDA update for decoding: each of n_seqs sequences advances
 * its cached state by n_tokens >= 1 tokens with the recurrence above, taken
 * one token at a time (ogis-ri NLP primer on Kimi K3, §3.1 "KDA": decay,
 * probe, delta, write, read-out), and emits their outputs.  Same layouts as
 * kda_chunk_fwd with n_seqs equal-length sequences of n_tokens tokens:
 *   q, k, log_alpha : [n_seqs * n_tokens, n_heads, d_k]   (dtype dt)
 *   v, o            : [n_seqs * n_tokens, n_heads, d_v]   (dtype dt)
 *   beta            : [n_seqs * n_tokens, n_heads]        (dtype dt)
 *   S_in            : [n_seqs, n_heads, d_k, d_v] float32, or NULL (zeros)
 *   S_out           : [n_seqs, n_heads, d_k, d_v] float32 (required); may be
 *                     the same buffer as S_in (updated in place)
 * Meant for a few tokens per call (the work per sequence and head is
 * sequential over its tokens); longer spans belong to kda_chunk_fwd, which
 * gives the same results.  Needs no workspace.  Supported: d_k == d_v in
 * {64, 128}, dt KDA_F32 or KDA_BF16; n_seqs * n_tokens < 2^31.  Enqueued on
 * `stream`, never synchronises; errors as for kda_chunk_fwd. */
kda_status kda_recurrent_fwd(kda_dtype dt, int32_t n_seqs, int32_t n_tokens, int32_t n_heads,
                             int32_t d_k, int32_t d_v,
                             const void* q, const void* k, const void* v,
                             const void* beta, const void* log_alpha,
                             const float* S_in, float* S_out, void* o, void* stream);

/* Speculative-decoding commit (orkas.ai "Kimi K3 architecture",
 * §"請求書はサービング側に回ってくる", speculative decoding: the state is
 * updated in place, so a rejected draft cannot be undone; only the much
 * smaller projected inputs are cached and the state is rebuilt on chip).
 * Same as kda_recurrent_fwd over n_tokens cached draft token slots per
 * sequence, except that sequence n takes only its first n_accept[n] of them:
 *   n_accept : device int32 [n_seqs] (4-byte aligned, required); each value
 *              is clamped to [0, n_tokens], so 0 leaves the state as S_in
 *              (copied to S_out when they differ)
 *   o        : as for kda_recurrent_fwd, or NULL (state only); only the rows
 *              of taken tokens are written, the others are left untouched
 * The usual flow keeps S_in, runs the draft with kda_recurrent_fwd into a
 * separate S_out, and once the verifier has fixed n_accept calls this with
 * S_out == S_in and o == NULL.  The state it leaves equals, bit for bit,
 * the one kda_recurrent_fwd reaches over the same accepted tokens.  Sizes,
 * dtypes, alignment and errors as for kda_recurrent_fwd.  Enqueued on
 * `stream`, never synchronises. */
kda_status kda_recurrent_commit(kda_dtype dt, int32_t n_seqs, int32_t n_tokens, int32_t n_heads,
                                int32_t d_k, int32_t d_v,
                                const void* q, const void* k, const void* v,
                                const void* beta, const void* log_alpha, const int32_t* n_accept,
                                const float* S_in, float* S_out, void* o, void* stream);

/* Output epilogue of a KDA layer (ogis-ri NLP primer on Kimi K3, §3.1
 * "KDA": the read-out is normalised by RMSNorm because its magnitude varies
 * with the state, then multiplied channel by channel by a gate in (0, 1)
 * made from the layer input; the output projection W_o follows and is not
 * part of this call).  The printed formula was lost; this library reads it
 * as, per row (one token of one head, d_v channels):
 *     y = o / sqrt(mean(o^2) + eps) * w * sigmoid(gate)
 *   o, gate, y : [n_rows, d_v] contiguous, dtype dt (n_rows = tokens x heads
 *                for the [T, H, d_v] layout of kda_chunk_fwd's o); y may be o
 *                (in place); gate holds the pre-activations
 *   weight     : [d_v] float32 per-channel scale, or NULL (ones)
 *   eps        : in [0, 1] (KDA_ERR_SHAPE otherwise, NaN included)
 * Supported: d_v in {64, 128}, dt KDA_F32 or KDA_BF16; pointers 16-byte
 * aligned.  n_rows == 0 is valid (nothing is done).  Needs no workspace;
 * enqueued on `stream`, never synchronises. */
kda_status kda_output_gate(kda_dtype dt, int64_t n_rows, int32_t d_v, const void* o, const void* gate,
                           const float* weight, float eps, void* y, void* stream);

/* Debug check of the value-range preconditions that the compute entry points
 * do not check: counts[0] receives the number of log_alpha elements outside
 * [-5, 0] or not finite, counts[1] the number of beta elements outside
 * [0, 1] or not finite, counts[2] the number of cu_seqlens entries that break
 * cu[0] == 0, cu[i] <= cu[i+1], cu[n_seqs] == total_tokens (0 when
 * cu_seqlens is NULL).  `counts` is caller-owned DEVICE memory for 3
 * uint64 values (8-byte aligned); the call clears and fills it on `stream`
 * and returns without synchronising, so read it after the stream has
 * reached this point.  Argument errors as for kda_chunk_fwd. */
kda_status kda_validate_inputs(kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads,
                               int32_t d_k, const void* beta, const void* log_alpha,
                               const int32_t* cu_seqlens, unsigned long long* counts, void* stream);

/* Bytes of device workspace kda_chunk_bwd needs for these sizes (0 if the
 * sizes are invalid or unsupported, including dt == KDA_F32).  256-byte
 * aligned.  It holds the forward quantities the backward pass keeps: the
 * state entering every chunk and the gradient of every chunk's outgoing state
 * (2 * d_k * d_v bf16 each per chunk and head) and three bf16 tensors of the
 * size of v. */
size_t kda_chunk_bwd_workspace_size(int64_t total_tokens, int32_t n_seqs, int32_t n_heads,
                                    int32_t d_k, int32_t d_v, int32_t chunk, kda_dtype dt);

/* Chunkwise KDA backward: the gradients of a loss L with respect to the
 * inputs of kda_chunk_fwd, given dO = dL/do and dS_T = dL/dS_T.  The forward
 * pass is evaluated again inside (its outputs are not an argument); the
 * gradients are those of the recurrence above taken token by token
 * (ogis-ri NLP primer on Kimi K3, §3.1 "KDA": decay, probe, delta, write,
 * read-out), computed through the chunked form with the same 16-token
 * sub-tiling as the forward (orkas.ai "Kimi K3 architecture",
 * §"GPU のコードパスを一本消した「下界」").
 *   q, k, v, beta, log_alpha, S0, cu_seqlens : as for kda_chunk_fwd (read only)
 *   dO         : [total_tokens, n_heads, d_v], dtype dt (required when total_tokens > 0)
 *   dS_T       : [n_seqs, n_heads, d_k, d_v] float32, or NULL (zero)
 *   dq, dk     : outputs [total_tokens, n_heads, d_k], dtype dt
 *   dv         : output  [total_tokens, n_heads, d_v], dtype dt
 *   dbeta      : output  [total_tokens, n_heads], dtype dt
 *   dlog_alpha : output  [total_tokens, n_heads, d_k], dtype dt (gradient of log alpha)
 *   dS0        : output  [n_seqs, n_heads, d_k, d_v] float32 (gradient of the
 *                initial state, also when S0 is NULL), or NULL (not written)
 *   workspace  : >= kda_chunk_bwd_workspace_size(...) bytes of device memory
 * Outputs are written, not accumulated into.  Supported: dt == KDA_BF16,
 * d_k == d_v in {64, 128}, chunk == 64 (KDA_ERR_UNSUPPORTED otherwise);
 * other rules, alignment and errors as for kda_chunk_fwd.  Enqueued on
 * `stream`, never synchronises. */
kda_status kda_chunk_bwd(kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads,
                         int32_t d_k, int32_t d_v, int32_t chunk,
                         const void* q, const void* k, const void* v,
                         const void* beta, const void* log_alpha,
                         const float* S0, const int32_t* cu_seqlens,
                         const void* dO, const float* dS_T,
                         void* dq, void* dk, void* dv, void* dbeta, void* dlog_alpha, float* dS0,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Measurement form of kda_chunk_bwd, as kda_chunk_fwd_profile is of
 * kda_chunk_fwd: same arguments and results, blocks until done, and writes
 * each launch's milliseconds to stage_ms[0 .. kda_profile_bwd_num_stages()-1]. */
kda_status kda_chunk_bwd_profile(kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads,
                                 int32_t d_k, int32_t d_v, int32_t chunk,
                                 const void* q, const void* k, const void* v,
                                 const void* beta, const void* log_alpha,
                                 const float* S0, const int32_t* cu_seqlens,
                                 const void* dO, const float* dS_T,
                                 void* dq, void* dk, void* dv, void* dbeta, void* dlog_alpha, float* dS0,
                                 void* workspace, size_t workspace_bytes, void* stream, float* stage_ms);

/* Training pair.  kda_chunk_fwd_train is kda_chunk_fwd that also keeps, in
 * a caller-owned context buffer, what the backward pass needs (the backward
 * operand set of every chunk, the state entering every chunk, and per token
 * U~); kda_chunk_bwd_ctx then computes the
 * gradients from that context without evaluating the forward again.  Same
 * math and results as kda_chunk_bwd (bit for bit), split across the two
 * calls; bf16 only.
 *   context : >= kda_chunk_train_context_size(...) bytes of device memory,
 *             256-byte aligned; written by kda_chunk_fwd_train, read by
 *             kda_chunk_bwd_ctx, which must get the same q, k, v, beta,
 *             log_alpha, cu_seqlens and sizes (S0 acts through the
 *             context); nothing checks that they match
 *   kda_chunk_fwd_train : arguments of kda_chunk_fwd plus the context; its
 *             workspace is kda_chunk_fwd_workspace_size(...) bytes; o is
 *             required, S_T optional
 *   kda_chunk_bwd_ctx : gradients as kda_chunk_bwd (dv, dbeta, ... written,
 *             dS0 optional); workspace >= kda_chunk_bwd_ctx_workspace_size(...)
 * Errors as for kda_chunk_fwd / kda_chunk_bwd (KDA_ERR_WORKSPACE also for a
 * missing, misaligned or short context).  Both enqueue on `stream` and never
 * synchronise. */
size_t kda_chunk_train_context_size(int64_t total_tokens, int32_t n_seqs, int32_t n_heads,
                                    int32_t d_k, int32_t d_v, int32_t chunk, kda_dtype dt);
size_t kda_chunk_bwd_ctx_workspace_size(int64_t total_tokens, int32_t n_seqs, int32_t n_heads,
                                        int32_t d_k, int32_t d_v, int32_t chunk, kda_dtype dt);
kda_status kda_chunk_fwd_train(kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads,
                               int32_t d_k, int32_t d_v, int32_t chunk,
                               const void* q, const void* k, const void* v,
                               const void* beta, const void* log_alpha,
                               const float* S0, const int32_t* cu_seqlens,
                               void* o, float* S_T, void* context, size_t context_bytes,
                               void* workspace, size_t workspace_bytes, void* stream);
kda_status kda_chunk_bwd_ctx(kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads,
                             int32_t d_k, int32_t d_v, int32_t chunk,
                             const void* q, const void* k, const void* v, const void* beta,
                             const void* log_alpha, const int32_t* cu_seqlens,
                             const void* context, size_t context_bytes,
                             const void* dO, const float* dS_T,
                             void* dq, void* dk, void* dv, void* dbeta, void* dlog_alpha, float* dS0,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Number of kernel launches one backward pass makes, and the name of launch i
 * (NULL when out of range). */
int32_t kda_profile_bwd_num_stages(void);
const char* kda_profile_bwd_stage_name(int32_t i);

/* Number of kernel launches one forward pass makes, and the name of launch i
 * (NULL when i is out of range); names match the kernel symbols a profiler
 * reports. */
int32_t kda_profile_num_stages(void);
const char* kda_profile_stage_name(int32_t i);

/* Static description of a status code (never NULL). */
const char* kda_status_string(kda_status s);

/* Library version, e.g. "0.1.0". */
const char* kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
