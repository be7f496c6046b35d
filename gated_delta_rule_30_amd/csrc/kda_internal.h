// Internal launch plan shared by the C ABI (kda_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/kda.h"

namespace kda {

struct ChunkInfo {
    int64_t tok0;   // first packed token of the chunk
    int32_t seq;    // sequence index
    int32_t len;    // valid tokens in the chunk, 1..64
};

struct Plan {
    bool bf16;
    int d;                    // d_k == d_v (the tuned kernels); d_k for the generic ones
    // The generic kernels (kda_generic.hip): any chunk size and d_k, d_v the
    // tuned ones do not cover.  Their workspace reuses the operand fields
    // below as fp32 arrays: ws_Qg, ws_Kg, ws_KhT (K . exp(b_L - b), rows)
    // [H, max_chunks, chunk, d_k], ws_TB and ws_M [H, max_chunks, chunk,
    // chunk], ws_gam [H, max_chunks, d_k].
    bool generic;
    int32_t chunk, d_k, d_v;     // chunk tokens and head dims (all plans)
    int64_t total_tokens;
    int32_t n_seqs, n_heads;
    int64_t fixed_len;        // tokens per sequence when cu_seqlens is NULL
    int32_t max_chunks;       // upper bound on the number of chunks
    const void *q, *k, *v, *beta, *g;
    const float* S0;
    const int32_t* cu_seqlens;
    void* o;
    float* S_T;
    float* S_ckpt;            // [slots, H, D, D] fp32 states at chosen chunk ends, or NULL
    int32_t ck_every;         // a state after every ck_every-th chunk of a sequence
    int32_t ck_slots;         // slots of S_ckpt
    bool no_pipeline;         // never split the forward into token blocks on a side stream
    // workspace carve-up
    int32_t* ws_n_chunks;
    int32_t* ws_seq_chunk0;
    ChunkInfo* ws_tab;
    // chunk operands, head-major: slot h * max_chunks + chunk
    void* ws_TB;              // [H, max_chunks, 64, 64] T diag(beta), operand dtype
    void* ws_M;               // [H, max_chunks, 64, 64] decayed causal Q K^T, operand dtype
    void* ws_Qg;              // [H, max_chunks, 64, D] Q . Gamma
    void* ws_Kg;              // [H, max_chunks, 64, D] K . Gamma
    void* ws_KhT;             // [H, max_chunks, D, 64] (K . exp(b_L - b))^T
    float* ws_gam;            // [H, max_chunks, D] exp(b_L), fp32
    float* ws_state2;         // [2, N, H, D, D] fp32: states between the blocks of a pipelined forward
    // What the workspace holds (carve_workspace) -- kWsFwd: the forward pass;
    // kWsBwd: the backward with the forward evaluated again inside;
    // kWsFwdTrain / kWsBwdCtx: the training pair, whose shared regions (Gamma_L,
    // beta, the backward operand set, S per chunk, U~) live in a separate
    // context buffer (carve_context).
    int ws_kind;
    const void* dO;           // [T, H, D] output gradients
    const float* dS_T;        // [N, H, D, D] final-state gradients or NULL
    void *dq, *dk, *dv, *dbeta, *dg;
    float* dS0;               // [N, H, D, D] or NULL
    float* ws_bet;            // [H, max_chunks, 64] beta per chunk, fp32
    // the backward operand set, same shapes as the forward one:
    void* ws_bTT;             // T^T                      [H, max_chunks, 64, 64]
    void* ws_bMT;             // M^T                      [H, max_chunks, 64, 64]
    void* ws_bKh;             // K . exp(b_L - b), rows    [H, max_chunks, 64, D]
    void* ws_bQgT;            // (Q . Gamma)^T             [H, max_chunks, D, 64]
    void* ws_bKgT;            // (K . Gamma)^T             [H, max_chunks, D, 64]
    void* ws_ckS;             // [H, max_chunks, D, D] state entering each chunk (bf16)
    void* ws_ckdS;            // [H, max_chunks, D, D] gradient of each chunk's outgoing state (bf16)
    void *ws_U, *ws_dZ;       // [T, H, D] bf16: U~ and dZ per token
    float* ws_dbp;            // [2, H, T] float32 dbeta shares of the two channel halves
    int32_t* ws_ck0;          // [n_seqs + 1] first checkpoint slot of each sequence (varlen checkpoints)
    int32_t* ws_prog;         // [n_seqs * H, d_v / 16] steps done per recurrence workgroup (pacing)
};

// Arguments of the per-chunk gradient kernel (kda_bwd.hip); bf16 tensors.
struct GradArgs {
    const __bf16 *q, *k, *v, *g, *beta, *dO, *U, *dZ, *ckS, *ckdS;
    const ChunkInfo* tab;
    const int32_t* n_chunks;
    int64_t fixed_len;        // > 0: equal-length sequences (chunk from the index)
    int32_t fixed_chunks;
    int32_t H;
    int64_t max_chunks;
    int64_t total_tokens;
    __bf16 *dq, *dk, *dv, *dbeta, *dg;
    float* dbp;               // [2, H, total_tokens] the halves' dbeta shares
};
hipError_t launch_grad(const GradArgs& a, int d, int32_t max_chunks, hipStream_t stream);
hipError_t launch_dbeta_sum(const GradArgs& a, hipStream_t stream);

enum { kWsFwd = 0, kWsBwd = 1, kWsFwdTrain = 2, kWsBwdCtx = 3 };

// Byte offsets of every workspace region for the given sizes and p->ws_kind;
// returns the total size.  `base` may be NULL (size query only).
size_t carve_workspace(Plan* p, void* base);
// The same for the training pair's context buffer.
size_t carve_context(Plan* p, void* base);

// kda_chunk_fwd with its checks; `pipeline` = false keeps every launch on
// `stream` (no side stream is created or used).
kda_status chunk_fwd_entry(kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads, int32_t d_k,
                           int32_t d_v, int32_t chunk, const void* q, const void* k, const void* v, const void* beta,
                           const void* log_alpha, const float* S0, const int32_t* cu_seqlens, void* o, float* S_T,
                           void* workspace, size_t workspace_bytes, void* stream, bool pipeline);

// The chunk table for chunks of `chunk` tokens (k_chunk_table).
void launch_chunk_table(const Plan& p, int32_t chunk, hipStream_t stream);

// The forward pass with the generic kernels (p.generic), same events as launch().
hipError_t launch_generic(const Plan& p, hipStream_t stream, hipEvent_t* ev);

// Kernel launches of one forward pass, in order.
constexpr int kNumStages = 3;
extern const char* const kStageNames[kNumStages];

// Enqueues the forward pass on `stream`.  If `ev` is non-NULL it must hold
// kNumStages + 1 events; ev[i] is recorded before stage i and
// ev[kNumStages] after the last.
hipError_t launch(const Plan& p, hipStream_t stream, hipEvent_t* ev = nullptr);

// Backward pass (bf16): kNumBwdStages launches, events as for launch().
constexpr int kNumBwdStages = 6;
extern const char* const kBwdStageNames[kNumBwdStages];
hipError_t launch_bwd(const Plan& p, hipStream_t stream, hipEvent_t* ev = nullptr);

// Training pair (bf16): the forward keeping the backward's inputs in the
// context regions, and the backward from them.
hipError_t launch_fwd_train(const Plan& p, hipStream_t stream);
hipError_t launch_bwd_ctx(const Plan& p, hipStream_t stream);

// The forward pass with v = 0 from S0 = I and no output (bf16 only): S_T
// receives each sequence's transition matrix (kda_chunk_transition).
hipError_t launch_transition(const Plan& p, hipStream_t stream);

// S_in[0] = S0 (or zeros), S_in[g+1] = P[g] S_in[g] + Z[g] (kda_compose_states).
hipError_t launch_compose(int32_t n_segments, int32_t n_heads, int32_t d, const float* P, const float* Z,
                          const float* S0, float* S_in, hipStream_t stream);

// Token-by-token update for decoding (kda_recurrent_fwd).
struct DecodePlan {
    bool bf16;
    int d;                    // d_k == d_v, 64 or 128
    int32_t n_seqs, n_tokens, n_heads;
    const void *q, *k, *v, *beta, *g;
    const float* S_in;        // may be NULL (zeros); may equal S_out
    float* S_out;
    void* o;                  // may be NULL when n_apply is set
    const int32_t* n_apply;   // device [n_seqs] tokens to take per sequence, or NULL (all)
};
hipError_t launch_decode(const DecodePlan& p, hipStream_t stream);

// Output epilogue y = RMSNorm(o) * sigmoid(z) over rows of d channels (kda_output_gate).
hipError_t launch_output_gate(bool bf16, int64_t n_rows, int32_t d, const void* o, const void* z, const float* w,
                              float eps, void* y, hipStream_t stream);

// Input validator (kda_validate_inputs): clears counts[0..2] and adds the
// number of violations found; see the header.
hipError_t launch_validate(bool bf16, int64_t total_tokens, int32_t n_seqs, int32_t n_heads, int32_t d_k,
                           const void* beta, const void* g, const int32_t* cu, unsigned long long* counts,
                           hipStream_t stream);

}  // namespace kda
