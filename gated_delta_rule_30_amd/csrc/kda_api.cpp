// C ABI of the KDA chunkwise forward library: argument validation, workspace
// carve-up and the launch sequence on the caller's stream.  No device code.
#include "../../include/kda.h"

#include <hip/hip_runtime.h>

#include "kda_internal.h"

namespace kda {

static constexpr int64_t kChunkTokens = 64;
static constexpr size_t kAlign = 256;

static size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

size_t carve_workspace(Plan* p, void* base) {
    const size_t es = p->bf16 ? 2 : 4;
    const size_t H = (size_t)p->n_heads, D = (size_t)p->d;
    const size_t mc = (size_t)p->max_chunks;
    const size_t T = (size_t)p->total_tokens;
    const int kind = p->ws_kind;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes);
        return base ? (void*)((char*)base + at) : nullptr;
    };
    p->ws_n_chunks = (int32_t*)take(sizeof(int32_t));
    p->ws_seq_chunk0 = (int32_t*)take(sizeof(int32_t) * ((size_t)p->n_seqs + 1));
    p->ws_tab = (ChunkInfo*)take(sizeof(ChunkInfo) * mc);
    if (p->generic) {   // fp32 operands of the generic kernels (kda_generic.hip)
        const size_t C = (size_t)p->chunk, DK = (size_t)p->d_k;
        p->ws_Qg = take(4 * mc * H * C * DK);
        p->ws_Kg = take(4 * mc * H * C * DK);
        p->ws_KhT = take(4 * mc * H * C * DK);
        p->ws_TB = take(4 * mc * H * C * C);
        p->ws_M = take(4 * mc * H * C * C);
        p->ws_gam = (float*)take(4 * mc * H * DK);
        return off;
    }
    if (kind != kWsBwdCtx) {   // the forward operand set
        p->ws_TB = take(es * mc * H * kChunkTokens * kChunkTokens);
        p->ws_M = take(es * mc * H * kChunkTokens * kChunkTokens);
        p->ws_Qg = take(es * mc * H * kChunkTokens * D);
        p->ws_Kg = take(es * mc * H * kChunkTokens * D);
        p->ws_KhT = take(es * mc * H * D * kChunkTokens);
    }
    if (kind == kWsFwd || kind == kWsBwd) p->ws_gam = (float*)take(4 * mc * H * D);
    if (kind == kWsFwd) p->ws_state2 = (float*)take(4 * 2 * (size_t)p->n_seqs * H * D * D);
    if (kind == kWsBwd) {
        p->ws_bet = (float*)take(4 * mc * H * kChunkTokens);
        p->ws_bTT = take(es * mc * H * kChunkTokens * kChunkTokens);
        p->ws_bMT = take(es * mc * H * kChunkTokens * kChunkTokens);
        p->ws_bKh = take(es * mc * H * kChunkTokens * D);
        p->ws_bQgT = take(es * mc * H * D * kChunkTokens);
        p->ws_bKgT = take(es * mc * H * D * kChunkTokens);
        p->ws_ckS = take(2 * mc * H * D * D);
        p->ws_U = take(2 * T * H * D);
    }
    if (kind == kWsBwd || kind == kWsBwdCtx) {
        p->ws_ckdS = take(2 * mc * H * D * D);
        p->ws_dZ = take(2 * T * H * D);
        p->ws_dbp = (float*)take(4 * 2 * T * H);
    }
    // first checkpoint slot of each sequence (kda_chunk_fwd_ckpt with cu_seqlens)
    p->ws_ck0 = (int32_t*)take(sizeof(int32_t) * ((size_t)p->n_seqs + 1));
    // last, so that the regions above keep their offsets
    p->ws_prog = (int32_t*)take(4 * (size_t)p->n_seqs * H * (D / 16));
    return off;
}

size_t carve_context(Plan* p, void* base) {
    const size_t es = 2;
    const size_t H = (size_t)p->n_heads, D = (size_t)p->d;
    const size_t mc = (size_t)p->max_chunks;
    const size_t T = (size_t)p->total_tokens;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes);
        return base ? (void*)((char*)base + at) : nullptr;
    };
    p->ws_gam = (float*)take(4 * mc * H * D);
    p->ws_bet = (float*)take(4 * mc * H * kChunkTokens);
    p->ws_bTT = take(es * mc * H * kChunkTokens * kChunkTokens);
    p->ws_bMT = take(es * mc * H * kChunkTokens * kChunkTokens);
    p->ws_bKh = take(es * mc * H * kChunkTokens * D);
    p->ws_bQgT = take(es * mc * H * D * kChunkTokens);
    p->ws_bKgT = take(es * mc * H * D * kChunkTokens);
    p->ws_ckS = take(2 * mc * H * D * D);
    p->ws_U = take(2 * T * H * D);
    return off;
}

}  // namespace kda

using kda::Plan;

// The sizes the tuned kernels cover: chunk 64, d_k = d_v, bf16 at 64 or 128, fp32 at 64.
static bool tuned_sizes(kda_dtype dt, int32_t d_k, int32_t d_v, int32_t chunk) {
    return chunk == kda::kChunkTokens && d_k == d_v && (d_k == 64 || (d_k == 128 && dt == KDA_BF16));
}

// `generic_ok`: the forward, which runs every other supported size (chunk
// 16, 32, 64 or 128; d_k, d_v in {64, 128}; either dtype) on the generic
// kernels; every other entry point takes the tuned sizes only.
static kda_status plan_sizes(Plan* p, kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads,
                             int32_t d_k, int32_t d_v, int32_t chunk, bool varlen, bool generic_ok = false) {
    if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_DTYPE;
    if (total_tokens < 0 || n_seqs < 1 || n_heads < 1 || d_k < 1 || d_v < 1 || chunk < 1) return KDA_ERR_SHAPE;
    if (!varlen && total_tokens % n_seqs != 0) return KDA_ERR_SHAPE;
    if ((d_k != 64 && d_k != 128) || (d_v != 64 && d_v != 128)) return KDA_ERR_UNSUPPORTED;
    if (chunk != 16 && chunk != 32 && chunk != 64 && chunk != 128) return KDA_ERR_UNSUPPORTED;
    const bool tuned = tuned_sizes(dt, d_k, d_v, chunk);
    if (!tuned && !generic_ok) return KDA_ERR_UNSUPPORTED;
    if (total_tokens >= ((int64_t)1 << 31) || n_heads > 65535) return KDA_ERR_UNSUPPORTED;
    const int64_t max_chunks = total_tokens / chunk + n_seqs;
    if (max_chunks >= ((int64_t)1 << 31) || (int64_t)n_seqs * n_heads * (d_v / 16) >= ((int64_t)1 << 31))
        return KDA_ERR_UNSUPPORTED;
    p->bf16 = dt == KDA_BF16;
    p->d = d_k;
    p->generic = !tuned;
    p->chunk = chunk;
    p->d_k = d_k;
    p->d_v = d_v;
    p->total_tokens = total_tokens;
    p->n_seqs = n_seqs;
    p->n_heads = n_heads;
    p->fixed_len = varlen ? 0 : total_tokens / n_seqs;
    p->max_chunks = (int32_t)max_chunks;
    return KDA_OK;
}

extern "C" {

size_t kda_chunk_fwd_workspace_size(int64_t total_tokens, int32_t n_seqs, int32_t n_heads, int32_t d_k,
                                    int32_t d_v, int32_t chunk, kda_dtype dt) {
    Plan p{};
    // Size for the variable-length case: it never needs less than equal lengths.
    if (plan_sizes(&p, dt, total_tokens, n_seqs, n_heads, d_k, d_v, chunk, true, true) != KDA_OK) return 0;
    return kda::carve_workspace(&p, nullptr);
}

static kda_status prepare(Plan* p, kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads,
                          int32_t d_k, int32_t d_v, int32_t chunk, const void* q, const void* k, const void* v,
                          const void* beta, const void* log_alpha, const float* S0, const int32_t* cu_seqlens,
                          void* o, float* S_T, void* workspace, size_t workspace_bytes, bool no_output = false,
                          bool generic_ok = false) {
    kda_status s = plan_sizes(p, dt, total_tokens, n_seqs, n_heads, d_k, d_v, chunk, cu_seqlens != nullptr,
                              generic_ok);
    if (s != KDA_OK) return s;
    if (total_tokens > 0 && (!q || !k || !v || !beta || !log_alpha || (!o && !no_output))) return KDA_ERR_NULL;
    const void* ptrs[] = {q, k, v, beta, log_alpha, S0, cu_seqlens, o, S_T};
    for (const void* ptr : ptrs)
        if (ptr && ((uintptr_t)ptr % 16) != 0) return KDA_ERR_SHAPE;
    if (!workspace) return KDA_ERR_WORKSPACE;
    if ((uintptr_t)workspace % kda::kAlign != 0) return KDA_ERR_WORKSPACE;
    Plan sz = *p;
    if (workspace_bytes < kda::carve_workspace(&sz, nullptr)) return KDA_ERR_WORKSPACE;
    p->q = q;
    p->k = k;
    p->v = v;
    p->beta = beta;
    p->g = log_alpha;
    p->S0 = S0;
    p->cu_seqlens = cu_seqlens;
    p->o = o;
    p->S_T = S_T;
    kda::carve_workspace(p, workspace);
    return KDA_OK;
}

kda_status kda_chunk_fwd(kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads, int32_t d_k,
                         int32_t d_v, int32_t chunk, const void* q, const void* k, const void* v,
                         const void* beta, const void* log_alpha, const float* S0, const int32_t* cu_seqlens,
                         void* o, float* S_T, void* workspace, size_t workspace_bytes, void* stream) {
    return kda::chunk_fwd_entry(dt, total_tokens, n_seqs, n_heads, d_k, d_v, chunk, q, k, v, beta, log_alpha, S0,
                                cu_seqlens, o, S_T, workspace, workspace_bytes, stream, true);
}

size_t kda_chunk_ckpt_size(int64_t total_tokens, int32_t n_seqs, int32_t n_heads, int32_t d_k, int32_t d_v,
                           int32_t every) {
    Plan p{};
    if (every < 1) return 0;
    if (plan_sizes(&p, KDA_BF16, total_tokens, n_seqs, n_heads, d_k, d_v, kda::kChunkTokens, true) != KDA_OK) return 0;
    const int64_t slots = (total_tokens / kda::kChunkTokens + n_seqs) / every;
    return (size_t)slots * (size_t)n_heads * (size_t)d_k * (size_t)d_v * sizeof(float);
}

kda_status kda_chunk_fwd_ckpt(kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads, int32_t d_k,
                              int32_t d_v, int32_t chunk, const void* q, const void* k, const void* v,
                              const void* beta, const void* log_alpha, const float* S0, const int32_t* cu_seqlens,
                              void* o, float* S_T, int32_t every, float* S_ckpt, size_t S_ckpt_bytes,
                              void* workspace, size_t workspace_bytes, void* stream) {
    if (dt == KDA_F32) return KDA_ERR_UNSUPPORTED;
    if (every < 1) return KDA_ERR_SHAPE;
    if (!S_ckpt) return KDA_ERR_NULL;
    if ((uintptr_t)S_ckpt % 16 != 0) return KDA_ERR_SHAPE;
    Plan p{};
    kda_status s = prepare(&p, dt, total_tokens, n_seqs, n_heads, d_k, d_v, chunk, q, k, v, beta, log_alpha, S0,
                           cu_seqlens, o, S_T, workspace, workspace_bytes);
    if (s != KDA_OK) return s;
    if (S_ckpt_bytes < kda_chunk_ckpt_size(total_tokens, n_seqs, n_heads, d_k, d_v, every)) return KDA_ERR_WORKSPACE;
    p.S_ckpt = S_ckpt;
    p.ck_every = every;
    p.ck_slots = (int32_t)((total_tokens / kda::kChunkTokens + n_seqs) / every);
    hipError_t e = kda::launch(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int32_t kda_profile_num_stages(void) { return kda::kNumStages; }

const char* kda_profile_stage_name(int32_t i) {
    return (i >= 0 && i < kda::kNumStages) ? kda::kStageNames[i] : nullptr;
}

kda_status kda_chunk_fwd_profile(kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads,
                                 int32_t d_k, int32_t d_v, int32_t chunk, const void* q, const void* k,
                                 const void* v, const void* beta, const void* log_alpha, const float* S0,
                                 const int32_t* cu_seqlens, void* o, float* S_T, void* workspace,
                                 size_t workspace_bytes, void* stream, float* stage_ms) {
    if (!stage_ms) return KDA_ERR_NULL;
    Plan p{};
    kda_status s = prepare(&p, dt, total_tokens, n_seqs, n_heads, d_k, d_v, chunk, q, k, v, beta, log_alpha, S0,
                           cu_seqlens, o, S_T, workspace, workspace_bytes, false, true);
    if (s != KDA_OK) return s;
    hipEvent_t ev[kda::kNumStages + 1];
    int made = 0;
    hipError_t e = hipSuccess;
    for (; made <= kda::kNumStages && e == hipSuccess; ++made) e = hipEventCreate(&ev[made]);
    if (e != hipSuccess) made -= 1;
    if (e == hipSuccess) e = kda::launch(p, static_cast<hipStream_t>(stream), ev);
    if (e == hipSuccess) e = hipEventSynchronize(ev[kda::kNumStages]);
    for (int i = 0; e == hipSuccess && i < kda::kNumStages; ++i) e = hipEventElapsedTime(&stage_ms[i], ev[i], ev[i + 1]);
    for (int i = 0; i < made; ++i) (void)hipEventDestroy(ev[i]);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_chunk_transition(kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads, int32_t d_k,
                                int32_t chunk, const void* k, const void* beta, const void* log_alpha,
                                const int32_t* cu_seqlens, float* P, void* workspace, size_t workspace_bytes,
                                void* stream) {
    if (dt == KDA_F32) return KDA_ERR_UNSUPPORTED;
    if (!P) return KDA_ERR_NULL;
    Plan p{};
    // q and v are not read: k stands in for both (sizes and alignment only)
    kda_status s = prepare(&p, dt, total_tokens, n_seqs, n_heads, d_k, d_k, chunk, k, k, k, beta, log_alpha,
                           nullptr, cu_seqlens, nullptr, P, workspace, workspace_bytes, true);
    if (s != KDA_OK) return s;
    hipError_t e = kda::launch_transition(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_compose_states(int32_t n_segments, int32_t n_heads, int32_t d, const float* P, const float* Z,
                              const float* S0, float* S_in, void* stream) {
    if (n_segments < 1 || n_heads < 1 || d < 1) return KDA_ERR_SHAPE;
    if (d != 64 && d != 128) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)n_heads * (d / 64) >= ((int64_t)1 << 31)) return KDA_ERR_UNSUPPORTED;
    if (!P || !Z || !S_in) return KDA_ERR_NULL;
    const void* ptrs[] = {P, Z, S0, S_in};
    for (const void* ptr : ptrs)
        if (ptr && ((uintptr_t)ptr % 16) != 0) return KDA_ERR_SHAPE;
    hipError_t e = kda::launch_compose(n_segments, n_heads, d, P, Z, S0, S_in, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

static kda_status recurrent(kda_dtype dt, int32_t n_seqs, int32_t n_tokens, int32_t n_heads, int32_t d_k,
                            int32_t d_v, const void* q, const void* k, const void* v, const void* beta,
                            const void* log_alpha, bool commit, const int32_t* n_apply, const float* S_in,
                            float* S_out, void* o, void* stream) {
    if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_DTYPE;
    if (n_seqs < 1 || n_tokens < 1 || n_heads < 1 || d_k < 1 || d_v < 1) return KDA_ERR_SHAPE;
    if (d_k != d_v || (d_k != 64 && d_k != 128)) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)n_seqs * n_tokens >= ((int64_t)1 << 31) || (int64_t)n_seqs * n_heads * (d_k / 64) >= ((int64_t)1 << 31))
        return KDA_ERR_UNSUPPORTED;
    if (!q || !k || !v || !beta || !log_alpha || !S_out || (!commit && !o) || (commit && !n_apply))
        return KDA_ERR_NULL;
    const void* ptrs[] = {q, k, v, beta, log_alpha, S_in, S_out, o};
    for (const void* ptr : ptrs)
        if (ptr && ((uintptr_t)ptr % 16) != 0) return KDA_ERR_SHAPE;
    if ((uintptr_t)n_apply % 4 != 0) return KDA_ERR_SHAPE;
    kda::DecodePlan p{};
    p.bf16 = dt == KDA_BF16;
    p.d = d_k;
    p.n_seqs = n_seqs;
    p.n_tokens = n_tokens;
    p.n_heads = n_heads;
    p.q = q;
    p.k = k;
    p.v = v;
    p.beta = beta;
    p.g = log_alpha;
    p.S_in = S_in;
    p.S_out = S_out;
    p.o = o;
    p.n_apply = n_apply;
    hipError_t e = kda::launch_decode(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_recurrent_fwd(kda_dtype dt, int32_t n_seqs, int32_t n_tokens, int32_t n_heads, int32_t d_k,
                             int32_t d_v, const void* q, const void* k, const void* v, const void* beta,
                             const void* log_alpha, const float* S_in, float* S_out, void* o, void* stream) {
    return recurrent(dt, n_seqs, n_tokens, n_heads, d_k, d_v, q, k, v, beta, log_alpha, false, nullptr, S_in, S_out,
                     o, stream);
}

kda_status kda_recurrent_commit(kda_dtype dt, int32_t n_seqs, int32_t n_tokens, int32_t n_heads, int32_t d_k,
                                int32_t d_v, const void* q, const void* k, const void* v, const void* beta,
                                const void* log_alpha, const int32_t* n_accept, const float* S_in, float* S_out,
                                void* o, void* stream) {
    return recurrent(dt, n_seqs, n_tokens, n_heads, d_k, d_v, q, k, v, beta, log_alpha, true, n_accept, S_in, S_out,
                     o, stream);
}

kda_status kda_validate_inputs(kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads, int32_t d_k,
                               const void* beta, const void* log_alpha, const int32_t* cu_seqlens,
                               unsigned long long* counts, void* stream) {
    if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_DTYPE;
    if (total_tokens < 0 || n_seqs < 1 || n_heads < 1 || d_k < 1) return KDA_ERR_SHAPE;
    if (!counts || (total_tokens > 0 && (!beta || !log_alpha))) return KDA_ERR_NULL;
    if ((uintptr_t)counts % 8 != 0) return KDA_ERR_SHAPE;
    hipError_t e = kda::launch_validate(dt == KDA_BF16, total_tokens, n_seqs, n_heads, d_k, beta, log_alpha,
                                        cu_seqlens, counts, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

size_t kda_chunk_bwd_workspace_size(int64_t total_tokens, int32_t n_seqs, int32_t n_heads, int32_t d_k,
                                    int32_t d_v, int32_t chunk, kda_dtype dt) {
    if (dt != KDA_BF16) return 0;
    Plan p{};
    if (plan_sizes(&p, dt, total_tokens, n_seqs, n_heads, d_k, d_v, chunk, true) != KDA_OK) return 0;
    if (p.max_chunks >= (1 << 30)) return 0;
    p.ws_kind = kda::kWsBwd;
    return kda::carve_workspace(&p, nullptr);
}

static kda_status prepare_bwd(Plan* p, kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads,
                              int32_t d_k, int32_t d_v, int32_t chunk, const void* q, const void* k, const void* v,
                              const void* beta, const void* log_alpha, const float* S0, const int32_t* cu_seqlens,
                              const void* dO, const float* dS_T, void* dq, void* dk, void* dv, void* dbeta,
                              void* dlog_alpha, float* dS0, void* workspace, size_t workspace_bytes,
                              int ws_kind = kda::kWsBwd) {
    if (dt == KDA_F32) return KDA_ERR_UNSUPPORTED;
    kda_status s = plan_sizes(p, dt, total_tokens, n_seqs, n_heads, d_k, d_v, chunk, cu_seqlens != nullptr);
    if (s != KDA_OK) return s;
    if (p->max_chunks >= (1 << 30)) return KDA_ERR_UNSUPPORTED;   // two gradient workgroups per chunk
    p->ws_kind = ws_kind;
    if (total_tokens > 0 && (!q || !k || !v || !beta || !log_alpha || !dO || !dq || !dk || !dv || !dbeta ||
                             !dlog_alpha))
        return KDA_ERR_NULL;
    const void* ptrs[] = {q, k, v, beta, log_alpha, S0, cu_seqlens, dO, dS_T, dq, dk, dv, dbeta, dlog_alpha, dS0};
    for (const void* ptr : ptrs)
        if (ptr && ((uintptr_t)ptr % 16) != 0) return KDA_ERR_SHAPE;
    if (!workspace || (uintptr_t)workspace % kda::kAlign != 0) return KDA_ERR_WORKSPACE;
    Plan sz = *p;
    if (workspace_bytes < kda::carve_workspace(&sz, nullptr)) return KDA_ERR_WORKSPACE;
    p->q = q;
    p->k = k;
    p->v = v;
    p->beta = beta;
    p->g = log_alpha;
    p->S0 = S0;
    p->cu_seqlens = cu_seqlens;
    p->dO = dO;
    p->dS_T = dS_T;
    p->dq = dq;
    p->dk = dk;
    p->dv = dv;
    p->dbeta = dbeta;
    p->dg = dlog_alpha;
    p->dS0 = dS0;
    kda::carve_workspace(p, workspace);
    return KDA_OK;
}

kda_status kda_chunk_bwd(kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads, int32_t d_k,
                         int32_t d_v, int32_t chunk, const void* q, const void* k, const void* v, const void* beta,
                         const void* log_alpha, const float* S0, const int32_t* cu_seqlens, const void* dO,
                         const float* dS_T, void* dq, void* dk, void* dv, void* dbeta, void* dlog_alpha, float* dS0,
                         void* workspace, size_t workspace_bytes, void* stream) {
    Plan p{};
    kda_status s = prepare_bwd(&p, dt, total_tokens, n_seqs, n_heads, d_k, d_v, chunk, q, k, v, beta, log_alpha, S0,
                               cu_seqlens, dO, dS_T, dq, dk, dv, dbeta, dlog_alpha, dS0, workspace,
                               workspace_bytes);
    if (s != KDA_OK) return s;
    hipError_t e = kda::launch_bwd(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

size_t kda_chunk_train_context_size(int64_t total_tokens, int32_t n_seqs, int32_t n_heads, int32_t d_k,
                                    int32_t d_v, int32_t chunk, kda_dtype dt) {
    if (dt != KDA_BF16) return 0;
    Plan p{};
    if (plan_sizes(&p, dt, total_tokens, n_seqs, n_heads, d_k, d_v, chunk, true) != KDA_OK) return 0;
    if (p.max_chunks >= (1 << 30)) return 0;
    return kda::carve_context(&p, nullptr);
}

size_t kda_chunk_bwd_ctx_workspace_size(int64_t total_tokens, int32_t n_seqs, int32_t n_heads, int32_t d_k,
                                        int32_t d_v, int32_t chunk, kda_dtype dt) {
    if (dt != KDA_BF16) return 0;
    Plan p{};
    if (plan_sizes(&p, dt, total_tokens, n_seqs, n_heads, d_k, d_v, chunk, true) != KDA_OK) return 0;
    if (p.max_chunks >= (1 << 30)) return 0;
    p.ws_kind = kda::kWsBwdCtx;
    return kda::carve_workspace(&p, nullptr);
}

// the context buffer: present, aligned and large enough; carves its regions
static kda_status take_context(Plan* p, void* context, size_t context_bytes) {
    if (!context || (uintptr_t)context % kda::kAlign != 0) return KDA_ERR_WORKSPACE;
    Plan sz = *p;
    if (context_bytes < kda::carve_context(&sz, nullptr)) return KDA_ERR_WORKSPACE;
    kda::carve_context(p, context);
    return KDA_OK;
}

kda_status kda_chunk_fwd_train(kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads, int32_t d_k,
                               int32_t d_v, int32_t chunk, const void* q, const void* k, const void* v,
                               const void* beta, const void* log_alpha, const float* S0, const int32_t* cu_seqlens,
                               void* o, float* S_T, void* context, size_t context_bytes, void* workspace,
                               size_t workspace_bytes, void* stream) {
    if (dt == KDA_F32) return KDA_ERR_UNSUPPORTED;
    Plan p{};
    kda_status s = prepare(&p, dt, total_tokens, n_seqs, n_heads, d_k, d_v, chunk, q, k, v, beta, log_alpha, S0,
                           cu_seqlens, o, S_T, workspace, workspace_bytes);
    if (s != KDA_OK) return s;
    if (p.max_chunks >= (1 << 30)) return KDA_ERR_UNSUPPORTED;
    p.ws_kind = kda::kWsFwdTrain;
    kda::carve_workspace(&p, workspace);
    s = take_context(&p, context, context_bytes);
    if (s != KDA_OK) return s;
    hipError_t e = kda::launch_fwd_train(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_chunk_bwd_ctx(kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads, int32_t d_k,
                             int32_t d_v, int32_t chunk, const void* q, const void* k, const void* v,
                             const void* beta, const void* log_alpha, const int32_t* cu_seqlens, const void* context,
                             size_t context_bytes, const void* dO, const float* dS_T, void* dq, void* dk, void* dv,
                             void* dbeta, void* dlog_alpha, float* dS0, void* workspace, size_t workspace_bytes,
                             void* stream) {
    if (dt == KDA_F32) return KDA_ERR_UNSUPPORTED;
    Plan p{};
    // S0 is not read: the context holds what it contributed
    kda_status s = prepare_bwd(&p, dt, total_tokens, n_seqs, n_heads, d_k, d_v, chunk, q, k, v, beta, log_alpha,
                               nullptr, cu_seqlens, dO, dS_T, dq, dk, dv, dbeta, dlog_alpha, dS0, workspace,
                               workspace_bytes, kda::kWsBwdCtx);
    if (s != KDA_OK) return s;
    s = take_context(&p, const_cast<void*>(context), context_bytes);
    if (s != KDA_OK) return s;
    hipError_t e = kda::launch_bwd_ctx(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int32_t kda_profile_bwd_num_stages(void) { return kda::kNumBwdStages; }

const char* kda_profile_bwd_stage_name(int32_t i) {
    return (i >= 0 && i < kda::kNumBwdStages) ? kda::kBwdStageNames[i] : nullptr;
}

kda_status kda_chunk_bwd_profile(kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads, int32_t d_k,
                                 int32_t d_v, int32_t chunk, const void* q, const void* k, const void* v,
                                 const void* beta, const void* log_alpha, const float* S0,
                                 const int32_t* cu_seqlens, const void* dO, const float* dS_T, void* dq, void* dk,
                                 void* dv, void* dbeta, void* dlog_alpha, float* dS0, void* workspace,
                                 size_t workspace_bytes, void* stream, float* stage_ms) {
    if (!stage_ms) return KDA_ERR_NULL;
    Plan p{};
    kda_status s = prepare_bwd(&p, dt, total_tokens, n_seqs, n_heads, d_k, d_v, chunk, q, k, v, beta, log_alpha, S0,
                               cu_seqlens, dO, dS_T, dq, dk, dv, dbeta, dlog_alpha, dS0, workspace,
                               workspace_bytes);
    if (s != KDA_OK) return s;
    constexpr int NS = kda::kNumBwdStages;
    hipEvent_t ev[NS + 1];
    int made = 0;
    hipError_t e = hipSuccess;
    for (; made <= NS && e == hipSuccess; ++made) e = hipEventCreate(&ev[made]);
    if (e != hipSuccess) made -= 1;
    if (e == hipSuccess) e = kda::launch_bwd(p, static_cast<hipStream_t>(stream), ev);
    if (e == hipSuccess) e = hipEventSynchronize(ev[NS]);
    for (int i = 0; e == hipSuccess && i < NS; ++i) e = hipEventElapsedTime(&stage_ms[i], ev[i], ev[i + 1]);
    for (int i = 0; i < made; ++i) (void)hipEventDestroy(ev[i]);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_output_gate(kda_dtype dt, int64_t n_rows, int32_t d_v, const void* o, const void* gate,
                           const float* weight, float eps, void* y, void* stream) {
    if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_DTYPE;
    if (n_rows < 0 || d_v < 1) return KDA_ERR_SHAPE;
    if (d_v != 64 && d_v != 128) return KDA_ERR_UNSUPPORTED;
    if (!(eps >= 0.f) || eps > 1.f) return KDA_ERR_SHAPE;   // also rejects NaN
    if (n_rows > 0 && (!o || !gate || !y)) return KDA_ERR_NULL;
    const void* ptrs[] = {o, gate, weight, y};
    for (const void* ptr : ptrs)
        if (ptr && ((uintptr_t)ptr % 16) != 0) return KDA_ERR_SHAPE;
    hipError_t e = kda::launch_output_gate(dt == KDA_BF16, n_rows, d_v, o, gate, weight, eps, y,
                                           static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "KDA_OK: success";
        case KDA_ERR_NULL: return "KDA_ERR_NULL: a required pointer is NULL";
        case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE: inconsistent sizes or misaligned tensor";
        case KDA_ERR_DTYPE: return "KDA_ERR_DTYPE: unknown dtype";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: sizes not supported by this build";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing, misaligned or too small";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: kernel launch failed";
    }
    return "KDA: unknown status";
}

const char* kda_version(void) { return "0.1.0"; }

}  // extern "C"

kda_status kda::chunk_fwd_entry(kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads, int32_t d_k,
                                int32_t d_v, int32_t chunk, const void* q, const void* k, const void* v,
                                const void* beta, const void* log_alpha, const float* S0,
                                const int32_t* cu_seqlens, void* o, float* S_T, void* workspace,
                                size_t workspace_bytes, void* stream, bool pipeline) {
    Plan p{};
    kda_status s = prepare(&p, dt, total_tokens, n_seqs, n_heads, d_k, d_v, chunk, q, k, v, beta, log_alpha, S0,
                           cu_seqlens, o, S_T, workspace, workspace_bytes, false, true);
    if (s != KDA_OK) return s;
    p.no_pipeline = !pipeline;
    hipError_t e = kda::launch(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}
