// kda_chunk_fwd_noalloc: the forward pass with its workspace in a fixed
// device array of this library, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  Same kernels and results as kda_chunk_fwd; the call
// itself allocates nothing.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)KDA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// The forward's workspace for this entry point.  Each GPU the library runs
// on holds its own copy until the process ends.  In host code `scratch` is
// only a handle for the runtime: the device address of a GPU's copy comes
// from hipGetSymbolAddress with that GPU current (scratch_on_current_device).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of the current GPU's scratch, looked up once per device.
void* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_ptr[dev] = ptr;
    }
    return g_ptr[dev];
}

}  // namespace

extern "C" kda_status kda_chunk_fwd_noalloc(kda_dtype dt, int64_t total_tokens, int32_t n_seqs, int32_t n_heads,
                                            int32_t d_k, int32_t d_v, int32_t chunk, const void* q, const void* k,
                                            const void* v, const void* beta, const void* log_alpha,
                                            const float* S0, const int32_t* cu_seqlens, void* o, float* S_T,
                                            void* stream) {
    const size_t need = kda_chunk_fwd_workspace_size(total_tokens, n_seqs, n_heads, d_k, d_v, chunk, dt);
    if (need == 0)   // invalid sizes: the same status kda_chunk_fwd returns for them
        return kda::chunk_fwd_entry(dt, total_tokens, n_seqs, n_heads, d_k, d_v, chunk, q, k, v, beta, log_alpha,
                                    S0, cu_seqlens, o, S_T, nullptr, 0, stream, false);
    if (need > kScratchBytes) return KDA_ERR_WORKSPACE;
    void* ws = scratch_on_current_device();
    if (!ws) return KDA_ERR_HIP;
    return kda::chunk_fwd_entry(dt, total_tokens, n_seqs, n_heads, d_k, d_v, chunk, q, k, v, beta, log_alpha, S0,
                                cu_seqlens, o, S_T, ws, kScratchBytes, stream, false);
}
