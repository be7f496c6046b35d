// Token-by-token KDA update for decoding, and the input validator.
//
// Decoding advances each cached state by a few tokens with the recurrence
// itself (ogis-ri NLP primer on Kimi K3, §3.1 "KDA（Kimi Delta Attention）":
// decay, probe, delta, write, read-out):
//   S <- Diag(alpha_t) S;  p = S^T k_t;  S <- S + beta_t k_t (v_t - p)^T;  o_t = S^T q_t
// which is exactly the order the chunked pass reproduces in bulk.  The work
// is bound by moving the fp32 state (2 d_k d_v 4 bytes per sequence and head
// and call), so one workgroup owns a 64-column block of one state, keeps it in
// registers for all the call's tokens, and reads and writes it once.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// ---------------------------------------------------------------- k_decode
// Workgroup: (sequence, head, 64-column block of S), 256 threads.  Thread
// (rg, col) = (tid / 64, tid % 64) holds rows [rg*D/4, (rg+1)*D/4) of column
// col0 + col; a wave therefore reads and writes whole 256-byte row segments.
// The two contractions over key channels (S^T k and S^T q) sum per thread,
// then across the four row groups through LDS.  With n_apply given, sequence
// n takes only its first n_apply[n] (clamped to [0, n_tokens]) of the
// n_tokens token slots it owns; o may then be NULL (state only).
template <typename E, int D>
__global__ __launch_bounds__(256) void k_decode(const E* __restrict__ q, const E* __restrict__ k,
                                                const E* __restrict__ v, const E* __restrict__ beta,
                                                const E* __restrict__ g, const float* S_in, float* S_out,
                                                E* __restrict__ o, int32_t n_tokens, int32_t H,
                                                const int32_t* __restrict__ n_apply) {
    constexpr int RPT = D / 4;          // rows per thread
    constexpr int NCB = D / 64;         // column blocks per state
    __shared__ float sQ[D], sK[D], sA[D];
    __shared__ float sPart[4][64];
    const int tid = threadIdx.x, rg = tid >> 6, col = tid & 63;
    const int cb = blockIdx.x % NCB;
    const int64_t sh = blockIdx.x / NCB;     // sequence * H + head
    const int64_t n = sh / H, h = sh % H;
    const int c = cb * 64 + col;
    const int64_t sbase = sh * D * D;

    float S[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) S[r] = S_in ? S_in[sbase + (int64_t)(rg * RPT + r) * D + c] : 0.f;

    int n_run = n_tokens;
    if (n_apply) n_run = min(max(n_apply[n], 0), n_tokens);
    for (int t = 0; t < n_run; ++t) {
        const int64_t tok = n * n_tokens + t;
        const int64_t row = (tok * H + h) * D;
        __syncthreads();   // the previous token's LDS reads are done
        for (int i = tid; i < 3 * D; i += 256) {
            const int ch = i % D;
            if (i < D) sQ[ch] = to_f(q[row + ch]);
            else if (i < 2 * D) sK[ch] = to_f(k[row + ch]);
            else sA[ch] = __expf(to_f(g[row + ch]));
        }
        const float bt = to_f(beta[tok * H + h]);
        const float vt = to_f(v[row + c]);
        __syncthreads();
        // decay, then probe p = S^T k
        float p = 0.f;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            S[r] *= sA[rg * RPT + r];
            p += sK[rg * RPT + r] * S[r];
        }
        sPart[rg][col] = p;
        __syncthreads();
        p = sPart[0][col] + sPart[1][col] + sPart[2][col] + sPart[3][col];
        // delta write, then read-out o = S^T q
        const float e = bt * (vt - p);
        float y = 0.f;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            S[r] += sK[rg * RPT + r] * e;
            y += sQ[rg * RPT + r] * S[r];
        }
        __syncthreads();   // everyone has read sPart
        sPart[rg][col] = y;
        __syncthreads();
        if (rg == 0 && o) o[row + c] = from_f<E>(sPart[0][col] + sPart[1][col] + sPart[2][col] + sPart[3][col]);
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r) S_out[sbase + (int64_t)(rg * RPT + r) * D + c] = S[r];
}

template <typename E, int D>
static hipError_t launch_decode_t(const DecodePlan& p, hipStream_t st) {
    const int64_t grid = (int64_t)p.n_seqs * p.n_heads * (D / 64);
    hipLaunchKernelGGL((k_decode<E, D>), dim3((unsigned)grid), dim3(256), 0, st, static_cast<const E*>(p.q),
                       static_cast<const E*>(p.k), static_cast<const E*>(p.v), static_cast<const E*>(p.beta),
                       static_cast<const E*>(p.g), p.S_in, p.S_out, static_cast<E*>(p.o), p.n_tokens,
                       p.n_heads, p.n_apply);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodePlan& p, hipStream_t st) {
    if (p.n_seqs == 0 || p.n_heads == 0) return hipSuccess;
    if (p.bf16) return p.d == 128 ? launch_decode_t<__bf16, 128>(p, st) : launch_decode_t<__bf16, 64>(p, st);
    return p.d == 128 ? launch_decode_t<float, 128>(p, st) : launch_decode_t<float, 64>(p, st);
}

// ---------------------------------------------------------------- k_compose
// Sequence-parallel state passing (orkas.ai "Kimi K3 architecture",
// §"請求書はサービング側に回ってくる": a segment's final state is its transition
// applied to the incoming state plus its zero-start state, so the states
// entering consecutive segments follow by composition):
//   S_in[0] = S0,  S_in[g+1] = P[g] S_in[g] + Z[g].
// Columns of S are independent, so a workgroup owns a 64-column block of one
// head and walks the segments in order, its block resident in LDS.  Thread
// (tr, tc) = (tid / 16, tid % 16) computes rows [tr*D/16, (tr+1)*D/16) x
// columns [4 tc, 4 tc + 4) of each product in fp32, P staged through LDS in
// 32-column panels.
template <int D>
__global__ __launch_bounds__(256) void k_compose(const float* __restrict__ P, const float* __restrict__ Z,
                                                 const float* __restrict__ S0, float* __restrict__ S_in,
                                                 int32_t G, int32_t H) {
    constexpr int RPT = D / 16, KP = 32;
    __shared__ float sS[D][64 + 4];
    __shared__ float sP[D][KP + 1];
    const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
    const int h = blockIdx.x / (D / 64), cb = blockIdx.x % (D / 64);
    const int col0 = cb * 64;
    const int64_t hs = (int64_t)D * D;          // one head's state
    const int64_t gs = (int64_t)H * hs;         // one segment's states
    for (int i = tid; i < D * 64; i += 256) {
        const int r = i / 64, c = i % 64;
        const float x = S0 ? S0[h * hs + (int64_t)r * D + col0 + c] : 0.f;
        sS[r][c] = x;
        S_in[h * hs + (int64_t)r * D + col0 + c] = x;
    }
    for (int g = 0; g < G; ++g) {
        float acc[RPT][4];
#pragma unroll
        for (int r = 0; r < RPT; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[r][c] = 0.f;
        const float* Pg = P + g * gs + h * hs;
        for (int l0 = 0; l0 < D; l0 += KP) {
            __syncthreads();   // sS is complete / the previous panel is consumed
            for (int i = tid; i < D * KP; i += 256) sP[i / KP][i % KP] = Pg[(int64_t)(i / KP) * D + l0 + i % KP];
            __syncthreads();
#pragma unroll 4
            for (int l = 0; l < KP; ++l) {
                float b[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) b[c] = sS[l0 + l][4 * tc + c];
#pragma unroll
                for (int r = 0; r < RPT; ++r) {
                    const float a = sP[tr * RPT + r][l];
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[r][c] += a * b[c];
                }
            }
        }
        __syncthreads();   // every product has read sS
        const float* Zg = Z + g * gs + h * hs;
        float* Sg = S_in + (g + 1) * gs + h * hs;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int row = tr * RPT + r;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int col = col0 + 4 * tc + c;
                const float x = acc[r][c] + Zg[(int64_t)row * D + col];
                sS[row][4 * tc + c] = x;
                Sg[(int64_t)row * D + col] = x;
            }
        }
    }
}

hipError_t launch_compose(int32_t G, int32_t H, int32_t d, const float* P, const float* Z, const float* S0,
                          float* S_in, hipStream_t st) {
    const unsigned grid = (unsigned)((int64_t)H * (d / 64));
    if (d == 128)
        hipLaunchKernelGGL((k_compose<128>), dim3(grid), dim3(256), 0, st, P, Z, S0, S_in, G, H);
    else
        hipLaunchKernelGGL((k_compose<64>), dim3(grid), dim3(256), 0, st, P, Z, S0, S_in, G, H);
    return hipGetLastError();
}

// ---------------------------------------------------------------- validator
// counts[0]: log_alpha elements outside [-5, 0] or not finite
// counts[1]: beta elements outside [0, 1] or not finite
// counts[2]: cu_seqlens entries that break cu[0] = 0, cu[i] <= cu[i+1],
//            cu[n_seqs] = total_tokens
__global__ __launch_bounds__(64) void k_validate_clear(unsigned long long* counts) {
    if (threadIdx.x < 3) counts[threadIdx.x] = 0ull;
}

template <typename E>
__global__ __launch_bounds__(256) void k_validate(const E* __restrict__ g, int64_t n_g, const E* __restrict__ beta,
                                                  int64_t n_beta, const int32_t* __restrict__ cu, int32_t n_seqs,
                                                  int64_t total_tokens, unsigned long long* counts) {
    unsigned long long bad_g = 0, bad_b = 0, bad_cu = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_g; i += stride) {
        const float x = to_f(g[i]);
        bad_g += !(x >= -5.f && x <= 0.f);   // NaN fails both comparisons
    }
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_beta; i += stride) {
        const float x = to_f(beta[i]);
        bad_b += !(x >= 0.f && x <= 1.f);
    }
    if (cu) {
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i <= n_seqs; i += stride) {
            const int64_t a = cu[i];
            if (i == 0) bad_cu += a != 0;
            if (i == n_seqs) bad_cu += a != total_tokens;
            if (i < n_seqs) bad_cu += a > (int64_t)cu[i + 1];
        }
    }
    // wave sums, then one vector atomic per wave and counter
    for (int off = 32; off > 0; off >>= 1) {
        bad_g += __shfl_down(bad_g, off);
        bad_b += __shfl_down(bad_b, off);
        bad_cu += __shfl_down(bad_cu, off);
    }
    if ((threadIdx.x & 63) == 0) {
        if (bad_g) atomicAdd(&counts[0], bad_g);
        if (bad_b) atomicAdd(&counts[1], bad_b);
        if (bad_cu) atomicAdd(&counts[2], bad_cu);
    }
}

hipError_t launch_validate(bool bf16, int64_t total_tokens, int32_t n_seqs, int32_t n_heads, int32_t d_k,
                           const void* beta, const void* g, const int32_t* cu, unsigned long long* counts,
                           hipStream_t st) {
    hipLaunchKernelGGL(k_validate_clear, dim3(1), dim3(64), 0, st, counts);
    const int64_t n_g = total_tokens * n_heads * d_k, n_beta = total_tokens * n_heads;
    const int64_t want = (n_g + 255) / 256;
    const unsigned grid = (unsigned)(want < 1 ? 1 : (want > 4096 ? 4096 : want));
    if (bf16)
        hipLaunchKernelGGL((k_validate<__bf16>), dim3(grid), dim3(256), 0, st, static_cast<const __bf16*>(g), n_g,
                           static_cast<const __bf16*>(beta), n_beta, cu, n_seqs, total_tokens, counts);
    else
        hipLaunchKernelGGL((k_validate<float>), dim3(grid), dim3(256), 0, st, static_cast<const float*>(g), n_g,
                           static_cast<const float*>(beta), n_beta, cu, n_seqs, total_tokens, counts);
    return hipGetLastError();
}

// ---------------------------------------------------------------- output epilogue
// y = RMSNorm(o) * sigmoid(z) per (token, head) row of d_v channels (ogis-ri
// NLP primer on Kimi K3, §3.1 "KDA": the read-out is normalised because its
// magnitude varies with the state, then multiplied channel by channel by a
// gate in (0, 1) made from the layer input; W_o follows outside).
// RMSNorm(x) = x / sqrt(mean(x^2) + eps) * w.  16 lanes per row, D/16
// consecutive channels per lane (one 16- or 8-byte load per operand), the
// sum of squares reduced by a 16-lane butterfly; each wave takes blocks of
// 4 * kGateRows consecutive rows, grid-stride, with every load of a block
// issued before the first use; o, z and y are streamed with non-temporal
// hints (each byte is touched once).  y may be o itself: a lane writes only
// the elements it has read, after its row's loads.
// Rows per lane group and pass of the output epilogue (at 2,097,152 rows of
// d = 128, bf16: 1, 2, 4, 8 rows gave 315, 308, 297, 301 us with plain loads
// and stores; 4 rows with non-temporal loads and stores, 284 us; one row per
// lane group and no hints, as first written, 348 us).
constexpr int kGateRows = 4;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

template <typename E, int D>
// y may be o itself (in place), so neither pointer is declared restrict.
__global__ __launch_bounds__(256) void k_output_gate(const E* o, const E* __restrict__ z,
                                                     const float* __restrict__ w, float eps, int64_t n_rows,
                                                     E* y) {
    constexpr int PER = D / 16;                            // channels per lane
    constexpr int NV = (PER * (int)sizeof(E) + 15) / 16;   // vectors per lane per row
    using V = typename std::conditional<PER * sizeof(E) >= 16, uint4, uint2>::type;
    using NT = typename std::conditional<PER * sizeof(E) >= 16, u32x4_t, u32x2_t>::type;   // for the streaming hints
    const int sub = threadIdx.x & 15;
    const int c0 = sub * PER;
    float wv[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) wv[e] = w ? w[c0 + e] : 1.f;
    // A wave takes 4 * kRows consecutive rows per pass (lane group g = lane / 16
    // has rows g, g + 4, ...), and issues all of their loads before any use,
    // so that each wave keeps kRows times more bytes in flight.
    const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
    const int64_t n_waves = (int64_t)gridDim.x * 4;
    const int g = (threadIdx.x >> 4) & 3;
    for (int64_t base = wave * 4 * kGateRows; base < n_rows; base += n_waves * 4 * kGateRows) {
        V vo[kGateRows][NV], vz[kGateRows][NV];
#pragma unroll
        for (int k = 0; k < kGateRows; ++k) {
            int64_t r = base + g + 4 * k;
            r = r < n_rows ? r : n_rows - 1;   // a valid row; its result is not stored
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                vo[k][i] = __builtin_bit_cast(V, __builtin_nontemporal_load(reinterpret_cast<const NT*>(o + r * D + c0) + i));
                vz[k][i] = __builtin_bit_cast(V, __builtin_nontemporal_load(reinterpret_cast<const NT*>(z + r * D + c0) + i));
            }
        }
#pragma unroll
        for (int k = 0; k < kGateRows; ++k) {
            const int64_t r = base + g + 4 * k;
            const E* eo = reinterpret_cast<const E*>(vo[k]);
            const E* ez = reinterpret_cast<const E*>(vz[k]);
            float ov[PER];
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                ov[e] = to_f(eo[e]);
                ss += ov[e] * ov[e];
            }
            ss += __shfl_xor(ss, 1);
            ss += __shfl_xor(ss, 2);
            ss += __shfl_xor(ss, 4);
            ss += __shfl_xor(ss, 8);
            const float inv = rsqrtf(ss / (float)D + eps);
            V vy[NV];
            E* ey = reinterpret_cast<E*>(vy);
#pragma unroll
            for (int e = 0; e < PER; ++e) ey[e] = from_f<E>(ov[e] * inv * wv[e] / (1.f + __expf(-to_f(ez[e]))));
            if (r < n_rows) {
#pragma unroll
                for (int i = 0; i < NV; ++i)
                    __builtin_nontemporal_store(__builtin_bit_cast(NT, vy[i]), reinterpret_cast<NT*>(y + r * D + c0) + i);
            }
        }
    }
}

hipError_t launch_output_gate(bool bf16, int64_t n_rows, int32_t d, const void* o, const void* z, const float* w,
                              float eps, void* y, hipStream_t st) {
    if (n_rows <= 0) return hipSuccess;
    const int64_t want = (n_rows + 16 * kGateRows - 1) / (16 * kGateRows);
    const unsigned blocks = (unsigned)(want < 16384 ? want : 16384);
#define KDA_GATE(E, D)                                                                                      \
    hipLaunchKernelGGL((k_output_gate<E, D>), dim3(blocks), dim3(256), 0, st, static_cast<const E*>(o),   \
                       static_cast<const E*>(z), w, eps, n_rows, static_cast<E*>(y))
    if (bf16) {
        if (d == 128) KDA_GATE(__bf16, 128);
        else KDA_GATE(__bf16, 64);
    } else {
        if (d == 128) KDA_GATE(float, 128);
        else KDA_GATE(float, 64);
    }
#undef KDA_GATE
    return hipGetLastError();
}

}  // namespace kda
