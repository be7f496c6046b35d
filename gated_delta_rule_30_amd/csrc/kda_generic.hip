// KDA chunkwise forward for every supported size outside the tuned one.
//
// The tuned kernels (kda_kernels.hip) cover chunk 64 with d_k = d_v: bf16 at
// 64 and 128, fp32 at 64.  These kernels take any chunk C in {16, 32, 64,
// 128}, any d_k, d_v in {64, 128} and either input type, with plain fp32
// arithmetic throughout (no MFMA, operands staged through LDS).  They
// compute the same chunked form (ogis-ri NLP primer on Kimi K3, §3.1
// "KDA（Kimi Delta Attention）": per chunk, the state carried in plus a
// causal intra-chunk term; §3.1 "chunk 内の減衰と、その数値範囲": per-channel
// decay ratios within a chunk), per chunk of C tokens with b the cumulative
// log-decay from the chunk start:
//   A[r][i] = beta_r sum_c k_rc k_ic e^{b_rc - b_ic}   (i < r)
//   M[r][i] =        sum_c q_rc k_ic e^{b_rc - b_ic}   (i <= r)
//   T diag(beta) with T = (I + A)^-1
//   Y  = V - (K . e^b) S,   U~ = T diag(beta) Y
//   O  = (Q . e^b) S + M U~
//   S' = Diag(e^{b_L}) S + (K . e^{b_L - b})^T U~
// Every exponent is <= 0 when log alpha <= 0 (r >= i), so in fp32 the decay
// ratios are formed directly for each token pair and channel: a long chunk
// only underflows terms that are negligible anyway.
//
//   kg_gram  (chunks, H, C/16)  16 rows of A and M per workgroup, and those
//                               rows of Q.e^b, K.e^b, K.e^{b_L-b}
//   kg_solve (chunks, H)        T diag(beta) in LDS by forward substitution
//   kg_recur (N*H*d_v/16)       sequential over one sequence's chunks for one
//                               head and 16 value columns of the state
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int kGenMaxC = 128, kGenMaxD = 128;
constexpr int kGenRows = 16;    // A and M rows per kg_gram workgroup
constexpr int kGenCols = 16;    // value columns per kg_recur workgroup

struct GenArgs {
    const void *q, *k, *v, *beta, *g;
    const float* S0;
    void* o;
    float* S_T;
    const int32_t* cu;
    const ChunkInfo* tab;
    const int32_t* n_chunks;
    const int32_t* seq_chunk0;
    int64_t total_tokens, fixed_len;
    int32_t n_seqs, H, C, DK, DV, max_chunks;
    float *Qg, *Kg, *Kh;     // [H][max_chunks][C][DK]
    float *TB, *M;           // [H][max_chunks][C][C] (TB holds A until kg_solve)
    float* gam;              // [H][max_chunks][DK]
};

// Tokens [tok0, tok0 + len) of chunk ci; false when ci is past the last chunk.
__device__ inline bool gen_chunk(const GenArgs& a, int32_t ci, int64_t& tok0, int& len) {
    if (!a.cu) {
        const int64_t per = (a.fixed_len + a.C - 1) / a.C;
        if (ci >= (int64_t)a.n_seqs * per) return false;
        const int64_t seq = ci / per, j = ci % per;
        const int64_t rem = a.fixed_len - j * a.C;
        tok0 = seq * a.fixed_len + j * a.C;
        len = (int)(rem < a.C ? rem : a.C);
        return true;
    }
    if (ci >= *a.n_chunks) return false;
    const ChunkInfo info = a.tab[ci];
    tok0 = info.tok0;
    len = info.len;
    return true;
}

template <typename E>
__device__ inline float ldf(const void* p, int64_t i) {
    return to_f(static_cast<const E*>(p)[i]);
}

// ------------------------------------------------------------------ kg_gram
template <typename E>
__global__ __launch_bounds__(256) void kg_gram(GenArgs a) {
    constexpr int P = kGenMaxD + 1;   // row pitch (floats): lanes reading different rows hit different banks
    __shared__ float sB[kGenMaxC * P];          // b, [token][channel]
    __shared__ float sK[kGenMaxC * P];          // k, [token][channel]
    __shared__ float sQ[kGenRows * P];          // q rows of this block
    __shared__ float sBeta[kGenRows];
    const int32_t ci = blockIdx.x;
    const int h = blockIdx.y, r0 = kGenRows * blockIdx.z;
    int64_t tok0;
    int len;
    if (!gen_chunk(a, ci, tok0, len)) return;
    const int C = a.C, DK = a.DK, tid = threadIdx.x;
    const int64_t rs = (int64_t)a.H * DK;
    const int64_t base = tok0 * rs + (int64_t)h * DK;
    // b: per-channel running sum over the chunk (tokens past its end add 0)
    for (int c = tid; c < DK; c += 256) {
        float run = 0.f;
        for (int t = 0; t < C; ++t) {
            run += t < len ? ldf<E>(a.g, base + t * rs + c) : 0.f;
            sB[t * P + c] = run;
        }
    }
    for (int x = tid; x < C * DK; x += 256) {
        const int t = x / DK, c = x % DK;
        sK[t * P + c] = t < len ? ldf<E>(a.k, base + t * rs + c) : 0.f;
    }
    for (int x = tid; x < kGenRows * DK; x += 256) {
        const int t = r0 + x / DK, c = x % DK;
        sQ[(x / DK) * P + c] = t < len ? ldf<E>(a.q, base + t * rs + c) : 0.f;
    }
    if (tid < kGenRows) {
        const int t = r0 + tid;
        sBeta[tid] = t < len ? ldf<E>(a.beta, (tok0 + t) * a.H + h) : 0.f;
    }
    __syncthreads();
    const int64_t slot = (int64_t)h * a.max_chunks + ci;
    // rows r0 .. r0+15 of A and M, every column (zero above the diagonal)
    for (int x = tid; x < kGenRows * C; x += 256) {
        const int rr = x / C, r = r0 + rr, i = x % C;
        float sa = 0.f, sm = 0.f;
        if (i <= r) {
            const float *br = sB + r * P, *bi = sB + i * P, *kr = sK + r * P, *ki = sK + i * P;
            const float* qr = sQ + rr * P;
            for (int c = 0; c < DK; ++c) {
                const float e = __expf(br[c] - bi[c]) * ki[c];
                sa += kr[c] * e;
                sm += qr[c] * e;
            }
        }
        a.TB[(slot * C + r) * C + i] = i < r ? sBeta[rr] * sa : 0.f;
        a.M[(slot * C + r) * C + i] = sm;
    }
    // rows r0 .. r0+15 of Q.e^b, K.e^b and K.e^{b_L - b}; b_L is the running
    // sum at the last slot (tokens past the end added nothing)
    for (int x = tid; x < kGenRows * DK; x += 256) {
        const int rr = x / DK, r = r0 + rr, c = x % DK;
        const float b = sB[r * P + c], bl = sB[(C - 1) * P + c];
        const float eb = __expf(b), kv = sK[r * P + c];
        const int64_t at = (slot * C + r) * DK + c;
        a.Qg[at] = sQ[rr * P + c] * eb;
        a.Kg[at] = kv * eb;
        a.Kh[at] = kv * __expf(bl - b);
    }
    if (blockIdx.z == 0)
        for (int c = tid; c < DK; c += 256) a.gam[slot * DK + c] = __expf(sB[(C - 1) * P + c]);
}

// ------------------------------------------------------------------ kg_solve
// T = (I + A)^-1 for the strictly lower A of one chunk, then T diag(beta),
// written over A.  Row r of T is e_r - sum_{i<r} A[r][i] T[i]; one thread per
// column walks the rows.
template <typename E>
__global__ __launch_bounds__(256) void kg_solve(GenArgs a) {
    constexpr int P = kGenMaxC + 1;
    __shared__ float sA[kGenMaxC * P];
    __shared__ float sT[kGenMaxC * P];
    const int32_t ci = blockIdx.x;
    const int h = blockIdx.y;
    int64_t tok0;
    int len;
    if (!gen_chunk(a, ci, tok0, len)) return;
    const int C = a.C, tid = threadIdx.x;
    const int64_t slot = (int64_t)h * a.max_chunks + ci;
    float* A = a.TB + slot * C * C;
    for (int x = tid; x < C * C; x += 256) sA[(x / C) * P + x % C] = A[x];
    __syncthreads();
    if (tid < C) {
        const int j = tid;
        for (int r = 0; r < C; ++r) {
            float s = r == j ? 1.f : 0.f;
            for (int i = j; i < r; ++i) s -= sA[r * P + i] * sT[i * P + j];
            sT[r * P + j] = r >= j ? s : 0.f;   // each thread reads only its own column of T
        }
    }
    __syncthreads();
    for (int x = tid; x < C * C; x += 256) {
        const int r = x / C, j = x % C;
        const float bj = j < len ? ldf<E>(a.beta, (tok0 + j) * a.H + h) : 0.f;
        A[x] = sT[r * P + j] * bj;
    }
}

// ------------------------------------------------------------------ kg_recur
template <typename E>
__global__ __launch_bounds__(256) void kg_recur(GenArgs a) {
    constexpr int PO = (kGenMaxC > kGenMaxD ? kGenMaxC : kGenMaxD) + 1;
    constexpr int W = kGenCols;
    __shared__ float sOp[kGenMaxC * PO];   // the operand of the current phase, [token][channel or token]
    __shared__ float sS[kGenMaxD * W];     // the state's 16 columns, [channel][column]
    __shared__ float sY[kGenMaxC * W];
    __shared__ float sU[kGenMaxC * W];
    const int C = a.C, DK = a.DK, DV = a.DV, tid = threadIdx.x;
    const int slabs = DV / W;
    const int32_t wg = blockIdx.x;
    const int32_t n = wg / (a.H * slabs);
    const int h = (wg / slabs) % a.H, col0 = W * (wg % slabs);
    const int col = tid % W, row = tid / W;   // 16 rows of 16 columns per pass
    int64_t s_start, s_len;
    if (a.cu) {
        int64_t b0 = a.cu[n], b1 = a.cu[n + 1];
        b0 = b0 < 0 ? 0 : (b0 > a.total_tokens ? a.total_tokens : b0);
        b1 = b1 < b0 ? b0 : (b1 > a.total_tokens ? a.total_tokens : b1);
        s_start = b0;
        s_len = b1 - b0;
    } else {
        s_start = (int64_t)n * a.fixed_len;
        s_len = a.fixed_len;
    }
    int32_t c0, nch = (int32_t)((s_len + C - 1) / C);
    if (a.cu) {
        c0 = a.seq_chunk0[n];
        if (nch > a.seq_chunk0[n + 1] - c0) nch = a.seq_chunk0[n + 1] - c0;
    } else {
        c0 = n * nch;
    }
    const int64_t sbase = ((int64_t)n * a.H + h) * DK * DV;
    for (int x = tid; x < DK * W; x += 256) {
        const int c = x / W, j = x % W;
        sS[x] = a.S0 ? a.S0[sbase + (int64_t)c * DV + col0 + j] : 0.f;
    }
    const int64_t vrs = (int64_t)a.H * DV;
    // copies an R x K fp32 matrix (row-major, K a multiple of 4) into sOp
    auto stage = [&](const float* src, int R, int K) {
        __syncthreads();
        const int kv = K / 4;
        for (int x = tid; x < R * kv; x += 256) {
            const int r = x / kv, c4 = x % kv;
            const float4 f = reinterpret_cast<const float4*>(src + (int64_t)r * K)[c4];
            float* d = sOp + r * PO + 4 * c4;
            d[0] = f.x;
            d[1] = f.y;
            d[2] = f.z;
            d[3] = f.w;
        }
        __syncthreads();
    };
    for (int j = 0; j < nch; ++j) {
        const int64_t slot = (int64_t)h * a.max_chunks + c0 + j;
        const int64_t tok0 = s_start + (int64_t)j * C;
        const int len = (int)(s_len - (int64_t)j * C < C ? s_len - (int64_t)j * C : C);
        // Y = V - (K . e^b) S
        stage(a.Kg + slot * C * DK, C, DK);
        for (int t = row; t < C; t += 256 / W) {
            float x = 0.f;
            for (int c = 0; c < DK; ++c) x += sOp[t * PO + c] * sS[c * W + col];
            const float vv = t < len ? ldf<E>(a.v, (tok0 + t) * vrs + (int64_t)h * DV + col0 + col) : 0.f;
            sY[t * W + col] = t < len ? vv - x : 0.f;
        }
        // U~ = T diag(beta) Y (lower triangular)
        stage(a.TB + slot * C * C, C, C);
        for (int t = row; t < C; t += 256 / W) {
            float u = 0.f;
            for (int i = 0; i <= t; ++i) u += sOp[t * PO + i] * sY[i * W + col];
            sU[t * W + col] = u;
        }
        // O = (Q . e^b) S + M U~
        // (a fixed number of rows per thread, so that the partial sums stay in registers)
        constexpr int kRowsPer = kGenMaxC / (256 / W);
        float acc[kRowsPer];
        stage(a.Qg + slot * C * DK, C, DK);
#pragma unroll
        for (int m = 0; m < kRowsPer; ++m) {
            const int t = row + m * (256 / W);
            float x = 0.f;
            if (t < C)
                for (int c = 0; c < DK; ++c) x += sOp[t * PO + c] * sS[c * W + col];
            acc[m] = x;
        }
        stage(a.M + slot * C * C, C, C);
#pragma unroll
        for (int m = 0; m < kRowsPer; ++m) {
            const int t = row + m * (256 / W);
            if (t >= C) continue;
            float x = acc[m];
            for (int i = 0; i <= t; ++i) x += sOp[t * PO + i] * sU[i * W + col];
            if (t < len) static_cast<E*>(a.o)[(tok0 + t) * vrs + (int64_t)h * DV + col0 + col] = from_f<E>(x);
        }
        // S <- Diag(e^{b_L}) S + (K . e^{b_L - b})^T U~
        stage(a.Kh + slot * C * DK, C, DK);
        constexpr int kChPer = kGenMaxD / (256 / W);
        float ns[kChPer];
#pragma unroll
        for (int m = 0; m < kChPer; ++m) {
            const int c = row + m * (256 / W);
            float x = 0.f;
            if (c < DK) {
                x = a.gam[slot * DK + c] * sS[c * W + col];
                for (int t = 0; t < C; ++t) x += sOp[t * PO + c] * sU[t * W + col];
            }
            ns[m] = x;
        }
        __syncthreads();   // every read of the old state is done
#pragma unroll
        for (int m = 0; m < kChPer; ++m) {
            const int c = row + m * (256 / W);
            if (c < DK) sS[c * W + col] = ns[m];
        }
    }
    __syncthreads();
    if (a.S_T)
        for (int x = tid; x < DK * W; x += 256) {
            const int c = x / W, jj = x % W;
            a.S_T[sbase + (int64_t)c * DV + col0 + jj] = sS[x];
        }
}

// ------------------------------------------------------------------ launch
template <typename E>
static hipError_t launch_gen(const Plan& p, hipStream_t st, hipEvent_t* ev) {
    auto mark = [&](int i) {
        if (ev) (void)hipEventRecord(ev[i], st);
    };
    GenArgs a{};
    a.q = p.q;
    a.k = p.k;
    a.v = p.v;
    a.beta = p.beta;
    a.g = p.g;
    a.S0 = p.S0;
    a.o = p.o;
    a.S_T = p.S_T;
    a.cu = p.cu_seqlens;
    a.tab = p.ws_tab;
    a.n_chunks = p.ws_n_chunks;
    a.seq_chunk0 = p.ws_seq_chunk0;
    a.total_tokens = p.total_tokens;
    a.fixed_len = p.fixed_len;
    a.n_seqs = p.n_seqs;
    a.H = p.n_heads;
    a.C = p.chunk;
    a.DK = p.d_k;
    a.DV = p.d_v;
    a.max_chunks = p.max_chunks;
    a.Qg = static_cast<float*>(p.ws_Qg);
    a.Kg = static_cast<float*>(p.ws_Kg);
    a.Kh = static_cast<float*>(p.ws_KhT);
    a.TB = static_cast<float*>(p.ws_TB);
    a.M = static_cast<float*>(p.ws_M);
    a.gam = p.ws_gam;
    mark(0);
    if (p.cu_seqlens) launch_chunk_table(p, p.chunk, st);
    mark(1);
    if (p.max_chunks > 0) {
        hipLaunchKernelGGL(kg_gram<E>, dim3(p.max_chunks, p.n_heads, p.chunk / kGenRows), dim3(256), 0, st, a);
        hipLaunchKernelGGL(kg_solve<E>, dim3(p.max_chunks, p.n_heads), dim3(256), 0, st, a);
    }
    mark(2);
    hipLaunchKernelGGL(kg_recur<E>, dim3(p.n_seqs * p.n_heads * (p.d_v / kGenCols)), dim3(256), 0, st, a);
    mark(3);
    return hipGetLastError();
}

hipError_t launch_generic(const Plan& p, hipStream_t st, hipEvent_t* ev) {
    if (p.chunk > kGenMaxC || p.chunk % kGenRows != 0 || p.d_k > kGenMaxD || p.d_v > kGenMaxD || p.d_v % kGenCols != 0 ||
        p.d_k % 4 != 0 || p.chunk % 4 != 0)
        return hipErrorInvalidValue;
    return p.bf16 ? launch_gen<__bf16>(p, st, ev) : launch_gen<float>(p, st, ev);
}

}  // namespace kda
