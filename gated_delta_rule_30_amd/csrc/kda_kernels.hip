// KDA chunkwise forward kernels for gfx950.
//
// Per sequence and head the recurrence is
//   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t
// (ogis-ri NLP primer on Kimi K3, §3.1 "KDA（Kimi Delta Attention）").  It is
// evaluated chunk by chunk (same page, §3.1: only the chunk-to-chunk step is
// sequential; inside a chunk everything is a matrix product).  For a chunk of
// L <= 64 tokens with incoming state S, per key channel c:
//   b_r      = sum_{s<=r} g_s                   cumulative log-decay (fp32)
//   Gamma_r  = exp(b_r); decay from token i to token r = exp(b_r - b_i)
//              (§3.1 "chunk 内の減衰と、その数値範囲": Gamma_j / Gamma_i)
//   A[r,i]   = beta_r sum_c k_rc k_ic exp(b_rc - b_ic)      (i < r)
//   T        = (I + A)^-1                       delta-rule correction
//   W = T diag(beta) (K . Gamma),   U = T diag(beta) V
//   U~ = U - W S                                 written deltas of the chunk
//   O  = (Q . Gamma) S + M U~,    M[r,i] = sum_c q_rc k_ic exp(b_rc - b_ic)  (i <= r)
//   S' = Diag(Gamma_L) S + (K . exp(b_L - b))^T U~
//
// Sub-tiling (orkas.ai "Kimi K3 architecture", §"GPU のコードパスを一本消した
// 「下界」"): with g >= -5, b varies by less than 80 inside a 16-token
// sub-tile, so for row sub-tile R with reference rho_R = b at the end of
// sub-tile R-1 (0 at the chunk start) the operands
//   row    : x_r . exp(b_r - rho_R)      factor in (e^-80, 1]
//   column : k_i . exp(rho_R - b_i)      factor in [1, e^80) on the diagonal
//                                        sub-tile, <= 1 left of it
// stay inside bf16 range, and every (R, J <= R) block of A and M -- the
// diagonal ones included -- is one dense MFMA contraction over d_k.
//
// Kernels (one launch each, all on the caller's stream):
//   k_chunk_table : chunk list from cu_seqlens (device side, no host sync)
//   k_cumsum      : b per chunk
//   k_wy          : A, T (LDS, fp32), W, U, K^ = K . exp(b_L - b), Gamma_L
//   k_state       : sequential over chunks per (sequence, head, value slab)
//   k_output      : M and O per chunk
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// ---------------------------------------------------------------- chunk table
// One workgroup.  Sequence n contributes ceil(len_n / 64) chunks; chunks are
// aligned to each sequence's first token and the last one may be partial.
__global__ __launch_bounds__(1024) void k_chunk_table(const int32_t* __restrict__ cu, int32_t n_seqs,
                                                      int64_t total_tokens, int64_t fixed_len,
                                                      int32_t max_chunks, ChunkInfo* __restrict__ tab,
                                                      int32_t* __restrict__ seq_chunk0,
                                                      int32_t* __restrict__ n_chunks_out) {
    __shared__ int32_t s_scan[1024];
    __shared__ int32_t s_carry;
    const int tid = threadIdx.x;
    if (tid == 0) s_carry = 0;
    __syncthreads();
    for (int32_t base = 0; base < n_seqs; base += 1024) {
        const int32_t n = base + tid;
        int64_t start = 0, len = 0;
        if (n < n_seqs) {
            if (cu) {
                start = cu[n];
                int64_t end = cu[n + 1];
                // Clamp so that malformed offsets can never address outside [0, total_tokens).
                start = start < 0 ? 0 : (start > total_tokens ? total_tokens : start);
                end = end < start ? start : (end > total_tokens ? total_tokens : end);
                len = end - start;
            } else {
                start = (int64_t)n * fixed_len;
                len = fixed_len;
            }
        }
        const int32_t cnt = (int32_t)((len + kChunk - 1) / kChunk);
        s_scan[tid] = cnt;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            int32_t add = tid >= off ? s_scan[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += add;
            __syncthreads();
        }
        const int32_t carry = s_carry;
        const int32_t first = carry + s_scan[tid] - cnt;
        if (n < n_seqs) {
            seq_chunk0[n] = first < max_chunks ? first : max_chunks;
            for (int32_t j = 0; j < cnt; ++j) {
                const int32_t c = first + j;
                if (c >= max_chunks) break;
                ChunkInfo ci;
                ci.tok0 = start + (int64_t)j * kChunk;
                ci.seq = n;
                const int64_t rem = len - (int64_t)j * kChunk;
                ci.len = (int32_t)(rem < kChunk ? rem : kChunk);
                tab[c] = ci;
            }
        }
        __syncthreads();
        if (tid == 1023) s_carry = carry + s_scan[1023];
        __syncthreads();
    }
    if (tid == 0) {
        const int32_t total = s_carry < max_chunks ? s_carry : max_chunks;
        seq_chunk0[n_seqs] = total;
        *n_chunks_out = total;
    }
}

// ---------------------------------------------------------------- cumsum
// b[t, h, c] = sum of g over the chunk's tokens up to and including t.
// One thread per key channel; grid (chunk, head).
template <typename E, int D>
__global__ __launch_bounds__(D) void k_cumsum(const E* __restrict__ g, const ChunkInfo* __restrict__ tab,
                                              const int32_t* __restrict__ n_chunks_p, int32_t H,
                                              float* __restrict__ bcum) {
    const int32_t ci = blockIdx.x;
    if (ci >= *n_chunks_p) return;
    const ChunkInfo info = tab[ci];
    const int64_t rs = (int64_t)H * D;
    const int64_t base = (info.tok0 * H + blockIdx.y) * D + threadIdx.x;
    float acc = 0.f;
    float buf[16];
    for (int r0 = 0; r0 < info.len; r0 += 16) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
            buf[j] = (r0 + j < info.len) ? to_f(g[base + (r0 + j) * rs]) : 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            acc += buf[j];
            if (r0 + j < info.len) bcum[base + (r0 + j) * rs] = acc;
        }
    }
}

// Strictly-lower (A, with beta) or inclusive-lower (M) block (R, J<=R) of the
// decayed Gram matrix between row operand X (q or k) and the keys, evaluated
// with the sub-tile reference of row block R.  sX/sK: [64][PE] elements,
// sB: [64][PB] fp32 cumulative log-decay.  Returns the MFMA accumulator.
template <typename E, int D, int PE, int PB>
__device__ inline f32x4 decayed_gram_block(const E* sX, const E* sK, const float* sB, int R, int J) {
    using M = Mma<E>;
    const int li = lane_id() & 15, lg = lane_id() >> 4;
    const int r = kSub * R + li;        // row token of this lane's A fragment
    const int i = kSub * J + li;        // column token of this lane's B fragment
    const float* rho = R ? sB + (kSub * R - 1) * PB : nullptr;
    f32x4 acc = zero4();
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += M::KS) {
        typename M::frag a, b;
        if constexpr (M::KW == 1) {
            const int c = k0 + lg;
            const float rh = rho ? rho[c] : 0.f;
            a = to_f(sX[r * PE + c]) * __expf(sB[r * PB + c] - rh);
            b = to_f(sK[i * PE + c]) * __expf(rh - sB[i * PB + c]);
        } else {
#pragma unroll
            for (int j = 0; j < M::KW; ++j) {
                const int c = k0 + lg * M::KW + j;
                const float rh = rho ? rho[c] : 0.f;
                a[j] = from_f<E>(to_f(sX[r * PE + c]) * __expf(sB[r * PB + c] - rh));
                b[j] = from_f<E>(to_f(sK[i * PE + c]) * __expf(rh - sB[i * PB + c]));
            }
        }
        acc = M::mma(a, b, acc);
    }
    return acc;
}

__device__ inline void block_of(int blk, int& R, int& J) {
    // (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3)
    R = blk < 1 ? 0 : blk < 3 ? 1 : blk < 6 ? 2 : 3;
    J = blk - (R * (R + 1)) / 2;
}

// ---------------------------------------------------------------- WY / UT transform
template <typename E, int D>
__global__ __launch_bounds__(kThreads) void k_wy(const E* __restrict__ k, const E* __restrict__ v,
                                                 const E* __restrict__ beta, const float* __restrict__ bcum,
                                                 const ChunkInfo* __restrict__ tab,
                                                 const int32_t* __restrict__ n_chunks_p, int32_t H,
                                                 E* __restrict__ W, E* __restrict__ U, E* __restrict__ Kh,
                                                 float* __restrict__ gam) {
    using M = Mma<E>;
    constexpr int C = kChunk;
    constexpr int PE = D + 8;     // row pitch (elements) of [token][channel] tiles
    constexpr int PB = D + 4;     // row pitch of the fp32 log-decay tile
    constexpr int PT = C + 4;     // row pitch of the fp32 C x C matrices
    constexpr int PO = C + 8;     // row pitch (elements) of [n][token] operand tiles
    // Region 1 (k tile, log-decay tile) is dead once A and (K . Gamma)^T are
    // formed; region 2 (T, scratch, T diag(beta)) reuses its bytes.
    constexpr int kReg1 = C * PE * (int)sizeof(E) + C * PB * 4;
    constexpr int kReg2 = C * PT * 4 + 4 * 16 * 17 * 4 + C * PO * (int)sizeof(E);
    __shared__ __attribute__((aligned(16))) unsigned char sR[kReg1 > kReg2 ? kReg1 : kReg2];
    E* sK = reinterpret_cast<E*>(sR);
    float* sB = reinterpret_cast<float*>(sR + C * PE * sizeof(E));
    float* sT = reinterpret_cast<float*>(sR);
    float* sX = sT + C * PT;
    E* sTo = reinterpret_cast<E*>(sX + 4 * 16 * 17);
    __shared__ __attribute__((aligned(16))) float sA[C * PT];
    __shared__ __attribute__((aligned(16))) E sKgt[D * PO];
    __shared__ __attribute__((aligned(16))) E sVt[D * PO];
    __shared__ float sBeta[C];

    const int32_t ci = blockIdx.x;
    if (ci >= *n_chunks_p) return;
    const ChunkInfo info = tab[ci];
    const int h = blockIdx.y;
    const int len = info.len;
    const int tid = threadIdx.x, wave = wave_id(), li = lane_id() & 15, lg = lane_id() >> 4;
    const int64_t rs = (int64_t)H * D;
    const int64_t base = (info.tok0 * H + h) * D;

    // 1. stage k, b, v^T and beta; rows past the chunk end are zero (b copies the last row)
    for (int idx = tid; idx < C * D; idx += kThreads) {
        const int r = idx / D, c = idx % D;
        const bool ok = r < len;
        const int64_t off = base + (int64_t)(ok ? r : len - 1) * rs + c;
        sK[r * PE + c] = ok ? k[off] : from_f<E>(0.f);
        sB[r * PB + c] = bcum[off];
        sVt[c * PO + r] = ok ? v[off] : from_f<E>(0.f);
    }
    for (int r = tid; r < C; r += kThreads)
        sBeta[r] = r < len ? to_f(beta[(info.tok0 + r) * H + h]) : 0.f;
    __syncthreads();

    // 2. A = diag(beta) StrictTril(decayed K K^T), 10 sub-tile blocks over 4 waves
    for (int blk = wave; blk < 10; blk += 4) {
        int R, J;
        block_of(blk, R, J);
        const f32x4 acc = decayed_gram_block<E, D, PE, PB>(sK, sK, sB, R, J);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int row = kSub * R + 4 * lg + rr, col = kSub * J + li;
            sA[row * PT + col] = (J < R || col < row) ? sBeta[row] * acc[rr] : 0.f;
        }
    }
    // 3. (K . Gamma)^T for W, and K^ = K . exp(b_L - b), Gamma_L to global
    {
        const float* bL = sB + (len - 1) * PB;
        for (int idx = tid; idx < C * D; idx += kThreads) {
            const int r = idx / D, c = idx % D;
            const float kv = to_f(sK[r * PE + c]);
            const float bv = sB[r * PB + c];
            sKgt[c * PO + r] = from_f<E>(kv * __expf(bv));
            if (r < len) Kh[base + (int64_t)r * rs + c] = from_f<E>(kv * __expf(bL[c] - bv));
        }
        for (int c = tid; c < D; c += kThreads) gam[((int64_t)ci * H + h) * D + c] = __expf(bL[c]);
    }
    __syncthreads();

    // 4a. inverses of the four unit-lower-triangular diagonal blocks (forward substitution)
    if (lg == 0) {
        const int R = wave, j = li;
        float x[kSub];
#pragma unroll
        for (int r = 0; r < kSub; ++r) {
            float s = (r == j) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) s -= sA[(kSub * R + r) * PT + kSub * R + i] * x[i];
            x[r] = s;
        }
#pragma unroll
        for (int r = 0; r < kSub; ++r) sT[(kSub * R + r) * PT + kSub * R + j] = x[r];
    }
    for (int idx = tid; idx < C * C; idx += kThreads) {
        const int r = idx / C, c = idx % C;
        if ((c >> 4) > (r >> 4)) sT[r * PT + c] = 0.f;
    }
    __syncthreads();
    // 4b. off-diagonal blocks: T_RJ = -T_RR sum_{K=J}^{R-1} A_RK T_KJ, by distance R-J
    for (int d = 1; d < kNSub; ++d) {
        const bool act = wave < kNSub - d;
        const int J = wave, R = wave + d;
        if (act) {
            f32x4 acc = zero4();
            for (int K = J; K < R; ++K)
#pragma unroll
                for (int kk = 0; kk < kSub; kk += 4)
                    acc = mma_f32(sA[(kSub * R + li) * PT + kSub * K + kk + lg],
                                  sT[(kSub * K + kk + lg) * PT + kSub * J + li], acc);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) sX[wave * 272 + (4 * lg + rr) * 17 + li] = acc[rr];
        }
        __syncthreads();
        if (act) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < kSub; kk += 4)
                acc = mma_f32(sT[(kSub * R + li) * PT + kSub * R + kk + lg],
                              sX[wave * 272 + (kk + lg) * 17 + li], acc);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) sT[(kSub * R + 4 * lg + rr) * PT + kSub * J + li] = -acc[rr];
        }
        __syncthreads();
    }
    // 5. T diag(beta) in the operand dtype
    for (int idx = tid; idx < C * C; idx += kThreads) {
        const int r = idx / C, i = idx % C;
        sTo[r * PO + i] = from_f<E>(sT[r * PT + i] * sBeta[i]);
    }
    __syncthreads();
    // 6. W = T diag(beta) (K . Gamma),  U = T diag(beta) V
    constexpr int NCT = D / kSub;
    for (int t = wave; t < 2 * kNSub * NCT; t += 4) {
        const int mat = t / (kNSub * NCT), rem = t % (kNSub * NCT);
        const int R = rem / NCT, ct = rem % NCT;
        const E* Bt = mat ? sVt : sKgt;
        const int kend = ((kSub * (R + 1) + M::KS - 1) / M::KS) * M::KS;
        f32x4 acc = zero4();
        for (int k0 = 0; k0 < kend; k0 += M::KS)
            acc = M::mma(M::load(&sTo[(kSub * R + li) * PO + k0 + lg * M::KW]),
                         M::load(&Bt[(kSub * ct + li) * PO + k0 + lg * M::KW]), acc);
        E* out = mat ? U : W;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int row = kSub * R + 4 * lg + rr;
            if (row < len) out[base + (int64_t)row * rs + kSub * ct + li] = from_f<E>(acc[rr]);
        }
    }
}

// ---------------------------------------------------------------- state propagation
// Sequential over the chunks of one sequence, for one head and one slab of
// kSlab value columns (columns of S evolve independently).  S stays in fp32
// registers; per chunk:  U~ = U - W S,  S <- Diag(Gamma_L) S + K^T U~.
// Emits S^T at every chunk start and U~^T (both in the operand dtype) for the
// output kernel, and S_T at the end.
constexpr int kSlab = 32;

template <typename E, int D>
__global__ __launch_bounds__(kThreads) void k_state(const E* __restrict__ W, const E* __restrict__ U,
                                                    const E* __restrict__ Kh, const float* __restrict__ gam,
                                                    const ChunkInfo* __restrict__ tab,
                                                    const int32_t* __restrict__ seq_chunk0, int32_t H,
                                                    const float* __restrict__ S0, float* __restrict__ ST,
                                                    E* __restrict__ Sc, E* __restrict__ Utg) {
    using M = Mma<E>;
    constexpr int C = kChunk;
    constexpr int NS = D / kSlab;          // slabs per head
    constexpr int RT = D / 64;             // 16-row state tiles per wave
    constexpr int PS = D + 8, PW = D + 8, PK = C + 8, PU = C + 8;
    __shared__ __attribute__((aligned(16))) E sSt[kSlab * PS];   // S^T  [col][channel]
    __shared__ __attribute__((aligned(16))) E sW[C * PW];        // W    [token][channel]
    __shared__ __attribute__((aligned(16))) E sKt[D * PK];       // K^T  [channel][token]
    __shared__ __attribute__((aligned(16))) E sUt[kSlab * PU];   // U~^T [col][token]
    __shared__ float sGam[D];

    const int sl = blockIdx.x % NS;
    const int h = (blockIdx.x / NS) % H;
    const int n = blockIdx.x / (NS * H);
    const int tid = threadIdx.x, wave = wave_id(), li = lane_id() & 15, lg = lane_id() >> 4;
    const int64_t rs = (int64_t)H * D;
    const int col0 = sl * kSlab;

    // S[a][b][rr] = state[channel 16*(RT*wave + a) + 4*lg + rr][column col0 + 16*b + li]
    f32x4 S[RT][2];
    const int64_t sbase = ((int64_t)n * H + h) * D * D;
#pragma unroll
    for (int a = 0; a < RT; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int ch = kSub * (RT * wave + a) + 4 * lg + rr;
                S[a][b][rr] = S0 ? S0[sbase + (int64_t)ch * D + col0 + kSub * b + li] : 0.f;
            }

    const int32_t c_begin = seq_chunk0[n], c_end = seq_chunk0[n + 1];
    for (int32_t ci = c_begin; ci < c_end; ++ci) {
        const ChunkInfo info = tab[ci];
        const int len = info.len;
        const int64_t base = (info.tok0 * H + h) * D;
        const int64_t cbase = ((int64_t)ci * H + h) * D;
        // S (operand dtype) to LDS as S^T and to the workspace for the output kernel
#pragma unroll
        for (int a = 0; a < RT; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int ch = kSub * (RT * wave + a) + 4 * lg + rr, col = kSub * b + li;
                    const E sv = from_f<E>(S[a][b][rr]);
                    sSt[col * PS + ch] = sv;
                    Sc[(cbase + col0 + col) * D + ch] = sv;
                }
        for (int idx = tid; idx < C * D; idx += kThreads) {
            const int r = idx / D, c = idx % D;
            const bool ok = r < len;
            sW[r * PW + c] = ok ? W[base + (int64_t)r * rs + c] : from_f<E>(0.f);
            sKt[c * PK + r] = ok ? Kh[base + (int64_t)r * rs + c] : from_f<E>(0.f);
        }
        for (int c = tid; c < D; c += kThreads) sGam[c] = gam[cbase + c];
        __syncthreads();
        // U~ = U - W S : wave -> token rows 16*wave.., two 16-column tiles
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            f32x4 acc = zero4();
#pragma unroll
            for (int k0 = 0; k0 < D; k0 += M::KS)
                acc = M::mma(M::load(&sW[(kSub * wave + li) * PW + k0 + lg * M::KW]),
                             M::load(&sSt[(kSub * b + li) * PS + k0 + lg * M::KW]), acc);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int tok = kSub * wave + 4 * lg + rr, col = kSub * b + li;
                const float u = tok < len ? to_f(U[base + (int64_t)tok * rs + col0 + col]) : 0.f;
                const E ut = from_f<E>(tok < len ? u - acc[rr] : 0.f);
                sUt[col * PU + tok] = ut;
                Utg[(cbase + col0 + col) * C + tok] = ut;
            }
        }
        __syncthreads();
        // S <- Diag(Gamma_L) S + K^T U~
#pragma unroll
        for (int a = 0; a < RT; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                f32x4 acc = zero4();
#pragma unroll
                for (int k0 = 0; k0 < C; k0 += M::KS)
                    acc = M::mma(M::load(&sKt[(kSub * (RT * wave + a) + li) * PK + k0 + lg * M::KW]),
                                 M::load(&sUt[(kSub * b + li) * PU + k0 + lg * M::KW]), acc);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int ch = kSub * (RT * wave + a) + 4 * lg + rr;
                    S[a][b][rr] = sGam[ch] * S[a][b][rr] + acc[rr];
                }
            }
        __syncthreads();
    }
    if (ST) {
#pragma unroll
        for (int a = 0; a < RT; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int ch = kSub * (RT * wave + a) + 4 * lg + rr;
                    ST[sbase + (int64_t)ch * D + col0 + kSub * b + li] = S[a][b][rr];
                }
    }
}

// ---------------------------------------------------------------- output
// O = (Q . Gamma) S + M U~ per chunk and head.
template <typename E, int D>
__global__ __launch_bounds__(kThreads) void k_output(const E* __restrict__ q, const E* __restrict__ k,
                                                     const float* __restrict__ bcum,
                                                     const E* __restrict__ Sc, const E* __restrict__ Utg,
                                                     const ChunkInfo* __restrict__ tab,
                                                     const int32_t* __restrict__ n_chunks_p, int32_t H,
                                                     E* __restrict__ o) {
    using M = Mma<E>;
    constexpr int C = kChunk;
    constexpr int PE = D + 8, PB = D + 4, PM = C + 8, PS = D + 8, PU = C + 8;
    __shared__ __attribute__((aligned(16))) E sQ[C * PE];
    __shared__ __attribute__((aligned(16))) E sK[C * PE];
    __shared__ __attribute__((aligned(16))) float sB[C * PB];
    __shared__ __attribute__((aligned(16))) E sM[C * PM];
    __shared__ __attribute__((aligned(16))) E sSt[D * PS];
    __shared__ __attribute__((aligned(16))) E sUt[D * PU];

    const int32_t ci = blockIdx.x;
    if (ci >= *n_chunks_p) return;
    const ChunkInfo info = tab[ci];
    const int h = blockIdx.y;
    const int len = info.len;
    const int tid = threadIdx.x, wave = wave_id(), li = lane_id() & 15, lg = lane_id() >> 4;
    const int64_t rs = (int64_t)H * D;
    const int64_t base = (info.tok0 * H + h) * D;
    const int64_t cbase = ((int64_t)ci * H + h) * D;

    for (int idx = tid; idx < C * D; idx += kThreads) {
        const int r = idx / D, c = idx % D;
        const bool ok = r < len;
        const int64_t off = base + (int64_t)(ok ? r : len - 1) * rs + c;
        sQ[r * PE + c] = ok ? q[off] : from_f<E>(0.f);
        sK[r * PE + c] = ok ? k[off] : from_f<E>(0.f);
        sB[r * PB + c] = bcum[off];
    }
    for (int idx = tid; idx < D * D; idx += kThreads) {
        const int col = idx / D, ch = idx % D;
        sSt[col * PS + ch] = Sc[(cbase + col) * D + ch];
    }
    for (int idx = tid; idx < D * C; idx += kThreads) {
        const int col = idx / C, tok = idx % C;
        sUt[col * PU + tok] = Utg[(cbase + col) * C + tok];
    }
    __syncthreads();
    // M = Tril_incl(decayed Q K^T), 10 blocks; upper blocks zero
    for (int blk = wave; blk < 10; blk += 4) {
        int R, J;
        block_of(blk, R, J);
        const f32x4 acc = decayed_gram_block<E, D, PE, PB>(sQ, sK, sB, R, J);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int row = kSub * R + 4 * lg + rr, col = kSub * J + li;
            sM[row * PM + col] = from_f<E>((J < R || col <= row) ? acc[rr] : 0.f);
        }
    }
    for (int idx = tid; idx < C * C; idx += kThreads) {
        const int r = idx / C, c = idx % C;
        if ((c >> 4) > (r >> 4)) sM[r * PM + c] = from_f<E>(0.f);
    }
    __syncthreads();
    // Q . Gamma in place
    for (int idx = tid; idx < C * D; idx += kThreads) {
        const int r = idx / D, c = idx % D;
        sQ[r * PE + c] = from_f<E>(to_f(sQ[r * PE + c]) * __expf(sB[r * PB + c]));
    }
    __syncthreads();
    constexpr int NCT = D / kSub;
    for (int t = wave; t < kNSub * NCT; t += 4) {
        const int R = t / NCT, ct = t % NCT;
        f32x4 acc = zero4();
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += M::KS)
            acc = M::mma(M::load(&sQ[(kSub * R + li) * PE + k0 + lg * M::KW]),
                         M::load(&sSt[(kSub * ct + li) * PS + k0 + lg * M::KW]), acc);
        const int kend = ((kSub * (R + 1) + M::KS - 1) / M::KS) * M::KS;
        for (int k0 = 0; k0 < kend; k0 += M::KS)
            acc = M::mma(M::load(&sM[(kSub * R + li) * PM + k0 + lg * M::KW]),
                         M::load(&sUt[(kSub * ct + li) * PU + k0 + lg * M::KW]), acc);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int row = kSub * R + 4 * lg + rr;
            if (row < len) o[base + (int64_t)row * rs + kSub * ct + li] = from_f<E>(acc[rr]);
        }
    }
}

// ---------------------------------------------------------------- launch sequence
// `ev`, when given, holds kNumStages + 1 events: ev[i] is recorded before
// stage i and ev[kNumStages] after the last one (stages that do not run for
// these sizes still get their pair of records, with nothing between them).
template <typename E, int D>
static hipError_t launch_all(const Plan& p, hipStream_t st, hipEvent_t* ev) {
    auto mark = [&](int i) {
        if (ev) hipEventRecord(ev[i], st);
    };
    const E* q = static_cast<const E*>(p.q);
    const E* kk = static_cast<const E*>(p.k);
    const E* v = static_cast<const E*>(p.v);
    const E* beta = static_cast<const E*>(p.beta);
    const E* g = static_cast<const E*>(p.g);
    E* W = static_cast<E*>(p.ws_W);
    E* U = static_cast<E*>(p.ws_U);
    E* Kh = static_cast<E*>(p.ws_Kh);
    E* Sc = static_cast<E*>(p.ws_Sc);
    E* Ut = static_cast<E*>(p.ws_Ut);
    const int32_t H = p.n_heads;

    const bool work = p.total_tokens > 0;
    const dim3 cgrid(p.max_chunks, H);
    mark(0);
    hipLaunchKernelGGL(k_chunk_table, dim3(1), dim3(1024), 0, st, p.cu_seqlens, p.n_seqs, p.total_tokens,
                       p.fixed_len, p.max_chunks, p.ws_tab, p.ws_seq_chunk0, p.ws_n_chunks);
    mark(1);
    if (work) hipLaunchKernelGGL((k_cumsum<E, D>), cgrid, dim3(D), 0, st, g, p.ws_tab, p.ws_n_chunks, H, p.ws_b);
    mark(2);
    if (work)
        hipLaunchKernelGGL((k_wy<E, D>), cgrid, dim3(kThreads), 0, st, kk, v, beta, p.ws_b, p.ws_tab,
                           p.ws_n_chunks, H, W, U, Kh, p.ws_gam);
    mark(3);
    hipLaunchKernelGGL((k_state<E, D>), dim3(p.n_seqs * H * (D / kSlab)), dim3(kThreads), 0, st, W, U, Kh,
                       p.ws_gam, p.ws_tab, p.ws_seq_chunk0, H, p.S0, p.S_T, Sc, Ut);
    mark(4);
    if (work)
        hipLaunchKernelGGL((k_output<E, D>), cgrid, dim3(kThreads), 0, st, q, kk, p.ws_b, Sc, Ut, p.ws_tab,
                           p.ws_n_chunks, H, static_cast<E*>(p.o));
    mark(5);
    return hipGetLastError();
}

const char* const kStageNames[kNumStages] = {"k_chunk_table", "k_cumsum", "k_wy", "k_state", "k_output"};

hipError_t launch(const Plan& p, hipStream_t st, hipEvent_t* ev) {
    if (p.bf16) {
        if (p.d == 128) return launch_all<__bf16, 128>(p, st, ev);
        return launch_all<__bf16, 64>(p, st, ev);
    }
    // fp32 operands are built for d = 64 only (their LDS tiles at d = 128
    // exceed one workgroup's LDS); the C ABI rejects other sizes.
    return launch_all<float, 64>(p, st, ev);
}

}  // namespace kda
