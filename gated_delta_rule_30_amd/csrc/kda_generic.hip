// KDA chunkwise forward for every supported size outside the tuned one.
//
// The tuned kernels (kda_kernels.hip) cover chunk 64 with d_k = d_v: bf16 at
// 64 and 128, fp32 at 64.  These kernels take any chunk C in {16, 32, 64,
// 128}, any d_k, d_v in {64, 128} and either input type, with fp32
// arithmetic throughout (fp32 operands in the workspace, every product on
// fp32 matrix cores: 16x16x4 MFMA steps accumulating in fp32).  They
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
// The decay ratios of A and M factor through b at the first row of each
// 16-token sub-tile (orkas.ai "Kimi K3 architecture", §"GPU のコードパスを
// 一本消した「下界」": with log alpha >= -5 a sub-tile spans at most 80 in
// log-decay), so every entry is a dot product of rows scaled once; factors
// that underflow over a long chunk belong to negligible terms.
//
//   kg_gram  (chunks, H)        A and M of one chunk, 16 rows at a time, and
//                               its rows of Q.e^b, K.e^b, K.e^{b_L-b}
//   kg_solve (chunks, H)        T diag(beta) in LDS, by 16 x 16 blocks
//   kg_recur (N*H*d_v/16)       sequential over one sequence's chunks for one
//                               head and 16 value columns of the state, at
//                               chunk 128 (kg_recur_res for chunks of at
//                               most 64 tokens)
// kg_gram and kg_solve are instantiated per chunk size, so that their LDS
// and thread layout fit it.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int kGenMaxC = 128, kGenMaxD = 128;
constexpr int kGenRows = 16;    // rows of a sub-tile
constexpr int kGenCols = 16;    // value columns per kg_recur workgroup
constexpr int kGenRecurThreads = 512;   // kg_recur threads: one wave per 16-token tile of a 128-token chunk

// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt unconstrained
// (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr unsigned kWaitVmcnt0 = 0x0F70;

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
    float *TB, *M;           // [H][max_chunks][C][C] (TB holds A until kg_solve); only the
                             // 16 x 16 blocks on and below the diagonal are written
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

// Recurrence workgroup -> (sequence n, head h, first value column col0).
// When the (sequence, head) count is a multiple of 8, the slabs of one
// (sequence, head) get workgroup ids congruent mod 8, which places them on
// one XCD: the chunk operands they all read are then fetched into one L2.
__device__ inline void gen_slab(const GenArgs& a, int slabs, int32_t& n, int& h, int& col0) {
    const int32_t bid = blockIdx.x, NH = a.n_seqs * a.H;
    int32_t nh, sl;
    if (NH % 8 == 0) {
        sl = (bid / 8) % slabs;
        nh = (bid % 8) + 8 * (bid / (8 * slabs));
    } else {
        sl = bid % slabs;
        nh = bid / slabs;
    }
    n = nh / a.H;
    h = nh % a.H;
    col0 = kGenCols * sl;
}

template <typename E>
__device__ inline float ldf(const void* p, int64_t i) {
    return to_f(static_cast<const E*>(p)[i]);
}

// 16 bytes of E from element `i` of p, widened to fp32: 8 (bf16) or 4 (fp32)
// values.  Callers keep i a multiple of the count (every row starts on
// 16 bytes: d_k and d_v are multiples of 8, the tensors 16-byte aligned).
template <typename E>
struct Vec16 {
    static constexpr int N = 16 / (int)sizeof(E);
    __device__ static inline void load(const void* p, int64_t i, float* out) {
        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const E*>(p) + i);
        if constexpr (sizeof(E) == 2) {
            const bf16x8 v = __builtin_bit_cast(bf16x8, u);
#pragma unroll
            for (int e = 0; e < 8; ++e) out[e] = (float)v[e];
        } else {
            const float4 f = __builtin_bit_cast(float4, u);
            out[0] = f.x;
            out[1] = f.y;
            out[2] = f.z;
            out[3] = f.w;
        }
    }
};

// ------------------------------------------------------------------ kg_gram
// A and M of one chunk, sub-tile after sub-tile (rows r0 .. r0+15).  With
// rho = b at row r0, e^{b_r - b_i} = e^{b_r - rho} e^{rho - b_i}: for r in
// the sub-tile the first factor lies in [e^-80, 1]; the second is <= 1 for
// i < r0 and <= e^80 for i in the sub-tile (16 tokens at log alpha >= -5),
// which fp32 holds.  So each entry is a plain dot product over channels of
// the rows scaled once, k_r e^{b_r - rho} (or q_r ...) and k_i e^{rho - b_i}:
// one exponential per (row, channel) instead of one per (pair, channel).
// The chunk's log-decay rows are loaded and summed once, k stays in
// registers, and each sub-tile's rows of A and M are 16 x 16 tiles on fp32
// matrix cores.
template <typename E, int CC, int NT>
__global__ __launch_bounds__(NT) void kg_gram(GenArgs a) {
    constexpr int P = kGenMaxD + 4;
    constexpr int NV = Vec16<E>::N;
    constexpr int kTileVec = CC * kGenMaxD / NV / NT;   // 16-byte vectors per thread of a full tile
    static_assert(kTileVec >= 1 && CC <= NT, "whole tiles per thread; one thread per row for beta");
    __shared__ __attribute__((aligned(16))) float sB[CC * P];    // g, then b
    __shared__ __attribute__((aligned(16))) float sKi[CC * P];   // k_i e^{rho - b_i} for the current sub-tile
    __shared__ __attribute__((aligned(16))) float sKr[kGenRows * P];
    __shared__ __attribute__((aligned(16))) float sQr[kGenRows * P];
    __shared__ float sBeta[CC];
    typedef float v4 __attribute__((ext_vector_type(4)));
    const int32_t ci = blockIdx.x;
    const int h = blockIdx.y;
    int64_t tok0;
    int len;
    if (!gen_chunk(a, ci, tok0, len)) return;
    constexpr int C = CC;
    const int DK = a.DK, tid = threadIdx.x;
    const int64_t rs = (int64_t)a.H * DK;
    const int64_t base = tok0 * rs + (int64_t)h * DK;
    const int64_t slot = (int64_t)h * a.max_chunks + ci;
    const int vpr = DK / NV;
    // g and k of every row in registers; rows past the chunk end are zero
    float gv[kTileVec * NV], kv[kTileVec * NV];
#pragma unroll
    for (int u = 0; u < kTileVec; ++u) {
        const int x = tid + NT * u, t = x / vpr, c = (x % vpr) * NV;
        const bool in = x < C * vpr && t < len;
        if (in) {
            Vec16<E>::load(a.g, base + t * rs + c, &gv[u * NV]);
            Vec16<E>::load(a.k, base + t * rs + c, &kv[u * NV]);
        }
#pragma unroll
        for (int e = 0; e < NV; ++e) {
            if (!in) gv[u * NV + e] = kv[u * NV + e] = 0.f;
        }
    }
    if (tid < C) sBeta[tid] = tid < len ? ldf<E>(a.beta, (tok0 + tid) * a.H + h) : 0.f;
#pragma unroll
    for (int u = 0; u < kTileVec; ++u) {
        const int x = tid + NT * u, t = x / vpr, c = (x % vpr) * NV;
        if (x < C * vpr)
#pragma unroll
            for (int e = 0; e < NV; ++e) sB[t * P + c + e] = gv[u * NV + e];
    }
    __syncthreads();
    // b: per-channel running sum over the chunk, eight rows read at a time
    for (int c = tid; c < DK; c += NT) {
        float run = 0.f;
        for (int t0 = 0; t0 < C; t0 += 8) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = sB[(t0 + e) * P + c];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                run += x[e];
                sB[(t0 + e) * P + c] = run;
            }
        }
        a.gam[slot * DK + c] = __expf(run);
    }
    __syncthreads();
    // this thread's elements of b (gv is dead)
#pragma unroll
    for (int u = 0; u < kTileVec; ++u) {
        const int x = tid + NT * u, t = x / vpr, c = (x % vpr) * NV;
        if (x < C * vpr)
#pragma unroll
            for (int e = 0; e < NV; ++e) gv[u * NV + e] = sB[t * P + c + e];
    }
    const int wave = tid / 64, lane = tid % 64, li = lane % 16, g = lane / 16;
    for (int z = 0; z < C / kGenRows; ++z) {
        const int r0 = kGenRows * z, nrow = r0 + kGenRows;
        const float* rho = sB + r0 * P;   // b at the sub-tile's first row
        // k_i e^{rho - b_i} for the rows i < nrow
#pragma unroll
        for (int u = 0; u < kTileVec; ++u) {
            const int x = tid + NT * u, t = x / vpr, c = (x % vpr) * NV;
            if (x < C * vpr && t < nrow)
#pragma unroll
                for (int e = 0; e < NV; ++e) sKi[t * P + c + e] = kv[u * NV + e] * __expf(rho[c + e] - gv[u * NV + e]);
        }
        // the sub-tile's rows: scaled operands, and Q.e^b, K.e^b, K.e^{b_L - b}
        for (int x = tid; x < kGenRows * vpr; x += NT) {
            const int rr = x / vpr, r = r0 + rr, c = (x % vpr) * NV;
            float kr[NV], qr[NV];
            if (r < len) {
                Vec16<E>::load(a.k, base + r * rs + c, kr);
                Vec16<E>::load(a.q, base + r * rs + c, qr);
            } else {
#pragma unroll
                for (int e = 0; e < NV; ++e) kr[e] = qr[e] = 0.f;
            }
            const int64_t at = (slot * C + r) * DK + c;
#pragma unroll
            for (int e4 = 0; e4 < NV; e4 += 4) {
                v4 oq, ok, oh;
#pragma unroll
                for (int e = e4; e < e4 + 4; ++e) {
                    const float bv = sB[r * P + c + e], bl = sB[(C - 1) * P + c + e];
                    const float er = __expf(bv - rho[c + e]), eb = __expf(bv);
                    sKr[rr * P + c + e] = kr[e] * er;
                    sQr[rr * P + c + e] = qr[e] * er;
                    oq[e - e4] = qr[e] * eb;
                    ok[e - e4] = kr[e] * eb;
                    oh[e - e4] = kr[e] * __expf(bl - bv);
                }
                *reinterpret_cast<v4*>(a.Qg + at + e4) = oq;
                *reinterpret_cast<v4*>(a.Kg + at + e4) = ok;
                *reinterpret_cast<v4*>(a.Kh + at + e4) = oh;
            }
        }
        __syncthreads();
        // the sub-tile's rows of A and M by 16 x 16 tiles over columns
        // i < nrow (the blocks above the diagonal blocks are zero by
        // structure: they are not written, and no kernel reads them)
        for (int x = wave; x < 2 * (z + 1); x += NT / 64) {
            const int J = x / 2;
            const bool isA = (x % 2) == 0;
            f32x4 acc = zero4();
            {
                const float* arow = (isA ? sKr : sQr) + li * P;
                const float* bcol = sKi + (kGenRows * J + li) * P;
                for (int k0 = 0; k0 < DK; k0 += 16) {
                    const v4 av = *reinterpret_cast<const v4*>(arow + k0 + 4 * g);
                    const v4 bv = *reinterpret_cast<const v4*>(bcol + k0 + 4 * g);
                    acc = mma_f32(av.x, bv.x, acc);
                    acc = mma_f32(av.y, bv.y, acc);
                    acc = mma_f32(av.z, bv.z, acc);
                    acc = mma_f32(av.w, bv.w, acc);
                }
            }
            const int i = kGenRows * J + li;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int r = r0 + 4 * g + rr;
                if (isA)
                    a.TB[(slot * C + r) * C + i] = i < r ? sBeta[r] * acc[rr] : 0.f;
                else
                    a.M[(slot * C + r) * C + i] = i <= r ? acc[rr] : 0.f;
            }
        }
        __syncthreads();   // sKi, sKr and sQr are rewritten for the next sub-tile
    }
}

// ------------------------------------------------------------------ kg_solve
// T = (I + A)^-1 for the strictly lower A of one chunk, by 16 x 16 blocks.
// The diagonal blocks first, all at once, by right-looking elimination
// inside each block (T_KK starts as I; once row i is final every later row
// r takes away A[r][i] times it).  Then block row by block row,
//   T_KL = -T_KK sum_{L <= M < K} A_KM T_ML     (L < K),
// each block of a row one wave's task, on fp32 matrix cores (16x16x4
// steps): A_KM comes from global memory as 16-byte fragments, T_ML from the
// finished rows, kept transposed in LDS so that its fragments are 16-byte
// reads too, and the product's accumulator is already the B operand of the
// multiplication by T_KK.  T diag(beta) is written over A at the end.
template <typename E, int CC>
__global__ __launch_bounds__(256) void kg_solve(GenArgs a) {
    constexpr int B = 16, C = CC, NB = C / B;
    constexpr int PT = C + 4;                       // pitch of the transposed rows
    constexpr int kRowsT = NB > 1 ? (NB - 1) * B : 1;   // T[r][j] kept at sTt[j][r] for column blocks < NB - 1
    __shared__ __attribute__((aligned(16))) float sTt[kRowsT * PT];
    __shared__ float sAd[NB][B][B + 1];            // diagonal blocks of A
    __shared__ float sTd[NB][B][B + 1];            // diagonal blocks of T
    typedef float v4 __attribute__((ext_vector_type(4)));
    const int32_t ci = blockIdx.x;
    const int h = blockIdx.y;
    int64_t tok0;
    int len;
    if (!gen_chunk(a, ci, tok0, len)) return;
    const int tid = threadIdx.x;
    const int64_t slot = (int64_t)h * a.max_chunks + ci;
    float* A = a.TB + slot * C * C;
    for (int x = tid; x < NB * B * B; x += 256) {
        const int K = x / (B * B), r = (x / B) % B, j = x % B;
        sAd[K][r][j] = A[(B * K + r) * C + B * K + j];
        sTd[K][r][j] = r == j ? 1.f : 0.f;
    }
    __syncthreads();
    // diagonal blocks: thread -> block K = tid / 32, column j, rows of parity g
    {
        const int K = tid / 32, j = tid % B, g = (tid / B) % 2;
        for (int i = 0; i < B - 1; ++i) {
            if (K < NB && j <= i) {
                const float ti = sTd[K][i][j];
                for (int r = i + 1 + ((g - (i + 1)) % 2 + 2) % 2; r < B; r += 2) sTd[K][r][j] -= sAd[K][r][i] * ti;
            }
            __syncthreads();
        }
    }
    // block rows
    const int wave = tid / 64, lane = tid % 64, li = lane % 16, g = lane / 16;
    for (int K = 1; K < NB; ++K) {
        // T_KK's row li, as A fragments for the four steps over k = 4 g' + u
        for (int L = wave; L < K; L += 4) {
            f32x4 x = zero4();
            for (int Mb = L; Mb < K; ++Mb) {
                const v4 av = *reinterpret_cast<const v4*>(A + (B * K + li) * C + B * Mb + 4 * g);
                v4 bv;
                if (Mb == L) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) bv[u] = sTd[L][4 * g + u][li];
                } else {
                    bv = *reinterpret_cast<const v4*>(&sTt[(B * L + li) * PT + B * Mb + 4 * g]);
                }
                x = mma_f32(av.x, bv.x, x);
                x = mma_f32(av.y, bv.y, x);
                x = mma_f32(av.z, bv.z, x);
                x = mma_f32(av.w, bv.w, x);
            }
            // T_KL = -T_KK X: lane (li, g) holds X[4 g + r][li], the B operand
            // of step r (k = 4 g + r) of the 16-deep product
            f32x4 y = zero4();
#pragma unroll
            for (int u = 0; u < 4; ++u) y = mma_f32(sTd[K][li][4 * g + u], x[u], y);
            *reinterpret_cast<v4*>(&sTt[(B * L + li) * PT + B * K + 4 * g]) = -y;
        }
        __syncthreads();   // block row K of T is final
    }
    // T diag(beta) over A (A is not read any more), its lower blocks only:
    // the recurrences' products stop at the diagonal block
    for (int x = tid; x < C * C; x += 256) {
        const int rr = x / C, jj = x % C;
        if (jj / B > rr / B) continue;
        const float bj = jj < len ? ldf<E>(a.beta, (tok0 + jj) * a.H + h) : 0.f;
        const float t = jj / B == rr / B ? sTd[rr / B][rr % B][jj % B] : sTt[jj * PT + rr];
        A[x] = t * bj;
    }
}

// ------------------------------------------------------------------ kg_recur
// One workgroup per (sequence, head, 16 value columns), sequential over the
// sequence's 128-token chunks, on fp32 matrix cores: every product is a set
// of 16 x 16 output tiles from 16x16x4 fp32 MFMA steps, wave w taking token
// tile w (X, P, Y, U~, O) and channel tile w (the state update).  A chunk's
// operands do not fit in LDS together, so they pass through two buffers in
// three rounds (K.e^b and Q.e^b; T diag(beta) and M; (K.e^{b_L-b})^T), each
// fetched into registers one phase before it is written to LDS.  As in
// kg_recur_res, the B operands (S, Y, U~) are kept column-major, so that a
// lane's fragments for four MFMA steps are one 16-byte LDS read each.
template <typename E>
__global__ __launch_bounds__(kGenRecurThreads) void kg_recur(GenArgs a) {
    constexpr int NT = kGenRecurThreads;
    constexpr int PO = kGenMaxD + 4;   // pitch of the staged operands and of S^T, Y^T, U~^T (kGenMaxC == kGenMaxD)
    constexpr int W = kGenCols;
    static_assert(kGenMaxC == kGenMaxD && NT == 64 * kGenMaxC / 16, "one token tile and one channel tile per wave");
    __shared__ __attribute__((aligned(16))) float bufA[kGenMaxC * PO];   // K.e^b, then T diag(beta), then (K.e^{b_L-b})^T
    __shared__ __attribute__((aligned(16))) float bufB[kGenMaxC * PO];   // Q.e^b, then M
    __shared__ __attribute__((aligned(16))) float sSt[W * PO];           // S^T   [column][channel]
    __shared__ __attribute__((aligned(16))) float sYt[W * PO];           // Y^T   [column][token]
    __shared__ __attribute__((aligned(16))) float sUt[W * PO];           // U~^T  [column][token]
    const int C = a.C, DK = a.DK, DV = a.DV, tid = threadIdx.x;
    const int slabs = DV / W;
    int32_t n;
    int h, col0;
    gen_slab(a, slabs, n, h, col0);
    const int wave = tid / 64, lane = tid % 64, li = lane % 16, g = lane / 16;
    const bool tw = 16 * wave < C, sw = 16 * wave < DK;   // this wave's token tile / channel tile exists
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
    for (int x = tid; x < DK * W; x += NT) {
        const int c = x / W, jj = x % W;
        sSt[jj * PO + c] = a.S0 ? a.S0[sbase + (int64_t)c * DV + col0 + jj] : 0.f;
    }
    const int64_t vrs = (int64_t)a.H * DV;
    // An R x K fp32 matrix (row-major, K a multiple of 4) is staged in two
    // halves: `fetch` issues its 16-byte loads into registers, `put` writes
    // them to dst as rows (transposed = false) or as columns (dst[k][r]).
    constexpr int kMaxV = kGenMaxC * kGenMaxD / 4 / NT;
    typedef float v4 __attribute__((ext_vector_type(4)));
    struct Fetched {
        v4 f[kMaxV];
    };
    auto fetch = [&](Fetched& pr, const float* src, int R, int K) __attribute__((always_inline)) {
        const int n4 = R * (K / 4);
#pragma unroll
        for (int u = 0; u < kMaxV; ++u) {
            const int x = tid + NT * u;
            pr.f[u] = reinterpret_cast<const v4*>(src)[x < n4 ? x : n4 - 1];
        }
    };
    auto put = [&](float* dst, const Fetched& pr, int R, int K, bool transposed) __attribute__((always_inline)) {
        const int kv = K / 4, n4 = R * kv;
#pragma unroll
        for (int u = 0; u < kMaxV; ++u) {
            const int x = tid + NT * u;
            if (x >= n4) continue;
            const int r = x / kv, c4 = 4 * (x % kv);
            if (transposed) {
                dst[(c4 + 0) * PO + r] = pr.f[u].x;
                dst[(c4 + 1) * PO + r] = pr.f[u].y;
                dst[(c4 + 2) * PO + r] = pr.f[u].z;
                dst[(c4 + 3) * PO + r] = pr.f[u].w;
            } else {
                *reinterpret_cast<v4*>(&dst[r * PO + c4]) = pr.f[u];
            }
        }
    };
    // acc += A B over kend (a multiple of 16) contraction indices, with A's
    // row li of this tile at `arow` and B's column li at `bcol`
    auto tile_mma = [&](const float* arow, const float* bcol, int kend, f32x4 acc) __attribute__((always_inline)) {
        for (int k0 = 0; k0 < kend; k0 += 16) {
            const v4 av = *reinterpret_cast<const v4*>(arow + k0 + 4 * g);
            const v4 bv = *reinterpret_cast<const v4*>(bcol + k0 + 4 * g);
            acc = mma_f32(av.x, bv.x, acc);
            acc = mma_f32(av.y, bv.y, acc);
            acc = mma_f32(av.z, bv.z, acc);
            acc = mma_f32(av.w, bv.w, acc);
        }
        return acc;
    };
    Fetched fa, fb;
    if (nch > 0) {
        const int64_t slot0 = (int64_t)h * a.max_chunks + c0;
        fetch(fa, a.Kg + slot0 * C * DK, C, DK);
        fetch(fb, a.Qg + slot0 * C * DK, C, DK);
        put(bufA, fa, C, DK, false);
        put(bufB, fb, C, DK, false);
    }
    const int T = wave;
    for (int j = 0; j < nch; ++j) {
        const int64_t slot = (int64_t)h * a.max_chunks + c0 + j;
        const int64_t tok0 = s_start + (int64_t)j * C;
        const int len = (int)(s_len - (int64_t)j * C < C ? s_len - (int64_t)j * C : C);
        __syncthreads();   // K.e^b, Q.e^b and the state are in LDS
        // this step's T diag(beta), M, value rows and e^{b_L}, ahead of use
        fetch(fa, a.TB + slot * C * C, C, C);
        fetch(fb, a.M + slot * C * C, C, C);
        float vr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * T + 4 * g + r;
            vr[r] = ldf<E>(a.v, (tok0 + (t < len ? t : 0)) * vrs + (int64_t)h * DV + col0 + li);
        }
        const v4 gm = *reinterpret_cast<const v4*>(a.gam + slot * DK + (sw ? 16 * wave + 4 * g : 0));
        // X = (K.e^b) S, P = (Q.e^b) S for token tile T; Y = V - X to LDS
        f32x4 accX = zero4(), accP = zero4();
        if (tw) {
            const float* ax = bufA + (16 * T + li) * PO;
            const float* ap = bufB + (16 * T + li) * PO;
            const float* bs = sSt + li * PO;
            for (int k0 = 0; k0 < DK; k0 += 16) {
                const v4 xv = *reinterpret_cast<const v4*>(ax + k0 + 4 * g);
                const v4 pv = *reinterpret_cast<const v4*>(ap + k0 + 4 * g);
                const v4 sv = *reinterpret_cast<const v4*>(bs + k0 + 4 * g);
                accX = mma_f32(xv.x, sv.x, accX);
                accP = mma_f32(pv.x, sv.x, accP);
                accX = mma_f32(xv.y, sv.y, accX);
                accP = mma_f32(pv.y, sv.y, accP);
                accX = mma_f32(xv.z, sv.z, accX);
                accP = mma_f32(pv.z, sv.z, accP);
                accX = mma_f32(xv.w, sv.w, accX);
                accP = mma_f32(pv.w, sv.w, accP);
            }
            v4 y;
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = 16 * T + 4 * g + r < len ? vr[r] - accX[r] : 0.f;
            *reinterpret_cast<v4*>(&sYt[li * PO + 16 * T + 4 * g]) = y;
        }
        __syncthreads();   // K.e^b and Q.e^b are dead
        put(bufA, fa, C, C, false);
        put(bufB, fb, C, C, false);
        __syncthreads();
        fetch(fa, a.Kh + slot * C * DK, C, DK);
        // U~ = T diag(beta) Y for tile T (lower triangular: k < 16 (T + 1))
        if (tw) {
            const f32x4 u = tile_mma(bufA + (16 * T + li) * PO, sYt + li * PO, 16 * (T + 1), zero4());
            *reinterpret_cast<v4*>(&sUt[li * PO + 16 * T + 4 * g]) = u;
        }
        __syncthreads();   // U~ is in LDS; T diag(beta) is dead
        put(bufA, fa, C, DK, true);
        if (j + 1 < nch) {   // the next chunk's K.e^b and Q.e^b, put after the state update
            fetch(fa, a.Kg + (slot + 1) * C * DK, C, DK);
            fetch(fb, a.Qg + (slot + 1) * C * DK, C, DK);
        }
        // O = P + M U~ for tile T
        if (tw) {
            accP = tile_mma(bufB + (16 * T + li) * PO, sUt + li * PO, 16 * (T + 1), accP);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * T + 4 * g + r;
                if (t < len) static_cast<E*>(a.o)[(tok0 + t) * vrs + (int64_t)h * DV + col0 + li] = from_f<E>(accP[r]);
            }
        }
        __syncthreads();   // (K.e^{b_L-b})^T is in LDS
        // S <- Diag(e^{b_L}) S + (K.e^{b_L-b})^T U~ for channels 16 wave ..
        f32x4 ns = zero4();
        if (sw) {
            const v4 s0 = *reinterpret_cast<const v4*>(&sSt[li * PO + 16 * wave + 4 * g]);
            ns = tile_mma(bufA + (16 * wave + li) * PO, sUt + li * PO, C, gm * s0);
        }
        __syncthreads();   // every read of the old state, of M and of (K.e^{b_L-b})^T is done
        if (sw) *reinterpret_cast<v4*>(&sSt[li * PO + 16 * wave + 4 * g]) = ns;
        if (j + 1 < nch) {
            put(bufA, fa, C, DK, false);
            put(bufB, fb, C, DK, false);
        }
    }
    __syncthreads();
    if (a.S_T)
        for (int x = tid; x < DK * W; x += NT) {
            const int c = x / W, jj = x % W;
            a.S_T[sbase + (int64_t)c * DV + col0 + jj] = sSt[jj * PO + c];
        }
}

// ------------------------------------------------------------------ kg_recur_res
// kg_recur for chunks of at most CM tokens (CM = 16, 32 or 64), on fp32 matrix
// cores.  All five operands of a chunk fit in LDS together: each step issues
// every load of the next chunk (operands, value rows, e^{b_L}) into
// registers right after its first barrier and writes them to LDS after its
// last one, so one round of loads per step overlaps the whole step.
//
// Every product is a set of 16 x 16 fp32 output tiles (16 tokens or key
// channels by the slab's 16 value columns) from 16x16x4 MFMA steps; a lane's
// A and B fragments for four consecutive steps are one 16-byte LDS read each
// (the contraction index of step u is 4 g + u within each 16-wide block, for
// lane group g), so B operands are kept column-major: S^T, Y^T and U~^T as
// [value column][k].  With nT = C / 16 token tiles, wave w < nT forms X and
// then U~ for tile w, wave nT + w forms P and then O for tile w, and wave c
// forms the state update for channels 16c .. 16c + 15.
template <typename E, int CM>
__global__ __launch_bounds__(512) void kg_recur_res(GenArgs a) {
    constexpr int NT = 512;
    constexpr int W = kGenCols;
    constexpr int PD = kGenMaxD + 4;          // [token][channel] and [column][channel] rows
    constexpr int PC = CM + 4;                // [token][token], [channel][token], [column][token] rows
    constexpr int kRowV = CM * kGenMaxD / 4 / NT;        // 16-byte vectors per thread of a [CM][d_k] operand
    constexpr int kTriV = (CM * CM / 4 + NT - 1) / NT;   // ... of a [CM][CM] operand
    static_assert(W == 16 && 2 * CM / 16 <= NT / 64 && kGenMaxD / 16 <= NT / 64, "one tile per wave and phase");
    __shared__ __attribute__((aligned(16))) float sKg[CM * PD];
    __shared__ __attribute__((aligned(16))) float sQg[CM * PD];
    __shared__ __attribute__((aligned(16))) float sKhT[kGenMaxD * PC];
    __shared__ __attribute__((aligned(16))) float sTB[CM * PC];
    __shared__ __attribute__((aligned(16))) float sM[CM * PC];
    __shared__ __attribute__((aligned(16))) float sSt[W * PD];
    __shared__ __attribute__((aligned(16))) float sYt[W * PC];
    __shared__ __attribute__((aligned(16))) float sUt[W * PC];
    __shared__ unsigned sTouch[NT];   // L2 warm-up loads land here, never read
    const int C = a.C, DK = a.DK, DV = a.DV, tid = threadIdx.x;
    const int slabs = DV / W;
    int32_t n;
    int h, col0;
    gen_slab(a, slabs, n, h, col0);
    const int wave = tid / 64, lane = tid % 64, li = lane % 16, g = lane / 16;
    const int nT = C / 16;
    const bool xw = wave < nT, pw = wave >= nT && wave < 2 * nT, sw = wave < DK / 16;
    const int T = xw ? wave : wave - nT;       // token tile of an X / P wave
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
    for (int x = tid; x < DK * W; x += NT) {
        const int c = x / W, jj = x % W;
        sSt[jj * PD + c] = a.S0 ? a.S0[sbase + (int64_t)c * DV + col0 + jj] : 0.f;
    }
    const int64_t vrs = (int64_t)a.H * DV;
    // the next chunk's loads, in registers between fetch and put
    typedef float v4 __attribute__((ext_vector_type(4)));
    v4 nKg[kRowV], nQg[kRowV], nKh[kRowV], nTB[kTriV], nM[kTriV], ng;
    E nv[4];          // raw: converting at the load would make the compiler wait for it there
    int nlen = 0;
    auto fetch = [&](int j) __attribute__((always_inline)) {
        const int64_t slot = (int64_t)h * a.max_chunks + c0 + j;
        const int64_t tok0 = s_start + (int64_t)j * C;
        const int len = (int)(s_len - (int64_t)j * C < C ? s_len - (int64_t)j * C : C);
        const int nr = C * DK / 4, nt = C * C / 4;
        const v4* kg = reinterpret_cast<const v4*>(a.Kg + slot * C * DK);
        const v4* qg = reinterpret_cast<const v4*>(a.Qg + slot * C * DK);
        const v4* kh = reinterpret_cast<const v4*>(a.Kh + slot * C * DK);
        const v4* tb = reinterpret_cast<const v4*>(a.TB + slot * C * C);
        const v4* mm = reinterpret_cast<const v4*>(a.M + slot * C * C);
        // unconditional loads (past the operand's end, its last vector again):
        // loads under a condition get moved to their uses
#pragma unroll
        for (int u = 0; u < kRowV; ++u) {
            const int x = tid + NT * u < nr ? tid + NT * u : nr - 1;
            nKg[u] = kg[x];
            nQg[u] = qg[x];
            nKh[u] = kh[x];
        }
#pragma unroll
        for (int u = 0; u < kTriV; ++u) {
            const int x = tid + NT * u < nt ? tid + NT * u : nt - 1;
            nTB[u] = tb[x];
            nM[u] = mm[x];
        }
        // an X wave's value rows 16 T + 4 g + r, column li (row 0 of the
        // chunk stands in for rows past its end: loaded, masked when used)
        nlen = len;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * T + 4 * g + r;
            nv[r] = static_cast<const E*>(a.v)[(tok0 + (t < len ? t : 0)) * vrs + (int64_t)h * DV + col0 + li];
        }
        ng = *reinterpret_cast<const v4*>(a.gam + slot * DK + (sw ? 16 * wave + 4 * g : 0));
    };
    auto put = [&]() __attribute__((always_inline)) {
        const int kv = DK / 4, nr = C * kv, tv = C / 4, nt = C * tv;
#pragma unroll
        for (int u = 0; u < kRowV; ++u) {
            const int x = tid + NT * u;
            if (x >= nr) continue;
            const int r = x / kv, c4 = 4 * (x % kv);
            *reinterpret_cast<v4*>(&sKg[r * PD + c4]) = nKg[u];
            *reinterpret_cast<v4*>(&sQg[r * PD + c4]) = nQg[u];
            sKhT[(c4 + 0) * PC + r] = nKh[u].x;
            sKhT[(c4 + 1) * PC + r] = nKh[u].y;
            sKhT[(c4 + 2) * PC + r] = nKh[u].z;
            sKhT[(c4 + 3) * PC + r] = nKh[u].w;
        }
#pragma unroll
        for (int u = 0; u < kTriV; ++u) {
            const int x = tid + NT * u;
            if (x >= nt) continue;
            const int r = x / tv, c4 = 4 * (x % tv);
            *reinterpret_cast<v4*>(&sTB[r * PC + c4]) = nTB[u];
            *reinterpret_cast<v4*>(&sM[r * PC + c4]) = nM[u];
        }
        // Every load of the fetch has landed by now; saying so here keeps the
        // compiler from waiting for the next fetch's fresh loads when it
        // reuses these registers (it cannot tell that the loads and their
        // uses above are under the same conditions).
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    };
    // L2 warm-up: one dword of every 128-byte line of the operands of the
    // chunk kAhead steps ahead, the slabs of a head taking every slabs-th
    // line each, so that the fetch of that chunk finds its lines in the L2
    // the slabs share instead of each waiting on HBM.  Direct loads into a
    // never-read LDS array: no register waits on them; they are older than
    // the next fetch's loads, so the wait at the end of the next put (loads
    // complete in order) covers them.
    constexpr int kAhead = 3;
    const int lines_k = C * DK / 32, lines_t = C * C / 32;   // 128-byte lines per operand
    const int n_lines = 3 * lines_k + 2 * lines_t;
    const int my_line = col0 / W + slabs * tid;   // this thread's line, if below n_lines
    auto touch = [&](int j) __attribute__((always_inline)) {
        if (my_line >= n_lines) return;
        const int64_t slot = (int64_t)h * a.max_chunks + c0 + j;
        int l = my_line;
        const float* base;
        if (l < lines_k) base = a.Kg + slot * C * DK;
        else if ((l -= lines_k) < lines_k) base = a.Qg + slot * C * DK;
        else if ((l -= lines_k) < lines_k) base = a.Kh + slot * C * DK;
        else if ((l -= lines_k) < lines_t) base = a.TB + slot * C * C;
        else {
            l -= lines_t;
            base = a.M + slot * C * C;
        }
        __builtin_amdgcn_global_load_lds(base + 32 * l, (__attribute__((address_space(3))) void*)(sTouch + 64 * wave), 4,
                                         0, 0);
    };
    // acc += A B over kend (a multiple of 16) contraction indices, with A's
    // row li of this tile at `arow` and B's column li at `bcol`, both
    // contiguous in the contraction index
    auto tile_mma = [&](const float* arow, const float* bcol, int kend, f32x4 acc) __attribute__((always_inline)) {
        for (int k0 = 0; k0 < kend; k0 += 16) {
            const v4 av = *reinterpret_cast<const v4*>(arow + k0 + 4 * g);
            const v4 bv = *reinterpret_cast<const v4*>(bcol + k0 + 4 * g);
            acc = mma_f32(av.x, bv.x, acc);
            acc = mma_f32(av.y, bv.y, acc);
            acc = mma_f32(av.z, bv.z, acc);
            acc = mma_f32(av.w, bv.w, acc);
        }
        return acc;
    };
    float vr[4] = {0.f, 0.f, 0.f, 0.f};
    v4 gm = {0.f, 0.f, 0.f, 0.f};
    auto take = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 4; ++r) vr[r] = 16 * T + 4 * g + r < nlen ? to_f(nv[r]) : 0.f;
        gm = ng;
    };
    if (nch > 0) {
        for (int jt = 1; jt < kAhead && jt < nch; ++jt) touch(jt);
        fetch(0);
        put();
        take();
    }
    for (int j = 0; j < nch; ++j) {
        const int64_t tok0 = s_start + (int64_t)j * C;
        const int len = (int)(s_len - (int64_t)j * C < C ? s_len - (int64_t)j * C : C);
        __syncthreads();   // chunk j's operands and the state are in LDS
        // the next chunk's loads (the last step loads its own chunk again,
        // unused: with the fetch and the put unconditional, the compiler
        // sees every load consumed before the next fetch reuses its
        // registers, and does not wait on the fresh loads at their issue)
        fetch(j + 1 < nch ? j + 1 : j);
        // X = (K.e^b) S (X waves; Y = V - X to LDS as Y^T), P = (Q.e^b) S (P waves)
        f32x4 acc = zero4();
        if (xw || pw) acc = tile_mma((xw ? sKg : sQg) + (16 * T + li) * PD, sSt + li * PD, DK, acc);
        if (xw) {
            v4 y;
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = 16 * T + 4 * g + r < len ? vr[r] - acc[r] : 0.f;
            *reinterpret_cast<v4*>(&sYt[li * PC + 16 * T + 4 * g]) = y;
        }
        __syncthreads();
        // U~ = T diag(beta) Y for tile T (lower triangular: k < 16 (T + 1))
        if (xw) {
            const f32x4 u = tile_mma(sTB + (16 * T + li) * PC, sYt + li * PC, 16 * (T + 1), zero4());
            *reinterpret_cast<v4*>(&sUt[li * PC + 16 * T + 4 * g]) = u;
        }
        __syncthreads();
        // O = P + M U~ for tile T
        if (pw) {
            acc = tile_mma(sM + (16 * T + li) * PC, sUt + li * PC, 16 * (T + 1), acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * T + 4 * g + r;
                if (t < len) static_cast<E*>(a.o)[(tok0 + t) * vrs + (int64_t)h * DV + col0 + li] = from_f<E>(acc[r]);
            }
        }
        // S <- Diag(e^{b_L}) S + (K.e^{b_L-b})^T U~ for channels 16 wave ..
        f32x4 ns = zero4();
        if (sw) {
            const v4 s0 = *reinterpret_cast<const v4*>(&sSt[li * PD + 16 * wave + 4 * g]);
            ns = tile_mma(sKhT + (16 * wave + li) * PC, sUt + li * PC, C, gm * s0);
        }
        __syncthreads();   // every read of chunk j's operands and of the old state is done
        if (sw) *reinterpret_cast<v4*>(&sSt[li * PD + 16 * wave + 4 * g]) = ns;
        put();
        take();
        if (j + kAhead < nch) touch(j + kAhead);
    }
    __syncthreads();
    if (a.S_T)
        for (int x = tid; x < DK * W; x += NT) {
            const int c = x / W, jj = x % W;
            a.S_T[sbase + (int64_t)c * DV + col0 + jj] = sSt[jj * PD + c];
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
        const dim3 sgrid(p.max_chunks, p.n_heads);
        switch (p.chunk) {
            case 16:
                hipLaunchKernelGGL((kg_gram<E, 16, 256>), sgrid, dim3(256), 0, st, a);
                hipLaunchKernelGGL((kg_solve<E, 16>), sgrid, dim3(256), 0, st, a);
                break;
            case 32:
                hipLaunchKernelGGL((kg_gram<E, 32, 256>), sgrid, dim3(256), 0, st, a);
                hipLaunchKernelGGL((kg_solve<E, 32>), sgrid, dim3(256), 0, st, a);
                break;
            case 64:
                hipLaunchKernelGGL((kg_gram<E, 64, 512>), sgrid, dim3(512), 0, st, a);
                hipLaunchKernelGGL((kg_solve<E, 64>), sgrid, dim3(256), 0, st, a);
                break;
            default:
                hipLaunchKernelGGL((kg_gram<E, 128, 512>), sgrid, dim3(512), 0, st, a);
                hipLaunchKernelGGL((kg_solve<E, 128>), sgrid, dim3(256), 0, st, a);
                break;
        }
    }
    mark(2);
    const dim3 rgrid(p.n_seqs * p.n_heads * (p.d_v / kGenCols));
    if (p.chunk <= 16)
        hipLaunchKernelGGL((kg_recur_res<E, 16>), rgrid, dim3(512), 0, st, a);
    else if (p.chunk <= 32)
        hipLaunchKernelGGL((kg_recur_res<E, 32>), rgrid, dim3(512), 0, st, a);
    else if (p.chunk <= 64)
        hipLaunchKernelGGL((kg_recur_res<E, 64>), rgrid, dim3(512), 0, st, a);
    else
        hipLaunchKernelGGL(kg_recur<E>, rgrid, dim3(kGenRecurThreads), 0, st, a);
    mark(3);
    return hipGetLastError();
}

hipError_t launch_generic(const Plan& p, hipStream_t st, hipEvent_t* ev) {
    if ((p.chunk != 16 && p.chunk != 32 && p.chunk != 64 && p.chunk != 128) || (p.d_k != 64 && p.d_k != 128) ||
        (p.d_v != 64 && p.d_v != 128))
        return hipErrorInvalidValue;
    return p.bf16 ? launch_gen<__bf16>(p, st, ev) : launch_gen<float>(p, st, ev);
}

}  // namespace kda
