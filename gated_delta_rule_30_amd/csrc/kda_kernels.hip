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
//   M[r,i]   = sum_c q_rc k_ic exp(b_rc - b_ic)             (i <= r)
//   U~ = T diag(beta) (V - (K . Gamma) S)        written deltas of the chunk
//   O  = (Q . Gamma) S + M U~
//   S' = Diag(Gamma_L) S + (K . exp(b_L - b))^T U~
//
// Sub-tiling (orkas.ai "Kimi K3 architecture", §"GPU のコードパスを一本消した
// 「下界」"): with g >= -5, b falls by at most 80 inside a 16-token sub-tile.
// For row sub-tile R let rho_R = b at the end of sub-tile R-1 (0 at the chunk
// start).  The diagonal block (R, R) of A and M is the product of
//   row operand    x_r . exp(b_r - rho_R)      factor in [e^-80, 1]
//   column operand k_i . exp(rho_R - b_i)      factor in [1, e^80]
// and an off-diagonal block (R, J < R) of
//   row operand    x_r . exp(b_r - rho_R)
//   column operand k_i . exp(rho_{J+1} - b_i) . exp(rho_R - rho_{J+1})   factors <= 1
// All factors stay inside bf16 range, so every block -- the diagonal ones
// included -- is one dense MFMA contraction over d_k.
//
// Launches (all on the caller's stream):
//   k_chunk_table : chunk list from cu_seqlens (device side, no host sync)
//   k_prep        : per (chunk, head), chunk-parallel: decay cumsum, A and M
//                   by sub-tiled MFMA, T = (I + A)^-1 in LDS (fp32); writes
//                   the chunk's operands Q . Gamma, K . Gamma,
//                   (K . exp(b_L - b))^T, T diag(beta), M and Gamma_L
//   k_recur_lds   : (bf16) per (sequence, head, slab of 16 or 32 columns of
//   / k_recur       S), sequential over the chunks: the state step and the
//                   chunk output from those operands (fp32 at d = 64: k_recur)
//
// Lane geometry shared by both kernels.  Wave w of a 256-thread workgroup
// owns token rows 16w .. 16w+15 of the chunk; lane = 16 * lg + li holds token
// 16w + li and the contiguous key-channel range [lg * D/4, (lg+1) * D/4).
// That is exactly the A-operand fragment of the 16-row tile w for a
// contraction over channels (k-step m covers channels lg*D/4 + m*KW + j), and
// also the B-operand fragment of column block w, so the diagonal sub-tile
// products need no data exchange.  The per-channel cumulative sum over
// tokens is a 16-lane row scan (DPP row shifts) plus carries between waves.
#include <atomic>
#include <mutex>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// ---------------------------------------------------------------- sequences
// Token range [start, start + len) of sequence n.  Device-side offsets are
// clamped to [0, total_tokens) so that malformed cu_seqlens can never address
// outside the tensors.
__device__ inline void seq_range(const int32_t* __restrict__ cu, int32_t n, int64_t total_tokens,
                                 int64_t fixed_len, int64_t& start, int64_t& len) {
    if (cu) {
        int64_t a = cu[n], e = cu[n + 1];
        a = a < 0 ? 0 : (a > total_tokens ? total_tokens : a);
        e = e < a ? a : (e > total_tokens ? total_tokens : e);
        start = a;
        len = e - a;
    } else {
        start = (int64_t)n * fixed_len;
        len = fixed_len;
    }
}

// Chunks c0 .. c0 + nch - 1 of sequence n of length s_len.  Equal lengths
// (cu == NULL) list sequence n's chunks from n * ceil(len / 64) on, which is
// what the chunk table holds for them, so no table is read; otherwise the
// table's first chunk of each sequence, clamped to its slots.
__device__ inline void seq_chunks(const int32_t* __restrict__ cu, const int32_t* __restrict__ seq_chunk0, int32_t n,
                                  int64_t fixed_len, int64_t s_len, int32_t& c0, int32_t& nch) {
    nch = (int32_t)((s_len + kChunk - 1) / kChunk);
    if (!cu) {
        c0 = n * (int32_t)((fixed_len + kChunk - 1) / kChunk);
        return;
    }
    c0 = seq_chunk0[n];
    if (nch > seq_chunk0[n + 1] - c0) nch = seq_chunk0[n + 1] - c0;
}

// ---------------------------------------------------------------- chunk table
// One workgroup.  Sequence n contributes ceil(len_n / C) chunks; chunks are
// aligned to each sequence's first token and the last one may be partial.
// Sequences are taken 1024 at a time: a prefix sum of their chunk counts
// gives each one's first chunk, then the whole workgroup writes the batch's
// chunk records, finding each chunk's sequence by binary search in the sums.
//
// With every > 0 it also writes ck0[n] = sum over m < n of floor(chunks_m /
// every), the first state-checkpoint slot of each sequence (ck0[n_seqs] is
// the total).
__global__ __launch_bounds__(1024) void k_chunk_table(const int32_t* __restrict__ cu, int32_t n_seqs,
                                                      int64_t total_tokens, int64_t fixed_len,
                                                      int32_t max_chunks, ChunkInfo* __restrict__ tab,
                                                      int32_t* __restrict__ seq_chunk0,
                                                      int32_t* __restrict__ n_chunks_out, int32_t every,
                                                      int32_t* __restrict__ ck0, int32_t C) {
    __shared__ int32_t s_scan[1024];     // inclusive prefix sum of chunk counts in the batch
    __shared__ int32_t s_ck[1024];       // the same for checkpoint counts (every > 0)
    __shared__ int64_t s_start[1024];
    __shared__ int64_t s_len[1024];
    __shared__ int32_t s_carry, s_ck_carry;
    const int tid = threadIdx.x;
    if (tid == 0) {
        s_carry = 0;
        s_ck_carry = 0;
    }
    __syncthreads();
    for (int32_t base = 0; base < n_seqs; base += 1024) {
        const int32_t n = base + tid;
        int64_t start = 0, len = 0;
        if (n < n_seqs) seq_range(cu, n, total_tokens, fixed_len, start, len);
        const int32_t cnt = (int32_t)((len + C - 1) / C);
        const int32_t ckc = every > 0 ? cnt / every : 0;
        s_scan[tid] = cnt;
        s_ck[tid] = ckc;
        s_start[tid] = start;
        s_len[tid] = len;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            const int32_t add = tid >= off ? s_scan[tid - off] : 0;
            const int32_t add_ck = tid >= off ? s_ck[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += add;
            s_ck[tid] += add_ck;
            __syncthreads();
        }
        const int32_t carry = s_carry;
        if (n < n_seqs) {
            const int32_t first = carry + s_scan[tid] - cnt;
            seq_chunk0[n] = first < max_chunks ? first : max_chunks;
            if (every > 0) ck0[n] = s_ck_carry + s_ck[tid] - ckc;
        }
        const int32_t batch = s_scan[1023];
        for (int32_t c = tid; c < batch; c += 1024) {
            const int32_t cg = carry + c;
            if (cg >= max_chunks) break;
            int lo = 0, hi = 1023;   // first i with s_scan[i] > c
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (s_scan[mid] > c) hi = mid; else lo = mid + 1;
            }
            const int32_t j = c - (lo > 0 ? s_scan[lo - 1] : 0);
            ChunkInfo ci;
            ci.tok0 = s_start[lo] + (int64_t)j * C;
            ci.seq = base + lo;
            const int64_t rem = s_len[lo] - (int64_t)j * C;
            ci.len = (int32_t)(rem < C ? rem : C);
            tab[cg] = ci;
        }
        __syncthreads();
        if (tid == 1023) {
            s_carry = carry + batch;
            s_ck_carry += s_ck[1023];
        }
        __syncthreads();
    }
    if (tid == 0) {
        const int32_t total = s_carry < max_chunks ? s_carry : max_chunks;
        seq_chunk0[n_seqs] = total;
        *n_chunks_out = total;
        if (every > 0) ck0[n_seqs] = s_ck_carry;
    }
}

// ---------------------------------------------------------------- shared stages
template <typename E, int D>
struct Geo {
    using M = Mma<E>;
    static constexpr int CPL = D / 4;                 // key channels per lane
    static constexpr int NKC = D / M::KS;             // k-steps of a contraction over channels
    static constexpr int EPV = 16 / (int)sizeof(E);   // elements per 16-byte vector
    static constexpr int VPL = CPL / EPV;             // 16-byte vectors per lane per row
    static constexpr int NKT = kChunk / M::KS;        // k-steps of a contraction over the chunk's tokens
    static constexpr int NVT = kChunk / 4 / EPV;      // 16-byte vectors per lane of a token contraction
    // chunk token of lane-element i (k-step order) for lane group lg
    __device__ static inline int tok_of(int i, int lg) { return M::KS * (i / M::KW) + M::KW * lg + i % M::KW; }
};

// One token row slice (this lane's channels) of a [T, H, D] tensor, as raw
// 16-byte vectors.  The load is unconditional (callers pass an address inside
// the tensor); rows past the chunk end read as zero through get().  Keeping
// the load free of branches lets prefetched loads stay in flight.
template <typename E, int D>
struct RowSlice {
    uint4 v[Geo<E, D>::VPL];
    bool ok;
    __device__ inline void load(const E* __restrict__ p, bool valid) {
        ok = valid;
#pragma unroll
        for (int i = 0; i < Geo<E, D>::VPL; ++i) v[i] = reinterpret_cast<const uint4*>(p)[i];
    }
    __device__ inline float get(int j) const {
        const E* e = reinterpret_cast<const E*>(v);
        return ok ? to_f(e[j]) : 0.f;
    }
};

// Chunk operands written by k_prep for k_recur, stored head-major: the
// operands of chunk ci of head h sit at slot h * max_chunks + ci, so one
// head's chunks are contiguous and the sequential kernel streams through
// memory.  Per slot (operand dtype E unless stated):
//   TB  64 x 64    T diag(beta), upper sub-tile blocks zero
//   Mm  64 x 64    M (decayed causal Q K^T incl. diagonal), upper blocks zero
//   Qg  64 x D     Q . Gamma
//   Kg  64 x D     K . Gamma
//   KhT D x 64     (K . exp(b_L - b))^T
//   gam [D] fp32   Gamma_L = exp(b_L)
// The matrices are stored fragment-major: each is a sequence of 16-row
// A-operand tiles, and a tile is [NV][64 lanes][16 bytes], where lane
// 16 * lg + li holds row li's contraction elements in k-step order (over
// channels: lg*D/4 + i; over the chunk's tokens: KS*(i/KW) + KW*lg + i%KW).
// One wave then loads a fragment vector as 1 KB of contiguous memory.
//
// The backward pass reuses the same five buffers for the transposed set its
// state-gradient recurrence needs (k_prep with kBwd):
//   TB  <- T^T                 Mm  <- M^T               Qg  <- K . exp(b_L - b)
//   Kg  <- (Q . Gamma)^T       KhT <- (K . Gamma)^T      gam (unchanged)
//   bet [64] fp32 beta of the chunk's tokens (0 past the end)
struct ChunkOps {
    void *TB, *Mm, *Qg, *Kg, *KhT;
    float* gam;
    int64_t max_chunks;   // slots per head
    float* bet;           // backward set only
};

// ---------------------------------------------------------------- k_prep
// One workgroup per (chunk, head), chunk-parallel.
//
// Decay factors.  With rho_w = b at the end of sub-tile w-1 and x = b - rho_w
// in [-80, 0] for the tokens of sub-tile w, every factor is a product of
// exponentials of bounded arguments:
//   exp(b)               = exp(rho_w) . exp(x)
//   exp(rho_{w+1} - b)   = exp(rho_{w+1} - rho_w) . exp(-x)
//   exp(rho_w - rho_{J+1}) = prod_{R=J+1}^{w-1} exp(rho_{R+1} - rho_R)
// The per-channel factors are computed once per chunk; per element only
// exp(x), exp(-x) and exp(b_L - b) remain.
//
// kBoth also writes the backward set of operands (see ChunkOps) into `ob`
// from the same quantities: K . exp(b_L - b) row-wise, (K . Gamma)^T and
// (Q . Gamma)^T through the transposing LDS stages, T^T and M^T, and beta
// (Gamma_L is shared: ob.gam is ops.gam).  kLean (with kBoth) leaves out Q .
// Gamma and M of the forward set: the backward pass that evaluates the
// forward again never reads them.
template <typename E, int D, bool kBoth = false, bool kLean = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(!kBoth && sizeof(E) == 2 ? 3 : 1))) void k_prep(const E* __restrict__ q, const E* __restrict__ k,
                                                   const E* __restrict__ g, const E* __restrict__ beta,
                                                   const ChunkInfo* __restrict__ tab,
                                                   const int32_t* __restrict__ n_chunks_p, int64_t fixed_len,
                                                   int32_t fixed_chunks, int32_t H, ChunkOps ops, ChunkOps ob,
                                                   int32_t blk_j0, int32_t blk_nj, int32_t xcd_hi) {
    constexpr bool kBwd = kBoth;
    using G = Geo<E, D>;
    using M = Mma<E>;
    constexpr int C = kChunk, CPL = G::CPL, EPV = G::EPV;
    constexpr int PC = D + 8;      // row pitch of the column-operand tiles
    constexpr int PM = C + 8;      // row pitch of the M staging tile (elements)
    constexpr int PK = C + 8;      // row pitch of the K^T staging tile (elements)
    // A and T are unit / strictly lower block-triangular: only their ten
    // 16 x 16 blocks (R, J <= R) are stored, block (R, J) at slot
    // R (R + 1) / 2 + J, rows of BP floats.
    constexpr int BP = kSub + 4;
    constexpr int kBlk = kSub * BP;
    constexpr int kTri = kNSub * (kNSub + 1) / 2 * kBlk;
    // Region 1: A and the T-inverse scratch; before A exists it stages K^T.
    // Region 2: the column bases; after the Gram blocks, T.
    constexpr int kKtBytes = D * PK * (int)sizeof(E);
    constexpr int kR1 = (kKtBytes / 4 > kTri + 4 * 16 * 17 ? kKtBytes / 4 : kTri + 4 * 16 * 17);
    constexpr int kColBytes = (kNSub - 1) * kSub * PC * (int)sizeof(E);
    constexpr int kR2 = (kColBytes / 4 > kTri ? kColBytes / 4 : kTri);
    __shared__ __attribute__((aligned(16))) float sR1[kR1];
    __shared__ __attribute__((aligned(16))) float sR2[kR2];
    __shared__ float sTot[kNSub * D];         // exp(rho_{R+1} - rho_R)
    __shared__ float sP30[D];                 // exp(rho_3 - rho_1)
    __shared__ float sERho[kNSub * D];        // exp(rho_R)
    __shared__ float sCarry[(kNSub + 1) * D]; // rho_0 .. rho_3, b_L
    __shared__ float sELr[kNSub * D];         // exp(b_L - rho_{R+1})
    __shared__ __attribute__((aligned(16))) E sM[C * PM];
    __shared__ __attribute__((aligned(16))) float sBeta[C];
    __shared__ __attribute__((aligned(16))) E sQt[kBwd ? D * PK : 8];   // (Q . Gamma)^T staging (kBwd)
    static_assert(!kBwd || sizeof(E) == 2, "backward operands: bf16 only");
    float* sA = sR1;
    float* sX = sR1 + kTri;
    E* sKt = reinterpret_cast<E*>(sR1);
    E* sColB = reinterpret_cast<E*>(sR2);
    float* sT = sR2;
    // K^T staging: the token index is rotated by 16 per channel group, so
    // the four lane groups that write one token column hit different banks.
    auto kt_at = [](int ch, int t_) { return ch * PK + ((t_ + kSub * (ch / CPL)) & (C - 1)); };
    // element (row, col) of a lower block-triangular 64 x 64 matrix (col's block <= row's block)
    auto blk = [](int R, int J) { return (R * (R + 1) / 2 + J) * kBlk; };
    auto tri = [&](int row, int col) { return blk(row >> 4, col >> 4) + (row & 15) * BP + (col & 15); };

    // Chunk ci: for equal-length sequences (fixed_len > 0) it follows from
    // the index (fixed_chunks chunks per sequence, in sequence order, as the
    // chunk table lists them); otherwise it is read from the chunk table.
    // With blk_nj > 0 (equal lengths only) the grid covers chunks
    // blk_j0 .. blk_j0 + blk_nj - 1 of every sequence.  With xcd_hi the
    // grid is twice the work (x a multiple of 8): workgroups on XCDs 0..3
    // (id mod 8 < 4) leave at once, so that k_prep runs on XCDs 4..7 only.
    int32_t ci = blockIdx.x;
    if (xcd_hi) {
        if (ci % 8 < 4) return;
        ci = (ci / 8) * 4 + ci % 8 - 4;
    }
    ChunkInfo info;
    if (fixed_len > 0) {
        const int32_t per = (int32_t)((fixed_len + kChunk - 1) / kChunk);
        if (blk_nj > 0) {
            const int32_t jj = blk_j0 + ci % blk_nj;
            if (jj >= per) return;
            ci = (ci / blk_nj) * per + jj;
        }
        if (ci >= fixed_chunks) return;
        const int32_t seq = ci / per, j = ci % per;
        const int64_t rem = fixed_len - (int64_t)j * kChunk;
        info.tok0 = (int64_t)seq * fixed_len + (int64_t)j * kChunk;
        info.seq = seq;
        info.len = (int32_t)(rem < kChunk ? rem : kChunk);
    } else {
        if (ci >= *n_chunks_p) return;
        info = tab[ci];
    }
    const int h = blockIdx.y, len = info.len;
    const int tid = threadIdx.x, w = wave_id(), li = lane_id() & 15, lg = lane_id() >> 4;
    const int tok = kSub * w + li;
    const bool ok = tok < len;
    const int64_t rs = (int64_t)H * D;
    const int64_t off = (info.tok0 * H + h) * D + (int64_t)(ok ? tok : 0) * rs + lg * CPL;
    const int64_t cbase = (int64_t)h * ops.max_chunks + ci;   // head-major operand slot

    RowSlice<E, D> xq, xk, xg;
    xq.load(q + off, ok);
    xk.load(k + off, ok);
    xg.load(g + off, ok);
    const float bet = ok ? to_f(beta[(info.tok0 + tok) * H + h]) : 0.f;
    if (lg == 0) sBeta[tok] = bet;
    if constexpr (kBwd) {
        if (lg == 0) ob.bet[((int64_t)h * ob.max_chunks + ci) * C + tok] = bet;
    }

    // Cumulative log-decay: 16-lane row scan per sub-tile, carries between
    // sub-tiles, and the per-channel factors.
    float b[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) b[j] = row_scan16(xg.get(j));
    if (li == 15) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) sTot[w * D + lg * CPL + j] = b[j];
    }
    __syncthreads();
    for (int c = tid; c < D; c += kThreads) {
        float run = 0.f;
#pragma unroll
        for (int r = 0; r < kNSub; ++r) {
            const float t = sTot[r * D + c];
            sCarry[r * D + c] = run;
            sERho[r * D + c] = __expf(run);
            sTot[r * D + c] = __expf(t);
            run += t;
        }
        sCarry[kNSub * D + c] = run;
#pragma unroll
        for (int r = 0; r < kNSub; ++r) sELr[r * D + c] = __expf(run - sCarry[(r + 1) * D + c]);
        sP30[c] = sTot[1 * D + c] * sTot[2 * D + c];
        ops.gam[cbase * D + c] = __expf(run);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < CPL; ++j) b[j] += sCarry[w * D + lg * CPL + j];

    // Operands: Gram rows scaled by exp(b - rho_w), the diagonal column
    // operand by exp(rho_w - b), the column base for later row blocks by
    // exp(rho_{w+1} - b), and the inter-chunk operands Q . Gamma, K . Gamma,
    // K . exp(b_L - b).
    // The diagonal block (w, w) is accumulated here, as each k-step's
    // operands are formed, so its column operand is never held in full.
    typename M::frag rq[G::NKC], rk[G::NKC];
    f32x4 accAd = zero4(), accMd = zero4();
    {
        const float* rho = sCarry + w * D + lg * CPL;
        const float* erho = sERho + w * D + lg * CPL;
        const float* elr = sELr + w * D + lg * CPL;
        const float* esub = sTot + w * D + lg * CPL;
        uint4* qg = reinterpret_cast<uint4*>(static_cast<E*>(ops.Qg) + cbase * C * D);
        uint4* kg = reinterpret_cast<uint4*>(static_cast<E*>(ops.Kg) + cbase * C * D);
        uint4* kh = reinterpret_cast<uint4*>(static_cast<E*>(ob.Qg) + cbase * C * D);
        uint4* cbv = reinterpret_cast<uint4*>(sColB + (w * kSub + li) * PC + lg * CPL);
        // Q . Gamma, K . Gamma (kBoth: and K . exp(b_L - b)) and the column
        // base are stored one 16-byte vector at a time, as soon as each is
        // complete.
        uint4 vq, vk, vh, vc;
        E* eq = reinterpret_cast<E*>(&vq);
        E* ek = reinterpret_cast<E*>(&vk);
        E* eh = reinterpret_cast<E*>(&vh);
        E* ec = reinterpret_cast<E*>(&vc);
#pragma unroll
        for (int m = 0; m < G::NKC; ++m) {
            typename M::frag cd;
#pragma unroll
            for (int j = 0; j < M::KW; ++j) {
                const int c = m * M::KW + j;
                const float x = b[c] - rho[c];
                const float fr = __expf(x), fd = __expf(-x), gm = erho[c] * fr;
                const float kv = xk.get(c), qv = xq.get(c);
                if constexpr (M::KW == 1) {
                    rq[m] = qv * fr;
                    rk[m] = kv * fr;
                    cd = kv * fd;
                } else {
                    rq[m][j] = from_f<E>(qv * fr);
                    rk[m][j] = from_f<E>(kv * fr);
                    cd[j] = from_f<E>(kv * fd);
                }
                const int cv = c % EPV;   // element within the current 16-byte vector
                // exp(rho_{w+1} - b) <= 1, and exp(b_L - b) is that times exp(b_L - rho_{w+1}) <= 1
                const float ew = esub[c] * fd;
                ec[cv] = from_f<E>(kv * ew);
                const float kh_v = kv * (elr[c] * ew);
                eq[cv] = from_f<E>(qv * gm);
                ek[cv] = from_f<E>(kv * gm);
                sKt[kt_at(lg * CPL + c, tok)] = from_f<E>(kh_v);
                if constexpr (kBwd) {
                    // row-wise K . exp(b_L - b); K . Gamma staged for its transpose
                    eh[cv] = from_f<E>(kh_v);
                    sQt[kt_at(lg * CPL + c, tok)] = ek[cv];
                }
                if (cv == EPV - 1) {
                    const int i = c / EPV;
                    if constexpr (!kLean) store_nt(&qg[(w * G::VPL + i) * 64 + lane_id()], vq);
                    store_nt(&kg[(w * G::VPL + i) * 64 + lane_id()], vk);
                    if constexpr (kBwd) store_nt(&kh[(w * G::VPL + i) * 64 + lane_id()], vh);
                    if (w < kNSub - 1) cbv[i] = vc;
                }
            }
            accAd = M::mma(rk[m], cd, accAd);
            accMd = M::mma(rq[m], cd, accMd);
        }
    }
    __syncthreads();
    // channel rows over the chunk's tokens, fragment-major, from a staged
    // [channel][token] tile.  With bf16 a lane's 8 tokens of one k-step are
    // consecutive (the rotation moves whole groups of 16), so each vector is
    // one 16-byte LDS read; eight lanes of consecutive channels then cover
    // all banks once (row pitch 144 bytes).
    auto store_transposed = [&](const E* st, void* dst) {
        uint4* out = reinterpret_cast<uint4*>(static_cast<E*>(dst) + cbase * D * C);
        for (int vi = tid; vi < D * C / EPV; vi += kThreads) {
            const int ln = vi % 64, v = (vi / 64) % G::NVT, ct = vi / (64 * G::NVT);
            const int r = kSub * ct + (ln & 15), lgp = ln >> 4;
            if constexpr (M::KW == EPV) {
                store_nt(&out[vi], *reinterpret_cast<const uint4*>(st + kt_at(r, G::tok_of(v * EPV, lgp))));
            } else {
                uint4 pk;
                E* pe = reinterpret_cast<E*>(&pk);
#pragma unroll
                for (int e = 0; e < EPV; ++e) pe[e] = st[kt_at(r, G::tok_of(v * EPV + e, lgp))];
                store_nt(&out[vi], pk);
            }
        }
    };
    store_transposed(sKt, ops.KhT);                     // (K . exp(b_L - b))^T
    if constexpr (kBwd) {
        store_transposed(sQt, ob.KhT);                  // (K . Gamma)^T
        __syncthreads();
        // (Q . Gamma)^T through the first stage again
        const float* rho = sCarry + w * D + lg * CPL;
        const float* erho = sERho + w * D + lg * CPL;
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            sKt[kt_at(lg * CPL + c, tok)] = from_f<E>(xq.get(c) * (erho[c] * __expf(b[c] - rho[c])));
        __syncthreads();
        store_transposed(sKt, ob.Kg);
    }
    __syncthreads();

    // Blocks (w, J) for J <= w of A (strict lower, rows scaled by beta) and M
    // (inclusive lower); blocks above the diagonal are never formed.
    for (int J = 0; J <= w; ++J) {
        f32x4 accA = accAd, accM = accMd;
        if (J < w) {
            accA = zero4();
            accM = zero4();
            // column operand: base of block J times exp(rho_w - rho_{J+1})
            // (1 when J = w-1; otherwise a per-channel factor from the table)
            const E* cb = sColB + (J * kSub + li) * PC + lg * CPL;
            const float* pf = (J == w - 2 ? sTot + (w - 1) * D : sP30) + lg * CPL;
            const bool scale = J < w - 1;
#pragma unroll
            for (int m = 0; m < G::NKC; ++m) {
                typename M::frag cf;
                if constexpr (M::KW == 1) {
                    cf = scale ? cb[m] * pf[m] : cb[m];
                } else {
                    cf = M::load(cb + m * M::KW);
                    if (scale) {
#pragma unroll
                        for (int j = 0; j < M::KW; ++j)
                            cf[j] = from_f<E>(to_f(cf[j]) * pf[m * M::KW + j]);
                    }
                }
                accA = M::mma(rk[m], cf, accA);
                accM = M::mma(rq[m], cf, accM);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = kSub * w + 4 * lg + r, col = kSub * J + li;
            sA[tri(row, col)] = (J < w || col < row) ? sBeta[row] * accA[r] : 0.f;
            sM[row * PM + col] = from_f<E>((J < w || col <= row) ? accM[r] : 0.f);
        }
    }
    __syncthreads();   // the column bases are dead from here; region 2 holds T

    // T = (I + A)^-1.  Diagonal 16 x 16 blocks by forward substitution (one
    // column per lane), then the off-diagonal blocks by distance R - J:
    // T_RJ = -T_RR sum_{K=J}^{R-1} A_RK T_KJ  (fp32 MFMA).
    if (lg == 0) {
        const int R = w, jc = li;
        float x[kSub];
#pragma unroll
        for (int r = 0; r < kSub; ++r) {
            float s = (r == jc) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) s -= sA[blk(R, R) + r * BP + i] * x[i];
            x[r] = s;
        }
#pragma unroll
        for (int r = 0; r < kSub; ++r) sT[blk(R, R) + r * BP + jc] = x[r];
    }
    __syncthreads();
    for (int d = 1; d < kNSub; ++d) {
        const bool act = w < kNSub - d;
        const int J = w, R = w + d;
        if (act) {
            f32x4 acc = zero4();
            for (int K = J; K < R; ++K)
#pragma unroll
                for (int kk = 0; kk < kSub; kk += 4)
                    acc = mma_f32(sA[blk(R, K) + li * BP + kk + lg], sT[blk(K, J) + (kk + lg) * BP + li], acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) sX[w * 272 + (4 * lg + r) * 17 + li] = acc[r];
        }
        __syncthreads();
        if (act) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < kSub; kk += 4)
                acc = mma_f32(sT[blk(R, R) + li * BP + kk + lg], sX[w * 272 + (kk + lg) * 17 + li],
                              acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) sT[blk(R, J) + (4 * lg + r) * BP + li] = -acc[r];
        }
        __syncthreads();
    }

    // Stores: T diag(beta) and M (kBoth: also T^T and M^T), fragment-major 16-byte vectors.
    uint4* otb = reinterpret_cast<uint4*>(static_cast<E*>(ops.TB) + cbase * C * C);
    uint4* omm = reinterpret_cast<uint4*>(static_cast<E*>(ops.Mm) + cbase * C * C);
    uint4* ott = reinterpret_cast<uint4*>(static_cast<E*>(ob.TB) + cbase * C * C);
    uint4* omt = reinterpret_cast<uint4*>(static_cast<E*>(ob.Mm) + cbase * C * C);
    for (int vi = tid; vi < C * C / EPV; vi += kThreads) {
        const int ln = vi % 64, v = (vi / 64) % G::NVT, wr = vi / (64 * G::NVT);
        const int r = kSub * wr + (ln & 15), lgp = ln >> 4;
        uint4 pt, pm, ptt, pmt;
        E* et = reinterpret_cast<E*>(&pt);
        E* em = reinterpret_cast<E*>(&pm);
        E* ett = reinterpret_cast<E*>(&ptt);
        E* emt = reinterpret_cast<E*>(&pmt);
        if constexpr (M::KW == EPV) {
            // bf16: the vector's 8 tokens are consecutive and in one 16-token
            // block, so T, beta and M come as whole 16-byte LDS reads
            const int t0 = G::tok_of(v * EPV, lgp);
            const bool upper = (t0 >> 4) > (r >> 4);            // blocks above the diagonal are zero
            const int tc = upper ? ((r >> 4) << 4) | (t0 & 15) : t0;   // an address inside the stored blocks
            const f32x4* tp = reinterpret_cast<const f32x4*>(sT + tri(r, tc));
            const f32x4* bp = reinterpret_cast<const f32x4*>(sBeta + t0);
            const f32x4 t_lo = tp[0], t_hi = tp[1], b_lo = bp[0], b_hi = bp[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                et[e] = from_f<E>(upper ? 0.f : t_lo[e] * b_lo[e]);
                et[e + 4] = from_f<E>(upper ? 0.f : t_hi[e] * b_hi[e]);
            }
            pm = upper ? uint4{0u, 0u, 0u, 0u} : *reinterpret_cast<const uint4*>(sM + r * PM + tc);
        }
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            const int t = G::tok_of(v * EPV + e, lgp);
            if constexpr (M::KW != EPV) {
                const bool upper = (t >> 4) > (r >> 4);   // blocks above the diagonal are zero
                et[e] = from_f<E>(upper ? 0.f : sT[tri(r, upper ? r : t)] * sBeta[t]);
                em[e] = upper ? from_f<E>(0.f) : sM[r * PM + t];
            }
            if constexpr (kBwd) {
                // element (r, t) of a transpose is (t, r): zero unless t's block >= r's
                const bool zero = (t >> 4) < (r >> 4);
                ett[e] = from_f<E>(zero ? 0.f : sT[tri(zero ? r : t, zero ? t : r)]);
                emt[e] = zero ? from_f<E>(0.f) : sM[t * PM + r];
            }
        }
        // bf16: the 32-token halves that are zero by structure (row tiles 0
        // and 1 over tokens 32..63; of the transposes, row tiles 2 and 3 over
        // tokens 0..31) are not stored: the bf16 recurrence never reads them.
        // (The fp32 recurrence reads whole tiles.)  A wave's 64 vectors are
        // one (row tile, half) block, so the skip is wave-uniform.
        constexpr bool kSkipZero = M::KW == EPV && G::NVT == 2;
        if (!(kSkipZero && wr < 2 && v == 1)) {
            store_nt(&otb[vi], pt);
            if constexpr (!kLean) store_nt(&omm[vi], pm);
        }
        if constexpr (kBwd) {
            if (!(kSkipZero && wr >= 2 && v == 0)) {
                store_nt(&ott[vi], ptt);
                store_nt(&omt[vi], pmt);
            }
        }
    }
}

// ---------------------------------------------------------------- k_recur
// Sequential over the chunks of one sequence for one head and one slab of
// 16 * CT value columns (columns of S evolve independently).  Per chunk:
//   X = (K . Gamma) S,  P = (Q . Gamma) S        rows 16w.. of wave w
//   U~ = T diag(beta) (V - X)                    rows 16w..
//   O  = P + M U~                                rows 16w.. -> o
//   S <- Diag(Gamma_L) S + (K . exp(b_L - b))^T U~
// S stays in fp32 registers in accumulator layout: wave w holds key-channel
// tiles RT*w .. RT*w+RT-1 of every column tile.  All chunk operands come
// from k_prep and are prefetched one chunk ahead into registers.
template <typename E, int D, int CT>
struct RecurIn {
    using G = Geo<E, D>;
    using F = typename Mma<E>::frag;
    static constexpr int RT = D / 64;
    uint4 qg[G::VPL], kg[G::VPL];            // A fragments over channels (rows 16w..)
    uint4 kt[RT][G::NVT];                    // A fragments of K^T (channel tiles), over tokens
    uint4 tb[G::NVT], mm[G::NVT];            // A fragments over tokens (rows 16w..)
    f32x4 gam[RT];                           // Gamma_L for this lane's state rows
    E v[CT][4];                              // value entries of rows 16w + 4lg + r (zeroed past the end at use)
    int len;
};

// Base pointers of one (sequence, head, slab) problem; chunk j of the
// sequence is chunk c0 + j of the workspace and starts at token start + 64 j.
template <typename E, int D>
struct RecurPtrs {
    const E *qg, *kg, *kt, *tb, *mm, *v;
    const float* gam;
    int64_t ops_step;     // elements between consecutive chunks of one head (C x D operands)
    int64_t sq_step;      // elements between consecutive chunks of one head (C x C operands)
    int64_t gam_step;     // floats between consecutive chunks of one head
    int64_t tok_step;     // elements between consecutive chunks in [T, H, D] tensors
};

// The operand loads of one chunk, in three groups that k_recur issues at
// three different points of a step, so the memory pipeline drains them in
// the background of the matrix work instead of stalling one burst.
// P.qg / P.kg / P.kt / P.tb / P.mm point at this lane's first 16-byte vector
// of chunk 0; vectors of one lane are 64 vectors apart.
template <typename E, int D, int CT>
__device__ inline void recur_load_a(RecurIn<E, D, CT>& in, const RecurPtrs<E, D>& P, int j) {
    using G = Geo<E, D>;
    const uint4* qg = reinterpret_cast<const uint4*>(P.qg + j * P.ops_step);
    const uint4* kg = reinterpret_cast<const uint4*>(P.kg + j * P.ops_step);
#pragma unroll
    for (int i = 0; i < G::VPL; ++i) {
        in.qg[i] = qg[i * 64];
        in.kg[i] = kg[i * 64];
    }
}

template <typename E, int D, int CT>
__device__ inline void recur_load_b(RecurIn<E, D, CT>& in, const RecurPtrs<E, D>& P, int j) {
    using G = Geo<E, D>;
    constexpr int RT = D / 64;
    const int w = wave_id();
    const uint4* kt = reinterpret_cast<const uint4*>(P.kt + j * P.ops_step);
#pragma unroll
    for (int v = 0; v < G::NVT; ++v)
#pragma unroll
        for (int a = 0; a < RT; ++a) in.kt[a][v] = kt[(a * G::NVT + v) * 64];
#pragma unroll
    for (int a = 0; a < RT; ++a)
        in.gam[a] = *reinterpret_cast<const f32x4*>(P.gam + j * P.gam_step + kSub * (RT * w + a));
}

template <typename E, int D, int CT>
__device__ inline void recur_load_c(RecurIn<E, D, CT>& in, const RecurPtrs<E, D>& P, int j, int len) {
    using G = Geo<E, D>;
    const int w = wave_id(), lg = lane_id() >> 4;
    const uint4* tb = reinterpret_cast<const uint4*>(P.tb + j * P.sq_step);
    const uint4* mm = reinterpret_cast<const uint4*>(P.mm + j * P.sq_step);
#pragma unroll
    for (int v = 0; v < G::NVT; ++v) {
        in.tb[v] = tb[v * 64];
        in.mm[v] = mm[v * 64];
    }
    in.len = len;
    const E* vj = P.v + j * P.tok_step;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int t = kSub * w + 4 * lg + r;
        const int64_t roff = (int64_t)(t < len ? t : len - 1) * ((int64_t)(P.tok_step / kChunk));
#pragma unroll
        for (int c = 0; c < CT; ++c) in.v[c][r] = vj[roff + kSub * c];
    }
}

template <typename E, int D, int CT>
__global__ __launch_bounds__(kThreads) void k_recur(const E* __restrict__ v, ChunkOps ops,
                                                    const int32_t* __restrict__ cu, int64_t total_tokens,
                                                    int64_t fixed_len, const int32_t* __restrict__ seq_chunk0,
                                                    int32_t NH, int32_t H, const float* __restrict__ S0,
                                                    float* __restrict__ ST, E* __restrict__ o) {
    using G = Geo<E, D>;
    using M = Mma<E>;
    using F = typename M::frag;
    constexpr int C = kChunk, CPL = G::CPL;
    constexpr int SW = kSub * CT;      // slab width (value columns)
    constexpr int NS = D / SW;         // slabs per head
    constexpr int RT = D / 64;         // key-channel tiles of S per wave
    constexpr int PS = D + 8;          // pitch of S^T      [col][channel]
    constexpr int PY = C + 8;          // pitch of Y^T, U~^T [col][token]
    __shared__ __attribute__((aligned(16))) E sSt[SW * PS];
    __shared__ __attribute__((aligned(16))) E sYt[SW * PY];
    __shared__ __attribute__((aligned(16))) E sUt[SW * PY];

    // Workgroup -> (sequence*head, slab).  When the (sequence, head) count is
    // a multiple of 8, all slabs of one (sequence, head) get workgroup ids
    // congruent mod 8 and so run on one XCD, sharing that XCD's L2 for the
    // chunk operands.
    int nh, sl;
    {
        const int bid = blockIdx.x;
        if (NH % 8 == 0) {
            sl = (bid / 8) % NS;
            nh = (bid % 8) + 8 * (bid / (8 * NS));
        } else {
            sl = bid % NS;
            nh = bid / NS;
        }
    }
    const int n = nh / H, h = nh % H;
    const int w = wave_id(), li = lane_id() & 15, lg = lane_id() >> 4;
    const int col0 = sl * SW;
    const int64_t rs = (int64_t)H * D;

    // Chunks of this sequence: c0 .. c0 + nch - 1 (the same list k_prep walked).
    int64_t s_start, s_len;
    seq_range(cu, n, total_tokens, fixed_len, s_start, s_len);
    int32_t c0, nch;
    seq_chunks(cu, seq_chunk0, n, fixed_len, s_len, c0, nch);

    RecurPtrs<E, D> P;
    {
        const int64_t cb = (int64_t)h * ops.max_chunks + c0;   // head-major operand slot
        const int tok = kSub * w + li;
        P.ops_step = (int64_t)C * D;
        P.sq_step = (int64_t)C * C;
        P.gam_step = (int64_t)D;
        P.tok_step = (int64_t)C * rs;
        const int lane = lane_id();
        P.qg = static_cast<const E*>(ops.Qg) + cb * C * D + (int64_t)(w * G::VPL * 64 + lane) * G::EPV;
        P.kg = static_cast<const E*>(ops.Kg) + cb * C * D + (int64_t)(w * G::VPL * 64 + lane) * G::EPV;
        P.kt = static_cast<const E*>(ops.KhT) + cb * D * C + (int64_t)(RT * w * G::NVT * 64 + lane) * G::EPV;
        P.tb = static_cast<const E*>(ops.TB) + cb * C * C + (int64_t)(w * G::NVT * 64 + lane) * G::EPV;
        P.mm = static_cast<const E*>(ops.Mm) + cb * C * C + (int64_t)(w * G::NVT * 64 + lane) * G::EPV;
        (void)tok;
        P.gam = ops.gam + cb * D + 4 * lg;
        P.v = v + (s_start * H + h) * D + col0 + li;
    }
    E* const o_base = o + (s_start * H + h) * D + col0 + li;

    // S[a][c][r] = state[channel 16*(RT*w + a) + 4*lg + r][column col0 + 16*c + li]
    f32x4 S[RT][CT];
    const int64_t sbase = ((int64_t)n * H + h) * D * D;
#pragma unroll
    for (int a = 0; a < RT; ++a)
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ch = kSub * (RT * w + a) + 4 * lg + r;
                S[a][c][r] = S0 ? S0[sbase + (int64_t)ch * D + col0 + kSub * c + li] : 0.f;
            }
    auto put_state = [&]() {
#pragma unroll
        for (int a = 0; a < RT; ++a)
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sSt[(kSub * c + li) * PS + kSub * (RT * w + a) + 4 * lg + r] = from_f<E>(S[a][c][r]);
    };
    put_state();

    auto chunk_len = [&](int j) -> int {
        const int64_t rem = s_len - (int64_t)j * C;
        return (int)(rem < C ? rem : C);
    };

    // One chunk step with the operands in `cur`; meanwhile the operands of
    // chunk jp (clamped to the last chunk) are loaded into `pre`, one group
    // after each barrier.  The scheduling barriers keep the three load groups
    // where they are placed.
    auto step = [&](const RecurIn<E, D, CT>& cur, int j, RecurIn<E, D, CT>& pre, int jp) {
        jp = jp < nch ? jp : nch - 1;
        __syncthreads();   // S^T of the previous step is in LDS
        __builtin_amdgcn_sched_barrier(0);
        recur_load_a<E, D, CT>(pre, P, jp);
        __builtin_amdgcn_sched_barrier(0);
        const F* fq = reinterpret_cast<const F*>(cur.qg);
        const F* fk = reinterpret_cast<const F*>(cur.kg);
        const F* ftb = reinterpret_cast<const F*>(cur.tb);
        const F* fmm = reinterpret_cast<const F*>(cur.mm);
        // X = (K . Gamma) S and P = (Q . Gamma) S for token rows 16w..
        f32x4 accX[CT], accO[CT];
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            accX[c] = zero4();
            accO[c] = zero4();
#pragma unroll
            for (int m = 0; m < G::NKC; ++m) {
                const F bs = M::load(&sSt[(kSub * c + li) * PS + lg * CPL + m * M::KW]);
                accX[c] = M::mma(fk[m], bs, accX[c]);
                accO[c] = M::mma(fq[m], bs, accO[c]);
            }
        }
        // Y = V - X, transposed to LDS
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = kSub * w + 4 * lg + r;
                const float vv = t < cur.len ? to_f(cur.v[c][r]) : 0.f;
                sYt[(kSub * c + li) * PY + t] = from_f<E>(vv - accX[c][r]);
            }
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        recur_load_b<E, D, CT>(pre, P, jp);
        __builtin_amdgcn_sched_barrier(0);
        // U~ = T diag(beta) Y  (rows 16w..; k-steps past the diagonal block skipped)
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            f32x4 accU = zero4();
#pragma unroll
            for (int m = 0; m < G::NKT; ++m)
                accU = M::mma(ftb[m], M::load(&sYt[(kSub * c + li) * PY + m * M::KS + lg * M::KW]), accU);
#pragma unroll
            for (int r = 0; r < 4; ++r) sUt[(kSub * c + li) * PY + kSub * w + 4 * lg + r] = from_f<E>(accU[r]);
        }
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        recur_load_c<E, D, CT>(pre, P, jp, chunk_len(jp));
        __builtin_amdgcn_sched_barrier(0);
        // S <- Diag(Gamma_L) S + K^T U~, then O = P + M U~ -> output rows 16w..
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            F bu[G::NKT];
#pragma unroll
            for (int m = 0; m < G::NKT; ++m) bu[m] = M::load(&sUt[(kSub * c + li) * PY + m * M::KS + lg * M::KW]);
#pragma unroll
            for (int a = 0; a < RT; ++a) {
                f32x4 acc = zero4();
                const F* fkt = reinterpret_cast<const F*>(cur.kt[a]);
#pragma unroll
                for (int m = 0; m < G::NKT; ++m) acc = M::mma(fkt[m], bu[m], acc);
#pragma unroll
                for (int r = 0; r < 4; ++r) S[a][c][r] = cur.gam[a][r] * S[a][c][r] + acc[r];
            }
#pragma unroll
            for (int m = 0; m < G::NKT; ++m) accO[c] = M::mma(fmm[m], bu[m], accO[c]);
        }
        // S^T is last read before the Y barrier of this step, so writing it
        // here is safe; the barrier at the top of the next step publishes it.
        put_state();
        E* oj = o_base + (int64_t)j * C * rs;
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = kSub * w + 4 * lg + r;
                if (t < cur.len) oj[(int64_t)t * rs + kSub * c] = from_f<E>(accO[c][r]);
            }
    };

    // Three operand buffers in rotation: while chunk j is processed, the
    // operands of chunk j+1 are already in flight and those of chunk j+2 are
    // issued.  Prefetching is unconditional (indices are clamped to the last
    // chunk): with no path that skips it, the compiler's load counters let
    // the prefetched loads stay outstanding across whole steps instead of
    // draining them before the first matrix product.
    RecurIn<E, D, CT> A, B, Cb;
    if (nch > 0) {
        auto prefetch_all = [&](RecurIn<E, D, CT>& buf, int jj) {
            jj = jj < nch ? jj : nch - 1;
            recur_load_a<E, D, CT>(buf, P, jj);
            recur_load_b<E, D, CT>(buf, P, jj);
            recur_load_c<E, D, CT>(buf, P, jj, chunk_len(jj));
        };
        prefetch_all(A, 0);
        prefetch_all(B, 1);
        for (int j = 0; j < nch; j += 3) {
            step(A, j, Cb, j + 2);
            if (j + 1 >= nch) break;
            step(B, j + 1, A, j + 3);
            if (j + 2 >= nch) break;
            step(Cb, j + 2, B, j + 4);
        }
    }
    if (ST) {
#pragma unroll
        for (int a = 0; a < RT; ++a)
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int ch = kSub * (RT * w + a) + 4 * lg + r;
                    ST[sbase + (int64_t)ch * D + col0 + kSub * c + li] = S[a][c][r];
                }
    }
}

// ---------------------------------------------------------------- k_recur_lds
// bf16 form of k_recur with producer waves.  The chunk operands travel
// global -> LDS by direct loads (global_load_lds_dwordx4: each lane moves 16
// bytes to LDS at M0 + 16 * lane), issued by producer waves that do nothing
// else, one per 16-token row tile (four).  A wave issues its instructions in order, so a
// compute wave that issued its own share of the loads would sit behind them
// for as long as the CU needs to stream a chunk's operands; with producers
// the streaming overlaps the compute waves' matrix work.  (A single producer
// is too slow -- one wave moves about 1 KB per 80 clocks this way -- and
// eight were slower than four: they take issue slots from the compute waves
// on the same SIMDs.)
//
// Buffers: two, alternating by chunk parity.  The compute waves read every
// operand of chunk j into registers before the second barrier of step j, so
// from that barrier on the buffer of chunk j is free and the producers fill
// it with chunk j+2; before the barrier that opens step j+1 they wait for
// chunk j+1 only (loads of one wave complete in issue order), so the loads of
// the next chunk stay in flight across the barriers.  The two buffers are
// distinct LDS arrays so that the compiler can tell the producers' loads into
// one from reads of the other.  Synchronisation is plain s_barrier with explicit
// counter waits: the workgroup fence of __syncthreads would drain the
// producers' in-flight loads at every barrier.
//
// L2 warm-up: four chunks ahead, the producers load one dword of each
// 128-byte line of a share of that chunk's data (operands, Gamma_L and the
// head's value rows) into an LDS scratch that nothing reads; the slab
// workgroups of a head take disjoint shares, so the direct loads of every
// slab later hit L2 rather than HBM.  Landing in LDS, these loads hold no
// registers and nothing waits for them except the counted waits below.
// Because of that sharing the slabs of a head have to stay within a few
// steps of each other; on long sequences the workgroup's last wave (the
// pacing wave) holds back a workgroup that runs too far ahead.
//
// Slab width: 16 value columns, or 32 (forward and transition passes) with
// XW = 2 groups of four compute waves, group x owning column tile x of the
// slab; both groups read the same operand fill.  A chunk's fill is the same
// 64 KB either way, so a 32-column workgroup does twice the work per fill:
// its step is longer (about 1.3 against 1.02 us at d = 128) but it does the
// work of two 16-column ones, which pays when more 16-column chains exist
// than CUs (many sequences or heads: the whole chip's throughput sets the
// time), and not when each chain has a CU to itself (its latency sets the
// time).  The template also takes CT column tiles per compute wave; every
// launch uses CT = 1 (one wave group taking both tiles, CT = 2, measured
// about 1.55 us per step).  With 32 columns the value rows of a region fill
// its misc block, so Gamma_L comes in by one more (4-byte) direct load per
// region into sGam0 / sGam1.
#define KDA_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt immediate (gfx9 encoding): vmcnt in bits 3:0 and 15:14, expcnt
// in 6:4 (7 = no wait), lgkmcnt in 11:8 (15 = no wait).
constexpr unsigned waitcnt_imm(int vm, int lgkm) {
    return (unsigned)((vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8));
}
template <int VM, int LGKM>
__device__ inline void wait_counts() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(VM, LGKM));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// This wave's LDS operations complete, then workgroup barrier.
__device__ inline void barrier_lds() {
    wait_counts<63, 0>();
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1.
template <int N, int I = 0, typename Fn>
__device__ inline void static_for(Fn&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

constexpr int kRecurWaves = 4;                              // compute waves per group (one per row tile)
constexpr int kProdPerWave = 1;                             // producer waves per row tile
constexpr int kProducers = kRecurWaves * kProdPerWave;

// Buffer layout: one region per compute wave w, in 1 KB blocks (64 lanes x
// 16 bytes: the fragment-major tiles of k_prep copied as they are):
//   [kQg, +VPL)  Q . Gamma, row tile w       [kKg, +VPL)  K . Gamma, row tile w
//   [kTb, +NVT)  T diag(beta), row tile w    [kMm, +NVT)  M, row tile w
//   [kKt, +RT*NVT) K^T, channel tiles RT*w ..
//   kMisc: bytes [0, 512) value rows 16w .. 16w+15 x the slab's 16 columns
//          (bf16, row-major); bytes [512, 512 + 64 RT) Gamma_L of channels
//          16 RT w .. (fp32); the rest unused.
template <int D>
struct LdsGeo {
    using G = Geo<__bf16, D>;
    static constexpr int RT = D / 64;
    static constexpr int kQg = 0;
    static constexpr int kKg = kQg + G::VPL;
    static constexpr int kTb = kKg + G::VPL;
    static constexpr int kMm = kTb + G::NVT;
    static constexpr int kKt = kMm + G::NVT;
    static constexpr int kMisc = kKt + RT * G::NVT;
    static constexpr int kBlocks = kMisc + 1;
    static constexpr int kWaveVec = kBlocks * 64;     // 16-byte vectors per compute wave per buffer
    static constexpr int kBufVec = kRecurWaves * kWaveVec;
};

// Modes of the sequential pass:
//   kFwd   the forward pass: o and S_T.
//   kTrans the same chunk steps with v = 0 from S = I and no output, so that
//          S_T is the sequence's transition matrix prod_t (I - beta_t k_t k_t^T)
//          Diag(alpha_t) (orkas.ai "Kimi K3 architecture", §"請求書はサービング側に回ってくる":
//          a segment's final state is its transition applied to the incoming
//          state plus its zero-start state).  v, S0 and o are not accessed.
//   kCkpt  the forward steps keeping what the backward pass needs: the state
//          entering every chunk (aux.ck, bf16 [slot][D][D]), and the
//          per-token U~ = T diag(beta) (V - (K . Gamma) S) (aux.u, bf16, laid
//          out as v); o and S_T as kFwd when given (o may be NULL).
//   kBwd   the state-gradient recurrence, chunks last to first, on the
//          backward operand set (see ChunkOps).  With dS' the gradient of a
//          chunk's outgoing state and dO its output gradients:
//            R  = (K . exp(b_L - b)) dS' + M^T dO        (= dU~)
//            dZ = T^T R,  dY = diag(beta) dZ             (dY is dv)
//            dS = Diag(Gamma_L) dS' + (Q . Gamma)^T dO - (K . Gamma)^T dY
//          Inputs: v = dO, S0 = dS_T (may be NULL); outputs: ST = dS0,
//          aux.ck = dS' of every chunk (bf16 [slot][D][D]), aux.y = dZ (dv is
//          written by the gradient kernel from dZ; o is not accessed).
//          These are the adjoints of the kFwd step (the chain rule through
//          U~ = T diag(beta) Y, O = (Q . Gamma) S + M U~ and
//          S' = Diag(Gamma_L) S + K^T U~).
//   kCkptLean kCkpt without o, for the backward pass that evaluates the
//          forward again: Q . Gamma and M are neither loaded nor used (its
//          k_prep does not write them), which takes 6 of the 17 blocks out of
//          every region's fill.
//   kFwdCk kFwd that also writes the fp32 state after every aux.every-th
//          chunk of a sequence to aux.sck (slot = the chunk's global index):
//          the prefix-cache checkpoints.  A mode of its own, so that the plain
//          forward carries no test for it.
enum { kFwd = 0, kTrans = 1, kCkpt = 2, kBwd = 3, kFwdCk = 4, kCkptLean = 5 };

struct RecurAux {
    __bf16* ck;        // kCkpt: S entering each chunk; kBwd: dS' of each chunk
    __bf16* y;         // kBwd: dZ
    __bf16* u;         // kCkpt: U~
    const float* bet;  // kBwd: per-chunk beta (ChunkOps::bet)
    float* sck;        // kFwdCk: fp32 state after every `every`-th chunk of a sequence
    int32_t every;
    int32_t n_slots;   // kFwdCk: slots of sck
    const int32_t* ck0;   // kFwdCk with cu_seqlens: first slot of each sequence (k_chunk_table)
    int32_t* prog;     // pacing: steps done per (sequence*head, slab), or NULL (no pacing)
};

// The two triangular tiles of a region (T diag(beta) and M in the forward
// modes, T^T and M^T in kBwd) have a 32-token half that is zero by structure:
// row tiles 0 and 1 of the lower-triangular forms over tokens 32..63, row
// tiles 2 and 3 of the transposes over tokens 0..31 (T continues as the
// identity past a chunk's end, so this holds for short chunks too).  Those
// halves are neither loaded nor read; the fragments are zero in registers.
template <int kMode>
struct ZeroHalf {
    static constexpr int kHalf = kMode == kBwd ? 0 : 1;   // which 32-token half is zero
    __device__ static bool zero(int region) { return kMode == kBwd ? region >= 2 : region < 2; }
};

template <int D, int kMode, int CT, int XW = 1>
__global__ __launch_bounds__((kRecurWaves * XW + kProducers + 1) * 64) void k_recur_lds(
    const __bf16* __restrict__ v, ChunkOps ops, const int32_t* __restrict__ cu, int64_t total_tokens,
    int64_t fixed_len, const int32_t* __restrict__ seq_chunk0, int32_t NH, int32_t H, const float* __restrict__ S0,
    float* __restrict__ ST, __bf16* __restrict__ o, RecurAux aux, int32_t jb, int32_t je, int32_t xcd_lo) {
    constexpr bool kTransition = kMode == kTrans;
    constexpr bool kBack = kMode == kBwd;
    constexpr bool kCk = kMode == kCkpt || kMode == kCkptLean;   // keeps the backward's inputs
    constexpr bool kNoQM = kMode == kCkptLean;                   // no Q . Gamma, no M
    using E = __bf16;
    using G = Geo<E, D>;
    using L = LdsGeo<D>;
    using M = Mma<E>;
    using F = typename M::frag;
    using Z = ZeroHalf<kMode>;
    static_assert(G::VPL == G::NKC && G::NVT == G::NKT, "one 16-byte vector per bf16 fragment");
    static_assert(kRecurWaves == kNSub, "one compute wave per 16-token row tile");
    static_assert(G::NKT == 2, "the zero halves are the two 32-token halves of a 64-token chunk");
    static_assert(CT * XW == 1 || (CT * XW == 2 && (kMode == kFwd || kMode == kTrans)),
                  "32-column slabs: forward and transition passes only");
    constexpr int C = kChunk, CPL = G::CPL, RT = L::RT;
    // Compute waves: XW groups of kRecurWaves, group x owning column tiles
    // x CT .. x CT + CT - 1 of the slab (wave w: row tile w mod 4); then the
    // producer waves, then the pacing wave.
    constexpr int NCW = kRecurWaves * XW;
    constexpr int kPacer = NCW + kProducers;
    constexpr int SW = kSub * CT * XW; // slab width (value columns)
    constexpr int NS = D / SW;         // slabs per head
    constexpr int PS = D + 8;          // pitch of S^T      [col][channel]
    constexpr int PY = C + 8;          // pitch of Y^T, U~^T [col][token]
    __shared__ __attribute__((aligned(16))) uint4 sBuf0[L::kBufVec];
    __shared__ __attribute__((aligned(16))) uint4 sBuf1[L::kBufVec];
    __shared__ __attribute__((aligned(16))) E sSt[SW * PS];
    __shared__ __attribute__((aligned(16))) E sYt[SW * PY];
    __shared__ __attribute__((aligned(16))) E sUt[SW * PY];
    __shared__ unsigned sTouch[kProducers * 64];   // warm-up loads land here, never read
    // 32-column slabs: the value rows fill the misc block, so Gamma_L of each region's
    // 16 RT channels comes in by 4-byte direct loads into these (one per
    // buffer; sized so that a load from all 64 lanes at the last region's
    // base would still stay inside).
    constexpr int kGamPer = 16 * RT;
    constexpr int kGamLen = SW > kSub ? (kRecurWaves - 1) * kGamPer + 64 : 1;
    __shared__ __attribute__((aligned(16))) float sGam0[kGamLen];
    __shared__ __attribute__((aligned(16))) float sGam1[kGamLen];

    // Workgroup -> (sequence*head, slab); slabs of one (sequence, head) share
    // an XCD (and its L2) when the (sequence, head) count is a multiple of 8.
    // With xcd_lo the grid is twice the work: workgroups on XCDs 4..7
    // (workgroup id mod 8 >= 4) leave at once, so that the recurrence holds
    // only XCDs 0..3 and their L2s (NH a multiple of 4).
    int nh, sl;
    {
        const int bid = blockIdx.x;
        if (xcd_lo) {
            if (bid % 8 >= 4) return;
            const int r = bid / 8;
            sl = r % NS;
            nh = (bid % 8) + 4 * (r / NS);
        } else if (NH % 8 == 0) {
            sl = (bid / 8) % NS;
            nh = (bid % 8) + 8 * (bid / (8 * NS));
        } else {
            sl = bid % NS;
            nh = bid / NS;
        }
    }
    const int n = nh / H, h = nh % H;
    const int w = wave_id(), lane = lane_id(), li = lane & 15, lg = lane >> 4;
    const int col0 = sl * SW;
    const int64_t rs = (int64_t)H * D;

    int64_t s_start, s_len;
    seq_range(cu, n, total_tokens, fixed_len, s_start, s_len);
    int32_t c0, nch;
    seq_chunks(cu, seq_chunk0, n, fixed_len, s_len, c0, nch);
    // This launch takes chunks [j_lo, j_lo + ns) of the sequence (all of
    // them when [jb, je) covers it): S0 is the state entering chunk j_lo and
    // ST the state after the last one.
    const int32_t j_lo = jb < nch ? jb : nch;
    const int32_t ns = (je < nch ? je : nch) > j_lo ? (je < nch ? je : nch) - j_lo : 0;
    const int64_t cb = (int64_t)h * ops.max_chunks + c0;   // head-major operand slot of chunk 0
    auto chunk_len = [&](int j) -> int {
        const int64_t rem = s_len - (int64_t)j * C;
        return (int)(rem < C ? rem : C);
    };
    // chunk processed at step s (the backward pass walks the chunks last to first)
    auto chunk_at = [&](int s_) -> int { return kBack ? j_lo + ns - 1 - s_ : j_lo + s_; };

    if (w == kPacer) {
        // ------------------------------------------------ pacing wave
        // The slab workgroups of a head share their chunk operands through
        // L2: each warms only its share of the lines ahead of use.  One that
        // falls further behind than L2 holds those lines loses that support,
        // misses on the other shares and falls further behind, so over a long
        // sequence the drift, not the step, sets the kernel time.  This wave
        // passes the same three barriers per step as the others (so it is at
        // the workgroup's step), and every kPaceEvery steps compares its
        // step count with its siblings' published counts, sleeps while it is
        // more than kPaceLag steps ahead of the slowest (which holds the
        // whole workgroup at the next barrier), then publishes its own.  Every wait ends: at most
        // kPaceBudget sleeps per workgroup.  Counts outside 0..ns (the
        // sentinel written at the end of a call, or memory never written)
        // are ignored.
        // Drift needs thousands of steps to build up; shorter sequences are
        // not paced at all (this wave then only passes the barriers).
        constexpr int kPaceEvery = 8, kPaceLead = 4, kPaceLag = 16, kPaceBudget = 1024, kPaceMinChunks = 2048;
        int32_t* const pg = (aux.prog && ns >= kPaceMinChunks) ? aux.prog + (int64_t)nh * NS : nullptr;
        auto post = [&](int v) {
            if (pg && lane == 0) __hip_atomic_store(pg + sl, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        };
        auto load = [&]() {
            return lane < NS ? __hip_atomic_load(pg + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                             : 0x7fffffff;
        };
        auto slowest = [&](int v) {
            v = (v < 0 || v > ns) ? 0x7fffffff : v;
            v = min(v, __shfl_xor(v, 1));
            v = min(v, __shfl_xor(v, 2));
            v = min(v, __shfl_xor(v, 4));
            return __builtin_amdgcn_readfirstlane(v);
        };
        // The counts are read kPaceLead steps before they are used, and this
        // wave's own count is published right after each check, so that the
        // wait for a load never covers a recent store (both are device-scope
        // accesses, with a long latency).  The counts seen are then up to
        // kPaceEvery + kPaceLead - 1 steps old, which kPaceLag allows for.
        int left = kPaceBudget;
        int seen = 0;
        post(0);
        for (int s_ = 0; s_ < ns; ++s_) {
            const bool on = pg && s_ + 1 < ns;
            barrier_lds();
            if (on && (s_ % kPaceEvery) == kPaceEvery - 1 - kPaceLead) seen = load();
            barrier_lds();
            barrier_lds();
            if (on && (s_ % kPaceEvery) == kPaceEvery - 1) {
                // sleep in proportion to the excess lead (about 0.4 us per
                // step), rather than until the slowest sibling publishes again
                const int excess = s_ + 1 - kPaceLag - slowest(seen);
                for (int n = excess > 0 ? min(2 * excess, 40) : 0; n > 0 && left > 0; --n, --left)
                    __builtin_amdgcn_s_sleep(8);
                post(s_ + 1);
            }
        }
        post(0x7fffffff);
        return;
    }
    if (w >= NCW) {
        // ------------------------------------------------ producer waves
        const int pw = w - NCW;
        const int cw = pw / kProdPerWave;   // the compute wave whose operands this wave loads
        const int part = pw % kProdPerWave; // which of its blocks: part, part + kProdPerWave, ...
        const E* qg = static_cast<const E*>(ops.Qg) + cb * C * D + lane * G::EPV;
        const E* kg = static_cast<const E*>(ops.Kg) + cb * C * D + lane * G::EPV;
        const E* kt = static_cast<const E*>(ops.KhT) + cb * D * C + lane * G::EPV;
        const E* tb = static_cast<const E*>(ops.TB) + cb * C * C + lane * G::EPV;
        const E* mm = static_cast<const E*>(ops.Mm) + cb * C * C + lane * G::EPV;
        constexpr int kVL = SW / 8;   // lanes per value row of the slab (16 bytes each)
        const E* vv = v + (s_start * H + h) * D + col0 + 8 * (lane % kVL);
        const int gi = (lane >= 32 && lane < 32 + 4 * RT) ? lane - 32 : 0;
        const float* gm = ops.gam + cb * D + 4 * gi;
        // kBwd: lanes 48..51 bring beta of the region's 16 rows (bytes 768..831)
        const bool is_bet = kBack && lane >= 48 && lane < 52;
        const float* bt = kBack ? aux.bet + cb * C + kSub * cw + 4 * (is_bet ? lane - 48 : 0) : nullptr;
        auto dma = [](const void* src, uint4* lds) {
            __builtin_amdgcn_global_load_lds(src, KDA_LDS_PTR(lds), 16, 0, 0);
        };
        // Direct loads per producer wave and chunk: blocks part, part + P, ...
        // of its compute wave's region; a part with one block fewer repeats
        // its last one, so that every producer issues the same count.
        constexpr int kDma = (L::kBlocks + kProdPerWave - 1) / kProdPerWave;
        // Block b of region cw for chunk j (b is a compile-time constant).
        auto block = [&](auto b_c, uint4* dst, int j, int len) {
            constexpr int b = decltype(b_c)::value;
            const int64_t oo = (int64_t)j * C * D, so = (int64_t)j * C * C;
            if constexpr (b < L::kKg)
                dma(qg + oo + (cw * G::VPL + b - L::kQg) * 64 * G::EPV, dst + b * 64);
            else if constexpr (b < L::kTb)
                dma(kg + oo + (cw * G::VPL + b - L::kKg) * 64 * G::EPV, dst + b * 64);
            else if constexpr (b < L::kMm)
                dma(tb + so + (cw * G::NVT + b - L::kTb) * 64 * G::EPV, dst + b * 64);
            else if constexpr (b < L::kKt)
                dma(mm + so + (cw * G::NVT + b - L::kMm) * 64 * G::EPV, dst + b * 64);
            else if constexpr (b < L::kMisc)
                dma(kt + oo + (cw * RT * G::NVT + b - L::kKt) * 64 * G::EPV, dst + b * 64);
            else {
                int row = kSub * cw + lane / kVL;
                row = row < len ? row : len - 1;
                const void* misc = (lane < 2 * SW && !kTransition)
                                       ? static_cast<const void*>(vv + ((int64_t)j * C + row) * rs)
                                   : is_bet ? static_cast<const void*>(bt + (int64_t)j * C)
                                            : static_cast<const void*>(gm + (int64_t)j * D + kSub * RT * cw);
                dma(misc, dst + b * 64);
            }
        };
        // Loads [lo, hi) of this producer's kDma loads for a chunk.  Blocks
        // that are zero for this region (ZeroHalf) are not loaded.
        auto issue_part = [&](auto part_c, auto lo_c, auto hi_c, uint4* dst, int j, int len) {
            constexpr int pt = decltype(part_c)::value;
            static_for<kDma>([&](auto i_c) {
                constexpr int i = decltype(i_c)::value;
                if constexpr (i >= decltype(lo_c)::value && i < decltype(hi_c)::value) {
                    constexpr int b0 = pt + kProdPerWave * i;
                    constexpr int b = b0 < L::kBlocks ? b0 : b0 - kProdPerWave;
                    if constexpr (kNoQM && ((b >= L::kQg && b < L::kKg) || (b >= L::kMm && b < L::kKt))) {
                    } else if constexpr (b == L::kTb + Z::kHalf || b == L::kMm + Z::kHalf) {
                        if (!Z::zero(cw)) block(std::integral_constant<int, b>{}, dst, j, len);
                    } else {
                        block(std::integral_constant<int, b>{}, dst, j, len);
                    }
                }
            });
        };
        auto issue = [&](uint4* buf, int s_, auto lo_c, auto hi_c) {
            const int j = chunk_at(s_);
            const int len = chunk_len(j);
            uint4* dst = buf + cw * L::kWaveVec;
            static_for<kProdPerWave>([&](auto p_c) {
                if (part == decltype(p_c)::value) issue_part(p_c, lo_c, hi_c, dst, j, len);
            });
            if constexpr (SW > kSub && decltype(hi_c)::value == kDma) {
                // Gamma_L of this region's channels (one more load per chunk)
                float* sg = (buf == sBuf0 ? sGam0 : sGam1) + cw * kGamPer;
                if (lane < kGamPer)
                    __builtin_amdgcn_global_load_lds(ops.gam + (cb + j) * D + kSub * RT * cw + lane, KDA_LDS_PTR(sg),
                                                     4, 0, 0);
            }
        };
        using All0 = std::integral_constant<int, 0>;
        using AllN = std::integral_constant<int, kDma>;
        // loads issued before the compute waves' second inner barrier, in
        // 17ths of the fill, measured at d = 128, 32 heads x 65536 tokens:
        // forward 6 (3, 6, 9, 12, 15, 17: 1.10, 1.10, 1.11, 1.12, 1.12,
        // 1.15 ms); kCkpt and kBwd 12 (3, 6, 9, 12, 17: 1.45 / 1.49,
        // 1.47 / 1.52, 1.46 / 1.46, 1.45 / 1.44, 1.51 / 1.47 ms)
        constexpr int kCut17 = (kCk || kMode == kBwd) ? 12 : 6;
        using Cut = std::integral_constant<int, (kDma * kCut17 + 8) / 17>;

        // Warm-up lines of this slab: kTouch per producer lane, over one
        // chunk's operands, Gamma_L and the head's value rows.
        constexpr int kAhead = 4;
        constexpr int64_t kBq = (int64_t)C * D * 2, kBs = (int64_t)C * C * 2;   // bytes per chunk slot
        constexpr int kQLines = (int)(kBq / 128);
        constexpr int kTriLines = (int)(kBs / 128) - 2 * 8;   // the two zero 1 KB halves skipped
        constexpr int kFullOps = 3 * kQLines + 2 * kTriLines;
        constexpr int kOpsLines = kNoQM ? 2 * kQLines + kTriLines : kFullOps;
        // byte offset of line t of a triangular tile's loaded blocks (tile
        // block 2 w + half; the zero ones are 1, 3 or, in kBwd, 4, 6)
        auto tri_off = [](int t) -> int64_t {
            const int k = t / 8;
            const int b = kMode == kBwd ? (k < 4 ? k : 2 * k - 3) : (k == 0 ? 0 : k == 1 ? 2 : k + 2);
            return (int64_t)b * 1024 + (t % 8) * 128;
        };
        constexpr int kGamLines = D * 4 / 128;
        constexpr int kVRowLines = D * 2 / 128;
        constexpr int kLines = kOpsLines + kGamLines + kChunk * kVRowLines;
        constexpr int kPerSlab = (kLines + NS - 1) / NS;
        constexpr int kTouch = (kPerSlab + 64 * kProducers - 1) / (64 * kProducers);
        const char* t_base[kTouch];   // line in chunk 0 (operands, Gamma_L) or at token 0 (value rows)
        int64_t t_step[kTouch];       // bytes between chunks (operands, Gamma_L)
        int t_vrow[kTouch];           // value row in the chunk, or -1
#pragma unroll
        for (int k = 0; k < kTouch; ++k) {
            int q = pw * 64 + lane + 64 * kProducers * k;
            q = q < kPerSlab ? q : kPerSlab - 1;
            int line = sl * kPerSlab + q;
            line = line < kLines ? line : kLines - 1;
            // kNoQM: its lines skip the Q . Gamma and M ones of the full list below
            if (kNoQM) line += line < 2 * kQLines + kTriLines ? kQLines : kQLines + kTriLines;
            const int64_t off = (int64_t)line * 128;
            t_vrow[k] = -1;
            if (off < kBq) { t_base[k] = (const char*)ops.Qg + cb * kBq + off; t_step[k] = kBq; }
            else if (off < 2 * kBq) { t_base[k] = (const char*)ops.Kg + cb * kBq + off - kBq; t_step[k] = kBq; }
            else if (off < 3 * kBq) { t_base[k] = (const char*)ops.KhT + cb * kBq + off - 2 * kBq; t_step[k] = kBq; }
            else if (line < 3 * kQLines + kTriLines) {
                t_base[k] = (const char*)ops.TB + cb * kBs + tri_off(line - 3 * kQLines);
                t_step[k] = kBs;
            } else if (line < kFullOps) {
                t_base[k] = (const char*)ops.Mm + cb * kBs + tri_off(line - 3 * kQLines - kTriLines);
                t_step[k] = kBs;
            } else if (line < kFullOps + kGamLines) {
                t_base[k] = (const char*)(ops.gam + cb * D) + (int64_t)(line - kFullOps) * 128;
                t_step[k] = (int64_t)D * 4;
            } else if (kTransition) {   // no value rows: warm Gamma_L again instead
                t_base[k] = (const char*)(ops.gam + cb * D);
                t_step[k] = (int64_t)D * 4;
            } else {
                const int vl = line - kFullOps - kGamLines;
                t_vrow[k] = vl / kVRowLines;
                t_base[k] = (const char*)(v + (s_start * H + h) * D) + (int64_t)(vl % kVRowLines) * 128;
                t_step[k] = 0;
            }
        }
        // Loads one dword per line of the chunk kAhead steps after step s
        // (clamped to the last step).
        auto touch = [&](int s_) {
            const int jt = chunk_at(s_ + kAhead < ns ? s_ + kAhead : ns - 1);
#pragma unroll
            for (int k = 0; k < kTouch; ++k) {
                const char* p;
                if (t_vrow[k] >= 0) {
                    const int64_t tok = (int64_t)jt * C + t_vrow[k];
                    p = t_base[k] + (tok < s_len ? tok : s_len - 1) * rs * 2;
                } else {
                    p = t_base[k] + jt * t_step[k];
                }
                __builtin_amdgcn_global_load_lds(p, KDA_LDS_PTR(sTouch + pw * 64), 4, 0, 0);
            }
        };
        // Loads per chunk fill of this producer: kDma, or kDma - 2 when its
        // region skips the zero halves of the two triangular tiles.
        const bool lean = Z::zero(cw);
        // loads per chunk fill (32 columns: Gamma_L apart; kNoQM: without Q . Gamma and M)
        constexpr int kFill = kDma + (SW > kSub ? 1 : 0) - (kNoQM ? G::VPL + G::NVT : 0);
        constexpr int kZeroSkip = kNoQM ? 1 : 2;   // zero-half blocks a lean region skips
        auto wait_fill = [&]() {
            if (lean) wait_counts<2 * kTouch + kFill - kZeroSkip, 15>();
            else wait_counts<2 * kTouch + kFill, 15>();
        };
        // One step j: open it; after the compute waves' first inner barrier
        // (chunk j's operands are in their registers) refill chunk j's buffer
        // with chunk j+2, part of the loads before their second inner barrier
        // and the rest after it, then warm up chunk j+kAhead and wait until
        // chunk j+1 has landed (the loads issued after it -- the previous
        // step's warm-up, this step's fill and warm-up -- may stay in
        // flight).  A wave needs about 80 clocks to issue each 1 KB direct
        // load, so the whole fill takes longer than the compute waves' work
        // between two barriers; split in two, it overlaps both stretches
        // that follow the first inner barrier instead of holding up the
        // second.
        auto pstep = [&](uint4* buf, int j) {
            barrier_lds();
            barrier_lds();
            const bool fill = j + 2 < ns;
            if (fill) issue(buf, j + 2, All0{}, Cut{});
            barrier_lds();
            if (fill) issue(buf, j + 2, Cut{}, AllN{});
            touch(j);
            if (fill)
                wait_fill();
            else
                wait_counts<2 * kTouch, 15>();
        };
        if (ns > 0) {
            issue(sBuf0, 0, All0{}, AllN{});
            if (ns > 1) issue(sBuf1, 1, All0{}, AllN{});
            touch(-2);
            touch(-1);
            if (ns > 1)   // chunk 0 has landed
                wait_fill();
            else
                wait_counts<2 * kTouch, 15>();
            for (int j = 0; j < ns; j += 2) {
                pstep(sBuf0, j);
                if (j + 1 >= ns) break;
                pstep(sBuf1, j + 1);
            }
        }
        // No direct LDS load may outlive the workgroup.  (The compiler drops a
        // counter wait right before the end of the program, which waits by
        // itself; this one is kept explicit.)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        return;
    }

    // ---------------------------------------------------- compute waves
    // row tile rt of the chunk; first column cb0 of this wave within the slab
    const int rt = w % kRecurWaves, cb0 = kSub * CT * (w / kRecurWaves);
    const int64_t o_off = (s_start * H + h) * D + col0 + cb0 + li;
    // kFwdCk: slot of this sequence's first checkpoint
    int32_t ck_first = 0;
    if constexpr (kMode == kFwdCk) ck_first = cu ? aux.ck0[n] : n * (nch / aux.every);
    // S[a][c][r] = state[channel 16*(RT*rt + a) + 4*lg + r][column col0 + cb0 + 16*c + li]
    // (kBwd: the state gradient); c is the wave's column tile (CT of them)
    f32x4 S[RT][CT];
    const int64_t sbase = ((int64_t)n * H + h) * D * D;
#pragma unroll
    for (int a = 0; a < RT; ++a)
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ch = kSub * (RT * rt + a) + 4 * lg + r, col = col0 + cb0 + kSub * c + li;
                if constexpr (kTransition) S[a][c][r] = ch == col ? 1.f : 0.f;
                else S[a][c][r] = S0 ? S0[sbase + (int64_t)ch * D + col] : 0.f;
            }
    auto put_state = [&]() {
#pragma unroll
        for (int a = 0; a < RT; ++a)
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sSt[(cb0 + kSub * c + li) * PS + kSub * (RT * rt + a) + 4 * lg + r] = from_f<E>(S[a][c][r]);
    };
    put_state();
    // kCkpt / kBwd: this slab's columns of the state (gradient) as chunk j
    // starts, into slot j of aux.ck (state_swz layout)
    auto keep_state = [&](int j) {
        E* ck = aux.ck + (cb + j) * D * D;
#pragma unroll
        for (int a = 0; a < RT; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ck[state_swz<D>(kSub * (RT * rt + a) + 4 * lg + r, col0 + cb0 + li)] = from_f<E>(S[a][0][r]);
    };

    // (the step bodies are forced inline: were one called as a function, its
    // captures would live in scratch memory)
    auto step = [&](const uint4* buf, int j) __attribute__((always_inline)) {
        const int len = chunk_len(j);
        const uint4* cur = buf + rt * L::kWaveVec;
        if constexpr (kCk) keep_state(j);
        barrier_lds();   // chunk j's operands are in `buf`; S^T of the previous step is in LDS
        const F* fr = reinterpret_cast<const F*>(cur) + lane;
        F fq[G::NKC], fk[G::NKC];
#pragma unroll
        for (int m = 0; m < G::NKC; ++m) {
            if constexpr (!kNoQM) fq[m] = fr[(L::kQg + m) * 64];
            fk[m] = fr[(L::kKg + m) * 64];
        }
        // X = (K . Gamma) S and P = (Q . Gamma) S for token rows 16w.. (each
        // A fragment serves the wave's CT column tiles)
        f32x4 accX[CT], accO[CT];
#pragma unroll
        for (int c = 0; c < CT; ++c) accX[c] = accO[c] = zero4();
#pragma unroll
        for (int m = 0; m < G::NKC; ++m)
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                const F bs = M::load(&sSt[(cb0 + kSub * c + li) * PS + lg * CPL + m * M::KW]);
                accX[c] = M::mma(fk[m], bs, accX[c]);
                if constexpr (!kNoQM) accO[c] = M::mma(fq[m], bs, accO[c]);
            }
        // Y = V - X, transposed to LDS (rows past the chunk end are zero)
        const E* vrows = reinterpret_cast<const E*>(cur + L::kMisc * 64);
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = kSub * rt + 4 * lg + r;
                const float vv = kTransition ? 0.f : to_f(vrows[(4 * lg + r) * SW + cb0 + kSub * c + li]);
                sYt[(cb0 + kSub * c + li) * PY + t] = from_f<E>(t < len ? vv - accX[c][r] : 0.f);
            }
        F ftb[G::NKT], fmm[G::NKT], fkt[RT][G::NKT];
        const bool zh = Z::zero(rt);
#pragma unroll
        for (int m = 0; m < G::NKT; ++m) {
            if (m == Z::kHalf && zh) {
                ftb[m] = F{};
                fmm[m] = F{};
            } else {
                ftb[m] = fr[(L::kTb + m) * 64];
                if constexpr (!kNoQM) fmm[m] = fr[(L::kMm + m) * 64];
            }
        }
#pragma unroll
        for (int a = 0; a < RT; ++a)
#pragma unroll
            for (int m = 0; m < G::NKT; ++m) fkt[a][m] = fr[(L::kKt + a * G::NKT + m) * 64];
        f32x4 gam[RT];
        const float* gl = SW > kSub ? (buf == sBuf0 ? sGam0 : sGam1) + rt * kGamPer
                                 : reinterpret_cast<const float*>(cur + L::kMisc * 64) + 128;
#pragma unroll
        for (int a = 0; a < RT; ++a) gam[a] = *reinterpret_cast<const f32x4*>(gl + kSub * a + 4 * lg);
        barrier_lds();
        // U~ = T diag(beta) Y  (rows 16w..)
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            f32x4 accU = zero4();
#pragma unroll
            for (int m = 0; m < G::NKT; ++m)
                accU = M::mma(ftb[m], M::load(&sYt[(cb0 + kSub * c + li) * PY + m * M::KS + lg * M::KW]), accU);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = kSub * rt + 4 * lg + r;
                const E u = from_f<E>(accU[r]);
                sUt[(cb0 + kSub * c + li) * PY + t] = u;
                if constexpr (kCk) {
                    if (t < len) aux.u[o_off + ((int64_t)j * C + t) * rs] = u;
                }
            }
        }
        barrier_lds();
        // S <- Diag(Gamma_L) S + K^T U~, then O = P + M U~ (rows 16w..)
        F bu[CT][G::NKT];
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int m = 0; m < G::NKT; ++m) bu[c][m] = M::load(&sUt[(cb0 + kSub * c + li) * PY + m * M::KS + lg * M::KW]);
#pragma unroll
        for (int a = 0; a < RT; ++a)
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                f32x4 acc = zero4();
#pragma unroll
                for (int m = 0; m < G::NKT; ++m) acc = M::mma(fkt[a][m], bu[c][m], acc);
#pragma unroll
                for (int r = 0; r < 4; ++r) S[a][c][r] = gam[a][r] * S[a][c][r] + acc[r];
            }
        // kFwdCk: the state after this chunk, when it is a chosen checkpoint;
        // the checkpoints are packed, sequence after sequence
        if constexpr (kMode == kFwdCk) {
            const int32_t slot = ck_first + (j + 1) / aux.every - 1;
            if ((j + 1) % aux.every == 0 && slot < aux.n_slots) {
                float* dst = aux.sck + ((int64_t)slot * H + h) * D * D + col0 + cb0 + li;
#pragma unroll
                for (int a = 0; a < RT; ++a)
#pragma unroll
                    for (int r = 0; r < 4; ++r) dst[(int64_t)(kSub * (RT * rt + a) + 4 * lg + r) * D] = S[a][0][r];
            }
        }
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int m = 0; m < G::NKT; ++m)
                if constexpr (!kNoQM) accO[c] = M::mma(fmm[m], bu[c][m], accO[c]);
        // S^T is last read before the Y barrier of this step; the barrier at
        // the top of the next step publishes the new one.
        put_state();
        if (kMode == kFwd || kMode == kFwdCk || (kMode == kCkpt && o)) {
            E* oj = o + o_off + (int64_t)j * C * rs;
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = kSub * rt + 4 * lg + r;
                    if (t < len) oj[(int64_t)t * rs + kSub * c] = from_f<E>(accO[c][r]);
                }
        }
    };

    // kBwd step.  Buffer slots: kQg K . exp(b_L - b) (rows over channels),
    // kKg (Q . Gamma)^T and kKt (K . Gamma)^T (channel tiles over tokens),
    // kTb T^T and kMm M^T (rows over tokens); the misc block holds the dO
    // rows, Gamma_L and beta.
    auto step_bwd = [&](const uint4* buf, int j) __attribute__((always_inline)) {
        const int len = chunk_len(j);
        const uint4* cur = buf + rt * L::kWaveVec;
        keep_state(j);
        barrier_lds();   // chunk j's operands are in `buf`; dS'^T is in LDS
        const F* fr = reinterpret_cast<const F*>(cur) + lane;
        F fkh[G::NKC];
#pragma unroll
        for (int m = 0; m < G::NKC; ++m) fkh[m] = fr[(L::kQg + m) * 64];
        // dO as the B operand over tokens: token 32m + 8lg + e of column li
        // sits in the value rows of region 2m + lg/2, row 8(lg & 1) + e.
        F bo[G::NKT];
#pragma unroll
        for (int m = 0; m < G::NKT; ++m) {
            const E* rows = reinterpret_cast<const E*>(buf + (2 * m + (lg >> 1)) * L::kWaveVec + L::kMisc * 64);
#pragma unroll
            for (int e = 0; e < M::KW; ++e) bo[m][e] = rows[(8 * (lg & 1) + e) * SW + cb0 + li];
        }
        F fmt[G::NKT];
#pragma unroll
        for (int m = 0; m < G::NKT; ++m) fmt[m] = (m == Z::kHalf && Z::zero(rt)) ? F{} : fr[(L::kMm + m) * 64];
        // R = K^ dS' + M^T dO  (rows 16w..), transposed to LDS
        f32x4 accR = zero4();
#pragma unroll
        for (int m = 0; m < G::NKC; ++m)
            accR = M::mma(fkh[m], M::load(&sSt[li * PS + lg * CPL + m * M::KW]), accR);
#pragma unroll
        for (int m = 0; m < G::NKT; ++m) accR = M::mma(fmt[m], bo[m], accR);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = kSub * rt + 4 * lg + r;
            sYt[li * PY + t] = from_f<E>(t < len ? accR[r] : 0.f);
        }
        F ftt[G::NKT], fqt[RT][G::NKT], fkt[RT][G::NKT];
#pragma unroll
        for (int m = 0; m < G::NKT; ++m) ftt[m] = (m == Z::kHalf && Z::zero(rt)) ? F{} : fr[(L::kTb + m) * 64];
#pragma unroll
        for (int a = 0; a < RT; ++a)
#pragma unroll
            for (int m = 0; m < G::NKT; ++m) {
                fqt[a][m] = fr[(L::kKg + a * G::NKT + m) * 64];
                fkt[a][m] = fr[(L::kKt + a * G::NKT + m) * 64];
            }
        f32x4 gam[RT];
        const float* gl = reinterpret_cast<const float*>(cur + L::kMisc * 64) + 128;
#pragma unroll
        for (int a = 0; a < RT; ++a) gam[a] = *reinterpret_cast<const f32x4*>(gl + kSub * a + 4 * lg);
        const f32x4 bet = *reinterpret_cast<const f32x4*>(gl + 64 + 4 * lg);   // bytes 768.. of the block
        barrier_lds();
        // dZ = T^T R (rows 16w..) out; -dY^T = -(diag(beta) dZ)^T to LDS
        {
            f32x4 accZ = zero4();
#pragma unroll
            for (int m = 0; m < G::NKT; ++m)
                accZ = M::mma(ftt[m], M::load(&sYt[li * PY + m * M::KS + lg * M::KW]), accZ);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = kSub * rt + 4 * lg + r;
                if (t < len) aux.y[o_off + ((int64_t)j * C + t) * rs] = from_f<E>(accZ[r]);
                sUt[li * PY + t] = from_f<E>(t < len ? -bet[r] * accZ[r] : 0.f);
            }
        }
        barrier_lds();
        // dS <- Diag(Gamma_L) dS' + (Q . Gamma)^T dO - (K . Gamma)^T dY
        F bu[G::NKT];
#pragma unroll
        for (int m = 0; m < G::NKT; ++m) bu[m] = M::load(&sUt[li * PY + m * M::KS + lg * M::KW]);
#pragma unroll
        for (int a = 0; a < RT; ++a) {
            f32x4 acc = zero4();
#pragma unroll
            for (int m = 0; m < G::NKT; ++m) {
                acc = M::mma(fqt[a][m], bo[m], acc);
                acc = M::mma(fkt[a][m], bu[m], acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) S[a][0][r] = gam[a][r] * S[a][0][r] + acc[r];
        }
        put_state();
    };

    auto run = [&](const uint4* buf, int s_) __attribute__((always_inline)) {
        if constexpr (kBack) step_bwd(buf, chunk_at(s_));
        else step(buf, chunk_at(s_));
    };
    for (int s_ = 0; s_ < ns; s_ += 2) {
        run(sBuf0, s_);
        if (s_ + 1 >= ns) break;
        run(sBuf1, s_ + 1);
    }
    if (ST) {
#pragma unroll
        for (int a = 0; a < RT; ++a)
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int ch = kSub * (RT * rt + a) + 4 * lg + r;
                    ST[sbase + (int64_t)ch * D + col0 + cb0 + kSub * c + li] = S[a][c][r];
                }
    }
}

// ---------------------------------------------------------------- launch sequence
// `ev`, when given, holds kNumStages + 1 events: ev[i] is recorded before
// stage i and ev[kNumStages] after the last one (a stage that does not run
// for these sizes still gets its pair of records, with nothing between them).
static ChunkOps chunk_ops(const Plan& p) {
    return ChunkOps{p.ws_TB, p.ws_M, p.ws_Qg, p.ws_Kg, p.ws_KhT, p.ws_gam, p.max_chunks, nullptr};
}
// the backward operand set (kda_chunk_bwd only)
static ChunkOps chunk_ops_bwd(const Plan& p) {
    return ChunkOps{p.ws_bTT, p.ws_bMT, p.ws_bKh, p.ws_bQgT, p.ws_bKgT, p.ws_gam, p.max_chunks, p.ws_bet};
}

// All chunks, or (equal lengths, nj > 0) chunks [j0, j0 + nj) of every sequence.
template <typename E, int D, bool kBoth, bool kLean = false>
static void launch_prep(const Plan& p, const E* q, hipStream_t st, int32_t j0 = 0, int32_t nj = 0,
                        bool xcd_hi = false) {
    if (p.total_tokens <= 0) return;
    int32_t grid = nj > 0 ? p.n_seqs * nj : p.max_chunks;
    if (xcd_hi) grid = 8 * ((grid + 3) / 4);
    hipLaunchKernelGGL((k_prep<E, D, kBoth, kLean>), dim3(grid, p.n_heads), dim3(kThreads), 0, st, q,
                       static_cast<const E*>(p.k), static_cast<const E*>(p.g), static_cast<const E*>(p.beta),
                       p.ws_tab, p.ws_n_chunks, p.cu_seqlens ? (int64_t)0 : p.fixed_len,
                       p.cu_seqlens ? 0 : (int32_t)(p.n_seqs * ((p.fixed_len + kChunk - 1) / kChunk)), p.n_heads,
                       chunk_ops(p), kBoth ? chunk_ops_bwd(p) : chunk_ops(p), j0, nj, (int32_t)xcd_hi);
}

// Chunks [jb, je) of every sequence (default: all of them).
template <int D, int kMode, int CT = 1, int XW = 1>
static void launch_recur_lds(const Plan& p, const void* v, const float* S0, float* ST, void* o, RecurAux aux,
                             hipStream_t st, int32_t jb = 0, int32_t je = 0x7fffffff, bool xcd_lo = false) {
    const int32_t NH = p.n_seqs * p.n_heads;
    aux.prog = p.ws_prog;
    hipLaunchKernelGGL((k_recur_lds<D, kMode, CT, XW>), dim3(NH * (D / (kSub * CT * XW)) * (xcd_lo ? 2 : 1)),
                       dim3((kRecurWaves * XW + kProducers + 1) * 64), 0, st,
                       static_cast<const __bf16*>(v), kMode == kBwd ? chunk_ops_bwd(p) : chunk_ops(p),
                       p.cu_seqlens, p.total_tokens, p.fixed_len, p.ws_seq_chunk0, NH, p.n_heads, S0, ST,
                       static_cast<__bf16*>(o), aux, jb, je, (int32_t)xcd_lo);
}

void launch_chunk_table(const Plan& p, int32_t chunk, hipStream_t st) {
    hipLaunchKernelGGL(k_chunk_table, dim3(1), dim3(1024), 0, st, p.cu_seqlens, p.n_seqs, p.total_tokens,
                       p.fixed_len, p.max_chunks, p.ws_tab, p.ws_seq_chunk0, p.ws_n_chunks,
                       p.S_ckpt ? p.ck_every : 0, p.ws_ck0, chunk);
}

static void launch_table(const Plan& p, hipStream_t st) { launch_chunk_table(p, kChunk, st); }

// ---------------------------------------------------------------- pipelined forward
// When the sequences have equal lengths and the recurrence's workgroups
// (one per sequence, head and 16-column slab) fill at most half of the CUs,
// the chunk-parallel k_prep of a token block runs on the idle CUs while the
// recurrence works on the block before it.  Block b's k_prep goes on a side
// stream that the library keeps per device; block b's recurrence waits for it
// on the caller's stream, takes its incoming state from the previous block
// (ws_state2, two fp32 buffers used in turn) and hands its final state on.
// k_prep of block b + 1 also waits for the recurrence of block b - 1, so
// that only one block of k_prep shares the GPU with a recurrence.
constexpr int kSideEvents = 96;
constexpr int kMaxDevices = 64;
constexpr int32_t kPipeMinChunks = 2048;   // per sequence
constexpr int32_t kPipeFirst = 256;        // chunks in the first block (its k_prep runs alone)
constexpr int32_t kPipeGrow = 150;         // each later block 1.5x the one before (64-chunk multiples) ...
constexpr int32_t kPipeBlock = 1536;       // ... up to this many chunks

struct SideStream {
    bool tried = false, ok = false;
    hipStream_t s = nullptr;
    hipEvent_t ev[kSideEvents] = {};
    int cus = 0;
};
static std::mutex g_side_mu;
static SideStream g_side[kMaxDevices];

// The current device's side stream (created on first use, default priority).
// Called with g_side_mu held.
static SideStream* side_stream() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    SideStream& ss = g_side[dev];
    if (!ss.tried) {
        ss.tried = true;
        bool ok = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) == hipSuccess;
        for (int i = 0; ok && i < kSideEvents; ++i)
            ok = hipEventCreateWithFlags(&ss.ev[i], hipEventDisableTiming) == hipSuccess;
        ok = ok && hipDeviceGetAttribute(&ss.cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess;
        ss.ok = ok;
    }
    return ss.ok ? &ss : nullptr;
}

// Block boundaries (in chunks of each sequence) for `per` chunks per sequence.
static int pipe_blocks(int32_t per, int32_t* j0, int max_blocks) {
    int32_t cap = kPipeBlock;
    int nb = 0;
    for (;;) {
        nb = 0;
        int32_t size = kPipeFirst;
        for (int32_t j = 0; j < per && nb <= max_blocks; j += size) {
            if (nb > 0) {
                const int32_t next = size * kPipeGrow / 100 / 64 * 64;
                size = next > cap ? cap : next;
            }
            j0[nb++] = j;
        }
        if (nb <= max_blocks) break;
        cap *= 2;
    }
    j0[nb] = per;
    return nb;
}

template <int D>
static bool launch_pipelined(const Plan& p, hipStream_t st) {
    constexpr int NS = D / kSub;
    if (p.no_pipeline || p.cu_seqlens || p.S_ckpt || !p.bf16 || p.total_tokens <= 0) return false;
    const int32_t per = (int32_t)((p.fixed_len + kChunk - 1) / kChunk);
    if (per < kPipeMinChunks) return false;
    std::lock_guard<std::mutex> lock(g_side_mu);
    SideStream* ss = side_stream();
    if (!ss || (int64_t)p.n_seqs * p.n_heads * NS * 2 > ss->cus) return false;
    constexpr int kMaxBlocks = (kSideEvents - 1) / 2;
    int32_t j0[kMaxBlocks + 2];
    const int nb = pipe_blocks(per, j0, kMaxBlocks);
    hipEvent_t* evp = ss->ev + 1;            // k_prep of block b done
    hipEvent_t* evr = ss->ev + 1 + nb;       // recurrence of block b done
    const __bf16* q = static_cast<const __bf16*>(p.q);
    const size_t state = (size_t)p.n_seqs * p.n_heads * D * D;
    if (hipEventRecord(ss->ev[0], st) != hipSuccess || hipStreamWaitEvent(ss->s, ss->ev[0], 0) != hipSuccess)
        return false;
    // On a device with 8 XCDs (256 CUs: workgroup i runs on XCD i mod 8),
    // the recurrence keeps XCDs 0..3 and the k_prep beside it XCDs 4..7, so
    // that the two do not share an L2 (1M tokens, 16 heads: 21.8 -> 18.6 ms
    // per pass).  Each kernel's workgroups that leave at once still need a
    // whole CU of the other half, so a kernel ends only once the other has
    // drained; the blocks grow by 1.5x (pipe_blocks), so that each k_prep
    // ends before the recurrence beside it (18.6 -> 18.4 ms).
    const bool xcd = ss->cus == 256 && (p.n_seqs * p.n_heads) % 4 == 0 &&
                     (int64_t)p.n_seqs * p.n_heads * NS <= ss->cus / 2;
    launch_prep<__bf16, D, false>(p, q, ss->s, j0[0], j0[1] - j0[0]);
    (void)hipEventRecord(evp[0], ss->s);
    for (int b = 0; b < nb; ++b) {
        if (b + 1 < nb) {
            if (b >= 1) (void)hipStreamWaitEvent(ss->s, evr[b - 1], 0);
            launch_prep<__bf16, D, false>(p, q, ss->s, j0[b + 1], j0[b + 2] - j0[b + 1], xcd);
            (void)hipEventRecord(evp[b + 1], ss->s);
        }
        (void)hipStreamWaitEvent(st, evp[b], 0);
        const float* s_in = b == 0 ? p.S0 : p.ws_state2 + (size_t)((b - 1) & 1) * state;
        float* s_out = b == nb - 1 ? p.S_T : p.ws_state2 + (size_t)(b & 1) * state;
        launch_recur_lds<D, kFwd>(p, p.v, s_in, s_out, p.o, RecurAux{}, st, j0[b], j0[b + 1], xcd);
        (void)hipEventRecord(evr[b], st);
    }
    return true;
}

// CUs of the current device (cached per device; 0 if unknown).
static int device_cus() {
    static std::atomic<int> cache[kMaxDevices];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c == 0 && hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
        cache[dev].store(c, std::memory_order_relaxed);
    return c;
}

template <typename E, int D, int kMode = kFwd>
static hipError_t launch_all(const Plan& p, hipStream_t st, hipEvent_t* ev) {
    auto mark = [&](int i) {
        if (ev) (void)hipEventRecord(ev[i], st);
    };
    constexpr int CT = 1;
    constexpr bool kTransition = kMode == kTrans;
    const E* q = static_cast<const E*>(kTransition ? p.k : p.q);   // the transition does not use q
    const int32_t NH = p.n_seqs * p.n_heads;

    if constexpr (kMode == kFwd && sizeof(E) == 2) {
        // the measurement entry point (ev) times the kernels one after another
        if (!ev && launch_pipelined<D>(p, st)) return hipGetLastError();
    }
    mark(0);
    if (p.cu_seqlens) launch_table(p, st);   // equal lengths: every kernel derives the chunks itself
    mark(1);
    launch_prep<E, D, false>(p, q, st);
    mark(2);
    static_assert(!kTransition || sizeof(E) == 2, "transition pass: bf16 operands only");
    if constexpr (sizeof(E) == 2) {
        if (kMode == kFwd && p.S_ckpt)
            launch_recur_lds<D, kFwdCk>(p, p.v, p.S0, p.S_T, p.o,
                                        RecurAux{nullptr, nullptr, nullptr, nullptr, p.S_ckpt, p.ck_every,
                                                 p.ck_slots, p.ws_ck0}, st);
        else if ((kMode == kFwd || kMode == kTrans) && (int64_t)NH * (D / kSub) > device_cus())
            // more 16-column chains than CUs: the throughput of the whole
            // chip, not one chain's latency, sets the time, and a 32-column
            // workgroup (two groups of compute waves) does two slabs' work
            // per chunk fill
            launch_recur_lds<D, kMode == kTrans ? kTrans : kFwd, 1, 2>(p, p.v, p.S0, p.S_T, p.o, RecurAux{}, st);
        else
            launch_recur_lds<D, kMode>(p, p.v, p.S0, p.S_T, p.o, RecurAux{}, st);
    }
    else
        hipLaunchKernelGGL((k_recur<E, D, CT>), dim3(NH * (D / (kSub * CT))), dim3(kThreads), 0, st,
                           static_cast<const E*>(p.v), chunk_ops(p), p.cu_seqlens, p.total_tokens, p.fixed_len,
                           p.ws_seq_chunk0, NH, p.n_heads, p.S0, p.S_T, static_cast<E*>(p.o));
    mark(3);
    return hipGetLastError();
}

const char* const kStageNames[kNumStages] = {"k_chunk_table", "k_prep", "k_recur"};

hipError_t launch(const Plan& p, hipStream_t st, hipEvent_t* ev) {
    if (p.generic) return launch_generic(p, st, ev);
    if (p.bf16) {
        if (p.d == 128) return launch_all<__bf16, 128>(p, st, ev);
        return launch_all<__bf16, 64>(p, st, ev);
    }
    // fp32 operands are built for d = 64 only; the C ABI rejects other sizes.
    return launch_all<float, 64>(p, st, ev);
}

hipError_t launch_transition(const Plan& p, hipStream_t st) {
    if (p.d == 128) return launch_all<__bf16, 128, kTrans>(p, st, nullptr);
    return launch_all<__bf16, 64, kTrans>(p, st, nullptr);
}

// Backward: both operand sets from one k_prep, forward again with
// checkpoints, the state-gradient recurrence, then the chunk-parallel
// gradients (kda_bwd.hip).
const char* const kBwdStageNames[kNumBwdStages] = {"k_chunk_table", "k_prep<fwd+bwd>", "k_recur_lds<ckpt>",
                                                   "k_recur_lds<bwd>", "k_grad", "k_dbeta_sum"};

// The chunk-parallel gradient kernels from the kept forward quantities.
template <int D>
static hipError_t launch_grads(const Plan& p, hipStream_t st, hipEvent_t ev_mid) {
    using E = __bf16;
    hipError_t e = hipGetLastError();
    GradArgs a{};
    if (e == hipSuccess && p.total_tokens > 0) {
        a.q = static_cast<const E*>(p.q);
        a.k = static_cast<const E*>(p.k);
        a.g = static_cast<const E*>(p.g);
        a.beta = static_cast<const E*>(p.beta);
        a.dO = static_cast<const E*>(p.dO);
        a.v = static_cast<const E*>(p.v);
        a.U = static_cast<const E*>(p.ws_U);
        a.dZ = static_cast<const E*>(p.ws_dZ);
        a.ckS = static_cast<const E*>(p.ws_ckS);
        a.ckdS = static_cast<const E*>(p.ws_ckdS);
        a.tab = p.ws_tab;
        a.n_chunks = p.ws_n_chunks;
        a.fixed_len = p.cu_seqlens ? (int64_t)0 : p.fixed_len;
        a.fixed_chunks = p.cu_seqlens ? 0 : (int32_t)(p.n_seqs * ((p.fixed_len + kChunk - 1) / kChunk));
        a.H = p.n_heads;
        a.max_chunks = p.max_chunks;
        a.total_tokens = p.total_tokens;
        a.dbp = p.ws_dbp;
        a.dq = static_cast<E*>(p.dq);
        a.dv = static_cast<E*>(p.dv);
        a.dk = static_cast<E*>(p.dk);
        a.dbeta = static_cast<E*>(p.dbeta);
        a.dg = static_cast<E*>(p.dg);
        e = launch_grad(a, D, p.max_chunks, st);
    }
    if (ev_mid) (void)hipEventRecord(ev_mid, st);
    if (e == hipSuccess && p.total_tokens > 0) e = launch_dbeta_sum(a, st);
    return e == hipSuccess ? hipGetLastError() : e;
}

template <int D>
static hipError_t launch_bwd_d(const Plan& p, hipStream_t st, hipEvent_t* ev) {
    using E = __bf16;
    auto mark = [&](int i) {
        if (ev) (void)hipEventRecord(ev[i], st);
    };
    mark(0);
    launch_table(p, st);
    mark(1);
    launch_prep<E, D, true, true>(p, static_cast<const E*>(p.q), st);
    mark(2);
    launch_recur_lds<D, kCkptLean>(p, p.v, p.S0, nullptr, nullptr,
                               RecurAux{static_cast<E*>(p.ws_ckS), nullptr, static_cast<E*>(p.ws_U), nullptr}, st);
    mark(3);
    launch_recur_lds<D, kBwd>(p, p.dO, p.dS_T, p.dS0, nullptr,
                              RecurAux{static_cast<E*>(p.ws_ckdS), static_cast<E*>(p.ws_dZ), nullptr, p.ws_bet}, st);
    mark(4);
    const hipError_t e = launch_grads<D>(p, st, ev ? ev[5] : nullptr);
    mark(6);
    return e;
}

// Training pair: the forward that keeps the backward's inputs in a context
// buffer, and the backward from that context.
template <int D>
static hipError_t launch_fwd_train_d(const Plan& p, hipStream_t st) {
    using E = __bf16;
    launch_table(p, st);
    launch_prep<E, D, true>(p, static_cast<const E*>(p.q), st);
    launch_recur_lds<D, kCkpt>(p, p.v, p.S0, p.S_T, p.o,
                               RecurAux{static_cast<E*>(p.ws_ckS), nullptr, static_cast<E*>(p.ws_U), nullptr}, st);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_ctx_d(const Plan& p, hipStream_t st) {
    using E = __bf16;
    launch_table(p, st);
    launch_recur_lds<D, kBwd>(p, p.dO, p.dS_T, p.dS0, nullptr,
                              RecurAux{static_cast<E*>(p.ws_ckdS), static_cast<E*>(p.ws_dZ), nullptr, p.ws_bet}, st);
    return launch_grads<D>(p, st, nullptr);
}

hipError_t launch_fwd_train(const Plan& p, hipStream_t st) {
    if (p.d == 128) return launch_fwd_train_d<128>(p, st);
    return launch_fwd_train_d<64>(p, st);
}

hipError_t launch_bwd_ctx(const Plan& p, hipStream_t st) {
    if (p.d == 128) return launch_bwd_ctx_d<128>(p, st);
    return launch_bwd_ctx_d<64>(p, st);
}

hipError_t launch_bwd(const Plan& p, hipStream_t st, hipEvent_t* ev) {
    if (p.d == 128) return launch_bwd_d<128>(p, st, ev);
    return launch_bwd_d<64>(p, st, ev);
}

}  // namespace kda
