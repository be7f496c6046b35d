// KDA backward: the per-chunk gradient kernel (gfx950).
//
// The backward pass of the chunkwise forward (ogis-ri NLP primer on Kimi K3,
// §3.1 "KDA": the chunked form; orkas.ai "Kimi K3 architecture",
// §"GPU のコードパスを一本消した「下界」": the 16-token sub-tiles) runs as
//   k_prep + k_recur_lds<kCkpt>  forward again, keeping per chunk the
//                                incoming state S and per token U~ = T diag(beta) Y
//                                with Y = V - (K.Gamma)S
//   k_prep<kBwd> + k_recur_lds<kBwd>  the state-gradient recurrence, last
//                                chunk first: dZ = T^T dU~ per token, the
//                                outgoing-state gradient dS' per chunk, dS0
//   k_grad (here)                everything else, chunk-parallel, dv = diag(beta) dZ
//                                included.
//
// Per chunk (b = cumsum of log alpha inside the chunk, Gamma = exp(b),
// gamma = Gamma at the last token, K^ = K . exp(b_L - b), dY = dv):
//   d(Q.Gamma) = dO S^T     d(K.Gamma) = -dY S^T     dK^ = U~ dS'^T   (dY = diag(beta) dZ)
//   dgamma_c = sum_j dS'_cj S_cj
//   dA  = -tril(dZ U~^T, -1)    (= -T^T dU~ Z^T T^T with Z = diag(beta) Y)
//   dGq =  tril(dO U~^T)
//   dbeta_r = sum_j dZ_rj Y_rj + sum_{i<r} dA_ri Gk_ri
// Y itself is not kept: its term is sum_j dZ_rj V_rj - sum_c (K.Gamma)_rc (dZ S^T)_rc,
// the second sum split between the two channel halves like the other products.
// where Gk and Gq are the decayed Gram matrices sum_c x_rc k_ic exp(b_rc - b_ic)
// of K and Q with K (A = diag(beta) Gk, M = Gq).  Their gradients reach the
// tokens' q, k and b:
//   row side    dKr = diag(beta) dKrA,  dKrA_rc = sum_i dA_ri k_ic e^{b_rc - b_ic}
//               dQr_rc = sum_i dGq_ri k_ic e^{b_rc - b_ic}
//   column side dKc_ic = sum_r (beta_r dA_ri k_rc + dGq_ri q_rc) e^{b_rc - b_ic}
// and sum_i dA_ri Gk_ri = sum_c k_rc dKrA_rc gives the second dbeta term.
// db collects every e^{+-b} factor's derivative; dg is its reverse
// cumulative sum over the chunk (b is the cumulative sum of g).
//
// Decay factors follow the forward's sub-tiling: with rho_R = b at the end of
// sub-tile R-1, every MFMA operand carries a factor <= 1 and the remaining
// factor in [1, e^80] is applied to the fp32 result:
//   row side, r in R, i in J <= R:
//     e^{b_r - b_i} = e^{b_r - rho_{R+1}} . e^{rho_{R+1} - rho_{J+1}} . e^{rho_{J+1} - b_i}
//   column side, i in J, r in R >= J:
//     e^{b_r - b_i} = e^{b_r - rho_R} . e^{rho_R - rho_J} . e^{rho_J - b_i}
//
// Geometry: two workgroups of 4 waves per (chunk, head), one per half of
// the key channels (both halves of a chunk run on the same XCD, so the token
// rows they both read come from one L2).  Wave w handles the chunk's token
// tile w.  Every product is formed transposed (rows = key channels, columns
// = tokens), so that lane 16 lg + li ends up holding token 16w + li and
// channels 16n + 4lg + r (n among the half's tiles, r < 4) of every result:
// the decay cumulative sum over tokens is a 16-lane row scan, and all
// per-element terms combine in registers.  The two halves' shares of dbeta
// meet in a float32 workspace; k_dbeta_sum adds them.  The results leave
// through LDS as whole 16-byte vectors per token row.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int kGradThreads = 256;

// 8 bf16 from LDS, each scaled by s in fp32, as an MFMA fragment
__device__ inline bf16x8 load_scaled(const __bf16* p, float s) {
    bf16x8 f = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (__bf16)((float)f[e] * s);
    return f;
}

__device__ inline bf16x8 as_frag(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

template <int D>
__global__ __launch_bounds__(kGradThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_grad(GradArgs a) {
    using E = __bf16;
    using M = Mma<E>;
    using F = M::frag;
    constexpr int C = kChunk;
    constexpr int HALF = D / 2;       // key channels per workgroup
    constexpr int NTH = HALF / 16;    // channel tiles per workgroup
    constexpr int CH = 4 * NTH;       // channels per lane
    constexpr int KV = D / M::KS;     // k-steps of a contraction over value columns
    constexpr int PSd = D + 8;        // pitch of the staged U~ rows (elements)
    constexpr int PT = C + 8;         // pitch of token-indexed rows
    constexpr int PO = HALF + 8;      // pitch of the output staging rows
    constexpr int kXs = 2 * HALF * D, kXu = C * PSd, kXg = 3 * HALF * PT, kXo = 3 * C * PO;
    constexpr int kX01 = kXs > kXu ? kXs : kXu, kX23 = kXg > kXo ? kXg : kXo;
    constexpr int kX = kX01 > kX23 ? kX01 : kX23;
    // Region X: the half's rows of S and dS' (state_swz layout, copied as
    // stored); then U~ ([token][value column]); then the Gram operands
    // ([channel][token]); last the outputs ([token][channel]).
    __shared__ __attribute__((aligned(16))) E sX[kX];
    __shared__ __attribute__((aligned(16))) E sdA[C * PT];     // dA      [r][i]
    __shared__ __attribute__((aligned(16))) E sdGq[C * PT];    // dGq     [r][i]
    __shared__ __attribute__((aligned(16))) E sdGkT[C * PT];   // beta dA [i][r]
    __shared__ __attribute__((aligned(16))) E sdGqT[C * PT];   // dGq     [i][r]
    __shared__ float sRho[(kNSub + 1) * HALF];   // rho_0 .. rho_3, b_L
    __shared__ float sTot[kNSub * HALF];         // sub-tile sums of log alpha
    __shared__ float sCol[kNSub * HALF];         // per tile: sum over tokens of dK^ . K^
    __shared__ float sRev[kNSub * HALF];         // per tile: sum of db
    __shared__ float sDgam[HALF];
    __shared__ float sCs[HALF];                  // the b_L terms of the chunk's last row, per channel
    __shared__ float sBeta[C];
    E* sS = sX;
    E* sdS = sX + HALF * D;
    E* sU = sX;
    E* sKD = sX;                  // k_i e^{rho_{J+1} - b_i}
    E* sKr = sX + HALF * PT;      // k_r e^{b_r - rho_R}
    E* sQr = sX + 2 * HALF * PT;  // q_r e^{b_r - rho_R}

    // workgroup -> (chunk, half): the two halves of 8 consecutive chunks sit
    // 8 workgroups apart, so that they share an XCD
    const int32_t bid = blockIdx.x;
    const int32_t ci = (bid & 7) + 8 * (bid >> 4);
    const int hh = (bid >> 3) & 1;
    ChunkInfo info;
    if (a.fixed_len > 0) {
        const int32_t per = (int32_t)((a.fixed_len + C - 1) / C);
        if (ci >= a.fixed_chunks) return;
        const int32_t seq = ci / per, j = ci % per;
        const int64_t rem = a.fixed_len - (int64_t)j * C;
        info.tok0 = (int64_t)seq * a.fixed_len + (int64_t)j * C;
        info.seq = seq;
        info.len = (int32_t)(rem < C ? rem : C);
    } else {
        if (ci >= *a.n_chunks) return;
        info = a.tab[ci];
    }
    const int h = blockIdx.y, len = info.len, H = a.H;
    const int tid = threadIdx.x, w = tid >> 6;
    const int lane = tid & 63, li = lane & 15, lg = lane >> 4;
    const int t = kSub * w + li;
    const bool ok = t < len;
    const int64_t rs = (int64_t)H * D;
    // this lane's token row; rows past the chunk end read the chunk's first
    // row (a valid address) and are zeroed in registers
    const int64_t row = (info.tok0 + (ok ? t : 0)) * rs + (int64_t)h * D;
    const int64_t slot = (int64_t)h * a.max_chunks + ci;
    auto lch = [&](int i, int r) { return kSub * i + 4 * lg + r; };   // local channel in the half
    const int c0 = hh * HALF;

    // ---- every load is issued before any is used
    // the half's rows of S and dS' go global -> LDS by direct loads, 1 KB per wave instruction
    {
        constexpr int kVec = HALF * D / 8;   // 16-byte vectors per matrix
        const E* gS = a.ckS + slot * D * D + (int64_t)c0 * D;
        const E* gD = a.ckdS + slot * D * D + (int64_t)c0 * D;
#pragma unroll
        for (int v0 = w * 64; v0 < kVec; v0 += kGradThreads) {
            __builtin_amdgcn_global_load_lds(gS + 8 * (v0 + lane), (__attribute__((address_space(3))) void*)(sS + 8 * v0), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(gD + 8 * (v0 + lane), (__attribute__((address_space(3))) void*)(sdS + 8 * v0), 16, 0, 0);
        }
    }
    uint2 rq[NTH], rk[NTH], rg[NTH];
#pragma unroll
    for (int i = 0; i < NTH; ++i) {
        const int64_t at = row + c0 + lch(i, 0);
        rq[i] = *reinterpret_cast<const uint2*>(a.q + at);
        rk[i] = *reinterpret_cast<const uint2*>(a.k + at);
        rg[i] = *reinterpret_cast<const uint2*>(a.g + at);
    }
    const E beta_raw = a.beta[(info.tok0 + (ok ? t : 0)) * H + h];
    // token rows of dO, U~, dZ (and V) as fragments over value columns
    uint4 fo[KV], fu[KV], fz[KV], fv[KV];
#pragma unroll
    for (int m = 0; m < KV; ++m) {
        const int64_t at = row + M::KS * m + M::KW * lg;
        fo[m] = *reinterpret_cast<const uint4*>(a.dO + at);
        fu[m] = *reinterpret_cast<const uint4*>(a.U + at);
        fz[m] = *reinterpret_cast<const uint4*>(a.dZ + at);
        if (hh == 0) fv[m] = *reinterpret_cast<const uint4*>(a.v + at);
    }
    // ---- zero the rows past the chunk end (bit masks: no branches, so the
    // loads above stay in flight until their first use)
    const unsigned msk = ok ? 0xffffffffu : 0u;
    const float okf = ok ? 1.f : 0.f;
    auto mask4 = [&](uint4& u) { u.x &= msk; u.y &= msk; u.z &= msk; u.w &= msk; };
    float qf[CH], kf[CH], b[CH];
#pragma unroll
    for (int i = 0; i < NTH; ++i) {
        const E* eq = reinterpret_cast<const E*>(&rq[i]);
        const E* ek = reinterpret_cast<const E*>(&rk[i]);
        const E* eg = reinterpret_cast<const E*>(&rg[i]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            qf[4 * i + r] = (float)eq[r] * okf;
            kf[4 * i + r] = (float)ek[r] * okf;
            b[4 * i + r] = (float)eg[r] * okf;
        }
    }
    const float bt = (float)beta_raw * okf;
    float dbeta = 0.f;
#pragma unroll
    for (int m = 0; m < KV; ++m) {
        mask4(fo[m]);
        mask4(fu[m]);
        mask4(fz[m]);
    }
    if (hh == 0) {   // dv = beta dZ, and sum_j dZ_tj V_tj of the first dbeta term (the other half adds none)
#pragma unroll
        for (int m = 0; m < KV; ++m) {
            const bf16x8 zf = as_frag(fz[m]), yf = as_frag(fv[m]);
            bf16x8 dvf;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                dbeta += (float)zf[e] * (float)yf[e];
                dvf[e] = (E)(bt * (float)zf[e]);
            }
            if (ok) *reinterpret_cast<bf16x8*>(a.dv + row + M::KS * m + M::KW * lg) = dvf;
        }
        dbeta += __shfl_xor(dbeta, 16);
        dbeta += __shfl_xor(dbeta, 32);
    }
    // decay cumulative sum: 16-lane row scan, carries between token tiles
#pragma unroll
    for (int x = 0; x < CH; ++x) b[x] = row_scan16(b[x]);
    if (lg == 0) sBeta[t] = bt;
    if (li == 15) {
#pragma unroll
        for (int i = 0; i < NTH; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) sTot[w * HALF + lch(i, r)] = b[4 * i + r];
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the direct loads into LDS have landed
    __syncthreads();
    for (int c = tid; c < HALF; c += kGradThreads) {
        float run = 0.f;
#pragma unroll
        for (int R = 0; R < kNSub; ++R) {
            sRho[R * HALF + c] = run;
            run += sTot[R * HALF + c];
        }
        sRho[kNSub * HALF + c] = run;
    }
    // dgamma_c = sum_j dS'_cj S_cj (the row's vectors in any order: both
    // matrices carry the same permutation)
    {
        constexpr int TPC = kGradThreads / HALF;   // threads per channel
        constexpr int VPT = D / 8 / TPC;           // 16-byte vectors per thread
        const int c = tid / TPC, part = tid % TPC;
        float acc = 0.f;
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const bf16x8 xs = *reinterpret_cast<const bf16x8*>(&sS[c * D + 8 * (part * VPT + v)]);
            const bf16x8 xd = *reinterpret_cast<const bf16x8*>(&sdS[c * D + 8 * (part * VPT + v)]);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc += (float)xs[e] * (float)xd[e];
        }
#pragma unroll
        for (int o = 1; o < TPC; o <<= 1) acc += __shfl_xor(acc, o);
        if (part == 0) sDgam[c] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NTH; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) b[4 * i + r] += sRho[w * HALF + lch(i, r)];

    // ---- products with the states: d(Q.Gamma), dK^ and dZ S^T, which gives
    // d(K.Gamma) = -dY S^T = -diag(beta) dZ S^T and the rest of the first
    // dbeta term
    float dq[CH], dk[CH], db[CH];
    float dbeta2 = 0.f;
#pragma unroll
    for (int i = 0; i < NTH; ++i) {
        f32x4 aq = zero4(), ah = zero4(), az = zero4();
#pragma unroll
        for (int m = 0; m < KV; ++m) {
            // row kSub*i + li, vector 4m + lg, permuted by the row (state_swz)
            const int at = (kSub * i + li) * D + ((((M::KS * m + M::KW * lg) >> 3) ^ (li & (D / 8 - 1))) << 3);
            const F fs = M::load(&sS[at]);
            const F fd = M::load(&sdS[at]);
            aq = M::mma(fs, as_frag(fo[m]), aq);
            az = M::mma(fs, as_frag(fz[m]), az);
            ah = M::mma(fd, as_frag(fu[m]), ah);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int x = 4 * i + r, c = lch(i, r);
            const float G = __expf(b[x]), eh = __expf(sRho[kNSub * HALF + c] - b[x]);
            const float dqg = aq[r], dkg = -bt * az[r], dkh = ah[r];
            dq[x] = dqg * G;
            dk[x] = dkg * G + dkh * eh;
            const float kz = kf[x] * G * az[r];   // (K.Gamma) . (dZ S^T)
            dbeta2 -= kz;
            const float hk = dkh * kf[x] * eh;    // dK^ . K^
            db[x] = dqg * qf[x] * G - bt * kz - hk;
            const float cs = row_scan16(hk);      // column sum over the tile's tokens
            if (li == 15) sCol[w * HALF + c] = cs;
        }
    }
    __syncthreads();   // S and dS' are dead: region X takes U~
#pragma unroll
    for (int m = 0; m < KV; ++m) *reinterpret_cast<uint4*>(&sU[t * PSd + M::KS * m + M::KW * lg]) = fu[m];
    __syncthreads();
    // ---- dA and dGq, row block w (blocks above the diagonal are written as zero)
#pragma unroll
    for (int J = 0; J < kNSub; ++J) {
        f32x4 accA = zero4(), accG = zero4();
        if (J <= w) {
#pragma unroll
            for (int m = 0; m < KV; ++m) {
                const F fj = M::load(&sU[(kSub * J + li) * PSd + M::KS * m + M::KW * lg]);
                accA = M::mma(as_frag(fz[m]), fj, accA);
                accG = M::mma(as_frag(fo[m]), fj, accG);
            }
        }
        bf16x4 tk, tq;   // rows 4lg .. 4lg+3 of column ii: consecutive in the transposes
        const int ii = kSub * J + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rr = kSub * w + 4 * lg + r;
            const float dA = ii < rr ? -accA[r] : 0.f;
            const float dG = ii <= rr ? accG[r] : 0.f;
            sdA[rr * PT + ii] = (E)dA;
            sdGq[rr * PT + ii] = (E)dG;
            tk[r] = (E)(sBeta[rr] * dA);
            tq[r] = (E)dG;
        }
        *reinterpret_cast<bf16x4*>(&sdGkT[ii * PT + kSub * w + 4 * lg]) = tk;
        *reinterpret_cast<bf16x4*>(&sdGqT[ii * PT + kSub * w + 4 * lg]) = tq;
    }
    __syncthreads();   // U~ is dead: region X takes the Gram operands
    // the b_L terms of the last row (sDgam and every tile's sCol are final):
    // one thread per channel, so that the last row's lane only adds them
    for (int c = tid; c < HALF; c += kGradThreads) {
        float cs = sDgam[c] * __expf(sRho[kNSub * HALF + c]);
#pragma unroll
        for (int W = 0; W < kNSub; ++W) cs += sCol[W * HALF + c];
        sCs[c] = cs;
    }
#pragma unroll
    for (int i = 0; i < NTH; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int x = 4 * i + r, c = lch(i, r);
            const float r0 = sRho[w * HALF + c], r1 = sRho[(w + 1) * HALF + c];
            sKD[c * PT + t] = (E)(kf[x] * __expf(r1 - b[x]));
            sKr[c * PT + t] = (E)(kf[x] * __expf(b[x] - r0));
            sQr[c * PT + t] = (E)(qf[x] * __expf(b[x] - r0));
        }
    __syncthreads();

    // ---- Gram gradients
#pragma unroll
    for (int i = 0; i < NTH; ++i) {
        const int cA = kSub * i + li;   // local channel of this lane's A-operand row
        // row side: output tokens r in tile R = w; contraction over i in blocks J <= R
        f32x4 accK = zero4(), accQ = zero4();
        {
            const int R = w;
            const float rR1 = sRho[(R + 1) * HALF + cA];
            for (int m = 0; m <= R / 2; ++m) {
                const int J = 2 * m + (lg >> 1);
                const float fac = J <= R ? __expf(rR1 - sRho[(J + 1) * HALF + cA]) : 1.f;
                const F fa = load_scaled(&sKD[cA * PT + M::KS * m + M::KW * lg], fac);
                accK = M::mma(fa, M::load(&sdA[(kSub * w + li) * PT + M::KS * m + M::KW * lg]), accK);
                accQ = M::mma(fa, M::load(&sdGq[(kSub * w + li) * PT + M::KS * m + M::KW * lg]), accQ);
            }
        }
        // column side: output tokens i in tile J = w; contraction over r in blocks R >= J
        f32x4 accC = zero4();
        {
            const int J = w;
            const float rJ = sRho[J * HALF + cA];
            for (int m = J / 2; m < C / M::KS; ++m) {
                const int R = 2 * m + (lg >> 1);
                const float fac = R > J ? __expf(sRho[R * HALF + cA] - rJ) : 1.f;
                const int at = cA * PT + M::KS * m + M::KW * lg;
                const int bt_at = (kSub * w + li) * PT + M::KS * m + M::KW * lg;
                accC = M::mma(load_scaled(&sKr[at], fac), M::load(&sdGkT[bt_at]), accC);
                accC = M::mma(load_scaled(&sQr[at], fac), M::load(&sdGqT[bt_at]), accC);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int x = 4 * i + r, c = lch(i, r);
            const float orow = __expf(b[x] - sRho[(w + 1) * HALF + c]);
            const float ocol = __expf(sRho[w * HALF + c] - b[x]);
            const float dkra = accK[r] * orow, dqr = accQ[r] * orow, dkc = accC[r] * ocol;
            const float dkr = bt * dkra;
            dq[x] += dqr;
            dk[x] += dkr + dkc;
            db[x] += kf[x] * (dkr - dkc) + qf[x] * dqr;
            dbeta2 += kf[x] * dkra;
        }
    }
    dbeta2 += __shfl_xor(dbeta2, 16);
    dbeta2 += __shfl_xor(dbeta2, 32);
    dbeta += dbeta2;

    // ---- b_L terms on the last row, then dg = reverse cumulative sum of db
    float rv[CH];
#pragma unroll
    for (int i = 0; i < NTH; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int x = 4 * i + r, c = lch(i, r);
            if (t == C - 1) db[x] += sCs[c];
            rv[x] = row_rscan16(db[x]);
            if (li == 0) sRev[w * HALF + c] = rv[x];
        }
    __syncthreads();   // also: every wave is past the Gram products, so region X is free
    // dq, dk, dlog_alpha of the half go through region X ([token][channel],
    // pitch PO) so that each token's 64 channels leave as whole 16-byte vectors
    E* sOq = sX;
    E* sOk = sX + C * PO;
    E* sOg = sX + 2 * C * PO;
#pragma unroll
    for (int i = 0; i < NTH; ++i) {
        bf16x4 oq, ok4, og;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int x = 4 * i + r, c = lch(i, r);
            float dgv = rv[x];
            // the later token tiles' totals (a fixed-length loop: every wave
            // issues the same loads at once, whatever its tile)
#pragma unroll
            for (int W = 1; W < kNSub; ++W) dgv += W > w ? sRev[W * HALF + c] : 0.f;
            oq[r] = (E)dq[x];
            ok4[r] = (E)dk[x];
            og[r] = (E)dgv;
        }
        *reinterpret_cast<bf16x4*>(&sOq[t * PO + lch(i, 0)]) = oq;
        *reinterpret_cast<bf16x4*>(&sOk[t * PO + lch(i, 0)]) = ok4;
        *reinterpret_cast<bf16x4*>(&sOg[t * PO + lch(i, 0)]) = og;
    }
    if (lg == 0 && ok) a.dbp[((int64_t)hh * H + h) * a.total_tokens + info.tok0 + t] = dbeta;   // [2][H][T]
    __syncthreads();
    {
        constexpr int VR = HALF / 8;   // 16-byte vectors per token row of the half
        for (int vi = tid; vi < 3 * C * VR; vi += kGradThreads) {
            const int m = vi / (C * VR), tt = (vi / VR) % C, v = vi % VR;
            if (tt >= len) continue;
            const E* src = (m == 0 ? sOq : m == 1 ? sOk : sOg) + tt * PO + 8 * v;
            E* dst = (m == 0 ? a.dq : m == 1 ? a.dk : a.dg) + (info.tok0 + tt) * rs + (int64_t)h * D + c0 + 8 * v;
            store_nt(dst, *reinterpret_cast<const uint4*>(src));   // streamed: read next by the caller
        }
    }
}

// dbeta[t][h] = the two halves' float32 shares ([2][H][T]), rounded once to bf16
__global__ __launch_bounds__(256) void k_dbeta_sum(const float* __restrict__ dbp, int64_t T, int32_t H,
                                                   __bf16* __restrict__ dbeta) {
    const int64_t n = T * H;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t h = i / T, t = i % T;   // i runs over the shares' layout, so their reads coalesce
        dbeta[t * H + h] = (__bf16)(dbp[i] + dbp[n + i]);
    }
}

hipError_t launch_grad(const GradArgs& a, int d, int32_t max_chunks, hipStream_t st) {
    if (max_chunks <= 0) return hipSuccess;
    // two workgroups per chunk, in groups of 16 (8 chunks x 2 halves)
    const int32_t groups = (max_chunks + 7) / 8;
    const dim3 grid(16 * groups, a.H);
    if (d == 128)
        hipLaunchKernelGGL(k_grad<128>, grid, dim3(kGradThreads), 0, st, a);
    else
        hipLaunchKernelGGL(k_grad<64>, grid, dim3(kGradThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_dbeta_sum(const GradArgs& a, hipStream_t st) {
    const int64_t n = a.total_tokens * a.H;
    const int64_t blocks = (n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192;
    if (n > 0) hipLaunchKernelGGL(k_dbeta_sum, dim3((unsigned)blocks), dim3(256), 0, st, a.dbp, a.total_tokens, a.H,
                                  a.dbeta);
    return hipGetLastError();
}

}  // namespace kda
