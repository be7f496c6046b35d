// Device-side building blocks shared by the KDA kernels (gfx950 / CDNA4).
//
// Matrix-core fragments.  Every contraction is built from 16x16 output tiles
// of `v_mfma_f32_16x16x32_bf16` (bf16 operands) or `v_mfma_f32_16x16x4_f32`
// (fp32 operands), accumulating in fp32.  For a 64-lane wave with
// lane = 16 * g + i (i in [0,16), g in [0,4)):
//   A fragment : A[i][k0 + g*KW + j],  j in [0, KW)    (row i of the tile)
//   B fragment : B[k0 + g*KW + j][i]                   (column i of the tile)
//   accumulator: acc[r] = D[4*g + r][i],  r in [0, 4)
// A and B fragments use the same k mapping, so any lane/k arrangement the
// hardware applies inside one instruction cancels out in the sum.  B operands
// are therefore staged "n-major" (one row per output column, k contiguous),
// which makes both fragment loads contiguous KW-element reads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;      // tokens per chunk
constexpr int kSub = 16;        // tokens per sub-tile (one MFMA tile edge)
constexpr int kNSub = kChunk / kSub;
constexpr int kThreads = 256;   // 4 waves per workgroup

template <typename E> struct Mma;

template <> struct Mma<__bf16> {
    static constexpr int KS = 32;   // k per instruction
    static constexpr int KW = 8;    // k elements per lane
    using frag = bf16x8;
    __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static inline frag load(const __bf16* p) {
        return *reinterpret_cast<const bf16x8*>(p);
    }
};

template <> struct Mma<float> {
    static constexpr int KS = 4;
    static constexpr int KW = 1;
    using frag = float;
    __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    __device__ static inline frag load(const float* p) { return *p; }
};

// fp32 16x16x4 step used where the operands are fp32 regardless of the
// input dtype (the triangular inverse).
__device__ inline f32x4 mma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ inline f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// 16-byte store / load with the non-temporal hint, for data that this kernel
// touches once (the next reader is another kernel).
typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));
__device__ inline void store_nt(void* p, uint4 v) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_nt, v), static_cast<u32x4_nt*>(p));
}
__device__ inline uint4 load_nt(const void* p) {
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(static_cast<const u32x4_nt*>(p)));
}

template <typename E> __device__ inline float to_f(E x) { return static_cast<float>(x); }
template <typename E> __device__ inline E from_f(float x) { return static_cast<E>(x); }

__device__ inline int lane_id() { return threadIdx.x & 63; }

// Layout of a d x d bf16 state kept for the backward pass (row = key
// channel, d = 64 or 128): row-major, with the 16-byte vectors of row c
// permuted by XOR with c mod (d/8).  Copied linearly into LDS, the A-operand
// reads of 16 consecutive rows at one k-step then touch 16 distinct vector
// positions, i.e. different banks.  Element index of (c, col):
template <int D>
__device__ inline int state_swz(int c, int col) {
    return c * D + ((((col >> 3) ^ (c & (D / 8 - 1)))) << 3) + (col & 7);
}

// Scans along the 16 lanes of a DPP row (lanes 16g .. 16g+15), zero fill:
// row_scan16 is the inclusive prefix sum, row_rscan16 the inclusive suffix sum.
template <int kShift>
__device__ inline float row_shr(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 | kShift, 0xf, 0xf, true));
}
template <int kShift>
__device__ inline float row_shl(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x100 | kShift, 0xf, 0xf, true));
}
__device__ inline float row_scan16(float x) {
    x += row_shr<1>(x);
    x += row_shr<2>(x);
    x += row_shr<4>(x);
    x += row_shr<8>(x);
    return x;
}
__device__ inline float row_rscan16(float x) {
    x += row_shl<1>(x);
    x += row_shl<2>(x);
    x += row_shl<4>(x);
    x += row_shl<8>(x);
    return x;
}
__device__ inline int wave_id() { return threadIdx.x >> 6; }

}  // namespace kda
