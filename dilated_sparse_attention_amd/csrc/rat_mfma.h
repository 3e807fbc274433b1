// MFMA tiles shared by the attention kernels (gfx950): the bf16 MFMA
// 16x16x32 and the XOR-swizzled LDS row tiles its fragments are read from.
//
// v_mfma_f32_16x16x32_bf16, D = A B + C (16 x 16, k = 32): lane (g, i),
// g = lane / 16, i = lane % 16, holds A[row i][k 8g .. 8g+7], B[k 8g .. 8g+7]
// [col i] and D[rows 4g .. 4g+3][col i].
#pragma once

#include "rat_device.h"

namespace rat {

typedef __attribute__((address_space(3))) shortx4 lds_s4;

__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}


template <int DK>
struct Geo {
    static constexpr int CH = DK / 8;           // 16-byte chunks per row
    static constexpr int ROWB = DK * 2;         // bytes per bf16 row
    static constexpr int KS = DK / 32;          // 32-dim k-steps of QK^T
    static constexpr int DB = DK / 16;          // 16-dim blocks of the output
    static constexpr int RPI = 1024 / ROWB;     // rows per 1 KiB wave load
};

// XOR key of row r: the low bits of r rotated left by one.  Over any CH
// consecutive rows it is a permutation (conflict-free K-fragment reads of
// one logical chunk), and over CH/2 consecutive rows it maps the chunk pair
// (2j, 2j+1) onto CH distinct chunks (conflict-free transposing V reads).
template <int DK>
__host__ __device__ __forceinline__ int swz_key(int r)
{
    constexpr int HALF = Geo<DK>::CH / 2;
    return ((r & (HALF - 1)) << 1) | ((r / HALF) & 1);
}

// byte offset of chunk c of row r in a swizzled tile
template <int DK>
__host__ __device__ __forceinline__ int swz(int r, int c)
{
    return r * Geo<DK>::ROWB + ((c ^ swz_key<DK>(r)) << 4);
}

__device__ __forceinline__ bf16x8 lds_b128(const lds_char* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ shortx4 lds_tr(const lds_char* p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)p);
}

}  // namespace rat
