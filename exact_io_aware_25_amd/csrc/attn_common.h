// attn_common.h -- device and host helpers shared by the forward and the
// backward kernels (gfx950).  Internal to the library: not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowsPerWave = 32;
constexpr int kBlockK = 64;  // keys per K/V tile

template <typename T> struct Vec8;
template <> struct Vec8<_Float16> { typedef f16x8 type; };
template <> struct Vec8<__bf16> { typedef bf16x8 type; };

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}


// Row of the K tile that feeds A-operand row m: bits 2 and 3 swapped.  With
// this order, accumulator register r (0..15) of lane half `hi` in a 32-key
// block holds key 16*(r/8) + 8*hi + r%8, i.e. 8 consecutive keys per 16-key
// slice -- the layout the B operand of the second product needs.
__device__ __forceinline__ int k_row_for_lane(int m)
{
    return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

template <bool CAUSAL, bool WINDOW>
__device__ __forceinline__ bool visible(int i, int j, int L, int window)
{
    if (j >= L) return false;
    if (CAUSAL && j > i) return false;
    if (WINDOW) {
        if (i - j > window) return false;
        if (!CAUSAL && j - i > window) return false;
    }
    return true;
}

// XOR swizzles of the 16-byte units of each LDS tile row (tiles are not
// padded).  A row of D 16-bit values has D/8 units; unit u of row r is stored
// at unit u ^ f(r).  The functions are chosen so that both reads are free of
// bank conflicts whether the LDS serves 8 lanes x 16 bytes (32 banks) or 16
// lanes x 16 bytes (64 banks) per cycle:
//  * K is read 16 bytes per lane from the 16 rows k_row_for_lane(0..15) of a
//    32-row block, all at the same logical unit: f must be a bijection on row
//    bits {0,1,3} (the first 8 of those rows) and on bits {1,2,3} for a fixed
//    bit 0 (16 rows over two 128-byte halves);
//  * V is read 8 bytes per lane by the transposing load, four consecutive rows
//    at a time with two (16 lanes) or four (32 lanes) consecutive units per
//    row: f must move the unit pair, and for 32 lanes the unit quad, of each
//    of the four rows to a different place.
template <int D> __device__ __forceinline__ int k_swizzle(int row)
{
    const int b0 = row & 1, b1 = (row >> 1) & 1, b2 = (row >> 2) & 1, b3 = (row >> 3) & 1;
    return (b0 ^ b2) | (b1 << 1) | (b3 << 2) | (D == 128 ? (b2 << 3) : 0);
}
template <int D> __device__ __forceinline__ int v_swizzle(int row)
{
    const int c = row & 3;
    return (c << 1) | (D == 128 ? ((c & 1) << 3) : 0);
}

// Copy 16 bytes per lane from a buffer into LDS without passing through
// VGPRs: lane i's bytes land at lds_dst + 16*i (lds_dst is wave-uniform).
__device__ __forceinline__ void copy_to_lds16(__amdgpu_buffer_rsrc_t src, void *lds_dst, int src_offset)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void *)lds_dst, 16,
                                             src_offset, 0, 0, 0);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposing 8-byte LDS read: within each group of 16 lanes, lane 4a+b gets
// element b of the 8-byte chunks addressed by lanes a, a+4, a+8 and a+12.
__device__ __forceinline__ s16x4 lds_read_tr16(const void *generic_lds_ptr)
{
    auto p = (__attribute__((address_space(3))) char *)(generic_lds_ptr);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
}

__device__ __forceinline__ float half_swap_max(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float sum8(f16x8 v, float acc)
{
    const f16x2 one = {1, 1};
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
    return __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
}

// XOR swizzle for a tile that is read both ways: 16 bytes per lane from the
// rows k_row_for_lane(0..31) (as K above) and by the transposing load from
// four consecutive rows (as V above).  Found by exhaustive search over the
// linear (XOR) functions of the row bits under both LDS bank models: for
// d=64 f = b1 | (b0^b2)<<1 | (b1^b3)<<2, for d=128
// f = b0 | b1<<1 | (b0^b3)<<2 | (b1^b2)<<3.  It depends on bit 2 of the row,
// so the second transposing read (rows +4) needs its own offset.
template <int D> __device__ __forceinline__ int dual_swizzle(int row)
{
    const int b0 = row & 1, b1 = (row >> 1) & 1, b2 = (row >> 2) & 1, b3 = (row >> 3) & 1;
    if (D == 64) return b1 | ((b0 ^ b2) << 1) | ((b1 ^ b3) << 2);
    return b0 | (b1 << 1) | ((b0 ^ b3) << 2) | ((b1 ^ b2) << 3);
}

// Do the byte ranges [a, a+na) and [b, b+nb) overlap?
inline bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return na && nb && pa < pb + nb && pb < pa + na;
}

}  // namespace
