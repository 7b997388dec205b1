// mfma_util.h -- device helpers shared by the two matrix-core partial passes (splitkv_mfma.hip:
// 32-row work units on v_mfma_f32_32x32x16_bf16; splitkv_mfma16.hip: 16-row units on
// v_mfma_f32_16x16x32_bf16): vector types, cache loads, cross-lane reductions, bf16 rounding,
// the E4M3 decode and the LDS swizzle of the value tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ad {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// A row's reference max only moves when a score clears it by more than this (log2 units).
constexpr float kLazyRescale = 8.f;

__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
// Whole-row loads (ROWS form): the lanes that share a row read all of it in one instruction, so
// whole lines are read once and the loads are nontemporal.
__device__ __forceinline__ u32x4 ld16_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
// The last read of a line whose pieces several instructions read: nontemporal, the line is done
// then (an fp8 cache: 164 -> 150 us per step on the ragged paged fp8 cache; on bf16 caches the same
// hint measured within a few percent either way and is not used).
__device__ __forceinline__ u32x4 ld16_last(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Both lanes l and l^32 get max / sum of their two values.
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Both lanes l and l^16 get max / sum of their two values.
__device__ __forceinline__ float pair16_max(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {  // round to nearest even
    bf16x2 r;
    r.x = (__bf16)lo;
    r.y = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}

// Two OCP E4M3 bytes of w (bytes 0-1, or 2-3 with HI) as a bf16 pair (exact), as a 32-bit word.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pair(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// 8 E4M3 bytes (two words) as 8 bf16 values, in order.
__device__ __forceinline__ u32x4 e4m3_x8(uint32_t w0, uint32_t w1) {
    return u32x4{e4m3_pair<false>(w0), e4m3_pair<true>(w0), e4m3_pair<false>(w1), e4m3_pair<true>(w1)};
}

// 16-byte chunk position of chunk c of LDS row k (rows of D bf16). Rows 0..15 of a store land on
// 16 distinct chunk positions; the 4 rows x 2 chunks of one transposing read land on 8.
template <int D>
__device__ __forceinline__ int swz(int k) {
    return ((2 * (k & 7)) | ((k >> 3) & 1)) & (D / 8 - 1);
}

// Transposing LDS read (ds_read_b64_tr_b16): the 16 lanes of a row group each give the address of
// 4 consecutive bf16 of one LDS row (lane i: row i / 4, columns 4 (i % 4) .. + 3 of a 16-column
// block); lane i receives column i of the 4 rows, in row order.
__device__ __forceinline__ s16x4 ds_read_tr(const lds_u8 *at) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)at);
}

}  // namespace ad
