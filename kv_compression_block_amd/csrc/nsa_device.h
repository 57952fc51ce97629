// Device helpers shared by the gfx950 kernels: vector types, the two element
// types (bfloat16 and float16: widening, packing, MFMA), cross-lane helpers.
// gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nsa_internal.h"

namespace nsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two floats -> two bf16 in one word (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D(32x32, f32) += A(32x16, bf16) * B(16x32, bf16).
// Lane l holds A[l%32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l%32] as the
// same k-slots; D element (row, col) sits in lane col + 32*((row/4)%2),
// register 4*(row/8) + row%4.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// The element types of q, k, v and the compression weight.  Tensors hold
// raw 16-bit patterns (uint16_t); a kernel templated on one of these structs
// widens them to float32, packs float32 pairs back (round to nearest even)
// and feeds eight-element operands to the 32x32x16 MFMA of that type (both
// MFMAs share the lane layout described at mfma32).
struct ElemBf16 {
    static constexpr int code = 0;
    __device__ static __forceinline__ float lo(uint32_t w) { return bf16_lo(w); }
    __device__ static __forceinline__ float hi(uint32_t w) { return bf16_hi(w); }
    __device__ static __forceinline__ float widen(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
    __device__ static __forceinline__ uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }
    __device__ static __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

struct ElemF16 {
    static constexpr int code = 1;
    __device__ static __forceinline__ float widen(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
    __device__ static __forceinline__ float lo(uint32_t w) { return widen((uint16_t)(w & 0xFFFFu)); }
    __device__ static __forceinline__ float hi(uint32_t w) { return widen((uint16_t)(w >> 16)); }
    __device__ static __forceinline__ uint32_t pack2(float lo, float hi)
    {
        f16x2 v = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
    __device__ static __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};

// Combine a value with the one held by the lane 32 positions away.
// The max as a compare and a select: equal to fmaxf for any two values that
// are not NaN, without the two quieting instructions fmaxf needs for
// operands that come out of a lane exchange.
__device__ __forceinline__ float half_max(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
    return a > b ? a : b;
}

__device__ __forceinline__ float half_sum(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Base-2 log-normaliser of a softmax row from its natural-unit max m and its
// sum L of exp(score - m): the row's probability is then
// exp2(score * |scale| * log2(e) - bias).  +inf (probability 0) for a row
// that sees nothing (L = 0).  The attention epilogue and the importance pass
// both derive it here, so either may compute it for the other.
__device__ __forceinline__ float row_bias(float m, float L)
{
    return L > 0.f ? fmaf(m, 1.4426950408889634f, __builtin_amdgcn_logf(L)) : __builtin_inff();
}

// Buffer resource over [base, base + bytes): raw (unstrided) loads at byte
// offsets >= bytes return zero, so a tile that runs past the end of its rows
// needs neither a clamp nor a branch per load.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voffset)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voffset, 0, 0);
}

// 16-byte chunk c of V row r sits at chunk v_swz(r, c) of that row.  The
// P.V operand reads (ds_read_b64_tr_b16) touch 8 consecutive rows and 4
// consecutive chunks per instruction; this XOR spreads them over all 64
// banks twice, the minimum for 512 bytes.
template <int D2>
__device__ __forceinline__ int v_swz(int r, int c)
{
    if constexpr (D2 == 128)
        return c ^ ((r & 3) << 2);
    else
        return c ^ (((r >> 1) & 1) << 2);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Copies 16 bytes per lane from a buffer into LDS: lane i's bytes land at
// lds + 16 i (the LDS address must be the same in every lane).
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}

// Largest b with tile_off(b) <= tile: tile ranges are ascending in b.
template <bool kAttn>
__device__ __forceinline__ int find_batch(const BatchEnt* bt, int B, int tile)
{
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        int off = kAttn ? bt[mid].tile_off_a : bt[mid].tile_off_c;
        if (off <= tile)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// Compressed blocks visible to local position t: i*d + l - 1 <= t.
__device__ __forceinline__ int n_visible(int t, int l, int d, int n_cmp)
{
    if (t < l - 1)
        return 0;
    int n = (t - l + 1) / d + 1;
    return n < n_cmp ? n : n_cmp;
}

}  // namespace nsa
