// Device helpers shared by the librbq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rbq_internal.h"

namespace rbq {

// ---- element conversions (exact widening; round-half-even narrowing) ----

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t u) { return __uint_as_float(u << 16); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t u) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)u);
}

template <int DT>
__device__ __forceinline__ float elem_to_f32(uint32_t u) {
    if constexpr (DT == RBQ_BF16) return bf16_bits_to_f32(u & 0xFFFFu);
    else return f16_bits_to_f32(u & 0xFFFFu);
}

// fp32 -> bf16 bits, round half to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// fp32 -> fp16 bits, round half to even (the hardware conversion in the
// default rounding mode; subnormal halves are kept).  The empty asm makes the
// fp32 value opaque: without it the compiler turned an fp64 -> fp32 rounding
// followed by this one into a single fp64 -> fp16 rounding, which differs
// where the two roundings compound (rotated rows rounded to fp16).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
    asm("" : "+v"(f));
    const _Float16 h = (_Float16)f;
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

template <int DT>
__device__ __forceinline__ uint32_t f32_to_elem_bits(float f) {
    if constexpr (DT == RBQ_BF16) return f32_to_bf16_bits(f);
    else return f32_to_f16_bits(f);
}

// ---- one 4-block of the SO(4) rotation ----
// y[j] = fp32(((x0*B[0][j] + x1*B[1][j]) + x2*B[2][j]) + x3*B[3][j]) in fp64.
// Every product of an fp16/bf16/fp32 value with an fp32 entry is exact in
// fp64, so fusing a product into the following add does not change a result.
__device__ __forceinline__ void rotate4(const float x[4], const float Bm[16], float y[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        double s = (double)x[0] * (double)Bm[j];
        s = s + (double)x[1] * (double)Bm[4 + j];
        s = s + (double)x[2] * (double)Bm[8 + j];
        s = s + (double)x[3] * (double)Bm[12 + j];
        y[j] = (float)s;
    }
}

// Inverse of rotate4 for one block: z[i] = fp32(sum_j y[j] * B[i][j]) in fp64.
__device__ __forceinline__ void unrotate4(const float y[4], const float Bm[16], float z[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        double s = (double)y[0] * (double)Bm[4 * i];
        s = s + (double)y[1] * (double)Bm[4 * i + 1];
        s = s + (double)y[2] * (double)Bm[4 * i + 2];
        s = s + (double)y[3] * (double)Bm[4 * i + 3];
        z[i] = (float)s;
    }
}

__device__ __forceinline__ void load_block(const float* __restrict__ rot, int blk, float Bm[16]) {
    if (rot != nullptr) {
        const float4* p = reinterpret_cast<const float4*>(rot + blk * 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float4 v = p[r];
            Bm[4 * r] = v.x;
            Bm[4 * r + 1] = v.y;
            Bm[4 * r + 2] = v.z;
            Bm[4 * r + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) Bm[e] = (e % 5 == 0) ? 1.0f : 0.0f;
    }
}

// Mean of the dequantised values c * s + b of column `col` over the keys
// [0, n) of one (b, kv head) slab whose first row is `row0` (n >= 1), summed
// in fp64 in key order and rounded once to fp32.  The SDPA on the quant_kv.py
// page fills the scores a boolean mask drops with the dtype's most negative
// value before its softmax, so a query row whose every key is dropped weights
// all of its keys alike: its output is this mean.  The attention kernels skip
// dropped keys, find such a row (no key kept, row sum 0) in their last stage
// and take this loop there instead; it runs only for such rows.
//   vw [rows][vwords] packed V words (little-endian bit stream of vbits-bit
//   codes), vs / vb [rows][ng] V scales and biases of groups of gs columns.
template <int DT>
__device__ float value_column_mean(const uint32_t* vw, const uint16_t* vs,
                                                const uint16_t* vb, int64_t row0, int n, int col,
                                                int vbits, int vwords, int ng, int gs) {
    const int p = vbits * col, wi = p >> 5, sh = p & 31;
    const bool straddle = sh + vbits > 32;
    const uint32_t m = (1u << vbits) - 1u;
    const int g = col / gs;
    double s = 0.0;
    for (int t = 0; t < n; ++t) {
        const int64_t r = row0 + t;
        const uint32_t* w = vw + r * vwords;
        uint32_t bits = w[wi] >> sh;
        if (straddle) bits |= w[wi + 1] << (32 - sh);
        const double c = (double)(bits & m);
        s += c * (double)elem_to_f32<DT>(vs[r * ng + g]) + (double)elem_to_f32<DT>(vb[r * ng + g]);
    }
    return (float)(s / (double)n);
}

// Four consecutive input elements (8 bytes, 8-byte aligned) as floats.
template <int DT>
__device__ __forceinline__ void load4(const uint16_t* __restrict__ p, float x[4]) {
    const uint2 raw = *reinterpret_cast<const uint2*>(p);
    x[0] = elem_to_f32<DT>(raw.x);
    x[1] = elem_to_f32<DT>(raw.x >> 16);
    x[2] = elem_to_f32<DT>(raw.y);
    x[3] = elem_to_f32<DT>(raw.y >> 16);
}

}  // namespace rbq
