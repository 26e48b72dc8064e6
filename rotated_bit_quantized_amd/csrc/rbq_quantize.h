// One cache row quantized and bit-packed by one wave64 (update_and_fetch
// on the quant_kv.py page, with the quantizer of mx.quantize): shared by the
// append kernel and by the attention kernel's fused append.
#pragma once

#include "rbq_common.h"

namespace rbq {

// min / max over the 16 lanes of a DPP row (one group of 64 values, 4 per
// lane): quad swaps, then the half-row and row mirrors; every lane ends with
// the result (min and max are exact, so the order does not matter).
// rint(fdiv_rn(x, s)), the code before clipping, with the correctly rounded
// division only where it can matter: q = x * rcp(s) is within a few ulp of
// x / s, so unless q lies within tol (at least 8 ulp) of a half-integer, the
// correctly rounded quotient rounds to the same integer.  Ties, near-ties
// and non-finite q (rcp of an fp32-denormal scale) take the exact division.
// A non-finite q is found from its exponent bits (an integer test), so that
// the decision holds in every translation unit, also one built with
// -fno-honor-nans, where a float compare against a NaN may be folded.
__device__ __forceinline__ float quant_code(float x, float s, float rinv) {
    const float q = x * rinv;
    const float fr = q - floorf(q);
    const float tol = fmaxf(fabsf(q), 1.0f) * 0x1p-20f;
    float c = rintf(q);
    const bool nonfinite = (__float_as_uint(q) & 0x7F800000u) == 0x7F800000u;
    const bool near = nonfinite || !(fabsf(fr - 0.5f) > tol);
    if (__any(near)) {  // rare: a wave-uniform branch, so the division is skipped otherwise
        if (near) c = rintf(__fdiv_rn(x, s));
    }
    return c;
}

template <int CTRL>
__device__ __forceinline__ float qdpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float qmin16(float x) {
    x = fminf(x, qdpp<0xB1>(x));   // quad_perm 1,0,3,2
    x = fminf(x, qdpp<0x4E>(x));   // quad_perm 2,3,0,1
    x = fminf(x, qdpp<0x141>(x));  // row_half_mirror
    return fminf(x, qdpp<0x140>(x));  // row_mirror
}
__device__ __forceinline__ float qmax16(float x) {
    x = fmaxf(x, qdpp<0xB1>(x));
    x = fmaxf(x, qdpp<0x4E>(x));
    x = fmaxf(x, qdpp<0x141>(x));
    return fmaxf(x, qdpp<0x140>(x));
}

// Quantize and pack one row of 256 values held 4 per lane.
// The arithmetic is the quantizer definition step by step, each step one
// IEEE fp32 operation: min/max (exact), (max - min) / (2^bits - 1) with a
// correctly rounded division, scale and bias rounded to the dtype, and
// rint((y - bias) / scale) clipped to [0, 2^bits - 1].
template <int DT, int BITS>
__device__ __forceinline__ void quantize_pack_row(const float y[4], int lane,
                                                  uint32_t* __restrict__ words,
                                                  uint16_t* __restrict__ scales,
                                                  uint16_t* __restrict__ biases) {
    constexpr float kLevels = (float)((1 << BITS) - 1);
    const float mn = qmin16(fminf(fminf(y[0], y[1]), fminf(y[2], y[3])));
    const float mx = qmax16(fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3])));
    const float s32 = __fdiv_rn(mx - mn, kLevels);
    const uint32_t s_bits = f32_to_elem_bits<DT>(s32);
    const uint32_t b_bits = f32_to_elem_bits<DT>(mn);
    const float s = elem_to_f32<DT>(s_bits);
    const float beta = elem_to_f32<DT>(b_bits);
    const float sdiv = (s == 0.0f) ? 1.0f : s;

    const float rinv = __builtin_amdgcn_rcpf(sdiv);
    uint32_t chunk = 0;  // 4 codes = 4*BITS bits, code i at bit BITS*i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float c = quant_code(y[i] - beta, sdiv, rinv);
        c = fminf(fmaxf(c, 0.0f), kLevels);
        chunk |= (uint32_t)c << (BITS * i);
    }

    // Lane j's chunk sits at stream bits [C*j, C*j + C), C = 4*BITS.  Lane w
    // (w < words per row) gathers every chunk overlapping bits [32w, 32w+32).
    constexpr int C = 4 * BITS;
    constexpr int kWords = 64 * C / 32;
    constexpr int kSpan = (32 + C - 1) / C + 1;  // max chunks touching one word
    const int w = lane < kWords ? lane : 0;
    const int j0 = (32 * w) / C;
    const int j1 = (32 * w + 31) / C;
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < kSpan; ++k) {
        const int j = j0 + k;
        const uint32_t val = __shfl(chunk, j < 64 ? j : 63);
        if (j <= j1) {
            const int sh = C * j - 32 * w;
            word |= sh >= 0 ? (val << sh) : (val >> (-sh));
        }
    }
    if (lane < kWords) words[lane] = word;

    const uint32_t sg = __shfl(s_bits, (lane & 3) * 16);
    const uint32_t bg = __shfl(b_bits, (lane & 3) * 16);
    if (lane < 4) {
        scales[lane] = (uint16_t)sg;
        biases[lane] = (uint16_t)bg;
    }
}

// The rotated row rounded to the input dtype (RBQ_FLAG_ROUND_ROTATED).
template <int DT>
__device__ __forceinline__ void round_row(float y[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = elem_to_f32<DT>(f32_to_elem_bits<DT>(y[i]));
}

}  // namespace rbq
