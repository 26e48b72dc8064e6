// One cache row quantized and bit-packed by one wave64 (update_and_fetch
// on the quant_kv.py page, with the quantizer of mx.quantize): shared by the
// append kernel and by the attention kernel's fused append.
#pragma once

#include "rbq_common.h"

namespace rbq {

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
    float mn = fminf(fminf(y[0], y[1]), fminf(y[2], y[3]));
    float mx = fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3]));
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, m));
        mx = fmaxf(mx, __shfl_xor(mx, m));
    }
    const float s32 = __fdiv_rn(mx - mn, kLevels);
    const uint32_t s_bits = f32_to_elem_bits<DT>(s32);
    const uint32_t b_bits = f32_to_elem_bits<DT>(mn);
    const float s = elem_to_f32<DT>(s_bits);
    const float beta = elem_to_f32<DT>(b_bits);
    const float sdiv = (s == 0.0f) ? 1.0f : s;

    uint32_t chunk = 0;  // 4 codes = 4*BITS bits, code i at bit BITS*i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float c = rintf(__fdiv_rn(y[i] - beta, sdiv));
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
