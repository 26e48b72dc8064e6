// General fused attention over the quantized cache (asym_quantized_sdpa on
// the quant_kv.py page, with the SO(4) rotation of q on entry and the inverse
// rotation of the output), for every supported configuration: head_dim 64,
// 128 or 256, group 32, 64 or 128, K and V widths 2, 3, 4, 5, 6 or 8 bits,
// and any number of query rows per kv head (G = H_q / H_kv x L, up to
// prefill-length blocks).
//
// Decomposition, three shapes, one workgroup per (b, kv head, block of
// query rows, key split), walking 32-key tiles:
// - four waves, 64 query rows (long blocks): wave w owns rows 16 w .. 16 w +
//   15 of the block; all 256 threads decode each tile into LDS once (K and V
//   codes as fp16 [key][dim]; scales and biases as fp32 [group][key]) from
//   a staging array filled by direct-to-LDS transfers one tile ahead, then
//   every wave with a live row runs its 16 rows against it;
// - one wave, up to 16 rows (short blocks): the same per wave;
// - one wave, up to 8 rows, 4-bit K codes and 2- to 4-bit V codes at
//   head_dim 64 or 128 (register-staged): each lane loads the packed words
//   of its units straight into registers two tiles ahead; the hi and lo
//   parts of the 8 query rows share one operand (rows 0-7 and 8-15) and K
//   codes enter the score MFMAs in place (nibble pairs masked as fp16
//   subnormals, the query operand permuted and scaled to match).
// V codes are converted once per tile to fp16 (exact: integers below 2^11),
// so the operand reads need no conversion.  (V codes taken as fp16
// subnormals, c * 2^-24, lose precision in the matrix cores when the other
// operand spans a wide range, as the probabilities do.)
//
// All products run as 16x16x32 MFMAs.  Lane l = 16 j + n: operand lanes hold
// row / column n and the 8 k-slots 8 j .. 8 j + 7 (the same slots in A and
// B, so the k order within them does not matter); accumulator lane (j, n)
// holds rows 4 j .. 4 j + 3 of column n.
// Scores: A = query rows, rotated, times scale * log2(e) and a per-row power
//   of two 2^E that puts the largest |q| in [2^14, 2^15), split into an fp16
//   hi and lo part (two MFMAs, or one with paired rows); B = K codes.  One accumulator per group g of
//   the row: score = 2^-E sum_g s_g acc_g + sum_g b_g (sum_{d in g} q_d),
//   folded on the vector units (base-2 scores).
// Values: A = P' = p s_{t,g} 2^F_g (the probability times the key's value
//   scale, with a per-tile, per-group power of two that puts the largest
//   scale in [2^14, 2^15)), split hi + lo; B = V codes of 8 keys x 16 columns
//   (a transposed byte read).  Each tile's product is folded into the output
//   accumulators with the softmax rescale and 2^-F_g; the group bias
//   enters as sum_t p_t b_{t,g}, kept per lane and reduced at the end.
// Online softmax in base 2 over the tile's 32 keys per row.  Every workgroup
// stores a record (m, l, unnormalised o) per row; a second kernel merges the
// key splits, normalises, rotates back and stores the fp32 output.
// Precondition of the fp16 value path: V codes times 2^F stay finite, i.e.
// no V scale is inf or NaN; tiny scales next to large ones in a tile lose
// relative precision below 2^-22 of the tile's largest P'.
#include <hip/hip_runtime.h>

#include "rbq_common.h"

namespace rbq {
namespace {

typedef _Float16 tf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 tf16x2 __attribute__((ext_vector_type(2)));
typedef float tf32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t tu32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t tu32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t tu32x3 __attribute__((ext_vector_type(3)));

constexpr int tTile = 32;                  // keys per tile
constexpr int tCPolNT = 2;                 // tile transfers: non-temporal (read once per call)
constexpr int tPS = tTile + 4;             // floats per row of a wave's P staging
constexpr float tLog2e = 1.44269504088896340736f;

// LDS of a workgroup of W waves (16 query rows each), NG groups per row.
// RK (register-staged shape): the K rows hold the packed 4-bit words as they
// are (D / 8 words, padded to D / 8 + 4: conflict-free 4-byte reads of 16
// keys x 4 words), the codes entering the matrix cores in place.
template <int D, int W, int NG, bool RK = false>
struct TileLds {
    static constexpr int KS = RK ? D / 2 + 16 : 2 * D + 16;            // bytes per key row of K codes
    static constexpr int VS = 2 * D + 32;                               // bytes per key row of V codes
    static constexpr int kc = 0;                                        // K codes, fp16 [32][KS / 2]
    static constexpr int vc = kc + tTile * KS;                          // V codes, fp16 [32][VS / 2]
    static constexpr int ksl = vc + tTile * VS;                         // fp32 [NG][32] K scales
    static constexpr int kbl = ksl + NG * tTile * 4;                    // K biases
    static constexpr int vsf = kbl + NG * tTile * 4;                    // V scales x 2^F
    static constexpr int vbl = vsf + NG * tTile * 4;                    // V biases
    static constexpr int vinv = vbl + NG * tTile * 4;                   // 2^-F per group
    static constexpr int vres = vinv + NG * 4;                          // 2^(F_new - F_old) per group
    static constexpr int pst = vres + NG * 4;                           // [W waves][16][tPS] fp32
    static constexpr int qst = pst + W * 16 * tPS * 4;                  // [W waves][NG groups][16 rows]
    static constexpr int frw = qst + W * NG * 16 * 4;                   // [W waves][16] 2^-E
    static constexpr int bytes = frw + W * 16 * 4;
};

struct TArgs {
    const uint16_t* q;
    const uint32_t* kw;
    const uint16_t* ks;
    const uint16_t* kb;
    const uint32_t* vw;
    const uint16_t* vs;
    const uint16_t* vb;
    const float* rot;
    float* rec_o;   // [units][S][RW rows][D]
    float* rec_ml;  // [units][S][RW rows][2]
    float* out;     // with one split the workgroups store the output directly
    int64_t capacity;
    int T, chunk, S, Hkv, n_rep, L, G, RBW, causal, round_rot;
    int GS, kbits, vbits;
    float qscale;  // scale * log2(e)
    int raw_vw, raw_meta;  // staging offsets of the V words and the scale / bias arrays
    const void* mask;
    int64_t msb, msh, msl;  // elements; key stride 1
    uint32_t mask_bytes;
    int mtype;  // 0 none, 1 bool (uint8), 2 fp32 additive, 3 dtype additive
};

__device__ __forceinline__ tf32x4 tmfma(tf16x8 a, tf16x8 b, tf32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 4 code bytes -> 4 fp16 codes, exact: the half with bits 0x6400 | c is
// 1024 + c, and 1024 is subtracted two halves at a time.
__device__ __forceinline__ tu32x2 bytes_f16(uint32_t d) {
    const tf16x2 k = {(_Float16)-1024.0f, (_Float16)-1024.0f};
    const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, d, 0x04010400u);
    const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, d, 0x04030402u);
    return (tu32x2){__builtin_bit_cast(uint32_t, __builtin_bit_cast(tf16x2, lo) + k),
                    __builtin_bit_cast(uint32_t, __builtin_bit_cast(tf16x2, hi) + k)};
}

template <int CTRL>
__device__ __forceinline__ float tdpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float tmax16(float x) {
    x = fmaxf(x, tdpp<0xB1>(x));
    x = fmaxf(x, tdpp<0x4E>(x));
    x = fmaxf(x, tdpp<0x141>(x));
    return fmaxf(x, tdpp<0x140>(x));
}
__device__ __forceinline__ float tsum16(float x) {
    x += tdpp<0xB1>(x);
    x += tdpp<0x4E>(x);
    x += tdpp<0x141>(x);
    return x + tdpp<0x140>(x);
}

// The 32 codes of BITS bits held in BITS consecutive words (stream bits
// [0, 32 BITS) of the words), as 8 words of 4 bytes: byte b of word i is code
// 4 i + b.  Code j sits at stream bits [BITS j, BITS j + BITS), little-endian.
template <int BITS>
__device__ __forceinline__ void unpack32(const uint32_t w[8], uint32_t out[8]) {
    if constexpr (BITS == 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = w[i];
    } else if constexpr (BITS == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = w[i] & 0x0F0F0F0Fu;          // codes 8i, 8i+2, 8i+4, 8i+6
            const uint32_t hi = (w[i] >> 4) & 0x0F0F0F0Fu;   // codes 8i+1, 8i+3, ...
            out[2 * i] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
            out[2 * i + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
        }
    } else {
        constexpr uint32_t m = (1u << BITS) - 1u;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t d = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int p = BITS * (4 * i + b);
                const int wi = p >> 5, sh = p & 31;
                uint32_t c;
                if (sh + BITS <= 32) c = (w[wi] >> sh) & m;
                else c = __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & m;
                d |= c << (8 * b);
            }
            out[i] = d;
        }
    }
}

__device__ __forceinline__ void unpack32_any(int bits, const uint32_t w[8], uint32_t out[8]) {
    switch (bits) {
        case 2: unpack32<2>(w, out); break;
        case 3: unpack32<3>(w, out); break;
        case 4: unpack32<4>(w, out); break;
        case 5: unpack32<5>(w, out); break;
        case 6: unpack32<6>(w, out); break;
        default: unpack32<8>(w, out); break;
    }
}

typedef __attribute__((address_space(3))) unsigned char tlds_u8;

// Raw tile staging (a separate LDS array, filled by direct-to-LDS loads: the
// compiler can then tell its transfers from every other LDS access): the
// tile's K words at 0, V words at raw_vw (key-major, as in memory) and its
// four scale / bias arrays [key][group], 16-bit, at raw_meta.  Sized by the
// call's widths (dynamic LDS): 32 keys x D x bits / 8 bytes per word array.
template <int D, int NG>
struct RawLds {
    static constexpr int meta_bytes = 64 * NG;      // one scale / bias array
};
__host__ __device__ constexpr int raw_vw_off(int D, int kbits) { return 4 * D * kbits; }
__host__ __device__ constexpr int raw_meta_off(int D, int kbits, int vbits) {
    return 4 * D * (kbits + vbits);
}
__host__ __device__ constexpr int raw_bytes(int D, int NG, int kbits, int vbits) {
    return raw_meta_off(D, kbits, vbits) + 4 * 64 * NG;
}

// Buffer resources of one (b, kv head) slab: the six arrays from row 0,
// ranges T rows (keys past T read as zero).
struct TRsrc {
    __amdgpu_buffer_rsrc_t kw, vw, m[4];
    bool k16, v16;  // 16-byte transfers of the word arrays, else 4-byte
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tmake_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// Issue the direct-to-LDS transfers of the tile at key t0 (wave `wave` of
// W takes every W-th instruction; each instruction moves 64 lanes x 16 or 4
// bytes to consecutive LDS bytes).
template <int D, int NG, int W>
__device__ __forceinline__ void issue_tile(const TArgs& a, const TRsrc& rs, int t0, int wave,
                                           int lane, tlds_u8* rawb) {
    using R = RawLds<D, NG>;
    // fully unrolled over the largest instruction counts (8-bit codes), each
    // instruction predicated on a uniform condition (a loop around the
    // transfers makes the compiler wait for the earlier ones at its head);
    // one lane offset per array, the instruction's chunk in the scalar offset
    constexpr int kMax16 = D / 32;  // 16-byte instructions of one word array
    constexpr int kMax4 = D / 8;    // 4-byte instructions of one word array
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
        const int words = kv ? D * a.vbits / 32 : D * a.kbits / 32;
        const __amdgpu_buffer_rsrc_t r = kv ? rs.vw : rs.kw;
        tlds_u8* dst = rawb + (kv ? a.raw_vw : 0);
        const uint32_t base = (uint32_t)t0 * words * 4u;
        if (kv ? rs.v16 : rs.k16) {
            const int nch = 8 * words;  // 16-byte chunks of the tile
            const uint32_t voff = base + 16u * lane;
#pragma unroll
            for (int m = 0; m < kMax16; ++m)
                if (m % W == wave && 64 * m < nch && (64 * m + 64 <= nch || lane < nch - 64 * m))
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst + 1024 * m, 16, voff, 1024 * m, 0, tCPolNT);
        } else {
            const int nch = 32 * words;  // 4-byte chunks
            const uint32_t voff = base + 4u * lane;
#pragma unroll
            for (int m = 0; m < kMax4; ++m)
                if (m % W == wave && 64 * m < nch && (64 * m + 64 <= nch || lane < nch - 64 * m))
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst + 256 * m, 4, voff, 256 * m, 0, tCPolNT);
        }
    }
    // the four scale / bias arrays: 32 keys x NG halves each = 16 NG words
    // (NG = 1: 2-byte rows, loaded into registers instead, as a 4-byte chunk
    // could straddle the end of row T - 1)
    if constexpr (NG > 1) {
        const uint32_t moff = (uint32_t)t0 * NG * 2u + 4u * lane;
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int h = 0; h < (16 * NG + 63) / 64; ++h)
                if ((4 * k + h) % W == wave && 64 * h + lane < 16 * NG)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.m[k], rawb + a.raw_meta + k * R::meta_bytes + 256 * h,
                                                              4, moff, 256 * h, 0, tCPolNT);
    }
}

// NG = 1: the scale / bias halves of key t0 + m (m < 32) into registers.
__device__ __forceinline__ void load_meta1(const TArgs& a, int64_t row0, int t0, int m, uint32_t meta[4]) {
    const int t = t0 + m;
    const uint16_t* src[4] = {a.ks, a.kb, a.vs, a.vb};
#pragma unroll
    for (int i = 0; i < 4; ++i) meta[i] = (t < a.T) ? src[i][row0 + t] : 0u;
}

// The packed words of unit u (u < D: K unit u, else V unit u - D; unit v of
// a row covers key v / (D / 32), codes 32 (v % (D / 32)) .. + 31).
template <int D, int NG>
__device__ __forceinline__ void read_unit(const TArgs& a, const unsigned char* rawb, int u,
                                          uint32_t w[8]) {
    using R = RawLds<D, NG>;
    constexpr int upk = D / 32;
    const bool isv = u >= D;
    const int uu = isv ? u - D : u;
    const int key = uu / upk, part = uu - key * upk;
    const int bits = isv ? a.vbits : a.kbits;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(rawb + (isv ? a.raw_vw : 0)) +
                          key * (D * bits / 32) + part * bits;
    // consecutive lanes read consecutive units (bits words apart): 2-, 4- and
    // 8-bit units as whole 8- or 16-byte reads (word reads at a stride of 4
    // or 8 words would hit the same banks), the others word by word (odd
    // strides spread over all banks)
    if (bits == 4) {
        const tu32x4 v = *reinterpret_cast<const tu32x4*>(src);
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = v[i];
#pragma unroll
        for (int i = 4; i < 8; ++i) w[i] = 0u;
    } else if (bits == 8) {
        const tu32x4 v0 = *reinterpret_cast<const tu32x4*>(src);
        const tu32x4 v1 = *reinterpret_cast<const tu32x4*>(src + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[i] = v0[i];
            w[4 + i] = v1[i];
        }
    } else if (bits == 2) {
        const tu32x2 v = *reinterpret_cast<const tu32x2*>(src);
        w[0] = v[0];
        w[1] = v[1];
#pragma unroll
        for (int i = 2; i < 8; ++i) w[i] = 0u;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = (i < bits) ? src[i] : 0u;
    }
}

// K and V codes of the tile into LDS as fp16 [key][dim], from the staged
// words: units u = tid, tid + threads, ...
template <int D, int W, int NG>
__device__ __forceinline__ void store_units(const TArgs& a, const unsigned char* rawb, int tid,
                                            unsigned char* smem) {
    using Ly = TileLds<D, W, NG>;
    constexpr int upk = D / 32;
#pragma unroll
    for (int u = tid; u < 2 * D; u += 64 * W) {
        {
            const bool isv = u >= D;
            const int uu = isv ? u - D : u;
            const int key = uu / upk, part = uu - key * upk;
            uint32_t w[8];
            read_unit<D, NG>(a, rawb, u, w);
            uint32_t c[8];
            unpack32_any(isv ? a.vbits : a.kbits, w, c);
            tu32x2 h[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) h[i] = bytes_f16(c[i]);
            tu32x4* dst = reinterpret_cast<tu32x4*>(
                smem + (isv ? Ly::vc + key * Ly::VS : Ly::kc + key * Ly::KS) + 64 * part);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dst[i] = (tu32x4){h[2 * i][0], h[2 * i][1], h[2 * i + 1][0], h[2 * i + 1][1]};
        }
    }
}

// Scale / bias item m of the staged tile: group m / 32, key m % 32.
template <int D, int NG>
__device__ __forceinline__ void read_meta(const unsigned char* rawb, int raw_meta, int m,
                                          uint32_t meta[4]) {
    using R = RawLds<D, NG>;
    const int g = m / tTile, key = m - g * tTile;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        meta[i] = (g < NG) ? *reinterpret_cast<const uint16_t*>(rawb + raw_meta + i * R::meta_bytes +
                                                                  2 * (key * NG + g))
                           : 0u;
}

// Per (group, key) the K scale and bias and the V bias as fp32, and the V
// scale times 2^F_g, with F_g the running power of two of group g: chosen
// so that the largest V scale seen so far, times 2^F_g, lies in [2^14,
// 2^15); when a tile raises that largest scale, F_g drops and vres[g] =
// 2^(F_new - F_old) tells the waves to rescale the output columns of group g
// (1 otherwise).  f_run is this thread's copy of F_g (1000 = no nonzero
// scale yet).  Called by all 64 lanes of a wave with items m = 64 q + lane
// (the maximum is a butterfly over the 32 lanes of a group).
template <int DT, int D, int W, int NG, bool RK = false>
__device__ __forceinline__ void store_meta(const uint32_t meta[4], int m, unsigned char* smem,
                                           int& f_run) {
    using Ly = TileLds<D, W, NG, RK>;
    const int g = m / tTile, key = m - g * tTile;
    const bool live = g < NG;
    const float s_v = elem_to_f32<DT>(meta[2]);
    // the maximum over the 32 lanes of a group: over each 16-lane row by DPP,
    // then across the row pair by one row swap
    float mx = tmax16(live ? fabsf(s_v) : 0.f);
    const auto rsw = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(rsw[0]), __uint_as_float(rsw[1]));
    int ex = 0;
    if (mx > 0.f) (void)frexpf(mx, &ex);
    const int f_new = (mx > 0.f) ? min(f_run, 15 - ex) : f_run;
    if (live) {
        float* f = reinterpret_cast<float*>(smem);
        f[Ly::ksl / 4 + g * tTile + key] = elem_to_f32<DT>(meta[0]);
        f[Ly::kbl / 4 + g * tTile + key] = elem_to_f32<DT>(meta[1]);
        f[Ly::vsf / 4 + g * tTile + key] = (f_new == 1000) ? 0.f : ldexpf(s_v, f_new);
        f[Ly::vbl / 4 + g * tTile + key] = elem_to_f32<DT>(meta[3]);
        if (key == 0) {
            f[Ly::vinv / 4 + g] = (f_new == 1000) ? 1.f : ldexpf(1.0f, -f_new);
            f[Ly::vres / 4 + g] = (f_run == 1000 || f_new == f_run) ? 1.f : ldexpf(1.0f, f_new - f_run);
        }
    }
    f_run = f_new;
}

// (hi, lo) fp16 pairs of x0, x1: hi rounded toward zero by the packed
// conversion, lo = fp16(x - hi) by one mixed-precision FMA per half
// (x - hi is exact in fp32).
__device__ __forceinline__ tu32x2 split_f16(float x0, float x1, float one) {
    const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x0, x1));
    uint32_t lo;
    asm("v_fma_mixlo_f16 %0, -%1, %2, %3 op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixhi_f16 %0, -%1, %2, %4 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "=&v"(lo)
        : "v"(hi), "v"(one), "v"(x0), "v"(x1));
    return (tu32x2){hi, lo};
}

// 4 halves of the transposing LDS read: lane i of each 16-lane group gets
// element i & 3 of the 8 bytes addressed by lanes 4 e + (i >> 2), e = 0..3.
__device__ __forceinline__ tu32x2 tr16_read(const unsigned char* p) {
    typedef short ts16x4 __attribute__((ext_vector_type(4)));
    const ts16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) ts16x4*)((__attribute__((address_space(3))) unsigned char*)p));
    return __builtin_bit_cast(tu32x2, v);
}

// Single-wave workgroups with the widths fixed at compile time (KB, VB > 0,
// head_dim up to 128): each lane loads the packed words of the units it
// decodes, and the scale / bias halves of its items, straight into
// registers, two tiles ahead (two register sets), instead of through an LDS
// staging array: the compiler then tracks every load by its registers and
// waits for exactly the tile it decodes, and the LDS a staging array would
// take is left for more workgroups per compute unit.  Lane l holds units
// l * UPL .. l * UPL + UPL - 1 of K and of V, all of one key: its words are
// one contiguous piece of the tile, loaded whole (past the buffer's range,
// keys at or after T, it reads as zero).
template <int D, int NG, int KB, int VB>
struct RegTile {
    static constexpr int UPL = D / 64;               // K (and V) units per lane
    static constexpr int NKW = UPL * KB, NVW = UPL * VB;
    static constexpr int NIT = (32 * NG + 63) / 64;  // scale / bias items per lane
    uint32_t kw[NKW];
    uint32_t vw[NVW];
    uint32_t meta[NIT][4];
};

// N consecutive words at byte offset off of buffer r, in as few loads as
// their count allows (non-temporal, as the staged transfers)
template <int N>
__device__ __forceinline__ void load_words(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t* w) {
#pragma unroll
    for (int i = 0; i + 4 <= N; i += 4) {
        const tu32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 4 * i, 0, tCPolNT);
        w[i] = v[0];
        w[i + 1] = v[1];
        w[i + 2] = v[2];
        w[i + 3] = v[3];
    }
    constexpr int b = N / 4 * 4;
    if constexpr (N - b == 3) {
        const tu32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, off + 4 * b, 0, tCPolNT);
        w[b] = v[0];
        w[b + 1] = v[1];
        w[b + 2] = v[2];
    } else if constexpr (N - b == 2) {
        const tu32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off + 4 * b, 0, tCPolNT);
        w[b] = v[0];
        w[b + 1] = v[1];
    } else if constexpr (N - b == 1) {
        w[b] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * b, 0, tCPolNT);
    }
}

// The register loads of the tile at key t0 (item m = 64 q + lane: group
// m / 32, key m % 32; items past the groups read from outside the range,
// i.e. zero).
template <int D, int NG, int KB, int VB>
__device__ __forceinline__ void reg_load(RegTile<D, NG, KB, VB>& R, const TRsrc& rs, int t0, int lane) {
    using RT = RegTile<D, NG, KB, VB>;
    load_words<RT::NKW>(rs.kw, ((uint32_t)t0 * (D * KB / 32) + (uint32_t)lane * RT::NKW) * 4u, R.kw);
    load_words<RT::NVW>(rs.vw, ((uint32_t)t0 * (D * VB / 32) + (uint32_t)lane * RT::NVW) * 4u, R.vw);
#pragma unroll
    for (int q = 0; q < RT::NIT; ++q) {
        const int m = 64 * q + lane;
        const int g = m / tTile, key = m - g * tTile;
        const uint32_t off = (g < NG) ? ((uint32_t)(t0 + key) * NG + g) * 2u : 0xFFFFFFF0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) R.meta[q][i] = __builtin_amdgcn_raw_buffer_load_b16(rs.m[i], off, 0, tCPolNT);
    }
}

// Decode this lane's BITS-bit units (words w[UPL * BITS]) into fp16 codes
// at dst + key * row_bytes + 64 * part.
template <int BITS, int D>
__device__ __forceinline__ void reg_decode_units(const uint32_t* words, int lane, unsigned char* dst,
                                                 int row_bytes) {
    constexpr int UPL = D / 64, upk = D / 32;
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
        const int u = lane * UPL + i;
        const int key = u / upk, part = u - key * upk;
        uint32_t w[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) w[b] = (b < BITS) ? words[i * BITS + b] : 0u;
        uint32_t c[8];
        unpack32<BITS>(w, c);
        tu32x2 h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = bytes_f16(c[e]);
        tu32x4* d = reinterpret_cast<tu32x4*>(dst + key * row_bytes + 64 * part);
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e] = (tu32x4){h[2 * e][0], h[2 * e][1], h[2 * e + 1][0], h[2 * e + 1][1]};
    }
}

// W = 4: long query blocks (64 rows per workgroup share every decoded tile);
// W = 1: up to 16 rows per kv head (decode, short verify blocks): one wave
// per workgroup decodes and computes its own tiles, so the compute units run
// many independent waves instead of one computing wave per four.  PRF: at
// most 8 rows per kv head, paired hi / lo operand rows (implied by KB > 0).
template <int DT, int D, int NG, int W, int KB = 0, int VB = 0, int PRF = 0>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2)))
void attn_tile_kernel(TArgs a) {
    constexpr bool RP = KB > 0;  // register-staged tiles (single wave, widths fixed)
    constexpr bool PR = RP || PRF > 0;  // paired rows (single wave, at most 8 rows)
    static_assert(!PR || W == 1, "paired rows: one wave");
    using Ly = TileLds<D, W, NG, RP>;
    static_assert(!RP || (W == 1 && D <= 128 && KB == 4 && VB > 0),
                  "register staging: one wave, head_dim <= 128, 4-bit K codes entering the MFMAs in place");
    constexpr int kThr = 64 * W;
    constexpr int kRW = 16 * W;  // query rows per workgroup
    constexpr int NC = D / 32;    // 32-dim chunks
    constexpr int NB = D / 16;    // 16-column output blocks
    constexpr int CPG = NC / NG;  // chunks per group
    constexpr int NPG = NB / NG;  // output blocks per group
    __shared__ __attribute__((aligned(16))) unsigned char smem[Ly::bytes];
    extern __shared__ __attribute__((aligned(16))) unsigned char rawb[];  // raw_bytes(...) at launch
    float* fs = reinterpret_cast<float*>(smem);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, n = lane & 15, j = lane >> 4;
    const int bhr = blockIdx.x / a.S;
    const int split = blockIdx.x - bhr * a.S;
    const int bh = bhr / a.RBW;
    const int r0 = kRW * (bhr - bh * a.RBW);
    const int b = bh / a.Hkv;
    const int kvh = bh - b * a.Hkv;
    const int T = a.T;
    const int64_t row0 = (int64_t)bh * a.capacity;
    const int t_begin = split * a.chunk;
    int t_end = t_begin + a.chunk;
    if (t_end > T) t_end = T;
    // keys past the last visible key of every row of the block are skipped
    const int rlast = min(r0 + kRW, a.G) - 1;
    int t_lim = t_end;
    if (a.causal && a.mask == nullptr) {
        const int i0 = r0 % a.L, i1 = rlast % a.L;
        const int imax = (rlast - r0 + 1 >= a.L || i1 < i0) ? a.L - 1 : i1;
        const int vmax = T - a.L + imax + 1;
        if (t_lim > vmax) t_lim = vmax;
    }

    // the first tile's transfers in flight during the set-up, later always
    // the next tile's during the compute of one
    TRsrc rs;
    {
        const int kwords = D * a.kbits / 32, vwords = D * a.vbits / 32;
        const uint32_t* kbase = a.kw + row0 * kwords;
        const uint32_t* vbase = a.vw + row0 * vwords;
        rs.kw = tmake_rsrc(kbase, (uint32_t)T * kwords * 4u);
        rs.vw = tmake_rsrc(vbase, (uint32_t)T * vwords * 4u);
        // 16-byte transfers need 16-byte aligned slabs and rows (a chunk must
        // not straddle the end of row T - 1: past the range it reads as zero)
        rs.k16 = (reinterpret_cast<uintptr_t>(kbase) & 15) == 0 && kwords % 4 == 0;
        rs.v16 = (reinterpret_cast<uintptr_t>(vbase) & 15) == 0 && vwords % 4 == 0;
        const uint16_t* mb[4] = {a.ks, a.kb, a.vs, a.vb};
#pragma unroll
        for (int k = 0; k < 4; ++k) rs.m[k] = tmake_rsrc(mb[k] + row0 * NG, (uint32_t)T * NG * 2u);
    }
    // the query row and the rotation matrix are loaded before the tile
    // transfers: loads complete in issue order, so a wait for them would
    // otherwise wait for the tiles too.  Query row: 16 wave + n of the block
    // (paired rows: n & 7), dims 32 c + 8 j + 0..7; the rotation matrix (D
    // float4s) is loaded once per workgroup and passed through LDS.
    const int rowA = PR ? r0 + (n & 7) : r0 + 16 * wave + n;
    const bool wave_live = r0 + 16 * wave < a.G;
    float xq[NC][8];
    {
        const uint16_t* qrow = nullptr;
        if (rowA < a.G) {
            const int h = kvh * a.n_rep + rowA / a.L;
            qrow = a.q + (((int64_t)b * a.Hkv * a.n_rep + h) * a.L + rowA % a.L) * D;
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int e = 0; e < 8; ++e) xq[c][e] = 0.f;
            if (qrow != nullptr) {
                load4<DT>(qrow + 32 * c + 8 * j, xq[c]);
                load4<DT>(qrow + 32 * c + 8 * j + 4, xq[c] + 4);
            }
        }
    }
    constexpr int NRS = (D + kThr - 1) / kThr;  // float4s of the rotation matrix per thread
    float4 rsl[NRS];
#pragma unroll
    for (int i = 0; i < NRS; ++i) {
        const int idx = tid + kThr * i;
        rsl[i] = (a.rot != nullptr && idx < D) ? reinterpret_cast<const float4*>(a.rot)[idx]
                                               : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    tlds_u8* rawl = (tlds_u8*)rawb;
    uint32_t meta1[4] = {0u, 0u, 0u, 0u};  // NG = 1: this thread's item, loaded a tile ahead
    // register staging: the first two tiles; a load that would pass the
    // split's last tile reads at row T instead, past the buffers' ranges (it
    // returns zeros without touching memory; its data is not used)
    const int t_last = (t_lim > t_begin) ? t_begin + (t_lim - 1 - t_begin) / tTile * tTile : t_begin;
    auto next_tile = [&](int t) { return t <= t_last ? t : T; };
    RegTile<D, NG, RP ? KB : 4, RP ? VB : 4> reg_a, reg_b;
    if constexpr (RP) {
        reg_load(reg_a, rs, t_begin, lane);
        reg_load(reg_b, rs, next_tile(t_begin + tTile), lane);
    } else if (t_begin < t_lim) {
        issue_tile<D, NG, W>(a, rs, t_begin, wave, lane, rawl);
        if (NG == 1 && tid < 32) load_meta1(a, row0, t_begin, tid, meta1);
    }

    // the rotation matrix into the K code area (free until the first tile
    // is decoded)
    static_assert(tTile * Ly::KS >= 16 * D, "the rotation matrix fits the K code area");
    float* rotl = reinterpret_cast<float*>(smem + Ly::kc);
#pragma unroll
    for (int i = 0; i < NRS; ++i) {
        const int idx = tid + kThr * i;
        if (idx < D) reinterpret_cast<float4*>(rotl)[idx] = rsl[i];
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // LDS only

    // ---- query operands (paired rows in the register-staged shape, at most
    //      8 rows per kv head: operand rows 0-7 hold the hi parts of the 8
    //      query rows, rows 8-15 their lo parts, so one MFMA takes both and
    //      the accumulators' hi and lo rows are added by a lane-half swap) ----
    tf16x8 qh[NC], ql[NC];
    {
        float qv[NC][8];
        float mx = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const float* x = xq[c];
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                float y[4];
                if (a.rot != nullptr) {
                    float Bm[16];
                    const float4* bp = reinterpret_cast<const float4*>(rotl + 16 * (8 * c + 2 * j + hb));
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float4 bv = bp[r];
                        Bm[4 * r] = bv.x;
                        Bm[4 * r + 1] = bv.y;
                        Bm[4 * r + 2] = bv.z;
                        Bm[4 * r + 3] = bv.w;
                    }
                    rotate4(x + 4 * hb, Bm, y);
                    if (a.round_rot) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) y[e] = elem_to_f32<DT>(f32_to_elem_bits<DT>(y[e]));
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) y[e] = x[4 * hb + e];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    qv[c][4 * hb + e] = y[e] * a.qscale;
                    mx = fmaxf(mx, fabsf(qv[c][4 * hb + e]));
                }
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        int ex = 0;
        if (mx > 0.f) (void)frexpf(mx, &ex);
        const int E = (mx > 0.f) ? 15 - ex : 0;
        float gsum[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) gsum[g] = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                gsum[c / CPG] += qv[c][e];
                if constexpr (RP) {
                    // slot e takes dim kPerm[e] of the block times 1 or 1/16
                    // (the K operand's nibble order and factors); rows 8-15
                    // of the operand take the lo parts
                    constexpr int kPerm[8] = {0, 4, 1, 5, 2, 6, 3, 7};
                    const float xs = ldexpf(qv[c][kPerm[e]], E) * ((e & 2) ? 0.0625f : 1.0f);
                    const _Float16 hi = (_Float16)xs;
                    qh[c][e] = (n >= 8) ? (_Float16)(xs - (float)hi) : hi;
                } else if constexpr (PR) {
                    // natural dim order; rows 8-15 of the operand take the lo parts
                    const float xs = ldexpf(qv[c][e], E);
                    const _Float16 hi = (_Float16)xs;
                    qh[c][e] = (n >= 8) ? (_Float16)(xs - (float)hi) : hi;
                } else {
                    const float xs = ldexpf(qv[c][e], E);
                    const _Float16 hi = (_Float16)xs;
                    qh[c][e] = hi;
                    ql[c][e] = (_Float16)(xs - (float)hi);
                }
            }
        }
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            float s = gsum[g];
            s += __shfl_xor(s, 16);
            s += __shfl_xor(s, 32);
            if (j == 0) fs[Ly::qst / 4 + (wave * NG + g) * 16 + n] = s;
        }
        if (j == 0) fs[Ly::frw / 4 + wave * 16 + n] = ldexpf(1.0f, -E);
    }

    // ---- per-lane softmax rows (accumulator rows 4 j + i) ----
    float frow[4], m_run[4], l_part[4];
    int vis[4];
    uint32_t moff[4];  // byte offset of the row's mask elements; 0xFFFFFFFF: no mask
    // LDS only: __syncthreads would also wait for the tile transfers in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int esize = (a.mtype == 1) ? 1 : (a.mtype == 2) ? 4 : 2;
    const int vis_lo = a.causal ? T - a.L + 1 : T;  // the first row's visible keys
    // paired rows: lane (j, n) keeps the softmax state of rows
    // rb + 2 p + hl (rb = 4 (j & 1), hl = j >> 1), p = 0, 1
    const int rb = 4 * (j & 1), hl = j >> 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rr = PR ? rb + 2 * (i & 1) + hl : 4 * j + i;
        frow[i] = fs[Ly::frw / 4 + wave * 16 + rr];
        m_run[i] = -INFINITY;
        l_part[i] = 0.f;
        const int R = r0 + 16 * wave + rr;
        vis[i] = (R < a.G && a.causal) ? T - a.L + (R % a.L) + 1 : T;
        moff[i] = 0xFFFFFFFFu;
        if (R < a.G && a.mask != nullptr) {
            const int h = kvh * a.n_rep + R / a.L;
            moff[i] = (uint32_t)(((int64_t)b * a.msb + (int64_t)h * a.msh + (int64_t)(R % a.L) * a.msl) * esize);
        }
    }
    __amdgpu_buffer_rsrc_t mask_r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(a.mask != nullptr ? a.mask : (const void*)a.q), (short)0,
        (int)a.mask_bytes, 0x00020000);

    // output accumulators: column group g holds sum_t p_t s_{t,g} 2^F_g c_{t,d}
    tf32x4 O[NB];
#pragma unroll
    for (int t = 0; t < NB; ++t) O[t] = (tf32x4){0.f, 0.f, 0.f, 0.f};
    float ob[4][NG];  // per lane: sum over its keys of p_t b_{t,g}
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < NG; ++g) ob[i][g] = 0.f;
    constexpr int NIT = (32 * NG + kThr - 1) / kThr;  // scale / bias items per thread
    int f_run[NIT];  // running scale powers of the groups of this thread's items
#pragma unroll
    for (int q = 0; q < NIT; ++q) f_run[q] = 1000;
    const float one = 1.0f;
    // this lane's address of the transposing V reads: lane 4 e + c of group j
    // reads key 8 j + 4 h + e, columns 4 c .. 4 c + 3 of an output block
    const unsigned char* vrd = smem + Ly::vc + (8 * j + (n >> 2)) * Ly::VS + 8 * (n & 3);

    // the arithmetic of one tile whose codes, scales and biases are in LDS
    auto compute_tile = [&](const int t0) __attribute__((always_inline)) {
        // ---- scores ----
        float sacc[2][4], bacc[2][4];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) sacc[nb][i] = bacc[nb][i] = 0.f;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            tf32x4 acc[2] = {(tf32x4){0.f, 0.f, 0.f, 0.f}, (tf32x4){0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int cc = 0; cc < CPG; ++cc) {
                const int c = g * CPG + cc;
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const tf16x8 kb8 = *reinterpret_cast<const tf16x8*>(
                        smem + Ly::kc + (16 * nb + n) * Ly::KS + 64 * c + 16 * j);
                    acc[nb] = tmfma(qh[c], kb8, acc[nb]);
                    acc[nb] = tmfma(ql[c], kb8, acc[nb]);
                }
            }
            const float s0 = fs[Ly::ksl / 4 + g * tTile + n], s1 = fs[Ly::ksl / 4 + g * tTile + 16 + n];
            const float b0 = fs[Ly::kbl / 4 + g * tTile + n], b1 = fs[Ly::kbl / 4 + g * tTile + 16 + n];
            const tf32x4 qs = *reinterpret_cast<const tf32x4*>(
                fs + Ly::qst / 4 + (wave * NG + g) * 16 + 4 * j);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sacc[0][i] += s0 * acc[0][i];
                sacc[1][i] += s1 * acc[1][i];
                bacc[0][i] += b0 * qs[i];
                bacc[1][i] += b1 * qs[i];
            }
        }
        float sc[2][4];
        // keys past the split or past a row's last visible key only in a
        // tile that reaches them (one vote over the wave)
        bool lane_full = t0 + tTile <= t_end;
#pragma unroll
        for (int i = 0; i < 4; ++i) lane_full = lane_full && t0 + tTile <= vis[i];
        const bool full = __all(lane_full);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + 16 * nb + n;
                float s = sacc[nb][i] * frow[i] + bacc[nb][i];
                if (!full && (t >= t_end || t >= vis[i])) s = -INFINITY;
                if (a.mtype != 0 && moff[i] != 0xFFFFFFFFu && s != -INFINITY) {
                    const uint32_t off = moff[i] + (uint32_t)t * esize;
                    if (a.mtype == 1) {
                        if (__builtin_amdgcn_raw_buffer_load_b8(mask_r, off, 0, 0) == 0) s = -INFINITY;
                    } else if (a.mtype == 2) {
                        s += __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(mask_r, off, 0, 0)) * tLog2e;
                    } else {
                        s += elem_to_f32<DT>(__builtin_amdgcn_raw_buffer_load_b16(mask_r, off, 0, 0)) * tLog2e;
                    }
                }
                sc[nb][i] = s;
            }

        // ---- online softmax (base 2, exact running maximum) ----
        float alpha[4], p[2][4];
        bool grow = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float tmx = tmax16(fmaxf(sc[0][i], sc[1][i]));
            const float m_new = fmaxf(m_run[i], tmx);
            if (m_new == -INFINITY) {
                alpha[i] = 1.f;
                p[0][i] = p[1][i] = 0.f;
            } else {
                // hardware exp2 (results below 2^-126, weights negligible
                // next to the row's largest, flush to zero)
                alpha[i] = __builtin_amdgcn_exp2f(m_run[i] - m_new);
                p[0][i] = __builtin_amdgcn_exp2f(sc[0][i] - m_new);
                p[1][i] = __builtin_amdgcn_exp2f(sc[1][i] - m_new);
            }
            grow |= m_new != m_run[i];
            m_run[i] = m_new;
            l_part[i] = l_part[i] * alpha[i] + (p[0][i] + p[1][i]);
        }
        if (__any(grow)) {  // rescale the accumulators only when some row's maximum moved
#pragma unroll
            for (int t = 0; t < NB; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) O[t][i] *= alpha[i];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int g = 0; g < NG; ++g) ob[i][g] *= alpha[i];
        }
        // group biases: sum_t p_t b_{t,g}, per lane over its keys n, 16 + n
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const float v0 = fs[Ly::vbl / 4 + g * tTile + n], v1 = fs[Ly::vbl / 4 + g * tTile + 16 + n];
#pragma unroll
            for (int i = 0; i < 4; ++i) ob[i][g] += p[0][i] * v0 + p[1][i] * v1;
        }
        // P to the operand layout (row n, keys 8 j .. 8 j + 7) through LDS
        float* pw = fs + Ly::pst / 4 + wave * 16 * tPS;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) pw[(4 * j + i) * tPS + 16 * nb + n] = p[nb][i];
        __builtin_amdgcn_wave_barrier();
        const tf32x4 pa0 = *reinterpret_cast<const tf32x4*>(pw + n * tPS + 8 * j);
        const tf32x4 pa1 = *reinterpret_cast<const tf32x4*>(pw + n * tPS + 8 * j + 4);

        // ---- P V, accumulated into O ----
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const float rs = fs[Ly::vres / 4 + g];
            if (rs != 1.0f) {  // the group's running scale power dropped
#pragma unroll
                for (int t = g * NPG; t < (g + 1) * NPG; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) O[t][i] *= rs;
            }
            const tf32x4 x0 = *reinterpret_cast<const tf32x4*>(fs + Ly::vsf / 4 + g * tTile + 8 * j);
            const tf32x4 x1 = *reinterpret_cast<const tf32x4*>(fs + Ly::vsf / 4 + g * tTile + 8 * j + 4);
            tu32x2 s01 = split_f16(pa0[0] * x0[0], pa0[1] * x0[1], one);
            tu32x2 s23 = split_f16(pa0[2] * x0[2], pa0[3] * x0[3], one);
            tu32x2 s45 = split_f16(pa1[0] * x1[0], pa1[1] * x1[1], one);
            tu32x2 s67 = split_f16(pa1[2] * x1[2], pa1[3] * x1[3], one);
            const tf16x8 ph = __builtin_bit_cast(tf16x8, (tu32x4){s01[0], s23[0], s45[0], s67[0]});
            const tf16x8 pl = __builtin_bit_cast(tf16x8, (tu32x4){s01[1], s23[1], s45[1], s67[1]});
#pragma unroll
            for (int t = g * NPG; t < (g + 1) * NPG; ++t) {
                const tu32x2 v0 = tr16_read(vrd + 32 * t);
                const tu32x2 v1 = tr16_read(vrd + 32 * t + 4 * Ly::VS);
                const tf16x8 vb8 = __builtin_bit_cast(tf16x8, (tu32x4){v0[0], v0[1], v1[0], v1[1]});
                O[t] = tmfma(ph, vb8, O[t]);
                O[t] = tmfma(pl, vb8, O[t]);
            }
        }
    };
    // the same with paired rows: one MFMA per operand pair (hi and lo rows
    // together), two softmax rows per lane
    auto compute_tile_pr = [&](const int t0) __attribute__((always_inline)) {
        // ---- scores: accumulator rows 4 j + i (j < 2: hi parts of rows
        //      rb + i, j >= 2: lo parts), column = key ----
        float sacc[2][4];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) sacc[nb][i] = 0.f;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            tf32x4 acc[2] = {(tf32x4){0.f, 0.f, 0.f, 0.f}, (tf32x4){0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int cc = 0; cc < CPG; ++cc) {
                const int c = g * CPG + cc;
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    if constexpr (RP) {
                        // word 4 c + j of key 16 nb + n: its nibble pairs
                        // masked in place are fp16 subnormals c 2^-24
                        // (nibbles 0, 4 and 2, 6) or 16 c 2^-24 (1, 5 and
                        // 3, 7), matching the query operand's slot order and
                        // factors
                        const uint32_t w = *reinterpret_cast<const uint32_t*>(
                            smem + Ly::kc + (16 * nb + n) * Ly::KS + 4 * (4 * c + j));
                        const uint32_t w8 = w >> 8;
                        const tu32x4 kv = {w & 0x000F000Fu, w & 0x00F000F0u, w8 & 0x000F000Fu, w8 & 0x00F000F0u};
                        acc[nb] = tmfma(qh[c], __builtin_bit_cast(tf16x8, kv), acc[nb]);
                    } else {
                        // the decoded codes, dims 32 c + 8 j .. 32 c + 8 j + 7
                        const tf16x8 kb8 = *reinterpret_cast<const tf16x8*>(
                            smem + Ly::kc + (16 * nb + n) * Ly::KS + 64 * c + 16 * j);
                        acc[nb] = tmfma(qh[c], kb8, acc[nb]);
                    }
                }
            }
            const float s0 = fs[Ly::ksl / 4 + g * tTile + n], s1 = fs[Ly::ksl / 4 + g * tTile + 16 + n];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sacc[0][i] += s0 * acc[0][i];
                sacc[1][i] += s1 * acc[1][i];
            }
        }
        // hi + lo by one lane-half swap per register pair: the lane's row p
        // (rb + 2 p + hl) of key 16 nb + n; keys past the split or past a
        // row's last visible key only in a tile that reaches them
        const bool full = t0 + tTile <= t_end && t0 + tTile <= vis_lo;
        float sc[2][2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                const auto sw = __builtin_amdgcn_permlane32_swap(
                    __float_as_uint(sacc[nb][2 * pp]), __float_as_uint(sacc[nb][2 * pp + 1]), false, false);
                const float tt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
                const int rr = rb + 2 * pp + hl;
                float bias = 0.f;
#pragma unroll
                for (int g = 0; g < NG; ++g)
                    bias += fs[Ly::kbl / 4 + g * tTile + 16 * nb + n] * fs[Ly::qst / 4 + g * 16 + rr];
                const int t = t0 + 16 * nb + n;
                // codes in place entered as c 2^-24
                float sv = tt * (RP ? 16777216.0f : 1.0f) * frow[pp] + bias;
                if (!full && (t >= t_end || t >= vis[pp])) sv = -INFINITY;
                if (a.mtype != 0 && moff[pp] != 0xFFFFFFFFu && sv != -INFINITY) {
                    const uint32_t off = moff[pp] + (uint32_t)t * esize;
                    if (a.mtype == 1) {
                        if (__builtin_amdgcn_raw_buffer_load_b8(mask_r, off, 0, 0) == 0) sv = -INFINITY;
                    } else if (a.mtype == 2) {
                        sv += __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(mask_r, off, 0, 0)) * tLog2e;
                    } else {
                        sv += elem_to_f32<DT>(__builtin_amdgcn_raw_buffer_load_b16(mask_r, off, 0, 0)) * tLog2e;
                    }
                }
                sc[nb][pp] = sv;
            }

        // ---- online softmax of the lane's two rows (base 2, exact running
        //      maximum) ----
        float alpha[2], pr[2][2];
        bool grow = false;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            const float tmx = tmax16(fmaxf(sc[0][pp], sc[1][pp]));
            const float m_new = fmaxf(m_run[pp], tmx);
            if (m_new == -INFINITY) {
                alpha[pp] = 1.f;
                pr[0][pp] = pr[1][pp] = 0.f;
            } else {
                alpha[pp] = __builtin_amdgcn_exp2f(m_run[pp] - m_new);
                pr[0][pp] = __builtin_amdgcn_exp2f(sc[0][pp] - m_new);
                pr[1][pp] = __builtin_amdgcn_exp2f(sc[1][pp] - m_new);
            }
            grow |= m_new != m_run[pp];
            m_run[pp] = m_new;
            l_part[pp] = l_part[pp] * alpha[pp] + (pr[0][pp] + pr[1][pp]);
        }
        if (__any(grow)) {
            // accumulator register i holds row rb + i (hi or lo part); rows
            // rb + hl and rb + 2 + hl are this lane's, the others its
            // partner's (lane ^ 32)
            const float pa0 = __shfl_xor(alpha[0], 32), pa1 = __shfl_xor(alpha[1], 32);
            const float alc[4] = {hl ? pa0 : alpha[0], hl ? alpha[0] : pa0, hl ? pa1 : alpha[1],
                                  hl ? alpha[1] : pa1};
#pragma unroll
            for (int t = 0; t < NB; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) O[t][i] *= alc[i];
#pragma unroll
            for (int pp = 0; pp < 2; ++pp)
#pragma unroll
                for (int g = 0; g < NG; ++g) ob[pp][g] *= alpha[pp];
        }
        // group biases: sum_t p_t b_{t,g} per lane over its keys n, 16 + n
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const float v0 = fs[Ly::vbl / 4 + g * tTile + n], v1 = fs[Ly::vbl / 4 + g * tTile + 16 + n];
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) ob[pp][g] += pr[0][pp] * v0 + pr[1][pp] * v1;
        }
        // P to the operand layout through LDS: operand row n reads query row
        // n & 7, keys 8 j .. 8 j + 7 (rows 8-15 take the lo parts below)
        float* pw = fs + Ly::pst / 4 + wave * 16 * tPS;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) pw[(rb + 2 * pp + hl) * tPS + 16 * nb + n] = pr[nb][pp];
        __builtin_amdgcn_wave_barrier();
        const tf32x4 pa0 = *reinterpret_cast<const tf32x4*>(pw + (n & 7) * tPS + 8 * j);
        const tf32x4 pa1 = *reinterpret_cast<const tf32x4*>(pw + (n & 7) * tPS + 8 * j + 4);
        const bool lo_row = n >= 8;

        // ---- P V, accumulated into O (one MFMA per output block) ----
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const float rsg = fs[Ly::vres / 4 + g];
            if (rsg != 1.0f) {  // the group's running scale power dropped
#pragma unroll
                for (int t = g * NPG; t < (g + 1) * NPG; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) O[t][i] *= rsg;
            }
            const tf32x4 x0 = *reinterpret_cast<const tf32x4*>(fs + Ly::vsf / 4 + g * tTile + 8 * j);
            const tf32x4 x1 = *reinterpret_cast<const tf32x4*>(fs + Ly::vsf / 4 + g * tTile + 8 * j + 4);
            const tu32x2 s01 = split_f16(pa0[0] * x0[0], pa0[1] * x0[1], one);
            const tu32x2 s23 = split_f16(pa0[2] * x0[2], pa0[3] * x0[3], one);
            const tu32x2 s45 = split_f16(pa1[0] * x1[0], pa1[1] * x1[1], one);
            const tu32x2 s67 = split_f16(pa1[2] * x1[2], pa1[3] * x1[3], one);
            const tf16x8 pp8 = __builtin_bit_cast(
                tf16x8, (tu32x4){lo_row ? s01[1] : s01[0], lo_row ? s23[1] : s23[0],
                                 lo_row ? s45[1] : s45[0], lo_row ? s67[1] : s67[0]});
#pragma unroll
            for (int t = g * NPG; t < (g + 1) * NPG; ++t) {
                const tu32x2 v0 = tr16_read(vrd + 32 * t);
                const tu32x2 v1 = tr16_read(vrd + 32 * t + 4 * Ly::VS);
                const tf16x8 vb8 = __builtin_bit_cast(tf16x8, (tu32x4){v0[0], v0[1], v1[0], v1[1]});
                O[t] = tmfma(pp8, vb8, O[t]);
            }
        }
    };
    if constexpr (!RP) {
        for (int t0 = t_begin; t0 < t_lim; t0 += tTile) {
            // the tile's transfers have landed (each wave waits for its own; the
            // barrier for all) and the previous tile's LDS reads are done
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            __syncthreads();
            store_units<D, W, NG>(a, rawb, tid, smem);
#pragma unroll
            for (int q = 0; q < NIT; ++q) {
                const int m = q * kThr + tid;
                if (m < 32 * NG) {  // whole 32-lane groups
                    uint32_t meta[4];
                    if constexpr (NG == 1) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) meta[i] = meta1[i];
                    } else {
                        read_meta<D, NG>(rawb, a.raw_meta, m, meta);
                    }
                    store_meta<DT, D, W, NG>(meta, m, smem, f_run[q]);
                }
            }
            __syncthreads();  // codes in place; the staging area is free
            if (t0 + tTile < t_lim) {
                issue_tile<D, NG, W>(a, rs, t0 + tTile, wave, lane, rawl);
                if (NG == 1 && tid < 32) load_meta1(a, row0, t0 + tTile, tid, meta1);
            }
            if (!wave_live) continue;
            if constexpr (PR)
                compute_tile_pr(t0);
            else
                compute_tile(t0);
        }
    } else {
        // one tile from a register set: decode it into LDS, refill the set
        // with the tile two ahead, compute (LDS-only barriers: the register
        // loads in flight stay in flight)
        auto step = [&](const int t0, RegTile<D, NG, KB, VB>& R) __attribute__((always_inline)) {
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            {
                // K words as they are: this lane's units of key u / (D / 32)
                constexpr int UPL = D / 64, upk = D / 32;
                const int u = lane * UPL;
                const int key = u / upk, part = u - key * upk;
                tu32x4* kd = reinterpret_cast<tu32x4*>(smem + Ly::kc + key * Ly::KS + 16 * part);
#pragma unroll
                for (int e = 0; e < UPL; ++e)
                    kd[e] = (tu32x4){R.kw[4 * e], R.kw[4 * e + 1], R.kw[4 * e + 2], R.kw[4 * e + 3]};
            }
            reg_decode_units<VB, D>(R.vw, lane, smem + Ly::vc, Ly::VS);
#pragma unroll
            for (int q = 0; q < NIT; ++q) {
                const int m = q * kThr + tid;
                if (m < 32 * NG) store_meta<DT, D, W, NG, RP>(R.meta[q], m, smem, f_run[q]);
            }
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            reg_load(R, rs, next_tile(t0 + 2 * tTile), lane);
            compute_tile_pr(t0);
        };
        int t0 = t_begin;
        for (; t0 + tTile < t_lim; t0 += 2 * tTile) {
            step(t0, reg_a);
            step(t0 + tTile, reg_b);
        }
        if (t0 < t_lim) step(t0, reg_a);
    }

    if constexpr (PR) {
        // paired rows: the hi and lo parts of output row rb + 2 p + hl come
        // together by one lane-half swap (every lane takes part before any
        // lane stores); then as below
        float vinv[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) vinv[g] = (t_begin < t_lim) ? fs[Ly::vinv / 4 + g] : 1.f;
        float lsum[2], bsum[2][NG];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            lsum[pp] = tsum16(l_part[pp]);
#pragma unroll
            for (int g = 0; g < NG; ++g) bsum[pp][g] = tsum16(ob[pp][g]);
        }
        auto comb = [](float x, float y) -> float {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
            return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        };
        if (a.S == 1) {
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                const int R = r0 + rb + 2 * pp + hl;
                const float inv = 1.0f / lsum[pp];
                // a boolean mask dropped every key of the row: the mean of its keys
                const bool uniform = a.mtype == 1 && lsum[pp] == 0.f && R < a.G;
                const int nv = a.causal ? T - a.L + (R % a.L) + 1 : T;
                const int hq = kvh * a.n_rep + R / a.L;
                float* orow = a.out + (((int64_t)b * a.Hkv * a.n_rep + hq) * a.L + R % a.L) * D;
#pragma unroll
                for (int t = 0; t < NB; ++t) {
                    const int g = t / NPG;
                    const int col = 16 * t + n;
                    float y = (comb(O[t][2 * pp], O[t][2 * pp + 1]) * vinv[g] + bsum[pp][g]) * inv;
                    if (uniform)
                        y = value_column_mean<DT>(a.vw, a.vs, a.vb, row0, nv, col, a.vbits,
                                                  D * a.vbits / 32, NG, a.GS);
                    float z = y;
                    if (a.rot != nullptr) {
                        const float4 v = *reinterpret_cast<const float4*>(a.rot + 16 * (col >> 2) + 4 * (col & 3));
                        const float y0 = tdpp<0x00>(y), y1 = tdpp<0x55>(y), y2 = tdpp<0xAA>(y), y3 = tdpp<0xFF>(y);
                        double s2 = (double)y0 * (double)v.x;
                        s2 = s2 + (double)y1 * (double)v.y;
                        s2 = s2 + (double)y2 * (double)v.z;
                        s2 = s2 + (double)y3 * (double)v.w;
                        z = (float)s2;
                    }
                    if (R < a.G) orow[col] = z;
                }
            }
            return;
        }
        const int64_t unit = (int64_t)bhr * a.S + split;
        float* ro = a.rec_o + unit * kRW * D;
        float* rml = a.rec_ml + unit * kRW * 2;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            const int rr = rb + 2 * pp + hl;
#pragma unroll
            for (int t = 0; t < NB; ++t) {
                const float val = comb(O[t][2 * pp], O[t][2 * pp + 1]) * vinv[t / NPG] + bsum[pp][t / NPG];
                if (r0 + rr < a.G) ro[rr * D + 16 * t + n] = val;
            }
            if (n == 0 && r0 + rr < a.G) {
                rml[2 * rr] = m_run[pp];
                rml[2 * rr + 1] = lsum[pp];
            }
        }
        return;
    }

    // ---- record: (m, l) and the unnormalised o of each row; with one split
    //      the normalised row itself, rotated back (a rotation block's four
    //      columns sit in one lane quad: DPP broadcasts, fp64 sum) ----
    if (!wave_live) return;
    if (a.S == 1) {
        float vinv1[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) vinv1[g] = (t_begin < t_lim) ? fs[Ly::vinv / 4 + g] : 1.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int R = r0 + 16 * wave + 4 * j + i;
            const float lsum = tsum16(l_part[i]);
            const float inv = 1.0f / lsum;
            if (R >= a.G) continue;  // uniform over the 16 lanes of the row
            // a boolean mask dropped every key of the row: the mean of its keys
            const bool uniform = a.mtype == 1 && lsum == 0.f;
            const int nv = a.causal ? T - a.L + (R % a.L) + 1 : T;
            const int hq = kvh * a.n_rep + R / a.L;
            float* orow = a.out + (((int64_t)b * a.Hkv * a.n_rep + hq) * a.L + R % a.L) * D;
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const float bias = tsum16(ob[i][g]);
#pragma unroll
                for (int t = g * NPG; t < (g + 1) * NPG; ++t) {
                    const int col = 16 * t + n;
                    float y = (O[t][i] * vinv1[g] + bias) * inv;
                    if (uniform)
                        y = value_column_mean<DT>(a.vw, a.vs, a.vb, row0, nv, col, a.vbits,
                                                  D * a.vbits / 32, NG, a.GS);
                    float z = y;
                    if (a.rot != nullptr) {
                        const float4 v = *reinterpret_cast<const float4*>(a.rot + 16 * (col >> 2) + 4 * (col & 3));
                        const float y0 = tdpp<0x00>(y), y1 = tdpp<0x55>(y), y2 = tdpp<0xAA>(y), y3 = tdpp<0xFF>(y);
                        double s2 = (double)y0 * (double)v.x;
                        s2 = s2 + (double)y1 * (double)v.y;
                        s2 = s2 + (double)y2 * (double)v.z;
                        s2 = s2 + (double)y3 * (double)v.w;
                        z = (float)s2;
                    }
                    orow[col] = z;
                }
            }
        }
        return;
    }
    const int64_t unit = (int64_t)bhr * a.S + split;
    float* ro = a.rec_o + unit * kRW * D;
    float* rml = a.rec_ml + unit * kRW * 2;
    float vinv[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g)  // the scale powers after the last tile (none: 1, O is 0)
        vinv[g] = (t_begin < t_lim) ? fs[Ly::vinv / 4 + g] : 1.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rr = 16 * wave + 4 * j + i;
        const float l = tsum16(l_part[i]);
        if (r0 + rr >= a.G) continue;  // past the last query row: nothing to record
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const float bias = tsum16(ob[i][g]);
#pragma unroll
            for (int t = g * NPG; t < (g + 1) * NPG; ++t)
                ro[rr * D + 16 * t + n] = O[t][i] * vinv[g] + bias;
        }
        if (n == 0) {
            rml[2 * rr] = m_run[i];
            rml[2 * rr + 1] = l;
        }
    }
}

struct TMArgs {
    const float* rec_o;
    const float* rec_ml;
    const float* rot;
    float* out;
    int S, Hkv, n_rep, L, G, RBW, RW;
    // boolean-mask calls: rows without a kept key take the mean of their
    // keys' values (value_column_mean) from the cache
    int bool_mask, dt, T, causal, vbits, GS;
    int64_t capacity;
    const uint32_t* vw;
    const uint16_t* vs;
    const uint16_t* vb;
};

constexpr int tMaxSplits = 1024;  // key splits of one call (the merge keeps a weight per split)

// Reduction over the 256 threads of a block through LDS slot array `red`.
template <bool MAX>
__device__ __forceinline__ float block_reduce(float x, float* red) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const float y = __shfl_xor(x, m);
        x = MAX ? fmaxf(x, y) : x + y;
    }
    const int tid = threadIdx.x;
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = x;
    __syncthreads();
    x = red[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) x = MAX ? fmaxf(x, red[w]) : x + red[w];
    return x;
}

// Merge of the key-split records of one query row (256 threads): m* =
// max_s m_s, weights w_s = 2^(m_s - m*) (0 for an empty split), l* =
// sum_s l_s w_s, o = sum_s w_s o_s / l*, the sum taken over split groups
// s = g mod (256 / (D / 4)) by thread (column quad, group) and the groups
// then added in order; then the inverse rotation of each 4-column block and
// the fp32 store.
template <int D>
__global__ __launch_bounds__(256) void attn_tile_merge_kernel(TMArgs a) {
    constexpr int NQ = D / 4;     // column quads
    constexpr int NSG = 256 / NQ;  // split groups
    __shared__ float wsh[tMaxSplits];
    __shared__ float red[4];
    __shared__ float4 part[NSG][NQ];
    const int rowg = blockIdx.x;  // (b, kv head, row block, row)
    const int RW = a.RW;
    const int rr = rowg % RW;
    const int bhr = rowg / RW;
    const int bh = bhr / a.RBW;
    const int R = RW * (bhr - bh * a.RBW) + rr;
    if (R >= a.G) return;  // uniform: one row per block
    const int tid = threadIdx.x;
    const int b = bh / a.Hkv, kvh = bh - b * a.Hkv;
    // the rotation block of this thread's column quad, loaded first (it is
    // needed last and depends on nothing)
    float Bm[16];
    load_block(a.rot, tid < NQ ? tid : 0, Bm);
    // the first kFirst records of this thread (column quad k, splits sg,
    // sg + NSG, ...) are loaded before the split weights are reduced, so that
    // their latency overlaps the reductions
    const int k = tid % NQ, sg = tid / NQ;
    const float* ro = a.rec_o + ((int64_t)bhr * a.S * RW + rr) * D + 4 * k;
    constexpr int kFirst = 16;
    float4 v1[kFirst];
#pragma unroll
    for (int u = 0; u < kFirst; ++u) {
        const int s1 = sg + u * NSG;
        v1[u] = (s1 < a.S) ? *reinterpret_cast<const float4*>(ro + (int64_t)s1 * RW * D)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // (m, l) of the splits tid, tid + 256, ... (tMaxSplits / 256 at most),
    // loaded once
    constexpr int kPer = tMaxSplits / 256;
    const float* ml = a.rec_ml + (int64_t)bhr * a.S * RW * 2 + 2 * rr;
    float mv[kPer], lv[kPer];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int s = tid + 256 * i;
        mv[i] = -INFINITY;
        lv[i] = 0.f;
        if (s < a.S) {
            const float2 p = *reinterpret_cast<const float2*>(ml + (int64_t)s * RW * 2);
            mv[i] = p.x;
            lv[i] = p.y;
        }
        mx = fmaxf(mx, mv[i]);
    }
    const float M = block_reduce<true>(mx, red);
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int s = tid + 256 * i;
        const float w = (mv[i] == -INFINITY) ? 0.f : exp2f(mv[i] - M);
        if (s < a.S) wsh[s] = w;
        lsum += lv[i] * w;
    }
    const float Ls = block_reduce<false>(lsum, red);  // its barriers also publish wsh
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    // the thread's records in split order: the first kFirst, then the rest
    // four loads in flight at a time
#pragma unroll
    for (int u = 0; u < kFirst; ++u) {
        const int s1 = sg + u * NSG;
        const float w = (s1 < a.S) ? wsh[s1] : 0.f;
        acc.x += v1[u].x * w;
        acc.y += v1[u].y * w;
        acc.z += v1[u].z * w;
        acc.w += v1[u].w * w;
    }
    int s = sg + kFirst * NSG;
    for (; s + 3 * NSG < a.S; s += 4 * NSG) {
        float4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            v[u] = *reinterpret_cast<const float4*>(ro + (int64_t)(s + u * NSG) * RW * D);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float w = wsh[s + u * NSG];
            acc.x += v[u].x * w;
            acc.y += v[u].y * w;
            acc.z += v[u].z * w;
            acc.w += v[u].w * w;
        }
    }
    for (; s < a.S; s += NSG) {
        const float w = wsh[s];
        const float4 v = *reinterpret_cast<const float4*>(ro + (int64_t)s * RW * D);
        acc.x += v.x * w;
        acc.y += v.y * w;
        acc.z += v.z * w;
        acc.w += v.w * w;
    }
    part[sg][k] = acc;
    __syncthreads();
    if (tid >= NQ) return;
    float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < NSG; ++g) {
        const float4 p = part[g][tid];
        o[0] += p.x;
        o[1] += p.y;
        o[2] += p.z;
        o[3] += p.w;
    }
    const float inv = 1.0f / Ls;
    float y[4] = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
    if (a.bool_mask && Ls == 0.f) {
        // no kept key in any split: the mean of the row's keys
        const int nv = a.causal ? a.T - a.L + (R % a.L) + 1 : a.T;
        const int64_t row0 = (int64_t)bh * a.capacity;
        const int vwords = D * a.vbits / 32, ng = D / a.GS;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            y[e] = (a.dt == RBQ_BF16)
                       ? value_column_mean<RBQ_BF16>(a.vw, a.vs, a.vb, row0, nv, 4 * tid + e, a.vbits,
                                                     vwords, ng, a.GS)
                       : value_column_mean<RBQ_F16>(a.vw, a.vs, a.vb, row0, nv, 4 * tid + e, a.vbits,
                                                    vwords, ng, a.GS);
    }
    float z[4] = {y[0], y[1], y[2], y[3]};
    if (a.rot != nullptr) unrotate4(y, Bm, z);
    const int hq = kvh * a.n_rep + R / a.L;
    float* dst = a.out + (((int64_t)b * a.Hkv * a.n_rep + hq) * a.L + R % a.L) * D + 4 * tid;
    *reinterpret_cast<float4*>(dst) = make_float4(z[0], z[1], z[2], z[3]);
}

}  // namespace

// Workgroups of one shape that fit a compute unit: LDS (160 KiB, the tile
// arrays and the staging for the call's widths) and two waves per SIMD at
// most.
template <int D, int NG, int W>
int tile_fit(int kbits, int vbits, bool reg) {
    // register-staged tiles need no staging array
    const int lds = reg ? TileLds<D, W, NG, true>::bytes
                        : TileLds<D, W, NG>::bytes + raw_bytes(D, NG, kbits, vbits);
    const int by_lds = 160 * 1024 / lds;
    const int by_waves = 8 / W;
    return by_lds < by_waves ? by_lds : by_waves;
}

static int tile_workgroups_per_cu(int D, int ng, int W, int kbits, int vbits, bool reg) {
#define RBQ_FIT(D_, NG_)                                                   \
    if (D == D_ && ng == NG_)                                              \
        return W == 4 ? tile_fit<D_, NG_, 4>(kbits, vbits, false) : tile_fit<D_, NG_, 1>(kbits, vbits, reg);
    RBQ_FIT(64, 1) RBQ_FIT(64, 2) RBQ_FIT(128, 1) RBQ_FIT(128, 2) RBQ_FIT(128, 4)
#undef RBQ_FIT
#define RBQ_FIT(D_, NG_) \
    if (D == D_ && ng == NG_) return W == 4 ? tile_fit<D_, NG_, 4>(kbits, vbits, false) : tile_fit<D_, NG_, 1>(kbits, vbits, false);
    RBQ_FIT(256, 2) RBQ_FIT(256, 4) RBQ_FIT(256, 8)
#undef RBQ_FIT
    return 1;
}

int tile_plan(const rbq_kv_cache* c, int32_t H_q, int32_t L, int32_t splits, TilePlan* p) {
    const int64_t G = (int64_t)(H_q / c->H_kv) * L;
    // waves per workgroup, 16 rows each: one wave for up to 8 rows (paired
    // hi / lo operand rows; at head_dim 256 with 4 groups per row 7 % faster
    // than four-wave blocks, with 2 groups 1.5 %), and for up to 16 rows at
    // head_dim <= 128 and at head_dim 256 with 8 groups per row (1.4x
    // faster there); four otherwise.  At head_dim 256 the one-wave builds
    // hold more than 256 registers, so they run one wave per SIMD with part
    // of their state in the accumulation registers: for 9 to 16 rows with 2
    // groups per row that is slower than four-wave blocks, and the unpaired
    // build for 4 groups per row gives wrong results (errors up to 0.7 that
    // grow with the tiles a workgroup walks) that the paired builds and the
    // 2- and 8-group builds of the same source do not show and that no
    // difference in the source explains; built with the matrix results kept
    // in VGPRs instead of AGPRs the same source gives the right results, and
    // for 9 to 16 rows it is no faster than four-wave blocks: that build is
    // not used
    const int ng = c->head_dim / c->group_size;
    const int W = (G <= 8 || (G <= 16 && (c->head_dim <= 128 || ng == 8))) ? 1 : 4;
    // up to 8 rows per kv head at head_dim <= 128 with 4-bit K codes (they
    // enter the MFMAs in place) and 2-, 3- or 4-bit V codes: single-wave
    // workgroups with register-staged tiles (the widths fixed at compile
    // time) and paired hi / lo operand rows
    const bool reg = W == 1 && G <= 8 && c->head_dim <= 128 && c->k_bits == 4 && c->v_bits >= 2 &&
                     c->v_bits <= 4;
    // other widths and head dims, up to 8 rows: staged tiles, paired rows
    const bool pr = W == 1 && G <= 8 && !reg;
    const int64_t RW = 16 * W;
    const int64_t RBW = (G + RW - 1) / RW;
    const int64_t T = c->offset;
    const int64_t units = (int64_t)c->B * c->H_kv * RBW;
    int64_t S = splits;
    if (S == 0) {
        // one round of workgroups over the 256 compute units, as many per
        // unit as LDS and registers allow (longer splits lose less to set-up
        // and records than a second round gains)
        const int per_cu = tile_workgroups_per_cu(c->head_dim, ng, W, c->k_bits, c->v_bits, reg);
        S = (256 * per_cu + units - 1) / units;
        const int64_t max_s = (T + tTile - 1) / tTile;
        if (S > max_s) S = max_s;
    }
    if (S < 1) S = 1;
    if (S > tMaxSplits) S = tMaxSplits;
    int64_t chunk = (T + S - 1) / S;
    chunk = (chunk + tTile - 1) / tTile * tTile;
    S = (T + chunk - 1) / chunk;
    if (units > 0x7FFFFFFF || units * S > 0x7FFFFFFF || units * RW > 0x7FFFFFFF)
        return RBQ_EUNSUPPORTED;
    // one launch of each kernel: at most 2^32 - 1 work-items along x
    if (units * S * 64 * W > 0xFFFFFFFFll ||
        (S > 1 && units * 16 * W * 256 > 0xFFFFFFFFll))
        return RBQ_EUNSUPPORTED;
    // 32-bit buffer offsets of the tile transfers, up to one tile past T
    const int64_t bits = c->k_bits > c->v_bits ? c->k_bits : c->v_bits;
    if ((T + tTile) * (int64_t)c->head_dim * bits / 8 > 0x7FFFFFFF) return RBQ_EUNSUPPORTED;
    p->S = (int)S;
    p->RBW = (int)RBW;
    p->W = W;
    p->reg = reg ? 1 : 0;
    p->pr = pr ? 1 : 0;
    p->chunk = chunk;
    p->o_floats = (size_t)(units * S) * RW * c->head_dim;
    // one split: the attention kernel stores the output itself
    p->ws_bytes = (S == 1) ? 0 : (p->o_floats + (size_t)(units * S) * RW * 2) * sizeof(float);
    return RBQ_OK;
}

// The register-staged kernels of head_dim D (at most 128), NG groups per
// row, 4-bit K and vbits-bit V (2, 3 or 4).
template <int D, int NG, typename F>
static void launch_reg(F&& launch, bool bf, int vbits) {
    if constexpr (D <= 128) {
        if (vbits == 2)
            bf ? launch(attn_tile_kernel<RBQ_BF16, D, NG, 1, 4, 2>) : launch(attn_tile_kernel<RBQ_F16, D, NG, 1, 4, 2>);
        else if (vbits == 3)
            bf ? launch(attn_tile_kernel<RBQ_BF16, D, NG, 1, 4, 3>) : launch(attn_tile_kernel<RBQ_F16, D, NG, 1, 4, 3>);
        else
            bf ? launch(attn_tile_kernel<RBQ_BF16, D, NG, 1, 4, 4>) : launch(attn_tile_kernel<RBQ_F16, D, NG, 1, 4, 4>);
    }
}

int tile_launch(const rbq_kv_cache* c, const void* q, int32_t H_q, int32_t L, float scale,
                int32_t causal, const AttnMask& mk, const float* rot_blocks, float* out,
                const TilePlan& p, void* ws, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    TArgs a;
    a.q = (const uint16_t*)q;
    a.kw = c->k_words;
    a.ks = (const uint16_t*)c->k_scales;
    a.kb = (const uint16_t*)c->k_biases;
    a.vw = c->v_words;
    a.vs = (const uint16_t*)c->v_scales;
    a.vb = (const uint16_t*)c->v_biases;
    a.rot = rot_blocks;
    a.rec_o = (float*)ws;
    a.rec_ml = (float*)ws + p.o_floats;
    a.out = out;
    a.capacity = c->capacity;
    a.T = (int)c->offset;
    a.chunk = (int)p.chunk;
    a.S = p.S;
    a.Hkv = c->H_kv;
    a.n_rep = H_q / c->H_kv;
    a.L = L;
    a.G = a.n_rep * L;
    a.RBW = p.RBW;
    a.causal = causal ? 1 : 0;
    a.round_rot = (c->flags & RBQ_FLAG_ROUND_ROTATED) ? 1 : 0;
    a.GS = c->group_size;
    a.kbits = c->k_bits;
    a.vbits = c->v_bits;
    a.qscale = scale * tLog2e;
    a.raw_vw = raw_vw_off(c->head_dim, c->k_bits);
    a.raw_meta = raw_meta_off(c->head_dim, c->k_bits, c->v_bits);
    const int ng = c->head_dim / c->group_size;
    const size_t dyn = p.reg ? 0 : (size_t)raw_bytes(c->head_dim, ng, c->k_bits, c->v_bits);
    a.mask = mk.ptr;
    a.msb = mk.sb;
    a.msh = mk.sh;
    a.msl = mk.sl;
    a.mask_bytes = mk.bytes;
    a.mtype = mk.ptr == nullptr ? 0 : mk.type;
    const int64_t units = (int64_t)c->B * c->H_kv * p.RBW;
    const dim3 grid((unsigned)(units * p.S)), block(64 * p.W);
    auto launch = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, block, dyn, s, a); };
    const bool bf = c->dtype == RBQ_BF16;
#define RBQ_TILE_CASE(D_, NG_)                                                                    \
    if (c->head_dim == D_ && ng == NG_) {                                                         \
        if (p.W == 4)                                                                             \
            bf ? launch(attn_tile_kernel<RBQ_BF16, D_, NG_, 4>) : launch(attn_tile_kernel<RBQ_F16, D_, NG_, 4>); \
        else if (p.reg && D_ <= 128)                                                              \
            launch_reg<D_, NG_>(launch, bf, c->v_bits);                                            \
        else if (p.pr)                                                                            \
            bf ? launch(attn_tile_kernel<RBQ_BF16, D_, NG_, 1, 0, 0, 1>)                         \
               : launch(attn_tile_kernel<RBQ_F16, D_, NG_, 1, 0, 0, 1>);                          \
        else                                                                                      \
            bf ? launch(attn_tile_kernel<RBQ_BF16, D_, NG_, 1>) : launch(attn_tile_kernel<RBQ_F16, D_, NG_, 1>); \
    } else
#define RBQ_TILE_CASE_PR(D_, NG_)                                                                 \
    if (c->head_dim == D_ && ng == NG_) {                                                         \
        if (p.W == 4)                                                                             \
            bf ? launch(attn_tile_kernel<RBQ_BF16, D_, NG_, 4>) : launch(attn_tile_kernel<RBQ_F16, D_, NG_, 4>); \
        else                                                                                      \
            bf ? launch(attn_tile_kernel<RBQ_BF16, D_, NG_, 1, 0, 0, 1>)                         \
               : launch(attn_tile_kernel<RBQ_F16, D_, NG_, 1, 0, 0, 1>);                          \
    } else
#define RBQ_TILE_CASE4(D_, NG_)                                                                   \
    if (c->head_dim == D_ && ng == NG_) {                                                         \
        bf ? launch(attn_tile_kernel<RBQ_BF16, D_, NG_, 4>) : launch(attn_tile_kernel<RBQ_F16, D_, NG_, 4>); \
    } else
    RBQ_TILE_CASE(64, 1) RBQ_TILE_CASE(64, 2) RBQ_TILE_CASE(128, 1) RBQ_TILE_CASE(128, 2)
    RBQ_TILE_CASE(128, 4) RBQ_TILE_CASE_PR(256, 2) RBQ_TILE_CASE_PR(256, 4) RBQ_TILE_CASE(256, 8) {
        return RBQ_EUNSUPPORTED;
    }
#undef RBQ_TILE_CASE
#undef RBQ_TILE_CASE4
#undef RBQ_TILE_CASE_PR
    if (p.S == 1) {
        const hipError_t e1 = hipGetLastError();
        if (e1 != hipSuccess) {
            set_hip_error((int)e1);
            return RBQ_EHIP;
        }
        return RBQ_OK;
    }
    TMArgs m;
    m.rec_o = a.rec_o;
    m.rec_ml = a.rec_ml;
    m.rot = rot_blocks;
    m.out = out;
    m.S = p.S;
    m.Hkv = a.Hkv;
    m.n_rep = a.n_rep;
    m.L = L;
    m.G = a.G;
    m.RBW = p.RBW;
    m.RW = 16 * p.W;
    m.bool_mask = (a.mtype == RBQ_MASK_BOOL) ? 1 : 0;
    m.dt = c->dtype;
    m.T = a.T;
    m.causal = a.causal;
    m.vbits = c->v_bits;
    m.GS = c->group_size;
    m.capacity = c->capacity;
    m.vw = a.vw;
    m.vs = a.vs;
    m.vb = a.vb;
    const dim3 mgrid((unsigned)(units * 16 * p.W)), mblock(256);
    switch (c->head_dim) {
        case 64: hipLaunchKernelGGL(attn_tile_merge_kernel<64>, mgrid, mblock, 0, s, m); break;
        case 128: hipLaunchKernelGGL(attn_tile_merge_kernel<128>, mgrid, mblock, 0, s, m); break;
        default: hipLaunchKernelGGL(attn_tile_merge_kernel<256>, mgrid, mblock, 0, s, m); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_hip_error((int)e);
        return RBQ_EHIP;
    }
    return RBQ_OK;
}

}  // namespace rbq
