// Prefill-length attention over the packed K4/V3 cache (asym_quantized_sdpa
// on the quant_kv.py page with many query rows per kv head: a prompt chunk
// of L tokens attending to the cache and to itself, causal at the offset) on
// the gfx950 matrix cores, for bf16 and fp16 caches with 4-bit K codes in
// groups of 64 or 128 (head_dim 64, 128 or 256, 2- to 4-bit V codes).
//
// Decomposition: one workgroup of 8 wave64s per (b, kv head, block of 128
// query rows, key split); wave w takes rows 16 w .. 16 w + 15 of the block,
// lane l = 16 j + n row n.  The workgroup walks the split's 32-key tiles:
// each tile is transferred once into LDS (direct-to-LDS, the next tile in
// flight while one is computed), decoded once, and then used by all 128
// rows, so the per-key work (unpacking, scaling) is spread over 128 rows
// instead of the 8 of the decode kernel.
//
// Both products are computed transposed, so that each lane holds one query
// row throughout (the softmax statistics, the probabilities and the output
// accumulators of row n live in lanes n, n + 16, n + 32, n + 48):
//   S^T = K Q^T: A = K codes of 16 keys (row = key), in place as fp16
//     subnormals (masking nibble pairs of a packed word gives c 2^-24 or
//     16 c 2^-24), B = the query (column = query row), hi and lo fp16 parts
//     scaled by a power of two per row, dims permuted and scaled by 1 or 1/16
//     to match the nibble masks.  One accumulator per 64-dim group g; the
//     score of (key t, row r) is 2^(24 - E_r) sum_g s_{t,g} acc_g plus
//     sum_g b_{t,g} sum_{d in g} q_{r,d} (one bf16 MFMA of the raw K bias
//     words against exact limbs of the query's group sums).  Accumulator
//     register i of lane (j, n) holds key 16 kb + 4 j + i of row n.
//   O^T = V'^T P^T: B = P^T, whose k-slot e of lane (j, n) is the lane's own
//     probability (kb = e / 4, i = e % 4), i.e. key 4 j + e (e < 4) or
//     16 + 4 j + e - 4: no transposition of P.  A = V'^T, V' = s_{t,g} 2^F_g
//     c_{t,d} in fp16, stored in LDS with its key rows in that same order
//     and read by the transposing LDS read (ds_read_b64_tr_b16).  For bf16
//     scales V' is exact (8 + 3 significant bits), with F_g a power of two
//     per group, from the split's largest |scale| and |bias|, that keeps
//     every V' and bias below 2^13 * 7 < 65504; the group bias enters as
//     sum_t p_t b_{t,g} 2^F_g through one more MFMA.  P enters as fp16 hi +
//     lo (two MFMAs), so P V' is exact up to fp32 accumulation.
// Online softmax in base 2 per row, the reference maximum moved only when a
// tile's maximum exceeds it by more than 8 (probabilities stay below 2^8).
// With one split the workgroup normalises, rotates back and stores the
// rows; with several it stores the records the merge kernel reads.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "rbq_common.h"
#include "rbq_internal.h"

namespace rbq {
namespace {

typedef _Float16 pf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 pf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 pbf16x8 __attribute__((ext_vector_type(8)));
typedef float pf32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t pu32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t pu32x2 __attribute__((ext_vector_type(2)));
typedef short ps16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char plds_u8;

constexpr int kPW = 8;                // waves per workgroup (4 or 8)
static_assert(kPW == 4 || kPW == 8, "4 or 8 waves");
constexpr int kPT = 64 * kPW;         // threads
constexpr int kPRows = 16 * kPW;      // query rows per workgroup
constexpr int kPTile = 32;            // keys per tile
constexpr int64_t kPGridYZ = 65535;   // workgroups per grid dimension y or z of one launch
constexpr float kPLog2e = 1.44269504088896340736f;
// Layout of one configuration: head_dim D (64, 128 or 256), blocks of 64 dims,
// 4-bit K codes, VB-bit V codes (2, 3 or 4).
//   A raw buffer holds one tile as the memory holds it: K words (16-byte
//   chunks of a key permuted, see k_chunk), V words, K scales, K biases, V
//   scales, V biases.  LDS (bytes): three raw buffers (tile i + 2 in flight
//   while tile i + 1 is decoded and tile i computed), two decoded tiles (V',
//   and for 4-bit codes its residual V'', see the decode), K scales and V
//   bias operands of both, the rotation blocks, group maxima, scale powers;
//   with fp16 caches also the K biases of both as bf16 hi and lo parts.
template <int D, int VB, int DT>
struct PCfg {
    static constexpr int NG = D / 64;                     // blocks of 64 dims (groups of 64)
    static constexpr int NB = D / 16;                     // 16-dim output blocks
    static constexpr int CPK = D / 32;                    // 16-byte K chunks per key
    static constexpr int KPB = 512 / D;                   // keys per 256 bytes of K words
    static constexpr int VWK = D * VB / 32;               // V words per key
    static constexpr int RK = 0;
    static constexpr int RV = RK + kPTile * D / 2;
    static constexpr int RKs = RV + kPTile * VWK * 4;
    static constexpr int MB = kPTile * NG * 2;            // bytes of each scale / bias array
    static constexpr int RKb = RKs + MB, RVs = RKb + MB, RVb = RVs + MB;
    static constexpr int RAW = (RVb + MB + 15) / 16 * 16;
    // V' = code x scale: up to 3 + 8 significant bits with bf16 scales (one
    // fp16 array), up to 4 + 8 or VB + 11 otherwise (V' + its residual V'')
    static constexpr bool VSPLIT = VB > 3 || DT == RBQ_F16;
    static constexpr int NDEC = VSPLIT ? 2 : 1;           // decoded arrays per tile
    // decoded rows: 2 D + 160 bytes apart, rows 8-15 and 24-31 shifted by 128
    // bytes, so that the transposing reads of 32 lanes (rows 8 j' + e of two
    // lane groups j') fall on distinct banks
    static constexpr int VROW = 2 * D + 160;
    static constexpr int DEC = kPTile * VROW + 128;       // one decoded array
    static constexpr int OffV = 3 * RAW;
    static constexpr int OffKs = OffV + 2 * NDEC * DEC;   // fp32 [NG][32] per tile
    static constexpr int OffVb = OffKs + 2 * NG * kPTile * 4;  // fp16 [NG][32] per tile
    static constexpr int OffKb2 = OffVb + 2 * NG * kPTile * 2;  // fp16 caches: bf16 [32][2 NG] per tile
    static constexpr int OffRot = OffKb2 + (DT == RBQ_F16 ? 2 * kPTile * 2 * NG * 2 : 0);
    static constexpr int OffRed = OffRot + D * 16;        // [8 waves][4] group maxima
    static constexpr int OffUnit = OffRed + kPW * 16;     // 2^F_g, then 2^-F_g
    static constexpr int BYTES = OffUnit + 32;
    static constexpr int KI = D / 64;                     // K transfers (64 lanes x 16 bytes)
    static constexpr int VCH = kPTile * VWK / 4;          // 16-byte V chunks
    static constexpr int VI = (VCH + 63) / 64;            // V transfers
    static constexpr int NI = KI + VI + 4;                // + one per scale / bias array
    static_assert(BYTES <= 160 * 1024, "LDS of one compute unit");
    static_assert(D <= kPT, "one float4 of the rotation blocks per thread");
    __host__ __device__ static constexpr int v_off(int r) { return r * VROW + ((r >> 3) & 1) * 128; }
};
static_assert(kRecordFloats == 2 * 8 + 8 * kHeadDim, "split record layout");

struct PArgs {
    const uint16_t* q;
    const uint32_t* kw;
    const uint16_t* ks;
    const uint16_t* kb;
    const uint32_t* vw;
    const uint16_t* vs;
    const uint16_t* vb;
    const float* rot;
    float* out;
    float* rec;
    const void* mask;
    int64_t msb, msh, msl;
    uint32_t mask_bytes;
    int64_t capacity;
    int T, chunk, S, Hkv, n_rep, L, G, RB, RW, causal, round_rot;
    int rw0, bh0;  // first row block and (b, kv head) of this launch (grid y and z)
    float qscale;
};

__device__ __forceinline__ pf32x4 mfma_f16(pf16x8 a, pf16x8 b, pf32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ pf32x4 mfma_bf16(pu32x4 a, pu32x4 b, pf32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(pbf16x8, a),
                                                     __builtin_bit_cast(pbf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t prsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// LDS transposing read of 8 bytes at byte offset `off`: lane i of each
// 16-lane group gets element i & 3 of the 8 bytes addressed by lanes
// 4 e + (i >> 2) of its group, as element e.
__device__ __forceinline__ pu32x2 tr_read(const unsigned char* smem, uint32_t off) {
    const ps16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) ps16x4*)((plds_u8*)smem + off));
    return __builtin_bit_cast(pu32x2, v);
}

// Direct-to-LDS buffer loads of 16 or 4 bytes per lane (wrapped: called with
// template-dependent arguments the builtin stops the host pass from
// instantiating the kernel)
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, plds_u8* dst, int off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t r, plds_u8* dst, int off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, off, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ T lds_ld(const unsigned char* smem, uint32_t off) {
    return *(const __attribute__((address_space(3))) T*)((const plds_u8*)smem + off);
}
template <typename T>
__device__ __forceinline__ void lds_st(unsigned char* smem, uint32_t off, T v) {
    *(__attribute__((address_space(3))) T*)((plds_u8*)smem + off) = v;
}

// max / sum over the 4 lanes n, n + 16, n + 32, n + 48 (one row)
__device__ __forceinline__ float row_max4(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row_sum4(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// (fp16(p0 - h0), fp16(p1 - h1)) for hi2 = (h0, h1) the fp16 roundings of
// p0, p1: fma(-h, 1, p) with h taken as fp16 and p as fp32, rounded once
// (p - h is exact in fp32).  `one` holds 1.0f.
__device__ __forceinline__ uint32_t lo_parts(uint32_t hi2, float p0, float p1, float one) {
    uint32_t r;
    asm("v_fma_mixlo_f16 %0, -%1, %2, %3 op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixhi_f16 %0, -%1, %2, %4 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "=&v"(r)
        : "v"(hi2), "v"(one), "v"(p0), "v"(p1));
    return r;
}

// 16-byte slot of K word chunk c (words 4c .. 4c+3) of tile key k in a raw
// buffer: the chunks of a key permuted by (k / KPB) mod CPK, so that the
// 8-byte reads of 32 lanes (16 keys x 2 halves of a chunk) hit distinct
// banks.
template <int D>
__device__ __forceinline__ int k_chunk(int k, int c) {
    constexpr int CPK = D / 32, KPB = 512 / D;
    return CPK * k + (c ^ ((k / KPB) & (CPK - 1)));
}

// Row of key k in the decoded V' tile: row 8 j + e holds key 4 j + e
// (e < 4) or 16 + 4 j + e - 4 (e >= 4), the k-slot order of the P operand.
__device__ __forceinline__ int v_row(int k) { return 8 * ((k & 15) >> 2) + (k & 3) + 4 * (k >> 4); }

template <int MK, int D, int VB, int DT, int GSH>
__global__ __launch_bounds__(kPT) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_prefill_kernel(PArgs a) {
    using C = PCfg<D, VB, DT>;
    constexpr int NG = C::NG, NB = C::NB;
    __shared__ __align__(16) unsigned char smem[C::BYTES];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane >> 4, n = lane & 15;

    // grid: x = key split, y = block of 128 query rows, z = (b, kv head)
    const int split = blockIdx.x;
    const int rw = a.rw0 + blockIdx.y;
    const int bh = a.bh0 + blockIdx.z;
    const int r0 = kPRows * rw;
    const int T = a.T;
    const int t_begin = split * a.chunk;
    const int t_end = min(t_begin + a.chunk, T);
    // keys past the last visible key of every row of the block are skipped
    int t_lim = t_end;
    if (a.causal) {
        const int rlast = min(r0 + kPRows, a.G) - 1;
        const int i0 = r0 % a.L, i1 = rlast % a.L;
        const int imax = (rlast - r0 + 1 >= a.L || i1 < i0) ? a.L - 1 : i1;
        t_lim = min(t_lim, T - a.L + imax + 1);
    }
    const int64_t row0 = (int64_t)bh * a.capacity;
    // the kernel works in blocks of 64 dims (NG per row); the cache's scale
    // and bias arrays hold NGS = NG >> GSH values per row, one per group of
    // 64 << GSH dims, and block g takes value g >> GSH (a group of 128 dims is
    // two blocks with its scale and bias: the same sums)
    constexpr int gsh = GSH;
    constexpr int NGS = NG >> gsh;
    static_assert(NGS >= 1, "a group spans at most the head");
    const __amdgpu_buffer_rsrc_t kw_r = prsrc(a.kw + row0 * (D / 8), (uint32_t)T * (D / 2));
    const __amdgpu_buffer_rsrc_t vw_r = prsrc(a.vw + row0 * C::VWK, (uint32_t)T * (C::VWK * 4));
    __amdgpu_buffer_rsrc_t m_r[4];
    m_r[0] = prsrc(a.ks + row0 * NGS, (uint32_t)T * (2 * NGS));
    m_r[1] = prsrc(a.kb + row0 * NGS, (uint32_t)T * (2 * NGS));
    m_r[2] = prsrc(a.vs + row0 * NGS, (uint32_t)T * (2 * NGS));
    m_r[3] = prsrc(a.vb + row0 * NGS, (uint32_t)T * (2 * NGS));

    // Direct-to-LDS transfer of the tile at key t0 into raw buffer `buf` (lane
    // l of an instruction lands at offset + 16 l or 4 l): NI instructions,
    // wave w issuing numbers w, w + kPW, ...: the K words in 64-lane pieces,
    // the V words likewise (the last piece on fewer lanes where it is short),
    // then one per scale / bias array.  Keys past the buffer ranges read as
    // zero.
    auto issue_tile = [&](plds_u8* buf, const int t0) __attribute__((always_inline)) {
#pragma unroll
        for (int x = 0; x < C::NI; x += kPW) {
            const int idx = x + wave;
            if (idx < C::KI) {
                const int p = 64 * idx + lane;
                const int k = p / C::CPK;
                const int c = (p % C::CPK) ^ ((k / C::KPB) & (C::CPK - 1));
                lds_dma16(kw_r, buf + C::RK + 1024 * idx, (t0 + k) * (D / 2) + 16 * c);
            } else if (idx < C::KI + C::VI) {
                const int m = idx - C::KI;
                if (64 * m + lane < C::VCH)
                    lds_dma16(vw_r, buf + C::RV + 1024 * m, t0 * (C::VWK * 4) + 16 * (64 * m + lane));
            } else if (idx < C::NI) {
                const int m = idx - C::KI - C::VI;
                const uint32_t dst = (m == 0) ? C::RKs : (m == 1) ? C::RKb : (m == 2) ? C::RVs : C::RVb;
                if (lane < 16 * NGS) lds_dma4(m_r[m], buf + dst, t0 * (2 * NGS) + 4 * lane);
            }
        }
    };
    // the first tile in flight during the set-up
    if (t_begin < t_lim) issue_tile((plds_u8*)smem, t_begin);

    // ---- the query row of this lane (dims 64 g + 16 j .. 64 g + 16 j + 15)
    //      and the rotation blocks into LDS ----
    const int R = r0 + 16 * wave + n;
    const bool row_ok = R < a.G;
    float x[NG][16];
    {
        const uint16_t* qr = a.q + ((int64_t)bh * a.G + (row_ok ? R : 0)) * D;
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                if (row_ok) {
                    load4<DT>(qr + 64 * g + 16 * j + 4 * q4, x[g] + 4 * q4);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[g][4 * q4 + e] = 0.f;
                }
            }
    }
    const bool rotated = a.rot != nullptr;
    // (D / 4 blocks of 16 floats: one float4 per thread of the first D)
    if (rotated && tid < D)
        lds_st<pf32x4>(smem, C::OffRot + 16 * tid, reinterpret_cast<const pf32x4*>(a.rot)[tid]);

    // ---- F_g: the power of two that keeps the split's V scales and biases
    //      of group g below 2^13 (over the keys this workgroup reads) ----
    float vmx[4] = {0.f, 0.f, 0.f, 0.f};
    for (int t = t_begin + tid; t < t_lim; t += kPT) {
#pragma unroll
        for (int g = 0; g < NG; ++g)
            vmx[g] = fmaxf(vmx[g], fmaxf(fabsf(elem_to_f32<DT>(a.vs[(row0 + t) * NGS + (g >> gsh)])),
                                         fabsf(elem_to_f32<DT>(a.vb[(row0 + t) * NGS + (g >> gsh)]))));
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) vmx[g] = fmaxf(vmx[g], __shfl_xor(vmx[g], o));
    }
    if (lane == 0) lds_st<pf32x4>(smem, C::OffRed + 16 * wave, (pf32x4){vmx[0], vmx[1], vmx[2], vmx[3]});
    __syncthreads();  // rotation blocks and group maxima in LDS
    {
        float mx[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kPW; ++w) {
            const pf32x4 v = lds_ld<pf32x4>(smem, C::OffRed + 16 * w);
#pragma unroll
            for (int g = 0; g < 4; ++g) mx[g] = fmaxf(mx[g], v[g]);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            int ex = 0;
            if (mx[g] > 0.f) (void)frexpf(mx[g], &ex);  // mx < 2^ex
            const int F = (mx[g] > 0.f) ? 13 - ex : 0;
            if (tid == g) {
                lds_st<float>(smem, C::OffUnit + 4 * g, ldexpf(1.0f, F));
                lds_st<float>(smem, C::OffUnit + 16 + 4 * g, ldexpf(1.0f, -F));
            }
        }
    }

    // ---- rotate, round (when the cache asks for it), scale by scale *
    //      log2(e); E: the power of two that brings the row's largest |q|
    //      into [2^14, 2^15); the group sums ----
    float E_f;
    pf16x8 qh[NG][2], ql[NG][2];
    pu32x4 qb = {0u, 0u, 0u, 0u};
    {
        float mx = 0.f;
        float gsum[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            gsum[g] = 0.f;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                float y[4];
                if (rotated) {
                    float Bm[16];
                    const int blk = 16 * g + 4 * j + q4;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const pf32x4 v = lds_ld<pf32x4>(smem, C::OffRot + 64 * blk + 16 * r);
#pragma unroll
                        for (int e = 0; e < 4; ++e) Bm[4 * r + e] = v[e];
                    }
                    rotate4(x[g] + 4 * q4, Bm, y);
                    if (a.round_rot) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) y[e] = elem_to_f32<DT>(f32_to_elem_bits<DT>(y[e]));
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) y[e] = x[g][4 * q4 + e];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v = y[e] * a.qscale;
                    x[g][4 * q4 + e] = v;
                    mx = fmaxf(mx, fabsf(v));
                    gsum[g] += v;
                }
            }
        }
        mx = row_max4(mx);
        int ex = 0;
        if (mx > 0.f) (void)frexpf(mx, &ex);
        const int E = (mx > 0.f) ? 15 - ex : 0;
        E_f = ldexpf(1.0f, 24 - E);
        // score operands: word 8 g + 2 j + h2 of a key covers dims
        // 64 g + 16 j + 8 h2 + 0..7; slot e takes dim kPerm[e] of those, times
        // 1/16 where the nibble mask leaves 16 c
        constexpr int kPerm[8] = {0, 4, 1, 5, 2, 6, 3, 7};
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float xs = ldexpf(x[g][8 * h2 + kPerm[e]], E) * ((e & 2) ? 0.0625f : 1.0f);
                    const _Float16 hi = (_Float16)xs;
                    qh[g][h2][e] = hi;
                    ql[g][h2][e] = (_Float16)(xs - (float)hi);
                }
        // bias operand: lane group j < 3 holds limb j of the NG group sums
        // (exact three-limb bf16 split) in k-slots 0 .. NG - 1; with fp16
        // caches again in k-slots NG .. 2 NG - 1, against the lo parts of the
        // K biases (an fp16 bias is its bf16 truncation plus an exact bf16 rest)
        uint32_t lb[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const float s = row_sum4(gsum[g]);
            const uint32_t u = __float_as_uint(s);
            const float hi = __uint_as_float(u & 0xFFFF0000u);
            const uint32_t u2 = __float_as_uint(s - hi);
            const float mid = __uint_as_float(u2 & 0xFFFF0000u);
            lb[g] = (j == 0) ? u >> 16 : (j == 1) ? u2 >> 16 : (j == 2) ? f32_to_bf16_bits(s - hi - mid) : 0u;
            if constexpr (DT == RBQ_F16) lb[NG + g] = lb[g];
        }
        qb = (pu32x4){lb[0] | lb[1] << 16, lb[2] | lb[3] << 16, lb[4] | lb[5] << 16, lb[6] | lb[7] << 16};
    }
    const float frow = E_f;
    // causal visibility of the lane's row, and the smallest over the wave's rows
    const int vis = (row_ok && a.causal) ? T - a.L + (R % a.L) + 1 : T;
    int vis_min = row_ok ? vis : T;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) vis_min = min(vis_min, __shfl_xor(vis_min, o));
    vis_min = __builtin_amdgcn_readfirstlane(vis_min);
    const bool wave_live = r0 + 16 * wave < a.G;

    // mask: byte offset of the lane's row (reads past the range return zero)
    constexpr int kME = (MK == RBQ_MASK_BOOL) ? 1 : (MK == RBQ_MASK_ADD_F32) ? 4 : 2;
    __amdgpu_buffer_rsrc_t mask_r;
    uint32_t mrow = 0x80000000u;
    if constexpr (MK != RBQ_MASK_NONE) {
        mask_r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.mask), (short)0,
                                                   (int)a.mask_bytes, 0x00020000);
        if (row_ok) {
            const int b = bh / a.Hkv;
            const int h = (bh - b * a.Hkv) * a.n_rep + R / a.L;
            mrow = (uint32_t)(((int64_t)b * a.msb + (int64_t)h * a.msh + (int64_t)(R % a.L) * a.msl) * kME);
        }
    }

    pf32x4 O[NB];
#pragma unroll
    for (int t = 0; t < NB; ++t) O[t] = (pf32x4){0.f, 0.f, 0.f, 0.f};
    pf32x4 Ob = {0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY, thr = -INFINITY, l_part = 0.f;
    const float one = 1.0f;
    const pf32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    // this lane's transposing-read address in the V' tile: lane 4 e + q of a
    // group reads row 8 j + e, columns 4 q .. 4 q + 3 of an output block
    const uint32_t vrd = C::OffV + C::v_off(8 * j + (n >> 2)) + 8 * (n & 3);

    // decode of the tile in raw buffer `raw` into decoded tile `db`: V' rows
    // (item = key i / (D / 16), dims 16 (i mod (D / 16)) .., 2 D items over
    // the threads), K scales to fp32 (waves 0-1), V bias operand (waves 2-3).
    // V' = code x scale x 2^F_g, exact in fp32; in fp16 exact for up to 3-bit
    // codes (8 + 3 significant bits); 4-bit codes keep the residual V'' =
    // V' - fp16(V') (exact) in a second array
    // With one group per row (head_dim 64, or 128 in groups of 128) the scale
    // and bias arrays hold 2 bytes per key, and the 4-byte transfers of a tile
    // that ends at an odd
    // key count T take the pair (T - 1, T) as one word outside the range:
    // it reads as zero, key T - 1's halves included.  The decode of that tile
    // takes key T - 1's four halves from memory instead and puts its K bias
    // into the raw buffer, where the score products read it.
    auto decode_tile = [&](const unsigned char* raw, const int db, const int t0) __attribute__((always_inline)) {
        constexpr int IPK = D / 16;  // items per key
        const int klast = T - 1 - t0;
        const bool fix_last = NGS == 1 && (T & 1) && klast >= 0 && klast < kPTile;
        const int64_t last = row0 + T - 1;  // (one group: element index = row)
#pragma unroll
        for (int item = tid; item < 2 * D; item += kPT) {
            const int k = item / IPK, p = item % IPK, g = p >> 2;
            const int bit0 = 16 * VB * p;
            const int wi = bit0 >> 5, sh = bit0 & 31;
            const uint32_t w0 = lds_ld<uint32_t>(raw, C::RV + 4 * (C::VWK * k + wi));
            const uint32_t w1 = lds_ld<uint32_t>(raw, C::RV + 4 * (C::VWK * k + wi + 1));
            const uint64_t bits = (((uint64_t)w1 << 32) | w0) >> sh;
            const uint32_t sv = (fix_last && k == klast) ? (uint32_t)a.vs[last]
                                                         : lds_ld<uint16_t>(raw, C::RVs + 2 * (NGS * k + (g >> gsh)));
            const float sf = elem_to_f32<DT>(sv) * lds_ld<float>(smem, C::OffUnit + 4 * g);
            constexpr uint32_t cm = (1u << VB) - 1u;
            uint32_t h[8], hl[8];
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                const float v0 = (float)(uint32_t)((bits >> (VB * 2 * d)) & cm) * sf;
                const float v1 = (float)(uint32_t)((bits >> (VB * (2 * d + 1))) & cm) * sf;
                const _Float16 h0 = (_Float16)v0, h1 = (_Float16)v1;
                h[d] = __builtin_bit_cast(uint32_t, (pf16x2){h0, h1});
                if constexpr (C::VSPLIT)
                    hl[d] = __builtin_bit_cast(uint32_t, (pf16x2){(_Float16)(v0 - (float)h0),
                                                                  (_Float16)(v1 - (float)h1)});
            }
            const uint32_t dst = C::OffV + db * C::NDEC * C::DEC + C::v_off(v_row(k)) + 32 * p;
            lds_st<pu32x4>(smem, dst, (pu32x4){h[0], h[1], h[2], h[3]});
            lds_st<pu32x4>(smem, dst + 16, (pu32x4){h[4], h[5], h[6], h[7]});
            if constexpr (C::VSPLIT) {
                lds_st<pu32x4>(smem, dst + C::DEC, (pu32x4){hl[0], hl[1], hl[2], hl[3]});
                lds_st<pu32x4>(smem, dst + C::DEC + 16, (pu32x4){hl[4], hl[5], hl[6], hl[7]});
            }
        }
        if (wave < 2) {
            if (tid < kPTile * NG) {
                const int kk = tid / NG, gg = tid % NG;
                uint32_t sk = lds_ld<uint16_t>(raw, C::RKs + 2 * (NGS * kk + (gg >> gsh)));
                uint32_t bk = 0u;
                if constexpr (DT == RBQ_F16) bk = lds_ld<uint16_t>(raw, C::RKb + 2 * (NGS * kk + (gg >> gsh)));
                if (fix_last && kk == klast) {
                    sk = a.ks[last];
                    bk = a.kb[last];
                    if constexpr (DT == RBQ_BF16)
                        lds_st<uint16_t>(const_cast<unsigned char*>(raw), C::RKb + 2 * kk, (uint16_t)bk);
                }
                if constexpr (DT == RBQ_F16) {
                    // bf16 truncation of the fp16 bias and the exact bf16 rest
                    const float bf = elem_to_f32<RBQ_F16>(bk);
                    const uint32_t hb = __float_as_uint(bf) & 0xFFFF0000u;
                    const uint32_t lo = __float_as_uint(bf - __uint_as_float(hb)) >> 16;
                    const uint32_t kb2 = C::OffKb2 + db * (kPTile * 2 * NG * 2) + 2 * (2 * NG * kk);
                    lds_st<uint16_t>(smem, kb2 + 2 * gg, (uint16_t)(hb >> 16));
                    lds_st<uint16_t>(smem, kb2 + 2 * (NG + gg), (uint16_t)lo);
                }
                lds_st<float>(smem, C::OffKs + db * (NG * kPTile * 4) + 4 * (gg * kPTile + kk),
                              elem_to_f32<DT>(sk));
            }
        } else if (wave < 4) {
            if (tid - 128 < kPTile * NG) {
                const int kk = (tid - 128) / NG, gg = (tid - 128) % NG;
                const uint32_t b = (fix_last && kk == klast) ? (uint32_t)a.vb[last]
                                                             : lds_ld<uint16_t>(raw, C::RVb + 2 * (NGS * kk + (gg >> gsh)));
                const float bu = elem_to_f32<DT>(b) * lds_ld<float>(smem, C::OffUnit + 4 * gg);
                lds_st<uint16_t>(smem, C::OffVb + db * (NG * kPTile * 2) + 2 * (gg * kPTile + v_row(kk)),
                                 __builtin_bit_cast(uint16_t, (_Float16)bu));
            }
        }
    };
    const int n_tiles = (t_lim > t_begin) ? (t_lim - t_begin + kPTile - 1) / kPTile : 0;
    // the second tile in flight too; the first decoded before the loop
    if (n_tiles > 1)
        issue_tile((plds_u8*)smem + C::RAW, t_begin + kPTile);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (n_tiles > 0) decode_tile(smem, 0, t_begin);

    for (int it = 0; it < n_tiles; ++it) {
        // raw buffer it % 3 holds tile it, (it + 1) % 3 tile it + 1 (landed at
        // the barrier), (it + 2) % 3 receives tile it + 2
        const unsigned char* raw = smem + (it % 3) * C::RAW;
        const unsigned char* raw_next = smem + ((it + 1) % 3) * C::RAW;
        plds_u8* raw_dma = (plds_u8*)smem + ((it + 2) % 3) * C::RAW;
        const int t0 = t_begin + it * kPTile;
        const int db = it & 1;
        // tile it + 1 has landed (each wave waits for its own transfers, the
        // barrier for all), tile it is decoded, every wave is done with tile
        // it - 1 (its raw and decoded buffers are free)
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        const bool dec_next = it + 1 < n_tiles;
        if (it + 2 < n_tiles) issue_tile(raw_dma, t0 + 2 * kPTile);
        if (!wave_live) {
            if (dec_next) decode_tile(raw_next, db ^ 1, t0 + kPTile);
            continue;
        }

        // mask values of the lane's row for keys t0 + 16 kb + 4 j + i
        uint32_t mv[2][4];
        if constexpr (MK != RBQ_MASK_NONE) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t off = mrow + (uint32_t)(t0 + 16 * kb + 4 * j + i) * kME;
                    if constexpr (MK == RBQ_MASK_BOOL)
                        mv[kb][i] = __builtin_amdgcn_raw_buffer_load_b8(mask_r, off, 0, 0);
                    else if constexpr (MK == RBQ_MASK_ADD_F32)
                        mv[kb][i] = __builtin_amdgcn_raw_buffer_load_b32(mask_r, off, 0, 0);
                    else
                        mv[kb][i] = __builtin_amdgcn_raw_buffer_load_b16(mask_r, off, 0, 0);
                }
        }

        // ---- scores S^T: register i of lane (j, n) = key 16 kb + 4 j + i, row n ----
        float sc[2][4];
        const bool full = t0 + kPTile <= t_end && t0 + kPTile <= vis_min;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int key = 16 * kb + n;
            pf32x4 acc[NG];
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const pu32x2 w2 = lds_ld<pu32x2>(raw, C::RK + 16 * k_chunk<D>(key, 2 * g + (j >> 1)) + 8 * (j & 1));
                acc[g] = zero4;
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const uint32_t w = w2[h2];
                    const uint32_t w8 = w >> 8;
                    const pu32x4 kv = {w & 0x000F000Fu, w & 0x00F000F0u, w8 & 0x000F000Fu, w8 & 0x00F000F0u};
                    const pf16x8 kop = __builtin_bit_cast(pf16x8, kv);
                    acc[g] = mfma_f16(kop, qh[g][h2], acc[g]);
                    acc[g] = mfma_f16(kop, ql[g][h2], acc[g]);
                }
            }
            // the key's NG bias halves in k-slots 0 .. NG - 1 (fp16 caches:
            // their bf16 hi parts there and the lo parts in NG .. 2 NG - 1)
            pu32x4 kbop = {0u, 0u, 0u, 0u};
            if constexpr (DT == RBQ_F16) {
                const uint32_t kb2 = C::OffKb2 + db * (kPTile * 2 * NG * 2) + 2 * (2 * NG * key);
                if constexpr (NG == 4) {
                    kbop = lds_ld<pu32x4>(smem, kb2);
                } else if constexpr (NG == 2) {
                    const pu32x2 w = lds_ld<pu32x2>(smem, kb2);
                    kbop = (pu32x4){w[0], w[1], 0u, 0u};
                } else {
                    kbop = (pu32x4){lds_ld<uint32_t>(smem, kb2), 0u, 0u, 0u};
                }
            } else if constexpr (NG == 4) {
                if constexpr (gsh == 0) {
                    const pu32x2 kbw = lds_ld<pu32x2>(raw, C::RKb + 8 * key);
                    kbop = (pu32x4){kbw[0], kbw[1], 0u, 0u};
                } else {  // two groups of 128: each half for both its blocks
                    const uint32_t w = lds_ld<uint32_t>(raw, C::RKb + 4 * key);
                    kbop = (pu32x4){(w & 0xFFFFu) * 0x10001u, (w >> 16) * 0x10001u, 0u, 0u};
                }
            } else if constexpr (NG == 2) {
                if constexpr (gsh == 0)
                    kbop = (pu32x4){lds_ld<uint32_t>(raw, C::RKb + 4 * key), 0u, 0u, 0u};
                else
                    kbop = (pu32x4){(uint32_t)lds_ld<uint16_t>(raw, C::RKb + 2 * key) * 0x10001u, 0u, 0u, 0u};
            } else {
                kbop = (pu32x4){(uint32_t)lds_ld<uint16_t>(raw, C::RKb + 2 * key), 0u, 0u, 0u};
            }
            const pf32x4 cb = mfma_bf16(kbop, qb, zero4);
            // the next tile's decode while the matrix cores work on these
            // products (its buffers are not read by this tile)
            if (kb == 1 && dec_next) decode_tile(raw_next, db ^ 1, t0 + kPTile);
            pf32x4 s4[NG];
#pragma unroll
            for (int g = 0; g < NG; ++g)
                s4[g] = lds_ld<pf32x4>(smem, C::OffKs + db * (NG * kPTile * 4) + 4 * (g * kPTile + 16 * kb + 4 * j));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float t = s4[0][i] * acc[0][i];
#pragma unroll
                for (int g = 1; g < NG; ++g) t = fmaf(s4[g][i], acc[g][i], t);
                float s = fmaf(t, frow, cb[i]);
                if constexpr (MK == RBQ_MASK_BOOL) {
                    if (mv[kb][i] == 0u) s = -INFINITY;
                } else if constexpr (MK == RBQ_MASK_ADD_F32) {
                    s = fmaf(__uint_as_float(mv[kb][i]), kPLog2e, s);
                } else if constexpr (MK == RBQ_MASK_ADD_DTYPE) {
                    s = fmaf(elem_to_f32<DT>(mv[kb][i]), kPLog2e, s);
                }
                sc[kb][i] = s;
            }
        }
        // keys past the split or past the row's last visible key, only in a
        // tile that reaches them
        if (__builtin_expect(!full, 0)) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tk = t0 + 16 * kb + 4 * j + i;
                    if (!(tk < t_end && tk < vis)) sc[kb][i] = -INFINITY;
                }
        }

        // ---- online softmax of row n (base 2; the reference moves only when
        //      the tile's maximum exceeds it by more than 8) ----
        float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                         fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
        mx = row_max4(mx);
        const bool need = mx > thr;
        if (__any(need)) {
            float al = 1.0f;
            if (need) {
                al = __builtin_amdgcn_exp2f(m_ref - mx);  // 0 before the first key
                m_ref = mx;
                thr = mx + 8.0f;
            }
#pragma unroll
            for (int t = 0; t < NB; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) O[t][i] *= al;
#pragma unroll
            for (int i = 0; i < 4; ++i) Ob[i] *= al;
            l_part *= al;
        }
        const float mu = (m_ref == -INFINITY) ? 0.f : m_ref;
        float p[2][4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[kb][i] = __builtin_amdgcn_exp2f(sc[kb][i] - mu);
                l_part += p[kb][i];
            }
        // P^T operand: k-slot e = (kb e / 4, register e % 4), fp16 hi + lo
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
                const float p0 = p[kb][2 * q2], p1 = p[kb][2 * q2 + 1];
                const uint32_t hi2 = __builtin_bit_cast(uint32_t, (pf16x2){(_Float16)p0, (_Float16)p1});
                hw[2 * kb + q2] = hi2;
                lw[2 * kb + q2] = lo_parts(hi2, p0, p1, one);
            }
        const pf16x8 ph = __builtin_bit_cast(pf16x8, (pu32x4){hw[0], hw[1], hw[2], hw[3]});
        const pf16x8 pl = __builtin_bit_cast(pf16x8, (pu32x4){lw[0], lw[1], lw[2], lw[3]});

        // ---- O^T += V'^T P^T (register i of block t: dim 16 t + 4 j + i) ----
        const uint32_t vdb = vrd + db * C::NDEC * C::DEC;
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            const pu32x2 v0 = tr_read(smem, vdb + 32 * t);
            const pu32x2 v1 = tr_read(smem, vdb + 32 * t + 4 * C::VROW);
            const pf16x8 vop = __builtin_bit_cast(pf16x8, (pu32x4){v0[0], v0[1], v1[0], v1[1]});
            O[t] = mfma_f16(vop, ph, O[t]);
            O[t] = mfma_f16(vop, pl, O[t]);
            if constexpr (C::VSPLIT) {
                // the residual against the hi part of P (its lo part's
                // product is below 2^-22 of the term)
                const pu32x2 r0 = tr_read(smem, vdb + C::DEC + 32 * t);
                const pu32x2 r1 = tr_read(smem, vdb + C::DEC + 32 * t + 4 * C::VROW);
                O[t] = mfma_f16(__builtin_bit_cast(pf16x8, (pu32x4){r0[0], r0[1], r1[0], r1[1]}), ph, O[t]);
            }
        }
        {
            // group biases: A row g < 4 = b_{key, g} 2^F_g over the k-slots
            pu32x4 vb4 = {0u, 0u, 0u, 0u};
            if (n < NG) vb4 = lds_ld<pu32x4>(smem, C::OffVb + db * (NG * kPTile * 2) + 2 * (n * kPTile + 8 * j));
            const pf16x8 vbop = __builtin_bit_cast(pf16x8, vb4);
            Ob = mfma_f16(vbop, ph, Ob);
            Ob = mfma_f16(vbop, pl, Ob);
        }
    }
    // no transfer into LDS in flight past the loop
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    // ---- epilogue: row sums, group biases (register g of lanes j = 0) ----
    const float l = row_sum4(l_part);
    float obg[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) obg[g] = row_sum4(Ob[g]);  // groups past NG: 0
    if (!row_ok) return;
    const pf32x4 vinv = lds_ld<pf32x4>(smem, C::OffUnit + 16);
    if (a.S == 1) {
        const float inv = 1.0f / l;
        // a boolean mask dropped every key of the row: the mean of its keys
        const bool uniform = MK == RBQ_MASK_BOOL && l == 0.f;
        float* orow = a.out + ((int64_t)bh * a.G + R) * D;
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            const int g = t >> 2;
            float y[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = (O[t][i] + obg[g]) * vinv[g] * inv;
            if (uniform) {
                const int nv = a.causal ? T - a.L + (R % a.L) + 1 : T;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    y[i] = value_column_mean<DT>(a.vw, a.vs, a.vb, row0, nv, 16 * t + 4 * j + i,
                                                       VB, C::VWK, NGS, 64 << gsh);
            }
            float z[4] = {y[0], y[1], y[2], y[3]};
            if (rotated) {
                float Bm[16];
                const int blk = 4 * t + j;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const pf32x4 v = lds_ld<pf32x4>(smem, C::OffRot + 64 * blk + 16 * r);
#pragma unroll
                    for (int e = 0; e < 4; ++e) Bm[4 * r + e] = v[e];
                }
                unrotate4(y, Bm, z);
            }
            *reinterpret_cast<float4*>(orow + 16 * t + 4 * j) = make_float4(z[0], z[1], z[2], z[3]);
        }
        return;
    }
    // this split's record of the lane's row (block of 8 rows R >> 3, row R & 7)
    constexpr int RF = record_floats(D);
    float* rec = a.rec + ((int64_t)(bh * a.RB + (R >> 3)) * a.S + split) * RF;
    const int ri = R & 7;
#pragma unroll
    for (int t = 0; t < NB; ++t) {
        const int g = t >> 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) rec[16 + (16 * t + 4 * j + i) * 8 + ri] = (O[t][i] + obg[g]) * vinv[g];
    }
    if (j == 0) *reinterpret_cast<float2*>(rec + 2 * ri) = make_float2(m_ref, l);
}

}  // namespace

// ---- host side ----

// The kernel of layout (D, VB) and cache dtype DT for mask type mt, handed
// to `launch`.
template <int D, int VB, int DT, int GSH, typename F>
static void launch_masked(int mt, F&& launch) {
    if (mt == RBQ_MASK_NONE) launch(attn_prefill_kernel<RBQ_MASK_NONE, D, VB, DT, GSH>);
    else if (mt == RBQ_MASK_BOOL) launch(attn_prefill_kernel<RBQ_MASK_BOOL, D, VB, DT, GSH>);
    else if (mt == RBQ_MASK_ADD_F32) launch(attn_prefill_kernel<RBQ_MASK_ADD_F32, D, VB, DT, GSH>);
    else launch(attn_prefill_kernel<RBQ_MASK_ADD_DTYPE, D, VB, DT, GSH>);
}

// The kernel of V width VB and group shift GSH (groups of 64 << GSH dims).
template <int D, int DT, int GSH, typename F>
static void launch_width(const rbq_kv_cache* c, int mt, F&& launch) {
    if (c->v_bits == 3) launch_masked<D, 3, DT, GSH>(mt, launch);
    else if (c->v_bits == 4) launch_masked<D, 4, DT, GSH>(mt, launch);
    else launch_masked<D, 2, DT, GSH>(mt, launch);
}

// The kernel of the cache's head_dim, group size and V width, for cache dtype DT.
template <int DT, typename F>
static void launch_layout(const rbq_kv_cache* c, int mt, F&& launch) {
    const bool g128 = c->group_size == 128;
    if (c->head_dim == 256) {
        if (g128) launch_width<256, DT, 1>(c, mt, launch);
        else launch_width<256, DT, 0>(c, mt, launch);
    } else if (c->head_dim == 128) {
        if (g128) launch_width<128, DT, 1>(c, mt, launch);
        else launch_width<128, DT, 0>(c, mt, launch);
    } else {  // groups of 128 dims exceed a head of 64: not taken
        launch_width<64, DT, 0>(c, mt, launch);
    }
}

bool prefill_takes(const rbq_kv_cache* c, int32_t H_q, int32_t L) {
    const int64_t G = (int64_t)(H_q / c->H_kv) * L;
    if (G < kPrefillMinRows || (c->dtype != RBQ_BF16 && c->dtype != RBQ_F16) || c->k_bits != 4 ||
        (c->group_size != 64 && c->group_size != 128) || c->group_size > c->head_dim ||
        (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256) || c->v_bits < 2 ||
        c->v_bits > 4)
        return false;
    return true;
}

int prefill_plan(const rbq_kv_cache* c, int32_t H_q, int32_t L, int32_t splits, MfmaPlan* p) {
    const int64_t G = (int64_t)(H_q / c->H_kv) * L;
    const int64_t RB = (G + 7) / 8;                 // blocks of 8 rows (the records)
    const int64_t RW = (G + kPRows - 1) / kPRows;   // blocks of 128 rows (the workgroups)
    const int64_t T = c->offset;
    const int64_t units = (int64_t)c->B * c->H_kv * RW;
    int64_t S = splits;
    if (S == 0) {
        S = (256 + units - 1) / units;  // about one workgroup per compute unit
        const int64_t max_s = (T + 8 * kPTile - 1) / (8 * kPTile);
        if (S > max_s) S = max_s;
    }
    if (S < 1) S = 1;
    int64_t chunk = (T + S - 1) / S;
    chunk = (chunk + kPTile - 1) / kPTile * kPTile;
    S = (T + chunk - 1) / chunk;
    const int64_t rec_units = (int64_t)c->B * c->H_kv * RB;
    if (units * S > 0x7FFFFFFF || rec_units * S > 0x7FFFFFFF) return RBQ_EUNSUPPORTED;
    // the merge kernel's one launch: at most 2^32 - 1 work-items along x
    if (S > 1 && rec_units * 8 * 512 > 0xFFFFFFFFll) return RBQ_EUNSUPPORTED;
    // 32-bit buffer offsets, up to one tile past T
    const int64_t row_bytes = (int64_t)c->head_dim * (c->k_bits > c->v_bits ? c->k_bits : c->v_bits) / 8;
    if ((T + kPTile) * row_bytes > 0x7FFFFFFF) return RBQ_EUNSUPPORTED;
    p->S = (int)S;
    p->RB = (int)RB;
    p->chunk = chunk;
    p->ws_bytes = (S == 1) ? 0 : (size_t)rec_units * S * record_floats(c->head_dim) * sizeof(float);
    return RBQ_OK;
}

int prefill_launch(const rbq_kv_cache* c, const void* q, int32_t H_q, int32_t L, float scale,
                   int32_t causal, const AttnMask& mk, const float* rot_blocks, float* out,
                   const MfmaPlan& p, void* ws, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    PArgs a;
    a.q = (const uint16_t*)q;
    a.kw = c->k_words;
    a.ks = (const uint16_t*)c->k_scales;
    a.kb = (const uint16_t*)c->k_biases;
    a.vw = c->v_words;
    a.vs = (const uint16_t*)c->v_scales;
    a.vb = (const uint16_t*)c->v_biases;
    a.rot = rot_blocks;
    a.out = out;
    a.rec = (float*)ws;
    a.mask = mk.ptr;
    a.msb = mk.sb;
    a.msh = mk.sh;
    a.msl = mk.sl;
    a.mask_bytes = mk.bytes;
    a.capacity = c->capacity;
    a.T = (int)c->offset;
    a.chunk = (int)p.chunk;
    a.S = p.S;
    a.Hkv = c->H_kv;
    a.n_rep = H_q / c->H_kv;
    a.L = L;
    a.G = a.n_rep * L;
    a.RB = p.RB;
    a.RW = (a.G + kPRows - 1) / kPRows;
    a.causal = causal ? 1 : 0;
    a.round_rot = (c->flags & RBQ_FLAG_ROUND_ROTATED) ? 1 : 0;
    a.qscale = scale * kPLog2e;
    const int64_t BH = (int64_t)c->B * c->H_kv;
    const int mt = mk.ptr == nullptr ? RBQ_MASK_NONE : mk.type;
    auto launch = [&](auto kernel) {
        for (int64_t bh0 = 0; bh0 < BH; bh0 += kPGridYZ)
            for (int64_t rw0 = 0; rw0 < a.RW; rw0 += kPGridYZ) {
                a.bh0 = (int)bh0;
                a.rw0 = (int)rw0;
                const dim3 grid((unsigned)p.S, (unsigned)std::min<int64_t>(kPGridYZ, a.RW - rw0),
                                (unsigned)std::min<int64_t>(kPGridYZ, BH - bh0));
                hipLaunchKernelGGL(kernel, grid, dim3(kPT), 0, s, a);
            }
    };
    if (c->dtype == RBQ_BF16) launch_layout<RBQ_BF16>(c, mt, launch);
    else launch_layout<RBQ_F16>(c, mt, launch);
    if (p.S > 1) merge_launch(c, a.rec, rot_blocks, out, p.S, p.RB, a.n_rep, L, a.causal, mt, stream);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_hip_error((int)e);
        return RBQ_EHIP;
    }
    return RBQ_OK;
}

}  // namespace rbq
