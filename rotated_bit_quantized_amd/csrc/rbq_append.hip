// Append path of the quantized cache (update_and_fetch on the quant_kv.py
// page): rotate each new K/V row by the SO(4) blocks, quantize it in groups
// (per-group scale and bias in the input dtype), bit-pack it as a
// little-endian bit stream and write it at row `offset`.  Also the growth
// copy of the cache buffers and the prefix copy behind cache snapshots.
//
// Mapping: one wave64 per (b, kv head, token) row; lane l owns elements
// [4l, 4l+4) = rotation block l, so a group of 64 is 16 lanes and the group
// min/max is a 16-lane butterfly.  K and V of the same row are done by the
// same wave.  The default configuration (head_dim 256, group 64, K 4-bit,
// V 3-bit: a row reads 2 x 512 B and writes 256 B, HBM-bound) has a kernel
// with those sizes compiled in; the others (head_dim 64 / 128 / 256, group
// 32 / 64 / 128, widths 2-8) share one kernel that takes them as arguments,
// lanes past head_dim / 4 idle.
#include <hip/hip_runtime.h>

#include "rbq_common.h"
#include "rbq_quantize.h"

namespace rbq {
namespace {

constexpr int kRowsPerBlock = 4;  // waves per workgroup

// Same definition with the sizes as arguments: head_dim D <= 256 (lanes
// l >= D / 4 hold zeros and write nothing), GS / 4 lanes per group, and
// 4 codes of `bits` bits per lane (a chunk of 4 * bits <= 32 bits).
template <int DT>
__device__ __forceinline__ void quantize_pack_row_any(const float y[4], int lane, int D, int GS,
                                                      int bits, uint32_t* __restrict__ words,
                                                      uint16_t* __restrict__ scales,
                                                      uint16_t* __restrict__ biases) {
    const float levels = (float)((1 << bits) - 1);
    float mn = fminf(fminf(y[0], y[1]), fminf(y[2], y[3]));
    float mx = fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3]));
    const int gl = GS / 4;  // lanes per group; groups are aligned lane ranges
    for (int m = 1; m < gl; m <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, m));
        mx = fmaxf(mx, __shfl_xor(mx, m));
    }
    const float s32 = __fdiv_rn(mx - mn, levels);
    const uint32_t s_bits = f32_to_elem_bits<DT>(s32);
    const uint32_t b_bits = f32_to_elem_bits<DT>(mn);
    const float s = elem_to_f32<DT>(s_bits);
    const float beta = elem_to_f32<DT>(b_bits);
    const float sdiv = (s == 0.0f) ? 1.0f : s;

    const float rinv = __builtin_amdgcn_rcpf(sdiv);
    uint32_t chunk = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float c = quant_code(y[i] - beta, sdiv, rinv);
        c = fminf(fmaxf(c, 0.0f), levels);
        chunk |= (uint32_t)c << (bits * i);
    }
    // word w gathers the chunks overlapping stream bits [32w, 32w + 32): at
    // most 5 (chunks of 8 bits); every such chunk belongs to a lane < D / 4
    const int C = 4 * bits;
    const int nwords = D * bits / 32;
    const int w = lane < nwords ? lane : 0;
    const int j0 = (32 * w) / C;
    const int j1 = (32 * w + 31) / C;
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < 5; ++k) {
        const int j = j0 + k;
        const uint32_t val = __shfl(chunk, j < 64 ? j : 63);
        if (j <= j1) {
            const int sh = C * j - 32 * w;
            word |= sh >= 0 ? (val << sh) : (val >> (-sh));
        }
    }
    if (lane < nwords) words[lane] = word;

    const int ngroups = D / GS;
    const uint32_t sg = __shfl(s_bits, (lane < ngroups ? lane : 0) * gl);
    const uint32_t bg = __shfl(b_bits, (lane < ngroups ? lane : 0) * gl);
    if (lane < ngroups) {
        scales[lane] = (uint16_t)sg;
        biases[lane] = (uint16_t)bg;
    }
}

template <int DT>
__global__ __launch_bounds__(64 * kRowsPerBlock) void quant_append_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int64_t n,
    const float* __restrict__ rot, uint32_t* __restrict__ kw, uint16_t* __restrict__ ks,
    uint16_t* __restrict__ kb, uint32_t* __restrict__ vw, uint16_t* __restrict__ vs,
    uint16_t* __restrict__ vb, int64_t capacity, int64_t offset, int64_t rows_total,
    int round_rot) {
    const int lane = threadIdx.x & 63;
    // the wave's row, wave-uniform (readfirstlane): its index arithmetic,
    // a 64-bit division included, runs on the scalar unit
    const int64_t row =
        (int64_t)blockIdx.x * kRowsPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= rows_total) return;  // uniform per wave
    const int64_t bh = row / n;
    const int64_t t = row - bh * n;
    const int64_t src = row * kHeadDim + lane * 4;
    const int64_t dst = bh * capacity + offset + t;

    // both rows' loads first: K and V are independent chains the wave interleaves
    float xk[4], xv[4];
    load4<DT>(k + src, xk);
    load4<DT>(v + src, xv);
    float Bm[16];
    load_block(rot, lane, Bm);

    float yk[4], yv[4];
    rotate4(xk, Bm, yk);
    rotate4(xv, Bm, yv);
    if (round_rot) {
        round_row<DT>(yk);
        round_row<DT>(yv);
    }
    quantize_pack_row<DT, kKBits>(yk, lane, kw + dst * kKWords, ks + dst * kGroups,
                                  kb + dst * kGroups);
    quantize_pack_row<DT, kVBits>(yv, lane, vw + dst * kVWords, vs + dst * kGroups,
                                  vb + dst * kGroups);
}

struct AnyCfg {
    int D, GS, kbits, vbits, round_rot;
};

template <int DT>
__global__ __launch_bounds__(64 * kRowsPerBlock) void quant_append_any_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int64_t n,
    const float* __restrict__ rot, uint32_t* __restrict__ kw, uint16_t* __restrict__ ks,
    uint16_t* __restrict__ kb, uint32_t* __restrict__ vw, uint16_t* __restrict__ vs,
    uint16_t* __restrict__ vb, int64_t capacity, int64_t offset, int64_t rows_total, AnyCfg g) {
    const int lane = threadIdx.x & 63;
    // the wave's row, wave-uniform (readfirstlane): its index arithmetic,
    // a 64-bit division included, runs on the scalar unit
    const int64_t row =
        (int64_t)blockIdx.x * kRowsPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= rows_total) return;  // uniform per wave
    const int64_t bh = row / n;
    const int64_t t = row - bh * n;
    const bool active = lane < g.D / 4;
    const int64_t src = row * g.D + lane * 4;
    const int64_t dst = bh * capacity + offset + t;
    const int kwords = g.D * g.kbits / 32, vwords = g.D * g.vbits / 32, ngroups = g.D / g.GS;

    float Bm[16];
    load_block(rot, active ? lane : 0, Bm);

    float x[4] = {0.f, 0.f, 0.f, 0.f}, y[4];
    if (active) load4<DT>(k + src, x);
    rotate4(x, Bm, y);
    if (g.round_rot) round_row<DT>(y);
    quantize_pack_row_any<DT>(y, lane, g.D, g.GS, g.kbits, kw + dst * kwords,
                              ks + dst * ngroups, kb + dst * ngroups);
    if (active) load4<DT>(v + src, x);
    rotate4(x, Bm, y);
    if (g.round_rot) round_row<DT>(y);
    quantize_pack_row_any<DT>(y, lane, g.D, g.GS, g.vbits, vw + dst * vwords,
                              vs + dst * ngroups, vb + dst * ngroups);
}

// dst rows [0, keep) <- src rows, dst rows [keep, dst_cap) <- 0, for an array
// of `wpr` 16-bit units per row and `bh` (b, kv head) slabs.
__global__ __launch_bounds__(256) void grow_copy_kernel(const uint16_t* __restrict__ src,
                                                        uint16_t* __restrict__ dst, int wpr,
                                                        int64_t bh, int64_t src_cap,
                                                        int64_t dst_cap, int64_t keep) {
    const int64_t total = bh * dst_cap * wpr;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t slab = i / (dst_cap * wpr);
        const int64_t rem = i - slab * dst_cap * wpr;
        const int64_t r = rem / wpr;
        const int64_t e = rem - r * wpr;
        dst[i] = (r < keep) ? src[(slab * src_cap + r) * wpr + e] : (uint16_t)0;
    }
}

// Prefix copy of the six arrays (snapshots, restore, batch tiling and row
// selection): for array a and destination slab (b, kv head), dst rows [0, n)
// <- rows [0, n) of source slab (b0 + b * bstep, kv head); rows at or past n
// of dst are not touched.  One launch for all six arrays: the grid is the
// concatenation, array by array, of slab-major runs of 8 KiB chunks of each
// slab's prefix (n rows x upr 16-bit units, contiguous in both caches).  A
// chunk is 4096 units (8 KiB), 16 per thread: two 16-byte non-temporal loads
// in flight per thread and non-temporal stores (the copy streams through the
// caches) when both slab bases are 16-byte aligned, 2-byte units otherwise.
constexpr int kCopyChunkUnits = 4096;
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

struct CopyArr {
    const uint16_t* src;
    uint16_t* dst;
    int64_t src_stride, dst_stride;  // units between consecutive slabs
    uint32_t chunks;                 // chunks per slab
    uint32_t first_block;            // first workgroup of this array
    int upr;                         // units per row
};
struct CopyArgs {
    CopyArr arr[6];  // K words, K scales, K biases, V words, V scales, V biases
    int64_t n;       // rows to copy
    int H, b0, bstep;  // kv heads; source batch entry of destination entry b: b0 + b * bstep
};

__global__ __launch_bounds__(256) void copy_prefix_kernel(CopyArgs a) {
    int ai = 0;
#pragma unroll
    for (int k = 1; k < 6; ++k)
        if (blockIdx.x >= a.arr[k].first_block) ai = k;
    const CopyArr& r = a.arr[ai];
    const uint32_t local = blockIdx.x - r.first_block;
    const uint32_t slab = local / r.chunks;
    const uint32_t chunk = local - slab * r.chunks;
    const int64_t units = a.n * r.upr;
    const uint32_t bd = slab / (uint32_t)a.H;
    const int64_t sslab = (int64_t)(a.b0 + (int)bd * a.bstep) * a.H + (slab - bd * (uint32_t)a.H);
    const uint16_t* src = r.src + sslab * r.src_stride;
    uint16_t* dst = r.dst + slab * r.dst_stride;
    const int64_t w0 = (int64_t)chunk * kCopyChunkUnits;
    const int tid = threadIdx.x;
    const bool vec = ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0;
    if (vec && w0 + kCopyChunkUnits <= units) {
        const u32x4v* s4 = reinterpret_cast<const u32x4v*>(src + w0);
        u32x4v* d4 = reinterpret_cast<u32x4v*>(dst + w0);
        const u32x4v v0 = __builtin_nontemporal_load(s4 + tid);
        const u32x4v v1 = __builtin_nontemporal_load(s4 + 256 + tid);
        __builtin_nontemporal_store(v0, d4 + tid);
        __builtin_nontemporal_store(v1, d4 + 256 + tid);
    } else {
        for (int i = 0; i < kCopyChunkUnits / 256; ++i) {
            const int64_t w = w0 + i * 256 + tid;
            if (w < units) dst[w] = src[w];
        }
    }
}

int launch_status(hipError_t e) {
    if (e != hipSuccess) {
        set_hip_error((int)e);
        return RBQ_EHIP;
    }
    return RBQ_OK;
}

}  // namespace
}  // namespace rbq

using namespace rbq;

extern "C" int rbq_kv_quant_append(rbq_kv_cache* c, const void* k, const void* v, int64_t n,
                                   const float* rot_blocks, void* stream) {
    int st = check_cache(c);
    if (st != RBQ_OK) return st;
    if (n < 0) return RBQ_EINVAL;
    if (n == 0) return RBQ_OK;
    if (k == nullptr || v == nullptr) return RBQ_EINVAL;
    if (n > c->capacity - c->offset) return RBQ_ECAPACITY;
    const int64_t rows = (int64_t)c->B * c->H_kv * n;  // <= kMaxTotalRows (check_cache)
    const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
    if (blocks > 0x7FFFFFFF) return RBQ_EUNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    const dim3 grid((unsigned)blocks), block(64 * kRowsPerBlock);
    auto* kw = c->k_words;
    auto* ks = (uint16_t*)c->k_scales;
    auto* kb = (uint16_t*)c->k_biases;
    auto* vw = c->v_words;
    auto* vs = (uint16_t*)c->v_scales;
    auto* vb = (uint16_t*)c->v_biases;
    const int round_rot = (c->flags & RBQ_FLAG_ROUND_ROTATED) ? 1 : 0;
    if (is_default_config(c)) {
        if (c->dtype == RBQ_BF16)
            hipLaunchKernelGGL(quant_append_kernel<RBQ_BF16>, grid, block, 0, s,
                               (const uint16_t*)k, (const uint16_t*)v, n, rot_blocks, kw, ks, kb,
                               vw, vs, vb, c->capacity, c->offset, rows, round_rot);
        else
            hipLaunchKernelGGL(quant_append_kernel<RBQ_F16>, grid, block, 0, s,
                               (const uint16_t*)k, (const uint16_t*)v, n, rot_blocks, kw, ks, kb,
                               vw, vs, vb, c->capacity, c->offset, rows, round_rot);
    } else {
        const AnyCfg g = {c->head_dim, c->group_size, c->k_bits, c->v_bits, round_rot};
        if (c->dtype == RBQ_BF16)
            hipLaunchKernelGGL(quant_append_any_kernel<RBQ_BF16>, grid, block, 0, s,
                               (const uint16_t*)k, (const uint16_t*)v, n, rot_blocks, kw, ks, kb,
                               vw, vs, vb, c->capacity, c->offset, rows, g);
        else
            hipLaunchKernelGGL(quant_append_any_kernel<RBQ_F16>, grid, block, 0, s,
                               (const uint16_t*)k, (const uint16_t*)v, n, rot_blocks, kw, ks, kb,
                               vw, vs, vb, c->capacity, c->offset, rows, g);
    }
    st = launch_status(hipGetLastError());
    if (st != RBQ_OK) return st;
    c->offset += n;
    return RBQ_OK;
}

extern "C" int rbq_kv_grow(const rbq_kv_cache* src, rbq_kv_cache* dst, void* stream) {
    int st = check_cache(src);
    if (st != RBQ_OK) return st;
    st = check_cache(dst);
    if (st != RBQ_OK) return st;
    if (src->B != dst->B || src->H_kv != dst->H_kv || src->dtype != dst->dtype ||
        src->head_dim != dst->head_dim || src->group_size != dst->group_size ||
        src->k_bits != dst->k_bits || src->v_bits != dst->v_bits || dst->capacity <= 0)
        return RBQ_EINVAL;
    const int64_t keep = (src->capacity == 0) ? 0
                         : (src->offset % kStep != 0) ? src->offset
                                                      : src->capacity;
    if (keep > dst->capacity) return RBQ_EINVAL;
    if (src->capacity > 0 && (src->k_words == dst->k_words || src->v_words == dst->v_words))
        return RBQ_EINVAL;
    const int64_t bh = (int64_t)src->B * src->H_kv;
    hipStream_t s = (hipStream_t)stream;
    const RowUnits u = row_units(src);
    struct Arr {
        const void* from;
        void* to;
        int wpr;
    } arrs[6] = {
        {src->k_words, dst->k_words, u.kw},     {src->k_scales, dst->k_scales, u.meta},
        {src->k_biases, dst->k_biases, u.meta}, {src->v_words, dst->v_words, u.vw},
        {src->v_scales, dst->v_scales, u.meta}, {src->v_biases, dst->v_biases, u.meta},
    };
    for (const Arr& a : arrs) {
        const int64_t total = bh * dst->capacity * a.wpr;
        int64_t nb = (total + 255) / 256;
        if (nb > 65536) nb = 65536;
        hipLaunchKernelGGL(grow_copy_kernel, dim3((unsigned)nb), dim3(256), 0, s,
                           (const uint16_t*)a.from, (uint16_t*)a.to, a.wpr, bh, src->capacity,
                           dst->capacity, keep);
        st = launch_status(hipGetLastError());
        if (st != RBQ_OK) return st;
    }
    dst->offset = src->offset;
    return RBQ_OK;
}

namespace rbq {
namespace {

// Shared body of the prefix copies: destination batch entry b receives
// source entry b0 + b * bstep.
int copy_batch(const rbq_kv_cache* src, int32_t b0, int32_t bstep, rbq_kv_cache* dst,
               void* stream) {
    int st = check_cache(src);
    if (st != RBQ_OK) return st;
    st = check_cache(dst);
    if (st != RBQ_OK) return st;
    if (src->H_kv != dst->H_kv || src->dtype != dst->dtype || src->head_dim != dst->head_dim ||
        src->group_size != dst->group_size || src->k_bits != dst->k_bits ||
        src->v_bits != dst->v_bits)
        return RBQ_EINVAL;
    const int64_t last = (int64_t)b0 + (int64_t)(dst->B - 1) * bstep;
    if (b0 < 0 || b0 >= src->B || last < 0 || last >= src->B) return RBQ_EINVAL;
    const int64_t n = src->offset;
    if (n > dst->capacity) return RBQ_ECAPACITY;
    if (n == 0) {
        dst->offset = 0;
        return RBQ_OK;
    }
    const int64_t bh = (int64_t)dst->B * dst->H_kv;
    const void* from[6] = {src->k_words, src->k_scales, src->k_biases,
                           src->v_words, src->v_scales, src->v_biases};
    void* to[6] = {dst->k_words, dst->k_scales, dst->k_biases,
                   dst->v_words, dst->v_scales, dst->v_biases};
    const RowUnits u = row_units(src);
    const int wpr[6] = {u.kw, u.meta, u.meta, u.vw, u.meta, u.meta};
    CopyArgs a;
    a.n = n;
    a.H = dst->H_kv;
    a.b0 = b0;
    a.bstep = bstep;
    int64_t blocks = 0;
    for (int i = 0; i < 6; ++i) {
        // the two caches' arrays must not overlap
        const char* s0 = (const char*)from[i];
        const char* s1 = s0 + (size_t)src->B * src->H_kv * src->capacity * wpr[i] * 2;
        const char* d0 = (const char*)to[i];
        const char* d1 = d0 + (size_t)bh * dst->capacity * wpr[i] * 2;
        if (s0 < d1 && d0 < s1) return RBQ_EINVAL;
        a.arr[i].src = (const uint16_t*)from[i];
        a.arr[i].dst = (uint16_t*)to[i];
        a.arr[i].src_stride = src->capacity * wpr[i];
        a.arr[i].dst_stride = dst->capacity * wpr[i];
        a.arr[i].upr = wpr[i];
        const int64_t chunks = (n * wpr[i] + kCopyChunkUnits - 1) / kCopyChunkUnits;
        if (blocks + chunks * bh > 0x7FFFFFFF) return RBQ_EUNSUPPORTED;
        a.arr[i].chunks = (uint32_t)chunks;
        a.arr[i].first_block = (uint32_t)blocks;
        blocks += chunks * bh;
    }
    hipLaunchKernelGGL(copy_prefix_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, a);
    st = launch_status(hipGetLastError());
    if (st != RBQ_OK) return st;
    dst->offset = n;
    return RBQ_OK;
}

}  // namespace
}  // namespace rbq

extern "C" int rbq_kv_copy_prefix(const rbq_kv_cache* src, rbq_kv_cache* dst, void* stream) {
    if (src == nullptr || dst == nullptr) return RBQ_EINVAL;
    if (src->B != dst->B) return RBQ_EINVAL;
    return copy_batch(src, 0, 1, dst, stream);
}

extern "C" int rbq_kv_copy_batch(const rbq_kv_cache* src, int32_t src_b0, int32_t src_b_step,
                                 rbq_kv_cache* dst, void* stream) {
    if (src == nullptr || dst == nullptr) return RBQ_EINVAL;
    return copy_batch(src, src_b0, src_b_step, dst, stream);
}
