// Fused decode attention over the packed K4/V3 cache on the gfx950 matrix
// cores (asym_quantized_sdpa on the quant_kv.py page, with the SO(4)
// rotation of q on entry and the inverse rotation of the output).  The G =
// (H_q / H_kv) x L query rows of a kv head (GQA group x verify block) are
// taken 8 at a time: one workgroup per block of 8 rows; blocks of the same
// keys run side by side, so their repeated reads are mostly served by the
// caches.
//
// Decomposition: one workgroup of 8 wave64s (about one per compute unit) per
// (b, kv head, key split).  Set-up is shared: wave w rotates query row w and
// builds one of the 8 score operand sets; all build the V decode table.  Each
// wave walks 32-key tiles of the split (its first tile's loads are issued
// before the set-up, the next tile's are in flight while one is computed)
// with an online softmax (base 2, rescaled only when the running maximum
// grows by more than 2^8); the 8 wave partials are merged in LDS.  With one
// split the workgroup normalises the rows, rotates them back and stores the
// output; with several it stores its record (m, l, unnormalised o), and a
// second small kernel merges the records of each (b, kv head), normalises and
// rotates back.
//
// All products run as 16x16x32 MFMAs.  Lane l = 16 j + n: j selects a k-slot
// group of the operands and a quarter of the accumulator rows, n a column.
// Scores: A = query (rows 0-7: fp16 hi part of the 8 query rows, rows 8-15:
//   lo part; each row scaled by a power of two so that hi spans [2^14, 2^15)),
//   B = K codes of 16 keys (column = key).  The codes enter as fp16
//   subnormals: masking nibble pairs of a packed word in place gives
//   c * 2^-24 (nibbles 0 and 2 of a byte pair) or 16 c * 2^-24 (nibbles 1 and
//   3), with the matching 1 or 1/16 folded into the query operand.  One
//   accumulator per 64-value group g; score = s_g acc_g (fp32, per key) plus
//   sum_g b_g sum_{d in g} q_d, the latter an MFMA of the raw bias words
//   against the query's group sums (split into exact limbs).
// Values: B = V codes of 8 keys per lane group x 16 columns.  The LDS
//   transposing read (ds_read_b64_tr_b16) returns, to lane i of a 16-lane
//   group, element i & 3 of the 8 bytes addressed by lanes 4e + (i >> 2),
//   e = 0..3.  Lane 4e + q addresses the entry of a 4096-entry decode table
//   (12 packed stream bits -> 4 fp16 codes) for chunk t of group q of key e,
//   so one read both decodes and transposes: lane i receives the codes of
//   4 keys in column 64 (i >> 2) + 4 t + (i & 3).  The same read on small
//   per-wave tables moves the per-(key, group) scales and biases, and P
//   (split hi + lo over the 16 rows), into the matching layouts.  Codes are
//   scaled in fp16 (exact for bf16 scales: 3 + 8 significant bits; fp16
//   scales are split into an exact 8-bit head and 3-bit tail); the group bias
//   enters as sum_t p_t b_{t,g} through one more MFMA.
// Range of the fp16 value path: the V scales and biases enter the fp16
// operands times 2^-F, with F a per-wave power of two that stays 0 while
// every |scale| and |bias| seen is below 2^13 and otherwise grows so that
// they stay below 2^13 * 2^F (codes times scales then stay below 65504); the
// accumulators are rescaled when F grows and the wave's record is taken
// back to unit scale.  So any finite bf16 values are taken, as long as the
// fp32 accumulators (the probability-weighted sums of values) stay finite.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "rbq_common.h"
#include "rbq_quantize.h"

namespace rbq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int kWaves = 8;                                  // one workgroup per compute unit
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;                                  // keys per wave iteration
constexpr int kRows = 8;                                   // query rows per kv head
// split record in the workspace: (m, l) per row, then o column-major
// [256 columns][8 rows]
constexpr int kRecFloats = kRecordFloats;
static_assert(kRecFloats == 2 * kRows + kRows * kHeadDim, "split record layout");
constexpr int kMergeNarrowUnits = 64;  // below this many units the merge takes 32-column blocks
constexpr int64_t kGridYZ = 65535;      // workgroups per grid dimension y or z of one launch
// wave record in LDS, in its own region so that a wave stores it as soon as
// its tiles are done: o column-major [256 columns][2 row quads][4 rows], the
// row quad of column c stored at slot quad ^ ((c >> 3) & 1) (conflict-free
// 16-byte reads of 64 consecutive columns), ob [4 groups][8 rows], m[8], l[8];
// then per wave the merge weights [8 waves][8 rows], M[8], L[8]
constexpr int kWaveRecFloats = kHeadDim * kRows + kGroups * kRows + 2 * kRows;
constexpr int kWeightFloats = kWaves * kRows + 2 * kRows;
constexpr int kLutBytes = 4096 * 8;
constexpr int kQaBytes = 8 * 64 * 16;                      // score query operands, per lane
// per wave: scale / scale-tail / bias tables [2 blocks][64 lanes] x 8 B and
// P hi/lo [2 blocks][16 keys][2 parts][2 row quads] x 8 B
constexpr int kStageBytes = 2 * 64 * 8;
constexpr int kP16Bytes = 2 * 16 * 2 * 2 * 8;
constexpr int kWaveBytes = 3 * kStageBytes + kP16Bytes;
constexpr int kStageOff = kLutBytes + kQaBytes;
constexpr int kSmemBytes = kStageOff + kWaves * kWaveBytes;
// Second LDS array (a separate object, so that the compiler can tell the
// direct-to-LDS tile transfers from every other LDS access): per wave a tile
// buffer during the tile loop, then the wave's record; then the merge weights.
// A tile buffer holds one 32-key tile as the memory holds it: K words, V
// words, K scales, K biases, V scales, V biases.
constexpr int kWaveAreaBytes = kWaveRecFloats * 4;
constexpr int kBufK = 0, kBufV = 4096, kBufKs = 7168, kBufKb = 7424, kBufVs = 7680, kBufVb = 7936;
constexpr int kTileBufBytes = 8192;
constexpr int kWeightOff = kWaves * kWaveAreaBytes;
constexpr int kTbufBytes = kWeightOff + kWaves * kWeightFloats * 4;
static_assert(kSmemBytes + kTbufBytes <= 160 * 1024, "LDS of one compute unit");
static_assert(kTileBufBytes <= kWaveAreaBytes && kWaveAreaBytes % 16 == 0,
              "a tile buffer fits a wave's record area");
constexpr float kLog2e = 1.44269504088896340736f;
static_assert(kWaves == kRows && kThreads == kRows * kHeadDim / 4, "one query block per thread");
static_assert(kWaves == 8, "one score operand set (group, half) per wave");
static_assert((kRows * kHeadDim + kRows * 8 + kHeadDim * 4) * 4 <= kWaves * kWaveBytes,
              "query rows, their statistics and the rotation blocks fit the staging area");
static_assert(kThreads * 2 == kHeadDim * 4, "8 bytes of the rotation blocks per thread");
static_assert(kThreads == 2 * kHeadDim && kRows == 8, "merge: one column and 4 rows per thread");

struct MArgs {
    // the fields the prologue needs come first, so that they arrive in one
    // batch of scalar loads
    const uint16_t* q;
    const uint32_t* kw;
    const uint16_t* ks;
    const uint16_t* kb;
    const uint32_t* vw;
    const uint16_t* vs;
    const uint16_t* vb;
    const float* rot;
    // fused append (no mask): rows [T - n_new, T) of the cache are quantized
    // from kn / vn ([B][H_kv][n_new][256], unrotated) and written by this
    // launch
    const uint16_t* kn;
    const uint16_t* vn;
    int64_t capacity;
    int T, chunk;
    int Hkv, n_rep, L, G, S, causal;
    int RB;        // blocks of 8 query rows per kv head
    int rb0, bh0;  // first row block and (b, kv head) of this launch (grid y and z)
    int n_new;
    int round_rot; // RBQ_FLAG_ROUND_ROTATED: the rotated query rounded to the dtype
    float qscale;  // scale * log2(e)
    float* out;
    float* rec;
    // optional mask over (query row, key): element [b][q head][row i][key t]
    // at mask + b*msb + h*msh + i*msl + t (elements; the key stride is 1)
    const void* mask;
    int64_t msb, msh, msl;
    uint32_t mask_bytes;  // extent read through a range-checked buffer resource
};

// Mask element types (the template argument MK of the attention kernel).
constexpr int kMaskNone = 0;
constexpr int kMaskBool = 1;     // uint8: nonzero = the key is attended
constexpr int kMaskAddF32 = 2;   // fp32 added to the scaled scores
constexpr int kMaskAddElem = 3;  // the same in the cache dtype (fp16 / bf16)

__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16bf(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                     __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                             0x00020000);
}

// LDS transposing read of 8 bytes at byte offset `off` of the shared buffer:
// lane i of each 16-lane group gets element i & 3 of the 8 bytes addressed by
// lanes 4e + (i >> 2) of its group, as element e.
__device__ __forceinline__ u32x2 tr16(unsigned char* smem, uint32_t off) {
    lds_u8* base = (lds_u8*)smem;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(base + off));
    return __builtin_bit_cast(u32x2, v);
}

// 4-byte LDS store at byte offset `off` of the shared buffer, through an
// LDS-typed pointer: through a generic one the compiler cannot tell the store
// from the direct-to-LDS tile transfers in flight and waits for them first.
__device__ __forceinline__ void lds_st32(unsigned char* smem, uint32_t off, uint32_t v) {
    *(__attribute__((address_space(3))) uint32_t*)((lds_u8*)smem + off) = v;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// max / sum over the 16 lanes of a row
__device__ __forceinline__ float max16(float x) {
    x = fmaxf(x, dpp<0xB1>(x));
    x = fmaxf(x, dpp<0x4E>(x));
    x = fmaxf(x, dpp<0x141>(x));
    return fmaxf(x, dpp<0x140>(x));
}
__device__ __forceinline__ float sum16(float x) {
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    return x + dpp<0x140>(x);
}

// Row col & 3 of the rotation block of column `col` (zeros without rotation);
// loaded before the results it multiplies are ready.
__device__ __forceinline__ float4 rot_row(const float* rot, int col) {
    if (rot == nullptr) return make_float4(0.f, 0.f, 0.f, 0.f);
    return *reinterpret_cast<const float4*>(rot + 16 * (col >> 2) + 4 * (col & 3));
}

// Normalise row `row` of column `col` (acc / Ls), rotate back and store it if
// row < G.  The 4 columns of a rotation block lie in one lane quad (lane & 3
// = col & 3): z = sum_k y[block column k] * B[col & 3][k], in fp64, with
// v = B[col & 3] from rot_row.
template <int D = kHeadDim>
__device__ __forceinline__ void store_out(float* out, bool rotated, float4 v, int bh, int G,
                                          int col, int row, float acc, float Ls) {
    const float y = acc * (1.0f / Ls);
    float z = y;
    if (rotated) {
        const float y0 = dpp<0x00>(y), y1 = dpp<0x55>(y), y2 = dpp<0xAA>(y), y3 = dpp<0xFF>(y);
        double s2 = (double)y0 * (double)v.x;
        s2 = s2 + (double)y1 * (double)v.y;
        s2 = s2 + (double)y2 * (double)v.z;
        s2 = s2 + (double)y3 * (double)v.w;
        z = (float)s2;
    }
    // the G rows of kv head bh are its n_rep q heads' L rows in (head, row)
    // order, i.e. rows bh * G + row of [B][H_q][L][D]
    if (row < G) out[((int64_t)bh * G + row) * D + col] = z;
}

// Workgroup barrier that orders LDS accesses only: the waves exchange data
// through LDS alone, so outstanding global loads, tile transfers into LDS
// included, stay in flight across it.  (A workgroup-scope LDS fence would
// wait for those transfers too, since they count as LDS writes; __syncthreads
// would wait for every global load.)  lgkmcnt(0) completes this wave's own
// LDS accesses; the memory clobber keeps the compiler from moving memory
// accesses across the barrier.  Data that a wave reads after the barrier
// from another wave's direct-to-LDS transfer is not covered: the tile loop
// waits for its own transfers (vmcnt) before reading them.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// (fp16(p0 - h0), fp16(p1 - h1)) for hi2 = (h0, h1) the fp16 roundings of
// p0, p1: one mixed-precision FMA per half, fma(-h, 1, p) with h taken as
// fp16 and p as fp32, rounded once to fp16 (p - h is exact in fp32, so this
// equals rounding the fp32 difference).  `one` holds 1.0f.
__device__ __forceinline__ uint32_t f16_residuals(uint32_t hi2, float p0, float p1, float one) {
    uint32_t r;
    asm("v_fma_mixlo_f16 %0, -%1, %2, %3 op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixhi_f16 %0, -%1, %2, %4 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "=&v"(r)
        : "v"(hi2), "v"(one), "v"(p0), "v"(p1));
    return r;
}

__device__ __forceinline__ uint32_t mul2(uint32_t a, uint32_t s) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, a) * __builtin_bit_cast(f16x2, s));
}

template <int DT>
__device__ __forceinline__ float meta_f32(uint32_t word, int half) {
    return elem_to_f32<DT>(half ? word >> 16 : word);
}

// Byte offset (index * 8) in the decode table of 12-bit chunk c (codes
// 4c..4c+3) of a 64-code V group held in words w[0..5].
template <int C>
__device__ __forceinline__ uint32_t chunk_offset(const uint32_t w[6]) {
    constexpr int start = 12 * C - 3;
    if constexpr (C == 0) {
        return (w[0] << 3) & 0x7FF8u;
    } else {
        constexpr int wi = start >> 5, sh = start & 31;
        if constexpr (wi + 1 < 6) return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & 0x7FF8u;
        else return (w[wi] >> sh) & 0x7FF8u;
    }
}

// Registers of one 32-key tile for this lane.  K data: key n of each block;
// V data: group n & 3 of key 4j + (n >> 2) of each block.
struct TileLoads {
    u32x2 kwv[2][4];   // K words 8g + 2j, 8g + 2j + 1
    u32x2 ksw[2];      // K scales (4 x 16 bit)
    u32x2 kbw[2];      // K biases
    uint32_t wv[2][6]; // V words of the lane's (key, group)
    uint32_t vsb[2];   // V scale of the lane's (key, group)
    uint32_t vbb[2];   // V bias of the lane's (key, group)
};

// 16-byte slot of K word chunk c (words 4c .. 4c+3) of tile key k in the tile
// buffer: the chunks of a key are permuted by (k >> 1) & 7 so that the
// 8-byte reads of 32 lanes (16 keys x 2 halves of a chunk) hit 64 distinct
// banks.
__device__ __forceinline__ int k_slot(int k, int c) { return 8 * k + (c ^ ((k >> 1) & 7)); }

// Direct-to-LDS loads of part PART of the tile at key t0 into this wave's
// buffer (lane l of an instruction lands at buffer offset + 16 l, or 4 l),
// each instruction reading whole 128-byte lines; keys past the buffer ranges
// read as zero.  Part 0: K words (4 instructions), part 1: V words (3),
// part 2: the four scale / bias arrays (4).  The loop issues the parts at
// three points of an iteration rather than all at once: while the memory
// system is saturated an issuing wave stalls until its requests are taken,
// and spread out those stalls overlap more of the other waves' arithmetic.
// Cache policy of the tile transfers: non-temporal (each cache byte is read
// once per call; the hint keeps the stream from displacing other lines and
// raises the read rate of a plain scan on this GPU by about 7 %).
constexpr int kTileCPol = 2;

template <int PART>
__device__ __forceinline__ void dma_tile_part(lds_u8* buf, int t0, int lane, __amdgpu_buffer_rsrc_t kw_r,
                                              __amdgpu_buffer_rsrc_t ks_r, __amdgpu_buffer_rsrc_t kb_r,
                                              __amdgpu_buffer_rsrc_t vw_r, __amdgpu_buffer_rsrc_t vs_r,
                                              __amdgpu_buffer_rsrc_t vb_r) {
    if constexpr (PART == 0) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int p = 64 * m + lane;
            const int k = p >> 3;
            const int c = (p & 7) ^ ((k >> 1) & 7);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kw_r, buf + kBufK + 1024 * m, 16,
                                                      (t0 + k) * 128 + 16 * c, 0, 0, kTileCPol);
        }
    } else if constexpr (PART == 1) {
#pragma unroll
        for (int m = 0; m < 3; ++m)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vw_r, buf + kBufV + 1024 * m, 16,
                                                      t0 * 96 + 16 * (64 * m + lane), 0, 0, kTileCPol);
    } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ks_r, buf + kBufKs, 4, t0 * 8 + 4 * lane, 0, 0, kTileCPol);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kb_r, buf + kBufKb, 4, t0 * 8 + 4 * lane, 0, 0, kTileCPol);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vs_r, buf + kBufVs, 4, t0 * 8 + 4 * lane, 0, 0, kTileCPol);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vb_r, buf + kBufVb, 4, t0 * 8 + 4 * lane, 0, 0, kTileCPol);
    }
}

// The k-th tile (counted within the split) of a wave, or n_tiles when the
// wave has no k-th tile.  Round robin over the waves, except for the last
// full round together with the remainder (8 to 15 tiles) when there are
// earlier rounds: positions 0-7 go to waves 0-3, two each, 8-11 to waves 4-7
// and 12-15 to waves 0-3 again.  The older half of a workgroup issues first
// on each SIMD and gets through its tiles sooner; with the same number of
// tiles each, it idles at the end while the younger half finishes.  A split
// of a single round stays round robin: there every wave's first tile is in
// flight from the start, and two tiles in a row on half the waves would
// double the wait.  The order is fixed, so results do not depend on timing.
__device__ __forceinline__ int wave_tile(int k, int wave, int n_tiles) {
    const int rounds = n_tiles / kWaves;
    if (rounds <= 1) {
        const int t = wave + kWaves * k;
        return (t < n_tiles) ? t : n_tiles;
    }
    if (k < rounds - 1) return wave + kWaves * k;
    const int jt = k - (rounds - 1);  // index among the wave's last-round tiles
    int pos = 2 * kWaves;             // none
    if (wave < kWaves / 2) {
        if (jt < 2) pos = 2 * wave + jt;
        else if (jt == 2) pos = 12 + wave;
    } else if (jt == 0) {
        pos = wave + 4;
    }
    const int tail_n = kWaves + n_tiles % kWaves;
    return (pos < tail_n) ? (rounds - 1) * kWaves + pos : n_tiles;
}

// The whole tile (the first one of each wave, before the set-up).
__device__ __forceinline__ void dma_tile(lds_u8* buf, int t0, int lane, __amdgpu_buffer_rsrc_t kw_r,
                                         __amdgpu_buffer_rsrc_t ks_r, __amdgpu_buffer_rsrc_t kb_r,
                                         __amdgpu_buffer_rsrc_t vw_r, __amdgpu_buffer_rsrc_t vs_r,
                                         __amdgpu_buffer_rsrc_t vb_r) {
    dma_tile_part<0>(buf, t0, lane, kw_r, ks_r, kb_r, vw_r, vs_r, vb_r);
    dma_tile_part<1>(buf, t0, lane, kw_r, ks_r, kb_r, vw_r, vs_r, vb_r);
    dma_tile_part<2>(buf, t0, lane, kw_r, ks_r, kb_r, vw_r, vs_r, vb_r);
}

// The lane's operands of the buffered tile.
__device__ __forceinline__ void read_tile(TileLoads& L, const unsigned char* buf, int n, int j) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const int k = 16 * blk + n;
#pragma unroll
        for (int g = 0; g < 4; ++g)
            L.kwv[blk][g] = *reinterpret_cast<const u32x2*>(
                buf + kBufK + 16 * k_slot(k, 2 * g + (j >> 1)) + 8 * (j & 1));
        L.ksw[blk] = *reinterpret_cast<const u32x2*>(buf + kBufKs + 8 * k);
        L.kbw[blk] = *reinterpret_cast<const u32x2*>(buf + kBufKb + 8 * k);
        const int vk = 16 * blk + 4 * j + (n >> 2);
        const int vg = n & 3;
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            const u32x2 z = *reinterpret_cast<const u32x2*>(buf + kBufV + 96 * vk + 24 * vg + 8 * m);
            L.wv[blk][2 * m] = z[0];
            L.wv[blk][2 * m + 1] = z[1];
        }
        L.vsb[blk] = *reinterpret_cast<const uint16_t*>(buf + kBufVs + 8 * vk + 2 * vg);
        L.vbb[blk] = *reinterpret_cast<const uint16_t*>(buf + kBufVb + 8 * vk + 2 * vg);
    }
}

// P.V for output tile t (columns 64 q + 4 t + (0..3), q = 0..3): decode and
// transpose the codes of both 16-key blocks in one read each, scale, MFMA.
template <int DT, int TT>
__device__ __forceinline__ void pv_tile(unsigned char* smem, const uint32_t wv0[6],
                                        const uint32_t wv1[6], const u32x2 sc[2],
                                        const u32x2 st[2], f16x8 pa, f32x4& o) {
    const u32x2 r0 = tr16(smem, chunk_offset<TT>(wv0));
    const u32x2 r1 = tr16(smem, chunk_offset<TT>(wv1));
    const u32x4 b = {mul2(r0[0], sc[0][0]), mul2(r0[1], sc[0][1]), mul2(r1[0], sc[1][0]),
                     mul2(r1[1], sc[1][1])};
    o = mfma16(pa, as_f16x8(b), o);
    if constexpr (DT == RBQ_F16) {
        const u32x4 e = {mul2(r0[0], st[0][0]), mul2(r0[1], st[0][1]), mul2(r1[0], st[1][0]),
                         mul2(r1[1], st[1][1])};
        o = mfma16(pa, as_f16x8(e), o);
    }
}

template <int DT, int MK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_mfma_kernel(MArgs a) {
    __shared__ __align__(16) unsigned char smem[kSmemBytes];
    __shared__ __align__(16) unsigned char tbuf[kTbufBytes];

    // Every argument the prologue uses, loaded in one batch of scalar loads:
    // left to itself the compiler loads each field where it is first used,
    // one round trip of the scalar memory path each, and the first tile
    // transfer waited behind three of them.
    asm volatile("" ::"s"(a.q), "s"(a.kw), "s"(a.ks), "s"(a.kb), "s"(a.vw), "s"(a.vs), "s"(a.vb),
                 "s"(a.rot), "s"(a.capacity), "s"(a.T), "s"(a.chunk), "s"(a.Hkv), "s"(a.n_rep),
                 "s"(a.L), "s"(a.G), "s"(a.S), "s"(a.RB), "s"(a.kn), "s"(a.vn), "s"(a.n_new),
                 "s"(a.causal), "s"(a.round_rot), "s"(a.rb0), "s"(a.bh0));
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int j = lane >> 4;
    const int n = lane & 15;
    const int r = n & 7;                // query row of this lane in the query operands
    const bool lo_part = n >= 8;
    const int rb = 4 * (j & 1);         // accumulator rows of this lane: rb .. rb+3

    // grid: x = key split, y = block of 8 query rows, z = (b, kv head)
    const int split = blockIdx.x;
    const int rblk = a.rb0 + blockIdx.y;
    const int bh = a.bh0 + blockIdx.z;
    const int bhr = bh * a.RB + rblk;           // (b, kv head, block of 8 rows)
    const int r0 = 8 * rblk;                    // first query row of the block
    const int T = a.T;
    const int t_begin = split * a.chunk;
    const int t_end = (t_begin + a.chunk < T) ? t_begin + a.chunk : T;

    // ---- loads first: query row `wave` (row bh * G + R of q: the G rows of
    //      a kv head are its q heads' L rows), 4-element block `lane`, and 8
    //      bytes of the rotation blocks (the workgroup reads them once, not
    //      once per wave: every workgroup reads the same 4 KB); then, with as
    //      little scalar work as possible in between, the wave's first tile.
    //      Their latency overlaps the table build, and waiting for the query
    //      does not wait for the tile. ----
    uint2 qraw = make_uint2(0u, 0u);
    if (r0 + wave < a.G)
        qraw = *reinterpret_cast<const uint2*>(
            a.q + ((int64_t)bh * a.G + r0 + wave) * kHeadDim + 4 * lane);
    const bool rotated = a.rot != nullptr;
    float2 rot2 = make_float2(0.f, 0.f);
    if (rotated) rot2 = reinterpret_cast<const float2*>(a.rot)[tid];
    const int64_t row0 = (int64_t)bh * a.capacity;
    const __amdgpu_buffer_rsrc_t kw_r = make_rsrc(a.kw + row0 * kKWords, (uint32_t)T * 128u);
    const __amdgpu_buffer_rsrc_t ks_r = make_rsrc(a.ks + row0 * kGroups, (uint32_t)T * 8u);
    const __amdgpu_buffer_rsrc_t kb_r = make_rsrc(a.kb + row0 * kGroups, (uint32_t)T * 8u);
    const __amdgpu_buffer_rsrc_t vw_r = make_rsrc(a.vw + row0 * kVWords, (uint32_t)T * 96u);
    const __amdgpu_buffer_rsrc_t vs_r = make_rsrc(a.vs + row0 * kGroups, (uint32_t)T * 8u);
    const __amdgpu_buffer_rsrc_t vb_r = make_rsrc(a.vb + row0 * kGroups, (uint32_t)T * 8u);
    const int n_tiles = (t_end - t_begin + kTile - 1) / kTile;
    const int it_first = wave_tile(0, wave, n_tiles);
    // fused append: the appended rows [T - n_new, T) that fall in this split,
    // [app_lo, app_lo + n_app), are quantized and written by this workgroup,
    // row app_lo + w by wave w, before any transfer of the workgroup reads
    // them.  With several blocks of query rows per kv head, the workgroup of
    // every block quantizes and writes the rows of its split itself: the
    // same code on the same inputs writes the same bytes, and each workgroup
    // reads only after its own stores are complete, so no workgroup depends
    // on another
    int app_lo = t_end, n_app = 0;
    if constexpr (MK == kMaskNone) {
        if (a.n_new > 0) {
            app_lo = max(T - a.n_new, t_begin);
            n_app = max(t_end - app_lo, 0);
        }
    }
    lds_u8* wbuf = (lds_u8*)tbuf + wave * kWaveAreaBytes;
    const unsigned char* wbuf_g = tbuf + wave * kWaveAreaBytes;
    const int t_first = t_begin + it_first * kTile;
    const bool defer_first = n_app > 0 && t_first < app_lo + n_app && t_first + kTile > app_lo;
    dma_tile(wbuf, defer_first ? T : t_first, lane, kw_r, ks_r, kb_r, vw_r, vs_r, vb_r);
    // the appended row of this wave, unrotated
    uint2 kraw = make_uint2(0u, 0u), vraw = make_uint2(0u, 0u);
    if constexpr (MK == kMaskNone) {
        if (wave < n_app) {
            const int64_t src =
                ((int64_t)bh * a.n_new + (app_lo + wave - (T - a.n_new))) * kHeadDim + 4 * lane;
            kraw = *reinterpret_cast<const uint2*>(a.kn + src);
            vraw = *reinterpret_cast<const uint2*>(a.vn + src);
        }
    }

    // ---- decode table: entry e = 4 fp16 codes (e >> 3k) & 7 ----
    for (int e = tid; e < 4096; e += kThreads) {
        uint32_t h[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            h[k] = __builtin_bit_cast(uint16_t, (_Float16)(float)((e >> (3 * k)) & 7));
        lds_st32(smem, 8 * e, h[0] | (h[1] << 16));
        lds_st32(smem, 8 * e + 4, h[2] | (h[3] << 16));
    }

    // ---- query row `wave` rotated and scaled by scale*log2(e) into LDS (the
    //      staging area of the tile loop, unused until then), with its
    //      statistics: the 4 group sums and E, the power of two that brings
    //      the largest |q| into [2^14, 2^15) (rows past G are zero) ----
    float* qrot = reinterpret_cast<float*>(smem + kStageOff);
    float* qstat = qrot + kRows * kHeadDim;  // [row][8]: group sums 0..3, E at 4
    float* rot_lds = qstat + kRows * 8;      // the 64 rotation blocks
    if (rotated) reinterpret_cast<float2*>(rot_lds)[tid] = rot2;
    lds_barrier();
    {
        const float x[4] = {elem_to_f32<DT>(qraw.x), elem_to_f32<DT>(qraw.x >> 16),
                            elem_to_f32<DT>(qraw.y), elem_to_f32<DT>(qraw.y >> 16)};
        float y[4];
        if (rotated) {
            float Bm[16];
            const float4* blk = reinterpret_cast<const float4*>(rot_lds + 16 * lane);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float4 v = blk[q4];
                Bm[4 * q4] = v.x;
                Bm[4 * q4 + 1] = v.y;
                Bm[4 * q4 + 2] = v.z;
                Bm[4 * q4 + 3] = v.w;
            }
            rotate4(x, Bm, y);
            if (a.round_rot) {
#pragma unroll
                for (int c = 0; c < 4; ++c) y[c] = elem_to_f32<DT>(f32_to_elem_bits<DT>(y[c]));
            }
        } else {
            y[0] = x[0]; y[1] = x[1]; y[2] = x[2]; y[3] = x[3];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) y[c] *= a.qscale;
        reinterpret_cast<float4*>(qrot)[wave * 64 + lane] = make_float4(y[0], y[1], y[2], y[3]);
        float mx = fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fmaxf(fabsf(y[2]), fabsf(y[3])));
        mx = max16(mx);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float gs = sum16(((y[0] + y[1]) + y[2]) + y[3]);  // group j = lane >> 4
        if (n == 0) qstat[wave * 8 + j] = gs;
        if (lane == 0) {
            int ex = 0;
            if (mx > 0.f) (void)frexpf(mx, &ex);
            qstat[wave * 8 + 4] = __int_as_float((mx > 0.f) ? 15 - ex : 0);
        }
    }
    if (wave < n_app) {
        // the appended row: rotated by the same blocks (from LDS), rounded to
        // the dtype when the cache asks for it, quantized and packed as the
        // append kernel does
        const float xk[4] = {elem_to_f32<DT>(kraw.x), elem_to_f32<DT>(kraw.x >> 16),
                             elem_to_f32<DT>(kraw.y), elem_to_f32<DT>(kraw.y >> 16)};
        const float xv[4] = {elem_to_f32<DT>(vraw.x), elem_to_f32<DT>(vraw.x >> 16),
                             elem_to_f32<DT>(vraw.y), elem_to_f32<DT>(vraw.y >> 16)};
        float yk[4], yv[4];
        if (rotated) {
            float Bm[16];
            const float4* blk = reinterpret_cast<const float4*>(rot_lds + 16 * lane);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float4 v = blk[q4];
                Bm[4 * q4] = v.x;
                Bm[4 * q4 + 1] = v.y;
                Bm[4 * q4 + 2] = v.z;
                Bm[4 * q4 + 3] = v.w;
            }
            rotate4(xk, Bm, yk);
            rotate4(xv, Bm, yv);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                yk[c] = xk[c];
                yv[c] = xv[c];
            }
        }
        if (a.round_rot) {
            round_row<DT>(yk);
            round_row<DT>(yv);
        }
        const int64_t dst = row0 + app_lo + wave;
        quantize_pack_row<DT, kKBits>(yk, lane, const_cast<uint32_t*>(a.kw) + dst * kKWords,
                                      const_cast<uint16_t*>(a.ks) + dst * kGroups,
                                      const_cast<uint16_t*>(a.kb) + dst * kGroups);
        quantize_pack_row<DT, kVBits>(yv, lane, const_cast<uint32_t*>(a.vw) + dst * kVWords,
                                      const_cast<uint16_t*>(a.vs) + dst * kGroups,
                                      const_cast<uint16_t*>(a.vb) + dst * kGroups);
    }
    lds_barrier();
    // ---- score operands, one (group g, half h2) set per wave: slot k of
    //      lane (j, n) holds element ci[k] of the 8 that word 8g + 2j + h2
    //      covers, of row r scaled by 2^E_r, times 1/16 for the slots fed by
    //      nibbles 1 and 3; fp16 hi part for n < 8, lo part for n >= 8 ----
    unsigned char* qa_lds = smem + kLutBytes;
    {
        constexpr int ci[8] = {0, 4, 1, 5, 2, 6, 3, 7};
        const int g = wave >> 1, h2 = wave & 1;
        const int Er = __float_as_int(qstat[r * 8 + 4]);
        // read through an LDS-typed pointer: through a generic one the compiler
        // cannot tell these reads from the tile transfer in flight and waits
        // for it
        typedef __attribute__((address_space(3))) const f32x4 lds_f32x4;
        const lds_f32x4* src = (const lds_f32x4*)((lds_u8*)smem + kStageOff +
                                                  4 * (r * kHeadDim + 64 * g + 16 * j + 8 * h2));
        const f32x4 v0 = src[0], v1 = src[1];
        const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        f16x8 qa;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            float x = ldexpf(v[ci[k]], Er);
            if (k & 2) x *= 0.0625f;
            const _Float16 hi = (_Float16)x;
            const _Float16 lo = (_Float16)(x - (float)hi);
            qa[k] = lo_part ? lo : hi;
        }
        *reinterpret_cast<f16x8*>(qa_lds + ((2 * g + h2) * 64 + lane) * 16) = qa;
    }
    // query operand of the bias MFMA: lane group j supplies k-slots
    // 8j+4..8j+7 (slots 8j..8j+3 are zero) against the 4 group biases of the
    // key, which every lane group of the key operand repeats (its slots
    // 8j..8j+3 hold the key's 4 group scales, which meet the zeros: the
    // operand is the tile's scale and bias words as they sit in registers).
    // Group j holds limb j of the 4 group sums.  Rows 0-7 are query rows 0-7, rows 8-14 query rows
    // 1-7 and row 15 is zero, so that accumulator registers 0 and 2 of lane
    // half hl hold rows rb + hl and rb + 2 + hl, the rows the lane keeps its
    // softmax state for.
    u32x4 qb_op = {0u, 0u, 0u, 0u};
    {
        const int rq = (n < 8) ? n : n - 7;
        if (rq < kRows) {
            float qsum[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) qsum[g] = qstat[rq * 8 + g];
            const int E = __float_as_int(qstat[rq * 8 + 4]);
            uint32_t x[4];
            if constexpr (DT == RBQ_BF16) {
                // exact three-limb bf16 split: hi, middle, low
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const uint32_t u = __float_as_uint(qsum[g]);
                    const float hi = __uint_as_float(u & 0xFFFF0000u);
                    const uint32_t u2 = __float_as_uint(qsum[g] - hi);
                    const float mid = __uint_as_float(u2 & 0xFFFF0000u);
                    x[g] = (j == 0) ? u >> 16
                         : (j == 1) ? u2 >> 16
                         : (j == 2) ? f32_to_bf16_bits(qsum[g] - hi - mid) : 0u;
                }
            } else {
                // fp16: sums scaled by 2^(E-6) (below 2^15 in magnitude), hi + lo
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float v = ldexpf(qsum[g], E - 6);
                    const _Float16 hi = (_Float16)v;
                    x[g] = (j == 0) ? (uint32_t)__builtin_bit_cast(uint16_t, hi)
                         : (j == 1) ? (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(v - (float)hi))
                                    : 0u;
                }
            }
            qb_op = (u32x4){0u, 0u, x[0] | x[1] << 16, x[2] | x[3] << 16};
        }
    }
    // the lane's two softmax rows rb + 2p + hl (p = 0, 1): power-of-two
    // factors and causal visibility
    const int hl = j >> 1;  // 0: lanes 0-31, 1: lanes 32-63
    float frow[2], grow[2];
    int vis[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int row = rb + 2 * p + hl;
        const int Er = __float_as_int(qstat[row * 8 + 4]);
        frow[p] = ldexpf(1.0f, 24 - Er);
        grow[p] = (DT == RBQ_BF16) ? 1.0f : ldexpf(1.0f, 6 - Er);
        const int R = r0 + row;
        vis[p] = (R < a.G && a.causal) ? T - a.L + (R % a.L) + 1 : T;
    }
    const int vis_min = min(vis[0], vis[1]);
    // the appended rows' stores are complete (written to the L2, which every
    // transfer of this compute unit reads through) before the barrier; the
    // transfers that read them are issued after it (a deferring wave's
    // placeholder transfer has landed before its buffer is refilled)
    if (wave < n_app || defer_first) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();  // query operands complete; query rows no longer read
    if (defer_first) dma_tile(wbuf, t_first, lane, kw_r, ks_r, kb_r, vw_r, vs_r, vb_r);
    // the 8 score operand sets, held in registers for the whole tile loop
    f16x8 qa_r[4][2];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
            qa_r[g][h2] = *reinterpret_cast<const f16x8*>(qa_lds + ((2 * g + h2) * 64 + lane) * 16);

    // per-wave staging for the transposing reads (byte offsets in smem)
    const uint32_t wbase = kStageOff + wave * kWaveBytes;
    const uint32_t s_off = wbase;                      // scales (or scale heads)
    const uint32_t t_off = wbase + kStageBytes;        // scale tails (fp16 caches)
    const uint32_t b_off = wbase + 2 * kStageBytes;    // biases
    const uint32_t p_off = wbase + 3 * kStageBytes;    // P hi/lo
    // P slot of (block, key, part, row quad)
    auto p_slot = [&](int blk, int key, int part, int quad) -> uint32_t {
        return p_off + ((((blk * 16 + key) * 2 + part) * 2 + quad) << 3);
    };
    // this lane's P store: key n, its row quad, lanes 32-63 the upper 4 bytes
    // (block 1: + 512, lo part: + 16)
    const uint32_t p_wr = p_slot(0, n, 0, j & 1) + 4 * hl;
    const float one = 1.0f;

    // mask: byte offsets of the lane's two rows (out of range past G: such
    // reads return zero) and the values for its keys n, 16 + n of a tile,
    // loaded one tile ahead
    constexpr int kMaskElem = (MK == kMaskBool) ? 1 : (MK == kMaskAddF32) ? 4 : 2;
    __amdgpu_buffer_rsrc_t mask_r;
    uint32_t mrow[2] = {0u, 0u};
    uint32_t mk[2][2] = {{0u, 0u}, {0u, 0u}};
    auto load_mask = [&](int tk, uint32_t (&m)[2][2]) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const uint32_t off = mrow[p] + (uint32_t)(tk + n + 16 * blk) * kMaskElem;
                if constexpr (MK == kMaskBool)
                    m[blk][p] = __builtin_amdgcn_raw_buffer_load_b8(mask_r, off, 0, 0);
                else if constexpr (MK == kMaskAddF32)
                    m[blk][p] = __builtin_amdgcn_raw_buffer_load_b32(mask_r, off, 0, 0);
                else
                    m[blk][p] = __builtin_amdgcn_raw_buffer_load_b16(mask_r, off, 0, 0);
            }
    };
    if constexpr (MK != kMaskNone) {
        mask_r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.mask), (short)0,
                                                   (int)a.mask_bytes, 0x00020000);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int R = r0 + rb + 2 * p + hl;
            mrow[p] = 0x80000000u;
            if (R < a.G) {
                const int b = bh / a.Hkv;
                const int h = (bh - b * a.Hkv) * a.n_rep + R / a.L;
                mrow[p] = (uint32_t)(((int64_t)b * a.msb + (int64_t)h * a.msh +
                                      (int64_t)(R % a.L) * a.msl) * kMaskElem);
            }
        }
        if (it_first < n_tiles) load_mask(t_begin + it_first * kTile, mk);
    }

    f32x4 O[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) O[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
    f32x4 Ob = {0.f, 0.f, 0.f, 0.f};
    // softmax state of the lane's two rows: reference maximum (raw score,
    // -inf until a key is seen), the partial row sum over the lane's keys, the
    // rescale threshold relative to the reference (8; -inf before the first
    // key) and, in bias-accumulator registers 0 and 2, -reference / grow (the
    // reference taken as 0 before the first key), so that the scores come out
    // already relative to the reference
    float m_ref[2] = {-INFINITY, -INFINITY};
    float l_part[2] = {0.f, 0.f};
    float thr[2] = {-INFINITY, -INFINITY};
    f32x4 cinit = {0.f, 0.f, 0.f, 0.f};
    // the value operands' power of two (wave-uniform): O and Ob hold the
    // products in units of 2^v_f; v_lim = 2^(13 + v_f)
    int v_f = 0;
    float v_lim = 8192.0f;

    for (int kth = 0, it = it_first; it < n_tiles; ++kth) {
        const int t0 = t_begin + it * kTile;
        const int it_next = wave_tile(kth + 1, wave, n_tiles);
        const int t_next = t_begin + it_next * kTile;
        // this tile's transfer is complete; its operands are read out, then the
        // buffer is refilled with the wave's next tile while this one is computed
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        TileLoads cur;
        read_tile(cur, wbuf_g, n, j);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        const bool more = it_next < n_tiles;  // the wave's next tile, in three parts
        if (more)
            dma_tile_part<0>(wbuf, t_next, lane, kw_r, ks_r, kb_r, vw_r, vs_r, vb_r);
        uint32_t mk_next[2][2] = {{0u, 0u}, {0u, 0u}};
        if constexpr (MK != kMaskNone)
            if (more) load_mask(t_next, mk_next);

        // ---- value scales and biases of the lane's (key, group) -> staging,
        //      each fp16 value repeated 4 times (the 8 bytes a transposing
        //      read takes one element of).  They enter the fp16 operands
        //      times 2^-F: F stays 0 until some |scale| or |bias| reaches
        //      2^13 * 2^F, then grows so that every one stays below 2^13
        //      (codes times scales below 7 * 2^13 < 65504) and the
        //      accumulators are rescaled to the new unit ----
        float vsf[2], vbf[2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            vsf[blk] = elem_to_f32<DT>(cur.vsb[blk]);
            vbf[blk] = elem_to_f32<DT>(cur.vbb[blk]);
        }
        {
            const float vm = fmaxf(fmaxf(fabsf(vsf[0]), fabsf(vsf[1])), fmaxf(fabsf(vbf[0]), fabsf(vbf[1])));
            if (__any(vm >= v_lim)) {  // rare: a wave-uniform branch
                float wm = max16(vm);
                wm = fmaxf(wm, __shfl_xor(wm, 16));
                wm = fmaxf(wm, __shfl_xor(wm, 32));
                int ex = 0;
                (void)frexpf(wm, &ex);  // wm < 2^ex
                const int f_new = __builtin_amdgcn_readfirstlane(max(v_f, ex - 13));
                const float r = ldexpf(1.0f, v_f - f_new);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
#pragma unroll
                    for (int t = 0; t < 16; ++t) O[t][c] *= r;
                    Ob[c] *= r;
                }
                v_f = f_new;
                v_lim = ldexpf(1.0f, 13 + v_f);
            }
            if (v_f != 0) {
                const float pf = ldexpf(1.0f, -v_f);
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) {
                    vsf[blk] *= pf;
                    vbf[blk] *= pf;
                }
            }
        }
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const uint32_t off = (blk * 64 + lane) << 3;
            uint32_t s2, b2;
            if constexpr (DT == RBQ_BF16) {
                const uint32_t x = __builtin_bit_cast(
                    uint32_t, (f16x2){(_Float16)vsf[blk], (_Float16)vbf[blk]});
                s2 = __builtin_amdgcn_perm(x, x, 0x01000100u);  // low half twice
                b2 = __builtin_amdgcn_perm(x, x, 0x03020302u);  // high half twice
            } else {
                // head: top 8 significant bits; tail: the other 3 (both exact
                // unless the scaled value falls below the fp16 normal range)
                const uint32_t sh = f32_to_f16_bits(vsf[blk]) & 0xFFF8u;
                const uint32_t st = __builtin_bit_cast(
                    uint16_t, (_Float16)(vsf[blk] - f16_bits_to_f32(sh)));
                s2 = sh * 0x10001u;
                b2 = f32_to_f16_bits(vbf[blk]) * 0x10001u;
                lds_st32(smem, t_off + off, st * 0x10001u);
                lds_st32(smem, t_off + off + 4, st * 0x10001u);
            }
            lds_st32(smem, s_off + off, s2);
            lds_st32(smem, s_off + off + 4, s2);
            lds_st32(smem, b_off + off, b2);
            lds_st32(smem, b_off + off + 4, b2);
        }

        // ---- scores: acc[row][key n] per group; scale, hi+lo, bias.  The hi
        //      and lo rows of accumulator registers (2p, 2p + 1) are combined
        //      by one lane-half swap: lanes 0-31 then hold row rb + 2p, lanes
        //      32-63 row rb + 2p + 1, i.e. the lane's row p ----
        float sc[2][2];  // [block][p], relative to the reference
        const bool full = (t0 + kTile <= t_end) && (t0 + kTile <= vis_min);
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            f32x4 acc[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                acc[g] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const uint32_t w = cur.kwv[blk][g][h2];
                    const uint32_t w8 = w >> 8;
                    const u32x4 kv = {w & 0x000F000Fu, w & 0x00F000F0u, w8 & 0x000F000Fu,
                                      w8 & 0x00F000F0u};
                    acc[g] = mfma16(qa_r[g][h2], as_f16x8(kv), acc[g]);
                }
            }
            const u32x4 kbop = {cur.ksw[blk][0], cur.ksw[blk][1], cur.kbw[blk][0], cur.kbw[blk][1]};
            f32x4 cb;
            if constexpr (DT == RBQ_BF16) cb = mfma16bf(qb_op, kbop, cinit);
            else cb = mfma16(as_f16x8(qb_op), as_f16x8(kbop), cinit);
            const float s0 = meta_f32<DT>(cur.ksw[blk][0], 0), s1 = meta_f32<DT>(cur.ksw[blk][0], 1);
            const float s2 = meta_f32<DT>(cur.ksw[blk][1], 0), s3 = meta_f32<DT>(cur.ksw[blk][1], 1);
            float t4[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                float t = s0 * acc[0][c];
                t = fmaf(s1, acc[1][c], t);
                t = fmaf(s2, acc[2][c], t);
                t4[c] = fmaf(s3, acc[3][c], t);
            }
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const auto sw = __builtin_amdgcn_permlane32_swap(
                    __float_as_uint(t4[2 * p]), __float_as_uint(t4[2 * p + 1]), false, false);
                const float tt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
                const float bias = (DT == RBQ_BF16) ? cb[2 * p] : cb[2 * p] * grow[p];
                sc[blk][p] = fmaf(tt, frow[p], bias);
            }
        }
        // the mask: a false boolean skips the key, an additive value (natural
        // log units, as the scaled scores) is added in base 2
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                if constexpr (MK == kMaskBool) {
                    if (mk[blk][p] == 0u) sc[blk][p] = -INFINITY;
                } else if constexpr (MK == kMaskAddF32) {
                    sc[blk][p] = fmaf(__uint_as_float(mk[blk][p]), kLog2e, sc[blk][p]);
                } else if constexpr (MK == kMaskAddElem) {
                    sc[blk][p] = fmaf(elem_to_f32<DT>(mk[blk][p]), kLog2e, sc[blk][p]);
                }
            }
        if (!full) {
            const int kb0 = t0 + n;
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const int key = kb0 + 16 * blk;
                    if (!(key < t_end && key < vis[p])) sc[blk][p] = -INFINITY;
                }
        }

        if (more)
            dma_tile_part<1>(wbuf, t_next, lane, kw_r, ks_r, kb_r, vw_r, vs_r, vb_r);
        // ---- online softmax per row (base 2), lazy rescale: the reference
        //      moves only when the tile maximum exceeds it by more than 2^8 ----
        float mx[2];
        bool need_any = false;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            mx[p] = max16(fmaxf(sc[0][p], sc[1][p]));
            need_any |= mx[p] > thr[p];
        }
        if (__any(need_any)) {
            float al[2];
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const bool need = mx[p] > thr[p];
                // new reference: this tile's maximum (raw = relative + old
                // reference, the latter 0 before the first key)
                const float mu = (m_ref[p] == -INFINITY) ? 0.f : m_ref[p];
                const float m_new = need ? mx[p] + mu : m_ref[p];
                al[p] = need ? __builtin_amdgcn_exp2f(m_ref[p] - m_new) : 1.0f;
                const float shift = need ? mx[p] : 0.f;
                sc[0][p] -= shift;
                sc[1][p] -= shift;
                l_part[p] *= al[p];
                m_ref[p] = m_new;
                if (need) thr[p] = 8.0f;
                cinit[2 * p] = (m_new == -INFINITY) ? 0.f : -m_new / grow[p];
            }
            // accumulator register c holds row rb + (0, 2, 1, 3)[c] (the P
            // operand's row order, below): rows rb + hl and rb + 2 + hl are
            // this lane's, the others the partner half's (lane ^ 32)
            const float pa0 = __shfl_xor(al[0], 32), pa1 = __shfl_xor(al[1], 32);
            const float alc[4] = {hl ? pa0 : al[0], hl ? pa1 : al[1], hl ? al[0] : pa0,
                                  hl ? al[1] : pa1};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
#pragma unroll
                for (int t = 0; t < 16; ++t) O[t][c] *= alc[c];
                Ob[c] *= alc[c];
            }
        }
        // p in fp16 hi + lo (exact: lo = p - hi) for the lane's two rows and
        // key n of each block.  P slot (block, key, part, row quad) holds rows
        // rb + 0, rb + 2, rb + 1, rb + 3 in that order: lanes 0-31 store the
        // first two, lanes 32-63 the last two.
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const float p0 = __builtin_amdgcn_exp2f(sc[blk][0]);
            const float p1 = __builtin_amdgcn_exp2f(sc[blk][1]);
            l_part[0] += p0;
            l_part[1] += p1;
            const uint32_t hi2 = __builtin_bit_cast(uint32_t, (f16x2){(_Float16)p0, (_Float16)p1});
            lds_st32(smem, p_wr + 512 * blk, hi2);
            lds_st32(smem, p_wr + 512 * blk + 16, f16_residuals(hi2, p0, p1, one));
        }
        if (more)
            dma_tile_part<2>(wbuf, t_next, lane, kw_r, ks_r, kb_r, vw_r, vs_r, vb_r);
        // A operand of P.V: row n (hi rows 0-7, lo rows 8-15; within each
        // quad of rows the slot order rb + 0, 2, 1, 3) x keys 4j + e of both
        // blocks; lane 4e + q addresses (key 4j + e, part q >> 1, quad q & 1)
        f16x8 pa;
        {
            const int e = n >> 2, q = n & 3;
            const u32x2 a0 = tr16(smem, p_slot(0, 4 * j + e, q >> 1, q & 1));
            const u32x2 a1 = tr16(smem, p_slot(1, 4 * j + e, q >> 1, q & 1));
            pa = as_f16x8((u32x4){a0[0], a0[1], a1[0], a1[1]});
        }

        // ---- P.V ----
        const uint32_t own = (uint32_t)lane << 3;
        u32x2 sc2[2], st2[2] = {{0u, 0u}, {0u, 0u}};
        sc2[0] = tr16(smem, s_off + own);
        sc2[1] = tr16(smem, s_off + 512 + own);
        if constexpr (DT == RBQ_F16) {
            st2[0] = tr16(smem, t_off + own);
            st2[1] = tr16(smem, t_off + 512 + own);
        }
        {
            const u32x2 b0 = tr16(smem, b_off + own);
            const u32x2 b1 = tr16(smem, b_off + 512 + own);
            Ob = mfma16(pa, as_f16x8((u32x4){b0[0], b0[1], b1[0], b1[1]}), Ob);
        }
        pv_tile<DT, 0>(smem, cur.wv[0], cur.wv[1], sc2, st2, pa, O[0]);
        pv_tile<DT, 1>(smem, cur.wv[0], cur.wv[1], sc2, st2, pa, O[1]);
        pv_tile<DT, 2>(smem, cur.wv[0], cur.wv[1], sc2, st2, pa, O[2]);
        pv_tile<DT, 3>(smem, cur.wv[0], cur.wv[1], sc2, st2, pa, O[3]);
        pv_tile<DT, 4>(smem, cur.wv[0], cur.wv[1], sc2, st2, pa, O[4]);
        pv_tile<DT, 5>(smem, cur.wv[0], cur.wv[1], sc2, st2, pa, O[5]);
        pv_tile<DT, 6>(smem, cur.wv[0], cur.wv[1], sc2, st2, pa, O[6]);
        pv_tile<DT, 7>(smem, cur.wv[0], cur.wv[1], sc2, st2, pa, O[7]);
        pv_tile<DT, 8>(smem, cur.wv[0], cur.wv[1], sc2, st2, pa, O[8]);
        pv_tile<DT, 9>(smem, cur.wv[0], cur.wv[1], sc2, st2, pa, O[9]);
        pv_tile<DT, 10>(smem, cur.wv[0], cur.wv[1], sc2, st2, pa, O[10]);
        pv_tile<DT, 11>(smem, cur.wv[0], cur.wv[1], sc2, st2, pa, O[11]);
        pv_tile<DT, 12>(smem, cur.wv[0], cur.wv[1], sc2, st2, pa, O[12]);
        pv_tile<DT, 13>(smem, cur.wv[0], cur.wv[1], sc2, st2, pa, O[13]);
        pv_tile<DT, 14>(smem, cur.wv[0], cur.wv[1], sc2, st2, pa, O[14]);
        pv_tile<DT, 15>(smem, cur.wv[0], cur.wv[1], sc2, st2, pa, O[15]);
        if constexpr (MK != kMaskNone) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int p = 0; p < 2; ++p) mk[blk][p] = mk_next[blk][p];
        }
        it = it_next;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // no transfer into the buffer in flight

    // ---- wave record, stored as soon as this wave's tiles are done: hi + lo
    //      rows combined two registers at a time (after the lane-half swap,
    //      lanes 0-31 hold the sums of the first register and lanes 32-63 those
    //      of the second), row sums over the 16 key lanes ----
    float* wrec = reinterpret_cast<float*>(tbuf) + wave * kWaveRecFloats;
    float* wob = wrec + kHeadDim * kRows;
    float* wml = wob + kGroups * kRows;
    // the value products back from units of 2^v_f (exact: a power of two)
    const float v_unit = ldexpf(1.0f, v_f);
    auto comb = [v_unit](float x, float y) -> float {
        const auto s2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false,
                                                         false);
        return (__uint_as_float(s2[0]) + __uint_as_float(s2[1])) * v_unit;
    };
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const int col = 64 * (n >> 2) + 4 * t + (n & 3);
        const float ra = comb(O[t][0], O[t][2]);  // row rb + hl
        const float rc = comb(O[t][1], O[t][3]);  // row rb + 2 + hl
        float* dst = wrec + col * kRows + 4 * ((j & 1) ^ ((col >> 3) & 1)) + hl;
        dst[0] = ra;
        dst[2] = rc;
    }
    {
        const float ra = comb(Ob[0], Ob[2]);
        const float rc = comb(Ob[1], Ob[3]);
        float* dst = wob + (n >> 2) * kRows + rb + hl;
        dst[0] = ra;
        dst[2] = rc;
    }
    {
        const float l0 = sum16(l_part[0]), l1 = sum16(l_part[1]);
        if (n == 0) {
            wml[rb + hl] = m_ref[0];
            wml[rb + 2 + hl] = m_ref[1];
            wml[kRows + rb + hl] = l0;
            wml[kRows + rb + 2 + hl] = l1;
        }
    }
    lds_barrier();

    // ---- merge the wave records.  Each wave first derives the weights
    //      2^(m_w - M) of all (wave w, row) pairs (lane = 8 w + row) into its
    //      own LDS area; then thread = (column col, rows 4h .. 4h+3) ----
    const int col = tid & (kHeadDim - 1);
    const int h = tid >> 8;
    const int grp = col >> 6;
    float M[4], Ls[4], acc[4];
    {
        const float* rml = reinterpret_cast<const float*>(tbuf) + (lane >> 3) * kWaveRecFloats +
                           kHeadDim * kRows + kGroups * kRows;
        const float mw = rml[lane & 7];
        const float lw = rml[kRows + (lane & 7)];
        float Mx = fmaxf(mw, __shfl_xor(mw, 8));
        Mx = fmaxf(Mx, __shfl_xor(Mx, 16));
        Mx = fmaxf(Mx, __shfl_xor(Mx, 32));
        const float wv = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - Mx);
        float Lw = wv * lw;
        Lw += __shfl_xor(Lw, 8);
        Lw += __shfl_xor(Lw, 16);
        Lw += __shfl_xor(Lw, 32);
        float* wts = reinterpret_cast<float*>(tbuf + kWeightOff) + wave * kWeightFloats;
        wts[lane] = wv;
        if (lane < kRows) {
            wts[kWaves * kRows + lane] = Mx;
            wts[kWaves * kRows + kRows + lane] = Lw;
        }
        const float4 Mv = *reinterpret_cast<const float4*>(wts + kWaves * kRows + 4 * h);
        const float4 Lv = *reinterpret_cast<const float4*>(wts + kWaves * kRows + kRows + 4 * h);
        M[0] = Mv.x; M[1] = Mv.y; M[2] = Mv.z; M[3] = Mv.w;
        Ls[0] = Lv.x; Ls[1] = Lv.y; Ls[2] = Lv.z; Ls[3] = Lv.w;
        acc[0] = acc[1] = acc[2] = acc[3] = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float* rw = reinterpret_cast<const float*>(tbuf) + w * kWaveRecFloats;
            const float4 o = *reinterpret_cast<const float4*>(rw + col * kRows + 4 * (h ^ ((col >> 3) & 1)));
            const float4 ob = *reinterpret_cast<const float4*>(rw + kHeadDim * kRows + grp * kRows + 4 * h);
            const float4 wt = *reinterpret_cast<const float4*>(wts + w * kRows + 4 * h);
            acc[0] = fmaf(wt.x, o.x + ob.x, acc[0]);
            acc[1] = fmaf(wt.y, o.y + ob.y, acc[1]);
            acc[2] = fmaf(wt.z, o.z + ob.z, acc[2]);
            acc[3] = fmaf(wt.w, o.w + ob.w, acc[3]);
        }
    }

    // ---- one split: the output; several: this split's record (the merge
    //      kernel that follows reads it) ----
    if (a.S == 1) {
        const float4 rv = rot_row(a.rot, col);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float av = acc[i], lv = Ls[i];
            if constexpr (MK == kMaskBool) {
                // a row whose every key the mask drops: the mean of its keys
                const int R = r0 + 4 * h + i;
                if (lv == 0.f && R < a.G) {
                    const int nv = a.causal ? T - a.L + (R % a.L) + 1 : T;
                    av = value_column_mean<DT>(a.vw, a.vs, a.vb, row0, nv, col, kVBits, kVWords,
                                               kGroups, kGroup);
                    lv = 1.f;
                }
            }
            store_out(a.out, rotated, rv, bh, a.G, col, r0 + 4 * h + i, av, lv);
        }
        return;
    }
    float* rp = a.rec + ((int64_t)bhr * a.S + split) * kRecFloats;
    if (col == 0) {
        *reinterpret_cast<float4*>(rp + 8 * h) = make_float4(M[0], Ls[0], M[1], Ls[1]);
        *reinterpret_cast<float4*>(rp + 8 * h + 4) = make_float4(M[2], Ls[2], M[3], Ls[3]);
    }
    *reinterpret_cast<float4*>(rp + 2 * kRows + col * kRows + 4 * h) =
        make_float4(acc[0], acc[1], acc[2], acc[3]);
}

// Merge of the split records of one (b, kv head) and one 64-column block:
// 128 threads, thread = (column, rows 4h .. 4h+3).  Records are read 16 at a
// time with all their loads in flight: thread t also reads (m, l) of row
// t >> 4 of member t & 15, from which the 16-lane reductions give the block's
// maximum M, the weights 2^(m - M) and the weighted row sum; blocks of 16 are
// folded into the running result rescaled to the larger maximum.
struct CArgs {
    const float* rec;
    const float* rot;
    float* out;
    int S, Hkv, n_rep, L, G, RB;
    // boolean-mask calls: rows without a kept key take the mean of their
    // keys' values (value_column_mean) from the cache
    int bool_mask, dt, T, causal;
    int64_t capacity;
    const uint32_t* vw;
    const uint16_t* vs;
    const uint16_t* vb;
    int vbits, vwords, ngroups, group;  // the cache's V layout
};

// NGR groups of 128 threads each take every NGR-th round of 16 records
// (group g: records 16 g .. 16 g + 15, then 16 (g + NGR) ..), with the same
// round count in every group so that all threads meet the same barriers (a
// round past the last record has no members and weight 0); the groups'
// (M, L, o) are then combined in group order.  NGR = 1 for up to 16 splits.
// RPT rows per thread: 4 (a workgroup per 64 columns, thread = (column,
// rows 4h .. 4h+3)) or 2 (per 32 columns, thread = (column, rows 2h, 2h+1)),
// the latter for calls with few (b, kv head) units, where the merge runs on
// few compute units.
template <int NGR, int RPT, int D>
__global__ __launch_bounds__(128 * NGR) void attn_mfma_merge_kernel(CArgs a) {
    constexpr int kCols = 128 * RPT / kRows;  // columns per workgroup: 64 or 32
    constexpr int kCB = D / kCols;            // column blocks per (b, kv head, 8 rows)
    constexpr int RF = 2 * kRows + kRows * D;  // floats per split record of head_dim D
    typedef float vecR __attribute__((ext_vector_type(RPT)));
    __shared__ float wts[NGR][kRows * 16];
    __shared__ float stat[NGR][2 * kRows];
    __shared__ float cmb[NGR > 1 ? NGR - 1 : 1][3][RPT][128];  // groups 1.. : M, L, o per (row i, thread)
    const int grp = threadIdx.x >> 7;
    const int tid = threadIdx.x & 127;
    const int bhr = blockIdx.x / kCB;
    const int bh = bhr / a.RB;
    const int r0 = 8 * (bhr - bh * a.RB);
    const int col = (blockIdx.x - bhr * kCB) * kCols + (tid % kCols);
    const int h = tid / kCols;  // rows RPT h .. RPT h + RPT - 1
    const float* base = a.rec + (int64_t)bhr * a.S * RF;
    const int wrow = tid >> 4, wmbr = tid & 15;
    const float4 rv = rot_row(a.rot, col);
    float M[RPT], Ls[RPT], acc[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        M[i] = -INFINITY;
        Ls[i] = 0.f;
        acc[i] = 0.f;
    }
    const int rounds = (a.S + 16 * NGR - 1) / (16 * NGR);
    for (int rd = 0; rd < rounds; ++rd) {
        const int m0 = 16 * (grp + NGR * rd);
        const int members = (a.S - m0 < 16) ? a.S - m0 : 16;  // <= 0: an empty round
        float2 ml = make_float2(-INFINITY, 0.f);
        if (wmbr < members)
            ml = *reinterpret_cast<const float2*>(base + (int64_t)(m0 + wmbr) * RF + 2 * wrow);
        vecR o[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int mbr = (k < members) ? m0 + k : 0;
            o[k] = *reinterpret_cast<const vecR*>(base + (int64_t)mbr * RF + 2 * kRows +
                                                  col * kRows + RPT * h);
        }
        const float Mx = max16(ml.x);
        const float wv = (ml.x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ml.x - Mx);
        const float Lsum = sum16(wv * ml.y);
        lds_barrier();  // the previous round's weights are read
        wts[grp][wrow * 16 + wmbr] = wv;
        if (wmbr == 0) {
            stat[grp][wrow] = Mx;
            stat[grp][kRows + wrow] = Lsum;
        }
        lds_barrier();
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int row = RPT * h + i;
            float ac = 0.f;
#pragma unroll
            for (int k = 0; k < 16; ++k) ac = fmaf(wts[grp][row * 16 + k], o[k][i], ac);
            const float Mc = stat[grp][row], Lc = stat[grp][kRows + row];
            const float Mn = fmaxf(M[i], Mc);
            const float fa = (M[i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M[i] - Mn);
            const float fc = (Mc == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(Mc - Mn);
            Ls[i] = fmaf(Lc, fc, Ls[i] * fa);
            acc[i] = fmaf(ac, fc, acc[i] * fa);
            M[i] = Mn;
        }
    }
    if constexpr (NGR > 1) {
        if (grp > 0) {
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                cmb[grp - 1][0][i][tid] = M[i];
                cmb[grp - 1][1][i][tid] = Ls[i];
                cmb[grp - 1][2][i][tid] = acc[i];
            }
        }
        lds_barrier();
        if (grp > 0) return;
#pragma unroll
        for (int g = 1; g < NGR; ++g)
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const float Mc = cmb[g - 1][0][i][tid];
                const float Mn = fmaxf(M[i], Mc);
                const float fa = (M[i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M[i] - Mn);
                const float fc = (Mc == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(Mc - Mn);
                Ls[i] = fmaf(cmb[g - 1][1][i][tid], fc, Ls[i] * fa);
                acc[i] = fmaf(cmb[g - 1][2][i][tid], fc, acc[i] * fa);
                M[i] = Mn;
            }
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        float av = acc[i], lv = Ls[i];
        const int R = r0 + RPT * h + i;
        if (a.bool_mask && lv == 0.f && R < a.G) {
            // no kept key in any split: the mean of the row's keys
            const int nv = a.causal ? a.T - a.L + (R % a.L) + 1 : a.T;
            const int64_t row0 = (int64_t)bh * a.capacity;
            av = (a.dt == RBQ_BF16)
                     ? value_column_mean<RBQ_BF16>(a.vw, a.vs, a.vb, row0, nv, col, a.vbits, a.vwords,
                                                   a.ngroups, a.group)
                     : value_column_mean<RBQ_F16>(a.vw, a.vs, a.vb, row0, nv, col, a.vbits, a.vwords,
                                                  a.ngroups, a.group);
            lv = 1.f;
        }
        store_out<D>(a.out, a.rot != nullptr, rv, bh, a.G, col, R, av, lv);
    }
}

}  // namespace

// ---- host side: planning and launch ----

int mfma_plan(const rbq_kv_cache* c, int32_t H_q, int32_t L, int32_t splits, MfmaPlan* p) {
    const int64_t G = (int64_t)(H_q / c->H_kv) * L;
    const int64_t RB = (G + kRows - 1) / kRows;  // blocks of 8 query rows, one workgroup each
    const int64_t T = c->offset;
    const int64_t units = (int64_t)c->B * c->H_kv * RB;
    int64_t S = splits;
    bool xcd_shared = false;
    if (S == 0) {
        S = (256 + units - 1) / units;  // about one workgroup per compute unit
        const int64_t max_s = (T + kWaves * kTile - 1) / (kWaves * kTile);
        if (S > max_s) S = max_s;
        // Several row blocks per (b, kv head): a split count that is a multiple
        // of 8 puts the row blocks of one (b, kv head, split) on one XCD, so
        // that they read their common tiles through that XCD's L2 (workgroups
        // go to the 8 XCDs round robin by linear index, and the split is the
        // fastest grid index).
        const int64_t s8 = (S + 7) / 8 * 8;
        if (RB > 1 && S > 1 && s8 <= max_s) {
            S = s8;
            xcd_shared = true;
        }
    }
    if (S < 1) S = 1;
    int64_t chunk = (T + S - 1) / S;
    // automatic plans give every split whole rounds of the 8 waves (whole
    // tiles where the split count is kept a multiple of 8); an explicit split
    // count is kept as closely as whole tiles allow
    const int64_t unit = (splits == 0 && !xcd_shared) ? (int64_t)kWaves * kTile : (int64_t)kTile;
    chunk = (chunk + unit - 1) / unit * unit;
    S = (T + chunk - 1) / chunk;
    if (units > 0x7FFFFFFF || units * S > 0x7FFFFFFF) return RBQ_EUNSUPPORTED;
    // the merge kernel's one launch: at most 2^32 - 1 work-items along x (8
    // column blocks x 512 threads per unit at most)
    if (S > 1 && units * 8 * 512 > 0xFFFFFFFFll) return RBQ_EUNSUPPORTED;
    // 32-bit buffer offsets, also for the tile reads past T (at most 4 tiles)
    if ((T + kWaves * kTile) * (int64_t)(kKWords * 4) > 0x7FFFFFFF) return RBQ_EUNSUPPORTED;
    p->S = (int)S;
    p->RB = (int)RB;
    p->chunk = chunk;
    p->ws_bytes = (S == 1) ? 0 : (size_t)units * S * kRecFloats * sizeof(float);
    return RBQ_OK;
}

// The merge of the split records of an attention call (one record per
// (b, kv head, block of 8 query rows, split), kRecordFloats floats each):
// normalisation, inverse rotation and the output rows.
void merge_launch(const rbq_kv_cache* c, const float* rec, const float* rot_blocks, float* out,
                  int S, int RB, int n_rep, int L, int causal, int mask_type, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    const int64_t units = (int64_t)c->B * c->H_kv * RB;
    CArgs m;
    m.rec = rec;
    m.rot = rot_blocks;
    m.out = out;
    m.S = S;
    m.Hkv = c->H_kv;
    m.n_rep = n_rep;
    m.L = L;
    m.G = n_rep * L;
    m.RB = RB;
    m.bool_mask = (mask_type == kMaskBool) ? 1 : 0;
    m.dt = c->dtype;
    m.T = (int)c->offset;
    m.causal = causal ? 1 : 0;
    m.capacity = c->capacity;
    m.vw = c->v_words;
    m.vs = (const uint16_t*)c->v_scales;
    m.vb = (const uint16_t*)c->v_biases;
    m.vbits = c->v_bits;
    m.vwords = c->head_dim * c->v_bits / 32;
    m.ngroups = c->head_dim / c->group_size;
    m.group = c->group_size;
    // up to 16 splits: one group of 128 threads; more: 2 or 4 groups side
    // by side, so that a long key range (many splits of few kv heads) is
    // merged in S / 64 rounds of loads instead of S / 16 (8 groups would
    // spill registers at 1024 threads)
    // few (b, kv head, 8 rows) units: 32 columns per workgroup, twice the
    // workgroups
    // (records of head_dim 256: the dedicated kernel's or the prefill
    // kernel's; 128 or 64: the prefill kernel's)
    const bool narrow = units < kMergeNarrowUnits;
    const int colblocks = c->head_dim / (narrow ? 32 : 64);
    const dim3 mg((unsigned)(units * colblocks));
    auto go = [&](auto k1, auto k2, auto k4) {
        if (S <= 16) hipLaunchKernelGGL(k1, mg, dim3(128), 0, s, m);
        else if (S <= 32) hipLaunchKernelGGL(k2, mg, dim3(256), 0, s, m);
        else hipLaunchKernelGGL(k4, mg, dim3(512), 0, s, m);
    };
    if (c->head_dim == kHeadDim) {
        if (narrow)
            go(attn_mfma_merge_kernel<1, 2, kHeadDim>, attn_mfma_merge_kernel<2, 2, kHeadDim>,
               attn_mfma_merge_kernel<4, 2, kHeadDim>);
        else
            go(attn_mfma_merge_kernel<1, 4, kHeadDim>, attn_mfma_merge_kernel<2, 4, kHeadDim>,
               attn_mfma_merge_kernel<4, 4, kHeadDim>);
    } else if (c->head_dim == 128) {
        if (narrow)
            go(attn_mfma_merge_kernel<1, 2, 128>, attn_mfma_merge_kernel<2, 2, 128>,
               attn_mfma_merge_kernel<4, 2, 128>);
        else
            go(attn_mfma_merge_kernel<1, 4, 128>, attn_mfma_merge_kernel<2, 4, 128>,
               attn_mfma_merge_kernel<4, 4, 128>);
    } else {
        if (narrow)
            go(attn_mfma_merge_kernel<1, 2, 64>, attn_mfma_merge_kernel<2, 2, 64>,
               attn_mfma_merge_kernel<4, 2, 64>);
        else
            go(attn_mfma_merge_kernel<1, 4, 64>, attn_mfma_merge_kernel<2, 4, 64>,
               attn_mfma_merge_kernel<4, 4, 64>);
    }
}

int mfma_launch(const rbq_kv_cache* c, const void* q, int32_t H_q, int32_t L, float scale,
                int32_t causal, const AttnMask& mk, const float* rot_blocks, float* out,
                const MfmaPlan& p, void* ws, void* stream, const FusedAppend* app) {
    hipStream_t s = (hipStream_t)stream;
    MArgs a;
    a.kn = app ? (const uint16_t*)app->k : nullptr;
    a.vn = app ? (const uint16_t*)app->v : nullptr;
    a.n_new = app ? app->n : 0;
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
    a.capacity = c->capacity;
    a.T = (int)c->offset;
    a.chunk = (int)p.chunk;
    a.Hkv = c->H_kv;
    a.n_rep = H_q / c->H_kv;
    a.L = L;
    a.G = a.n_rep * L;
    a.S = p.S;
    a.RB = p.RB;
    a.causal = causal ? 1 : 0;
    a.qscale = scale * kLog2e;
    a.mask = mk.ptr;
    a.msb = mk.sb;
    a.msh = mk.sh;
    a.msl = mk.sl;
    a.mask_bytes = mk.bytes;
    a.round_rot = (c->flags & RBQ_FLAG_ROUND_ROTATED) ? 1 : 0;
    // grid x = key split, y = row block, z = (b, kv head); y and z in pieces
    // of at most kGridYZ, launched one after another with their offsets
    const int64_t BH = (int64_t)c->B * c->H_kv;
    const int mt = mk.ptr == nullptr ? kMaskNone : mk.type;
    auto launch = [&](auto kernel) {
        for (int64_t bh0 = 0; bh0 < BH; bh0 += kGridYZ)
            for (int64_t rb0 = 0; rb0 < p.RB; rb0 += kGridYZ) {
                a.bh0 = (int)bh0;
                a.rb0 = (int)rb0;
                const dim3 grid((unsigned)p.S, (unsigned)std::min<int64_t>(kGridYZ, p.RB - rb0),
                                (unsigned)std::min<int64_t>(kGridYZ, BH - bh0));
                hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, s, a);
            }
    };
    if (c->dtype == RBQ_BF16) {
        if (mt == kMaskNone) launch(attn_mfma_kernel<RBQ_BF16, kMaskNone>);
        else if (mt == kMaskBool) launch(attn_mfma_kernel<RBQ_BF16, kMaskBool>);
        else if (mt == kMaskAddF32) launch(attn_mfma_kernel<RBQ_BF16, kMaskAddF32>);
        else launch(attn_mfma_kernel<RBQ_BF16, kMaskAddElem>);
    } else {
        if (mt == kMaskNone) launch(attn_mfma_kernel<RBQ_F16, kMaskNone>);
        else if (mt == kMaskBool) launch(attn_mfma_kernel<RBQ_F16, kMaskBool>);
        else if (mt == kMaskAddF32) launch(attn_mfma_kernel<RBQ_F16, kMaskAddF32>);
        else launch(attn_mfma_kernel<RBQ_F16, kMaskAddElem>);
    }
    if (p.S > 1) merge_launch(c, a.rec, rot_blocks, out, p.S, p.RB, a.n_rep, L, a.causal, mt, stream);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_hip_error((int)e);
        return RBQ_EHIP;
    }
    return RBQ_OK;
}

// ---- C ABI: argument checks, planning, dispatch ----

namespace {

int check_attn(const rbq_kv_cache* c, int32_t H_q, int32_t L, int32_t splits) {
    int st = check_cache(c);
    if (st != RBQ_OK) return st;
    if (H_q <= 0 || H_q % c->H_kv != 0 || splits < 0) return RBQ_EINVAL;
    if (L < 1 || (int64_t)L > c->offset) return RBQ_ERANGE;
    if ((int64_t)(H_q / c->H_kv) * L > 0x3FFFFFFF) return RBQ_EUNSUPPORTED;
    return RBQ_OK;
}

// Which kernel runs a call, and its plan: the prefill kernel where it takes
// the call (prefill_takes: from kPrefillMinRows query rows per kv head, bf16,
// 4-bit K in groups of 64); otherwise the dedicated kernel for the default
// configuration and the tile kernel for every other.
struct AttnPlan {
    bool tile;
    bool prefill;
    MfmaPlan mp;
    TilePlan tp;
    int S;
    size_t ws_bytes;
};

int attn_plan(const rbq_kv_cache* c, int32_t H_q, int32_t L, int32_t splits, AttnPlan* p) {
    const int64_t G = (int64_t)(H_q / c->H_kv) * L;
    p->prefill = prefill_takes(c, H_q, L);
    p->tile = !p->prefill && !(is_default_config(c) && G <= kDedicatedMaxRows);
    int st;
    if (p->prefill) {
        st = prefill_plan(c, H_q, L, splits, &p->mp);
        p->S = p->mp.S;
        p->ws_bytes = p->mp.ws_bytes;
    } else if (p->tile) {
        st = tile_plan(c, H_q, L, splits, &p->tp);
        p->S = p->tp.S;
        p->ws_bytes = p->tp.ws_bytes;
    } else {
        st = mfma_plan(c, H_q, L, splits, &p->mp);
        p->S = p->mp.S;
        p->ws_bytes = p->mp.ws_bytes;
    }
    return st;
}

// Mask arguments: type, non-negative strides, and the byte extent of the
// elements the call can read (the last row's keys [0, offset)), which must
// fit the kernel's 31-bit buffer offsets.
int check_mask(const rbq_kv_cache* c, int32_t H_q, int32_t L, const void* mask, int32_t type,
               int64_t sb, int64_t sh, int64_t sl, AttnMask* m) {
    m->ptr = mask;
    m->type = RBQ_MASK_NONE;
    m->sb = m->sh = m->sl = 0;
    m->bytes = 0;
    if (mask == nullptr) return type == RBQ_MASK_NONE ? RBQ_OK : RBQ_EINVAL;
    if (type != RBQ_MASK_BOOL && type != RBQ_MASK_ADD_F32 && type != RBQ_MASK_ADD_DTYPE)
        return RBQ_EINVAL;
    if (sb < 0 || sh < 0 || sl < 0) return RBQ_EINVAL;
    if (sb > (int64_t)1 << 40 || sh > (int64_t)1 << 40 || sl > (int64_t)1 << 40)
        return RBQ_EUNSUPPORTED;
    const int64_t esize = (type == RBQ_MASK_BOOL) ? 1 : (type == RBQ_MASK_ADD_F32) ? 4 : 2;
    // each term below 2^31 * 2^40: the sum in 128 bits
    const __int128 last = (__int128)(c->B - 1) * sb + (__int128)(H_q - 1) * sh +
                          (__int128)(L - 1) * sl + c->offset;
    if (last * esize > 0x7FFFFFFF - 64 * 4) return RBQ_EUNSUPPORTED;
    m->type = type;
    m->sb = sb;
    m->sh = sh;
    m->sl = sl;
    m->bytes = (uint32_t)(last * esize);
    return RBQ_OK;
}

// ---- the fixed scratch array of rbq_quant_attn_decode_noalloc ----
// The split records of that entry point live here instead of in a caller's
// workspace: RBQ_SCRATCH_BYTES per device, allocated with the code object and
// held until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is a stand-in, not a device address): the device
// address comes from hipGetSymbolAddress, taken once per device with that
// device current and kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[RBQ_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch array.
int scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        set_hip_error((int)e);
        return RBQ_EHIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return RBQ_EUNSUPPORTED;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || p == nullptr) {
                set_hip_error((int)e);
                return RBQ_EHIP;
            }
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return RBQ_OK;
}

// Checks, plan and launch of one attention call with the split records in
// `ws` (ws_fixed: the scratch array, whose size is RBQ_SCRATCH_BYTES).
int attn_call(const rbq_kv_cache* c, const void* q, int32_t H_q, int32_t L, float scale,
              int32_t causal, const void* mask, int32_t mask_type, int64_t msb, int64_t msh,
              int64_t msl, const float* rot_blocks, float* out, int32_t splits, void* ws,
              size_t ws_bytes, bool ws_fixed, void* stream) {
    int st = check_attn(c, H_q, L, splits);
    if (st != RBQ_OK) return st;
    if (q == nullptr || out == nullptr) return RBQ_EINVAL;
    if ((reinterpret_cast<uintptr_t>(q) & 7) != 0 || (reinterpret_cast<uintptr_t>(out) & 15) != 0 ||
        (reinterpret_cast<uintptr_t>(rot_blocks) & 15) != 0 || (reinterpret_cast<uintptr_t>(ws) & 15) != 0)
        return RBQ_EINVAL;
    AttnMask mk;
    st = check_mask(c, H_q, L, mask, mask_type, msb, msh, msl, &mk);
    if (st != RBQ_OK) return st;
    AttnPlan ap;
    st = attn_plan(c, H_q, L, splits, &ap);
    if (st != RBQ_OK) return st;
    if (ws_fixed) {
        if (ap.ws_bytes > RBQ_SCRATCH_BYTES) return RBQ_ESCRATCH;
        if (ap.ws_bytes > 0) {
            st = scratch_address(&ws);
            if (st != RBQ_OK) return st;
        }
    } else if (ap.ws_bytes > 0 && (ws == nullptr || ws_bytes < ap.ws_bytes)) {
        return RBQ_EWORKSPACE;
    }
    if (ap.tile) return tile_launch(c, q, H_q, L, scale, causal, mk, rot_blocks, out, ap.tp, ws, stream);
    if (ap.prefill) return prefill_launch(c, q, H_q, L, scale, causal, mk, rot_blocks, out, ap.mp, ws, stream);
    return mfma_launch(c, q, H_q, L, scale, causal, mk, rot_blocks, out, ap.mp, ws, stream);
}

}  // namespace

}  // namespace rbq

using namespace rbq;

extern "C" int32_t rbq_quant_attn_splits(const rbq_kv_cache* c, int32_t H_q, int32_t L) {
    int st = check_attn(c, H_q, L, 0);
    if (st != RBQ_OK) return st;
    AttnPlan ap;
    st = attn_plan(c, H_q, L, 0, &ap);
    return st != RBQ_OK ? st : ap.S;
}

extern "C" size_t rbq_quant_attn_workspace_bytes(const rbq_kv_cache* c, int32_t H_q, int32_t L,
                                                 int32_t splits) {
    if (check_attn(c, H_q, L, splits) != RBQ_OK) return 0;
    AttnPlan ap;
    return attn_plan(c, H_q, L, splits, &ap) == RBQ_OK ? ap.ws_bytes : 0;
}

extern "C" int rbq_quant_attn_decode_mask(const rbq_kv_cache* c, const void* q, int32_t H_q,
                                          int32_t L, float scale, int32_t causal, const void* mask,
                                          int32_t mask_type, int64_t mask_stride_b,
                                          int64_t mask_stride_h, int64_t mask_stride_l,
                                          const float* rot_blocks, float* out, int32_t splits,
                                          void* ws, size_t ws_bytes, void* stream) {
    return attn_call(c, q, H_q, L, scale, causal, mask, mask_type, mask_stride_b, mask_stride_h,
                     mask_stride_l, rot_blocks, out, splits, ws, ws_bytes, false, stream);
}

extern "C" int rbq_quant_attn_decode_noalloc(const rbq_kv_cache* c, const void* q, int32_t H_q,
                                             int32_t L, float scale, int32_t causal,
                                             const float* rot_blocks, float* out, int32_t splits,
                                             void* stream) {
    return attn_call(c, q, H_q, L, scale, causal, nullptr, RBQ_MASK_NONE, 0, 0, 0, rot_blocks, out,
                     splits, nullptr, 0, true, stream);
}

extern "C" int rbq_kv_append_attn_decode(rbq_kv_cache* c, const void* k, const void* v,
                                         int64_t n, const void* q, int32_t H_q, int32_t L,
                                         float scale, int32_t causal, const float* rot_blocks,
                                         float* out, int32_t splits, void* ws, size_t ws_bytes,
                                         void* stream) {
    // every argument of both steps is checked before anything is launched
    int st = check_cache(c);
    if (st != RBQ_OK) return st;
    if (n < 0) return RBQ_EINVAL;
    if (n > 0 && (k == nullptr || v == nullptr)) return RBQ_EINVAL;
    if (c->offset + n > c->capacity) return RBQ_ECAPACITY;
    rbq_kv_cache after = *c;
    after.offset += n;
    st = check_attn(&after, H_q, L, splits);
    if (st != RBQ_OK) return st;
    if (q == nullptr || out == nullptr) return RBQ_EINVAL;
    if ((reinterpret_cast<uintptr_t>(q) & 7) != 0 || (reinterpret_cast<uintptr_t>(out) & 15) != 0 ||
        (reinterpret_cast<uintptr_t>(rot_blocks) & 15) != 0 || (reinterpret_cast<uintptr_t>(ws) & 15) != 0)
        return RBQ_EINVAL;
    AttnPlan ap;
    st = attn_plan(&after, H_q, L, splits, &ap);
    if (st != RBQ_OK) return st;
    if (ap.ws_bytes > 0 && (ws == nullptr || ws_bytes < ap.ws_bytes)) return RBQ_EWORKSPACE;
    const bool fused = n > 0 && !ap.tile && !ap.prefill && n <= kWaves &&
                       (reinterpret_cast<uintptr_t>(k) & 7) == 0 &&
                       (reinterpret_cast<uintptr_t>(v) & 7) == 0;
    if (!fused) {
        // the two steps as two launches: the append kernel, then the attention
        st = rbq_kv_quant_append(c, k, v, n, rot_blocks, stream);
        if (st != RBQ_OK) return st;
        return rbq_quant_attn_decode(c, q, H_q, L, scale, causal, rot_blocks, out, splits, ws,
                                     ws_bytes, stream);
    }
    AttnMask mk;
    st = check_mask(&after, H_q, L, nullptr, RBQ_MASK_NONE, 0, 0, 0, &mk);
    if (st != RBQ_OK) return st;
    const FusedAppend fa = {k, v, (int)n};
    st = mfma_launch(&after, q, H_q, L, scale, causal, mk, rot_blocks, out, ap.mp, ws, stream, &fa);
    if (st != RBQ_OK) return st;
    c->offset += n;
    return RBQ_OK;
}

extern "C" int rbq_quant_attn_decode(const rbq_kv_cache* c, const void* q, int32_t H_q, int32_t L,
                                     float scale, int32_t causal, const float* rot_blocks,
                                     float* out, int32_t splits, void* ws, size_t ws_bytes,
                                     void* stream) {
    return rbq_quant_attn_decode_mask(c, q, H_q, L, scale, causal, nullptr, RBQ_MASK_NONE, 0, 0, 0,
                                      rot_blocks, out, splits, ws, ws_bytes, stream);
}
