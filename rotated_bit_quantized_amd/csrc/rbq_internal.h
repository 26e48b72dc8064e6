// Internal helpers shared by the host-side C++ and the HIP translation units
// of librbq.  Not part of the public ABI (that is include/rbq.h).
#pragma once

#include <stdint.h>

#include "rbq.h"

namespace rbq {

constexpr int kHeadDim = 256;
constexpr int kGroup = 64;
constexpr int kKBits = 4;
constexpr int kVBits = 3;
constexpr int kStep = 256;               // cache growth step (update_and_fetch)
constexpr int kKWords = kHeadDim * kKBits / 32;   // 32
constexpr int kVWords = kHeadDim * kVBits / 32;   // 24
constexpr int kGroups = kHeadDim / kGroup;        // 4

// Size limits of a descriptor (RBQ_EUNSUPPORTED beyond them): rows per
// (b, kv head), (b, kv head) slabs, and rows of all slabs together.  Far
// beyond any device memory, they keep every size and offset computation of
// the host code and the kernels inside int64 (and the grids inside their
// 32-bit counts, which the launch planning checks on its own).
constexpr int64_t kMaxRows = (int64_t)1 << 40;
constexpr int64_t kMaxSlabs = ((int64_t)1 << 31) - 1;
constexpr int64_t kMaxTotalRows = (int64_t)1 << 44;

// Records the hipError_t of the last failed HIP call on this thread.
void set_hip_error(int err);

// Validates the descriptor fields shared by every device entry point:
// non-null buffers, positive B/H_kv, 0 <= offset <= capacity, known flags,
// and a supported configuration (RBQ_EUNSUPPORTED otherwise).
int check_cache(const rbq_kv_cache* c);

// True for the configuration with dedicated kernels: head_dim 256, group 64,
// K 4-bit, V 3-bit.
inline bool is_default_config(const rbq_kv_cache* c) {
    return c->head_dim == kHeadDim && c->group_size == kGroup && c->k_bits == kKBits &&
           c->v_bits == kVBits;
}

// Row sizes of the six arrays in 16-bit units (a scale or bias row of one
// group is a single 16-bit element).
struct RowUnits {
    int kw, meta, vw;  // K words, each scale / bias array, V words
};
inline RowUnits row_units(const rbq_kv_cache* c) {
    return {c->head_dim * c->k_bits / 16, c->head_dim / c->group_size,
            c->head_dim * c->v_bits / 16};
}

// Launch plan of the matrix-core attention path: key splits, their length,
// blocks of 8 query rows, and the workspace for the split records.
// Optional attention mask (rbq_quant_attn_decode_mask): element strides for
// batch, q head and query row; `bytes` = extent the kernel may read.
struct AttnMask {
    const void* ptr;
    int type;  // RBQ_MASK_*
    int64_t sb, sh, sl;
    uint32_t bytes;
};

struct MfmaPlan {
    int S;           // key splits
    int RB;          // blocks of 8 query rows per kv head
    int64_t chunk;   // keys per split
    size_t ws_bytes;
};
int mfma_plan(const rbq_kv_cache* c, int32_t H_q, int32_t L, int32_t splits, MfmaPlan* p);

// Split record of the dedicated and prefill attention kernels, one per (b,
// kv head, block of 8 query rows, key split): (m, l) of the 8 rows (m the
// row's reference score in base 2, l its sum of 2^(score - m)), then the
// unnormalised output column-major [head_dim columns][8 rows]; floats per
// record at head_dim D: record_floats(D) (kRecordFloats at 256).
constexpr int record_floats(int D) { return 2 * 8 + 8 * D; }
constexpr int kRecordFloats = record_floats(kHeadDim);
// The merge of the records of a call with S > 1 splits (RB blocks of 8 rows
// per kv head; head_dim 256, 128 or 64, the cache's V layout for the rows below):
// normalisation, inverse rotation, output rows; mask_type RBQ_MASK_BOOL: rows
// without a kept key take the mean of their keys' values.
void merge_launch(const rbq_kv_cache* c, const float* rec, const float* rot_blocks, float* out,
                  int S, int RB, int n_rep, int L, int causal, int mask_type, void* stream);

// Prefill-length attention over bf16 or fp16 caches with 4-bit K codes in groups of
// 64 or 128 (head_dim 64, 128 or 256, V codes of 2 to 4 bits), blocks of 128 query rows
// per kv head sharing each decoded tile: used from kPrefillMinRows query rows
// per kv head (prefill_takes), with any split count.
constexpr int64_t kPrefillMinRows = 96;
bool prefill_takes(const rbq_kv_cache* c, int32_t H_q, int32_t L);
int prefill_plan(const rbq_kv_cache* c, int32_t H_q, int32_t L, int32_t splits, MfmaPlan* p);
int prefill_launch(const rbq_kv_cache* c, const void* q, int32_t H_q, int32_t L, float scale,
                   int32_t causal, const AttnMask& mk, const float* rot_blocks, float* out,
                   const MfmaPlan& p, void* ws, void* stream);

// Launch plan of the general tile attention (every configuration, any number
// of query rows): waves per workgroup (16 query rows each: 1 up to 16 rows
// per kv head, else 4), key splits, row blocks, and the workspace of the
// split records (o floats, then (m, l) pairs).
struct TilePlan {
    int W;
    int reg;  // single-wave workgroups with register-staged tiles (fixed widths)
    int pr;   // single-wave workgroups, staged tiles, paired hi / lo operand rows
    int S;
    int RBW;
    int64_t chunk;
    size_t o_floats;
    size_t ws_bytes;
};
int tile_plan(const rbq_kv_cache* c, int32_t H_q, int32_t L, int32_t splits, TilePlan* p);
int tile_launch(const rbq_kv_cache* c, const void* q, int32_t H_q, int32_t L, float scale,
                int32_t causal, const AttnMask& mk, const float* rot_blocks, float* out,
                const TilePlan& p, void* ws, void* stream);

// The default configuration runs the dedicated kernel at every number of
// query rows per kv head (H_q / H_kv x L): measured against the tile kernel
// it is 1.4-1.7x faster from 64 to 2048 rows and equal on a 2048-token
// prefill chunk.  Every other configuration runs the tile kernel.
constexpr int kDedicatedMaxRows = 0x3FFFFFFF;
// Rows appended by the attention launch itself (the dedicated kernel, no
// mask, one block of query rows per kv head): the last n cache rows below
// c->offset are quantized from k / v ([B][H_kv][n][256], unrotated).
struct FusedAppend {
    const void* k;
    const void* v;
    int n;
};
int mfma_launch(const rbq_kv_cache* c, const void* q, int32_t H_q, int32_t L, float scale,
                int32_t causal, const AttnMask& mk, const float* rot_blocks, float* out,
                const MfmaPlan& p, void* ws, void* stream, const FusedAppend* app = nullptr);

}  // namespace rbq
