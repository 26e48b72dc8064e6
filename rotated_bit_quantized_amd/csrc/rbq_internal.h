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

// Records the hipError_t of the last failed HIP call on this thread.
void set_hip_error(int err);

// Validates the descriptor fields shared by every device entry point:
// non-null buffers, positive B/H_kv, 0 <= offset <= capacity, reserved == 0,
// and the supported configuration (RBQ_EUNSUPPORTED otherwise).
int check_cache(const rbq_kv_cache* c);

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
int mfma_launch(const rbq_kv_cache* c, const void* q, int32_t H_q, int32_t L, float scale,
                int32_t causal, const AttnMask& mk, const float* rot_blocks, float* out,
                const MfmaPlan& p, void* ws, void* stream);

}  // namespace rbq
