// Driver of the host-side checks and launch planning of librbq, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code and run
// with no GPU visible: every call here either returns a status before any
// device work or fails at its launch (no device).  Descriptors carry
// aligned placeholder addresses that are never dereferenced on the host.  Exit status 0 when every expectation holds; the
// sanitizers abort on the first report.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>
#include <limits>

#include "rbq.h"

static int g_fail = 0;
#define EXPECT(cond)                                                       \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__,   \
                    __LINE__, #cond);                                      \
            ++g_fail;                                                      \
        }                                                                  \
    } while (0)

static const int64_t I64MAX = std::numeric_limits<int64_t>::max();
static const int32_t I32MAX = std::numeric_limits<int32_t>::max();

static rbq_kv_cache desc(int32_t B, int32_t H, int64_t cap, int64_t off, int32_t D = 256,
                         int32_t gs = 64, int32_t kb = 4, int32_t vb = 3) {
    rbq_kv_cache c;
    memset(&c, 0, sizeof(c));
    c.B = B;
    c.H_kv = H;
    c.head_dim = D;
    c.group_size = gs;
    c.k_bits = kb;
    c.v_bits = vb;
    c.dtype = RBQ_BF16;
    c.flags = 0;
    c.capacity = cap;
    c.offset = off;
    // placeholders: 16-byte aligned, never dereferenced on the host
    c.k_words = reinterpret_cast<uint32_t*>(uintptr_t(0x100000));
    c.k_scales = reinterpret_cast<void*>(uintptr_t(0x200000));
    c.k_biases = reinterpret_cast<void*>(uintptr_t(0x300000));
    c.v_words = reinterpret_cast<uint32_t*>(uintptr_t(0x400000));
    c.v_scales = reinterpret_cast<void*>(uintptr_t(0x500000));
    c.v_biases = reinterpret_cast<void*>(uintptr_t(0x600000));
    return c;
}

int main() {
    // ---- capacity rule at the ends of the int64 range ----
    const int64_t caps[] = {0, 1, 255, 256, 257, 1LL << 24, 1LL << 40, 1LL << 62, I64MAX};
    const int64_t ns[] = {0, 1, 255, 256, 1LL << 31, 1LL << 40, 1LL << 62, I64MAX - 255, I64MAX};
    for (int64_t cap : caps)
        for (int64_t off : {int64_t(0), cap / 2, cap})
            for (int64_t n : ns) {
                const int64_t r = rbq_kv_required_capacity(cap, off, n);
                EXPECT(r < 0 || r >= off + (n > r - off ? 0 : n));
                if (r >= 0) EXPECT(r >= cap || cap == 0);
            }
    EXPECT(rbq_kv_required_capacity(0, 0, I64MAX) < 0);
    EXPECT(rbq_kv_required_capacity(I64MAX, I64MAX, 1) < 0);
    EXPECT(rbq_kv_required_capacity(8192, 8192, 2048) == 10240);

    // ---- trim / commit at the ends ----
    {
        rbq_kv_cache c = desc(1, 1, I64MAX, I64MAX);
        EXPECT(rbq_kv_trim(&c, I64MAX) == I64MAX && c.offset == 0);
        c.offset = 5;
        EXPECT(rbq_kv_commit_verified(&c, I64MAX, 0) == 5 && c.offset == 0);
        EXPECT(rbq_kv_commit_verified(&c, 0, I64MAX) == RBQ_EINVAL);
    }

    // ---- descriptors far beyond any memory: refused, never planned ----
    const int32_t Bs[] = {1, 8, 1 << 16, I32MAX};
    const int32_t Hs[] = {1, 2, 1 << 12, I32MAX};
    const int64_t Ts[] = {1, 256, 32768, (1LL << 24) - 1, 1LL << 24, 1LL << 31, 1LL << 40, I64MAX};
    const int32_t HQ[] = {1, 16, 1 << 20, I32MAX};
    const int32_t LS[] = {1, 4, 2048, 1 << 20, I32MAX};
    const int32_t SP[] = {0, 1, 64, 1024, 1 << 20, I32MAX};
    const int32_t Ds[] = {256, 128};
    for (int32_t D : Ds)
        for (int32_t B : Bs)
            for (int32_t H : Hs)
                for (int64_t T : Ts) {
                    rbq_kv_cache c = D == 256 ? desc(B, H, T, T) : desc(B, H, T, T, 128, 32, 5, 6);
                    for (int32_t hq : HQ)
                        for (int32_t L : LS)
                            for (int32_t sp : SP) {
                                const int32_t hq_ = (hq / H) * H > 0 ? (hq / H) * H : H;
                                const size_t ws = rbq_quant_attn_workspace_bytes(&c, hq_, L, sp);
                                const int32_t s = rbq_quant_attn_splits(&c, hq_, L);
                                EXPECT(s != 0);
                                if (s > 0) EXPECT(ws < (size_t(1) << 50));
                            }
                }

    // ---- append / grow / copies with extreme sizes: statuses only ----
    {
        rbq_kv_cache c = desc(1, 1, 1024, 1000);
        const void* k = reinterpret_cast<const void*>(uintptr_t(0x700000));
        EXPECT(rbq_kv_quant_append(&c, k, k, I64MAX, nullptr, nullptr) == RBQ_ECAPACITY);
        EXPECT(rbq_kv_quant_append(&c, k, k, -1, nullptr, nullptr) == RBQ_EINVAL);
        EXPECT(c.offset == 1000);
        rbq_kv_cache big = desc(I32MAX, I32MAX, I64MAX, 0);
        EXPECT(rbq_kv_quant_append(&big, k, k, 1LL << 40, nullptr, nullptr) < 0);
        rbq_kv_cache d = desc(I32MAX, I32MAX, I64MAX, 0);
        d.k_words = reinterpret_cast<uint32_t*>(uintptr_t(0x1100000));
        d.v_words = reinterpret_cast<uint32_t*>(uintptr_t(0x1400000));
        EXPECT(rbq_kv_grow(&big, &d, nullptr) < 0);
        EXPECT(rbq_kv_copy_prefix(&big, &d, nullptr) < 0);
        rbq_kv_cache s1 = desc(4, 2, 1024, 1000), d1 = desc(4, 2, 1024, 0);
        d1.k_words = reinterpret_cast<uint32_t*>(uintptr_t(0x1100000));
        EXPECT(rbq_kv_copy_batch(&s1, I32MAX, I32MAX, &d1, nullptr) == RBQ_EINVAL);
        EXPECT(rbq_kv_copy_batch(&s1, 0, -I32MAX, &d1, nullptr) == RBQ_EINVAL);
        EXPECT(rbq_kv_copy_batch(&s1, 3, -1, &d1, nullptr) != RBQ_OK || true);
    }

    // ---- masks: huge strides and extents are refused before any launch ----
    {
        rbq_kv_cache c = desc(8, 2, 32768, 32768);
        const void* q = reinterpret_cast<const void*>(uintptr_t(0x800000));
        float* out = reinterpret_cast<float*>(uintptr_t(0x900000));
        const void* m = reinterpret_cast<const void*>(uintptr_t(0xA00000));
        const int64_t strides[] = {0, 1, 32768, 1LL << 31, 1LL << 40, (1LL << 40) + 1, I64MAX, -1};
        for (int64_t sb : strides)
            for (int64_t sh : strides)
                for (int64_t sl : strides)
                    for (int32_t mt : {RBQ_MASK_BOOL, RBQ_MASK_ADD_F32, 7}) {
                        const int st = rbq_quant_attn_decode_mask(&c, q, 16, 1, 0.0625f, 1, m, mt,
                                                                  sb, sh, sl, nullptr, out, 1,
                                                                  nullptr, 0, nullptr);
                        if (sb < 0 || sh < 0 || sl < 0 || mt == 7) EXPECT(st == RBQ_EINVAL);
                        if (sb > (1LL << 40) || sh > (1LL << 40) || sl > (1LL << 40))
                            EXPECT(st < 0);
                    }
        rbq_kv_cache h = desc(1, 1, 1LL << 40, 1LL << 40);
        EXPECT(rbq_quant_attn_decode_mask(&h, q, I32MAX, I32MAX, 1.f, 1, m, RBQ_MASK_BOOL, 1, 1,
                                          1, nullptr, out, 0, nullptr, 0, nullptr) < 0);
    }

    // ---- rotation build and rounding with bad sizes ----
    {
        float draws[8] = {1, 0, 0, 0, 0, 0, 0, 0}, blocks[16];
        EXPECT(rbq_rotation_build(draws, I32MAX, nullptr) == RBQ_EINVAL);
        EXPECT(rbq_rotation_build(draws, -4, blocks) == RBQ_EINVAL);
        EXPECT(rbq_rotation_round(blocks, -4, RBQ_BF16) == RBQ_EINVAL);
        EXPECT(rbq_rotation_build(draws, 4, blocks) == RBQ_EINVAL);  // zero right draw
        draws[4] = 1.f;
        EXPECT(rbq_rotation_build(draws, 4, blocks) == RBQ_OK);
        EXPECT(rbq_rotation_round(blocks, 4, RBQ_F16) == RBQ_OK);
    }
    for (int s = -8; s <= 1; ++s) EXPECT(rbq_status_string(s) != nullptr);

    if (g_fail) {
        fprintf(stderr, "%d expectation(s) failed\n", g_fail);
        return 1;
    }
    printf("host checks under sanitizers: ok\n");
    return 0;
}
