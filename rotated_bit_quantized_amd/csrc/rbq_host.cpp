// Host-only parts of librbq: the rotation block build, the cache capacity
// rule, trim/commit bookkeeping, descriptor validation and status strings.
//
// Built with -ffp-contract=off: the rotation build below must perform exactly
// the IEEE double operations it spells out, in that order, with no fused
// multiply-add, so that its float results are reproducible bit for bit.
#include <math.h>
#include <string.h>

#include "rbq_internal.h"

namespace rbq {

namespace {
thread_local int g_last_hip_error = 0;
}

void set_hip_error(int err) { g_last_hip_error = err; }

int check_cache(const rbq_kv_cache* c) {
    if (c == nullptr) return RBQ_EINVAL;
    if (c->B <= 0 || c->H_kv <= 0 || c->capacity < 0 || c->offset < 0 ||
        c->offset > c->capacity || (c->flags & ~RBQ_FLAG_ROUND_ROTATED) != 0)
        return RBQ_EINVAL;
    auto width_ok = [](int b) { return b == 2 || b == 3 || b == 4 || b == 5 || b == 6 || b == 8; };
    if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256) return RBQ_EUNSUPPORTED;
    if (c->group_size != 32 && c->group_size != 64 && c->group_size != 128) return RBQ_EUNSUPPORTED;
    if (c->head_dim % c->group_size != 0) return RBQ_EUNSUPPORTED;
    if (!width_ok(c->k_bits) || !width_ok(c->v_bits)) return RBQ_EUNSUPPORTED;
    if (c->dtype != RBQ_F16 && c->dtype != RBQ_BF16) return RBQ_EUNSUPPORTED;
    const int64_t slabs = (int64_t)c->B * c->H_kv;
    if (c->capacity > kMaxRows || slabs > kMaxSlabs || c->capacity > kMaxTotalRows / slabs)
        return RBQ_EUNSUPPORTED;
    if (c->capacity > 0 &&
        (c->k_words == nullptr || c->k_scales == nullptr || c->k_biases == nullptr ||
         c->v_words == nullptr || c->v_scales == nullptr || c->v_biases == nullptr))
        return RBQ_EINVAL;
    // the kernels move the word arrays in 16-byte and the scale / bias arrays
    // in 4-byte pieces from the array bases
    auto misaligned = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; };
    if (misaligned(c->k_words, 16) || misaligned(c->v_words, 16) || misaligned(c->k_scales, 4) ||
        misaligned(c->k_biases, 4) || misaligned(c->v_scales, 4) || misaligned(c->v_biases, 4))
        return RBQ_EINVAL;
    return RBQ_OK;
}

}  // namespace rbq

using namespace rbq;

namespace {

// Left-multiplication matrix of quaternion (w, x, y, z) with the entries of
// _quat_left on the quant_kv.py page ("SO(4) block rotation").
void quat_left(const double q[4], double m[4][4]) {
    const double w = q[0], x = q[1], y = q[2], z = q[3];
    const double rows[4][4] = {{w, -x, -y, -z}, {x, w, -z, y}, {y, z, w, -x}, {z, -y, x, w}};
    memcpy(m, rows, sizeof(rows));
}

// The matrix printed for _quat_right_conj on the same page, taken as printed
// (it is the transpose of quat_left(q)).
void quat_right_conj(const double q[4], double m[4][4]) {
    const double w = q[0], x = q[1], y = q[2], z = q[3];
    const double rows[4][4] = {{w, x, y, z}, {-x, w, z, -y}, {-y, -z, w, x}, {-z, y, -x, w}};
    memcpy(m, rows, sizeof(rows));
}

// Matrix of v -> v * conj(q) for quaternions as column vectors (w, x, y, z):
// the map the _quat_right_conj docstring on the same page describes.  With
// p = conj(q) = (w, -x, -y, -z), the Hamilton product v * p has components
// (v0 p0 - v1 p1 - v2 p2 - v3 p3, v0 p1 + v1 p0 + v2 p3 - v3 p2,
//  v0 p2 - v1 p3 + v2 p0 + v3 p1, v0 p3 + v1 p2 - v2 p1 + v3 p0).
void quat_right_mul_conj(const double q[4], double m[4][4]) {
    const double p0 = q[0], p1 = -q[1], p2 = -q[2], p3 = -q[3];
    const double rows[4][4] = {{p0, -p1, -p2, -p3}, {p1, p0, p3, -p2}, {p2, -p3, p0, p1},
                               {p3, p2, -p1, p0}};
    memcpy(m, rows, sizeof(rows));
}

// q = a / |a| in double: squares summed left to right, correctly rounded
// sqrt and divisions.  Returns false for a zero vector.
bool normalize(const float a[4], double q[4]) {
    const double a0 = a[0], a1 = a[1], a2 = a[2], a3 = a[3];
    double s = a0 * a0;
    s = s + a1 * a1;
    s = s + a2 * a2;
    s = s + a3 * a3;
    const double n = sqrt(s);
    if (!(n > 0.0)) return false;
    q[0] = a0 / n;
    q[1] = a1 / n;
    q[2] = a2 / n;
    q[3] = a3 / n;
    return true;
}

// x rounded half to even to the grid of a binary format with `mant_bits`
// fraction bits, smallest normal exponent `emin` (subnormals below it) and
// largest finite value `maxval`; beyond it the result is an infinity.  The
// scaling by powers of two and the rounding to an integer are exact in double
// for every float x, and nearbyint rounds half to even in the default mode.
float round_to_format(float x, int mant_bits, int emin, double maxval) {
    if (x == 0.0f) return x;
    int e = 0;
    (void)frexp((double)x, &e);  // |x| in [2^(e-1), 2^e)
    int ex = e - 1;
    if (ex < emin) ex = emin;
    const double q = ldexp(nearbyint(ldexp((double)x, mant_bits - ex)), ex - mant_bits);
    if (fabs(q) > maxval) return x < 0 ? -INFINITY : INFINITY;
    return (float)q;
}

}  // namespace

extern "C" {

int rbq_rotation_round(float* blocks, int32_t head_dim, int32_t dtype) {
    if (blocks == nullptr || head_dim <= 0 || head_dim % 4 != 0) return RBQ_EINVAL;
    if (dtype != RBQ_F16 && dtype != RBQ_BF16) return RBQ_EUNSUPPORTED;
    const int n = head_dim * 4;
    for (int i = 0; i < n; ++i)
        if (!isfinite(blocks[i])) return RBQ_EINVAL;
    for (int i = 0; i < n; ++i)
        blocks[i] = (dtype == RBQ_F16) ? round_to_format(blocks[i], 10, -14, 65504.0)
                                       : round_to_format(blocks[i], 7, -126, 0x1.FEp127);
    return RBQ_OK;
}

int rbq_rotation_build(const float* draws, int32_t head_dim, float* blocks) {
    return rbq_rotation_build_mode(draws, head_dim, RBQ_ROT_PRINTED, blocks);
}

int rbq_rotation_build_mode(const float* draws, int32_t head_dim, int32_t mode, float* blocks) {
    if (draws == nullptr || blocks == nullptr || head_dim <= 0 || head_dim % 4 != 0)
        return RBQ_EINVAL;
    if (mode != RBQ_ROT_PRINTED && mode != RBQ_ROT_TWO_SIDED) return RBQ_EINVAL;
    const int nb = head_dim / 4;
    for (int b = 0; b < nb; ++b) {
        double qL[4], qR[4], Lm[4][4], Rm[4][4];
        if (!normalize(draws + b * 8, qL) || !normalize(draws + b * 8 + 4, qR))
            return RBQ_EINVAL;
        quat_left(qL, Lm);
        if (mode == RBQ_ROT_PRINTED) quat_right_conj(qR, Rm);
        else quat_right_mul_conj(qR, Rm);
        float* out = blocks + b * 16;
        for (int i = 0; i < 4; ++i) {
            for (int j = 0; j < 4; ++j) {
                double s = Lm[i][0] * Rm[0][j];
                s = s + Lm[i][1] * Rm[1][j];
                s = s + Lm[i][2] * Rm[2][j];
                s = s + Lm[i][3] * Rm[3][j];
                out[i * 4 + j] = (float)s;
            }
        }
    }
    return RBQ_OK;
}

int64_t rbq_kv_required_capacity(int64_t capacity, int64_t offset, int64_t n) {
    if (n < 0 || offset < 0 || capacity < 0 || offset > capacity) return RBQ_EINVAL;
    if (capacity > kMaxRows || n > kMaxRows) return RBQ_EUNSUPPORTED;
    if (capacity > 0 && offset + n <= capacity) return capacity;
    const int64_t new_steps = (n + kStep - 1) / kStep * kStep;
    if (capacity == 0) return new_steps;
    const int64_t kept = (offset % kStep != 0) ? offset : capacity;
    if (kept + new_steps > kMaxRows) return RBQ_EUNSUPPORTED;
    return kept + new_steps;
}

int64_t rbq_kv_trim(rbq_kv_cache* c, int64_t n) {
    if (c == nullptr || n < 0) return RBQ_EINVAL;
    const int64_t t = n < c->offset ? n : c->offset;
    c->offset -= t;
    return t;
}

int64_t rbq_kv_commit_verified(rbq_kv_cache* c, int64_t verified_len, int64_t accepted_len) {
    if (c == nullptr || verified_len < 0 || accepted_len < 0 || accepted_len > verified_len)
        return RBQ_EINVAL;
    const int64_t rejected = verified_len - accepted_len;
    return rejected ? rbq_kv_trim(c, rejected) : 0;
}

const char* rbq_status_string(int status) {
    switch (status) {
        case RBQ_OK: return "ok";
        case RBQ_EINVAL: return "invalid argument";
        case RBQ_EUNSUPPORTED: return "unsupported configuration";
        case RBQ_ECAPACITY: return "cache capacity exceeded";
        case RBQ_ERANGE: return "query block length out of range (need 1 <= L <= offset)";
        case RBQ_EWORKSPACE: return "workspace missing or too small";
        case RBQ_EHIP: return "HIP runtime error";
        case RBQ_ESCRATCH: return "the call needs more than the fixed scratch array holds";
        default: return "unknown status";
    }
}

int rbq_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
