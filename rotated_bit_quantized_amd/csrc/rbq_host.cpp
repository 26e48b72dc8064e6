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
        c->offset > c->capacity || c->reserved != 0)
        return RBQ_EINVAL;
    if (c->head_dim != kHeadDim || c->group_size != kGroup || c->k_bits != kKBits ||
        c->v_bits != kVBits)
        return RBQ_EUNSUPPORTED;
    if (c->dtype != RBQ_F16 && c->dtype != RBQ_BF16) return RBQ_EUNSUPPORTED;
    if (c->capacity > 0 &&
        (c->k_words == nullptr || c->k_scales == nullptr || c->k_biases == nullptr ||
         c->v_words == nullptr || c->v_scales == nullptr || c->v_biases == nullptr))
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

}  // namespace

extern "C" {

int rbq_rotation_build(const float* draws, int32_t head_dim, float* blocks) {
    if (draws == nullptr || blocks == nullptr || head_dim <= 0 || head_dim % 4 != 0)
        return RBQ_EINVAL;
    const int nb = head_dim / 4;
    for (int b = 0; b < nb; ++b) {
        double qL[4], qR[4], Lm[4][4], Rm[4][4];
        if (!normalize(draws + b * 8, qL) || !normalize(draws + b * 8 + 4, qR))
            return RBQ_EINVAL;
        quat_left(qL, Lm);
        quat_right_conj(qR, Rm);
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
    if (capacity > 0 && offset + n <= capacity) return capacity;
    const int64_t new_steps = (n + kStep - 1) / kStep * kStep;
    if (capacity == 0) return new_steps;
    const int64_t kept = (offset % kStep != 0) ? offset : capacity;
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
        default: return "unknown status";
    }
}

int rbq_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
