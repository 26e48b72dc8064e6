// Fused decode/verify attention over the packed K4/V3 cache
// (asym_quantized_sdpa on the quant_kv.py page) with the SO(4) rotation of q
// on entry and the inverse rotation of the output, plus the split-T
// log-sum-exp combine.
//
// Work decomposition: a workgroup owns one (b, kv head, row block, key
// split).  The rows of a kv head are the G = (H_q/H_kv) * L query rows that
// read it (q head h reads kv head h / n_rep); a row block holds up to RB of
// them.  Keys of the split are scanned in tiles of 64 with an online softmax;
// the partial (m, l, o) is either finalised in place (one split) or written
// to the workspace for attn_combine_kernel.
#include <hip/hip_runtime.h>

#include "rbq_common.h"

namespace rbq {
namespace {

constexpr int kTile = 64;

struct AttnArgs {
    const uint16_t* q;  // [B][Hq][L][256]
    const uint32_t* kw;
    const uint16_t* ks;
    const uint16_t* kb;
    const uint32_t* vw;
    const uint16_t* vs;
    const uint16_t* vb;
    const float* rot;   // [64][4][4] or null
    float* out;         // [B][Hq][L][256]
    float* ws_o;        // partial outputs [B][Hkv][n_rb][S][RB][256]
    float* ws_ml;       // partial (m, l)  [B][Hkv][n_rb][S][RB][2]
    int64_t capacity;
    int64_t T;          // keys in the cache (offset)
    int64_t chunk;      // keys per split
    int Hkv, n_rep, L, G, n_rb, S, causal;
    float scale;
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
    return x;
}

// One wave per workgroup.  QK: lane = key (dequantise its K row, dot with the
// rotated, scaled q rows held in LDS).  PV: lane = 4 output channels (one
// rotation block), keys read from an LDS copy of the V tile.
template <int DT, int RB>
__global__ __launch_bounds__(64) void attn_valu_kernel(AttnArgs a) {
    __shared__ float q_s[RB][kHeadDim];
    __shared__ float p_s[RB][kTile];
    __shared__ uint32_t v_s[kTile * kVWords + 4];
    __shared__ uint16_t vm_s[kTile][2 * kGroups];  // scales then biases

    const int lane = threadIdx.x;
    const int split = blockIdx.x;
    const int kvh = blockIdx.y / a.n_rb;
    const int rb = blockIdx.y - kvh * a.n_rb;
    const int b = blockIdx.z;
    const int64_t bh = (int64_t)b * a.Hkv + kvh;

    float Bm[16];
    load_block(a.rot, lane, Bm);

    // rows of this block: global row gr = rb*RB + rr -> q head kvh*n_rep + gr/L, position gr%L;
    // vis[rr] = keys visible to the row (causal: t <= T - L + i)
    int vis[RB];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
        const int gr = rb * RB + rr;
        float y[4] = {0.f, 0.f, 0.f, 0.f};
        vis[rr] = 0;
        if (gr < a.G) {
            const int h = kvh * a.n_rep + gr / a.L;
            const int i = gr % a.L;
            float x[4];
            load4<DT>(a.q + (((int64_t)b * a.Hkv * a.n_rep + h) * a.L + i) * kHeadDim + lane * 4,
                      x);
            if (a.rot != nullptr) rotate4(x, Bm, y);
            else {
                y[0] = x[0]; y[1] = x[1]; y[2] = x[2]; y[3] = x[3];
            }
            vis[rr] = (int)(a.causal ? a.T - a.L + i + 1 : a.T);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) q_s[rr][lane * 4 + e] = y[e] * a.scale;
    }

    float m[RB], lsum[RB], o[RB][4];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
        m[rr] = -INFINITY;
        lsum[rr] = 0.f;
        o[rr][0] = o[rr][1] = o[rr][2] = o[rr][3] = 0.f;
    }

    const int64_t t_begin = (int64_t)split * a.chunk;
    int64_t t_end = t_begin + a.chunk;
    if (t_end > a.T) t_end = a.T;

    const uint32_t* kw_bh = a.kw + bh * a.capacity * kKWords;
    const uint16_t* ks_bh = a.ks + bh * a.capacity * kGroups;
    const uint16_t* kb_bh = a.kb + bh * a.capacity * kGroups;
    const uint32_t* vw_bh = a.vw + bh * a.capacity * kVWords;
    const uint16_t* vs_bh = a.vs + bh * a.capacity * kGroups;
    const uint16_t* vb_bh = a.vb + bh * a.capacity * kGroups;

    const int g_own = lane >> 4;          // group of this lane's 4 channels in PV
    const int bit0 = 12 * lane;           // first bit of this lane's 4 V codes in a row
    const int wlo = bit0 >> 5, sh = bit0 & 31;

    __syncthreads();
    for (int64_t t0 = t_begin; t0 < t_end; t0 += kTile) {
        const int nt = (int)((t_end - t0) < kTile ? (t_end - t0) : kTile);
        // stage the V tile (nt rows x 24 words) and its scales/biases in LDS
        for (int u = lane; u < nt * kVWords; u += 64) v_s[u] = vw_bh[t0 * kVWords + u];
        for (int u = lane; u < nt * kGroups; u += 64) {
            vm_s[u / kGroups][u % kGroups] = vs_bh[t0 * kGroups + u];
            vm_s[u / kGroups][kGroups + u % kGroups] = vb_bh[t0 * kGroups + u];
        }

        // ---- QK: lane = key t ----
        const int64_t t = t0 + lane;
        float acc[RB];
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) acc[rr] = 0.f;
        if (lane < nt) {
            const uint4* krow = reinterpret_cast<const uint4*>(kw_bh + t * kKWords);
            const uint2 sraw = *reinterpret_cast<const uint2*>(ks_bh + t * kGroups);
            const uint2 braw = *reinterpret_cast<const uint2*>(kb_bh + t * kGroups);
            const uint32_t sw[2] = {sraw.x, sraw.y}, bw[2] = {braw.x, braw.y};
#pragma unroll
            for (int g = 0; g < kGroups; ++g) {
                const float sg = elem_to_f32<DT>(sw[g >> 1] >> (16 * (g & 1)));
                const float bg = elem_to_f32<DT>(bw[g >> 1] >> (16 * (g & 1)));
#pragma unroll
                for (int qd = 0; qd < 2; ++qd) {
                    const uint4 w4 = krow[g * 2 + qd];
                    const uint32_t ws4[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
                    for (int wi = 0; wi < 4; ++wi) {
                        const int d0 = g * 64 + qd * 32 + wi * 8;
#pragma unroll
                        for (int nib = 0; nib < 8; ++nib) {
                            const float kh = fmaf((float)((ws4[wi] >> (4 * nib)) & 15u), sg, bg);
#pragma unroll
                            for (int rr = 0; rr < RB; ++rr)
                                acc[rr] = fmaf(q_s[rr][d0 + nib], kh, acc[rr]);
                        }
                    }
                }
            }
        }

        // ---- online softmax (m is wave-uniform, l kept per lane) ----
        float alpha[RB];
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) {
            const float sc = (lane < nt && t < vis[rr]) ? acc[rr] : -INFINITY;
            const float m_new = fmaxf(m[rr], wave_max(sc));
            float p;
            if (m_new == -INFINITY) {
                alpha[rr] = 1.f;
                p = 0.f;
            } else {
                alpha[rr] = expf(m[rr] - m_new);
                p = expf(sc - m_new);
            }
            lsum[rr] = lsum[rr] * alpha[rr] + p;
            m[rr] = m_new;
            p_s[rr][lane] = p;
        }
        __syncthreads();

        // ---- PV: lane = channels [4*lane, 4*lane+4) ----
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) {
            o[rr][0] *= alpha[rr];
            o[rr][1] *= alpha[rr];
            o[rr][2] *= alpha[rr];
            o[rr][3] *= alpha[rr];
        }
        for (int j = 0; j < nt; ++j) {
            const uint32_t lo = v_s[j * kVWords + wlo];
            const uint32_t hi = v_s[j * kVWords + wlo + 1];  // padded: stays in the array
            const uint32_t bits = (uint32_t)((((uint64_t)hi << 32) | lo) >> sh);
            const float sg = elem_to_f32<DT>(vm_s[j][g_own]);
            const float bg = elem_to_f32<DT>(vm_s[j][kGroups + g_own]);
            float vh[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) vh[e] = fmaf((float)((bits >> (3 * e)) & 7u), sg, bg);
#pragma unroll
            for (int rr = 0; rr < RB; ++rr) {
                const float p = p_s[rr][j];
#pragma unroll
                for (int e = 0; e < 4; ++e) o[rr][e] = fmaf(p, vh[e], o[rr][e]);
            }
        }
        __syncthreads();
    }

    // ---- epilogue ----
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
        const int gr = rb * RB + rr;
        const float l_tot = wave_sum(lsum[rr]);
        if (gr >= a.G) continue;
        const int h = kvh * a.n_rep + gr / a.L;
        const int i = gr % a.L;
        if (a.S == 1) {
            const float inv = 1.0f / l_tot;
            float y[4] = {o[rr][0] * inv, o[rr][1] * inv, o[rr][2] * inv, o[rr][3] * inv};
            float z[4];
            if (a.rot != nullptr) unrotate4(y, Bm, z);
            else {
                z[0] = y[0]; z[1] = y[1]; z[2] = y[2]; z[3] = y[3];
            }
            float4* dst = reinterpret_cast<float4*>(
                a.out + (((int64_t)b * a.Hkv * a.n_rep + h) * a.L + i) * kHeadDim + lane * 4);
            *dst = make_float4(z[0], z[1], z[2], z[3]);
        } else {
            const int64_t pidx = ((bh * a.n_rb + rb) * a.S + split) * RB + rr;
            *reinterpret_cast<float4*>(a.ws_o + pidx * kHeadDim + lane * 4) =
                make_float4(o[rr][0], o[rr][1], o[rr][2], o[rr][3]);
            if (lane == 0) {
                a.ws_ml[pidx * 2] = m[rr];
                a.ws_ml[pidx * 2 + 1] = l_tot;
            }
        }
    }
}

// Merge the S partials of one query row in split order, normalise, rotate back.
// grid (G, Hkv, B), one wave: lane = channels [4*lane, 4*lane+4).
__global__ __launch_bounds__(64) void attn_combine_kernel(AttnArgs a, int RB) {
    const int lane = threadIdx.x;
    const int gr = blockIdx.x;
    const int kvh = blockIdx.y;
    const int b = blockIdx.z;
    const int rb = gr / RB, rr = gr - rb * RB;
    const int64_t bh = (int64_t)b * a.Hkv + kvh;
    const int64_t base = ((bh * a.n_rb + rb) * a.S) * RB + rr;  // partial of split 0

    float mx = -INFINITY;
    for (int s = 0; s < a.S; ++s) mx = fmaxf(mx, a.ws_ml[(base + (int64_t)s * RB) * 2]);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    float l_tot = 0.f;
    for (int s = 0; s < a.S; ++s) {
        const int64_t p = base + (int64_t)s * RB;
        const float ms = a.ws_ml[p * 2];
        if (ms == -INFINITY) continue;
        const float w = expf(ms - mx);
        l_tot = fmaf(w, a.ws_ml[p * 2 + 1], l_tot);
        const float4 ov = *reinterpret_cast<const float4*>(a.ws_o + p * kHeadDim + lane * 4);
        acc[0] = fmaf(w, ov.x, acc[0]);
        acc[1] = fmaf(w, ov.y, acc[1]);
        acc[2] = fmaf(w, ov.z, acc[2]);
        acc[3] = fmaf(w, ov.w, acc[3]);
    }
    const float inv = 1.0f / l_tot;
    float y[4] = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    float z[4];
    if (a.rot != nullptr) {
        float Bm[16];
        load_block(a.rot, lane, Bm);
        unrotate4(y, Bm, z);
    } else {
        z[0] = y[0]; z[1] = y[1]; z[2] = y[2]; z[3] = y[3];
    }
    const int h = kvh * a.n_rep + gr / a.L;
    const int i = gr % a.L;
    *reinterpret_cast<float4*>(a.out + (((int64_t)b * a.Hkv * a.n_rep + h) * a.L + i) * kHeadDim +
                               lane * 4) = make_float4(z[0], z[1], z[2], z[3]);
}

// ---- launch planning ----

struct Plan {
    int RB, n_rb, S;
    int64_t chunk;
    size_t ws_bytes;
};

int rows_per_block(int G) {
    int rb = 1;
    while (rb < G && rb < 16) rb <<= 1;
    return rb;
}

int make_plan(const rbq_kv_cache* c, int32_t H_q, int32_t L, int32_t splits, Plan* p) {
    int st = check_cache(c);
    if (st != RBQ_OK) return st;
    if (H_q <= 0 || H_q % c->H_kv != 0 || splits < 0) return RBQ_EINVAL;
    if (L < 1 || (int64_t)L > c->offset) return RBQ_ERANGE;
    const int n_rep = H_q / c->H_kv;
    const int64_t G64 = (int64_t)n_rep * L;
    if (G64 > 4096 || c->offset >= ((int64_t)1 << 31)) return RBQ_EUNSUPPORTED;
    const int G = (int)G64;
    p->RB = rows_per_block(G);
    p->n_rb = (G + p->RB - 1) / p->RB;
    const int64_t T = c->offset;
    int64_t S = splits;
    if (S == 0) S = auto_splits(c, H_q, L);
    if (S > T) S = T;
    if (S < 1) S = 1;
    if (S > 65535) return RBQ_EUNSUPPORTED;
    p->S = (int)S;
    p->chunk = (T + S - 1) / S;
    p->ws_bytes = (S == 1) ? 0
                           : (size_t)c->B * c->H_kv * p->n_rb * S * p->RB *
                                                   (kHeadDim + 2) * sizeof(float);
    return RBQ_OK;
}

template <int DT, int RB>
void launch_valu(const AttnArgs& a, dim3 grid, hipStream_t s) {
    hipLaunchKernelGGL((attn_valu_kernel<DT, RB>), grid, dim3(64), 0, s, a);
}

template <int DT>
void launch_valu_rb(int RB, const AttnArgs& a, dim3 grid, hipStream_t s) {
    switch (RB) {
        case 1: launch_valu<DT, 1>(a, grid, s); break;
        case 2: launch_valu<DT, 2>(a, grid, s); break;
        case 4: launch_valu<DT, 4>(a, grid, s); break;
        case 8: launch_valu<DT, 8>(a, grid, s); break;
        default: launch_valu<DT, 16>(a, grid, s); break;
    }
}

}  // namespace

int32_t auto_splits(const rbq_kv_cache* c, int32_t H_q, int32_t L) {
    const int n_rep = H_q / c->H_kv;
    const int G = n_rep * L;
    const int RB = rows_per_block(G);
    const int64_t units = (int64_t)c->B * c->H_kv * ((G + RB - 1) / RB);
    // aim for about 2048 single-wave workgroups, at least 128 keys per split
    int64_t S = (2048 + units - 1) / units;
    const int64_t max_s = (c->offset + 127) / 128;
    if (S > max_s) S = max_s;
    if (S < 1) S = 1;
    return (int32_t)S;
}

}  // namespace rbq

using namespace rbq;

namespace {

bool use_mfma(const rbq_kv_cache* c, int32_t H_q, int32_t L) {
    return (int64_t)(H_q / c->H_kv) * L <= kMfmaMaxRows;
}

// Shared argument checks of the attention entry points.
int check_attn(const rbq_kv_cache* c, int32_t H_q, int32_t L, int32_t splits) {
    int st = check_cache(c);
    if (st != RBQ_OK) return st;
    if (H_q <= 0 || H_q % c->H_kv != 0 || splits < 0) return RBQ_EINVAL;
    if (L < 1 || (int64_t)L > c->offset) return RBQ_ERANGE;
    return RBQ_OK;
}

}  // namespace

extern "C" int32_t rbq_quant_attn_splits(const rbq_kv_cache* c, int32_t H_q, int32_t L) {
    int st = check_attn(c, H_q, L, 0);
    if (st != RBQ_OK) return st;
    if (use_mfma(c, H_q, L)) {
        MfmaPlan mp;
        st = mfma_plan(c, H_q, L, 0, &mp);
        return st != RBQ_OK ? st : mp.S;
    }
    Plan p;
    st = make_plan(c, H_q, L, 0, &p);
    return st != RBQ_OK ? st : p.S;
}

extern "C" size_t rbq_quant_attn_workspace_bytes(const rbq_kv_cache* c, int32_t H_q, int32_t L,
                                                 int32_t splits) {
    if (check_attn(c, H_q, L, splits) != RBQ_OK) return 0;
    if (use_mfma(c, H_q, L)) {
        MfmaPlan mp;
        return mfma_plan(c, H_q, L, splits, &mp) == RBQ_OK ? mp.ws_bytes : 0;
    }
    Plan p;
    if (make_plan(c, H_q, L, splits, &p) != RBQ_OK) return 0;
    return p.ws_bytes;
}

extern "C" int rbq_quant_attn_decode(const rbq_kv_cache* c, const void* q, int32_t H_q, int32_t L,
                                     float scale, int32_t causal, const float* rot_blocks,
                                     float* out, int32_t splits, void* ws, size_t ws_bytes,
                                     void* stream) {
    int st = check_attn(c, H_q, L, splits);
    if (st != RBQ_OK) return st;
    if (q == nullptr || out == nullptr) return RBQ_EINVAL;
    if (use_mfma(c, H_q, L)) {
        MfmaPlan mp;
        st = mfma_plan(c, H_q, L, splits, &mp);
        if (st != RBQ_OK) return st;
        if (mp.ws_bytes > 0 && (ws == nullptr || ws_bytes < mp.ws_bytes)) return RBQ_EWORKSPACE;
        return mfma_launch(c, q, H_q, L, scale, causal, rot_blocks, out, mp, ws, stream);
    }
    Plan p;
    st = make_plan(c, H_q, L, splits, &p);
    if (st != RBQ_OK) return st;
    if (p.ws_bytes > 0 && (ws == nullptr || ws_bytes < p.ws_bytes)) return RBQ_EWORKSPACE;

    AttnArgs a;
    a.q = (const uint16_t*)q;
    a.kw = c->k_words;
    a.ks = (const uint16_t*)c->k_scales;
    a.kb = (const uint16_t*)c->k_biases;
    a.vw = c->v_words;
    a.vs = (const uint16_t*)c->v_scales;
    a.vb = (const uint16_t*)c->v_biases;
    a.rot = rot_blocks;
    a.out = out;
    const size_t n_part = (size_t)c->B * c->H_kv * p.n_rb * p.S * p.RB;
    a.ws_o = p.ws_bytes ? (float*)ws : nullptr;
    a.ws_ml = p.ws_bytes ? a.ws_o + n_part * kHeadDim : nullptr;
    a.capacity = c->capacity;
    a.T = c->offset;
    a.chunk = p.chunk;
    a.Hkv = c->H_kv;
    a.n_rep = H_q / c->H_kv;
    a.L = L;
    a.G = a.n_rep * L;
    a.n_rb = p.n_rb;
    a.S = p.S;
    a.causal = causal ? 1 : 0;
    a.scale = scale;

    hipStream_t s = (hipStream_t)stream;
    const dim3 grid((unsigned)p.S, (unsigned)(c->H_kv * p.n_rb), (unsigned)c->B);
    if (c->dtype == RBQ_BF16) launch_valu_rb<RBQ_BF16>(p.RB, a, grid, s);
    else launch_valu_rb<RBQ_F16>(p.RB, a, grid, s);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && p.S > 1) {
        hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)a.G, (unsigned)c->H_kv,
                                                     (unsigned)c->B),
                           dim3(64), 0, s, a, p.RB);
        e = hipGetLastError();
    }
    if (e != hipSuccess) {
        set_hip_error((int)e);
        return RBQ_EHIP;
    }
    return RBQ_OK;
}
