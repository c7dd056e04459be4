// gemv_ops.h - device pieces of the bandwidth-bound projections (decode
// rows): 16-byte weight loads, activation chunks with the RMSNorm
// statistics, dot products and the cross-wave merge. Used by the GEMV
// kernels and by the single-row projection + attention launch.
#pragma once

#include "common.h"
#include "launch.h"

namespace sttd {

constexpr int CHUNK = 512;  // K elements per wave per step (64 lanes x 8)

// 8 consecutive weights in their storage form.
template <class WT>
struct Raw8;
template <>
struct Raw8<BF16> {
    u32x4 v;
    __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const u32x4*>(p); }
    __device__ __forceinline__ void widen(float* o) const {
        o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xFFFF0000u);
        o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xFFFF0000u);
        o[4] = __uint_as_float(v.z << 16); o[5] = __uint_as_float(v.z & 0xFFFF0000u);
        o[6] = __uint_as_float(v.w << 16); o[7] = __uint_as_float(v.w & 0xFFFF0000u);
    }
};
template <>
struct Raw8<F32> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = *reinterpret_cast<const f32x4*>(p);
        b = *reinterpret_cast<const f32x4*>(p + 4);
    }
    __device__ __forceinline__ void widen(float* o) const {
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
};

// Butterfly reduction of V partial sums per lane (V a power of two, V <= 64).
// The first log2(V) steps exchange halves with a partner lane (partners by
// lane bit 3, 2, 1, 0 through DPP, then bit 4, 5 through permlane swaps): the lane
// whose deciding bit is set keeps the upper half. Remaining steps add plainly.
// On return every lane holds the full sum of value index multi_index<V>(lane).
template <int CTRL>
__device__ __forceinline__ float lane_partner(float v, int off) {
    if (CTRL != 0) return dpp_move<CTRL>(v);
    return off == 16 ? xor16(v) : xor32(v);
}

constexpr int kStepBit[6] = {3, 2, 1, 0, 4, 5};

template <int V>
__device__ __forceinline__ int multi_index(int lane) {
    int idx = 0, width = V;
#pragma unroll
    for (int st = 0; st < 6; ++st) {
        if (width > 1) {
            idx = idx * 2 + ((lane >> kStepBit[st]) & 1);
            width /= 2;
        }
    }
    return idx;
}

// true for one lane per value index (the lanes whose plain-sum bits are zero)
template <int V>
__device__ __forceinline__ bool multi_writer(int lane) {
    int width = V, mask = 0;
#pragma unroll
    for (int st = 0; st < 6; ++st) {
        if (width > 1) width /= 2;
        else mask |= 1 << kStepBit[st];
    }
    return (lane & mask) == 0;
}

template <int V, int ST, int CTRL, int OFF>
__device__ __forceinline__ void butterfly_step(float (&v)[V], int& width, int lane) {
    if (width > 1) {
        const int half = width / 2;
        const bool upper = (lane >> kStepBit[ST]) & 1;
#pragma unroll
        for (int i = 0; i < V / 2; ++i) {
            if (i < half) {
                const float send = upper ? v[i] : v[i + half];
                const float keep = upper ? v[i + half] : v[i];
                v[i] = keep + lane_partner<CTRL>(send, OFF);
            }
        }
        width = half;
    } else {
        v[0] += lane_partner<CTRL>(v[0], OFF);
    }
}

template <int V>
__device__ __forceinline__ float wave_reduce_multi(float (&v)[V]) {
    const int lane = threadIdx.x % WAVE;
    int width = V;
    butterfly_step<V, 0, DPP_ROW_MIRROR, 0>(v, width, lane);
    butterfly_step<V, 1, DPP_ROW_HALF_MIRROR, 0>(v, width, lane);
    butterfly_step<V, 2, DPP_XOR2, 0>(v, width, lane);
    butterfly_step<V, 3, DPP_XOR1, 0>(v, width, lane);
    butterfly_step<V, 4, 0, 16>(v, width, lane);
    butterfly_step<V, 5, 0, 32>(v, width, lane);
    return v[0];
}

// This wave's activation chunks from per-row pointers: xv[c][b][i] = xr[b][k_c + i]
// (* gain when NORM), zero where k_c + i >= K or b >= nb; ss[b] += sum of x^2
// over those elements. xr[b] must be readable for every b (rows past nb repeat a
// valid one).
template <class WT, int KCH, int BT, bool NORM, class MEM = PlainMem>
__device__ __forceinline__ void load_activation_rows(const float* const (&xr)[BT], int nb, int K,
                                                     const typename WT::T* __restrict__ gain, const int (&kk)[KCH],
                                                     float (&xv)[KCH][BT][8], float (&ss)[BT]) {
#pragma unroll
    for (int b = 0; b < BT; ++b) ss[b] = 0.f;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
        const bool in = kk[c] < K;
        const int k = in ? kk[c] : 0;
        float gv[8];
        if (NORM) load8(gain + k, gv, WT());
#pragma unroll
        for (int b = 0; b < BT; ++b) {
            float v[8];
            MEM::ld8(xr[b] + k, v);
            const bool use = in && b < nb;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float xi = use ? v[i] : 0.f;
                ss[b] = fmaf(xi, xi, ss[b]);
                xv[c][b][i] = NORM ? xi * gv[i] : xi;
            }
        }
    }
}

// The same for rows x + b * ldx, b < nb.
template <class WT, int KCH, int BT, bool NORM, class MEM = PlainMem>
__device__ __forceinline__ void load_activations(const float* __restrict__ x, int64_t ldx, int nb, int K,
                                                 const typename WT::T* __restrict__ gain, const int (&kk)[KCH],
                                                 float (&xv)[KCH][BT][8], float (&ss)[BT]) {
    const float* xr[BT];
#pragma unroll
    for (int b = 0; b < BT; ++b) xr[b] = x + (int64_t)(b < nb ? b : 0) * ldx;
    load_activation_rows<WT, KCH, BT, NORM, MEM>(xr, nb, K, gain, kk, xv, ss);
}

// Activation chunks merged from attention split partials (see GemvArgs::xpart):
// per 8-element chunk (8 divides head_dim) every split's (m, l, o[8]) is loaded
// first, up to kMergeMaxSplits of them, so the loads overlap; then
// o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s with M the largest m_s.
template <int KCH, int BT, class MEM = PlainMem>
__device__ __forceinline__ void load_activations_merged(const GemvArgs& a, int b0, int nb, const int (&kk)[KCH],
                                                        float (&xv)[KCH][BT][8]) {
    constexpr int MS = kMergeMaxSplits;
    const int n_heads = a.K / a.head_dim;
    const int rec = a.head_dim + 4;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
        const bool in = kk[c] < a.K;
        const int k = in ? kk[c] : 0;
        const int h = k / a.head_dim, e0 = k % a.head_dim;
#pragma unroll
        for (int b = 0; b < BT; ++b) {
            const bool use = in && b < nb;
            const float* pr = a.xpart + ((int64_t)((b0 + (b < nb ? b : 0)) * n_heads + h) * a.n_splits) * rec;
            float ms[MS], ls[MS], os[MS][8];
#pragma unroll
            for (int sp = 0; sp < MS; ++sp) {
                const float* p = pr + (int64_t)(sp < a.n_splits ? sp : 0) * rec;
                ms[sp] = MEM::ld(p);
                ls[sp] = MEM::ld(p + 1);
                MEM::ld8(p + 4 + e0, os[sp]);
            }
            float M = -INFINITY;
#pragma unroll
            for (int sp = 0; sp < MS; ++sp)
                if (sp < a.n_splits) M = fmaxf(M, ms[sp]);
            float L = 0.f, O[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) O[i] = 0.f;
#pragma unroll
            for (int sp = 0; sp < MS; ++sp) {
                const float w = (sp < a.n_splits && M != -INFINITY) ? exp2f(ms[sp] - M) : 0.f;
                L = fmaf(w, ls[sp], L);
#pragma unroll
                for (int i = 0; i < 8; ++i) O[i] = fmaf(w, os[sp][i], O[i]);
            }
            const float inv = L > 0.f ? 1.0f / L : 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) xv[c][b][i] = use ? O[i] * inv : 0.f;
        }
    }
}

// Dot products of the loaded weight chunks with the activation chunks.
template <class WT, int KCH, int NR, int BT>
__device__ __forceinline__ void chunk_dots(const Raw8<WT> (&w)[KCH][NR], const float (&xv)[KCH][BT][8],
                                           float (&acc)[NR * BT]) {
#pragma unroll
    for (int i = 0; i < NR * BT; ++i) acc[i] = 0.f;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            float wf[8];
            w[c][r].widen(wf);
#pragma unroll
            for (int b = 0; b < BT; ++b)
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[r * BT + b] = fmaf(wf[i], xv[c][b][i], acc[r * BT + b]);
        }
    }
}

// Merge the waves: on return dot holds the full sum of value index t = r*BT + b
// for threads t < NR*BT, and rs[b] the row scale (1 when !NORM), in every thread.
template <int V, int BT, bool NORM>
__device__ __forceinline__ void block_merge(float (&acc)[V], float (&ss)[BT], float (*red)[V + BT], int K, float eps,
                                            float& dot, float (&rs)[BT]) {
    const int lane = threadIdx.x % WAVE, wave = threadIdx.x / WAVE;
    const float s = wave_reduce_multi<V>(acc);
    if (multi_writer<V>(lane)) red[wave][multi_index<V>(lane)] = s;
    if (NORM) {
#pragma unroll
        for (int b = 0; b < BT; ++b) {
            const float t = wave_sum(ss[b]);
            if (lane == 0) red[wave][V + b] = t;
        }
    }
    __syncthreads();
    const int t = threadIdx.x;
    dot = t < V ? red[0][t] + red[1][t] + red[2][t] + red[3][t] : 0.f;
#pragma unroll
    for (int b = 0; b < BT; ++b)
        rs[b] = NORM ? 1.0f / sqrtf((red[0][V + b] + red[1][V + b] + red[2][V + b] + red[3][V + b]) / (float)K + eps)
                     : 1.f;
}

}  // namespace sttd
