// kernels_attn.hip - causal grouped-query attention over the KV cache.
//
// Both kernels compute, for query head h of a row at position p,
//   o_h = sum_c softmax_c(q_h . K[c]_j / sqrt(d)) V[c]_j,  c = 0..p,
// with j = floor(h / (n_heads / n_kv)) the head's KV group (Qwen3-ASR decoder
// page, file header; the causal mask of run() on the model page keeps
// columns c <= r). Masked columns are never read, so no mask tensor exists.
// Exponentials run in base 2 on scores pre-scaled by log2(e)/sqrt(d).
#include "common.h"
#include "launch.h"

namespace sttd {

// ------------------------------------------------------------------ split-K rows
// Grid (row, kv head, split). The split's share of cache rows [0, p] is
// ceil((p + 1) / n_splits) rows, so the work follows the actual position even
// though the grid is sized from a host bound. Within a workgroup, groups of
// LPK = d/8 lanes read one cache row (16 bytes per lane for f16, coalesced)
// and keep a running (max, sum, output) per query head of the group; the
// groups then merge through LDS and the workgroup writes one partial
// (m, l, o[d]) per query head. attn_combine merges the splits.
template <class KT, int D, int G>
__global__ __launch_bounds__(256) void attn_rows_kernel(const float* __restrict__ q, int64_t ldq, int n_heads,
                                                        RowMap rm, KVLayer kv, int n_splits, float* __restrict__ part,
                                                        uint32_t* err) {
    typedef typename KT::T T;
    constexpr int LPK = D / 8;            // lanes per cache row
    constexpr int GROUPS = 256 / LPK;     // cache rows in flight per step
    __shared__ float m_lds[GROUPS][G], l_lds[GROUPS][G];
    __shared__ float o_lds[GROUPS][G][D + 1];

    const int r = blockIdx.x, j = blockIdx.y, split = blockIdx.z;
    const int tid = threadIdx.x;
    const int grp = tid / LPK, sub = tid % LPK;
    const int pos = row_pos(rm, r);
    const int seq = row_seq(rm, r);
    const bool ok = pos >= 0 && pos < kv.n_ctx && seq >= 0 && seq < kv.n_seq;
    if (!ok && tid == 0 && split == 0 && j == 0) record_error(err, pos < 0 || pos >= kv.n_ctx ? 1u : 2u);
    const int n_keys = ok ? pos + 1 : 0;
    const int chunk = (n_keys + n_splits - 1) / n_splits;
    const int c0 = split * chunk;
    const int c1 = min(c0 + chunk, n_keys);

    const float scale = 1.4426950408889634f / sqrtf((float)D);
    float qv[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float* qh = q + (int64_t)r * ldq + (j * G + g) * D + sub * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) qv[g][i] = qh[i] * scale;
    }
    float m[G], l[G], o[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[g][i] = 0.f;
    }
    const int64_t slab = ((int64_t)(ok ? seq : 0) * kv.n_kv + j) * kv.n_ctx * D;
    const T* Kp = (const T*)kv.k + slab + sub * 8;
    const T* Vp = (const T*)kv.v + slab + sub * 8;
    for (int c = c0 + grp; c < c1; c += GROUPS) {
        float kr[8], vr[8];
        load8(Kp + (int64_t)c * D, kr, KT());
        load8(Vp + (int64_t)c * D, vr, KT());
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) s = fmaf(qv[g][i], kr[i], s);
#pragma unroll
            for (int off = LPK / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, WAVE);
            const float mn = fmaxf(m[g], s);
            const float alpha = exp2f(m[g] - mn);
            const float p = exp2f(s - mn);
            l[g] = l[g] * alpha + p;
#pragma unroll
            for (int i = 0; i < 8; ++i) o[g][i] = fmaf(o[g][i], alpha, p * vr[i]);
            m[g] = mn;
        }
    }
    // merge the groups
    if (sub == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            m_lds[grp][g] = m[g];
            l_lds[grp][g] = l[g];
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < 8; ++i) o_lds[grp][g][sub * 8 + i] = o[g][i];
    __syncthreads();
    // thread t < G*D: head g = t / D, element e = t % D
    for (int t = tid; t < G * D; t += 256) {
        const int g = t / D, e = t % D;
        float M = -INFINITY;
        for (int k = 0; k < GROUPS; ++k) M = fmaxf(M, m_lds[k][g]);
        float L = 0.f, O = 0.f;
        if (M != -INFINITY) {
            for (int k = 0; k < GROUPS; ++k) {
                const float w = exp2f(m_lds[k][g] - M);
                L += w * l_lds[k][g];
                O += w * o_lds[k][g][e];
            }
        }
        float* pp = part + (((int64_t)r * n_heads + j * G + g) * n_splits + split) * (D + 2);
        if (e == 0) {
            pp[0] = M;
            pp[1] = L;
        }
        pp[2 + e] = O;
    }
}

// Merge the splits of each (row, query head): o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
template <int D>
__global__ __launch_bounds__(D) void attn_combine_kernel(const float* __restrict__ part, int n_heads, int n_splits,
                                                         float* __restrict__ out_f32, uint16_t* __restrict__ out_bf16,
                                                         uint16_t* __restrict__ out_lo, int64_t ldo) {
    const int r = blockIdx.x, h = blockIdx.y, e = threadIdx.x;
    const float* pp = part + ((int64_t)r * n_heads + h) * n_splits * (D + 2);
    float M = -INFINITY;
    for (int s = 0; s < n_splits; ++s) M = fmaxf(M, pp[s * (D + 2)]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
        for (int s = 0; s < n_splits; ++s) {
            const float w = exp2f(pp[s * (D + 2)] - M);
            L += w * pp[s * (D + 2) + 1];
            O += w * pp[s * (D + 2) + 2 + e];
        }
    }
    const float v = L > 0.f ? O / L : 0.f;
    const int64_t idx = (int64_t)r * ldo + h * D + e;
    if (out_f32) {
        out_f32[idx] = v;
    } else {
        uint16_t hi, lo;
        split_bf16(v, hi, lo);
        out_bf16[idx] = hi;
        if (out_lo) out_lo[idx] = lo;
    }
}

template <class KT, int D>
static void rows_dispatch_g(const float* q, int64_t ldq, int R, int n_heads, RowMap rm, KVLayer kv, int n_splits,
                            float* part, uint32_t* err, hipStream_t s) {
    const int G = n_heads / kv.n_kv;
    dim3 grid(R, kv.n_kv, n_splits);
    switch (G) {
        case 1: attn_rows_kernel<KT, D, 1><<<grid, 256, 0, s>>>(q, ldq, n_heads, rm, kv, n_splits, part, err); break;
        case 2: attn_rows_kernel<KT, D, 2><<<grid, 256, 0, s>>>(q, ldq, n_heads, rm, kv, n_splits, part, err); break;
        case 4: attn_rows_kernel<KT, D, 4><<<grid, 256, 0, s>>>(q, ldq, n_heads, rm, kv, n_splits, part, err); break;
        case 8: attn_rows_kernel<KT, D, 8><<<grid, 256, 0, s>>>(q, ldq, n_heads, rm, kv, n_splits, part, err); break;
        default: break;
    }
}

hipError_t launch_attn_rows(const float* q, int64_t ldq, int R, int n_heads, RowMap rm, KVLayer kv, int n_splits,
                            float* part, float* out_f32, uint16_t* out_bf16, uint16_t* out_bf16_lo, int64_t ldo,
                            uint32_t* err, hipStream_t s) {
    if (R <= 0) return hipSuccess;
    const int G = n_heads / kv.n_kv;
    if (G != 1 && G != 2 && G != 4 && G != 8) return hipErrorInvalidValue;
    if (kv.d == 128) {
        if (kv.type == KV_F16) rows_dispatch_g<F16, 128>(q, ldq, R, n_heads, rm, kv, n_splits, part, err, s);
        else rows_dispatch_g<F32, 128>(q, ldq, R, n_heads, rm, kv, n_splits, part, err, s);
        attn_combine_kernel<128><<<dim3(R, n_heads), 128, 0, s>>>(part, n_heads, n_splits, out_f32, out_bf16, out_bf16_lo, ldo);
    } else if (kv.d == 64) {
        if (kv.type == KV_F16) rows_dispatch_g<F16, 64>(q, ldq, R, n_heads, rm, kv, n_splits, part, err, s);
        else rows_dispatch_g<F32, 64>(q, ldq, R, n_heads, rm, kv, n_splits, part, err, s);
        attn_combine_kernel<64><<<dim3(R, n_heads), 64, 0, s>>>(part, n_heads, n_splits, out_f32, out_bf16, out_bf16_lo, ldo);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------ causal flash prefill (MFMA, f16 cache)
// Grid (query tile of 64 rows, query head). Each wave owns 16 query rows; the
// workgroup walks the cache in blocks of 64 keys up to the tile's last
// position. Per block: K [64 x D] and V transposed [D x 64] are staged in LDS;
// S = Q K^T with v_mfma_f32_16x16x32_f16 (Q fragments live in registers);
// online softmax per row (row max and sum across the 16 lanes sharing the
// row's 4-lane slot); P (f16) goes through a per-wave LDS tile into the A
// layout; O += P V with the same MFMA. Output rows are rounded to bf16 for the
// O-projection GEMM.
template <int D>
__global__ __launch_bounds__(256) void attn_prefill_kernel(const uint16_t* __restrict__ q16, int64_t ldq, int T,
                                                           int pos0, int seq, int n_heads, KVLayer kv,
                                                           uint16_t* __restrict__ out, uint16_t* __restrict__ out_lo,
                                                           int64_t ldo) {
    constexpr int KB = 64;                 // keys per block
    constexpr int KS = D + 8;              // K row stride in LDS (f16)
    constexpr int VS = KB + 8;             // V^T row stride in LDS
    constexpr int PS = KB + 8;             // P row stride
    __shared__ __attribute__((aligned(16))) uint16_t Ks[KB * KS];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VS];
    __shared__ __attribute__((aligned(16))) uint16_t Ps[4][16 * PS];

    const int tile = gridDim.x - 1 - blockIdx.x;  // heavy (late) tiles first
    const int h = blockIdx.y;
    const int j = h / (n_heads / kv.n_kv);
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int t0 = tile * 64 + wave * 16;         // this wave's first row
    const int64_t slab = ((int64_t)seq * kv.n_kv + j) * kv.n_ctx * D;
    const uint16_t* Kg = (const uint16_t*)kv.k + slab;
    const uint16_t* Vg = (const uint16_t*)kv.v + slab;

    // Q fragments: row t0 + lane%16, K elements ks*32 + (lane/16)*8 ..
    f16x8 qf[D / 32];
    {
        const int t = t0 + lane % 16;
        const bool ok = t < T;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            const uint16_t* src = q16 + (int64_t)(ok ? t : 0) * ldq + h * D + ks * 32 + (lane / 16) * 8;
            u32x4 u = ok ? *reinterpret_cast<const u32x4*>(src) : u32x4{0u, 0u, 0u, 0u};
            qf[ks] = __builtin_bit_cast(f16x8, u);
        }
    }
    const float sl2 = 1.4426950408889634f / sqrtf((float)D);
    float m_i[4], l_i[4];
    f32x4 o[D / 16];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        m_i[rr] = -INFINITY;
        l_i[rr] = 0.f;
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int tile_last = min(tile * 64 + 63, T - 1);
    const int n_keys = pos0 + tile_last + 1;       // keys any row of the tile can see
    const int n_blocks = (n_keys + KB - 1) / KB;
    for (int kb = 0; kb < n_blocks; ++kb) {
        const int c0 = kb * KB;
        __syncthreads();
        // stage K rows and V^T (rows beyond n_keys are zero; they are masked anyway)
        for (int v = tid; v < KB * D / 8; v += 256) {
            const int c = v / (D / 8), e = (v % (D / 8)) * 8;
            u32x4 ku = u32x4{0u, 0u, 0u, 0u}, vu = u32x4{0u, 0u, 0u, 0u};
            if (c0 + c < n_keys) {
                ku = *reinterpret_cast<const u32x4*>(Kg + (int64_t)(c0 + c) * D + e);
                vu = *reinterpret_cast<const u32x4*>(Vg + (int64_t)(c0 + c) * D + e);
            }
            *reinterpret_cast<u32x4*>(&Ks[c * KS + e]) = ku;
#pragma unroll
            for (int i = 0; i < 8; ++i) Vt[(e + i) * VS + c] = (uint16_t)(vu[i / 2] >> (16 * (i % 2)));
        }
        __syncthreads();
        // S = Q K^T for 4 key tiles of 16
        f32x4 s[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            s[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                const f16x8 kf =
                    *reinterpret_cast<const f16x8*>(&Ks[(nt * 16 + lane % 16) * KS + ks * 32 + (lane / 16) * 8]);
                s[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qf[ks], kf, s[nt], 0, 0, 0);
            }
        }
        // mask, online softmax; lane holds rows (lane/16)*4 + rr, keys nt*16 + lane%16
        float p[4][4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int t = t0 + (lane / 16) * 4 + rr;
            const int pmax = pos0 + t;  // last visible key of this row
            float mx = -INFINITY;
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int c = c0 + nt * 16 + lane % 16;
                float v = s[nt][rr] * sl2;
                if (c > pmax) v = -INFINITY;
                p[nt][rr] = v;
                mx = fmaxf(mx, v);
            }
#pragma unroll
            for (int off = 8; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, WAVE));
            const float mn = fmaxf(m_i[rr], mx);
            const float alpha = mn == -INFINITY ? 1.f : exp2f(m_i[rr] - mn);
            float rs = 0.f;
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const float e = mn == -INFINITY ? 0.f : exp2f(p[nt][rr] - mn);
                p[nt][rr] = e;
                rs += e;
            }
            l_i[rr] = l_i[rr] * alpha + rs;
            m_i[rr] = mn;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) o[dt][rr] *= alpha;
        }
        // P -> LDS (row-major [16][64]) -> A fragments
        uint16_t* P = Ps[wave];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
                P[((lane / 16) * 4 + rr) * PS + nt * 16 + lane % 16] = f32_to_f16_bits(p[nt][rr]);
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): LDS writes done before the reads below
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int ks = 0; ks < KB / 32; ++ks) {
            const f16x8 pf = *reinterpret_cast<const f16x8*>(&P[(lane % 16) * PS + ks * 32 + (lane / 16) * 8]);
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                const f16x8 vf =
                    *reinterpret_cast<const f16x8*>(&Vt[(dt * 16 + lane % 16) * VS + ks * 32 + (lane / 16) * 8]);
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf, vf, o[dt], 0, 0, 0);
            }
        }
    }
    // finish rows: the row sum is spread over the 16 lanes sharing (lane/16)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        float lsum = l_i[rr];
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off, WAVE);
        const int t = t0 + (lane / 16) * 4 + rr;
        if (t >= T) continue;
        const float inv = 1.0f / lsum;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            uint16_t hi, lo;
            split_bf16(o[dt][rr] * inv, hi, lo);
            const int64_t idx = (int64_t)t * ldo + h * D + dt * 16 + lane % 16;
            out[idx] = hi;
            if (out_lo) out_lo[idx] = lo;
        }
    }
}

hipError_t launch_attn_prefill(const uint16_t* q16, int64_t ldq, int T, int pos0, int seq, int n_heads, KVLayer kv,
                               uint16_t* out_bf16, uint16_t* out_bf16_lo, int64_t ldo, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    dim3 grid((T + 63) / 64, n_heads);
    if (kv.d == 128)
        attn_prefill_kernel<128><<<grid, 256, 0, s>>>(q16, ldq, T, pos0, seq, n_heads, kv, out_bf16, out_bf16_lo, ldo);
    else if (kv.d == 64)
        attn_prefill_kernel<64><<<grid, 256, 0, s>>>(q16, ldq, T, pos0, seq, n_heads, kv, out_bf16, out_bf16_lo, ldo);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace sttd
