// kernels_gemv.hip - bandwidth-bound projections for decode rows (and the
// fp32-weight path): y = x W^T over a few activation rows, with the block's
// RMSNorm fused in front and residual / SwiGLU / argmax fused behind.
//
// Layout: W is [N, K] row-major (bf16 or fp32). A wave owns RW output rows
// (SwiGLU: RW gate rows and the RW matching up rows); each lane streams
// 8 consecutive K elements per 512-wide chunk with 16-byte loads, so a wave
// reads 1 KB (bf16) of a row per instruction, fully coalesced. Activations
// are fp32 and stay fp32: products are exact, accumulation is fp32. A
// workgroup of 4 waves serves BT activation rows; more rows tile blockIdx.y.
#include "common.h"
#include "launch.h"

namespace sttd {

template <class WT, int BT>
__device__ __forceinline__ void row_scales(const float* __restrict__ x, int64_t ldx, int nb, int K, float eps,
                                           float* rs /*[BT]*/) {
    __shared__ float red[4][BT];
    const int lane = threadIdx.x % WAVE, wave = threadIdx.x / WAVE;
    float ss[BT];
#pragma unroll
    for (int b = 0; b < BT; ++b) {
        ss[b] = 0.f;
        if (b < nb) {
            const float* xr = x + b * ldx;
            for (int i = threadIdx.x * 4; i < K; i += 1024) {
                float4 v = *reinterpret_cast<const float4*>(xr + i);
                ss[b] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
            }
        }
        ss[b] = wave_sum(ss[b]);
    }
    if (lane == 0) {
#pragma unroll
        for (int b = 0; b < BT; ++b) red[wave][b] = ss[b];
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < BT; ++b) rs[b] = 1.0f / sqrtf((red[0][b] + red[1][b] + red[2][b] + red[3][b]) / (float)K + eps);
}

// Dot products of NR weight rows with BT activation rows, one wave; results
// are complete (wave-reduced) in every lane.
template <class WT, int NR, int BT, bool NORM>
__device__ __forceinline__ void wave_dots(const typename WT::T* const* wr, const bool* valid,
                                          const float* __restrict__ x, int64_t ldx, int nb, int K,
                                          const typename WT::T* __restrict__ gain, float (&acc)[NR][BT]) {
    const int lane = threadIdx.x % WAVE;
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int b = 0; b < BT; ++b) acc[r][b] = 0.f;
#pragma unroll 2
    for (int k = lane * 8; k < K; k += 512) {
        float wv[NR][8];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            if (valid[r]) load8(wr[r] + k, wv[r], WT());
            else {
#pragma unroll
                for (int i = 0; i < 8; ++i) wv[r][i] = 0.f;
            }
        }
        float gv[8];
        if (NORM) load8(gain + k, gv, WT());
#pragma unroll
        for (int b = 0; b < BT; ++b) {
            if (b < nb) {
                float xv[8];
                load8(x + b * ldx + k, xv, F32());
                if (NORM) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) xv[i] *= gv[i];
                }
#pragma unroll
                for (int r = 0; r < NR; ++r)
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[r][b] = fmaf(wv[r][i], xv[i], acc[r][b]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int b = 0; b < BT; ++b) acc[r][b] = wave_sum(acc[r][b]);
}

template <class WT, int EPI, int BT, int RW, bool NORM>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
    typedef typename WT::T T;
    constexpr int NR = EPI == GEMV_SWIGLU ? 2 * RW : RW;
    const int lane = threadIdx.x % WAVE, wave = threadIdx.x / WAVE;
    const int b0 = blockIdx.y * BT;
    const int nb = min(BT, a.rows - b0);
    const float* x = a.x + (int64_t)b0 * a.ldx;

    float rs[BT];
    if (NORM) row_scales<WT, BT>(x, a.ldx, nb, a.K, a.eps, rs);
    else {
#pragma unroll
        for (int b = 0; b < BT; ++b) rs[b] = 1.f;
    }

    const int n0 = (blockIdx.x * 4 + wave) * RW;  // first output column of this wave
    if (n0 >= a.N) return;
    const T* wr[NR];
    bool valid[NR];
    if (EPI == GEMV_SWIGLU) {
        const T* W = (const T*)a.w[0];
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            valid[r] = valid[RW + r] = (n0 + r) < a.N;
            wr[r] = W + (int64_t)(n0 + r) * a.K;
            wr[RW + r] = W + (int64_t)(n0 + r + a.N) * a.K;
        }
    } else {
        const bool s2 = n0 >= a.seg_end[1], s1 = n0 >= a.seg_end[0];
        const int start = s2 ? a.seg_end[1] : (s1 ? a.seg_end[0] : 0);
        const T* W = (const T*)(s2 ? a.w[2] : (s1 ? a.w[1] : a.w[0]));
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            valid[r] = (n0 + r) < a.N;
            wr[r] = W + (int64_t)(n0 + r - start) * a.K;
        }
    }

    float acc[NR][BT];
    wave_dots<WT, NR, BT, NORM>(wr, valid, x, a.ldx, nb, a.K, (const T*)a.gain, acc);

    // epilogue: lane (r * BT + b) writes output (b, n0 + r)
#pragma unroll
    for (int r = 0; r < RW; ++r) {
#pragma unroll
        for (int b = 0; b < BT; ++b) {
            if (lane != r * BT + b || b >= nb || !valid[r]) continue;
            const int64_t row = b0 + b;
            const int n = n0 + r;
            float v = acc[r][b] * rs[b];
            if (EPI == GEMV_SWIGLU) {
                const float u = acc[RW + r][b] * rs[b];
                v = v / (1.0f + expf(-v)) * u;
            } else if (EPI == GEMV_RESID) {
                v += a.resid[row * a.ldr + n];
            }
            a.y[row * a.ldy + n] = v;
        }
    }
}

template <class WT, int EPI, int RW, bool NORM>
static void launch_bt(const GemvArgs& a, hipStream_t s) {
    const int waves = (a.N + RW - 1) / RW;
    dim3 grid((waves + 3) / 4, 1);
    if (a.rows == 1) {
        gemv_kernel<WT, EPI, 1, RW, NORM><<<grid, 256, 0, s>>>(a);
    } else if (a.rows == 2) {
        gemv_kernel<WT, EPI, 2, RW, NORM><<<grid, 256, 0, s>>>(a);
    } else {
        grid.y = (a.rows + 3) / 4;
        gemv_kernel<WT, EPI, 4, RW, NORM><<<grid, 256, 0, s>>>(a);
    }
}

template <class WT>
static void launch_wt(const GemvArgs& a, GemvEpi epi, hipStream_t s) {
    const bool norm = a.gain != nullptr;
    if (epi == GEMV_SWIGLU) {
        if (norm) launch_bt<WT, GEMV_SWIGLU, 1, true>(a, s);
        else launch_bt<WT, GEMV_SWIGLU, 1, false>(a, s);
    } else if (epi == GEMV_RESID) {
        if (norm) launch_bt<WT, GEMV_RESID, 2, true>(a, s);
        else launch_bt<WT, GEMV_RESID, 2, false>(a, s);
    } else {
        if (norm) launch_bt<WT, GEMV_STORE, 2, true>(a, s);
        else launch_bt<WT, GEMV_STORE, 2, false>(a, s);
    }
}

hipError_t launch_gemv(const GemvArgs& a, WType wt, GemvEpi epi, hipStream_t s) {
    if (a.rows <= 0 || a.N <= 0) return hipSuccess;
    if (wt == W_BF16) launch_wt<BF16>(a, epi, s);
    else launch_wt<F32>(a, epi, s);
    return hipGetLastError();
}

// ------------------------------------------------------------------ lm_head + argmax
// Final RMSNorm and the tied head (build_step_graph on the Qwen3-ASR decoder
// page: logits = E * (RMSNorm(x) * g), then argmax on device). Each wave scores
// RW vocabulary rows; the workgroup's best (logit, index) per activation row is
// folded into a 64-bit slot with one atomic max, the key being
// (order-preserving bits of the logit) << 32 | ~index, so the largest logit
// wins and, among equal logits, the lowest index (the strict greater-than scan
// of run() on the model page). The last workgroup to finish (atomic counter)
// reads the slots, writes the ids, gathers the next input rows E[id], bumps the
// positions and re-zeroes slots and counter for the next call.
template <class WT, int BT, int RW>
__global__ __launch_bounds__(256) void lm_head_kernel(HeadArgs a) {
    typedef typename WT::T T;
    __shared__ unsigned long long best_lds[4][BT];
    __shared__ int last_lds;
    const int lane = threadIdx.x % WAVE, wave = threadIdx.x / WAVE;
    const int b0 = blockIdx.y * BT;
    const int nb = min(BT, a.rows - b0);
    const float* x = a.x + (int64_t)b0 * a.ldx;
    float rs[BT];
    row_scales<WT, BT>(x, a.ldx, nb, a.hidden, a.eps, rs);

    const int n0 = (blockIdx.x * 4 + wave) * RW;
    const T* E = (const T*)a.embed;
    const T* wr[RW];
    bool valid[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        valid[r] = (n0 + r) < a.vocab;
        wr[r] = E + (int64_t)(valid[r] ? n0 + r : 0) * a.hidden;
    }
    float acc[RW][BT];
    wave_dots<WT, RW, BT, true>(wr, valid, x, a.ldx, nb, a.hidden, (const T*)a.gain, acc);

    unsigned long long best[BT];
#pragma unroll
    for (int b = 0; b < BT; ++b) {
        best[b] = 0ull;
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            if (!valid[r]) continue;
            const float v = acc[r][b] * rs[b];
            const unsigned long long key =
                ((unsigned long long)float_order_key(v) << 32) | (unsigned long long)(~(uint32_t)(n0 + r));
            best[b] = key > best[b] ? key : best[b];
            if (a.logits && b < nb && lane == r) a.logits[(int64_t)(b0 + b) * a.vocab + n0 + r] = v;
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int b = 0; b < BT; ++b) best_lds[wave][b] = best[b];
    }
    __syncthreads();
    if (threadIdx.x < BT && threadIdx.x < nb) {
        const int b = threadIdx.x;
        unsigned long long m = best_lds[0][b];
        for (int w = 1; w < 4; ++w) m = best_lds[w][b] > m ? best_lds[w][b] : m;
        atomicMax(&a.slots[b0 + b], m);
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = atomicAdd(&a.counters[blockIdx.y], 1u);
        last_lds = prev == gridDim.x - 1;
    }
    __syncthreads();
    if (!last_lds) return;
    __threadfence();
    __shared__ int ids_lds[BT];
    if (threadIdx.x < nb) {
        const int b = threadIdx.x;
        const unsigned long long key =
            __hip_atomic_load(&a.slots[b0 + b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int id = (int)(~(uint32_t)(key & 0xFFFFFFFFull));
        ids_lds[b] = id;
        a.ids[b0 + b] = id;
        if (a.pos) a.pos[b0 + b] += 1;
        a.slots[b0 + b] = 0ull;
    }
    if (threadIdx.x == 0) a.counters[blockIdx.y] = 0u;
    __syncthreads();
    if (a.next_x) {
        for (int b = 0; b < nb; ++b) {
            const int id = ids_lds[b];
            const bool ok = id >= 0 && id < a.vocab;
            if (!ok && threadIdx.x == 0) record_error(a.err, 4u);
            float* xr = a.next_x + (int64_t)(b0 + b) * a.hidden;
            for (int i = threadIdx.x; i < a.hidden; i += 256) xr[i] = ok ? WT::ld(E, (int64_t)id * a.hidden + i) : 0.f;
        }
    }
}

hipError_t launch_lm_head_argmax(const HeadArgs& a, WType wt, hipStream_t s) {
    if (a.rows <= 0) return hipSuccess;
    constexpr int RW = 2;
    const int waves = (a.vocab + RW - 1) / RW;
    dim3 grid((waves + 3) / 4, 1);
#define HEAD_LAUNCH(WT_)                                                    \
    do {                                                                    \
        if (a.rows == 1) lm_head_kernel<WT_, 1, RW><<<grid, 256, 0, s>>>(a); \
        else if (a.rows == 2) lm_head_kernel<WT_, 2, RW><<<grid, 256, 0, s>>>(a); \
        else {                                                              \
            grid.y = (a.rows + 3) / 4;                                      \
            lm_head_kernel<WT_, 4, RW><<<grid, 256, 0, s>>>(a);             \
        }                                                                   \
    } while (0)
    if (wt == W_BF16) HEAD_LAUNCH(BF16);
    else HEAD_LAUNCH(F32);
#undef HEAD_LAUNCH
    return hipGetLastError();
}

}  // namespace sttd
