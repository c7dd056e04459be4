// kernels_misc.hip - RMSNorm rows, per-head Q/K RMSNorm + NeoX RoPE + KV write,
// token-embedding gather, fills.
#include "common.h"
#include "launch.h"

namespace sttd {

// ------------------------------------------------------------------ RMSNorm rows
// Pre-LN RMSNorm of the block (Qwen3-ASR decoder page, file header; the
// final norm of build_prefill_graph has the same form): one workgroup per row,
// the mean square reduced over waves, output rounded to bf16 for the MFMA GEMM.
template <class GT>
__global__ __launch_bounds__(256) void rmsnorm_rows_bf16_kernel(const float* __restrict__ x, int64_t ldx,
                                                                const typename GT::T* __restrict__ g,
                                                                uint16_t* __restrict__ out,
                                                                uint16_t* __restrict__ out_lo, int64_t ldo, int H,
                                                                float eps) {
    __shared__ float red[4];
    const float* xr = x + (int64_t)blockIdx.x * ldx;
    uint16_t* o = out + (int64_t)blockIdx.x * ldo;
    float ss = 0.f;
    for (int i = threadIdx.x * 4; i < H; i += 1024) {
        float4 v = *reinterpret_cast<const float4*>(xr + i);
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = block_sum<4>(ss, red);
    const float rs = 1.0f / sqrtf(ss / (float)H + eps);
    for (int i = threadIdx.x * 4; i < H; i += 1024) {
        float4 v = *reinterpret_cast<const float4*>(xr + i);
        const float a0 = v.x * rs * GT::ld(g, i), a1 = v.y * rs * GT::ld(g, i + 1);
        const float a2 = v.z * rs * GT::ld(g, i + 2), a3 = v.w * rs * GT::ld(g, i + 3);
        uint16_t h0, h1, h2, h3, l0, l1, l2, l3;
        split_bf16(a0, h0, l0);
        split_bf16(a1, h1, l1);
        split_bf16(a2, h2, l2);
        split_bf16(a3, h3, l3);
        uint2 pk;
        pk.x = (uint32_t)h0 | ((uint32_t)h1 << 16);
        pk.y = (uint32_t)h2 | ((uint32_t)h3 << 16);
        *reinterpret_cast<uint2*>(o + i) = pk;
        if (out_lo) {
            pk.x = (uint32_t)l0 | ((uint32_t)l1 << 16);
            pk.y = (uint32_t)l2 | ((uint32_t)l3 << 16);
            *reinterpret_cast<uint2*>(out_lo + (int64_t)blockIdx.x * ldo + i) = pk;
        }
    }
}

hipError_t launch_rmsnorm_rows_bf16(const float* x, int64_t ldx, const void* gain, WType gt, uint16_t* out,
                                    uint16_t* out_lo, int64_t ldo, int R, int H, float eps, hipStream_t s) {
    if (R <= 0) return hipSuccess;
    if (gt == W_BF16)
        rmsnorm_rows_bf16_kernel<BF16><<<R, 256, 0, s>>>(x, ldx, (const uint16_t*)gain, out, out_lo, ldo, H, eps);
    else
        rmsnorm_rows_bf16_kernel<F32><<<R, 256, 0, s>>>(x, ldx, (const float*)gain, out, out_lo, ldo, H, eps);
    return hipGetLastError();
}

// ------------------------------------------------------------------ Q/K norm + RoPE + KV write
// One wave per (row, head item); items are the n_heads query heads, then the
// n_kv key heads, then the n_kv value heads. Lane i < d/2 owns the NeoX pair
// (i, i + d/2). Query and key heads: RMSNorm over head_dim with the shared
// gain, then the pair turns by the table angle pos * theta^(-2i/d). Keys and
// values go to cache row `pos` of the row's slab; values are copied as is.
// (Qwen3-ASR decoder page, file header; the cache index equals the position:
// build_step_graph's kv_idx and run() on the model page.)
template <class GT, class KT>
__global__ __launch_bounds__(256) void qk_norm_rope_kv_kernel(
    const float* __restrict__ qkv, int64_t ldqkv, int R, int n_heads, int n_kv, int d,
    const typename GT::T* __restrict__ qg, const typename GT::T* __restrict__ kg, float eps,
    const float* __restrict__ rope, int max_pos, RowMap rm, KVLayer kv, void* __restrict__ q_out, bool q_f16,
    int64_t ldq, uint32_t* err) {
    const int lane = threadIdx.x % WAVE;
    const int items = n_heads + 2 * n_kv;
    const int item = blockIdx.x * 4 + threadIdx.x / WAVE;
    if (item >= R * items) return;
    const int r = item / items, hi = item % items;
    const int half = d / 2;
    const int pos = row_pos(rm, r);
    const int seq = row_seq(rm, r);
    if (pos < 0 || pos >= kv.n_ctx || pos >= max_pos) {
        if (lane == 0) record_error(err, 1u);
        return;
    }
    if (seq < 0 || seq >= kv.n_seq) {
        if (lane == 0) record_error(err, 2u);
        return;
    }
    const bool act = lane < half;
    const float* src = qkv + (int64_t)r * ldqkv;
    int col;
    if (hi < n_heads) col = hi * d;
    else if (hi < n_heads + n_kv) col = n_heads * d + (hi - n_heads) * d;
    else col = n_heads * d + n_kv * d + (hi - n_heads - n_kv) * d;
    float u0 = act ? src[col + lane] : 0.f;
    float u1 = act ? src[col + lane + half] : 0.f;
    if (hi >= n_heads + n_kv) {  // value head: straight copy into the cache
        const int j = hi - n_heads - n_kv;
        const int64_t off = ((int64_t)(seq * kv.n_kv + j) * kv.n_ctx + pos) * d;
        if (act) {
            KT::st((typename KT::T*)kv.v, off + lane, u0);
            KT::st((typename KT::T*)kv.v, off + lane + half, u1);
        }
        return;
    }
    const bool is_q = hi < n_heads;
    const typename GT::T* g = is_q ? qg : kg;
    const float ss = wave_sum(u0 * u0 + u1 * u1);
    const float rs = 1.0f / sqrtf(ss / (float)d + eps);
    float a = 0.f, b = 0.f, c = 1.f, sn = 0.f;
    if (act) {
        a = u0 * rs * GT::ld(g, lane);
        b = u1 * rs * GT::ld(g, lane + half);
        const float2 cs = reinterpret_cast<const float2*>(rope)[(int64_t)pos * half + lane];
        c = cs.x;
        sn = cs.y;
    }
    const float r0 = a * c - b * sn;
    const float r1 = a * sn + b * c;
    if (!act) return;
    if (is_q) {
        const int64_t off = (int64_t)r * ldq + hi * d;
        if (q_f16) {
            F16::st((uint16_t*)q_out, off + lane, r0);
            F16::st((uint16_t*)q_out, off + lane + half, r1);
        } else {
            ((float*)q_out)[off + lane] = r0;
            ((float*)q_out)[off + lane + half] = r1;
        }
    } else {
        const int j = hi - n_heads;
        const int64_t off = ((int64_t)(seq * kv.n_kv + j) * kv.n_ctx + pos) * d;
        KT::st((typename KT::T*)kv.k, off + lane, r0);
        KT::st((typename KT::T*)kv.k, off + lane + half, r1);
    }
}

hipError_t launch_qk_norm_rope_kv(const float* qkv, int64_t ldqkv, int R, int n_heads, int n_kv, int d,
                                  const void* q_gain, const void* k_gain, WType gt, float eps, const float* rope,
                                  int max_pos, RowMap rm, KVLayer kv, void* q_out, bool q_f16, int64_t ldq,
                                  uint32_t* err, hipStream_t s) {
    if (R <= 0) return hipSuccess;
    const int items = R * (n_heads + 2 * n_kv);
    const int grid = (items + 3) / 4;
#define QK_LAUNCH(GT_, KT_)                                                                                     \
    qk_norm_rope_kv_kernel<GT_, KT_><<<grid, 256, 0, s>>>(qkv, ldqkv, R, n_heads, n_kv, d,                     \
                                                          (const typename GT_::T*)q_gain,                     \
                                                          (const typename GT_::T*)k_gain, eps, rope, max_pos, \
                                                          rm, kv, q_out, q_f16, ldq, err)
    if (gt == W_BF16) {
        if (kv.type == KV_F16) QK_LAUNCH(BF16, F16);
        else QK_LAUNCH(BF16, F32);
    } else {
        if (kv.type == KV_F16) QK_LAUNCH(F32, F16);
        else QK_LAUNCH(F32, F32);
    }
#undef QK_LAUNCH
    return hipGetLastError();
}

// ------------------------------------------------------------------ embedding gather
// x[b, :] = embed[ids[b], :] widened to fp32 (the tied table's get_rows in
// build_step_graph). An id outside [0, vocab) gives a zero row and an error bit.
template <class WT>
__global__ __launch_bounds__(256) void embed_gather_kernel(const typename WT::T* __restrict__ E, int vocab,
                                                           int hidden, const int32_t* __restrict__ ids,
                                                           float* __restrict__ x, uint32_t* err) {
    const int b = blockIdx.x;
    const int id = ids[b];
    const bool ok = id >= 0 && id < vocab;
    if (!ok && threadIdx.x == 0) record_error(err, 4u);
    float* xr = x + (int64_t)b * hidden;
    for (int i = threadIdx.x; i < hidden; i += 256) xr[i] = ok ? WT::ld(E, (int64_t)id * hidden + i) : 0.f;
}

hipError_t launch_embed_gather(const void* embed, WType wt, int vocab, int hidden, int B, const int32_t* ids,
                               float* x, uint32_t* err, hipStream_t s) {
    if (B <= 0) return hipSuccess;
    if (wt == W_BF16)
        embed_gather_kernel<BF16><<<B, 256, 0, s>>>((const uint16_t*)embed, vocab, hidden, ids, x, err);
    else
        embed_gather_kernel<F32><<<B, 256, 0, s>>>((const float*)embed, vocab, hidden, ids, x, err);
    return hipGetLastError();
}

// ------------------------------------------------------------------ zero fill
__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* __restrict__ p, size_t n16, uint8_t* tail,
                                                        size_t ntail) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
    if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
    if (bytes == 0) return hipSuccess;
    const size_t n16 = bytes / 16;
    size_t grid = (n16 + 255) / 256;
    if (grid > 8192) grid = 8192;
    if (grid == 0) grid = 1;
    fill_zero_kernel<<<(unsigned)grid, 256, 0, s>>>((uint4*)p, n16, (uint8_t*)p + n16 * 16, bytes - n16 * 16);
    return hipGetLastError();
}

}  // namespace sttd
