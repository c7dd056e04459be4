// kernels_misc.hip - RMSNorm rows, per-head Q/K RMSNorm + NeoX RoPE + KV write,
// token-embedding gather, fills.
#include "common.h"
#include "headops.h"
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
                                                                float eps, const int32_t* __restrict__ xrow,
                                                                int n_xrows, uint32_t* err, uint64_t* clk) {
    __shared__ float red[4];
    clock_begin(clk);
    int src = blockIdx.x;
    if (xrow) {
        src = xrow[blockIdx.x];
        if (src < 0 || src >= n_xrows) {
            if (threadIdx.x == 0) record_error(err, kDevErrRow);
            src = 0;
        }
    }
    const float* xr = x + (int64_t)src * ldx;
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
    clock_end(clk);
}

hipError_t launch_rmsnorm_rows_bf16(const float* x, int64_t ldx, const void* gain, WType gt, uint16_t* out,
                                    uint16_t* out_lo, int64_t ldo, int R, int H, float eps, hipStream_t s,
                                    const int32_t* xrow, int n_xrows, uint32_t* err) {
    if (R <= 0) return hipSuccess;
    if (gt == W_BF16)
        launch_kernel(rmsnorm_rows_bf16_kernel<BF16>, R, 256, 0, s, x, ldx, (const uint16_t*)gain, out, out_lo, ldo, H, eps,
                                                         xrow, n_xrows, err, clock_slot());
    else
        launch_kernel(rmsnorm_rows_bf16_kernel<F32>, R, 256, 0, s, x, ldx, (const float*)gain, out, out_lo, ldo, H, eps, xrow,
                                                        n_xrows, err, clock_slot());
    return hipGetLastError();
}

// ------------------------------------------------------------------ Q/K norm + RoPE + KV write
// One wave per (row, head item); see qk_head_item.
template <class GT, class KT>
__global__ __launch_bounds__(256) void qk_norm_rope_kv_kernel(const float* __restrict__ qkv, int64_t ldqkv, int R,
                                                              QkRope p) {
    clock_begin(p.clk);
    const int items = p.n_heads + 2 * p.n_kv;
    const int item = blockIdx.x * 4 + threadIdx.x / WAVE;
    if (item < R * items) qk_head_item<GT, KT>(qkv + (int64_t)(item / items) * ldqkv, item / items, item % items, p);
    clock_end(p.clk);
}

hipError_t launch_qk_norm_rope_kv(const float* qkv, int64_t ldqkv, int R, WType gt, const QkRope& qr, hipStream_t s) {
    if (R <= 0) return hipSuccess;
    QkRope q = qr;
    q.clk = clock_slot();
    const int items = R * (q.n_heads + 2 * q.n_kv);
    const int grid = (items + 3) / 4;
    if (gt == W_BF16) {
        if (q.kv.type == KV_F16) launch_kernel(qk_norm_rope_kv_kernel<BF16, F16>, grid, 256, 0, s, qkv, ldqkv, R, q);
        else launch_kernel(qk_norm_rope_kv_kernel<BF16, F32>, grid, 256, 0, s, qkv, ldqkv, R, q);
    } else {
        if (q.kv.type == KV_F16) launch_kernel(qk_norm_rope_kv_kernel<F32, F16>, grid, 256, 0, s, qkv, ldqkv, R, q);
        else launch_kernel(qk_norm_rope_kv_kernel<F32, F32>, grid, 256, 0, s, qkv, ldqkv, R, q);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------ embedding gather
// x[b, :] = embed[ids[b], :] widened to fp32 (the tied table's get_rows in
// build_step_graph). With keep and/or dense, the prompt/audio injection blend
// of the batched prefill graphs: x[b, :] = embed[ids[b], :] * keep[b] +
// dense[b, :] (keep broadcasts over the hidden axis). An id outside
// [0, vocab) contributes a zero row and sets an error bit.
template <class WT>
__global__ __launch_bounds__(256) void embed_gather_kernel(const typename WT::T* __restrict__ E, int vocab,
                                                           int hidden, const int32_t* __restrict__ ids,
                                                           const float* __restrict__ keep,
                                                           const float* __restrict__ dense, float* __restrict__ x,
                                                           uint32_t* err) {
    const int b = blockIdx.x;
    const int id = ids[b];
    const bool ok = id >= 0 && id < vocab;
    if (!ok && threadIdx.x == 0) record_error(err, 4u);
    const float kb = keep ? keep[b] : 1.f;
    float* xr = x + (int64_t)b * hidden;
    const float* dr = dense ? dense + (int64_t)b * hidden : nullptr;
    for (int i = threadIdx.x; i < hidden; i += 256) {
        const float e = ok ? WT::ld(E, (int64_t)id * hidden + i) : 0.f;
        xr[i] = dense ? e * kb + dr[i] : (keep ? e * kb : e);
    }
}

hipError_t launch_embed_gather(const void* embed, WType wt, int vocab, int hidden, int B, const int32_t* ids,
                               const float* keep, const float* dense, float* x, uint32_t* err, hipStream_t s) {
    if (B <= 0) return hipSuccess;
    if (wt == W_BF16)
        launch_kernel(embed_gather_kernel<BF16>, B, 256, 0, s, (const uint16_t*)embed, vocab, hidden, ids, keep, dense, x, err);
    else
        launch_kernel(embed_gather_kernel<F32>, B, 256, 0, s, (const float*)embed, vocab, hidden, ids, keep, dense, x, err);
    return hipGetLastError();
}

// ------------------------------------------------------------------ packed-sequence row maps
// Row r of a packed batched prefill: its sequence is the last one starting at
// or before r; position pos0 + (r - start), slab seq.
__global__ __launch_bounds__(256) void expand_segments_kernel(Segments sg, int R, int32_t* __restrict__ pos,
                                                              int32_t* __restrict__ seq) {
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r >= R) return;
    int i = 0;
    for (int k = 1; k < sg.n; ++k)
        if (sg.start[k] <= r) i = k;
    pos[r] = sg.pos0[i] + (r - sg.start[i]);
    seq[r] = sg.seq[i];
}

hipError_t launch_expand_segments(const Segments& sg, int R, int32_t* pos, int32_t* seq, hipStream_t s) {
    if (R <= 0) return hipSuccess;
    launch_kernel(expand_segments_kernel, (R + 255) / 256, 256, 0, s, sg, R, pos, seq);
    return hipGetLastError();
}

// ------------------------------------------------------------------ greedy stopping rules
// One workgroup walks the rows. An active row appends its token. With
// `advance` its next input position moves on by one; the first call after the
// prefill leaves it at the prompt length. The row goes on while the token is
// not EOS, fewer than max_new tokens exist and the next position is inside the
// context (the step loop's condition in run() on the Qwen3-ASR model page).
// A row that stops gets pos -1, which the block step skips, and is truncated
// unless it stopped on EOS.
__global__ __launch_bounds__(256) void greedy_stop_kernel(int B, const int32_t* __restrict__ ids, int eos_id,
                                                          int max_new, int n_ctx, int advance, int32_t* pos,
                                                          int32_t* active, int32_t* n_gen, int32_t* tokens,
                                                          int32_t* truncated, int32_t* n_active) {
    __shared__ int count;
    if (threadIdx.x == 0) count = 0;
    __syncthreads();
    int mine = 0;
    for (int b = threadIdx.x; b < B; b += 256) {
        if (!active[b]) continue;
        const int tok = ids[b];
        const int n = n_gen[b];
        if (n < max_new) tokens[(int64_t)b * max_new + n] = tok;
        n_gen[b] = n + 1;
        const int next = pos[b] + (advance ? 1 : 0);
        const bool go = tok != eos_id && n + 1 < max_new && next + 1 <= n_ctx;
        if (go) {
            pos[b] = next;
            ++mine;
        } else {
            pos[b] = -1;
            active[b] = 0;
            truncated[b] = tok != eos_id ? 1 : 0;
        }
    }
    if (mine) atomicAdd(&count, mine);
    __syncthreads();
    if (threadIdx.x == 0 && n_active) *n_active = count;
}

hipError_t launch_greedy_stop(int B, const int32_t* ids, int eos_id, int max_new, int n_ctx, int advance,
                              int32_t* pos, int32_t* active, int32_t* n_gen, int32_t* tokens, int32_t* truncated,
                              int32_t* n_active, hipStream_t s) {
    if (B <= 0) return hipSuccess;
    launch_kernel(greedy_stop_kernel, 1, 256, 0, s, B, ids, eos_id, max_new, n_ctx, advance, pos, active, n_gen, tokens,
                                          truncated, n_active);
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
    launch_kernel(fill_zero_kernel, (unsigned)grid, 256, 0, s, (uint4*)p, n16, (uint8_t*)p + n16 * 16, bytes - n16 * 16);
    return hipGetLastError();
}

// ------------------------------------------------------------------ clock slot reduction
// One workgroup per slot: first start (min over recorded starts) and last end.
__global__ __launch_bounds__(256) void clock_reduce_kernel(const uint64_t* __restrict__ slots,
                                                           uint64_t* __restrict__ out) {
    __shared__ uint64_t lo_s[4], hi_s[4];
    const uint64_t* e = slots + (size_t)blockIdx.x * kClockEntries * 2;
    uint64_t lo = ~0ull, hi = 0ull;
    for (int i = threadIdx.x; i < kClockEntries; i += 256) {
        const uint64_t a = e[2 * i], b = e[2 * i + 1];
        if (a && a < lo) lo = a;
        if (b > hi) hi = b;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint64_t a = __shfl_xor(lo, off, WAVE), b = __shfl_xor(hi, off, WAVE);
        lo = a < lo ? a : lo;
        hi = b > hi ? b : hi;
    }
    if (threadIdx.x % WAVE == 0) {
        lo_s[threadIdx.x / WAVE] = lo;
        hi_s[threadIdx.x / WAVE] = hi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < 4; ++w) {
            lo = lo_s[w] < lo ? lo_s[w] : lo;
            hi = hi_s[w] > hi ? hi_s[w] : hi;
        }
        out[2 * blockIdx.x] = lo;
        out[2 * blockIdx.x + 1] = hi;
    }
}

hipError_t launch_clock_reduce(const uint64_t* slots, int n, uint64_t* out, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    launch_kernel(clock_reduce_kernel, n, 256, 0, s, slots, out);
    return hipGetLastError();
}

}  // namespace sttd
