// headops.h - per-head Q/K RMSNorm + NeoX RoPE + KV-cache write of one
// (row, head item), run by one wave. Used by the standalone kernel and by the
// fused epilogue of the Q|K|V projection.
#pragma once

#include "common.h"
#include "launch.h"

namespace sttd {

// Items of a row: the n_heads query heads, then the n_kv key heads, then the
// n_kv value heads. Lane i < d/2 owns the NeoX pair (i, i + d/2). Query and
// key heads: RMSNorm over head_dim with the shared gain, then pair i turns by
// the table angle pos * theta^(-2i/d). Keys and values go to cache row `pos`
// of the row's slab; values are copied as they are. (Qwen3-ASR decoder page,
// file header; the cache index equals the position: kv_idx in
// build_step_graph and run() on the model page.) `src` is the row's
// [n_heads + 2 n_kv] * d projection outputs.
template <class GT, class KT>
__device__ __forceinline__ void qk_head_item(const float* __restrict__ src, int r, int hi, const QkRope& p) {
    const int lane = threadIdx.x % WAVE;
    const int d = p.d, half = d / 2;
    const int pos = row_pos(p.rm, r);
    const int seq = row_seq(p.rm, r);
    if (pos < 0 || pos >= p.kv.n_ctx || pos >= p.max_pos) {
        if (lane == 0) record_error(p.err, 1u);
        return;
    }
    if (seq < 0 || seq >= p.kv.n_seq) {
        if (lane == 0) record_error(p.err, 2u);
        return;
    }
    const bool act = lane < half;
    const int col = hi * d;  // items are laid out in the same order as the projection outputs
    const float u0 = act ? src[col + lane] : 0.f;
    const float u1 = act ? src[col + lane + half] : 0.f;
    const int n_heads = p.n_heads, n_kv = p.n_kv;
    if (hi >= n_heads + n_kv) {  // value head
        const int j = hi - n_heads - n_kv;
        const int64_t off = ((int64_t)(seq * n_kv + j) * p.kv.n_ctx + pos) * d;
        if (act) {
            KT::st((typename KT::T*)p.kv.v, off + lane, u0);
            KT::st((typename KT::T*)p.kv.v, off + lane + half, u1);
        }
        return;
    }
    const bool is_q = hi < n_heads;
    const typename GT::T* g = (const typename GT::T*)(is_q ? p.q_gain : p.k_gain);
    const float ss = wave_sum(u0 * u0 + u1 * u1);
    const float rs = 1.0f / sqrtf(ss / (float)d + p.eps);
    if (!act) return;
    const float a = u0 * rs * GT::ld(g, lane);
    const float b = u1 * rs * GT::ld(g, lane + half);
    const float2 cs = reinterpret_cast<const float2*>(p.rope)[(int64_t)pos * half + lane];
    const float r0 = a * cs.x - b * cs.y;
    const float r1 = a * cs.y + b * cs.x;
    if (is_q) {
        const int64_t off = (int64_t)r * p.ldq + hi * d;
        if (p.q_f16) {
            F16::st((uint16_t*)p.q_out, off + lane, r0);
            F16::st((uint16_t*)p.q_out, off + lane + half, r1);
        } else {
            ((float*)p.q_out)[off + lane] = r0;
            ((float*)p.q_out)[off + lane + half] = r1;
        }
    } else {
        const int j = hi - n_heads;
        const int64_t off = ((int64_t)(seq * n_kv + j) * p.kv.n_ctx + pos) * d;
        KT::st((typename KT::T*)p.kv.k, off + lane, r0);
        KT::st((typename KT::T*)p.kv.k, off + lane + half, r1);
    }
}

}  // namespace sttd
