// attn_rows.h - split-K grouped-query attention of independent rows (one
// workgroup item: row r, KV head j, split), used by the rows attention
// kernel and by the single-row projection + attention launch.
#pragma once

#include <type_traits>

#include "common.h"
#include "launch.h"

// Cache rows per group per streaming step (0: by query heads per KV head) and
// the depth of the register ring they stream through.
#ifndef STTD_ATTN_RIF
#define STTD_ATTN_RIF 0
#endif
#ifndef STTD_ATTN_DEPTH
#define STTD_ATTN_DEPTH 2
#endif

namespace sttd {

// ------------------------------------------------------------------ rows attention (decode)
// Grid (row, kv head, split), NW waves per workgroup. The split's share of
// cache rows [0, p] is ceil((p + 1) / n_splits) rows, so the work follows the
// actual position although the grid is sized from a host bound.
//
// FUSE (decode rows, one row per slab): the workgroup starts from the raw
// Q|K|V projection of its row: waves RMSNorm + rotate the G query heads of
// the group into LDS, and the workgroup whose split holds position p also
// norms + rotates the new key, writes key and value to cache row p and keeps
// them in LDS, so no other kernel or workgroup is waited on. Without FUSE the
// query rows come normed and rotated and the cache already holds every key
// (prefill rows on an f32 cache).
//
// Groups of LPK = d/8 lanes read one cache row (16 bytes per lane for f16,
// coalesced), RIF rows per step through a register ring two steps deep, and
// keep a running (max, sum, output) per query head, rescaled once per step;
// groups merge by shuffles inside a wave and through LDS across
// waves. One split: the workgroup writes o = O / L. Several: it writes the
// partial (M, L, O); attn_combine merges the splits into o, or, when no
// output is given, the consumer (the O-projection GEMV) merges them as it
// loads its activations.
struct RowsArgs {
    const float* q;      // FUSE: raw projection rows [R][(nq + 2 nkv) d]; else q rows [R][nq d]
    int64_t ldq;
    int n_heads;
    RowMap rm;
    KVLayer kv;
    int n_splits;
    float* part;
    float* out_f32;
    uint16_t* out_bf16;
    uint16_t* out_lo;
    int64_t ldo;
    uint32_t* err;
    const void* q_gain;  // FUSE only
    const void* k_gain;
    float eps;
    const float* rope;
    int max_pos;
    // non-null with several splits and an output to write: [rows][n_kv] zeroed
    // counts; the last split of a (row, KV head) to finish merges all of them
    uint32_t* merge_ctr;
    // Tagged hand-off (the single-row projection + attention launch): the raw
    // projection row arrives as 64-bit words (tag << 32 | value bits) in qtag,
    // written while this workgroup already runs; it polls until every word it
    // reads carries `tag`. The last of n_consumers workgroups to finish reading
    // advances *tag_gen (never to 0) and zeroes *tag_done for the next launch.
    const uint64_t* qtag;
    uint32_t tag;
    uint32_t* tag_gen;
    uint32_t* tag_done;
    int n_consumers;
    uint64_t* clk;
};

constexpr uint64_t kTagSpinTicks = 20000000;  // a hand-off poll gives up after 200 ms (100 MHz clock)

// Eight cache elements as loaded (16 bytes of f16, or 32 of fp32), widened at use,
// so a wave holds twice the rows in flight for the registers of fp32 copies.
template <class KT>
struct KvRaw;
template <>
struct KvRaw<F16> {
    u32x4 v;
    __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const u32x4*>(p); }
    __device__ __forceinline__ void widen(float* o) const {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = f16_bits_to_f32((uint16_t)(w[i] & 0xFFFFu));
            o[2 * i + 1] = f16_bits_to_f32((uint16_t)(w[i] >> 16));
        }
    }
};
template <>
struct KvRaw<F32> {
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

// Fold another (m, l, o) running state into this one (base-2 exponents).
template <int G>
__device__ __forceinline__ void merge_state(float (&m)[G], float (&l)[G], float (&o)[G][8], const float (&m2)[G],
                                            const float (&l2)[G], const float (&o2)[G][8]) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float M = fmaxf(m[g], m2[g]);
        const float a = M == -INFINITY ? 0.f : exp2f(m[g] - M);
        const float b = M == -INFINITY ? 0.f : exp2f(m2[g] - M);
        l[g] = l[g] * a + l2[g] * b;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[g][i] = o[g][i] * a + o2[g][i] * b;
        m[g] = M;
    }
}

template <int G>
__device__ __forceinline__ void step_state(float (&m)[G], float (&l)[G], float (&o)[G][8], const float (&s)[G],
                                           const float (&vr)[8]) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float mn = fmaxf(m[g], s[g]);
        const float alpha = exp2f(m[g] - mn);
        const float p = exp2f(s[g] - mn);
        l[g] = l[g] * alpha + p;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[g][i] = fmaf(o[g][i], alpha, p * vr[i]);
        m[g] = mn;
    }
}

// Sum over the LPK lanes that share one cache row.
template <int LPK>
__device__ __forceinline__ float group_sum(float v) {
    return LPK == 16 ? row16_sum(v) : row8_sum(v);
}

template <class KT, class GT, int D, int G, int NW, bool FUSE, class MEM = PlainMem, bool TAGGED = false>
__device__ __forceinline__ void attn_rows_item(const RowsArgs& a, const int r, const int j, const int split) {
    static_assert(!TAGGED || FUSE, "the tagged hand-off carries raw projection rows");
    typedef typename KT::T T;
    constexpr int LPK = D / 8;                 // lanes per cache row
    constexpr int GPW = WAVE / LPK;            // groups per wave
    constexpr int NG = NW * GPW;               // groups per workgroup
    constexpr int HALF = D / 2;
    constexpr int SLOTS = NW * (16 / LPK);     // states per workgroup after the in-wave merge
    static_assert(LPK == 8 || LPK == 16, "head_dim 64 or 128");
    __shared__ float q_lds[G][D];
    __shared__ float kn_lds[D], vn_lds[D];
    __shared__ float wm_lds[SLOTS][G], wl_lds[SLOTS][G];
    __shared__ float wo_lds[SLOTS][G][D];

    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int grp = tid / LPK, sub = tid % LPK;
    const float scale = 1.4426950408889634f / sqrtf((float)D);

    // 1. the row's position and slab, this wave's raw head items of the
    //    projection (items: G query heads, then the key, then the value; wave w
    //    takes items w, w + NW, ...) and their gains: independent loads, all
    //    issued before the first wait (addresses clamped, not branched around)
    //    (decode rows always come with device position and slab arrays)
    const int pos_v = FUSE ? a.rm.pos[r] : row_pos(a.rm, r);
    const int seq_v = FUSE ? a.rm.seq[r] : row_seq(a.rm, r);
    constexpr int IPW = (G + 2 + NW - 1) / NW;  // items per wave
    const int lc = lane < HALF ? lane : 0;
    float u0[IPW], u1[IPW];
    typename GT::T g0r[IPW], g1r[IPW];
    // projection column of this wave's item k
    auto item_col = [&](int k) {
        const int it = wave + k * NW;
        const int itc = it < G + 2 ? it : 0;
        return itc < G ? (j * G + itc) * D : (itc == G ? (a.n_heads + j) * D : (a.n_heads + a.kv.n_kv + j) * D);
    };
    if (FUSE) {
        const float* src = a.q + (int64_t)r * a.ldq;
#pragma unroll
        for (int k = 0; k < IPW; ++k) {
            const int it = wave + k * NW;
            const int itc = it < G + 2 ? it : 0;
            const int col = item_col(k);
            if (!TAGGED) {
                u0[k] = MEM::ld(src + col + lc);
                u1[k] = MEM::ld(src + col + lc + HALF);
            }
            const typename GT::T* gain = (const typename GT::T*)(itc < G ? a.q_gain : a.k_gain);
            g0r[k] = gain[lc];
            g1r[k] = gain[lc + HALF];
        }
    }
    // keep the scheduler from pulling the first use of a loaded value (and its
    // wait) above the loads issued after it
    __builtin_amdgcn_sched_barrier(0);
    // 2. position-dependent loads: the rotation row, then the first cache rows of each group
    const int pos = pos_v, seq = seq_v;
    const bool ok = pos >= 0 && pos < a.kv.n_ctx && pos < (FUSE ? a.max_pos : a.kv.n_ctx) && seq >= 0 &&
                    seq < a.kv.n_seq;
    // pos -1 marks a row whose greedy loop has stopped: skipped, not an error
    if (!ok && pos != -1 && tid == 0 && split == 0 && j == 0)
        record_error(a.err, pos < 0 || pos >= a.kv.n_ctx ? 1u : 2u);
    float2 cs = make_float2(1.f, 0.f);
    if (FUSE) cs = reinterpret_cast<const float2*>(a.rope)[(int64_t)(ok ? pos : 0) * HALF + lc];
    const int n_keys = ok ? pos + 1 : 0;
    const int ns = a.n_splits;
    const int chunk = (n_keys + ns - 1) / ns;
    const int c0 = split * chunk;
    const int c1 = min(c0 + chunk, n_keys);
    const bool owner = FUSE && ok && c0 <= pos && pos < c1;  // this split holds the new key
    const int64_t slab = ((int64_t)(ok ? seq : 0) * a.kv.n_kv + j) * a.kv.n_ctx * D;
    const T* Kp = (const T*)a.kv.k + slab + sub * 8;
    const T* Vp = (const T*)a.kv.v + slab + sub * 8;
    const int cend = owner ? pos : c1;  // the new key (owner) is folded in from LDS below
    // The cache rows stream through a register ring of DEPTH steps of RIF rows per
    // group (row cb + grp + q * NG of the step at cb); the step DEPTH ahead is fetched
    // as soon as a step has been used. Every fetch is issued, clamped to the last row
    // of the span past its end, so the count of loads in flight is the same on every
    // path and each wait leaves the later steps in flight. (The former form, one step
    // in flight fetched between a step's scores and its state update, with per-group
    // trip counts, waited for all loads each step: 18.0 us for 16 rows of 150-1500
    // positions.)
    // (per launch in a 28-block decode of 16 rows at 151-1535 positions, G = 2, two
    // steps deep: 2 rows per step 16.2 us, 4 rows 16.7, 8 rows 21.1, 1 row 16.9 (a
    // rescale per row; four steps deep 16.4); three or four steps deep 16.4-17.7)
    // 4-wave workgroups (single rows, and the one-launch projection + attention, whose
    // sums must match the two-launch form bit for bit: the rescale per step makes the
    // rounding depend on the step) keep 4
    constexpr int RIF = STTD_ATTN_RIF > 0 ? STTD_ATTN_RIF
                                          : (G <= 2 ? (NW == 4 ? 4 : 2) : (G == 4 ? 2 : 1));
    // (the single-row projection + attention launch: splits of a few dozen rows, within
    // one step, where a second step only adds loads: 8.5 -> 9.1 us per launch)
    constexpr int DEPTH = TAGGED ? 1 : STTD_ATTN_DEPTH;
    constexpr int STEP = RIF * NG;
    const int last = cend > 0 ? cend - 1 : 0;
    KvRaw<KT> kr[DEPTH][RIF], vr[DEPTH][RIF];
    auto fetch = [&](KvRaw<KT>(&kk)[RIF], KvRaw<KT>(&vv)[RIF], const int cb) {
#pragma unroll
        for (int q = 0; q < RIF; ++q) {
            const int cq = min(cb + grp + q * NG, last);
            kk[q].load(Kp + (int64_t)cq * D);
            vv[q].load(Vp + (int64_t)cq * D);
        }
    };
#pragma unroll
    for (int b = 0; b < DEPTH; ++b) {
        fetch(kr[b], vr[b], c0 + b * STEP);
        __builtin_amdgcn_sched_barrier(0);  // the steps in order, as the loop waits for them
    }
    __builtin_amdgcn_sched_barrier(0);
    // 2b. tagged hand-off: with the cache rows above in flight, poll this wave's
    //     raw head items until each word carries this launch's tag (bounded wait)
    if (TAGGED) {
        const uint64_t* src = a.qtag + (int64_t)r * a.ldq;
        const uint64_t t0 = wall_clock64();
        while (true) {
            bool good = true;
#pragma unroll
            for (int k = 0; k < IPW; ++k) {
                const int col = item_col(k);
                const uint64_t w0 = __hip_atomic_load(src + col + lc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const uint64_t w1 = __hip_atomic_load(src + col + lc + HALF, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                good = good && (uint32_t)(w0 >> 32) == a.tag && (uint32_t)(w1 >> 32) == a.tag;
                u0[k] = __uint_as_float((uint32_t)w0);
                u1[k] = __uint_as_float((uint32_t)w1);
            }
            if (__all(good)) break;
            if (wall_clock64() - t0 > kTagSpinTicks) {
                if (lane == 0) record_error(a.err, kDevErrSync);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    // 3. finish the head items: RMSNorm + rotation (queries, key); the owner
    //    writes key and value to cache row pos
    if (FUSE) {
#pragma unroll
        for (int k = 0; k < IPW; ++k) {
            const int it = wave + k * NW;
            if (it >= G + 2 || !ok) continue;
            const float v0 = lane < HALF ? u0[k] : 0.f, v1 = lane < HALF ? u1[k] : 0.f;
            if (it <= G) {
                const float rs = 1.0f / sqrtf(wave_sum(v0 * v0 + v1 * v1) / (float)D + a.eps);
                if (lane < HALF) {
                    const float x0 = v0 * rs * GT::cvt(g0r[k]), x1 = v1 * rs * GT::cvt(g1r[k]);
                    const float r0 = x0 * cs.x - x1 * cs.y, r1 = x0 * cs.y + x1 * cs.x;
                    if (it < G) {
                        q_lds[it][lane] = r0 * scale;
                        q_lds[it][lane + HALF] = r1 * scale;
                    } else if (owner) {
                        kn_lds[lane] = r0;
                        kn_lds[lane + HALF] = r1;
                        KT::st((T*)a.kv.k, slab + (int64_t)pos * D + lane, r0);
                        KT::st((T*)a.kv.k, slab + (int64_t)pos * D + lane + HALF, r1);
                    }
                }
            } else if (owner && lane < HALF) {
                vn_lds[lane] = v0;
                vn_lds[lane + HALF] = v1;
                KT::st((T*)a.kv.v, slab + (int64_t)pos * D + lane, v0);
                KT::st((T*)a.kv.v, slab + (int64_t)pos * D + lane + HALF, v1);
            }
        }
    } else {
        for (int t = tid; t < G * D; t += NW * 64)
            q_lds[t / D][t % D] = ok ? MEM::ld(a.q + (int64_t)r * a.ldq + (j * G + t / D) * D + t % D) * scale : 0.f;
    }
    __syncthreads();
    // every wave of this workgroup is done with the tagged words: count out; the
    // last consumer of the launch moves the tag on and re-arms the count
    if (TAGGED && tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(a.tag_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old == (uint32_t)(a.n_consumers - 1)) {
            __hip_atomic_store(a.tag_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.tag_gen, a.tag + 1u == 0u ? 1u : a.tag + 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    float qv[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < 8; ++i) qv[g][i] = q_lds[g][sub * 8 + i];
    float m[G], l[G], o[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[g][i] = 0.f;
    }
    // 4. cache rows [c0, cend), a step of RIF rows per group at a time: the scores,
    //    one rescale of the running state to the step's maximum, then the weighted
    //    values (rows past the end score -inf and weigh 0)
    auto consume = [&](const KvRaw<KT>(&kk)[RIF], const KvRaw<KT>(&vv)[RIF], const int cb) {
        float sc[RIF][G];
#pragma unroll
        for (int q = 0; q < RIF; ++q) {
            float kf[8];
            kk[q].widen(kf);
            const bool valid = cb + grp + q * NG < cend;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float t = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) t = fmaf(qv[g][i], kf[i], t);
                t = group_sum<LPK>(t);
                sc[q][g] = valid ? t : -INFINITY;
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float M = m[g];
#pragma unroll
            for (int q = 0; q < RIF; ++q) M = fmaxf(M, sc[q][g]);
            const float Ms = M == -INFINITY ? 0.f : M;
            // v_exp_f32 itself: results below 2^-126 (weights that small against the
            // running maximum's 1) flush to 0, and exp2(-inf) is 0 (exp2f's denormal
            // range handling cost 12.7 -> 11.6 us on one 1535-position row). Moving the
            // reference maximum only when passed by more than 2^8, skipping most
            // rescales, took 11.6 -> 11.0 us there but nothing on 16 mixed rows: not kept
            const float alpha = __builtin_amdgcn_exp2f(m[g] - Ms);
            float lsum = l[g] * alpha;
#pragma unroll
            for (int q = 0; q < RIF; ++q) {
                sc[q][g] = __builtin_amdgcn_exp2f(sc[q][g] - Ms);
                lsum += sc[q][g];
            }
            l[g] = lsum;
            m[g] = M;
#pragma unroll
            for (int i = 0; i < 8; ++i) o[g][i] *= alpha;
        }
#pragma unroll
        for (int q = 0; q < RIF; ++q) {
            float vf[8];
            vv[q].widen(vf);
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int i = 0; i < 8; ++i) o[g][i] = fmaf(sc[q][g], vf[i], o[g][i]);
        }
    };
    // uniform trip count: every wave runs the same steps
    for (int cb = c0; cb < cend; cb += DEPTH * STEP) {
#pragma unroll
        for (int b = 0; b < DEPTH; ++b) {
            // a step wholly past the end is not computed (a uniform branch holding no
            // loads, so the counts of loads in flight stay exact)
            if (cb + b * STEP < cend) consume(kr[b], vr[b], cb + b * STEP);
            // keep each refetch right after its step's use (the scheduler would
            // otherwise sink them all to the end of the loop body)
            __builtin_amdgcn_sched_barrier(0);
            fetch(kr[b], vr[b], cb + (b + DEPTH) * STEP);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // 5. the new key (held in LDS by the owner), folded in by group 0
    if (owner && grp == 0) {
        float kn[8], vn[8], s[G];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            kn[i] = kn_lds[sub * 8 + i];
            vn[i] = vn_lds[sub * 8 + i];
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float t1 = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) t1 = fmaf(qv[g][i], kn[i], t1);
            s[g] = group_sum<LPK>(t1);
        }
        step_state<G>(m, l, o, s, vn);
    }
    // 6. merge across rows of the wave (lane bits 4, 5) with permlane swaps; the
    //    16-lane rows (for head_dim 64: both 8-lane groups of a row) then go to LDS
    {
        float m2[G], l2[G], o2[G][8];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            m2[g] = xor16(m[g]);
            l2[g] = xor16(l[g]);
#pragma unroll
            for (int i = 0; i < 8; ++i) o2[g][i] = xor16(o[g][i]);
        }
        merge_state<G>(m, l, o, m2, l2, o2);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            m2[g] = xor32(m[g]);
            l2[g] = xor32(l[g]);
#pragma unroll
            for (int i = 0; i < 8; ++i) o2[g][i] = xor32(o[g][i]);
        }
        merge_state<G>(m, l, o, m2, l2, o2);
    }
    if (lane < 16) {
        const int slot = wave * (16 / LPK) + lane / LPK;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (sub == 0) {
                wm_lds[slot][g] = m[g];
                wl_lds[slot][g] = l[g];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) wo_lds[slot][g][sub * 8 + i] = o[g][i];
        }
    }
    __syncthreads();
    // 7. merge the slots; write o (one split) or the split's partial record
    for (int t = tid; t < G * D; t += NW * 64) {
        const int g = t / D, e = t % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < SLOTS; ++w) M = fmaxf(M, wm_lds[w][g]);
        float L = 0.f, O = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < SLOTS; ++w) {
                const float f = exp2f(wm_lds[w][g] - M);
                L += f * wl_lds[w][g];
                O += f * wo_lds[w][g][e];
            }
        }
        if (ns == 1) {
            const float v = L > 0.f ? O / L : 0.f;
            const int64_t idx = (int64_t)r * a.ldo + (j * G + g) * D + e;
            if (a.out_f32) {
                MEM::st(a.out_f32 + idx, v);
            } else {
                uint16_t hi, lo;
                split_bf16(v, hi, lo);
                a.out_bf16[idx] = hi;
                if (a.out_lo) a.out_lo[idx] = lo;
            }
        } else {
            float* pp = a.part + (((int64_t)r * a.n_heads + j * G + g) * a.n_splits + split) * (D + 4);
            if (e == 0) {
                MEM::st(pp, M);
                MEM::st(pp + 1, L);
            }
            MEM::st(pp + 4 + e, O);
        }
    }
    // 8. several splits and an output: the split of this (row, KV head) that
    //    finishes last merges all partial records and writes o, so no combine
    //    pass runs. The partials were published with device-scope stores, which
    //    each wave waits for before the count. The merging split copies the
    //    G * n_splits records into LDS with device-scope loads, every thread's
    //    loads in flight at once (records of neighbouring pairs share cache
    //    lines, which a plain load could find stale in this XCD's L2), then
    //    merges from LDS. It resets the count for the next launch. Only the
    //    publishing instantiation carries this (and its LDS).
    if constexpr (std::is_same<MEM, PubMem>::value) {
        if (a.merge_ctr && ns > 1) {
            constexpr int MREC = 64;  // records staged: G * n_splits <= MREC (checked on the host)
            __shared__ __attribute__((aligned(16))) float mrg[MREC * (D + 4)];
            __shared__ int is_last;
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores have completed
            __syncthreads();
            if (tid == 0) {
                uint32_t* c = a.merge_ctr + (int64_t)r * a.kv.n_kv + j;
                const uint32_t old = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                is_last = old == (uint32_t)(ns - 1);
                if (is_last) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
            if (is_last) {
                // the G heads' records are contiguous: record (g, split) at (g * n_splits + split) * (D + 4);
                // this row's are splits [0, ns) of each head
                const int nrec = G * a.n_splits;
                const uint64_t* src = reinterpret_cast<const uint64_t*>(
                    a.part + ((int64_t)r * a.n_heads + j * G) * a.n_splits * (D + 4));
                uint64_t* dst = reinterpret_cast<uint64_t*>(mrg);
                for (int i = tid; i < nrec * (D + 4) / 2; i += NW * 64)
                    dst[i] = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __syncthreads();
                for (int t = tid; t < G * D; t += NW * 64) {
                    const int g = t / D, e = t % D;
                    const float* rec = mrg + g * a.n_splits * (D + 4);
                    float M = -INFINITY;
                    for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, rec[sp * (D + 4)]);
                    float L = 0.f, O = 0.f;
                    if (M != -INFINITY) {
                        for (int sp = 0; sp < ns; ++sp) {
                            const float w = exp2f(rec[sp * (D + 4)] - M);
                            L = fmaf(w, rec[sp * (D + 4) + 1], L);
                            O = fmaf(w, rec[sp * (D + 4) + 4 + e], O);
                        }
                    }
                    const float v = L > 0.f ? O / L : 0.f;
                    const int64_t idx = (int64_t)r * a.ldo + (j * G + g) * D + e;
                    if (a.out_f32) {
                        a.out_f32[idx] = v;
                    } else {
                        uint16_t hi, lo;
                        split_bf16(v, hi, lo);
                        a.out_bf16[idx] = hi;
                        if (a.out_lo) a.out_lo[idx] = lo;
                    }
                }
            }
        }
    }
}

}  // namespace sttd
