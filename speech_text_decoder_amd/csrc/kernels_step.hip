// kernels_step.hip - one decode step of one block for a single row, as one
// persistent launch (bf16 weights, f16 cache).
//
// The block is the chain: RMSNorm + Q|K|V projection -> per-head Q/K norm,
// NeoX RoPE, cache write and split-K attention -> O projection + residual ->
// RMSNorm + packed gate_up + SwiGLU -> down projection + residual (the step
// graph on the Qwen3-ASR decoder page: build_step_graph over block_step). For
// one row every stage is a bandwidth-bound pass over its weights, and the
// stages are short: at the 1.7B shape the whole block reads about 100 MB, 12.6
// us at 8 TB/s. As separate kernels each stage pays a launch gap and a load
// ramp. Here one grid of workgroups runs all five. A workgroup issues the weight
// loads of its next item before it waits for the stage that item depends on.
// The hand-off latency is then spent streaming weights.
//
// Hand-offs. Data that another workgroup of this launch reads (the Q|K|V row,
// the attention partials, the attention residual h, the SwiGLU activations)
// is written with device-scope stores that go through to memory (PubMem).
// Each of these buffers is written in one stage and read only after it, so
// the readers' plain loads cannot meet a stale L2 line. They fill from memory
// once per XCD and hit in L2 after that. This is why the O stage writes h to
// a buffer of its own instead of updating x, which the Q stage has read. After
// its writes of a stage, each wave waits for them to complete.
// Then thread 0 adds one to the stage's counter. Workgroup w counts on
// sub-counter w % 64 of the stage, 256 bytes apart, so that the atomics of
// the 512 workgroups spread over addresses and memory channels. A waiting
// workgroup's first wave polls the 64 sub-counters, one per lane, until each
// holds its share. The poll gives up after kSpinTicks of the 100 MHz
// device clock, or as soon as another wait has given up. It then records
// kDevErrSync, so every wait ends even if the workgroups were not all resident.
// The last workgroup out (a two-level count) zeroes the counters for the next
// launch.
//
// Work split (grid of nwg workgroups of 4 waves, item i to workgroup i % nwg):
//   Q: 8 rows of the concatenated Q|K|V weights per item (RMSNorm in front);
//   A: one (KV head, split) of the row's cache span per item;
//   O: 4 rows of W_o per item, the attention splits merged as they load;
//   F: 4 gate rows and the 4 matching up rows per item, SwiGLU behind;
//   D: 4 rows of W_down per item, residual behind.
// Two items' weights are in flight per workgroup: the next one loads while the
// current one reduces.
//
// Measured on MI355X (1.7B block, 300 cached rows, 512 workgroups, per-stage
// device-clock stamps): a hand-off where all 512 workgroups signal at once
// takes 2-4 us from the last signal to the waiters' release. Write-through of
// the published values takes up to 1.5 us, and the counter atomics and polls
// queue behind the weight stream that the design overlaps with them. A hand-off
// where only the 40 attention workgroups signal late takes 0.8-1.3 us. The
// block takes 33.9 us, against 34.5 us for one launch per stage with their
// launch gaps, so the per-stage launches remain the default
// (STTD_OPT_FUSED_STEP = 0).
#include <mutex>
#include <utility>
#include <vector>

#include "attn_rows.h"
#include "common.h"
#include "gemv_ops.h"
#include "launch.h"

namespace sttd {

namespace {

constexpr int kSub = 64;                 // sub-counters per stage: one per lane of the polling wave
constexpr int kLine = 64;                // words between sub-counters (256 bytes)
constexpr int kStages = 4;               // counted hand-offs: Q, A, O, F
constexpr int kDone1 = kStages;          // row of the first level of the exit count
constexpr int kDone2 = kStages + 1;      // its second level (sub-counter 0)
constexpr uint64_t kSpinTicks = 20000000;  // 200 ms of the 100 MHz device clock
constexpr int NRQ = 8, NRO = 4, NCF = 4, NRD = 4;  // rows (F: act columns) per item
static_assert((kDone2 + 1) * kSub * kLine <= kStepSyncWords, "sync area");
static_assert(kSub == WAVE, "one sub-counter per lane of the polling wave");

__device__ __forceinline__ uint32_t* ctr(uint32_t* sync, int row, int sub) { return sync + (row * kSub + sub) * kLine; }

// Every wave's stores so far have completed (s_waitcnt vmcnt(0)).
__device__ __forceinline__ void stores_done() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// This workgroup's device-scope stores of `stage` are complete: count it in.
__device__ __forceinline__ void stage_signal(uint32_t* sync, int stage) {
    stores_done();
    __syncthreads();
    if (threadIdx.x == 0)
        __hip_atomic_fetch_add(ctr(sync, stage, blockIdx.x % kSub), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every workgroup has counted in `stage`.
__device__ __forceinline__ void stage_wait(uint32_t* sync, int stage, int nwg, uint32_t* err) {
    if (threadIdx.x < WAVE) {
        const int sub = threadIdx.x;
        const uint32_t target = (uint32_t)((nwg - sub + kSub - 1) / kSub);
        const uint32_t* c = ctr(sync, stage, sub);
        const uint64_t t0 = wall_clock64();
        while (true) {
            const uint32_t v = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (__all(v >= target)) break;
            const uint32_t e = __builtin_amdgcn_readfirstlane(
                __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            if ((e & kDevErrSync) || wall_clock64() - t0 > kSpinTicks) {
                if (sub == 0) atomicOr(err, kDevErrSync);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    __syncthreads();
}

// Count this workgroup out; the last one zeroes every counter for the next launch.
__device__ __forceinline__ void step_exit(uint32_t* sync, int nwg) {
    stores_done();
    __syncthreads();
    if (threadIdx.x != 0) return;
    const int sub = blockIdx.x % kSub;
    const uint32_t n_sub = (uint32_t)((nwg - sub + kSub - 1) / kSub);
    const uint32_t o1 = __hip_atomic_fetch_add(ctr(sync, kDone1, sub), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (o1 != n_sub - 1) return;
    const uint32_t n_top = (uint32_t)min(nwg, kSub);
    const uint32_t o2 = __hip_atomic_fetch_add(ctr(sync, kDone2, 0), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (o2 != n_top - 1) return;
    for (int row = 0; row <= kDone2; ++row)
        for (int i = 0; i < kSub; ++i) __hip_atomic_store(ctr(sync, row, i), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Items first, first + stride, ... < n with two items' weights in flight.
// issue(it, w) starts the weight loads of item it; ready() runs once before the
// first compute (the wait for the previous stage and the activation loads);
// compute(it, w) reduces and stores item it.
template <int KCH, int NR, class Issue, class Ready, class Compute>
__device__ __forceinline__ void run_items(int first, int n, int stride, Issue issue, Ready ready, Compute compute) {
    if (first >= n) return;
    Raw8<BF16> w0[KCH][NR], w1[KCH][NR];
    issue(first, w0);
    if (first + stride < n) issue(first + stride, w1);
    ready();
    for (int it = first; it < n; it += 2 * stride) {
        compute(it, w0);
        if (it + 2 * stride < n) issue(it + 2 * stride, w0);
        if (it + stride < n) {
            compute(it + stride, w1);
            if (it + 3 * stride < n) issue(it + 3 * stride, w1);
        }
    }
}

template <int KCH>
__device__ __forceinline__ void chunk_offsets(int (&kk)[KCH]) {
    const int lane = threadIdx.x % WAVE, wave = threadIdx.x / WAVE;
#pragma unroll
    for (int c = 0; c < KCH; ++c) kk[c] = (c * 4 + wave) * CHUNK + lane * 8;
}

// Loads of NR weight rows (row r at base + r * rstride), the chunks of this lane.
template <int KCH, int NR>
__device__ __forceinline__ void load_rows(const uint16_t* base, int64_t rstride, int K, const int (&kk)[KCH],
                                          Raw8<BF16> (&w)[KCH][NR]) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
        const int k = kk[c] < K ? kk[c] : 0;
#pragma unroll
        for (int r = 0; r < NR; ++r) w[c][r].load(base + (int64_t)r * rstride + k);
    }
}

}  // namespace

// KH: chunks of 2048 over the hidden size; KQ over n_heads * d; KI over the FFN width.
template <int KH, int KQ, int KI, int G, bool MERGE>
__global__ __launch_bounds__(256) void step_fused_kernel(StepFusedArgs a, RowsArgs ra, uint64_t* clk) {
    __shared__ float red_q[4][NRQ + 1];
    __shared__ float red_o[4][NRO + 1];
    __shared__ float red_f[4][2 * NCF + 1];
    __shared__ float vals_f[2 * NCF];
    __shared__ float red_d[4][NRD + 1];
    clock_begin(clk);
    const int nwg = gridDim.x, wg = blockIdx.x, t = threadIdx.x;
    const int H = a.H, I = a.I, qd = a.n_heads * a.d, kvd = a.n_kv * a.d;
    const uint16_t* attn_norm = (const uint16_t*)a.attn_norm;
    const uint16_t* ffn_norm = (const uint16_t*)a.ffn_norm;

    // ---- Q: RMSNorm(x) * g, then 8 rows of Q|K|V per item
    {
        int kk[KH];
        chunk_offsets(kk);
        float xv[KH][1][8], ss[1];
        auto issue = [&](int it, Raw8<BF16> (&w)[KH][NRQ]) {
            const int n0 = it * NRQ;
            const uint16_t* W = n0 >= qd + kvd ? (const uint16_t*)a.wv + (int64_t)(n0 - qd - kvd) * H
                              : n0 >= qd       ? (const uint16_t*)a.wk + (int64_t)(n0 - qd) * H
                                               : (const uint16_t*)a.wq + (int64_t)n0 * H;
            load_rows<KH, NRQ>(W, H, H, kk, w);
        };
        auto ready = [&]() { load_activations<BF16, KH, 1, true>(a.x, H, 1, H, attn_norm, kk, xv, ss); };
        auto compute = [&](int it, Raw8<BF16> (&w)[KH][NRQ]) {
            float acc[NRQ], dot, rs[1];
            chunk_dots<BF16, KH, NRQ, 1>(w, xv, acc);
            block_merge<NRQ, 1, true>(acc, ss, red_q, H, a.eps, dot, rs);
            if (t < NRQ) PubMem::st(a.qkv + it * NRQ + t, dot * rs[0]);
            __syncthreads();
        };
        run_items<KH, NRQ>(wg, (qd + 2 * kvd) / NRQ, nwg, issue, ready, compute);
    }
    stage_signal(a.sync, 0);

    // ---- A: Q/K norm, RoPE, cache write and attention, one (KV head, split) per item
    {
        const int n = a.n_kv * a.n_splits;
        if (wg < n) stage_wait(a.sync, 0, nwg, a.err);
        for (int it = wg; it < n; it += nwg) {
            attn_rows_item<F16, BF16, 128, G, 4, true, PubMem>(ra, 0, it / a.n_splits, it % a.n_splits);
            __syncthreads();
        }
    }
    stage_signal(a.sync, 1);

    // ---- O: h = x + attn W_o^T, 4 rows per item
    {
        int kk[KQ];
        chunk_offsets(kk);
        float xv[KQ][1][8], ss[1] = {0.f};
        auto issue = [&](int it, Raw8<BF16> (&w)[KQ][NRO]) {
            load_rows<KQ, NRO>((const uint16_t*)a.wo + (int64_t)it * NRO * qd, qd, qd, kk, w);
        };
        auto ready = [&]() {
            stage_wait(a.sync, 1, nwg, a.err);
            if (MERGE) {
                GemvArgs g{};
                g.K = qd; g.xpart = a.part; g.n_splits = a.n_splits; g.head_dim = a.d;
                load_activations_merged<KQ, 1>(g, 0, 1, kk, xv);
            } else {
                load_activations<BF16, KQ, 1, false>(a.attn_o, qd, 1, qd, nullptr, kk, xv, ss);
            }
        };
        auto compute = [&](int it, Raw8<BF16> (&w)[KQ][NRO]) {
            float acc[NRO], dot, rs[1];
            chunk_dots<BF16, KQ, NRO, 1>(w, xv, acc);
            block_merge<NRO, 1, false>(acc, ss, red_o, qd, a.eps, dot, rs);
            if (t < NRO) PubMem::st(a.h + it * NRO + t, a.x[it * NRO + t] + dot);
            __syncthreads();
        };
        run_items<KQ, NRO>(wg, H / NRO, nwg, issue, ready, compute);
    }
    stage_signal(a.sync, 2);

    // ---- F: RMSNorm(h) * g, 4 gate rows + the 4 matching up rows per item, SwiGLU
    {
        int kk[KH];
        chunk_offsets(kk);
        float xv[KH][1][8], ss[1];
        auto issue = [&](int it, Raw8<BF16> (&w)[KH][2 * NCF]) {
            const uint16_t* W = (const uint16_t*)a.w_gate_up + (int64_t)it * NCF * H;
#pragma unroll
            for (int c = 0; c < KH; ++c) {
                const int k = kk[c] < H ? kk[c] : 0;
#pragma unroll
                for (int r = 0; r < NCF; ++r) {
                    w[c][r].load(W + (int64_t)r * H + k);
                    w[c][NCF + r].load(W + (int64_t)(I + r) * H + k);
                }
            }
        };
        auto ready = [&]() {
            stage_wait(a.sync, 2, nwg, a.err);
            load_activations<BF16, KH, 1, true>(a.h, H, 1, H, ffn_norm, kk, xv, ss);
        };
        auto compute = [&](int it, Raw8<BF16> (&w)[KH][2 * NCF]) {
            float acc[2 * NCF], dot, rs[1];
            chunk_dots<BF16, KH, 2 * NCF, 1>(w, xv, acc);
            block_merge<2 * NCF, 1, true>(acc, ss, red_f, H, a.eps, dot, rs);
            if (t < 2 * NCF) vals_f[t] = dot;
            __syncthreads();
            if (t < NCF) {
                const float gt = vals_f[t] * rs[0], up = vals_f[NCF + t] * rs[0];
                PubMem::st(a.act + it * NCF + t, gt / (1.0f + expf(-gt)) * up);
            }
            __syncthreads();
        };
        run_items<KH, 2 * NCF>(wg, I / NCF, nwg, issue, ready, compute);
    }
    stage_signal(a.sync, 3);

    // ---- D: x = h + act W_down^T, 4 rows per item (x was last read in stage Q)
    {
        int kk[KI];
        chunk_offsets(kk);
        float xv[KI][1][8], ss[1] = {0.f};
        auto issue = [&](int it, Raw8<BF16> (&w)[KI][NRD]) {
            load_rows<KI, NRD>((const uint16_t*)a.w_down + (int64_t)it * NRD * I, I, I, kk, w);
        };
        auto ready = [&]() {
            stage_wait(a.sync, 3, nwg, a.err);
            load_activations<BF16, KI, 1, false>(a.act, I, 1, I, nullptr, kk, xv, ss);
        };
        auto compute = [&](int it, Raw8<BF16> (&w)[KI][NRD]) {
            float acc[NRD], dot, rs[1];
            chunk_dots<BF16, KI, NRD, 1>(w, xv, acc);
            block_merge<NRD, 1, false>(acc, ss, red_d, I, a.eps, dot, rs);
            if (t < NRD) a.x[it * NRD + t] = a.h[it * NRD + t] + dot;  // read by the next launch
            __syncthreads();
        };
        run_items<KI, NRD>(wg, H / NRD, nwg, issue, ready, compute);
    }
    step_exit(a.sync, nwg);
    clock_end(clk);
}

namespace {

typedef void (*StepKernel)(StepFusedArgs, RowsArgs, uint64_t*);

template <int KH, int KQ, int KI, int G>
StepKernel pick_merge(bool merge) {
    return merge ? step_fused_kernel<KH, KQ, KI, G, true> : step_fused_kernel<KH, KQ, KI, G, false>;
}

int chunks(int K) { return (K + 4 * CHUNK - 1) / (4 * CHUNK); }

// Built shapes: hidden and n_heads * d up to 2048 (one chunk), FFN width up to
// 8192, GQA groups 1, 2, 4, 8.
StepKernel pick(const StepFusedArgs& a) {
    if (chunks(a.H) != 1 || chunks(a.n_heads * a.d) != 1) return nullptr;
    const bool m = a.n_splits > 1;
    const int g = a.n_heads / a.n_kv;
#define PICK_I(KI_)                                                       \
    switch (g) {                                                          \
        case 1: return pick_merge<1, 1, KI_, 1>(m);                       \
        case 2: return pick_merge<1, 1, KI_, 2>(m);                       \
        case 4: return pick_merge<1, 1, KI_, 4>(m);                       \
        case 8: return pick_merge<1, 1, KI_, 8>(m);                       \
        default: return nullptr;                                          \
    }
    switch (chunks(a.I)) {
        case 1: PICK_I(1)
        case 2: PICK_I(2)
        case 3: PICK_I(3)
        case 4: PICK_I(4)
        default: return nullptr;
    }
#undef PICK_I
}

}  // namespace

bool step_fused_supported(int H, int n_heads, int n_kv, int d, int I, int n_splits, WType wt, KVType kt) {
    if (wt != W_BF16 || kt != KV_F16 || d != 128) return false;
    if (n_splits < 1 || n_splits > kMergeMaxSplits) return false;
    if (H % (NRQ * 4) || H % NRO || H % NRD || I % NCF || (n_heads * d) % NRQ) return false;
    StepFusedArgs a{};
    a.H = H; a.n_heads = n_heads; a.n_kv = n_kv; a.d = d; a.I = I; a.n_splits = n_splits;
    return pick(a) != nullptr;
}

hipError_t launch_step_fused(const StepFusedArgs& a, hipStream_t s) {
    StepKernel k = pick(a);
    if (!k || !a.rm.pos || !a.rm.seq || !a.sync) return hipErrorInvalidValue;
    // Every workgroup must be resident at once: at most what the occupancy
    // allows (two per CU suffice), and no more than 512, the items of the
    // 1.7B shape's Q, O and down stages.
    struct GridOf {
        StepKernel k;
        int dev, grid;
    };
    static std::mutex mu;
    static std::vector<GridOf> grids;  // per (kernel, device)
    int dev = 0, grid = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    {
        std::lock_guard<std::mutex> lk(mu);
        for (const auto& g : grids)
            if (g.k == k && g.dev == dev) grid = g.grid;
        if (!grid) {
            int cus = 0, per_cu = 0;
            e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
            if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)k, 256, 0);
            if (e != hipSuccess) return e;
            if (per_cu < 1 || cus < 1) return hipErrorInvalidValue;
            grid = min(cus * min(per_cu, 2), 512);
            grids.push_back({k, dev, grid});
        }
    }
    RowsArgs ra{};
    ra.q = a.qkv; ra.ldq = a.n_heads * a.d + 2 * a.n_kv * a.d; ra.n_heads = a.n_heads; ra.rm = a.rm; ra.kv = a.kv;
    ra.n_splits = a.n_splits; ra.part = a.part; ra.out_f32 = a.n_splits > 1 ? nullptr : a.attn_o;
    ra.ldo = a.n_heads * a.d; ra.err = a.err; ra.q_gain = a.q_norm; ra.k_gain = a.k_norm; ra.eps = a.eps;
    ra.rope = a.rope; ra.max_pos = a.max_pos;
    launch_kernel(k, grid, 256, 0, s, a, ra, clock_slot());
    return hipGetLastError();
}

}  // namespace sttd
