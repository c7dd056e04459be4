// kernels_gemv.hip - bandwidth-bound projections for decode rows (and the
// fp32-weight path): y = x W^T over a few activation rows, with the block's
// RMSNorm fused in front and residual / SwiGLU / argmax fused behind.
//
// Layout: W is [N, K] row-major (bf16 or fp32). A workgroup of 4 waves owns
// NR weight rows; the K axis is dealt to the waves in 512-element chunks
// (wave w takes chunks w, w+4, ...), and in each chunk lane l reads the 8
// consecutive elements at 8l with one 16-byte load per row (bf16), so a wave
// reads 1 KB of a row per instruction, fully coalesced. Every weight load of
// the workgroup is issued before anything waits on memory: addresses are
// clamped instead of branched around, and the RMSNorm statistics come from
// the same activation chunks the dot products use, summed in the one LDS
// reduction that also merges the waves' partial dot products (a butterfly
// leaves one (row, activation-row) sum per lane group). Activations are fp32
// and stay fp32: products are exact, accumulation is fp32. BT activation rows
// per workgroup; more tile blockIdx.y.
#include "common.h"
#include "gemv_ops.h"
#include "launch.h"

namespace sttd {

template <class WT, int EPI, int BT, int NR, int KCH, bool NORM, bool XPART>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
    typedef typename WT::T T;
    constexpr int V = NR * BT;
    __shared__ float red[4][V + BT];
    __shared__ float vals[V];
    clock_begin(a.clk);
    const int lane = threadIdx.x % WAVE, wave = threadIdx.x / WAVE, t = threadIdx.x;
    const int b0 = blockIdx.y * BT;
    const int nb = min(BT, a.rows - b0);
    const float* x = a.x + (int64_t)b0 * a.ldx;

    // weight rows of this workgroup (clamped to valid rows)
    const T* wr[NR];
    int n0;
    if (EPI == GEMV_SWIGLU) {
        constexpr int NP = NR / 2;
        n0 = blockIdx.x * NP;
        const T* W = (const T*)a.w[0];
#pragma unroll
        for (int r = 0; r < NP; ++r) {
            const int n = min(n0 + r, a.N - 1);
            wr[r] = W + (int64_t)n * a.K;
            wr[NP + r] = W + (int64_t)(n + a.N) * a.K;
        }
    } else {
        n0 = blockIdx.x * NR;
        const bool s2 = n0 >= a.seg_end[1], s1 = n0 >= a.seg_end[0];
        const int start = s2 ? a.seg_end[1] : (s1 ? a.seg_end[0] : 0);
        const int end = s2 ? a.seg_end[2] : (s1 ? a.seg_end[1] : a.seg_end[0]);
        const T* W = (const T*)(s2 ? a.w[2] : (s1 ? a.w[1] : a.w[0]));
#pragma unroll
        for (int r = 0; r < NR; ++r) wr[r] = W + (int64_t)(min(n0 + r, end - 1) - start) * a.K;
    }
    // 1. every weight load of the workgroup, in flight at once
    int kk[KCH];
    Raw8<WT> w[KCH][NR];
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
        kk[c] = (c * 4 + wave) * CHUNK + lane * 8;
        const int k = kk[c] < a.K ? kk[c] : 0;
#pragma unroll
        for (int r = 0; r < NR; ++r) w[c][r].load(wr[r] + k);
    }
    // 2. activations (and the RMSNorm statistics) of the same chunks
    float xv[KCH][BT][8], ss[BT];
    if (XPART) {
        load_activations_merged<KCH, BT>(a, b0, nb, kk, xv);
#pragma unroll
        for (int b = 0; b < BT; ++b) ss[b] = 0.f;
    } else {
        load_activations<WT, KCH, BT, NORM>(x, a.ldx, nb, a.K, (const T*)a.gain, kk, xv, ss);
    }
    // 3. dot products, merged over the waves
    float acc[V];
    chunk_dots<WT, KCH, NR, BT>(w, xv, acc);
    float dot, rs[BT];
    block_merge<V, BT, NORM>(acc, ss, red, a.K, a.eps, dot, rs);

    if (EPI == GEMV_SWIGLU) {
        if (t < V) vals[t] = dot;
        __syncthreads();
        constexpr int NP = NR / 2;
        if (t < NP * BT) {
            const int r = t / BT, b = t % BT;
            if (b < nb && n0 + r < a.N) {
                const float gt = vals[r * BT + b] * rs[b];
                const float up = vals[(NP + r) * BT + b] * rs[b];
                a.y[(int64_t)(b0 + b) * a.ldy + n0 + r] = gt / (1.0f + expf(-gt)) * up;
            }
        }
        clock_end(a.clk);
        return;
    }
    if (t < V) {
        const int r = t / BT, b = t % BT;
        if (b < nb && n0 + r < a.N) {
            float v = dot * rs[b];
            const int64_t row = b0 + b;
            if (EPI == GEMV_RESID) v += a.resid[row * a.ldr + n0 + r];
            a.y[row * a.ldy + n0 + r] = v;
        }
    }
    clock_end(a.clk);
}

template <class WT, int EPI, int NR, int KCH, bool NORM, bool XPART>
static void launch_bt(const GemvArgs& a, hipStream_t s) {
    const int per_wg = EPI == GEMV_SWIGLU ? NR / 2 : NR;
    dim3 grid((a.N + per_wg - 1) / per_wg, 1);
    if (a.rows == 1) {
        launch_kernel(gemv_kernel<WT, EPI, 1, NR, KCH, NORM, XPART>, grid, 256, 0, s, a);
    } else if (a.rows == 2) {
        launch_kernel(gemv_kernel<WT, EPI, 2, NR, KCH, NORM, XPART>, grid, 256, 0, s, a);
    } else {
        grid.y = (a.rows + 3) / 4;
        launch_kernel(gemv_kernel<WT, EPI, 4, NR, KCH, NORM, XPART>, grid, 256, 0, s, a);
    }
}

template <class WT, int EPI, int NR, bool NORM, bool XPART = false>
static hipError_t launch_k(const GemvArgs& a, hipStream_t s) {
    const int kch = (a.K + 4 * CHUNK - 1) / (4 * CHUNK);
    switch (kch) {
        case 1: launch_bt<WT, EPI, NR, 1, NORM, XPART>(a, s); break;
        case 2: launch_bt<WT, EPI, NR, 2, NORM, XPART>(a, s); break;
        case 3: launch_bt<WT, EPI, NR, 3, NORM, XPART>(a, s); break;
        case 4: launch_bt<WT, EPI, NR, 4, NORM, XPART>(a, s); break;
        default: return hipErrorInvalidValue;  // K > 8192
    }
    return hipGetLastError();
}

// Weight rows per workgroup of the RESID projections without a split merge (the
// down projection of a decode row): 4 measured best on the 28-block greedy job
// (down 5.97 us with 2 rows, 5.64 with 4, 6.73 with 1)
// Weight rows per workgroup of the SwiGLU projection (gate and up rows of half as
// many act columns): 4 measured 9.50 us for a decode row, 8 measured 10.28, 2 9.96
#ifndef STTD_GEMV_SWIGLU_NR
#define STTD_GEMV_SWIGLU_NR 4
#endif
#ifndef STTD_GEMV_RESID_NR
#define STTD_GEMV_RESID_NR 4
#endif

template <class WT>
static hipError_t launch_wt(const GemvArgs& a, GemvEpi epi, hipStream_t s) {
    // Rows per workgroup, measured on the decode shapes: more, shorter workgroups
    // overlap one another's load latency and reduction tails better than fewer,
    // wider ones (2-4 rows beat 8-16 by 10-40%). A fixed grid of 256-1024
    // workgroups walking the tiles (activations loaded once, the next tile's
    // weights in flight while one reduces) measured slower on every projection
    // (gate_up 9.6 -> 9.9-13.6 us, QKV 4.2 -> 5.0-6.7 us).
    const bool norm = a.gain != nullptr;
    if (epi == GEMV_SWIGLU)
        return norm ? launch_k<WT, GEMV_SWIGLU, STTD_GEMV_SWIGLU_NR, true>(a, s)
                    : launch_k<WT, GEMV_SWIGLU, STTD_GEMV_SWIGLU_NR, false>(a, s);
    if (epi == GEMV_RESID) {
        // merging the attention splits on load costs n_splits times the activation
        // reads of a plain row, so fewer, wider workgroups pay it fewer times
        if (a.xpart) return launch_k<WT, GEMV_RESID, 8, false, true>(a, s);
        return norm ? launch_k<WT, GEMV_RESID, STTD_GEMV_RESID_NR, true>(a, s)
                    : launch_k<WT, GEMV_RESID, STTD_GEMV_RESID_NR, false>(a, s);
    }
    return norm ? launch_k<WT, GEMV_STORE, 4, true>(a, s) : launch_k<WT, GEMV_STORE, 4, false>(a, s);
}

hipError_t launch_gemv(const GemvArgs& args, WType wt, GemvEpi epi, hipStream_t s) {
    if (args.rows <= 0 || args.N <= 0) return hipSuccess;
    GemvArgs a = args;
    a.clk = clock_slot();
    return wt == W_BF16 ? launch_wt<BF16>(a, epi, s) : launch_wt<F32>(a, epi, s);
}

// ------------------------------------------------------------------ lm_head + argmax
// Final RMSNorm and the tied head (build_step_graph on the Qwen3-ASR decoder
// page: logits = E * (RMSNorm(x) * g), then argmax on device). A persistent
// grid walks the vocabulary in blocks of NR rows, fetching the next block's
// weights while it finishes the current one. Each workgroup keeps, per
// activation row, its best (logit, index) as the 64-bit key
// (order-preserving bits of the logit) << 32 | ~index, so the larger logit
// wins and, among equal logits, the lower index (the strict greater-than scan
// of run() on the model page), and writes it to a partials array;
// lm_head_finalize reduces them, writes the ids, gathers the next input rows
// E[id] and bumps the positions. No atomics, nothing to re-arm. (512 or 768
// workgroups instead of 1024 measured the same: 107.6-111.4 against 109.6 us.)
template <class WT, int BT, int NR, int KCH>
__global__ __launch_bounds__(256) void lm_head_kernel(HeadArgs a) {
    typedef typename WT::T T;
    constexpr int V = NR * BT;
    __shared__ float red[4][V + BT];
    __shared__ unsigned long long keys[V];
    clock_begin(a.clk);
    const int lane = threadIdx.x % WAVE, wave = threadIdx.x / WAVE, t = threadIdx.x;
    const int b0 = blockIdx.y * BT;
    const int nb = min(BT, a.rows - b0);
    // activation row of each of this workgroup's rows (the caller's row index, if any)
    const float* xr[BT];
#pragma unroll
    for (int b = 0; b < BT; ++b) {
        int src = b0 + (b < nb ? b : 0);
        if (a.xrow) {
            src = a.xrow[src];
            if (src < 0 || src >= a.n_xrows) {
                if (b < nb && blockIdx.x == 0 && t == 0) record_error(a.err, kDevErrRow);
                src = 0;
            }
        }
        xr[b] = a.x + (int64_t)src * a.ldx;
    }
    const T* E = (const T*)a.embed;
    const int n_blocks = (a.vocab + NR - 1) / NR;

    int kk[KCH];
#pragma unroll
    for (int c = 0; c < KCH; ++c) kk[c] = (c * 4 + wave) * CHUNK + lane * 8;
    auto fetch = [&](int blk, Raw8<WT> (&w)[KCH][NR]) {
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const int k = kk[c] < a.hidden ? kk[c] : 0;
#pragma unroll
            for (int r = 0; r < NR; ++r) w[c][r].load(E + (int64_t)min(blk * NR + r, a.vocab - 1) * a.hidden + k);
        }
    };
    Raw8<WT> wc[KCH][NR], wn[KCH][NR];
    int blk = blockIdx.x;
    if (blk < n_blocks) fetch(blk, wc);
    float xv[KCH][BT][8], ss[BT];
    load_activation_rows<WT, KCH, BT, true>(xr, nb, a.hidden, (const T*)a.gain, kk, xv, ss);
    float rs[BT];
    {
        // row scales once per workgroup
#pragma unroll
        for (int b = 0; b < BT; ++b) {
            const float s = wave_sum(ss[b]);
            if (lane == 0) red[wave][b] = s;
        }
        __syncthreads();
#pragma unroll
        for (int b = 0; b < BT; ++b)
            rs[b] = 1.0f / sqrtf((red[0][b] + red[1][b] + red[2][b] + red[3][b]) / (float)a.hidden + a.eps);
        __syncthreads();
    }
    unsigned long long best = 0ull;  // thread t < BT: best key of activation row t
    for (; blk < n_blocks; blk += gridDim.x) {
        const int nxt = blk + gridDim.x;
        if (nxt < n_blocks) fetch(nxt, wn);
        float acc[V];
        chunk_dots<WT, KCH, NR, BT>(wc, xv, acc);
        float dot, dummy[BT];
        float no_ss[BT];
#pragma unroll
        for (int b = 0; b < BT; ++b) no_ss[b] = 0.f;
        block_merge<V, BT, false>(acc, no_ss, red, a.hidden, a.eps, dot, dummy);
        if (t < V) {
            const int r = t / BT, b = t % BT;
            unsigned long long key = 0ull;
            const int n = blk * NR + r;
            if (b < nb && n < a.vocab) {
                const float v = dot * rs[b];
                key = ((unsigned long long)float_order_key(v) << 32) | (unsigned long long)(~(uint32_t)n);
                if (a.logits) a.logits[(int64_t)(b0 + b) * a.vocab + n] = v;
            }
            keys[t] = key;
        }
        __syncthreads();
        if (t < BT) {
#pragma unroll
            for (int r = 0; r < NR; ++r) best = keys[r * BT + t] > best ? keys[r * BT + t] : best;
        }
#pragma unroll
        for (int c = 0; c < KCH; ++c)
#pragma unroll
            for (int r = 0; r < NR; ++r) wc[c][r] = wn[c][r];
    }
    if (t < nb) a.partials[(int64_t)(b0 + t) * gridDim.x + blockIdx.x] = best;
    clock_end(a.clk);
}

// One workgroup per activation row: reduce the partial keys, emit the id.
template <class WT>
__global__ __launch_bounds__(256) void lm_head_finalize_kernel(HeadArgs a, int n_partials) {
    typedef typename WT::T T;
    __shared__ unsigned long long red[4];
    __shared__ int id_lds;
    clock_begin(a.clk, 1);
    const int b = blockIdx.x;
    const int lane = threadIdx.x % WAVE, wave = threadIdx.x / WAVE;
    unsigned long long best = 0ull;
    for (int i = threadIdx.x; i < n_partials; i += 256) {
        const unsigned long long k = a.partials[(int64_t)b * n_partials + i];
        best = k > best ? k : best;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const unsigned long long o = __shfl_xor(best, off, WAVE);
        best = o > best ? o : best;
    }
    if (lane == 0) red[wave] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long m = red[0];
        for (int w = 1; w < 4; ++w) m = red[w] > m ? red[w] : m;
        const int id = (int)(~(uint32_t)(m & 0xFFFFFFFFull));
        id_lds = id;
        a.ids[b] = id;
        if (a.pos) a.pos[b] += 1;
    }
    __syncthreads();
    if (a.next_x) {
        const int id = id_lds;
        const bool ok = id >= 0 && id < a.vocab;
        if (!ok && threadIdx.x == 0) record_error(a.err, 4u);
        const T* E = (const T*)a.embed;
        float* xr = a.next_x + (int64_t)b * a.hidden;
        for (int i = threadIdx.x; i < a.hidden; i += 256) xr[i] = ok ? WT::ld(E, (int64_t)id * a.hidden + i) : 0.f;
    }
    clock_end(a.clk, 1);
}

// Vocabulary rows per block of the persistent head (each workgroup fetches the
// next block while it reduces one): 4 measured 105.3 us per single-row head on
// the 28-block greedy job, 8 measured 111.0 and 16 measured 127.9.
#ifndef STTD_HEAD_NR
#define STTD_HEAD_NR 4
#endif

template <class WT, int KCH>
static void launch_head_k(const HeadArgs& a, dim3 grid, hipStream_t s) {
    constexpr int NR = STTD_HEAD_NR;
    if (a.rows == 1) launch_kernel(lm_head_kernel<WT, 1, NR, KCH>, grid, 256, 0, s, a);
    else if (a.rows == 2) launch_kernel(lm_head_kernel<WT, 2, NR, KCH>, grid, 256, 0, s, a);
    else {
        grid.y = (a.rows + 3) / 4;
        launch_kernel(lm_head_kernel<WT, 4, NR, KCH>, grid, 256, 0, s, a);
    }
}

template <class WT>
static hipError_t launch_head_wt(const HeadArgs& a, hipStream_t s) {
    constexpr int NR = STTD_HEAD_NR;
    const int n_blocks = (a.vocab + NR - 1) / NR;
    const int grid_x = n_blocks < a.max_partials ? n_blocks : a.max_partials;
    const dim3 grid(grid_x, 1);
    switch ((a.hidden + 4 * CHUNK - 1) / (4 * CHUNK)) {
        case 1: launch_head_k<WT, 1>(a, grid, s); break;
        case 2: launch_head_k<WT, 2>(a, grid, s); break;
        case 3: launch_head_k<WT, 3>(a, grid, s); break;
        case 4: launch_head_k<WT, 4>(a, grid, s); break;
        default: return hipErrorInvalidValue;
    }
    launch_kernel(lm_head_finalize_kernel<WT>, a.rows, 256, 0, s, a, grid_x);
    return hipGetLastError();
}


// Batches of rows (bf16 embedding): the normed rows z = RMSNorm(x) * g are
// first rounded to bf16 high and low parts, then a weight-stationary MFMA
// pass streams the embedding once for up to 16 rows: each workgroup walks
// vocabulary tiles of 32 rows; each wave holds the A fragments (rows x its
// quarter of K, high and low) in registers for the whole walk and feeds the
// tile's embedding rows straight from global memory as B fragments, the next
// tile's already in flight while a tile is computed and reduced. The
// waves' partial logits meet in LDS; each thread keeps the best key of its
// activation row over its two columns of every tile, and the 16 threads of a
// row merge their keys at the end into the workgroup's partial.
template <int KSW>
__global__ __launch_bounds__(256) void head_mfma_kernel(HeadArgs a, const uint16_t* __restrict__ zh,
                                                        const uint16_t* __restrict__ zl, int b0, int nb) {
    constexpr int PD = KSW < 8 ? KSW : 8;  // K-steps of embedding loads in flight per wave
    __shared__ float red[4][16][33];
    clock_begin(a.clk);
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int n_steps = a.hidden / 32;
    const int per = (n_steps + 3) / 4;
    const int s0 = min(wave * per, n_steps), s1 = min(s0 + per, n_steps);
    const int koff = (lane / 16) * 8;
    // A fragments of this wave's K steps, rows b0 + lane % 16 (clamped)
    u32x4 ah[KSW], al[KSW];
    {
        const int row = min(lane % 16, nb - 1);
#pragma unroll
        for (int i = 0; i < KSW; ++i) {
            const int k = min(s0 + i, n_steps - 1) * 32 + koff;
            ah[i] = *reinterpret_cast<const u32x4*>(zh + (int64_t)row * a.hidden + k);
            al[i] = *reinterpret_cast<const u32x4*>(zl + (int64_t)row * a.hidden + k);
        }
        // steps past this wave's share multiply zeros: the step loop below has no
        // branch (one would let the compiler sink each load to its use, unbatched)
#pragma unroll
        for (int i = 0; i < KSW; ++i)
            if (s0 + i >= s1) ah[i] = al[i] = u32x4{0u, 0u, 0u, 0u};
    }
    const uint16_t* E = (const uint16_t*)a.embed;
    const int n_tiles = (a.vocab + 31) / 32;
    const int my_row = tid / 16, my_col = (tid % 16) * 2;
    unsigned long long best = 0ull;
    // batch b (PD K-steps) of a tile's 32 embedding rows (clamped to the last tile and
    // the last vocabulary row), addressed from the base each time
    constexpr int NB = KSW / PD;
    u32x4 wb[NB][PD][2];
    auto fetch = [&](int tile, int b) {
        const int t = min(tile, n_tiles - 1);
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const int64_t row = min(t * 32 + f * 16 + lane % 16, a.vocab - 1);
#pragma unroll
            for (int p = 0; p < PD; ++p)
                wb[b][p][f] = *reinterpret_cast<const u32x4*>(E + row * a.hidden + koff +
                                                              min(s0 + b * PD + p, n_steps - 1) * 32);
        }
    };
    // every batch of the next tile is fetched as soon as this tile's MFMAs have used
    // its registers, so a whole tile is in flight while one is computed and reduced;
    // the fences keep each batch issued whole (left alone, the compiler issues one
    // load at a time, each waited on at once)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        fetch(blockIdx.x, b);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
        f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
            for (int p = 0; p < PD; ++p) {
#pragma unroll
                for (int f = 0; f < 2; ++f) {
                    const bf16x8 bw = __builtin_bit_cast(bf16x8, wb[b][p][f]);
                    acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ah[b * PD + p]), bw,
                                                                     acc[f], 0, 0, 0);
                    acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, al[b * PD + p]), bw,
                                                                     acc[f], 0, 0, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            fetch(tile + gridDim.x, b);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave][(lane / 16) * 4 + i][f * 16 + lane % 16] = acc[f][i];
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int col = my_col + c, n = tile * 32 + col;
            const float v = red[0][my_row][col] + red[1][my_row][col] + red[2][my_row][col] + red[3][my_row][col];
            if (my_row < nb && n < a.vocab) {
                const unsigned long long key =
                    ((unsigned long long)float_order_key(v) << 32) | (unsigned long long)(~(uint32_t)n);
                best = key > best ? key : best;
                if (a.logits) a.logits[(int64_t)(b0 + my_row) * a.vocab + n] = v;
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) {
        const unsigned long long o = __shfl_xor(best, off, WAVE);
        best = o > best ? o : best;
    }
    if (tid % 16 == 0 && my_row < nb) a.partials[(int64_t)(b0 + my_row) * gridDim.x + blockIdx.x] = best;
    clock_end(a.clk);
}

// Workgroups of the MFMA head: one per CU, each walking ~19 vocabulary tiles with the
// next tile's loads in flight (16 rows: 112.9 us at 256 workgroups, 116.5 at 512, 131.4
// at 1024; 133.4 at 1024 before the cross-tile prefetch, when each K-step's loads were
// waited on at once and only the grid's width hid the latency)
#ifndef STTD_HEAD_MFMA_WGS
#define STTD_HEAD_MFMA_WGS 256
#endif
// MFMA head for batches: norm to bf16 planes, then 16-row chunks, then the finalize pass.
static hipError_t launch_head_mfma(const HeadArgs& a, hipStream_t s) {
    uint16_t* zh = a.zbuf;
    uint16_t* zl = a.zbuf + (size_t)a.rows * a.hidden;
    hipError_t e = launch_rmsnorm_rows_bf16(a.x, a.ldx, a.gain, W_BF16, zh, zl, a.hidden, a.rows, a.hidden, a.eps, s,
                                            a.xrow, a.n_xrows, a.err);
    if (e != hipSuccess) return e;
    const int n_tiles = (a.vocab + 31) / 32;
    const int cap = a.max_partials < STTD_HEAD_MFMA_WGS ? a.max_partials : STTD_HEAD_MFMA_WGS;
    const int grid = n_tiles < cap ? n_tiles : cap;
    const int ksw = (a.hidden / 32 + 3) / 4;
    for (int b0 = 0; b0 < a.rows; b0 += 16) {
        const int nb = a.rows - b0 < 16 ? a.rows - b0 : 16;
        const uint16_t* h = zh + (size_t)b0 * a.hidden;
        const uint16_t* l = zl + (size_t)b0 * a.hidden;
        if (ksw <= 4) launch_kernel(head_mfma_kernel<4>, grid, 256, 0, s, a, h, l, b0, nb);
        else if (ksw <= 8) launch_kernel(head_mfma_kernel<8>, grid, 256, 0, s, a, h, l, b0, nb);
        else launch_kernel(head_mfma_kernel<16>, grid, 256, 0, s, a, h, l, b0, nb);
    }
    launch_kernel(lm_head_finalize_kernel<BF16>, a.rows, 256, 0, s, a, grid);
    return hipGetLastError();
}

hipError_t launch_lm_head_argmax(const HeadArgs& args, WType wt, hipStream_t s) {
    if (args.rows <= 0) return hipSuccess;
    HeadArgs a = args;
    a.clk = clock_slot();
    if (wt == W_BF16 && a.zbuf && a.rows > 4 && a.hidden % 32 == 0 && a.hidden <= 2048) return launch_head_mfma(a, s);
    return wt == W_BF16 ? launch_head_wt<BF16>(a, s) : launch_head_wt<F32>(a, s);
}

}  // namespace sttd
