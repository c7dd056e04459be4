// kernels_attn.hip - causal grouped-query attention over the KV cache.
//
// Both kernels compute, for query head h of a row at position p,
//   o_h = sum_c softmax_c(q_h . K[c]_j / sqrt(d)) V[c]_j,  c = 0..p,
// with j = floor(h / (n_heads / n_kv)) the head's KV group (Qwen3-ASR decoder
// page, file header; the causal mask of run() on the model page keeps
// columns c <= r). Masked columns are never read, so no mask tensor exists.
// Exponentials run in base 2 on scores pre-scaled by log2(e)/sqrt(d).
#include "attn_rows.h"
#include "common.h"
#include "gemv_ops.h"
#include "launch.h"

namespace sttd {

// ------------------------------------------------------------------ rows attention (decode)
// The item body (attn_rows.h) runs one (row, KV head, split) per workgroup.
// PUB: the partials are published with device-scope stores, for the last split
// of a (row, KV head) to merge in this launch (RowsArgs::merge_ctr); otherwise
// plain stores, read by the next launch.
template <class KT, class GT, int D, int G, int NW, bool FUSE, bool PUB>
__global__ __launch_bounds__(NW * 64) void attn_rows_kernel(RowsArgs a) {
    clock_begin(a.clk);
    if (PUB) attn_rows_item<KT, GT, D, G, NW, FUSE, PubMem>(a, blockIdx.x, blockIdx.y, blockIdx.z);
    else attn_rows_item<KT, GT, D, G, NW, FUSE, PlainMem>(a, blockIdx.x, blockIdx.y, blockIdx.z);
    clock_end(a.clk);
}

// Merge the splits of each (row, query head): o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// Partial records are [m, l, -, -, o[D]] (D + 4 floats, 16-byte aligned).
template <int D>
__global__ __launch_bounds__(D) void attn_combine_kernel(const float* __restrict__ part, int n_heads, int n_splits,
                                                         float* __restrict__ out_f32, uint16_t* __restrict__ out_bf16,
                                                         uint16_t* __restrict__ out_lo, int64_t ldo, uint64_t* clk) {
    clock_begin(clk, 1);
    const int r = blockIdx.x, h = blockIdx.y, e = threadIdx.x;
    const float* pp = part + ((int64_t)r * n_heads + h) * n_splits * (D + 4);
    float M = -INFINITY;
#pragma unroll 16
    for (int s = 0; s < n_splits; ++s) M = fmaxf(M, pp[s * (D + 4)]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll 16
        for (int s = 0; s < n_splits; ++s) {
            const float w = exp2f(pp[s * (D + 4)] - M);
            L += w * pp[s * (D + 4) + 1];
            O += w * pp[s * (D + 4) + 4 + e];
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
    clock_end(clk, 1);
}

// Waves of a workgroup whose split spans more than 128 cache rows. 16 (1024 threads, 64
// lane groups per split) measured slower on 16 rows of 151-1535 positions: 14.3 -> 16.4
// us per launch, one 1535-position row alone 11.5 -> 13.4 us (the slot merge and the
// barriers grow with the waves); valid only for groups of up to 2 query heads, whose
// registers fit 4 waves per SIMD
// Split span (cache rows) above which a rows-attention workgroup has 8 waves, not 4:
// 160 lets the 4097-4352-position decode row's 32 splits of ~136 rows keep 4 waves
// (10.98 -> 10.86 us per launch, 405.5k -> 407k tok/s on that block's job)
#ifndef STTD_ATTN_WIDE_ROWS
#define STTD_ATTN_WIDE_ROWS 160
#endif
#ifndef STTD_ATTN_WIDE_NW
#define STTD_ATTN_WIDE_NW 8
#endif
template <class KT, class GT, int D, bool FUSE>
static hipError_t rows_dispatch(const RowsArgs& a, int R, bool wide, hipStream_t s) {
    const int G = a.n_heads / a.kv.n_kv;
    const dim3 grid(R, a.kv.n_kv, a.n_splits);
    // 4 waves per workgroup for groups of up to 2 query heads (the shorter merge tail beats
    // the extra rows in flight) unless a split spans more than STTD_ATTN_WIDE_ROWS cache rows; 8 for
    // larger groups
    const bool pub = a.merge_ctr != nullptr;
#define ROWS_LAUNCH(G_)                                                                             \
    do {                                                                                            \
        if (G_ <= 2 && !wide) {                                                                     \
            if (pub) launch_kernel(attn_rows_kernel<KT, GT, D, G_, 4, FUSE, true>, grid, 4 * 64, 0, s, a);     \
            else launch_kernel(attn_rows_kernel<KT, GT, D, G_, 4, FUSE, false>, grid, 4 * 64, 0, s, a);        \
        } else {                                                                                    \
            constexpr int NWW = STTD_ATTN_WIDE_NW;                                                      \
            if (pub) launch_kernel(attn_rows_kernel<KT, GT, D, G_, NWW, FUSE, true>, grid, NWW * 64, 0, s, a); \
            else launch_kernel(attn_rows_kernel<KT, GT, D, G_, NWW, FUSE, false>, grid, NWW * 64, 0, s, a);    \
        }                                                                                           \
    } while (0)
    switch (G) {
        case 1: ROWS_LAUNCH(1); break;
        case 2: ROWS_LAUNCH(2); break;
        case 4: ROWS_LAUNCH(4); break;
        case 8: ROWS_LAUNCH(8); break;
        default: return hipErrorInvalidValue;
    }
#undef ROWS_LAUNCH
    if (a.n_splits > 1 && (a.out_f32 || a.out_bf16) && !a.merge_ctr)
        launch_kernel(attn_combine_kernel<D>, dim3(R, a.n_heads), D, 0, s, a.part, a.n_heads, a.n_splits, a.out_f32, a.out_bf16,
                                                                a.out_lo, a.ldo, a.clk);
    return hipGetLastError();
}

template <class GT, bool FUSE>
static hipError_t rows_dispatch_kv(const RowsArgs& a, int R, bool wide, hipStream_t s) {
    if (a.kv.d == 128)
        return a.kv.type == KV_F16 ? rows_dispatch<F16, GT, 128, FUSE>(a, R, wide, s)
                                   : rows_dispatch<F32, GT, 128, FUSE>(a, R, wide, s);
    if (a.kv.d == 64)
        return a.kv.type == KV_F16 ? rows_dispatch<F16, GT, 64, FUSE>(a, R, wide, s)
                                   : rows_dispatch<F32, GT, 64, FUSE>(a, R, wide, s);
    return hipErrorInvalidValue;
}

hipError_t launch_attn_rows(const float* q, int64_t ldq, int R, int n_heads, RowMap rm, KVLayer kv, int n_splits,
                            int span_bound, float* part, float* out_f32, uint16_t* out_bf16, uint16_t* out_bf16_lo,
                            int64_t ldo, uint32_t* err, const QkRope* fuse, WType gt, hipStream_t s,
                            uint32_t* merge_ctr) {
    if (R <= 0) return hipSuccess;
    if (n_splits < 1 || n_splits > 64 || (fuse && (!rm.pos || !rm.seq))) return hipErrorInvalidValue;
    RowsArgs a{};
    a.q = q; a.ldq = ldq; a.n_heads = n_heads; a.rm = rm; a.kv = kv; a.n_splits = n_splits; a.part = part;
    a.out_f32 = out_f32; a.out_bf16 = out_bf16; a.out_lo = out_bf16_lo; a.ldo = ldo; a.err = err;
    // the last split merges up to kMergeMaxSplits splits itself (their G * n_splits
    // records staged in LDS), so no combine pass runs (measured: 2 splits of 16 rows,
    // 23.5 -> 22 us per block). With many splits every split's wait for its
    // write-through stores costs more than the combine launch (32 splits of one
    // 4200-row span: 13.8 us in-kernel against 11.6 us with the combine pass; with the
    // register-ring rows loop, 4097-4352 positions: 14.5 against 10.9 us).
    const int group = n_heads / kv.n_kv;
    a.merge_ctr = n_splits > 1 && n_splits <= kMergeMaxSplits && group * n_splits <= 64 && (out_f32 || out_bf16)
                      ? merge_ctr
                      : nullptr;
    a.clk = clock_slot();
    if (fuse) {
        a.q_gain = fuse->q_gain; a.k_gain = fuse->k_gain; a.eps = fuse->eps; a.rope = fuse->rope;
        a.max_pos = fuse->max_pos;
        const bool wide = span_bound > STTD_ATTN_WIDE_ROWS;
        return gt == W_BF16 ? rows_dispatch_kv<BF16, true>(a, R, wide, s) : rows_dispatch_kv<F32, true>(a, R, wide, s);
    }
    return rows_dispatch_kv<BF16, false>(a, R, false, s);
}

// ------------------------------------------------------------------ one decode row: projection + attention
// One launch for the Q|K|V projection of a single decode row and its attention.
// Workgroups [0, n_prod) each compute STTD_QA_NR columns of the fused-RMSNorm
// projection with the GEMV's arithmetic (the same loads, dot products and merge,
// so the values are bit-identical to the GEMV's), ordered KV head major: tiles
// j * TPH .. of head j are its G query heads' columns, then its key's, then its
// value's. Each column
// is published as one 64-bit word (tag << 32 | value bits) with a device-scope
// store. Workgroups [n_prod, n_prod + n_kv * n_splits) are the attention items
// (KV head, split): they load the position, rotation row and first cache rows,
// then poll their head's words until they carry the launch's tag (the word a
// launch's last consumer advances; attn_rows_item, TAGGED). Producers precede
// consumers in dispatch order, so a poll only ever waits on producers that are
// running or done; it still gives up after 200 ms and flags SYNC. Measured on
// the 1.7B shape (512 producers, 64 consumers): 8.5 us for the launch against
// 4.2 + 3.6 us for the two kernels and the ~1.5 us gap between them; the
// attention work left after the hand-off (the poll's round trip, the second
// half of each split's cache rows, the partials) is what remains exposed.
// Projection columns per producer workgroup: on the 28-block greedy job 8 (512
// producers) measured 8.51 us per launch, 4 measured 8.69 and 2 measured 10.1.
// Taking the O projection into this launch too (its workgroups polling per-split
// ready words) measured 20.7 us against 10.6 + 6.5 us for the two launches: they
// saw the last split's word 2-5 us after it was set, then needed 2.6 us more.
// Merging the splits in this launch instead (the last split of each KV head merges
// them, as the batched rows do) took the O projection from 4.58 to 2.54 us but this
// launch from 8.53 to 11.15 us: 949 -> 926 tok/s on the 28-block greedy job.
// Taking the split count per launch from the row's position (ceil((pos + 1) / 128)
// splits, so the O projection merges 2-4 records instead of 8 at 153-408 cached
// rows) took the O projection from 4.26 to 4.10 us but this launch from 8.54 to
// 9.42 us: eight short splits finish sooner than a few long ones (953 -> 932 tok/s).
// Fewer, longer attention splits (4 of 256 cache rows, or 2 of 512) halve what the
// O projection merges (4.51 -> 4.11 us) but lengthen this launch (8.45 -> 8.64 and
// 9.34 us): 950 against 943 and 918 tok/s, so splits stay at 128 rows.
#ifndef STTD_QA_NR
#define STTD_QA_NR 8
#endif

template <int KCH, int G, int D>
__global__ __launch_bounds__(256) void qkv_attn_kernel(QkvTagArgs p, RowsArgs a, int n_prod) {
    clock_begin(a.clk);
    const uint32_t tag = __builtin_amdgcn_readfirstlane(*a.tag_gen);
    if ((int)blockIdx.x < n_prod) {
        constexpr int NR = STTD_QA_NR, TQ = G * D / NR, TK = D / NR, TPH = TQ + 2 * TK;
        __shared__ float red[4][NR + 1];
        const int t = blockIdx.x, j = t / TPH, u = t % TPH;
        const uint16_t* W;
        int row0, col0;
        if (u < TQ) {
            W = p.wq; row0 = j * G * D + u * NR; col0 = row0;
        } else if (u < TQ + TK) {
            W = p.wk; row0 = j * D + (u - TQ) * NR; col0 = p.nq * D + row0;
        } else {
            W = p.wv; row0 = j * D + (u - TQ - TK) * NR; col0 = (p.nq + p.nkv) * D + row0;
        }
        const int lane = threadIdx.x % WAVE, wave = threadIdx.x / WAVE;
        int kk[KCH];
        Raw8<BF16> w[KCH][NR];
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            kk[c] = (c * 4 + wave) * CHUNK + lane * 8;
            const int k = kk[c] < p.K ? kk[c] : 0;
#pragma unroll
            for (int r = 0; r < NR; ++r) w[c][r].load(W + (int64_t)(row0 + r) * p.K + k);
        }
        float xv[KCH][1][8], ss[1];
        load_activations<BF16, KCH, 1, true>(p.x, p.K, 1, p.K, p.gain, kk, xv, ss);
        float acc[NR];
        chunk_dots<BF16, KCH, NR, 1>(w, xv, acc);
        float dot, rs[1];
        block_merge<NR, 1, true>(acc, ss, red, p.K, p.eps, dot, rs);
        if ((int)threadIdx.x < NR) {
            const float v = dot * rs[0];
            __hip_atomic_store(p.qtag + col0 + threadIdx.x, ((uint64_t)tag << 32) | __float_as_uint(v),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        clock_end(a.clk);
        return;
    }
    const int c = blockIdx.x - n_prod;
    RowsArgs b = a;
    b.tag = tag;
    attn_rows_item<F16, BF16, D, G, 4, true, PlainMem, true>(b, 0, c / a.n_splits, c % a.n_splits);
    clock_end(a.clk);
}

bool qkv_attn_fits(int n_heads, int n_kv, int d, int K, int n_splits, int span_bound, KVType kv) {
    const int G = n_kv > 0 ? n_heads / n_kv : 0;
    return kv == KV_F16 && d == 128 && (G == 1 || G == 2) && G * n_kv == n_heads && K % 8 == 0 && K <= 2 * 4 * CHUNK &&
           n_splits >= 1 && n_splits <= kMergeMaxSplits && span_bound <= 128;
}

hipError_t launch_qkv_attn(const QkvTagArgs& p, RowMap rm, KVLayer kv, int n_splits, int span_bound, float* part,
                           uint32_t* err, const QkRope& fuse, uint32_t* tag_gen, uint32_t* tag_done, hipStream_t s) {
    if (!qkv_attn_fits(p.nq, p.nkv, p.d, p.K, n_splits, span_bound, kv.type) || !rm.pos || !rm.seq)
        return hipErrorInvalidValue;
    RowsArgs a{};
    a.q = nullptr; a.ldq = (p.nq + 2 * p.nkv) * p.d; a.n_heads = p.nq; a.rm = rm; a.kv = kv; a.n_splits = n_splits;
    a.part = part; a.err = err;
    a.q_gain = fuse.q_gain; a.k_gain = fuse.k_gain; a.eps = fuse.eps; a.rope = fuse.rope; a.max_pos = fuse.max_pos;
    a.qtag = p.qtag; a.tag_gen = tag_gen; a.tag_done = tag_done; a.n_consumers = p.nkv * n_splits;
    a.clk = clock_slot();
    const int n_prod = (p.nq + 2 * p.nkv) * p.d / STTD_QA_NR;
    const int grid = n_prod + a.n_consumers;
    const int G = p.nq / p.nkv;
    const bool k1 = p.K <= 4 * CHUNK;
    if (G == 1) {
        if (k1) launch_kernel(qkv_attn_kernel<1, 1, 128>, grid, 256, 0, s, p, a, n_prod);
        else launch_kernel(qkv_attn_kernel<2, 1, 128>, grid, 256, 0, s, p, a, n_prod);
    } else {
        if (k1) launch_kernel(qkv_attn_kernel<1, 2, 128>, grid, 256, 0, s, p, a, n_prod);
        else launch_kernel(qkv_attn_kernel<2, 2, 128>, grid, 256, 0, s, p, a, n_prod);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------ causal prefill (MFMA flash)
// A workgroup takes the query tiles of 128 rows of one head in pairs, tile i
// and tile n - 1 - i, so every workgroup has the same causal work (when there
// are enough tiles to fill the chip; otherwise one tile each). Its 8 waves
// are 4 row groups of 32 query rows (two 16-row fragments) times 2 key groups:
// key group k takes keys 32k .. 32k + 31 of every 64-key block, so each K and
// V^T fragment read from LDS feeds two MFMAs (one per row fragment), half the
// LDS reads per MFMA of one 16-row fragment per wave. Per block and wave:
//   S^T = K Q^T     A: K rows staged in LDS; B: the wave's Q rows, in registers
//   online softmax; a lane owns one query row of each fragment
//   O^T += V^T P^T  A: V^T staged in LDS; B: P^T straight from the S^T registers
// At the end the second key group hands its (m, l, O) state to the first
// through LDS, which merges the two and writes the rows.
// Working on the transposes keeps every per-row quantity (max, sum, the O
// rescale) in the lanes that own the row. The S^T fragment gives lane l the
// keys 4g .. 4g + 3 (g = l / 16) of each 16-key tile, so V^T is staged with
// the keys of each 32-key group permuted to match the B operand: position
// 8g + j holds key 4g + j (j < 4) or 16 + 4g + j - 4 (j >= 4). K and V^T are
// double-buffered in LDS; the next block's rows load while the current one
// computes. Exponentials in base 2 on scores scaled by log2(e) / sqrt(d).
// One 16-row fragment per wave instead of two (64-row tiles, half the O and score
// registers) measured slower at 4096 rows: 121 -> 160 us, and 139 us with the
// registers held to 128 for two workgroups per CU (four waves per SIMD): each K and
// V^T fragment read then feeds one MFMA instead of two. Computing each block's
// scores one iteration ahead (K staged a block ahead of V, so the S MFMAs of block
// kb + 1 could overlap block kb's softmax; 240 VGPRs, no spills) measured slower
// too: 126 -> 130-135 us.
constexpr float kLazy = 8.f;  // lazy-rescale threshold of the flash kernel (base-2 exponent)

// SEG: packed sequences in one launch, sequence blockIdx.z of `sg` (rows, length,
// first position and slab from the table; its tiles are the first of gridDim.x,
// the workgroups past them leave at once).
template <int D, bool SEG>
__global__ __launch_bounds__(512) void attn_prefill_kernel(const uint16_t* __restrict__ q16, int64_t ldq, int T,
                                                           int pos0, int seq, int n_heads, KVLayer kv,
                                                           uint16_t* __restrict__ out, uint16_t* __restrict__ out_lo,
                                                           int64_t ldo, int paired, uint64_t* clk, Segments sg) {
    constexpr int NT = 512;                // 8 waves: 4 row groups x 2 key groups
    constexpr int RF = 2;                  // 16-row fragments per wave
    constexpr int KB = 64, TQ = 4 * 16 * RF;
    constexpr int KS = D;  // K and V rows unpadded; 16-byte chunks XOR-swizzled by the row (swz below)
    constexpr int KSTEPS = D / 32, DF = D / 16;
    constexpr int KVECS = KB * D / 8 / NT;                  // 16-byte K (and V) pieces per thread per block
    constexpr int HO = DF / 2 * RF * 4;                     // O values per lane in each half of the hand-over
    static_assert(HO * 256 * 4 <= 2 * KB * KS * 2, "hand-over fits the buffers");
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KB * KS];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][KB * KS];
    __shared__ float ml[2][RF][256];
    // element offset of 16-byte chunk c of an LDS row r of `stride` elements
    auto swz = [](int r, int c, int stride) { return r * stride + ((c ^ (r & 7)) * 8); };


    clock_begin(clk);
    if constexpr (SEG) {
        const int si = blockIdx.z, r0 = sg.start[si];
        q16 += (int64_t)r0 * ldq;
        out += (int64_t)r0 * ldo;
        if (out_lo) out_lo += (int64_t)r0 * ldo;
        T = sg.len[si];
        pos0 = sg.pos0[si];
        seq = sg.seq[si];
    }
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int g4 = lane / 16, r16 = lane % 16;
    const int kg = wave / 4, wr = wave % 4;  // key group, row group
    // XCD-aware order: workgroup b runs on XCD b % 8, so each XCD is given a
    // contiguous run of logical ids, KV head major; the XCD's workgroups then
    // re-read one KV head's rows, which stay in its L2, instead of all of them
    const int nx = gridDim.x, nwg = nx * gridDim.y, b = blockIdx.x + nx * blockIdx.y;
    const int L = nwg % 8 ? b : (b % 8) * (nwg / 8) + b / 8;
    const int G = n_heads / kv.n_kv;
    const int j = L / (G * nx), h = j * G + (L / nx) % G, px = L % nx;
    const int n_tiles = (T + TQ - 1) / TQ;
    const int64_t slab = ((int64_t)seq * kv.n_kv + j) * kv.n_ctx * D;
    const uint16_t* Kg = (const uint16_t*)kv.k + slab;
    const uint16_t* Vg = (const uint16_t*)kv.v + slab;
    const float sl2 = 1.4426950408889634f / sqrtf((float)D);

    for (int pass = 0; pass < 2; ++pass) {
        // paired: tiles x and n - 1 - x; otherwise one tile each, the heavy (late) ones first
        const int tile = !paired ? n_tiles - 1 - px : (pass == 0 ? px : n_tiles - 1 - px);
        if (pass == 1 && (!paired || tile <= px)) break;  // an odd count leaves the middle tile single
        if (tile < 0) break;                              // (SEG) past this sequence's tiles
        __syncthreads();                                  // the LDS buffers are free again
        const int t0 = tile * TQ + wr * 16 * RF;          // this wave's first query row

        // Q^T fragments (B operand): query row t0 + 16 rf + r16, dims 32 ks + 8 g4 ..
        f16x8 qf[RF][KSTEPS];
#pragma unroll
        for (int rf = 0; rf < RF; ++rf) {
            const int t = t0 + rf * 16 + r16;
            const uint16_t* src = q16 + (int64_t)(t < T ? t : T - 1) * ldq + h * D + g4 * 8;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const f16x8 q = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(src + ks * 32));
#pragma unroll
                for (int i = 0; i < 8; ++i) qf[rf][ks][i] = (_Float16)((float)q[i] * sl2);  // scores come out scaled
            }
        }
        // O^T, and the row sums as one more MFMA product: a fragment of ones times
        // P^T puts the sum of the row's (f16) probabilities in every element
        f32x4 o[DF][RF], lacc[RF];
        float m[RF];
#pragma unroll
        for (int rf = 0; rf < RF; ++rf) {
            m[rf] = -INFINITY;
            lacc[rf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int df = 0; df < DF; ++df) o[df][rf] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        f16x8 ones;
#pragma unroll
        for (int i = 0; i < 8; ++i) ones[i] = (_Float16)1.0f;

        const int tile_last = min(tile * TQ + TQ - 1, T - 1);
        const int n_keys = pos0 + tile_last + 1;  // keys any row of the tile can see
        const int n_blocks = (n_keys + KB - 1) / KB;

        // staging: K and V rows alike, as 16-byte row pieces (V is read transposed
        // later). Rows past the tile's last key are clamped to it: they are real,
        // finite cache rows whose scores the diagonal mask sets to -inf, so they add
        // 0 to O
        u32x4 kreg[KVECS], vreg[KVECS];
        auto fetch = [&](int kb) {
#pragma unroll
            for (int i = 0; i < KVECS; ++i) {
                const int v = tid + i * NT;
                const int64_t off = (int64_t)min(kb * KB + v / (D / 8), n_keys - 1) * D + (v % (D / 8)) * 8;
                kreg[i] = *reinterpret_cast<const u32x4*>(Kg + off);
                vreg[i] = *reinterpret_cast<const u32x4*>(Vg + off);
            }
        };
        auto stash = [&](int buf) {
#pragma unroll
            for (int i = 0; i < KVECS; ++i) {
                const int v = tid + i * NT;
                *reinterpret_cast<u32x4*>(&Ks[buf][swz(v / (D / 8), v % (D / 8), KS)]) = kreg[i];
                *reinterpret_cast<u32x4*>(&Vs[buf][swz(v / (D / 8), v % (D / 8), KS)]) = vreg[i];
            }
        };
        // V^T fragment (A operand) of dims 16 df .. 16 df + 15 over the key group's 32
        // keys by two LDS transpose reads (ds_read_b64_tr_b16). Within each 16-lane
        // group the lanes hand in 16 rows of four 16-bit values and lane i receives
        // element i % 4 of rows i / 4, i / 4 + 4, i / 4 + 8 and i / 4 + 12 (checked on
        // the device). Lane (g4, r16) hands in key row 4 g4 + r16 / 4 (then + 16) at
        // dims 16 df + 4 (r16 % 4) .. + 3, so it receives dim 16 df + r16 of keys
        // 4 g4 .. 4 g4 + 3 and 16 + 4 g4 .. 16 + 4 g4 + 3: the keys the S^T fragment
        // gives the same lane in the P^T B operand. (V rows XOR-swizzled by 2r instead
        // of r, which spreads these reads over distinct banks in a 32- or 64-bank
        // model, measured no faster at 4096 rows: 108-109 against 104-107 us.)
        auto vt_frag = [&](int buf, int df) {
            const int row = kg * 32 + 4 * g4 + r16 / 4, dim = df * 16 + 4 * (r16 % 4);
            const int o0 = swz(row, dim / 8, KS) + dim % 8, o1 = swz(row + 16, dim / 8, KS) + dim % 8;
            typedef short s16x4 __attribute__((ext_vector_type(4)));
            typedef short s16x8 __attribute__((ext_vector_type(8)));
            const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(&Vs[buf][o0]));
            const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(&Vs[buf][o1]));
            return __builtin_bit_cast(f16x8, (s16x8)__builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        fetch(0);
        stash(0);
        if (n_blocks > 1) fetch(1);
        __syncthreads();
        for (int kb = 0; kb < n_blocks; ++kb) {
            const int buf = kb & 1, c0 = kb * KB + kg * 32;  // this key group's first key of the block
            // S^T: lane holds query row r16 of fragment rf, keys c0 + 16 kf + 4 g4 + i
            f32x4 sc[2][RF];
#pragma unroll
            for (int kf = 0; kf < 2; ++kf) {
#pragma unroll
                for (int rf = 0; rf < RF; ++rf) sc[kf][rf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks) {
                    const f16x8 kfr =
                        *reinterpret_cast<const f16x8*>(&Ks[buf][swz(kg * 32 + kf * 16 + r16, ks * 4 + g4, KS)]);
#pragma unroll
                    for (int rf = 0; rf < RF; ++rf)
                        sc[kf][rf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kfr, qf[rf][ks], sc[kf][rf], 0, 0, 0);
                }
            }
            // online softmax; P^T packed as the B fragment of the group's 32-key step
            f16x8 pb[RF];
            const bool diag = c0 + 31 > pos0 + t0;  // some key of the group lies past some row of the wave
#pragma unroll
            for (int rf = 0; rf < RF; ++rf) {
                const int t_abs = pos0 + t0 + rf * 16 + r16;  // last key this query row sees
                float mx = -INFINITY;
                if (diag) {
#pragma unroll
                    for (int kf = 0; kf < 2; ++kf)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (c0 + kf * 16 + g4 * 4 + i > t_abs) sc[kf][rf][i] = -INFINITY;
                }
#pragma unroll
                for (int kf = 0; kf < 2; ++kf)
#pragma unroll
                    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[kf][rf][i]);
                mx = fmaxf(mx, xor16(mx));
                mx = fmaxf(mx, xor32(mx));
                // lazy rescale: the reference m moves only when a score exceeds it by more
                // than kLazy (base 2), so probabilities stay below 2^kLazy (exact in f16's
                // range) and the O rescale is skipped by every wave whose rows need none
                if (__ballot(mx > m[rf] + kLazy) != 0ull) {
                    const float mn = mx > m[rf] + kLazy ? mx : m[rf];
                    // a row may see no key of its group yet (m = -inf): its state is empty,
                    // so any finite factor (here 0) leaves it so
                    const float alpha = m[rf] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[rf] - mn);
                    lacc[rf] *= alpha;
#pragma unroll
                    for (int df = 0; df < DF; ++df) o[df][rf] *= alpha;
                    m[rf] = mn;
                }
                // exponents against 0 while the row has seen no key: masked scores give 0
                const float mref = m[rf] == -INFINITY ? 0.f : m[rf];
#pragma unroll
                for (int kf = 0; kf < 2; ++kf)
#pragma unroll
                    for (int i = 0; i < 4; ++i) sc[kf][rf][i] = __builtin_amdgcn_exp2f(sc[kf][rf][i] - mref);
                // two probabilities per conversion (round toward zero; they lie in [0, 1])
                const u32x4 pk{
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(sc[0][rf][0], sc[0][rf][1])),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(sc[0][rf][2], sc[0][rf][3])),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(sc[1][rf][0], sc[1][rf][1])),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(sc[1][rf][2], sc[1][rf][3]))};
                pb[rf] = __builtin_bit_cast(f16x8, pk);
            }
            // O^T += V^T P^T over the group's 32 keys; the row sums likewise
#pragma unroll
            for (int rf = 0; rf < RF; ++rf) lacc[rf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb[rf], lacc[rf], 0, 0, 0);
#pragma unroll
            for (int df = 0; df < DF; ++df) {
                const f16x8 vfr = vt_frag(buf, df);
#pragma unroll
                for (int rf = 0; rf < RF; ++rf)
                    o[df][rf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vfr, pb[rf], o[df][rf], 0, 0, 0);
            }
            if (kb + 1 < n_blocks) {
                stash(buf ^ 1);  // that buffer was last read before the previous barrier
                if (kb + 2 < n_blocks) fetch(kb + 2);
            }
            __syncthreads();
        }
        // hand-over: key group 1 leaves m, l and O in LDS (the K/V
        // buffers are free after the loop's last barrier), lane-minor so that a
        // wave's 64 stores hit 64 consecutive words
        float* xo0 = reinterpret_cast<float*>(&Ks[0][0]);  // O values of df < DF / 2
        float* xo1 = reinterpret_cast<float*>(&Vs[0][0]);  // and of the rest
        const int slot = wr * WAVE + lane;
        if (kg == 1) {
#pragma unroll
            for (int rf = 0; rf < RF; ++rf) {
                ml[0][rf][slot] = m[rf];
                ml[1][rf][slot] = lacc[rf][0];
#pragma unroll
                for (int df = 0; df < DF; ++df)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float* x = df < DF / 2 ? xo0 : xo1;
                        x[(((df % (DF / 2)) * RF + rf) * 4 + i) * 256 + slot] = o[df][rf][i];
                    }
            }
        }
        __syncthreads();
        if (kg == 0) {
#pragma unroll
            for (int rf = 0; rf < RF; ++rf) {
                const float m2 = ml[0][rf][slot], l2 = ml[1][rf][slot];
                const float M = fmaxf(m[rf], m2);
                const float mref = M == -INFINITY ? 0.f : M;
                const float a = __builtin_amdgcn_exp2f(m[rf] - mref), b = __builtin_amdgcn_exp2f(m2 - mref);
                const float lsum = lacc[rf][0] * a + l2 * b;
                const int t = t0 + rf * 16 + r16;
                if (t >= T) continue;
                const float inv = 1.0f / lsum;
#pragma unroll
                for (int df = 0; df < DF; ++df)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float* x = df < DF / 2 ? xo0 : xo1;
                        const float v = (o[df][rf][i] * a + x[(((df % (DF / 2)) * RF + rf) * 4 + i) * 256 + slot] * b) * inv;
                        uint16_t hi, lo;
                        split_bf16(v, hi, lo);
                        const int64_t idx = (int64_t)t * ldo + h * D + df * 16 + g4 * 4 + i;
                        out[idx] = hi;
                        if (out_lo) out_lo[idx] = lo;
                    }
            }
        }
    }
    clock_end(clk);
}

hipError_t launch_attn_prefill(const uint16_t* q16, int64_t ldq, int T, int pos0, int seq, int n_heads, KVLayer kv,
                               uint16_t* out_bf16, uint16_t* out_bf16_lo, int64_t ldo, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    const int n_tiles = (T + 127) / 128;
    // pairing evens out causal work once there are enough tiles to fill the chip
    const int paired = n_tiles * n_heads >= 512;
    dim3 grid(paired ? (n_tiles + 1) / 2 : n_tiles, n_heads);
    const Segments none{};
    if (kv.d == 128)
        launch_kernel(attn_prefill_kernel<128, false>, grid, 512, 0, s, q16, ldq, T, pos0, seq, n_heads, kv, out_bf16,
                      out_bf16_lo, ldo, paired, clock_slot(), none);
    else if (kv.d == 64)
        launch_kernel(attn_prefill_kernel<64, false>, grid, 512, 0, s, q16, ldq, T, pos0, seq, n_heads, kv, out_bf16,
                      out_bf16_lo, ldo, paired, clock_slot(), none);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_attn_prefill_packed(const uint16_t* q16, int64_t ldq, const Segments& sg, int n_heads, KVLayer kv,
                                      uint16_t* out_bf16, uint16_t* out_bf16_lo, int64_t ldo, hipStream_t s) {
    if (sg.n <= 0) return hipSuccess;
    if (sg.n > kMaxSegments) return hipErrorInvalidValue;
    int max_len = 0;
    for (int i = 0; i < sg.n; ++i) max_len = sg.len[i] > max_len ? sg.len[i] : max_len;
    if (max_len <= 0) return hipSuccess;
    const dim3 grid((max_len + 127) / 128, n_heads, sg.n);
    if (kv.d == 128)
        launch_kernel(attn_prefill_kernel<128, true>, grid, 512, 0, s, q16, ldq, 0, 0, 0, n_heads, kv, out_bf16,
                      out_bf16_lo, ldo, 0, clock_slot(), sg);
    else if (kv.d == 64)
        launch_kernel(attn_prefill_kernel<64, true>, grid, 512, 0, s, q16, ldq, 0, 0, 0, n_heads, kv, out_bf16,
                      out_bf16_lo, ldo, 0, clock_slot(), sg);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace sttd
