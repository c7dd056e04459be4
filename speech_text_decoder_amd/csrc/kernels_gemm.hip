// kernels_gemm.hip - bf16 MFMA GEMM for prefill rows: C[M, N] = A[M, K] W[N, K]^T
// with fp32 accumulation, and the block's epilogues fused behind it:
//   STORE   C = A W^T (the Q|K|V projections, three weight segments stacked)
//   RESID   C += A W^T (O and down projections add into the residual stream)
//   SWIGLU  act[:, n] = silu(g) * u with g, u the packed gate_up outputs n and I + n
//
// Tile BM x BN x 64 per workgroup of 4 waves (2 x 2); each wave computes a
// (BM/2) x (BN/2) block with v_mfma_f32_16x16x32_bf16. A and W tiles are staged
// through LDS (16-byte chunks of each row XOR-swizzled by the row so the
// fragment reads hit distinct banks); the next K tile is fetched into registers
// while the current one feeds the MFMAs.
//
// Split activations (A_lo given): every MFMA step runs twice, on the bf16
// high part and on the bf16 remainder of the activation, so the product sees
// about 16 significant bits of each activation (the weights are exact bf16).
//
// Fragment layout of v_mfma_f32_16x16x32_bf16 (checked on the device): lane l
// supplies row l%16 and K elements (l/16)*8 .. +8 of both operands; the 16x16
// result gives lane l column l%16 and rows (l/16)*4 + i, i < 4.
#include "common.h"
#include "launch.h"

namespace sttd {

constexpr int BK = 64;
constexpr int LDS_STRIDE = BK;  // bf16 elements per staged row (unpadded; chunks swizzled)

// LDS offset (elements) of 16-byte chunk c of staged row r: the chunk index is
// XOR-swizzled by the row so fragment reads and staging writes avoid bank conflicts.
__device__ __forceinline__ int lds_off(int r, int c) { return r * LDS_STRIDE + ((c ^ (r & 7)) * 8); }

template <int V>
__device__ __forceinline__ void fetch_rows(u32x4 (&reg)[V], const uint16_t* const (&p)[V], const bool (&ok)[V],
                                           int64_t k0) {
#pragma unroll
    for (int i = 0; i < V; ++i) reg[i] = ok[i] ? *reinterpret_cast<const u32x4*>(p[i] + k0) : u32x4{0u, 0u, 0u, 0u};
}

template <int V>
__device__ __forceinline__ void stash_rows(const u32x4 (&reg)[V], uint16_t* lds, int tid) {
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int v = tid + i * 256;
        *reinterpret_cast<u32x4*>(&lds[lds_off(v / (BK / 8), v % (BK / 8))]) = reg[i];
    }
}

template <int BM, int BN, int EPI, bool SPLIT>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs g) {
    constexpr int FM = BM / 32;  // 16-row fragments per wave
    constexpr int FN = BN / 32;  // 16-col fragments per wave
    constexpr int A_VECS = BM * BK / 8 / 256;
    constexpr int B_VECS = BN * BK / 8 / 256;
    __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) uint16_t Als[SPLIT ? BM * LDS_STRIDE : 8];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDS_STRIDE];

    clock_begin(g.clk);
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int wm = wave / 2, wn = wave % 2;
    const int m0 = blockIdx.y * BM;
    const int tile_n = blockIdx.x;

    // Global source row of each staged B row.
    const uint16_t* brow_ptr[B_VECS];
    bool brow_ok[B_VECS];
#pragma unroll
    for (int i = 0; i < B_VECS; ++i) {
        brow_ok[i] = true;
        const int v = tid + i * 256;
        const int r = v / (BK / 8);
        int grow;
        const uint16_t* W;
        if (EPI == GEMM_SWIGLU) {
            // rows [0, BN/2): gate rows of act columns tile_n*BN/2 ..; rows [BN/2, BN): the up rows
            const int c = tile_n * (BN / 2) + (r % (BN / 2));
            grow = r < BN / 2 ? c : g.N + c;
            W = g.w[0];
        } else {
            const int n0 = tile_n * BN + r;
            brow_ok[i] = n0 < g.N;
            const int n = brow_ok[i] ? n0 : 0;
            const bool s2 = n >= g.seg_end[1], s1 = n >= g.seg_end[0];
            grow = n - (s2 ? g.seg_end[1] : (s1 ? g.seg_end[0] : 0));
            W = s2 ? g.w[2] : (s1 ? g.w[1] : g.w[0]);
        }
        brow_ptr[i] = W + (int64_t)grow * g.K + (v % (BK / 8)) * 8;
    }
    const uint16_t* arow_ptr[A_VECS];
    const uint16_t* alo_ptr[A_VECS];
    bool arow_ok[A_VECS];
#pragma unroll
    for (int i = 0; i < A_VECS; ++i) {
        const int v = tid + i * 256;
        const int r = v / (BK / 8);
        arow_ok[i] = (m0 + r) < g.M;
        const int64_t off = (int64_t)(arow_ok[i] ? m0 + r : 0) * g.lda + (v % (BK / 8)) * 8;
        arow_ptr[i] = g.A + off;
        alo_ptr[i] = SPLIT ? g.A_lo + off : g.A + off;
    }

    u32x4 areg[A_VECS], alreg[A_VECS], breg[B_VECS];
    // LDS row of each B fragment of this wave
    int bfrag_row[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        if (EPI == GEMM_SWIGLU)
            bfrag_row[j] = j < FN / 2 ? wn * (BN / 4) + j * 16 : BN / 2 + wn * (BN / 4) + (j - FN / 2) * 16;
        else
            bfrag_row[j] = wn * (BN / 2) + j * 16;
    }

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // K range of this workgroup: split over gridDim.z (RESID only; partial sums add with atomics)
    const int nk_all = g.K / BK;
    const int nk_per = (nk_all + gridDim.z - 1) / gridDim.z;
    const int kt0 = min((int)blockIdx.z * nk_per, nk_all);
    const int nk = min(nk_per, nk_all - kt0);
    const int64_t kbase = (int64_t)kt0 * BK;
    auto fetch = [&](int64_t k0) {
        k0 += kbase;
        fetch_rows<A_VECS>(areg, arow_ptr, arow_ok, k0);
        if (SPLIT) fetch_rows<A_VECS>(alreg, alo_ptr, arow_ok, k0);
        fetch_rows<B_VECS>(breg, brow_ptr, brow_ok, k0);
    };
    auto stash = [&]() {
        stash_rows<A_VECS>(areg, As, tid);
        if (SPLIT) stash_rows<A_VECS>(alreg, Als, tid);
        stash_rows<B_VECS>(breg, Bs, tid);
    };
    if (nk > 0) fetch(0);
    stash();
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) fetch((int64_t)(kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            bf16x8 af[FM], afl[FM], bfr[FN];
            const int kc = ks * 32 + (lane / 16) * 8;
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int o = lds_off(wm * (BM / 2) + i * 16 + lane % 16, kc / 8);
                af[i] = *reinterpret_cast<const bf16x8*>(&As[o]);
                if (SPLIT) afl[i] = *reinterpret_cast<const bf16x8*>(&Als[o]);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8*>(&Bs[lds_off(bfrag_row[j] + lane % 16, kc / 8)]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
                    if (SPLIT) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afl[i], bfr[j], acc[i][j], 0, 0, 0);
                }
        }
        __syncthreads();
        if (kt + 1 < nk) {
            stash();
            __syncthreads();
        }
    }

    // epilogue
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int m = m0 + wm * (BM / 2) + i * 16 + (lane / 16) * 4 + rr;
            if (m >= g.M) continue;
            if (EPI == GEMM_SWIGLU) {
#pragma unroll
                for (int j = 0; j < FN / 2; ++j) {
                    const int c = tile_n * (BN / 2) + wn * (BN / 4) + j * 16 + lane % 16;
                    const float gt = acc[i][j][rr], up = acc[i][j + FN / 2][rr];
                    const float a = gt / (1.0f + expf(-gt)) * up;
                    uint16_t hi, lo;
                    split_bf16(a, hi, lo);
                    g.Cb[(int64_t)m * g.ldcb + c] = hi;
                    if (g.Cb_lo) g.Cb_lo[(int64_t)m * g.ldcb + c] = lo;
                }
            } else {
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int n = tile_n * BN + wn * (BN / 2) + j * 16 + lane % 16;
                    if (n >= g.N) continue;
                    float* dst = g.C + (int64_t)m * g.ldc + n;
                    if (EPI == GEMM_RESID) {
                        if (gridDim.z == 1) *dst += acc[i][j][rr];
                        else atomicAdd(dst, acc[i][j][rr]);
                    } else {
                        *dst = acc[i][j][rr];
                    }
                }
            }
        }
    }
    clock_end(g.clk);
}


// ------------------------------------------------------------------ mid-M, weights streamed
// C = A W^T for a few hundred rows, where one K-step in flight per workgroup
// leaves each step waiting on its loads. Tile (16 FM) x (64 FN) per workgroup of
// 4 waves; every wave owns all 16 FM rows and FN column fragments of its own, so
// its weight rows go from global memory straight into B fragments (lane l:
// column l % 16, K elements (l / 16) * 8 .. + 8 of each 32-deep half-step) and
// only A (bf16 high and low planes) is staged, through two LDS buffers, once per
// workgroup. Loads run D K-steps of 64 ahead in a register ring: the loads of
// step t + D are issued as soon as step t has fed the MFMAs, so D - 1 steps of
// MFMA work cover each load's latency. Per 32-deep half-step a wave reads 2 FM
// A fragments from LDS for 2 FM FN MFMAs.
// SWIGLU: fragments [0, FN/2) of a wave are gate columns, [FN/2, FN) the up
// columns of the same act columns.
// What bounds it (153 rows, gate_up): the bytes each CU requests. With one
// workgroup per CU a CU keeps about 32 KB of loads in flight, which at loaded
// latencies is ~20 GB/s from HBM and ~40 GB/s from L2; each workgroup requests
// 512 KB of weights and 640 KB of A planes. Timed alone (in an 8-wave form of
// this kernel), the weight loads took
// 27 us, the A loads 17 us, the LDS staging and MFMAs without global loads 24 us,
// and the loads alone (no LDS, no MFMA) 34.5 us, about the whole kernel. Measured
// and not kept: 8 waves with the K-step halves split between wave pairs (two
// waves per SIMD), each K-half wave walking a contiguous K range, and per-
// workgroup rotation of the K order (all within 1 us); ring depth 3, 4 and 6
// (36, 36 and 40 us against 34 us at 2); 64-row tiles at 153 rows (three row
// tiles, 288 workgroups: 46 us); one 160-row tile with one column fragment per
// wave for QKV, O and down, so each weight byte is requested once (QKV 22.4 ->
// 26.1 us, down 22.6 -> 26.8 us). For calibration, a probe reading the same
// A-tile pattern (80 rows 4 KB apart, 128 B each per step, a ring with a barrier
// per step) gets ~130 GB/s per workgroup from L2. Staging the weight tile through
// LDS too, loaded in row pieces (the fragment-shaped loads read L2 at a third of
// that rate, and each weight tile's second row tile finds it in L2), measured
// slower: gate_up 36.3 -> 38.8 us, the LDS traffic outweighing the faster loads.
template <int EPI, int FM, int FN, int D, bool SPLIT>
__global__ __launch_bounds__(256) void gemm_stream_kernel(GemmArgs g) {
    constexpr int BM = FM * 16, BN = FN * 64;
    constexpr int AVT = BM * BK / 8;            // 16-byte vectors of one A plane per K-step
    constexpr int AV = (AVT + 255) / 256;       // per thread
    constexpr int NP = SPLIT ? 2 : 1;           // A planes
    __shared__ __attribute__((aligned(16))) uint16_t As[2][NP][BM * LDS_STRIDE];

    clock_begin(g.clk);
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int m0 = blockIdx.y * BM;
    const int tile_n = blockIdx.x;

    // weight row of each of this lane's column fragments
    const uint16_t* wrow[FN];
    bool wok[FN];
#pragma unroll
    for (int f = 0; f < FN; ++f) {
        if (EPI == GEMM_SWIGLU) {
            const int c = tile_n * (BN / 2) + wave * (FN / 2) * 16 + (f % (FN / 2)) * 16 + lane % 16;
            wok[f] = c < g.N;
            const int cc = wok[f] ? c : 0;
            wrow[f] = g.w[0] + (int64_t)(f < FN / 2 ? cc : g.N + cc) * g.K;
        } else {
            const int n0 = tile_n * BN + wave * FN * 16 + f * 16 + lane % 16;
            wok[f] = n0 < g.N;
            const int n = wok[f] ? n0 : 0;
            const bool s2 = n >= g.seg_end[1], s1 = n >= g.seg_end[0];
            const int grow = n - (s2 ? g.seg_end[1] : (s1 ? g.seg_end[0] : 0));
            wrow[f] = (s2 ? g.w[2] : (s1 ? g.w[1] : g.w[0])) + (int64_t)grow * g.K;
        }
        wrow[f] += (lane / 16) * 8;
    }
    // A rows this thread stages: vector v = tid + 256 i is row v / 8, 16-byte chunk v % 8
    const uint16_t* aptr[AV];
    const uint16_t* alptr[AV];
    bool aok[AV], astage[AV];
#pragma unroll
    for (int i = 0; i < AV; ++i) {
        const int v = tid + i * 256;
        astage[i] = v < AVT;
        const int r = astage[i] ? v / 8 : 0;
        aok[i] = astage[i] && m0 + r < g.M;
        const int64_t off = (int64_t)(aok[i] ? m0 + r : 0) * g.lda + (v % 8) * 8;
        aptr[i] = g.A + off;
        alptr[i] = SPLIT ? g.A_lo + off : g.A + off;
    }

    // K range of this workgroup: split over gridDim.z (partial sums add with atomics)
    const int nk_all = g.K / BK;
    const int nk_per = (nk_all + gridDim.z - 1) / gridDim.z;
    const int kt0 = min((int)blockIdx.z * nk_per, nk_all);
    const int nk = min(nk_per, nk_all - kt0);
    const int64_t kbase = (int64_t)kt0 * BK;

    u32x4 ra[D][NP][AV], rb[D][FN][2];
    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int f = 0; f < FN; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Every fetch is unconditional (steps past the end reload the last one, rows
    // past M reload a valid row and are zeroed when staged), so the number of
    // loads issued after each ring slot is fixed and each wait covers only its
    // own slot.
#define STREAM_FETCH(U, KT)                                                                  \
    do {                                                                                     \
        const int64_t k0_ = kbase + (int64_t)min((KT), nk - 1) * BK;                         \
        _Pragma("unroll") for (int i = 0; i < AV; ++i) {                                     \
            ra[U][0][i] = *reinterpret_cast<const u32x4*>(aptr[i] + k0_);                    \
            if (SPLIT) ra[U][NP - 1][i] = *reinterpret_cast<const u32x4*>(alptr[i] + k0_);   \
        }                                                                                    \
        _Pragma("unroll") for (int f = 0; f < FN; ++f) {                                     \
            rb[U][f][0] = *reinterpret_cast<const u32x4*>(wrow[f] + k0_);                     \
            rb[U][f][1] = *reinterpret_cast<const u32x4*>(wrow[f] + k0_ + 32);                \
        }                                                                                    \
    } while (0)

    if (nk > 0) {
        // slot by slot, so the oldest slot's loads are the oldest in flight on every pass
#pragma unroll
        for (int u = 0; u < D; ++u) {
            STREAM_FETCH(u, u);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int kb = 0; kb < nk; kb += D) {
#pragma unroll
            for (int u = 0; u < D; ++u) {
                const int kt = kb + u;
                // stage this step's A planes (buffer kt & 1 was last read two steps
                // ago, before every wave passed the previous step's barrier)
                uint16_t(*buf)[BM * LDS_STRIDE] = As[kt & 1];
#pragma unroll
                for (int pl = 0; pl < NP; ++pl)
#pragma unroll
                    for (int i = 0; i < AV; ++i) {
                        if (!astage[i]) continue;
                        const int v = tid + i * 256;
                        const u32x4 z{0u, 0u, 0u, 0u};
                        *reinterpret_cast<u32x4*>(&buf[pl][lds_off(v / 8, v % 8)]) = aok[i] ? ra[u][pl][i] : z;
                    }
                __syncthreads();
                __builtin_amdgcn_sched_barrier(0);
                if (kt < nk) {
                    // all of the step's A fragments are read first (one wave per SIMD has
                    // no other wave to cover LDS latency), then the MFMAs run plane by
                    // plane, so FM FN independent products separate two on one accumulator
                    bf16x8 af[2][NP][FM];
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                        for (int pl = 0; pl < NP; ++pl)
#pragma unroll
                            for (int i = 0; i < FM; ++i)
                                af[ks][pl][i] = *reinterpret_cast<const bf16x8*>(
                                    &buf[pl][lds_off(i * 16 + lane % 16, ks * 4 + lane / 16)]);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                        for (int pl = 0; pl < NP; ++pl)
#pragma unroll
                            for (int i = 0; i < FM; ++i)
#pragma unroll
                                for (int f = 0; f < FN; ++f)
                                    acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                        af[ks][pl][i], __builtin_bit_cast(bf16x8, rb[u][f][ks]), acc[i][f], 0, 0, 0);
                }
                // keep the compiler from moving this slot's refetch above its use
                __builtin_amdgcn_sched_barrier(0);
                STREAM_FETCH(u, kt + D);
            }
        }
    }
#undef STREAM_FETCH

    // epilogue: lane l holds column l % 16 and rows (l / 16) * 4 + rr of each fragment
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int m = m0 + i * 16 + (lane / 16) * 4 + rr;
            if (m >= g.M) continue;
            if (EPI == GEMM_SWIGLU) {
#pragma unroll
                for (int f = 0; f < FN / 2; ++f) {
                    if (!wok[f]) continue;
                    const int c = tile_n * (BN / 2) + wave * (FN / 2) * 16 + f * 16 + lane % 16;
                    const float gt = acc[i][f][rr], up = acc[i][f + FN / 2][rr];
                    const float a = gt / (1.0f + expf(-gt)) * up;
                    uint16_t hi, lo;
                    split_bf16(a, hi, lo);
                    g.Cb[(int64_t)m * g.ldcb + c] = hi;
                    if (g.Cb_lo) g.Cb_lo[(int64_t)m * g.ldcb + c] = lo;
                }
            } else {
#pragma unroll
                for (int f = 0; f < FN; ++f) {
                    if (!wok[f]) continue;
                    const int n = tile_n * BN + wave * FN * 16 + f * 16 + lane % 16;
                    float* dst = g.C + (int64_t)m * g.ldc + n;
                    if (EPI == GEMM_RESID) {
                        if (gridDim.z == 1) *dst += acc[i][f][rr];
                        else atomicAdd(dst, acc[i][f][rr]);
                    } else {
                        *dst = acc[i][f][rr];
                    }
                }
            }
        }
    }
    clock_end(g.clk);
}

// ------------------------------------------------------------------ large-M tiles
// For prefills of many rows (the GEMMs are MFMA-bound there): 256 x 256 output
// tiles, 8 waves in 4 x 2 each owning 64 x 128 (4 x 8 fragments of
// v_mfma_f32_16x16x32_bf16), two waves per SIMD so one issues MFMAs while the
// other waits; K in steps of 64 through two LDS buffers so one barrier per
// step separates staging from use. Per SIMD and 32-deep step the fragments
// cost 24 KB of LDS reads for 64 MFMAs, about three quarters of what LDS
// delivers in that time; the staging writes add the rest, so these GEMMs run
// near the LDS limit (about 45% MFMA busy).
//
// Tiles are handed out XCD-aware: workgroup i runs on XCD i % 8, so the tile
// index is remapped to give each XCD a contiguous run of tiles with the row
// tile varying fastest; the workgroups of one XCD then share weight tiles in
// their L2.
//
// SWIGLU: LDS weight rows [128 wn, 128 wn + 64) hold gate rows and
// [128 wn + 64, 128 wn + 128) the matching up rows of act columns
// 128 tile_n + 64 wn .. + 64, so wave column wn finds gate (fragments 0..3)
// and up (fragments 4..7) of the same columns in its own accumulators.
constexpr int BIG_BM = 256, BIG_BN = 256, BIG_BK = 64, BIG_STR = BIG_BK;

// LDS offset (elements) of 16-byte chunk c of staged row r: unpadded rows of 64
// elements with the chunk index XOR-swizzled by the row. The fragment reads (16 rows,
// one chunk) and the staging writes (8 chunks of a row) then hit no bank twice; the
// SQ_LDS_BANK_CONFLICT counter reads 0, against 37% of LDS cycles with padded rows.
__device__ __forceinline__ int big_lds_off(int r, int c) { return r * BIG_BK + ((c ^ (r & 7)) * 8); }

// KSPLIT > 1 (residual outputs only): the grid holds KSPLIT copies of the tile
// grid, copy s taking the s-th part of K and adding its partial sums into C
// (which already holds the residual) with fp32 atomics. Copies follow one
// another in the grid, so each keeps the XCD-aware tile order.
#ifndef STTD_BIG_WM
#define STTD_BIG_WM 4
#endif
#ifndef STTD_BIG_SPLIT
#define STTD_BIG_SPLIT 1  // split activations (hi/lo) take the large tiles too
#endif
// WM: waves along M (4: 8 waves of 64 x BN/2; 2: 4 waves of 128 x BN/2, one per
// SIMD, with the accumulators in AGPRs). One wave per SIMD reads a third less LDS
// per MFMA but measured much slower at 4096 rows (gate_up 189 -> 284 us, down
// 113 -> 175 us): a single wave cannot hide its LDS and global latency.
// SPLIT: the activations come as bf16 high and low planes (A, A_lo); both are
// staged and every B fragment feeds two MFMAs, one per plane. The K-step per
// tile is 32 then, so the three staged tiles fit LDS twice over; rows of 32
// elements (4 chunks) need no swizzle: a fragment read (16 rows x 4 chunks) and a
// staging write (16 rows x 4 chunks) each cover 1 KB of consecutive LDS.
template <int EPI, int BN, int KSPLIT = 1, int WM = STTD_BIG_WM, bool SPLIT = false>
__global__ __launch_bounds__(WM * 128) void gemm_big_kernel(GemmArgs g, int tiles_m, int tiles_n) {
    static_assert(EPI != GEMM_SWIGLU || BN == BIG_BN, "SwiGLU pairs gate and up inside 256-row weight tiles");
    static_assert(KSPLIT == 1 || EPI == GEMM_RESID, "split K adds into a residual");
    constexpr int BK = SPLIT ? 32 : BIG_BK;          // K per staged tile
    constexpr int NT = WM * 128;                     // threads
    constexpr int WR = BIG_BM / WM;                  // rows per wave
    constexpr int FM = WR / 16, FN = BN / 32;
    constexpr int VECS = BIG_BM * BK / 8 / NT;       // 16-byte vectors per thread and step: A
    constexpr int BVECS = BN * BK / 8 / NT;          // and B
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BIG_BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t Als[SPLIT ? 2 : 1][SPLIT ? BIG_BM * BK : 8];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * BK];
    auto lds_off = [](int r, int c) { return SPLIT ? r * BK + c * 8 : big_lds_off(r, c); };

    clock_begin(g.clk);
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int wm = wave / 2, wn = wave % 2;  // WM x 2 waves, each WR x BN / 2
    // XCD-aware tile order when the tile count splits evenly over the 8 XCDs
    const int n_tiles = tiles_m * tiles_n;
    const int id = KSPLIT > 1 ? (int)blockIdx.x % n_tiles : (int)blockIdx.x;
    const int k_part = KSPLIT > 1 ? (int)blockIdx.x / n_tiles : 0;
    const int64_t k_begin = (int64_t)k_part * (g.K / KSPLIT);
    const int t = n_tiles % 8 ? id : (id % 8) * (n_tiles / 8) + id / 8;
    const int tile_m = t % tiles_m, tile_n = t / tiles_m;
    const int m0 = tile_m * BIG_BM;

    const uint16_t* aptr[VECS];
    const uint16_t* alptr[VECS];
    const uint16_t* bptr[BVECS];
    bool bok[BVECS];
#pragma unroll
    for (int i = 0; i < VECS; ++i) {
        const int v = tid + i * NT;
        const int r = v / (BK / 8), ck = (v % (BK / 8)) * 8;
        const int am = m0 + r < g.M ? m0 + r : 0;
        aptr[i] = g.A + (int64_t)am * g.lda + k_begin + ck;
        alptr[i] = (SPLIT ? g.A_lo : g.A) + (int64_t)am * g.lda + k_begin + ck;
    }
#pragma unroll
    for (int i = 0; i < BVECS; ++i) {
        const int v = tid + i * NT;
        const int r = v / (BK / 8), ck = (v % (BK / 8)) * 8;
        int grow;
        const uint16_t* W;
        bok[i] = true;
        if (EPI == GEMM_SWIGLU) {
            const int wsel = r / 128, within = r % 128;
            const int c = tile_n * 128 + wsel * 64 + (within % 64);
            grow = within < 64 ? c : g.N + c;
            W = g.w[0];
        } else {
            const int n0 = tile_n * BN + r;
            bok[i] = n0 < g.N;
            const int n = bok[i] ? n0 : 0;
            const bool s2 = n >= g.seg_end[1], s1 = n >= g.seg_end[0];
            grow = n - (s2 ? g.seg_end[1] : (s1 ? g.seg_end[0] : 0));
            W = s2 ? g.w[2] : (s1 ? g.w[1] : g.w[0]);
        }
        bptr[i] = W + (int64_t)grow * g.K + k_begin + ck;
    }
    u32x4 areg[VECS], alreg[SPLIT ? VECS : 1], breg[BVECS];
    auto fetch = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < VECS; ++i) areg[i] = *reinterpret_cast<const u32x4*>(aptr[i] + k0);
        if (SPLIT) {
#pragma unroll
            for (int i = 0; i < VECS; ++i) alreg[SPLIT ? i : 0] = *reinterpret_cast<const u32x4*>(alptr[i] + k0);
        }
#pragma unroll
        for (int i = 0; i < BVECS; ++i)
            breg[i] = bok[i] ? *reinterpret_cast<const u32x4*>(bptr[i] + k0) : u32x4{0u, 0u, 0u, 0u};
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int i = 0; i < VECS; ++i) {
            const int v = tid + i * NT;
            const int o = lds_off(v / (BK / 8), v % (BK / 8));
            *reinterpret_cast<u32x4*>(&As[buf][o]) = areg[i];
            if (SPLIT) *reinterpret_cast<u32x4*>(&Als[SPLIT ? buf : 0][o]) = alreg[SPLIT ? i : 0];
            if (i < BVECS) *reinterpret_cast<u32x4*>(&Bs[buf][o]) = breg[i < BVECS ? i : 0];
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = g.K / BK / KSPLIT;
    fetch(0);
    stash(0);
    if (nk > 1) fetch(BK);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        const uint16_t* Ab = As[buf];
        const uint16_t* Alb = Als[SPLIT ? buf : 0];
        const uint16_t* Bb = Bs[buf];
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            const int kc = ks * 32 + (lane / 16) * 8;
            bf16x8 af[FM], al[SPLIT ? FM : 1], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                af[i] = *reinterpret_cast<const bf16x8*>(&Ab[lds_off(wm * WR + i * 16 + lane % 16, kc / 8)]);
                if (SPLIT)
                    al[SPLIT ? i : 0] =
                        *reinterpret_cast<const bf16x8*>(&Alb[lds_off(wm * WR + i * 16 + lane % 16, kc / 8)]);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8*>(&Bb[lds_off(wn * (BN / 2) + j * 16 + lane % 16, kc / 8)]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
                    if (SPLIT)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[SPLIT ? i : 0], bfr[j], acc[i][j], 0, 0, 0);
                }
            // between the two K-steps: stage the next tile (the other buffer was last read
            // before the previous barrier) and start loading the one after, so the LDS
            // writes and the global loads overlap the second step's MFMAs
            if (ks == 0 && kt + 1 < nk) {
                stash(buf ^ 1);
                if (kt + 2 < nk) fetch((int64_t)(kt + 2) * BK);
            }
        }
        __syncthreads();
    }

    if (EPI == GEMM_QKROPE) {
        // the wave's 128 columns are one head (query, key or value) of its 64 rows:
        // lane l holds columns 16 j + l % 16, so the NeoX pair (c, c + 64) is
        // fragments j and j + 4 of the same lane and a row's sum of squares over
        // the head is a sum over the 16 lanes of a DPP row (qk_head_item's
        // arithmetic). Gains are loaded once; the table rows of a fragment's 4
        // rows are all requested before any is used.
        const QkRope& q = g.qk;
        const int hi = (tile_n * BN + wn * (BN / 2)) / 128;
        const int c0 = lane % 16;
        const bool is_v = hi >= q.n_heads + q.n_kv, is_q = hi < q.n_heads;
        float gn[FN];
        const uint16_t* gain = (const uint16_t*)(is_q ? q.q_gain : q.k_gain);
#pragma unroll
        for (int j = 0; j < FN; ++j) gn[j] = is_v ? 1.f : BF16::ld(gain, j * 16 + c0);
        const float2* table = reinterpret_cast<const float2*>(q.rope);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            int pos[4], seq[4];
            bool ok[4];
            float2 cs[4][FN / 2];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int m = m0 + wm * WR + i * 16 + (lane / 16) * 4 + rr;
                const int mc = m < g.M ? m : g.M - 1;
                pos[rr] = row_pos(q.rm, mc);
                seq[rr] = row_seq(q.rm, mc);
                ok[rr] = m < g.M && pos[rr] >= 0 && pos[rr] < q.kv.n_ctx && pos[rr] < q.max_pos && seq[rr] >= 0 &&
                         seq[rr] < q.kv.n_seq;
            }
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
#pragma unroll
                for (int j = 0; j < FN / 2; ++j)
                    cs[rr][j] = is_v ? float2{1.f, 0.f} : table[(int64_t)(ok[rr] ? pos[rr] : 0) * 64 + j * 16 + c0];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int m = m0 + wm * WR + i * 16 + (lane / 16) * 4 + rr;
                if (!ok[rr]) {  // the same for the 16 lanes of a DPP row (one row m)
                    if (m < g.M && c0 == 0 && wn == 0)
                        record_error(q.err, pos[rr] < 0 || pos[rr] >= q.kv.n_ctx ? 1u : 2u);
                    continue;
                }
                float v[FN];
#pragma unroll
                for (int j = 0; j < FN; ++j) v[j] = acc[i][j][rr];
                if (is_v) {  // value head: copied as it is
                    const int64_t off =
                        ((int64_t)(seq[rr] * q.n_kv + hi - q.n_heads - q.n_kv) * q.kv.n_ctx + pos[rr]) * 128;
#pragma unroll
                    for (int j = 0; j < FN; ++j) F16::st((uint16_t*)q.kv.v, off + j * 16 + c0, v[j]);
                    continue;
                }
                float ss = 0.f;
#pragma unroll
                for (int j = 0; j < FN; ++j) ss = fmaf(v[j], v[j], ss);
                ss = row16_sum(ss);
                const float rs = 1.0f / sqrtf(ss / 128.f + q.eps);
                const int64_t off =
                    is_q ? (int64_t)m * q.ldq + hi * 128
                         : ((int64_t)(seq[rr] * q.n_kv + hi - q.n_heads) * q.kv.n_ctx + pos[rr]) * 128;
                uint16_t* out = is_q ? (uint16_t*)q.q_out : (uint16_t*)q.kv.k;
#pragma unroll
                for (int j = 0; j < FN / 2; ++j) {
                    const int c = j * 16 + c0;
                    const float a = v[j] * rs * gn[j];
                    const float b = v[j + FN / 2] * rs * gn[j + FN / 2];
                    F16::st(out, off + c, a * cs[rr][j].x - b * cs[rr][j].y);
                    F16::st(out, off + c + 64, a * cs[rr][j].y + b * cs[rr][j].x);
                }
            }
        }
        clock_end(g.clk);
        return;
    }

    // epilogue
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int m = m0 + wm * WR + i * 16 + (lane / 16) * 4 + rr;
            if (m >= g.M) continue;
            if (EPI == GEMM_SWIGLU) {
#pragma unroll
                for (int j = 0; j < FN / 2; ++j) {
                    const int c = tile_n * 128 + wn * 64 + j * 16 + lane % 16;
                    const float gt = acc[i][j][rr], up = acc[i][j + FN / 2][rr];
                    const float a = gt / (1.0f + expf(-gt)) * up;
                    uint16_t hi, lo;
                    split_bf16(a, hi, lo);
                    g.Cb[(int64_t)m * g.ldcb + c] = hi;
                    if (g.Cb_lo) g.Cb_lo[(int64_t)m * g.ldcb + c] = lo;
                }
            } else {
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int n = tile_n * BN + wn * (BN / 2) + j * 16 + lane % 16;
                    if (n >= g.N) continue;
                    float* dst = g.C + (int64_t)m * g.ldc + n;
                    if (KSPLIT > 1) atomicAdd(dst, acc[i][j][rr]);
                    else if (EPI == GEMM_RESID) *dst += acc[i][j][rr];
                    else *dst = acc[i][j][rr];
                }
            }
        }
    }
    clock_end(g.clk);
}

// Whether the large tiles apply: many rows and shapes that tile.
bool gemm_qkrope_fits(int M, int N, int K, int head_dim) {
    return head_dim == 128 && M >= 1024 && K % BIG_BK == 0 && N % BIG_BN == 0 &&
           ((M + BIG_BM - 1) / BIG_BM) * (N / BIG_BN) >= 256;
}

bool gemm_split_large_tiles() { return STTD_BIG_SPLIT != 0; }

static bool big_tiles_fit(const GemmArgs& g, GemmEpi epi) {
    if (epi == GEMM_QKROPE) return (!g.A_lo || STTD_BIG_SPLIT) && gemm_qkrope_fits(g.M, g.N, g.K, g.qk.d);
    if (g.M < 1024 || g.K % BIG_BK || (g.A_lo && !STTD_BIG_SPLIT)) return false;
    // split activations into a residual: the large tiles only when 256 x 128 tiles
    // fill the CUs; narrower grids lose to the 64-row tiles' split K (1224 rows,
    // 2048 columns: O 48 -> 58 us, down 122 -> 147 us on the large tiles)
    if (g.A_lo && epi == GEMM_RESID && ((g.M + BIG_BM - 1) / BIG_BM) * ((g.N + 127) / 128) < 256) return false;
    return !(epi == GEMM_SWIGLU && g.N % 128);
}

template <bool SPLIT>
static void launch_gemm_big_t(const GemmArgs& g, GemmEpi epi, hipStream_t s) {
    constexpr int WM = STTD_BIG_WM;
    const int tiles_m = (g.M + BIG_BM - 1) / BIG_BM;
    if (epi == GEMM_SWIGLU) {
        const int tiles_n = g.N / 128;
        launch_kernel(gemm_big_kernel<GEMM_SWIGLU, BIG_BN, 1, WM, SPLIT>, tiles_m * tiles_n, WM * 128, 0, s, g, tiles_m,
                      tiles_n);
        return;
    }
    // residual outputs too narrow to fill the CUs even with 256 x 128 tiles: two
    // K halves of each 256 x 256 tile, added into the residual with atomics
    // (measured at 1224 rows and 2048 columns: down 104 -> 89 us, O 46 -> 38 us;
    // at 4096 rows, where 256 x 128 tiles already make 256 workgroups, the split
    // was slower: O 55 -> 68 us, and down (K = 6144) 125 -> 137-144 us)
    const int tiles256 = tiles_m * ((g.N + BIG_BN - 1) / BIG_BN);
    const int tiles128 = tiles_m * ((g.N + 127) / 128);
    if (epi == GEMM_RESID && tiles128 < 256 && tiles256 % 8 == 0 && (g.K / BIG_BK) % 2 == 0 &&
        g.K / BIG_BK >= 16) {
        launch_kernel(gemm_big_kernel<GEMM_RESID, BIG_BN, 2, WM, SPLIT>, tiles256 * 2, WM * 128, 0, s, g, tiles_m,
                      (g.N + BIG_BN - 1) / BIG_BN);
        return;
    }
    // narrow outputs: 128-column tiles so that about a full wave of workgroups runs
    const bool narrow = tiles256 < 256;
    const int bn = narrow ? 128 : BIG_BN;
    const int tiles_n = (g.N + bn - 1) / bn;
    const int grid = tiles_m * tiles_n;
    if (epi == GEMM_RESID) {
        if (narrow) launch_kernel(gemm_big_kernel<GEMM_RESID, 128, 1, WM, SPLIT>, grid, WM * 128, 0, s, g, tiles_m, tiles_n);
        else launch_kernel(gemm_big_kernel<GEMM_RESID, BIG_BN, 1, WM, SPLIT>, grid, WM * 128, 0, s, g, tiles_m, tiles_n);
    } else {
        if (narrow) launch_kernel(gemm_big_kernel<GEMM_STORE, 128, 1, WM, SPLIT>, grid, WM * 128, 0, s, g, tiles_m, tiles_n);
        else launch_kernel(gemm_big_kernel<GEMM_STORE, BIG_BN, 1, WM, SPLIT>, grid, WM * 128, 0, s, g, tiles_m, tiles_n);
    }
}

static void launch_gemm_big(const GemmArgs& g, GemmEpi epi, hipStream_t s) {
    if (epi == GEMM_QKROPE) {
        const int tiles_m = (g.M + BIG_BM - 1) / BIG_BM, tiles_n = g.N / BIG_BN;
        if (g.A_lo)
            launch_kernel(gemm_big_kernel<GEMM_QKROPE, BIG_BN, 1, STTD_BIG_WM, true>, tiles_m * tiles_n,
                          STTD_BIG_WM * 128, 0, s, g, tiles_m, tiles_n);
        else
            launch_kernel(gemm_big_kernel<GEMM_QKROPE, BIG_BN>, tiles_m * tiles_n, STTD_BIG_WM * 128, 0, s, g, tiles_m,
                          tiles_n);
        return;
    }
    if (g.A_lo && STTD_BIG_SPLIT) launch_gemm_big_t<true>(g, epi, s);
    else launch_gemm_big_t<false>(g, epi, s);
}

#ifndef STTD_SKINNY_CA
#define STTD_SKINNY_CA 1
#endif
#ifndef STTD_SKINNY_PD
#define STTD_SKINNY_PD 8
#endif
// SWIGLU column fragments per workgroup (gate + up rows, so CF * 8 act columns). 3 makes
// the 1.7B FFN (6144 act columns) exactly 256 workgroups, one per CU: 16-row gate_up
// 16.1 -> 13.6 us against 4 (192 workgroups, a quarter of the CUs idle), 8.93k -> 9.34k
// tok/s batched. 2 (384 workgroups, each re-reading the activation rows) measured slower
// than 4 (16.0 -> 17.1 us)
#ifndef STTD_SKINNY_SW_CF
#define STTD_SKINNY_SW_CF 3
#endif
#ifndef STTD_SKINNY_PD_SW
#define STTD_SKINNY_PD_SW 2
#endif
// Two values split as split_bf16 does (hi = bf16(v), lo = bf16(v - hi), nearest even),
// each pair packed (element 0 in the low half): one v_cvt_pk_bf16_f32 per pair and
// part instead of one per value, and no packing shifts (the skinny NORM loop's
// per-step VALU count 81 -> about 48)
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
    const float ha = __uint_as_float(hi << 16), hb = __uint_as_float(hi & 0xFFFF0000u);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a - ha, b - hb}, bf16x2_t));
}

// ------------------------------------------------------------------ few rows (decode batches)
// C[R, N] (+)= A[R, K] W[N, K]^T for R <= 16 RF rows: weight-stationary MFMA.
// Each workgroup owns CF column fragments of 16 (SWIGLU: the gate and the up
// fragment of 16 act columns) and a share of K, split over its 4 waves and
// over gridDim.y workgroups (RESID only; those add into C with atomics). Weight
// rows stream from global memory straight into B fragments (lane l: column
// l % 16, K elements (l / 16) * 8 .. + 8), so every weight byte is read once;
// the few activation rows (bf16 high and low parts, or the fp32 rows under NORM)
// are the A fragments, re-read from L2 by every workgroup. Up to 32 rows they come
// in whole-row pieces through a wave-private LDS area (CA below): at 16 rows that
// took the 28-block batched decode from 7.97k to 8.61k tok/s (down 10.8 -> 8.4 us,
// O 4.5 -> 3.7, gate_up 17.4 -> 16.3, QKV 8.1 -> 7.7). Loads run PD K-steps ahead.
// NORM: the rows' RMSNorm is done here (STORE and SWIGLU, whose workgroups each
// cover all of K): the A fragments are the fp32 rows times the gain, split into
// bf16 high + low parts in registers, the sums of squares come from the same
// loads, and the outputs are scaled by each row's 1 / rms.
template <int EPI, int RF, int CF, bool NORM>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs g) {
    // K-steps of 32 per load batch. With fragment-shaped activation loads, 8 measured
    // slower (gate_up 17.4 -> 18.0 us, down 10.8 -> 11.7 us), and two alternating
    // batches of 4 too (QKV 7.6 -> 9.0 us, down 10.8 -> 13.0 us). With row-piece
    // activation loads (CA): 8 for the single-fragment-row STORE / RESID forms (at 16 rows
    // QKV 7.62 -> 7.44 us, O 3.66 -> 3.47, down 8.40 -> 8.18 against 4; 8.62k -> 8.69k
    // tok/s), 2 for SWIGLU at 3 fragments (gate_up 13.6 us against 15.0 with 1, 15.5 with 3,
    // 13.9 with 4 and 15.7 with 8; at 4 fragments 4 was best: 16.0 against 18.2 with 8 and
    // 16.1 with 2) and 4 for wider row counts (2 measured slower everywhere)
    constexpr int PD = RF > 1 ? 4 : (EPI == GEMM_SWIGLU ? STTD_SKINNY_PD_SW : STTD_SKINNY_PD);
    __shared__ float red[4][RF * 16][CF * 16 + 1];
    __shared__ float ssred[NORM ? 4 : 1][RF * 16];
    // CA: the activation rows come in whole-row pieces (two fp32 rows or four bf16 rows
    // of a batch per wave instruction) into a wave-private LDS area, and the fragments
    // are read from there: a fragment-shaped load (16 rows x 64 B per instruction)
    // reads L2 at about a third of the rate of row-shaped ones. Rows padded by 16 B so
    // the 16 rows of a fragment read fall in distinct banks.
    constexpr bool CA = STTD_SKINNY_CA && RF * PD <= 8;  // the LDS areas fit beside the reduction
    constexpr int AROWS = RF * 16, AXS = PD * 32 + 4, AHS = PD * 32 + 8;
    constexpr int ABYTES = CA ? (NORM ? AROWS * AXS * 4 : 2 * AROWS * AHS * 2) : 16;
    __shared__ __attribute__((aligned(16))) unsigned char a_lds[4][ABYTES];
    clock_begin(g.clk);
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int ct = blockIdx.x;
    // weight row of each column fragment for this lane
    const uint16_t* wrow[CF];
    bool wok[CF];
#pragma unroll
    for (int f = 0; f < CF; ++f) {
        if (EPI == GEMM_SWIGLU) {
            // the tile's CF * 16 weight rows: the gate rows of its CF * 8 act columns,
            // then their up rows (an odd CF splits the middle fragment between the two)
            constexpr int GC = CF * 8;
            const int j = f * 16 + lane % 16;
            const int c = ct * GC + (j < GC ? j : j - GC);  // act column
            wok[f] = c < g.N;
            const int cc = wok[f] ? c : 0;
            wrow[f] = g.w[0] + (int64_t)(j < GC ? cc : g.N + cc) * g.K;
        } else {
            const int n0 = (ct * CF + f) * 16 + lane % 16;
            wok[f] = n0 < g.N;
            const int n = wok[f] ? n0 : 0;
            const bool s2 = n >= g.seg_end[1], s1 = n >= g.seg_end[0];
            const int grow = n - (s2 ? g.seg_end[1] : (s1 ? g.seg_end[0] : 0));
            wrow[f] = (s2 ? g.w[2] : (s1 ? g.w[1] : g.w[0])) + (int64_t)grow * g.K;
        }
    }
    const uint16_t* arow[RF];
    const uint16_t* alrow[RF];
    const float* xrow[RF];
#pragma unroll
    for (int r = 0; r < RF; ++r) {
        const int m = min(r * 16 + lane % 16, g.M - 1);
        if (NORM) {
            xrow[r] = g.X + (int64_t)m * g.ldx;
        } else {
            arow[r] = g.A + (int64_t)m * g.lda;
            alrow[r] = (g.A_lo ? g.A_lo : g.A) + (int64_t)m * g.lda;
        }
    }
    const bool lo = NORM ? g.x_lo : g.A_lo != nullptr;
    float ss[RF];
#pragma unroll
    for (int r = 0; r < RF; ++r) ss[r] = 0.f;
    // this wave's K-steps: [s0, s1) of K / 32
    const int n_steps = g.K / 32;
    const int parts = gridDim.y * 4;
    const int per = (n_steps + parts - 1) / parts;
    const int s0 = min((int)(blockIdx.y * 4 + wave) * per, n_steps);
    const int s1 = min(s0 + per, n_steps);
    const int koff = (lane / 16) * 8;

    f32x4 acc[RF][CF];
#pragma unroll
    for (int r = 0; r < RF; ++r)
#pragma unroll
        for (int f = 0; f < CF; ++f) acc[r][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 wb[PD][CF], ab[PD][RF], alb[PD][RF], gb[PD];
    f32x4 xa[PD][RF], xb[PD][RF];
    for (int s = s0; s < s1; s += PD) {
        // a batch of PD steps (clamped reads past s1 are loaded but not used)
        // row-piece loads per lane: a batch of a row is PD * 32 elements, in 16-byte
        // pieces of 4 fp32 (8 PD per row) or 8 bf16 (4 PD per row and plane)
        constexpr int PPR = NORM ? 8 * PD : 4 * PD;               // pieces per row (and plane)
        constexpr int NAP = AROWS * PPR / 64;                      // loads per lane and plane
        constexpr int NAI = CA ? (NORM ? NAP : 2 * NAP) : 1;
        u32x4 areg[NAI];
        if constexpr (CA) {
            // row pieces, issued before the weight loads so their wait leaves those in flight
#pragma unroll
            for (int i = 0; i < NAI; ++i) {
                // piece e of the plane: row e / PPR, element c of the row's batch
                const int e = (i % NAP) * 64 + lane;
                const int row = min(e / PPR, g.M - 1), c = (e % PPR) * (NORM ? 4 : 8);
                const int64_t kk = (int64_t)min(s + c / 32, n_steps - 1) * 32 + c % 32;
                if (NORM) {
                    areg[i] = *reinterpret_cast<const u32x4*>(g.X + (int64_t)row * g.ldx + kk);
                } else {  // loads [0, NAP) the high plane, then the low one
                    const uint16_t* base = i < NAP ? g.A : (g.A_lo ? g.A_lo : g.A);
                    areg[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)row * g.lda + kk);
                }
            }
        }
#pragma unroll
        for (int p = 0; p < PD; ++p) {
            const int k = min(s + p, n_steps - 1) * 32 + koff;
#pragma unroll
            for (int f = 0; f < CF; ++f) wb[p][f] = *reinterpret_cast<const u32x4*>(wrow[f] + k);
            if (CA) {
                if (NORM) gb[p] = *reinterpret_cast<const u32x4*>(g.gain + k);
            } else if (NORM) {
                gb[p] = *reinterpret_cast<const u32x4*>(g.gain + k);
#pragma unroll
                for (int r = 0; r < RF; ++r) {
                    xa[p][r] = *reinterpret_cast<const f32x4*>(xrow[r] + k);
                    xb[p][r] = *reinterpret_cast<const f32x4*>(xrow[r] + k + 4);
                }
            } else {
#pragma unroll
                for (int r = 0; r < RF; ++r) {
                    ab[p][r] = *reinterpret_cast<const u32x4*>(arow[r] + k);
                    if (lo) alb[p][r] = *reinterpret_cast<const u32x4*>(alrow[r] + k);
                }
            }
        }
        if constexpr (CA) {
            // the wave's own LDS area: write the row pieces, read the fragments back
            // (a wave's LDS operations complete in order, so no barrier)
            if (NORM) {
                float* ax = reinterpret_cast<float*>(a_lds[wave]);
#pragma unroll
                for (int i = 0; i < NAI; ++i) {
                    const int e = i * 64 + lane;
                    *reinterpret_cast<u32x4*>(&ax[(e / PPR) * AXS + (e % PPR) * 4]) = areg[i];
                }
#pragma unroll
                for (int p = 0; p < PD; ++p)
#pragma unroll
                    for (int r = 0; r < RF; ++r) {
                        const float* src = &ax[(r * 16 + lane % 16) * AXS + p * 32 + koff];
                        xa[p][r] = *reinterpret_cast<const f32x4*>(src);
                        xb[p][r] = *reinterpret_cast<const f32x4*>(src + 4);
                    }
            } else {
                uint16_t* ah = reinterpret_cast<uint16_t*>(a_lds[wave]);
#pragma unroll
                for (int i = 0; i < NAI; ++i) {
                    const int pl = i / NAP, e = (i % NAP) * 64 + lane;
                    *reinterpret_cast<u32x4*>(&ah[(pl * AROWS + e / PPR) * AHS + (e % PPR) * 8]) = areg[i];
                }
#pragma unroll
                for (int p = 0; p < PD; ++p)
#pragma unroll
                    for (int r = 0; r < RF; ++r) {
                        const int o = (r * 16 + lane % 16) * AHS + p * 32 + koff;
                        ab[p][r] = *reinterpret_cast<const u32x4*>(&ah[o]);
                        alb[p][r] = *reinterpret_cast<const u32x4*>(&ah[AROWS * AHS + o]);
                    }
            }
        }
#pragma unroll
        for (int p = 0; p < PD; ++p) {
            if (s + p >= s1) break;
            if (NORM) {  // x * gain as bf16 high + low parts; x^2 into the row's sum
                const uint32_t gw[4] = {gb[p].x, gb[p].y, gb[p].z, gb[p].w};
#pragma unroll
                for (int r = 0; r < RF; ++r) {
                    const float xv[8] = {xa[p][r].x, xa[p][r].y, xa[p][r].z, xa[p][r].w,
                                         xb[p][r].x, xb[p][r].y, xb[p][r].z, xb[p][r].w};
                    uint32_t hw[4], lw[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        ss[r] = fmaf(xv[2 * i], xv[2 * i], ss[r]);
                        ss[r] = fmaf(xv[2 * i + 1], xv[2 * i + 1], ss[r]);
                        split_bf16x2(xv[2 * i] * __uint_as_float(gw[i] << 16),
                                     xv[2 * i + 1] * __uint_as_float(gw[i] & 0xFFFF0000u), hw[i], lw[i]);
                    }
                    ab[p][r] = u32x4{hw[0], hw[1], hw[2], hw[3]};
                    alb[p][r] = u32x4{lw[0], lw[1], lw[2], lw[3]};
                }
            }
#pragma unroll
            for (int r = 0; r < RF; ++r)
#pragma unroll
                for (int f = 0; f < CF; ++f) {
                    const bf16x8 bw = __builtin_bit_cast(bf16x8, wb[p][f]);
                    acc[r][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ab[p][r]), bw,
                                                                        acc[r][f], 0, 0, 0);
                    if (lo)
                        acc[r][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, alb[p][r]),
                                                                            bw, acc[r][f], 0, 0, 0);
                }
        }
    }
    // merge the 4 waves' K shares (and the rows' sums of squares: lanes l, l + 16,
    // l + 32, l + 48 hold row l % 16's)
#pragma unroll
    for (int r = 0; r < RF; ++r)
#pragma unroll
        for (int f = 0; f < CF; ++f)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave][r * 16 + (lane / 16) * 4 + i][f * 16 + lane % 16] = acc[r][f][i];
    if (NORM) {
#pragma unroll
        for (int r = 0; r < RF; ++r) {
            float t = ss[r] + xor16(ss[r]);
            t += xor32(t);
            if (lane < 16) ssred[wave][r * 16 + lane] = t;
        }
    }
    __syncthreads();
    constexpr int OUTS = RF * 16 * CF * 16;
    for (int o = tid; o < OUTS; o += 256) {
        const int row = o / (CF * 16), col = o % (CF * 16);
        if (row >= g.M) continue;
        float v = red[0][row][col] + red[1][row][col] + red[2][row][col] + red[3][row][col];
        float rs = 1.f;
        if (NORM) {
            rs = 1.0f / sqrtf((ssred[0][row] + ssred[1][row] + ssred[2][row] + ssred[3][row]) / (float)g.K + g.eps);
            v *= rs;
        }
        if (EPI == GEMM_SWIGLU) {
            constexpr int GC = CF * 8;  // gate columns of the tile; the up ones follow
            if (col >= GC) continue;  // the up half is read with its gate
            const int c = ct * GC + col;
            if (c >= g.N) continue;
            const float up = (red[0][row][col + GC] + red[1][row][col + GC] + red[2][row][col + GC] +
                              red[3][row][col + GC]) * rs;
            const float a = v / (1.0f + expf(-v)) * up;
            uint16_t hi, lo16;
            split_bf16(a, hi, lo16);
            g.Cb[(int64_t)row * g.ldcb + c] = hi;
            if (g.Cb_lo) g.Cb_lo[(int64_t)row * g.ldcb + c] = lo16;
        } else {
            const int n = ct * CF * 16 + col;
            if (n >= g.N) continue;
            float* dst = g.C + (int64_t)row * g.ldc + n;
            if (EPI == GEMM_STORE) *dst = v;
            else if (gridDim.y == 1) *dst += v;
            else atomicAdd(dst, v);
        }
    }
    clock_end(g.clk);
}

// Grid bound of few-row RESID launches that split K (atomic adds). At 16 rows,
// 512 and 1024 measured slower (down 12.3 -> 12.8 and 15.8 us): every split adds
// rows x N atomics. Again with the row-piece activation loads: 512 took O 3.44 -> 5.18
// us and down 8.32 -> 9.51 (with batches of 4 K-steps 4.20 and 8.62). Splitting the K of STORE and SWIGLU launches too, with the
// column tile's last workgroup merging the published partials, measured slower at
// 384-1024 workgroups (gate_up 18.0 -> 23.8-25.7 us, QKV 8.2 -> 10.4-11.2 us). So
// did staging the 16 activation rows once per workgroup in LDS (128 KB, normed and
// split on the way in) with only weight loads in the K loop, two batches in
// flight: gate_up 17.4 -> 21.4 us, QKV (32 columns per workgroup) 8.1 -> 15.0 us.
// So did 8 waves per workgroup splitting K eight ways (two waves per SIMD, twice
// the loads in flight per CU): 16 rows, 7.99k -> 7.93k tok/s, down 10.8 -> 11.7 us;
// and again with the row-piece activation loads: QKV 7.43 -> 7.59 us, O 3.44 -> 4.64,
// down 8.29 -> 9.27, gate_up 13.6 -> 13.9.
// So did two batch buffers again with every load unconditional and the waits
// checked in the ISA to cover one step each (batches of 4, 3 and 2 steps): gate_up
// 16.8 -> 19.6, 20.1 and 18.0 us, 8.05k -> 7.38k, 7.25k and 7.88k tok/s.
// Column fragments per RESID workgroup. 2, with K split twice as often so the grid stays
// at 256 (half the activation bytes per workgroup, twice the atomic adds), measured
// slower at 16 rows: O 3.44 -> 4.82 us, down 8.28 -> 9.12 (with batches of 4 K-steps
// O 3.67, down 8.10, QKV 6.94 -> 7.43: 9.61k -> 9.58k tok/s)
#ifndef STTD_SKINNY_RESID_CF
#define STTD_SKINNY_RESID_CF 1
#endif
#ifndef STTD_SKINNY_RESID_WGS
#define STTD_SKINNY_RESID_WGS 256
#endif

// Rows a skinny launch takes (16 per row fragment, up to 4 fragments).
#ifndef STTD_SKINNY_MAX_ROWS
constexpr int kSkinnyMaxRows = 64;
#else
constexpr int kSkinnyMaxRows = STTD_SKINNY_MAX_ROWS;
#endif

template <int EPI, int CF, bool NORM = false>
static void launch_skinny_rf(const GemmArgs& g, dim3 grid, hipStream_t s) {
    if (g.M <= 16) launch_kernel(gemm_skinny_kernel<EPI, 1, CF, NORM>, grid, 256, 0, s, g);
    else if (g.M <= 32) launch_kernel(gemm_skinny_kernel<EPI, 2, CF, NORM>, grid, 256, 0, s, g);
    else launch_kernel(gemm_skinny_kernel<EPI, 4, CF, NORM>, grid, 256, 0, s, g);
}

static void launch_gemm_skinny(const GemmArgs& g, GemmEpi epi, hipStream_t s) {
    if (epi == GEMM_SWIGLU) {
        constexpr int SCF = STTD_SKINNY_SW_CF, ACOLS = SCF * 8;
        if (g.X) launch_skinny_rf<GEMM_SWIGLU, SCF, true>(g, dim3((g.N + ACOLS - 1) / ACOLS, 1), s);
        else launch_skinny_rf<GEMM_SWIGLU, SCF>(g, dim3((g.N + ACOLS - 1) / ACOLS, 1), s);
        return;
    }
    constexpr int RCF = STTD_SKINNY_RESID_CF;
    const int tiles = (g.N + 15) / 16;
    const int rtiles = (g.N + 16 * RCF - 1) / (16 * RCF);
    // RESID may split K over workgroups (atomic adds) until about 256 workgroups run
    int ks = 1;
    if (epi == GEMM_RESID)
        while (rtiles * ks * 2 <= STTD_SKINNY_RESID_WGS && g.K / 32 >= ks * 2 * 4 * 4) ks *= 2;
    if (epi == GEMM_RESID) launch_skinny_rf<GEMM_RESID, RCF>(g, dim3(rtiles, ks), s);
    else if (g.X) launch_skinny_rf<GEMM_STORE, 1, true>(g, dim3(tiles, 1), s);
    else launch_skinny_rf<GEMM_STORE, 1>(g, dim3(tiles, 1), s);
}

template <int BM, bool SPLIT>
static hipError_t launch_gemm_bm(const GemmArgs& g, GemmEpi epi, hipStream_t s) {
    constexpr int BN = 128;
    const unsigned gy = (g.M + BM - 1) / BM;
    if (epi == GEMM_SWIGLU) {
        // 64-column tiles (32 act columns) when 128-column ones would leave CUs idle
        if ((unsigned)(g.N / (BN / 2)) * gy < 512 && g.N % 32 == 0)
            launch_kernel(gemm_bf16_kernel<BM, 64, GEMM_SWIGLU, SPLIT>, dim3(g.N / 32, gy, 1), 256, 0, s, g);
        else
            launch_kernel(gemm_bf16_kernel<BM, BN, GEMM_SWIGLU, SPLIT>, dim3(g.N / (BN / 2), gy, 1), 256, 0, s, g);
        return hipSuccess;
    }
    dim3 grid((g.N + BN - 1) / BN, gy, 1);
    // Few workgroups: split K over them (atomic adds into C, which a STORE zeroes first)
    // while fewer than ~512 run (two per CU hide each K-step's load latency) and each
    // keeps >= 4 K-steps
    while (grid.x * grid.y * grid.z * 2 <= 512 && g.K / BK >= (int)grid.z * 2 * 4) grid.z *= 2;
    if (epi == GEMM_STORE && grid.z > 1 && g.ldc != g.N) grid.z = 1;  // zeroing needs contiguous rows
    if (epi == GEMM_STORE && grid.z > 1) {
        const hipError_t e = launch_fill_zero(g.C, (size_t)g.M * g.N * sizeof(float), s);
        if (e != hipSuccess) return e;
        launch_kernel(gemm_bf16_kernel<BM, BN, GEMM_RESID, SPLIT>, grid, 256, 0, s, g);
    } else if (epi == GEMM_RESID) {
        launch_kernel(gemm_bf16_kernel<BM, BN, GEMM_RESID, SPLIT>, grid, 256, 0, s, g);
    } else {
        launch_kernel(gemm_bf16_kernel<BM, BN, GEMM_STORE, SPLIT>, grid, 256, 0, s, g);
    }
    return hipSuccess;
}

#ifndef STTD_STREAM_D
#define STTD_STREAM_D 2
#endif
#ifndef STTD_STREAM_WGS
#define STTD_STREAM_WGS 256
#endif
#ifndef STTD_STREAM_FM
#define STTD_STREAM_FM 0
#endif
#ifndef STTD_STREAM_MAX_ROWS
#define STTD_STREAM_MAX_ROWS 320
#endif

template <int FM, bool SPLIT>
static hipError_t launch_gemm_stream_fm(const GemmArgs& g, GemmEpi epi, hipStream_t s) {
    constexpr int FN = 2, BN = FN * 64, D = STTD_STREAM_D;
    const unsigned gy = (g.M + FM * 16 - 1) / (FM * 16);
    if (epi == GEMM_SWIGLU) {
        launch_kernel(gemm_stream_kernel<GEMM_SWIGLU, FM, FN, D, SPLIT>, dim3((g.N + BN / 2 - 1) / (BN / 2), gy, 1),
                      256, 0, s, g);
        return hipSuccess;
    }
    dim3 grid((g.N + BN - 1) / BN, gy, 1);
    // split K over workgroups (atomic adds into C, which a STORE zeroes first) while
    // the grid stays within about STTD_STREAM_WGS and each split keeps 2 D K-steps
    while (grid.x * grid.y * grid.z * 2 <= STTD_STREAM_WGS && g.K / BK >= (int)grid.z * 2 * 2 * D) grid.z *= 2;
    if (epi == GEMM_STORE && grid.z > 1 && g.ldc != g.N) grid.z = 1;  // zeroing needs contiguous rows
    if (epi == GEMM_STORE && grid.z > 1) {
        const hipError_t e = launch_fill_zero(g.C, (size_t)g.M * g.N * sizeof(float), s);
        if (e != hipSuccess) return e;
        launch_kernel(gemm_stream_kernel<GEMM_RESID, FM, FN, D, SPLIT>, grid, 256, 0, s, g);
    } else if (epi == GEMM_RESID) {
        launch_kernel(gemm_stream_kernel<GEMM_RESID, FM, FN, D, SPLIT>, grid, 256, 0, s, g);
    } else {
        launch_kernel(gemm_stream_kernel<GEMM_STORE, FM, FN, D, SPLIT>, grid, 256, 0, s, g);
    }
    return hipSuccess;
}

// 80-row tiles where they pad fewer rows than 64-row ones (153 rows: 160 against 192).
// Up to 320 rows: at 1224 rows (the packed prompts' narrow O and down residuals)
// this kernel measured the same as the 64-row tiles (down 123 -> 125 us).
template <bool SPLIT>
static hipError_t launch_gemm_stream(const GemmArgs& g, GemmEpi epi, hipStream_t s) {
    const int pad64 = (g.M + 63) / 64 * 64, pad80 = (g.M + 79) / 80 * 80;
    if (STTD_STREAM_FM == 4) return launch_gemm_stream_fm<4, SPLIT>(g, epi, s);
    if (STTD_STREAM_FM == 5) return launch_gemm_stream_fm<5, SPLIT>(g, epi, s);
    // residual outputs over a short K (the O projection) keep 64-row tiles: at 153 rows
    // O 14.0 -> 12.2 us with them, while down (K = 6144) 22.8 -> 25.5, gate_up 38.2 ->
    // 43.4; requiring twice the K-steps per split instead (8 -> 4 splits) left O at 13.9
    if (epi == GEMM_RESID && g.K <= 2048) return launch_gemm_stream_fm<4, SPLIT>(g, epi, s);
    return pad80 < pad64 ? launch_gemm_stream_fm<5, SPLIT>(g, epi, s) : launch_gemm_stream_fm<4, SPLIT>(g, epi, s);
}

// 64-row tiles. One 160-row tile per workgroup (every row of a 153-row prefill, so
// each weight tile streams once) measured slower at 153 rows: gate_up 42.8 -> 59.4 us,
// QKV 19.3 -> 26.2, O 14.3 -> 18.2, down 24.7 -> 31.5 (fewer, larger workgroups at
// one or two waves per SIMD hide less of each K-step's load latency).
template <bool SPLIT>
static hipError_t launch_gemm_t(const GemmArgs& g, GemmEpi epi, hipStream_t s) {
    if (g.M <= STTD_STREAM_MAX_ROWS) return launch_gemm_stream<SPLIT>(g, epi, s);
    return launch_gemm_bm<64, SPLIT>(g, epi, s);
}

bool gemm_fuses_norm(int M, int K) { return M <= kSkinnyMaxRows && K % 32 == 0; }

hipError_t launch_gemm(const GemmArgs& args, GemmEpi epi, hipStream_t s) {
    if (args.M <= 0) return hipSuccess;
    GemmArgs g = args;
    g.clk = clock_slot();
    if (epi == GEMM_QKROPE && !big_tiles_fit(g, epi)) return hipErrorInvalidValue;
    // the fused RMSNorm: STORE / SWIGLU on the few-row path only
    if (g.X && (epi == GEMM_RESID || epi == GEMM_QKROPE || !gemm_fuses_norm(g.M, g.K))) return hipErrorInvalidValue;
    if (g.M <= kSkinnyMaxRows && g.K % 32 == 0) launch_gemm_skinny(g, epi, s);
    else if (big_tiles_fit(g, epi)) launch_gemm_big(g, epi, s);
    else if (g.A_lo) {
        const hipError_t e = launch_gemm_t<true>(g, epi, s);
        if (e != hipSuccess) return e;
    } else {
        const hipError_t e = launch_gemm_t<false>(g, epi, s);
        if (e != hipSuccess) return e;
    }
    return hipGetLastError();
}

}  // namespace sttd
