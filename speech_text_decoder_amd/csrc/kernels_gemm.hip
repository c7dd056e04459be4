// kernels_gemm.hip - bf16 MFMA GEMM for prefill rows: C[M, N] = A[M, K] W[N, K]^T
// with fp32 accumulation, and the block's epilogues fused behind it:
//   STORE   C = A W^T (the Q|K|V projections, three weight segments stacked)
//   RESID   C += A W^T (O and down projections add into the residual stream)
//   SWIGLU  act[:, n] = silu(g) * u with g, u the packed gate_up outputs n and I + n
//
// Tile BM x BN x 64 per workgroup of 4 waves (2 x 2); each wave computes a
// (BM/2) x (BN/2) block with v_mfma_f32_16x16x32_bf16. A and W tiles are staged
// through LDS (rows padded to 72 bf16 so the 16-lane column reads of the
// fragments hit distinct banks); the next K tile is fetched into registers
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
constexpr int LDS_STRIDE = BK + 8;  // bf16 elements per staged row

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
        *reinterpret_cast<u32x4*>(&lds[(v / (BK / 8)) * LDS_STRIDE + (v % (BK / 8)) * 8]) = reg[i];
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
            const int n = tile_n * BN + r;
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

    const int nk = g.K / BK;
    auto fetch = [&](int64_t k0) {
        fetch_rows<A_VECS>(areg, arow_ptr, arow_ok, k0);
        if (SPLIT) fetch_rows<A_VECS>(alreg, alo_ptr, arow_ok, k0);
        fetch_rows<B_VECS>(breg, brow_ptr, brow_ok, k0);
    };
    auto stash = [&]() {
        stash_rows<A_VECS>(areg, As, tid);
        if (SPLIT) stash_rows<A_VECS>(alreg, Als, tid);
        stash_rows<B_VECS>(breg, Bs, tid);
    };
    fetch(0);
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
                const int o = (wm * (BM / 2) + i * 16 + lane % 16) * LDS_STRIDE + kc;
                af[i] = *reinterpret_cast<const bf16x8*>(&As[o]);
                if (SPLIT) afl[i] = *reinterpret_cast<const bf16x8*>(&Als[o]);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8*>(&Bs[(bfrag_row[j] + lane % 16) * LDS_STRIDE + kc]);
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
                    float* dst = g.C + (int64_t)m * g.ldc + n;
                    if (EPI == GEMM_RESID) *dst += acc[i][j][rr];
                    else *dst = acc[i][j][rr];
                }
            }
        }
    }
    clock_end(g.clk);
}

template <bool SPLIT>
static void launch_gemm_t(const GemmArgs& g, GemmEpi epi, hipStream_t s) {
    constexpr int BM = 64, BN = 128;
    dim3 grid(epi == GEMM_SWIGLU ? g.N / (BN / 2) : g.N / BN, (g.M + BM - 1) / BM);
    if (epi == GEMM_SWIGLU) gemm_bf16_kernel<BM, BN, GEMM_SWIGLU, SPLIT><<<grid, 256, 0, s>>>(g);
    else if (epi == GEMM_RESID) gemm_bf16_kernel<BM, BN, GEMM_RESID, SPLIT><<<grid, 256, 0, s>>>(g);
    else gemm_bf16_kernel<BM, BN, GEMM_STORE, SPLIT><<<grid, 256, 0, s>>>(g);
}

hipError_t launch_gemm(const GemmArgs& args, GemmEpi epi, hipStream_t s) {
    if (args.M <= 0) return hipSuccess;
    GemmArgs g = args;
    g.clk = clock_slot();
    if (g.A_lo) launch_gemm_t<true>(g, epi, s);
    else launch_gemm_t<false>(g, epi, s);
    return hipGetLastError();
}

}  // namespace sttd
