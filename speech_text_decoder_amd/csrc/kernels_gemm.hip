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
// Fragment layout of v_mfma_f32_16x16x32_bf16 (checked on the device): lane l
// supplies row l%16 and K elements (l/16)*8 .. +8 of both operands; the 16x16
// result gives lane l column l%16 and rows (l/16)*4 + i, i < 4.
#include "common.h"
#include "launch.h"

namespace sttd {

constexpr int BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // bf16 elements per staged row

template <int AV, int BV>
__device__ __forceinline__ void gemm_fetch(u32x4 (&areg)[AV], u32x4 (&breg)[BV], const uint16_t* const (&ap)[AV],
                                           const bool (&aok)[AV], const uint16_t* const (&bp)[BV], int k0) {
#pragma unroll
    for (int i = 0; i < AV; ++i)
        areg[i] = aok[i] ? *reinterpret_cast<const u32x4*>(ap[i] + k0) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < BV; ++i) breg[i] = *reinterpret_cast<const u32x4*>(bp[i] + k0);
}

template <int AV, int BV>
__device__ __forceinline__ void gemm_stash(const u32x4 (&areg)[AV], const u32x4 (&breg)[BV], uint16_t* As,
                                           uint16_t* Bs, int tid) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
        const int v = tid + i * 256;
        *reinterpret_cast<u32x4*>(&As[(v / (BK / 8)) * LDS_STRIDE + (v % (BK / 8)) * 8]) = areg[i];
    }
#pragma unroll
    for (int i = 0; i < BV; ++i) {
        const int v = tid + i * 256;
        *reinterpret_cast<u32x4*>(&Bs[(v / (BK / 8)) * LDS_STRIDE + (v % (BK / 8)) * 8]) = breg[i];
    }
}

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs g) {
    constexpr int FM = BM / 32;  // 16-row fragments per wave
    constexpr int FN = BN / 32;  // 16-col fragments per wave
    constexpr int A_VECS = BM * BK / 8 / 256;
    constexpr int B_VECS = BN * BK / 8 / 256;
    __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDS_STRIDE];

    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int wm = wave / 2, wn = wave % 2;
    const int m0 = blockIdx.y * BM;
    const int tile_n = blockIdx.x;

    // Global source row of each staged B row.
    const uint16_t* brow_ptr[B_VECS];
#pragma unroll
    for (int i = 0; i < B_VECS; ++i) {
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
    bool arow_ok[A_VECS];
#pragma unroll
    for (int i = 0; i < A_VECS; ++i) {
        const int v = tid + i * 256;
        const int r = v / (BK / 8);
        arow_ok[i] = (m0 + r) < g.M;
        arow_ptr[i] = g.A + (int64_t)(arow_ok[i] ? m0 + r : 0) * g.lda + (v % (BK / 8)) * 8;
    }

    u32x4 areg[A_VECS], breg[B_VECS];
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
    gemm_fetch<A_VECS, B_VECS>(areg, breg, arow_ptr, arow_ok, brow_ptr, 0);
    gemm_stash<A_VECS, B_VECS>(areg, breg, As, Bs, tid);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) gemm_fetch<A_VECS, B_VECS>(areg, breg, arow_ptr, arow_ok, brow_ptr, (kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            bf16x8 af[FM], bfr[FN];
            const int kc = ks * 32 + (lane / 16) * 8;
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(&As[(wm * (BM / 2) + i * 16 + lane % 16) * LDS_STRIDE + kc]);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8*>(&Bs[(bfrag_row[j] + lane % 16) * LDS_STRIDE + kc]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
        if (kt + 1 < nk) {
            gemm_stash<A_VECS, B_VECS>(areg, breg, As, Bs, tid);
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
                    g.Cb[(int64_t)m * g.ldcb + c] = f32_to_bf16_bits(a);
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
}

hipError_t launch_gemm(const GemmArgs& g, GemmEpi epi, hipStream_t s) {
    if (g.M <= 0) return hipSuccess;
    constexpr int BM = 64, BN = 128;
    dim3 grid(epi == GEMM_SWIGLU ? g.N / (BN / 2) : g.N / BN, (g.M + BM - 1) / BM);
    if (epi == GEMM_SWIGLU) gemm_bf16_kernel<BM, BN, GEMM_SWIGLU><<<grid, 256, 0, s>>>(g);
    else if (epi == GEMM_RESID) gemm_bf16_kernel<BM, BN, GEMM_RESID><<<grid, 256, 0, s>>>(g);
    else gemm_bf16_kernel<BM, BN, GEMM_STORE><<<grid, 256, 0, s>>>(g);
    return hipGetLastError();
}

}  // namespace sttd
