// launch.h - host-side launchers of the gfx950 kernels (internal to libsttd).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace sttd {

// Per-kernel event timing (sttd_profile_enable): while a timed kernel family's
// eager call is being issued, each of its launches takes a start/stop event pair
// (true) that hipExtLaunchKernel binds to the dispatch itself, so the pair times
// that kernel alone (dispatch to completion), not the gaps around it.
bool next_launch_events(hipEvent_t* start, hipEvent_t* stop);

template <typename Tup, size_t... I>
inline void tuple_addresses(Tup& t, void** out, std::index_sequence<I...>) {
    ((out[I] = (void*)&std::get<I>(t)), ...);
}

// kernel<<<grid, block, shmem, s>>>(args...), with the event pair above when timed.
template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t s,
                          Args&&... args) {
    hipEvent_t start = nullptr, stop = nullptr;
    if (next_launch_events(&start, &stop)) {
        std::tuple<KArgs...> t(std::forward<Args>(args)...);
        void* argv[sizeof...(KArgs)];
        tuple_addresses(t, argv, std::index_sequence_for<KArgs...>{});
        (void)hipExtLaunchKernel((const void*)kernel, grid, block, argv, shmem, s, start, stop, 0);
        return;
    }
    kernel<<<grid, block, shmem, s>>>(std::forward<Args>(args)...);
}

// Device-clock slot: kClockEntries (start, end) pairs, one per workgroup id;
// ids from kClockBank1 up belong to a second kernel launched under the slot.
constexpr int kClockEntries = 16384;
constexpr int kClockBank1 = 12288;

// Up to this many attention splits the O-projection GEMV merges the partials
// itself (GemvArgs::xpart); above, a combine pass writes the merged rows.
constexpr int kMergeMaxSplits = 8;

// Clock slot of the launch being issued when device-clock timing is on, else
// nullptr (kClockEntries (start, end) pairs, see common.h).
uint64_t* clock_slot();
// out[2i], out[2i+1] = first start and last end recorded in slot i (~0, 0 if none).
hipError_t launch_clock_reduce(const uint64_t* slots, int n, uint64_t* out, hipStream_t s);

enum WType { W_F32 = 0, W_BF16 = 1 };
enum KVType { KV_F32 = 0, KV_F16 = 2 };

// Where a row of a block call sits: position and KV slab, either per row from
// device arrays or pos0 + row / seq0 for a prefill.
struct RowMap {
    const int32_t* pos;  // device [rows] or nullptr: row r at pos0 + r
    const int32_t* seq;  // device [rows] or nullptr: seq0, or row r's own slab r when seq0 < 0
    int pos0, seq0;
};

__device__ __forceinline__ int row_pos(const RowMap& m, int r) { return m.pos ? m.pos[r] : m.pos0 + r; }
__device__ __forceinline__ int row_seq(const RowMap& m, int r) { return m.seq ? m.seq[r] : (m.seq0 < 0 ? r : m.seq0); }

// Sequences packed back to back in one batched prefill call: sequence i holds
// rows [start[i], start[i] + len[i]) at positions pos0[i].. of slab seq[i].
constexpr int kMaxSegments = 64;
struct Segments {
    int n;
    int start[kMaxSegments], len[kMaxSegments], pos0[kMaxSegments], seq[kMaxSegments];
};
// pos[r], seq[r] of every packed row r < R.
hipError_t launch_expand_segments(const Segments& sg, int R, int32_t* pos, int32_t* seq, hipStream_t s);

// KV slab addressing for one layer: slab s, head j, row c at
// base + ((s * n_kv + j) * n_ctx + c) * d elements.
struct KVLayer {
    void* k;
    void* v;
    int n_seq, n_kv, n_ctx, d;
    KVType type;
};

// Everything one (row, head) item of the per-head Q/K RMSNorm + RoPE + KV
// write needs (qk_head_item in headops.h).
struct QkRope {
    const void* q_gain;
    const void* k_gain;
    float eps;
    const float* rope;   // [max_pos][d/2] (cos, sin)
    int max_pos;
    RowMap rm;
    KVLayer kv;
    void* q_out;         // [rows][n_heads * d], fp32 or f16 (q_f16)
    bool q_f16;
    int64_t ldq;
    uint32_t* err;
    int n_heads, n_kv, d;
    uint64_t* clk;
};

// ---- norms, rotary, gathers (kernels_misc.hip)
// out[r, :] = x[r, :] / sqrt(mean(x[r]^2) + eps) * gain, rows r < R; out bf16.
// With out_lo, the value is also split: out = bf16(v), out_lo = bf16(v - out).
// With xrow, output row r normalises input row xrow[r] (an index outside
// [0, n_xrows) reads row 0 and records kDevErrRow in err).
constexpr uint32_t kDevErrRow = 16u;  // STTD_DEVERR_ROW
hipError_t launch_rmsnorm_rows_bf16(const float* x, int64_t ldx, const void* gain, WType gt, uint16_t* out,
                                    uint16_t* out_lo, int64_t ldo, int R, int H, float eps, hipStream_t s,
                                    const int32_t* xrow = nullptr, int n_xrows = 0, uint32_t* err = nullptr);
// Per-head Q/K RMSNorm + NeoX RoPE (table) + K/V cache write; q written to q_out
// as fp32 (q_f16 false) or f16 (q_f16 true) with row stride ldq.
hipError_t launch_qk_norm_rope_kv(const float* qkv, int64_t ldqkv, int R, WType gt, const QkRope& q, hipStream_t s);
// x[b] = embed[ids[b]] * (keep ? keep[b] : 1) + (dense ? dense[b] : 0), b < B
hipError_t launch_embed_gather(const void* embed, WType wt, int vocab, int hidden, int B, const int32_t* ids,
                               const float* keep, const float* dense, float* x, uint32_t* err, hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
// Greedy stopping rules after a head call (see sttd_greedy_stop).
hipError_t launch_greedy_stop(int B, const int32_t* ids, int eos_id, int max_new, int n_ctx, int advance,
                              int32_t* pos, int32_t* active, int32_t* n_gen, int32_t* tokens, int32_t* truncated,
                              int32_t* n_active, hipStream_t s);

// ---- GEMV family (kernels_gemv.hip): rows <= 4 per group, fp32 activations.
enum GemvEpi { GEMV_STORE = 0, GEMV_RESID = 1, GEMV_SWIGLU = 2 };
struct GemvArgs {
    const void* w[3];    // up to three weight segments stacked along the output
    int seg_end[3];      // cumulative output-row ends of the segments
    int N;               // output columns (SWIGLU: I, the gate rows; up row of n is n + I)
    int K;               // reduction length
    const float* x;      // activation rows [rows, K] (ldx)
    int64_t ldx;
    int rows;
    const void* gain;    // fused RMSNorm gain over K (nullptr: no norm)
    float eps;
    float* y;            // output rows (ldy)
    int64_t ldy;
    const float* resid;  // RESID: y = resid + x W^T (may equal y)
    int64_t ldr;
    // Optional: the activation rows are attention split partials to merge on
    // load: records [m, l, -, -, o[head_dim]] at ((row * (K / head_dim) + h) *
    // n_splits + s) * (head_dim + 4); x[row][h * head_dim + e] = sum_s 2^(m_s - M)
    // o_s[e] / sum_s 2^(m_s - M) l_s.
    const float* xpart;
    int n_splits;
    int head_dim;
    uint64_t* clk;
};
hipError_t launch_gemv(const GemvArgs& a, WType wt, GemvEpi epi, hipStream_t s);

// Final RMSNorm + tied head + argmax (kernels_gemv.hip).
struct HeadArgs {
    const void* gain;
    const void* embed;
    int vocab, hidden;
    float eps;
    const float* x;
    int64_t ldx;
    int rows;
    const int32_t* xrow; // optional [rows]: row b reads x + xrow[b] * ldx (else x + b * ldx)
    int n_xrows;         // with xrow: rows x holds; an index outside [0, n_xrows) reads row 0 and flags kDevErrRow
    int32_t* ids;
    float* logits;       // optional [rows, vocab]
    float* next_x;       // optional [rows, hidden]
    int32_t* pos;        // optional, += 1
    unsigned long long* partials;  // [rows][max_partials] per-workgroup best keys
    int max_partials;              // workgroups of the head GEMV (its grid width)
    uint32_t* err;
    uint16_t* zbuf;      // optional scratch of 2 * rows * hidden bf16: lets batches of rows take the MFMA head
    uint64_t* clk;
};
hipError_t launch_lm_head_argmax(const HeadArgs& a, WType wt, hipStream_t s);

// ---- MFMA GEMM (kernels_gemm.hip): C = A W^T, A bf16 [M, K], W bf16 [N, K].
// GEMM_QKROPE: the Q|K|V projection of a prefill with the per-head Q/K RMSNorm,
// NeoX RoPE, f16 query write and cache write done in the epilogue (GemmArgs::qk;
// large-M tiles only, see gemm_qkrope_fits)
enum GemmEpi { GEMM_STORE = 0, GEMM_RESID = 1, GEMM_SWIGLU = 2, GEMM_QKROPE = 3 };
// A_lo (optional) holds bf16(a - bf16(a)) of every A element with the same
// stride: the product then takes A + A_lo, an activation operand with about
// 16 significant bits, at twice the MFMA work (used where HBM bounds the GEMM).
// SWIGLU with Cb_lo writes the act output split the same way.
struct GemmArgs {
    const uint16_t* A;
    const uint16_t* A_lo;
    int64_t lda;
    int M, K;
    const uint16_t* w[3];
    int seg_end[3];
    int N;               // STORE/RESID: output columns; SWIGLU: I (act columns)
    float* C;            // STORE / RESID output (fp32, ldc)
    int64_t ldc;
    uint16_t* Cb;        // SWIGLU output (bf16, ldcb)
    uint16_t* Cb_lo;     // optional low half of the SWIGLU output
    int64_t ldcb;
    QkRope qk;           // GEMM_QKROPE: gains, table, row map, cache and q output (q_f16)
    // RMSNorm in front (STORE / SWIGLU on few rows, see gemm_fuses_norm): with X set,
    // A / A_lo are not read; the operand is X (fp32, ldx) times gain, split into bf16
    // high + low parts when x_lo, and each output row is scaled by 1 / rms of its X row
    const float* X;
    int64_t ldx;
    const uint16_t* gain;
    float eps;
    bool x_lo;
    uint64_t* clk;
};
hipError_t launch_gemm(const GemmArgs& g, GemmEpi epi, hipStream_t s);
// Whether launch_gemm takes the RMSNorm of X itself (GemmArgs::X) for M rows over K:
// the few-row weight-stationary path. Otherwise the caller norms the rows first.
bool gemm_fuses_norm(int M, int K);
// Whether launch_gemm takes GEMM_QKROPE for this shape: at least 1024 rows,
// head_dim 128, and enough 256 x 256 tiles to fill the CUs.
bool gemm_qkrope_fits(int M, int N, int K, int head_dim);
// Whether the large tiles take split (hi/lo) activations (then GEMM_QKROPE does too).
bool gemm_split_large_tiles();

// ---- attention (kernels_attn.hip)
// Split-K GQA attention of independent rows (decode, and prefill on f32 caches):
// row r attends slab rows [0, pos_r] of its head group; partials then combine.
// With `fuse`, q holds the raw Q|K|V projection rows (one row per slab):
// the kernel norms and rotates the queries itself and writes the new key and
// value at each row's position (Q/K norm + RoPE + KV write fused); without
// it q holds normed, rotated query rows and the cache holds every key.
// span_bound: an upper bound on the cache rows one split of a row covers.
// merge_ctr: [R][n_kv] zeroed counts; with it, 2..kMergeMaxSplits splits and an
// output, the last split of each (row, KV head) merges the splits in the same
// launch (and zeroes its count) instead of a combine pass.
hipError_t launch_attn_rows(const float* q, int64_t ldq, int R, int n_heads, RowMap rm, KVLayer kv, int n_splits,
                            int span_bound, float* part, float* out_f32, uint16_t* out_bf16, uint16_t* out_bf16_lo,
                            int64_t ldo, uint32_t* err, const QkRope* fuse, WType gt, hipStream_t s,
                            uint32_t* merge_ctr = nullptr);
// One decode row: the fused-RMSNorm Q|K|V projection and the split attention in
// one launch (kernels_attn.hip, qkv_attn_kernel), handing the projection over
// through 64-bit tagged words in qtag. The splits' partial records go to `part`
// for the O-projection GEMV to merge. tag_gen: a device word, never 0, that the
// launch advances; tag_done: a device word, zero between launches.
struct QkvTagArgs {
    const uint16_t* wq;
    const uint16_t* wk;
    const uint16_t* wv;
    const uint16_t* gain;  // attention RMSNorm gain (bf16)
    const float* x;        // the row, [K] fp32
    int K, nq, nkv, d;
    float eps;
    uint64_t* qtag;  // [(nq + 2 nkv) d] tagged projection words
};
bool qkv_attn_fits(int n_heads, int n_kv, int d, int K, int n_splits, int span_bound, KVType kv);
hipError_t launch_qkv_attn(const QkvTagArgs& p, RowMap rm, KVLayer kv, int n_splits, int span_bound, float* part,
                           uint32_t* err, const QkRope& fuse, uint32_t* tag_gen, uint32_t* tag_done, hipStream_t s);
// Causal flash attention (MFMA, f16 cache) of T rows of one slab at positions pos0..
hipError_t launch_attn_prefill(const uint16_t* q16, int64_t ldq, int T, int pos0, int seq, int n_heads, KVLayer kv,
                               uint16_t* out_bf16, uint16_t* out_bf16_lo, int64_t ldo, hipStream_t s);
// The same for packed sequences, all in one launch: sequence i's rows start at row
// sg.start[i] of q16 and of the output, sg.len[i] of them, at positions sg.pos0[i]..
// of slab sg.seq[i].
hipError_t launch_attn_prefill_packed(const uint16_t* q16, int64_t ldq, const Segments& sg, int n_heads, KVLayer kv,
                                      uint16_t* out_bf16, uint16_t* out_bf16_lo, int64_t ldo, hipStream_t s);

constexpr uint32_t kDevErrSync = 8u;  // a tagged hand-off poll timed out (STTD_DEVERR_SYNC)

}  // namespace sttd
