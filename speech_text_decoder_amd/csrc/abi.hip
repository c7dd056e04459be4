// abi.hip - the C ABI of include/sttd.h: validation, allocation, and the
// kernel sequences of one block call.
#include <math.h>

#include <algorithm>
#include <string.h>

#include <mutex>
#include <new>
#include <utility>
#include <vector>

#include "launch.h"
#include "sttd.h"

using namespace sttd;


struct sttd_kv_cache {
    int n_layers, n_seq, n_ctx, n_kv, d;
    sttd_dtype type;
    size_t elem;
    void* k;
    void* v;
};

struct sttd_workspace {
    sttd_block_params p;
    int max_rows, max_pos, vocab;
    int part_cap;  // (row, split) slots of the attention partials
    void* base;
    size_t bytes;
    float* rope;        // [max_pos][d/2][2]
    uint16_t* xn;       // [2][max_rows][hidden] bf16: normed rows for the MFMA GEMMs, then their low parts
    float* qkv;         // [max_rows][(nq + 2 nkv) d]
    void* qbuf;         // [max_rows][nq d] fp32 (or f16)
    float* attn_o;      // [max_rows][nq d] fp32, or two bf16 planes (high, low)
    float* act;         // [max_rows][ffn] fp32, or two bf16 planes (high, low)
    float* part;        // [part_cap][nq][d + 4] attention split partials
    unsigned long long* partials;  // [max_rows][kHeadPartials] head argmax partials
    uint32_t* err;                 // [1]
    int32_t* iota;                 // [max_rows]: 0, 1, ... (slab b of row b when no slab ids are given)
    int32_t* rowpos;               // [max_rows]: per-row positions of a packed batched prefill
    int32_t* rowseq;               // [max_rows]: per-row slabs of a packed batched prefill
    uint32_t* merge_ctr;           // [max_rows][n_kv] attention split counts (zero between launches)
    uint64_t* qtag;                // [(nq + 2 nkv) d] tagged projection words of a single decode row
    uint32_t* tag_gen;             // [1] the next hand-off tag (never 0)
    uint32_t* tag_done;            // [1] hand-off consumers counted out (zero between launches)
    bool qkv_attn;                 // STTD_OPT_QKV_ATTN
    uint32_t split_mask;           // STTD_OPT_ACT_SPLIT: GEMM inputs kept as bf16 high + low parts at any row count
};

namespace {

// ------------------------------------------------------------ per-kernel timing
struct Profiler {
    std::mutex mu;
    uint32_t mask = 0;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> timed[STTD_KERN_COUNT];  // one pair per kernel launch
    int64_t calls[STTD_KERN_COUNT] = {};                                    // timed calls of each family
    std::vector<hipEvent_t> pool;

    hipEvent_t get() {
        if (!pool.empty()) {
            hipEvent_t e = pool.back();
            pool.pop_back();
            return e;
        }
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        return e;
    }
};
Profiler g_prof;
// Event pairs of the launches of the call being issued on this thread (nullptr: not timed).
thread_local std::vector<std::pair<hipEvent_t, hipEvent_t>>* t_pairs = nullptr;

// Device-clock timing: one slot of kClockEntries (start, end) pairs per timed launch.
struct ClockProf {
    std::mutex mu;
    uint32_t mask = 0;
    uint64_t* slots = nullptr;  // device [cap][kClockEntries][2]
    uint64_t* red = nullptr;    // device [cap][2]: reduced spans
    int cap = 0, used = 0;
    std::vector<int> kinds;     // kernel family of each used slot
    uint64_t* current = nullptr;
};
ClockProf g_clk;

constexpr size_t kClockSlotBytes = (size_t)kClockEntries * 2 * sizeof(uint64_t);

hipError_t clock_fill(int n) {
    return n ? hipMemset(g_clk.slots, 0, kClockSlotBytes * (size_t)n) : hipSuccess;
}

// Reduced (start, end) of the used slots into h (host, 2 * used).
hipError_t clock_collect(std::vector<uint64_t>& h) {
    h.assign(2 * (size_t)g_clk.used, 0);
    if (!g_clk.used) return hipSuccess;
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess) e = launch_clock_reduce(g_clk.slots, g_clk.used, g_clk.red, nullptr);
    if (e == hipSuccess) e = hipMemcpy(h.data(), g_clk.red, h.size() * sizeof(uint64_t), hipMemcpyDeviceToHost);
    return e;
}

// Times the launches of one kernel family: an event pair bound to each kernel's
// dispatch (eager launches) and/or a device-clock slot (eager or captured
// launches), as enabled.
class ProfScope {
  public:
    ProfScope(int kind, hipStream_t s) : kind_(kind) {
        if (g_clk.mask & (1u << kind)) {
            std::lock_guard<std::mutex> lk(g_clk.mu);
            if (g_clk.used < g_clk.cap) {
                g_clk.current = g_clk.slots + (size_t)kClockEntries * 2 * (size_t)g_clk.used++;
                g_clk.kinds.push_back(kind);
            }
        }
        if (!(g_prof.mask & (1u << kind))) return;
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
        timed_ = true;
        t_pairs = &pairs_;
    }
    ~ProfScope() {
        g_clk.current = nullptr;
        if (!timed_) return;
        t_pairs = nullptr;
        std::lock_guard<std::mutex> lk(g_prof.mu);
        for (auto& pr : pairs_) g_prof.timed[kind_].push_back(pr);
        g_prof.calls[kind_] += 1;
    }

  private:
    int kind_;
    bool timed_ = false;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> pairs_;
};

constexpr int kGemvMaxRows = 4;    // rows beyond this take the MFMA GEMMs (bf16 weights)
constexpr int kSplitMaxRows = 512; // up to here the GEMMs are HBM-bound: split activations (hi + lo)
constexpr int kMaxSplits = 64;
constexpr int kHeadPartials = 1024;  // workgroups of the persistent head GEMV

sttd_status from_hip(hipError_t e) {
    if (e == hipSuccess) return STTD_OK;
    if (e == hipErrorOutOfMemory) return STTD_ERR_OOM;
    return STTD_ERR_BACKEND;
}

#define TRY(expr)                                  \
    do {                                           \
        hipError_t e_ = (expr);                    \
        if (e_ != hipSuccess) return from_hip(e_); \
    } while (0)

bool params_ok(const sttd_block_params* p) {
    if (!p) return false;
    if (p->hidden <= 0 || p->n_heads <= 0 || p->n_kv_heads <= 0 || p->ffn <= 0) return false;
    if (p->n_heads % p->n_kv_heads) return false;
    if (!(p->rms_eps >= 0.f) || !(p->rope_theta > 0.f)) return false;
    return true;
}

sttd_status params_supported(const sttd_block_params* p) {
    if (p->head_dim != 64 && p->head_dim != 128) return STTD_ERR_UNSUPPORTED;
    if (p->hidden % 64 || p->ffn % 64) return STTD_ERR_UNSUPPORTED;
    // the decode GEMVs keep a whole input row in registers: K <= 8192
    if (p->hidden > 8192 || p->ffn > 8192 || p->n_heads * p->head_dim > 8192) return STTD_ERR_UNSUPPORTED;
    const int g = p->n_heads / p->n_kv_heads;
    if (g != 1 && g != 2 && g != 4 && g != 8) return STTD_ERR_UNSUPPORTED;
    if (p->wtype != STTD_BF16 && p->wtype != STTD_F32) return STTD_ERR_UNSUPPORTED;
    return STTD_OK;
}

bool same_shape(const sttd_block_params* a, const sttd_block_params* b) {
    return a->hidden == b->hidden && a->n_heads == b->n_heads && a->n_kv_heads == b->n_kv_heads &&
           a->head_dim == b->head_dim && a->ffn == b->ffn && a->wtype == b->wtype;
}

bool weights_ok(const sttd_block_weights* w) {
    return w && w->attn_norm && w->wq && w->wk && w->wv && w->q_norm && w->k_norm && w->wo && w->ffn_norm &&
           w->w_gate_up && w->w_down;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

KVLayer kv_layer(const sttd_kv_cache* kv, int layer) {
    KVLayer l;
    const size_t per_layer = (size_t)kv->n_seq * kv->n_kv * kv->n_ctx * kv->d * kv->elem;
    l.k = (char*)kv->k + per_layer * layer;
    l.v = (char*)kv->v + per_layer * layer;
    l.n_seq = kv->n_seq;
    l.n_kv = kv->n_kv;
    l.n_ctx = kv->n_ctx;
    l.d = kv->d;
    l.type = kv->type == STTD_F16 ? KV_F16 : KV_F32;
    return l;
}

// Splits of each row's cache span over workgroups: about 128 positions each,
// but for batches of rows no more than about one 8-wave workgroup per CU
// (256), so each workgroup streams a longer run of rows (measured on 16 rows of
// 150-1500 positions: 256 workgroups of 8 waves beat 512 of 4 and any larger grid;
// 256 workgroups dealt to the rows by length (22.8 us per block) and one split per
// row (27.8 us) both lost to two equal splits per row (21.0 us): the split merge
// costs a write-through, an atomic and a reload, not the streaming). Splits per
// row that follow each row's own length (ceil(keys / span), up to 8, the spare
// workgroups exiting at once) lost too: 17.9 us per block against 22.9, 25.5 and
// 28.0 us at spans of 384, 512 and 256 rows. Re-measured with the register-ring
// rows loop (one layer's launch, 16 rows of 151-1535 positions): ceil(keys / 600) up
// to 3 splits 18.1 us and ceil(keys / 400) up to 4 16.7 us, against 14.3 us for two
// equal splits; a lone 1535-position row 14.9 / 13.1 against 11.5 us, whatever the
// slab stride of the cache (2048 to 2176 rows).
// Packed sequences' flash attention in one launch (8 prompts of 153 rows, 28 blocks:
// 15.2 -> 11.3 ms, 224 launches of 18 us -> 28 of 19.6 us); 0 launches per sequence
#ifndef STTD_PACKED_FLASH_ONE_LAUNCH
#define STTD_PACKED_FLASH_ONE_LAUNCH 1
#endif
#ifndef STTD_ATTN_FILL
#define STTD_ATTN_FILL 256
#endif
int choose_splits(int rows, int n_kv, int pos_bound, int part_cap) {
    int s = (pos_bound + 127) / 128;
    // long single rows: fewer, longer splits (8-wave workgroups) and one combine
    // (at 4096-4352 positions, capping a single row at 16 splits measured within
    // 1% of 32, and at 8, which the O projection then merges, 5% slower)
    if (s > 32) s = 32;
    const int fill = (STTD_ATTN_FILL + rows * n_kv - 1) / (rows * n_kv);
    if (rows > 1 && s > fill) s = fill;
    if (s > kMaxSplits) s = kMaxSplits;
    if (s > part_cap / rows) s = part_cap / rows;
    return s < 1 ? 1 : s;
}

// One block over R rows. prefill: a causal prefill, of one slab at positions
// rm.pos0.. or, with segs, of several sequences packed back to back (rm then
// holds the expanded per-row positions and slabs); otherwise decode rows.
sttd_status run_block(const sttd_block_params* p, const sttd_block_weights* w, sttd_workspace* ws,
                      const sttd_kv_cache* kv, int layer, int R, RowMap rm, int pos_bound, bool prefill,
                      bool last_row_only, float* x, hipStream_t s, const Segments* segs = nullptr) {
    const WType wt = p->wtype == STTD_BF16 ? W_BF16 : W_F32;
    const int H = p->hidden, nq = p->n_heads, nkv = p->n_kv_heads, d = p->head_dim, I = p->ffn;
    const int qd = nq * d, kvd = nkv * d, qkv_cols = qd + 2 * kvd;
    const float eps = p->rms_eps;
    const KVLayer kl = kv_layer(kv, layer);
    const bool mfma = wt == W_BF16 && R > kGemvMaxRows;
    bool flash = mfma && prefill && kl.type == KV_F16;
    if (flash && segs)  // every packed sequence must be long enough for the flash tiles' query layout
        for (int i = 0; i < segs->n; ++i) flash = flash && segs->len[i] > kGemvMaxRows;
    // which GEMM inputs are split into bf16 high + low parts: all of them up to
    // kSplitMaxRows rows (HBM-bound there, so the doubled MFMA work is free), and
    // beyond that the ones the workspace's STTD_OPT_ACT_SPLIT mask names (all four
    // by default: on the 28-block stack plain bf16 ones drift the logits past the
    // parity bound)
    const bool split_all = R <= kSplitMaxRows;
    const uint32_t sm = ws->split_mask;
    uint16_t* xn_lo_base = ws->xn + (size_t)ws->max_rows * H;
    uint16_t* xn_lo = split_all || (sm & STTD_SPLIT_QKV) ? xn_lo_base : nullptr;
    uint16_t* ffn_lo = split_all || (sm & STTD_SPLIT_GATE_UP) ? xn_lo_base : nullptr;
    uint16_t* ao = (uint16_t*)ws->attn_o;
    uint16_t* ao_lo = split_all || (sm & STTD_SPLIT_O) ? ao + (size_t)ws->max_rows * qd : nullptr;
    uint16_t* act = (uint16_t*)ws->act;
    uint16_t* act_lo = split_all || (sm & STTD_SPLIT_DOWN) ? act + (size_t)ws->max_rows * I : nullptr;

    // --- a single decode row: the Q|K|V projection and the attention in one launch
    // (tagged hand-off), when the shape allows and the attention splits merge in the
    // O projection
    int qa_splits = 0;
    bool qkv_attn = false;
    if (!prefill && R == 1 && !mfma && wt == W_BF16 && ws->qkv_attn) {
        qa_splits = choose_splits(R, nkv, pos_bound, ws->part_cap);
        const int span = (pos_bound + qa_splits - 1) / qa_splits;
        qkv_attn = qa_splits > 1 && qkv_attn_fits(nq, nkv, d, H, qa_splits, span, kl.type);
    }
    // --- attention half: norm + QKV projection
    bool qk_fused = false;  // the Q|K|V GEMM's epilogue does the Q/K norm, RoPE and cache write
    QkRope qr{};
    qr.q_gain = w->q_norm; qr.k_gain = w->k_norm; qr.eps = eps; qr.rope = ws->rope; qr.max_pos = ws->max_pos;
    qr.rm = rm; qr.kv = kl; qr.q_out = ws->qbuf; qr.q_f16 = flash; qr.ldq = qd; qr.err = ws->err;
    qr.n_heads = nq; qr.n_kv = nkv; qr.d = d;
    if (mfma) {
        GemmArgs g{};
        if (gemm_fuses_norm(R, H)) {  // few rows: the projection norms them itself
            g.X = x; g.ldx = H; g.gain = (const uint16_t*)w->attn_norm; g.eps = eps; g.x_lo = xn_lo != nullptr;
        } else {
            ProfScope ps(STTD_KERN_RMSNORM, s);
            TRY(launch_rmsnorm_rows_bf16(x, H, w->attn_norm, wt, ws->xn, xn_lo, H, R, H, eps, s));
        }
        g.A = ws->xn; g.A_lo = xn_lo; g.lda = H; g.M = R; g.K = H;
        g.w[0] = (const uint16_t*)w->wq; g.w[1] = (const uint16_t*)w->wk; g.w[2] = (const uint16_t*)w->wv;
        g.seg_end[0] = qd; g.seg_end[1] = qd + kvd; g.seg_end[2] = qkv_cols;
        g.N = qkv_cols; g.C = ws->qkv; g.ldc = qkv_cols;
        // long prefills: per-head norm, RoPE and the cache write in the projection's epilogue
        qk_fused = flash && gemm_qkrope_fits(R, qkv_cols, H, d) && (!xn_lo || gemm_split_large_tiles());
        if (qk_fused) g.qk = qr;
        ProfScope ps(STTD_KERN_QKV_GEMM, s);
        TRY(launch_gemm(g, qk_fused ? GEMM_QKROPE : GEMM_STORE, s));
    } else if (!qkv_attn) {
        GemvArgs a{};
        a.w[0] = w->wq; a.w[1] = w->wk; a.w[2] = w->wv;
        a.seg_end[0] = qd; a.seg_end[1] = qd + kvd; a.seg_end[2] = qkv_cols;
        a.N = qkv_cols; a.K = H; a.x = x; a.ldx = H; a.rows = R; a.gain = w->attn_norm; a.eps = eps;
        a.y = ws->qkv; a.ldy = qkv_cols;
        ProfScope ps(STTD_KERN_QKV_GEMV, s);
        TRY(launch_gemv(a, wt, GEMV_STORE, s));
    }
    // --- per-head Q/K norm + RoPE + cache write, then attention. Prefill rows of
    // one sequence need every key written first (separate kernel); decode rows
    // (one per slab) do it inside the attention kernel.
    if (prefill && !qk_fused) {
        ProfScope ps(STTD_KERN_QK_ROPE_KV, s);
        TRY(launch_qk_norm_rope_kv(ws->qkv, qkv_cols, R, wt, qr, s));
    }
    int splits = 1;
    bool defer = false;
    if (segs && flash && STTD_PACKED_FLASH_ONE_LAUNCH) {
        // packed sequences, each attending its own slab causally from its pos0: every
        // sequence's query tiles in one launch (one launch per sequence gave each of
        // them 2 x n_heads workgroups at 153 rows, a few dozen CUs of 256)
        ProfScope ps(STTD_KERN_ATTN_PREFILL, s);
        TRY(launch_attn_prefill_packed((const uint16_t*)ws->qbuf, qd, *segs, nq, kl, mfma ? ao : nullptr,
                                       mfma ? ao_lo : nullptr, qd, s));
    } else if (segs) {
        // packed sequences: each attends its own slab, causally from its pos0
        for (int i = 0; i < segs->n; ++i) {
            const int r0 = segs->start[i], Ti = segs->len[i], p0 = segs->pos0[i];
            uint16_t* aoi = mfma ? ao + (size_t)r0 * qd : nullptr;
            uint16_t* aoli = mfma && ao_lo ? ao_lo + (size_t)r0 * qd : nullptr;
            if (flash) {
                ProfScope ps(STTD_KERN_ATTN_PREFILL, s);
                TRY(launch_attn_prefill((const uint16_t*)ws->qbuf + (size_t)r0 * qd, qd, Ti, p0, segs->seq[i], nq,
                                        kl, aoi, aoli, qd, s));
            } else {
                const RowMap ri{rm.pos + r0, rm.seq + r0, 0, 0};
                const int sp = choose_splits(Ti, nkv, p0 + Ti, ws->part_cap);
                ProfScope ps(STTD_KERN_ATTN_ROWS, s);
                TRY(launch_attn_rows((const float*)ws->qbuf + (size_t)r0 * qd, qd, Ti, nq, ri, kl, sp,
                                     (p0 + Ti + sp - 1) / sp, ws->part, mfma ? nullptr : ws->attn_o + (size_t)r0 * qd,
                                     aoi, aoli, qd, ws->err, nullptr, wt, s, ws->merge_ctr + (size_t)r0 * nkv));
            }
        }
    } else if (flash) {
        ProfScope ps(STTD_KERN_ATTN_PREFILL, s);
        TRY(launch_attn_prefill((const uint16_t*)ws->qbuf, qd, R, rm.pos0, rm.seq0, nq, kl, ao, ao_lo, qd, s));
    } else if (qkv_attn) {
        splits = qa_splits;
        defer = true;
        QkvTagArgs p{};
        p.wq = (const uint16_t*)w->wq; p.wk = (const uint16_t*)w->wk; p.wv = (const uint16_t*)w->wv;
        p.gain = (const uint16_t*)w->attn_norm; p.x = x; p.K = H; p.nq = nq; p.nkv = nkv; p.d = d; p.eps = eps;
        p.qtag = ws->qtag;
        ProfScope ps(STTD_KERN_QKV_ATTN, s);
        TRY(launch_qkv_attn(p, rm, kl, splits, (pos_bound + splits - 1) / splits, ws->part, ws->err, qr, ws->tag_gen,
                            ws->tag_done, s));
    } else {
        splits = choose_splits(R, nkv, pos_bound, ws->part_cap);
        // GEMV path: a split result stays as partials and the O projection merges them on load
        // GEMV path with a few splits: the O projection merges the partials as it loads
        // them (every one of its workgroups re-reads them all); with many, one combine
        // pass is cheaper
        defer = !mfma && splits > 1 && splits <= kMergeMaxSplits;
        ProfScope ps(STTD_KERN_ATTN_ROWS, s);
        const int span = ((prefill ? rm.pos0 + R : pos_bound) + splits - 1) / splits;
        TRY(launch_attn_rows(prefill ? (const float*)ws->qbuf : ws->qkv, prefill ? qd : qkv_cols, R, nq, rm, kl,
                             splits, span, ws->part, mfma || defer ? nullptr : ws->attn_o, mfma ? ao : nullptr,
                             mfma ? ao_lo : nullptr, qd, ws->err, prefill ? nullptr : &qr, wt, s, ws->merge_ctr));
    }
    // --- O projection + residual
    if (mfma) {
        GemmArgs g{};
        g.A = ao; g.A_lo = ao_lo; g.lda = qd; g.M = R; g.K = qd;
        g.w[0] = (const uint16_t*)w->wo; g.seg_end[0] = g.seg_end[1] = g.seg_end[2] = H;
        g.N = H; g.C = x; g.ldc = H;
        ProfScope ps(STTD_KERN_O_GEMM, s);
        TRY(launch_gemm(g, GEMM_RESID, s));
    } else {
        GemvArgs a{};
        a.w[0] = w->wo; a.seg_end[0] = a.seg_end[1] = a.seg_end[2] = H;
        a.N = H; a.K = qd; a.x = ws->attn_o; a.ldx = qd; a.rows = R; a.y = x; a.ldy = H; a.resid = x; a.ldr = H;
        if (defer) {
            a.xpart = ws->part; a.n_splits = splits; a.head_dim = d;
        }
        ProfScope ps(STTD_KERN_O_GEMV, s);
        TRY(launch_gemv(a, wt, GEMV_RESID, s));
    }
    // --- FFN: norm, packed gate_up + SwiGLU, down + residual
    const int r0 = last_row_only ? R - 1 : 0;
    const int nr = last_row_only ? 1 : R;
    float* xf = x + (int64_t)r0 * H;
    if (mfma && nr > kGemvMaxRows) {
        GemmArgs g{};
        if (gemm_fuses_norm(nr, H)) {
            g.X = xf; g.ldx = H; g.gain = (const uint16_t*)w->ffn_norm; g.eps = eps; g.x_lo = ffn_lo != nullptr;
        } else {
            ProfScope ps(STTD_KERN_RMSNORM, s);
            TRY(launch_rmsnorm_rows_bf16(xf, H, w->ffn_norm, wt, ws->xn, ffn_lo, H, nr, H, eps, s));
        }
        g.A = ws->xn; g.A_lo = ffn_lo; g.lda = H; g.M = nr; g.K = H;
        g.w[0] = (const uint16_t*)w->w_gate_up; g.seg_end[0] = g.seg_end[1] = g.seg_end[2] = 2 * I;
        g.N = I; g.Cb = act; g.Cb_lo = act_lo; g.ldcb = I;
        {
            ProfScope ps(STTD_KERN_GATEUP_GEMM, s);
            TRY(launch_gemm(g, GEMM_SWIGLU, s));
        }
        GemmArgs g2{};
        g2.A = act; g2.A_lo = act_lo; g2.lda = I; g2.M = nr; g2.K = I;
        g2.w[0] = (const uint16_t*)w->w_down; g2.seg_end[0] = g2.seg_end[1] = g2.seg_end[2] = H;
        g2.N = H; g2.C = xf; g2.ldc = H;
        ProfScope ps(STTD_KERN_DOWN_GEMM, s);
        TRY(launch_gemm(g2, GEMM_RESID, s));
    } else {
        GemvArgs a{};
        a.w[0] = w->w_gate_up; a.seg_end[0] = a.seg_end[1] = a.seg_end[2] = I;
        a.N = I; a.K = H; a.x = xf; a.ldx = H; a.rows = nr; a.gain = w->ffn_norm; a.eps = eps;
        a.y = ws->act; a.ldy = I;
        {
            ProfScope ps(STTD_KERN_GATEUP_GEMV, s);
            TRY(launch_gemv(a, wt, GEMV_SWIGLU, s));
        }
        GemvArgs b{};
        b.w[0] = w->w_down; b.seg_end[0] = b.seg_end[1] = b.seg_end[2] = H;
        b.N = H; b.K = I; b.x = ws->act; b.ldx = I; b.rows = nr; b.y = xf; b.ldy = H; b.resid = xf; b.ldr = H;
        ProfScope ps(STTD_KERN_DOWN_GEMV, s);
        TRY(launch_gemv(b, wt, GEMV_RESID, s));
    }
    return STTD_OK;
}

}  // namespace

uint64_t* sttd::clock_slot() { return g_clk.current; }

bool sttd::next_launch_events(hipEvent_t* start, hipEvent_t* stop) {
    if (!t_pairs) return false;
    std::lock_guard<std::mutex> lk(g_prof.mu);
    hipEvent_t b = g_prof.get(), e = g_prof.get();
    if (!b || !e) return false;
    t_pairs->emplace_back(b, e);
    *start = b;
    *stop = e;
    return true;
}

extern "C" {

const char* sttd_status_string(sttd_status s) {
    switch (s) {
        case STTD_OK: return "ok";
        case STTD_ERR_INVALID_ARG: return "invalid argument";
        case STTD_ERR_OOM: return "out of device memory";
        case STTD_ERR_BACKEND: return "HIP call or kernel launch failed";
        case STTD_ERR_CONTEXT_FULL: return "positions pass the KV cache's n_ctx";
        case STTD_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    }
    return "unknown status";
}

sttd_status sttd_kv_cache_alloc(int n_layers, int n_seq, int n_ctx, int n_kv_heads, int head_dim, sttd_dtype kv_type,
                                sttd_kv_cache** out) {
    if (!out) return STTD_ERR_INVALID_ARG;
    *out = nullptr;
    if (n_layers <= 0 || n_seq <= 0 || n_ctx <= 0 || n_kv_heads <= 0 || head_dim <= 0) return STTD_ERR_INVALID_ARG;
    if (kv_type != STTD_F16 && kv_type != STTD_F32) return STTD_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return STTD_ERR_UNSUPPORTED;
    const size_t elem = kv_type == STTD_F16 ? 2 : 4;
    const double total = (double)n_layers * n_seq * n_ctx * n_kv_heads * head_dim * elem;
    if (total > 1e15) return STTD_ERR_OOM;
    const size_t bytes = (size_t)n_layers * n_seq * n_ctx * n_kv_heads * head_dim * elem;
    sttd_kv_cache* kv = new (std::nothrow) sttd_kv_cache();
    if (!kv) return STTD_ERR_OOM;
    kv->n_layers = n_layers; kv->n_seq = n_seq; kv->n_ctx = n_ctx; kv->n_kv = n_kv_heads; kv->d = head_dim;
    kv->type = kv_type; kv->elem = elem;
    if (hipMalloc(&kv->k, bytes) != hipSuccess) {
        (void)hipGetLastError();
        delete kv;
        return STTD_ERR_OOM;
    }
    if (hipMalloc(&kv->v, bytes) != hipSuccess) {
        (void)hipGetLastError();
        (void)hipFree(kv->k);
        delete kv;
        return STTD_ERR_OOM;
    }
    if (hipMemset(kv->k, 0, bytes) != hipSuccess || hipMemset(kv->v, 0, bytes) != hipSuccess) {
        (void)hipFree(kv->k);
        (void)hipFree(kv->v);
        delete kv;
        return STTD_ERR_BACKEND;
    }
    *out = kv;
    return STTD_OK;
}

int sttd_kv_context_for(int needed, int ceiling) {
    if (needed < 1 || ceiling < 1) return 0;
    int n;
    if (needed <= 1024) n = 1024;
    else if (needed <= 2048) n = 2048;
    else n = (int)(((int64_t)needed + 4095) / 4096 * 4096 > INT32_MAX ? INT32_MAX : ((int64_t)needed + 4095) / 4096 * 4096);
    return n < ceiling ? n : ceiling;
}

sttd_status sttd_kv_cache_free(sttd_kv_cache* kv) {
    if (!kv) return STTD_ERR_INVALID_ARG;
    const hipError_t a = hipFree(kv->k), b = hipFree(kv->v);
    delete kv;
    return (a == hipSuccess && b == hipSuccess) ? STTD_OK : STTD_ERR_BACKEND;
}

sttd_status sttd_kv_cache_clear(sttd_kv_cache* kv, void* stream) {
    if (!kv) return STTD_ERR_INVALID_ARG;
    const size_t bytes = (size_t)kv->n_layers * kv->n_seq * kv->n_ctx * kv->n_kv * kv->d * kv->elem;
    TRY(launch_fill_zero(kv->k, bytes, (hipStream_t)stream));
    TRY(launch_fill_zero(kv->v, bytes, (hipStream_t)stream));
    return STTD_OK;
}

sttd_status sttd_kv_cache_view(const sttd_kv_cache* kv, int layer, int seq, void** k, void** v, int64_t* head_stride,
                               int64_t* pos_stride) {
    if (!kv || !k || !v || !head_stride || !pos_stride) return STTD_ERR_INVALID_ARG;
    if (layer < 0 || layer >= kv->n_layers || seq < 0 || seq >= kv->n_seq) return STTD_ERR_INVALID_ARG;
    const KVLayer l = kv_layer(kv, layer);
    const size_t off = (size_t)seq * kv->n_kv * kv->n_ctx * kv->d * kv->elem;
    *k = (char*)l.k + off;
    *v = (char*)l.v + off;
    *head_stride = (int64_t)kv->n_ctx * kv->d;
    *pos_stride = kv->d;
    return STTD_OK;
}

sttd_status sttd_workspace_alloc(const sttd_block_params* p, int max_rows, int max_pos, int vocab,
                                 sttd_workspace** out) {
    if (!out) return STTD_ERR_INVALID_ARG;
    *out = nullptr;
    if (!params_ok(p) || max_rows <= 0 || max_pos <= 0 || vocab < 0) return STTD_ERR_INVALID_ARG;
    const sttd_status sup = params_supported(p);
    if (sup != STTD_OK) return sup;
    const int H = p->hidden, nq = p->n_heads, nkv = p->n_kv_heads, d = p->head_dim, I = p->ffn;
    const size_t R = (size_t)max_rows;
    const int part_cap = max_rows > 64 * kMaxSplits ? max_rows : 64 * kMaxSplits;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return o;
    };
    const size_t o_rope = take((size_t)max_pos * d * sizeof(float));
    const size_t o_xn = take(R * H * 2 * 2);
    const size_t o_qkv = take(R * (nq + 2 * nkv) * d * sizeof(float));
    const size_t o_q = take(R * nq * d * sizeof(float));
    const size_t o_ao = take(R * nq * d * sizeof(float));
    const size_t o_act = take(R * I * sizeof(float));
    const size_t o_part = take((size_t)part_cap * nq * (d + 4) * sizeof(float));
    const size_t o_partials = take(R * kHeadPartials * sizeof(unsigned long long));
    const size_t o_err = take(sizeof(uint32_t));
    const size_t o_iota = take(R * sizeof(int32_t));
    const size_t o_rowpos = take(R * sizeof(int32_t));
    const size_t o_rowseq = take(R * sizeof(int32_t));
    const size_t o_merge = take(R * nkv * sizeof(uint32_t));
    const size_t o_qtag = take((size_t)(nq + 2 * nkv) * d * sizeof(uint64_t));
    const size_t o_tag = take(2 * sizeof(uint32_t));
    sttd_workspace* ws = new (std::nothrow) sttd_workspace();
    if (!ws) return STTD_ERR_OOM;
    ws->p = *p;
    ws->max_rows = max_rows;
    ws->max_pos = max_pos;
    ws->vocab = vocab;
    ws->part_cap = part_cap;
    ws->bytes = off;
    if (hipMalloc(&ws->base, off) != hipSuccess) {
        (void)hipGetLastError();
        delete ws;
        return STTD_ERR_OOM;
    }
    char* b = (char*)ws->base;
    ws->rope = (float*)(b + o_rope);
    ws->xn = (uint16_t*)(b + o_xn);
    ws->qkv = (float*)(b + o_qkv);
    ws->qbuf = b + o_q;
    ws->attn_o = (float*)(b + o_ao);
    ws->act = (float*)(b + o_act);
    ws->part = (float*)(b + o_part);
    ws->partials = (unsigned long long*)(b + o_partials);
    ws->err = (uint32_t*)(b + o_err);
    ws->iota = (int32_t*)(b + o_iota);
    ws->rowpos = (int32_t*)(b + o_rowpos);
    ws->rowseq = (int32_t*)(b + o_rowseq);
    ws->merge_ctr = (uint32_t*)(b + o_merge);
    ws->qtag = (uint64_t*)(b + o_qtag);
    ws->tag_gen = (uint32_t*)(b + o_tag);
    ws->tag_done = ws->tag_gen + 1;
    ws->qkv_attn = true;
    ws->split_mask = STTD_SPLIT_QKV | STTD_SPLIT_O | STTD_SPLIT_GATE_UP | STTD_SPLIT_DOWN;
    // RoPE table in fp64 on the host: pair i of position pos turns by pos * theta^(-2i/d)
    std::vector<float> table((size_t)max_pos * d);
    const int half = d / 2;
    for (int i = 0; i < half; ++i) {
        const double omega = pow((double)p->rope_theta, -2.0 * i / d);
        for (int pos = 0; pos < max_pos; ++pos) {
            const double a = pos * omega;
            table[((size_t)pos * half + i) * 2] = (float)cos(a);
            table[((size_t)pos * half + i) * 2 + 1] = (float)sin(a);
        }
    }
    std::vector<int32_t> iota(R);
    for (size_t i = 0; i < R; ++i) iota[i] = (int32_t)i;
    const uint32_t first_tag = 1;  // the zeroed words carry tag 0, which no launch uses
    if (hipMemset(ws->base, 0, off) != hipSuccess ||
        hipMemcpy(ws->tag_gen, &first_tag, sizeof(uint32_t), hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(ws->rope, table.data(), table.size() * sizeof(float), hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(ws->iota, iota.data(), R * sizeof(int32_t), hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(ws->base);
        delete ws;
        return STTD_ERR_BACKEND;
    }
    *out = ws;
    return STTD_OK;
}

sttd_status sttd_workspace_free(sttd_workspace* ws) {
    if (!ws) return STTD_ERR_INVALID_ARG;
    const hipError_t e = hipFree(ws->base);
    delete ws;
    return e == hipSuccess ? STTD_OK : STTD_ERR_BACKEND;
}

sttd_status sttd_workspace_set_option(sttd_workspace* ws, int option, int value) {
    if (!ws) return STTD_ERR_INVALID_ARG;
    if (option == STTD_OPT_QKV_ATTN && (value == 0 || value == 1)) {
        ws->qkv_attn = value == 1;
        return STTD_OK;
    }
    if (option == STTD_OPT_ACT_SPLIT && value >= 0 && value <= 15) {
        ws->split_mask = (uint32_t)value;
        return STTD_OK;
    }
    return STTD_ERR_INVALID_ARG;
}

sttd_status sttd_workspace_error(sttd_workspace* ws, uint32_t* bits) {
    if (!ws || !bits) return STTD_ERR_INVALID_ARG;
    TRY(hipDeviceSynchronize());
    TRY(hipMemcpy(bits, ws->err, sizeof(uint32_t), hipMemcpyDeviceToHost));
    TRY(hipMemset(ws->err, 0, sizeof(uint32_t)));
    return STTD_OK;
}

sttd_status sttd_embed_gather(const void* embed, sttd_dtype wtype, int vocab, int hidden, int B, const int32_t* ids,
                              float* x, sttd_workspace* ws, void* stream) {
    if (!embed || !ids || !x || vocab <= 0 || hidden <= 0 || B <= 0) return STTD_ERR_INVALID_ARG;
    if (wtype != STTD_BF16 && wtype != STTD_F32) return STTD_ERR_UNSUPPORTED;
    TRY(launch_embed_gather(embed, wtype == STTD_BF16 ? W_BF16 : W_F32, vocab, hidden, B, ids, nullptr, nullptr, x,
                            ws ? ws->err : nullptr, (hipStream_t)stream));
    return STTD_OK;
}

sttd_status sttd_embed_inject(const void* embed, sttd_dtype wtype, int vocab, int hidden, int T, const int32_t* ids,
                              const float* keep, const float* audio_dense, float* x, sttd_workspace* ws,
                              void* stream) {
    if (!embed || !ids || !keep || !audio_dense || !x || vocab <= 0 || hidden <= 0 || T <= 0)
        return STTD_ERR_INVALID_ARG;
    if (wtype != STTD_BF16 && wtype != STTD_F32) return STTD_ERR_UNSUPPORTED;
    TRY(launch_embed_gather(embed, wtype == STTD_BF16 ? W_BF16 : W_F32, vocab, hidden, T, ids, keep, audio_dense, x,
                            ws ? ws->err : nullptr, (hipStream_t)stream));
    return STTD_OK;
}

static sttd_status check_block(const sttd_block_params* p, const sttd_block_weights* w, const sttd_workspace* ws,
                               const sttd_kv_cache* kv, int layer, int rows, const float* x) {
    if (!params_ok(p) || !weights_ok(w) || !ws || !kv || !x) return STTD_ERR_INVALID_ARG;
    const sttd_status sup = params_supported(p);
    if (sup != STTD_OK) return sup;
    if (!same_shape(p, &ws->p)) return STTD_ERR_INVALID_ARG;
    if (kv->n_kv != p->n_kv_heads || kv->d != p->head_dim) return STTD_ERR_INVALID_ARG;
    if (layer < 0 || layer >= kv->n_layers) return STTD_ERR_INVALID_ARG;
    if (rows <= 0 || rows > ws->max_rows) return STTD_ERR_INVALID_ARG;
    return STTD_OK;
}

sttd_status sttd_block_prefill(const sttd_block_params* p, const sttd_block_weights* w, sttd_workspace* ws,
                               sttd_kv_cache* kv, int layer, int seq, int pos0, int T, float* x, uint32_t flags,
                               void* stream) {
    const sttd_status st = check_block(p, w, ws, kv, layer, T, x);
    if (st != STTD_OK) return st;
    if (seq < 0 || seq >= kv->n_seq || pos0 < 0) return STTD_ERR_INVALID_ARG;
    if ((int64_t)pos0 + T > kv->n_ctx || (int64_t)pos0 + T > ws->max_pos) return STTD_ERR_CONTEXT_FULL;
    if (flags & ~(uint32_t)STTD_LAST_ROW_FFN_ONLY) return STTD_ERR_INVALID_ARG;
    RowMap rm{nullptr, nullptr, pos0, seq};
    return run_block(p, w, ws, kv, layer, T, rm, pos0 + T, true, (flags & STTD_LAST_ROW_FFN_ONLY) != 0, x,
                     (hipStream_t)stream);
}

sttd_status sttd_block_prefill_batched(const sttd_block_params* p, const sttd_block_weights* w, sttd_workspace* ws,
                                       sttd_kv_cache* kv, int layer, int n, const int32_t* seq, const int32_t* pos0,
                                       const int32_t* T, float* x, void* stream) {
    if (!seq || !pos0 || !T || n < 1 || n > kMaxSegments) return STTD_ERR_INVALID_ARG;
    Segments sg{};
    sg.n = n;
    int64_t rows = 0;
    for (int i = 0; i < n; ++i) {
        if (T[i] < 1 || pos0[i] < 0 || !kv || seq[i] < 0 || seq[i] >= kv->n_seq) return STTD_ERR_INVALID_ARG;
        for (int j = 0; j < i; ++j)
            if (seq[j] == seq[i]) return STTD_ERR_INVALID_ARG;  // two sequences in one slab
        sg.start[i] = (int)rows;
        sg.len[i] = T[i];
        sg.pos0[i] = pos0[i];
        sg.seq[i] = seq[i];
        rows += T[i];
    }
    if (rows > INT32_MAX) return STTD_ERR_INVALID_ARG;
    const sttd_status st = check_block(p, w, ws, kv, layer, (int)rows, x);
    if (st != STTD_OK) return st;
    int bound = 0;
    for (int i = 0; i < n; ++i) {
        if ((int64_t)pos0[i] + T[i] > kv->n_ctx || (int64_t)pos0[i] + T[i] > ws->max_pos)
            return STTD_ERR_CONTEXT_FULL;
        bound = std::max(bound, pos0[i] + T[i]);
    }
    hipStream_t s = (hipStream_t)stream;
    TRY(launch_expand_segments(sg, (int)rows, ws->rowpos, ws->rowseq, s));
    RowMap rm{ws->rowpos, ws->rowseq, 0, 0};
    return run_block(p, w, ws, kv, layer, (int)rows, rm, bound, true, false, x, s, &sg);
}

sttd_status sttd_block_step(const sttd_block_params* p, const sttd_block_weights* w, sttd_workspace* ws,
                            sttd_kv_cache* kv, int layer, int B, const int32_t* seq, const int32_t* pos,
                            int pos_bound, float* x, void* stream) {
    const sttd_status st = check_block(p, w, ws, kv, layer, B, x);
    if (st != STTD_OK) return st;
    if (!pos || pos_bound <= 0) return STTD_ERR_INVALID_ARG;
    if (pos_bound > kv->n_ctx || pos_bound > ws->max_pos) return STTD_ERR_CONTEXT_FULL;
    if (!seq && B > kv->n_seq) return STTD_ERR_INVALID_ARG;
    RowMap rm{pos, seq ? seq : ws->iota, 0, -1};
    return run_block(p, w, ws, kv, layer, B, rm, pos_bound, false, false, x, (hipStream_t)stream);
}

sttd_status sttd_lm_head_argmax(const void* final_norm, const void* embed, sttd_dtype wtype, int vocab, int hidden,
                                float rms_eps, sttd_workspace* ws, int B, const float* x, int64_t x_row_stride,
                                const int32_t* x_rows, int n_x_rows, int32_t* ids, float* logits, float* next_x,
                                int32_t* pos, void* stream) {
    if (!final_norm || !embed || !ws || !x || !ids || vocab <= 0 || hidden <= 0 || B <= 0) return STTD_ERR_INVALID_ARG;
    if (wtype != STTD_BF16 && wtype != STTD_F32) return STTD_ERR_UNSUPPORTED;
    if (hidden % 64 || hidden > 8192) return STTD_ERR_UNSUPPORTED;
    if (B > ws->max_rows || vocab > ws->vocab || x_row_stride < hidden) return STTD_ERR_INVALID_ARG;
    if (x_rows && n_x_rows < 1) return STTD_ERR_INVALID_ARG;
    HeadArgs a{};
    a.gain = final_norm; a.embed = embed; a.vocab = vocab; a.hidden = hidden; a.eps = rms_eps;
    a.x = x; a.ldx = x_row_stride; a.rows = B; a.ids = ids; a.logits = logits; a.next_x = next_x; a.pos = pos;
    a.xrow = x_rows; a.n_xrows = n_x_rows;
    a.partials = ws->partials; a.max_partials = kHeadPartials; a.err = ws->err;
    a.zbuf = hidden <= ws->p.hidden ? ws->xn : nullptr;  // 2 * B * hidden bf16 fit in the normed-row planes
    ProfScope ps(STTD_KERN_LM_HEAD, (hipStream_t)stream);
    TRY(launch_lm_head_argmax(a, wtype == STTD_BF16 ? W_BF16 : W_F32, (hipStream_t)stream));
    return STTD_OK;
}

}  // extern "C"

// ------------------------------------------------------------ allocation-free head
// Scratch of sttd_lm_head_argmax_static: per row the persistent head's 1024
// workgroup keys, then (hidden <= 2048) the normed rows as bf16 high and low
// planes for the MFMA head. One copy per device for the process's lifetime;
// host code reaches it only through the address hipGetSymbolAddress returns.
namespace {
constexpr int kStaticHeadHidden = 2048;  // widest row the MFMA head's planes hold
constexpr size_t kStaticPartialBytes = (size_t)STTD_STATIC_HEAD_MAX_ROWS * kHeadPartials * sizeof(unsigned long long);
constexpr size_t kStaticPlaneBytes = (size_t)2 * STTD_STATIC_HEAD_MAX_ROWS * kStaticHeadHidden * sizeof(uint16_t);
constexpr size_t kStaticScratchBytes = kStaticPartialBytes + kStaticPlaneBytes;
constexpr int kMaxDevices = 64;

std::mutex g_static_mu;
void* g_static_ptr[kMaxDevices] = {};
}  // namespace

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// The device address of this device's scratch copy, looked up once per device.
static sttd_status static_scratch(void** out) {
    int dev = -1;
    TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return STTD_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_static_mu);
    if (!g_static_ptr[dev]) {
        void* p = nullptr;
        TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p) return STTD_ERR_BACKEND;
        g_static_ptr[dev] = p;
    }
    *out = g_static_ptr[dev];
    return STTD_OK;
}

extern "C" {

sttd_status sttd_lm_head_argmax_static(const void* final_norm, const void* embed, sttd_dtype wtype, int vocab,
                                       int hidden, float rms_eps, int B, const float* x, int64_t x_row_stride,
                                       const int32_t* x_rows, int n_x_rows, int32_t* ids, float* logits,
                                       float* next_x, int32_t* pos, uint32_t* err, void* stream) {
    if (!final_norm || !embed || !x || !ids || vocab <= 0 || hidden <= 0 || B <= 0) return STTD_ERR_INVALID_ARG;
    if (wtype != STTD_BF16 && wtype != STTD_F32) return STTD_ERR_UNSUPPORTED;
    if (hidden % 64 || hidden > 8192) return STTD_ERR_UNSUPPORTED;
    if (B > STTD_STATIC_HEAD_MAX_ROWS || x_row_stride < hidden) return STTD_ERR_INVALID_ARG;
    if (x_rows && n_x_rows < 1) return STTD_ERR_INVALID_ARG;
    void* base = nullptr;
    const sttd_status st = static_scratch(&base);
    if (st != STTD_OK) return st;
    HeadArgs a{};
    a.gain = final_norm; a.embed = embed; a.vocab = vocab; a.hidden = hidden; a.eps = rms_eps;
    a.x = x; a.ldx = x_row_stride; a.rows = B; a.ids = ids; a.logits = logits; a.next_x = next_x; a.pos = pos;
    a.xrow = x_rows; a.n_xrows = n_x_rows;
    a.partials = (unsigned long long*)base; a.max_partials = kHeadPartials; a.err = err;
    a.zbuf = hidden <= kStaticHeadHidden ? (uint16_t*)((char*)base + kStaticPartialBytes) : nullptr;
    ProfScope ps(STTD_KERN_LM_HEAD, (hipStream_t)stream);
    TRY(launch_lm_head_argmax(a, wtype == STTD_BF16 ? W_BF16 : W_F32, (hipStream_t)stream));
    return STTD_OK;
}

sttd_status sttd_greedy_stop(const sttd_stop_rules* r, int B, const int32_t* ids, int advance, int32_t* pos,
                             int32_t* active, int32_t* n_gen, int32_t* tokens, int32_t* truncated, int32_t* n_active,
                             void* stream) {
    if (!r || !ids || !pos || !active || !n_gen || !tokens || !truncated || B <= 0) return STTD_ERR_INVALID_ARG;
    if (r->max_new < 1 || r->n_ctx < 1 || (advance != 0 && advance != 1)) return STTD_ERR_INVALID_ARG;
    TRY(launch_greedy_stop(B, ids, r->eos_id, r->max_new, r->n_ctx, advance, pos, active, n_gen, tokens, truncated,
                           n_active, (hipStream_t)stream));
    return STTD_OK;
}

sttd_status sttd_profile_enable(uint32_t mask) {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    g_prof.mask = mask & ((1u << STTD_KERN_COUNT) - 1);
    return STTD_OK;
}

sttd_status sttd_clock_enable(uint32_t mask, int max_launches) {
    if (max_launches < 0) return STTD_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lk(g_clk.mu);
    if (max_launches > g_clk.cap) {
        if (g_clk.slots) (void)hipFree(g_clk.slots);
        if (g_clk.red) (void)hipFree(g_clk.red);
        g_clk.slots = g_clk.red = nullptr;
        g_clk.cap = 0;
        if (hipMalloc(&g_clk.slots, kClockSlotBytes * (size_t)max_launches) != hipSuccess ||
            hipMalloc(&g_clk.red, 2 * sizeof(uint64_t) * (size_t)max_launches) != hipSuccess) {
            (void)hipGetLastError();
            if (g_clk.slots) (void)hipFree(g_clk.slots);
            g_clk.slots = nullptr;
            return STTD_ERR_OOM;
        }
        g_clk.cap = max_launches;
    }
    g_clk.used = 0;
    g_clk.kinds.clear();
    TRY(clock_fill(g_clk.cap));
    g_clk.mask = mask & ((1u << STTD_KERN_COUNT) - 1);
    return STTD_OK;
}

sttd_status sttd_clock_disable(void) {
    std::lock_guard<std::mutex> lk(g_clk.mu);
    g_clk.mask = 0;
    return STTD_OK;
}

sttd_status sttd_clock_reset(void) {
    std::lock_guard<std::mutex> lk(g_clk.mu);
    TRY(hipDeviceSynchronize());
    TRY(clock_fill(g_clk.used));
    return STTD_OK;
}

sttd_status sttd_clock_read(int kernel, int64_t* launches, double* total_us) {
    if (kernel < 0 || kernel >= STTD_KERN_COUNT || !launches || !total_us) return STTD_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lk(g_clk.mu);
    std::vector<uint64_t> h;
    TRY(clock_collect(h));
    int64_t n = 0;
    double us = 0.0;
    for (int i = 0; i < g_clk.used; ++i) {
        if (g_clk.kinds[i] != kernel || h[2 * i] == ~0ull || h[2 * i + 1] < h[2 * i]) continue;
        ++n;
        us += (double)(h[2 * i + 1] - h[2 * i]) * 0.01;  // 100 MHz clock
    }
    *launches = n;
    *total_us = us;
    return STTD_OK;
}

sttd_status sttd_clock_spans(int max, int* kinds, uint64_t* start_end, int* n) {
    if (max < 0 || !n || (max > 0 && (!kinds || !start_end))) return STTD_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lk(g_clk.mu);
    std::vector<uint64_t> h;
    TRY(clock_collect(h));
    const int m = max < g_clk.used ? max : g_clk.used;
    for (int i = 0; i < m; ++i) {
        kinds[i] = g_clk.kinds[i];
        start_end[2 * i] = h[2 * i];
        start_end[2 * i + 1] = h[2 * i + 1];
    }
    *n = m;
    return STTD_OK;
}

sttd_status sttd_profile_read(int kernel, int64_t* launches, double* total_ms) {
    if (kernel < 0 || kernel >= STTD_KERN_COUNT || !launches || !total_ms) return STTD_ERR_INVALID_ARG;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> pairs;
    int64_t calls = 0;
    {
        std::lock_guard<std::mutex> lk(g_prof.mu);
        pairs.swap(g_prof.timed[kernel]);
        calls = g_prof.calls[kernel];
        g_prof.calls[kernel] = 0;
    }
    double sum = 0.0;
    sttd_status st = STTD_OK;
    for (auto& pr : pairs) {
        float ms = 0.f;
        if (hipEventSynchronize(pr.second) != hipSuccess || hipEventElapsedTime(&ms, pr.first, pr.second) != hipSuccess)
            st = STTD_ERR_BACKEND;
        sum += ms;
    }
    {
        std::lock_guard<std::mutex> lk(g_prof.mu);
        for (auto& pr : pairs) {
            g_prof.pool.push_back(pr.first);
            g_prof.pool.push_back(pr.second);
        }
    }
    *launches = calls;
    *total_ms = sum;
    return st;
}

}  // extern "C"
