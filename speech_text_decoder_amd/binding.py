"""ctypes binding of libsttd.so (include/sttd.h): same names, argument marshalling only.

Every pointer argument is an integer device address (e.g. torch_tensor.data_ptr())
or 0 for NULL; `stream` is a hipStream_t as an integer (0: default stream;
torch.cuda.current_stream().cuda_stream for torch's current stream).
A non-OK status raises SttdError. Loading fails loudly when the library is
missing: there is no fallback path.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsttd.so")

OK, ERR_INVALID_ARG, ERR_OOM, ERR_BACKEND, ERR_CONTEXT_FULL, ERR_UNSUPPORTED = range(6)
F32, BF16, F16 = 0, 1, 2
LAST_ROW_FFN_ONLY = 1
DEVERR_POSITION, DEVERR_SLAB, DEVERR_TOKEN, DEVERR_SYNC, DEVERR_ROW = 1, 2, 4, 8, 16
OPT_ACT_SPLIT, OPT_QKV_ATTN = 2, 3
SPLIT_QKV, SPLIT_O, SPLIT_GATE_UP, SPLIT_DOWN = 1, 2, 4, 8
SPLIT_ALL = 15

EXPORTS = [
    "sttd_status_string", "sttd_kv_context_for", "sttd_kv_cache_alloc", "sttd_kv_cache_free", "sttd_kv_cache_clear", "sttd_kv_cache_view",
    "sttd_workspace_alloc", "sttd_workspace_free", "sttd_workspace_error", "sttd_workspace_set_option",
    "sttd_embed_gather", "sttd_embed_inject",
    "sttd_block_prefill", "sttd_block_prefill_batched", "sttd_block_step", "sttd_lm_head_argmax",
    "sttd_lm_head_argmax_static",
    "sttd_greedy_stop", "sttd_profile_enable", "sttd_profile_read",
    "sttd_clock_enable", "sttd_clock_disable", "sttd_clock_reset", "sttd_clock_read", "sttd_clock_spans",
]


class SttdError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_string(status)})")


class StopRules(ctypes.Structure):
    _fields_ = [("eos_id", ctypes.c_int32), ("max_new", ctypes.c_int32), ("n_ctx", ctypes.c_int32)]


class BlockParams(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("wtype", ctypes.c_int)]


WEIGHT_SLOTS = ["attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "ffn_norm", "w_gate_up", "w_down"]


class BlockWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_SLOTS]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        P = ctypes.POINTER
        L.sttd_status_string.restype = ctypes.c_char_p
        L.sttd_status_string.argtypes = [i32]
        L.sttd_kv_context_for.restype = i32
        L.sttd_kv_context_for.argtypes = [i32, i32]
        sigs = {
            "sttd_kv_cache_alloc": [i32, i32, i32, i32, i32, i32, P(vp)],
            "sttd_kv_cache_free": [vp],
            "sttd_kv_cache_clear": [vp, vp],
            "sttd_kv_cache_view": [vp, i32, i32, P(vp), P(vp), P(i64), P(i64)],
            "sttd_workspace_alloc": [P(BlockParams), i32, i32, i32, P(vp)],
            "sttd_workspace_free": [vp],
            "sttd_workspace_error": [vp, P(ctypes.c_uint32)],
            "sttd_workspace_set_option": [vp, i32, i32],
            "sttd_embed_gather": [vp, i32, i32, i32, i32, vp, vp, vp, vp],
            "sttd_embed_inject": [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp],
            "sttd_block_prefill": [P(BlockParams), P(BlockWeights), vp, vp, i32, i32, i32, i32, vp, ctypes.c_uint32,
                                   vp],
            "sttd_block_prefill_batched": [P(BlockParams), P(BlockWeights), vp, vp, i32, i32, P(i32), P(i32), P(i32),
                                           vp, vp],
            "sttd_block_step": [P(BlockParams), P(BlockWeights), vp, vp, i32, i32, vp, vp, i32, vp, vp],
            "sttd_lm_head_argmax": [vp, vp, i32, i32, i32, f32, vp, i32, vp, i64, vp, i32, vp, vp, vp, vp, vp],
            "sttd_lm_head_argmax_static": [vp, vp, i32, i32, i32, f32, i32, vp, i64, vp, i32, vp, vp, vp, vp, vp,
                                           vp],
            "sttd_greedy_stop": [P(StopRules), i32, vp, i32, vp, vp, vp, vp, vp, vp, vp],
            "sttd_profile_enable": [ctypes.c_uint32],
            "sttd_profile_read": [i32, P(i64), P(ctypes.c_double)],
            "sttd_clock_enable": [ctypes.c_uint32, i32],
            "sttd_clock_disable": [],
            "sttd_clock_reset": [],
            "sttd_clock_read": [i32, P(i64), P(ctypes.c_double)],
            "sttd_clock_spans": [i32, P(i32), P(ctypes.c_uint64), P(i32)],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = i32
        _lib = L
    return _lib


def status_string(status):
    return lib().sttd_status_string(status).decode()


def _check(status, what):
    if status != OK:
        raise SttdError(status, what)


def block_params(hidden, n_heads, n_kv_heads, head_dim, ffn, rms_eps, rope_theta, wtype):
    return BlockParams(hidden, n_heads, n_kv_heads, head_dim, ffn, rms_eps, rope_theta, wtype)


def block_weights(ptrs):
    """ptrs: mapping slot name -> device address."""
    return BlockWeights(*[ptrs[n] for n in WEIGHT_SLOTS])


def kv_cache_alloc(n_layers, n_seq, n_ctx, n_kv_heads, head_dim, kv_type):
    h = ctypes.c_void_p()
    _check(lib().sttd_kv_cache_alloc(n_layers, n_seq, n_ctx, n_kv_heads, head_dim, kv_type, ctypes.byref(h)),
           "sttd_kv_cache_alloc")
    return h.value


def kv_context_for(needed, ceiling):
    return lib().sttd_kv_context_for(needed, ceiling)


def kv_cache_free(kv):
    _check(lib().sttd_kv_cache_free(kv), "sttd_kv_cache_free")


def kv_cache_clear(kv, stream=0):
    _check(lib().sttd_kv_cache_clear(kv, stream), "sttd_kv_cache_clear")


def kv_cache_view(kv, layer, seq):
    k, v = ctypes.c_void_p(), ctypes.c_void_p()
    hs, ps = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().sttd_kv_cache_view(kv, layer, seq, ctypes.byref(k), ctypes.byref(v), ctypes.byref(hs),
                                    ctypes.byref(ps)), "sttd_kv_cache_view")
    return k.value, v.value, hs.value, ps.value


def workspace_alloc(params, max_rows, max_pos, vocab):
    h = ctypes.c_void_p()
    _check(lib().sttd_workspace_alloc(ctypes.byref(params), max_rows, max_pos, vocab, ctypes.byref(h)),
           "sttd_workspace_alloc")
    return h.value


def workspace_free(ws):
    _check(lib().sttd_workspace_free(ws), "sttd_workspace_free")


def workspace_set_option(ws, option, value):
    _check(lib().sttd_workspace_set_option(ws, option, value), "sttd_workspace_set_option")


def workspace_error(ws):
    bits = ctypes.c_uint32()
    _check(lib().sttd_workspace_error(ws, ctypes.byref(bits)), "sttd_workspace_error")
    return bits.value


def embed_gather(embed, wtype, vocab, hidden, B, ids, x, ws=0, stream=0):
    _check(lib().sttd_embed_gather(embed, wtype, vocab, hidden, B, ids, x, ws, stream), "sttd_embed_gather")


def embed_inject(embed, wtype, vocab, hidden, T, ids, keep, audio_dense, x, ws=0, stream=0):
    _check(lib().sttd_embed_inject(embed, wtype, vocab, hidden, T, ids, keep, audio_dense, x, ws, stream),
           "sttd_embed_inject")


def block_prefill(params, weights, ws, kv, layer, seq, pos0, T, x, flags=0, stream=0):
    _check(lib().sttd_block_prefill(ctypes.byref(params), ctypes.byref(weights), ws, kv, layer, seq, pos0, T, x,
                                    flags, stream), "sttd_block_prefill")


def block_prefill_batched(params, weights, ws, kv, layer, seq, pos0, T, x, stream=0):
    """seq, pos0, T: host sequences of ints (one entry per packed sequence)."""
    n = len(T)
    arr = ctypes.c_int32 * n
    _check(lib().sttd_block_prefill_batched(ctypes.byref(params), ctypes.byref(weights), ws, kv, layer, n,
                                            arr(*seq), arr(*pos0), arr(*T), x, stream), "sttd_block_prefill_batched")


def block_step(params, weights, ws, kv, layer, B, seq, pos, pos_bound, x, stream=0):
    _check(lib().sttd_block_step(ctypes.byref(params), ctypes.byref(weights), ws, kv, layer, B, seq, pos, pos_bound,
                                 x, stream), "sttd_block_step")


def greedy_stop(eos_id, max_new, n_ctx, B, ids, advance, pos, active, n_gen, tokens, truncated, n_active=0,
                stream=0):
    r = StopRules(eos_id, max_new, n_ctx)
    _check(lib().sttd_greedy_stop(ctypes.byref(r), B, ids, advance, pos, active, n_gen, tokens, truncated, n_active,
                                  stream), "sttd_greedy_stop")


def profile_enable(mask):
    _check(lib().sttd_profile_enable(mask), "sttd_profile_enable")


def profile_read(kernel):
    n, ms = ctypes.c_int64(), ctypes.c_double()
    _check(lib().sttd_profile_read(kernel, ctypes.byref(n), ctypes.byref(ms)), "sttd_profile_read")
    return n.value, ms.value


def clock_enable(mask, max_launches):
    _check(lib().sttd_clock_enable(mask, max_launches), "sttd_clock_enable")


def clock_disable():
    _check(lib().sttd_clock_disable(), "sttd_clock_disable")


def clock_reset():
    _check(lib().sttd_clock_reset(), "sttd_clock_reset")


def clock_read(kernel):
    n, us = ctypes.c_int64(), ctypes.c_double()
    _check(lib().sttd_clock_read(kernel, ctypes.byref(n), ctypes.byref(us)), "sttd_clock_read")
    return n.value, us.value


def clock_spans(max_slots):
    """[(kind, start_tick, end_tick)] of the slots handed out, in launch order."""
    kinds = (ctypes.c_int * max_slots)()
    se = (ctypes.c_uint64 * (2 * max_slots))()
    n = ctypes.c_int()
    _check(lib().sttd_clock_spans(max_slots, kinds, se, ctypes.byref(n)), "sttd_clock_spans")
    return [(kinds[i], se[2 * i], se[2 * i + 1]) for i in range(n.value)]


def lm_head_argmax(final_norm, embed, wtype, vocab, hidden, rms_eps, ws, B, x, x_row_stride, ids, logits=0,
                   next_x=0, pos=0, stream=0, x_rows=0, n_x_rows=0):
    """x_rows: device int32 [B] row indices into x (0: row b at x + b * x_row_stride)."""
    _check(lib().sttd_lm_head_argmax(final_norm, embed, wtype, vocab, hidden, rms_eps, ws, B, x, x_row_stride,
                                     x_rows, n_x_rows, ids, logits, next_x, pos, stream), "sttd_lm_head_argmax")


STATIC_HEAD_MAX_ROWS = 16


def lm_head_argmax_static(final_norm, embed, wtype, vocab, hidden, rms_eps, B, x, x_row_stride, ids, logits=0,
                          next_x=0, pos=0, err=0, stream=0, x_rows=0, n_x_rows=0):
    """The allocation-free head (no workspace; at most STATIC_HEAD_MAX_ROWS rows)."""
    _check(lib().sttd_lm_head_argmax_static(final_norm, embed, wtype, vocab, hidden, rms_eps, B, x, x_row_stride,
                                            x_rows, n_x_rows, ids, logits, next_x, pos, err, stream),
           "sttd_lm_head_argmax_static")
