"""Seeded synthetic inputs shared by the HIP path's tests and bench and by the oracle's callers.

This module draws numbers and lays them out; it holds none of the decoder's
arithmetic. The generator itself (counter-based splitmix64 + Box-Muller in
fp64) is the host C file csrc/synth.c, built into libsttd_synth.so.

Recipe (every tensor has its own stream, so any one can be regenerated alone):
  stream id = workload_cfg_id * 1024 + layer * 32 + slot
  matrices (Wq, Wk, Wv, Wo, W_gate, W_up, W_down, E) ~ N(0, 0.02^2)
  RMSNorm gains (attention, FFN, Q-norm, K-norm, final) ~ 1 + N(0, 0.02^2)
  input rows ~ N(0, 1); KV fills (batched decode) ~ N(0, 1)
  values are drawn in fp64, rounded to fp32 (RNE), and for bf16 storage
  rounded again to bf16 (RNE on the fp32 bits).
The packed gate_up matrix is [2*ffn, hidden]: gate rows first, then up rows.
"""
import ctypes
import os

import numpy as np

SEED = 0x5EED2026

# per-block tensor slots
SLOT = dict(attn_norm=0, wq=1, wk=2, wv=3, q_norm=4, k_norm=5, wo=6, ffn_norm=7,
            w_gate=8, w_up=9, w_down=10, kv_fill_k=12, kv_fill_v=13)
# workload-wide tensors live under layer 31
GLOBAL_LAYER = 31
GSLOT = dict(embed=0, final_norm=1, x_prefill=2, x_step=3, ctx_len=6, prompt_ids=7, audio_rows=8)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsttd_synth.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build          # host-only C, builds in a second
            build.build_synth()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.sttd_synth_normal_f32.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                              ctypes.c_double, ctypes.c_double, ctypes.c_void_p]
        lib.sttd_synth_uniform_int.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                               ctypes.c_int32, ctypes.c_void_p]
        lib.sttd_synth_f32_to_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
        _lib = lib
    return _lib


def stream_id(cfg_id: int, layer: int, slot: int) -> int:
    assert 0 <= layer < 32 and 0 <= slot < 32
    return cfg_id * 1024 + layer * 32 + slot


def normal(stream: int, shape, std: float = 1.0, mean: float = 0.0, offset: int = 0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    if n:
        _load().sttd_synth_normal_f32(SEED, stream, offset, n, mean, std, out.ctypes.data)
    return out.reshape(shape)


def uniform_int(stream: int, n: int, lo: int, hi: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    if n:
        _load().sttd_synth_uniform_int(SEED, stream, n, lo, hi, out.ctypes.data)
    return out


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    if a.size:
        _load().sttd_synth_f32_to_bf16(a.ctypes.data, out.ctypes.data, a.size)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_f16_bits(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def stored(a: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 values in their storage form: fp32 as is, bf16 as uint16 bits."""
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        return to_bf16_bits(a)
    raise ValueError(dtype)


def widen(a: np.ndarray) -> np.ndarray:
    """Storage form back to fp32 values (exact): uint16 means bf16 bits."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a)
    return np.asarray(a, dtype=np.float32)


def block_weights(cfg_id: int, layer: int, shape) -> dict:
    """One block's weights in storage form (dict of numpy arrays).

    Keys follow the block's ten weight slots; gate and up are returned packed
    as w_gate_up [2*ffn, hidden] (gate rows first)."""
    h, d, i = shape.hidden, shape.head_dim, shape.ffn
    s = lambda slot: stream_id(cfg_id, layer, SLOT[slot])
    dt = shape.wdtype
    w = {
        "attn_norm": normal(s("attn_norm"), (h,), 0.02, 1.0),
        "wq": normal(s("wq"), (shape.q_dim, h), 0.02),
        "wk": normal(s("wk"), (shape.kv_dim, h), 0.02),
        "wv": normal(s("wv"), (shape.kv_dim, h), 0.02),
        "q_norm": normal(s("q_norm"), (d,), 0.02, 1.0),
        "k_norm": normal(s("k_norm"), (d,), 0.02, 1.0),
        "wo": normal(s("wo"), (h, shape.q_dim), 0.02),
        "ffn_norm": normal(s("ffn_norm"), (h,), 0.02, 1.0),
        "w_gate_up": np.concatenate([normal(s("w_gate"), (i, h), 0.02), normal(s("w_up"), (i, h), 0.02)], axis=0),
        "w_down": normal(s("w_down"), (h, i), 0.02),
    }
    return {k: stored(v, dt) for k, v in w.items()}


def embedding(cfg_id: int, shape) -> np.ndarray:
    return stored(normal(stream_id(cfg_id, GLOBAL_LAYER, GSLOT["embed"]), (shape.vocab, shape.hidden), 0.02),
                  shape.wdtype)


def final_norm(cfg_id: int, shape) -> np.ndarray:
    return stored(normal(stream_id(cfg_id, GLOBAL_LAYER, GSLOT["final_norm"]), (shape.hidden,), 0.02, 1.0),
                  shape.wdtype)


def prefill_rows(cfg_id: int, n_rows: int, hidden: int) -> np.ndarray:
    return normal(stream_id(cfg_id, GLOBAL_LAYER, GSLOT["x_prefill"]), (n_rows, hidden))


def step_rows(cfg_id: int, step: int, n_rows: int, hidden: int) -> np.ndarray:
    """Fresh N(0,1) decode input rows for step `step` (non-greedy workloads)."""
    return normal(stream_id(cfg_id, GLOBAL_LAYER, GSLOT["x_step"]), (n_rows, hidden), offset=step * n_rows * hidden)


def injected_prompts(cfg_id: int, n_prompts: int, split, hidden: int, vocab: int):
    """n_prompts prompts of prefix + audio + suffix rows, packed back to back:
    token ids uniform over the vocabulary, keep 0 at the audio rows and 1
    elsewhere, N(0,1) audio rows at the audio positions (zero elsewhere), the
    inputs of the injection blend. Returns (ids int32 [n*T], keep f32 [n*T],
    dense f32 [n*T, hidden])."""
    pre, n_audio, suf = split
    T = pre + n_audio + suf
    ids = uniform_int(stream_id(cfg_id, GLOBAL_LAYER, GSLOT["prompt_ids"]), n_prompts * T, 0, vocab - 1)
    keep = np.ones(n_prompts * T, dtype=np.float32)
    dense = np.zeros((n_prompts * T, hidden), dtype=np.float32)
    audio = normal(stream_id(cfg_id, GLOBAL_LAYER, GSLOT["audio_rows"]), (n_prompts * n_audio, hidden))
    for b in range(n_prompts):
        r = slice(b * T + pre, b * T + pre + n_audio)
        keep[r] = 0.0
        dense[r] = audio[b * n_audio:(b + 1) * n_audio]
    return ids, keep, dense


def context_lengths(cfg_id: int, batch: int, lo: int, hi: int) -> np.ndarray:
    return uniform_int(stream_id(cfg_id, GLOBAL_LAYER, GSLOT["ctx_len"]), batch, lo, hi)


def kv_fill(cfg_id: int, layer: int, seq: int, n_rows: int, shape, n_ctx: int):
    """Seeded N(0,1) K and V rows [n_rows, n_kv_heads, head_dim] for one (layer, sequence) slab.

    Row r of sequence `seq` draws from counter offset (seq*n_ctx + r)*kv_dim of
    the layer's K (or V) stream, so slabs are independent of each other."""
    kvd = shape.kv_dim
    off = seq * n_ctx * kvd
    k = normal(stream_id(cfg_id, layer, SLOT["kv_fill_k"]), (n_rows, shape.n_kv_heads, shape.head_dim), offset=off)
    v = normal(stream_id(cfg_id, layer, SLOT["kv_fill_v"]), (n_rows, shape.n_kv_heads, shape.head_dim), offset=off)
    return k, v


def kv_stored(a: np.ndarray, kvdtype: str) -> np.ndarray:
    """KV values in cache storage form: f32 as is, f16 as uint16 bits (RNE)."""
    return np.ascontiguousarray(a, np.float32) if kvdtype == "f32" else to_f16_bits(a)


def kv_widen(a: np.ndarray) -> np.ndarray:
    return a.view(np.float16).astype(np.float32) if a.dtype == np.uint16 else np.asarray(a, np.float32)
