"""Device-side plumbing around the C ABI: torch supplies memory and streams,
every step of the decoder runs in libsttd's kernels.

DecoderSession holds one model's device weights, a KV cache and a workspace,
and strings the ABI calls together for a prefill, a decode step, the head, and
a greedy step loop (optionally captured once into a HIP graph and replayed).
"""
import numpy as np
import torch

from . import binding as B

WT_CODE = {"f32": B.F32, "bf16": B.BF16}
KV_CODE = {"f32": B.F32, "f16": B.F16}


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Host array in storage form to a device tensor (uint16 storage travels as int16 bits)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def stream_handle(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


class DecoderSession:
    def __init__(self, shape, layers, embed=None, final_norm=None, n_ctx=1024, n_seq=1, max_rows=1, device="cuda"):
        """shape: a DecoderShape; layers: list of host weight dicts (storage form);
        embed / final_norm: host arrays (storage form) or None."""
        self.shape = shape
        self.device = device
        self.params = B.block_params(shape.hidden, shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.ffn,
                                     shape.rms_eps, shape.rope_theta, WT_CODE[shape.wdtype])
        self.layer_tensors = [{k: to_device(v, device) for k, v in w.items()} for w in layers]
        self.layer_weights = [B.block_weights({k: t.data_ptr() for k, t in lt.items()}) for lt in self.layer_tensors]
        self.embed = to_device(embed, device) if embed is not None else None
        self.final_norm = to_device(final_norm, device) if final_norm is not None else None
        self.vocab = embed.shape[0] if embed is not None else 0
        self.n_ctx = n_ctx
        self.n_seq = n_seq
        self.max_rows = max_rows
        self.kv = B.kv_cache_alloc(len(layers), n_seq, n_ctx, shape.n_kv_heads, shape.head_dim,
                                   KV_CODE[shape.kvdtype])
        self.ws = B.workspace_alloc(self.params, max_rows, n_ctx, self.vocab)

    # ---------------------------------------------------------------- calls
    def prefill(self, x, pos0=0, seq=0, slice_last=False, layers=None, stream=None):
        """x: cuda float32 [T, hidden], overwritten with the last block's output."""
        s = stream_handle(stream)
        T = x.shape[0]
        idx = range(len(self.layer_weights)) if layers is None else layers
        last = len(self.layer_weights) - 1
        for l in idx:
            flags = B.LAST_ROW_FFN_ONLY if (slice_last and l == last) else 0
            B.block_prefill(self.params, self.layer_weights[l], self.ws, self.kv, l, seq, pos0, T, x.data_ptr(),
                            flags, s)
        return x

    def prefill_batched(self, x, T, seq, pos0=None, layers=None, stream=None):
        """x: cuda float32 [sum(T), hidden], the sequences packed back to back;
        sequence i has T[i] rows at positions pos0[i].. of slab seq[i]."""
        s = stream_handle(stream)
        pos0 = [0] * len(T) if pos0 is None else list(pos0)
        idx = range(len(self.layer_weights)) if layers is None else layers
        for l in idx:
            B.block_prefill_batched(self.params, self.layer_weights[l], self.ws, self.kv, l, list(seq), pos0,
                                    list(T), x.data_ptr(), s)
        return x

    def inject(self, ids, keep, audio_dense, x, stream=None):
        """x[t] = embed[ids[t]] * keep[t] + audio_dense[t] (cuda tensors)."""
        B.embed_inject(self.embed.data_ptr(), WT_CODE[self.shape.wdtype], self.vocab, self.shape.hidden, ids.shape[0],
                       ids.data_ptr(), keep.data_ptr(), audio_dense.data_ptr(), x.data_ptr(), self.ws,
                       stream_handle(stream))
        return x

    def step(self, x, pos, seq=None, pos_bound=None, layers=None, stream=None):
        """x: cuda float32 [B, hidden]; pos: cuda int32 [B]; seq: cuda int32 [B] or None (row b -> slab b)."""
        s = stream_handle(stream)
        Bn = x.shape[0]
        pb = self.n_ctx if pos_bound is None else pos_bound
        idx = range(len(self.layer_weights)) if layers is None else layers
        for l in idx:
            B.block_step(self.params, self.layer_weights[l], self.ws, self.kv, l, Bn,
                         0 if seq is None else seq.data_ptr(), pos.data_ptr(), pb, x.data_ptr(), s)
        return x

    def head(self, x, ids, logits=None, next_x=None, pos=None, row_stride=None, rows=None, x_rows=None, stream=None):
        """x_rows: optional cuda int32 [B] row indices into x (e.g. each packed prompt's last row)."""
        s = stream_handle(stream)
        if x_rows is not None:
            Bn = x_rows.shape[0]
        else:
            Bn = x.shape[0] if rows is None else rows
        B.lm_head_argmax(self.final_norm.data_ptr(), self.embed.data_ptr(), WT_CODE[self.shape.wdtype], self.vocab,
                         self.shape.hidden, self.shape.rms_eps, self.ws, Bn, x.data_ptr(),
                         self.shape.hidden if row_stride is None else row_stride, ids.data_ptr(),
                         0 if logits is None else logits.data_ptr(), 0 if next_x is None else next_x.data_ptr(),
                         0 if pos is None else pos.data_ptr(), s,
                         x_rows=0 if x_rows is None else x_rows.data_ptr(),
                         n_x_rows=0 if x_rows is None else x.shape[0])

    def gather(self, ids, x, stream=None):
        B.embed_gather(self.embed.data_ptr(), WT_CODE[self.shape.wdtype], self.vocab, self.shape.hidden,
                       ids.shape[0], ids.data_ptr(), x.data_ptr(), self.ws, stream_handle(stream))

    # ---------------------------------------------------------------- cache access (tests, fills)
    def kv_slab(self, layer, seq):
        """(K, V) device views of one slab as torch tensors [n_kv, n_ctx, d] (float32 or int16 bits)."""
        k, v, hs, ps = B.kv_cache_view(self.kv, layer, seq)
        sh = self.shape
        n = sh.n_kv_heads * self.n_ctx * sh.head_dim
        dt = torch.float32 if sh.kvdtype == "f32" else torch.int16
        return (_wrap(k, n, dt, self.device).view(sh.n_kv_heads, self.n_ctx, sh.head_dim),
                _wrap(v, n, dt, self.device).view(sh.n_kv_heads, self.n_ctx, sh.head_dim))

    def set_qkv_attn(self, enabled: bool):
        """STTD_OPT_QKV_ATTN: a single decode row's projection and attention in one launch (default on)."""
        B.workspace_set_option(self.ws, B.OPT_QKV_ATTN, 1 if enabled else 0)

    def set_act_split(self, mask: int):
        """STTD_OPT_ACT_SPLIT: GEMM inputs (B.SPLIT_* bits) kept as bf16 high + low parts above 512 rows."""
        B.workspace_set_option(self.ws, B.OPT_ACT_SPLIT, int(mask))

    def error_bits(self):
        return B.workspace_error(self.ws)

    def close(self):
        if self.kv:
            B.kv_cache_free(self.kv)
            self.kv = None
        if self.ws:
            B.workspace_free(self.ws)
            self.ws = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class _Raw:
    """Wraps a device address as a __cuda_array_interface__ producer for torch.as_tensor."""

    def __init__(self, ptr, n, typestr):
        self.__cuda_array_interface__ = {"shape": (n,), "typestr": typestr, "data": (ptr, False), "version": 3}


def _wrap(ptr, n, dtype, device):
    typestr = {torch.float32: "<f4", torch.int16: "<i2"}[dtype]
    return torch.as_tensor(_Raw(ptr, n, typestr), device=device)


def kv_to_f32(t: torch.Tensor) -> np.ndarray:
    """A cache slab view (float32, or int16 holding f16 bits) to host fp32."""
    a = t.detach().cpu().numpy()
    return a.view(np.float16).astype(np.float32) if a.dtype == np.int16 else a
