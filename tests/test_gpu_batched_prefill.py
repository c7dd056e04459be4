"""Prompt/audio injection and the packed batched prefill through the C ABI,
against the oracle: several sequences packed back to back through one block
call (each attending only its own slab), a batch with short sequences (the
rows-attention path), a batch mixing a later chunk of one sequence with the
start of another, the injection blend, and injection -> batched prefill of a
2-block stack -> per-sequence last row -> head, with per-row greedy ids."""
import numpy as np
import pytest
import torch

import oracle as O
from speech_text_decoder_amd import binding as B
from speech_text_decoder_amd import synth
from speech_text_decoder_amd.device import DecoderSession, kv_to_f32
from speech_text_decoder_amd.workloads import WORKLOADS, DecoderShape
from dataclasses import replace
from tests.helpers import MARGIN, check, log, rel_err_rows, widen_layer

pytestmark = pytest.mark.gpu

SMALL128 = DecoderShape(hidden=512, n_heads=8, n_kv_heads=2, head_dim=128, ffn=768)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def packed_case(sh, cfg, Ts, slabs, pos0s=None, n_ctx=512, pre=None):
    """pre: {slab: rows} prefilled single-sequence first (earlier chunks)."""
    w = synth.block_weights(cfg, 0, sh)
    ow = widen_layer(w)
    n_seq = max(slabs) + 1
    pos0s = pos0s or [0] * len(Ts)
    total = sum(Ts)
    max_rows = max([total] + [len(r) for r in (pre or {}).values()])
    sess = DecoderSession(sh, [w], n_ctx=n_ctx, n_seq=n_seq, max_rows=max_rows)
    cache = O.KVCache(1, n_seq, n_ctx, sh.n_kv_heads, sh.head_dim)
    for slab, rows in (pre or {}).items():
        sess.prefill(dev(rows), seq=slab)
        O.block(rows, np.arange(len(rows)), np.full(len(rows), slab), ow, sh, cache, 0)
    x = synth.prefill_rows(cfg, total, sh.hidden)
    positions = np.concatenate([np.arange(p0, p0 + T) for p0, T in zip(pos0s, Ts)])
    seqs = np.concatenate([np.full(T, s) for s, T in zip(slabs, Ts)])
    want = O.block(x, positions, seqs, ow, sh, cache, 0)
    xd = dev(x)
    sess.prefill_batched(xd, Ts, slabs, pos0s)
    torch.cuda.synchronize()
    e = check(xd.cpu().numpy(), want, False, f"packed T={Ts} slabs={slabs} pos0={pos0s}")
    for s, p0, T in zip(slabs, pos0s, Ts):
        k, v = sess.kv_slab(0, s)
        gk = kv_to_f32(k)[:, p0:p0 + T].transpose(1, 0, 2).reshape(T, -1)
        gv = kv_to_f32(v)[:, p0:p0 + T].transpose(1, 0, 2).reshape(T, -1)
        check(gk, cache.k[0, s, p0:p0 + T].reshape(T, -1), False, f"K slab {s}")
        check(gv, cache.v[0, s, p0:p0 + T].reshape(T, -1), False, f"V slab {s}")
    assert sess.error_bits() == 0
    sess.close()
    return e, x, w


def test_packed_prefill_three_sequences_1p7b_block():
    wl = WORKLOADS["qwen3_1p7b_block_t153"]
    e, x, w = packed_case(wl.shape, 51, [17, 64, 153], [2, 0, 1], n_ctx=1024)
    log(f"packed 17+64+153 rows, 1.7B block: {e:.2e}")


def test_packed_prefill_matches_separate_calls():
    """The same rows through one packed call and through one call per sequence."""
    sh = SMALL128
    Ts, slabs = [33, 7, 90], [1, 2, 0]
    w = synth.block_weights(52, 0, sh)
    x = synth.prefill_rows(52, sum(Ts), sh.hidden)
    a = DecoderSession(sh, [w], n_ctx=256, n_seq=3, max_rows=sum(Ts))
    b = DecoderSession(sh, [w], n_ctx=256, n_seq=3, max_rows=sum(Ts))
    xa = dev(x)
    a.prefill_batched(xa, Ts, slabs)
    xb = dev(x)
    r0 = 0
    for T, s in zip(Ts, slabs):
        b.prefill(xb[r0:r0 + T], seq=s)
        r0 += T
    torch.cuda.synchronize()
    d = rel_err_rows(xa.cpu().numpy(), xb.cpu().numpy())
    log(f"packed vs separate: {d:.2e}")
    assert d <= 2e-3
    a.close()
    b.close()


@pytest.mark.parametrize("Ts", [[3, 40], [1, 2, 1], [5, 5, 5, 5]])
def test_packed_prefill_short_sequences(Ts):
    """A sequence of at most 4 rows sends the batch through the rows-attention
    kernel; a batch of at most 4 rows through the decode GEMVs."""
    e, _, _ = packed_case(SMALL128, 53, Ts, list(range(len(Ts))))
    log(f"packed {Ts}: {e:.2e}")


def test_packed_prefill_later_chunk_and_fresh_sequence():
    sh = SMALL128
    first = synth.prefill_rows(54, 100, sh.hidden) * 0.5
    e, _, _ = packed_case(sh, 55, [53, 30], [0, 1], pos0s=[100, 0], pre={0: first})
    log(f"chunk at 100 + fresh sequence: {e:.2e}")


def test_packed_prefill_argument_errors():
    sh = SMALL128
    sess = DecoderSession(sh, [synth.block_weights(56, 0, sh)], n_ctx=64, n_seq=2, max_rows=16)
    x = torch.zeros(16, sh.hidden, device="cuda")
    for seq, pos0, T, status in [([0, 0], [0, 0], [4, 4], B.ERR_INVALID_ARG),     # one slab twice
                                 ([0, 2], [0, 0], [4, 4], B.ERR_INVALID_ARG),     # slab out of range
                                 ([0, 1], [0, 0], [4, 0], B.ERR_INVALID_ARG),     # empty sequence
                                 ([0, 1], [0, 0], [12, 8], B.ERR_INVALID_ARG),    # 20 rows > max_rows
                                 ([0, 1], [60, 0], [8, 4], B.ERR_CONTEXT_FULL)]:  # 68 > n_ctx
        with pytest.raises(B.SttdError) as ex:
            B.block_prefill_batched(sess.params, sess.layer_weights[0], sess.ws, sess.kv, 0, seq, pos0, T,
                                    x.data_ptr())
        assert ex.value.status == status
    sess.close()


def test_injection_blend_bit_exact():
    sh = replace(SMALL128, vocab=3000)
    E = synth.embedding(57, sh)
    T, pre, n_audio = 40, 9, 25
    rng = np.random.default_rng(57)
    ids = rng.integers(0, sh.vocab, T).astype(np.int32)
    keep = np.ones(T, np.float32)
    keep[pre:pre + n_audio] = 0
    dense = np.zeros((T, sh.hidden), np.float32)
    dense[pre:pre + n_audio] = rng.standard_normal((n_audio, sh.hidden)).astype(np.float32)
    sess = DecoderSession(sh, [synth.block_weights(57, 0, sh)], embed=E, final_norm=synth.final_norm(57, sh),
                          n_ctx=64, max_rows=T)
    x = torch.zeros(T, sh.hidden, device="cuda")
    sess.inject(dev(ids), dev(keep), dev(dense), x)
    torch.cuda.synchronize()
    want = O.inject(synth.widen(E), ids, keep, dense)
    assert np.array_equal(x.cpu().numpy(), want.astype(np.float32))
    bad = ids.copy()
    bad[3] = sh.vocab
    sess.inject(dev(bad), dev(keep), dev(dense), x)
    torch.cuda.synchronize()
    assert np.all(x[3].cpu().numpy() == 0) and sess.error_bits() & B.DEVERR_TOKEN
    sess.close()


def test_injection_then_packed_stack_prefill_and_per_sequence_ids():
    """Two utterances: token embeddings with an audio block each, packed through
    a 2-block stack, each sequence's last row through the head."""
    sh = replace(SMALL128, n_layers=2, vocab=4000)
    layers = [synth.block_weights(58, l, sh) for l in range(2)]
    E = synth.embedding(58, sh)
    g = synth.final_norm(58, sh)
    Ts, slabs = [30, 47], [1, 0]
    rng = np.random.default_rng(58)
    ids = rng.integers(0, sh.vocab, sum(Ts)).astype(np.int32)
    keep = np.ones(sum(Ts), np.float32)
    dense = np.zeros((sum(Ts), sh.hidden), np.float32)
    for a, b in [(4, 20), (35, 66)]:        # audio rows of utterance 0 and 1
        keep[a:b] = 0
        dense[a:b] = rng.standard_normal((b - a, sh.hidden)).astype(np.float32)
    sess = DecoderSession(sh, layers, embed=E, final_norm=g, n_ctx=128, n_seq=2, max_rows=sum(Ts))
    x = torch.zeros(sum(Ts), sh.hidden, device="cuda")
    sess.inject(dev(ids), dev(keep), dev(dense), x)
    sess.prefill_batched(x, Ts, slabs)
    last = [Ts[0] - 1, sum(Ts) - 1]
    xl = x[last].contiguous()
    out_ids = torch.zeros(2, dtype=torch.int32, device="cuda")
    logits = torch.zeros(2, sh.vocab, device="cuda")
    sess.head(xl, out_ids, logits=logits)
    torch.cuda.synchronize()
    ol = [widen_layer(w) for w in layers]
    x0 = O.inject(synth.widen(E), ids, keep, dense)
    cache = O.KVCache(2, 2, 128, sh.n_kv_heads, sh.head_dim)
    positions = np.concatenate([np.arange(T) for T in Ts])
    seqs = np.concatenate([np.full(T, s) for s, T in zip(slabs, Ts)])
    xo = x0
    for l in range(2):
        xo = O.block(xo, positions, seqs, ol[l], sh, cache, l)
    want = O.final_logits(xo[last], synth.widen(g), synth.widen(E), sh.rms_eps)
    check(logits.cpu().numpy(), want, False, "per-sequence logits")
    got = out_ids.cpu().numpy()
    for b in range(2):
        if O.top2_margin(want[b]) > MARGIN:
            assert got[b] == O.greedy_token(want[b])
    assert sess.error_bits() == 0
    sess.close()


def test_packed_prefill_fp32_cache_rows_attention():
    """bf16 weights on an f32 cache: the packed rows go through the rows-attention
    kernel with per-row positions and slabs (no flash tiles)."""
    sh = replace(SMALL128, kvdtype="f32")
    e, _, _ = packed_case(sh, 59, [21, 9, 40], [1, 2, 0], pos0s=[0, 0, 0])
    log(f"packed on an f32 cache: {e:.2e}")


def test_packed_prefill_fp32_weights_tiny_block():
    """The fp32 block (fp32 weights, f32 cache) packed: 1e-4 relative bound."""
    sh = WORKLOADS["tiny_fp32_block"].shape
    w = synth.block_weights(60, 0, sh)
    ow = widen_layer(w)
    Ts, slabs = [12, 20], [1, 0]
    x = synth.prefill_rows(60, sum(Ts), sh.hidden)
    sess = DecoderSession(sh, [w], n_ctx=64, n_seq=2, max_rows=sum(Ts))
    cache = O.KVCache(1, 2, 64, sh.n_kv_heads, sh.head_dim)
    positions = np.concatenate([np.arange(T) for T in Ts])
    seqs = np.concatenate([np.full(T, s) for s, T in zip(slabs, Ts)])
    want = O.block(x, positions, seqs, ow, sh, cache, 0)
    xd = dev(x)
    sess.prefill_batched(xd, Ts, slabs)
    torch.cuda.synchronize()
    check(xd.cpu().numpy(), want, True, "packed fp32 block")
    assert sess.error_bits() == 0
    sess.close()
