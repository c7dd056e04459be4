"""The single-row projection + attention launch (STTD_OPT_QKV_ATTN, tagged
hand-off between the projection's and the attention's workgroups) against the
two-launch form of the same step and against the oracle.

The two forms run the same arithmetic in the same order (the projection
workgroups reuse the GEMV's loads, dot products and merge; the attention items
are the same code), so from one cache state they must give the same block
output and cache rows bit for bit. Both forms therefore start every step from
the same state: one session, its cache saved before and restored between the
two forms (two separate prefills would already differ in their last bits: the
prefill GEMMs split K with fp32 atomic adds).
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle as O
from speech_text_decoder_amd import binding as B
from speech_text_decoder_amd import synth
from speech_text_decoder_amd.device import DecoderSession
from speech_text_decoder_amd.workloads import WORKLOADS, DecoderShape
from tests.helpers import check, log, widen_layer

pytestmark = pytest.mark.gpu

MHA128 = DecoderShape(hidden=512, n_heads=4, n_kv_heads=4, head_dim=128, ffn=384)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def cache_views(sess, n_layers):
    return [t for l in range(n_layers) for t in sess.kv_slab(l, 0)]


def both_forms_steps(sh, cfg, T, steps, n_ctx, pos_bound_of):
    """Prefill T rows once, then `steps` single-row steps on the same layer; each
    step runs with the option on, the cache is restored, and it runs again with
    the option off. Checks the one-launch output against the oracle and both
    forms against each other, bit for bit (outputs and the cache rows written)."""
    w = synth.block_weights(cfg, 0, sh)
    ow = widen_layer(w)
    x = synth.prefill_rows(cfg, T, sh.hidden)
    sess = DecoderSession(sh, [w], n_ctx=n_ctx, max_rows=T)
    sess.prefill(dev(x))
    cache = O.KVCache(1, 1, n_ctx, sh.n_kv_heads, sh.head_dim)
    O.block(x, np.arange(T), np.zeros(T, int), ow, sh, cache, 0)
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    views = cache_views(sess, 1)
    for k in range(steps):
        xs = synth.step_rows(cfg, k, 1, sh.hidden)
        want = O.block(xs, [T + k], [0], ow, sh, cache, 0)
        saved = [v.clone() for v in views]
        out, rows = {}, {}
        for on in (True, False):
            for v, s in zip(views, saved):
                v.copy_(s)
            sess.set_qkv_attn(on)
            xd = dev(xs)
            pos.fill_(T + k)
            sess.step(xd, pos, pos_bound=pos_bound_of(T + k))
            torch.cuda.synchronize()
            out[on] = xd.cpu().numpy()
            rows[on] = [v[:, T + k].cpu().numpy() for v in views]
        check(out[True], want, False, f"step {k}")
        assert np.array_equal(out[True], out[False]), f"step {k}: one launch differs from two"
        for a, b in zip(rows[True], rows[False]):
            assert np.array_equal(a, b), f"step {k}: cache row differs"
    assert sess.error_bits() == 0
    sess.close()


@pytest.mark.parametrize("pos_bound", ["tight", "n_ctx"])
def test_one_launch_equals_two_launches_1p7b_block(pos_bound):
    """1.7B-shaped block after a 153-row prefill, 24 steps on one layer (every
    launch must take fresh words, not the previous launch's): 2-3 splits
    (tight bound) and 8 splits of 128 rows (the greedy graph's bound)."""
    wl = WORKLOADS["qwen3_1p7b_block_t153"]
    bound = (lambda p: p + 1) if pos_bound == "tight" else (lambda p: wl.n_ctx)
    both_forms_steps(wl.shape, wl.cfg_id, wl.prefill_rows, 24, wl.n_ctx, bound)
    log(f"one launch = two launches bit for bit over 24 steps ({pos_bound} bound)")


def test_one_launch_mha_group1_against_oracle():
    """Groups of one query head per KV head (the other instantiation)."""
    both_forms_steps(MHA128, 43, 150, 6, 512, lambda p: 512)


def test_one_launch_graph_replays_match_eager_loops():
    """Two 0.6B-shaped blocks (hidden 1024) and the head in a greedy loop from one
    prefilled state: the loop captured once in a HIP graph and replayed (every
    replay takes a new tag, advanced by the launch itself, no host update) gives
    the logits and ids of the eager one-launch loop and of the eager two-launch
    loop, bit for bit."""
    wl = WORKLOADS["qwen3_0p6b_stack28_greedy256"]
    sh = replace(wl.shape, n_layers=2, vocab=4096)
    layers = [synth.block_weights(44, l, sh) for l in range(2)]
    E = synth.embedding(44, sh)
    g = synth.final_norm(44, sh)
    T, steps, n_ctx = 140, 16, 512
    sess = DecoderSession(sh, layers, embed=E, final_norm=g, n_ctx=n_ctx, max_rows=T)
    x = dev(synth.prefill_rows(44, T, sh.hidden))
    sess.prefill(x, slice_last=True)
    ids = torch.zeros(1, dtype=torch.int32, device="cuda")
    pos = torch.full((1,), T, dtype=torch.int32, device="cuda")
    xs = torch.zeros(1, sh.hidden, device="cuda")
    logits = torch.zeros(1, sh.vocab, device="cuda")
    sess.head(x[T - 1:], ids, next_x=xs)
    torch.cuda.synchronize()
    views = cache_views(sess, 2)
    saved = [v.clone() for v in views]
    xs0, ids0 = xs.clone(), int(ids.item())

    def reset():
        for v, s in zip(views, saved):
            v.copy_(s)
        xs.copy_(xs0)
        pos.fill_(T)
        torch.cuda.synchronize()

    def loop(one_launch, replay=None):
        reset()
        sess.set_qkv_attn(one_launch)
        out, lg = [ids0], []
        for _ in range(steps):
            if replay is not None:
                replay()
            else:
                sess.step(xs, pos, pos_bound=n_ctx)
                sess.head(xs, ids, logits=logits, next_x=xs, pos=pos)
            torch.cuda.synchronize()
            out.append(int(ids.item()))
            lg.append(logits.cpu().numpy()[0].copy())
        return out, lg

    ids_e2, lg_e2 = loop(False)
    ids_e1, lg_e1 = loop(True)
    sess.set_qkv_attn(True)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(graph, stream=st):
            sess.step(xs, pos, pos_bound=n_ctx)
            sess.head(xs, ids, logits=logits, next_x=xs, pos=pos)
    torch.cuda.current_stream().wait_stream(st)
    ids_g, lg_g = loop(True, replay=graph.replay)
    assert ids_g == ids_e1 == ids_e2
    for k in range(steps):
        assert np.array_equal(lg_g[k], lg_e1[k]), f"replay {k}: graph differs from the eager one-launch loop"
        assert np.array_equal(lg_e1[k], lg_e2[k]), f"step {k}: one-launch loop differs from two-launch loop"
    assert sess.error_bits() == 0
    sess.close()
    log(f"{steps} replays = eager loops bit for bit: ids {ids_g[:6]}...")


def test_qkv_attn_option_validation():
    sh = MHA128
    sess = DecoderSession(sh, [synth.block_weights(45, 0, sh)], n_ctx=64, max_rows=4)
    with pytest.raises(B.SttdError) as e:
        B.workspace_set_option(sess.ws, B.OPT_QKV_ATTN, 2)
    assert e.value.status == B.ERR_INVALID_ARG
    sess.set_qkv_attn(False)
    sess.set_qkv_attn(True)
    sess.close()
