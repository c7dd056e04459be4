"""The fused single-row decode step (one persistent launch per block, stages
handed over through device counters) against the per-stage launches of the
same block and against the oracle: the 1.7B-shaped block after a 153-row
prefill, a GQA-group-8 block with head_dim 128, and a greedy loop captured in
a HIP graph and replayed."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle as O
from speech_text_decoder_amd import binding as B
from speech_text_decoder_amd import synth
from speech_text_decoder_amd.device import DecoderSession, kv_to_f32
from speech_text_decoder_amd.workloads import WORKLOADS, DecoderShape
from tests.helpers import check, log, rel_err_rows, widen_layer

pytestmark = pytest.mark.gpu

# fused and per-stage steps run the same arithmetic; only the order of the
# fp32 partial sums differs (4 or 8 rows per workgroup), so they agree to a few
# fp32 ulps of the row scale; the f16 cache rows may differ in their last bit
TOL_SAME = 1e-5
GROUP8 = DecoderShape(hidden=512, n_heads=8, n_kv_heads=1, head_dim=128, ffn=384)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_fused_step_matches_per_stage_launches_1p7b_block():
    wl = WORKLOADS["qwen3_1p7b_block_t153"]
    sh, T, steps = wl.shape, wl.prefill_rows, 24
    w = synth.block_weights(wl.cfg_id, 0, sh)
    ow = widen_layer(w)
    x = synth.prefill_rows(wl.cfg_id, T, sh.hidden)
    sess = {f: DecoderSession(sh, [w], n_ctx=wl.n_ctx, max_rows=T) for f in (True, False)}
    for f, s in sess.items():
        s.set_fused_step(f)
        s.prefill(dev(x))
    cache = O.KVCache(1, 1, wl.n_ctx, sh.n_kv_heads, sh.head_dim)
    O.block(x, np.arange(T), np.zeros(T, int), ow, sh, cache, 0)
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    worst = 0.0
    for k in range(steps):
        xs = synth.step_rows(wl.cfg_id, k, 1, sh.hidden)
        want = O.block(xs, [T + k], [0], ow, sh, cache, 0)
        out = {}
        for f, s in sess.items():
            xd = dev(xs)
            pos.fill_(T + k)
            s.step(xd, pos, pos_bound=T + k + 1)
            torch.cuda.synchronize()
            out[f] = xd.cpu().numpy()
        check(out[True], want, False, f"fused step {k}")
        e = rel_err_rows(out[True], out[False])
        worst = max(worst, e)
        assert e <= TOL_SAME, f"step {k}: fused vs per-stage {e:.3g}"
    kf = kv_to_f32(sess[True].kv_slab(0, 0)[0])[:, :T + steps]
    ku = kv_to_f32(sess[False].kv_slab(0, 0)[0])[:, :T + steps]
    vf = kv_to_f32(sess[True].kv_slab(0, 0)[1])[:, :T + steps]
    vu = kv_to_f32(sess[False].kv_slab(0, 0)[1])[:, :T + steps]
    assert np.max(np.abs(kf - ku)) <= 2e-3 * np.max(np.abs(ku))
    assert np.max(np.abs(vf - vu)) <= 2e-3 * np.max(np.abs(vu))
    for s in sess.values():
        assert s.error_bits() == 0
        s.close()
    log(f"fused vs per-stage, {steps} steps: max row-relative difference {worst:.2e}")


@pytest.mark.parametrize("pos0", [1, 127, 300])
def test_fused_step_group8_head128_against_oracle(pos0):
    """One attention split (short span, the attention output is written whole)
    and several (the O stage merges the split partials as it loads)."""
    sh = GROUP8
    w = synth.block_weights(41, 0, sh)
    ow = widen_layer(w)
    n_ctx = 1024
    x = synth.prefill_rows(41, pos0, sh.hidden)
    sess = DecoderSession(sh, [w], n_ctx=n_ctx, max_rows=pos0)
    sess.set_fused_step(True)
    sess.prefill(dev(x))
    cache = O.KVCache(1, 1, n_ctx, sh.n_kv_heads, sh.head_dim)
    O.block(x, np.arange(pos0), np.zeros(pos0, int), ow, sh, cache, 0)
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    for k in range(3):
        xs = synth.step_rows(41, k, 1, sh.hidden)
        want = O.block(xs, [pos0 + k], [0], ow, sh, cache, 0)
        xd = dev(xs)
        pos.fill_(pos0 + k)
        sess.step(xd, pos, pos_bound=pos0 + k + 1)
        torch.cuda.synchronize()
        check(xd.cpu().numpy(), want, False, f"group-8 step at {pos0 + k}")
    assert sess.error_bits() == 0
    sess.close()


def test_fused_step_graph_replay_matches_eager_and_per_stage():
    """Two 1.7B-wide blocks and the head in a greedy loop: the fused steps
    captured once in a HIP graph and replayed give the ids of the eager fused
    loop and of the eager per-stage loop; the counters come back to zero
    after every launch (each replay reuses them)."""
    wl = WORKLOADS["qwen3_1p7b_block_t153"]
    sh = replace(wl.shape, n_layers=2, vocab=4096)
    layers = [synth.block_weights(42, l, sh) for l in range(2)]
    E = synth.embedding(42, sh)
    g = synth.final_norm(42, sh)
    T, steps = 20, 12
    x0 = synth.prefill_rows(42, T, sh.hidden)

    def run(fused, use_graph):
        sess = DecoderSession(sh, layers, embed=E, final_norm=g, n_ctx=256, max_rows=T)
        sess.set_fused_step(fused)
        x = dev(x0)
        sess.prefill(x, slice_last=True)
        ids = torch.zeros(1, dtype=torch.int32, device="cuda")
        pos = torch.full((1,), T, dtype=torch.int32, device="cuda")
        xs = torch.zeros(1, sh.hidden, device="cuda")
        logits = torch.zeros(1, sh.vocab, device="cuda")
        sess.head(x[T - 1:], ids, next_x=xs)
        out, lg = [int(ids.item())], []
        if use_graph:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.stream(s):
                with torch.cuda.graph(graph, stream=s):
                    sess.step(xs, pos, pos_bound=T + steps + 1)
                    sess.head(xs, ids, logits=logits, next_x=xs, pos=pos)
            torch.cuda.current_stream().wait_stream(s)
        for _ in range(steps):
            if use_graph:
                graph.replay()
            else:
                sess.step(xs, pos, pos_bound=T + steps + 1)
                sess.head(xs, ids, logits=logits, next_x=xs, pos=pos)
            torch.cuda.synchronize()
            out.append(int(ids.item()))
            lg.append(logits.cpu().numpy()[0].copy())
        assert int(pos.item()) == T + steps
        assert sess.error_bits() == 0
        sess.close()
        return out, np.array(lg)

    fe, lfe = run(True, False)
    fg, lfg = run(True, True)
    pe, lpe = run(False, False)
    log(f"fused eager {fe}\nfused graph {fg}\nper-stage   {pe}")
    assert fe == fg
    # the prefill's split-K GEMMs add with fp32 atomics, so two runs differ in
    # the last bits of the cache; the replayed steps must agree to that level
    assert np.max(np.abs(lfe - lfg)) <= 1e-4 * np.max(np.abs(lfe))
    # the two schedules may round differently; they must pick the same ids
    # wherever the logits' top-2 margin is clear of that rounding
    for k in range(steps):
        top2 = np.sort(lpe[k])[-2:]
        if top2[1] - top2[0] > 1e-3:
            assert fe[k + 1] == pe[k + 1], f"step {k}"
    assert np.max(np.abs(lfe - lpe)) <= 1e-3 * np.max(np.abs(lpe))


def test_fused_step_option_validation():
    sh = GROUP8
    sess = DecoderSession(sh, [synth.block_weights(43, 0, sh)], n_ctx=32, max_rows=1)
    B.workspace_set_option(sess.ws, B.OPT_FUSED_STEP, 1)
    B.workspace_set_option(sess.ws, B.OPT_FUSED_STEP, 0)
    with pytest.raises(B.SttdError) as e:
        B.workspace_set_option(sess.ws, B.OPT_FUSED_STEP, 2)
    assert e.value.status == B.ERR_INVALID_ARG
    with pytest.raises(B.SttdError) as e:
        B.workspace_set_option(sess.ws, 99, 1)
    assert e.value.status == B.ERR_INVALID_ARG
    sess.close()
