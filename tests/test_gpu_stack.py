"""GPU parity at the full workload sizes, on outputs the oracle can afford:

* 28-block 1.7B-shaped stack and 28-block 0.6B-shaped stack (the MOSS
  decoder: attention width 2048 over a 1024-wide residual), 153-row prefill
  (last-row slice on), tied head, then 8 teacher-forced greedy steps (the
  oracle's tokens are fed back): first-block output, last-row output, logits
  and ids.
* batched decode, B = 16 slabs with seeded context lengths in [150, 1500]
  and seeded KV fills: the GPU steps all 16 rows; three sampled rows are
  recomputed by the oracle for two steps.
* one 1.7B-shaped block with a 4096-row prefill (sampled rows; the oracle
  needs every row's K and V but attention only for the samples), then 16
  decode steps at positions 4096..4111.
"""
import numpy as np
import pytest
import torch

import oracle as O
from speech_text_decoder_amd import synth
from speech_text_decoder_amd.device import DecoderSession, kv_to_f32
from speech_text_decoder_amd.workloads import WORKLOADS
from tests.helpers import MARGIN, check, log, widen_layer_f64

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("workload", ["qwen3_1p7b_stack28_greedy256", "qwen3_0p6b_stack28_greedy256"])
def test_stack28_prefill153_head_and_teacher_forced_steps(workload):
    wl = WORKLOADS[workload]
    sh = wl.shape
    T, n_check = wl.prefill_rows, 8
    log("generating 28 blocks + embedding")
    layers = [synth.block_weights(wl.cfg_id, l, sh) for l in range(sh.n_layers)]
    E = synth.embedding(wl.cfg_id, sh)
    g = synth.final_norm(wl.cfg_id, sh)
    x = synth.prefill_rows(wl.cfg_id, T, sh.hidden)
    sess = DecoderSession(sh, layers, embed=E, final_norm=g, n_ctx=wl.n_ctx, max_rows=T)

    # GPU: prefill block 0 alone (dump point), then the rest with the last-row slice
    xd = dev(x)
    sess.prefill(xd, layers=[0])
    torch.cuda.synchronize()
    gpu_b0 = xd.cpu().numpy()
    for l in range(1, sh.n_layers):
        flags_last = l == sh.n_layers - 1
        sess.prefill(xd, layers=[l], slice_last=flags_last)
    ids = torch.zeros(1, dtype=torch.int32, device="cuda")
    logits = torch.zeros(1, sh.vocab, device="cuda")
    xs = torch.zeros(1, sh.hidden, device="cuda")
    sess.head(xd[T - 1:], ids, logits=logits)
    torch.cuda.synchronize()
    gpu_last = xd[T - 1].cpu().numpy()
    gpu_logits = [logits[0].cpu().numpy()]
    gpu_ids = [int(ids.item())]

    log("oracle prefill")
    ol = [widen_layer_f64(w) for w in layers]
    Ef = synth.widen(E).astype(np.float64)
    gf = synth.widen(g)
    cache = O.KVCache(sh.n_layers, 1, T + n_check + 1, sh.n_kv_heads, sh.head_dim)
    keep = {}
    last = O.prefill_stack(x, ol, sh, cache, slice_last=True, keep=keep)
    e0 = check(gpu_b0, keep[0], False, "block 0 output")
    e1 = check(gpu_last[None], last, False, "last block, last row")
    log(f"block 0 output err {e0:.3g}; last block last row err {e1:.3g}")
    o_logits = [O.final_logits(last, gf, Ef, sh.rms_eps)[0]]
    o_ids = [O.greedy_token(o_logits[0])]

    pos = torch.full((1,), T, dtype=torch.int32, device="cuda")
    for k in range(1, n_check):
        feed = o_ids[-1]
        # GPU step fed the oracle's token
        sess.gather(dev(np.array([feed], np.int32)), xs)
        sess.step(xs, pos, pos_bound=T + k)
        sess.head(xs, ids, logits=logits, pos=pos)
        torch.cuda.synchronize()
        gpu_logits.append(logits[0].cpu().numpy())
        gpu_ids.append(int(ids.item()))
        # oracle step
        xo = O.step_stack(Ef[feed][None], [T + k - 1], [0], ol, sh, cache)
        o_logits.append(O.final_logits(xo, gf, Ef, sh.rms_eps)[0])
        o_ids.append(O.greedy_token(o_logits[-1]))
        log(f"step {k}: gpu {gpu_ids[-1]} oracle {o_ids[-1]} margin {O.top2_margin(o_logits[-1]):.3g}")
    from tests.helpers import rel_err_rows
    errs = [rel_err_rows(gl[None], ol_[None]) for gl, ol_ in zip(gpu_logits, o_logits)]
    log("logits row-RMS-relative errors: " + " ".join(f"{e:.3g}" for e in errs))
    errs = [check(gl[None], ol_[None], False, f"logits {i}") for i, (gl, ol_) in enumerate(zip(gpu_logits, o_logits))]
    for i, (a, b) in enumerate(zip(gpu_ids, o_ids)):
        m = O.top2_margin(o_logits[i])
        if m > MARGIN:
            assert a == b, f"token {i}: gpu {a} oracle {b} (margin {m:.3g})"
        else:   # near-tie: the GPU's pick must be one of the near-maximal logits
            assert o_logits[i][a] >= o_logits[i].max() - MARGIN
    log(f"stack28 logits max row-rel err {max(errs):.2e}; ids gpu {gpu_ids} oracle {o_ids}")
    assert sess.error_bits() == 0
    sess.close()


def test_batched_decode_b16_sampled_rows():
    wl = WORKLOADS["qwen3_1p7b_stack28_batched_decode_b16"]
    sh = wl.shape
    Bn, n_ctx = wl.batch, wl.n_ctx
    lens = synth.context_lengths(wl.cfg_id, Bn, *wl.ctx_len_range)
    sample = [int(np.argmin(lens)), 7, int(np.argmax(lens))]
    log(f"context lengths {lens.tolist()}, sampled rows {sample}")
    layers = [synth.block_weights(wl.cfg_id, l, sh) for l in range(sh.n_layers)]
    E = synth.embedding(wl.cfg_id, sh)
    g = synth.final_norm(wl.cfg_id, sh)
    sess = DecoderSession(sh, layers, embed=E, final_norm=g, n_ctx=n_ctx, n_seq=Bn, max_rows=Bn)
    n_steps = 2
    cache = O.KVCache(sh.n_layers, len(sample), int(lens.max()) + n_steps + 1, sh.n_kv_heads, sh.head_dim)
    for l in range(sh.n_layers):
        for b in range(Bn):
            k, v = synth.kv_fill(wl.cfg_id, l, b, int(lens[b]), sh, n_ctx)
            kq, vq = synth.kv_stored(k, sh.kvdtype), synth.kv_stored(v, sh.kvdtype)
            gk, gv = sess.kv_slab(l, b)
            gk[:, :lens[b], :] = dev(kq.view(np.int16)).permute(1, 0, 2)
            gv[:, :lens[b], :] = dev(vq.view(np.int16)).permute(1, 0, 2)
            if b in sample:
                s = sample.index(b)
                cache.k[l, s, :lens[b]] = synth.kv_widen(kq)
                cache.v[l, s, :lens[b]] = synth.kv_widen(vq)
    log("KV slabs filled")
    ol = [widen_layer_f64(w) for w in layers]
    Ef = synth.widen(E).astype(np.float64)
    gf = synth.widen(g)
    x = synth.step_rows(wl.cfg_id, 0, Bn, sh.hidden)
    xd = dev(x)
    pos = dev(lens.astype(np.int32))
    ids = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    logits = torch.zeros(Bn, sh.vocab, device="cuda")
    xo = x[sample].astype(np.float64)
    for k in range(n_steps):
        sess.step(xd, pos, pos_bound=int(lens.max()) + k + 1)
        torch.cuda.synchronize()
        gx = xd.cpu().numpy()
        sess.head(xd, ids, logits=logits, pos=pos)
        torch.cuda.synchronize()
        xo = O.step_stack(xo, lens[sample] + k, list(range(len(sample))), ol, sh, cache)
        check(gx[sample], xo, False, f"step {k} block outputs")
        o_logits = O.final_logits(xo, gf, Ef, sh.rms_eps)
        check(logits.cpu().numpy()[sample], o_logits, False, f"step {k} logits")
        got = ids.cpu().numpy()
        o_ids = [O.greedy_token(r) for r in o_logits]
        for i, b in enumerate(sample):
            if O.top2_margin(o_logits[i]) > MARGIN:
                assert got[b] == o_ids[i], f"step {k} row {b}: gpu {got[b]} oracle {o_ids[i]}"
        log(f"step {k}: ids gpu {got[sample].tolist()} oracle {o_ids}")
        # teacher forcing for the sampled rows, the GPU's own ids elsewhere
        feed = got.copy()
        feed[sample] = o_ids
        sess.gather(dev(feed.astype(np.int32)), xd)
        xo = Ef[o_ids]
    assert pos.cpu().numpy().tolist() == (lens + n_steps).tolist()
    assert sess.error_bits() == 0
    sess.close()


@pytest.mark.parametrize("act_split", [0, 15])
def test_long4096_block_sampled_prefill_rows_and_16_steps(act_split):
    """act_split 0: plain bf16 activations (the single-block long-prefill figure);
    15: every activation split (the library default)."""
    wl = WORKLOADS["qwen3_1p7b_block_long4096"]
    sh = wl.shape
    T = wl.prefill_rows
    w = synth.block_weights(wl.cfg_id, 0, sh)
    ow = widen_layer_f64(w)
    x = synth.prefill_rows(wl.cfg_id, T, sh.hidden)
    sess = DecoderSession(sh, [w], n_ctx=wl.n_ctx, max_rows=T)
    sess.set_act_split(act_split)
    xd = dev(x)
    sess.prefill(xd)
    torch.cuda.synchronize()
    gx = xd.cpu().numpy()
    sample = [0, 1, 2, 63, 64, 65, 127, 128, 1000, 2047, 2048, 3333, 4094, 4095]
    cache = O.KVCache(1, 1, T + 16 + 1, sh.n_kv_heads, sh.head_dim)
    log("oracle sampled prefill rows")
    want = O.block_rows_subset(x, 0, ow, sh, cache, 0, sample)
    check(gx[sample], want, False, "prefill 4096 sampled rows")
    gk, gv = sess.kv_slab(0, 0)
    gk = kv_to_f32(gk)[:, :T].transpose(1, 0, 2)
    gv = kv_to_f32(gv)[:, :T].transpose(1, 0, 2)
    check(gk.reshape(T, -1), cache.k[0, 0, :T].reshape(T, -1), False, "K cache rows")
    check(gv.reshape(T, -1), cache.v[0, 0, :T].reshape(T, -1), False, "V cache rows")
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    errs = []
    for k in range(16):
        xs = synth.step_rows(wl.cfg_id, k, 1, sh.hidden)
        want = O.block(xs, [T + k], [0], ow, sh, cache, 0)
        xsd = dev(xs)
        pos.fill_(T + k)
        sess.step(xsd, pos, pos_bound=T + k + 1)
        torch.cuda.synchronize()
        errs.append(check(xsd.cpu().numpy(), want, False, f"step {k}"))
    log(f"long4096 steps max err {max(errs):.2e}")
    assert sess.error_bits() == 0
    sess.close()
