"""GPU parity of the 28-block 1.7B-shaped stack on whole jobs, against the oracle:

* the greedy job (153-row prefill with the last-row slice, then all 255 decode
  steps) driven through the same captured HIP graph of 28 block steps + head
  that the benchmark replays, teacher-forced: after each replay the oracle's
  token is fed back, and every one of the 256 logits rows and ids is checked;
* the packed prefill job: 8 injected prompts of 153 rows (1224 rows per block
  call, above the 512-row precision switch) through 28 blocks, then one head
  call over each prompt's last row picked by row index on the device;
* the same with ragged prompt lengths;
* the batched-decode job: 16 rows with cache lengths 150-1500 through the
  captured graph the benchmark replays, every row of 6 replays checked.

Tolerances: per row, max |gpu - oracle| / RMS(oracle row) <= 3e-2 on hidden
states and logits; ids equal wherever the oracle's top-2 margin exceeds 1e-2,
else the GPU pick lies within 1e-2 of the largest logit.
"""
import numpy as np
import pytest
import torch

import oracle as O
from speech_text_decoder_amd import synth
from speech_text_decoder_amd.device import DecoderSession
from speech_text_decoder_amd.workloads import WORKLOADS
from tests.helpers import MARGIN, check, log, rel_err_rows, widen_layer_f64

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def check_ids(got, o_logits, what):
    """C-21: the oracle's id where its top-2 margin exceeds MARGIN, else a near-maximal pick."""
    for i, a in enumerate(got):
        m = O.top2_margin(o_logits[i])
        if m > MARGIN:
            assert a == O.greedy_token(o_logits[i]), f"{what} {i}: gpu {a} oracle {O.greedy_token(o_logits[i])} " \
                                                     f"(margin {m:.3g})"
        else:
            assert o_logits[i][a] >= np.nanmax(o_logits[i]) - MARGIN, f"{what} {i}: gpu pick {a} not near the max"


_WEIGHTS = {}


def stack_weights(wl):
    """Host weights of a 28-block workload (storage form and fp64), cached per workload."""
    if wl.name not in _WEIGHTS:
        _WEIGHTS.clear()
        sh = wl.shape
        log(f"generating {sh.n_layers} blocks + embedding for {wl.name}")
        layers = [synth.block_weights(wl.cfg_id, l, sh) for l in range(sh.n_layers)]
        E = synth.embedding(wl.cfg_id, sh)
        g = synth.final_norm(wl.cfg_id, sh)
        _WEIGHTS[wl.name] = (layers, E, g, [widen_layer_f64(w) for w in layers], synth.widen(E).astype(np.float64),
                             synth.widen(g))
    return _WEIGHTS[wl.name]


def test_stack28_greedy256_all_tokens_teacher_forced_through_the_replayed_graph():
    wl = WORKLOADS["qwen3_1p7b_stack28_greedy256"]
    sh = wl.shape
    T, n_new = wl.prefill_rows, wl.steps + 1
    layers, E, g, ol, Ef, gf = stack_weights(wl)
    x = synth.prefill_rows(wl.cfg_id, T, sh.hidden)
    sess = DecoderSession(sh, layers, embed=E, final_norm=g, n_ctx=wl.n_ctx, max_rows=T)
    xs = torch.zeros(1, sh.hidden, device="cuda")
    ids = torch.zeros(1, dtype=torch.int32, device="cuda")
    pos = torch.full((1,), T, dtype=torch.int32, device="cuda")
    logits = torch.zeros(1, sh.vocab, device="cuda")
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    # the decode step as the benchmark captures it (28 block steps + head, device
    # token feedback and position bump), with the logits kept for the check
    with torch.cuda.stream(stream):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            sess.step(xs, pos, pos_bound=wl.n_ctx)
            sess.head(xs, ids, logits=logits, next_x=xs, pos=pos)
    torch.cuda.synchronize()
    pos.fill_(T)
    with torch.cuda.stream(stream):
        xd = dev(x)
        sess.prefill(xd, slice_last=True)
        sess.head(xd[T - 1:], ids, logits=logits, next_x=xs)
    torch.cuda.synchronize()
    gpu_ids = [int(ids.item())]
    gpu_logits = [logits[0].cpu().numpy()]

    log("oracle prefill")
    cache = O.KVCache(sh.n_layers, 1, T + n_new + 1, sh.n_kv_heads, sh.head_dim)
    last = O.prefill_stack(x, ol, sh, cache, slice_last=True)
    check(xd[T - 1:].cpu().numpy(), last, False, "prefill last row")
    o_logits = [O.final_logits(last, gf, Ef, sh.rms_eps)[0]]
    o_ids = [O.greedy_token(o_logits[0])]
    for k in range(1, n_new):
        feed = o_ids[-1]
        if gpu_ids[-1] != feed:   # teacher forcing: the next input row is the oracle token's
            with torch.cuda.stream(stream):
                sess.gather(dev(np.array([feed], np.int32)), xs)
        with torch.cuda.stream(stream):
            graph.replay()
        xo = O.step_stack(Ef[feed][None], [T + k - 1], [0], ol, sh, cache)
        o_logits.append(O.final_logits(xo, gf, Ef, sh.rms_eps)[0])
        o_ids.append(O.greedy_token(o_logits[-1]))
        torch.cuda.synchronize()
        gpu_logits.append(logits[0].cpu().numpy())
        gpu_ids.append(int(ids.item()))
        if k % 32 == 0:
            log(f"step {k}: gpu {gpu_ids[-1]} oracle {o_ids[-1]} "
                f"logits err {rel_err_rows(gpu_logits[-1][None], o_logits[-1][None]):.3g}")
    assert int(pos.item()) == T + n_new - 1
    errs = [check(a[None], b[None], False, f"logits {i}") for i, (a, b) in enumerate(zip(gpu_logits, o_logits))]
    check_ids(gpu_ids, o_logits, "token")
    agree = sum(a == b for a, b in zip(gpu_ids, o_ids))
    log(f"256 tokens: logits max row-rel err {max(errs):.3g} (mean {np.mean(errs):.3g}); ids agree {agree}/256")
    assert sess.error_bits() == 0
    sess.close()


def packed_stack_case(wl, Ts, ids_h, keep_h, dense_h):
    """Inject + pack len(Ts) prompts through every block, then one head call over
    the prompts' last rows picked by device row index. Returns the largest errors."""
    sh = wl.shape
    layers, E, g, ol, Ef, gf = stack_weights(wl)
    n, total = len(Ts), int(sum(Ts))
    sess = DecoderSession(sh, layers, embed=E, final_norm=g, n_ctx=wl.n_ctx, n_seq=n, max_rows=total)
    x = torch.empty(total, sh.hidden, device="cuda")
    sess.inject(dev(ids_h), dev(keep_h), dev(dense_h), x)
    sess.prefill_batched(x, list(Ts), list(range(n)))
    last = np.cumsum(Ts) - 1
    out_ids = torch.zeros(n, dtype=torch.int32, device="cuda")
    logits = torch.zeros(n, sh.vocab, device="cuda")
    sess.head(x, out_ids, logits=logits, x_rows=dev(last.astype(np.int32)))
    torch.cuda.synchronize()
    g_last = x[torch.from_numpy(last).cuda()].cpu().numpy()
    g_logits = logits.cpu().numpy()
    g_ids = out_ids.cpu().numpy()
    assert sess.error_bits() == 0
    sess.close()
    errs_x, errs_l = [], []
    o_logits = []
    start = 0
    for b, Tb in enumerate(Ts):
        r = slice(start, start + Tb)
        start += Tb
        cache = O.KVCache(sh.n_layers, 1, Tb, sh.n_kv_heads, sh.head_dim)
        x0 = O.inject(Ef, ids_h[r], keep_h[r], dense_h[r])
        lo = O.prefill_stack(x0, ol, sh, cache)[-1:]
        ll = O.final_logits(lo, gf, Ef, sh.rms_eps)
        o_logits.append(ll[0])
        errs_x.append(check(g_last[b:b + 1], lo, False, f"prompt {b} last row"))
        errs_l.append(check(g_logits[b:b + 1], ll, False, f"prompt {b} logits"))
    check_ids(g_ids, o_logits, "prompt")
    log(f"packed {list(Ts)}: last rows max err {max(errs_x):.3g}, logits max err {max(errs_l):.3g}, "
        f"ids {g_ids.tolist()} oracle {[O.greedy_token(l) for l in o_logits]}")
    return max(errs_x), max(errs_l)


def test_stack28_packed_prefill_8x153_injected_with_device_last_rows():
    """The packed-prefill job as benchmarked: 1224 rows per block call."""
    wl = WORKLOADS["qwen3_1p7b_stack28_packed_prefill_b8"]
    sh = wl.shape
    ids_h, keep_h, dense_h = synth.injected_prompts(wl.cfg_id, wl.batch, wl.prompt_split, sh.hidden, sh.vocab)
    packed_stack_case(wl, [wl.prefill_rows] * wl.batch, ids_h, keep_h, dense_h)


def test_stack28_packed_prefill_ragged_prompts_one_head_call():
    """Ragged prompts (1198 rows packed): each prompt's last row sits at its own
    offset, gathered by the head's row index in one call (more than 4 rows: the
    MFMA head)."""
    wl = WORKLOADS["qwen3_1p7b_stack28_packed_prefill_b8"]
    sh = wl.shape
    Ts = [153, 97, 201, 64, 180, 133, 250, 120]
    rng = np.random.default_rng(77)
    total = sum(Ts)
    ids_h = rng.integers(0, sh.vocab, total).astype(np.int32)
    keep_h = np.ones(total, np.float32)
    dense_h = np.zeros((total, sh.hidden), np.float32)
    start = 0
    for Tb in Ts:                     # an audio block inside each prompt
        a, b = start + 9, start + Tb - 6
        keep_h[a:b] = 0
        dense_h[a:b] = rng.standard_normal((b - a, sh.hidden)).astype(np.float32)
        start += Tb
    packed_stack_case(wl, Ts, ids_h, keep_h, dense_h)


def test_batched_decode_b16_all_rows_through_the_replayed_graph():
    """The batched-decode job as benchmarked: 16 rows with seeded cache lengths
    150-1500 through the captured graph (28 block steps + head with device token
    feedback and position bump), 6 replays. Every row of every replay is checked:
    the oracle steps each row through its own slab, following the GPU's tokens,
    and must agree on the logits (C-20) and on the ids (C-21)."""
    wl = WORKLOADS["qwen3_1p7b_stack28_batched_decode_b16"]
    sh = wl.shape
    Bn, n_ctx, steps = wl.batch, wl.n_ctx, 6
    lens = synth.context_lengths(wl.cfg_id, Bn, *wl.ctx_len_range)
    layers, E, g, ol, Ef, gf = stack_weights(wl)
    sess = DecoderSession(sh, layers, embed=E, final_norm=g, n_ctx=n_ctx, n_seq=Bn, max_rows=Bn)
    stored = {}
    for l in range(sh.n_layers):
        for b in range(Bn):
            k, v = synth.kv_fill(wl.cfg_id, l, b, int(lens[b]), sh, n_ctx)
            kq, vq = synth.kv_stored(k, sh.kvdtype), synth.kv_stored(v, sh.kvdtype)
            gk, gv = sess.kv_slab(l, b)
            gk[:, :lens[b], :] = dev(kq.view(np.int16)).permute(1, 0, 2)
            gv[:, :lens[b], :] = dev(vq.view(np.int16)).permute(1, 0, 2)
            stored[l, b] = (kq, vq)
    log("KV slabs filled")
    x0 = synth.step_rows(wl.cfg_id, 0, Bn, sh.hidden)
    x = dev(x0)
    pos = dev(lens.astype(np.int32))
    ids = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    logits = torch.zeros(Bn, sh.vocab, device="cuda")
    bound = int(lens.max()) + steps + 1
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            sess.step(x, pos, pos_bound=bound)
            sess.head(x, ids, logits=logits, next_x=x, pos=pos)
    torch.cuda.synchronize()
    g_logits, g_ids = [], []
    for _ in range(steps):
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
        g_logits.append(logits.cpu().numpy().copy())
        g_ids.append(ids.cpu().numpy().copy())
    assert pos.cpu().numpy().tolist() == (lens + steps).tolist()
    assert sess.error_bits() == 0
    sess.close()
    errs = []
    for b in range(Bn):
        L = int(lens[b])
        cache = O.KVCache(sh.n_layers, 1, L + steps + 1, sh.n_kv_heads, sh.head_dim)
        for l in range(sh.n_layers):
            kq, vq = stored[l, b]
            cache.k[l, 0, :L] = synth.kv_widen(kq)
            cache.v[l, 0, :L] = synth.kv_widen(vq)
        xo = x0[b:b + 1].astype(np.float64)
        o_logits = []
        for k in range(steps):
            xo = O.step_stack(xo, [L + k], [0], ol, sh, cache)
            o_logits.append(O.final_logits(xo, gf, Ef, sh.rms_eps)[0])
            xo = Ef[int(g_ids[k][b])][None]          # follow the GPU's token
        errs += [check(g_logits[k][b:b + 1], o_logits[k][None], False, f"row {b} step {k} logits")
                 for k in range(steps)]
        check_ids([int(g_ids[k][b]) for k in range(steps)], o_logits, f"row {b} step")
    log(f"16 rows x {steps} replays: logits max row-rel err {max(errs):.3g} (mean {np.mean(errs):.3g})")
