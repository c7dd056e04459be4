"""GPU parity of one decoder block through the C ABI against the CPU oracle:
the tiny fp32 block, small bf16 blocks with ragged row counts, chunked
prefill, batched decode rows, the 1.7B-shaped block at T = 153, the head's
argmax, device-side bounds checks, and HIP-graph replay of a step loop."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle as O
from speech_text_decoder_amd import binding as B
from speech_text_decoder_amd import synth
from speech_text_decoder_amd.device import DecoderSession, kv_to_f32
from speech_text_decoder_amd.workloads import WORKLOADS, DecoderShape
from tests.helpers import MARGIN, check, log, widen_layer

pytestmark = pytest.mark.gpu

SMALL64 = DecoderShape(hidden=256, n_heads=4, n_kv_heads=2, head_dim=64, ffn=512)
SMALL128 = DecoderShape(hidden=512, n_heads=8, n_kv_heads=1, head_dim=128, ffn=384)


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t if dtype is None else t.to(dtype)


def oracle_kv_rows(cache, layer, seq, positions):
    """Oracle cache rows [len(positions), n_kv, d]."""
    return cache.k[layer, seq, positions], cache.v[layer, seq, positions]


def gpu_kv_rows(sess, layer, seq, positions):
    k, v = sess.kv_slab(layer, seq)
    k = kv_to_f32(k)[:, positions, :].transpose(1, 0, 2)
    v = kv_to_f32(v)[:, positions, :].transpose(1, 0, 2)
    return k, v


def run_block_case(shape, cfg_id, T, steps, n_ctx, chunks=None, seed_layer=0, act_split=None):
    """Prefill T rows (optionally in chunks) then `steps` single-row decode steps; compare every output.
    act_split: STTD_OPT_ACT_SPLIT mask for calls above 512 rows (None: the library default, all split)."""
    fp32 = shape.wdtype == "f32"
    w = synth.block_weights(cfg_id, seed_layer, shape)
    ow = widen_layer(w)
    x = synth.prefill_rows(cfg_id, T, shape.hidden)
    sess = DecoderSession(shape, [w], n_ctx=n_ctx, max_rows=max(T, 1))
    if act_split is not None:
        sess.set_act_split(act_split)
    cache = O.KVCache(1, 1, n_ctx, shape.n_kv_heads, shape.head_dim)
    want = O.block(x, np.arange(T), np.zeros(T, int), ow, shape, cache, 0)
    xd = dev(x)
    bounds = chunks or [T]
    start = 0
    for n in bounds:
        sess.prefill(xd[start:start + n], pos0=start)
        start += n
    torch.cuda.synchronize()
    e = check(xd.cpu().numpy(), want, fp32, f"prefill T={T} chunks={bounds}")
    gk, gv = gpu_kv_rows(sess, 0, 0, np.arange(T))
    ok_, ov_ = oracle_kv_rows(cache, 0, 0, np.arange(T))
    check(gk.reshape(T, -1), ok_.reshape(T, -1), fp32, "K cache")
    check(gv.reshape(T, -1), ov_.reshape(T, -1), fp32, "V cache")
    errs = [e]
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    for k in range(steps):
        xs = synth.step_rows(cfg_id, k, 1, shape.hidden)
        want = O.block(xs, [T + k], [0], ow, shape, cache, 0)
        xsd = dev(xs)
        pos.fill_(T + k)
        sess.step(xsd, pos, pos_bound=T + k + 1)
        torch.cuda.synchronize()
        errs.append(check(xsd.cpu().numpy(), want, fp32, f"step {k}"))
    assert sess.error_bits() == 0
    sess.close()
    return errs


def test_tiny_fp32_block_prefill_32_then_8_steps():
    wl = WORKLOADS["tiny_fp32_block"]
    errs = run_block_case(wl.shape, wl.cfg_id, wl.prefill_rows, wl.steps, wl.n_ctx)
    log(f"tiny fp32 max rel errors: prefill {errs[0]:.2e}, steps {max(errs[1:]):.2e}")


@pytest.mark.parametrize("T", [1, 3, 4, 5, 17, 64, 65, 130])
def test_small_bf16_block_ragged_rows(T):
    errs = run_block_case(SMALL64, 11, T, 2, 256)
    log(f"SMALL64 T={T}: {max(errs):.2e}")


@pytest.mark.parametrize("T", [1, 7, 96, 161])
def test_small_bf16_head128_group8(T):
    errs = run_block_case(SMALL128, 12, T, 2, 256)
    log(f"SMALL128 T={T}: {max(errs):.2e}")


@pytest.mark.parametrize("act_split", [0, B.SPLIT_ALL, B.SPLIT_O | B.SPLIT_DOWN])
def test_many_rows_large_tiles_with_row_and_column_tails(act_split):
    """1100 rows: with plain bf16 activations the 256 x 256 MFMA tiles (4 full row tiles
    and a ragged one; the hidden size 320 leaves a partial column tile in the O and down
    projections); with split ones (the default) the 64 x 128 tiles on hi/lo planes; and
    a mixed mask."""
    sh = DecoderShape(hidden=320, n_heads=4, n_kv_heads=2, head_dim=64, ffn=768)
    errs = run_block_case(sh, 15, 1100, 1, 1200, act_split=act_split)
    log(f"T=1100 H=320 split {act_split}: {max(errs):.2e}")


@pytest.mark.parametrize("T", [513, 700])
@pytest.mark.parametrize("act_split", [0, B.SPLIT_ALL])
def test_mid_size_prefill_rows_with_split_k(T, act_split):
    """513-1023 rows: the 64x128-tile GEMMs with plain or split activations, with K split
    over workgroups (atomic adds) where few of them run."""
    errs = run_block_case(SMALL128, 18, T, 1, 768, act_split=act_split)
    log(f"SMALL128 T={T} split {act_split}: {max(errs):.2e}")


@pytest.mark.parametrize("act_split", [0, B.SPLIT_ALL])
def test_chunked_prefill_with_a_large_tile_chunk(act_split):
    """A 1030-row chunk (256x256 MFMA tiles with plain activations, flash attention at
    pos0 = 70) after a 70-row one."""
    sh = DecoderShape(hidden=320, n_heads=4, n_kv_heads=2, head_dim=64, ffn=768)
    errs = run_block_case(sh, 19, 1100, 1, 1200, chunks=[70, 1030], act_split=act_split)
    log(f"chunks [70, 1030] H=320 split {act_split}: {max(errs):.2e}")


def test_small_fp32_kv_cache_bf16_weights():
    sh = replace(SMALL64, kvdtype="f32")
    errs = run_block_case(sh, 13, 40, 3, 128)
    log(f"bf16 weights + f32 KV: {max(errs):.2e}")


@pytest.mark.parametrize("chunks", [[70, 60], [1, 64, 65], [64, 64, 2]])
def test_chunked_prefill_matches_single_shot(chunks):
    errs = run_block_case(SMALL64, 14, sum(chunks), 1, 256, chunks=chunks)
    log(f"chunks {chunks}: {max(errs):.2e}")


@pytest.mark.parametrize("Bn", [1, 2, 3, 4, 5, 16, 40])
def test_batched_decode_rows_match_independent_rows(Bn):
    """Rows of one step sit in distinct slabs at different positions."""
    sh = SMALL64
    w = synth.block_weights(15, 0, sh)
    ow = widen_layer(w)
    n_ctx = 96
    lens = synth.context_lengths(15, Bn, 1, 60)
    sess = DecoderSession(sh, [w], n_ctx=n_ctx, n_seq=Bn, max_rows=Bn)
    cache = O.KVCache(1, Bn, n_ctx, sh.n_kv_heads, sh.head_dim)
    for b in range(Bn):
        k, v = synth.kv_fill(15, 0, b, int(lens[b]), sh, n_ctx)
        kq, vq = synth.kv_stored(k, sh.kvdtype), synth.kv_stored(v, sh.kvdtype)
        gk, gv = sess.kv_slab(0, b)
        gk[:, :lens[b], :] = dev(kq.view(np.int16)).permute(1, 0, 2)
        gv[:, :lens[b], :] = dev(vq.view(np.int16)).permute(1, 0, 2)
        cache.k[0, b, :lens[b]] = synth.kv_widen(kq)
        cache.v[0, b, :lens[b]] = synth.kv_widen(vq)
    order = np.arange(Bn)[::-1].copy()          # rows name slabs in reverse order
    x = synth.step_rows(15, 0, Bn, sh.hidden)
    want = O.block(x, lens[order], order, ow, sh, cache, 0)
    xd = dev(x)
    sess.step(xd, dev(lens[order].astype(np.int32)), seq=dev(order.astype(np.int32)), pos_bound=int(lens.max()) + 1)
    torch.cuda.synchronize()
    e = check(xd.cpu().numpy(), want, False, f"batched step B={Bn}")
    assert sess.error_bits() == 0
    log(f"batched step B={Bn}: {e:.2e}")
    sess.close()


def test_qwen3_1p7b_block_t153_prefill_then_64_steps():
    wl = WORKLOADS["qwen3_1p7b_block_t153"]
    errs = run_block_case(wl.shape, wl.cfg_id, wl.prefill_rows, wl.steps, wl.n_ctx)
    log(f"1.7B block T=153: prefill {errs[0]:.2e}, steps max {max(errs[1:]):.2e}")


@pytest.mark.parametrize("n_rows", [3, 21])
def test_lm_head_argmax_planted_ties_nan_and_feedback(n_rows):
    """3 rows take the GEMV head; 21 rows the MFMA head (norm planes, a 16-row and a 5-row chunk).
    Planted: a tie (lowest index wins), a maximum at the last vocabulary row, a NaN
    embedding row (a NaN logit in every row, never chosen), and a row of x holding a
    NaN (every logit NaN: id 0, as the oracle's scan with NaN read as -inf)."""
    sh = replace(SMALL64, vocab=5000)
    rng = np.random.default_rng(3)
    E = synth.to_bf16_bits(rng.standard_normal((sh.vocab, sh.hidden)).astype(np.float32) * 0.02)
    g = synth.to_bf16_bits(np.ones(sh.hidden, np.float32))
    x = rng.standard_normal((n_rows, sh.hidden)).astype(np.float32)
    # row 0: rows 4321 and 17 of E both equal the row's direction -> tie, lowest index wins
    z = x[0] / np.sqrt(np.mean(x[0] ** 2) + 1e-6)
    E[4321] = synth.to_bf16_bits(z * 0.5)
    E[17] = E[4321]
    # row 1: a single planted maximum at the last vocabulary row
    z1 = x[1] / np.sqrt(np.mean(x[1] ** 2) + 1e-6)
    E[4999] = synth.to_bf16_bits(z1 * 0.5)
    # every row: vocabulary row 2500 is NaN, so is its logit
    nan_col = 2500
    E[nan_col] = 0x7FC0
    E[nan_col, 1:] = 0
    # the last row: a NaN activation makes every logit of that row NaN
    x[n_rows - 1, 7] = np.nan
    sess = DecoderSession(sh, [synth.block_weights(16, 0, sh)], embed=E, final_norm=g, n_ctx=16, max_rows=n_rows)
    xd = dev(x)
    ids = torch.zeros(n_rows, dtype=torch.int32, device="cuda")
    logits = torch.zeros(n_rows, sh.vocab, dtype=torch.float32, device="cuda")
    nx = torch.zeros(n_rows, sh.hidden, dtype=torch.float32, device="cuda")
    pos0 = np.arange(5, 5 + n_rows, dtype=np.int32)
    pos = dev(pos0)
    with np.errstate(invalid="ignore"):
        want_logits = O.final_logits(x, synth.widen(g), synth.widen(E), sh.rms_eps)
    finite_rows = n_rows - 1
    keep_cols = np.arange(sh.vocab) != nan_col
    for rep in range(3):        # slots and counters must re-arm themselves between calls
        sess.head(xd, ids, logits=logits, next_x=nx, pos=pos)
        torch.cuda.synchronize()
        got = ids.cpu().numpy()
        gl = logits.cpu().numpy()
        check(gl[:finite_rows][:, keep_cols], want_logits[:finite_rows][:, keep_cols], False, "logits")
        assert np.all(np.isnan(gl[:, nan_col])) and np.all(np.isnan(gl[n_rows - 1]))
        assert got[0] == 17, got
        assert got[1] == 4999, got
        assert got[n_rows - 1] == 0 == O.greedy_token(want_logits[n_rows - 1]), got
        assert nan_col not in got.tolist()
        for b in range(2, finite_rows):
            if O.top2_margin(want_logits[b]) > MARGIN:
                assert got[b] == O.greedy_token(want_logits[b]), b
            else:   # near-tie: the GPU's pick is one of the near-maximal logits
                assert want_logits[b][got[b]] >= np.nanmax(want_logits[b]) - MARGIN, b
        np.testing.assert_array_equal(nx.cpu().numpy(), synth.widen(E)[got])
        assert pos.cpu().numpy().tolist() == (pos0 + 1 + rep).tolist()
    sess.close()


@pytest.mark.parametrize("n_rows", [3, 13])
def test_lm_head_device_row_index(n_rows):
    """Head rows picked by a device index array (the per-sequence last-row gather
    of a packed prefill): equal to passing the gathered rows, for the GEMV (3) and
    the MFMA (13) head; an index outside the rows reads row 0 and is flagged."""
    sh = replace(SMALL64, vocab=3000)
    rng = np.random.default_rng(5)
    E = synth.to_bf16_bits(rng.standard_normal((sh.vocab, sh.hidden)).astype(np.float32) * 0.02)
    g = synth.to_bf16_bits(1 + 0.02 * rng.standard_normal(sh.hidden).astype(np.float32))
    n_x = 40
    x = rng.standard_normal((n_x, sh.hidden)).astype(np.float32)
    rows = rng.choice(n_x, n_rows, replace=False).astype(np.int32)
    sess = DecoderSession(sh, [synth.block_weights(21, 0, sh)], embed=E, final_norm=g, n_ctx=16, max_rows=n_x)
    xd = dev(x)
    ids = torch.zeros(n_rows, dtype=torch.int32, device="cuda")
    logits = torch.zeros(n_rows, sh.vocab, device="cuda")
    sess.head(xd, ids, logits=logits, x_rows=dev(rows))
    ids2 = torch.zeros(n_rows, dtype=torch.int32, device="cuda")
    logits2 = torch.zeros(n_rows, sh.vocab, device="cuda")
    sess.head(dev(x[rows]), ids2, logits=logits2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), ids2.cpu().numpy())
    np.testing.assert_array_equal(logits.cpu().numpy(), logits2.cpu().numpy())
    want = O.final_logits(x[rows], synth.widen(g), synth.widen(E), sh.rms_eps)
    check(logits.cpu().numpy(), want, False, "indexed-row logits")
    assert sess.error_bits() == 0
    bad = rows.copy()
    bad[1] = n_x
    sess.head(xd, ids, logits=logits, x_rows=dev(bad))
    torch.cuda.synchronize()
    assert sess.error_bits() == B.DEVERR_ROW
    clamped = rows.copy()
    clamped[1] = 0                    # what the flagged row reads instead
    sess.head(dev(x[clamped]), ids2, logits=logits2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(logits.cpu().numpy(), logits2.cpu().numpy())
    sess.close()


def test_embed_gather_and_bad_token_ids_are_flagged():
    sh = replace(SMALL64, vocab=100)
    E = synth.to_bf16_bits(np.arange(100 * sh.hidden, dtype=np.float32).reshape(100, sh.hidden) % 251)
    sess = DecoderSession(sh, [synth.block_weights(17, 0, sh)], embed=E,
                          final_norm=synth.to_bf16_bits(np.ones(sh.hidden, np.float32)), n_ctx=16, max_rows=4)
    ids = dev(np.array([3, 99, 0, 100], np.int32))
    x = torch.full((4, sh.hidden), 7.0, device="cuda")
    sess.gather(ids, x)
    torch.cuda.synchronize()
    got = x.cpu().numpy()
    np.testing.assert_array_equal(got[:3], synth.widen(E)[[3, 99, 0]])
    assert np.all(got[3] == 0)
    assert sess.error_bits() == B.DEVERR_TOKEN
    assert sess.error_bits() == 0
    sess.close()


def test_out_of_range_device_positions_are_flagged_not_faulting():
    sh = SMALL64
    sess = DecoderSession(sh, [synth.block_weights(18, 0, sh)], n_ctx=32, n_seq=2, max_rows=2)
    x = torch.zeros(2, sh.hidden, device="cuda")
    sess.step(x, dev(np.array([40, 3], np.int32)), pos_bound=32)    # 40 >= n_ctx
    torch.cuda.synchronize()
    assert sess.error_bits() & B.DEVERR_POSITION
    sess.step(x, dev(np.array([1, 3], np.int32)), seq=dev(np.array([0, 5], np.int32)), pos_bound=32)
    torch.cuda.synchronize()
    assert sess.error_bits() & B.DEVERR_SLAB
    sess.close()


def test_host_validation_errors():
    sh = SMALL64
    sess = DecoderSession(sh, [synth.block_weights(19, 0, sh)], n_ctx=32, max_rows=8)
    x = torch.zeros(8, sh.hidden, device="cuda")
    with pytest.raises(B.SttdError) as e:
        sess.prefill(x[:8], pos0=30)                  # 30 + 8 > n_ctx
    assert e.value.status == B.ERR_CONTEXT_FULL
    with pytest.raises(B.SttdError) as e:
        B.block_prefill(sess.params, sess.layer_weights[0], sess.ws, sess.kv, 1, 0, 0, 4, x.data_ptr())  # layer 1
    assert e.value.status == B.ERR_INVALID_ARG
    with pytest.raises(B.SttdError) as e:
        B.block_prefill(sess.params, sess.layer_weights[0], sess.ws, sess.kv, 0, 0, 0, 9, x.data_ptr())  # > max_rows
    assert e.value.status == B.ERR_INVALID_ARG
    bad = B.block_params(sh.hidden, sh.n_heads, sh.n_kv_heads, 96, sh.ffn, 1e-6, 1e6, B.BF16)
    with pytest.raises(B.SttdError) as e:
        B.workspace_alloc(bad, 4, 32, 0)
    assert e.value.status == B.ERR_UNSUPPORTED
    with pytest.raises(B.SttdError) as e:
        B.kv_cache_alloc(1 << 20, 1 << 10, 1 << 20, 8, 128, B.F16)
    assert e.value.status == B.ERR_OOM
    sess.close()


def test_kv_cache_clear_zeroes_every_slab():
    sh = SMALL64
    sess = DecoderSession(sh, [synth.block_weights(20, 0, sh)], n_ctx=32, n_seq=2, max_rows=8)
    x = dev(synth.prefill_rows(20, 8, sh.hidden))
    sess.prefill(x, seq=1)
    k, v = sess.kv_slab(0, 1)
    torch.cuda.synchronize()
    assert torch.count_nonzero(k) > 0
    B.kv_cache_clear(sess.kv)
    torch.cuda.synchronize()
    assert torch.count_nonzero(k) == 0 and torch.count_nonzero(v) == 0
    sess.close()


def test_step_loop_graph_replay_matches_eager():
    """A greedy loop of (blocks, head with next-row feedback and position bump)
    captured once into a HIP graph and replayed gives the eager loop's ids."""
    sh = replace(SMALL64, n_layers=2, vocab=3000)
    layers = [synth.block_weights(21, l, sh) for l in range(2)]
    E = synth.embedding(21, sh)
    g = synth.final_norm(21, sh)
    T, steps = 12, 6
    x0 = synth.prefill_rows(21, T, sh.hidden)

    def run(use_graph):
        sess = DecoderSession(sh, layers, embed=E, final_norm=g, n_ctx=64, max_rows=T)
        x = dev(x0)
        sess.prefill(x, slice_last=True)
        ids = torch.zeros(1, dtype=torch.int32, device="cuda")
        pos = torch.full((1,), T, dtype=torch.int32, device="cuda")
        xs = torch.zeros(1, sh.hidden, device="cuda")
        sess.head(x[T - 1:], ids, next_x=xs)
        out = [int(ids.item())]
        if use_graph:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.stream(s):
                with torch.cuda.graph(graph, stream=s):
                    sess.step(xs, pos, pos_bound=64)
                    sess.head(xs, ids, next_x=xs, pos=pos)
            torch.cuda.current_stream().wait_stream(s)
            for _ in range(steps):
                graph.replay()
                torch.cuda.synchronize()
                out.append(int(ids.item()))
        else:
            for _ in range(steps):
                sess.step(xs, pos, pos_bound=64)
                sess.head(xs, ids, next_x=xs, pos=pos)
                torch.cuda.synchronize()
                out.append(int(ids.item()))
        assert int(pos.item()) == T + steps
        sess.close()
        return out

    eager = run(False)
    graphed = run(True)
    log(f"eager {eager} graph {graphed}")
    assert eager == graphed
