"""Pins of the CPU oracle to facts outside itself (closed forms, library special
cases, brute force, invariants of the method, the pages' one printed figure).

Each test is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, a swapped gate/up, an interleaved
GQA grouping, V normed or rotated) fails at least one of them.
"""
import math
import os
from types import SimpleNamespace

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import decoder as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def params(nq, nkv, d, ffn, eps=1e-6, theta=1e6):
    return SimpleNamespace(n_heads=nq, n_kv_heads=nkv, head_dim=d, ffn=ffn, rms_eps=eps, rope_theta=theta)


def rand_block(rng, H, nq, nkv, d, I, scale=0.2):
    return {
        "attn_norm": 1 + 0.1 * rng.standard_normal(H),
        "wq": scale * rng.standard_normal((nq * d, H)),
        "wk": scale * rng.standard_normal((nkv * d, H)),
        "wv": scale * rng.standard_normal((nkv * d, H)),
        "q_norm": 1 + 0.1 * rng.standard_normal(d),
        "k_norm": 1 + 0.1 * rng.standard_normal(d),
        "wo": scale * rng.standard_normal((H, nq * d)),
        "ffn_norm": 1 + 0.1 * rng.standard_normal(H),
        "w_gate_up": scale * rng.standard_normal((2 * I, H)),
        "w_down": scale * rng.standard_normal((H, I)),
    }


# ------------------------------------------------------------------ RMSNorm

def test_rmsnorm_matches_torch_rms_norm():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64)) * np.array([1e-3, 1, 10, 100, 0.5])[:, None]
    g = 1 + 0.1 * rng.standard_normal(64)
    ref = F.rms_norm(torch.tensor(x), (64,), torch.tensor(g), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rms_norm(x, g, 1e-6), ref, rtol=1e-13, atol=0)


def test_rmsnorm_unit_rms_before_gain():
    # with gain 1 the output's RMS is sqrt(ms / (ms + eps)): ~1, and visibly below 1 when ms ~ eps
    rng = np.random.default_rng(2)
    for scale in [1.0, 3e-3, 1e-3]:
        x = scale * rng.standard_normal(256)
        ms = np.mean(x * x)
        y = O.rms_norm(x, np.ones(256), 1e-6)
        assert math.isclose(np.sqrt(np.mean(y * y)), math.sqrt(ms / (ms + 1e-6)), rel_tol=1e-12)


# ------------------------------------------------------------------ RoPE

def test_rope_identity_at_position_zero():
    rng = np.random.default_rng(3)
    u = rng.standard_normal((1, 3, 64))
    assert np.array_equal(O.rope_neox(u, np.array([0]), 1e6), u)


def test_rope_neox_closed_form_d4():
    # d = 4, theta = 1e6: omega = (1, 1e-3); NeoX pairs are (0, 2) and (1, 3)
    u = np.array([[[0.3, -1.2, 0.7, 2.0]]])
    p = 3
    a0, a1 = p * 1.0, p * 1e-3
    want = [0.3 * math.cos(a0) - 0.7 * math.sin(a0),
            -1.2 * math.cos(a1) - 2.0 * math.sin(a1),
            0.3 * math.sin(a0) + 0.7 * math.cos(a0),
            -1.2 * math.sin(a1) + 2.0 * math.cos(a1)]
    np.testing.assert_allclose(O.rope_neox(u, np.array([p]), 1e6)[0, 0], want, rtol=0, atol=1e-15)


def test_rope_frequencies_and_isometry():
    rng = np.random.default_rng(4)
    d = 128
    u = rng.standard_normal((1, 1, d))
    p = 1000
    r = O.rope_neox(u, np.array([p]), 1e6)[0, 0]
    half = d // 2
    # each pair keeps its length
    np.testing.assert_allclose(u[0, 0, :half] ** 2 + u[0, 0, half:] ** 2, r[:half] ** 2 + r[half:] ** 2, rtol=1e-12)
    # the turned angle of pair i is p * theta^(-2i/d), mod 2 pi
    for i in [0, 1, 17, half - 1]:
        z0 = complex(u[0, 0, i], u[0, 0, i + half])
        z1 = complex(r[i], r[i + half])
        ang = math.atan2((z1 / z0).imag, (z1 / z0).real)
        want = math.remainder(p * 1e6 ** (-2 * i / d), 2 * math.pi)
        assert abs(math.remainder(ang - want, 2 * math.pi)) < 1e-9


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    dot = lambda m, n: float(np.sum(O.rope_neox(q, np.array([m]), 1e6) * O.rope_neox(k, np.array([n]), 1e6)))
    for m, n, s in [(5, 2, 7), (100, 0, 31), (3000, 2999, 1000)]:
        assert math.isclose(dot(m, n), dot(m + s, n + s), rel_tol=1e-9, abs_tol=1e-10)
    assert not math.isclose(dot(5, 2), dot(5, 3), rel_tol=1e-6)


# ------------------------------------------------------------------ SiLU / softmax

def test_silu_matches_torch():
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(O.silu(z), F.silu(torch.tensor(z)).numpy(), rtol=1e-14, atol=1e-300)


def test_softmax_brute_force():
    rng = np.random.default_rng(6)
    s = rng.standard_normal(7) * 5
    e = [math.exp(v) for v in s]
    tot = math.fsum(e)
    np.testing.assert_allclose(O.softmax(s), [v / tot for v in e], rtol=1e-14)
    big = np.array([1000.0, 999.0, -1000.0])            # needs the max subtraction
    np.testing.assert_allclose(O.softmax(big), [1 / (1 + math.exp(-1)), math.exp(-1) / (1 + math.exp(-1)), 0.0],
                               rtol=1e-14, atol=1e-300)


# ------------------------------------------------------------------ attention

def _causal_rows(q, K, V):
    """q [T, nq, d], K/V [T, nkv, d]: oracle row attention with row t seeing keys 0..t."""
    return np.stack([O.gqa_attention_row(q[t], K, V, t + 1) for t in range(q.shape[0])])


def test_attention_gqa_matches_torch_sdpa():
    rng = np.random.default_rng(7)
    T, nq, nkv, d = 9, 8, 2, 16
    q, K, V = rng.standard_normal((T, nq, d)), rng.standard_normal((T, nkv, d)), rng.standard_normal((T, nkv, d))
    ours = _causal_rows(q, K, V)
    tq, tk, tv = (torch.tensor(a).permute(1, 0, 2)[None] for a in (q, K, V))
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, enable_gqa=True)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-13)


def test_attention_mha_special_case():
    # n_kv_heads == n_heads: plain multi-head causal attention
    rng = np.random.default_rng(8)
    T, nh, d = 6, 4, 8
    q, K, V = rng.standard_normal((T, nh, d)), rng.standard_normal((T, nh, d)), rng.standard_normal((T, nh, d))
    ours = _causal_rows(q, K, V)
    ref = np.empty_like(ours)
    for h in range(nh):
        s = q[:, h] @ K[:, h].T / math.sqrt(d)
        s[np.triu_indices(T, 1)] = -np.inf
        p = np.exp(s - s.max(1, keepdims=True))
        ref[:, h] = (p / p.sum(1, keepdims=True)) @ V[:, h]
    np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-13)


def test_attention_brute_force_tiny_shapes():
    rng = np.random.default_rng(9)
    for d, n_keys in [(2, 1), (2, 3), (4, 4), (3, 2)]:
        q = rng.standard_normal((2, d))
        K = rng.standard_normal((n_keys, 1, d))
        V = rng.standard_normal((n_keys, 1, d))
        got = O.gqa_attention_row(q, K, V, n_keys)
        for h in range(2):
            s = [math.fsum(q[h, i] * K[c, 0, i] for i in range(d)) / math.sqrt(d) for c in range(n_keys)]
            w = [math.exp(v) for v in s]
            tot = math.fsum(w)
            want = [math.fsum(w[c] / tot * V[c, 0, i] for c in range(n_keys)) for i in range(d)]
            np.testing.assert_allclose(got[h], want, rtol=1e-13, atol=1e-15)


def test_attention_single_key_returns_v0():
    rng = np.random.default_rng(10)
    q = rng.standard_normal((4, 8)) * 50
    K = rng.standard_normal((3, 2, 8))
    V = rng.standard_normal((3, 2, 8))
    out = O.gqa_attention_row(q, K, V, 1)
    assert np.array_equal(out, V[0, [0, 0, 1, 1]])


def test_attention_equal_keys_average_values_over_causal_extent():
    rng = np.random.default_rng(11)
    K = np.tile(rng.standard_normal((1, 2, 8)), (6, 1, 1))
    V = rng.standard_normal((6, 2, 8))
    q = rng.standard_normal((4, 8))
    for n_keys in [1, 3, 6]:
        out = O.gqa_attention_row(q, K, V, n_keys)
        np.testing.assert_allclose(out, V[:n_keys].mean(0)[[0, 0, 1, 1]], rtol=1e-13)


# ------------------------------------------------------------------ block wiring

def test_block_is_identity_when_output_projections_are_zero():
    rng = np.random.default_rng(12)
    p = params(4, 2, 8, 48)
    w = rand_block(rng, 32, 4, 2, 8, 48)
    w["wo"][:] = 0
    w["w_down"][:] = 0
    x = rng.standard_normal((5, 32))
    cache = O.KVCache(1, 1, 8, 2, 8)
    assert np.array_equal(O.block(x, np.arange(5), np.zeros(5, int), w, p, cache, 0), x)


def test_block_closed_form_value_path_grouping_and_ffn():
    # H = 8, 4 query heads over 2 KV heads of d = 4, one row at position 0:
    # a single key makes each head's output its KV head's v (unnormed, unrotated);
    # Wv = I gives v = xn. Wo picks query head 1 into the first half of the
    # output and query head 2 into the second half; with contiguous groups
    # (head h reads KV head h // 2) that is [v_0 | v_1] = xn, so h = x + xn.
    # FFN with ffn = 8: W_gate = a I, W_up = b I, W_down = I gives
    # out = h + silu(a hn) * (b hn), hn = RMSNorm(h) * g_ffn.
    rng = np.random.default_rng(13)
    H, nq, nkv, d, I = 8, 4, 2, 4, 8
    a, b = 1.7, -0.6
    w = rand_block(rng, H, nq, nkv, d, I)
    w["wv"] = np.eye(8)
    wo = np.zeros((8, 16))
    wo[0:4, 4:8] = np.eye(4)      # query head 1 -> output 0..3
    wo[4:8, 8:12] = np.eye(4)     # query head 2 -> output 4..7
    w["wo"] = wo
    w["w_gate_up"] = np.concatenate([a * np.eye(8), b * np.eye(8)])
    w["w_down"] = np.eye(8)
    p = params(nq, nkv, d, I)
    x = rng.standard_normal((1, 8)) * 2
    out = O.block(x, np.array([0]), np.array([0]), w, p, O.KVCache(1, 1, 4, nkv, d), 0)
    ms = np.mean(x * x)
    xn = x / np.sqrt(ms + 1e-6) * w["attn_norm"]
    h = x + xn
    hn = h / np.sqrt(np.mean(h * h) + 1e-6) * w["ffn_norm"]
    want = h + (a * hn / (1 + np.exp(-a * hn))) * (b * hn)
    np.testing.assert_allclose(out, want, rtol=1e-13)


def _small():
    H, nq, nkv, d, I = 32, 4, 2, 8, 48
    return params(nq, nkv, d, I), H


def test_causal_prefill_last_row_equals_stepwise_decode():
    rng = np.random.default_rng(14)
    p, H = _small()
    layers = [rand_block(rng, H, 4, 2, 8, 48) for _ in range(2)]
    x = rng.standard_normal((10, H))
    c1 = O.KVCache(2, 1, 16, 2, 8)
    full = O.prefill_stack(x, layers, p, c1)
    c2 = O.KVCache(2, 1, 16, 2, 8)
    part = O.prefill_stack(x[:7], layers, p, c2)
    np.testing.assert_allclose(part, full[:7], rtol=1e-12, atol=1e-12)
    for t in range(7, 10):
        row = O.step_stack(x[t:t + 1], [t], [0], layers, p, c2)
        np.testing.assert_allclose(row[0], full[t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(c2.k, c1.k, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(c2.v, c1.v, rtol=1e-12, atol=1e-13)


def test_prefill_prefix_invariance():
    rng = np.random.default_rng(15)
    p, H = _small()
    layers = [rand_block(rng, H, 4, 2, 8, 48)]
    x = rng.standard_normal((8, H))
    full = O.prefill_stack(x, layers, p, O.KVCache(1, 1, 8, 2, 8))
    for t in [0, 3, 6]:
        pre = O.prefill_stack(x[:t + 1], layers, p, O.KVCache(1, 1, 8, 2, 8))
        np.testing.assert_allclose(pre, full[:t + 1], rtol=1e-12, atol=1e-12)


def test_slice_last_gives_same_last_row():
    rng = np.random.default_rng(16)
    p, H = _small()
    layers = [rand_block(rng, H, 4, 2, 8, 48) for _ in range(3)]
    x = rng.standard_normal((6, H))
    full = O.prefill_stack(x, layers, p, O.KVCache(3, 1, 8, 2, 8))
    sl = O.prefill_stack(x, layers, p, O.KVCache(3, 1, 8, 2, 8), slice_last=True)
    assert sl.shape == (1, H)
    np.testing.assert_allclose(sl[0], full[-1], rtol=1e-13, atol=1e-13)


def test_rows_subset_matches_full_prefill():
    rng = np.random.default_rng(17)
    p, H = _small()
    w = rand_block(rng, H, 4, 2, 8, 48)
    x = rng.standard_normal((12, H))
    full = O.block(x, 5 + np.arange(12), np.zeros(12, int), w, p, O.KVCache(1, 1, 20, 2, 8), 0)
    c = O.KVCache(1, 1, 20, 2, 8)
    sub = O.block_rows_subset(x, 5, w, p, c, 0, [0, 4, 11])
    np.testing.assert_allclose(sub, full[[0, 4, 11]], rtol=1e-12, atol=1e-12)


def test_batched_step_equals_independent_steps():
    rng = np.random.default_rng(18)
    p, H = _small()
    layers = [rand_block(rng, H, 4, 2, 8, 48) for _ in range(2)]
    lens = [3, 9, 5]
    caches = []
    bc = O.KVCache(2, 3, 16, 2, 8)
    for s, L in enumerate(lens):
        pre = rng.standard_normal((L, H))
        c = O.KVCache(2, 1, 16, 2, 8)
        O.prefill_stack(pre, layers, p, c)
        bc.k[:, s], bc.v[:, s] = c.k[:, 0], c.v[:, 0]
        caches.append(c)
    xs = rng.standard_normal((3, H))
    batched = O.step_stack(xs, lens, [0, 1, 2], layers, p, bc)
    for s, L in enumerate(lens):
        single = O.step_stack(xs[s:s + 1], [L], [0], layers, p, caches[s])
        np.testing.assert_allclose(batched[s], single[0], rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ head / argmax

def test_argmax_planted_ties_nan_and_monotone():
    rng = np.random.default_rng(19)
    l = rng.standard_normal(1000)
    l[417] = 9.0
    assert O.greedy_token(l) == 417
    l[12] = 9.0
    l[900] = 9.0
    assert O.greedy_token(l) == 12                     # lowest index among equal maxima
    l[3] = np.nan
    assert O.greedy_token(l) == 12                     # NaN never wins
    l2 = rng.standard_normal(5000)
    assert O.greedy_token(l2) == int(np.argmax(O.softmax(l2)))   # softmax is monotone
    # the decision is made on fp32-rounded logits: values equal in fp32 tie
    l3 = np.array([1.0, 1.0 + 1e-12, 0.5])
    assert O.greedy_token(l3) == 0


def test_top2_margin_closed_forms():
    """The margin that gates every greedy-id check: largest minus second largest,
    whatever the order of the row, with ties at the top giving 0 and NaN counted
    as -inf (the same rule as the argmax)."""
    assert O.top2_margin([3.0, 1.0, 2.0]) == 1.0                    # unsorted
    assert O.top2_margin([-5.0, -2.0, -7.0]) == 3.0                 # all negative
    assert O.top2_margin([1.0, 4.0, 4.0, 0.0]) == 0.0               # tie at the top
    assert O.top2_margin([0.5, 4.0, 2.5, 4.0 - 2 ** -20]) == 2 ** -20
    assert O.top2_margin([np.nan, 2.0, 1.0]) == 1.0                 # NaN never counts as the top
    assert O.top2_margin([2.0, np.nan, 5.0, -1.0]) == 3.0
    assert O.top2_margin([np.nan, 7.0, np.nan]) == np.inf           # one finite value
    rng = np.random.default_rng(11)
    row = rng.standard_normal(151936)
    row[90000] = 9.0
    row[123] = 8.75
    assert O.top2_margin(row) == 0.25
    assert O.top2_margin(row[::-1]) == 0.25


def test_final_logits_tied_head_closed_form():
    rng = np.random.default_rng(20)
    E = rng.standard_normal((50, 16))
    g = 1 + 0.1 * rng.standard_normal(16)
    x = rng.standard_normal((2, 16))
    z = x / np.sqrt(np.mean(x * x, 1, keepdims=True) + 1e-6) * g
    np.testing.assert_allclose(O.final_logits(x, g, E, 1e-6), z @ E.T, rtol=1e-13)
    # a row of E equal to the normalised input direction wins
    E[31] = 10 * z[0] / np.linalg.norm(z[0])
    assert O.greedy_token(O.final_logits(x[:1], g, E, 1e-6)[0]) == 31


def test_greedy_generate_equals_prefill_of_whole_sequence():
    # step k at position T + k - 1 with input E[token] gives the same last-row
    # logits as a prefill over the prompt followed by the fed rows
    rng = np.random.default_rng(21)
    p, H = _small()
    layers = [rand_block(rng, H, 4, 2, 8, 48) for _ in range(2)]
    E = rng.standard_normal((40, H))
    g = 1 + 0.1 * rng.standard_normal(H)
    x = rng.standard_normal((5, H))
    r = O.greedy_generate(x, layers, p, E, g, n_new=4, n_ctx=16)
    seq = np.concatenate([x, E[r["tokens"][:3]]])
    full = O.prefill_stack(seq, layers, p, O.KVCache(2, 1, 16, 2, 8))
    logits = O.final_logits(full[4:], g, E, 1e-6)
    np.testing.assert_allclose(r["logits"], logits, rtol=1e-11, atol=1e-11)
    assert r["tokens"] == [O.greedy_token(l) for l in logits]


def test_kv_bytes_per_token_matches_pages_figure():
    vals = {}
    with open(os.path.join(GOLDEN, "kv_bytes_per_token.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if line:
                vals[line[0]] = int(line[1])
    assert vals["bytes"] == 14 * 2 ** 30
    c = O.KVCache(vals["n_layers"], 1, 1, vals["n_kv_heads"], vals["head_dim"])
    assert c.bytes_per_token(vals["elem_bytes"]) * vals["tokens"] == vals["bytes"]
    assert c.bytes_per_token(2) == 114688


def test_injection_blend_equals_the_three_way_concat():
    """The pages give the audio injection in two forms: the single-sequence
    prefill graph concatenates prefix embeddings, the encoder rows and suffix
    embeddings (Qwen3-ASR decoder page, build_prefill_graph); the batched
    graphs blend embed[ids] * keep + audio_dense. With one contiguous audio
    block they must agree, and with no audio the blend is the plain gather."""
    rng = np.random.default_rng(7)
    V, H, pre, n_audio, suf = 50, 16, 5, 7, 3
    T = pre + n_audio + suf
    E = rng.standard_normal((V, H))
    ids = rng.integers(0, V, T)
    audio = rng.standard_normal((n_audio, H))
    keep = np.ones(T)
    keep[pre:pre + n_audio] = 0.0
    dense = np.zeros((T, H))
    dense[pre:pre + n_audio] = audio
    concat = np.concatenate([E[ids[:pre]], audio, E[ids[pre + n_audio:]]], axis=0)
    assert np.array_equal(O.inject(E, ids, keep, dense), concat)
    assert np.array_equal(O.inject(E, ids, np.ones(T), np.zeros((T, H))), E[ids])
    # non-contiguous audio positions (MOSS): rows land where keep is 0
    pos = np.array([1, 4, 9])
    keep2 = np.ones(T)
    keep2[pos] = 0.0
    dense2 = np.zeros((T, H))
    dense2[pos] = audio[:3]
    out = O.inject(E, ids, keep2, dense2)
    assert np.array_equal(out[pos], audio[:3])
    rest = np.setdiff1d(np.arange(T), pos)
    assert np.array_equal(out[rest], E[ids[rest]])


def test_greedy_loop_stopping_rules_closed_forms():
    """The step loop's three exits (run() on the Qwen3-ASR model page): EOS,
    the token budget, the end of the context; truncated unless EOS."""
    seq = lambda pos, tok: 100 + pos          # a token per input position
    assert O.greedy_loop(7, seq, 10, 7, 50, 64) == ([7], False)              # the prefill's token is EOS
    toks, tr = O.greedy_loop(1, seq, 10, 999, 5, 64)                          # budget: 5 tokens in all
    assert toks == [1, 110, 111, 112, 113] and tr
    toks, tr = O.greedy_loop(1, seq, 60, 999, 50, 64)                         # context: steps at 60..63
    assert toks == [1, 160, 161, 162, 163] and tr
    toks, tr = O.greedy_loop(1, seq, 10, 113, 50, 64)                         # EOS produced at position 13
    assert toks == [1, 110, 111, 112, 113] and not tr
    assert O.greedy_loop(1, seq, 64, 999, 50, 64) == ([1], True)            # context already full
    assert O.greedy_loop(1, seq, 10, 999, 1, 64) == ([1], True)             # budget of one token
