"""CPU oracle for the Qwen3-style decoder block: plain fp64 numpy, slow and obvious.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import or call this module. The HIP path
never does, and this module imports nothing from it.

What the block computes comes from the transcribe.cpp pages:
  * Qwen3-ASR decoder page (transcribe-cpp-sys 0.2.0,
    src/arch/qwen3_asr/decoder.cpp), file header: the shared causal-LM
    block is pre-LN RMSNorm, grouped-query attention with a per-head
    RMSNorm on Q and K, NeoX rotary embedding at theta = 1e6, a KV-cache
    write then read, and SwiGLU on one packed gate_up projection.
  * same page, to_block_view / to_block_params: the ten weight slots
    (no biases) and the parameters n_heads, n_kv_heads, head_dim,
    rms_eps, rope_theta.
  * same page, build_prefill_graph: the layer stack, the final RMSNorm
    followed by the tied lm_head (the token-embedding table), and the
    last-row slice; build_step_graph: the next step's input is the
    embedding row of the chosen token, and argmax runs on the logits.
  * Qwen3-ASR model page (transcribe-cpp-sys 0.2.0,
    src/arch/qwen3_asr/model.cpp), run(): prefill positions are 0..T-1,
    the causal mask lets row r see columns c <= r, the first new token is
    the argmax of the prefill's last row, each step writes the cache at
    index = position, and the host argmax keeps the lowest index on ties.

Where the pages leave a detail open, the plainest reading is taken (each
one is listed in the repository's design notes):
  RMSNorm: x / sqrt(mean(x^2) + eps) * gain, eps inside the root.
  Q/K norm: one gain vector of length head_dim shared by all heads; norm,
    then RoPE, then the cache write; V is neither normed nor rotated.
  NeoX RoPE: pairs (i, i + d/2) over the whole head, omega_i = theta^(-2i/d).
  Positions are 1-D (the multimodal rotary reduces to one index stream).
  Attention: scale 1/sqrt(head_dim); query head h reads KV head
    floor(h / (n_heads / n_kv_heads)); no bias, soft-cap or window.
  gate_up is [2*ffn, hidden] with the gate rows first; SiLU on the gate.
  Argmax is taken on fp32-rounded logits (the precision of the logits
    tensor); NaN is never chosen; ties go to the lowest index.

Everything is fp64: weights arrive as fp32 (bf16 values widen exactly),
activations and the KV cache stay fp64.
"""
import numpy as np


def f64(a):
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------- primitives

def rms_norm(x, gain, eps):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * gain."""
    x = f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * f64(gain)


def rope_neox(u, positions, theta):
    """NeoX rotary embedding of head vectors u[rows, heads, d] at positions[rows].

    For i < d/2 the pair (u[i], u[i + d/2]) turns by the angle p * theta^(-2i/d)."""
    u = f64(u)
    d = u.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    omega = np.power(float(theta), -2.0 * i / d)
    ang = f64(positions)[:, None] * omega[None, :]          # [rows, d/2]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a, b = u[..., :half], u[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def silu(z):
    z = f64(z)
    return z / (1.0 + np.exp(-z))


def softmax(s):
    """Two-pass softmax over the last axis (max subtracted, then normalised)."""
    s = f64(s)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def gqa_attention_row(q, K, V, n_keys):
    """One query row against the first n_keys cache rows.

    q: [n_heads, d]; K, V: [>= n_keys, n_kv_heads, d]. Returns [n_heads, d]."""
    q = f64(q)
    n_heads, d = q.shape
    n_kv = K.shape[1]
    group = n_heads // n_kv
    out = np.empty((n_heads, d), dtype=np.float64)
    for h in range(n_heads):
        j = h // group
        s = (K[:n_keys, j, :] @ q[h]) / np.sqrt(d)           # [n_keys]
        out[h] = softmax(s) @ V[:n_keys, j, :]
    return out


# ---------------------------------------------------------------- KV cache

class KVCache:
    """fp64 K and V per layer and sequence slab: [n_layers, n_seq, n_ctx, n_kv_heads, d].

    The row index of a token is its position."""

    def __init__(self, n_layers, n_seq, n_ctx, n_kv_heads, head_dim):
        shape = (n_layers, n_seq, n_ctx, n_kv_heads, head_dim)
        self.k = np.zeros(shape, dtype=np.float64)
        self.v = np.zeros(shape, dtype=np.float64)
        self.n_ctx = n_ctx

    def bytes_per_token(self, elem_bytes):
        """KV bytes one token occupies over all layers: n_kv_heads * d * n_layers * 2 elements."""
        n_layers, _, _, n_kv, d = self.k.shape
        return n_kv * d * n_layers * 2 * elem_bytes


# ---------------------------------------------------------------- one block

def block(x, positions, seqs, w, p, cache, layer, ffn_rows=None):
    """One decoder block over rows x[R, hidden] at positions[R] of slabs seqs[R].

    w: dict of the ten weight slots as float arrays (w_gate_up packed, gate rows first).
    p: object with n_heads, n_kv_heads, head_dim, ffn, rms_eps, rope_theta.
    Every row's K and V are written to the cache first; row r then attends
    cache rows [0, positions[r]] of its slab, so rows of one sequence given
    in position order see exactly their causal prefix.
    ffn_rows: None for all rows, else the row indices that run the FFN
    (the last-row slice); the result then holds only those rows.
    Returns the block output rows (fp64)."""
    x = f64(x)
    R = x.shape[0]
    nq, nkv, d, eps = p.n_heads, p.n_kv_heads, p.head_dim, p.rms_eps
    positions = np.asarray(positions, dtype=np.int64)
    seqs = np.asarray(seqs, dtype=np.int64)

    # pre-attention RMSNorm and the three projections (no bias)
    xn = rms_norm(x, w["attn_norm"], eps)
    q = (xn @ f64(w["wq"]).T).reshape(R, nq, d)
    k = (xn @ f64(w["wk"]).T).reshape(R, nkv, d)
    v = (xn @ f64(w["wv"]).T).reshape(R, nkv, d)

    # per-head Q/K RMSNorm, then NeoX RoPE; V untouched
    q = rope_neox(rms_norm(q, w["q_norm"], eps), positions, p.rope_theta)
    k = rope_neox(rms_norm(k, w["k_norm"], eps), positions, p.rope_theta)

    # KV-cache write at index = position
    for r in range(R):
        cache.k[layer, seqs[r], positions[r]] = k[r]
        cache.v[layer, seqs[r], positions[r]] = v[r]

    # causal GQA attention of each row over its slab's rows [0, pos]
    o = np.empty((R, nq * d), dtype=np.float64)
    for r in range(R):
        o[r] = gqa_attention_row(q[r], cache.k[layer, seqs[r]], cache.v[layer, seqs[r]],
                                 positions[r] + 1).reshape(-1)

    # output projection + residual
    h = x + o @ f64(w["wo"]).T

    # FFN: RMSNorm, packed gate_up, SwiGLU, down projection + residual
    rows = np.arange(R) if ffn_rows is None else np.asarray(ffn_rows)
    hs = h[rows]
    hn = rms_norm(hs, w["ffn_norm"], eps)
    gu = hn @ f64(w["w_gate_up"]).T
    gate, up = gu[:, :p.ffn], gu[:, p.ffn:]
    return hs + (silu(gate) * up) @ f64(w["w_down"]).T


def block_rows_subset(x, pos0, w, p, cache, layer, sample_rows):
    """A causal prefill of x[T, hidden] at positions pos0.. of slab 0, with the
    attention, O projection and FFN evaluated only on sample_rows.

    K and V depend on a row alone, so they are computed for every row and all
    written; a sampled row's output needs nothing else. Returns the sampled
    rows' block outputs."""
    x = f64(x)
    T = x.shape[0]
    nq, nkv, d, eps = p.n_heads, p.n_kv_heads, p.head_dim, p.rms_eps
    positions = pos0 + np.arange(T)
    xn = rms_norm(x, w["attn_norm"], eps)
    k = rope_neox(rms_norm((xn @ f64(w["wk"]).T).reshape(T, nkv, d), w["k_norm"], eps), positions, p.rope_theta)
    v = (xn @ f64(w["wv"]).T).reshape(T, nkv, d)
    cache.k[layer, 0, positions] = k
    cache.v[layer, 0, positions] = v
    sample_rows = np.asarray(sample_rows)
    xs = x[sample_rows]
    ps = positions[sample_rows]
    qs = rope_neox(rms_norm((xn[sample_rows] @ f64(w["wq"]).T).reshape(len(sample_rows), nq, d), w["q_norm"], eps),
                   ps, p.rope_theta)
    o = np.stack([gqa_attention_row(qs[i], cache.k[layer, 0], cache.v[layer, 0], ps[i] + 1).reshape(-1)
                  for i in range(len(sample_rows))])
    h = xs + o @ f64(w["wo"]).T
    hn = rms_norm(h, w["ffn_norm"], eps)
    gu = hn @ f64(w["w_gate_up"]).T
    return h + (silu(gu[:, :p.ffn]) * gu[:, p.ffn:]) @ f64(w["w_down"]).T


# ---------------------------------------------------------------- head

def inject(embed, ids, keep, audio_dense):
    """Prompt/audio injection ahead of the first block. The batched prefill
    graph on the Qwen3-ASR model page (build_prefill_graph_batched) and the
    MOSS page (build_injection, prefill_chunked) blend the token embeddings
    with the encoder rows: x = embed[ids] * keep + audio_dense. keep is 0 at
    the audio positions and 1 elsewhere, and audio_dense holds the encoder
    rows at the audio positions and zeros elsewhere."""
    rows = f64(embed)[np.asarray(ids)]
    return rows * f64(keep)[:, None] + f64(audio_dense)


def greedy_loop(first, next_token, prompt_len, eos_id, max_new, n_ctx):
    """The step loop of run() on the Qwen3-ASR model page. It starts from the
    prefill's token and steps while the newest token is not EOS, fewer than
    max_new tokens exist and the next input position (the prompt length plus
    the steps taken) still fits: position + 1 <= n_ctx. next_token(position,
    token) gives the token a step at that input position produces. Returns
    (tokens, truncated), where truncated means the loop ended other than on
    EOS."""
    tokens = [int(first)]
    cur = int(prompt_len)
    while tokens[-1] != eos_id and len(tokens) < max_new and cur + 1 <= n_ctx:
        tokens.append(int(next_token(cur, tokens[-1])))
        cur += 1
    return tokens, tokens[-1] != eos_id


def final_logits(x_rows, final_gain, embed, eps):
    """Final RMSNorm then the tied lm_head: logits = E @ (RMSNorm(x) * g)."""
    z = rms_norm(x_rows, final_gain, eps)
    return z @ f64(embed).T


def greedy_token(logits):
    """Argmax of one logits row, taken on its fp32 rounding; lowest index wins a tie; NaN never wins."""
    l32 = np.asarray(logits, dtype=np.float32).copy()
    l32[np.isnan(l32)] = -np.inf
    return int(np.argmax(l32))          # numpy returns the first maximal index


def top2_margin(logits):
    """Gap between the largest and the second-largest logit of one row: the
    quantity the greedy-token check compares with its 1e-2 threshold. NaN counts
    as -inf, as in greedy_token; equal top values give 0; a row with one finite
    value gives +inf."""
    l = np.asarray(logits, dtype=np.float64).copy()
    l[np.isnan(l)] = -np.inf
    i = int(np.argmax(l))
    top = l[i]
    l[i] = -np.inf
    second = np.max(l)
    if top == second:
        return 0.0
    return float(top - second)


# ---------------------------------------------------------------- drivers

def prefill_stack(x, layers, p, cache, pos0=0, seq=0, slice_last=False, keep=None):
    """Run T rows through every block. Returns the last block's output
    (only the final row when slice_last) and, if keep is a dict, stores each
    block output under keep[layer]."""
    x = f64(x)
    T = x.shape[0]
    positions = pos0 + np.arange(T)
    seqs = np.full(T, seq)
    n = len(layers)
    for l, w in enumerate(layers):
        ffn_rows = [T - 1] if (slice_last and l == n - 1) else None
        x = block(x, positions, seqs, w, p, cache, l, ffn_rows=ffn_rows)
        if keep is not None:
            keep[l] = x
    return x


def step_stack(x_rows, positions, seqs, layers, p, cache):
    """One decode step of B rows (distinct slabs) through every block."""
    x = f64(x_rows)
    for l, w in enumerate(layers):
        x = block(x, positions, seqs, w, p, cache, l)
    return x


def greedy_generate(x_prompt, layers, p, embed, final_gain, n_new, n_ctx, slice_last=True, forced=None):
    """Prefill x_prompt then generate n_new tokens greedily (the first from the
    prefill's last row, then one per step at positions T, T+1, ...).

    forced: optional list of token ids to feed instead of the argmax
    (teacher forcing); the chosen ids are still reported.
    Returns dict(tokens, logits[n_new, V], margins, x_last_rows)."""
    T = np.asarray(x_prompt).shape[0]
    n_kv, d = p.n_kv_heads, p.head_dim
    cache = KVCache(len(layers), 1, n_ctx, n_kv, d)
    x = prefill_stack(x_prompt, layers, p, cache, slice_last=slice_last)
    logits = [final_logits(x[-1:], final_gain, embed, p.rms_eps)[0]]
    tokens = [greedy_token(logits[-1])]
    x_last = [x[-1]]
    E = embed
    for k in range(1, n_new):
        feed = tokens[-1] if forced is None else int(forced[k - 1])
        xr = f64(E[feed])[None, :]
        xo = step_stack(xr, [T + k - 1], [0], layers, p, cache)
        x_last.append(xo[0])
        logits.append(final_logits(xo, final_gain, embed, p.rms_eps)[0])
        tokens.append(greedy_token(logits[-1]))
    return dict(tokens=tokens, logits=np.stack(logits), margins=[top2_margin(l) for l in logits],
                x_last=np.stack(x_last), cache=cache)
