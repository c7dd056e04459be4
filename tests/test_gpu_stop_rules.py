"""Device-side greedy stopping rules (sttd_greedy_stop) against the oracle's
step loop: planted token streams with EOS, budget and context exits per row
(bit-exact integer state), and a batched greedy loop of a 2-block stack whose
stop step is captured in the replayed HIP graph: rows stop at their own EOS,
stopped rows no longer touch their cache, and each row's tokens equal the same
loop run without stopping, cut where the oracle's loop rules cut it."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle as O
from speech_text_decoder_amd import binding as B
from speech_text_decoder_amd import synth
from speech_text_decoder_amd.device import DecoderSession
from speech_text_decoder_amd.workloads import DecoderShape
from tests.helpers import log

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class StopState:
    def __init__(self, prompt_lens, max_new):
        Bn = len(prompt_lens)
        self.B, self.max_new = Bn, max_new
        self.pos = dev(np.asarray(prompt_lens, np.int32))
        self.active = torch.ones(Bn, dtype=torch.int32, device="cuda")
        self.n_gen = torch.zeros(Bn, dtype=torch.int32, device="cuda")
        self.tokens = torch.full((Bn, max_new), -7, dtype=torch.int32, device="cuda")
        self.truncated = torch.zeros(Bn, dtype=torch.int32, device="cuda")
        self.n_active = torch.zeros(1, dtype=torch.int32, device="cuda")

    def stop(self, rules, ids, advance, stream=0):
        B.greedy_stop(*rules, self.B, ids.data_ptr(), advance, self.pos.data_ptr(), self.active.data_ptr(),
                      self.n_gen.data_ptr(), self.tokens.data_ptr(), self.truncated.data_ptr(),
                      self.n_active.data_ptr(), stream)

    def rows(self):
        n = self.n_gen.cpu().numpy()
        t = self.tokens.cpu().numpy()
        return [t[b, :n[b]].tolist() for b in range(self.B)], self.truncated.cpu().numpy().astype(bool).tolist()


def test_stop_rules_planted_streams_match_the_oracle_loop():
    eos, max_new, n_ctx = 5, 9, 40
    prompt = [10, 10, 36, 3, 20, 38]
    rng = np.random.default_rng(3)
    # step k's token of row b; row 1 meets EOS at step 4, row 3 at the prefill
    table = rng.integers(6, 1000, (len(prompt), max_new + 2)).astype(np.int32)
    table[1, 4] = eos
    table[3, 0] = eos
    table[4, 7] = eos          # row 4: EOS at its eighth token, inside the budget of 9
    st = StopState(prompt, max_new)
    rules = (eos, max_new, n_ctx)
    for k in range(max_new + 2):
        st.stop(rules, dev(table[:, k]), 0 if k == 0 else 1)
    torch.cuda.synchronize()
    got, trunc = st.rows()
    for b, T in enumerate(prompt):
        want, wtr = O.greedy_loop(table[b, 0], lambda pos, tok, b=b, T=T: table[b, pos - T + 1], T, eos, max_new,
                                  n_ctx)
        assert got[b] == want, f"row {b}: {got[b]} vs {want}"
        assert trunc[b] == wtr, f"row {b}"
    assert st.active.sum().item() == 0 and st.n_active.item() == 0
    assert (st.pos.cpu().numpy() == -1).all()
    log(f"rows {got} truncated {trunc}")


@pytest.mark.parametrize("Bn", [3, 1])
def test_stop_rules_in_a_replayed_batched_greedy_loop(Bn):
    """Bn = 1 with a 256-position cache runs each step's projection and attention
    as one launch (two attention splits): a stopped row (position -1) must leave
    its cache alone there too."""
    sh = replace(DecoderShape(hidden=256, n_heads=4, n_kv_heads=2, head_dim=128, ffn=512), n_layers=2, vocab=2000)
    layers = [synth.block_weights(61, l, sh) for l in range(2)]
    E = synth.embedding(61, sh)
    g = synth.final_norm(61, sh)
    T, max_new = 12, 20
    n_ctx = 64 if Bn > 1 else 256
    x0 = synth.prefill_rows(61, Bn * T, sh.hidden)

    def loop(rules):
        sess = DecoderSession(sh, layers, embed=E, final_norm=g, n_ctx=n_ctx, n_seq=Bn, max_rows=Bn * T)
        x = dev(x0)
        sess.prefill_batched(x, [T] * Bn, list(range(Bn)))
        ids = torch.zeros(Bn, dtype=torch.int32, device="cuda")
        xs = torch.zeros(Bn, sh.hidden, device="cuda")
        sess.head(x[T - 1:], ids, next_x=xs, row_stride=T * sh.hidden, rows=Bn)
        st = StopState([T] * Bn, max_new)
        st.stop(rules, ids, 0)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                sess.step(xs, st.pos, pos_bound=n_ctx)
                sess.head(xs, ids, next_x=xs)
                st.stop(rules, ids, 1, stream=s.cuda_stream)
        torch.cuda.current_stream().wait_stream(s)
        snap = None
        for k in range(max_new + 2):
            torch.cuda.synchronize()
            if st.n_active.item() == 0 and k > 0:
                break
            if snap is None and st.active[0].item() == 0:   # row 0 stopped: its cache must stay as it is
                k0, v0 = sess.kv_slab(0, 0)
                snap = (k0.clone(), v0.clone())
            graph.replay()
        torch.cuda.synchronize()
        if snap is not None:
            k0, v0 = sess.kv_slab(0, 0)
            assert torch.equal(k0, snap[0]) and torch.equal(v0, snap[1])
        out = st.rows()
        assert sess.error_bits() == 0
        sess.close()
        return out

    # without stopping (no token is EOS, budget and context large): the plain greedy streams
    free, _ = loop((-1, max_new, n_ctx))
    # EOS = row 0's fifth token; each row must be its free stream cut by the oracle's rules
    eos = free[0][4]
    got, trunc = loop((eos, max_new, n_ctx))
    for b in range(Bn):
        want, wtr = O.greedy_loop(free[b][0], lambda pos, tok, b=b: free[b][pos - T + 1], T, eos, max_new, n_ctx)
        assert got[b] == want and trunc[b] == wtr, f"row {b}: {got[b]} vs {want}"
    log(f"free {free}\nstopped {got} truncated {trunc}")
