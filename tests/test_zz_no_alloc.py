"""The allocation-free head (sttd_lm_head_argmax_static: static device scratch,
no workspace) against the workspace head on the same inputs, through the C ABI:
two calls in a row, the second with fewer rows (the scratch keeps the first
call's contents), on the 1.7B-shaped head (151,936 x 2048 bf16 tied table)."""
import numpy as np
import pytest
import torch

from speech_text_decoder_amd import binding as B
from speech_text_decoder_amd import synth
from speech_text_decoder_amd.device import DecoderSession
from speech_text_decoder_amd.workloads import WORKLOADS
from tests.helpers import log

pytestmark = pytest.mark.gpu


def test_static_head_matches_workspace_head_twice_then_rejects_oversize():
    wl = WORKLOADS["qwen3_1p7b_stack28_greedy256"]
    sh = wl.shape
    E = synth.embedding(wl.cfg_id, sh)
    g = synth.final_norm(wl.cfg_id, sh)
    n_x = 40
    x = synth.prefill_rows(wl.cfg_id, n_x, sh.hidden)
    sess = DecoderSession(sh, [synth.block_weights(wl.cfg_id, 0, sh)], embed=E, final_norm=g, n_ctx=64,
                          max_rows=B.STATIC_HEAD_MAX_ROWS)
    xd = torch.from_numpy(x).cuda()
    wt = B.BF16
    # call 1: 16 rows picked by index (the MFMA head); call 2: 3 rows by stride (the GEMV head)
    for n_rows, rows in [(16, np.arange(2, 40, 2.4).astype(np.int32)[:16]), (3, None)]:
        ids_s = torch.full((n_rows,), -7, dtype=torch.int32, device="cuda")
        ids_w = torch.full((n_rows,), -9, dtype=torch.int32, device="cuda")
        lg_s = torch.zeros(n_rows, sh.vocab, device="cuda")
        lg_w = torch.zeros(n_rows, sh.vocab, device="cuda")
        nx_s = torch.zeros(n_rows, sh.hidden, device="cuda")
        nx_w = torch.zeros(n_rows, sh.hidden, device="cuda")
        pos_s = torch.arange(n_rows, dtype=torch.int32, device="cuda")
        pos_w = pos_s.clone()
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        xr = torch.from_numpy(rows).cuda() if rows is not None else None
        s = torch.cuda.current_stream().cuda_stream
        B.lm_head_argmax_static(sess.final_norm.data_ptr(), sess.embed.data_ptr(), wt, sh.vocab, sh.hidden,
                                sh.rms_eps, n_rows, xd.data_ptr(), sh.hidden, ids_s.data_ptr(), lg_s.data_ptr(),
                                nx_s.data_ptr(), pos_s.data_ptr(), err.data_ptr(), s,
                                x_rows=0 if xr is None else xr.data_ptr(), n_x_rows=n_x if xr is not None else 0)
        B.lm_head_argmax(sess.final_norm.data_ptr(), sess.embed.data_ptr(), wt, sh.vocab, sh.hidden, sh.rms_eps,
                         sess.ws, n_rows, xd.data_ptr(), sh.hidden, ids_w.data_ptr(), lg_w.data_ptr(),
                         nx_w.data_ptr(), pos_w.data_ptr(), s,
                         x_rows=0 if xr is None else xr.data_ptr(), n_x_rows=n_x if xr is not None else 0)
        torch.cuda.synchronize()
        log(f"{n_rows} rows: static ids {ids_s.cpu().numpy().tolist()}")
        np.testing.assert_array_equal(ids_s.cpu().numpy(), ids_w.cpu().numpy())
        assert (ids_s.cpu().numpy() >= 0).all()
        np.testing.assert_array_equal(lg_s.cpu().numpy(), lg_w.cpu().numpy())
        np.testing.assert_array_equal(nx_s.cpu().numpy(), nx_w.cpu().numpy())
        np.testing.assert_array_equal(pos_s.cpu().numpy(), np.arange(n_rows) + 1)
        assert int(err.item()) == 0
    with pytest.raises(B.SttdError) as e:
        B.lm_head_argmax_static(sess.final_norm.data_ptr(), sess.embed.data_ptr(), wt, sh.vocab, sh.hidden,
                                sh.rms_eps, B.STATIC_HEAD_MAX_ROWS + 1, xd.data_ptr(), sh.hidden, ids_s.data_ptr())
    assert e.value.status == B.ERR_INVALID_ARG
    assert sess.error_bits() == 0
    sess.close()
