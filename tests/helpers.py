"""Shared pieces of the GPU parity tests: tolerances and oracle plumbing."""
import numpy as np

from speech_text_decoder_amd import synth

# fp32 path: max |gpu - oracle| / max |oracle| per tensor
TOL_F32 = 1e-4
# bf16-weight path: per row, max |gpu - oracle| / RMS(oracle row)
TOL_BF16 = 3e-2
# greedy ids must agree wherever the oracle's top-2 logit margin exceeds this
MARGIN = 1e-2


def widen_layer(w):
    return {k: synth.widen(v) for k, v in w.items()}


def widen_layer_f64(w):
    return {k: synth.widen(v).astype(np.float64) for k, v in w.items()}


def rel_err_tensor(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    return float(np.max(np.abs(g - o)) / np.max(np.abs(o)))


def rel_err_rows(g, o):
    g = np.asarray(g, np.float64).reshape(-1, np.shape(o)[-1])
    o = np.asarray(o, np.float64).reshape(-1, np.shape(o)[-1])
    rms = np.sqrt(np.mean(o * o, axis=1))
    return float(np.max(np.max(np.abs(g - o), axis=1) / rms))


def check(g, o, fp32, what=""):
    if fp32:
        e = rel_err_tensor(g, o)
        assert e <= TOL_F32, f"{what}: max rel error {e:.3g} > {TOL_F32}"
    else:
        e = rel_err_rows(g, o)
        assert e <= TOL_BF16, f"{what}: max row-RMS-relative error {e:.3g} > {TOL_BF16}"
    return e


def log(msg):
    print(msg, flush=True)
