"""Workload shapes against the one figure the pages print about them."""
import os

from speech_text_decoder_amd.workloads import QWEN3_0P6B, QWEN3_1P7B

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_kv():
    vals = {}
    with open(os.path.join(GOLDEN, "kv_bytes_per_token.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if line:
                vals[line[0]] = int(line[1])
    return vals


def test_0p6b_shape_meets_the_moss_pages_cache_figure():
    """The MOSS page's ~14 GiB at 131072 tokens is a figure about its own
    Qwen3-0.6B decoder: the supplied 0.6B sizes must reproduce it."""
    vals = golden_kv()
    assert QWEN3_0P6B.kv_bytes_per_token() * vals["tokens"] == vals["bytes"]
    assert QWEN3_0P6B.q_dim == 2 * QWEN3_0P6B.hidden   # attention wider than the residual stream


def test_1p7b_shape_kv_bytes_per_token():
    assert QWEN3_1P7B.kv_bytes_per_token() == 114688
