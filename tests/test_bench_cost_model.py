"""The benchmark's algorithmic cost model, the numerator of every roofline
fraction it prints, against closed forms worked out by hand.

The shape is the 1.7B-sized decoder block: hidden 2048, 16 query heads and 8 KV
heads of 128, FFN 6144, vocabulary 151936, bf16 weights and an f16 KV cache.
Every expected value below is a literal, with its arithmetic beside it. An
inflated byte or flop count would inflate a reported fraction, and this catches
it. The rules are: each weight byte is read once; activations are read and
written once, in fp32; the norm gain is read once; causal attention counts only
the lower triangle.
"""
import bench
from speech_text_decoder_amd.workloads import QWEN3_1P7B

S = QWEN3_1P7B
cost = bench.kernel_cost


def test_shape_is_the_one_the_literals_assume():
    assert (S.hidden, S.n_heads, S.n_kv_heads, S.head_dim, S.ffn, S.vocab) == (2048, 16, 8, 128, 6144, 151936)
    assert (S.wdtype, S.kvdtype) == ("bf16", "f16")


def test_decode_gemv_bytes_and_flops_one_row():
    # Q|K|V: 4096 x 2048 bf16 = 16,777,216; gain 4,096; x in 8,192; q|k|v out 16,384
    assert cost("qkv_gemv", S, 1) == (16_805_888, 16_777_216.0)
    # O: 2048 x 2048 bf16 = 8,388,608; attention row in 8,192; residual in + out 16,384
    assert cost("o_gemv", S, 1) == (8_413_184, 8_388_608.0)
    # gate_up: 12288 x 2048 bf16 = 50,331,648; gain 4,096; x in 8,192; act out 24,576
    assert cost("gateup_gemv", S, 1) == (50_368_512, 50_331_648.0)
    # down: 2048 x 6144 bf16 = 25,165,824; act in 24,576; residual in + out 16,384
    assert cost("down_gemv", S, 1) == (25_206_784, 25_165_824.0)
    # tied head: 151936 x 2048 bf16 = 622,329,856; x in 8,192
    assert cost("lm_head", S, 1) == (622_338_048, 622_329_856.0)


def test_decode_attention_counts_real_cache_rows_only():
    # 154 keys (position 153): K and V rows 154 x 8 x 128 x 2 x 2 B = 630,784;
    # q in + o out 2 x 2048 x 4 = 16,384; flops 4 x 2048 x 154
    assert cost("attn_rows", S, 1, 154) == (647_168, 1_261_568.0)


def test_one_launch_projection_attention_is_the_sum_of_its_parts():
    # the Q|K|V projection (16,805,888 B) and the attention over 154 keys (647,168 B)
    # of one decode row in one launch: their bytes and flops add, nothing more
    assert cost("qkv_attn", S, 1, 154) == (16_805_888 + 647_168, 16_777_216.0 + 1_261_568.0)


def test_prefill_4096_rows_flops():
    T = 4096
    # causal: 4 x 2048 x 4096 x 4097 / 2
    assert cost("attn_prefill", S, T)[1] == 68_736_253_952.0
    # 4096 x (q in + o out 2 x 2048 x 4 + new K, V rows 2 x 1024 x 2)
    assert cost("attn_prefill", S, T)[0] == 83_886_080
    gemm = sum(cost(n, S, T)[1] for n in ("qkv_gemm", "o_gemm", "gateup_gemm", "down_gemm"))
    # 2 x 4096 x 2048 x (4096 + 2048 + 12288) + 2 x 4096 x 6144 x 2048
    assert gemm == 412_316_860_416.0
    assert gemm + cost("attn_prefill", S, T)[1] == 481_053_114_368.0


def test_prefill_153_rows_flops():
    T = 153
    total = sum(cost(n, S, T)[1] for n in ("qkv_gemm", "o_gemm", "gateup_gemm", "down_gemm", "attn_prefill"))
    # 2 x 153 x 2048 x 24576 + 4 x 2048 x 153 x 154 / 2
    assert total == 15_497_994_240.0


def test_block_weights_and_greedy_step_bytes():
    # matrices 50,331,648 bf16 elements + gains 2 x 2048 + 2 x 128
    assert S.block_weight_bytes() == 100_672_000
    # first greedy step after a 153-row prompt (154 keys) and the last of 256 new
    # tokens (409 keys): 28 x (weights + keys x 4096 + new K, V 4096) + head and
    # its gain 622,333,952 + x in and out 16,384
    assert bench.decode_step_bytes(S, 28, 1, 154, True) == 3_458_942_976
    assert bench.decode_step_bytes(S, 28, 1, 409, True) == 3_488_188_416
