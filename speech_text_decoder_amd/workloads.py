"""Decoder shapes and the five synthetic workloads the path is tested and timed on.

Pure data: sizes, dtypes, step counts. No arithmetic of the method lives here.

The 1.7B-shaped decoder: the Canary-Qwen page (src/arch/canary_qwen/model.cpp,
file header) describes a Qwen3-1.7B causal LM of 28 blocks on a 2048-wide
hidden state with a tied lm_head and a greedy loop capped at 256 new tokens.
Head counts (16 query, 8 KV), head dim 128, FFN width 6144 and the 151936-row
vocabulary are not printed on the pages; they are the standard Qwen3-1.7B
sizes. eps 1e-6 and theta 1e6 follow the Qwen3-ASR decoder page
(src/arch/qwen3_asr/decoder.cpp, file header).

The 0.6B-shaped decoder: the MOSS-Transcribe-Diarize page
(src/arch/moss/model.cpp, file header) drives a Qwen3-0.6B causal LM through
the same causal_lm driver. Its sizes are not printed either. They are the
standard Qwen3-0.6B sizes: hidden 1024, 16 query heads and 8 KV heads of
128, so the attention width (2048) is twice the hidden width; FFN 3072; 28
blocks; the same tied vocabulary. The page's own figure, a ~14 GiB worst-case
cache at 131072 tokens in its run() comment, fixes n_kv_heads * head_dim *
n_layers = 28672 for f16 KV, which these sizes meet.
"""
from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class DecoderShape:
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    n_layers: int = 1
    vocab: int = 0               # 0: no lm_head in this workload
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    wdtype: str = "bf16"         # "bf16" | "f32" storage of matrices and gains
    kvdtype: str = "f16"         # "f16" | "f32" storage of the KV cache

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def kv_bytes_per_token(self) -> int:
        """K and V bytes one token adds over all layers (both tensors)."""
        return self.n_kv_heads * self.head_dim * self.n_layers * 2 * (2 if self.kvdtype == "f16" else 4)

    def block_weight_bytes(self) -> int:
        wb = 2 if self.wdtype == "bf16" else 4
        h, i = self.hidden, self.ffn
        mats = self.q_dim * h + 2 * self.kv_dim * h + h * self.q_dim + 2 * i * h + h * i
        gains = 2 * h + 2 * self.head_dim
        return (mats + gains) * wb


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int                  # seeds the input streams
    shape: DecoderShape
    prefill_rows: int            # T of the causal prefill (0: decode only)
    steps: int                   # decode steps after the prefill
    batch: int = 1
    n_ctx: int = 1024
    ctx_len_range: tuple = ()    # (lo, hi) inclusive: batched decode context lengths
    slice_last: bool = False     # last block runs FFN on the final row only
    greedy: bool = False         # decode rows come from the tied table (argmax feedback)
    packed: bool = False         # batch prompts packed back to back through one prefill call per block
    prompt_split: tuple = ()     # (prefix, audio, suffix) rows of each prompt: token ids / injected rows / ids
    description: str = ""


TINY = DecoderShape(hidden=256, n_heads=4, n_kv_heads=2, head_dim=64, ffn=704, wdtype="f32", kvdtype="f32")
QWEN3_1P7B_BLOCK = DecoderShape(hidden=2048, n_heads=16, n_kv_heads=8, head_dim=128, ffn=6144)
QWEN3_1P7B = replace(QWEN3_1P7B_BLOCK, n_layers=28, vocab=151936)
QWEN3_0P6B = DecoderShape(hidden=1024, n_heads=16, n_kv_heads=8, head_dim=128, ffn=3072, n_layers=28, vocab=151936)

WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32_block", 1, TINY, prefill_rows=32, steps=8, n_ctx=64,
                 description="one tiny fp32 block: 32-row causal prefill then 8 decode steps, batch 1"),
        Workload("qwen3_1p7b_block_t153", 2, QWEN3_1P7B_BLOCK, prefill_rows=153, steps=64, n_ctx=1024,
                 description="one 1.7B-shaped bf16 block: 153-row prefill then 64 decode steps, batch 1"),
        Workload("qwen3_1p7b_stack28_greedy256", 3, QWEN3_1P7B, prefill_rows=153, steps=255, n_ctx=1024,
                 slice_last=True, greedy=True,
                 description="28-block 1.7B-shaped stack + final norm + tied lm_head: 153-row prefill, "
                             "then greedy argmax to 256 new tokens (1 from the prefill + 255 steps), batch 1"),
        Workload("qwen3_1p7b_stack28_batched_decode_b16", 4, QWEN3_1P7B, prefill_rows=0, steps=128, batch=16,
                 n_ctx=2048, ctx_len_range=(150, 1500), greedy=True,
                 description="28-block stack + lm_head, 16 sequences with seeded context lengths in "
                             "[150, 1500], 128 lockstep greedy decode steps"),
        Workload("qwen3_1p7b_block_long4096", 5, QWEN3_1P7B_BLOCK, prefill_rows=4096, steps=256, n_ctx=8192,
                 description="one 1.7B-shaped bf16 block: 4096-row causal prefill then 256 decode steps"),
        Workload("qwen3_1p7b_stack28_packed_prefill_b8", 7, QWEN3_1P7B, prefill_rows=153, steps=0, batch=8,
                 packed=True, prompt_split=(9, 138, 6),
                 description="28-block 1.7B-shaped stack + tied head: 8 prompts of 153 rows (9 prefix token "
                             "embeddings, 138 injected audio rows, 6 suffix token embeddings) injected, packed "
                             "through one prefill call per block, each prompt's last row through the head"),
        Workload("qwen3_0p6b_stack28_greedy256", 6, QWEN3_0P6B, prefill_rows=153, steps=255, n_ctx=1024,
                 slice_last=True, greedy=True,
                 description="28-block 0.6B-shaped stack (the MOSS decoder) + final norm + tied lm_head: "
                             "153-row prefill, then greedy argmax to 256 new tokens, batch 1"),
    ]
}
