"""CPU oracle of the Qwen3-style decoder block (fp64 numpy).

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import it; the HIP path never does.

Parity status of each function (what pins it is in tests/test_oracle_pins.py):
  rms_norm, rope_neox, silu, softmax, gqa_attention_row, block,
  block_rows_subset, final_logits, greedy_token, prefill_stack, step_stack,
  greedy_generate, inject, greedy_loop, top2_margin: pinned by closed forms, library special cases,
  brute force, the causal / batching invariants, and (inject) the pages'
  second form of the same injection, the 3-way concat. The pages print no numeric worked
  example of any decoder output, so no value of the pages' own pins them;
  the only printed figure used is the KV bytes per token (tests/golden).
"""
from .decoder import (KVCache, block, block_rows_subset, final_logits, gqa_attention_row, greedy_generate,
                      greedy_loop, greedy_token, inject, prefill_stack, rms_norm, rope_neox, silu, softmax, step_stack,
                      top2_margin)
