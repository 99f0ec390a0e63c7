"""CPU oracle for one context-parallel rank's share of ring attention.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The product path (the HIP library
and its Python binding) never imports, calls or links anything here, and this
package shares no code with it: it computes everything from the definitions
on the pages, in fp64 numpy (plus a pure-Python brute-force tier for tiny
inputs).

Sources (the pages are cited by title and section):
  [SP-concept]  "序列並行（Sequence Parallelism）" concept page -- section
                "Ring Attention 的不同思路" (ring procedure), section
                "二、Ring Attention 的塊級線上 Softmax" (online-softmax update,
                S = Q K^T / sqrt(d_k)), section "三、Ulysses 的 AllToAll 轉置"
                (worked N=4 layout).
  [CP-TE]       "Context Parallelism" page on Transformer Engine / Megatron --
                section 2.2 (ring step order), 2.3 (Ulysses), 3.3 and 5.2
                (mask offsets must follow the CP split), 4.1 (workload).
  [How-to]      DeepSpeed-Ulysses vs Ring-Attention how-to page -- section 2
                (GQA head limit), 3 (ring_flash_attn_func interface, sp_group),
                5 (head-divisibility assertion, causal load imbalance).
  [XTuner-09]   XTuner chapter 09 -- section 9.5 (cu_seqlens keeps packed
                documents from attending to each other).
  [LongCtx]     Long-context sequence-parallel deep-dive page -- "线索三"
                (online softmax makes attention aggregatable across blocks)
                and the timeline table (Striped Attention, zigzag/stripe).

Parity pins: every function here is pinned by a CPU test against something
other than itself (brute force, a library routine, closed forms, the pages'
worked layout example, invariants). See tests/test_oracle_*.py.
"""
from .partition import positions, doc_bounds, visible_matrix, visible_counts
from .attention import (attention_rows, attention_rank, step_partials, lse_merge, merge_steps,
                        online_softmax_blocks, ring_chunk_order)
from .layouts import cp_reorder, ulysses_permute
from .classify import classify_tiles, SKIP, PARTIAL, FULL
from .backward import attention_rows_backward, attention_rank_backward, ring_step_gradients
from .usp import usp_device_shards, usp_forward

__all__ = [
    "positions", "doc_bounds", "visible_matrix", "visible_counts",
    "attention_rows", "attention_rank", "step_partials", "lse_merge", "merge_steps",
    "online_softmax_blocks", "ring_chunk_order",
    "cp_reorder", "ulysses_permute", "classify_tiles", "SKIP", "PARTIAL", "FULL",
    "attention_rows_backward", "attention_rank_backward", "ring_step_gradients",
    "usp_device_shards", "usp_forward",
]
