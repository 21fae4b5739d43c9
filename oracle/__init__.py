"""Plain, slow, float64 CPU oracle for grouped-query attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.  It
shares no code, constants, tables or helpers with the HIP library, and it
imports nothing from it.

The oracle is written from the text of five web pages on grouped-query
attention.  Citations name the page by a short label and the section,
equation or table inside it:

  [EffSeq]    "序列计算与存储" -- note.the0xka1.cc, deep-learning-done-right,
              efficient-sequence-models (sections 分组查询注意力, 头与投影,
              缓存字节, 分块注意力, 在线 softmax, 两块算例, 资源变化)
  [AttnVar]   "第三章：MHA 的局限与 MQA、GQA、Flash Attention" --
              zongyangbigpolo.github.io awesome-ai-roadmap, 03-attention-variants
              (sections 3.1 to 3.7)
  [MhaMqaGqa] zane-jiang.github.io 2026/11/05 mha-mqa-gqa (parameter table,
              sections 1 to 9)
  [AttnEvo]   "04 注意力表示与 KV Cache 演进" -- datawhalechina llm-algo-leetcode,
              04_attention_evolution (evidence-ladder tables)
  [Ch09]      "第 09 章 GQA、MLA 与跨层 KV 共享" -- book.ozine.me llms-from-scratch,
              09_gqa_mla_kv_sharing (sections 09.1 to 09.6)

Modules:
  sdpa      -- the materialized definition O_a = softmax(Q_a K_g(a)^T * scale + M) V_g(a)
  online    -- the block-wise online-softmax state (m, l, u) and the merge of two states
  ledgers   -- the cache-byte, FLOP and arithmetic-intensity formulas
  rope      -- rotary position encoding of query and key rows (the rotation is a
               stated reading: the pages require it but print no formula)
  backward  -- gradients dQ, dK, dV of the materialized attention (group heads
               summed into their K/V head) and the saved row log-sum-exp

Every function is pinned by ``tests/test_oracle_*.py`` and ``tests/test_ledgers.py``
against values the pages print, closed forms, invariants and brute force.
"""

from .sdpa import (
    attention,
    group_index,
    default_scale,
    visibility,
    softmax_rows,
    default_q_pos,
)
from .online import online_states, online_attention_row, merge_states, finish_state
from . import ledgers
from .rope import rope, inv_freq
from .backward import attention_backward, row_logsumexp

__all__ = [
    "attention",
    "group_index",
    "default_scale",
    "visibility",
    "softmax_rows",
    "default_q_pos",
    "online_states",
    "online_attention_row",
    "merge_states",
    "finish_state",
    "ledgers",
    "rope",
    "inv_freq",
    "attention_backward",
    "row_logsumexp",
]
