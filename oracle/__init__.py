"""CPU fp64 oracle for the FlashAttention forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.
The product (``io_aware_attention_attn_amd``) never imports it, and it imports
nothing from the product: the two share no code.  The only module both sides
use is ``workloads`` (seeded input generators, no attention arithmetic).

What it computes is plain *standard* attention, the one that materialises the
score matrix S and the probability matrix P (and its gradient, by the same
materialised P), written from these pages:

  [FA-notes]   "flash-attn" notes, minjae-portfolio.vercel.app/notes/flash-attn
  [FA-evo]     "Attention is All You Need부터 FlashAttention-3까지: Transformer Attention
               메커니즘의 진화와 O(1) 메모리 최적화 실전 구현", tildalice.io
  [LLM-basics] "LLM 기초 — Attention부터 FlashAttention까지", gylee815.github.io/llmso/w1
  [FA3-entry]  "FlashAttention-3 (FA-3)", itpe.jackerlab.com

Every function is pinned by ``tests/test_oracle.py`` to something other than
itself (the pages' worked example, closed forms, invariants, brute force on tiny
inputs, a library routine).  No function here is "parity unpinned".
"""
from .attention import (  # noqa: F401
    attention,
    attention_backward,
    attention_probs,
    attention_varlen,
    decode_attention,
    decode_attention_paged,
    lse_merge,
    block_state,
    merge_states,
    online_attention_rows,
    safe_softmax,
    visible,
)
