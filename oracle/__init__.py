"""CPU oracle for one fixed-budget ragged pass over a blocked KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link
or execute anything in this package: only the test suite, the smoke check and
the benchmark's CPU-baseline leg use it.  It shares no code with the GPU path
(no kernels, headers, helpers, tables or pre/post-processing); the only thing
both sides consume is the seeded input generator, which holds none of the
method's arithmetic.

What it computes, in plain numpy float64 (slow and obviously correct):

* ``compose``   — the Dynamic SplitFuse composition of one pass (token budget
  filled by decode tokens first, then prompt tokens in arrival order, the last
  prompt cut to fill the budget exactly) plus the block allocation it implies.
  Sources: DeepSpeed-FastGen paper card by Holmes et al. (2024), "Summary" and
  "Interesting ideas" (fixed token budget per pass; long prompts split over
  several passes; short prompts and generation tokens packed to fill it); the
  reading notes page "DeepSpeed-FastGen: High-throughput Text Generation for
  LLMs via MII and DeepSpeed-Inference", method paragraph (each request split
  into prompt and generation work); blog "1. Introduction" (generation must
  not be preempted by prompt processing).
* ``append``    — the scatter of a pass's new K/V rows into the paged cache
  (paper card "Key points": a blocked KV cache as in PagedAttention).
* ``attention`` — exact causal softmax attention of every new query token over
  its sequence's whole cached history, gathered through the block table
  (paper card "Key points" and "References": FlashAttention, an exact
  attention, is the kernel family used).
* ``serving``   — the multi-pass loop around the pass: closed-loop clients,
  continuous batching, retirement of finished requests and reuse of their
  blocks (paper card "Key points": continuous batching, blocked KV cache, 1 to
  32 clients and 512 requests).
* ``linear``    — the dense projections either side of attention, y = x . w^T
  (paper card "Key points": the surrounding kernels come from
  FasterTransformer).

Parity pins live in ``tests/test_oracle_*.py`` and ``tests/test_serving.py`` (brute force, closed forms,
block-permutation and chunking invariants, hand-derived fixtures under
``tests/golden/``).  No oracle function is "parity unpinned".
"""
from .bf16 import bf16_bits_to_f64
from .compose import FreeList, OracleBatch, SeqState, splitfuse_compose, commit_pass
from .append import kv_append
from .attention import ragged_attention
from .layout import k_pool_shape, v_pool_shape, v_slot
from .linear import linear
from .serving import serve

__all__ = [
    "bf16_bits_to_f64", "FreeList", "OracleBatch", "SeqState", "splitfuse_compose",
    "commit_pass", "kv_append", "ragged_attention", "linear", "serve", "k_pool_shape",
    "v_pool_shape", "v_slot",
]
