"""Dynamic SplitFuse composition of one pass, restated plainly (test infrastructure).

Policy (DeepSpeed-FastGen paper card by Holmes et al. 2024, "Summary" and
"Interesting ideas"; blog "1. Introduction"):

* every pass works on a fixed token budget B, the scheduler's single knob;
* a sequence in its generation phase contributes exactly one token, and these
  go first, because generation must not be stalled by prompt processing;
* prompt tokens then fill what is left, sequences taken in arrival order (the
  order of the ``seqs`` list); a prompt longer than what is left is cut, so
  the budget is filled exactly whenever demand allows;
* if demand is below B the pass is simply shorter (no padding).

Readings where the pages are silent:

* phase: a sequence is in its prompt phase while ``n_cached < prompt_len``,
  otherwise it decodes one token;
* block allocation: before a sequence is scheduled for ``n`` tokens it must own
  ``ceil((n_cached + n) / block_size)`` blocks; missing blocks are popped from
  the free list; if the pool cannot supply them the sequence gets as many
  tokens as fit (a decode gets 0 or 1); a sequence never owns more than
  ``max_blocks`` blocks;
* the free list is a stack: the initial ids are handed out in the order given,
  released ids are pushed on top (the last one released is handed out first);
* the batch lists the scheduled sequences in ``seqs`` order; sequences that got
  no token are left out; block-table rows are padded with -1.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


class FreeList:
    def __init__(self, ids):
        # stack; the top is the end of the list, so ids[0] is handed out first
        self._stack = [int(b) for b in reversed(list(ids))]

    def available(self) -> int:
        return len(self._stack)

    def pop(self) -> int:
        return self._stack.pop()

    def release(self, ids):
        for b in ids:
            self._stack.append(int(b))

    def snapshot(self):
        return list(self._stack)


@dataclass
class SeqState:
    seq_id: int
    n_cached: int
    prompt_len: int
    blocks: list
    max_blocks: int
    n_scheduled: int = 0


@dataclass
class OracleBatch:
    query_start: np.ndarray   # [S+1] int32
    n_query: np.ndarray       # [S]   int32
    context_len: np.ndarray   # [S]   int32, tokens cached before this pass
    block_table: np.ndarray   # [S][width] int32, -1 padded
    seq_index: np.ndarray     # [S]   int32, index into the seqs list
    seq_id: np.ndarray        # [S]   int64

    @property
    def num_seqs(self) -> int:
        return int(self.n_query.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.query_start[-1])


def _grant(seq: SeqState, want: int, free: FreeList, block_size: int) -> int:
    """Tokens this sequence can take (<= want), allocating the blocks they need."""
    c = seq.n_cached
    want = min(want, seq.max_blocks * block_size - c)
    if want <= 0:
        return 0
    need_blocks = -(-(c + want) // block_size)
    missing = need_blocks - len(seq.blocks)
    if missing > free.available():
        # take every free block and shrink the grant to the room that gives
        want = (len(seq.blocks) + free.available()) * block_size - c
        missing = free.available()
        if want <= 0:
            return 0
    for _ in range(max(0, missing)):
        seq.blocks.append(free.pop())
    return want


def splitfuse_compose(seqs, budget: int, free: FreeList, block_size: int, table_width: int):
    """Compose one pass.  Mutates ``seqs[*].blocks`` / ``n_scheduled`` and ``free``.

    Returns ``(batch, status)`` with status ``"ok"`` or ``"no_blocks"`` (there was
    demand but the pool could not take a single token).
    """
    if budget <= 0:
        raise ValueError("budget must be positive")
    for s in seqs:
        s.n_scheduled = 0
        if s.max_blocks > table_width:
            raise ValueError("table width smaller than a sequence's block capacity")
    left = budget
    # generation tokens first: one per decoding sequence
    for s in seqs:
        if left == 0:
            break
        if s.n_cached >= s.prompt_len:
            n = _grant(s, 1, free, block_size)
            s.n_scheduled = n
            left -= n
    # then prompt tokens, arrival order, the last one cut to fill the budget
    for s in seqs:
        if left == 0:
            break
        if s.n_cached < s.prompt_len:
            n = _grant(s, min(s.prompt_len - s.n_cached, left), free, block_size)
            s.n_scheduled = n
            left -= n

    chosen = [i for i, s in enumerate(seqs) if s.n_scheduled > 0]
    S = len(chosen)
    qs = np.zeros(S + 1, np.int32)
    nq = np.zeros(S, np.int32)
    cl = np.zeros(S, np.int32)
    bt = np.full((S, table_width), -1, np.int32)
    si = np.zeros(S, np.int32)
    sid = np.zeros(S, np.int64)
    for k, i in enumerate(chosen):
        s = seqs[i]
        nq[k] = s.n_scheduled
        qs[k + 1] = qs[k] + s.n_scheduled
        cl[k] = s.n_cached
        bt[k, :len(s.blocks)] = s.blocks
        si[k] = i
        sid[k] = s.seq_id
    batch = OracleBatch(qs, nq, cl, bt, si, sid)
    status = "no_blocks" if (S == 0 and len(seqs) > 0) else "ok"
    return batch, status


def commit_pass(seqs):
    """After the pass ran: the scheduled tokens are now cached."""
    for s in seqs:
        s.n_cached += s.n_scheduled
        s.n_scheduled = 0
