"""Continuous batching over Dynamic SplitFuse passes, restated plainly (test infrastructure).

Sources: DeepSpeed-FastGen paper card by Holmes et al. (2024), "Key points" (FastGen builds on
continuous batching as in Orca and on a blocked KV cache as in PagedAttention; the benchmark
drives it with 1 to 32 concurrent clients and 512 requests) and "Summary" (every forward pass
runs at the fixed token budget; long prompts are chunked over passes, short prompts and
generation tokens fill it); blog "1. Introduction" (each request is prompt processing, then
generation, one token per step).

Readings where the pages are silent:

* a request with P prompt tokens and O generated tokens: the pass that takes its last prompt
  token yields the first generated token; every later pass feeds one generated token back
  and yields the next, so it caches P + O - 1 positions (``stop_len``) and is finished after
  the pass that brings ``n_cached`` to that count;
* clients are closed loops: client c sends requests c, c + C, c + 2C, ... (C clients), the
  first ones at the start in client order, each next one right after the pass that finished
  its predecessor; new requests join the end of the running list (arrival order);
* after a pass: commit, then retire every finished request -- their blocks go back to the free
  stack, requests in running-list order and each one's blocks in logical order -- then the
  clients of the retired requests send their next ones, in that same order.

Every pass is one call of ``splitfuse_compose`` (decode tokens first, then prompt tokens in
arrival order, the last prompt cut to fill the budget exactly).
"""
from __future__ import annotations

from dataclasses import dataclass, field

from .compose import FreeList, SeqState, commit_pass, splitfuse_compose


@dataclass
class ServingTrace:
    batches: list = field(default_factory=list)       # OracleBatch of every pass
    first_token_pass: dict = field(default_factory=dict)  # request id -> pass index
    finish_pass: dict = field(default_factory=dict)       # request id -> pass index
    admit_pass: dict = field(default_factory=dict)        # request id -> first pass it can join
    free_after: list = field(default_factory=list)       # free-stack size after every pass


def serve(requests, clients: int, budget: int, free_ids, block_size: int, table_width: int,
          max_passes: int = 1_000_000) -> ServingTrace:
    """Run the whole request stream.  ``requests``: objects with ``rid``, ``prompt_len``,
    ``output_len``; request k belongs to client ``k % clients``."""
    if clients < 1:
        raise ValueError("at least one client")
    free = FreeList(free_ids)
    queues = [list(range(c, len(requests), clients)) for c in range(clients)]
    stop = {}
    running = []
    trace = ServingTrace()

    def admit(client, p):
        if not queues[client]:
            return
        k = queues[client].pop(0)
        r = requests[k]
        if r.prompt_len < 1 or r.output_len < 1:
            raise ValueError("a request needs a prompt token and a generated token")
        s = r.prompt_len + r.output_len - 1
        stop[r.rid] = (s, client)
        running.append(SeqState(r.rid, 0, r.prompt_len, [], -(-s // block_size)))
        trace.admit_pass[r.rid] = p

    for c in range(clients):
        admit(c, 0)
    p = 0
    while running:
        if p >= max_passes:
            raise RuntimeError("pass limit reached")
        batch, status = splitfuse_compose(running, budget, free, block_size, table_width)
        if status != "ok":
            raise RuntimeError("the pool cannot take a single token")
        trace.batches.append(batch)
        commit_pass(running)
        for s in running:
            if s.n_cached >= s.prompt_len and s.seq_id not in trace.first_token_pass:
                trace.first_token_pass[s.seq_id] = p
        done = [s for s in running if s.n_cached >= stop[s.seq_id][0]]
        for s in done:
            free.release(s.blocks)
            trace.finish_pass[s.seq_id] = p
        running[:] = [s for s in running if s.n_cached < stop[s.seq_id][0]]
        for s in done:
            admit(stop[s.seq_id][1], p + 1)
        trace.free_after.append(free.available())
        p += 1
    return trace
