"""Seeded synthetic workloads for one fixed-budget ragged pass.

Input generation only: this module draws sequence lengths, which physical
blocks each sequence already owns, the order of the free list, and the
Q/K/V values of every token position.  It holds none of the method's
arithmetic (no composition, no scatter into the cache, no attention); both
the oracle and the GPU path consume what it produces.

Shapes follow the pages' workload description (DeepSpeed-FastGen paper card
by Holmes et al. 2024, "Key points": prompt and generation lengths drawn from
normal distributions with means 2600 and 60 and "30% variance", read as a
coefficient of variation of 0.3) and the attention shapes of the model
families the card lists (LLaMA-2-7B: 32 heads of 128; Mistral-7B: 32 query
heads over 8 KV heads of 128).

Values are keyed by (seed, kind, sequence id, 64-position chunk), so the rows
of any position range are the same no matter which pass asks for them.  That
is what makes "k passes of chunks" and "one whole pass" see identical inputs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

KIND_K, KIND_V, KIND_Q = 1, 2, 3
CHUNK = 64  # positions per independently seeded value chunk


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest even), return the bits as uint16.

    Inputs are finite normals, so no NaN/Inf handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


@dataclass
class SeqInit:
    """Initial state of one request before the pass."""
    seq_id: int
    n_cached: int          # tokens whose K/V are already in the cache
    prompt_len: int        # n_cached < prompt_len  =>  still in its prompt phase
    blocks: list           # physical block ids owned, in logical order (history)


@dataclass
class Workload:
    name: str
    dtype: str              # "f32" or "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    budget: int
    scale: float
    value_scale: float
    seed: int
    seqs: list = field(default_factory=list)
    free_ids: np.ndarray = None   # int32, in the order the allocator hands them out
    table_width: int = 0          # block-table row capacity (max blocks per sequence)
    passes: int = 1               # number of consecutive passes the workload asks for
    q_scale: float = 1.0          # extra factor on Q only (steep-logit stress cases)

    # ---- value streams ---------------------------------------------------
    def _chunk(self, kind: int, seq_id: int, chunk: int, heads: int, extra: float) -> np.ndarray:
        ss = np.random.SeedSequence([self.seed, kind, seq_id, chunk])
        rng = np.random.Generator(np.random.PCG64(ss))
        x = rng.standard_normal((CHUNK, heads, self.head_dim), dtype=np.float32)
        if self.value_scale * extra != 1.0:
            x *= np.float32(self.value_scale * extra)
        return x

    def _rows(self, kind: int, seq_id: int, p0: int, p1: int, heads: int,
              extra: float = 1.0) -> np.ndarray:
        if p1 <= p0:
            shape = (0, heads, self.head_dim)
            return np.zeros(shape, np.uint16 if self.dtype == "bf16" else np.float32)
        c0, c1 = p0 // CHUNK, (p1 + CHUNK - 1) // CHUNK
        x = np.concatenate([self._chunk(kind, seq_id, c, heads, extra) for c in range(c0, c1)])
        x = x[p0 - c0 * CHUNK:p1 - c0 * CHUNK]
        return f32_to_bf16_bits(x) if self.dtype == "bf16" else np.ascontiguousarray(x)

    def k_rows(self, seq_id: int, p0: int, p1: int) -> np.ndarray:
        """K rows of positions [p0, p1): [p1-p0][Hkv][D] (uint16 bf16 bits or float32)."""
        return self._rows(KIND_K, seq_id, p0, p1, self.num_kv_heads)

    def v_rows(self, seq_id: int, p0: int, p1: int) -> np.ndarray:
        return self._rows(KIND_V, seq_id, p0, p1, self.num_kv_heads)

    def q_rows(self, seq_id: int, p0: int, p1: int) -> np.ndarray:
        """Q rows of positions [p0, p1): [p1-p0][Hq][D]."""
        return self._rows(KIND_Q, seq_id, p0, p1, self.num_q_heads, self.q_scale)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def fresh_states(self):
        """Deep copy of the initial sequence states (lists are mutated by composition)."""
        return [SeqInit(s.seq_id, s.n_cached, s.prompt_len, list(s.blocks)) for s in self.seqs]


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def _normal_len(rng, mean, sd, lo, hi, size=None):
    x = np.rint(rng.normal(mean, sd, size=size))
    return np.clip(x, lo, hi).astype(np.int64)


def _assign_blocks(rng, seq_specs, num_blocks, block_size):
    """Random permutation of the pool; history blocks first, the rest is the free list."""
    perm = rng.permutation(num_blocks).astype(np.int32)
    pos = 0
    seqs = []
    for sid, cached, plen in seq_specs:
        nb = -(-cached // block_size)
        seqs.append(SeqInit(sid, int(cached), int(plen), [int(b) for b in perm[pos:pos + nb]]))
        pos += nb
    return seqs, perm[pos:].copy()


def _finish(name, dtype, hq, hkv, d, bs, budget, value_scale, seed, specs, num_blocks, rng,
            passes=1):
    seqs, free = _assign_blocks(rng, specs, num_blocks, bs)
    width = max(-(-max(p, c + 1) // bs) for _, c, p in specs)
    return Workload(name=name, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                    block_size=bs, num_blocks=num_blocks, budget=budget,
                    scale=1.0 / math.sqrt(d), value_scale=value_scale, seed=seed,
                    seqs=seqs, free_ids=free, table_width=width, passes=passes)


def _blocks_upper_bound(specs, bs, budget):
    """Pool size that can hold every sequence's history plus what one pass could add."""
    total = 0
    for _, c, p in specs:
        extra = 1 if c >= p else min(p - c, budget)
        total += -(-(c + extra) // bs)
    return total


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def tiny_f32(seed: int = 1) -> Workload:
    """4 sequences (2 prompt chunks + 2 decode tokens), fp32, 4 heads of 64, blocks of 16,
    a 64-block permuted pool, budget 64, prior contexts uniform in [0, 100]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    c = rng.integers(0, 101, size=4)
    n_a = int(rng.integers(1, 62))
    n_b = 62 - n_a
    extra = int(rng.integers(0, 51))
    specs = [
        (100 + 0, int(c[0]), int(c[0]) + n_a),              # prompt: finishes in this pass
        (100 + 1, int(c[1]), int(c[1])),                    # decoding
        (100 + 2, int(c[2]), int(c[2]) + n_b + extra),      # prompt: chunked to fill the budget
        (100 + 3, int(c[3]), int(c[3])),                    # decoding
    ]
    return _finish("tiny_f32", "f32", 4, 4, 64, 16, 64, 1.0, seed, specs, 64, rng)


def _mixed(name, seed, hq, hkv, budget, n_decode, dec_clip, prompt_clip, value_scale):
    rng = np.random.Generator(np.random.PCG64(seed))
    specs = []
    dec = _normal_len(rng, 2600, 780, dec_clip[0], dec_clip[1], size=n_decode)
    for i, c in enumerate(dec):
        specs.append((1000 + i, int(c), int(c)))
    # prompt queue: one continuation prompt, then fresh prompts until the budget is covered
    need = budget - n_decode
    L = int(_normal_len(rng, 2600, 780, prompt_clip[0], prompt_clip[1]))
    c0 = int(rng.integers(0, L))
    specs.append((2000, c0, L))
    have = L - c0
    k = 1
    while have < need:
        L = int(_normal_len(rng, 2600, 780, prompt_clip[0], prompt_clip[1]))
        specs.append((2000 + k, 0, L))
        have += L
        k += 1
    nb = _blocks_upper_bound(specs, 64, budget)
    return _finish(name, "bf16", hq, hkv, 128, 64, budget, value_scale, seed, specs, nb, rng)


def llama2_mixed(seed: int = 2) -> Workload:
    """LLaMA-2-7B attention shape: 24 decodes + prompt chunks filling a 2048-token budget."""
    return _mixed("llama2_7b_mixed", seed, 32, 32, 2048, 24, (64, 4096), (64, 4096), 0.5)


def decode_only(seed: int = 3, num_seqs: int = 256) -> Workload:
    """256 single-token decodes over long contexts (HBM-bound)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = _normal_len(rng, 2660, 800, 64, 8192, size=num_seqs)
    specs = [(3000 + i, int(c), int(c)) for i, c in enumerate(ctx)]
    nb = sum(-(-(int(c) + 1) // 64) for c in ctx)
    return _finish("decode_only", "bf16", 32, 32, 128, 64, num_seqs, 1.0, seed, specs, nb, rng)


def chunked_prefill(seed: int = 4, prompt_len: int = 16384, chunk: int = 512) -> Workload:
    """One long prompt processed in passes of `chunk` tokens over a 256-block permuted pool."""
    rng = np.random.Generator(np.random.PCG64(seed))
    specs = [(4000, 0, prompt_len)]
    nb = max(256, -(-prompt_len // 64))
    return _finish("chunked_prefill", "bf16", 32, 32, 128, 64, chunk, 1.0, seed, specs, nb, rng,
                   passes=-(-prompt_len // chunk))


def mistral_gqa(seed: int = 5) -> Workload:
    """Mistral-7B GQA shape (32 query heads over 8 KV heads): 64 decodes + prompt chunks
    filling a 4096-token budget."""
    return _mixed("mistral_7b_gqa", seed, 32, 8, 4096, 64, (64, 8192), (64, 8192), 1.0)


def custom(seed, *, dtype="bf16", hq=8, hkv=8, d=128, bs=64, budget=256, n_decode=4,
           decode_ctx=(64, 600), prompts=((0, 300),), value_scale=1.0, extra_blocks=0,
           q_scale=1.0):
    """Small mixed workload for parity cases: `n_decode` decodes with contexts uniform in
    `decode_ctx`, then prompts given as (n_cached, prompt_len) pairs, in that order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    specs = []
    for i in range(n_decode):
        c = int(rng.integers(decode_ctx[0], decode_ctx[1] + 1))
        specs.append((5000 + i, c, c))
    for j, (c, L) in enumerate(prompts):
        specs.append((6000 + j, int(c), int(L)))
    nb = _blocks_upper_bound(specs, bs, budget) + extra_blocks
    w = _finish("custom", dtype, hq, hkv, d, bs, budget, value_scale, seed, specs, nb, rng)
    w.scale = 1.0 / math.sqrt(d)
    w.q_scale = float(q_scale)
    return w


def uniform_pass(S: int, n: int, c: int, seed: int = 8, hq: int = 32, hkv: int = 32,
                 d: int = 128, bs: int = 64) -> Workload:
    """S sequences, each with c cached tokens and n new ones (a pass of T = S*n tokens): the
    shape family of the profiling sweeps (paper card "Interesting ideas": pass latency is
    driven by the total token count; throughput saturates and is concave in it)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    specs = [(7000 + i, int(c), int(c + n)) for i in range(S)]
    nb = S * -(-(c + n) // bs)
    return _finish(f"uniform_S{S}_n{n}_c{c}", "bf16", hq, hkv, d, bs, S * n, 1.0, seed, specs,
                   nb, rng)


# ---------------------------------------------------------------------------
# request streams for the multi-pass serving loop
# ---------------------------------------------------------------------------

@dataclass
class Request:
    rid: int           # also the sequence id of its value streams
    prompt_len: int    # P >= 1
    output_len: int    # O >= 1 generated tokens

    @property
    def stop_len(self) -> int:
        """Positions whose K/V the request caches: its P prompt tokens and the first O - 1
        generated ones (the last generated token is never fed back)."""
        return self.prompt_len + self.output_len - 1


@dataclass
class ServingWorkload:
    """Requests of `clients` closed-loop clients: client c sends requests c, c + clients,
    c + 2*clients, ... one at a time, the next as soon as the previous finished."""
    name: str
    requests: list
    clients: int
    budget: int
    values: Workload        # shapes, value streams (keyed by request id) and pool size

    @property
    def table_width(self) -> int:
        bs = self.values.block_size
        return max(-(-r.stop_len // bs) for r in self.requests)


def serving_stream(seed: int = 6, n_requests: int = 512, clients: int = 32, budget: int = 2048,
                   prompt_mean: float = 2600.0, output_mean: float = 60.0, cv: float = 0.3,
                   prompt_clip=(64, 8192), output_clip=(1, 512), dtype: str = "bf16",
                   hq: int = 32, hkv: int = 32, d: int = 128, bs: int = 64,
                   value_scale: float = 1.0, name: str = "serving_llama2_7b") -> ServingWorkload:
    """The card's request stream ("Key points": prompt and generation lengths normal with
    means 2600 and 60 and a 30% coefficient of variation; 1 to 32 clients; 512 requests), at
    an attention shape of the model families it names (LLaMA-2-7B by default).  The pool
    holds the largest possible running set: `clients` requests of the largest block count."""
    rng = np.random.Generator(np.random.PCG64(seed))
    P = _normal_len(rng, prompt_mean, cv * prompt_mean, prompt_clip[0], prompt_clip[1],
                    size=n_requests)
    O = _normal_len(rng, output_mean, cv * output_mean, output_clip[0], output_clip[1],
                    size=n_requests)
    reqs = [Request(10000 + i, int(p), int(o)) for i, (p, o) in enumerate(zip(P, O))]
    width = max(-(-r.stop_len // bs) for r in reqs)
    nb = min(clients, n_requests) * width
    free = rng.permutation(nb).astype(np.int32)
    vals = Workload(name=name, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                    block_size=bs, num_blocks=nb, budget=budget, scale=1.0 / math.sqrt(d),
                    value_scale=value_scale, seed=seed, seqs=[], free_ids=free,
                    table_width=width)
    return ServingWorkload(name=name, requests=reqs, clients=int(clients), budget=int(budget),
                           values=vals)


def serving_small(seed: int = 7, dtype: str = "bf16", n_requests: int = 10, clients: int = 3,
                  budget: int = 96, bs: int = 16) -> ServingWorkload:
    """A small stream for parity: prompts ~N(120, 36), outputs ~N(6, 2), 4 query heads over
    2 KV heads of 128."""
    return serving_stream(seed, n_requests, clients, budget, 120.0, 6.0, 0.3, (8, 400), (1, 20),
                          dtype, 4, 2, 128, bs, 1.0, "serving_small")


CONFIGS = {
    1: tiny_f32,
    2: llama2_mixed,
    3: decode_only,
    4: chunked_prefill,
    5: mistral_gqa,
}


def make(config: int, seed: int | None = None, **kw) -> Workload:
    fn = CONFIGS[config]
    return fn(config if seed is None else seed, **kw)


def fill_pools_device(k_pool, v_pool, seed: int, value_scale: float = 1.0):
    """Fill two device pools with i.i.d. N(0, value_scale^2) values from torch's seeded
    device generator (for passes whose cache is too large to generate on the host).
    Every slot gets a finite value, history or not."""
    import torch
    g = torch.Generator(device=k_pool.device)
    g.manual_seed(int(seed))
    for t in (k_pool, v_pool):
        # fill in slabs so the fp32 intermediate stays small
        flat = t.view(t.shape[0], -1)
        step = max(1, (1 << 27) // max(1, flat.shape[1]))
        for i in range(0, flat.shape[0], step):
            x = torch.randn(flat[i:i + step].shape, generator=g, device=t.device,
                            dtype=torch.float32)
            if value_scale != 1.0:
                x.mul_(value_scale)
            flat[i:i + step].copy_(x)
