"""Seeded synthetic inputs for paged-attention workloads.

This module only draws inputs (lengths, token ids, Q/K/V, sink logits, the
pool's initial free order). It holds none of the method's arithmetic and is the
one module both the oracle-based tests and the product-side harness import.

Conventions (one recipe for every workload):

* ``numpy.random.default_rng(seed)``; the draws happen in a fixed order:
  lengths, pool free order, token ids, Q, K, V, sinks;
* values ~ N(0, 1) drawn in float32, then rounded to bf16 with
  round-to-nearest-even when the storage type is bf16 (raw uint16 bits);
* block size 16; the pool holds the blocks the workload needs times 1.25,
  rounded up to a multiple of 64, and its free list starts as a seeded random
  permutation, so consecutive logical blocks land on scattered physical blocks;
* the query rows of a sequence are its last ``q_len`` positions; their K/V are
  the "new" tokens that a step scatters into the pool, the rest of the context
  is resident before the step;
* a shared prefix has the same token ids and the same K/V in every sequence
  that carries it (same token at the same position).

The five named workloads follow the shapes of the paged-attention passages of
the TensorSharp pages (4 sequences of about 800 tokens on a 32/8-head,
128-dim model; 48 conversations sharing a 2900-token system prompt with
1024-token prefill chunks in between; 8-row speculative verify windows).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

BLOCK = 16


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest-even), returning raw uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


@dataclass
class Seq:
    ctx: int                 # context length after the step's tokens are appended
    q_len: int               # query rows (the last q_len positions)
    tokens: np.ndarray       # int32 [ctx]
    k: np.ndarray            # [ctx, Hkv, D] storage dtype
    v: np.ndarray            # [ctx, Hkv, D] storage dtype
    n_step: int              # tokens scattered by the timed step (the last n_step)


@dataclass
class Workload:
    name: str
    dtype: str               # 'bf16' | 'f32' (storage and Q type) | 'fp8' / 'fp4' (bf16 rows, 8- / 4-bit pools)
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    seqs: List[Seq]
    q: np.ndarray            # [total_rows, Hq, D] storage dtype
    sinks: Optional[np.ndarray]
    num_blocks: int
    free_order: np.ndarray   # int32 permutation of range(num_blocks)
    block_size: int = BLOCK
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def qsl(self) -> np.ndarray:
        out = np.zeros(len(self.seqs) + 1, dtype=np.int32)
        out[1:] = np.cumsum([s.q_len for s in self.seqs])
        return out

    @property
    def context_lens(self) -> np.ndarray:
        return np.array([s.ctx for s in self.seqs], dtype=np.int32)

    @property
    def total_rows(self) -> int:
        return int(sum(s.q_len for s in self.seqs))

    @property
    def max_blocks_per_seq(self) -> int:
        return max(1, max(-(-s.ctx // self.block_size) for s in self.seqs))


def _normal(rng, shape, dtype):
    """N(0, 1) values; bf16 bits for bf16 workloads and for 8- and 4-bit-pool
    ("fp8", "fp4") workloads, whose queries and new K/V rows arrive in bf16."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype in ("bf16", "fp8", "fp4") else x


def _pool_size(unique_blocks: int, exact: Optional[int] = None) -> int:
    if exact is not None:
        return exact
    return int(math.ceil(unique_blocks * 1.25 / 64.0) * 64)


def build(name, dtype, Hq, Hkv, D, ctxs, q_lens, seed, *, shared_prefix=0, n_shared=0,
          sinks=False, scale=None, pool_blocks=None, n_step=None, vocab=32000):
    """Generic recipe. The first ``n_shared`` sequences carry the same
    ``shared_prefix`` leading tokens (and K/V); ``n_step[s]`` defaults to q_len.
    """
    rng = np.random.default_rng(seed)
    S = len(ctxs)
    ctxs = [int(c) for c in ctxs]
    q_lens = [int(x) for x in q_lens]
    for c, ql in zip(ctxs, q_lens):
        if not (1 <= ql <= c):
            raise ValueError("need 1 <= q_len <= ctx")
    shared_full = shared_prefix // BLOCK if n_shared > 1 else 0
    unique = sum(-(-c // BLOCK) for c in ctxs) - shared_full * max(0, n_shared - 1)
    nb = _pool_size(unique, pool_blocks)
    free_order = rng.permutation(nb).astype(np.int32)
    prefix_tokens = rng.integers(0, vocab, size=shared_prefix, dtype=np.int32)
    toks = []
    for s in range(S):
        if s < n_shared:
            tail = rng.integers(0, vocab, size=ctxs[s] - shared_prefix, dtype=np.int32)
            toks.append(np.concatenate([prefix_tokens, tail]))
        else:
            toks.append(rng.integers(0, vocab, size=ctxs[s], dtype=np.int32))
    total_rows = sum(q_lens)
    q = _normal(rng, (total_rows, Hq, D), dtype)
    pk = _normal(rng, (shared_prefix, Hkv, D), dtype)
    ks = []
    for s in range(S):
        if s < n_shared:
            ks.append(np.concatenate([pk, _normal(rng, (ctxs[s] - shared_prefix, Hkv, D), dtype)]))
        else:
            ks.append(_normal(rng, (ctxs[s], Hkv, D), dtype))
    pv = _normal(rng, (shared_prefix, Hkv, D), dtype)
    vs = []
    for s in range(S):
        if s < n_shared:
            vs.append(np.concatenate([pv, _normal(rng, (ctxs[s] - shared_prefix, Hkv, D), dtype)]))
        else:
            vs.append(_normal(rng, (ctxs[s], Hkv, D), dtype))
    sk = rng.standard_normal(size=Hq, dtype=np.float32) if sinks else None
    steps = q_lens if n_step is None else [int(x) for x in n_step]
    seqs = [Seq(ctxs[s], q_lens[s], toks[s], ks[s], vs[s], steps[s]) for s in range(S)]
    return Workload(name, dtype, Hq, Hkv, D, (1.0 / math.sqrt(D)) if scale is None else float(scale),
                    seqs, q, sk, nb, free_order, BLOCK, seed)


def _log_uniform_int(rng, lo, hi, n):
    return np.round(np.exp(rng.uniform(math.log(lo), math.log(hi), size=n))).astype(np.int64)


# Named workloads ------------------------------------------------------------

NAMES = ["tiny_decode", "mid_decode", "sink_decode", "mixed_step", "verify_window"]


def tiny_decode(seed=1001):
    """4 decode rows, contexts {37, 64, 100, 129}, 4 q / 2 KV heads, D 64, fp32,
    a 64-block pool in seeded random order, scale 1/8."""
    return build("tiny_decode", "f32", 4, 2, 64, [37, 64, 100, 129], [1] * 4, seed,
                 pool_blocks=64, scale=1.0 / 8.0)


def _named(name, dtype):
    return name if dtype == "bf16" else f"{name}_{dtype}"


def mid_decode(seed=1002, dtype="bf16"):
    """4 decode rows, contexts ~ U[780, 820], 32 q / 8 KV heads, D 128, bf16
    (dtype "fp8": the same bf16 rows stored in 8-bit pools)."""
    rng = np.random.default_rng(seed)
    ctxs = rng.integers(780, 820, size=4, endpoint=True)
    return build(_named("mid_decode", dtype), dtype, 32, 8, 128, ctxs, [1] * 4, seed + 10_000)


def sink_decode(seed=1003, dtype="bf16"):
    """32 decode rows, contexts log-uniform in [1024, 8192], 64 q / 8 KV heads,
    D 64, bf16, one sink logit ~ N(0, 1) per query head."""
    rng = np.random.default_rng(seed)
    ctxs = _log_uniform_int(rng, 1024, 8192, 32)
    return build(_named("sink_decode", dtype), dtype, 64, 8, 64, ctxs, [1] * 32, seed + 10_000, sinks=True)


def mixed_step(seed=1004, n_decode=48, prefix=2900, tail=(64, 1024), n_prefill=2, chunk=1024, dtype="bf16"):
    """48 decode rows sharing a 2900-token prefix with private tails ~ U[64, 1024]
    plus one new token each, and 2 prefill chunks of 1024 causal rows on fresh
    1024-token contexts; 32 q / 8 KV heads, D 128, bf16."""
    rng = np.random.default_rng(seed)
    tails = rng.integers(tail[0], tail[1], size=n_decode, endpoint=True)
    ctxs = [prefix + int(t) + 1 for t in tails] + [chunk] * n_prefill
    q_lens = [1] * n_decode + [chunk] * n_prefill
    return build(_named("mixed_step", dtype), dtype, 32, 8, 128, ctxs, q_lens, seed + 10_000,
                 shared_prefix=prefix, n_shared=n_decode)


def verify_window(seed=1005, n=16, lo=4096, hi=16384, window=8, dtype="bf16"):
    """16 sequences, contexts ~ U[4096, 16384] including 8 draft rows each,
    causal inside the window; 32 q / 8 KV heads, D 128, bf16."""
    rng = np.random.default_rng(seed)
    ctxs = rng.integers(lo, hi, size=n, endpoint=True)
    return build(_named("verify_window", dtype), dtype, 32, 8, 128, ctxs, [window] * n, seed + 10_000)


def by_name(name, **kw):
    """A named workload; the suffix "_fp8" or "_fp4" selects 8- or 4-bit pools
    for the same rows."""
    for fmt in ("fp8", "fp4"):
        if name.endswith("_" + fmt):
            return by_name(name[:-4], dtype=fmt, **kw)
    return {"tiny_decode": tiny_decode, "mid_decode": mid_decode, "sink_decode": sink_decode,
            "mixed_step": mixed_step, "verify_window": verify_window}[name](**kw)
