"""Oracle for batched attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything under ``oracle/``.
The product (``paged_kv_attention_block_amd``) never imports, links or calls
it, and the two share no code: this package does its own allocation, its own
scatter, its own gather and its own attention.

Sources (the TensorSharp "高级功能" page):

* section "连续批处理与分页 KV 缓存": the KV cache is cut into fixed-size
  blocks drawn from one shared pool, and every full block is content-hashed so
  that identical prefixes are shared between concurrent and later requests
  instead of being recomputed;
* section "原生分页注意力": a paged-attention call gathers K/V out of the paged
  buffers and runs attention per sequence, with a variant that takes sink
  logits;
* "批量前向" paragraph of the same section: new K/V are scatter-written into
  the paged buffers;
* section "内存优化", paged KV pool item: LRU eviction and cross-session
  content-hash reuse.

The pages fix no memory layout, no hash function and no allocation order. The
readings used here (the library's documented interface) are:

* pool layout, block size B, X = 16 // element size (8 for bf16, 4 for fp32):
  ``K_pool[num_blocks][Hkv][D // X][B][X]`` and ``V_pool[num_blocks][Hkv][D][B]``;
  token t of a sequence lives in physical block ``bt[t // B]`` at slot
  ``t % B``; slot id = block * B + offset;
* chained FNV-1a-64 over (parent hash as 8 little-endian bytes, then the B
  token ids as int32 little-endian), root parent hash 0; only full blocks are
  hashed;
* a lookup hit needs the same hash, the same token ids and the same physical
  parent block instance (block id and its reuse generation), so a hash
  collision can never share a block;
* free list is FIFO, initialised in the caller's order; popping a cached block
  evicts its hash entry; a release pushes a sequence's blocks to the back,
  last block first, keeping their hash entries (LRU reuse).

``attention`` is the fp64 C routine in ``attention.c``; everything else is
numpy or plain Python.
"""
from __future__ import annotations

import ctypes
import os
import struct
import subprocess
from collections import deque

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_LIB = None

# ----------------------------------------------------------------------------
# build / load of the C part
# ----------------------------------------------------------------------------


def build(force: bool = True) -> str:
    """Compile attention.c into liboracle.so with gcc (OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        src = os.path.join(_HERE, "attention.c")
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_attention.restype = ctypes.c_int
        lib.oracle_attention.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]
        _LIB = lib
    return _LIB


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# ----------------------------------------------------------------------------
# element conversion (exact)
# ----------------------------------------------------------------------------


def to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored elements to float32 ('bf16' = raw uint16 bits)."""
    if dtype == "bf16":
        return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype}")


def storage_dtype(dtype: str):
    return {"bf16": np.uint16, "f32": np.float32}[dtype]


def chunk_elems(dtype: str) -> int:
    """X: elements per 16-byte chunk of the K layout."""
    return 16 // np.dtype(storage_dtype(dtype)).itemsize


# ----------------------------------------------------------------------------
# pool: allocation of empty pools, scatter, gather
# ----------------------------------------------------------------------------


def empty_pools(num_blocks, num_kv_heads, head_dim, block_size, dtype, fill=None):
    X = chunk_elems(dtype)
    if head_dim % X:
        raise ValueError("head_dim must be a multiple of the 16-byte chunk")
    sd = storage_dtype(dtype)
    kp = np.zeros((num_blocks, num_kv_heads, head_dim // X, block_size, X), dtype=sd)
    vp = np.zeros((num_blocks, num_kv_heads, head_dim, block_size), dtype=sd)
    if fill is not None:
        kp[...] = fill
        vp[...] = fill
    return kp, vp


def scatter(k_pool, v_pool, k_new, v_new, slots):
    """Write new tokens into the pools (bit copy). slot -1 = skip.

    k_new, v_new: [n, Hkv, D] in storage dtype; slots: [n] int.
    """
    nb, hkv, dx, B, X = k_pool.shape
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots >= 0
    b = slots[keep] // B
    o = slots[keep] % B
    kn = np.asarray(k_new)[keep]
    vn = np.asarray(v_new)[keep]
    k_pool[b, :, :, o, :] = kn.reshape(kn.shape[0], hkv, dx, X)
    v_pool[b, :, :, o] = vn


def gather(k_pool, v_pool, block_table_row, ctx):
    """Dense K, V [ctx, Hkv, D] of one sequence, read through its block table."""
    nb, hkv, dx, B, X = k_pool.shape
    t = np.arange(ctx, dtype=np.int64)
    bt = np.asarray(block_table_row, dtype=np.int64)
    b = bt[t // B]
    if ctx and (b.min() < 0 or b.max() >= nb):
        raise ValueError("block table points outside the pool")
    o = t % B
    k = k_pool[b, :, :, o, :].reshape(ctx, hkv, dx * X)
    v = v_pool[b, :, :, o]
    return k, v


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------


def attention(q, k_seqs, v_seqs, qsl, num_q_heads, num_kv_heads, scale, sinks=None,
              dtype="f32", threads=None):
    """fp64 attention over gathered K/V (see attention.c).

    q: [total_rows, Hq, D] storage dtype; k_seqs/v_seqs: lists of [ctx_s, Hkv, D];
    qsl: [S+1]; sinks: [Hq] float32 or None. Returns float64 [total_rows, Hq, D].
    """
    q32 = np.ascontiguousarray(to_f32(q, dtype))
    D = q32.shape[-1]
    ctxs = [int(k.shape[0]) for k in k_seqs]
    key_start = np.zeros(len(ctxs) + 1, dtype=np.int64)
    key_start[1:] = np.cumsum(ctxs)
    if len(k_seqs):
        k32 = np.ascontiguousarray(np.concatenate([to_f32(k, dtype).reshape(-1, num_kv_heads, D) for k in k_seqs]))
        v32 = np.ascontiguousarray(np.concatenate([to_f32(v, dtype).reshape(-1, num_kv_heads, D) for v in v_seqs]))
    else:
        k32 = np.zeros((0, num_kv_heads, D), np.float32)
        v32 = k32
    qsl = np.ascontiguousarray(np.asarray(qsl, dtype=np.int32))
    out = np.zeros((int(qsl[-1]), num_q_heads, D), dtype=np.float64)
    sk = None if sinks is None else np.ascontiguousarray(np.asarray(sinks, dtype=np.float32))
    rc = _lib().oracle_attention(
        q32.ctypes.data, k32.ctypes.data, v32.ctypes.data, key_start.ctypes.data, qsl.ctypes.data,
        len(ctxs), num_q_heads, num_kv_heads, D, float(scale),
        None if sk is None else sk.ctypes.data, out.ctypes.data,
        int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_attention: inconsistent sizes")
    return out


def paged_attention(q, k_pool, v_pool, block_tables, context_lens, qsl, num_q_heads,
                    num_kv_heads, scale, sinks=None, dtype="f32", threads=None):
    """Gather every sequence through its block table, then attention()."""
    ks, vs = [], []
    for s, ctx in enumerate(context_lens):
        k, v = gather(k_pool, v_pool, block_tables[s], int(ctx))
        ks.append(k)
        vs.append(v)
    return attention(q, ks, vs, qsl, num_q_heads, num_kv_heads, scale, sinks, dtype, threads)


# ----------------------------------------------------------------------------
# block allocation with chained-hash prefix sharing
# ----------------------------------------------------------------------------

FNV64_OFFSET = 0xCBF29CE484222325
FNV64_PRIME = 0x100000001B3
_MASK64 = (1 << 64) - 1


def fnv1a64(data: bytes, h: int = FNV64_OFFSET) -> int:
    """FNV-1a, 64-bit (Fowler/Noll/Vo): per byte, xor then multiply."""
    for byte in data:
        h ^= byte
        h = (h * FNV64_PRIME) & _MASK64
    return h


def block_hash(parent_hash: int, tokens) -> int:
    data = struct.pack("<Q", parent_hash) + struct.pack("<%di" % len(tokens), *[int(t) for t in tokens])
    return fnv1a64(data)


class OutOfBlocks(Exception):
    pass


class Allocator:
    """Block pool with FIFO free list, refcounts and chained-hash sharing."""

    def __init__(self, num_blocks: int, block_size: int, initial_free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if initial_free_order is None else [int(b) for b in initial_free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("initial_free_order must be a permutation of 0..num_blocks-1")
        self.B = block_size
        self.n = num_blocks
        self.free = deque(order)
        self.in_free = [True] * num_blocks
        self.ref = [0] * num_blocks
        self.gen = [0] * num_blocks
        self.blk_hash = [None] * num_blocks       # hash under which the block is registered
        self.table = {}                             # hash -> (block, parent_id, parent_gen, tokens)
        self.seqs = {}                              # seq -> dict(tokens, blocks, hashes)
        self.hash_fn = block_hash                   # replaceable by tests (collision injection)

    # -- helpers ---------------------------------------------------------------
    def _pop(self):
        b = self.free.popleft()
        self.in_free[b] = False
        h = self.blk_hash[b]
        if h is not None:
            del self.table[h]
            self.blk_hash[b] = None
        self.gen[b] += 1
        self.ref[b] = 1
        return b

    def _register(self, b, h, parent, tokens):
        if h in self.table:
            return
        pid, pgen = (-1, -1) if parent is None else (parent, self.gen[parent])
        self.table[h] = (b, pid, pgen, tuple(int(t) for t in tokens))
        self.blk_hash[b] = h

    # -- API -------------------------------------------------------------------
    def alloc(self, seq_id: int, new_tokens, max_blocks: int):
        """Append tokens to a sequence. Returns (block_table_row, num_blocks, ctx, slot_mapping).

        Raises OutOfBlocks (state unchanged) when the free list is too short and
        ValueError when the sequence would need more than max_blocks blocks.
        """
        B = self.B
        new_tokens = [int(t) for t in new_tokens]
        st = self.seqs.get(seq_id)
        tokens = [] if st is None else st["tokens"]
        blocks = [] if st is None else st["blocks"]
        hashes = [] if st is None else st["hashes"]
        n0 = len(tokens)
        n1 = n0 + len(new_tokens)
        nb0 = -(-n0 // B)
        nb1 = -(-n1 // B)
        if nb1 > max_blocks:
            raise ValueError("sequence needs more blocks than max_blocks")
        all_tokens = tokens + new_tokens

        # phase 1 (read only): hits can only form an unbroken run of full new
        # blocks starting at a block boundary
        hits = []
        if n0 % B == 0:
            parent_hash = hashes[-1] if hashes else 0
            parent = blocks[-1] if blocks else None
            for j in range(nb0, nb1):
                blk_tokens = all_tokens[j * B:(j + 1) * B]
                if len(blk_tokens) < B:
                    break
                h = self.hash_fn(parent_hash, blk_tokens)
                e = self.table.get(h)
                if e is None:
                    break
                b, pid, pgen, etok = e
                want = (-1, -1) if parent is None else (parent, self.gen[parent])
                if (pid, pgen) != want or etok != tuple(blk_tokens):
                    break
                hits.append((b, h))
                parent_hash, parent = h, b
        n_revive = sum(1 for b, _ in hits if self.in_free[b])
        n_pop = (nb1 - nb0) - len(hits)
        if n_pop > len(self.free) - n_revive:
            raise OutOfBlocks("pool exhausted")

        # phase 2: commit
        st = self.seqs.setdefault(seq_id, {"tokens": [], "blocks": [], "hashes": []})
        slots = []
        # fill the existing partial block
        if n0 % B:
            b = st["blocks"][-1]
            take = min(B - n0 % B, len(new_tokens))
            slots += [b * B + (n0 % B) + i for i in range(take)]
            if (n0 % B) + take == B:
                j = nb0 - 1
                ph = st["hashes"][-1] if st["hashes"] else 0
                h = self.hash_fn(ph, all_tokens[j * B:(j + 1) * B])
                st["hashes"].append(h)
                self._register(b, h, st["blocks"][j - 1] if j > 0 else None, all_tokens[j * B:(j + 1) * B])
        for b, h in hits:
            if self.in_free[b]:
                self.free.remove(b)
                self.in_free[b] = False
            self.ref[b] += 1
            st["blocks"].append(b)
            st["hashes"].append(h)
            slots += [-1] * B
        for j in range(nb0 + len(hits), nb1):
            b = self._pop()
            blk_tokens = all_tokens[j * B:(j + 1) * B]
            first = max(n0, j * B)
            slots += [b * B + (t - j * B) for t in range(first, min(n1, (j + 1) * B))]
            parent = st["blocks"][-1] if st["blocks"] else None
            st["blocks"].append(b)
            if len(blk_tokens) == B:
                ph = st["hashes"][-1] if st["hashes"] else 0
                h = self.hash_fn(ph, blk_tokens)
                st["hashes"].append(h)
                self._register(b, h, parent, blk_tokens)
        st["tokens"] = all_tokens
        row = st["blocks"] + [-1] * (max_blocks - len(st["blocks"]))
        return row, len(st["blocks"]), n1, slots

    def release(self, seq_id: int):
        st = self.seqs.pop(seq_id, None)
        if st is None:
            raise KeyError(seq_id)
        for b in reversed(st["blocks"]):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
                self.in_free[b] = True

    def stats(self):
        free = len(self.free)
        cached = sum(1 for b in self.free if self.blk_hash[b] is not None)
        live = sum(1 for r in self.ref if r > 0)
        return free, cached, live
