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
        for fn in (lib.oracle_attention, lib.oracle_attention_kv64):
            fn.restype = ctypes.c_int
            fn.argtypes = [
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]
        lib.oracle_attention_masked.restype = ctypes.c_int
        lib.oracle_attention_masked.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32]
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


def gather(k_pool, v_pool, block_table_row, ctx, dropped_nan=False):
    """Dense K, V [ctx, Hkv, D] of one sequence, read through its block table.
    dropped_nan: table entries -1 (blocks freed below a sliding window) give
    NaN rows instead of an error."""
    nb, hkv, dx, B, X = k_pool.shape
    t = np.arange(ctx, dtype=np.int64)
    bt = np.asarray(block_table_row, dtype=np.int64)
    b = bt[t // B]
    gone = b < 0 if dropped_nan else np.zeros(ctx, dtype=bool)
    if ctx and (b[~gone].min(initial=0) < 0 or b.max(initial=0) >= nb):
        raise ValueError("block table points outside the pool")
    b = np.where(gone, 0, b)
    o = t % B
    k = k_pool[b, :, :, o, :].reshape(ctx, hkv, dx * X)
    v = v_pool[b, :, :, o]
    if gone.any():
        nan = np.uint16(0x7FC0) if k.dtype == np.uint16 else np.float32(np.nan)
        k = k.copy()
        v = v.copy()
        k[gone] = nan
        v[gone] = nan
    return k, v


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------


def attention(q, k_seqs, v_seqs, qsl, num_q_heads, num_kv_heads, scale, sinks=None,
              dtype="f32", threads=None, tree_mask=None, window=0):
    """fp64 attention over gathered K/V (see attention.c).

    q: [total_rows, Hq, D] storage dtype; k_seqs/v_seqs: lists of [ctx_s, Hkv, D];
    qsl: [S+1]; sinks: [Hq] float32 or None; tree_mask: [total_rows] uint32 or
    None (causal); window: sliding window in keys, 0 = none.
    Returns float64 [total_rows, Hq, D].
    """
    kv64 = dtype in ("fp8", "fp4")   # K/V come as float64 dequantized values; q is bf16
    q32 = np.ascontiguousarray(to_f32(q, "bf16" if kv64 else dtype))
    D = q32.shape[-1]
    ctxs = [int(k.shape[0]) for k in k_seqs]
    key_start = np.zeros(len(ctxs) + 1, dtype=np.int64)
    key_start[1:] = np.cumsum(ctxs)
    conv = (lambda a: np.asarray(a, dtype=np.float64)) if kv64 else (lambda a: to_f32(a, dtype))
    if len(k_seqs):
        k32 = np.ascontiguousarray(np.concatenate([conv(k).reshape(-1, num_kv_heads, D) for k in k_seqs]))
        v32 = np.ascontiguousarray(np.concatenate([conv(v).reshape(-1, num_kv_heads, D) for v in v_seqs]))
    else:
        k32 = np.zeros((0, num_kv_heads, D), np.float64 if kv64 else np.float32)
        v32 = k32
    qsl = np.ascontiguousarray(np.asarray(qsl, dtype=np.int32))
    out = np.zeros((int(qsl[-1]), num_q_heads, D), dtype=np.float64)
    sk = None if sinks is None else np.ascontiguousarray(np.asarray(sinks, dtype=np.float32))
    nthr = int(threads or default_threads())
    if tree_mask is None and not window:
        fn = _lib().oracle_attention_kv64 if kv64 else _lib().oracle_attention
        rc = fn(
            q32.ctypes.data, k32.ctypes.data, v32.ctypes.data, key_start.ctypes.data, qsl.ctypes.data,
            len(ctxs), num_q_heads, num_kv_heads, D, float(scale),
            None if sk is None else sk.ctypes.data, out.ctypes.data, nthr)
    else:
        tm = None
        if tree_mask is not None:
            tm = np.ascontiguousarray(np.asarray(tree_mask, dtype=np.uint32))
            if tm.shape != (int(qsl[-1]),):
                raise ValueError("tree_mask needs one word per query row")
        rc = _lib().oracle_attention_masked(
            q32.ctypes.data, k32.ctypes.data, v32.ctypes.data, int(kv64), key_start.ctypes.data,
            qsl.ctypes.data, len(ctxs), num_q_heads, num_kv_heads, D, float(scale),
            None if sk is None else sk.ctypes.data, None if tm is None else tm.ctypes.data, int(window),
            out.ctypes.data, nthr)
    if rc != 0:
        raise ValueError("oracle_attention: inconsistent sizes")
    return out


def paged_attention(q, k_pool, v_pool, block_tables, context_lens, qsl, num_q_heads,
                    num_kv_heads, scale, sinks=None, dtype="f32", threads=None, tree_mask=None, window=0):
    """Gather every sequence through its block table, then attention()."""
    ks, vs = [], []
    dropped = bool(window)   # blocks below a sliding window may be freed (-1)
    for s, ctx in enumerate(context_lens):
        if dtype == "fp8":
            k, v = fp8_gather(k_pool, v_pool, block_tables[s], int(ctx), dropped)
        elif dtype == "fp4":
            k, v = fp4_gather(k_pool, v_pool, block_tables[s], int(ctx), dropped)
        else:
            k, v = gather(k_pool, v_pool, block_tables[s], int(ctx), dropped)
        ks.append(k)
        vs.append(v)
    return attention(q, ks, vs, qsl, num_q_heads, num_kv_heads, scale, sinks, dtype, threads,
                     tree_mask=tree_mask, window=window)


# ----------------------------------------------------------------------------
# 8-bit pools: FP8 E4M3 codes with one float32 scale per (token, KV head)
# ----------------------------------------------------------------------------
#
# The pages name 8-bit KV codecs but define none (TensorSharp "高级功能",
# section "内存优化": quantized paged KV blocks). The reading used here:
#
# * each (token, KV head) row x of D values (bf16) gets a scale
#   s = amax / 448 in float32 (amax = max |x|, 448 the largest E4M3 value), and
#   codes c = E4M3(round to nearest even, x / s clamped to [-448, 448]), the
#   division in float32; a row of zeros has s = 0 and all codes 0;
# * the stored value is decode(c) * s;
# * E4M3 is the OCP 8-bit floating-point format E4M3FN: 1 sign bit, 4 exponent
#   bits with bias 7, 3 mantissa bits, subnormals at exponent 0, no infinities,
#   NaN only at S.1111.111, largest finite value 448.
#
# Layout of a (block, KV head) tile: 16*D code bytes then 16 float32 scales
# (one per token slot), 16*D + 64 bytes in all; pools are
# uint8 [num_blocks][Hkv][16*D + 64]. Within the codes:
#   K: token t, channel c = 64 p + 32 jj + 8 g + e  ->  byte ((p*4 + g)*16 + t)*16 + jj*8 + e
#   V: token t = 8 h + e, channel c = 16 (2 d + dd) + n  ->  byte (((d*16 + n)*2 + h)*2 + dd)*8 + e

FP8_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """float64 value of every E4M3FN code (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    normal = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = sign * (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, sub, normal)
    return np.where((e == 15) & ((c & 7) == 7), np.nan, val)


_E4M3_POS = e4m3_decode(np.arange(0x7F))   # codes 0x00 .. 0x7E, ascending values


def e4m3_encode(x) -> np.ndarray:
    """Codes of float values |x| <= 448 by round to nearest, ties to the even
    code (even mantissa); the sign bit follows x (negative zero keeps it)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > FP8_MAX):
        raise ValueError("e4m3_encode needs finite |x| <= 448")
    a = np.abs(x)
    hi = np.searchsorted(_E4M3_POS, a, side="left").clip(0, 0x7E)   # first code with value >= a
    lo = (hi - 1).clip(0, 0x7E)
    dlo = a - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(a == _E4M3_POS[hi], hi, np.where(pick_hi, hi, lo))
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def fp8_quantize_rows(x_bf16):
    """Rows [..., D] of bf16 bits -> (codes uint8 [..., D], scales float32 [...])."""
    x = to_f32(x_bf16, "bf16")
    amax = np.max(np.abs(x), axis=-1)
    s = (amax.astype(np.float32) / np.float32(FP8_MAX)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    r = (x / safe[..., None]).astype(np.float32)
    r = np.clip(r, np.float32(-FP8_MAX), np.float32(FP8_MAX))
    codes = e4m3_encode(r)
    codes = np.where((s > 0)[..., None], codes, np.uint8(0)).astype(np.uint8)
    return codes, s


def fp8_dequantize(codes, scales) -> np.ndarray:
    """float64 values decode(c) * s."""
    return e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[..., None]


def _fp8_k_offsets(D):
    """Byte offset of (token t, channel c) in the code area of a K tile: [16, D]."""
    t = np.arange(16)[:, None]
    c = np.arange(D)[None, :]
    p, jj, g, e = c // 64, (c // 32) % 2, (c // 8) % 4, c % 8
    return ((p * 4 + g) * 16 + t) * 16 + jj * 8 + e


def _fp8_v_offsets(D):
    """Byte offset of (token t, channel c) in the code area of a V tile: [16, D]."""
    t = np.arange(16)[:, None]
    c = np.arange(D)[None, :]
    dt, n = c // 16, c % 16
    d, dd = dt // 2, dt % 2
    h, e = t // 8, t % 8
    return (((d * 16 + n) * 2 + h) * 2 + dd) * 8 + e


def fp8_empty_pools(num_blocks, num_kv_heads, head_dim, fill=None):
    if head_dim % 64:
        raise ValueError("8-bit pools need head_dim a multiple of 64")
    tile = 16 * head_dim + 64
    kp = np.zeros((num_blocks, num_kv_heads, tile), dtype=np.uint8)
    vp = np.zeros((num_blocks, num_kv_heads, tile), dtype=np.uint8)
    if fill is not None:
        kp[...] = fill
        vp[...] = fill
    return kp, vp


def fp8_scatter(k_pool, v_pool, k_new_bf16, v_new_bf16, slots):
    """Quantize new tokens ([n, Hkv, D] bf16 bits) and write codes and scales
    at their slots (-1 = skip)."""
    nb, hkv, tile = k_pool.shape
    D = (tile - 64) // 16
    offk, offv = _fp8_k_offsets(D), _fp8_v_offsets(D)
    kc, ks = fp8_quantize_rows(k_new_bf16)
    vc, vs = fp8_quantize_rows(v_new_bf16)
    for i, slot in enumerate(np.asarray(slots, dtype=np.int64)):
        if slot < 0:
            continue
        b, o = int(slot // 16), int(slot % 16)
        for h in range(hkv):
            k_pool[b, h, offk[o]] = kc[i, h]
            v_pool[b, h, offv[o]] = vc[i, h]
            k_pool[b, h, 16 * D + 4 * o:16 * D + 4 * o + 4] = np.frombuffer(ks[i, h].tobytes(), np.uint8)
            v_pool[b, h, 16 * D + 4 * o:16 * D + 4 * o + 4] = np.frombuffer(vs[i, h].tobytes(), np.uint8)


def fp8_gather(k_pool, v_pool, block_table_row, ctx, dropped_nan=False):
    """Dequantized float64 K, V [ctx, Hkv, D] of one sequence (dropped_nan as
    for gather)."""
    nb, hkv, tile = k_pool.shape
    D = (tile - 64) // 16
    offk, offv = _fp8_k_offsets(D), _fp8_v_offsets(D)
    bt = np.asarray(block_table_row, dtype=np.int64)
    k = np.zeros((ctx, hkv, D))
    v = np.zeros((ctx, hkv, D))
    for t in range(ctx):
        b, o = int(bt[t // 16]), t % 16
        if b < 0 and dropped_nan:
            k[t] = np.nan
            v[t] = np.nan
            continue
        if b < 0 or b >= nb:
            raise ValueError("block table points outside the pool")
        sk = k_pool[b, :, 16 * D + 4 * o:16 * D + 4 * o + 4].copy().view(np.float32)[:, 0]
        sv = v_pool[b, :, 16 * D + 4 * o:16 * D + 4 * o + 4].copy().view(np.float32)[:, 0]
        k[t] = fp8_dequantize(k_pool[b][:, offk[o]], sk)
        v[t] = fp8_dequantize(v_pool[b][:, offv[o]], sv)
    return k, v


# ----------------------------------------------------------------------------
# 4-bit pools: FP4 E2M1 codes with one float32 scale per (token, KV head)
# ----------------------------------------------------------------------------
#
# The same page's KV block codec also has a 4-bit (and a 2-bit) setting, which
# brings a block to a quarter of its 16-bit size; again no format is given.
# The 4-bit reading here takes the OCP FP4 E2M1 element format (the format of
# the MXFP4 weights the same page lists among its native quantized types): a sign bit,
# two exponent bits with bias 1, one mantissa bit; magnitudes 0, 0.5, 1, 1.5,
# 2, 3, 4, 6; no infinities or NaN. As for 8 bits: s = amax / 6 (float32),
# codes = E2M1(x / s) with x / s in float32 clamped to [-6, 6], nearest code,
# ties to the even code; zero rows have s = 0 and zero codes.
#
# Tile of a (block, KV head): 8 * D code bytes (two codes a byte, the even
# nibble index in the low half), then the 16 tokens' float32 scales. Nibble
# index of token t, channel c:
#   K: c = 32 j + 8 g + e  at  ((g * 16 + t) * (D / 32) + j) * 8 + e
#   V: t = 8 h + e, c = 16 dt + n  at  ((n * 2 + h) * (D / 16) + dt) * 8 + e

FP4_MAX = 6.0


def e2m1_decode(codes) -> np.ndarray:
    """float64 value of every E2M1 code (low 4 bits)."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 1).astype(np.float64)
    normal = (1.0 + m / 2.0) * np.exp2(e.astype(np.float64) - 1.0)
    sub = m * 0.5
    return sign * np.where(e == 0, sub, normal)


_E2M1_POS = e2m1_decode(np.arange(8))   # codes 0 .. 7, ascending magnitudes


def e2m1_encode(x) -> np.ndarray:
    """Codes of float values |x| <= 6 by round to nearest, ties to the even
    code (mantissa bit 0); the sign bit follows x (negative zero keeps it)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > FP4_MAX):
        raise ValueError("e2m1_encode needs finite |x| <= 6")
    a = np.abs(x)
    hi = np.searchsorted(_E2M1_POS, a, side="left").clip(0, 7)
    lo = (hi - 1).clip(0, 7)
    dlo = a - _E2M1_POS[lo]
    dhi = _E2M1_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(a == _E2M1_POS[hi], hi, np.where(pick_hi, hi, lo))
    return (code | np.where(np.signbit(x), 0x8, 0)).astype(np.uint8)


def fp4_quantize_rows(x_bf16):
    """Rows [..., D] of bf16 bits -> (codes uint8 [..., D] one code each, scales float32 [...])."""
    x = to_f32(x_bf16, "bf16")
    amax = np.max(np.abs(x), axis=-1)
    s = (amax.astype(np.float32) / np.float32(FP4_MAX)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    r = (x / safe[..., None]).astype(np.float32)
    r = np.clip(r, np.float32(-FP4_MAX), np.float32(FP4_MAX))
    codes = e2m1_encode(r)
    codes = np.where((s > 0)[..., None], codes, np.uint8(0)).astype(np.uint8)
    return codes, s


def fp4_dequantize(codes, scales) -> np.ndarray:
    """float64 values decode(c) * s."""
    return e2m1_decode(codes) * np.asarray(scales, dtype=np.float64)[..., None]


def _fp4_k_nibbles(D):
    """Nibble index of (token t, channel c) in the code area of a K tile: [16, D]."""
    t = np.arange(16)[:, None]
    c = np.arange(D)[None, :]
    j, g, e = c // 32, (c // 8) % 4, c % 8
    return ((g * 16 + t) * (D // 32) + j) * 8 + e


def _fp4_v_nibbles(D):
    """Nibble index of (token t, channel c) in the code area of a V tile: [16, D]."""
    t = np.arange(16)[:, None]
    c = np.arange(D)[None, :]
    dt, n = c // 16, c % 16
    h, e = t // 8, t % 8
    return ((n * 2 + h) * (D // 16) + dt) * 8 + e


def fp4_empty_pools(num_blocks, num_kv_heads, head_dim, fill=None):
    if head_dim % 64:
        raise ValueError("4-bit pools need head_dim a multiple of 64")
    tile = 8 * head_dim + 64
    kp = np.zeros((num_blocks, num_kv_heads, tile), dtype=np.uint8)
    vp = np.zeros((num_blocks, num_kv_heads, tile), dtype=np.uint8)
    if fill is not None:
        kp[...] = fill
        vp[...] = fill
    return kp, vp


def _fp4_put(pool, blocks, offs, nibbles, codes, scales):
    """Write tokens' codes ([m, Hkv, D], nibble index nibbles [m, D] within
    the tile) and scales ([m, Hkv]) into tiles pool[blocks[i], h] at token
    offsets offs[i]. Each nibble is cleared, then set (ufunc.at applies every
    index, repeated bytes included, so two tokens sharing a byte both land)."""
    m, hkv, D = codes.shape
    shape = (m, hkv, D)
    bi = np.broadcast_to(blocks[:, None, None], shape)
    hi = np.broadcast_to(np.arange(hkv)[None, :, None], shape)
    by = np.broadcast_to((nibbles // 2)[:, None, :], shape)
    sh = np.broadcast_to((4 * (nibbles % 2))[:, None, :], shape).astype(np.uint8)
    np.bitwise_and.at(pool, (bi, hi, by), (~(np.uint8(0xF) << sh)).astype(np.uint8))
    np.bitwise_or.at(pool, (bi, hi, by), (codes.astype(np.uint8) << sh).astype(np.uint8))
    sb = np.ascontiguousarray(scales.astype(np.float32)).view(np.uint8).reshape(m, hkv, 4)
    col = (8 * D + 4 * offs)[:, None, None] + np.arange(4)[None, None, :]
    pool[blocks[:, None, None], np.arange(hkv)[None, :, None], col] = sb


def fp4_scatter(k_pool, v_pool, k_new_bf16, v_new_bf16, slots, chunk=2048):
    """Quantize new tokens ([n, Hkv, D] bf16 bits) and write codes and scales
    at their slots (-1 = skip)."""
    nb, hkv, tile = k_pool.shape
    D = (tile - 64) // 8
    nk, nv = _fp4_k_nibbles(D), _fp4_v_nibbles(D)
    slots = np.asarray(slots, dtype=np.int64)
    for a in range(0, slots.size, chunk):
        sl = slots[a:a + chunk]
        keep = sl >= 0
        if not keep.any():
            continue
        kc, ks = fp4_quantize_rows(np.asarray(k_new_bf16[a:a + chunk])[keep])
        vc, vs = fp4_quantize_rows(np.asarray(v_new_bf16[a:a + chunk])[keep])
        b, o = sl[keep] // 16, sl[keep] % 16
        _fp4_put(k_pool, b, o, nk[o], kc, ks)
        _fp4_put(v_pool, b, o, nv[o], vc, vs)


def _fp4_take(pool, blocks, offs, nibbles):
    """Codes [m, Hkv, D] and scales [m, Hkv] (float32) of tokens at offsets
    offs of tiles pool[blocks[i], h]."""
    m = blocks.size
    hkv, D = pool.shape[1], nibbles.shape[1]
    h = np.arange(hkv)[None, :, None]
    by = pool[blocks[:, None, None], h, (nibbles // 2)[:, None, :]].astype(np.int64)
    codes = np.where((nibbles % 2)[:, None, :] == 1, by >> 4, by & 0xF)
    col = (8 * D + 4 * offs)[:, None, None] + np.arange(4)[None, None, :]
    sc = np.ascontiguousarray(pool[blocks[:, None, None], h, col]).view(np.float32).reshape(m, hkv)
    return codes, sc


def fp4_gather(k_pool, v_pool, block_table_row, ctx, dropped_nan=False):
    """Dequantized float64 K, V [ctx, Hkv, D] of one sequence (dropped_nan as
    for gather)."""
    nb, hkv, tile = k_pool.shape
    D = (tile - 64) // 8
    nk, nv = _fp4_k_nibbles(D), _fp4_v_nibbles(D)
    bt = np.asarray(block_table_row, dtype=np.int64)
    t = np.arange(ctx)
    b, o = bt[t // 16], t % 16
    gone = b < 0
    if (gone.any() and not dropped_nan) or np.any(b >= nb):
        raise ValueError("block table points outside the pool")
    b = np.where(gone, 0, b)
    k = fp4_dequantize(*_fp4_take(k_pool, b, o, nk[o]))
    v = fp4_dequantize(*_fp4_take(v_pool, b, o, nv[o]))
    k[gone] = np.nan
    v[gone] = np.nan
    return k, v


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
        dropped = st is not None and st.get("dropped", False)
        if n0 % B == 0 and not dropped:
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
        st = self.seqs.setdefault(seq_id, {"tokens": [], "blocks": [], "hashes": [], "dropped": False})
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
                if not st["dropped"]:
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
                if not st["dropped"]:
                    self._register(b, h, parent, blk_tokens)
        st["tokens"] = all_tokens
        row = st["blocks"] + [-1] * (max_blocks - len(st["blocks"]))
        return row, len(st["blocks"]), n1, slots

    def release(self, seq_id: int):
        st = self.seqs.pop(seq_id, None)
        if st is None:
            raise KeyError(seq_id)
        for b in reversed(st["blocks"]):
            if b < 0:
                continue
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
                self.in_free[b] = True

    def drop_prefix(self, seq_id: int, first_kept: int):
        """Free the blocks wholly below position first_kept (a sliding window's
        rows never see them again); they read -1 in the table from now on, and
        the sequence neither shares nor registers blocks afterwards."""
        st = self.seqs.get(seq_id)
        if st is None:
            raise KeyError(seq_id)
        if first_kept < 0:
            raise ValueError("first_kept must be >= 0")
        upto = min(first_kept, len(st["tokens"])) // self.B
        for j in reversed(range(upto)):
            b = st["blocks"][j]
            if b < 0:
                continue
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
                self.in_free[b] = True
            st["blocks"][j] = -1
            st["dropped"] = True

    def truncate(self, seq_id: int, new_len: int):
        """Roll a sequence back to its first new_len tokens (rejected drafts,
        TensorFold page, GPU accept kernel section: a rollback restores every
        state after the accepted path, the KV cache included).

        Blocks wholly past new_len go back as release() returns them (last
        block first, hash entries kept). When new_len ends inside a block that
        was full, the slots after it will be written again: a block the
        sequence alone holds loses its hash entry and starts a new reuse
        generation (so no chain through its old contents can be followed); a
        block other sequences also hold is replaced by a fresh block popped
        from the free list, and (src, dst) is returned for the caller to copy
        on the device before writing to it. Returns (src, dst) or (-1, -1).
        Raises OutOfBlocks with the state unchanged when a copy needs a block
        and none would be free.
        """
        st = self.seqs.get(seq_id)
        if st is None:
            raise KeyError(seq_id)
        n = len(st["tokens"])
        if not 0 <= new_len <= n:
            raise ValueError("new_len must lie in 0 .. context length")
        B = self.B
        keep = -(-new_len // B)
        drop = st["blocks"][keep:]
        tail_was_full = new_len % B != 0 and len(st["hashes"]) >= keep
        tail = st["blocks"][keep - 1] if tail_was_full else None
        if tail_was_full and tail < 0:
            raise ValueError("new_len ends inside a dropped block")
        shared = tail_was_full and self.ref[tail] > 1
        if shared:
            freed = sum(1 for b in drop if b >= 0 and self.ref[b] == 1)
            if len(self.free) + freed < 1:
                raise OutOfBlocks("no free block for the copy of a shared tail block")
        for b in reversed(drop):
            if b < 0:
                continue
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
                self.in_free[b] = True
        st["blocks"] = st["blocks"][:keep]
        st["hashes"] = st["hashes"][:new_len // B]
        st["tokens"] = st["tokens"][:new_len]
        if not tail_was_full:
            return -1, -1
        if shared:
            self.ref[tail] -= 1
            dst = self._pop()
            st["blocks"][keep - 1] = dst
            return tail, dst
        h = self.blk_hash[tail]
        if h is not None:
            del self.table[h]
            self.blk_hash[tail] = None
        self.gen[tail] += 1
        return -1, -1

    def table_row(self, seq_id: int, max_blocks: int):
        st = self.seqs[seq_id]
        return st["blocks"] + [-1] * (max_blocks - len(st["blocks"]))

    def stats(self):
        free = len(self.free)
        cached = sum(1 for b in self.free if self.blk_hash[b] is not None)
        live = sum(1 for r in self.ref if r > 0)
        return free, cached, live


def copy_blocks(k_pool, v_pool, src, dst):
    """Copy whole blocks (every KV head, every slot) src[i] -> dst[i] in both
    pools, in order; the copy a truncate into a shared block asks for."""
    for a, b in zip(np.asarray(src, dtype=np.int64), np.asarray(dst, dtype=np.int64)):
        k_pool[b] = k_pool[a]
        v_pool[b] = v_pool[a]


# ----------------------------------------------------------------------------
# tree verify windows
# ----------------------------------------------------------------------------
#
# TensorFold page, section on the GPU accept kernel: a verify round lays its
# drafts out as a chain or a tree of at most 16 rows, the tree carrying
# alternative paths; the accept step walks from the root along the first child
# whose draft token equals the target model's choice. Window row r's parent is
# parents[r] (a row before r, or -1 for the token before the window).


def tree_masks(parents):
    """Ancestor masks of a window: bit j of masks[r] is set when row j is r or
    one of its ancestors."""
    masks = []
    for r, p in enumerate(parents):
        p = int(p)
        if not -1 <= p < r:
            raise ValueError("a parent must be -1 or an earlier row")
        masks.append((1 << r) | (masks[p] if p >= 0 else 0))
    return np.array(masks, dtype=np.uint32)


def accept_path(parents, draft_tokens, choices, root_choice):
    """Walk the tree: from the root, while some child of the current node has
    draft token equal to the current choice, move to the first such child (in
    row order); the choice is then that row's. choices[r] is the target's
    token after row r; root_choice the target's token after the root.
    Returns (accepted rows in path order, the target's token after the path)."""
    path, cur, want = [], -1, int(root_choice)
    while True:
        nxt = next((r for r in range(len(parents)) if int(parents[r]) == cur and int(draft_tokens[r]) == want), None)
        if nxt is None:
            return path, want
        path.append(nxt)
        cur, want = nxt, int(choices[nxt])


# ----------------------------------------------------------------------------
# QK-norm + RoPE before the scatter-write
# ----------------------------------------------------------------------------
#
# TensorSharp "高级功能" page: for Qwen 3.5/3.6 one kernel applies QK-Norm and
# NeoX RoPE on the prefill path; the batched forward pairs its projection with
# the paged K/V scatter-write. The pages fix no formula beyond those names.
# The reading used here:
#
# * QK-norm: RMSNorm over the head dimension, per (token, head) row:
#   y = x / sqrt(mean(x^2) + eps) * (offset + w), w one weight per dimension
#   (bf16), offset 0 (weights multiply) or 1 (zero-centred weights);
# * NeoX RoPE on the first rotary_dim dimensions: pairs (i, i + rotary_dim/2),
#   i < rotary_dim/2, turned by the angle pos * theta^(-2i/rotary_dim):
#   (a, b) -> (a cos - b sin, b cos + a sin); later dimensions pass through;
# * exact arithmetic, one rounding to bf16 (nearest, ties to even) at the end;
# * K (normed, rotated) and V (as given) then go into the pools at their
#   slots, as the scatter-write puts them.


def f64_to_bf16_bits(x):
    """Round float64 values to bf16 once (nearest, ties to even), raw bits.
    The quantum of x is 2^(e - 8) for x in [2^(e-1), 2^e), at least 2^-133
    (bf16's subnormal step)."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    qexp = np.maximum(e - 8, -133)
    r = np.rint(np.ldexp(x, -qexp))             # np.rint rounds halves to even
    v = np.ldexp(r, qexp).astype(np.float32)    # exact: 8 significant bits fit
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def rms_norm(x, weight, eps, weight_offset=0.0):
    """x [..., D] float64; weight [D] float64 (or None: no weight)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    y = x / np.sqrt(ms + float(eps))
    if weight is not None:
        y = y * (float(weight_offset) + np.asarray(weight, dtype=np.float64))
    return y


def rope_neox(x, positions, theta, rotary_dim):
    """x [n, H, D] float64, positions [n]: NeoX rotation of the first
    rotary_dim dimensions."""
    x = np.array(x, dtype=np.float64)
    half = rotary_dim // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = float(theta) ** (-2.0 * i / rotary_dim)                     # [half]
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None]  # [n, half]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., :half].copy(), x[..., half:rotary_dim].copy()
    x[..., :half] = a * c - b * s
    x[..., half:rotary_dim] = b * c + a * s
    return x


def qknorm_rope(q, k, positions, q_weight, k_weight, eps, theta, rotary_dim, weight_offset=0.0):
    """q [n, Hq, D], k [n, Hkv, D] bf16 bits; weights [D] bf16 bits or None
    (no weight: the normalized row itself). Returns (q_out, k_out) bf16 bits."""
    qw = None if q_weight is None else to_f32(q_weight, "bf16").astype(np.float64)
    kw = None if k_weight is None else to_f32(k_weight, "bf16").astype(np.float64)
    qn = rms_norm(to_f32(q, "bf16"), qw, eps, weight_offset)
    kn = rms_norm(to_f32(k, "bf16"), kw, eps, weight_offset)
    return (f64_to_bf16_bits(rope_neox(qn, positions, theta, rotary_dim)),
            f64_to_bf16_bits(rope_neox(kn, positions, theta, rotary_dim)))


def qknorm_rope_scatter(k_pool, v_pool, q, k, v, positions, slots, q_weight, k_weight, eps, theta,
                        rotary_dim, weight_offset=0.0):
    """The whole producer step: normed, rotated Q is returned; normed,
    rotated K and V are written into the (bf16) pools at the slots."""
    q_out, k_out = qknorm_rope(q, k, positions, q_weight, k_weight, eps, theta, rotary_dim, weight_offset)
    scatter(k_pool, v_pool, k_out, np.asarray(v), slots)
    return q_out
