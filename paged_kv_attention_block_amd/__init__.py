"""Batched attention over a paged KV cache on MI355X (gfx950): Python binding.

Thin ctypes binding over ``libpagedkv.so`` (declared in ``include/pagedkv.h``).
Functions carry the C names and only marshal arguments: torch tensors are
passed by device pointer, shapes become the size arguments, and every step of
the computation runs in the library's HIP kernels. PyTorch supplies device
memory and streams. If the library is missing the import fails: there is no
fallback path.

Pool layout (see the header): with X = 16 bytes / element size,
``K_pool [num_blocks, Hkv, D // X, 16, X]`` and ``V_pool [num_blocks, Hkv, D, 16]``
for float32 and bf16 pools; 8-bit pools (E4M3 codes with a float32 scale per
token and KV head) are ``torch.uint8 [num_blocks, Hkv, 16 * D + 64]`` each and
4-bit pools (E2M1 codes, two a byte, with the same scales) ``torch.uint8
[num_blocks, Hkv, 8 * D + 64]``, both with bf16 queries and bf16 new K/V rows;
the head size the rows carry tells the two apart.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "KV_OK", "KV_EINVAL", "KV_ENOMEM", "KV_EUNSUPPORTED", "KV_EDEVICE", "KV_EINTERNAL",
    "KV_F32", "KV_BF16", "KV_FP8", "KV_FP4", "KVError", "lib_path", "kv_abi_version", "kv_last_error",
    "kv_pool_create", "kv_pool_destroy", "kv_pool_alloc", "kv_pool_release", "kv_pool_stats",
    "kv_pool_set_hash_mask", "kv_pool_truncate", "kv_pool_drop_prefix", "kv_tree_masks", "kv_append_scatter",
    "kv_copy_blocks", "kv_accept_paths", "kv_qknorm_rope_scatter", "paged_attention_workspace_size", "paged_attention_forward",
    "paged_attention_forward_noalloc", "paged_attention_prefix_forward", "paged_attention_append_forward", "paged_attention_masked_forward", "empty_pools", "BLOCK_SIZE",
]

KV_OK, KV_EINVAL, KV_ENOMEM, KV_EUNSUPPORTED, KV_EDEVICE, KV_EINTERNAL = 0, -1, -2, -3, -4, -5
KV_F32, KV_BF16, KV_FP8, KV_FP4 = 0, 1, 2, 3
BLOCK_SIZE = 16

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libpagedkv.so")

if not os.path.exists(lib_path):
    raise ImportError(f"{lib_path} is missing: build it with __graft_entry__.build() "
                      "or python paged_kv_attention_block_amd/build.py")

_lib = ctypes.CDLL(lib_path)

_i32, _i64, _u64, _f32, _p, _sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float,
                                   ctypes.c_void_p, ctypes.c_size_t)
_lib.kv_abi_version.restype = ctypes.c_int
_lib.kv_last_error.restype = ctypes.c_char_p
_lib.kv_pool_create.argtypes = [_i32, _i32, _p, ctypes.POINTER(_p)]
_lib.kv_pool_destroy.argtypes = [_p]
_lib.kv_pool_destroy.restype = None
_lib.kv_pool_alloc.argtypes = [_p, _i64, _p, _i32, _p, _i32, _p, _p, _p]
_lib.kv_pool_release.argtypes = [_p, _i64]
_lib.kv_pool_stats.argtypes = [_p, _p, _p, _p]
_lib.kv_pool_set_hash_mask.argtypes = [_p, _u64]
_lib.kv_pool_truncate.argtypes = [_p, _i64, _i32, _p, _p]
_lib.kv_pool_drop_prefix.argtypes = [_p, _i64, _i32]
_lib.kv_tree_masks.argtypes = [_p, _i32, _p]
_lib.kv_copy_blocks.argtypes = [_p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _p]
_lib.kv_accept_paths.argtypes = [_p, _p, _p, _p, _p, _i32, _p, _p, _p, _p]
_lib.kv_qknorm_rope_scatter.argtypes = [_p, _p, _p, _p, _p, _p, _f32, _f32, _f32, _i32, _p, _i32, _p, _p, _p,
                                        _i32, _i32, _i32, _i32, _i32, _i32, _p]
_lib.kv_append_scatter.argtypes = [_p, _p, _p, _i32, _p, _p, _i32, _i32, _i32, _i32, _i32, _p]
_lib.paged_attention_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32]
_lib.paged_attention_workspace_size.restype = _sz
_lib.paged_attention_forward.argtypes = [
    _p, _p, _p, _i32, _p, _i32, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
    _f32, _p, _p, _p, _sz, _p]
_lib.paged_attention_prefix_forward.argtypes = [
    _p, _p, _p, _i32, _p, _i32, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
    _f32, _p, _i32, _i32, _p, _p, _sz, _p]
_lib.paged_attention_forward_noalloc.argtypes = [
    _p, _p, _p, _i32, _p, _i32, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
    _f32, _p, _p, _p]
_lib.paged_attention_append_forward.argtypes = [
    _p, _p, _p, _p, _p, _p, _i32, _p, _i32, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
    _f32, _p, _p, _p, _sz, _p]
_lib.paged_attention_masked_forward.argtypes = [
    _p, _p, _p, _i32, _p, _i32, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
    _f32, _p, _p, _i32, _p, _p, _sz, _p]
for _name in ("kv_pool_create", "kv_pool_alloc", "kv_pool_release", "kv_pool_stats",
              "kv_pool_set_hash_mask", "kv_pool_truncate", "kv_pool_drop_prefix", "kv_tree_masks",
              "kv_append_scatter", "kv_copy_blocks", "kv_accept_paths", "kv_qknorm_rope_scatter",
              "paged_attention_forward", "paged_attention_forward_noalloc", "paged_attention_prefix_forward",
              "paged_attention_append_forward", "paged_attention_masked_forward"):
    getattr(_lib, _name).restype = ctypes.c_int


class KVError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code
        self.message = message


def _check(rc: int):
    if rc != KV_OK:
        raise KVError(rc, _lib.kv_last_error().decode(errors="replace"))


def kv_abi_version() -> int:
    return _lib.kv_abi_version()


def kv_last_error() -> str:
    return _lib.kv_last_error().decode(errors="replace")


# ---------------------------------------------------------------------------
# host block manager
# ---------------------------------------------------------------------------

class _Pool:
    __slots__ = ("ptr", "num_blocks", "block_size")

    def __init__(self, ptr, num_blocks, block_size):
        self.ptr, self.num_blocks, self.block_size = ptr, num_blocks, block_size

    def __del__(self):
        # at interpreter exit the module's globals may already be cleared
        if getattr(self, "ptr", None) and _lib is not None:
            _lib.kv_pool_destroy(self.ptr)
            self.ptr = None


def kv_pool_create(num_blocks: int, block_size: int = BLOCK_SIZE, initial_free_order=None) -> _Pool:
    out = _p()
    order = None
    if initial_free_order is not None:
        order = np.ascontiguousarray(np.asarray(initial_free_order, dtype=np.int32))
        if order.size != num_blocks:
            raise KVError(KV_EINVAL, "initial_free_order must hold num_blocks entries")
    _check(_lib.kv_pool_create(num_blocks, block_size, None if order is None else order.ctypes.data,
                               ctypes.byref(out)))
    return _Pool(out.value, num_blocks, block_size)


def kv_pool_destroy(pool: _Pool) -> None:
    if pool.ptr:
        _lib.kv_pool_destroy(pool.ptr)
        pool.ptr = None


def kv_pool_alloc(pool: _Pool, seq_id: int, new_token_ids, max_blocks: int):
    """Returns (block_table_row int32[max_blocks], num_blocks, context_len, slot_mapping int32[n])."""
    toks = np.ascontiguousarray(np.asarray(new_token_ids, dtype=np.int32).reshape(-1))
    row = np.empty(max_blocks, dtype=np.int32)
    slots = np.empty(max(1, toks.size), dtype=np.int32)
    nb, ctx = _i32(), _i32()
    _check(_lib.kv_pool_alloc(pool.ptr, seq_id, toks.ctypes.data if toks.size else None, toks.size,
                              row.ctypes.data, max_blocks, ctypes.byref(nb), ctypes.byref(ctx),
                              slots.ctypes.data))
    return row, nb.value, ctx.value, slots[:toks.size]


def kv_pool_release(pool: _Pool, seq_id: int) -> None:
    _check(_lib.kv_pool_release(pool.ptr, seq_id))


def kv_pool_stats(pool: _Pool):
    f, c, l = _i32(), _i32(), _i32()
    _check(_lib.kv_pool_stats(pool.ptr, ctypes.byref(f), ctypes.byref(c), ctypes.byref(l)))
    return f.value, c.value, l.value


def kv_pool_set_hash_mask(pool: _Pool, mask: int) -> None:
    _check(_lib.kv_pool_set_hash_mask(pool.ptr, mask & 0xFFFFFFFFFFFFFFFF))


def kv_pool_truncate(pool: _Pool, seq_id: int, new_len: int):
    """Roll a sequence back to new_len tokens; returns (copy_src, copy_dst), -1 when no copy is needed."""
    a, b = _i32(), _i32()
    _check(_lib.kv_pool_truncate(pool.ptr, seq_id, new_len, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def kv_pool_drop_prefix(pool: _Pool, seq_id: int, first_kept: int) -> None:
    _check(_lib.kv_pool_drop_prefix(pool.ptr, seq_id, first_kept))


def kv_tree_masks(parents) -> np.ndarray:
    """Ancestor masks (uint32 [n]) of one tree window from its parent rows."""
    par = np.ascontiguousarray(np.asarray(parents, dtype=np.int32).reshape(-1))
    out = np.zeros(max(1, par.size), dtype=np.uint32)
    _check(_lib.kv_tree_masks(par.ctypes.data if par.size else out.ctypes.data, par.size, out.ctypes.data))
    return out[:par.size]


# ---------------------------------------------------------------------------
# device entry points (torch tensors in, device pointers out)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return KV_BF16
    if t.dtype == torch.float32:
        return KV_F32
    raise KVError(KV_EUNSUPPORTED, f"unsupported element type {t.dtype}")


def _stream_ptr(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on(stream):
    """Allocation context for buffers a call creates: torch's caching
    allocator ties a block to the stream current at allocation and hands it
    out again, once freed, to later allocations on that stream only. Buffers
    the kernels of `stream` use are therefore allocated on `stream`, so that
    their reuse is ordered after those kernels."""
    import contextlib
    if stream is None:
        return contextlib.nullcontext()
    return _torch().cuda.stream(stream)


def _need(t, name, dtype=None, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise KVError(KV_EINVAL, f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise KVError(KV_EINVAL, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise KVError(KV_EINVAL, f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise KVError(KV_EINVAL, f"{name} must have {ndim} dimensions")
    return t.data_ptr()


def empty_pools(num_blocks: int, num_kv_heads: int, head_dim: int, dtype, device="cuda"):
    """Allocate (K_pool, V_pool) device tensors in the library's layout;
    dtype torch.uint8 or "fp8" gives 8-bit pools, "fp4" 4-bit pools."""
    torch = _torch()
    if isinstance(dtype, str) or dtype == torch.uint8:
        fmt = "fp8" if dtype == torch.uint8 else dtype
        if fmt not in ("fp8", "fp4"):
            raise KVError(KV_EUNSUPPORTED, f"unknown pool format {dtype!r}")
        tile = (16 if fmt == "fp8" else 8) * head_dim + 64
        dtype = torch.uint8
        return (torch.empty((num_blocks, num_kv_heads, tile), dtype=dtype, device=device),
                torch.empty((num_blocks, num_kv_heads, tile), dtype=dtype, device=device))
    X = 16 // torch.empty((), dtype=dtype).element_size()
    k = torch.empty((num_blocks, num_kv_heads, head_dim // X, BLOCK_SIZE, X), dtype=dtype, device=device)
    v = torch.empty((num_blocks, num_kv_heads, head_dim, BLOCK_SIZE), dtype=dtype, device=device)
    return k, v


def _pools(k_pool, v_pool, elem_dtype, hkv, d):
    """Check the pools against the element type of the rows that go with them
    (queries or new K/V) and return (dtype code, num_blocks)."""
    torch = _torch()
    if k_pool.dtype == torch.uint8:
        if elem_dtype != torch.bfloat16:
            raise KVError(KV_EINVAL, "8- and 4-bit pools take bf16 queries and bf16 new K/V rows")
        _need(k_pool, "k_pool", dtype=torch.uint8, ndim=3)
        _need(v_pool, "v_pool", dtype=torch.uint8, ndim=3)
        nb = k_pool.shape[0]
        h = hkv if hkv is not None else k_pool.shape[1]
        for code, tile in ((KV_FP8, 16 * d + 64), (KV_FP4, 8 * d + 64)):
            if tuple(k_pool.shape) == (nb, h, tile) and tuple(v_pool.shape) == (nb, h, tile):
                return code, nb
        raise KVError(KV_EINVAL, f"8-bit pools must be [num_blocks, Hkv, {16 * d + 64}], "
                                 f"4-bit pools [num_blocks, Hkv, {8 * d + 64}]")
    _need(k_pool, "k_pool", dtype=elem_dtype, ndim=5)
    _need(v_pool, "v_pool", dtype=elem_dtype, ndim=4)
    nb = k_pool.shape[0]
    h = hkv if hkv is not None else k_pool.shape[1]
    if tuple(v_pool.shape) != (nb, h, d, BLOCK_SIZE) or k_pool.shape[1] != h or \
            k_pool.shape[2] * k_pool.shape[4] != d or k_pool.shape[3] != BLOCK_SIZE:
        raise KVError(KV_EINVAL, "pool shapes do not match the rows")
    return _dtype_code(k_pool), nb


def kv_append_scatter(k_new, v_new, slot_mapping, k_pool, v_pool, stream=None) -> None:
    """Scatter-write k_new/v_new [n, Hkv, D] into the pools at slot_mapping [n] (int32, -1 = skip);
    8- and 4-bit pools quantize each (token, KV head) row."""
    torch = _torch()
    _need(k_new, "k_new", ndim=3)
    _need(v_new, "v_new", dtype=k_new.dtype, ndim=3)
    _need(slot_mapping, "slot_mapping", dtype=torch.int32, ndim=1)
    n, hkv, d = k_new.shape
    if v_new.shape != k_new.shape or slot_mapping.shape[0] != n:
        raise KVError(KV_EINVAL, "k_new, v_new and slot_mapping sizes disagree")
    code, nb = _pools(k_pool, v_pool, k_new.dtype, hkv, d)
    _check(_lib.kv_append_scatter(k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr(), n,
                                  k_pool.data_ptr(), v_pool.data_ptr(), nb, hkv, d, BLOCK_SIZE,
                                  code, _stream_ptr(stream)))


def kv_copy_blocks(k_pool, v_pool, src, dst, stream=None) -> None:
    """Copy whole blocks src[i] -> dst[i] (device int32 [n]) in both pools."""
    torch = _torch()
    _need(src, "src", dtype=torch.int32, ndim=1)
    _need(dst, "dst", dtype=torch.int32, ndim=1)
    if src.shape != dst.shape:
        raise KVError(KV_EINVAL, "src and dst sizes disagree")
    if k_pool.dtype == torch.uint8:
        # a copy moves whole tiles: an 8-bit tile of (tile - 64) / 16 channels
        # has the byte size of either format's tile
        hkv, d = k_pool.shape[1], (k_pool.shape[2] - 64) // 16
        elem = torch.bfloat16
    else:
        hkv, d, elem = k_pool.shape[1], k_pool.shape[2] * k_pool.shape[4], k_pool.dtype
    code, nb = _pools(k_pool, v_pool, elem, hkv, d)
    _check(_lib.kv_copy_blocks(k_pool.data_ptr(), v_pool.data_ptr(), src.data_ptr(), dst.data_ptr(), src.shape[0],
                               nb, hkv, d, BLOCK_SIZE, code, _stream_ptr(stream)))


def kv_accept_paths(parents, draft_tokens, choices, root_choices, query_start_loc, path=None, path_len=None,
                    bonus=None, stream=None):
    """The accept walk of every sequence's verify window on the device; returns (path, path_len, bonus)."""
    torch = _torch()
    for t, name in ((parents, "parents"), (draft_tokens, "draft_tokens"), (choices, "choices"),
                    (root_choices, "root_choices"), (query_start_loc, "query_start_loc")):
        _need(t, name, dtype=torch.int32, ndim=1)
    rows, S = parents.shape[0], root_choices.shape[0]
    if draft_tokens.shape[0] != rows or choices.shape[0] != rows or query_start_loc.shape[0] != S + 1:
        raise KVError(KV_EINVAL, "parents, draft_tokens, choices, root_choices and query_start_loc disagree")
    with _on(stream):
        if path is None:
            path = torch.empty(rows, dtype=torch.int32, device=parents.device)
        if path_len is None:
            path_len = torch.empty(S, dtype=torch.int32, device=parents.device)
        if bonus is None:
            bonus = torch.empty(S, dtype=torch.int32, device=parents.device)
    for t, name, n in ((path, "path", rows), (path_len, "path_len", S), (bonus, "bonus", S)):
        _need(t, name, dtype=torch.int32, ndim=1)
        if t.shape[0] != n:
            raise KVError(KV_EINVAL, f"{name} has the wrong size")
    _check(_lib.kv_accept_paths(parents.data_ptr(), draft_tokens.data_ptr(), choices.data_ptr(),
                                root_choices.data_ptr(), query_start_loc.data_ptr(), S, path.data_ptr(),
                                path_len.data_ptr(), bonus.data_ptr(), _stream_ptr(stream)))
    return path, path_len, bonus


def kv_qknorm_rope_scatter(q, k, v, positions, slot_mapping, k_pool, v_pool, q_norm_weight=None,
                           k_norm_weight=None, eps: float = 1e-6, weight_offset: float = 0.0,
                           rope_theta: float = 1e6, rotary_dim=None, q_out=None, stream=None):
    """QK-norm + NeoX RoPE of q [n, Hq, D] and k [n, Hkv, D] (bf16), rotated Q returned (q_out), rotated
    K and v written into the bf16 pools at slot_mapping [n] (see pagedkv.h)."""
    torch = _torch()
    _need(q, "q", dtype=torch.bfloat16, ndim=3)
    _need(k, "k", dtype=torch.bfloat16, ndim=3)
    _need(v, "v", dtype=torch.bfloat16, ndim=3)
    _need(positions, "positions", dtype=torch.int32, ndim=1)
    _need(slot_mapping, "slot_mapping", dtype=torch.int32, ndim=1)
    n, hq, d = q.shape
    if k.shape[0] != n or v.shape != k.shape or k.shape[2] != d or positions.shape[0] != n or \
            slot_mapping.shape[0] != n:
        raise KVError(KV_EINVAL, "q, k, v, positions and slot_mapping sizes disagree")
    hkv = k.shape[1]
    code, nb = _pools(k_pool, v_pool, torch.bfloat16, hkv, d)
    for w, name in ((q_norm_weight, "q_norm_weight"), (k_norm_weight, "k_norm_weight")):
        if w is not None:
            _need(w, name, dtype=torch.bfloat16, ndim=1)
            if w.shape[0] != d:
                raise KVError(KV_EINVAL, f"{name} needs head_dim values")
    if q_out is None:
        with _on(stream):
            q_out = torch.empty_like(q)
    _need(q_out, "q_out", dtype=torch.bfloat16, ndim=3)
    if q_out.shape != q.shape:
        raise KVError(KV_EINVAL, "q_out has the wrong shape")
    _check(_lib.kv_qknorm_rope_scatter(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), positions.data_ptr(),
        None if q_norm_weight is None else q_norm_weight.data_ptr(),
        None if k_norm_weight is None else k_norm_weight.data_ptr(), float(eps), float(weight_offset),
        float(rope_theta), d if rotary_dim is None else int(rotary_dim), slot_mapping.data_ptr(), n,
        q_out.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), nb, hq, hkv, d, BLOCK_SIZE, code,
        _stream_ptr(stream)))
    return q_out


def paged_attention_workspace_size(num_seqs: int, total_q_rows: int, num_q_heads: int, head_dim: int,
                                   max_context_len: int) -> int:
    return int(_lib.paged_attention_workspace_size(num_seqs, total_q_rows, num_q_heads, head_dim,
                                                   max_context_len))


def _forward_args(q, k_pool, v_pool, block_tables, context_lens, query_start_loc, max_context_len, sinks, out,
                  workspace, stream):
    torch = _torch()
    _need(q, "q", ndim=3)
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    _need(query_start_loc, "query_start_loc", dtype=torch.int32, ndim=1)
    total, hq, d = q.shape
    code, nb = _pools(k_pool, v_pool, q.dtype, None, d)
    hkv = k_pool.shape[1]
    S = context_lens.shape[0]
    if query_start_loc.shape[0] != S + 1 or block_tables.shape[0] != S:
        raise KVError(KV_EINVAL, "context_lens, query_start_loc and block_tables disagree on num_seqs")
    if sinks is not None:
        _need(sinks, "sinks", dtype=torch.float32, ndim=1)
        if sinks.shape[0] != hq:
            raise KVError(KV_EINVAL, "sinks must hold num_q_heads values")
    if out is None:
        with _on(stream):
            out = torch.empty((total, hq, d), dtype=torch.float32, device=q.device)
    _need(out, "out", dtype=torch.float32, ndim=3)
    if tuple(out.shape) != (total, hq, d):
        raise KVError(KV_EINVAL, "out has the wrong shape")
    need = paged_attention_workspace_size(S, total, hq, d, max_context_len)
    if workspace is None:
        # freed when the call returns: only allocations on `stream` reuse it
        with _on(stream):
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size()
    return S, total, hq, hkv, d, nb, code, out, workspace, ws_bytes


def paged_attention_forward(q, k_pool, v_pool, block_tables, context_lens, query_start_loc, max_q_len: int,
                            max_context_len: int, scale: float, sinks=None, out=None, workspace=None,
                            stream=None):
    """out [total_rows, Hq, D] float32 = attention of q over the paged cache (see pagedkv.h)."""
    S, total, hq, hkv, d, nb, code, out, workspace, ws_bytes = _forward_args(
        q, k_pool, v_pool, block_tables, context_lens, query_start_loc, max_context_len, sinks, out, workspace, stream)
    _check(_lib.paged_attention_forward(
        q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), code, block_tables.data_ptr(),
        block_tables.shape[1], context_lens.data_ptr(), query_start_loc.data_ptr(), S, total, max_q_len,
        max_context_len, hq, hkv, d, BLOCK_SIZE, nb, float(scale),
        None if sinks is None else sinks.data_ptr(), out.data_ptr(), workspace.data_ptr(), ws_bytes,
        _stream_ptr(stream)))
    return out


def paged_attention_prefix_forward(q, k_pool, v_pool, block_tables, context_lens, query_start_loc, max_q_len: int,
                                   max_context_len: int, scale: float, prefix_seqs: int, prefix_tokens: int,
                                   sinks=None, out=None, workspace=None, stream=None):
    """paged_attention_forward for a batch whose first prefix_seqs sequences
    (decode rows) hold their first prefix_tokens positions in the same
    physical blocks (see pagedkv.h); the same bits, shared splits read once
    per group of sequences."""
    S, total, hq, hkv, d, nb, code, out, workspace, ws_bytes = _forward_args(
        q, k_pool, v_pool, block_tables, context_lens, query_start_loc, max_context_len, sinks, out, workspace,
        stream)
    _check(_lib.paged_attention_prefix_forward(
        q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), code, block_tables.data_ptr(),
        block_tables.shape[1], context_lens.data_ptr(), query_start_loc.data_ptr(), S, total, max_q_len,
        max_context_len, hq, hkv, d, BLOCK_SIZE, nb, float(scale),
        None if sinks is None else sinks.data_ptr(), int(prefix_seqs), int(prefix_tokens), out.data_ptr(),
        workspace.data_ptr(), ws_bytes, _stream_ptr(stream)))
    return out


def paged_attention_forward_noalloc(q, k_pool, v_pool, block_tables, context_lens, query_start_loc, max_q_len: int,
                                    max_context_len: int, scale: float, sinks=None, out=None, stream=None):
    """paged_attention_forward with the library's own scratch array for the
    split states (see pagedkv.h): no workspace argument; `out` must be given
    by callers that cannot allocate."""
    torch = _torch()
    _need(q, "q", ndim=3)
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    _need(query_start_loc, "query_start_loc", dtype=torch.int32, ndim=1)
    total, hq, d = q.shape
    code, nb = _pools(k_pool, v_pool, q.dtype, None, d)
    hkv = k_pool.shape[1]
    S = context_lens.shape[0]
    if query_start_loc.shape[0] != S + 1 or block_tables.shape[0] != S:
        raise KVError(KV_EINVAL, "context_lens, query_start_loc and block_tables disagree on num_seqs")
    if sinks is not None:
        _need(sinks, "sinks", dtype=torch.float32, ndim=1)
        if sinks.shape[0] != hq:
            raise KVError(KV_EINVAL, "sinks must hold num_q_heads values")
    if out is None:
        with _on(stream):
            out = torch.empty((total, hq, d), dtype=torch.float32, device=q.device)
    _need(out, "out", dtype=torch.float32, ndim=3)
    if tuple(out.shape) != (total, hq, d):
        raise KVError(KV_EINVAL, "out has the wrong shape")
    _check(_lib.paged_attention_forward_noalloc(
        q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), code, block_tables.data_ptr(),
        block_tables.shape[1], context_lens.data_ptr(), query_start_loc.data_ptr(), S, total, max_q_len,
        max_context_len, hq, hkv, d, BLOCK_SIZE, nb, float(scale),
        None if sinks is None else sinks.data_ptr(), out.data_ptr(), _stream_ptr(stream)))
    return out


def paged_attention_append_forward(q, k_new, v_new, slot_mapping, k_pool, v_pool, block_tables, context_lens,
                                   query_start_loc, max_q_len: int, max_context_len: int, scale: float,
                                   sinks=None, out=None, workspace=None, stream=None):
    """kv_append_scatter of each row's own token (k_new, v_new [total_rows, Hkv, D], slot_mapping
    [total_rows]) and paged_attention_forward in one call (see pagedkv.h); returns out."""
    torch = _torch()
    S, total, hq, hkv, d, nb, code, out, workspace, ws_bytes = _forward_args(
        q, k_pool, v_pool, block_tables, context_lens, query_start_loc, max_context_len, sinks, out, workspace, stream)
    _need(k_new, "k_new", dtype=q.dtype, ndim=3)
    _need(v_new, "v_new", dtype=q.dtype, ndim=3)
    _need(slot_mapping, "slot_mapping", dtype=torch.int32, ndim=1)
    if tuple(k_new.shape) != (total, hkv, d) or tuple(v_new.shape) != (total, hkv, d) or \
            slot_mapping.shape[0] != total:
        raise KVError(KV_EINVAL, "k_new, v_new and slot_mapping must hold one row per query row")
    _check(_lib.paged_attention_append_forward(
        q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr(), k_pool.data_ptr(),
        v_pool.data_ptr(), code, block_tables.data_ptr(), block_tables.shape[1], context_lens.data_ptr(),
        query_start_loc.data_ptr(), S, total, max_q_len, max_context_len, hq, hkv, d, BLOCK_SIZE, nb, float(scale),
        None if sinks is None else sinks.data_ptr(), out.data_ptr(), workspace.data_ptr(), ws_bytes,
        _stream_ptr(stream)))
    return out


def paged_attention_masked_forward(q, k_pool, v_pool, block_tables, context_lens, query_start_loc, max_q_len: int,
                                   max_context_len: int, scale: float, sinks=None, tree_mask=None,
                                   sliding_window: int = 0, out=None, workspace=None, stream=None):
    """paged_attention_forward with tree-window masks (device uint32 [total_rows] or None) and a
    sliding window (0 = none); see pagedkv.h."""
    torch = _torch()
    S, total, hq, hkv, d, nb, code, out, workspace, ws_bytes = _forward_args(
        q, k_pool, v_pool, block_tables, context_lens, query_start_loc, max_context_len, sinks, out, workspace, stream)
    if tree_mask is not None:
        _need(tree_mask, "tree_mask", dtype=torch.int32, ndim=1)
        if tree_mask.shape[0] != total:
            raise KVError(KV_EINVAL, "tree_mask needs one word per query row")
    _check(_lib.paged_attention_masked_forward(
        q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), code, block_tables.data_ptr(), block_tables.shape[1],
        context_lens.data_ptr(), query_start_loc.data_ptr(), S, total, max_q_len, max_context_len, hq, hkv, d,
        BLOCK_SIZE, nb, float(scale), None if sinks is None else sinks.data_ptr(),
        None if tree_mask is None else tree_mask.data_ptr(), int(sliding_window), out.data_ptr(),
        workspace.data_ptr(), ws_bytes, _stream_ptr(stream)))
    return out
