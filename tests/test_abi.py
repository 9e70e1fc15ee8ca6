"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects invalid host arguments before touching a device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedkv.h")


@pytest.fixture(scope="module")
def pk():
    import paged_kv_attention_block_amd as pk
    return pk


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ["kv_pool_alloc", "kv_append_scatter", "paged_attention_forward",
                 "paged_attention_workspace_size", "kv_pool_create", "kv_pool_release",
                 "kv_last_error", "kv_abi_version"]:
        assert want in names


def test_library_exports_every_declared_symbol(pk):
    lib = ctypes.CDLL(pk.lib_path)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version(pk):
    assert pk.kv_abi_version() == 1


def _lib(pk):
    return pk._lib


def test_forward_rejects_bad_host_arguments(pk):
    lib = _lib(pk)
    fake = ctypes.c_void_p(256)   # never dereferenced: validation fails first
    base = dict(q=fake, k=fake, v=fake, dtype=pk.KV_BF16, bt=fake, mb=64, ctx=fake, qsl=fake, S=2,
                rows=2, mq=1, mctx=1000, hq=32, hkv=8, d=128, bs=16, nb=100, scale=0.1,
                sinks=None, out=fake, ws=fake, wsb=1 << 30, st=None)

    def call(**kw):
        a = dict(base, **kw)
        return lib.paged_attention_forward(a["q"], a["k"], a["v"], a["dtype"], a["bt"], a["mb"], a["ctx"],
                                           a["qsl"], a["S"], a["rows"], a["mq"], a["mctx"], a["hq"],
                                           a["hkv"], a["d"], a["bs"], a["nb"], a["scale"], a["sinks"],
                                           a["out"], a["ws"], a["wsb"], a["st"])

    assert call(hq=30) == pk.KV_EINVAL                # Hq % Hkv
    assert call(d=96) == pk.KV_EUNSUPPORTED
    assert call(bs=32) == pk.KV_EUNSUPPORTED
    assert call(dtype=7) == pk.KV_EUNSUPPORTED
    assert call(q=None) == pk.KV_EINVAL
    assert call(wsb=16) == pk.KV_EINVAL               # workspace too small
    assert "workspace" in pk.kv_last_error()
    assert call(mb=10) == pk.KV_EINVAL                # table cannot hold max_context_len
    assert call(mq=0) == pk.KV_EINVAL
    assert call(scale=float("nan")) == pk.KV_EINVAL
    assert call(q=ctypes.c_void_p(258)) == pk.KV_EINVAL   # misaligned
    assert call(S=0) == pk.KV_OK                      # empty batch: nothing to do
    assert call(rows=0) == pk.KV_OK


def test_append_forward_rejects_bad_host_arguments(pk):
    lib = _lib(pk)
    f = ctypes.c_void_p(256)
    ws = pk.paged_attention_workspace_size(4, 4, 32, 128, 800)

    def call(**kw):
        a = dict(q=f, kn=f, vn=f, slots=f, k=f, v=f, dtype=pk.KV_BF16, bt=f, mb=64, ctx=f, qsl=f, S=4, rows=4,
                 mq=1, mctx=800, hq=32, hkv=8, d=128, bs=16, nb=1000, scale=0.088, sinks=None, out=f, ws=f,
                 wsb=ws, st=None)
        a.update(kw)
        return lib.paged_attention_append_forward(
            a["q"], a["kn"], a["vn"], a["slots"], a["k"], a["v"], a["dtype"], a["bt"], a["mb"], a["ctx"],
            a["qsl"], a["S"], a["rows"], a["mq"], a["mctx"], a["hq"], a["hkv"], a["d"], a["bs"], a["nb"],
            a["scale"], a["sinks"], a["out"], a["ws"], a["wsb"], a["st"])

    assert call(kn=None) == pk.KV_EINVAL
    assert "k_new" in pk.kv_last_error()
    assert call(slots=None) == pk.KV_EINVAL
    assert call(vn=ctypes.c_void_p(260)) == pk.KV_EINVAL   # misaligned
    assert call(hq=30) == pk.KV_EINVAL                      # the forward's own checks still apply
    assert call(wsb=16) == pk.KV_EINVAL
    assert call(S=0) == pk.KV_OK


def test_scatter_rejects_bad_host_arguments(pk):
    lib = _lib(pk)
    f = ctypes.c_void_p(256)
    assert lib.kv_append_scatter(f, f, f, 4, f, f, 10, 8, 128, 16, 9, None) == pk.KV_EUNSUPPORTED
    assert lib.kv_append_scatter(f, f, f, 4, f, f, 10, 8, 100, 16, pk.KV_BF16, None) == pk.KV_EUNSUPPORTED
    assert lib.kv_append_scatter(None, f, f, 4, f, f, 10, 8, 128, 16, pk.KV_BF16, None) == pk.KV_EINVAL
    assert lib.kv_append_scatter(f, f, f, -1, f, f, 10, 8, 128, 16, pk.KV_BF16, None) == pk.KV_EINVAL
    assert lib.kv_append_scatter(f, f, f, 0, f, f, 10, 8, 128, 16, pk.KV_BF16, None) == pk.KV_OK


def test_workspace_size_formula_grows_with_context(pk):
    a = pk.paged_attention_workspace_size(4, 4, 32, 128, 800)
    b = pk.paged_attention_workspace_size(4, 4, 32, 128, 8000)
    assert 0 < a < b
    assert pk.paged_attention_workspace_size(-1, 4, 32, 128, 800) == 0


def test_pool_create_validation(pk):
    with pytest.raises(pk.KVError) as e:
        pk.kv_pool_create(4, 16, [0, 1, 1, 2])
    assert e.value.code == pk.KV_EINVAL
    with pytest.raises(pk.KVError):
        pk.kv_pool_create(0, 16)
    p = pk.kv_pool_create(4, 16)
    with pytest.raises(pk.KVError) as e:
        pk.kv_pool_release(p, 99)
    assert e.value.code == pk.KV_EINVAL
    with pytest.raises(pk.KVError) as e:
        pk.kv_pool_alloc(p, 1, range(100), 4)      # needs 7 blocks > max_blocks
    assert e.value.code == pk.KV_EINVAL
    assert pk.kv_pool_stats(p) == (4, 0, 0)


def test_noalloc_forward_rejects_batches_beyond_its_scratch_on_the_host(pk):
    """The size check comes before any device call: 2096 rows x 32 heads x 7
    splits of 128 channels need about 244 MB of split states, more than the
    64 MiB array."""
    lib = _lib(pk)
    fake = ctypes.c_void_p(256)   # never dereferenced: the size check fails first
    need = pk.paged_attention_workspace_size(50, 2096, 32, 128, 3925)
    assert need > 64 << 20
    rc = lib.paged_attention_forward_noalloc(fake, fake, fake, pk.KV_BF16, fake, 256, fake, fake, 50, 2096, 1024,
                                             3925, 32, 8, 128, 16, 64, 0.1, None, fake, None)
    assert rc == pk.KV_EINVAL
    assert str(need) in pk.kv_last_error() and "67108864" in pk.kv_last_error()
