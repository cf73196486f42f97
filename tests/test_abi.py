"""CPU-side checks of the C ABI: the library loads, exports every function
include/mla.h declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    from mla_latent_kv_07_amd import _lib
    if not os.path.exists(_lib.lib_path()):
        import mla_latent_kv_07_amd.build as b
        b.build()
    return _lib.load()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "mla.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"mla_cache_insert", "mla_decode", "mla_decode_workspace_bytes",
            "mla_status_string", "mla_abi_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.mla_abi_version() == 1


def test_status_strings(lib):
    for s in range(8):
        assert lib.mla_status_string(s) and lib.mla_status_string(s) != b"unknown status"
    assert lib.mla_status_string(99) == b"unknown status"


def test_debug_checks_toggle(lib):
    """mla_debug_checks: -1 queries, 1/0 set, and the previous value comes back."""
    start = lib.mla_debug_checks(-1)
    assert start in (0, 1)
    assert lib.mla_debug_checks(1) == start
    assert lib.mla_debug_checks(-1) == 1
    assert lib.mla_debug_checks(0) == 1
    assert lib.mla_debug_checks(-1) == 0
    lib.mla_debug_checks(start)


def _dims(heads=16, **kw):
    from mla_latent_kv_07_amd._lib import Dims
    d = dict(heads=heads, kv_lora=512, rope=64, qk_nope=128, v_dim=128, page=64)
    d.update(kw)
    return Dims(**d)


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _decode(lib, d, **kw):
    a = dict(q=FAKE, kv_b=FAKE, cache=FAKE, nb=10, bt=FAKE, bts=4, sl=FAKE, B=2, q_len=1,
             maxlen=256, scale=0.07, out=FAKE, ws=FAKE, wsb=0, hint=0)
    a.update(kw)
    return lib.mla_decode(ctypes.byref(d) if d is not None else None, a["q"], a["kv_b"],
                          a["cache"], a["nb"], a["bt"], a["bts"], a["sl"], a["B"], a["q_len"],
                          a["maxlen"], a["scale"], a["out"], a["ws"], a["wsb"], a["hint"], None)


def test_decode_validation(lib):
    assert _decode(lib, None) == 1
    assert _decode(lib, _dims(heads=24)) == 3
    assert _decode(lib, _dims(heads=256)) == 3
    assert _decode(lib, _dims(kv_lora=256)) == 3
    assert _decode(lib, _dims(page=32)) == 3
    assert _decode(lib, _dims(), q_len=0) == 2
    assert _decode(lib, _dims(), q_len=9) == 2
    assert _decode(lib, _dims(), maxlen=0) == 2
    assert _decode(lib, _dims(), bts=3) == 2           # 256 positions need 4 blocks
    assert _decode(lib, _dims(), scale=-1.0) == 2
    assert _decode(lib, _dims(), scale=float("nan")) == 2
    assert _decode(lib, _dims(), hint=65) == 2
    assert _decode(lib, _dims(), B=-1) == 2
    assert _decode(lib, _dims(), q=None) == 1
    assert _decode(lib, _dims(), out=None) == 1
    assert _decode(lib, _dims(), ws=None) == 4
    assert _decode(lib, _dims(), wsb=16) == 4           # far too small
    assert _decode(lib, _dims(), B=0, q=None, ws=None) == 0  # empty batch: no-op


def test_workspace_bytes(lib):
    d = _dims(heads=128)
    w0 = lib.mla_decode_workspace_bytes(ctypes.byref(d), 64, 1, 8192, 0)
    w1 = lib.mla_decode_workspace_bytes(ctypes.byref(d), 64, 1, 8192, 4)
    # absorbed query (bf16) and, with 4 splits, the bf16 split partials
    assert w0 > 64 * 128 * 576 * 2 and w1 > 64 * 4 * 128 * 512 * 2
    assert lib.mla_decode_workspace_bytes(ctypes.byref(d), 64, 1, 0, 0) == 0
    assert lib.mla_decode_workspace_bytes(ctypes.byref(_dims(heads=8)), 64, 1, 8192, 0) == 0


def test_insert_validation(lib):
    d = _dims()
    f = lambda **kw: lib.mla_cache_insert(
        ctypes.byref(d), kw.get("kv_a", FAKE), FAKE, kw.get("eps", 1e-6), kw.get("base", 1e4),
        FAKE, kw.get("bts", 4), FAKE, kw.get("B", 2), kw.get("q_len", 1), kw.get("cache", FAKE),
        kw.get("nb", 10), None)
    assert f(q_len=0) == 2
    assert f(eps=-1.0) == 2
    assert f(base=0.0) == 2
    assert f(nb=0) == 2
    assert f(kv_a=None) == 1
    assert f(cache=None) == 1
    assert f(B=0, kv_a=None) == 0
    assert lib.mla_cache_insert(None, FAKE, FAKE, 1e-6, 1e4, FAKE, 4, FAKE, 2, 1, FAKE, 10, None) == 1


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    from mla_latent_kv_07_amd import _lib
    monkeypatch.setattr(_lib, "PKG", str(tmp_path))
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.delenv("MLA_LIB", raising=False)
    with pytest.raises(RuntimeError, match="no fallback"):
        _lib.load()
