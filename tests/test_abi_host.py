"""Host-side checks of the C ABI library (no GPU needed): it loads, exports every function the
header declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


@pytest.fixture(scope="module")
def lib():
    import paged_kv_cache_fwd_amd as pkv
    if not os.path.exists(pkv.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return pkv.load()


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("paged_kv_alloc", "paged_kv_free", "paged_kv_append", "chunk_attn_fwd", "chunk_attn_bwd",
              "page_topk_select", "paged_kv_gather", "pkv_last_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    import paged_kv_cache_fwd_amd as pkv
    out = subprocess.run(["nm", "-D", "--defined-only", pkv.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if " T " in line)
    for n in _declared():
        assert n in exported, n
        assert getattr(lib, n) is not None
    assert set(_declared()) == set(pkv.EXPORTED)


def test_argument_errors_without_device(lib):
    h = ctypes.c_void_p()
    assert lib.paged_kv_alloc(None, 4, 64, 1, 64, 0) == -1
    assert lib.paged_kv_alloc(ctypes.byref(h), 4, 96, 1, 64, 0) == -2
    assert b"not supported" in lib.pkv_last_error()
    assert lib.paged_kv_alloc(ctypes.byref(h), 4, 64, 1, 48, 0) == -2
    assert lib.paged_kv_alloc(ctypes.byref(h), 0, 64, 1, 64, 0) == -1
    assert lib.paged_kv_alloc(ctypes.byref(h), 4, 64, 1, 64, 0x80) == -1
    assert lib.paged_kv_free(None) == 0
    assert lib.pkv_last_error() == b""
    assert lib.chunk_attn_fwd(None, None, 0, 0, None, 0, 1, 0, 1, None, 64, 4, 0.1, None, None, None, 0, None) == -1
    assert lib.chunk_attn_bwd(None, None, 0, None, None, 0, 0, None, 0, 1, 0, 1, None, None, None, None, 64, 4, 0.1,
                              None, None, 0, None) == -1
    assert lib.page_topk_select(None, None, 0, 0, None, 64, 4, 1, 0, 1, None, None, None, 0, None) == -1
    assert lib.paged_kv_append(None, None, 0, 0, 0, None, None, None) == -1
    assert lib.paged_kv_gather(None, None, None, 0, None, 0, 0, None, None, 0, 0, None) == -1
    assert lib.paged_kv_grad_offload(None, None, 0, None, None, 0, None, 0, 0, 1, None) == -1
    assert lib.paged_kv_copy(None, None, 1, 0, 0, None) == -1
    assert lib.paged_kv_check(None) == -1
    assert lib.pkv_mfma_probe(0, 1, None, None, None) == -1
    assert lib.pkv_mfma_probe(1, 0, None, None, None) == -1
    assert lib.pkv_mfma_probe(1, 1, None, None, None) == -1
    assert lib.paged_kv_data(None, 0) is None
    # A scale that is not a positive finite number is rejected before anything else.
    for bad in (0.0, -0.1, float("nan"), float("inf")):
        assert lib.chunk_attn_fwd(None, None, 0, 0, None, 0, 1, 0, 1, None, 64, 4, bad, None, None, None, 0,
                                  None) == -1
        assert b"scale" in lib.pkv_last_error()
        assert lib.chunk_attn_bwd(None, None, 0, None, None, 0, 0, None, 0, 1, 0, 1, None, None, None, None, 64, 4,
                                  bad, None, None, 0, None) == -1
        assert b"scale" in lib.pkv_last_error()
    assert lib.paged_kv_page_alloc(None, 1, None) == -1
    assert lib.paged_kv_page_release(None, 1, None) == -1
    assert lib.paged_kv_pages_available(None) == -1
    assert lib.chunk_attn_fwd_ws_bytes(None, 0, -1, 1, 1, 64, 4) == 0
    assert lib.page_topk_ws_bytes(None, 0, 64, 4, 1) == 0


def test_binding_fails_loudly_without_library():
    import paged_kv_cache_fwd_amd as pkv
    with pytest.raises(RuntimeError, match="missing"):
        pkv.load(os.path.join(ROOT, "no_such_dir", "libpkv.so"))


def test_product_path_does_not_use_the_oracle():
    pkg = os.path.join(ROOT, "paged_kv_cache_fwd_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "synth" not in text, f
