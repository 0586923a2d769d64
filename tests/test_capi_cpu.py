"""The C-ABI library loads and exports what include/sparse_ffn.h declares;
argument checks that reject before any GPU work (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

import activation_sparse_ffn_amd as sffn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in os.listdir(inc):
        if not fn.endswith(".h"):
            continue
        src = open(os.path.join(inc, fn)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^\s*[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", src, flags=re.M):
            if m.group(1) not in ("if", "while", "for", "sizeof"):
                names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def lib():
    return sffn.load_library()


def test_header_declares_the_boundary():
    names = _declared_functions()
    assert set(sffn.EXPORTED_SYMBOLS) <= names
    assert {"sparse_ffn_create", "sparse_ffn_forward", "bank_topk"} <= names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", sffn.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = _declared_functions() - exported
    assert not missing, f"declared but not exported: {missing}"
    for n in _declared_functions():
        assert hasattr(lib, n)


def _cfg(**kw):
    base = dict(d=4096, d_i=14336, rank=448, bank=64, keep=16, dtype=1, gate=0)
    base.update(kw)
    return sffn.Config(**base)


def test_packed_size_and_config_checks(lib):
    size = lib.sparse_ffn_packed_size(ctypes.byref(_cfg()))
    e = 2
    d, di, r = 4096, 14336, 448
    # A, B, W_g, W_u and W_d^T (one copy of the down projection) and the bias
    assert size >= e * (r * d + di * r + 3 * di * d) + 4 * di
    assert size < e * (r * d + di * r + 3 * di * d) + 4 * di + 8 * 256
    for bad in (dict(bank=32), dict(keep=0), dict(keep=65), dict(d_i=1000), dict(d=100),
                dict(rank=40), dict(d=0), dict(dtype=7), dict(gate=3), dict(d_i=65536 + 64),
                dict(flags=2), dict(flags=-1)):
        assert lib.sparse_ffn_packed_size(ctypes.byref(_cfg(**bad))) == 0, bad
    assert lib.sparse_ffn_packed_size(None) == 0
    # SFFN_FLAG_BACKWARD adds W_g^T and W_u^T (bf16, [d, d_i] each)
    with_t = lib.sparse_ffn_packed_size(ctypes.byref(_cfg(flags=sffn.SFFN_FLAG_BACKWARD)))
    assert with_t == size + 2 * e * d * di


def test_bank_topk_rejections(lib):
    assert lib.bank_topk(None, 0, 1024, 16, None, None, None) == sffn.SFFN_OK   # T = 0: no-op
    assert lib.bank_topk(None, -1, 1024, 16, None, None, None) == sffn.SFFN_ERR_INVALID_ARG
    assert lib.bank_topk(None, 4, 1000, 16, None, None, None) == sffn.SFFN_ERR_INVALID_ARG
    assert lib.bank_topk(None, 4, 1024, 0, None, None, None) == sffn.SFFN_ERR_INVALID_ARG
    assert b"keep" in lib.sparse_ffn_last_error()
    assert lib.bank_topk(None, 4, 1024, 65, None, None, None) == sffn.SFFN_ERR_INVALID_ARG
    assert lib.bank_topk(None, 4, 1024, 16, None, None, None) == sffn.SFFN_ERR_INVALID_ARG
    odd = ctypes.c_void_p(0x1008)   # never dereferenced: rejected as misaligned
    assert lib.bank_topk(odd, 4, 1024, 16, ctypes.c_void_p(0x2000), None, None) == sffn.SFFN_ERR_INVALID_ARG
    assert b"aligned" in lib.sparse_ffn_last_error()


def test_create_and_forward_rejections(lib):
    h = ctypes.c_void_p()
    fake = ctypes.c_void_p(0x10000)
    args = [fake] * 5 + [None, fake, 1 << 40, None, ctypes.byref(h)]
    assert lib.sparse_ffn_create(ctypes.byref(_cfg(keep=0)), *args) == sffn.SFFN_ERR_INVALID_ARG
    assert lib.sparse_ffn_create(ctypes.byref(_cfg(bank=16)), *args) == sffn.SFFN_ERR_UNSUPPORTED
    args_null = [None] + [fake] * 4 + [None, fake, 1 << 40, None, ctypes.byref(h)]
    assert lib.sparse_ffn_create(ctypes.byref(_cfg()), *args_null) == sffn.SFFN_ERR_INVALID_ARG
    small = [fake] * 5 + [None, fake, 1024, None, ctypes.byref(h)]
    assert lib.sparse_ffn_create(ctypes.byref(_cfg()), *small) == sffn.SFFN_ERR_WORKSPACE
    assert h.value is None
    assert lib.sparse_ffn_forward(None, fake, 1, fake, None, None, fake, 1 << 30, None) \
        == sffn.SFFN_ERR_INVALID_ARG
    assert lib.sparse_ffn_workspace_size(None, 8) == 0


def test_status_strings(lib):
    for s in range(5):
        assert lib.sparse_ffn_status_string(s)
    assert lib.sparse_ffn_status_string(99) == b"unknown status"
