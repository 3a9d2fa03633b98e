"""The C-ABI library loads and exports every symbol include/iso.h declares, and its
host-only logic (argument checks, workspace sizing, status strings) behaves as
documented.  No kernel is launched here."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from lower_convex_hull_amd import iso

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "iso.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w \*]*?\b(iso_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(iso.LIB_PATH):
        pytest.fail("libiso.so is not built (run __graft_entry__.build())")
    return iso.lib()


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(iso.EXPORTS)


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings(L):
    for s in (0, 1, -1, -2, -3, -4, -5, -6, -7):
        assert iso.iso_status_str(s) and iso.iso_status_str(s) != "unknown status"
    assert iso.iso_status_str(42) == "unknown status"


def test_workspace_sizing(L):
    assert iso.iso_workspace_bytes(0, 10) == 0
    assert iso.iso_workspace_bytes(5, 0) == 0
    assert iso.iso_workspace_bytes(-1, 10) == 0
    short = iso.iso_workspace_bytes(1024, 1024)
    assert 0 < short <= 1024 * 4 + 256
    n = 10_000_000
    unw = iso.iso_workspace_bytes(1, n)
    wtd = iso.iso_workspace_bytes(1, n, iso.ISO_F_WEIGHTED_HINT)
    cpy = iso.iso_workspace_bytes(1, n, iso.ISO_F_COPY_CONTROL)
    assert unw > 0 and wtd > unw and cpy > unw
    m = -(-n // iso.iso_chunk_size(n))
    # chunk slots of C+1 vertices (index + S) dominate
    assert unw >= m * (iso.iso_chunk_size(n) + 1) * 10


def test_chunking_contract(L):
    smax = iso.iso_short_row_max()
    assert smax >= 1024
    assert iso.iso_chunk_size(smax) == smax
    assert iso.iso_chunk_size(smax + 1) >= 1024


def test_argument_errors_launch_nothing(L):
    f = L.iso_fit_ex
    buf = ctypes.create_string_buffer(64)
    p = ctypes.addressof(buf)
    # NULL y or out
    assert f(None, None, 1, 4, p, None, p, 64, None, 0) == iso.ISO_ERR_ARG
    assert f(p, None, 1, 4, None, None, p, 64, None, 0) == iso.ISO_ERR_ARG
    # negative sizes
    assert f(p, None, -1, 4, p + 32, None, p, 64, None, 0) == iso.ISO_ERR_ARG
    assert f(p, None, 1, -4, p + 32, None, p, 64, None, 0) == iso.ISO_ERR_ARG
    # unknown flag bits
    assert f(p, None, 1, 4, p + 32, None, p, 64, None, 1 << 20) == iso.ISO_ERR_ARG
    # empty shapes are a no-op
    assert f(p, None, 0, 4, p + 32, None, None, 0, None, 0) == iso.ISO_OK
    assert f(p, None, 3, 0, p + 32, None, None, 0, None, 0) == iso.ISO_OK
    # output overlapping the input
    assert f(p, None, 1, 4, p + 8, None, p, 64, None, 0) == iso.ISO_ERR_ARG
    # misaligned pointers
    assert f(p + 1, None, 1, 4, p + 32, None, p, 64, None, 0) == iso.ISO_ERR_ARG
    # workspace too small (checked before anything is launched)
    assert f(p, None, 1, 10_000, p + 40_000, None, p, 64, None, 0) == iso.ISO_ERR_WORKSPACE
    assert f(p, None, 1, 4, p + 32, None, None, 0, None, 0) == iso.ISO_ERR_WORKSPACE
    # iso_fit: argument errors before any device call
    assert L.iso_fit(None, None, 1, 4, p) == iso.ISO_ERR_ARG
    assert L.iso_fit(p, None, 0, 4, p) == iso.ISO_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(iso, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(iso, "_lib", None)
    with pytest.raises(RuntimeError):
        iso.lib()
