"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
symbol declared in include/tt_bag.h, and rejects bad arguments before enqueuing
anything (these calls return from the host validation and touch no device)."""
import ctypes
import os
import re

import pytest

from tensor_train_compressed_ttembeddingbag_amd import abi, workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "tt_bag.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tt_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = abi.lib()
    names = _declared()
    assert "tt_bag_forward" in names and "tt_cache_lookup" in names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(abi.EXPORTS)


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert abi.status_string(code)
    assert abi.status_string(-99) == "unknown status"


def test_workspace_size_and_shape_envelope():
    wl = W.WORKLOADS["readme"]
    d = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E)
    n = abi.tt_bag_workspace_size(d, 10240, 512)
    assert n > 10240 * 16
    assert abi.tt_bag_workspace_size(d, 20480, 512) > n
    L = abi.lib()
    bad = [abi.make_desc(wl.p, (3, 4, 4), wl.ranks, wl.E),        # q1 = 3
           abi.make_desc(wl.p, wl.q, (65, 32), wl.E),             # rank above 64
           abi.make_desc(wl.p, wl.q, (0, 32), wl.E),              # rank 0
           abi.make_desc((10, 10, 10), wl.q, wl.ranks, 1001),     # E > prod(p)
           abi.make_desc((9000, 2, 2), wl.q, wl.ranks, 100),      # too many bins
           abi.make_desc(wl.p, (4, 4, 17), wl.ranks, wl.E)]       # q3 > 16
    for b in bad:
        assert L.tt_bag_workspace_size(ctypes.byref(b), 100, 10, 0) == 0
    # a cache needs a single table
    d8 = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E, num_tables=8)
    assert L.tt_bag_workspace_size(ctypes.byref(d8), 100, 10, 1000) == 0
    assert L.tt_bag_workspace_size(ctypes.byref(d8), 100, 10, 0) > 0


def test_entry_points_reject_bad_arguments_without_device_work():
    wl = W.WORKLOADS["tiny"]
    L = abi.lib()
    d = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E)
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced: validation fails first
    cores = (ctypes.c_void_p * 3)(0x1000, 0x2000, 0x3000)
    null_cores = (ctypes.c_void_p * 3)(0x1000, 0, 0x3000)
    # negative nnz / zero bags
    assert L.tt_bag_forward(ctypes.byref(d), cores, fake, -1, fake, 8, None, None, fake, fake,
                            1 << 20, None, None) == -1
    assert L.tt_bag_forward(ctypes.byref(d), cores, fake, 10, fake, 0, None, None, fake, fake,
                            1 << 20, None, None) == -1
    # a null core pointer
    assert L.tt_bag_forward(ctypes.byref(d), null_cores, fake, 10, fake, 8, None, None, fake, fake,
                            1 << 20, None, None) == -1
    # workspace too small or misaligned
    assert L.tt_bag_forward(ctypes.byref(d), cores, fake, 10, fake, 8, None, None, fake, fake,
                            16, None, None) == -3
    assert L.tt_bag_forward(ctypes.byref(d), cores, fake, 10, fake, 8, None, None, fake,
                            P(0x1004), 1 << 20, None, None) == -3
    # shape outside the envelope
    d3 = abi.make_desc(wl.p, (3, 2, 2), wl.ranks, wl.E)
    assert L.tt_bag_backward_sgd(ctypes.byref(d3), cores, fake, 10, fake, 8, None, None, fake,
                                 ctypes.c_float(0.1), fake, 1 << 20, None, None) == -2
    # non-finite learning rate
    assert L.tt_bag_backward_sgd(ctypes.byref(d), cores, fake, 10, fake, 8, None, None, fake,
                                 ctypes.c_float(float("nan")), fake, 1 << 20, None, None) == -1
    # cache handle checks
    assert L.tt_cache_lookup(None, fake, 10, fake, 1, None, None) == -1
    assert L.tt_cache_destroy(None) == -1
    h = ctypes.c_void_p()
    d8 = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E, num_tables=2)
    assert L.tt_cache_create(ctypes.byref(h), ctypes.byref(d8), 10, 100) == -2
    assert L.tt_cache_create(ctypes.byref(h), ctypes.byref(d), 0, 100) == -1


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(abi, "_lib", None)
    monkeypatch.setattr(abi, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError):
        abi.lib()
