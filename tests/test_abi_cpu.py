"""Host-side checks of the C ABI that need no GPU: exports, plan logic, argument errors.

No call here reaches a kernel launch: argument checks run before any device
work, and the one path that gets as far as the device query expects it to
report TTT_E_NODEV on a machine without a gfx950.
"""
import ctypes
import os
import re

import pytest
import torch

import chunk_wise_weight_amd as ttt
from chunk_wise_weight_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttt.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ttt_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    L = ttt.lib()
    names = declared_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(L, n), f"libttt.so does not export {n}"
    assert sorted(binding.EXPORTS) == names


def test_error_codes_match_header():
    src = open(HEADER).read()
    codes = dict((k, int(v)) for k, v in re.findall(r"(TTT_E_\w+)\s*=\s*(-\d+)", src))
    assert {v: k for k, v in codes.items()} == binding.ERRORS


@pytest.mark.parametrize("T,C,G,exp", [
    (1024, 128, 0, dict(G=8, L=1024, ngroups=1, T_pad=1024)),
    (131072, 256, 0, dict(G=4, L=1024, ngroups=128, T_pad=131072)),
    (131072, 128, 0, dict(G=8, L=1024, ngroups=128, T_pad=131072)),
    (32768, 256, 0, dict(G=4, L=1024, ngroups=32, T_pad=32768)),
    (3000, 100, 0, dict(G=16, L=1600, ngroups=2, T_pad=3072)),
    (1000, 3, 0, dict(G=384, L=1000, ngroups=1, T_pad=1024)),  # one group covers T
    (5000, 3, 0, dict(G=384, L=1152, ngroups=5, T_pad=5120)),
    (5000, 1, 0, dict(G=1024, L=1024, ngroups=5, T_pad=5120)),
    (300, 4096, 0, dict(G=1, L=304, ngroups=1, T_pad=512)),   # single chunk
    (4096, 4096, 0, dict(G=1, L=4096, ngroups=1, T_pad=4096)),
    (10000, 3000, 0, dict(G=8, L=10000, ngroups=1, T_pad=10240)),
    (30000, 3000, 0, dict(G=8, L=24000, ngroups=2, T_pad=30208)),
    (2048, 128, 2, dict(G=2, L=256, ngroups=8, T_pad=2048)),
    (0, 128, 0, dict(ngroups=0, T_pad=0)),
])
def test_plan(T, C, G, exp):
    p = ttt.ttt_plan(T, C, G)
    for k, v in exp.items():
        assert p[k] == v, (k, p)
    if T > 0:
        assert p["L"] % 8 == 0
        if p["ngroups"] > 1:
            assert p["L"] % 64 == 0
        assert p["ngroups"] * p["L"] >= T and (p["ngroups"] - 1) * p["L"] < T
        assert p["T_pad"] % 256 == 0 and p["T_pad"] >= T


def test_plan_errors():
    with pytest.raises(ttt.TTTError) as e:
        ttt.ttt_plan(100, 0)
    assert e.value.code == -2
    with pytest.raises(ttt.TTTError) as e:
        ttt.ttt_plan(1 << 24, 128)
    assert e.value.code == -2
    with pytest.raises(ttt.TTTError) as e:
        ttt.ttt_plan(1000, 3, 8)  # 24 is not a multiple of 64
    assert e.value.code == -2
    assert "multiple of 64" in ttt.ttt_last_error()


def _raw_init(W=(16, 32, 48), d=64, f=64, C=8, eta=0.1, dt=0, mb=1):
    L = ttt.lib()
    h = ctypes.c_void_p(123)
    ptrs = [ctypes.c_void_p(v) for v in W]
    rc = L.ttt_init(ctypes.byref(h), *ptrs, d, f, C, ctypes.c_float(eta), dt, mb, None)
    return rc, h


def test_init_argument_errors():
    L = ttt.lib()
    assert L.ttt_init(None, None, None, None, 64, 64, 8, ctypes.c_float(0.1), 0, 1, None) == -1
    rc, h = _raw_init(W=(0, 1, 1))
    assert rc == -1 and not h.value
    assert _raw_init(dt=7)[0] == -3
    assert _raw_init(d=60)[0] == -2
    assert _raw_init(f=0)[0] == -2
    assert _raw_init(d=64, f=64, dt=1)[0] == -2  # bf16 needs multiples of 256
    assert _raw_init(C=0)[0] == -2
    assert _raw_init(mb=0)[0] == -2
    assert _raw_init(eta=float("nan"))[0] == -7
    assert _raw_init(eta=float("inf"))[0] == -7
    assert _raw_init(W=(16, 34, 48))[0] == -7  # weights must be 16-byte aligned
    assert "aligned" in ttt.ttt_last_error()


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_init_without_device_reports_nodev():
    rc, h = _raw_init()
    assert rc == -6 and not h.value
    assert "device" in ttt.ttt_last_error()


def test_null_handle_paths():
    L = ttt.lib()
    assert L.ttt_forward_chunked(None, None, None, None, 1, 1, 1, None, None, None) == -1
    assert L.ttt_reset(None, -1, None) == -1
    assert L.ttt_set_group_chunks(None, 2) == -1
    assert L.ttt_set_clip(None, 1.0) == -1
    assert L.ttt_set_target_conv(None, None, 0, None, None) == -1
    assert L.ttt_forward_docs(None, None, None, None, 1, 1, 1, None, None, None, None, None) == -1
    assert L.ttt_set_profiling(None, 1) == -1
    buf = (ctypes.c_float * 6)()
    assert L.ttt_phase_times(None, buf, 6) == -1
    n = ctypes.c_size_t()
    assert L.ttt_workspace_bytes(None, ctypes.byref(n)) == -1
    assert L.ttt_set_output_f32(None, 1) == -1
    assert L.ttt_state_delta(None, None, 1, None) == -1
    assert L.ttt_forward_chunked_noalloc(None, None, None, None, 1, 1, 1, None, None, None) == -1
    L.ttt_destroy(None)  # no-op
    assert "NULL" in ttt.ttt_last_error()


def test_noalloc_workspace_size_matches_header():
    src = open(HEADER).read()
    m = re.search(r"#define TTT_NOALLOC_WORKSPACE_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m, "TTT_NOALLOC_WORKSPACE_BYTES not found"
    assert int(m.group(1)) << int(m.group(2)) == binding.NOALLOC_WORKSPACE_BYTES
