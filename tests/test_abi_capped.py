"""CPU tests of cbk_cap_patterns (the capped, lossy codebook step): the library's result equals
the oracle's (oracle/capped.py) exactly, and bad arguments are rejected."""
import ctypes

import numpy as np
import pytest

import synth
from oracle import capped


@pytest.fixture(scope="module")
def cbk():
    import os
    import fly_decode_amd
    if not os.path.exists(fly_decode_amd.library_path()):
        from fly_decode_amd import build
        build.build()
    fly_decode_amd.load_library()
    return fly_decode_amd


def _cases():
    rng = np.random.default_rng(70)
    specials = synth.gaussian_bf16((5000,), 0.02, seed=[71])
    specials[rng.choice(5000, 9, replace=False)] = np.array([0x7F80, 0xFF80, 0x7FC0, 0x7FC0, 0xFFC1, 0x7F80,
                                                             0x8000, 0x0000, 0x0001], dtype=np.uint16)
    return [
        ("gaussian_K2048", synth.gaussian_bf16((64, 4096), 0.02, seed=[72]), 2048),
        ("gaussian_K300", synth.gaussian_bf16((20, 1000), 0.02, seed=[73]), 300),
        ("t2_K512", synth.student_t_bf16((30, 1000), 2.0, 0.02, seed=[74]), 512),
        ("specials_K64", specials, 64),
        ("fits", synth.with_distinct_count(1000, 100, seed=[75]), 100),
        ("K1", np.array([0x3F80, 0x4000, 0x3F80, 0xC000], dtype=np.uint16), 1),
        ("every_pattern_finite_K1000", np.array([v for v in range(65536) if ((v >> 7) & 0xFF) != 0xFF], dtype=np.uint16), 1000),
    ]


@pytest.mark.parametrize("name,w,K", _cases(), ids=[c[0] for c in _cases()])
def test_library_equals_oracle(cbk, name, w, K):
    got, U = cbk.cap_patterns(w, K)
    want = capped.cap(w, K)
    assert np.array_equal(got, want)
    assert U == np.unique(want).size == min(np.unique(w).size, K)


def test_encode_with_cap_roundtrips_to_the_capped_tensor(cbk, oracle_mod):
    w = synth.gaussian_bf16((64, 4096), 0.02, seed=[76])
    c = cbk.encode(w, cap=1024)
    assert c.U == 1024 and c.b == 10
    e = oracle_mod.encode(capped.cap(w, 1024))
    assert np.array_equal(c.words, e.words) and np.array_equal(c.codebook, e.codebook)


def test_rejects_bad_arguments(cbk):
    lib = cbk.load_library()
    U = ctypes.c_uint32()
    w = np.array([0x7F80, 0xFF80, 0x3F80], dtype=np.uint16)
    out = np.empty_like(w)
    assert lib.cbk_cap_patterns(w.ctypes.data, 3, 0, out.ctypes.data, ctypes.byref(U)) == 1
    assert lib.cbk_cap_patterns(None, 3, 2, out.ctypes.data, ctypes.byref(U)) == 1
    assert lib.cbk_cap_patterns(w.ctypes.data, 3, 2, out.ctypes.data, None) == 1
    assert lib.cbk_cap_patterns(w.ctypes.data, 3, 2, out.ctypes.data, ctypes.byref(U)) == 4   # no room for 1.0
    assert lib.cbk_cap_patterns(w.ctypes.data, 3, 3, out.ctypes.data, ctypes.byref(U)) == 0
