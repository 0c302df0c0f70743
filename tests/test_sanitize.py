"""The library's host code (cbk_api.cpp, cbk_ec_host.cpp) and the C oracle built with
AddressSanitizer + UndefinedBehaviorSanitizer, and the threaded encoder with ThreadSanitizer, on
the host only (g++/gcc; the GPU launchers are replaced by stubs that abort if reached).  The
driver, tests/sanitize/harness.cpp, checks the library's encoder against the oracle byte for byte
on seeded synthetic tensors, runs the capped-codebook and entropy-coded host passes into buffers of
exactly their announced sizes, and calls the GPU entry points with bad arguments."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "fly_decode_amd", "csrc")

pytestmark = pytest.mark.skipif(not (shutil.which("g++") and shutil.which("gcc")), reason="needs g++ and gcc")


def _build(tmp, flags, name):
    inc = ["-I", SAN, "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    common = ["-g", "-O1", "-fno-omit-frame-pointer"] + flags
    oracle_o = os.path.join(tmp, name + "_oracle.o")
    subprocess.run(["gcc", "-std=c11", "-c", os.path.join(ROOT, "oracle", "cbk_oracle.c"), "-o", oracle_o] + common,
                   check=True)
    exe = os.path.join(tmp, name)
    srcs = [os.path.join(SAN, "harness.cpp"), os.path.join(SAN, "stubs.cpp"), os.path.join(CSRC, "cbk_api.cpp"),
            os.path.join(CSRC, "cbk_ec_host.cpp")]
    subprocess.run(["g++", "-std=c++17", "-pthread"] + inc + common + srcs + [oracle_o, "-o", exe], check=True)
    return exe


def _write_inputs(path, records):
    with open(path, "wb") as f:
        for w, K in records:
            w = np.ascontiguousarray(w, dtype=np.uint16).reshape(-1)
            np.array([w.size], dtype=np.uint64).tofile(f)
            np.array([K, 0], dtype=np.uint32).tofile(f)
            w.tofile(f)


def _records(big):
    recs = [(np.zeros(0, np.uint16), 0), (np.array([0x3F80], np.uint16), 1), (np.full(7, 0x3C00, np.uint16), 2),
            (np.array([0x0000, 0x8000, 0x8000], np.uint16), 1)]
    for U, n, K in [(2, 33, 1), (3, 100, 2), (255, 1000, 16), (257, 3001, 256), (4097, 9000, 2048),
                    (32769, 40000, 8192), (65536, 65536, 1024)]:
        recs.append((synth.with_distinct_count(n, U, seed=[101, U]), K))
    recs.append((synth.gaussian_bf16((300, 1000), 0.02, seed=[102]), 1024))
    recs.append((synth.student_t_bf16((200, 999), 4.0, 0.02, seed=[103]), 4096))
    if big:  # above 2^22 weights: the encoder's threaded presence and pack passes
        recs.append((synth.gaussian_bf16((1100, 4096), 0.02, seed=[104]), 0))
    return recs


def _run(exe, inp, env_extra):
    env = dict(os.environ, **env_extra)
    r = subprocess.run([exe, inp], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "records ok" in r.stdout


def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = _build(str(tmp_path), ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"], "asan")
    inp = str(tmp_path / "in.bin")
    _write_inputs(inp, _records(big=True))
    _run(exe, inp, {"ASAN_OPTIONS": "abort_on_error=1:detect_leaks=0", "UBSAN_OPTIONS": "print_stacktrace=1"})


def test_threaded_encoder_under_thread_sanitizer(tmp_path):
    exe = _build(str(tmp_path), ["-fsanitize=thread"], "tsan")
    inp = str(tmp_path / "in.bin")
    _write_inputs(inp, [(synth.gaussian_bf16((1100, 4096), 0.02, seed=[104]), 0)])
    _run(exe, inp, {"TSAN_OPTIONS": "halt_on_error=1"})
