"""The boundary from plain C: include/cbk.h and include/cbk_ec.h compile as C99 (pedantic, warnings
as errors), and a C program linked against libcbk.so calls the host entry points with C types.

The program encodes ten patterns with four distinct values and checks the result against the
format written out by hand:
* codebook = the distinct patterns ascending, U = 4, b = 2;
* field i = index of pattern i, bits [2i, 2i + 2) of a little-endian uint32 stream, LSB first;
* the size helpers and the status strings;
* validation without a device: a GPU call with a null tensor returns CBK_E_INVALID before any HIP
  call.
No GPU is used.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "cbk.h"
#include "cbk_ec.h"

#define CHECK(c) do { if (!(c)) { printf("failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

int main(void) {
    /* indices of the sorted distinct values {0x0001, 0x3F80, 0x8000, 0xBF80}: 0 1 2 3 */
    const uint16_t w[10] = {0x3F80, 0x3F80, 0x8000, 0x0001, 0xBF80, 0x3F80, 0x0001, 0x8000, 0xBF80, 0x3F80};
    const uint32_t idx[10] = {1, 1, 2, 0, 3, 1, 0, 2, 3, 1};
    uint16_t codebook[65536];
    uint32_t U = 0, b = 0, words[8];
    uint64_t need = 0, expect = 0;
    int i;
    memset(words, 0xAB, sizeof(words));
    CHECK(cbk_encode(w, 10, codebook, &U, &b, NULL, 0, &need) == CBK_E_CAPACITY);
    CHECK(need == cbk_words_for(10, 2) && need == 4);
    CHECK(cbk_encode(w, 10, codebook, &U, &b, words, 8, &need) == CBK_OK);
    CHECK(U == 4 && b == 2 && b == cbk_bits_for(U));
    CHECK(codebook[0] == 0x0001 && codebook[1] == 0x3F80 && codebook[2] == 0x8000 && codebook[3] == 0xBF80);
    for (i = 0; i < 10; ++i) expect |= (uint64_t)idx[i] << (2 * i);
    CHECK(words[0] == (uint32_t)expect);
    CHECK(words[1] == 0 && words[2] == 0 && words[3] == 0);  /* zero padding to 16 bytes */
    CHECK(words[4] == 0xABABABABu);                          /* nothing written past need */
    CHECK(cbk_compressed_bytes(10, 4) == 2 * 4 + 3);         /* 2U + ceil(10 * 2 / 8) */
    CHECK(strcmp(cbk_status_str(CBK_OK), "ok") == 0);
    CHECK(cbk_gemv(NULL, NULL, NULL, NULL) == CBK_E_INVALID);
    CHECK(cbk_gemv_chain_bytes(1) > 256);
    printf("c abi ok\n");
    return 0;
}
"""


@pytest.fixture(scope="module")
def lib():
    import fly_decode_amd
    if not os.path.exists(fly_decode_amd.library_path()):
        from fly_decode_amd import build
        build.build()
    return fly_decode_amd.library_path()


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_headers_compile_as_c99_and_a_c_program_links_and_runs(lib, tmp_path):
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(lib)
    rocm_lib = "/opt/rocm/lib"
    cmd = ["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           str(src), "-o", str(exe), "-L", libdir, "-lcbk", f"-Wl,-rpath,{libdir}",
           "-Wl,--allow-shlib-undefined"]
    if os.path.isdir(rocm_lib):
        cmd += [f"-Wl,-rpath-link,{rocm_lib}", f"-Wl,-rpath,{rocm_lib}"]
    subprocess.run(cmd, check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "c abi ok" in out.stdout
