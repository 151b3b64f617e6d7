"""Host logic: the multiply-high division the head-split epilogues use to
split row and column indices (token -> sequence, position; column -> head,
channel) must equal integer division for every divisor and dividend the
layer can produce.  The header is plain C++, so it is compiled here with
the host compiler and checked against '/' exhaustively for small operands
and on random and boundary ones up to the 2^31 bound."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HEADER_DIR = os.path.join(os.path.dirname(HERE), "transformer_encoder_layer_amd", "csrc")

PROGRAM = r"""
#include "fastdiv.h"
#include <stdio.h>
#include <stdint.h>
static uint64_t state = 88172645463325252ull;
static uint32_t rnd() { state ^= state << 13; state ^= state >> 7; state ^= state << 17; return (uint32_t)(state >> 33); }
int main() {
    long bad = 0, checked = 0;
    auto check = [&](uint32_t d, uint32_t n) {
        const tel::FastDiv f(d);
        const uint32_t q = f.div(n);
        ++checked;
        if (q != n / d || f.mod(n, q) != n % d) {
            if (bad < 5) printf("mismatch d=%u n=%u got %u want %u\n", d, n, q, n / d);
            ++bad;
        }
    };
    for (uint32_t d = 1; d <= 2048; ++d)            // every divisor up to 2048, every n < 2^17
        for (uint32_t n = 0; n < (1u << 17); ++n) check(d, n);
    const uint32_t edge[] = {1u, 2u, 3u, 7u, 64u, 96u, 128u, 511u, 512u, 768u, 1000u, 1024u, 3072u, 4096u,
                             65535u, 65536u, 1000003u, (1u << 30) - 1u, 1u << 30, (1u << 31) - 1u};
    for (uint32_t d : edge) {
        for (int i = 0; i < 200000; ++i) check(d, rnd() & 0x7FFFFFFFu);
        for (uint32_t k = 1; k < 64; ++k) {                // multiples of d and their neighbours
            const uint64_t base = (uint64_t)d * (uint64_t)(rnd() % 1000003u + k);
            for (int delta = -1; delta <= 1; ++delta) {
                const int64_t n = (int64_t)base + delta;
                if (n >= 0 && n < (1ll << 31)) check(d, (uint32_t)n);
            }
        }
        check(d, (1u << 31) - 1u);
        check(d, 0u);
    }
    for (int i = 0; i < 2000000; ++i) {                 // random divisors and dividends
        const uint32_t d = ((rnd() & 0x7FFFFFFFu) | 1u) >> (rnd() % 31), n = rnd() & 0x7FFFFFFFu;
        check(d ? d : 1u, n);
    }
    printf("checked %ld bad %ld\n", checked, bad);
    return bad != 0;
}
"""


def test_fastdiv_matches_integer_division(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    src = tmp_path / "fd.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "fd"
    subprocess.run([cxx, "-O2", "-std=c++17", "-I", HEADER_DIR, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " bad 0" in r.stdout
