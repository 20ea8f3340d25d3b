"""Pins for oracle.philox: Philox4x32-10 and the per-element draw layout.

Independent references: rocrand's Philox4x32-10 (compiled from its header on
the host), agreement of the two oracle implementations, and uniformity of the
16-bit draws (chi-square).
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import philox

ROCRAND_SRC = r"""
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
struct E : rocrand_device::philox4x32_10_engine {
  uint4 t(uint4 c, uint2 k) { return ten_rounds(c, k); }
};
int main() {
  E e; unsigned a, b, c, d, k0, k1;
  while (scanf("%u %u %u %u %u %u", &a, &b, &c, &d, &k0, &k1) == 6) {
    uint4 r = e.t(uint4{a, b, c, d}, uint2{k0, k1});
    printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
}
"""


def random_blocks(n, seed=0):
    r = np.random.default_rng(seed)
    return r.integers(0, 2 ** 32, size=(n, 6), dtype=np.uint64)


def test_scalar_matches_vectorised():
    blk = random_blocks(500)
    vec = philox.philox4x32_10(blk[:, 0], blk[:, 1], blk[:, 2], blk[:, 3], 0, 0)
    for i in range(blk.shape[0]):
        k0, k1 = int(blk[i, 4]), int(blk[i, 5])
        v = philox.philox4x32_10(blk[i, 0], blk[i, 1], blk[i, 2], blk[i, 3], k0, k1)
        s = philox.philox4x32_10_scalar(blk[i, :4], (k0, k1))
        assert tuple(int(x) for x in v) == s
        if k0 == 0 and k1 == 0:
            assert tuple(int(w[i]) for w in vec) == s


def test_against_rocrand(tmp_path):
    exe = _rocrand_exe(tmp_path)
    blk = random_blocks(2000, seed=5)
    blk[:10, :4] = 0
    blk[10:20, :4] = 0xFFFFFFFF
    text = "\n".join(" ".join(str(int(x)) for x in row) for row in blk) + "\n"
    out = subprocess.run([str(exe)], input=text, capture_output=True, text=True, check=True).stdout.split("\n")
    for row, line in zip(blk, out):
        ref = tuple(int(x) for x in line.split())
        assert philox.philox4x32_10_scalar(row[:4], row[4:6]) == ref


def test_draw_layout():
    seed, offset = 0x123456789ABCDEF0, 77
    e = np.array([0, 1, 2, 3, 6, 7, 8, 9, 12345, (1 << 33) + 5], dtype=np.uint64)
    got = philox.sr_draws_u16(e, seed, offset)
    for ei, g in zip(e, got):
        ei = int(ei)
        b = ei >> 3
        w = philox.philox4x32_10_scalar((b & 0xFFFFFFFF, b >> 32, offset, 0), (seed & 0xFFFFFFFF, seed >> 32))
        word = w[(ei >> 1) & 3]
        assert int(g) == (word >> (16 * (ei & 1))) & 0xFFFF


def test_draws_uniform_chi_square():
    from scipy import stats
    d = philox.sr_draws_u16(np.arange(1 << 20, dtype=np.uint64), seed=0, offset=3)
    for part in (d >> 8, d & 0xFF):
        counts = np.bincount(part.astype(np.int64), minlength=256)
        p = stats.chisquare(counts).pvalue
        assert p > 1e-4
    # different offsets give different streams
    d2 = philox.sr_draws_u16(np.arange(4096, dtype=np.uint64), seed=0, offset=4)
    assert np.mean(d[:4096] == d2) < 0.01


def test_rht_signs_distinct_per_offset():
    masks = {philox.rht_signs(0, o) for o in range(0, 64, 2)}
    assert len(masks) > 24
    assert all(0 <= m < 65536 for m in masks)


def _rocrand_exe(tmp_path):
    inc = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"
    if not (shutil.which("g++") and os.path.exists(inc)):
        pytest.skip("rocrand header or g++ not available")
    src = tmp_path / "rr.cpp"
    src.write_text(ROCRAND_SRC)
    exe = tmp_path / "rr"
    subprocess.run(["g++", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    return exe


def test_rht_signs_against_rocrand(tmp_path):
    """The sign mask of one product pair is the low 16 bits of word 0 of the Philox4x32-10 block
    with counter (0xFFFFFFFF, 0xFFFFFFFF, lo offset, hi offset) and key (lo seed, hi seed),
    computed here by rocrand's generator (a wrong counter word, word or half fails)."""
    exe = _rocrand_exe(tmp_path)
    cases = [(0, 0), (0, 2), (0, 8), (1, 0), (0x123456789ABCDEF0, 77), ((1 << 64) - 1, (1 << 64) - 1),
             (42, (1 << 32) + 3), (7, 1 << 40)]
    rows = []
    for seed, off in cases:
        rows.append((0xFFFFFFFF, 0xFFFFFFFF, off & 0xFFFFFFFF, off >> 32, seed & 0xFFFFFFFF, seed >> 32))
    text = "\n".join(" ".join(str(x) for x in r) for r in rows) + "\n"
    out = subprocess.run([str(exe)], input=text, capture_output=True, text=True, check=True).stdout.split("\n")
    for (seed, off), line in zip(cases, out):
        word0 = int(line.split()[0])
        assert philox.rht_signs(seed, off) == word0 & 0xFFFF, (seed, off)
