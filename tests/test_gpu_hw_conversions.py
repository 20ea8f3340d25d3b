"""Conformance of gfx950's stochastic-rounding conversion instructions with the oracle's rule.

The quantizers round stochastically with v_cvt_scalef32_sr_pk_fp4_f32 / _sr_fp8_f32,
the 16-bit draw in the top half of the random operand.  The oracle's rule is
"round up iff u + floor(t) >= 65536" with t = 65536 * (position of |v| inside its
grid gap).  This test runs the instruction exactly at each value's threshold
(u* - 1 must round down, u* must round up) plus extreme and random draws, on a
dense sample of fp32 values covering every binade of both grids, and requires
bit-exact agreement.  The tests/hw program is compiled here with hipcc."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import formats

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def prog(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    d = tmp_path_factory.mktemp("hw")
    exe = d / "sr_conformance"
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O2", os.path.join(HERE, "hw", "sr_conformance.hip"),
                    "-o", str(exe)], check=True, capture_output=True)
    return exe, d


def f32_range(lo, hi, stride):
    a = int(np.float32(lo).view(np.uint32))
    b = int(np.float32(hi).view(np.uint32))
    return np.arange(a, b + 1, stride, dtype=np.uint32).view(np.float32)


def thresholds(v, grid):
    """floor(t) per value, computed as the oracle does (fp32 exact)."""
    a = np.abs(v)
    lo = np.clip(np.searchsorted(grid, a.astype(np.float64), side="right") - 1, 0, len(grid) - 1)
    hi = np.minimum(lo + 1, len(grid) - 1)
    gap = (grid[hi] - grid[lo]).astype(np.float32)
    p = np.where(gap > 0, (a - grid[lo].astype(np.float32)) / np.where(gap > 0, gap, 1), 0).astype(np.float32)
    return np.floor((p * np.float32(65536)).astype(np.float32)).astype(np.int64)


def cases(v, grid, seed):
    ft = thresholds(v, grid)
    ustar = 65536 - ft
    rng = np.random.default_rng(seed)
    us = [np.clip(ustar - 1, 0, 65535), np.clip(ustar, 0, 65535), np.zeros_like(ustar), np.full_like(ustar, 65535),
          rng.integers(0, 65536, size=v.shape)]
    vv = np.concatenate([v] * len(us)).astype(np.float32)
    uu = np.concatenate(us).astype(np.uint32)
    return vv, uu


def run(prog, v, u):
    exe, d = prog
    inp, out = d / "in.bin", d / "out.bin"
    with open(inp, "wb") as f:
        np.array([v.size], np.int64).tofile(f)
        v.astype(np.float32).tofile(f)
        u.astype(np.uint32).tofile(f)
    subprocess.run([str(exe), str(inp), str(out)], check=True, timeout=120)
    o = np.fromfile(out, dtype=np.uint8)
    return o[: v.size], o[v.size:]


def test_fp4_sr_instruction_matches_oracle(prog):
    grid = formats.E2M1_MAG
    v = np.concatenate([f32_range(2.0 ** -12, 6.0, 97), f32_range(0.0, 2.0 ** -12, 1 << 16),
                        grid, (grid[1:] + grid[:-1]) / 2, [6.0, 0.0]]).astype(np.float32)
    v = np.concatenate([v, -v])
    vv, uu = cases(v, grid, 1)
    got4, _ = run(prog, vv, uu)
    ref = formats.e2m1_sr(vv, uu.astype(np.uint16))
    bad = np.nonzero(got4 != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, e.g. v={vv[bad[:5]]} u={uu[bad[:5]]} got={got4[bad[:5]]} ref={ref[bad[:5]]}"


def test_fp8_sr_instruction_matches_oracle(prog):
    grid = formats.E4M3_POS
    v = np.concatenate([f32_range(2.0 ** -14, 448.0, 211), grid, (grid[1:] + grid[:-1]) / 2]).astype(np.float32)
    v = np.concatenate([v, -v])
    vv, uu = cases(v, grid, 2)
    _, got8 = run(prog, vv, uu)
    ref = formats.e4m3_sr(vv, uu.astype(np.uint16))
    bad = np.nonzero(got8 != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, e.g. v={vv[bad[:5]]} u={uu[bad[:5]]} got={got8[bad[:5]]} ref={ref[bad[:5]]}"
