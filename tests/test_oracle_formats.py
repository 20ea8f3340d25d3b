"""Pins for oracle.formats: E2M1 / E4M3FN codecs and element rounding rules.

Independent references: the published E2M1 grid, numpy's round-half-even
(np.rint) applied to a closed-form rescaling, torch's float8_e4m3fn
conversion, and statistical unbiasedness E[SR(x)] = x (TetraJet-v2 technical
summary, section 2.A).
"""
import numpy as np
import pytest
import torch

from oracle import formats


def all_f32_between(lo: float, hi: float, stride: int = 1) -> np.ndarray:
    a = int(np.float32(lo).view(np.uint32))
    b = int(np.float32(hi).view(np.uint32))
    return np.arange(a, b + 1, stride, dtype=np.uint32).view(np.float32)


def e2m1_rne_closed_form(v: np.ndarray) -> np.ndarray:
    """Independent RNE onto E2M1 magnitudes: per-binade rescale, np.rint (ties to even), rescale."""
    a = np.abs(v.astype(np.float64))
    # quantum: 0.5 below 2 (subnormal 0.5 step and binade [1,2)), 1 in [2,4), 2 in [4,8)
    q = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    r = np.rint(a / q) * q
    return np.minimum(r, 6.0)


def test_e2m1_grid_and_sign():
    assert list(formats.e2m1_decode(np.arange(8))) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    neg = formats.e2m1_decode(np.arange(8, 16))
    assert list(-neg) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert np.signbit(neg[0])  # code 8 is -0


@pytest.mark.parametrize("lo,hi,stride", [(0.0, 2.0 ** -4, 4099), (2.0 ** -4, 0.5, 1), (0.5, 2.0, 1), (2.0, 6.0, 1)])
def test_e2m1_rtn_exhaustive_vs_rint(lo, hi, stride):
    # every fp32 in [2^-4, 6] (stride 1), a strided sweep below
    v = all_f32_between(lo, hi, stride)
    for chunk in np.array_split(v, max(1, v.size // (1 << 22))):
        for sgn in (1.0, -1.0):
            c = chunk * np.float32(sgn)
            got = formats.e2m1_decode(formats.e2m1_rtn(c))
            ref = e2m1_rne_closed_form(c)
            np.testing.assert_array_equal(np.abs(got), ref)
            assert np.all(np.signbit(got) == np.signbit(c))


def test_e2m1_rtn_page_tie_example():
    # The pages' example: 0.25 sits exactly between the adjacent bins 0 and 0.5.
    codes = formats.e2m1_rtn(np.array([0.25, np.nextafter(np.float32(0.25), np.float32(1)),
                                       np.nextafter(np.float32(0.25), np.float32(0)), -0.25], np.float32))
    assert list(formats.e2m1_decode(codes)) == [0.0, 0.5, 0.0, -0.0]
    # every tie between neighbours goes to the even mantissa bit
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    assert list(formats.e2m1_decode(formats.e2m1_rtn(ties))) == [0, 1, 1, 2, 2, 4, 4]


def test_e2m1_sr_fixed_points_and_support():
    g = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    u = np.arange(0, 65536, 97, dtype=np.uint16)
    for x in g:
        out = formats.e2m1_decode(formats.e2m1_sr(np.full(u.shape, x, np.float32), u))
        assert np.all(out == x)
    v = np.float32(2.6)
    out = formats.e2m1_decode(formats.e2m1_sr(np.full(u.shape, v), u))
    assert set(np.unique(out)) <= {2.0, 3.0}


@pytest.mark.parametrize("x", [0.1, 0.3, 0.7, 1.2, 2.2, 3.3, 4.9, 5.5, -0.3, -4.9])
def test_e2m1_sr_unbiased(x):
    n = 1 << 20
    u = np.random.default_rng(123).integers(0, 65536, size=n, dtype=np.uint16)
    out = formats.e2m1_decode(formats.e2m1_sr(np.full(n, x, np.float32), u))
    mean = out.mean()
    gap = 2.0 if abs(x) >= 4 else 1.0 if abs(x) >= 2 else 0.5
    sigma = 0.5 * gap / np.sqrt(n)
    # 16-bit draws round up with probability floor(65536 p)/65536, so the mean sits below x
    # (towards zero) by less than gap/65536
    assert abs(mean - np.float32(x)) <= 5 * sigma + gap / 65536


def test_e2m1_sr_up_probability_within_draw_resolution():
    """Over all 65536 draws, the fraction rounded up differs from the exact position p of the
    value inside its grid gap (fp64, from the E2M1 grid) by less than 2^-16 and never exceeds
    it: E[SR(x)] = x up to the resolution of a 16-bit draw, with any bias towards zero."""
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    u = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = np.random.default_rng(9).uniform(0.0, 6.0, size=40).astype(np.float32)
    vals = np.concatenate([vals, np.float32([0.25, 1.25, 2.5, 5.0, 0.0001, 5.9999])])
    for v in vals:
        out = formats.e2m1_decode(formats.e2m1_sr(np.full(65536, v), u)).astype(np.float64)
        k = np.searchsorted(grid, float(v), side="right") - 1
        lo, hi = grid[k], grid[min(k + 1, 7)]
        assert set(np.unique(out)) <= {lo, hi}
        if hi == lo:
            continue
        p = (float(v) - lo) / (hi - lo)
        frac = np.count_nonzero(out == hi) / 65536.0
        assert p - 2.0 ** -16 < frac <= p, (float(v), frac, p)


def test_e2m1_sr_exact_probability():
    # with all 65536 draws the draws that round up are the largest ones (u >= 65536 - floor(t)),
    # the form gfx950's stochastic conversion takes its random operand in
    u = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = np.float32(1.2)  # between 1 and 1.5; fraction 0.4 -> t = 26214.4
    out = formats.e2m1_decode(formats.e2m1_sr(np.full(65536, v), u))
    assert (out == 1.5).sum() == 26214
    assert np.all(out[65536 - 26214:] == 1.5) and np.all(out[: 65536 - 26214] == 1.0)
    # a fraction of exactly one half: the top half of the draws rounds up
    out = formats.e2m1_decode(formats.e2m1_sr(np.full(65536, np.float32(1.25)), u))
    assert (out == 1.5).sum() == 32768 and out[32768] == 1.5 and out[32767] == 1.0


def test_e4m3_decode_vs_torch_and_constants():
    codes = np.arange(256, dtype=np.uint8)
    ours = formats.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    pos = formats.E4M3_POS
    assert pos.size == 127 and np.all(np.diff(pos) > 0)  # 0 plus 126 positive finite values
    assert pos[-1] == 448.0 and pos[1] == 2.0 ** -9 and pos[8] == 2.0 ** -6


def e4m3_dense_inputs():
    sample = all_f32_between(2.0 ** -12, 448.0, 61)
    grid = formats.E4M3_POS[1:].astype(np.float32)
    near = np.concatenate([grid, np.nextafter(grid, np.float32(0)), np.nextafter(grid, np.float32(1e9)),
                           ((grid[1:] + grid[:-1]) / 2).astype(np.float32)])
    near = near[(near > 0) & (near <= 448.0)]
    return np.concatenate([sample, near]).astype(np.float32)


def test_e4m3_round_up_vs_closed_form():
    r = e4m3_dense_inputs()
    got = formats.e4m3_decode(formats.e4m3_round_up(r))
    # closed form: quantum 2^-9 below 2^-6, else 2^(floor(log2 r) - 3); ceil to the quantum
    rr = r.astype(np.float64)
    m, e = np.frexp(rr)  # rr = m * 2^e, m in [0.5, 1)
    quantum = np.where(rr < 2.0 ** -6, 2.0 ** -9, np.ldexp(1.0, e - 1 - 3))
    ref = np.minimum(np.ceil(rr / quantum) * quantum, 448.0)
    np.testing.assert_array_equal(got, ref)
    assert np.all(got >= rr)


def test_e4m3_rne_vs_torch():
    v = e4m3_dense_inputs()
    v = np.concatenate([v, -v, [0.0, -0.0]]).astype(np.float32)
    ours = formats.e4m3_rne(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)


@pytest.mark.parametrize("x", [0.003, 0.3, 7.3, 100.0, 333.3])
def test_e4m3_sr_unbiased(x):
    n = 1 << 20
    u = np.random.default_rng(7).integers(0, 65536, size=n, dtype=np.uint16)
    out = formats.e4m3_decode(formats.e4m3_sr(np.full(n, x, np.float32), u))
    lo = formats.E4M3_POS[np.searchsorted(formats.E4M3_POS, x, side="right") - 1]
    hi = formats.E4M3_POS[np.searchsorted(formats.E4M3_POS, x, side="right")]
    gap = hi - lo
    assert set(np.unique(out)) <= {lo, hi}
    assert abs(out.mean() - np.float32(x)) <= 5 * 0.5 * gap / np.sqrt(n) + gap / 65536
