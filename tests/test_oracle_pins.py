"""Pins of the CPU oracle against what the pages and mathematics fix.

None of these checks retypes the oracle's own code: each compares it with a
closed form, an independent implementation (integer bit rules, exact rational
arithmetic, numpy routines), an invariant, a special case, or a fixture taken
from the pages. A plausible slip in the oracle (a dropped term, a wrong sign or
index, a transposed operand, a reversed coefficient order, an unfused
multiply-add, a wrong precedence among pred/ignore_src/src_size) fails at
least one of them.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from software_pipelining_amd import workloads
from tests.fp32_exact import bits, fma_f32, round_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- row shift
def _load_row_shift_golden():
    a, b = [], []
    with open(os.path.join(GOLDEN, "row_shift_arange_64x4.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            v = [int(t) for t in line.split()]
            a.append(v[1:5])
            b.append(v[5:9])
    return np.array(a, np.float32), np.array(b, np.float32)


def test_row_shift_worked_example_matches_page():
    # "Asynchronous Copies", "A Global-to-Shared Copy": arange(256) as 64x4,
    # expected output = roll(A, -1, dims=0)
    a, b_expected = _load_row_shift_golden()
    a_gen = workloads.arange_rows(64).numpy()
    assert np.array_equal(a, a_gen)
    b = oracle.row_shift(a_gen)
    assert np.array_equal(b.view(np.uint32), b_expected.view(np.uint32))
    # closed form of the same example: B[i, j] = 4 * ((i + 1) mod 64) + j
    i, j = np.meshgrid(np.arange(64), np.arange(4), indexing="ij")
    assert np.array_equal(b, (4 * ((i + 1) % 64) + j).astype(np.float32))


@pytest.mark.parametrize("rows", [1, 2, 3, 63, 64, 65, 1024])
def test_row_shift_equals_numpy_roll_bitwise(rows):
    a = workloads.random_rows(rows, seed=rows).numpy()
    b = oracle.row_shift(a)
    assert np.array_equal(b.view(np.uint32), np.roll(a, -1, axis=0).view(np.uint32))


@pytest.mark.parametrize("rows", [1, 5, 64])
def test_row_shift_invariants(rows):
    a = workloads.random_rows(rows, seed=100 + rows).numpy()
    b = a.copy()
    for _ in range(rows):
        b = oracle.row_shift(b)
    assert np.array_equal(b.view(np.uint32), a.view(np.uint32))   # order `rows` is identity
    one = oracle.row_shift(a).view(np.uint32)
    assert sorted(map(tuple, one)) == sorted(map(tuple, a.view(np.uint32)))  # a permutation of rows


# ------------------------------------------------------------------ scale2
def _double_bits_rule(u: np.ndarray) -> np.ndarray:
    """Bits of 2*x from the bits of x by integer rules of the binary32 format."""
    u = u.astype(np.uint64)
    sign = u & 0x80000000
    exp = (u >> 23) & 0xFF
    mant = u & 0x7FFFFF
    out = u + 0x800000                                   # normal: exponent + 1
    sub = exp == 0
    out = np.where(sub, sign | (mant << 1), out)         # zero/subnormal: shift mantissa
    out = np.where(exp == 254, sign | 0x7F800000, out)   # overflow to infinity
    out = np.where(exp == 255, u, out)                   # inf stays inf (NaN checked apart)
    return out.astype(np.uint32)


def test_scale2_integer_bit_rule():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    specials = np.array([0, 0x80000000, 1, 0x80000001, 0x007FFFFF, 0x00400000, 0x00800000,
                         0x7F7FFFFF, 0xFF7FFFFF, 0x7F000000, 0x7EFFFFFF, 0x7F800000,
                         0xFF800000, 0x3F800000, 0xBF800000], dtype=np.uint32)
    u = np.concatenate([specials, u])
    x = u.view(np.float32)
    y = oracle.pipelined_map(x, "scale2").view(np.uint32)
    nan = np.isnan(x)
    assert np.all(np.isnan(y.view(np.float32)[nan]))
    assert np.array_equal(y[~nan], _double_bits_rule(u)[~nan])


def test_scale2_on_workload_grid_and_copy_op():
    x = workloads.uniform_pm1(1 << 16, seed=1).numpy()
    y = oracle.pipelined_map(x, "scale2")
    assert np.array_equal(y.view(np.uint32), _double_bits_rule(x.view(np.uint32)))
    c = oracle.pipelined_map(x, "copy")
    assert np.array_equal(c.view(np.uint32), x.view(np.uint32))


# ---------------------------------------------------------------- horner32
def _coeffs_exact():
    return [round_f32(Fraction(1, k + 1)) for k in range(32)]


def test_horner_coefficients_are_rne_of_reciprocals():
    c = oracle.horner32_coeffs()
    ref = _coeffs_exact()
    assert [bits(v) for v in c] == [bits(v) for v in ref]
    for k in range(32):
        # within half an ulp of 1/(k+1)
        ulp = np.spacing(np.float32(c[k]))
        assert abs(Fraction(float(c[k])) - Fraction(1, k + 1)) <= Fraction(float(ulp)) / 2
        if (k + 1) & k == 0:   # k+1 a power of two: exact
            assert Fraction(float(c[k])) == Fraction(1, k + 1)
    assert np.all(np.diff(c) < 0)


def test_horner_at_zero_is_last_coefficient():
    # p(0) = c_31 = 1/32 for ascending k (descending k would give 1.0)
    for z in (0.0, -0.0):
        y = oracle.pipelined_map(np.array([z], np.float32), "horner32")
        assert bits(y[0]) == bits(np.float32(0.03125))


def _emulated_horner(x: np.float32, c) -> np.float32:
    y = np.float32(0.0)
    for k in range(32):
        y = fma_f32(y, x, c[k])
    return y


def test_fma_emulator_pins():
    # exact when the double result is exact: then one rounding to f32 is the fma
    rng = np.random.default_rng(11)
    a, b, c = (rng.standard_normal(300).astype(np.float32) for _ in range(3))
    n_checked = 0
    for ai, bi, ci in zip(a, b, c):
        d = float(ai) * float(bi) + float(ci)
        if Fraction(d) == Fraction(float(ai)) * Fraction(float(bi)) + Fraction(float(ci)):
            assert bits(fma_f32(ai, bi, ci)) == bits(np.float32(d))
            n_checked += 1
    assert n_checked > 50
    # a case where the unfused a*b+c differs from the fused result
    a1 = np.float32(1.0 + 2.0 ** -12)
    fused = fma_f32(a1, a1, np.float32(-1.0))             # exact: 2^-11 + 2^-24
    unfused = np.float32(np.float32(a1 * a1) - np.float32(1.0))   # a*a rounds first: 2^-11
    assert Fraction(float(fused)) == Fraction(2) ** -11 + Fraction(2) ** -24
    assert Fraction(float(unfused)) == Fraction(2) ** -11
    assert bits(fused) != bits(unfused)
    # ties to even and subnormal results
    assert bits(round_f32(Fraction(2 ** 24 + 1))) == bits(np.float32(2 ** 24))
    assert bits(round_f32(Fraction(2 ** 24 + 3))) == bits(np.float32(2 ** 24 + 4))
    assert bits(round_f32(Fraction(1, 2 ** 149))) == 1
    assert bits(round_f32(Fraction(1, 2 ** 150))) == 0       # tie to even (zero)
    assert bits(round_f32(Fraction(3, 2 ** 151))) == 1


def test_horner_matches_exact_rational_emulation():
    rng = np.random.default_rng(5)
    xs = workloads.uniform_pm1(1500, seed=4).numpy()
    edge = np.array([-1.0, -0.5, -2.0 ** -24, 0.0, -0.0, 2.0 ** -24, 2.0 ** -23, 0.5,
                     1.0 - 2.0 ** -24, 1.0, -1.0 + 2.0 ** -23, 0.999, -0.999, 1.5, -2.0, 3.0,
                     1e-30, -1e-30], np.float32)
    xs = np.concatenate([edge, xs, rng.uniform(-1, 1, 200).astype(np.float32)])
    got = oracle.pipelined_map(xs, "horner32")
    c = _coeffs_exact()
    for x, y in zip(xs, got):
        assert bits(y) == bits(_emulated_horner(x, c)), x


def test_horner_within_error_bound_of_exact_polynomial():
    # p(x) = sum_k x^(31-k) / (k+1) exactly; Horner with one rounding per step
    # plus rounded coefficients stays within (2*33) u sum_k |x|^(31-k)/(k+1).
    u = Fraction(1, 2 ** 24)
    xs = np.concatenate([np.array([-1.0, 1.0, -0.99, 0.99, -0.75, 0.75, 0.5, -0.5], np.float32),
                         workloads.uniform_pm1(300, seed=9).numpy()])
    got = oracle.pipelined_map(xs, "horner32")
    for x, y in zip(xs, got):
        fx = Fraction(float(x))
        p = sum(fx ** (31 - k) / (k + 1) for k in range(32))
        s = sum(abs(fx) ** (31 - k) / (k + 1) for k in range(32))
        assert abs(Fraction(float(y)) - p) <= 66 * u * s, x
    # at x = 1 the chain sums the harmonic numbers; at x = -1 an alternating sum
    assert abs(float(got[1]) - 4.0584954543) < 1e-5
    assert abs(float(got[0]) - float(sum(Fraction((-1) ** (31 - k), k + 1) for k in range(32)))) < 1e-5


def _subnormal_steps_exact(x: np.float32, c) -> int:
    """Independent count for one input: the exact products y*x of the chain
    (Fractions, so nothing rounds) that are nonzero and below 2^-126, with y
    advanced by the exact-rational fma."""
    tiny = Fraction(1, 2 ** 126)
    y, count = np.float32(0.0), 0
    for k in range(32):
        prod = Fraction(float(y)) * Fraction(float(x))
        if prod != 0 and abs(prod) < tiny:
            count += 1
        y = fma_f32(y, x, c[k])
    return count


def test_horner_subnormal_counter_positive_controls():
    # Closed forms. For a tiny x the products y*x are far below half an ulp of
    # c_k >= 2^-5, so every step returns y = c_k and step k >= 1 forms the
    # product c_{k-1} * x:
    #   x subnormal (1e-39, 2^-149, either sign): all 31 products from k = 1 on;
    #   x = 2^-122: c_{k-1} * 2^-122 < 2^-126 exactly when c_{k-1} < 1/16, i.e.
    #     k = 17..31 (k = 16 gives exactly 2^-126, the smallest normal): 15;
    #   x = 2^-120 or larger, x = 0: no product below 2^-126: 0.
    cases = {np.float32(1e-39): 31, np.float32(-1e-39): 31, np.float32(2.0 ** -149): 31,
             np.float32(2.0 ** -122): 15, np.float32(-(2.0 ** -122)): 15,
             np.float32(2.0 ** -120): 0, np.float32(0.0): 0, np.float32(-0.0): 0,
             np.float32(0.5): 0, np.float32(-1.0): 0}
    for x, n in cases.items():
        assert oracle.horner32_subnormal_steps(np.array([x], np.float32)) == n, float(x)
    # the counts add over inputs
    xs = np.array(list(cases), np.float32)
    assert oracle.horner32_subnormal_steps(xs) == sum(cases.values())
    # brute force against the exact-rational chain on a sweep of binades
    c = _coeffs_exact()
    rng = np.random.default_rng(5)
    sweep = [np.float32(s * m * 2.0 ** e) for e in range(-150, -110, 3)
             for s, m in ((1, 1.0), (-1, 1.37), (1, 1.9))]
    sweep += [np.float32(v) for v in rng.uniform(-1, 1, 20)]
    for x in sweep:
        assert oracle.horner32_subnormal_steps(np.array([x], np.float32)) == \
            _subnormal_steps_exact(x, c), float(x)


def test_horner_workload_sample_has_no_subnormal_steps():
    # rounding reading: the workload's inputs never produce a subnormal
    # intermediate, so flush-to-zero modes could not change a result on it
    x = workloads.uniform_pm1(1 << 20, seed=4).numpy()
    assert oracle.horner32_subnormal_steps(x) == 0


def test_map_range_split_does_not_change_results():
    x = workloads.uniform_pm1(300_001, seed=21).numpy()
    for op in ("scale2", "horner32"):
        a = oracle.pipelined_map(x, op, threads=1)
        b = oracle.pipelined_map(x, op, threads=7)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ---------------------------------------------------------------- 2-D map
def _window(rng, rows, cols, pad_cols, row0=2, col0=3):
    """A (rows, cols) view at (row0, col0) of a larger row-major buffer."""
    buf = rng.standard_normal((rows + row0 + 1, cols + col0 + pad_cols)).astype(np.float32)
    return buf, buf[row0:row0 + rows, col0:col0 + cols]


@pytest.mark.parametrize("rows,cols,spad,dpad", [(1, 1, 0, 0), (7, 13, 5, 0), (33, 64, 1, 9),
                                                  (5, 300, 17, 3), (64, 4, 60, 0)])
def test_map_2d_copy_and_scale2_equal_numpy_slices(rows, cols, spad, dpad):
    # a library routine (numpy slicing, exact multiply by two) on the same window
    rng = np.random.default_rng(rows * 1000 + cols)
    sbuf, src = _window(rng, rows, cols, spad)
    for op, ref in (("copy", lambda a: a.copy()), ("scale2", lambda a: a * np.float32(2))):
        dbuf, dst = _window(rng, rows, cols, dpad, row0=1, col0=0)
        before = dbuf.copy()
        oracle.map_2d(src, dst, op)
        expect = before.copy()
        expect[1:1 + rows, 0:cols] = ref(src)
        assert np.array_equal(dbuf.view(np.uint32), expect.view(np.uint32)), op


def test_map_2d_reduces_to_the_1d_map():
    # a contiguous window (stride == cols) is the 1-D map over rows*cols floats,
    # and any strided window is the 1-D map of its gathered elements
    x = workloads.uniform_pm1(37 * 29, seed=9).numpy()
    for op in ("scale2", "horner32", "copy"):
        dst = np.zeros((37, 29), np.float32)
        oracle.map_2d(x.reshape(37, 29), dst, op)
        assert np.array_equal(dst.reshape(-1).view(np.uint32),
                              oracle.pipelined_map(x, op).view(np.uint32))
    rng = np.random.default_rng(5)
    sbuf, src = _window(rng, 40, 50, 11)
    dbuf, dst = _window(rng, 40, 50, 3)
    oracle.map_2d(src, dst, "horner32", threads=3)
    gathered = oracle.pipelined_map(np.ascontiguousarray(src).reshape(-1), "horner32")
    assert np.array_equal(np.ascontiguousarray(dst).reshape(-1).view(np.uint32),
                          gathered.view(np.uint32))


def test_map_2d_empty_and_untouched():
    rng = np.random.default_rng(1)
    sbuf, src = _window(rng, 9, 9, 2)
    dbuf, _ = _window(rng, 9, 9, 2)
    before = dbuf.copy()
    oracle.map_2d(src[:0], dbuf[2:2, 3:12], "scale2")
    oracle.map_2d(src[:, :0], dbuf[2:11, 3:3], "scale2")
    assert np.array_equal(dbuf.view(np.uint32), before.view(np.uint32))
    with pytest.raises(ValueError):
        oracle.map_2d(src, dbuf[2:11, 3:11], "scale2")      # shapes differ


# -------------------------------------------------------------- chunk copy
def _golden_chunk_cases():
    cases = []
    with open(os.path.join(GOLDEN, "chunk_copy_rules.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            t = line.split()
            cases.append((int(t[0]), int(t[1]), int(t[2]), bytes.fromhex(t[3]),
                          bytes.fromhex(t[4]), bytes.fromhex(t[5])))
    return cases


def test_chunk_copy_golden_rules():
    cases = _golden_chunk_cases()
    n = len(cases)
    src = np.frombuffer(b"".join(c[3] for c in cases), np.uint8)
    dst = np.frombuffer(b"".join(c[4] for c in cases), np.uint8)
    pred = np.array([c[0] for c in cases], np.uint8)
    ign = np.array([c[1] for c in cases], np.uint8)
    size = np.array([c[2] for c in cases], np.uint8)
    out = oracle.chunk_copy(src, dst, pred, size, ign).reshape(n, 16)
    for k, c in enumerate(cases):
        assert out[k].tobytes() == c[5], k


@pytest.mark.parametrize("width", [4, 8, 16])
def test_chunk_copy_brute_force_all_operand_combinations(width):
    pred_vals = [0, 1, 7, 255]
    ign_vals = [0, 1, 200]
    size_vals = list(range(17)) + [17, 100, 255]
    combos = [(p, g, s) for p in pred_vals for g in ign_vals for s in size_vals]
    n = len(combos)
    rng = np.random.default_rng(3 + width)
    src = rng.integers(1, 256, size=(n, width), dtype=np.uint8)     # no zero bytes
    dst = rng.integers(1, 256, size=(n, width), dtype=np.uint8)
    pred = np.array([c[0] for c in combos], np.uint8)
    ign = np.array([c[1] for c in combos], np.uint8)
    size = np.array([c[2] for c in combos], np.uint8)
    out = oracle.chunk_copy(src, dst, pred, size, ign, chunk_bytes=width).reshape(n, width)
    for k, (p, g, s) in enumerate(combos):
        if p == 0:
            expect = dst[k]
        elif g != 0:
            expect = np.zeros(width, np.uint8)
        else:
            m = min(s, width)
            expect = np.concatenate([src[k, :m], np.zeros(width - m, np.uint8)])
        assert np.array_equal(out[k], expect), (width, p, g, s)


@pytest.mark.parametrize("width", [4, 8])
def test_chunk_copy_narrow_widths_special_cases(width):
    rng = np.random.default_rng(width)
    n = 5000
    src = rng.integers(0, 256, size=(n, width), dtype=np.uint8)
    dst = rng.integers(0, 256, size=(n, width), dtype=np.uint8)
    zeros, ones = np.zeros(n, np.uint8), np.ones(n, np.uint8)
    cc = lambda *m: oracle.chunk_copy(src, dst, *m, chunk_bytes=width)
    assert np.array_equal(cc(zeros, None, ones), dst)                       # all pred false
    assert np.array_equal(cc(None, None, None), src)                         # defaults: copy
    assert np.array_equal(cc(ones, np.full(n, width, np.uint8), zeros), src)
    assert not cc(None, zeros, None).any() and not cc(None, None, ones).any()
    # a chunk of `width` bytes equals the first `width` bytes of the 16-byte
    # chunk with the same operands and src_size capped at `width`
    size = rng.integers(0, 20, size=n).astype(np.uint8)
    pred = rng.integers(0, 2, size=n).astype(np.uint8)
    ign = (rng.random(n) < 0.1).astype(np.uint8)
    wide_src = np.zeros((n, 16), np.uint8)
    wide_src[:, :width] = src
    wide_dst = np.zeros((n, 16), np.uint8)
    wide_dst[:, :width] = dst
    wide = oracle.chunk_copy(wide_src, wide_dst, pred, np.minimum(size, width).astype(np.uint8), ign)
    assert np.array_equal(cc(pred, size, ign), wide[:, :width])
    with pytest.raises(ValueError):
        oracle.chunk_copy(src, dst, chunk_bytes=12)


def test_chunk_copy_special_cases_and_defaults():
    inp = workloads.chunk_copy_inputs(4096, seed=3)
    src, dst = inp.src.numpy(), inp.dst_init.numpy()
    n = src.shape[0]
    zeros = np.zeros(n, np.uint8)
    ones = np.ones(n, np.uint8)
    # every pred false: destination untouched
    assert np.array_equal(oracle.chunk_copy(src, dst, zeros, inp.src_size.numpy(), ones), dst)
    # size 16 and no ignore: a plain copy; all defaults (None): the same copy
    assert np.array_equal(oracle.chunk_copy(src, dst, ones, np.full(n, 16, np.uint8), zeros), src)
    assert np.array_equal(oracle.chunk_copy(src, dst), src)
    # size 0, or ignore set: zeros
    assert not oracle.chunk_copy(src, dst, None, zeros, None).any()
    assert not oracle.chunk_copy(src, dst, None, None, ones).any()
    # masked-assignment composition in numpy agrees on the workload's inputs
    p, s, g = inp.pred.numpy(), inp.src_size.numpy(), inp.ignore_src.numpy()
    eff = np.where(g != 0, 0, np.minimum(s, 16))
    keep = np.arange(16)[None, :] < eff[:, None]
    expect = np.where((p != 0)[:, None], np.where(keep, src, 0), dst)
    assert np.array_equal(oracle.chunk_copy(src, dst, p, s, g), expect)


def test_chunk_copy_in_place_and_range_split():
    inp = workloads.chunk_copy_inputs(70_001, seed=8)
    src, dst = inp.src.numpy(), inp.dst_init.numpy()
    meta = (inp.pred.numpy(), inp.src_size.numpy(), inp.ignore_src.numpy())
    a = oracle.chunk_copy(src, dst, *meta, threads=1)
    b = oracle.chunk_copy(src, dst, *meta, threads=5)
    assert np.array_equal(a, b)
    # src == dst: the result equals the copy from a separate source
    c = oracle.chunk_copy(src, src, *meta)
    assert np.array_equal(c, oracle.chunk_copy(src, src.copy(), *meta))


def test_workload_generators_are_deterministic_and_in_range():
    a = workloads.uniform_pm1(100_000, seed=2)
    b = workloads.uniform_pm1(100_000, seed=2)
    assert a.equal(b)
    x = a.numpy().astype(np.float64)
    assert x.min() >= -1.0 and x.max() < 1.0
    assert np.all(x * 2 ** 23 == np.round(x * 2 ** 23))      # on the 2^-23 grid
    inp = workloads.chunk_copy_inputs(200_000, seed=3)
    assert set(np.unique(inp.src_size.numpy())) <= {0, 4, 8, 12, 16}
    assert abs(inp.pred.numpy().mean() - 0.9) < 0.01
    assert abs(inp.ignore_src.numpy().mean() - 0.01) < 0.003
    assert np.all(inp.dst_init.numpy().view(np.uint32) == 0xDEADBEEF)


# ------------------------------------------------------- copies between workgroups
def _chunk_index_pattern(n):
    """n 256-byte chunks, chunk k made of the 32-bit word k repeated."""
    return np.repeat(np.arange(n, dtype=np.uint32), 64).view(np.uint8)


def test_workgroup_copy_closed_form():
    # "Copies between CTAs": each group's 256-byte chunk arrives in the next
    # group, which writes it: output chunk k holds the word k - 1 for k >= 1,
    # and chunk 0, which no group sends to, keeps its prior contents
    for n in (2, 3, 64, 1000):
        src = _chunk_index_pattern(n)
        fill = np.full(n * 64, 0xDEADBEEF, np.uint32).view(np.uint8)
        out = oracle.workgroup_copy(src, fill).view(np.uint32).reshape(n, 64)
        assert np.all(out[0] == 0xDEADBEEF)
        assert np.array_equal(out[1:], np.repeat(np.arange(n - 1, dtype=np.uint32)[:, None], 64, 1))


def test_workgroup_copy_against_numpy_roll():
    # a library routine: every chunk but the first equals numpy's roll of the
    # source by one chunk; random bytes catch a partial chunk or a byte order slip
    rng = np.random.default_rng(3)
    for n in (2, 7, 513):
        src = rng.integers(0, 256, n * 256, dtype=np.uint8)
        dst = rng.integers(0, 256, n * 256, dtype=np.uint8)
        out = oracle.workgroup_copy(src, dst, threads=3)
        rolled = np.roll(src.reshape(n, 256), 1, axis=0)
        assert np.array_equal(out.reshape(n, 256)[1:], rolled[1:])
        assert np.array_equal(out[:256], dst[:256])


def test_workgroup_copy_iterated_fills_from_chunk_zero():
    # invariant: feeding the output back n - 1 times (dst = the previous
    # output) carries chunk 0 into every chunk
    n = 9
    x = _chunk_index_pattern(n).copy()
    for _ in range(n - 1):
        x = oracle.workgroup_copy(x, x)
    assert np.all(x.view(np.uint32) == 0)


def test_workgroup_copy_degenerate_sizes():
    # no chunk or a single chunk: no group receives anything
    assert oracle.workgroup_copy(np.zeros(0, np.uint8), np.zeros(0, np.uint8)).size == 0
    one = np.arange(256, dtype=np.uint8)
    assert np.array_equal(oracle.workgroup_copy(np.zeros(256, np.uint8), one), one)
    with pytest.raises(ValueError):
        oracle.workgroup_copy(np.zeros(300, np.uint8), np.zeros(300, np.uint8))
