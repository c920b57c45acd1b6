"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each ``pin_*`` function takes the oracle module and raises AssertionError when
the oracle disagrees with a closed form, an invariant, brute force on tiny
inputs, a library routine, or a value printed on the pages.  The same functions
are run against deliberately broken copies of the oracle in
``test_oracle_mutations.py`` to show that each plausible mistake is caught.
"""
from __future__ import annotations

import functools
import math
import pathlib

import numpy as np

GOLDEN = pathlib.Path(__file__).parent / "golden"
SIZES = (4, 16, 64, 256, 1024)


# ---------------------------------------------------------------- helpers
def _closed_form_entry(i: int, j: int, g: int) -> int:
    """(-1)^(number of base-4 digits where i and j agree), by digit loops."""
    equal = 0
    n = g
    while n > 1:
        if i % 4 == j % 4:
            equal += 1
        i //= 4
        j //= 4
        n //= 4
    return -1 if equal % 2 else 1


def _sylvester(n: int) -> np.ndarray:
    h = np.ones((1, 1))
    h2 = np.array([[1.0, 1.0], [1.0, -1.0]])
    while h.shape[0] < n:
        h = np.kron(h, h2)
    return h


@functools.lru_cache(maxsize=1)
def _order4_hadamards():
    """All order-4 +-1 matrices M with M M^T = 4 I, by exhaustive enumeration of 2^16."""
    bits = np.arange(1 << 16, dtype=np.int64)[:, None] >> np.arange(16)[None, :]
    mats = np.where(bits & 1, 1.0, -1.0).reshape(-1, 4, 4)
    gram = np.einsum("aij,akj->aik", mats, mats)
    keep = np.all(gram == 4 * np.eye(4), axis=(1, 2))
    return tuple(mats[keep])


def _is_regular(h: np.ndarray) -> bool:
    rs = h.sum(axis=1)
    cs = h.sum(axis=0)
    return bool(np.all(rs == rs[0]) and np.all(cs == rs[0]))


def _bf16_values(rng, shape, scale=1.0):
    import torch
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()


# ---------------------------------------------------------------- group size
def pin_power_of_four_golden(o):
    """Golden cases: the author's sizes and the 2^58 case of the review."""
    for line in (GOLDEN / "power_of_four.txt").read_text().splitlines():
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        verdict, expr = line.split(None, 1)
        value = eval(expr, {"__builtins__": {}})  # integer literals / powers only
        assert o.is_power_of_four(value) == (verdict == "accept"), (verdict, expr)
        if verdict == "reject":
            try:
                o.check_group_size(value)
            except ValueError as e:
                assert str(e) == f"Regular Hadamard size must be a power of 4, got {value}"
            else:
                raise AssertionError(f"{expr} accepted")
    # The float test the review replaces really does reject 4^29.
    assert math.log(2 ** 58, 4) % 1 != 0
    assert o.is_power_of_four(2 ** 58)


# ---------------------------------------------------------------- Hadamard
def pin_hadamard_definition(o):
    """Def. 2.1: entries +-1 and H H^T = g I."""
    for g in SIZES:
        h = o.regular_hadamard(g)
        assert h.shape == (g, g)
        assert np.all(np.abs(h) == 1.0)
        assert np.array_equal(h @ h.T, g * np.eye(g))


def pin_regular(o):
    """Def. 2.3 (reading): every row and column sums to the same value, +sqrt(g)."""
    for g in SIZES:
        h = o.regular_hadamard(g)
        r = math.isqrt(g)
        assert np.all(h.sum(axis=0) == r) and np.all(h.sum(axis=1) == r)


def pin_closed_form_entries(o):
    """Thm. 2.3 (Kronecker construction): entry formula over base-4 digits."""
    for g in (4, 16, 64, 256):
        h = o.regular_hadamard(g)
        ref = np.array([[_closed_form_entry(i, j, g) for j in range(g)] for i in range(g)])
        assert np.array_equal(h, ref)
    h = o.regular_hadamard(1024)
    rng = np.random.default_rng(7)
    for i, j in rng.integers(0, 1024, size=(4000, 2)):
        assert h[i, j] == _closed_form_entry(int(i), int(j), 1024)


def pin_symmetric_involution(o):
    for g in SIZES:
        h = o.regular_hadamard(g)
        assert np.array_equal(h, h.T)
        assert np.array_equal(h @ h, g * np.eye(g))


def pin_column_sum_squared(o):
    """Thm. 2.1 (reading): sum_j (column sum_j)^2 = g^2 for every H-matrix."""
    rng = np.random.default_rng(3)
    for g in SIZES:
        mats = [o.regular_hadamard(g), _sylvester(g)]
        for _ in range(3):
            p = np.eye(g)[rng.permutation(g)]
            d = np.diag(rng.choice([-1.0, 1.0], size=g))
            mats.append(d @ p @ _sylvester(g))
        for h in mats:
            assert np.sum(h.sum(axis=0) ** 2) == g * g


def pin_order4_enumeration(o):
    """Brute force over all 2^16 order-4 +-1 matrices.

    768 are Hadamard.  Every one has column discrepancy max_j |column sum| >= 2
    = sqrt(4) (Thm. 2.1 with Def. 2.2, reading); the 48 regular ones (Def. 2.3)
    attain that minimum, and the base matrix is one of them.
    """
    had = _order4_hadamards()
    assert len(had) == 768
    disc = [np.max(np.abs(h.sum(axis=0))) for h in had]
    assert min(disc) == 2
    regular = [h for h in had if _is_regular(h)]
    assert len(regular) == 48
    assert all(np.max(np.abs(h.sum(axis=0))) == 2 for h in regular)
    base = o.base_regular_hadamard()
    assert any(np.array_equal(base, h) for h in regular)
    assert np.all(base.sum(axis=0) == 2)


def pin_kronecker_closure(o):
    """Thm. 2.3: Kronecker products of regular H-matrices are regular H-matrices."""
    regular = [h for h in _order4_hadamards() if _is_regular(h)]
    for a in regular:
        for b in regular:
            k = np.kron(a, b)
            assert np.array_equal(k @ k.T, 16 * np.eye(16))
            assert _is_regular(k)
    for g in SIZES[1:]:
        assert _is_regular(o.regular_hadamard(g))


def pin_sylvester_not_regular(o):
    s = _sylvester(256)
    cs = s.sum(axis=0)
    assert sorted(set(cs.tolist())) == [0.0, 256.0]
    assert not _is_regular(s)
    assert _is_regular(o.regular_hadamard(256))


# ---------------------------------------------------------------- rotation
def pin_rotation_constant_row(o):
    """A constant row rotates to the same constant (equal column sums; Fig. 1)."""
    for g in SIZES:
        for c in (3.0, -0.75, 3.0 * 2.0 ** -20):
            x = np.full((2, 2 * g), c)
            y = o.rotate_groups(x, g)
            assert np.array_equal(y, x)


def pin_rotation_vs_sylvester_energy(o):
    """Fig. 1/2 direction: Sylvester concentrates a row-wise outlier, regular does not."""
    g, c = 256, 3.0
    x = np.full((1, g), c)
    syl = (x @ _sylvester(g).T) / 16.0
    assert np.max(np.abs(syl)) == 48.0
    assert np.max(np.abs(o.rotate_groups(x, g))) == 3.0


def pin_rotation_one_hot(o):
    for g in SIZES:
        h = o.regular_hadamard(g)
        for j in (0, 1, g // 3, g - 1):
            x = np.zeros((1, g))
            x[0, j] = 1.0
            y = o.rotate_groups(x, g)
            assert np.array_equal(y[0], h[j] / math.isqrt(g))
            ref = np.array([_closed_form_entry(i, j, g) for i in range(g)]) / math.isqrt(g)
            assert np.array_equal(y[0], ref)


def pin_rotation_involution(o):
    """(H/sqrt g)^2 = I: rotating twice returns small-integer inputs exactly."""
    rng = np.random.default_rng(5)
    for g in SIZES:
        x = rng.integers(-20, 21, size=(3, 3 * g)).astype(np.float64)
        assert np.array_equal(o.rotate_groups(o.rotate_groups(x, g), g), x)


def pin_rotation_norm_linearity(o):
    rng = np.random.default_rng(6)
    for g in SIZES:
        x = rng.standard_normal((4, 2 * g))
        z = rng.standard_normal((4, 2 * g))
        yx = o.rotate_groups(x, g)
        for w in range(2):
            a = np.linalg.norm(x[:, w * g:(w + 1) * g], axis=1)
            b = np.linalg.norm(yx[:, w * g:(w + 1) * g], axis=1)
            assert np.allclose(a, b, rtol=1e-13)
        assert np.allclose(o.rotate_groups(2 * x - z, g), 2 * yx - o.rotate_groups(z, g),
                           rtol=1e-12, atol=1e-12)


def pin_rotation_brute_force_padded(o):
    """Pure-Python loops on tiny ragged rows, zero padding to whole windows."""
    rng = np.random.default_rng(8)
    for g, K in ((4, 7), (16, 37), (64, 65), (16, 16)):
        x = rng.integers(-9, 10, size=(3, K)).astype(np.float64) / 4.0
        y = o.rotate_groups(x, g)
        Kp = -(-K // g) * g
        assert y.shape == (3, Kp)
        k = int(round(math.log(g, 4)))
        for m in range(3):
            for p in range(Kp):
                w0 = (p // g) * g
                acc = 0.0
                for j in range(g):
                    xv = x[m, w0 + j] if w0 + j < K else 0.0
                    acc += _closed_form_entry(p - w0, j, g) * xv
                assert y[m, p] == acc / 2 ** k


def pin_rotation_exact_fsum(o):
    """The float64 rotation equals the exactly rounded sum (math.fsum) on bf16 data."""
    rng = np.random.default_rng(9)
    for g in (16, 256, 1024):
        x = _bf16_values(rng, (3, 2 * g), scale=1.0)
        x[0, :] *= 50.0
        x[:, 5] *= 30.0
        y = o.rotate_groups(x, g)
        k = int(round(math.log(g, 4)))
        for _ in range(40):
            m = int(rng.integers(0, 3))
            p = int(rng.integers(0, 2 * g))
            w0 = (p // g) * g
            terms = [_closed_form_entry(p - w0, j, g) * float(x[m, w0 + j]) for j in range(g)]
            assert y[m, p] == math.fsum(terms) / 2 ** k


def _rne_f32_exact(v: float) -> float:
    """Round-to-nearest-even of a finite float64 to the float32 grid, in exact rational
    arithmetic: the quantum is 2^(e - 23) in the binade [2^e, 2^(e + 1)), and 2^-149 below
    2^-126 (the subnormals)."""
    from fractions import Fraction
    if v == 0.0:
        return v
    a = Fraction(abs(v))
    e = math.frexp(abs(v))[1] - 1          # 2^e <= |v| < 2^(e + 1)
    quantum = Fraction(2) ** (max(e, -126) - 23)
    n = a / quantum
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return math.copysign(float(lo * quantum), v)


def pin_to_f32(o):
    """The single fp64 -> fp32 rounding of the rotated values (it fixes every scale and code):
    round to nearest, ties to the even significand, also among the subnormals.  Checked
    against exact rational rounding and against C's float conversion (struct 'f'), on random
    values of every magnitude and on values constructed exactly halfway between adjacent
    float32 numbers (and one float64 step to either side of the midpoint)."""
    import struct
    rng = np.random.default_rng(40)
    mags = np.concatenate([rng.uniform(-126, 127, 3000), rng.uniform(-149, -126, 1000)])
    vals = np.exp2(mags) * rng.uniform(1.0, 2.0, mags.size)
    vals *= np.where(rng.random(vals.size) < 0.5, -1.0, 1.0)
    got = o.to_f32(vals)
    assert got.dtype == np.float32
    for v, r in zip(vals.tolist(), got.tolist()):
        want = _rne_f32_exact(v)
        assert r == want, (v, r, want)
        assert struct.unpack("<f", struct.pack("<f", v))[0] == want
    # midpoints between float32 neighbours b and b + 1: normal, subnormal, binade edges
    bits = np.concatenate([rng.integers(0x00800000, 0x7F7FFFFE, 3000),
                           rng.integers(0, 0x007FFFFF, 1000),
                           [0, 1, 2, 0x007FFFFE, 0x007FFFFF, 0x00800000, 0x3F7FFFFF,
                            0x3F800000, 0x7F7FFFFD]]).astype(np.uint32)
    lo = bits.view(np.float32).astype(np.float64)
    hi = (bits + np.uint32(1)).view(np.float32).astype(np.float64)
    mid = (lo + hi) / 2.0                   # exact: both have 24-bit significands
    even = np.where(bits % 2 == 0, lo, hi)
    below, above = np.nextafter(mid, -np.inf), np.nextafter(mid, np.inf)
    for sign in (1.0, -1.0):
        assert np.array_equal(o.to_f32(sign * mid).astype(np.float64), sign * even)
        assert np.array_equal(o.to_f32(sign * below).astype(np.float64), sign * lo)
        assert np.array_equal(o.to_f32(sign * above).astype(np.float64), sign * hi)
    assert np.signbit(o.to_f32(np.array([-0.0, -2.0 ** -151]))).all()   # -0 stays -0


# ---------------------------------------------------------------- quantization
def pin_quant_round_trip(o):
    """Rows s * (integers in [-7, 7]) with 7 present come back exactly."""
    rng = np.random.default_rng(10)
    ints = rng.integers(-7, 8, size=(6, 64))
    ints[:, 3] = 7
    ints[2, 3] = -7
    ints[2, 9] = 5
    s = (rng.integers(1, 64, size=6) * np.exp2(rng.integers(-10, 4, size=6))).astype(np.float32)
    yf = (ints * s[:, None].astype(np.float64)).astype(np.float32)
    sc = o.row_scales(yf)
    assert np.array_equal(sc, s)
    assert np.array_equal(o.quantize(yf, sc), ints.astype(np.int8))


def pin_quant_absmax_and_range(o):
    rng = np.random.default_rng(11)
    yf = (rng.standard_normal((50, 300)) * np.exp2(rng.integers(-8, 8, size=(50, 1)))).astype(np.float32)
    s = o.row_scales(yf)
    q = o.quantize(yf, s)
    am = np.argmax(np.abs(yf), axis=1)
    assert np.array_equal(np.abs(q[np.arange(50), am]), np.full(50, 7))
    assert q.min() >= -7 and q.max() <= 7


def pin_quant_power_of_two_scaling(o):
    rng = np.random.default_rng(12)
    yf = rng.standard_normal((8, 128)).astype(np.float32)
    s = o.row_scales(yf)
    q = o.quantize(yf, s)
    for e in (-5, 3):
        y2 = (yf * np.float32(2.0 ** e)).astype(np.float32)
        s2 = o.row_scales(y2)
        assert np.array_equal(s2, (s * np.float32(2.0 ** e)).astype(np.float32))
        assert np.array_equal(o.quantize(y2, s2), q)


def pin_quant_zero_row(o):
    yf = np.zeros((2, 32), dtype=np.float32)
    yf[1, 4] = 1.0
    s = o.row_scales(yf)
    assert s[0] == 0.0
    q = o.quantize(yf, s)
    assert np.all(q[0] == 0)
    assert q[1, 4] == 7


def pin_quant_ties_even(o):
    """Round half to even: 2.5 -> 2, 3.5 -> 4, -2.5 -> -2, 0.5 -> 0, 1.5 -> 2."""
    yf = np.array([[7.0, 2.5, 3.5, -2.5, 0.5, -0.5, 1.5, -6.5]], dtype=np.float32)
    s = o.row_scales(yf)
    assert s[0] == np.float32(1.0)
    assert o.quantize(yf, s).tolist() == [[7, 2, 4, -2, 0, 0, 2, -6]]


def pin_pack_layout(o):
    assert o.pack_int4(np.array([[1, -1]])).tolist() == [[0xF1]]
    assert o.pack_int4(np.array([[-8, 7]])).tolist() == [[0x78]]
    assert o.pack_int4(np.array([[0, -8, 3, 2]])).tolist() == [[0x80, 0x23]]
    allb = np.arange(256, dtype=np.uint8).reshape(2, 128)
    assert np.array_equal(o.pack_int4(o.unpack_int4(allb)), allb)
    codes = np.array([[c0, c1] for c0 in range(-8, 8) for c1 in range(-8, 8)]).reshape(1, -1)
    assert np.array_equal(o.unpack_int4(o.pack_int4(codes)), codes.astype(np.int8))
    # brute-force nibble reading: element 2j low nibble, 2j+1 high nibble
    b = o.pack_int4(codes)
    for j in range(b.shape[1]):
        lo, hi = int(b[0, j]) & 15, int(b[0, j]) >> 4
        assert (lo - 16 if lo >= 8 else lo) == codes[0, 2 * j]
        assert (hi - 16 if hi >= 8 else hi) == codes[0, 2 * j + 1]


# ---------------------------------------------------------------- GEMM, dequant
def pin_int_gemm_brute_force(o):
    rng = np.random.default_rng(13)
    for M, N, K in ((3, 5, 64), (7, 2, 16), (16, 16, 64)):
        qx = rng.integers(-8, 8, size=(M, K))
        qw = rng.integers(-8, 8, size=(N, K))
        acc = o.int_gemm(qx.astype(np.int8), qw.astype(np.int8))
        for m in range(M):
            for n in range(N):
                s = 0
                for k in range(K):
                    s += int(qx[m, k]) * int(qw[n, k])
                assert acc[m, n] == s
    K = 16384
    full = np.full((1, K), -8, dtype=np.int8)
    assert o.int_gemm(full, full)[0, 0] == 64 * K


def pin_bf16_rounding_vs_torch(o):
    import torch
    rng = np.random.default_rng(14)
    z = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, size=20000))).astype(np.float32)
    u = z.view(np.uint32).copy()
    u[:2000] = (u[:2000] & 0xFFFF0000) | 0x8000       # exact ties
    u[2000:4000] = (u[2000:4000] & 0xFFFF0000) | 0x7FFF
    u[4000:6000] = (u[4000:6000] & 0xFFFF0000) | 0x8001
    z = u.view(np.float32)
    ref = torch.from_numpy(z.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(o.f32_to_bf16_bits(z), ref)
    assert np.array_equal(o.bf16_bits_to_f32(ref),
                          torch.from_numpy(ref.view(np.int16).copy()).view(torch.bfloat16)
                          .to(torch.float32).numpy())


def pin_end_to_end_closed_form(o):
    """Constant rows: codes +-7, scales |c|/7, acc = 49 K' sign, out = bf16(K' c d + b)."""
    import torch
    for g, K, c, d, b in ((16, 64, 7.0, 14.0, 0.5), (16, 64, 0.875, 0.4375, 3.0),
                          (256, 512, -3.5, 1.75, None),
                          (64, 100, 0.875, -7.0, -2.0), (1024, 1024, 2.0, 3.5, None)):
        Kp = -(-K // g) * g
        x = np.full((3, K), c)
        w = np.full((2, K), d)
        bias = None if b is None else np.full(2, b, dtype=np.float32)
        r = o.convlinear4bit(x, w, bias, g)
        padded = Kp != K
        if not padded:
            assert np.all(np.abs(r["x"]["codes"]) == 7) and np.all(np.abs(r["w"]["codes"]) == 7)
            assert np.all(r["x"]["scale"] == np.float32(abs(c) / 7))
            assert np.all(r["w"]["scale"] == np.float32(abs(d) / 7))
            assert np.all(r["acc"] == 49 * Kp * int(np.sign(c) * np.sign(d)))
        exact = K * c * d + (0.0 if b is None else b)
        want = torch.tensor([exact], dtype=torch.float32).to(torch.bfloat16).view(torch.int16)
        if not padded:
            assert np.all(r["out_bits"] == np.uint16(want.numpy().view(np.uint16)[0]))
        else:
            out = o.bf16_bits_to_f32(r["out_bits"])
            assert np.allclose(out, exact, rtol=0.15)


def pin_int4_linear_semantics(o):
    """[KITCHEN] int4_linear: x @ w^T on unpacked codes, row scale, column scale, bias."""
    rng = np.random.default_rng(15)
    qx = rng.integers(-8, 8, size=(5, 32)).astype(np.int8)
    qw = rng.integers(-8, 8, size=(4, 32)).astype(np.int8)
    sx = np.array([0.5, 0.25, 2.0, 1.0, 0.125], dtype=np.float32)
    sw = np.array([1.0, 0.5, 4.0, 0.0625], dtype=np.float32)
    b = np.array([1.0, -2.0, 0.0, 0.5], dtype=np.float32)
    r = o.w4a4_linear_from_codes(qx, sx, qw, sw, b)
    acc = qx.astype(np.int64) @ qw.astype(np.int64).T
    exact = acc * sx[:, None].astype(np.float64) * sw[None, :].astype(np.float64) + b[None, :]
    # power-of-two scales keep every product exact; bf16 of exact values
    import torch
    want = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(r["out_bits"], want.view(np.uint16))
    assert np.array_equal(r["acc"], acc)


# ---------------------------------------------------------------- INT8 variant ([HSWQ])
def pin_int8_round_trip(o):
    """Rows 2^e * (integers in [-127, 127]) with |127| present come back exactly, and the
    row scale is 2^e (127 * 2^e / 127 is exact)."""
    rng = np.random.default_rng(20)
    ints = rng.integers(-127, 128, size=(6, 96))
    ints[:, 5] = 127
    ints[3, 5] = -127
    e = rng.integers(-12, 6, size=6)
    s = np.exp2(e).astype(np.float32)
    yf = (ints * s[:, None].astype(np.float64)).astype(np.float32)
    r = o.row_scales(yf, o.INT8_QMAX)
    assert np.array_equal(r, s)
    assert np.array_equal(o.quantize(yf, r, o.INT8_QMAX, o.INT8_QMIN), ints.astype(np.int8))


def pin_int8_rotate_quantize(o):
    """The INT8 path is the same rotation with q_max 127: scale = fp32(absmax / 127), the
    absmax element maps to +-127, codes in [-127, 127], and |code - rotated/scale| <= 1/2."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((9, 300)).astype(np.float32)
    x[2] *= 40.0
    for g in (16, 64, 256):
        r = o.rotate_quantize_int8(x, g)
        yf = o.to_f32(o.rotate_groups(x, g))
        assert np.array_equal(r["yf"], yf)
        amax = np.max(np.abs(yf), axis=1)
        assert np.array_equal(r["scale"], (amax / np.float32(127)).astype(np.float32))
        q = r["codes"].astype(np.int64)
        assert q.shape == yf.shape and q.min() >= -127 and q.max() <= 127
        am = np.argmax(np.abs(yf), axis=1)
        assert np.array_equal(np.abs(q[np.arange(9), am]), np.full(9, 127))
        z = yf.astype(np.float64) / r["scale"][:, None].astype(np.float64)
        assert np.max(np.abs(q - z)) <= 0.5 + 1e-6
        # the same rotation and scales, only q_max differs from the int4 path
        r4 = o.rotate_quantize(x, g)
        assert np.array_equal(r4["yf"], r["yf"])
        assert np.array_equal(r4["scale"], (amax / np.float32(7)).astype(np.float32))


def pin_int8_gemm_brute_force(o):
    """Exact int32 sums over the full int8 range, by a triple loop; the largest magnitude
    16384 K' still fits int32 at K' = 65536 - 128."""
    rng = np.random.default_rng(22)
    for M, N, K in ((4, 3, 64), (2, 5, 32)):
        qx = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
        qw = rng.integers(-128, 128, size=(N, K)).astype(np.int8)
        acc = o.int_gemm(qx, qw)
        for m in range(M):
            for n in range(N):
                assert acc[m, n] == sum(int(qx[m, k]) * int(qw[n, k]) for k in range(K))
    K = 65536 - 128
    full = np.full((1, K), -128, dtype=np.int8)
    assert o.int_gemm(full, full)[0, 0] == 16384 * K < 2 ** 31


def pin_int8_dequant_rounds_large_sums(o):
    """fp32(acc) is the round-to-nearest-even conversion once |acc| >= 2^24."""
    acc = np.array([[2 ** 24 + 1, 2 ** 24 + 3, -(2 ** 25 + 2), 127 * 127 * 3072]], dtype=np.int64)
    one = np.ones(1, dtype=np.float32)
    ones = np.ones(4, dtype=np.float32)
    got = o.bf16_bits_to_f32(o.dequantize(acc, one, ones)).astype(np.float64)
    want = [float(np.float32(v)) for v in acc[0]]            # IEEE RNE int -> fp32
    import torch
    want = torch.tensor(want, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got[0], want)
    assert float(np.float32(2 ** 24 + 1)) == 2.0 ** 24 and float(np.float32(2 ** 24 + 3)) == 2.0 ** 24 + 4


def pin_int8_end_to_end_closed_form(o):
    """Constant rows: codes +-127, scales |c|/127, acc = 127^2 K sign, out = bf16(K c d)."""
    import torch
    for g, K, c, d in ((16, 64, 2.0, 0.5), (256, 512, -4.0, 0.25), (64, 128, 1.0, -1.0)):
        x = np.full((2, K), c)
        w = np.full((3, K), d)
        r = o.convlinear8bit(x, w, None, g)
        assert np.all(np.abs(r["x"]["codes"]) == 127) and np.all(np.abs(r["w"]["codes"]) == 127)
        assert np.all(r["x"]["scale"] == np.float32(abs(c) / 127))
        assert np.all(r["acc"] == 127 * 127 * K * int(np.sign(c) * np.sign(d)))
        z = np.float32(np.float32(np.float32(127 * 127 * K * np.sign(c * d)) * np.float32(abs(c) / 127))
                       * np.float32(abs(d) / 127))
        want = torch.tensor([float(z)], dtype=torch.float32).to(torch.bfloat16).view(torch.int16)
        assert np.all(r["out_bits"] == np.uint16(want.numpy().view(np.uint16)[0]))
        assert abs(float(z) - K * c * d) <= 1e-5 * abs(K * c * d)


# ------------------------------------------------- MXFP4 (OCP Microscaling v1.0)
def _rne_e2m1_by_binade(a: float) -> float:
    """Independent E2M1 rounding of a magnitude: one mantissa bit above 1 (steps of 2^(e-1) in
    [2^e, 2^(e+1))), steps of 0.5 below 1, Python's round() for ties to even, clamp at 6."""
    if a < 1.0:
        r = round(2.0 * a) / 2.0
    else:
        e = math.floor(math.log2(a))
        step = 2.0 ** (e - 1)
        r = round(a / step) * step
    return min(r, 6.0)


def pin_e2m1_format(o):
    """E2M1: eight magnitudes 0 < 0.5 < 1 < ... < 6 (largest normal 1.5 * 2^2, smallest
    subnormal 0.5), codes 8-15 the negatives, and every magnitude encodes back to its code."""
    v = o.e2m1_decode(np.arange(16))
    assert np.all(np.diff(v[:8]) > 0) and v[0] == 0.0
    assert v[7] == 1.5 * 2 ** 2 and v[1] == 0.5 and v[2] == 1.0
    assert np.array_equal(v[8:], -v[:8])
    assert np.array_equal(o.e2m1_encode(v[:8]), np.arange(8))
    assert np.array_equal(o.e2m1_encode(-v[1:8]), np.arange(9, 16))
    assert o.e2m1_encode(np.array([-0.0]))[0] == 8 and o.e2m1_encode(np.array([0.0]))[0] == 0


def pin_e2m1_rounding(o):
    """Nearest value with ties to the even mantissa and saturation at 6, against an
    independent per-binade rounding (Python's round) on random and tie inputs."""
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0]
    assert list(o.e2m1_decode(o.e2m1_encode(np.array(ties)))) == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0,
                                                                  4.0, 6.0]
    rng = np.random.default_rng(30)
    a = np.concatenate([rng.uniform(0, 8, 2000), rng.uniform(0, 100, 200), np.array(ties)])
    got = o.e2m1_decode(o.e2m1_encode(a))
    want = np.array([_rne_e2m1_by_binade(float(t)) for t in a])
    assert np.array_equal(got, want)
    assert np.array_equal(o.e2m1_decode(o.e2m1_encode(-a)), -want)


def pin_mx_block_scale(o):
    """The shared exponent puts every nonzero block's absmax / scale in [4, 8): the block
    maximum always encodes to 4 or 6; an all-zero block takes 2^-127; scaling a block by 2^j
    shifts its exponent by j and leaves its codes alone."""
    rng = np.random.default_rng(31)
    y = rng.standard_normal((5, 256)) * np.exp2(rng.integers(-20, 20, size=(5, 1)))
    y[2, 32:64] = 0.0
    e = o.mx_block_exponents(y)
    assert e.shape == (5, 8), "one shared exponent per 32 values"
    blocks = np.abs(y.reshape(5, 8, 32)).max(axis=2)
    live = blocks > 0
    ratio = blocks[live] / np.exp2(e[live].astype(np.float64))
    assert np.all((ratio >= 4) & (ratio < 8))
    assert e[2, 1] == -127
    codes, e8 = o.quantize_mxfp4(y)
    top = np.abs(o.e2m1_decode(codes)).reshape(5, 8, 32).max(axis=2)
    assert np.all(np.isin(top[live], [4.0, 6.0]))
    codes2, e82 = o.quantize_mxfp4(y * 2.0 ** 7)
    assert np.array_equal(codes2, codes) and np.array_equal(e82[live], e8[live] + 7)
    assert np.array_equal(e8, (e + 127).astype(np.uint8))


def pin_mxfp4_round_trip(o):
    """Blocks of E2M1 values times 2^j whose largest magnitude is 4 or 6 come back exactly."""
    rng = np.random.default_rng(32)
    vals = o.e2m1_decode(rng.integers(0, 16, size=(4, 128)))
    vals[:, ::32] = rng.choice([4.0, -4.0, 6.0, -6.0], size=(4, 4))
    j = rng.integers(-30, 30, size=(4, 4))
    y = vals * np.repeat(np.exp2(j.astype(np.float64)), 32, axis=1)
    codes, e8 = o.quantize_mxfp4(y)
    assert np.array_equal(o.mxfp4_values(codes, e8), y)
    assert np.array_equal(e8.astype(np.int64), j + 127)


def pin_mxfp4_gemm_brute_force(o):
    """The float64 sum of decoded products equals exact rational arithmetic (fractions)."""
    from fractions import Fraction
    rng = np.random.default_rng(33)
    for M, N, K in ((3, 2, 64), (2, 3, 32)):
        cx = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
        cw = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
        ex = rng.integers(120, 136, size=(M, K // 32)).astype(np.uint8)
        ew = rng.integers(120, 136, size=(N, K // 32)).astype(np.uint8)
        r = o.mxfp4_linear_from_codes(cx, ex, cw, ew)
        vx = [[Fraction(float(o.e2m1_decode(np.array([cx[m, k]]))[0])) *
               Fraction(2) ** (int(ex[m, k // 32]) - 127) for k in range(K)] for m in range(M)]
        vw = [[Fraction(float(o.e2m1_decode(np.array([cw[n, k]]))[0])) *
               Fraction(2) ** (int(ew[n, k // 32]) - 127) for k in range(K)] for n in range(N)]
        for m in range(M):
            for n in range(N):
                exact = sum(a * b for a, b in zip(vx[m], vw[n]))
                assert Fraction(float(r["sum"][m, n])) == exact
                assert Fraction(float(r["abs_sum"][m, n])) == sum(abs(a * b) for a, b in zip(vx[m], vw[n]))
    # block scales spanning ~100 binades: float64 rounding, far below any kernel tolerance
    cx = rng.integers(0, 16, size=(1, 64)).astype(np.uint8)
    ex = np.array([[80, 180]], dtype=np.uint8)
    r = o.mxfp4_linear_from_codes(cx, ex, cx, ex)
    vx = [Fraction(float(o.e2m1_decode(np.array([cx[0, k]]))[0])) *
          Fraction(2) ** (int(ex[0, k // 32]) - 127) for k in range(64)]
    exact = sum(a * a for a in vx)
    assert abs(Fraction(float(r["sum"][0, 0])) - exact) <= Fraction(2) ** -50 * exact


def pin_mxfp4_end_to_end_closed_form(o):
    """Constant rows c = 6 * 2^i and d = 4 * 2^j: the regular rotation keeps them constant,
    every code is 6 resp. 4 with block scale 2^i resp. 2^j, and out = bf16(K' c d + b)."""
    import torch
    for g, K, i, j in ((64, 128, 0, -3), (256, 512, -2, 1), (1024, 1024, 3, -5)):
        c, d = 6.0 * 2.0 ** i, -4.0 * 2.0 ** j
        x = np.full((2, K), c)
        w = np.full((3, K), d)
        b = np.array([0.5, -1.0, 0.0], dtype=np.float32)
        r = o.convlinear_fp4(x, w, b, g)
        assert np.all(o.e2m1_decode(r["x"]["codes"]) == 6.0)
        assert np.all(o.e2m1_decode(r["w"]["codes"]) == -4.0)
        assert np.all(r["x"]["scales"] == 127 + i) and np.all(r["w"]["scales"] == 127 + j)
        assert np.all(r["sum"] == K * c * d)
        want = torch.tensor(np.float32(K * c * d) + b, dtype=torch.float32).to(torch.bfloat16)
        assert np.array_equal(r["out_bits"], np.tile(want.view(torch.int16).numpy().view(np.uint16), (2, 1)))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
