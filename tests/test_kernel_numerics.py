"""The number formats and formulas the HIP kernels rely on, checked on the
CPU with numpy emulations of the same bit operations (no GPU, no library).

* The three-part bf16 split (truncate to the upper 16 bits, subtract, twice
  more): the parts sum exactly to the fp32 value, each is a bf16 value, and
  the product of two such parts is exact in fp32. This is what makes the
  bf16 MFMA products of generation and of the window Grams exact.
* The branch-free tanh of the soft cap (odd Taylor polynomial below 0.3,
  (1 - e) / (1 + e) with e = exp(-2u) above) and the sigmoid as
  1 / (1 + 2^(-z log2 e)), evaluated step by step in fp32: within a few ulp
  of the exact functions (the GPU's exp2 and reciprocal add about one ulp
  each).
"""
import numpy as np

f32 = np.float32
MASK = np.uint32(0xFFFF0000)


def trunc_bf16(x):
    return (x.view(np.uint32) & MASK).view(np.float32)


def split3(x):
    h = trunc_bf16(x)
    r = (x - h).astype(np.float32)
    m = trunc_bf16(r)
    r2 = (r - m).astype(np.float32)
    lo = trunc_bf16(r2)
    return h, m, lo, (r2 - lo).astype(np.float32)


def test_three_part_bf16_split_is_exact():
    rng = np.random.default_rng(0)
    n = 2_000_000
    mant = rng.uniform(1.0, 2.0, n)
    expo = rng.integers(-100, 100, n)
    sign = rng.choice([-1.0, 1.0], n)
    x = (sign * np.ldexp(mant, expo)).astype(np.float32)
    h, m, lo, rest = split3(x)
    assert not rest.any()                                   # nothing is left over
    assert np.array_equal(h.astype(np.float64) + m.astype(np.float64) + lo.astype(np.float64),
                          x.astype(np.float64))
    for part in (h, m, lo):
        assert not (part.view(np.uint32) & np.uint32(0xFFFF)).any()   # bf16 values


def test_bf16_part_products_are_exact_in_fp32():
    rng = np.random.default_rng(1)
    a = trunc_bf16(rng.standard_normal(200_000).astype(np.float32))
    b = trunc_bf16((rng.standard_normal(200_000) * 1e-3).astype(np.float32))
    exact = a.astype(np.float64) * b.astype(np.float64)
    assert np.array_equal((a * b).astype(np.float64), exact)


def test_nine_part_products_give_the_dot_product():
    """k^ . k^ from the nine part products, summed in fp64 here, is the exact
    dot product of the fp32 vectors (the kernel sums them in fp32)."""
    rng = np.random.default_rng(2)
    a = rng.standard_normal((1000, 32)).astype(np.float32)
    b = rng.standard_normal((1000, 32)).astype(np.float32)
    pa, pb = split3(a)[:3], split3(b)[:3]
    tot = sum((p.astype(np.float64) * q.astype(np.float64)).sum(axis=1) for p in pa for q in pb)
    exact = (a.astype(np.float64) * b.astype(np.float64)).sum(axis=1)
    assert np.allclose(tot, exact, rtol=0, atol=1e-12 * np.abs(exact).max())


def tanh_pos_f32(u):
    u = u.astype(np.float32)
    u2 = u * u
    p = f32(21844.0 / 6081075.0)
    for c in (-1382.0 / 155925.0, 62.0 / 2835.0, -17.0 / 315.0, 2.0 / 15.0, -1.0 / 3.0):
        p = (p * u2 + f32(c)).astype(np.float32)
    ts = (u * u2 * p + u).astype(np.float32)
    e = np.exp2((u * f32(-2.8853900817779268)).astype(np.float32)).astype(np.float32)
    tl = ((f32(1) - e) * (f32(1) / (f32(1) + e))).astype(np.float32)
    return np.where(u < f32(0.3), ts, tl)


def test_branch_free_tanh_within_a_few_ulp():
    u = np.concatenate([np.geomspace(1e-3, 30.0, 200_000), [0.29999, 0.3, 0.30001]]).astype(np.float32)
    got = tanh_pos_f32(u).astype(np.float64)
    ref = np.tanh(u.astype(np.float64))
    ulps = np.abs(got - ref) / (ref * 2.0 ** -24)
    assert ulps.max() <= 6.0, ulps.max()


def test_sigmoid_as_exp2_and_reciprocal_within_a_few_ulp():
    """Within 4 ulp, plus up to 2 |z| ulp from the fp32 argument y = z log2(e)
    (log2(e) rounded to fp32, and the product rounded: each moves 2^y by up to
    |y| 2^-24 ln 2 = |z| 2^-24 relative): at most 4e-6 relative on [-30, 30],
    where sigmoid(-30) is 1e-13; within 3 ulp for z >= 0."""
    z = np.linspace(-30.0, 30.0, 200_001).astype(np.float32)
    e = np.exp2((z * f32(-1.4426950408889634)).astype(np.float32)).astype(np.float32)
    got = (f32(1) / (f32(1) + e)).astype(np.float64)
    ref = 1.0 / (1.0 + np.exp(-z.astype(np.float64)))
    ulps = np.abs(got - ref) / (ref * 2.0 ** -24)
    assert (ulps <= 4.0 + 2.0 * np.abs(z)).all(), (ulps - 2.0 * np.abs(z)).max()
    assert (ulps[z >= 0] <= 3.0).all()
