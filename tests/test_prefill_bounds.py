"""Arithmetic behind the slope-bias prefill's early stop with key norms.

The kernel stops a tile's key walk once fold * B + bias(nearest remaining key)
lies the zero cut below the running max, where B bounds |q . k| over the
remaining keys by Cauchy-Schwarz on the e4m3 codes: B = |q|_32 * 1.001 *
max_block |k|_32 * 1.0001, the norms being fp32 square roots of fp32 sums of
the codes' squares. These tests check, with numpy's fp32 arithmetic standing in
for the kernel's, that the margins cover every rounding: each square of an
e4m3 value is exact in fp32, a 128-term fp32 sum of them stays within the
margin of the exact sum in any order, and the fp32 dot product of two code
vectors (what the MFMA accumulates, in any order) never exceeds B.
"""
import numpy as np

from oracle.codecs import e4m3_decode, e4m3_encode

CODES = np.arange(256, dtype=np.uint8)
VALUES = e4m3_decode(CODES).astype(np.float64)
FINITE = VALUES[np.isfinite(VALUES)]


def _fp32_sum_sequential(x):
    acc = np.float32(0.0)
    for v in x.astype(np.float32):
        acc = np.float32(acc + v)
    return acc


def _fp32_sum_pairwise(x):
    x = x.astype(np.float32)
    while x.size > 1:
        if x.size % 2:
            x = np.append(x, np.float32(0.0))
        x = (x[0::2] + x[1::2]).astype(np.float32)
    return x[0]


def test_e4m3_squares_are_exact_in_fp32():
    sq32 = (FINITE.astype(np.float32) * FINITE.astype(np.float32)).astype(np.float64)
    assert np.array_equal(sq32, FINITE * FINITE)


def _norm32(x, order):
    sq = (x.astype(np.float32) * x.astype(np.float32)).astype(np.float32)
    s = _fp32_sum_sequential(sq) if order == "seq" else _fp32_sum_pairwise(sq)
    return np.float32(np.sqrt(s))


def test_key_norm_margin_covers_fp32_summation():
    rng = np.random.default_rng(11)
    cases = [rng.choice(FINITE, 128) for _ in range(300)]
    # adversarial: one huge value first, then many tiny ones that fp32 drops
    cases.append(np.concatenate([[448.0], np.full(127, 2.0 ** -9)]))
    cases.append(np.concatenate([np.full(127, 2.0 ** -9), [448.0]]))
    cases.append(np.full(128, 448.0))
    for x in cases:
        exact = np.sqrt((x * x).sum())
        for order in ("seq", "pairwise"):
            k32 = np.float32(_norm32(x, order) * np.float32(1.0001))
            assert float(k32) >= exact, (order, float(k32), exact)
            assert float(k32) <= exact * (1 + 2e-4) + 1e-30


def test_cauchy_schwarz_bound_covers_the_fp32_dot_product():
    """|fp32 dot(q, k)| <= |q|_32 * 1.001 * |k|_32 * 1.0001 for code vectors,
    including aligned ones where Cauchy-Schwarz is tight."""
    rng = np.random.default_rng(12)
    for t in range(400):
        q = rng.choice(FINITE, 128)
        k = q.copy() if t % 4 == 0 else rng.choice(FINITE, 128)   # tight case: k = q
        if t % 8 == 1:
            k = -q
        prod = (q.astype(np.float32) * k.astype(np.float32)).astype(np.float32)   # exact products
        dots = [abs(float(_fp32_sum_sequential(prod))), abs(float(_fp32_sum_pairwise(prod))),
                abs(float(_fp32_sum_sequential(prod[::-1])))]
        qn = np.float32(_norm32(q, "seq") * np.float32(1.001))
        kn = np.float32(_norm32(k, "pairwise") * np.float32(1.0001))
        bound = float(np.float32(qn * kn))
        assert max(dots) <= bound, (t, max(dots), bound)


def test_looser_l1_bound_is_never_tighter_on_gaussian_codes():
    """The 448 * sum|q| bound (kept when no workspace is passed) is at least
    the Cauchy-Schwarz one whenever every key code is at most 448; on N(0,1)
    keys calibrated to amax/448 it is several times larger."""
    rng = np.random.default_rng(13)
    q = rng.standard_normal((64, 128))
    k = rng.standard_normal((4096, 128))
    qs, ks = np.abs(q).max() / 448, np.abs(k).max() / 448
    qc = e4m3_decode(e4m3_encode((q / qs).astype(np.float32))).astype(np.float64)
    kc = e4m3_decode(e4m3_encode((k / ks).astype(np.float32))).astype(np.float64)
    l1 = 448.0 * np.abs(qc).sum(-1)
    cs = np.sqrt((qc ** 2).sum(-1)) * np.sqrt((kc ** 2).sum(-1)).max()
    assert np.all(l1 >= cs)
    assert np.median(l1 / cs) > 3.0
    assert np.all(np.abs(qc @ kc.T).max(-1) <= cs * (1 + 1e-9))
