"""Precision of the probability operand of PV, the reason decode splits P
into two e4m3 terms (and prefill uses fp16 P) instead of one e4m3 term.

vLLM PR 54705, evidence "Tier 0": the FA4 port scales P by 2^8 and casts it
to e4m3 (one term, lazy rescale under log2(448) - 8). On diffuse attention
(N(0,1) queries and keys, scores of order 1 over thousands of keys) one e4m3
term per weight misses the relative-L2 bound 5e-3 on the output, while two
e4m3 terms (hi = e4m3(2^8 p), lo = e4m3(2^8 p - hi)), bf16 P and fp16 P stay
within it. The emulation uses the oracle's e4m3 codec and bf16 rounding, and
numpy's float16 for fp16 P; each scheme normalises by the sum of its own
rounded weights, as the kernels do, and the outputs are rounded to bf16 like
the kernels' outputs.
"""
import numpy as np
import pytest

from oracle.codecs import e4m3_encode, e4m3_decode, bf16_round

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _e4m3(x):
    return e4m3_decode(e4m3_encode(np.asarray(x, dtype=np.float32)))


def _attend(w, v):
    return bf16_round((w @ v) / w.sum(axis=-1, keepdims=True))


def _case(seed, heads, keys, dim, peak=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((heads, dim))
    k = rng.standard_normal((keys, dim))
    v = rng.standard_normal((keys, dim))
    s = peak * (q @ k.T) / np.sqrt(dim)
    p = np.exp(s - s.max(axis=-1, keepdims=True))      # <= 1, exact in fp64
    exact = (p @ v) / p.sum(axis=-1, keepdims=True)
    return p, v, exact


def _rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("seed,keys,dim", [(0, 257, 64), (1, 8192, 128), (2, 512, 128)])
def test_single_e4m3_term_misses_and_two_terms_meet_the_bound(seed, keys, dim):
    p, v, exact = _case(seed, 8, keys, dim)
    y = np.float32(256.0) * p.astype(np.float32)       # P = 2^8 p, as on the page
    hi = _e4m3(y)
    lo = _e4m3(y - hi)
    one_term = _rel_l2(_attend(hi, v), exact)
    two_terms = _rel_l2(_attend(hi + lo, v), exact)
    bf16_p = _rel_l2(_attend(bf16_round(p), v), exact)
    f16_p = _rel_l2(_attend(p.astype(np.float16).astype(np.float64), v), exact)
    rounding_only = _rel_l2(bf16_round(exact), exact)
    assert one_term > 5e-3, one_term
    assert two_terms < 5e-3 and bf16_p < 5e-3 and f16_p < 5e-3, (two_terms, bf16_p, f16_p)
    # the kept schemes add little beyond the bf16 rounding of the output,
    # fp16 P (11 significant bits) least of all
    assert two_terms < 2.5 * rounding_only and bf16_p < 2.5 * rounding_only
    assert f16_p < 1.5 * rounding_only and f16_p < bf16_p


def test_two_terms_represent_p_to_eight_bits():
    """hi + lo holds 2^8 p to a relative error below 2^-8 over p >= 2^-6 (where
    the second term is still a normal e4m3 value); hi alone is off by more
    than 2^-5 somewhere in that range (3 mantissa bits)."""
    rng = np.random.default_rng(3)
    p = np.exp(-rng.uniform(0.0, 6.0 * np.log(2.0), 20000)).astype(np.float32)
    y = np.float32(256.0) * p
    hi = _e4m3(y)
    lo = _e4m3(y - hi)
    rel = np.abs(hi + lo - y) / y
    assert rel.max() < 2.0 ** -8
    assert (np.abs(hi - y) / y).max() > 2.0 ** -5


def test_zero_gaps_of_the_prefill_block_skip():
    """The prefill skips a block when every exponent argument x - m lies at
    least 26 below the running max (fp16 P = 2^(x - m)) or 19 below it (e4m3
    P = 2^(x - m + 8), one term or two): every such P rounds to exactly zero,
    also when exp2 returns a few ulp high. One unit less would not do: the
    next power of two, a few ulp high, rounds up to a nonzero value."""
    high = np.float32(1.0 + 4 * 2.0 ** -23)                    # 4 ulp above the exact power
    # fp16: 2^-26 and anything a little above it round to 0 (below half the
    # smallest subnormal 2^-24); 2^-25 a little high rounds up to 2^-24
    assert np.float16(np.float32(2.0 ** -26) * high) == 0
    assert np.float16(np.float32(2.0 ** -25)) == 0              # the tie goes to the even zero
    assert np.float16(np.float32(2.0 ** -25) * high) == np.float16(2.0 ** -24)
    # e4m3 (the oracle's codec): 2^(x - m + 8) with x - m = -19 is 2^-11
    y = np.float32(2.0 ** -11) * high
    hi = _e4m3(y)
    assert hi == 0 and _e4m3(y - hi) == 0                       # both terms
    y = np.float32(2.0 ** -10) * high
    assert _e4m3(y) == np.float32(2.0 ** -9)                    # one unit less: nonzero

