"""The error bound of the router screen, against a worst case of its arithmetic.

For T > 8 the routing first screens every logit with bf16 MFMAs: each fp32
router weight w is split into hi = bf16(w) and lo = bf16(w - hi), the products
x*hi and x*lo (bf16 x bf16, exact in fp32) are accumulated in fp32 over four
slices of the input width, the slices are summed in float64 and rounded to
fp32.  The exact top-k then recomputes in float64 every expert whose screened
logit lies within 2B of the k-th largest screened one, with

    B = (c1 * |x| * max_e |w_e| + 2^-22 * (max_e |screened_e| + 1)) * (1 + 2^-10)
    c1 = 2^-17 + (n + 32) * 2^-24 + 2^-23,   n = 128 * ceil((H / 64) / 4)

(|.| the Euclidean norm; n the products of one slice, hi and lo).  The bound
assumes the fp32 accumulation rounds at most once per product to nearest
(unit roundoff 2^-24); an MFMA that sums products internally in wider
precision rounds less.  Here the arithmetic is emulated on the CPU with one
fp32 round-to-nearest addition per product, in the order that makes the
rounding errors add up: a large term first, then terms just over half an ulp
of the running sum, each of which rounds up by almost half an ulp.  The bound
must hold and must not be loose by more than the hi/lo split's factor of two
(only the hi products can be made to round maximally).  CPU only.
"""
import numpy as np
import pytest

SPLIT = 4  # slices of the input width


def bf16_rn(a):
    """float32 -> nearest bfloat16 value (ties to even), as float32."""
    u = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def screen_bound(x, W, screened):
    """The bound B of the exact top-k step for one token (float64)."""
    H = x.size
    G = H // 64
    n = 128.0 * ((G + SPLIT - 1) // SPLIT)
    c1 = 2.0 ** -17 + (n + 32.0) * 2.0 ** -24 + 2.0 ** -23
    xn = np.sqrt(np.sum(x.astype(np.float64) ** 2)) * (1 + 1e-6)
    wn = np.sqrt(np.max(np.sum(W.astype(np.float64) ** 2, axis=1))) * (1 + 1e-6)
    amx = float(np.max(np.abs(screened)))
    return (c1 * xn * wn + 2.0 ** -22 * (amx + 1.0)) * (1 + 2.0 ** -10)


def screen_emulated(x, w, order=None):
    """One screened logit: hi/lo split, fp32 sums of the products of each
    slice (one rounding per addition, in `order` within each slice), slices
    summed in float64, rounded to fp32."""
    H = x.size
    hi = bf16_rn(w)
    lo = bf16_rn(w - hi)
    per = H // SPLIT
    total = 0.0
    for s in range(SPLIT):
        idx = np.arange(s * per, (s + 1) * per)
        if order is not None:
            idx = idx[order[s]]
        terms = np.concatenate([x[idx] * hi[idx], x[idx] * lo[idx]]).astype(np.float32)
        acc = np.float32(0.0)
        for t in terms:  # one fp32 round-to-nearest addition per product
            acc = np.float32(acc + t)
        total += float(acc)
    return np.float32(total)


def adversarial_row(H):
    """x, w whose products are 1.0 at the start of each slice, then terms of
    2^-24 * (1 + 2^-7): just over half an ulp of a running sum near 1, so each
    addition rounds up by nearly half an ulp and the errors add up."""
    x = np.full(H, 2.0 ** -12, np.float32)
    w = np.full(H, 2.0 ** -12 * (1 + 2.0 ** -7), np.float32)
    per = H // SPLIT
    for s in range(SPLIT):
        x[s * per] = 1.0
        w[s * per] = 1.0
    return x, w


@pytest.mark.parametrize("H", [2048, 8192])
def test_bound_covers_the_worst_accumulation(H):
    x, w = adversarial_row(H)
    assert np.array_equal(bf16_rn(x), x) and np.array_equal(bf16_rn(w), w)  # exact bf16 inputs, lo = 0
    exact = float(np.dot(x.astype(np.float64), w.astype(np.float64)))
    got = float(screen_emulated(x, w))
    err = abs(got - exact)
    B = screen_bound(x, w[None, :], np.array([got]))
    # Each slice: a term of 1.0, then H/4 - 1 terms that each round up by about 2^-24.
    assert err > 0.9 * SPLIT * (H // SPLIT - 1) * 2.0 ** -24 * (1 - 2.0 ** -7)
    assert err <= B, (err, B)
    # Only the hi products (half of the n roundings counted) can round this way.
    assert err >= 0.4 * B, (err, B)


def test_bound_for_the_smaller_constant_fails():
    """The same worst case against the bound with n computed for H = 2048 on
    an H = 8192 row (the slice count of products a quarter of the truth) is
    violated, so the test above would catch that mistake."""
    H = 8192
    x, w = adversarial_row(H)
    exact = float(np.dot(x.astype(np.float64), w.astype(np.float64)))
    err = abs(float(screen_emulated(x, w)) - exact)
    n_small = 128.0 * ((2048 // 64 + SPLIT - 1) // SPLIT)
    c1 = 2.0 ** -17 + (n_small + 32.0) * 2.0 ** -24 + 2.0 ** -23
    xn, wn = np.linalg.norm(x.astype(np.float64)), np.linalg.norm(w.astype(np.float64))
    assert err > c1 * xn * wn


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bound_with_cancellation_and_shuffled_orders(seed):
    """Heavy cancellation (alternating signs, magnitudes over 2^16) in random,
    ascending and descending orders: the bound holds in every case."""
    rng = np.random.default_rng(seed)
    H = 2048
    x = bf16_rn((rng.choice([-1.0, 1.0], H) * 2.0 ** rng.uniform(-8, 8, H)).astype(np.float32))
    w = (rng.standard_normal(H) * 2.0 ** rng.uniform(-6, 2, H)).astype(np.float32)
    exact = float(np.dot(x.astype(np.float64), w.astype(np.float64)))
    per = H // SPLIT
    mags = np.abs(x * w)
    orders = {
        "natural": None,
        "random": [rng.permutation(per) for _ in range(SPLIT)],
        "ascending": [np.argsort(mags[s * per:(s + 1) * per]) for s in range(SPLIT)],
        "descending": [np.argsort(-mags[s * per:(s + 1) * per]) for s in range(SPLIT)],
    }
    for name, order in orders.items():
        got = float(screen_emulated(x, w, order))
        B = screen_bound(x, w[None, :], np.array([got]))
        assert abs(got - exact) <= B, (name, abs(got - exact), B)
