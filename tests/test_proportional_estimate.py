"""The proportional split's shortcuts (CPU).  Each share is estimated in
double as R / f_r / sum_j (1 / f_j).  Where the estimate's fractional part
lies at least 1e-4 from a whole number, its floor is taken as the floor;
otherwise the floor is settled exactly.  The remainders are ordered by the
estimates less the floors, and compared exactly only where two estimates lie
within 1e-4 of each other.  Both shortcuts are sound if every estimate lies
within 1e-5 of the exact share R P_r / S.  Checked on pools below 2^31 over
up to 16 hosts whose loads are below 2^31 -- equal loads (exact ties), loads
that make the shares whole numbers, and random ones: the floors taken from
estimates equal the exact floors, and the resulting shares equal the exact
largest-remainder deal."""
from fractions import Fraction
import math
import random

BAND, BOUND = 1e-4, 1e-5


def _estimates(R, f):
    tot = 0.0
    for x in f:
        tot += 1.0 / float(x)
    return [float(R) / float(x) / tot for x in f]


def _exact(R, f):
    w = [Fraction(1, x) for x in f]
    t = sum(w)
    return [R * wi / t for wi in w]


def _deal(R, f):
    """Shares as the kernel deals them: floors from the estimates away from
    whole numbers (exact ones near them), then the remainders ordered by the
    estimates, exactly where two are within the band."""
    ex, est = _exact(R, f), _estimates(R, f)
    q = []
    for e, v in zip(est, ex):
        part = e - math.floor(e)
        q.append(math.floor(v) if part < BAND or part > 1.0 - BAND else min(max(math.floor(e), 0), R))
    assert q == [math.floor(v) for v in ex], (R, f)
    frac = [e - qi for e, qi in zip(est, q)]
    rem = [v - qi for v, qi in zip(ex, q)]
    left = R - sum(q)
    give = list(q)
    for r in range(len(f)):
        above = 0
        for j in range(len(f)):
            if j == r:
                continue
            d = frac[j] - frac[r]
            if d > BAND:
                above += 1
            elif d >= -BAND:
                above += 1 if (rem[j] > rem[r] or (rem[j] == rem[r] and j < r)) else 0
        if above < left:
            give[r] += 1
    return give, max(abs(e - float(v)) for e, v in zip(est, ex))


def _reference(R, f):
    ex = _exact(R, f)
    give = [math.floor(v) for v in ex]
    left = R - sum(give)
    for r in sorted(range(len(f)), key=lambda r: (-(ex[r] - give[r]), r))[:left]:
        give[r] += 1
    return give


def _pools():
    rng = random.Random(5)
    top = (1 << 31) - 1
    yield top, [1] * 16                                 # equal loads: every remainder ties
    yield top, [top] * 16
    yield 3 * 5 * 7 * 16, [3, 5, 7, 1, 2, 4, 8, 16]     # whole-number shares
    yield top, [1, top, 2, top - 1, 3, 1 << 30]
    for _ in range(400):
        m = rng.randint(2, 16)
        R = rng.choice([rng.randint(0, 64), rng.randint(0, 1 << 20), rng.randint(top - 1000, top)])
        f = [rng.choice([rng.randint(1, 16), rng.randint(1, 1 << 24), rng.randint(1 << 30, top)]) for _ in range(m)]
        if rng.random() < 0.3:
            f[rng.randrange(m)] = f[0]                  # a repeated load: a remainder tie
        yield R, f


def test_band_ordering_equals_exact_deal():
    worst = 0.0
    for R, f in _pools():
        give, err = _deal(R, f)
        worst = max(worst, err)
        assert err < BOUND, (R, f, err)
        assert give == _reference(R, f), (R, f)
        assert sum(give) == R
    assert worst > 0.0  # the estimates are not exact: the band is exercised
