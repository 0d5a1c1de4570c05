"""The Top-P rule the GPU selection kernels implement, modelled in numpy and
checked against the oracle's sorted-prefix Top-P (Prism review, pipeline
step (6)): with fixed-point masses m_j = floor(e_j 2^31), e_j = 2^(x_j - max)
and the target ceil(p Z), the kept set is the shortest prefix of the order
(e descending, block ascending) whose mass reaches the target.

The model below finds that prefix by bisection on the key (the bit pattern of
e): T = the largest key with mass(key >= T) >= target, every key above T is
kept, and the first ceil((target - mass(key > T)) / m(T)) entries with key T
in block order. It is the description of the long-row kernel, written here
in numpy so the equivalence can be checked on the CPU (it shares nothing
with either the kernels or the oracle).
"""
import numpy as np
import pytest

import oracle.prism_oracle as po


def bisect_select(x_log2: np.ndarray, p: float) -> np.ndarray:
    x = x_log2.astype(np.float32)
    e = np.exp2(x - x.max()).astype(np.float32)
    key = e.view(np.uint32)
    m = (e * np.float32(2.0 ** 31)).astype(np.uint64)

    def S(t, strict=False):
        return int(m[key > t].sum()) if strict else int(m[key >= t].sum())

    Z = S(1)
    target = int(np.ceil(Z * float(np.float32(p))))
    lo, hi = 1, 0x3F800001
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if S(mid) >= target:
            lo = mid
        else:
            hi = mid
    T = lo
    mT = int(np.float32(np.uint32(T).view(np.float32)) * np.float32(2.0 ** 31))
    take = -(-(target - S(T, True)) // mT)
    sel = key > T
    sel[np.nonzero(key == T)[0][:take]] = True
    return sel


def sorted_prefix_fixed_point(x_log2: np.ndarray, p: float) -> np.ndarray:
    """The same rule by an explicit stable sort (reference for the model)."""
    x = x_log2.astype(np.float32)
    e = np.exp2(x - x.max()).astype(np.float32)
    m = (e * np.float32(2.0 ** 31)).astype(np.uint64)
    target = int(np.ceil(int(m.sum()) * float(np.float32(p))))
    order = np.lexsort((np.arange(len(e)), -e.astype(np.float64)))
    csum = np.cumsum(m[order].astype(np.int64))
    n = int(np.searchsorted(csum, target)) + 1
    sel = np.zeros(len(e), bool)
    sel[order[:n]] = True
    return sel


@pytest.mark.parametrize("n,p,seed", [(3, 0.95, 0), (100, 0.95, 1), (1000, 0.93, 2), (4100, 0.95, 3),
                                      (8192, 0.5, 4), (257, 0.999, 5)])
def test_bisection_equals_sorted_prefix(n, p, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(n) * 3).astype(np.float32)
    assert np.array_equal(bisect_select(x, p), sorted_prefix_fixed_point(x, p))


def test_bisection_ties_taken_in_block_order():
    # 40 equal logits below a dominant one: the needed count is taken from the left
    x = np.array([5.0] + [0.0] * 40, np.float32)
    sel = bisect_select(x, 0.99)
    ref = sorted_prefix_fixed_point(x, 0.99)
    assert np.array_equal(sel, ref)
    tied = np.nonzero(sel[1:])[0]
    assert len(tied) and np.array_equal(tied, np.arange(len(tied)))


@pytest.mark.parametrize("seed", range(6))
def test_bisection_matches_oracle_top_p_off_ties(seed):
    """Against the oracle's float64 Top-P on the same probabilities: equal
    except where the oracle's cumulative mass sits within 1e-4 of p (the mask
    parity rule's mass ties)."""
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(50, 3000))
    x = (rng.standard_normal(n) * 2).astype(np.float32)
    s = np.exp2(x.astype(np.float64) - x.max())
    s /= s.sum()
    p = 0.95
    ref = np.zeros(n, bool)
    ref[po.top_p(s, p)] = True
    got = bisect_select(x, p)
    diff = np.nonzero(got != ref)[0]
    if diff.size:
        order = np.lexsort((np.arange(n), -s))
        cum = np.cumsum(s[order])
        pos = {int(j): r for r, j in enumerate(order)}
        for j in diff:
            r = pos[int(j)]
            before = cum[r - 1] if r else 0.0
            assert abs(before - p) < 1e-4 or abs(cum[r] - p) < 1e-4, (j, before, cum[r])
