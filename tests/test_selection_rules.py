"""The Top-P rule the GPU selection kernels implement, modelled in numpy and
checked against the oracle's sorted-prefix Top-P (Prism review, pipeline
step (6)): with fixed-point masses m_j = floor(e_j 2^31), e_j = 2^(x_j - max)
and the target ceil(p Z), the kept set is the shortest prefix of the order
(e descending, block ascending) whose mass reaches the target.

The kernels find that prefix by a radix select on the key (the bit pattern
of e, monotone in e) instead of a sort, with the row held in registers (16
to 128 entries per lane, rows of up to 8192 blocks); the model below restates
its level structure in numpy so the equivalence with the sorted prefix can be
checked on the CPU (it shares nothing with the kernels or the oracle): 64
bins per level, level 0 in quarter octaves below e = 1 with a tail bin, then
the threshold bin split on the next 6 key bits (or the tail window moved
down), until the threshold bin holds one entry or one key value.
"""
import numpy as np
import pytest

import oracle.prism_oracle as po


def _keys(x_log2):
    x = x_log2.astype(np.float32)
    e = np.exp2(x - x.max()).astype(np.float32)
    key = e.view(np.uint32).astype(np.int64)
    m = (e * np.float32(2.0 ** 31)).astype(np.uint64).astype(np.int64)
    return key, m


def _take_ties(sel, key, m, T, target, above):
    """keep the first ceil((target - above) / m(T)) entries with key T"""
    mT = int(m[np.nonzero(key == T)[0][0]])
    take = -(-(target - above) // mT)
    sel[np.nonzero(key == T)[0][:take]] = True
    return sel


def radix_select_registers(x_log2: np.ndarray, p: float) -> np.ndarray:
    key, m = _keys(x_log2)
    target = int(np.ceil(int(m.sum()) * float(np.float32(p))))
    shift, base, tail = 21, 508, True
    und = key != 0
    above = 0
    while True:
        b = np.clip(base - (key >> shift), 0, 63)
        mass = np.bincount(b[und], weights=m[und], minlength=64).astype(np.int64)
        cnt = np.bincount(b[und], minlength=64)
        cum = np.cumsum(mass)
        bstar = int(np.argmax(cum >= target - above))
        above += int(cum[bstar] - mass[bstar])
        c = int(cnt[bstar])
        lo = 1 if (tail and bstar == 63) else (base - bstar) << shift
        hi = (base - bstar + 1) << shift
        if c <= 1:
            return key >= lo
        if tail and bstar == 63:
            base -= 63
        elif shift == 0:
            break
        else:
            bits = min(shift, 6)
            shift -= bits
            base = ((base - bstar) << bits) + (1 << bits) - 1
            tail = False
        und = (key >= lo) & (key < hi)
    return _take_ties(key >= hi, key, m, lo, target, above)


def sorted_prefix_fixed_point(x_log2: np.ndarray, p: float) -> np.ndarray:
    """The same rule by an explicit stable sort (reference for the models)."""
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


MODELS = [radix_select_registers]


@pytest.mark.parametrize("model", MODELS)
@pytest.mark.parametrize("n,p,seed,spread", [(3, 0.95, 0, 3), (100, 0.95, 1, 3), (1000, 0.93, 2, 3),
                                             (4100, 0.95, 3, 3), (8192, 0.5, 4, 3), (257, 0.999, 5, 3),
                                             (1024, 0.95, 6, 0.3), (600, 0.9999, 7, 12), (2048, 0.95, 8, 40)])
def test_radix_equals_sorted_prefix(model, n, p, seed, spread):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(n) * spread).astype(np.float32)
    assert np.array_equal(model(x, p), sorted_prefix_fixed_point(x, p))


@pytest.mark.parametrize("model", MODELS)
def test_radix_ties_taken_in_block_order(model):
    # 40 equal logits below a dominant one: the needed count is taken from the left
    x = np.array([5.0] + [0.0] * 40, np.float32)
    sel = model(x, 0.99)
    assert np.array_equal(sel, sorted_prefix_fixed_point(x, 0.99))
    tied = np.nonzero(sel[1:])[0]
    assert len(tied) and np.array_equal(tied, np.arange(len(tied)))


@pytest.mark.parametrize("model", MODELS)
def test_radix_threshold_in_the_tail(model):
    """p close to 1 over a spread of 60 octaves puts the threshold below
    2^-16 of the maximum (the tail window moves down)."""
    x = np.linspace(0.0, -60.0, 300).astype(np.float32)
    for p in (0.99999, 0.9999999):
        assert np.array_equal(model(x, p), sorted_prefix_fixed_point(x, p))


@pytest.mark.parametrize("model", MODELS)
@pytest.mark.parametrize("seed", range(6))
def test_radix_matches_oracle_top_p_off_ties(model, seed):
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
    got = model(x, p)
    diff = np.nonzero(got != ref)[0]
    if diff.size:
        order = np.lexsort((np.arange(n), -s))
        cum = np.cumsum(s[order])
        pos = {int(j): r for r, j in enumerate(order)}
        for j in diff:
            r = pos[int(j)]
            before = cum[r - 1] if r else 0.0
            assert abs(before - p) < 1e-4 or abs(cum[r] - p) < 1e-4, (j, before, cum[r])
