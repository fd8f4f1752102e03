"""Pins of the oracle's MoE combine (out[t] = sum over k of w[t,k] * dm[t*K+k],
one fp32 fmaf per term, k ascending).

The pins do not reuse the oracle's loop:
  * a hand-worked example;
  * identities (K = 1 with weight 1, zero weights, a one-hot weight row);
  * exact single rounding: with |w|, |dm| in [0.5, 1) and K <= 4 every partial
    sum acc + w*d is exact in binary64 (at most 50 significant bits), so the
    fmaf chain equals rounding the binary64 step to binary32 once per term;
    the two-rounding form (product rounded, then the sum) and the reversed
    k order both differ from it on these inputs, so each would fail;
  * at K = 10 on normal inputs, the error against the exact sum stays within
    K units of the last place of the sum of |w * d|.
"""
import numpy as np

from oracle import oracle


def test_hand_worked():
    dm = np.arange(12, dtype=np.float32).reshape(4, 3)
    w = np.array([[1.0, 2.0], [0.5, 0.25]], np.float32)
    out = oracle.combine(dm, w)
    # token 0: [0,1,2] + 2*[3,4,5]; token 1: 0.5*[6,7,8] + 0.25*[9,10,11]
    assert out.tolist() == [[6.0, 9.0, 12.0], [5.25, 6.0, 6.75]]


def test_identities():
    rng = np.random.default_rng(1)
    dm = rng.standard_normal((5, 64)).astype(np.float32)
    assert np.array_equal(oracle.combine(dm, np.ones((5, 1), np.float32)), dm)
    dm3 = rng.standard_normal((15, 64)).astype(np.float32)
    assert np.all(oracle.combine(dm3, np.zeros((5, 3), np.float32)) == 0.0)
    onehot = np.zeros((5, 3), np.float32)
    onehot[np.arange(5), [2, 0, 1, 2, 0]] = 1.0
    out = oracle.combine(dm3, onehot)
    sel = dm3.reshape(5, 3, 64)[np.arange(5), [2, 0, 1, 2, 0]]
    assert np.array_equal(out, sel)


def _mag_half_one(rng, shape):
    m = rng.uniform(0.5, 1.0, shape)
    s = rng.choice([-1.0, 1.0], shape)
    return (m * s).astype(np.float32)


def _emulate(dm, w, order, two_roundings=False):
    T, K = w.shape
    d = dm.reshape(T, K, -1).astype(np.float64)
    acc = np.zeros((T, d.shape[2]), np.float32)
    for k in order:
        prod = w[:, k:k + 1].astype(np.float64) * d[:, k]
        if two_roundings:
            prod = prod.astype(np.float32).astype(np.float64)
        acc = (acc.astype(np.float64) + prod).astype(np.float32)
    return acc


def test_exact_single_rounding_in_k_order():
    rng = np.random.default_rng(7)
    T, K, H = 64, 4, 256
    w = _mag_half_one(rng, (T, K))
    dm = _mag_half_one(rng, (T * K, H))
    out = oracle.combine(dm, w)
    ref = _emulate(dm, w, range(K))
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))
    # the test tells the readings apart
    assert not np.array_equal(ref, _emulate(dm, w, range(K), two_roundings=True))
    assert not np.array_equal(ref, _emulate(dm, w, reversed(range(K))))


def test_error_bound_top10():
    rng = np.random.default_rng(11)
    T, K, H = 40, 10, 512
    w = rng.dirichlet(np.ones(K), T).astype(np.float32)
    dm = (rng.standard_normal((T * K, H)) * 3).astype(np.float32)
    out = oracle.combine(dm, w).astype(np.float64)
    prods = w.astype(np.float64)[:, :, None] * dm.reshape(T, K, H).astype(np.float64)
    exact = prods.sum(axis=1)
    bound = K * 2.0 ** -24 * np.abs(prods).sum(axis=1) + 1e-45
    assert np.all(np.abs(out - exact) <= bound)
