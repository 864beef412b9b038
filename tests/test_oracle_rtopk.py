"""Pins of the rTop-k oracle (oracle/rtopk_ef.py) against facts fixed outside it: a worked
example computed by hand, an independent threshold-based selection, the partition and
tie properties, exhaustive enumeration of the random subsets, the contraction property
of a compression operator, and exact error-feedback identities.  CPU only.

Each pin takes the oracle module as its argument so that test_oracle_rtopk_mutations.py
can run the same pins against planted mistakes."""

import itertools
import os

import numpy as np
import pytest

from oracle import rtopk_ef as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rtopk_worked_example.txt")


def _golden():
    out = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, val = (s.strip() for s in line.split("=", 1))
        out[key] = np.array([float(t) for t in val.split()])
    return out


def _key(m):
    """Magnitude order written independently of the oracle: |m| as float64, NaN last
    resolved separately by the pins that need it."""
    return np.abs(np.asarray(m, dtype=np.float64))


def _tied_input(rng, d):
    """Values from a small set (many exact ties, both signs, zeros) plus a few
    continuous values."""
    base = rng.choice([0.0, 0.5, 1.0, 2.0, 3.0], size=d).astype(np.float32)
    base *= rng.choice([-1.0, 1.0], size=d).astype(np.float32)
    cont = rng.random(d) < 0.3
    base[cont] = rng.standard_normal(int(cont.sum())).astype(np.float32)
    return base


def pin_worked_example(mod):
    g = _golden()
    W, k, r = int(g["workers"][0]), int(g["k"][0]), int(g["r"][0])
    G = np.stack([g["g0"], g["g1"]]).astype(np.float32)
    E = np.stack([g["e0"], g["e1"]]).astype(np.float32)
    ranks = np.stack([g["ranks0"], g["ranks1"]]).astype(np.int64)
    st = mod.compress_tensor(G, E, r, k, ranks)
    M = G + E
    for w in range(W):
        assert np.array_equal(mod.top_set(M[w], r), g[f"top{w}"].astype(np.int64))
        assert np.array_equal(st.index[w], g[f"index{w}"].astype(np.int64))
        assert np.array_equal(st.value[w], g[f"value{w}"].astype(np.float32))
        assert np.array_equal(st.errors[w], g[f"error{w}"].astype(np.float32))
    assert np.array_equal(st.update, g["update"])


def pin_threshold_selection(mod, seed=21):
    """Top set = everything strictly above the r-th largest magnitude T, plus the
    lowest-index entries equal to T; T found by np.partition (a selection, not a sort)."""
    rng = np.random.default_rng(seed)
    for d in (1, 7, 64, 257, 1000):
        m = _tied_input(rng, d)
        a = _key(m)
        for r in sorted({1, 2, max(1, d // 3), max(1, d - 1), d}):
            t = np.partition(a, d - r)[d - r]
            above = np.flatnonzero(a > t)
            ties = np.flatnonzero(a == t)[: r - above.size]
            want = np.sort(np.concatenate([above, ties]))
            assert np.array_equal(mod.top_set(m, r), want), (d, r)


def pin_partition_property(mod, seed=22):
    rng = np.random.default_rng(seed)
    for _ in range(30):
        d = int(rng.integers(1, 40))
        r = int(rng.integers(1, d + 1))
        m = _tied_input(rng, d)
        s = mod.top_set(m, r)
        a = _key(m)
        assert s.size == r and np.all(np.diff(s) > 0)
        inside = np.zeros(d, bool)
        inside[s] = True
        for i in np.flatnonzero(inside):
            for j in np.flatnonzero(~inside):
                assert a[i] > a[j] or (a[i] == a[j] and i < j), (i, j)


def pin_special_cases(mod, seed=23):
    rng = np.random.default_rng(seed)
    m = rng.standard_normal(50).astype(np.float32)
    # r = 1: the (first) position of the largest magnitude
    assert np.array_equal(mod.top_set(m, 1), [int(np.argmax(np.abs(m)))])
    # r = d: everything
    assert np.array_equal(mod.top_set(m, 50), np.arange(50))
    # k = r: the whole top set is sent whatever the permutation
    for _ in range(5):
        idx, val = mod.rtopk(m, 8, 8, rng.permutation(8))
        assert np.array_equal(idx, mod.top_set(m, 8))
        assert np.array_equal(val, m[idx])
    # r = d, k = 1: the single entry of rank 0
    perm = rng.permutation(50)
    idx, val = mod.rtopk(m, 50, 1, perm)
    assert idx.tolist() == [int(np.flatnonzero(perm == 0)[0])] and val[0] == m[idx[0]]


def pin_subset_enumeration(mod):
    """Over every permutation of a 4-entry top set, each 2-subset is sent equally often
    (a uniform random subset), and it is always a subset of the top set."""
    m = np.array([0.1, -5.0, 0.2, 3.0, 0.0, -4.0, 2.5], dtype=np.float32)
    top = mod.top_set(m, 4)
    assert top.tolist() == [1, 3, 5, 6]
    counts = {}
    for perm in itertools.permutations(range(4)):
        idx, val = mod.rtopk(m, 4, 2, np.array(perm))
        assert idx.size == 2 and set(idx.tolist()) <= set(top.tolist())
        assert np.all(np.diff(idx) > 0)
        counts[tuple(idx)] = counts.get(tuple(idx), 0) + 1
    assert len(counts) == 6 and set(counts.values()) == {4}


def pin_contraction(mod, seed=24):
    """Averaged over the random subset, ||M - C(M)||^2 = ||M||^2 - (k/r)||top_r(M)||^2,
    which is at most (1 - k/d)||M||^2: the compression-operator property under which
    error feedback converges."""
    rng = np.random.default_rng(seed)
    for d, r, k in ((7, 4, 2), (6, 3, 1), (8, 5, 3)):
        m = rng.standard_normal(d).astype(np.float32)
        mm = m.astype(np.float64)
        resid = []
        for perm in itertools.permutations(range(r)):
            idx, val = mod.rtopk(m, r, k, np.array(perm))
            e = mod.new_error(m, idx).astype(np.float64)
            resid.append(float(e @ e))
        top = np.sort(np.abs(mm))[::-1][:r]
        closed = float(mm @ mm) - (k / r) * float(top @ top)
        assert abs(np.mean(resid) - closed) <= 1e-9 * float(mm @ mm)
        assert np.mean(resid) <= (1 - k / d) * float(mm @ mm) + 1e-12


def pin_ef_identities(mod, seed=25, W=3, d=50, r=10, k=4):
    rng = np.random.default_rng(seed)
    G = rng.standard_normal((W, d)).astype(np.float32)
    E = (0.3 * rng.standard_normal((W, d))).astype(np.float32)
    ranks = np.stack([rng.permutation(r) for _ in range(W)])
    st = mod.compress_tensor(G, E, r, k, ranks)
    M = G + E
    total = np.zeros(d)
    for w in range(W):
        idx = st.index[w]
        assert idx.size == k and np.all(idx >= 0) and np.all(np.diff(idx) > 0)
        sent = np.zeros(d, np.float32)
        sent[idx] = st.value[w]
        assert np.array_equal(sent + st.errors[w], M[w])        # M = C(M) + E'
        assert np.all(st.errors[w][idx] == 0)
        assert np.array_equal(st.value[w], M[w][idx])
        total += sent
    assert np.allclose(st.update * W, total, rtol=0, atol=1e-12)


def pin_ef_telescoping(mod, seed=26, W=2, d=40, r=8, k=3, steps=6):
    """With integer gradients every float32 sum is exact, and what was sent plus what
    is still held equals everything that arrived."""
    rng = np.random.default_rng(seed)
    E = np.zeros((W, d), np.float32)
    sent_total = np.zeros((W, d))
    grad_total = np.zeros((W, d))
    for _ in range(steps):
        G = rng.integers(-8, 9, size=(W, d)).astype(np.float32)
        ranks = np.stack([rng.permutation(r) for _ in range(W)])
        st = mod.compress_tensor(G, E, r, k, ranks)
        for w in range(W):
            ok = st.index[w] >= 0
            np.add.at(sent_total[w], st.index[w][ok], st.value[w][ok])
        grad_total += G
        E = st.errors
    assert np.array_equal(sent_total + E, grad_total)


def pin_selection_in_float32(mod):
    """The selection is decided on M rounded to float32: 1 + 2^-25 rounds to 1 and ties
    with an exact 1, so the lower index wins."""
    G = np.array([[1.0, 1.0, 0.5]], np.float32)
    E = np.array([[0.0, 2.0 ** -25, 0.0]], np.float32)
    st = mod.compress_tensor(G, E, 1, 1, np.array([[0]]))
    assert st.index[0].tolist() == [0]


def pin_invalid_ranks(mod, seed=27):
    rng = np.random.default_rng(seed)
    m = rng.standard_normal(30).astype(np.float32)
    top = mod.top_set(m, 6)
    idx, val = mod.rtopk(m, 6, 3, np.zeros(6, np.int64))       # every rank below k
    assert np.array_equal(idx, top[:3]) and np.array_equal(val, m[top[:3]])
    idx, val = mod.rtopk(m, 6, 3, np.full(6, 9, np.int64))     # no rank below k
    assert idx.tolist() == [-1, -1, -1] and np.all(val == 0)
    assert np.array_equal(mod.new_error(m, idx), m)


def pin_nan_above_infinity(mod):
    """The magnitude key is the bit pattern of |m|: NaN (0x7fc00000) orders above
    infinity (0x7f800000), which orders above every finite value."""
    m = np.array([1.0, np.inf, -3.0, np.nan, -np.inf], np.float32)
    assert mod.top_set(m, 1).tolist() == [3]
    assert mod.top_set(m, 3).tolist() == [1, 3, 4]
    assert mod.top_set(m, 4).tolist() == [1, 2, 3, 4]


PINS = [
    pin_worked_example,
    pin_threshold_selection,
    pin_partition_property,
    pin_special_cases,
    pin_subset_enumeration,
    pin_contraction,
    pin_ef_identities,
    pin_ef_telescoping,
    pin_selection_in_float32,
    pin_invalid_ranks,
    pin_nan_above_infinity,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_rtopk_oracle_pin(pin):
    pin(O)


def test_compress_layers_is_per_tensor():
    rng = np.random.default_rng(28)
    shapes = [(2, 30), (2, 7)]
    G = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    E = [np.zeros(s, np.float32) for s in shapes]
    ranks = [np.stack([rng.permutation(6) for _ in range(2)]), np.stack([rng.permutation(2) for _ in range(2)])]
    out = O.compress_layers(G, E, [6, 2], [2, 1], ranks)
    for g, e, r, k, rk, st in zip(G, E, [6, 2], [2, 1], ranks, out):
        ref = O.compress_tensor(g, e, r, k, rk)
        assert np.array_equal(st.index, ref.index) and np.array_equal(st.errors, ref.errors)
