"""Pins of the Spectral-ATOMO oracle (oracle/atomo.py) to facts other than itself.

The review page "ATOMO: Communication-efficient Learning via Atomic Sparsification"
("Proposed method", "Main findings") defines the estimator, the budget and the
variance-minimising probabilities, and names two special cases (TernGrad and 1-bit
QSGD).  Each pin below checks one of those facts, or a closed form or invariant of the
singular value decomposition, by a route that does not reuse the oracle's own
arithmetic; test_oracle_atomo_mutations.py plants mistakes in the oracle and checks
that some pin fails for every one.
"""

import itertools
import os

import numpy as np
import pytest
from scipy.optimize import minimize

from oracle import atomo as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "atomo_worked_example.txt")


def _golden():
    out = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            rows = [np.array([float(v) for v in r.split()]) for r in val.split(";")]
            out[key] = np.stack(rows) if len(rows) > 1 else rows[0]
    return out


def _element_estimate(O, g, s, x):
    """The estimator with element-wise atoms a_i = e_i, lambda_i = g_i."""
    g = np.asarray(g, np.float64)
    p = O.probabilities(g, s)
    t = O.sample(p, x)
    return p, O.sparsify(g, list(np.eye(g.size)), p, t)


# ------------------------------------------------------------------ pins
def pin_worked_example(O):
    G = _golden()
    for tag in ("A", "B", "C"):
        sig, _, _ = O.svd_atoms(G[f"{tag}.g"])
        if f"{tag}.sigma" in G:
            assert np.allclose(sig, G[f"{tag}.sigma"], atol=1e-12)
        p = O.probabilities(sig, G[f"{tag}.s"].item())
        assert np.allclose(p, G[f"{tag}.p"], atol=1e-12)
    for tag, xs, gs in (("A", "A.x1", "A.ghat1"), ("A", "A.x2", "A.ghat2"), ("B", "B.x", "B.ghat"),
                        ("C", "C.x", "C.ghat")):
        r = O.compress_matrix(G[f"{tag}.g"], G[f"{tag}.s"].item(), G[xs])
        assert np.allclose(r.estimate, G[gs], atol=1e-12)
        assert np.allclose(r.a.T @ r.b, G[gs], atol=1e-12)
    for tag in ("A", "B"):
        sig, _, _ = O.svd_atoms(G[f"{tag}.g"])
        v = O.expected_square_norm(sig, O.probabilities(sig, G[f"{tag}.s"].item()))
        assert abs(v - G[f"{tag}.variance"].item()) < 1e-12
    p, gh = _element_estimate(O, G["D.g"], G["D.terngrad_s"].item(), G["D.x"])
    assert np.allclose(p, G["D.terngrad_p"], atol=1e-12)
    assert np.allclose(gh, G["D.terngrad_ghat"], atol=1e-12)


def pin_numerical_optimum(O):
    """The closed form is the minimiser of sum lam^2/p on the budget simplex: compare with
    a general-purpose constrained optimiser started away from it."""
    rng = np.random.default_rng(11)
    for trial in range(25):
        k = int(rng.integers(2, 7))
        lam = rng.choice([-1.0, 1.0], k) * rng.uniform(0.05, 1.0, k)
        s = float(rng.uniform(0.3, k - 0.2))
        p = O.probabilities(lam, s)
        obj = lambda q: float(np.sum(lam ** 2 / q))
        res = minimize(obj, np.full(k, s / k), method="SLSQP", bounds=[(1e-9, 1.0)] * k,
                       constraints=[{"type": "eq", "fun": lambda q: np.sum(q) - s}],
                       options={"ftol": 1e-14, "maxiter": 500})
        assert res.success
        assert obj(p) <= res.fun * (1 + 1e-7), (trial, obj(p), res.fun)
        assert np.allclose(p, res.x, atol=2e-4), (trial, p, res.x)


def pin_optimality_conditions(O):
    """KKT conditions of the budgeted problem: every atom below 1 has the same
    |lam_i| / p_i; saturated atoms have |lam_i| at least as large as that ratio times 1;
    the budget is spent (or every nonzero atom is certain); zero atoms get p = 0."""
    rng = np.random.default_rng(12)
    for _ in range(200):
        k = int(rng.integers(1, 12))
        lam = rng.standard_normal(k) * np.exp(2 * rng.standard_normal(k))
        lam[rng.random(k) < 0.15] = 0.0
        s = float(rng.uniform(0.05, k + 2))
        p = O.probabilities(lam, s)
        a = np.abs(lam)
        nnz = np.count_nonzero(a)
        assert np.all(p >= 0) and np.all(p <= 1 + 1e-12)
        assert np.all(p[a == 0] == 0)
        assert abs(p.sum() - min(s, nnz)) < 1e-9 * max(1, s)
        free = (a > 0) & (p < 1 - 1e-12)
        if free.any():
            ratio = a[free] / p[free]
            assert np.ptp(ratio) <= 1e-9 * ratio.max()
            sat = (a > 0) & ~free
            assert np.all(a[sat] >= ratio.max() * (1 - 1e-9))


def pin_enumeration(O):
    """Exact expectations over all 2^k outcomes of t: E[g_hat] = g and E||g_hat||^2 =
    sum sigma^2 / p, for spectral atoms of small random matrices."""
    rng = np.random.default_rng(13)
    for n, m, s in ((3, 5, 1.0), (4, 4, 2.5), (5, 3, 0.7), (2, 6, 1.7)):
        g = rng.standard_normal((n, m))
        sig, left, right = O.svd_atoms(g)
        p = O.probabilities(sig, s)
        atoms = [np.outer(left[:, i], right[i]) for i in range(sig.size)]
        mean = np.zeros((n, m))
        sq = 0.0
        for t in itertools.product([False, True], repeat=sig.size):
            t = np.array(t)
            w = np.prod(np.where(t, p, 1 - p))
            if w == 0:
                continue
            gh = O.sparsify(sig, atoms, p, t)
            mean += w * gh
            sq += w * float(np.sum(gh ** 2))
        assert np.allclose(mean, g, atol=1e-12)
        assert abs(sq - O.expected_square_norm(sig, p)) < 1e-10 * sq


def pin_sampling_frequencies(O):
    """sample() draws t_i = 1 with probability p_i: with evenly spaced uniforms the
    fraction of draws that send atom i is p_i to within the grid step."""
    p = np.array([0.0, 0.13, 0.5, 0.999, 1.0])
    xs = (np.arange(10000) + 0.5) / 10000
    freq = np.mean([O.sample(p, np.full(p.size, x)) for x in xs], axis=0)
    assert np.allclose(freq, p, atol=1e-4)


def pin_special_cases(O):
    """The two special cases the page names, with element-wise atoms: TernGrad (budget
    ||g||_1/||g||_inf, sent values +-||g||_inf) and 1-bit QSGD (budget ||g||_1/||g||_2,
    sent values +-||g||_2)."""
    rng = np.random.default_rng(14)
    for _ in range(20):
        g = rng.standard_normal(int(rng.integers(2, 40)))
        x = rng.random(g.size)
        for norm in (np.max(np.abs(g)), np.linalg.norm(g)):
            s = float(np.sum(np.abs(g)) / norm)
            p, gh = _element_estimate(O, g, s, x)
            assert np.allclose(p, np.abs(g) / norm, atol=1e-12)
            sent = x < np.abs(g) / norm
            assert np.allclose(gh, np.where(sent, np.sign(g) * norm, 0.0), atol=1e-12)


def pin_decomposition(O):
    """Closed forms and invariants of the singular value decomposition."""
    rng = np.random.default_rng(15)
    a, b = rng.standard_normal(6), rng.standard_normal(4)
    sig, left, right = O.svd_atoms(np.outer(a, b))                    # rank one
    assert abs(sig[0] - np.linalg.norm(a) * np.linalg.norm(b)) < 1e-12 and np.all(sig[1:] < 1e-12)
    assert abs(abs(left[:, 0] @ a) - np.linalg.norm(a)) < 1e-12
    d = np.array([0.5, -3.0, 2.0, 0.0])
    sig, _, _ = O.svd_atoms(np.diag(d))                               # diagonal
    assert np.allclose(sig, [3.0, 2.0, 0.5, 0.0], atol=1e-14)
    q, _ = np.linalg.qr(rng.standard_normal((7, 7)))
    sig, _, _ = O.svd_atoms(q[:, :5])                                 # orthonormal columns
    assert np.allclose(sig, 1.0, atol=1e-13)
    for n, m in ((5, 9), (9, 5), (6, 6), (2, 17)):
        g = rng.standard_normal((n, m))
        sig, left, right = O.svd_atoms(g)
        k = min(n, m)
        assert sig.shape == (k,) and np.all(np.diff(sig) <= 0) and np.all(sig >= 0)
        assert np.allclose(left.T @ left, np.eye(k), atol=1e-13)
        assert np.allclose(right @ right.T, np.eye(k), atol=1e-13)
        assert np.allclose(sum(sig[i] * np.outer(left[:, i], right[i]) for i in range(k)), g, atol=1e-12)
        assert abs(np.sum(sig ** 2) - np.sum(g ** 2)) < 1e-12 * np.sum(g ** 2)


def pin_message(O):
    """The sent factors: estimate = a^T b; the unit factor is on the side of length
    min(n, m); a full budget reproduces g whatever the uniforms; an atom with p = 1 is
    sent by every uniform in [0, 1)."""
    rng = np.random.default_rng(16)
    for n, m in ((4, 9), (9, 4), (5, 5)):
        g = rng.standard_normal((n, m))
        k = min(n, m)
        r = O.compress_matrix(g, 1.3, rng.random(k))
        assert np.allclose(r.a.T @ r.b, r.estimate, atol=1e-12)
        unit = r.a if n <= m else r.b
        assert np.allclose(np.linalg.norm(unit, axis=1), 1.0, atol=1e-12)
        other = r.b if n <= m else r.a
        assert np.allclose(np.linalg.norm(other, axis=1), r.sigma[r.index] / r.prob[r.index], rtol=1e-12)
        assert np.all(np.diff(r.index) > 0)
        full = O.compress_matrix(g, float(k), np.nextafter(1.0, 0.0) * np.ones(k))
        assert full.index.size == k and np.allclose(full.estimate, g, atol=1e-12)


def pin_step(O):
    """A whole step: uncompressed tensors are averaged; the update is the workers' mean
    of their estimates; each worker uses its own row of uniforms."""
    rng = np.random.default_rng(17)
    W = 3
    grads = [rng.standard_normal((W, 4, 6)), rng.standard_normal((W, 1, 5)), rng.standard_normal((W, 8)),
             rng.standard_normal((W, 6, 3))]
    xs = [rng.random((W, 4)), None, None, rng.random((W, 3))]
    out = O.compress_layers(grads, 1.5, xs)
    assert np.allclose(out[1].update, grads[1].mean(axis=0)) and not out[1].workers
    assert np.allclose(out[2].update, grads[2].mean(axis=0)) and not out[2].workers
    for li in (0, 3):
        per = [O.compress_matrix(grads[li][w], 1.5, xs[li][w]) for w in range(W)]
        assert np.allclose(out[li].update, sum(r.a.T @ r.b for r in per) / W, atol=1e-12)
        for w in range(W):
            assert np.array_equal(out[li].workers[w].index, np.flatnonzero(xs[li][w] < per[w].prob))


PINS = [
    pin_worked_example,
    pin_numerical_optimum,
    pin_optimality_conditions,
    pin_enumeration,
    pin_sampling_frequencies,
    pin_special_cases,
    pin_decomposition,
    pin_message,
    pin_step,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_atomo_oracle_pin(pin):
    pin(O)


def test_budget_must_be_positive():
    with pytest.raises(ValueError):
        O.probabilities(np.ones(3), 0.0)
