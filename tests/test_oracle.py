"""Pins for the CPU oracle (oracle/powersgd_ef.py), checked against facts that do not come
from the oracle itself: a thin QR from LAPACK, SVD bounds, closed forms and invariants
that the PowerSGD review page (section "Proposed method") and linear algebra fix.

The pins are written as ``pin_*`` functions over a module-like object so that
test_oracle_mutations.py can run the same checks on deliberately broken copies of the
oracle and show that every planted mistake is caught.
"""

import numpy as np
import pytest

from oracle import powersgd_ef as O

RNG = np.random.default_rng(12345)


def _rand(*shape, rng=None):
    return (rng or RNG).standard_normal(shape)


def _signed_qr(a):
    q, r = np.linalg.qr(a)
    return q * np.sign(np.diag(r))[None, :]


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ----------------------------------------------------------------------- pins
def pin_single_worker_is_thin_qr(mod, n=40, m=25, r=3, seed=1):
    """W=1, full-rank P: P = Q-factor of thin QR of M Q (diag R > 0); Q' = M^T P;
    U = P P^T M; E' = M - U.  LAPACK's Householder QR is independent of the oracle's
    Gram-Schmidt."""
    rng = np.random.default_rng(seed)
    g, e, q = _rand(1, n, m, rng=rng), _rand(1, n, m, rng=rng), _rand(m, r, rng=rng)
    res = mod.compress_matrix(g, e, q)
    M = g[0] + e[0]
    P = _signed_qr(M @ q)
    assert _rel(res.p_hat, P) < 1e-12
    assert _rel(res.q_bar, M.T @ P) < 1e-12
    assert _rel(res.update, P @ P.T @ M) < 1e-12
    assert _rel(res.errors[0], M - P @ P.T @ M) < 1e-12


def pin_rank1_is_power_iteration(mod, n=30, m=20, seed=2):
    """r=1 reduces to one normalised power-iteration step: P = MQ/||MQ||."""
    rng = np.random.default_rng(seed)
    g, q = _rand(1, n, m, rng=rng), _rand(m, 1, rng=rng)
    e = np.zeros_like(g)
    res = mod.compress_matrix(g, e, q)
    v = g[0] @ q
    assert _rel(res.p_hat, v / np.linalg.norm(v)) < 1e-12
    assert _rel(res.q_bar, g[0].T @ (v / np.linalg.norm(v))) < 1e-12


def pin_workers_reduce_to_mean_matrix(mod, W=5, n=24, m=18, r=2, seed=3):
    """Linearity (the page's reason all-reduce works): with a shared Q the mean of the
    workers' P equals P of the mean matrix, and P, Q, U equal those of a single worker
    holding mean_w (G_w + E_w); each worker's error is its own M_w - U."""
    rng = np.random.default_rng(seed)
    g, e, q = _rand(W, n, m, rng=rng), _rand(W, n, m, rng=rng), _rand(m, r, rng=rng)
    res = mod.compress_matrix(g, e, q)
    Mbar = (g + e).mean(axis=0)
    assert _rel(res.p_bar, Mbar @ q) < 1e-12
    one = mod.compress_matrix(Mbar[None], np.zeros((1, n, m)), q)
    assert _rel(res.p_hat, one.p_hat) < 1e-12
    assert _rel(res.q_bar, one.q_bar) < 1e-12
    assert _rel(res.update, one.update) < 1e-12
    for w in range(W):
        assert _rel(res.errors[w], g[w] + e[w] - one.update) < 1e-12


def pin_exact_when_rank_at_most_r(mod, W=4, n=32, m=20, r=3, seed=4):
    """If mean M has rank <= r and Q is generic, the step reconstructs it exactly:
    U = mean M and the workers' errors average to zero."""
    rng = np.random.default_rng(seed)
    low = _rand(n, 2, rng=rng) @ _rand(2, m, rng=rng)  # rank 2 <= r
    dev = _rand(W, n, m, rng=rng)
    dev -= dev.mean(axis=0, keepdims=True)  # zero-mean worker deviations
    g = low[None] + dev
    e = np.zeros_like(g)
    q = _rand(m, r, rng=rng)
    res = mod.compress_matrix(g, e, q)
    assert _rel(res.update, low) < 1e-12
    assert np.linalg.norm(res.errors.mean(axis=0)) < 1e-12 * np.linalg.norm(low)


def pin_identity_and_orthonormality(mod, W=3, n=50, m=30, r=4, seed=5):
    """M_w = U + E'_w for every worker; P^T P = I; P^T (mean E') = 0."""
    rng = np.random.default_rng(seed)
    g, e, q = _rand(W, n, m, rng=rng), _rand(W, n, m, rng=rng), _rand(m, r, rng=rng)
    res = mod.compress_matrix(g, e, q)
    for w in range(W):
        assert _rel(res.update + res.errors[w], g[w] + e[w]) < 1e-13
    assert np.abs(res.p_hat.T @ res.p_hat - np.eye(r)).max() < 1e-12
    resid = res.p_hat.T @ res.errors.mean(axis=0)
    assert np.abs(resid).max() < 1e-12 * np.linalg.norm(g + e)


def pin_svd_bounds(mod, n=12, m=9, r=2, seed=6, trials=20):
    """Eckart-Young: ||Mbar - U|| >= sqrt(sum_{i>r} sigma_i^2); U is a projection of
    Mbar, so ||Mbar - U|| <= ||Mbar||."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        W = 1 + rng.integers(3)
        g, e, q = _rand(W, n, m, rng=rng), _rand(W, n, m, rng=rng), _rand(m, r, rng=rng)
        res = mod.compress_matrix(g, e, q)
        Mbar = (g + e).mean(axis=0)
        s = np.linalg.svd(Mbar, compute_uv=False)
        err = np.linalg.norm(Mbar - res.update)
        assert err >= np.sqrt((s[r:] ** 2).sum()) * (1 - 1e-12)
        assert err <= np.linalg.norm(Mbar) * (1 + 1e-12)


def pin_warm_start_reaches_svd_bound(mod, n=64, m=48, r=2, steps=40, seed=7):
    """With a fixed matrix and the error reset each step, warm-starting from the
    previous Q is subspace iteration: the error falls to the best rank-r error (the
    page: warm start narrows the gap to the best rank-r approximation).  A fresh Q every
    step does not get there."""
    rng = np.random.default_rng(seed)
    U0, _ = np.linalg.qr(_rand(n, n, rng=rng))
    V0, _ = np.linalg.qr(_rand(m, m, rng=rng))
    s = 0.6 ** np.arange(m)
    M = (U0[:, :m] * s) @ V0.T
    best = np.sqrt((s[r:] ** 2).sum())
    q = _rand(m, r, rng=rng)
    for _ in range(steps):
        res = mod.compress_matrix(M[None], np.zeros((1, n, m)), q)
        q = res.q_bar
    warm = np.linalg.norm(M - res.update)
    assert abs(warm - best) / best < 1e-8
    cold = []
    for _ in range(steps):
        res = mod.compress_matrix(M[None], np.zeros((1, n, m)), _rand(m, r, rng=rng))
        cold.append(np.linalg.norm(M - res.update))
    assert np.median(cold) > best * (1 + 1e-3)


def pin_equivariances(mod, W=3, n=20, m=14, r=3, seed=8):
    """alpha*M scales P-bar, Q, U, E by alpha and leaves P fixed; -Q flips P and Q but
    not U; an orthogonal O on the left maps P to O P and U to O U; permuting workers
    permutes the errors only."""
    rng = np.random.default_rng(seed)
    g, e, q = _rand(W, n, m, rng=rng), _rand(W, n, m, rng=rng), _rand(m, r, rng=rng)
    base = mod.compress_matrix(g, e, q)
    a = 2.5
    sc = mod.compress_matrix(a * g, a * e, q)
    assert _rel(sc.p_hat, base.p_hat) < 1e-12
    assert _rel(sc.q_bar, a * base.q_bar) < 1e-12
    assert _rel(sc.update, a * base.update) < 1e-12
    assert _rel(sc.errors, a * base.errors) < 1e-12
    neg = mod.compress_matrix(g, e, -q)
    assert _rel(neg.p_hat, -base.p_hat) < 1e-12
    assert _rel(neg.q_bar, -base.q_bar) < 1e-12
    assert _rel(neg.update, base.update) < 1e-12
    Orth, _ = np.linalg.qr(_rand(n, n, rng=rng))
    rot = mod.compress_matrix(np.einsum("ij,wjk->wik", Orth, g), np.einsum("ij,wjk->wik", Orth, e), q)
    assert _rel(rot.p_hat, Orth @ base.p_hat) < 1e-12
    assert _rel(rot.q_bar, base.q_bar) < 1e-12
    assert _rel(rot.update, Orth @ base.update) < 1e-12
    perm = rng.permutation(W)
    pr = mod.compress_matrix(g[perm], e[perm], q)
    assert _rel(pr.update, base.update) < 1e-12
    assert _rel(pr.errors, base.errors[perm]) < 1e-12


def pin_dependent_column_dropped(mod, n=16, m=10, seed=9):
    """A rank-1 matrix at r=2: the second column of P-bar is a multiple of the first,
    so it is dropped (zero) rather than normalising rounding noise; U is still exact
    and nothing is NaN.  An all-zero gradient gives all-zero outputs."""
    rng = np.random.default_rng(seed)
    M = np.outer(_rand(n, rng=rng), _rand(m, rng=rng))
    q = _rand(m, 2, rng=rng)
    res = mod.compress_matrix(M[None], np.zeros((1, n, m)), q)
    assert np.all(res.p_hat[:, 1] == 0.0)
    assert _rel(res.update, M) < 1e-13
    z = mod.compress_matrix(np.zeros((2, n, m)), np.zeros((2, n, m)), q)
    assert np.all(z.p_hat == 0) and np.all(z.q_bar == 0) and np.all(z.update == 0)
    assert np.all(np.isfinite(z.errors))


def pin_local_q_error(mod, W=3, n=22, m=15, r=2, seed=10):
    """With each worker's own Q in the error, E'_w = (I - P P^T) M_w, and the worker
    mean of the errors is the same as with the aggregated Q."""
    rng = np.random.default_rng(seed)
    g, e, q = _rand(W, n, m, rng=rng), _rand(W, n, m, rng=rng), _rand(m, r, rng=rng)
    loc = mod.compress_matrix(g, e, q, local_q_error=True)
    glob = mod.compress_matrix(g, e, q)
    proj = np.eye(n) - loc.p_hat @ loc.p_hat.T
    for w in range(W):
        assert _rel(loc.errors[w], proj @ (g[w] + e[w])) < 1e-12
    assert _rel(loc.errors.mean(axis=0), glob.errors.mean(axis=0)) < 1e-12


def pin_uncompressed_mean(mod, seed=11):
    """Tensors that are not compressed are averaged over workers."""
    rng = np.random.default_rng(seed)
    g = _rand(7, 1, 33, rng=rng)
    assert _rel(mod.average_tensor(g), g.sum(axis=0) / 7.0) < 1e-15


def pin_momentum_closed_form(mod, seed=12):
    """Constant update U from mom=0: mom_t = U (1 - mu^t)/(1 - mu) and
    x_t = x_0 - lr * sum_s mom_s (heavy ball); Nesterov adds mu*mom_s to each step."""
    rng = np.random.default_rng(seed)
    U, x0 = _rand(5, 4, rng=rng), _rand(5, 4, rng=rng)
    lr, mu, T = 0.1, 0.9, 25
    mom, x = np.zeros_like(U), x0.copy()
    momn, xn = np.zeros_like(U), x0.copy()
    acc, accn = np.zeros_like(U), np.zeros_like(U)
    for t in range(1, T + 1):
        mom, x = mod.momentum_sgd(mom, x, U, lr, mu)
        momn, xn = mod.momentum_sgd(momn, xn, U, lr, mu, nesterov=True)
        mt = U * (1 - mu ** t) / (1 - mu)
        assert _rel(mom, mt) < 1e-13
        acc += mt
        accn += U + mu * mt
        assert _rel(x, x0 - lr * acc) < 1e-12
        assert _rel(xn, x0 - lr * accn) < 1e-12


def pin_power_iterations_reach_svd(mod, n=40, m=30, r=3, seed=13):
    """Many power iterations inside one step from a random Q converge to the top-r
    singular subspace: U is then the SVD-optimal rank-r approximation (Eckart-Young
    equality), and one iteration is the plain step."""
    rng = np.random.default_rng(seed)
    U0, _ = np.linalg.qr(_rand(n, n, rng=rng))
    V0, _ = np.linalg.qr(_rand(m, m, rng=rng))
    s = 0.5 ** np.arange(m)
    M = (U0[:, :m] * s) @ V0.T
    q = _rand(m, r, rng=rng)
    z = np.zeros((1, n, m))
    many = mod.compress_matrix(M[None], z, q, iterations=60)
    best = (U0[:, :r] * s[:r]) @ V0[:, :r].T
    assert _rel(many.update, best) < 1e-10
    one = mod.compress_matrix(M[None], z, q, iterations=1)
    plain = mod.compress_matrix(M[None], z, q)
    assert _rel(one.update, plain.update) == 0.0


PINS = [
    pin_single_worker_is_thin_qr,
    pin_rank1_is_power_iteration,
    pin_workers_reduce_to_mean_matrix,
    pin_exact_when_rank_at_most_r,
    pin_identity_and_orthonormality,
    pin_svd_bounds,
    pin_warm_start_reaches_svd_bound,
    pin_equivariances,
    pin_dependent_column_dropped,
    pin_local_q_error,
    pin_uncompressed_mean,
    pin_momentum_closed_form,
    pin_power_iterations_reach_svd,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(O)


def test_compress_layers_dispatch():
    """compress_layers averages tensors without a Q and compresses the rest."""
    rng = np.random.default_rng(13)
    g1, e1, q1 = _rand(2, 6, 5, rng=rng), _rand(2, 6, 5, rng=rng), _rand(5, 2, rng=rng)
    g2 = _rand(2, 1, 7, rng=rng)
    out = O.compress_layers([O.LayerState(g1, e1, q1), O.LayerState(g2, np.zeros_like(g2), None)])
    ref = O.compress_matrix(g1, e1, q1)
    assert _rel(out[0].update, ref.update) < 1e-15
    assert _rel(out[1], g2.mean(axis=0)) < 1e-15
