"""GPU parity of the Spectral-ATOMO step (libpsgd through its C ABI) against the CPU oracle.

What is unique is compared with the float64 oracle: the singular values, the
probabilities, which atoms are sent, and, where the singular values are separated,
the sent factors themselves (up to the sign a singular vector does not fix) and the
update.  Inside clusters of close singular values the vectors are not unique; there
every sent atom is checked to be a valid one: a unit eigenvector of the Gram matrix
for its singular value (residual test), orthogonal to the other sent atoms, with the
second factor equal to G^T u / p (or G v / p), and the update equal to the workers'
mean of the atoms actually sent.

Tolerances (float32 Gram matrix, Householder tridiagonalisation, bisection):
  * singular values: |d sigma_i| <= TOL_SIGMA * sigma_max.  The eigenvalues of the
    computed Gram matrix carry an error of a few sqrt(k) * 2^-24 * sigma_max^2, so
    d sigma_i <= that / (2 sigma_i); the inputs here keep sigma_i >= sigma_max / 8;
  * probabilities: |d p_i| <= TOL_P (p is c * sigma_i with c a sum of sigma);
  * a separated atom: angle to the oracle's vector <= TOL_VEC, from the eigenvalue
    error over the gap to the neighbouring eigenvalues (>= 1.5% of sigma_max^2 here);
  * the update: relative Frobenius error <= TOL_U, the atoms' error times the few
    atoms sent.
Uniforms closer than 1e-4 to the oracle's p_i are moved away, so both sides take the
same Bernoulli decisions.  Every case prints what names it before touching the GPU.
"""

import numpy as np
import pytest

from distributed_sgd_gradient_ef_amd import psgd as P
from distributed_sgd_gradient_ef_amd import workloads as WL
from oracle import atomo as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda:0"

TOL_SIGMA = 2e-5
TOL_P = 1e-4
TOL_VEC = 2e-4
TOL_U = 2e-4
TOL_RESID = 2e-5   # ||B u - sigma^2 u|| / sigma_max^2 for a sent atom
TOL_ORTH = 1e-4
MARGIN = 1e-4


class AtomoRun:
    """Device buffers of one ATOMO plan, filled with garbage where the step must write."""

    def __init__(self, shapes, budget, W):
        self.shapes = [tuple(s) for s in shapes]
        self.plan = P.psgd_atomo_plan_create(shapes, budget, W)
        s = self.plan.sizes
        self.W = W
        self.stride = s["worker_stride"]
        sv = max(1, s["sv_total"])
        self.g = torch.zeros((W, self.stride), dtype=torch.float32, device=DEV)
        self.x = torch.zeros((W, sv), dtype=torch.float32, device=DEV)
        self.sigma = torch.full((W, sv), float("nan"), dtype=torch.float32, device=DEV)
        self.prob = torch.full((W, sv), float("nan"), dtype=torch.float32, device=DEV)
        self.index = torch.full((W, sv), 0x7EADBEEF, dtype=torch.int32, device=DEV)
        self.count = torch.full((W, max(1, s["n_matrices"])), -7, dtype=torch.int32, device=DEV)
        self.atoms = torch.full((W, max(1, s["atom_total"])), float("nan"), dtype=torch.float32, device=DEV)
        self.update = torch.full((self.stride,), float("nan"), dtype=torch.float32, device=DEV)
        self.ws = torch.full((max(256, s["workspace_bytes"]),), 0xAB, dtype=torch.uint8, device=DEV)

    def set_grads(self, per_layer):
        self.g.copy_(torch.from_numpy(P.pack(self.plan, [np.asarray(a, np.float32) for a in per_layer])).to(DEV))

    def set_uniforms(self, per_matrix):
        rows = P.pack_sv(self.plan, per_matrix)
        self.x[:, :rows.shape[1]].copy_(torch.from_numpy(rows).to(DEV))

    def step(self, update=True):
        P.psgd_atomo_step(self.plan, self.g, self.x, self.sigma, self.prob, self.index, self.count, self.atoms,
                          self.update if update else None, self.ws)
        torch.cuda.synchronize()

    def fetch(self):
        return dict(sigma=self.sigma.cpu().numpy(), prob=self.prob.cpu().numpy(), index=self.index.cpu().numpy(),
                    count=self.count.cpu().numpy(), atoms=self.atoms.cpu().numpy(),
                    update=self.update.cpu().numpy())


def _haar(rng, n, k):
    q, r = np.linalg.qr(rng.standard_normal((n, k)))
    return q * np.sign(np.diag(r))


def _spectral(rng, n, m, sig):
    k = min(n, m)
    return (_haar(rng, n, k) * sig) @ _haar(rng, m, k).T


def _separated_sigma(k, w):
    """Singular values from 2 down to 0.5, evenly spaced, scaled per worker."""
    return (2.0 - 1.5 * np.arange(k) / max(1, k - 1)) * (1.0 + 0.1 * w)


def _nudge(x, p):
    """Move uniforms that lie within MARGIN of p away from it (staying in [0, 1))."""
    x = np.array(x, dtype=np.float32)
    close = np.abs(x.astype(np.float64) - p) < MARGIN
    x[close] = np.float32((x[close] + 3 * MARGIN) % 1.0)
    return x


def _run_case(name, shapes, budget, W, grads, xs):
    """One step on the GPU and the oracle on every (worker, matrix); returns both."""
    print(f"[atomo] case {name}: shapes={shapes} W={W} budget={budget}", flush=True)
    run = AtomoRun(shapes, budget, W)
    oracle = {}
    for li, L in enumerate(run.plan.layers):
        if L.compressed:
            per = []
            for w in range(W):
                g64 = np.asarray(grads[li][w], np.float32).astype(np.float64)
                p = O.probabilities(O.svd_atoms(g64)[0], budget)
                xs[li][w] = _nudge(xs[li][w], p)
                per.append(O.compress_matrix(g64, budget, xs[li][w]))
            oracle[li] = per
    run.set_grads(grads)
    run.set_uniforms({li: xs[li] for li in oracle})
    run.step()
    return run, run.fetch(), oracle


def _check_layer(plan, out, li, orc, g_layer, compare_vectors=True, check_update=True):
    """out holds the step's outputs for len(orc) workers (rows of every [W][...] array)
    and g_layer their gradients of layer li."""
    L = plan.layers[li]
    W = len(orc)
    sig = P.sv_slice(plan, out["sigma"], li)
    prb = P.sv_slice(plan, out["prob"], li)
    idx = P.sv_slice(plan, out["index"], li)
    est = np.zeros((L.rows, L.cols))
    for w in range(W):
        o = orc[w]
        smax = max(o.sigma[0], 1e-30)
        assert np.max(np.abs(sig[w] - o.sigma)) <= TOL_SIGMA * smax, \
            f"layer {li} w{w}: sigma differs by {np.max(np.abs(sig[w] - o.sigma)) / smax:.2e} of sigma_max"
        assert np.max(np.abs(prb[w] - o.prob)) <= TOL_P, f"layer {li} w{w}: prob differs"
        cnt = int(out["count"][w, L.matrix_index])
        assert cnt == o.index.size, f"layer {li} w{w}: {cnt} atoms sent, oracle {o.index.size}"
        assert np.array_equal(idx[w, :cnt], o.index) and np.all(idx[w, cnt:] == -1), f"layer {li} w{w}: index"
        a, b = P.atom_factors(plan, out["atoms"], out["count"], li, w)
        g = np.asarray(g_layer[w], np.float32).astype(np.float64)
        unit, other = (a, b) if L.rows <= L.cols else (b, a)
        gram = g @ g.T if L.rows <= L.cols else g.T @ g
        for j, i in enumerate(o.index):
            u = unit[j].astype(np.float64)
            assert abs(np.linalg.norm(u) - 1.0) <= 1e-5, f"layer {li} w{w} atom {i}: not a unit vector"
            res = np.linalg.norm(gram @ u - (float(sig[w, i]) ** 2) * u) / smax ** 2
            assert res <= TOL_RESID, f"layer {li} w{w} atom {i}: eigen-residual {res:.2e}"
            second = (g.T @ u if L.rows <= L.cols else g @ u) / float(prb[w, i])
            assert np.linalg.norm(other[j] - second) <= 1e-5 * np.linalg.norm(second) + 1e-30, \
                f"layer {li} w{w} atom {i}: second factor is not G^T u / p"
            if compare_vectors:
                ou, oo = (o.a[j], o.b[j]) if L.rows <= L.cols else (o.b[j], o.a[j])
                sgn = 1.0 if u @ ou >= 0 else -1.0
                assert np.linalg.norm(sgn * u - ou) <= TOL_VEC, f"layer {li} w{w} atom {i}: vector"
                assert np.linalg.norm(sgn * other[j] - oo) <= TOL_VEC * np.linalg.norm(oo), \
                    f"layer {li} w{w} atom {i}: second factor vs oracle"
        if cnt > 1:
            gm = unit[:cnt].astype(np.float64) @ unit[:cnt].astype(np.float64).T
            assert np.max(np.abs(gm - np.eye(cnt))) <= TOL_ORTH, f"layer {li} w{w}: sent atoms not orthonormal"
        est += a.astype(np.float64).T @ b.astype(np.float64)
    if not check_update:
        return
    upd = P.unpack(plan, out["update"], li).astype(np.float64)
    mean_sent = est / W
    assert np.linalg.norm(upd - mean_sent) <= 1e-5 * max(np.linalg.norm(mean_sent), 1e-30), \
        f"layer {li}: update is not the mean of the sent atoms"
    if compare_vectors:
        ref = sum(r.estimate for r in orc) / W
        assert np.linalg.norm(upd - ref) <= TOL_U * max(np.linalg.norm(ref), 1e-30), f"layer {li}: update"


def _check_vectors(run, out, grads):
    for li, L in enumerate(run.plan.layers):
        if not L.compressed:
            ref = np.asarray(grads[li], np.float32).astype(np.float64).mean(axis=0)
            upd = P.unpack(run.plan, out["update"], li)
            assert np.allclose(upd, ref, rtol=1e-6, atol=1e-7), f"layer {li}: uncompressed mean"


SMALL = [(6, 9), (9, 6), (2, 5), (5, 2), (1, 30), (20, 33), (33, 20), (64, 27), (3, 200), (7, 1), (40, 40)]


@pytest.mark.parametrize("budget", [0.6, 1.7, 4.0])
def test_separated_spectra_match_oracle(budget):
    rng = np.random.default_rng(400 + int(10 * budget))
    W = 3
    grads, xs = [], []
    for n, m in SMALL:
        if min(n, m) >= 2:
            grads.append(np.stack([_spectral(rng, n, m, _separated_sigma(min(n, m), w)) for w in range(W)]))
            xs.append(rng.random((W, min(n, m))).astype(np.float32))
        else:
            grads.append(rng.standard_normal((W, n, m)))
            xs.append(None)
    run, out, orc = _run_case(f"separated s={budget}", SMALL, budget, W, grads, xs)
    for li in orc:
        _check_layer(run.plan, out, li, orc[li], grads[li])
    _check_vectors(run, out, grads)


def test_full_budget_reconstructs_the_gradient():
    """s >= k: every atom is sent with p = 1, so the estimate is G itself, also for noise
    matrices whose singular values cluster."""
    rng = np.random.default_rng(410)
    shapes = [(48, 100), (100, 48), (128, 300), (12, 12), (2, 9)]
    W = 2
    grads = [rng.standard_normal((W, n, m)) for n, m in shapes]
    xs = [rng.random((W, min(n, m))).astype(np.float32) for n, m in shapes]
    run, out, orc = _run_case("full budget", shapes, 1e6, W, grads, xs)
    for li, L in enumerate(run.plan.layers):
        assert np.all(out["count"][:, L.matrix_index] == L.k)
        assert np.all(P.sv_slice(run.plan, out["prob"], li) == 1.0)
        _check_layer(run.plan, out, li, orc[li], grads[li], compare_vectors=False)
        ref = np.asarray(grads[li], np.float32).astype(np.float64).mean(axis=0)
        upd = P.unpack(run.plan, out["update"], li)
        assert np.linalg.norm(upd - ref) <= 1e-4 * np.linalg.norm(ref), f"layer {li}: not reconstructed"


def test_resnet18_workload():
    """The benchmarked workload at full size (W = 16, s = 2): sampled workers against
    the oracle; every worker's update against its sent atoms."""
    wl = WL.workload("resnet18_atomo")
    shapes = [s for _, s in wl.shapes]
    W, budget = wl.workers, wl.atomo_budget
    grads = WL.grads(wl, 0)
    plan_probe = P.psgd_atomo_plan_create(shapes, budget, W)
    xs = [np.stack([WL.atomo_uniforms(wl, 0, w, li, L.k) for w in range(W)]) if L.compressed else None
          for li, L in enumerate(plan_probe.layers)]
    del plan_probe
    sampled = (0, 7, 15)
    print(f"[atomo] case resnet18_atomo: W={W} s={budget} sampled workers {sampled}", flush=True)
    run = AtomoRun(shapes, budget, W)
    oracle = {}
    for li, L in enumerate(run.plan.layers):
        if L.compressed:
            per = []
            for w in sampled:
                g64 = grads[li][w].astype(np.float64)
                p = O.probabilities(O.svd_atoms(g64)[0], budget)
                xs[li][w] = _nudge(xs[li][w], p)
                per.append(O.compress_matrix(g64, budget, xs[li][w]))
            oracle[li] = per
    run.set_grads(grads)
    run.set_uniforms({li: xs[li] for li in oracle})
    run.step()
    out = run.fetch()
    for li, per in oracle.items():
        L = run.plan.layers[li]
        sub = {k: (v[list(sampled)] if k != "update" else v) for k, v in out.items()}
        _check_layer(run.plan, sub, li, per, grads[li][list(sampled)], compare_vectors=False, check_update=False)
        # every worker: the update is the mean of the atoms sent
        est = np.zeros((L.rows, L.cols))
        for w in range(W):
            a, b = P.atom_factors(run.plan, out["atoms"], out["count"], li, w)
            est += a.astype(np.float64).T @ b.astype(np.float64)
        upd = P.unpack(run.plan, out["update"], li)
        assert np.linalg.norm(upd - est / W) <= 1e-5 * np.linalg.norm(est / W), f"layer {li}: update"
    _check_vectors(run, out, grads)


def test_degenerate_inputs():
    """A zero matrix sends nothing; equal singular values give equal probabilities; a
    2 x 2 and a 2 x n problem."""
    rng = np.random.default_rng(420)
    shapes = [(8, 11), (6, 6), (2, 2), (2, 7), (7, 2)]
    W = 2
    grads = [np.zeros((W, 8, 11)),
             np.stack([3.0 * _haar(rng, 6, 6) for _ in range(W)]),
             rng.standard_normal((W, 2, 2)), rng.standard_normal((W, 2, 7)), rng.standard_normal((W, 7, 2))]
    xs = [rng.random((W, min(n, m))).astype(np.float32) for n, m in shapes]
    run, out, orc = _run_case("degenerate", shapes, 1.5, W, grads, xs)
    L0 = run.plan.layers[0]
    assert np.all(out["count"][:, L0.matrix_index] == 0)
    assert np.all(P.sv_slice(run.plan, out["sigma"], 0) == 0) and np.all(P.sv_slice(run.plan, out["prob"], 0) == 0)
    assert np.all(P.unpack(run.plan, out["update"], 0) == 0)
    p1 = P.sv_slice(run.plan, out["prob"], 1)
    assert np.allclose(p1, 1.5 / 6, atol=1e-5)
    _check_layer(run.plan, out, 1, orc[1], grads[1], compare_vectors=False)   # any basis of the one cluster
    for li in (2, 3, 4):
        _check_layer(run.plan, out, li, orc[li], grads[li])


def test_largest_k():
    rng = np.random.default_rng(430)
    k = P.PSGD_ATOMO_MAX_K
    shapes = [(k, k + 6)]
    grads = [_spectral(rng, k, k + 6, 2.0 - 1.2 * np.arange(k) / (k - 1))[None]]
    xs = [rng.random((1, k)).astype(np.float32)]
    run, out, orc = _run_case("k = 1024", shapes, 3.0, 1, grads, xs)
    _check_layer(run.plan, out, 0, orc[0], grads[0], compare_vectors=False)


def test_step_is_reproducible_and_update_optional():
    rng = np.random.default_rng(440)
    shapes = [(30, 70), (70, 30), (1, 50)]
    W = 4
    grads = [rng.standard_normal((W, n, m)) for n, m in shapes]
    print("[atomo] case reproducibility", flush=True)
    run = AtomoRun(shapes, 2.0, W)
    run.set_grads(grads)
    run.set_uniforms({0: rng.random((W, 30)).astype(np.float32), 1: rng.random((W, 30)).astype(np.float32)})
    run.step()
    first = run.fetch()
    run.update.fill_(float("nan"))
    run.step(update=False)
    second = run.fetch()
    for key in ("sigma", "prob", "index", "count", "atoms"):
        assert np.array_equal(first[key], second[key], equal_nan=True), key
    assert np.all(np.isnan(second["update"]))


def test_lstm_shaped_matrices():
    """k = 650 in both orientations (the widest width class, 1 < k / 512), with the
    separated spectra of the parity cases."""
    rng = np.random.default_rng(450)
    shapes = [(2000, 650), (650, 1300)]
    W = 2
    grads = [np.stack([_spectral(rng, n, m, _separated_sigma(min(n, m), w)) for w in range(W)]) for n, m in shapes]
    xs = [rng.random((W, 650)).astype(np.float32) for _ in shapes]
    run, out, orc = _run_case("lstm-shaped", shapes, 3.0, W, grads, xs)
    for li in orc:
        _check_layer(run.plan, out, li, orc[li], grads[li], compare_vectors=False)


def test_plan_without_matrices():
    """Only 1-D tensors: no decomposition runs and the update is the workers' mean."""
    rng = np.random.default_rng(460)
    shapes = [(1, 300), (5, 1), (1, 4097)]
    W = 3
    grads = [rng.standard_normal((W, n, m)) for n, m in shapes]
    print("[atomo] case vectors only", flush=True)
    run = AtomoRun(shapes, 2.0, W)
    assert run.plan.sizes["n_matrices"] == 0 and run.plan.sizes["sv_total"] == 0
    run.set_grads(grads)
    run.step()
    _check_vectors(run, run.fetch(), grads)


def test_width_class_129_to_256():
    """Widest k in 129..256 (several band panels, a chase longer than one LDS chunk of the
    back-transform's smaller cases), both orientations and k = 256, with the separated
    spectra of the parity cases.  The gaps between neighbouring singular values are
    0.15-0.3% of sigma_max here, too close for a vector-by-vector comparison, so sent
    atoms are checked for validity (as in the other wide cases)."""
    rng = np.random.default_rng(470)
    shapes = [(200, 300), (256, 256), (300, 129), (1, 40)]
    W = 2
    grads = []
    for n, m in shapes:
        if min(n, m) >= 2:
            grads.append(np.stack([_spectral(rng, n, m, _separated_sigma(min(n, m), w)) for w in range(W)]))
        else:
            grads.append(rng.standard_normal((W, n, m)))
    xs = [rng.random((W, min(n, m))).astype(np.float32) if min(n, m) >= 2 else None for n, m in shapes]
    run, out, orc = _run_case("k in 129..256", shapes, 3.0, W, grads, xs)
    for li in orc:
        _check_layer(run.plan, out, li, orc[li], grads[li], compare_vectors=False)
    _check_vectors(run, out, grads)
