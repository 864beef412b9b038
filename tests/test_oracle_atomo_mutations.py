"""Plant mistakes in (a patched copy of) the Spectral-ATOMO oracle and check that the
pins in test_oracle_atomo.py catch every one of them.  CPU only; pytest's monkeypatch
restores the real module after each case."""

import numpy as np
import pytest

from oracle import atomo as O
from tests.test_oracle_atomo import PINS

_REAL_PROB = O.probabilities
_REAL_SVD = O.svd_atoms
_REAL_COMPRESS = O.compress_matrix


def _prob_proportional_no_cap(lam, s):
    a = np.abs(np.asarray(lam, np.float64))
    return np.minimum(1.0, s * a / a.sum()) if a.sum() > 0 else np.zeros_like(a)


def _prob_sqrt(lam, s):
    a = np.asarray(lam, np.float64) ** 2
    return _REAL_PROB(np.sqrt(np.sqrt(a)), s)    # p proportional to sqrt|lam| instead of |lam|


def _prob_uniform(lam, s):
    a = np.abs(np.asarray(lam, np.float64))
    return np.where(a > 0, min(1.0, s / max(1, np.count_nonzero(a))), 0.0)


def _prob_saturates_smallest(lam, s):
    a = np.abs(np.asarray(lam, np.float64))
    return _REAL_PROB(np.where(a > 0, 1.0 / np.where(a > 0, a, 1.0), 0.0), s)


def _sparsify_no_rescale(lam, atoms, p, t):
    out = np.zeros(np.shape(atoms[0]))
    for li, ai, ti in zip(lam, atoms, t):
        if ti:
            out += li * np.asarray(ai, np.float64)
    return out


def _sparsify_divides_by_p_squared(lam, atoms, p, t):
    out = np.zeros(np.shape(atoms[0]))
    for li, ai, pi, ti in zip(lam, atoms, p, t):
        if ti:
            out += li / pi ** 2 * np.asarray(ai, np.float64)
    return out


def _svd_ascending(g):
    s, u, vt = _REAL_SVD(g)
    return s[::-1].copy(), u[:, ::-1].copy(), vt[::-1].copy()


def _svd_squared(g):
    s, u, vt = _REAL_SVD(g)
    return s ** 2, u, vt


def _svd_swapped_right(g):
    s, u, vt = _REAL_SVD(g)
    return s, u, vt[::-1].copy() if vt.shape[0] > 1 else -vt


def _compress_unscaled_factor(g, s, x):
    r = _REAL_COMPRESS(g, s, x)
    n, m = np.shape(g)
    if n <= m:
        r.b = r.b * (r.prob[r.index] / np.where(r.sigma[r.index] > 0, r.sigma[r.index], 1))[:, None]
    else:
        r.a = r.a * (r.prob[r.index] / np.where(r.sigma[r.index] > 0, r.sigma[r.index], 1))[:, None]
    return r


def _compress_wrong_unit_side(g, s, x):
    r = _REAL_COMPRESS(g, s, x)
    scale = (r.sigma[r.index] / r.prob[r.index])[:, None]
    safe = np.where(scale > 0, scale, 1.0)
    if np.shape(g)[0] <= np.shape(g)[1]:
        r.a, r.b = r.a * scale, r.b / safe
    else:
        r.a, r.b = r.a / safe, r.b * scale
    return r


def _sample_le(p, x):
    return np.asarray(x, np.float64) <= np.asarray(p, np.float64)


def _sample_inverted(p, x):
    return np.asarray(x, np.float64) > 1.0 - np.asarray(p, np.float64) * 0.5


def _compress_layer_sum(g, s, x):
    g = np.asarray(g, np.float64)
    W = g.shape[0]
    if not O.is_matrix(g.shape[1:]):
        return O.AtomoLayer([], g.mean(axis=0))
    per = [O.compress_matrix(g[w], s, x[w]) for w in range(W)]
    return O.AtomoLayer(per, sum(r.estimate for r in per))


def _compress_layer_first_uniforms(g, s, x):
    g = np.asarray(g, np.float64)
    W = g.shape[0]
    if not O.is_matrix(g.shape[1:]):
        return O.AtomoLayer([], g.mean(axis=0))
    per = [O.compress_matrix(g[w], s, x[0]) for w in range(W)]
    return O.AtomoLayer(per, sum(r.estimate for r in per) / W)


MUTATIONS = {
    "probabilities capped without redistributing": ("probabilities", _prob_proportional_no_cap),
    "probabilities proportional to sqrt|lambda|": ("probabilities", _prob_sqrt),
    "uniform probabilities": ("probabilities", _prob_uniform),
    "the smallest atoms saturate first": ("probabilities", _prob_saturates_smallest),
    "estimate not rescaled by 1/p": ("sparsify", _sparsify_no_rescale),
    "estimate rescaled by 1/p^2": ("sparsify", _sparsify_divides_by_p_squared),
    "singular values ascending": ("svd_atoms", _svd_ascending),
    "squared singular values as weights": ("svd_atoms", _svd_squared),
    "right vectors out of order": ("svd_atoms", _svd_swapped_right),
    "sent factor not scaled by sigma/p": ("compress_matrix", _compress_unscaled_factor),
    "unit factor on the long side": ("compress_matrix", _compress_wrong_unit_side),
    "atom sent when x == p": ("sample", _sample_le),
    "sampling rule inverted": ("sample", _sample_inverted),
    "update sums instead of averaging": ("compress_layer", _compress_layer_sum),
    "every worker uses worker 0's uniforms": ("compress_layer", _compress_layer_first_uniforms),
}


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin(O)
        except Exception:  # an assertion or a shape error both count as caught
            failed.append(pin.__name__)
    assert failed, f"mutation '{name}' passed every pin"
