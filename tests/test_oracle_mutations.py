"""Plant mistakes in (a patched copy of) the CPU oracle and check that the pins in
test_oracle.py catch every one of them.  Runs on the CPU only; the real oracle module
is restored after each case by pytest's monkeypatch."""

import numpy as np
import pytest

from oracle import powersgd_ef as O
from tests.test_oracle import PINS


def _f(a):
    return np.asarray(a, dtype=np.float64)


def _cgs_no_drop(p, tol=O.DROP_TOL):
    p = _f(p)
    out = np.zeros_like(p)
    for k in range(p.shape[1]):
        v = p[:, k] - out[:, :k] @ (out[:, :k].T @ p[:, k])
        out[:, k] = v / np.linalg.norm(v)
    return out


MUTATIONS = {
    "ef_add drops the error": ("ef_add", lambda g, e: _f(g)),
    "ef_add subtracts the error": ("ef_add", lambda g, e: _f(g) - _f(e)),
    "all-reduce sums instead of averaging": ("all_reduce_mean", lambda parts: sum(_f(x) for x in parts)),
    "all-reduce keeps worker 0 only": ("all_reduce_mean", lambda parts: _f(parts[0])),
    "no orthonormalisation": ("orthonormalise", lambda p, tol=O.DROP_TOL: _f(p)),
    "normalise without orthogonalising": ("orthonormalise", lambda p, tol=O.DROP_TOL: _f(p) / np.linalg.norm(_f(p), axis=0)),
    "no drop rule for dependent columns": ("orthonormalise", _cgs_no_drop),
    "P from the transposed warm start": ("worker_p", lambda m, q: _f(m) @ _f(q)[::-1]),
    "Q from P-bar rows reversed": ("worker_q", lambda m, p: _f(m).T @ _f(p)[::-1]),
    "decompress with the wrong sign": ("decompress", lambda p, q: -(_f(p) @ _f(q).T)),
    "error keeps M + U": ("new_error", lambda m, u: _f(m) + _f(u)),
    "error forgets the compression": ("new_error", lambda m, u: _f(m)),
    "uncompressed tensors summed": ("average_tensor", lambda g: _f(g).sum(axis=0)),
    "momentum applies U, not mom": ("momentum_sgd", lambda mom, x, u, lr, mu, nesterov=False:
                                    (mu * _f(mom) + _f(u), _f(x) - lr * _f(u))),
    "momentum decays the update": ("momentum_sgd", lambda mom, x, u, lr, mu, nesterov=False:
                                   (mu * (_f(mom) + _f(u)), _f(x) - lr * mu * (_f(mom) + _f(u)))),
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
