"""Plain CPU oracle for one PowerSGD rank-r compression step with error feedback.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the benchmark's
CPU-baseline leg may import this module.  The GPU library never calls it and shares no
code with it: the two meet only at the seeded inputs.

What it follows
---------------
The review page "PowerSGD: Practical Low-Rank Gradient Compression for Distributed
Optimization" (Vogels, Karimireddy et al., 2019), section "Proposed method" (提案手法):

* each layer's gradient is reshaped to an n x m matrix and compressed on its own, as
  P Q^T with P in R^{n x r}, Q in R^{m x r} and a small rank r (1-4);
* the factors come from one step of subspace (power) iteration warm-started from the
  previous step's Q;
* because the compressor is linear, the W workers' P and Q are aggregated by
  all-reduce;
* error feedback: the error left after compression is added back to the next
  gradient, which is what lets a biased compressor converge;
* the update is decompressed as P Q^T and applied by momentum SGD.

Readings where the page leaves a step open (each is the plainest reading that the rest
of the page supports):

* all-reduce = mean over workers (gradient averaging); P's scale does not matter after
  orthonormalisation, Q's does;
* one warm-start Q per matrix, shared by all workers (linearity needs it); the next
  step's Q is this step's aggregated Q, not re-normalised;
* orthonormalisation = modified Gram-Schmidt over the columns in index order, no
  re-orthogonalisation.  A column whose residual norm is at most 1e-4 times its norm
  before orthogonalisation (or exactly zero) is set to zero instead of normalised;
* the new error uses the aggregated Q: E'_w = M_w - P Q^T, one decompressed update per
  matrix;
* tensors that are not compressed (1-D tensors, or a matrix whose smaller side is at
  most r) are averaged over workers and keep no error;
* momentum SGD is heavy-ball: mom <- mu*mom + U; x <- x - lr*mom (Nesterov optional);
* arithmetic is float64 throughout; inputs are widened exactly.

Every function here is pinned by tests/test_oracle.py against facts fixed by the page
and by linear algebra (thin QR, SVD bounds, closed forms, invariants); none is "parity
unpinned".  Columns zeroed by the drop rule are deterministic but nothing on the page
fixes them, so tests compare U and E' there rather than P and Q.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence

import numpy as np

DROP_TOL = 1e-4


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------- one matrix, W workers
def ef_add(g: np.ndarray, e: np.ndarray) -> np.ndarray:
    """Error feedback: the remembered compression error is added to the new gradient."""
    return _f64(g) + _f64(e)


def worker_p(m_w: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Power-iteration half step on one worker: P_w = M_w Q (Q = warm start)."""
    return _f64(m_w) @ _f64(q)


def worker_q(m_w: np.ndarray, p_hat: np.ndarray) -> np.ndarray:
    """Second half step on one worker: Q_w = M_w^T P_hat."""
    return _f64(m_w).T @ _f64(p_hat)


def all_reduce_mean(parts: Sequence[np.ndarray]) -> np.ndarray:
    """Aggregation of a linear message across workers: the mean of the W copies."""
    acc = np.zeros_like(_f64(parts[0]))
    for x in parts:
        acc = acc + _f64(x)
    return acc / len(parts)


def orthonormalise(p: np.ndarray, tol: float = DROP_TOL) -> np.ndarray:
    """Modified Gram-Schmidt on the columns of p (n x r), in column order.

    Column k is orthogonalised against the already finished columns one at a time,
    each projection using the partly reduced vector.  If what is left has norm
    <= tol * (norm of the original column), or is zero, the column becomes zero.
    """
    p = _f64(p)
    n, r = p.shape
    out = np.zeros((n, r))
    for k in range(r):
        v = p[:, k].copy()
        before = np.sqrt(np.dot(v, v))
        for l in range(k):
            v = v - np.dot(out[:, l], v) * out[:, l]
        after = np.sqrt(np.dot(v, v))
        if after > 0.0 and after > tol * before:
            out[:, k] = v / after
    return out


def decompress(p_hat: np.ndarray, q_bar: np.ndarray) -> np.ndarray:
    """Decompressed update U = P Q^T."""
    return _f64(p_hat) @ _f64(q_bar).T


def new_error(m_w: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Error left after compression, remembered for the next step: M_w - U."""
    return _f64(m_w) - _f64(u)


@dataclass
class MatrixStep:
    p_bar: np.ndarray  # mean_w P_w, before orthonormalisation (n x r)
    p_hat: np.ndarray  # orthonormalised P (n x r)
    q_bar: np.ndarray  # mean_w Q_w (m x r); the next step's warm start
    update: np.ndarray  # U = P_hat Q_bar^T (n x m)
    errors: np.ndarray  # E'_w = M_w - U, (W, n, m)


def compress_matrix(g: np.ndarray, e: np.ndarray, q_in: np.ndarray,
                    tol: float = DROP_TOL, local_q_error: bool = False,
                    iterations: int = 1) -> MatrixStep:
    """One warm-started compression step with error feedback for one matrix.

    g, e: (W, n, m) gradients and error memories; q_in: (m, r) shared warm start.
    Steps, in the page's order: EF add; P_w = M_w Q; all-reduce P; orthonormalise;
    Q_w = M_w^T P; all-reduce Q; decompress P Q^T; keep the error M_w - P Q^T.
    ``local_q_error`` switches the error to M_w - P Q_w^T (each worker's own Q).
    ``iterations`` > 1 repeats the power-iteration half steps (P, all-reduce,
    orthonormalise, Q, all-reduce) that many times from the previous Q before the
    decompression; the page uses one step per gradient (warm start replaces more).
    """
    g, e = _f64(g), _f64(e)
    W = g.shape[0]
    m_w = [ef_add(g[w], e[w]) for w in range(W)]
    q_cur = _f64(q_in)
    for _ in range(max(1, iterations)):
        p_bar = all_reduce_mean([worker_p(m_w[w], q_cur) for w in range(W)])
        p_hat = orthonormalise(p_bar, tol)
        q_w = [worker_q(m_w[w], p_hat) for w in range(W)]
        q_bar = all_reduce_mean(q_w)
        q_cur = q_bar
    u = decompress(p_hat, q_bar)
    if local_q_error:
        err = np.stack([new_error(m_w[w], decompress(p_hat, q_w[w])) for w in range(W)])
    else:
        err = np.stack([new_error(m_w[w], u) for w in range(W)])
    return MatrixStep(p_bar, p_hat, q_bar, u, err)


def average_tensor(g: np.ndarray) -> np.ndarray:
    """Uncompressed tensor: plain mean over the W workers, no error memory."""
    g = _f64(g)
    return all_reduce_mean([g[w] for w in range(g.shape[0])])


def momentum_sgd(mom: np.ndarray, x: np.ndarray, u: np.ndarray, lr: float, mu: float,
                 nesterov: bool = False):
    """Momentum SGD applied to the decompressed update; returns (mom', x')."""
    mom = mu * _f64(mom) + _f64(u)
    if nesterov:
        x = _f64(x) - lr * (_f64(u) + mu * mom)
    else:
        x = _f64(x) - lr * mom
    return mom, x


# ---------------------------------------------------------------- a whole layer set
@dataclass
class LayerState:
    """Inputs of one tensor for one step. q is None for uncompressed tensors."""

    g: np.ndarray  # (W, rows, cols)
    e: np.ndarray  # (W, rows, cols); ignored for uncompressed tensors
    q: np.ndarray | None  # (cols, r)


def compress_layers(layers: Sequence[LayerState], tol: float = DROP_TOL) -> List[object]:
    """One step over a layer set: MatrixStep for compressed tensors, the mean otherwise."""
    out: List[object] = []
    for ls in layers:
        if ls.q is None:
            out.append(average_tensor(ls.g))
        else:
            out.append(compress_matrix(ls.g, ls.e, ls.q, tol))
    return out
