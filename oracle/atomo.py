"""Plain CPU oracle for one Spectral-ATOMO step (unbiased sparsification of the singular
value decomposition of every layer gradient).

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the benchmark's
CPU-baseline leg may import this module.  The GPU library never calls it and shares no
code with it: the two meet only at the seeded inputs.

What it follows
---------------
The review page "ATOMO: Communication-efficient Learning via Atomic Sparsification"
(Wang, Sievert et al., 2018), section "Proposed method" (提出的方法), its abstract and
its main findings (主要发现):

* a gradient is written as a weighted sum of unit-norm atoms, g = sum_i lambda_i a_i;
* the sparsified gradient keeps atom i with probability p_i and rescales it by 1/p_i,
  g_hat = sum_i (lambda_i t_i / p_i) a_i with independent t_i ~ Bernoulli(p_i), so that
  E[g_hat] = g;
* the probabilities minimise E||g_hat||^2 = sum_i lambda_i^2 / p_i under the budget
  sum_i p_i = s (and 0 <= p_i <= 1), which has a closed form;
* Spectral-ATOMO takes the atoms of a layer's gradient matrix from its singular value
  decomposition: lambda_i = sigma_i and a_i = u_i v_i^T (unit Frobenius norm).

The closed form, derived here from the optimality conditions of that problem: for
every atom that is not kept with certainty, lambda_i^2 / p_i^2 equals one common
multiplier, so p_i = min(1, c |lambda_i|) with c > 0 fixed by the budget.  The atoms
with the largest |lambda| are the ones that saturate at 1; `probabilities` finds them
in order of decreasing |lambda|.

Readings where the page leaves a step open (each the plainest one the rest supports):

* the budget s is per layer matrix (every matrix spends the same expected number of
  atoms).  When s is at least the number of nonzero singular values every nonzero atom
  has p_i = 1 and g_hat = g; atoms with sigma_i = 0 have p_i = 0 and are never sent;
* the Bernoulli draws are inputs: one uniform x_i in [0, 1) per singular value, in
  descending-sigma order, and atom i is sent when x_i < p_i;
* each worker compresses its own gradient (no error feedback: the estimator is
  unbiased) and the update is the workers' mean of their g_hat;
* a sent atom travels as two factors with g_hat = sum_j a_j b_j^T.  The factor whose
  length is min(n, m) is the unit singular vector on that side (the left one when
  n <= m), and the other is the opposite singular vector times sigma_i / p_i;
* tensors that are not matrices with min(n, m) >= 2 (biases, norm scales) are averaged
  over the workers without compression, as in the PowerSGD path.

Pins: tests/test_oracle_atomo.py checks the closed form against a numerical optimiser
and the optimality conditions, unbiasedness and the variance formula by exact
enumeration of all outcomes, the two special cases the page names (with element-wise
atoms the closed form reproduces TernGrad's and 1-bit QSGD's ternary codes), and the
decomposition against closed forms (rank one, diagonal, orthogonal matrices) and exact
invariants (reconstruction, orthonormality, sum of sigma^2 = ||g||_F^2).
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence

import numpy as np


# ------------------------------------------------------------------ the decomposition
def svd_atoms(g: np.ndarray):
    """Spectral atoms of a matrix in float64: g = sum_i sigma[i] * left[:, i] right[i, :]
    with sigma descending and orthonormal left columns and right rows.  Each atom
    left_i right_i^T has unit Frobenius norm."""
    left, sigma, right = np.linalg.svd(np.asarray(g, dtype=np.float64), full_matrices=False)
    return sigma, left, right


# ------------------------------------------------------------------ the probabilities
def probabilities(lam: np.ndarray, s: float) -> np.ndarray:
    """The p that minimises sum_i lam_i^2 / p_i subject to sum_i p_i = s, 0 <= p_i <= 1
    (p_i = 0 exactly where lam_i = 0): p_i = min(1, c |lam_i|).  Atoms are saturated one
    at a time in order of decreasing |lam| while the largest remaining one would get a
    probability above 1; the rest share what is left of the budget in proportion to
    |lam|."""
    if not s > 0:
        raise ValueError("the budget s must be positive")
    a = np.abs(np.asarray(lam, dtype=np.float64))
    order = np.argsort(-a, kind="stable")
    srt = a[order]
    nnz = int(np.count_nonzero(srt))
    p_sorted = np.zeros_like(srt)
    j = 0
    while j < nnz:
        rest = srt[j:nnz].sum()
        c = (s - j) / rest
        if srt[j] * c <= 1.0:
            p_sorted[j:nnz] = srt[j:nnz] * c
            break
        p_sorted[j] = 1.0
        j += 1
    p = np.empty_like(p_sorted)
    p[order] = p_sorted
    return p


def sample(p: np.ndarray, x: np.ndarray) -> np.ndarray:
    """t_i ~ Bernoulli(p_i) from the given uniforms: t_i = (x_i < p_i)."""
    return np.asarray(x, dtype=np.float64) < np.asarray(p, dtype=np.float64)


def expected_square_norm(lam: np.ndarray, p: np.ndarray) -> float:
    """E||g_hat||^2 = sum_i lam_i^2 / p_i for orthonormal atoms (terms with lam_i = 0
    contribute nothing)."""
    lam = np.asarray(lam, dtype=np.float64)
    nz = lam != 0
    return float(np.sum(lam[nz] ** 2 / np.asarray(p, dtype=np.float64)[nz]))


def sparsify(lam: np.ndarray, atoms: Sequence[np.ndarray], p: np.ndarray, t: np.ndarray) -> np.ndarray:
    """g_hat = sum_i (lam_i t_i / p_i) a_i for any indexable sequence of atoms (arrays of
    one shape), in index order; atoms that are not sent are never read."""
    out = np.zeros(np.shape(atoms[0]), dtype=np.float64)
    for i in range(len(lam)):
        if t[i]:
            out += (lam[i] / p[i]) * np.asarray(atoms[i], dtype=np.float64)
    return out


class OuterAtoms:
    """The spectral atoms left[:, i] right[i, :] of a decomposition, each built when read."""

    def __init__(self, left: np.ndarray, right: np.ndarray):
        self.left, self.right = left, right

    def __len__(self) -> int:
        return self.left.shape[1]

    def __getitem__(self, i: int) -> np.ndarray:
        if not 0 <= i < len(self):
            raise IndexError(i)
        return np.outer(self.left[:, i], self.right[i, :])


# ------------------------------------------------------------------ one matrix, one worker
@dataclass
class AtomoMatrix:
    sigma: np.ndarray      # [k] singular values, descending
    prob: np.ndarray       # [k] p_i
    index: np.ndarray      # [count] sent atoms (positions in descending-sigma order), ascending
    a: np.ndarray          # [count, n] left factors
    b: np.ndarray          # [count, m] right factors; estimate = a^T b
    estimate: np.ndarray   # [n, m] g_hat


def compress_matrix(g: np.ndarray, s: float, x: np.ndarray) -> AtomoMatrix:
    """One worker's Spectral-ATOMO message and estimate for one layer matrix g (n x m),
    budget s and uniforms x (one per singular value, min(n, m) of them)."""
    g = np.asarray(g, dtype=np.float64)
    n, m = g.shape
    sigma, left, right = svd_atoms(g)
    p = probabilities(sigma, s)
    t = sample(p, x)
    index = np.flatnonzero(t)
    if n <= m:   # the unit factor is the left singular vector
        a = left[:, index].T.copy()
        b = (sigma[index] / p[index])[:, None] * right[index, :]
    else:        # the unit factor is the right singular vector
        a = (sigma[index] / p[index])[:, None] * left[:, index].T
        b = right[index, :].copy()
    estimate = sparsify(sigma, OuterAtoms(left, right), p, t)
    return AtomoMatrix(sigma, p, index, a, b, estimate)


def is_matrix(shape: Sequence[int]) -> bool:
    """Layer tensors that Spectral-ATOMO compresses: matrices with min(n, m) >= 2."""
    return len(shape) == 2 and min(shape) >= 2


# ------------------------------------------------------------------ a whole step
@dataclass
class AtomoLayer:
    workers: List[AtomoMatrix]   # empty for uncompressed tensors
    update: np.ndarray           # mean over workers of g_hat (or of g for uncompressed tensors)


def compress_layer(g: np.ndarray, s: float, x: np.ndarray) -> AtomoLayer:
    """All W workers of one layer: g is [W, n, m] (or [W, ...] for an uncompressed
    tensor), x is [W, min(n, m)]."""
    g = np.asarray(g, dtype=np.float64)
    W = g.shape[0]
    if not is_matrix(g.shape[1:]):
        return AtomoLayer([], g.mean(axis=0))
    per = [compress_matrix(g[w], s, x[w]) for w in range(W)]
    update = sum(r.estimate for r in per) / W
    return AtomoLayer(per, update)


def compress_layers(grads: Sequence[np.ndarray], s: float, uniforms: Sequence[np.ndarray]) -> List[AtomoLayer]:
    """One Spectral-ATOMO step over every layer; uniforms[l] is [W, min(n, m)] for a
    compressed layer (ignored otherwise)."""
    return [compress_layer(g, s, x) for g, x in zip(grads, uniforms)]
