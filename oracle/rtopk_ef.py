"""Plain CPU oracle for one rTop-k sparsification step with error feedback.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the benchmark's
CPU-baseline leg may import this module.  The GPU library never calls it and shares no
code with it: the two meet only at the seeded inputs.

What it follows
---------------
The review page "rTop-k: A Statistical Estimation Approach to Distributed SGD" (Barnes,
Inan et al., 2020), section "Proposed method" (제안 방법) and the abstract:

* the compressor first restricts attention to the entries of largest magnitude (a
  top-k selection) and then sends a randomly chosen subset of them (a random-k
  selection): the concatenation of the two sparsifiers;
* rTop-k is a compression operator of the kind the error-feedback convergence results
  cover, which is how it is used: the part not sent is kept and added to the next
  gradient.

Notation and readings where the page leaves a step open (each is the plainest reading
the rest of the page supports):

* every tensor (flattened in row-major order) is compressed on its own, with two
  counts per tensor: r, the size of the top set, and k, the size of the random subset
  actually sent (1 <= k <= r <= d).  The page's review text names only "top-k" and "a
  random subset"; r and k are this oracle's names;
* magnitude order is the order of the IEEE-754 bit pattern of |m| read as an unsigned
  integer (that is |m| for every number, with NaN above infinity); equal magnitudes
  are ordered by position, the lower index first;
* the random subset is uniform over the k-subsets of the top set.  Its randomness is an
  input: `ranks`, a permutation of 0..r-1 given to the top set's entries in ascending
  index order; the entries whose rank is below k are sent.  If `ranks` is not a
  permutation, the entries with rank below k are still the ones sent, the first k of
  them in index order, and unused output slots hold index -1 and value 0;
* sent values are the entries of M themselves, not rescaled;
* error feedback: M_w = G_w + E_w in float32 (the precision the selection is decided
  in); the new error is M_w with the sent entries set to zero; the update is the
  workers' mean of their sent (scattered) entries, in float64 here.

Every function here is pinned by tests/test_oracle_rtopk.py: a worked example computed
by hand (tests/golden/rtopk_worked_example.txt), an independent threshold-based
selection, the partition and tie properties on inputs with many ties, exhaustive
enumeration of the random subsets, the compression-operator contraction property and
exact error-feedback identities.  No function is "parity unpinned".
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence

import numpy as np

SIGN_CLEAR = np.uint32(0x7FFFFFFF)


# ------------------------------------------------------------------ one tensor, one worker
def ef_add(g: np.ndarray, e: np.ndarray) -> np.ndarray:
    """M = G + E in float32 (error feedback; the selection is decided on this M)."""
    return np.asarray(g, dtype=np.float32) + np.asarray(e, dtype=np.float32)


def magnitude_key(m: np.ndarray) -> np.ndarray:
    """Unsigned magnitude key: the bit pattern of m with the sign bit cleared."""
    return np.ascontiguousarray(m, dtype=np.float32).view(np.uint32) & SIGN_CLEAR


def top_set(m: np.ndarray, r: int) -> np.ndarray:
    """Indices of the r entries of largest magnitude (lower index first among equal
    magnitudes), returned in ascending index order."""
    m = np.ravel(m)
    key = magnitude_key(m).astype(np.int64)
    order = np.lexsort((np.arange(m.size), -key))  # by key descending, then index
    return np.sort(order[:r])


def random_subset(top: np.ndarray, ranks: np.ndarray, k: int) -> np.ndarray:
    """The entries of the top set (ascending index order) whose rank is below k; at
    most k of them, the first in index order."""
    ranks = np.asarray(ranks, dtype=np.int64)
    return top[ranks < k][:k]


def rtopk(m: np.ndarray, r: int, k: int, ranks: np.ndarray):
    """rTop-k of one tensor: (sent indices padded with -1 to length k, sent values)."""
    m = np.ravel(np.asarray(m, dtype=np.float32))
    if not (1 <= k <= r <= m.size):
        raise ValueError("need 1 <= k <= r <= numel")
    sent = random_subset(top_set(m, r), ranks, k)
    idx = np.full(k, -1, dtype=np.int64)
    val = np.zeros(k, dtype=np.float32)
    idx[: sent.size] = sent
    val[: sent.size] = m[sent]
    return idx, val


def new_error(m: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """E' = M - C(M): M with the sent entries set to zero."""
    e = np.array(np.ravel(m), dtype=np.float32, copy=True)
    e[idx[idx >= 0]] = 0.0
    return e


def scatter_mean(idx_w: Sequence[np.ndarray], val_w: Sequence[np.ndarray], d: int) -> np.ndarray:
    """Update = mean over workers of the sent entries scattered into a dense tensor
    (the all-reduce of the sparse messages), in float64."""
    u = np.zeros(d, dtype=np.float64)
    for idx, val in zip(idx_w, val_w):
        ok = idx >= 0
        u[idx[ok]] += val[ok].astype(np.float64)
    return u / len(idx_w)


@dataclass
class TensorStep:
    index: np.ndarray   # [W, k] sent indices (ascending, -1 padded)
    value: np.ndarray   # [W, k] sent values (float32)
    errors: np.ndarray  # [W, d] new error memory (float32)
    update: np.ndarray  # [d] mean of the scattered messages (float64)
    m: np.ndarray       # [W, d] the EF-added gradients the selection saw (float32)


def compress_tensor(g: np.ndarray, e: np.ndarray, r: int, k: int, ranks: np.ndarray) -> TensorStep:
    """One step for one tensor and W workers.  g, e: [W, d]; ranks: [W, r]."""
    g = np.asarray(g)
    W = g.shape[0]
    m = ef_add(g.reshape(W, -1), np.asarray(e).reshape(W, -1))
    idx = np.empty((W, k), dtype=np.int64)
    val = np.empty((W, k), dtype=np.float32)
    err = np.empty_like(m)
    for w in range(W):
        idx[w], val[w] = rtopk(m[w], r, k, ranks[w])
        err[w] = new_error(m[w], idx[w])
    upd = scatter_mean(list(idx), list(val), m.shape[1])
    return TensorStep(idx, val, err, upd, m)


def compress_layers(grads: Sequence[np.ndarray], errors: Sequence[np.ndarray], tops: Sequence[int],
                    keeps: Sequence[int], ranks: Sequence[np.ndarray]) -> List[TensorStep]:
    """One step over a list of tensors, each compressed on its own (per-tensor counts)."""
    return [compress_tensor(g, e, r, k, rk) for g, e, r, k, rk in zip(grads, errors, tops, keeps, ranks)]
