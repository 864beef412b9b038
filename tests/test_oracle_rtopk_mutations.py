"""Plant mistakes in (a patched copy of) the rTop-k oracle and check that the pins in
test_oracle_rtopk.py catch every one of them.  CPU only; pytest's monkeypatch restores
the real module after each case."""

import numpy as np
import pytest

from oracle import rtopk_ef as O
from tests.test_oracle_rtopk import PINS


def _top_signed(m, r):
    m = np.ravel(np.asarray(m, np.float32)).astype(np.float64)
    order = np.lexsort((np.arange(m.size), -m))
    return np.sort(order[:r])


def _top_high_index_first(m, r):
    key = O.magnitude_key(np.ravel(m)).astype(np.int64)
    order = np.lexsort((-np.arange(key.size), -key))
    return np.sort(order[:r])


def _top_unsorted(m, r):
    key = O.magnitude_key(np.ravel(m)).astype(np.int64)
    return np.lexsort((np.arange(key.size), -key))[:r]


def _ef_add_f64(g, e):
    return np.asarray(g, np.float64) + np.asarray(e, np.float64)


def _rtopk_f64(m, r, k, ranks):
    m = np.ravel(np.asarray(m, np.float64))
    order = np.lexsort((np.arange(m.size), -np.abs(m)))
    sent = O.random_subset(np.sort(order[:r]), ranks, k)
    idx = np.full(k, -1, np.int64)
    val = np.zeros(k, np.float32)
    idx[: sent.size] = sent
    val[: sent.size] = m[sent]
    return idx, val


def _key_with_sign(m):
    return np.ascontiguousarray(m, dtype=np.float32).view(np.uint32)


def _scatter_sum(idx_w, val_w, d):
    u = np.zeros(d)
    for idx, val in zip(idx_w, val_w):
        ok = idx >= 0
        u[idx[ok]] += val[ok]
    return u


def _rescaled_rtopk(m, r, k, ranks):
    m = np.ravel(np.asarray(m, np.float32))
    sent = O.random_subset(O.top_set(m, r), ranks, k)
    idx = np.full(k, -1, np.int64)
    val = np.zeros(k, np.float32)
    idx[: sent.size] = sent
    val[: sent.size] = m[sent] * np.float32(r / k)
    return idx, val


MUTATIONS = {
    "top set by signed value": ("top_set", _top_signed),
    "ties prefer the higher index": ("top_set", _top_high_index_first),
    "top set in selection order, not index order": ("top_set", _top_unsorted),
    "magnitude key keeps the sign bit": ("magnitude_key", _key_with_sign),
    "random subset keeps rank <= k": ("random_subset", lambda top, ranks, k: top[np.asarray(ranks) <= k][:k]),
    "random subset ignores the ranks": ("random_subset", lambda top, ranks, k: top[:k]),
    "random subset keeps the highest ranks": ("random_subset",
                                              lambda top, ranks, k: top[np.asarray(ranks) >= top.size - k][:k]),
    "sent values rescaled by r/k": ("rtopk", _rescaled_rtopk),
    "error keeps the sent entries": ("new_error", lambda m, idx: np.array(np.ravel(m), np.float32)),
    "error zeroes everything": ("new_error", lambda m, idx: np.zeros(np.size(m), np.float32)),
    "update sums instead of averaging": ("scatter_mean", _scatter_sum),
    "ef_add drops the error": ("ef_add", lambda g, e: np.asarray(g, np.float32)),
    "selection decided in float64": [("ef_add", _ef_add_f64), ("rtopk", _rtopk_f64)],
}


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    patches = MUTATIONS[name]
    for attr, fn in patches if isinstance(patches, list) else [patches]:
        monkeypatch.setattr(O, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin(O)
        except Exception:  # an assertion or a shape error both count as caught
            failed.append(pin.__name__)
    assert failed, f"mutation '{name}' passed every pin"
