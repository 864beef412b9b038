"""The Spectral-ATOMO half of the C ABI without a GPU: plan validation, the packed
layout and per-matrix offsets, byte accounting, and argument checks of psgd_atomo_step
that happen before any device call (the fake addresses below are never dereferenced)."""

import math
import os

import numpy as np
import pytest

from distributed_sgd_gradient_ef_amd import psgd
from distributed_sgd_gradient_ef_amd import workloads as WL

pytestmark = pytest.mark.usefixtures("built_library")

SHAPES = [(64, 27), (1, 64), (10, 512), (3, 5), (7, 1), (2, 2)]


def _plan(W=4, budget=2.0, shapes=SHAPES):
    return psgd.psgd_atomo_plan_create(shapes, budget, W)


@pytest.mark.parametrize("budget", [0.0, -1.0, float("nan"), float("inf"), 1e31])
def test_plan_create_rejects_bad_budgets(budget):
    with pytest.raises(psgd.PsgdError) as e:
        _plan(budget=budget)
    assert e.value.status == psgd.PSGD_ERR_INVALID_ARG


def test_plan_create_rejects_bad_arguments():
    lib = psgd.load_library()
    for W in (0, 65536):
        with pytest.raises(psgd.PsgdError) as e:
            _plan(W=W)
        assert e.value.status == psgd.PSGD_ERR_INVALID_ARG
    with pytest.raises(psgd.PsgdError) as e:
        psgd.psgd_atomo_plan_create(SHAPES, 2.0, 2, flags=1)
    assert e.value.status == psgd.PSGD_ERR_UNSUPPORTED
    with pytest.raises(psgd.PsgdError) as e:                        # min(rows, cols) above the maximum
        psgd.psgd_atomo_plan_create([(psgd.PSGD_ATOMO_MAX_K + 1, 2000)], 2.0, 1)
    assert e.value.status == psgd.PSGD_ERR_UNSUPPORTED
    psgd.psgd_atomo_plan_create([(psgd.PSGD_ATOMO_MAX_K, 2000)], 2.0, 1)  # the maximum itself
    with pytest.raises(psgd.PsgdError) as e:
        psgd.psgd_atomo_plan_create([(65536, 32768)], 2.0, 1)       # 2^31 elements
    assert e.value.status == psgd.PSGD_ERR_INVALID_ARG
    with pytest.raises(psgd.PsgdError):
        psgd.psgd_atomo_plan_create([(0, 5)], 2.0, 1)
    assert lib.psgd_atomo_plan_create(None, 1, 2.0, 1, 0, None) == psgd.PSGD_ERR_INVALID_ARG


def test_layout_and_offsets():
    plan = _plan()
    s = plan.sizes
    assert s["n_layers"] == len(SHAPES) and s["n_workers"] == 4 and s["budget"] == 2.0
    assert s["numel"] == sum(r * c for r, c in SHAPES)
    mats = [(r, c) for r, c in SHAPES if min(r, c) >= 2]
    assert s["n_matrices"] == len(mats)
    assert s["sv_total"] == sum(min(r, c) for r, c in mats)
    assert s["atom_total"] == sum(min(r, c) * (r + c) for r, c in mats)
    assert s["worker_stride"] % 64 == 0
    end, sv, at, mi = 0, 0, 0, 0
    for L, (r, c) in zip(plan.layers, SHAPES):
        assert L.offset % 64 == 0 and L.offset >= end
        assert (L.rows, L.cols, L.numel) == (r, c, r * c)
        end = L.offset + L.numel
        if min(r, c) >= 2:
            assert L.compressed == 1 and L.matrix_index == mi and L.k == min(r, c)
            assert L.sv_offset == sv and L.atom_offset == at
            sv += L.k
            at += L.k * (r + c)
            mi += 1
        else:
            assert L.compressed == 0 and L.matrix_index == -1 and L.k == 0
    assert end <= s["worker_stride"]


def test_model_bytes():
    W = 16
    plan = _plan(W=W)
    want = sum((8 * W + 4 if min(r, c) >= 2 else 4 * W + 4) * r * c for r, c in SHAPES)
    assert plan.sizes["model_bytes"] == want


def test_workspace_covers_the_problems():
    """Two k*k float buffers per matrix and worker, plus four k-vectors."""
    W = 3
    plan = _plan(W=W)
    k2 = sum(math.ceil(min(r, c) ** 2 / 64) * 64 for r, c in SHAPES if min(r, c) >= 2)
    assert plan.sizes["workspace_bytes"] >= W * 4 * (2 * k2 + 4 * plan.sizes["sv_total"])


def _args(plan, **over):
    a = dict(grads=0x10000000, uniforms=0x20000000, sigma=0x30000000, prob=0x40000000, index=0x50000000,
             count=0x60000000, atoms=0x70000000, update=0x80000000, workspace=0x90000000)
    a.update(over)
    assert plan.sizes["workspace_bytes"] < 0x10000000
    return a


@pytest.mark.parametrize("bad", [dict(grads=None), dict(uniforms=None), dict(sigma=None), dict(prob=None),
                                 dict(index=None), dict(count=None), dict(atoms=None), dict(workspace=None),
                                 dict(grads=0x10000004), dict(atoms=0x70000008), dict(prob=0x30000000),
                                 dict(update=0x10000010)])
def test_step_rejects_bad_pointers_before_any_device_call(bad):
    lib = psgd.load_library()
    plan = _plan()
    a = _args(plan, **bad)
    st = lib.psgd_atomo_step(plan.handle, a["grads"], a["uniforms"], a["sigma"], a["prob"], a["index"], a["count"],
                             a["atoms"], a["update"], a["workspace"], None)
    assert st == psgd.PSGD_ERR_INVALID_ARG
    assert lib.psgd_last_error()


def test_step_rejects_null_plan():
    lib = psgd.load_library()
    assert lib.psgd_atomo_step(None, 0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 0x7000, None, 0x8000,
                               None) == psgd.PSGD_ERR_INVALID_ARG


def test_timing_calls_without_gpu():
    plan = _plan()
    psgd.psgd_atomo_plan_set_timing(plan, True)
    assert psgd.psgd_atomo_plan_kernel_stats(plan) == {}
    psgd.psgd_atomo_plan_set_timing(plan, False)


def test_pack_sv_and_factor_slices():
    plan = _plan(W=3)
    rng = np.random.default_rng(0)
    per = {li: rng.random((3, L.k)).astype(np.float32) for li, L in enumerate(plan.layers) if L.compressed}
    rows = psgd.pack_sv(plan, per)
    assert rows.shape == (3, plan.sizes["sv_total"])
    for li, a in per.items():
        assert np.array_equal(psgd.sv_slice(plan, rows, li), a)
    atoms = np.arange(3 * plan.sizes["atom_total"], dtype=np.float32).reshape(3, -1)
    count = np.full((3, plan.sizes["n_matrices"]), 2, dtype=np.int32)
    L = plan.layers[0]
    a, b = psgd.atom_factors(plan, atoms, count, 0, 1)
    blk = atoms[1, L.atom_offset:L.atom_offset + 2 * (L.rows + L.cols)].reshape(2, -1)
    assert np.array_equal(a, blk[:, :L.rows]) and np.array_equal(b, blk[:, L.rows:])


def test_workload_plan():
    wl = WL.workload("resnet18_atomo")
    plan = psgd.psgd_atomo_plan_create([s for _, s in wl.shapes], wl.atomo_budget, wl.workers)
    assert plan.sizes["n_matrices"] == 21 and max(L.k for L in plan.layers) == 512
    x = WL.atomo_uniforms(wl, 0, 3, 0, 27)
    assert x.dtype == np.float32 and x.shape == (27,) and np.all((x >= 0) & (x < 1))
