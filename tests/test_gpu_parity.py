"""GPU parity: the HIP library (through its C ABI) against the CPU oracle, element by
element on the same seeded inputs, at <= 1e-4 relative Frobenius error per matrix (per
worker for the errors); 2e-2 for bf16 gradients against the oracle on the fp32
originals.  Multi-step runs are checked at every step with the oracle fed the GPU's
state before the step."""

import numpy as np
import pytest

from oracle import powersgd_ef as O
from distributed_sgd_gradient_ef_amd import workloads as WL
from tests.gpu_harness import DeviceRun, compare_step, device_layers, log, rel, snapshot

pytestmark = pytest.mark.gpu
TOL = 1e-4


@pytest.fixture(scope="module")
def torch_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU visible")
    from distributed_sgd_gradient_ef_amd import psgd

    psgd.load_library()  # a missing library is an error here, not a skip
    return torch


def _shapes(wl):
    return [s for _, s in wl.shapes]


def _q0_all(wl):
    return {i: WL.q0(wl, i) for i, (_, s) in enumerate(wl.shapes) if WL.is_matrix(s, wl.rank)}


# ----------------------------------------------------------------------- single matrix
def test_single_matrix_ten_steps(torch_gpu):
    """256x128, r=1, W=1, 10 warm-started steps with error feedback."""
    wl = WL.workload("single")
    log(f"[case] single 256x128 r=1 W=1 seed={wl.seed}")
    run = DeviceRun(_shapes(wl), wl.rank, wl.workers)
    run.set_q_host(_q0_all(wl))
    e_free, q_free = np.zeros((1, 256, 128)), WL.q0(wl, 0).astype(np.float64)
    drift = []
    for t in range(wl.steps):
        g = WL.grads(wl, t)
        run.set_grads_host(g)
        snap = snapshot(run, [0])
        run.compress()
        compare_step(run, snap, O, TOL, what=f"step {t}")
        free = O.compress_matrix(g[0], e_free, q_free)
        e_free, q_free = free.errors, free.q_bar
        drift.append(rel(run.errors_layer(0)[0], e_free[0], 1.0))
    log(f"free-running error divergence per step (not gated): {['%.1e' % d for d in drift]}")


@pytest.mark.parametrize("W,r", [(1, 1), (4, 2), (3, 4)])
def test_exact_low_rank_is_reconstructed(torch_gpu, W, r):
    """mean M of rank <= r with a generic Q: U = mean M and the errors average to zero."""
    log(f"[case] exactness W={W} r={r}")
    rng = np.random.default_rng(20 + W)
    n, m = 200, 150
    low = (rng.standard_normal((n, r)) @ rng.standard_normal((r, m))).astype(np.float32)
    dev = rng.standard_normal((W, n, m)).astype(np.float32)
    dev -= dev.mean(axis=0, keepdims=True)
    run = DeviceRun([(n, m)], r, W)
    run.set_grads_host([low[None] + dev])
    run.set_q_host({0: rng.standard_normal((m, r)).astype(np.float32)})
    run.compress()
    U = run.layer(run.host(run.update), 0)
    E = run.errors_layer(0)
    scale = np.linalg.norm(low)
    assert np.linalg.norm(U - low) <= 1e-5 * scale
    assert np.linalg.norm(E.astype(np.float64).mean(axis=0)) <= 1e-5 * scale
    P = run.p_layer(0).astype(np.float64)
    assert np.abs(P.T @ P - np.eye(r)).max() < 1e-5


def test_dependent_column_dropped(torch_gpu):
    """rank-1 matrix at r=2: the second column of P is zero, U = M, nothing is NaN."""
    log("[case] drop rule rank-1 at r=2")
    rng = np.random.default_rng(5)
    M = np.outer(rng.standard_normal(96), rng.standard_normal(80)).astype(np.float32)
    run = DeviceRun([(96, 80)], 2, 1)
    run.set_grads_host([M[None]])
    run.set_q_host({0: rng.standard_normal((80, 2)).astype(np.float32)})
    run.compress()
    P = run.p_layer(0)
    assert np.all(P[:, 1] == 0.0) and np.all(np.isfinite(P))
    U = run.layer(run.host(run.update), 0)
    assert np.linalg.norm(U - M) <= 1e-5 * np.linalg.norm(M)


def test_zero_gradients(torch_gpu):
    log("[case] zero gradients")
    run = DeviceRun([(64, 48), (1, 7)], 2, 3)
    run.set_q_host({0: np.ones((48, 2), np.float32)})
    run.compress()
    for t in (run.update, run.errors, run.p, run.q):
        assert torch_gpu.all(t == 0).item()


# ----------------------------------------------------------------------- tiles and tails
RAGGED = [
    # several stream tiles, m % 4 != 0, 1-D tensors of odd length, a thin matrix that stays
    # uncompressed, a tall matrix with many row blocks, a 1x1 tensor
    [(37, 29), (1, 10), (130, 1030), (5, 3), (2000, 66), (1, 1), (300, 2), (17, 4096)],
    [(1, 3), (64, 27), (9, 9), (4100, 5), (1, 4097), (256, 2304)],
]


@pytest.mark.parametrize("shapes", RAGGED, ids=["set0", "set1"])
@pytest.mark.parametrize("W,r", [(1, 1), (3, 2), (16, 3), (5, 4)])
def test_ragged_layer_sets(torch_gpu, shapes, W, r):
    log(f"[case] ragged shapes={shapes} W={W} r={r}")
    rng = np.random.default_rng(hash((len(shapes), W, r)) % 2**32)
    run = DeviceRun(shapes, r, W)
    g = [rng.standard_normal((W,) + s).astype(np.float32) for s in shapes]
    e = [0.3 * rng.standard_normal((W,) + s).astype(np.float32) for s in shapes]
    run.set_grads_host(g)
    run.set_errors_host(e)
    qs = {i: rng.standard_normal((s[1], r)).astype(np.float32)
          for i, s in enumerate(shapes) if WL.is_matrix(s, r)}
    run.set_q_host(qs)
    for step in range(2):
        snap = snapshot(run, range(len(shapes)))
        run.compress()
        compare_step(run, snap, O, TOL, what=f"step {step}")
        run.set_grads_host([rng.standard_normal((W,) + s).astype(np.float32) for s in shapes])


def test_padding_and_uncompressed_errors_untouched(torch_gpu):
    """Padding between tensors and the error slots of uncompressed tensors are neither
    read into results nor written."""
    log("[case] padding sentinel")
    shapes = [(37, 29), (1, 10), (70, 33)]
    run = DeviceRun(shapes, 2, 3)
    rng = np.random.default_rng(3)
    run.set_grads_host([rng.standard_normal((3,) + s).astype(np.float32) for s in shapes])
    run.set_q_host({0: rng.standard_normal((29, 2)).astype(np.float32),
                    2: rng.standard_normal((33, 2)).astype(np.float32)})
    nan = float("nan")
    mask = torch_gpu.ones(run.ld, dtype=torch_gpu.bool, device=run.dev)
    for L in run.plan.layers:
        if L.compressed:
            mask[L.offset:L.offset + L.rows * L.cols] = False
    upd_mask = torch_gpu.ones(run.ld, dtype=torch_gpu.bool, device=run.dev)
    for L in run.plan.layers:
        upd_mask[L.offset:L.offset + L.rows * L.cols] = False
    run.errors[:, mask] = nan
    run.update[upd_mask] = 12345.0
    run.compress()
    torch_gpu.cuda.synchronize()
    assert torch_gpu.isnan(run.errors[:, mask]).all().item()
    assert (run.update[upd_mask] == 12345.0).all().item()
    assert torch_gpu.isfinite(run.errors[:, ~mask]).all().item()


def test_update_null_and_side_stream(torch_gpu):
    log("[case] update=NULL on a side stream")
    shapes = [(120, 80), (1, 9)]
    run = DeviceRun(shapes, 2, 2)
    rng = np.random.default_rng(9)
    run.set_grads_host([rng.standard_normal((2,) + s).astype(np.float32) for s in shapes])
    run.set_q_host({0: rng.standard_normal((80, 2)).astype(np.float32)})
    run.update.fill_(7.0)
    s = torch_gpu.cuda.Stream()
    s.wait_stream(torch_gpu.cuda.current_stream())
    with torch_gpu.cuda.stream(s):
        run.compress(update=False, stream=s)
    s.synchronize()
    assert (run.update == 7.0).all().item()
    assert torch_gpu.isfinite(run.errors).all().item()


def test_stream_copy(torch_gpu):
    from distributed_sgd_gradient_ef_amd import psgd

    log("[case] stream copy")
    src = torch_gpu.randn(1 << 20, device="cuda:0")
    dst = torch_gpu.zeros_like(src)
    psgd.psgd_stream_copy(src, dst, 4 * src.numel())
    torch_gpu.cuda.synchronize()
    assert torch_gpu.equal(src, dst)


def test_deterministic(torch_gpu):
    """Same inputs twice give bitwise identical outputs (fixed-order reductions)."""
    log("[case] determinism")
    shapes = [(512, 2304), (64, 27), (1, 64), (10, 512)]
    rng = np.random.default_rng(11)
    g = [rng.standard_normal((16,) + s).astype(np.float32) for s in shapes]
    q = {i: rng.standard_normal((s[1], 2)).astype(np.float32) for i, s in enumerate(shapes) if WL.is_matrix(s, 2)}
    outs = []
    for _ in range(2):
        run = DeviceRun(shapes, 2, 16)
        run.set_grads_host(g)
        run.set_q_host(q)
        run.compress()
        outs.append([run.host(t).copy() for t in (run.errors, run.update, run.p, run.q)])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ----------------------------------------------------------------------- carried error mean
CARRY_SHAPES = [(64, 27), (1, 64), (128, 576), (512, 4608), (37, 29), (1, 10), (10, 512)]


@pytest.mark.parametrize("W,r", [(16, 2), (5, 3)])
def test_carry_error_mean_each_step(torch_gpu, W, r):
    """With the carried error mean the first pass reads only the gradients; every step
    still matches the oracle run on the errors actually stored on the GPU."""
    from distributed_sgd_gradient_ef_amd import psgd

    log(f"[case] carry W={W} r={r}")
    rng = np.random.default_rng(31 + W)
    run = DeviceRun(CARRY_SHAPES, r, W, flags=psgd.PSGD_FLAG_CARRY_ERROR_MEAN)
    run.set_q_host({i: rng.standard_normal((s[1], r)).astype(np.float32)
                    for i, s in enumerate(CARRY_SHAPES) if WL.is_matrix(s, r)})
    for t in range(4):
        run.set_grads_host([rng.standard_normal((W,) + s).astype(np.float32) for s in CARRY_SHAPES])
        snap = snapshot(run, range(len(CARRY_SHAPES)))
        run.compress()
        compare_step(run, snap, O, TOL, what=f"carry step {t}")


def test_carry_is_used_and_reset_restores_exactness(torch_gpu):
    """Writing the errors behind the plan's back makes the carried mean stale (which
    shows the carry path is live); psgd_plan_reset_carry makes the next step exact."""
    from distributed_sgd_gradient_ef_amd import psgd

    log("[case] carry reset")
    shapes = [(256, 1152), (1, 64)]
    W, r = 4, 2
    rng = np.random.default_rng(8)
    run = DeviceRun(shapes, r, W, flags=psgd.PSGD_FLAG_CARRY_ERROR_MEAN)
    run.set_q_host({0: rng.standard_normal((1152, r)).astype(np.float32)})
    g = [rng.standard_normal((W,) + s).astype(np.float32) for s in shapes]
    run.set_grads_host(g)
    run.compress()
    run.set_errors_host([np.zeros((W,) + s, np.float32) for s in shapes])  # behind the plan's back
    snap = snapshot(run, [0])
    run.compress()
    with pytest.raises(AssertionError):
        compare_step(run, snap, O, TOL, what="stale carry")
    run.set_errors_host([np.zeros((W,) + s, np.float32) for s in shapes])
    psgd.psgd_plan_reset_carry(run.plan)
    snap = snapshot(run, [0, 1])
    run.compress()
    compare_step(run, snap, O, TOL, what="after reset")
    # a different workspace buffer also falls back to a full read
    run.set_errors_host([np.zeros((W,) + s, np.float32) for s in shapes])
    run.workspace = run.torch.empty_like(run.workspace)
    snap = snapshot(run, [0, 1])
    run.compress()
    compare_step(run, snap, O, TOL, what="new workspace")


# ----------------------------------------------------------------------- deferred error
@pytest.mark.parametrize("W,r", [(16, 2), (5, 3), (4, 4)])
def test_deferred_error_each_step(torch_gpu, W, r):
    """Deferred mode: the error buffer keeps M_w and the subtraction of U moves into the
    next step.  The materialised errors, P, Q and U match the oracle at every step."""
    from distributed_sgd_gradient_ef_amd import psgd

    log(f"[case] deferred W={W} r={r}")
    rng = np.random.default_rng(41 + W)
    run = DeviceRun(CARRY_SHAPES, r, W, flags=psgd.PSGD_FLAG_DEFERRED_ERROR)
    run.set_q_host({i: rng.standard_normal((s[1], r)).astype(np.float32)
                    for i, s in enumerate(CARRY_SHAPES) if WL.is_matrix(s, r)})
    run.set_errors_host([0.2 * rng.standard_normal((W,) + s).astype(np.float32) for s in CARRY_SHAPES])
    for t in range(4):
        run.set_grads_host([rng.standard_normal((W,) + s).astype(np.float32) for s in CARRY_SHAPES])
        before = run.plain_errors()
        snap = snapshot(run, range(len(CARRY_SHAPES)), errors_source=before)
        run.compress()
        after = run.plain_errors()
        worst = compare_step(run, snap, O, TOL, what=f"deferred step {t}", errors_source=after)
        log(f"step {t} worst rel: " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()))


def test_deferred_materialize_in_place_and_reset(torch_gpu):
    """In-place materialisation turns the buffer plain (the next step subtracts nothing
    more); psgd_plan_reset_carry declares externally written errors plain."""
    from distributed_sgd_gradient_ef_amd import psgd

    log("[case] deferred materialize in place")
    shapes = [(300, 700), (1, 33), (64, 27), (90, 518)]  # 518 columns: the 2-wide row path
    W, r = 3, 2
    rng = np.random.default_rng(17)
    run = DeviceRun(shapes, r, W, flags=psgd.PSGD_FLAG_DEFERRED_ERROR)
    run.set_q_host({0: rng.standard_normal((700, r)).astype(np.float32),
                    2: rng.standard_normal((27, r)).astype(np.float32)})
    run.set_grads_host([rng.standard_normal((W,) + s).astype(np.float32) for s in shapes])
    run.compress()
    psgd.psgd_errors_materialize(run.plan, run.errors, run.errors, run.workspace)
    snap = snapshot(run, [0, 1, 2])  # plain now
    run.compress()
    compare_step(run, snap, O, TOL, what="after in-place materialise", errors_source=run.plain_errors())
    run.set_errors_host([0.5 * rng.standard_normal((W,) + s).astype(np.float32) for s in shapes])
    psgd.psgd_plan_reset_carry(run.plan)
    snap = snapshot(run, [0, 1, 2])
    run.compress()
    compare_step(run, snap, O, TOL, what="after reset", errors_source=run.plain_errors())


def test_deferred_momentum_matches_eager(torch_gpu):
    """Momentum SGD in deferred mode gives the eager mode's update, momentum and
    parameters (to float rounding) over 20 steps, with update=NULL in deferred mode."""
    from distributed_sgd_gradient_ef_amd import psgd

    log("[case] deferred momentum vs eager")
    shapes = [(128, 576), (1, 128), (512, 256), (70, 130)]
    W, r = 16, 4
    rng = np.random.default_rng(23)
    q0 = {0: rng.standard_normal((576, r)).astype(np.float32), 2: rng.standard_normal((256, r)).astype(np.float32)}
    x0 = [0.01 * rng.standard_normal(s).astype(np.float32) for s in shapes]
    runs = []
    for flags in (0, psgd.PSGD_FLAG_DEFERRED_ERROR):
        run = DeviceRun(shapes, r, W, flags=flags, momentum=True)
        run.set_q_host(q0)
        run.set_params_host(x0)
        runs.append(run)
    for t in range(20):
        g = [rng.standard_normal((W,) + s).astype(np.float32) for s in shapes]
        for k, run in enumerate(runs):
            run.set_grads_host(g)
            run.momentum_step(0.1, 0.9, update=(k == 0))
    eager, defer = runs
    torch_gpu.cuda.synchronize()
    for name in ("params", "momentum"):
        a, b = getattr(eager, name), getattr(defer, name)
        err = ((a - b).norm() / a.norm()).item()
        assert err < TOL, (name, err)
    e_plain = defer.plain_errors()
    err = ((eager.errors - e_plain).norm() / eager.errors.norm()).item()
    assert err < TOL, err


# ----------------------------------------------------------------------- warm-start ablation
@pytest.mark.parametrize("iters", [2, 3])
@pytest.mark.parametrize("mode", ["plain", "deferred"])
def test_power_iterations_match_oracle(torch_gpu, mode, iters):
    """k power iterations per step (psgd_plan_set_power_iterations) against the oracle
    run with the same k, at every step."""
    from distributed_sgd_gradient_ef_amd import psgd

    log(f"[case] power iterations k={iters} mode={mode}")
    shapes = [(200, 96), (1, 17), (64, 27), (300, 1030), (5000, 22)]  # tall: two-pass Gram-Schmidt
    W, r = 4, 2
    rng = np.random.default_rng(70 + iters)
    flags = psgd.PSGD_FLAG_DEFERRED_ERROR if mode == "deferred" else 0
    run = DeviceRun(shapes, r, W, flags=flags)
    psgd.psgd_plan_set_power_iterations(run.plan, iters)
    run.set_q_host({i: rng.standard_normal((s[1], r)).astype(np.float32)
                    for i, s in enumerate(shapes) if WL.is_matrix(s, r)})
    for t in range(3):
        run.set_grads_host([rng.standard_normal((W,) + s).astype(np.float32) for s in shapes])
        before = run.plain_errors()
        snap = snapshot(run, range(len(shapes)), errors_source=before)
        run.compress()
        compare_step(run, snap, O, TOL, what=f"k={iters} step {t}", errors_source=run.plain_errors(),
                     iterations=iters)


def _svd_gap(mbar, u, r):
    s = np.linalg.svd(mbar, compute_uv=False)
    best = np.sqrt((s[r:] ** 2).sum())
    return (np.linalg.norm(mbar - u) - best) / best


def test_warm_start_ablation_gap_to_svd(torch_gpu):
    """The page's RQ3 (how the warm start of the power iteration affects the
    approximation over time) on the single-matrix workload at r=2: 256x128, planted
    spectrum 10*0.7^i plus 0.01*N(0,1) noise redrawn each step.  Per step, the relative
    gap of ||Mbar - U|| above the SVD-optimal rank-2 error, for a warm start, a fresh
    N(0,1) Q every step (cold) and two iterations per step.  With the error memory
    cleared every step the best subspace is stable and the warm start must close the
    gap (cold must not); with error feedback on, the dropped directions are added back
    each step and the gaps are only logged."""
    from distributed_sgd_gradient_ef_amd import psgd

    log("[case] warm-start ablation")
    wl = WL.workload("single", rank=2)
    results = {}
    for ef in (False, True):
        runs = {}
        for name, iters in (("warm", 1), ("cold", 1), ("warm_k2", 2)):
            run = DeviceRun(_shapes(wl), wl.rank, wl.workers)
            psgd.psgd_plan_set_power_iterations(run.plan, iters)
            run.set_q_host(_q0_all(wl))
            runs[name] = run
        rng = np.random.default_rng(99)
        gaps = {k: [] for k in runs}
        for t in range(wl.steps):
            g = WL.grads(wl, t)
            for name, run in runs.items():
                if name == "cold":
                    run.set_q_host({0: rng.standard_normal((128, wl.rank)).astype(np.float32)})
                if not ef:
                    run.errors.zero_()
                run.set_grads_host(g)
                mbar = (run.grads_layer(0).astype(np.float64) + run.errors_layer(0)).mean(axis=0)
                run.compress()
                gaps[name].append(_svd_gap(mbar, run.layer(run.host(run.update), 0), wl.rank))
        for name, v in gaps.items():
            log(f"gap to SVD optimum ({'EF on' if ef else 'no EF'}), {name}: " + " ".join(f"{x:.2e}" for x in v))
        results[ef] = {k: np.array(v) for k, v in gaps.items()}
    warm, cold, k2 = (results[False][k] for k in ("warm", "cold", "warm_k2"))
    assert warm[-1] < 1e-2 * warm[0] and warm[-1] < 1e-3
    assert np.median(cold) > 100 * warm[-1]
    assert k2[-1] <= warm[-1] * 1.5 + 1e-6


# ----------------------------------------------------------------------- more edge cases
@pytest.mark.parametrize("mode", ["carry", "deferred"])
@pytest.mark.parametrize("W", [4, 3])
def test_bf16_in_cross_step_modes(torch_gpu, mode, W):
    """bf16 gradients with the carried mean or the deferred error (W=3 takes the generic
    worker loop): every step matches the oracle run on the bf16 values the GPU read."""
    from distributed_sgd_gradient_ef_amd import psgd

    log(f"[case] bf16 {mode} W={W}")
    shapes = [(130, 520), (1, 33), (64, 27), (96, 1024), (40, 262)]
    r = 2
    rng = np.random.default_rng(5 + W)
    flags = psgd.PSGD_FLAG_DEFERRED_ERROR if mode == "deferred" else psgd.PSGD_FLAG_CARRY_ERROR_MEAN
    run = DeviceRun(shapes, r, W, bf16=True, flags=flags)
    run.set_q_host({i: rng.standard_normal((s[1], r)).astype(np.float32)
                    for i, s in enumerate(shapes) if WL.is_matrix(s, r)})
    for t in range(3):
        run.set_grads_host([WL.to_bf16_values(rng.standard_normal((W,) + s).astype(np.float32)) for s in shapes])
        before = run.plain_errors()
        snap = snapshot(run, range(len(shapes)), errors_source=before)
        run.compress()
        compare_step(run, snap, O, TOL, what=f"bf16 {mode} step {t}", errors_source=run.plain_errors())


# Row counts that are not multiples of 2 or 4 end a multi-row first-pass wave early; the
# set also has a 2-wide row (518 columns), a 1-wide row (29 columns), a flat matrix (66
# columns), a matrix over one 256-column strip and 1-D tensors.
MULTIROW_SHAPES = [(37, 29), (1, 10), (130, 518), (17, 1024), (203, 66), (6, 300), (1, 7)]


@pytest.mark.parametrize("mode", ["plain", "carry", "deferred"])
@pytest.mark.parametrize("W,bf16", [(1, False), (2, False), (4, False), (4, True), (2, True)])
def test_multi_row_first_pass(torch_gpu, mode, W, bf16):
    """Worker counts 1, 2 and 4 run the first pass over several rows per wave: every
    first-pass form matches the oracle at every step (bf16: on the values the GPU read)."""
    from distributed_sgd_gradient_ef_amd import psgd

    log(f"[case] multi-row first pass mode={mode} W={W} bf16={bf16}")
    shapes = MULTIROW_SHAPES
    r = 2
    rng = np.random.default_rng(61 + 7 * W + bf16)
    flags = {"plain": 0, "carry": psgd.PSGD_FLAG_CARRY_ERROR_MEAN, "deferred": psgd.PSGD_FLAG_DEFERRED_ERROR}[mode]
    run = DeviceRun(shapes, r, W, bf16=bf16, flags=flags)
    run.set_q_host({i: rng.standard_normal((s[1], r)).astype(np.float32)
                    for i, s in enumerate(shapes) if WL.is_matrix(s, r)})
    run.set_errors_host([0.2 * rng.standard_normal((W,) + s).astype(np.float32) for s in shapes])
    for t in range(3):
        g = [rng.standard_normal((W,) + s).astype(np.float32) for s in shapes]
        run.set_grads_host([WL.to_bf16_values(x) for x in g] if bf16 else g)
        before = run.plain_errors()
        snap = snapshot(run, range(len(shapes)), errors_source=before)
        run.compress()
        compare_step(run, snap, O, TOL, what=f"multi-row {mode} W={W} step {t}", errors_source=run.plain_errors())


@pytest.mark.parametrize("mode", ["plain", "deferred"])
def test_nesterov_and_update_null(torch_gpu, mode):
    """Nesterov momentum against the oracle's closed step, and a run with update=NULL
    giving bitwise the same momentum and parameters."""
    from distributed_sgd_gradient_ef_amd import psgd

    log(f"[case] nesterov {mode}")
    shapes = [(128, 576), (1, 64), (10, 512)]
    W, r, lr, mu = 4, 2, 0.05, 0.9
    rng = np.random.default_rng(61)
    flags = psgd.PSGD_FLAG_NESTEROV | (psgd.PSGD_FLAG_DEFERRED_ERROR if mode == "deferred" else 0)
    q0 = {i: rng.standard_normal((s[1], r)).astype(np.float32) for i, s in enumerate(shapes) if WL.is_matrix(s, r)}
    x0 = [0.01 * rng.standard_normal(s).astype(np.float32) for s in shapes]
    a = DeviceRun(shapes, r, W, flags=flags, momentum=True)
    b = DeviceRun(shapes, r, W, flags=flags, momentum=True)
    for run in (a, b):
        run.set_q_host(q0)
        run.set_params_host(x0)
    for t in range(5):
        g = [rng.standard_normal((W,) + s).astype(np.float32) for s in shapes]
        a.set_grads_host(g)
        b.set_grads_host(g)
        mom0 = {li: a.vec_layer(a.momentum, li).astype(np.float64) for li in range(len(shapes))}
        xx0 = {li: a.vec_layer(a.params, li).astype(np.float64) for li in range(len(shapes))}
        a.momentum_step(lr, mu, update=True)
        b.momentum_step(lr, mu, update=False)
        upd = a.host(a.update)
        for li in range(len(shapes)):
            u = a.layer(upd, li).astype(np.float64)
            m_ref, x_ref = O.momentum_sgd(mom0[li], xx0[li], u, lr, mu, nesterov=True)
            sc = np.linalg.norm(xx0[li]) + np.linalg.norm(u)
            assert rel(a.vec_layer(a.momentum, li), m_ref, sc) <= TOL
            assert rel(a.vec_layer(a.params, li), x_ref, sc) <= TOL
    torch_gpu.cuda.synchronize()
    assert torch_gpu.equal(a.params, b.params) and torch_gpu.equal(a.momentum, b.momentum)


def test_vectors_only_plan_accepts_null_factors(torch_gpu):
    """A plan with no compressed matrix: errors, q and p may be NULL; the update is the
    worker mean."""
    from distributed_sgd_gradient_ef_amd import psgd

    log("[case] vectors only")
    shapes = [(1, 100), (5, 3), (2, 2)]  # (5,3) and (2,2) stay uncompressed at r=4
    W = 6
    plan = psgd.psgd_plan_create(shapes, 4, W)
    assert plan.sizes["n_matrices"] == 0
    rng = np.random.default_rng(2)
    g = [rng.standard_normal((W,) + s).astype(np.float32) for s in shapes]
    dev = "cuda:0"
    grads = torch_gpu.from_numpy(psgd.pack(plan, g)).to(dev)
    update = torch_gpu.zeros(plan.sizes["worker_stride"], device=dev)
    ws = torch_gpu.empty(plan.sizes["workspace_bytes"], dtype=torch_gpu.uint8, device=dev)
    psgd.psgd_compress_step(plan, grads, None, None, None, update, ws)
    torch_gpu.cuda.synchronize()
    u = update.cpu().numpy()
    for li, a in enumerate(g):
        assert rel(psgd.unpack(plan, u, li), O.average_tensor(a), 1.0) <= 1e-6


def test_nonfinite_input_propagates_like_the_oracle(torch_gpu):
    """A NaN in one worker's gradient: the GPU's NaN pattern in P, Q, U and E' is the
    oracle's, and the finite entries still match."""
    log("[case] NaN propagation")
    shapes = [(48, 40)]
    W, r = 2, 2
    rng = np.random.default_rng(77)
    g = rng.standard_normal((W, 48, 40)).astype(np.float32)
    g[1, 5, 7] = np.nan
    q = rng.standard_normal((40, r)).astype(np.float32)
    run = DeviceRun(shapes, r, W)
    run.set_grads_host([g])
    run.set_q_host({0: q})
    run.compress()
    ref = O.compress_matrix(g, np.zeros_like(g), q)
    got = {"p": run.p_layer(0), "q": run.q_layer(0), "u": run.layer(run.host(run.update), 0),
           "e": run.errors_layer(0)}
    want = {"p": ref.p_hat, "q": ref.q_bar, "u": ref.update, "e": ref.errors}
    for k in got:
        assert np.array_equal(np.isnan(got[k]), np.isnan(want[k])), k
        fin = np.isfinite(want[k])
        if fin.any():
            assert np.allclose(got[k][fin], want[k][fin], rtol=1e-4, atol=1e-5), k


# ----------------------------------------------------------------------- workloads
def test_resnet18_three_steps(torch_gpu):
    """ResNet-18 shapes, r=2, W=16, three steps with fresh worker noise, every tensor."""
    wl = WL.workload("resnet18")
    log(f"[case] resnet18 r=2 W=16 seed={wl.seed}")
    run = DeviceRun(_shapes(wl), wl.rank, wl.workers)
    run.set_q_host(_q0_all(wl))
    for t in range(wl.steps):
        run.set_grads_host(WL.grads(wl, t))
        snap = snapshot(run, range(len(wl.shapes)))
        run.compress()
        worst = compare_step(run, snap, O, TOL, what=f"step {t}")
        log(f"step {t} worst rel: " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()))


def test_lstm_two_steps(torch_gpu):
    """LSTM shapes (tied 33278x650 embedding with 5% nonzero rows, 6 x 2600x650), r=4, W=8."""
    wl = WL.workload("lstm")
    log(f"[case] lstm r=4 W=8 seed={wl.seed}")
    run = DeviceRun(_shapes(wl), wl.rank, wl.workers)
    run.set_q_host(_q0_all(wl))
    for t in range(2):
        WL.device_grads(wl, t, device_layers(run), run.grads)
        snap = snapshot(run, range(len(wl.shapes)))
        run.compress()
        worst = compare_step(run, snap, O, TOL, what=f"step {t}")
        log(f"step {t} worst rel: " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()))


STRESS_SAMPLE = [0, 1, 64]  # two 4096^2 and one 8192^2 matrix, every worker


@pytest.mark.parametrize("r", [1, 2, 4])
@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_stress_full_size_sampled(torch_gpu, r, bf16):
    """64 x 4096^2 + 8 x 8192^2, W=4, at full size on the GPU; the oracle checks a fixed
    sample of whole matrices (every matrix is compressed on its own), the rest is
    checked through the identity M = U + E' and P's orthonormality."""
    wl = WL.workload("stress", rank=r)
    log(f"[case] stress r={r} W=4 bf16={bf16} seed={wl.seed}")
    run = DeviceRun(_shapes(wl), r, wl.workers, bf16=bf16)
    q0 = _q0_all(wl)
    run.set_q_host(q0)
    f32 = torch_gpu.zeros((run.W, run.ld), dtype=torch_gpu.float32, device=run.dev) if bf16 else run.grads
    WL.device_grads(wl, 0, device_layers(run), f32)
    originals = {li: f32[:, run.plan.layers[li].offset:run.plan.layers[li].offset
                          + run.plan.layers[li].rows * run.plan.layers[li].cols].cpu().numpy()
                 for li in STRESS_SAMPLE}
    if bf16:
        run.grads.copy_(f32.to(torch_gpu.bfloat16))
        del f32
    snap = snapshot(run, STRESS_SAMPLE)
    run.compress()
    worst = compare_step(run, snap, O, TOL, what=f"stress r={r} bf16={bf16}")
    log("vs oracle on the consumed values: " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()))
    if bf16:
        bad = 0.0
        for li in STRESS_SAMPLE:
            L = run.plan.layers[li]
            g = originals[li].reshape(run.W, L.rows, L.cols)
            ref = O.compress_matrix(g, np.zeros_like(g), q0[li])
            mb = np.linalg.norm(g.astype(np.float64).mean(axis=0))
            bad = max(bad, rel(run.vec_layer(run.update, li), ref.update, mb))
        log(f"bf16 vs oracle on the fp32 originals: U rel {bad:.2e}")
        assert bad <= 2e-2
    # whole-set properties: E' + U = G + E (E was zero) for every matrix, P orthonormal
    upd = run.update
    for li, L in enumerate(run.plan.layers):
        n = L.rows * L.cols
        gsl = run.grads[:, L.offset:L.offset + n].float()
        esl = run.errors[:, L.offset:L.offset + n]
        d = (esl + upd[L.offset:L.offset + n][None] - gsl).abs().max().item()
        assert d <= 1e-5 * max(1.0, gsl.abs().max().item()), (li, d)
        P = run.p[L.p_offset:L.p_offset + L.rows * r].view(L.rows, r).double()
        assert (P.T @ P - torch_gpu.eye(r, dtype=torch_gpu.float64, device=run.dev)).abs().max().item() < 1e-5


def test_largest_tensor_sampled(torch_gpu):
    """One tensor of 2^31 - 2^16 elements (the largest a plan accepts is < 2^31), r=1,
    W=1: every output is checked on sampled rows and columns against the oracle's
    per-element definitions, and M = U + E' everywhere."""
    n, m = 32768, 65534
    log(f"[case] largest tensor {n}x{m} r=1 W=1")
    torch = torch_gpu
    run = DeviceRun([(n, m)], 1, 1)
    g = torch.Generator(device=run.dev)
    g.manual_seed(77)
    torch.randn(n * m, generator=g, device=run.dev, out=run.grads[0, : n * m])
    col = torch.randn(m, generator=g, device=run.dev)
    run.grads[0, : n * m].view(n, m).add_(torch.randn(n, 1, generator=g, device=run.dev) * col[None])
    q = np.random.default_rng(4).standard_normal((m, 1)).astype(np.float32)
    run.set_q_host({0: q})
    run.compress()
    torch.cuda.synchronize()
    G = run.grads[0, : n * m].view(n, m)
    E = run.errors[0, : n * m].view(n, m)
    U = run.update[: n * m].view(n, m)
    assert (E + U - G).abs().max().item() <= 1e-5 * G.abs().max().item()
    P = run.p_layer(0).astype(np.float64)[:, 0]
    Q = run.q_layer(0).astype(np.float64)[:, 0]
    assert abs(np.dot(P, P) - 1.0) < 1e-5
    rows = np.random.default_rng(1).choice(n, 16, replace=False)
    cols = np.random.default_rng(2).choice(m, 16, replace=False)
    Gr = G[torch.as_tensor(rows, device=run.dev)].double().cpu().numpy()
    pbar_rows = Gr @ q.astype(np.float64)[:, 0]  # rows of P-bar = M Q
    # P is P-bar / ||P-bar||: ratios of sampled rows must agree
    ratio = pbar_rows / P[rows]
    assert np.abs(ratio / ratio.mean() - 1).max() < 1e-4
    Gc = G[:, torch.as_tensor(cols, device=run.dev)].double().cpu().numpy()
    q_ref = Gc.T @ P  # sampled entries of Q = M^T P
    assert np.abs(q_ref - Q[cols]).max() <= 1e-4 * np.abs(Q).max()
    Us = U[torch.as_tensor(rows, device=run.dev)][:, torch.as_tensor(cols, device=run.dev)].double().cpu().numpy()
    assert np.abs(Us - np.outer(P[rows], Q[cols])).max() <= 1e-5 * np.abs(Us).max()


def test_grid_fallback_past_2_32_threads(torch_gpu):
    """A 69,000,000 x 31 matrix at W=3: over 2^32 worker-pass threads, so k_first and
    k_apply take the 2-D grid.  The worker mean of the new errors plus U equals the mean
    gradient everywhere; P, Q and U are checked on sampled rows (and all 31 columns)
    against the oracle's per-element definitions."""
    n, m, W = 69_000_000, 31, 3
    log(f"[case] 2-D grid fallback {n}x{m} r=1 W={W}")
    torch = torch_gpu
    run = DeviceRun([(n, m)], 1, W)
    g = torch.Generator(device=run.dev)
    g.manual_seed(78)
    col = torch.randn(m, generator=g, device=run.dev)
    for w in range(W):
        torch.randn(n * m, generator=g, device=run.dev, out=run.grads[w, : n * m])
        run.grads[w, : n * m].view(n, m).add_(torch.randn(n, 1, generator=g, device=run.dev) * col[None])
    q = np.random.default_rng(5).standard_normal((m, 1)).astype(np.float32)
    run.set_q_host({0: q})
    run.compress()
    torch.cuda.synchronize()
    Gm = run.grads[:, : n * m].view(W, n, m).mean(0)
    Em = run.errors[:, : n * m].view(W, n, m).mean(0)
    U = run.update[: n * m].view(n, m)
    assert (Em + U - Gm).abs().max().item() <= 1e-5 * Gm.abs().max().item()
    del Em
    P = run.p_layer(0).astype(np.float64)[:, 0]
    Q = run.q_layer(0).astype(np.float64)[:, 0]
    assert abs(np.dot(P, P) - 1.0) < 1e-5
    rows = np.sort(np.random.default_rng(3).choice(n, 64, replace=False))
    ridx = torch.as_tensor(rows, device=run.dev)
    Gr = run.grads[:, : n * m].view(W, n, m)[:, ridx].double().mean(0).cpu().numpy()
    ratio = (Gr @ q.astype(np.float64)[:, 0]) / P[rows]
    assert np.abs(ratio / ratio.mean() - 1).max() < 1e-4
    Pd = torch.as_tensor(P, device=run.dev)
    q_ref = torch.zeros(m, dtype=torch.float64, device=run.dev)  # Q = Mbar^T P, by row chunks
    for r0 in range(0, n, 1 << 23):
        q_ref += Gm[r0:r0 + (1 << 23)].double().T @ Pd[r0:r0 + (1 << 23)]
    q_ref = q_ref.cpu().numpy()
    assert np.abs(q_ref - Q).max() <= 1e-4 * np.abs(Q).max()
    Us = U[ridx].double().cpu().numpy()
    assert np.abs(Us - np.outer(P[rows], Q)).max() <= 1e-5 * np.abs(Us).max()


def test_momentum_200_steps(torch_gpu):
    """EF-SGD with momentum (mu=0.9, lr=0.1) on ResNet-18 shapes, r=4, W=16, drifting
    subspace, 200 steps.  Every step: a fixed sample of tensors against the oracle fed
    the GPU's pre-step state (errors, Q, momentum, params).  Steps 0 and 199: every
    tensor."""
    wl = WL.workload("resnet18_momentum")
    log(f"[case] momentum r=4 W=16 200 steps seed={wl.seed}")
    run = DeviceRun(_shapes(wl), wl.rank, wl.workers, momentum=True)
    run.set_q_host(_q0_all(wl))
    run.set_params_host([WL.params0(wl, i) for i in range(len(wl.shapes))])
    sample = [0, 1, 2, 3, 60, 61]  # conv1, bn1 weight/bias, a 64x576 conv, the FC weight and bias
    every = list(range(len(wl.shapes)))
    worst_all = 0.0
    for t in range(wl.steps):
        WL.device_grads(wl, t, device_layers(run), run.grads)
        layers = every if t in (0, wl.steps - 1) else sample
        snap = snapshot(run, layers)
        mom0 = {li: run.vec_layer(run.momentum, li).astype(np.float64) for li in layers}
        x0 = {li: run.vec_layer(run.params, li).astype(np.float64) for li in layers}
        run.momentum_step(wl.lr, wl.mu)
        worst = compare_step(run, snap, O, TOL, what=f"step {t}")
        upd = run.host(run.update)
        for li in layers:
            u_ref = run.layer(upd, li).astype(np.float64)  # U itself is checked above
            m_ref, x_ref = O.momentum_sgd(mom0[li], x0[li], u_ref, wl.lr, wl.mu)
            sc = np.linalg.norm(x0[li]) + np.linalg.norm(u_ref)
            em = rel(run.vec_layer(run.momentum, li), m_ref, sc)
            ex = rel(run.vec_layer(run.params, li), x_ref, sc)
            assert em <= TOL and ex <= TOL, (t, li, em, ex)
            worst_all = max(worst_all, em, ex)
        if t % 50 == 0 or t == wl.steps - 1:
            log(f"step {t}: worst " + " ".join(f"{k}={v:.2e}" for k, v in worst.items())
                + f" mom/x={worst_all:.2e}")


# ----------------------------------------------------------------------- local-Q error
@pytest.mark.parametrize("W,r,bf16", [(1, 2, False), (3, 1, False), (4, 3, False), (16, 2, False), (5, 4, True)])
def test_local_q_error_matches_oracle(torch_gpu, W, r, bf16):
    """PSGD_FLAG_LOCAL_Q_ERROR: every worker keeps M_w - P Q_w^T with its own Q_w; P, Q-bar
    and U are those of the aggregated-Q step.  Three steps against the oracle's local-Q
    reading, ragged shapes including the 2-wide and tall row paths."""
    from distributed_sgd_gradient_ef_amd import psgd

    log(f"[case] local-Q W={W} r={r} bf16={bf16}")
    shapes = [(37, 29), (1, 10), (130, 1030), (64, 27), (256, 2304), (4100, 6), (1, 65)]
    rng = np.random.default_rng(100 + W * 7 + r)
    run = DeviceRun(shapes, r, W, bf16=bf16, flags=psgd.PSGD_FLAG_LOCAL_Q_ERROR)
    e = [0.3 * rng.standard_normal((W,) + s).astype(np.float32) for s in shapes]
    run.set_errors_host(e)
    qs = {i: rng.standard_normal((s[1], r)).astype(np.float32) for i, s in enumerate(shapes) if WL.is_matrix(s, r)}
    run.set_q_host(qs)
    for step in range(3):
        g = [rng.standard_normal((W,) + s).astype(np.float32) for s in shapes]
        if bf16:
            g = [WL.to_bf16_values(a) for a in g]
        run.set_grads_host(g)
        snap = snapshot(run, range(len(shapes)))
        run.compress()
        compare_step(run, snap, O, TOL, what=f"local-Q step {step}", local_q=True)


# ----------------------------------------------------------------------- flat rows
# Matrices with at least 32 columns that are not a multiple of 32 start their rows
# anywhere in a 128-byte line; the worker passes stream them as flat runs whose lanes
# can straddle two rows.  33x35, 7x1001 and 50x257 end inside a float4; 5000x35 takes
# the two-pass orthonormalisation; 64x64 and 64x27 keep the row-strip tiles.
FLAT_SHAPES = [(33, 35), (1, 40), (7, 1001), (64, 64), (50, 257), (5000, 35), (130, 650), (64, 27)]


@pytest.mark.parametrize("mode", ["plain", "carry", "deferred", "local", "iter2", "bf16", "momentum"])
def test_flat_rows_every_mode(torch_gpu, mode):
    from distributed_sgd_gradient_ef_amd import psgd

    W, r = (4, 2) if mode == "bf16" else (3, 3)
    flags = {"carry": psgd.PSGD_FLAG_CARRY_ERROR_MEAN, "deferred": psgd.PSGD_FLAG_DEFERRED_ERROR,
             "local": psgd.PSGD_FLAG_LOCAL_Q_ERROR, "bf16": psgd.PSGD_FLAG_DEFERRED_ERROR,
             "momentum": psgd.PSGD_FLAG_DEFERRED_ERROR}.get(mode, 0)
    log(f"[case] flat rows mode={mode} W={W} r={r}")
    rng = np.random.default_rng(90 + len(mode))
    run = DeviceRun(FLAT_SHAPES, r, W, bf16=(mode == "bf16"), flags=flags, momentum=(mode == "momentum"))
    iters = 2 if mode == "iter2" else 1
    if iters > 1:
        psgd.psgd_plan_set_power_iterations(run.plan, iters)
    run.set_q_host({i: rng.standard_normal((s[1], r)).astype(np.float32)
                    for i, s in enumerate(FLAT_SHAPES) if WL.is_matrix(s, r)})
    if mode != "carry":  # carry mode must start from the errors it has seen (zero)
        run.set_errors_host([0.3 * rng.standard_normal((W,) + s).astype(np.float32) for s in FLAT_SHAPES])
        psgd.psgd_plan_reset_carry(run.plan)
    for t in range(3):
        g = [rng.standard_normal((W,) + s).astype(np.float32) for s in FLAT_SHAPES]
        if mode == "bf16":
            g = [WL.to_bf16_values(a) for a in g]
        run.set_grads_host(g)
        before = run.plain_errors()
        snap = snapshot(run, range(len(FLAT_SHAPES)), errors_source=before)
        if mode == "momentum":
            run.momentum_step(0.1, 0.9)
        else:
            run.compress()
        compare_step(run, snap, O, TOL, what=f"flat {mode} step {t}", errors_source=run.plain_errors(),
                     iterations=iters, local_q=(mode == "local"))


def test_flat_rows_deterministic_and_update_matches_subtraction(torch_gpu):
    """Two plans stepped from the same state give bit-identical outputs; in deferred mode
    the U written by the update pass is exactly what the next first pass subtracts (the
    materialised errors equal M_w - U bit for bit)."""
    from distributed_sgd_gradient_ef_amd import psgd

    log("[case] flat rows determinism")
    W, r = 4, 2
    rng = np.random.default_rng(77)
    g = [rng.standard_normal((W,) + s).astype(np.float32) for s in FLAT_SHAPES]
    qs = {i: rng.standard_normal((s[1], r)).astype(np.float32) for i, s in enumerate(FLAT_SHAPES) if WL.is_matrix(s, r)}
    outs = []
    for _ in range(2):
        run = DeviceRun(FLAT_SHAPES, r, W, flags=psgd.PSGD_FLAG_DEFERRED_ERROR)
        run.set_q_host(qs)
        run.set_grads_host(g)
        run.compress()
        m = run.host(run.errors).copy()        # M_w (deferred: the buffer holds M_w)
        u = run.host(run.update).copy()
        plain = run.host(run.plain_errors())
        outs.append([m, u, plain, run.host(run.p).copy(), run.host(run.q).copy()])
        for li, L in enumerate(run.plan.layers):
            if L.compressed:
                n = L.rows * L.cols
                seg = slice(L.offset, L.offset + n)
                assert np.array_equal(plain[:, seg], (m[:, seg] - u[None, seg]).astype(np.float32)), li
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_local_q_error_mean_equals_aggregated(torch_gpu):
    """The two error readings differ per worker but share the workers' mean error and
    produce the same P, Q-bar and U (up to float rounding)."""
    from distributed_sgd_gradient_ef_amd import psgd

    log("[case] local-Q vs aggregated-Q")
    shapes = [(200, 96), (1, 17), (300, 1030)]
    W, r = 4, 2
    rng = np.random.default_rng(5)
    g = [rng.standard_normal((W,) + s).astype(np.float32) for s in shapes]
    e = [0.3 * rng.standard_normal((W,) + s).astype(np.float32) for s in shapes]
    qs = {i: rng.standard_normal((s[1], r)).astype(np.float32) for i, s in enumerate(shapes) if WL.is_matrix(s, r)}
    runs = []
    for flags in (0, psgd.PSGD_FLAG_LOCAL_Q_ERROR):
        run = DeviceRun(shapes, r, W, flags=flags)
        run.set_grads_host(g)
        run.set_errors_host(e)
        run.set_q_host(qs)
        run.compress()
        torch_gpu.cuda.synchronize()
        runs.append(run)
    for li in (0, 2):
        a, b = runs[0], runs[1]
        scale = np.abs(a.vec_layer(a.update, li)).max()
        assert np.allclose(a.p_layer(li), b.p_layer(li), atol=1e-6)
        assert np.allclose(a.q_layer(li), b.q_layer(li), atol=1e-5 * scale)
        assert np.allclose(a.vec_layer(a.update, li), b.vec_layer(b.update, li), atol=1e-6 * scale)
        ea, eb = a.errors_layer(li), b.errors_layer(li)
        assert np.allclose(ea.mean(axis=0), eb.mean(axis=0), atol=1e-5 * scale)
        assert not np.allclose(ea, eb, atol=1e-3 * scale)  # per worker they differ
