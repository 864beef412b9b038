"""Seeded synthetic workloads for the PowerSGD, rTop-k and Spectral-ATOMO compression steps.

This module only draws inputs (gradients, the initial Q, parameters, the random ranks
that pick rTop-k's subset, the uniforms behind Spectral-ATOMO's Bernoulli draws) and
lists layer shapes.  It holds none of the compression arithmetic, so both the GPU library's tests
and the CPU oracle can consume what it produces.

Every draw comes from a Philox4x32-10 counter-based stream (numpy's ``Philox`` bit
generator) keyed by ``(seed, purpose, step, worker, layer)``, so any single layer of any
worker at any step can be regenerated on its own.

Shapes follow the workloads the PowerSGD review page reports on (section "Main
findings", results table and the bullets under it): CIFAR-10 ResNet-18 and a
Wikitext-2 three-layer LSTM; the remaining two workloads are a single small matrix and
a bandwidth stress set.  Datasets are not used: the gradients are synthetic stand-ins
with a planted low-rank part plus worker noise, as described per workload below.
"""

from __future__ import annotations

import functools
import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

Shape = Tuple[int, int]  # (rows, cols); a 1-D tensor of length d is (1, d)

# purpose tags for the stream keys
_P_FACTOR_U, _P_FACTOR_V, _P_NOISE, _P_Q0, _P_PARAM, _P_ROWS, _P_DRIFT, _P_RANKS, _P_UNIFORM = range(9)


# --------------------------------------------------------------------------- shapes
def resnet18_cifar_shapes() -> List[Tuple[str, Shape]]:
    """Parameter tensors of the CIFAR variant of ResNet-18 (3x3 stem, 10 classes).

    Convolution weights are listed as out_ch x (in_ch*k*k) matrices, the way the
    PowerSGD page says each layer's gradient is reshaped to a matrix (section
    "Proposed method").  Batch-norm weights/biases and the classifier bias are 1-D.
    Order is the usual parameter order of the network.
    """
    out: List[Tuple[str, Shape]] = []

    def conv(name, cout, cin, k):
        out.append((name + ".weight", (cout, cin * k * k)))

    def bn(name, c):
        out.append((name + ".weight", (1, c)))
        out.append((name + ".bias", (1, c)))

    conv("conv1", 64, 3, 3)
    bn("bn1", 64)
    cin = 64
    for stage, cout in enumerate([64, 128, 256, 512], start=1):
        for blk in range(2):
            pre = f"layer{stage}.{blk}"
            stride_change = blk == 0 and cout != cin
            conv(pre + ".conv1", cout, cin, 3)
            bn(pre + ".bn1", cout)
            conv(pre + ".conv2", cout, cout, 3)
            bn(pre + ".bn2", cout)
            if stride_change:
                conv(pre + ".shortcut.0", cout, cin, 1)
                bn(pre + ".shortcut.1", cout)
            cin = cout
    out.append(("linear.weight", (10, 512)))
    out.append(("linear.bias", (1, 10)))
    return out


def lstm_wikitext2_shapes(tied: bool = True) -> List[Tuple[str, Shape]]:
    """Three-layer LSTM language model on a 33,278-word vocabulary, 650 hidden units.

    The embedding and decoder share one 33,278 x 650 matrix when ``tied``; otherwise
    they are two matrices.  Each layer has an input and a recurrent weight of
    (4*650) x 650.  Biases are left out.
    """
    out: List[Tuple[str, Shape]] = [("encoder.weight", (33278, 650))]
    for layer in range(3):
        out.append((f"rnn.weight_ih_l{layer}", (2600, 650)))
        out.append((f"rnn.weight_hh_l{layer}", (2600, 650)))
    if not tied:
        out.append(("decoder.weight", (33278, 650)))
    return out


def stress_shapes() -> List[Tuple[str, Shape]]:
    """64 square 4096x4096 matrices plus 8 square 8192x8192 matrices."""
    out = [(f"sq4096.{i}", (4096, 4096)) for i in range(64)]
    out += [(f"sq8192.{i}", (8192, 8192)) for i in range(8)]
    return out


# --------------------------------------------------------------------------- configs
@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, rank, workers, step count and signal recipe."""

    name: str
    shapes: Tuple[Tuple[str, Shape], ...]
    rank: int
    workers: int
    steps: int
    seed: int
    signal: str  # "single", "resnet", "lstm", "stress"
    grad_dtype: str = "f32"  # "f32" or "bf16"
    drift_rad: float = 0.0  # per-step rotation of the planted subspaces
    lr: float = 0.0
    mu: float = 0.0
    keep_frac: float = 0.01  # rTop-k: entries sent per tensor, as a fraction of its size
    top_factor: int = 2      # rTop-k: top-set size as a multiple of the sent count
    atomo_budget: float = 2.0  # Spectral-ATOMO: expected atoms sent per matrix (sum of p_i)

    @property
    def matrix_shapes(self) -> List[Shape]:
        return [s for _, s in self.shapes if is_matrix(s, self.rank)]

    def numel(self) -> int:
        return sum(r * c for _, (r, c) in self.shapes)


def is_matrix(shape: Shape, rank: int) -> bool:
    """A tensor is compressed when it is 2-D and its smaller side exceeds the rank."""
    r, c = shape
    return r > 1 and c > 1 and min(r, c) > rank


def workload(name: str, **overrides) -> Workload:
    base = {
        # one 256x128 matrix, r=1, one worker, 10 warm-started steps
        "single": dict(name="single", shapes=(("w", (256, 128)),), rank=1, workers=1,
                       steps=10, seed=1001, signal="single"),
        # ResNet-18 (CIFAR) shapes, r=2, 16 simulated workers
        "resnet18": dict(name="resnet18", shapes=tuple(resnet18_cifar_shapes()), rank=2,
                         workers=16, steps=3, seed=1002, signal="resnet"),
        # LSTM language model shapes, r=4, 8 workers
        "lstm": dict(name="lstm", shapes=tuple(lstm_wikitext2_shapes()), rank=4, workers=8,
                     steps=10, seed=1003, signal="lstm"),
        # bandwidth stress, W=4, r in {1,2,4}
        "stress": dict(name="stress", shapes=tuple(stress_shapes()), rank=2, workers=4,
                       steps=2, seed=1004, signal="stress"),
        # rTop-k on ResNet-18 shapes: same gradient recipe, 16 workers, 1% of each
        # tensor sent, drawn from its top 2%
        "resnet18_rtopk": dict(name="resnet18_rtopk", shapes=tuple(resnet18_cifar_shapes()), rank=2,
                               workers=16, steps=3, seed=1006, signal="resnet"),
        # rTop-k on the LSTM shapes (a 5%-row-sparse embedding gradient), 8 workers
        "lstm_rtopk": dict(name="lstm_rtopk", shapes=tuple(lstm_wikitext2_shapes()), rank=4, workers=8,
                           steps=2, seed=1007, signal="lstm"),
        # Spectral-ATOMO on ResNet-18 shapes: same gradient recipe, 16 workers, an
        # expected two atoms per matrix (about PowerSGD rank 2's message size)
        "resnet18_atomo": dict(name="resnet18_atomo", shapes=tuple(resnet18_cifar_shapes()), rank=2,
                               workers=16, steps=3, seed=1008, signal="resnet", atomo_budget=2.0),
        # full EF-SGD with momentum on ResNet-18 shapes, drifting subspace
        "resnet18_momentum": dict(name="resnet18_momentum", shapes=tuple(resnet18_cifar_shapes()),
                                  rank=4, workers=16, steps=200, seed=1005, signal="resnet",
                                  drift_rad=0.02, lr=0.1, mu=0.9),
    }[name]
    base.update(overrides)
    return Workload(**base)


# --------------------------------------------------------------------------- streams
def stream(seed: int, purpose: int, step: int = 0, worker: int = 0, layer: int = 0) -> np.random.Generator:
    """Independent Philox4x32-10 stream for one (seed, purpose, step, worker, layer)."""
    ss = np.random.SeedSequence([seed, purpose, step, worker, layer])
    return np.random.Generator(np.random.Philox(ss))


def haar_orthonormal(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    """n x k matrix with orthonormal columns, Haar distributed (sign-fixed QR of a Gaussian)."""
    a = rng.standard_normal((n, k))
    q, r = np.linalg.qr(a)
    return q * np.sign(np.diag(r))[None, :]


def student_t3(rng: np.random.Generator, size, dtype=np.float32) -> np.ndarray:
    """Student-t with 3 degrees of freedom as Z / sqrt(chi2_3 / 3)."""
    z = rng.standard_normal(size)
    chi2 = rng.standard_normal((3,) + tuple(np.atleast_1d(size)))
    chi2 = (chi2 * chi2).sum(axis=0)
    return (z / np.sqrt(chi2 / 3.0)).astype(dtype)


# --------------------------------------------------------------------------- signals
@dataclass
class Planted:
    """Shared low-rank part U diag(s) V^T of one matrix (identical on every worker)."""

    u: np.ndarray  # n x k, orthonormal columns
    v: np.ndarray  # m x k
    s: np.ndarray  # k

    def dense(self) -> np.ndarray:
        return ((self.u * self.s[None, :]) @ self.v.T).astype(np.float32)


def _spectrum(signal: str, n: int, m: int) -> np.ndarray:
    if signal in ("single", "lstm"):
        k = min(16, n, m)
        return 10.0 * 0.7 ** np.arange(k)
    if signal == "resnet":
        k = min(16, n, m)
        return 0.7 ** np.arange(k)
    if signal == "stress":
        k = min(8, n, m)
        edge = math.sqrt(3.0) * (math.sqrt(n) + math.sqrt(m))
        return 2.0 * edge * 0.7 ** np.arange(k)
    raise ValueError(signal)


@functools.lru_cache(maxsize=4096)
def planted(wl: Workload, layer: int, step: int = 0) -> Optional[Planted]:
    """Planted low-rank part of matrix ``layer`` at ``step`` (None for tensors without one).

    With ``drift_rad`` > 0 the subspaces turn by exactly that angle per step (see
    ``_drift``); step 0 is the undrifted draw.  Results are cached, so walking the steps
    in order costs one rotation per step.
    """
    name, (n, m) = wl.shapes[layer]
    if not is_matrix((n, m), wl.rank):
        return None
    if wl.signal == "lstm" and name.startswith(("encoder", "decoder")):
        return None  # sparse rows instead of a planted part
    s = _spectrum(wl.signal, n, m)
    k = len(s)
    if step == 0 or not wl.drift_rad:
        u = haar_orthonormal(stream(wl.seed, _P_FACTOR_U, 0, 0, layer), n, k)
        v = haar_orthonormal(stream(wl.seed, _P_FACTOR_V, 0, 0, layer), m, k)
        return Planted(u, v, s)
    prev = planted(wl, layer, step - 1)
    u = _drift(prev.u, wl.drift_rad, stream(wl.seed, _P_DRIFT, step, 0, 2 * layer))
    v = _drift(prev.v, wl.drift_rad, stream(wl.seed, _P_DRIFT, step, 0, 2 * layer + 1))
    return Planted(u, v, s)


def _drift(basis: np.ndarray, angle: float, rng: np.random.Generator) -> np.ndarray:
    """Turn span(basis) by ``angle`` radians.

    The rotation acts in the plane of a = basis @ c (c uniform on the unit sphere) and a
    random unit vector b orthogonal to span(basis); every column of basis is rotated,
    so the columns stay orthonormal and the principal angle moved is exactly ``angle``.
    """
    n, k = basis.shape
    c = rng.standard_normal(k)
    c /= np.linalg.norm(c)
    a = basis @ c
    b = rng.standard_normal(n)
    b -= basis @ (basis.T @ b)
    b -= basis @ (basis.T @ b)
    b /= np.linalg.norm(b)
    ca, cb = a @ basis, b @ basis  # (k,) coordinates of each column along a and b
    cos, sin = math.cos(angle), math.sin(angle)
    return (basis + (cos - 1.0) * (np.outer(a, ca) + np.outer(b, cb))
            + sin * (np.outer(b, ca) - np.outer(a, cb)))


def grad_layer(wl: Workload, layer: int, step: int, worker: int,
               low_rank: Optional[np.ndarray] = None) -> np.ndarray:
    """Gradient of one tensor for one worker at one step, float32, shape (rows, cols).

    ``low_rank`` may pass the dense planted part so callers that loop over workers
    build it once.
    """
    _, (n, m) = wl.shapes[layer]
    rng = stream(wl.seed, _P_NOISE, step, worker, layer)
    sig = wl.signal
    if not is_matrix((n, m), wl.rank):
        scale = {"single": 0.01, "resnet": 0.05, "lstm": 0.01, "stress": 1.0}[sig]
        return scale * rng.standard_normal((n, m), dtype=np.float32)
    if low_rank is None:
        p = planted(wl, layer, step)
        low_rank = None if p is None else p.dense()
    if sig == "lstm" and low_rank is None:
        # sparse embedding gradient: 5% of rows nonzero, drawn N(0,1)
        g = np.zeros((n, m), dtype=np.float32)
        k = int(round(0.05 * n))
        rows = rng.choice(n, size=k, replace=False)
        g[rows] = rng.standard_normal((k, m), dtype=np.float32)
        return g
    if sig == "stress":
        noise = student_t3(rng, (n, m))
    else:
        scale = {"single": 0.01, "resnet": 0.05, "lstm": 0.01}[sig]
        noise = scale * rng.standard_normal((n, m), dtype=np.float32)
    return (low_rank + noise).astype(np.float32)


def grads(wl: Workload, step: int, layers: Optional[Sequence[int]] = None) -> List[np.ndarray]:
    """All workers' gradients at ``step``: one (W, rows, cols) float32 array per tensor."""
    if layers is None:
        layers = range(len(wl.shapes))
    out = []
    for li in layers:
        _, (n, m) = wl.shapes[li]
        p = planted(wl, li, step)
        lr = None if p is None else p.dense()
        a = np.empty((wl.workers, n, m), dtype=np.float32)
        for w in range(wl.workers):
            a[w] = grad_layer(wl, li, step, w, lr)
        out.append(a)
    return out


def rtopk_counts(wl: Workload) -> Tuple[List[int], List[int]]:
    """Per-tensor (top, keep) counts: keep = max(1, ceil(keep_frac * numel)) and
    top = min(numel, top_factor * keep)."""
    tops, keeps = [], []
    for _, (n, m) in wl.shapes:
        d = n * m
        k = max(1, int(math.ceil(wl.keep_frac * d)))
        tops.append(min(d, wl.top_factor * k))
        keeps.append(k)
    return tops, keeps


def rtopk_ranks(wl: Workload, step: int, worker: int, layer: int, top: int) -> np.ndarray:
    """Random ranks of one tensor's top set: a uniform permutation of 0..top-1 (uint32)."""
    return stream(wl.seed, _P_RANKS, step, worker, layer).permutation(top).astype(np.uint32)


def atomo_uniforms(wl: Workload, step: int, worker: int, layer: int, k: int) -> np.ndarray:
    """Spectral-ATOMO's Bernoulli draws for one worker's matrix: k uniforms in [0, 1)
    (float32), one per singular value in descending order."""
    return stream(wl.seed, _P_UNIFORM, step, worker, layer).random(k, dtype=np.float32)


def q0(wl: Workload, layer: int) -> np.ndarray:
    """Initial warm-start factor Q0 ~ N(0,1), shape (cols, rank), float32."""
    _, (n, m) = wl.shapes[layer]
    return stream(wl.seed, _P_Q0, 0, 0, layer).standard_normal((m, wl.rank), dtype=np.float32)


def params0(wl: Workload, layer: int) -> np.ndarray:
    """Initial parameters 0.01*N(0,1), shape (rows, cols), float32."""
    _, (n, m) = wl.shapes[layer]
    return 0.01 * stream(wl.seed, _P_PARAM, 0, 0, layer).standard_normal((n, m), dtype=np.float32)


def to_bf16_values(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even) and return the values as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    nan = np.isnan(a)
    out = rounded.astype(np.uint32).view(np.float32).copy()
    out[nan] = np.nan
    return out


def bf16_bits(a_bf16_values: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bfloat16-representable."""
    return (np.ascontiguousarray(a_bf16_values, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------- on device
def device_grads(wl: Workload, step: int, layers, out, low_rank_cache: Optional[dict] = None) -> None:
    """Fill ``out`` (a torch float32 tensor [W, worker_stride] on a ROCm device) with the
    gradients of ``step``, drawn on the device for workloads too large to draw on the
    host.  ``layers`` lists (offset, rows, cols) per tensor in the packed layout.

    Same recipe as ``grad_layer`` (planted part from the host, noise drawn with torch's
    seeded device generator), but not the same bits: tests feed the CPU oracle with the
    values read back from ``out``.
    """
    import torch

    dev = out.device
    W = out.shape[0]
    sig = wl.signal
    for li, (off, n, m) in enumerate(layers):
        numel = n * m
        lr = None
        if is_matrix((n, m), wl.rank):
            p = planted(wl, li, step)
            if p is not None:
                key = (li, step)
                if low_rank_cache is not None and key in low_rank_cache:
                    lr = low_rank_cache[key]
                else:
                    lr = torch.from_numpy(p.dense().reshape(-1)).to(dev)
                    if low_rank_cache is not None and not wl.drift_rad:
                        low_rank_cache[key] = lr
        for w in range(W):
            g = torch.Generator(device=dev)
            g.manual_seed(int(np.random.SeedSequence([wl.seed, _P_NOISE, step, w, li]).generate_state(1)[0]))
            dst = out[w, off:off + numel]
            if sig == "lstm" and lr is None and is_matrix((n, m), wl.rank):
                dst.zero_()
                k = int(round(0.05 * n))
                rows = torch.randperm(n, generator=g, device=dev)[:k]
                vals = torch.randn((k, m), generator=g, device=dev)
                dst.view(n, m)[rows] = vals
                continue
            if sig == "stress" and is_matrix((n, m), wl.rank):
                z = torch.randn(numel, generator=g, device=dev)
                chi = torch.randn((3, numel), generator=g, device=dev).square_().sum(dim=0)
                dst.copy_(z / torch.sqrt(chi / 3.0))
                del z, chi
            else:
                scale = {"single": 0.01, "resnet": 0.05, "lstm": 0.01, "stress": 1.0}[sig]
                torch.randn(numel, generator=g, device=dev, out=dst)
                dst.mul_(scale)
            if lr is not None:
                dst.add_(lr)
