"""Seeded synthetic workloads for the PowerSGD compression step.

This module only *makes data*: layer-shape lists and seeded gradient
generators with the shapes and spectra of the workloads the PowerSGD pages
evaluate on (ResNet18 on CIFAR-10 and a 3-layer LSTM on WikiText-2, from the
"Key results" section of the anthology note on PowerSGD) plus a 7B-transformer
shaped set and a decaying-spectrum matrix for the rank sweep and the PowerSGD+
subspace refresh.  No dataset item is used or reproduced: every value is drawn
from a seeded generator.

It holds none of the method's arithmetic and is shared, unchanged, by the GPU
tests, the benchmark and the oracle tests, so that both sides see the very same
fp32 inputs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

Shape = Tuple[int, ...]

# --------------------------------------------------------------------------
# Layer-shape lists
# --------------------------------------------------------------------------


def single_256x128() -> List[Tuple[str, Shape]]:
    """One 256x128 matrix (the small worked case, rank 2)."""
    return [("w", (256, 128))]


def resnet18_cifar_set() -> List[Tuple[str, Shape]]:
    """ResNet18 for 32x32 inputs, in model order.

    Conv weights keep their 4-D (out, in, kh, kw) shape; the plan reshapes them
    to (out, in*kh*kw).  Each BatchNorm contributes a weight and a bias vector;
    the classifier is 10x512 with a bias.  11,164,352 matrix elements and 9,610
    vector elements.
    """
    t: List[Tuple[str, Shape]] = []

    def bn(name: str, c: int) -> None:
        t.append((name + ".weight", (c,)))
        t.append((name + ".bias", (c,)))

    t.append(("conv1.weight", (64, 3, 3, 3)))
    bn("bn1", 64)
    cin = 64
    for li, cout in enumerate((64, 128, 256, 512), start=1):
        for b in range(2):
            pre = f"layer{li}.{b}"
            first_in = cin if b == 0 else cout
            t.append((pre + ".conv1.weight", (cout, first_in, 3, 3)))
            bn(pre + ".bn1", cout)
            t.append((pre + ".conv2.weight", (cout, cout, 3, 3)))
            bn(pre + ".bn2", cout)
            if b == 0 and first_in != cout:
                t.append((pre + ".shortcut.0.weight", (cout, first_in, 1, 1)))
                bn(pre + ".shortcut.1", cout)
        cin = cout
    t.append(("linear.weight", (10, 512)))
    t.append(("linear.bias", (10,)))
    return t


def lstm3_wikitext_set() -> List[Tuple[str, Shape]]:
    """3-layer LSTM language model, 650 hidden units, 33,278-word vocabulary,
    tied embedding/decoder weight.  Biases (b_ih, b_hh per layer, decoder bias)
    are vectors and pass through uncompressed."""
    t: List[Tuple[str, Shape]] = [("encoder.weight", (33278, 650))]
    for l in range(3):
        t.append((f"rnn.weight_ih_l{l}", (2600, 650)))
        t.append((f"rnn.weight_hh_l{l}", (2600, 650)))
        t.append((f"rnn.bias_ih_l{l}", (2600,)))
        t.append((f"rnn.bias_hh_l{l}", (2600,)))
    t.append(("decoder.bias", (33278,)))
    return t


def llama7b_set(layers: int = 32) -> List[Tuple[str, Shape]]:
    """7B-transformer shaped matrix set: per layer q,k,v,o 4096x4096, gate and
    up 11008x4096, down 4096x11008; plus a 32000x4096 embedding and head.
    With 32 layers: 226 matrices, 6,738,149,376 elements."""
    t: List[Tuple[str, Shape]] = [("embed", (32000, 4096))]
    for l in range(layers):
        for p in ("q", "k", "v", "o"):
            t.append((f"l{l}.{p}", (4096, 4096)))
        t.append((f"l{l}.gate", (11008, 4096)))
        t.append((f"l{l}.up", (11008, 4096)))
        t.append((f"l{l}.down", (4096, 11008)))
    t.append(("head", (32000, 4096)))
    return t


def matrix_view(shape: Shape) -> Tuple[int, int]:
    """(rows, cols) of the row-major 2-D view of a tensor of this shape."""
    if len(shape) == 0:
        return (1, 1)
    if len(shape) == 1:
        return (shape[0], 1)
    return (shape[0], int(np.prod(shape[1:])))


# --------------------------------------------------------------------------
# Seeding
# --------------------------------------------------------------------------


def rng(*key: int) -> np.random.Generator:
    """Independent numpy generator for an integer key tuple."""
    return np.random.default_rng(list(int(k) for k in key))


def orthonormal(g: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """Seeded random matrix with orthonormal columns (QR of a Gaussian)."""
    a = g.standard_normal((rows, cols))
    q, _ = np.linalg.qr(a)
    return q


# --------------------------------------------------------------------------
# Workload 1: one 256x128 matrix, rank 2, 10 steps
# --------------------------------------------------------------------------


@dataclass
class SmallMatrixWorkload:
    """G_t = U diag(1/k, k=1..8) V^T + N(0, 0.01^2), fresh noise per step.

    Draw order from one generator seeded with `seed`: U, V, Q0, then the
    per-step noise.
    """

    seed: int = 1
    m: int = 256
    n: int = 128
    k: int = 8
    rank: int = 2
    steps: int = 10
    noise: float = 0.01
    U: np.ndarray = field(init=False)
    V: np.ndarray = field(init=False)
    Q0: np.ndarray = field(init=False)
    grads: List[np.ndarray] = field(init=False)

    def __post_init__(self) -> None:
        g = np.random.default_rng(self.seed)
        self.U = orthonormal(g, self.m, self.k)
        self.V = orthonormal(g, self.n, self.k)
        self.Q0 = g.standard_normal((self.n, self.rank)).astype(np.float32)
        s = 1.0 / np.arange(1, self.k + 1)
        signal = (self.U * s) @ self.V.T
        self.grads = []
        for _ in range(self.steps):
            nz = g.standard_normal((self.m, self.n)) * self.noise
            self.grads.append((signal + nz).astype(np.float32))


# --------------------------------------------------------------------------
# Workloads 2 and 3: a model's set, fixed low-rank signal + fresh noise
# --------------------------------------------------------------------------


@dataclass
class ModelSetWorkload:
    """Gradient set for a list of tensors.

    Each >=2-D tensor's row-major matrix view gets a fixed signal
    S = U diag(sigma) V^T (seeded per tensor) plus Gaussian noise redrawn every
    step (seeded per tensor and step).  Vectors get noise only.

    kind = "resnet18": noise N(0, 1e-3^2); rank-4 signal, sigma_j ~ 1/j, scaled
        so that ||S||_F / E||N||_F = 0.8 / 0.6 (the signal carries about 80% of
        the Frobenius norm when S and N are orthogonal).
    kind = "lstm3": full-rank signal with sigma_k ~ k^-1.5 (all min(m, n)
        directions), entries of order 1e-3; noise at 5% of ||S||_F.
    kind = "plain": standard normal entries only (for edge-case sweeps).
    """

    tensors: Sequence[Tuple[str, Shape]]
    kind: str
    seed: int
    _signal: Dict[int, np.ndarray] = field(default_factory=dict, init=False)

    def shapes(self) -> List[Shape]:
        return [s for _, s in self.tensors]

    def _make_signal(self, i: int) -> Optional[np.ndarray]:
        shape = self.tensors[i][1]
        if len(shape) < 2 or self.kind == "plain":
            return None
        m, n = matrix_view(shape)
        g = rng(self.seed, i, 1)
        if self.kind == "resnet18":
            k = min(4, m, n)
            U = orthonormal(g, m, k)
            V = orthonormal(g, n, k)
            s = 1.0 / np.arange(1, k + 1)
            S = (U * s) @ V.T
            target = (0.8 / 0.6) * 1e-3 * math.sqrt(m * n)
            return S * (target / np.linalg.norm(S))
        if self.kind == "lstm3":
            k = min(m, n)
            U = orthonormal(g, m, k)
            V = orthonormal(g, n, k)
            s = np.arange(1, k + 1, dtype=np.float64) ** -1.5
            S = (U * s) @ V.T
            return S * (1e-3 * math.sqrt(m * n) / np.linalg.norm(S))
        raise ValueError(self.kind)

    def signal(self, i: int) -> Optional[np.ndarray]:
        if i not in self._signal:
            self._signal[i] = self._make_signal(i)
        return self._signal[i]

    def grad(self, i: int, step: int) -> np.ndarray:
        """fp32 gradient of tensor i at step `step` (1-based), in its
        row-major matrix view (vectors are returned as 1-D)."""
        shape = self.tensors[i][1]
        g = rng(self.seed, i, 2, step)
        if len(shape) < 2:
            std = 1.0 if self.kind == "plain" else 1e-3
            return (g.standard_normal(shape[0]) * std).astype(np.float32)
        m, n = matrix_view(shape)
        S = self.signal(i)
        if S is None:
            return g.standard_normal((m, n)).astype(np.float32)
        if self.kind == "resnet18":
            N = g.standard_normal((m, n)) * 1e-3
        else:
            N = g.standard_normal((m, n)) * (0.05 * np.linalg.norm(S) / math.sqrt(m * n))
        return (S + N).astype(np.float32)

    def q0(self, i: int, rank: int) -> np.ndarray:
        """Seeded N(0,1) warm-start factor (cols x rank) for tensor i."""
        m, n = matrix_view(self.tensors[i][1])
        return rng(self.seed, i, 3).standard_normal((n, rank)).astype(np.float32)


# --------------------------------------------------------------------------
# Workload 5: decaying spectrum sigma_k = exp(-k/20), K = 512
# --------------------------------------------------------------------------


def decaying_spectrum_matrix(m: int, n: int, seed: int = 5, K: int = 512,
                             decay: float = 20.0) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """A = U diag(exp(-k/decay), k=1..K) V^T built in fp64 from seeded QR, cast
    to fp32.  Returns (A_fp32, V_fp64 (n x K), sigma (K,)) so that tests know
    the exact leading right-singular subspace."""
    K = min(K, m, n)
    g = rng(seed, m, n)
    U = orthonormal(g, m, K)
    V = orthonormal(g, n, K)
    s = np.exp(-np.arange(1, K + 1, dtype=np.float64) / decay)
    A = (U * s) @ V.T
    return A.astype(np.float32), V, s


def gaussian_q0(n: int, rank: int, seed: int) -> np.ndarray:
    return rng(seed, n, rank, 7).standard_normal((n, rank)).astype(np.float32)


# --------------------------------------------------------------------------
# Workload 4: 7B-shaped set, generated on the device with torch
# --------------------------------------------------------------------------


def _mix(*key: int) -> int:
    """Deterministic 63-bit seed from an integer key (splitmix64 finaliser)."""
    x = 0x9E3779B97F4A7C15
    for k in key:
        x = (x ^ (int(k) & 0xFFFFFFFFFFFFFFFF)) & 0xFFFFFFFFFFFFFFFF
        x = (x * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        x ^= x >> 31
        x = (x * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
        x ^= x >> 29
    return x & 0x7FFFFFFFFFFFFFFF


def llama7b_grad_(out, m: int, n: int, index: int, step: int, seed: int = 4,
                  signal_rank: int = 16):
    """Fill the (m, n) fp32 torch tensor `out` (any device) with one matrix of
    the 7B-shaped set: a rank-16 signal (sigma_j ~ 1/j, fixed per matrix) plus
    N(0,1) noise (fresh per step) with ||S||_F/||N||_F = 0.7/0.714, then scaled
    to unit Frobenius norm.  Deterministic per (seed, index, step) on a given
    device type."""
    import torch

    dev = out.device
    gs = torch.Generator(device=dev)
    gs.manual_seed(_mix(seed, index, 1))
    U = torch.randn(m, signal_rank, generator=gs, device=dev) / math.sqrt(m)
    V = torch.randn(n, signal_rank, generator=gs, device=dev) / math.sqrt(n)
    s = 1.0 / torch.arange(1, signal_rank + 1, device=dev, dtype=torch.float32)
    gn = torch.Generator(device=dev)
    gn.manual_seed(_mix(seed, index, 2, step))
    torch.randn(m, n, generator=gn, device=dev, out=out)
    nn = torch.linalg.vector_norm(out)
    S = (U * s) @ V.T
    S *= (0.7 / 0.714) * nn / torch.linalg.vector_norm(S)
    out += S
    del S
    out /= torch.linalg.vector_norm(out)
    return out


def llama7b_q0(n: int, rank: int, index: int, seed: int = 4, device="cpu"):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(_mix(seed, index, 3))
    return torch.randn(n, rank, generator=g, device=device)
