"""PowerSGD compression step: plain fp64 reference oracle.

TEST INFRASTRUCTURE.  Only the tests, the package smoke entry and the
benchmark's CPU-baseline leg import this module; the GPU library never does,
and the two share no code.  Everything is numpy in float64; fp32 inputs are
upcast exactly.  The code follows the method's steps in the order the pages
give them, one matrix at a time, with no blocking, fusion or reordering.

Sources, cited by page and section:
  [N152]  anthology-of-the-sota record, note 152 (PowerSGD): sections
          "Contribution", "Key insight", "Method", "Concepts", "Limitations".
  [GLOSS] inferensys glossary entry "PowerSGD": the paragraphs on the
          factorisation, the warm-started power iteration, error feedback,
          momentum compression and temporal coherence.
  [PSGD+] "From PowerSGD to PowerSGD+: Low-Rank Gradient Compression for
          Distributed Optimization with Convergence Guarantees", Abstract.

Readings taken where the pages leave a step open (each is also listed in the
design notes of the repository):
  R1  one warm-started power iteration per step ([N152] Method; the glossary's
      "one or two" is read as the first of the two).
  R2  the warm start uses the raw Q = M^T P_hat of the previous step, not an
      orthonormalised copy.
  R3  orthogonalisation is modified Gram-Schmidt in natural column order with
      positive normalisation; a column whose norm after projection is at most
      1e-4 of its norm before projection (or whose input norm is zero) becomes
      the zero column.
  R4  the residual uses the post-aggregation Q, i.e. the same M_hat that
      decompression returns.
  R5  1-D tensors are vectors and pass through; >=2-D tensors are viewed as
      (dim0, prod(rest)) and compressed iff r*(m+n) < m*n, otherwise they pass
      through.  Pass-through tensors carry no error-feedback state.
  R6  momentum variant: u <- beta*u + G (no dampening, u_0 = 0), then the
      compressor input is u (pass-through tensors transmit u as well).
  R7  PowerSGD+ refresh: at a refresh step, before P = M Q, repeat `iters`
      times Q <- GS(M^T GS(M Q)) on the current M, starting from the current
      warm-start Q; the normal step then follows from the refreshed Q.
  R8  several power iterations in one step (the glossary's "one or two"):
      P = M Q, aggregate, P_hat = GS(P), Q = M^T P_hat, aggregate, repeated,
      each iteration starting from the previous one's Q.
  R9  post-compression momentum ([N152] Concepts): heavy-ball SGD on the
      decompressed, aggregated update D: m <- mu m + D, x <- x - lr m; with
      the Nesterov option of standard SGD ([GLOSS], momentum paragraph: the
      scheme works with the usual optimizers), x <- x - lr (D + mu m).
  R10 the first Q, and a cold start's fresh Q every step, is i.i.d. N(0, 1)
      from a seeded counter-based generator (module philox).
  R11 compound compression ([GLOSS]: the factors PowerSGD produces can
      themselves be quantised): the two transmitted factors, P before its
      aggregation and Q before its aggregation, are rounded to bfloat16 from
      their fp32 values (round to nearest, ties to even); everything after a
      hook uses the values as received, so the residual, and with it the
      error memory, carries the quantisation error too.
  R12 compound compression to 8 bits: each column of each transmitted factor
      (P, then Q, before its aggregation, as in R11) is sent as an OCP FP8
      E4M3 code per value times one power of two per column, 2^k with k the
      smallest integer for which the column's largest magnitude (of its fp32
      values) is at most 448 * 2^k, the format's largest finite value; each
      value becomes 2^k * e4m3(x / 2^k), rounded to nearest with ties to
      even, so it stays exact in fp32 and no value overflows.  An all-zero
      column stays zero.  Pass-through values are not rounded.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, List, Optional, Sequence, Tuple

import numpy as np

ZERO_COLUMN_REL = 1e-4

KIND_VECTOR = 0
KIND_PASSTHRU = 1
KIND_COMPRESSED = 2

Hook = Optional[Callable[[np.ndarray], np.ndarray]]


# --------------------------------------------------------------------------
# Plan: which tensors are compressed ([N152] Method; reading R5)
# --------------------------------------------------------------------------


def matrix_view(shape: Sequence[int]) -> Tuple[int, int]:
    """Per-layer approximation with conv tensors reshaped to matrices
    ([N152] Method, last bullet): (dim0, product of the other dims)."""
    if len(shape) < 2:
        return (int(shape[0]) if len(shape) else 1, 1)
    return int(shape[0]), int(np.prod(shape[1:]))


def classify(shape: Sequence[int], rank: int) -> int:
    """Bias vectors and small tensors travel uncompressed ([N152] Method).
    'Small' is read as: the rank-r factors would not be smaller than the
    matrix, r(m+n) >= mn (the O(r(m+n)) vs O(mn) payload of [GLOSS])."""
    if len(shape) < 2:
        return KIND_VECTOR
    m, n = matrix_view(shape)
    return KIND_COMPRESSED if rank * (m + n) < m * n else KIND_PASSTHRU


@dataclass
class Plan:
    shapes: List[Tuple[int, ...]]
    rank: int

    def __post_init__(self) -> None:
        self.kinds = [classify(s, self.rank) for s in self.shapes]
        self.views = [matrix_view(s) for s in self.shapes]

    def numel(self, i: int) -> int:
        return int(np.prod(self.shapes[i])) if self.shapes[i] else 1

    @property
    def compressed(self) -> List[int]:
        return [i for i, k in enumerate(self.kinds) if k == KIND_COMPRESSED]

    @property
    def passthrough(self) -> List[int]:
        return [i for i, k in enumerate(self.kinds) if k != KIND_COMPRESSED]

    def payload(self) -> Tuple[int, int, int]:
        """(sum m*r, sum n*r, pass-through elements): floats exchanged per step.
        The dense alternative exchanges sum m*n + pass-through ([GLOSS],
        factorisation paragraph)."""
        pm = sum(self.views[i][0] * self.rank for i in self.compressed)
        qn = sum(self.views[i][1] * self.rank for i in self.compressed)
        pt = sum(self.numel(i) for i in self.passthrough)
        return pm, qn, pt

    def dense_elems(self) -> int:
        return sum(self.views[i][0] * self.views[i][1] for i in self.compressed)


# --------------------------------------------------------------------------
# Orthogonalisation ([N152] Method: "Gram-Schmidt orthogonalization of the P
# factor"; reading R3)
# --------------------------------------------------------------------------


def gram_schmidt(P: np.ndarray) -> np.ndarray:
    """Modified Gram-Schmidt on the columns of P (m x r), natural order,
    positive normalisation, near-dependent columns set to zero."""
    P = np.asarray(P, dtype=np.float64)
    m, r = P.shape
    out = np.zeros((m, r), dtype=np.float64)
    for k in range(r):
        v = P[:, k].copy()
        nu0 = float(np.sqrt(v @ v))
        for j in range(k):
            v = v - (out[:, j] @ v) * out[:, j]
        nv = float(np.sqrt(v @ v))
        if nu0 == 0.0 or nv <= ZERO_COLUMN_REL * nu0:
            continue  # column stays zero
        out[:, k] = v / nv
    return out


# --------------------------------------------------------------------------
# One compression of one matrix ([N152] Method and Concepts)
# --------------------------------------------------------------------------


@dataclass
class MatrixResult:
    P_hat: np.ndarray   # m x r, orthonormal (or zero) columns
    Q: np.ndarray       # n x r, also the next warm start (R2)
    M_hat: np.ndarray   # P_hat Q^T, the reconstructed gradient
    E: np.ndarray       # new error-feedback memory M - M_hat
    P: np.ndarray       # P = M Q_warm (after the P hook), before GS


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Payload quantiser of reading R11: the value as the kernels hold it
    (fp32), rounded to the nearest bfloat16 with ties to even, returned in
    fp64.  bfloat16 keeps fp32's exponent range and 8 significant bits, so the
    spacing at |x| in [2^e, 2^(e+1)) is 2^(e-7), and 2^-133 below 2^-126 (the
    subnormal range); np.rint rounds halves to even.  Finite inputs only."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    out = np.zeros_like(f)
    nz = f != 0.0
    e = np.floor(np.log2(np.abs(f[nz])))
    # guard the binade against log2 rounding at exact powers of two
    e = np.where(np.abs(f[nz]) < 2.0 ** e, e - 1, e)
    e = np.where(np.abs(f[nz]) >= 2.0 ** (e + 1), e + 1, e)
    step = 2.0 ** np.maximum(e - 7, -133)
    out[nz] = np.rint(f[nz] / step) * step
    return out


FP8_E4M3_MAX = 448.0  # (1 + 6/8) * 2^8: the largest finite E4M3 value


def round_fp8_e4m3(y: np.ndarray) -> np.ndarray:
    """The nearest OCP FP8 E4M3 value (ties to even) to each y, |y| <= 448,
    in fp64.  E4M3 has 3 fraction bits and exponents -6..8: in the binade
    [2^e, 2^(e+1)) its values are 2^(e-3) apart, and below 2^-6 (the
    subnormals, m/8 * 2^-6) 2^-9 apart; np.rint rounds halves to even."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    if (a > FP8_E4M3_MAX).any():
        raise ValueError("round_fp8_e4m3: magnitude above 448")
    out = np.zeros_like(a)
    nz = a != 0.0
    e = np.floor(np.log2(a[nz]))
    e = np.where(a[nz] < 2.0 ** e, e - 1, e)  # guard log2 rounding at powers of two
    e = np.where(a[nz] >= 2.0 ** (e + 1), e + 1, e)
    step = 2.0 ** (np.maximum(e, -6.0) - 3.0)
    out[nz] = np.rint(a[nz] / step) * step
    return np.copysign(out, y)


def fp8_column_exponent(amax: float) -> int:
    """Reading R12: the smallest integer k with amax <= 448 * 2^k (0 for a
    zero column).  With amax = f 2^E, f in [0.5, 1) (frexp) and
    448 = 0.875 * 2^9: k = E - 9 when f <= 0.875, else E - 8."""
    if amax == 0.0:
        return 0
    f, E = np.frexp(float(amax))
    return int(E) - 9 if f <= 0.875 else int(E) - 8


def round_fp8_columns(F: np.ndarray) -> np.ndarray:
    """Payload quantiser of reading R12 on a factor (rows x r): the values as
    the kernels hold them (fp32), each column scaled by its power of two,
    rounded to E4M3 and scaled back; returned in fp64."""
    f = np.asarray(F, dtype=np.float64).astype(np.float32).astype(np.float64)
    f = f.reshape(f.shape[0], -1)
    out = np.zeros_like(f)
    for c in range(f.shape[1]):
        k = fp8_column_exponent(np.abs(f[:, c]).max() if f.shape[0] else 0.0)
        out[:, c] = np.ldexp(round_fp8_e4m3(np.ldexp(f[:, c], -k)), k)
    return out.reshape(np.shape(F))


def compress_matrix(M: np.ndarray, Q_warm: np.ndarray, hook_p: Hook = None,
                    hook_q: Hook = None, power_iters: int = 1,
                    quantize: Optional[Callable[[np.ndarray], np.ndarray]] = None) -> MatrixResult:
    """One warm-started subspace iteration on M ([N152] Method):
    right multiply P = M Q, aggregate P, orthogonalise to P_hat, left multiply
    Q = M^T P_hat, aggregate Q.  Then the reconstruction P_hat Q^T and the
    error-feedback residual M - P_hat Q^T ([GLOSS] error-feedback paragraph;
    [N152] Concepts, "Error feedback").  power_iters > 1 repeats the
    iteration from the new Q (reading R8).  `quantize` (reading R11 or R12)
    is applied to P and to Q as they are formed, before their hooks."""
    M = np.asarray(M, dtype=np.float64)
    Q = np.asarray(Q_warm, dtype=np.float64)
    for _ in range(max(1, power_iters)):
        P = M @ Q
        if quantize is not None:
            P = quantize(P)
        if hook_p is not None:
            P = hook_p(P)
        P_hat = gram_schmidt(P)
        Q = M.T @ P_hat
        if quantize is not None:
            Q = quantize(Q)
        if hook_q is not None:
            Q = hook_q(Q)
    M_hat = P_hat @ Q.T
    E = M - M_hat
    return MatrixResult(P_hat=P_hat, Q=Q, M_hat=M_hat, E=E, P=P)


def decompress(P_hat: np.ndarray, Q: np.ndarray) -> np.ndarray:
    """G ~ P Q^T ([GLOSS], factorisation paragraph)."""
    return np.asarray(P_hat, np.float64) @ np.asarray(Q, np.float64).T


def refresh(M: np.ndarray, Q: np.ndarray, iters: int) -> np.ndarray:
    """PowerSGD+ periodic re-alignment of the projection subspace ([PSGD+]
    Abstract: via an SVD).  Reading R7: the SVD's leading right subspace is
    approached by `iters` rounds of orthonormalised block power iteration."""
    M = np.asarray(M, dtype=np.float64)
    Q = np.asarray(Q, dtype=np.float64)
    for _ in range(iters):
        P_hat = gram_schmidt(M @ Q)
        Q = gram_schmidt(M.T @ P_hat)
    return Q


def sgd_momentum_step(x: np.ndarray, m: np.ndarray, D: np.ndarray, lr: float, mu: float, nesterov: bool = False):
    """Post-compression momentum ([N152] Concepts; reading R9): SGD with
    momentum on the decompressed update D.  Returns (x, m)."""
    D = np.asarray(D, np.float64)
    m = mu * np.asarray(m, np.float64) + D
    direction = D + mu * m if nesterov else m
    return np.asarray(x, np.float64) - lr * direction, m


def momentum_input(u: np.ndarray, G: np.ndarray, beta: float) -> np.ndarray:
    """Compress the momentum term instead of the raw gradient ([GLOSS],
    momentum paragraph).  Reading R6: heavy-ball u <- beta*u + G."""
    return beta * np.asarray(u, np.float64) + np.asarray(G, np.float64)


# --------------------------------------------------------------------------
# One step over a whole model's tensor set
# --------------------------------------------------------------------------


@dataclass
class SetState:
    """Per-worker state the caller owns: error memories and warm-start Qs of the
    compressed tensors, momentum buffers of every tensor (momentum variant)."""
    E: List[Optional[np.ndarray]]
    Q: List[Optional[np.ndarray]]
    u: Optional[List[np.ndarray]] = None


def init_state(plan: Plan, q0: Sequence[Optional[np.ndarray]], momentum: bool = False) -> SetState:
    E: List[Optional[np.ndarray]] = []
    Q: List[Optional[np.ndarray]] = []
    for i, k in enumerate(plan.kinds):
        if k == KIND_COMPRESSED:
            m, n = plan.views[i]
            E.append(np.zeros((m, n)))
            Q.append(np.asarray(q0[i], np.float64).copy())
        else:
            E.append(None)
            Q.append(None)
    u = None
    if momentum:
        u = [np.zeros(plan.views[i]) if plan.kinds[i] != KIND_VECTOR else np.zeros(plan.numel(i))
             for i in range(len(plan.shapes))]
    return SetState(E=E, Q=Q, u=u)


@dataclass
class SetResult:
    P_hat: List[Optional[np.ndarray]]
    Q: List[Optional[np.ndarray]]
    M_hat: List[np.ndarray]             # reconstructed tensors (pass-through: the value sent)
    M: List[Optional[np.ndarray]]       # compressor inputs X + E of compressed tensors
    P: List[Optional[np.ndarray]] = field(default_factory=list)  # P = M Q before orthogonalisation


def step_set(plan: Plan, grads: Sequence[np.ndarray], state: SetState, beta: float = 0.0,
             refresh_iters: int = 0, hook_p: Hook = None, hook_q: Hook = None, power_iters: int = 1,
             error_feedback: bool = True, quantize: Optional[Callable[[np.ndarray], np.ndarray]] = None) -> SetResult:
    """One compression step over a model's set, updating `state` in place.

    Per compressed matrix: X = G (or the momentum u), M = X + E (M = X when
    error feedback is off, an ablation), optional refresh of the warm-start
    Q, then `compress_matrix`; E and Q are replaced by the new residual and Q.
    Pass-through tensors send X unchanged."""
    Ph: List[Optional[np.ndarray]] = []
    Qs: List[Optional[np.ndarray]] = []
    Mh: List[np.ndarray] = []
    Ms: List[Optional[np.ndarray]] = []
    Pr: List[Optional[np.ndarray]] = []
    for i, kind in enumerate(plan.kinds):
        G = np.asarray(grads[i], dtype=np.float64).reshape(plan.views[i] if kind != KIND_VECTOR else -1)
        if state.u is not None:
            state.u[i] = momentum_input(state.u[i], G, beta)
            X = state.u[i]
        else:
            X = G
        if kind != KIND_COMPRESSED:
            Ph.append(None)
            Qs.append(None)
            Mh.append(X.copy())
            Ms.append(None)
            Pr.append(None)
            continue
        M = X + state.E[i] if error_feedback else X.copy()
        Qw = state.Q[i]
        if refresh_iters > 0:
            Qw = refresh(M, Qw, refresh_iters)
        res = compress_matrix(M, Qw, hook_p, hook_q, power_iters=power_iters, quantize=quantize)
        state.E[i] = res.E
        state.Q[i] = res.Q
        Ph.append(res.P_hat)
        Qs.append(res.Q)
        Mh.append(res.M_hat)
        Ms.append(M)
        Pr.append(res.P)
    return SetResult(P_hat=Ph, Q=Qs, M_hat=Mh, M=Ms, P=Pr)


# --------------------------------------------------------------------------
# W simulated workers in lockstep ([N152] Concepts, "Linearity of
# compressor"): the aggregation hooks average across workers.
# --------------------------------------------------------------------------


def compress_workers(Ms: Sequence[np.ndarray], Q_warm: np.ndarray,
                     power_iters: int = 1) -> Tuple[np.ndarray, np.ndarray, List[np.ndarray]]:
    """Each worker forms P_i = M_i Q; the all-reduce gives mean P; every worker
    orthogonalises the same mean into P_hat, forms Q_i = M_i^T P_hat; the
    all-reduce gives mean Q.  power_iters > 1 repeats this from the mean Q
    (reading R8).  Residuals use the aggregated reconstruction (reading R4).
    Returns (P_hat, Q, [E_i])."""
    Q = np.asarray(Q_warm, np.float64)
    Ms = [np.asarray(M, np.float64) for M in Ms]
    for _ in range(max(1, power_iters)):
        P = sum(M @ Q for M in Ms) / len(Ms)
        P_hat = gram_schmidt(P)
        Q = sum(M.T @ P_hat for M in Ms) / len(Ms)
    M_hat = P_hat @ Q.T
    return P_hat, Q, [M - M_hat for M in Ms]


# --------------------------------------------------------------------------
# Diagnostics
# --------------------------------------------------------------------------


def orthonormality_error(P_hat: np.ndarray) -> float:
    """||P_hat^T P_hat - I||_F over the non-zero columns."""
    P_hat = np.asarray(P_hat, np.float64)
    nz = np.linalg.norm(P_hat, axis=0) > 0
    A = P_hat[:, nz]
    return float(np.linalg.norm(A.T @ A - np.eye(A.shape[1])))


def principal_angle_sines(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """Sines of the principal angles between span(A) and span(B), largest
    first.  Both are orthonormalised with this module's Gram-Schmidt; the
    sines are the singular values of the lower-dimensional basis X with its
    component in the other basis Y removed, (I - Y Y^T) X, which resolves
    small angles to working precision (unlike sqrt(1 - cos^2))."""
    Qa = gram_schmidt(A)
    Qb = gram_schmidt(B)
    Qa = Qa[:, np.linalg.norm(Qa, axis=0) > 0]
    Qb = Qb[:, np.linalg.norm(Qb, axis=0) > 0]
    X, Y = (Qa, Qb) if Qa.shape[1] <= Qb.shape[1] else (Qb, Qa)
    R = X - Y @ (Y.T @ X)
    s = np.linalg.svd(R, compute_uv=False)
    return np.sort(np.clip(s, 0.0, 1.0))[::-1]


def compression_error(E: np.ndarray, M: np.ndarray) -> float:
    """||E||_F / ||M||_F: the share of the compressor's input that error
    feedback keeps for later steps ([GLOSS] error-feedback paragraph: e_t =
    G_t - compress(G_t)); 0 for a zero M."""
    nm = float(np.linalg.norm(np.asarray(M, np.float64)))
    return float(np.linalg.norm(np.asarray(E, np.float64))) / nm if nm > 0 else 0.0


def subspace_overlap(Qa: np.ndarray, Qb: np.ndarray) -> float:
    """Mean cosine of the principal angles between span(Qa) and span(Qb)
    ([GLOSS] temporal-coherence paragraph: the subspaces of consecutive steps
    overlap with cosine similarity often above 0.9).  Both n x r factors are
    orthonormalised with this module's Gram-Schmidt (dependent columns become
    zero); the cosines are the singular values of Qa_hat^T Qb_hat and the
    mean is taken over the r columns, so a zero column counts as a cosine of
    0."""
    A = gram_schmidt(Qa)
    B = gram_schmidt(Qb)
    r = np.asarray(Qa).shape[1]
    return float(np.sum(np.linalg.svd(A.T @ B, compute_uv=False)) / r)

