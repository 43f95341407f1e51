"""Buffer-owning convenience layer over the C ABI, with PyTorch supplying the
device memory and the stream.  It allocates and views buffers and marshals
pointers; every step of the computation runs in libpsgd.so.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import torch

from . import binding as B


def matrix_view(shape: Sequence[int]) -> Tuple[int, int]:
    """(rows, cols) the plan sees for a tensor shape; cols = 1 for vectors."""
    shape = tuple(int(s) for s in shape)
    if len(shape) == 0:
        return (1, 1)
    if len(shape) == 1:
        return (shape[0], 1)
    n = 1
    for s in shape[1:]:
        n *= s
    return (shape[0], n)


class PowerSGD:
    """A plan plus the flat buffers one worker owns for it.

    grads  flat gradient buffer (write the gradients here, or pass your own);
           float32, or bfloat16 with grads_dtype=torch.bfloat16
    err    error-feedback memory (zero-initialised)
    mom    momentum buffer (momentum variant only, zero-initialised)
    q      packed warm-start / output Q
    p      packed P_hat followed by the pass-through values
    mhat   flat decompressed gradient (allocated on request)
    """

    def __init__(self, shapes: Sequence[Sequence[int]], rank: int, device="cuda", momentum_beta: Optional[float] = None,
                 offsets: Optional[Sequence[int]] = None, with_mhat: bool = True, grads: Optional[torch.Tensor] = None,
                 grads_dtype: torch.dtype = torch.float32):
        self.shapes = [tuple(int(x) for x in s) for s in shapes]
        self.views = [matrix_view(s) for s in self.shapes]
        self.rank = int(rank)
        if grads_dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("gradients must be float32 or bfloat16")
        flags = B.PSGD_FLAG_MOMENTUM if momentum_beta is not None else 0
        if grads_dtype == torch.bfloat16:
            flags |= B.PSGD_FLAG_GRADS_BF16
        self.plan = B.psgd_plan_create([v[0] for v in self.views],
                                       [v[1] if len(s) >= 2 else 1 for v, s in zip(self.views, self.shapes)],
                                       self.rank, flags, float(momentum_beta or 0.0), offsets)
        self.info = B.psgd_plan_get_info(self.plan)
        self.tensors = [B.psgd_plan_tensor(self.plan, i) for i in range(len(self.shapes))]
        self.device = torch.device(device)
        n = self.info["flat_elems"]
        f32 = dict(dtype=torch.float32, device=self.device)
        self.grads = grads if grads is not None else torch.zeros(n, dtype=grads_dtype, device=self.device)
        assert self.grads.numel() >= n and self.grads.dtype == grads_dtype
        self.err = torch.zeros(n, **f32)
        self.mom = torch.zeros(n, **f32) if momentum_beta is not None else None
        self.q = torch.zeros(max(1, self.info["q_elems"]), **f32)
        self.p = torch.zeros(max(1, self.info["p_buffer_elems"]), **f32)
        self.mhat = torch.zeros(n, **f32) if with_mhat else None
        self.ws_bytes = int(self.info["workspace_bytes"])
        self.workspace = torch.zeros(max(256, self.ws_bytes), dtype=torch.uint8, device=self.device)
        assert self.workspace.data_ptr() % 256 == 0
        B.psgd_workspace_init(self.plan, self.workspace.data_ptr(), self.ws_bytes, self._stream())

    # ---------------------------------------------------------------- views
    def kind(self, i: int) -> int:
        return self.tensors[i][0]

    def compressed(self) -> List[int]:
        return [i for i in range(len(self.shapes)) if self.kind(i) == B.PSGD_KIND_COMPRESSED]

    def view(self, buf: torch.Tensor, i: int) -> torch.Tensor:
        """Tensor i of a flat buffer, as its (rows, cols) matrix (or vector)."""
        _, off, _, _ = self.tensors[i]
        m, n = self.views[i]
        v = buf[off: off + m * n]
        return v if len(self.shapes[i]) < 2 else v.view(m, n)

    def p_hat(self, i: int) -> torch.Tensor:
        kind, _, poff, _ = self.tensors[i]
        m, n = self.views[i]
        if kind != B.PSGD_KIND_COMPRESSED:
            return self.p[poff: poff + m * n]
        return self.p[poff: poff + self.rank * m].view(self.rank, m).t()

    def q_of(self, i: int) -> torch.Tensor:
        _, _, _, qoff = self.tensors[i]
        m, n = self.views[i]
        return self.q[qoff: qoff + self.rank * n].view(self.rank, n).t()

    def set_q(self, i: int, q0) -> None:
        t = torch.as_tensor(q0, dtype=torch.float32)
        self.q_of(i).copy_(t.to(self.device))

    # ----------------------------------------------------------------- calls
    @staticmethod
    def _stream() -> int:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else 0

    def compress(self, mhat: bool = False, hook=None, mhat_buf: Optional[torch.Tensor] = None,
                 refresh_iters: int = 0, power_iters: int = 0, error_feedback: bool = True,
                 params: Optional[torch.Tensor] = None, sgd_buf: Optional[torch.Tensor] = None, sgd_lr: float = 0.0,
                 sgd_momentum: float = 0.0, nesterov: bool = False, defer_residual: bool = False,
                 residual_deferred: bool = False, payload_bf16: bool = False, payload_fp8: bool = False,
                 noalloc: bool = False, zero_cols: Optional[torch.Tensor] = None) -> None:
        """One psgd_compress call on the owned buffers; noalloc=True takes
        psgd_compress_noalloc (the library's static scratch, no workspace)."""
        out = mhat_buf if mhat_buf is not None else (self.mhat if mhat else None)
        opts = None
        flags = (0 if error_feedback else B.PSGD_STEP_NO_ERROR_FEEDBACK) | (B.PSGD_STEP_NESTEROV if nesterov else 0)
        flags |= (B.PSGD_STEP_DEFER_RESIDUAL if defer_residual else 0)
        flags |= (B.PSGD_STEP_RESIDUAL_DEFERRED if residual_deferred else 0)
        flags |= (B.PSGD_STEP_PAYLOAD_BF16 if payload_bf16 else 0)
        flags |= (B.PSGD_STEP_PAYLOAD_FP8 if payload_fp8 else 0)
        if refresh_iters or power_iters or flags or params is not None or zero_cols is not None:
            if zero_cols is not None:
                assert zero_cols.dtype == torch.int32 and zero_cols.numel() >= self.info["ncompressed"]
            opts = B.step_opts(power_iters, refresh_iters, flags, sgd_lr, sgd_momentum, params.data_ptr() if params is not None else 0,
                               sgd_buf.data_ptr() if sgd_buf is not None else 0,
                               zero_cols.data_ptr() if zero_cols is not None else 0)
        if noalloc:
            B.psgd_compress_noalloc(self.plan, self.grads.data_ptr(), self.err.data_ptr(),
                                    self.mom.data_ptr() if self.mom is not None else 0, self.q.data_ptr(),
                                    self.p.data_ptr(), out.data_ptr() if out is not None else 0, opts, hook,
                                    self._stream())
            return
        B.psgd_compress(self.plan, self.grads.data_ptr(), self.err.data_ptr(),
                        self.mom.data_ptr() if self.mom is not None else 0, self.q.data_ptr(), self.p.data_ptr(),
                        out.data_ptr() if out is not None else 0, opts, hook, self.workspace.data_ptr(),
                        self.ws_bytes, self._stream())

    def decompress(self, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        out = out if out is not None else self.mhat
        B.psgd_decompress(self.plan, self.p.data_ptr(), self.q.data_ptr(), out.data_ptr(), self.workspace.data_ptr(),
                          self.ws_bytes, self._stream())
        return out

    def init_q(self, seed: int) -> None:
        """Seeded N(0, 1) start Q for every compressed tensor (psgd_init_q)."""
        B.psgd_init_q(self.plan, self.q.data_ptr(), int(seed), self.workspace.data_ptr(), self.ws_bytes,
                      self._stream())

    def refresh(self, i: int, m_buf: torch.Tensor, iters: int) -> None:
        B.psgd_refresh(self.plan, i, m_buf.data_ptr(), self.q.data_ptr(), iters, self.workspace.data_ptr(),
                       self.ws_bytes, self._stream())

    def step_stats(self) -> torch.Tensor:
        """(ncompressed, 2) fp64 on the device: ||E||^2 and ||M||^2 per
        compressed matrix after a compress with mhat=True (psgd_step_stats)."""
        out = torch.empty((max(1, self.info["ncompressed"]), 2), dtype=torch.float64, device=self.device)
        B.psgd_step_stats(self.plan, self.err.data_ptr(), self.mhat.data_ptr(), out.data_ptr(),
                          self.workspace.data_ptr(), self.ws_bytes, self._stream())
        return out[: self.info["ncompressed"]]

    def compression_errors(self) -> torch.Tensor:
        """||E|| / ||M|| per compressed matrix (0 where M is zero)."""
        st = self.step_stats()
        return torch.where(st[:, 1] > 0, (st[:, 0] / st[:, 1].clamp_min(1e-300)).sqrt(), torch.zeros_like(st[:, 0]))

    def subspace_overlap(self, q_other: torch.Tensor, q: Optional[torch.Tensor] = None) -> torch.Tensor:
        """(ncompressed,) fp64 on the device: mean cosine of the principal
        angles between each matrix's factor in q_other and in q (default:
        the current Q), psgd_subspace_overlap."""
        q = self.q if q is None else q
        scratch = torch.empty(2 * max(1, self.info["q_elems"]), dtype=torch.float32, device=self.device)
        out = torch.empty(max(1, self.info["ncompressed"]), dtype=torch.float64, device=self.device)
        B.psgd_subspace_overlap(self.plan, q_other.data_ptr(), q.data_ptr(), scratch.data_ptr(), out.data_ptr(),
                                self.workspace.data_ptr(), self.ws_bytes, self._stream())
        return out[: self.info["ncompressed"]]

    def close(self) -> None:
        if self.plan:
            B.psgd_plan_destroy(self.plan)
            self.plan = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
