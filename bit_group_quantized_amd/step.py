"""Step driver: runs an ordered chain of quantized GEMV stages on one GPU.

A stage is one activation vector x (bf16 [k]) multiplied by one or more packed
Q4 matrices that share it (q, k, v share the attention input; gate and up share
the FFN input). Stages run in order: a stage may consume the previous stage's
outputs, so no stage starts its products before the previous one has finished.
This is the per-frame temporal step's weight stream (blog translation,
pipeline diagram: 32 layers of width 4096) and the Depformer's per-codebook
step (same page, MultiLinear figure).

Three executors:
* ``launches``: one q4_gemv (or, for several activation rows, q4_gemm_small)
  call per matrix, in order, on the current stream
  (capturable into a HIP graph with ``torch.cuda.graph``);
* ``chain``: the whole chain in one persistent launch (q4_chain_run);
* ``batches``: for 5..16 activation rows and stages that read no output of
  the chain, every product at once, one q4_gemm_batch_run launch per distinct
  k (the products are unordered, so a stage may not consume another's output).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import torch

from . import (q4_chain_build, q4_chain_run, q4_chain_workspace_bytes, q4_gemm_batch_build, q4_gemm_batch_run,
               q4_gemm_small, q4_gemv)


@dataclass
class Q4Matrix:
    packed: torch.Tensor   # int32 [n, k/8]
    scales: torch.Tensor   # bf16 [n, k/32]
    biases: torch.Tensor   # bf16 [n, k/32]

    @property
    def n(self) -> int:
        return self.packed.shape[0]

    @property
    def k(self) -> int:
        return self.packed.shape[1] * 8

    def nbytes(self) -> int:
        return self.packed.numel() * 4 + self.scales.numel() * 2 + self.biases.numel() * 2

    def rows(self, start: int, count: int) -> "Q4Matrix":
        """Rows [start, start + count) as views of the same storage (the
        Depformer's per-step slice of a stacked tensor: a pointer offset)."""
        return Q4Matrix(self.packed[start:start + count], self.scales[start:start + count],
                        self.biases[start:start + count])


@dataclass
class Stage:
    x: torch.Tensor                     # bf16 [k], or [m, k] for m activation rows
    mats: List[Q4Matrix]
    outs: List[Optional[torch.Tensor]] = field(default_factory=list)
    # Parts of a decoder layer fused into the chain (persistent executor only):
    norm: Optional[torch.Tensor] = None   # RMSNorm weight bf16 [k]: x is normalized first (one row)
    eps: float = 0.0
    gated: bool = False                   # two matrices (gate, up): outs[0] = silu(gate) * up
    residuals: Optional[List[Optional[torch.Tensor]]] = None  # added to each product (may be its out)

    def fused(self) -> bool:
        return self.norm is not None or self.gated or any(r is not None for r in (self.residuals or []))


class Chain:
    def __init__(self, stages: List[Stage], out_dtype: torch.dtype = torch.bfloat16):
        self.stages = stages
        self.out_dtype = out_dtype
        dev = stages[0].x.device
        for st in stages:
            if not st.outs:
                shape = (st.x.shape[0],) if st.x.dim() == 2 else ()
                st.outs = [None if (st.gated and i == 1) else torch.empty(shape + (m.n,), dtype=out_dtype, device=dev)
                           for i, m in enumerate(st.mats)]
        self._plan = None
        self._ws: Optional[torch.Tensor] = None
        self._batches = None
        self.device = dev

    def weight_bytes(self) -> int:
        return sum(m.nbytes() for st in self.stages for m in st.mats)

    def num_matrices(self) -> int:
        return sum(len(st.mats) for st in self.stages)

    # ---- executor 1: one launch per matrix
    def run_launches(self) -> None:
        if any(st.fused() for st in self.stages):
            raise ValueError("norm, gate and residual are fused in the persistent executor only")
        for st in self.stages:
            for m, y in zip(st.mats, st.outs):
                if st.x.dim() == 1:
                    q4_gemv(st.x, m.packed, m.scales, m.biases, out=y)
                else:
                    q4_gemm_small(st.x, m.packed, m.scales, m.biases, out=y)

    # ---- executor 2: one persistent launch for the whole chain
    def prepare_chain(self) -> None:
        if self._plan is None:
            self._plan = q4_chain_build(self.stages, self.out_dtype)
            self._ws = torch.zeros(q4_chain_workspace_bytes() // 4, dtype=torch.int32, device=self.device)

    def run_chain(self) -> None:
        self.prepare_chain()
        q4_chain_run(self._plan, self._ws)

    # ---- executor 3: all products at once, one launch per distinct k
    def prepare_batches(self) -> None:
        if self._batches is not None:
            return
        if any(st.fused() for st in self.stages):
            raise ValueError("norm, gate and residual are fused in the persistent executor only")

        def span(t: torch.Tensor):
            return t.data_ptr(), t.data_ptr() + t.numel() * t.element_size()

        outs = [span(y) for st in self.stages for y in st.outs if y is not None]
        by_k = {}
        for st in self.stages:
            if st.x.dim() != 2 or not 5 <= st.x.shape[0] <= 16:
                raise ValueError("the product batch takes x of 5..16 activation rows")
            lo, hi = span(st.x)
            if any(lo < b and a < hi for a, b in outs):
                raise ValueError("a stage reads an output of the chain: the batch runs every product at once")
            xs, mats, ys = by_k.setdefault(st.x.shape[-1], ([], [], []))
            for m, y in zip(st.mats, st.outs):
                xs.append(st.x)
                mats.append((m.packed, m.scales, m.biases))
                ys.append(y)
        self._batches = [q4_gemm_batch_build(*v) for _, v in sorted(by_k.items())]

    def run_batches(self) -> None:
        self.prepare_batches()
        for plan in self._batches:
            q4_gemm_batch_run(plan)

    def chain_status(self) -> int:
        """Device-side status word of the persistent executor (0 = ok)."""
        self.prepare_chain()
        return int(self._ws[0].item())
