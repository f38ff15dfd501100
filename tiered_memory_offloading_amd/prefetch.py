"""Copy-based offloading: the baseline the direct-access split operators are
measured against.

DAK paper §2.3 "Limitation of Copy-Based Offloading" and Fig. 2, the
walkthrough's section on the prefetch path's three hidden costs, and BOOST
§2.5 "Page Migration Schemes" describe it: data kept in host memory is copied
over the link into an HBM staging buffer ahead of its use, and the kernel then
reads it from HBM.  Here each op's host units are copied one op ahead of their
use (a double-buffered, layer-ahead prefetcher: while op i runs, the host
units of the next op with any are copied), by the DMA engine (hipMemcpyAsync
from pinned memory) on a copy stream of their own at the default priority.
The op then runs entirely from HBM: the same split kernels, with the host part
marked as a staged device copy (DAK_FLAG_STAGED_HOST), so every output is
bit-identical to the direct split at the same placement.

The costs the pages name are all present and measurable here:
  * the staging buffer holds `depth` slots of the largest op's host part in
    HBM, capacity the direct split leaves to weights and KV;
  * every offloaded byte is written into HBM by the copy and read back by the
    kernel, and the copy's writes compete with the kernels' reads (see
    probe_copy_interference);
  * an op waits for its copy whenever the copy outlasts the op before it (a
    pipeline bubble), and the first copy of a step has nothing to hide behind
    unless steps run back to back.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, List, Optional, Sequence, Tuple, Union

import torch

from . import LaunchConfig, SplitKV, SplitMatrix, SplitMatrixFP8

Operand = Union[SplitMatrix, SplitMatrixFP8, SplitKV]
Launch = Callable[[Operand, Optional[LaunchConfig]], object]


def host_part_bytes(op: Operand) -> int:
    """Bytes of an operand's host part (both K and V for a KV cache)."""
    return int(op.host_bytes)


def _host_sources(op: Operand) -> List[torch.Tensor]:
    """Flat views of exactly the host bytes the operand's descriptor names."""
    if isinstance(op, SplitKV):
        n = op.host_units * op.ctx * op.head_dim
        return [op.k_host.reshape(-1)[:n], op.v_host.reshape(-1)[:n]]
    n = op.h * op.m * op.K
    return [op.host.reshape(-1)[:n]]


def _staged(op: Operand, views: List[torch.Tensor]) -> Operand:
    """The operand with its host part replaced by staging-buffer views."""
    if isinstance(op, SplitKV):
        shp = (op.host_units, op.ctx, op.head_dim)
        return SplitKV(views[0].view(shp), views[1].view(shp), op.k_hbm, op.v_hbm, op.batch, op.h, op.n_kv_heads,
                       op.head_dim, op.ctx, op.unit, op.ctx_lens)
    rows = op.h * op.m
    if isinstance(op, SplitMatrixFP8):
        return SplitMatrixFP8(views[0].view(rows, op.K), op.hbm, op.row_scale, op.M, op.K, op.m, op.h)
    return SplitMatrix(views[0].view(rows, op.K), op.hbm, op.M, op.K, op.m, op.h)


def concurrent_copy_stream(compute_stream=None, device=None, tries: int = 12) -> torch.cuda.Stream:
    """A stream (default priority) whose host-to-device copies run beside the
    kernels of `compute_stream` (default: the current stream).

    HIP maps streams onto a few hardware queues per process (GPU_MAX_HW_QUEUES,
    4 on MI355X boxes), and two streams that share a queue run in order with
    each other: a copy stream on the compute stream's queue would make the
    prefetcher wait for every kernel and the kernels for every copy (measured:
    2 of 10 streams from torch's pool shared the default stream's queue).
    Candidates from the pool are tried with the library's copy-interference
    probe (a 16 MiB copy against 64 MiB reads) until one overlaps."""
    from . import probe_copy_interference
    device = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    compute_stream = compute_stream if compute_stream is not None else torch.cuda.current_stream(device)
    hbm = torch.empty(64 << 20, dtype=torch.uint8, device=device)
    src = torch.empty(16 << 20, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(16 << 20, dtype=torch.uint8, device=device)
    try:
        for _ in range(tries):
            cand = torch.cuda.Stream(device=device)
            if cand.cuda_stream == compute_stream.cuda_stream:
                continue
            _, _, _, n = probe_copy_interference(hbm, 512, 2, src, dst, reps=8, stream=compute_stream,
                                                 copy_stream=cand)
            if n > 0:
                return cand
    finally:
        del hbm, src, dst
    raise RuntimeError(f"no stream out of {tries} ran copies beside the compute stream")


@dataclass
class _Entry:
    op: Operand
    launch: Launch
    nbytes: int
    sources: List[torch.Tensor]


class PrefetchStep:
    """A sequence of split operators run the copy-based way.

    ops: (operand, launch) pairs in execution order; launch(operand, cfg)
    launches the op on the current stream with the given operand and launch
    configuration (for example ``lambda A, cfg: splitk_gemm(A, x, y=y,
    cfg=cfg)``).  depth: staging slots (2 = double buffering, copies one op
    ahead).  The staging buffer is allocated once here: depth slots of the
    largest host part, in HBM.  The ops run on the stream current at
    construction (step() switches to it), the copies on a stream checked to
    run beside it (concurrent_copy_stream), or on `copy_stream` if given."""

    def __init__(self, ops: Sequence[Tuple[Operand, Launch]], depth: int = 2, device=None,
                 copy_stream: Optional[torch.cuda.Stream] = None):
        if depth < 2:
            raise ValueError("depth must be at least 2 (one slot computing, one filling)")
        self.device = device if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.entries = [_Entry(op, fn, host_part_bytes(op), []) for op, fn in ops]
        for e in self.entries:
            e.sources = _host_sources(e.op) if e.nbytes else []
        self.depth = depth
        self.slot_bytes = max([e.nbytes for e in self.entries] + [16])
        self.slot_bytes = -(-self.slot_bytes // 256) * 256
        self.staging = torch.empty((depth, self.slot_bytes), dtype=torch.uint8, device=self.device)
        self.compute_stream = torch.cuda.current_stream(self.device)
        self.copy_stream = copy_stream if copy_stream is not None else concurrent_copy_stream(self.compute_stream,
                                                                                              self.device)
        self.ready = [torch.cuda.Event() for _ in range(depth)]
        self.free = [torch.cuda.Event() for _ in range(depth)]
        self.host_ops = [i for i, e in enumerate(self.entries) if e.nbytes]
        self._staged = {}
        for j, i in enumerate(self.host_ops):
            e = self.entries[i]
            views, off = [], 0
            for src in e.sources:
                n = src.numel() * src.element_size()
                views.append(self.staging[j % depth, off:off + n].view(src.dtype))
                off += n
            self._staged[i] = (_staged(e.op, views), views)
        self.cfg = LaunchConfig(staged_host=True)

    @property
    def staging_bytes(self) -> int:
        """HBM the staging buffer occupies."""
        return self.staging.numel()

    def _copy(self, j: int) -> None:
        i = self.host_ops[j]
        slot = j % self.depth
        _, views = self._staged[i]
        with torch.cuda.stream(self.copy_stream):
            self.copy_stream.wait_event(self.free[slot])      # the op that last used the slot is done
            for dst, src in zip(views, self.entries[i].sources):
                dst.copy_(src, non_blocking=True)             # pinned -> HBM, DMA engine
            self.ready[slot].record(self.copy_stream)

    def step(self) -> None:
        """One pass over the ops on the compute stream."""
        with torch.cuda.stream(self.compute_stream):
            self._step()

    def _step(self) -> None:
        cur = self.compute_stream
        ahead = self.depth - 1
        for j in range(min(ahead, len(self.host_ops))):
            self._copy(j)
        j = 0
        for i, e in enumerate(self.entries):
            if not e.nbytes:
                e.launch(e.op, None)
                continue
            if j + ahead < len(self.host_ops):
                self._copy(j + ahead)
            slot = j % self.depth
            cur.wait_event(self.ready[slot])
            e.launch(self._staged[i][0], self.cfg)
            self.free[slot].record(cur)
            j += 1
