"""A decoder's split operators placed across pinned host memory and HBM by the
planner, and one decode step over them.

DAK paper §3 (Overview, Fig. 4): the global offload ratio follows from the
footprint and the HBM capacity; the planner of §4.2.2 turns it into per-op
ratios; each op's weights (tile-rows) or KV cache (requests) are then stored
across the two tiers and the split kernels run over them.  The walkthrough's
capacity section gives x_global >= max(0, (M - H) / M).

Per layer the step runs QKV (split GEMM), decode attention (split KV), O,
gate+up and down (split GEMMs) with N = batch activations.  Norms, rotary
embeddings, activation functions and residual adds are not part of the split
operators and are left out; every op reads fixed synthetic activations of its
shape (the layers are not chained), so the step measures exactly the bytes the
split operators read.

Weights ~ N(0, 0.02) and KV ~ N(0, 1) are generated on the GPU with a seeded
device generator, in chunks (HBM is nearly full): fp32 normals, scaled, rounded
to bf16.  With FP8 weights (the pages run their models in FP8), each weight is
an e4m3 code of N(0, 1) / 16 (cast by torch, round to nearest even) and every
row's scale is 0.02 * 16, so the logical weights are again ~N(0, 0.02); a
tile-row then holds m * K bytes.  The KV cache's host units are whole requests
or, with kv_unit = KV_UNIT_HEAD, single (request, KV head) pairs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch

from . import Op, SplitKV, SplitMatrix, op_time, plan_offload, plan_uniform, min_offload_ratio, splitk_decode_attn
from . import splitk_gemm
from . import KV_UNIT_HEAD, KV_UNIT_REQUEST, SplitMatrixFP8, decode_attn_workspace_bytes, splitk_gemm_fp8


@dataclass(frozen=True)
class DecoderShape:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    layers: int

    def linears(self):
        """(name, M, K) of the decode linears (QKV and gate+up fused)."""
        qkv = (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim
        return [("qkv", qkv, self.hidden), ("o", self.hidden, self.n_q_heads * self.head_dim),
                ("gate_up", 2 * self.ffn, self.hidden), ("down", self.hidden, self.ffn)]


LLAMA70B = DecoderShape(hidden=8192, n_q_heads=64, n_kv_heads=8, head_dim=128, ffn=28672, layers=80)
LLAMA8B = DecoderShape(hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=14336, layers=32)
LLAMA8B_ONE_LAYER = DecoderShape(hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=14336, layers=1)


@dataclass
class OpSlot:
    layer: int
    kind: str              # qkv, attn, o, gate_up, down
    units: int
    unit_bytes: int
    host_units: int = 0
    tensors: dict = field(default_factory=dict)
    desc: object = None

    @property
    def bytes(self):
        return self.units * self.unit_bytes


def _fill_normal_(t: torch.Tensor, std: float, gen: torch.Generator, stage: torch.Tensor):
    """Fill a bf16 tensor (device or pinned host) with std * N(0, 1), or a
    uint8 tensor with the e4m3 codes of std * N(0, 1), one staging-buffer chunk
    at a time (fp32 normals drawn into `stage`, scaled, rounded by the cast)."""
    flat = t.view(-1)
    n = flat.numel()
    chunk = stage.numel()
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        v = stage[:m]
        torch.randn((m,), generator=gen, out=v)
        if std != 1.0:
            v.mul_(std)
        if t.dtype == torch.uint8:
            flat[i:i + m].copy_(v.to(torch.float8_e4m3fn).view(torch.uint8))
        else:
            flat[i:i + m].copy_(v)


class DecodeModel:
    """Weights and KV of a decoder spread over two tiers by the greedy planner."""

    def __init__(self, shape: DecoderShape, batch: int, ctx: int, b_hbm: float, b_host: float,
                 hbm_bytes: int, m: int = 64, seed: int = 0, t_comp=None, log=print,
                 x_global: Optional[float] = None, policy: str = "greedy", weights: str = "bf16",
                 kv_unit: int = KV_UNIT_REQUEST):
        if weights not in ("bf16", "fp8"):
            raise ValueError("weights must be 'bf16' or 'fp8'")
        if kv_unit not in (KV_UNIT_REQUEST, KV_UNIT_HEAD):
            raise ValueError("kv_unit must be KV_UNIT_REQUEST or KV_UNIT_HEAD")
        self.shape, self.batch, self.ctx, self.m = shape, batch, ctx, m
        self.b_hbm, self.b_host = b_hbm, b_host
        self.weights, self.kv_unit = weights, kv_unit
        s = shape
        kv_req = 2 * s.n_kv_heads * ctx * s.head_dim * 2       # K and V of one request, one layer
        attn_units = batch if kv_unit == KV_UNIT_REQUEST else batch * s.n_kv_heads
        wbytes = 1 if weights == "fp8" else 2
        self.slots: List[OpSlot] = []
        lin = s.linears()
        for layer in range(s.layers):
            for name, M, K in lin:
                if name == "o":
                    self.slots.append(OpSlot(layer, "attn", attn_units, kv_req * batch // attn_units))
                self.slots.append(OpSlot(layer, name, M // m, m * K * wbytes))
        # order within a layer: qkv, attn, o, gate_up, down
        self.footprint = sum(o.bytes for o in self.slots)
        self.hbm_bytes = hbm_bytes
        self.x_global = min_offload_ratio(self.footprint, hbm_bytes) if x_global is None else float(x_global)
        tc = t_comp or (lambda slot: 0.0)
        self.t_comp = [float(tc(o)) for o in self.slots]
        ops = [Op(o.units, o.unit_bytes, t) for o, t in zip(self.slots, self.t_comp)]
        self._ops = ops
        if policy == "greedy":
            # DAK §4.2.2: the greedy per-op ratios under the global budget.
            self.host_units, self.modeled_s = plan_offload(ops, b_hbm, b_host, self.x_global)
        elif policy == "uniform":
            # Every op at the global ratio (the baseline the pages' greedy
            # planner is measured against).
            self.host_units, self.modeled_s = plan_uniform(ops, b_hbm, b_host, self.x_global)
        else:
            raise ValueError("policy must be 'greedy' or 'uniform'")
        self.policy = policy
        for o, h in zip(self.slots, self.host_units):
            o.host_units = h
        self.host_bytes = sum(o.host_units * o.unit_bytes for o in self.slots)
        log(f"footprint {self.footprint / 2**30:.2f} GiB, HBM budget {hbm_bytes / 2**30:.2f} GiB, "
            f"x_global {self.x_global:.5f}, host {self.host_bytes / 2**30:.3f} GiB, "
            f"modelled step {self.modeled_s * 1e3:.3f} ms")
        self._allocate(seed, log)

    # ------------------------------------------------------------------
    def _allocate(self, seed: int, log):
        """Allocate every op's two tiers first, then fill them through one
        staging buffer (interleaving temporaries with the large allocations
        fragments a nearly full HBM)."""
        s = self.shape
        dev = torch.device("cuda")
        gen = torch.Generator(device="cuda").manual_seed(seed)
        stage = torch.empty((1 << 26,), dtype=torch.float32, device=dev)
        lin = {name: (M, K) for name, M, K in s.linears()}
        fills = []
        fp8 = self.weights == "fp8"
        wdt = torch.uint8 if fp8 else torch.bfloat16
        scales = {}
        for i, o in enumerate(self.slots):
            if o.kind == "attn":
                # unit blocks [ctx, D] in (request, KV head) order either way
                shp = (self.ctx, s.head_dim)
                units = self.batch * s.n_kv_heads
                hu = o.host_units * (s.n_kv_heads if self.kv_unit == KV_UNIT_REQUEST else 1)
                kh = vh = kg = vg = None
                if hu:
                    kh = torch.empty((hu,) + shp, dtype=torch.bfloat16, pin_memory=True)
                    vh = torch.empty((hu,) + shp, dtype=torch.bfloat16, pin_memory=True)
                if hu < units:
                    kg = torch.empty((units - hu,) + shp, dtype=torch.bfloat16, device=dev)
                    vg = torch.empty((units - hu,) + shp, dtype=torch.bfloat16, device=dev)
                fills += [(t, 1.0) for t in (kh, vh, kg, vg) if t is not None]
                o.desc = SplitKV(kh, vh, kg, vg, self.batch, o.host_units, s.n_kv_heads, s.head_dim, self.ctx,
                                 self.kv_unit)
            else:
                M, K = lin[o.kind]
                rows = o.host_units * self.m
                ah = ag = None
                if rows:
                    ah = torch.empty((rows, K), dtype=wdt, pin_memory=True)
                if rows < M:
                    ag = torch.empty((M - rows, K), dtype=wdt, device=dev)
                # FP8: codes of N(0, 1) / 16 (well inside e4m3's range), row scale 0.02 * 16
                fills += [(t, 1.0 / 16 if fp8 else 0.02) for t in (ah, ag) if t is not None]
                if fp8:
                    if M not in scales:
                        scales[M] = torch.full((M,), 0.02 * 16, dtype=torch.float32, device=dev)
                    o.desc = SplitMatrixFP8(ah, ag, scales[M], M, K, self.m, o.host_units)
                else:
                    o.desc = SplitMatrix(ah, ag, M, K, self.m, o.host_units)
        log(f"  allocated {len(self.slots)} ops; filling {len(fills)} tensors")
        for i, (t, std) in enumerate(fills):
            _fill_normal_(t, std, gen, stage)
            if i % 100 == 0:
                log(f"  filled {i + 1}/{len(fills)} tensors")
        del stage
        # activations, outputs and workspace shared by all layers
        self.x = {}
        self.y = {}
        for name, (M, K) in lin.items():
            self.x[name] = (torch.randn((self.batch, K), generator=gen, device=dev) * 1.0).to(torch.bfloat16)
            self.y[name] = torch.empty((self.batch, M), dtype=torch.float32, device=dev)
        self.q = torch.randn((self.batch, s.n_q_heads, s.head_dim), generator=gen, device=dev).to(torch.bfloat16)
        self.out = torch.empty((self.batch, s.n_q_heads, s.head_dim), dtype=torch.float32, device=dev)
        attn0 = next(o for o in self.slots if o.kind == "attn")
        self.ws = torch.empty((decode_attn_workspace_bytes(attn0.desc, s.n_q_heads),), dtype=torch.uint8,
                              device=dev)
        self.scale = 1.0 / math.sqrt(s.head_dim)
        torch.cuda.synchronize()

    # ------------------------------------------------------------------
    def run_op(self, i: int):
        """Launch op i alone; its output lands in self.out (attention) or
        self.y[kind] (the GEMMs), which every layer's op of that kind shares."""
        o = self.slots[i]
        if o.kind == "attn":
            splitk_decode_attn(self.q, o.desc, self.scale, out=self.out, ws=self.ws)
        elif self.weights == "fp8":
            splitk_gemm_fp8(o.desc, self.x[o.kind], y=self.y[o.kind])
        else:
            splitk_gemm(o.desc, self.x[o.kind], y=self.y[o.kind])

    def step(self, events=None):
        """One decode step: every layer's five split operators, in order."""
        for i in range(len(self.slots)):
            if events is not None:
                events[i][0].record()
            self.run_op(i)
            if events is not None:
                events[i][1].record()

    def weight_rows(self, i: int, rows):
        """Rows `rows` of GEMM op i's logical weight matrix, read back from
        whichever tier holds each, as a CPU tensor (bf16, or uint8 e4m3
        codes), with the rows' fp32 scales for FP8 weights (else None)."""
        o = self.slots[i]
        d = o.desc
        split = d.h * d.m
        rows = [int(r) for r in rows]
        idx_h = [r for r in rows if r < split]
        idx_g = [r - split for r in rows if r >= split]
        parts = {}
        if idx_h:
            parts.update(zip(idx_h, d.host[torch.tensor(idx_h)]))
        if idx_g:
            got = d.hbm[torch.tensor(idx_g, device=d.hbm.device)].cpu()
            parts.update(zip([r + split for r in idx_g], got))
        out = torch.stack([parts[r] for r in rows])
        scale = d.row_scale[torch.tensor(rows, device=d.row_scale.device)].cpu() if self.weights == "fp8" else None
        return out, scale

    def kv_block(self, i: int, b: int, g: int):
        """(K, V) [ctx, head_dim] bf16 of request b's KV head g in attention
        op i, read back from whichever tier holds that unit."""
        d = self.slots[i].desc
        u = b * self.shape.n_kv_heads + g
        hu = d.host_units
        if u < hu:
            return d.k_host[u].clone(), d.v_host[u].clone()
        return d.k_hbm[u - hu].cpu(), d.v_hbm[u - hu].cpu()

    def op_model_s(self, i: int) -> float:
        """Modelled time of op i at its planned host units (the library's T_i(h))."""
        return op_time(self._ops[i], self.slots[i].host_units, self.b_hbm, self.b_host)
