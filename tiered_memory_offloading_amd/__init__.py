"""Direct-access split operators over pinned host memory and HBM on MI355X.

Python binding of libdak.so (include/dak.h).  Every step of the split operators
runs in the library's HIP kernels; this module only marshals arguments and uses
PyTorch to allocate device and pinned host memory and to name streams.

Entry points (same names as the C ABI, without the ``dak_`` prefix):
  min_offload_ratio, plan_offload, plan_uniform, op_time, op_turning_points,
  host_workgroups, splitk_gemm, splitk_gemm_fp8, decode_attn_workspace_bytes,
  splitk_decode_attn, splitk_decode_attn_noalloc, paged_decode_attn, probe_read,
  probe_read_concurrent, probe_mfma.
Placement (DAK paper §4.1 "Data Partition"; §5 batch split of the KV cache):
  place_matrix, place_kv.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

from . import _lib as L

__all__ = [
    "DakError", "LaunchConfig", "SplitMatrix", "SplitKV", "Op",
    "min_offload_ratio", "plan_offload", "plan_uniform", "op_time", "op_turning_points", "host_workgroups",
    "place_matrix", "place_kv", "KV_UNIT_REQUEST", "KV_UNIT_HEAD", "splitk_gemm", "decode_attn_workspace_bytes",
    "SplitMatrixFP8", "place_matrix_fp8", "splitk_gemm_fp8",
    "splitk_decode_attn", "splitk_decode_attn_noalloc", "decode_attn_scratch_max_bytes",
    "PagedKV", "place_paged_kv", "paged_decode_attn_workspace_bytes", "paged_decode_attn",
    "probe_read", "probe_read_concurrent", "probe_copy_interference", "probe_mfma", "library",
    "FLAG_STAGED_HOST",
]


class DakError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"dak status {status}: {message}")
        self.status = status


def library() -> C.CDLL:
    return L.load()


def _check(status: int) -> None:
    if status != L.DAK_OK:
        lib = library()
        raise DakError(status, lib.dak_last_error().decode(errors="replace"))


def _stream_handle(stream) -> C.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return C.c_void_p(stream.cuda_stream)
    return C.c_void_p(int(stream))


# ----------------------------------------------------------------------------
# Planning (CPU)
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Op:
    units: int
    unit_bytes: int
    t_comp_s: float = 0.0


def min_offload_ratio(footprint_bytes: int, hbm_bytes: int) -> float:
    return library().dak_min_offload_ratio(int(footprint_bytes), int(hbm_bytes))


def plan_offload(ops: Sequence[Op], b_hbm: float, b_host: float, x_global: float):
    """(host units per op, modelled time in seconds)."""
    lib = library()
    arr = (L.OpDesc * len(ops))(*[L.OpDesc(o.units, o.unit_bytes, o.t_comp_s) for o in ops])
    out = (C.c_uint64 * len(ops))()
    t = C.c_double()
    _check(lib.dak_plan_offload(arr, len(ops), float(b_hbm), float(b_host), float(x_global), out, C.byref(t)))
    return [int(v) for v in out], t.value


def op_time(op: Op, h: int, b_hbm: float, b_host: float) -> float:
    """Modelled seconds of one op with h units on the host (the planner's T_i(h))."""
    d = L.OpDesc(op.units, op.unit_bytes, op.t_comp_s)
    t = C.c_double()
    _check(library().dak_op_time(C.byref(d), int(h), float(b_hbm), float(b_host), C.byref(t)))
    return t.value


def plan_uniform(ops: Sequence[Op], b_hbm: float, b_host: float, x: float):
    """(host units per op at one uniform ratio x, modelled time in seconds)."""
    lib = library()
    arr = (L.OpDesc * len(ops))(*[L.OpDesc(o.units, o.unit_bytes, o.t_comp_s) for o in ops])
    out = (C.c_uint64 * len(ops))()
    t = C.c_double()
    _check(lib.dak_plan_uniform(arr, len(ops), float(b_hbm), float(b_host), float(x), out, C.byref(t)))
    return [int(v) for v in out], t.value


def op_turning_points(op: Op, b_hbm: float, b_host: float):
    """(a, b, memory_bound) of one op."""
    lib = library()
    d = L.OpDesc(op.units, op.unit_bytes, op.t_comp_s)
    a, b, mb = C.c_uint64(), C.c_uint64(), C.c_int32()
    _check(lib.dak_op_turning_points(C.byref(d), float(b_hbm), float(b_host), C.byref(a), C.byref(b), C.byref(mb)))
    return a.value, b.value, bool(mb.value)


def host_workgroups(items: int, cap: int) -> int:
    return library().dak_host_workgroups(int(items), int(cap))


# ----------------------------------------------------------------------------
# Launch configuration
# ----------------------------------------------------------------------------
FLAG_STAGED_HOST = L.DAK_FLAG_STAGED_HOST


@dataclass
class LaunchConfig:
    host_cus: int = 0              # 0 = library default
    window: int = 0                # 0 = library default
    byte_counters: Optional[torch.Tensor] = None   # int64 [2] on the GPU: host, HBM bytes loaded
    staged_host: bool = False      # the host part is a device copy staged by a prefetcher
    record_xcc: bool = False       # N > 256: byte_counters[2 + q] gets host group q's XCD bit mask

    def as_c(self) -> L.LaunchCfg:
        flags = L.DAK_FLAG_STAGED_HOST if self.staged_host else 0
        ptr = None
        if self.byte_counters is not None:
            t = self.byte_counters
            need = 2 + 256 if self.record_xcc else 2
            if t.dtype != torch.int64 or t.numel() < need or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"byte_counters must be a contiguous int64 CUDA tensor of {need} elements")
            flags |= L.DAK_FLAG_COUNT_BYTES
            if self.record_xcc:
                flags |= L.DAK_FLAG_RECORD_XCC
            ptr = t.data_ptr()
        elif self.record_xcc:
            raise ValueError("record_xcc needs byte_counters")
        return L.LaunchCfg(int(self.host_cus), int(self.window), flags, 0, ptr)


def _cfg_ptr(cfg: Optional[LaunchConfig]):
    if cfg is None:
        return None, None
    c = cfg.as_c()
    return c, C.byref(c)


def _check_buf(t: Optional[torch.Tensor], name: str, numel: int, dtype) -> None:
    """A descriptor's tensor must hold at least `numel` elements of `dtype`,
    contiguously.  The library checks each pointer's tier and that the bytes
    it needs lie inside the allocation holding the pointer; under PyTorch's
    caching allocator that allocation is a whole pool segment, so a short view
    would otherwise let a kernel read or write its neighbours."""
    if numel <= 0:
        return
    if t is None:
        raise ValueError(f"{name} is missing ({numel} elements needed)")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, not {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, {numel} needed")


# ----------------------------------------------------------------------------
# Placement (tile-rows and requests across the two tiers)
# ----------------------------------------------------------------------------
@dataclass
class SplitMatrix:
    """A [M, K] bf16 weight matrix whose first h tile-rows (of m rows) live in
    pinned host memory and the rest in HBM."""
    host: Optional[torch.Tensor]   # [h*m, K] bf16, pinned CPU
    hbm: Optional[torch.Tensor]    # [M - h*m, K] bf16, CUDA
    M: int
    K: int
    m: int
    h: int

    def desc(self) -> L.SplitMatrixDesc:
        hp = self.host.data_ptr() if self.host is not None and self.host.numel() else None
        gp = self.hbm.data_ptr() if self.hbm is not None and self.hbm.numel() else None
        return L.SplitMatrixDesc(hp, gp, self.M, self.K, self.m, 0, self.h)

    @property
    def host_bytes(self) -> int:
        return self.h * self.m * self.K * 2

    def check(self) -> None:
        """Both tiers hold the rows the descriptor names."""
        rows = self.h * self.m
        _check_buf(self.host, "A.host", rows * self.K, torch.bfloat16)
        _check_buf(self.hbm, "A.hbm", (self.M - rows) * self.K, torch.bfloat16)


def _pinned_like(n_rows: int, K: int) -> torch.Tensor:
    return torch.empty((n_rows, K), dtype=torch.bfloat16, pin_memory=True)


def place_matrix(A: torch.Tensor, m: int, h: int, device=None) -> SplitMatrix:
    """Copy tile-rows [0, h) of A into pinned host memory and the rest into HBM."""
    if A.dtype != torch.bfloat16 or A.dim() != 2:
        raise ValueError("A must be a 2-D bf16 tensor")
    M, K = A.shape
    if M % m or not (0 <= h <= M // m):
        raise ValueError("M must be a multiple of m and 0 <= h <= M/m")
    device = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    rows = h * m
    host = None
    if rows:
        host = _pinned_like(rows, K)
        host.copy_(A[:rows])
    hbm = None
    if rows < M:
        hbm = A[rows:].to(device, copy=True).contiguous()
    return SplitMatrix(host, hbm, M, K, m, h)


KV_UNIT_REQUEST = 0
KV_UNIT_HEAD = 1


@dataclass
class SplitKV:
    """KV caches of `batch` requests; the first h units (whole requests, or
    (request, KV head) pairs with unit=KV_UNIT_HEAD) in pinned host memory."""
    k_host: Optional[torch.Tensor]   # host units' [ctx, D] blocks in unit order, bf16 pinned
    v_host: Optional[torch.Tensor]
    k_hbm: Optional[torch.Tensor]    # the other units' blocks, bf16 CUDA
    v_hbm: Optional[torch.Tensor]
    batch: int
    h: int
    n_kv_heads: int
    head_dim: int
    ctx: int
    unit: int = KV_UNIT_REQUEST
    ctx_lens: Optional[torch.Tensor] = None   # int32 [batch] on the GPU: valid tokens per request

    def desc(self) -> L.SplitKVDesc:
        def p(t):
            return t.data_ptr() if t is not None and t.numel() else None
        return L.SplitKVDesc(p(self.k_host), p(self.v_host), p(self.k_hbm), p(self.v_hbm), self.batch, self.h,
                             self.n_kv_heads, self.head_dim, self.ctx, self.unit, 0, p(self.ctx_lens))

    @property
    def host_units(self) -> int:
        """Host units in (request, KV head) pairs."""
        return self.h * self.n_kv_heads if self.unit == KV_UNIT_REQUEST else self.h

    @property
    def host_bytes(self) -> int:
        """Bytes of K and V stored on the host."""
        return 2 * self.host_units * self.ctx * self.head_dim * 2

    def check(self) -> None:
        """Both tiers hold the unit blocks the descriptor names."""
        if self.unit not in (KV_UNIT_REQUEST, KV_UNIT_HEAD):
            return   # the library refuses the unit code itself
        units = self.batch * self.n_kv_heads
        blk = self.ctx * self.head_dim
        hu = self.host_units
        if not 0 <= hu <= units:
            raise ValueError(f"{hu} host units of {units}")
        for n, t in (("k_host", self.k_host), ("v_host", self.v_host)):
            _check_buf(t, n, hu * blk, torch.bfloat16)
        for n, t in (("k_hbm", self.k_hbm), ("v_hbm", self.v_hbm)):
            _check_buf(t, n, (units - hu) * blk, torch.bfloat16)
        if self.ctx_lens is not None:
            _check_buf(self.ctx_lens, "ctx_lens", self.batch, torch.int32)


def place_kv(K: torch.Tensor, V: torch.Tensor, h: int, device=None, unit: int = KV_UNIT_REQUEST,
             ctx_lens: Optional[torch.Tensor] = None) -> SplitKV:
    """Copy the first h units of K, V [B, Hkv, ctx, D] (requests, or (request,
    KV head) pairs with unit=KV_UNIT_HEAD) into pinned host memory and the rest
    into HBM.  ctx_lens: optional valid-token counts per request (any integer
    tensor of B entries)."""
    if K.shape != V.shape or K.dim() != 4 or K.dtype != torch.bfloat16 or V.dtype != torch.bfloat16:
        raise ValueError("K and V must be bf16 tensors of equal shape [B, Hkv, ctx, D]")
    B, Hkv, ctx, D = K.shape
    units = B if unit == KV_UNIT_REQUEST else B * Hkv
    if unit not in (KV_UNIT_REQUEST, KV_UNIT_HEAD) or not 0 <= h <= units:
        raise ValueError("unit must be KV_UNIT_REQUEST or KV_UNIT_HEAD, with 0 <= h <= its unit count")
    device = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    hu = h * Hkv if unit == KV_UNIT_REQUEST else h
    Kf, Vf = K.reshape(B * Hkv, ctx, D), V.reshape(B * Hkv, ctx, D)
    kh = vh = kg = vg = None
    if hu:
        kh = torch.empty((hu, ctx, D), dtype=torch.bfloat16, pin_memory=True)
        vh = torch.empty((hu, ctx, D), dtype=torch.bfloat16, pin_memory=True)
        kh.copy_(Kf[:hu])
        vh.copy_(Vf[:hu])
    if hu < B * Hkv:
        kg = Kf[hu:].to(device, copy=True).contiguous()
        vg = Vf[hu:].to(device, copy=True).contiguous()
    lens = None if ctx_lens is None else ctx_lens.to(device=device, dtype=torch.int32).contiguous()
    return SplitKV(kh, vh, kg, vg, B, h, Hkv, D, ctx, unit, lens)


# ----------------------------------------------------------------------------
# Compute entry points
# ----------------------------------------------------------------------------
def _gemm_workspace(need: int, ws: Optional[torch.Tensor], device, stream) -> Optional[torch.Tensor]:
    # The K-split workspace of a tiled launch: the caller's, or one from
    # torch's allocator, kept alive for the stream the launch runs on.
    if need == 0:
        return None
    if ws is None:
        ws = torch.empty((need,), dtype=torch.uint8, device=device)
        if isinstance(stream, torch.cuda.Stream):
            ws.record_stream(stream)
        return ws
    if not ws.is_cuda or not ws.is_contiguous() or ws.numel() * ws.element_size() < need:
        raise ValueError(f"ws must be a contiguous CUDA tensor of at least {need} bytes")
    return ws


def splitk_gemm(A: SplitMatrix, x: torch.Tensor, y: Optional[torch.Tensor] = None,
                cfg: Optional[LaunchConfig] = None, stream=None, ws: Optional[torch.Tensor] = None,
                split: bool = True) -> torch.Tensor:
    """y[n, r] = sum_k A[r, k] x[n, k]; x bf16 [N, K] on the GPU, y fp32 [N, M].

    Shapes that the library splits along K (dak_splitk_gemm_workspace_bytes >
    0) get a workspace: `ws`, or one allocated here; split=False runs them
    unsplit (dak_splitk_gemm)."""
    lib = library()
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D bf16 CUDA tensor")
    N = x.shape[0]
    if x.shape[1] != A.K:
        raise ValueError(f"x has {x.shape[1]} columns, A has K = {A.K}")
    A.check()
    if y is None:
        y = torch.empty((N, A.M), dtype=torch.float32, device=x.device)
    if y.dtype != torch.float32 or not y.is_contiguous() or tuple(y.shape) != (N, A.M):
        raise ValueError("y must be a contiguous fp32 [N, M] tensor")
    d = A.desc()
    c, cp = _cfg_ptr(cfg)
    need = int(lib.dak_splitk_gemm_workspace_bytes(A.M, A.K, N)) if split else 0
    w = _gemm_workspace(need, ws, x.device, stream)
    _check(lib.dak_splitk_gemm_ws(C.byref(d), x.data_ptr(), N, y.data_ptr(), None if w is None else w.data_ptr(),
                                  need, cp, _stream_handle(stream)))
    return y


@dataclass
class SplitMatrixFP8:
    """A [M, K] matrix of FP8 (OCP E4M3) weight codes with one fp32 scale per
    row; tile-rows [0, h) of m rows in pinned host memory, the rest in HBM."""
    host: Optional[torch.Tensor]   # [h*m, K] uint8, pinned CPU
    hbm: Optional[torch.Tensor]    # [M - h*m, K] uint8, CUDA
    row_scale: torch.Tensor        # [M] fp32, CUDA
    M: int
    K: int
    m: int
    h: int

    def desc(self) -> L.SplitMatrixFP8Desc:
        hp = self.host.data_ptr() if self.host is not None and self.host.numel() else None
        gp = self.hbm.data_ptr() if self.hbm is not None and self.hbm.numel() else None
        return L.SplitMatrixFP8Desc(hp, gp, self.M, self.K, self.m, 0, self.h, self.row_scale.data_ptr())

    @property
    def host_bytes(self) -> int:
        return self.h * self.m * self.K

    def check(self) -> None:
        """Both tiers hold the code rows the descriptor names, and every row has a scale."""
        rows = self.h * self.m
        _check_buf(self.host, "A.host", rows * self.K, torch.uint8)
        _check_buf(self.hbm, "A.hbm", (self.M - rows) * self.K, torch.uint8)
        _check_buf(self.row_scale, "A.row_scale", self.M, torch.float32)


def place_matrix_fp8(codes: torch.Tensor, row_scale: torch.Tensor, m: int, h: int, device=None) -> SplitMatrixFP8:
    """Copy tile-rows [0, h) of the e4m3 codes [M, K] (uint8, or a
    float8_e4m3fn tensor) into pinned host memory and the rest into HBM; the
    per-row scales [M] go to HBM as fp32."""
    if codes.dtype == torch.float8_e4m3fn:
        codes = codes.view(torch.uint8)
    if codes.dtype != torch.uint8 or codes.dim() != 2:
        raise ValueError("codes must be a 2-D uint8 (or float8_e4m3fn) tensor")
    M, K = codes.shape
    if M % m or not (0 <= h <= M // m):
        raise ValueError("M must be a multiple of m and 0 <= h <= M/m")
    if row_scale.numel() != M:
        raise ValueError("one scale per row")
    device = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    rows = h * m
    host = None
    if rows:
        host = torch.empty((rows, K), dtype=torch.uint8, pin_memory=True)
        host.copy_(codes[:rows])
    hbm = None
    if rows < M:
        hbm = codes[rows:].to(device, copy=True).contiguous()
    scale = row_scale.detach().to(device=device, dtype=torch.float32).contiguous()
    return SplitMatrixFP8(host, hbm, scale, M, K, m, h)


def splitk_gemm_fp8(A: SplitMatrixFP8, x: torch.Tensor, y: Optional[torch.Tensor] = None,
                    cfg: Optional[LaunchConfig] = None, stream=None, ws: Optional[torch.Tensor] = None,
                    split: bool = True) -> torch.Tensor:
    """y[n, r] = row_scale[r] * sum_k e4m3(A[r, k]) x[n, k]; x bf16 [N, K] on
    the GPU (N <= 2048; N > 64 takes the compute-bound tiled kernel), y fp32
    [N, M]."""
    lib = library()
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D bf16 CUDA tensor")
    N = x.shape[0]
    if x.shape[1] != A.K:
        raise ValueError(f"x has {x.shape[1]} columns, A has K = {A.K}")
    A.check()
    if y is None:
        y = torch.empty((N, A.M), dtype=torch.float32, device=x.device)
    if y.dtype != torch.float32 or not y.is_contiguous() or tuple(y.shape) != (N, A.M):
        raise ValueError("y must be a contiguous fp32 [N, M] tensor")
    d = A.desc()
    c, cp = _cfg_ptr(cfg)
    need = int(lib.dak_splitk_gemm_fp8_workspace_bytes(A.M, A.K, N)) if split else 0
    w = _gemm_workspace(need, ws, x.device, stream)
    _check(lib.dak_splitk_gemm_fp8_ws(C.byref(d), x.data_ptr(), N, y.data_ptr(),
                                      None if w is None else w.data_ptr(), need, cp, _stream_handle(stream)))
    return y


def decode_attn_workspace_bytes(kv: SplitKV, n_q_heads: int) -> int:
    d = kv.desc()
    return int(library().dak_decode_attn_workspace_bytes(C.byref(d), int(n_q_heads)))


def _check_q(q: torch.Tensor, batch: int, n_kv_heads: int, head_dim: int) -> None:
    if q.dtype != torch.bfloat16 or q.dim() != 3 or not q.is_cuda or not q.is_contiguous():
        raise ValueError("q must be a contiguous bf16 CUDA tensor [B, Hq, D]")
    B, Hq, D = q.shape
    if B != batch or D != head_dim or Hq % n_kv_heads:
        raise ValueError(f"q is {tuple(q.shape)}; the KV cache needs [{batch}, a multiple of {n_kv_heads}, {head_dim}]")


def _check_attn_buffers(q: torch.Tensor, out: torch.Tensor, ws: Optional[torch.Tensor], need: int) -> None:
    # The library checks that each buffer lies in a device allocation of the
    # size it needs, but it sees a base pointer, not a view's strides or size.
    B, Hq, D = q.shape
    if out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != (B, Hq, D) or not out.is_cuda:
        raise ValueError("out must be a contiguous fp32 CUDA tensor [B, Hq, D]")
    if ws is not None:
        if not ws.is_contiguous() or not ws.is_cuda:
            raise ValueError("ws must be a contiguous CUDA tensor")
        if ws.numel() * ws.element_size() < need:
            raise ValueError(f"ws holds {ws.numel() * ws.element_size()} bytes, {need} needed")


def splitk_decode_attn(q: torch.Tensor, kv: SplitKV, scale: float, out: Optional[torch.Tensor] = None,
                       ws: Optional[torch.Tensor] = None, cfg: Optional[LaunchConfig] = None,
                       stream=None) -> torch.Tensor:
    """out [B, Hq, D] fp32 from q bf16 [B, Hq, D] on the GPU."""
    lib = library()
    _check_q(q, kv.batch, kv.n_kv_heads, kv.head_dim)
    kv.check()
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    need = decode_attn_workspace_bytes(kv, Hq)
    if ws is None:
        ws = torch.empty((max(need, 16),), dtype=torch.uint8, device=q.device)
    _check_attn_buffers(q, out, ws, need)
    d = kv.desc()
    c, cp = _cfg_ptr(cfg)
    _check(lib.dak_splitk_decode_attn(q.data_ptr(), C.byref(d), Hq, C.c_float(scale), out.data_ptr(),
                                      ws.data_ptr(), ws.numel() * ws.element_size(), cp, _stream_handle(stream)))
    return out


def decode_attn_scratch_max_bytes() -> int:
    """Bytes of the per-device array splitk_decode_attn_noalloc works in."""
    return int(library().dak_decode_attn_scratch_max_bytes())


def splitk_decode_attn_noalloc(q: torch.Tensor, kv: SplitKV, scale: float, out: torch.Tensor,
                               cfg: Optional[LaunchConfig] = None, stream=None) -> torch.Tensor:
    """splitk_decode_attn for callers that cannot allocate: the caller passes
    `out`, and the workspace is the library's fixed per-device array (calls
    that overlap on one device race on it)."""
    lib = library()
    _check_q(q, kv.batch, kv.n_kv_heads, kv.head_dim)
    kv.check()
    _check_attn_buffers(q, out, None, 0)
    d = kv.desc()
    c, cp = _cfg_ptr(cfg)
    _check(lib.dak_splitk_decode_attn_noalloc(q.data_ptr(), C.byref(d), q.shape[1], C.c_float(scale),
                                              out.data_ptr(), cp, _stream_handle(stream)))
    return out


@dataclass
class PagedKV:
    """A paged KV cache: pages of `page` tokens of one (request, KV head) unit
    in a host pool (pinned) and an HBM pool; page_table [units, max_pages]
    gives each unit's pages in its tier's pool, unit_order lists the host units
    first (n_host_units of them)."""
    k_host: Optional[torch.Tensor]   # [host_pages, page, D] bf16 pinned
    v_host: Optional[torch.Tensor]
    k_hbm: Optional[torch.Tensor]    # [hbm_pages, page, D] bf16 CUDA
    v_hbm: Optional[torch.Tensor]
    page_table: torch.Tensor         # int32 [B * Hkv, max_pages] CUDA
    ctx_lens: torch.Tensor           # int32 [B] CUDA
    unit_order: torch.Tensor         # int32 [B * Hkv] CUDA
    batch: int
    n_kv_heads: int
    head_dim: int
    page: int
    n_host_units: int

    @property
    def max_pages(self) -> int:
        return self.page_table.shape[1]

    @property
    def host_pages(self) -> int:
        return 0 if self.k_host is None else self.k_host.shape[0]

    @property
    def hbm_pages(self) -> int:
        return 0 if self.k_hbm is None else self.k_hbm.shape[0]

    @property
    def host_bytes(self) -> int:
        return 2 * self.host_pages * self.page * self.head_dim * 2

    def check(self) -> None:
        """Pools, page table, lengths and unit order have the shapes the
        descriptor names (their contents are checked by the kernel)."""
        units = self.batch * self.n_kv_heads
        for n, t in (("k_host", self.k_host), ("v_host", self.v_host), ("k_hbm", self.k_hbm),
                     ("v_hbm", self.v_hbm)):
            if t is not None:
                # the descriptor takes the pool's page count from its first dimension
                if t.dim() != 3:
                    raise ValueError(f"{n} must be [pages, page, head_dim]")
                _check_buf(t, n, t.shape[0] * self.page * self.head_dim, torch.bfloat16)
        if (self.k_host is None) != (self.v_host is None) or (self.k_hbm is None) != (self.v_hbm is None):
            raise ValueError("K and V pools must come in pairs")
        for a, b in ((self.k_host, self.v_host), (self.k_hbm, self.v_hbm)):
            if a is not None and a.shape != b.shape:
                raise ValueError("K and V pools of a tier must have equal shapes")
        if self.page_table.dim() != 2 or self.page_table.shape[0] != units:
            raise ValueError(f"page_table must be [{units}, max_pages]")
        _check_buf(self.page_table, "page_table", self.page_table.numel(), torch.int32)
        _check_buf(self.ctx_lens, "ctx_lens", self.batch, torch.int32)
        if self.unit_order.numel() != units:
            raise ValueError(f"unit_order must hold {units} entries")
        _check_buf(self.unit_order, "unit_order", units, torch.int32)

    def desc(self) -> L.PagedKVDesc:
        def p(t):
            return t.data_ptr() if t is not None and t.numel() else None
        return L.PagedKVDesc(p(self.k_host), p(self.v_host), p(self.k_hbm), p(self.v_hbm), self.host_pages,
                             self.hbm_pages, self.batch, self.n_kv_heads, self.head_dim, self.page, self.max_pages,
                             p(self.page_table), p(self.ctx_lens), p(self.unit_order), self.n_host_units)


def place_paged_kv(K: torch.Tensor, V: torch.Tensor, ctx_lens, page: int, host_units=(), seed: Optional[int] = None,
                   device=None) -> PagedKV:
    """Page K, V [B, Hkv, ctx, D] into two pools.  Unit u = b * Hkv + g is a
    host unit iff u is in host_units; each unit gets ceil(len_b / page) pages
    of its tier's pool (len_b = ctx_lens[b] clamped to [0, ctx]).  With a seed
    the pages' pool indices are a seeded random permutation (a pool after
    churn), otherwise they are in unit order."""
    if K.shape != V.shape or K.dim() != 4 or K.dtype != torch.bfloat16 or V.dtype != torch.bfloat16:
        raise ValueError("K and V must be bf16 tensors of equal shape [B, Hkv, ctx, D]")
    if page < 16 or page & (page - 1):
        raise ValueError("page must be a power of two >= 16")
    B, Hkv, ctx, D = K.shape
    units = B * Hkv
    device = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    lens = [min(max(int(v), 0), ctx) for v in torch.as_tensor(ctx_lens).tolist()]
    if len(lens) != B:
        raise ValueError("ctx_lens needs one entry per request")
    host = sorted(set(int(u) for u in host_units))
    if any(not 0 <= u < units for u in host):
        raise ValueError("host unit out of range")
    hs = set(host)
    order = host + [u for u in range(units) if u not in hs]
    max_pages = max(1, -(-ctx // page))
    table = torch.full((units, max_pages), -1, dtype=torch.int32)
    padded = max_pages * page
    Kf, Vf = K.reshape(units, ctx, D), V.reshape(units, ctx, D)
    gen = None
    if seed is not None:
        gen = torch.Generator().manual_seed(seed)
    pools = []
    for tier_units, pinned in ((host, True), ([u for u in range(units) if u not in hs], False)):
        pairs = [(u, i) for u in tier_units for i in range(-(-lens[u // Hkv] // page))]
        n = len(pairs)
        if n == 0:
            pools.append((None, None))
            continue
        idx = torch.randperm(n, generator=gen) if gen is not None else torch.arange(n)
        uu = torch.tensor([u for u, _ in pairs])
        ii = torch.tensor([i for _, i in pairs])
        table[uu, ii] = idx.to(torch.int32)
        kp, vp = [], []
        for src in (Kf, Vf):
            s = src.to(device)
            if padded != ctx:
                s = torch.nn.functional.pad(s, (0, 0, 0, padded - ctx))
            s = s.reshape(units, max_pages, page, D)
            pool = torch.empty((n, page, D), dtype=torch.bfloat16, device=device)
            pool[idx.to(device)] = s[uu.to(device), ii.to(device)]
            if pinned:
                ph = torch.empty((n, page, D), dtype=torch.bfloat16, pin_memory=True)
                ph.copy_(pool)
                pool = ph
            (kp if src is Kf else vp).append(pool)
        pools.append((kp[0], vp[0]))
    (kh, vh), (kg, vg) = pools
    return PagedKV(kh, vh, kg, vg, table.to(device), torch.tensor(lens, dtype=torch.int32, device=device),
                   torch.tensor(order, dtype=torch.int32, device=device), B, Hkv, D, page, len(host))


def paged_decode_attn_workspace_bytes(kv: PagedKV, n_q_heads: int) -> int:
    d = kv.desc()
    return int(library().dak_paged_decode_attn_workspace_bytes(C.byref(d), int(n_q_heads)))


def paged_decode_attn(q: torch.Tensor, kv: PagedKV, scale: float, out: Optional[torch.Tensor] = None,
                      ws: Optional[torch.Tensor] = None, cfg: Optional[LaunchConfig] = None,
                      stream=None) -> torch.Tensor:
    """out [B, Hq, D] fp32 from q bf16 [B, Hq, D] over a paged split KV cache."""
    lib = library()
    _check_q(q, kv.batch, kv.n_kv_heads, kv.head_dim)
    kv.check()
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    need = paged_decode_attn_workspace_bytes(kv, Hq)
    if ws is None:
        ws = torch.empty((max(need, 16),), dtype=torch.uint8, device=q.device)
    _check_attn_buffers(q, out, ws, need)
    d = kv.desc()
    c, cp = _cfg_ptr(cfg)
    _check(lib.dak_paged_decode_attn(q.data_ptr(), C.byref(d), Hq, C.c_float(scale), out.data_ptr(),
                                     ws.data_ptr(), ws.numel() * ws.element_size(), cp, _stream_handle(stream)))
    return out


# ----------------------------------------------------------------------------
# Probes
# ----------------------------------------------------------------------------
def probe_read(buf: torch.Tensor, workgroups: int, window: int, reps: int = 5, nbytes: Optional[int] = None,
               stream=None) -> float:
    """Median milliseconds to stream `nbytes` (default: all of buf)."""
    lib = library()
    nb = buf.numel() * buf.element_size() if nbytes is None else int(nbytes)
    ms = C.c_float()
    _check(lib.dak_probe_read(buf.data_ptr(), nb, int(workgroups), int(window), int(reps), _stream_handle(stream),
                              C.byref(ms)))
    return ms.value


def probe_mfma(workgroups: int = 1024, iters: int = 4096, reps: int = 5, stream=None):
    """(median ms, TFLOP/s) of the matrix-core peak probe."""
    lib = library()
    ms, tf = C.c_float(), C.c_double()
    _check(lib.dak_probe_mfma(int(workgroups), int(iters), int(reps), _stream_handle(stream), C.byref(ms),
                              C.byref(tf)))
    return ms.value, tf.value


def probe_copy_interference(hbm: torch.Tensor, workgroups: int, window: int, host_src: torch.Tensor,
                            dev_dst: torch.Tensor, reps: int = 24, stream=None, copy_stream=None):
    """(ms of the HBM read alone, ms beside a host-to-HBM copy of host_src into
    dev_dst, ms of the copy, reads that overlapped the copy)."""
    lib = library()
    nb = host_src.numel() * host_src.element_size()
    if dev_dst.numel() * dev_dst.element_size() < nb:
        raise ValueError("dev_dst is smaller than host_src")
    if copy_stream is None:
        raise ValueError("copy_stream: the copy needs a stream of its own")
    a, w, c, n = C.c_float(), C.c_float(), C.c_float(), C.c_int32()
    _check(lib.dak_probe_copy_interference(hbm.data_ptr(), hbm.numel() * hbm.element_size(), int(workgroups),
                                           int(window), host_src.data_ptr(), dev_dst.data_ptr(), nb, int(reps),
                                           _stream_handle(stream), _stream_handle(copy_stream), C.byref(a),
                                           C.byref(w), C.byref(c), C.byref(n)))
    return a.value, w.value, c.value, n.value


def probe_read_concurrent(hbm: torch.Tensor, hbm_wgs: int, hbm_window: int, host: torch.Tensor, host_wgs: int,
                          host_window: int, hbm_bytes: Optional[int] = None, host_bytes: Optional[int] = None,
                          stream=None):
    """(ms total, ms of the HBM role, ms of the host role) of one concurrent launch."""
    lib = library()
    gb = hbm.numel() * hbm.element_size() if hbm_bytes is None else int(hbm_bytes)
    hb = host.numel() * host.element_size() if host_bytes is None else int(host_bytes)
    t, g, h = C.c_float(), C.c_float(), C.c_float()
    _check(lib.dak_probe_read_concurrent(hbm.data_ptr(), gb, int(hbm_wgs), int(hbm_window), host.data_ptr(), hb,
                                         int(host_wgs), int(host_window), _stream_handle(stream), C.byref(t),
                                         C.byref(g), C.byref(h)))
    return t.value, g.value, h.value
