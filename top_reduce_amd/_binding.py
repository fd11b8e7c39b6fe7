"""ctypes binding of libtopreduce.so (C ABI in include/topreduce.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, and their device pointers plus the current HIP stream are passed
to the library. The workspace is allocated here, by the caller side, as a
torch uint8 tensor; the library itself allocates nothing.
"""

from __future__ import annotations

import ctypes as C
import math
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libtopreduce.so"

ABI_VERSION = 5
BF16, F32 = 0, 1
IDX_I32, IDX_I64 = 0, 1
FLAG_GEMM_FORCE_TILED = 0x1
FLAG_GEMM_FORCE_STREAM = 0x2
FLAG_NO_XE = 0x4
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024

_STATUS = {0: "TR_OK", -1: "TR_EINVAL", -2: "TR_EUNSUPPORTED", -3: "TR_EWORKSPACE", -4: "TR_EHIP"}


class TopReduceError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class Desc(C.Structure):
    _fields_ = [("T", C.c_int64), ("K", C.c_int32), ("E", C.c_int32),
                ("expert_begin", C.c_int64), ("H", C.c_int64), ("I", C.c_int64),
                ("dtype", C.c_int32), ("idx_dtype", C.c_int32), ("flags", C.c_int32),
                ("reserved", C.c_int32)]


class PlanStruct(C.Structure):
    _fields_ = [("d", Desc), ("R_cap", C.c_int64), ("ws", C.c_void_p), ("ws_bytes", C.c_size_t),
                ("counts", C.c_void_p), ("offsets", C.c_void_p), ("row_map", C.c_void_p),
                ("row_src", C.c_void_p), ("row_k", C.c_void_p), ("stats", C.c_void_p),
                ("scan_tmp", C.c_void_p), ("Xe", C.c_void_p), ("h", C.c_void_p),
                ("O", C.c_void_p), ("scan_blocks", C.c_int32),
                ("scan_rows_per_block", C.c_int32), ("row_dst", C.c_void_p),
                ("tok_rest", C.c_void_p), ("block_rows", C.c_int32), ("reserved2", C.c_int32),
                ("block_counts", C.c_void_p)]


_lib = None


def lib_path() -> str:
    """The in-tree library, or the build named by TOP_REDUCE_LIB (the
    host-sanitizer build of the same sources, for CPU checks)."""
    return os.environ.get("TOP_REDUCE_LIB") or os.path.join(_HERE, _LIB_NAME)


def load_library():
    """Load the built library; raises if it is missing (no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m top_reduce_amd.build` "
                          "(there is no non-HIP fallback)")
    lib = C.CDLL(path)
    vp, st = C.c_void_p, C.c_int
    lib.moe_workspace_size.restype = C.c_size_t
    lib.moe_workspace_size.argtypes = [C.POINTER(Desc)]
    lib.moe_plan.restype = st
    lib.moe_plan.argtypes = [C.POINTER(Desc), vp, vp, C.c_size_t, vp, C.POINTER(PlanStruct)]
    lib.moe_plan_padded.restype = st
    lib.moe_plan_padded.argtypes = [C.POINTER(Desc), vp, C.c_int32, vp, vp, C.c_size_t, vp,
                                    C.POINTER(PlanStruct)]
    lib.moe_compact_rows.restype = st
    lib.moe_compact_rows.argtypes = [C.c_int64, C.c_int32, vp, C.c_int64, vp, vp, C.c_int32, vp,
                                     vp]
    lib.moe_forward.restype = st
    lib.moe_forward.argtypes = [C.POINTER(PlanStruct), vp, vp, vp, vp, vp, vp]
    lib.moe_expand.restype = st
    lib.moe_expand.argtypes = [C.POINTER(PlanStruct), vp, vp]
    lib.moe_grouped_gemm.restype = st
    lib.moe_grouped_gemm.argtypes = [C.POINTER(PlanStruct), vp, vp, vp]
    lib.moe_grouped_gemm_up.restype = st
    lib.moe_grouped_gemm_up.argtypes = [C.POINTER(PlanStruct), vp, vp]
    lib.moe_grouped_gemm_down.restype = st
    lib.moe_grouped_gemm_down.argtypes = [C.POINTER(PlanStruct), vp, vp]
    lib.moe_combine_reduce.restype = st
    lib.moe_combine_reduce.argtypes = [C.POINTER(PlanStruct), vp, vp, vp, vp]
    lib.moe_grouped_gemm_down_y.restype = st
    lib.moe_grouped_gemm_down_y.argtypes = [C.POINTER(PlanStruct), vp, vp, vp, vp]
    lib.moe_combine_reduce_multi.restype = st
    lib.moe_combine_reduce_multi.argtypes = [C.POINTER(PlanStruct), vp, vp, vp]
    lib.moe_grouped_gemm_up_x.restype = st
    lib.moe_grouped_gemm_up_x.argtypes = [C.POINTER(PlanStruct), vp, vp, vp]
    lib.moe_combine_epilogue.restype = st
    lib.moe_combine_epilogue.argtypes = [C.c_int64, C.c_int32, C.c_int64, C.c_int32, vp, vp,
                                         C.c_int64, vp, vp]
    lib.moe_forward_noalloc.restype = st
    lib.moe_forward_noalloc.argtypes = [C.POINTER(Desc), vp, vp, vp, vp, vp, vp, vp]
    lib.moe_plan_stats.restype = st
    lib.moe_plan_stats.argtypes = [C.POINTER(PlanStruct), C.POINTER(C.c_int32), vp]
    lib.moe_last_error.restype = C.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_abi_version.restype = C.c_int32
    lib.moe_abi_version.argtypes = []
    v = lib.moe_abi_version()
    if v != ABI_VERSION:
        raise ImportError(f"{path}: ABI version {v}, binding expects {ABI_VERSION}")
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        msg = load_library().moe_last_error().decode(errors="replace")
        raise TopReduceError(status, msg)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return BF16
    if dt == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {dt} (bfloat16 or float32)")


def _torch_dtype(code: int) -> torch.dtype:
    return torch.bfloat16 if code == BF16 else torch.float32


def _stream_ptr(stream: Optional[torch.cuda.Stream], device) -> C.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return C.c_void_p(s.cuda_stream)


def _dev_tensor(t: torch.Tensor, name: str, dtype=None, shape=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t.data_ptr()


def make_desc(T: int, K: int, E: int, H: int, I: int, dtype=torch.bfloat16,
              idx_dtype=torch.int64, expert_begin: int = 0, flags: int = 0) -> Desc:
    return Desc(T=T, K=K, E=E, expert_begin=expert_begin, H=H, I=I,
                dtype=_dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype),
                idx_dtype=IDX_I64 if idx_dtype in (torch.int64, IDX_I64) else IDX_I32,
                flags=flags, reserved=0)


def workspace_size(desc: Desc) -> int:
    n = load_library().moe_workspace_size(C.byref(desc))
    if n == 0:
        _check(-1)
    return int(n)


class MoePlan:
    """Host handle of a planned batch; owns (a reference to) its workspace."""

    def __init__(self, desc: Desc, ws: torch.Tensor, st: PlanStruct):
        self.desc = desc
        self.ws = ws
        self.struct = st
        self.block_counts = None      # moe_plan_padded: the counts it was given

    @property
    def T(self):
        return self.desc.T

    @property
    def R_cap(self):
        return self.struct.R_cap

    def _view(self, ptr: int, n: int, dtype: torch.dtype, shape) -> torch.Tensor:
        base = self.ws.data_ptr()
        off = int(ptr) - base
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return self.ws[off:off + nbytes].view(dtype).view(*shape)

    def views(self) -> dict:
        """Views of the plan's device buffers inside the workspace (Xe is None
        for a plan made with FLAG_NO_XE)."""
        d, s = self.desc, self.struct
        dt = _torch_dtype(d.dtype)
        return dict(
            counts=self._view(s.counts, d.E, torch.int32, (d.E,)),
            offsets=self._view(s.offsets, d.E + 1, torch.int32, (d.E + 1,)),
            row_map=self._view(s.row_map, d.T * d.K, torch.int32, (d.T, d.K)),
            row_src=self._view(s.row_src, s.R_cap, torch.int32, (s.R_cap,)),
            row_k=self._view(s.row_k, s.R_cap, torch.int32, (s.R_cap,)),
            row_dst=self._view(s.row_dst, s.R_cap, torch.int32, (s.R_cap,)),
            tok_rest=self._view(s.tok_rest, d.T, torch.int32, (d.T,)),
            stats=self._view(s.stats, 8, torch.int32, (8,)),
            Xe=None if not s.Xe else self._view(s.Xe, s.R_cap * d.H, dt, (s.R_cap, d.H)),
            h=self._view(s.h, s.R_cap * d.I, dt, (s.R_cap, d.I)),
            O=self._view(s.O, s.R_cap * d.H, dt, (s.R_cap, d.H)),
        )


def plan(topk_idx: torch.Tensor, E: int, H: int, I: int, dtype=torch.bfloat16,
         expert_begin: int = 0, flags: int = 0, ws: Optional[torch.Tensor] = None,
         stream: Optional[torch.cuda.Stream] = None, block_rows: int = 0,
         block_counts: Optional[torch.Tensor] = None) -> MoePlan:
    """moe_plan: route scan of topk_idx [T, K] (int32 or int64, global ids or -1).

    With block_rows > 0 this is moe_plan_padded: the rows form blocks of
    block_rows rows (one per DP worker) and block j carries tokens in its first
    block_counts[j] rows only (block_counts: int32 on the GPU, one per block);
    the other rows are padding whatever their ids. The plan keeps a reference
    to block_counts."""
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [T, K]")
    if topk_idx.dtype not in (torch.int32, torch.int64):
        raise TypeError("topk_idx must be int32 or int64")
    T, K = topk_idx.shape
    desc = make_desc(T, K, E, H, I, dtype, topk_idx.dtype, expert_begin, flags)
    need = workspace_size(desc)
    dev = topk_idx.device
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _dev_tensor(ws, "ws", torch.uint8)
    idx_ptr = _dev_tensor(topk_idx, "topk_idx") if T > 0 else 0
    st = PlanStruct()
    if block_rows:
        nb = -(-T // block_rows) if block_rows > 0 else 0
        if block_counts is None:
            raise ValueError("block_counts is required with block_rows")
        bc = _dev_tensor(block_counts, "block_counts", torch.int32, (nb,)) if T > 0 else 0
        _check(load_library().moe_plan_padded(C.byref(desc), C.c_void_p(idx_ptr or None),
                                              block_rows, C.c_void_p(bc or None),
                                              C.c_void_p(ws.data_ptr()), ws.numel(),
                                              _stream_ptr(stream, dev), C.byref(st)))
    else:
        _check(load_library().moe_plan(C.byref(desc), C.c_void_p(idx_ptr or None),
                                       C.c_void_p(ws.data_ptr()), ws.numel(),
                                       _stream_ptr(stream, dev), C.byref(st)))
    mp = MoePlan(desc, ws, st)
    if block_rows:
        mp.block_counts = block_counts
    return mp


def _opt_weights(p: MoePlan, topk_weights) -> Optional[int]:
    if topk_weights is None:
        return None
    return _dev_tensor(topk_weights, "topk_weights", torch.float32, (p.desc.T, p.desc.K))


def forward(p: MoePlan, x: torch.Tensor, topk_weights: Optional[torch.Tensor],
            w1: torch.Tensor, w2: torch.Tensor, y: Optional[torch.Tensor] = None,
            stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """moe_forward: y [T, H] = weighted sum of the local experts' SwiGLU MLPs."""
    d = p.desc
    dt = _torch_dtype(d.dtype)
    if y is None:
        y = torch.empty((d.T, d.H), dtype=dt, device=p.ws.device)
    xp = _dev_tensor(x, "x", dt, (d.T, d.H))
    w1p = _dev_tensor(w1, "w1", dt, (d.E, 2 * d.I, d.H))
    w2p = _dev_tensor(w2, "w2", dt, (d.E, d.H, d.I))
    yp = _dev_tensor(y, "y", dt, (d.T, d.H))
    wp = _opt_weights(p, topk_weights)
    _check(load_library().moe_forward(C.byref(p.struct), C.c_void_p(xp or None),
                                      C.c_void_p(wp), C.c_void_p(w1p or None),
                                      C.c_void_p(w2p or None), C.c_void_p(yp or None),
                                      _stream_ptr(stream, p.ws.device)))
    return y


def forward_noalloc(topk_idx: torch.Tensor, x: torch.Tensor, topk_weights: Optional[torch.Tensor],
                    w1: torch.Tensor, w2: torch.Tensor, y: torch.Tensor, E: int,
                    expert_begin: int = 0, flags: int = 0, stream=None) -> torch.Tensor:
    """moe_forward_noalloc: plan + forward in the library's static workspace
    (no workspace argument; y must be given, since this call is for callers
    that allocate nothing)."""
    if topk_idx.dim() != 2 or topk_idx.dtype not in (torch.int32, torch.int64):
        raise TypeError("topk_idx must be an int32 or int64 [T, K] tensor")
    T, K = topk_idx.shape
    if w1.dim() != 3:
        raise ValueError("w1 must be [E, 2I, H]")
    H, I = x.shape[1], w1.shape[1] // 2
    dt = x.dtype
    desc = make_desc(T, K, E, H, I, dt, topk_idx.dtype, expert_begin, flags)
    ip = _dev_tensor(topk_idx, "topk_idx") if T > 0 else 0
    xp = _dev_tensor(x, "x", dt, (T, H))
    w1p = _dev_tensor(w1, "w1", dt, (E, 2 * I, H))
    w2p = _dev_tensor(w2, "w2", dt, (E, H, I))
    yp = _dev_tensor(y, "y", dt, (T, H))
    wp = None if topk_weights is None else _dev_tensor(topk_weights, "topk_weights",
                                                       torch.float32, (T, K))
    _check(load_library().moe_forward_noalloc(C.byref(desc), C.c_void_p(ip or None),
                                              C.c_void_p(xp or None), C.c_void_p(wp),
                                              C.c_void_p(w1p or None), C.c_void_p(w2p or None),
                                              C.c_void_p(yp or None),
                                              _stream_ptr(stream, x.device)))
    return y


def expand(p: MoePlan, x: torch.Tensor, stream=None) -> None:
    d = p.desc
    xp = _dev_tensor(x, "x", _torch_dtype(d.dtype), (d.T, d.H))
    _check(load_library().moe_expand(C.byref(p.struct), C.c_void_p(xp or None),
                                     _stream_ptr(stream, p.ws.device)))


def grouped_gemm(p: MoePlan, w1: torch.Tensor, w2: torch.Tensor, stream=None) -> None:
    d = p.desc
    dt = _torch_dtype(d.dtype)
    w1p = _dev_tensor(w1, "w1", dt, (d.E, 2 * d.I, d.H))
    w2p = _dev_tensor(w2, "w2", dt, (d.E, d.H, d.I))
    _check(load_library().moe_grouped_gemm(C.byref(p.struct), C.c_void_p(w1p or None),
                                           C.c_void_p(w2p or None),
                                           _stream_ptr(stream, p.ws.device)))


def grouped_gemm_up_x(p: MoePlan, x: torch.Tensor, w1: torch.Tensor, stream=None) -> None:
    """moe_grouped_gemm_up_x: GEMM1 + SwiGLU gathering the received rows x (no Xe)."""
    d = p.desc
    dt = _torch_dtype(d.dtype)
    xp = _dev_tensor(x, "x", dt, (d.T, d.H))
    w1p = _dev_tensor(w1, "w1", dt, (d.E, 2 * d.I, d.H))
    _check(load_library().moe_grouped_gemm_up_x(C.byref(p.struct), C.c_void_p(xp or None),
                                                C.c_void_p(w1p or None),
                                                _stream_ptr(stream, p.ws.device)))


def grouped_gemm_up(p: MoePlan, w1: torch.Tensor, stream=None) -> None:
    d = p.desc
    w1p = _dev_tensor(w1, "w1", _torch_dtype(d.dtype), (d.E, 2 * d.I, d.H))
    _check(load_library().moe_grouped_gemm_up(C.byref(p.struct), C.c_void_p(w1p or None),
                                              _stream_ptr(stream, p.ws.device)))


def grouped_gemm_down(p: MoePlan, w2: torch.Tensor, stream=None) -> None:
    d = p.desc
    w2p = _dev_tensor(w2, "w2", _torch_dtype(d.dtype), (d.E, d.H, d.I))
    _check(load_library().moe_grouped_gemm_down(C.byref(p.struct), C.c_void_p(w2p or None),
                                                _stream_ptr(stream, p.ws.device)))


def grouped_gemm_down_y(p: MoePlan, w2: torch.Tensor, topk_weights: Optional[torch.Tensor],
                        y: torch.Tensor, stream=None) -> None:
    """moe_grouped_gemm_down_y: GEMM2 writing rows of received rows with one
    local slot straight to y (weighted), the others to O."""
    d = p.desc
    dt = _torch_dtype(d.dtype)
    w2p = _dev_tensor(w2, "w2", dt, (d.E, d.H, d.I))
    yp = _dev_tensor(y, "y", dt, (d.T, d.H))
    wp = _opt_weights(p, topk_weights)
    _check(load_library().moe_grouped_gemm_down_y(C.byref(p.struct), C.c_void_p(w2p or None),
                                                  C.c_void_p(wp), C.c_void_p(yp or None),
                                                  _stream_ptr(stream, p.ws.device)))


def combine_reduce_multi(p: MoePlan, topk_weights: Optional[torch.Tensor], y: torch.Tensor,
                         stream=None) -> torch.Tensor:
    """moe_combine_reduce_multi: the reduce for received rows with zero or
    several local slots (after grouped_gemm_down_y)."""
    d = p.desc
    yp = _dev_tensor(y, "y", _torch_dtype(d.dtype), (d.T, d.H))
    wp = _opt_weights(p, topk_weights)
    _check(load_library().moe_combine_reduce_multi(C.byref(p.struct), C.c_void_p(wp),
                                                   C.c_void_p(yp or None),
                                                   _stream_ptr(stream, p.ws.device)))
    return y


def combine_reduce(p: MoePlan, topk_weights: Optional[torch.Tensor],
                   y: Optional[torch.Tensor] = None, expert_out: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """moe_combine_reduce: y [T, H] from expert_out (default: the plan's O)."""
    d = p.desc
    dt = _torch_dtype(d.dtype)
    if y is None:
        y = torch.empty((d.T, d.H), dtype=dt, device=p.ws.device)
    yp = _dev_tensor(y, "y", dt, (d.T, d.H))
    op = None
    if expert_out is not None:
        op = _dev_tensor(expert_out, "expert_out", dt)
        if expert_out.dim() != 2 or expert_out.shape[1] != d.H:
            raise ValueError("expert_out must be [rows, H]")
    wp = _opt_weights(p, topk_weights)
    _check(load_library().moe_combine_reduce(C.byref(p.struct), C.c_void_p(op), C.c_void_p(wp),
                                             C.c_void_p(yp or None),
                                             _stream_ptr(stream, p.ws.device)))
    return y


def combine_epilogue(src: torch.Tensor, recv: torch.Tensor, y: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """moe_combine_epilogue: y [T, H], y[t] = sum of recv[src[t][j]] over src[t][j] >= 0.
    src: int32 [T, J] on the GPU; recv: [N, H] bfloat16 or float32 on the GPU."""
    if src.dim() != 2 or src.dtype != torch.int32:
        raise TypeError("src must be an int32 [T, J] tensor")
    if recv.dim() != 2:
        raise ValueError("recv must be [N, H]")
    T, J = src.shape
    N, H = recv.shape
    dt = recv.dtype
    if y is None:
        y = torch.empty((T, H), dtype=dt, device=recv.device)
    sp = _dev_tensor(src, "src") if T > 0 else 0
    rp = _dev_tensor(recv, "recv", dt) if N > 0 else 0
    yp = _dev_tensor(y, "y", dt, (T, H)) if T > 0 else 0
    _check(load_library().moe_combine_epilogue(T, J, H, _dtype_code(dt), C.c_void_p(sp or None),
                                               C.c_void_p(rp or None), N, C.c_void_p(yp or None),
                                               _stream_ptr(stream, recv.device)))
    return y


def compact_rows(src: torch.Tensor, block_rows: int, block_counts: torch.Tensor,
                 dst: Optional[torch.Tensor] = None, to_padded: bool = False,
                 n_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """moe_compact_rows over the first dimension of src (any dtype, rows of a
    multiple of 4 bytes). Padded -> compact: dst gets the carrying rows of
    src [T, ...] (dst allocated with T rows if None; the first n rows hold
    them). Compact -> padded (to_padded): dst [T, ...] must be given; its
    carrying rows are overwritten from src and its padding rows left as they
    are. n_out: int32 [1] on the GPU, receives the carrying-row count."""
    if src.dim() < 1:
        raise ValueError("src needs a row dimension")
    if to_padded:
        if dst is None:
            raise ValueError("to_padded needs dst (the padded buffer)")
        T = dst.shape[0]
    else:
        T = src.shape[0]
        if dst is None:
            dst = torch.empty_like(src)
    row_bytes = math.prod(src.shape[1:]) * src.element_size()
    nb = -(-T // block_rows) if block_rows > 0 else 0
    bc = _dev_tensor(block_counts, "block_counts", torch.int32, (nb,)) if T > 0 else 0
    sp = _dev_tensor(src, "src") if src.numel() else 0
    dp = _dev_tensor(dst, "dst") if dst.numel() else 0
    if dst.dtype != src.dtype or tuple(dst.shape[1:]) != tuple(src.shape[1:]):
        raise ValueError("src and dst must have the same dtype and row shape")
    np_ = _dev_tensor(n_out, "n_out", torch.int32, (1,)) if n_out is not None else 0
    dev = src.device if src.is_cuda else dst.device
    _check(load_library().moe_compact_rows(T, block_rows, C.c_void_p(bc or None), row_bytes,
                                           C.c_void_p(sp or None), C.c_void_p(dp or None),
                                           1 if to_padded else 0, C.c_void_p(np_ or None),
                                           _stream_ptr(stream, dev)))
    return dst


def plan_stats(p: MoePlan, stream=None) -> Tuple[int, int, int, int]:
    """(R, rows with a local route, ignored slots, empty experts); syncs the stream."""
    out = (C.c_int32 * 4)()
    _check(load_library().moe_plan_stats(C.byref(p.struct), out, _stream_ptr(stream, p.ws.device)))
    return tuple(int(v) for v in out)
