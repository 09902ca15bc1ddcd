"""ctypes binding of libspeed3r.so (see include/speed3r.h for every contract).

Argument marshalling only: tensors are passed as device pointers with their strides, the
current torch (HIP) stream is passed as the stream, and the status code is turned into an
exception. All computation happens in the library's HIP kernels; if the library is missing
this module raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspeed3r.so")

(S3R_OK, S3R_ERR_INVALID_ARG, S3R_ERR_UNSUPPORTED, S3R_ERR_WORKSPACE, S3R_ERR_HIP,
 S3R_ERR_SCRATCH) = range(6)
CMP_AUTO, CMP_TWO_PASS, CMP_SINGLE = range(3)  # s3r_cmp_mode


class Params(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
        ("block", ctypes.c_int32), ("topk", ctypes.c_int32), ("scale", ctypes.c_float),
        ("forced_blocks", ctypes.c_int32),
        ("q_stride_t", ctypes.c_int64), ("q_stride_h", ctypes.c_int64),
        ("k_stride_t", ctypes.c_int64), ("k_stride_h", ctypes.c_int64),
        ("v_stride_t", ctypes.c_int64), ("v_stride_h", ctypes.c_int64),
        ("gate_stride_t", ctypes.c_int64), ("dtype", ctypes.c_int32),
        ("force_own", ctypes.c_int32), ("cmp_mode", ctypes.c_int32),
    ]


class Windows(ctypes.Structure):
    """Token layout for 2-D pooling windows: views x (special + grid_h * grid_w)."""
    _fields_ = [
        ("views", ctypes.c_int64), ("special", ctypes.c_int32), ("grid_h", ctypes.c_int32),
        ("grid_w", ctypes.c_int32), ("win_h", ctypes.c_int32), ("win_w", ctypes.c_int32),
    ]


_DTYPES = {torch.bfloat16: 0, torch.float16: 1}  # s3r_dtype


class Speed3RError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)}")
        self.status = status


EXPORTS = {
    "speed3r_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "speed3r_num_blocks": (ctypes.c_int64, [ctypes.POINTER(Params)]),
    "speed3r_num_selected": (ctypes.c_int64, [ctypes.POINTER(Params)]),
    "speed3r_score_row_stride": (ctypes.c_int64, [ctypes.POINTER(Params)]),
    "speed3r_tiles_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Params)]),
    "speed3r_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Params)]),
    "speed3r_dense_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Params)]),
    "speed3r_sparse_attn_fwd": (ctypes.c_int, [ctypes.POINTER(Params)] + [ctypes.c_void_p] * 6 +
                                [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "speed3r_pool": (ctypes.c_int, [ctypes.POINTER(Params), ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p]),
    "speed3r_cmp_lse": (ctypes.c_int, [ctypes.POINTER(Params), ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]),
    "speed3r_cmp_fused": (ctypes.c_int, [ctypes.POINTER(Params), ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "speed3r_cmp_fused_topk": (ctypes.c_int, [ctypes.POINTER(Params), ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "speed3r_redo_flag_count": (ctypes.c_int64, [ctypes.POINTER(Params)]),
    "speed3r_cmp_lse_bound": (ctypes.c_int, [ctypes.POINTER(Params), ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                             ctypes.c_void_p]),
    "speed3r_cmp_single_topk": (ctypes.c_int, [ctypes.POINTER(Params), ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_size_t] +
                                [ctypes.c_void_p] * 6),
    "speed3r_topk": (ctypes.c_int, [ctypes.POINTER(Params), ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p]),
    "speed3r_sel_combine": (ctypes.c_int, [ctypes.POINTER(Params), ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_size_t] +
                            [ctypes.c_void_p] * 6),
    "speed3r_dense_attn_fwd": (ctypes.c_int, [ctypes.POINTER(Params)] + [ctypes.c_void_p] * 5 +
                               [ctypes.c_size_t, ctypes.c_void_p]),
    "speed3r_train_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Params)]),
    "speed3r_sparse_attn_fwd_train": (ctypes.c_int, [ctypes.POINTER(Params)] +
                                      [ctypes.c_void_p] * 6 +
                                      [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "speed3r_bwd_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Params)]),
    "speed3r_sparse_attn_bwd": (ctypes.c_int, [ctypes.POINTER(Params)] + [ctypes.c_void_p] * 5 +
                                [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                 ctypes.c_size_t] + [ctypes.c_void_p] * 5 +
                                [ctypes.c_size_t, ctypes.c_void_p]),
    "speed3r_window_source": (ctypes.c_int64, [ctypes.POINTER(Windows), ctypes.c_int64]),
    "speed3r_window_permute": (ctypes.c_int, [ctypes.POINTER(Windows), ctypes.c_int32,
                                              ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                              ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                              ctypes.c_int32, ctypes.c_void_p]),
    "speed3r_windows_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Params),
                                                         ctypes.POINTER(Windows)]),
    "speed3r_sparse_attn_fwd_windows": (ctypes.c_int, [ctypes.POINTER(Params),
                                                       ctypes.POINTER(Windows)] +
                                        [ctypes.c_void_p] * 6 +
                                        [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "speed3r_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "speed3r_sparse_attn_fwd_noalloc": (ctypes.c_int, [ctypes.POINTER(Params)] +
                                        [ctypes.c_void_p] * 6 + [ctypes.c_void_p]),
    "speed3r_calib_copy": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                          ctypes.c_void_p]),
    "speed3r_calib_mfma_flops": (ctypes.c_int64, [ctypes.c_int32, ctypes.c_int32]),
    "speed3r_calib_mfma": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_void_p]),
}

_lib = None


def lib():
    """The loaded library. Raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_global_attention_block_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().speed3r_status_string(int(s)).decode()


def _check(fn: str, st: int):
    if st != S3R_OK:
        raise Speed3RError(fn, st)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def make_params(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block: int, topk: int,
                scale: float = 0.0, gates: Optional[torch.Tensor] = None,
                forced_blocks: int = 0, force_own: bool = False,
                cmp_mode: int = CMP_AUTO) -> Params:
    """Params for [T, H, 64] bf16 or fp16 token tensors (one type for q, k, v; any token/head
    strides, last dim contiguous). ``forced_blocks`` key blocks 0..F-1 are selected for every
    query block on top of the top-k of the rest; with ``force_own`` each query block also
    keeps its own key block. ``cmp_mode``: CMP_AUTO, CMP_TWO_PASS or CMP_SINGLE."""
    T, H, D = q.shape
    for x in (q, k, v):
        if x.dtype not in _DTYPES or x.dtype != q.dtype or tuple(x.shape) != (T, H, D) or \
                x.stride(2) != 1:
            raise ValueError("q, k, v must be one of bf16/fp16, [T, H, D] with a contiguous "
                             "last dimension")
        if x.device != q.device or x.device.type != "cuda":
            raise ValueError("q, k, v must be on one GPU (the kernels read device memory)")
    gst = 0
    if gates is not None and gates.dim() == 3:
        gst = gates.stride(0)
    return Params(T, H, D, block, topk, float(scale), forced_blocks, q.stride(0), q.stride(1),
                  k.stride(0), k.stride(1), v.stride(0), v.stride(1), gst, _DTYPES[q.dtype],
                  int(force_own), int(cmp_mode))


def num_blocks(p: Params) -> int:
    return int(lib().speed3r_num_blocks(ctypes.byref(p)))


def num_selected(p: Params) -> int:
    """Entries per selection row: forced prefix + chosen blocks."""
    return int(lib().speed3r_num_selected(ctypes.byref(p)))


def score_row_stride(p: Params) -> int:
    return int(lib().speed3r_score_row_stride(ctypes.byref(p)))


def workspace_size(p: Params) -> int:
    return int(lib().speed3r_workspace_size(ctypes.byref(p)))


def tiles_workspace_size(p: Params) -> int:
    return int(lib().speed3r_tiles_workspace_size(ctypes.byref(p)))


def dense_workspace_size(p: Params) -> int:
    return int(lib().speed3r_dense_workspace_size(ctypes.byref(p)))


def runs_single(p: Params) -> bool:
    """Whether the forward pass with these params runs the single compression pass: CMP_SINGLE,
    or CMP_AUTO where the single pass applies (B <= 64, at most 64 chosen blocks, Nb >= 8) and
    k <= 48 or at most 64 candidate blocks (the rule the library applies, include/speed3r.h)."""
    Nb = num_blocks(p)
    if Nb < 0:
        raise ValueError("invalid params")
    forced = min(p.forced_blocks, Nb)
    most = min(p.topk, Nb - forced)
    ok = p.block <= 64 and most <= 64 and Nb >= 8
    if p.cmp_mode == CMP_SINGLE:
        return ok
    return ok and p.cmp_mode == CMP_AUTO and (4 * most <= 3 * 64 or Nb - forced <= 64)


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _check_out(out: torch.Tensor, q: torch.Tensor, what: str = "out"):
    """A [T, H, 64] result buffer: q's shape, type and device, contiguous."""
    _need(isinstance(out, torch.Tensor) and tuple(out.shape) == tuple(q.shape) and
          out.dtype == q.dtype and out.device == q.device and out.is_contiguous(),
          f"{what} must be a contiguous {q.dtype} tensor of shape {tuple(q.shape)} on "
          f"{q.device}")


def _check_gates(gates: torch.Tensor, q: torch.Tensor):
    """Gates are float32 [H, 2] (contiguous) or per token [T, H, 2] with strides (2H, 2, 1)."""
    T, H, _ = q.shape
    ok = isinstance(gates, torch.Tensor) and gates.dtype == torch.float32 and \
        gates.device == q.device
    if ok and gates.dim() == 2:
        ok = tuple(gates.shape) == (H, 2) and gates.is_contiguous()
    elif ok and gates.dim() == 3:
        ok = tuple(gates.shape) == (T, H, 2) and tuple(gates.stride()) == (2 * H, 2, 1)
    else:
        ok = False
    _need(ok, f"gates must be float32 [H, 2] (contiguous) or [T, H, 2] with strides "
              f"(2H, 2, 1) on {q.device}")


def _check_sel(sel_idx: torch.Tensor, p: Params, device):
    """A selection buffer: int32 [H, Nb, num_selected(p)], contiguous, on the inputs' device."""
    shape = (p.H, num_blocks(p), num_selected(p))
    _need(isinstance(sel_idx, torch.Tensor) and sel_idx.dtype == torch.int32 and
          tuple(sel_idx.shape) == shape and sel_idx.is_contiguous() and
          sel_idx.device == device,
          f"sel_idx must be a contiguous int32 tensor of shape {shape} on {device}")


def _check_workspace(ws: torch.Tensor, device):
    _need(isinstance(ws, torch.Tensor) and ws.dtype == torch.uint8 and ws.is_contiguous() and
          ws.device == device, f"workspace must be a contiguous uint8 tensor on {device}")


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator hands out 512-byte aligned blocks, more than the 256 required
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def sparse_attn_fwd(q, k, v, gates, block: int, topk: int, scale: float = 0.0,
                    out: Optional[torch.Tensor] = None, sel_idx: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, forced_blocks: int = 0,
                    force_own: bool = False, cmp_mode: int = CMP_AUTO
                    ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Full forward pass. Returns (out [T, H, 64] in the input type, sel_idx or None)."""
    p = make_params(q, k, v, block, topk, scale, gates, forced_blocks, force_own, cmp_mode)
    _check_gates(gates, q)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    _check_out(out, q)
    if sel_idx is not None:
        _check_sel(sel_idx, p, q.device)
    if workspace is None:
        workspace = alloc_workspace(workspace_size(p), q.device)
    _check_workspace(workspace, q.device)
    st = lib().speed3r_sparse_attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(gates),
                                       _ptr(out), _ptr(sel_idx), _ptr(workspace),
                                       workspace.numel(), _stream())
    _check("speed3r_sparse_attn_fwd", st)
    return out, sel_idx


def noalloc_scratch_bytes() -> int:
    """Largest workspace sparse_attn_fwd_noalloc takes (the library's fixed device array)."""
    return int(lib().speed3r_noalloc_scratch_bytes())


def sparse_attn_fwd_noalloc(q, k, v, gates, block: int, topk: int, out: torch.Tensor,
                            sel_idx: Optional[torch.Tensor] = None, scale: float = 0.0,
                            forced_blocks: int = 0, force_own: bool = False,
                            cmp_mode: int = CMP_AUTO):
    """The forward pass with the library's fixed workspace array: nothing is allocated, by
    the library or here (out, and sel_idx if wanted, come from the caller). Calls on one GPU
    must not overlap."""
    p = make_params(q, k, v, block, topk, scale, gates, forced_blocks, force_own, cmp_mode)
    _check_gates(gates, q)
    _check_out(out, q)
    if sel_idx is not None:
        _check_sel(sel_idx, p, q.device)
    st = lib().speed3r_sparse_attn_fwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                               _ptr(gates), _ptr(out), _ptr(sel_idx),
                                               _stream())
    _check("speed3r_sparse_attn_fwd_noalloc", st)
    return out, sel_idx


def pool(p: Params, k, v, workspace, k_mean=None, v_mean=None):
    _check("speed3r_pool", lib().speed3r_pool(ctypes.byref(p), _ptr(k), _ptr(v), _ptr(workspace),
                                              workspace.numel(), _ptr(k_mean), _ptr(v_mean),
                                              _stream()))


def cmp_lse(p: Params, q, workspace, lse):
    _check("speed3r_cmp_lse", lib().speed3r_cmp_lse(ctypes.byref(p), _ptr(q), _ptr(workspace),
                                                    workspace.numel(), _ptr(lse), _stream()))


def cmp_fused(p: Params, q, workspace, lse, o_cmp, score):
    _check("speed3r_cmp_fused", lib().speed3r_cmp_fused(
        ctypes.byref(p), _ptr(q), _ptr(workspace), workspace.numel(), _ptr(lse), _ptr(o_cmp),
        _ptr(score), _stream()))


def cmp_fused_topk(p: Params, q, workspace, lse, o_cmp, sel_idx):
    _check("speed3r_cmp_fused_topk", lib().speed3r_cmp_fused_topk(
        ctypes.byref(p), _ptr(q), _ptr(workspace), workspace.numel(), _ptr(lse), _ptr(o_cmp),
        _ptr(sel_idx), _stream()))


def redo_flag_count(p: Params) -> int:
    return int(lib().speed3r_redo_flag_count(ctypes.byref(p)))


def cmp_lse_bound(p: Params, q, workspace, lse_bound):
    _check("speed3r_cmp_lse_bound", lib().speed3r_cmp_lse_bound(
        ctypes.byref(p), _ptr(q), _ptr(workspace), workspace.numel(), _ptr(lse_bound),
        _stream()))


def cmp_single_topk(p: Params, q, workspace, lse_bound, lse, o_cmp, sel_idx, redo):
    _check("speed3r_cmp_single_topk", lib().speed3r_cmp_single_topk(
        ctypes.byref(p), _ptr(q), _ptr(workspace), workspace.numel(), _ptr(lse_bound),
        _ptr(lse), _ptr(o_cmp), _ptr(sel_idx), _ptr(redo), _stream()))


def topk(p: Params, score, sel_idx):
    _check("speed3r_topk", lib().speed3r_topk(ctypes.byref(p), _ptr(score), _ptr(sel_idx),
                                              _stream()))


def sel_combine(p: Params, q, workspace, sel_idx, o_cmp, gates, out, o_sel=None):
    _check("speed3r_sel_combine", lib().speed3r_sel_combine(
        ctypes.byref(p), _ptr(q), _ptr(workspace), workspace.numel(), _ptr(sel_idx),
        _ptr(o_cmp), _ptr(gates), _ptr(out), _ptr(o_sel), _stream()))


def dense_attn_fwd(q, k, v, scale: float = 0.0, out=None, workspace=None):
    p = make_params(q, k, v, 64, 1, scale)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    _check_out(out, q)
    if workspace is None:
        workspace = alloc_workspace(dense_workspace_size(p), q.device)
    _check_workspace(workspace, q.device)
    _check("speed3r_dense_attn_fwd", lib().speed3r_dense_attn_fwd(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(workspace),
        workspace.numel(), _stream()))
    return out


def train_workspace_size(p: Params) -> int:
    return int(lib().speed3r_train_workspace_size(ctypes.byref(p)))


def bwd_workspace_size(p: Params) -> int:
    return int(lib().speed3r_bwd_workspace_size(ctypes.byref(p)))


class Trained:
    """State of a training forward pass: the output, the selection and the workspace the
    backward pass reads."""

    def __init__(self, p, q, k, v, gates, out, sel, workspace):
        self.p, self.q, self.k, self.v, self.gates = p, q, k, v, gates
        self.out, self.sel, self.workspace = out, sel, workspace


def sparse_attn_fwd_train(q, k, v, gates, block: int, topk: int, scale: float = 0.0,
                          forced_blocks: int = 0, workspace: Optional[torch.Tensor] = None,
                          force_own: bool = False, cmp_mode: int = CMP_AUTO) -> Trained:
    """Forward pass that keeps the state speed3r_sparse_attn_bwd needs."""
    p = make_params(q, k, v, block, topk, scale, gates, forced_blocks, force_own, cmp_mode)
    _check_gates(gates, q)
    out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    sel = torch.empty(q.shape[1], num_blocks(p), num_selected(p), dtype=torch.int32,
                      device=q.device)
    if workspace is None:
        workspace = alloc_workspace(train_workspace_size(p), q.device)
    _check_workspace(workspace, q.device)
    _check("speed3r_sparse_attn_fwd_train", lib().speed3r_sparse_attn_fwd_train(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(gates), _ptr(out), _ptr(sel),
        _ptr(workspace), workspace.numel(), _stream()))
    return Trained(p, q, k, v, gates, out, sel, workspace)


def sparse_attn_bwd(st: Trained, dout: torch.Tensor, workspace: Optional[torch.Tensor] = None):
    """Gradients (dq, dk, dv f32 [T, H, 64], dgates f32 shaped like the gates) of the forward
    pass recorded in `st`, for the output gradient dout ([T, H, 64], the type of q)."""
    if dout.dtype != st.q.dtype or tuple(dout.shape) != tuple(st.q.shape) or \
            dout.stride(2) != 1:
        raise ValueError("dout must have the type and shape of q ([T, H, 64]) with a "
                         "contiguous last dimension")
    f32 = dict(dtype=torch.float32, device=st.q.device)
    dq, dk, dv = (torch.empty(st.q.shape, **f32) for _ in range(3))
    dg = torch.empty(st.gates.shape, **f32) if st.gates.dim() == 2 else \
        torch.empty_strided(st.gates.shape, st.gates.stride(), **f32)
    if workspace is None:
        workspace = alloc_workspace(bwd_workspace_size(st.p), st.q.device)
    _check("speed3r_sparse_attn_bwd", lib().speed3r_sparse_attn_bwd(
        ctypes.byref(st.p), _ptr(st.q), _ptr(st.k), _ptr(st.v), _ptr(st.gates), _ptr(dout),
        dout.stride(0), dout.stride(1), _ptr(st.workspace), st.workspace.numel(), _ptr(dq),
        _ptr(dk), _ptr(dv), _ptr(dg), _ptr(workspace), workspace.numel(), _stream()))
    return dq, dk, dv, dg


def make_windows(layout) -> Windows:
    """layout = (views, special, grid_h, grid_w, win_h, win_w)."""
    return Windows(*[int(x) for x in layout])


def window_source(layout, pos: int) -> int:
    return int(lib().speed3r_window_source(ctypes.byref(make_windows(layout)), pos))


def window_permute(layout, src: torch.Tensor, dst: Optional[torch.Tensor] = None,
                   inverse: bool = False) -> torch.Tensor:
    """Reorder a [T, H, 64] bf16/fp16 tensor into window order (or back, inverse=True)."""
    w = make_windows(layout)
    _need(src.dim() == 3 and src.dtype in _DTYPES and src.stride(2) == 1,
          "src must be a bf16/fp16 [T, H, 64] tensor with a contiguous last dimension")
    if dst is None:
        dst = torch.empty(src.shape, dtype=src.dtype, device=src.device)
    _need(tuple(dst.shape) == tuple(src.shape) and dst.dtype == src.dtype and
          dst.device == src.device and dst.stride(2) == 1,
          "dst must have src's shape, type and device, with a contiguous last dimension")
    _check("speed3r_window_permute", lib().speed3r_window_permute(
        ctypes.byref(w), src.shape[1], _ptr(src), src.stride(0), src.stride(1), _ptr(dst),
        dst.stride(0), dst.stride(1), int(inverse), _stream()))
    return dst


def windows_workspace_size(p: Params, layout) -> int:
    return int(lib().speed3r_windows_workspace_size(ctypes.byref(p),
                                                     ctypes.byref(make_windows(layout))))


def sparse_attn_fwd_windows(q, k, v, gates, block: int, topk: int, layout, scale: float = 0.0,
                            out: Optional[torch.Tensor] = None,
                            sel_idx: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None, forced_blocks: int = 0,
                            force_own: bool = False, cmp_mode: int = CMP_AUTO
                            ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Forward pass with 2-D windows as blocks; out in the caller's token order, sel_idx over
    blocks of the window order."""
    p = make_params(q, k, v, block, topk, scale, gates, forced_blocks, force_own, cmp_mode)
    _check_gates(gates, q)
    w = make_windows(layout)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    _check_out(out, q)
    if sel_idx is not None:
        _check_sel(sel_idx, p, q.device)
    if workspace is None:
        workspace = alloc_workspace(windows_workspace_size(p, layout), q.device)
    _check_workspace(workspace, q.device)
    _check("speed3r_sparse_attn_fwd_windows", lib().speed3r_sparse_attn_fwd_windows(
        ctypes.byref(p), ctypes.byref(w), _ptr(q), _ptr(k), _ptr(v), _ptr(gates), _ptr(out),
        _ptr(sel_idx), _ptr(workspace), workspace.numel(), _stream()))
    return out, sel_idx


class Stages:
    """Runs the forward pass one stage at a time and keeps every intermediate result:
    k_mean, v_mean [H, Nb, 64] f32, lse [H, T] f32, o_cmp [T, H, 64] f32,
    score [H, Nb, ld] f32, sel [H, Nb, k_eff] int32 (k_eff = forced prefix + chosen blocks),
    o_sel [T, H, 64] f32, out (input type); for the single compression pass also
    lse_bound [H, T] f32 and redo (int32 flags, 4 per 256 queries per head)."""

    def __init__(self, q, k, v, gates, block: int, topk_: int, scale: float = 0.0,
                 keep_o_sel: bool = True, keep_score: bool = True, forced_blocks: int = 0,
                 force_own: bool = False):
        self.q, self.k, self.v, self.gates = q, k, v, gates
        self.p = make_params(q, k, v, block, topk_, scale, gates, forced_blocks, force_own)
        T, H, D = q.shape
        dev = q.device
        self.Nb = num_blocks(self.p)
        self.ld = score_row_stride(self.p)
        self.k_eff = num_selected(self.p)
        self.forced = min(forced_blocks, self.Nb)
        self.own = bool(force_own) and self.forced < self.Nb
        self.topk = topk_
        self.ws = alloc_workspace(tiles_workspace_size(self.p), dev)
        f32 = dict(dtype=torch.float32, device=dev)
        self.k_mean = torch.empty(H, self.Nb, D, **f32)
        self.v_mean = torch.empty(H, self.Nb, D, **f32)
        self.lse = torch.empty(H, T, **f32)
        self.o_cmp = torch.empty(T, H, D, **f32)
        self.score = torch.empty(H, self.Nb, self.ld, **f32) if keep_score else None
        self.sel = torch.empty(H, self.Nb, self.k_eff, dtype=torch.int32, device=dev)
        self.o_sel = torch.empty(T, H, D, **f32) if keep_o_sel else None
        self.out = torch.empty(T, H, D, dtype=q.dtype, device=dev)
        self.lse_bound = torch.empty(H, T, **f32)
        self.redo = torch.empty(redo_flag_count(self.p), dtype=torch.int32, device=dev)

    def run_pool(self):
        pool(self.p, self.k, self.v, self.ws, self.k_mean, self.v_mean)

    def run_lse(self):
        cmp_lse(self.p, self.q, self.ws, self.lse)

    def run_fused(self, lse=None):
        cmp_fused(self.p, self.q, self.ws, self.lse if lse is None else lse, self.o_cmp,
                  self.score)

    def run_topk(self, score=None):
        topk(self.p, self.score if score is None else score, self.sel)

    def run_fused_topk(self, lse=None, sel=None):
        """Pass 2 with the running top-k: o_cmp and the selection, no score matrix."""
        cmp_fused_topk(self.p, self.q, self.ws, self.lse if lse is None else lse, self.o_cmp,
                       self.sel if sel is None else sel)

    @property
    def folds_topk(self) -> bool:
        return self.p.block <= 64 and min(self.topk, self.Nb - self.forced) <= 64

    @property
    def single_ok(self) -> bool:
        """The single compression pass applies: folded selection and Nb >= 8."""
        return self.folds_topk and self.Nb >= 8

    def run_lse_bound(self, out=None):
        cmp_lse_bound(self.p, self.q, self.ws, self.lse_bound if out is None else out)

    def run_single_topk(self, lse_bound=None, sel=None, lse=None, o_cmp=None):
        """The single compression pass (with its exact reruns) from lse_bound: writes lse,
        o_cmp, the selection and the redo flags."""
        cmp_single_topk(self.p, self.q, self.ws,
                        self.lse_bound if lse_bound is None else lse_bound,
                        self.lse if lse is None else lse, self.o_cmp if o_cmp is None else o_cmp,
                        self.sel if sel is None else sel, self.redo)

    def run_sel(self, sel=None, o_cmp=None):
        sel_combine(self.p, self.q, self.ws, self.sel if sel is None else sel,
                    self.o_cmp if o_cmp is None else o_cmp, self.gates, self.out, self.o_sel)

    def run_all(self):
        self.run_pool()
        self.run_lse()
        self.run_fused()
        self.run_topk()
        self.run_sel()
        return self


def calib_copy(src: torch.Tensor, dst: torch.Tensor) -> int:
    """Streaming copy kernel (a measured HBM ceiling): copies src into dst (same size, 16-byte
    multiple, contiguous). Returns the bytes it moves through HBM (read + written)."""
    _need(src.is_contiguous() and dst.is_contiguous() and src.device == dst.device and
          src.numel() * src.element_size() == dst.numel() * dst.element_size(),
          "src and dst must be contiguous tensors of one size on one device")
    n = src.numel() * src.element_size()
    _check("speed3r_calib_copy", lib().speed3r_calib_copy(_ptr(src), _ptr(dst), n, _stream()))
    return 2 * n


def calib_mfma(sink: torch.Tensor, work_groups: int, iters: int) -> int:
    """Loop of bf16 matrix products (a measured MFMA ceiling). sink: float32, at least
    work_groups * 256 elements. Returns the floating-point operations performed."""
    _need(sink.dtype == torch.float32 and sink.is_contiguous() and
          sink.numel() >= work_groups * 256, "sink must be float32 [work_groups * 256]")
    _check("speed3r_calib_mfma", lib().speed3r_calib_mfma(_ptr(sink), work_groups, iters,
                                                          _stream()))
    return int(lib().speed3r_calib_mfma_flops(work_groups, iters))
