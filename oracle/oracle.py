"""Python front end of the CPU oracle (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` use
this module. It loads ``liboracle.so`` built from ``speed3r_oracle.c`` with plain gcc (no HIP),
and shares nothing with the GPU library.

Inputs are torch or numpy arrays of bf16 values; they are upcast exactly to float32 before the
call, and every computation inside runs in float64 (see the C file for the step-by-step
definition and the pages it follows).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import time
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "speed3r_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_dbl = ctypes.c_double


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        L.s3r_oracle_pool.argtypes = [_i64, _i32, _i32, _i32, _f32p, _i64, _i64, _f64p]
        L.s3r_oracle_pool.restype = None
        L.s3r_oracle_cmp_row.argtypes = [_i64, _i32, _i32, _i32, _dbl, _f32p, _i64, _i64, _f64p,
                                         _f64p, _i32, _i64, _f64p, _f64p, _f64p]
        L.s3r_oracle_cmp_row.restype = None
        L.s3r_oracle_topk.argtypes = [_f32p, _i64, _i32, _i32p]
        L.s3r_oracle_topk.restype = _i32
        L.s3r_oracle_sel_row.argtypes = [_i64, _i32, _i32, _i32, _dbl, _f32p, _i64, _i64, _f32p,
                                         _i64, _i64, _f32p, _i64, _i64, _i32, _i64, _i32p, _i32,
                                         _f64p]
        L.s3r_oracle_sel_row.restype = None
        L.s3r_oracle_dense_rows.argtypes = [_i64, _i32, _i32, _dbl, _f32p, _i64, _i64, _f32p,
                                            _i64, _i64, _f32p, _i64, _i64, _i32, _i64, _i64,
                                            _f64p]
        L.s3r_oracle_dense_rows.restype = None
        L.s3r_oracle_num_selected.argtypes = [_i64, _i32, _i32, _i32, _i32]
        L.s3r_oracle_num_selected.restype = _i32
        L.s3r_oracle_forward_rows.argtypes = [
            _i64, _i32, _i32, _i32, _i32, _i32, _i32, _dbl, _f32p, _i64, _i64, _f32p, _i64, _i64,
            _f32p,
            _i64, _i64, _f64p, _f64p, _f32p, _i64, _i64, _i32p, _i64p,
            ctypes.c_void_p, _f64p, _f64p, _f32p, _i32p, _f64p, _f64p]
        L.s3r_oracle_forward_rows.restype = None
        L.s3r_oracle_backward.argtypes = [
            _i64, _i32, _i32, _i32, _dbl, _f32p, _i64, _i64, _f32p, _i64, _i64, _f32p, _i64,
            _i64, _f32p, _i64, _f32p, _i64, _i64, _i32p, _i32, _f64p, _f64p, _f64p, _f64p]
        L.s3r_oracle_backward.restype = None
        L.s3r_oracle_num_threads.argtypes = []
        L.s3r_oracle_num_threads.restype = ctypes.c_int
        L.s3r_oracle_set_num_threads.argtypes = [ctypes.c_int]
        L.s3r_oracle_set_num_threads.restype = None
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().s3r_oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's loops over independent rows (results do not depend on it)."""
    lib().s3r_oracle_set_num_threads(int(n))


def _f32(x) -> np.ndarray:
    """Exact float32 copy of a [T, H, D] bf16/float tensor (torch or numpy), contiguous."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu", torch.float32).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def n_blocks(T: int, B: int) -> int:
    return -(-T // B)


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)


def pool(x, B: int) -> np.ndarray:
    """Block means of a [T, H, D] tensor -> [H, Nb, D] float64."""
    a = _f32(x)
    T, H, D = a.shape
    out = np.empty((H, n_blocks(T, B), D), np.float64)
    lib().s3r_oracle_pool(T, H, D, B, a, H * D, D, out)
    return out


def cmp_row(q, kc: np.ndarray, vc: np.ndarray, B: int, h: int, i: int,
            scale: Optional[float] = None):
    """Compression branch of one (head, query block): returns (lse [n], ocmp [n, D],
    score [Nb]) in float64."""
    a = _f32(q)
    T, H, D = a.shape
    Nb = n_blocks(T, B)
    n = min(T, (i + 1) * B) - i * B
    lse = np.empty(B, np.float64)
    oc = np.empty((B, D), np.float64)
    sc = np.empty(Nb, np.float64)
    lib().s3r_oracle_cmp_row(T, H, D, B, default_scale(D) if scale is None else scale, a,
                             H * D, D, np.ascontiguousarray(kc), np.ascontiguousarray(vc), h, i,
                             lse, oc, sc)
    return lse[:n], oc[:n], sc


def lse_group_bound(q, k, B: int, group: int = 8, scale: Optional[float] = None) -> np.ndarray:
    """Lower bound of the compression branch's log-sum-exp used by the single-pass variant
    (an implementation choice, not part of the pages' method): the pooled keys Kc_0..Kc_{Nb-1}
    are cut into floor(Nb / group) full groups (a short last group is left out), each group is
    replaced by its mean G_g, and the bound is

        lse_bound[h, t] = log sum_g group * exp(scale * q_t . G_g)        ([H, T] float64).

    exp is convex and the logit is linear in the key, so by Jensen's inequality
    group * exp(mean of the group's logits) <= sum of exp over the group's keys: the bound is
    at most the log-sum-exp over all pooled keys, with equality when every group's keys are
    equal and no block is left out."""
    a = _f32(q).astype(np.float64)
    T, H, D = a.shape
    kc = pool(k, B)
    G = kc.shape[1] // group
    if G < 1:
        raise ValueError("fewer pooled keys than one group")
    means = kc[:, :G * group].reshape(H, G, group, D).mean(axis=2)       # [H, G, D]
    s = default_scale(D) if scale is None else scale
    logits = s * np.matmul(a.transpose(1, 0, 2), means.transpose(0, 2, 1))  # [H, T, G]
    m = logits.max(axis=-1, keepdims=True)
    return m[..., 0] + np.log(np.exp(logits - m).sum(axis=-1)) + math.log(group)


def topk(score_row, k: int) -> np.ndarray:
    """Top-k block indices of one float32 score row (value desc, index asc), ascending."""
    s = np.ascontiguousarray(np.asarray(score_row, dtype=np.float32))
    out = np.empty(max(1, min(k, s.size)), np.int32)
    n = lib().s3r_oracle_topk(s, s.size, k, out)
    return out[:n]


def sel_row(q, k, v, B: int, h: int, i: int, sel: Sequence[int],
            scale: Optional[float] = None) -> np.ndarray:
    """Selection branch of one (head, query block) over the listed key blocks -> [n, D]."""
    a, b, c = _f32(q), _f32(k), _f32(v)
    T, H, D = a.shape
    n = min(T, (i + 1) * B) - i * B
    s = np.ascontiguousarray(np.asarray(sel, dtype=np.int32))
    out = np.empty((B, D), np.float64)
    lib().s3r_oracle_sel_row(T, H, D, B, default_scale(D) if scale is None else scale,
                             a, H * D, D, b, H * D, D, c, H * D, D, h, i, s, s.size, out)
    return out[:n]


def dense_rows(q, k, v, h: int, t0: int, nt: int, scale: Optional[float] = None) -> np.ndarray:
    """Plain softmax attention of queries t0..t0+nt-1 of head h over all keys -> [nt, D]."""
    a, b, c = _f32(q), _f32(k), _f32(v)
    T, H, D = a.shape
    out = np.empty((nt, D), np.float64)
    lib().s3r_oracle_dense_rows(T, H, D, default_scale(D) if scale is None else scale, a, H * D,
                                D, b, H * D, D, c, H * D, D, h, t0, nt, out)
    return out


def num_selected(T: int, B: int, topk_: int, forced: int = 0, own: bool = False) -> int:
    return int(lib().s3r_oracle_num_selected(T, B, topk_, forced, int(own)))


def forward_rows(q, k, v, gates, B: int, topk_: int, rows_h: Sequence[int],
                 rows_i: Sequence[int], kc: Optional[np.ndarray] = None,
                 vc: Optional[np.ndarray] = None, sel_in: Optional[np.ndarray] = None,
                 scale: Optional[float] = None, forced: int = 0,
                 own: bool = False) -> Dict[str, np.ndarray]:
    """Whole forward pass for the listed (head, query block) rows.

    Returns per-row arrays: lse [R, B], ocmp [R, B, D], score [R, Nb] (float32), sel
    [R, n_sel], osel [R, B, D], out [R, B, D]; rows of a short last block are valid for their
    first n_i entries only. ``kc``/``vc`` may be passed in to reuse a pooling. ``forced``
    blocks (the first F) are always selected, with ``own`` each query block's own key block
    too, and top-k runs over the rest (rows that hold fewer blocks end with -1).
    """
    a, b, c = _f32(q), _f32(k), _f32(v)
    T, H, D = a.shape
    Nb = n_blocks(T, B)
    k_eff = num_selected(T, B, topk_, forced, own)
    if kc is None:
        kc = pool(b, B)
    if vc is None:
        vc = pool(c, B)
    g = _f32(gates)
    gate_st = 0 if g.ndim == 2 else H * 2
    rh = np.ascontiguousarray(np.asarray(rows_h, dtype=np.int32))
    ri = np.ascontiguousarray(np.asarray(rows_i, dtype=np.int64))
    R = rh.size
    res = {
        "lse": np.zeros((R, B), np.float64), "ocmp": np.zeros((R, B, D), np.float64),
        "score": np.zeros((R, Nb), np.float32), "sel": np.zeros((R, k_eff), np.int32),
        "osel": np.zeros((R, B, D), np.float64), "out": np.zeros((R, B, D), np.float64),
    }
    sel_ptr = None
    if sel_in is not None:
        sel_in = np.ascontiguousarray(np.asarray(sel_in, dtype=np.int32).reshape(R, k_eff))
        sel_ptr = sel_in.ctypes.data
    lib().s3r_oracle_forward_rows(
        T, H, D, B, topk_, forced, int(own), default_scale(D) if scale is None else scale, a,
        H * D, D,
        b, H * D,
        D, c, H * D, D, np.ascontiguousarray(kc), np.ascontiguousarray(vc), g.reshape(-1),
        gate_st, R, rh, ri, sel_ptr, res["lse"], res["ocmp"], res["score"], res["sel"],
        res["osel"], res["out"])
    return res


def forward_all(q, k, v, gates, B: int, topk_: int, scale: Optional[float] = None,
                forced: int = 0, own: bool = False):
    """Forward pass over every row, reassembled into token-major tensors:
    out/ocmp/osel [T, H, D], lse [H, T], score [H, Nb, Nb] float32, sel [H, Nb, n_sel]."""
    a = _f32(q)
    T, H, D = a.shape
    Nb = n_blocks(T, B)
    rows_h = np.repeat(np.arange(H), Nb)
    rows_i = np.tile(np.arange(Nb), H)
    r = forward_rows(q, k, v, gates, B, topk_, rows_h, rows_i, scale=scale, forced=forced,
                     own=own)
    k_eff = r["sel"].shape[1]
    full = {}
    for name in ("ocmp", "osel", "out"):
        x = r[name].reshape(H, Nb * B, D)[:, :T]          # [H, T, D]
        full[name] = np.ascontiguousarray(x.transpose(1, 0, 2))
    full["lse"] = r["lse"].reshape(H, Nb * B)[:, :T]
    full["score"] = r["score"].reshape(H, Nb, Nb)
    full["sel"] = r["sel"].reshape(H, Nb, k_eff)
    return full


def backward(q, k, v, gates, dout, B: int, sel, scale: Optional[float] = None):
    """Gradients of the forward pass with the selection `sel` ([H, Nb, n_sel], e.g. the
    forward's own choice) held fixed. dout is the gradient of out ([T, H, D]). Returns dq, dk,
    dv ([T, H, D] float64) and dgates (the shape of gates: [H, 2] or [T, H, 2])."""
    a, b, c = _f32(q), _f32(k), _f32(v)
    T, H, D = a.shape
    g = _f32(gates)
    gate_st = 0 if g.ndim == 2 else H * 2
    go = _f32(dout)
    s = np.ascontiguousarray(np.asarray(sel, dtype=np.int32))
    n_sel = s.shape[-1]
    dq = np.empty((T, H, D), np.float64)
    dk = np.empty((T, H, D), np.float64)
    dv = np.empty((T, H, D), np.float64)
    dg = np.empty(g.shape, np.float64)
    lib().s3r_oracle_backward(T, H, D, B, default_scale(D) if scale is None else scale, a,
                              H * D, D, b, H * D, D, c, H * D, D, g.reshape(-1), gate_st, go,
                              H * D, D, s.reshape(-1), n_sel, dq, dk, dv, dg)
    return {"dq": dq, "dk": dk, "dv": dv, "dgates": dg}


def window_order(views: int, special: int, grid_h: int, grid_w: int, win_h: int,
                 win_w: int) -> np.ndarray:
    """Token order that makes contiguous blocks spatial windows (2-D pooling windows).

    The compression branch pools by spatial downsampling of the patch grid (the summary,
    "Methodologie" 1) and the model takes image sides in multiples of 56 pixels, i.e. patch
    grids in multiples of 4 (README "Notice" 1). Reading used here: each view is `special`
    tokens followed by a row-major grid_h x grid_w patch grid; the grid is cut into
    win_h x win_w windows. Position p of the reordered sequence holds token order[p]:
    for each view, its windows in row-major window order, each window's patches row-major;
    after all views, every view's special tokens (view by view, in their own order).
    """
    if grid_h % win_h or grid_w % win_w:
        raise ValueError("windows must tile the patch grid")
    per_view = special + grid_h * grid_w
    order = []
    for v in range(views):
        base = v * per_view + special
        for a in range(grid_h // win_h):
            for b in range(grid_w // win_w):
                for r in range(win_h):
                    row = base + (a * win_h + r) * grid_w + b * win_w
                    order.extend(range(row, row + win_w))
    for v in range(views):
        order.extend(range(v * per_view, v * per_view + special))
    return np.asarray(order, dtype=np.int64)


def forward_windows(q, k, v, gates, B: int, topk_: int, layout: Sequence[int],
                    scale: Optional[float] = None, forced: int = 0, own: bool = False):
    """The forward pass on window-ordered tokens: reorder q, k, v (and per-token gates) by
    window_order(*layout), run forward_all, and put out/ocmp/osel back in the caller's token
    order. lse stays in the caller's order too; score and sel refer to blocks of the
    reordered sequence."""
    order = window_order(*layout)
    a, b, c = _f32(q), _f32(k), _f32(v)
    if order.size != a.shape[0]:
        raise ValueError("layout does not match the token count")
    g = _f32(gates)
    gp = g[order] if g.ndim == 3 else g
    r = forward_all(a[order], b[order], c[order], gp, B, topk_, scale=scale, forced=forced,
                    own=own)
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size)
    for name in ("out", "ocmp", "osel"):
        r[name] = np.ascontiguousarray(r[name][inv])
    r["lse"] = np.ascontiguousarray(r["lse"][:, inv])
    r["order"] = order
    return r


def timed(fn, *args, **kw):
    t0 = time.perf_counter()
    r = fn(*args, **kw)
    return r, time.perf_counter() - t0
