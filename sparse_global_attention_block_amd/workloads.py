"""Named workloads and seeded synthetic inputs for the sparse global attention path.

This module only draws random numbers and lays them out as tensors. It holds none of the
attention arithmetic, so the HIP library and the CPU oracle can both be fed from it.

Shapes follow the multi-view transformer setting that Speed3R accelerates (project README,
"Overview"; gist.science summary, "Technische samenvatting"): every view of a 518x518 image
cut into 14x14 patches contributes a 37x37 grid (1369 tokens) plus 5 special tokens (one
camera token and four register tokens), all views are concatenated along the token axis, and
global attention runs over the whole sequence with 16 heads of width 64.

Generators:
  * ``iid``: q, k, v ~ N(0, 1) * ``iid_scale`` independently.
  * ``structured``: x[t, h, :] = N(0, I_64) + alpha * e_view(t) @ W_h, with one 8-dim view
    embedding e_v ~ N(0, I_8) per view and per-head projections W ~ N(0, 1/8) of shape [8, 64].
    q and k share the projection (so tokens of the same view attract each other), v has its
    own. Optionally the k and v rows of each view's 5 special tokens are multiplied by
    ``special_mult`` to create heavy-hitter keys.
  * Window workloads (``grid`` set) add to q and k a smooth term of each patch's grid
    position: ``spatial`` * phi(row, col) @ W_pos[h], with phi the 8 features cos/sin of
    pi*m*row/grid_h and pi*m*col/grid_w (m = 1, 2), W_pos ~ N(0, 1/8) per head; zero on the
    special tokens.
  * Gates: sigmoid(N(0, 1)) per head and branch, shape [H, 2] (column 0 weights the
    compression branch, column 1 the selection branch).

Everything is drawn in float32 with a ``torch.Generator`` seeded per tensor, then rounded once
to bfloat16 (or float16 for ``dtype="fp16"``; round to nearest even). Both sides of a parity check consume the same bfloat16
values: the GPU path directly, the oracle after an exact upcast to float.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import torch

D_HEAD = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    views: int
    tokens_per_view: int
    special: int          # special tokens at the start of each view
    H: int
    block: int
    topk: int
    gen: str              # "iid" or "structured"
    seed: int
    iid_scale: float = 1.0
    alpha: float = 0.5
    special_mult: float = 1.0
    D: int = D_HEAD
    forced: int = 0       # leading key blocks every query block attends (reference view)
    grid: Optional[Tuple[int, int]] = None    # patch grid (rows, cols) after the specials
    window: Optional[Tuple[int, int]] = None  # 2-D pooling window (rows, cols): window order
    spatial: float = 0.0  # weight of the smooth 2-D position term (grid workloads only)
    dtype: str = "bf16"   # element type of q, k, v: "bf16" or "fp16"
    own: bool = False     # each query block also keeps its own key block

    @property
    def T(self) -> int:
        return self.views * self.tokens_per_view

    @property
    def n_blocks(self) -> int:
        return -(-self.T // self.block)

    def layout(self, views: Optional[int] = None):
        """(views, special, grid_h, grid_w, win_h, win_w) of a window workload, else None."""
        if self.window is None:
            return None
        return (views or self.views, self.special, *self.grid, *self.window)

    @property
    def k_eff(self) -> int:
        """Entries per selection row: the forced blocks (and own block) plus the chosen ones."""
        f = min(self.forced, self.n_blocks)
        o = 1 if self.own and f < self.n_blocks else 0
        return f + o + min(self.topk, self.n_blocks - f - o)

    def describe(self) -> Dict:
        return {
            "workload": self.name, "views": self.views, "tokens_per_view": self.tokens_per_view,
            "T": self.T, "H": self.H, "D": self.D, "block": self.block, "topk": self.topk,
            "generator": self.gen, "seed": self.seed,
            "dtype": self.dtype,
            **({"forced_blocks": self.forced} if self.forced else {}),
            **({"own_block": True} if self.own else {}),
            **({"grid": list(self.grid)} if self.grid else {}),
            **({"window": list(self.window), "spatial": self.spatial} if self.window else {}),
            **({"iid_scale": self.iid_scale} if self.gen == "iid" else
               {"alpha": self.alpha, "special_tokens": self.special,
                "special_kv_mult": self.special_mult}),
        }


WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    # 4 views of a 16x16 grid, iid N(0,1)/8 inputs, block 16, top-8.
    Workload("tiny", 4, 256, 0, 4, 16, 8, "iid", seed=0, iid_scale=1.0 / 8.0),
    # same, k = all 64 blocks (selection branch then equals dense attention)
    Workload("tiny_all", 4, 256, 0, 4, 16, 64, "iid", seed=0, iid_scale=1.0 / 8.0),
    # same shape with the structured generator, so that top-k has clear winners
    Workload("tiny_s", 4, 256, 0, 4, 16, 8, "structured", seed=1),
    # 8 views of the full per-view shape (used for quick parity at the real block size)
    Workload("v8", 8, 1374, 5, 16, 64, 16, "structured", seed=8, special_mult=3.0),
    Workload("v32", 32, 1374, 5, 16, 64, 16, "structured", seed=32),
    Workload("v100", 100, 1374, 5, 16, 64, 16, "structured", seed=100, special_mult=3.0),
    Workload("v1000_k16", 1000, 1374, 5, 16, 64, 16, "structured", seed=1000, special_mult=3.0),
    Workload("v1000_k32", 1000, 1374, 5, 16, 64, 32, "structured", seed=1000, special_mult=3.0),
    # k = 48: the largest k for which the automatic mode takes the single compression pass
    Workload("v1000_k48", 1000, 1374, 5, 16, 64, 48, "structured", seed=1000, special_mult=3.0),
    # same as v1000_k16, with the 22 key blocks that cover the first (reference) view attended
    # by every query block in addition to its top-16
    Workload("v1000_k16_ref", 1000, 1374, 5, 16, 64, 16, "structured", seed=1000,
             special_mult=3.0, forced=22),
    # ... and each query block also attending its own key block
    Workload("v1000_k16_ref_own", 1000, 1374, 5, 16, 64, 16, "structured", seed=1000,
             special_mult=3.0, forced=22, own=True),
    # the same in fp16 (the model runs in bf16 or fp16)
    Workload("v1000_k16_fp16", 1000, 1374, 5, 16, 64, 16, "structured", seed=1000,
             special_mult=3.0, dtype="fp16"),
    # 2-D windows: 560x560 images (a multiple of 56) give a 40x40 patch grid; 8x8 windows are
    # the 64-token blocks; a smooth position term makes nearby patches alike
    Workload("v1000_win8", 1000, 5 + 40 * 40, 5, 16, 64, 16, "structured", seed=1001,
             special_mult=3.0, grid=(40, 40), window=(8, 8), spatial=0.5),
    # 504x504 images: 36x36 grid in 4x4 windows of 16 tokens
    Workload("v8_win4", 8, 5 + 36 * 36, 5, 4, 16, 8, "structured", seed=9, special_mult=3.0,
             grid=(36, 36), window=(4, 4), spatial=0.5),
]}


def _gen(seed: int, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1009 + stream)
    return g


def _randn(shape, seed, stream, device, std=1.0):
    return torch.randn(shape, generator=_gen(seed, stream, device), device=device,
                       dtype=torch.float32) * std


def make_inputs(w: Workload, device="cpu", T: Optional[int] = None,
                views: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Return q, k, v as contiguous [T, H, 64] tensors of the workload's type (bfloat16 or
    float16) and gates [H, 2] float32.

    ``views`` (or ``T``) overrides the length of the sequence while keeping the recipe, which
    is how tests build small instances of a large workload.
    """
    nv = views if views is not None else w.views
    TT = T if T is not None else nv * w.tokens_per_view
    nv = max(1, -(-TT // w.tokens_per_view))
    H, D = w.H, w.D
    dev = torch.device(device)
    elt = {"bf16": torch.bfloat16, "fp16": torch.float16}[w.dtype]
    out = {}
    if w.gen == "iid":
        for i, name in enumerate(("q", "k", "v")):
            x = _randn((TT, H, D), w.seed, i, dev, w.iid_scale)
            out[name] = x.to(elt)
    elif w.gen == "structured":
        e = _randn((nv, 8), w.seed, 10, dev)                         # view embeddings
        w_qk = _randn((H, 8, D), w.seed, 11, dev, math.sqrt(1.0 / 8.0))
        w_v = _randn((H, 8, D), w.seed, 12, dev, math.sqrt(1.0 / 8.0))
        view_of_t = torch.div(torch.arange(TT, device=dev), w.tokens_per_view,
                              rounding_mode="floor")
        emb_qk = torch.einsum("ve,hed->vhd", e, w_qk)                # [views, H, D]
        emb_v = torch.einsum("ve,hed->vhd", e, w_v)
        pos = torch.arange(TT, device=dev) % w.tokens_per_view
        special = (pos < w.special) if w.special > 0 else None
        pos_qk = None
        if w.grid is not None and w.spatial != 0.0:
            # smooth position term on the patch grid: 8 Fourier features of (row, col)
            # projected per head (q and k share it, so nearby patches attract)
            gh, gw = w.grid
            cell = (pos - w.special).clamp(min=0)
            r = torch.div(cell, gw, rounding_mode="floor").float() / gh
            c = (cell % gw).float() / gw
            feats = torch.stack([f(math.pi * m * x) for x in (r, c) for m in (1, 2)
                                 for f in (torch.cos, torch.sin)], dim=1)  # [TT, 8]
            feats[pos < w.special] = 0.0
            w_pos = _randn((H, 8, D), w.seed, 13, dev, math.sqrt(1.0 / 8.0))
            pos_qk = feats, w_pos
        for i, name in enumerate(("q", "k", "v")):
            x = _randn((TT, H, D), w.seed, i, dev)
            x.add_((emb_v if name == "v" else emb_qk)[view_of_t], alpha=w.alpha)
            if pos_qk is not None and name != "v":
                x.add_(torch.einsum("tf,hfd->thd", *pos_qk), alpha=w.spatial)
            if name in ("k", "v") and special is not None and w.special_mult != 1.0:
                x[special] *= w.special_mult
            out[name] = x.to(elt)
            del x
    else:
        raise ValueError(f"unknown generator {w.gen!r}")
    out["gates"] = torch.sigmoid(_randn((H, 2), w.seed, 7, dev))
    return out
