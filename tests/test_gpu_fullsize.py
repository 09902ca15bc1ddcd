"""Parity at the full workload sizes (32, 100 and 1000 views of 1374 tokens, 16 heads), run
through speed3r_sparse_attn_fwd exactly as the benchmark launches it. The oracle recomputes a
sample of (head, query block) rows one by one: the first block, the short last block, a block
holding a view's special tokens, and random blocks."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_global_attention_block_amd import speed3r as S
from sparse_global_attention_block_amd import workloads as W
from tests.helpers import check_out, check_selection, cuda_inputs

pytestmark = pytest.mark.gpu


def sample_rows(w: W.Workload, n_random: int, seed: int):
    Nb = w.n_blocks
    rng = np.random.default_rng(seed)
    mid_view_start = (w.views // 2) * w.tokens_per_view
    rows = {0, Nb - 1, mid_view_start // w.block, (mid_view_start + w.tokens_per_view) // w.block}
    rows.update(int(r) for r in rng.integers(0, Nb, n_random))
    return sorted(r for r in rows if r < Nb)


@pytest.mark.parametrize("name", ["v32", "v100", "v1000_k16", "v1000_k32", "v1000_k16_ref",
                                  "v1000_k16_ref_own", "v1000_k16_fp16"])
def test_fullsize_sampled_rows(name):
    w = W.WORKLOADS[name]
    print(f"[fullsize {name}] T={w.T} H={w.H} B={w.block} k={w.topk} F={w.forced} own={w.own}",
          flush=True)
    x = cuda_inputs(w)
    Nb, k_eff = w.n_blocks, w.k_eff
    sel = torch.empty(w.H, Nb, k_eff, dtype=torch.int32, device="cuda")
    out, _ = S.sparse_attn_fwd(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk, sel_idx=sel,
                               forced_blocks=w.forced, force_own=w.own)
    torch.cuda.synchronize()
    rows = sample_rows(w, 3, w.seed)
    heads = [0, w.H - 1]
    for h in heads:
        hq, hk, hv = (x[n][:, h:h + 1].contiguous().cpu() for n in ("q", "k", "v"))
        hg = x["gates"][h:h + 1].cpu()
        kc, vc = O.pool(hk, w.block), O.pool(hv, w.block)
        zeros = np.zeros(len(rows), np.int32)
        ora = O.forward_rows(hq, hk, hv, hg, w.block, w.topk, zeros, rows, kc=kc, vc=vc,
                             forced=w.forced, own=w.own)
        gsel = sel[h, rows].cpu().numpy()
        F = min(w.forced, Nb)
        frac, differing = check_selection(gsel, ora["score"], ora["sel"], w.topk, forced=F,
                                          qblocks=rows if w.own and F < Nb else None)
        ref = ora
        if differing:
            ref = O.forward_rows(hq, hk, hv, hg, w.block, w.topk, zeros, rows, kc=kc, vc=vc,
                                 sel_in=gsel, forced=w.forced, own=w.own)
        for a, i in enumerate(rows):
            n = min(w.T, (i + 1) * w.block) - i * w.block
            check_out(out[i * w.block:i * w.block + n, h], ref["out"][a, :n],
                      what=f"{name} h={h} block={i}")
        print(f"[fullsize {name}] head {h}: rows {rows} exact-index fraction {frac:.0%}, "
              f"near-tie rows {len(differing)}", flush=True)
    del x, out, sel
    torch.cuda.empty_cache()


def test_fullsize_windows_sampled_rows():
    """1000 views of 560x560 images (5 special tokens + a 40x40 grid, 8x8 windows as the
    64-token blocks, 25,079 blocks) through speed3r_sparse_attn_fwd_windows; the oracle
    reorders each sampled head itself and recomputes sampled query blocks."""
    w = W.WORKLOADS["v1000_win8"]
    layout = w.layout()
    print(f"[fullsize {w.name}] T={w.T} H={w.H} B={w.block} k={w.topk} layout={layout}",
          flush=True)
    x = cuda_inputs(w)
    Nb, k_eff = w.n_blocks, w.k_eff
    sel = torch.empty(w.H, Nb, k_eff, dtype=torch.int32, device="cuda")
    out, _ = S.sparse_attn_fwd_windows(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk,
                                       layout, sel_idx=sel)
    torch.cuda.synchronize()
    order = O.window_order(*layout)
    grid_blocks = w.views * w.grid[0] * w.grid[1] // w.block
    rng = np.random.default_rng(w.seed)
    rows = sorted({0, 1, grid_blocks - 1, grid_blocks, Nb - 1,
                   *(int(r) for r in rng.integers(0, Nb, 3))})
    idx = torch.from_numpy(order)
    for h in (0, w.H - 1):
        hq, hk, hv = (x[n][:, h:h + 1].cpu()[idx].contiguous() for n in ("q", "k", "v"))
        hg = x["gates"][h:h + 1].cpu()
        kc, vc = O.pool(hk, w.block), O.pool(hv, w.block)
        zeros = np.zeros(len(rows), np.int32)
        ora = O.forward_rows(hq, hk, hv, hg, w.block, w.topk, zeros, rows, kc=kc, vc=vc)
        gsel = sel[h, rows].cpu().numpy()
        frac, differing = check_selection(gsel, ora["score"], ora["sel"], k_eff)
        ref = ora
        if differing:
            ref = O.forward_rows(hq, hk, hv, hg, w.block, w.topk, zeros, rows, kc=kc, vc=vc,
                                 sel_in=gsel)
        for a, i in enumerate(rows):
            n = min(w.T, (i + 1) * w.block) - i * w.block
            toks = torch.from_numpy(order[i * w.block:i * w.block + n]).cuda()
            check_out(out[toks, h], ref["out"][a, :n], what=f"{w.name} h={h} block={i}")
        print(f"[fullsize {w.name}] head {h}: rows {rows} exact-index fraction {frac:.0%}, "
              f"near-tie rows {len(differing)}", flush=True)
    del x, out, sel
    torch.cuda.empty_cache()
