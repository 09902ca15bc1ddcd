"""GPU parity of the 2-D window path: the reordering kernel against the oracle's window order
(byte-exact), and speed3r_sparse_attn_fwd_windows against the oracle's windowed forward."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_global_attention_block_amd import speed3r as S
from sparse_global_attention_block_amd import workloads as W
from tests.helpers import check_out, check_selection, cuda_inputs, host, own_rows

pytestmark = pytest.mark.gpu

_w4 = W.WORKLOADS["v8_win4"]
_w8 = W.WORKLOADS["v1000_win8"]
CASES = {
    # 4x4 windows of a 36x36 grid as blocks of 16, 2 views (T = 2602, ragged special tail)
    "win4_b16": (dataclasses.replace(_w4, views=2), {}),
    # 8x8 windows of a 40x40 grid as blocks of 64, 3 views, 16 heads
    "win8_b64": (dataclasses.replace(_w8, views=3), {}),
    # the same with the first view's 25 windows forced
    "win8_forced": (dataclasses.replace(_w8, views=3, forced=25), {}),
    # ... and each window block also keeping itself
    "win8_forced_own": (dataclasses.replace(_w8, views=3, forced=25, own=True), {}),
    # fp16 inputs and output
    "win8_fp16": (dataclasses.replace(_w8, views=3, dtype="fp16"), {}),
    # 4x4 windows grouped four to a block of 64 (4x16 strips), per-token gates, no specials
    "win4_b64_strips": (dataclasses.replace(_w4, views=2, special=0, tokens_per_view=36 * 36,
                                            block=64, topk=4, H=2), {"token_gates": True}),
    # no special tokens and full-width one-row windows: the plain forward
    "rows_identity": (dataclasses.replace(_w4, views=2, special=0, tokens_per_view=36 * 36,
                                          window=(1, 36)), {}),
}


@pytest.mark.parametrize("layout", [(2, 1, 4, 4, 2, 2), (3, 5, 8, 12, 4, 4), (2, 5, 40, 40, 8, 8)])
def test_window_permute_byte_exact(layout):
    V, Sp, Gh, Gw, wh, ww = layout
    T, H = V * (Sp + Gh * Gw), 3
    print(f"[permute] layout {layout} T={T}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(11)
    base = torch.randn(T, 2 * H, 64, generator=g, device="cuda").to(torch.bfloat16)
    src = base[:, ::2]                                  # strided heads
    fwd = S.window_permute(layout, src)
    back = S.window_permute(layout, fwd, inverse=True)
    torch.cuda.synchronize()
    order = torch.from_numpy(O.window_order(*layout)).cuda()
    assert torch.equal(fwd, src[order])
    assert torch.equal(back, src)


def run_case(name):
    w, opt = CASES[name]
    layout = w.layout()
    print(f"[case {name}] layout {layout} T={w.T} H={w.H} B={w.block} k={w.topk} F={w.forced} "
          f"own={w.own}", flush=True)
    x = cuda_inputs(w)
    gates = x["gates"]
    if opt.get("token_gates"):
        gates = torch.rand(w.T, w.H, 2, device="cuda",
                           generator=torch.Generator(device="cuda").manual_seed(3))
    p = S.make_params(x["q"], x["k"], x["v"], w.block, w.topk, 0.0, gates, w.forced, w.own)
    sel = torch.empty(w.H, S.num_blocks(p), S.num_selected(p), dtype=torch.int32, device="cuda")
    out, _ = S.sparse_attn_fwd_windows(x["q"], x["k"], x["v"], gates, w.block, w.topk, layout,
                                       sel_idx=sel, forced_blocks=w.forced, force_own=w.own)
    torch.cuda.synchronize()
    hx = {n: host(t) for n, t in x.items()}
    hg = host(gates)
    ora = O.forward_windows(hx["q"], hx["k"], hx["v"], hg, w.block, w.topk, layout,
                            forced=w.forced, own=w.own)
    return w, layout, x, hx, hg, out, host(sel).numpy(), ora


@pytest.mark.parametrize("name", list(CASES))
def test_windowed_forward_against_oracle(name):
    w, layout, x, hx, hg, out, gsel, ora = run_case(name)
    H, Nb = gsel.shape[:2]
    F = min(w.forced, Nb)
    frac, diff = check_selection(gsel, ora["score"], ora["sel"], w.topk, forced=F,
                                 qblocks=own_rows(H, Nb, w.own and F < Nb), dtype=w.dtype)
    print(f"[{name}] exact-index rows {frac:.1%}, near-tie rows differing {len(diff)}")
    ref = ora["out"]
    if not np.array_equal(gsel, ora["sel"]):
        # rows where a near-tie flipped the set: the oracle on the GPU's own indices
        order = ora["order"]
        gp = hg[order] if hg.dim() == 3 else hg
        r = O.forward_rows(hx["q"][order], hx["k"][order], hx["v"][order], gp, w.block, w.topk,
                           np.repeat(np.arange(H), Nb), np.tile(np.arange(Nb), H),
                           sel_in=gsel.reshape(H * Nb, -1), forced=w.forced, own=w.own)
        T = x["q"].shape[0]
        perm_out = r["out"].reshape(H, Nb * w.block, 64)[:, :T].transpose(1, 0, 2)
        ref = np.empty_like(perm_out)
        ref[order] = perm_out
    mx, mean = check_out(out, ref)
    print(f"[{name}] out max-abs {mx:.3e} mean-abs {mean:.3e}")


def test_identity_layout_equals_plain_forward():
    """Full-width one-row windows and no specials: byte-identical to speed3r_sparse_attn_fwd."""
    w, _ = CASES["rows_identity"]
    x = cuda_inputs(w)
    a, _ = S.sparse_attn_fwd_windows(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk,
                                     w.layout())
    b, _ = S.sparse_attn_fwd(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
