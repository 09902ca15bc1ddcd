"""Large bf16 values: the P.V products take fp16 value records, so bf16 values are held as
fp16 after a multiplication by 2^-8 (outputs multiplied back). Values up to about 1.68e7 in
magnitude must then give the oracle's outputs; a value beyond that limit must make exactly
the output elements that attend to it non-finite, never a wrong finite number."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_global_attention_block_amd import speed3r as S
from sparse_global_attention_block_amd import workloads as W
from tests.helpers import bf16_half_ulp, check_selection, cuda_inputs, host

pytestmark = pytest.mark.gpu

W_TINY = W.WORKLOADS["tiny_s"]  # 1024 tokens, 4 heads, B = 16, k = 8


def oracle_out(hx, w, gsel):
    """The oracle's output on the GPU's selection, after the selection itself is checked
    (values do not steer top-k, so it is the selection of the unmodified inputs)."""
    ref = O.forward_all(hx["q"], hx["k"], hx["v"], hx["gates"], w.block, w.topk)
    check_selection(gsel, ref["score"], ref["sel"], w.topk)
    H, Nb, T = w.H, gsel.shape[1], hx["q"].shape[0]
    r = O.forward_rows(hx["q"], hx["k"], hx["v"], hx["gates"], w.block, w.topk,
                       np.repeat(np.arange(H), Nb), np.tile(np.arange(Nb), H),
                       sel_in=gsel.reshape(H * Nb, -1))
    return np.ascontiguousarray(r["out"].reshape(H, Nb * w.block, 64)[:, :T].transpose(1, 0, 2))


def plant(v: torch.Tensor, values, seed=3):
    """Writes each value at a random (token, head, dim) of v; returns the positions."""
    rng = np.random.default_rng(seed)
    T, H, D = v.shape
    pos = []
    for x in values:
        t, h, d = int(rng.integers(T)), int(rng.integers(H)), int(rng.integers(D))
        v[t, h, d] = x
        pos.append((t, h, d))
    return pos


def test_large_values_in_range():
    """|v| from 6e4 (below fp16's maximum) to 1.6e7 (just below the represented limit),
    both signs, in the values of every head: out matches the oracle within the rounding of
    the output plus 1e-3 of the largest |v| of the head."""
    w = W_TINY
    x = cuda_inputs(w)
    vals = [6e4, -6e4, 1e5, -1e5, 1e6, 3e6, -1.6e7, 1.6e7]
    plant(x["v"], vals)
    T, H, D = x["q"].shape
    sel = torch.empty(H, T // w.block, w.topk, dtype=torch.int32, device="cuda")
    out, _ = S.sparse_attn_fwd(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk,
                               sel_idx=sel)
    torch.cuda.synchronize()
    hx = {n: host(t) for n, t in x.items()}
    ref = oracle_out(hx, w, sel.cpu().numpy())
    g = out.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(g).all(), "in-range values gave non-finite outputs"
    vmax = hx["v"].float().abs().amax(dim=(0, 2)).numpy()          # [H]
    excess = np.maximum(np.abs(g - ref) - bf16_half_ulp(ref), 0.0)
    worst = (excess.max(axis=(0, 2)) / vmax).max()
    print(f"[range] largest |v| per head {vmax}, worst error beyond output rounding "
          f"{worst:.2e} of it", flush=True)
    assert worst <= 1e-3


def test_value_beyond_the_limit_is_loud():
    """One value of 3e7 (beyond 65504 * 2^8): the output elements of its head and dim in the
    query blocks that select its key block are non-finite; every other output element is
    finite and matches the oracle (the block mean stays in range, so the compression branch
    is exact)."""
    w = W_TINY
    x = cuda_inputs(w)
    T, H, D = x["q"].shape
    Nb = T // w.block
    sel = torch.empty(H, Nb, w.topk, dtype=torch.int32, device="cuda")
    S.sparse_attn_fwd(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk, sel_idx=sel)
    torch.cuda.synchronize()
    # the value goes into the key block that head 1 selects most often (values do not steer
    # the selection, so it stays the same)
    h, d = 1, 7
    j = int(np.bincount(sel[h].cpu().numpy().ravel(), minlength=Nb).argmax())
    t = j * w.block + 3
    x["v"][t, h, d] = 3e7
    out, _ = S.sparse_attn_fwd(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk,
                               sel_idx=sel)
    torch.cuda.synchronize()
    g = out.float().cpu().numpy().astype(np.float64)
    s = sel.cpu().numpy()
    readers = np.nonzero((s[h] == j).any(axis=1))[0]               # query blocks selecting j
    assert readers.size > 0
    bad = np.zeros(g.shape, bool)
    for i in readers:
        bad[i * w.block:(i + 1) * w.block, h, d] = True
    print(f"[range] 3e7 at token {t} head {h} dim {d}: {readers.size} query blocks select "
          f"its block", flush=True)
    assert not np.isfinite(g[bad]).any(), "an output reading the out-of-range value is finite"
    assert np.isfinite(g[~bad]).all()
    hx = {n: host(tt) for n, tt in x.items()}
    ref = oracle_out(hx, w, s)
    excess = np.maximum(np.abs(g - ref) - bf16_half_ulp(ref), 0.0)[~bad]
    scale = np.abs(ref[~bad]).max()
    assert excess.max() <= 1e-3 * scale + 2e-2
