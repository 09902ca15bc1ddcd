"""Pins of the CPU oracle against facts fixed by the mathematics (no GPU).

The pages print no numeric example of the method, so the oracle is pinned by a hand-derived
worked example (tests/golden), by special cases that reduce to textbook attention (computed
here with torch's CPU scaled_dot_product_attention / softmax in float64), by invariants of
the definition, and by brute force on tiny inputs. Each test names the slip it would catch.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import oracle as O
from sparse_global_attention_block_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_tensor(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16)


def sdpa(q, k, v, scale, mask=None):
    """Textbook softmax attention, [T, H, D] float tensors, float64, via torch."""
    qh, kh, vh = (x.double().permute(1, 0, 2) for x in (q, k, v))
    o = F.scaled_dot_product_attention(qh.unsqueeze(0), kh.unsqueeze(0), vh.unsqueeze(0),
                                       attn_mask=mask, scale=scale)[0]
    return o.permute(1, 0, 2).numpy()


def s(x):
    return 1.0 / (1.0 + math.exp(-x))


# ----------------------------------------------------------------------------- worked example
def test_worked_example_closed_forms():
    """Hand-derived example (golden/worked_example.md): catches any slip in pooling, scale,
    softmax, score summation, top-k direction, block-to-token mapping and gating."""
    ex = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    T, H, D, B = ex["T"], ex["H"], ex["D"], ex["B"]
    q = np.array(ex["q"], np.float32).reshape(T, H, D)
    k = np.array(ex["k"], np.float32).reshape(T, H, D)
    v = np.array(ex["v"], np.float32).reshape(T, H, D)
    g = np.array(ex["gates"], np.float32).reshape(H, 2)
    r = O.forward_all(q, k, v, g, B, ex["topk"], scale=ex["scale"])
    kc = O.pool(k, B)
    vc = O.pool(v, B)
    np.testing.assert_array_equal(kc[0], [[2, 0], [0, 2]])
    np.testing.assert_array_equal(vc[0], [[2, 0], [0, 2]])
    e = math.e
    lse = [math.log(e ** 2 + 1)] * 3 + [math.log(1 + e)]
    ocmp = [(2 * s(2), 2 * s(-2)), (2 * s(2), 2 * s(-2)), (2 * s(-2), 2 * s(2)),
            (2 * s(-1), 2 * s(1))]
    score = [(2 * s(2), 2 * s(-2)), (s(-2) + s(-1), s(2) + s(1))]
    osel = [(1 + 2 * s(2), 0), (1 + 2 * s(2), 0), (0, 4 * s(-2)), (0, 4 * s(-1))]
    out = [tuple(0.25 * a + 0.75 * b for a, b in zip(x, y)) for x, y in zip(ocmp, osel)]
    np.testing.assert_allclose(r["lse"][0], lse, rtol=0, atol=1e-14)
    np.testing.assert_allclose(r["ocmp"][:, 0], ocmp, rtol=0, atol=1e-14)
    np.testing.assert_allclose(r["score"][0], np.array(score, np.float32), rtol=0, atol=0)
    np.testing.assert_array_equal(r["sel"][0], [[0], [1]])
    np.testing.assert_allclose(r["osel"][:, 0], osel, rtol=0, atol=1e-14)
    np.testing.assert_allclose(r["out"][:, 0], out, rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------- pooling
def test_pool_identical_keys_exact_including_short_last_block():
    """A block of identical keys pools to exactly that key; the short last block (4 of 16
    tokens) must be divided by its own length, not by B."""
    T, H, D, B = 100, 3, 64, 16
    base = bf16_tensor((7, H, D), 1).float()
    x = base[torch.arange(T) // B]
    kc = O.pool(x, B)
    for j in range(7):
        np.testing.assert_array_equal(kc[:, j], base[j].double().numpy())


def test_pool_block1_is_identity_and_translation():
    T, H, D = 37, 2, 64
    x = bf16_tensor((T, H, D), 2).float()
    np.testing.assert_array_equal(O.pool(x, 1), x.double().permute(1, 0, 2).numpy())
    c = 0.5
    a = O.pool(x, 8)
    b = O.pool(x + c, 8)
    np.testing.assert_allclose(b, a + c, rtol=0, atol=1e-6)


# ----------------------------------------------------------------------------- compression
@pytest.mark.parametrize("T", [40, 33])
def test_block1_compression_is_dense_attention(T):
    """With B = 1 every token is its own coarse token: LSE, O_cmp and the score matrix must be
    textbook attention's log-sum-exp, output and probability matrix."""
    H, D = 2, 64
    q, k, v = (bf16_tensor((T, H, D), 10 + i, 0.5) for i in range(3))
    g = torch.tensor([[1.0, 0.0]] * H)
    r = O.forward_all(q, k, v, g, 1, 4)
    scale = 1 / 8
    logits = torch.einsum("thd,uhd->htu", q.double(), k.double()) * scale
    np.testing.assert_allclose(r["lse"], torch.logsumexp(logits, -1).numpy(), atol=1e-12)
    np.testing.assert_allclose(r["ocmp"], sdpa(q, k, v, scale), atol=1e-12)
    np.testing.assert_allclose(r["score"], torch.softmax(logits, -1).float().numpy(),
                               rtol=1e-6, atol=1e-7)


def test_compression_is_attention_over_block_means():
    """General B (ragged tail): O_cmp is softmax attention over numpy block means."""
    T, H, D, B = 90, 2, 64, 16
    q, k, v = (bf16_tensor((T, H, D), 20 + i, 0.7) for i in range(3))
    Nb = -(-T // B)
    def means(x):
        a = x.double().numpy()
        return np.stack([a[j * B:min(T, (j + 1) * B)].mean(0) for j in range(Nb)])  # [Nb,H,D]
    kc, vc = means(k), means(v)
    r = O.forward_all(q, k, v, torch.ones(H, 2), B, 2)
    ref = sdpa(q, torch.from_numpy(kc), torch.from_numpy(vc), 1 / 8)
    np.testing.assert_allclose(r["ocmp"], ref, atol=1e-12)


def test_softmax_rows_and_score_rows_sum():
    """Probabilities of a query sum to one; summed over a block's n_i queries the score row
    must therefore sum to n_i (64 ... 64, then 26 for the ragged last block)."""
    T, H, D, B = 8 * 64 + 26, 2, 64, 64
    q, k, v = (bf16_tensor((T, H, D), 30 + i) for i in range(3))
    r = O.forward_all(q, k, v, torch.ones(H, 2), B, 3)
    n = np.array([64] * 8 + [26], np.float64)
    np.testing.assert_allclose(r["score"].astype(np.float64).sum(-1), np.tile(n, (H, 1)),
                               rtol=2e-6)
    assert (r["score"] >= 0).all()


def test_identical_keys_give_uniform_attention():
    """All keys equal -> every coarse logit equal -> P uniform 1/Nb, O_cmp = mean of Vc."""
    T, H, D, B = 96, 1, 64, 16
    q = bf16_tensor((T, H, D), 40)
    k = bf16_tensor((1, H, D), 41).expand(T, H, D).contiguous()
    v = bf16_tensor((T, H, D), 42)
    r = O.forward_all(q, k, v, torch.ones(H, 2), B, 2)
    vc = O.pool(v, B)
    np.testing.assert_allclose(r["ocmp"][:, 0], np.tile(vc[0].mean(0), (T, 1)), atol=1e-13)
    np.testing.assert_allclose(r["score"][0], np.full((6, 6), 16 / 6, np.float32), rtol=1e-6)


def test_key_block_permutation_permutes_scores():
    """Moving whole key/value blocks moves the score columns and the chosen indices with
    them (catches a score column written to the wrong block)."""
    T, H, D, B = 128, 2, 64, 16
    w = W.WORKLOADS["tiny_s"]
    x = W.make_inputs(w, T=T)
    perm = np.array([3, 0, 7, 5, 1, 6, 2, 4])
    tok = torch.from_numpy((perm[:, None] * B + np.arange(B)[None]).reshape(-1))
    a = O.forward_all(x["q"], x["k"], x["v"], x["gates"], B, 3)
    b = O.forward_all(x["q"], x["k"][tok], x["v"][tok], x["gates"], B, 3)
    np.testing.assert_allclose(b["score"], a["score"][:, :, perm], rtol=1e-5, atol=1e-6)
    inv = np.argsort(perm)
    mapped = np.sort(inv[a["sel"]], axis=-1)
    np.testing.assert_array_equal(b["sel"], mapped)
    np.testing.assert_allclose(b["osel"], a["osel"], atol=1e-12)


# ----------------------------------------------------------------------------- top-k
def brute_topk(row, k):
    idx = np.lexsort((np.arange(row.size), -row.astype(np.float64)))
    return np.sort(idx[:min(k, row.size)])


@pytest.mark.parametrize("levels", [None, 3, 1])
def test_topk_brute_force_with_ties(levels):
    rng = np.random.default_rng(5)
    for n in (1, 7, 64, 300, 2047):
        for k in (1, 8, 16, 32, n, n + 3):
            row = rng.random(n).astype(np.float32)
            if levels is not None:
                row = (np.floor(row * levels) / max(levels, 1)).astype(np.float32)
            np.testing.assert_array_equal(O.topk(row, k), brute_topk(row, k))


def test_topk_all_equal_takes_smallest_indices():
    np.testing.assert_array_equal(O.topk(np.full(50, 0.25, np.float32), 8), np.arange(8))


def test_heavy_hitter_block_is_always_selected():
    """A key block whose keys are a large multiple of the mean query must win top-1 on every
    row (catches selecting the smallest scores)."""
    T, H, D, B = 256, 2, 64, 16
    q = bf16_tensor((T, H, D), 50).float() + 0.5
    k = bf16_tensor((T, H, D), 51).float()
    hot = 11
    k[hot * B:(hot + 1) * B] = 4.0 * q.mean(0, keepdim=True)
    v = bf16_tensor((T, H, D), 52).float()
    r = O.forward_all(q, k, v, torch.ones(H, 2), B, 1)
    assert (r["sel"][..., 0] == hot).all()


# ----------------------------------------------------------------------------- selection
@pytest.mark.parametrize("name", ["tiny_all"])
def test_all_blocks_selected_is_dense_attention(name):
    """k = all blocks: the selection branch must equal dense attention (the contract's own
    brute-force check), here against torch's SDPA in float64."""
    w = W.WORKLOADS[name]
    x = W.make_inputs(w)
    r = O.forward_all(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk)
    np.testing.assert_allclose(r["osel"], sdpa(x["q"], x["k"], x["v"], 1 / 8), atol=1e-12)
    np.testing.assert_allclose(O.dense_rows(x["q"], x["k"], x["v"], 1, 100, 20),
                               sdpa(x["q"], x["k"], x["v"], 1 / 8)[100:120, 1], atol=1e-12)


def test_selection_equals_masked_attention():
    """For any selection, O_sel is SDPA with a boolean mask that admits exactly the tokens of
    the chosen blocks (catches block/token index slips and duplicate handling)."""
    T, H, D, B, k = 100, 2, 64, 16, 3
    w = W.WORKLOADS["tiny_s"]
    x = W.make_inputs(w, T=T)
    r = O.forward_all(x["q"], x["k"], x["v"], x["gates"], B, k)
    Nb = -(-T // B)
    blk = torch.arange(T) // B
    for h in range(H):
        mask = torch.zeros(T, T, dtype=torch.bool)
        for i in range(Nb):
            rows = blk == i
            cols = torch.isin(blk, torch.from_numpy(r["sel"][h, i].astype(np.int64)))
            mask[rows.nonzero()[:, None, 0], cols.nonzero()[None, :, 0]] = True
        ref = sdpa(x["q"][:, h:h + 1], x["k"][:, h:h + 1], x["v"][:, h:h + 1], 1 / 8,
                   mask=mask.unsqueeze(0))
        np.testing.assert_allclose(r["osel"][:, h], ref[:, 0], atol=1e-12)
    # a duplicated index in an externally supplied list counts once
    sel = np.array([[2, 2, 5]], np.int32)
    a = O.forward_rows(x["q"], x["k"], x["v"], x["gates"], B, 3, [0], [1], sel_in=sel)
    b = O.sel_row(x["q"], x["k"], x["v"], B, 0, 1, [2, 5])
    np.testing.assert_allclose(a["osel"][0], b, atol=1e-14)


# ----------------------------------------------------------------------------- gating, linearity
def test_gates_isolate_branches_and_value_linearity():
    w = W.WORKLOADS["tiny_s"]
    x = W.make_inputs(w, T=200)
    B, k = 16, 4
    a = O.forward_all(x["q"], x["k"], x["v"], torch.tensor([[1.0, 0.0]] * w.H), B, k)
    np.testing.assert_allclose(a["out"], a["ocmp"], atol=0)
    b = O.forward_all(x["q"], x["k"], x["v"], torch.tensor([[0.0, 1.0]] * w.H), B, k)
    np.testing.assert_allclose(b["out"], b["osel"], atol=0)
    # outputs are linear in V (the selection depends on q and k only)
    v2 = bf16_tensor(tuple(x["v"].shape), 60)
    g = x["gates"]
    r1 = O.forward_all(x["q"], x["k"], x["v"], g, B, k)
    r2 = O.forward_all(x["q"], x["k"], v2, g, B, k)
    r12 = O.forward_all(x["q"], x["k"], x["v"].float() + v2.float(), g, B, k)
    np.testing.assert_array_equal(r12["sel"], r1["sel"])
    np.testing.assert_allclose(r12["out"], r1["out"] + r2["out"], atol=1e-12)


def test_per_token_gates():
    """Per-token gates [T, H, 2] are read per token (the per-token gating reading)."""
    w = W.WORKLOADS["tiny_s"]
    x = W.make_inputs(w, T=64)
    gt = torch.rand(64, w.H, 2, generator=torch.Generator().manual_seed(3))
    r = O.forward_all(x["q"], x["k"], x["v"], gt, 16, 2)
    ref = gt[..., :1].double().numpy() * r["ocmp"] + gt[..., 1:].double().numpy() * r["osel"]
    np.testing.assert_allclose(r["out"], ref, atol=1e-14)


# ----------------------------------------------------------------------------- workload facts
def test_tiny_iid_has_no_clear_topk_rows_but_tiny_s_does():
    """The iid N(0,1)/8 workload makes every block score ~n/Nb, so no row has a top-k gap
    above 1e-3 and index parity is vacuous there; the structured tiny_s workload fixes that."""
    def gap_fraction(name):
        w = W.WORKLOADS[name]
        x = W.make_inputs(w)
        r = O.forward_all(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk)
        sc = -np.sort(-r["score"].astype(np.float64), axis=-1)
        gap = sc[..., w.topk - 1] - sc[..., w.topk]
        return (gap > 1e-3).mean()
    assert gap_fraction("tiny") == 0.0
    assert gap_fraction("tiny_s") > 0.5


# ----------------------------------------------------------------------------- forced blocks
@pytest.mark.parametrize("forced", [1, 3, 7])
def test_forced_prefix_then_topk_of_the_rest(forced):
    """Forced reference blocks (the VGGT hybrid keeps the reference frame dense): the first F
    blocks are always kept and the other k are the brute-force top-k of the remaining scores;
    the selection branch is masked SDPA over exactly those blocks."""
    T, B, k = 320, 16, 4
    w = W.WORKLOADS["tiny_s"]
    x = W.make_inputs(w, T=T)
    r = O.forward_all(x["q"], x["k"], x["v"], x["gates"], B, k, forced=forced)
    Nb = -(-T // B)
    assert r["sel"].shape[-1] == O.num_selected(T, B, k, forced) == forced + k
    for h in range(w.H):
        for i in range(Nb):
            row = r["sel"][h, i]
            np.testing.assert_array_equal(row[:forced], np.arange(forced))
            np.testing.assert_array_equal(row[forced:], forced + brute_topk(r["score"][h, i, forced:], k))
    blk = torch.arange(T) // B
    h = 1
    mask = torch.zeros(T, T, dtype=torch.bool)
    for i in range(Nb):
        cols = torch.isin(blk, torch.from_numpy(r["sel"][h, i].astype(np.int64)))
        mask[(blk == i).nonzero()[:, None, 0], cols.nonzero()[None, :, 0]] = True
    ref = sdpa(x["q"][:, h:h + 1], x["k"][:, h:h + 1], x["v"][:, h:h + 1], 1 / 8,
               mask=mask.unsqueeze(0))
    np.testing.assert_allclose(r["osel"][:, h], ref[:, 0], atol=1e-12)


def test_forced_zero_is_the_plain_method_and_all_forced_is_dense():
    w = W.WORKLOADS["tiny_s"]
    x = W.make_inputs(w, T=200)
    a = O.forward_all(x["q"], x["k"], x["v"], x["gates"], 16, 3)
    b = O.forward_all(x["q"], x["k"], x["v"], x["gates"], 16, 3, forced=0)
    np.testing.assert_array_equal(a["sel"], b["sel"])
    np.testing.assert_array_equal(a["out"], b["out"])
    c = O.forward_all(x["q"], x["k"], x["v"], x["gates"], 16, 3, forced=50)  # F >= Nb = 13
    assert c["sel"].shape[-1] == 13
    np.testing.assert_allclose(c["osel"], sdpa(x["q"], x["k"], x["v"], 1 / 8), atol=1e-12)


# ----------------------------------------------------------------------------- 2-D windows
def test_window_order_hand_enumerated():
    """2 views, 1 special token, 4x4 grid, 2x2 windows (17 tokens per view), written out by
    hand: view 0's grid starts at token 1, so window (0,0) holds rows 0-1, cols 0-1 =
    tokens 1,2,5,6; view 1 starts at 17 (its grid at 18); the specials 0 and 17 go last."""
    want = [1, 2, 5, 6, 3, 4, 7, 8, 9, 10, 13, 14, 11, 12, 15, 16,
            18, 19, 22, 23, 20, 21, 24, 25, 26, 27, 30, 31, 28, 29, 32, 33,
            0, 17]
    np.testing.assert_array_equal(O.window_order(2, 1, 4, 4, 2, 2), want)


@pytest.mark.parametrize("layout", [(3, 5, 8, 12, 4, 4), (2, 0, 16, 16, 8, 8), (1, 2, 6, 4, 3, 2),
                                    (4, 5, 8, 8, 4, 8)])
def test_window_order_is_a_bijection_of_spatial_windows(layout):
    """Every position is used once, and each run of win_h*win_w grid positions is exactly one
    win_h x win_w rectangle of one view's grid (catches swapped row/col strides, a window
    stepping across views, specials left inside the grid part)."""
    V, S, Gh, Gw, wh, ww = layout
    order = O.window_order(*layout)
    per = S + Gh * Gw
    assert sorted(order.tolist()) == list(range(V * per))
    grid = order[:V * Gh * Gw].reshape(-1, wh * ww)
    for blk in grid:
        view, r = blk // per, blk % per - S
        assert (view == view[0]).all() and (r >= 0).all()
        rows, cols = r // Gw, r % Gw
        assert rows.min() % wh == 0 and rows.max() - rows.min() == wh - 1
        assert cols.min() % ww == 0 and cols.max() - cols.min() == ww - 1
        assert len(set(zip(rows.tolist(), cols.tolist()))) == wh * ww
    specials = order[V * Gh * Gw:]
    assert specials.tolist() == [v * per + s for v in range(V) for s in range(S)]


def test_window_order_full_width_rows_is_identity_on_the_grid():
    """Windows one row high and one grid wide keep row-major order: only specials move."""
    order = O.window_order(3, 2, 4, 6, 1, 6)
    per = 2 + 24
    want = [v * per + 2 + i for v in range(3) for i in range(24)] + \
           [v * per + s for v in range(3) for s in range(2)]
    np.testing.assert_array_equal(order, want)


def test_window_blocks_pool_spatial_windows():
    """No special tokens, k and v constant on every 4x4 window of an 8x8 grid, B = 16: with
    window order every block is one constant window, so the compression branch equals dense
    softmax attention over all tokens (every block has the same size). With plain 1-D
    blocks each block mixes rows of two windows and the equality fails."""
    V, Gh, Gw, wh, ww, H, D = 2, 8, 8, 4, 4, 2, 64
    T = V * Gh * Gw
    nwin = V * (Gh // wh) * (Gw // ww)
    kw, vw = bf16_tensor((nwin, H, D), 41, 0.8), bf16_tensor((nwin, H, D), 42)
    t = np.arange(T)
    view, r = t // (Gh * Gw), t % (Gh * Gw)
    win = view * (Gh // wh) * (Gw // ww) + (r // Gw) // wh * (Gw // ww) + (r % Gw) // ww
    win = torch.from_numpy(win)
    k, v = kw[win].contiguous(), vw[win].contiguous()
    q = bf16_tensor((T, H, D), 43)
    gates = torch.ones(H, 2)
    dense = sdpa(q, k, v, 1 / 8)
    rw = O.forward_windows(q, k, v, gates, wh * ww, 2, (V, 0, Gh, Gw, wh, ww))
    np.testing.assert_allclose(rw["ocmp"], dense, atol=1e-12)
    r1 = O.forward_all(q, k, v, gates, wh * ww, 2)
    assert np.abs(r1["ocmp"] - dense).max() > 1e-3


def test_window_forward_is_the_plain_forward_on_reordered_tokens():
    """Identity layout (no specials, full-width rows) gives forward_all unchanged; with
    k = all blocks the selection branch is dense attention in any token order; per-token
    gates travel with their tokens."""
    w = W.WORKLOADS["tiny_s"]
    x = W.make_inputs(w)
    T = x["q"].shape[0]
    a = O.forward_windows(x["q"], x["k"], x["v"], x["gates"], 16, 4, (4, 0, 16, 16, 1, 16))
    b = O.forward_all(x["q"], x["k"], x["v"], x["gates"], 16, 4)
    for n in ("out", "ocmp", "osel", "lse", "sel"):
        np.testing.assert_array_equal(a[n], b[n])
    layout = (4, 0, 16, 16, 4, 4)
    c = O.forward_windows(x["q"], x["k"], x["v"], x["gates"], 16, 64, layout)
    np.testing.assert_allclose(c["osel"], sdpa(x["q"], x["k"], x["v"], 1 / 8), atol=1e-12)
    g = torch.rand(T, w.H, 2, generator=torch.Generator().manual_seed(5))
    d = O.forward_windows(x["q"], x["k"], x["v"], g, 16, 4, layout)
    gd = g.double().numpy()
    np.testing.assert_allclose(d["out"], gd[..., :1] * d["ocmp"] + gd[..., 1:] * d["osel"],
                               atol=1e-12)


# ----------------------------------------------------------------------------- backward
def _out_with_sel(q, k, v, g, B, sel):
    """out [T, H, D] of the forward pass with the selection held fixed (oracle forward)."""
    T, H, D = q.shape
    Nb = -(-T // B)
    r = O.forward_rows(q, k, v, g, B, sel.shape[-1], np.repeat(np.arange(H), Nb),
                       np.tile(np.arange(Nb), H), sel_in=sel.reshape(H * Nb, -1))
    return r["out"].reshape(H, Nb * B, D)[:, :T].transpose(1, 0, 2)


@pytest.mark.parametrize("token_gates", [False, True])
def test_backward_matches_finite_differences(token_gates):
    """Central differences of the oracle's own forward (selection fixed, since top-k is
    piecewise constant) against the backward, for every element of q, k, v and the gates.
    Small width D = 8 and a ragged last block; steps of 2^-12 on bf16-valued inputs are exact
    in float32. Catches any dropped term, sign or index slip of the chain rule."""
    T, H, D, B, kk = 22, 2, 8, 4, 2
    q, k, v = (bf16_tensor((T, H, D), 60 + i, 0.7).float().numpy() for i in range(3))
    gshape = (T, H, 2) if token_gates else (H, 2)
    g = torch.rand(gshape, generator=torch.Generator().manual_seed(64)).to(torch.bfloat16)
    g = g.float().numpy()
    W = bf16_tensor((T, H, D), 65).double().numpy()
    sel = O.forward_all(q, k, v, g, B, kk)["sel"]
    grads = O.backward(q, k, v, g, W, B, sel)
    step = 2.0 ** -12

    def loss(qq, kk_, vv, gg):
        return float((_out_with_sel(qq, kk_, vv, gg, B, sel) * W).sum())

    args = [q, k, v, g]
    for which, name in enumerate(("dq", "dk", "dv", "dgates")):
        x = args[which]
        fd = np.empty(x.shape)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + step
            up = loss(*args)
            x[idx] = old - step
            dn = loss(*args)
            x[idx] = old
            fd[idx] = (up - dn) / (2 * step)
        np.testing.assert_allclose(grads[name], fd, rtol=1e-5, atol=1e-6, err_msg=name)


def _sdpa_grads(q, k, v, dout, scale):
    """Dense attention gradients by torch autograd in float64 (a library routine)."""
    qh, kh, vh = (torch.from_numpy(np.ascontiguousarray(x)).double().permute(1, 0, 2)
                  .requires_grad_() for x in (q, k, v))
    o = F.scaled_dot_product_attention(qh[None], kh[None], vh[None], scale=scale)[0]
    o.backward(torch.from_numpy(np.ascontiguousarray(dout)).double().permute(1, 0, 2))
    return [t.grad.permute(1, 0, 2).numpy() for t in (qh, kh, vh)], o.detach().permute(1, 0, 2)


def test_backward_special_cases_are_dense_attention_backward():
    """B = 1 with gates (1, 0): the compression branch is dense attention over all tokens;
    k = all blocks with gates (0, 1): so is the selection branch. Both gradients must equal
    torch's float64 SDPA backward, and the gate gradients are dout . O_branch."""
    T, H, D = 40, 2, 64
    q, k, v = (bf16_tensor((T, H, D), 70 + i, 0.8).float().numpy() for i in range(3))
    dout = bf16_tensor((T, H, D), 73).float().numpy()
    (gq, gk, gv), o = _sdpa_grads(q, k, v, dout, 1 / 8)
    g10 = np.tile(np.array([[1.0, 0.0]], np.float32), (H, 1))
    sel = O.forward_all(q, k, v, g10, 1, 3)["sel"]
    r = O.backward(q, k, v, g10, dout, 1, sel)
    for name, ref in (("dq", gq), ("dk", gk), ("dv", gv)):
        np.testing.assert_allclose(r[name], ref, atol=1e-11, err_msg=f"B=1 {name}")
    np.testing.assert_allclose(r["dgates"][:, 0], (dout * o.numpy()).sum(axis=(0, 2)),
                               atol=1e-11)
    g01 = np.tile(np.array([[0.0, 1.0]], np.float32), (H, 1))
    B = 16
    sel = O.forward_all(q, k, v, g01, B, 10)["sel"]     # k = all 3 blocks
    r = O.backward(q, k, v, g01, dout, B, sel)
    for name, ref in (("dq", gq), ("dk", gk), ("dv", gv)):
        np.testing.assert_allclose(r[name], ref, atol=1e-11, err_msg=f"k=all {name}")
    np.testing.assert_allclose(r["dgates"][:, 1], (dout * o.numpy()).sum(axis=(0, 2)),
                               atol=1e-11)


def test_backward_invariants():
    """Shifting every key by one vector leaves every softmax unchanged, so sum_t dk_t = 0 per
    head; the attention weights sum to one, so sum_t dv_t = sum_t (g0 + g1) dout_t."""
    w = W.WORKLOADS["tiny_s"]
    x = W.make_inputs(w, T=300)
    dout = bf16_tensor((300, w.H, 64), 80)
    f = O.forward_all(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk)
    r = O.backward(x["q"], x["k"], x["v"], x["gates"], dout, w.block, f["sel"])
    np.testing.assert_allclose(r["dk"].sum(axis=0), 0.0, atol=1e-10)
    gsum = x["gates"].double().numpy().sum(axis=1)[None, :, None]
    np.testing.assert_allclose(r["dv"].sum(axis=0), (gsum * dout.double().numpy()).sum(axis=0),
                               atol=1e-10)
    # per-token gates: dgates[t, h] = (dout_t . O_cmp_t, dout_t . O_sel_t)
    gt = torch.rand(300, w.H, 2, generator=torch.Generator().manual_seed(81))
    rt = O.backward(x["q"], x["k"], x["v"], gt, dout, w.block, f["sel"])
    d = dout.double().numpy()
    np.testing.assert_allclose(rt["dgates"][..., 0], (d * f["ocmp"]).sum(-1), atol=1e-11)
    np.testing.assert_allclose(rt["dgates"][..., 1], (d * f["osel"]).sum(-1), atol=1e-11)


@pytest.mark.parametrize("forced", [0, 3])
def test_own_block_then_topk_of_the_rest(forced):
    """With own blocks, row i holds the forced prefix, block i, and the top-k of the other
    blocks by (score desc, index asc) from a brute-force lexsort, ascending; rows whose own
    block is forced hold one block fewer and end with -1."""
    w = W.WORKLOADS["tiny_s"]
    x = W.make_inputs(w, T=320)
    B, k = 16, 4
    r = O.forward_all(x["q"], x["k"], x["v"], x["gates"], B, k, forced=forced, own=True)
    Nb = 20
    assert r["sel"].shape[-1] == O.num_selected(320, B, k, forced, True) == forced + 1 + k
    for h in range(w.H):
        for i in range(Nb):
            sc = r["score"][h, i].astype(np.float64)
            fixed = set(range(forced)) | {i}
            cand = [j for j in range(Nb) if j not in fixed]
            order = sorted(cand, key=lambda j: (-sc[j], j))
            want = sorted(fixed | set(order[:k]))
            got = r["sel"][h, i]
            pad = len(got) - len(want)
            assert pad == (1 if i < forced else 0)
            np.testing.assert_array_equal(got[:len(want)], want)
            assert (got[len(want):] == -1).all()


def test_own_block_with_all_blocks_is_dense():
    """Own block plus k = Nb - 1: every block is selected, so the selection branch is dense
    attention (SDPA); every row contains its own block."""
    w = W.WORKLOADS["tiny_s"]
    x = W.make_inputs(w)
    r = O.forward_all(x["q"], x["k"], x["v"], x["gates"], 16, 63, own=True)
    np.testing.assert_allclose(r["osel"], sdpa(x["q"], x["k"], x["v"], 1 / 8), atol=1e-12)
    r4 = O.forward_all(x["q"], x["k"], x["v"], x["gates"], 16, 4, own=True)
    for i in range(64):
        assert (r4["sel"][:, i] == i).any(axis=-1).all()


# ------------------------------------------------------------- log-sum-exp bound (single pass)
def _group_constant_keys(T, H, B, group, seed):
    """Keys constant over every run of `group` consecutive blocks (one random vector each)."""
    n_groups = -(-T // (B * group))
    base = bf16_tensor((n_groups, H, 64), seed)
    return base[torch.arange(T) // (B * group)].contiguous()


def test_group_bound_equals_lse_when_groups_are_constant():
    """Every group of 8 blocks holds one key and Nb is a multiple of 8: Jensen is an equality,
    so the bound is the exact log-sum-exp (catches a wrong log(group) term, a mean over the
    wrong axis, or a missing scale)."""
    T, H, B = 64 * 8 * 3, 2, 64
    q = bf16_tensor((T, H, 64), 1)
    k = _group_constant_keys(T, H, B, 8, 2)
    v = bf16_tensor((T, H, 64), 3)
    lse = O.forward_all(q, k, v, torch.ones(H, 2), B, 4)["lse"]
    np.testing.assert_allclose(O.lse_group_bound(q, k, B), lse, rtol=0, atol=1e-12)


def test_group_bound_leaves_out_the_short_last_group():
    """All keys equal (logit c for every pooled key): the log-sum-exp is c + log Nb, the bound
    c + log(8 floor(Nb / 8)) (catches counting the partial group, or its keys, in the bound)."""
    T, H, B = 64 * 21 + 17, 1, 64   # Nb = 22: two full groups and 6 blocks left out
    q = bf16_tensor((T, H, 64), 4)
    kv = bf16_tensor((1, H, 64), 5)
    k = kv.expand(T, H, 64).contiguous()
    c = (q.double() * kv.double()).sum(-1)[:, 0].numpy() / 8.0
    np.testing.assert_allclose(O.lse_group_bound(q, k, B)[0], c + math.log(16), rtol=0,
                               atol=1e-12)
    lse = O.forward_all(q, k, k, torch.ones(H, 2), B, 4)["lse"][0]
    np.testing.assert_allclose(lse, c + math.log(22), rtol=0, atol=1e-12)


def test_group_bound_is_below_the_lse():
    """Jensen: on random keys the bound lies below the exact log-sum-exp for every query, and
    the gap closes as the keys within each group become alike (catches a sign slip, or a max
    in place of the mean, which would lift the bound above the log-sum-exp)."""
    w = W.WORKLOADS["tiny_s"]
    x = W.make_inputs(w, T=1536)  # 96 blocks: 12 full groups, none left out
    lse = O.forward_all(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk)["lse"]
    bnd = O.lse_group_bound(x["q"], x["k"], w.block)
    assert (bnd <= lse + 1e-12).all()
    assert (lse - bnd).max() > 1e-3
    # keys pulled toward their group's constant key: the gap shrinks with the spread
    T, H, B = 1536, x["q"].shape[1], w.block
    kc = _group_constant_keys(T, H, B, 8, 6).float()
    noise = bf16_tensor((T, H, 64), 7).float()
    for eps, most in ((1.0, None), (0.01, 0.01)):
        k = (kc + eps * noise).to(torch.bfloat16)
        gap = (O.forward_all(x["q"], k, x["v"], x["gates"], B, w.topk)["lse"] -
               O.lse_group_bound(x["q"], k, B))
        assert gap.min() >= -1e-12
        if most is not None:
            assert gap.max() < most
