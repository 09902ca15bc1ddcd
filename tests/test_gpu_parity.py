"""GPU parity: every stage of the HIP path against the float64 CPU oracle, element by element,
at sizes the oracle finishes in seconds (several tiles, ragged tails, all block sizes)."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_global_attention_block_amd import speed3r as S
from sparse_global_attention_block_amd import workloads as W
from tests import helpers as H
from tests.helpers import check_out, check_selection, cuda_inputs, host, own_rows

pytestmark = pytest.mark.gpu

_tiny_s = W.WORKLOADS["tiny_s"]
CASES = {
    "tiny": (W.WORKLOADS["tiny"], None),
    "tiny_all": (W.WORKLOADS["tiny_all"], None),
    "tiny_s": (_tiny_s, None),
    # 3 views of the 1374-token shape: Nb = 65 with a 26-token last block, 16 heads
    "v3_ragged": (W.WORKLOADS["v8"], 3 * 1374),
    "b32_ragged": (dataclasses.replace(_tiny_s, name="b32", H=2, block=32, topk=5), 1000),
    "b128": (dataclasses.replace(_tiny_s, name="b128", H=2, block=128, topk=3), 1100),
    "b16_many_tiles": (dataclasses.replace(_tiny_s, name="b16", H=1, block=16, topk=6), 3000),
    "shorter_than_block": (dataclasses.replace(W.WORKLOADS["v8"], name="short", H=2), 40),
    # forced leading blocks: the 16 blocks of the first view, 3 blocks, or every block
    "tiny_s_ref": (dataclasses.replace(_tiny_s, name="tiny_s_ref", forced=16), None),
    "tiny_forced3": (dataclasses.replace(W.WORKLOADS["tiny"], name="tiny_f3", forced=3), None),
    "v3_ref": (dataclasses.replace(W.WORKLOADS["v8"], name="v3_ref", forced=22), 3 * 1374),
    "b128_forced": (dataclasses.replace(_tiny_s, name="b128_f", H=2, block=128, topk=3,
                                        forced=2), 1100),
    "forced_all": (dataclasses.replace(_tiny_s, name="forced_all", H=2, block=32, topk=5,
                                       forced=100), 1000),
    # fp16 inputs and output (f16 matrix products, fp16 hi + lo pooled keys)
    "tiny_s_fp16": (dataclasses.replace(_tiny_s, name="tiny_s_fp16", dtype="fp16"), None),
    "v3_fp16": (dataclasses.replace(W.WORKLOADS["v8"], name="v3_fp16", dtype="fp16"), 3 * 1374),
    "b128_fp16": (dataclasses.replace(_tiny_s, name="b128_fp16", H=2, block=128, topk=3,
                                      dtype="fp16"), 1100),
    # each query block also keeps its own key block: alone, after a prefix (rows of the prefix
    # keep one entry less and end in -1), with B = 128, and with every block kept
    "tiny_s_own": (dataclasses.replace(_tiny_s, name="tiny_s_own", own=True), None),
    "v3_ref_own": (dataclasses.replace(W.WORKLOADS["v8"], name="v3_ref_own", forced=22,
                                       own=True), 3 * 1374),
    "tiny_f3_own": (dataclasses.replace(W.WORKLOADS["tiny"], name="tiny_f3_own", forced=3,
                                        own=True), None),
    "b128_own": (dataclasses.replace(_tiny_s, name="b128_own", H=2, block=128, topk=3,
                                     forced=1, own=True), 1100),
    "tiny_all_own": (dataclasses.replace(W.WORKLOADS["tiny_all"], name="tiny_all_own",
                                         forced=2, own=True), None),
    "forced_all_own": (dataclasses.replace(_tiny_s, name="forced_all_own", H=2, block=32,
                                           topk=5, forced=100, own=True), 1000),
    "v3_own_fp16": (dataclasses.replace(W.WORKLOADS["v8"], name="v3_own_fp16", own=True,
                                        dtype="fp16"), 3 * 1374),
    # two query blocks per wave in the running top-k (B = 32), with a prefix and own blocks
    "b32_forced_own": (dataclasses.replace(_tiny_s, name="b32_fo", H=2, block=32, topk=5,
                                           forced=3, own=True), 1000),
    # a sequence shorter than one tile of pooled keys: one query block, every block kept
    "one_block_own": (dataclasses.replace(_tiny_s, name="one_block_own", H=1, block=64, topk=4,
                                          own=True), 50),
    # a single token, and a second block of a single token
    "t1": (dataclasses.replace(_tiny_s, name="t1", H=2, block=16, topk=8), 1),
    "t17": (dataclasses.replace(_tiny_s, name="t17", H=2, block=16, topk=1), 17),
}

_cache = {}


def run_case(name):
    if name in _cache:
        return _cache[name]
    w, T = CASES[name]
    print(f"[case {name}] T={T or w.T} H={w.H} B={w.block} k={w.topk} F={w.forced} "
          f"own={w.own} {w.dtype}", flush=True)
    x = cuda_inputs(w, T=T)
    st = S.Stages(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk,
                  forced_blocks=w.forced, force_own=w.own).run_all()
    torch.cuda.synchronize()
    hx = {n: host(t) for n, t in x.items()}
    ora = O.forward_all(hx["q"], hx["k"], hx["v"], hx["gates"], w.block, w.topk,
                        forced=w.forced, own=w.own)
    ora["k_mean"] = O.pool(hx["k"], w.block)
    ora["v_mean"] = O.pool(hx["v"], w.block)
    _cache[name] = (w, x, hx, st, ora)
    return _cache[name]


@pytest.mark.parametrize("name", list(CASES))
def test_pool_means(name):
    w, x, hx, st, ora = run_case(name)
    for n in ("k_mean", "v_mean"):
        g = host(getattr(st, n)).double().numpy()
        np.testing.assert_allclose(g, ora[n], rtol=1e-6, atol=1e-6, err_msg=n)


def test_pool_identical_keys_bitwise():
    """Blocks of identical keys (including a short last block) pool to exactly that key."""
    T, H, B = 1000, 2, 64
    base = torch.randn(16, H, 64, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    k = base[torch.arange(T) // B].contiguous().cuda()
    st = S.Stages(k, k, k, torch.ones(H, 2, device="cuda"), B, 4)
    st.run_pool()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(st.k_mean).numpy(), base.float().permute(1, 0, 2).numpy())


@pytest.mark.parametrize("name", list(CASES))
def test_cmp_lse(name):
    w, x, hx, st, ora = run_case(name)
    g = host(st.lse).double().numpy()
    d = np.abs(g - ora["lse"])
    assert d.max() < 1e-4, f"max |dLSE| {d.max():.3e}"


@pytest.mark.parametrize("name", list(CASES))
def test_cmp_output_and_scores(name):
    w, x, hx, st, ora = run_case(name)
    oc = host(st.o_cmp).double().numpy()
    d = np.abs(oc - ora["ocmp"])
    assert d.max() < 1e-2 and d.mean() < 1e-3, f"O_cmp max {d.max():.3e} mean {d.mean():.3e}"
    sc = host(st.score).double().numpy()
    Nb = st.Nb
    assert (sc[:, :, Nb:] == 0).all(), "score padding columns must be zero"
    ds = np.abs(sc[:, :, :Nb] - ora["score"].astype(np.float64))
    tol = 2e-4 + 2e-4 * np.abs(ora["score"].astype(np.float64))
    assert (ds <= tol).all(), f"score max diff {ds.max():.3e}"


@pytest.mark.parametrize("name", list(CASES))
def test_score_error_within_the_derived_index_rule(name):
    """The derived index rules (tests/helpers.py) take 10x the GPU's measured score error as
    their gap threshold; this keeps that measurement true: relative error at most
    SCORE_REL_ERR for the input type, and at 3 views x 1374 tokens (B = 64) an absolute error
    of at most GAP_ABS / 10."""
    w, x, hx, st, ora = run_case(name)
    sc = host(st.score).double().numpy()[:, :, :st.Nb]
    osc = ora["score"].astype(np.float64)
    d = np.abs(sc - osc)
    rel = float((d / np.maximum(osc, 1e-30)).max())
    print(f"[{name}] score error: max-abs {d.max():.3e}, max relative {rel:.3e}")
    assert rel <= H.SCORE_REL_ERR[w.dtype], f"relative score error {rel:.3e}"
    if name == "v3_ragged":
        assert d.max() <= H.GAP_ABS / 10, f"absolute score error {d.max():.3e}"


@pytest.mark.parametrize("name", list(CASES))
def test_topk_bit_exact_on_gpu_scores(name):
    """Integer stage: on identical f32 score rows the GPU's choice must equal the oracle's
    (forced prefix, the own block, top-k of the remaining blocks, -1 padding) on every row."""
    w, x, hx, st, ora = run_case(name)
    sc = host(st.score).numpy()[:, :, :st.Nb]
    got = host(st.sel).numpy()
    F = st.forced
    for h in range(sc.shape[0]):
        for i in range(sc.shape[1]):
            keep = list(range(F))
            cand = np.arange(F, st.Nb)
            if st.own and i >= F:
                keep.append(i)
                cand = cand[cand != i]
            if len(cand):
                keep += list(cand[O.topk(sc[h, i, cand], w.topk)])
            want = np.full(st.k_eff, -1, np.int32)
            want[:len(keep)] = np.sort(keep)
            np.testing.assert_array_equal(got[h, i], want, err_msg=f"row h={h} i={i}")


@pytest.mark.parametrize("name", list(CASES))
def test_fused_topk_equals_separate_topk(name):
    """The running top-k inside the compression pass must choose exactly what the separate
    top-k chooses on the score matrix, and leave O_cmp bit-identical."""
    w, x, hx, st, ora = run_case(name)
    if not st.folds_topk:
        pytest.skip("B = 128 or k > 64 goes through the score matrix")
    ref_sel = st.sel.clone()
    ref_ocmp = st.o_cmp.clone()
    sel = torch.full_like(st.sel, -7)
    st.run_fused_topk(sel=sel)
    torch.cuda.synchronize()
    assert torch.equal(sel, ref_sel)
    assert torch.equal(st.o_cmp, ref_ocmp)


def test_topk_ties_and_fallback():
    """Heavy ties (all scores equal, few distinct levels) force the exact fallback path."""
    H, Nb, k = 2, 700, 16
    T = Nb * 64
    q = torch.zeros(T, H, 64, dtype=torch.bfloat16, device="cuda")
    p = S.make_params(q, q, q, 64, k)
    ld = S.score_row_stride(p)
    rng = np.random.default_rng(0)
    rows = np.zeros((H, Nb, ld), np.float32)
    rows[0, :, :Nb] = 0.25                                          # all tied
    rows[1, :, :Nb] = np.floor(rng.random((Nb, Nb)) * 3) / 3        # 3 levels
    rows[1, 5, :Nb] = rng.random(Nb)                                # no ties
    score = torch.from_numpy(rows).cuda()
    sel = torch.empty(H, Nb, k, dtype=torch.int32, device="cuda")
    S.topk(p, score, sel)
    torch.cuda.synchronize()
    got = host(sel).numpy()
    for h in range(H):
        for i in range(Nb):
            np.testing.assert_array_equal(got[h, i], O.topk(rows[h, i, :Nb], k))


@pytest.mark.parametrize("name", list(CASES))
def test_selection_indices(name):
    w, x, hx, st, ora = run_case(name)
    frac, diff = check_selection(host(st.sel).numpy(), ora["score"], ora["sel"], w.topk,
                                 forced=st.forced, qblocks=own_rows(w.H, st.Nb, st.own),
                                 dtype=w.dtype)
    print(f"[{name}] rows held to exact index parity: {frac:.1%}, near-tie rows differing: {len(diff)}")
    if name in ("tiny_s", "v3_ragged", "tiny_s_ref", "v3_ref", "tiny_s_own", "v3_ref_own"):
        assert frac > 0.5


@pytest.mark.parametrize("name", list(CASES))
def test_selection_branch_on_oracle_indices(name):
    """Feed the oracle's indices and O_cmp to the selection kernel: O_sel and the gated output
    must match the oracle's."""
    w, x, hx, st, ora = run_case(name)
    sel = torch.from_numpy(ora["sel"]).cuda()
    ocmp = torch.from_numpy(ora["ocmp"]).float().cuda()
    st.run_sel(sel=sel, o_cmp=ocmp)
    torch.cuda.synchronize()
    mx, mean = check_out(st.o_sel, ora["osel"], what="O_sel")
    print(f"[{name}] O_sel max-abs {mx:.3e} mean-abs {mean:.3e}")
    check_out(st.out, ora["out"])


@pytest.mark.parametrize("mode", ["two_pass", "single"])
@pytest.mark.parametrize("name", list(CASES))
def test_end_to_end(name, mode):
    """speed3r_sparse_attn_fwd with either compression mode against the oracle; rows where a
    near-tie flipped the chosen set are compared with the oracle run on the GPU's own
    indices."""
    w, x, hx, st, ora = run_case(name)
    if mode == "single" and not st.single_ok:
        pytest.skip("the single pass needs B <= 64, at most 64 chosen blocks and Nb >= 8")
    Nb = st.Nb
    k_eff = st.k_eff
    sel = torch.empty(w.H, Nb, k_eff, dtype=torch.int32, device="cuda")
    out, _ = S.sparse_attn_fwd(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk, sel_idx=sel,
                               forced_blocks=w.forced, force_own=w.own,
                               cmp_mode=S.CMP_SINGLE if mode == "single" else S.CMP_TWO_PASS)
    torch.cuda.synchronize()
    gsel = host(sel).numpy()
    ref = ora["out"]
    if not np.array_equal(gsel, ora["sel"]):
        rows_h = np.repeat(np.arange(w.H), Nb)
        rows_i = np.tile(np.arange(Nb), w.H)
        r = O.forward_rows(hx["q"], hx["k"], hx["v"], hx["gates"], w.block, w.topk, rows_h,
                           rows_i, sel_in=gsel.reshape(-1, k_eff), forced=w.forced, own=w.own)
        T = x["q"].shape[0]
        ref = np.ascontiguousarray(r["out"].reshape(w.H, Nb * w.block, 64)[:, :T]
                                   .transpose(1, 0, 2))
    mx, mean = check_out(out, ref)
    print(f"[{name}] {mode} out max-abs {mx:.3e} mean-abs {mean:.3e}")
    if mode == "two_pass":
        # the entry point runs the same kernels as the staged path: same indices
        np.testing.assert_array_equal(gsel, host(st.sel).numpy())
    else:
        check_selection(gsel, ora["score"], ora["sel"], w.topk, forced=st.forced,
                        qblocks=own_rows(w.H, Nb, st.own), dtype=w.dtype)


def test_deterministic_and_strided_inputs():
    """Two runs give identical bytes; q/k/v as strided views of one fused [T, 3, H, 64]
    tensor give the same bytes as contiguous copies; per-token gates are honoured."""
    w = W.WORKLOADS["tiny_s"]
    x = cuda_inputs(w)
    T, H, D = x["q"].shape
    a, sa = S.sparse_attn_fwd(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk,
                              sel_idx=torch.empty(H, T // w.block, w.topk, dtype=torch.int32,
                                                  device="cuda"))
    b, sb = S.sparse_attn_fwd(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk,
                              sel_idx=torch.empty_like(sa))
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(sa, sb)
    fused = torch.stack([x["q"], x["k"], x["v"]], dim=1)  # [T, 3, H, D]
    c, sc = S.sparse_attn_fwd(fused[:, 0], fused[:, 1], fused[:, 2], x["gates"], w.block,
                              w.topk, sel_idx=torch.empty_like(sa))
    torch.cuda.synchronize()
    assert torch.equal(a, c) and torch.equal(sa, sc)
    gt = x["gates"].expand(T, H, 2).contiguous()
    d, _ = S.sparse_attn_fwd(x["q"], x["k"], x["v"], gt, w.block, w.topk)
    torch.cuda.synchronize()
    assert torch.equal(a, d)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_dense_against_oracle(dtype):
    for name, T in (("tiny", None), ("v8", 3 * 1374 + 7)):
        w = dataclasses.replace(W.WORKLOADS[name], dtype=dtype)
        x = cuda_inputs(w, T=T)
        out = S.dense_attn_fwd(x["q"], x["k"], x["v"])
        torch.cuda.synchronize()
        hx = {n: host(t) for n, t in x.items()}
        T = x["q"].shape[0]
        for h in (0, w.H - 1):
            for t0, nt in ((0, 37), (T - 50, 50)):
                ref = O.dense_rows(hx["q"], hx["k"], hx["v"], h, t0, nt)
                # dense outputs here are dominated by the x3 special-token values (|x| of
                # 2-8, where bf16 rounding alone averages 4e-3-8e-3): the error beyond the
                # output's rounding is held to both bounds, the plain mean is not
                check_out(out[t0:t0 + nt, h], ref, what=f"dense {name} h={h} t0={t0}",
                          plain_mean=False)


def test_invalid_call_touches_nothing():
    """A rejected call launches nothing: the output keeps its sentinel."""
    w = W.WORKLOADS["tiny"]
    x = cuda_inputs(w)
    out = torch.full(x["q"].shape, 7.0, dtype=torch.bfloat16, device="cuda")
    ws = S.alloc_workspace(1024, "cuda")
    with pytest.raises(S.Speed3RError) as e:
        S.sparse_attn_fwd(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk, out=out,
                          workspace=ws)
    assert e.value.status == S.S3R_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (out == 7.0).all()
