"""GPU parity of the single compression pass (speed3r_cmp_lse_bound + speed3r_cmp_single_topk)
against the float64 oracle, and of its exact reruns.

The single pass must give what the two exact passes give: the log-sum-exp and O_cmp to the
same tolerances, and a selection that passes the same index-parity rule. Its failure paths
are driven from the host through the bound it is handed: a bound above the true log-sum-exp
fails every wave's Z check (so the exact passes rerun everywhere), a bound far below it makes
Z_t leave [1, 2^15] (the same), and one moderately below it leaves every check to pass on
large weights."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_global_attention_block_amd import speed3r as S
from sparse_global_attention_block_amd import workloads as W
from tests.helpers import check_out, check_selection, cuda_inputs, host, own_rows

pytestmark = pytest.mark.gpu

_tiny_s = W.WORKLOADS["tiny_s"]
_v8 = W.WORKLOADS["v8"]
CASES = {
    # B = 16: four query blocks per wave; Nb = 64, every candidate fits the list of 64
    "tiny_s": (_tiny_s, None),
    # B = 64, Nb = 65 with a 26-token last block: one candidate more than the list holds
    "v3_ragged": (_v8, 3 * 1374),
    # B = 32: two query blocks per wave, Nb = 94
    "b32_ragged": (dataclasses.replace(_tiny_s, name="b32", H=2, block=32, topk=5), 3000),
    # B = 16 over 188 blocks
    "b16_many": (dataclasses.replace(_tiny_s, name="b16", H=1, block=16, topk=6), 3000),
    # 300 blocks of 64 in 14 views: the list of 64 holds a fifth of the candidates
    "v14": (dataclasses.replace(_v8, name="v14", H=2), 14 * 1374),
    "v14_fp16": (dataclasses.replace(_v8, name="v14_fp16", H=2, dtype="fp16"), 14 * 1374),
    # a forced prefix and own blocks
    "v14_ref_own": (dataclasses.replace(_v8, name="v14_ref_own", H=2, forced=22, own=True),
                    14 * 1374),
    "b32_forced_own": (dataclasses.replace(_tiny_s, name="b32_fo", H=2, block=32, topk=5,
                                           forced=3, own=True), 3000),
    # k = 32 and k = 48 (the automatic mode's limit): the list of 64 holds only 2k and 4k/3,
    # so more query blocks fail the check, and work-groups rerun with some waves idle
    "v14_k32": (dataclasses.replace(_v8, name="v14_k32", H=2, topk=32), 14 * 1374),
    "v14_k48": (dataclasses.replace(_v8, name="v14_k48", H=2, topk=48), 14 * 1374),
    # large k with several query blocks per wave (each with its own smallest Z_t, and reruns
    # of waves that hold four or two query blocks)
    "b16_k40": (dataclasses.replace(_tiny_s, name="b16_k40", H=1, block=16, topk=40), 3000),
    "b32_k48": (dataclasses.replace(_tiny_s, name="b32_k48", H=2, block=32, topk=48), 3000),
    # exactly one group of 8 blocks
    "one_group": (dataclasses.replace(_tiny_s, name="one_group", H=2, block=64, topk=3), 8 * 64),
}

_cache = {}


def run_case(name):
    if name in _cache:
        return _cache[name]
    w, T = CASES[name]
    print(f"[single {name}] T={T or w.T} H={w.H} B={w.block} k={w.topk} F={w.forced} "
          f"own={w.own} {w.dtype}", flush=True)
    x = cuda_inputs(w, T=T)
    st = S.Stages(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk, keep_score=False,
                  forced_blocks=w.forced, force_own=w.own)
    assert st.single_ok
    st.run_pool()
    st.run_lse_bound()
    bound = st.lse_bound.clone()
    st.run_single_topk()
    torch.cuda.synchronize()
    hx = {n: host(t) for n, t in x.items()}
    ora = O.forward_all(hx["q"], hx["k"], hx["v"], hx["gates"], w.block, w.topk,
                        forced=w.forced, own=w.own)
    ora["bound"] = O.lse_group_bound(hx["q"], hx["k"], w.block)
    _cache[name] = (w, x, st, bound, ora)
    return _cache[name]


def check_cmp(name, st, ora, w):
    g = host(st.lse).double().numpy()
    d = np.abs(g - ora["lse"])
    assert d.max() < 1e-4, f"max |dLSE| {d.max():.3e}"
    oc = host(st.o_cmp).double().numpy()
    d = np.abs(oc - ora["ocmp"])
    assert d.max() < 1e-2 and d.mean() < 1e-3, f"O_cmp max {d.max():.3e} mean {d.mean():.3e}"
    frac, diff = check_selection(host(st.sel).numpy(), ora["score"], ora["sel"], w.topk,
                                 forced=st.forced, qblocks=own_rows(w.H, st.Nb, st.own),
                                 dtype=w.dtype)
    print(f"[{name}] rows held to exact index parity: {frac:.1%}, near-tie rows differing: "
          f"{len(diff)}", flush=True)


def valid_waves(st):
    """Redo flags of the waves that hold at least one query (the others never fail)."""
    T, H = st.q.shape[0], st.q.shape[1]
    n_wg = -(-T // 256)
    first = (np.arange(n_wg * 4) * 64)        # first query of each wave of one head
    return np.tile(first < T, H)


def bound_tolerance(hq, hk, w):
    """[H, T] limit on |GPU bound - oracle bound| (natural log). The bound pass multiplies the
    queries by the group keys' hi parts alone, the scaled keys rounded to the input type: each
    element x moves by at most u|x| (u = 2^-8 for bf16, 2^-11 for fp16, whose values below
    2^-14 move by at most 2^-25 instead), so the logit of group g by at most
    u * scale * sum_d |q_d G_gd| (+ 2^-25 ln2 sum_d |q_d| for fp16), and a log-sum-exp moves by
    at most the largest change of its terms. 1 % and 1e-5 more cover the f32 arithmetic."""
    q = np.abs(hq.double().numpy()).transpose(1, 0, 2)            # [H, T, D]
    kc = O.pool(hk, w.block)
    G = kc.shape[1] // 8
    means = np.abs(kc[:, :G * 8].reshape(kc.shape[0], G, 8, -1).mean(axis=2))  # [H, G, D]
    scale = q.shape[-1] ** -0.5
    u = 2.0 ** -11 if w.dtype == "fp16" else 2.0 ** -8
    tol = u * scale * np.matmul(q, means.transpose(0, 2, 1)).max(axis=-1)
    if w.dtype == "fp16":
        tol += 2.0 ** -25 * np.log(2.0) * q.sum(axis=-1)
    return 1.01 * tol + 1e-5


@pytest.mark.parametrize("name", list(CASES))
def test_lse_bound(name):
    """The bound pass against the oracle's group-mean bound, within what rounding the group
    keys to the input type allows, and (within the same) below the exact LSE."""
    w, x, st, bound, ora = run_case(name)
    g = host(bound).double().numpy()
    tol = bound_tolerance(host(x["q"]), host(x["k"]), w)
    d = np.abs(g - ora["bound"])
    print(f"[{name}] bound: max |d| {d.max():.2e}, max |d|/limit {(d / tol).max():.2f}", flush=True)
    assert (d <= tol).all(), f"max |d bound| {d.max():.3e}"
    assert (g <= ora["lse"] + tol).all()


@pytest.mark.parametrize("name", list(CASES))
def test_single_pass_against_oracle(name):
    w, x, st, bound, ora = run_case(name)
    check_cmp(name, st, ora, w)
    redo = host(st.redo).numpy()
    print(f"[{name}] waves redone: {int((redo != 0).sum())} of {int(valid_waves(st).sum())} "
          f"(log-sum-exp too: {int((redo & 2 != 0).sum())})", flush=True)
    assert set(np.unique(redo)) <= {0, 1, 2, 3}
    assert (redo[~valid_waves(st)] == 0).all()


@pytest.mark.parametrize("name", ["v14", "b32_forced_own", "tiny_s"])
def test_bound_above_lse_reruns_everything(name):
    """A 'bound' 0.5 above the true LSE makes Z < 1 for every query: every wave with queries
    fails its Z check (flag bit 1) and the exact passes recompute everything."""
    w, x, st, bound, ora = run_case(name)
    high = torch.from_numpy(ora["lse"] + 0.5).float().cuda()
    st.sel.fill_(-7)
    st.o_cmp.fill_(float("nan"))
    st.run_single_topk(lse_bound=high)
    torch.cuda.synchronize()
    redo = host(st.redo).numpy()
    v = valid_waves(st)
    assert ((redo[v] & 2) != 0).all() and (redo[~v] == 0).all()
    check_cmp(name, st, ora, w)


@pytest.mark.parametrize("name,drop", [("v14", 12.0), ("v3_ragged", 40.0), ("b16_many", 20.0),
                                       ("v14_fp16", 100.0)])
def test_far_low_bound_fails_the_z_check(name, drop):
    """A bound 12-100 below the LSE (Z_t = e^12..e^100, past 2^15, up to f32 overflow): the
    fp16 operands of P.V may overflow, the Z check fails everywhere, and the exact passes
    give the results."""
    w, x, st, bound, ora = run_case(name)
    low = torch.from_numpy(ora["lse"] - drop).float().cuda()
    st.run_single_topk(lse_bound=low)
    torch.cuda.synchronize()
    redo = host(st.redo).numpy()
    v = valid_waves(st)
    assert ((redo[v] & 2) != 0).all() and (redo[~v] == 0).all()
    check_cmp(name, st, ora, w)


@pytest.mark.parametrize("name", ["v14", "b16_many", "v14_fp16"])
def test_low_bound_within_range(name):
    """A bound 8 below the LSE (Z_t about e^8 = 2^11.5, inside [1, 2^15]): weights up to
    2^11.5 pass P.V in fp16, the Z check holds, and the results stay those of the exact
    method."""
    w, x, st, bound, ora = run_case(name)
    low = torch.from_numpy(ora["lse"] - 8.0).float().cuda()
    st.run_single_topk(lse_bound=low)
    torch.cuda.synchronize()
    redo = host(st.redo).numpy()
    assert ((redo & 2) == 0).all()
    check_cmp(name, st, ora, w)
    print(f"[{name}] waves redone: {int((redo != 0).sum())}", flush=True)


@pytest.mark.parametrize("name", ["v14", "v14_ref_own", "b32_ragged"])
def test_uneven_bound(name):
    """Each query's bound lowered by its own random amount in [0, 4): the upper bounds rank the
    blocks differently from the scores, which the check must catch or survive."""
    w, x, st, bound, ora = run_case(name)
    gen = torch.Generator(device="cuda").manual_seed(11)
    low = bound - 4.0 * torch.rand(bound.shape, device="cuda", generator=gen)
    st.run_single_topk(lse_bound=low)
    torch.cuda.synchronize()
    check_cmp(name, st, ora, w)
    print(f"[{name}] waves redone: {int((host(st.redo) != 0).sum())}", flush=True)


@pytest.mark.parametrize("name", ["v14", "v14_k32", "b32_ragged", "b32_k48"])
def test_rerun_with_proven_waves_in_the_work_group(name):
    """Work-groups where only some waves failed the selection check. The bound is lowered by
    6 for every other query of waves 0 and 2 of every work-group of 256 queries: the Z_t of
    each of their query blocks then spread over about e^6 (inside [1, 2^15]), which loosens
    its check, while waves 1 and 3 keep the exact bound. The scores-only rerun recomputes the flagged waves only and
    must leave the others' rows as the single pass wrote them; every row must match the
    oracle either way."""
    w, x, st, bound, ora = run_case(name)
    t = torch.arange(bound.shape[1], device="cuda")
    lowered = (((t // 64) % 2) == 0) & ((t % 2) == 0)
    st.run_single_topk(lse_bound=bound - 6.0 * lowered.float())
    torch.cuda.synchronize()
    check_cmp(name, st, ora, w)
    redo = host(st.redo).numpy().reshape(-1, 4)
    assert ((redo & 2) == 0).all(), "the Z check holds: Z_t stays inside [1, 2^15]"
    flagged = (redo & 1) != 0
    mixed = int((flagged.any(axis=1) & ~flagged.all(axis=1)).sum())
    print(f"[{name}] waves redone: {int(flagged.sum())} (waves 0 and 2: "
          f"{int(flagged[:, ::2].sum())}); work-groups with proven waves beside flagged "
          f"ones: {mixed}", flush=True)
    assert mixed > 0


@pytest.mark.parametrize("name", ["v14", "v14_ref_own", "b32_forced_own", "v14_fp16"])
def test_forward_single_vs_two_pass(name):
    """The whole forward pass in either mode against the oracle's output and selection."""
    w, x, st, bound, ora = run_case(name)
    hx_out = ora["out"]
    for mode in (S.CMP_SINGLE, S.CMP_TWO_PASS):
        sel = torch.empty(w.H, st.Nb, st.k_eff, dtype=torch.int32, device="cuda")
        out, _ = S.sparse_attn_fwd(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk,
                                   sel_idx=sel, forced_blocks=w.forced, force_own=w.own,
                                   cmp_mode=mode)
        torch.cuda.synchronize()
        check_selection(host(sel).numpy(), ora["score"], ora["sel"], w.topk, forced=st.forced,
                        qblocks=own_rows(w.H, st.Nb, st.own), dtype=w.dtype)
        check_out(out, hx_out, what=f"out mode {mode}")


def test_tight_bound_lifted_by_rounding():
    """Keys constant over each group of 8 blocks make the group-mean bound exact (Jensen's
    inequality is then an equality), so rounding the scaled group keys to bf16 in the bound
    pass can lift the GPU's bound above the true log-sum-exp. The Z check must flag those
    waves, and the exact reruns must give the oracle's results."""
    T, H, B, k = 1024, 2, 16, 8
    gen = torch.Generator().manual_seed(31)
    q = torch.randn(T, H, 64, generator=gen).to(torch.bfloat16)
    groups = torch.randn(T // (8 * B), H, 64, generator=gen) * 2.0
    kk = groups.repeat_interleave(8 * B, dim=0).to(torch.bfloat16)
    v = torch.randn(T, H, 64, generator=gen).to(torch.bfloat16)
    gates = torch.rand(H, 2, generator=gen)
    print(f"[single tight] T={T} H={H} B={B} k={k}", flush=True)
    x = {"q": q.cuda(), "k": kk.cuda(), "v": v.cuda(), "gates": gates.cuda()}
    st = S.Stages(x["q"], x["k"], x["v"], x["gates"], B, k, keep_score=False)
    assert st.single_ok
    st.run_pool()
    st.run_lse_bound()
    bound = host(st.lse_bound).double().numpy()
    st.run_single_topk()
    torch.cuda.synchronize()
    ora = O.forward_all(q, kk, v, gates, B, k)
    exact_bound = O.lse_group_bound(q, kk, B)
    assert np.abs(exact_bound - ora["lse"]).max() < 1e-9  # the bound is exact here
    above = int((bound > ora["lse"]).sum())
    redo = host(st.redo).numpy()
    print(f"[single tight] queries whose GPU bound exceeds the LSE: {above} of {bound.size}; "
          f"waves flagged by the Z check: {int(((redo & 2) != 0).sum())}", flush=True)
    w = dataclasses.replace(_tiny_s, name="tight", H=H, block=B, topk=k)
    check_cmp("tight", st, ora, w)
