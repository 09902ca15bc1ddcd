"""GPU parity of the backward pass (speed3r_sparse_attn_fwd_train + speed3r_sparse_attn_bwd)
against the float64 oracle's backward, element by element, and its invariants at full size.

The backward holds the forward's selection fixed. The GPU selection is first checked against
the oracle's own (exact on rows with a clear top-k gap, within the gap elsewhere); the oracle
backward then runs on that validated selection, which is one of the valid ones."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_global_attention_block_amd import speed3r as S
from sparse_global_attention_block_amd import workloads as W
from tests.helpers import check_selection, cuda_inputs, host, own_rows

pytestmark = pytest.mark.gpu

# gradient tolerances, relative to the reference tensor's own scale (bf16 operands in the
# products feeding dq, dk, dv: 2^-9 relative rounding per term)
GRAD_MAX_REL = 2e-2   # max |gpu - ref| / max |ref|
GRAD_MEAN_REL = 4e-3  # mean |gpu - ref| / mean |ref|

_tiny_s = W.WORKLOADS["tiny_s"]
CASES = {
    "tiny_s": (_tiny_s, None, {}),
    "tiny_all": (W.WORKLOADS["tiny_all"], None, {}),
    "b32_ragged": (dataclasses.replace(_tiny_s, name="b32", H=2, block=32, topk=5), 1000, {}),
    "b128": (dataclasses.replace(_tiny_s, name="b128", H=2, block=128, topk=3), 1100, {}),
    "v3_ragged": (W.WORKLOADS["v8"], 3 * 1374, {}),
    "tiny_s_ref": (dataclasses.replace(_tiny_s, name="tiny_s_ref", forced=16), None, {}),
    "token_gates": (_tiny_s, 700, {"token_gates": True}),
    "strided_dout": (dataclasses.replace(_tiny_s, name="b64", H=2, block=64, topk=4), 900,
                     {"strided": True}),
    # fp16 inputs and output gradient
    "tiny_s_fp16": (dataclasses.replace(_tiny_s, name="tiny_s_fp16", dtype="fp16"), None, {}),
    "v3_fp16": (dataclasses.replace(W.WORKLOADS["v8"], name="v3_fp16", dtype="fp16"), 3 * 1374,
                {}),
    "b128_fp16": (dataclasses.replace(_tiny_s, name="b128_fp16", H=2, block=128, topk=3,
                                      dtype="fp16"), 1100, {}),
    # own blocks after a prefix: rows of the prefix end in -1
    "v3_ref_own": (dataclasses.replace(W.WORKLOADS["v8"], name="v3_ref_own", forced=22,
                                       own=True), 3 * 1374, {}),
    "tiny_f3_own": (dataclasses.replace(W.WORKLOADS["tiny"], name="tiny_f3_own", forced=3,
                                        own=True), None, {}),
    # the first 2 key blocks are chosen by every one of more than 1024 query blocks, so the
    # dk/dv kernel lists their selecting blocks in several chunks
    "b16_chunked": (dataclasses.replace(_tiny_s, name="b16_chunked", H=1, block=16, topk=2,
                                        forced=2), 1100 * 16 + 5, {}),
    "b64_chunked": (dataclasses.replace(_tiny_s, name="b64_chunked", H=1, block=64, topk=2,
                                        forced=2), 1030 * 64 + 17, {}),
    # a second block of a single token, and a single token
    "t17": (dataclasses.replace(_tiny_s, name="t17", H=2, block=16, topk=1), 17, {}),
    # one token: both softmaxes have a single key, so dq and dk vanish in exact arithmetic
    "t1": (dataclasses.replace(_tiny_s, name="t1", H=2, block=16, topk=8), 1,
           {"vanishing_dqdk": True}),
}


def compare(name, what, gpu, ref):
    g = host(gpu).double().numpy()
    d = np.abs(g - ref)
    mx = d.max() / max(np.abs(ref).max(), 1e-30)
    mean = d.mean() / max(np.abs(ref).mean(), 1e-30)
    print(f"[{name}] {what}: max-rel {mx:.2e} mean-rel {mean:.2e}", flush=True)
    assert np.isfinite(g).all(), f"{what}: non-finite values"
    assert mx <= GRAD_MAX_REL and mean <= GRAD_MEAN_REL, f"{what}: max-rel {mx:.2e} mean-rel {mean:.2e}"


def check_dgates(name, gpu, ref, dout, ora_f):
    """dgates is a sum over tokens of dout . O_branch (per head) or one such dot (per token):
    its error is the forward's O error carried through the sum, so it is bounded relative to
    the size of the summands, sum |dout_td O_td| (2e-3: the mean-abs bound on O)."""
    d = dout.double().numpy()
    mag = np.stack([np.abs(d * ora_f["ocmp"]).sum(-1), np.abs(d * ora_f["osel"]).sum(-1)], -1)
    if ref.ndim == 2:
        mag = mag.sum(0)
    err = np.abs(host(gpu).double().numpy() - ref)
    print(f"[{name}] dgates: max err/magnitude {(err / mag).max():.2e}", flush=True)
    assert (err <= 2e-3 * mag + 1e-6).all(), "dgates"


def run_case(name):
    w, T, opt = CASES[name]
    print(f"[bwd {name}] T={T or w.T} H={w.H} B={w.block} k={w.topk} F={w.forced} own={w.own} "
          f"{w.dtype} {opt}", flush=True)
    x = cuda_inputs(w, T=T)
    T = x["q"].shape[0]
    gates = x["gates"]
    if opt.get("token_gates"):
        gates = torch.rand(T, w.H, 2, device="cuda",
                           generator=torch.Generator(device="cuda").manual_seed(5))
    gen = torch.Generator(device="cuda").manual_seed(17)
    dout = torch.randn(T, w.H, 64, device="cuda", generator=gen).to(x["q"].dtype)
    if opt.get("strided"):
        big = torch.zeros(T, w.H, 2, 64, dtype=dout.dtype, device="cuda")
        big[:, :, 1] = dout
        dout = big[:, :, 1]
    st = S.sparse_attn_fwd_train(x["q"], x["k"], x["v"], gates, w.block, w.topk,
                                 forced_blocks=w.forced, force_own=w.own)
    dq, dk, dv, dg = S.sparse_attn_bwd(st, dout)
    torch.cuda.synchronize()
    hx = {n: host(t) for n, t in x.items()}
    hg = host(gates)
    ora_f = O.forward_all(hx["q"], hx["k"], hx["v"], hg, w.block, w.topk, forced=w.forced,
                          own=w.own)
    gsel = host(st.sel).numpy()
    Nb = gsel.shape[1]
    F = min(w.forced, Nb)
    check_selection(gsel, ora_f["score"], ora_f["sel"], w.topk, forced=F,
                    qblocks=own_rows(w.H, Nb, w.own and F < Nb), dtype=w.dtype)
    ref = O.backward(hx["q"], hx["k"], hx["v"], hg, host(dout), w.block, gsel)
    ref["forward"] = ora_f
    ref["dout"] = host(dout)
    return (dq, dk, dv, dg), ref, st, dout


@pytest.mark.parametrize("name", list(CASES))
def test_backward_against_oracle(name):
    (dq, dk, dv, dg), ref, _, _ = run_case(name)
    if CASES[name][2].get("vanishing_dqdk"):
        # a relative bound means nothing against an exact zero: the GPU's dq, dk are the
        # rounding of cancelling terms (dP with bf16 operands against the f32 D), held to
        # 1 % of the gradient scale that dv shows
        assert np.abs(ref["dq"]).max() < 1e-9 and np.abs(ref["dk"]).max() < 1e-9
        scale = np.abs(ref["dv"]).max()
        for what, t in (("dq", dq), ("dk", dk)):
            a = np.abs(host(t).double().numpy()).max()
            print(f"[{name}] {what}: max |gpu| {a:.2e} vs dv scale {scale:.2e}", flush=True)
            assert a <= 1e-2 * scale, what
    else:
        compare(name, "dq", dq, ref["dq"])
        compare(name, "dk", dk, ref["dk"])
    compare(name, "dv", dv, ref["dv"])
    check_dgates(name, dg, ref["dgates"], ref["dout"], ref["forward"])


def test_backward_deterministic():
    """Two backward passes of one forward give identical bytes."""
    (dq, dk, dv, dg), _, st, dout = run_case("v3_ragged")
    dq2, dk2, dv2, dg2 = S.sparse_attn_bwd(st, dout)
    torch.cuda.synchronize()
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2), (dg, dg2)):
        assert torch.equal(a, b)


def test_backward_invariants_at_1000_views():
    """At 1000 views (the oracle's full backward would take hours) check what holds at any
    size: shifting all keys leaves every softmax unchanged, so sum_t dk_t = 0 per head; the
    weights sum to one, so sum_t dv_t = sum_t (g0 + g1) dout_t; and dgates = dout . O."""
    w = W.WORKLOADS["v1000_k16"]
    print(f"[bwd full] T={w.T} H={w.H}", flush=True)
    x = cuda_inputs(w)
    dout = torch.randn(w.T, w.H, 64, device="cuda",
                       generator=torch.Generator(device="cuda").manual_seed(23)).to(torch.bfloat16)
    st = S.sparse_attn_fwd_train(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk)
    dq, dk, dv, dg = S.sparse_attn_bwd(st, dout)
    torch.cuda.synchronize()
    assert all(torch.isfinite(t).all() for t in (dq, dk, dv, dg))
    sk = dk.double().sum(0)
    assert (sk.abs() <= 1e-3 * dk.double().abs().sum(0) + 1e-6).all(), "sum of dk"
    gs = x["gates"].double().sum(1)[None, :, None]
    want = (gs * dout.double()).sum(0)
    assert (dv.double().sum(0) - want).abs().max() <= 1e-3 * (gs * dout.double()).abs().sum(0).max()
    del dq, dk, dv, st
    torch.cuda.empty_cache()
