"""speed3r_sparse_attn_fwd_noalloc (the forward pass on the library's fixed device array, for
callers that cannot allocate) against speed3r_sparse_attn_fwd with a caller workspace: the
same kernels on the same inputs, so the outputs and selections must be identical. Two calls in
a row, the second on a smaller problem (the array keeps the first call's contents), then one
with a problem too large for the array."""
import dataclasses

import pytest
import torch

from sparse_global_attention_block_amd import speed3r as S
from sparse_global_attention_block_amd import workloads as W
from tests.helpers import cuda_inputs

pytestmark = pytest.mark.gpu


def run_both(w, T):
    x = cuda_inputs(w, T=T)
    Tq, H, D = x["q"].shape
    p = S.make_params(x["q"], x["k"], x["v"], w.block, w.topk, 0.0, x["gates"], w.forced, w.own)
    assert S.workspace_size(p) <= S.noalloc_scratch_bytes()
    shape = (H, S.num_blocks(p), S.num_selected(p))
    ref_sel = torch.full(shape, -5, dtype=torch.int32, device="cuda")
    ref, _ = S.sparse_attn_fwd(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk,
                               sel_idx=ref_sel, forced_blocks=w.forced, force_own=w.own)
    out = torch.full_like(ref, 3.0)
    sel = torch.full(shape, -5, dtype=torch.int32, device="cuda")
    S.sparse_attn_fwd_noalloc(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk, out,
                              sel_idx=sel, forced_blocks=w.forced, force_own=w.own)
    torch.cuda.synchronize()
    print(f"[noalloc] T={Tq} H={H} B={w.block} k={w.topk} F={w.forced} own={w.own}: "
          f"workspace {S.workspace_size(p)} of {S.noalloc_scratch_bytes()} bytes", flush=True)
    assert torch.equal(out, ref), "output differs from the workspace entry point"
    assert torch.equal(sel, ref_sel), "selection differs from the workspace entry point"


def test_noalloc_matches_workspace_entry_point_twice():
    # 3 views of the 1374-token shape, 16 heads, forced reference blocks and own blocks; then a
    # smaller problem (1024 tokens, 4 heads) on the same array
    run_both(dataclasses.replace(W.WORKLOADS["v8"], name="v3_ref_own", forced=22, own=True),
             3 * 1374)
    run_both(W.WORKLOADS["tiny_s"], None)


def test_noalloc_rejects_problems_beyond_the_array():
    w = W.WORKLOADS["v100"]
    x = cuda_inputs(w)
    p = S.make_params(x["q"], x["k"], x["v"], w.block, w.topk, 0.0, x["gates"])
    assert S.workspace_size(p) > S.noalloc_scratch_bytes()
    out = torch.full_like(x["q"], 7.0)
    with pytest.raises(S.Speed3RError) as e:
        S.sparse_attn_fwd_noalloc(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk, out)
    assert e.value.status == S.S3R_ERR_SCRATCH
    torch.cuda.synchronize()
    assert (out == 7.0).all()
