"""C-ABI checks that need no GPU: the library loads, exports every entry point the header
declares, and rejects bad arguments before touching the device (every call here returns from
validation, so nothing is launched)."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import oracle as O
from sparse_global_attention_block_amd import speed3r as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "speed3r.h")

FAKE = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: validation fails first


def declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"\b(speed3r_\w+)\s*\(", txt)))


def test_header_symbols_are_exported():
    L = S.lib()
    names = declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), f"{n} declared in speed3r.h but not exported"
    assert set(names) == set(S.EXPORTS), "binding and header disagree"


def test_status_strings():
    for code, name in enumerate(["S3R_OK", "S3R_ERR_INVALID_ARG", "S3R_ERR_UNSUPPORTED",
                                 "S3R_ERR_WORKSPACE", "S3R_ERR_HIP", "S3R_ERR_SCRATCH"]):
        assert S.status_string(code) == name
    assert S.status_string(99) == "S3R_ERR_UNKNOWN"


def params(T=1024, H=4, D=64, B=16, k=8, scale=0.0, st=None, forced=0, dtype=0, own=0,
           mode=0):
    st = st or (H * D, D)
    return S.Params(T, H, D, B, k, scale, forced, st[0], st[1], st[0], st[1], st[0], st[1], 0,
                    dtype, own, mode)


def test_size_queries():
    p = params()
    assert S.num_blocks(p) == 64
    assert S.score_row_stride(p) == 64
    p2 = params(T=1000)
    assert S.num_blocks(p2) == 63 and S.score_row_stride(p2) == 64
    sizes = [S.workspace_size(params(T=t)) for t in (16, 1000, 5000, 20000)]
    assert all(a < b for a, b in zip(sizes, sizes[1:])), "workspace must grow with T"
    assert S.tiles_workspace_size(p) < S.workspace_size(p)
    assert S.dense_workspace_size(p) > 0
    # 1000 views x 1374 tokens, 16 heads, B = 64, k = 16: about 11.7 GB
    big = params(T=1_374_000, H=16, B=64, k=16)
    assert 10e9 < S.workspace_size(big) < 13e9
    big128 = params(T=1_374_000, H=16, B=128, k=16)
    assert S.workspace_size(big128) > 14e9  # B = 128 keeps the score matrix
    assert S.num_blocks(big) == 21469


@pytest.mark.parametrize("kw,code", [
    (dict(D=32), S.S3R_ERR_UNSUPPORTED),
    (dict(B=48), S.S3R_ERR_UNSUPPORTED),
    (dict(B=0), S.S3R_ERR_INVALID_ARG),
    (dict(k=0), S.S3R_ERR_INVALID_ARG),
    (dict(T=0), S.S3R_ERR_INVALID_ARG),
    (dict(H=0), S.S3R_ERR_INVALID_ARG),
    (dict(scale=-1.0), S.S3R_ERR_INVALID_ARG),
    (dict(scale=float("nan")), S.S3R_ERR_INVALID_ARG),
    (dict(st=(4 * 64 + 4, 64)), S.S3R_ERR_INVALID_ARG),   # token stride not a multiple of 8
    (dict(st=(-256, 64)), S.S3R_ERR_INVALID_ARG),
    (dict(T=24577 * 16, B=16, k=65), S.S3R_ERR_UNSUPPORTED),  # > 24576 blocks, not folded
    (dict(forced=-1), S.S3R_ERR_INVALID_ARG),
    (dict(dtype=2), S.S3R_ERR_INVALID_ARG),
    (dict(mode=3), S.S3R_ERR_INVALID_ARG),
    (dict(mode=-1), S.S3R_ERR_INVALID_ARG),
])
def test_bad_params_rejected_everywhere(kw, code):
    p = params(**kw)
    L = S.lib()
    ws = ctypes.c_void_p(1 << 20)
    big = ctypes.c_size_t(1 << 40)
    calls = [
        L.speed3r_sparse_attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, ws, big,
                                  None),
        L.speed3r_pool(ctypes.byref(p), FAKE, FAKE, ws, big, None, None, None),
        L.speed3r_cmp_lse(ctypes.byref(p), FAKE, ws, big, FAKE, None),
        L.speed3r_cmp_fused(ctypes.byref(p), FAKE, ws, big, FAKE, FAKE, FAKE, None),
        L.speed3r_cmp_fused_topk(ctypes.byref(p), FAKE, ws, big, FAKE, FAKE, FAKE, None),
        L.speed3r_cmp_lse_bound(ctypes.byref(p), FAKE, ws, big, FAKE, None),
        L.speed3r_cmp_single_topk(ctypes.byref(p), FAKE, ws, big, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  None),
        L.speed3r_topk(ctypes.byref(p), FAKE, FAKE, None),
        L.speed3r_sel_combine(ctypes.byref(p), FAKE, ws, big, FAKE, FAKE, FAKE, FAKE, None, None),
        L.speed3r_dense_attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, ws, big, None),
    ]
    assert calls == [code] * len(calls)
    assert S.workspace_size(p) == 0 and S.num_blocks(p) == -1 and S.num_selected(p) == -1
    assert S.redo_flag_count(p) == -1


@pytest.mark.parametrize("T,B,k,F,n_sel", [
    (1024, 16, 8, 0, 8), (1024, 16, 8, 3, 11), (1024, 16, 100, 0, 64), (1024, 16, 60, 10, 64),
    (1024, 16, 8, 64, 64), (1024, 16, 8, 1000, 64), (40, 16, 8, 1, 3), (1, 64, 16, 2, 1),
])
def test_num_selected_counts_forced_prefix(T, B, k, F, n_sel):
    """Rows hold F' = min(F, Nb) forced blocks and min(k, Nb - F') chosen ones."""
    assert S.num_selected(params(T=T, B=B, k=k, forced=F)) == n_sel


@pytest.mark.parametrize("T,B,k,F,n_sel", [
    (1024, 16, 8, 0, 9), (1024, 16, 8, 3, 12), (1024, 16, 100, 0, 64), (1024, 16, 8, 64, 64),
    (40, 16, 8, 1, 3), (1, 64, 16, 0, 1),
])
def test_num_selected_with_own_block(T, B, k, F, n_sel):
    """With own blocks a row holds F' + 1 + min(k, Nb - F' - 1) entries (F' < Nb)."""
    assert S.num_selected(params(T=T, B=B, k=k, forced=F, own=1)) == n_sel


def test_null_and_misaligned_pointers():
    p = params()
    L = S.lib()
    ws, big = ctypes.c_void_p(1 << 20), ctypes.c_size_t(1 << 40)
    odd = ctypes.c_void_p((1 << 20) + 2)
    assert L.speed3r_sparse_attn_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, ws, big, None) \
        == S.S3R_ERR_INVALID_ARG
    assert L.speed3r_sparse_attn_fwd(ctypes.byref(p), None, FAKE, FAKE, FAKE, FAKE, None, ws,
                                     big, None) == S.S3R_ERR_INVALID_ARG
    assert L.speed3r_sparse_attn_fwd(ctypes.byref(p), odd, FAKE, FAKE, FAKE, FAKE, None, ws, big,
                                     None) == S.S3R_ERR_INVALID_ARG
    assert L.speed3r_sparse_attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, None, FAKE, None, ws,
                                     big, None) == S.S3R_ERR_INVALID_ARG
    assert L.speed3r_topk(ctypes.byref(p), None, FAKE, None) == S.S3R_ERR_INVALID_ARG
    assert L.speed3r_cmp_lse(ctypes.byref(p), FAKE, ws, big, None, None) == S.S3R_ERR_INVALID_ARG


def test_workspace_too_small_or_missing():
    p = params()
    L = S.lib()
    need = S.workspace_size(p)
    ws = ctypes.c_void_p(1 << 20)
    for w, n in ((ws, need - 1), (None, need), (ctypes.c_void_p((1 << 20) + 128), need)):
        assert L.speed3r_sparse_attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, w,
                                         n, None) == S.S3R_ERR_WORKSPACE
    tiles = S.tiles_workspace_size(p)
    assert L.speed3r_pool(ctypes.byref(p), FAKE, FAKE, ws, tiles - 1, None, None, None) \
        == S.S3R_ERR_WORKSPACE
    assert L.speed3r_dense_attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, ws,
                                    S.dense_workspace_size(p) - 1, None) == S.S3R_ERR_WORKSPACE


def test_block_limit_only_without_folded_selection():
    """More than 24576 blocks: fine when the selection folds into the compression pass (no
    score row to hold), rejected by the separate top-k kernel."""
    p = params(T=25079 * 64, H=16, B=64, k=16)
    assert S.num_blocks(p) == 25079 and S.workspace_size(p) > 0
    assert S.lib().speed3r_topk(ctypes.byref(p), FAKE, FAKE, None) == S.S3R_ERR_UNSUPPORTED
    assert S.workspace_size(params(T=25079 * 64, H=16, B=128, k=16)) > 0  # 12540 blocks
    assert S.workspace_size(params(T=25079 * 128, H=16, B=128, k=16)) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(S, "_lib", None)
    monkeypatch.setattr(S, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        S.lib()


def test_fused_topk_limits():
    """The selection folds into the compression pass only for B <= 64 and k <= 64."""
    L = S.lib()
    ws, big = ctypes.c_void_p(1 << 20), ctypes.c_size_t(1 << 40)
    for kw in (dict(B=128, T=4096), dict(k=65, T=100 * 64, B=64),
               dict(k=65, T=100 * 64, B=64, forced=20)):
        p = params(**kw)
        assert L.speed3r_cmp_fused_topk(ctypes.byref(p), FAKE, ws, big, FAKE, FAKE, FAKE,
                                        None) == S.S3R_ERR_UNSUPPORTED
    # the limit is on the chosen blocks: 60 forced + 40 chosen of the remaining 40 folds in
    p = params(k=65, T=100 * 64, B=64, forced=60)
    assert S.num_selected(p) == 100
    assert S.workspace_size(p) < S.workspace_size(params(k=65, T=100 * 64, B=64))


@pytest.mark.parametrize("layout", [(2, 1, 4, 4, 2, 2), (3, 5, 8, 12, 4, 4), (2, 0, 16, 16, 8, 8),
                                    (4, 5, 40, 40, 8, 8)])
def test_window_source_matches_oracle_order(layout):
    """Host index function of the library against the oracle's own window order."""
    order = O.window_order(*layout)
    got = [S.window_source(layout, p) for p in range(order.size)]
    np.testing.assert_array_equal(got, order)
    assert S.window_source(layout, -1) == -1 and S.window_source(layout, order.size) == -1


@pytest.mark.parametrize("layout", [(0, 5, 8, 8, 4, 4), (2, -1, 8, 8, 4, 4), (2, 5, 8, 8, 3, 4),
                                    (2, 5, 8, 10, 4, 4), (2, 5, 8, 8, 0, 4)])
def test_bad_window_layouts_rejected(layout):
    L = S.lib()
    w = S.make_windows(layout)
    assert S.window_source(layout, 0) == -1
    p = params(T=2 * (5 + 64), H=4, B=16, k=4)
    assert S.windows_workspace_size(p, layout) == 0
    assert L.speed3r_window_permute(ctypes.byref(w), 4, FAKE, 256, 64, FAKE, 256, 64, 0,
                                    None) == S.S3R_ERR_INVALID_ARG
    ws, big = ctypes.c_void_p(1 << 20), ctypes.c_size_t(1 << 40)
    assert L.speed3r_sparse_attn_fwd_windows(ctypes.byref(p), ctypes.byref(w), FAKE, FAKE, FAKE,
                                             FAKE, FAKE, None, ws, big, None) \
        == S.S3R_ERR_INVALID_ARG


def test_window_forward_checks():
    """Token count must match the layout; per-token gates need an even stride; the workspace
    adds the reordered copies to the plain forward's."""
    L = S.lib()
    layout = (2, 5, 8, 8, 4, 4)
    w = S.make_windows(layout)
    ws, big = ctypes.c_void_p(1 << 20), ctypes.c_size_t(1 << 40)
    p = params(T=2 * 69, H=4, B=16, k=4)
    need = S.windows_workspace_size(p, layout)
    assert need > S.workspace_size(p) + 4 * 138 * 4 * 64 * 2 - 1
    bad_T = params(T=2 * 69 + 1, H=4, B=16, k=4)
    assert S.windows_workspace_size(bad_T, layout) == 0
    assert L.speed3r_sparse_attn_fwd_windows(ctypes.byref(bad_T), ctypes.byref(w), FAKE, FAKE,
                                             FAKE, FAKE, FAKE, None, ws, big, None) \
        == S.S3R_ERR_INVALID_ARG
    odd = params(T=2 * 69, H=4, B=16, k=4)
    odd.gate_stride_t = 9
    assert L.speed3r_sparse_attn_fwd_windows(ctypes.byref(odd), ctypes.byref(w), FAKE, FAKE,
                                             FAKE, FAKE, FAKE, None, ws, big, None) \
        == S.S3R_ERR_INVALID_ARG
    assert L.speed3r_sparse_attn_fwd_windows(ctypes.byref(p), ctypes.byref(w), FAKE, FAKE, FAKE,
                                             FAKE, FAKE, None, ws, ctypes.c_size_t(need - 1),
                                             None) == S.S3R_ERR_WORKSPACE


def test_params_layout_matches_header():
    """The ctypes mirror of s3r_params has the C layout: 104 bytes (int64 alignment), dtype
    at offset 88, cmp_mode at 96."""
    assert ctypes.sizeof(S.Params) == 104
    assert S.Params.dtype.offset == 88 and S.Params.gate_stride_t.offset == 80
    assert S.Params.force_own.offset == 92 and S.Params.cmp_mode.offset == 96


def test_single_pass_limits():
    """The single compression pass needs the folded selection (B <= 64, k_eff - F' <= 64) and
    at least one group of 8 blocks; the forward pass refuses CMP_SINGLE elsewhere and the
    automatic mode then takes the two passes."""
    L = S.lib()
    ws, big = ctypes.c_void_p(1 << 20), ctypes.c_size_t(1 << 40)
    single = lambda p, redo=FAKE: L.speed3r_cmp_single_topk(  # noqa: E731
        ctypes.byref(p), FAKE, ws, big, FAKE, FAKE, FAKE, FAKE, redo, None)
    fwd = lambda p: L.speed3r_sparse_attn_fwd(  # noqa: E731
        ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, ws, big, None)
    for kw in (dict(B=128, T=4096), dict(k=65, T=100 * 64, B=64), dict(T=7 * 16, B=16)):
        assert single(params(**kw)) == S.S3R_ERR_UNSUPPORTED
        assert fwd(params(mode=S.CMP_SINGLE, **kw)) == S.S3R_ERR_UNSUPPORTED
        # automatic and two-pass modes take the two passes: no redo flags in the workspace
        assert S.workspace_size(params(**kw)) == S.workspace_size(
            params(mode=S.CMP_TWO_PASS, **kw))
    assert L.speed3r_cmp_lse_bound(ctypes.byref(params(T=7 * 16, B=16)), FAKE, ws, big, FAKE,
                                   None) == S.S3R_ERR_UNSUPPORTED
    p = params(T=8 * 16, B=16)  # one group: both apply
    assert S.redo_flag_count(p) == 4 * 1 * 4
    assert single(p, redo=None) == S.S3R_ERR_INVALID_ARG
    assert single(p, redo=ctypes.c_void_p((1 << 20) + 4)) == S.S3R_ERR_INVALID_ARG
    big_p = params(T=1_374_000, H=16, B=64, k=16)
    assert S.redo_flag_count(big_p) == 16 * 5368 * 4
    # the forward workspace holds the redo flags only when the single pass runs
    two = S.workspace_size(params(T=1_374_000, H=16, B=64, k=16, mode=S.CMP_TWO_PASS))
    assert S.workspace_size(big_p) == two + S.redo_flag_count(big_p) * 4
    # automatic mode: the single pass for k <= 48 or when every candidate fits the list of 64
    assert S.workspace_size(params(T=1_374_000, H=16, B=64, k=49)) == S.workspace_size(
        params(T=1_374_000, H=16, B=64, k=49, mode=S.CMP_TWO_PASS))
    assert S.workspace_size(params(T=1_374_000, H=16, B=64, k=48)) > S.workspace_size(
        params(T=1_374_000, H=16, B=64, k=48, mode=S.CMP_TWO_PASS))
    assert S.workspace_size(params(T=60 * 64, B=64, k=40)) > S.workspace_size(
        params(T=60 * 64, B=64, k=40, mode=S.CMP_TWO_PASS))


def test_training_entry_points_validate_before_launching():
    """The training forward and the backward reject bad parameters, null or misaligned
    pointers, bad dout strides and short workspaces on the host (no launch, no GPU needed)."""
    L = S.lib()
    p = params()
    tw, bw = S.lib().speed3r_train_workspace_size(ctypes.byref(p)), \
        S.lib().speed3r_bwd_workspace_size(ctypes.byref(p))
    assert tw > S.workspace_size(p) > 0 and bw > 0
    ws = ctypes.c_void_p(1 << 20)
    fwd = lambda pp, q=FAKE, w=ws, n=tw: L.speed3r_sparse_attn_fwd_train(  # noqa: E731
        ctypes.byref(pp), q, FAKE, FAKE, FAKE, FAKE, None, w, ctypes.c_size_t(n), None)
    assert fwd(params(D=32)) == S.S3R_ERR_UNSUPPORTED
    assert fwd(params(k=0)) == S.S3R_ERR_INVALID_ARG
    assert fwd(p, q=None) == S.S3R_ERR_INVALID_ARG
    assert fwd(p, n=tw - 1) == S.S3R_ERR_WORKSPACE
    assert fwd(p, w=None) == S.S3R_ERR_WORKSPACE

    def bwd(pp, dout=FAKE, st=(4 * 64, 64), train=tw, w=ws, n=bw, dq=FAKE):
        return L.speed3r_sparse_attn_bwd(ctypes.byref(pp), FAKE, FAKE, FAKE, FAKE, dout,
                                         ctypes.c_int64(st[0]), ctypes.c_int64(st[1]), ws,
                                         ctypes.c_size_t(train), dq, FAKE, FAKE, FAKE, w,
                                         ctypes.c_size_t(n), None)
    assert bwd(params(B=48)) == S.S3R_ERR_UNSUPPORTED
    assert bwd(p, dout=None) == S.S3R_ERR_INVALID_ARG
    assert bwd(p, dq=None) == S.S3R_ERR_INVALID_ARG
    assert bwd(p, dout=ctypes.c_void_p((1 << 20) + 2)) == S.S3R_ERR_INVALID_ARG
    assert bwd(p, st=(4 * 64 + 4, 64)) == S.S3R_ERR_INVALID_ARG  # stride not a multiple of 8
    assert bwd(p, train=tw - 1) == S.S3R_ERR_WORKSPACE
    assert bwd(p, n=bw - 1) == S.S3R_ERR_WORKSPACE


@pytest.mark.parametrize("T,B,k,F,own", [
    (1_374_000, 64, 16, 0, 0), (1_374_000, 64, 32, 0, 0), (1_374_000, 64, 33, 22, 1),
    (1_374_000, 64, 48, 0, 0), (1_374_000, 64, 49, 0, 0), (1_374_000, 64, 49, 2, 1),
    (60 * 64, 64, 30, 0, 0), (7 * 16, 16, 4, 0, 0), (8 * 16, 16, 4, 0, 0), (4096, 128, 4, 0, 0),
    (100 * 64, 64, 65, 0, 0), (100 * 64, 64, 30, 40, 0), (1000, 32, 5, 3, 1),
])
def test_runs_single_matches_the_library(T, B, k, F, own):
    """The binding's rule for the automatic mode agrees with the library's choice (seen through
    the workspace, which holds the redo flags only when the single pass runs)."""
    for mode in (S.CMP_AUTO, S.CMP_TWO_PASS, S.CMP_SINGLE):
        p = params(T=T, H=4, B=B, k=k, forced=F, own=own, mode=mode)
        two = S.workspace_size(params(T=T, H=4, B=B, k=k, forced=F, own=own, mode=S.CMP_TWO_PASS))
        got = S.workspace_size(p)
        if mode == S.CMP_SINGLE and got == 0:
            continue
        assert S.runs_single(p) == (got > two), (mode, got, two)


def test_binding_rejects_bad_result_buffers():
    """The binding checks every tensor it turns into a pointer (no GPU needed: the checks
    run before any call). q, k, v must sit on one GPU; out must be q's shape, type and
    device, contiguous; gates float32 [H, 2] or [T, H, 2] with strides (2H, 2, 1); sel_idx
    int32 [H, Nb, num_selected] contiguous (a selection with forced or own blocks is longer
    than topk, and a short buffer would take out-of-bounds device writes)."""
    import torch

    T, H = 256, 2
    q = torch.zeros(T, H, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="one GPU"):
        S.make_params(q, q, q, 16, 4)
    # result buffers, checked against q's own device (CPU here)
    S._check_out(torch.empty_like(q), q)
    for bad in (torch.empty(T, H, 64, dtype=torch.float32),       # wrong type
                torch.empty(T, H + 1, 64, dtype=torch.bfloat16),   # wrong shape
                torch.empty(T, 64, H, dtype=torch.bfloat16).transpose(1, 2)):  # strided
        with pytest.raises(ValueError, match="out"):
            S._check_out(bad, q)
    S._check_gates(torch.ones(H, 2), q)
    S._check_gates(torch.ones(T, H, 2), q)
    for bad in (torch.ones(H, 2, dtype=torch.bfloat16), torch.ones(2, H).t(), torch.ones(H, 3),
                torch.ones(T, H, 4)[:, :, :2], torch.ones(T + 1, H, 2)):
        with pytest.raises(ValueError, match="gates"):
            S._check_gates(bad, q)
    p = params(T=T, H=H, B=16, k=4, forced=3, own=1)
    n_sel = S.num_selected(p)
    assert n_sel == 3 + 1 + 4
    S._check_sel(torch.empty(H, T // 16, n_sel, dtype=torch.int32), p, q.device)
    for bad in (torch.empty(H, T // 16, 4, dtype=torch.int32),      # sized for topk only
                torch.empty(H, T // 16, n_sel, dtype=torch.int64),
                torch.empty(H, n_sel, T // 16, dtype=torch.int32).transpose(1, 2)):
        with pytest.raises(ValueError, match="sel_idx"):
            S._check_sel(bad, p, q.device)
    with pytest.raises(ValueError, match="workspace"):
        S._check_workspace(torch.empty(64, dtype=torch.float32), q.device)


def test_noalloc_entry_point_validates_before_touching_the_device():
    """The allocation-free forward pass rejects bad arguments and problems larger than its
    fixed array before its first device call (so these run without a GPU)."""
    L = S.lib()
    cap = S.noalloc_scratch_bytes()
    assert cap == 512 << 20
    call = lambda pp, q=FAKE: L.speed3r_sparse_attn_fwd_noalloc(  # noqa: E731
        ctypes.byref(pp), q, FAKE, FAKE, FAKE, FAKE, None, None)
    assert call(params(k=0)) == S.S3R_ERR_INVALID_ARG
    assert call(params(D=32)) == S.S3R_ERR_UNSUPPORTED
    assert call(params(), q=None) == S.S3R_ERR_INVALID_ARG
    big = params(T=137_400, H=16, B=64, k=16)
    assert S.workspace_size(big) > cap
    assert call(big) == S.S3R_ERR_SCRATCH
    assert S.workspace_size(params(T=43_968, H=16, B=64, k=16)) <= cap
