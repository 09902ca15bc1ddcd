#!/usr/bin/env python3
"""Benchmark of the sparse global attention forward pass on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic tokens: block pooling
(+ packing of the raw keys/values), the compression branch (by default the single pass from
the group-mean bound of the log-sum-exp, with its exact reruns; --cmp-mode two_pass for the
two exact passes), block scores and top-k selection, selection attention + gated combine.
Inputs are generated on the GPU and resident in HBM before timing starts. The dense attention
comparator is timed separately at the same shape. Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload v1000_k16]
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from sparse_global_attention_block_amd import speed3r as S  # noqa: E402
from sparse_global_attention_block_amd import workloads as W  # noqa: E402

METRIC = "sparse global-attn fwd tokens/s at 1000 views; MFMA/HBM roofline %; x vs dense"
PEAK_BF16 = 2.5e15       # dense MFMA, bf16/fp16 (MI355X)
PEAK_HBM = 8.0e12        # bytes/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_work(w: W.Workload, T: int, Nb: int):
    """Per-launch algorithmic flops / bytes of each kernel (per-unit figures times units)."""
    H, D, B, k = w.H, w.D, w.block, w.k_eff
    th = T * H
    Nb_g = Nb // 8
    sel_keys = sum(min(T, (j + 1) * B) - j * B for j in range(min(k, Nb)))  # ~ k*B
    return {
        # reads k and v once (2 x 128 B per token-head), writes 12 KB per 32 pooled tokens
        "pool": {"bytes": th * 256 + H * math.ceil(Nb / 32) * 12288, "bound": "hbm"},
        # reads k and v, writes them back as packed tiles
        "pack": {"bytes": th * 256 * 2, "bound": "hbm"},
        # logits q.Kc over all coarse tokens: 2*D flops per (token, head, block)
        "cmp_lse": {"flops": 2 * D * th * Nb, "bound": "mfma"},
        # logits + P.Vc: 4*D flops per (token, head, block)
        "cmp_fused": {"flops": 4 * D * th * Nb, "bound": "mfma"},
        # bound pass: logits over the group keys (means of 8 pooled keys), 2*D per pair
        "cmp_bound": {"flops": 2 * D * th * Nb_g, "bound": "mfma"},
        # single pass: logits + P.Vc once over all coarse tokens, 4*D flops per pair (its
        # rescoring of the listed blocks and the exact reruns are not counted)
        "cmp_single": {"flops": 4 * D * th * Nb, "bound": "mfma"},
        # reads the score matrix once (4 B per (head, query block, key block))
        "topk": {"bytes": 4 * H * Nb * Nb, "bound": "hbm"},
        # q.k and p.v over the k*B selected tokens: 4*D flops per (token, head, key)
        "sel": {"flops": 4 * D * th * sel_keys, "bound": "mfma"},
    }


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` (its demangled name, e.g. the compressed-attention
    pass-2 kernel), from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary (already
    scaled by the copy calibration). None when no summary exists for this workload, the kernel
    is not in it, or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_bytes_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in ("s3r_cmp.hip", "s3r_common.hpp"):
        h.update(open(os.path.join(ROOT, "sparse_global_attention_block_amd", "csrc", f), "rb").read())
    if rec.get("cmp_fused_source_sha256") != h.hexdigest():
        return None
    v = rec["kernels"].get(kernel)
    return None if v is None else v["read_bytes"] + v["write_bytes"]


def timed_stages(st: "S.Stages", reps: int, single: bool):
    """Runs the hot path stage by stage with HIP events between stages (on the stream the
    library launches on) and returns the mean duration of each stage in ms."""
    if single:  # the single compression pass (its exact reruns inside cmp_single)
        names = ["pool", "cmp_bound", "cmp_single", "sel"]
        fns = [st.run_pool, st.run_lse_bound, st.run_single_topk, st.run_sel]
    elif st.folds_topk:  # the two passes with top-k inside pass 2
        names = ["pool", "cmp_lse", "cmp_fused", "sel"]
        fns = [st.run_pool, st.run_lse, st.run_fused_topk, st.run_sel]
    else:
        names = ["pool", "cmp_lse", "cmp_fused", "topk", "sel"]
        fns = [st.run_pool, st.run_lse, st.run_fused, st.run_topk, st.run_sel]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(reps)]
    torch.cuda.synchronize()
    for r in range(reps):
        ev[r][0].record()
        for i, f in enumerate(fns):
            f()
            ev[r][i + 1].record()
    torch.cuda.synchronize()
    out = {n: sum(ev[r][i].elapsed_time(ev[r][i + 1]) for r in range(reps)) / reps
           for i, n in enumerate(names)}
    return out


def cpu_baseline(w, x, sel_gpu, out_gpu, n_rows=48, seed=0):
    """Times the float64 CPU oracle on one head: pooling over all tokens plus n_rows sampled
    query blocks, and checks the GPU rows against it. The full-job time is extrapolated as
    H * (pool + Nb * mean row time)."""
    import numpy as np
    from oracle import oracle as O

    T, H = x["q"].shape[0], w.H
    Nb = -(-T // w.block)
    h = 0
    rng = np.random.default_rng(seed)
    rows = sorted(set([0, Nb - 1] + [int(r) for r in rng.integers(0, Nb, n_rows - 2)]))
    t0 = time.perf_counter()
    # window workloads: the oracle reorders the head's tokens itself (its own window order)
    order = O.window_order(*w.layout()) if w.window else np.arange(T)
    t_order = time.perf_counter() - t0
    hq, hk, hv = (x[n][:, h:h + 1].cpu()[torch.from_numpy(order)].contiguous()
                  for n in ("q", "k", "v"))
    hg = x["gates"][h:h + 1].cpu()
    t0 = time.perf_counter()
    kc, vc = O.pool(hk, w.block), O.pool(hv, w.block)
    t_pool = time.perf_counter() - t0
    t0 = time.perf_counter()
    r = O.forward_rows(hq, hk, hv, hg, w.block, w.topk, np.zeros(len(rows), np.int32), rows,
                       kc=kc, vc=vc, forced=w.forced, own=w.own)
    t_rows = time.perf_counter() - t0
    per_row = t_rows / len(rows)
    t_full = t_order + H * (t_pool + Nb * per_row)
    # parity of the sampled rows
    gsel = sel_gpu[h, rows].cpu().numpy()
    same = float((gsel == r["sel"]).all(axis=-1).mean())
    err_max, err_sum, n = 0.0, 0.0, 0
    exc_max, exc_sum = 0.0, 0.0  # error beyond the output's own rounding (half an ulp of ref)
    bits = 11 if out_gpu.dtype == torch.float16 else 8
    ref = r
    if same < 1.0:
        ref = O.forward_rows(hq, hk, hv, hg, w.block, w.topk, np.zeros(len(rows), np.int32),
                             rows, kc=kc, vc=vc, sel_in=gsel, forced=w.forced, own=w.own)
    for a, i in enumerate(rows):
        nn = min(T, (i + 1) * w.block) - i * w.block
        toks = torch.from_numpy(order[i * w.block:i * w.block + nn]).to(out_gpu.device)
        g = out_gpu[toks, h].float().cpu().numpy()
        d = abs(g - ref["out"][a, :nn])
        err_max = max(err_max, float(d.max()))
        err_sum += float(d.sum())
        ax = np.maximum(np.abs(ref["out"][a, :nn]), 2.0 ** -14 if bits == 11 else 2.0 ** -126)
        exc = np.maximum(d - np.exp2(np.floor(np.log2(ax)) - bits), 0.0)
        exc_max = max(exc_max, float(exc.max()))
        exc_sum += float(exc.sum())
        n += d.size
    return {
        "value": T / t_full, "unit": "tokens/s", "cores": O.num_threads(), "kind": "oracle",
        "sample": f"head 0 of {H}: pooling over all {T} tokens ({t_pool:.2f} s) + {len(rows)} "
                  f"query blocks of {w.block} ({t_rows:.2f} s); full job extrapolated as "
                  f"H*(pool + Nb*row) = {t_full:.0f} s",
    }, {"rows": len(rows), "rows_same_selection": same, "out_max_abs": err_max,
        "out_mean_abs": err_sum / max(1, n), "out_max_beyond_rounding": exc_max,
        "out_mean_beyond_rounding": exc_sum / max(1, n)}


def time_backward(w: W.Workload, x, reps: int):
    """Times the training forward pass and the backward pass on the same inputs (HIP events
    on the library's stream). Algorithmic flops of the backward: per (query, key) pair and
    head, the compression and selection branches each recompute the logits (2D) and dP (2D)
    and form dq, dk, dv (2D each): 10D per pair, over T*Nb pooled pairs and T*(k*B) selected
    pairs."""
    T, H, D = x["q"].shape
    gen = torch.Generator(device=x["q"].device).manual_seed(29)
    dout = torch.randn(T, H, D, device=x["q"].device, generator=gen).to(torch.bfloat16)
    p = S.make_params(x["q"], x["k"], x["v"], w.block, w.topk, 0.0, x["gates"], w.forced, w.own)
    tws = S.alloc_workspace(S.train_workspace_size(p), x["q"].device)
    bws = S.alloc_workspace(S.bwd_workspace_size(p), x["q"].device)
    st = S.sparse_attn_fwd_train(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk,
                                 forced_blocks=w.forced, force_own=w.own, workspace=tws)
    S.sparse_attn_bwd(st, dout, workspace=bws)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    f_ms = b_ms = 0.0
    for _ in range(reps):
        ev[0].record()
        st = S.sparse_attn_fwd_train(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk,
                                     forced_blocks=w.forced, force_own=w.own, workspace=tws)
        ev[1].record()
        S.sparse_attn_bwd(st, dout, workspace=bws)
        ev[2].record()
        torch.cuda.synchronize()
        f_ms += ev[0].elapsed_time(ev[1]) / reps
        b_ms += ev[1].elapsed_time(ev[2]) / reps
    Nb = -(-T // w.block)
    sel_keys = w.k_eff * w.block
    flops = 10 * D * T * H * (Nb + sel_keys)
    del tws, bws, st
    return {"ms": b_ms, "fwd_train_ms": f_ms, "flops": flops, "achieved": flops / (b_ms * 1e-3) / 1e12,
            "unit": "TFLOP/s", "frac": flops / (b_ms * 1e-3) / PEAK_BF16,
            "note": "algorithmic flops 10*D per (query, key) pair and head, pooled and selected pairs"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="v1000_k16", choices=sorted(W.WORKLOADS))
    ap.add_argument("--dense-reps", type=int, default=1)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cmp-mode", default="auto", choices=["auto", "two_pass", "single"],
                    help="compression branch: automatic (the single pass where it applies), "
                         "the two exact passes, or the single pass")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run one device-to-device copy of MIB MiB (the reference kernel "
                         "for scaling HBM byte counters) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n}))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the attention shards by head; see the design notes). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    w = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] workload {w.name}: T={w.T} H={w.H} B={w.block} k={w.topk} F={w.forced} "
        f"own={w.own}")
    x = W.make_inputs(w, device=dev)
    torch.cuda.synchronize()
    T, H, D = x["q"].shape
    mode = {"auto": S.CMP_AUTO, "two_pass": S.CMP_TWO_PASS, "single": S.CMP_SINGLE}[args.cmp_mode]
    p = S.make_params(x["q"], x["k"], x["v"], w.block, w.topk, 0.0, x["gates"], w.forced, w.own,
                      mode)
    single = S.runs_single(p)
    Nb = S.num_blocks(p)
    layout = w.layout()
    ws = S.alloc_workspace(S.windows_workspace_size(p, layout) if layout else
                           S.workspace_size(p), dev)
    out = torch.empty(T, H, D, dtype=x["q"].dtype, device=dev)
    sel = torch.empty(H, Nb, w.k_eff, dtype=torch.int32, device=dev)

    def step():
        if layout:  # 2-D windows: reorder in, forward, reorder out
            S.sparse_attn_fwd_windows(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk,
                                      layout, out=out, sel_idx=sel, workspace=ws,
                                      forced_blocks=w.forced, force_own=w.own, cmp_mode=mode)
        else:
            S.sparse_attn_fwd(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk, out=out,
                              sel_idx=sel, workspace=ws, forced_blocks=w.forced,
                              force_own=w.own, cmp_mode=mode)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps
    log(f"[bench] sparse forward {ms:.3f} ms/step (wall {1e3 * t_wall / args.steps:.3f}), "
        f"compression {'single pass' if single else 'two passes'}")
    two_pass = None
    if single and not layout:
        # the same step with the two exact passes, for comparison (not the reported value)
        del ws
        torch.cuda.empty_cache()
        ws = S.alloc_workspace(S.workspace_size(S.make_params(
            x["q"], x["k"], x["v"], w.block, w.topk, 0.0, x["gates"], w.forced, w.own,
            S.CMP_TWO_PASS)), dev)
        reps = max(1, min(3, args.steps))
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            S.sparse_attn_fwd(x["q"], x["k"], x["v"], x["gates"], w.block, w.topk, out=out,
                              workspace=ws, forced_blocks=w.forced, force_own=w.own,
                              cmp_mode=S.CMP_TWO_PASS)
        t1.record()
        torch.cuda.synchronize()
        two_pass = {"ms_per_step": t0.elapsed_time(t1) / reps,
                    "value": T / (t0.elapsed_time(t1) / reps * 1e-3)}
        log(f"[bench] the same step with the two exact passes: {two_pass['ms_per_step']:.3f} ms")

    # per-kernel durations: the same kernels launched stage by stage
    del ws
    torch.cuda.empty_cache()
    folds = w.block <= 64 and min(w.topk, Nb - min(w.forced, Nb)) <= 64
    xs, perm_ms = x, None
    if layout:
        # window order once; the reordering (3 tensors in, 1 out) is timed on its own
        xs = {n: S.window_permute(layout, x[n]) for n in ("q", "k", "v")}
        xs["gates"] = x["gates"]
        tmp = torch.empty_like(out)
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        p0.record()
        for n in ("q", "k", "v"):
            S.window_permute(layout, x[n], dst=tmp)
        S.window_permute(layout, xs["q"], dst=tmp, inverse=True)
        p1.record()
        torch.cuda.synchronize()
        perm_ms = p0.elapsed_time(p1)
        del tmp
    st = S.Stages(xs["q"], xs["k"], xs["v"], xs["gates"], w.block, w.topk, keep_o_sel=False,
                  keep_score=not folds, forced_blocks=w.forced, force_own=w.own)
    st.run_pool()
    st.run_lse()
    stage_ms = timed_stages(st, max(1, min(3, args.steps)), single)
    redone = int((st.redo != 0).sum().item()) if single else None
    if perm_ms is not None:
        stage_ms["window_permute"] = perm_ms
    log(f"[bench] stages (ms): " + ", ".join(f"{k} {v:.3f}" for k, v in stage_ms.items()))
    work = algorithmic_work(w, T, Nb)
    # pool stage = pool kernel + pack kernel; report the pool stage against both kernels' bytes
    kernels = {}
    for name, ms_k in stage_ms.items():
        if name == "pool":
            wk = {"bytes": work["pool"]["bytes"] + work["pack"]["bytes"], "bound": "hbm"}
        elif name == "window_permute":  # 4 tensors, each read and written once
            wk = {"bytes": 4 * 2 * T * H * D * 2, "bound": "hbm"}
        else:
            wk = work[name]
        if wk["bound"] == "hbm":
            ach = wk["bytes"] / (ms_k * 1e-3)
            kernels[name] = {"ms": ms_k, "bound": "hbm", "achieved": ach / 1e9, "unit": "GB/s",
                             "frac": ach / PEAK_HBM}
        else:
            ach = wk["flops"] / (ms_k * 1e-3)
            kernels[name] = {"ms": ms_k, "bound": "mfma", "achieved": ach / 1e12,
                             "unit": "TFLOP/s", "frac": ach / PEAK_BF16}
    if folds and not layout:
        # the separate top-k kernel (the path for B = 128 or more than 64 chosen blocks) on this
        # workload's score matrix: reported beside the step, not part of it
        del st
        torch.cuda.empty_cache()
        st = S.Stages(xs["q"], xs["k"], xs["v"], xs["gates"], w.block, w.topk, keep_o_sel=False,
                      keep_score=True, forced_blocks=w.forced, force_own=w.own)
        st.run_pool()
        st.run_lse()
        st.run_fused()
        st.run_topk()
        reps = max(1, min(3, args.steps))
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(reps):
            st.run_topk()
        t1.record()
        torch.cuda.synchronize()
        ms_k = t0.elapsed_time(t1) / reps
        ach = work["topk"]["bytes"] / (ms_k * 1e-3)
        kernels["topk_separate"] = {"ms": ms_k, "bound": "hbm", "achieved": ach / 1e9,
                                    "unit": "GB/s", "frac": ach / PEAK_HBM,
                                    "note": "separate top-k kernel on the score matrix; not in "
                                            "the step, where top-k runs inside pass 2"}
        log(f"[bench] separate top-k on the score matrix {ms_k:.3f} ms")
    # the compression kernel instance the step launched: <fused, query blocks per wave, waves,
    # running top-k, fp16, single pass, tiles in flight (0: default)>
    pass2_kernel = (f"s3r::cmp_kernel<true, {64 // w.block if w.block <= 64 else 1}, 4, "
                    f"{'true' if folds else 'false'}, {'true' if w.dtype == 'fp16' else 'false'}, "
                    f"{'true' if single else 'false'}, 0>")
    cands = ("cmp_single", "cmp_bound", "sel") if single else ("cmp_fused", "cmp_lse", "sel")
    dom = max(cands, key=lambda n: stage_ms[n])
    roof = {"kernel": dom, "bound": "mfma", "achieved": kernels[dom]["achieved"],
            "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s", "frac": kernels[dom]["frac"],
            "traffic": measured_traffic(w.name, pass2_kernel) if dom == cands[0] else None}
    del st, xs
    torch.cuda.empty_cache()

    backward = None
    if not args.no_backward and not layout:
        backward = time_backward(w, x, max(1, min(3, args.steps)))
        log(f"[bench] training forward {backward['fwd_train_ms']:.1f} ms, backward "
            f"{backward['ms']:.1f} ms ({backward['achieved']:.0f} TFLOP/s algorithmic)")
        torch.cuda.empty_cache()

    dense = None
    if not args.no_dense:
        small = W.make_inputs(W.WORKLOADS["tiny"], device=dev)
        S.dense_attn_fwd(small["q"], small["k"], small["v"])  # load the kernel code
        dws = S.alloc_workspace(S.dense_workspace_size(p), dev)
        dout = torch.empty_like(out)
        torch.cuda.synchronize()
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record()
        for _ in range(args.dense_reps):
            S.dense_attn_fwd(x["q"], x["k"], x["v"], out=dout, workspace=dws)
        d1.record()
        torch.cuda.synchronize()
        dense_ms = d0.elapsed_time(d1) / args.dense_reps
        dense = {"ms": dense_ms, "tflops": 4 * D * T * T * H / (dense_ms * 1e-3) / 1e12}
        log(f"[bench] dense {dense_ms:.1f} ms ({dense['tflops']:.0f} TFLOP/s)")
        del dws, dout

    cpu, parity = None, None
    if not args.no_cpu:
        cpu, parity = cpu_baseline(w, x, sel, out)
        log(f"[bench] cpu oracle {cpu['value']:.1f} tokens/s; parity {parity}")

    rec = {
        "metric": METRIC, "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded structured q/k/v, generated on the GPU)",
        "config": {**w.describe(), "parallelism": "none (1 GPU)",
                   "compression": "single pass" if single else "two passes"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "single_pass_waves_redone": redone,
        "two_pass": two_pass,
        "backward": backward,
        "dense": dense,
        "x_vs_dense": (dense["ms"] / ms) if dense else None,
        "parity_sampled": parity,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
