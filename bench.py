#!/usr/bin/env python3
"""Benchmark of the sparse global attention forward pass on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic tokens: block pooling
(+ packing of the raw keys/values), the compression branch (by default the single pass from
the group-mean bound of the log-sum-exp, with its exact reruns; --cmp-mode two_pass for the
two exact passes), block scores and top-k selection, selection attention + gated combine.
Inputs are generated on the GPU and resident in HBM before timing starts. The dense attention
comparator is timed separately at the same shape. Prints one JSON line.

Roofline fractions are given against the vendor peaks (HBM 8 TB/s, bf16 MFMA 2.5 PFLOP/s) and
against ceilings measured in the same run with two plain kernels of the library (a streaming
copy and a loop of bf16 matrix products); matrix-core kernels report algorithmic flops (what
the method needs) and executed flops (what the kernels issue: hi + lo pooled keys, the
ones-row denominators).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload v1000_k16]
  python bench.py --table          # every configuration of the workload list, one line each
"""
import argparse
import hashlib
import json
import math
import os
import platform
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


def events(n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def calibrate(dev):
    """Measured ceilings: the library's streaming copy over 4 GiB and its loop of bf16 matrix
    products, each the best of 3 runs (HIP events on the launch stream)."""
    n = 4 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    S.calib_copy(src, dst)
    best = math.inf
    for _ in range(3):
        e0, e1 = events(2)
        e0.record()
        moved = S.calib_copy(src, dst)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    copy_gbps = moved / (best * 1e-3) / 1e9
    del src, dst
    wg, iters = 4096, 4000
    sink = torch.empty(wg * 256, dtype=torch.float32, device=dev)
    S.calib_mfma(sink, wg, 10)
    best = math.inf
    for _ in range(3):
        e0, e1 = events(2)
        e0.record()
        flops = S.calib_mfma(sink, wg, iters)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    mfma_tf = flops / (best * 1e-3) / 1e12
    torch.cuda.empty_cache()
    return {"hbm_copy_GBps": copy_gbps, "mfma_bf16_TFLOPs": mfma_tf,
            "copy": f"speed3r_calib_copy of 4 GiB (reads + writes), best of 3",
            "mfma": f"speed3r_calib_mfma: {wg} work-groups x 4 waves x {iters} rounds of 8 "
                    f"independent 16x16x32 bf16 products, best of 3"}


def work_of(w: W.Workload, T: int, Nb: int, topk: int):
    """Per-launch algorithmic work of each kernel (the per-unit figure of the method times the
    units one launch processes) and, for matrix-core kernels, the executed flops."""
    H, D, B = w.H, w.D, w.block
    th = T * H
    Nb_g = Nb // 8
    forced = min(w.forced, Nb)
    own = 1 if w.own and forced < Nb else 0
    k_eff = forced + own + min(topk, Nb - forced - own)
    sel_keys = sum(min(T, (j + 1) * B) - j * B for j in range(min(k_eff, Nb)))  # ~ k*B
    return {
        # the pool stage (packing kernel, then pooling from the blocks' column sums): reads k
        # and v once (2 x 128 B per token-head), writes them back as packed raw tiles and
        # writes 12 KB per 32 pooled tokens
        "pool": {"bytes": th * 256 * 2 + H * math.ceil(Nb / 32) * 12288, "bound": "hbm"},
        # logits q.Kc over all pooled keys: 2D per (token, head, block); the kernel multiplies
        # by the hi and the lo part of every pooled key (4D)
        "cmp_lse": {"flops": 2 * D * th * Nb, "flops_exec": 4 * D * th * Nb, "bound": "mfma"},
        # logits + P.Vc: 4D per pair; executed 6D (hi + lo logits, P.V)
        "cmp_fused": {"flops": 4 * D * th * Nb, "flops_exec": 6 * D * th * Nb, "bound": "mfma"},
        # bound pass: logits over the group keys (means of 8 pooled keys), hi parts only
        "cmp_bound": {"flops": 2 * D * th * Nb_g, "flops_exec": 2 * D * th * Nb_g,
                      "bound": "mfma"},
        # single pass: the method's 4D per pair (logits, P.Vc); executed 6D as pass 2 (its
        # rescoring of 64 listed blocks per query block and the exact reruns not counted)
        "cmp_single": {"flops": 4 * D * th * Nb, "flops_exec": 6 * D * th * Nb,
                       "bound": "mfma"},
        # reads the score matrix once (4 B per (head, query block, key block))
        "topk": {"bytes": 4 * H * Nb * Nb, "bound": "hbm"},
        # q.k and p.v over the ~k*B selected keys: 4D per (token, head, key); executed 4.5D
        # (the softmax denominator is one more product per four P.V products)
        "sel": {"flops": 4 * D * th * sel_keys, "flops_exec": 4.5 * D * th * sel_keys,
                "bound": "mfma"},
        "dense": {"flops": 4 * D * th * T, "flops_exec": 4.5 * D * th * T, "bound": "mfma"},
    }


def rate(name, ms, wk, ceil):
    """Achieved rate of one kernel and its fractions of the vendor peak and the measured
    ceiling."""
    if wk["bound"] == "hbm":
        ach = wk["bytes"] / (ms * 1e-3)
        r = {"ms": ms, "bound": "hbm", "achieved": ach / 1e9, "unit": "GB/s",
             "frac": ach / PEAK_HBM}
        if ceil:
            r["frac_of_measured"] = ach / 1e9 / ceil["hbm_copy_GBps"]
        return r
    ach = wk["flops"] / (ms * 1e-3)
    exe = wk["flops_exec"] / (ms * 1e-3)
    r = {"ms": ms, "bound": "mfma", "achieved": ach / 1e12, "unit": "TFLOP/s",
         "frac": ach / PEAK_BF16, "achieved_executed": exe / 1e12,
         "frac_executed": exe / PEAK_BF16}
    if ceil:
        r["frac_of_measured"] = ach / 1e12 / ceil["mfma_bf16_TFLOPs"]
        r["frac_executed_of_measured"] = exe / 1e12 / ceil["mfma_bf16_TFLOPs"]
    return r


def source_hash():
    h = hashlib.sha256()
    for f in ("s3r_cmp.hip", "s3r_common.hpp"):
        h.update(open(os.path.join(ROOT, "sparse_global_attention_block_amd", "csrc", f),
                      "rb").read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` (its demangled name) from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary (already scaled by the copy calibration). None when no
    summary exists for this workload, the kernel is not in it, or the compression kernel's
    source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_bytes_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("cmp_fused_source_sha256") != source_hash():
        return None
    v = rec["kernels"].get(kernel)
    return None if v is None else v["read_bytes"] + v["write_bytes"]


def cmp_kernel_name(w: W.Workload, folds: bool, single: bool) -> str:
    """Demangled name of the compression kernel instance the step launches:
    <fused, query blocks per wave, waves, running top-k, fp16, single pass, tiles in flight
    (0: default), scores only>."""
    return (f"s3r::cmp_kernel<true, {64 // w.block if w.block <= 64 else 1}, 4, "
            f"{'true' if folds else 'false'}, {'true' if w.dtype == 'fp16' else 'false'}, "
            f"{'true' if single else 'false'}, 0, false>")


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
    ev = [events(len(fns) + 1) for _ in range(reps)]
    torch.cuda.synchronize()
    for r in range(reps):
        ev[r][0].record()
        for i, f in enumerate(fns):
            f()
            ev[r][i + 1].record()
    torch.cuda.synchronize()
    return {n: sum(ev[r][i].elapsed_time(ev[r][i + 1]) for r in range(reps)) / reps
            for i, n in enumerate(names)}


def stage_kernels(w, x, topk, reps, single, ceil, T, Nb):
    """Per-kernel durations and rates: the same kernels launched stage by stage."""
    st = S.Stages(x["q"], x["k"], x["v"], x["gates"], w.block, topk, keep_o_sel=False,
                  keep_score=not (w.block <= 64 and min(topk, Nb - min(w.forced, Nb)) <= 64),
                  forced_blocks=w.forced, force_own=w.own)
    st.run_pool()
    st.run_lse()
    stage_ms = timed_stages(st, reps, single)
    redone = int((st.redo != 0).sum().item()) if single else None
    work = work_of(w, T, Nb, topk)
    kernels = {}
    for name, ms_k in stage_ms.items():
        kernels[name] = rate(name, ms_k, work[name], ceil)
    del st
    torch.cuda.empty_cache()
    return kernels, redone


def sample_rows(w: W.Workload, Nb: int, n: int, seed: int):
    """Stratified query blocks of one head: the first, the short last, blocks that hold a
    view's special tokens (about a quarter of the sample), and random blocks."""
    import numpy as np
    rng = np.random.default_rng(seed)
    rows = {0, Nb - 1}
    views = max(1, -(-w.T // w.tokens_per_view))
    if w.special:
        for v in rng.choice(views, size=min(views, max(1, n // 4)), replace=False):
            rows.add(int(v) * w.tokens_per_view // w.block)
    while len(rows) < min(n, Nb):
        rows.add(int(rng.integers(0, Nb)))
    return sorted(rows)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_leg(w, x, topk, sel_gpu, out_gpu, heads, rows_per_head, rows_1t, seed=0):
    """The float64 CPU oracle on a bounded, stratified sample of the same workload, timed on
    the host's cores (all threads, and one thread on a smaller part of the sample), and the
    GPU rows checked against it. Full-job time is extrapolated as H * (pool + Nb * row)."""
    import numpy as np
    from oracle import oracle as O
    from tests import helpers as TH

    T, H = x["q"].shape[0], w.H
    Nb = -(-T // w.block)
    all_threads = O.num_threads()
    t_pool = t_rows = t_rows1 = t_pool1 = 0.0
    n_rows = n_rows1 = 0
    sel_stats = {"same_set": 0.0, "exact_rule": 0.0, "contract_gap": 0.0, "rel_gap": 0.0}
    gpu_out, ref_out = [], []
    for h in heads:
        rows = sample_rows(w, Nb, rows_per_head, seed + h)
        hq, hk, hv = (x[n][:, h:h + 1].contiguous().cpu() for n in ("q", "k", "v"))
        hg = x["gates"][h:h + 1].cpu()
        O.set_num_threads(all_threads)
        t0 = time.perf_counter()
        kc, vc = O.pool(hk, w.block), O.pool(hv, w.block)
        t_pool += time.perf_counter() - t0
        zeros = np.zeros(len(rows), np.int32)
        t0 = time.perf_counter()
        r = O.forward_rows(hq, hk, hv, hg, w.block, topk, zeros, rows, kc=kc, vc=vc,
                           forced=w.forced, own=w.own)
        t_rows += time.perf_counter() - t0
        n_rows += len(rows)
        sub = rows[:: max(1, len(rows) // rows_1t)][:rows_1t]
        O.set_num_threads(1)
        if h == heads[0]:
            t0 = time.perf_counter()
            O.pool(hk, w.block), O.pool(hv, w.block)
            t_pool1 = time.perf_counter() - t0
        t0 = time.perf_counter()
        O.forward_rows(hq, hk, hv, hg, w.block, topk, np.zeros(len(sub), np.int32), sub, kc=kc,
                       vc=vc, forced=w.forced, own=w.own)
        t_rows1 += time.perf_counter() - t0
        n_rows1 += len(sub)
        O.set_num_threads(all_threads)
        gsel = sel_gpu[h, rows].cpu().numpy()
        F = min(w.forced, Nb)
        st = {}
        _, differing = TH.check_selection(gsel, r["score"], r["sel"], topk, forced=F,
                                          qblocks=rows if w.own and F < Nb else None,
                                          dtype=w.dtype, stats=st)
        for key in sel_stats:
            sel_stats[key] += st[key] * len(rows)
        ref = r
        if differing:
            ref = O.forward_rows(hq, hk, hv, hg, w.block, topk, zeros, rows, kc=kc, vc=vc,
                                 sel_in=gsel, forced=w.forced, own=w.own)
        for a, i in enumerate(rows):
            nn = min(T, (i + 1) * w.block) - i * w.block
            gpu_out.append(out_gpu[i * w.block:i * w.block + nn, h].float().cpu().numpy())
            ref_out.append(ref["out"][a, :nn])
    g, ref = np.concatenate(gpu_out), np.concatenate(ref_out)
    d = np.abs(g - ref)
    bits = 11 if out_gpu.dtype == torch.float16 else 8
    ax = np.maximum(np.abs(ref), 2.0 ** -14 if bits == 11 else 2.0 ** -126)
    exc = np.maximum(d - np.exp2(np.floor(np.log2(ax)) - bits), 0.0)
    per_row, per_row1 = t_rows / n_rows, t_rows1 / n_rows1
    pool_head = t_pool / len(heads)
    t_full = H * (pool_head + Nb * per_row)
    t_full1 = H * (t_pool1 + Nb * per_row1)
    cpu = {
        "value": T / t_full, "unit": "tokens/s", "cores": all_threads, "kind": "oracle",
        "sample": f"{n_rows} (head, query block) rows over heads {list(heads)}, stratified "
                  f"(first, short last, special-token and random blocks), plus pooling of "
                  f"those heads ({t_pool:.2f} s); rows took {t_rows:.2f} s on {all_threads} "
                  f"threads; full job extrapolated as H*(pool + Nb*row) = {t_full:.0f} s",
        "one_thread": {"value": T / t_full1, "rows": n_rows1, "seconds": t_rows1,
                       "extrapolated_s": t_full1},
        "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
        "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS"),
    }
    n = max(1, n_rows)
    parity = {"rows": n_rows, "rows_same_selection": sel_stats["same_set"] / n,
              "rows_exact_rule": sel_stats["exact_rule"] / n,
              "rows_contract_gap": sel_stats["contract_gap"] / n,
              "rows_relative_gap": sel_stats["rel_gap"] / n,
              "out_max_abs": float(d.max()), "out_mean_abs": float(d.mean()),
              "out_max_beyond_rounding": float(exc.max()),
              "out_mean_beyond_rounding": float(exc.mean())}
    return cpu, parity


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
    ev = events(3)
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
    return {"ms": b_ms, "fwd_train_ms": f_ms, "flops": flops,
            "achieved": flops / (b_ms * 1e-3) / 1e12, "unit": "TFLOP/s",
            "frac": flops / (b_ms * 1e-3) / PEAK_BF16,
            "note": "algorithmic flops 10*D per (query, key) pair and head, pooled and "
                    "selected pairs"}


class Forward:
    """The forward entry point on fixed buffers (workspace, output, selection)."""

    def __init__(self, w, x, topk, mode, dev):
        self.w, self.x, self.topk, self.mode = w, x, topk, mode
        T, H, D = x["q"].shape
        self.p = S.make_params(x["q"], x["k"], x["v"], w.block, topk, 0.0, x["gates"],
                               w.forced, w.own, mode)
        self.single = S.runs_single(self.p)
        self.Nb = S.num_blocks(self.p)
        self.layout = w.layout()
        self.ws = S.alloc_workspace(S.windows_workspace_size(self.p, self.layout)
                                    if self.layout else S.workspace_size(self.p), dev)
        self.out = torch.empty(T, H, D, dtype=x["q"].dtype, device=dev)
        self.sel = torch.empty(H, self.Nb, S.num_selected(self.p), dtype=torch.int32,
                               device=dev)

    def __call__(self):
        w, x = self.w, self.x
        if self.layout:  # 2-D windows: reorder in, forward, reorder out
            S.sparse_attn_fwd_windows(x["q"], x["k"], x["v"], x["gates"], w.block, self.topk,
                                      self.layout, out=self.out, sel_idx=self.sel,
                                      workspace=self.ws, forced_blocks=w.forced,
                                      force_own=w.own, cmp_mode=self.mode)
        else:
            S.sparse_attn_fwd(x["q"], x["k"], x["v"], x["gates"], w.block, self.topk,
                              out=self.out, sel_idx=self.sel, workspace=self.ws,
                              forced_blocks=w.forced, force_own=w.own, cmp_mode=self.mode)

    def time(self, steps, warmup):
        for _ in range(warmup):
            self()
        torch.cuda.synchronize()
        e0, e1 = events(2)
        t_wall = time.perf_counter()
        e0.record()
        for _ in range(steps):
            self()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps, (time.perf_counter() - t_wall) * 1e3 / steps

    def free(self):
        del self.ws
        torch.cuda.empty_cache()


def time_dense(x, p, dev, reps):
    small = W.make_inputs(W.WORKLOADS["tiny"], device=dev)
    S.dense_attn_fwd(small["q"], small["k"], small["v"])  # load the kernel code
    dws = S.alloc_workspace(S.dense_workspace_size(p), dev)
    dout = torch.empty_like(x["q"])
    torch.cuda.synchronize()
    d0, d1 = events(2)
    d0.record()
    for _ in range(reps):
        S.dense_attn_fwd(x["q"], x["k"], x["v"], out=dout, workspace=dws)
    d1.record()
    torch.cuda.synchronize()
    del dws, dout
    torch.cuda.empty_cache()
    return d0.elapsed_time(d1) / reps


def roofline_of(kernels, single, w, folds):
    cands = ("cmp_single", "cmp_bound", "sel") if single else ("cmp_fused", "cmp_lse", "sel")
    dom = max((c for c in cands if c in kernels), key=lambda n: kernels[n]["ms"])
    k = kernels[dom]
    roof = {"kernel": dom, "bound": "mfma", "achieved": k["achieved"], "peak": PEAK_BF16 / 1e12,
            "unit": "TFLOP/s", "frac": k["frac"],
            "traffic": measured_traffic(w.name, cmp_kernel_name(w, folds, single))
            if dom == cands[0] else None,
            "achieved_executed": k["achieved_executed"], "frac_executed": k["frac_executed"]}
    if "frac_of_measured" in k:
        roof["frac_of_measured_ceiling"] = k["frac_of_measured"]
    return roof


def run_table(args, dev):
    """Every configuration of the workload list: step time, per-kernel rates, dense where the
    list asks for it, and parity against the oracle (whole problem for the tiny shapes,
    sampled rows otherwise). One JSON line per configuration, then a markdown table."""
    import numpy as np
    from oracle import oracle as O
    from tests import helpers as TH

    ceil = calibrate(dev)
    log(f"[table] ceilings {ceil}")
    rows = []
    plan = [("tiny", 8, False), ("tiny_all", 64, False), ("tiny_s", 8, False),
            ("v32", 16, False), ("v100", 16, True), ("v1000_k16", 16, True),
            ("v1000_k32", 32, False)]
    for name, topk, dense in plan:
        w = W.WORKLOADS[name]
        x = W.make_inputs(w, device=dev)
        torch.cuda.synchronize()
        T = x["q"].shape[0]
        f = Forward(w, x, topk, S.CMP_AUTO, dev)
        steps = 3 if T > 1e6 else 10
        ms, _ = f.time(steps, 2)
        kernels, redone = stage_kernels(w, x, topk, 3, f.single, ceil, T, f.Nb)
        rec = {"workload": name, "T": T, "topk": topk, "ms": ms, "tokens_per_s": T / (ms * 1e-3),
               "compression": "single pass" if f.single else "two passes",
               "kernels": kernels, "waves_redone": redone}
        if dense:
            dms = time_dense(x, f.p, dev, 1)
            rec["dense_ms"] = dms
            rec["x_vs_dense"] = dms / ms
        if T <= 5000:  # the whole problem through the oracle
            hx = {n: t.cpu() for n, t in x.items()}
            ora = O.forward_all(hx["q"], hx["k"], hx["v"], hx["gates"], w.block, topk)
            st = {}
            gsel = f.sel.cpu().numpy()
            _, differing = TH.check_selection(gsel, ora["score"], ora["sel"], topk,
                                              dtype=w.dtype, stats=st)
            ref = ora["out"]
            if differing:
                H, Nb = w.H, f.Nb
                r = O.forward_rows(hx["q"], hx["k"], hx["v"], hx["gates"], w.block, topk,
                                   np.repeat(np.arange(H), Nb), np.tile(np.arange(Nb), H),
                                   sel_in=gsel.reshape(H * Nb, -1))
                ref = r["out"].reshape(H, Nb * w.block, 64)[:, :T].transpose(1, 0, 2)
            d = np.abs(f.out.float().cpu().numpy() - ref)
            par = {"rows": st["rows"], "rows_same_selection": st["same_set"],
                   "rows_exact_rule": st["exact_rule"], "rows_contract_gap": st["contract_gap"],
                   "out_max_abs": float(d.max()), "out_mean_abs": float(d.mean())}
        else:
            heads = (0, 5, 10, 15)
            _, par = cpu_leg(w, x, topk, f.sel, f.out, heads, 16, 2, seed=7)
        rec["parity"] = par
        print(json.dumps(rec), flush=True)
        rows.append(rec)
        f.free()
        del f, x
        torch.cuda.empty_cache()

    def g(r, k, key="achieved"):
        kk = r["kernels"].get(k)
        if not kk:
            return "—"
        if kk["bound"] == "hbm":
            return f"{kk[key]:.0f} ({kk['frac']:.0%})"
        return f"{kk['achieved']:.0f} ({kk['frac']:.0%} / {kk['frac_executed']:.0%})"

    def opt(v):  # a figure only some configurations have (the dense comparator's)
        return "—" if v is None else f"{v:.1f}"

    lines = ["| config | T | k | t_sparse (ms) | tokens/s | pool+pack GB/s (%HBM) | "
             "cmp TF/s (%MFMA alg / exec) | sel TF/s (%MFMA alg / exec) | t_dense (ms) | "
             "x vs dense | rows checked / identical sel / exact rule | max-abs / mean-abs |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        cmp = "cmp_single" if "cmp_single" in r["kernels"] else "cmp_fused"
        p = r["parity"]
        lines.append(
            f"| {r['workload']} | {r['T']:,} | {r['topk']} | {r['ms']:.3f} | "
            f"{r['tokens_per_s']:.3e} | {g(r, 'pool')} | {g(r, cmp)} | {g(r, 'sel')} | "
            f"{opt(r.get('dense_ms'))} | {opt(r.get('x_vs_dense'))} | {p['rows']} / "
            f"{p['rows_same_selection']:.1%} / {p['rows_exact_rule']:.1%} | "
            f"{p['out_max_abs']:.2e} / {p['out_mean_abs']:.2e} |")
    log("\n".join(lines))
    if args.table_out:
        with open(args.table_out, "w") as fh:
            fh.write("\n".join(lines) + "\n")


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
    ap.add_argument("--no-calib", action="store_true")
    ap.add_argument("--no-k32", action="store_true",
                    help="skip the top-k 32 record of the 1000-view workload")
    ap.add_argument("--table", action="store_true",
                    help="run every configuration of the workload list and print a table")
    ap.add_argument("--table-out", default=None)
    ap.add_argument("--cmp-mode", default="auto", choices=["auto", "two_pass", "single"],
                    help="compression branch: automatic (the single pass where it applies), "
                         "the two exact passes, or the single pass")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run the library's streaming copy over MIB MiB (the reference "
                         "kernel for scaling HBM byte counters) and exit")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the attention shards by head; see the design notes). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        S.calib_copy(src, dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n}))
        return
    if args.table:
        run_table(args, dev)
        return

    w = W.WORKLOADS[args.workload]
    log(f"[bench] workload {w.name}: T={w.T} H={w.H} B={w.block} k={w.topk} F={w.forced} "
        f"own={w.own}")
    ceil = None if args.no_calib else calibrate(dev)
    if ceil:
        log(f"[bench] measured ceilings: copy {ceil['hbm_copy_GBps']:.0f} GB/s, bf16 MFMA loop "
            f"{ceil['mfma_bf16_TFLOPs']:.0f} TFLOP/s")
    x = W.make_inputs(w, device=dev)
    torch.cuda.synchronize()
    T, H, D = x["q"].shape
    mode = {"auto": S.CMP_AUTO, "two_pass": S.CMP_TWO_PASS, "single": S.CMP_SINGLE}[args.cmp_mode]
    fwd = Forward(w, x, w.topk, mode, dev)
    single, Nb, layout = fwd.single, fwd.Nb, fwd.layout
    ms, wall = fwd.time(args.steps, args.warmup)
    log(f"[bench] sparse forward {ms:.3f} ms/step (wall {wall:.3f}), "
        f"compression {'single pass' if single else 'two passes'}")
    fwd.free()
    reps = max(1, min(3, args.steps))
    two_pass = None
    if single and not layout:
        # the same step with the two exact passes, for comparison (not the reported value)
        f2 = Forward(w, x, w.topk, S.CMP_TWO_PASS, dev)
        ms2, _ = f2.time(reps, 1)
        two_pass = {"ms_per_step": ms2, "value": T / (ms2 * 1e-3)}
        log(f"[bench] the same step with the two exact passes: {ms2:.3f} ms")
        f2.free()
        del f2

    # per-kernel durations: the same kernels launched stage by stage
    folds = w.block <= 64 and min(w.topk, Nb - min(w.forced, Nb)) <= 64
    xs, perm_ms = x, None
    if layout:
        # window order once; the reordering (3 tensors in, 1 out) is timed on its own
        xs = {n: S.window_permute(layout, x[n]) for n in ("q", "k", "v")}
        xs["gates"] = x["gates"]
        tmp = torch.empty_like(fwd.out)
        p0, p1 = events(2)
        torch.cuda.synchronize()
        p0.record()
        for n in ("q", "k", "v"):
            S.window_permute(layout, x[n], dst=tmp)
        S.window_permute(layout, xs["q"], dst=tmp, inverse=True)
        p1.record()
        torch.cuda.synchronize()
        perm_ms = p0.elapsed_time(p1)
        del tmp
    kernels, redone = stage_kernels(w, xs, w.topk, reps, single, ceil, T, Nb)
    if perm_ms is not None:
        kernels["window_permute"] = rate("window_permute", perm_ms,
                                         {"bytes": 4 * 2 * T * H * D * 2, "bound": "hbm"}, ceil)
    log("[bench] stages (ms): " + ", ".join(f"{k} {v['ms']:.3f}" for k, v in kernels.items()))
    if folds and not layout:
        # the separate top-k kernel (the path for B = 128 or more than 64 chosen blocks) on this
        # workload's score matrix: reported beside the step, not part of it
        st = S.Stages(xs["q"], xs["k"], xs["v"], xs["gates"], w.block, w.topk, keep_o_sel=False,
                      keep_score=True, forced_blocks=w.forced, force_own=w.own)
        st.run_pool()
        st.run_lse()
        st.run_fused()
        st.run_topk()
        t0, t1 = events(2)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(reps):
            st.run_topk()
        t1.record()
        torch.cuda.synchronize()
        kernels["topk_separate"] = rate("topk", t0.elapsed_time(t1) / reps,
                                        work_of(w, T, Nb, w.topk)["topk"], ceil)
        kernels["topk_separate"]["note"] = ("separate top-k kernel on the score matrix; not in "
                                            "the step, where top-k runs inside pass 2")
        log(f"[bench] separate top-k on the score matrix {kernels['topk_separate']['ms']:.3f} ms")
        del st
        torch.cuda.empty_cache()
    roof = roofline_of(kernels, single, w, folds)
    if xs is not x:
        del xs
        torch.cuda.empty_cache()

    # top-k 32 at the same shape (the 1000-view configuration asks for k = 16 and k = 32)
    k32 = None
    if w.name == "v1000_k16" and not args.no_k32:
        f32 = Forward(w, x, 32, mode, dev)
        ms32, _ = f32.time(reps, 1)
        kern32, redone32 = stage_kernels(w, x, 32, reps, f32.single, ceil, T, Nb)
        k32 = {"topk": 32, "ms_per_step": ms32, "value": T / (ms32 * 1e-3),
               "compression": "single pass" if f32.single else "two passes",
               "roofline": roofline_of(kern32, f32.single, dataclass_k(w, 32), True),
               "kernels": kern32, "single_pass_waves_redone": redone32}
        log(f"[bench] top-k 32: {ms32:.3f} ms/step ({T / (ms32 * 1e-3):.3e} tokens/s)")
        if not args.no_cpu:
            _, k32["parity_sampled"] = cpu_leg(w, x, 32, f32.sel, f32.out, (0, 15), 32, 1,
                                               seed=11)
            log(f"[bench] top-k 32 parity {k32['parity_sampled']}")
        f32.free()
        del f32

    backward = None
    if not args.no_backward and not layout:
        backward = time_backward(w, x, reps)
        log(f"[bench] training forward {backward['fwd_train_ms']:.1f} ms, backward "
            f"{backward['ms']:.1f} ms ({backward['achieved']:.0f} TFLOP/s algorithmic)")
        torch.cuda.empty_cache()

    dense = None
    if not args.no_dense:
        dense_ms = time_dense(x, fwd.p, dev, args.dense_reps)
        dk = rate("dense", dense_ms, work_of(w, T, Nb, w.topk)["dense"], ceil)
        dense = {"ms": dense_ms, "tflops": dk["achieved"], "frac": dk["frac"],
                 "frac_executed": dk["frac_executed"]}
        log(f"[bench] dense {dense_ms:.1f} ms ({dense['tflops']:.0f} TFLOP/s)")

    cpu, parity = None, None
    if not args.no_cpu:
        cpu, parity = cpu_leg(w, x, w.topk, fwd.sel, fwd.out, (0, 5, 10, 15), 64, 8)
        log(f"[bench] cpu oracle {cpu['value']:.1f} tokens/s on {cpu['cores']} threads, "
            f"{cpu['one_thread']['value']:.1f} on one; parity {parity}")

    rec = {
        "metric": METRIC, "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16"
        if w.dtype == "bf16" else "fp16",
        "data": "synthetic (seeded structured q/k/v, generated on the GPU)",
        "config": {**w.describe(), "parallelism": "none (1 GPU)",
                   "compression": "single pass" if single else "two passes"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "ceilings_measured": ceil,
        "kernels": kernels,
        "single_pass_waves_redone": redone,
        "two_pass": two_pass,
        "topk32": k32,
        "backward": backward,
        "dense": dense,
        "x_vs_dense": (dense["ms"] / ms) if dense else None,
        "parity_sampled": parity,
    }
    print(json.dumps(rec), flush=True)


def dataclass_k(w, topk):
    import dataclasses
    return dataclasses.replace(w, name=f"{w.name[:-4]}_k{topk}" if w.name.endswith("_k16")
                               else w.name, topk=topk)


if __name__ == "__main__":
    main()
