"""Address and undefined-behaviour sanitizer builds of the host code, on the CPU.

1. The C oracle, built with gcc -fsanitize=address,undefined, runs every entry point on small
   problems (ragged last blocks, forced and own blocks, a given selection, the backward pass)
   in a child process that preloads gcc's sanitizer runtimes.
2. The library's host half (argument validation, sizes, workspace layout, the entry points'
   rejection paths), built with the sanitizers on the host side only (device code is compiled
   as usual), runs the same calls the ABI tests make, in a child process that preloads the
   compiler's address-sanitizer runtime. No GPU is touched: every call returns from
   validation or from a size query.

Any sanitizer report aborts the child (halt_on_error, no recovery) and fails the test.
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV_SAN = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _child(script: str, preload: str, tmp) -> subprocess.CompletedProcess:
    path = os.path.join(tmp, "child.py")
    with open(path, "w") as f:
        f.write(textwrap.dedent(script))
    env = dict(os.environ, LD_PRELOAD=preload, PYTHONPATH=ROOT, **ENV_SAN)
    return subprocess.run([sys.executable, path], capture_output=True, text=True, env=env,
                          timeout=600, cwd=ROOT)


ORACLE_CHILD = r"""
import sys
sys.modules["torch"] = None          # keep torch (not instrumented) out of this process
import numpy as np
from oracle import oracle as O
O._LIB = "{lib}"
rng = np.random.default_rng(0)
T, H, D, B = 203, 2, 64, 16
q, k, v = (rng.standard_normal((T, H, D)).astype(np.float32) for _ in range(3))
g = rng.random((H, 2)).astype(np.float32)
kc, vc = O.pool(k, B), O.pool(v, B)
O.cmp_row(q, kc, vc, B, 1, 12)
O.topk(rng.random(50).astype(np.float32), 7)
O.topk(np.zeros(5, np.float32), 9)
O.sel_row(q, k, v, B, 0, 3, [0, 3, 3, 12])
O.dense_rows(q, k, v, 1, 190, 13)
Nb = O.n_blocks(T, B)
for forced, own in ((0, False), (3, True), (Nb + 2, False)):
    r = O.forward_rows(q, k, v, g, B, 4, [0, 1, 1], [0, 5, Nb - 1], forced=forced, own=own)
    O.forward_rows(q, k, v, g, B, 4, [0, 1, 1], [0, 5, Nb - 1], sel_in=r["sel"],
                   forced=forced, own=own)
gt = rng.random((T, H, 2)).astype(np.float32)
full = O.forward_all(q, k, v, gt, B, 5)
dout = rng.standard_normal((T, H, D)).astype(np.float32)
O.backward(q, k, v, gt, dout, B, full["sel"])
O.set_num_threads(1)
O.forward_rows(q, k, v, g, B, 4, [1], [2])
print("oracle ok")
"""

ABI_CHILD = r"""
import ctypes
L = ctypes.CDLL("{lib}")

class Params(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
                ("block", ctypes.c_int32), ("topk", ctypes.c_int32), ("scale", ctypes.c_float),
                ("forced_blocks", ctypes.c_int32), ("q_stride_t", ctypes.c_int64),
                ("q_stride_h", ctypes.c_int64), ("k_stride_t", ctypes.c_int64),
                ("k_stride_h", ctypes.c_int64), ("v_stride_t", ctypes.c_int64),
                ("v_stride_h", ctypes.c_int64), ("gate_stride_t", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("force_own", ctypes.c_int32),
                ("cmp_mode", ctypes.c_int32)]

class Windows(ctypes.Structure):
    _fields_ = [("views", ctypes.c_int64), ("special", ctypes.c_int32), ("grid_h", ctypes.c_int32),
                ("grid_w", ctypes.c_int32), ("win_h", ctypes.c_int32), ("win_w", ctypes.c_int32)]

def P(T=1024, H=4, D=64, B=16, k=8, forced=0, own=0, mode=0, scale=0.0, st=None, dtype=0):
    st = st or (H * D, D)
    return Params(T, H, D, B, k, scale, forced, st[0], st[1], st[0], st[1], st[0], st[1], 0,
                  dtype, own, mode)

for fn in ("speed3r_workspace_size", "speed3r_tiles_workspace_size", "speed3r_dense_workspace_size",
           "speed3r_train_workspace_size", "speed3r_bwd_workspace_size"):
    getattr(L, fn).restype = ctypes.c_size_t
for fn in ("speed3r_num_blocks", "speed3r_num_selected", "speed3r_score_row_stride",
           "speed3r_redo_flag_count"):
    getattr(L, fn).restype = ctypes.c_int64
L.speed3r_status_string.restype = ctypes.c_char_p
FAKE = ctypes.c_void_p(1 << 20)
sizes = 0
cases = [P(), P(T=1), P(T=17, B=16, k=1), P(T=1374000, H=16, B=64, k=16),
         P(T=1374000, H=16, B=64, k=33, forced=22, own=1), P(T=4096, B=128, k=4),
         P(T=100 * 64, B=64, k=65), P(T=1000, B=32, k=5, forced=3, own=1, mode=2),
         P(dtype=1), P(k=0), P(D=32), P(B=48), P(T=0), P(scale=-1.0), P(st=(4 * 64 + 4, 64)),
         P(T=25079 * 128, H=16, B=128, k=16), P(forced=-1), P(mode=7), P(H=70000)]
for p in cases:
    for fn in ("speed3r_workspace_size", "speed3r_tiles_workspace_size",
               "speed3r_dense_workspace_size", "speed3r_train_workspace_size",
               "speed3r_bwd_workspace_size", "speed3r_num_blocks", "speed3r_num_selected",
               "speed3r_score_row_stride", "speed3r_redo_flag_count"):
        sizes += getattr(L, fn)(ctypes.byref(p))
    # rejection paths: null and misaligned pointers, short workspaces
    ws = ctypes.c_void_p(1 << 20)
    L.speed3r_sparse_attn_fwd(ctypes.byref(p), None, FAKE, FAKE, FAKE, FAKE, None, ws,
                              ctypes.c_size_t(1 << 40), None)
    L.speed3r_sparse_attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, ws,
                              ctypes.c_size_t(1), None)
    L.speed3r_sparse_attn_fwd_train(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, ws,
                                    ctypes.c_size_t(1), None)
    L.speed3r_sparse_attn_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None,
                              ctypes.c_int64(256), ctypes.c_int64(64), ws, ctypes.c_size_t(1),
                              FAKE, FAKE, FAKE, FAKE, ws, ctypes.c_size_t(1), None)
    L.speed3r_topk(ctypes.byref(p), None, FAKE, None)
    L.speed3r_sel_combine(ctypes.byref(p), FAKE, ws, ctypes.c_size_t(1), FAKE, FAKE, FAKE, FAKE,
                          None, None)
    L.speed3r_dense_attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, ws, ctypes.c_size_t(1),
                             None)
    L.speed3r_sparse_attn_fwd_noalloc(ctypes.byref(p), None, FAKE, FAKE, FAKE, FAKE, None, None)
L.speed3r_sparse_attn_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, ctypes.c_size_t(1), None)
for code in range(-1, 8):
    L.speed3r_status_string(code)
for w in (Windows(2, 5, 4, 4, 2, 2), Windows(0, 5, 4, 4, 2, 2), Windows(2, 5, 4, 4, 3, 2),
          Windows(1 << 40, 5, 37, 37, 1, 1)):
    for pos in (-1, 0, 5, 36, 1 << 50):
        L.speed3r_window_source(ctypes.byref(w), ctypes.c_int64(pos))
    L.speed3r_windows_workspace_size.restype = ctypes.c_size_t
    L.speed3r_windows_workspace_size(ctypes.byref(P(T=42)), ctypes.byref(w))
L.speed3r_calib_copy(None, FAKE, ctypes.c_size_t(16), None)
L.speed3r_calib_mfma_flops.restype = ctypes.c_int64
L.speed3r_calib_mfma_flops(0, 5)
print("abi ok", sizes)
"""


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    lib = os.path.join(tmp_path, "liboracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-omit-frame-pointer", "-o", lib,
                           os.path.join(ROOT, "oracle", "speed3r_oracle.c"), "-lm"])
    pre = " ".join(subprocess.check_output(["gcc", f"-print-file-name={n}"], text=True).strip()
                   for n in ("libasan.so", "libubsan.so"))
    r = _child(ORACLE_CHILD.replace("{lib}", lib), pre, str(tmp_path))
    assert r.returncode == 0 and "oracle ok" in r.stdout, r.stdout[-3000:] + r.stderr[-6000:]


def test_abi_host_layer_under_address_and_ub_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("the compiler's address-sanitizer runtime was not found")
    csrc = os.path.join(ROOT, "sparse_global_attention_block_amd", "csrc")
    srcs = sorted(glob.glob(os.path.join(csrc, "*.hip")))
    objs = [os.path.join(tmp_path, os.path.basename(src) + ".o") for src in srcs]

    def compile_one(src, obj):
        # sanitizers on the host side only: each -fsanitize= follows -Xarch_host
        r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                            "-Xarch_host", "-fsanitize=address",
                            "-Xarch_host", "-fsanitize=undefined",
                            "-Xarch_host", "-fno-sanitize-recover=all",
                            "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(compile_one, srcs, objs))
    lib = os.path.join(tmp_path, "libspeed3r_san.so")
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
                           "-Xarch_host", "-fsanitize=address",
                           "-Xarch_host", "-fsanitize=undefined", "-o", lib, *objs])
    r = _child(ABI_CHILD.replace("{lib}", lib), rt[-1], str(tmp_path))
    assert r.returncode == 0 and "abi ok" in r.stdout, r.stdout[-3000:] + r.stderr[-6000:]
