"""GPU parity of the selection stage on hand-made selection rows, at every block size: -1
padding, entries past the last block or negative, a block repeated right after itself (or
after invalid entries only), empty rows, and rows longer than 64 entries (which the B >= 64
kernel walks in 64-entry chunks instead of scheduling one tile step per lane).

Speed3R technical summary (gist.science), "Methodologie" section 1: the selection branch
attends to the tokens of the chosen key blocks. The oracle takes the union of a row's valid
entries; the kernels drop an entry equal to the last block they took. The rows below repeat a
block only where the two rules agree (no other valid block in between)."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_global_attention_block_amd import speed3r as S
from sparse_global_attention_block_amd import workloads as W
from tests.helpers import check_out, cuda_inputs, host

pytestmark = pytest.mark.gpu

# name: (block, entries per row, T)
CASES = {
    "b64_short": (64, 12, 64 * 40 + 5),    # 24 tile steps: one step per lane
    "b64_long": (64, 70, 64 * 100 + 17),   # two 64-entry chunks, walked
    "b128_short": (128, 9, 128 * 30),      # 36 steps: one step per lane
    "b128_long": (128, 20, 128 * 50 + 3),  # 80 steps: walked
    "b32": (32, 20, 32 * 80 + 7),
    "b16": (16, 24, 16 * 90 + 9),
}
BAD = (-5, -1, 2**31 - 1)  # plus Nb and Nb + 7, per case


def make_rows(rng, H, Nb, k_eff):
    bad = list(BAD) + [Nb, Nb + 7]
    rows = np.full((H, Nb, k_eff), -1, np.int32)
    for h in range(H):
        for i in range(Nb):
            if rng.random() < 0.05:
                continue  # an empty row
            m = int(rng.integers(1, min(k_eff, Nb) + 1))
            seq = []
            for b in rng.choice(Nb, size=m, replace=False):
                seq.append(int(b))
                r = rng.random()
                if r < 0.15:
                    seq.append(int(b))  # repeated right away
                elif r < 0.25:
                    seq += [int(bad[rng.integers(len(bad))]), int(b)]  # after an invalid one
                elif r < 0.35:
                    seq.append(int(bad[rng.integers(len(bad))]))
            seq = seq[:k_eff]
            rows[h, i, :len(seq)] = seq
    return rows


@pytest.mark.parametrize("name", list(CASES))
def test_selection_rows_with_padding_repeats_and_invalid_entries(name):
    block, k_eff, T = CASES[name]
    w = dataclasses.replace(W.WORKLOADS["tiny_s"], name=name, H=2, block=block, topk=k_eff)
    print(f"[sel rows {name}] T={T} B={block} entries={k_eff}", flush=True)
    x = cuda_inputs(w, T=T)
    st = S.Stages(x["q"], x["k"], x["v"], x["gates"], block, k_eff)
    assert st.k_eff == k_eff
    Nb, H = st.Nb, w.H
    rng = np.random.default_rng(7 + block + k_eff)
    rows = make_rows(rng, H, Nb, k_eff)
    ocmp = torch.from_numpy(rng.standard_normal((T, H, 64)).astype(np.float32)).cuda()
    st.run_pool()
    st.run_sel(sel=torch.from_numpy(rows).cuda(), o_cmp=ocmp)
    torch.cuda.synchronize()
    hx = {n: host(t) for n, t in x.items()}
    g = host(x["gates"]).double().numpy()
    # rows checked: the first and last query block of each head and a random sample
    pick = sorted({(h, i) for h in range(H) for i in (0, Nb - 1)} |
                  {(int(rng.integers(H)), int(rng.integers(Nb))) for _ in range(40)})
    osel_g, osel_r, out_g, out_r = [], [], [], []
    for h, i in pick:
        ref = O.sel_row(hx["q"], hx["k"], hx["v"], block, h, i, rows[h, i])
        n = ref.shape[0]
        t = slice(i * block, i * block + n)
        osel_g.append(st.o_sel[t, h])
        osel_r.append(ref)
        gh = g[t, h] if g.ndim == 3 else np.broadcast_to(g[h], (n, 2))
        out_g.append(st.out[t, h])
        out_r.append(gh[:, :1] * host(ocmp[t, h]).double().numpy() + gh[:, 1:] * ref)
    mx, mean = check_out(torch.cat(osel_g), np.concatenate(osel_r), what="O_sel")
    print(f"[sel rows {name}] {len(pick)} rows: O_sel max-abs {mx:.3e} mean-abs {mean:.3e}")
    check_out(torch.cat(out_g), np.concatenate(out_r))
