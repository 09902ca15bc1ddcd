"""The separate top-k kernel on score rows longer than one 1024-entry chunk (its streaming
loops) and up to the 21,469 key blocks of the 1000-view workload, compared bit for bit with
the oracle's top-k on every row.

The kernel serves every configuration that does not fold the selection into the compression
pass (block 128, or more than 64 chosen blocks). Rows here are synthetic score rows, several
patterns per matrix: random values, three levels (ties far beyond the kernel's candidate
buffer: its exact fallback), all equal (fallback), ties planted at the k-th value (few
candidates, tie-break by index), the largest values all owned by one thread of the work-group
(its re-read), mixed signs with +0 and -0, and a single huge entry. Each matrix runs with no
forced blocks and with a forced prefix of 22 blocks plus each row's own block.
"""
import concurrent.futures as cf

import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_global_attention_block_amd import speed3r as S

pytestmark = pytest.mark.gpu

PATTERNS = ("random", "levels3", "all_equal", "planted_ties", "one_thread", "signs", "spike")


def score_rows(Nb: int, ld: int, n_rows: int, k: int, seed: int) -> np.ndarray:
    """[n_rows, ld] float32, row r of pattern PATTERNS[r % 7], padding columns 0."""
    rng = np.random.default_rng(seed)
    m = np.zeros((n_rows, ld), np.float32)
    m[:, :Nb] = rng.random((n_rows, Nb), dtype=np.float32) * 1e-2
    for r in range(n_rows):
        pat = PATTERNS[r % len(PATTERNS)]
        row = m[r, :Nb]
        if pat == "levels3":
            row[:] = np.floor(rng.random(Nb) * 3).astype(np.float32) / 3
        elif pat == "all_equal":
            row[:] = np.float32(0.25)
        elif pat == "planted_ties":
            kth = np.sort(row)[::-1][k - 1]
            row[rng.choice(Nb, 5, replace=False)] = kth
        elif pat == "one_thread":
            # entries 1024c + 0..3 belong to thread 0 of the work-group
            own = np.concatenate([np.arange(c * 1024, min(Nb, c * 1024 + 4))
                                  for c in range((Nb + 1023) // 1024)])
            row[own[: 2 * k]] = 1.0 + rng.random(min(len(own), 2 * k), dtype=np.float32)
        elif pat == "signs":
            row[:] = rng.standard_normal(Nb).astype(np.float32)
            row[rng.choice(Nb, 40, replace=False)] = 0.0
            row[rng.choice(Nb, 40, replace=False)] = -0.0
        elif pat == "spike":
            row[rng.integers(Nb)] = 1e30
    return m


def expected_row(row: np.ndarray, i: int, k: int, F: int, own: bool, n_sel: int) -> np.ndarray:
    """Forced prefix, the own block (row i, when past the prefix), then the oracle's top-k of
    the remaining blocks; ascending, -1 padded."""
    Nb = row.size
    keep = list(range(min(F, Nb)))
    cand = np.arange(min(F, Nb), Nb)
    if own and i >= F:
        keep.append(i)
        cand = cand[cand != i]
    if cand.size:
        keep += list(cand[O.topk(row[cand], k)])
    want = np.full(n_sel, -1, np.int32)
    want[:len(keep)] = np.sort(keep)
    return want


@pytest.mark.parametrize("Nb,k", [(1025, 16), (4100, 80), (21469, 16)])
@pytest.mark.parametrize("F,own", [(0, False), (22, True)])
def test_topk_long_rows_bit_exact(Nb, k, F, own):
    H = 1
    T = Nb * 64
    p = S.Params(T, H, 64, 64, k, 0.0, F, H * 64, 64, H * 64, 64, H * 64, 64, 0, 0, int(own),
                 S.CMP_TWO_PASS)
    ld, n_sel = S.score_row_stride(p), S.num_selected(p)
    assert S.num_blocks(p) == Nb and ld >= Nb
    print(f"[topk long] Nb={Nb} k={k} F={F} own={own} rows={H * Nb} ld={ld} n_sel={n_sel}",
          flush=True)
    rows = score_rows(Nb, ld, H * Nb, k, seed=Nb + F)
    score = torch.from_numpy(rows).cuda()
    sel = torch.full((H, Nb, n_sel), -7, dtype=torch.int32, device="cuda")
    S.topk(p, score, sel)
    torch.cuda.synchronize()
    got = sel.cpu().numpy().reshape(H * Nb, n_sel)
    del score, sel
    torch.cuda.empty_cache()

    def check(r):
        want = expected_row(rows[r, :Nb], r % Nb, k, F, own, n_sel)
        return None if np.array_equal(got[r], want) else (r, got[r], want)

    # the oracle's top-k releases the GIL: rows are checked in parallel on the host
    with cf.ThreadPoolExecutor(max_workers=16) as ex:
        bad = [b for b in ex.map(check, range(H * Nb), chunksize=64) if b is not None]
    print(f"[topk long] Nb={Nb}: {H * Nb} rows checked, {len(bad)} differ", flush=True)
    assert not bad, f"{len(bad)} rows differ; first: row {bad[0][0]} ({PATTERNS[bad[0][0] % 7]})" \
                    f" GPU {bad[0][1]} oracle {bad[0][2]}"
