"""GPU parity of 64-token block selection (HS2_FLAG_BLOCK_SELECT) against the
oracle's block mode: structure (the global part is whole candidate blocks,
K/64 of them), rows equal to the oracle's except where two block scores tie
within fp32 resolution (then the GPU's block scores within 1e-5 of the K/64-th),
and the sparse layer on the GPU's rows (A4)."""
import numpy as np
import pytest

import synthgen
from hs2_testlib import A4_TOL, GpuCase, log, sample_tokens

pytestmark = pytest.mark.gpu
BS = 64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_level_sparse_hs2_amd as hs2
    hs2.load_library()


def check_block_row(row, t, K, W):
    n_c = max(0, t - W + 1)
    got = row[row >= 0]
    assert (np.diff(got) > 0).all() and (got <= t).all() and (row[len(got):] == -1).all()
    window = np.arange(max(0, t - W + 1), t + 1)
    assert np.array_equal(got[len(got) - len(window):], window)
    glob = got[got < n_c]
    if n_c <= K:
        assert np.array_equal(glob, np.arange(n_c))
        return set()
    blocks = set((glob // BS).tolist())
    assert len(blocks) == K // BS
    for b in blocks:
        assert np.array_equal(glob[glob // BS == b], np.arange(b * BS, min((b + 1) * BS, n_c)))
    return blocks


def run_blocks(w, tokens=None):
    import oracle
    import token_level_sparse_hs2_amd as hs2
    log(f"blocks {w.name}: lengths={w.lengths[:8]} Hq={w.Hq} Hkv={w.Hkv} K={w.K} W={w.W}")
    inp = synthgen.make_inputs(w)
    case = GpuCase(w, inp, flags=hs2.HS2_FLAG_BLOCK_SELECT)
    idx_t, kth_t = case.select()
    idx, kth = idx_t.cpu().numpy(), kth_t.cpu().numpy().reshape(-1)
    cu = inp["cu_seqlens"]
    T = case.T
    toks = np.arange(T) if tokens is None else tokens
    rows = (toks[:, None] * w.Hkv + np.arange(w.Hkv)[None, :]).ravel()
    o_idx, o_kth = oracle.select(inp["q_full"], inp["k"], cu, w.Hq, w.Hkv, w.K, w.W,
                                 scale=w.scale, rows=rows, block=BS)
    g_rows = idx.reshape(T * w.Hkv, -1)[rows]
    same = worst = 0
    worst = np.inf
    for r, row_id in enumerate(rows):
        tg, g = divmod(int(row_id), w.Hkv)
        t = int(tg - cu[np.searchsorted(cu, tg, side="right") - 1])
        blocks = check_block_row(g_rows[r], t, w.K, w.W)
        if np.array_equal(g_rows[r], o_idx[r]):
            same += 1
            continue
        S, _, _ = oracle.group_scores(inp["q_full"], inp["k"], cu, w.Hq, w.Hkv, tg, g,
                                      scale=w.scale)
        n_c = t - w.W + 1
        score = [S[b * BS:min((b + 1) * BS, n_c)].sum() for b in blocks]
        worst = min(worst, min(score) - o_kth[r])
    log(f"  rows {len(rows)} identical {same} worst block margin {worst:.3g}")
    assert same >= 0.999 * len(rows) and worst >= -1e-5
    sel = o_kth > 0
    if sel.any():
        rel = np.abs(kth[rows][sel] - o_kth[sel]) / o_kth[sel]
        log(f"  kth relative diff: max {rel.max():.3g}")
        assert rel.max() <= 1e-3
    out32 = case.sparse(case.q_sparse[0], idx_t, precise=True).cpu().numpy()
    o64, _ = oracle.sparse_attn(inp["q_sparse"][0], inp["k"], inp["v"], cu, w.Hq, w.Hkv, idx,
                                scale=w.scale, tokens=toks, want_bf16=False)
    err = np.abs(out32[toks] - o64).max()
    log(f"  sparse A4 max-abs {err:.3g}")
    assert err <= A4_TOL


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_block_selection_ragged_every_group_size(G):
    w = synthgen.custom([1, 33, 128, 129, 700, 2100, 4500], Hq=2 * G, Hkv=2, K=256, W=32,
                        n_sparse=1, seed=80 + G)
    run_blocks(w)


def test_block_selection_8k_sampled():
    w = synthgen.workload("8k")
    run_blocks(w, tokens=sample_tokens(w.lengths, w.K, w.W, head=64, tail=16, stride=97))
