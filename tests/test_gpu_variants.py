"""GPU parity of the selection variants of hs2_select_ex against the oracle:
the output-aware metric (oam_beta > 0: key j's group score weighted by
max(1, |v_j|_2)^beta) in token mode (sampled threshold and the exact path) and
block mode, and the position-decaying budget (decay_mu: top_k at a sequence's
first position down to floor(mu top_k + 0.5) at its last), alone and with the
metric. V rows are rescaled so their norms straddle 1 and the weights change
selections."""
import numpy as np
import pytest

import synthgen
from hs2_testlib import A1_TOL, A2_MIN, GpuCase, check_structure, local_t, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_level_sparse_hs2_amd as hs2
    hs2.load_library()


def weighted_inputs(w):
    inp = synthgen.make_inputs(w)
    T = w.total
    f = np.exp(synthgen.normal_f64(w.seed, 51, T * w.Hkv)).reshape(T, w.Hkv, 1) * 0.1
    inp["v"] = synthgen.float_to_bf16(synthgen.bf16_to_float(inp["v"]).astype(np.float64) * f)
    return inp


def run_variant(w, beta=0.0, mu=0.0, flags=0, block=0):
    import oracle
    import torch
    import token_level_sparse_hs2_amd as hs2
    log(f"variant {w.name}: lengths={w.lengths[:8]} Hq={w.Hq} Hkv={w.Hkv} K={w.K} W={w.W} "
        f"beta={beta} mu={mu} flags={flags}")
    inp = weighted_inputs(w)
    case = GpuCase(w, inp, flags=flags)
    idx_t = case.new_idx()
    kth_t = case.guarded_empty((case.T, w.Hkv), torch.float32)
    hs2.hs2_select_ex(case.dims, case.varlen, case.q_full, case.k, idx_t, kth_t, v=case.v,
                      oam_beta=beta, decay_mu=mu, workspace=case.workspace)
    case.check_guards()
    idx = idx_t.cpu().numpy()
    cu = inp["cu_seqlens"]
    o_idx, o_kth = oracle.select(inp["q_full"], inp["k"], cu, w.Hq, w.Hkv, w.K, w.W,
                                 scale=w.scale, block=block, v=inp["v"], oam_beta=beta,
                                 decay_mu=mu)
    tl = local_t(cu, np.arange(w.total))
    n_c = np.maximum(0, tl - w.W + 1)
    o3 = o_idx.reshape(w.total, w.Hkv, -1)
    o_glob = ((o3 >= 0) & (o3 < n_c[:, None, None])).sum(axis=2)  # min(n_c, K_t) per row
    if not block:
        check_structure(idx, cu, w.K, w.W, n_glob=o_glob)  # budgets bit-exact
    plain, _ = oracle.select(inp["q_full"], inp["k"], cu, w.Hq, w.Hkv, w.K, w.W, scale=w.scale,
                             block=block)
    wv = np.maximum(1.0, np.linalg.norm(synthgen.bf16_to_float(inp["v"]).astype(np.float64),
                                        axis=2)) ** beta
    g_rows = idx.reshape(-1, w.K + w.W)
    inter = tot = same = 0
    worst = np.inf
    for r in range(len(g_rows)):
        a, b = g_rows[r][g_rows[r] >= 0], o_idx[r][o_idx[r] >= 0]
        inter += len(np.intersect1d(a, b))
        tot += len(b)
        if len(a) == len(b) and (a == b).all():
            same += 1
            continue
        tg, g = divmod(r, w.Hkv)
        i = int(np.searchsorted(cu, tg, side="right") - 1)
        nc = int(n_c[tg])
        S, _, _ = oracle.group_scores(inp["q_full"], inp["k"], cu, w.Hq, w.Hkv, tg, g, scale=w.scale)
        Sw = S[:nc] * wv[int(cu[i]):int(cu[i]) + nc, g]
        glob = a[a < nc]
        if block:
            vals = [Sw[bb * block:(bb + 1) * block].sum() for bb in set((glob // block).tolist())]
        else:
            vals = Sw[glob]
        if len(glob):
            worst = min(worst, min(vals) - o_kth[r])
    changed = (plain != o_idx).any(axis=1).mean()
    overlap = inter / max(1, tot)
    log(f"  rows {len(g_rows)} identical {same} overlap {overlap:.6f} A1 margin {worst:.3g} "
        f"rows changed by the variant {changed:.3f}")
    assert changed > 0.05
    assert overlap >= A2_MIN and worst >= -A1_TOL
    kth = kth_t.cpu().numpy().reshape(-1)
    sel = o_kth > 0
    assert ((kth < 0) == ~sel).all()
    rel = np.abs(kth[sel] - o_kth[sel]) / o_kth[sel]
    log(f"  kth relative diff: max {rel.max():.3g}")
    assert rel.max() <= 1e-3


@pytest.mark.parametrize("G", [1, 4, 16])
def test_oam_token_selection(G):
    w = synthgen.custom([1, 33, 700, 2100, 4500], Hq=2 * G, Hkv=2, K=256, W=32, n_sparse=1,
                        seed=100 + G)
    run_variant(w, beta=0.7)


def test_oam_exact_path():
    import token_level_sparse_hs2_amd as hs2
    w = synthgen.custom([300, 5000], Hq=8, Hkv=2, K=256, W=32, n_sparse=1, seed=110)
    run_variant(w, beta=0.7, flags=hs2.HS2_FLAG_EXACT_SELECT)


def test_oam_block_selection():
    import token_level_sparse_hs2_amd as hs2
    w = synthgen.custom([1, 700, 4500], Hq=8, Hkv=2, K=256, W=32, n_sparse=1, seed=111)
    run_variant(w, beta=0.7, flags=hs2.HS2_FLAG_BLOCK_SELECT, block=64)


@pytest.mark.parametrize("G,mu", [(1, 0.5), (4, 0.25), (8, 0.5), (16, 0.75)])
def test_position_decay(G, mu):
    w = synthgen.custom([1, 33, 700, 2100, 4500], Hq=2 * G, Hkv=2, K=256, W=32, n_sparse=1,
                        seed=120 + G)
    run_variant(w, mu=mu)


def test_position_decay_with_oam_and_exact_path():
    import token_level_sparse_hs2_amd as hs2
    w = synthgen.custom([700, 5000], Hq=8, Hkv=2, K=256, W=32, n_sparse=1, seed=130)
    run_variant(w, beta=0.7, mu=0.5)
    run_variant(w, mu=0.5, flags=hs2.HS2_FLAG_EXACT_SELECT)


def test_position_decay_long_rows_sampled_threshold():
    """A long sequence (rows past the candidate cap take the sampled threshold) at
    the full-size budget."""
    w = synthgen.custom([12000], Hq=8, Hkv=2, K=1024, W=128, n_sparse=1, seed=131)
    run_variant(w, mu=0.5)
