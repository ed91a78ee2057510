"""Seeded random configurations through the whole path as hs2_prefill_block runs it
(selection, shared-gather plan or per-token layers, one to three sparse layers), each
checked against the CPU oracle on every row: group sizes 1 to 16, one to sixteen KV
groups, budgets from 0 past the register-ranked limit (2048; above it the rows are
ranked from their candidate lists when a sequence is longer than two lists, else by the
dense exact path), windows from 0, ragged packed lengths (up to 8 sequences, many
under 200 tokens, and one batch of 500 sequences), and the exact flag.

Per case: the index rows' structure and A1/A2 on all rows; A4 for every layer's fp32
output and A3 for its bf16 output, both on the GPU's own index rows; and the bf16 call
selects the same rows as the fp32 call (the selection does not depend on the output
mode or on scheduling). The same configurations drive the full layer's own output
(hs2_full_attn): A4 / A3 against the oracle's dense causal attention and the rows'
log2-domain log-sum-exp, on sampled tokens (every sequence's first and last tokens,
the tiles' edges and a stride).
"""
import numpy as np
import pytest

import synthgen
from hs2_testlib import (A3_TOL, A4_TOL, GpuCase, acceptance_select, assert_select_ok,
                         check_structure, from_dev_bf16, log, sample_tokens)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_level_sparse_hs2_amd as hs2
    hs2.load_library()  # the in-tree HIP library; nothing falls back to the CPU


def _configs(n=20, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.choice([1, 2, 4, 8, 16]))
        Hkv = int(rng.choice([1, 2, 3]))
        K = int(rng.choice([0, 1, 17, 128, 300, 1024, 1500, 2100, 2600]))
        W = int(rng.choice([0, 1, 7, 64, 128, 200]))
        if K + W == 0:
            W = 1
        B = int(rng.integers(1, 5))
        # long enough that large budgets still leave rows to rank
        hi = max(3500, K + W + 2000)
        lengths = [int(x) for x in rng.integers(1, hi, size=B)]
        n_sparse = int(rng.integers(1, 3))
        exact = bool(rng.random() < 0.2)
        out.append((i, G, Hkv, K, W, lengths, n_sparse, exact))
    return out


def _wide_configs(n=20, seed=77):
    """More KV groups (4, 5, 8, 16), up to 8 packed sequences, half of the cases
    with sequences under 200 tokens, budgets at the register-ranking edges."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.choice([1, 2, 4, 8, 16]))
        Hkv = int(rng.choice([4, 5, 8, 16])) if G <= 4 else int(rng.choice([4, 5, 8]))
        K = int(rng.choice([0, 1, 5, 64, 256, 1024, 2048, 2049]))
        W = int(rng.choice([0, 1, 3, 63, 64, 65, 128]))
        if K + W == 0:
            W = 1
        B = int(rng.integers(1, 9))
        if rng.random() < 0.5:
            lengths = [int(x) for x in rng.integers(1, 200, size=B)]
        else:
            lengths = [int(x) for x in rng.integers(1, max(3000, K + W + 1500), size=B)]
        n_sparse = int(rng.integers(1, 4))
        exact = bool(rng.random() < 0.25)
        out.append((1000 + i, G, Hkv, K, W, lengths, n_sparse, exact))
    return out


def _list_ranked_configs():
    """Budgets above the register-ranked limit with one sequence longer than two
    candidate lists (2 * 2K slots), so the rows are ranked from their lists."""
    rng = np.random.default_rng(31)
    out = []
    for i, K in enumerate((2049, 2500, 3000)):
        G = int(rng.choice([1, 4, 8]))
        Hkv = int(rng.choice([1, 2]))
        W = int(rng.choice([0, 64, 128]))
        C = (2 * K + 63) // 64 * 64
        lengths = [int(x) for x in rng.integers(1, 3000, size=2)] + [2 * C + 300 + 100 * i]
        out.append((3000 + i, G, Hkv, K, W, lengths, 2, False))
    return out


def _many_sequences():
    """500 packed sequences of 1-399 tokens (100k tokens)."""
    rng = np.random.default_rng(99)
    return [(2000, 4, 2, 64, 16, [int(x) for x in rng.integers(1, 400, size=500)], 2, False)]


@pytest.mark.parametrize("cfg", _configs() + _wide_configs() + _list_ranked_configs() +
                         _many_sequences(), ids=lambda c: f"case{c[0]}")
def test_random_configuration(cfg):
    import oracle
    import token_level_sparse_hs2_amd as hs2
    i, G, Hkv, K, W, lengths, n_sparse, exact = cfg
    w = synthgen.custom(lengths, Hq=G * Hkv, Hkv=Hkv, K=K, W=W, n_sparse=n_sparse,
                        seed=900 + i)
    log(f"random case {i}: lengths={lengths} G={G} Hkv={Hkv} K={K} W={W} "
        f"n_sparse={n_sparse} exact={exact}")
    inp = synthgen.make_inputs(w)
    case = GpuCase(w, inp, flags=hs2.HS2_FLAG_EXACT_SELECT if exact else 0)
    idx_t, outs32 = case.prefill_block(precise=True)
    idx = idx_t.cpu().numpy()
    cu = inp["cu_seqlens"]
    check_structure(idx, cu, K, W)
    stats = acceptance_select(idx, inp, w)
    log(f"  select: rows {stats['rows']} identical {stats['exact_rows']} overlap "
        f"{stats['overlap']:.6f} A1 margin {stats['a1_worst_margin']:.3g}")
    assert_select_ok(stats)
    idx16_t, outs16 = case.prefill_block(precise=False)
    assert (idx16_t.cpu().numpy() == idx).all(), "the bf16 call selected other rows"
    for l, qs_np in enumerate(inp["q_sparse"]):
        o64, o16 = oracle.sparse_attn(qs_np, inp["k"], inp["v"], cu, w.Hq, w.Hkv, idx,
                                      scale=w.scale)
        err4 = np.abs(outs32[l].cpu().numpy() - o64).max()
        g = synthgen.bf16_to_float(from_dev_bf16(outs16[l])).astype(np.float64)
        err3 = np.abs(g - synthgen.bf16_to_float(o16).astype(np.float64)).max()
        log(f"  layer {l}: A4 max-abs {err4:.3g} A3 max-abs {err3:.3g}")
        assert err4 <= A4_TOL and err3 <= A3_TOL
    case.release_guarded()


@pytest.mark.parametrize("cfg", _configs() + _wide_configs() + _many_sequences(),
                         ids=lambda c: f"case{c[0]}")
def test_random_full_output(cfg):
    import oracle
    import torch
    import token_level_sparse_hs2_amd as hs2
    i, G, Hkv, K, W, lengths, n_sparse, exact = cfg
    w = synthgen.custom(lengths, Hq=G * Hkv, Hkv=Hkv, K=K, W=W, n_sparse=n_sparse, seed=900 + i)
    log(f"random full case {i}: lengths={lengths} G={G} Hkv={Hkv}")
    inp = synthgen.make_inputs(w)
    case = GpuCase(w, inp)
    cu = inp["cu_seqlens"]
    T = case.T
    toks = sample_tokens(w.lengths, 64, 0, head=12, tail=12, stride=97)
    o64, o16 = oracle.full_attn(inp["q_full"], inp["k"], inp["v"], cu, w.Hq, w.Hkv,
                                scale=w.scale, tokens=toks)
    for precise in (True, False):
        out = case.guarded_empty((T, w.Hq, w.d), torch.float32 if precise else torch.bfloat16)
        lse2 = case.guarded_empty((T, w.Hq), torch.float32)
        hs2.hs2_full_attn(case.dims, case.varlen, case.q_full, case.k, case.v, out,
                          hs2.HS2_OUT_F32 if precise else hs2.HS2_OUT_BF16, lse2)
        case.check_guards()
        if precise:
            err = np.abs(out.cpu().numpy()[toks] - o64).max()
            log(f"  fp32 max-abs {err:.3g}")
            assert err <= A4_TOL
        else:
            g16 = synthgen.bf16_to_float(from_dev_bf16(out)[toks]).astype(np.float64)
            err = np.abs(g16 - synthgen.bf16_to_float(o16).astype(np.float64)).max()
            log(f"  bf16 max-abs {err:.3g}")
            assert err <= A3_TOL
        got = lse2.cpu().numpy()
        worst = 0.0
        for tg in toks[::5]:
            for g in range(w.Hkv):
                _, m, l = oracle.group_scores(inp["q_full"], inp["k"], cu, w.Hq, w.Hkv, int(tg),
                                              g, scale=w.scale)
                ref = (m + np.log(l)) / np.log(2.0)
                worst = max(worst, np.abs(got[tg, g * G:(g + 1) * G] - ref).max())
        log(f"  lse2 max-abs {worst:.3g}")
        assert worst <= 1e-4
    case.release_guarded()
