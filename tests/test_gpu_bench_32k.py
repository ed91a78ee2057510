"""GPU parity at the 32k workload (B=1, L=32768, Hq=32, Hkv=8, K=1024, W=128, needle
keys, three sparse layers) for every call bench.py times there, in the configuration
it times it:

  - hs2_prefill_block with three sparse layers and bf16 output (the benchmark step,
    its layers from the shared-gather plan), plus the same block in fp32 mode;
  - hs2_full_attn and hs2_select_full (the full layer's own output, fp32 and bf16);
  - the FP8 cache with scales 1/16: the quantizer's codes (every element) and the
    planned FP8 layer;
  - hs2_select_ex with the output-aware metric (beta 0.5) and with the
    position-decaying budget (mu 0.5);
  - 64-token block selection;
  - top_k 3000 (above the register-ranked limit: rows ranked from their candidate
    lists) and the exact path (the exact flag at top_k 1024);
  - run-to-run identity of the selection, and identity when the workspace forces
    one selection task per chunk.

The oracle runs on a fixed token sample (head and tail of the prompt, a stride, and
the rows around the budget boundaries), every KV group of each sampled token; the
structural checks cover every row. Tolerances are the acceptance bounds A1-A4.
"""
import numpy as np
import pytest

import synthgen
from hs2_testlib import (A1_TOL, A2_MIN, A3_TOL, A4_TOL, GpuCase, acceptance_select,
                         assert_select_ok, check_structure, from_dev_bf16, local_t, log,
                         sample_tokens)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w32():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_level_sparse_hs2_amd as hs2
    hs2.load_library()
    w = synthgen.workload("32k")
    assert w.n_sparse == 3 and w.total == 32768
    log(f"32k workload: Hq={w.Hq} Hkv={w.Hkv} K={w.K} W={w.W} layers={w.n_sparse}")
    inp = synthgen.make_inputs(w)
    case = GpuCase(w, inp)
    toks = sample_tokens(w.lengths, w.K, w.W, head=96, tail=16, stride=1021)
    yield w, inp, case, toks
    case.release_guarded()


@pytest.fixture(autouse=True)
def _release(w32):
    yield
    w32[2].release_guarded()


def bf16_err(gpu_t, toks, o16):
    g = synthgen.bf16_to_float(from_dev_bf16(gpu_t)[toks]).astype(np.float64)
    return np.abs(g - synthgen.bf16_to_float(o16).astype(np.float64)).max()


def test_prefill_block_as_benched(w32):
    import oracle
    import torch
    w, inp, case, toks = w32
    cu = inp["cu_seqlens"]
    idx_t, outs = case.prefill_block(precise=False)
    idx = idx_t.cpu().numpy()
    check_structure(idx, cu, w.K, w.W)
    stats = acceptance_select(idx, inp, w, tokens=toks)
    log(f"  select: rows {stats['rows']} identical {stats['exact_rows']} overlap "
        f"{stats['overlap']:.6f} A1 margin {stats['a1_worst_margin']:.3g}")
    assert_select_ok(stats)
    # every layer's bf16 output against the oracle's bf16 output on the GPU's rows (A3)
    for l in range(w.n_sparse):
        _, o16 = oracle.sparse_attn(inp["q_sparse"][l], inp["k"], inp["v"], cu, w.Hq, w.Hkv,
                                    idx, scale=w.scale, tokens=toks, want_f64=False)
        err = bf16_err(outs[l], toks, o16)
        log(f"  layer {l}: bf16 max-abs {err:.3g}")
        assert err <= A3_TOL
    # the same block in fp32 mode: same rows, each layer within A4 of the fp64 oracle
    idx32_t, outs32 = case.prefill_block(precise=True)
    assert torch.equal(idx32_t, idx_t), "the selection must not depend on the output mode"
    for l in range(w.n_sparse):
        o64, _ = oracle.sparse_attn(inp["q_sparse"][l], inp["k"], inp["v"], cu, w.Hq, w.Hkv,
                                    idx, scale=w.scale, tokens=toks, want_bf16=False)
        err = np.abs(outs32[l].cpu().numpy()[toks] - o64).max()
        log(f"  layer {l}: fp32 max-abs {err:.3g}")
        assert err <= A4_TOL


def test_full_layer_output_as_benched(w32):
    import oracle
    import torch
    import token_level_sparse_hs2_amd as hs2
    w, inp, case, toks = w32
    cu = inp["cu_seqlens"]
    T = case.T
    o64, o16 = oracle.full_attn(inp["q_full"], inp["k"], inp["v"], cu, w.Hq, w.Hkv,
                                scale=w.scale, tokens=toks)
    for precise in (False, True):
        dt = torch.float32 if precise else torch.bfloat16
        mode = hs2.HS2_OUT_F32 if precise else hs2.HS2_OUT_BF16
        out_a = case.guarded_empty((T, w.Hq, w.d), dt)
        lse2 = case.guarded_empty((T, w.Hq), torch.float32)
        hs2.hs2_full_attn(case.dims, case.varlen, case.q_full, case.k, case.v, out_a, mode, lse2)
        out_s = case.guarded_empty((T, w.Hq, w.d), dt)
        idx_t = case.new_idx()
        hs2.hs2_select_full(case.dims, case.varlen, case.q_full, case.k, case.v, idx_t, out_s,
                            mode, workspace=case.workspace)
        case.check_guards()
        assert torch.equal(out_a, out_s), "hs2_full_attn is hs2_select_full's output sweep"
        if precise:
            err = np.abs(out_a.cpu().numpy()[toks] - o64).max()
            log(f"  full output fp32 max-abs {err:.3g}")
            assert err <= A4_TOL
        else:
            err = bf16_err(out_a, toks, o16)
            log(f"  full output bf16 max-abs {err:.3g}")
            assert err <= A3_TOL
        # the row statistics written beside the output: log2 of sum_j exp(z_j), z = scale q.k
        got = lse2.cpu().numpy()[toks]
        worst = 0.0
        for n, tg in enumerate(toks[::7]):
            for g in range(w.Hkv):
                _, m, l = oracle.group_scores(inp["q_full"], inp["k"], cu, w.Hq, w.Hkv, int(tg),
                                              g, scale=w.scale)
                ref = (m + np.log(l)) / np.log(2.0)
                worst = max(worst, np.abs(got[7 * n, g * (w.Hq // w.Hkv):(g + 1) * (w.Hq // w.Hkv)]
                                          - ref).max())
        log(f"  lse2 max-abs {worst:.3g}")
        assert worst <= 1e-4
        # the selection inside hs2_select_full meets the selection's acceptance
        stats = acceptance_select(idx_t.cpu().numpy(), inp, w, tokens=toks)
        log(f"  select_full rows: overlap {stats['overlap']:.6f} A1 margin "
            f"{stats['a1_worst_margin']:.3g}")
        assert_select_ok(stats)
        case.release_guarded()


def test_fp8_cache_as_benched(w32):
    import oracle
    import torch
    import token_level_sparse_hs2_amd as hs2
    w, inp, case, toks = w32
    cu = inp["cu_seqlens"]
    T = case.T
    ks, vs = 1.0 / 16, 1.0 / 16
    k8 = case.guarded_empty((T, w.Hkv, w.d), torch.uint8)
    v8 = case.guarded_empty((T, w.Hkv, w.d), torch.uint8)
    hs2.hs2_quantize_fp8(case.k, k8, 1.0 / ks)
    hs2.hs2_quantize_fp8(case.v, v8, 1.0 / vs)
    case.check_guards()
    k8_ref = oracle.quantize_fp8(inp["k"], 1.0 / ks)
    v8_ref = oracle.quantize_fp8(inp["v"], 1.0 / vs)
    assert np.array_equal(k8.cpu().numpy(), k8_ref) and np.array_equal(v8.cpu().numpy(), v8_ref)
    idx_t, _ = case.select()
    n = hs2.hs2_workspace_size(case.dims, case.varlen, hs2.HS2_OP_SPARSE_PLAN)
    plan = torch.empty(n, dtype=torch.uint8, device="cuda")
    hs2.hs2_sparse_plan(case.dims, case.varlen, idx_t, plan)
    idx = idx_t.cpu().numpy()
    o64, o16 = oracle.sparse_attn_fp8(inp["q_sparse"][0], k8_ref, v8_ref, ks, vs, cu, w.Hq, w.Hkv,
                                      idx, scale=w.scale, tokens=toks)
    for precise in (False, True):
        dt = torch.float32 if precise else torch.bfloat16
        out = case.guarded_empty((T, w.Hq, w.d), dt)
        hs2.hs2_sparse_attn_planned_fp8(case.dims, case.varlen, case.q_sparse[0], k8, v8, ks, vs,
                                        plan, out, hs2.HS2_OUT_F32 if precise else hs2.HS2_OUT_BF16)
        case.check_guards()
        if precise:
            err = np.abs(out.cpu().numpy()[toks] - o64).max()
            log(f"  planned FP8 layer fp32 max-abs {err:.3g}")
            assert err <= A4_TOL
        else:
            err = bf16_err(out, toks, o16)
            log(f"  planned FP8 layer bf16 max-abs {err:.3g}")
            assert err <= A3_TOL


def decay_budget(K, k_end, t, L):
    """Per-position budget of the decaying selection, for the structural check only
    (the selection itself is compared with the oracle on the sampled rows)."""
    if L <= 1 or k_end == K:
        return np.full_like(t, K)
    return K - ((K - k_end) * t) // (L - 1)


@pytest.mark.parametrize("beta,mu", [(0.5, 0.0), (0.0, 0.5)])
def test_select_variants_as_benched(w32, beta, mu):
    import oracle
    import torch
    import token_level_sparse_hs2_amd as hs2
    w, inp, case, toks = w32
    cu = inp["cu_seqlens"]
    T = case.T
    idx_t = case.new_idx()
    kth_t = case.guarded_empty((T, w.Hkv), torch.float32)
    hs2.hs2_select_ex(case.dims, case.varlen, case.q_full, case.k, idx_t, kth_t, v=case.v,
                      oam_beta=beta, decay_mu=mu, workspace=case.workspace)
    case.check_guards()
    idx = idx_t.cpu().numpy()
    tl = local_t(cu, np.arange(T))
    n_c = np.maximum(0, tl - w.W + 1)
    k_end = oracle.decay_k_end(w.K, mu)
    n_glob = np.minimum(n_c, decay_budget(w.K, k_end, tl, T))
    check_structure(idx, cu, w.K, w.W, n_glob=np.repeat(n_glob[:, None], w.Hkv, axis=1))
    rows = (toks[:, None] * w.Hkv + np.arange(w.Hkv)[None, :]).ravel()
    o_idx, o_kth = oracle.select(inp["q_full"], inp["k"], cu, w.Hq, w.Hkv, w.K, w.W,
                                 scale=w.scale, rows=rows, v=inp["v"], oam_beta=beta,
                                 decay_mu=mu)
    wv = np.maximum(1.0, np.linalg.norm(synthgen.bf16_to_float(inp["v"]).astype(np.float64),
                                        axis=2)) ** beta
    g_rows = idx.reshape(T * w.Hkv, -1)[rows]
    inter = tot = same = 0
    worst = np.inf
    for r, row_id in enumerate(rows):
        a, b = g_rows[r][g_rows[r] >= 0], o_idx[r][o_idx[r] >= 0]
        inter += len(np.intersect1d(a, b))
        tot += len(b)
        if len(a) == len(b) and (a == b).all():
            same += 1
            continue
        tg, g = divmod(int(row_id), w.Hkv)
        nc = int(n_c[tg])
        S, _, _ = oracle.group_scores(inp["q_full"], inp["k"], cu, w.Hq, w.Hkv, tg, g,
                                      scale=w.scale)
        glob = a[a < nc]
        if len(glob):
            worst = min(worst, (S[glob] * wv[glob, g]).min() - o_kth[r])
    overlap = inter / max(1, tot)
    log(f"  beta {beta} mu {mu}: rows {len(rows)} identical {same} overlap {overlap:.6f} "
        f"A1 margin {worst:.3g}")
    assert overlap >= A2_MIN and worst >= -A1_TOL
    kth = kth_t.cpu().numpy().reshape(-1)[rows]
    sel = o_kth > 0
    assert ((kth < 0) == ~sel).all()
    rel = np.abs(kth[sel] - o_kth[sel]) / o_kth[sel]
    log(f"  kth relative diff: max {rel.max():.3g}")
    assert rel.max() <= 1e-3


def test_block_selection_as_benched(w32):
    import oracle
    import torch
    import token_level_sparse_hs2_amd as hs2
    from test_gpu_blocks import BS, check_block_row
    w, inp, case, toks = w32
    cu = inp["cu_seqlens"]
    T = case.T
    dims = hs2.make_dims(w.Hq, w.Hkv, w.K, w.W, w.scale, flags=hs2.HS2_FLAG_BLOCK_SELECT)
    assert (hs2.hs2_workspace_size(dims, case.varlen, hs2.HS2_OP_SELECT)
            <= case.workspace.numel())
    idx_t = case.new_idx()
    kth_t = case.guarded_empty((T, w.Hkv), torch.float32)
    hs2.hs2_select(dims, case.varlen, case.q_full, case.k, idx_t, kth_t, case.workspace)
    case.check_guards()
    idx, kth = idx_t.cpu().numpy(), kth_t.cpu().numpy().reshape(-1)
    rows = (toks[:, None] * w.Hkv + np.arange(w.Hkv)[None, :]).ravel()
    o_idx, o_kth = oracle.select(inp["q_full"], inp["k"], cu, w.Hq, w.Hkv, w.K, w.W,
                                 scale=w.scale, rows=rows, block=BS)
    g_rows = idx.reshape(T * w.Hkv, -1)[rows]
    same = 0
    worst = np.inf
    for r, row_id in enumerate(rows):
        tg, g = divmod(int(row_id), w.Hkv)
        t = int(local_t(cu, np.array([tg]))[0])
        blocks = check_block_row(g_rows[r], t, w.K, w.W)
        if np.array_equal(g_rows[r], o_idx[r]):
            same += 1
            continue
        S, _, _ = oracle.group_scores(inp["q_full"], inp["k"], cu, w.Hq, w.Hkv, tg, g,
                                      scale=w.scale)
        n_c = t - w.W + 1
        worst = min(worst, min(S[b * BS:min((b + 1) * BS, n_c)].sum() for b in blocks) - o_kth[r])
    log(f"  blocks: rows {len(rows)} identical {same} worst block margin {worst:.3g}")
    assert same >= 0.999 * len(rows) and worst >= -1e-5
    sel = o_kth > 0
    rel = np.abs(kth[rows][sel] - o_kth[sel]) / o_kth[sel]
    log(f"  kth relative diff: max {rel.max():.3g}")
    assert rel.max() <= 1e-3


@pytest.mark.parametrize("K,flags", [(3000, 0), (1024, 1)], ids=["large_budget", "exact_flag"])
def test_large_budget_and_exact_path_as_benched(w32, K, flags):
    """bench.py's large_budget figure (top_k 3000: every row with more candidates is
    ranked from its candidate list by the exact kernel) and exact_path figure (the
    exact flag at top_k 1024: every such row ranked over its whole row of scores)."""
    import torch
    import token_level_sparse_hs2_amd as hs2
    w, inp, case, toks = w32
    dims = hs2.make_dims(w.Hq, w.Hkv, K, w.W, w.scale,
                         flags=hs2.HS2_FLAG_EXACT_SELECT if flags else 0)
    ws = torch.empty(hs2.hs2_workspace_size(dims, case.varlen, hs2.HS2_OP_SELECT),
                     dtype=torch.uint8, device="cuda")
    idx_t = case.new_idx(K + w.W)
    hs2.hs2_select(dims, case.varlen, case.q_full, case.k, idx_t, None, ws)
    case.check_guards()
    idx = idx_t.cpu().numpy()
    check_structure(idx, inp["cu_seqlens"], K, w.W)
    wk = synthgen.workload("32k")
    wk.K = K
    stats = acceptance_select(idx, inp, wk, tokens=toks)
    log(f"  K={K} flags={flags}: rows {stats['rows']} identical {stats['exact_rows']} overlap "
        f"{stats['overlap']:.6f} A1 margin {stats['a1_worst_margin']:.3g}")
    assert_select_ok(stats)


def test_selection_is_deterministic_and_chunk_independent(w32):
    """The collect sweep appends candidates in scheduling order (LDS atomics); the
    top-K ranks them through position bitmaps, so the index rows (and K-th scores)
    must not depend on that order, on the run, or on how the work is chunked: a
    workspace of hs2_workspace_size(HS2_OP_SELECT_MIN) runs one task per chunk."""
    import torch
    import token_level_sparse_hs2_amd as hs2
    w, inp, case, toks = w32
    idx_a, kth_a = case.select()
    idx_b, kth_b = case.select()
    assert torch.equal(idx_a, idx_b) and torch.equal(kth_a, kth_b)
    n_min = hs2.hs2_workspace_size(case.dims, case.varlen, hs2.HS2_OP_SELECT_MIN)
    n_full = hs2.hs2_workspace_size(case.dims, case.varlen, hs2.HS2_OP_SELECT)
    log(f"  workspace: full {n_full} bytes, minimum {n_min} bytes")
    assert n_min < n_full
    ws = torch.empty(n_min, dtype=torch.uint8, device="cuda")
    idx_c = case.new_idx()
    kth_c = case.guarded_empty((case.T, w.Hkv), torch.float32)
    hs2.hs2_select(case.dims, case.varlen, case.q_full, case.k, idx_c, kth_c, ws)
    case.check_guards()
    assert torch.equal(idx_a, idx_c) and torch.equal(kth_a, kth_c)
