"""GPU parity of the shared-gather plan through the C ABI: hs2_sparse_plan,
hs2_sparse_attn_planned(_fp8), and hs2_prefill_block, which runs its sparse
layers from a plan when its workspace holds one.

Plan (index work, bit-exact): every union list equals, entry for entry, the
sorted union of its tokens' index rows computed here on the host from the same
rows, each entry with the mask of the tokens that hold it; every count matches.
Planned layers: A4 (fp32 mode) and A3 (bf16) against the oracle on the GPU's
index rows, as for hs2_sparse_attn, and the per-token layer within A4.
"""
import numpy as np
import pytest

import synthgen
from hs2_testlib import A3_TOL, A4_TOL, GpuCase, from_dev_bf16, log, sample_tokens

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_level_sparse_hs2_amd as hs2
    hs2.load_library()


def plan_tokens(G):
    return 16 // G if G >= 2 else 8


def host_unions(idx, cu, Hkv, G):
    """Expected unions: {(grp, g): (rows relative to base0 ascending, masks)}."""
    T = int(cu[-1])
    NT = plan_tokens(G)
    seq_of = np.searchsorted(cu, np.arange(T), side="right") - 1
    out = {}
    for grp in range((T + NT - 1) // NT):
        toks = np.arange(grp * NT, min(T, grp * NT + NT))
        base0 = int(cu[seq_of[toks[0]]])
        for g in range(Hkv):
            rels, masks = [], []
            for a, tg in enumerate(toks):
                base = int(cu[seq_of[tg]])
                t = int(tg) - base
                row = idx[tg, g]
                row = row[(row >= 0) & (row <= t)]
                rels.append(base - base0 + row.astype(np.int64))
                masks.append(np.full(len(row), 1 << a, dtype=np.int64))
            r = np.concatenate(rels)
            m = np.concatenate(masks)
            u, inv = np.unique(r, return_inverse=True)
            um = np.zeros(len(u), dtype=np.int64)
            np.bitwise_or.at(um, inv, m)
            out[(grp, g)] = (u, um)
    return out


def gpu_plan(case, idx_t):
    import torch
    hs2 = case.hs2
    n = hs2.hs2_workspace_size(case.dims, case.varlen, hs2.HS2_OP_SPARSE_PLAN)
    plan = torch.empty(n, dtype=torch.uint8, device="cuda")
    hs2.hs2_sparse_plan(case.dims, case.varlen, idx_t, plan)
    torch.cuda.synchronize()
    return plan


def check_plan_lists(case, idx_t, plan):
    """The plan's lists against host_unions, bit-exact (the layout: one word per
    entry, row | mask << 24, [n_grp * Hkv, NT * KW], then the counts, 256-aligned)."""
    w = case.w
    G = w.Hq // w.Hkv
    NT = plan_tokens(G)
    T, KW = case.T, case.KW
    n_grp = (T + NT - 1) // NT
    cap = NT * KW
    lists = n_grp * w.Hkv
    off_count = (lists * cap * 4 + 255) // 256 * 256
    raw = plan.cpu().numpy()
    words = raw[:lists * cap * 4].view(np.uint32).reshape(lists, cap)
    counts = raw[off_count:off_count + lists * 4].view(np.int32)
    expect = host_unions(idx_t.cpu().numpy(), case.inputs["cu_seqlens"], w.Hkv, G)
    total = shared = 0
    for (grp, g), (u, um) in expect.items():
        wid = grp * w.Hkv + g
        n = int(counts[wid])
        assert n == len(u), (grp, g, n, len(u))
        got = words[wid, :n]
        assert (got & 0xFFFFFF == u).all(), (grp, g)
        assert (got >> 24 == um).all(), (grp, g)
        total += n
        shared += int(np.bitwise_count(um.astype(np.uint64)).sum()) if hasattr(np, "bitwise_count") \
            else int(sum(bin(int(x)).count("1") for x in um))
    log(f"  plan: {len(expect)} unions, {total} entries for {shared} (token, row) pairs "
        f"({total / max(1, shared):.3f} gathered per pair)")


def planned(case, plan, q, precise):
    import torch
    hs2 = case.hs2
    out = torch.empty((case.T, case.w.Hq, case.w.d),
                      dtype=torch.float32 if precise else torch.bfloat16, device="cuda")
    hs2.hs2_sparse_attn_planned(case.dims, case.varlen, q, case.k, case.v, plan, out,
                                hs2.HS2_OUT_F32 if precise else hs2.HS2_OUT_BF16)
    torch.cuda.synchronize()
    return out


def check_planned_layers(case, idx_t, plan, tokens=None):
    import oracle
    w, inp = case.w, case.inputs
    idx = idx_t.cpu().numpy()
    toks = np.arange(case.T, dtype=np.int64) if tokens is None else tokens
    for l, (qs_np, qs) in enumerate(zip(inp["q_sparse"], case.q_sparse)):
        out32 = planned(case, plan, qs, True).cpu().numpy()
        o64, o16 = oracle.sparse_attn(qs_np, inp["k"], inp["v"], inp["cu_seqlens"], w.Hq, w.Hkv,
                                      idx, scale=w.scale, tokens=toks)
        err4 = np.abs(out32[toks] - o64).max()
        g16 = synthgen.bf16_to_float(from_dev_bf16(planned(case, plan, qs, False))[toks])
        err3 = np.abs(g16.astype(np.float64) - synthgen.bf16_to_float(o16)).max()
        per_tok = case.sparse(qs, idx_t, precise=True).cpu().numpy()
        diff = np.abs(out32 - per_tok).max()
        log(f"  layer {l}: A4 max-abs {err4:.3g} A3 max-abs {err3:.3g}; "
            f"planned vs per-token {diff:.3g}")
        assert err4 <= A4_TOL and err3 <= A3_TOL and diff <= A4_TOL


def run_plan_case(w, select_fn=None, tokens=None):
    log(f"plan case {w.name}: lengths={w.lengths[:8]} Hq={w.Hq} Hkv={w.Hkv} K={w.K} W={w.W}")
    inp = synthgen.make_inputs(w)
    case = GpuCase(w, inp)
    idx_t = select_fn(case) if select_fn else case.select()[0]
    plan = gpu_plan(case, idx_t)
    if tokens is None:
        check_plan_lists(case, idx_t, plan)
    check_planned_layers(case, idx_t, plan, tokens)
    return case, idx_t, plan


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_plan_ragged_varlen_every_group_size(G):
    """Tiny sequences put several sequences into one token group; the sum of
    lengths leaves a partial last group."""
    w = synthgen.custom([1, 2, 3, 33, 130, 700, 2101], Hq=2 * G, Hkv=2, K=128, W=16,
                        n_sparse=1, seed=300 + G)
    run_plan_case(w)


@pytest.mark.parametrize("lengths", [[1], [3], [1, 1, 1], [2, 1, 70]])
def test_plan_batches_smaller_than_a_group(lengths):
    """Fewer tokens than a group holds (4 at G = 4), several sequences in one group."""
    w = synthgen.custom(lengths, Hq=8, Hkv=2, K=16, W=4, n_sparse=1, seed=320 + len(lengths))
    run_plan_case(w)


@pytest.mark.parametrize("K,W", [(0, 32), (256, 0), (1, 1)])
def test_plan_budget_edges(K, W):
    w = synthgen.custom([5, 64, 65, 1500], Hq=8, Hkv=2, K=K, W=W, n_sparse=1, seed=310)
    run_plan_case(w)


def test_plan_padded_rows_of_a_decaying_budget():
    """Rows shortened by the position-decaying budget end in -1 padding."""
    import torch

    def select_decay(case):
        hs2 = case.hs2
        idx = case.new_idx()
        hs2.hs2_select_ex(case.dims, case.varlen, case.q_full, case.k, idx, decay_mu=0.25,
                          workspace=case.workspace)
        case.check_guards()
        return idx

    w = synthgen.custom([700, 3000], Hq=8, Hkv=2, K=512, W=32, n_sparse=1, seed=311)
    _, idx_t, _ = run_plan_case(w, select_fn=select_decay)
    assert (idx_t.cpu().numpy() < 0).any()


@pytest.mark.parametrize("flag", ["block", "exact"])
def test_plan_of_block_and_exact_rows(flag):
    """Rows from the 64-token block selection (runs of 64 positions: dense bitmap
    words) and from the exact path (every row ranked over its whole candidate range)."""
    import torch

    def select_flag(case):
        hs2 = case.hs2
        f = hs2.HS2_FLAG_BLOCK_SELECT if flag == "block" else hs2.HS2_FLAG_EXACT_SELECT
        dims = hs2.make_dims(case.w.Hq, case.w.Hkv, case.w.K, case.w.W, case.w.scale, flags=f)
        idx = case.new_idx()
        hs2.hs2_select(dims, case.varlen, case.q_full, case.k, idx, None, case.workspace)
        case.check_guards()
        return idx

    w = synthgen.custom([70, 1500, 2600], Hq=8, Hkv=2, K=256, W=32, n_sparse=1, seed=313)
    run_plan_case(w, select_fn=select_flag)


def test_plan_fp8_cache():
    import oracle
    import torch
    w = synthgen.custom([3, 700, 2100], Hq=8, Hkv=2, K=256, W=32, n_sparse=1, seed=312)
    inp = synthgen.make_inputs(w)
    case = GpuCase(w, inp)
    idx_t, _ = case.select()
    plan = gpu_plan(case, idx_t)
    ks, vs = 0.037, 0.05
    k8 = oracle.quantize_fp8(inp["k"], 1.0 / ks)
    v8 = oracle.quantize_fp8(inp["v"], 1.0 / vs)
    k8_d, v8_d = torch.from_numpy(k8).cuda(), torch.from_numpy(v8).cuda()
    hs2 = case.hs2
    qs_np, qs = inp["q_sparse"][0], case.q_sparse[0]
    out32 = torch.empty((case.T, w.Hq, w.d), dtype=torch.float32, device="cuda")
    out16 = torch.empty((case.T, w.Hq, w.d), dtype=torch.bfloat16, device="cuda")
    hs2.hs2_sparse_attn_planned_fp8(case.dims, case.varlen, qs, k8_d, v8_d, ks, vs, plan, out32,
                                    hs2.HS2_OUT_F32)
    hs2.hs2_sparse_attn_planned_fp8(case.dims, case.varlen, qs, k8_d, v8_d, ks, vs, plan, out16,
                                    hs2.HS2_OUT_BF16)
    torch.cuda.synchronize()
    o64, o16 = oracle.sparse_attn_fp8(qs_np, k8, v8, ks, vs, inp["cu_seqlens"], w.Hq, w.Hkv,
                                      idx_t.cpu().numpy(), scale=w.scale)
    err4 = np.abs(out32.cpu().numpy() - o64).max()
    g = synthgen.bf16_to_float(from_dev_bf16(out16)).astype(np.float64)
    err3 = np.abs(g - synthgen.bf16_to_float(o16).astype(np.float64)).max()
    log(f"  fp8 planned: A4 max-abs {err4:.3g} A3 max-abs {err3:.3g}")
    assert err4 <= A4_TOL and err3 <= A3_TOL


def test_prefill_block_runs_the_plan():
    """With the workspace of hs2_workspace_size(HS2_OP_PREFILL_BLOCK) the block's layers
    equal hs2_sparse_plan + hs2_sparse_attn_planned bit for bit. (A workspace too small
    for the plan runs them as hs2_sparse_attn; at these sizes the selection's scratch
    is the larger of the two, so the plan always fits.)"""
    import torch
    w = synthgen.custom([1000, 3000], Hq=8, Hkv=2, K=256, W=32, n_sparse=2, seed=9)
    inp = synthgen.make_inputs(w)
    case = GpuCase(w, inp)
    hs2 = case.hs2
    n_plan = hs2.hs2_workspace_size(case.dims, case.varlen, hs2.HS2_OP_SPARSE_PLAN)
    assert n_plan <= case.workspace.numel()
    idx_b, outs = case.prefill_block()
    idx_s, _ = case.select()
    assert torch.equal(idx_b, idx_s)
    plan = gpu_plan(case, idx_s)
    for qs, ob in zip(case.q_sparse, outs):
        assert torch.equal(planned(case, plan, qs, False), ob)


def run_sampled_workload(name, head, tail, stride):
    """A bench configuration (or a given one-sequence workload): the unions of the
    groups holding sampled tokens checked against the host union, the planned layer
    on the sampled tokens."""
    w = synthgen.workload(name) if isinstance(name, str) else name
    name = w.name
    w.n_sparse = 1
    toks = sample_tokens(w.lengths, w.K, w.W, head=head, tail=tail, stride=stride)
    inp = synthgen.make_inputs(w)
    case = GpuCase(w, inp)
    idx_t, _ = case.select()
    plan = gpu_plan(case, idx_t)
    G = w.Hq // w.Hkv
    NT = plan_tokens(G)
    T, KW = case.T, case.KW
    n_grp = (T + NT - 1) // NT
    lists = n_grp * w.Hkv
    off_count = (lists * NT * KW * 4 + 255) // 256 * 256
    raw = plan.cpu().numpy()
    words = raw[:lists * NT * KW * 4].view(np.uint32).reshape(lists, NT * KW)
    counts = raw[off_count:off_count + lists * 4].view(np.int32)
    idx = idx_t.cpu().numpy()
    grps = np.unique(toks // NT)
    for grp in grps:  # one sequence: rows relative to base 0 are the positions
        sub = idx[grp * NT:min(T, grp * NT + NT)]
        for g in range(w.Hkv):
            rows = sub[:, g]
            u, inv = np.unique(rows[rows >= 0], return_inverse=True)
            a = np.nonzero(rows >= 0)[0]
            um = np.zeros(len(u), dtype=np.int64)
            np.bitwise_or.at(um, inv, 1 << a)
            wid = grp * w.Hkv + g
            assert counts[wid] == len(u)
            got = words[wid, :len(u)]
            assert (got & 0xFFFFFF == u).all() and (got >> 24 == um).all()
    log(f"  {name}: {len(grps)} groups' unions exact; mean union {counts.mean():.0f} of {NT * KW}")
    check_planned_layers(case, idx_t, plan, tokens=toks)


def test_32k_workload_planned_sampled():
    run_sampled_workload("32k", head=128, tail=16, stride=1021)


def test_128k_workload_planned_sampled():
    """G = 8: two tokens per group."""
    run_sampled_workload("128k", head=64, tail=8, stride=4093)


def test_prefill_block_without_sparse_layers():
    """n_sparse = 0: the block is the selection alone (no plan is built, and the
    workspace of hs2_workspace_size(HS2_OP_PREFILL_BLOCK, 0) is the selection's)."""
    import torch
    w = synthgen.custom([700, 3000], Hq=8, Hkv=2, K=256, W=32, n_sparse=1, seed=19)
    inp = synthgen.make_inputs(w)
    case = GpuCase(w, inp)
    hs2 = case.hs2
    n0 = hs2.hs2_workspace_size(case.dims, case.varlen, hs2.HS2_OP_PREFILL_BLOCK, 0)
    assert n0 == hs2.hs2_workspace_size(case.dims, case.varlen, hs2.HS2_OP_SELECT)
    ws = torch.empty(n0, dtype=torch.uint8, device="cuda")
    idx_b = case.new_idx()
    hs2.hs2_prefill_block(case.dims, case.varlen, case.q_full, case.k, case.v, [], [], idx_b,
                          hs2.HS2_OUT_BF16, ws)
    case.check_guards()
    idx_s, _ = case.select()
    assert torch.equal(idx_b, idx_s)


def test_longest_sequence_planned_sampled():
    """One sequence of the longest length the boundary accepts (HS2_MAX_SEQLEN)."""
    import token_level_sparse_hs2_amd as hs2
    w = synthgen.custom([hs2.HS2_MAX_SEQLEN], Hq=8, Hkv=2, K=1024, W=128, n_sparse=1, seed=2622)
    run_sampled_workload(w, head=16, tail=8, stride=32749)
