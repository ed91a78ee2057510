"""GPU parity of the full layer's own attention output (hs2_select_full) against
the oracle's dense causal attention: fp32 mode (P in three bf16 parts) within
1e-5 max-abs of the fp64 oracle, bf16 mode within 2e-2 of the oracle's bf16
output. The selection inside hs2_select_full takes its row statistics from the
output sweep, so its index rows meet the selection's own acceptance against the
oracle (structure, A1 margin, A2 overlap); the share equal to hs2_select's is
logged."""
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
    hs2.load_library()


def run_full(w, tokens=None):
    import oracle
    import torch
    import token_level_sparse_hs2_amd as hs2
    log(f"full {w.name}: lengths={w.lengths[:8]} Hq={w.Hq} Hkv={w.Hkv}")
    inp = synthgen.make_inputs(w)
    case = GpuCase(w, inp)
    T = case.T
    toks = np.arange(T) if tokens is None else tokens
    o64, o16 = oracle.full_attn(inp["q_full"], inp["k"], inp["v"], inp["cu_seqlens"], w.Hq, w.Hkv,
                                scale=w.scale, tokens=toks)
    idx_ref, _ = case.select()
    for precise in (True, False):
        out = case.guarded_empty((T, w.Hq, w.d), torch.float32 if precise else torch.bfloat16)
        idx = case.new_idx()
        hs2.hs2_select_full(case.dims, case.varlen, case.q_full, case.k, case.v, idx, out,
                            hs2.HS2_OUT_F32 if precise else hs2.HS2_OUT_BF16,
                            workspace=case.workspace)
        case.check_guards()
        idx_np = idx.cpu().numpy()
        check_structure(idx_np, inp["cu_seqlens"], w.K, w.W)
        same = (idx_np == idx_ref.cpu().numpy()).all(axis=2).mean()
        stats = acceptance_select(idx_np, inp, w, tokens=tokens)
        log(f"  select: rows equal to hs2_select {same:.6f}; vs oracle overlap "
            f"{stats['overlap']:.6f} A1 margin {stats['a1_worst_margin']:.3g}")
        assert_select_ok(stats)
        if precise:
            err = np.abs(out.cpu().numpy()[toks] - o64).max()
            log(f"  fp32 max-abs {err:.3g}")
            assert err <= A4_TOL
        else:
            g = synthgen.bf16_to_float(from_dev_bf16(out)[toks]).astype(np.float64)
            err = np.abs(g - synthgen.bf16_to_float(o16).astype(np.float64)).max()
            log(f"  bf16 max-abs {err:.3g}")
            assert err <= A3_TOL


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_full_output_ragged_every_group_size(G):
    w = synthgen.custom([1, 33, 128, 129, 700, 2100], Hq=2 * G, Hkv=2, K=256, W=32, n_sparse=1,
                        seed=90 + G)
    run_full(w)


def test_full_output_8k_sampled():
    w = synthgen.workload("8k")
    run_full(w, tokens=sample_tokens(w.lengths, w.K, w.W, head=64, tail=16, stride=509))


def test_full_output_128k_sampled():
    # the largest configuration the bench times the full layer's output on (G = 8)
    w = synthgen.workload("128k")
    run_full(w, tokens=sample_tokens(w.lengths, w.K, w.W, head=16, tail=8, stride=8191))


def test_full_output_varlen_sampled():
    # the mixed-length batch the bench times (8 sequences, 290k tokens, up to 97k each)
    w = synthgen.workload("varlen")
    run_full(w, tokens=sample_tokens(w.lengths, w.K, w.W, head=8, tail=4, stride=16381))
