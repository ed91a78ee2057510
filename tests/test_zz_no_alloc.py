"""The decode sparse layer's entry point that allocates nothing
(hs2_decode_sparse_attn_noalloc), through the C ABI, against the entry point it
varies (hs2_decode_sparse_attn with a caller workspace): the same kernels on the
same split, so the outputs must be bit-identical, in bf16 and fp32 mode. Two
calls in a row on one GPU share the library's scratch; the second has a smaller
input (fewer, shorter caches and a different split), so stale partials of the
first must not leak into it. The index rows come from hs2_decode_select, and the
fp32 output is also held to the oracle (A4)."""
import numpy as np
import pytest

import synthgen
from hs2_testlib import A4_TOL, log, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_level_sparse_hs2_amd as hs2
    hs2.load_library()


def decode_case(w):
    import torch
    import token_level_sparse_hs2_amd as hs2
    inp = synthgen.make_decode_inputs(w)
    cu = inp["cu_seqlens"]
    cu_dev = torch.from_numpy(cu.astype(np.int32)).cuda()
    cache = hs2.VarlenArgs(cu_dev, [int(x) for x in cu])
    dims = hs2.make_dims(w.Hq, w.Hkv, w.K, w.W, w.scale)
    dev = {"k": to_dev_bf16(inp["k"]), "v": to_dev_bf16(inp["v"]),
           "q": to_dev_bf16(inp["q_dec"]), "qs": to_dev_bf16(inp["q_sparse_dec"][0])}
    ws = torch.empty(max(1, hs2.hs2_workspace_size(dims, cache, hs2.HS2_OP_DECODE_SELECT, 0)),
                     dtype=torch.uint8, device="cuda")
    B = len(w.lengths)
    idx = torch.empty((B, w.Hkv, w.K + w.W), dtype=torch.int32, device="cuda")
    hs2.hs2_decode_select(dims, cache, dev["q"], dev["k"], idx, None, ws)
    torch.cuda.synchronize()
    return inp, cache, dims, dev, idx


def run_pair(w):
    import oracle
    import torch
    import token_level_sparse_hs2_amd as hs2
    inp, cache, dims, dev, idx = decode_case(w)
    B = len(w.lengths)
    n_ws = hs2.hs2_workspace_size(dims, cache, hs2.HS2_OP_DECODE_SPARSE, 0)
    log(f"no-alloc decode: lengths {w.lengths} Hq={w.Hq} Hkv={w.Hkv} K={w.K} W={w.W} "
        f"partials {n_ws} bytes (scratch {hs2.HS2_NOALLOC_SCRATCH_BYTES})")
    assert 0 < n_ws <= hs2.HS2_NOALLOC_SCRATCH_BYTES  # the split path, through the scratch
    ws = torch.empty(n_ws, dtype=torch.uint8, device="cuda")
    outs = {}
    for mode, dt in ((hs2.HS2_OUT_BF16, torch.bfloat16), (hs2.HS2_OUT_F32, torch.float32)):
        ref = torch.empty((B, w.Hq, w.d), dtype=dt, device="cuda")
        got = torch.full((B, w.Hq, w.d), float("nan"), dtype=dt, device="cuda")
        hs2.hs2_decode_sparse_attn(dims, cache, dev["qs"], dev["k"], dev["v"], idx, ref, mode, ws)
        hs2.hs2_decode_sparse_attn_noalloc(dims, cache, dev["qs"], dev["k"], dev["v"], idx, got,
                                           mode)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16) if dt == torch.bfloat16 else got.view(torch.int32),
                           ref.view(torch.int16) if dt == torch.bfloat16 else ref.view(torch.int32))
        outs[mode] = got
    o64, _ = oracle.decode_sparse_attn(inp["q_sparse_dec"][0], inp["k"], inp["v"],
                                       inp["cu_seqlens"], w.Hq, w.Hkv, idx.cpu().numpy(),
                                       scale=w.scale, want_bf16=False)
    err = np.abs(outs[hs2.HS2_OUT_F32].cpu().numpy() - o64).max()
    log(f"  bit-identical to the workspace entry point; fp32 vs oracle max-abs {err:.3g}")
    assert err <= A4_TOL


def test_noalloc_matches_workspace_entry_point_twice_second_smaller():
    first = synthgen.custom([32768, 9000, 70001, 1, 4097, 20000, 3000, 12345], Hq=32, Hkv=8,
                            K=1024, W=128, n_sparse=1, seed=1301)
    second = synthgen.custom([5000, 700, 2], Hq=8, Hkv=2, K=256, W=32, n_sparse=1, seed=1302)
    run_pair(first)
    run_pair(second)


def test_noalloc_validation():
    """Validation errors come back before anything runs, as for the workspace entry point."""
    import torch
    import token_level_sparse_hs2_amd as hs2
    w = synthgen.custom([300, 40], Hq=8, Hkv=2, K=64, W=16, n_sparse=1, seed=1303)
    inp, cache, dims, dev, idx = decode_case(w)
    out = torch.empty((2, w.Hq, w.d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(hs2.HS2Error) as e:
        hs2.hs2_decode_sparse_attn_noalloc(dims, cache, dev["qs"], dev["k"], dev["v"], idx, out, 7)
    assert e.value.status == hs2.HS2_ERR_INVALID_ARG
    with pytest.raises(hs2.HS2Error) as e:
        hs2.hs2_decode_sparse_attn_noalloc(dims, cache, dev["qs"], dev["k"], dev["v"], None, out)
    assert e.value.status == hs2.HS2_ERR_INVALID_ARG
