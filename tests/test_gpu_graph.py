"""The library's calls inside captured HIP graphs (torch.cuda.CUDAGraph is a HIP
graph on ROCm): the library allocates, copies to the host and clears memory
nowhere, so a decode step or a prefill block can be captured once and replayed.

Each graph is captured on torch's capture stream, then replayed several times on
changing inputs (copied into the captured buffers between replays, with eager
work of the program in between), and every replay's outputs must be
bit-identical to an eager call on the same inputs.
"""
import numpy as np
import pytest

import synthgen
from hs2_testlib import GpuCase, log, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_level_sparse_hs2_amd as hs2
    hs2.load_library()


def _capture(fn):
    import torch
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the graph, as torch asks
        fn(torch.cuda.current_stream())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(torch.cuda.current_stream())
    torch.cuda.synchronize()
    return g


def _replay_and_compare(g, inputs, buffers, outputs, eager):
    """For each input set: copy it into the captured buffers, replay, compare every
    output with the eager results for that set."""
    import torch
    # the input sets lead to different results, so a replay that ignored them would fail
    assert not all(torch.equal(a, b) for a, b in zip(eager[0], eager[1]))
    for n, (src, ref) in enumerate(zip(inputs, eager)):
        for b, x in zip(buffers, src):
            b.copy_(x)
        junk = torch.randn(1 << 16, device="cuda").sum()  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outputs, ref):
            assert torch.equal(o, r), f"replay {n} differs from the eager call"
        del junk
    log(f"  {len(inputs)} replays bit-identical to eager calls")


@pytest.mark.parametrize("noalloc", [False, True])
def test_decode_step_in_a_graph(noalloc):
    import torch
    import token_level_sparse_hs2_amd as hs2
    w = synthgen.custom([4000, 33, 9000, 1500], Hq=16, Hkv=4, K=256, W=64, n_sparse=2, seed=401)
    inp = synthgen.make_decode_inputs(w)
    cu = inp["cu_seqlens"]
    B, KW = len(w.lengths), w.K + w.W
    cache = hs2.VarlenArgs(torch.from_numpy(cu.astype(np.int32)).cuda(), [int(x) for x in cu])
    dims = hs2.make_dims(w.Hq, w.Hkv, w.K, w.W, w.scale)
    k, v = to_dev_bf16(inp["k"]), to_dev_bf16(inp["v"])
    q = to_dev_bf16(inp["q_dec"])
    qs = [to_dev_bf16(x) for x in inp["q_sparse_dec"]]
    ws = torch.empty(max(1, hs2.hs2_workspace_size(dims, cache, hs2.HS2_OP_DECODE_SELECT, 0)),
                     dtype=torch.uint8, device="cuda")
    ws_sp = torch.empty(max(1, hs2.hs2_workspace_size(dims, cache, hs2.HS2_OP_DECODE_SPARSE, 0)),
                        dtype=torch.uint8, device="cuda")
    idx = torch.empty((B, w.Hkv, KW), dtype=torch.int32, device="cuda")
    outs = [torch.empty((B, w.Hq, w.d), dtype=torch.float32, device="cuda") for _ in qs]

    def step(stream):
        hs2.hs2_decode_select(dims, cache, q, k, idx, None, ws, stream=stream)
        for i in range(len(qs)):
            if noalloc:
                hs2.hs2_decode_sparse_attn_noalloc(dims, cache, qs[i], k, v, idx, outs[i],
                                                   hs2.HS2_OUT_F32, stream=stream)
            else:
                hs2.hs2_decode_sparse_attn(dims, cache, qs[i], k, v, idx, outs[i],
                                           hs2.HS2_OUT_F32, ws_sp, stream=stream)

    # three query sets: the generated one and two perturbations of it
    rng = np.random.default_rng(5)
    sets = []
    for n in range(3):
        scale = 1.0 if n == 0 else float(rng.uniform(0.5, 2.0))
        sets.append([(q.float() * scale).to(torch.bfloat16)] +
                    [(x.float() * scale).to(torch.bfloat16) for x in qs])
    eager = []
    for src in sets:
        for b, x in zip([q] + qs, src):
            b.copy_(x)
        step(torch.cuda.current_stream())
        torch.cuda.synchronize()
        eager.append([idx.clone()] + [o.clone() for o in outs])
    g = _capture(step)
    log(f"decode step graph (noalloc={noalloc}): B={B} Hq={w.Hq} Hkv={w.Hkv} K={w.K} W={w.W}")
    _replay_and_compare(g, sets + sets[:1], [q] + qs, [idx] + outs, eager + eager[:1])


def test_prefill_block_in_a_graph():
    import torch
    import token_level_sparse_hs2_amd as hs2
    w = synthgen.custom([1500, 64, 3000], Hq=8, Hkv=2, K=256, W=32, n_sparse=2, seed=402)
    inp = synthgen.make_inputs(w)
    case = GpuCase(w, inp)
    idx = case.new_idx()
    outs = [torch.empty((case.T, w.Hq, w.d), dtype=torch.float32, device="cuda")
            for _ in case.q_sparse]

    def block(stream):
        hs2.hs2_prefill_block(case.dims, case.varlen, case.q_full, case.k, case.v, case.q_sparse,
                              outs, idx, hs2.HS2_OUT_F32, case.workspace, stream=stream)

    bufs = [case.q_full] + list(case.q_sparse)
    sets = []
    for scale in (1.0, 0.7, 1.6):
        sets.append([(x.float() * scale).to(torch.bfloat16) for x in bufs])
    eager = []
    for src in sets:
        for b, x in zip(bufs, src):
            b.copy_(x)
        block(torch.cuda.current_stream())
        torch.cuda.synchronize()
        eager.append([idx.clone()] + [o.clone() for o in outs])
    g = _capture(block)
    log(f"prefill block graph: lengths={w.lengths} Hq={w.Hq} Hkv={w.Hkv} K={w.K} W={w.W}")
    _replay_and_compare(g, sets + sets[:1], bufs, [idx] + outs, eager + eager[:1])
