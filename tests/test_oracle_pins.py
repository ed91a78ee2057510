"""Pins of the CPU oracle against facts fixed outside it (runs without a GPU).

Each test checks the oracle against something it does not share code with:
library routines (torch scaled_dot_product_attention, scipy softmax), brute force
on tiny inputs, closed forms, and invariants of the selection rule. The
selection rule itself is: per query token t and KV group g, keep the K best
candidates outside the forced recent window of W tokens, by the sum over the
group's heads of each head's softmax probability (HySparse2 news summary,
token-granularity and KV-reuse paragraphs; readings R1-R6 in the oracle header).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synthgen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf(a):
    return synthgen.bf16_to_float(a).astype(np.float64)


def rand_inputs(lengths, Hq, Hkv, d, seed, scale_q=1.0):
    T = int(sum(lengths))
    q = synthgen.normal_bf16(seed, 1, (T, Hq, d))
    k = synthgen.normal_bf16(seed, 2, (T, Hkv, d))
    v = synthgen.normal_bf16(seed, 3, (T, Hkv, d))
    if scale_q != 1.0:
        q = synthgen.float_to_bf16(bf(q) * scale_q)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return q, k, v, cu


def group_scores_ref(q, k, cu, Hq, Hkv, tg, g, scale):
    """Independent S row: scipy softmax per head over causal keys, summed over the group."""
    i = int(np.searchsorted(cu, tg, side="right") - 1)
    base, t = int(cu[i]), int(tg - cu[i])
    G = Hq // Hkv
    kk = bf(k[base:base + t + 1, g, :])
    S = np.zeros(t + 1)
    for hh in range(G):
        z = scale * (kk @ bf(q[tg, g * G + hh, :]))
        S += scipy.special.softmax(z)
    return S


# ----------------------------------------------------------------------------
# C1: with K + W >= L every row is [0, t] and the sparse layer is dense causal
# attention (library routine: torch SDPA, fp64, per sequence, GQA expanded).
# ----------------------------------------------------------------------------
def test_c1_dense_equivalence_against_sdpa():
    lengths, Hq, Hkv, d = [37, 50, 1], 8, 2, 128
    K, W = 40, 16
    q, k, v, cu = rand_inputs(lengths, Hq, Hkv, d, seed=11)
    qs = synthgen.normal_bf16(11, 10, q.shape)
    idx, _ = oracle.select(q, k, cu, Hq, Hkv, K, W)
    T = int(cu[-1])
    idx3 = idx.reshape(T, Hkv, K + W)
    for i in range(len(lengths)):
        for t in range(lengths[i]):
            row = idx3[cu[i] + t]
            for g in range(Hkv):
                assert list(row[g, :t + 1]) == list(range(t + 1))
                assert (row[g, t + 1:] == -1).all()
    o64, _ = oracle.sparse_attn(qs, k, v, cu, Hq, Hkv, idx3, want_bf16=False)
    G = Hq // Hkv
    for i in range(len(lengths)):
        a, b = int(cu[i]), int(cu[i + 1])
        Q = torch.from_numpy(bf(qs[a:b])).permute(1, 0, 2)[None]
        Kt = torch.from_numpy(bf(k[a:b])).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        Vt = torch.from_numpy(bf(v[a:b])).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, is_causal=True)
        ref = ref[0].permute(1, 0, 2).numpy()
        np.testing.assert_allclose(o64[a:b], ref, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# C2: brute force over all size-K subsets on tiny inputs.
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("G,Hkv", [(1, 2), (2, 1), (3, 1)])
def test_c2_bruteforce_topk(G, Hkv):
    Hq, d = G * Hkv, 8
    for L in (5, 9, 12):
        q, k, _, cu = rand_inputs([L], Hq, Hkv, d, seed=100 + L + G, scale_q=3.0)
        scale = 1.0 / math.sqrt(d)
        for K in (1, 2, 3):
            for W in (0, 1, 2):
                if K + W == 0:
                    continue
                idx, kth = oracle.select(q, k, cu, Hq, Hkv, K, W, scale=scale)
                for t in range(L):
                    for g in range(Hkv):
                        S = group_scores_ref(q, k, cu, Hq, Hkv, t, g, scale)
                        row = idx[t * Hkv + g]
                        cand = list(range(0, max(0, t - W + 1)))
                        sel = [int(j) for j in row if 0 <= j < t - W + 1]
                        if len(cand) <= K:
                            assert sel == cand
                            assert kth[t * Hkv + g] == -1.0
                            continue
                        best = max(sum(S[list(c)]) for c in itertools.combinations(cand, K))
                        assert len(sel) == K
                        assert abs(sum(S[sel]) - best) <= 1e-12
                        unsel = [j for j in cand if j not in sel]
                        assert min(S[sel]) >= max(S[unsel]) - 1e-15
                        assert abs(kth[t * Hkv + g] - min(S[sel])) <= 1e-15


# ----------------------------------------------------------------------------
# C3 + C4: structural invariants on ragged varlen batches.
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("K,W", [(20, 7), (1, 0), (0, 5), (64, 1)])
def test_c3_c4_structure(K, W):
    lengths, Hq, Hkv, d = [1, 5, 130, 300, 64], 4, 2, 32
    q, k, _, cu = rand_inputs(lengths, Hq, Hkv, d, seed=5)
    idx, kth = oracle.select(q, k, cu, Hq, Hkv, K, W)
    T = int(cu[-1])
    idx3 = idx.reshape(T, Hkv, K + W)
    for i, L in enumerate(lengths):
        for t in range(L):
            for g in range(Hkv):
                row = idx3[cu[i] + t, g]
                n_t = min(t + 1, K + W)
                valid = row[:n_t]
                assert (row[n_t:] == -1).all()
                assert (valid >= 0).all() and (valid <= t).all()
                assert (np.diff(valid) > 0).all()
                window = set(range(max(0, t - W + 1), t + 1))
                assert window <= set(valid.tolist())  # C3
                n_glob = sum(1 for j in valid if j < t - W + 1)
                assert n_glob == min(K, max(0, t - W + 1))


# ----------------------------------------------------------------------------
# C5: the group score sums to G over the causal keys (probabilities sum to 1).
# ----------------------------------------------------------------------------
def test_c5_group_score_sums_to_G():
    lengths, Hq, Hkv, d = [200, 77], 8, 2, 128
    q, k, _, cu = rand_inputs(lengths, Hq, Hkv, d, seed=9, scale_q=2.0)
    G = Hq // Hkv
    for tg in (0, 1, 150, 199, 200, 276):
        for g in range(Hkv):
            S, m, l = oracle.group_scores(q, k, cu, Hq, Hkv, tg, g)
            assert abs(S.sum() - G) <= 1e-12
            assert (S > 0).all()
            np.testing.assert_allclose(S, group_scores_ref(q, k, cu, Hq, Hkv, tg, g, 1 / math.sqrt(d)),
                                       rtol=1e-12, atol=1e-15)


# ----------------------------------------------------------------------------
# C6: Q = 0 makes every score equal; the tie rule (lower position first) then
# gives T_t = [0, min(K, t-W+1)) and kth = G/(t+1).
# ----------------------------------------------------------------------------
def test_c6_zero_query_tie_break():
    lengths, Hq, Hkv, d, K, W = [90, 41], 4, 2, 128, 10, 6
    q, k, _, cu = rand_inputs(lengths, Hq, Hkv, d, seed=3)
    q[:] = 0
    idx, kth = oracle.select(q, k, cu, Hq, Hkv, K, W)
    G = Hq // Hkv
    for i, L in enumerate(lengths):
        for t in range(L):
            for g in range(Hkv):
                r = (int(cu[i]) + t) * Hkv + g
                row = idx[r]
                glob = [int(j) for j in row if 0 <= j < t - W + 1]
                assert glob == list(range(min(K, max(0, t - W + 1))))
                if t - W + 1 > K:
                    assert abs(kth[r] - G / (t + 1)) <= 1e-15
                else:
                    assert kth[r] == -1.0


# ----------------------------------------------------------------------------
# C7: sparse attention equals dense attention with -inf outside the index set
# (masking before the softmax), computed with torch.softmax in fp64.
# ----------------------------------------------------------------------------
def test_c7_masked_dense_equivalence():
    lengths, Hq, Hkv, d, KW = [60, 33], 8, 2, 128, 24
    q, k, v, cu = rand_inputs(lengths, Hq, Hkv, d, seed=21)
    T = int(cu[-1])
    rng = np.random.default_rng(0)
    idx = np.full((T, Hkv, KW), -1, dtype=np.int32)
    for i, L in enumerate(lengths):
        for t in range(L):
            for g in range(Hkv):
                n = int(rng.integers(1, min(t + 1, KW) + 1))
                sel = np.sort(rng.choice(t + 1, size=n, replace=False))
                idx[cu[i] + t, g, :n] = sel
    o64, _ = oracle.sparse_attn(q, k, v, cu, Hq, Hkv, idx, want_bf16=False)
    G = Hq // Hkv
    scale = 1 / math.sqrt(d)
    for i, L in enumerate(lengths):
        a = int(cu[i])
        Kt = torch.from_numpy(bf(k[a:a + L]))
        Vt = torch.from_numpy(bf(v[a:a + L]))
        for t in range(L):
            for h in range(Hq):
                g = h // G
                mask = torch.full((L,), float("-inf"), dtype=torch.float64)
                sel = idx[a + t, g][idx[a + t, g] >= 0]
                mask[torch.from_numpy(sel.astype(np.int64))] = 0.0
                z = scale * (Kt[:, g, :] @ torch.from_numpy(bf(q[a + t, h]))) + mask
                ref = torch.softmax(z, 0) @ Vt[:, g, :]
                np.testing.assert_allclose(o64[a + t, h], ref.numpy(), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# C8: a packed varlen batch gives the per-sequence results concatenated.
# ----------------------------------------------------------------------------
def test_c8_varlen_packing_independence():
    lengths, Hq, Hkv, d, K, W = [70, 3, 129], 4, 2, 64, 16, 8
    q, k, v, cu = rand_inputs(lengths, Hq, Hkv, d, seed=8)
    idx, kth = oracle.select(q, k, cu, Hq, Hkv, K, W)
    T = int(cu[-1])
    o64, _ = oracle.sparse_attn(q, k, v, cu, Hq, Hkv, idx.reshape(T, Hkv, K + W), want_bf16=False)
    for i, L in enumerate(lengths):
        a, b = int(cu[i]), int(cu[i + 1])
        cu1 = np.array([0, L], dtype=np.int32)
        idx1, kth1 = oracle.select(q[a:b], k[a:b], cu1, Hq, Hkv, K, W)
        assert (idx1 == idx[a * Hkv:b * Hkv]).all()
        assert (kth1 == kth[a * Hkv:b * Hkv]).all()
        o1, _ = oracle.sparse_attn(q[a:b], k[a:b], v[a:b], cu1, Hq, Hkv,
                                   idx1.reshape(L, Hkv, K + W), want_bf16=False)
        assert (o1 == o64[a:b]).all()


# ----------------------------------------------------------------------------
# C9: permuting the heads within a group leaves the selection unchanged.
# ----------------------------------------------------------------------------
def test_c9_head_permutation_invariance():
    lengths, Hq, Hkv, d, K, W = [150], 8, 2, 128, 12, 4
    q, k, _, cu = rand_inputs(lengths, Hq, Hkv, d, seed=13)
    G = Hq // Hkv
    perm = np.concatenate([g * G + np.array([2, 0, 3, 1]) for g in range(Hkv)])
    qp = np.ascontiguousarray(q[:, perm, :])
    idx1, kth1 = oracle.select(q, k, cu, Hq, Hkv, K, W)
    idx2, kth2 = oracle.select(qp, k, cu, Hq, Hkv, K, W)
    assert (idx1 == idx2).all()
    for tg in (5, 80, 149):
        for g in range(Hkv):
            s1, _, _ = oracle.group_scores(q, k, cu, Hq, Hkv, tg, g)
            s2, _, _ = oracle.group_scores(qp, k, cu, Hq, Hkv, tg, g)
            assert (np.abs(s1 - s2) <= 1e-15 * np.abs(s1)).all()


# ----------------------------------------------------------------------------
# Hand-worked example with closed forms (d = 1, one head, scale 1).
# k = [0, 1, 2, 0.5], q = 1 -> z_j = k_j. At t = 3 with K = 2, W = 1:
# window {3}, candidates {0,1,2} with S_j = e^{k_j} / (1 + e + e^2 + e^0.5);
# the top-2 are {2, 1}, so I_3 = [1, 2, 3] and kth = e / (1 + e + e^2 + sqrt(e)).
# The sparse layer with q' = 1 and v = [10, 20, 30, 40] then gives
# o_3 = (20 e + 30 e^2 + 40 sqrt(e)) / (e + e^2 + sqrt(e)).
# ----------------------------------------------------------------------------
def test_hand_worked_example():
    one = synthgen.float_to_bf16(np.array([1.0]))[0]
    kv = synthgen.float_to_bf16(np.array([0.0, 1.0, 2.0, 0.5]))
    vv = synthgen.float_to_bf16(np.array([10.0, 20.0, 30.0, 40.0]))
    q = np.full((4, 1, 1), one, dtype=np.uint16)
    k = kv.reshape(4, 1, 1).astype(np.uint16)
    v = vv.reshape(4, 1, 1).astype(np.uint16)
    cu = np.array([0, 4], dtype=np.int32)
    idx, kth = oracle.select(q, k, cu, 1, 1, 2, 1, scale=1.0)
    e = math.e
    Z = 1 + e + e * e + math.sqrt(e)
    assert list(idx[3]) == [1, 2, 3]
    assert abs(kth[3] - e / Z) <= 1e-15
    # t = 2: window {2}, candidates {0,1}: both taken (|C| = 2 <= K)
    assert list(idx[2]) == [0, 1, 2] and kth[2] == -1.0
    S, m, l = oracle.group_scores(q, k, cu, 1, 1, 3, 0, scale=1.0)
    np.testing.assert_allclose(S, np.array([1, e, e * e, math.sqrt(e)]) / Z, rtol=1e-15)
    assert m[0] == 2.0
    o64, o16 = oracle.sparse_attn(q, k, v, cu, 1, 1, idx.reshape(4, 1, 3), scale=1.0)
    ref = (20 * e + 30 * e * e + 40 * math.sqrt(e)) / (e + e * e + math.sqrt(e))
    assert abs(o64[3, 0, 0] - ref) <= 1e-12
    # t = 0: only itself -> v_0
    assert o64[0, 0, 0] == 10.0


# ----------------------------------------------------------------------------
# The selection budget printed on the HySparse2 page (1024 global + 128 recent).
# ----------------------------------------------------------------------------
def test_paper_budget_structure():
    with open(os.path.join(GOLDEN, "paper_budget.json")) as f:
        cfg = json.load(f)
    K, W = cfg["K"], cfg["W"]
    L, Hq, Hkv, d = 1300, 2, 1, 16
    q, k, _, cu = rand_inputs([L], Hq, Hkv, d, seed=17)
    rows = np.array([0, 127, 128, 1150, 1151, 1152, 1299], dtype=np.int64)
    idx, kth = oracle.select(q, k, cu, Hq, Hkv, K, W, rows=rows)
    for r, t in enumerate(rows):
        valid = idx[r][idx[r] >= 0]
        assert len(valid) == min(t + 1, K + W)
        if t + 1 >= K + W:
            assert (valid[-W:] == np.arange(t - W + 1, t + 1)).all()
            assert (valid[:K] < t - W + 1).all()
            assert (kth[r] > 0) if t - W + 1 > K else (kth[r] == -1.0)
        else:
            assert (valid == np.arange(t + 1)).all()


# ----------------------------------------------------------------------------
# Regression fixture written by tests/golden/make_golden.py (oracle only).
# ----------------------------------------------------------------------------
def test_golden_regression():
    path = os.path.join(GOLDEN, "oracle_small.json")
    with open(path) as f:
        gold = json.load(f)
    w = gold["workload"]
    q, k, v, cu = rand_inputs(w["lengths"], w["Hq"], w["Hkv"], w["d"], seed=w["seed"])
    idx, kth = oracle.select(q, k, cu, w["Hq"], w["Hkv"], w["K"], w["W"])
    T = int(cu[-1])
    o64, o16 = oracle.sparse_attn(q, k, v, cu, w["Hq"], w["Hkv"], idx.reshape(T, w["Hkv"], -1))
    for r, row in gold["idx_rows"].items():
        assert idx[int(r)].tolist() == row
    for r, val in gold["kth"].items():
        assert kth[int(r)] == pytest.approx(val, rel=1e-13, abs=0)
    np.testing.assert_allclose(o64.sum(axis=(1, 2)), np.array(gold["o_token_sums"]), rtol=1e-12,
                               atol=1e-12)


def test_bf16_rounding_of_oracle_and_generator():
    """Both double->bf16 routines return the nearest bf16, ties to even (brute-force check)."""
    rng = np.random.default_rng(1)
    xs = np.concatenate([rng.normal(size=2000) * 10.0 ** rng.integers(-6, 6, 2000),
                         [0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -2.5e-39]])
    for x in xs:
        for fn in (oracle.bf16_round, synthgen.bf16_from_double):
            b = fn(float(x))
            val = float(synthgen.bf16_to_float(np.array([b], dtype=np.uint16))[0])
            lo = float(synthgen.bf16_to_float(np.array([b - 1 if b & 0x7FFF else b], dtype=np.uint16))[0])
            hi = float(synthgen.bf16_to_float(np.array([b + 1], dtype=np.uint16))[0])
            err = abs(val - x)
            assert err <= abs(lo - x) + 0.0 and err <= abs(hi - x) + 0.0, (x, b)
            if err == abs(lo - x) and lo != val or err == abs(hi - x) and hi != val:
                assert (b & 1) == 0  # tie -> even


@pytest.mark.parametrize("G", [1, 4, 8])
def test_decode_rows_equal_the_last_prefill_rows(G):
    """Decode step: the new token's query sits at the last cached position, so its
    selection and sparse output must be exactly the prefill rows of that position
    (pinned above). Checks the decode wrappers' indexing (query row, position,
    index row) on ragged cache lengths, including a one-token cache."""
    lengths = [1, 2, 7, 40, 300, 1100]
    Hkv, d, K, W = 2, 128, 16, 4
    Hq = G * Hkv
    q, k, v, cu = rand_inputs(lengths, Hq, Hkv, d, seed=90 + G)
    last = cu[1:] - 1
    rows = (last[:, None] * Hkv + np.arange(Hkv)[None, :]).ravel()
    o_idx, o_kth = oracle.select(q, k, cu, Hq, Hkv, K, W, rows=rows)
    q_dec = np.ascontiguousarray(q[last])
    d_idx, d_kth = oracle.decode_select(q_dec, k, cu, Hq, Hkv, K, W)
    assert (d_idx == o_idx).all()
    assert np.array_equal(d_kth, o_kth)
    # sparse layer with a fresh query over those index rows
    T = int(cu[-1])
    qs = synthgen.normal_bf16(91, 10, (T, Hq, d))
    full_idx = np.full((T, Hkv, K + W), -1, dtype=np.int32)
    full_idx[last] = o_idx.reshape(len(lengths), Hkv, -1)
    p64, p16 = oracle.sparse_attn(qs, k, v, cu, Hq, Hkv, full_idx, tokens=last)
    d64, d16 = oracle.decode_sparse_attn(np.ascontiguousarray(qs[last]), k, v, cu, Hq, Hkv,
                                         o_idx.reshape(len(lengths), Hkv, -1))
    assert np.array_equal(d64, p64) and np.array_equal(d16, p16)


def test_decode_rejects_empty_cache():
    q, k, v, cu = rand_inputs([3, 0, 5], 4, 1, 128, seed=3)
    with pytest.raises(ValueError):
        oracle.decode_select(q[:3], k, cu, 4, 1, 4, 2)


def test_block_size_one_is_token_selection():
    q, k, v, cu = rand_inputs([1, 30, 90, 200], 8, 2, 128, seed=21)
    a_idx, a_kth = oracle.select(q, k, cu, 8, 2, 16, 4)
    b_idx, b_kth = oracle.select(q, k, cu, 8, 2, 16, 4, block=1)
    assert (a_idx == b_idx).all() and np.array_equal(a_kth, b_kth)


@pytest.mark.parametrize("bs,K,W", [(4, 8, 3), (4, 12, 0), (5, 10, 2)])
def test_block_selection_bruteforce(bs, K, W):
    """Block mode against a brute force over block subsets: the chosen blocks are
    the subset of K/bs blocks with the largest total score (blocks cut from the
    candidates [0, t-W], scored by the sum of the pinned group score S)."""
    lengths = [3, 17, 40, 41]
    Hq, Hkv, d = 4, 2, 128
    q, k, v, cu = rand_inputs(lengths, Hq, Hkv, d, seed=22 + bs + K)
    idx, kth = oracle.select(q, k, cu, Hq, Hkv, K, W, block=bs)
    T = int(cu[-1])
    for r in range(T * Hkv):
        tg, g = divmod(r, Hkv)
        i = int(np.searchsorted(cu, tg, side="right") - 1)
        t = tg - int(cu[i])
        n_c = max(0, t - W + 1)
        window = set(range(max(0, t - W + 1), t + 1))
        if n_c <= K:
            want = set(range(n_c)) | window
            assert kth[r] == -1.0
        else:
            S, _, _ = oracle.group_scores(q, k, cu, Hq, Hkv, tg, g)
            nb = -(-n_c // bs)
            score = [S[b * bs:min((b + 1) * bs, n_c)].sum() for b in range(nb)]
            best = max(itertools.combinations(range(nb), K // bs),
                       key=lambda c: sum(score[b] for b in c))
            want = {j for b in best for j in range(b * bs, min((b + 1) * bs, n_c))} | window
            assert abs(kth[r] - min(score[b] for b in best)) <= 1e-12
        got = idx[r][idx[r] >= 0]
        assert list(got) == sorted(want), (r, t)
        assert (idx[r][len(got):] == -1).all()


def test_full_attn_against_sdpa():
    """The full layer's dense causal output equals torch SDPA (fp64, causal, GQA)
    per sequence, on the whole batch and on a token subset."""
    lengths, Hq, Hkv, d = [37, 1, 90], 8, 2, 128
    q, k, v, cu = rand_inputs(lengths, Hq, Hkv, d, seed=31)
    o64, o16 = oracle.full_attn(q, k, v, cu, Hq, Hkv)
    G = Hq // Hkv
    for i in range(len(lengths)):
        a, b = int(cu[i]), int(cu[i + 1])
        Q = torch.from_numpy(bf(q[a:b])).permute(1, 0, 2)[None]
        Kt = torch.from_numpy(bf(k[a:b])).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        Vt = torch.from_numpy(bf(v[a:b])).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, is_causal=True)
        np.testing.assert_allclose(o64[a:b], ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    toks = np.array([0, 36, 37, 38, 127])
    s64, s16 = oracle.full_attn(q, k, v, cu, Hq, Hkv, tokens=toks)
    assert np.array_equal(s64, o64[toks]) and np.array_equal(s16, o16[toks])


@pytest.mark.parametrize("block", [0, 4])
def test_oam_selection_against_numpy_ranking(block):
    """Output-aware metric: the selection equals a numpy ranking of the pinned
    group score S times max(1, |v_j|)^beta (token mode: K best by value desc,
    position asc; block mode: blocks by summed weighted score). beta = 0 is the
    plain selection. V rows are scaled so that norms straddle 1."""
    lengths, Hq, Hkv, d, K, W, beta = [40, 90], 4, 2, 128, 8, 3, 0.7
    q, k, v, cu = rand_inputs(lengths, Hq, Hkv, d, seed=41)
    T = int(cu[-1])
    scale_rows = np.exp(synthgen.normal_f64(41, 50, T * Hkv)).reshape(T, Hkv, 1) * 0.1
    v = synthgen.float_to_bf16(bf(v) * scale_rows)
    a0, k0 = oracle.select(q, k, cu, Hq, Hkv, K, W, block=block)
    b0, kb0 = oracle.select(q, k, cu, Hq, Hkv, K, W, block=block, v=v, oam_beta=0.0)
    assert (a0 == b0).all() and np.array_equal(k0, kb0)
    idx, kth = oracle.select(q, k, cu, Hq, Hkv, K, W, block=block, v=v, oam_beta=beta)
    wv = np.maximum(1.0, np.linalg.norm(bf(v), axis=2)) ** beta  # [T, Hkv]
    changed = 0
    for r in range(T * Hkv):
        tg, g = divmod(r, Hkv)
        i = int(np.searchsorted(cu, tg, side="right") - 1)
        t = tg - int(cu[i])
        n_c = max(0, t - W + 1)
        if n_c <= K:
            continue
        S, _, _ = oracle.group_scores(q, k, cu, Hq, Hkv, tg, g)
        Sw = S[:n_c] * wv[int(cu[i]):int(cu[i]) + n_c, g]
        if block:
            nb = -(-n_c // block)
            bs = np.array([Sw[b * block:(b + 1) * block].sum() for b in range(nb)])
            order = sorted(range(nb), key=lambda b: (-bs[b], b))[:K // block]
            glob = sorted(j for b in order for j in range(b * block, min((b + 1) * block, n_c)))
            ref_kth = bs[order[-1]]
        else:
            order = sorted(range(n_c), key=lambda j: (-Sw[j], j))[:K]
            glob = sorted(order)
            ref_kth = Sw[order[-1]]
        got = idx[r][(idx[r] >= 0) & (idx[r] < n_c)]
        assert list(got) == glob, r
        assert abs(kth[r] - ref_kth) <= 1e-12 * max(1.0, abs(ref_kth))
        changed += not np.array_equal(idx[r], a0[r])
    assert changed > 0  # the metric changes some selections


def _row_positions(cu, Hkv):
    """(t, L) of every row t_global * Hkv + g."""
    T = int(cu[-1])
    tg = np.arange(T * Hkv) // Hkv
    seq = np.searchsorted(cu, tg, side="right") - 1
    return tg - cu[seq], cu[seq + 1] - cu[seq]


@pytest.mark.parametrize("mu,beta", [(0.25, 0.0), (0.5, 0.0), (0.6, 0.7)])
def test_position_decay_rows_are_plain_rows_with_the_row_budget(mu, beta):
    """Position-decaying budget: the budget K_t of each row, read off its index row
    (entries below t - W + 1 are the chosen candidates, min(n_c, K_t) of them), starts
    at K on the first position of a sequence, ends at k_end = floor(mu K + 0.5) on the
    last, never grows, and stays within one token of the straight line between them;
    and every row equals the row the already pinned plain selection (or the
    output-aware one) gives with top_k = K_t, index for index and in kth."""
    lengths, Hq, Hkv, d, K, W = [300, 1, 45, 700], 4, 2, 64, 64, 16
    q, k, v, cu = rand_inputs(lengths, Hq, Hkv, d, seed=43)
    T = int(cu[-1])
    v = synthgen.float_to_bf16(bf(v) * np.exp(synthgen.normal_f64(43, 50, T * Hkv)).reshape(T, Hkv, 1) * 0.1)
    k_end = oracle.decay_k_end(K, mu)
    assert k_end == math.floor(mu * K + 0.5)
    idx, kth = oracle.select(q, k, cu, Hq, Hkv, K, W, v=v, oam_beta=beta, decay_mu=mu)
    t, L = _row_positions(cu, Hkv)
    n_c = np.maximum(0, t - W + 1)
    chosen = ((idx >= 0) & (idx < n_c[:, None])).sum(axis=1)
    # rows with more candidates than budget reveal K_t exactly
    lin = K - (K - k_end) * t / np.maximum(1, L - 1)
    full = n_c > K
    assert (chosen[full] <= np.ceil(lin[full] + 1e-9)).all() and (chosen[full] >= np.floor(lin[full])).all()
    long = (L == 700) & full
    for s in (0, 1):  # non-increasing along the sequence
        c = chosen[long][s::Hkv]
        assert (np.diff(c) <= 0).all()
    last = (L == 700) & (t == 699)
    assert (chosen[last] == k_end).all()
    # every row equals the plain selection with its own budget
    budgets = {}
    for r in np.nonzero(full)[0]:
        budgets.setdefault(int(chosen[r]), []).append(r)
    assert len(budgets) > 10
    for Kt, rows in sorted(budgets.items())[:: max(1, len(budgets) // 12)]:
        rows = np.array(rows, dtype=np.int64)
        ref, ref_kth = oracle.select(q, k, cu, Hq, Hkv, Kt, W, rows=rows, v=v, oam_beta=beta)
        got = idx[rows]
        assert (got[:, :Kt + W] == ref).all() and (got[:, Kt + W:] == -1).all()
        assert np.array_equal(kth[rows], ref_kth)
    # rows with no more candidates than the budget take them all, as in plain selection
    plain, _ = oracle.select(q, k, cu, Hq, Hkv, K, W)
    few = n_c <= k_end
    assert (idx[few] == plain[few]).all()


def test_position_decay_mu_one_is_plain_and_budget_mean():
    """mu = 1 leaves the budget at K everywhere (the plain selection); the pages keep
    the total budget of a uniform K0 when the budget decays from k_start =
    2 K0 / (1 + mu): the mean of K_t over a long sequence is then K0 to within a
    token. Block selection with a decaying budget is rejected."""
    lengths, Hq, Hkv, d, K, W = [200, 33], 2, 1, 64, 32, 8
    q, k, v, cu = rand_inputs(lengths, Hq, Hkv, d, seed=44)
    a, ka = oracle.select(q, k, cu, Hq, Hkv, K, W)
    b, kb = oracle.select(q, k, cu, Hq, Hkv, K, W, decay_mu=1.0)
    assert (a == b).all() and np.array_equal(ka, kb)
    # budget law, read from a sequence long enough for every row to be full
    L, K0, mu = 4000, 64, 0.5
    k_start = round(2 * K0 / (1 + mu))
    qq, kk, vv, cc = rand_inputs([L], 1, 1, 16, seed=45)
    idx, _ = oracle.select(qq, kk, cc, 1, 1, k_start, 0, decay_mu=mu)
    t = np.arange(L)
    chosen = ((idx >= 0)).sum(axis=1)
    Kt = chosen[t >= k_start]
    assert abs(Kt.mean() - K0) < 1.0 + 1e-9 and chosen[-1] == oracle.decay_k_end(k_start, mu)
    with pytest.raises(ValueError):
        oracle.select(q, k, cu, Hq, Hkv, K, W, block=32, decay_mu=0.5)
    with pytest.raises(ValueError):
        oracle.select(q, k, cu, Hq, Hkv, K, W, decay_mu=1.5)


# ---- FP8 KV cache: E4M3 codes against torch's float8_e4m3fn (a library routine) ----

def _torch_e4m3_codes(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_code_values_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([oracle.fp8_value(c) for c in codes])
    assert ((ref == mine) | (np.isnan(ref) & np.isnan(mine))).all()
    assert np.isnan(mine[[0x7F, 0xFF]]).all() and np.isfinite(np.delete(mine, [0x7F, 0xFF])).all()
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6


def test_fp8_encoding_rounds_to_nearest_even_and_saturates():
    """Every code value, every midpoint between neighbouring codes (ties go to the
    even code), one float32 step either side of each midpoint and random values in
    range all encode as torch does; beyond 448 the encoding saturates."""
    vals = np.array(sorted({oracle.fp8_value(c) for c in range(0x7F)}), dtype=np.float64)  # >= 0
    mids = (vals[:-1] + vals[1:]) / 2
    xs = [vals.astype(np.float32), mids.astype(np.float32),
          np.nextafter(mids.astype(np.float32), np.float32(0)),
          np.nextafter(mids.astype(np.float32), np.float32(1000))]
    rng = np.random.default_rng(7)
    xs.append((rng.uniform(-1, 1, 20000) * 448).astype(np.float32))
    xs.append((rng.uniform(-1, 1, 5000) * 2.0 ** -6).astype(np.float32))  # subnormal range
    x = np.concatenate(xs)
    x = np.concatenate([x, -x])
    assert (np.abs(x) <= 448).all()
    mine = np.array([oracle.fp8_encode(v) for v in x], dtype=np.uint8)
    ref = _torch_e4m3_codes(x)
    assert (mine == ref).all(), x[mine != ref][:5]
    # ties: the midpoint of codes n and n+1 goes to the even one
    for n in range(1, 0x7E):
        m = np.float32((oracle.fp8_value(n) + oracle.fp8_value(n + 1)) / 2)
        assert oracle.fp8_encode(m) == (n if n % 2 == 0 else n + 1)
    for v, code in ((448.5, 0x7E), (1000.0, 0x7E), (3e38, 0x7E), (-500.0, 0xFE), (float("inf"), 0x7E)):
        assert oracle.fp8_encode(v) == code
    assert oracle.fp8_encode(float("nan")) & 0x7F == 0x7F


def test_fp8_quantizer_rounds_the_float32_product():
    x = synthgen.normal_bf16(61, 1, (4096,))
    x = synthgen.float_to_bf16(bf(x) * 200.0)  # some beyond 448 at inverse scales >= 1
    for inv in (1.0, 0.37, 3.0):
        codes = oracle.quantize_fp8(x, inv)
        prod = synthgen.bf16_to_float(x).astype(np.float32) * np.float32(inv)
        ok = np.abs(prod) <= 448
        assert ok.sum() > 1000 and (inv < 1 or (~ok).sum() > 50)
        assert (codes[ok] == _torch_e4m3_codes(prod[ok])).all()
        assert (codes[~ok] == np.where(prod[~ok] > 0, 0x7E, 0xFE)).all()


def _fp8_cache(seed, shape, scale):
    """E4M3 codes of N(0, 1) values at this scale, and the same values in bf16 (exact
    when the scale is a power of two)."""
    x = synthgen.normal_bf16(seed, 9, shape)
    codes = oracle.quantize_fp8(x, 1.0 / scale)
    vals = np.vectorize(oracle.fp8_value)(codes) * scale
    return codes, synthgen.float_to_bf16(vals), vals


@pytest.mark.parametrize("G", [1, 4])
def test_fp8_sparse_attention_equals_bf16_on_exact_values(G):
    """With power-of-two scales every cached value is exact in bf16, and the FP8
    sparse attention (prefill and decode) equals the pinned bf16 one on those values
    bit for bit."""
    lengths, Hkv, d, K, W = [300, 1, 90], 2, 128, 32, 8
    Hq = G * Hkv
    q, k, v, cu = rand_inputs(lengths, Hq, Hkv, d, seed=62)
    T = int(cu[-1])
    k8, kb, _ = _fp8_cache(63, (T, Hkv, d), 0.5)
    v8, vb, _ = _fp8_cache(64, (T, Hkv, d), 4.0)
    idx, _ = oracle.select(q, kb, cu, Hq, Hkv, K, W)
    idx = idx.reshape(T, Hkv, K + W)
    a64, a16 = oracle.sparse_attn_fp8(q, k8, v8, 0.5, 4.0, cu, Hq, Hkv, idx)
    b64, b16 = oracle.sparse_attn(q, kb, vb, cu, Hq, Hkv, idx)
    assert np.array_equal(a64, b64) and np.array_equal(a16, b16)
    qd = synthgen.normal_bf16(65, 1, (len(lengths), Hq, d))
    didx, _ = oracle.decode_select(qd, kb, cu, Hq, Hkv, K, W)
    didx = didx.reshape(len(lengths), Hkv, K + W)
    c64, _ = oracle.decode_sparse_attn_fp8(qd, k8, v8, 0.5, 4.0, cu, Hq, Hkv, didx)
    e64, _ = oracle.decode_sparse_attn(qd, kb, vb, cu, Hq, Hkv, didx)
    assert np.array_equal(c64, e64)


def test_fp8_sparse_attention_against_torch_masked_softmax():
    """Arbitrary scales: the FP8 sparse output equals a float64 torch softmax over
    the dequantised keys with every unselected logit at -inf."""
    lengths, Hq, Hkv, d, K, W = [200, 50], 4, 2, 128, 16, 8
    q, k, v, cu = rand_inputs(lengths, Hq, Hkv, d, seed=66)
    T = int(cu[-1])
    ks, vs = 0.37, 1.9
    k8, _, kval = _fp8_cache(67, (T, Hkv, d), ks)
    v8, _, vval = _fp8_cache(68, (T, Hkv, d), vs)
    idx, _ = oracle.select(q, k, cu, Hq, Hkv, K, W)
    idx = idx.reshape(T, Hkv, K + W)
    toks = np.array([0, 5, 199, 200, 249])
    o64, _ = oracle.sparse_attn_fp8(q, k8, v8, ks, vs, cu, Hq, Hkv, idx, tokens=toks)
    G = Hq // Hkv
    for n, tg in enumerate(toks):
        i = int(np.searchsorted(cu, tg, side="right") - 1)
        base, t = int(cu[i]), int(tg - cu[i])
        for h in range(Hq):
            g = h // G
            sel = idx[tg, g][(idx[tg, g] >= 0) & (idx[tg, g] <= t)]
            mask = torch.full((t + 1,), -float("inf"), dtype=torch.float64)
            mask[torch.from_numpy(sel.astype(np.int64))] = 0.0
            kk = torch.from_numpy(kval[base:base + t + 1, g])
            logits = (kk @ torch.from_numpy(bf(q[tg, h]))) / np.sqrt(d) + mask
            ref = torch.softmax(logits, 0) @ torch.from_numpy(vval[base:base + t + 1, g])
            assert np.allclose(o64[n, h], ref.numpy(), rtol=1e-12, atol=1e-13)


def test_fp8_decode_selection():
    """Decode selection over an FP8 key cache: with a power-of-two scale it equals
    the pinned bf16 decode selection on the same (exactly representable) keys, bit
    for bit; with any scale it equals a numpy ranking of the group score computed
    from the dequantised keys (S desc, position asc)."""
    lengths, Hq, Hkv, d, K, W = [1, 40, 300, 97], 8, 2, 128, 24, 8
    G = Hq // Hkv
    q, k, v, cu = rand_inputs(lengths, Hq, Hkv, d, seed=71)
    T, B = int(cu[-1]), len(lengths)
    qd = synthgen.normal_bf16(72, 1, (B, Hq, d))
    k8, kb, _ = _fp8_cache(73, (T, Hkv, d), 0.25)
    a, ka = oracle.decode_select_fp8(qd, k8, 0.25, cu, Hq, Hkv, K, W)
    b, kb_ = oracle.decode_select(qd, kb, cu, Hq, Hkv, K, W)
    assert (a == b).all() and np.array_equal(ka, kb_)
    ks = 0.037
    k8, _, kval = _fp8_cache(74, (T, Hkv, d), ks)
    idx, kth = oracle.decode_select_fp8(qd, k8, ks, cu, Hq, Hkv, K, W)
    for bi in range(B):
        base, L = int(cu[bi]), int(cu[bi + 1] - cu[bi])
        t, n_c = L - 1, max(0, L - W)
        for g in range(Hkv):
            z = (bf(qd[bi, g * G:(g + 1) * G]) @ kval[base:base + L, g].T) / np.sqrt(d)
            p = np.exp(z - z.max(1, keepdims=True))
            S = (p / p.sum(1, keepdims=True)).sum(0)
            order = sorted(range(n_c), key=lambda j: (-S[j], j))
            take = order if n_c <= K else order[:K]
            want = sorted(set(take) | set(range(n_c, L)))
            row = idx[bi * Hkv + g]
            assert list(row[row >= 0]) == want
            if n_c > K:
                assert abs(kth[bi * Hkv + g] - S[order[K - 1]]) <= 1e-12


def test_oracle_results_do_not_depend_on_the_thread_count():
    """The oracle splits its rows over threads; each row is computed whole by one
    thread in a fixed order, so every result must be bit-identical for 1 and 16
    threads (selection in token, block, output-aware and decaying modes; sparse,
    full and decode attention)."""
    w = synthgen.custom([1, 37, 300, 901], Hq=8, Hkv=2, K=64, W=16, n_sparse=1, seed=404)
    inp = synthgen.make_inputs(w)
    cu = inp["cu_seqlens"]
    runs = []
    for nt in (1, 16):
        r = {}
        r["sel"] = oracle.select(inp["q_full"], inp["k"], cu, w.Hq, w.Hkv, w.K, w.W,
                                 scale=w.scale, nthreads=nt)
        r["blk"] = oracle.select(inp["q_full"], inp["k"], cu, w.Hq, w.Hkv, w.K, w.W,
                                 scale=w.scale, nthreads=nt, block=16)
        r["oam"] = oracle.select(inp["q_full"], inp["k"], cu, w.Hq, w.Hkv, w.K, w.W,
                                 scale=w.scale, nthreads=nt, v=inp["v"], oam_beta=0.7,
                                 decay_mu=0.5)
        idx = r["sel"][0].reshape(w.total, w.Hkv, -1)
        r["sp"] = oracle.sparse_attn(inp["q_sparse"][0], inp["k"], inp["v"], cu, w.Hq, w.Hkv, idx,
                                     scale=w.scale, nthreads=nt)
        r["full"] = oracle.full_attn(inp["q_full"], inp["k"], inp["v"], cu, w.Hq, w.Hkv,
                                     scale=w.scale, nthreads=nt)
        qd = inp["q_full"][cu[1:] - 1]
        r["dec"] = oracle.decode_select(qd, inp["k"], cu, w.Hq, w.Hkv, w.K, w.W, scale=w.scale,
                                        nthreads=nt)
        runs.append(r)
    for key in runs[0]:
        for a, b in zip(runs[0][key], runs[1][key]):
            assert np.array_equal(a, b), key
