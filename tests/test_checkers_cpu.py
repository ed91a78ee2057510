"""The checks the GPU parity tests rely on, shown to catch wrong index rows (CPU only).

The GPU tests judge the library's index rows with ``check_structure`` (window
present, n_t = min(t+1, K+W), ascending and unique, in [0, t], -1 padding) and with
``acceptance_select`` / ``assert_select_ok`` (A1: every selected global position
scores at least the oracle's K-th score - 1e-5; A2: overlap >= 99.9 %). Here the
oracle's own rows pass them, and copies with one planted mistake each of the kinds a
selection kernel could make must fail them.
"""
import types

import numpy as np
import pytest

import oracle
import synthgen
from hs2_testlib import acceptance_select, assert_select_ok, check_structure, local_t

LENGTHS = [40, 70]
HQ, HKV, D, K, W = 4, 2, 32, 8, 4


@pytest.fixture(scope="module")
def case():
    T = sum(LENGTHS)
    inp = {"q_full": synthgen.normal_bf16(7, 1, (T, HQ, D)),
           "k": synthgen.normal_bf16(7, 2, (T, HKV, D)),
           "cu_seqlens": np.array([0, LENGTHS[0], T], dtype=np.int32)}
    w = types.SimpleNamespace(Hq=HQ, Hkv=HKV, K=K, W=W, scale=D ** -0.5)
    idx, _ = oracle.select(inp["q_full"], inp["k"], inp["cu_seqlens"], HQ, HKV, K, W,
                           scale=w.scale)
    return inp, w, idx.reshape(T, HKV, K + W)


def _row(inp, tg):
    """A token whose rows hold a full global part: t - W + 1 > K."""
    t = int(local_t(inp["cu_seqlens"], np.array([tg]))[0])
    assert t - W + 1 > K
    return t


def test_oracle_rows_pass(case):
    inp, w, idx = case
    check_structure(idx, inp["cu_seqlens"], K, W)
    stats = acceptance_select(idx, inp, w)
    assert stats["exact_rows"] == stats["rows"]
    assert_select_ok(stats)


def _corrupt(idx, tg, g, fn):
    bad = idx.copy()
    row = bad[tg, g]
    fn(row)
    return bad


@pytest.mark.parametrize("kind", ["window", "duplicate", "order", "padding", "future",
                                  "dropped", "extra"])
def test_structure_catches_planted_mistakes(case, kind):
    inp, _, idx = case
    tg, g = LENGTHS[0] + 60, 1
    t = _row(inp, tg)
    n = K + W  # a full row

    def window(r):        # the newest window token replaced by an older candidate
        r[n - 1] = r[0] - 1 if r[0] > 0 else r[1] - 1
        r[:n] = np.sort(r[:n])

    def duplicate(r):     # one global entry repeated
        r[1] = r[0]

    def order(r):         # two global entries swapped
        r[0], r[1] = r[1], r[0]

    def padding(r):       # a short row padded with 0 instead of -1
        r[:n - 1] = r[1:n]
        r[n - 1] = 0

    def future(r):        # a position past the query
        r[n - 1] = t + 1

    def dropped(r):       # one global entry missing, the row shifted and -1 padded
        r[:n - 1] = r[1:n]
        r[n - 1] = -1

    fns = dict(window=window, duplicate=duplicate, order=order, padding=padding,
               future=future, dropped=dropped)
    if kind == "extra":
        # a row of a short prefix (t = 5 < K + W: [0, 5], then padding) with one
        # entry too many
        bad = idx.copy()
        bad[5, 0, 6] = 6
    else:
        bad = _corrupt(idx, tg, g, fns[kind])
    with pytest.raises(AssertionError):
        check_structure(bad, inp["cu_seqlens"], K, W)


def test_a1_catches_a_low_scoring_pick(case):
    inp, w, idx = case
    tg, g = LENGTHS[0] + 60, 0
    t = _row(inp, tg)
    S, _, _ = oracle.group_scores(inp["q_full"], inp["k"], inp["cu_seqlens"], HQ, HKV, tg, g,
                                  scale=w.scale)
    row = idx[tg, g]
    glob = row[(row >= 0) & (row < t - W + 1)]
    rest = np.setdiff1d(np.arange(t - W + 1), glob)
    worst = rest[np.argmin(S[rest])]
    # the lowest-scoring selected entry replaced by the lowest-scoring candidate
    new = np.sort(np.concatenate([np.delete(glob, np.argmin(S[glob])), [worst],
                                  row[(row >= t - W + 1)]]))
    bad = idx.copy()
    bad[tg, g, :len(new)] = new
    check_structure(bad, inp["cu_seqlens"], K, W)  # still a well-formed row
    stats = acceptance_select(bad, inp, w)  # every row: one changed entry keeps A2 above 99.9 %
    assert stats["overlap"] >= 0.999 and stats["a1_worst_margin"] < -1e-5
    with pytest.raises(AssertionError, match="A1"):
        assert_select_ok(stats)


def test_a2_catches_a_shifted_selection(case):
    inp, w, idx = case
    # every global entry of every row moved to the next position: well formed where
    # it stays below the window, but the sets no longer match
    bad = idx.copy()
    T = bad.shape[0]
    for tg in range(T):
        t = int(local_t(inp["cu_seqlens"], np.array([tg]))[0])
        for g in range(HKV):
            r = bad[tg, g]
            glob = (r >= 0) & (r < t - W)
            r[glob] += 1
    stats = acceptance_select(bad, inp, w)
    assert stats["overlap"] < 0.999
    with pytest.raises(AssertionError):
        assert_select_ok(stats)
