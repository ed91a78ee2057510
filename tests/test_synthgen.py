"""The shared seeded input generator: determinism, distribution, needles, varlen draw."""
import math

import numpy as np

import synthgen


def test_deterministic_and_chunk_independent():
    a = synthgen.normal_bf16(5, 1, (1000, 3))
    b = synthgen.normal_bf16(5, 1, (1000, 3))
    assert (a == b).all()
    # element e of the stream does not depend on where a request starts
    c = synthgen.normal_bf16(5, 1, (1,), start=1777)
    assert c[0] == a.ravel()[1777]
    tail = synthgen.normal_bf16(5, 1, (1000,), start=2000)
    assert (tail == a.ravel()[2000:]).all()
    assert not (synthgen.normal_bf16(6, 1, (100,)) == a.ravel()[:100]).all()
    assert not (synthgen.normal_bf16(5, 2, (100,)) == a.ravel()[:100]).all()


def test_large_threaded_fill_matches_serial_prefix():
    big = synthgen.normal_bf16(9, 4, (300000,))
    small = synthgen.normal_bf16(9, 4, (1000,), start=150000)
    assert (big[150000:151000] == small).all()


def test_normal_moments():
    x = synthgen.normal_f64(1, 1, 400000)
    assert abs(x.mean()) < 0.01
    assert abs(x.std() - 1.0) < 0.01
    assert abs((x > 1.96).mean() - 0.025) < 0.002


def test_needles_structure():
    L, Hq, Hkv, d, W = 2048, 4, 2, 128, 128
    q = synthgen.normal_bf16(3, 1, (L, Hq, d))
    k = synthgen.normal_bf16(3, 2, (L, Hkv, d))
    k0 = k.copy()
    pos = synthgen.add_needles(q, k, Hq, Hkv, d, W, seed=3)
    assert pos.shape == (Hkv, 3, 16)
    G = Hq // Hkv
    for g in range(Hkv):
        p = pos[g][pos[g] >= 0]
        assert len(set(p.tolist())) == len(p) == 48
        for b in range(1, 4):
            pb = pos[g, b - 1]
            assert (pb >= 0).all() and (pb < 512 * b - W).all()
            u = synthgen.bf16_to_float(q[512 * b:512 * (b + 1), g * G:(g + 1) * G]).astype(np.float64)
            u = u.sum(axis=(0, 1))
            u /= np.linalg.norm(u)
            kn = synthgen.bf16_to_float(k[pb, g]).astype(np.float64)
            # needle = 3 sqrt(d) u + N(0, I): projection on u is about 3 sqrt(d)
            proj = kn @ u
            assert (np.abs(proj - 3 * math.sqrt(d)) < 5).all()
        untouched = np.setdiff1d(np.arange(L), p)
        assert (k[untouched, g] == k0[untouched, g]).all()


def test_varlen_lengths_draw():
    L, s = synthgen.varlen_lengths(1005)
    assert len(L) == 8 and sum(L) <= 600 * 1024
    assert all(4096 <= x <= 196608 for x in L)
    assert synthgen.varlen_lengths(1005) == (L, s)


def test_decode_inputs_are_the_last_prefill_rows():
    w = synthgen.custom([1, 5, 300], 8, 2, 16, 4, n_sparse=2, seed=5)
    a, b = synthgen.make_inputs(w), synthgen.make_decode_inputs(w)
    last = w.cu_seqlens[1:] - 1
    assert (a["q_full"][last] == b["q_dec"]).all()
    assert (a["k"] == b["k"]).all() and (a["v"] == b["v"]).all()
    for x, y in zip(a["q_sparse"], b["q_sparse_dec"]):
        assert (x[last] == y).all()
