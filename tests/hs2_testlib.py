"""Helpers shared by the GPU parity tests, the smoke check and the benchmark.

GPU side: seeded inputs (synthgen) copied to the device, library calls through
the C ABI binding. Acceptance checks compare against the CPU oracle:
  A1 every GPU-selected global index j of row (t, g) has
     S_oracle[t,g,j] >= kth_oracle[t,g] - 1e-5
  A2 overlap sum |I_gpu & I_oracle| / sum |I_oracle| >= 99.9 %
  A3 bf16 sparse output vs the oracle's bf16 output on the same index sets: max-abs <= 2e-2
  A4 fp32 sparse output on identical index sets vs the oracle's fp64: max-abs <= 1e-5
plus the structural invariants of an index row (window present, n_t = min(t+1, K+W),
ascending, unique, in [0, t], -1 padded).
"""
from __future__ import annotations

import sys
import time

import numpy as np

import synthgen

A1_TOL = 1e-5
A2_MIN = 0.999
A3_TOL = 2e-2
A4_TOL = 1e-5


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev_bf16(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def from_dev_bf16(t) -> np.ndarray:
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


GUARD_BYTES = 4096
GUARD_FILL = 0xA5


class GpuCase:
    """Device copies of one workload plus the library arguments.

    Every output buffer it hands out (index rows, K-th scores, sparse outputs) sits
    between two 4 KiB guard regions filled with 0xA5; each library call made through
    the case checks afterwards that no guard byte changed (a write out of bounds)."""

    def __init__(self, w: synthgen.Workload, inputs: dict, flags: int = 0):
        import torch
        import token_level_sparse_hs2_amd as hs2
        self.w, self.inputs = w, inputs
        self.hs2 = hs2
        cu = inputs["cu_seqlens"]
        self.cu_host = [int(x) for x in cu]
        self.T = int(cu[-1])
        self.cu_dev = torch.from_numpy(cu.astype(np.int32)).cuda()
        self.q_full = to_dev_bf16(inputs["q_full"])
        self.k = to_dev_bf16(inputs["k"])
        self.v = to_dev_bf16(inputs["v"])
        self.q_sparse = [to_dev_bf16(x) for x in inputs["q_sparse"]]
        self.dims = hs2.make_dims(w.Hq, w.Hkv, w.K, w.W, w.scale, flags=flags)
        self.varlen = hs2.VarlenArgs(self.cu_dev, self.cu_host)
        nbytes = hs2.hs2_workspace_size(self.dims, self.varlen, hs2.HS2_OP_PREFILL_BLOCK,
                                        len(self.q_sparse))
        self.workspace = torch.empty(max(1, nbytes), dtype=torch.uint8, device="cuda")
        self.KW = w.K + w.W
        self._guarded = []

    def guarded_empty(self, shape, dtype):
        """An uninitialised device tensor between two guard regions (checked by check_guards)."""
        import torch
        n = 1
        for x in shape:
            n *= int(x)
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        buf = torch.full((nbytes + 2 * GUARD_BYTES,), GUARD_FILL, dtype=torch.uint8, device="cuda")
        self._guarded.append(buf)
        return buf[GUARD_BYTES:GUARD_BYTES + nbytes].view(dtype).view(*shape)

    def check_guards(self):
        import torch
        torch.cuda.synchronize()
        for buf in self._guarded:
            head, tail = buf[:GUARD_BYTES], buf[buf.numel() - GUARD_BYTES:]
            assert bool((head == GUARD_FILL).all()) and bool((tail == GUARD_FILL).all()), \
                "a library call wrote outside its output buffer"

    def new_idx(self, kw=None):
        import torch
        return self.guarded_empty((self.T, self.w.Hkv, kw or self.KW), torch.int32)

    def select(self, flags=None):
        import torch
        dims = self.dims
        if flags is not None:
            dims = self.hs2.make_dims(self.w.Hq, self.w.Hkv, self.w.K, self.w.W, self.w.scale,
                                      flags=flags)
        idx = self.new_idx()
        kth = self.guarded_empty((self.T, self.w.Hkv), torch.float32)
        self.hs2.hs2_select(dims, self.varlen, self.q_full, self.k, idx, kth, self.workspace)
        self.check_guards()
        return idx, kth

    def sparse(self, q, idx, precise=False):
        import torch
        dt = torch.float32 if precise else torch.bfloat16
        out = self.guarded_empty((self.T, self.w.Hq, self.w.d), dt)
        self.hs2.hs2_sparse_attn(self.dims, self.varlen, q, self.k, self.v, idx, out,
                                 self.hs2.HS2_OUT_F32 if precise else self.hs2.HS2_OUT_BF16)
        self.check_guards()
        return out

    def prefill_block(self, precise=False):
        import torch
        dt = torch.float32 if precise else torch.bfloat16
        outs = [self.guarded_empty((self.T, self.w.Hq, self.w.d), dt) for _ in self.q_sparse]
        idx = self.new_idx()
        self.hs2.hs2_prefill_block(self.dims, self.varlen, self.q_full, self.k, self.v,
                                   self.q_sparse, outs, idx,
                                   self.hs2.HS2_OUT_F32 if precise else self.hs2.HS2_OUT_BF16,
                                   self.workspace)
        self.check_guards()
        return idx, outs

    def release_guarded(self):
        """Drop the guarded buffers handed out so far (after a final check)."""
        self.check_guards()
        self._guarded = []


def local_t(cu: np.ndarray, tg: np.ndarray) -> np.ndarray:
    i = np.searchsorted(cu, tg, side="right") - 1
    return tg - cu[i]


def check_structure(idx: np.ndarray, cu: np.ndarray, K: int, W: int, chunk: int = 8192,
                    n_glob=None):
    """Structural invariants of every index row, in token chunks. idx [T, Hkv, K+W].
    n_glob [T, Hkv] (optional): the expected number of global entries of each row
    (default min(K, t-W+1)), e.g. the oracle's under a position-decaying budget."""
    T, Hkv, KW = idx.shape
    for a in range(0, T, chunk):
        e = min(T, a + chunk)
        _check_structure_rows(idx[a:e], local_t(cu, np.arange(a, e)), K, W,
                              None if n_glob is None else n_glob[a:e])


def _check_structure_rows(idx, tloc, K, W, n_glob=None):
    KW = idx.shape[2]
    t = tloc[:, None, None]
    tt = np.broadcast_to(tloc[:, None], idx.shape[:2])
    if n_glob is None:
        n_glob = np.minimum(K, np.maximum(0, tt - W + 1))
    n_t = (n_glob + np.minimum(W, tt + 1))[:, :, None]
    pos = np.arange(KW)[None, None, :]
    valid = np.broadcast_to(pos < n_t, idx.shape)
    assert (idx[~valid] == -1).all(), "padding must be -1"
    assert (idx[valid] >= 0).all(), "entries >= 0"
    assert (np.where(valid, idx, -1) <= t).all(), "entries <= t"
    d = np.diff(idx, axis=2)
    assert (d[valid[:, :, 1:]] > 0).all(), "ascending and unique"
    # window: the last min(W, t+1) valid entries are t-W+1 .. t
    nt = np.broadcast_to(n_t[:, :, 0], idx.shape[:2])
    for w_ in range(1, W + 1):
        need = tt - w_ + 1 >= 0
        col = np.clip(nt - w_, 0, KW - 1)
        vals = np.take_along_axis(idx, col[:, :, None], axis=2)[:, :, 0]
        assert (~need | (vals == tt - w_ + 1)).all(), f"window position t-{w_ - 1} missing"
    # global part: exactly n_glob entries below the window
    got = (np.where(valid, idx, 1 << 30) < (t - W + 1)).sum(axis=2)
    assert (got == n_glob).all(), "global count"


def sample_tokens(lengths, K, W, head=256, tail=32, stride=509):
    cu = np.concatenate([[0], np.cumsum(lengths)])
    toks = set()
    for i, L in enumerate(lengths):
        base = int(cu[i])
        for t in list(range(min(head, L))) + list(range(max(0, L - tail), L)) + \
                list(range(0, L, stride)) + [W - 1, W, K + W - 1, K + W, K + W + 1]:
            if 0 <= t < L:
                toks.add(base + t)
    return np.array(sorted(toks), dtype=np.int64)


def acceptance_select(gpu_idx: np.ndarray, inputs: dict, w, tokens=None, oracle_threads=None):
    """A1 and A2 over the rows of `tokens` (all tokens if None). Returns a stats dict."""
    import oracle
    cu = inputs["cu_seqlens"]
    T = int(cu[-1])
    Hkv = w.Hkv
    if tokens is None:
        tokens = np.arange(T, dtype=np.int64)
    rows = (tokens[:, None] * Hkv + np.arange(Hkv)[None, :]).ravel()
    t0 = time.time()
    o_idx, o_kth = oracle.select(inputs["q_full"], inputs["k"], cu, w.Hq, Hkv, w.K, w.W,
                                 scale=w.scale, rows=rows, nthreads=oracle_threads)
    t_oracle = time.time() - t0
    g_rows = gpu_idx.reshape(T * Hkv, -1)[rows]
    inter = tot = 0
    a1_worst = np.inf
    exact_rows = 0
    for r in range(len(rows)):
        a = g_rows[r][g_rows[r] >= 0]
        b = o_idx[r][o_idx[r] >= 0]
        inter += len(np.intersect1d(a, b, assume_unique=True))
        tot += len(b)
        if len(a) == len(b) and (a == b).all():
            exact_rows += 1
            continue
        # A1 on rows that differ: every selected global position scores >= kth - tol
        tg, g = int(rows[r] // Hkv), int(rows[r] % Hkv)
        t = int(local_t(cu, np.array([tg]))[0])
        S, _, _ = oracle.group_scores(inputs["q_full"], inputs["k"], cu, w.Hq, Hkv, tg, g,
                                      scale=w.scale)
        glob = a[a < t - w.W + 1]
        if len(glob):
            margin = S[glob].min() - o_kth[r]
            a1_worst = min(a1_worst, margin)
    overlap = inter / max(1, tot)
    return {"rows": len(rows), "exact_rows": exact_rows, "overlap": overlap,
            "a1_worst_margin": float(a1_worst), "oracle_s": t_oracle, "oracle_idx": o_idx,
            "oracle_kth": o_kth, "row_ids": rows}


def assert_select_ok(stats):
    assert stats["overlap"] >= A2_MIN, f"A2 overlap {stats['overlap']:.6f}"
    assert stats["a1_worst_margin"] >= -A1_TOL, f"A1 margin {stats['a1_worst_margin']:.3g}"
