"""CPU oracle for token-level sparse attention prefill -- TEST INFRASTRUCTURE ONLY.

Plain fp64 C implementation (``hs2_oracle.c``) of the selection (per-head row
statistics, group probability score, top-K outside a forced recent window,
ascending index row) and of the sparse attention over the selected positions.
Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library never calls it.

Every function here is a thin ctypes wrapper; the arithmetic is in the C file,
whose header lists the passages it follows and the readings taken where the
pages are silent.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libhs2_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile libhs2_oracle.so in-tree with gcc (plain -O2, no fast-math)."""
    src = os.path.join(_HERE, "hs2_oracle.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", src,
                               "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # HS2_ORACLE_LIB: another build of the same source (the sanitizer test's)
    path = os.environ.get("HS2_ORACLE_LIB") or _LIB_PATH
    if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(path)
    vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.hs2o_select.argtypes = [vp, vp, vp, i32, i32, i32, i32, f64, i32, i32, vp, i64, vp, vp, i32]
    lib.hs2o_select.restype = i32
    lib.hs2o_group_scores.argtypes = [vp, vp, vp, i32, i32, i32, i32, f64, i64, i32, vp, vp, vp]
    lib.hs2o_group_scores.restype = i32
    lib.hs2o_sparse_attn.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, f64, i32, vp, vp, i64,
                                     vp, vp, i32]
    lib.hs2o_sparse_attn.restype = i32
    lib.hs2o_select_blocks.argtypes = [vp, vp, vp, i32, i32, i32, i32, f64, i32, i32, i32, vp,
                                       i64, vp, vp, i32]
    lib.hs2o_select_blocks.restype = i32
    lib.hs2o_select_ex.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, f64, i32, i32, i32, f64, i32,
                                    vp, i64, vp, vp, i32]
    lib.hs2o_select_ex.restype = i32
    lib.hs2o_full_attn.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, f64, vp, i64, vp, vp, i32]
    lib.hs2o_full_attn.restype = i32
    lib.hs2o_decode_select.argtypes = [vp, vp, vp, i32, i32, i32, i32, f64, i32, i32, vp, vp, i32]
    lib.hs2o_decode_select.restype = i32
    lib.hs2o_decode_sparse_attn.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, f64, i32, vp, vp,
                                            vp, i32]
    lib.hs2o_decode_sparse_attn.restype = i32
    lib.hs2o_bf16_round.argtypes = [f64]
    lib.hs2o_bf16_round.restype = ctypes.c_uint16
    lib.hs2o_fp8_value.argtypes = [ctypes.c_uint8]
    lib.hs2o_fp8_value.restype = f64
    lib.hs2o_fp8_encode.argtypes = [ctypes.c_float]
    lib.hs2o_fp8_encode.restype = ctypes.c_uint8
    lib.hs2o_quantize_fp8.argtypes = [vp, vp, i64, ctypes.c_float]
    lib.hs2o_quantize_fp8.restype = i32
    lib.hs2o_sparse_attn_fp8.argtypes = [vp, vp, vp, f64, f64, vp, i32, i32, i32, i32, f64, i32, vp,
                                         vp, i64, vp, vp, i32]
    lib.hs2o_sparse_attn_fp8.restype = i32
    lib.hs2o_decode_sparse_attn_fp8.argtypes = [vp, vp, vp, f64, f64, vp, i32, i32, i32, i32, f64,
                                                i32, vp, vp, vp, i32]
    lib.hs2o_decode_sparse_attn_fp8.restype = i32
    lib.hs2o_decode_select_fp8.argtypes = [vp, vp, f64, vp, i32, i32, i32, i32, f64, i32, i32, vp,
                                           vp, i32]
    lib.hs2o_decode_select_fp8.restype = i32
    _lib = lib
    return lib


def default_threads() -> int:
    return max(1, min(64, os.cpu_count() or 1))


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, "bf16 tensors are passed as uint16 bit patterns"
    return a


def _cu(cu):
    return np.ascontiguousarray(np.asarray(cu, dtype=np.int32))


def decay_k_end(K, decay_mu):
    """Budget at a sequence's last position for the position-decaying budget:
    k_end = floor(mu * K + 0.5), mu taken as a 32-bit float (as callers pass it);
    mu = 0 means no decay (k_end = K)."""
    if not decay_mu:
        return K
    mu = float(np.float32(decay_mu))
    if not 0.0 < mu <= 1.0:
        raise ValueError("decay_mu must lie in (0, 1]")
    return int(math.floor(mu * K + 0.5))


def select(q, k, cu_seqlens, Hq, Hkv, K, W, scale=None, rows=None, nthreads=None, block=0,
           v=None, oam_beta=0.0, decay_mu=0.0):
    """Index rows and K-th scores.

    q [T,Hq,d], k [T,Hkv,d] bf16 bits; rows: None (all T*Hkv rows, row id = t*Hkv+g)
    or an int64 array of row ids. block > 0 selects aligned blocks of that many
    candidate tokens (K a multiple of block) by the sum of S over the block; kth is
    then the lowest selected block's score. oam_beta > 0 (needs v [T,Hkv,d]) ranks by the
    output-aware metric S_j * max(1, |v_j|_2)^oam_beta. decay_mu in (0, 1] gives the
    position-decaying budget: position t of a sequence of L tokens keeps
    K - floor((K - k_end) t / (L - 1)) candidates, k_end = decay_k_end(K, decay_mu)
    (token selection only). Returns (idx [n, K+W] int32, kth [n] float64).
    """
    lib = _load()
    q, k, cu = _u16(q), _u16(k), _cu(cu_seqlens)
    d = q.shape[-1]
    B = len(cu) - 1
    T = int(cu[-1])
    scale = float(scale if scale is not None else 1.0 / np.sqrt(d))
    if rows is not None:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = len(rows)
    else:
        n = T * Hkv
    idx = np.empty((n, K + W), dtype=np.int32)
    kth = np.empty(n, dtype=np.float64)
    if n == 0:
        return idx, kth
    if oam_beta or decay_mu:
        v = _u16(v) if oam_beta else None
        r = lib.hs2o_select_ex(q.ctypes.data, k.ctypes.data, v.ctypes.data if v is not None else None,
                               cu.ctypes.data, B, Hq, Hkv, d, scale, K, W, int(block),
                               float(oam_beta), decay_k_end(K, decay_mu),
                               rows.ctypes.data if rows is not None else None, n, idx.ctypes.data,
                               kth.ctypes.data, nthreads or default_threads())
    else:
        r = lib.hs2o_select_blocks(q.ctypes.data, k.ctypes.data, cu.ctypes.data, B, Hq, Hkv, d,
                                   scale, K, W, int(block),
                                   rows.ctypes.data if rows is not None else None, n,
                                   idx.ctypes.data, kth.ctypes.data, nthreads or default_threads())
    if r != 0:
        raise ValueError("hs2o_select: bad arguments")
    return idx, kth


def group_scores(q, k, cu_seqlens, Hq, Hkv, t_global, g, scale=None):
    """(S [t+1], m [G], l [G]) of row (t_global, g): group score over causal keys and head stats."""
    lib = _load()
    q, k, cu = _u16(q), _u16(k), _cu(cu_seqlens)
    d = q.shape[-1]
    B = len(cu) - 1
    i = int(np.searchsorted(cu, t_global, side="right") - 1)
    t = int(t_global - cu[i])
    G = Hq // Hkv
    S = np.empty(t + 1, dtype=np.float64)
    m = np.empty(G, dtype=np.float64)
    l = np.empty(G, dtype=np.float64)
    scale = float(scale if scale is not None else 1.0 / np.sqrt(d))
    r = lib.hs2o_group_scores(q.ctypes.data, k.ctypes.data, cu.ctypes.data, B, Hq, Hkv, d, scale,
                              int(t_global), int(g), S.ctypes.data, m.ctypes.data, l.ctypes.data)
    if r != 0:
        raise ValueError("hs2o_group_scores: bad arguments")
    return S, m, l


def sparse_attn(q, k, v, cu_seqlens, Hq, Hkv, idx, scale=None, tokens=None, nthreads=None,
                want_f64=True, want_bf16=True):
    """Sparse attention over idx rows. idx [T, Hkv, KW] int32 (local positions, -1 = none).

    Returns (o64 [n,Hq,d] float64 or None, o16 [n,Hq,d] bf16 bits or None).
    """
    lib = _load()
    q, k, v, cu = _u16(q), _u16(k), _u16(v), _cu(cu_seqlens)
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    d = q.shape[-1]
    B = len(cu) - 1
    T = int(cu[-1])
    KW = idx.shape[-1]
    assert idx.size == T * Hkv * KW
    scale = float(scale if scale is not None else 1.0 / np.sqrt(d))
    if tokens is not None:
        tokens = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
        n = len(tokens)
    else:
        n = T
    o64 = np.empty((n, Hq, d), dtype=np.float64) if want_f64 else None
    o16 = np.empty((n, Hq, d), dtype=np.uint16) if want_bf16 else None
    if n == 0:
        return o64, o16
    r = lib.hs2o_sparse_attn(q.ctypes.data, k.ctypes.data, v.ctypes.data, cu.ctypes.data, B, Hq,
                             Hkv, d, scale, KW, idx.ctypes.data,
                             tokens.ctypes.data if tokens is not None else None, n,
                             o64.ctypes.data if o64 is not None else None,
                             o16.ctypes.data if o16 is not None else None,
                             nthreads or default_threads())
    if r != 0:
        raise ValueError("hs2o_sparse_attn: bad arguments")
    return o64, o16


def full_attn(q, k, v, cu_seqlens, Hq, Hkv, scale=None, tokens=None, nthreads=None,
              want_f64=True, want_bf16=True):
    """The full layer's dense causal attention output over [0, t] for `tokens`
    (None = all T). Returns (o64 [n,Hq,d] float64 or None, o16 [n,Hq,d] bf16 bits or None)."""
    lib = _load()
    q, k, v, cu = _u16(q), _u16(k), _u16(v), _cu(cu_seqlens)
    d = q.shape[-1]
    B = len(cu) - 1
    T = int(cu[-1])
    scale = float(scale if scale is not None else 1.0 / np.sqrt(d))
    if tokens is not None:
        tokens = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
        n = len(tokens)
    else:
        n = T
    o64 = np.empty((n, Hq, d), dtype=np.float64) if want_f64 else None
    o16 = np.empty((n, Hq, d), dtype=np.uint16) if want_bf16 else None
    if n == 0:
        return o64, o16
    r = lib.hs2o_full_attn(q.ctypes.data, k.ctypes.data, v.ctypes.data, cu.ctypes.data, B, Hq, Hkv,
                           d, scale, tokens.ctypes.data if tokens is not None else None, n,
                           o64.ctypes.data if o64 is not None else None,
                           o16.ctypes.data if o16 is not None else None,
                           nthreads or default_threads())
    if r != 0:
        raise ValueError("hs2o_full_attn: bad arguments")
    return o64, o16


def decode_select(q_dec, k, cu_seqlens, Hq, Hkv, K, W, scale=None, nthreads=None):
    """Decode-step selection: one query per sequence at its last cached position.

    q_dec [B,Hq,d], k [T,Hkv,d] bf16 bits; cu_seqlens describes the cache (every
    sequence holds >= 1 token). Returns (idx [B*Hkv, K+W] int32, kth [B*Hkv] float64),
    row b*Hkv + g.
    """
    lib = _load()
    q_dec, k, cu = _u16(q_dec), _u16(k), _cu(cu_seqlens)
    d = q_dec.shape[-1]
    B = len(cu) - 1
    assert q_dec.size == B * Hq * d
    scale = float(scale if scale is not None else 1.0 / np.sqrt(d))
    idx = np.empty((B * Hkv, K + W), dtype=np.int32)
    kth = np.empty(B * Hkv, dtype=np.float64)
    if B == 0:
        return idx, kth
    r = lib.hs2o_decode_select(q_dec.ctypes.data, k.ctypes.data, cu.ctypes.data, B, Hq, Hkv, d,
                               scale, K, W, idx.ctypes.data, kth.ctypes.data,
                               nthreads or default_threads())
    if r != 0:
        raise ValueError("hs2o_decode_select: bad arguments")
    return idx, kth


def decode_sparse_attn(q_dec, k, v, cu_seqlens, Hq, Hkv, idx, scale=None, nthreads=None,
                       want_f64=True, want_bf16=True):
    """Sparse attention of the decode queries q_dec [B,Hq,d] over idx [B,Hkv,KW].

    Returns (o64 [B,Hq,d] float64 or None, o16 [B,Hq,d] bf16 bits or None).
    """
    lib = _load()
    q_dec, k, v, cu = _u16(q_dec), _u16(k), _u16(v), _cu(cu_seqlens)
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    d = q_dec.shape[-1]
    B = len(cu) - 1
    KW = idx.shape[-1]
    assert idx.size == B * Hkv * KW and q_dec.size == B * Hq * d
    scale = float(scale if scale is not None else 1.0 / np.sqrt(d))
    o64 = np.empty((B, Hq, d), dtype=np.float64) if want_f64 else None
    o16 = np.empty((B, Hq, d), dtype=np.uint16) if want_bf16 else None
    if B == 0:
        return o64, o16
    r = lib.hs2o_decode_sparse_attn(q_dec.ctypes.data, k.ctypes.data, v.ctypes.data,
                                    cu.ctypes.data, B, Hq, Hkv, d, scale, KW, idx.ctypes.data,
                                    o64.ctypes.data if o64 is not None else None,
                                    o16.ctypes.data if o16 is not None else None,
                                    nthreads or default_threads())
    if r != 0:
        raise ValueError("hs2o_decode_sparse_attn: bad arguments")
    return o64, o16


def bf16_round(x: float) -> int:
    return int(_load().hs2o_bf16_round(float(x)))


# ---- FP8 KV cache (E4M3 codes, one fp32 scale per tensor) ----

def fp8_value(code: int) -> float:
    """Value of an E4M3 code (nan for the NaN codes)."""
    return float(_load().hs2o_fp8_value(int(code) & 0xFF))


def fp8_encode(x: float) -> int:
    """Nearest E4M3 code of a float32 value (ties to even, saturating at +-448)."""
    return int(_load().hs2o_fp8_encode(float(x)))


def quantize_fp8(x, inv_scale: float):
    """E4M3 codes of bf16 bits x: code = E4M3(float32(x) * float32(inv_scale))."""
    x = _u16(x)
    out = np.empty(x.shape, dtype=np.uint8)
    if _load().hs2o_quantize_fp8(x.ctypes.data, out.ctypes.data, x.size, float(inv_scale)):
        raise ValueError("hs2o_quantize_fp8: bad arguments")
    return out


def _u8(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint8, "FP8 tensors are passed as uint8 codes"
    return a


def sparse_attn_fp8(q, k8, v8, k_scale, v_scale, cu_seqlens, Hq, Hkv, idx, scale=None,
                    tokens=None, nthreads=None, want_f64=True, want_bf16=True):
    """sparse_attn over an FP8 cache: k = k_scale * E4M3(k8), v = v_scale * E4M3(v8)."""
    lib = _load()
    q, k8, v8, cu = _u16(q), _u8(k8), _u8(v8), _cu(cu_seqlens)
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    d = q.shape[-1]
    B = len(cu) - 1
    T = int(cu[-1])
    KW = idx.shape[-1]
    assert idx.size == T * Hkv * KW
    scale = float(scale if scale is not None else 1.0 / np.sqrt(d))
    if tokens is not None:
        tokens = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
        n = len(tokens)
    else:
        n = T
    o64 = np.empty((n, Hq, d), dtype=np.float64) if want_f64 else None
    o16 = np.empty((n, Hq, d), dtype=np.uint16) if want_bf16 else None
    if n == 0:
        return o64, o16
    r = lib.hs2o_sparse_attn_fp8(q.ctypes.data, k8.ctypes.data, v8.ctypes.data, float(k_scale),
                                 float(v_scale), cu.ctypes.data, B, Hq, Hkv, d, scale, KW,
                                 idx.ctypes.data, tokens.ctypes.data if tokens is not None else None,
                                 n, o64.ctypes.data if o64 is not None else None,
                                 o16.ctypes.data if o16 is not None else None,
                                 nthreads or default_threads())
    if r != 0:
        raise ValueError("hs2o_sparse_attn_fp8: bad arguments")
    return o64, o16


def decode_sparse_attn_fp8(q_dec, k8, v8, k_scale, v_scale, cu_seqlens, Hq, Hkv, idx, scale=None,
                           nthreads=None, want_f64=True, want_bf16=True):
    """decode_sparse_attn over an FP8 cache."""
    lib = _load()
    q_dec, k8, v8, cu = _u16(q_dec), _u8(k8), _u8(v8), _cu(cu_seqlens)
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    d = q_dec.shape[-1]
    B = len(cu) - 1
    KW = idx.shape[-1]
    assert idx.size == B * Hkv * KW and q_dec.size == B * Hq * d
    scale = float(scale if scale is not None else 1.0 / np.sqrt(d))
    o64 = np.empty((B, Hq, d), dtype=np.float64) if want_f64 else None
    o16 = np.empty((B, Hq, d), dtype=np.uint16) if want_bf16 else None
    if B == 0:
        return o64, o16
    r = lib.hs2o_decode_sparse_attn_fp8(q_dec.ctypes.data, k8.ctypes.data, v8.ctypes.data,
                                        float(k_scale), float(v_scale), cu.ctypes.data, B, Hq, Hkv,
                                        d, scale, KW, idx.ctypes.data,
                                        o64.ctypes.data if o64 is not None else None,
                                        o16.ctypes.data if o16 is not None else None,
                                        nthreads or default_threads())
    if r != 0:
        raise ValueError("hs2o_decode_sparse_attn_fp8: bad arguments")
    return o64, o16


def decode_select_fp8(q_dec, k8, k_scale, cu_seqlens, Hq, Hkv, K, W, scale=None, nthreads=None):
    """decode_select over an FP8 key cache: k = k_scale * E4M3(k8)."""
    lib = _load()
    q_dec, k8, cu = _u16(q_dec), _u8(k8), _cu(cu_seqlens)
    d = q_dec.shape[-1]
    B = len(cu) - 1
    assert q_dec.size == B * Hq * d
    scale = float(scale if scale is not None else 1.0 / np.sqrt(d))
    idx = np.empty((B * Hkv, K + W), dtype=np.int32)
    kth = np.empty(B * Hkv, dtype=np.float64)
    if B == 0:
        return idx, kth
    r = lib.hs2o_decode_select_fp8(q_dec.ctypes.data, k8.ctypes.data, float(k_scale), cu.ctypes.data,
                                   B, Hq, Hkv, d, scale, K, W, idx.ctypes.data, kth.ctypes.data,
                                   nthreads or default_threads())
    if r != 0:
        raise ValueError("hs2o_decode_select_fp8: bad arguments")
    return idx, kth
