"""Seeded synthetic inputs shared by the CPU oracle tests and the GPU library.

This package holds none of the attention method's arithmetic: it produces
input bytes only (bf16 N(0,1) tensors, needle keys, varlen lengths) so that the
oracle and the HIP path consume identical data. The generator is counter-based
SplitMix64 + Box-Muller, implemented in ``synthgen.c``.

Workload presets follow the five evaluation shapes of this path:
  tiny    B=1, L=1024,  Hq=4,  Hkv=1, K=256,  W=32,  1 sparse layer
  8k      B=1, L=8192,  Hq=32, Hkv=8, K=1024, W=128, 1 sparse layer
  32k     B=1, L=32768, Hq=32, Hkv=8, K=1024, W=128, needles, 3 sparse layers
  128k    B=1, L=131072, Hq=64, Hkv=8, K=1024, W=128, needles, 3 sparse layers
  varlen  B=8, lognormal lengths (median 48k, clipped to [4k, 192k], total <= 600k),
          Hq=32, Hkv=8, K=1024, W=128, 1 sparse layer
K=1024 global tokens and W=128 forced recent tokens are the selection budget the
HySparse2 news summary (MiMo-V3 architecture story) gives in its
token-granularity paragraph.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynthgen.so")
_lib = None

# tensor ids of the streams (the seed selects the workload)
TID_Q_FULL = 1
TID_K = 2
TID_V = 3
TID_Q_SPARSE0 = 10  # sparse layer l uses TID_Q_SPARSE0 + l
TID_NEEDLE_POS = 20
TID_NEEDLE_EPS = 21
TID_VARLEN = 30


def build(force: bool = False) -> str:
    """Compile libsynthgen.so in-tree with gcc."""
    src = os.path.join(_HERE, "synthgen.c")
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
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i64, i32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int
    vp = ctypes.c_void_p
    lib.sg_normal_bf16.argtypes = [u64, u64, u64, u64, vp, i32]
    lib.sg_normal_bf16.restype = None
    lib.sg_normal_f64.argtypes = [u64, u64, u64, u64, vp, i32]
    lib.sg_normal_f64.restype = None
    lib.sg_bf16_from_double.argtypes = [ctypes.c_double]
    lib.sg_bf16_from_double.restype = ctypes.c_uint16
    lib.sg_stream_key.argtypes = [u64, u64]
    lib.sg_stream_key.restype = u64
    lib.sg_u64.argtypes = [u64, u64]
    lib.sg_u64.restype = u64
    lib.sg_add_needles.argtypes = [vp, vp, i64, i32, i32, i32, i32, i32, i32, ctypes.c_double,
                                   u64, u64, u64, vp]
    lib.sg_add_needles.restype = i64
    _lib = lib
    return lib


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_bf16(seed: int, tensor_id: int, shape, start: int = 0) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(0,1) stream elements [start, start+prod(shape))."""
    lib = _load()
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint16)
    if n:
        lib.sg_normal_bf16(seed, tensor_id, start, n, out.ctypes.data, _threads())
    return out.reshape(shape)


def normal_f64(seed: int, tensor_id: int, n: int, start: int = 0) -> np.ndarray:
    lib = _load()
    out = np.empty(n, dtype=np.float64)
    if n:
        lib.sg_normal_f64(seed, tensor_id, start, n, out.ctypes.data, _threads())
    return out


def bf16_from_double(x: float) -> int:
    return int(_load().sg_bf16_from_double(float(x)))


def bf16_to_float(a: np.ndarray) -> np.ndarray:
    """bf16 bits (uint16) -> float32 values (exact)."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def float_to_bf16(x: np.ndarray) -> np.ndarray:
    """float64/float32 values -> bf16 bits, round to nearest even (via the C routine)."""
    lib = _load()
    flat = np.asarray(x, dtype=np.float64).ravel()
    out = np.empty(flat.shape, dtype=np.uint16)
    for i, v in enumerate(flat):
        out[i] = lib.sg_bf16_from_double(float(v))
    return out.reshape(np.shape(x))


def add_needles(q: np.ndarray, k: np.ndarray, Hq: int, Hkv: int, d: int, W: int, seed: int,
                block: int = 512, per_block: int = 16, mag_over_sqrt_d: float = 3.0) -> np.ndarray:
    """Plant needle keys in k (in place) for one sequence; returns their positions [Hkv, nblk, per_block]."""
    lib = _load()
    assert q.dtype == np.uint16 and k.dtype == np.uint16
    assert q.flags.c_contiguous and k.flags.c_contiguous
    L = k.shape[0]
    nblk = (L + block - 1) // block
    pos = np.full((Hkv, nblk - 1 if nblk > 1 else 0, per_block), -1, dtype=np.int32)
    r = lib.sg_add_needles(q.ctypes.data, k.ctypes.data, L, Hq, Hkv, d, block, per_block, W,
                           mag_over_sqrt_d * math.sqrt(d), seed, TID_NEEDLE_POS, TID_NEEDLE_EPS,
                           pos.ctypes.data if pos.size else None)
    if r < 0:
        raise ValueError("sg_add_needles: bad arguments")
    return pos


def varlen_lengths(seed: int, batch: int = 8, median: int = 48 * 1024, lo: int = 4 * 1024,
                   hi: int = 192 * 1024, total_max: int = 600 * 1024, max_attempts: int = 1000):
    """Lognormal lengths clip(round(exp(N(ln median, s^2))), lo, hi), s = sqrt(2 ln(68/48)).

    s makes the unclipped mean 68k for a 48k median (mean = median * exp(s^2/2)).
    All `batch` lengths are redrawn with the next seed until their total <= total_max.
    Returns (lengths, seed_used).
    """
    sigma = math.sqrt(2.0 * math.log(68.0 / 48.0))
    for a in range(max_attempts):
        z = normal_f64(seed + a, TID_VARLEN, batch)
        L = [int(min(hi, max(lo, round(math.exp(math.log(median) + sigma * zi))))) for zi in z]
        if sum(L) <= total_max:
            return L, seed + a
    raise RuntimeError("varlen_lengths: no draw under total_max")


@dataclass
class Workload:
    name: str
    lengths: list
    Hq: int
    Hkv: int
    d: int
    K: int
    W: int
    n_sparse: int
    needles: bool
    seed: int
    meta: dict = field(default_factory=dict)

    @property
    def total(self) -> int:
        return int(sum(self.lengths))

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int32)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


def workload(name: str) -> Workload:
    """The five named workloads; seed = 1000 + index (1-based)."""
    if name == "tiny":
        return Workload("tiny", [1024], 4, 1, 128, 256, 32, 1, False, 1001)
    if name == "8k":
        return Workload("8k", [8192], 32, 8, 128, 1024, 128, 1, False, 1002)
    if name == "32k":
        return Workload("32k", [32768], 32, 8, 128, 1024, 128, 3, True, 1003)
    if name == "128k":
        return Workload("128k", [131072], 64, 8, 128, 1024, 128, 3, True, 1004)
    if name == "varlen":
        L, s = varlen_lengths(1005)
        return Workload("varlen", L, 32, 8, 128, 1024, 128, 1, False, 1005, {"length_seed": s})
    raise KeyError(name)


def custom(lengths, Hq, Hkv, K, W, n_sparse=1, seed=7, d=128, needles=False) -> Workload:
    return Workload("custom", list(lengths), Hq, Hkv, d, K, W, n_sparse, needles, seed)


def make_inputs(w: Workload) -> dict:
    """bf16 bit arrays: q_full [T,Hq,d], k/v [T,Hkv,d], q_sparse list of [T,Hq,d]; cu_seqlens int32.

    Every tensor is one stream over the packed [T, H, d] layout. With needles,
    each sequence gets its needles from its own slice (only B=1 workloads use them).
    """
    T = w.total
    q_full = normal_bf16(w.seed, TID_Q_FULL, (T, w.Hq, w.d))
    k = normal_bf16(w.seed, TID_K, (T, w.Hkv, w.d))
    v = normal_bf16(w.seed, TID_V, (T, w.Hkv, w.d))
    q_sparse = [normal_bf16(w.seed, TID_Q_SPARSE0 + l, (T, w.Hq, w.d)) for l in range(w.n_sparse)]
    out = {"q_full": q_full, "k": k, "v": v, "q_sparse": q_sparse, "cu_seqlens": w.cu_seqlens}
    if w.needles:
        cu = w.cu_seqlens
        pos = []
        for i in range(len(w.lengths)):
            a, b = int(cu[i]), int(cu[i + 1])
            qs = np.ascontiguousarray(q_full[a:b])
            ks = np.ascontiguousarray(k[a:b])
            pos.append(add_needles(qs, ks, w.Hq, w.Hkv, w.d, w.W, w.seed + 7919 * i))
            k[a:b] = ks
        out["needle_pos"] = pos
    return out


def decode_workload(name: str) -> Workload:
    """Decode-step workloads (the lengths are the cache lengths; one new query per sequence)."""
    if name == "decode-32k":
        return Workload("decode-32k", [32768] * 8, 32, 8, 128, 1024, 128, 3, False, 1101)
    if name == "decode-varlen":
        L, s = varlen_lengths(1005)
        return Workload("decode-varlen", L, 32, 8, 128, 1024, 128, 1, False, 1102,
                        {"length_seed": s})
    raise KeyError(name)


def make_decode_inputs(w: Workload) -> dict:
    """Decode step over a cache of w.lengths tokens per sequence: k/v [T,Hkv,d] (as in
    make_inputs), q_dec [B,Hq,d] and q_sparse_dec list of [B,Hq,d] = the rows of the
    q_full / q_sparse streams at each sequence's last position (generated directly, so a
    decode step equals the last prefill row of the same inputs). No needles."""
    assert not w.needles, "decode inputs carry no needles"
    T = w.total
    cu = w.cu_seqlens
    last = [int(x) - 1 for x in cu[1:]]
    assert all(cu[i + 1] > cu[i] for i in range(len(w.lengths))), "every cache holds >= 1 token"
    row = w.Hq * w.d

    def rows(tid):
        return np.stack([normal_bf16(w.seed, tid, (w.Hq, w.d), start=t * row) for t in last])

    return {"k": normal_bf16(w.seed, TID_K, (T, w.Hkv, w.d)),
            "v": normal_bf16(w.seed, TID_V, (T, w.Hkv, w.d)),
            "q_dec": rows(TID_Q_FULL),
            "q_sparse_dec": [rows(TID_Q_SPARSE0 + l) for l in range(w.n_sparse)],
            "cu_seqlens": cu}

