"""Token-level sparse attention prefill (HySparse2-style) on AMD Instinct MI355X.

Thin Python binding of the C ABI in ``include/hs2.h`` (library ``libhs2.so``,
hand-written HIP kernels for gfx950). Functions carry the ABI's names and only
marshal arguments: torch tensors are passed as raw device pointers, the stream
is torch's current HIP stream unless one is given. Every step of the path runs
in the library's kernels; there is no fallback. If the library is missing the
import of any entry point raises.

Layouts (token-major over a packed varlen batch, T tokens; the decode calls take
one query row per sequence, [B, ...], against the cache described by cu_seqlens):
  q, q_sparse, out  [T, Hq, 128]   bf16 (out: bf16 or float32)
  k, v              [T, Hkv, 128]  bf16
  idx               [T, Hkv, K+W]  int32, local positions ascending, -1 padded
  cu_seqlens        [B+1] int32 on the device, plus its host copy
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
# HS2_LIBRARY: another build of the library (e.g. the host-sanitizer build of its C ABI)
LIB_PATH = os.environ.get("HS2_LIBRARY") or os.path.join(_PKG, "libhs2.so")

HS2_OK = 0
HS2_ERR_INVALID_ARG = -1
HS2_ERR_UNSUPPORTED = -2
HS2_ERR_WORKSPACE = -3
HS2_ERR_HIP = -4
HS2_ERR_SCRATCH = -5
HS2_NOALLOC_SCRATCH_BYTES = 20 << 20
HS2_OUT_BF16 = 0
HS2_OUT_F32 = 1
HS2_OP_SELECT = 1
HS2_OP_SPARSE = 2
HS2_OP_PREFILL_BLOCK = 3
HS2_OP_DECODE_SELECT = 4
HS2_OP_DECODE_SPARSE = 5
HS2_OP_SPARSE_PLAN = 6
HS2_OP_SELECT_MIN = 7
HS2_FLAG_EXACT_SELECT = 1
HS2_FLAG_BLOCK_SELECT = 2
HS2_MAX_SEQLEN = 262144


class HS2Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"hs2 status {status}: {msg}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("window", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("flags", ctypes.c_uint32)]


class SelectOptions(ctypes.Structure):
    _fields_ = [("oam_beta", ctypes.c_float), ("decay_mu", ctypes.c_float),
                ("reserved", ctypes.c_float * 2)]


class Varlen(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("cu_seqlens", ctypes.c_void_p),
                ("cu_seqlens_host", ctypes.POINTER(ctypes.c_int32)),
                ("max_seqlen", ctypes.c_int32), ("total_tokens", ctypes.c_int64)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libhs2.so (raises FileNotFoundError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} not built; run __graft_entry__.build() or "
                                "python token_level_sparse_hs2_amd/_build.py")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    D, V = ctypes.POINTER(Dims), ctypes.POINTER(Varlen)
    lib.hs2_workspace_size.argtypes = [D, V, i32, i32, ctypes.POINTER(sz)]
    lib.hs2_workspace_size.restype = i32
    lib.hs2_select.argtypes = [D, V, vp, vp, vp, vp, vp, sz, vp]
    lib.hs2_select.restype = i32
    lib.hs2_sparse_attn.argtypes = [D, V, vp, vp, vp, vp, vp, i32, vp]
    lib.hs2_sparse_attn.restype = i32
    lib.hs2_prefill_block.argtypes = [D, V, vp, vp, vp, i32, ctypes.POINTER(vp),
                                      ctypes.POINTER(vp), i32, vp, vp, sz, vp]
    lib.hs2_prefill_block.restype = i32
    lib.hs2_select_ex.argtypes = [D, V, ctypes.POINTER(SelectOptions), vp, vp, vp, vp, vp, vp, sz,
                                  vp]
    lib.hs2_select_ex.restype = i32
    lib.hs2_select_full.argtypes = [D, V, vp, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    lib.hs2_select_full.restype = i32
    lib.hs2_full_attn.argtypes = [D, V, vp, vp, vp, vp, i32, vp, vp]
    lib.hs2_full_attn.restype = i32
    lib.hs2_decode_select.argtypes = [D, V, vp, vp, vp, vp, vp, sz, vp]
    lib.hs2_decode_select.restype = i32
    lib.hs2_decode_sparse_attn.argtypes = [D, V, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    lib.hs2_decode_sparse_attn.restype = i32
    lib.hs2_decode_sparse_attn_noalloc.argtypes = [D, V, vp, vp, vp, vp, vp, i32, vp]
    lib.hs2_decode_sparse_attn_noalloc.restype = i32
    f32 = ctypes.c_float
    lib.hs2_quantize_fp8.argtypes = [vp, vp, i64, f32, vp]
    lib.hs2_quantize_fp8.restype = i32
    lib.hs2_sparse_attn_fp8.argtypes = [D, V, vp, vp, vp, f32, f32, vp, vp, i32, vp]
    lib.hs2_sparse_plan.argtypes = [D, V, vp, vp, sz, vp]
    lib.hs2_sparse_plan.restype = i32
    lib.hs2_sparse_attn_planned.argtypes = [D, V, vp, vp, vp, vp, sz, vp, i32, vp]
    lib.hs2_sparse_attn_planned.restype = i32
    lib.hs2_sparse_attn_planned_fp8.argtypes = [D, V, vp, vp, vp, f32, f32, vp, sz, vp, i32, vp]
    lib.hs2_sparse_attn_planned_fp8.restype = i32
    lib.hs2_sparse_attn_fp8.restype = i32
    lib.hs2_decode_sparse_attn_fp8.argtypes = [D, V, vp, vp, vp, f32, f32, vp, vp, i32, vp, sz, vp]
    lib.hs2_decode_sparse_attn_fp8.restype = i32
    lib.hs2_decode_select_fp8.argtypes = [D, V, vp, vp, f32, vp, vp, vp, sz, vp]
    lib.hs2_decode_select_fp8.restype = i32
    lib.hs2_status_string.argtypes = [i32]
    lib.hs2_status_string.restype = ctypes.c_char_p
    lib.hs2_plan_task.argtypes = [ctypes.POINTER(ctypes.c_int32), i32, i32, i64,
                                  ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    lib.hs2_plan_task.restype = i64
    lib.hs2_version.argtypes = []
    lib.hs2_version.restype = i32
    _lib = lib
    return lib


def _check(status: int):
    if status != HS2_OK:
        raise HS2Error(status, hs2_status_string(status))


def hs2_status_string(status: int) -> str:
    return load_library().hs2_status_string(status).decode()


def make_dims(num_q_heads: int, num_kv_heads: int, top_k: int, window: int,
              softmax_scale: Optional[float] = None, head_dim: int = 128, flags: int = 0) -> Dims:
    if softmax_scale is None:
        softmax_scale = head_dim ** -0.5
    return Dims(num_q_heads, num_kv_heads, head_dim, top_k, window, float(softmax_scale), flags)


class VarlenArgs:
    """cu_seqlens on the device and on the host, kept alive together."""

    def __init__(self, cu_seqlens_dev, cu_host: Sequence[int], max_seqlen: Optional[int] = None):
        cu_host = [int(x) for x in cu_host]
        self.B = len(cu_host) - 1
        self._host = (ctypes.c_int32 * max(1, len(cu_host)))(*cu_host)
        self._dev = cu_seqlens_dev
        lens = [cu_host[i + 1] - cu_host[i] for i in range(self.B)]
        self.max_seqlen = int(max_seqlen if max_seqlen is not None else max(lens, default=0))
        self.total = cu_host[-1] if cu_host else 0
        self.struct = Varlen(self.B, ctypes.c_void_p(_ptr(cu_seqlens_dev)), self._host,
                             self.max_seqlen, self.total)


def _ptr(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to libhs2 must be contiguous")
    return int(t.data_ptr())


def _stream(stream) -> int:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def hs2_workspace_size(dims: Dims, varlen: VarlenArgs, op: int = HS2_OP_PREFILL_BLOCK,
                       n_sparse: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().hs2_workspace_size(ctypes.byref(dims), ctypes.byref(varlen.struct), op,
                                             n_sparse, ctypes.byref(out)))
    return int(out.value)


def hs2_select(dims: Dims, varlen: VarlenArgs, q, k, idx_out, kth_score_out=None, workspace=None,
               stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().hs2_select(ctypes.byref(dims), ctypes.byref(varlen.struct), _ptr(q),
                                     _ptr(k), _ptr(idx_out), _ptr(kth_score_out), _ptr(workspace),
                                     ws_bytes, _stream(stream)))


def hs2_sparse_attn(dims: Dims, varlen: VarlenArgs, q, k, v, idx, out, out_dtype: int = HS2_OUT_BF16,
                    stream=None) -> None:
    _check(load_library().hs2_sparse_attn(ctypes.byref(dims), ctypes.byref(varlen.struct), _ptr(q),
                                          _ptr(k), _ptr(v), _ptr(idx), _ptr(out), out_dtype,
                                          _stream(stream)))


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def hs2_sparse_plan(dims: Dims, varlen: VarlenArgs, idx, plan, stream=None) -> None:
    _check(load_library().hs2_sparse_plan(ctypes.byref(dims), ctypes.byref(varlen.struct),
                                          _ptr(idx), _ptr(plan), _nbytes(plan), _stream(stream)))


def hs2_sparse_attn_planned(dims: Dims, varlen: VarlenArgs, q, k, v, plan, out,
                            out_dtype: int = HS2_OUT_BF16, stream=None) -> None:
    _check(load_library().hs2_sparse_attn_planned(ctypes.byref(dims), ctypes.byref(varlen.struct),
                                                  _ptr(q), _ptr(k), _ptr(v), _ptr(plan),
                                                  _nbytes(plan), _ptr(out), out_dtype,
                                                  _stream(stream)))


def hs2_sparse_attn_planned_fp8(dims: Dims, varlen: VarlenArgs, q, k8, v8, k_scale: float,
                                v_scale: float, plan, out, out_dtype: int = HS2_OUT_BF16,
                                stream=None) -> None:
    _check(load_library().hs2_sparse_attn_planned_fp8(
        ctypes.byref(dims), ctypes.byref(varlen.struct), _ptr(q), _ptr(k8), _ptr(v8),
        float(k_scale), float(v_scale), _ptr(plan), _nbytes(plan), _ptr(out), out_dtype,
        _stream(stream)))


def hs2_prefill_block(dims: Dims, varlen: VarlenArgs, q_full, k, v, q_sparse: Sequence,
                      outs: Sequence, idx_out, out_dtype: int = HS2_OUT_BF16, workspace=None,
                      stream=None) -> None:
    n = len(q_sparse)
    if len(outs) != n:
        raise ValueError("one output per sparse layer")
    qa = (ctypes.c_void_p * max(1, n))(*[_ptr(x) for x in q_sparse])
    oa = (ctypes.c_void_p * max(1, n))(*[_ptr(x) for x in outs])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().hs2_prefill_block(ctypes.byref(dims), ctypes.byref(varlen.struct),
                                            _ptr(q_full), _ptr(k), _ptr(v), n, qa, oa, out_dtype,
                                            _ptr(idx_out), _ptr(workspace), ws_bytes,
                                            _stream(stream)))


def hs2_select_ex(dims: Dims, varlen: VarlenArgs, q, k, idx_out, kth_score_out=None, v=None,
                  oam_beta: float = 0.0, decay_mu: float = 0.0, workspace=None,
                  stream=None) -> None:
    """hs2_select with the selection variants: the output-aware metric (key j's group
    score weighted by max(1, |v_j|_2)^oam_beta; v [T,Hkv,128] needed when oam_beta > 0)
    and the position-decaying budget (top_k at a sequence's first position down to
    floor(decay_mu * top_k + 0.5) at its last; 0 = none)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    opts = SelectOptions(float(oam_beta), float(decay_mu))
    _check(load_library().hs2_select_ex(ctypes.byref(dims), ctypes.byref(varlen.struct),
                                        ctypes.byref(opts), _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(idx_out), _ptr(kth_score_out), _ptr(workspace),
                                        ws_bytes, _stream(stream)))


def hs2_select_full(dims: Dims, varlen: VarlenArgs, q, k, v, idx_out, out_full,
                    out_dtype: int = HS2_OUT_BF16, kth_score_out=None, workspace=None,
                    stream=None) -> None:
    """hs2_select plus the full layer's own attention output out_full [T,Hq,128]."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().hs2_select_full(ctypes.byref(dims), ctypes.byref(varlen.struct), _ptr(q),
                                          _ptr(k), _ptr(v), _ptr(idx_out), _ptr(kth_score_out),
                                          _ptr(out_full), out_dtype, _ptr(workspace), ws_bytes,
                                          _stream(stream)))


def hs2_full_attn(dims: Dims, varlen: VarlenArgs, q, k, v, out, out_dtype: int = HS2_OUT_BF16,
                  lse2_out=None, stream=None) -> None:
    """The full layer's own attention output out [T,Hq,128] alone (no selection);
    lse2_out (optional, float32 [T,Hq]): each row's base-2 log-sum-exp of the scaled logits."""
    _check(load_library().hs2_full_attn(ctypes.byref(dims), ctypes.byref(varlen.struct), _ptr(q),
                                        _ptr(k), _ptr(v), _ptr(out), out_dtype, _ptr(lse2_out),
                                        _stream(stream)))


def hs2_decode_select(dims: Dims, cache: VarlenArgs, q, k, idx_out, kth_score_out=None,
                      workspace=None, stream=None) -> None:
    """Decode step selection: q [B,Hq,128] (row b = sequence b's newest token, at its
    last cached position), k the cache described by `cache`; idx_out [B,Hkv,K+W]."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().hs2_decode_select(ctypes.byref(dims), ctypes.byref(cache.struct), _ptr(q),
                                            _ptr(k), _ptr(idx_out), _ptr(kth_score_out),
                                            _ptr(workspace), ws_bytes, _stream(stream)))


def hs2_decode_sparse_attn(dims: Dims, cache: VarlenArgs, q, k, v, idx, out,
                           out_dtype: int = HS2_OUT_BF16, workspace=None, stream=None) -> None:
    """One sparse layer of the decode step: q, out [B,Hq,128], idx [B,Hkv,K+W]."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().hs2_decode_sparse_attn(ctypes.byref(dims), ctypes.byref(cache.struct),
                                                 _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(out),
                                                 out_dtype, _ptr(workspace), ws_bytes,
                                                 _stream(stream)))


def hs2_decode_sparse_attn_noalloc(dims: Dims, cache: VarlenArgs, q, k, v, idx, out,
                                   out_dtype: int = HS2_OUT_BF16, stream=None) -> None:
    """hs2_decode_sparse_attn without a workspace: the library's own per-GPU scratch holds
    the split rows' partials (calls that overlap on one GPU race)."""
    _check(load_library().hs2_decode_sparse_attn_noalloc(ctypes.byref(dims),
                                                         ctypes.byref(cache.struct), _ptr(q),
                                                         _ptr(k), _ptr(v), _ptr(idx), _ptr(out),
                                                         out_dtype, _stream(stream)))


def hs2_quantize_fp8(src, dst, inv_scale: float, stream=None) -> None:
    """FP8 cache codes: dst (uint8, same element count) = E4M3(float(src) * inv_scale)."""
    n = src.numel()
    assert dst.numel() == n
    _check(load_library().hs2_quantize_fp8(_ptr(src), _ptr(dst), n, float(inv_scale),
                                           _stream(stream)))


def hs2_sparse_attn_fp8(dims: Dims, varlen: VarlenArgs, q, k8, v8, k_scale: float, v_scale: float,
                        idx, out, out_dtype: int = HS2_OUT_BF16, stream=None) -> None:
    """hs2_sparse_attn over an FP8 cache: k = k_scale * E4M3(k8), v = v_scale * E4M3(v8)."""
    _check(load_library().hs2_sparse_attn_fp8(ctypes.byref(dims), ctypes.byref(varlen.struct),
                                              _ptr(q), _ptr(k8), _ptr(v8), float(k_scale),
                                              float(v_scale), _ptr(idx), _ptr(out), out_dtype,
                                              _stream(stream)))


def hs2_decode_select_fp8(dims: Dims, cache: VarlenArgs, q, k8, k_scale: float, idx_out,
                          kth_score_out=None, workspace=None, stream=None) -> None:
    """hs2_decode_select over an FP8 key cache: k = k_scale * E4M3(k8)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().hs2_decode_select_fp8(
        ctypes.byref(dims), ctypes.byref(cache.struct), _ptr(q), _ptr(k8), float(k_scale),
        _ptr(idx_out), _ptr(kth_score_out), _ptr(workspace), ws_bytes, _stream(stream)))


def hs2_decode_sparse_attn_fp8(dims: Dims, cache: VarlenArgs, q, k8, v8, k_scale: float,
                               v_scale: float, idx, out, out_dtype: int = HS2_OUT_BF16,
                               workspace=None, stream=None) -> None:
    """hs2_decode_sparse_attn over an FP8 cache."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().hs2_decode_sparse_attn_fp8(
        ctypes.byref(dims), ctypes.byref(cache.struct), _ptr(q), _ptr(k8), _ptr(v8),
        float(k_scale), float(v_scale), _ptr(idx), _ptr(out), out_dtype, _ptr(workspace),
        ws_bytes, _stream(stream)))


def hs2_plan_task(cu_host: Sequence[int], rows_per_task: int, task: int):
    """(n_tasks, seq, tile) of the selection task order (host only)."""
    arr = (ctypes.c_int32 * max(1, len(cu_host)))(*[int(x) for x in cu_host])
    s, t = ctypes.c_int32(-1), ctypes.c_int32(-1)
    n = load_library().hs2_plan_task(arr, len(cu_host) - 1, rows_per_task, task, ctypes.byref(s),
                                     ctypes.byref(t))
    if n < 0:
        raise HS2Error(int(n), hs2_status_string(int(n)))
    return int(n), int(s.value), int(t.value)


def hs2_version() -> int:
    return int(load_library().hs2_version())


def tokens_per_task(G: int) -> int:
    """Tokens of one selection task (workgroup) for group size G."""
    rt = 4 if G >= 4 else G
    return 4 * 16 * rt // G
