"""Python binding of libds4attn (ctypes): argument marshalling only.

Every step of the attention path runs in the library's HIP kernels; torch is
used only to own device memory and to name the stream.  There is no CPU or
eager fallback: if the library is missing, or no GPU is present, calls raise.
"""
from __future__ import annotations

import ctypes
import glob
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libds4attn.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "ds4attn.h")

DS4A_F32, DS4A_BF16, DS4A_F16 = 0, 1, 2
STATUS = {0: "OK", -1: "E_NULL", -2: "E_SHAPE", -3: "E_UNSUPPORTED", -4: "E_ALIGN", -5: "E_WORKSPACE",
          -6: "E_DTYPE", -7: "E_HIP"}

_lib = None


class Ds4aError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} -> {STATUS.get(code, code)}: {msg}")
        self.code = code


def hip_runtimes_mapped() -> list[str]:
    """Paths of every libamdhip64 mapped into this process (one expected)."""
    with open("/proc/self/maps") as f:
        return sorted(set(re.findall(r"\S*libamdhip64\S*", f.read())))


def lib() -> ctypes.CDLL:
    """Load libds4attn.so (built in-tree).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m sparse_compressed_kv_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, sz, dbl, flt = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t,
                                 ctypes.c_double, ctypes.c_float)
    L.ds4a_version.argtypes, L.ds4a_version.restype = [], i32
    L.ds4a_last_error.argtypes, L.ds4a_last_error.restype = [], ctypes.c_char_p
    L.ds4a_workspace_bytes.argtypes = [i32, i32, i32, i64, i32, i32, i32]
    L.ds4a_workspace_bytes.restype = sz
    L.ds4a_indexer_score.argtypes = [i32, i32, i64, i32, i32, P, P, P, P, P, P]
    L.ds4a_indexer_score.restype = i32
    L.ds4a_topk_select.argtypes = [i32, i32, i64, i32, P, P, P, P, sz, P]
    L.ds4a_topk_select.restype = i32
    L.ds4a_indexer_topk.argtypes = [i32, i32, i64, i32, i32, i32, P, P, P, P, P, P, sz, P]
    L.ds4a_indexer_topk.restype = i32
    L.ds4a_indexer_score_fp8.argtypes = [i32, i32, i64, i32, i32, P, P, P, P, P, P, P]
    L.ds4a_indexer_score_fp8.restype = i32
    L.ds4a_indexer_topk_fp8.argtypes = [i32, i32, i64, i32, i32, i32, P, P, P, P, P, P, P, sz, P]
    L.ds4a_indexer_topk_fp8.restype = i32
    L.ds4a_sparse_mqa.argtypes = [i32, i32, i32, i32, i32, i32, i64, i32, P, i32, P, dbl, P, P, P, P, flt, P, P, sz,
                                  P]
    L.ds4a_sparse_mqa.restype = i32
    # U T N Hi Di K idx_q idx_w idx_k n_vis H D n_rot W q q_dtype q_pos theta raw raw_vis comp scale idx out ws nb s
    L.ds4a_indexer_topk_mqa.argtypes = [i32, i32, i64, i32, i32, i32, P, P, P, P, i32, i32, i32, i32, P, i32, P, dbl,
                                        P, P, P, flt, P, P, P, sz, P]
    L.ds4a_indexer_topk_mqa.restype = i32
    L.ds4a_indexer_topk_mqa_fp8.argtypes = [i32, i32, i64, i32, i32, i32, P, P, P, P, P, i32, i32, i32, i32, P, i32,
                                            P, dbl, P, P, P, P, flt, P, P, P, sz, P]
    L.ds4a_indexer_topk_mqa_fp8.restype = i32
    L.ds4a_sparse_mqa_noalloc.argtypes = [i32, i32, i32, i32, i32, i32, i64, i32, P, i32, P, dbl, P, P, P, P, flt,
                                          P, P]
    L.ds4a_sparse_mqa_noalloc.restype = i32
    L.ds4a_dense_mqa.argtypes = [i32, i32, i32, i32, i32, i32, i64, P, i32, P, dbl, P, P, P, P, flt, P, P, sz, P]
    L.ds4a_dense_mqa.restype = i32
    L.ds4a_sparse_mqa_fp8.argtypes = [i32, i32, i32, i32, i32, i32, i64, i32, P, i32, P, dbl, P, P, P, P, P, flt, P,
                                      P, sz, P]
    L.ds4a_sparse_mqa_fp8.restype = i32
    L.ds4a_dense_mqa_fp8.argtypes = [i32, i32, i32, i32, i32, i32, i64, P, i32, P, dbl, P, P, P, P, P, flt, P, P, sz,
                                     P]
    L.ds4a_dense_mqa_fp8.restype = i32
    L.ds4a_compress_rows.argtypes = [i32, i32, i32, P, P, P, flt, i32, P, dbl, i32, P, i64, P]
    L.ds4a_compress_rows.restype = i32
    L.ds4a_compress_append.argtypes = [i32, i32, i32, P, P, P, flt, i32, P, P, dbl, i32, P, P, i64, P, P]
    L.ds4a_compress_append.restype = i32
    L.ds4a_push_raw.argtypes = [i32, i32, i32, i32, P, P, P, P]
    L.ds4a_push_raw.restype = i32
    L.ds4a_frontier_push.argtypes = [i32, i32, i32, P, P, P, P, P, P, P]
    L.ds4a_frontier_push.restype = i32
    L.ds4a_ceiling_read.argtypes = [P, i64, i32, P, P]
    L.ds4a_ceiling_read.restype = i32
    L.ds4a_ceiling_mfma.argtypes = [i64, i32, P, ctypes.POINTER(ctypes.c_double), P]
    L.ds4a_ceiling_mfma.restype = i32
    L.ds4a_rope_q.argtypes = [i32, i32, i32, i32, i32, P, i32, P, dbl, P, P]
    L.ds4a_rope_q.restype = i32
    _lib = L
    return L


def declared_symbols() -> list[str]:
    """Function names the public headers (include/*.h) declare."""
    names = set()
    for h in sorted(glob.glob(os.path.join(os.path.dirname(HEADER), "*.h"))):
        names |= set(re.findall(r"\b(ds4a_[a-z0-9_]+)\s*\(", open(h).read()))
    return sorted(names)


def last_error() -> str:
    return lib().ds4a_last_error().decode()


def _check(fn: str, rc: int):
    if rc != 0:
        raise Ds4aError(fn, rc, last_error())


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def workspace_bytes(which: int, U: int, T: int, N: int, K: int, H: int = 0, W: int = 0) -> int:
    return int(lib().ds4a_workspace_bytes(which, U, T, N, K, H, W))


def _workspace(nbytes: int, device, ws):
    """A workspace of at least nbytes: the caller's, or a new zero-filled one (the attention
    keeps counters at its start that must be zero before its first use; calls leave them zero)."""
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    return ws, ws.numel() * ws.element_size()


def indexer_score(idx_q, idx_w, idx_k, n_vis=None, out=None, stream=None):
    """A1.  idx_q bf16 [U,T,64,128], idx_w f32 [U,T,64], idx_k bf16 [U,N,128] -> f32 [U,T,N]."""
    U, T, Hi, Di = idx_q.shape
    N = idx_k.shape[1]
    _need(idx_q, "idx_q", torch.bfloat16)
    _need(idx_w, "idx_w", torch.float32, (U, T, Hi))
    _need(idx_k, "idx_k", torch.bfloat16, (U, N, Di))
    if n_vis is not None:
        _need(n_vis, "n_vis", torch.int32, (U, T))
    if out is None:
        out = torch.empty((U, T, N), dtype=torch.float32, device=idx_q.device)
    _need(out, "out", torch.float32, (U, T, N))
    _check("ds4a_indexer_score", lib().ds4a_indexer_score(U, T, N, Hi, Di, _ptr(idx_q), _ptr(idx_w), _ptr(idx_k),
                                                          _ptr(n_vis), _ptr(out), _stream(stream)))
    return out


def topk_select(scores, K: int, n_vis=None, out=None, workspace=None, stream=None):
    """A2.  scores f32 [U,T,N] -> int32 [U,T,K]: ascending selected rows, -1 padded."""
    _need(scores, "scores", torch.float32)
    U, T, N = scores.shape
    if n_vis is not None:
        _need(n_vis, "n_vis", torch.int32, (U, T))
    if out is None:
        out = torch.empty((U, T, K), dtype=torch.int32, device=scores.device)
    _need(out, "out", torch.int32, (U, T, K))
    ws, nb = _workspace(workspace_bytes(0, U, T, N, K), scores.device, workspace)
    _check("ds4a_topk_select", lib().ds4a_topk_select(U, T, N, K, _ptr(scores), _ptr(n_vis), _ptr(out), _ptr(ws),
                                                      nb, _stream(stream)))
    return out


def indexer_topk(idx_q, idx_w, idx_k, K: int, n_vis=None, out=None, workspace=None, stream=None):
    """A1 + A2 in one call: the selected rows int32 [U,T,K] that topk_select would return on
    indexer_score's scores, without writing the scores (decode shapes)."""
    _need(idx_q, "idx_q", torch.bfloat16)
    U, T, Hi, Di = idx_q.shape
    N = idx_k.shape[1]
    _need(idx_w, "idx_w", torch.float32, (U, T, Hi))
    _need(idx_k, "idx_k", torch.bfloat16, (U, N, Di))
    if n_vis is not None:
        _need(n_vis, "n_vis", torch.int32, (U, T))
    if out is None:
        out = torch.empty((U, T, K), dtype=torch.int32, device=idx_q.device)
    _need(out, "out", torch.int32, (U, T, K))
    ws, nb = _workspace(workspace_bytes(2, U, T, N, K), idx_q.device, workspace)
    _check("ds4a_indexer_topk", lib().ds4a_indexer_topk(U, T, N, Hi, Di, K, _ptr(idx_q), _ptr(idx_w), _ptr(idx_k),
                                                        _ptr(n_vis), _ptr(out), _ptr(ws), nb, _stream(stream)))
    return out


def _fp8_keys(idx_k8, idx_k_scale, U, Di):
    """E4M3 key codes (uint8 or float8_e4m3fn) [U,N,Di] and their f32 row scales [U,N]."""
    if not isinstance(idx_k8, torch.Tensor) or idx_k8.dim() != 3:
        raise TypeError("idx_k8 must be a 3-d torch.Tensor")
    if idx_k8.dtype == torch.float8_e4m3fn:
        idx_k8 = idx_k8.view(torch.uint8)
    N = idx_k8.shape[1]
    _need(idx_k8, "idx_k8", torch.uint8, (U, N, Di))
    _need(idx_k_scale, "idx_k_scale", torch.float32, (U, N))
    return idx_k8, N


def indexer_score_fp8(idx_q, idx_w, idx_k8, idx_k_scale, n_vis=None, out=None, stream=None):
    """A1 on FP8-stored keys: codes [U,N,128] (E4M3FN), scales f32 [U,N] -> f32 [U,T,N]."""
    _need(idx_q, "idx_q", torch.bfloat16)
    U, T, Hi, Di = idx_q.shape
    idx_k8, N = _fp8_keys(idx_k8, idx_k_scale, U, Di)
    _need(idx_w, "idx_w", torch.float32, (U, T, Hi))
    if n_vis is not None:
        _need(n_vis, "n_vis", torch.int32, (U, T))
    if out is None:
        out = torch.empty((U, T, N), dtype=torch.float32, device=idx_q.device)
    _need(out, "out", torch.float32, (U, T, N))
    _check("ds4a_indexer_score_fp8",
           lib().ds4a_indexer_score_fp8(U, T, N, Hi, Di, _ptr(idx_q), _ptr(idx_w), _ptr(idx_k8), _ptr(idx_k_scale),
                                        _ptr(n_vis), _ptr(out), _stream(stream)))
    return out


def indexer_topk_fp8(idx_q, idx_w, idx_k8, idx_k_scale, K: int, n_vis=None, out=None, workspace=None, stream=None):
    """A1 + A2 on FP8-stored keys (as indexer_topk; same workspace size)."""
    _need(idx_q, "idx_q", torch.bfloat16)
    U, T, Hi, Di = idx_q.shape
    idx_k8, N = _fp8_keys(idx_k8, idx_k_scale, U, Di)
    _need(idx_w, "idx_w", torch.float32, (U, T, Hi))
    if n_vis is not None:
        _need(n_vis, "n_vis", torch.int32, (U, T))
    if out is None:
        out = torch.empty((U, T, K), dtype=torch.int32, device=idx_q.device)
    _need(out, "out", torch.int32, (U, T, K))
    ws, nb = _workspace(workspace_bytes(2, U, T, N, K), idx_q.device, workspace)
    _check("ds4a_indexer_topk_fp8",
           lib().ds4a_indexer_topk_fp8(U, T, N, Hi, Di, K, _ptr(idx_q), _ptr(idx_w), _ptr(idx_k8), _ptr(idx_k_scale),
                                       _ptr(n_vis), _ptr(out), _ptr(ws), nb, _stream(stream)))
    return out


def _q_dtype(q):
    if q.dtype == torch.float32:
        return DS4A_F32
    if q.dtype == torch.bfloat16:
        return DS4A_BF16
    raise TypeError(f"q must be float32 or bfloat16 (got {q.dtype})")


def _comp_rows(comp_kv, comp_scale, U, N, D):
    """bf16 rows, or E4M3 codes (uint8 / float8_e4m3fn) with f32 row scales -> (rows, fp8)."""
    if comp_scale is None:
        _need(comp_kv, "comp_kv", torch.bfloat16, (U, N, D))
        return comp_kv, False
    if comp_kv.dtype == torch.float8_e4m3fn:
        comp_kv = comp_kv.view(torch.uint8)
    _need(comp_kv, "comp_kv8", torch.uint8, (U, N, D))
    _need(comp_scale, "comp_scale", torch.float32, (U, N))
    return comp_kv, True


def _raw_vis(raw_vis, U, T, W):
    if raw_vis is None or W == 0:
        return None
    return _need(raw_vis, "raw_vis", torch.int32, (U, T))


def sparse_mqa(q, q_pos, raw_kv, comp_kv, idx, scale: float, theta: float = 10000.0, W: int = 128,
               out=None, workspace=None, stream=None, comp_scale=None, raw_vis=None):
    """A3-A6.  q [U,T,H,512] f32|bf16, q_pos i64 [U,T], raw_kv f16 [U,T+W-1,512],
    comp_kv bf16 [U,N,512] (or E4M3 codes [U,N,512] with comp_scale f32 [U,N]),
    idx i32 [U,T,K], raw_vis i32 [U,T] (raw rows taking part) or None -> f32 [U,T,H,512]."""
    if not isinstance(q, torch.Tensor):
        raise TypeError("q must be a torch.Tensor")
    U, T, H, D = q.shape
    N = comp_kv.shape[1]
    K = idx.shape[2]
    _need(q, "q", q.dtype)
    qd = _q_dtype(q)
    _need(q_pos, "q_pos", torch.int64, (U, T))
    if W > 0:
        _need(raw_kv, "raw_kv", torch.float16, (U, T + W - 1, D))
    comp_kv, fp8 = _comp_rows(comp_kv, comp_scale, U, N, D)
    _need(idx, "idx", torch.int32, (U, T, K))
    if out is None:
        out = torch.empty((U, T, H, D), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (U, T, H, D))
    ws, nb = _workspace(workspace_bytes(1, U, T, N, K, H, W), q.device, workspace)
    raw = _ptr(raw_kv) if W > 0 else None
    rv = _ptr(_raw_vis(raw_vis, U, T, W))
    if fp8:
        _check("ds4a_sparse_mqa_fp8", lib().ds4a_sparse_mqa_fp8(
            U, T, H, D, 64, W, N, K, _ptr(q), qd, _ptr(q_pos), float(theta), raw, rv, _ptr(comp_kv),
            _ptr(comp_scale), _ptr(idx), float(scale), _ptr(out), _ptr(ws), nb, _stream(stream)))
    else:
        _check("ds4a_sparse_mqa", lib().ds4a_sparse_mqa(
            U, T, H, D, 64, W, N, K, _ptr(q), qd, _ptr(q_pos), float(theta), raw, rv, _ptr(comp_kv), _ptr(idx),
            float(scale), _ptr(out), _ptr(ws), nb, _stream(stream)))
    return out


def indexer_topk_mqa(idx_q, idx_w, idx_k, K: int, q, q_pos, raw_kv, comp_kv, scale: float,
                     theta: float = 10000.0, W: int = 128, n_vis=None, raw_vis=None, idx=None, out=None,
                     workspace=None, stream=None, idx_k_scale=None, comp_scale=None):
    """A1 + A2 + A3-A6 in one call: (idx i32 [U,T,K], out f32 [U,T,H,512]) as indexer_topk then
    sparse_mqa would give.  FP8 storage: idx_k as E4M3 codes with idx_k_scale and comp_kv as E4M3
    codes with comp_scale (both, or neither)."""
    if not isinstance(q, torch.Tensor):
        raise TypeError("q must be a torch.Tensor")
    U, T, Hi, Di = idx_q.shape
    _, _, H, D = q.shape
    _need(idx_q, "idx_q", torch.bfloat16)
    _need(idx_w, "idx_w", torch.float32, (U, T, Hi))
    fp8 = idx_k_scale is not None
    if fp8 != (comp_scale is not None):
        raise ValueError("FP8 keys and FP8 rows go together (idx_k_scale and comp_scale)")
    if fp8:
        idx_k, N = _fp8_keys(idx_k, idx_k_scale, U, Di)
    else:
        N = idx_k.shape[1]
        _need(idx_k, "idx_k", torch.bfloat16, (U, N, Di))
    if n_vis is not None:
        _need(n_vis, "n_vis", torch.int32, (U, T))
    _need(q, "q", q.dtype, (U, T, H, D))
    qd = _q_dtype(q)
    _need(q_pos, "q_pos", torch.int64, (U, T))
    if W > 0:
        _need(raw_kv, "raw_kv", torch.float16, (U, T + W - 1, D))
    comp_kv, _ = _comp_rows(comp_kv, comp_scale, U, N, D)
    if idx is None:
        idx = torch.empty((U, T, K), dtype=torch.int32, device=q.device)
    _need(idx, "idx", torch.int32, (U, T, K))
    if out is None:
        out = torch.empty((U, T, H, D), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (U, T, H, D))
    ws, nb = _workspace(workspace_bytes(4, U, T, N, K, H, W), q.device, workspace)
    raw = _ptr(raw_kv) if W > 0 else None
    rv = _ptr(_raw_vis(raw_vis, U, T, W))
    if fp8:
        _check("ds4a_indexer_topk_mqa_fp8", lib().ds4a_indexer_topk_mqa_fp8(
            U, T, N, Hi, Di, K, _ptr(idx_q), _ptr(idx_w), _ptr(idx_k), _ptr(idx_k_scale), _ptr(n_vis), H, D, 64, W,
            _ptr(q), qd, _ptr(q_pos), float(theta), raw, rv, _ptr(comp_kv), _ptr(comp_scale), float(scale),
            _ptr(idx), _ptr(out), _ptr(ws), nb, _stream(stream)))
    else:
        _check("ds4a_indexer_topk_mqa", lib().ds4a_indexer_topk_mqa(
            U, T, N, Hi, Di, K, _ptr(idx_q), _ptr(idx_w), _ptr(idx_k), _ptr(n_vis), H, D, 64, W, _ptr(q), qd,
            _ptr(q_pos), float(theta), raw, rv, _ptr(comp_kv), float(scale), _ptr(idx), _ptr(out), _ptr(ws), nb,
            _stream(stream)))
    return idx, out


def sparse_mqa_noalloc(q, q_pos, raw_kv, comp_kv, idx, scale: float, theta: float = 10000.0, W: int = 128,
                       out=None, stream=None, raw_vis=None):
    """sparse_mqa without a workspace: split unions use the library's own device scratch
    (ds4a_sparse_mqa_noalloc; bf16 rows).  Calls that may overlap on one GPU race on it."""
    if not isinstance(q, torch.Tensor):
        raise TypeError("q must be a torch.Tensor")
    U, T, H, D = q.shape
    N = comp_kv.shape[1]
    K = idx.shape[2]
    _need(q, "q", q.dtype)
    qd = _q_dtype(q)
    _need(q_pos, "q_pos", torch.int64, (U, T))
    if W > 0:
        _need(raw_kv, "raw_kv", torch.float16, (U, T + W - 1, D))
    _need(comp_kv, "comp_kv", torch.bfloat16, (U, N, D))
    _need(idx, "idx", torch.int32, (U, T, K))
    if out is None:
        out = torch.empty((U, T, H, D), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (U, T, H, D))
    raw = _ptr(raw_kv) if W > 0 else None
    rv = _ptr(_raw_vis(raw_vis, U, T, W))
    _check("ds4a_sparse_mqa_noalloc", lib().ds4a_sparse_mqa_noalloc(
        U, T, H, D, 64, W, N, K, _ptr(q), qd, _ptr(q_pos), float(theta), raw, rv, _ptr(comp_kv), _ptr(idx),
        float(scale), _ptr(out), _stream(stream)))
    return out


def dense_mqa(q, q_pos, raw_kv, comp_kv, scale: float, theta: float = 10000.0, W: int = 128, n_vis=None,
              out=None, workspace=None, stream=None, comp_scale=None, raw_vis=None):
    """Dense attention (layers without an indexer).  q [U,T,H,512] f32|bf16, q_pos i64 [U,T],
    raw_kv f16 [U,T+W-1,512] (or None when W = 0), comp_kv bf16 [U,N,512] (N may be 0, or None;
    or E4M3 codes with comp_scale f32 [U,N]), n_vis i32 [U,T] or None -> f32 [U,T,H,512]."""
    if not isinstance(q, torch.Tensor):
        raise TypeError("q must be a torch.Tensor")
    U, T, H, D = q.shape
    N = 0 if comp_kv is None else comp_kv.shape[1]
    _need(q, "q", q.dtype)
    qd = _q_dtype(q)
    _need(q_pos, "q_pos", torch.int64, (U, T))
    if W > 0:
        _need(raw_kv, "raw_kv", torch.float16, (U, T + W - 1, D))
    fp8 = comp_scale is not None
    if N > 0:
        comp_kv, fp8 = _comp_rows(comp_kv, comp_scale, U, N, D)
    if n_vis is not None:
        _need(n_vis, "n_vis", torch.int32, (U, T))
    if out is None:
        out = torch.empty((U, T, H, D), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (U, T, H, D))
    ws, nb = _workspace(workspace_bytes(3, U, T, N, 0, H, W), q.device, workspace)
    raw = _ptr(raw_kv) if W > 0 else None
    rv = _ptr(_raw_vis(raw_vis, U, T, W))
    comp = _ptr(comp_kv) if N > 0 else None
    nv = _ptr(n_vis) if n_vis is not None else None
    if fp8:
        _check("ds4a_dense_mqa_fp8", lib().ds4a_dense_mqa_fp8(
            U, T, H, D, 64, W, N, _ptr(q), qd, _ptr(q_pos), float(theta), raw, rv, comp,
            _ptr(comp_scale) if N > 0 else None, nv, float(scale), _ptr(out), _ptr(ws), nb, _stream(stream)))
    else:
        _check("ds4a_dense_mqa", lib().ds4a_dense_mqa(
            U, T, H, D, 64, W, N, _ptr(q), qd, _ptr(q_pos), float(theta), raw, rv, comp, nv, float(scale),
            _ptr(out), _ptr(ws), nb, _stream(stream)))
    return out


def compress_rows(state_kv, state_score, gain, row_pos, eps: float = 1e-6, n_rot: int = 64,
                  theta: float = 10000.0, fp8: bool = True, out=None, stream=None):
    """Compressor row emission.  state_kv, state_score f32 [U, ratio, width], gain f32 [U, width],
    row_pos i64 [U] -> bf16 [U, width] (or into `out`, a bf16 tensor whose rows are
    out[u] = the row of unit u, e.g. cache[:, n, :] of a [U, N, width] cache)."""
    U, ratio, width = state_kv.shape
    _need(state_kv, "state_kv", torch.float32, (U, ratio, width))
    _need(state_score, "state_score", torch.float32, (U, ratio, width))
    _need(gain, "gain", torch.float32, (U, width))
    _need(row_pos, "row_pos", torch.int64, (U,))
    if out is None:
        out = torch.empty((U, width), dtype=torch.bfloat16, device=state_kv.device)
    if out.dtype != torch.bfloat16 or out.shape != (U, width) or out.stride(1) != 1 or out.device.type != "cuda":
        raise ValueError("out must be a bf16 [U, width] view with unit-stride rows on the GPU")
    stride = out.stride(0) if U > 1 else width
    _check("ds4a_compress_rows", lib().ds4a_compress_rows(
        U, width, ratio, _ptr(state_kv), _ptr(state_score), _ptr(gain), float(eps), int(n_rot), _ptr(row_pos),
        float(theta), 1 if fp8 else 0, _ptr(out), stride, _stream(stream)))
    return out


ROW_BF16, ROW_BF16_FP8RT, ROW_E4M3 = 0, 1, 2


def compress_append(state_kv, state_score, gain, pos, row_pos, comp, n_comp, comp_scale=None, eps: float = 1e-6,
                    n_rot: int = 64, theta: float = 10000.0, fp8: bool = True, stream=None):
    """Compressed-row append: units whose token closes a group (pos mod ratio == ratio - 1) emit
    a row into row n_comp[u] of their cache and count it.  comp: bf16 [U, cap, width] (rows
    with or without the FP8 round trip, by `fp8`), or uint8 / float8_e4m3fn [U, cap, width]
    codes with comp_scale f32 [U, cap] (the FP8 row as stored)."""
    U, ratio, width = state_kv.shape
    _need(state_kv, "state_kv", torch.float32, (U, ratio, width))
    _need(state_score, "state_score", torch.float32, (U, ratio, width))
    _need(gain, "gain", torch.float32, (U, width))
    _need(pos, "pos", torch.int64, (U,))
    _need(row_pos, "row_pos", torch.int64, (U,))
    _need(n_comp, "n_comp", torch.int32, (U,))
    if not isinstance(comp, torch.Tensor) or comp.dim() != 3:
        raise TypeError("comp must be a 3-d torch.Tensor")
    cap = comp.shape[1]
    if comp.dtype == torch.bfloat16:
        fmt = ROW_BF16_FP8RT if fp8 else ROW_BF16
        _need(comp, "comp", torch.bfloat16, (U, cap, width))
        if comp_scale is not None:
            raise ValueError("comp_scale is for E4M3 caches only")
    else:
        if comp.dtype == torch.float8_e4m3fn:
            comp = comp.view(torch.uint8)
        fmt = ROW_E4M3
        _need(comp, "comp", torch.uint8, (U, cap, width))
        _need(comp_scale, "comp_scale", torch.float32, (U, cap))
    _check("ds4a_compress_append", lib().ds4a_compress_append(
        U, width, ratio, _ptr(state_kv), _ptr(state_score), _ptr(gain), float(eps), int(n_rot), _ptr(pos),
        _ptr(row_pos), float(theta), fmt, _ptr(comp), _ptr(comp_scale), cap, _ptr(n_comp), _stream(stream)))


def push_raw(kv, raw, n_raw, stream=None):
    """Raw-window push: kv f32 [U, T, D] into raw f16 [U, cap, D] holding n_raw int32 [U] rows."""
    U, T, D = kv.shape
    cap = raw.shape[1]
    _need(kv, "kv", torch.float32, (U, T, D))
    _need(raw, "raw", torch.float16, (U, cap, D))
    _need(n_raw, "n_raw", torch.int32, (U,))
    _check("ds4a_push_raw", lib().ds4a_push_raw(U, T, D, cap, _ptr(kv), _ptr(raw), _ptr(n_raw), _stream(stream)))


def frontier_push(kv, score, ape, pos, state_kv, state_score, stream=None):
    """A token into the compressor frontier: row pos mod ratio of state_kv / state_score
    f32 [U, ratio, width] takes kv [U, width] and score [U, width] + ape[pos mod ratio]."""
    U, ratio, width = state_kv.shape
    _need(kv, "kv", torch.float32, (U, width))
    _need(score, "score", torch.float32, (U, width))
    _need(ape, "ape", torch.float32, (ratio, width))
    _need(pos, "pos", torch.int64, (U,))
    _need(state_kv, "state_kv", torch.float32, (U, ratio, width))
    _need(state_score, "state_score", torch.float32, (U, ratio, width))
    _check("ds4a_frontier_push", lib().ds4a_frontier_push(U, width, ratio, _ptr(kv), _ptr(score), _ptr(ape),
                                                          _ptr(pos), _ptr(state_kv), _ptr(state_score),
                                                          _stream(stream)))


def rope_q(q, q_pos, theta: float = 10000.0, out=None, stream=None):
    """A3 alone: rotated query as f32 [U,T,H,512]."""
    U, T, H, D = q.shape
    qd = _q_dtype(q)
    _need(q, "q", q.dtype)
    _need(q_pos, "q_pos", torch.int64, (U, T))
    if out is None:
        out = torch.empty((U, T, H, D), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (U, T, H, D))
    _check("ds4a_rope_q", lib().ds4a_rope_q(U, T, H, D, 64, _ptr(q), qd, _ptr(q_pos), float(theta), _ptr(out),
                                            _stream(stream)))
    return out


class Step:
    """The whole hot path for fixed shapes: indexer -> top-k -> attention, with every
    intermediate, output and workspace allocated once up front.  fused=True runs A1 + A2
    as ds4a_indexer_topk (no score buffer in decode shapes); fused=False runs the separate
    calls and keeps the scores in self.scores; one_call=True runs the whole path as
    ds4a_indexer_topk_mqa (same idx and out, bit for bit)."""

    def __init__(self, U, T, N, H=64, K=512, W=128, q_dtype=torch.float32, device="cuda", fused=False,
                 one_call=False):
        self.U, self.T, self.N, self.H, self.K, self.W = U, T, N, H, K, W
        self.fused = fused or one_call
        self.one_call = one_call
        dev = torch.device(device)
        self.scores = None if self.fused else torch.empty((U, T, N), dtype=torch.float32, device=dev)
        self.idx = torch.empty((U, T, K), dtype=torch.int32, device=dev)
        self.out = torch.empty((U, T, H, 512), dtype=torch.float32, device=dev)
        nb0 = workspace_bytes(2 if self.fused else 0, U, T, N, K)
        nb1 = workspace_bytes(1, U, T, N, K, H, W)
        self.ws_topk = torch.zeros(max(nb0, 1), dtype=torch.uint8, device=dev)
        self.ws_mqa = torch.zeros(max(nb1, 1), dtype=torch.uint8, device=dev)   # counters start at zero
        self.ws_step = None
        if one_call:
            self.ws_step = torch.zeros(workspace_bytes(4, U, T, N, K, H, W), dtype=torch.uint8, device=dev)

    def select(self, x: dict, n_vis=None, stream=None):
        """A1 + A2 into self.idx."""
        if self.fused:
            indexer_topk(x["idx_q"], x["idx_w"], x["idx_k"], self.K, n_vis=n_vis, out=self.idx,
                         workspace=self.ws_topk, stream=stream)
        else:
            indexer_score(x["idx_q"], x["idx_w"], x["idx_k"], n_vis=n_vis, out=self.scores, stream=stream)
            topk_select(self.scores, self.K, n_vis=n_vis, out=self.idx, workspace=self.ws_topk, stream=stream)
        return self.idx

    def __call__(self, x: dict, n_vis=None, scale=1.0 / 512 ** 0.5, theta=10000.0, stream=None, raw_vis=None):
        """raw_vis: int32 [U, T] raw-window rows that take part (a window not yet full), or None."""
        if self.one_call:
            indexer_topk_mqa(x["idx_q"], x["idx_w"], x["idx_k"], self.K, x["q"], x["pos"], x["raw"], x["comp"],
                             scale, theta, W=self.W, n_vis=n_vis, raw_vis=raw_vis, idx=self.idx, out=self.out,
                             workspace=self.ws_step, stream=stream)
            return self.out
        self.select(x, n_vis=n_vis, stream=stream)
        sparse_mqa(x["q"], x["pos"], x["raw"], x["comp"], self.idx, scale, theta, W=self.W, out=self.out,
                   workspace=self.ws_mqa, stream=stream, raw_vis=raw_vis)
        return self.out


def ceiling_read(src, grid: int = 8192, sink=None, stream=None):
    """Launch the HBM read-stream ceiling kernel over the bytes of src (a CUDA tensor)."""
    if sink is None:
        sink = torch.empty(grid * 256, dtype=torch.int32, device=src.device)
    rc = lib().ds4a_ceiling_read(_ptr(src), src.numel() * src.element_size(), grid, _ptr(sink), _stream(stream))
    if rc != 0:
        raise Ds4aError("ds4a_ceiling_read", rc, "bad argument" if rc == -1 else "launch failed")
    return sink


def ceiling_mfma(iters: int, grid: int = 2048, sink=None, stream=None) -> float:
    """Launch the bf16 matrix-core ceiling kernel; returns the launch's dense flop count."""
    if sink is None:
        sink = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    fl = ctypes.c_double(0.0)
    rc = lib().ds4a_ceiling_mfma(int(iters), grid, _ptr(sink), ctypes.byref(fl), _stream(stream))
    if rc != 0:
        raise Ds4aError("ds4a_ceiling_mfma", rc, "bad argument" if rc == -1 else "launch failed")
    return fl.value
