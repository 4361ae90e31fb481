"""Python face of the plain CPU oracle (ds4o.c), for tests and baselines only.

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's
CPU-baseline leg import this module.  It loads liboracle.so, built from
ds4o.c with gcc (IEEE double, no fast-math, no FMA contraction), and shares
nothing with the GPU library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SOURCES = [os.path.join(HERE, "ds4o.c")]


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc.  Returns its path."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, *SOURCES, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True, cwd=HERE)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.ds4o_f16_to_f64.argtypes, L.ds4o_f16_to_f64.restype = [ctypes.c_uint16], dbl
        L.ds4o_bf16_to_f64.argtypes, L.ds4o_bf16_to_f64.restype = [ctypes.c_uint16], dbl
        L.ds4o_round_f16.argtypes, L.ds4o_round_f16.restype = [ctypes.c_float], ctypes.c_uint16
        L.ds4o_indexer_score.argtypes = [i64, i32, i32, P, P, P, i64, P]
        L.ds4o_indexer_score.restype = None
        L.ds4o_topk.argtypes, L.ds4o_topk.restype = [i64, i32, P, P], i32
        L.ds4o_rope_q.argtypes = [i32, i32, i32, i64, dbl, P, P]
        L.ds4o_rope_q.restype = None
        L.ds4o_sparse_mqa.argtypes = [i32, i32, i32, i32, P, P, P, P, dbl, P]
        L.ds4o_sparse_mqa.restype = i32
        L.ds4o_step.argtypes = [i32, i32, i64, i32, i32, i32, i32, i32, i32, i32,
                                P, i32, P, dbl, P, P, P, P, P, P, dbl, P, i64, i32, P, P, P]
        L.ds4o_step.restype = i32
        L.ds4o_round_bf16.argtypes, L.ds4o_round_bf16.restype = [dbl], ctypes.c_uint16
        L.ds4o_e4m3_to_f64.argtypes, L.ds4o_e4m3_to_f64.restype = [ctypes.c_uint8], dbl
        L.ds4o_round_e4m3.argtypes, L.ds4o_round_e4m3.restype = [dbl], ctypes.c_uint8
        L.ds4o_indexer_score_fp8.argtypes = [i64, i32, i32, P, P, P, P, i64, P]
        L.ds4o_indexer_score_fp8.restype = None
        L.ds4o_sparse_mqa_fp8.argtypes = [i32, i32, i32, i32, P, P, P, P, P, dbl, P]
        L.ds4o_sparse_mqa_fp8.restype = i32
        L.ds4o_compress_row.argtypes = [i32, i32, P, P, P, dbl, i32, i64, dbl, i32, P, P, P]
        L.ds4o_compress_row.restype = i32
        L.ds4o_compress_row_e4m3.argtypes = [i32, i32, P, P, P, dbl, i32, i64, dbl, P, P]
        L.ds4o_compress_row_e4m3.restype = i32
        L.ds4o_push_raw.argtypes = [i32, i32, i32, P, P, P]
        L.ds4o_push_raw.restype = None
        L.ds4o_frontier_push.argtypes = [i32, i32, i64, P, P, P, P, P]
        L.ds4o_frontier_push.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.uint16)


def f16_to_f64(bits) -> np.ndarray:
    bits = _u16(bits)
    f = lib().ds4o_f16_to_f64
    return np.array([f(int(b)) for b in bits.ravel()], dtype=np.float64).reshape(bits.shape)


def bf16_to_f64(bits) -> np.ndarray:
    bits = _u16(bits)
    f = lib().ds4o_bf16_to_f64
    return np.array([f(int(b)) for b in bits.ravel()], dtype=np.float64).reshape(bits.shape)


def round_f16(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    f = lib().ds4o_round_f16
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def indexer_score(qI, w, kI, n_vis: int | None = None) -> np.ndarray:
    """One query.  qI bf16 bits [Hi, Di], w f32 [Hi], kI bf16 bits [N, Di] -> float64 [N]."""
    qI, kI = _u16(qI), _u16(kI)
    w = np.ascontiguousarray(w, dtype=np.float32)
    Hi, Di = qI.shape
    N = kI.shape[0]
    assert kI.shape[1] == Di and w.shape == (Hi,)
    s = np.empty(N, dtype=np.float64)
    lib().ds4o_indexer_score(N, Hi, Di, _p(qI), _p(w), _p(kI), N if n_vis is None else int(n_vis), _p(s))
    return s


def indexer_score_fp8(qI, w, k8, scale, n_vis: int | None = None) -> np.ndarray:
    """One query over FP8-stored keys.  qI bf16 bits [Hi, Di], w f32 [Hi], k8 E4M3FN codes
    uint8 [N, Di], scale f32 [N] -> float64 [N]."""
    qI = _u16(qI)
    k8 = np.ascontiguousarray(k8, dtype=np.uint8)
    w = np.ascontiguousarray(w, dtype=np.float32)
    scale = np.ascontiguousarray(scale, dtype=np.float32)
    Hi, Di = qI.shape
    N = k8.shape[0]
    assert k8.shape[1] == Di and w.shape == (Hi,) and scale.shape == (N,)
    s = np.empty(N, dtype=np.float64)
    lib().ds4o_indexer_score_fp8(N, Hi, Di, _p(qI), _p(w), _p(k8), _p(scale), N if n_vis is None else int(n_vis),
                                 _p(s))
    return s


def topk(scores, K: int, n_vis: int | None = None) -> np.ndarray:
    """One query: indices of the best min(K, n_vis) rows in rank order, -1 padded to K."""
    s = np.ascontiguousarray(scores, dtype=np.float64)
    idx = np.empty(K, dtype=np.int32)
    lib().ds4o_topk(s.shape[0] if n_vis is None else int(n_vis), K, _p(s), _p(idx))
    return idx


def rope_q(q, pos: int, theta: float = 10000.0, n_rot: int = 64) -> np.ndarray:
    """One query: q float64 [H, D] -> rotated copy."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    H, D = q.shape
    out = np.empty_like(q)
    lib().ds4o_rope_q(H, D, n_rot, int(pos), float(theta), _p(q), _p(out))
    return out


def sparse_mqa(q_rot, raw, comp, idx, scale: float) -> np.ndarray:
    """One query: q_rot float64 [H, D], raw f16 bits [W, D], comp bf16 bits [N, D], idx int32 [K]."""
    q_rot = np.ascontiguousarray(q_rot, dtype=np.float64)
    raw, comp = _u16(raw), _u16(comp)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    H, D = q_rot.shape
    W = raw.shape[0] if raw.size else 0
    if W == 0:
        raw = np.zeros((1, D), dtype=np.uint16)
    if comp.size == 0:
        comp = np.zeros((1, D), dtype=np.uint16)
    out = np.empty((H, D), dtype=np.float64)
    lib().ds4o_sparse_mqa(H, D, W, idx.shape[0], _p(q_rot), _p(raw), _p(comp), _p(idx), float(scale), _p(out))
    return out


def sparse_mqa_fp8(q_rot, raw, comp8, comp_scale, idx, scale: float) -> np.ndarray:
    """One query over FP8-stored compressed rows: comp8 E4M3FN codes uint8 [N, D], comp_scale
    f32 [N]; the rest as sparse_mqa."""
    q_rot = np.ascontiguousarray(q_rot, dtype=np.float64)
    raw = _u16(raw)
    comp8 = np.ascontiguousarray(comp8, dtype=np.uint8)
    cs = np.ascontiguousarray(comp_scale, dtype=np.float32)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    H, D = q_rot.shape
    W = raw.shape[0] if raw.size else 0
    if W == 0:
        raw = np.zeros((1, D), dtype=np.uint16)
    if comp8.size == 0:
        comp8, cs = np.zeros((1, D), dtype=np.uint8), np.ones(1, dtype=np.float32)
    out = np.empty((H, D), dtype=np.float64)
    lib().ds4o_sparse_mqa_fp8(H, D, W, idx.shape[0], _p(q_rot), _p(raw), _p(comp8), _p(cs), _p(idx), float(scale),
                              _p(out))
    return out


def step(w, x: dict, sel=None, nthreads: int = 1, want=("scores", "idx", "out")) -> dict:
    """Whole step for a synthetic workload (synth.Workload) and its inputs (synth.make_config).

    sel: optional list of flattened (u*T + t) pairs; outputs are compact over sel.
    """
    U, T, N, H, D, W, K = w.U, w.T, w.N, w.H, w.D, w.W, w.K
    if sel is None:
        sel_arr, n = None, U * T
    else:
        sel_arr = np.ascontiguousarray(sel, dtype=np.int64)
        n = sel_arr.shape[0]
    q = np.ascontiguousarray(x["q"])
    q_is_bf16 = 1 if q.dtype == np.uint16 else 0
    if not q_is_bf16:
        q = np.ascontiguousarray(q, dtype=np.float32)
    arrs = {
        "pos": np.ascontiguousarray(x["pos"], dtype=np.int64),
        "raw": _u16(x["raw"]), "comp": _u16(x["comp"]), "idx_k": _u16(x["idx_k"]),
        "idx_q": _u16(x["idx_q"]), "idx_w": np.ascontiguousarray(x["idx_w"], dtype=np.float32),
        "n_vis": np.ascontiguousarray(x["n_vis"], dtype=np.int32),
    }
    res = {}
    scores = np.empty((n, N), dtype=np.float64) if "scores" in want else None
    idx = np.empty((n, K), dtype=np.int32) if "idx" in want else None
    out = np.empty((n, H, D), dtype=np.float64) if "out" in want else None
    null = ctypes.c_void_p(0)
    rc = lib().ds4o_step(U, T, N, H, D, w.n_rot, W, w.Hi, w.Di, K, _p(q), q_is_bf16, _p(arrs["pos"]),
                         float(w.theta), _p(arrs["raw"]), _p(arrs["comp"]), _p(arrs["idx_k"]),
                         _p(arrs["idx_q"]), _p(arrs["idx_w"]), _p(arrs["n_vis"]), float(w.scale),
                         _p(sel_arr) if sel_arr is not None else null, n, int(nthreads),
                         _p(scores) if scores is not None else null, _p(idx) if idx is not None else null,
                         _p(out) if out is not None else null)
    if rc != 0:
        raise ValueError(f"ds4o_step rejected its arguments (rc={rc})")
    if scores is not None:
        res["scores"] = scores
    if idx is not None:
        res["idx"] = idx
    if out is not None:
        res["out"] = out
    return res


def round_bf16(x) -> np.ndarray:
    """Nearest bfloat16 of each float64 (ties to even) -> bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    f = lib().ds4o_round_bf16
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def e4m3_to_f64(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    f = lib().ds4o_e4m3_to_f64
    return np.array([f(int(v)) for v in c.ravel()], dtype=np.float64).reshape(c.shape)


def round_e4m3(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    f = lib().ds4o_round_e4m3
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint8).reshape(x.shape)


def compress_row(state_kv, state_score, gain, eps: float = 1e-6, n_rot: int = 64, pos: int = 0,
                 theta: float = 10000.0, fp8: bool = True):
    """One emitted row: state_kv, state_score f32 [ratio, width], gain f32 [width]
    -> (bf16 bits [width], y before the FP8 step float64 [width], the row's FP8 scale)."""
    kv = np.ascontiguousarray(state_kv, dtype=np.float32)
    sc = np.ascontiguousarray(state_score, dtype=np.float32)
    g = np.ascontiguousarray(gain, dtype=np.float32)
    ratio, width = kv.shape
    assert sc.shape == kv.shape and g.shape == (width,)
    out = np.empty(width, dtype=np.uint16)
    y = np.empty(width, dtype=np.float64)
    scale = ctypes.c_double(0.0)
    rc = lib().ds4o_compress_row(width, ratio, _p(kv), _p(sc), _p(g), float(eps), int(n_rot), int(pos),
                                 float(theta), 1 if fp8 else 0, _p(y), ctypes.byref(scale), _p(out))
    if rc != 0:
        raise ValueError(f"ds4o_compress_row rejected its arguments (rc={rc})")
    return out, y, scale.value


def compress_row_e4m3(state_kv, state_score, gain, eps: float = 1e-6, n_rot: int = 64, pos: int = 0,
                      theta: float = 10000.0):
    """The FP8 row of compress_row as stored: (E4M3FN codes uint8 [width], the row's scale)."""
    kv = np.ascontiguousarray(state_kv, dtype=np.float32)
    sc = np.ascontiguousarray(state_score, dtype=np.float32)
    g = np.ascontiguousarray(gain, dtype=np.float32)
    ratio, width = kv.shape
    codes = np.empty(width, dtype=np.uint8)
    scale = ctypes.c_double(0.0)
    rc = lib().ds4o_compress_row_e4m3(width, ratio, _p(kv), _p(sc), _p(g), float(eps), int(n_rot), int(pos),
                                      float(theta), _p(codes), ctypes.byref(scale))
    if rc != 0:
        raise ValueError(f"ds4o_compress_row_e4m3 rejected its arguments (rc={rc})")
    return codes, scale.value


def push_raw(raw, n_raw: int, kv):
    """Raw-window push of one unit: raw f16 bits [cap, D] holding n_raw rows, kv f32 [T, D]
    -> (new window f16 bits [cap, D], new n_raw).  The inputs are not modified."""
    w = np.array(raw, dtype=np.uint16, copy=True, order="C")
    x = np.ascontiguousarray(kv, dtype=np.float32)
    cap, D = w.shape
    T = x.shape[0]
    assert x.shape == (T, D)
    n = ctypes.c_int32(int(n_raw))
    lib().ds4o_push_raw(cap, D, T, _p(x), _p(w), ctypes.byref(n))
    return w, n.value


def frontier_push(state_kv, state_score, pos: int, kv, score, ape):
    """One token into one unit's frontier -> (new state_kv, new state_score), f32 [ratio, width]."""
    skv = np.array(state_kv, dtype=np.float32, copy=True, order="C")
    ssc = np.array(state_score, dtype=np.float32, copy=True, order="C")
    ratio, width = skv.shape
    k = np.ascontiguousarray(kv, dtype=np.float32)
    s = np.ascontiguousarray(score, dtype=np.float32)
    a = np.ascontiguousarray(ape, dtype=np.float32)
    assert k.shape == (width,) and s.shape == (width,) and a.shape == (ratio, width)
    lib().ds4o_frontier_push(width, ratio, int(pos), _p(k), _p(s), _p(a), _p(skv), _p(ssc))
    return skv, ssc
