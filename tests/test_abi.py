"""The C-ABI library: loads, exports what the header declares, and validates its
arguments on the host (no GPU needed: every call here is rejected before any HIP call)."""
import ctypes

import pytest

from sparse_compressed_kv_amd import ops

A = 0x10000          # a 16-byte aligned stand-in for a device pointer (never dereferenced)
MIS = 0x10004        # misaligned stand-in
S = None             # null stream


@pytest.fixture(scope="module")
def L():
    return ops.lib()


def test_exports_every_declared_symbol(L):
    names = ops.declared_symbols()
    assert {"ds4a_indexer_score", "ds4a_topk_select", "ds4a_indexer_topk", "ds4a_sparse_mqa", "ds4a_dense_mqa",
            "ds4a_compress_rows", "ds4a_rope_q", "ds4a_indexer_score_fp8", "ds4a_indexer_topk_fp8",
            "ds4a_compress_append", "ds4a_push_raw", "ds4a_frontier_push", "ds4a_sparse_mqa_fp8",
            "ds4a_dense_mqa_fp8", "ds4a_indexer_topk_mqa", "ds4a_indexer_topk_mqa_fp8", "ds4a_workspace_bytes",
            "ds4a_last_error", "ds4a_version"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_ceiling_validation(L):
    """The measured-ceiling kernels refuse bad arguments before launching anything."""
    import ctypes as ct
    sink = A
    assert L.ds4a_ceiling_read(None, 1 << 20, 64, sink, S) == -1
    assert L.ds4a_ceiling_read(MIS, 1 << 20, 64, sink, S) == -1
    assert L.ds4a_ceiling_read(A, (1 << 20) + 4, 64, sink, S) == -1
    assert L.ds4a_ceiling_read(A, 1 << 20, 0, sink, S) == -1
    assert L.ds4a_ceiling_read(A, 1 << 20, 64, None, S) == -1
    fl = ct.c_double(0.0)
    assert L.ds4a_ceiling_mfma(0, 64, sink, ct.byref(fl), S) == -1
    assert L.ds4a_ceiling_mfma(10, 0, sink, ct.byref(fl), S) == -1
    assert L.ds4a_ceiling_mfma(10, 64, None, ct.byref(fl), S) == -1


def test_version(L):
    assert L.ds4a_version() == 3


def test_indexer_validation(L):
    f = L.ds4a_indexer_score
    assert f(0, 1, 10, 64, 128, A, A, A, None, A, S) == -2
    assert f(1, 1, 0, 64, 128, A, A, A, None, A, S) == -2
    assert f(1, 1, 10, 32, 128, A, A, A, None, A, S) == -3
    assert "Hi=32" in ops.last_error()
    assert f(1, 1, 10, 64, 64, A, A, A, None, A, S) == -3
    assert f(1, 1, 10, 64, 128, None, A, A, None, A, S) == -1
    assert "idx_q" in ops.last_error()
    assert f(1, 1, 10, 64, 128, A, A, A, None, None, S) == -1
    assert f(1, 1, 10, 64, 128, A, MIS, A, None, A, S) == -4
    assert f(1, 1, 10, 64, 128, A, A, A, MIS, A, S) == -4
    assert f(1, 1, 1 << 31, 64, 128, A, A, A, None, A, S) == -2


def test_topk_validation(L):
    f = L.ds4a_topk_select
    assert f(1, 1, 100, 0, A, None, A, None, 0, S) == -2
    assert f(1, 1, 100, 4096, A, None, A, None, 0, S) == -3
    assert f(1, 1, 100, 16, None, None, A, None, 0, S) == -1
    assert f(1, 1, 100, 16, A, None, MIS, None, 0, S) == -4
    # the multi-workgroup path needs a workspace
    need = ops.workspace_bytes(0, 2, 1, 65536, 512)
    assert need > 0
    assert f(2, 1, 65536, 512, A, None, A, None, 0, S) == -5
    assert f(2, 1, 65536, 512, A, None, A, A, need - 1, S) == -5
    assert "workspace" in ops.last_error()
    assert f(2, 1, 65536, 512, A, None, A, MIS, need, S) == -4


def test_indexer_topk_validation(L):
    f = L.ds4a_indexer_topk
    assert f(0, 1, 10, 64, 128, 8, A, A, A, None, A, None, 0, S) == -2
    assert f(1, 1, 10, 32, 128, 8, A, A, A, None, A, None, 0, S) == -3
    assert f(1, 1, 10, 64, 128, 0, A, A, A, None, A, None, 0, S) == -2
    assert f(1, 1, 10, 64, 128, 4096, A, A, A, None, A, None, 0, S) == -3
    assert f(1, 1, 10, 64, 128, 8, None, A, A, None, A, None, 0, S) == -1
    assert f(1, 1, 10, 64, 128, 8, A, A, A, None, None, None, 0, S) == -1
    assert f(1, 1, 10, 64, 128, 8, A, A, A, MIS, A, None, 0, S) == -4
    # more than one 8192-row chunk: candidate lists need a workspace
    need = ops.workspace_bytes(2, 2, 1, 65536, 512)
    assert need > 0
    assert f(2, 1, 65536, 64, 128, 512, A, A, A, None, A, None, 0, S) == -5
    assert f(2, 1, 65536, 64, 128, 512, A, A, A, None, A, A, need - 1, S) == -5
    assert f(2, 1, 65536, 64, 128, 512, A, A, A, None, A, MIS, need, S) == -4


def test_indexer_fp8_validation(L):
    f = L.ds4a_indexer_score_fp8
    assert f(0, 1, 10, 64, 128, A, A, A, A, None, A, S) == -2
    assert f(1, 1, 10, 64, 64, A, A, A, A, None, A, S) == -3
    assert f(1, 1, 10, 64, 128, A, A, None, A, None, A, S) == -1
    assert "idx_k8" in ops.last_error()
    assert f(1, 1, 10, 64, 128, A, A, A, None, None, A, S) == -1
    assert "idx_k_scale" in ops.last_error()
    assert f(1, 1, 10, 64, 128, A, A, MIS, A, None, A, S) == -4
    assert f(1, 1, 10, 64, 128, A, A, A, MIS, None, A, S) == -4
    assert "idx_k_scale" in ops.last_error()
    assert f(1, 1, 10, 64, 128, A, A, A, A, None, None, S) == -1
    g = L.ds4a_indexer_topk_fp8
    assert g(1, 1, 10, 64, 128, 0, A, A, A, A, None, A, None, 0, S) == -2
    assert g(1, 1, 10, 64, 128, 8, A, A, None, A, None, A, None, 0, S) == -1
    assert "ds4a_indexer_topk_fp8" in ops.last_error() and "idx_k8" in ops.last_error()
    assert g(1, 1, 10, 64, 128, 8, A, A, A, None, None, A, None, 0, S) == -1
    assert g(1, 1, 10, 64, 128, 8, A, A, A, A, None, None, None, 0, S) == -1
    need = ops.workspace_bytes(2, 2, 1, 65536, 512)
    assert g(2, 1, 65536, 64, 128, 512, A, A, A, A, None, A, None, 0, S) == -5
    assert g(2, 1, 65536, 64, 128, 512, A, A, A, A, None, A, MIS, need, S) == -4
    # the bf16 entry point still names its own key argument
    assert L.ds4a_indexer_topk(1, 1, 10, 64, 128, 8, A, A, None, None, A, None, 0, S) == -1
    assert "idx_k " in ops.last_error() or ops.last_error().endswith("idx_k is NULL")


def test_cache_upkeep_validation(L):
    p = L.ds4a_push_raw
    assert p(0, 1, 512, 128, A, A, A, S) == -2
    assert p(1, 0, 512, 128, A, A, A, S) == -2
    assert p(1, 1, 500, 128, A, A, A, S) == -2
    assert p(1, 1, 512, 0, A, A, A, S) == -2
    assert p(1, 1, 512, 2048, A, A, A, S) == -3
    assert p(1, 1, 8192, 128, A, A, A, S) == -3
    assert p(1, 1, 512, 128, None, A, A, S) == -1
    assert p(1, 1, 512, 128, A, A, None, S) == -1 and "n_raw" in ops.last_error()
    assert p(1, 1, 512, 128, A, MIS, A, S) == -4
    f = L.ds4a_frontier_push
    assert f(1, 6, 4, A, A, A, A, A, A, S) == -2
    assert f(1, 128, 0, A, A, A, A, A, A, S) == -2
    assert f(1, 2048, 4, A, A, A, A, A, A, S) == -3
    assert f(1, 128, 4, A, A, None, A, A, A, S) == -1 and "ape" in ops.last_error()
    assert f(1, 128, 4, A, A, A, A, A, MIS, S) == -4
    c = L.ds4a_compress_append

    def ca(**kw):
        a = dict(U=2, width=128, ratio=4, kv=A, sc=A, gain=A, eps=1e-6, n_rot=64, pos=A, row_pos=A, theta=1e4,
                 fmt=2, comp=A, scale=A, cap=16, n=A)
        a.update(kw)
        return c(a["U"], a["width"], a["ratio"], a["kv"], a["sc"], a["gain"], a["eps"], a["n_rot"], a["pos"],
                 a["row_pos"], a["theta"], a["fmt"], a["comp"], a["scale"], a["cap"], a["n"], S)

    assert ca(fmt=3) == -6
    assert ca(cap=0) == -2
    assert ca(cap=1 << 40) == -2
    assert ca(width=130) == -2
    assert ca(ratio=2000) == -3
    assert ca(scale=None) == -1 and "comp_scale" in ops.last_error()
    assert ca(n=None) == -1 and "n_comp" in ops.last_error()
    assert ca(pos=MIS) == -4
    assert ca(eps=-1.0) == -2


def _mqa(L, **kw):
    a = dict(U=1, T=1, H=64, D=512, n_rot=64, W=128, N=1000, K=512, q=A, q_dtype=0, q_pos=A, theta=10000.0,
             raw=A, raw_vis=None, comp=A, idx=A, scale=0.044, out=A, ws=A, ws_bytes=1 << 30)
    a.update(kw)
    return L.ds4a_sparse_mqa(a["U"], a["T"], a["H"], a["D"], a["n_rot"], a["W"], a["N"], a["K"], a["q"],
                             a["q_dtype"], a["q_pos"], a["theta"], a["raw"], a["raw_vis"], a["comp"], a["idx"],
                             a["scale"], a["out"], a["ws"], a["ws_bytes"], S)


def test_mqa_validation(L):
    assert _mqa(L, D=256) == -3
    assert _mqa(L, n_rot=32) == -3
    assert _mqa(L, H=48 + 1) == -3
    assert _mqa(L, H=144) == -3
    assert _mqa(L, W=100) == -3
    assert _mqa(L, K=0) == -2
    assert _mqa(L, K=4096) == -3
    assert _mqa(L, q_dtype=2) == -3
    assert _mqa(L, q_dtype=7) == -6
    assert _mqa(L, theta=0.0) == -2
    assert _mqa(L, scale=float("nan")) == -2
    assert _mqa(L, q=None) == -1
    assert _mqa(L, comp=MIS) == -4
    assert _mqa(L, raw_vis=MIS) == -4 and "raw_vis" in ops.last_error()
    assert _mqa(L, U=0) == -2
    need = ops.workspace_bytes(1, 1, 1, 1000, 512, 64, 128)
    assert need > 0                       # one query: the union is split over workgroups
    assert _mqa(L, ws=None, ws_bytes=0) == -5
    assert _mqa(L, ws_bytes=need - 1) == -5
    assert _mqa(L, U=1 << 16, T=1 << 9) == -2     # U*T above 2^24 (keeps every grid below 2^31)


def test_indexer_topk_mqa_validation(L):
    """A1 + A2 + A3-A6 in one call validates both halves' arguments before anything is enqueued,
    and always needs a workspace (the top-k's and the attention's)."""
    def st(fp8=False, **kw):
        a = dict(U=43, T=1, N=65536, Hi=64, Di=128, K=512, iq=A, iw=A, ik=A, iks=A, n_vis=None, H=64, D=512,
                 n_rot=64, W=128, q=A, q_dtype=0, q_pos=A, theta=10000.0, raw=A, raw_vis=None, comp=A, cs=A,
                 scale=0.044, idx=A, out=A, ws=A, ws_bytes=1 << 40)
        a.update(kw)
        if fp8:
            return L.ds4a_indexer_topk_mqa_fp8(
                a["U"], a["T"], a["N"], a["Hi"], a["Di"], a["K"], a["iq"], a["iw"], a["ik"], a["iks"], a["n_vis"],
                a["H"], a["D"], a["n_rot"], a["W"], a["q"], a["q_dtype"], a["q_pos"], a["theta"], a["raw"],
                a["raw_vis"], a["comp"], a["cs"], a["scale"], a["idx"], a["out"], a["ws"], a["ws_bytes"], S)
        return L.ds4a_indexer_topk_mqa(
            a["U"], a["T"], a["N"], a["Hi"], a["Di"], a["K"], a["iq"], a["iw"], a["ik"], a["n_vis"], a["H"], a["D"],
            a["n_rot"], a["W"], a["q"], a["q_dtype"], a["q_pos"], a["theta"], a["raw"], a["raw_vis"], a["comp"],
            a["scale"], a["idx"], a["out"], a["ws"], a["ws_bytes"], S)

    assert st(Hi=32) == -3 and "ds4a_indexer_topk_mqa" in ops.last_error()
    assert st(D=256) == -3
    assert st(K=0) == -2
    assert st(K=4096) == -3
    assert st(W=100) == -3
    assert st(N=0) == -2
    assert st(scale=float("inf")) == -2
    assert st(iq=None) == -1 and "idx_q" in ops.last_error()
    assert st(ik=MIS) == -4
    assert st(comp=None) == -1 and "comp_kv" in ops.last_error()
    assert st(out=None) == -1
    assert st(raw_vis=MIS) == -4
    assert st(idx=MIS) == -4                  # idx may be NULL, but not misaligned
    need = ops.workspace_bytes(4, 43, 1, 65536, 512, 64, 128)
    assert need >= ops.workspace_bytes(2, 43, 1, 65536, 512, 0, 0) + 43 * 512 * 4
    assert st(ws=None, ws_bytes=0) == -5 and "workspace" in ops.last_error()
    assert st(ws_bytes=need - 1) == -5
    assert st(ws=MIS) == -4
    assert st(fp8=True, ik=None) == -1 and "idx_k8" in ops.last_error()
    assert st(fp8=True, iks=None) == -1 and "idx_k_scale" in ops.last_error()
    assert st(fp8=True, cs=None) == -1 and "comp_scale" in ops.last_error()
    assert ops.workspace_bytes(4, 1, 1, 1000, 512, 48 + 1, 128) == 0


def test_mqa_noalloc_validation(L):
    """The allocation-free attention validates as ds4a_sparse_mqa and refuses, before touching
    the GPU, a split whose records would not fit the library's scratch."""
    def na(**kw):
        a = dict(U=1, T=1, H=64, D=512, n_rot=64, W=128, N=1000, K=512, q=A, q_dtype=0, q_pos=A, theta=10000.0,
                 raw=A, raw_vis=None, comp=A, idx=A, scale=0.044, out=A)
        a.update(kw)
        return L.ds4a_sparse_mqa_noalloc(a["U"], a["T"], a["H"], a["D"], a["n_rot"], a["W"], a["N"], a["K"], a["q"],
                                         a["q_dtype"], a["q_pos"], a["theta"], a["raw"], a["raw_vis"], a["comp"],
                                         a["idx"], a["scale"], a["out"], S)

    assert na(D=256) == -3
    assert na(K=0) == -2
    assert na(q=None) == -1 and "ds4a_sparse_mqa_noalloc" in ops.last_error()
    assert na(comp=MIS) == -4
    # 32 queries x 128 heads over a 3072-row union: two chunks of 16.8 MB of records
    need = ops.workspace_bytes(1, 32, 1, 4096, 2048, 128, 1024)
    assert need > (16 << 20)
    assert na(U=32, H=128, W=1024, N=4096, K=2048) == -5 and "scratch" in ops.last_error()


def test_mqa_fp8_validation(L):
    def sp(**kw):
        a = dict(U=1, T=1, H=64, D=512, n_rot=64, W=128, N=1000, K=512, q=A, q_dtype=0, q_pos=A, theta=10000.0,
                 raw=A, raw_vis=None, comp=A, cs=A, idx=A, scale=0.044, out=A, ws=None, ws_bytes=0)
        a.update(kw)
        return L.ds4a_sparse_mqa_fp8(a["U"], a["T"], a["H"], a["D"], a["n_rot"], a["W"], a["N"], a["K"], a["q"],
                                     a["q_dtype"], a["q_pos"], a["theta"], a["raw"], a["raw_vis"], a["comp"],
                                     a["cs"], a["idx"], a["scale"], a["out"], a["ws"], a["ws_bytes"], S)

    assert sp(D=256) == -3
    assert sp(comp=None) == -1 and "comp_kv8" in ops.last_error()
    assert sp(cs=None) == -1 and "comp_scale" in ops.last_error()
    assert sp(cs=MIS) == -4
    assert sp(raw_vis=MIS) == -4 and "raw_vis" in ops.last_error()
    assert sp(idx=None) == -1
    assert sp() == -5                      # one query: the union is split, a workspace is needed

    def de(**kw):
        a = dict(U=1, T=1, H=64, D=512, n_rot=64, W=128, N=1000, q=A, q_dtype=0, q_pos=A, theta=10000.0,
                 raw=A, raw_vis=None, comp=A, cs=A, n_vis=None, scale=0.044, out=A, ws=None, ws_bytes=0)
        a.update(kw)
        return L.ds4a_dense_mqa_fp8(a["U"], a["T"], a["H"], a["D"], a["n_rot"], a["W"], a["N"], a["q"], a["q_dtype"],
                                    a["q_pos"], a["theta"], a["raw"], a["raw_vis"], a["comp"], a["cs"], a["n_vis"],
                                    a["scale"], a["out"], a["ws"], a["ws_bytes"], S)

    assert de(cs=None) == -1 and "ds4a_dense_mqa_fp8" in ops.last_error()
    assert de(N=-1) == -2
    assert de() == -5
    # the bf16 entry point still names its own argument
    assert _mqa(L, comp=None) == -1 and "comp_kv " in ops.last_error() + " "


def _dense(L, **kw):
    a = dict(U=1, T=1, H=64, D=512, n_rot=64, W=128, N=1000, q=A, q_dtype=0, q_pos=A, theta=10000.0,
             raw=A, raw_vis=None, comp=A, n_vis=None, scale=0.044, out=A, ws=A, ws_bytes=1 << 30)
    a.update(kw)
    return L.ds4a_dense_mqa(a["U"], a["T"], a["H"], a["D"], a["n_rot"], a["W"], a["N"], a["q"], a["q_dtype"],
                            a["q_pos"], a["theta"], a["raw"], a["raw_vis"], a["comp"], a["n_vis"], a["scale"],
                            a["out"], a["ws"], a["ws_bytes"], S)


def test_dense_mqa_validation(L):
    assert _dense(L, U=0) == -2
    assert _dense(L, N=-1) == -2
    assert _dense(L, N=(1 << 20) + 1) == -3
    assert _dense(L, W=0, N=0) == -2                 # nothing to attend
    assert _dense(L, H=40) == -3
    assert _dense(L, W=100) == -3
    assert _dense(L, q_dtype=7) == -6
    assert _dense(L, scale=float("inf")) == -2
    assert _dense(L, q=None) == -1
    assert _dense(L, comp=None) == -1                # N > 0 needs the rows
    assert _dense(L, raw=None) == -1                 # W > 0 needs the window
    assert _dense(L, n_vis=MIS) == -4
    assert _dense(L, raw_vis=MIS) == -4 and "raw_vis" in ops.last_error()
    need = ops.workspace_bytes(3, 1, 1, 1000, 0, 64, 128)
    assert need > 0                                  # one query: split over workgroups
    assert _dense(L, ws=None, ws_bytes=0) == -5
    assert _mqa(L, N=(1 << 22)) == -3                # 32-bit row offsets: at most 2^22 - 1 rows
    # one query, raw window only (8 steps of 16 rows): split over 2 workgroups
    assert ops.workspace_bytes(3, 1, 1, 0, 0, 64, 128) > 0
    assert ops.workspace_bytes(3, 4, 1, 3000, 0, 128, 128) > 0     # 4 Pro queries: split
    assert ops.workspace_bytes(3, 1, 1, 0, 0, 64, 0) == 0          # nothing to attend
    assert ops.workspace_bytes(3, 1, 1, -1, 0, 64, 128) == 0
    assert ops.workspace_bytes(3, 300, 1, 0, 0, 64, 128) == 0      # enough queries: no split
    assert ops.workspace_bytes(3, 1, 300, 3000, 0, 16, 32) == 0    # 190 steps: one chunk
    assert ops.workspace_bytes(3, 1, 300, 3100, 0, 16, 32) > 0     # 196 steps > 192 per chunk: split


def _compress(L, **kw):
    a = dict(U=2, width=512, ratio=4, kv=A, sc=A, gain=A, eps=1e-6, n_rot=64, pos=A, theta=10000.0, fp8=1, out=None,
             stride=512)
    a.update(kw)
    return L.ds4a_compress_rows(a["U"], a["width"], a["ratio"], a["kv"], a["sc"], a["gain"], a["eps"], a["n_rot"],
                                a["pos"], a["theta"], a["fp8"], a["out"], a["stride"], S)


def test_compress_rows_validation(L):
    assert _compress(L, U=0) == -2
    assert _compress(L, width=511) == -2
    assert _compress(L, width=514) == -2             # a multiple of 4
    assert _compress(L, ratio=0) == -2
    assert _compress(L, n_rot=63) == -2
    assert _compress(L, n_rot=514) == -2            # more than width
    assert _compress(L, width=2048, n_rot=64, stride=2048) == -3
    assert _compress(L, ratio=2048) == -3
    assert _compress(L, eps=-1.0) == -2
    assert _compress(L, theta=0.0) == -2
    assert _compress(L, fp8=2) == -2
    assert _compress(L, stride=100) == -2
    assert _compress(L, kv=None) == -1
    assert _compress(L, pos=MIS) == -4
    assert _compress(L) == -1                       # out is NULL: checked last, nothing enqueued
    assert "out" in ops.last_error()


def test_rope_validation(L):
    f = L.ds4a_rope_q
    assert f(1, 1, 64, 512, 64, None, 0, A, 10000.0, A, S) == -1
    assert f(1, 1, 64, 512, 32, A, 0, A, 10000.0, A, S) == -3
    assert f(1, 1, 64, 512, 64, A, 5, A, 10000.0, A, S) == -6


def test_workspace_bytes(L):
    assert ops.workspace_bytes(0, 43, 1, 8192, 512) == 0             # one workgroup per query
    assert ops.workspace_bytes(0, 2048, 1, 16384, 512) == 0          # many queries: still direct
    assert ops.workspace_bytes(0, 43, 1, 16384, 512) > 0             # chunked: candidate lists
    assert ops.workspace_bytes(0, 8, 1, 262144, 512) >= 2 * 8 * 16 * 512 * 8
    assert ops.workspace_bytes(3, 1, 1, 10, 10) == 0                  # unknown `which`
    assert ops.workspace_bytes(1, 1, 2048, 8192, 512, 64, 128) == 0   # prefill: no split
    assert ops.workspace_bytes(1, 1, 1, 10, 512, 64, 100) == 0        # invalid W
    assert ops.workspace_bytes(2, 256, 1, 2048, 512) == 0            # fused: one chunk, no candidates
    assert ops.workspace_bytes(2, 4, 1, 65536, 1024) >= 4 * 65536 * 4  # too few chunks: scores kept
    assert ops.workspace_bytes(2, 43, 1, 65536, 512) >= 2 * 43 * 11 * 512 * 8  # 11 chunks of candidates
    assert ops.workspace_bytes(2, 1, 2048, 8192, 512) >= 2048 * 8192 * 4       # many queries: scores


@pytest.mark.parametrize("U,T,N,K", [
    (300, 1, 2048, 512), (100, 3, 2048, 512), (200, 1, 8197, 512), (43, 1, 65536, 512),
    (43, 1, 16384, 512), (43, 1, 65537, 1024), (8, 1, 262144, 512), (40, 1, 100000, 2048),
    (50, 3, 20000, 7), (70, 2, 3000, 64), (130, 1, 9000, 512), (4, 1, 65536, 1024),
    (3, 1, 8193, 512), (1, 2, 100000, 2048), (1, 4, 65536, 512), (64, 1, 4096, 512),
])
def test_indexer_topk_routing_matches_library(U, T, N, K):
    """The host restatement of the fused call's chunk rule agrees with the library's sizes."""
    from tests import routing
    got = ops.workspace_bytes(2, U, T, N, K)
    if routing.uses_fused(U, T, N, K):
        assert got == routing.fused_workspace_bytes(U, T, N, K)
    else:
        assert got >= ((U * T * N * 4 + 255) & ~255)


def test_last_error_is_text(L):
    L.ds4a_topk_select(1, 1, 100, 0, A, None, A, None, 0, S)
    assert isinstance(ops.last_error(), str) and "K=0" in ops.last_error()


def test_single_hip_runtime_after_torch():
    import torch  # noqa: F401  torch's runtime is loaded first, the library reuses it
    ops.lib()
    assert len(ops.hip_runtimes_mapped()) == 1, ops.hip_runtimes_mapped()
