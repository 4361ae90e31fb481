"""GPU parity: every step of the HIP path against the CPU oracle on the same seeded inputs.

Bars (from the problem statement): selected index sets bit-exact on identical fp32
scores, and against the fp64 oracle equal apart from rows whose scores lie within
1e-5 (relative) of the K-th score; attention outputs within a normwise relative
error of 2e-3 per (unit, query).  The hi/lo bf16 operand design is also held to
1e-4, far inside that bar, so that losing one of the split terms is caught.
"""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from sparse_compressed_kv_amd import ops
from synth import inputs as gen
from tests import routing
from tests.util import bits_to_torch, normwise_err, tie_band_ok, upload

pytestmark = pytest.mark.gpu

CONTRACT_ERR = 2e-3
DESIGN_ERR = 1e-4


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ops.lib()
    return torch.device("cuda")


def bf16_f64(bits):
    return gen.bf16_bits_to_f32(bits).astype(np.float64)


# ------------------------------------------------------------------- RoPE

@pytest.mark.parametrize("qd", ["f32", "bf16"])
def test_rope_matches_oracle(qd):
    rng = np.random.default_rng(5)
    U, T, H = 2, 3, 32
    qf = rng.standard_normal((U, T, H, 512)).astype(np.float32)
    pos = np.array([[0, 1, 8191], [262143, 1048575, 4096]], dtype=np.int64)
    if qd == "bf16":
        qb = gen.bf16_bits_from_f32(qf)
        q_dev, q64 = bits_to_torch(qb, torch.bfloat16), bf16_f64(qb)
    else:
        q_dev, q64 = torch.from_numpy(qf).cuda(), qf.astype(np.float64)
    got = ops.rope_q(q_dev, torch.from_numpy(pos).cuda()).cpu().numpy()
    for u in range(U):
        for t in range(T):
            ref = orc.rope_q(q64[u, t], pos[u, t])
            assert np.all(np.abs(got[u, t] - ref) <= 1e-6 * (1.0 + np.abs(ref))), (u, t)
            assert np.array_equal(got[u, t, :, :448], ref[:, :448].astype(np.float32))


# ---------------------------------------------------------------- indexer

INDEXER_CASES = [
    dict(U=1, T=1, N=1, nv=None),
    dict(U=2, T=3, N=700, nv=[[700, 0, 333], [1, 699, 16]]),
    dict(U=3, T=1, N=4097, nv=None, heavy=0.01),
    dict(U=1, T=5, N=257, nv=[[0, 1, 128, 256, 257]]),
    # many queries per unit: the key-tile-sharing path (8 queries per workgroup, split key ranges)
    dict(U=2, T=9, N=700, nv="rand"),
    dict(U=1, T=16, N=1001, nv="rand"),
    dict(U=1, T=8, N=4096, nv="full"),
    dict(U=1, T=24, N=2048, nv="causal"),
]


def _indexer_nv(case, U, T, N):
    nv = case["nv"]
    if nv is None or nv == "full":
        return np.full((U, T), N, np.int32)
    if nv == "rand":
        r = np.random.default_rng(5).integers(0, N + 1, (U, T)).astype(np.int32)
        r.flat[0], r.flat[-1] = 0, N
        return r
    if nv == "causal":
        return np.tile((N // 2 + 37 * np.arange(T)).clip(0, N).astype(np.int32), (U, 1))
    return np.array(nv, dtype=np.int32)


@pytest.mark.parametrize("case", INDEXER_CASES, ids=lambda c: f"U{c['U']}T{c['T']}N{c['N']}")
def test_indexer_matches_oracle(case):
    w = gen.Workload("idx", 101, U=case["U"], T=case["T"], N=case["N"], H=16, K=64,
                     heavy_frac=case.get("heavy", 0.0))
    x = gen.make_config(w, seed=1)
    nv = _indexer_nv(case, w.U, w.T, w.N)
    d = upload(x)
    got = ops.indexer_score(d["idx_q"], d["idx_w"], d["idx_k"], n_vis=torch.from_numpy(nv).cuda()).cpu().numpy()
    for u in range(w.U):
        kabs = np.abs(bf16_f64(x["idx_k"][u]))
        for t in range(w.T):
            ref = orc.indexer_score(x["idx_q"][u, t], x["idx_w"][u, t], x["idx_k"][u], n_vis=int(nv[u, t]))
            v = int(nv[u, t])
            assert np.all(np.isneginf(got[u, t, v:]))
            # fp32 accumulation bound: a few ulps of the absolute-value sum of all terms
            bound = (x["idx_w"][u, t].astype(np.float64)[:, None] *
                     (np.abs(bf16_f64(x["idx_q"][u, t])) @ kabs.T)).sum(0)[:v]
            err = np.abs(got[u, t, :v].astype(np.float64) - ref[:v])
            assert np.all(err <= 2e-6 * bound + 1e-30), (u, t, float((err / np.maximum(bound, 1e-30)).max()))


# ------------------------------------------------------------------ top-k

def _scores(pattern, n, rng):
    if pattern == "normal":
        return rng.standard_normal(n).astype(np.float32) * np.float32(50.0)
    if pattern == "ties":
        return rng.integers(0, 40, n).astype(np.float32)
    if pattern == "equal":
        return np.full(n, 3.25, np.float32)
    if pattern == "zeros":   # +0 and -0 are equal floats
        s = np.zeros(n, np.float32)
        s[rng.random(n) < 0.5] = -0.0
        s[rng.random(n) < 0.01] = 1.0
        return s
    if pattern == "low":     # keys with a zero top byte (large negative scores) hold the boundary
        s = np.float32(-3e38) * (np.float32(1.0) - rng.random(n).astype(np.float32) * np.float32(1e-3))
        few = rng.random(n) < 0.05
        s[few] = rng.standard_normal(int(few.sum())).astype(np.float32) * np.float32(50.0)
        return s
    if pattern == "heavy":
        s = np.abs(rng.standard_normal(n)).astype(np.float32) * np.float32(100.0) + np.float32(10.0)
        s[rng.choice(n, max(1, n // 100), replace=False)] *= np.float32(4.0)
        return s
    raise ValueError(pattern)


TOPK_CASES = [
    (1, 1, 1, "normal"), (2, 63, 64, "normal"), (1, 64, 64, "ties"), (3, 511, 512, "normal"),
    (1, 512, 512, "equal"), (2, 513, 512, "ties"), (2, 4095, 512, "zeros"), (2, 16384, 512, "heavy"),
    (2, 16384, 2048, "ties"), (2, 16385, 512, "normal"), (2, 40961, 1024, "heavy"), (1, 65537, 512, "equal"),
    (2, 65537, 1024, "ties"), (1, 262144, 512, "normal"), (1, 100000, 2048, "zeros"), (3, 20000, 7, "normal"),
    (3, 4095, 512, "low"), (3, 40000, 1024, "low"),
]


@pytest.mark.parametrize("Q,N,K,pattern", TOPK_CASES, ids=lambda v: str(v))
def test_topk_bit_exact_on_identical_scores(Q, N, K, pattern):
    rng = np.random.default_rng(N * 31 + K)
    s = np.stack([_scores(pattern, N, rng) for _ in range(Q)]).reshape(Q, 1, N)
    nv = rng.integers(0, N + 1, Q).astype(np.int32)
    nv[0] = N
    if Q > 1:
        nv[1] = min(N, max(0, K - 3))
    sd = torch.from_numpy(s).cuda()
    out = torch.full((Q, 1, K), -7, dtype=torch.int32, device="cuda")
    ops.topk_select(sd, K, n_vis=torch.from_numpy(nv.reshape(Q, 1)).cuda(), out=out)
    got = out.cpu().numpy()
    for i in range(Q):
        ref = orc.topk(s[i, 0].astype(np.float64), K, n_vis=int(nv[i]))
        n_sel = min(K, int(nv[i]))
        assert np.array_equal(got[i, 0, :n_sel], np.sort(ref[:n_sel])), (i, int(nv[i]))
        assert np.all(got[i, 0, n_sel:] == -1)


# ------------------------------------------------------- fused indexer + top-k

FUSED_CASES = [
    # too few chunk workgroups: scores through the workspace
    dict(U=3, T=1, N=1, K=1, nv=None, ept=None),
    dict(U=3, T=1, N=8193, K=512, nv=[[8193], [0], [300]], ept=None),
    dict(U=1, T=2, N=100000, K=2048, nv=[[100000, 2047]], ept=None),
    # fused: every chunk size, one chunk (direct output) to two merge levels
    dict(U=200, T=1, N=2048, K=512, nv="edges", ept=4),        # one chunk
    dict(U=100, T=3, N=2048, K=512, nv="edges", ept=4),
    dict(U=200, T=1, N=8197, K=512, nv="edges", ept=4),
    dict(U=43, T=1, N=65536, K=512, nv=None, heavy=0.01, ept=12),
    dict(U=43, T=1, N=65537, K=1024, nv="edges", ept=8),
    dict(U=8, T=1, N=262144, K=512, nv="edges", ept=8),
    dict(U=8, T=1, N=262144, K=2048, nv="edges", ept=16),      # two merge levels
    dict(U=64, T=1, N=50000, K=512, nv="edges", ept=16),
    dict(U=40, T=1, N=100000, K=2048, nv="edges", ept=12),
    dict(U=50, T=3, N=20000, K=7, nv=None, ept=8),
    dict(U=64, T=1, N=4096, K=512, nv="edges", ept=4),
    dict(U=70, T=2, N=3000, K=64, nv="edges", ept=4),
    dict(U=128, T=1, N=2000, K=2048, nv="edges", ept=4),      # chunks of fewer than 2K key slots
]


def _fused_nv(case, rows):
    """Visible rows per query: random, with the first queries on the edges of K and of a chunk."""
    U, T, N, K = case["U"], case["T"], case["N"], case["K"]
    nv = case["nv"]
    if nv is None:
        return np.full((U, T), N, np.int32)
    if nv != "edges":
        return np.array(nv, dtype=np.int32)
    r = np.random.default_rng(7).integers(0, N + 1, U * T)
    edges = [0, 1, K - 1, K, K + 1, rows - 1, rows, rows + 1, 2 * rows + 3, N - 1, N]
    edges = [e for e in edges if 0 <= e <= N]
    r[:len(edges)] = edges[:len(r)]
    return r.reshape(U, T).astype(np.int32)


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: f"U{c['U']}T{c['T']}N{c['N']}K{c['K']}")
def test_indexer_topk_equals_separate_calls(case):
    """ds4a_indexer_topk returns exactly topk_select(indexer_score(...)): same bits, same set."""
    U, T, N, K = case["U"], case["T"], case["N"], case["K"]
    fused = routing.uses_fused(U, T, N, K)
    assert fused == (case["ept"] is not None)
    if fused:
        assert routing.fused_shape(U * T, N, K)[0] == case["ept"]
    w = gen.Workload("fus", 105, U=U, T=T, N=N, H=16, K=K, heavy_frac=case.get("heavy", 0.0))
    x = gen.make_indexer_config(w, seed=2)
    nv = _fused_nv(case, routing.fused_shape(U * T, N, K)[1])
    iq = bits_to_torch(x["idx_q"], torch.bfloat16)
    iw = torch.from_numpy(x["idx_w"]).cuda()
    ik = bits_to_torch(x["idx_k"], torch.bfloat16)
    del x
    nvd = torch.from_numpy(nv).cuda()
    scores = ops.indexer_score(iq, iw, ik, n_vis=nvd)
    ref = ops.topk_select(scores, K, n_vis=nvd)
    del scores
    got = torch.full_like(ref, -7)
    ops.indexer_topk(iq, iw, ik, K, n_vis=nvd, out=got)
    assert torch.equal(got, ref)


def test_indexer_topk_all_tied():
    """Every score equal (zero query): the set is rows 0..K-1 across chunk boundaries."""
    w = gen.Workload("fut", 106, U=130, T=1, N=9000, H=16, K=512)
    assert routing.uses_fused(w.U, w.T, w.N, w.K) and routing.fused_shape(w.U, w.N, w.K) == (4, 1296, 7)
    x = gen.make_indexer_config(w, seed=3)
    x["idx_q"][:] = 0
    got = ops.indexer_topk(bits_to_torch(x["idx_q"], torch.bfloat16), torch.from_numpy(x["idx_w"]).cuda(),
                           bits_to_torch(x["idx_k"], torch.bfloat16), w.K).cpu().numpy()
    assert np.array_equal(got[:, 0], np.broadcast_to(np.arange(512, dtype=np.int32), (w.U, 512)))


# ------------------------------------------------------- FP8-stored indexer keys

def _fp8_inputs(U, T, N, seed, heavy=0.0):
    w = gen.Workload("fp8", 107, U=U, T=T, N=N, H=16, K=64, heavy_frac=heavy)
    x = gen.make_indexer_fp8_config(w, seed=seed)
    x["idx_k8"][:, 0, :16] = np.arange(16, dtype=np.uint8)          # zero and subnormal codes
    d = {
        "iq": bits_to_torch(x["idx_q"], torch.bfloat16),
        "iw": torch.from_numpy(x["idx_w"]).cuda(),
        "k8": torch.from_numpy(x["idx_k8"]).cuda(),
        "sc": torch.from_numpy(x["idx_k_scale"]).cuda(),
    }
    return x, d


def _fp8_as_bf16(k8, sc):
    """bf16 keys code value * scale, through torch's own types (exact: the scales are powers of 2)."""
    kf = k8.view(torch.float8_e4m3fn).to(torch.float32) * sc[..., None]
    kb = kf.to(torch.bfloat16)
    assert torch.equal(kb.to(torch.float32), kf)
    return kb


FP8_SCORE_CASES = [c for c in INDEXER_CASES if c["N"] in (1, 700, 4097, 257, 2048)]


@pytest.mark.parametrize("case", FP8_SCORE_CASES, ids=lambda c: f"U{c['U']}T{c['T']}N{c['N']}")
def test_indexer_fp8_matches_oracle_and_bf16_bits(case):
    """FP8 keys: scores within the fp32 bound of the oracle's fp64 scores on the decoded keys, and
    bit-identical to the bf16 entry point's scores on keys code value * scale (both the one-query
    score kernel and the many-queries kernel)."""
    U, T, N = case["U"], case["T"], case["N"]
    x, d = _fp8_inputs(U, T, N, seed=4, heavy=case.get("heavy", 0.0))
    nv = _indexer_nv(case, U, T, N)
    nvd = torch.from_numpy(nv).cuda()
    got_t = ops.indexer_score_fp8(d["iq"], d["iw"], d["k8"], d["sc"], n_vis=nvd)
    ref_t = ops.indexer_score(d["iq"], d["iw"], _fp8_as_bf16(d["k8"], d["sc"]), n_vis=nvd)
    assert torch.equal(got_t.view(torch.int32), ref_t.view(torch.int32))
    got = got_t.cpu().numpy()
    dec = d["k8"].view(torch.float8_e4m3fn).to(torch.float64).cpu().numpy() * x["idx_k_scale"][..., None]
    for u in range(U):
        kabs = np.abs(dec[u])
        for t in range(T):
            v = int(nv[u, t])
            ref = orc.indexer_score_fp8(x["idx_q"][u, t], x["idx_w"][u, t], x["idx_k8"][u], x["idx_k_scale"][u],
                                        n_vis=v)
            assert np.all(np.isneginf(got[u, t, v:]))
            bound = (x["idx_w"][u, t].astype(np.float64)[:, None] *
                     (np.abs(bf16_f64(x["idx_q"][u, t])) @ kabs.T)).sum(0)[:v]
            err = np.abs(got[u, t, :v].astype(np.float64) - ref[:v])
            assert np.all(err <= 2e-6 * bound + 1e-30), (u, t, float((err / np.maximum(bound, 1e-30)).max()))


FP8_TOPK_CASES = [
    dict(U=3, T=1, N=8193, K=512, nv=[[8193], [0], [300]], ept=None),        # scores through the workspace
    dict(U=2, T=16, N=3000, K=512, nv="edges", ept=None),                    # many queries per unit
    dict(U=100, T=3, N=2048, K=512, nv="edges", ept=4),
    dict(U=200, T=1, N=8197, K=512, nv="edges", ept=4),
    dict(U=43, T=1, N=65536, K=512, nv=None, heavy=0.01, ept=12),
    dict(U=8, T=1, N=262144, K=512, nv="edges", ept=8),
    dict(U=64, T=1, N=50000, K=512, nv="edges", ept=16),
    dict(U=70, T=2, N=3000, K=64, nv="edges", ept=4),
]


@pytest.mark.parametrize("case", FP8_TOPK_CASES, ids=lambda c: f"U{c['U']}T{c['T']}N{c['N']}K{c['K']}")
def test_indexer_topk_fp8_equals_bf16(case):
    """ds4a_indexer_topk_fp8 selects exactly the rows ds4a_indexer_topk selects on keys code value *
    scale, on every route (fused chunk sizes, scores through the workspace, many queries)."""
    U, T, N, K = case["U"], case["T"], case["N"], case["K"]
    assert routing.uses_fused(U, T, N, K) == (case["ept"] is not None)
    if case["ept"] is not None:
        assert routing.fused_shape(U * T, N, K)[0] == case["ept"]
    x, d = _fp8_inputs(U, T, N, seed=5, heavy=case.get("heavy", 0.0))
    del x
    nvd = torch.from_numpy(_fused_nv(case, routing.fused_shape(U * T, N, K)[1])).cuda()
    ref = ops.indexer_topk(d["iq"], d["iw"], _fp8_as_bf16(d["k8"], d["sc"]), K, n_vis=nvd)
    got = torch.full_like(ref, -7)
    ops.indexer_topk_fp8(d["iq"], d["iw"], d["k8"], d["sc"], K, n_vis=nvd, out=got)
    assert torch.equal(got, ref)


def test_indexer_topk_fp8_matches_oracle_sets():
    """Decode shape through the fused kernel against the oracle's FP8 scores and top-k: equal
    sets apart from rows within 1e-5 of the K-th score."""
    U, T, N, K = 8, 1, 40000, 512
    assert routing.uses_fused(U, T, N, K)
    x, d = _fp8_inputs(U, T, N, seed=6, heavy=0.01)
    got = ops.indexer_topk_fp8(d["iq"], d["iw"], d["k8"], d["sc"], K).cpu().numpy()
    for u in range(U):
        s = orc.indexer_score_fp8(x["idx_q"][u, 0], x["idx_w"][u, 0], x["idx_k8"][u], x["idx_k_scale"][u])
        ok, nd = tie_band_ok(got[u, 0], orc.topk(s, K), s)
        assert ok, (u, nd)


# -------------------------------------------------------------- attention

def _mqa_case(H, q_dtype, W, N, K, seed, U=2, T=2):
    w = gen.Workload("mqa", 102, U=U, T=T, N=N, H=H, K=K, W=W, q_dtype=q_dtype, heavy_frac=0.01,
                     pos_base=12345)
    return w, gen.make_config(w, seed=seed)


def _oracle_out(w, x, u, t, idx):
    q = x["q"][u, t]
    q64 = bf16_f64(q) if q.dtype == np.uint16 else q.astype(np.float64)
    qr = orc.rope_q(q64, int(x["pos"][u, t]))
    raw = x["raw"][u, t:t + w.W] if w.W else np.zeros((0, 512), np.uint16)
    return orc.sparse_mqa(qr, raw, x["comp"][u], idx, w.scale)


@pytest.mark.parametrize("H,qd,W,K", [(64, "f32", 128, 512), (64, "bf16", 128, 512), (128, "f32", 128, 1024),
                                      (16, "f32", 32, 40), (32, "bf16", 0, 96)])
def test_mqa_matches_oracle_on_given_sets(H, qd, W, K):
    N = 3000
    w, x = _mqa_case(H, qd, W, N, K, seed=3)
    rng = np.random.default_rng(9)
    idx = np.stack([np.stack([np.sort(rng.choice(N, K, replace=False)) for _ in range(w.T)]) for _ in range(w.U)])
    idx = idx.astype(np.int32)
    # holes, a duplicate and out-of-range entries (treated as -1)
    idx[0, 0, 3] = -1
    idx[0, 0, 5] = idx[0, 0, 6]
    idx[1, 1, -1] = N + 5
    idx[1, 0, :K // 2] = -1
    d = upload(x)
    out = torch.full((w.U, w.T, H, 512), float("nan"), device="cuda")
    ops.sparse_mqa(d["q"], d["pos"], d["raw"], d["comp"], torch.from_numpy(idx).cuda(), w.scale, W=W, out=out)
    got = out.cpu().numpy()
    for u in range(w.U):
        for t in range(w.T):
            ix = idx[u, t].copy()
            ix[(ix < 0) | (ix >= N)] = -1
            ref = _oracle_out(w, x, u, t, ix)
            e = normwise_err(got[u, t], ref)
            assert e <= CONTRACT_ERR and e <= DESIGN_ERR, (u, t, e)


DENSE_CASES = [
    # (H, q dtype, W, N, U, T, n_vis): ratio-128 layers (all compressed rows, no indexer) and
    # ratio-0 layers (raw window only), decode and prefill-like shapes
    dict(H=64, qd="f32", W=128, N=2048, U=3, T=1, nv=None),
    dict(H=64, qd="f32", W=128, N=0, U=2, T=1, nv=None),
    dict(H=64, qd="bf16", W=128, N=700, U=1, T=6, nv=[[100, 300, 0, 699, 700, 50]]),
    dict(H=128, qd="f32", W=128, N=1000, U=2, T=1, nv=None),
    dict(H=32, qd="bf16", W=0, N=500, U=2, T=2, nv=[[500, 1], [250, 499]]),
    dict(H=64, qd="f32", W=128, N=8192, U=2, T=1, nv=None),
    dict(H=16, qd="bf16", W=32, N=4000, U=1, T=300, nv="causal"),
]


def _dense_nv(case):
    nv = case["nv"]
    if nv is None:
        return None
    if nv == "causal":
        return (case["N"] // 2 + 7 * np.arange(case["T"])).clip(0, case["N"]).astype(np.int32)[None, :]
    return np.array(nv, dtype=np.int32)


@pytest.mark.parametrize("case", DENSE_CASES, ids=lambda c: f"H{c['H']}{c['qd']}W{c['W']}N{c['N']}U{c['U']}T{c['T']}")
def test_dense_mqa_matches_oracle(case):
    """ds4a_dense_mqa against the oracle's union softmax over raw rows + compressed rows [0, n_vis)."""
    H, W, N, U, T = case["H"], case["W"], case["N"], case["U"], case["T"]
    w, x = _mqa_case(H, case["qd"], W, max(N, 1), 1, seed=4, U=U, T=T)
    nv = _dense_nv(case)
    d = upload(x)
    comp = d["comp"] if N > 0 else None
    out = torch.full((U, T, H, 512), float("nan"), device="cuda")
    ops.dense_mqa(d["q"], d["pos"], d["raw"] if W else None, comp, w.scale, W=W,
                  n_vis=torch.from_numpy(nv).cuda() if nv is not None else None, out=out)
    got = out.cpu().numpy()
    checks = [(u, t) for u in range(U) for t in range(T)]
    if len(checks) > 12:                      # many queries: a spread of them, ends included
        checks = checks[:4] + checks[len(checks) // 2:len(checks) // 2 + 4] + checks[-4:]
    for u, t in checks:
        n = N if nv is None else int(nv[u, t])
        ref = _oracle_out(w, x, u, t, np.arange(n, dtype=np.int32))
        e = normwise_err(got[u, t], ref)
        assert e <= CONTRACT_ERR and e <= DESIGN_ERR, (u, t, e)


def test_dense_equals_sparse_over_all_rows():
    """The dense call is the sparse call with idx = 0..N-1: the same bits."""
    H, W, N, U, T = 64, 128, 1500, 3, 2
    w, x = _mqa_case(H, "f32", W, N, N, seed=6, U=U, T=T)
    d = upload(x)
    idx = torch.arange(N, dtype=torch.int32, device="cuda").expand(U, T, N).contiguous()
    a = ops.sparse_mqa(d["q"], d["pos"], d["raw"], d["comp"], idx, w.scale, W=W)
    b = ops.dense_mqa(d["q"], d["pos"], d["raw"], d["comp"], w.scale, W=W)
    assert torch.equal(a, b)


COMPRESS_CASES = [
    # (U, width, ratio, n_rot, fp8): ratio-4 and ratio-128 KV rows, the indexer's 128-wide
    # keys, no FP8, one-row frontiers, a width that is not a multiple of the workgroup
    dict(U=43, width=512, ratio=4, n_rot=64, fp8=True),
    dict(U=20, width=512, ratio=128, n_rot=64, fp8=True),
    dict(U=21, width=128, ratio=4, n_rot=64, fp8=True),
    dict(U=5, width=128, ratio=4, n_rot=0, fp8=True),
    dict(U=3, width=512, ratio=4, n_rot=64, fp8=False),
    dict(U=4, width=512, ratio=1, n_rot=64, fp8=True),
    dict(U=2, width=1000, ratio=7, n_rot=512, fp8=True),
]


def _compress_inputs(case, seed):
    rng = np.random.default_rng(seed)
    U, r, wd = case["U"], case["ratio"], case["width"]
    kv = rng.standard_normal((U, r, wd)).astype(np.float32)
    sc = (rng.standard_normal((U, r, wd)) * 2.0).astype(np.float32)
    gain = rng.uniform(0.5, 1.5, (U, wd)).astype(np.float32)
    pos = (4 * rng.integers(1, 1 << 18, U)).astype(np.int64)
    return kv, sc, gain, pos


def _near_midpoint(x, a, b, rel=1e-5):
    """x (exact) lies within rel of the midpoint of the two representable values a and b."""
    return abs(x - (a + b) / 2) <= rel * max(abs(x), 1e-30)


@pytest.mark.parametrize("case", COMPRESS_CASES, ids=lambda c: f"U{c['U']}w{c['width']}r{c['ratio']}rot{c['n_rot']}{'fp8' if c['fp8'] else ''}")
def test_compress_rows_matches_oracle(case):
    """Emitted rows against the oracle: identical bf16 rows, except that a value may take the
    neighbouring code where the oracle's exact value lies on a rounding midpoint (fp32 here,
    fp64 there)."""
    kv, sc, gain, pos = _compress_inputs(case, 31)
    U, wd = case["U"], case["width"]
    N = 3
    cache = torch.full((U, N, wd), 7.0, dtype=torch.bfloat16, device="cuda")   # rows 0 and 2 must stay 7
    ops.compress_rows(torch.from_numpy(kv).cuda(), torch.from_numpy(sc).cuda(), torch.from_numpy(gain).cuda(),
                      torch.from_numpy(pos).cuda(), eps=1e-6, n_rot=case["n_rot"], fp8=case["fp8"], out=cache[:, 1, :])
    host = cache.cpu()
    assert torch.all(host[:, 0] == 7.0) and torch.all(host[:, 2] == 7.0)
    got = host[:, 1].view(torch.int16).numpy().view(np.uint16)
    for u in range(U):
        ref, y, s = orc.compress_row(kv[u], sc[u], gain[u], eps=1e-6, n_rot=case["n_rot"], pos=int(pos[u]),
                                     fp8=case["fp8"])
        g_v, r_v = bf16_f64(got[u]), bf16_f64(ref)
        if case["fp8"]:
            amax = np.max(np.abs(y)) / 448.0
            if abs(amax / 2.0 ** round(math.log2(amax)) - 1.0) < 1e-6:
                continue                                  # scale on a power of two: either is right
        diff = np.nonzero(got[u] != ref)[0]
        for j in diff:
            x = y[j] / s if case["fp8"] else y[j]
            a, b = (g_v[j] / s, r_v[j] / s) if case["fp8"] else (g_v[j], r_v[j])
            assert _near_midpoint(x, a, b), (u, j, x, a, b)
        assert len(diff) <= max(2, wd // 100), (u, len(diff))


@pytest.mark.parametrize("order,U,T", [("rising", 1, 1), ("falling", 2, 2), ("rising", 1, 256), ("falling", 1, 256)])
def test_mqa_wide_logit_range(order, U, T):
    """Selected rows scaled so that logits climb (or fall) by tens across the union: the
    softmax reference has to move many times inside one workgroup and across the
    split-union merge.  256 queries take the 64-head kernel (a sample is checked)."""
    N, K, W = 2000, 512, 128
    w, x = _mqa_case(64, "f32", W, N, K, seed=5, U=U, T=T)
    rng = np.random.default_rng(11)
    if T <= 2:
        idx = np.stack([np.stack([rng.choice(N, K, replace=False) for _ in range(T)]) for _ in range(U)]).astype(np.int32)
    else:                                     # one set per unit, so each row is scaled once
        idx = np.ascontiguousarray(np.stack([np.broadcast_to(rng.choice(N, K, replace=False), (T, K)) for _ in range(U)]),
                                   dtype=np.int32)
    comp = bf16_f64(x["comp"]).astype(np.float32)
    for u in range(U):
        for t in range(T if T <= 2 else 1):
            for i, j in enumerate(idx[u, t]):
                f = 1.0 + (i if order == "rising" else K - 1 - i) / 16.0
                comp[u, j] *= np.float32(f)
    x = dict(x)
    x["comp"] = gen.bf16_bits_from_f32(comp.copy())
    d = upload(x)
    out = torch.full((U, T, 64, 512), float("nan"), device="cuda")
    ops.sparse_mqa(d["q"], d["pos"], d["raw"], d["comp"], torch.from_numpy(idx).cuda(), w.scale, W=W, out=out)
    got = out.cpu().numpy()
    # Logits reach ~100 here, so the split query's 16 significant bits leave ~1e-3 absolute
    # logit error: the contract bound applies, the unit-scale design bound does not.  A
    # reference that moved without rescaling O or the sum would be off by O(1).
    checks = [(u, t) for u in range(U) for t in range(T)]
    if len(checks) > 8:
        checks = checks[:3] + checks[len(checks) // 2:len(checks) // 2 + 2] + checks[-3:]
    for u, t in checks:
        ref = _oracle_out(w, x, u, t, idx[u, t])
        e = normwise_err(got[u, t], ref)
        assert e <= CONTRACT_ERR, (u, t, e)


def test_mqa_empty_union_is_zero():
    w, x = _mqa_case(16, "f32", 0, 100, 64, seed=4, U=1, T=1)
    d = upload(x)
    idx = torch.full((1, 1, 64), -1, dtype=torch.int32, device="cuda")
    out = torch.full((1, 1, 16, 512), float("nan"), device="cuda")
    ops.sparse_mqa(d["q"], d["pos"], d["raw"], d["comp"], idx, w.scale, W=0, out=out)
    assert torch.count_nonzero(out).item() == 0


def _poison_outside(raw, comp, cs, rv, n_bad_comp):
    """NaN / infinity in every buffer row outside the union: raw rows at or past raw_vis, the
    first n_bad_comp compressed rows (not yet emitted at a session's start) and their scales."""
    raw = raw.clone()
    for u in range(raw.shape[0]):
        for t in range(rv.shape[1]):
            v = min(max(int(rv[u, t]), 0), 128)
            raw[u, t + v:t + 128] = float("nan") if (u + t) % 2 else float("inf")
    comp = comp.clone()
    if comp.dtype == torch.uint8:
        comp[:, :n_bad_comp] = 0x7F                       # E4M3 NaN code
    else:
        comp[:, :n_bad_comp] = float("nan")
        comp[:, :n_bad_comp, ::3] = float("-inf")
    if cs is not None:
        cs = cs.clone()
        cs[:, :n_bad_comp] = float("nan")
    return raw, comp, cs


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16rows", "e4m3rows"])
@pytest.mark.parametrize("qd", ["f32", "bf16"])
def test_rows_outside_the_union_never_reach_the_output(qd, fp8):
    """A session's start: the raw window holds raw_vis in {0, 1} valid rows and the compressed
    cache no emitted row yet (n_vis = 0 for the dense call, every index -1 for the sparse one),
    while the rest of both buffers holds NaN and infinities.  Outputs are finite: zero for an
    empty union, the oracle's attention over the valid raw row otherwise."""
    N, K = 64, 64
    w, x = _mqa_case(64, qd, 128, N, K, seed=21, U=4, T=1)   # one query per unit: windows do not overlap
    d = upload(x)
    rv_h = np.array([[0], [1], [1], [0]], dtype=np.int32)
    rv = torch.from_numpy(rv_h).cuda()
    codes = sc = None
    comp, cs = d["comp"], None
    if fp8:
        codes, sc, comp, cs = _fp8_comp(w.U, N, seed=22, pow2=False)
    raw_p, comp_p, cs_p = _poison_outside(d["raw"], comp, cs, rv_h, N)
    none = torch.full((w.U, w.T, K), -1, dtype=torch.int32, device="cuda")
    zero = torch.zeros((w.U, w.T), dtype=torch.int32, device="cuda")
    sp = ops.sparse_mqa(d["q"], d["pos"], raw_p, comp_p, none, w.scale, W=w.W, comp_scale=cs_p,
                        raw_vis=rv).cpu().numpy()
    dn = ops.dense_mqa(d["q"], d["pos"], raw_p, comp_p, w.scale, W=w.W, n_vis=zero, comp_scale=cs_p,
                       raw_vis=rv).cpu().numpy()
    assert np.isfinite(sp).all() and np.isfinite(dn).all()
    for u in range(w.U):
        for t in range(w.T):
            if rv_h[u, t] == 0:
                assert not sp[u, t].any() and not dn[u, t].any(), (u, t)
                continue
            ref = _raw_ref(w, x, u, t, 1, np.full(K, -1, np.int32))
            for got in (sp[u, t], dn[u, t]):
                e = normwise_err(got, ref)
                assert e <= DESIGN_ERR, (u, t, e)


# A window that is not yet full: raw_vis[u][t] raw rows take part (clamped to [0, W]); values
# below 0, 0, 1, a tile's width and its neighbours, W - 1, W and above W.
RAW_VIS = [[0, 1, 17, -5], [127, 128, 200, 64]]


def _raw_ref(w, x, u, t, v, ix, codes=None, sc=None):
    v = min(max(v, 0), w.W)
    q = x["q"][u, t]
    q64 = bf16_f64(q) if q.dtype == np.uint16 else q.astype(np.float64)
    qr = orc.rope_q(q64, int(x["pos"][u, t]))
    raw = x["raw"][u, t:t + v]
    if codes is None:
        return orc.sparse_mqa(qr, raw, x["comp"][u], ix, w.scale)
    return orc.sparse_mqa_fp8(qr, raw, codes[u], sc[u], ix, w.scale)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16rows", "e4m3rows"])
@pytest.mark.parametrize("qd", ["f32", "bf16"])
def test_mqa_raw_vis_matches_oracle(qd, fp8):
    """ds4a_sparse_mqa(_fp8) with raw_vis: only the first raw_vis rows of each query's window
    enter the union, against the oracle on those rows."""
    N, K = 3000, 512
    w, x = _mqa_case(64, qd, 128, N, K, seed=13, U=2, T=4)
    d = upload(x)
    idx = _given_sets(w.U, w.T, N, K, 14)
    idx[1, 2, :] = -1                      # raw rows only (every one of the window: 200 clamps to W)
    rv = torch.tensor(RAW_VIS, dtype=torch.int32, device="cuda")
    codes = sc = None
    comp, cs = d["comp"], None
    if fp8:
        codes, sc, comp, cs = _fp8_comp(w.U, N, seed=15, pow2=False)
    got = ops.sparse_mqa(d["q"], d["pos"], d["raw"], comp, torch.from_numpy(idx).cuda(), w.scale, W=w.W,
                         comp_scale=cs, raw_vis=rv).cpu().numpy()
    for u in range(w.U):
        for t in range(w.T):
            ix = idx[u, t].copy()
            ix[(ix < 0) | (ix >= N)] = -1
            ref = _raw_ref(w, x, u, t, RAW_VIS[u][t], ix, codes, sc)
            e = normwise_err(got[u, t], ref)
            assert e <= CONTRACT_ERR and e <= DESIGN_ERR, (u, t, RAW_VIS[u][t], e)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16rows", "e4m3rows"])
def test_dense_mqa_raw_vis_matches_oracle(fp8):
    """ds4a_dense_mqa(_fp8) with raw_vis and n_vis together (a session's first tokens: part of
    the window and few compressed rows)."""
    N = 700
    w, x = _mqa_case(64, "bf16", 128, N, 1, seed=16, U=2, T=4)
    d = upload(x)
    nv = np.array([[0, 5, 700, 0], [699, 1, 350, 700]], dtype=np.int32)
    rv = torch.tensor(RAW_VIS, dtype=torch.int32, device="cuda")
    codes = sc = None
    comp, cs = d["comp"], None
    if fp8:
        codes, sc, comp, cs = _fp8_comp(w.U, N, seed=17, pow2=False)
    out = torch.full((w.U, w.T, 64, 512), float("nan"), device="cuda")
    ops.dense_mqa(d["q"], d["pos"], d["raw"], comp, w.scale, W=w.W, n_vis=torch.from_numpy(nv).cuda(),
                  comp_scale=cs, raw_vis=rv, out=out)
    got = out.cpu().numpy()
    for u in range(w.U):
        for t in range(w.T):
            v = RAW_VIS[u][t]
            ref = _raw_ref(w, x, u, t, v, np.arange(nv[u, t], dtype=np.int32), codes, sc)
            if min(max(v, 0), w.W) == 0 and nv[u, t] == 0:
                assert not got[u, t].any(), (u, t)          # empty union: zeros
                continue
            e = normwise_err(got[u, t], ref)
            assert e <= CONTRACT_ERR and e <= DESIGN_ERR, (u, t, v, e)


def test_raw_vis_full_window_is_null_and_fp8_bits_hold():
    """raw_vis = W everywhere gives the NULL call's bits; with power-of-two row scales the FP8
    entry point still gives the bf16 entry point's bits under a partial raw_vis."""
    N, K = 2000, 512
    w, x = _mqa_case(64, "f32", 128, N, K, seed=18, U=2, T=4)
    d = upload(x)
    idx = torch.from_numpy(_given_sets(w.U, w.T, N, K, 19)).cuda()
    full = torch.full((w.U, w.T), w.W, dtype=torch.int32, device="cuda")
    a = ops.sparse_mqa(d["q"], d["pos"], d["raw"], d["comp"], idx, w.scale, W=w.W)
    b = ops.sparse_mqa(d["q"], d["pos"], d["raw"], d["comp"], idx, w.scale, W=w.W, raw_vis=full)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    codes, sc, c8, s8 = _fp8_comp(w.U, N, seed=20)
    kb = (c8.view(torch.float8_e4m3fn).to(torch.float32) * s8[..., None]).to(torch.bfloat16)
    rv = torch.tensor(RAW_VIS, dtype=torch.int32, device="cuda")
    ref = ops.sparse_mqa(d["q"], d["pos"], d["raw"], kb, idx, w.scale, W=w.W, raw_vis=rv)
    got = ops.sparse_mqa(d["q"], d["pos"], d["raw"], c8, idx, w.scale, W=w.W, comp_scale=s8, raw_vis=rv)
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))


# -------------------------------------------------------------- end to end

def _run_step(w, d, nv=True, fused=False):
    step = ops.Step(w.U, w.T, w.N, H=w.H, K=w.K, W=w.W, fused=fused)
    if step.scores is not None:
        step.scores.fill_(float("nan"))
    step.idx.fill_(-7)
    step.out.fill_(float("nan"))
    step(d, n_vis=d["n_vis"] if nv else None, scale=w.scale, theta=w.theta)
    torch.cuda.synchronize()
    return step


def _oracle_attn_on(w, x, ut, idx_row):
    """The oracle's A3-A6 for one (unit, query) over a given selected set (section 3 of the
    method page: the raw window and the selected compressed rows, one softmax)."""
    u, t = divmod(int(ut), w.T)
    q = x["q"][u, t]
    q64 = bf16_f64(q) if q.dtype == np.uint16 else q.astype(np.float64)
    qr = orc.rope_q(q64, int(x["pos"][u, t]), theta=w.theta, n_rot=w.n_rot)
    return orc.sparse_mqa(qr, x["raw"][u, t:t + w.W], x["comp"][u], np.asarray(idx_row, np.int32), w.scale)


def _host_threads():
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _check_e2e(w, x, step, sel):
    """Every (unit, query) in sel: scores (when the path writes them) within 1e-5 of the
    oracle's, the selected set equal to the oracle's apart from rows inside the tie band, and
    the attention output within the bars.  Where the sets differ inside the band, the output
    is held to the oracle's attention over the GPU's own set (section 3-3: the set that
    reaches the attention is the selected one).  Returns (worst error, units whose set
    differed)."""
    ref = orc.step(w, x, sel=sel, nthreads=_host_threads())
    scores = None if step.scores is None else step.scores.cpu().numpy().reshape(w.U * w.T, w.N)
    idx = step.idx.cpu().numpy().reshape(w.U * w.T, w.K)
    out = step.out.cpu().numpy().reshape(w.U * w.T, w.H, 512)
    assert not np.isnan(out).any() and (idx != -7).all()
    assert scores is None or not np.isnan(scores).any()
    worst, differed = 0.0, 0
    for i, ut in enumerate(sel):
        nv = int(x["n_vis"].reshape(-1)[ut])
        r = ref["scores"][i]
        vis = r[:nv]
        if scores is not None:
            assert np.all(np.isneginf(scores[ut, nv:]))
        if nv and scores is not None:
            den = np.maximum(np.abs(vis), 1e-6 * np.abs(vis).max() + 1e-30)
            rel = np.abs(scores[ut, :nv].astype(np.float64) - vis) / den
            assert rel.max() <= 1e-5, (ut, float(rel.max()))
        ok, ndiff = tie_band_ok(idx[ut], ref["idx"][i], r)
        assert ok, (ut, ndiff)
        if ndiff:
            differed += 1
            ref_out = _oracle_attn_on(w, x, ut, idx[ut])
        else:
            ref_out = ref["out"][i]
        e = normwise_err(out[ut], ref_out)
        assert e <= CONTRACT_ERR and e <= DESIGN_ERR, (ut, ndiff, e)
        worst = max(worst, e)
    return worst, differed


# prefill queries checked end to end: the edges of the raw window and of the visible range,
# plus 64 spread over the chunk
PREFILL_SEL = sorted(set([0, 1, 2, 126, 127, 128, 129, 1023, 1024, 2046, 2047] +
                         np.linspace(0, 2047, 64).round().astype(int).tolist()))


def test_e2e_decode_1layer_n2048():
    w = gen.CONFIGS["decode_1layer_n2048"]
    x = gen.make_config(w)
    step = _run_step(w, upload(x))
    _check_e2e(w, x, step, sel=[0])


def test_e2e_decode_43layers_n16384_all_units():
    w = gen.CONFIGS["decode_43layers_n16384"]
    x = gen.make_config(w)
    d = upload(x)
    step = _run_step(w, d)
    _check_e2e(w, x, step, sel=list(range(w.U)))
    # repeat-run determinism (bitwise)
    s1, i1, o1 = step.scores.clone(), step.idx.clone(), step.out.clone()
    step(d, n_vis=d["n_vis"], scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(step.scores, s1) and torch.equal(step.idx, i1) and torch.equal(step.out, o1)
    # the fused A1 + A2 path gives the same set and so the same output, bit for bit
    fs = _run_step(w, d, fused=True)
    assert torch.equal(fs.idx, i1) and torch.equal(fs.out, o1)


def test_e2e_decode_43layers_n65536_fused_all_units():
    """The bench's main workload through the fused path, every unit against the oracle."""
    w = gen.CONFIGS["decode_43layers_n65536"]
    x = gen.make_config(w)
    step = _run_step(w, upload(x), fused=True)
    _check_e2e(w, x, step, sel=list(range(w.U)))


def test_e2e_prefill_2048q_n8192_sampled():
    w = gen.CONFIGS["prefill_2048q_n8192"]
    x = gen.make_config(w)
    step = _run_step(w, upload(x))
    assert len(PREFILL_SEL) >= 64
    _check_e2e(w, x, step, sel=PREFILL_SEL)


def test_e2e_decode_8sessions_n262144_all_sessions():
    w = gen.CONFIGS["decode_8sessions_n262144"]
    x = gen.make_config(w)
    step = _run_step(w, upload(x), nv=False)
    _check_e2e(w, x, step, sel=list(range(w.U)))


def test_e2e_pro_decode_4sessions_n65536_all_sessions():
    w = gen.CONFIGS["pro_decode_4sessions_n65536"]
    x = gen.make_config(w)
    step = _run_step(w, upload(x), nv=False)
    _check_e2e(w, x, step, sel=list(range(w.U)))


class _GivenStep:
    """A step result assembled by hand: a selected set and the GPU's attention over it."""
    scores = None

    def __init__(self, idx, out):
        self.idx, self.out = idx, out


def test_e2e_check_uses_oracle_on_gpu_set_inside_tie_band():
    """_check_e2e's tie-band branch.  Row B is given the indexer key of the oracle's K-th row,
    so the two tie exactly and the oracle keeps the lower row; a set that keeps B instead is
    valid (inside the band) and its attention output, which differs from the oracle set's,
    must be judged against the oracle's attention over that same set."""
    w = gen.Workload("tie", 105, U=1, T=1, N=3000, K=512)
    x = gen.make_config(w)
    ref0 = orc.step(w, x, nthreads=_host_threads())
    kth = int(ref0["idx"][0][w.K - 1])
    chosen = set(ref0["idx"][0].tolist())
    b = next(j for j in range(kth + 1, w.N) if j not in chosen)
    x["idx_k"][0, b] = x["idx_k"][0, kth]
    ref = orc.step(w, x, nthreads=_host_threads())
    assert set(ref["idx"][0].tolist()) == chosen          # ties go to the lower row
    alt = ref["idx"][0].copy()
    alt[w.K - 1] = b
    d = upload(x)
    alt_d = torch.from_numpy(alt.reshape(1, 1, w.K)).cuda()
    out = ops.sparse_mqa(d["q"], d["pos"], d["raw"], d["comp"], alt_d, w.scale, W=w.W)
    torch.cuda.synchronize()
    assert normwise_err(out.cpu().numpy()[0, 0], ref["out"][0]) > DESIGN_ERR   # the sets' outputs differ
    worst, differed = _check_e2e(w, x, _GivenStep(alt_d, out), sel=[0])
    assert differed == 1 and worst <= DESIGN_ERR


def test_e2e_degenerate_all_scores_equal():
    """idx_q = 0 makes every indexer score 0, so the top-k is rows 0..K-1 (ties to the lower index)."""
    w = gen.Workload("deg", 103, U=2, T=1, N=20000, K=512)
    x = gen.make_config(w)
    x["idx_q"][:] = 0
    step = _run_step(w, upload(x), nv=False)
    idx = step.idx.cpu().numpy()
    assert np.array_equal(idx[:, 0], np.broadcast_to(np.arange(512, dtype=np.int32), (2, 512)))
    _check_e2e(w, x, step, sel=[0, 1])


def test_e2e_ragged_prefill_small():
    """Several queries per unit, ragged visibility (0 .. N), K above some n_vis."""
    w = gen.Workload("rag", 104, U=2, T=5, N=777, K=512, q_dtype="bf16", vis_base=0, pos_base=100)
    x = gen.make_config(w)
    x["n_vis"] = np.array([[0, 1, 300, 512, 777], [777, 600, 513, 2, 40]], dtype=np.int32)
    step = _run_step(w, upload(x))
    _check_e2e(w, x, step, sel=list(range(10)))


# ------------------------------------------------------------ cache upkeep

PUSH_CASES = [
    dict(cap=128, D=512, T=1, n0=[0, 1, 64, 127, 128, 128]),
    dict(cap=128, D=512, T=3, n0=[0, 126, 127, 128]),
    dict(cap=128, D=512, T=128, n0=[0, 5, 128]),
    dict(cap=128, D=512, T=300, n0=[0, 77, 128]),
    dict(cap=4, D=64, T=9, n0=[0, 1, 3, 4, 7, -2]),
    dict(cap=1024, D=512, T=2, n0=[1024, 1023]),
]


@pytest.mark.parametrize("case", PUSH_CASES, ids=lambda c: f"cap{c['cap']}D{c['D']}T{c['T']}")
def test_push_raw_matches_oracle(case):
    """Window rows and counts bit-exact against the oracle's push (f16 rounding: overflow,
    underflow, subnormals, -0); rows past the new count untouched."""
    cap, D, T, n0 = case["cap"], case["D"], case["T"], case["n0"]
    U = len(n0)
    rng = np.random.default_rng(cap + 7 * T + D)
    raw = rng.integers(0, 0x7C00, (U, cap, D), dtype=np.uint16)
    kv = (rng.standard_normal((U, T, D)) * 10.0 ** rng.integers(-9, 6, (U, T, D))).astype(np.float32)
    kv[:, 0, :4] = [70000.0, -1e-8, 6.1e-5, -0.0]
    raw_d = torch.from_numpy(raw.view(np.int16)).cuda().view(torch.float16)
    n_d = torch.tensor(n0, dtype=torch.int32, device="cuda")
    ops.push_raw(torch.from_numpy(kv).cuda(), raw_d, n_d)
    got = raw_d.view(torch.int16).cpu().numpy().view(np.uint16)
    got_n = n_d.cpu().numpy()
    for u in range(U):
        ref, n = orc.push_raw(raw[u], min(max(n0[u], 0), cap), kv[u])
        assert got_n[u] == n, (u, got_n[u], n)
        assert np.array_equal(got[u, :n], ref[:n]), u
        assert np.array_equal(got[u, n:], raw[u, n:]), u


@pytest.mark.parametrize("ratio,width", [(4, 512), (4, 128), (128, 512), (1, 8)])
def test_frontier_push_matches_oracle(ratio, width):
    rng = np.random.default_rng(ratio * width)
    U = 6
    skv = rng.standard_normal((U, ratio, width)).astype(np.float32)
    ssc = rng.standard_normal((U, ratio, width)).astype(np.float32)
    kv = rng.standard_normal((U, width)).astype(np.float32)
    sc = rng.standard_normal((U, width)).astype(np.float32)
    ape = rng.standard_normal((ratio, width)).astype(np.float32)
    pos = np.array([0, ratio - 1, ratio, 12345, 2 ** 40 + 3, 7 * ratio + ratio // 2], dtype=np.int64)
    d_kv, d_sc = torch.from_numpy(skv).cuda(), torch.from_numpy(ssc).cuda()
    ops.frontier_push(torch.from_numpy(kv).cuda(), torch.from_numpy(sc).cuda(), torch.from_numpy(ape).cuda(),
                      torch.from_numpy(pos).cuda(), d_kv, d_sc)
    g_kv, g_sc = d_kv.cpu().numpy(), d_sc.cpu().numpy()
    for u in range(U):
        r_kv, r_sc = orc.frontier_push(skv[u], ssc[u], int(pos[u]), kv[u], sc[u], ape)
        assert np.array_equal(g_kv[u], r_kv) and np.array_equal(g_sc[u].view(np.uint32), r_sc.view(np.uint32)), u


def _codes_agree(got, ref, y, s, g_dec, r_dec):
    """E4M3 codes equal (+-0 alike) except where the exact value lies on a rounding midpoint."""
    same = (got == ref) | (((got & 0x7F) == 0) & ((ref & 0x7F) == 0))
    for j in np.nonzero(~same)[0]:
        assert _near_midpoint(y[j] / s, g_dec[j], r_dec[j]), (j, y[j] / s, g_dec[j], r_dec[j])
    return int((~same).sum())


@pytest.mark.parametrize("fmt", ["bf16", "bf16_fp8rt", "e4m3"])
def test_compress_append_matches_oracle(fmt):
    """Only units whose token closes a group emit; the row lands at n_comp[u] (not written past
    cap, still counted); bf16 rows as compress_rows, E4M3 codes and scales as the oracle's
    stored form."""
    rng = np.random.default_rng({"bf16": 1, "bf16_fp8rt": 2, "e4m3": 3}[fmt])
    ratio, width, cap = 4, 128, 5
    pos = np.array([3, 7, 4, 5, 6, 11, 1003, 1002, 15, 19], dtype=np.int64)
    n0 = np.array([0, 4, 0, 1, 2, 5, 3, 3, 2, 1], dtype=np.int32)
    U = len(pos)
    kv = rng.standard_normal((U, ratio, width)).astype(np.float32)
    sc = (rng.standard_normal((U, ratio, width)) * 2.0).astype(np.float32)
    gain = rng.uniform(0.5, 1.5, (U, width)).astype(np.float32)
    row_pos = (pos // ratio).astype(np.int64)
    n_d = torch.from_numpy(n0.copy()).cuda()
    if fmt == "e4m3":
        comp = torch.full((U, cap, width), 0x55, dtype=torch.uint8, device="cuda")
        scl = torch.full((U, cap), -1.0, dtype=torch.float32, device="cuda")
    else:
        comp = torch.full((U, cap, width), 7.0, dtype=torch.bfloat16, device="cuda")
        scl = None
    ops.compress_append(torch.from_numpy(kv).cuda(), torch.from_numpy(sc).cuda(), torch.from_numpy(gain).cuda(),
                        torch.from_numpy(pos).cuda(), torch.from_numpy(row_pos).cuda(), comp, n_d, comp_scale=scl,
                        fp8=(fmt != "bf16"))
    got_n = n_d.cpu().numpy()
    host = comp.cpu()
    for u in range(U):
        emits = pos[u] % ratio == ratio - 1
        assert got_n[u] == n0[u] + (1 if emits else 0), u
        rows = [r for r in range(cap) if not (emits and r == n0[u])]
        if fmt == "e4m3":
            assert torch.all(host[u, rows] == 0x55) and torch.all(scl[u, rows].cpu() == -1.0), u
        else:
            assert torch.all(host[u, rows] == 7.0), u
        if not emits or n0[u] >= cap:
            continue
        r = int(n0[u])
        if fmt == "e4m3":
            codes, s = orc.compress_row_e4m3(kv[u], sc[u], gain[u], n_rot=64, pos=int(row_pos[u]))
            _, y, _ = orc.compress_row(kv[u], sc[u], gain[u], n_rot=64, pos=int(row_pos[u]), fp8=True)
            amax = np.max(np.abs(y)) / 448.0
            if abs(amax / 2.0 ** round(math.log2(amax)) - 1.0) < 1e-6:
                continue                                  # scale on a power of two: either is right
            assert float(scl[u, r]) == s, u
            got = host[u, r].numpy()
            dec = lambda c: torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
            assert _codes_agree(got, codes, y, s, dec(got), dec(codes)) <= 2, u
        else:
            ref, y, s = orc.compress_row(kv[u], sc[u], gain[u], n_rot=64, pos=int(row_pos[u]), fp8=(fmt != "bf16"))
            got = host[u, r].view(torch.int16).numpy().view(np.uint16)
            diff = np.nonzero(got != ref)[0]
            g_v, r_v = bf16_f64(got), bf16_f64(ref)
            for j in diff:
                x = y[j] / s if fmt != "bf16" else y[j]
                a, b = (g_v[j] / s, r_v[j] / s) if fmt != "bf16" else (g_v[j], r_v[j])
                assert _near_midpoint(x, a, b), (u, j)
            assert len(diff) <= 2, u


def test_decode_loop_cache_upkeep_matches_oracle():
    """Twelve decode tokens through the device-side cache upkeep (frontier push, E4M3 index-key
    append, raw-window push), counters kept on the GPU, against the oracle's loop."""
    rng = np.random.default_rng(44)
    U, ratio, width, cap, D, W = 3, 4, 128, 6, 64, 8
    ape = rng.standard_normal((ratio, width)).astype(np.float32)
    gain = rng.uniform(0.5, 1.5, (U, width)).astype(np.float32)
    pos0 = np.array([0, 4 * 50, 4 * 77], dtype=np.int64)
    d_skv = torch.zeros((U, ratio, width), dtype=torch.float32, device="cuda")
    d_ssc = torch.zeros((U, ratio, width), dtype=torch.float32, device="cuda")
    d_codes = torch.zeros((U, cap, width), dtype=torch.uint8, device="cuda")
    d_scale = torch.zeros((U, cap), dtype=torch.float32, device="cuda")
    d_ncomp = torch.zeros(U, dtype=torch.int32, device="cuda")
    d_raw = torch.zeros((U, W, D), dtype=torch.float16, device="cuda")
    d_nraw = torch.zeros(U, dtype=torch.int32, device="cuda")
    o_skv = np.zeros((U, ratio, width), np.float32)
    o_ssc = np.zeros((U, ratio, width), np.float32)
    o_codes = np.zeros((U, cap, width), np.uint8)
    o_scale = np.zeros((U, cap))
    o_ncomp = [0] * U
    o_raw = np.zeros((U, W, D), np.uint16)
    o_nraw = [0] * U
    for step in range(12):
        pos = pos0 + step
        kv = rng.standard_normal((U, width)).astype(np.float32)
        sc = rng.standard_normal((U, width)).astype(np.float32)
        rkv = rng.standard_normal((U, 1, D)).astype(np.float32)
        d_pos = torch.from_numpy(pos).cuda()
        ops.frontier_push(torch.from_numpy(kv).cuda(), torch.from_numpy(sc).cuda(), torch.from_numpy(ape).cuda(),
                          d_pos, d_skv, d_ssc)
        ops.compress_append(d_skv, d_ssc, torch.from_numpy(gain).cuda(), d_pos, d_pos // ratio, d_codes, d_ncomp,
                            comp_scale=d_scale)
        ops.push_raw(torch.from_numpy(rkv).cuda(), d_raw, d_nraw)
        for u in range(U):
            o_skv[u], o_ssc[u] = orc.frontier_push(o_skv[u], o_ssc[u], int(pos[u]), kv[u], sc[u], ape)
            if pos[u] % ratio == ratio - 1:
                c, s = orc.compress_row_e4m3(o_skv[u], o_ssc[u], gain[u], n_rot=64, pos=int(pos[u] // ratio))
                o_codes[u, o_ncomp[u]], o_scale[u, o_ncomp[u]] = c, s
                o_ncomp[u] += 1
            o_raw[u], o_nraw[u] = orc.push_raw(o_raw[u], o_nraw[u], rkv[u])
    assert d_ncomp.cpu().tolist() == o_ncomp == [3, 3, 3]
    assert d_nraw.cpu().tolist() == o_nraw == [W] * U
    assert np.array_equal(d_skv.cpu().numpy(), o_skv) and np.array_equal(d_ssc.cpu().numpy(), o_ssc)
    assert np.array_equal(d_raw.view(torch.int16).cpu().numpy().view(np.uint16), o_raw)
    assert np.array_equal(d_scale.cpu().numpy()[:, :3], o_scale[:, :3])
    g = d_codes.cpu().numpy()
    mism = ((g != o_codes) & ~(((g & 0x7F) == 0) & ((o_codes & 0x7F) == 0))).sum()
    assert mism <= 3, mism                               # rounding-midpoint codes only


def test_step_raw_vis_passes_through():
    """ops.Step with raw_vis = W everywhere gives the bits of the call without it; a partial
    raw_vis changes the output (the argument reaches the attention call)."""
    w = gen.Workload("stepvis", 110, U=2, T=1, N=3000, H=64, K=512, heavy_frac=0.01)
    x = gen.make_config(w, seed=1)
    d = upload(x)
    step = ops.Step(w.U, w.T, w.N, H=w.H, K=w.K, W=w.W, fused=True)
    a = step(d, scale=w.scale).clone()
    full = torch.full((w.U, w.T), w.W, dtype=torch.int32, device="cuda")
    b = step(d, scale=w.scale, raw_vis=full).clone()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    part = torch.tensor([[5], [w.W]], dtype=torch.int32, device="cuda")
    c = step(d, scale=w.scale, raw_vis=part)
    assert not torch.equal(c[0], a[0]) and torch.equal(c[1].view(torch.int32), a[1].view(torch.int32))


def test_session_start_push_then_attend_with_raw_vis():
    """A prompt's rows pushed into an empty window and into a nearly full one, then a decode
    query over that window with raw_vis = the window's row count (the counter ds4a_push_raw
    keeps, read by the attention call on the device), against the oracle's push and attention."""
    N, K, W, T_new = 1000, 512, 128, 40
    w, x = _mqa_case(64, "f32", W, N, K, seed=21, U=2, T=1)
    d = upload(x)
    rng = np.random.default_rng(22)
    n0 = np.array([0, 100], dtype=np.int32)
    raw0 = x["raw"].copy()                               # [U][W][512] f16 bits, rows past n0 stale
    rkv = (rng.standard_normal((w.U, T_new, 512)) * 0.5).astype(np.float32)
    d_raw = bits_to_torch(raw0, torch.float16)
    d_n = torch.from_numpy(n0.copy()).cuda()
    ops.push_raw(torch.from_numpy(rkv).cuda(), d_raw, d_n)
    idx = _given_sets(w.U, 1, N, K, 23)
    got = ops.sparse_mqa(d["q"], d["pos"], d_raw, d["comp"], torch.from_numpy(idx).cuda(), w.scale, W=W,
                         raw_vis=d_n.view(w.U, 1)).cpu().numpy()
    for u in range(w.U):
        o_raw, o_n = orc.push_raw(raw0[u], int(n0[u]), rkv[u])
        assert o_n == int(d_n[u].item()) == [40, 128][u]
        ix = idx[u, 0].copy()
        ix[(ix < 0) | (ix >= N)] = -1
        q = x["q"][u, 0].astype(np.float64)
        qr = orc.rope_q(q, int(x["pos"][u, 0]))
        ref = orc.sparse_mqa(qr, o_raw[:o_n], x["comp"][u], ix, w.scale)
        e = normwise_err(got[u, 0], ref)
        assert e <= CONTRACT_ERR and e <= DESIGN_ERR, (u, e)


# ------------------------------------------------ FP8-stored compressed rows (attention)

def _fp8_comp(U, N, seed, pow2=True):
    rng = np.random.default_rng(seed)
    codes = gen.e4m3_codes(rng, (U, N, 512))
    if pow2:
        sc = np.ldexp(np.float32(1.0), rng.integers(-8, -5, (U, N))).astype(np.float32)
    else:
        sc = (rng.uniform(0.5, 2.0, (U, N)) * 2.0 ** -7).astype(np.float32)
    c8 = torch.from_numpy(codes).cuda()
    s8 = torch.from_numpy(sc).cuda()
    return codes, sc, c8, s8


def _given_sets(U, T, N, K, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([np.stack([np.sort(rng.choice(N, K, replace=False)) for _ in range(T)]) for _ in range(U)])
    idx = idx.astype(np.int32)
    idx[0, 0, 3] = -1
    idx[0, 0, 5] = idx[0, 0, 6]
    idx[-1, -1, -1] = N + 5
    return idx


@pytest.mark.parametrize("H,qd,W,K", [(64, "f32", 128, 512), (64, "bf16", 128, 512), (128, "f32", 128, 1024),
                                      (32, "bf16", 0, 96), (16, "f32", 32, 40)])
def test_mqa_fp8_rows_bit_identical_to_bf16(H, qd, W, K):
    """E4M3 rows with power-of-two scales give the bf16 entry point's output on rows
    code value * scale, bit for bit (sparse)."""
    N = 3000
    w, x = _mqa_case(H, qd, W, N, K, seed=5)
    d = upload(x)
    codes, sc, c8, s8 = _fp8_comp(w.U, N, seed=H + K)
    kb = (c8.view(torch.float8_e4m3fn).to(torch.float32) * s8[..., None]).to(torch.bfloat16)
    idx = torch.from_numpy(_given_sets(w.U, w.T, N, K, 11)).cuda()
    ref = ops.sparse_mqa(d["q"], d["pos"], d["raw"], kb, idx, w.scale, W=W)
    got = ops.sparse_mqa(d["q"], d["pos"], d["raw"], c8, idx, w.scale, W=W, comp_scale=s8)
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))


@pytest.mark.parametrize("H,qd,W,N,T", [(64, "f32", 128, 2048, 1), (64, "bf16", 0, 500, 2), (32, "f32", 32, 0, 2),
                                        (16, "bf16", 32, 4000, 3)])
def test_dense_mqa_fp8_rows_bit_identical_to_bf16(H, qd, W, N, T):
    w = gen.Workload("dfp8", 108, U=2, T=T, N=max(N, 1), H=H, K=1, W=W, q_dtype=qd, pos_base=777)
    x = gen.make_config(w, seed=6)
    d = upload(x)
    codes, sc, c8, s8 = _fp8_comp(2, N, seed=N + H)
    kb = (c8.view(torch.float8_e4m3fn).to(torch.float32) * s8[..., None]).to(torch.bfloat16)
    nv = torch.tensor([[N] * T, [max(0, N // 2 - 1)] * T], dtype=torch.int32, device="cuda")
    raw = d["raw"] if W > 0 else None
    ref = ops.dense_mqa(d["q"], d["pos"], raw, kb, w.scale, W=W, n_vis=nv)
    got = ops.dense_mqa(d["q"], d["pos"], raw, c8, w.scale, W=W, n_vis=nv, comp_scale=s8)
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))


@pytest.mark.parametrize("H,qd,W,K", [(64, "f32", 128, 512), (128, "bf16", 128, 1024)])
def test_mqa_fp8_rows_match_oracle(H, qd, W, K):
    """Arbitrary positive row scales against the oracle's FP8-row attention."""
    N = 3000
    w, x = _mqa_case(H, qd, W, N, K, seed=7)
    d = upload(x)
    codes, sc, c8, s8 = _fp8_comp(w.U, N, seed=3 * K, pow2=False)
    idx = _given_sets(w.U, w.T, N, K, 12)
    got = ops.sparse_mqa(d["q"], d["pos"], d["raw"], c8, torch.from_numpy(idx).cuda(), w.scale, W=W,
                         comp_scale=s8).cpu().numpy()
    for u in range(w.U):
        for t in range(w.T):
            ix = idx[u, t].copy()
            ix[(ix < 0) | (ix >= N)] = -1
            q = x["q"][u, t]
            q64 = bf16_f64(q) if q.dtype == np.uint16 else q.astype(np.float64)
            qr = orc.rope_q(q64, int(x["pos"][u, t]))
            ref = orc.sparse_mqa_fp8(qr, x["raw"][u, t:t + W], codes[u], sc[u], ix, w.scale)
            e = normwise_err(got[u, t], ref)
            assert e <= CONTRACT_ERR and e <= DESIGN_ERR, (u, t, e)


def test_e2e_fp8_caches_decode():
    """A decode step over FP8 caches end to end (E4M3 indexer keys and compressed rows with
    power-of-two row scales, as ds4a_compress_append stores them): ds4a_indexer_topk_fp8 then
    ds4a_sparse_mqa_fp8 against the oracle's FP8 scores, top-k and FP8-row attention, with
    12,000 of 20,000 rows visible and heavy rows."""
    w = gen.Workload("e2e_fp8", 109, U=6, T=1, N=20000, H=64, K=512, heavy_frac=0.01, vis_base=12000)
    x = gen.make_config(w, seed=8)
    x8 = gen.make_indexer_fp8_config(w, seed=8)
    codes, sc, c8, s8 = _fp8_comp(w.U, w.N, seed=19)
    d = upload(x)
    nv = d["n_vis"]
    idx = ops.indexer_topk_fp8(d["idx_q"], d["idx_w"], torch.from_numpy(x8["idx_k8"]).cuda(),
                               torch.from_numpy(x8["idx_k_scale"]).cuda(), w.K, n_vis=nv)
    out = ops.sparse_mqa(d["q"], d["pos"], d["raw"], c8, idx, w.scale, w.theta, W=w.W, comp_scale=s8)
    idx_h, out_h = idx.cpu().numpy(), out.cpu().numpy()
    compared = 0
    for u in range(w.U):
        v = int(x["n_vis"][u, 0])
        s = orc.indexer_score_fp8(x8["idx_q"][u, 0], x8["idx_w"][u, 0], x8["idx_k8"][u], x8["idx_k_scale"][u], n_vis=v)
        ok, ndiff = tie_band_ok(idx_h[u, 0], orc.topk(s, w.K, n_vis=v), s)
        assert ok, (u, ndiff)
        ix = idx_h[u, 0].copy()
        q = x["q"][u, 0]
        q64 = bf16_f64(q) if q.dtype == np.uint16 else q.astype(np.float64)
        qr = orc.rope_q(q64, int(x["pos"][u, 0]))
        ref = orc.sparse_mqa_fp8(qr, x["raw"][u, 0:w.W], codes[u], sc[u], ix, w.scale)
        e = normwise_err(out_h[u, 0], ref)
        assert e <= CONTRACT_ERR and e <= DESIGN_ERR, (u, e)
        compared += 1
    assert compared == w.U
