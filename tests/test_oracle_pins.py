"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test ties one oracle function to a library routine, a closed form, an
invariant or brute force on tiny inputs, chosen so that a plausible slip (a
dropped term, a wrong sign or index, a transposed operand, a wrong pairing)
fails at least one of them.  CPU only.
"""
import itertools
import math

import numpy as np
import pytest
import torch

from synth import inputs as gen


def bf16_f64(bits):
    """bf16 bit patterns -> float64 through torch's own bfloat16 type (independent of the oracle)."""
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16).copy())
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def f16_f64(bits):
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def rand_bf16(rng, shape, scale=1.0):
    return gen.bf16_bits_from_f32(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


# ------------------------------------------------------------------ dtypes

def test_f16_decode_all_patterns(oracle_mod):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle_mod.f16_to_f64(bits)
    ref = f16_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_decode_matches_torch(oracle_mod):
    rng = np.random.default_rng(1)
    bits = np.concatenate([rng.integers(0, 65536, 20000).astype(np.uint16),
                           np.array([0, 0x8000, 0x0001, 0x007f, 0x0080, 0x7f7f, 0xff7f, 0x3f80], np.uint16)])
    bits = bits[~np.isnan(bf16_f64(bits))]
    assert np.array_equal(oracle_mod.bf16_to_f64(bits), bf16_f64(bits))


def _f16_probe_values():
    allf = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)
    finite = allf[np.isfinite(allf)]
    pos = np.unique(finite[finite >= 0]).astype(np.float64)
    mids = (pos[:-1] + pos[1:]) / 2.0                       # exact ties (representable in f32)
    mids32 = mids.astype(np.float32)
    assert np.array_equal(mids32.astype(np.float64), mids)
    up = np.nextafter(mids32, np.float32(np.inf))
    dn = np.nextafter(mids32, np.float32(-np.inf))
    extra = np.array([65504.0, 65519.99, 65520.0, 65536.0, 1e6, 3e38, 2.0 ** -25, 2.0 ** -25 * 1.0001,
                      2.0 ** -26, 1e-30, 6.0e-5, 6.1035156e-05], dtype=np.float32)
    rng = np.random.default_rng(7)
    rand = (rng.standard_normal(50000) * np.exp(rng.uniform(-20, 12, 50000))).astype(np.float32)
    v = np.concatenate([finite, mids32, up, dn, extra, rand])
    return np.concatenate([v, -v])


def test_round_f16_matches_numpy_cast(oracle_mod):
    v = _f16_probe_values()
    got = oracle_mod.round_f16(v)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first x={v[bad[0]]!r}: {got[bad[0]]:#06x} vs {ref[bad[0]]:#06x}"


def test_round_f16_specials_and_idempotence(oracle_mod):
    sp = np.array([np.inf, -np.inf, np.nan, 0.0, -0.0], dtype=np.float32)
    got = oracle_mod.round_f16(sp)
    assert got[0] == 0x7C00 and got[1] == 0xFC00 and (got[2] & 0x7C00) == 0x7C00 and (got[2] & 0x3FF)
    assert got[3] == 0 and got[4] == 0x8000
    v = _f16_probe_values()[::7]
    once = oracle_mod.round_f16(v)
    twice = oracle_mod.round_f16(once.view(np.float16).astype(np.float32))
    fin = np.isfinite(once.view(np.float16))
    assert np.array_equal(once[fin], twice[fin])


def test_generator_bf16_rounding_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(1_000_000).astype(np.float32) * np.float32(3.0),
        # exact ties between neighbouring bf16 values, both parities, and their neighbours
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x7FFF).view(np.float32),
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8001).view(np.float32),
        np.array([0.0, -0.0, 1e-40, -1e-40, 3.3e38], dtype=np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gen.bf16_bits_from_f32(x), ref)


# ----------------------------------------------------------------- indexer

def test_indexer_zero_query_gives_zero(oracle_mod):
    rng = np.random.default_rng(11)
    kI = rand_bf16(rng, (37, 128))
    s = oracle_mod.indexer_score(np.zeros((64, 128), np.uint16), rng.random(64, dtype=np.float32), kI)
    assert np.array_equal(s, np.zeros(37))


@pytest.mark.parametrize("h", [0, 17, 63])
def test_indexer_one_hot_weight_is_relu_of_matmul(oracle_mod, h):
    rng = np.random.default_rng(20 + h)
    qI, kI = rand_bf16(rng, (64, 128)), rand_bf16(rng, (53, 128))
    w = np.zeros(64, np.float32)
    w[h] = 1.0
    ref = np.maximum(bf16_f64(kI) @ bf16_f64(qI)[h], 0.0)
    got = oracle_mod.indexer_score(qI, w, kI)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-12)
    assert (ref == 0).any() and (ref > 0).any()          # both ReLU branches exercised


def test_indexer_linear_in_head_weights(oracle_mod):
    rng = np.random.default_rng(31)
    qI, kI = rand_bf16(rng, (64, 128)), rand_bf16(rng, (40, 128))
    w1, w2 = rng.random(64, dtype=np.float32), rng.random(64, dtype=np.float32)
    s1, s2 = oracle_mod.indexer_score(qI, w1, kI), oracle_mod.indexer_score(qI, w2, kI)
    s12 = oracle_mod.indexer_score(qI, (w1.astype(np.float64) + w2).astype(np.float32), kI)
    # w1 + w2 is rounded to f32, so compare against the exactly-rounded weights' combination
    w12 = (w1.astype(np.float64) + w2).astype(np.float32).astype(np.float64)
    per_head = np.stack([oracle_mod.indexer_score(qI, np.eye(64, dtype=np.float32)[h], kI) for h in range(64)])
    np.testing.assert_allclose(s12, w12 @ per_head, rtol=1e-12, atol=1e-10)
    np.testing.assert_allclose(s1 + s2, (w1.astype(np.float64) + w2) @ per_head, rtol=1e-12, atol=1e-10)


def test_indexer_heavy_row_scales_exactly(oracle_mod):
    rng = np.random.default_rng(41)
    qI, kI = rand_bf16(rng, (64, 128)), rand_bf16(rng, (16, 128))
    w = rng.random(64, dtype=np.float32)
    k4 = kI.copy()
    k4[5] = gen.bf16_bits_from_f32(gen.bf16_bits_to_f32(kI[5]) * np.float32(4.0))
    s, s4 = oracle_mod.indexer_score(qI, w, kI), oracle_mod.indexer_score(qI, w, k4)
    assert s4[5] == 4.0 * s[5]
    assert np.array_equal(np.delete(s4, 5), np.delete(s, 5))


def test_indexer_visibility_mask(oracle_mod):
    rng = np.random.default_rng(43)
    qI, kI = rand_bf16(rng, (64, 128)), rand_bf16(rng, (30, 128))
    w = rng.random(64, dtype=np.float32)
    full = oracle_mod.indexer_score(qI, w, kI)
    part = oracle_mod.indexer_score(qI, w, kI, n_vis=11)
    assert np.array_equal(part[:11], full[:11]) and np.all(np.isneginf(part[11:]))


# ------------------------------------------------------------------- top-k

def brute_topk(s, K, n_vis):
    order = sorted(range(n_vis), key=lambda j: (-s[j], j))[:K]
    return order + [-1] * (K - len(order))


def test_topk_brute_force_tiny(oracle_mod):
    rng = np.random.default_rng(51)
    for n in range(0, 65):
        for trial in range(3):
            if trial == 0:
                s = rng.standard_normal(n)
            elif trial == 1:
                s = rng.integers(-2, 3, n).astype(np.float64)     # many ties
            else:
                s = np.full(n, 1.5)                                # all tied
            for K in sorted({1, 2, 7, max(1, n - 1), max(1, n), n + 5}):
                for n_vis in sorted({n, n // 2}):
                    got = oracle_mod.topk(s if n else np.zeros(1), K, n_vis=n_vis)
                    assert got.tolist() == brute_topk(s, K, n_vis), (n, trial, K, n_vis)


def test_topk_nested_and_monotone_invariant(oracle_mod):
    rng = np.random.default_rng(52)
    s = rng.standard_normal(3000)
    prev = oracle_mod.topk(s, 200)
    for K in (201, 350, 512):
        cur = oracle_mod.topk(s, K)
        assert np.array_equal(cur[:prev.size], prev)
        prev = cur
    for f in (lambda x: np.exp(x / 3.0), lambda x: x ** 3, lambda x: 2.0 * x - 7.0):
        assert np.array_equal(oracle_mod.topk(f(s), 512), oracle_mod.topk(s, 512))


def test_topk_k_at_least_visible_returns_all(oracle_mod):
    s = np.random.default_rng(53).standard_normal(100)
    got = oracle_mod.topk(s, 512, n_vis=77)
    assert sorted(got[:77].tolist()) == list(range(77)) and np.all(got[77:] == -1)


def test_selection_invariant_to_permuting_unselected_rows(oracle_mod):
    rng = np.random.default_rng(54)
    qI, kI = rand_bf16(rng, (64, 128)), rand_bf16(rng, (400, 128))
    w = rng.random(64, dtype=np.float32)
    sel = oracle_mod.topk(oracle_mod.indexer_score(qI, w, kI), 64)
    rest = np.setdiff1d(np.arange(400), sel)
    perm = np.arange(400)
    perm[rest] = rng.permutation(rest)
    kp = kI[perm]
    sel_p = oracle_mod.topk(oracle_mod.indexer_score(qI, w, kp), 64)
    assert np.array_equal(np.sort(sel_p), np.sort(sel))          # selected rows did not move
    assert {kp[j].tobytes() for j in sel_p} == {kI[j].tobytes() for j in sel}


# -------------------------------------------------------------------- RoPE

def test_rope_position_zero_is_identity(oracle_mod):
    q = np.random.default_rng(61).standard_normal((64, 512))
    assert np.array_equal(oracle_mod.rope_q(q, 0), q)


@pytest.mark.parametrize("pos", [1, 8191, 262143, 1048575])
def test_rope_matches_complex_rotation_of_tail(oracle_mod, pos):
    rng = np.random.default_rng(62)
    q = rng.standard_normal((8, 512))
    got = oracle_mod.rope_q(q, pos, 10000.0, 64)
    assert np.array_equal(got[:, :448], q[:, :448])
    z = q[:, 448::2] + 1j * q[:, 449::2]
    freq = 10000.0 ** (-np.arange(32) / 32.0)
    zr = z * np.exp(1j * pos * freq)
    # numpy's and libm's pow() may differ by an ulp; the angle error grows with pos
    atol = 1e-13 + 4e-16 * pos * np.abs(z).max()
    np.testing.assert_allclose(got[:, 448::2], zr.real, rtol=0, atol=atol)
    np.testing.assert_allclose(got[:, 449::2], zr.imag, rtol=0, atol=atol)


def test_rope_preserves_pair_norms_and_composes(oracle_mod):
    rng = np.random.default_rng(63)
    q = rng.standard_normal((16, 512))
    a = oracle_mod.rope_q(q, 1234567)
    n0 = np.hypot(q[:, 448::2], q[:, 449::2])
    n1 = np.hypot(a[:, 448::2], a[:, 449::2])
    np.testing.assert_allclose(n1, n0, rtol=1e-14)
    ab = oracle_mod.rope_q(oracle_mod.rope_q(q, 1000), 2345)
    np.testing.assert_allclose(ab, oracle_mod.rope_q(q, 3345), rtol=0, atol=1e-12)


def test_rope_relative_position_property(oracle_mod):
    rng = np.random.default_rng(64)
    x, y = rng.standard_normal((1, 512)), rng.standard_normal((1, 512))
    m, n = 70001, 12345
    lhs = float(oracle_mod.rope_q(x, m)[0, 448:] @ oracle_mod.rope_q(y, n)[0, 448:])
    rhs = float(oracle_mod.rope_q(x, m - n)[0, 448:] @ y[0, 448:])
    assert abs(lhs - rhs) < 1e-10


# --------------------------------------------------------------- attention

def sdpa64(q, rows, scale):
    """Dense softmax attention with key = value = rows, by torch's own routine in float64 on the CPU."""
    qt = torch.from_numpy(q)[None]                 # [1, H, D]
    rt = torch.from_numpy(rows)[None, None].expand(1, q.shape[0], *rows.shape)[0]  # [H, R, D]
    out = torch.nn.functional.scaled_dot_product_attention(qt.transpose(0, 1), rt, rt, scale=scale)
    return out[:, 0, :].numpy()


def _attn_inputs(seed, H=8, D=512, W=128, N=300):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((H, D))
    raw = gen.f16_bits_from_f32(rng.standard_normal((W, D)).astype(np.float32))
    comp = rand_bf16(rng, (N, D))
    return rng, q, raw, comp


def test_attention_all_rows_selected_equals_dense(oracle_mod):
    rng, q, raw, comp = _attn_inputs(71)
    idx = rng.permutation(300).astype(np.int32)
    scale = 1 / math.sqrt(512)
    got = oracle_mod.sparse_mqa(q, raw, comp, idx, scale)
    rows = np.concatenate([f16_f64(raw), bf16_f64(comp)])
    np.testing.assert_allclose(got, sdpa64(q, rows, scale), rtol=1e-11, atol=1e-12)


def test_attention_duplicates_count_twice_and_pads_skip(oracle_mod):
    rng, q, raw, comp = _attn_inputs(72, W=4, N=10)
    idx = np.array([3, -1, 3, 7, -1], np.int32)
    got = oracle_mod.sparse_mqa(q, raw, comp, idx, 0.05)
    rows = np.concatenate([f16_f64(raw), bf16_f64(comp[[3, 3, 7]])])
    np.testing.assert_allclose(got, sdpa64(q, rows, 0.05), rtol=1e-11, atol=1e-12)


def test_attention_zero_query_is_mean_of_union(oracle_mod):
    rng, q, raw, comp = _attn_inputs(73, W=128, N=64)
    idx = rng.choice(64, 40, replace=False).astype(np.int32)
    got = oracle_mod.sparse_mqa(np.zeros_like(q), raw, comp, idx, 0.3)
    mean = np.concatenate([f16_f64(raw), bf16_f64(comp[idx])]).mean(axis=0)
    np.testing.assert_allclose(got, np.broadcast_to(mean, got.shape), rtol=1e-12, atol=1e-14)


def test_attention_single_row_and_empty_union(oracle_mod):
    rng, q, raw, comp = _attn_inputs(74, W=0, N=20)
    got = oracle_mod.sparse_mqa(q, np.zeros((0, 512), np.uint16), comp, np.array([-1, 9, -1], np.int32), 0.04)
    np.testing.assert_array_equal(got, np.broadcast_to(bf16_f64(comp[9]), got.shape))
    empty = oracle_mod.sparse_mqa(q, np.zeros((0, 512), np.uint16), comp, np.array([-1, -1], np.int32), 0.04)
    assert np.array_equal(empty, np.zeros_like(q))


def test_attention_permutation_invariant_and_dominant_row(oracle_mod):
    rng, q, raw, comp = _attn_inputs(75, W=16, N=50)
    idx = rng.choice(50, 30, replace=False).astype(np.int32)
    a = oracle_mod.sparse_mqa(q, raw, comp, idx, 0.04)
    b = oracle_mod.sparse_mqa(q, raw, comp, idx[::-1].copy(), 0.04)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    # A query aligned with one row and a large scale returns (almost) that row.
    target = bf16_f64(comp[idx[4]])
    qd = np.broadcast_to(target, q.shape).copy()
    out = oracle_mod.sparse_mqa(qd, raw, comp, idx, 10.0)
    np.testing.assert_allclose(out, np.broadcast_to(target, q.shape), rtol=0, atol=1e-9)


# --------------------------------------------------------------- whole step

def test_step_composes_the_parts_and_threads_agree(oracle_mod):
    w = gen.Workload("tiny", 90, U=2, T=3, N=700, H=8, K=64, q_dtype="bf16", vis_base=500, pos_base=2000,
                     heavy_frac=0.02)
    x = gen.make_config(w, seed=5)
    r1 = oracle_mod.step(w, x, nthreads=1)
    r4 = oracle_mod.step(w, x, nthreads=4)
    for k in ("scores", "idx", "out"):
        assert np.array_equal(r1[k], r4[k])
    for u, t in itertools.product(range(2), range(3)):
        i = u * 3 + t
        nv = int(x["n_vis"][u, t])
        s = oracle_mod.indexer_score(x["idx_q"][u, t], x["idx_w"][u, t], x["idx_k"][u], n_vis=nv)
        assert np.array_equal(r1["scores"][i], s)
        ix = oracle_mod.topk(s, 64, n_vis=nv)
        assert np.array_equal(r1["idx"][i], ix)
        q = oracle_mod.rope_q(bf16_f64(x["q"][u, t]), x["pos"][u, t])
        o = oracle_mod.sparse_mqa(q, x["raw"][u, t:t + 128], x["comp"][u], ix, w.scale)
        assert np.array_equal(r1["out"][i], o)
    sub = oracle_mod.step(w, x, sel=[5, 1], nthreads=2)
    assert np.array_equal(sub["out"][0], r1["out"][5]) and np.array_equal(sub["idx"][1], r1["idx"][1])


# ------------------------------------------------------------ compressor (section 3-2)

def _e4m3_torch(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8).copy())
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_decode_matches_torch_all_codes(oracle_mod):
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = oracle_mod.e4m3_to_f64(codes), _e4m3_torch(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2          # S.1111.111 only
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7e] == 448.0 and ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9


def test_e4m3_rounding_matches_torch(oracle_mod):
    rng = np.random.default_rng(21)
    finite = _e4m3_torch(np.arange(256, dtype=np.uint8))
    finite = np.unique(finite[np.isfinite(finite)])
    mids = (finite[1:] + finite[:-1]) / 2                                  # every tie
    x = np.concatenate([finite, mids, rng.uniform(-448, 448, 2000), rng.standard_normal(2000) * 1e-2,
                        rng.standard_normal(500) * 1e-3])
    x = x.astype(np.float32).astype(np.float64)                            # torch casts from f32
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = oracle_mod.round_e4m3(x)
    same = (ours == ref) | ((ours & 0x7f) == 0) & ((ref & 0x7f) == 0)       # +-0 alike
    assert same.all(), x[~same][:5]
    assert (oracle_mod.round_e4m3(np.array([448.0, 449.0, 464.0, 1e6, -1e6])) == [0x7e, 0x7e, 0x7e, 0x7e, 0xfe]).all()


def _fp8_keys(rng, n, di=128):
    """Codes over the whole finite range (zeros and subnormals included) and positive scales."""
    k8 = gen.e4m3_codes(rng, (n, di))
    k8[0, :16] = np.arange(16, dtype=np.uint8)                               # zero and subnormals
    k8[1, :8] = np.array([0x80, 0x81, 0x87, 0x88, 0x7E, 0xFE, 0x00, 0x08], np.uint8)
    return k8


def test_indexer_fp8_pow2_scale_equals_bf16_keys(oracle_mod):
    """Power-of-two scales: code value * scale is exact in bf16, so the FP8 score equals the bf16
    indexer score on those keys, made here through torch's own E4M3 and bf16 types."""
    rng = np.random.default_rng(24)
    N = 40
    k8 = _fp8_keys(rng, N)
    scale = np.ldexp(np.float32(1.0), rng.integers(-12, 4, N)).astype(np.float32)
    qI, w = rand_bf16(rng, (64, 128)), rng.random(64, dtype=np.float32)
    kv = torch.from_numpy(k8.copy()).view(torch.float8_e4m3fn).to(torch.float32) * torch.from_numpy(scale)[:, None]
    kb = kv.to(torch.bfloat16)
    assert torch.equal(kb.to(torch.float32), kv)                               # exact
    kI = kb.view(torch.int16).numpy().view(np.uint16)
    got = oracle_mod.indexer_score_fp8(qI, w, k8, scale, n_vis=31)
    ref = oracle_mod.indexer_score(qI, w, kI, n_vis=31)
    assert np.array_equal(got, ref)
    assert np.isneginf(ref[31:]).all() and (ref[:31] > 0).any()


def test_indexer_fp8_one_hot_weight_and_scale_homogeneity(oracle_mod):
    """One head: ReLU of the matmul with the torch-decoded keys times their scales; any positive
    scale factors out of the score (the ReLU is positively homogeneous)."""
    rng = np.random.default_rng(25)
    N = 33
    k8 = _fp8_keys(rng, N)
    scale = rng.uniform(0.01, 3.0, N).astype(np.float32)
    qI = rand_bf16(rng, (64, 128))
    dec = torch.from_numpy(k8.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for h in (0, 40):
        w = np.zeros(64, np.float32)
        w[h] = 1.0
        ref = np.maximum((dec * scale.astype(np.float64)[:, None]) @ bf16_f64(qI)[h], 0.0)
        np.testing.assert_allclose(oracle_mod.indexer_score_fp8(qI, w, k8, scale), ref, rtol=1e-13, atol=1e-13)
        assert (ref == 0).any() and (ref > 0).any()
    w = rng.random(64, dtype=np.float32)
    ones = oracle_mod.indexer_score_fp8(qI, w, k8, np.ones(N, np.float32))
    full = oracle_mod.indexer_score_fp8(qI, w, k8, scale)
    np.testing.assert_allclose(full, ones * scale, rtol=1e-13, atol=0)
    part = oracle_mod.indexer_score_fp8(qI, w, k8, scale, n_vis=5)
    assert np.all(np.isneginf(part[5:])) and np.array_equal(part[:5], full[:5])


def test_round_bf16_matches_torch(oracle_mod):
    rng = np.random.default_rng(22)
    x = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000), [0.0, -0.0, 1.00390625,
                        1.005859375, -3.0e38, 1e-40]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle_mod.round_bf16(x.astype(np.float64)), ref)


def _frontier(rng, ratio, width, spread=1.0):
    kv = rng.standard_normal((ratio, width)).astype(np.float32)
    sc = (rng.standard_normal((ratio, width)) * spread).astype(np.float32)
    return kv, sc


def test_compress_equal_scores_is_mean(oracle_mod):
    """Equal scores: the softmax weights are uniform, so the pooled row is the plain mean."""
    rng = np.random.default_rng(23)
    kv, _ = _frontier(rng, 4, 512)
    sc = np.full_like(kv, 0.37)
    ones = np.ones(512, np.float32)
    _, y, _ = oracle_mod.compress_row(kv, sc, ones, eps=0.0, n_rot=0, fp8=False)
    m = kv.astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(y, m / np.sqrt(np.mean(m * m)), rtol=1e-12, atol=1e-14)


def test_compress_dominant_score_picks_its_row(oracle_mod):
    rng = np.random.default_rng(24)
    kv, sc = _frontier(rng, 128, 128)
    sc[77] += 60.0                                                          # e^-60 for the others
    _, y, _ = oracle_mod.compress_row(kv, sc, np.ones(128, np.float32), eps=0.0, n_rot=0, fp8=False)
    r = kv[77].astype(np.float64)
    np.testing.assert_allclose(y, r / np.sqrt(np.mean(r * r)), rtol=1e-12)


def test_compress_ratio_one_and_permutation(oracle_mod):
    rng = np.random.default_rng(25)
    kv, sc = _frontier(rng, 16, 512, spread=3.0)
    g = rng.uniform(0.5, 2.0, 512).astype(np.float32)
    a = oracle_mod.compress_row(kv, sc, g, n_rot=64, pos=777, fp8=True)
    perm = rng.permutation(16)
    b = oracle_mod.compress_row(kv[perm], sc[perm], g, n_rot=64, pos=777, fp8=True)
    assert np.array_equal(a[0], b[0])                                       # frontier order is irrelevant
    _, y1, _ = oracle_mod.compress_row(kv[:1], sc[:1], np.ones(512, np.float32), eps=0.0, n_rot=0, fp8=False)
    r = kv[0].astype(np.float64)
    np.testing.assert_allclose(y1, r / np.sqrt(np.mean(r * r)), rtol=1e-12)   # one row: itself


def test_compress_rms_gain_and_scale_invariance(oracle_mod):
    rng = np.random.default_rng(26)
    kv, sc = _frontier(rng, 4, 512)
    g = np.full(512, 2.0, np.float32)
    _, y, _ = oracle_mod.compress_row(kv, sc, g, eps=0.0, n_rot=0, fp8=False)
    assert abs(np.mean(y * y) - 4.0) < 1e-12                                # RMS of the output = gain
    _, y2, _ = oracle_mod.compress_row(kv * np.float32(8.0), sc, g, eps=0.0, n_rot=0, fp8=False)
    np.testing.assert_allclose(y2, y, rtol=1e-12)                           # scale of kv divides out
    _, y3, _ = oracle_mod.compress_row(kv, sc, g, eps=1e-2, n_rot=0, fp8=False)
    assert np.mean(y3 * y3) < np.mean(y * y)                                # eps only shrinks


def test_compress_tail_rope_is_complex_rotation(oracle_mod):
    rng = np.random.default_rng(27)
    kv, sc = _frontier(rng, 4, 512)
    g = np.ones(512, np.float32)
    _, y0, _ = oracle_mod.compress_row(kv, sc, g, n_rot=64, pos=0, fp8=False)
    _, yn, _ = oracle_mod.compress_row(kv, sc, g, n_rot=0, pos=0, fp8=False)
    np.testing.assert_array_equal(y0, yn)                                   # position 0: no rotation
    pos = 123457
    _, yp, _ = oracle_mod.compress_row(kv, sc, g, n_rot=64, pos=pos, fp8=False)
    np.testing.assert_array_equal(yp[:448], yn[:448])
    z = yn[448::2] + 1j * yn[449::2]
    ang = pos * 10000.0 ** (-2.0 * np.arange(32) / 64.0)
    zr = z * np.exp(1j * ang)
    np.testing.assert_allclose(yp[448::2], zr.real, atol=1e-12)
    np.testing.assert_allclose(yp[449::2], zr.imag, atol=1e-12)


def test_compress_fp8_round_trip_bounds(oracle_mod):
    """The stored row is E4M3 values times one power of two, within half an E4M3 step of y."""
    rng = np.random.default_rng(28)
    for trial in range(20):
        kv, sc = _frontier(rng, 4 if trial % 2 else 128, 512, spread=2.0)
        g = rng.uniform(0.1, 3.0, 512).astype(np.float32)
        out, y, s = oracle_mod.compress_row(kv, sc, g, n_rot=64, pos=trial * 1000, fp8=True)
        v = bf16_f64(out)
        assert s == 2.0 ** round(math.log2(s))
        assert np.max(np.abs(y)) / s <= 448.0 and np.max(np.abs(y)) / s > 224.0
        q = v / s
        assert np.array_equal(_e4m3_torch(oracle_mod.round_e4m3(q)), q)     # every value is an E4M3 value
        step = np.where(np.abs(y / s) < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(y / s), 1e-300))) - 3))
        assert np.all(np.abs(q - y / s) <= step / 2 + 1e-12)


# ------------------------------------------------------------ cache upkeep

def test_compress_row_e4m3_codes_decode_to_the_emitted_row(oracle_mod):
    """The stored form (codes, scale) decodes, through torch's E4M3 type, to exactly the bf16 row
    the compressor emits with its FP8 round trip."""
    rng = np.random.default_rng(26)
    for width, ratio, n_rot in ((512, 4, 64), (128, 4, 64), (512, 128, 64), (40, 3, 0)):
        kv, sc = _frontier(rng, ratio, width, spread=2.0)
        gain = rng.uniform(0.5, 1.5, width).astype(np.float32)
        out, _, s = oracle_mod.compress_row(kv, sc, gain, n_rot=n_rot, pos=1234, fp8=True)
        codes, s2 = oracle_mod.compress_row_e4m3(kv, sc, gain, n_rot=n_rot, pos=1234)
        assert s2 == s and math.log2(s) == round(math.log2(s))
        assert not np.any((codes & 0x7F) == 0x7F)
        assert np.array_equal(_e4m3_torch(codes) * s, bf16_f64(out))


def _window_model(rows, cap, new_rows):
    """The window as a list of rows: append each new row (f16-rounded by numpy), keep the last cap."""
    out = [r for r in rows]
    for r in new_rows:
        with np.errstate(over="ignore"):                                 # f16 overflow -> inf, as intended
            out.append(np.asarray(r, np.float32).astype(np.float16).view(np.uint16))
        out = out[-cap:]
    return out


@pytest.mark.parametrize("cap,n0,T", [(4, 0, 3), (4, 2, 3), (4, 4, 1), (4, 1, 9), (8, 8, 8), (128, 127, 2),
                                      (128, 0, 128), (128, 128, 300)])
def test_push_raw_matches_window_model(oracle_mod, cap, n0, T):
    rng = np.random.default_rng(cap * 1000 + n0 * 10 + T)
    D = 16
    raw = np.zeros((cap, D), np.uint16)
    raw[:n0] = rng.integers(0, 0x7C00, (n0, D), dtype=np.uint16)       # finite f16 patterns
    raw[n0:] = 0xBEEF                                                   # rows past n_raw: never read
    kv = (rng.standard_normal((T, D)) * 10.0 ** rng.integers(-9, 6, (T, D))).astype(np.float32)
    kv[0, :3] = [70000.0, -1e-8, 6.1e-5]                                # overflow, underflow, subnormal
    got, n = oracle_mod.push_raw(raw, n0, kv)
    ref = _window_model(list(raw[:n0]), cap, kv)
    assert n == len(ref) == min(cap, n0 + T)
    assert np.array_equal(got[:n], np.stack(ref))
    assert np.all(got[n:] == 0xBEEF)
    # T rows at once == one row at a time
    w, m = raw, n0
    for t in range(T):
        w, m = oracle_mod.push_raw(w, m, kv[t:t + 1])
    assert m == n and np.array_equal(w, got)


def test_frontier_push_rows_and_bias(oracle_mod):
    """Tokens at positions p0 .. p0+ratio-1 (p0 a multiple of ratio) fill rows 0 .. ratio-1 in
    order; each push touches only its row; scores carry the bias row of their position (an f32
    add, as numpy does it)."""
    rng = np.random.default_rng(27)
    ratio, width = 4, 24
    ape = rng.standard_normal((ratio, width)).astype(np.float32)
    skv = np.full((ratio, width), 9.0, np.float32)
    ssc = np.full((ratio, width), 9.0, np.float32)
    p0 = 4 * 1001
    toks = [(rng.standard_normal(width).astype(np.float32), rng.standard_normal(width).astype(np.float32))
            for _ in range(ratio)]
    for i, (k, s) in enumerate(toks):
        prev_kv, prev_sc = skv, ssc
        skv, ssc = oracle_mod.frontier_push(skv, ssc, p0 + i, k, s, ape)
        others = [r for r in range(ratio) if r != i]
        assert np.array_equal(skv[others], prev_kv[others]) and np.array_equal(ssc[others], prev_sc[others])
    for i, (k, s) in enumerate(toks):
        assert np.array_equal(skv[i], k)
        assert np.array_equal(ssc[i], s + ape[i])


@pytest.mark.parametrize("mult", [1.0, 1.5, 1.25])
def test_attention_fp8_rows_equal_bf16_rows(oracle_mod, mult):
    """Row scales of 1, 1.5 or 1.25 times a power of two: code value * scale has at most 6
    significant bits, so it is exact in bf16; the FP8-row attention must then equal the bf16
    attention on those rows (made through torch's own E4M3 and bf16 types)."""
    rng = np.random.default_rng(int(mult * 100))
    H, D, W, N, K = 4, 64, 3, 20, 9
    q = rng.standard_normal((H, D)) * 0.2
    raw = gen.f16_bits_from_f32(rng.standard_normal((W, D)).astype(np.float32))
    k8 = gen.e4m3_codes(rng, (N, D))
    scale = (mult * np.ldexp(1.0, rng.integers(-9, -4, N))).astype(np.float32)
    kv = torch.from_numpy(k8.copy()).view(torch.float8_e4m3fn).to(torch.float64) * torch.from_numpy(scale).double()[:, None]
    kb = kv.to(torch.bfloat16)
    assert torch.equal(kb.to(torch.float64), kv)
    comp = kb.view(torch.int16).numpy().view(np.uint16)
    idx = np.array([3, 0, 19, -1, 3, 7, -1, 11, 2], dtype=np.int32)
    got = oracle_mod.sparse_mqa_fp8(q, raw, k8, scale, idx, 0.3)
    ref = oracle_mod.sparse_mqa(q, raw, comp, idx, 0.3)
    assert np.array_equal(got, ref)
    # and the rows' scales matter: doubling one selected row's scale changes the output
    s2 = scale.copy()
    s2[7] *= 2
    assert not np.allclose(oracle_mod.sparse_mqa_fp8(q, raw, k8, s2, idx, 0.3), got)
