"""Error budget of the attention's operand precision (CPU, numpy).

The attention multiplies on bf16 / f16 matrix cores with fp32 accumulation.  Stored rows
enter in their own type (compressed rows bf16, raw-window rows f16: exact).  The question is
what the other operands need: the query (f32 in decode; bf16 in prefill, its rotated tail not
bf16 any more) and the probabilities P.  This test emulates the rounding of those operands
against exact fp64 attention (one softmax over raw window and selected rows, section 3 of
the method page) and pins the design:

* rounding query and P plainly to bf16 breaks the 2e-3 normwise contract;
* the split the kernels use (every operand that is not already of the row's type carried as a
  hi + lo pair of it, P included) stays far inside it, below the 1e-4 the GPU parity tests
  hold the kernels to.

Emulation: hi = round(x), lo = round(x - hi) to the row type (RNE); each product pass is an
fp32 matrix product (numpy float32 matmul, i.e. fp32 accumulation) and the hi and lo passes
are summed in fp32, as the kernels sum their two accumulators; softmax in fp32 with the sum
taken over the unrounded fp32 probabilities.  Inputs follow the synthetic recipe: rows
N(0,1) rounded to their stored type, 1 % (decode) heavy rows scaled by 4.
"""
import numpy as np
import pytest
import torch

D, W, K = 512, 128, 512
CONTRACT = 2e-3
KERNEL_BAR = 1e-4


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def _f16(x):
    return np.asarray(x, np.float32).astype(np.float16).astype(np.float32)


def _split(x, rnd):
    hi = rnd(x)
    lo = rnd(np.asarray(x, np.float32) - hi)
    return hi, lo


def _rows(rng, n, heavy):
    raw = _f16(rng.standard_normal((W, D)))
    comp = _bf16(rng.standard_normal((n, D)))
    if heavy:
        hv = rng.choice(n, max(1, round(heavy * n)), replace=False)
        comp[hv] *= np.float32(4.0)
    return raw, comp


def _exact(q, raw, comp, scale):
    rows = np.concatenate([raw, comp]).astype(np.float64)
    lg = scale * (q.astype(np.float64) @ rows.T)
    p = np.exp(lg - lg.max(1, keepdims=True))
    return (p @ rows) / p.sum(1, keepdims=True)


def _emulated(q, raw, comp, scale, q_mode, p_mode, tail_only=False):
    """q_mode / p_mode: 'plain' (one bf16 or f16 pass) or 'split' (hi + lo passes).
    tail_only: the query is bf16 already except its rotated dims 448..511."""
    def qk(rows, rnd):
        if q_mode == "plain":
            return rnd(q) @ rows.T
        hi, lo = _split(q, rnd)
        if tail_only:
            lo[:, :D - 64] = 0.0
        return (hi @ rows.T).astype(np.float32) + (lo @ rows.T).astype(np.float32)

    lg = np.concatenate([qk(raw, _f16), qk(comp, _bf16)], axis=1) * np.float32(scale)
    p = np.exp(lg - lg.max(1, keepdims=True)).astype(np.float32)
    z = p.sum(1, dtype=np.float32)

    def pv(pp, rows, rnd):
        if p_mode == "plain":
            return rnd(pp) @ rows
        hi, lo = _split(pp, rnd)
        return (hi @ rows).astype(np.float32) + (lo @ rows).astype(np.float32)

    o = pv(p[:, :W], raw, _f16) + pv(p[:, W:], comp, _bf16)
    return o / z[:, None]


def _normwise(got, ref):
    return float(np.abs(got - ref).max() / np.abs(ref).max())


def _worst(trials, H, q_kind, heavy, q_mode, p_mode, seed):
    rng = np.random.default_rng(seed)
    scale = 1.0 / np.sqrt(D)
    worst = 0.0
    for _ in range(trials):
        raw, comp = _rows(rng, K, heavy)
        q = rng.standard_normal((H, D)).astype(np.float32)
        tail_only = q_kind == "bf16"
        if tail_only:                          # bf16 query, then its tail rotated (not bf16)
            q = _bf16(q)
            th = rng.uniform(0, 2 * np.pi, 32)
            a, b = q[:, D - 64::2].copy(), q[:, D - 63::2].copy()
            q[:, D - 64::2] = (a * np.cos(th) - b * np.sin(th)).astype(np.float32)
            q[:, D - 63::2] = (a * np.sin(th) + b * np.cos(th)).astype(np.float32)
        ref = _exact(q, raw, comp, scale)
        got = _emulated(q, raw, comp, scale, q_mode, p_mode, tail_only)
        worst = max(worst, _normwise(got, ref))
    return worst


@pytest.mark.parametrize("H,q_kind,heavy", [(64, "f32", 0.01), (64, "bf16", 0.0), (128, "f32", 0.005)],
                         ids=["decode", "prefill", "pro_decode"])
def test_split_operands_stay_inside_the_kernel_bar(H, q_kind, heavy):
    worst = _worst(12, H, q_kind, heavy, "split", "split", seed=H + len(q_kind))
    assert worst <= KERNEL_BAR, worst


@pytest.mark.parametrize("H,q_kind,heavy", [(64, "f32", 0.01), (128, "f32", 0.005)], ids=["decode", "pro_decode"])
def test_plain_bf16_query_and_p_break_the_contract(H, q_kind, heavy):
    """Without the split, query and P rounded to bf16 exceed 2e-3 (so the split is needed)."""
    worst = _worst(12, H, q_kind, heavy, "plain", "plain", seed=7 * H)
    assert worst > CONTRACT, worst


def test_p_split_is_the_larger_share_of_the_margin():
    """With the query split but P plain, the error sits close to the contract: P's split
    is what buys the margin (decode shape)."""
    p_plain = _worst(12, 64, "f32", 0.01, "split", "plain", seed=11)
    both = _worst(12, 64, "f32", 0.01, "split", "split", seed=11)
    assert both * 20 < p_plain, (both, p_plain)
    assert p_plain > 2e-4, p_plain
