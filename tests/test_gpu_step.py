"""GPU: A1 + A2 + A3-A6 in one call (ds4a_indexer_topk_mqa) against the two calls it stands for.

The one-call path selects the final rows inside the attention kernel in decode shapes (the
last merge level of the chunked top-k) and otherwise launches what the two calls launch; in
every case idx and out must be those of ds4a_indexer_topk followed by ds4a_sparse_mqa, bit for
bit (the two calls are themselves held to the oracle by test_gpu_parity.py).
"""
import pytest
import torch

from sparse_compressed_kv_amd import ops

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ops.lib()


def _inputs(U, T, N, H, W, qdt, seed, ragged):
    g = torch.Generator(device="cuda").manual_seed(seed)
    dev = "cuda"
    x = {
        "idx_q": torch.randn(U, T, 64, 128, generator=g, device=dev).to(torch.bfloat16),
        "idx_w": torch.rand(U, T, 64, generator=g, device=dev),
        "idx_k": torch.randn(U, N, 128, generator=g, device=dev).to(torch.bfloat16),
        "q": torch.randn(U, T, H, 512, generator=g, device=dev).to(qdt),
        "pos": torch.randint(0, 1 << 20, (U, T), generator=g, device=dev, dtype=torch.int64),
        "raw": torch.randn(U, T + W - 1, 512, generator=g, device=dev).to(torch.float16),
        "comp": torch.randn(U, N, 512, generator=g, device=dev).to(torch.bfloat16),
    }
    n_vis = raw_vis = None
    if ragged:
        # visible rows from a few hundred (fewer than K: -1 padding) to all N; raw windows not full
        n_vis = torch.randint(300, N + 1, (U, T), generator=g, device=dev, dtype=torch.int32)
        n_vis[0, 0] = 300
        n_vis[-1, -1] = N
        raw_vis = torch.randint(0, W + 1, (U, T), generator=g, device=dev, dtype=torch.int32)
        raw_vis[0, 0] = 0
    return x, n_vis, raw_vis


CASES = [
    # name, U, T, N, H, K, W, q dtype, ragged.  Routes (tests/routing.py and the attention's
    # plan): the first seven select inside the attention kernel (11, 11, 7, 11 and 22 chunks per
    # query; the K = 768 case after one intermediate merge level of 16,896 candidates; the two
    # split_union cases with the union split over several workgroups per head group, each of
    # which selects the whole set and attends its part), the last two launch the two calls
    # (too few chunk workgroups for the fused select; four queries per unit).
    ("decode_merge", 43, 1, 16384, 64, 512, 128, torch.float32, False),
    ("decode_merge_ragged", 43, 1, 16384, 64, 512, 128, torch.float32, True),
    ("decode_merge_bf16q", 36, 1, 20000, 64, 512, 96, torch.bfloat16, True),
    ("decode_main_shape", 43, 1, 65536, 64, 512, 128, torch.float32, True),
    ("decode_merge_after_a_level", 43, 1, 40000, 64, 768, 128, torch.float32, True),
    ("split_union_merge", 8, 1, 65536, 64, 512, 128, torch.float32, True),
    ("split_union_merge_w64", 12, 1, 30000, 64, 512, 64, torch.bfloat16, True),
    ("pro_split_union", 4, 1, 16384, 128, 1024, 128, torch.float32, True),
    ("many_queries", 2, 4, 8192, 64, 512, 128, torch.bfloat16, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_one_call_equals_two_calls(case):
    name, U, T, N, H, K, W, qdt, ragged = case
    print(f"[one call] {name}", flush=True)
    x, n_vis, raw_vis = _inputs(U, T, N, H, W, qdt, seed=hash(name) % 1000, ragged=ragged)
    scale = 1.0 / 512 ** 0.5
    idx2 = ops.indexer_topk(x["idx_q"], x["idx_w"], x["idx_k"], K, n_vis=n_vis)
    out2 = ops.sparse_mqa(x["q"], x["pos"], x["raw"], x["comp"], idx2, scale, W=W, raw_vis=raw_vis)
    idx1 = torch.full((U, T, K), -7, dtype=torch.int32, device="cuda")
    out1 = torch.full((U, T, H, 512), float("nan"), device="cuda")
    ws = torch.zeros(ops.workspace_bytes(4, U, T, N, K, H, W), dtype=torch.uint8, device="cuda")
    for rep in range(2):                      # the workspace's counters are left zero for the next call
        ops.indexer_topk_mqa(x["idx_q"], x["idx_w"], x["idx_k"], K, x["q"], x["pos"], x["raw"], x["comp"], scale,
                             W=W, n_vis=n_vis, raw_vis=raw_vis, idx=idx1, out=out1, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(idx1, idx2), (name, rep)
        assert torch.equal(out1, out2), (name, rep)


def test_one_call_without_idx():
    """idx may be omitted: the output is the same."""
    U, T, N, H, K, W = 43, 1, 16384, 64, 512, 128
    x, n_vis, raw_vis = _inputs(U, T, N, H, W, torch.float32, seed=11, ragged=True)
    scale = 0.05
    idx2 = ops.indexer_topk(x["idx_q"], x["idx_w"], x["idx_k"], K, n_vis=n_vis)
    out2 = ops.sparse_mqa(x["q"], x["pos"], x["raw"], x["comp"], idx2, scale, W=W, raw_vis=raw_vis)
    out1 = torch.full((U, T, H, 512), float("nan"), device="cuda")
    ws = torch.zeros(ops.workspace_bytes(4, U, T, N, K, H, W), dtype=torch.uint8, device="cuda")
    ops.lib()
    # idx=None through the C ABI
    L = ops.lib()
    rc = L.ds4a_indexer_topk_mqa(U, T, N, 64, 128, K, ops._ptr(x["idx_q"]), ops._ptr(x["idx_w"]),
                                 ops._ptr(x["idx_k"]), ops._ptr(n_vis), H, 512, 64, W, ops._ptr(x["q"]), 0,
                                 ops._ptr(x["pos"]), 10000.0, ops._ptr(x["raw"]), ops._ptr(raw_vis),
                                 ops._ptr(x["comp"]), scale, None, ops._ptr(out1), ops._ptr(ws),
                                 ws.numel(), None)
    assert rc == 0, ops.last_error()
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)


def _e4m3(g, shape):
    c = torch.randint(0, 256, shape, generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E                  # no NaN codes
    return c


FP8_CASES = [
    # name, U, N: the union kept whole (43 queries) and split over several workgroups per head
    # group (8 queries), both with the final merge inside the attention kernel
    ("fp8_whole_union", 43, 16384),
    ("fp8_split_union", 8, 65536),
]


@pytest.mark.parametrize("case", FP8_CASES, ids=[c[0] for c in FP8_CASES])
def test_one_call_fp8_equals_two_calls(case):
    name, U, N = case
    T, H, K, W = 1, 64, 512, 128
    print(f"[one call] {name}", flush=True)
    x, n_vis, raw_vis = _inputs(U, T, N, H, W, torch.float32, seed=21, ragged=True)
    g = torch.Generator(device="cuda").manual_seed(22)
    k8 = _e4m3(g, (U, N, 128))
    ks = torch.pow(2.0, torch.randint(-6, 3, (U, N), generator=g, device="cuda").float())
    c8 = _e4m3(g, (U, N, 512))
    cs = torch.pow(2.0, torch.randint(-8, 1, (U, N), generator=g, device="cuda").float())
    scale = 1.0 / 512 ** 0.5
    idx2 = ops.indexer_topk_fp8(x["idx_q"], x["idx_w"], k8, ks, K, n_vis=n_vis)
    out2 = ops.sparse_mqa(x["q"], x["pos"], x["raw"], c8, idx2, scale, W=W, comp_scale=cs, raw_vis=raw_vis)
    idx1, out1 = ops.indexer_topk_mqa(x["idx_q"], x["idx_w"], k8, K, x["q"], x["pos"], x["raw"], c8, scale, W=W,
                                      n_vis=n_vis, raw_vis=raw_vis, idx_k_scale=ks, comp_scale=cs)
    torch.cuda.synchronize()
    assert torch.equal(idx1, idx2)
    assert torch.equal(out1, out2)
