"""The allocation-free attention (ds4a_sparse_mqa_noalloc) against ds4a_sparse_mqa with a
caller's workspace: the same kernels and the same plan, so the outputs must be bit-identical.
Two calls in a row on split unions (the library's scratch holds counters and records), the
second smaller than the first, then one that needs no split."""
import numpy as np
import pytest
import torch

from sparse_compressed_kv_amd import ops

pytestmark = pytest.mark.gpu


def _case(U, T, H, N, K, W, seed, q_dtype=torch.float32):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(U, T, H, 512, generator=g).to(q_dtype).cuda()
    pos = torch.randint(4 * N, 8 * N, (U, T), generator=g, dtype=torch.int64).cuda()
    raw = torch.randn(U, T + W - 1, 512, generator=g).to(torch.float16).cuda()
    comp = torch.randn(U, N, 512, generator=g).to(torch.bfloat16).cuda()
    idx = torch.stack([torch.randperm(N, generator=g)[:K] for _ in range(U * T)]).view(U, T, K)
    idx = idx.to(torch.int32).sort(-1).values
    idx[0, 0, :3] = -1                        # holes take no part
    return q, pos, raw, comp, idx.cuda()


def _both(U, T, H, N, K, W, seed, q_dtype=torch.float32):
    q, pos, raw, comp, idx = _case(U, T, H, N, K, W, seed, q_dtype)
    scale = 512 ** -0.5
    print(f"noalloc case U={U} T={T} H={H} N={N} K={K} W={W} seed={seed}", flush=True)
    ws_bytes = ops.workspace_bytes(1, U, T, N, K, H, W)
    ref = ops.sparse_mqa(q, pos, raw, comp, idx, scale, W=W,
                         workspace=torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device="cuda"))
    got = ops.sparse_mqa_noalloc(q, pos, raw, comp, idx, scale, W=W)
    torch.cuda.synchronize()
    return ws_bytes, ref, got


def test_noalloc_matches_workspace_entry_two_calls():
    # Pro decode shape: 4 queries x 128 heads, K = 1024 -> split union with records
    ws1, ref1, got1 = _both(4, 1, 128, 4096, 1024, 128, seed=1)
    assert ws1 > 0
    assert torch.equal(got1, ref1)
    # smaller, also split: 2 queries x 64 heads, K = 256
    ws2, ref2, got2 = _both(2, 1, 64, 2000, 256, 128, seed=2)
    assert 0 < ws2 < ws1
    assert torch.equal(got2, ref2)
    assert torch.isfinite(got2).all()


def test_noalloc_without_split_and_bf16_query():
    # 48 queries x 64 heads: no split, the scratch is not touched
    ws, ref, got = _both(48, 1, 64, 3000, 512, 128, seed=3)
    assert ws == 0
    assert torch.equal(got, ref)
    # a bf16 query, split again after the unsplit call
    ws, ref, got = _both(3, 1, 64, 2500, 512, 128, seed=4, q_dtype=torch.bfloat16)
    assert ws > 0
    assert torch.equal(got, ref)
