"""How ds4a_indexer_topk splits a call, restated on the host for the tests.

The library picks, per call, either the score buffer path (indexer scores to the
workspace, then the top-k) or the fused path (each workgroup scores one chunk of a
query's rows in LDS and selects there), and for the fused path a chunk of 512 * ept
rows.  The CPU tests check this restatement against the library's workspace sizes,
and the GPU tests use it to make sure every chunk shape is exercised.
"""
from __future__ import annotations

NT = 512               # threads of a selecting workgroup
CUS = 256              # CUs the chunk rule plans for
SLOTS = 2 * CUS        # chunk workgroups resident at once
MANY_QUERIES = 4       # queries per unit from which the prefill indexer is used
MERGE_MAX = 12288      # candidates one merge workgroup takes
LEVEL_CHUNK = 8192     # candidates per workgroup of an intermediate merge level


def fused_shape(Q: int, N: int, K: int) -> tuple[int, int, int]:
    """(keys per thread, rows per chunk, chunks per query): the busiest CU's makespan model."""
    cmin = max(1, -(-N // 8192))
    cmax = min(N // (4 * K), cmin + 32)
    cmax = max(cmax, cmin)
    best, best_cost = None, None
    for c in range(cmin, cmax + 1):
        rows = (-(-N // c) + 15) // 16 * 16
        ept = (rows + 2047) // 2048 * 4
        wgs = Q * c
        levels, stride = 0, c * K
        while stride > MERGE_MAX:
            stride = -(-stride // LEVEL_CHUNK) * K
            levels += 1
        cost = -(-wgs // CUS) * rows + -(-wgs // SLOTS) * (370 + 24 * ept) + c * K // 16 + 1000 * levels
        if best_cost is None or cost < best_cost:
            best, best_cost = (ept, rows, c), cost
    return best


def uses_fused(U: int, T: int, N: int, K: int) -> bool:
    Q = U * T
    return T < MANY_QUERIES and Q * fused_shape(Q, N, K)[2] >= 128


def _align256(x: int) -> int:
    return (x + 255) & ~255


def fused_workspace_bytes(U: int, T: int, N: int, K: int) -> int:
    """Two (keys, ids) candidate sets of Q x chunks x K words; none for a single chunk."""
    Q = U * T
    chunks = fused_shape(Q, N, K)[2]
    return 4 * _align256(Q * chunks * K * 4) if chunks > 1 else 0
