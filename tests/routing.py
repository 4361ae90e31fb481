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
ATTN_MERGE_MAX = 6144  # candidates the decode attention kernel merges itself


RATE1 = 23.0           # bytes/ns: one chunk workgroup alone on a CU
RATE2 = 26.0           # two chunk workgroups on one CU, together
RATE_ALL = 6100.0      # the device


def fused_shape(Q: int, N: int, K: int) -> tuple[int, int, int]:
    """(keys per thread, rows per chunk, chunks per query): the modelled time in ns."""
    cmin = max(1, -(-N // 8192))
    cmax = min(N // (2 * K), cmin + 64)
    cmax = max(cmax, cmin)
    best, best_cost = None, None
    for c in range(cmin, cmax + 1):
        rows = (-(-N // c) + 15) // 16 * 16
        ept = (rows + 2047) // 2048 * 4
        wgs = Q * c
        rounds = -(-wgs // SLOTS)
        last = wgs - (rounds - 1) * SLOTS
        chunk_bytes = rows * 256.0
        cu_ns = (rounds - 1) * 2.0 * chunk_bytes / RATE2
        cu_ns += chunk_bytes / RATE1 if last <= CUS else 2.0 * chunk_bytes / RATE2
        all_ns = Q * N * 256.0 / RATE_ALL
        levels, stride = 0, c * K
        while stride > MERGE_MAX:
            stride = -(-stride // LEVEL_CHUNK) * K
            levels += 1
        if stride > ATTN_MERGE_MAX:      # the one-call step would merge once more
            levels += 1
        merge_ns = 3000.0 + 0.6 * stride + 8000.0 * levels if c > 1 else 0.0
        cost = max(cu_ns, all_ns) + rounds * (3000.0 + 150.0 * ept) + merge_ns
        if best_cost is None or cost < best_cost:
            best, best_cost = (ept, rows, c), cost
    return best


def uses_fused(U: int, T: int, N: int, K: int) -> bool:
    """Enough chunk workgroups while chunks keep at least 4 rows per candidate."""
    Q = U * T
    cmin = max(1, -(-N // 8192))
    c4 = max(min(N // (4 * K), cmin + 32), cmin)
    return T < MANY_QUERIES and Q * c4 >= 128


def _align256(x: int) -> int:
    return (x + 255) & ~255


def fused_workspace_bytes(U: int, T: int, N: int, K: int) -> int:
    """Two (keys, ids) candidate sets of Q x chunks x K words; none for a single chunk."""
    Q = U * T
    chunks = fused_shape(Q, N, K)[2]
    return 4 * _align256(Q * chunks * K * 4) if chunks > 1 else 0
