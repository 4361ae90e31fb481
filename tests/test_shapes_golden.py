"""The workloads use the attention shape constants the pages print (tests/golden/shape_constants.txt)."""
import os

from synth.inputs import CONFIGS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "shape_constants.txt")


def load_golden():
    table = {}
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].split()
        if line:
            table[line[0]] = (int(line[1]), int(line[2]))
    return table


def test_workload_shapes_match_printed_constants():
    g = load_golden()
    for key, w in CONFIGS.items():
        col = 1 if w.H == 128 else 0
        assert w.H == g["n_head"][col], key
        assert w.D == g["n_head_dim"][col]
        assert w.n_rot == g["n_rot"][col]
        assert w.W == g["n_swa"][col]
        assert w.Hi == g["n_indexer_head"][col]
        assert w.Di == g["n_indexer_head_dim"][col]
        assert w.K == g["n_indexer_top_k"][col]
    assert g["n_head_kv"] == (1, 1)
