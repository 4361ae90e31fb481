"""The workloads use the attention shape constants of tests/golden/shape_constants.txt: the
Flash column as the method page prints it, the Pro column partly printed there (heads,
top-k) and otherwise taken from the Pro-sized decode workload, each value labelled."""
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


def load_pro_sources():
    src = {}
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].split()
        if line:
            src[line[0]] = line[3]
    return src


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


def test_pro_column_provenance_is_labelled():
    """Only the Pro head count and indexer top-k are printed by the page (section 2 of part
    1/8); every other Pro value is labelled as the workload's."""
    src = load_pro_sources()
    assert set(src.values()) <= {"page", "workload"}
    assert {k for k, v in src.items() if v == "page"} == {"n_head", "n_indexer_top_k"}


def test_indexer_only_inputs_equal_full_inputs():
    """make_indexer_config draws the same indexer values as make_config (own streams per tensor)."""
    import numpy as np

    from synth.inputs import Workload, make_config, make_indexer_config
    w = Workload("tiny", 9, U=3, T=2, N=300, heavy_frac=0.05)
    a, b = make_config(w, seed=4), make_indexer_config(w, seed=4)
    for key in ("idx_k", "idx_q", "idx_w"):
        assert np.array_equal(a[key], b[key]), key
