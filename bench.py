#!/usr/bin/env python3
"""Benchmark of one layer's compressed sparse attention step on one MI355X.

One step = the whole hot path over one batch: indexer scores + top-k -> RoPE + sparse
multi-query attention, for every unit of the workload, as one ds4a_indexer_topk_mqa call
(the same results as ds4a_indexer_topk followed by ds4a_sparse_mqa, bit for bit; in decode
shapes the last top-k merge level runs inside the attention kernel).  The two calls are
also timed one by one for the per-call figures.

Main line: decode at the DeepSeek V4 Flash shape, 43 independent layers with
N = 65,536 compressed rows each (64 query heads x 512 dims, one KV head,
128-row raw window, indexer 64 x 128, top-k 512).  `value` is decode
tokens/s/layer = layer-units per second.  The main line is also timed with the
step captured as a HIP graph (each replay checked against the eager result),
and per step (p10 / p50 / p90).  Also measured in the same run: the same
decode at N = 16,384 and 32,768 rows, 8 sessions at N = 262,144, the Pro shape
(4 sessions, 128 heads, top-1024, N = 65,536), the attention of a whole Flash
decode step (all 43 layers by their compression ratio, 262,144 tokens of
context), compressor row emission for the 41 layers that compress, and
chunked prefill (2,048 queries, N = 8,192).  The CPU baseline runs the oracle on the main line's
units and also reports how the GPU results agree with it.

Inputs are synthetic (synth.inputs), uploaded to HBM before timing.  Several
replicas of each input set are rotated step by step so that no step finds its
inputs in the 256 MB last-level cache.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--only-main | --prefill-only]
                    [--copy-probe BYTES]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
LLC_BYTES = 256 << 20        # Infinity Cache
METRIC = "sparse-attn decode tokens/s/layer at 64K rows; prefill query-tok/s; % HBM/MFMA peak"
# device code behind ds4a_indexer_topk in decode shapes (the step's dominant call)
SELECT_SOURCES = ["sparse_compressed_kv_amd/csrc/fused.hip", "sparse_compressed_kv_amd/csrc/indexer_core.hpp",
                  "sparse_compressed_kv_amd/csrc/select.hpp", "sparse_compressed_kv_amd/csrc/topk.hip",
                  "sparse_compressed_kv_amd/csrc/common.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "indexer_topk_decode_43layers_n65536_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


KEY_BYTES_BF16 = 128 * 2          # one indexer key row in bf16
KEY_BYTES_FP8 = 128 + 4           # E4M3 codes plus the row's f32 scale


def indexer_bytes_per_unit(N: int, T: int = 1, key_bytes: int = KEY_BYTES_BF16) -> int:
    """Algorithmic HBM bytes of the indexer for one unit: keys read once, the query block and
    head weights read, scores written."""
    return N * key_bytes + T * (64 * 128 * 2 + 64 * 4) + T * N * 4


def select_bytes_per_unit(N: int, K: int, key_bytes: int = KEY_BYTES_BF16) -> int:
    """Algorithmic HBM bytes of the fused A1 + A2 call for one decode unit: keys read once, the
    query block and head weights read, the K selected rows written."""
    return N * key_bytes + 64 * 128 * 2 + 64 * 4 + K * 4


def decode_bytes_per_unit(N: int, H: int, K: int, W: int = 128, key_bytes: int = KEY_BYTES_BF16) -> int:
    """Algorithmic HBM bytes of a whole decode step for one unit (keys, selected rows, raw rows,
    query, output, indexer query and weights)."""
    return N * key_bytes + K * 512 * 2 + W * 512 * 2 + H * 512 * 4 * 2 + 64 * 128 * 2 + 64 * 4


def prefill_flops(w) -> float:
    nv = w.n_vis().astype("float64").sum()
    return 2.0 * 64 * 128 * nv + w.U * w.T * 4.0 * w.H * 512 * (w.K + w.W)


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def upload(x: dict) -> dict:
    """Host arrays from synth.make_config -> device tensors in the library's dtypes."""
    import numpy as np
    import torch

    def bits(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(dt).cuda()

    q = x["q"]
    return {
        "q": bits(q, torch.bfloat16) if q.dtype == np.uint16 else torch.from_numpy(q).cuda(),
        "pos": torch.from_numpy(np.ascontiguousarray(x["pos"], dtype=np.int64)).cuda(),
        "raw": bits(x["raw"], torch.float16), "comp": bits(x["comp"], torch.bfloat16),
        "idx_k": bits(x["idx_k"], torch.bfloat16), "idx_q": bits(x["idx_q"], torch.bfloat16),
        "idx_w": torch.from_numpy(np.ascontiguousarray(x["idx_w"], dtype=np.float32)).cuda(),
        "n_vis": torch.from_numpy(np.ascontiguousarray(x["n_vis"], dtype=np.int32)).cuda(),
    }


class Bench:
    """Device-resident replicas of one workload, and timed steps over them.  A step is one
    ds4a_indexer_topk_mqa call (A1 + A2 + A3-A6), or ds4a_indexer_topk_mqa_fp8 with `fp8_keys`
    (the indexer keys as E4M3 codes and row scales, synth.make_indexer_fp8_config) and
    `fp8_rows`; with FP8 keys and bf16 rows it is ds4a_indexer_topk_fp8 then ds4a_sparse_mqa."""

    def __init__(self, w, x, replicas: int, fp8_keys=None, fp8_rows: bool = False):
        import torch

        from sparse_compressed_kv_amd import ops

        self.torch, self.ops, self.w = torch, ops, w
        self.reps = [upload(x) for _ in range(replicas)]
        self.fp8 = fp8_keys is not None
        self.fp8_rows = fp8_rows
        if self.fp8:
            for d in self.reps:
                d["k8"] = torch.from_numpy(fp8_keys["idx_k8"]).cuda()
                d["sc"] = torch.from_numpy(fp8_keys["idx_k_scale"]).cuda()
        if fp8_rows:
            for i, d in enumerate(self.reps):
                d["comp8"], d["comp_s"] = fp8_rows_on_device(torch, w, seed=100 + i)
                del d["comp"]
        self.step = ops.Step(w.U, w.T, w.N, H=w.H, K=w.K, W=w.W, fused=True)
        self.sep = ops.Step(w.U, w.T, w.N, H=w.H, K=w.K, W=w.W, fused=False)
        self.nvis = w.vis_base is not None
        self.one_call = self.fp8 == fp8_rows
        self.ws_step = torch.zeros(ops.workspace_bytes(4, w.U, w.T, w.N, w.K, w.H, w.W), dtype=torch.uint8,
                                   device="cuda") if self.one_call else None

    def one(self, i: int, stream):
        """Step i on `stream`, over input replica i mod replicas."""
        w, st = self.w, self.step
        d = self.reps[i % len(self.reps)]
        nv = d["n_vis"] if self.nvis else None
        if not self.one_call:
            self.select(d, nv, stream)
            self.attend(d, stream)
        elif self.fp8:
            self.ops.indexer_topk_mqa(d["idx_q"], d["idx_w"], d["k8"], w.K, d["q"], d["pos"], d["raw"], d["comp8"],
                                      w.scale, w.theta, W=w.W, n_vis=nv, idx=st.idx, out=st.out,
                                      workspace=self.ws_step, stream=stream, idx_k_scale=d["sc"],
                                      comp_scale=d["comp_s"])
        else:
            self.ops.indexer_topk_mqa(d["idx_q"], d["idx_w"], d["idx_k"], w.K, d["q"], d["pos"], d["raw"], d["comp"],
                                      w.scale, w.theta, W=w.W, n_vis=nv, idx=st.idx, out=st.out,
                                      workspace=self.ws_step, stream=stream)

    def attend(self, d, stream):
        w, st = self.w, self.step
        if self.fp8_rows:
            self.ops.sparse_mqa(d["q"], d["pos"], d["raw"], d["comp8"], st.idx, w.scale, w.theta, W=w.W,
                                out=st.out, workspace=st.ws_mqa, stream=stream, comp_scale=d["comp_s"])
        else:
            self.ops.sparse_mqa(d["q"], d["pos"], d["raw"], d["comp"], st.idx, w.scale, w.theta, W=w.W,
                                out=st.out, workspace=st.ws_mqa, stream=stream)

    def select(self, d, nv, stream):
        st = self.step
        if self.fp8:
            self.ops.indexer_topk_fp8(d["idx_q"], d["idx_w"], d["k8"], d["sc"], self.w.K, n_vis=nv, out=st.idx,
                                      workspace=st.ws_topk, stream=stream)
        else:
            st.select(d, n_vis=nv, stream=stream)

    def run(self, steps: int, warmup: int):
        torch, ops, w = self.torch, self.ops, self.w
        st, sep = self.step, self.sep
        stream = torch.cuda.current_stream()
        n = len(self.reps)

        def one(i):
            self.one(i, stream)

        for i in range(warmup):
            one(i)
        # Timed region: exactly `steps` steps, events only at its two ends (an event between
        # kernels costs the stream several microseconds).
        t_begin = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t_begin.record(stream)
        for i in range(steps):
            one(warmup + i)
        t_end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        total_ms = t_begin.elapsed_time(t_end)
        # Per-call averages: each call launched `steps` times back to back on the launch stream
        # (inputs rotated as in the step), HIP events at the two ends only.  The separate A1 and
        # A2 calls are timed too, for comparison with the fused call the step uses.
        calls = {
            "select": lambda d, nv: self.select(d, nv, stream),
            "mqa": lambda d, nv: self.attend(d, stream),
            "indexer": (lambda d, nv: ops.indexer_score_fp8(d["idx_q"], d["idx_w"], d["k8"], d["sc"], n_vis=nv,
                                                            out=sep.scores, stream=stream)) if self.fp8 else
                       (lambda d, nv: ops.indexer_score(d["idx_q"], d["idx_w"], d["idx_k"], n_vis=nv,
                                                        out=sep.scores, stream=stream)),
            "topk": lambda d, nv: ops.topk_select(sep.scores, w.K, n_vis=nv, out=sep.idx, workspace=sep.ws_topk,
                                                  stream=stream),
        }
        k_ms = {}
        for name, call in calls.items():
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(steps):
                d = self.reps[(warmup + i) % n]
                call(d, d["n_vis"] if self.nvis else None)
            e1.record(stream)
            torch.cuda.synchronize()
            k_ms[name] = e0.elapsed_time(e1) / steps
        return {"ms_per_step": total_ms / steps, "wall_ms_per_step": 1e3 * wall / steps,
                **{f"{k}_ms": v for k, v in k_ms.items()}}

    def warm(self, steps: int, warmup: int = 5):
        """The same step over input replica 0 only, so that inputs that fit in the Infinity
        Cache stay there between steps (the warm figure; the headline rotates replicas)."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        for _ in range(warmup):
            self.one(0, stream)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            self.one(0, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def percentiles(self, steps: int):
        """Per-step times (an event pair around every step, so this pass is not the headline)."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for i in range(steps):
            self.one(i, stream)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        t = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
        return {"p10_ms": t[steps // 10], "p50_ms": t[steps // 2], "p90_ms": t[(9 * steps) // 10]}

    def graph_run(self, steps: int):
        """The step captured once per input replica as a HIP graph and replayed in rotation.
        Before timing, every graph is replayed twice with eager steps in between, and each
        replay's selection and output are compared with the eager result of its replica."""
        torch = self.torch
        st = self.step
        n = len(self.reps)
        cur = torch.cuda.current_stream()
        ref = []
        for j in range(n):
            self.one(j, cur)
            torch.cuda.synchronize()
            ref.append((st.idx.clone(), st.out.clone()))
        graphs = []
        side = torch.cuda.Stream()
        for j in range(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                self.one(j, torch.cuda.current_stream())
            graphs.append(g)
        torch.cuda.synchronize()
        same = True
        for _ in range(2):
            for j in range(n):
                graphs[j].replay()
                torch.cuda.synchronize()
                same = same and torch.equal(st.idx, ref[j][0]) and torch.equal(st.out, ref[j][1])
                self.one(j + 1, cur)
                torch.cuda.synchronize()
        for i in range(n):
            graphs[i % n].replay()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(cur)
        for i in range(steps):
            graphs[i % n].replay()
        t1.record(cur)
        torch.cuda.synchronize()
        one_ms = t0.elapsed_time(t1) / steps
        del graphs
        # The same with 20 consecutive steps (replicas in rotation) captured as one graph: what a
        # replay costs on top of its kernels is then paid once per 20 steps.
        per = 20
        g20 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g20, stream=side):
            for i in range(per):
                self.one(i, torch.cuda.current_stream())
        torch.cuda.synchronize()
        g20.replay()
        torch.cuda.synchronize()
        j = (per - 1) % n
        same = same and torch.equal(st.idx, ref[j][0]) and torch.equal(st.out, ref[j][1])
        reps = max(1, steps // per)
        torch.cuda.synchronize()
        t0.record(cur)
        for _ in range(reps):
            g20.replay()
        t1.record(cur)
        torch.cuda.synchronize()
        del g20
        return {"ms_per_step": one_ms, "ms_per_step_20_steps_per_graph": t0.elapsed_time(t1) / (reps * per),
                "replays_match_eager": bool(same)}

    def results(self, j: int = 0):
        """Host copies of the selection, the output and the separate call's scores for replica j."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        d = self.reps[j]
        nv = d["n_vis"] if self.nvis else None
        self.one(j, stream)
        self.ops.indexer_score(d["idx_q"], d["idx_w"], d["idx_k"], n_vis=nv, out=self.sep.scores, stream=stream)
        torch.cuda.synchronize()
        return {"idx": self.step.idx.cpu().numpy(), "out": self.step.out.cpu().numpy(),
                "scores": self.sep.scores.cpu().numpy()}


def fp8_rows_on_device(torch, w, seed: int):
    """Compressed rows as stored in FP8 (E4M3 codes [U][N][512] + f32 row scales [U][N]) for the
    timing runs, drawn on the GPU with a seeded torch generator: sign uniform, exponent field
    round(N(11, 1.5)) clipped to 0..15, fraction uniform, the NaN pattern moved to S.1111.110;
    scales 2^e, e uniform in -8..-6 (the recipe of synth.inputs.e4m3_codes)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    shape = (w.U, w.N, 512)
    e = (torch.randn(shape, device="cuda", generator=g) * 1.5 + 11.0).round().clamp(0, 15).to(torch.uint8)
    m = torch.randint(0, 8, shape, device="cuda", generator=g, dtype=torch.uint8)
    sg = torch.randint(0, 2, shape, device="cuda", generator=g, dtype=torch.uint8)
    codes = (sg << 7) | (e << 3) | m
    codes = torch.where((codes & 0x7F) == 0x7F, codes - 1, codes)
    ex = torch.randint(-8, -5, (w.U, w.N), device="cuda", generator=g).to(torch.float32)
    return codes.contiguous(), torch.exp2(ex).contiguous()


def replicas_for(w) -> int:
    per = w.U * (w.N * 128 * 2 + w.K * 512 * 2)          # bytes a step streams from its inputs
    return max(2, math.ceil(2 * LLC_BYTES / max(per, 1)) + 1)


def cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo (empty if it cannot be read)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def cpu_baseline(w, x, gpu=None, budget_s: float = 20.0):
    """The oracle, as it stands, on the host cores: whole decode units of the same workload.
    With `gpu` (host copies of the GPU's selection, output and scores for the same inputs), also
    how the GPU results agree with the oracle's on the units it ran."""
    import numpy as np

    from oracle import oracle

    cores = len(os.sched_getaffinity(0))
    # one unit first (single thread) to size the sample
    t0 = time.perf_counter()
    oracle.step(w, x, sel=[0], nthreads=1)
    per_unit = time.perf_counter() - t0
    n = int(max(1, min(w.U * w.T, cores * max(1, int(budget_s / max(per_unit, 1e-3))))))
    n = min(n, w.U * w.T)
    sel = list(range(n))
    t0 = time.perf_counter()
    ref = oracle.step(w, x, sel=sel, nthreads=min(cores, n))
    el = time.perf_counter() - t0
    rec = {"value": n / el, "unit": "decode tokens/s/layer", "cores": min(cores, n), "kind": "oracle",
           "sample": f"{n} of {w.U} layer-units of {w.name} (full indexer, top-k and attention per unit), "
                     f"1 pass, {el:.1f} s on {min(cores, n)} threads; 1-thread unit time {per_unit:.2f} s",
           "one_thread_units_per_s": 1.0 / per_unit, "cpu_model": cpu_model()}
    if gpu is not None:
        g_idx = gpu["idx"].reshape(w.U * w.T, w.K)[:n]
        g_out = gpu["out"].reshape(w.U * w.T, w.H, 512)[:n]
        g_sc = gpu["scores"].reshape(w.U * w.T, w.N)[:n]
        attn_err, score_err, outside, inside = 0.0, 0.0, 0, 0
        for i in range(n):
            o = ref["out"][i]
            attn_err = max(attn_err, float(np.max(np.abs(g_out[i] - o)) / np.max(np.abs(o))))
            s = ref["scores"][i]
            vis = np.isfinite(s)
            if vis.any():
                score_err = max(score_err, float(np.max(np.abs(g_sc[i][vis] - s[vis])) / np.max(np.abs(s[vis]))))
            r_set = set(int(j) for j in ref["idx"][i] if j >= 0)
            g_set = set(int(j) for j in g_idx[i] if j >= 0)
            kth = min((s[j] for j in r_set), default=0.0)
            for j in r_set ^ g_set:
                if abs(s[j] - kth) <= 1e-5 * abs(kth):
                    inside += 1
                else:
                    outside += 1
        rec["agreement"] = {"units": n, "max_normwise_attention_error": attn_err,
                            "max_score_rel_error": score_err, "topk_diff_rows_inside_tie_band": inside,
                            "topk_diff_rows_outside_tie_band": outside,
                            "bounds": {"attention": 2e-3, "tie_band_rel": 1e-5}}
    return rec


def full_schedule(steps: int, warmup: int):
    """Attention of one whole Flash decode step, all 43 layers, at 262,144 tokens of context,
    with the layer schedule of "Reading the architecture of DwarfStar (ds4.c), part 1/8",
    section 3-2: layers 0-1 keep only the raw window (ds4a_dense_mqa with N = 0), even layers
    from 2 on are ratio 4 (65,536 rows: ds4a_indexer_topk_mqa, top-512) and odd
    layers from 3 on ratio 128 (2,048 rows, all of them: ds4a_dense_mqa)."""
    import torch

    from sparse_compressed_kv_amd import ops
    from synth import inputs as gen

    ctx = 262144
    w4 = gen.Workload("flash_ratio4_layers_ctx262144", 6, U=21, T=1, N=ctx // 4, heavy_frac=0.01, pos_base=ctx - 1)
    w128 = gen.Workload("flash_ratio128_layers_ctx262144", 7, U=20, T=1, N=ctx // 128, pos_base=ctx - 1)
    w0 = gen.Workload("flash_ratio0_layers_ctx262144", 8, U=2, T=1, N=1, pos_base=ctx - 1)
    r4 = [upload(gen.make_config(w4)) for _ in range(replicas_for(w4))]
    x128 = gen.make_config(w128)
    r128 = [upload(x128) for _ in range(2)]
    x0 = gen.make_config(w0)
    r0 = [upload(x0) for _ in range(2)]
    st4 = ops.Step(w4.U, 1, w4.N, one_call=True)
    out128 = torch.empty((w128.U, 1, 64, 512), dtype=torch.float32, device="cuda")
    ws128 = torch.zeros(max(ops.workspace_bytes(3, w128.U, 1, w128.N, 0, 64, 128), 1), dtype=torch.uint8,
                        device="cuda")
    out0 = torch.empty((w0.U, 1, 64, 512), dtype=torch.float32, device="cuda")
    ws0 = torch.zeros(max(ops.workspace_bytes(3, w0.U, 1, 0, 0, 64, 128), 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    scale, theta = w4.scale, w4.theta

    def g4(i):
        st4(r4[i % len(r4)], scale=scale, theta=theta, stream=stream)

    def g128(i):
        d = r128[i % len(r128)]
        ops.dense_mqa(d["q"], d["pos"], d["raw"], d["comp"], scale, theta, W=128, out=out128, workspace=ws128,
                      stream=stream)

    def g0(i):
        d = r0[i % len(r0)]
        ops.dense_mqa(d["q"], d["pos"], d["raw"], None, scale, theta, W=128, out=out0, workspace=ws0, stream=stream)

    def timed(fn, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            fn(warmup + i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def whole(i):
        g0(i)
        g4(i)
        g128(i)

    for i in range(warmup):
        whole(i)
    ms = timed(whole, steps)
    parts = {"ratio0_us": 1e3 * timed(g0, steps), "ratio4_us": 1e3 * timed(g4, steps),
             "ratio128_us": 1e3 * timed(g128, steps)}
    by = (w4.U * decode_bytes_per_unit(w4.N, 64, 512, 128)
          + w128.U * (w128.N * 1024 + 128 * 1024 + 64 * 512 * 4 * 2)
          + w0.U * (128 * 1024 + 64 * 512 * 4 * 2))
    return {"workload": "flash_43layers_ctx262144 (2 raw-only + 21 ratio-4 + 20 ratio-128 layers)",
            "ms_per_step": ms, "value": 1e3 / ms, "unit": "decode tokens/s (all 43 layers' attention)",
            "algorithmic_bytes": by, "frac_hbm": by / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, "parts_back_to_back": parts}


def compressor(steps: int):
    """Compressor row emission for one decode token that closes a block in every layer that
    compresses: 21 ratio-4 layers (a 512-wide KV row and a 128-wide indexer key each) and 20
    ratio-128 layers (a 512-wide KV row), written into caches of 65,536 / 2,048 rows.  The
    frontier inputs are synthetic."""
    import torch

    from sparse_compressed_kv_amd import ops

    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    groups = [("ratio4_kv", 21, 4, 512, 65536), ("ratio4_index_keys", 21, 4, 128, 65536),
              ("ratio128_kv", 20, 128, 512, 2048)]
    calls = []
    by = 0
    for name, U, ratio, width, rows in groups:
        kv = torch.randn(U, ratio, width, device="cuda", generator=g)
        sc = torch.randn(U, ratio, width, device="cuda", generator=g) * 2
        gain = torch.rand(U, width, device="cuda", generator=g) + 0.5
        pos = torch.full((U,), 262143, dtype=torch.int64, device="cuda")
        cache = torch.zeros(U, rows, width, dtype=torch.bfloat16, device="cuda")
        out = cache[:, rows - 1, :]
        calls.append(lambda kv=kv, sc=sc, gain=gain, pos=pos, out=out: ops.compress_rows(
            kv, sc, gain, pos, eps=1e-6, n_rot=64, fp8=True, out=out))
        by += U * (2 * ratio * width * 4 + width * 4 + width * 2 + 8)
    for _ in range(5):
        for c in calls:
            c()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        for c in calls:
            c()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    gus = graph_us(torch, lambda: [c() for c in calls], steps)
    return {"workload": "compressor_emit_41layers (21 x ratio-4 KV + index key, 20 x ratio-128 KV)",
            "us_per_token": us, "graph_us_per_token": gus, "launches": len(calls), "algorithmic_bytes": by,
            "GB_per_s": by / (gus / 1e6) / 1e9}


def graph_us(torch, fn, replays: int, per_graph: int = 20) -> float:
    """Average GPU time of one call of fn: per_graph calls captured back to back as one HIP
    graph, replayed `replays` times (the host's launch overhead and the graph's own launch
    cost are spread over per_graph calls; fn must be safe to repeat)."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        for _ in range(per_graph):
            fn()
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream()
    torch.cuda.synchronize()
    e0.record(cur)
    for _ in range(replays):
        g.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e3 / (replays * per_graph)


def cache_upkeep(steps: int):
    """Cache upkeep after one decode token of a whole Flash model (43 layers), device-side
    counters throughout: the raw-window push of every layer (full 128-row windows, so each
    push slides), the frontier push of the 41 compressing layers' compressors (21 ratio-4 KV,
    21 indexer keys, 20 ratio-128 KV), and their append at a token that closes both a
    ratio-4 and a ratio-128 group (index keys stored as E4M3 codes + scale, KV rows as bf16
    after the FP8 round trip).  Inputs are synthetic."""
    import torch

    from sparse_compressed_kv_amd import ops

    g = torch.Generator(device="cuda")
    g.manual_seed(4321)
    L, cap, D = 43, 128, 512
    raw = (torch.randn(L, cap, D, device="cuda", generator=g)).to(torch.float16)
    n_raw = torch.full((L,), cap, dtype=torch.int32, device="cuda")
    kv_tok = torch.randn(L, 1, D, device="cuda", generator=g)
    pos_val = 262143
    groups = [("ratio4_kv", 21, 4, 512, 65536, False), ("ratio4_index_keys", 21, 4, 128, 65536, True),
              ("ratio128_kv", 20, 128, 512, 2048, False)]
    fronts, appends, poss = [], [], []
    by_front = by_app = 0
    for name, U, ratio, width, rows, e4m3 in groups:
        skv = torch.randn(U, ratio, width, device="cuda", generator=g)
        ssc = torch.randn(U, ratio, width, device="cuda", generator=g) * 2
        gain = torch.rand(U, width, device="cuda", generator=g) + 0.5
        ape = torch.randn(ratio, width, device="cuda", generator=g)
        kv = torch.randn(U, width, device="cuda", generator=g)
        sc = torch.randn(U, width, device="cuda", generator=g)
        pos = torch.full((U,), pos_val, dtype=torch.int64, device="cuda")
        poss.append(pos)
        row_pos = pos // ratio
        if e4m3:
            comp = torch.zeros(U, rows, width, dtype=torch.uint8, device="cuda")
            cs = torch.zeros(U, rows, dtype=torch.float32, device="cuda")
        else:
            comp = torch.zeros(U, rows, width, dtype=torch.bfloat16, device="cuda")
            cs = None
        # every timed call appends one row; the caches have room for all of them
        n_comp = torch.zeros((U,), dtype=torch.int32, device="cuda")
        fronts.append(lambda kv=kv, sc=sc, ape=ape, pos=pos, skv=skv, ssc=ssc: ops.frontier_push(
            kv, sc, ape, pos, skv, ssc))
        appends.append(lambda skv=skv, ssc=ssc, gain=gain, pos=pos, row_pos=row_pos, comp=comp, n=n_comp, cs=cs:
                       ops.compress_append(skv, ssc, gain, pos, row_pos, comp, n, comp_scale=cs))
        by_front += U * (2 * width * 4 + width * 4 + 2 * width * 4)
        by_app += U * (2 * ratio * width * 4 + width * 4 + width * (1 if e4m3 else 2) + 16)

    def push():                                    # the window stays full: every push slides
        ops.push_raw(kv_tok, raw, n_raw)

    def timed(fn, n):
        for _ in range(5):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    def whole():
        push()
        for f in fronts:
            f()
        for a in appends:
            a()

    steps = min(steps, 20)                         # replays of 20 tokens: the appends of the eager and
                                                   # graph passes fit the 2,048-row caches
    by_push = L * ((cap - 1) * D * 2 * 2 + D * 4 + D * 2)
    eager_us = timed(whole, steps)
    # GPU time of each part and of the whole upkeep, as HIP graphs (the eager calls are bound
    # by host launch overhead: seven short kernels)
    push_us = graph_us(torch, push, steps)
    front_us = graph_us(torch, lambda: [f() for f in fronts], steps)
    append_us = graph_us(torch, lambda: [a() for a in appends], steps)
    whole_us = graph_us(torch, whole, steps)
    # a token that closes no group (3 of every 4 tokens): the appends only check and leave
    for p in poss:
        p.fill_(pos_val - 2)
    quiet_us = graph_us(torch, whole, steps)
    return {"workload": "cache_upkeep_43layers (raw push x 43, frontier push + append x 62)",
            "no_emit_us_per_token": quiet_us,
            "us_per_token": whole_us, "timing": "HIP graph of 20 tokens' 7 launches each, replayed back to back",
            "eager_us_per_token": eager_us, "launches": 1 + 2 * len(groups),
            "parts_us": {"push_raw": push_us, "frontier_push": front_us, "append": append_us},
            "push_raw_bytes": by_push, "push_raw_GB_per_s": by_push / (push_us / 1e6) / 1e9,
            "frontier_push_bytes": by_front, "append_bytes": by_app}


def traffic_for(kernel_hash: str, units: int):
    """HBM bytes per ds4a_indexer_topk call from committed rocprofv3 FETCH_SIZE/WRITE_SIZE counters
    (both kernels of the call), scaled by the same counters' reading of a plain copy of known size;
    None if taken on other kernel code."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash or t.get("units") != units:
        return None
    return t.get("hbm_bytes_per_launch")


def attention_record(w, units: int, mqa_ms: float) -> dict:
    """The decode attention (A3-A6) alone: per unit, W + K rows of 1 KiB gathered, the f32 query
    read and the f32 output written (64 heads x 512 dims each)."""
    per_unit = (w.W + w.K) * 1024 + 2 * w.H * 512 * 4
    gbs = units * per_unit / (mqa_ms / 1e3) / 1e9
    return {"kernel": "attn_dq_kernel (ds4a_sparse_mqa: one workgroup per query and 16 heads)",
            "algorithmic_bytes": units * per_unit, "bytes_per_unit": per_unit, "avg_launch_us": mqa_ms * 1e3,
            "GB_per_s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS}


def measured_ceilings(torch, ops) -> dict:
    """HBM read stream over 4 GiB (larger than every cache) and the bf16 MFMA loop, each timed
    with HIP events over repeated launches after warm-up launches."""
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps

    nbytes, grid_r = 4 << 30, 8192
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink_r = torch.empty(grid_r * 256, dtype=torch.int32, device="cuda")
    t_r = timed(lambda: ops.ceiling_read(buf, grid_r, sink=sink_r), 10)
    del buf, sink_r
    iters, grid_m = 2000, 2048
    sink_m = torch.empty(grid_m * 256, dtype=torch.float32, device="cuda")
    flops = ops.ceiling_mfma(iters, grid_m, sink=sink_m)
    t_m = timed(lambda: ops.ceiling_mfma(iters, grid_m, sink=sink_m), 10)
    torch.cuda.empty_cache()
    return {
        "hbm_read": {"GB_per_s": nbytes / t_r / 1e9, "frac_of_spec": nbytes / t_r / 1e9 / HBM_PEAK_GBS,
                     "bytes": nbytes, "grid": grid_r, "us": t_r * 1e6,
                     "kernel": "ceiling_read_kernel (16 B non-temporal loads, grid-stride, 4 in flight)"},
        "mfma_bf16": {"TFLOP_per_s": flops / t_m / 1e12, "frac_of_spec": flops / t_m / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                      "flops": flops, "grid": grid_m, "us": t_m * 1e6,
                      "kernel": "ceiling_mfma_kernel (v_mfma_f32_16x16x32_bf16, 8 chains per wave, 8 waves per SIMD)"},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--only-main", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the prefill workload (for counter runs); prints its record alone")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="after timing, run one device copy of this many bytes (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on one GPU only; the sharded multi-GPU path is a design "
              "(see the sharding section of the design notes), not an implementation.", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    from sparse_compressed_kv_amd import ops
    from synth import inputs as gen

    ops.lib()
    torch.cuda.set_device(0)

    if args.prefill_only:
        w3 = gen.CONFIGS["prefill_2048q_n8192"]
        b3 = Bench(w3, gen.make_config(w3), 2)
        r3 = b3.run(args.steps, args.warmup)
        print(json.dumps({"workload": w3.name, "ms_per_step": r3["ms_per_step"],
                          "kernel_us": {"indexer_topk": r3["select_ms"] * 1e3, "mqa": r3["mqa_ms"] * 1e3}}), flush=True)
        return

    # ---- main line: decode, 43 layers x 65,536 rows
    w = gen.CONFIGS["decode_43layers_n65536"]
    t0 = time.perf_counter()
    x = gen.make_config(w)
    log(f"[bench] generated {w.name} in {time.perf_counter() - t0:.1f}s")
    reps = replicas_for(w)
    b = Bench(w, x, reps)
    r = b.run(args.steps, args.warmup)
    log(f"[bench] {w.name}: {r}")
    pct = b.percentiles(min(args.steps, 100))
    gr = b.graph_run(args.steps)
    warm_ms = b.warm(args.steps)
    log(f"[bench] {w.name}: per step {pct}, graph {gr}, warm {warm_ms:.4f} ms")
    gpu_res = b.results(0) if not args.no_cpu else None
    units = w.U * w.T
    value = units / (r["ms_per_step"] / 1e3)
    sel_bytes = units * select_bytes_per_unit(w.N, w.K)
    achieved = sel_bytes / (r["select_ms"] / 1e3) / 1e9
    khash = source_hash(SELECT_SOURCES)
    idx_bytes = units * indexer_bytes_per_unit(w.N)
    idx_gbs = idx_bytes / (r["indexer_ms"] / 1e3) / 1e9
    step_bytes = units * decode_bytes_per_unit(w.N, w.H, w.K, w.W)
    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "decode tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "units": w.U, "rows_per_unit": w.N, "query_heads": w.H, "head_dim": 512,
                   "top_k": w.K, "raw_window": w.W, "indexer": "64x128", "input_replicas": reps},
        "roofline": {"kernel": "ds4a_indexer_topk (indexer_select_kernel + topk_cand_kernel)", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic_for(khash, units), "algorithmic_bytes": sel_bytes,
                     "avg_launch_us": r["select_ms"] * 1e3, "kernel_hash": khash},
        "indexer_alone": {"kernel": "indexer_score_kernel", "achieved": idx_gbs, "frac": idx_gbs / HBM_PEAK_GBS,
                          "algorithmic_bytes": idx_bytes, "avg_launch_us": r["indexer_ms"] * 1e3},
        "step": {"algorithmic_bytes": step_bytes, "GB_per_s": step_bytes / (r["ms_per_step"] / 1e3) / 1e9,
                 "frac_hbm": step_bytes / (r["ms_per_step"] / 1e3) / 1e9 / HBM_PEAK_GBS,
                 "kernel_us": {"indexer_topk": r["select_ms"] * 1e3, "mqa": r["mqa_ms"] * 1e3,
                               "indexer_alone": r["indexer_ms"] * 1e3, "topk_alone": r["topk_ms"] * 1e3},
                 "wall_ms_per_step": r["wall_ms_per_step"]},
        "attention": attention_record(w, units, r["mqa_ms"]),
        "per_step": pct,
        "warm": {"ms_per_step": warm_ms, "value": units / (warm_ms / 1e3), "input_replicas": 1},
        "hip_graph": {"ms_per_step": gr["ms_per_step"], "value": units / (gr["ms_per_step"] / 1e3),
                      "ms_per_step_20_steps_per_graph": gr["ms_per_step_20_steps_per_graph"],
                      "replays_match_eager": gr["replays_match_eager"]},
    }
    del b
    torch.cuda.empty_cache()

    if not args.only_main:
        # ---- decode at 16,384 and 32,768 rows (43 layers), long context (8 sessions x 262,144
        # rows) and the Pro shape (128 heads, top-1024)
        for key, name in (("decode_43layers_n16384", "decode_n16384"), ("decode_43layers_n32768", "decode_n32768"),
                          ("decode_8sessions_n262144", "decode_8sessions_n262144"),
                          ("pro_decode_4sessions_n65536", "pro_decode_4sessions_n65536")):
            w4 = gen.CONFIGS[key]
            x4 = gen.make_config(w4)
            b4 = Bench(w4, x4, replicas_for(w4))
            r4 = b4.run(args.steps, args.warmup)
            r4["warm_ms"] = b4.warm(args.steps)
            log(f"[bench] {w4.name}: {r4}")
            by4 = w4.U * decode_bytes_per_unit(w4.N, w4.H, w4.K, w4.W)
            rec[name] = {
                "workload": w4.name, "value": w4.U / (r4["ms_per_step"] / 1e3), "unit": "decode tokens/s/layer",
                "ms_per_step": r4["ms_per_step"], "frac_hbm": by4 / (r4["ms_per_step"] / 1e3) / 1e9 / HBM_PEAK_GBS,
                "warm_ms_per_step": r4["warm_ms"],
                "indexer_topk_frac_hbm": w4.U * select_bytes_per_unit(w4.N, w4.K) / (r4["select_ms"] / 1e3) / 1e9
                / HBM_PEAK_GBS,
                "kernel_us": {"indexer_topk": r4["select_ms"] * 1e3, "mqa": r4["mqa_ms"] * 1e3,
                              "indexer_alone": r4["indexer_ms"] * 1e3, "topk_alone": r4["topk_ms"] * 1e3},
            }
            del b4, x4
            torch.cuda.empty_cache()
        # ---- the main workload with FP8-stored indexer keys (E4M3 codes + one scale per row)
        x8 = gen.make_indexer_fp8_config(w)
        b8 = Bench(w, x, reps, fp8_keys=x8)
        del x8
        r8 = b8.run(args.steps, args.warmup)
        log(f"[bench] {w.name} fp8 keys: {r8}")
        sel8 = units * select_bytes_per_unit(w.N, w.K, KEY_BYTES_FP8)
        by8 = units * decode_bytes_per_unit(w.N, w.H, w.K, w.W, KEY_BYTES_FP8)
        rec["decode_n65536_fp8_keys"] = {
            "workload": w.name + "_fp8keys", "value": units / (r8["ms_per_step"] / 1e3),
            "unit": "decode tokens/s/layer", "ms_per_step": r8["ms_per_step"],
            "frac_hbm": by8 / (r8["ms_per_step"] / 1e3) / 1e9 / HBM_PEAK_GBS,
            "indexer_topk_frac_hbm": sel8 / (r8["select_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS,
            "indexer_alone_frac_hbm": units * indexer_bytes_per_unit(w.N, 1, KEY_BYTES_FP8) / (r8["indexer_ms"] / 1e3)
            / 1e9 / HBM_PEAK_GBS,
            "kernel_us": {"indexer_topk": r8["select_ms"] * 1e3, "mqa": r8["mqa_ms"] * 1e3,
                          "indexer_alone": r8["indexer_ms"] * 1e3, "topk_alone": r8["topk_ms"] * 1e3},
        }
        del b8
        torch.cuda.empty_cache()
        # ---- the same with the compressed rows the attention reads stored in FP8 too
        x8 = gen.make_indexer_fp8_config(w)
        b9 = Bench(w, x, reps, fp8_keys=x8, fp8_rows=True)
        del x8
        r9 = b9.run(args.steps, args.warmup)
        log(f"[bench] {w.name} fp8 keys + fp8 rows: {r9}")
        by9 = units * (decode_bytes_per_unit(w.N, w.H, w.K, w.W, KEY_BYTES_FP8) - w.K * 512 * 2 + w.K * (512 + 4))
        rec["decode_n65536_fp8_keys_rows"] = {
            "workload": w.name + "_fp8keys_fp8rows", "value": units / (r9["ms_per_step"] / 1e3),
            "unit": "decode tokens/s/layer", "ms_per_step": r9["ms_per_step"],
            "frac_hbm": by9 / (r9["ms_per_step"] / 1e3) / 1e9 / HBM_PEAK_GBS,
            "kernel_us": {"indexer_topk": r9["select_ms"] * 1e3, "mqa": r9["mqa_ms"] * 1e3},
        }
        del b9
        torch.cuda.empty_cache()
        # ---- a whole Flash decode step: the 43 layers' attention by their compression ratio
        fs = full_schedule(args.steps, args.warmup)
        log(f"[bench] {fs['workload']}: {fs}")
        rec["full_schedule_ctx262144"] = fs
        torch.cuda.empty_cache()
        # ---- compressor row emission for the layers that compress
        cm = compressor(args.steps)
        log(f"[bench] {cm['workload']}: {cm}")
        rec["compressor_emit"] = cm
        # ---- cache upkeep after a token: raw-window push, frontier push, compressed-row append
        cu = cache_upkeep(args.steps)
        log(f"[bench] {cu['workload']}: {cu}")
        rec["cache_upkeep"] = cu
        # ---- chunked prefill: 2,048 queries, 8,192 rows
        w3 = gen.CONFIGS["prefill_2048q_n8192"]
        x3 = gen.make_config(w3)
        b3 = Bench(w3, x3, 2)
        # A prefill step is ~0.5 ms: half the main line's step count, and more warm-up steps than
        # the decode lines (the first steps over freshly allocated 128 MB query and 256 MB
        # output tensors run slower: their pages are first touched there).
        steps3 = max(5, args.steps // 2)
        warm3 = max(2, args.warmup // 2)
        r3 = b3.run(steps3, warm3)
        log(f"[bench] {w3.name}: {r3}")
        fl = prefill_flops(w3)
        tf = fl / (r3["ms_per_step"] / 1e3) / 1e12
        rec["prefill"] = {
            "workload": w3.name, "value": w3.T / (r3["ms_per_step"] / 1e3), "unit": "query-tok/s",
            "steps": steps3, "ms_per_step": r3["ms_per_step"], "algorithmic_flops": fl,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf / MFMA_BF16_PEAK_TFLOPS},
            "kernel_us": {"indexer_topk": r3["select_ms"] * 1e3, "mqa": r3["mqa_ms"] * 1e3,
                          "indexer_alone": r3["indexer_ms"] * 1e3, "topk_alone": r3["topk_ms"] * 1e3},
        }
        del b3
        # ---- the same prefill over E4M3 indexer keys and E4M3 attention rows (half the gathered
        # bytes); flops as above
        b38 = Bench(w3, x3, 2, fp8_keys=gen.make_indexer_fp8_config(w3), fp8_rows=True)
        r38 = b38.run(steps3, warm3)
        log(f"[bench] {w3.name} fp8 keys + fp8 rows: {r38}")
        tf8 = fl / (r38["ms_per_step"] / 1e3) / 1e12
        rec["prefill_fp8_keys_rows"] = {
            "workload": w3.name + "_fp8keys_fp8rows", "value": w3.T / (r38["ms_per_step"] / 1e3),
            "unit": "query-tok/s", "steps": steps3, "ms_per_step": r38["ms_per_step"],
            "frac_mfma": tf8 / MFMA_BF16_PEAK_TFLOPS,
            "kernel_us": {"indexer_topk": r38["select_ms"] * 1e3, "mqa": r38["mqa_ms"] * 1e3},
        }
        del b38, x3

    # ---- measured ceilings (outside every timed region above): a plain HBM read stream and a
    # plain bf16 matrix-core loop, each kernel's fraction is also given against these
    rec["ceilings"] = measured_ceilings(torch, ops)
    hbm_c = rec["ceilings"]["hbm_read"]["GB_per_s"]
    mfma_c = rec["ceilings"]["mfma_bf16"]["TFLOP_per_s"]
    rec["roofline"]["ceiling"] = hbm_c
    rec["roofline"]["frac_of_ceiling"] = rec["roofline"]["achieved"] / hbm_c
    rec["indexer_alone"]["frac_of_ceiling"] = rec["indexer_alone"]["achieved"] / hbm_c
    rec["step"]["frac_of_hbm_ceiling"] = rec["step"]["GB_per_s"] / hbm_c
    if "attention" in rec:
        rec["attention"]["frac_of_ceiling"] = rec["attention"]["GB_per_s"] / hbm_c
    if "prefill" in rec:
        rec["prefill"]["roofline"]["ceiling"] = mfma_c
        rec["prefill"]["roofline"]["frac_of_ceiling"] = rec["prefill"]["roofline"]["achieved"] / mfma_c

    if args.copy_probe > 0:
        n = args.copy_probe
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        rec["copy_probe_bytes"] = n

    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(w, x, gpu_res)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
