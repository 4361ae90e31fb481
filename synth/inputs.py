"""Seeded synthetic workloads shaped like DeepSeek V4 Flash / Pro attention layers.

Shapes follow the model-shape constants printed in "Reading the architecture of
DwarfStar (ds4.c), part 1/8" (Qiita), section 2 ("target model"): 64 query
heads (128 for Pro), one 512-dim KV head, RoPE on the last 64 dims, a 128-row
raw sliding window, an indexer with 64 heads of 128 dims, top-k 512 (1024 for
Pro).  The same article's section 3-1 rounds every raw-window value to f16,
so raw rows are generated already f16-rounded.

Recipe (every tensor of every unit has its own stream):
    rng = numpy.random.Generator(PCG64(SeedSequence([0xD54A, cfg_id, seed, unit, tensor_id])))
    tensor ids: q=0, raw=1, comp=2, idx_k=3, idx_q=4, idx_w=5, heavy=6, idx_k8=7, idx_k_scale=8
Normal values are drawn as float32 N(0,1) and rounded once, round-to-nearest-even,
to the stored dtype (bf16 or f16); f32 tensors are stored as drawn.  Indexer
head weights are float32 U(0,1).  "Heavy" rows: round(frac*N) distinct rows
whose compressed row and indexer-key row are both multiplied by 4 (exact in
bf16).

FP8-stored indexer keys (the compressor's output format: OCP E4M3FN codes and one
power-of-two scale per row) are drawn as codes directly: sign uniform, exponent
field round(N(11, 1.5)) clipped to 0..15, fraction uniform 0..7, the NaN pattern
S.1111.111 replaced by S.1111.110; row scales 2^e with e uniform in -8..-6 (about
the N(0,1) magnitudes of the bf16 keys), heavy rows' scales times 4.

This module draws and rounds numbers only; it contains none of the
attention arithmetic.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os

import numpy as np

TENSOR_IDS = {"q": 0, "raw": 1, "comp": 2, "idx_k": 3, "idx_q": 4, "idx_w": 5, "heavy": 6, "idx_k8": 7,
              "idx_k_scale": 8}
_CHUNK_ELEMS = 1 << 22


def bf16_bits_from_f32(x) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return the 16-bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    t = b >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    t += b
    t >>= np.uint32(16)
    return t.astype(np.uint16)


def f16_bits_from_f32(x) -> np.ndarray:
    """Round float32 values to IEEE binary16 (numpy's cast is round-to-nearest-even)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One call's worth of work: U independent units (layers or sessions), T query tokens each."""

    name: str
    cfg_id: int
    U: int
    T: int
    N: int
    H: int = 64
    D: int = 512
    n_rot: int = 64
    W: int = 128
    Hi: int = 64
    Di: int = 128
    K: int = 512
    q_dtype: str = "f32"          # "f32" (decode) or "bf16" (prefill)
    heavy_frac: float = 0.0
    vis_base: int | None = None   # prefill: query t sees compressed rows < vis_base + t
    pos_base: int | None = None   # absolute position of query 0 (default 4N - T)
    theta: float = 10000.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def n_vis(self) -> np.ndarray:
        """[U, T] int32: number of visible compressed rows per query."""
        if self.vis_base is None:
            v = np.full(self.T, self.N, dtype=np.int64)
        else:
            v = np.minimum(self.vis_base + np.arange(self.T, dtype=np.int64), self.N)
        return np.broadcast_to(v.astype(np.int32), (self.U, self.T)).copy()

    def positions(self) -> np.ndarray:
        """[U, T] int64 absolute positions.  Decode default: 4N - 1 (one compressed row per 4 tokens)."""
        base = self.pos_base if self.pos_base is not None else 4 * self.N - self.T
        p = base + np.arange(self.T, dtype=np.int64)
        return np.broadcast_to(p, (self.U, self.T)).copy()

    def n_heavy(self) -> int:
        return int(round(self.heavy_frac * self.N))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the benchmark plan, plus the 32K- and 64K-row decode points.
CONFIGS: dict[str, Workload] = {
    "decode_1layer_n2048": Workload("decode_1layer_n2048", 1, U=1, T=1, N=2048, pos_base=8191),
    "decode_43layers_n16384": Workload("decode_43layers_n16384", 2, U=43, T=1, N=16384, heavy_frac=0.01),
    "decode_43layers_n32768": Workload("decode_43layers_n32768", 2, U=43, T=1, N=32768, heavy_frac=0.01),
    "decode_43layers_n65536": Workload("decode_43layers_n65536", 2, U=43, T=1, N=65536, heavy_frac=0.01),
    "prefill_2048q_n8192": Workload("prefill_2048q_n8192", 3, U=1, T=2048, N=8192, q_dtype="bf16",
                   vis_base=4096, pos_base=4096),
    "decode_8sessions_n262144": Workload("decode_8sessions_n262144", 4, U=8, T=1, N=262144),
    "pro_decode_4sessions_n65536": Workload("pro_decode_4sessions_n65536", 5, U=4, T=1, N=65536, H=128, K=1024,
                   heavy_frac=0.005),
}


def _rng(w: Workload, seed: int, unit: int, tensor: str) -> np.random.Generator:
    ss = np.random.SeedSequence([0xD54A, w.cfg_id, seed, unit, TENSOR_IDS[tensor]])
    return np.random.Generator(np.random.PCG64(ss))


def _normal_bf16(rng, rows: int, cols: int) -> np.ndarray:
    """N(0,1) draws rounded to bf16, filled in cache-sized chunks (same stream as one big draw)."""
    out = np.empty((rows, cols), dtype=np.uint16)
    step = max(1, _CHUNK_ELEMS // max(cols, 1))
    buf = np.empty((step, cols), dtype=np.float32)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        x = buf[: r1 - r0]
        rng.standard_normal(out=x, dtype=np.float32)
        out[r0:r1] = bf16_bits_from_f32(x)
    return out


def make_unit(w: Workload, unit: int, seed: int = 0) -> dict[str, np.ndarray]:
    """Inputs of one unit.  bf16 and f16 tensors are returned as uint16 bit patterns."""
    T, H, D, W, N, Hi, Di = w.T, w.H, w.D, w.W, w.N, w.Hi, w.Di
    r = _rng(w, seed, unit, "q")
    if w.q_dtype == "f32":
        q = r.standard_normal((T, H, D), dtype=np.float32)
    elif w.q_dtype == "bf16":
        q = bf16_bits_from_f32(r.standard_normal((T, H, D), dtype=np.float32))
    else:
        raise ValueError(f"q_dtype {w.q_dtype!r}")
    raw = f16_bits_from_f32(_rng(w, seed, unit, "raw").standard_normal((T + W - 1, D), dtype=np.float32))
    comp = _normal_bf16(_rng(w, seed, unit, "comp"), N, D)
    ix = make_indexer_unit(w, unit, seed)
    heavy = ix["heavy"]
    if heavy.size:
        comp[heavy] = bf16_bits_from_f32(bf16_bits_to_f32(comp[heavy]) * np.float32(4.0))
    return {
        "q": q, "raw": raw, "comp": comp, "idx_k": ix["idx_k"], "idx_q": ix["idx_q"], "idx_w": ix["idx_w"],
        "heavy": heavy, "n_vis": w.n_vis()[unit], "pos": w.positions()[unit],
    }


def make_indexer_unit(w: Workload, unit: int, seed: int = 0) -> dict[str, np.ndarray]:
    """The indexer inputs of one unit alone (the same values make_unit returns for them)."""
    T, N, Hi, Di = w.T, w.N, w.Hi, w.Di
    idx_k = _normal_bf16(_rng(w, seed, unit, "idx_k"), N, Di)
    idx_q = bf16_bits_from_f32(_rng(w, seed, unit, "idx_q").standard_normal((T, Hi, Di), dtype=np.float32))
    idx_w = _rng(w, seed, unit, "idx_w").random((T, Hi), dtype=np.float32)
    heavy = np.sort(_rng(w, seed, unit, "heavy").choice(N, size=w.n_heavy(), replace=False)).astype(np.int64)
    if heavy.size:
        idx_k[heavy] = bf16_bits_from_f32(bf16_bits_to_f32(idx_k[heavy]) * np.float32(4.0))
    return {"idx_k": idx_k, "idx_q": idx_q, "idx_w": idx_w, "heavy": heavy}


def e4m3_codes(rng, shape) -> np.ndarray:
    """Finite OCP E4M3FN codes (uint8) with the exponent spread described above."""
    n = int(np.prod(shape))
    e = np.clip(np.rint(rng.normal(11.0, 1.5, n)), 0, 15).astype(np.uint8)
    m = rng.integers(0, 8, n, dtype=np.uint8)
    sign = rng.integers(0, 2, n, dtype=np.uint8)
    c = (sign << np.uint8(7)) | (e << np.uint8(3)) | m
    c[(c & np.uint8(0x7F)) == np.uint8(0x7F)] -= np.uint8(1)
    return c.reshape(shape)


def make_indexer_fp8_unit(w: Workload, unit: int, seed: int = 0) -> dict[str, np.ndarray]:
    """Indexer inputs of one unit with FP8-stored keys: idx_k8 uint8 [N, Di] codes, idx_k_scale
    f32 [N] powers of two; idx_q, idx_w and the heavy rows as make_indexer_unit draws them."""
    T, N, Hi, Di = w.T, w.N, w.Hi, w.Di
    idx_q = bf16_bits_from_f32(_rng(w, seed, unit, "idx_q").standard_normal((T, Hi, Di), dtype=np.float32))
    idx_w = _rng(w, seed, unit, "idx_w").random((T, Hi), dtype=np.float32)
    k8 = e4m3_codes(_rng(w, seed, unit, "idx_k8"), (N, Di))
    scale = np.ldexp(np.float32(1.0), _rng(w, seed, unit, "idx_k_scale").integers(-8, -5, N)).astype(np.float32)
    heavy = np.sort(_rng(w, seed, unit, "heavy").choice(N, size=w.n_heavy(), replace=False)).astype(np.int64)
    if heavy.size:
        scale[heavy] *= np.float32(4.0)
    return {"idx_k8": k8, "idx_k_scale": scale, "idx_q": idx_q, "idx_w": idx_w, "heavy": heavy}


def make_indexer_fp8_config(w: Workload, seed: int = 0, threads: int | None = None) -> dict[str, np.ndarray]:
    """make_indexer_fp8_unit for all U units, stacked."""
    n = threads or min(16, os.cpu_count() or 1, w.U)
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, n)) as ex:
        units = list(ex.map(lambda u: make_indexer_fp8_unit(w, u, seed), range(w.U)))
    return {key: np.stack([x[key] for x in units]) for key in ("idx_k8", "idx_k_scale", "idx_q", "idx_w")}


def make_config(w: Workload, seed: int = 0, threads: int | None = None) -> dict[str, np.ndarray]:
    """All U units stacked on a leading axis (the layout the library's calls take).

    Units are drawn on a thread pool (each unit has its own streams, so the
    result does not depend on the thread count)."""
    n = threads or min(16, os.cpu_count() or 1, w.U)
    if n > 1:
        with concurrent.futures.ThreadPoolExecutor(max_workers=n) as ex:
            units = list(ex.map(lambda u: make_unit(w, u, seed), range(w.U)))
    else:
        units = [make_unit(w, u, seed) for u in range(w.U)]
    out = {}
    for key in ("q", "raw", "comp", "idx_k", "idx_q", "idx_w", "n_vis", "pos"):
        out[key] = np.stack([x[key] for x in units])
    out["heavy"] = [x["heavy"] for x in units]
    return out


def make_indexer_config(w: Workload, seed: int = 0, threads: int | None = None) -> dict[str, np.ndarray]:
    """The indexer inputs (idx_k, idx_q, idx_w) of all U units, stacked, without the attention rows."""
    n = threads or min(16, os.cpu_count() or 1, w.U)
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, n)) as ex:
        units = list(ex.map(lambda u: make_indexer_unit(w, u, seed), range(w.U)))
    return {key: np.stack([x[key] for x in units]) for key in ("idx_k", "idx_q", "idx_w")}
