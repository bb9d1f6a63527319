"""Seeded synthetic inputs for the partition-attention path.

This module only draws random numbers and packs them as bfloat16 bits. It holds
none of the method's arithmetic (no scoring, no rotation, no softmax): both the
CPU oracle and the HIP path receive the arrays it returns, unchanged.

Workload shapes follow the PackForcing pages:
  * block of B_f latent frames patchifies to n = B_f*h*w tokens
    [PackForcing, arXiv HTML, "KV Caching"]; defaults B_f=4, h=30, w=52 give
    n = 6,240 [same page, "Compressed Mid Tokens"];
  * a compressed mid block holds N_c = floor(B_f/2)*floor(h/4)*floor(w/4) tokens
    [same page, "Compressed Mid Tokens"];
  * N_sink = 8 frames (2 blocks), N_recent = 4 frames (1 block), N_top = 16
    [same page, "Implementation Details"];
  * 30 layers, hidden 1536 = 12 heads x 128 [PackForcing digest
    (paper.rainbus.top), "研究动机"; arXiv HTML, "HR Branch" and
    "The Position Misalignment Problem"].

Every array is row-major [rows][heads][128] of uint16 bfloat16 bits.
Draw order per cache: Q, K_sink, V_sink, K_pool, V_pool, K_recent, V_recent,
K_cur, V_cur, then (where used) block offsets, query offsets and deltas.
Values are float32 standard normals times a scale, rounded to bfloat16 with
round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

HEAD_DIM = 128


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    heads: int
    block_frames: int          # B_f
    h: int                     # latent height after patchification
    w: int                     # latent width after patchification
    sink_blocks: int           # N_sink / B_f
    pool_blocks: int           # compressed blocks held in the mid pool
    top_k: int                 # N_top
    recent_blocks: int         # N_recent / B_f
    scale: float               # std of the Q/K/V draws
    pool_offset_std: float = 0.0   # block-wise mean offset on pool keys
    query_offset_std: float = 0.0  # per-head mean offset on queries
    delta_range: Optional[tuple] = None  # (lo, hi) inclusive: drawn deltas
    layers: int = 1
    steps: int = 1
    seed: int = 0
    q_mult: float = 1.0        # multiplies Q after drawing ("sharp" variant)

    @property
    def n(self) -> int:
        return self.block_frames * self.h * self.w

    @property
    def n_c(self) -> int:
        return (self.block_frames // 2) * (self.h // 4) * (self.w // 4)

    @property
    def n_sink(self) -> int:
        return self.sink_blocks * self.n

    @property
    def n_recent(self) -> int:
        return self.recent_blocks * self.n

    @property
    def n_keys(self) -> int:
        return self.n_sink + self.top_k * self.n_c + self.n_recent + self.n

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


# The five workloads. C0 is the tiny case the oracle finishes in seconds, C1 the
# default single layer, C2 the 2-minute pool (116 blocks: 2 sink + 116 mid +
# 1 recent + 1 current = 120 blocks of history), C3 the full 30-layer x
# 4-step generation step at C2 shapes, C4 the unbounded contrast (748,800
# full-resolution keys, no compression, no selection).
C0 = Config("C0-tiny", heads=2, block_frames=4, h=8, w=8, sink_blocks=2,
            pool_blocks=10, top_k=4, recent_blocks=1, scale=1.0,
            delta_range=(1, 20), seed=1000)
C1 = Config("C1-default", heads=12, block_frames=4, h=30, w=52, sink_blocks=2,
            pool_blocks=40, top_k=16, recent_blocks=1, scale=float(1 / np.sqrt(2)),
            seed=1001)
C2 = C1.replace(name="C2-2min-pool", pool_blocks=116, pool_offset_std=0.5, seed=1002)
C2Q = C2.replace(name="C2q-2min-pool-query-offset", query_offset_std=1.0, seed=1012)
C3 = C2.replace(name="C3-full-step", layers=30, steps=4, seed=1003)
C4 = Config("C4-unbounded", heads=12, block_frames=4, h=30, w=52, sink_blocks=2,
            pool_blocks=0, top_k=0, recent_blocks=117, scale=float(1 / np.sqrt(2)),
            seed=1004)

CONFIGS = {c.name: c for c in (C0, C1, C2, C2Q, C3, C4)}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest even (inputs are finite)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def _normal(rng: np.random.Generator, rows: int, heads: int, scale: float) -> np.ndarray:
    a = rng.standard_normal((rows, heads, HEAD_DIM), dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return a


def make_cache(cfg: Config, seed: int, pool_blocks: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw one layer's cache and the current block's queries.

    Returns bf16-bit arrays q, sink_k, sink_v, pool_k, pool_v, recent_k,
    recent_v, cur_k, cur_v, plus int32 'deltas' when the config draws them.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    H, s = cfg.heads, cfg.scale
    M = cfg.pool_blocks if pool_blocks is None else pool_blocks
    out: Dict[str, np.ndarray] = {}
    q = _normal(rng, cfg.n, H, s)
    sink_k = _normal(rng, cfg.n_sink, H, s)
    sink_v = _normal(rng, cfg.n_sink, H, s)
    pool_k = _normal(rng, M * cfg.n_c, H, s)
    pool_v = _normal(rng, M * cfg.n_c, H, s)
    recent_k = _normal(rng, cfg.n_recent, H, s)
    recent_v = _normal(rng, cfg.n_recent, H, s)
    cur_k = _normal(rng, cfg.n, H, s)
    cur_v = _normal(rng, cfg.n, H, s)
    if cfg.pool_offset_std > 0 and M > 0:
        off = rng.standard_normal((M, 1, H, HEAD_DIM), dtype=np.float32) * np.float32(cfg.pool_offset_std)
        pool_k = (pool_k.reshape(M, cfg.n_c, H, HEAD_DIM) + off).reshape(M * cfg.n_c, H, HEAD_DIM)
    if cfg.query_offset_std > 0:
        nu = rng.standard_normal((1, H, HEAD_DIM), dtype=np.float32) * np.float32(cfg.query_offset_std)
        q = q + nu
    if cfg.q_mult != 1.0:
        q = q * np.float32(cfg.q_mult)
    if cfg.delta_range is not None:
        lo, hi = cfg.delta_range
        out["deltas"] = rng.integers(lo, hi + 1, size=max(cfg.top_k, 1), dtype=np.int64).astype(np.int32)
    for name, arr in (("q", q), ("sink_k", sink_k), ("sink_v", sink_v), ("pool_k", pool_k),
                      ("pool_v", pool_v), ("recent_k", recent_k), ("recent_v", recent_v),
                      ("cur_k", cur_k), ("cur_v", cur_v)):
        out[name] = bf16_bits(arr)
    return out


def make(cfg: Config, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """One layer's cache for a single-layer config (C0, C1, C2, C2q, C4)."""
    return make_cache(cfg, cfg.seed if seed is None else seed)


def layer_seed(cfg: Config, layer: int, seed: Optional[int] = None) -> int:
    ss = np.random.SeedSequence([cfg.seed if seed is None else seed, layer])
    return int(ss.generate_state(1, dtype=np.uint64)[0])


def step_queries(cfg: Config, layer: int, step: int, seed: Optional[int] = None) -> np.ndarray:
    """Queries of the current block at one (layer, denoising step) of C3."""
    ss = np.random.SeedSequence([cfg.seed if seed is None else seed, layer, step, 1])
    rng = np.random.Generator(np.random.PCG64(ss))
    q = _normal(rng, cfg.n, cfg.heads, cfg.scale)
    if cfg.query_offset_std > 0:
        q = q + rng.standard_normal((1, cfg.heads, HEAD_DIM), dtype=np.float32) * np.float32(cfg.query_offset_std)
    return bf16_bits(q)


def rollin_block(cfg: Config, layer: int, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """The synthetic compressed block that slides into a layer's pool after the step."""
    ss = np.random.SeedSequence([cfg.seed if seed is None else seed, layer, 99])
    rng = np.random.Generator(np.random.PCG64(ss))
    k = _normal(rng, cfg.n_c, cfg.heads, cfg.scale)
    v = _normal(rng, cfg.n_c, cfg.heads, cfg.scale)
    if cfg.pool_offset_std > 0:
        k = k + rng.standard_normal((1, cfg.heads, HEAD_DIM), dtype=np.float32) * np.float32(cfg.pool_offset_std)
    return {"k": bf16_bits(k), "v": bf16_bits(v)}


def planted_pool(cfg: Config, seed: int, chosen: List[int], margin: float = 4.0) -> Dict[str, np.ndarray]:
    """A cache whose top-k blocks are known by construction.

    A per-head query mean nu_h is added to every query; the chosen blocks' keys
    get +margin * nu_h/|nu_h| so their pooled affinity stands far above the rest.
    Only random draws and additions happen here.
    """
    base = make_cache(cfg.replace(query_offset_std=0.0), seed)
    rng = np.random.Generator(np.random.PCG64(seed + 7))
    H = cfg.heads
    nu = rng.standard_normal((H, HEAD_DIM)).astype(np.float32)
    unit = nu / np.linalg.norm(nu, axis=1, keepdims=True)
    q = _from_bits(base["q"]) + nu[None]
    pk = _from_bits(base["pool_k"]).reshape(cfg.pool_blocks, cfg.n_c, H, HEAD_DIM)
    for j in chosen:
        pk[j] += np.float32(margin) * unit[None]
    base["q"] = bf16_bits(q)
    base["pool_k"] = bf16_bits(pk.reshape(-1, H, HEAD_DIM))
    return base


def _from_bits(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# HR-branch compressor inputs: a latent block and synthetic weights
# ---------------------------------------------------------------------------
# The latent block is what the VAE yields for one generated block: B_f = 4
# latent frames of 60 x 104 (the 30 x 52 token grid before the 1x2x2 patch
# embedding) [PackForcing, arXiv HTML, "HR Branch" and "Feature Fusion"], with
# 16 latent channels (the base model's VAE; the pages do not print it). The
# stage widths are this library's reading (the pages give none): 256, 512,
# 1024, 2048, then the hidden width 1536. Trained weights are not available;
# these are seeded draws with fan-in scaling, so activations stay of order 1.

HR_LATENT = dict(frames=4, height=60, width=104, channels=16)
HR_WIDTHS = (256, 512, 1024, 2048)
HR_HIDDEN = 1536
HR_KERNELS = ((2, 1, 1), (1, 2, 2), (1, 2, 2), (1, 2, 2))


def hr_latent(seed: int, batch: int = 1, frames: int = 4, height: int = 60, width: int = 104,
              channels: int = 16) -> np.ndarray:
    """[batch][frames][height][width][channels] standard normals as bf16 bits."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return bf16_bits(rng.standard_normal((batch, frames, height, width, channels), dtype=np.float32))


def hr_weights(seed: int, channels: int = 16, widths=HR_WIDTHS, hidden: int = HR_HIDDEN,
               kernels=HR_KERNELS, bias_std: float = 0.1):
    """Seeded weights for the strided stages and the projection.

    Returns (stages, proj): stages is a list of (w_bits [C_out][kt][kh][kw][C_in],
    bias float32 [C_out]); proj is (w_bits [hidden][C_last], bias float32).
    Each weight is N(0, 2/fan_in), each bias N(0, bias_std^2).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    stages = []
    c_in = channels
    for c_out, (kt, kh, kw) in zip(widths, kernels):
        fan_in = kt * kh * kw * c_in
        w = rng.standard_normal((c_out, kt, kh, kw, c_in), dtype=np.float32) * np.float32(np.sqrt(2.0 / fan_in))
        b = rng.standard_normal(c_out, dtype=np.float32) * np.float32(bias_std)
        stages.append((bf16_bits(w), b))
        c_in = c_out
    wp = rng.standard_normal((hidden, c_in), dtype=np.float32) * np.float32(np.sqrt(1.0 / c_in))
    bp = rng.standard_normal(hidden, dtype=np.float32) * np.float32(bias_std)
    return stages, (bf16_bits(wp), bp)
