"""Seeded synthetic inputs for one HSA chunk-layer over an HKV page pool.

This module only draws numbers. It holds none of the method's arithmetic:
no means, scores, softmax, selection or attention. Both the float64 CPU
oracle and the HIP path receive the exact arrays returned here, so the two
sides see identical bits.

Shapes follow the efficiency settings of the WorldAttention pages (Wan 1.3B
and 14B, 480p and 720p, 60 s and 90 s horizons; news summary, kernel
paragraph and Table 11) with the HKV constants Psize = 8 frames and Kp = 4
(news summary, HKV paragraph, Table 5) and the HSA constants Binter = 128,
Bintra = 64, tau_min = 0.35, tau_max = 1.00 (news summary, HSA paragraph and
Table 4). Values are synthetic stand-ins for real activations:

* Q, V ~ N(0, 1) i.i.d.
* K of page p, head h = mu[p, h] + N(0, 0.5) noise with mu[p, h] ~ N(0, I_d)
  for the clustered workloads; the current chunk's keys get their own mean.
  N(m, s) names a variance s throughout, so N(0, 0.5) has std sqrt(0.5).
* Linformer projections E, F ~ N(0, 1/L), L = Kp*Tp + Lq.
* Gate weights w_g ~ N(0, 1/d), bias b_g = 0.
* tau_h per head: alternating 0.35 / 1.0 for the tiny case, else U[tau_min, 1).
* Upstream gradient of the output (backward cases) ~ N(0, 1) in the storage
  type; a stand-in for the sparse branch's output, where the backward needs
  one without running the sparse branch, ~ N(0, 1/4) in float32.

bf16 tensors are drawn in float32 and rounded once, round-to-nearest-even,
and returned as uint16 bit patterns. float32 tensors are returned as
float32. Every page and every chunk tensor has its own seed stream, so any
single page can be regenerated without holding the whole pool.
"""

from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = [
    "Shape",
    "SHAPES",
    "shape",
    "round_bf16_bits",
    "bf16_bits_to_f32",
    "draw_page",
    "draw_pool",
    "draw_chunk",
    "draw_tau",
    "page_prompts",
    "draw_upstream",
]

# Stream tags inside one workload seed.
_TAG_PAGE = 1
_TAG_CHUNK = 2
_TAG_TAU = 3
_TAG_PROMPT = 4
_TAG_UPSTREAM = 5


@dataclasses.dataclass(frozen=True)
class Shape:
    """One chunk-layer workload. Every size is a plain count of elements."""

    name: str
    dtype: str              # "f32" or "bf16": q/k/v/pool/E/F/out storage type
    H: int                  # heads
    d: int                  # head dimension
    Lq: int                 # current-chunk tokens (queries = intra keys)
    tokens_per_frame: int
    Psize: int              # frames per page
    P: int                  # pages in the HBM pool
    Kp: int                 # pages retrieved per chunk-layer
    Binter: int             # history key-block size
    Bintra: int             # current-chunk key-block size
    Bq: int                 # query-block size
    r: int                  # Linformer rank
    clustered: bool         # per-(page, head) key means, else i.i.d. keys
    prompt_law: str         # "mod2", "all0" or "seg16"
    cur_prompt: int
    tau_law: str            # "alt" or "uniform"
    tau_min: float = 0.35
    seed: int = 1000

    @property
    def Tp(self) -> int:
        return self.Psize * self.tokens_per_frame

    @property
    def L(self) -> int:
        """Linformer sequence length: every slot's tokens plus the chunk."""
        return self.Kp * self.Tp + self.Lq

    def with_(self, **kw) -> "Shape":
        return dataclasses.replace(self, **kw)


SHAPES: Dict[str, Shape] = {
    # Tiny fp32 single layer: 6 pages x 128 tokens, prompt ids p mod 2.
    "tiny": Shape("tiny", "f32", H=2, d=64, Lq=256, tokens_per_frame=16, Psize=8,
                  P=6, Kp=2, Binter=128, Bintra=64, Bq=64, r=32, clustered=False,
                  prompt_law="mod2", cur_prompt=0, tau_law="alt", seed=1000),
    # Wan-1.3B-shaped 480p: 1560 tokens/frame, 3-frame chunk, 32-page pool.
    "wan1.3b-480p": Shape("wan1.3b-480p", "bf16", H=12, d=128, Lq=4680,
                          tokens_per_frame=1560, Psize=8, P=32, Kp=4, Binter=128,
                          Bintra=64, Bq=64, r=256, clustered=True, prompt_law="all0",
                          cur_prompt=0, tau_law="uniform", seed=1001),
    # Same shape, 60 s horizon: 96 pages in 6 prompt segments of 16; the
    # current prompt is the oldest segment, so the matches are non-recent.
    "wan1.3b-480p-60s": Shape("wan1.3b-480p-60s", "bf16", H=12, d=128, Lq=4680,
                              tokens_per_frame=1560, Psize=8, P=96, Kp=4, Binter=128,
                              Bintra=64, Bq=64, r=256, clustered=True,
                              prompt_law="seg16", cur_prompt=0, tau_law="uniform",
                              seed=1002),
    # Wan-14B-shaped 480p.
    "wan14b-480p": Shape("wan14b-480p", "bf16", H=40, d=128, Lq=4680,
                         tokens_per_frame=1560, Psize=8, P=32, Kp=4, Binter=128,
                         Bintra=64, Bq=64, r=256, clustered=True, prompt_law="all0",
                         cur_prompt=0, tau_law="uniform", seed=1003),
    # Wan-14B-shaped 720p, 90 s horizon: 3600 tokens/frame, 24-page pool.
    "wan14b-720p-90s": Shape("wan14b-720p-90s", "bf16", H=40, d=128, Lq=10800,
                             tokens_per_frame=3600, Psize=8, P=24, Kp=4, Binter=128,
                             Bintra=64, Bq=64, r=512, clustered=True, prompt_law="all0",
                             cur_prompt=0, tau_law="uniform", seed=1004),
}


def shape(name: str, **overrides) -> Shape:
    s = SHAPES[name]
    return s.with_(**overrides) if overrides else s


# ---------------------------------------------------------------------------
# storage-type helpers (bit handling only)

def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even.

    Inputs here are finite normals, so no NaN handling is needed.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = b + (np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the exactly equal float32 values."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16_bits(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def _rng(s: Shape, *tags: int) -> np.random.Generator:
    return np.random.default_rng([s.seed, *tags])


def _normal(rng: np.random.Generator, shape, var: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if var != 1.0:
        x *= np.float32(np.sqrt(var))
    return x


# ---------------------------------------------------------------------------
# pages

def _keys(rng: np.random.Generator, s: Shape, n_tok: int) -> np.ndarray:
    if not s.clustered:
        return _normal(rng, (n_tok, s.H, s.d))
    mu = _normal(rng, (1, s.H, s.d))
    noise = _normal(rng, (n_tok, s.H, s.d), 0.5)
    noise += mu
    return noise


def draw_page(s: Shape, p: int) -> Tuple[np.ndarray, np.ndarray]:
    """K and V of pool page p, each [Tp][H][d] in the storage type."""
    rng = _rng(s, _TAG_PAGE, p)
    k = _store(_keys(rng, s, s.Tp), s.dtype)
    v = _store(_normal(rng, (s.Tp, s.H, s.d)), s.dtype)
    return k, v


def draw_pool(s: Shape, threads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """The whole pool, pool_k and pool_v each [P][Tp][H][d] in the storage type."""
    st = np.uint16 if s.dtype == "bf16" else np.float32
    pool_k = np.empty((s.P, s.Tp, s.H, s.d), dtype=st)
    pool_v = np.empty((s.P, s.Tp, s.H, s.d), dtype=st)

    def one(p: int) -> None:
        k, v = draw_page(s, p)
        pool_k[p] = k
        pool_v[p] = v

    n = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(n) as ex:
        list(ex.map(one, range(s.P)))
    return pool_k, pool_v


def page_prompts(s: Shape) -> np.ndarray:
    """Integer prompt tag of every page, int32 [P]."""
    p = np.arange(s.P, dtype=np.int64)
    if s.prompt_law == "mod2":
        ids = p % 2
    elif s.prompt_law == "all0":
        ids = np.zeros_like(p)
    elif s.prompt_law == "seg16":
        ids = p // 16
    else:
        raise ValueError(s.prompt_law)
    return ids.astype(np.int32)


def draw_tau(s: Shape) -> np.ndarray:
    """Per-head mass threshold tau_h, float32 [H]."""
    if s.tau_law == "alt":
        return np.array([0.35 if h % 2 == 0 else 1.0 for h in range(s.H)], dtype=np.float32)
    if s.tau_law == "uniform":
        rng = _rng(s, _TAG_TAU)
        return rng.uniform(s.tau_min, 1.0, size=s.H).astype(np.float32)
    raise ValueError(s.tau_law)


def draw_chunk(s: Shape) -> Dict[str, np.ndarray]:
    """Per-chunk tensors: q, k_intra, v_intra [Lq][H][d]; E, F [r][L];
    w_g [H][d] f32; b_g [H] f32; tau [H] f32; page_prompt [P] i32."""
    rng = _rng(s, _TAG_CHUNK)
    q = _store(_normal(rng, (s.Lq, s.H, s.d)), s.dtype)
    k_intra = _store(_keys(rng, s, s.Lq), s.dtype)
    v_intra = _store(_normal(rng, (s.Lq, s.H, s.d)), s.dtype)
    E = _store(_normal(rng, (s.r, s.L), 1.0 / s.L), s.dtype)
    F = _store(_normal(rng, (s.r, s.L), 1.0 / s.L), s.dtype)
    w_g = _normal(rng, (s.H, s.d), 1.0 / s.d).astype(np.float32)
    b_g = np.zeros((s.H,), dtype=np.float32)
    return {
        "q": q, "k_intra": k_intra, "v_intra": v_intra, "E": E, "F": F,
        "w_g": w_g, "b_g": b_g, "tau": draw_tau(s), "page_prompt": page_prompts(s),
    }


def draw_upstream(s: Shape) -> Dict[str, np.ndarray]:
    """Backward inputs: d_out [Lq][H][d] in the storage type (the upstream
    gradient of the output) and o_sparse [Lq][H][d] float32 (a stand-in for
    the sparse branch's output where a case does not run that branch)."""
    rng = _rng(s, _TAG_UPSTREAM)
    d_out = _store(_normal(rng, (s.Lq, s.H, s.d)), s.dtype)
    o_sparse = _normal(rng, (s.Lq, s.H, s.d), 0.25).astype(np.float32)
    return {"d_out": d_out, "o_sparse": o_sparse}
