"""Seeded synthetic weights and inputs for the jina-ocr-v1 decoder shapes.

This module is the only code shared by the HIP product path and the CPU
oracle. It draws random numbers and lays them out; it holds none of the
decoder's arithmetic (no norm, attention, routing, GEMV or argmax).

Shapes come from the model tables of the jina-ocr-v1 announcement and blog
("Model parameters" / spec table: 12 layers, d=1280, 64 routed + 2 shared
experts, top-6, vocabulary 129,280, RoPE theta 1e6, one recursive draft
block).  Head count (10 x 128), expert width 896 and draft FFN width 3,584
are a reading of what the pages leave open; with them the decoder has ~575M
active and ~3.14B total parameters, in line with the active and total decoder
sizes the pages state (about 570M and 3B).

Recipe (stated once, used everywhere):
  * every tensor t (index i in ``weight_specs`` order) is split into blocks of
    2**22 elements; block j is drawn from ``numpy.random.default_rng([seed, i, j])``
    as ``standard_normal(float32)``;
  * matrices and the embedding table: value = 0.02 * draw (float32), then, for a
    bf16 model, rounded to bf16 with round-to-nearest-even;
  * RMSNorm gains: value = 1 + 0.02 * draw (float32, always stored as float32);
  * vision-prefix rows: ``default_rng([seed, 1, b])`` standard normal float32;
  * prompt ids: ``default_rng([seed, 2, b])`` integers uniform in [0, vocab).
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

BLOCK = 1 << 22


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    n_layers: int = 12
    d_model: int = 1280
    n_heads: int = 10
    head_dim: int = 128
    n_experts: int = 64
    n_shared: int = 2
    top_k: int = 6
    d_expert: int = 896
    d_draft_ffn: int = 3584
    vocab: int = 129280
    rope_theta: float = 1.0e6
    norm_eps: float = 1.0e-6
    dtype: str = "bf16"          # "bf16" or "f32": storage type of matrices / embedding

    @property
    def qkv_dim(self) -> int:
        return self.n_heads * self.head_dim


# The decoder of the pages at the widths read for it above.
FULL = ModelConfig()


def weight_specs(cfg: ModelConfig) -> List[Tuple[str, Tuple[int, ...], str]]:
    """Canonical weight list: (name, shape, kind), kind in {"matrix", "gain"}.

    Matrices follow the y = W x convention: shape [out, in], row-major.
    ``wqkv`` stacks the q, k and v projections (rows 0..Hd-1 = q, then k, then v,
    each head-major).  Expert tensors hold the routed experts 0..E-1 followed by
    the shared experts E..E+S-1.  This order is also the order of the
    ``weight_ptrs`` array of ``ocrdec_create``.
    """
    d, V, Hd = cfg.d_model, cfg.vocab, cfg.qkv_dim
    E, I, F = cfg.n_experts + cfg.n_shared, cfg.d_expert, cfg.d_draft_ffn
    specs: List[Tuple[str, Tuple[int, ...], str]] = [
        ("embed", (V, d), "matrix"),
        ("lm_head", (V, d), "matrix"),
        ("final_norm", (d,), "gain"),
    ]
    for l in range(cfg.n_layers):
        specs += [
            (f"l{l}.attn_norm", (d,), "gain"),
            (f"l{l}.wqkv", (3 * Hd, d), "matrix"),
            (f"l{l}.wo", (d, Hd), "matrix"),
            (f"l{l}.ffn_norm", (d,), "gain"),
            (f"l{l}.router", (cfg.n_experts, d), "matrix"),
            (f"l{l}.w_gate", (E, I, d), "matrix"),
            (f"l{l}.w_up", (E, I, d), "matrix"),
            (f"l{l}.w_down", (E, d, I), "matrix"),
        ]
    specs += [
        ("draft.norm_h", (d,), "gain"),
        ("draft.norm_e", (d,), "gain"),
        ("draft.fuse", (d, 2 * d), "matrix"),
        ("draft.attn_norm", (d,), "gain"),
        ("draft.wqkv", (3 * Hd, d), "matrix"),
        ("draft.wo", (d, Hd), "matrix"),
        ("draft.ffn_norm", (d,), "gain"),
        ("draft.w_gate", (F, d), "matrix"),
        ("draft.w_up", (F, d), "matrix"),
        ("draft.w_down", (d, F), "matrix"),
        ("draft.out_norm", (d,), "gain"),
    ]
    return specs


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw_tensor(seed: int, index: int, n: int, kind: str, out: np.ndarray, pool) -> None:
    nblk = (n + BLOCK - 1) // BLOCK

    def one(j: int) -> None:
        lo, hi = j * BLOCK, min(n, (j + 1) * BLOCK)
        x = np.random.default_rng([seed, index, j]).standard_normal(hi - lo, dtype=np.float32)
        x *= np.float32(0.02)
        if kind == "gain":
            x += np.float32(1.0)
        out[lo:hi] = x

    if pool is None or nblk == 1:
        for j in range(nblk):
            one(j)
    else:
        list(pool.map(one, range(nblk)))


class Weights:
    """Seeded weights of one model.  ``f32[name]`` holds the exact values the
    model uses (bf16 models: the bf16-rounded values widened to float32);
    ``device_arrays()`` gives the arrays in their storage dtype (matrices as
    uint16 bf16 bits for bf16 models, float32 otherwise; gains float32)."""

    def __init__(self, cfg: ModelConfig, seed: int, threads: int = 16):
        self.cfg = cfg
        self.seed = seed
        self.specs = weight_specs(cfg)
        self.f32: Dict[str, np.ndarray] = {}
        self._bits: Dict[str, np.ndarray] = {}
        pool = ThreadPoolExecutor(max_workers=threads) if threads > 1 else None
        try:
            for i, (name, shape, kind) in enumerate(self.specs):
                n = int(np.prod(shape))
                flat = np.empty(n, dtype=np.float32)
                _draw_tensor(seed, i, n, kind, flat, pool)
                if kind == "matrix" and cfg.dtype == "bf16":
                    bits = _parallel_round(flat, pool)
                    self._bits[name] = bits.reshape(shape)
                    flat = bf16_bits_to_f32(bits)
                self.f32[name] = flat.reshape(shape)
        finally:
            if pool is not None:
                pool.shutdown()

    def storage(self, name: str) -> np.ndarray:
        return self._bits.get(name, self.f32[name])

    def device_arrays(self) -> List[np.ndarray]:
        return [self.storage(name) for name, _, _ in self.specs]

    def drop_f32_matrices(self) -> None:
        """Free the widened copies of bf16 matrices (keeps storage bits)."""
        if self.cfg.dtype == "bf16":
            for name, _, kind in self.specs:
                if kind == "matrix":
                    self.f32.pop(name, None)


def _parallel_round(flat: np.ndarray, pool) -> np.ndarray:
    n = flat.size
    out = np.empty(n, dtype=np.uint16)
    nblk = (n + BLOCK - 1) // BLOCK

    def one(j: int) -> None:
        lo, hi = j * BLOCK, min(n, (j + 1) * BLOCK)
        out[lo:hi] = f32_to_bf16_bits(flat[lo:hi])

    if pool is None or nblk == 1:
        for j in range(nblk):
            one(j)
    else:
        list(pool.map(one, range(nblk)))
    return out


def vision_prefix(cfg: ModelConfig, seed: int, b: int, n_vision: int) -> np.ndarray:
    """Stand-in for the vision encoder's output: n_vision rows ~ N(0, 1), float32."""
    return np.random.default_rng([seed, 1, b]).standard_normal((n_vision, cfg.d_model), dtype=np.float32)


def prompt_ids(cfg: ModelConfig, seed: int, b: int, n_prompt: int) -> np.ndarray:
    return np.random.default_rng([seed, 2, b]).integers(0, cfg.vocab, size=n_prompt, dtype=np.int64).astype(np.int32)


@dataclasses.dataclass
class Page:
    """One synthetic page: vision rows followed by prompt ids; n_out output tokens."""
    vision: np.ndarray       # [n_vision, d] float32
    prompt: np.ndarray       # [n_prompt] int32
    n_out: int

    @property
    def prefix_len(self) -> int:
        return self.vision.shape[0] + self.prompt.shape[0]


def make_pages(cfg: ModelConfig, seed: int, n_vision: Sequence[int], n_prompt: Sequence[int],
               n_out: Sequence[int]) -> List[Page]:
    return [Page(vision_prefix(cfg, seed, b, nv), prompt_ids(cfg, seed, b, npr), int(no))
            for b, (nv, npr, no) in enumerate(zip(n_vision, n_prompt, n_out))]


def concurrent_page_lengths(seed: int, batch: int, mean_out: float = 1085.0, sigma: float = 0.5,
                            cap: int = 4096) -> Tuple[np.ndarray, np.ndarray]:
    """Per-sequence Gundam tile count n ~ U{0..9} (prefix 256 + 100 n vision rows) and output
    length ~ round(LogNormal(mu, sigma)) with mean ``mean_out`` before the cap of
    ``cap`` (the usage example's max_tokens)."""
    rng = np.random.default_rng([seed, 3])
    n = rng.integers(0, 10, size=batch)
    mu = math.log(mean_out) - sigma * sigma / 2.0
    out = np.minimum(np.rint(rng.lognormal(mu, sigma, size=batch)).astype(np.int64), cap)
    return (256 + 100 * n).astype(np.int64), np.maximum(out, 1)


def longctx_kv(cfg: ModelConfig, seed: int, n_pos: int) -> np.ndarray:
    """Synthetic verifier cache of one sequence for the long-context layer
    benchmark: keys and values ~ N(0, 1) rounded to bf16, as bf16 bit patterns
    in the library's cache order [layer][K|V][head][pos][head_dim] (uint16)."""
    shape = (cfg.n_layers, 2, cfg.n_heads, n_pos, cfg.head_dim)
    a = np.random.default_rng([seed, 4]).standard_normal(shape, dtype=np.float32)
    return f32_to_bf16_bits(a)


def zipf_router_logits(seed: int, rows: int, n_layers: int = 1, n_experts: int = 64, s: float = 1.1) -> np.ndarray:
    """Skewed routing for the long-context layer benchmark: logit_e = log pi(e) +
    Gumbel(0, 1), pi(e) proportional to rank(e)^-s over a seeded permutation of the
    experts, so top-6 by logit samples 6 experts without replacement with
    probabilities pi.  float32 [n_layers][rows][n_experts]."""
    rng = np.random.default_rng([seed, 5])
    out = np.empty((n_layers, rows, n_experts), dtype=np.float32)
    for l in range(n_layers):
        rank = np.empty(n_experts, dtype=np.int64)
        rank[rng.permutation(n_experts)] = np.arange(1, n_experts + 1)
        logp = -s * np.log(rank.astype(np.float64))
        logp -= np.log(np.exp(logp).sum())
        g = rng.gumbel(size=(rows, n_experts))
        out[l] = (logp[None, :] + g).astype(np.float32)
    return out


# Named workloads (shapes, lengths and seeds).  Weight seeds: 1230 for the
# 2-layer fp32 model, 1234 for the 12-layer bf16 model; input seeds 2000 + index.
WORKLOADS = {
    "tiny_fp32_2layer": dict(cfg=dataclasses.replace(FULL, n_layers=2, dtype="f32"), weight_seed=1230,
                             input_seed=2000, n_vision=256, n_prompt=16, n_out=64, batch=1),
    "base_page_bf16": dict(cfg=FULL, weight_seed=1234, input_seed=2001, n_vision=256, n_prompt=32,
                           n_out=1085, batch=1),
    "gundam_page_bf16": dict(cfg=FULL, weight_seed=1234, input_seed=2002, n_vision=1156, n_prompt=32,
                             n_out=3568, batch=1),
    "concurrent32_bf16": dict(cfg=FULL, weight_seed=1234, input_seed=2003, n_vision=None, n_prompt=32,
                              n_out=None, batch=32),
    "longctx_layer_bf16": dict(cfg=dataclasses.replace(FULL, n_layers=1), weight_seed=1234,
                               input_seed=2004, n_vision=None, n_prompt=None, n_out=None, batch=None,
                               n_cached=32764, batches=(1, 4, 16, 64), kv_seed=5000),
}

# Per-slot replacement probability p for the controlled-acceptance drafts: the
# solution of sum_{j=1..K} (1-p)^j = K * alpha for the acceptance rates of the
# L4 table (82.6 / 69.1 / 57.6 % for K = 1 / 2 / 3; 82.9 % for the K=1 graph row).
def replacement_probability(alpha: float, k: int) -> float:
    lo, hi = 0.0, 1.0
    for _ in range(200):
        p = 0.5 * (lo + hi)
        s = sum((1.0 - p) ** j for j in range(1, k + 1))
        if s > k * alpha:
            lo = p
        else:
            hi = p
    return 0.5 * (lo + hi)
