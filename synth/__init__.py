"""Seeded synthetic inputs for the routed MoE FFN layer.

This module only draws random numbers and stores them in the bit formats the
layer consumes (bf16 activations and router weights, MXFP4 or Q8_0 expert
blocks, an int32 expert->slot map, an optional fp32 router bias). It holds none
of the layer's arithmetic: no routing, no decoding of the block formats, no
matrix products. It is shared by the CPU oracle's tests, the GPU parity tests
and the benchmark, so both sides see the same bytes.

Workload shapes follow the models that the expert-offloading pages run:
GPT-OSS-20B (24 layers x 32 experts, top-4; tinyserve README, "Performance"),
Mixtral 8x7B and a 30B-A3B Qwen MoE (tinyserve README, "Supported models").
Hidden and intermediate sizes, the value distributions and the Zipf load skew
are this project's synthetic stand-ins for those models' real weights, which
are not used.

Layout of what is generated ("canonical" layout, indexed by pool slot):
  x       uint16 [T, H]        bf16 bit patterns, ~N(0, 1) rounded to nearest even
  wr      uint16 [E, H]        bf16 bit patterns, ~N(0, 1/H)
  bias    float32 [E] or None  b_e = -s * ln(r_e), r a seeded permutation of 1..E
  slot_map int32 [E]           expert e lives in pool slot slot_map[e]
  MXFP4:  *_q uint8 [S, rows, K/2]  two E2M1 codes per byte, element 2j in the low nibble
          *_s uint8 [S, rows, K/32] E8M0 scale bytes
  Q8_0:   *_q int8  [S, rows, K]    two's-complement codes
          *_s uint16 [S, rows, K/32] fp16 bit patterns of the block scale d
  Q4_K:   *_q uint8 [S, rows, K/2]  two 4-bit codes per byte, element 2j in the low nibble
          *_s uint8 [S, rows, K/16 + K/64]  per row: (sc_b, m_b) bytes for each 32-block,
                                      then (d_s, dmin_s) fp16 bits for each 256-super-block
  Q5_K:   *_q uint8 [S, rows, K/2 + K/8]  low nibbles as Q4_K, then the high bits (element
                                      8j + i in bit i of byte j); *_s as Q4_K
  Q6_K:   *_q uint8 [S, rows, K/2 + K/4]  low nibbles as Q4_K, then 2-bit high parts
                                      (element 4j + i in bits 2i, 2i+1 of byte j)
          *_s uint8 [S, rows, K/16 + K/128] int8 scale per 16-element sub-block, then fp16 d
                                      per 256-element super-block
  gate/up: rows = I, K = H;  down: rows = H, K = I.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = ["CONFIGS", "Config", "Layer", "make_layer", "make_x", "redraw_x_row",
           "make_router", "make_bias", "make_slot_map", "make_expert", "config"]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    fmt: str            # "mxfp4", "q8_0", "q4_k", "q5_k" or "q6_k"
    zipf_s: float | None
    slot: str           # "identity" or "perm"
    seed: int
    layers: int         # independent layers run back to back when timing

    @property
    def n_pairs(self) -> int:
        return self.T * self.k


# The five workloads, with T variants as separate entries.
CONFIGS: dict[str, Config] = {c.name: c for c in [
    # tiny single layer
    Config("tiny", 64, 256, 512, 8, 2, "mxfp4", None, "identity", 101, 1),
    # GPT-OSS-20B-shaped decode
    Config("gptoss_decode_t1", 1, 2880, 2880, 32, 4, "mxfp4", None, "perm", 202, 24),
    Config("gptoss_decode_t4", 4, 2880, 2880, 32, 4, "mxfp4", None, "perm", 202, 24),
    # GPT-OSS-20B-shaped prefill with a Zipf(1.1) expert load
    Config("gptoss_prefill", 16384, 2880, 2880, 32, 4, "mxfp4", 1.1, "perm", 303, 1),
    # Mixtral-8x7B-shaped layer in Q8_0
    Config("mixtral_q8_decode", 1, 4096, 14336, 8, 2, "q8_0", None, "perm", 404, 8),
    Config("mixtral_q8_prefill", 4096, 4096, 14336, 8, 2, "q8_0", None, "perm", 404, 1),
    # Qwen3-30B-A3B-shaped fine-grained layer with a Zipf(1.2) expert load
    Config("qwen_a3b_decode", 1, 2048, 768, 128, 8, "mxfp4", 1.2, "perm", 505, 64),
    Config("qwen_a3b_prefill", 8192, 2048, 768, 128, 8, "mxfp4", 1.2, "perm", 505, 1),
    # the same two shapes with Q4_K experts (K a multiple of the 256-element super-block)
    Config("tiny_q4k", 64, 256, 512, 8, 2, "q4_k", None, "perm", 606, 1),
    Config("qwen_a3b_q4k_decode", 1, 2048, 768, 128, 8, "q4_k", 1.2, "perm", 707, 64),
    Config("qwen_a3b_q4k_prefill", 8192, 2048, 768, 128, 8, "q4_k", 1.2, "perm", 707, 1),
    Config("mixtral_q4k_decode", 1, 4096, 14336, 8, 2, "q4_k", None, "perm", 808, 8),
    # Q5_K experts on the same shapes
    Config("tiny_q5k", 64, 256, 512, 8, 2, "q5_k", None, "perm", 909, 1),
    Config("qwen_a3b_q5k_decode", 1, 2048, 768, 128, 8, "q5_k", 1.2, "perm", 1010, 64),
    Config("qwen_a3b_q5k_prefill", 8192, 2048, 768, 128, 8, "q5_k", 1.2, "perm", 1010, 1),
    Config("mixtral_q5k_decode", 1, 4096, 14336, 8, 2, "q5_k", None, "perm", 1111, 8),
    # Q6_K experts on the same shapes
    Config("tiny_q6k", 64, 256, 512, 8, 2, "q6_k", None, "perm", 1212, 1),
    Config("qwen_a3b_q6k_decode", 1, 2048, 768, 128, 8, "q6_k", 1.2, "perm", 1313, 64),
    Config("qwen_a3b_q6k_prefill", 8192, 2048, 768, 128, 8, "q6_k", 1.2, "perm", 1313, 1),
    Config("mixtral_q6k_decode", 1, 4096, 14336, 8, 2, "q6_k", None, "perm", 1414, 8),
]}


def config(name: str, **overrides) -> Config:
    """A named workload, optionally with fields replaced (e.g. a smaller T)."""
    return dataclasses.replace(CONFIGS[name], **overrides)


# --------------------------------------------------------------------------------------
# storage-format encoders for the generator (input preparation only)
# --------------------------------------------------------------------------------------

def _f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Store fp64 draws as bf16 bit patterns: fp64 -> fp32 (nearest) -> bf16 (nearest even).

    The stored bits are the ground truth for every consumer; how they were reached
    only shapes the input distribution.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _f64_to_fp16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float16).view(np.uint16)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


# stream tags
_X, _ROUTER, _EXPERT, _ZIPF, _SLOT, _REDRAW = 1, 2, 3, 4, 5, 7


def make_x(cfg: Config, layer: int = 0, T: int | None = None) -> np.ndarray:
    """Activations: bf16 bits [T, H], ~N(0, 1). Row t does not depend on T."""
    T = cfg.T if T is None else T
    g = _rng(cfg.seed, _X, layer)
    return _f64_to_bf16_bits(g.standard_normal((T, cfg.H)))


def redraw_x_row(cfg: Config, layer: int, t: int, attempt: int) -> np.ndarray:
    """A replacement activation row for token t, from a seed derived from (t, attempt)."""
    g = _rng(cfg.seed, _REDRAW, layer, t, attempt)
    return _f64_to_bf16_bits(g.standard_normal(cfg.H))


def make_router(cfg: Config, layer: int = 0) -> np.ndarray:
    """Router weights: bf16 bits [E, H], ~N(0, 1/H)."""
    g = _rng(cfg.seed, _ROUTER, layer)
    return _f64_to_bf16_bits(g.standard_normal((cfg.E, cfg.H)) / np.sqrt(cfg.H))


def make_bias(cfg: Config) -> np.ndarray | None:
    """Per-expert router offset giving a Zipf(s) prior over experts, or None.

    b_e = -s * ln(r_e) with r a seeded permutation of 1..E, so exp(b_e) = r_e^-s.
    """
    if cfg.zipf_s is None:
        return None
    g = _rng(cfg.seed, _ZIPF)
    r = g.permutation(cfg.E) + 1
    return (-cfg.zipf_s * np.log(r.astype(np.float64))).astype(np.float32)


def make_slot_map(cfg: Config, layer: int = 0) -> np.ndarray:
    if cfg.slot == "identity":
        return np.arange(cfg.E, dtype=np.int32)
    g = _rng(cfg.seed, _SLOT, layer)
    return g.permutation(cfg.E).astype(np.int32)


def _mxfp4_matrix(g: np.random.Generator, rows: int, K: int):
    codes = g.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)       # 16 codes equally likely
    scales = g.integers(120, 123, size=(rows, K // 32), dtype=np.uint8)   # exponents -7, -6, -5
    return codes, scales


def _q8_0_matrix(g: np.random.Generator, rows: int, K: int):
    q = g.integers(-127, 128, size=(rows, K), dtype=np.int8)
    d = _f64_to_fp16_bits(g.uniform(1e-3, 4e-3, size=(rows, K // 32)))
    return q, d


def _q4_k_matrix(g: np.random.Generator, rows: int, K: int):
    if K % 256:
        raise ValueError(f"Q4_K needs K to be a multiple of 256, got {K}")
    nb, ns = K // 32, K // 256
    codes = g.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)      # 16 codes equally likely
    sc = g.integers(32, 64, size=(rows, nb), dtype=np.uint8)             # 6-bit scales
    m = g.integers(32, 64, size=(rows, nb), dtype=np.uint8)              # 6-bit mins
    d = _f64_to_fp16_bits(g.uniform(1.5e-4, 2.5e-4, size=(rows, ns)))
    dmin = _f64_to_fp16_bits(g.uniform(1.2e-3, 2.0e-3, size=(rows, ns)))
    scales = np.empty((rows, 2 * nb + 4 * ns), dtype=np.uint8)
    scales[:, 0:2 * nb:2] = sc
    scales[:, 1:2 * nb:2] = m
    sup = np.stack([d, dmin], axis=-1).reshape(rows, 2 * ns)
    scales[:, 2 * nb:] = np.ascontiguousarray(sup).view(np.uint8)
    return codes, scales


def _q5_k_matrix(g: np.random.Generator, rows: int, K: int):
    lo, scales = _q4_k_matrix(g, rows, K)
    # d halved: with codes 0..31 (mean 15.5) the weights keep Q4_K's spread and a mean
    # near zero against the same mins
    nb, ns = K // 32, K // 256
    sup = np.ascontiguousarray(scales[:, 2 * nb:]).view(np.uint16).reshape(rows, ns, 2)
    sup[..., 0] = _f64_to_fp16_bits(g.uniform(0.75e-4, 1.25e-4, size=(rows, ns)))
    scales[:, 2 * nb:] = sup.reshape(rows, 2 * ns).view(np.uint8)
    hb = g.integers(0, 256, size=(rows, K // 8), dtype=np.uint8)
    return np.concatenate([lo, hb], axis=1), scales


def _q6_k_matrix(g: np.random.Generator, rows: int, K: int):
    if K % 256:
        raise ValueError(f"Q6_K needs K to be a multiple of 256, got {K}")
    codes = g.integers(0, 256, size=(rows, K // 2 + K // 4), dtype=np.uint8)   # q uniform 0..63
    sc = g.integers(-127, 128, size=(rows, K // 16)).astype(np.int8)          # signed scales
    d = _f64_to_fp16_bits(g.uniform(3.0e-5, 5.0e-5, size=(rows, K // 256)))
    scales = np.concatenate([sc.view(np.uint8), np.ascontiguousarray(d).view(np.uint8)], axis=1)
    return codes, scales


_MAKERS = {"mxfp4": _mxfp4_matrix, "q8_0": _q8_0_matrix, "q4_k": _q4_k_matrix,
           "q5_k": _q5_k_matrix, "q6_k": _q6_k_matrix}


def make_expert(cfg: Config, layer: int, e: int) -> dict[str, np.ndarray]:
    """Weights of logical expert e of one layer (canonical layout, no slot axis)."""
    g = _rng(cfg.seed, _EXPERT, layer, e)
    mk = _MAKERS[cfg.fmt]
    gq, gs = mk(g, cfg.I, cfg.H)
    uq, us = mk(g, cfg.I, cfg.H)
    dq, ds = mk(g, cfg.H, cfg.I)
    return dict(gate_q=gq, gate_s=gs, up_q=uq, up_s=us, down_q=dq, down_s=ds)


@dataclasses.dataclass
class Layer:
    cfg: Config
    x: np.ndarray
    wr: np.ndarray
    bias: np.ndarray | None
    slot_map: np.ndarray
    gate_q: np.ndarray
    gate_s: np.ndarray
    up_q: np.ndarray
    up_s: np.ndarray
    down_q: np.ndarray
    down_s: np.ndarray

    @property
    def planes(self) -> dict[str, np.ndarray]:
        return {n: getattr(self, n) for n in
                ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")}


def make_layer(cfg: Config, layer: int = 0, T: int | None = None) -> Layer:
    """One whole layer: inputs, router, and a pool with expert e stored at slot_map[e]."""
    slot_map = make_slot_map(cfg, layer)
    planes: dict[str, np.ndarray] = {}
    for e in range(cfg.E):
        w = make_expert(cfg, layer, e)
        s = int(slot_map[e])
        for n, a in w.items():
            if n not in planes:
                planes[n] = np.empty((cfg.E,) + a.shape, dtype=a.dtype)
            planes[n][s] = a
    return Layer(cfg, make_x(cfg, layer, T), make_router(cfg, layer), make_bias(cfg),
                 slot_map, **planes)
