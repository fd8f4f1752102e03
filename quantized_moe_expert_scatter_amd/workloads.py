"""Seeded synthetic inputs for the prefill routed-expert product.

This module only draws random inputs and lays them out in the storage formats
the library and the oracle both read. It holds none of the method's
arithmetic (no quantization, no products, no activation), so the oracle and
the GPU path can both be fed from it without sharing any computation.

Storage formats (byte layouts are this project's own; the pages name the
formats but never print their bits):

* Activations X: float32, row-major [T, hidden].
* Routing ids: int32, row-major [T, topk]; entry t*topk + k is the k-th expert
  of token t.
* Q2_0 weight matrix of one expert, [rows, cols] (rows = output features,
  cols = the contraction dimension, a multiple of 64), two planes:
    - codes: rows * cols/64 blocks of 16 bytes, row-major by (row, block).
      Inside a block, value 16*j + b (j < 4, b < 16) is the 2-bit code in
      byte b, bits 2j..2j+1.  The represented weight is d * (code - 2), so
      codes {0,1,2,3} mean {-2,-1,0,1}.
    - scales: rows * cols/64 IEEE binary16 values d, row-major by (row, block).
  Expert bytes: rows*cols/64*18 (codes plane first, scales plane after it).
* NL4 (4-bit non-linear) weight matrix of one expert, [rows, cols] with cols a
  multiple of 32, two planes:
    - codes: rows * cols/32 blocks of 16 bytes.  Value b (b < 16) is the low
      nibble of byte b, value 16 + b the high nibble.  The represented weight
      is d * codebook[code] with a 16-entry int8 codebook.
    - scales: rows * cols/32 binary16 values.
  Expert bytes: rows*cols/32*18.
* All experts of one product live in one buffer; expert e starts at byte
  offset[e] (16-byte aligned).  By default experts are stored in id order;
  ``shuffle_slots`` stores them in a random slot order with gaps so that
  consumers must go through the offset table.

Workloads (the pages' benchmark layers; the real model weights and prompts
they were measured on are not available, these seeded draws stand in):

    tiny : T=64,    hidden 256,  n_ff 128, 8 experts,   top-2, uniform routing
    2k   : T=2048,  hidden 2560, n_ff 640, 512 experts, top-10, uniform
    8k   : T=8192,  same layer,  lognormal expert popularity (sigma 1.0)
    16k  : T=16384, same layer,  uniform
    t128 : T=128,   same layer,  uniform, down product in NL4
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

Q2_0 = 1
NL4 = 2

Q2_0_BLOCK = 64
NL4_BLOCK = 32
BLOCK_BYTES = 18  # 16 bytes of codes + one binary16 scale, both formats


@dataclass(frozen=True)
class LayerConfig:
    name: str
    tokens: int
    hidden: int
    n_ff: int
    n_expert: int
    topk: int
    routing: str  # "uniform" | "lognormal" | "flat32"
    down_type: int = Q2_0
    sigma: float = 1.0
    gu_type: int = Q2_0
    x_seed: int = 0
    ids_seed: int = 0
    gu_seed: int = 0
    down_seed: int = 0

    @property
    def rows(self) -> int:
        return self.tokens * self.topk


# One layer shared by 2k / 8k / 16k (same weight seeds); t128 reuses the gate/up
# seed and draws its own NL4 down product.
_LAYER_GU_SEED = 1001
_LAYER_DOWN_SEED = 1002

CONFIGS = {
    "tiny": LayerConfig("tiny", 64, 256, 128, 8, 2, "uniform",
                        x_seed=11, ids_seed=12, gu_seed=13, down_seed=14),
    "2k": LayerConfig("2k", 2048, 2560, 640, 512, 10, "uniform",
                      x_seed=21, ids_seed=22, gu_seed=_LAYER_GU_SEED, down_seed=_LAYER_DOWN_SEED),
    "8k": LayerConfig("8k", 8192, 2560, 640, 512, 10, "lognormal", sigma=1.0,
                      x_seed=31, ids_seed=32, gu_seed=_LAYER_GU_SEED, down_seed=_LAYER_DOWN_SEED),
    "16k": LayerConfig("16k", 16384, 2560, 640, 512, 10, "uniform",
                       x_seed=41, ids_seed=42, gu_seed=_LAYER_GU_SEED, down_seed=_LAYER_DOWN_SEED),
    "t128": LayerConfig("t128", 128, 2560, 640, 512, 10, "uniform", down_type=NL4,
                        x_seed=51, ids_seed=52, gu_seed=_LAYER_GU_SEED, down_seed=1052),
    # both products in NL4 (32-value blocks, codebook weights) at the 2K shape
    "2k_nl4": LayerConfig("2k_nl4", 2048, 2560, 640, 512, 10, "uniform", down_type=NL4,
                          gu_type=NL4, x_seed=61, ids_seed=62, gu_seed=1061, down_seed=1052),
}


# The rows-per-expert sweep: prompt chunks of 768..4096 tokens under skewed
# (lognormal sigma 0.5, 1.0) and flat (32 rows per routed expert, at most 512
# experts) routings, on the same layer as 2k / 8k / 16k.
SWEEP_TOKENS = (768, 1024, 1536, 4096)
SWEEP_ROUTINGS = (("ln0.5", "lognormal", 0.5), ("ln1.0", "lognormal", 1.0), ("flat32", "flat32", 1.0))
SWEEP = {}
for _t in SWEEP_TOKENS:
    for _i, (_tag, _kind, _sigma) in enumerate(SWEEP_ROUTINGS):
        _name = f"sw{_t}_{_tag}"
        SWEEP[_name] = LayerConfig(_name, _t, 2560, 640, 512, 10, _kind, sigma=_sigma,
                                   x_seed=6000 + 10 * _t + _i, ids_seed=7000 + 10 * _t + _i,
                                   gu_seed=_LAYER_GU_SEED, down_seed=_LAYER_DOWN_SEED)


def block_of(wtype: int) -> int:
    return Q2_0_BLOCK if wtype == Q2_0 else NL4_BLOCK


def expert_bytes(wtype: int, rows: int, cols: int) -> int:
    return rows * (cols // block_of(wtype)) * BLOCK_BYTES


# --------------------------------------------------------------------------- X
def activations(tokens: int, hidden: int, seed: int, scale: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((tokens, hidden), dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


# --------------------------------------------------------------------- routing
def routing_uniform(tokens: int, n_expert: int, topk: int, seed: int) -> np.ndarray:
    """topk distinct experts per token, uniform without replacement."""
    rng = np.random.default_rng(seed)
    ids = np.empty((tokens, topk), dtype=np.int32)
    step = 4096
    for t0 in range(0, tokens, step):
        keys = rng.random((min(step, tokens - t0), n_expert))
        ids[t0:t0 + keys.shape[0]] = np.argsort(keys, axis=1)[:, :topk]
    return ids


def routing_lognormal(tokens: int, n_expert: int, topk: int, sigma: float, seed: int) -> np.ndarray:
    """Expert popularity w_e = exp(sigma * z_e), z_e ~ N(0,1); each token draws
    topk distinct experts by weighted sampling without replacement (the
    Gumbel-top-k construction: the topk largest log w_e + Gumbel noise)."""
    rng = np.random.default_rng(seed)
    logw = sigma * rng.standard_normal(n_expert)
    ids = np.empty((tokens, topk), dtype=np.int32)
    step = 4096
    for t0 in range(0, tokens, step):
        n = min(step, tokens - t0)
        g = rng.gumbel(size=(n, n_expert))
        ids[t0:t0 + n] = np.argsort(-(logw[None, :] + g), axis=1)[:, :topk]
    return ids


def routing_flat(tokens: int, n_expert: int, topk: int, per_expert: int, seed: int) -> np.ndarray:
    """Every routed expert gets the same number of rows: the first
    min(n_expert, tokens*topk/per_expert) experts of a seeded permutation,
    taken round robin over the flattened (token, slot) order, so a token's
    topk experts are distinct whenever at least topk experts are used."""
    rng = np.random.default_rng(seed)
    used = max(topk, min(n_expert, (tokens * topk) // per_expert))
    experts = rng.permutation(n_expert)[:used].astype(np.int32)
    flat = np.arange(tokens * topk, dtype=np.int64) % used
    return experts[flat].reshape(tokens, topk)


def routing_weights(tokens: int, topk: int, seed: int) -> np.ndarray:
    """float32 [T, topk]: a softmax over the token's topk of standard normal
    logits (what a router hands the combine), computed in float64."""
    z = np.random.default_rng(seed).standard_normal((tokens, topk))
    if tokens == 0:
        return z.astype(np.float32)
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def routing(cfg: LayerConfig) -> np.ndarray:
    if cfg.routing == "uniform":
        return routing_uniform(cfg.tokens, cfg.n_expert, cfg.topk, cfg.ids_seed)
    if cfg.routing == "lognormal":
        return routing_lognormal(cfg.tokens, cfg.n_expert, cfg.topk, cfg.sigma, cfg.ids_seed)
    if cfg.routing == "flat32":
        return routing_flat(cfg.tokens, cfg.n_expert, cfg.topk, 32, cfg.ids_seed)
    raise ValueError(cfg.routing)


# --------------------------------------------------------------------- weights
@dataclass
class ExpertWeights:
    """All experts of one product in one byte buffer plus the offset table."""
    wtype: int
    rows: int
    cols: int
    n_expert: int
    buf: np.ndarray            # uint8, the whole weight buffer
    offsets: np.ndarray        # uint64 [n_expert], byte offset of expert e
    codebook: Optional[np.ndarray] = None  # int8 [16], NL4 only

    @property
    def per_expert(self) -> int:
        return expert_bytes(self.wtype, self.rows, self.cols)

    def expert(self, e: int) -> np.ndarray:
        o = int(self.offsets[e])
        return self.buf[o:o + self.per_expert]


def _scales_f16(rng: np.random.Generator, n: int, lo: float = 0.01, hi: float = 0.05) -> np.ndarray:
    # fp32 uniform draw, rounded to nearest-even binary16 by numpy's cast
    u = rng.random(n, dtype=np.float32)
    return (np.float32(lo) + u * np.float32(hi - lo)).astype(np.float16)


def nl4_codebook(seed: int) -> np.ndarray:
    """16 distinct integers drawn uniformly without replacement from
    [-127, 127], sorted ascending."""
    rng = np.random.default_rng(seed)
    cb = rng.choice(np.arange(-127, 128), size=16, replace=False)
    return np.sort(cb).astype(np.int8)


def expert_weights(wtype: int, rows: int, cols: int, n_expert: int, seed: int,
                   shuffle_slots: bool = False, scale_range=(0.01, 0.05)) -> ExpertWeights:
    """Uniform codes (random bytes: every 2-bit or 4-bit field is uniform and
    independent), binary16 scales uniform in ``scale_range``."""
    blk = block_of(wtype)
    if cols % blk or rows <= 0:
        raise ValueError("cols must be a multiple of the block size")
    rng = np.random.default_rng(seed)
    nblk = rows * (cols // blk)
    per = nblk * BLOCK_BYTES
    pad = (-per) % 256
    stride = per + pad
    if shuffle_slots:
        # the slot order has its own stream, so the contents of every expert
        # are the same as in id order
        n_slots = n_expert + max(1, n_expert // 4)
        slots = np.random.default_rng(seed + 104729).permutation(n_slots)[:n_expert]
    else:
        n_slots = n_expert
        slots = np.arange(n_expert)
    buf = np.zeros(n_slots * stride, dtype=np.uint8)
    offsets = (slots.astype(np.uint64) * np.uint64(stride))
    codebook = nl4_codebook(seed + 7919) if wtype == NL4 else None
    for e in range(n_expert):
        o = int(offsets[e])
        codes = np.frombuffer(rng.bytes(nblk * 16), dtype=np.uint8)
        buf[o:o + nblk * 16] = codes
        sc = _scales_f16(rng, nblk, *scale_range)
        buf[o + nblk * 16:o + per] = sc.view(np.uint8)
    return ExpertWeights(wtype, rows, cols, n_expert, buf, offsets, codebook)


def interleave_gate_up(w: ExpertWeights) -> ExpertWeights:
    """The same gate/up matrices stored with alternating rows: row 2j is gate
    row j, row 2j+1 up row j (both planes), same offsets."""
    F = w.rows // 2
    nb = w.cols // block_of(w.wtype)
    n = w.rows * nb
    order = np.empty(w.rows, np.int64)
    order[0::2] = np.arange(F)
    order[1::2] = F + np.arange(F)
    buf = w.buf.copy()
    for e in range(w.n_expert):
        o = int(w.offsets[e])
        codes = w.buf[o:o + 16 * n].reshape(w.rows, nb * 16)
        scales = w.buf[o + 16 * n:o + 18 * n].reshape(w.rows, nb * 2)
        buf[o:o + 16 * n] = codes[order].reshape(-1)
        buf[o + 16 * n:o + 18 * n] = scales[order].reshape(-1)
    return ExpertWeights(w.wtype, w.rows, w.cols, w.n_expert, buf, w.offsets.copy(), w.codebook)


# ----------------------------------------------------------------------- layer
@dataclass
class Layer:
    cfg: LayerConfig
    x: np.ndarray
    ids: np.ndarray
    w_gu: ExpertWeights
    w_down: ExpertWeights
    route_w: Optional[np.ndarray] = None     # float32 [T, topk] routing weights
    extra: dict = field(default_factory=dict)


def make_layer(cfg: LayerConfig, shuffle_slots: bool = False) -> Layer:
    x = activations(cfg.tokens, cfg.hidden, cfg.x_seed)
    ids = routing(cfg)
    w_gu = expert_weights(cfg.gu_type, 2 * cfg.n_ff, cfg.hidden, cfg.n_expert, cfg.gu_seed,
                          shuffle_slots=shuffle_slots)
    w_down = expert_weights(cfg.down_type, cfg.hidden, cfg.n_ff, cfg.n_expert, cfg.down_seed,
                            shuffle_slots=shuffle_slots)
    route_w = routing_weights(cfg.tokens, cfg.topk, cfg.ids_seed + 5003)
    return Layer(cfg, x, ids, w_gu, w_down, route_w)


def small_config(name: str, tokens: int, hidden: int, n_ff: int, n_expert: int, topk: int,
                 routing_kind: str = "uniform", down_type: int = Q2_0, seed: int = 0,
                 gu_type: int = Q2_0) -> LayerConfig:
    """An ad-hoc config for tests (ragged shapes, other routings)."""
    return LayerConfig(name, tokens, hidden, n_ff, n_expert, topk, routing_kind,
                       down_type=down_type, gu_type=gu_type, x_seed=seed * 10 + 1, ids_seed=seed * 10 + 2,
                       gu_seed=seed * 10 + 3, down_seed=seed * 10 + 4)
